"""Host checks of the measurement code: the algorithmic work that the
benchmark divides by its times (relative_bias_amd/metrics.py) against a
brute-force count over every (row, key) pair, and the benchmark's refusal of
more than one GPU."""
import os
import subprocess
import sys

import pytest

from relative_bias_amd import metrics
from relative_bias_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _brute(w, kv_elem_bytes=2, rel_elem_bytes=4):
    """Count visible pairs, band entries and the keys each request touches
    by looping over every row and key."""
    H, Hkv, D, BS, R = w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, w.rel_extent
    left, right = w.window_size
    pairs = band = kv = pages = 0
    for lq, lk in zip(w.q_lens, w.k_lens):
        keys = set()
        for i in range(lq):
            qa = i + lk - lq
            for t in range(lk):
                vis = (not w.causal or t <= qa) and (left < 0 or t >= qa - left) and (right < 0 or t <= qa + right)
                if not vis:
                    continue
                pairs += 1
                keys.add(t)
                if 0 <= qa - t < R:
                    band += 1
        if keys:
            lo, hi = min(keys), max(keys)
            kv += (hi - lo + 1) * Hkv * D * 2 * kv_elem_bytes
            pages += (hi // BS - lo // BS + 1) * 4
    T = sum(w.q_lens)
    total = kv + 2 * T * H * D * 2 + T * H * 4 + band * H * rel_elem_bytes + pages + (2 * len(w.q_lens) + 1) * 4
    return {"bytes": total, "flops": 4 * D * pairs * H, "kv_bytes": kv}


@pytest.mark.parametrize("case", [
    ([1, 1, 16], [47, 312, 128], True, (-1, -1), 32),
    ([5, 1, 30], [40, 9, 30], True, (7, 0), 6),
    ([3, 2], [20, 11], False, (4, 3), 5),
    ([4, 1], [2, 0], True, (-1, -1), 3),
])
def test_work_matches_a_pairwise_count(case):
    ql, kl, causal, win, R = case
    w = wl.build(ql, kl, num_heads=4, num_kv_heads=2, head_dim=16, rel_extent=R, causal=causal, window_size=win,
                 seed=3)
    got = metrics.work(w)
    want = _brute(w)
    assert got["flops"] == want["flops"] and got["bytes"] == want["bytes"] and got["kv_bytes"] == want["kv_bytes"]
    got8 = metrics.work(w, kv_elem_bytes=1)
    assert got8["bytes"] == _brute(w, kv_elem_bytes=1)["bytes"]


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
