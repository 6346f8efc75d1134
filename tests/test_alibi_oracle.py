"""Pins for the ALiBi term of the oracle (reading R11 of oracle/attention.py).

The bias is slope_h * (t - q_abs), added after scaling.  It is pinned by a
closed form (with zero queries the softmax weights are a geometric series in
the distance), a two-key example worked by hand that separates a scaled from
an unscaled slope and both signs, the absolute-position form of the
BI-V100 decode (same output, LSE shifted by slope * q_abs), the scalar
brute force, and zero slopes reducing to no ALiBi.
"""
import math

import pytest
import torch

from oracle import attention as orc
from oracle import brute
from relative_bias_amd import workloads as wl


def _args(w):
    return (w.block_table, w.cache_seqlens, w.cu_seqlens_q, w.softmax_scale, w.causal, w.window_size,
            w.rel_extent, w.rel_logits)


@pytest.mark.parametrize("slope,lk", [(0.5, 40), (0.0625, 300), (2.0, 7)])
def test_zero_queries_give_geometric_weights(slope, lk):
    """q = 0, no relative bias, one decode row at q_abs = lk - 1: the logit of
    key t is -slope * (lk - 1 - t), so lse = ln sum_{d<lk} exp(-slope d) =
    ln((1 - e^(-slope lk)) / (1 - e^(-slope))) and the weights fall by e^-slope
    per key of distance."""
    w = wl.build([1], [lk], num_heads=2, num_kv_heads=1, head_dim=8, seed=1)
    w.q = torch.zeros_like(w.q)
    sl = torch.tensor([slope, 0.0], dtype=torch.float32)
    out, lse = orc.attention(w.q, w.key_cache, w.value_cache, *_args(w), alibi_slopes=sl)
    r = math.exp(-slope)
    want_lse = math.log((1 - r ** lk) / (1 - r))
    assert abs(lse[0, 0].item() - want_lse) < 1e-12
    # Output: sum_t r^(lk-1-t) v_t / sum_d r^d, from the gathered V rows.
    pages = w.block_table[0].tolist()
    V = torch.stack([w.value_cache[pages[t // 16], t % 16, 0].double() for t in range(lk)])
    wts = torch.tensor([r ** (lk - 1 - t) for t in range(lk)], dtype=torch.float64)
    want = (wts[:, None] * V).sum(0) / wts.sum()
    assert torch.allclose(out[0, 0], want, atol=1e-12, rtol=0)
    # Head 1 has slope 0: the plain mean of V.
    assert torch.allclose(out[0, 1], V.mean(0), atol=1e-12, rtol=0)
    assert abs(lse[0, 1].item() - math.log(lk)) < 1e-12


def test_two_keys_worked_by_hand():
    """Two keys t = 0, 1 and a decode row at q_abs = 1, scale 0.5, slope 1:
    logits 0.5*a - 1 and 0.5*b (a, b the dot products).  With q = e0 and
    k0 = 4 e0, k1 = 2 e0: a = 4, b = 2 -> logits 1 and 1, weights 1/2 each.
    (A slope applied before the scale would give 1.5 and 1; a reversed sign
    3 and 1.)"""
    w = wl.build([1], [2], num_heads=1, num_kv_heads=1, head_dim=4, seed=2, permute_pages=False,
                 softmax_scale=0.5)
    w.q = torch.zeros_like(w.q)
    w.q[0, 0, 0] = 1.0
    w.key_cache.zero_()
    w.key_cache[0, 0, 0, 0] = 4.0
    w.key_cache[0, 1, 0, 0] = 2.0
    w.value_cache.zero_()
    w.value_cache[0, 0, 0, 0] = 1.0
    w.value_cache[0, 1, 0, 1] = 1.0
    out, lse = orc.attention(w.q, w.key_cache, w.value_cache, *_args(w),
                             alibi_slopes=torch.tensor([1.0]))
    assert torch.allclose(out[0, 0], torch.tensor([0.5, 0.5, 0.0, 0.0], dtype=torch.float64), atol=1e-15)
    assert abs(lse[0, 0].item() - (1 + math.log(2))) < 1e-15


def test_absolute_position_form_shifts_only_the_lse():
    """The BI-V100 decode adds slope * t (absolute key position): each row's
    logits move by slope * q_abs, so out is unchanged and lse moves by it."""
    w = wl.build([1, 1, 1], [50, 17, 129], num_heads=4, num_kv_heads=2, head_dim=16, rel_extent=8, seed=3)
    sl = torch.tensor([0.25, 0.5, 1 / 16, 1.0], dtype=torch.float32)
    o1, l1 = orc.attention(w.q, w.key_cache, w.value_cache, *_args(w), alibi_slopes=sl)
    # The absolute form as a relative bias: rel_logits' = rel_logits + slope * t
    # cannot express it (t is not a distance); compute it directly.
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    cu = w.cu_seqlens_q.tolist()
    for b, lk in enumerate(w.k_lens):
        tok = cu[b]
        pages = w.block_table[b].tolist()
        for h in range(4):
            K = torch.stack([w.key_cache[pages[t // 16], t % 16, h // 2].double() for t in range(lk)])
            V = torch.stack([w.value_cache[pages[t // 16], t % 16, h // 2].double() for t in range(lk)])
            s = (K @ w.q[tok, h].double()) * float(torch.tensor(w.softmax_scale, dtype=torch.float32))
            s = s + orc.bias_matrix(w.rel_logits[[tok], h, :], torch.tensor([lk - 1]), lk, 8)[0]
            s = s + float(sl[h]) * torch.arange(lk, dtype=torch.float64)
            m = s.max()
            p = torch.exp(s - m)
            o2[tok, h] = (p[:, None] * V).sum(0) / p.sum()
            l2[tok, h] = m + torch.log(p.sum())
            shift = float(sl[h]) * (lk - 1)
            assert abs((l2[tok, h] - l1[tok, h]).item() - shift) < 1e-9
    assert torch.allclose(o1, o2, atol=1e-12, rtol=0)


def test_brute_force_agrees_with_alibi():
    for seed, (ql, kl, win) in enumerate([([1, 4, 2], [20, 33, 2], (-1, -1)), ([3, 1], [40, 9], (7, 0)),
                                          ([5], [5], (-1, 2))]):
        w = wl.build(ql, kl, num_heads=4, num_kv_heads=2, head_dim=8, rel_extent=5, window_size=win,
                     causal=win[1] != 2, seed=10 + seed)
        sl = torch.tensor([0.5, 0.125, 1.0, 0.0], dtype=torch.float32)
        o, l = orc.attention(w.q, w.key_cache, w.value_cache, *_args(w), alibi_slopes=sl)
        ob, lb = brute.attention(w.q, w.key_cache, w.value_cache, *_args(w), alibi_slopes=sl)
        ob = torch.as_tensor(ob, dtype=torch.float64)
        lb = torch.as_tensor(lb, dtype=torch.float64)
        assert torch.allclose(o, ob, atol=1e-12, rtol=0)
        fin = torch.isfinite(l)
        assert torch.equal(fin, torch.isfinite(lb))
        assert torch.allclose(l[fin], lb[fin], atol=1e-12, rtol=0)


def test_zero_slopes_are_no_alibi():
    w = wl.tiny()
    o1, l1 = orc.attention(w.q, w.key_cache, w.value_cache, *_args(w), alibi_slopes=torch.zeros(4))
    o2, l2 = orc.attention(w.q, w.key_cache, w.value_cache, *_args(w))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_alibi_equals_a_relative_bias_of_minus_slope_times_distance():
    """Causal rows see only d = q_abs - t >= 0, so with a band that covers
    every key (R >= Lk) ALiBi is the relative bias rel_logits[tok, h, d] =
    -slope_h * d: two different code paths of the oracle must agree."""
    w = wl.build([1, 6, 2], [60, 40, 9], num_heads=4, num_kv_heads=2, head_dim=16, seed=21)
    sl = torch.tensor([0.5, 0.25, 0.125, 1.0], dtype=torch.float32)
    R = 64
    d = torch.arange(R, dtype=torch.float64)
    rel = (-(sl.double()[None, :, None]) * d[None, None, :]).expand(w.num_tokens, 4, R).contiguous()
    o1, l1 = orc.attention(w.q, w.key_cache, w.value_cache, w.block_table, w.cache_seqlens, w.cu_seqlens_q,
                           w.softmax_scale, True, (-1, -1), 0, None, alibi_slopes=sl)
    o2, l2 = orc.attention(w.q, w.key_cache, w.value_cache, w.block_table, w.cache_seqlens, w.cu_seqlens_q,
                           w.softmax_scale, True, (-1, -1), R, rel)
    assert torch.allclose(o1, o2, atol=1e-12, rtol=0) and torch.allclose(l1, l2, atol=1e-12, rtol=0)
