"""GPU parity of the FP8 KV cache against oracle/fp8.py.

rpa_kv_cache_write_fp8 is integer work once the fp32 quotient is formed, so
its codes are compared bit for bit (the oracle forms the same fp32 quotient).
rpa_attn_varlen_fp8 is compared with the fp64 oracle over the dequantised
caches to the attention tolerances (out max 2e-2, mean 2e-3; lse 1e-3).
"""
import math

import pytest
import torch

from oracle import fp8 as ofp8
from oracle import kv_cache as okv
from relative_bias_amd import binding as bnd
from relative_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu

OUT_MAX, OUT_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need a GPU"
    bnd.lib()


# ------------------------------------------------------------- KV write

SPECIAL = [0.0, -0.0, 1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, -(2.0 ** -12), 447.0, 448.0, 460.0,
           464.0, 1e30, -1e30, math.inf, -math.inf, math.nan, 1e-40, -3e-39, 2.0 ** -6, 2.0 ** -7 * 1.9375]


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.0371, 3.0), (0.125, 2.0 ** -7), (7.5, 0.01)])
def test_kv_write_fp8_is_bit_exact(k_scale, v_scale):
    w = wl.build([1, 5, 33, 2, 1], [40, 5, 100, 300, 17], num_heads=16, num_kv_heads=8, head_dim=128,
                 block_size=16, seed=8)
    g = torch.Generator().manual_seed(9)
    T = w.num_tokens
    key = (torch.randn((T, 8, 128), generator=g) * 4).to(torch.bfloat16)
    val = (torch.randn((T, 8, 128), generator=g) * 0.3).to(torch.bfloat16)
    sp = torch.tensor(SPECIAL, dtype=torch.float32).to(torch.bfloat16)
    key.view(-1)[: sp.numel()] = sp
    val.view(-1)[-sp.numel():] = sp
    # Values near the rounding boundaries of x / scale.
    key[3, 2] = (torch.linspace(-500, 500, 128) * k_scale).to(torch.bfloat16)
    kc = torch.randint(0, 256, w.key_cache.shape, generator=g, dtype=torch.int32).to(torch.uint8)
    vc = torch.randint(0, 256, w.key_cache.shape, generator=g, dtype=torch.int32).to(torch.uint8)
    slots = okv.slot_mapping(w.block_table, w.k_lens, w.cu_seqlens_q.tolist(), 16)
    want_k, want_v = ofp8.kv_cache_write_fp8(key, val, slots, kc, vc, k_scale, v_scale)
    kg, vg = kc.cuda(), vc.cuda()
    bnd.rpa_kv_cache_write_fp8(key.cuda(), val.cuda(), slots.cuda(), kg, vg, k_scale, v_scale)
    torch.cuda.synchronize()
    assert torch.equal(kg.cpu(), want_k)
    assert torch.equal(vg.cpu(), want_v)


def test_kv_write_fp8_every_bf16_value():
    """All 65536 bf16 bit patterns through the quantiser at two scales."""
    allb = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    T, Hkv, D = 512, 1, 128
    key = allb.reshape(T, Hkv, D).contiguous()
    val = allb.flip(0).reshape(T, Hkv, D).contiguous()
    slots = torch.arange(T, dtype=torch.int64)
    kc = torch.zeros((T // 16, 16, Hkv, D), dtype=torch.uint8)
    vc = torch.zeros_like(kc)
    for ks, vs in ((1.0, 1.0), (0.3, 5.0)):
        want_k, want_v = ofp8.kv_cache_write_fp8(key, val, slots, kc, vc, ks, vs)
        kg, vg = kc.cuda(), vc.cuda()
        bnd.rpa_kv_cache_write_fp8(key.cuda(), val.cuda(), slots.cuda(), kg, vg, ks, vs)
        torch.cuda.synchronize()
        assert torch.equal(kg.cpu(), want_k), f"key codes differ at scale {ks}"
        assert torch.equal(vg.cpu(), want_v), f"value codes differ at scale {vs}"


# ------------------------------------------------------------- attention

def _fp8_workload(q_lens, k_lens, H, Hkv, D, R, k_scale, v_scale, seed, window=(-1, -1), extra_pages=0,
                  block_size=16, poison=False):
    w = wl.build(q_lens, k_lens, num_heads=H, num_kv_heads=Hkv, head_dim=D, block_size=block_size, rel_extent=R,
                 window_size=window, seed=seed, extra_pages=extra_pages)
    g = torch.Generator().manual_seed(seed + 1000)
    # Codes of N(0, 1) keys / values at the given scales (inputs, not results).
    k8 = (torch.randn(w.key_cache.shape, generator=g) / k_scale).to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = (torch.randn(w.key_cache.shape, generator=g) / v_scale).to(torch.float8_e4m3fn).view(torch.uint8)
    if poison:
        # NaN codes in every page no request references and in every slot past
        # a request's last key: a correct kernel never lets them into a result.
        used = torch.zeros(k8.shape[0], dtype=torch.bool)
        for b, lk in enumerate(w.k_lens):
            n = (lk + block_size - 1) // block_size
            for j in range(n):
                pg = int(w.block_table[b, j])
                used[pg] = True
                if j == n - 1 and lk % block_size:
                    k8[pg, lk % block_size:] = 0x7F
                    v8[pg, lk % block_size:] = 0xFF
        k8[~used] = 0x7F
        v8[~used] = 0x7F
    return w, k8, v8


def _run_fp8(w, k8, v8, k_scale, v_scale, S=0):
    wg = w.to("cuda")
    out, lse = bnd.rpa_attn_varlen_fp8(
        wg.q, k8.cuda(), v8.cuda(), k_scale=k_scale, v_scale=v_scale, block_table=wg.block_table,
        cache_seqlens=wg.cache_seqlens, cu_seqlens_q=wg.cu_seqlens_q, max_seqlen_q=wg.max_seqlen_q,
        softmax_scale=wg.softmax_scale, causal=wg.causal, window_size=wg.window_size,
        rel_extent=wg.rel_extent, rel_logits=wg.rel_logits, num_splits=S, return_lse=True)
    torch.cuda.synchronize()
    return out.float().cpu().double(), lse.cpu().double()


def _compare(out, lse, ref_out, ref_lse, tag):
    assert not torch.isnan(out).any(), f"{tag}: NaN in GPU output"
    err = (out - ref_out).abs()
    assert err.max().item() <= OUT_MAX, f"{tag}: out max err {err.max().item():.3e}"
    assert err.mean().item() <= OUT_MEAN, f"{tag}: out mean err {err.mean().item():.3e}"
    inf = torch.isinf(ref_lse)
    assert torch.equal(torch.isinf(lse), inf), f"{tag}: lse -inf pattern differs"
    if inf.any():
        assert (out[inf] == 0).all()
    if (~inf).any():
        le = (lse[~inf] - ref_lse[~inf]).abs().max().item()
        assert le <= LSE_MAX, f"{tag}: lse max err {le:.3e}"


CASES = {
    # name: (q_lens, k_lens, H, Hkv, D, R, k_scale, v_scale, window)
    "ragged_d128": ([1] * 12, [1, 15, 16, 17, 100, 333, 1024, 1500, 2048, 2999, 64, 700], 32, 8, 128, 64,
                    1 / 32, 1 / 16, (-1, -1)),
    "g1_d64_nobias": ([1] * 5, [5, 900, 31, 2000, 129], 8, 8, 64, 0, 0.05, 0.2, (-1, -1)),
    "g16_bias_wider_than_kv": ([1] * 4, [70, 10, 300, 1], 128, 8, 128, 400, 0.02, 0.03, (-1, -1)),
    "two_tokens_g8": ([2, 2, 2], [2, 500, 1200], 64, 8, 128, 32, 1 / 64, 1 / 8, (-1, -1)),
    "window": ([1] * 6, [3000, 100, 2000, 700, 4096, 256], 32, 8, 128, 128, 1 / 32, 1 / 16, (255, 0)),
    "empty_rows": ([1, 2, 1, 1], [0, 1, 40, 0], 16, 8, 128, 16, 0.1, 0.1, (-1, -1)),
    "scales_above_one": ([1] * 3, [800, 77, 1600], 32, 8, 128, 50, 4.0, 3.0, (-1, -1)),
}


CASES.update({
    # other kv-head counts (balanced decode of one (request, kv head) pair per unit)
    "gqa4_d128": ([1] * 7, [1, 17, 300, 1024, 2500, 64, 999], 8, 2, 128, 64, 1 / 32, 1 / 16, (-1, -1)),
    "mha_d64": ([1] * 3, [33, 700, 129], 4, 4, 64, 16, 0.05, 0.2, (-1, -1)),
    # prefill chunks and mixed batches (split mode: prefill tiles and decode items)
    "prefill_d128": ([300, 77, 129], [900, 77, 1500], 16, 8, 128, 256, 1 / 32, 1 / 16, (-1, -1)),
    "prefill_d64_gqa2": ([64, 200], [64, 333], 4, 2, 64, 40, 0.05, 0.2, (-1, -1)),
    "mixed_window": ([1, 130, 1, 40, 1], [2000, 500, 70, 3000, 1], 16, 2, 128, 100, 1 / 32, 1 / 16, (127, 0)),
    "prefill_nobias_mha": ([100, 3], [400, 3], 4, 4, 128, 0, 0.1, 0.1, (-1, -1)),
    # one q-tile per request over 1 to 5 key tiles, the last one partial: the
    # prefill's raw K tiles two ahead of their QK run past the end (zero-filled)
    "prefill_tile_counts": ([32] * 5, [40, 100, 150, 250, 300], 16, 4, 128, 64, 1 / 32, 1 / 16, (-1, -1)),
    "prefill_tile_counts_d64_window": ([32] * 4, [70, 130, 200, 260], 8, 2, 64, 32, 0.05, 0.2, (100, 0)),
})

# Split counts per case: 0 (balanced when it applies, else 1) always, and
# explicit splits for a few.
SPLITS = {name: [0] for name in CASES}
SPLITS.update({"ragged_d128": [0, 1, 3], "gqa4_d128": [0, 4], "prefill_d128": [1, 2], "mixed_window": [1, 3],
               "two_tokens_g8": [0, 2], "prefill_tile_counts": [1, 2], "prefill_tile_counts_d64_window": [1, 2]})
PARAMS = [(n, S) for n in CASES for S in SPLITS[n]]


@pytest.mark.parametrize("name,S", PARAMS)
def test_fp8_attention_matches_oracle(name, S):
    ql, kl, H, Hkv, D, R, ks, vs, win = CASES[name]
    w, k8, v8 = _fp8_workload(ql, kl, H, Hkv, D, R, ks, vs, seed=21, window=win, extra_pages=3)
    ref_out, ref_lse = ofp8.attention_fp8(w.q, k8, v8, ks, vs, w.block_table, w.cache_seqlens, w.cu_seqlens_q,
                                          w.softmax_scale, w.causal, w.window_size, w.rel_extent, w.rel_logits)
    out, lse = _run_fp8(w, k8, v8, ks, vs, S=S)
    _compare(out, lse, ref_out, ref_lse, f"{name} S={S}")


def test_fp8_attention_is_repeatable_and_page_invariant():
    ql, kl = [1] * 40, [int(x) for x in torch.randint(1, 5000, (40,), generator=torch.Generator().manual_seed(4))]
    w, k8, v8 = _fp8_workload(ql, kl, 32, 8, 128, 128, 1 / 32, 1 / 16, seed=22)
    a = _run_fp8(w, k8, v8, 1 / 32, 1 / 16)
    b = _run_fp8(w, k8, v8, 1 / 32, 1 / 16)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # The same logical pages at other physical places.
    NB = k8.shape[0]
    perm = torch.randperm(NB, generator=torch.Generator().manual_seed(5))
    inv = torch.argsort(perm)
    bt = w.block_table.clone()
    valid = bt >= 0
    bt[valid] = inv[bt[valid].long()].to(torch.int32)
    w2 = w.to("cpu")
    w2.block_table = bt
    c = _run_fp8(w2, k8[perm].contiguous(), v8[perm].contiguous(), 1 / 32, 1 / 16)
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])


@pytest.mark.parametrize("BS", [32, 48])
@pytest.mark.parametrize("kind", ["decode_heads", "decode_pairs", "prefill"])
def test_fp8_block_sizes_and_nan_poison(BS, kind):
    """Block sizes other than 16 (48: not a power of two) with NaN codes in
    unreferenced pages and tail slots."""
    if kind == "decode_heads":
        args = ([1] * 5, [1, 100, 777, 2000, 48], 32, 8, 128, 64)
    elif kind == "decode_pairs":
        args = ([1] * 4, [3, 96, 1000, 500], 8, 2, 128, 32)
    else:
        args = ([70, 1, 33], [300, 40, 33], 8, 2, 64, 16)
    ql, kl, H, Hkv, D, R = args
    w, k8, v8 = _fp8_workload(ql, kl, H, Hkv, D, R, 1 / 32, 1 / 16, seed=24, extra_pages=2, block_size=BS,
                              poison=True)
    ref_out, ref_lse = ofp8.attention_fp8(w.q, k8, v8, 1 / 32, 1 / 16, w.block_table, w.cache_seqlens,
                                          w.cu_seqlens_q, w.softmax_scale, w.causal, w.window_size, w.rel_extent,
                                          w.rel_logits)
    for S in (0, 2):
        out, lse = _run_fp8(w, k8, v8, 1 / 32, 1 / 16, S=S)
        _compare(out, lse, ref_out, ref_lse, f"{kind} BS={BS} S={S}")


def test_fp8_graph_replay():
    """A captured E4M3 decode replayed over new lengths equals the eager call."""
    B, kmax = 10, 2000
    w, k8, v8 = _fp8_workload([1] * B, [kmax] * B, 32, 8, 128, 64, 1 / 32, 1 / 16, seed=25)
    wg = w.to("cuda")
    k8g, v8g = k8.cuda(), v8.cuda()
    T, H, D = wg.q.shape
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty((bnd.rpa_workspace_bytes(0, T, H, D),), dtype=torch.uint8, device="cuda")

    def call(o, l):
        bnd.rpa_attn_varlen_fp8(wg.q, k8g, v8g, k_scale=1 / 32, v_scale=1 / 16, block_table=wg.block_table,
                                cache_seqlens=wg.cache_seqlens, cu_seqlens_q=wg.cu_seqlens_q, max_seqlen_q=1,
                                softmax_scale=wg.softmax_scale, rel_extent=wg.rel_extent, rel_logits=wg.rel_logits,
                                num_splits=0, out=o, lse=l, workspace=ws)

    call(out, lse)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        call(out, lse)
    gen = torch.Generator().manual_seed(26)
    for _ in range(3):
        kl = torch.randint(1, kmax + 1, (B,), generator=gen, dtype=torch.int32)
        wg.cache_seqlens.copy_(kl)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone())
        eo, el = torch.empty_like(out), torch.empty_like(lse)
        call(eo, el)
        torch.cuda.synchronize()
        assert torch.equal(got[0], eo) and torch.equal(got[1], el)
        wc = w.to("cpu")
        wc.cache_seqlens = kl
        ref_out, ref_lse = ofp8.attention_fp8(wc.q, k8, v8, 1 / 32, 1 / 16, wc.block_table, wc.cache_seqlens,
                                              wc.cu_seqlens_q, wc.softmax_scale, wc.causal, wc.window_size,
                                              wc.rel_extent, wc.rel_logits)
        _compare(got[0].float().cpu().double(), got[1].cpu().double(), ref_out, ref_lse, "fp8 graph replay")


def test_fp8_bad_scales_raise():
    w, k8, v8 = _fp8_workload([1, 1], [100, 200], 32, 8, 128, 0, 0.1, 0.1, seed=23)
    for ks, vs in ((0.0, 0.1), (0.1, -1.0), (float("nan"), 0.1)):
        with pytest.raises(bnd.RpaError):
            _run_fp8(w, k8, v8, ks, vs)


def test_fp8_chunked_prefill_full_size_sampled():
    """The 8-request chunked prefill (H=32, Hkv=8, D=128, R=256) over E4M3
    caches, one split as the benchmark runs it; two requests' tokens (a
    sample of 64 rows each) checked against the oracle."""
    w = wl.chunked_prefill()
    ks, vs = 1 / 32, 1 / 16
    k8 = (w.key_cache.float() / ks).to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = (w.value_cache.float() / vs).to(torch.float8_e4m3fn).view(torch.uint8)
    out, lse = _run_fp8(w, k8, v8, ks, vs, S=1)
    reqs = [2, 6]
    sub, sk8, sv8, qi = _subset(w, k8, v8, reqs)
    g = torch.Generator().manual_seed(3)
    local = sorted(torch.randperm(sub.num_tokens, generator=g)[:128].tolist())
    ref_out, ref_lse = ofp8.attention_fp8(sub.q, sk8, sv8, ks, vs, sub.block_table, sub.cache_seqlens,
                                          sub.cu_seqlens_q, sub.softmax_scale, sub.causal, sub.window_size,
                                          sub.rel_extent, sub.rel_logits, tokens=local)
    li = torch.tensor(local, dtype=torch.long)
    _compare(out[qi][li], lse[qi][li], ref_out[li], ref_lse[li], "chunked_prefill fp8")


def _subset(w, k8, v8, reqs):
    """The requests `reqs` of a workload with only their pages (test
    plumbing: pages are copied, nothing is computed)."""
    BS = w.block_size
    pages, rows, cu, q_idx = [], [], [0], []
    cu_all = w.cu_seqlens_q.tolist()
    for b in reqs:
        n = (w.k_lens[b] + BS - 1) // BS
        rows.append(list(range(len(pages), len(pages) + n)))
        pages += w.block_table[b, :n].tolist()
        q_idx += list(range(cu_all[b], cu_all[b + 1]))
        cu.append(cu[-1] + w.q_lens[b])
    width = max(len(r) for r in rows) + 1
    bt = torch.full((len(reqs), width), -1, dtype=torch.int32)
    for i, r in enumerate(rows):
        bt[i, :len(r)] = torch.tensor(r, dtype=torch.int32)
    idx = torch.tensor(pages, dtype=torch.long)
    qi = torch.tensor(q_idx, dtype=torch.long)
    sub = w.to("cpu")
    sub.q = w.q[qi]
    sub.rel_logits = None if w.rel_logits is None else w.rel_logits[qi]
    sub.block_table = bt
    sub.cache_seqlens = torch.tensor([w.k_lens[b] for b in reqs], dtype=torch.int32)
    sub.cu_seqlens_q = torch.tensor(cu, dtype=torch.int32)
    sub.q_lens = [w.q_lens[b] for b in reqs]
    sub.k_lens = [w.k_lens[b] for b in reqs]
    return sub, k8[idx], v8[idx], qi


def test_fp8_full_size_batched_decode_sampled():
    """The 32-request batched decode (H=32, Hkv=8, D=128, R=128) with E4M3
    caches of its K/V at scales 1/32 and 1/16, in the launch the benchmark
    times (balanced decode); six requests checked against the oracle."""
    w = wl.batched_decode()
    ks, vs = 1 / 32, 1 / 16
    k8 = (w.key_cache.float() / ks).to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = (w.value_cache.float() / vs).to(torch.float8_e4m3fn).view(torch.uint8)
    out, lse = _run_fp8(w, k8, v8, ks, vs)
    reqs = [0, 5, 11, 17, 26, 31]
    sub, sk8, sv8, qi = _subset(w, k8, v8, reqs)
    ref_out, ref_lse = ofp8.attention_fp8(sub.q, sk8, sv8, ks, vs, sub.block_table, sub.cache_seqlens,
                                          sub.cu_seqlens_q, sub.softmax_scale, sub.causal, sub.window_size,
                                          sub.rel_extent, sub.rel_logits)
    _compare(out[qi], lse[qi], ref_out, ref_lse, "batched_decode fp8")


@pytest.mark.parametrize("H,S", [(16, 0), (16, 1), (64, 1)])
def test_fp8_every_code_decodes_exactly(H, S):
    """One key per request: out = v exactly, so every E4M3 code (two kv heads
    of head_dim 128 hold all 256) must come out as its value in bf16, bit for
    bit (NaN codes as NaN), through the balanced decode (S=0), the split-mode
    decode items (S=1, G=8) and the prefill tiles (G=32)."""
    w = wl.build([1, 1], [1, 1], num_heads=H, num_kv_heads=2, head_dim=128, seed=27)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    k8 = torch.full(w.key_cache.shape, 0x38, dtype=torch.uint8)  # keys 1.0: any finite score
    v8 = torch.zeros(w.key_cache.shape, dtype=torch.uint8)
    for b in range(2):
        pg = int(w.block_table[b, 0])
        v8[pg, 0] = codes.view(2, 128)
    out, lse = _run_fp8(w, k8, v8, 1.0, 1.0, S=S)
    want = ofp8.e4m3_decode(codes).view(2, 128)
    G = H // 2
    for tok in range(2):
        for h in range(H):
            got = out[tok, h]
            exp = want[h // G]
            nan = torch.isnan(exp)
            assert torch.equal(torch.isnan(got), nan), f"tok {tok} head {h}: NaN pattern"
            assert torch.equal(got[~nan], exp[~nan]), f"tok {tok} head {h}: decoded values differ"


def test_kv_write_fp8_rounds_the_fp32_quotient():
    """The two values whose exact quotient sits just below an E4M3 midpoint
    while the fp32 quotient is the midpoint: the kernel's codes are the
    oracle's (one fp32 division, then ties to even), not those of rounding
    the exact quotient."""
    import numpy as np
    ks = float(np.array([0x40EE38E4], dtype=np.uint32).view(np.float32)[0])
    vs = float(np.array([0x40EB5AD7], dtype=np.uint32).view(np.float32)[0])
    key = torch.full((1, 1, 128), 50.25, dtype=torch.bfloat16)
    val = torch.full((1, 1, 128), 57.0, dtype=torch.bfloat16)
    slots = torch.zeros((1,), dtype=torch.int64)
    kc = torch.zeros((1, 16, 1, 128), dtype=torch.uint8)
    vc = torch.zeros_like(kc)
    want_k, want_v = ofp8.kv_cache_write_fp8(key, val, slots, kc, vc, ks, vs)
    assert int(want_k[0, 0, 0, 0]) == 0x4E and int(want_v[0, 0, 0, 0]) == 0x50
    kg, vg = kc.cuda(), vc.cuda()
    bnd.rpa_kv_cache_write_fp8(key.cuda(), val.cuda(), slots.cuda(), kg, vg, ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(kg.cpu(), want_k) and torch.equal(vg.cpu(), want_v)
