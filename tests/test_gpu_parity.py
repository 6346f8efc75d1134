"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances (bf16 inputs, bf16 output, fp32 accumulation):
    out  max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <= 2e-3
    lse  max |gpu - oracle| <= 1e-3, and -inf exactly where the oracle has it.
Small cases are compared element by element on every output; the full-size
workloads, in the split configuration the benchmark times, are compared on
sampled tokens / heads that the oracle computes one by one.
"""
import dataclasses
import math

import pytest
import torch

from oracle import attention as orc
from relative_bias_amd import binding as bnd
from relative_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu

OUT_MAX, OUT_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need a GPU"
    bnd.lib()


def _oracle(w, **kw):
    return orc.attention(w.q, w.key_cache, w.value_cache, w.block_table, w.cache_seqlens,
                         w.cu_seqlens_q, w.softmax_scale, w.causal, w.window_size, w.rel_extent,
                         w.rel_logits, **kw)


def _gpu_run(wg, S, **kw):
    out, lse = bnd.attn_workload(wg, num_splits=S, return_lse=True, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().double(), lse.cpu().double()


def _compare(out, lse, ref_out, ref_lse, tokens=None, heads=None, tag=""):
    if tokens is not None:
        idx = torch.as_tensor(sorted(set(tokens)), dtype=torch.long)
        out, lse, ref_out, ref_lse = out[idx], lse[idx], ref_out[idx], ref_lse[idx]
    if heads is not None:
        hidx = torch.as_tensor(sorted(set(heads)), dtype=torch.long)
        out, lse, ref_out, ref_lse = out[:, hidx], lse[:, hidx], ref_out[:, hidx], ref_lse[:, hidx]
    assert not torch.isnan(ref_out).any(), "oracle rows missing from the comparison set"
    assert not torch.isnan(out).any(), f"{tag}: NaN in GPU output"
    assert not torch.isnan(lse).any(), f"{tag}: NaN in GPU lse"
    err = (out - ref_out).abs()
    assert err.max().item() <= OUT_MAX, f"{tag}: out max err {err.max().item():.3e}"
    assert err.mean().item() <= OUT_MEAN, f"{tag}: out mean err {err.mean().item():.3e}"
    ref_inf = torch.isinf(ref_lse)
    assert torch.equal(torch.isinf(lse), ref_inf), f"{tag}: lse -inf pattern differs"
    if ref_inf.any():
        assert (lse[ref_inf] == -math.inf).all()
        assert (out[ref_inf] == 0).all(), f"{tag}: empty rows must give 0"
    fin = ~ref_inf
    if fin.any():
        le = (lse[fin] - ref_lse[fin]).abs().max().item()
        assert le <= LSE_MAX, f"{tag}: lse max err {le:.3e}"


# ------------------------------------------------------------- small cases

@pytest.mark.parametrize("S", [1, 4])
def test_tiny_mixed_batch(S):
    w = wl.tiny(num_splits=S)
    ref = _oracle(w)
    out, lse = _gpu_run(w.to("cuda"), S)
    _compare(out, lse, *ref, tag=f"tiny S={S}")


CASES = {
    # name: (q_lens, k_lens, H, Hkv, D, BS, R, causal, window)
    "decode_gqa4_d128": ([1, 1, 1, 1], [1, 17, 300, 1024], 8, 2, 128, 16, 64, True, (-1, -1)),
    "decode_gqa8_d128": ([1, 1, 1], [33, 129, 700], 16, 2, 128, 16, 40, True, (-1, -1)),
    "decode_gqa16": ([1, 1], [250, 77], 16, 1, 64, 16, 8, True, (-1, -1)),
    "decode_two_tokens": ([2, 2, 3], [40, 259, 3], 8, 2, 128, 16, 16, True, (-1, -1)),
    "prefill_ragged_d128": ([200, 37, 129], [300, 37, 700], 8, 2, 128, 16, 32, True, (-1, -1)),
    "prefill_ragged_d64": ([150, 65], [150, 400], 6, 2, 64, 16, 5, True, (-1, -1)),
    "prefill_mha": ([70], [130], 4, 4, 128, 32, 12, True, (-1, -1)),
    "prefill_gqa32": ([3, 1], [90, 50], 32, 1, 64, 16, 9, True, (-1, -1)),
    "window_left": ([100, 1, 1], [500, 900, 30], 8, 2, 128, 16, 64, True, (63, 0)),
    "window_both_noncausal": ([40, 1], [200, 120], 4, 2, 64, 16, 10, False, (20, 7)),
    "noncausal_full": ([33, 5], [90, 70], 4, 1, 128, 48, 0, False, (-1, -1)),
    "no_bias": ([50, 1], [200, 333], 8, 2, 128, 16, 0, True, (-1, -1)),
    "bias_wider_than_kv": ([20, 1], [25, 40], 4, 2, 64, 16, 512, True, (-1, -1)),
    "empty_rows": ([5, 0, 3, 1], [2, 10, 0, 0], 4, 2, 64, 16, 4, True, (-1, -1)),
    "block_size_64": ([9, 1], [300, 170], 8, 2, 128, 64, 32, True, (-1, -1)),
    # Bias bands wider than a key tile: full-band tiles, band-only tiles
    # below the diagonal and band-covers-visible tiles at the diagonal.
    "prefill_wide_band": ([300, 97], [700, 500], 8, 2, 128, 16, 130, True, (-1, -1)),
    # Keys past qa visible (right window): band tiles that need both masks.
    "prefill_band_right_window": ([150, 40], [400, 260], 8, 2, 128, 16, 100, False, (-1, 40)),
}


@pytest.mark.parametrize("S", [1, 3, 0])
@pytest.mark.parametrize("name", list(CASES))
def test_small_cases(name, S):
    ql, kl, H, Hkv, D, BS, R, causal, win = CASES[name]
    w = wl.build(ql, kl, num_heads=H, num_kv_heads=Hkv, head_dim=D, block_size=BS, rel_extent=R,
                 causal=causal, window_size=win, seed=sum(map(ord, name)), extra_pages=3, poison=True)
    ref = _oracle(w)
    out, lse = _gpu_run(w.to("cuda"), S)
    _compare(out, lse, *ref, tag=f"{name} S={S}")


@pytest.mark.parametrize("scale", [-0.09, 0.0, 1e-35, 0.3])
@pytest.mark.parametrize("D", [64, 128])
def test_softmax_scale_signs(scale, D):
    """Negative, zero and vanishing scales (the prefill path folds the bias
    into the score accumulator as bias/scale and handles these by negating or
    zeroing Q) and a large one, on prefill and decode rows with the bias band."""
    w = wl.build([90, 1, 1], [200, 150, 70], num_heads=8, num_kv_heads=2, head_dim=D, rel_extent=48,
                 softmax_scale=scale, seed=31, extra_pages=2, poison=True)
    ref = _oracle(w)
    for S in (1, 2):
        out, lse = _gpu_run(w.to("cuda"), S)
        _compare(out, lse, *ref, tag=f"scale={scale} D={D} S={S}")


# Decode-only batches for the balanced decode (num_splits = 0): work cut
# into equal per-CU shares of 16-key units, pairs split across workgroups.
BAL_CASES = {
    # name: (q_lens, k_lens, H, Hkv, D, BS, R, causal, window, scale)
    "fewer_units_than_cus": ([1], [20], 4, 1, 128, 16, 8, True, (-1, -1), None),
    "one_key": ([1, 1], [1, 2], 8, 2, 64, 16, 4, True, (-1, -1), None),
    "long_and_short": ([1, 1, 1], [20000, 3, 900], 16, 2, 128, 16, 128, True, (-1, -1), None),
    "zero_q_and_empty_kv": ([1, 0, 1, 2, 1], [0, 5, 1, 1, 40], 8, 2, 128, 16, 16, True, (-1, -1), None),
    "sixteen_columns": ([4, 2, 1], [300, 57, 1000], 16, 4, 128, 16, 64, True, (-1, -1), None),
    "window_left": ([1, 1, 3], [5000, 200, 2000], 8, 2, 128, 16, 64, True, (255, 0), None),
    "window_both_noncausal": ([2, 1], [300, 120], 4, 2, 64, 16, 10, False, (20, 7), None),
    "bs48_d64": ([1, 1], [1000, 333], 8, 1, 64, 48, 100, True, (-1, -1), None),
    "bs32_no_bias": ([1, 1, 1], [2049, 31, 64], 8, 2, 128, 32, 0, True, (-1, -1), None),
    "gqa16_d64": ([1, 1], [4000, 77], 16, 1, 64, 16, 8, True, (-1, -1), None),
    "bias_wider_than_kv": ([1, 1], [25, 300], 4, 2, 128, 16, 512, True, (-1, -1), None),
    "negative_scale": ([1, 2], [700, 90], 8, 2, 128, 16, 48, True, (-1, -1), -0.09),
    "zero_scale": ([1, 1], [300, 1500], 8, 2, 64, 16, 48, True, (-1, -1), 0.0),
}


@pytest.mark.parametrize("heads8", [False, True], ids=["kv_heads_as_listed", "kv_heads_8"])
@pytest.mark.parametrize("name", list(BAL_CASES))
def test_balanced_decode_cases(name, heads8):
    """heads8 runs the case with eight kv heads (same GQA group size), the
    form where every wave of a workgroup streams its own kv head."""
    ql, kl, H, Hkv, D, BS, R, causal, win, scale = BAL_CASES[name]
    if heads8:
        H, Hkv = H * 8 // Hkv, 8
    kw = {} if scale is None else {"softmax_scale": scale}
    w = wl.build(ql, kl, num_heads=H, num_kv_heads=Hkv, head_dim=D, block_size=BS, rel_extent=R,
                 causal=causal, window_size=win, seed=sum(map(ord, name)), extra_pages=3, poison=True, **kw)
    ref = _oracle(w)
    out, lse = _gpu_run(w.to("cuda"), 0)
    _compare(out, lse, *ref, tag=f"{name} balanced")


@pytest.mark.parametrize("Hkv", [2, 8])
def test_balanced_decode_many_requests(Hkv):
    """More requests than CUs, ragged lengths 0..1500: pieces of many pairs
    per workgroup, and pairs cut across workgroup boundaries."""
    g = torch.Generator().manual_seed(77)
    B = 300
    kl = [int(x) for x in torch.randint(0, 1500, (B,), generator=g)]
    w = wl.build([1] * B, kl, num_heads=4 * Hkv, num_kv_heads=Hkv, head_dim=128, rel_extent=64, seed=78,
                 extra_pages=2, poison=True)
    ref = _oracle(w)
    out, lse = _gpu_run(w.to("cuda"), 0)
    _compare(out, lse, *ref, tag="many requests balanced")


@pytest.mark.parametrize("Hkv", [2, 8])
def test_balanced_decode_repeatable_and_page_permutation_exact(Hkv):
    w = wl.build([1, 1, 2], [5000, 300, 2000], num_heads=4 * Hkv, num_kv_heads=Hkv, head_dim=128,
                 rel_extent=64, seed=41, extra_pages=4)
    wg = w.to("cuda")
    a = bnd.attn_workload(wg, num_splits=0)
    b = bnd.attn_workload(wg, num_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    nb = w.key_cache.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(10))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(nb)
    w2 = w.to("cpu")
    w2.key_cache = w.key_cache[perm].contiguous()
    w2.value_cache = w.value_cache[perm].contiguous()
    bt = w.block_table.clone()
    m = bt >= 0
    bt[m] = inv[bt[m].long()].int()
    w2.block_table = bt
    c = bnd.attn_workload(w2.to("cuda"), num_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])


def test_many_splits_with_short_ranges():
    """More splits than key tiles: most splits are empty and give (0, -inf)
    partials that the combine must ignore."""
    w = wl.build([1, 4, 1], [20, 90, 600], num_heads=8, num_kv_heads=2, head_dim=128, rel_extent=16,
                 seed=5)
    ref = _oracle(w)
    out, lse = _gpu_run(w.to("cuda"), 128)
    _compare(out, lse, *ref, tag="S=128")


def test_split_combine_entry_point():
    g = torch.Generator().manual_seed(3)
    S, T, H, D = 5, 7, 3, 128
    po = torch.randn((S, T, H, D), generator=g, dtype=torch.float32)
    pl = 3 * torch.randn((S, T, H), generator=g, dtype=torch.float32)
    pl[:, 0, 0] = -math.inf       # every split empty
    pl[1:, 1, 1] = -math.inf      # one split only
    pl[2, 2, 2] = -math.inf
    po[pl == -math.inf] = 0
    ref_o, ref_l = orc.combine(po.double(), pl.double())
    out, lse = bnd.rpa_split_combine(po.cuda(), pl.cuda())
    torch.cuda.synchronize()
    _compare(out.float().cpu().double(), lse.cpu().double(), ref_o, ref_l, tag="combine")


def test_split_combine_ignores_nan_in_empty_splits():
    """A split with lse = -inf has weight 0: its partial row is skipped, so a
    NaN there (external partials need not zero their empty splits) does not
    reach the output."""
    g = torch.Generator().manual_seed(4)
    S, T, H, D = 6, 9, 4, 128
    po = torch.randn((S, T, H, D), generator=g, dtype=torch.float32)
    pl = 2 * torch.randn((S, T, H), generator=g, dtype=torch.float32)
    pl[:, 0, 0] = -math.inf       # every split empty
    pl[1:, 1, 1] = -math.inf      # one split only
    pl[::2, 3] = -math.inf        # every other split of a token
    empty = pl == -math.inf
    clean = po.clone()
    clean[empty] = 0
    ref_o, ref_l = orc.combine(clean.double(), pl.double())
    po[empty] = math.nan
    out, lse = bnd.rpa_split_combine(po.cuda(), pl.cuda())
    torch.cuda.synchronize()
    _compare(out.float().cpu().double(), lse.cpu().double(), ref_o, ref_l, tag="combine with NaN partials")


def test_wrappers_refuse_wrong_output_shapes():
    """Caller-supplied out / lse of another shape are refused before any
    launch (the kernels would write T*H*D and T*H values)."""
    w = wl.build([1, 3], [40, 70], num_heads=4, num_kv_heads=2, head_dim=64, rel_extent=8, seed=2)
    wg = w.to("cuda")
    T, H, D = w.q.shape
    small_out = torch.empty((T - 1, H, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="out must be"):
        bnd.attn_workload(wg, num_splits=1, out=small_out)
    small_lse = torch.empty((T, H - 1), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="lse must be"):
        bnd.attn_workload(wg, num_splits=1, lse=small_lse)
    po = torch.zeros((2, T, H, D), device="cuda")
    pl = torch.zeros((2, T, H), device="cuda")
    with pytest.raises(ValueError, match="out must be"):
        bnd.rpa_split_combine(po, pl, out=small_out)
    with pytest.raises(ValueError, match="needs out or num_tokens"):
        bnd.rpa_slot_mapping(wg.block_table, wg.cache_seqlens, wg.cu_seqlens_q, 16)


# --------------------------------------------------------------- invariants

def test_bitwise_repeatable_and_page_permutation_exact():
    w = wl.build([1, 70, 1], [500, 300, 2000], num_heads=8, num_kv_heads=2, head_dim=128,
                 rel_extent=64, seed=21, extra_pages=4)
    wg = w.to("cuda")
    a = bnd.attn_workload(wg, num_splits=4)
    b = bnd.attn_workload(wg, num_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # Physically permute the pages and remap the table: same bits.
    nb = w.key_cache.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(9))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(nb)
    w2 = w.to("cpu")
    w2.key_cache = w.key_cache[perm].contiguous()
    w2.value_cache = w.value_cache[perm].contiguous()
    bt = w.block_table.clone()
    m = bt >= 0
    bt[m] = inv[bt[m].long()].int()
    w2.block_table = bt
    c = bnd.attn_workload(w2.to("cuda"), num_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])


def test_nan_poison_changes_no_bits():
    kw = dict(num_heads=8, num_kv_heads=2, head_dim=128, rel_extent=32, seed=22, extra_pages=3)
    a = wl.build([1, 40], [333, 97], poison=False, **kw)
    b = wl.build([1, 40], [333, 97], poison=True, **kw)
    for S in (1, 2):
        oa = bnd.attn_workload(a.to("cuda"), num_splits=S)
        ob = bnd.attn_workload(b.to("cuda"), num_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(oa[0], ob[0]) and torch.equal(oa[1], ob[1])


def test_split_count_invariance():
    w = wl.build([1, 1, 30], [3000, 1500, 2048], num_heads=16, num_kv_heads=2, head_dim=128,
                 rel_extent=128, seed=23).to("cuda")
    base = _gpu_run(w, 1)
    for S in (2, 7, 16, 64, 0):
        o, l = _gpu_run(w, S)
        assert (o - base[0]).abs().max().item() <= 1e-2
        fin = torch.isfinite(base[1])
        assert (l[fin] - base[1][fin]).abs().max().item() <= 1e-4


def test_zero_bias_equals_no_bias_on_gpu():
    w = wl.build([1, 50], [700, 300], num_heads=8, num_kv_heads=2, head_dim=128, rel_extent=64, seed=24)
    wg = w.to("cuda")
    a = bnd.attn_workload(wg, num_splits=2)
    wg.rel_logits.zero_()
    b = bnd.attn_workload(wg, num_splits=2)
    wg.rel_extent, wg.rel_logits = 0, None
    c = bnd.attn_workload(wg, num_splits=2)
    torch.cuda.synchronize()
    # Same values up to fp32 rounding: the bias-free tile variant may contract
    # the scale and the max subtraction into one FMA, the bias variant cannot.
    assert (b[0].float() - c[0].float()).abs().max().item() <= 8e-3
    assert (b[1] - c[1]).abs().max().item() <= 1e-5
    assert not torch.equal(a[0], b[0])


# ------------------------------------------------- full-size workloads

def _sample_tokens(w, per_req=4, seed=0):
    g = torch.Generator().manual_seed(seed)
    cu = w.cu_seqlens_q.tolist()
    toks = []
    for b in range(w.batch):
        a, e = cu[b], cu[b + 1]
        if e <= a:
            continue
        toks += [a, e - 1]
        toks += [int(x) for x in torch.randint(a, e, (per_req,), generator=g)]
    return sorted(set(toks))


@pytest.mark.timeout(600)
def test_batched_decode_full():
    w = wl.batched_decode()
    S = bnd.rpa_choose_splits(w.batch, 1, w.num_heads, w.num_kv_heads, max(w.k_lens))
    ref = _oracle(w)
    out, lse = _gpu_run(w.to("cuda"), S)
    _compare(out, lse, *ref, tag=f"batched_decode S={S}")


@pytest.mark.timeout(600)
def test_chunked_prefill_sampled():
    w = wl.chunked_prefill()
    toks = _sample_tokens(w, per_req=3)
    ref = _oracle(w, tokens=toks)
    out, lse = _gpu_run(w.to("cuda"), 1)
    _compare(out, lse, *ref, tokens=toks, tag="chunked_prefill")


@pytest.mark.timeout(600)
def test_continuous_batch_sampled():
    w = wl.continuous_batch()
    cu = w.cu_seqlens_q.tolist()
    toks = _sample_tokens(w, per_req=2)
    toks = [t for t in toks if t < cu[4]] + list(range(cu[4], cu[-1], 4))
    ref = _oracle(w, tokens=toks)
    out, lse = _gpu_run(w.to("cuda"), 1)
    _compare(out, lse, *ref, tokens=toks, tag="continuous_batch")


@pytest.mark.timeout(600)
def test_long_decode_sampled_heads():
    """1,048,576-token decode, generated on the GPU; the oracle checks two kv
    groups (16 q heads) for the split counts the benchmark times: the
    planner's (balanced) and 16, 32, 64 and 128 partitions (the range the
    walkthrough's planner caps at through 1M KV tokens)."""
    wg = wl.long_decode(device="cuda")
    heads = list(range(0, 8)) + list(range(56, 64))
    wc = wg.to("cpu")
    ref = _oracle(wc, heads=heads)
    del wc
    for S in (bnd.rpa_choose_splits(1, 1, 64, 8, 1 << 20), 16, 32, 64, 128):
        out, lse = _gpu_run(wg, S)
        _compare(out, lse, *ref, heads=heads, tag=f"long_decode S={S}")


# ------------------------------------------------------ seeded random cases

def _random_case(seed):
    """A seeded random configuration: batch mix of decode and prefill
    requests, GQA group, head_dim, block size, bias extent, mask and scale."""
    g = torch.Generator().manual_seed(1000 + seed)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=g))
    Hkv = [1, 2, 4, 8][ri(0, 3)]
    G = [1, 2, 4, 8][ri(0, 3)]
    D = [64, 128][ri(0, 1)]
    BS = [16, 32, 48][ri(0, 2)]
    B = ri(1, 6)
    q_lens, k_lens = [], []
    for _ in range(B):
        kind = ri(0, 2)
        lq = 1 if kind == 0 else (ri(1, 3) if kind == 1 else ri(4, 160))
        lk = ri(0, 700) + (lq if ri(0, 4) else 0)
        q_lens.append(lq)
        k_lens.append(lk)
    R = [0, 1, 7, 64, 300][ri(0, 4)]
    causal = bool(ri(0, 3))
    left = [-1, -1, 0, 37, 200][ri(0, 4)]
    right = [-1, 0, 0, 5][ri(0, 3)] if not causal else [-1, 0][ri(0, 1)]
    scale = [None, None, 0.05, -0.08][ri(0, 3)]
    S = [1, 1, 2, 5, 0][ri(0, 4)]
    return dict(q_lens=q_lens, k_lens=k_lens, H=G * Hkv, Hkv=Hkv, D=D, BS=BS, R=R, causal=causal,
                window=(left, right), scale=scale, S=S)


@pytest.mark.parametrize("G", [64, 128, 256])
def test_large_gqa_groups(G):
    """GQA groups of 64 to 256 query heads per kv head: a 128-row q-tile
    holds two tokens, one token or half of one token's heads; decode tokens
    run as prefill q-tiles (more than 16 columns)."""
    w = wl.build([3, 1, 20, 0], [50, 200, 40, 7], num_heads=G, num_kv_heads=1, head_dim=64, rel_extent=9,
                 seed=G, extra_pages=2, poison=True)
    ref = _oracle(w)
    for S in (1, 2):
        out, lse = _gpu_run(w.to("cuda"), S)
        _compare(out, lse, *ref, tag=f"G={G} S={S}")


@pytest.mark.parametrize("causal", [True, False])
def test_windows_past_every_key(causal):
    """Window sides that reach past every key (up to 2^31 - 1) give exactly
    the unbounded result, rows with Lk < Lq included; sides just short of
    that reach still match the oracle."""
    w = wl.build([1, 40, 3, 90], [300, 97, 3, 60], num_heads=8, num_kv_heads=2, head_dim=64, rel_extent=24,
                 causal=causal, seed=31)
    wg = w.to("cuda")
    base = _gpu_run(dataclasses.replace(wg, window_size=(-1, -1)), 1)
    big = 2 ** 31 - 1
    for win in [(big, big), (big, -1), (-1, big), (big, 0)]:
        got = _gpu_run(dataclasses.replace(wg, window_size=win), 1)
        if win[1] != 0:
            assert torch.equal(got[0], base[0]) and torch.equal(got[1], base[1]), f"window {win}"
        ref = _oracle(dataclasses.replace(w, window_size=win))
        _compare(*got, *ref, tag=f"window {win} causal={causal}")
    # The widest sides the device still applies: max_pages_per_seq * block_size - 1
    # on the left, max_seqlen_q - 1 on the right.
    win = (w.block_table.shape[1] * w.block_size - 1, w.max_seqlen_q - 1)
    got = _gpu_run(dataclasses.replace(wg, window_size=win), 1)
    _compare(*got, *_oracle(dataclasses.replace(w, window_size=win)), tag=f"window {win} causal={causal}")


@pytest.mark.parametrize("B", [63, 64, 65])
def test_prefill_request_order_edges(B):
    """Batches at the 64-request limit of the longest-first order of prefill
    requests (65 keeps request order): prefill requests of equal KV lengths
    (ties), empty query ranges and decode requests mixed in, a window on half
    of the cases.  Every q-tile must be computed exactly once."""
    g = torch.Generator().manual_seed(500 + B)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=g))
    q_lens, k_lens = [], []
    for i in range(B):
        kind = ri(0, 3)
        lq = 0 if kind == 0 else (ri(1, 4) if kind == 1 else ri(5, 90))
        lk = (300 if i % 5 == 0 else ri(0, 400)) + lq
        q_lens.append(lq)
        k_lens.append(lk)
    window = (63, 0) if B % 2 else (-1, -1)
    w = wl.build(q_lens, k_lens, num_heads=8, num_kv_heads=2, head_dim=64, rel_extent=40, window_size=window,
                 seed=B, extra_pages=2, poison=True)
    ref = _oracle(w)
    out, lse = _gpu_run(w.to("cuda"), 1)
    _compare(out, lse, *ref, tag=f"request order B={B}")


@pytest.mark.parametrize("seed", list(range(24)))
def test_random_configurations(seed):
    """Parity on 24 seeded random configurations (mixed decode and prefill
    batches, every GQA group size, both head sizes, three block sizes,
    windows, bias extents from 0 to 300, negative and small scales, split
    counts 0/1/2/5)."""
    cfg = _random_case(seed)
    kw = {} if cfg["scale"] is None else {"softmax_scale": cfg["scale"]}
    w = wl.build(cfg["q_lens"], cfg["k_lens"], num_heads=cfg["H"], num_kv_heads=cfg["Hkv"], head_dim=cfg["D"],
                 block_size=cfg["BS"], rel_extent=cfg["R"], causal=cfg["causal"], window_size=cfg["window"],
                 seed=seed, extra_pages=2, poison=True, **kw)
    ref = _oracle(w)
    out, lse = _gpu_run(w.to("cuda"), cfg["S"])
    _compare(out, lse, *ref, tag=f"random seed={seed} {cfg}")
