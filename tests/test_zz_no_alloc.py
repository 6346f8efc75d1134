"""GPU test of rpa_attn_varlen_noalloc, the entry point for callers that
cannot allocate: called through the C ABI, it must give the same results as
rpa_attn_varlen_ex with a caller-given workspace (bit for bit: same kernels,
same split count), on two calls in a row, the second with a smaller batch,
and it must refuse a call whose partials do not fit its static scratch.
One case is also checked against the fp64 oracle at the parity tolerances.
"""
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


def _lengths(n, lo, hi, seed):
    g = torch.Generator().manual_seed(seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


def _fp8(w, seed, ks=1 / 32, vs=1 / 16):
    g = torch.Generator().manual_seed(seed)
    k8 = (torch.randn(w.key_cache.shape, generator=g) / ks).to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = (torch.randn(w.key_cache.shape, generator=g) / vs).to(torch.float8_e4m3fn).view(torch.uint8)
    return k8, v8, ks, vs


def _both(w, S, fp8=None, alibi=None):
    """(out, lse) of the reference entry point and of the no-alloc one."""
    wg = w.to("cuda")
    T, H, D = w.q.shape
    kc, vc = wg.key_cache, wg.value_cache
    kw = {}
    if fp8 is not None:
        k8, v8, ks, vs = fp8
        kc, vc = k8.cuda(), v8.cuda()
        kw = dict(kv_e4m3=True, k_scale=ks, v_scale=vs)
    al = None if alibi is None else alibi.cuda()
    common = dict(block_table=wg.block_table, cache_seqlens=wg.cache_seqlens, cu_seqlens_q=wg.cu_seqlens_q,
                  max_seqlen_q=wg.max_seqlen_q, softmax_scale=wg.softmax_scale, causal=wg.causal,
                  window_size=wg.window_size, rel_extent=wg.rel_extent, rel_logits=wg.rel_logits,
                  num_splits=S, alibi_slopes=al)
    if fp8 is not None:
        ref = bnd.rpa_attn_varlen_fp8(wg.q, kc, vc, k_scale=kw["k_scale"], v_scale=kw["v_scale"],
                                      return_lse=True, **common)
    else:
        ref = bnd.rpa_attn_varlen(wg.q, kc, vc, return_lse=True, **common)
    out = torch.full((T, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    got = bnd.rpa_attn_varlen_noalloc(wg.q, kc, vc, out=out, lse=lse, **kw, **common)
    torch.cuda.synchronize()
    return ref, got


def _same(ref, got, tag):
    assert torch.equal(ref[0], got[0]), f"{tag}: out differs from rpa_attn_varlen_ex"
    assert torch.equal(ref[1], got[1]), f"{tag}: lse differs from rpa_attn_varlen_ex"


@pytest.mark.parametrize("name,S,H,Hkv,D,R", [
    ("balanced, eight kv heads", 0, 32, 8, 128, 64),
    ("balanced, two kv heads", 0, 16, 2, 128, 32),
    ("balanced, head_dim 64", 0, 8, 8, 64, 16),
    ("five splits", 5, 16, 4, 128, 48),
])
def test_noalloc_matches_workspace_entry_twice(name, S, H, Hkv, D, R):
    """Two calls in a row on the shared scratch, the second on a smaller
    batch; each equals the workspace entry point bit for bit."""
    big = wl.build([1] * 40, _lengths(40, 30, 3000, 1), num_heads=H, num_kv_heads=Hkv, head_dim=D,
                   rel_extent=R, seed=11)
    small = wl.build([1] * 7, _lengths(7, 1, 900, 2), num_heads=H, num_kv_heads=Hkv, head_dim=D,
                     rel_extent=R, seed=12)
    for tag, w in (("first call", big), ("second, smaller call", small)):
        ref, got = _both(w, S)
        _same(ref, got, f"{name}, {tag}")


def test_noalloc_mixed_batch_with_splits_then_smaller():
    """Prefill chunks and decodes in one launch, split into three, then a
    smaller mixed batch split into two."""
    big = wl.build([1, 70, 3, 1, 130], [900, 400, 1203, 17, 2500], num_heads=16, num_kv_heads=4, head_dim=128,
                   rel_extent=40, seed=21)
    small = wl.build([1, 9], [300, 60], num_heads=16, num_kv_heads=4, head_dim=128, rel_extent=40, seed=22)
    _same(*_both(big, 3), "mixed batch, S=3")
    _same(*_both(small, 2), "smaller mixed batch, S=2")


def test_noalloc_e4m3_caches_and_alibi_then_smaller():
    H = 32
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32)
    big = wl.build([1] * 24, _lengths(24, 50, 2500, 3), num_heads=H, num_kv_heads=8, head_dim=128,
                   rel_extent=96, seed=31)
    small = wl.build([1] * 5, _lengths(5, 5, 700, 4), num_heads=H, num_kv_heads=8, head_dim=128,
                     rel_extent=96, seed=32)
    _same(*_both(big, 0, fp8=_fp8(big, 33), alibi=slopes), "E4M3 + ALiBi, balanced")
    _same(*_both(small, 0, fp8=_fp8(small, 34), alibi=slopes), "smaller E4M3 + ALiBi, balanced")


def test_noalloc_matches_the_oracle():
    """The tiny mixed workload of the parity suite through the no-alloc entry,
    at four splits, against the fp64 oracle."""
    w = wl.tiny()
    ref_out, ref_lse = orc.attention(w.q, w.key_cache, w.value_cache, w.block_table, w.cache_seqlens,
                                     w.cu_seqlens_q, w.softmax_scale, w.causal, w.window_size, w.rel_extent,
                                     w.rel_logits)
    _, (out, lse) = _both(w, 4)
    out, lse = out.float().cpu().double(), lse.cpu().double()
    err = (out - ref_out).abs()
    assert err.max().item() <= OUT_MAX and err.mean().item() <= OUT_MEAN
    fin = ~torch.isinf(ref_lse)
    assert torch.equal(torch.isinf(lse), ~fin)
    assert (lse[fin] - ref_lse[fin]).abs().max().item() <= LSE_MAX


def test_noalloc_refuses_partials_beyond_the_scratch():
    """64 splits of 600 tokens x 32 heads x 129 fp32 values need about 630 MB,
    more than the scratch holds: refused before any launch, the output
    untouched."""
    w = wl.build([300, 300], [600, 700], num_heads=32, num_kv_heads=8, head_dim=128, seed=41)
    wg = w.to("cuda")
    T, H, D = w.q.shape
    need = bnd.rpa_workspace_bytes(64, T, H, D)
    assert need > (40 << 20)
    out = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bnd.RpaError) as e:
        bnd.rpa_attn_varlen_noalloc(wg.q, wg.key_cache, wg.value_cache, out=out, block_table=wg.block_table,
                                    cache_seqlens=wg.cache_seqlens, cu_seqlens_q=wg.cu_seqlens_q,
                                    max_seqlen_q=wg.max_seqlen_q, softmax_scale=wg.softmax_scale, num_splits=64)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert not out.any()
    # One split needs no scratch at all.
    got = bnd.rpa_attn_varlen_noalloc(wg.q, wg.key_cache, wg.value_cache, out=out, block_table=wg.block_table,
                                      cache_seqlens=wg.cache_seqlens, cu_seqlens_q=wg.cu_seqlens_q,
                                      max_seqlen_q=wg.max_seqlen_q, softmax_scale=wg.softmax_scale, num_splits=1)
    ref = bnd.rpa_attn_varlen(wg.q, wg.key_cache, wg.value_cache, block_table=wg.block_table,
                              cache_seqlens=wg.cache_seqlens, cu_seqlens_q=wg.cu_seqlens_q,
                              max_seqlen_q=wg.max_seqlen_q, softmax_scale=wg.softmax_scale, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert not math.isnan(got.float().sum().item())
