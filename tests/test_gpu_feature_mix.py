"""GPU parity on seeded random configurations that mix the optional
features — E4M3 caches, ALiBi slopes, bf16 rel_logits — with the shapes of
the main parity suite (decode/prefill mixes, GQA groups, head sizes, block
sizes, windows, non-causal rows, bias extents, split counts), against the
fp64 oracle (the FP8 oracle for E4M3 caches)."""
import pytest
import torch

from oracle import attention as orc
from oracle import fp8 as ofp8
from relative_bias_amd import binding as bnd
from relative_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu

OUT_MAX, OUT_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need a GPU"
    bnd.lib()


def _case(seed):
    g = torch.Generator().manual_seed(2000 + seed)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=g))
    Hkv = [1, 2, 8, 8][ri(0, 3)]
    G = [1, 2, 4, 8][ri(0, 3)]
    D = [64, 128][ri(0, 1)]
    BS = [16, 32, 48][ri(0, 2)]
    B = ri(1, 6)
    q_lens, k_lens = [], []
    decode_only = ri(0, 2) == 0
    for _ in range(B):
        kind = 0 if decode_only else ri(0, 2)
        lq = 1 if kind == 0 else (ri(1, 3) if kind == 1 else ri(4, 160))
        lk = ri(0, 900) + (lq if ri(0, 4) else 0)
        q_lens.append(lq)
        k_lens.append(lk)
    causal = bool(ri(0, 3))
    return dict(q_lens=q_lens, k_lens=k_lens, H=G * Hkv, Hkv=Hkv, D=D, BS=BS, R=[0, 5, 64, 300][ri(0, 3)],
                causal=causal, window=([-1, -1, 31, 200][ri(0, 3)], ([-1, 0][ri(0, 1)] if causal else [-1, 6][ri(0, 1)])),
                S=[0, 0, 1, 3][ri(0, 3)], fp8=bool(ri(0, 1)), alibi=bool(ri(0, 1)), rel_bf16=bool(ri(0, 1)))


@pytest.mark.parametrize("seed", list(range(24)))
def test_feature_mix(seed):
    c = _case(seed)
    w = wl.build(c["q_lens"], c["k_lens"], num_heads=c["H"], num_kv_heads=c["Hkv"], head_dim=c["D"],
                 block_size=c["BS"], rel_extent=c["R"], causal=c["causal"], window_size=c["window"], seed=seed,
                 extra_pages=2)
    if c["rel_bf16"] and w.rel_logits is not None:
        w.rel_logits = w.rel_logits.to(torch.bfloat16)
    H = c["H"]
    g = torch.Generator().manual_seed(seed)
    sl = (torch.rand(H, generator=g) * 0.3).to(torch.float32) if c["alibi"] else None
    args = (w.block_table, w.cache_seqlens, w.cu_seqlens_q, w.softmax_scale, w.causal, w.window_size, w.rel_extent,
            w.rel_logits)
    wg = w.to("cuda")
    common = dict(block_table=wg.block_table, cache_seqlens=wg.cache_seqlens, cu_seqlens_q=wg.cu_seqlens_q,
                  max_seqlen_q=wg.max_seqlen_q, softmax_scale=wg.softmax_scale, causal=wg.causal,
                  window_size=wg.window_size, rel_extent=wg.rel_extent, rel_logits=wg.rel_logits,
                  num_splits=c["S"], return_lse=True, alibi_slopes=None if sl is None else sl.cuda())
    if c["fp8"]:
        ks, vs = 1 / 16, 1 / 8
        k8 = (torch.randn(w.key_cache.shape, generator=g) / ks).to(torch.float8_e4m3fn).view(torch.uint8)
        v8 = (torch.randn(w.key_cache.shape, generator=g) / vs).to(torch.float8_e4m3fn).view(torch.uint8)
        ref_out, ref_lse = ofp8.attention_fp8(w.q, k8, v8, ks, vs, *args, alibi_slopes=sl)
        out, lse = bnd.rpa_attn_varlen_fp8(wg.q, k8.cuda(), v8.cuda(), k_scale=ks, v_scale=vs, **common)
    else:
        ref_out, ref_lse = orc.attention(w.q, w.key_cache, w.value_cache, *args, alibi_slopes=sl)
        out, lse = bnd.rpa_attn_varlen(wg.q, wg.key_cache, wg.value_cache, **common)
    torch.cuda.synchronize()
    out = out.float().cpu().double()
    lse = lse.cpu().double()
    tag = f"seed={seed} {c}"
    assert not torch.isnan(out).any(), tag
    err = (out - ref_out).abs()
    assert err.max().item() <= OUT_MAX, f"{tag}: out max err {err.max().item():.3e}"
    assert err.mean().item() <= OUT_MEAN, f"{tag}: out mean err {err.mean().item():.3e}"
    inf = torch.isinf(ref_lse)
    assert torch.equal(torch.isinf(lse), inf), f"{tag}: lse -inf pattern"
    if inf.any():
        assert (out[inf] == 0).all(), tag
    if (~inf).any():
        assert (lse[~inf] - ref_lse[~inf]).abs().max().item() <= LSE_MAX, f"{tag}: lse"
