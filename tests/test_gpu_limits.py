"""GPU parity at size limits: the balanced decode at 2048 requests (the most
its LDS prefix holds) and 2049 (num_splits = 0 then runs as one split), with
bf16 and E4M3 caches, checked against the oracle on sampled requests; pages
of up to 272 slots."""
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


def _compare(out, lse, ref_out, ref_lse, idx, tag):
    out, lse, ref_out, ref_lse = out[idx], lse[idx], ref_out[idx], ref_lse[idx]
    assert not torch.isnan(ref_out).any()
    err = (out - ref_out).abs()
    assert err.max().item() <= OUT_MAX, f"{tag}: out max err {err.max().item():.3e}"
    assert err.mean().item() <= OUT_MEAN, f"{tag}: out mean err {err.mean().item():.3e}"
    inf = torch.isinf(ref_lse)
    assert torch.equal(torch.isinf(lse), inf)
    if (~inf).any():
        assert (lse[~inf] - ref_lse[~inf]).abs().max().item() <= LSE_MAX, f"{tag}: lse"


def _batch(B, Hkv, seed):
    g = torch.Generator().manual_seed(seed)
    kl = torch.randint(0, 121, (B,), generator=g).tolist()
    return wl.build([1] * B, kl, num_heads=2 * Hkv, num_kv_heads=Hkv, head_dim=64, rel_extent=16, seed=seed)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("B", [2048, 2049])
@pytest.mark.parametrize("Hkv", [2, 8])
@pytest.mark.parametrize("fp8", [False, True])
def test_balanced_decode_batch_limits(B, Hkv, fp8):
    w = _batch(B, Hkv, seed=50 + Hkv)
    sample = sorted(set(torch.randint(0, B, (48,), generator=torch.Generator().manual_seed(B)).tolist()) |
                    {0, B - 1})
    wg = w.to("cuda")
    if fp8:
        g = torch.Generator().manual_seed(51)
        k8 = (torch.randn(w.key_cache.shape, generator=g) * 16).to(torch.float8_e4m3fn).view(torch.uint8)
        v8 = (torch.randn(w.key_cache.shape, generator=g) * 16).to(torch.float8_e4m3fn).view(torch.uint8)
        out, lse = bnd.rpa_attn_varlen_fp8(
            wg.q, k8.cuda(), v8.cuda(), k_scale=1 / 16, v_scale=1 / 16, block_table=wg.block_table,
            cache_seqlens=wg.cache_seqlens, cu_seqlens_q=wg.cu_seqlens_q, max_seqlen_q=1,
            softmax_scale=wg.softmax_scale, rel_extent=wg.rel_extent, rel_logits=wg.rel_logits, num_splits=0,
            return_lse=True)
        ref_out, ref_lse = ofp8.attention_fp8(w.q, k8, v8, 1 / 16, 1 / 16, w.block_table, w.cache_seqlens,
                                              w.cu_seqlens_q, w.softmax_scale, w.causal, w.window_size,
                                              w.rel_extent, w.rel_logits, tokens=sample)
    else:
        out, lse = bnd.attn_workload(wg, num_splits=0)
        ref_out, ref_lse = orc.attention(w.q, w.key_cache, w.value_cache, w.block_table, w.cache_seqlens,
                                         w.cu_seqlens_q, w.softmax_scale, w.causal, w.window_size, w.rel_extent,
                                         w.rel_logits, tokens=sample)
    torch.cuda.synchronize()
    idx = torch.tensor(sample, dtype=torch.long)
    _compare(out.float().cpu().double(), lse.cpu().double(), ref_out, ref_lse, idx,
             f"B={B} Hkv={Hkv} fp8={fp8}")


@pytest.mark.parametrize("BS", [128, 256, 272])
@pytest.mark.parametrize("S", [0, 1, 3])
def test_large_block_sizes(BS, S):
    """Pages of 128, 256 and 272 slots (272: not a power of two) on a mixed
    batch, the balanced decode and split decode items, against the oracle."""
    ql, kl = ([1, 1, 1, 1], [1, 300, 1000, 2700]) if S == 0 else ([1, 90, 1, 33], [2700, 300, 1, 600])
    w = wl.build(ql, kl, num_heads=16, num_kv_heads=8, head_dim=128, block_size=BS, rel_extent=40, seed=60 + BS,
                 extra_pages=1, poison=True)
    ref_out, ref_lse = orc.attention(w.q, w.key_cache, w.value_cache, w.block_table, w.cache_seqlens,
                                     w.cu_seqlens_q, w.softmax_scale, w.causal, w.window_size, w.rel_extent,
                                     w.rel_logits)
    out, lse = bnd.attn_workload(w.to("cuda"), num_splits=S)
    torch.cuda.synchronize()
    idx = torch.arange(w.num_tokens)
    _compare(out.float().cpu().double(), lse.cpu().double(), ref_out, ref_lse, idx, f"BS={BS} S={S}")
