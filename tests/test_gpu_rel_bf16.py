"""GPU parity with bf16 rel_logits (rpa_attn_varlen_ex, rel_logits_bf16 = 1)
against the fp64 oracle on the same bf16 values (widened exactly), on every
kernel path, including an odd-sized rel_logits whose last element is the
second half of a dword past the array's end, and together with an E4M3 cache
and ALiBi slopes."""
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


def _compare(out, lse, ref_out, ref_lse, tag):
    assert not torch.isnan(out).any(), f"{tag}: NaN"
    err = (out - ref_out).abs()
    assert err.max().item() <= OUT_MAX, f"{tag}: out max err {err.max().item():.3e}"
    assert err.mean().item() <= OUT_MEAN, f"{tag}: out mean err {err.mean().item():.3e}"
    inf = torch.isinf(ref_lse)
    assert torch.equal(torch.isinf(lse), inf), f"{tag}: lse -inf pattern differs"
    if (~inf).any():
        le = (lse[~inf] - ref_lse[~inf]).abs().max().item()
        assert le <= LSE_MAX, f"{tag}: lse max err {le:.3e}"


CASES = {
    # name: (q_lens, k_lens, H, Hkv, D, R, window, splits)
    "decode_heads8": ([1] * 8, [1, 16, 17, 300, 1024, 2000, 77, 3001], 32, 8, 128, 64, (-1, -1), [0, 3]),
    "decode_pairs_odd": ([1] * 3, [5, 40, 300], 3, 1, 64, 5, (-1, -1), [0, 2]),  # 3*3*5 = 45 elements
    "decode_gqa4": ([1] * 5, [1, 33, 400, 1500, 64], 8, 2, 128, 128, (-1, -1), [0]),
    "prefill_d128": ([300, 77, 129], [900, 77, 1500], 16, 8, 128, 256, (-1, -1), [1, 2]),
    "prefill_d64_odd": ([33, 1], [33, 70], 3, 1, 64, 7, (-1, -1), [1]),  # 34*3*7 = 714 elements
    "mixed_window": ([1, 130, 1, 40, 1], [2000, 500, 70, 3000, 1], 16, 2, 128, 100, (127, 0), [1, 3]),
    # Many band tiles away from the array's ends (the 12-byte group loads) with an odd R, so that
    # groups start at odd and even elements; and MHA rows (G = 1) with a window.
    "prefill_odd_R": ([200, 333], [700, 1000], 8, 2, 128, 257, (-1, -1), [1]),
    "prefill_mha_odd_R": ([150, 90], [400, 300], 4, 4, 64, 33, (63, 0), [1, 2]),
}
PARAMS = [(n, S) for n in CASES for S in CASES[n][-1]]


def _bf16_rel(w):
    return None if w.rel_logits is None else w.rel_logits.to(torch.bfloat16)


@pytest.mark.parametrize("name,S", PARAMS)
def test_bf16_rel_logits_match_oracle(name, S):
    ql, kl, H, Hkv, D, R, win, _ = CASES[name]
    w = wl.build(ql, kl, num_heads=H, num_kv_heads=Hkv, head_dim=D, rel_extent=R, window_size=win, seed=41)
    w.rel_logits = _bf16_rel(w)
    ref_out, ref_lse = orc.attention(w.q, w.key_cache, w.value_cache, w.block_table, w.cache_seqlens,
                                     w.cu_seqlens_q, w.softmax_scale, w.causal, w.window_size, w.rel_extent,
                                     w.rel_logits)
    out, lse = bnd.attn_workload(w.to("cuda"), num_splits=S)
    torch.cuda.synchronize()
    _compare(out.float().cpu().double(), lse.cpu().double(), ref_out, ref_lse, f"{name} S={S}")


def test_bf16_rel_logits_equal_fp32_holding_the_same_values():
    w = wl.build([1] * 6 + [50], [100, 2000, 5, 777, 1500, 64, 300], num_heads=32, num_kv_heads=8, head_dim=128,
                 rel_extent=64, seed=42)
    w.rel_logits = w.rel_logits.to(torch.bfloat16).float()  # fp32 copies of bf16 values
    wg = w.to("cuda")
    a = bnd.attn_workload(wg, num_splits=1)
    wg.rel_logits = wg.rel_logits.to(torch.bfloat16)
    b = bnd.attn_workload(wg, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("S", [0, 1])
def test_bf16_rel_with_fp8_cache_and_alibi(S):
    ql, kl = ([1] * 6, [100, 2000, 5, 777, 1500, 64]) if S == 0 else ([1, 90, 1], [500, 300, 1000])
    w = wl.build(ql, kl, num_heads=32, num_kv_heads=8, head_dim=128, rel_extent=64, seed=43)
    w.rel_logits = _bf16_rel(w)
    g = torch.Generator().manual_seed(44)
    ks, vs = 1 / 32, 1 / 16
    k8 = (torch.randn(w.key_cache.shape, generator=g) / ks).to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = (torch.randn(w.key_cache.shape, generator=g) / vs).to(torch.float8_e4m3fn).view(torch.uint8)
    sl = torch.tensor([2.0 ** (-8.0 * (i + 1) / 32) for i in range(32)], dtype=torch.float32)
    ref_out, ref_lse = ofp8.attention_fp8(w.q, k8, v8, ks, vs, w.block_table, w.cache_seqlens, w.cu_seqlens_q,
                                          w.softmax_scale, w.causal, w.window_size, w.rel_extent, w.rel_logits,
                                          alibi_slopes=sl)
    wg = w.to("cuda")
    out, lse = bnd.rpa_attn_varlen_fp8(
        wg.q, k8.cuda(), v8.cuda(), k_scale=ks, v_scale=vs, block_table=wg.block_table,
        cache_seqlens=wg.cache_seqlens, cu_seqlens_q=wg.cu_seqlens_q, max_seqlen_q=wg.max_seqlen_q,
        softmax_scale=wg.softmax_scale, rel_extent=wg.rel_extent, rel_logits=wg.rel_logits, num_splits=S,
        return_lse=True, alibi_slopes=sl.cuda())
    torch.cuda.synchronize()
    _compare(out.float().cpu().double(), lse.cpu().double(), ref_out, ref_lse, f"fp8+alibi+bf16 rel S={S}")
