"""GPU parity at full size for the benchmark's variant workloads, in the
launch configuration the benchmark times them: the 1,048,576-token decode
over E4M3 caches, the 32-request batched decode and the 8-request chunked
prefill with ALiBi slopes, and the chunked prefill with bf16 rel_logits.
The oracle computes sampled rows (prefill), sampled kv groups (1M-token
decode) or everything (batched decode).  Tolerances as for the other parity
tests."""
import math

import pytest
import torch

from oracle import attention as orc
from oracle import fp8 as ofp8
from relative_bias_amd import binding as bnd
from relative_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu

OUT_MAX, OUT_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3
K_SCALE, V_SCALE = 1 / 32, 1 / 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need a GPU"
    bnd.lib()


def _slopes(H):
    return torch.tensor([2.0 ** (-8.0 * (i + 1) / H) for i in range(H)], dtype=torch.float32)


def _compare(out, lse, ref_out, ref_lse, tag):
    assert not torch.isnan(ref_out).any(), f"{tag}: oracle rows missing from the comparison set"
    assert not torch.isnan(out).any() and not torch.isnan(lse).any(), f"{tag}: NaN"
    err = (out - ref_out).abs()
    assert err.max().item() <= OUT_MAX, f"{tag}: out max err {err.max().item():.3e}"
    assert err.mean().item() <= OUT_MEAN, f"{tag}: out mean err {err.mean().item():.3e}"
    inf = torch.isinf(ref_lse)
    assert torch.equal(torch.isinf(lse), inf), f"{tag}: lse -inf pattern differs"
    if (~inf).any():
        le = (lse[~inf] - ref_lse[~inf]).abs().max().item()
        assert le <= LSE_MAX, f"{tag}: lse max err {le:.3e}"


def _sample_tokens(w, per_req, seed):
    g = torch.Generator().manual_seed(seed)
    cu = w.cu_seqlens_q.tolist()
    toks = []
    for b in range(w.batch):
        a, e = cu[b], cu[b + 1]
        if e > a:
            toks += [a, e - 1] + [int(x) for x in torch.randint(a, e, (per_req,), generator=g)]
    return sorted(set(toks))


def _oracle(w, **kw):
    return orc.attention(w.q, w.key_cache, w.value_cache, w.block_table, w.cache_seqlens, w.cu_seqlens_q,
                         w.softmax_scale, w.causal, w.window_size, w.rel_extent, w.rel_logits, **kw)


@pytest.mark.timeout(900)
def test_long_decode_fp8_sampled_kv_groups():
    """1M keys, H=64, Hkv=8, R=256 over E4M3 codes of the bf16 caches (scales
    1/32 and 1/16), balanced decode as benchmarked and 16 splits; kv groups 0
    and 7 (q heads 0-7 and 56-63) checked against the oracle on a cache that
    holds only those two kv heads (test plumbing: a slice, nothing computed)."""
    wg = wl.long_decode(device="cuda")
    k8 = (wg.key_cache.float() / K_SCALE).to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = (wg.value_cache.float() / V_SCALE).to(torch.float8_e4m3fn).view(torch.uint8)
    kv_sel, heads = [0, 7], list(range(0, 8)) + list(range(56, 64))
    sk8, sv8 = k8[:, :, kv_sel].cpu(), v8[:, :, kv_sel].cpu()
    hq = torch.tensor(heads)
    q_sub = wg.q[:, hq].cpu()
    rel_sub = wg.rel_logits[:, hq].cpu()
    ref_out, ref_lse = ofp8.attention_fp8(q_sub, sk8, sv8, K_SCALE, V_SCALE, wg.block_table.cpu(),
                                          wg.cache_seqlens.cpu(), wg.cu_seqlens_q.cpu(), wg.softmax_scale,
                                          wg.causal, wg.window_size, wg.rel_extent, rel_sub)
    del sk8, sv8
    for S in (0, 16):
        out, lse = bnd.rpa_attn_varlen_fp8(
            wg.q, k8, v8, k_scale=K_SCALE, v_scale=V_SCALE, block_table=wg.block_table,
            cache_seqlens=wg.cache_seqlens, cu_seqlens_q=wg.cu_seqlens_q, max_seqlen_q=wg.max_seqlen_q,
            softmax_scale=wg.softmax_scale, causal=wg.causal, window_size=wg.window_size,
            rel_extent=wg.rel_extent, rel_logits=wg.rel_logits, num_splits=S, return_lse=True)
        torch.cuda.synchronize()
        _compare(out[:, hq].float().cpu().double(), lse[:, hq].cpu().double(), ref_out, ref_lse,
                 f"long_decode fp8 S={S}")


@pytest.mark.timeout(600)
def test_batched_decode_alibi_full():
    """The 32-request batched decode with slopes 2^(-8 (h + 1) / H), balanced
    decode as benchmarked; every output checked."""
    w = wl.batched_decode()
    sl = _slopes(w.num_heads)
    ref_out, ref_lse = _oracle(w, alibi_slopes=sl)
    out, lse = bnd.attn_workload(w.to("cuda"), num_splits=0, alibi_slopes=sl.cuda())
    torch.cuda.synchronize()
    _compare(out.float().cpu().double(), lse.cpu().double(), ref_out, ref_lse, "batched_decode alibi")


@pytest.mark.timeout(600)
def test_chunked_prefill_alibi_sampled():
    w = wl.chunked_prefill()
    sl = _slopes(w.num_heads)
    toks = _sample_tokens(w, per_req=3, seed=5)
    ref_out, ref_lse = _oracle(w, tokens=toks, alibi_slopes=sl)
    out, lse = bnd.attn_workload(w.to("cuda"), num_splits=1, alibi_slopes=sl.cuda())
    torch.cuda.synchronize()
    idx = torch.tensor(toks)
    _compare(out[idx].float().cpu().double(), lse[idx].cpu().double(), ref_out[idx], ref_lse[idx],
             "chunked_prefill alibi")


@pytest.mark.timeout(600)
def test_chunked_prefill_relbf16_sampled():
    """bf16 rel_logits (the fp32 values rounded to bf16; the oracle reads the
    same bf16 values, widened exactly)."""
    w = wl.chunked_prefill()
    w.rel_logits = w.rel_logits.to(torch.bfloat16)
    toks = _sample_tokens(w, per_req=3, seed=6)
    ref_out, ref_lse = _oracle(w, tokens=toks)
    out, lse = bnd.attn_workload(w.to("cuda"), num_splits=1)
    torch.cuda.synchronize()
    idx = torch.tensor(toks)
    assert not math.isnan(ref_lse[idx].sum().item())
    _compare(out[idx].float().cpu().double(), lse[idx].cpu().double(), ref_out[idx], ref_lse[idx],
             "chunked_prefill relbf16")
