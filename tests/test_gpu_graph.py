"""Graph capture of the attention call (HIP graphs through torch.cuda.CUDAGraph).

rpa_attn_varlen resolves every work item on the device from cu_seqlens_q,
cache_seqlens and block_table, enqueues only kernel launches (no memset, no
copy, no allocation, no host read of device data), and its grid depends
only on host sizes (batch, num_tokens, num_heads, max_seqlen_q, num_splits,
the CU count).  So one captured call serves every later step whose lengths
change in place on the device, the decode loop the vLLM V1 walkthrough
("vLLM V1 Attention — Part 2", its CUDA-graph remarks) wants to replay.

Each test captures one call, then for several length sets: rewrites the
device metadata and q in place, replays the graph, runs the same call
eagerly into other buffers, and checks that the replay equals the eager
call bit for bit and matches the fp64 oracle to the parity tolerances.
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


def _check_oracle(wc, out, lse, tag, alibi=None):
    ref_out, ref_lse = orc.attention(wc.q, wc.key_cache, wc.value_cache, wc.block_table, wc.cache_seqlens,
                                     wc.cu_seqlens_q, wc.softmax_scale, wc.causal, wc.window_size,
                                     wc.rel_extent, wc.rel_logits, alibi_slopes=alibi)
    out = out.float().cpu().double()
    lse = lse.cpu().double()
    err = (out - ref_out).abs()
    assert err.max().item() <= OUT_MAX, f"{tag}: out max err {err.max().item():.3e}"
    assert err.mean().item() <= OUT_MEAN, f"{tag}: out mean err {err.mean().item():.3e}"
    inf = torch.isinf(ref_lse)
    assert torch.equal(torch.isinf(lse), inf), f"{tag}: lse -inf pattern differs"
    if (~inf).any():
        assert (lse[~inf] - ref_lse[~inf]).abs().max().item() <= LSE_MAX, f"{tag}: lse"


def _run_graph_case(base, S, length_sets, seed, alibi=None):
    """base: a CPU workload whose block table covers the longest lengths of
    every set.  length_sets: list of (q_lens, k_lens) with sum(q_lens) and
    max(q_lens) bounded by base's.  alibi: optional fp32 [H] slopes (CPU)."""
    dev = "cuda"
    w = base.to(dev)
    slopes = None if alibi is None else alibi.to(dev)
    T, H, D = w.q.shape
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    nb = bnd.rpa_workspace_bytes(S, T, H, D) if S != 1 else 0
    ws = torch.empty((max(nb, 1),), dtype=torch.uint8, device=dev)

    def call(o, l):
        bnd.rpa_attn_varlen(w.q, w.key_cache, w.value_cache, block_table=w.block_table,
                            cache_seqlens=w.cache_seqlens, cu_seqlens_q=w.cu_seqlens_q,
                            max_seqlen_q=w.max_seqlen_q, softmax_scale=w.softmax_scale, causal=w.causal,
                            window_size=w.window_size, rel_extent=w.rel_extent, rel_logits=w.rel_logits,
                            num_splits=S, out=o, lse=l, workspace=ws, alibi_slopes=slopes)

    # Warm-up outside the capture (library load, first launches).
    call(out, lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, lse)
    torch.cuda.synchronize()

    gen = torch.Generator().manual_seed(seed)
    for i, (q_lens, k_lens) in enumerate(length_sets):
        assert sum(q_lens) == T and max(q_lens) <= w.max_seqlen_q and len(q_lens) == base.batch
        cu = [0]
        for x in q_lens:
            cu.append(cu[-1] + x)
        # New lengths and new queries, written in place.
        w.cu_seqlens_q.copy_(torch.tensor(cu, dtype=torch.int32))
        w.cache_seqlens.copy_(torch.tensor(k_lens, dtype=torch.int32))
        newq = torch.randn((T, H, D), generator=gen).to(torch.bfloat16)
        w.q.copy_(newq)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_out, got_lse = out.clone(), lse.clone()
        e_out = torch.empty_like(out)
        e_lse = torch.empty_like(lse)
        call(e_out, e_lse)
        torch.cuda.synchronize()
        tag = f"set {i} S={S}"
        assert torch.equal(got_out, e_out), f"{tag}: replay differs from the eager call"
        assert torch.equal(got_lse, e_lse), f"{tag}: replay lse differs from the eager call"
        wc = base.to("cpu")
        wc.q = newq
        wc.cu_seqlens_q = torch.tensor(cu, dtype=torch.int32)
        wc.cache_seqlens = torch.tensor(k_lens, dtype=torch.int32)
        wc.q_lens, wc.k_lens = list(q_lens), list(k_lens)
        _check_oracle(wc, got_out, got_lse, tag, alibi)


def _decode_sets(B, kmax, seed):
    g = torch.Generator().manual_seed(seed)
    sets = []
    for lo, hi in ((kmax // 2, kmax), (1, kmax // 4), (1, kmax)):
        k = torch.randint(lo, hi + 1, (B,), generator=g).tolist()
        sets.append(([1] * B, k))
    return sets


@pytest.mark.parametrize("S", [0, 1, 4])
def test_graph_decode_eight_kv_heads(S):
    B, kmax = 12, 2500
    base = wl.build([1] * B, [kmax] * B, num_heads=32, num_kv_heads=8, head_dim=128, rel_extent=64,
                    seed=11, name="graph_decode8")
    _run_graph_case(base, S, _decode_sets(B, kmax, 1), seed=2)


@pytest.mark.parametrize("S", [0, 3])
def test_graph_decode_two_kv_heads(S):
    B, kmax = 9, 1800
    base = wl.build([1] * B, [kmax] * B, num_heads=8, num_kv_heads=2, head_dim=128, rel_extent=40,
                    seed=12, name="graph_decode2")
    _run_graph_case(base, S, _decode_sets(B, kmax, 3), seed=4)


@pytest.mark.parametrize("S", [1, 2])
def test_graph_mixed_batch(S):
    # 5 requests, 70 tokens, max_seqlen_q 40; the length sets move the prefill
    # chunk between requests and change every KV length.
    base = wl.build([1, 1, 40, 1, 27], [900, 900, 900, 900, 900], num_heads=8, num_kv_heads=2, head_dim=64,
                    rel_extent=32, window_size=(-1, -1), seed=13, name="graph_mixed")
    sets = [([1, 1, 40, 1, 27], [300, 17, 640, 1, 100]),
            ([40, 1, 1, 27, 1], [899, 45, 2, 27, 513]),
            ([27, 40, 1, 1, 1], [30, 40, 800, 65, 5])]
    _run_graph_case(base, S, sets, seed=6)


def test_graph_window_decode():
    B, kmax = 6, 3000
    base = wl.build([1] * B, [kmax] * B, num_heads=16, num_kv_heads=8, head_dim=128, rel_extent=128,
                    window_size=(511, 0), seed=14, name="graph_window")
    _run_graph_case(base, 1, _decode_sets(B, kmax, 5), seed=7)


@pytest.mark.parametrize("S", [1, 3])
def test_graph_mixed_batch_bf16_rel_and_alibi(S):
    # The prefill variant with bf16 rel_logits and ALiBi slopes under replay:
    # band tiles of the moving prefill chunk take the 12-byte group loads in
    # the middle of the array and the per-value form at its ends.
    base = wl.build([1, 1, 48, 1, 30], [1200, 1200, 1200, 1200, 1200], num_heads=8, num_kv_heads=2,
                    head_dim=128, rel_extent=77, window_size=(-1, -1), seed=15, name="graph_mixed_bf16")
    base.rel_logits = base.rel_logits.to(torch.bfloat16)
    sets = [([1, 1, 48, 1, 30], [300, 17, 700, 1, 100]),
            ([48, 1, 1, 30, 1], [1199, 45, 2, 30, 513]),
            ([30, 48, 1, 1, 1], [31, 48, 900, 65, 5])]
    H = base.q.shape[1]
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32)
    _run_graph_case(base, S, sets, seed=8, alibi=slopes)
