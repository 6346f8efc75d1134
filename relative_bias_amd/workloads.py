"""Seeded synthetic inputs for paged, varlen relative-bias attention.

This module only builds inputs: request lengths, a randomly permuted physical
page pool with its block table, bf16 q/k/v and fp32 rel_logits.  It contains
none of the attention arithmetic, so both the CPU oracle (``oracle/``) and the
HIP path may use it without sharing any of the method's code.

Layouts follow the Inkling FA4 relative-attention walkthrough (nxmr.cn,
"主函数 inkling_fa4_rel_attention", parameter list):

* ``q``            bf16 ``[num_tokens, num_heads, head_dim]`` (varlen packed)
* ``key_cache``    bf16 ``[num_blocks, block_size, num_kv_heads, head_dim]``
* ``value_cache``  same as ``key_cache``
* ``block_table``  int32 ``[batch, max_blocks_per_seq]``, padded with -1
* ``cache_seqlens`` int32 ``[batch]``: KV length including this step's tokens
* ``cu_seqlens_q`` int32 ``[batch + 1]``: prefix sums of the query lengths
* ``rel_logits``   fp32 ``[num_tokens, num_heads, rel_extent]``

Generation order is fixed (lengths, page permutation, q, k, v, rel_logits)
from one ``torch.Generator`` so that a seed names a unique input.  bf16 tensors
are fp32 ``randn`` rounded to nearest even; rel_logits are ``0.5 * randn``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch


@dataclass
class Workload:
    name: str
    q: torch.Tensor
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    block_table: torch.Tensor
    cache_seqlens: torch.Tensor
    cu_seqlens_q: torch.Tensor
    rel_logits: Optional[torch.Tensor]
    q_lens: list
    k_lens: list
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    rel_extent: int
    softmax_scale: float
    causal: bool
    window_size: tuple
    max_seqlen_q: int
    num_splits: Optional[int] = None
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.q_lens)

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.key_cache.shape[0])

    def to(self, device) -> "Workload":
        """Copy every tensor to ``device`` (bit-identical)."""
        def mv(t):
            return None if t is None else t.to(device)
        return Workload(
            name=self.name, q=mv(self.q), key_cache=mv(self.key_cache),
            value_cache=mv(self.value_cache), block_table=mv(self.block_table),
            cache_seqlens=mv(self.cache_seqlens), cu_seqlens_q=mv(self.cu_seqlens_q),
            rel_logits=mv(self.rel_logits), q_lens=list(self.q_lens),
            k_lens=list(self.k_lens), num_heads=self.num_heads,
            num_kv_heads=self.num_kv_heads, head_dim=self.head_dim,
            block_size=self.block_size, rel_extent=self.rel_extent,
            softmax_scale=self.softmax_scale, causal=self.causal,
            window_size=tuple(self.window_size), max_seqlen_q=self.max_seqlen_q,
            num_splits=self.num_splits, meta=dict(self.meta))


def _bf16_randn(shape, gen, device):
    return torch.randn(shape, generator=gen, dtype=torch.float32, device=device).to(torch.bfloat16)


def build(q_lens: Sequence[int], k_lens: Sequence[int], *, num_heads: int, num_kv_heads: int,
          head_dim: int, block_size: int = 16, rel_extent: int = 0, softmax_scale: Optional[float] = None,
          causal: bool = True, window_size=(-1, -1), seed: int = 0, gen: Optional[torch.Generator] = None,
          extra_pages: int = 0, extra_table_cols: int = 1, permute_pages: bool = True,
          poison: bool = False, device: str = "cpu", name: str = "custom",
          num_splits: Optional[int] = None) -> Workload:
    """Build one workload from explicit per-request lengths.

    ``extra_pages`` adds physical pages that no request references; with
    ``poison=True`` those pages and every tail slot past a request's KV length
    hold NaN, which a correct implementation never reads into its result.
    ``device`` selects where the random tensors are drawn (a CUDA generator
    gives different numbers from a CPU one for the same seed).
    """
    q_lens = [int(x) for x in q_lens]
    k_lens = [int(x) for x in k_lens]
    assert len(q_lens) == len(k_lens)
    if gen is None:
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
    B = len(q_lens)
    pages_per_seq = [(lk + block_size - 1) // block_size for lk in k_lens]
    total_pages = sum(pages_per_seq)
    nb = total_pages + extra_pages
    # Page permutation: logical page j of request b -> physical page perm[offset_b + j].
    if permute_pages and nb > 0:
        perm = torch.randperm(nb, generator=gen, device=device).to("cpu", torch.int32)
    else:
        perm = torch.arange(max(nb, 0), dtype=torch.int32)
    width = max(pages_per_seq + [0]) + extra_table_cols
    block_table = torch.full((B, max(width, 1)), -1, dtype=torch.int32)
    off = 0
    for b, npg in enumerate(pages_per_seq):
        if npg:
            block_table[b, :npg] = perm[off:off + npg]
        off += npg
    T = sum(q_lens)
    cu = [0]
    for ql in q_lens:
        cu.append(cu[-1] + ql)
    q = _bf16_randn((T, num_heads, head_dim), gen, device)
    kc = _bf16_randn((max(nb, 1), block_size, num_kv_heads, head_dim), gen, device)
    vc = _bf16_randn((max(nb, 1), block_size, num_kv_heads, head_dim), gen, device)
    rel = None
    if rel_extent > 0:
        rel = 0.5 * torch.randn((T, num_heads, rel_extent), generator=gen, dtype=torch.float32, device=device)
    if poison:
        used = torch.zeros(kc.shape[0], dtype=torch.bool)
        nan = float("nan")
        for b, lk in enumerate(k_lens):
            npg = pages_per_seq[b]
            for j in range(npg):
                pg = int(block_table[b, j])
                used[pg] = True
            if npg and lk % block_size:
                last = int(block_table[b, npg - 1])
                kc[last, lk % block_size:] = nan
                vc[last, lk % block_size:] = nan
        unused = (~used).nonzero().flatten().to(kc.device)
        if unused.numel():
            kc[unused] = nan
            vc[unused] = nan
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    return Workload(
        name=name, q=q, key_cache=kc, value_cache=vc, block_table=block_table.to(device),
        cache_seqlens=torch.tensor(k_lens, dtype=torch.int32, device=device),
        cu_seqlens_q=torch.tensor(cu, dtype=torch.int32, device=device), rel_logits=rel,
        q_lens=q_lens, k_lens=k_lens, num_heads=num_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=block_size, rel_extent=rel_extent,
        softmax_scale=float(softmax_scale), causal=bool(causal),
        window_size=(int(window_size[0]), int(window_size[1])),
        max_seqlen_q=max(q_lens + [0]), num_splits=num_splits,
        meta={"seed": seed})


# ---------------------------------------------------------------------------
# The five named workloads.  Lengths are drawn first from the same generator.
# ---------------------------------------------------------------------------

def _randint(gen, lo, hi_inclusive, n, device):
    return [int(x) for x in torch.randint(lo, hi_inclusive + 1, (n,), generator=gen, device=device).tolist()]


def tiny(seed: int = 0, num_splits: int = 1, device: str = "cpu", poison: bool = False) -> Workload:
    """3 requests, q_lens [1,1,16], cache_seqlens [47,312,128]; H=4, Hkv=2,
    D=64, BS=16, permuted pages, R=32, scale 1/8, causal, no window."""
    return build([1, 1, 16], [47, 312, 128], num_heads=4, num_kv_heads=2, head_dim=64,
                 block_size=16, rel_extent=32, softmax_scale=1.0 / 8.0, causal=True,
                 seed=seed, device=device, name="tiny_mixed", num_splits=num_splits,
                 poison=poison, extra_pages=2 if poison else 0)


def batched_decode(seed: int = 0, device: str = "cpu", batch: int = 32) -> Workload:
    """32 decode requests, cache_seqlens ~ U{1024..8192}; H=32, Hkv=8, D=128,
    BS=16, R=128, causal."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    k_lens = _randint(gen, 1024, 8192, batch, device)
    return build([1] * batch, k_lens, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                 rel_extent=128, causal=True, gen=gen, device=device, name="batched_decode",
                 seed=seed)


def chunked_prefill(seed: int = 0, device: str = "cpu", batch: int = 8) -> Workload:
    """8 requests, q_len ~ U{512..2048}, prior context ~ U{0..4096},
    seqlen_k = context + q_len; H=32, Hkv=8, D=128, BS=16, R=256, causal, S=1."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q_lens = _randint(gen, 512, 2048, batch, device)
    ctx = _randint(gen, 0, 4096, batch, device)
    k_lens = [c + ql for c, ql in zip(ctx, q_lens)]
    return build(q_lens, k_lens, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                 rel_extent=256, causal=True, gen=gen, device=device, name="chunked_prefill",
                 seed=seed, num_splits=1)


def long_decode(seed: int = 0, device: str = "cpu", seqlen_k: int = 1 << 20,
                num_splits: Optional[int] = None) -> Workload:
    """Batch-1 decode over 1,048,576 cached tokens; H=64, Hkv=8, D=128, BS=16,
    65,536 permuted pages, R=256, causal, split-KV."""
    return build([1], [seqlen_k], num_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
                 rel_extent=256, causal=True, seed=seed, device=device, name="long_decode",
                 num_splits=num_splits)


def continuous_batch(seed: int = 0, device: str = "cpu", n_decode: int = 64, n_prefill: int = 4,
                     chunk: int = 1024, context: int = 8192) -> Workload:
    """4 prefill chunks of 1024 tokens on 8192-token prior context, then 64
    decodes with cache_seqlens = floor(exp(U(ln 256, ln 131072))); H=64, Hkv=8,
    D=128, BS=16, window (4095, 0), R=512, causal, one launch."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    u = torch.rand((n_decode,), generator=gen, dtype=torch.float64, device=device).cpu()
    lo, hi = math.log(256.0), math.log(131072.0)
    dec = [int(math.floor(math.exp(lo + (hi - lo) * float(x)))) for x in u]
    dec = [min(max(d, 256), 131072) for d in dec]
    q_lens = [chunk] * n_prefill + [1] * n_decode
    k_lens = [context + chunk] * n_prefill + dec
    return build(q_lens, k_lens, num_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
                 rel_extent=512, causal=True, window_size=(4095, 0), gen=gen, device=device,
                 name="continuous_batch", seed=seed, num_splits=1)


NAMED = {
    "tiny_mixed": tiny,
    "batched_decode": batched_decode,
    "chunked_prefill": chunked_prefill,
    "long_decode": long_decode,
    "continuous_batch": continuous_batch,
}
