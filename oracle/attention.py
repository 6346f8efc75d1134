"""fp64 CPU oracle for paged, varlen, causal attention with a relative bias.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library.

It computes the plain definition, materialising the whole score matrix of each
(request, head); it never tiles, never uses an online softmax and never splits
unless asked to emulate split partials.  Pages cited below:

* [FA4-REL]  "vllm中提取Inkling FA4 Relative Attention算子基础的base优化版本"
  (nxmr.cn/news/19446): the op's signature, the score_mod that adds the
  relative bias, and the tiled loop "qk = Q·K·softmax_scale; qk = score_mod;
  online softmax; acc += P·V".
* [V1-ATTN]  "vLLM V1 Attention — Part 2: 标准Attention后端实现"
  (devpress.csdn.net): 附录O (slot mapping and query positions), 附录U
  (block_table page walk), 附录DD (GQA head grouping), 10.x (window masks).
* [PA-V2]    "paged_attention_v2_pytorch.py — BI-V100 PagedAttention V2"
  (dev.modelhub.org.cn): partitioned attention and its phase-2 combine.
* [STEP15]   "Step 15: FlashAttention 封装" (mini-vllm-tutorial): cu_seqlens
  packing and the paged block_table of flash_attn_with_kvcache.

Readings taken where the pages are silent, garbled or disagree (each also
listed in the design notes):
  R1 bias applies iff 0 <= d < R with d = q_abs - kv_pos (the comparison
     operators of the score_mod were lost in extraction; clamping to
     [0, R-1] and keeping the bias only when the clamp did nothing is the
     prose's description).
  R2 s = softmax_scale * <q, k> + bias; the bias is not scaled ([FA4-REL]
     loop order: scale first, then score_mod).
  R3 causal alignment is bottom-right: q_abs = i + Lk - Lq ([FA4-REL]
     score_mod offset seqlen_k - seqlen_q; [V1-ATTN] 附录O start =
     seq_len - query_len).
  R4 window (left, right): visible iff (left < 0 or t >= q_abs - left) and
     (right < 0 or t <= q_abs + right), ANDed with causal; -1 = unbounded.
  R5 rel_extent == 0 means no bias.
  R6 a row with no visible key gives out = 0, lse = -inf.
  R7 split partials are normalised; combine weights by exp(lse_s - LSE)
     (the [PA-V2] phase-2 formula double-weights by the partition sum when
     its partials are unnormalised, so it is not followed literally).
  R8 lse = natural log of the sum of exp of the scaled, biased logits.
  R9 kv head of q head h is h // (H / Hkv) ([V1-ATTN] 附录DD).
  R10 cache_seqlens includes this step's query tokens; only the first
     ceil(Lk / BS) block_table entries are read.
  R11 ALiBi (optional, alibi_slopes fp32 [H]): the logit of key t gains
     slope_h * (t - q_abs), added like the relative bias after scaling
     ([V1-ATTN] FlexAttention chapter, score_modify example 1: scores plus
     slopes times (k_pos - q_pos)).  [PA-V2]'s decode adds slopes times the
     absolute key position instead, which shifts each row by slope_h * q_abs:
     the same softmax, an LSE larger by that shift; the relative form is
     taken.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import torch

__all__ = [
    "page_walk", "cu_seqlens_from_lengths", "query_positions", "visible_mask",
    "bias_matrix", "alibi_matrix", "attention", "attention_split_partials", "combine",
]

_F64 = torch.float64


def cu_seqlens_from_lengths(lengths: Sequence[int]) -> list:
    """Prefix sums [0, l0, l0+l1, ...]; request b owns packed rows
    [cu[b], cu[b+1]).  [STEP15] "cu_seqlens 的具体含义"; [V1-ATTN] 附录Q."""
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return out


def page_walk(block_table_row: Sequence[int], seqlen_k: int, block_size: int):
    """Physical pages holding a request's KV and the fill of its last page.

    Token t lives in page block_table_row[t // block_size] at slot
    t % block_size; a request with seqlen_k tokens uses the first
    ceil(seqlen_k / block_size) entries and its last page holds
    seqlen_k % block_size tokens, or a full page when that is 0.
    [V1-ATTN] 附录U (block_table -> paged_kv_indices / last_page_len);
    [STEP15] flash_attn_with_kvcache block_table example.
    """
    n_pages = (int(seqlen_k) + block_size - 1) // block_size
    pages = [int(block_table_row[j]) for j in range(n_pages)]
    last = 0 if n_pages == 0 else (int(seqlen_k) % block_size or block_size)
    return pages, last


def query_positions(q_len: int, k_len: int) -> torch.Tensor:
    """Absolute KV position of each query row: k_len - q_len + i.
    [V1-ATTN] 附录O Step 2 (logical_pos = seq_len - query_len + j);
    [FA4-REL] score_mod (q_idx + seqlen_k - seqlen_q)."""
    return torch.arange(q_len, dtype=torch.int64) + (int(k_len) - int(q_len))


def visible_mask(qa: torch.Tensor, k_len: int, causal: bool, window_size) -> torch.Tensor:
    """[n, k_len] boolean: which keys each query row may attend to (R3, R4).
    [FA4-REL] window translation (-1,-1) = none; [V1-ATTN] 10.x window mask
    keeps [q - w, q]."""
    left, right = int(window_size[0]), int(window_size[1])
    t = torch.arange(int(k_len), dtype=torch.int64)[None, :]
    q = qa[:, None]
    vis = torch.ones((qa.numel(), int(k_len)), dtype=torch.bool)
    if causal:
        vis &= t <= q
    if left >= 0:
        vis &= t >= q - left
    if right >= 0:
        vis &= t <= q + right
    return vis


def bias_matrix(rel_rows: torch.Tensor, qa: torch.Tensor, k_len: int, rel_extent: int) -> torch.Tensor:
    """[n, k_len] additive bias for one head (R1, R5).

    rel_rows is rel_logits[tok, h, :] for the n query rows.  The distance
    d = q_abs - t indexes it when 0 <= d < rel_extent; elsewhere the bias is
    zero.  [FA4-REL] _get_score_mod: rel_dist, clamp, gather
    rel_logits[global_q_idx, h_idx, rel_idx], zero unless unclamped.
    """
    n = qa.numel()
    if rel_extent <= 0 or n == 0 or k_len == 0:
        return torch.zeros((n, int(k_len)), dtype=_F64)
    d = qa[:, None] - torch.arange(int(k_len), dtype=torch.int64)[None, :]
    band = (d >= 0) & (d < rel_extent)
    idx = d.clamp(0, rel_extent - 1)
    vals = torch.gather(rel_rows.to(_F64), 1, idx)
    return torch.where(band, vals, torch.zeros((), dtype=_F64))


def alibi_matrix(slope: float, qa: torch.Tensor, k_len: int) -> torch.Tensor:
    """[n, k_len] ALiBi bias of one head: slope * (t - q_abs) (R11), with the
    slope taken as its fp32 value."""
    sl = float(torch.tensor(slope, dtype=torch.float32).item())
    t = torch.arange(int(k_len), dtype=_F64)[None, :]
    return sl * (t - qa.to(_F64)[:, None])


def _gather_head(cache: torch.Tensor, pages: list, g: int, k_len: int) -> torch.Tensor:
    """K_b[t] = cache[pages[t // BS], t % BS, g, :] for t < k_len, as fp64."""
    if k_len == 0:
        return torch.zeros((0, cache.shape[-1]), dtype=_F64)
    idx = torch.tensor(pages, dtype=torch.int64)
    rows = cache[idx, :, g, :].reshape(-1, cache.shape[-1])[:k_len]
    return rows.to(_F64)


def _softmax_rows(S: torch.Tensor, V: torch.Tensor):
    """Row softmax of S (with -inf for hidden keys) applied to V, plus lse.
    Rows with no finite entry give (0, -inf) (R6)."""
    n = S.shape[0]
    D = V.shape[1]
    out = torch.zeros((n, D), dtype=_F64)
    lse = torch.full((n,), -math.inf, dtype=_F64)
    if S.shape[1] == 0 or n == 0:
        return out, lse
    m = S.max(dim=1).values
    ok = torch.isfinite(m)
    if ok.any():
        Sk = S[ok]
        mk = m[ok]
        P = torch.exp(Sk - mk[:, None])
        l = P.sum(dim=1)
        out[ok] = (P @ V) / l[:, None]
        lse[ok] = mk + torch.log(l)
    return out, lse


def _iter_requests(cu_seqlens_q, cache_seqlens):
    cu = [int(x) for x in torch.as_tensor(cu_seqlens_q).tolist()]
    lk = [int(x) for x in torch.as_tensor(cache_seqlens).tolist()]
    for b in range(len(lk)):
        yield b, cu[b], cu[b + 1] - cu[b], lk[b]


def _scores(q, K, h, rows_tok, qa, k_len, rel_logits, rel_extent, scale, vis, alibi_slopes=None):
    """Scaled, biased, masked logits of q head h for the given rows (R2, R11)."""
    Q = q[rows_tok, h, :].to(_F64)
    S = (Q @ K.T) * scale
    if rel_extent > 0 and rel_logits is not None:
        S = S + bias_matrix(rel_logits[rows_tok, h, :], qa, k_len, rel_extent)
    if alibi_slopes is not None:
        S = S + alibi_matrix(float(alibi_slopes[h]), qa, k_len)
    return torch.where(vis, S, torch.full((), -math.inf, dtype=_F64))


def attention(q, key_cache, value_cache, block_table, cache_seqlens, cu_seqlens_q, softmax_scale,
              causal=True, window_size=(-1, -1), rel_extent=0, rel_logits=None, *,
              tokens: Optional[Iterable[int]] = None, heads: Optional[Iterable[int]] = None,
              alibi_slopes=None):
    """out [T, H, D] fp64 and lse [T, H] fp64 of the whole method.

    For request b with query rows i (packed token tok = cu[b] + i) and q head
    h of kv head g = h // (H / Hkv):
        s_t = scale * <q[tok, h], K_b[t, g]> + bias(tok, h, q_abs - t)
        out = sum_t softmax(s)_t V_b[t, g],  lse = ln sum_t exp(s_t)
    over the visible keys t.  ``tokens``/``heads`` restrict which outputs are
    computed (the rest stay NaN).  Inputs may be any float dtype on the CPU;
    everything is upcast to fp64 exactly.  ``softmax_scale`` is used as the
    fp32 value handed to the GPU.
    """
    T, H, D = q.shape
    Hkv = key_cache.shape[2]
    BS = key_cache.shape[1]
    assert H % Hkv == 0
    G = H // Hkv
    scale = float(torch.tensor(softmax_scale, dtype=torch.float32).item())
    out = torch.full((T, H, D), math.nan, dtype=_F64)
    lse = torch.full((T, H), math.nan, dtype=_F64)
    want_tok = None if tokens is None else sorted(set(int(t) for t in tokens))
    head_list = list(range(H)) if heads is None else sorted(set(int(h) for h in heads))
    bt = torch.as_tensor(block_table)
    for b, tok0, lq, lk in _iter_requests(cu_seqlens_q, cache_seqlens):
        if lq == 0:
            continue
        local = torch.arange(lq, dtype=torch.int64)
        if want_tok is not None:
            local = torch.tensor([t - tok0 for t in want_tok if tok0 <= t < tok0 + lq], dtype=torch.int64)
            if local.numel() == 0:
                continue
        qa = query_positions(lq, lk)[local]
        rows_tok = local + tok0
        vis = visible_mask(qa, lk, causal, window_size)
        pages, _ = page_walk(bt[b].tolist(), lk, BS)
        for g in sorted(set(h // G for h in head_list)):
            K = _gather_head(key_cache, pages, g, lk)
            V = _gather_head(value_cache, pages, g, lk)
            for h in head_list:
                if h // G != g:
                    continue
                S = _scores(q, K, h, rows_tok, qa, lk, rel_logits, rel_extent, scale, vis, alibi_slopes)
                o, l = _softmax_rows(S, V)
                out[rows_tok, h, :] = o
                lse[rows_tok, h] = l
    return out, lse


def attention_split_partials(q, key_cache, value_cache, block_table, cache_seqlens, cu_seqlens_q,
                             softmax_scale, causal=True, window_size=(-1, -1), rel_extent=0,
                             rel_logits=None, *, num_splits: int):
    """Split emulation: per-split normalised partials (R7).

    The keys [0, Lk) of each request are cut into num_splits contiguous
    chunks of ceil(Lk / num_splits); chunk s gives, for every row, the
    softmax-weighted mean of its visible keys in that chunk and the lse of
    those keys, or (0, -inf) when it has none.  [PA-V2] partitioned
    attention (per-partition max / exp-sum / partial P·V).
    Returns partial_out [S, T, H, D] and partial_lse [S, T, H], fp64.
    """
    T, H, D = q.shape
    Hkv = key_cache.shape[2]
    BS = key_cache.shape[1]
    G = H // Hkv
    S_ = int(num_splits)
    scale = float(torch.tensor(softmax_scale, dtype=torch.float32).item())
    po = torch.zeros((S_, T, H, D), dtype=_F64)
    pl = torch.full((S_, T, H), -math.inf, dtype=_F64)
    bt = torch.as_tensor(block_table)
    for b, tok0, lq, lk in _iter_requests(cu_seqlens_q, cache_seqlens):
        if lq == 0:
            continue
        local = torch.arange(lq, dtype=torch.int64)
        qa = query_positions(lq, lk)
        rows_tok = local + tok0
        vis = visible_mask(qa, lk, causal, window_size)
        pages, _ = page_walk(bt[b].tolist(), lk, BS)
        chunk = max(1, -(-lk // S_)) if lk else 1
        for g in range(Hkv):
            K = _gather_head(key_cache, pages, g, lk)
            V = _gather_head(value_cache, pages, g, lk)
            for h in range(g * G, (g + 1) * G):
                Sfull = _scores(q, K, h, rows_tok, qa, lk, rel_logits, rel_extent, scale, vis)
                for s in range(S_):
                    a, e = s * chunk, min(lk, (s + 1) * chunk)
                    if a >= e:
                        continue
                    o, l = _softmax_rows(Sfull[:, a:e], V[a:e])
                    po[s, rows_tok, h, :] = o
                    pl[s, rows_tok, h] = l
    return po, pl


def combine(partial_out: torch.Tensor, partial_lse: torch.Tensor):
    """Merge normalised split partials (R7).

    LSE = M + ln sum_s exp(lse_s - M) with M = max_s lse_s, and
    out = sum_s exp(lse_s - LSE) * o_s; rows whose every split is empty give
    (0, -inf).  [PA-V2] phase 2 (log-sum-exp rescaling across partitions),
    with the partition sums folded into lse_s.
    """
    po = partial_out.to(_F64)
    pl = partial_lse.to(_F64)
    M = pl.max(dim=0).values
    ok = torch.isfinite(M)
    Msafe = torch.where(ok, M, torch.zeros_like(M))
    w = torch.exp(pl - Msafe[None])
    W = w.sum(dim=0)
    lse = torch.where(ok, Msafe + torch.log(torch.where(ok, W, torch.ones_like(W))),
                      torch.full_like(M, -math.inf))
    wn = torch.where(ok[None], w / torch.where(ok, W, torch.ones_like(W))[None], torch.zeros_like(w))
    out = (wn[..., None] * po).sum(dim=0)
    return out, lse
