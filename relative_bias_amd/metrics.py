"""Algorithmic work of one attention call, from host-side lengths only.

bytes = K and V of every key visible to at least one row of a request, read
        once per kv head (2 * Hkv * D * kv_elem_bytes B per key: 2 for bf16
        caches, 1 for E4M3 caches)
      + q and out (bf16), lse (fp32)
      + the rel_logits entries inside the bias band of visible keys (4 B each,
        2 B when the workload's rel_logits are bf16)
      + one int32 block_table entry per page touched, and the length arrays.
flops = 4 * D * (number of visible (query row, key) pairs) * H  (Q·Kᵀ and P·V;
        exp, bias and masking are not counted).
Split partials, re-reads and masked or padded work are implementation
overhead and are not counted.
"""
from __future__ import annotations


def _row_bounds(qa: int, lk: int, causal: bool, left: int, right: int):
    lo, hi = 0, lk - 1
    if causal:
        hi = min(hi, qa)
    if left >= 0:
        lo = max(lo, qa - left)
    if right >= 0:
        hi = min(hi, qa + right)
    return lo, hi


def work(w, kv_elem_bytes: int = 2) -> dict:
    H, Hkv, D, BS, R = w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, w.rel_extent
    left, right = w.window_size
    kv_bytes = 0
    page_bytes = 0
    pairs = 0
    band = 0
    for lq, lk in zip(w.q_lens, w.k_lens):
        if lq == 0 or lk == 0:
            continue
        umin, umax = None, None
        for i in range(lq):
            qa = i + lk - lq
            lo, hi = _row_bounds(qa, lk, w.causal, left, right)
            if hi < lo:
                continue
            pairs += hi - lo + 1
            if R > 0:
                blo, bhi = max(lo, qa - R + 1), min(hi, qa)
                if bhi >= blo:
                    band += bhi - blo + 1
            umin = lo if umin is None else min(umin, lo)
            umax = hi if umax is None else max(umax, hi)
        if umin is not None:
            kv_bytes += (umax - umin + 1) * Hkv * D * 2 * kv_elem_bytes
            page_bytes += (umax // BS - umin // BS + 1) * 4
    T = sum(w.q_lens)
    qo_bytes = 2 * T * H * D * 2
    lse_bytes = T * H * 4
    rel = getattr(w, "rel_logits", None)
    rel_eb = 2 if rel is not None and str(getattr(rel, "dtype", "")) == "torch.bfloat16" else 4
    rel_bytes = band * H * rel_eb
    meta_bytes = (2 * len(w.q_lens) + 1) * 4
    total = kv_bytes + qo_bytes + lse_bytes + rel_bytes + page_bytes + meta_bytes
    return {
        "bytes": total, "kv_bytes": kv_bytes, "qo_bytes": qo_bytes, "rel_bytes": rel_bytes,
        "lse_bytes": lse_bytes, "page_bytes": page_bytes, "pairs": pairs * H,
        "flops": 4 * D * pairs * H,
    }
