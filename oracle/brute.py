"""Pure-Python scalar brute force for tiny inputs.

TEST INFRASTRUCTURE ONLY (see oracle/attention.py).  A second, independent
transcription of the definition in the Inkling FA4 relative-attention
walkthrough (nxmr.cn, "_get_score_mod() 的内部" and the FA4 loop summary):
every (request, query row, head, key) is visited one at a time with Python
floats and ``math.fsum``; the clamp-then-compare form of the score_mod is
applied literally.  It pins the vectorised oracle on small cases and shares
no code with it.
"""
from __future__ import annotations

import math


def _to_lists(x):
    return x.tolist() if hasattr(x, "tolist") else x


def attention(q, key_cache, value_cache, block_table, cache_seqlens, cu_seqlens_q, softmax_scale,
              causal=True, window_size=(-1, -1), rel_extent=0, rel_logits=None, alibi_slopes=None):
    """Nested lists out[T][H][D], lse[T][H] (floats).  Keep inputs tiny."""
    import torch  # only to read tensors; all arithmetic below is scalar Python
    qf = _to_lists(torch.as_tensor(q).double())
    kf = _to_lists(torch.as_tensor(key_cache).double())
    vf = _to_lists(torch.as_tensor(value_cache).double())
    bt = _to_lists(torch.as_tensor(block_table))
    lks = [int(x) for x in _to_lists(torch.as_tensor(cache_seqlens))]
    cu = [int(x) for x in _to_lists(torch.as_tensor(cu_seqlens_q))]
    rl = None if rel_logits is None else _to_lists(torch.as_tensor(rel_logits).double())
    scale = float(torch.tensor(softmax_scale, dtype=torch.float32).item())
    slopes = None if alibi_slopes is None else _to_lists(torch.as_tensor(alibi_slopes, dtype=torch.float32).double())
    T = len(qf)
    H = len(qf[0]) if T else 0
    D = len(qf[0][0]) if T else 0
    BS = len(kf[0])
    Hkv = len(kf[0][0])
    group = H // Hkv
    left, right = int(window_size[0]), int(window_size[1])
    out = [[[0.0] * D for _ in range(H)] for _ in range(T)]
    lse = [[-math.inf] * H for _ in range(T)]
    for b in range(len(lks)):
        lq = cu[b + 1] - cu[b]
        lk = lks[b]
        for i in range(lq):
            tok = cu[b] + i
            pos = lk - lq + i  # absolute position of this query among the keys
            for h in range(H):
                kvh = h // group
                logits = []
                values = []
                for t in range(lk):
                    if causal and t > pos:
                        continue
                    if left >= 0 and t < pos - left:
                        continue
                    if right >= 0 and t > pos + right:
                        continue
                    page = int(bt[b][t // BS])
                    slot = t % BS
                    krow = kf[page][slot][kvh]
                    dot = math.fsum(qf[tok][h][c] * krow[c] for c in range(D))
                    s = scale * dot
                    if rel_extent > 0 and rl is not None:
                        rel_dist = pos - t
                        rel_idx = rel_dist if rel_dist > 0 else 0
                        rel_idx = rel_idx if rel_idx < rel_extent else rel_extent - 1
                        if rel_dist == rel_idx:
                            s += rl[tok][h][rel_idx]
                    if slopes is not None:
                        s += slopes[h] * (t - pos)  # ALiBi: slope times (key position - query position)
                    logits.append(s)
                    values.append(vf[page][slot][kvh])
                if not logits:
                    continue
                m = max(logits)
                ws = [math.exp(s - m) for s in logits]
                z = math.fsum(ws)
                for c in range(D):
                    out[tok][h][c] = math.fsum(w * v[c] for w, v in zip(ws, values)) / z
                lse[tok][h] = m + math.log(z)
    return out, lse
