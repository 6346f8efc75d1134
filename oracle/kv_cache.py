"""CPU oracle for the paged KV write that precedes the attention call.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library.

Page cited: [V1-ATTN] "vLLM V1 Attention — Part 2: 标准Attention后端实现"
(devpress.csdn.net):
* 附录O.1, Step 2 (building slot_mapping): the j-th new token of request i,
  which holds seq_len tokens after this step and query_len new ones, sits at
  logical position seq_len - query_len + j; its slot is
  block_tables[i, pos // block_size] * block_size + pos % block_size.
* 6.5 (FlashInferImpl.forward, step 2): the new keys and values, viewed as
  [num_tokens, num_kv_heads, head_size], are written into the
  [num_blocks, block_size, num_kv_heads, head_size] caches at their slots
  (reshape_and_cache_flash).

Readings (also listed in the design notes):
  K1 a token whose position is negative (cache_seqlens < query length, the
     case the attention call treats as rows without keys) gets slot -1;
  K2 a negative slot writes nothing (vLLM's padding convention); a slot at or
     past num_blocks * block_size writes nothing either (the library checks
     it on the device rather than fault);
  K3 slots of one call are distinct (two tokens writing one slot is left
     undefined).
"""
from __future__ import annotations

from typing import Sequence

import torch


def slot_mapping(block_table: torch.Tensor, cache_seqlens: Sequence[int], cu_seqlens_q: Sequence[int],
                 block_size: int) -> torch.Tensor:
    """Slot of every packed query token ([V1-ATTN] 附录O.1 Step 2), int64."""
    bt = block_table.tolist()
    seq_lens = [int(x) for x in cache_seqlens]
    cu = [int(x) for x in cu_seqlens_q]
    out = []
    for i in range(len(seq_lens)):
        q_len = cu[i + 1] - cu[i]
        start = seq_lens[i] - q_len
        for j in range(q_len):
            pos = start + j
            if pos < 0:
                out.append(-1)  # K1
                continue
            page = bt[i][pos // block_size]
            out.append(page * block_size + pos % block_size)
    return torch.tensor(out, dtype=torch.int64)


def kv_cache_write(key: torch.Tensor, value: torch.Tensor, slots: torch.Tensor, key_cache: torch.Tensor,
                   value_cache: torch.Tensor):
    """Copies of the caches with token t's rows written at slot slots[t]
    ([V1-ATTN] 6.5, step 2).  key/value: [T, Hkv, D]; caches:
    [num_blocks, block_size, Hkv, D]."""
    kc = key_cache.clone()
    vc = value_cache.clone()
    nb, bs = kc.shape[0], kc.shape[1]
    for t, s in enumerate(slots.tolist()):
        if s < 0 or s >= nb * bs:  # K2
            continue
        kc[s // bs, s % bs] = key[t]
        vc[s // bs, s % bs] = value[t]
    return kc, vc
