"""Pins for the paged-KV-write oracle (oracle/kv_cache.py).

The slot formula is pinned by the slots worked by hand from [V1-ATTN]
附录O.1 Step 2 (tests/golden/query_positions_v1_appo.json) and by the
attention oracle's own page walk; the write is pinned by reading the tokens
back through the page walk, by what it must leave untouched, and by planted
mistakes.
"""
import json
import os

import torch

from oracle import attention as orc
from oracle import kv_cache as okv
from relative_bias_amd import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_slot_mapping_matches_the_appendix_worked_slots():
    g = _gold("query_positions_v1_appo.json")
    bt = torch.tensor(g["block_tables"], dtype=torch.int32)
    cu = orc.cu_seqlens_from_lengths(g["query_lens"])
    s = okv.slot_mapping(bt, g["seq_lens"], cu, g["block_size"])
    assert s.dtype == torch.int64
    assert s.tolist() == [x for row in g["slots"] for x in row]


def test_slot_mapping_agrees_with_the_page_walk():
    """Every new token's slot is where the attention oracle's page walk
    looks for key seq_len - query_len + j."""
    w = wl.build([1, 5, 33, 2], [40, 5, 100, 300], num_heads=2, num_kv_heads=1, head_dim=8, block_size=16,
                 seed=4)
    s = okv.slot_mapping(w.block_table, w.k_lens, w.cu_seqlens_q.tolist(), 16).tolist()
    cu = w.cu_seqlens_q.tolist()
    for b, (ql, lk) in enumerate(zip(w.q_lens, w.k_lens)):
        pages, _ = orc.page_walk(w.block_table[b].tolist(), lk, 16)
        for j in range(ql):
            pos = lk - ql + j
            assert s[cu[b] + j] == pages[pos // 16] * 16 + pos % 16


def test_slot_mapping_negative_positions_have_no_slot():
    """Lk < Lq: the first Lq - Lk tokens have no cache position (K1)."""
    bt = torch.tensor([[3, 0]], dtype=torch.int32)
    s = okv.slot_mapping(bt, [2], [0, 5], 16)
    assert s.tolist() == [-1, -1, -1, 48, 49]


def test_write_then_read_back_through_the_page_walk():
    w = wl.build([3, 1, 7], [20, 33, 7], num_heads=4, num_kv_heads=2, head_dim=16, block_size=16, seed=9)
    g = torch.Generator().manual_seed(2)
    T = w.num_tokens
    key = torch.randn((T, 2, 16), generator=g).to(torch.bfloat16)
    val = torch.randn((T, 2, 16), generator=g).to(torch.bfloat16)
    s = okv.slot_mapping(w.block_table, w.k_lens, w.cu_seqlens_q.tolist(), 16)
    kc, vc = okv.kv_cache_write(key, val, s, w.key_cache, w.value_cache)
    cu = w.cu_seqlens_q.tolist()
    for b, (ql, lk) in enumerate(zip(w.q_lens, w.k_lens)):
        pages, _ = orc.page_walk(w.block_table[b].tolist(), lk, 16)
        for j in range(ql):
            pos = lk - ql + j
            assert torch.equal(kc[pages[pos // 16], pos % 16], key[cu[b] + j])
            assert torch.equal(vc[pages[pos // 16], pos % 16], val[cu[b] + j])
    # Every other row is unchanged.
    written = set(s.tolist())
    for p in range(kc.shape[0]):
        for o in range(16):
            if p * 16 + o not in written:
                assert torch.equal(kc[p, o], w.key_cache[p, o])
                assert torch.equal(vc[p, o], w.value_cache[p, o])


def test_write_skips_negative_and_out_of_range_slots():
    kc0 = torch.zeros((2, 16, 1, 8), dtype=torch.bfloat16)
    key = torch.ones((3, 1, 8), dtype=torch.bfloat16)
    kc, vc = okv.kv_cache_write(key, 2 * key, torch.tensor([-1, 32, 5]), kc0, kc0)
    assert torch.count_nonzero(kc).item() == 8 and torch.equal(kc[0, 5], key[2])
    assert torch.equal(vc[0, 5], 2 * key[2])
    assert torch.equal(kc0, torch.zeros_like(kc0))  # inputs are not modified


def test_planted_slot_mistakes_are_caught():
    """Slips a slot builder could make (query start at seq_len instead of
    seq_len - query_len; page index by modulo; slot = page + offset) all
    disagree with the appendix's worked slots."""
    g = _gold("query_positions_v1_appo.json")
    BS = g["block_size"]
    want = [x for row in g["slots"] for x in row]

    def build(start_of, page_of, combine):
        out = []
        for row, sl, ql in zip(g["block_tables"], g["seq_lens"], g["query_lens"]):
            for j in range(ql):
                pos = start_of(sl, ql) + j
                out.append(combine(row[page_of(pos)], pos % BS))
        return out

    ok = build(lambda sl, ql: sl - ql, lambda pos: pos // BS, lambda pg, o: pg * BS + o)
    assert ok == want
    assert build(lambda sl, ql: sl - 1, lambda pos: pos // BS, lambda pg, o: pg * BS + o) != want
    assert build(lambda sl, ql: sl - ql, lambda pos: pos % 4, lambda pg, o: pg * BS + o) != want
    assert build(lambda sl, ql: sl - ql, lambda pos: pos // BS, lambda pg, o: pg + o) != want
