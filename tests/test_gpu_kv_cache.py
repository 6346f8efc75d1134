"""GPU parity of the paged KV write (rpa_slot_mapping, rpa_kv_cache_write)
against the CPU oracle in oracle/kv_cache.py: both are integer / copy work,
so every comparison is bit-exact."""
import pytest
import torch

from oracle import kv_cache as okv
from relative_bias_amd import binding as bnd
from relative_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu

SLOT_CASES = {
    # name: (q_lens, k_lens, block_size)
    "decode": ([1, 1, 1, 1], [1, 17, 300, 1024], 16),
    "mixed": ([1, 5, 33, 2], [40, 5, 100, 300], 16),
    "fewer_keys_than_queries": ([5, 1, 3], [2, 9, 0], 16),
    "empty_requests": ([0, 4, 0, 1], [3, 7, 0, 1], 16),
    "block_size_48": ([7, 1, 60], [50, 200, 300], 48),
}


@pytest.mark.parametrize("name", list(SLOT_CASES))
def test_slot_mapping_matches_oracle(name):
    ql, kl, BS = SLOT_CASES[name]
    w = wl.build(ql, kl, num_heads=2, num_kv_heads=1, head_dim=64, block_size=BS, seed=5)
    want = okv.slot_mapping(w.block_table, w.k_lens, w.cu_seqlens_q.tolist(), BS)
    wg = w.to("cuda")
    got = bnd.rpa_slot_mapping(wg.block_table, wg.cache_seqlens, wg.cu_seqlens_q, BS, num_tokens=w.num_tokens)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), want)


def test_slot_mapping_many_requests():
    g = torch.Generator().manual_seed(3)
    B = 700
    ql = [int(x) for x in torch.randint(0, 9, (B,), generator=g)]
    kl = [q + int(x) for q, x in zip(ql, torch.randint(0, 300, (B,), generator=g))]
    w = wl.build(ql, kl, num_heads=2, num_kv_heads=1, head_dim=64, block_size=16, seed=6)
    want = okv.slot_mapping(w.block_table, w.k_lens, w.cu_seqlens_q.tolist(), 16)
    wg = w.to("cuda")
    got = bnd.rpa_slot_mapping(wg.block_table, wg.cache_seqlens, wg.cu_seqlens_q, 16, num_tokens=w.num_tokens)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), want)


def _kv(T, Hkv, D, NB, BS, seed):
    g = torch.Generator().manual_seed(seed)
    key = torch.randn((T, Hkv, D), generator=g).to(torch.bfloat16)
    val = torch.randn((T, Hkv, D), generator=g).to(torch.bfloat16)
    kc = torch.randn((NB, BS, Hkv, D), generator=g).to(torch.bfloat16)
    vc = torch.randn((NB, BS, Hkv, D), generator=g).to(torch.bfloat16)
    return key, val, kc, vc


@pytest.mark.parametrize("T,Hkv,D,NB,BS", [(1, 1, 64, 3, 16), (37, 2, 64, 9, 16), (200, 8, 128, 40, 16),
                                           (65, 4, 128, 5, 48), (300, 8, 64, 20, 32)])
def test_kv_cache_write_matches_oracle(T, Hkv, D, NB, BS):
    """Distinct random slots, with padding (-1) and slots past the cache
    mixed in; both caches are compared whole, bit for bit."""
    key, val, kc, vc = _kv(T, Hkv, D, NB, BS, seed=T + D)
    g = torch.Generator().manual_seed(11 + T)
    slots = torch.randperm(NB * BS, generator=g)[:T].to(torch.int64)
    slots[::7] = -1
    slots[3::11] = NB * BS + 5
    want_k, want_v = okv.kv_cache_write(key, val, slots, kc, vc)
    kg, vg = kc.cuda(), vc.cuda()
    bnd.rpa_kv_cache_write(key.cuda(), val.cuda(), slots.cuda(), kg, vg)
    torch.cuda.synchronize()
    assert torch.equal(kg.cpu(), want_k)
    assert torch.equal(vg.cpu(), want_v)


def test_kv_cache_write_chunked_prefill_shape():
    """The chunked-prefill batch's 8173 tokens written through the slots
    rpa_slot_mapping computes (8 kv heads, head_dim 128)."""
    w = wl.chunked_prefill(device="cpu")
    T = w.num_tokens
    g = torch.Generator().manual_seed(2)
    key = torch.randn((T, 8, 128), generator=g).to(torch.bfloat16)
    val = torch.randn((T, 8, 128), generator=g).to(torch.bfloat16)
    slots = okv.slot_mapping(w.block_table, w.k_lens, w.cu_seqlens_q.tolist(), 16)
    want_k, want_v = okv.kv_cache_write(key, val, slots, w.key_cache, w.value_cache)
    wg = w.to("cuda")
    got_slots = bnd.rpa_slot_mapping(wg.block_table, wg.cache_seqlens, wg.cu_seqlens_q, 16, num_tokens=T)
    bnd.rpa_kv_cache_write(key.cuda(), val.cuda(), got_slots, wg.key_cache, wg.value_cache)
    torch.cuda.synchronize()
    assert torch.equal(got_slots.cpu(), slots)
    assert torch.equal(wg.key_cache.cpu(), want_k)
    assert torch.equal(wg.value_cache.cpu(), want_v)


def test_write_then_attend_reproduces_the_cache():
    """Clearing the step's rows and writing them back through the two entry
    points leaves a cache on which attention gives bit-identical results."""
    w = wl.build([1, 7, 40, 1], [90, 7, 300, 1025], num_heads=16, num_kv_heads=8, head_dim=128,
                 rel_extent=32, seed=8)
    wg = w.to("cuda")
    ref_out, ref_lse = bnd.attn_workload(wg, num_splits=1)
    slots = bnd.rpa_slot_mapping(wg.block_table, wg.cache_seqlens, wg.cu_seqlens_q, w.block_size,
                                 num_tokens=w.num_tokens)
    torch.cuda.synchronize()
    s = slots.cpu()
    bs = w.block_size
    key = torch.stack([w.key_cache[int(x) // bs, int(x) % bs] for x in s]).cuda()
    val = torch.stack([w.value_cache[int(x) // bs, int(x) % bs] for x in s]).cuda()
    for x in s.tolist():
        wg.key_cache[x // bs, x % bs] = 0
        wg.value_cache[x // bs, x % bs] = 0
    bnd.rpa_kv_cache_write(key, val, slots, wg.key_cache, wg.value_cache)
    out, lse = bnd.attn_workload(wg, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(wg.key_cache.cpu(), w.key_cache)
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
