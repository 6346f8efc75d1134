"""Pins for the CPU oracle: worked examples from the pages, closed forms,
a library routine (float64 SDPA), a scalar brute force, and invariants.

Each pin is chosen so that a plausible slip in the oracle (dropped bias,
scaled bias, reversed distance, wrong query offset, kv-head mapping by
modulo, wrong page lookup, missing mask) fails at least one of them; the
planted-mistake tests at the bottom check that claim for several slips.
"""
import json
import math
import os

import pytest
import torch

from oracle import attention as orc
from oracle import brute
from relative_bias_amd import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _run(w, **kw):
    return orc.attention(w.q, w.key_cache, w.value_cache, w.block_table, w.cache_seqlens,
                         w.cu_seqlens_q, w.softmax_scale, w.causal, w.window_size, w.rel_extent,
                         w.rel_logits, **kw)


def _brute(w):
    out, lse = brute.attention(w.q, w.key_cache, w.value_cache, w.block_table, w.cache_seqlens,
                               w.cu_seqlens_q, w.softmax_scale, w.causal, w.window_size,
                               w.rel_extent, w.rel_logits)
    return torch.tensor(out, dtype=torch.float64), torch.tensor(lse, dtype=torch.float64)


def _assert_close(a, b, tol=1e-12):
    a = torch.as_tensor(a, dtype=torch.float64)
    b = torch.as_tensor(b, dtype=torch.float64)
    fa, fb = torch.isfinite(a), torch.isfinite(b)
    assert torch.equal(fa, fb), "finite/inf pattern differs"
    assert torch.equal(a[~fa], b[~fb]), "non-finite values differ"
    if fa.any():
        err = (a[fa] - b[fb]).abs().max().item()
        assert err <= tol, f"max abs err {err} > {tol}"


# ----------------------------------------------------------------- goldens

@pytest.mark.parametrize("name", ["cu_seqlens_step15.json", "cu_seqlens_v1_appq.json"])
def test_cu_seqlens_golden(name):
    g = _gold(name)
    assert orc.cu_seqlens_from_lengths(g["lengths"]) == g["cu_seqlens"]
    w = wl.build([int(x) for x in g["lengths"]], [int(x) for x in g["lengths"]], num_heads=1,
                 num_kv_heads=1, head_dim=8)
    assert w.cu_seqlens_q.tolist() == g["cu_seqlens"]


def test_page_walk_v1_appu():
    g = _gold("page_walk_v1_appu.json")
    indptr, indices, last = [0], [], []
    for row, sl in zip(g["block_tables"], g["seq_lens"]):
        pages, lp = orc.page_walk(row, sl, g["block_size"])
        indices += pages
        indptr.append(len(indices))
        last.append(lp)
    assert indptr == g["paged_kv_indptr"]
    assert indices == g["paged_kv_indices"]
    assert last == g["paged_kv_last_page_len"]


def test_page_walk_step15_zero_padding():
    g = _gold("page_walk_step15_zero_pad.json")
    for row, sl, want in zip(g["block_table"], g["cache_seqlens"], g["pages"]):
        pages, lp = orc.page_walk(row, sl, g["block_size"])
        assert pages == want
        assert lp == g["block_size"]


def test_query_positions_and_slots_v1_appo():
    g = _gold("query_positions_v1_appo.json")
    BS = g["block_size"]
    for b, (row, sl, ql) in enumerate(zip(g["block_tables"], g["seq_lens"], g["query_lens"])):
        qa = orc.query_positions(ql, sl).tolist()
        assert qa == g["positions"][b]
        pages, _ = orc.page_walk(row, sl, BS)
        assert [pages[p // BS] * BS + p % BS for p in qa] == g["slots"][b]
        vis = orc.visible_mask(torch.tensor(qa), sl, True, (-1, -1))
        assert vis.sum(dim=1).tolist() == g["visible_keys_causal"][b]


def test_query_positions_drive_the_result():
    """With every key identical and no bias, row i of a request averages
    exactly the values at positions 0..q_abs(i): pins the bottom-right
    offset inside the full oracle, on the appendix geometry."""
    g = _gold("query_positions_v1_appo.json")
    w = wl.build(g["query_lens"], g["seq_lens"], num_heads=2, num_kv_heads=1, head_dim=8,
                 block_size=g["block_size"], seed=3)
    w.key_cache[:] = w.key_cache[0, 0, 0]
    out, _ = _run(w)
    cu = w.cu_seqlens_q.tolist()
    for b, (sl, ql) in enumerate(zip(g["seq_lens"], g["query_lens"])):
        pages, _ = orc.page_walk(w.block_table[b].tolist(), sl, w.block_size)
        V = torch.stack([w.value_cache[pages[t // 16], t % 16, 0].double() for t in range(sl)])
        for i, pos in enumerate(g["positions"][b]):
            _assert_close(out[cu[b] + i, 0], V[: pos + 1].mean(0), 1e-12)


def test_two_key_softmax_golden():
    g = _gold("two_key_softmax.json")
    ev = {"ln3-1": math.log(3.0) - 1.0, "ln5": math.log(5.0), "ln4": math.log(4.0),
          "ln6": math.log(6.0), "1/6": 1 / 6, "5/6": 5 / 6}

    def num(x):
        if isinstance(x, list):
            return [num(y) for y in x]
        return ev[x] if isinstance(x, str) else float(x)

    q = torch.tensor(num(g["q"]), dtype=torch.float64)
    kc = torch.zeros((1, g["block_size"], 1, 2), dtype=torch.float64)
    vc = torch.zeros_like(kc)
    kc[0, :2] = torch.tensor(num(g["k_page"]))
    vc[0, :2] = torch.tensor(num(g["v_page"]))
    rel = torch.tensor(num(g["rel_logits"]), dtype=torch.float64)
    out, lse = orc.attention(q, kc, vc, torch.tensor([[0]]), torch.tensor([2]), torch.tensor([0, 1]),
                             g["softmax_scale"], True, (-1, -1), g["rel_extent"], rel)
    _assert_close(out, torch.tensor(num(g["expected_out"]), dtype=torch.float64), 1e-12)
    _assert_close(lse, torch.tensor(num(g["expected_lse"]), dtype=torch.float64), 1e-12)


# ------------------------------------------------------------ brute force

def _random_small(seed, *, causal=True, window=(-1, -1), rel_extent=5, G=2, Hkv=2, D=8, BS=16,
                  q_lens=None, k_lens=None, poison=False):
    g = torch.Generator()
    g.manual_seed(1000 + seed)
    B = int(torch.randint(1, 4, (1,), generator=g))
    if k_lens is None:
        k_lens = [int(x) for x in torch.randint(1, 65, (B,), generator=g)]
    if q_lens is None:
        q_lens = [int(torch.randint(1, lk + 1, (1,), generator=g)) if lk else 0 for lk in k_lens]
        q_lens = [min(q, 9) for q in q_lens]
    return wl.build(q_lens, k_lens, num_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, block_size=BS,
                    rel_extent=rel_extent, causal=causal, window_size=window, seed=seed,
                    extra_pages=2, poison=poison)


def test_brute_vs_oracle_tiny_config():
    for s in (1, 4):
        w = wl.tiny(num_splits=s)
        o1, l1 = _run(w)
        o2, l2 = _brute(w)
        _assert_close(o1, o2)
        _assert_close(l1, l2)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("R", [0, 1, 5, 32])
def test_brute_vs_oracle_random(seed, R):
    causal = seed % 3 != 2
    window = [(-1, -1), (7, 0), (3, 2), (-1, 4), (5, -1), (0, 0)][seed]
    w = _random_small(seed, causal=causal, window=window, rel_extent=R, G=1 + seed % 3)
    o1, l1 = _run(w)
    o2, l2 = _brute(w)
    _assert_close(o1, o2)
    _assert_close(l1, l2)


# ------------------------------------------------------- library routine

def test_matches_float64_sdpa_with_explicit_mask():
    """Per (request, head), after gathering pages, the oracle equals torch's
    scaled_dot_product_attention in float64 given the dense additive mask
    (bias in the band, 0 elsewhere, -inf where hidden); lse equals logsumexp
    of the same logits."""
    w = wl.build([1, 5, 12], [40, 29, 77], num_heads=6, num_kv_heads=2, head_dim=16, block_size=16,
                 rel_extent=20, window_size=(30, 0), seed=11)
    out, lse = _run(w)
    G = w.num_heads // w.num_kv_heads
    cu = w.cu_seqlens_q.tolist()
    for b in range(w.batch):
        lq, lk = w.q_lens[b], w.k_lens[b]
        K = torch.stack([w.key_cache[w.block_table[b, t // 16], t % 16] for t in range(lk)]).double()
        V = torch.stack([w.value_cache[w.block_table[b, t // 16], t % 16] for t in range(lk)]).double()
        for h in range(w.num_heads):
            mask = torch.full((lq, lk), -math.inf, dtype=torch.float64)
            for i in range(lq):
                pos = lk - lq + i
                for t in range(max(0, pos - 30), pos + 1):
                    d = pos - t
                    mask[i, t] = float(w.rel_logits[cu[b] + i, h, d]) if d < 20 else 0.0
            qh = w.q[cu[b]:cu[b + 1], h].double()
            ref = torch.nn.functional.scaled_dot_product_attention(
                qh[None, None], K[:, h // G][None, None].contiguous(), V[:, h // G][None, None],
                attn_mask=mask[None, None], scale=float(torch.tensor(w.softmax_scale, dtype=torch.float32)))
            _assert_close(out[cu[b]:cu[b + 1], h], ref[0, 0], 1e-12)
            logits = qh @ K[:, h // G].T * float(torch.tensor(w.softmax_scale, dtype=torch.float32)) + mask
            _assert_close(lse[cu[b]:cu[b + 1], h], torch.logsumexp(logits, dim=1), 1e-12)


# ------------------------------------------------------------ closed forms

def test_single_key_gives_that_value():
    w = wl.build([1, 1], [1, 1], num_heads=2, num_kv_heads=1, head_dim=8, rel_extent=3, seed=5)
    out, lse = _run(w)
    sc = float(torch.tensor(w.softmax_scale, dtype=torch.float32))
    for b in range(2):
        pg = int(w.block_table[b, 0])
        for h in range(2):
            _assert_close(out[b, h], w.value_cache[pg, 0, 0].double())
            s0 = sc * float(w.q[b, h].double() @ w.key_cache[pg, 0, 0].double()) + float(w.rel_logits[b, h, 0])
            assert abs(lse[b, h].item() - s0) < 1e-12


def test_equal_values_give_that_value():
    w = _random_small(2, rel_extent=7)
    w.value_cache[:] = w.value_cache[0, 0, 0]
    out, _ = _run(w)
    ok = torch.isfinite(out[..., 0])
    ref = w.value_cache[0, 0, 0].double().expand_as(out)
    _assert_close(out[ok], ref[ok])


def test_equal_keys_no_bias_give_mean_of_visible_values():
    w = wl.build([4], [30], num_heads=2, num_kv_heads=2, head_dim=8, window_size=(5, 0), seed=8)
    w.key_cache[:] = w.key_cache[0, 0, 0]
    out, _ = _run(w)
    for i in range(4):
        pos = 26 + i
        lo = max(0, pos - 5)
        for h in range(2):
            V = torch.stack([w.value_cache[w.block_table[0, t // 16], t % 16, h] for t in range(lo, pos + 1)]).double()
            _assert_close(out[i, h], V.mean(0))


def test_constant_bias_shifts_lse_only():
    w = _random_small(4, rel_extent=64)
    c = 0.75
    out0, lse0 = orc.attention(w.q, w.key_cache, w.value_cache, w.block_table, w.cache_seqlens,
                               w.cu_seqlens_q, w.softmax_scale, True, (-1, -1), 0, None)
    rel = torch.full_like(w.rel_logits, c)
    out1, lse1 = orc.attention(w.q, w.key_cache, w.value_cache, w.block_table, w.cache_seqlens,
                               w.cu_seqlens_q, w.softmax_scale, True, (-1, -1), 64, rel)
    _assert_close(out1, out0, 1e-12)
    _assert_close(lse1, lse0 + c, 1e-12)


@pytest.mark.parametrize("d0", [0, 1, 6])
def test_bias_spike_selects_the_key_at_that_distance(d0):
    """rel_logits[tok, h, d0] = +60 (others 0) puts all weight on the key at
    position q_abs - d0, for that token and q head only."""
    w = wl.build([3, 2], [20, 11], num_heads=4, num_kv_heads=2, head_dim=8, rel_extent=8, seed=9)
    w.rel_logits.zero_()
    tok, h = 3, 1  # request 1, local row 0 -> q_abs = 11 - 2 + 0 = 9
    w.rel_logits[tok, h, d0] = 60.0
    out, _ = _run(w)
    pos = 9 - d0
    v = w.value_cache[w.block_table[1, pos // 16], pos % 16, h // 2].double()
    assert (out[tok, h] - v).abs().max().item() < 1e-12
    others = [(tok, 0), (tok, 2), (4, h)]
    for t2, h2 in others:
        assert (out[t2, h2] - v).abs().max().item() > 1e-3


# -------------------------------------------------------------- invariants

@pytest.mark.parametrize("S", [1, 2, 3, 4, 7, 64])
def test_split_emulation_invariance(S):
    w = wl.tiny()
    out, lse = _run(w)
    po, pl = orc.attention_split_partials(w.q, w.key_cache, w.value_cache, w.block_table,
                                          w.cache_seqlens, w.cu_seqlens_q, w.softmax_scale,
                                          w.causal, w.window_size, w.rel_extent, w.rel_logits,
                                          num_splits=S)
    o2, l2 = orc.combine(po, pl)
    _assert_close(o2, out)
    _assert_close(l2, lse)


def test_combine_special_cases():
    po = torch.randn(3, 2, 2, 4, dtype=torch.float64)
    pl = torch.randn(3, 2, 2, dtype=torch.float64)
    pl[:, 0, 0] = -math.inf
    po[:, 0, 0] = 0
    o, l = orc.combine(po, pl)
    assert torch.equal(o[0, 0], torch.zeros(4, dtype=torch.float64))
    assert l[0, 0].item() == -math.inf
    o1, l1 = orc.combine(po[:1], pl[:1])
    _assert_close(o1[0, 1], po[0, 0, 1])
    _assert_close(l1, pl[0])


def test_zero_bias_equals_no_bias():
    w = _random_small(1, rel_extent=16)
    a = orc.attention(w.q, w.key_cache, w.value_cache, w.block_table, w.cache_seqlens, w.cu_seqlens_q,
                      w.softmax_scale, True, (-1, -1), 16, torch.zeros_like(w.rel_logits))
    b = orc.attention(w.q, w.key_cache, w.value_cache, w.block_table, w.cache_seqlens, w.cu_seqlens_q,
                      w.softmax_scale, True, (-1, -1), 0, None)
    _assert_close(a[0], b[0])
    _assert_close(a[1], b[1])


def test_page_permutation_invariance():
    w = _random_small(3, rel_extent=9)
    out, lse = _run(w)
    nb = w.key_cache.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(77))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(nb)
    w.key_cache = w.key_cache[perm]       # new page p holds old page perm[p]
    w.value_cache = w.value_cache[perm]
    bt = w.block_table.clone()
    valid = bt >= 0
    bt[valid] = inv[bt[valid].long()].int()
    w.block_table = bt
    o2, l2 = _run(w)
    _assert_close(o2, out)
    _assert_close(l2, lse)


def test_mha_expansion_invariance():
    w = _random_small(5, rel_extent=6, G=3, Hkv=2)
    out, lse = _run(w)
    G = 3
    w.key_cache = w.key_cache.repeat_interleave(G, dim=2)
    w.value_cache = w.value_cache.repeat_interleave(G, dim=2)
    o2, l2 = _run(w)
    _assert_close(o2, out)
    _assert_close(l2, lse)


def test_wide_window_equals_no_window():
    w = _random_small(6, rel_extent=4)
    out, lse = _run(w)
    w.window_size = (100, 100)
    o2, l2 = _run(w)
    _assert_close(o2, out)
    _assert_close(l2, lse)


def test_prefill_row_equals_decode_call():
    """Row i of a prefill chunk equals a one-token request whose KV length is
    q_abs + 1 over the same pages, q row and rel_logits row."""
    w = wl.build([6], [21], num_heads=4, num_kv_heads=2, head_dim=8, rel_extent=5, seed=12)
    out, lse = _run(w)
    for i in range(6):
        pos = 21 - 6 + i
        o, l = orc.attention(w.q[i:i + 1], w.key_cache, w.value_cache, w.block_table, [pos + 1], [0, 1],
                             w.softmax_scale, True, (-1, -1), 5, w.rel_logits[i:i + 1])
        _assert_close(o[0], out[i])
        _assert_close(l[0], lse[i])


def test_request_reordering_invariance():
    w = wl.build([2, 1, 3], [9, 30, 17], num_heads=2, num_kv_heads=1, head_dim=8, rel_extent=4, seed=13)
    out, lse = _run(w)
    order = [2, 0, 1]
    cu = w.cu_seqlens_q.tolist()
    toks = torch.cat([torch.arange(cu[b], cu[b + 1]) for b in order])
    q_lens = [w.q_lens[b] for b in order]
    o2, l2 = orc.attention(w.q[toks], w.key_cache, w.value_cache, w.block_table[order],
                           torch.tensor([w.k_lens[b] for b in order]),
                           torch.tensor(orc.cu_seqlens_from_lengths(q_lens)), w.softmax_scale, True,
                           (-1, -1), 4, w.rel_logits[toks])
    _assert_close(o2, out[toks])
    _assert_close(l2, lse[toks])


def test_nan_poison_in_unreferenced_storage_changes_nothing():
    a = _random_small(7, rel_extent=5, poison=False)
    b = _random_small(7, rel_extent=5, poison=True)
    assert torch.isnan(b.key_cache.float()).any()
    oa, la = _run(a)
    ob, lb = _run(b)
    _assert_close(ob, oa)
    _assert_close(lb, la)


def test_rows_without_visible_keys():
    """Lk < Lq makes the first rows see nothing; Lk == 0 makes all rows empty:
    out = 0 and lse = -inf, with no NaN."""
    w = wl.build([4, 2], [2, 0], num_heads=2, num_kv_heads=1, head_dim=8, rel_extent=3, seed=14)
    out, lse = _run(w)
    assert not torch.isnan(out).any()
    assert lse[0].tolist() == [-math.inf, -math.inf] and lse[1].tolist() == [-math.inf, -math.inf]
    assert torch.isfinite(lse[2]).all() and torch.isfinite(lse[3]).all()
    assert (out[4:] == 0).all() and (lse[4:] == -math.inf).all()
    o2, l2 = _brute(w)
    _assert_close(out, o2)
    _assert_close(lse, l2)


# ------------------------------------------------------ planted mistakes

def _pins_pass():
    """Run a compact set of pins; True iff all hold."""
    checks = [test_two_key_softmax_golden, test_query_positions_drive_the_result,
              lambda: test_bias_spike_selects_the_key_at_that_distance(1),
              test_mha_expansion_invariance, test_matches_float64_sdpa_with_explicit_mask,
              test_equal_keys_no_bias_give_mean_of_visible_values]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def test_pins_hold_for_the_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("mistake", ["scaled_bias", "reversed_distance", "top_left_causal",
                                     "kv_head_modulo", "no_window", "bias_off_by_one"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    real_bias = orc.bias_matrix
    real_qpos = orc.query_positions
    real_vis = orc.visible_mask
    real_gather = orc._gather_head
    if mistake == "scaled_bias":
        real_scores = orc._scores

        def scores(q, K, h, rows_tok, qa, k_len, rel, R, scale, vis, alibi_slopes=None):
            S = real_scores(q, K, h, rows_tok, qa, k_len, None, 0, scale, vis, alibi_slopes)
            if R > 0 and rel is not None:
                S = S + scale * real_bias(rel[rows_tok, h, :], qa, k_len, R)
            return torch.where(vis, S, torch.full((), -math.inf, dtype=torch.float64))
        monkeypatch.setattr(orc, "_scores", scores)
    elif mistake == "reversed_distance":
        def bias(rows, qa, k_len, R):
            n = qa.numel()
            d = torch.arange(k_len)[None, :] - qa[:, None]
            band = (d >= 0) & (d < R)
            vals = torch.gather(rows.double(), 1, d.clamp(0, R - 1))
            return torch.where(band, vals, torch.zeros((), dtype=torch.float64)) if n else torch.zeros((0, k_len))
        monkeypatch.setattr(orc, "bias_matrix", bias)
    elif mistake == "top_left_causal":
        monkeypatch.setattr(orc, "query_positions", lambda ql, kl: torch.arange(ql, dtype=torch.int64))
    elif mistake == "kv_head_modulo":
        # q head h read from kv head h % Hkv instead of h // G
        real_att = orc.attention

        def att(q, kc, vc, *a, **k):
            Hkv = kc.shape[2]
            H = q.shape[1]
            G = H // Hkv
            f = [(h % Hkv) * G + h // Hkv for h in range(H)]
            finv = [0] * H
            for h, p in enumerate(f):
                finv[p] = h
            args = list(a)
            if len(args) > 7 and args[7] is not None:
                args[7] = args[7][:, finv, :]
            o, l = real_att(q[:, finv, :], kc, vc, *args, **k)
            return o[:, f, :], l[:, f]
        monkeypatch.setattr(orc, "attention", att)
    elif mistake == "no_window":
        monkeypatch.setattr(orc, "visible_mask", lambda qa, kl, c, w: real_vis(qa, kl, c, (-1, -1)))
    elif mistake == "bias_off_by_one":
        monkeypatch.setattr(orc, "bias_matrix", lambda rows, qa, kl, R: real_bias(rows, qa - 1, kl, R))
    assert not _pins_pass(), f"planted mistake {mistake} went unnoticed"
    del real_qpos, real_gather
