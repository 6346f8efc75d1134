"""Host-side checks of librpa.so that need no GPU: the library loads, exports
every entry point include/rpa.h declares, and rejects bad arguments before
any HIP call.  The split planner is checked for its stated properties only
(its exact choices are our own tuning, not a formula the pages fix)."""
import ctypes
import os
import re

import pytest

from relative_bias_amd import binding as bnd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rpa.h")

OK, NULL, SHAPE, UNSUP, WS = 0, -1, -2, -3, -4
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


# RPA_TEST_LIB selects another build of the same C ABI (the sanitizer build
# of the host layer that tests/test_host_sanitizer.py runs these tests on).
_TEST_LIB = os.environ.get("RPA_TEST_LIB")


@pytest.fixture(scope="module")
def L():
    if _TEST_LIB:
        bnd._lib = None
        bnd.LIB_PATH = _TEST_LIB
    elif not os.path.exists(bnd.LIB_PATH):
        from relative_bias_amd import build
        build.build()
    return bnd.lib()


def _declared():
    with open(HEADER) as f:
        src = f.read()
    return sorted(set(re.findall(r"\b(rpa_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("rpa_attn_varlen", "rpa_split_combine", "rpa_choose_splits", "rpa_workspace_bytes",
              "rpa_status_string", "rpa_slot_mapping", "rpa_kv_cache_write", "rpa_attn_varlen_fp8",
              "rpa_kv_cache_write_fp8", "rpa_attn_varlen_ex"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for n in _declared():
        assert hasattr(L, n), f"{n} declared in rpa.h but not exported"


def test_status_strings(L):
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert L.rpa_status_string(s)


def test_workspace_bytes(L):
    assert bnd.rpa_workspace_bytes(1, 100, 8, 128) == 0
    assert bnd.rpa_workspace_bytes(-1, 100, 8, 128) == 0
    assert bnd.rpa_workspace_bytes(4, -1, 8, 128) == 0
    # num_splits = 0 (balanced decode): per-workgroup records plus two
    # partial slots of eight kv heads x 16 columns per workgroup (up to 512
    # workgroups), whatever the batch.
    for D in (64, 128):
        n0 = bnd.rpa_workspace_bytes(0, 100, 8, D)
        assert n0 == bnd.rpa_workspace_bytes(0, 1, 64, D)
        assert n0 % 256 == 0
        need = 512 * 8 * 4 + 2 * 512 * 8 * 16 * (D + 1) * 4
        assert need <= n0 < need + 256
    for S, T, H, D in [(2, 1, 1, 64), (4, 32, 32, 128), (128, 1, 64, 128), (3, 17, 6, 64)]:
        n = bnd.rpa_workspace_bytes(S, T, H, D)
        assert n >= S * T * H * (D + 1) * 4
        assert n % 256 == 0
        assert n < S * T * H * (D + 1) * 4 + 512


def _attn(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, P=4, seqlens=FAKE, cu=FAKE, B=2, T=3, H=4, Hkv=2, D=64,
             NB=8, BS=16, maxq=2, scale=0.125, causal=1, left=-1, right=-1, R=0, rel=None, S=1,
             ws=None, wsb=0, out=FAKE, lse=None)
    a.update(kw)
    return L.rpa_attn_varlen(a["q"], a["k"], a["v"], a["bt"], a["P"], a["seqlens"], a["cu"], a["B"],
                             a["T"], a["H"], a["Hkv"], a["D"], a["NB"], a["BS"], a["maxq"], a["scale"],
                             a["causal"], a["left"], a["right"], a["R"], a["rel"], a["S"], a["ws"],
                             a["wsb"], a["out"], a["lse"], None)


@pytest.mark.parametrize("field", ["q", "k", "v", "bt", "seqlens", "cu", "out"])
def test_null_pointers(L, field):
    assert _attn(L, **{field: None}) == NULL


def test_rel_logits_required_when_extent_positive(L):
    assert _attn(L, R=8, rel=None) == NULL


@pytest.mark.parametrize("kw", [dict(H=6, Hkv=4), dict(S=-1), dict(S=129), dict(B=-1), dict(T=-2),
                                dict(H=0), dict(Hkv=0), dict(BS=0), dict(left=-2), dict(right=-5),
                                dict(R=-1), dict(maxq=-1), dict(P=-1), dict(B=0, T=3),
                                dict(scale=float("nan")), dict(scale=float("inf"))])
def test_bad_shapes(L, kw):
    assert _attn(L, **kw) == SHAPE


def test_key_positions_must_fit_32_bits(L):
    # max_pages_per_seq * block_size + max_seqlen_q + rel_extent + 128 must stay below 2^31.
    P = (2 ** 31 - 130) // 16
    assert _attn(L, P=P, BS=16, maxq=2, q=None) == NULL
    assert _attn(L, P=P + 1, BS=16, maxq=2, q=None) == SHAPE
    R = 2 ** 31 - 4 * 16 - 2 - 128
    assert _attn(L, R=R - 1, rel=FAKE, q=None) == NULL
    assert _attn(L, R=R, rel=FAKE, q=None) == SHAPE
    # Windows of any size up to 2^31 - 1 are accepted.
    assert _attn(L, left=2 ** 31 - 1, right=2 ** 31 - 1, q=None) == NULL


@pytest.mark.parametrize("kw", [dict(D=96), dict(D=256), dict(D=32), dict(BS=8), dict(BS=24)])
def test_unsupported(L, kw):
    assert _attn(L, **kw) == UNSUP


def test_workspace_checks(L):
    assert _attn(L, S=4, ws=None) == WS
    need = bnd.rpa_workspace_bytes(4, 3, 4, 64)
    assert _attn(L, S=4, ws=FAKE, wsb=need - 1) == WS
    assert _attn(L, S=0, ws=None) == WS
    need0 = bnd.rpa_workspace_bytes(0, 3, 4, 64)
    assert _attn(L, S=0, ws=FAKE, wsb=need0 - 1) == WS


def test_empty_batch_is_a_no_op(L):
    # Nothing to compute: returns OK before touching any pointer or HIP.
    assert _attn(L, T=0, B=0, q=None, out=None) == OK
    assert _attn(L, T=0, B=3) == OK


def test_combine_argument_errors(L):
    c = L.rpa_split_combine
    assert c(FAKE, FAKE, 0, 4, 2, 64, FAKE, None, None) == SHAPE
    assert c(FAKE, FAKE, 129, 4, 2, 64, FAKE, None, None) == SHAPE
    assert c(FAKE, FAKE, 2, 4, 2, 96, FAKE, None, None) == UNSUP
    assert c(None, FAKE, 2, 4, 2, 64, FAKE, None, None) == NULL
    assert c(FAKE, FAKE, 2, 4, 2, 64, None, None, None) == NULL
    assert c(None, None, 2, 0, 2, 64, None, None, None) == OK


def test_slot_mapping_argument_errors(L):
    f = L.rpa_slot_mapping
    assert f(FAKE, 4, FAKE, FAKE, -1, 3, 16, FAKE, None) == SHAPE
    assert f(FAKE, 4, FAKE, FAKE, 2, -1, 16, FAKE, None) == SHAPE
    assert f(FAKE, 4, FAKE, FAKE, 2, 3, 0, FAKE, None) == SHAPE
    assert f(FAKE, -1, FAKE, FAKE, 2, 3, 16, FAKE, None) == SHAPE
    assert f(FAKE, 4, FAKE, FAKE, 0, 3, 16, FAKE, None) == SHAPE
    assert f(None, 4, FAKE, FAKE, 2, 3, 16, FAKE, None) == NULL
    assert f(FAKE, 4, FAKE, FAKE, 2, 3, 16, None, None) == NULL
    assert f(None, 4, None, None, 2, 0, 16, None, None) == OK


def test_kv_cache_write_argument_errors(L):
    f = L.rpa_kv_cache_write
    assert f(FAKE, FAKE, FAKE, -1, 2, 64, 4, 16, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 3, 0, 64, 4, 16, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 3, 2, 0, 4, 16, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 3, 2, 64, -1, 16, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 3, 2, 64, 4, 0, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 3, 1, 12, 4, 16, FAKE, FAKE, None) == UNSUP  # 24-byte rows
    assert f(None, FAKE, FAKE, 3, 2, 64, 4, 16, FAKE, FAKE, None) == NULL
    assert f(FAKE, FAKE, None, 3, 2, 64, 4, 16, FAKE, FAKE, None) == NULL
    assert f(FAKE, FAKE, FAKE, 3, 2, 64, 4, 16, FAKE, None, None) == NULL
    assert f(None, None, None, 0, 2, 64, 4, 16, None, None, None) == OK


def _attn8(L, ks=1.0, vs=1.0, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, P=4, seqlens=FAKE, cu=FAKE, B=2, T=2, H=32, Hkv=8, D=128,
             NB=8, BS=16, maxq=1, scale=0.125, causal=1, left=-1, right=-1, R=0, rel=None, S=0,
             ws=FAKE, wsb=bnd.rpa_workspace_bytes(0, 2, 32, 128), out=FAKE, lse=None)
    a.update(kw)
    return L.rpa_attn_varlen_fp8(a["q"], a["k"], a["v"], ks, vs, a["bt"], a["P"], a["seqlens"], a["cu"], a["B"],
                                 a["T"], a["H"], a["Hkv"], a["D"], a["NB"], a["BS"], a["maxq"], a["scale"],
                                 a["causal"], a["left"], a["right"], a["R"], a["rel"], a["S"], a["ws"],
                                 a["wsb"], a["out"], a["lse"], None)


@pytest.mark.parametrize("ks,vs", [(0.0, 1.0), (1.0, 0.0), (-1.0, 1.0), (1.0, -2.0), (float("nan"), 1.0),
                                   (1.0, float("inf"))])
def test_fp8_attention_rejects_bad_scales(L, ks, vs):
    assert _attn8(L, ks, vs) == SHAPE


def test_fp8_attention_argument_errors(L):
    # The same validation as the bf16 entry point, before any HIP call.
    assert _attn8(L, k=None) == NULL
    assert _attn8(L, v=None) == NULL
    assert _attn8(L, R=4, rel=None) == NULL
    assert _attn8(L, D=96) == UNSUP
    assert _attn8(L, BS=24) == UNSUP
    assert _attn8(L, H=12, Hkv=8) == SHAPE
    assert _attn8(L, ws=None) == WS
    assert _attn8(L, S=4, ws=None) == WS
    assert _attn8(L, T=0, B=0, q=None, out=None) == OK


def test_ex_entry_validates_like_the_others(L):
    f = L.rpa_attn_varlen_ex
    def call(kv, ks, vs, D=128, S=1, ws=None, wsb=0, q=FAKE, T=2, B=2):
        return f(q, FAKE, FAKE, kv, ks, vs, FAKE, 4, FAKE, FAKE, B, T, 32, 8, D, 8, 16, 1, 0.125, 1, -1, -1,
                 0, None, 0, FAKE, S, ws, wsb, FAKE, None, None)
    assert call(1, 0.0, 1.0) == SHAPE        # E4M3 caches need positive scales
    assert call(0, 0.0, 1.0, D=96) == UNSUP  # bf16 caches ignore them
    assert call(1, 1.0, 1.0, S=4) == WS
    assert call(0, 1.0, 1.0, q=None) == NULL
    assert call(1, 1.0, 1.0, T=0, B=0, q=None) == OK


def test_ex_entry_limits_the_width_of_bf16_rel_logits(L):
    # A prefill tile reads its rows' bf16 rel_logits through one buffer
    # resource: (128 / G + 2) * H * R * 2 bytes must stay below 2 GiB.
    f = L.rpa_attn_varlen_ex
    def call(R, bf16, maxq, q=FAKE):
        return f(q, FAKE, FAKE, 0, 1.0, 1.0, FAKE, 4, FAKE, FAKE, 2, 2, 32, 8, 128, 8, 16, maxq, 0.125, 1, -1, -1,
                 R, FAKE, bf16, None, 1, None, 0, FAKE, None, None)
    wide = 1 << 21                            # (32 + 2) * 32 * 2^21 * 2 bytes = 4.6 GB
    assert call(wide, 1, 64) == UNSUP
    assert call(wide, 1, 1, q=None) == NULL   # decode-only batches never build prefill tiles
    assert call(wide, 0, 64, q=None) == NULL  # fp32 rel_logits have a per-value form for such tiles
    assert call(1 << 14, 1, 64, q=None) == NULL
    # bf16 rel_logits are read as dwords: the array must start on a 4-byte boundary.
    odd = ctypes.c_void_p(0x1002)
    assert f(FAKE, FAKE, FAKE, 0, 1.0, 1.0, FAKE, 4, FAKE, FAKE, 2, 2, 32, 8, 128, 8, 16, 1, 0.125, 1, -1, -1,
             64, odd, 1, None, 1, None, 0, FAKE, None, None) == UNSUP
    assert f(None, FAKE, FAKE, 0, 1.0, 1.0, FAKE, 4, FAKE, FAKE, 2, 2, 32, 8, 128, 8, 16, 1, 0.125, 1, -1, -1,
             64, odd, 0, None, 1, None, 0, FAKE, None, None) == NULL  # fp32 rel_logits: no such check


def test_kv_cache_write_fp8_argument_errors(L):
    f = L.rpa_kv_cache_write_fp8
    assert f(FAKE, FAKE, FAKE, 3, 2, 64, 4, 16, 0.0, 1.0, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 3, 2, 64, 4, 16, 1.0, float("nan"), FAKE, FAKE, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 3, 2, 64, 4, 16, -1.0, 1.0, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, -1, 2, 64, 4, 16, 1.0, 1.0, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 3, 1, 12, 4, 16, 1.0, 1.0, FAKE, FAKE, None) == UNSUP
    assert f(None, FAKE, FAKE, 3, 2, 64, 4, 16, 1.0, 1.0, FAKE, FAKE, None) == NULL
    assert f(FAKE, FAKE, FAKE, 3, 2, 64, 4, 16, 1.0, 1.0, None, FAKE, None) == NULL
    assert f(None, None, None, 0, 2, 64, 4, 16, 1.0, 1.0, None, None, None) == OK


# ------------------------------------------------------------------ planner

def test_planner_rejects_bad_sizes(L):
    assert L.rpa_choose_splits(1, 1, 6, 4, 100, 0, 256) == SHAPE
    assert L.rpa_choose_splits(-1, 1, 8, 8, 100, 0, 256) == SHAPE
    assert L.rpa_choose_splits(1, 1, 8, 0, 100, 0, 256) == SHAPE


@pytest.mark.parametrize("B,maxq,H,Hkv,maxk", [(32, 1, 32, 8, 8192), (1, 1, 64, 8, 1 << 20),
                                               (8, 2048, 32, 8, 6144), (68, 1024, 64, 8, 131072),
                                               (3, 16, 4, 2, 312), (1, 1, 8, 1, 100), (256, 1, 32, 8, 4096),
                                               (1, 4, 64, 8, 1 << 20), (3000, 1, 32, 8, 4096),
                                               (4, 3, 32, 4, 5000)])
def test_planner_properties(L, B, maxq, H, Hkv, maxk):
    s = bnd.rpa_choose_splits(B, maxq, H, Hkv, maxk)
    G = H // Hkv
    if maxq * G <= 16 and B <= 2048:
        assert s == 0                    # decode batch: the balanced decode
    else:
        assert 1 <= s <= bnd.RPA_MAX_SPLITS
        if s > 1:
            assert maxk // s >= 512      # at least 512 keys per split
        # more requests never ask for more splits
        assert bnd.rpa_choose_splits(2 * B, maxq, H, Hkv, maxk) <= s
    assert bnd.rpa_choose_splits(B, maxq, H, Hkv, maxk, is_local=True) == 1


def test_planner_splits_long_context_prefill_rows(L):
    # A query longer than one decode column group cannot take the balanced
    # decode: split by length.
    assert bnd.rpa_choose_splits(1, 32, 64, 8, 1 << 20) >= 16
    assert bnd.rpa_choose_splits(8, 2048, 32, 8, 6144) == 1


def test_planner_balances_decode_batches(L):
    assert L.rpa_choose_splits(32, 1, 32, 8, 8192, 0, 256) == 0
    assert L.rpa_choose_splits(1, 1, 64, 8, 1 << 20, 0, 256) == 0
    # More requests than the balanced decode takes: one split each.
    assert L.rpa_choose_splits(3000, 1, 32, 8, 8192, 0, 256) == 1


def _attn_noalloc(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, P=4, seqlens=FAKE, cu=FAKE, B=2, T=3, H=4, Hkv=2, D=64,
             NB=8, BS=16, maxq=2, scale=0.125, causal=1, left=-1, right=-1, R=0, rel=None, S=1, out=FAKE)
    a.update(kw)
    return L.rpa_attn_varlen_noalloc(a["q"], a["k"], a["v"], 0, 1.0, 1.0, a["bt"], a["P"], a["seqlens"], a["cu"],
                                     a["B"], a["T"], a["H"], a["Hkv"], a["D"], a["NB"], a["BS"], a["maxq"],
                                     a["scale"], a["causal"], a["left"], a["right"], a["R"], a["rel"], 0, None,
                                     a["S"], a["out"], None, None)


def test_noalloc_argument_errors(L):
    """The no-alloc entry validates like the others before it looks up its
    scratch, and refuses partials larger than the scratch (no HIP call)."""
    assert _attn_noalloc(L, q=None) == NULL
    assert _attn_noalloc(L, out=None) == NULL
    assert _attn_noalloc(L, H=6, Hkv=4) == SHAPE
    assert _attn_noalloc(L, S=129) == SHAPE
    assert _attn_noalloc(L, D=96) == UNSUP
    assert _attn_noalloc(L, T=0, B=0, q=None, out=None) == OK
    # 64 splits x 600 tokens x 32 heads x 129 fp32 values: about 630 MB.
    assert _attn_noalloc(L, B=2, T=600, H=32, Hkv=8, D=128, maxq=300, S=64) == WS


def test_requested_build_is_the_one_loaded(L):
    """When another build of the ABI is requested (RPA_TEST_LIB), that file is
    the one mapped into this process, and a sanitizer build runs with its
    runtime present."""
    if not _TEST_LIB:
        pytest.skip("testing the default build")
    with open("/proc/self/maps") as f:
        maps = f.read()
    assert os.path.realpath(_TEST_LIB) in maps
    if "hostsan" in os.path.basename(_TEST_LIB):
        assert "libasan" in maps and "libubsan" in maps
