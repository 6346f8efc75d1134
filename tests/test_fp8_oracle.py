"""Pins for the FP8 KV-cache oracle (oracle/fp8.py).

The E4M3 code is pinned by torch's float8_e4m3fn (an independent library
conversion), by values worked from the format's bit fields, by the
round-trip of every finite code and by hand-picked ties and saturation
cases.  Quantise-at-store is pinned by the division it must do (a planted
multiply is caught) and by the format's half-ulp error bound; attention over
an FP8 cache is pinned against the bf16 oracle on the same values, with the
scales placed where the pages put them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as orc
from oracle import brute
from oracle import fp8
from oracle import kv_cache as okv
from relative_bias_amd import workloads as wl

ALL = torch.arange(256, dtype=torch.int32).to(torch.uint8)


def test_decode_matches_torch_float8_e4m3fn_on_every_code():
    mine = fp8.e4m3_decode(ALL)
    lib = ALL.view(torch.float8_e4m3fn).to(torch.float64)
    for c in range(256):
        a, b = mine[c].item(), lib[c].item()
        assert (math.isnan(a) and math.isnan(b)) or (a == b and math.copysign(1, a) == math.copysign(1, b)), hex(c)


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0), (0x39, 1.125),
    (0x3F, 1.875), (0x40, 2.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0), (0x30, 0.5),
])
def test_decode_worked_values(code, value):
    v = fp8.e4m3_decode(torch.tensor([code], dtype=torch.uint8)).item()
    assert v == value


def test_nan_codes_and_negative_zero():
    v = fp8.e4m3_decode(torch.tensor([0x7F, 0xFF, 0x80], dtype=torch.uint8))
    assert math.isnan(v[0]) and math.isnan(v[1])
    assert v[2].item() == 0.0 and math.copysign(1, v[2].item()) < 0


def test_every_finite_code_round_trips():
    vals = fp8.e4m3_decode(ALL)
    fin = ~torch.isnan(vals)
    assert torch.equal(fp8.e4m3_encode(vals[fin].float()), ALL[fin])


def test_encode_matches_torch_inside_the_range():
    g = torch.Generator().manual_seed(0)
    x = torch.cat([torch.randn(50000, generator=g) * s for s in (1e-3, 0.05, 1.0, 30.0, 120.0)])
    x = x[x.abs() < 440]
    assert torch.equal(fp8.e4m3_encode(x), x.to(torch.float8_e4m3fn).view(torch.uint8))


@pytest.mark.parametrize("y,code", [
    (1.0625, 0x38),          # midway 1.0 / 1.125: the even code 0x38
    (1.1875, 0x3A),          # midway 1.125 / 1.25: the even code 0x3A
    (1.0625 + 2 ** -20, 0x39),
    (2.0 ** -10, 0x00),      # midway 0 / 2^-9: 0
    (3 * 2.0 ** -10, 0x02),  # midway 2^-9 / 2^-8: code 2
    (-(2.0 ** -12), 0x80),   # rounds to -0
    (448.0, 0x7E), (460.0, 0x7E), (464.0, 0x7E), (1e9, 0x7E), (-1e30, 0xFE),
    (math.inf, 0x7E), (-math.inf, 0xFE), (math.nan, 0x7F),
])
def test_encode_ties_saturation_and_specials(y, code):
    assert fp8.e4m3_encode(torch.tensor([y], dtype=torch.float32)).item() == code


def test_quantize_divides_by_the_scale():
    x = torch.tensor([1.0, -3.0, 0.75], dtype=torch.bfloat16)
    # x / 2 = 0.5, -1.5, 0.375 (a planted x * 2 would give 2, -6, 1.5)
    assert fp8.quantize(x, 2.0).tolist() == [0x30, 0xBC, 0x2C]
    # 1 / 3 in fp32 lies above the midpoint of 0.3125 and 0.34375
    assert fp8.quantize(torch.tensor([1.0]), 3.0).item() == 0x2B


def test_quantize_error_bound():
    """|dequant(quant(x)) - x| <= half an E4M3 ulp of x / scale, times the
    scale, for values in the normal range."""
    g = torch.Generator().manual_seed(1)
    x = (torch.randn(20000, generator=g) * 4).to(torch.bfloat16)
    scale = 0.0371
    y = x.float().double() / np.float32(scale)
    keep = (y.abs() >= 2 ** -6) & (y.abs() <= 448)
    back = fp8.dequantize(fp8.quantize(x, scale), scale)
    e = torch.floor(torch.log2(y.abs()))
    half_ulp = 2.0 ** (e - 4) * float(np.float32(scale))
    err = (back - x.double()).abs()
    # one extra fp32 rounding of x / scale
    assert (err[keep] <= half_ulp[keep] * (1 + 2 ** -20) + 1e-12).all()


def test_kv_cache_write_fp8_quantises_rows_at_their_slots():
    w = wl.build([3, 1, 4], [20, 9, 40], num_heads=4, num_kv_heads=2, head_dim=16, block_size=16, seed=5)
    slots = okv.slot_mapping(w.block_table, w.k_lens, w.cu_seqlens_q.tolist(), 16)
    g = torch.Generator().manual_seed(2)
    T = w.num_tokens
    key = torch.randn((T, 2, 16), generator=g).to(torch.bfloat16)
    val = torch.randn((T, 2, 16), generator=g).to(torch.bfloat16)
    kc = torch.randint(0, 256, w.key_cache.shape, generator=g, dtype=torch.int32).to(torch.uint8)
    vc = torch.randint(0, 256, w.key_cache.shape, generator=g, dtype=torch.int32).to(torch.uint8)
    nk, nv = fp8.kv_cache_write_fp8(key, val, slots, kc, vc, 0.5, 0.25)
    for t, s in enumerate(slots.tolist()):
        assert torch.equal(nk[s // 16, s % 16], fp8.quantize(key[t], 0.5))
        assert torch.equal(nv[s // 16, s % 16], fp8.quantize(val[t], 0.25))
    written = torch.zeros(kc.shape[0] * 16, dtype=torch.bool)
    written[slots] = True
    written = written.view(kc.shape[0], 16)
    assert torch.equal(nk[~written], kc[~written]) and torch.equal(nv[~written], vc[~written])


def _fp8_case(seed, R=6, window=(-1, -1)):
    w = wl.build([1, 5, 2], [30, 47, 2], num_heads=4, num_kv_heads=2, head_dim=16, block_size=16, rel_extent=R,
                 window_size=window, seed=seed)
    g = torch.Generator().manual_seed(seed + 100)
    k8 = torch.randint(0, 256, w.key_cache.shape, generator=g, dtype=torch.int32).to(torch.uint8)
    v8 = torch.randint(0, 256, w.key_cache.shape, generator=g, dtype=torch.int32).to(torch.uint8)
    k8[(k8 & 0x7F) == 0x7F] = 0x11  # no NaN codes
    v8[(v8 & 0x7F) == 0x7F] = 0x22
    return w, k8, v8


def test_attention_fp8_is_the_bf16_definition_on_decoded_values():
    """Unit scales: E4M3 values are exact in bf16, so the FP8 oracle equals
    the bf16 oracle on a cache holding the decoded values, and the scalar
    brute force."""
    w, k8, v8 = _fp8_case(7)
    kb = fp8.e4m3_decode(k8).to(torch.bfloat16)
    vb = fp8.e4m3_decode(v8).to(torch.bfloat16)
    assert torch.equal(kb.double(), fp8.e4m3_decode(k8))
    args = (w.block_table, w.cache_seqlens, w.cu_seqlens_q, w.softmax_scale, w.causal, w.window_size,
            w.rel_extent, w.rel_logits)
    o8, l8 = fp8.attention_fp8(w.q, k8, v8, 1.0, 1.0, *args)
    ob, lb = orc.attention(w.q, kb, vb, *args)
    assert torch.allclose(o8, ob, atol=1e-12, rtol=0) and torch.allclose(l8, lb, atol=1e-12, rtol=0)
    ob2, lb2 = brute.attention(w.q, kb, vb, *args)
    assert torch.allclose(o8, torch.as_tensor(ob2, dtype=torch.float64), atol=1e-10, rtol=0)
    assert torch.allclose(l8, torch.as_tensor(lb2, dtype=torch.float64), atol=1e-10, rtol=0)


def test_k_scale_multiplies_keys_only_and_v_scale_values_only():
    """k_scale = 2 equals doubling the softmax scale (the bias stays
    unscaled); v_scale = 4 multiplies the output by 4 and leaves the LSE."""
    w, k8, v8 = _fp8_case(8, R=40)
    args = (w.block_table, w.cache_seqlens, w.cu_seqlens_q)
    tail = (w.causal, w.window_size, w.rel_extent, w.rel_logits)
    o1, l1 = fp8.attention_fp8(w.q, k8, v8, 2.0, 1.0, *args, w.softmax_scale, *tail)
    o2, l2 = orc.attention(w.q, fp8.e4m3_decode(k8), fp8.e4m3_decode(v8), *args, 2 * w.softmax_scale, *tail)
    assert torch.allclose(o1, o2, atol=1e-12, rtol=0) and torch.allclose(l1, l2, atol=1e-12, rtol=0)
    # A planted k_scale on the bias too would differ by far more than that.
    o3, l3 = orc.attention(w.q, fp8.e4m3_decode(k8), fp8.e4m3_decode(v8), *args, 2 * w.softmax_scale,
                           w.causal, w.window_size, w.rel_extent, 2 * w.rel_logits)
    assert (l3 - l1).abs().max() > 1e-3
    o4, l4 = fp8.attention_fp8(w.q, k8, v8, 1.0, 4.0, *args, w.softmax_scale, *tail)
    o5, l5 = fp8.attention_fp8(w.q, k8, v8, 1.0, 1.0, *args, w.softmax_scale, *tail)
    assert torch.allclose(o4, 4 * o5, atol=1e-12, rtol=0) and torch.equal(l4, l5)


@pytest.mark.parametrize("x,scale_bits,two_step,direct", [
    (50.25, 0x40EE38E4, 0x4E, 0x4D),
    (57.0, 0x40EB5AD7, 0x50, 0x4F),
])
def test_quantize_rounds_the_fp32_quotient(x, scale_bits, two_step, direct):
    """Reading F3: x / scale is rounded to fp32 first.  For these values the
    exact quotient lies just below the midpoint of two E4M3 values and its
    fp32 rounding lands on the midpoint, so rounding once from the exact
    quotient would give the lower code (found by search, checked here with
    exact rationals)."""
    from fractions import Fraction
    scale = float(np.array([scale_bits], dtype=np.uint32).view(np.float32)[0])
    got = fp8.quantize(torch.tensor([x], dtype=torch.bfloat16), scale).item()
    assert got == two_step
    q = Fraction(x) / Fraction(scale)
    lo, hi = fp8.e4m3_decode(torch.tensor([direct], dtype=torch.uint8)).item(), \
        fp8.e4m3_decode(torch.tensor([two_step], dtype=torch.uint8)).item()
    assert Fraction(lo) < q < (Fraction(lo) + Fraction(hi)) / 2  # exact rounding would give `direct`
    assert float(np.float32(x) / np.float32(scale)) == (lo + hi) / 2  # the fp32 quotient is the midpoint
