"""CPU oracle for the FP8 KV cache: the E4M3 code, quantise-at-store and
attention over dequantised pages.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library.

Pages cited:
* [PA-V2] "paged_attention_v2_pytorch.py — BI-V100 PagedAttention V2"
  (dev.modelhub.org.cn): the op takes ``kv_cache_dtype``, ``k_scale`` and
  ``v_scale``; the gathered key rows are turned into floats and multiplied
  by k_scale (values by v_scale) before the scores are formed.
* [V1-ATTN] "vLLM V1 Attention — Part 2: 标准Attention后端实现", chapter 12
  (TurboQuant): the cache holds K/V in a low-precision type such as FP8 with
  a scale factor; values are quantised when stored and dequantised when
  attention reads them.

Readings where the pages are silent (also listed in the design notes):
  F1 the FP8 type is OCP E4M3 ("e4m3fn"): 1 sign, 4 exponent bits with bias
     7, 3 mantissa bits, subnormals m * 2^-9, largest finite 448, no
     infinities, S.1111.111 is NaN.
  F2 one k_scale and one v_scale per cache (per-tensor, fp32, > 0): a
     stored code c stands for decode(c) * scale.
  F3 storing x: y = x / scale rounded once to fp32, then rounded to the
     nearest E4M3 value, ties to the even code; |y| beyond 448 (infinity
     included) saturates to +-448; NaN stores a NaN code with x's sign.
  F4 attention over an FP8 cache is the bf16 definition with K and V
     replaced by their dequantised values: the bias and the softmax scale
     are untouched by k_scale, and v_scale does not enter the LSE.

Every value here is computed in fp64 from the bit fields; no library FP8
conversion is used (the tests compare against torch's float8_e4m3fn as an
independent pin).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import attention as _attn
from . import kv_cache as _kv

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_encode", "quantize", "dequantize", "kv_cache_write_fp8",
           "attention_fp8"]

E4M3_MAX = 448.0


def _value_of_code(c: int) -> float:
    """F1: the real number an E4M3 code stands for (NaN for S.1111.111)."""
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_value_of_code(c) for c in range(256)], dtype=np.float64)
# Non-negative finite codes 0x00..0x7E in increasing order of value.
_POS = _TABLE[:0x7F].copy()


def e4m3_decode(codes: torch.Tensor) -> torch.Tensor:
    """fp64 values of uint8 E4M3 codes (F1)."""
    c = codes.to(torch.uint8).numpy().astype(np.int64)
    return torch.from_numpy(_TABLE[c])


def e4m3_encode(y) -> torch.Tensor:
    """uint8 E4M3 codes of fp32 values y, round to nearest, ties to the even
    code, saturating at +-448 (F3).  The distances to the two neighbouring
    grid values are exact in fp64 (an fp32 value minus an E4M3 value)."""
    a = torch.as_tensor(y, dtype=torch.float32).numpy().astype(np.float64)
    neg = np.signbit(a)
    nan = np.isnan(a)
    mag = np.abs(a)
    sat = ~nan & (mag >= E4M3_MAX)
    m = np.where(nan | sat, 0.0, mag)
    k = np.searchsorted(_POS, m, side="right") - 1  # _POS[k] <= m < _POS[k + 1]
    lo, hi = _POS[k], _POS[k + 1]
    dlo, dhi = m - lo, hi - m
    tie = np.where(k % 2 == 0, k, k + 1)  # the even code
    code = np.where(dlo < dhi, k, np.where(dlo > dhi, k + 1, tie))
    code = np.where(sat, 0x7E, code)
    code = np.where(nan, 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return torch.from_numpy(code.astype(np.uint8).reshape(a.shape))


def quantize(x: torch.Tensor, scale: float) -> torch.Tensor:
    """Codes of x / scale (F3): one fp32 division, then E4M3 rounding."""
    xf = x.to(torch.float32).numpy()
    y = xf / np.float32(scale)  # IEEE fp32 division, rounded once
    return e4m3_encode(torch.from_numpy(np.asarray(y, dtype=np.float32)))


def dequantize(codes: torch.Tensor, scale: float) -> torch.Tensor:
    """fp64 decode(code) * scale (F2), scale taken as its fp32 value."""
    s = float(np.float32(scale))
    return e4m3_decode(codes) * s


def kv_cache_write_fp8(key: torch.Tensor, value: torch.Tensor, slots: torch.Tensor, key_cache: torch.Tensor,
                       value_cache: torch.Tensor, k_scale: float, v_scale: float):
    """The paged KV write into uint8 E4M3 caches: each new row is quantised
    with its cache's scale (F3) and stored at its slot exactly as the bf16
    write stores it ([V1-ATTN] 6.5 step 2 and chapter 12)."""
    kq = quantize(key, k_scale)
    vq = quantize(value, v_scale)
    return _kv.kv_cache_write(kq, vq, slots, key_cache, value_cache)


def attention_fp8(q, key_cache8, value_cache8, k_scale, v_scale, block_table, cache_seqlens, cu_seqlens_q,
                  softmax_scale, causal=True, window_size=(-1, -1), rel_extent=0, rel_logits=None, **kw):
    """out [T, H, D] and lse [T, H] (fp64) of the method over uint8 E4M3
    caches: the definition of ``attention`` with K = decode(K8) * k_scale
    and V = decode(V8) * v_scale (F2, F4; [PA-V2] k_scale / v_scale)."""
    kc = dequantize(key_cache8, k_scale)
    vc = dequantize(value_cache8, v_scale)
    return _attn.attention(q, kc, vc, block_table, cache_seqlens, cu_seqlens_q, softmax_scale, causal,
                           window_size, rel_extent, rel_logits, **kw)
