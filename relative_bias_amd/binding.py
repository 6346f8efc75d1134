"""ctypes binding for librpa.so: argument marshalling only.

Every step of the computation runs in the library's HIP kernels.  These
wrappers check dtypes, devices and contiguity of torch tensors, allocate
outputs and workspace with torch when the caller does not pass them, and
forward raw device pointers plus the current HIP stream through the C ABI
declared in include/rpa.h.  If the library is missing they raise; there is no
fallback implementation.

The keyword signature of ``rpa_attn_varlen`` mirrors the op wrapper in the
Inkling FA4 relative-attention walkthrough ("主函数
inkling_fa4_rel_attention"): window (-1, -1) means none, ``out=None``
allocates, ``num_splits=None`` asks the planner.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librpa.so")

RPA_OK = 0
RPA_MAX_SPLITS = 128
_STATUS = {0: "RPA_OK", -1: "RPA_ERR_NULL", -2: "RPA_ERR_SHAPE", -3: "RPA_ERR_UNSUPPORTED",
           -4: "RPA_ERR_WORKSPACE", -5: "RPA_ERR_HIP"}

_lib = None


class RpaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().rpa_status_string(status).decode() if _lib is not None else ""
        super().__init__(f"{where}: {_STATUS.get(status, status)} ({msg})")


def lib():
    """Load librpa.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m relative_bias_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.rpa_attn_varlen.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                  f32, ctypes.c_int, i32, i32, i32, vp, i32, vp, sz, vp, vp, vp]
    L.rpa_attn_varlen.restype = ctypes.c_int
    L.rpa_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.rpa_workspace_bytes.restype = sz
    L.rpa_split_combine.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp]
    L.rpa_split_combine.restype = ctypes.c_int
    L.rpa_choose_splits.argtypes = [i32, i32, i32, i32, i64, ctypes.c_int, i32]
    L.rpa_choose_splits.restype = ctypes.c_int
    L.rpa_status_string.argtypes = [ctypes.c_int]
    L.rpa_status_string.restype = ctypes.c_char_p
    L.rpa_slot_mapping.argtypes = [vp, i32, vp, vp, i32, i32, i32, vp, vp]
    L.rpa_slot_mapping.restype = ctypes.c_int
    L.rpa_kv_cache_write.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
    L.rpa_kv_cache_write.restype = ctypes.c_int
    L.rpa_attn_varlen_fp8.argtypes = [vp, vp, vp, f32, f32, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                      i32, f32, ctypes.c_int, i32, i32, i32, vp, i32, vp, sz, vp, vp, vp]
    L.rpa_attn_varlen_fp8.restype = ctypes.c_int
    L.rpa_kv_cache_write_fp8.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, f32, f32, vp, vp, vp]
    L.rpa_kv_cache_write_fp8.restype = ctypes.c_int
    L.rpa_attn_varlen_ex.argtypes = [vp, vp, vp, ctypes.c_int, f32, f32, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                     i32, i32, i32, f32, ctypes.c_int, i32, i32, i32, vp, ctypes.c_int, vp, i32, vp,
                                     sz, vp, vp, vp]
    L.rpa_attn_varlen_ex.restype = ctypes.c_int
    L.rpa_attn_varlen_noalloc.argtypes = [vp, vp, vp, ctypes.c_int, f32, f32, vp, i32, vp, vp, i32, i32, i32, i32,
                                          i32, i32, i32, i32, f32, ctypes.c_int, i32, i32, i32, vp, ctypes.c_int, vp,
                                          i32, vp, vp, vp]
    L.rpa_attn_varlen_noalloc.restype = ctypes.c_int
    _lib = L
    return L


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _alibi(alibi_slopes, H: int, device):
    if alibi_slopes is None:
        return None
    a = alibi_slopes.contiguous()
    _check(a, "alibi_slopes", torch.float32, device, 1)
    if a.shape[0] != H:
        raise ValueError(f"alibi_slopes must have {H} entries, got {a.shape[0]}")
    return a


def _check(t: torch.Tensor, name: str, dtype, device, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def rpa_workspace_bytes(num_splits: int, num_tokens: int, num_heads: int, head_dim: int) -> int:
    return int(lib().rpa_workspace_bytes(num_splits, num_tokens, num_heads, head_dim))


def rpa_choose_splits(batch: int, max_seqlen_q: int, num_heads: int, num_kv_heads: int,
                      max_seqlen_k: int, is_local: bool = False, num_cus: int = 0) -> int:
    s = int(lib().rpa_choose_splits(batch, max_seqlen_q, num_heads, num_kv_heads, max_seqlen_k,
                                    int(bool(is_local)), num_cus))
    if s < 0:
        raise RpaError(s, "rpa_choose_splits")
    return s


def _attn(where: str, kv8: bool, k_scale: float, v_scale: float, q, key_cache, value_cache, block_table,
          cache_seqlens, cu_seqlens_q, max_seqlen_q, softmax_scale, causal, window_size, rel_extent, rel_logits,
          num_splits, max_seqlen_k, out, lse, return_lse, workspace, alibi_slopes, noalloc=False):
    """Checks shared by the attention wrappers, then the C call.

    Every tensor is checked for dtype, device, contiguity and shape before
    anything is launched: the kernels write T*H*D bf16 values to ``out`` and
    T*H fp32 values to ``lse``, so a buffer of another shape is refused here
    rather than written past its end.  ``noalloc`` calls
    rpa_attn_varlen_noalloc and allocates nothing: ``out`` must be given."""
    if noalloc:
        if out is None:
            raise ValueError(f"{where} allocates nothing: pass out (and lse to get the LSE)")
        if workspace is not None:
            raise ValueError(f"{where} takes no workspace (it uses the library's static scratch)")
        if return_lse and lse is None:
            raise ValueError(f"{where} allocates nothing: pass lse to get the LSE")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    _check(q, "q", torch.bfloat16, dev, 3)
    if kv8:
        key_cache = _fp8_cache(key_cache, "key_cache", dev)
        value_cache = _fp8_cache(value_cache, "value_cache", dev)
    else:
        _check(key_cache, "key_cache", torch.bfloat16, dev, 4)
        _check(value_cache, "value_cache", torch.bfloat16, dev, 4)
    if key_cache.shape != value_cache.shape:
        raise ValueError("key_cache and value_cache shapes differ")
    _check(block_table, "block_table", torch.int32, dev, 2)
    _check(cache_seqlens, "cache_seqlens", torch.int32, dev, 1)
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev, 1)
    T, H, D = q.shape
    NB, BS, Hkv, Dk = key_cache.shape
    if Dk != D:
        raise ValueError("head_dim of q and the caches differ")
    B = cache_seqlens.shape[0]
    if cu_seqlens_q.shape[0] != B + 1 or block_table.shape[0] != B:
        raise ValueError("batch sizes of cu_seqlens_q / block_table / cache_seqlens disagree")
    R = int(rel_extent)
    if R > 0:
        if rel_logits is None:
            raise ValueError("rel_extent > 0 needs rel_logits")
        if noalloc and not rel_logits.is_contiguous():
            raise ValueError(f"{where} allocates nothing: rel_logits must be contiguous")
        rel_logits = rel_logits.contiguous()  # the walkthrough's wrapper does the same
        _check(rel_logits, "rel_logits", torch.bfloat16 if rel_logits.dtype == torch.bfloat16 else torch.float32,
               dev, 3)
        if tuple(rel_logits.shape) != (T, H, R):
            raise ValueError(f"rel_logits must be {(T, H, R)}, got {tuple(rel_logits.shape)}")
    if num_splits is None:
        if max_seqlen_k is None:
            raise ValueError("num_splits=None needs max_seqlen_k for the planner")
        is_local = tuple(window_size) != (-1, -1)
        num_splits = rpa_choose_splits(B, max_seqlen_q, H, Hkv, max_seqlen_k, is_local)
    S = int(num_splits)
    if out is None:
        out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, dev, 3)
    if tuple(out.shape) != (T, H, D):
        raise ValueError(f"out must be {(T, H, D)}, got {tuple(out.shape)}")
    want_lse = return_lse or lse is not None
    if want_lse and lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", torch.float32, dev, 2)
        if tuple(lse.shape) != (T, H):
            raise ValueError(f"lse must be {(T, H)}, got {tuple(lse.shape)}")
    ws_bytes = rpa_workspace_bytes(S, T, H, D) if S != 1 and not noalloc else 0
    if ws_bytes and workspace is None:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    ws_given = 0 if workspace is None else workspace.numel() * workspace.element_size()
    alibi = _alibi(alibi_slopes, H, dev)
    rel_bf16 = int(R > 0 and rel_logits.dtype == torch.bfloat16)
    rel = _ptr(rel_logits) if R > 0 else None
    caches = (_ptr(q), _ptr(key_cache), _ptr(value_cache))
    meta = (_ptr(block_table), block_table.shape[1], _ptr(cache_seqlens), _ptr(cu_seqlens_q), B, T, H, Hkv, D, NB,
            BS, int(max_seqlen_q), float(softmax_scale), int(bool(causal)), int(window_size[0]),
            int(window_size[1]), R)
    tail = (S, _ptr(workspace), ws_given, _ptr(out), _ptr(lse), _stream(dev))
    L = lib()
    if noalloc:
        st = L.rpa_attn_varlen_noalloc(*caches, int(kv8), float(k_scale), float(v_scale), *meta, rel, rel_bf16,
                                       _ptr(alibi), S, _ptr(out), _ptr(lse), _stream(dev))
    elif alibi is not None or rel_bf16:
        st = L.rpa_attn_varlen_ex(*caches, int(kv8), float(k_scale), float(v_scale), *meta, rel, rel_bf16,
                                  _ptr(alibi), *tail)
    elif kv8:
        st = L.rpa_attn_varlen_fp8(*caches, float(k_scale), float(v_scale), *meta, rel, *tail)
    else:
        st = L.rpa_attn_varlen(*caches, *meta, rel, *tail)
    if st != RPA_OK:
        raise RpaError(st, where)
    return (out, lse) if want_lse else out


def rpa_attn_varlen(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor, *,
                    block_table: torch.Tensor, cache_seqlens: torch.Tensor,
                    cu_seqlens_q: torch.Tensor, max_seqlen_q: int, softmax_scale: float,
                    causal: bool = True, window_size: Tuple[int, int] = (-1, -1),
                    rel_extent: int = 0, rel_logits: Optional[torch.Tensor] = None,
                    num_splits: Optional[int] = None, max_seqlen_k: Optional[int] = None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    return_lse: bool = False, workspace: Optional[torch.Tensor] = None,
                    alibi_slopes: Optional[torch.Tensor] = None):
    """Paged varlen causal attention with the additive relative bias
    (rel_logits fp32 or bf16; optional ALiBi slopes, fp32 [H]: both through
    rpa_attn_varlen_ex).

    Returns ``out`` (bf16 [T, H, D]), or ``(out, lse)`` when ``return_lse``
    or an ``lse`` tensor is given.  ``num_splits=None`` uses
    rpa_choose_splits, which needs ``max_seqlen_k`` (host int) to be given.
    """
    return _attn("rpa_attn_varlen", False, 1.0, 1.0, q, key_cache, value_cache, block_table, cache_seqlens,
                 cu_seqlens_q, max_seqlen_q, softmax_scale, causal, window_size, rel_extent, rel_logits,
                 num_splits, max_seqlen_k, out, lse, return_lse, workspace, alibi_slopes)


def rpa_attn_varlen_noalloc(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor, *,
                            out: torch.Tensor, block_table: torch.Tensor, cache_seqlens: torch.Tensor,
                            cu_seqlens_q: torch.Tensor, max_seqlen_q: int, softmax_scale: float,
                            causal: bool = True, window_size: Tuple[int, int] = (-1, -1), rel_extent: int = 0,
                            rel_logits: Optional[torch.Tensor] = None, num_splits: int = 0,
                            lse: Optional[torch.Tensor] = None, kv_e4m3: bool = False, k_scale: float = 1.0,
                            v_scale: float = 1.0, alibi_slopes: Optional[torch.Tensor] = None):
    """rpa_attn_varlen_ex without a workspace or any allocation (the library's
    static per-device scratch holds the split partials): for callers that
    cannot allocate.  ``out`` (and ``lse`` when wanted) are the caller's; E4M3
    caches are passed with ``kv_e4m3=True`` and their scales.  Returns ``out``,
    or ``(out, lse)`` when ``lse`` is given."""
    if kv_e4m3:
        key_cache = _fp8_cache(key_cache, "key_cache", q.device)
        value_cache = _fp8_cache(value_cache, "value_cache", q.device)
    return _attn("rpa_attn_varlen_noalloc", bool(kv_e4m3), k_scale, v_scale, q, key_cache, value_cache,
                 block_table, cache_seqlens, cu_seqlens_q, max_seqlen_q, softmax_scale, causal, window_size,
                 rel_extent, rel_logits, num_splits, None, out, lse, False, None, alibi_slopes, noalloc=True)


def _fp8_cache(t: torch.Tensor, name: str, device) -> torch.Tensor:
    """An E4M3 cache given as uint8 codes or torch.float8_e4m3fn, seen as uint8."""
    if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    _check(t, name, torch.uint8, device, 4)
    return t


def rpa_attn_varlen_fp8(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor, *,
                        k_scale: float, v_scale: float, block_table: torch.Tensor, cache_seqlens: torch.Tensor,
                        cu_seqlens_q: torch.Tensor, max_seqlen_q: int, softmax_scale: float,
                        causal: bool = True, window_size: Tuple[int, int] = (-1, -1),
                        rel_extent: int = 0, rel_logits: Optional[torch.Tensor] = None,
                        num_splits: Optional[int] = 0, max_seqlen_k: Optional[int] = None,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        return_lse: bool = False, workspace: Optional[torch.Tensor] = None,
                        alibi_slopes: Optional[torch.Tensor] = None):
    """rpa_attn_varlen over E4M3 caches (uint8 codes or float8_e4m3fn) with
    per-cache scales: k = e4m3(code) * k_scale, v = e4m3(code) * v_scale."""
    return _attn("rpa_attn_varlen_fp8", True, k_scale, v_scale, q, key_cache, value_cache, block_table,
                 cache_seqlens, cu_seqlens_q, max_seqlen_q, softmax_scale, causal, window_size, rel_extent,
                 rel_logits, num_splits, max_seqlen_k, out, lse, return_lse, workspace, alibi_slopes)


def rpa_kv_cache_write_fp8(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
                           key_cache: torch.Tensor, value_cache: torch.Tensor, k_scale: float,
                           v_scale: float) -> None:
    """Quantise key/value [T, Hkv, D] (bf16) to E4M3 with k_scale / v_scale
    and write the codes into the paged caches at their slots."""
    dev = key.device
    _check(key, "key", torch.bfloat16, dev, 3)
    _check(value, "value", torch.bfloat16, dev, 3)
    _check(slot_mapping, "slot_mapping", torch.int64, dev, 1)
    key_cache = _fp8_cache(key_cache, "key_cache", dev)
    value_cache = _fp8_cache(value_cache, "value_cache", dev)
    T, Hkv, D = key.shape
    NB, BS = key_cache.shape[0], key_cache.shape[1]
    if tuple(value.shape) != (T, Hkv, D) or slot_mapping.shape[0] != T:
        raise ValueError("key / value / slot_mapping shapes disagree")
    if tuple(key_cache.shape) != (NB, BS, Hkv, D) or tuple(value_cache.shape) != (NB, BS, Hkv, D):
        raise ValueError("cache shapes disagree with key")
    st = lib().rpa_kv_cache_write_fp8(_ptr(key), _ptr(value), _ptr(slot_mapping), T, Hkv, D, NB, BS,
                                      float(k_scale), float(v_scale), _ptr(key_cache), _ptr(value_cache),
                                      _stream(dev))
    if st != RPA_OK:
        raise RpaError(st, "rpa_kv_cache_write_fp8")


def rpa_split_combine(partial_out: torch.Tensor, partial_lse: torch.Tensor,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Merge normalised split partials [S, T, H, D] / [S, T, H] -> (out, lse)."""
    dev = partial_out.device
    _check(partial_out, "partial_out", torch.float32, dev, 4)
    _check(partial_lse, "partial_lse", torch.float32, dev, 3)
    S, T, H, D = partial_out.shape
    if tuple(partial_lse.shape) != (S, T, H):
        raise ValueError("partial_lse shape does not match partial_out")
    if out is None:
        out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    _check(out, "out", torch.bfloat16, dev, 3)
    _check(lse, "lse", torch.float32, dev, 2)
    if tuple(out.shape) != (T, H, D) or tuple(lse.shape) != (T, H):
        raise ValueError(f"out must be {(T, H, D)} and lse {(T, H)}, got {tuple(out.shape)} and {tuple(lse.shape)}")
    st = lib().rpa_split_combine(_ptr(partial_out), _ptr(partial_lse), S, T, H, D, _ptr(out),
                                 _ptr(lse), _stream(dev))
    if st != RPA_OK:
        raise RpaError(st, "rpa_split_combine")
    return out, lse


def rpa_slot_mapping(block_table: torch.Tensor, cache_seqlens: torch.Tensor, cu_seqlens_q: torch.Tensor,
                     block_size: int, out: Optional[torch.Tensor] = None,
                     num_tokens: Optional[int] = None) -> torch.Tensor:
    """Cache slot (int64) of every packed query token; -1 where a request has
    fewer keys than queries.

    The token count is a host value: pass ``out`` (int64 [T]) or
    ``num_tokens``.  It is never read back from ``cu_seqlens_q`` on the
    device, so the call stays asynchronous and can be captured in a graph."""
    dev = cu_seqlens_q.device
    _check(block_table, "block_table", torch.int32, dev, 2)
    _check(cache_seqlens, "cache_seqlens", torch.int32, dev, 1)
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev, 1)
    B = cache_seqlens.shape[0]
    if cu_seqlens_q.shape[0] != B + 1 or block_table.shape[0] != B:
        raise ValueError("batch sizes of block_table / cache_seqlens / cu_seqlens_q disagree")
    if out is None:
        if num_tokens is None:
            raise ValueError("rpa_slot_mapping needs out or num_tokens (the host-side token count)")
        out = torch.empty((int(num_tokens),), dtype=torch.int64, device=dev)
    elif num_tokens is not None and out.shape[0] != int(num_tokens):
        raise ValueError(f"out holds {out.shape[0]} slots, num_tokens is {num_tokens}")
    T = out.shape[0]
    _check(out, "slot_mapping", torch.int64, dev, 1)
    st = lib().rpa_slot_mapping(_ptr(block_table), block_table.shape[1], _ptr(cache_seqlens), _ptr(cu_seqlens_q),
                                B, T, block_size, _ptr(out), _stream(dev))
    if st != RPA_OK:
        raise RpaError(st, "rpa_slot_mapping")
    return out


def rpa_kv_cache_write(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
                       key_cache: torch.Tensor, value_cache: torch.Tensor) -> None:
    """Write key/value [T, Hkv, D] rows into the paged caches at their slots."""
    dev = key.device
    _check(key, "key", torch.bfloat16, dev, 3)
    _check(value, "value", torch.bfloat16, dev, 3)
    _check(slot_mapping, "slot_mapping", torch.int64, dev, 1)
    _check(key_cache, "key_cache", torch.bfloat16, dev, 4)
    _check(value_cache, "value_cache", torch.bfloat16, dev, 4)
    T, Hkv, D = key.shape
    NB, BS = key_cache.shape[0], key_cache.shape[1]
    if tuple(value.shape) != (T, Hkv, D) or slot_mapping.shape[0] != T:
        raise ValueError("key / value / slot_mapping shapes disagree")
    if tuple(key_cache.shape) != (NB, BS, Hkv, D) or tuple(value_cache.shape) != (NB, BS, Hkv, D):
        raise ValueError("cache shapes disagree with key")
    st = lib().rpa_kv_cache_write(_ptr(key), _ptr(value), _ptr(slot_mapping), T, Hkv, D, NB, BS,
                                  _ptr(key_cache), _ptr(value_cache), _stream(dev))
    if st != RPA_OK:
        raise RpaError(st, "rpa_kv_cache_write")


def attn_workload(w, *, num_splits: Optional[int] = None, return_lse: bool = True, out=None, lse=None,
                  workspace=None, alibi_slopes=None):
    """Run rpa_attn_varlen on a relative_bias_amd.workloads.Workload (on the GPU)."""
    S = num_splits if num_splits is not None else w.num_splits
    return rpa_attn_varlen(
        w.q, w.key_cache, w.value_cache, block_table=w.block_table, cache_seqlens=w.cache_seqlens,
        cu_seqlens_q=w.cu_seqlens_q, max_seqlen_q=w.max_seqlen_q, softmax_scale=w.softmax_scale,
        causal=w.causal, window_size=w.window_size, rel_extent=w.rel_extent, rel_logits=w.rel_logits,
        num_splits=S, max_seqlen_k=max(w.k_lens + [0]), return_lse=return_lse, out=out, lse=lse,
        workspace=workspace, alibi_slopes=alibi_slopes)
