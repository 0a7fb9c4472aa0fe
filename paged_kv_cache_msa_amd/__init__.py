"""MiniMax-M3 MSA fused producer on AMD Instinct MI355X (gfx950).

Thin ctypes binding of libmsa_produce.so (C ABI in include/msa_produce.h).  Every function here
only marshals arguments (tensor data pointers, strides, the current HIP stream); all
computation runs in the library's HIP kernels.  If the library is not built the functions raise.

Entry points (same names as the C ABI):
  msa_produce(...)      one fused producer launch: per-head RMSNorm + neox RoPE on Q, K, index-Q
                        and index-K; compact bf16 Q / index-Q; K, V, index-K written into paged HND
                        caches (fp8 e4m3 or bf16) at the slot page_table[seq][pos // P] * P + pos % P,
                        padded or out-of-range slots skipped.
  msa_rope_table(...)   the RoPE coefficients alone.
  msa_quantize(...)     the output casts alone.
  msa_rms_scale(...)    the RMSNorm scale alone.
  msa_index_scores(...) indexer: block max of the exact dot products of index-Q with the visible keys
                        of the index-K cache (include/msa_index.h).
  msa_index_topk(...)   indexer: the top-k blocks of every (index-Q head, token) row.
  msa_project(...)      the packed projection x = bf16(h w^T) on the matrix cores (include/msa_project.h).
  msa_project_produce(...)  the same projection with the producer as its epilogue: the packed row
                        never touches memory.
  msa_slots(...)        the cache slot of every token (include/msa_unfused.h).
  msa_produce_unfused(...)  the same outputs as msa_produce through the unfused path: separate
                        main and index norm/RoPE producers, then division, remainder, index cast
                        and scatter per cache (14 launches per layer); takes any positive,
                        non-overlapping cache strides.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmsa_produce.so")

MSA_CACHE_FP8_E4M3 = 0
MSA_CACHE_BF16 = 1

STATUS = {
    0: "MSA_OK", 1: "MSA_ERR_NULL_POINTER", 2: "MSA_ERR_UNSUPPORTED", 3: "MSA_ERR_SHAPE",
    4: "MSA_ERR_STRIDE", 5: "MSA_ERR_ALIGNMENT", 6: "MSA_ERR_DTYPE", 7: "MSA_ERR_OVERFLOW",
    8: "MSA_ERR_LAUNCH", 9: "MSA_ERR_WORKSPACE",
}


class MsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({string(status)})")


class MsaCacheView(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("stride_page", ctypes.c_int64),
        ("stride_head", ctypes.c_int64),
        ("stride_token", ctypes.c_int64),
        ("num_heads", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmsa_produce.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32, f32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_double
        cv = ctypes.POINTER(MsaCacheView)
        L.msa_produce.argtypes = [p, i64, i32, i32, i32, i32, i32, i32, p, p, p, i64, i32, i32, i32, i64,
                                  p, p, p, p, f32, f64, p, p, cv, cv, cv, p, p]
        L.msa_produce.restype = ctypes.c_int
        L.msa_rope_table.argtypes = [p, i64, f64, i32, p, p, p]
        L.msa_rope_table.restype = ctypes.c_int
        L.msa_quantize.argtypes = [p, i64, i32, p, p, p]
        L.msa_quantize.restype = ctypes.c_int
        L.msa_rms_scale.argtypes = [p, i64, i32, f32, p, p]
        L.msa_rms_scale.restype = ctypes.c_int
        L.msa_index_scores.argtypes = [p, i32, i32, i32, p, p, p, i64, i32, i32, i32, i64, cv, i32, i32, p, p]
        L.msa_index_scores.restype = ctypes.c_int
        L.msa_index_topk.argtypes = [p, i32, i32, i32, p, p, p]
        L.msa_index_topk.restype = ctypes.c_int
        u64 = ctypes.c_uint64
        L.msa_slots.argtypes = [p, p, i32, p, i64, i32, i32, i32, i64, p, p]
        L.msa_slots.restype = ctypes.c_int
        L.msa_produce_unfused_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(u64)]
        L.msa_produce_unfused_workspace_size.restype = ctypes.c_int
        L.msa_produce_unfused.argtypes = [p, i64, i32, i32, i32, i32, i32, i32, p, p, i32, i64,
                                          p, p, p, p, f32, f64, p, p, cv, cv, cv, p, u64, p]
        L.msa_produce_unfused.restype = ctypes.c_int
        L.msa_project_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(u64)]
        L.msa_project_workspace_size.restype = ctypes.c_int
        L.msa_project.argtypes = [p, i64, i32, i32, p, i64, i32, p, i64, p, u64, p]
        L.msa_project.restype = ctypes.c_int
        L.msa_project_produce.argtypes = [p, i64, i32, i32, p, i64, i32, i32, i32, i32, i32, p, p, p, i32, i64,
                                          p, p, p, p, f32, p, p, cv, cv, cv, p, u64, p]
        L.msa_project_produce.restype = ctypes.c_int
        L.msa_status_string.argtypes = [ctypes.c_int]
        L.msa_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def string(status: int) -> str:
    return lib().msa_status_string(int(status)).decode()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def cache_view(cache, scale=None) -> Optional[MsaCacheView]:
    """Descriptor of a 4-D tensor view [num_pages, heads, page_size, head_dim] (dim stride 1).
    1-byte elements are taken as fp8 e4m3 (scale: a 1-element float32 device tensor), 2-byte
    elements as bf16."""
    if cache is None:
        return None
    if cache.dim() != 4 or cache.stride(3) != 1:
        raise ValueError("cache must be a 4-D view [pages, heads, page_size, head_dim] with dim stride 1")
    es = cache.element_size()
    if es not in (1, 2):
        raise ValueError("cache elements must be 1 byte (fp8 e4m3) or 2 bytes (bf16)")
    dtype = MSA_CACHE_FP8_E4M3 if es == 1 else MSA_CACHE_BF16
    return MsaCacheView(cache.data_ptr(), cache.stride(0), cache.stride(1), cache.stride(2), cache.shape[1], dtype,
                        None if scale is None else scale.data_ptr())


def msa_produce(x, positions, seq_idx, page_table, q_norm_weight, k_norm_weight, iq_norm_weight, ik_norm_weight,
                q_out, iq_out, k_cache, v_cache, ik_cache=None, *, k_scale=None, v_scale=None, ik_scale=None,
                num_pages: Optional[int] = None, rms_eps: float = 1e-6, rope_theta: float = 1e4,
                slots_out=None, stream=None) -> None:
    """One fused-producer launch on the current (or given) stream.

    x [T, >= W] bf16 rows (column stride 1); positions, seq_idx int32 [T]; page_table int32
    [num_seqs, max_pages] (row stride taken from the tensor); *_norm_weight bf16 [128] (None for an
    empty stream); q_out bf16 [T, Hq, 128]; iq_out bf16 [T, Hiq, 128]; caches 4-D views
    [num_pages, H, page_size, 128] of 1-byte (fp8, with a float32 [1] scale) or 2-byte (bf16)
    elements.  Head counts, page size and pool size are read from the output and cache shapes.
    """
    T = x.shape[0]
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    hq, hiq = q_out.shape[1], iq_out.shape[1]
    hkv = k_cache.shape[1] if k_cache is not None else 0
    hik = ik_cache.shape[1] if ik_cache is not None else 0
    ref = k_cache if k_cache is not None else ik_cache
    page_size = ref.shape[2]
    pages = ref.shape[0] if num_pages is None else num_pages
    kv = cache_view(k_cache, k_scale)
    vv = cache_view(v_cache, v_scale)
    iv = cache_view(ik_cache, ik_scale)
    st = lib().msa_produce(
        _ptr(x), x.stride(0), T, 128, hq, hkv, hiq, hik, _ptr(positions), _ptr(seq_idx), _ptr(page_table),
        page_table.stride(0), page_table.shape[0], page_table.shape[1], page_size, pages,
        _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(iq_norm_weight), _ptr(ik_norm_weight),
        float(rms_eps), float(rope_theta), _ptr(q_out), _ptr(iq_out),
        None if kv is None else ctypes.byref(kv), None if vv is None else ctypes.byref(vv),
        None if iv is None else ctypes.byref(iv), _ptr(slots_out), _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_produce")


def msa_rope_table(positions, cos_out, sin_out, rope_theta: float = 1e4, head_dim: int = 128, stream=None) -> None:
    st = lib().msa_rope_table(_ptr(positions), positions.numel(), float(rope_theta), head_dim, _ptr(cos_out),
                              _ptr(sin_out), _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_rope_table")


def msa_quantize(values, codes_out, dtype: int, scale=None, stream=None) -> None:
    st = lib().msa_quantize(_ptr(values), values.numel(), int(dtype), _ptr(scale), _ptr(codes_out), _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_quantize")


def msa_rms_scale(sum_sq, r_out, rms_eps: float, head_dim: int = 128, stream=None) -> None:
    st = lib().msa_rms_scale(_ptr(sum_sq), sum_sq.numel(), head_dim, float(rms_eps), _ptr(r_out), _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_rms_scale")


def msa_index_scores(iq, positions, seq_idx, page_table, ik_cache, block_scores, *, ik_scale=None,
                     num_pages: Optional[int] = None, block_tokens: int = 128, stream=None) -> None:
    """Indexer block scores.  iq [T, Hiq, 128] bf16; ik_cache a 4-D index-K cache view
    [num_pages, Hik, page_size, 128] (1-byte fp8 with a float32 [1] scale, or 2-byte bf16);
    block_scores float64 [Hiq, T, max_blocks]."""
    T, hiq = iq.shape[0], iq.shape[1]
    view = cache_view(ik_cache, ik_scale)
    pages = ik_cache.shape[0] if num_pages is None else num_pages
    st = lib().msa_index_scores(_ptr(iq), T, 128, hiq, _ptr(positions), _ptr(seq_idx), _ptr(page_table),
                                page_table.stride(0), page_table.shape[0], page_table.shape[1], ik_cache.shape[2],
                                pages, ctypes.byref(view), int(block_tokens), block_scores.shape[-1],
                                _ptr(block_scores), _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_index_scores")


def msa_index_topk(block_scores, block_ids, counts=None, stream=None) -> None:
    """Top-k blocks of every row of block_scores [..., max_blocks] into block_ids [..., top_k] (int32)."""
    nb = block_scores.shape[-1]
    rows = block_scores.numel() // nb if nb else 0
    st = lib().msa_index_topk(_ptr(block_scores), rows, nb, block_ids.shape[-1], _ptr(block_ids), _ptr(counts),
                              _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_index_topk")


def msa_slots(positions, seq_idx, page_table, slots_out, *, page_size: int, num_pages: int, stream=None) -> None:
    """slots_out[t] = page_table[seq][pos // page_size] * page_size + pos % page_size, or -1."""
    st = lib().msa_slots(_ptr(positions), _ptr(seq_idx), positions.numel(), _ptr(page_table), page_table.stride(0),
                         page_table.shape[0], page_table.shape[1], int(page_size), int(num_pages), _ptr(slots_out),
                         _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_slots")


def msa_produce_unfused_workspace_size(num_tokens: int, num_kv_heads: int, num_ik_heads: int) -> int:
    n = ctypes.c_uint64(0)
    st = lib().msa_produce_unfused_workspace_size(int(num_tokens), int(num_kv_heads), int(num_ik_heads),
                                                  ctypes.byref(n))
    if st != 0:
        raise MsaError(st, "msa_produce_unfused_workspace_size")
    return n.value


def msa_produce_unfused(x, positions, slots, q_norm_weight, k_norm_weight, iq_norm_weight, ik_norm_weight,
                        q_out, iq_out, k_cache, v_cache, ik_cache=None, *, workspace, k_scale=None, v_scale=None,
                        ik_scale=None, num_pages: Optional[int] = None, rms_eps: float = 1e-6,
                        rope_theta: float = 1e4, stream=None) -> None:
    """msa_produce's outputs through the unfused path.  slots int64 [T] (msa_slots); workspace a
    device byte tensor of at least msa_produce_unfused_workspace_size bytes, 256-byte aligned."""
    T = x.shape[0]
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    hq, hiq = q_out.shape[1], iq_out.shape[1]
    hkv = k_cache.shape[1] if k_cache is not None else 0
    hik = ik_cache.shape[1] if ik_cache is not None else 0
    ref = k_cache if k_cache is not None else ik_cache
    pages = ref.shape[0] if num_pages is None else num_pages
    kv = cache_view(k_cache, k_scale)
    vv = cache_view(v_cache, v_scale)
    iv = cache_view(ik_cache, ik_scale)
    st = lib().msa_produce_unfused(
        _ptr(x), x.stride(0), T, 128, hq, hkv, hiq, hik, _ptr(positions), _ptr(slots), ref.shape[2], pages,
        _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(iq_norm_weight), _ptr(ik_norm_weight),
        float(rms_eps), float(rope_theta), _ptr(q_out), _ptr(iq_out),
        None if kv is None else ctypes.byref(kv), None if vv is None else ctypes.byref(vv),
        None if iv is None else ctypes.byref(iv), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_produce_unfused")


def msa_project_workspace_size(num_tokens: int, hidden: int, num_heads: int) -> int:
    """Bytes of (256-byte aligned) workspace the projection needs; 0 above 1,024 tokens."""
    n = ctypes.c_uint64(0)
    st = lib().msa_project_workspace_size(int(num_tokens), int(hidden), int(num_heads), ctypes.byref(n))
    if st != 0:
        raise MsaError(st, "msa_project_workspace_size")
    return n.value


def _ws(workspace):
    if workspace is None:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def msa_project(h, w, x_out, *, workspace=None, stream=None) -> None:
    """x_out[T, N] = bf16(h[T, K] @ w[N, K]^T); row strides taken from the tensors (unit column stride)."""
    for name, t in (("h", h), ("w", w), ("x_out", x_out)):
        if t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be 2-D with unit column stride")
    wp, wb = _ws(workspace)
    st = lib().msa_project(_ptr(h), h.stride(0), h.shape[0], h.shape[1], _ptr(w), w.stride(0), w.shape[0],
                           _ptr(x_out), x_out.stride(0), wp, wb, _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_project")


def msa_project_produce(h, w, rope_cos, rope_sin, slots, q_norm_weight, k_norm_weight, iq_norm_weight,
                        ik_norm_weight, q_out, iq_out, k_cache, v_cache, ik_cache=None, *, workspace=None,
                        k_scale=None, v_scale=None, ik_scale=None, num_pages: Optional[int] = None,
                        rms_eps: float = 1e-6, stream=None) -> None:
    """The projection with the producer as its epilogue.  h [T, K] bf16; w [W, K] bf16 (packed rows Q,
    K, V, index-Q, index-K); rope_cos / rope_sin float32 [T, 64] (msa_rope_table); slots int64 [T]
    (msa_slots); the rest as in msa_produce.  Head counts come from q_out, iq_out and the caches."""
    for name, t in (("h", h), ("w", w)):
        if t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be 2-D with unit column stride")
    hq, hiq = q_out.shape[1], iq_out.shape[1]
    hkv = k_cache.shape[1] if k_cache is not None else 0
    hik = ik_cache.shape[1] if ik_cache is not None else 0
    ref = k_cache if k_cache is not None else ik_cache
    pages = ref.shape[0] if num_pages is None else num_pages
    kv = cache_view(k_cache, k_scale)
    vv = cache_view(v_cache, v_scale)
    iv = cache_view(ik_cache, ik_scale)
    wp, wb = _ws(workspace)
    st = lib().msa_project_produce(
        _ptr(h), h.stride(0), h.shape[0], h.shape[1], _ptr(w), w.stride(0), 128, hq, hkv, hiq, hik,
        _ptr(rope_cos), _ptr(rope_sin), _ptr(slots), ref.shape[2], pages,
        _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(iq_norm_weight), _ptr(ik_norm_weight), float(rms_eps),
        _ptr(q_out), _ptr(iq_out), None if kv is None else ctypes.byref(kv), None if vv is None else ctypes.byref(vv),
        None if iv is None else ctypes.byref(iv), wp, wb, _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_project_produce")
