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
                        of the index-K cache (include/msa_index.h); group_tokens > 1 calls
                        msa_index_scores_grouped (the same scores, key loads shared within groups).
  msa_index_topk(...)   indexer: the top-k blocks of every (index-Q head, token) row.
  msa_project(...)      the packed projection x = bf16(h w^T) on the matrix cores (include/msa_project.h).
  msa_project_produce(...)  the same projection with the producer as its epilogue: the packed row
                        never touches memory.
  msa_slots(...)        the cache slot of every token (include/msa_unfused.h).
  msa_produce_unfused(...)  the same outputs as msa_produce through the unfused path: separate
                        main and index norm/RoPE producers, then division, remainder, index cast
                        and scatter per cache (14 launches per layer); takes any positive,
                        non-overlapping cache strides.
  msa_project_produce_noalloc(...)  msa_project_produce with the library's static per-GPU scratch in place
                        of a workspace (allocates nothing; calls on one GPU must not overlap).
  msa_check_device_pointers(...)  the residency check eager calls run on their operands, alone.

Every wrapper checks its tensors' dtypes, shapes, extents and devices against the counts it hands to
the library and raises ValueError before anything is launched; the library then checks the
arguments it can see (counts, strides, alignment, operand residency) and returns a status, raised
here as MsaError.
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
    8: "MSA_ERR_LAUNCH", 9: "MSA_ERR_WORKSPACE", 10: "MSA_ERR_NOT_DEVICE",
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
        L.msa_index_scores_grouped.argtypes = [p, i32, i32, i32, p, p, p, i64, i32, i32, i32, i64, cv, i32, i32, i32,
                                               p, p]
        L.msa_index_scores_grouped.restype = ctypes.c_int
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
        L.msa_project_produce_noalloc.argtypes = [p, i64, i32, i32, p, i64, i32, i32, i32, i32, i32, p, p, p, i32,
                                                  i64, p, p, p, p, f32, p, p, cv, cv, cv, p]
        L.msa_project_produce_noalloc.restype = ctypes.c_int
        L.msa_status_string.argtypes = [ctypes.c_int]
        L.msa_status_string.restype = ctypes.c_char_p
        L.msa_status_str.argtypes = [ctypes.c_int]
        L.msa_status_str.restype = ctypes.c_char_p
        L.msa_check_device_pointers.argtypes = [p, p, i32, ctypes.POINTER(i32)]
        L.msa_check_device_pointers.restype = ctypes.c_int
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


# ------------------------------------------------------------------ tensor checks (before any launch)

def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _bytes(t) -> int:
    return t.element_size()


def _tensor(name, t, *, size=None, dim=None, contiguous=False, unit_last=False):
    """t must be a tensor of `size`-byte elements (a tuple: any of them), `dim` dims, contiguous or
    with a unit last stride as asked."""
    _need(t is not None, f"{name} is required")
    _need(hasattr(t, "data_ptr") and hasattr(t, "element_size"), f"{name} must be a tensor")
    if size is not None:
        sizes = size if isinstance(size, tuple) else (size,)
        _need(t.element_size() in sizes, f"{name} must have {' or '.join(map(str, sizes))}-byte elements, "
                                         f"got {t.dtype}")
    if dim is not None:
        _need(t.dim() == dim, f"{name} must have {dim} dimensions, got shape {tuple(t.shape)}")
    if contiguous:
        _need(t.is_contiguous(), f"{name} must be contiguous")
    if unit_last and t.dim() > 0:
        _need(t.stride(-1) == 1, f"{name} must have a unit last-dimension stride")


def _float(name, t, bits):
    import torch
    want = {32: torch.float32, 64: torch.float64}[bits]
    _need(t is not None and t.dtype == want, f"{name} must be a {want} tensor")


def _int(name, t, bits, min_numel):
    import torch
    want = {32: torch.int32, 64: torch.int64}[bits]
    _tensor(name, t, contiguous=True)
    _need(t.dtype == want, f"{name} must be a {want} tensor, got {t.dtype}")
    _need(t.numel() >= min_numel, f"{name} holds {t.numel()} elements, needs at least {min_numel}")


def _page_table(page_table):
    import torch
    _tensor("page_table", page_table, dim=2, unit_last=True)
    _need(page_table.dtype == torch.int32, f"page_table must be an int32 tensor, got {page_table.dtype}")


def _weights(ws, heads):
    for name, w, h in zip(("q_norm_weight", "k_norm_weight", "iq_norm_weight", "ik_norm_weight"), ws, heads):
        if h == 0 and w is None:
            continue
        _tensor(name, w, size=2, contiguous=True)
        _need(w.numel() == 128, f"{name} must hold 128 elements, got {w.numel()}")


def _rows_out(name, t, T, heads):
    """A compact [>= T, heads, 128] output of 2-byte elements."""
    if heads == 0 and t is None:
        return
    _tensor(name, t, size=2, dim=3, contiguous=True)
    _need(t.shape[1] == heads and t.shape[2] == 128, f"{name} must be [T, {heads}, 128], got {tuple(t.shape)}")
    _need(t.shape[0] >= T, f"{name} has {t.shape[0]} rows, needs {T}")


def _caches(k_cache, v_cache, ik_cache, num_pages, k_scale, v_scale, ik_scale):
    """Head counts, page size and pool size of three cache views, checked against each other."""
    _need((k_cache is None) == (v_cache is None), "k_cache and v_cache must be given together")
    present = [c for c in (k_cache, v_cache, ik_cache) if c is not None]
    _need(len(present) > 0, "at least one cache is required")
    for name, c, sc in (("k_cache", k_cache, k_scale), ("v_cache", v_cache, v_scale), ("ik_cache", ik_cache, ik_scale)):
        if c is None:
            continue
        _tensor(name, c, size=(1, 2), dim=4)
        _need(c.stride(3) == 1, f"{name} must have a unit head_dim stride")
        _need(c.shape[3] == 128, f"{name} must have head_dim 128, got {tuple(c.shape)}")
        if c.element_size() == 1:
            _float(f"{name}'s scale", sc, 32)
            _need(sc.numel() >= 1, f"{name}'s scale must hold one element")
    ref = present[0]
    page_size = ref.shape[2]
    pages = ref.shape[0] if num_pages is None else int(num_pages)
    for name, c in (("k_cache", k_cache), ("v_cache", v_cache), ("ik_cache", ik_cache)):
        if c is None:
            continue
        _need(c.shape[2] == page_size, f"{name} has page size {c.shape[2]}, the first cache {page_size}")
        _need(c.shape[0] >= pages, f"{name} holds {c.shape[0]} pages, the call addresses {pages}")
    if k_cache is not None:
        _need(v_cache.shape[1] == k_cache.shape[1], "k_cache and v_cache must have the same number of heads")
    hkv = k_cache.shape[1] if k_cache is not None else 0
    hik = ik_cache.shape[1] if ik_cache is not None else 0
    return hkv, hik, page_size, pages


def _same_device(*tensors):
    devs = {t.device for t in tensors if t is not None}
    for d in devs:
        _need(d.type == "cuda", f"every tensor must be a CUDA tensor, got one on {d}")
    _need(len(devs) <= 1, f"every tensor must be on one device, got {sorted(map(str, devs))}")
    if devs:
        import torch
        d = next(iter(devs))
        _need(d.index is None or d.index == torch.cuda.current_device(),
              f"the tensors are on {d}, the current device is cuda:{torch.cuda.current_device()}")


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


def _ref(v):
    return None if v is None else ctypes.byref(v)


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
    _tensor("x", x, size=2, dim=2, unit_last=True)
    T = x.shape[0]
    hkv, hik, page_size, pages = _caches(k_cache, v_cache, ik_cache, num_pages, k_scale, v_scale, ik_scale)
    _tensor("q_out", q_out, dim=3)
    _tensor("iq_out", iq_out, dim=3)
    hq, hiq = q_out.shape[1], iq_out.shape[1]
    _rows_out("q_out", q_out, T, hq)
    _rows_out("iq_out", iq_out, T, hiq)
    W = (hq + 2 * hkv + hiq + hik) * 128
    _need(x.shape[1] >= W, f"x has {x.shape[1]} columns, the heads need {W}")
    _int("positions", positions, 32, T)
    _int("seq_idx", seq_idx, 32, T)
    _page_table(page_table)
    _weights((q_norm_weight, k_norm_weight, iq_norm_weight, ik_norm_weight), (hq, hkv, hiq, hik))
    if slots_out is not None:
        _int("slots_out", slots_out, 64, T)
    _same_device(x, positions, seq_idx, page_table, q_norm_weight, k_norm_weight, iq_norm_weight, ik_norm_weight,
                 q_out, iq_out, k_cache, v_cache, ik_cache, k_scale if k_cache is not None else None,
                 v_scale if v_cache is not None else None, ik_scale if ik_cache is not None else None, slots_out)
    kv, vv, iv = cache_view(k_cache, k_scale), cache_view(v_cache, v_scale), cache_view(ik_cache, ik_scale)
    st = lib().msa_produce(
        _ptr(x), x.stride(0), T, 128, hq, hkv, hiq, hik, _ptr(positions), _ptr(seq_idx), _ptr(page_table),
        page_table.stride(0), page_table.shape[0], page_table.shape[1], page_size, pages,
        _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(iq_norm_weight), _ptr(ik_norm_weight),
        float(rms_eps), float(rope_theta), _ptr(q_out), _ptr(iq_out), _ref(kv), _ref(vv), _ref(iv),
        _ptr(slots_out), _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_produce")


def msa_rope_table(positions, cos_out, sin_out, rope_theta: float = 1e4, head_dim: int = 128, stream=None) -> None:
    """cos_out / sin_out float32 [n, 64] for positions int32 [n]."""
    _int("positions", positions, 32, 0)
    n = positions.numel()
    for name, t in (("cos_out", cos_out), ("sin_out", sin_out)):
        _tensor(name, t, contiguous=True)
        _float(name, t, 32)
        _need(t.numel() >= n * (head_dim // 2), f"{name} holds {t.numel()} elements, needs {n * (head_dim // 2)}")
    _same_device(positions, cos_out, sin_out)
    st = lib().msa_rope_table(_ptr(positions), n, float(rope_theta), head_dim, _ptr(cos_out), _ptr(sin_out),
                              _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_rope_table")


def msa_quantize(values, codes_out, dtype: int, scale=None, stream=None) -> None:
    """codes_out (1-byte for fp8, 2-byte for bf16) [n] from float32 values [n]."""
    _tensor("values", values, contiguous=True)
    _float("values", values, 32)
    n = values.numel()
    _tensor("codes_out", codes_out, size=1 if dtype == MSA_CACHE_FP8_E4M3 else 2, contiguous=True)
    _need(codes_out.numel() >= n, f"codes_out holds {codes_out.numel()} elements, needs {n}")
    if dtype == MSA_CACHE_FP8_E4M3:
        _float("scale", scale, 32)
    _same_device(values, codes_out, scale if dtype == MSA_CACHE_FP8_E4M3 else None)
    st = lib().msa_quantize(_ptr(values), n, int(dtype), _ptr(scale), _ptr(codes_out), _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_quantize")


def msa_rms_scale(sum_sq, r_out, rms_eps: float, head_dim: int = 128, stream=None) -> None:
    """r_out float32 [n] from binary64 sums of squares [n]."""
    _tensor("sum_sq", sum_sq, contiguous=True)
    _float("sum_sq", sum_sq, 64)
    _tensor("r_out", r_out, contiguous=True)
    _float("r_out", r_out, 32)
    _need(r_out.numel() >= sum_sq.numel(), "r_out is shorter than sum_sq")
    _same_device(sum_sq, r_out)
    st = lib().msa_rms_scale(_ptr(sum_sq), sum_sq.numel(), head_dim, float(rms_eps), _ptr(r_out), _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_rms_scale")


def msa_index_scores(iq, positions, seq_idx, page_table, ik_cache, block_scores, *, ik_scale=None,
                     num_pages: Optional[int] = None, block_tokens: int = 128, group_tokens: int = 1,
                     stream=None) -> None:
    """Indexer block scores.  iq [T, Hiq, 128] bf16; ik_cache a 4-D index-K cache view
    [num_pages, Hik, page_size, 128] (1-byte fp8 with a float32 [1] scale, or 2-byte bf16);
    block_scores float64 [Hiq, T, max_blocks].  group_tokens > 1 calls msa_index_scores_grouped
    (the same scores; consecutive tokens of one sequence share their key loads, e.g. verify windows)."""
    _tensor("iq", iq, size=2, dim=3, contiguous=True)
    T, hiq = iq.shape[0], iq.shape[1]
    _need(iq.shape[2] == 128, f"iq must be [T, Hiq, 128], got {tuple(iq.shape)}")
    _, _, page_size, pages = _caches(None, None, ik_cache, num_pages, None, None, ik_scale)
    _int("positions", positions, 32, T)
    _int("seq_idx", seq_idx, 32, T)
    _page_table(page_table)
    _tensor("block_scores", block_scores, dim=3, contiguous=True)
    _float("block_scores", block_scores, 64)
    _need(block_scores.shape[0] == hiq and block_scores.shape[1] == T,
          f"block_scores must be [{hiq}, {T}, max_blocks], got {tuple(block_scores.shape)}")
    _same_device(iq, positions, seq_idx, page_table, ik_cache, ik_scale if ik_cache.element_size() == 1 else None,
                 block_scores)
    view = cache_view(ik_cache, ik_scale)
    common = (_ptr(iq), T, 128, hiq, _ptr(positions), _ptr(seq_idx), _ptr(page_table), page_table.stride(0),
              page_table.shape[0], page_table.shape[1], page_size, pages, ctypes.byref(view), int(block_tokens),
              block_scores.shape[-1])
    if group_tokens == 1:
        st = lib().msa_index_scores(*common, _ptr(block_scores), _stream(stream))
    else:
        st = lib().msa_index_scores_grouped(*common, int(group_tokens), _ptr(block_scores), _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_index_scores" if group_tokens == 1 else "msa_index_scores_grouped")


def msa_index_topk(block_scores, block_ids, counts=None, stream=None) -> None:
    """Top-k blocks of every row of block_scores [..., max_blocks] into block_ids [..., top_k] (int32)."""
    import torch
    _tensor("block_scores", block_scores, contiguous=True)
    _float("block_scores", block_scores, 64)
    _need(block_scores.dim() >= 1, "block_scores must have a block dimension")
    nb = block_scores.shape[-1]
    rows = block_scores.numel() // nb if nb else 0
    _tensor("block_ids", block_ids, contiguous=True)
    _need(block_ids.dtype == torch.int32 and block_ids.dim() >= 1, "block_ids must be an int32 tensor [..., top_k]")
    k = block_ids.shape[-1]
    _need(block_ids.numel() >= rows * k, f"block_ids holds {block_ids.numel()} elements, needs {rows * k}")
    if counts is not None:
        _int("counts", counts, 32, rows)
    _same_device(block_scores, block_ids, counts)
    st = lib().msa_index_topk(_ptr(block_scores), rows, nb, k, _ptr(block_ids), _ptr(counts), _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_index_topk")


def msa_slots(positions, seq_idx, page_table, slots_out, *, page_size: int, num_pages: int, stream=None) -> None:
    """slots_out[t] = page_table[seq][pos // page_size] * page_size + pos % page_size, or -1."""
    _int("positions", positions, 32, 0)
    T = positions.numel()
    _int("seq_idx", seq_idx, 32, T)
    _page_table(page_table)
    _int("slots_out", slots_out, 64, T)
    _same_device(positions, seq_idx, page_table, slots_out)
    st = lib().msa_slots(_ptr(positions), _ptr(seq_idx), T, _ptr(page_table), page_table.stride(0),
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


def _workspace(workspace, need):
    if need == 0 and workspace is None:
        return None, 0
    _tensor("workspace", workspace, contiguous=True)
    nbytes = workspace.numel() * workspace.element_size()
    _need(nbytes >= need, f"workspace holds {nbytes} bytes, the call needs {need}")
    return workspace.data_ptr(), nbytes


def msa_produce_unfused(x, positions, slots, q_norm_weight, k_norm_weight, iq_norm_weight, ik_norm_weight,
                        q_out, iq_out, k_cache, v_cache, ik_cache=None, *, workspace, k_scale=None, v_scale=None,
                        ik_scale=None, num_pages: Optional[int] = None, rms_eps: float = 1e-6,
                        rope_theta: float = 1e4, stream=None) -> None:
    """msa_produce's outputs through the unfused path.  slots int64 [T] (msa_slots); workspace a
    device byte tensor of at least msa_produce_unfused_workspace_size bytes, 256-byte aligned."""
    _tensor("x", x, size=2, dim=2, unit_last=True)
    T = x.shape[0]
    hkv, hik, page_size, pages = _caches(k_cache, v_cache, ik_cache, num_pages, k_scale, v_scale, ik_scale)
    _tensor("q_out", q_out, dim=3)
    _tensor("iq_out", iq_out, dim=3)
    hq, hiq = q_out.shape[1], iq_out.shape[1]
    _rows_out("q_out", q_out, T, hq)
    _rows_out("iq_out", iq_out, T, hiq)
    W = (hq + 2 * hkv + hiq + hik) * 128
    _need(x.shape[1] >= W, f"x has {x.shape[1]} columns, the heads need {W}")
    _int("positions", positions, 32, T)
    _int("slots", slots, 64, T)
    _weights((q_norm_weight, k_norm_weight, iq_norm_weight, ik_norm_weight), (hq, hkv, hiq, hik))
    wp, wb = _workspace(workspace, msa_produce_unfused_workspace_size(T, hkv, hik))
    _same_device(x, positions, slots, q_norm_weight, k_norm_weight, iq_norm_weight, ik_norm_weight, q_out, iq_out,
                 k_cache, v_cache, ik_cache, workspace)
    kv, vv, iv = cache_view(k_cache, k_scale), cache_view(v_cache, v_scale), cache_view(ik_cache, ik_scale)
    st = lib().msa_produce_unfused(
        _ptr(x), x.stride(0), T, 128, hq, hkv, hiq, hik, _ptr(positions), _ptr(slots), page_size, pages,
        _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(iq_norm_weight), _ptr(ik_norm_weight),
        float(rms_eps), float(rope_theta), _ptr(q_out), _ptr(iq_out), _ref(kv), _ref(vv), _ref(iv), wp, wb,
        _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_produce_unfused")


def msa_project_workspace_size(num_tokens: int, hidden: int, num_heads: int) -> int:
    """Bytes of (256-byte aligned) workspace the projection needs; 0 above 1,024 tokens.  Allocate it
    zero-filled (torch.zeros) before its first use: the split-K launch exchanges partial sums in it and
    every completed call leaves it all zero again."""
    n = ctypes.c_uint64(0)
    st = lib().msa_project_workspace_size(int(num_tokens), int(hidden), int(num_heads), ctypes.byref(n))
    if st != 0:
        raise MsaError(st, "msa_project_workspace_size")
    return n.value


def _gemm_operands(h, w):
    _tensor("h", h, size=2, dim=2, unit_last=True)
    _tensor("w", w, size=2, dim=2, unit_last=True)
    _need(w.shape[1] == h.shape[1], f"w has {w.shape[1]} columns, h has {h.shape[1]}")
    return h.shape[0], h.shape[1], w.shape[0]


def msa_project(h, w, x_out, *, workspace=None, stream=None) -> None:
    """x_out[T, N] = bf16(h[T, K] @ w[N, K]^T); row strides taken from the tensors (unit column stride)."""
    T, K, N = _gemm_operands(h, w)
    _tensor("x_out", x_out, size=2, dim=2, unit_last=True)
    _need(x_out.shape[0] >= T and x_out.shape[1] >= N, f"x_out must be at least [{T}, {N}], got {tuple(x_out.shape)}")
    need = msa_project_workspace_size(T, K, N // 128) if N % 128 == 0 and K % 64 == 0 and N > 0 else 0
    wp, wb = _workspace(workspace, need)
    _same_device(h, w, x_out, workspace)
    st = lib().msa_project(_ptr(h), h.stride(0), T, K, _ptr(w), w.stride(0), N, _ptr(x_out), x_out.stride(0), wp, wb,
                           _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_project")


def msa_project_produce(h, w, rope_cos, rope_sin, slots, q_norm_weight, k_norm_weight, iq_norm_weight,
                        ik_norm_weight, q_out, iq_out, k_cache, v_cache, ik_cache=None, *, workspace=None,
                        k_scale=None, v_scale=None, ik_scale=None, num_pages: Optional[int] = None,
                        rms_eps: float = 1e-6, stream=None) -> None:
    """The projection with the producer as its epilogue.  h [T, K] bf16; w [W, K] bf16 (packed rows Q,
    K, V, index-Q, index-K); rope_cos / rope_sin float32 [T, 64] (msa_rope_table); slots int64 [T]
    (msa_slots); the rest as in msa_produce.  Head counts come from q_out, iq_out and the caches."""
    T, K, N = _gemm_operands(h, w)
    hkv, hik, page_size, pages = _caches(k_cache, v_cache, ik_cache, num_pages, k_scale, v_scale, ik_scale)
    _tensor("q_out", q_out, dim=3)
    _tensor("iq_out", iq_out, dim=3)
    hq, hiq = q_out.shape[1], iq_out.shape[1]
    _rows_out("q_out", q_out, T, hq)
    _rows_out("iq_out", iq_out, T, hiq)
    heads = hq + 2 * hkv + hiq + hik
    _need(N == heads * 128, f"w has {N} rows, the heads need {heads * 128}")
    for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
        _tensor(name, t, contiguous=True)
        _float(name, t, 32)
        _need(t.numel() >= T * 64, f"{name} holds {t.numel()} elements, needs {T * 64}")
    _int("slots", slots, 64, T)
    _weights((q_norm_weight, k_norm_weight, iq_norm_weight, ik_norm_weight), (hq, hkv, hiq, hik))
    need = msa_project_workspace_size(T, K, heads) if K % 64 == 0 else 0
    wp, wb = _workspace(workspace, need)
    _same_device(h, w, rope_cos, rope_sin, slots, q_norm_weight, k_norm_weight, iq_norm_weight, ik_norm_weight,
                 q_out, iq_out, k_cache, v_cache, ik_cache, workspace)
    kv, vv, iv = cache_view(k_cache, k_scale), cache_view(v_cache, v_scale), cache_view(ik_cache, ik_scale)
    st = lib().msa_project_produce(
        _ptr(h), h.stride(0), T, K, _ptr(w), w.stride(0), 128, hq, hkv, hiq, hik,
        _ptr(rope_cos), _ptr(rope_sin), _ptr(slots), page_size, pages,
        _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(iq_norm_weight), _ptr(ik_norm_weight), float(rms_eps),
        _ptr(q_out), _ptr(iq_out), _ref(kv), _ref(vv), _ref(iv), wp, wb, _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_project_produce")


def msa_project_produce_noalloc(h, w, rope_cos, rope_sin, slots, q_norm_weight, k_norm_weight, iq_norm_weight,
                                ik_norm_weight, q_out, iq_out, k_cache, v_cache, ik_cache=None, *, k_scale=None,
                                v_scale=None, ik_scale=None, num_pages: Optional[int] = None, rms_eps: float = 1e-6,
                                stream=None) -> None:
    """msa_project_produce with the library's own 32 MiB per-GPU scratch instead of a workspace: allocates
    nothing.  Calls on one GPU share the scratch, so calls that overlap in time on one GPU race.  A call
    that needs more scratch than that raises MsaError (MSA_ERR_WORKSPACE)."""
    T, K, N = _gemm_operands(h, w)
    hkv, hik, page_size, pages = _caches(k_cache, v_cache, ik_cache, num_pages, k_scale, v_scale, ik_scale)
    _tensor("q_out", q_out, dim=3)
    _tensor("iq_out", iq_out, dim=3)
    hq, hiq = q_out.shape[1], iq_out.shape[1]
    _rows_out("q_out", q_out, T, hq)
    _rows_out("iq_out", iq_out, T, hiq)
    heads = hq + 2 * hkv + hiq + hik
    _need(N == heads * 128, f"w has {N} rows, the heads need {heads * 128}")
    for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
        _tensor(name, t, contiguous=True)
        _float(name, t, 32)
        _need(t.numel() >= T * 64, f"{name} holds {t.numel()} elements, needs {T * 64}")
    _int("slots", slots, 64, T)
    _weights((q_norm_weight, k_norm_weight, iq_norm_weight, ik_norm_weight), (hq, hkv, hiq, hik))
    _same_device(h, w, rope_cos, rope_sin, slots, q_norm_weight, k_norm_weight, iq_norm_weight, ik_norm_weight,
                 q_out, iq_out, k_cache, v_cache, ik_cache)
    kv, vv, iv = cache_view(k_cache, k_scale), cache_view(v_cache, v_scale), cache_view(ik_cache, ik_scale)
    st = lib().msa_project_produce_noalloc(
        _ptr(h), h.stride(0), T, K, _ptr(w), w.stride(0), 128, hq, hkv, hiq, hik,
        _ptr(rope_cos), _ptr(rope_sin), _ptr(slots), page_size, pages,
        _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(iq_norm_weight), _ptr(ik_norm_weight), float(rms_eps),
        _ptr(q_out), _ptr(iq_out), _ref(kv), _ref(vv), _ref(iv), _stream(stream))
    if st != 0:
        raise MsaError(st, "msa_project_produce_noalloc")


def msa_check_device_pointers(ptrs, nbytes=None):
    """The library's residency check on raw addresses (ints; None passes), each with an extent in bytes
    (default 1).  Returns (status, index of the first failing pointer or -1).  Launches nothing."""
    n = len(ptrs)
    arr = (ctypes.c_void_p * max(n, 1))(*[p for p in ptrs])
    sizes = None
    if nbytes is not None:
        sizes = (ctypes.c_uint64 * max(n, 1))(*[int(b) for b in nbytes])
    bad = ctypes.c_int32(-2)
    st = lib().msa_check_device_pointers(arr, sizes, n, ctypes.byref(bad))
    return st, bad.value
