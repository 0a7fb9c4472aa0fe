"""Python access to the plain CPU oracle of the MSA fused producer (msa_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may use this package; the product path never does.

The oracle follows the AFTER figure and change list of the page "Fuse MiniMax-M3
QKV and index projection" (the packed projection of the hidden states, per-head
Q/K RMSNorm + neox RoPE on Q, K, index-Q and index-K, compact Q/index-Q, paged
HND cache writes with invalid slots skipped),
and the slot rule page = slot / page_size, offset = slot % page_size of "Fuse
MiniMax-M3 MSA per-layer KV-cache writes into one kernel" ("The problem").

Parity pins: every function here is pinned by tests/test_oracle_*.py against
brute force, closed forms, invariants or library routines (see the docstrings
there).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "libmsa_oracle.so")

FP8_E4M3 = 0
BF16 = 1

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile msa_oracle.c with gcc into libmsa_oracle.so next to it."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        p, i64, i32, f32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_double
        L.msa_oracle_bf16.argtypes = [f32]
        L.msa_oracle_bf16.restype = ctypes.c_uint16
        L.msa_oracle_e4m3.argtypes = [f32]
        L.msa_oracle_e4m3.restype = ctypes.c_uint8
        L.msa_oracle_encode_bf16.argtypes = [p, i64, p]
        L.msa_oracle_encode_bf16.restype = None
        L.msa_oracle_encode_e4m3.argtypes = [p, i64, p]
        L.msa_oracle_encode_e4m3.restype = None
        L.msa_oracle_rope_table.argtypes = [p, i64, f64, i32, p, p]
        L.msa_oracle_rope_table.restype = None
        L.msa_oracle_rms_scale.argtypes = [p, i64, i32, f32, p]
        L.msa_oracle_rms_scale.restype = None
        L.msa_oracle_slots.argtypes = [p, p, i64, p, i64, i32, i32, i32, i64, p]
        L.msa_oracle_slots.restype = None
        L.msa_oracle_produce_rows.argtypes = (
            [p, i64, i64, i32, i32, i32, i32, i32, p, p, p, i64, i32, i32, i32, i64, p, p, p, p, f32, f64]
            + [i32, i32, i32, f32, f32, f32, p, p, p, p, p, p, i32])
        L.msa_oracle_produce_rows.restype = ctypes.c_int
        L.msa_oracle_produce.argtypes = (
            [p, i64, i64, i32, i32, i32, i32, i32, p, p, p, i64, i32, i32, i32, i64, p, p, p, p, f32, f64]
            + [p, i64, i64, i64, i32, f32] * 3 + [p, p, p, i32])
        L.msa_oracle_produce.restype = ctypes.c_int
        L.msa_oracle_index_scores.argtypes = [p, i64, i32, i32, p, p, p, i64, i32, i32, i32, i64, p, i64, i64, i64,
                                              i32, i32, f32, i32, i32, p]
        L.msa_oracle_index_scores.restype = ctypes.c_int
        L.msa_oracle_index_topk.argtypes = [p, i32, i64, i32, i32, p, p]
        L.msa_oracle_index_topk.restype = ctypes.c_int
        L.msa_oracle_bf16_of_f64.argtypes = [f64]
        L.msa_oracle_bf16_of_f64.restype = ctypes.c_uint16
        L.msa_oracle_project.argtypes = [p, i64, i64, i64, p, i64, i64, p, i64, p, p, i32]
        L.msa_oracle_project.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def encode_bf16(v) -> np.ndarray:
    v = _c(v, np.float32).reshape(-1)
    out = np.empty(v.shape, np.uint16)
    lib().msa_oracle_encode_bf16(_ptr(v), v.size, _ptr(out))
    return out


def encode_e4m3(v) -> np.ndarray:
    v = _c(v, np.float32).reshape(-1)
    out = np.empty(v.shape, np.uint8)
    lib().msa_oracle_encode_e4m3(_ptr(v), v.size, _ptr(out))
    return out


def rope_table(positions, theta: float, head_dim: int):
    """cos, sin as float32 [n, head_dim // 2]."""
    pos = _c(positions, np.int32).reshape(-1)
    c = np.empty((pos.size, head_dim // 2), np.float32)
    s = np.empty_like(c)
    lib().msa_oracle_rope_table(_ptr(pos), pos.size, float(theta), head_dim, _ptr(c), _ptr(s))
    return c, s


def rms_scale(ss, head_dim: int, eps: float) -> np.ndarray:
    ss = _c(ss, np.float64).reshape(-1)
    out = np.empty(ss.shape, np.float32)
    lib().msa_oracle_rms_scale(_ptr(ss), ss.size, head_dim, float(eps), _ptr(out))
    return out


def slots(positions, seq_idx, page_table, num_seqs, max_pages, page_size, num_pages, pt_stride=None):
    pos = _c(positions, np.int32).reshape(-1)
    seq = _c(seq_idx, np.int32).reshape(-1)
    pt = _c(page_table, np.int32)
    stride = pt.shape[-1] if pt_stride is None else pt_stride
    out = np.empty(pos.shape, np.int64)
    lib().msa_oracle_slots(_ptr(pos), _ptr(seq), pos.size, _ptr(pt), stride, num_seqs, max_pages,
                           page_size, num_pages, _ptr(out))
    return out


class OracleError(RuntimeError):
    pass


def _esize(dt):
    return 1 if dt == FP8_E4M3 else 2


def _npdt(dt):
    return np.uint8 if dt == FP8_E4M3 else np.uint16


def produce_rows(x, x_stride, T, head_dim, hq, hkv, hiq, hik, positions, seq_idx, page_table, pt_stride,
                 num_seqs, max_pages, page_size, num_pages, w_q, w_k, w_iq, w_ik, eps, theta,
                 dtypes=(FP8_E4M3, FP8_E4M3, FP8_E4M3), scales=(1.0, 1.0, 1.0), num_threads=1):
    """Dense per-token outputs.

    x is a uint16 (bf16 bits) array whose flat buffer holds row t at element t * x_stride.
    Returns dict(q, iq, k, v, ik, slots); k/v/ik are cache codes [T, H, D] (uint8 fp8 / uint16 bf16).
    """
    x = np.ascontiguousarray(x, dtype=np.uint16)
    need = (T - 1) * x_stride + (hq + 2 * hkv + hiq + hik) * head_dim if T > 0 else 0
    if x.size < need:
        raise OracleError("x buffer too small")
    pos = _c(positions, np.int32)
    seq = _c(seq_idx, np.int32)
    pt = _c(page_table, np.int32)
    ws = [None if w is None else _c(w, np.uint16) for w in (w_q, w_k, w_iq, w_ik)]
    q = np.empty((T, hq, head_dim), np.uint16)
    iq = np.empty((T, hiq, head_dim), np.uint16)
    rows = [np.empty((T, h, head_dim), _npdt(dt)) for h, dt in zip((hkv, hkv, hik), dtypes)]
    sl = np.empty(T, np.int64)
    rc = lib().msa_oracle_produce_rows(
        _ptr(x), x_stride, T, head_dim, hq, hkv, hiq, hik, _ptr(pos), _ptr(seq), _ptr(pt), pt_stride,
        num_seqs, max_pages, page_size, num_pages, *[_ptr(w) for w in ws], float(eps), float(theta),
        int(dtypes[0]), int(dtypes[1]), int(dtypes[2]), float(scales[0]), float(scales[1]), float(scales[2]),
        _ptr(q), _ptr(iq), _ptr(rows[0]), _ptr(rows[1]), _ptr(rows[2]), _ptr(sl), int(num_threads))
    if rc != 0:
        raise OracleError(f"msa_oracle_produce_rows returned {rc}")
    return dict(q=q, iq=iq, k=rows[0], v=rows[1], ik=rows[2], slots=sl)


def produce(x, x_stride, T, head_dim, hq, hkv, hiq, hik, positions, seq_idx, page_table, pt_stride,
            num_seqs, max_pages, page_size, num_pages, w_q, w_k, w_iq, w_ik, eps, theta, caches,
            num_threads=1):
    """Cache form.  caches: three dicts (k, v, ik) with keys
    storage (np array, modified in place), strides (sp, sh, st in elements), dtype, scale.
    Returns dict(q, iq, slots)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    pos = _c(positions, np.int32)
    seq = _c(seq_idx, np.int32)
    pt = _c(page_table, np.int32)
    ws = [None if w is None else _c(w, np.uint16) for w in (w_q, w_k, w_iq, w_ik)]
    q = np.empty((T, hq, head_dim), np.uint16)
    iq = np.empty((T, hiq, head_dim), np.uint16)
    sl = np.empty(T, np.int64)
    cargs = []
    for c in caches:
        st = c["storage"]
        if not st.flags.c_contiguous:
            raise OracleError("cache storage must be a contiguous array")
        cargs += [_ptr(st), *[int(v) for v in c["strides"]], int(c["dtype"]), float(c["scale"])]
    rc = lib().msa_oracle_produce(
        _ptr(x), x_stride, T, head_dim, hq, hkv, hiq, hik, _ptr(pos), _ptr(seq), _ptr(pt), pt_stride,
        num_seqs, max_pages, page_size, num_pages, *[_ptr(w) for w in ws], float(eps), float(theta),
        *cargs, _ptr(q), _ptr(iq), _ptr(sl), int(num_threads))
    if rc != 0:
        raise OracleError(f"msa_oracle_produce returned {rc}")
    return dict(q=q, iq=iq, slots=sl)


def index_scores(iq, positions, seq_idx, page_table, pt_stride, num_seqs, max_pages, page_size, num_pages,
                 ik_storage, ik_strides, hik, ik_dtype, ik_scale, block_tokens, max_blocks):
    """Block scores [hiq, T, max_blocks] (float64) of the indexer reading (see msa_oracle.c).
    iq: uint16 bf16 bits [T, hiq, D]; ik_storage: the index-K cache storage (uint8 fp8 codes or uint16
    bf16 bits), element (page, head, token, d) at page*sp + head*sh + token*st + d."""
    iq = np.ascontiguousarray(iq, dtype=np.uint16)
    T, hiq, D = iq.shape
    pos = _c(positions, np.int32)
    seq = _c(seq_idx, np.int32)
    pt = _c(page_table, np.int32)
    st = np.ascontiguousarray(ik_storage)
    out = np.empty((hiq, T, max_blocks), np.float64)
    sp, sh, stt = (int(v) for v in ik_strides)
    rc = lib().msa_oracle_index_scores(_ptr(iq), T, hiq, D, _ptr(pos), _ptr(seq), _ptr(pt), pt_stride, num_seqs,
                                       max_pages, page_size, num_pages, _ptr(st), sp, sh, stt, hik, int(ik_dtype),
                                       float(ik_scale), block_tokens, max_blocks, _ptr(out))
    if rc != 0:
        raise OracleError(f"msa_oracle_index_scores returned {rc}")
    return out


def index_topk(block_scores, top_k):
    """ids [hiq, T, top_k] int32 and counts [hiq, T] of the top-k blocks (descending score, ties to the
    lower block index, -1 padding)."""
    bs = np.ascontiguousarray(block_scores, dtype=np.float64)
    hiq, T, nb = bs.shape
    ids = np.empty((hiq, T, top_k), np.int32)
    counts = np.empty((hiq, T), np.int32)
    rc = lib().msa_oracle_index_topk(_ptr(bs), hiq, T, nb, top_k, _ptr(ids), _ptr(counts))
    if rc != 0:
        raise OracleError(f"msa_oracle_index_topk returned {rc}")
    return ids, counts


def bf16_of_f64(v: float) -> int:
    """One binary64 value rounded once to bf16 (bits)."""
    return int(lib().msa_oracle_bf16_of_f64(float(v)))


def project(h, w, num_threads: int = 1, want_sums: bool = False):
    """x = bf16(h @ w.T) with a binary64 ascending-k sum per element (msa_oracle_project).
    h: uint16 bf16 bits [T, K]; w: uint16 bf16 bits [N, K].  Returns x (uint16 [T, N]) or, with
    want_sums, (x, sum, abs_sum) where sum is the binary64 sum and abs_sum = sum_k |h w|."""
    h = _c(h, np.uint16)
    w = _c(w, np.uint16)
    T, K = h.shape
    N, K2 = w.shape
    if K2 != K:
        raise OracleError("h and w disagree on K")
    x = np.empty((T, N), np.uint16)
    sm = np.empty((T, N), np.float64) if want_sums else None
    ab = np.empty((T, N), np.float64) if want_sums else None
    rc = lib().msa_oracle_project(_ptr(h), K, T, K, _ptr(w), K, N, _ptr(x), N, _ptr(sm), _ptr(ab),
                                  int(num_threads))
    if rc != 0:
        raise OracleError(f"msa_oracle_project returned {rc}")
    return (x, sm, ab) if want_sums else x
