"""Shared test helpers: code decoders, an fp64 torch/transformers reference of the producer's
mathematics (for tolerance-level pins of the oracle), golden-file readers, and device-side
workload staging for the GPU tests.  None of this is used by the product path."""
from __future__ import annotations

import math
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3 code -> float64 value (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 15
    M = c & 7
    mag = np.where(E == 0, M * 2.0 ** -9, (8 + M) * np.exp2(E.astype(np.float64) - 10))
    mag = np.where((E == 15) & (M == 7), np.nan, mag)
    return sign * mag


def read_points(name: str):
    rows = []
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            v, code = line.split()
            val = float(v) if v.lstrip("-") in ("inf", "nan") else float.fromhex(v)
            if v == "-nan":
                val = -float("nan")
            rows.append((val, int(code, 16)))
    return rows


def torch_reference(wl, head_dim=128):
    """fp64 reference of the producer's per-token values, from library routines:
    torch.nn.functional.rms_norm (per-head RMSNorm with a [D] weight) and transformers'
    apply_rotary_pos_emb (neox rotate-half RoPE), with cos/sin of pos * theta^(-2i/D) in fp64.

    Returns dict stream -> float64 [T, H, D] of the values each output holds before its final cast
    (V is the raw input)."""
    import torch.nn.functional as F
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb

    D = head_dim
    T = wl.T
    counts = [wl.hq, wl.hkv, wl.hkv, wl.hiq, wl.hik]
    names = ["q", "k", "v", "iq", "ik"]
    x = torch.from_numpy(bf16_bits_to_f32(wl.x[:, : wl.W]).astype(np.float64))
    pos = torch.from_numpy(wl.positions.astype(np.float64))
    i = torch.arange(0, D, 2, dtype=torch.float64)
    freq = wl.theta ** (-i / D)
    ang = pos[:, None] * freq[None, :]
    cos = torch.cat([ang.cos(), ang.cos()], dim=-1)[:, None, :]   # [T, 1, D]
    sin = torch.cat([ang.sin(), ang.sin()], dim=-1)[:, None, :]
    out = {}
    col = 0
    wmap = {"q": 0, "k": 1, "iq": 2, "ik": 3}
    for n, h in zip(names, counts):
        a = x[:, col: col + h * D].reshape(T, h, D)
        col += h * D
        if n == "v" or h == 0:
            out[n] = a.numpy()
            continue
        w = torch.from_numpy(bf16_bits_to_f32(wl.weights[wmap[n]]).astype(np.float64))
        y = F.rms_norm(a, (D,), weight=w, eps=wl.eps)
        # apply_rotary_pos_emb expects [batch, heads, seq, D] and cos [batch, seq, D]
        yq = y.reshape(T, h, 1, D)
        o, _ = apply_rotary_pos_emb(yq, yq, cos, sin, unsqueeze_dim=1)
        out[n] = o.reshape(T, h, D).numpy()
    return out


def e4m3_half_spacing(z: np.ndarray) -> np.ndarray:
    """Half the E4M3 grid spacing at magnitude |z| (fp64)."""
    a = np.abs(z)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 0.5 * np.exp2(e - 3)


def bf16_half_spacing(z: np.ndarray) -> np.ndarray:
    a = np.abs(z)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 0.5 * np.exp2(e - 7)


def ulp32(z: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(z, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 23)


def cache_fill(spec, sentinel=0x7F):
    """Host cache storage filled with the sentinel byte (uint8 for fp8, uint16 for bf16)."""
    if spec.dtype == 0:
        return np.full(spec.storage_shape, sentinel, np.uint8)
    return np.full(spec.storage_shape, sentinel * 0x0101, np.uint16)


def oracle_caches(wl):
    """Run the oracle's cache form on sentinel-filled host caches; returns (result, storages)."""
    import oracle
    st = [cache_fill(c) for c in wl.caches]
    caches = [dict(storage=s, strides=c.strides, dtype=c.dtype, scale=c.scale) for s, c in zip(st, wl.caches)]
    r = oracle.produce(wl.x, wl.x_stride, wl.T, wl.head_dim, wl.hq, wl.hkv, wl.hiq, wl.hik, wl.positions,
                       wl.seq_idx, wl.page_table, wl.max_pages, wl.num_seqs, wl.max_pages, wl.page_size,
                       wl.num_pages, *wl.weights, wl.eps, wl.theta, caches)
    return r, st


def oracle_rows(wl, num_threads=1):
    import oracle
    return oracle.produce_rows(wl.x, wl.x_stride, wl.T, wl.head_dim, wl.hq, wl.hkv, wl.hiq, wl.hik,
                               wl.positions, wl.seq_idx, wl.page_table, wl.max_pages, wl.num_seqs,
                               wl.max_pages, wl.page_size, wl.num_pages, *wl.weights, wl.eps, wl.theta,
                               dtypes=[c.dtype for c in wl.caches], scales=[c.scale for c in wl.caches],
                               num_threads=num_threads)


def math_cos32(x: float) -> float:
    return float(np.float32(math.cos(x)))
