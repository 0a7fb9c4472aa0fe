"""The comparison the GPU parity tests apply: a device result of the producer (fused, unfused or fused
into the projection) against the CPU oracle, element by element.

Bar: slots and every cache byte bit-exact; Q and index-Q within one bf16 ulp (|gpu - oracle| <=
2^-7 |oracle|, NaN where the oracle has NaN); every cache element outside the set the oracle wrote
(untouched slots, padded heads, other pages) still holds the sentinel, compared exactly.

Which NaN (sign, payload) an IEEE-754 operation returns is not fixed by the standard (x86 and the GPU
differ), so where the oracle wrote a NaN code the device code only has to be a NaN too.  That
leniency applies inside the written set only: the fp8 sentinel 0x7F is itself an E4M3 NaN, so
outside the written set a NaN-for-NaN comparison would accept a stray 0xFF.

The pure-numpy parts (written_mask, storage_mismatches, code_diff) need no GPU; check() stages
device tensors back to the host.
"""
from __future__ import annotations

import os
import sys

import numpy as np

from paged_kv_cache_msa_amd import workloads as W
from tests import helpers as H

THREADS = min(16, os.cpu_count() or 1)


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def sentinel_code(dtype: int) -> int:
    return W.SENTINEL_BYTE if dtype == W.FP8_E4M3 else W.SENTINEL_BYTE * 0x0101


def is_nan_code(c, dtype):
    c = np.asarray(c)
    if dtype == W.FP8_E4M3:
        return (c & 0x7F) == 0x7F
    return (c & 0x7FFF) > 0x7F80


def code_diff(gpu, ref, dtype):
    """Indices where two arrays of cache codes written by the producer disagree: identical codes,
    except that where the oracle's code is a NaN the device code only has to be a NaN."""
    nan_r = is_nan_code(ref, dtype)
    ok = np.where(nan_r, is_nan_code(gpu, dtype), gpu == ref)
    return np.flatnonzero(~ok)


def written_elements(spec, slots, page_size, head_dim=W.HEAD_DIM):
    """Flat storage indices of every cache element a producer call with these slots writes:
    (page, head, offset, d) at page * sp + head * sh + offset * st + d for every slot >= 0."""
    s = np.asarray(slots, np.int64)
    s = s[s >= 0]
    if spec.heads == 0 or s.size == 0:
        return np.zeros(0, np.int64)
    sp, sh, st = (int(v) for v in spec.strides)
    base = (s // page_size) * sp + (s % page_size) * st
    idx = base[:, None, None] + (np.arange(spec.heads, dtype=np.int64) * sh)[None, :, None] \
        + np.arange(head_dim, dtype=np.int64)[None, None, :]
    return idx.reshape(-1)


def written_mask(spec, slots, page_size, head_dim=W.HEAD_DIM):
    mask = np.zeros(spec.storage_elems, bool)
    mask[written_elements(spec, slots, page_size, head_dim)] = True
    return mask


def storage_mismatches(gpu, ref, mask, dtype):
    """Indices where a device cache storage disagrees with the oracle's: inside the written set
    (mask) by code_diff; outside it every element must equal the sentinel exactly."""
    gpu = np.asarray(gpu).reshape(-1)
    ref = np.asarray(ref).reshape(-1)
    inside = np.flatnonzero(mask)
    bad_in = inside[code_diff(gpu[inside], ref[inside], dtype)]
    bad_out = np.flatnonzero(~mask & (gpu != sentinel_code(dtype)))
    return np.union1d(bad_in, bad_out)


def check_q(name, gpu_bits, ref_bits):
    g = H.bf16_bits_to_f32(gpu_bits).astype(np.float64)
    r = H.bf16_bits_to_f32(ref_bits).astype(np.float64)
    nan_g, nan_r = np.isnan(g), np.isnan(r)
    assert np.array_equal(nan_g, nan_r), f"{name}: NaN positions differ"
    fin = ~nan_r
    with np.errstate(invalid="ignore"):
        ok = (g[fin] == r[fin]) | (np.abs(g[fin] - r[fin]) <= 2.0 ** -7 * np.abs(r[fin]))
    bad = np.flatnonzero(~ok)
    assert bad.size == 0, f"{name}: {bad.size} elements beyond 1 bf16 ulp, first {g[fin][bad[:4]]} vs {r[fin][bad[:4]]}"
    n_inexact = int(np.count_nonzero(gpu_bits != ref_bits))
    say(f"  {name}: within 1 bf16 ulp; bit-identical elements {gpu_bits.size - n_inexact}/{gpu_bits.size}")


def _codes(t, dtype):
    a = t.cpu().numpy()
    return a.view(np.uint8) if dtype == W.FP8_E4M3 else a.view(np.uint16)


def check(wl, d, full=None, ref=None):
    """Compare a device result d (workloads.DeviceWorkload) with the oracle on workload wl.

    full=True compares whole cache storages with the oracle's cache form (written set by code,
    the rest against the sentinel); otherwise (large pools) the rows at the oracle's slots are
    gathered on the device and compared, and every other element of each storage must hold the
    sentinel: the device count of non-sentinel elements must equal that count within the gathered
    rows.  `ref`: the oracle's per-token result if already computed."""
    import torch

    if full is None:
        full = all(c.storage_elems <= (1 << 26) for c in wl.caches)
    ref = H.oracle_rows(wl, num_threads=THREADS) if ref is None else ref
    slots = d.slots.cpu().numpy()
    np.testing.assert_array_equal(slots, ref["slots"])
    check_q("q", d.q_out.cpu().numpy().view(np.uint16), ref["q"])
    check_q("iq", d.iq_out.cpu().numpy().view(np.uint16), ref["iq"])
    valid = np.flatnonzero(ref["slots"] >= 0)
    if full:
        _, st = H.oracle_caches(wl)
        for name, spec, s_ref, s_gpu in zip(("k", "v", "ik"), wl.caches, st, d.storages):
            if spec.heads == 0:
                continue
            mask = written_mask(spec, ref["slots"], wl.page_size, wl.head_dim)
            r = s_ref.reshape(-1)
            # the oracle itself wrote nothing outside the written set
            assert np.all(r[~mask] == sentinel_code(spec.dtype)), f"{name}: oracle wrote outside its slots"
            bad = storage_mismatches(_codes(s_gpu, spec.dtype), r, mask, spec.dtype)
            assert bad.size == 0, f"{name} cache: {bad.size} elements differ, first at {bad[:4]}"
        say(f"  caches: whole storages identical, untouched elements hold the sentinel ({len(valid)} tokens written)")
        return
    pg = torch.from_numpy(ref["slots"][valid] // wl.page_size).cuda()
    off = torch.from_numpy(ref["slots"][valid] % wl.page_size).cuda()
    for name, spec, view, store in zip(("k", "v", "ik"), wl.caches, d.caches, d.storages):
        if spec.heads == 0:
            continue
        rows = _codes(view[pg, :, off, :], spec.dtype)          # [n_valid, H, D]
        exp = ref[name][valid]
        diff = code_diff(rows.reshape(-1), exp.reshape(-1), spec.dtype)
        assert diff.size == 0, f"{name} cache rows: {len(diff)} elements differ, first {diff[:4]}"
        sent = sentinel_code(spec.dtype)
        changed = int((store != sent).sum().item())
        in_rows = int(np.count_nonzero(rows != sent))
        assert changed == in_rows, f"{name}: {changed - in_rows} elements changed outside the written rows"
    say(f"  caches: gathered rows identical, every other element holds the sentinel ({len(valid)} tokens written)")
