"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what fixes the expected value: the OCP FP8 / bfloat16 format tables
(tests/golden), brute-force nearest-code search, closed forms of cos/sin and RMSNorm,
invariants of the method (RoPE identity at position 0, pair-norm preservation, RMS of the
normalised head equal to the weight, slot = page_table[seq][pos // P] * P + pos % P, untouched
slots keep their sentinel), and library routines (torch's float8/bfloat16 casts,
torch.nn.functional.rms_norm, transformers' apply_rotary_pos_emb).
"""
import math
import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_msa_amd import workloads as W
from tests import helpers as H


# ----------------------------------------------------------------------------- encoders

def test_e4m3_format_table_points(oracle_lib):
    """OCP OFP8 E4M3 table points and tie/saturation consequences (tests/golden/e4m3_ocp_points.txt)."""
    for v, code in H.read_points("e4m3_ocp_points.txt"):
        got = oracle.encode_e4m3(np.array([v], np.float32))[0]
        assert got == code, (v, hex(got), hex(code))


def test_bf16_format_points(oracle_lib):
    for v, code in H.read_points("bf16_points.txt"):
        got = oracle.encode_bf16(np.array([v], np.float32))[0]
        assert got == code, (v, hex(got), hex(code))


@pytest.mark.slow
def test_encoders_exhaustive_bruteforce(oracle_lib):
    """All 2^32 binary32 inputs: oracle encoders == brute-force nearest-code search."""
    src = os.path.join(H.HERE, "encoder_sweep.c")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "sweep")
        subprocess.check_call(["gcc", "-O2", "-fopenmp", src, "-o", exe, "-lm", "-ldl"])
        r = subprocess.run([exe, oracle.build()], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "e4m3 mismatches: 0" in r.stdout and "bf16 mismatches: 0" in r.stdout


def _all_bf16_values():
    u = np.arange(1 << 16, dtype=np.uint32) << 16
    return u.view(np.float32)


def test_e4m3_matches_torch_cast_below_overflow(oracle_lib):
    """torch's float8_e4m3fn cast (round-to-nearest-even) agrees wherever no saturation is involved."""
    rng = np.random.default_rng(5)
    v = np.concatenate([_all_bf16_values(),
                        rng.standard_normal(2_000_000).astype(np.float32) * np.float32(40),
                        (rng.random(2_000_000).astype(np.float32) * np.float32(2 ** -5))])
    v = v[np.isfinite(v) & (np.abs(v) < 448)]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.encode_e4m3(v), ref)


def test_e4m3_nan_keeps_sign(oracle_lib):
    nan = np.array([np.nan, -np.nan], np.float32)
    nan[1] = -np.abs(nan[1])
    ref = torch.from_numpy(nan).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.encode_e4m3(nan), ref)      # 0x7f, 0xff


def test_bf16_matches_torch_cast(oracle_lib):
    rng = np.random.default_rng(6)
    u = rng.integers(0, 1 << 32, 4_000_000, dtype=np.uint64).astype(np.uint32)
    v = u.view(np.float32)
    v = v[~np.isnan(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.encode_bf16(v), ref)


# ----------------------------------------------------------------------------- RoPE coefficients

def test_rope_identity_at_position_zero(oracle_lib):
    """Invariant: at position 0 every angle is 0, so cos = 1 and sin = 0 exactly."""
    c, s = oracle.rope_table([0], 1e4, 128)
    assert np.all(c == 1.0) and np.all(s == 0.0)


def test_rope_frequencies_closed_form(oracle_lib):
    """f_i = theta^(-2i/D): at theta = 1e4, D = 128, f_0 = 1, f_16 = 0.1, f_32 = 0.01, f_48 = 0.001.
    cos/sin of pos * f_i from numpy agree within 1 ulp of binary32 (a wrong exponent would not)."""
    pos = np.array([1, 2, 3, 77, 1000, 8191, 9199, 32767, 65535], np.int32)
    c, s = oracle.rope_table(pos, 1e4, 128)
    for i, f in [(0, 1.0), (16, 0.1), (32, 0.01), (48, 0.001)]:
        ang = pos.astype(np.float64) * f
        for got, ref in [(c[:, i], np.cos(ang)), (s[:, i], np.sin(ang))]:
            assert np.all(np.abs(got.astype(np.float64) - ref) <= H.ulp32(ref) + 1e-12), (i, got, ref)


def test_rope_coefficients_unit_circle(oracle_lib):
    rng = np.random.default_rng(1)
    pos = rng.integers(0, 1 << 20, 500).astype(np.int32)
    c, s = oracle.rope_table(pos, 1e4, 128)
    r = c.astype(np.float64) ** 2 + s.astype(np.float64) ** 2
    assert np.max(np.abs(r - 1)) < 2.5e-7


def test_rope_theta_and_dim_enter(oracle_lib):
    """Other theta / head_dim: f_1 = theta^(-2/D)."""
    for theta, D in [(1e6, 128), (5e5, 64), (10.0, 16)]:
        c, s = oracle.rope_table([5], theta, D)
        ref = 5 * theta ** (-2.0 / D)
        assert abs(float(c[0, 1]) - math.cos(ref)) <= 2 * 2 ** -24
        assert abs(float(s[0, 1]) - math.sin(ref)) <= 2 * 2 ** -24


# ----------------------------------------------------------------------------- RMSNorm scale

def test_rms_scale_closed_form(oracle_lib):
    """ss = D * 4^k with eps = 0 gives r = 2^-k exactly; ss = 0 gives 1/sqrt(eps)."""
    k = np.arange(-20, 21)
    ss = 128.0 * 4.0 ** k
    r = oracle.rms_scale(ss, 128, 0.0)
    np.testing.assert_array_equal(r, (2.0 ** -k).astype(np.float32))
    r0 = oracle.rms_scale([0.0], 128, 1e-6)[0]
    assert abs(r0 - 1 / math.sqrt(float(np.float32(1e-6)))) <= 1e-7 * r0
    # eps enters as mean + eps
    r1 = oracle.rms_scale([128.0], 128, 1.0)[0]
    assert r1 == np.float32(1 / math.sqrt(2.0))


# ----------------------------------------------------------------------------- slots

def _slot_bruteforce(wl):
    out = []
    for t in range(wl.T):
        p, s = int(wl.positions[t]), int(wl.seq_idx[t])
        if s < 0 or s >= wl.num_seqs or p < 0 or p // wl.page_size >= wl.max_pages:
            out.append(-1)
            continue
        pg = int(wl.page_table[s, p // wl.page_size])
        out.append(pg * wl.page_size + p % wl.page_size if 0 <= pg < wl.num_pages else -1)
    return np.array(out, np.int64)


@pytest.mark.parametrize("make", [W.tiny_decode, W.tiny_decode_no_index_k, lambda: W.ragged(37, seed=3)])
def test_slots_closed_form(oracle_lib, make):
    """Invariant: slot = page_table[seq][pos // P] * P + pos % P for every valid token, -1 otherwise."""
    wl = make()
    got = oracle.slots(wl.positions, wl.seq_idx, wl.page_table, wl.num_seqs, wl.max_pages, wl.page_size,
                       wl.num_pages)
    np.testing.assert_array_equal(got, _slot_bruteforce(wl))


def test_slots_invalid_cases(oracle_lib):
    pt = np.array([[3, 1], [0, 2]], np.int32)
    pos = np.array([0, 65, -1, 130, 5, 70, 1], np.int32)
    seq = np.array([0, 0, 0, 0, -1, 1, 2], np.int32)
    got = oracle.slots(pos, seq, pt, 2, 2, 64, 3)   # page 3 is outside a 3-page pool
    np.testing.assert_array_equal(got, [-1, 1 * 64 + 1, -1, -1, -1, 2 * 64 + 6, -1])


def test_slots_exhaustive_small_table(oracle_lib):
    """Brute force: every (seq, pos) pair over a small table, including position 0, page boundaries,
    the last logical page, negative positions/sequences and entries outside the pool."""
    rng = np.random.default_rng(3)
    S, max_pages, P, num_pages = 3, 4, 4, 10
    pt = rng.integers(-2, num_pages + 3, (S, max_pages)).astype(np.int32)
    pairs = [(s, p) for s in range(-2, S + 2) for p in range(-3, P * max_pages + 4)]
    seq = np.array([s for s, _ in pairs], np.int32)
    pos = np.array([p for _, p in pairs], np.int32)
    got = oracle.slots(pos, seq, pt, S, max_pages, P, num_pages)
    for (s, p), g in zip(pairs, got):
        if 0 <= s < S and 0 <= p < P * max_pages and 0 <= pt[s, p // P] < num_pages:
            assert g == pt[s, p // P] * P + p % P, (s, p, g)
        else:
            assert g == -1, (s, p, g)


def test_slot_set_bruteforce_tiny(oracle_lib):
    """Config 0: the set of slots written equals the enumerated expectation, and is all-distinct."""
    wl = W.tiny_decode()
    r, st = H.oracle_caches(wl)
    exp = _slot_bruteforce(wl)
    np.testing.assert_array_equal(r["slots"], exp)
    k = st[0].reshape(wl.num_pages, wl.hkv, wl.page_size, wl.head_dim)
    written = {(pg, off) for pg in range(wl.num_pages) for off in range(wl.page_size)
               if np.any(k[pg, :, off, :] != 0x7F)}
    assert written == {(int(s) // 64, int(s) % 64) for s in exp if s >= 0}


# ----------------------------------------------------------------------------- whole pipeline

def _check_against_torch(wl, got_q, got_iq, rows):
    ref = H.torch_reference(wl)
    for name, got in [("q", got_q), ("iq", got_iq)]:
        r = ref[name]
        g = H.bf16_bits_to_f32(got).astype(np.float64)
        # bf16 rounding of a binary32 pipeline result: half a bf16 spacing plus a few binary32 ulps
        # of the terms that met in the rotation
        tol = H.bf16_half_spacing(r) * (1 + 1e-6) + 8 * 2.0 ** -24 * (np.abs(r) + 4)
        bad = np.abs(g - r) > tol
        assert not bad.any(), (name, np.argwhere(bad)[:5], g[bad][:5], r[bad][:5])
    for ci, name in enumerate(["k", "v", "ik"]):
        spec = wl.caches[ci]
        if spec.heads == 0:
            continue
        r = ref[name]
        codes = rows[name]
        if spec.dtype == W.FP8_E4M3:
            inv = float(np.float32(1.0) / np.float32(spec.scale))
            z = r * inv
            g = H.e4m3_decode(codes)
            zc = np.clip(z, -448, 448)
            tol = H.e4m3_half_spacing(zc) * (1 + 1e-5) + 8 * 2.0 ** -24 * (np.abs(zc) + 4 * inv)
        else:
            zc = r
            g = H.bf16_bits_to_f32(codes).astype(np.float64)
            tol = H.bf16_half_spacing(zc) * (1 + 1e-6) + 8 * 2.0 ** -24 * (np.abs(zc) + 4)
        bad = np.abs(g - zc) > tol
        assert not bad.any(), (name, np.argwhere(bad)[:5], g[bad][:5], zc[bad][:5])


@pytest.mark.parametrize("make", [
    W.tiny_decode, W.tiny_decode_no_index_k,
    lambda: W.ragged(23, seed=11, cache_dtypes=(W.BF16, W.BF16, W.BF16), row_pad=64),
    lambda: W.ragged(9, seed=12, heads=(3, 1, 2, 2), cache_dtypes=(W.FP8_E4M3, W.BF16, W.FP8_E4M3), sigma=3.0),
])
def test_pipeline_matches_torch_transformers_reference(oracle_lib, make):
    """Composition pin: per-head torch rms_norm + transformers' rotate-half RoPE in fp64, then the
    final casts, bound the oracle's Q, index-Q and cache codes to within rounding."""
    wl = make()
    rows = H.oracle_rows(wl)
    _check_against_torch(wl, rows["q"], rows["iq"], rows)


def test_one_hot_worked_example(oracle_lib):
    """Input e_j (1 at column j of a head, 0 elsewhere) with weight 1: RMSNorm gives r at j, with
    r = fl32(1/sqrt(1/128 + eps)); RoPE then puts r*cos(pos*f_j) at j and r*sin(pos*f_j) at j+64.
    This fixes the rotation's orientation and its (i, i+64) pairing."""
    D, pos, j = 128, 1234, 5
    wl = W.tiny_decode()
    wl.x[:] = 0
    wl.x[0, j] = 0x3F80                       # Q head 0 of token 0 = e_j (bf16 1.0)
    wl.weights = [np.full(D, 0x3F80, np.uint16) if w is not None else None for w in wl.weights]
    wl.positions[0] = pos
    rows = H.oracle_rows(wl)
    q = H.bf16_bits_to_f32(rows["q"][0, 0]).astype(np.float64)
    r = 1 / math.sqrt(1 / 128 + float(np.float32(wl.eps)))
    f = 1e4 ** (-2 * j / D)
    exp = np.zeros(D)
    exp[j] = r * math.cos(pos * f)
    exp[j + 64] = r * math.sin(pos * f)
    assert np.all(np.abs(q - exp) <= H.bf16_half_spacing(exp) * 1.001 + 1e-30), (q[[j, j + 64]], exp[[j, j + 64]])


def test_column_layout(oracle_lib):
    """Head h of the packed row (Q heads, then K, V, index-Q, index-K) carries a one-hot at column
    (h mod 64); after RMSNorm + RoPE each output head is non-zero only at {h mod 64, h mod 64 + 64},
    and V heads carry their raw input, so every stream lands in its own output."""
    wl = W.ragged(4, seed=2, heads=(3, 2, 2, 2), cache_dtypes=(W.BF16, W.BF16, W.BF16), pad_frac=0.0)
    D = 128
    H_total = 3 + 2 + 2 + 2 + 2
    wl.x[:] = 0
    for h in range(H_total):
        wl.x[:, h * D + (h % 64)] = 0x4000     # 2.0
    wl = _with_positions(wl, 100)
    rows = H.oracle_rows(wl)
    order = [("q", 3, 0), ("k", 2, 3), ("v", 2, 5), ("iq", 2, 7), ("ik", 2, 9)]
    for name, n, first in order:
        arr = rows[name]
        for t in range(4):
            for hl in range(n):
                h = first + hl
                vals = H.bf16_bits_to_f32(arr[t, hl])
                nz = set(np.flatnonzero(vals).tolist())
                if name == "v":
                    assert nz == {h % 64} and vals[h % 64] == 2.0
                else:
                    assert nz <= {h % 64, h % 64 + 64} and (h % 64) in nz


def test_rms_of_normalised_head_equals_weight(oracle_lib):
    """Invariant: with a constant weight c and RoPE at position 0 (identity), the RMS of each output
    head equals |c| (up to eps and the bf16 output cast)."""
    wl = _with_positions(W.ragged(16, seed=4, heads=(4, 1, 2, 1), cache_dtypes=(W.BF16, W.BF16, W.BF16),
                                  pad_frac=0.0), 0)
    c = 0.75
    wl.weights = [np.full(128, 0x3F40, np.uint16) for _ in range(4)]   # bf16 0.75
    rows = H.oracle_rows(wl)
    for name in ("q", "iq", "k", "ik"):
        y = H.bf16_bits_to_f32(rows[name]).astype(np.float64)
        rms = np.sqrt(np.mean(y ** 2, axis=-1))
        assert np.all(np.abs(rms - c) <= c * 2.0 ** -8), (name, rms)


def test_rope_preserves_pair_norms(oracle_lib):
    """Invariant: (o_i, o_{i+64}) has the norm of (y_i, y_{i+64}); compare position p with position 0."""
    base = W.ragged(8, seed=5, heads=(4, 1, 1, 1), cache_dtypes=(W.BF16, W.BF16, W.BF16), pad_frac=0.0)
    rows0 = H.oracle_rows(_with_positions(base, 0))
    rowsp = H.oracle_rows(_with_positions(base, 3000))
    y = H.bf16_bits_to_f32(rows0["q"]).astype(np.float64)
    o = H.bf16_bits_to_f32(rowsp["q"]).astype(np.float64)
    ny = np.hypot(y[..., :64], y[..., 64:])
    no = np.hypot(o[..., :64], o[..., 64:])
    assert np.all(np.abs(no - ny) <= 2 * 2.0 ** -8 * ny + 1e-6)


def _with_positions(wl, p):
    """Same rows, every token moved to position p; each token's page entry for p is made distinct."""
    import copy
    w2 = copy.deepcopy(wl)
    w2.positions[:] = p
    perm = np.random.default_rng(0).permutation(w2.num_pages)
    for t in range(w2.T):
        if w2.seq_idx[t] >= 0:
            w2.page_table[w2.seq_idx[t], p // w2.page_size] = perm[t]
    return w2


def test_v_bytes_closed_form(oracle_lib):
    """Invariant: an fp8 V cache byte is e4m3(bf16 input * fl32(1/scale)), with no norm or RoPE."""
    wl = W.decode_batch256_padded()
    rows = H.oracle_rows(wl)
    D = 128
    v_cols = slice((wl.hq + wl.hkv) * D, (wl.hq + 2 * wl.hkv) * D)
    a = H.bf16_bits_to_f32(wl.x[:, v_cols]).reshape(wl.T, wl.hkv, D)
    inv = np.float32(1.0) / np.float32(wl.caches[1].scale)
    z = (a * inv).astype(np.float32)
    ref = torch.from_numpy(z).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(rows["v"], ref)


@pytest.mark.parametrize("make", [W.tiny_decode, W.tiny_decode_no_index_k, W.decode_batch256_padded, lambda: W.ragged(50, seed=8, pad_frac=0.3)])
def test_sentinel_and_written_count(oracle_lib, make):
    """Invariants: slots never written keep their sentinel, and the number of changed cache
    elements is exactly (#valid tokens) * heads * D per cache (padding of the view included)."""
    wl = make()
    r, st = H.oracle_caches(wl)
    valid = int(np.count_nonzero(r["slots"] >= 0))
    assert valid == wl.n_written
    for spec, s in zip(wl.caches, st):
        sent = 0x7F if spec.dtype == W.FP8_E4M3 else 0x7F7F
        changed = int(np.count_nonzero(s != sent))
        assert changed == valid * spec.heads * 128


def test_padded_tokens_still_emit_q(oracle_lib):
    """Q and index-Q are produced for every row, padded or not (only cache writes are skipped)."""
    wl = W.decode_batch256_padded()
    rows = H.oracle_rows(wl)
    pad = np.flatnonzero(wl.seq_idx < 0)
    assert pad.size == 26
    assert np.all(np.any(rows["q"][pad] != 0, axis=(1, 2)))
    assert np.all(rows["slots"][pad] == -1)


def test_duplicate_slots_rejected(oracle_lib):
    wl = W.tiny_decode()
    wl.seq_idx[1] = wl.seq_idx[0]
    wl.positions[1] = wl.positions[0]
    with pytest.raises(oracle.OracleError):
        H.oracle_rows(wl)


def test_threads_do_not_change_results(oracle_lib):
    wl = W.ragged(333, seed=9)
    a = H.oracle_rows(wl, num_threads=1)
    b = H.oracle_rows(wl, num_threads=4)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_verify_window_slots_follow_pages(oracle_lib):
    """Verify rows: consecutive tokens of a sequence take consecutive offsets of one page, and a
    token at offset 0 starts the page the table lists for its logical page."""
    wl = W.verify_window(draft_len=3, seqs=64)
    sl = oracle.slots(wl.positions, wl.seq_idx, wl.page_table, wl.num_seqs, wl.max_pages, wl.page_size,
                      wl.num_pages)
    crossings = 0
    for t in range(1, wl.T):
        if wl.seq_idx[t] != wl.seq_idx[t - 1]:
            continue
        p = int(wl.positions[t])
        if p % 64 == 0:
            crossings += 1
            assert sl[t] == wl.page_table[wl.seq_idx[t], p // 64] * 64
        else:
            assert sl[t] == sl[t - 1] + 1
    assert crossings > 0
