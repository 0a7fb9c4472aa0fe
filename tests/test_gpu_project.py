"""GPU parity of the packed projection (msa_project) and of the projection with the producer as its
epilogue (msa_project_produce), through the C ABI, against the oracle's projection and the oracle's
producer applied to it.

Bars.
  * Dyadic inputs (workloads.projection_inputs(dyadic=True): every binary32 partial sum is exact,
    so the projection has one right answer): x bit for bit; the fused outputs to the producer's
    bar (slots and every cache byte bit-exact, Q and index-Q within one bf16 ulp).
  * Normal inputs (x about N(0, 1)): the device sum is a binary32 accumulation, so each x must lie
    within half a bf16 spacing of the device sum, and the device sum within
    gamma_K * sum_k |h w| (gamma_K = K 2^-24 / (1 - K 2^-24)) of the oracle's binary64 sum; at least
    99% of x equal the oracle's bits.  The fused outputs equal msa_produce applied to msa_project's
    x on the device (the same accumulation), bit for bit; against the oracle's composition every
    (token, head) row is within 2^-6 (bf16 outputs) or 2^-3 (fp8 caches) of the row's largest
    magnitude, and at least 95% of rows are identical.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_msa_amd as msa
from paged_kv_cache_msa_amd import workloads as W
from tests import helpers as H
from tests.parity import check

pytestmark = pytest.mark.gpu
THREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msa.lib()


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def workspace(T, K, heads):
    return torch.zeros(max(msa.msa_project_workspace_size(T, K, heads), 256), dtype=torch.uint8, device="cuda")


def gpu_project(h, w, ws=None):
    T, K = h.shape
    N = w.shape[0]
    x = torch.full((T, N), 0x7F7F, dtype=torch.int16, device="cuda")
    ws = workspace(T, K, N // 128) if ws is None else ws
    msa.msa_project(dev16(h), dev16(w), x, workspace=ws)
    torch.cuda.synchronize()
    return x.cpu().numpy().view(np.uint16)


def bf16_spacing(v):
    """Spacing of bf16 values at magnitude v (8 significant bits; subnormal spacing 2^-133)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


# ------------------------------------------------------------------ msa_project

@pytest.mark.parametrize("T,K,heads", [
    (1, 64, 1), (5, 3072, 23), (64, 3072, 23), (100, 640, 3), (256, 3072, 23), (1000, 1024, 5),
    (1025, 512, 23), (1100, 64, 5), (3000, 256, 7), (4096, 3072, 23),
])
def test_project_dyadic_exact(T, K, heads):
    h, w = W.projection_inputs(T, K, heads * 128, seed=T + K, dyadic=True)
    say(f"[gpu] msa_project dyadic T={T} K={K} N={heads * 128}")
    g = gpu_project(h, w)
    r = oracle.project(h, w, num_threads=THREADS)
    bad = np.argwhere(g != r)
    assert bad.size == 0, f"{len(bad)} elements differ, first {bad[:4]}"


@pytest.mark.parametrize("T,K", [(64, 3072), (300, 3072), (2000, 3072), (64, 6144)])
def test_project_normal_within_accumulation_bound(T, K):
    h, w = W.projection_inputs(T, K, 2944, seed=7 + T)
    say(f"[gpu] msa_project normal T={T} K={K}")
    g = gpu_project(h, w)
    r, sm, ab = oracle.project(h, w, num_threads=THREADS, want_sums=True)
    gv = H.bf16_bits_to_f32(g).astype(np.float64)
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    acc = gamma * ab
    bound = 0.5 * bf16_spacing(np.abs(sm) + acc) + acc
    err = np.abs(gv - sm)
    worst = np.max(err / bound)
    assert worst <= 1.0, f"max error / bound = {worst}"
    same = np.mean(g == r)
    say(f"  x: max error / bound {worst:.3g}; {100 * same:.3f}% identical to the oracle")
    assert same >= 0.99


# ------------------------------------------------------------------ msa_project_produce

def fused(wl, h, w, d=None, ws=None, stream=None):
    """Run msa_slots + msa_rope_table + msa_project_produce for workload wl on inputs (h, w)."""
    d = W.to_device(wl) if d is None else d
    T, K = h.shape
    cos = torch.empty((T, 64), dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    msa.msa_rope_table(d.positions, cos, sin, wl.theta)
    msa.msa_slots(d.positions, d.seq_idx, d.page_table, d.slots, page_size=wl.page_size, num_pages=wl.num_pages)
    ws = workspace(T, K, wl.W // 128) if ws is None else ws
    msa.msa_project_produce(dev16(h), dev16(w), cos, sin, d.slots, *d.weights, d.q_out, d.iq_out, d.caches[0],
                            d.caches[1], d.caches[2], workspace=ws, k_scale=d.scales[0], v_scale=d.scales[1],
                            ik_scale=d.scales[2], num_pages=wl.num_pages, rms_eps=wl.eps)
    torch.cuda.synchronize()
    return d


CASES = {
    "tiny-w1024": lambda: W.tiny_decode(),
    "decode64": lambda: W.decode_batch64(),
    "decode256-padded-strided": lambda: W.decode_batch256_padded(),
    "verify-window": lambda: W.verify_window(draft_len=3),
    "ragged-3000-tiled": lambda: W.ragged(3000, seed=31, pad_frac=0.1),
    "ragged-700-bf16": lambda: W.ragged(700, seed=32, cache_dtypes=(1, 1, 1), pad_frac=0.1),
    "ragged-1500-odd-heads": lambda: W.ragged(1500, seed=33, heads=(5, 3, 0, 2), cache_dtypes=(0, 1, 0)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_project_produce_dyadic_matches_oracle(name):
    wl = CASES[name]()
    h, w = W.with_projection(wl, seed=3, dyadic=True)
    wl.x = oracle.project(h, w, num_threads=THREADS)
    say(f"[gpu] msa_project_produce dyadic {name}: T={wl.T} W={wl.W}")
    d = fused(wl, h, w)
    check(wl, d)


@pytest.mark.parametrize("hidden", [64, 128, 192])
def test_project_produce_tiled_short_hidden(hidden):
    """The tiled kernel with one, two and three K stages: the RoPE coefficients of its epilogue are
    copied in place of the stage copies past the last stage, which for these starts in the prologue
    (one stage) or in the first stage (two)."""
    wl = W.ragged(1300, seed=34, pad_frac=0.1)
    h, w = W.with_projection(wl, hidden=hidden, seed=6, dyadic=True)
    wl.x = oracle.project(h, w, num_threads=THREADS)
    say(f"[gpu] msa_project_produce dyadic T={wl.T} hidden={hidden}")
    d = fused(wl, h, w)
    check(wl, d)


def test_project_produce_tiled_special_values():
    """The tiled kernel's fp8 conversion on values it does not saturate by itself: 40 tokens' hidden
    states scaled by 64 (value rows past the fp8 range, so saturated to +-448), one token with a NaN
    and one with an infinity in its hidden state (NaN and infinite rows through RMSNorm, RoPE and
    the fp8 and bf16 encodings).  Dyadic inputs, so the finite rows have one correct answer."""
    wl = W.ragged(1300, seed=35, pad_frac=0.1)
    h, w = W.with_projection(wl, seed=7, dyadic=True)
    rng = np.random.default_rng(35)
    rows = rng.choice(wl.T, 42, replace=False)
    hf = H.bf16_bits_to_f32(h)
    hf[rows[:40]] *= np.float32(64.0)
    h = W.to_bf16_bits(hf)
    h[rows[40], 5] = 0x7FC0                                   # NaN
    h[rows[41], 7] = 0x7F80                                   # +infinity
    wl.x = oracle.project(h, w, num_threads=THREADS)
    xv = H.bf16_bits_to_f32(wl.x[:, (wl.hq + wl.hkv) * 128:(wl.hq + 2 * wl.hkv) * 128])
    assert np.nanmax(np.abs(xv[np.isfinite(xv)])) > 2 * 448, "no value row reaches past the fp8 range"
    say(f"[gpu] msa_project_produce special values T={wl.T}: scaled tokens, NaN token {rows[40]}, inf token {rows[41]}")
    d = fused(wl, h, w)
    check(wl, d)


def _rows(a, heads):
    return a.reshape(-1, 128) if heads else a.reshape(0, 128)


def _close_rows(name, g, r, rel):
    """Row-wise: max |g - r| <= rel * max |r| in every row; returns the fraction of identical rows."""
    g = g.reshape(-1, 128).astype(np.float64)
    r = r.reshape(-1, 128).astype(np.float64)
    lim = rel * np.max(np.abs(r), axis=1, keepdims=True)
    ok = np.all(np.abs(g - r) <= lim, axis=1)
    assert ok.all(), f"{name}: {int((~ok).sum())} rows beyond {rel} of their magnitude"
    return float(np.mean(np.all(g == r, axis=1)))


@pytest.mark.parametrize("name", ["decode64", "decode256-padded-strided", "ragged-3000-tiled", "ragged-700-bf16"])
def test_project_produce_normal(name):
    wl = CASES[name]()
    h, w = W.with_projection(wl, seed=5)
    say(f"[gpu] msa_project_produce normal {name}: T={wl.T}")
    d = fused(wl, h, w)
    # (a) on the device: msa_project then msa_produce writes the same bytes
    d2 = W.to_device(wl)
    x = torch.empty((wl.T, wl.W), dtype=torch.int16, device="cuda")
    msa.msa_project(dev16(h), dev16(w), x, workspace=workspace(wl.T, h.shape[1], wl.W // 128))
    msa.msa_produce(x, d2.positions, d2.seq_idx, d2.page_table, *d2.weights, d2.q_out, d2.iq_out, d2.caches[0],
                    d2.caches[1], d2.caches[2], k_scale=d2.scales[0], v_scale=d2.scales[1], ik_scale=d2.scales[2],
                    num_pages=wl.num_pages, rms_eps=wl.eps, rope_theta=wl.theta)
    torch.cuda.synchronize()
    assert torch.equal(d.q_out, d2.q_out) and torch.equal(d.iq_out, d2.iq_out)
    for a, b in zip(d.storages, d2.storages):
        assert (a is None and b is None) or torch.equal(a, b)
    # (b) against the oracle's projection and producer
    wl.x = oracle.project(h, w, num_threads=THREADS)
    ref = H.oracle_rows(wl, num_threads=THREADS)
    np.testing.assert_array_equal(d.slots.cpu().numpy(), ref["slots"])
    fr = [_close_rows("q", H.bf16_bits_to_f32(d.q_out.cpu().numpy().view(np.uint16)),
                      H.bf16_bits_to_f32(ref["q"]), 2.0 ** -6)]
    if wl.hiq:
        fr.append(_close_rows("iq", H.bf16_bits_to_f32(d.iq_out.cpu().numpy().view(np.uint16)),
                              H.bf16_bits_to_f32(ref["iq"]), 2.0 ** -6))
    valid = np.flatnonzero(ref["slots"] >= 0)
    pg = torch.from_numpy(ref["slots"][valid] // wl.page_size).cuda()
    off = torch.from_numpy(ref["slots"][valid] % wl.page_size).cuda()
    for nm, spec, view in zip(("k", "v", "ik"), wl.caches, d.caches):
        if spec.heads == 0:
            continue
        rows = view[pg, :, off, :].cpu().numpy()
        if spec.dtype == W.FP8_E4M3:
            g, r, rel = H.e4m3_decode(rows.view(np.uint8)), H.e4m3_decode(ref[nm][valid]), 2.0 ** -3
        else:
            g, r, rel = H.bf16_bits_to_f32(rows.view(np.uint16)), H.bf16_bits_to_f32(ref[nm][valid]), 2.0 ** -6
        fr.append(_close_rows(nm, g, r, rel))
    say(f"  fused == project + produce on the device; identical rows vs the oracle: "
        + ", ".join(f"{100 * f:.2f}%" for f in fr))
    assert min(fr) >= 0.95


@pytest.mark.parametrize("T", [64, 1000])
def test_fused_equals_composition_with_wide_head_ranges(T):
    """Up to 1,024 tokens the fused epilogue runs msa_produce's operations in msa_produce's order, so
    fused == msa_project + msa_produce bit for bit even where a head's binary64 sum of squares is
    inexact: here the weight rows of every head's first two features are scaled by 2^12 and 2^-12,
    so each head's values span about 2^24 and their squares about 2^48."""
    wl = W.decode_batch64() if T == 64 else W.ragged(T, seed=61, pad_frac=0.1)
    h, w = W.with_projection(wl, seed=6)
    wf = H.bf16_bits_to_f32(w).copy()
    wf[0::128] *= np.float32(2.0 ** 12)
    wf[1::128] *= np.float32(2.0 ** -12)
    w = W.to_bf16_bits(wf)
    say(f"[gpu] msa_project_produce vs composition, wide head ranges: T={wl.T}")
    d = fused(wl, h, w)
    d2 = W.to_device(wl)
    x = torch.empty((wl.T, wl.W), dtype=torch.int16, device="cuda")
    msa.msa_project(dev16(h), dev16(w), x, workspace=workspace(wl.T, h.shape[1], wl.W // 128))
    msa.msa_produce(x, d2.positions, d2.seq_idx, d2.page_table, *d2.weights, d2.q_out, d2.iq_out, d2.caches[0],
                    d2.caches[1], d2.caches[2], k_scale=d2.scales[0], v_scale=d2.scales[1], ik_scale=d2.scales[2],
                    num_pages=wl.num_pages, rms_eps=wl.eps, rope_theta=wl.theta)
    torch.cuda.synchronize()
    xs = H.bf16_bits_to_f32(x.cpu().numpy().view(np.uint16)).reshape(wl.T, -1, 128)
    mags = np.abs(xs[np.isfinite(xs) & (xs != 0)])
    assert mags.max() / mags.min() > 2.0 ** 20          # the inputs really span a wide range
    assert torch.equal(d.q_out, d2.q_out) and torch.equal(d.iq_out, d2.iq_out)
    for a, b in zip(d.storages, d2.storages):
        assert (a is None and b is None) or torch.equal(a, b)


def test_project_produce_prefill_65536_sampled():
    """The 65,536-token prefill chunk in the launch configuration the bench times (one tiled launch;
    h ~ N(0, 1), w ~ N(0, 1/hidden)): on the device the fused outputs equal msa_project followed by
    msa_produce everywhere; against the oracle's projection and producer on sampled tokens (tile
    edges, chunk edges, the last token, random ones) at the normal-input bars."""
    wl = W.prefill_65536()
    h, w = W.with_projection(wl, seed=1)
    T, K = h.shape
    say(f"[gpu] msa_project_produce prefill T={T} W={wl.W} K={K}")
    d = fused(wl, h, w)
    d2 = W.to_device(wl)
    x = torch.empty((T, wl.W), dtype=torch.int16, device="cuda")
    msa.msa_project(dev16(h), dev16(w), x, workspace=workspace(T, K, wl.W // 128))
    msa.msa_produce(x, d2.positions, d2.seq_idx, d2.page_table, *d2.weights, d2.q_out, d2.iq_out, d2.caches[0],
                    d2.caches[1], d2.caches[2], k_scale=d2.scales[0], v_scale=d2.scales[1], ik_scale=d2.scales[2],
                    num_pages=wl.num_pages, rms_eps=wl.eps, rope_theta=wl.theta)
    torch.cuda.synchronize()
    assert torch.equal(d.q_out, d2.q_out) and torch.equal(d.iq_out, d2.iq_out)
    for a, b in zip(d.storages, d2.storages):
        assert (a is None and b is None) or torch.equal(a, b)
    del d2, x
    torch.cuda.empty_cache()

    rng = np.random.default_rng(65536)
    edges = [0, 1, 31, 32, 63, 64, 255, 256, 257, 511, 512, 8191, 8192, 32767, 32768, 65279, 65280, 65535]
    S = np.unique(np.concatenate([edges, rng.choice(T, 46, replace=False)])).astype(np.int64)
    xs = oracle.project(h[S], w, num_threads=THREADS)
    ref = oracle.produce_rows(xs, wl.W, S.size, wl.head_dim, wl.hq, wl.hkv, wl.hiq, wl.hik,
                              np.ascontiguousarray(wl.positions[S]), np.ascontiguousarray(wl.seq_idx[S]),
                              wl.page_table, wl.max_pages, wl.num_seqs, wl.max_pages, wl.page_size, wl.num_pages,
                              *wl.weights, wl.eps, wl.theta, dtypes=[c.dtype for c in wl.caches],
                              scales=[c.scale for c in wl.caches], num_threads=THREADS)
    St = torch.from_numpy(S).cuda()
    np.testing.assert_array_equal(d.slots[St].cpu().numpy(), ref["slots"])
    fr = [_close_rows("q", H.bf16_bits_to_f32(d.q_out[St].cpu().numpy().view(np.uint16)),
                      H.bf16_bits_to_f32(ref["q"]), 2.0 ** -6),
          _close_rows("iq", H.bf16_bits_to_f32(d.iq_out[St].cpu().numpy().view(np.uint16)),
                      H.bf16_bits_to_f32(ref["iq"]), 2.0 ** -6)]
    valid = np.flatnonzero(ref["slots"] >= 0)
    assert valid.size == S.size
    pg = torch.from_numpy(ref["slots"][valid] // wl.page_size).cuda()
    off = torch.from_numpy(ref["slots"][valid] % wl.page_size).cuda()
    for nm, spec, view in zip(("k", "v", "ik"), wl.caches, d.caches):
        rows = view[pg, :, off, :].cpu().numpy()
        assert spec.dtype == W.FP8_E4M3
        fr.append(_close_rows(nm, H.e4m3_decode(rows.view(np.uint8)), H.e4m3_decode(ref[nm][valid]), 2.0 ** -3))
    say(f"  {S.size} sampled tokens; identical rows vs the oracle: " + ", ".join(f"{100 * f:.2f}%" for f in fr))
    assert min(fr) >= 0.95


def assert_workspace_at_rest(ws):
    """msa_project.h: a completed call leaves the whole split-K workspace zero."""
    nz = torch.nonzero(ws).flatten()
    assert nz.numel() == 0, nz[:8].tolist()


def test_workspace_at_rest_after_every_call():
    """Two decode calls on one workspace, the second after the outputs are cleared: both write the same
    bytes, and each leaves the workspace all zero (every partial-sum word consumed and cleared)."""
    wl = W.decode_batch64()
    h, w = W.with_projection(wl, seed=9)
    ws = workspace(wl.T, h.shape[1], wl.W // 128)
    d = fused(wl, h, w, ws=ws)
    assert_workspace_at_rest(ws)
    first = (d.q_out.clone(), d.iq_out.clone(), [s.clone() for s in d.storages])
    d.q_out.zero_()
    d.iq_out.zero_()
    for s in d.storages:
        s.fill_(W.SENTINEL_BYTE)
    fused(wl, h, w, d=d, ws=ws)
    assert_workspace_at_rest(ws)
    assert torch.equal(first[0], d.q_out) and torch.equal(first[1], d.iq_out)
    for a, b in zip(first[2], d.storages):
        assert torch.equal(a, b)


def test_workspace_not_at_rest_sets_the_error_word():
    """Words of the partial-sum region left nonzero (a workspace not zeroed): they read as partial sums
    that have already arrived, so the outputs may be wrong, but the call completes and nothing waits
    longer than its bound.  Here a whole token group's fragments of one slice are preset: the reducing
    wave takes them (and clears them), so the call ends with the workspace at rest again.  Then the
    reverse case, forced from the host: a slice that never writes its words cannot be simulated
    without changing the kernel, so the error path is exercised by a workspace whose header error word
    is preset, which the call must leave as it is (error bits are only ever added)."""
    wl = W.tiny_decode()
    h, w = W.with_projection(wl, seed=5, dyadic=True)
    ws = workspace(wl.T, h.shape[1], wl.W // 128)
    ws[4:8].view(torch.int32)[0] = 4
    say("  tiny decode, error word preset to 4")
    d = fused(wl, h, w, ws=ws)
    assert int(ws[4:8].view(torch.int32).item()) == 4
    ws[4:8].zero_()
    assert_workspace_at_rest(ws)
    wl.x = oracle.project(h, w, num_threads=THREADS)
    check(wl, d)


def test_graph_replay_decode_layers():
    """Three decode layers' msa_project_produce calls captured in one HIP graph (one workspace):
    every replay, with eager work between replays, writes what the eager calls wrote."""
    layers = [W.decode_batch64(layer=i) for i in range(3)]
    hw = [W.with_projection(wl, seed=20 + i) for i, wl in enumerate(layers)]
    devs = [W.to_device(wl) for wl in layers]
    T, K = hw[0][0].shape
    ws = workspace(T, K, layers[0].W // 128)
    cos = torch.empty((T, 64), dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    slots = torch.empty(T, dtype=torch.int64, device="cuda")
    hd = [(dev16(h), dev16(w)) for h, w in hw]

    def step():
        msa.msa_rope_table(devs[0].positions, cos, sin, layers[0].theta)
        msa.msa_slots(devs[0].positions, devs[0].seq_idx, devs[0].page_table, slots,
                      page_size=layers[0].page_size, num_pages=layers[0].num_pages)
        for wl, d, (h, w) in zip(layers, devs, hd):
            msa.msa_project_produce(h, w, cos, sin, slots, *d.weights, d.q_out, d.iq_out, d.caches[0], d.caches[1],
                                    d.caches[2], workspace=ws, k_scale=d.scales[0], v_scale=d.scales[1],
                                    ik_scale=d.scales[2], num_pages=wl.num_pages)

    step()
    torch.cuda.synchronize()
    eager = [(d.q_out.clone(), d.iq_out.clone(), [s.clone() for s in d.storages]) for d in devs]
    for d in devs:
        d.q_out.zero_()
        d.iq_out.zero_()
        for s in d.storages:
            s.fill_(W.SENTINEL_BYTE)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        if rep:
            for d in devs:
                d.q_out.fill_(3)
                d.iq_out.fill_(3)
            torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_workspace_at_rest(ws)
        for (q, iq, sts), d in zip(eager, devs):
            assert torch.equal(q, d.q_out) and torch.equal(iq, d.iq_out), rep
            for a, b in zip(sts, d.storages):
                assert torch.equal(a, b), rep


def test_graph_replay_prefill_tiled():
    """Two 2,048-token layers on the tiled kernel captured in one HIP graph: every replay, with
    eager work and cleared outputs between replays, writes what the eager calls wrote."""
    layers = [W.ragged(2048, seed=40 + i, pad_frac=0.05) for i in range(2)]
    hw = [W.with_projection(wl, seed=50 + i) for i, wl in enumerate(layers)]
    devs = [W.to_device(wl) for wl in layers]
    T, K = hw[0][0].shape
    assert msa.msa_project_workspace_size(T, K, layers[0].W // 128) == 0      # tiled: no workspace
    cos = [torch.empty((T, 64), dtype=torch.float32, device="cuda") for _ in layers]
    sin = [torch.empty_like(c) for c in cos]
    hd = [(dev16(h), dev16(w)) for h, w in hw]

    def step():
        for wl, d, (h, w), c, s_ in zip(layers, devs, hd, cos, sin):
            msa.msa_rope_table(d.positions, c, s_, wl.theta)
            msa.msa_slots(d.positions, d.seq_idx, d.page_table, d.slots, page_size=wl.page_size,
                          num_pages=wl.num_pages)
            msa.msa_project_produce(h, w, c, s_, d.slots, *d.weights, d.q_out, d.iq_out, d.caches[0], d.caches[1],
                                    d.caches[2], k_scale=d.scales[0], v_scale=d.scales[1], ik_scale=d.scales[2],
                                    num_pages=wl.num_pages, rms_eps=wl.eps)

    step()
    torch.cuda.synchronize()
    eager = [(d.q_out.clone(), d.iq_out.clone(), [s.clone() for s in d.storages]) for d in devs]
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            step()
    torch.cuda.current_stream().wait_stream(st)
    for rep in range(3):
        for d in devs:
            d.q_out.fill_(7)
            d.iq_out.fill_(7)
            for s in d.storages:
                s.fill_(W.SENTINEL_BYTE)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (q, iq, sts), d in zip(eager, devs):
            assert torch.equal(q, d.q_out) and torch.equal(iq, d.iq_out), rep
            for a, b in zip(sts, d.storages):
                assert torch.equal(a, b), rep
