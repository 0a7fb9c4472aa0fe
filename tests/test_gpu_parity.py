"""GPU parity: the HIP producer (through the C ABI) against the CPU oracle, element by element.

Bar (per element): slots and every cache byte bit-exact; Q and index-Q within one bf16 ulp
(|gpu - oracle| <= 2^-7 |oracle|, NaN where the oracle has NaN); untouched cache bytes keep
the sentinel.  Workloads: the tiny decode (W = 1024) and its no-index-K variant (W = 896), decode
batch 64, decode batch 256 with padded / out-of-pool tokens and strided input and cache views,
the 65,536-token prefill, the mixed batch whose cache offsets exceed 32 bits (bf16 and fp8), and
ragged token counts that leave partial work-groups and exercise every launch shape.
"""
import os
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_msa_amd as msa
from paged_kv_cache_msa_amd import workloads as W
from tests import helpers as H
from tests.parity import THREADS, check, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msa.lib()


def run(wl):
    d = W.to_device(wl)
    say(f"[gpu] msa_produce {wl.name}: T={wl.T} heads={wl.hq}/{wl.hkv}/{wl.hiq}/{wl.hik}")
    msa.msa_produce(d.x, d.positions, d.seq_idx, d.page_table, *d.weights, d.q_out, d.iq_out,
                    d.caches[0], d.caches[1], d.caches[2], k_scale=d.scales[0], v_scale=d.scales[1],
                    ik_scale=d.scales[2], num_pages=wl.num_pages, rms_eps=wl.eps, rope_theta=wl.theta,
                    slots_out=d.slots)
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("make", [W.tiny_decode, W.tiny_decode_no_index_k], ids=["tiny-w1024", "tiny-w896-no-index-k"])
def test_tiny_decode(make):
    wl = make()
    check(wl, run(wl), full=True)


def test_decode_batch_64():
    wl = W.decode_batch64()
    check(wl, run(wl))


def test_decode_batch_256_padded_strided():
    wl = W.decode_batch256_padded()
    d = run(wl)
    assert int((d.slots < 0).sum()) == 31
    check(wl, d)


def test_prefill_65536():
    wl = W.prefill_65536()
    check(wl, run(wl))


@pytest.mark.parametrize("dtype", [W.BF16, W.FP8_E4M3], ids=["bf16", "fp8"])
def test_mixed_64bit_offsets(dtype):
    wl = W.mixed_batch_64bit(dtype)
    assert wl.num_pages * wl.caches[2].strides[0] > 2 ** 31
    d = run(wl)
    check(wl, d)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,heads,dtypes,pad", [
    (1, W.DECODE_HEADS, (0, 0, 0), 0.0),
    (3, (4, 1, 1, 1), (1, 1, 1), 0.5),
    (7, (5, 3, 0, 2), (0, 1, 0), 0.2),
    (63, (16, 2, 2, 0), (0, 0, 0), 0.1),
    (65, (0, 1, 0, 1), (1, 0, 1), 0.1),
    (255, (8, 1, 8, 1), (0, 0, 1), 0.0),
    (1000, W.DECODE_HEADS, (1, 1, 0), 0.1),
    (2049, (1, 1, 1, 1), (0, 0, 0), 0.05),
    (5000, (32, 2, 2, 1), (0, 0, 0), 0.1),     # 5 passes: two waves per token
    (9000, (8, 2, 2, 1), (0, 1, 0), 0.1),      # 2 passes per wave
    (20001, W.DECODE_HEADS, (0, 0, 0), 0.1),   # 3 passes per wave, ragged last block
])
def test_ragged_and_launch_shapes(T, heads, dtypes, pad):
    wl = W.ragged(T, seed=T, heads=heads, cache_dtypes=dtypes, pad_frac=pad, row_pad=8 * (T % 3))
    check(wl, run(wl))


@pytest.mark.parametrize("T", [64, 8000], ids=["one-pass-waves", "three-pass-waves"])
def test_bf16_cache_scale_pointer_is_ignored(T):
    """A bf16 cache takes no scale: a stray (here misaligned) scale pointer passed with bf16 caches is
    never read and changes nothing."""
    wl = W.ragged(T, seed=11, cache_dtypes=(W.BF16, W.BF16, W.BF16), pad_frac=0.1)
    d = W.to_device(wl)
    stray = torch.zeros(16, dtype=torch.uint8, device="cuda")[1:]
    say(f"[gpu] msa_produce {wl.name} with a stray bf16 scale pointer: T={wl.T}")
    msa.msa_produce(d.x, d.positions, d.seq_idx, d.page_table, *d.weights, d.q_out, d.iq_out,
                    d.caches[0], d.caches[1], d.caches[2], k_scale=stray, v_scale=stray, ik_scale=stray,
                    num_pages=wl.num_pages, rms_eps=wl.eps, rope_theta=wl.theta, slots_out=d.slots)
    torch.cuda.synchronize()
    check(wl, d)


@pytest.mark.parametrize("P,T", [(1, 300), (16, 2000), (48, 300), (48, 8000), (100, 300), (256, 8000)])
def test_other_page_sizes(P, T):
    """Page sizes other than 64: one token per page, a power of two, sizes that take the division
    path (48, 100), and a large one; one-pass (T = 300) and multi-pass (T = 8000) launch shapes."""
    wl = W.ragged(T, seed=P + T, cache_dtypes=(W.FP8_E4M3, W.BF16, W.FP8_E4M3), page_size=P)
    check(wl, run(wl))


@pytest.mark.parametrize("theta,eps", [(1e6, 1e-5), (5e5, 0.0), (10.0, 1e-6)])
def test_other_rope_theta_and_eps(theta, eps):
    """RoPE bases and RMSNorm epsilons other than the workloads' 1e4 / 1e-6 (including eps = 0),
    through the whole producer; positions up to 4095."""
    wl = W.ragged(700, seed=int(theta) % 1000 + 5, cache_dtypes=(W.FP8_E4M3, W.FP8_E4M3, W.BF16))
    wl.theta, wl.eps = theta, eps
    check(wl, run(wl))


def test_special_values():
    """NaN, infinities, huge and tiny values, all-zero heads and saturating scales."""
    wl = W.ragged(64, seed=77, cache_dtypes=(0, 0, 1), pad_frac=0.0)
    rng = np.random.default_rng(1)
    specials = np.array([0x7FC0, 0xFFC0, 0x7F81, 0x7F80, 0xFF80, 0x7F7F, 0xFF7F, 0x0001, 0x8001, 0x0000, 0x8000],
                        np.uint16)
    flat = wl.x.reshape(-1)
    idx = rng.choice(flat.size, 400, replace=False)
    flat[idx] = rng.choice(specials, idx.size)
    wl.x[5, :] = 0                                  # every head of token 5 all-zero
    wl.x[6, : 128 * 20] = 0x4380                    # 256.0: saturates the fp8 cast after scaling
    wl.caches[0].scale = 0.01
    wl.caches[1].scale = 1e-3
    check(wl, run(wl), full=True)


# ------------------------------------------------------------------ step-level entry points

def _oracle_rope(pos, theta, threads=THREADS):
    """The oracle's table, in parallel chunks (the C oracle releases the interpreter lock)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    parts = np.array_split(pos, threads)
    with ThreadPoolExecutor(threads) as ex:
        out = list(ex.map(lambda p: oracle.rope_table(p, theta, 128), parts))
    return np.concatenate([c for c, _ in out]), np.concatenate([s for _, s in out])


def _gpu_rope(pos, theta):
    dp = torch.from_numpy(pos).cuda()
    c = torch.empty((pos.size, 64), dtype=torch.float32, device="cuda")
    s = torch.empty_like(c)
    msa.msa_rope_table(dp, c, s, theta)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("theta,n", [(1e4, 1 << 20), (5e5, 1 << 17), (1e6, 1 << 17)])
def test_rope_table_exhaustive(theta, n):
    """Every position in [0, n) against the oracle, bit for bit: at theta = 1e4 over 2^20 positions
    (a million-token context), and at the other two bases over [0, 131072), which holds every
    position the workloads use.  This pins the single binary32 rounding of the binary64 cos / sin
    of the two implementations over those domains."""
    pos = np.arange(n, dtype=np.int32)
    say(f"[gpu] msa_rope_table theta={theta}: positions [0, {n})")
    gc, gs = _gpu_rope(pos, theta)
    rc, rs = _oracle_rope(pos, theta)
    bad_c = np.flatnonzero(gc.view(np.uint32) != rc.view(np.uint32))
    bad_s = np.flatnonzero(gs.view(np.uint32) != rs.view(np.uint32))
    assert bad_c.size == 0 and bad_s.size == 0, (
        f"cos differs at {bad_c.size} (first (pos, i) {np.unravel_index(bad_c[:3], gc.shape)}), "
        f"sin at {bad_s.size} (first {np.unravel_index(bad_s[:3], gs.shape)})")


def test_rope_table_other_theta_sampled():
    """Random positions over the whole int32 range (negative ones included) at three bases: within
    one binary32 ulp of the oracle (the binary64 sincos of the two implementations may differ in
    its last bit for huge angles)."""
    import oracle
    rng = np.random.default_rng(3)
    for theta in (1e6, 5e5, 1e4):
        pos = np.concatenate([rng.integers(-2 ** 31, 2 ** 31 - 1, 20000), [0, 1, -1, 2 ** 31 - 1, -2 ** 31]]).astype(np.int32)
        gc, gs = _gpu_rope(pos, theta)
        rc, rs = oracle.rope_table(pos, theta, 128)
        n_diff = int(np.count_nonzero(gc.view(np.uint32) != rc.view(np.uint32)) +
                     np.count_nonzero(gs.view(np.uint32) != rs.view(np.uint32)))
        assert np.all(np.abs(gc.astype(np.float64) - rc) <= H.ulp32(rc)), theta
        assert np.all(np.abs(gs.astype(np.float64) - rs) <= H.ulp32(rs)), theta
        say(f"  rope theta={theta}: {n_diff} of {2 * gc.size} coefficients differ by one ulp")


def _encode_chunks(fn, values, threads=THREADS):
    from concurrent.futures import ThreadPoolExecutor
    parts = np.array_split(values, threads)
    with ThreadPoolExecutor(threads) as ex:
        return np.concatenate(list(ex.map(fn, parts)))


@pytest.mark.timeout(900)
def test_quantize_exhaustive_fp32():
    """All 2^32 binary32 inputs through the device casts (scale 1 for fp8) against the oracle."""
    import oracle
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    chunk = 1 << 28
    for base in range(0, 1 << 32, chunk):
        u = np.arange(base, base + chunk, dtype=np.uint64).astype(np.uint32)
        v = u.view(np.float32)
        dv = torch.from_numpy(v).cuda()
        out8 = torch.empty(chunk, dtype=torch.uint8, device="cuda")
        out16 = torch.empty(chunk, dtype=torch.int16, device="cuda")
        msa.msa_quantize(dv, out8, msa.MSA_CACHE_FP8_E4M3, one)
        msa.msa_quantize(dv, out16, msa.MSA_CACHE_BF16)
        torch.cuda.synchronize()
        g8 = out8.cpu().numpy()
        g16 = out16.cpu().numpy().view(np.uint16)
        r8 = _encode_chunks(oracle.encode_e4m3, v)
        r16 = _encode_chunks(oracle.encode_bf16, v)
        bad8, bad16 = np.flatnonzero(g8 != r8), np.flatnonzero(g16 != r16)
        assert bad8.size == 0, f"e4m3: {bad8.size} mismatches from 0x{base:08x}, first input 0x{u[bad8[0]]:08x}"
        assert bad16.size == 0, f"bf16: {bad16.size} mismatches from 0x{base:08x}, first input 0x{u[bad16[0]]:08x}"
        del dv, out8, out16
        say(f"  quantize chunk 0x{base:08x} ok")
    say("  quantize: all 2^32 inputs identical for e4m3 (scale 1) and bf16")


def test_quantize_scales():
    """e4m3(v * fl32(1/scale)) for many scales: exercises the binary32 reciprocal's rounding."""
    import oracle
    rng = np.random.default_rng(4)
    v = (rng.standard_normal(1 << 20) * 30).astype(np.float32)
    for sc in np.concatenate([rng.uniform(0.5, 2.0, 24), [3.0, 7.0, 0.1, 1e-3, 448.0, 1e-30, 1e30]]).astype(np.float32):
        dv = torch.from_numpy(v).cuda()
        ds = torch.tensor([sc], dtype=torch.float32, device="cuda")
        out = torch.empty(v.size, dtype=torch.uint8, device="cuda")
        msa.msa_quantize(dv, out, msa.MSA_CACHE_FP8_E4M3, ds)
        torch.cuda.synchronize()
        inv = np.float32(1.0) / sc
        ref = oracle.encode_e4m3((v * inv).astype(np.float32))
        assert np.array_equal(out.cpu().numpy(), ref), float(sc)


def test_rms_scale_random_and_edges():
    import oracle
    rng = np.random.default_rng(5)
    ss = np.concatenate([rng.uniform(0, 2000, 1 << 20), np.exp2(rng.uniform(-300, 300, 1 << 18)),
                         [0.0, 1e-300, 128.0, 1e300]]).astype(np.float64)
    for eps in (1e-6, 0.0, 1e-5, 0.5):
        d = torch.from_numpy(ss).cuda()
        r = torch.empty(ss.size, dtype=torch.float32, device="cuda")
        msa.msa_rms_scale(d, r, eps)
        torch.cuda.synchronize()
        ref = oracle.rms_scale(ss, 128, eps)
        assert np.array_equal(r.cpu().numpy().view(np.uint32), ref.view(np.uint32)), eps


# ------------------------------------------------------------------ HIP graph replay

def test_graph_replay_matches_eager():
    """Three layer calls captured in one HIP graph: every replay (with eager work and
    synchronisation between replays) writes exactly what the eager calls wrote."""
    layers = [W.decode_batch64(layer=i) for i in range(3)]
    devs = [W.to_device(wl) for wl in layers]

    def call(wl, d):
        msa.msa_produce(d.x, d.positions, d.seq_idx, d.page_table, *d.weights, d.q_out, d.iq_out,
                        d.caches[0], d.caches[1], d.caches[2], k_scale=d.scales[0], v_scale=d.scales[1],
                        ik_scale=d.scales[2], num_pages=wl.num_pages, slots_out=d.slots)

    for wl, d in zip(layers, devs):
        call(wl, d)
    torch.cuda.synchronize()
    eager = [(d.q_out.clone(), d.iq_out.clone(), [s.clone() for s in d.storages]) for d in devs]
    for d in devs:
        d.q_out.zero_()
        d.iq_out.zero_()
        for s in d.storages:
            s.fill_(W.SENTINEL_BYTE if s.dtype == torch.uint8 else W.SENTINEL_BYTE * 0x0101)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for wl, d in zip(layers, devs):
                call(wl, d)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        if rep:
            # eager work between replays: clobber the outputs the graph rewrites
            for d in devs:
                d.q_out.fill_(3)
                d.iq_out.fill_(3)
            torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (q, iq, sts), d in zip(eager, devs):
            assert torch.equal(q, d.q_out) and torch.equal(iq, d.iq_out), rep
            for a, b in zip(sts, d.storages):
                assert torch.equal(a, b), rep
    check(layers[0], devs[0])


def _reset(devs):
    for d in devs:
        d.q_out.fill_(3)
        d.iq_out.fill_(3)
        d.slots.fill_(-7)
        for st in d.storages:
            st.fill_(W.SENTINEL_BYTE if st.dtype == torch.uint8 else W.SENTINEL_BYTE * 0x0101)


def test_decode_graph_steps_with_metadata_updated_in_place():
    """The serving loop's decode step: three layer calls captured once, then four steps, each after
    the host wrote that step's metadata into the same device buffers (every position advanced by one,
    eight tokens crossing into a new page; a logical page remapped to another physical page; four
    tokens padded; one page-table entry outside the pool).  Before every replay the caches are refilled
    with the sentinel and the outputs clobbered, so each replay must write everything itself: every
    layer of every step equals the oracle on that step's metadata, and every other cache element
    still holds the sentinel."""
    import dataclasses
    layers = [W.decode_batch64(layer=i) for i in range(3)]
    P = layers[0].page_size
    pos = layers[0].positions.copy()
    pos[:8] = (pos[:8] // P) * P + P - 1            # the next step starts a new page for these
    seq = layers[0].seq_idx.copy()
    pt = np.ascontiguousarray(layers[0].page_table.copy())
    layers = [dataclasses.replace(wl, positions=pos.copy()) for wl in layers]
    devs = [W.to_device(wl) for wl in layers]
    d0 = devs[0]
    for d in devs[1:]:
        d.positions, d.seq_idx, d.page_table = d0.positions, d0.seq_idx, d0.page_table

    def call(wl, d):
        msa.msa_produce(d.x, d.positions, d.seq_idx, d.page_table, *d.weights, d.q_out, d.iq_out,
                        d.caches[0], d.caches[1], d.caches[2], k_scale=d.scales[0], v_scale=d.scales[1],
                        ik_scale=d.scales[2], num_pages=wl.num_pages, slots_out=d.slots)

    for wl, d in zip(layers, devs):
        call(wl, d)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for wl, d in zip(layers, devs):
                call(wl, d)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for step in range(4):
        if step >= 1:
            pos += 1
        if step == 2:
            for t in range(4):                     # remap the page these tokens just entered
                lp = pos[t] // P
                pt[t, lp], pt[t + 32, 0] = pt[t + 32, 0], pt[t, lp]
            seq[10:14] = -1
        if step == 3:
            seq[10:14] = np.arange(10, 14)
            pt[20, pos[20] // P] = layers[0].num_pages + 5
        d0.positions.copy_(torch.from_numpy(pos))
        d0.seq_idx.copy_(torch.from_numpy(seq))
        d0.page_table.copy_(torch.from_numpy(pt))
        _reset(devs)
        torch.cuda.synchronize()
        say(f"[gpu] decode graph step {step}: replay of 3 layer calls")
        g.replay()
        torch.cuda.synchronize()
        n_valid = int(np.count_nonzero(d0.slots.cpu().numpy() >= 0))
        if step == 2:
            assert n_valid == 60
        if step == 3:
            assert n_valid == 63
        for wl, d in zip(layers, devs):
            check(dataclasses.replace(wl, positions=pos.copy(), seq_idx=seq.copy(), page_table=pt.copy()), d)


# ------------------------------------------------------------------ operand residency (eager calls)

def test_check_device_pointers():
    """The residency check alone (nothing is launched): device memory of this device passes with an
    extent inside its allocation; pageable host memory, or an extent past the allocation, fails with
    the index of the pointer; pinned host memory passes."""
    dev = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    host = torch.empty(1 << 20, dtype=torch.uint8)
    pinned = torch.empty(1 << 20, dtype=torch.uint8, pin_memory=True)
    assert msa.msa_check_device_pointers([dev.data_ptr()], [1 << 20]) == (0, -1)
    assert msa.msa_check_device_pointers([dev.data_ptr() + 4096, None], [4096, 0]) == (0, -1)
    assert msa.msa_check_device_pointers([dev.data_ptr(), host.data_ptr()], [64, 64]) == (10, 1)
    assert msa.msa_check_device_pointers([dev.data_ptr()], [1 << 50]) == (10, 0)
    assert msa.msa_check_device_pointers([pinned.data_ptr()], [1 << 20]) == (0, -1)
    # host cost of the check, for the record
    import time
    ptrs = [dev.data_ptr()] * 16
    t0 = time.perf_counter()
    for _ in range(200):
        msa.msa_check_device_pointers(ptrs, [64] * 16)
    say(f"  residency check of 16 pointers: {(time.perf_counter() - t0) / 200 * 1e6:.1f} us on the host")


def test_eager_call_with_cache_past_its_allocation_is_refused():
    """A call whose cache view, by the page count it is given, reaches past the end of the cache's
    allocation returns MSA_ERR_NOT_DEVICE and launches nothing (caches keep the sentinel, Q keeps its
    contents).  Every page-table entry stays inside the real allocation, so even a launch would only
    touch memory the call owns."""
    import ctypes
    torch.cuda.empty_cache()
    wl = W.decode_batch64()
    d = W.to_device(wl)
    L = msa.lib()
    views = [msa.cache_view(c, sc) for c, sc in zip(d.caches, d.scales)]
    st = L.msa_produce(d.x.data_ptr(), d.x.stride(0), wl.T, 128, wl.hq, wl.hkv, wl.hiq, wl.hik,
                       d.positions.data_ptr(), d.seq_idx.data_ptr(), d.page_table.data_ptr(), d.page_table.stride(0),
                       wl.num_seqs, wl.max_pages, wl.page_size, 1000 * wl.num_pages,
                       *[w.data_ptr() for w in d.weights], 1e-6, 1e4, d.q_out.data_ptr(), d.iq_out.data_ptr(),
                       *[ctypes.byref(v) for v in views], d.slots.data_ptr(),
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 10, msa.string(st)
    assert int((d.q_out != 0).sum()) == 0
    assert int((d.slots != -7).sum()) == 0
    for store in d.storages:
        assert int((store != W.SENTINEL_BYTE).sum()) == 0


# ------------------------------------------------------------------ speculative-decoding verify rows

@pytest.mark.parametrize("draft_len,seqs,dtype", [(3, 64, W.FP8_E4M3), (7, 256, W.FP8_E4M3), (1, 64, W.BF16)])
def test_verify_window_rows(draft_len, seqs, dtype):
    """1 + draft_len consecutive tokens per sequence (windows straddle page boundaries)."""
    wl = W.verify_window(draft_len=draft_len, seqs=seqs, cache_dtype=dtype)
    check(wl, run(wl))


def test_target_and_draft_geometries():
    """A target-model layer and a draft-model layer with its own, smaller page pool and page table
    (bf16 caches) produced back to back: each matches the oracle and leaves the other's caches
    untouched (each storage's written-element count is exact)."""
    target = W.verify_window(draft_len=3, seqs=64, seed=21)
    draft = W.verify_window(draft_len=3, seqs=64, seed=22, num_pages=3000, max_pages=160, cache_dtype=W.BF16)
    dt, dd = run(target), run(draft)
    check(target, dt)
    check(draft, dd)
