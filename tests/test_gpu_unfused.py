"""GPU parity of the unfused path (msa_slots + msa_produce_unfused, through the C ABI) against the
CPU oracle, to the same bar as the fused producer: slots and every cache byte bit-exact, Q and
index-Q within one bf16 ulp, untouched cache bytes keep the sentinel.  Also: cache layouts the
fused kernel rejects (strides that are not multiples of 8 elements, bases aligned only to their
element), and HIP graph replay of the 14-launch layer calls."""
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_msa_amd as msa
from paged_kv_cache_msa_amd import workloads as W
from tests import helpers as H
from tests.parity import check, storage_mismatches, written_mask

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msa.lib()


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def workspace(wl):
    n = msa.msa_produce_unfused_workspace_size(wl.T, wl.hkv, wl.hik)
    return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")


def call_unfused(wl, d, ws):
    msa.msa_slots(d.positions, d.seq_idx, d.page_table, d.slots, page_size=wl.page_size, num_pages=wl.num_pages)
    msa.msa_produce_unfused(d.x, d.positions, d.slots, *d.weights, d.q_out, d.iq_out, d.caches[0], d.caches[1],
                            d.caches[2], workspace=ws, k_scale=d.scales[0], v_scale=d.scales[1],
                            ik_scale=d.scales[2], num_pages=wl.num_pages, rms_eps=wl.eps, rope_theta=wl.theta)


def run(wl, d=None):
    d = W.to_device(wl) if d is None else d
    say(f"[gpu] msa_slots + msa_produce_unfused {wl.name}: T={wl.T} heads={wl.hq}/{wl.hkv}/{wl.hiq}/{wl.hik}")
    call_unfused(wl, d, workspace(wl))
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
    """The full 65,536-token prefill chunk, the size the benchmark times this path at."""
    wl = W.prefill_65536()
    check(wl, run(wl))
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [W.BF16, W.FP8_E4M3], ids=["bf16", "fp8"])
def test_mixed_64bit_offsets(dtype):
    wl = W.mixed_batch_64bit(dtype)
    assert wl.num_pages * wl.caches[2].strides[0] > 2 ** 31
    check(wl, run(wl))
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,heads,dtypes,pad", [
    (1, W.DECODE_HEADS, (0, 0, 0), 0.0),
    (7, (5, 3, 0, 2), (0, 1, 0), 0.2),
    (65, (0, 1, 0, 1), (1, 0, 1), 0.1),
    (255, (8, 1, 8, 1), (0, 0, 1), 0.0),
    (2049, (1, 1, 1, 1), (0, 0, 0), 0.05),
    (5000, (32, 2, 2, 1), (1, 1, 0), 0.1),
])
def test_ragged_shapes(T, heads, dtypes, pad):
    wl = W.ragged(T, seed=T + 1, heads=heads, cache_dtypes=dtypes, pad_frac=pad, row_pad=8 * (T % 3))
    check(wl, run(wl))


@pytest.mark.parametrize("P,T", [(1, 300), (48, 2000), (100, 300)])
def test_other_page_sizes(P, T):
    """The per-cache division, remainder and index cast with page sizes other than 64 (one token per
    page, and sizes that are not powers of two)."""
    wl = W.ragged(T, seed=P + T + 1, cache_dtypes=(W.FP8_E4M3, W.BF16, W.FP8_E4M3), page_size=P)
    check(wl, run(wl))


def test_special_values():
    """NaN, infinities, huge and tiny values, all-zero heads and saturating scales."""
    wl = W.ragged(64, seed=78, cache_dtypes=(0, 0, 1), pad_frac=0.0)
    rng = np.random.default_rng(2)
    specials = np.array([0x7FC0, 0xFFC0, 0x7F81, 0x7F80, 0xFF80, 0x7F7F, 0xFF7F, 0x0001, 0x8001, 0x0000, 0x8000],
                        np.uint16)
    flat = wl.x.reshape(-1)
    idx = rng.choice(flat.size, 400, replace=False)
    flat[idx] = rng.choice(specials, idx.size)
    wl.x[5, :] = 0
    wl.x[6, : 128 * 20] = 0x4380
    wl.caches[0].scale = 0.01
    wl.caches[1].scale = 1e-3
    check(wl, run(wl), full=True)


def odd_layout(heads, dtype, scale, num_pages, st, head_pad, page_pad):
    """A cache whose token, head and page strides need not be multiples of 8 elements."""
    sh = 64 * st + head_pad
    sp = heads * sh + page_pad
    return W.CacheSpec(heads, dtype, scale, (num_pages * sp,), (sp, sh, st))


@pytest.mark.parametrize("base_off", [(0, 0, 0), (3, 1, 5)], ids=["aligned-base", "odd-base"])
def test_layouts_the_fused_kernel_rejects(base_off):
    """Token strides of 129..133 elements, odd head and page padding, and bases offset by a few
    elements: msa_produce refuses these views; the unfused path writes exactly the oracle's bytes
    into them and nothing else (whole storages compared, offset prefixes untouched)."""
    wl = W.ragged(300, seed=91, pad_frac=0.1)
    np_ = wl.num_pages
    wl.caches = [odd_layout(2, W.FP8_E4M3, 0.75, np_, 132, 4, 3),
                 odd_layout(2, W.BF16, 1.0, np_, 130, 1, 7),
                 odd_layout(1, W.FP8_E4M3, 1.25, np_, 129, 5, 1)]
    d = W.to_device(wl)
    # move each cache to a storage with a prefix of `off` elements ahead of the view's base
    for i, (c, off) in enumerate(zip(wl.caches, base_off)):
        s = d.storages[i]
        s2 = torch.cat([torch.full((off,), s[0].item(), dtype=s.dtype, device="cuda"), s])
        d.storages[i] = s2
        d.caches[i] = s2.as_strided((np_, c.heads, wl.page_size, 128), (*c.strides, 1), off)
    with pytest.raises(msa.MsaError) as e:
        msa.msa_produce(d.x, d.positions, d.seq_idx, d.page_table, *d.weights, d.q_out, d.iq_out,
                        d.caches[0], d.caches[1], d.caches[2], k_scale=d.scales[0], v_scale=d.scales[1],
                        ik_scale=d.scales[2], num_pages=np_)
    assert e.value.status in (4, 5)
    run(wl, d)
    ref = H.oracle_rows(wl)
    np.testing.assert_array_equal(d.slots.cpu().numpy(), ref["slots"])
    _, st = H.oracle_caches(wl)
    for name, spec, s_ref, s_gpu, off in zip(("k", "v", "ik"), wl.caches, st, d.storages, base_off):
        g = s_gpu.cpu().numpy()
        g = g.view(np.uint8) if spec.dtype == W.FP8_E4M3 else g.view(np.uint16)
        assert np.all(g[:off] == s_ref.reshape(-1)[0]), f"{name}: prefix written"
        mask = written_mask(spec, ref["slots"], wl.page_size)
        diff = storage_mismatches(g[off:], s_ref.reshape(-1), mask, spec.dtype)
        assert diff.size == 0, f"{name} cache: {diff.size} elements differ, first at {diff[:4]}"
    say(f"  odd layouts {base_off}: whole storages identical, every unwritten element holds the sentinel")


def test_graph_replay_matches_eager_and_fused():
    """Three layers of (slots once, then 14 launches per layer) captured in one HIP graph: every
    replay writes what the eager calls wrote, and that is byte for byte what the fused producer
    writes from the same inputs."""
    layers = [W.decode_batch64(layer=i) for i in range(3)]
    devs = [W.to_device(wl) for wl in layers]
    wss = [workspace(wl) for wl in layers]

    def step():
        msa.msa_slots(devs[0].positions, devs[0].seq_idx, devs[0].page_table, devs[0].slots,
                      page_size=layers[0].page_size, num_pages=layers[0].num_pages)
        for wl, d, ws in zip(layers, devs, wss):
            msa.msa_produce_unfused(d.x, d.positions, devs[0].slots, *d.weights, d.q_out, d.iq_out, d.caches[0],
                                    d.caches[1], d.caches[2], workspace=ws, k_scale=d.scales[0],
                                    v_scale=d.scales[1], ik_scale=d.scales[2], num_pages=wl.num_pages)

    def clear():
        for d in devs:
            d.q_out.zero_()
            d.iq_out.zero_()
            for s in d.storages:
                s.fill_(W.SENTINEL_BYTE if s.dtype == torch.uint8 else W.SENTINEL_BYTE * 0x0101)

    step()
    torch.cuda.synchronize()
    eager = [(d.q_out.clone(), d.iq_out.clone(), [s.clone() for s in d.storages]) for d in devs]
    # the fused producer on the same inputs
    clear()
    for wl, d in zip(layers, devs):
        msa.msa_produce(d.x, d.positions, d.seq_idx, d.page_table, *d.weights, d.q_out, d.iq_out,
                        d.caches[0], d.caches[1], d.caches[2], k_scale=d.scales[0], v_scale=d.scales[1],
                        ik_scale=d.scales[2], num_pages=wl.num_pages)
    torch.cuda.synchronize()
    for (q, iq, sts), d in zip(eager, devs):
        assert torch.equal(q, d.q_out) and torch.equal(iq, d.iq_out)
        for a, b in zip(sts, d.storages):
            assert torch.equal(a, b)
    clear()
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
            for ws in wss:
                ws.fill_(0xA5)
            torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (q, iq, sts), d in zip(eager, devs):
            assert torch.equal(q, d.q_out) and torch.equal(iq, d.iq_out), rep
            for a, b in zip(sts, d.storages):
                assert torch.equal(a, b), rep
    check(layers[0], devs[0])
