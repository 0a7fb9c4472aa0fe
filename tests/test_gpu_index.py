"""GPU parity of the indexer (msa_index_scores + msa_index_topk, through the C ABI) against the CPU
oracle.  Block scores are exact binary64 sums on both sides, so they are compared bit for bit, and so
are the selected block ids and the per-row counts.

Inputs never come from the HIP path: the standalone cases draw index-Q and a pre-populated index-K
cache from the seeded generator; the chained cases run the GPU producer then the GPU indexer, and
the oracle producer then the oracle indexer, from the same generated inputs."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_msa_amd as msa
from paged_kv_cache_msa_amd import workloads as W
from tests import helpers as H

pytestmark = pytest.mark.gpu
THREADS = min(16, os.cpu_count() or 1)
TOPK = 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msa.lib()


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def ik_device(wl, fill):
    c = wl.caches[2]
    if c.dtype == W.FP8_E4M3:
        st = torch.from_numpy(fill).cuda()
    else:
        st = torch.from_numpy(fill.view(np.int16)).cuda()
    view = st.as_strided((wl.num_pages, c.heads, wl.page_size, 128), (*c.strides, 1))
    scale = torch.tensor([c.scale], dtype=torch.float32, device="cuda")
    return st, view, scale


def gpu_index(wl, iq_dev, pos, seq, pt, ik_view, ik_scale, nb, block_tokens=128):
    bs = torch.full((iq_dev.shape[1], wl.T, nb), 7.0, dtype=torch.float64, device="cuda")
    ids = torch.full((iq_dev.shape[1], wl.T, TOPK), -9, dtype=torch.int32, device="cuda")
    counts = torch.full((iq_dev.shape[1], wl.T), -9, dtype=torch.int32, device="cuda")
    msa.msa_index_scores(iq_dev, pos, seq, pt, ik_view, bs, ik_scale=ik_scale, num_pages=wl.num_pages,
                         block_tokens=block_tokens)
    msa.msa_index_topk(bs, ids, counts)
    torch.cuda.synchronize()
    return bs.cpu().numpy(), ids.cpu().numpy(), counts.cpu().numpy()


def oracle_index(wl, iq_bits, ik_storage, nb, block_tokens=128):
    c = wl.caches[2]
    bs = oracle.index_scores(iq_bits, wl.positions, wl.seq_idx, wl.page_table, wl.max_pages, wl.num_seqs,
                             wl.max_pages, wl.page_size, wl.num_pages, ik_storage, c.strides, c.heads, c.dtype,
                             c.scale, block_tokens, nb)
    ids, counts = oracle.index_topk(bs, TOPK)
    return bs, ids, counts


def compare(name, got, ref):
    gbs, gids, gc = got
    rbs, rids, rc = ref
    diff = np.argwhere(~((gbs == rbs) | (np.isneginf(gbs) & np.isneginf(rbs))))
    assert diff.size == 0, f"{name}: {len(diff)} block scores differ, first {diff[:3]}"
    np.testing.assert_array_equal(gids, rids)
    np.testing.assert_array_equal(gc, rc)
    say(f"  {name}: block scores, ids and counts identical ({rbs.shape[1]} tokens x {rbs.shape[0]} heads, "
        f"{int(np.isfinite(rbs).sum())} scored blocks)")


@pytest.mark.parametrize("dtype", [W.FP8_E4M3, W.BF16], ids=["fp8", "bf16"])
def test_index_standalone_decode64(dtype):
    wl = W.decode_batch64()
    if dtype == W.BF16:
        wl.caches[2].dtype = W.BF16
    fill = W.index_cache_fill(wl)
    iq = W.index_queries(wl.T, wl.hiq)
    nb = W.index_blocks(wl)
    st, view, scale = ik_device(wl, fill)
    dev = W.to_device(wl)
    say(f"[gpu] msa_index_scores/topk standalone decode-64, {nb} blocks, {'fp8' if dtype == 0 else 'bf16'}")
    got = gpu_index(wl, torch.from_numpy(iq.view(np.int16)).cuda(), dev.positions, dev.seq_idx, dev.page_table,
                    view, scale, nb)
    compare("standalone", got, oracle_index(wl, iq, fill, nb))


@pytest.mark.parametrize("make", [lambda: W.decode_batch64(), lambda: W.decode_batch256_padded(), lambda: W.verify_window(draft_len=3)],
                         ids=["decode64", "decode256-padded", "verify-window"])
def test_producer_then_indexer(make):
    """The chain of one sparse layer's front half: produce (writes this step's index-K), then score and
    select with this step's index-Q."""
    wl = make()
    fill = W.index_cache_fill(wl)
    nb = W.index_blocks(wl)
    d = W.to_device(wl)
    c = wl.caches[2]
    ik_store = torch.from_numpy(fill).cuda() if c.dtype == W.FP8_E4M3 else torch.from_numpy(fill.view(np.int16)).cuda()
    d.storages[2] = ik_store
    d.caches[2] = ik_store.as_strided((wl.num_pages, c.heads, wl.page_size, 128), (*c.strides, 1))
    say(f"[gpu] produce then index: {wl.name}, {nb} blocks")
    msa.msa_produce(d.x, d.positions, d.seq_idx, d.page_table, *d.weights, d.q_out, d.iq_out,
                    d.caches[0], d.caches[1], d.caches[2], k_scale=d.scales[0], v_scale=d.scales[1],
                    ik_scale=d.scales[2], num_pages=wl.num_pages, rms_eps=wl.eps, rope_theta=wl.theta,
                    slots_out=d.slots)
    got = gpu_index(wl, d.iq_out.view(torch.int16), d.positions, d.seq_idx, d.page_table, d.caches[2],
                    d.scales[2], nb)
    # oracle chain on host copies of the same generated inputs
    host = [H.cache_fill(wl.caches[0]), H.cache_fill(wl.caches[1]), fill.copy()]
    caches = [dict(storage=s, strides=cs.strides, dtype=cs.dtype, scale=cs.scale) for s, cs in zip(host, wl.caches)]
    r = oracle.produce(wl.x, wl.x_stride, wl.T, wl.head_dim, wl.hq, wl.hkv, wl.hiq, wl.hik, wl.positions,
                       wl.seq_idx, wl.page_table, wl.max_pages, wl.num_seqs, wl.max_pages, wl.page_size,
                       wl.num_pages, *wl.weights, wl.eps, wl.theta, caches, num_threads=THREADS)
    compare("chain", got, oracle_index(wl, r["iq"], host[2], nb))


@pytest.mark.parametrize("hiq,hik,dtype", [(4, 1, 0), (4, 2, 0), (1, 1, 0), (3, 1, 0), (1, 1, 1), (3, 1, 1)])
def test_index_head_groups(hiq, hik, dtype):
    """Several index-Q heads per index-K head and several index-K heads (head h reads h // (hiq/hik)),
    fp8 and bf16 keys: launches of two heads and of one (one head per wave takes batches of 8 steps;
    with bf16 keys one batch at a time)."""
    wl = W.ragged(40, seed=hiq * 10 + hik, heads=(2, 1, hiq, hik), pad_frac=0.1, cache_dtypes=(0, 0, dtype))
    fill = W.index_cache_fill(wl, seed=hiq)
    iq = W.index_queries(wl.T, hiq, seed=hik)
    nb = W.index_blocks(wl) + 3          # extra, never-visible blocks stay -inf
    st, view, scale = ik_device(wl, fill)
    dev = W.to_device(wl)
    got = gpu_index(wl, torch.from_numpy(iq.view(np.int16)).cuda(), dev.positions, dev.seq_idx, dev.page_table,
                    view, scale, nb)
    compare(f"groups {hiq}/{hik}", got, oracle_index(wl, iq, fill, nb))


@pytest.mark.parametrize("block_tokens", [100, 36, 256, 8, 24, 136, 2048, 64, 192, 4096])
def test_index_other_block_sizes(block_tokens):
    """Block sizes that are not multiples of the 8-key step (steps straddle pages: per-key page
    lookups), larger ones, and multiples of 8 whose two wave parts are uneven or (8) leave the
    second part empty; 2048 spans more than 64 steps per part (page entries fetched in chunks).
    Multiples of 64 up to 2048 take the batch-in-page kernel (64: one pair of batches; 192: an odd
    number of batches, the second of the last pair discarded); 4096 does not."""
    wl = W.ragged(48, seed=block_tokens, pad_frac=0.1)
    fill = W.index_cache_fill(wl, seed=block_tokens)
    iq = W.index_queries(wl.T, wl.hiq, seed=block_tokens)
    nb = int(wl.positions.max()) // block_tokens + 1
    st, view, scale = ik_device(wl, fill)
    dev = W.to_device(wl)
    got = gpu_index(wl, torch.from_numpy(iq.view(np.int16)).cuda(), dev.positions, dev.seq_idx, dev.page_table,
                    view, scale, nb, block_tokens=block_tokens)
    compare(f"block {block_tokens}", got, oracle_index(wl, iq, fill, nb, block_tokens=block_tokens))


@pytest.mark.parametrize("P", [16, 48, 100, 128, 192])
def test_index_other_page_sizes(P):
    """Page sizes other than 64 under 128-token blocks: a power of two, a multiple of 8 that takes the
    division path, and one that is not a multiple of the 8-key step (per-key page lookups); 128 and
    192 take the batch-in-page kernel (192 by division)."""
    wl = W.ragged(48, seed=300 + P, pad_frac=0.1, page_size=P)
    fill = W.index_cache_fill(wl, seed=P)
    iq = W.index_queries(wl.T, wl.hiq, seed=P)
    nb = int(wl.positions.max()) // 128 + 1
    st, view, scale = ik_device(wl, fill)
    dev = W.to_device(wl)
    got = gpu_index(wl, torch.from_numpy(iq.view(np.int16)).cuda(), dev.positions, dev.seq_idx, dev.page_table,
                    view, scale, nb)
    compare(f"page size {P}", got, oracle_index(wl, iq, fill, nb))


@pytest.mark.parametrize("dtype", [W.FP8_E4M3, W.BF16], ids=["fp8", "bf16"])
def test_index_special_values(dtype):
    """NaN keys (fp8 codes S.1111.111, bf16 NaN), infinite bf16 keys and a query row holding a NaN: a
    NaN score never wins a block, +-inf scores rank as the extremes they are."""
    wl = W.ragged(96, seed=410 + dtype, pad_frac=0.05, cache_dtypes=(W.FP8_E4M3, W.FP8_E4M3, dtype))
    fill = W.index_cache_fill(wl, seed=411)
    rng = np.random.default_rng(412)
    n = fill.size
    if dtype == W.FP8_E4M3:
        fill[rng.choice(n, n // 100, replace=False)] = rng.choice(np.array([0x7F, 0xFF], np.uint8), n // 100)
    else:
        pick = rng.choice(n, n // 500, replace=False)
        fill[pick] = rng.choice(np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1], np.uint16), pick.size)
    iq = W.index_queries(wl.T, wl.hiq, seed=413)
    iq[5, 0, 17] = 0x7FC0                     # one query row of one head holds a NaN
    iq[9, 1, 3] = 0x7F80                      # another holds +inf
    nb = int(wl.positions.max()) // 128 + 1
    st, view, scale = ik_device(wl, fill)
    dev = W.to_device(wl)
    got = gpu_index(wl, torch.from_numpy(iq.view(np.int16)).cuda(), dev.positions, dev.seq_idx, dev.page_table,
                    view, scale, nb)
    ref = oracle_index(wl, iq, fill, nb)
    assert dtype == W.FP8_E4M3 or np.isposinf(ref[0]).any()      # the +inf case is exercised
    compare(f"special values ({'fp8' if dtype == W.FP8_E4M3 else 'bf16'})", got, ref)


@pytest.mark.parametrize("nb", [7, 72, 100, 128, 129, 255, 256, 257, 511, 512, 513, 4096])
def test_topk_rows_with_ties_and_gaps(nb):
    """Rows with repeated scores, -inf gaps and NaN entries; row lengths on both sides of each switch:
    4, 2 and 1 threads per candidate in the rank-based selection (<= 128, <= 256, <= 512 blocks; odd
    lengths pad the last pairs) and the round-based selection beyond."""
    rng = np.random.default_rng(8 + nb)
    rows = 64
    bs = rng.integers(-20, 20, (rows, nb)).astype(np.float64)      # many exact ties
    bs[rng.random((rows, nb)) < 0.3] = -np.inf
    bs[rng.random((rows, nb)) < 0.01] = np.nan
    bs[5, :] = -np.inf                                              # nothing selectable
    bs[6, :10] = 1.0                                                # fewer than k candidates, all tied
    bs[6, 10:] = -np.inf
    bs[7, :] = 3.0                                                  # one long tie
    for k in (1, 16, 64):
        d = torch.from_numpy(bs).cuda()
        ids = torch.full((rows, k), -9, dtype=torch.int32, device="cuda")
        cnt = torch.full((rows,), -9, dtype=torch.int32, device="cuda")
        msa.msa_index_topk(d, ids, cnt)
        torch.cuda.synchronize()
        rids, rc = oracle.index_topk(bs[None], k)
        np.testing.assert_array_equal(ids.cpu().numpy(), rids[0])
        np.testing.assert_array_equal(cnt.cpu().numpy(), rc[0])


def test_index_graph_replay_matches_eager():
    """Scores and top-k of three layers' index-K caches captured in one HIP graph: every replay, with
    eager work and synchronisations between replays, reproduces the eager result bit for bit (and the
    eager result is the oracle's)."""
    wls = [W.decode_batch64(layer=i) for i in range(3)]
    wl = wls[0]
    nb = W.index_blocks(wl)
    pos = torch.from_numpy(wl.positions).cuda()
    seq = torch.from_numpy(wl.seq_idx).cuda()
    pt = torch.from_numpy(np.ascontiguousarray(wl.page_table)).cuda()
    layers = []
    for i, lw in enumerate(wls):
        fill = W.index_cache_fill(lw, seed=50 + i)
        iq = W.index_queries(lw.T, lw.hiq, seed=60 + i)
        st, view, scale = ik_device(lw, fill)
        bs = torch.empty((lw.hiq, lw.T, nb), dtype=torch.float64, device="cuda")
        ids = torch.empty((lw.hiq, lw.T, TOPK), dtype=torch.int32, device="cuda")
        cnt = torch.empty((lw.hiq, lw.T), dtype=torch.int32, device="cuda")
        layers.append(dict(lw=lw, fill=fill, iq=iq, iq_dev=torch.from_numpy(iq.view(np.int16)).cuda(), st=st,
                           view=view, scale=scale, bs=bs, ids=ids, cnt=cnt))

    def step():
        for L in layers:
            msa.msa_index_scores(L["iq_dev"], pos, seq, pt, L["view"], L["bs"], ik_scale=L["scale"],
                                 num_pages=L["lw"].num_pages)
            msa.msa_index_topk(L["bs"], L["ids"], L["cnt"])

    say("[gpu] indexer: 3 layers eager, then captured and replayed 3 times")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    eager = [(L["bs"].cpu().numpy(), L["ids"].cpu().numpy(), L["cnt"].cpu().numpy()) for L in layers]
    for L, got in zip(layers, eager):
        compare("eager", got, oracle_index(L["lw"], L["iq"], L["fill"], nb))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        for L in layers:                       # eager work between replays: clobber the outputs
            L["bs"].fill_(float(rep))
            L["ids"].fill_(-5)
            L["cnt"].fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for L, (ebs, eids, ecnt) in zip(layers, eager):
            gbs = L["bs"].cpu().numpy()
            assert np.array_equal(gbs.view(np.int64), ebs.view(np.int64)), f"replay {rep}: block scores differ"
            np.testing.assert_array_equal(L["ids"].cpu().numpy(), eids)
            np.testing.assert_array_equal(L["cnt"].cpu().numpy(), ecnt)
    say("  3 replays identical to the eager result")
