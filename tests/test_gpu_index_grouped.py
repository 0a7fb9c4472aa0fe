"""GPU parity of msa_index_scores_grouped (through the C ABI) against the CPU oracle: block scores are
exact binary64 sums, so every block score, selected id and count is compared bit for bit, as for
msa_index_scores.  The grouping only decides which tokens share key loads; any grouping (windows of
one sequence, groups that straddle sequences, padded tokens, a partial last group) must give the
same scores.  Inputs are seeded and synthetic (the index-K cache pre-populated by the generator)."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_msa_amd as msa
from paged_kv_cache_msa_amd import workloads as W

pytestmark = pytest.mark.gpu
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
    st = torch.from_numpy(fill if c.dtype == W.FP8_E4M3 else fill.view(np.int16)).cuda()
    view = st.as_strided((wl.num_pages, c.heads, wl.page_size, 128), (*c.strides, 1))
    scale = torch.tensor([c.scale], dtype=torch.float32, device="cuda")
    return st, view, scale


def run(wl, fill, iq, nb, group, block_tokens=128):
    """Grouped scores + top-k on the device, and the oracle's, for workload wl."""
    st, view, scale = ik_device(wl, fill)
    dev = W.to_device(wl)
    hiq = iq.shape[1]
    bs = torch.full((hiq, wl.T, nb), 7.0, dtype=torch.float64, device="cuda")
    ids = torch.full((hiq, wl.T, TOPK), -9, dtype=torch.int32, device="cuda")
    cnt = torch.full((hiq, wl.T), -9, dtype=torch.int32, device="cuda")
    msa.msa_index_scores(torch.from_numpy(iq.view(np.int16)).cuda(), dev.positions, dev.seq_idx, dev.page_table,
                         view, bs, ik_scale=scale, num_pages=wl.num_pages, block_tokens=block_tokens,
                         group_tokens=group)
    msa.msa_index_topk(bs, ids, cnt)
    torch.cuda.synchronize()
    c = wl.caches[2]
    rbs = oracle.index_scores(iq, wl.positions, wl.seq_idx, wl.page_table, wl.max_pages, wl.num_seqs, wl.max_pages,
                              wl.page_size, wl.num_pages, fill, c.strides, c.heads, c.dtype, c.scale, block_tokens,
                              nb)
    rids, rc = oracle.index_topk(rbs, TOPK)
    return (bs.cpu().numpy(), ids.cpu().numpy(), cnt.cpu().numpy()), (rbs, rids, rc)


def compare(name, got, ref):
    gbs, gids, gc = got
    rbs, rids, rc = ref
    same = (gbs == rbs) | (np.isneginf(gbs) & np.isneginf(rbs)) | (np.isnan(gbs) & np.isnan(rbs))
    diff = np.argwhere(~same)
    assert diff.size == 0, f"{name}: {len(diff)} block scores differ, first {diff[:3]}"
    np.testing.assert_array_equal(gids, rids)
    np.testing.assert_array_equal(gc, rc)
    say(f"  {name}: identical ({rbs.shape[1]} tokens x {rbs.shape[0]} heads, {int(np.isfinite(rbs).sum())} "
        f"scored blocks)")


@pytest.mark.parametrize("draft_len,dtype", [(3, W.FP8_E4M3), (3, W.BF16), (1, W.FP8_E4M3), (7, W.FP8_E4M3),
                                             (7, W.BF16)], ids=["w4-fp8", "w4-bf16", "w2-fp8", "w8-fp8", "w8-bf16"])
def test_verify_windows_one_group_per_window(draft_len, dtype):
    """Verify windows of 1 + draft_len tokens scored one window per group (a window of 8 runs one
    index-Q head per launch: 8 tokens x 2 heads would exceed the 8 queries of a wave); a quarter of
    the windows straddle a page boundary."""
    wl = W.verify_window(draft_len=draft_len, seqs=48, seed=20 + draft_len, cache_dtype=dtype)
    fill = W.index_cache_fill(wl, seed=21)
    iq = W.index_queries(wl.T, wl.hiq, seed=22)
    nb = W.index_blocks(wl)
    say(f"[gpu] grouped indexer, {wl.name}, group {1 + draft_len}, {'fp8' if dtype == 0 else 'bf16'}")
    compare(f"window {1 + draft_len}", *run(wl, fill, iq, nb, 1 + draft_len))


@pytest.mark.parametrize("group", [2, 3, 5, 8])
def test_groups_that_straddle_windows(group):
    """Windows of 4 scored in groups of 2, 3, 5 and 8: groups holding two or three sequences take one
    pass per sequence; 256 tokens leave a partial last group for 3 and 5."""
    wl = W.verify_window(draft_len=3, seqs=64, seed=30)
    fill = W.index_cache_fill(wl, seed=31)
    iq = W.index_queries(wl.T, wl.hiq, seed=32)
    nb = W.index_blocks(wl)
    say(f"[gpu] grouped indexer, windows of 4 in groups of {group}")
    compare(f"groups of {group}", *run(wl, fill, iq, nb, group))


@pytest.mark.parametrize("make,group", [(lambda: W.decode_batch64(), 4), (lambda: W.decode_batch256_padded(), 4),
                                        (lambda: W.decode_batch256_padded(), 8)],
                         ids=["decode64-g4", "decode256-padded-g4", "decode256-padded-g8"])
def test_one_token_per_sequence(make, group):
    """Decode batches (one token per sequence): every group holds as many sequences as tokens, so each
    pass scores one token; padded tokens and tokens whose page lies past the pool select nothing."""
    wl = make()
    fill = W.index_cache_fill(wl, seed=41)
    iq = W.index_queries(wl.T, wl.hiq, seed=42)
    nb = W.index_blocks(wl)
    say(f"[gpu] grouped indexer, {wl.name}, groups of {group}")
    compare(f"{wl.name} g{group}", *run(wl, fill, iq, nb, group))


@pytest.mark.parametrize("hiq,hik,dtype,group", [(4, 1, 0, 4), (4, 2, 0, 2), (1, 1, 0, 8), (3, 1, 0, 4),
                                                 (3, 1, 1, 3), (1, 1, 1, 5)])
def test_head_groups(hiq, hik, dtype, group):
    """Index-Q heads per index-K head 4, 2, 1, 3 with fp8 and bf16 keys: launches of two heads (group x 2
    <= 8) and of one, a last single head after pairs (3 heads), padded tokens."""
    wl = W.ragged(40, seed=hiq * 10 + hik + group, heads=(2, 1, hiq, hik), pad_frac=0.1, cache_dtypes=(0, 0, dtype))
    fill = W.index_cache_fill(wl, seed=hiq)
    iq = W.index_queries(wl.T, hiq, seed=hik)
    nb = W.index_blocks(wl) + 3                   # extra, never-visible blocks stay -inf
    say(f"[gpu] grouped indexer, heads {hiq}/{hik}, {'fp8' if dtype == 0 else 'bf16'}, groups of {group}")
    compare(f"heads {hiq}/{hik} g{group}", *run(wl, fill, iq, nb, group))


@pytest.mark.parametrize("block_tokens", [64, 192, 2048, 100, 4096])
def test_block_sizes(block_tokens):
    """Blocks of 64 (two batches), 192 (an odd number of batches) and 2,048 (64 batches) take the grouped
    kernel; 100 and 4,096 run the per-token kernels (same results)."""
    wl = W.verify_window(draft_len=3, seqs=32, seed=50)
    fill = W.index_cache_fill(wl, seed=51)
    iq = W.index_queries(wl.T, wl.hiq, seed=52)
    nb = int(wl.positions.max()) // block_tokens + 1
    say(f"[gpu] grouped indexer, windows of 4, blocks of {block_tokens}")
    compare(f"block {block_tokens}", *run(wl, fill, iq, nb, 4, block_tokens=block_tokens))


@pytest.mark.parametrize("dtype", [W.FP8_E4M3, W.BF16], ids=["fp8", "bf16"])
def test_special_values(dtype):
    """NaN keys, infinite bf16 keys and query rows holding a NaN or an infinity, in windows of 4."""
    wl = W.verify_window(draft_len=3, seqs=32, seed=60 + dtype, cache_dtype=dtype)
    fill = W.index_cache_fill(wl, seed=61)
    rng = np.random.default_rng(62)
    n = fill.size
    if dtype == W.FP8_E4M3:
        fill[rng.choice(n, n // 100, replace=False)] = rng.choice(np.array([0x7F, 0xFF], np.uint8), n // 100)
    else:
        pick = rng.choice(n, n // 500, replace=False)
        fill[pick] = rng.choice(np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1], np.uint16), pick.size)
    iq = W.index_queries(wl.T, wl.hiq, seed=63)
    iq[5, 0, 17] = 0x7FC0
    iq[9, 1, 3] = 0x7F80
    nb = W.index_blocks(wl)
    say(f"[gpu] grouped indexer, special values, {'fp8' if dtype == 0 else 'bf16'}")
    compare("special values", *run(wl, fill, iq, nb, 4))


def test_grouped_equals_per_token_in_a_graph():
    """Both entry points captured in one HIP graph on the same verify windows: every replay writes the
    same block scores from both, equal to the oracle's."""
    wl = W.verify_window(draft_len=3, seqs=64, seed=70)
    fill = W.index_cache_fill(wl, seed=71)
    iq = W.index_queries(wl.T, wl.hiq, seed=72)
    nb = W.index_blocks(wl)
    st, view, scale = ik_device(wl, fill)
    dev = W.to_device(wl)
    q = torch.from_numpy(iq.view(np.int16)).cuda()
    a = torch.empty((wl.hiq, wl.T, nb), dtype=torch.float64, device="cuda")
    b = torch.empty_like(a)

    def step():
        msa.msa_index_scores(q, dev.positions, dev.seq_idx, dev.page_table, view, a, ik_scale=scale,
                             num_pages=wl.num_pages)
        msa.msa_index_scores(q, dev.positions, dev.seq_idx, dev.page_table, view, b, ik_scale=scale,
                             num_pages=wl.num_pages, group_tokens=4)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    c = wl.caches[2]
    ref = oracle.index_scores(iq, wl.positions, wl.seq_idx, wl.page_table, wl.max_pages, wl.num_seqs, wl.max_pages,
                              wl.page_size, wl.num_pages, fill, c.strides, c.heads, c.dtype, c.scale, 128, nb)
    for rep in range(3):
        a.fill_(float(rep))
        b.fill_(-float(rep))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ga, gb = a.cpu().numpy(), b.cpu().numpy()
        assert np.array_equal(ga.view(np.int64), gb.view(np.int64)), rep
        assert np.array_equal(ga.view(np.int64), ref.view(np.int64)), rep
    say("  3 replays: grouped == per-token == oracle")
