"""Pins of the oracle's indexer (CPU only): block scores and top-k selection against an independent
numpy formulation (decode the cache from the format definition, fp64 matmul, masked block max,
lexicographic sort), a one-hot closed form, and invariants (scale does not change the selection,
count = min(k, visible blocks), only visible blocks are picked, ties go to the lower block index)."""
import numpy as np
import pytest

import oracle
from paged_kv_cache_msa_amd import workloads as W
from tests import helpers as H


def small_case(seed=0, dtype=W.FP8_E4M3, hiq=2, hik=1, T=6, pos_hi=700, max_pages=16):
    rng = np.random.default_rng(seed)
    P, S = 64, T
    num_pages = 4 * S * max_pages
    pos = rng.integers(0, pos_hi, T).astype(np.int32)
    seq = np.arange(T, dtype=np.int32)
    pt = rng.permutation(num_pages)[: S * max_pages].astype(np.int32).reshape(S, max_pages)
    shape = (num_pages, hik, P, 128)
    strides = (hik * P * 128, P * 128, 128)
    if dtype == W.FP8_E4M3:
        cache = rng.integers(0, 254, np.prod(shape), dtype=np.uint16).astype(np.uint8)
        cache[cache >= 0x7F] += 1
    else:
        cache = W.to_bf16_bits(rng.standard_normal(np.prod(shape), dtype=np.float32))
    iq = W.index_queries(T, hiq, seed=seed)
    return dict(pos=pos, seq=seq, pt=pt, P=P, S=S, max_pages=max_pages, num_pages=num_pages, cache=cache,
                strides=strides, hik=hik, dtype=dtype, iq=iq, hiq=hiq, T=T)


def run_oracle(c, scale=1.5, block=128, nb=None, k=16):
    nb = nb if nb is not None else int(c["pos"].max()) // block + 1
    bs = oracle.index_scores(c["iq"], c["pos"], c["seq"], c["pt"], c["max_pages"], c["S"], c["max_pages"], c["P"],
                             c["num_pages"], c["cache"], c["strides"], c["hik"], c["dtype"], scale, block, nb)
    ids, counts = oracle.index_topk(bs, k)
    return bs, ids, counts


def numpy_reference(c, scale=1.5, block=128, nb=None, k=16):
    """Independent formulation: gather each sequence's visible keys, decode them from the format
    definition (tests/helpers), one fp64 matmul per token, masked max per block, lexsort."""
    nb = nb if nb is not None else int(c["pos"].max()) // block + 1
    hiq, hik, T, P = c["hiq"], c["hik"], c["T"], c["P"]
    sp, sh, st = c["strides"]
    dec = H.e4m3_decode(c["cache"]) if c["dtype"] == W.FP8_E4M3 else H.bf16_bits_to_f32(c["cache"]).astype(np.float64)
    sc = scale if c["dtype"] == W.FP8_E4M3 else 1.0
    q = H.bf16_bits_to_f32(c["iq"]).astype(np.float64)
    bs = np.full((hiq, T, nb), -np.inf)
    for t in range(T):
        p = np.arange(c["pos"][t] + 1)
        pages = c["pt"][c["seq"][t], p // P].astype(np.int64)
        for h in range(hiq):
            g = h // (hiq // hik)
            idx = pages[:, None] * sp + g * sh + (p % P)[:, None] * st + np.arange(128)[None, :]
            keys = dec[idx]                                  # [n_keys, 128]
            s = (keys @ q[t, h]) * sc
            for b in range(min(nb, p[-1] // block + 1)):
                bs[h, t, b] = s[b * block:(b + 1) * block].max()
    ids = np.full((hiq, T, k), -1, np.int32)
    for h in range(hiq):
        for t in range(T):
            row = bs[h, t]
            cand = np.flatnonzero(row > -np.inf)
            order = cand[np.lexsort((cand, -row[cand]))]
            ids[h, t, : min(k, order.size)] = order[:k]
    return bs, ids


@pytest.mark.parametrize("dtype,hiq,hik", [(W.FP8_E4M3, 2, 1), (W.BF16, 2, 1), (W.FP8_E4M3, 4, 2)])
def test_index_matches_numpy_formulation(oracle_lib, dtype, hiq, hik):
    c = small_case(seed=hiq + dtype, dtype=dtype, hiq=hiq, hik=hik)
    bs, ids, counts = run_oracle(c)
    rbs, rids = numpy_reference(c)
    np.testing.assert_array_equal(bs, rbs)     # sums of exact products: exact in any order
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_array_equal(counts, (rids >= 0).sum(-1))


def test_one_hot_query_closed_form(oracle_lib):
    """q = e_j: the score of key p is its j-th element times the scale, so a block's score is the
    largest j-th element among its visible keys."""
    c = small_case(seed=3, T=3)
    j = 37
    c["iq"][:] = 0
    c["iq"][:, :, j] = 0x3F80
    bs, _, _ = run_oracle(c, scale=2.0)
    dec = H.e4m3_decode(c["cache"])
    sp, sh, st = c["strides"]
    for t in range(c["T"]):
        pos = c["pos"][t]
        for b in range(pos // 128 + 1):
            p = np.arange(b * 128, min(b * 128 + 128, pos + 1))
            pages = c["pt"][c["seq"][t], p // 64].astype(np.int64)
            vals = dec[pages * sp + (p % 64) * st + j]
            assert bs[0, t, b] == 2.0 * vals.max()


def test_selection_invariants(oracle_lib):
    c = small_case(seed=4, T=8, pos_hi=3000, max_pages=48)
    _, ids1, counts = run_oracle(c, scale=1.0)
    _, ids2, _ = run_oracle(c, scale=37.0)
    np.testing.assert_array_equal(ids1, ids2)                      # a positive scale does not reorder
    nvis = c["pos"] // 128 + 1
    np.testing.assert_array_equal(counts, np.minimum(16, nvis)[None, :].repeat(2, 0))
    for h in range(2):
        for t in range(8):
            sel = ids1[h, t][ids1[h, t] >= 0]
            assert len(set(sel.tolist())) == sel.size and np.all(sel <= c["pos"][t] // 128)


def test_padded_token_selects_nothing(oracle_lib):
    c = small_case(seed=5)
    c["seq"][2] = -1
    bs, ids, counts = run_oracle(c)
    assert np.all(bs[:, 2] == -np.inf) and np.all(ids[:, 2] == -1) and np.all(counts[:, 2] == 0)


def test_topk_ties_go_to_lower_index(oracle_lib):
    bs = np.array([[[1.0, 3.0, 3.0, -np.inf, 2.0, 3.0, np.nan, 2.0]]])
    ids, counts = oracle.index_topk(bs, 5)
    np.testing.assert_array_equal(ids[0, 0], [1, 2, 5, 4, 7])
    assert counts[0, 0] == 5
    ids, counts = oracle.index_topk(bs, 8)
    np.testing.assert_array_equal(ids[0, 0], [1, 2, 5, 4, 7, 0, -1, -1])
    assert counts[0, 0] == 6
