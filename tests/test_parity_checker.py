"""The GPU parity checker itself, on the CPU: it must catch a stray write anywhere outside the
oracle's written set (including a NaN code written where the sentinel, itself an E4M3 NaN, should
stay), and must accept exactly the oracle's storages.  Device results are stood in for by copies
of the oracle's own storages with mistakes planted in them."""
import numpy as np
import pytest

from paged_kv_cache_msa_amd import workloads as W
from tests import helpers as H
from tests.parity import code_diff, sentinel_code, storage_mismatches, written_elements, written_mask


@pytest.fixture(scope="module")
def tiny(oracle_lib):
    wl = W.ragged(40, seed=5, cache_dtypes=(W.FP8_E4M3, W.BF16, W.FP8_E4M3), pad_frac=0.2)
    res, st = H.oracle_caches(wl)
    return wl, res, st


def test_written_set_is_the_oracles(tiny):
    """The mask built from slots and strides covers exactly the elements the oracle changed (the
    workload's values never encode to the sentinel), and its size is tokens x heads x 128."""
    wl, res, st = tiny
    for spec, s in zip(wl.caches, st):
        mask = written_mask(spec, res["slots"], wl.page_size)
        changed = s.reshape(-1) != sentinel_code(spec.dtype)
        assert np.array_equal(mask, changed)
        n_valid = int(np.count_nonzero(res["slots"] >= 0))
        assert mask.sum() == n_valid * spec.heads * 128
        assert np.unique(written_elements(spec, res["slots"], wl.page_size)).size == mask.sum()


def test_accepts_the_oracles_storages(tiny):
    wl, res, st = tiny
    for spec, s in zip(wl.caches, st):
        mask = written_mask(spec, res["slots"], wl.page_size)
        assert storage_mismatches(s.copy(), s, mask, spec.dtype).size == 0


@pytest.mark.parametrize("stray", [0xFF, 0x7E, 0x00, 0x80])
def test_catches_a_stray_fp8_byte_outside_the_written_set(tiny, stray):
    """0xFF is the case a NaN-for-NaN comparison would miss: the sentinel 0x7F is a NaN code too."""
    wl, res, st = tiny
    spec, s = wl.caches[0], st[0]
    mask = written_mask(spec, res["slots"], wl.page_size)
    gpu = s.reshape(-1).copy()
    where = np.flatnonzero(~mask)[[0, 12345, -1]]
    gpu[where] = stray
    bad = storage_mismatches(gpu, s, mask, spec.dtype)
    assert np.array_equal(bad, np.sort(where))
    # the element-wise NaN leniency alone does not see it
    if stray == 0xFF:
        assert code_diff(gpu, s.reshape(-1), spec.dtype).size == 0


def test_catches_a_stray_bf16_element(tiny):
    wl, res, st = tiny
    spec, s = wl.caches[1], st[1]
    mask = written_mask(spec, res["slots"], wl.page_size)
    gpu = s.reshape(-1).copy()
    k = np.flatnonzero(~mask)[777]
    gpu[k] = 0xFFC0                                   # a NaN
    assert storage_mismatches(gpu, s, mask, spec.dtype).tolist() == [k]


def test_nan_leniency_only_inside_the_written_set(tiny):
    """Inside the written set, a device NaN of another sign or payload where the oracle wrote a NaN
    passes; a non-NaN there, or a changed finite code, fails."""
    wl, res, st = tiny
    spec, s = wl.caches[0], st[0]
    mask = written_mask(spec, res["slots"], wl.page_size)
    ref = s.reshape(-1).copy()
    k0, k1, k2 = np.flatnonzero(mask)[[3, 40, 99]]
    ref[k0] = 0x7F                                    # the oracle wrote +NaN here
    gpu = ref.copy()
    gpu[k0] = 0xFF                                    # the device wrote -NaN: accepted
    assert storage_mismatches(gpu, ref, mask, spec.dtype).size == 0
    gpu[k1] = ref[k1] ^ 0x01                          # a finite code off by one: caught
    gpu[k2] = 0x7F if ref[k2] != 0x7F else 0x00       # a NaN where the oracle has a number: caught
    assert storage_mismatches(gpu, ref, mask, spec.dtype).tolist() == sorted([k1, k2])
