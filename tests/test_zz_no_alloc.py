"""msa_project_produce_noalloc (the library's static per-GPU scratch in place of a caller workspace)
against msa_project_produce with a workspace, through the C ABI: the same kernels in the same order,
so every output (Q, index-Q, slots and every byte of the three cache storages) must be identical.
Two calls in a row, the second with a smaller batch (the scratch keeps the first call's partial
sums, which the second must not read), then a batch whose need exceeds the scratch (refused before
anything is launched) and a batch large enough to need none."""
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_msa_amd as msa
from paged_kv_cache_msa_amd import workloads as W

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 32 << 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msa.lib()


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def stage(wl, seed):
    """Device inputs of workload wl plus projection inputs, RoPE table and slots."""
    h, w = W.with_projection(wl, seed=seed)
    d = W.to_device(wl)
    cos = torch.empty((wl.T, 64), dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    msa.msa_rope_table(d.positions, cos, sin, wl.theta)
    msa.msa_slots(d.positions, d.seq_idx, d.page_table, d.slots, page_size=wl.page_size, num_pages=wl.num_pages)
    torch.cuda.synchronize()
    return d, dev16(h), dev16(w), cos, sin


def run(wl, d, h, w, cos, sin, noalloc):
    for st in d.storages:
        st.fill_(W.SENTINEL_BYTE if st.dtype == torch.uint8 else W.SENTINEL_BYTE * 0x0101)
    d.q_out.fill_(3)
    d.iq_out.fill_(3)
    kw = dict(k_scale=d.scales[0], v_scale=d.scales[1], ik_scale=d.scales[2], num_pages=wl.num_pages,
              rms_eps=wl.eps)
    args = (h, w, cos, sin, d.slots, *d.weights, d.q_out, d.iq_out, d.caches[0], d.caches[1], d.caches[2])
    if noalloc:
        msa.msa_project_produce_noalloc(*args, **kw)
    else:
        ws = torch.zeros(max(msa.msa_project_workspace_size(wl.T, h.shape[1], wl.W // 128), 256), dtype=torch.uint8,
                         device="cuda")
        msa.msa_project_produce(*args, workspace=ws, **kw)
    torch.cuda.synchronize()
    return d.q_out.clone(), d.iq_out.clone(), [s.clone() for s in d.storages]


def same(a, b, what):
    qa, ia, sa = a
    qb, ib, sb = b
    assert torch.equal(qa, qb), f"{what}: Q differs"
    assert torch.equal(ia, ib), f"{what}: index-Q differs"
    for x, y in zip(sa, sb):
        assert torch.equal(x, y), f"{what}: cache bytes differ"


def test_noalloc_matches_workspace_entry_point_twice_then_smaller():
    first = W.decode_batch64(layer=5)                       # 64 tokens: 5.9 MB of partial sums
    second = W.ragged(20, seed=44, pad_frac=0.1)            # 20 tokens after it, same scratch
    assert msa.msa_project_workspace_size(first.T, W.PROJECTION_HIDDEN, first.W // 128) <= SCRATCH_BYTES
    for wl, seed in ((first, 1), (second, 2)):
        say(f"[gpu] msa_project_produce_noalloc vs msa_project_produce: {wl.name}, T={wl.T}")
        staged = stage(wl, seed)
        ref = run(wl, *staged, noalloc=False)
        got = run(wl, *staged, noalloc=True)
        same(got, ref, wl.name)
        assert int((staged[0].q_out != 3).sum()) > 0


def test_noalloc_batch_beyond_the_scratch_is_refused():
    """1,024 tokens of 23 heads need 94 MB of partial sums: MSA_ERR_WORKSPACE, nothing launched."""
    wl = W.ragged(1024, seed=45, pad_frac=0.0)
    need = msa.msa_project_workspace_size(wl.T, W.PROJECTION_HIDDEN, wl.W // 128)
    assert need > SCRATCH_BYTES
    d, h, w, cos, sin = stage(wl, 3)
    d.q_out.fill_(3)
    torch.cuda.synchronize()
    with pytest.raises(msa.MsaError) as e:
        msa.msa_project_produce_noalloc(h, w, cos, sin, d.slots, *d.weights, d.q_out, d.iq_out, d.caches[0],
                                        d.caches[1], d.caches[2], k_scale=d.scales[0], v_scale=d.scales[1],
                                        ik_scale=d.scales[2], num_pages=wl.num_pages)
    torch.cuda.synchronize()
    assert e.value.status == 9
    assert int((d.q_out != 3).sum()) == 0
    for st in d.storages:
        assert int((st != W.SENTINEL_BYTE).sum()) == 0


def test_noalloc_large_batch_needs_no_scratch():
    """Above 1,024 tokens the tiled kernel runs and no scratch is used."""
    wl = W.ragged(1500, seed=46, pad_frac=0.1)
    say(f"[gpu] msa_project_produce_noalloc vs msa_project_produce: {wl.name}, T={wl.T}")
    staged = stage(wl, 4)
    ref = run(wl, *staged, noalloc=False)
    got = run(wl, *staged, noalloc=True)
    same(got, ref, wl.name)
