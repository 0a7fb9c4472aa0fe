"""The Python binding's tensor checks, on the CPU: every mismatch between the tensors and the counts a
wrapper hands to the library raises ValueError before the library is asked to launch anything.
The tensors here live on the CPU; a launching library entry point is replaced by one that fails the
test if reached, so a check that let a bad call through would show as that failure."""
import pytest
import torch

import paged_kv_cache_msa_amd as msa

LAUNCHING = {"msa_produce", "msa_rope_table", "msa_quantize", "msa_rms_scale", "msa_index_scores",
             "msa_index_topk", "msa_slots", "msa_produce_unfused", "msa_project", "msa_project_produce"}


class _NoLaunch:
    """The real library for host-only queries (workspace sizes, status text); launching entry points
    fail the test."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in LAUNCHING:
            def reached(*a, **k):
                raise AssertionError(f"{name} reached the library")
            return reached
        return getattr(self._real, name)


@pytest.fixture(autouse=True)
def no_launch(monkeypatch):
    real = msa.lib()
    monkeypatch.setattr(msa, "lib", lambda: _NoLaunch(real))


T, HQ, HKV, HIQ, HIK, PAGES, P = 8, 4, 1, 1, 1, 16, 64
W = (HQ + 2 * HKV + HIQ + HIK) * 128


def produce_args():
    i16 = torch.int16
    a = dict(
        x=torch.zeros((T, W), dtype=i16), positions=torch.zeros(T, dtype=torch.int32),
        seq_idx=torch.zeros(T, dtype=torch.int32), page_table=torch.zeros((T, 8), dtype=torch.int32),
        q_norm_weight=torch.zeros(128, dtype=i16), k_norm_weight=torch.zeros(128, dtype=i16),
        iq_norm_weight=torch.zeros(128, dtype=i16), ik_norm_weight=torch.zeros(128, dtype=i16),
        q_out=torch.zeros((T, HQ, 128), dtype=i16), iq_out=torch.zeros((T, HIQ, 128), dtype=i16),
        k_cache=torch.zeros((PAGES, HKV, P, 128), dtype=torch.uint8),
        v_cache=torch.zeros((PAGES, HKV, P, 128), dtype=torch.uint8),
        ik_cache=torch.zeros((PAGES, HIK, P, 128), dtype=torch.uint8),
        k_scale=torch.ones(1), v_scale=torch.ones(1), ik_scale=torch.ones(1),
        slots_out=torch.zeros(T, dtype=torch.int64))
    return a


def call_produce(a):
    a = dict(a)
    pos = [a.pop(k) for k in ("x", "positions", "seq_idx", "page_table", "q_norm_weight", "k_norm_weight",
                              "iq_norm_weight", "ik_norm_weight", "q_out", "iq_out", "k_cache", "v_cache",
                              "ik_cache")]
    return msa.msa_produce(*pos, **a)


MUTATIONS = {
    "x-float32": (lambda a: a.update(x=torch.zeros((T, W), dtype=torch.float32)), "x must have 2-byte"),
    "x-narrow": (lambda a: a.update(x=torch.zeros((T, W - 128), dtype=torch.int16)), "columns"),
    "x-column-stride": (lambda a: a.update(x=torch.zeros((W, T), dtype=torch.int16).t()), "unit last"),
    "positions-int64": (lambda a: a.update(positions=torch.zeros(T, dtype=torch.int64)), "positions must be"),
    "positions-short": (lambda a: a.update(positions=torch.zeros(T - 1, dtype=torch.int32)), "positions holds"),
    "seq_idx-short": (lambda a: a.update(seq_idx=torch.zeros(3, dtype=torch.int32)), "seq_idx holds"),
    "page_table-int64": (lambda a: a.update(page_table=torch.zeros((T, 8), dtype=torch.int64)), "page_table"),
    "page_table-1d": (lambda a: a.update(page_table=torch.zeros(8, dtype=torch.int32)), "page_table"),
    "q_out-rows": (lambda a: a.update(q_out=torch.zeros((T - 1, HQ, 128), dtype=torch.int16)), "q_out has"),
    "q_out-head_dim": (lambda a: a.update(q_out=torch.zeros((T, HQ, 64), dtype=torch.int16)), "q_out must be"),
    "q_out-strided": (lambda a: a.update(q_out=torch.zeros((T, HQ, 256), dtype=torch.int16)[:, :, :128]),
                      "contiguous"),
    "iq_out-float": (lambda a: a.update(iq_out=torch.zeros((T, HIQ, 128))), "iq_out must have 2-byte"),
    "weight-length": (lambda a: a.update(k_norm_weight=torch.zeros(64, dtype=torch.int16)), "k_norm_weight"),
    "weight-missing": (lambda a: a.update(q_norm_weight=None), "q_norm_weight is required"),
    "v-heads": (lambda a: a.update(v_cache=torch.zeros((PAGES, 2, P, 128), dtype=torch.uint8)), "same number"),
    "v-page-size": (lambda a: a.update(v_cache=torch.zeros((PAGES, HKV, 32, 128), dtype=torch.uint8)), "page size"),
    "ik-head_dim": (lambda a: a.update(ik_cache=torch.zeros((PAGES, HIK, P, 64), dtype=torch.uint8)), "head_dim"),
    "cache-pages": (lambda a: a.update(num_pages=PAGES + 1), "pages"),
    "cache-dim-stride": (lambda a: a.update(k_cache=torch.zeros((PAGES, HKV, 128, P), dtype=torch.uint8)
                                            .transpose(2, 3)), "unit head_dim"),
    "cache-4byte": (lambda a: a.update(k_cache=torch.zeros((PAGES, HKV, P, 128)),
                                       v_cache=torch.zeros((PAGES, HKV, P, 128))), "1 or 2-byte"),
    "fp8-no-scale": (lambda a: a.update(k_scale=None), "scale"),
    "fp8-scale-dtype": (lambda a: a.update(v_scale=torch.ones(1, dtype=torch.float64)), "scale"),
    "k-without-v": (lambda a: a.update(v_cache=None), "together"),
    "slots-int32": (lambda a: a.update(slots_out=torch.zeros(T, dtype=torch.int32)), "slots_out must be"),
    "slots-short": (lambda a: a.update(slots_out=torch.zeros(2, dtype=torch.int64)), "slots_out holds"),
    "x-too-many-heads": (lambda a: a.update(q_out=torch.zeros((T, HQ + 1, 128), dtype=torch.int16)), "columns"),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_produce_rejects_mismatch(name):
    a = produce_args()
    mutate, msg = MUTATIONS[name]
    mutate(a)
    with pytest.raises(ValueError, match=msg):
        call_produce(a)


def test_produce_consistent_cpu_tensors_stop_at_the_device_check():
    with pytest.raises(ValueError, match="CUDA tensor"):
        call_produce(produce_args())


def unfused_args():
    a = produce_args()
    a.pop("seq_idx")
    a.pop("page_table")
    a["slots"] = a.pop("slots_out")
    a["workspace"] = torch.zeros(msa.msa_produce_unfused_workspace_size(T, HKV, HIK), dtype=torch.uint8)
    return a


def call_unfused(a):
    a = dict(a)
    pos = [a.pop(k) for k in ("x", "positions", "slots", "q_norm_weight", "k_norm_weight", "iq_norm_weight",
                              "ik_norm_weight", "q_out", "iq_out", "k_cache", "v_cache", "ik_cache")]
    return msa.msa_produce_unfused(*pos, **a)


@pytest.mark.parametrize("mutate,msg", [
    (lambda a: a.update(workspace=torch.zeros(16, dtype=torch.uint8)), "workspace holds"),
    (lambda a: a.update(slots=torch.zeros(T, dtype=torch.int32)), "slots must be"),
    (lambda a: a.update(positions=torch.zeros(1, dtype=torch.int32)), "positions holds"),
    (lambda a: a.update(num_pages=PAGES * 2), "pages"),
    (lambda a: None, "CUDA tensor"),
], ids=["workspace-small", "slots-int32", "positions-short", "pages", "cpu"])
def test_unfused_rejects_mismatch(mutate, msg):
    a = unfused_args()
    mutate(a)
    with pytest.raises(ValueError, match=msg):
        call_unfused(a)


def test_index_scores_rejects_mismatch():
    iq = torch.zeros((T, 2, 128), dtype=torch.int16)
    pos = torch.zeros(T, dtype=torch.int32)
    pt = torch.zeros((T, 8), dtype=torch.int32)
    ik = torch.zeros((PAGES, 1, P, 128), dtype=torch.uint8)
    sc = torch.ones(1)
    good = torch.zeros((2, T, 4), dtype=torch.float64)
    with pytest.raises(ValueError, match="block_scores must be"):
        msa.msa_index_scores(iq, pos, pos, pt, ik, torch.zeros((1, T, 4), dtype=torch.float64), ik_scale=sc)
    with pytest.raises(ValueError, match="block_scores must be a torch.float64"):
        msa.msa_index_scores(iq, pos, pos, pt, ik, good.float(), ik_scale=sc)
    with pytest.raises(ValueError, match="scale"):
        msa.msa_index_scores(iq, pos, pos, pt, ik, good)
    with pytest.raises(ValueError, match="iq must be"):
        msa.msa_index_scores(iq[:, :, :64].contiguous(), pos, pos, pt, ik, good, ik_scale=sc)
    with pytest.raises(ValueError, match="CUDA tensor"):
        msa.msa_index_scores(iq, pos, pos, pt, ik, good, ik_scale=sc)


def test_index_topk_rejects_mismatch():
    bs = torch.zeros((2, T, 40), dtype=torch.float64)
    with pytest.raises(ValueError, match="block_ids holds"):
        msa.msa_index_topk(bs, torch.zeros((2, T - 1, 16), dtype=torch.int32))
    with pytest.raises(ValueError, match="int32"):
        msa.msa_index_topk(bs, torch.zeros((2, T, 16), dtype=torch.int64))
    with pytest.raises(ValueError, match="counts holds"):
        msa.msa_index_topk(bs, torch.zeros((2, T, 16), dtype=torch.int32), torch.zeros(3, dtype=torch.int32))


def test_step_entry_points_reject_mismatch():
    pos = torch.zeros(10, dtype=torch.int32)
    with pytest.raises(ValueError, match="cos_out holds"):
        msa.msa_rope_table(pos, torch.zeros((9, 64)), torch.zeros((10, 64)))
    with pytest.raises(ValueError, match="float32"):
        msa.msa_rope_table(pos, torch.zeros((10, 64), dtype=torch.float64), torch.zeros((10, 64)))
    with pytest.raises(ValueError, match="codes_out must have 1-byte"):
        msa.msa_quantize(torch.zeros(10), torch.zeros(10, dtype=torch.int16), msa.MSA_CACHE_FP8_E4M3, torch.ones(1))
    with pytest.raises(ValueError, match="codes_out holds"):
        msa.msa_quantize(torch.zeros(10), torch.zeros(9, dtype=torch.int16), msa.MSA_CACHE_BF16)
    with pytest.raises(ValueError, match="r_out is shorter"):
        msa.msa_rms_scale(torch.zeros(10, dtype=torch.float64), torch.zeros(9), 1e-6)
    with pytest.raises(ValueError, match="slots_out holds"):
        msa.msa_slots(pos, pos, torch.zeros((10, 4), dtype=torch.int32), torch.zeros(5, dtype=torch.int64),
                      page_size=64, num_pages=4)


def test_project_rejects_mismatch():
    h = torch.zeros((T, 256), dtype=torch.int16)
    w = torch.zeros((W, 256), dtype=torch.int16)
    with pytest.raises(ValueError, match="w has 128 columns"):
        msa.msa_project(h, w[:, :128], torch.zeros((T, W), dtype=torch.int16))
    with pytest.raises(ValueError, match="x_out must be at least"):
        msa.msa_project(h, w, torch.zeros((T, W - 128), dtype=torch.int16))
    with pytest.raises(ValueError, match="workspace"):
        msa.msa_project(h, w, torch.zeros((T, W), dtype=torch.int16), workspace=torch.zeros(8, dtype=torch.uint8))
    a = produce_args()
    cos = torch.zeros((T, 64))
    ws = torch.zeros(msa.msa_project_workspace_size(T, 256, W // 128), dtype=torch.uint8)
    args = (h, w, cos, cos, a["slots_out"], a["q_norm_weight"], a["k_norm_weight"], a["iq_norm_weight"],
            a["ik_norm_weight"], a["q_out"], a["iq_out"], a["k_cache"], a["v_cache"], a["ik_cache"])
    kw = dict(workspace=ws, k_scale=a["k_scale"], v_scale=a["v_scale"], ik_scale=a["ik_scale"])
    with pytest.raises(ValueError, match="w has .* rows"):
        msa.msa_project_produce(h, w[:-128], *args[2:], **kw)
    with pytest.raises(ValueError, match="rope_sin holds"):
        msa.msa_project_produce(*args[:3], cos[:-1], *args[4:], **kw)
    with pytest.raises(ValueError, match="CUDA tensor"):
        msa.msa_project_produce(*args, **kw)
