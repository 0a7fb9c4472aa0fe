"""C-ABI checks that need no GPU: the library loads, exports every entry point that
the headers under include/ declare, and rejects invalid arguments on the host before any launch
(so no call here reaches the device; every pointer below is a never-dereferenced address)."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_msa_amd as msa
from paged_kv_cache_msa_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", n) for n in sorted(os.listdir(os.path.join(ROOT, "include")))
           if n.endswith(".h")]

OK, NULLP, UNSUP, SHAPE, STRIDE, ALIGN, DTYPE, OVERFLOW, LAUNCH, WORKSPACE, NOT_DEVICE = range(11)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(msa.LIB_PATH):
        _build.build()
    return msa.lib()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) >= {"msa_produce", "msa_rope_table", "msa_quantize", "msa_rms_scale", "msa_status_string",
                          "msa_status_str", "msa_check_device_pointers", "msa_index_scores", "msa_index_topk",
                          "msa_index_scores_grouped",
                          "msa_slots", "msa_produce_unfused", "msa_produce_unfused_workspace_size"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(11):
        assert msa.string(code) and msa.string(code) != "unknown status"
        assert L.msa_status_str(code) == L.msa_status_string(code)
    assert msa.string(99) == "unknown status"


def test_device_pointer_check_without_a_device(L):
    """With no GPU every non-NULL pointer fails the residency check (reported with its index); NULL
    entries and an empty list pass; a negative count or a NULL array is an argument error."""
    assert msa.msa_check_device_pointers([]) == (OK, -1)
    assert msa.msa_check_device_pointers([None, None]) == (OK, -1)
    assert msa.msa_check_device_pointers([None, X, Q]) == (NOT_DEVICE, 1)
    assert msa.msa_check_device_pointers([X], [0]) == (OK, -1)          # an empty extent touches nothing
    assert L.msa_check_device_pointers(None, None, -1, None) == SHAPE
    assert L.msa_check_device_pointers(None, None, 2, None) == NULLP


def test_valid_call_without_a_device_launches_nothing(L):
    """Arguments that pass every host check, T > 0, no GPU: the operand check (the capture query, or
    the residency of the first operand) fails and the call returns before any launch."""
    assert call(L, T=64) in (LAUNCH, NOT_DEVICE)


# Fake, aligned device addresses: validation returns before anything could dereference them.
X, POS, SEQ, PT, W, Q, IQ, SLOTS, DATA, SCALE = (0x10000 * (i + 1) for i in range(10))


def view(data=DATA, sp=2 * 64 * 128, sh=64 * 128, st=128, heads=2, dtype=0, scale=SCALE):
    return msa.MsaCacheView(data, sp, sh, st, heads, dtype, scale)


def call(L, **kw):
    a = dict(x=X, xs=2944, T=64, D=128, hq=16, hkv=2, hiq=2, hik=1, pos=POS, seq=SEQ, pt=PT, pts=160, S=64,
             maxp=160, P=64, pages=10240, wq=W, wk=W, wiq=W, wik=W, eps=1e-6, theta=1e4, q=Q, iq=IQ,
             k=view(), v=view(), ik=view(sp=64 * 128, heads=1), slots=SLOTS, stream=None, force_T0=True)
    a.update(kw)
    T = 0 if a.pop("force_T0") and kw.get("T") is None else a["T"]
    ref = lambda v: None if v is None else ctypes.byref(v)
    return L.msa_produce(a["x"], a["xs"], T, a["D"], a["hq"], a["hkv"], a["hiq"], a["hik"], a["pos"], a["seq"],
                         a["pt"], a["pts"], a["S"], a["maxp"], a["P"], a["pages"], a["wq"], a["wk"], a["wiq"],
                         a["wik"], a["eps"], a["theta"], a["q"], a["iq"], ref(a["k"]), ref(a["v"]), ref(a["ik"]),
                         a["slots"], a["stream"])


def test_valid_arguments_with_zero_tokens_enqueue_nothing(L):
    assert call(L) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), UNSUP),
    (dict(T=-1), SHAPE),
    (dict(hq=-1), SHAPE),
    (dict(hq=0, hkv=0, hiq=0, hik=0, k=None, v=None, ik=None), SHAPE),
    (dict(P=0), SHAPE),
    (dict(pages=-1), SHAPE),
    (dict(eps=-1.0), SHAPE),
    (dict(theta=0.0), SHAPE),
    (dict(xs=2943), STRIDE),
    (dict(xs=2948), STRIDE),
    (dict(pts=100), STRIDE),
    (dict(wq=None), NULLP),
    (dict(wik=None), NULLP),
    (dict(k=None), NULLP),
    (dict(v=view(data=None)), NULLP),
    (dict(x=X + 8), ALIGN),
    (dict(q=Q + 2), ALIGN),
    (dict(slots=SLOTS + 4), ALIGN),
    (dict(wk=W + 2), ALIGN),
    (dict(k=view(data=DATA + 8)), ALIGN),
    (dict(k=view(heads=3)), SHAPE),
    (dict(ik=view(heads=2)), SHAPE),
    (dict(k=view(dtype=7)), DTYPE),
    (dict(k=view(scale=None)), DTYPE),
    (dict(k=view(st=64)), STRIDE),                       # token rows overlap within a head
    (dict(k=view(sh=128)), STRIDE),                      # heads overlap tokens
    (dict(k=view(sp=64 * 128)), STRIDE),                 # pages overlap heads
    (dict(k=view(st=132)), STRIDE),                      # not a multiple of 8 elements
    (dict(k=view(sp=-16384)), STRIDE),
    (dict(pages=1 << 50), OVERFLOW),
])
def test_rejects_invalid_arguments(L, kw, status):
    assert call(L, **kw) == status


def test_bf16_cache_needs_no_scale(L):
    assert call(L, k=view(dtype=1, scale=None), v=view(dtype=1, scale=None)) == OK


def test_permuted_nhd_storage_view_is_accepted(L):
    """An NHD allocation [pages, tokens, heads, D] seen as an HND view is a legal strided layout."""
    nhd = view(sp=64 * 2 * 128, sh=128, st=2 * 128)
    assert call(L, k=nhd, v=nhd) == OK


def test_padded_head_stride_view_is_accepted(L):
    padded = view(sp=2 * 65 * 128, sh=65 * 128, st=128)
    assert call(L, k=padded, v=padded) == OK


def test_index_k_optional(L):
    assert call(L, hik=0, wik=None, ik=None, xs=2816) == OK


def test_step_entry_points_validate(L):
    assert L.msa_rope_table(POS, 10, 1e4, 64, X, Q, None) == UNSUP
    assert L.msa_rope_table(POS, -1, 1e4, 128, X, Q, None) == SHAPE
    assert L.msa_rope_table(None, 10, 1e4, 128, X, Q, None) == NULLP
    assert L.msa_rope_table(POS, 0, 1e4, 128, None, None, None) == OK
    assert L.msa_quantize(X, 10, 3, SCALE, Q, None) == DTYPE
    assert L.msa_quantize(X, 10, 0, None, Q, None) == DTYPE
    assert L.msa_quantize(X + 2, 10, 0, SCALE, Q, None) == ALIGN
    assert L.msa_quantize(X, 0, 0, SCALE, Q, None) == OK
    assert L.msa_rms_scale(X, 10, 127, 1e-6, Q, None) == UNSUP
    assert L.msa_rms_scale(X + 4, 10, 128, 1e-6, Q, None) == ALIGN
    assert L.msa_rms_scale(X, 10, 128, -1.0, Q, None) == SHAPE


def test_python_binding_raises_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(msa, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(msa, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        msa.lib()


def _has_gpu():
    import torch
    return torch.cuda.device_count() > 0


@pytest.mark.skipif(_has_gpu(), reason="fake addresses with T > 0 are only exercised where no device exists")
@pytest.mark.parametrize("kw", [dict(x=None), dict(pos=None), dict(seq=None), dict(q=None), dict(iq=None),
                                dict(pt=None)])
def test_rejects_null_inputs_with_tokens(L, kw):
    assert call(L, T=64, **kw) == NULLP


def test_index_entry_points_validate(L):
    ik = view(sp=64 * 128, heads=1)
    ref = ctypes.byref
    # head_dim, negative counts, group mismatch, block size, null cache, overflow of block starts
    assert L.msa_index_scores(Q, 64, 64, 2, POS, SEQ, PT, 160, 64, 160, 64, 10240, ref(ik), 128, 72, SLOTS, None) == UNSUP
    assert L.msa_index_scores(Q, -1, 128, 2, POS, SEQ, PT, 160, 64, 160, 64, 10240, ref(ik), 128, 72, SLOTS, None) == SHAPE
    assert L.msa_index_scores(Q, 0, 128, 3, POS, SEQ, PT, 160, 64, 160, 64, 10240, ref(view(sp=2 * 64 * 128)), 128, 72,
                              SLOTS, None) == SHAPE
    assert L.msa_index_scores(Q, 0, 128, 2, POS, SEQ, PT, 160, 64, 160, 64, 10240, ref(ik), 0, 72, SLOTS, None) == SHAPE
    assert L.msa_index_scores(Q, 0, 128, 2, POS, SEQ, PT, 160, 64, 160, 64, 10240, None, 128, 72, SLOTS, None) == NULLP
    assert L.msa_index_scores(Q, 0, 128, 2, POS, SEQ, PT, 160, 64, 160, 64, 10240, ref(ik), 1 << 20, 1 << 12, SLOTS,
                              None) == SHAPE
    assert L.msa_index_scores(Q + 8, 0, 128, 2, POS, SEQ, PT, 160, 64, 160, 64, 10240, ref(ik), 128, 72, SLOTS, None) == ALIGN
    assert L.msa_index_scores(Q, 0, 128, 2, POS, SEQ, PT, 160, 64, 160, 64, 10240, ref(ik), 128, 72, SLOTS, None) == OK
    # the grouped entry point: the same checks first, then its group size (1 ..= 8)
    G = L.msa_index_scores_grouped
    assert G(Q, 64, 64, 2, POS, SEQ, PT, 160, 64, 160, 64, 10240, ref(ik), 128, 72, 4, SLOTS, None) == UNSUP
    assert G(Q, 0, 128, 3, POS, SEQ, PT, 160, 64, 160, 64, 10240, ref(view(sp=2 * 64 * 128)), 128, 72, 4, SLOTS,
             None) == SHAPE
    assert G(Q + 8, 0, 128, 2, POS, SEQ, PT, 160, 64, 160, 64, 10240, ref(ik), 128, 72, 4, SLOTS, None) == ALIGN
    for g in (0, 9, -1):
        assert G(Q, 0, 128, 2, POS, SEQ, PT, 160, 64, 160, 64, 10240, ref(ik), 128, 72, g, SLOTS, None) == SHAPE
    for g in (1, 4, 8):
        assert G(Q, 0, 128, 2, POS, SEQ, PT, 160, 64, 160, 64, 10240, ref(ik), 128, 72, g, SLOTS, None) == OK
    assert L.msa_index_topk(SLOTS, 10, 72, 0, Q, None, None) == SHAPE
    assert L.msa_index_topk(SLOTS, 10, 72, 65, Q, None, None) == SHAPE
    assert L.msa_index_topk(SLOTS, 10, 5000, 16, Q, None, None) == SHAPE
    assert L.msa_index_topk(SLOTS + 4, 10, 72, 16, Q, None, None) == ALIGN
    assert L.msa_index_topk(SLOTS, 0, 72, 16, Q, None, None) == OK


# ------------------------------------------------------------------ unfused path

WS = 0x200000


def call_unfused(L, **kw):
    a = dict(x=X, xs=2944, T=0, D=128, hq=16, hkv=2, hiq=2, hik=1, pos=POS, slots=SLOTS, P=64, pages=10240,
             wq=W, wk=W, wiq=W, wik=W, eps=1e-6, theta=1e4, q=Q, iq=IQ, k=view(), v=view(),
             ik=view(sp=64 * 128, heads=1), ws=WS, wsb=1 << 30, stream=None)
    a.update(kw)
    ref = lambda v: None if v is None else ctypes.byref(v)
    return L.msa_produce_unfused(a["x"], a["xs"], a["T"], a["D"], a["hq"], a["hkv"], a["hiq"], a["hik"], a["pos"],
                                 a["slots"], a["P"], a["pages"], a["wq"], a["wk"], a["wiq"], a["wik"], a["eps"],
                                 a["theta"], a["q"], a["iq"], ref(a["k"]), ref(a["v"]), ref(a["ik"]), a["ws"],
                                 a["wsb"], a["stream"])


def test_unfused_workspace_size(L):
    n = ctypes.c_uint64(0)
    assert L.msa_produce_unfused_workspace_size(64, 2, 1, ctypes.byref(n)) == OK
    # binary32 K (64 x 2 x 128) and index-K (64 x 1 x 128) rows, nine int64 [64] arrays, 256-B regions
    assert n.value == 64 * 2 * 128 * 4 + 64 * 1 * 128 * 4 + 9 * 512
    assert L.msa_produce_unfused_workspace_size(0, 2, 1, ctypes.byref(n)) == OK and n.value == 0
    assert L.msa_produce_unfused_workspace_size(-1, 2, 1, ctypes.byref(n)) == SHAPE
    assert L.msa_produce_unfused_workspace_size(1, 2, 1, None) == NULLP


@pytest.mark.parametrize("layout", [
    dict(st=132, sh=64 * 132, sp=2 * 64 * 132),     # token stride not a multiple of 8 elements
    dict(sp=2 * 65 * 128 + 1, sh=65 * 128 + 3),     # odd page and head strides
    dict(data=DATA + 1),                            # fp8 base aligned to its 1-byte element only
])
def test_unfused_takes_layouts_the_fused_kernel_rejects(L, layout):
    k = view(**layout)
    assert call(L, k=k) in (STRIDE, ALIGN)
    assert call_unfused(L, k=k) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), UNSUP),
    (dict(T=-1), SHAPE),
    (dict(P=0), SHAPE),
    (dict(xs=2948), STRIDE),
    (dict(k=view(st=64)), STRIDE),                  # overlapping rows are still rejected
    (dict(k=view(data=DATA + 1, dtype=1, scale=None)), ALIGN),   # bf16 base must be 2-byte aligned
    (dict(k=view(scale=None)), DTYPE),
    (dict(wk=None), NULLP),
    (dict(T=64, slots=None), NULLP),
    (dict(T=64, ws=None), WORKSPACE),
    (dict(T=64, ws=WS + 64), WORKSPACE),
    (dict(T=64, wsb=1000), WORKSPACE),
    (dict(pages=1 << 50), OVERFLOW),
])
def test_unfused_rejects_invalid_arguments(L, kw, status):
    assert call_unfused(L, **kw) == status


def test_slots_entry_point_validates(L):
    assert L.msa_slots(POS, SEQ, 0, PT, 160, 64, 160, 64, 10240, SLOTS, None) == OK
    assert L.msa_slots(POS, SEQ, -1, PT, 160, 64, 160, 64, 10240, SLOTS, None) == SHAPE
    assert L.msa_slots(POS, SEQ, 4, PT, 100, 64, 160, 64, 10240, SLOTS, None) == STRIDE
    assert L.msa_slots(POS, SEQ, 4, PT, 160, 64, 160, 0, 10240, SLOTS, None) == SHAPE
    assert L.msa_slots(POS, SEQ, 4, PT, 160, 64, 160, 64, 10240, None, None) == NULLP
    assert L.msa_slots(POS, SEQ, 4, PT, 160, 64, 160, 64, 10240, SLOTS + 4, None) == ALIGN


# ------------------------------------------------------------------ projection

HID, WMAT, XOUT, COS, SIN = (0x200000 + 0x10000 * i for i in range(5))


def test_project_workspace_size(L):
    n = ctypes.c_uint64(0)
    by = ctypes.byref(n)
    assert L.msa_project_workspace_size(64, 3072, 23, by) == OK
    # decode batch 64 at hidden 3072: a 256-byte header (the error word), then 8 K slices of 384 columns
    # per head with 8,192 binary32 partial sums each
    assert n.value == 256 + 23 * 8 * 8192 * 4
    assert L.msa_project_workspace_size(1024, 3072, 23, by) == OK and n.value == 256 + 16 * 23 * 8 * 8192 * 4
    # at most 63 K slices of 384 columns per (head, chunk) on the split-K path; the tiled path has no limit
    assert L.msa_project_workspace_size(64, 63 * 384, 23, by) == OK
    assert L.msa_project_workspace_size(64, 63 * 384 + 64, 23, by) == SHAPE
    assert L.msa_project_workspace_size(1025, 63 * 384 + 64, 23, by) == OK and n.value == 0
    assert L.msa_project_workspace_size(1025, 3072, 23, by) == OK and n.value == 0   # the tiled kernel needs none
    assert L.msa_project_workspace_size(0, 3072, 23, by) == OK and n.value == 0
    assert L.msa_project_workspace_size(64, 100, 23, by) == SHAPE
    assert L.msa_project_workspace_size(-1, 3072, 23, by) == SHAPE
    assert L.msa_project_workspace_size(64, 3072, 0, by) == SHAPE
    assert L.msa_project_workspace_size(64, 3072, 4097, by) == SHAPE
    assert L.msa_project_workspace_size(64, 3072, 23, None) == NULLP


def call_project(L, **kw):
    a = dict(h=HID, hs=3072, T=0, K=3072, w=WMAT, ws=3072, N=2944, x=XOUT, xs=2944, wsp=WS, wsb=1 << 30, stream=None)
    a.update(kw)
    return L.msa_project(a["h"], a["hs"], a["T"], a["K"], a["w"], a["ws"], a["N"], a["x"], a["xs"], a["wsp"],
                         a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(), OK),
    (dict(K=100), SHAPE),
    (dict(K=0), SHAPE),
    (dict(N=100), SHAPE),
    (dict(N=4097 * 128), SHAPE),
    (dict(T=-1), SHAPE),
    (dict(hs=3000), STRIDE),
    (dict(hs=3076), STRIDE),
    (dict(ws=3071), STRIDE),
    (dict(xs=2940), STRIDE),
    (dict(xs=2948), STRIDE),
    (dict(T=1025, hs=1 << 22), STRIDE),             # the tiled kernel's 32-bit row offsets
    (dict(T=1025, ws=1 << 22), STRIDE),
    (dict(T=64, h=None), NULLP),
    (dict(T=64, x=None), NULLP),
    (dict(h=HID + 8), ALIGN),
    (dict(x=XOUT + 8), ALIGN),
    (dict(T=1 << 24, hs=1 << 40), OVERFLOW),
    (dict(T=64, wsp=None), WORKSPACE),
    (dict(T=64, wsp=WS + 64), WORKSPACE),
    (dict(T=64, wsb=1000), WORKSPACE),
])
def test_project_rejects_invalid_arguments(L, kw, status):
    assert call_project(L, **kw) == status


def call_project_produce(L, **kw):
    a = dict(h=HID, hs=3072, T=0, K=3072, w=WMAT, ws=3072, D=128, hq=16, hkv=2, hiq=2, hik=1, cos=COS, sin=SIN,
             slots=SLOTS, P=64, pages=10240, wq=W, wk=W, wiq=W, wik=W, eps=1e-6, q=Q, iq=IQ, k=view(), v=view(),
             ik=view(sp=64 * 128, heads=1), wsp=WS, wsb=1 << 30, stream=None)
    a.update(kw)
    ref = lambda v: None if v is None else ctypes.byref(v)
    return L.msa_project_produce(a["h"], a["hs"], a["T"], a["K"], a["w"], a["ws"], a["D"], a["hq"], a["hkv"],
                                 a["hiq"], a["hik"], a["cos"], a["sin"], a["slots"], a["P"], a["pages"], a["wq"],
                                 a["wk"], a["wiq"], a["wik"], a["eps"], a["q"], a["iq"], ref(a["k"]), ref(a["v"]),
                                 ref(a["ik"]), a["wsp"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(), OK),
    (dict(hik=0, ik=None, wik=None), OK),           # index-K is optional
    (dict(D=64), UNSUP),
    (dict(hq=-1), SHAPE),
    (dict(hq=0, hkv=0, hiq=0, hik=0), SHAPE),
    (dict(P=0), SHAPE),
    (dict(eps=-1.0), SHAPE),
    (dict(K=100), SHAPE),
    (dict(hs=3076), STRIDE),
    (dict(T=1025, hs=1 << 22), STRIDE),
    (dict(T=64, cos=None), NULLP),
    (dict(T=64, slots=None), NULLP),
    (dict(T=64, q=None), NULLP),
    (dict(wk=None), NULLP),
    (dict(cos=COS + 4), ALIGN),
    (dict(slots=SLOTS + 4), ALIGN),
    (dict(q=Q + 8), ALIGN),
    (dict(k=view(scale=None)), DTYPE),
    (dict(k=view(st=64)), STRIDE),                  # overlapping rows
    (dict(ik=view(sp=64 * 128, heads=2)), SHAPE),   # head count of the view differs from the call's
    (dict(T=64, wsp=None), WORKSPACE),
    (dict(T=64, wsb=1000), WORKSPACE),
])
def test_project_produce_rejects_invalid_arguments(L, kw, status):
    assert call_project_produce(L, **kw) == status
