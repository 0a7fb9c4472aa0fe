"""Benchmark of the MSA fused producer on one MI355X.

The metric has two parts, measured on two workloads:
  * producer HBM GB/s (% of peak): the 65,536-token prefill chunk (8 sequences x 8192 tokens, local
    heads Q=16 / KV=2 / index-Q=2 / index-K=1, head_dim 128, fp8 e4m3 HND caches in a 12,000-page
    pool).  A step is one msa_produce launch over the whole chunk.  The prefill runs first, on input
    staged before any device work: at least `--warmup` untimed steps, continued until `--warm-ms`
    of device time has run (the engine clock needs tens of milliseconds of load to settle), then
    `--steps` timed ones, with HIP events on the launch stream, alternating two input sets.
    `value`, `ms_per_step` and `roofline` are this kernel's.
  * us per layer call at decode batch 64: 64 sequences x 1 token at positions 7000..9199, the same
    heads, fp8 caches of 10,240 pages per layer; one step = every position advanced by one in place,
    then 60 layer calls (each with its own input row, norm weights, scales and caches), captured
    once in a HIP graph and replayed, so every replay writes new slots.  Reported as
    `us_per_layer_call` (step time / 60) and `us_per_decode_step`, with their own roofline under
    `decode`.
Also reported: speculative-decoding verify rows, 64 sequences x (1 + 3) tokens through the same
60-layer graph (`verify`); the indexer at decode batch 64 (`indexer`); the same decode step and prefill chunk
through the unfused path (`unfused`: 14 launches per layer instead of one, identical bytes); and
the packed projection of hidden states (hidden 3072) alone and with the producer as its epilogue,
against torch.mm (hipBLASLt) followed by the producer (`projection`).
Inputs are resident in HBM before every timed region.  `cpu_baseline` is the CPU oracle on a
bounded sample of the prefill workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--warm-ms MS] [--layers 60] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "producer HBM GB/s (% of peak) + µs per layer call at decode batch 64"
# sources the fused producer kernel is compiled from (the counters are tied to their digest)
KERNEL_SRCS = [os.path.join(ROOT, "paged_kv_cache_msa_amd", "csrc", n)
               for n in ("msa_produce.hip", "msa_device.h", "msa_common.h")]
COUNTERS = os.path.join(ROOT, "profiles", "produce_kernel_hbm_counters.json")
# the indexer's kernels and their counter record
INDEX_SRCS = [os.path.join(ROOT, "paged_kv_cache_msa_amd", "csrc", n) for n in ("msa_index.hip", "msa_common.h")]
INDEX_COUNTERS = os.path.join(ROOT, "profiles", "index_kernels_hbm_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_digest(srcs=None) -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS if srcs is None else srcs:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(workload_key: str, path=None, srcs=None):
    """Measured HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel
    calibration) if they were taken on the current kernel source; else None."""
    try:
        with open(COUNTERS if path is None else path) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_sha256_16") != (kernel_digest() if srcs is None else kernel_digest(srcs)):
        return None
    return c.get("bytes_per_launch", {}).get(workload_key)


def call(msa, wl, d, stream=None):
    msa.msa_produce(d.x, d.positions, d.seq_idx, d.page_table, *d.weights, d.q_out, d.iq_out,
                    d.caches[0], d.caches[1], d.caches[2], k_scale=d.scales[0], v_scale=d.scales[1],
                    ik_scale=d.scales[2], num_pages=wl.num_pages, rms_eps=wl.eps, rope_theta=wl.theta,
                    slots_out=d.slots, stream=stream)


def bench_decode(msa, W, torch, layers, steps, warmup):
    """The decode step: every replay first advances each sequence's position by one in place (one
    small elementwise node), then runs the `layers` producer launches, which read the new positions
    from the same device buffers: consecutive steps write new slots and cross page boundaries, as a
    serving loop that updates its metadata in place and replays the captured step does."""
    log(f"[bench] staging {layers} decode-64 layers")
    wls = [W.decode_batch64(layer=i) for i in range(layers)]
    devs = [W.to_device(wl) for wl in wls]
    # share the metadata buffers across layers (one batch, many layers)
    for d in devs[1:]:
        d.positions, d.seq_idx, d.page_table = devs[0].positions, devs[0].seq_idx, devs[0].page_table
    # the page table covers 160 pages (10,240 positions) per sequence: room for every replay
    replays = 1 + warmup + steps
    assert int(wls[0].positions.max()) + replays < wls[0].max_pages * wls[0].page_size
    pos = devs[0].positions
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()

    def step():
        pos.add_(1)
        for wl, d in zip(wls, devs):
            call(msa, wl, d)

    with torch.cuda.stream(s):
        for wl, d in zip(wls, devs):      # one eager pass before capture
            call(msa, wl, d)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    log(f"[bench] decode graph captured (position update + {layers} launches); warmup {warmup}, timing {steps} steps")
    with torch.cuda.stream(s):
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(steps):
            g.replay()
        e1.record(s)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    bytes_per_call = wls[0].algorithmic_bytes()
    return dict(ms_total=ms, ms_per_step=ms / steps, bytes_per_call=bytes_per_call,
                bytes_per_step=bytes_per_call * layers, launches=steps * layers, wls=wls, devs=devs)


def bench_verify(msa, W, torch, np, wls, devs, steps, warmup, draft_len=3):
    """Speculative-decoding verify rows through the same producer: 64 sequences x (1 + draft_len)
    consecutive tokens (windows that cross page boundaries), one call per layer for the decode step's
    layers, all captured in one HIP graph.  The caches, norm weights and scales of the decode layers
    are reused (same pool geometry); each layer gets its own input rows and outputs."""
    import dataclasses
    vw = W.verify_window(draft_len=draft_len)
    T = vw.T
    pos = torch.from_numpy(vw.positions).cuda()
    seq = torch.from_numpy(vw.seq_idx).cuda()
    pt = torch.from_numpy(np.ascontiguousarray(vw.page_table)).cuda()
    slots = torch.empty(T, dtype=torch.int64, device="cuda")
    rng = np.random.default_rng(17)
    vdevs = []
    for wl, d in zip(wls, devs):
        x = torch.from_numpy(W.to_bf16_bits(rng.standard_normal((T, wl.W), dtype=np.float32)).view(np.int16)).cuda()
        q = torch.empty((T, wl.hq, wl.head_dim), dtype=torch.int16, device="cuda")
        iq = torch.empty((T, wl.hiq, wl.head_dim), dtype=torch.int16, device="cuda")
        vdevs.append(dataclasses.replace(d, x=x, positions=pos, seq_idx=seq, page_table=pt, q_out=q, iq_out=iq,
                                         slots=slots))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        for wl, d in zip(wls, vdevs):
            call(msa, wl, d)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for wl, d in zip(wls, vdevs):
                call(msa, wl, d)
    torch.cuda.synchronize()
    log(f"[bench] verify-window graph captured ({len(wls)} launches of {T} tokens)")
    with torch.cuda.stream(s):
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(steps):
            g.replay()
        e1.record(s)
        torch.cuda.synchronize()
    us_step = e0.elapsed_time(e1) * 1000 / steps
    bytes_per_call = vw.algorithmic_bytes()      # the same heads and fp8 caches as the decode layers
    us_call = us_step / len(wls)
    return {"workload": f"{vw.name}; the decode layers' caches", "tokens": T, "draft_len": draft_len,
            "layers": len(wls), "steps": steps, "warmup": warmup, "us_per_layer_call": us_call,
            "us_per_step": us_step, "algorithmic_bytes_per_layer_call": bytes_per_call,
            "algorithmic_gbs": bytes_per_call / (us_call * 1e-6) / 1e9}


def unfused_call(msa, wl, d, slots, ws, stream=None):
    msa.msa_produce_unfused(d.x, d.positions, slots, *d.weights, d.q_out, d.iq_out, d.caches[0], d.caches[1],
                            d.caches[2], workspace=ws, k_scale=d.scales[0], v_scale=d.scales[1],
                            ik_scale=d.scales[2], num_pages=wl.num_pages, rms_eps=wl.eps, rope_theta=wl.theta,
                            stream=stream)


def unfused_launches(wl):
    """Launches of one msa_produce_unfused call: two norm/RoPE producers plus four per cache."""
    prods = int(wl.hq + wl.hkv > 0) + int(wl.hiq + wl.hik > 0)
    return prods + 4 * (2 * int(wl.hkv > 0) + int(wl.hik > 0))


def bench_decode_unfused(msa, torch, wls, devs, steps, warmup):
    """The same decode step through the unfused path: one msa_slots launch, then per layer the main
    and index norm/RoPE producers and division, remainder, index cast and scatter for each of K, V
    and index-K, all captured in one HIP graph.  One workspace serves every layer (stream order)."""
    ws = torch.empty(msa.msa_produce_unfused_workspace_size(wls[0].T, wls[0].hkv, wls[0].hik), dtype=torch.uint8,
                     device="cuda")
    slots = devs[0].slots
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()

    def step():
        msa.msa_slots(devs[0].positions, devs[0].seq_idx, devs[0].page_table, slots, page_size=wls[0].page_size,
                      num_pages=wls[0].num_pages)
        for wl, d in zip(wls, devs):
            unfused_call(msa, wl, d, slots, ws)

    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    launches = 1 + sum(unfused_launches(wl) for wl in wls)
    log(f"[bench] unfused decode graph captured ({launches} launches); warmup {warmup}, timing {steps} steps")
    with torch.cuda.stream(s):
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(steps):
            g.replay()
        e1.record(s)
        torch.cuda.synchronize()
    us_step = e0.elapsed_time(e1) * 1000 / steps
    return dict(us_per_step=us_step, us_per_layer_call=us_step / len(wls), launches_per_step=launches,
                steps=steps, warmup=warmup)


def copy_reference(torch, nbytes: int, reps: int = 20):
    """The runtime's device-to-device copy moving the same number of bytes as one prefill launch
    (half read, half written), timed like the prefill: context for the producer's bandwidth."""
    n = nbytes // 2 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000 / reps
    del src, dst
    return dict(bytes=2 * n * 4, us=us, gbs=2 * n * 4 / (us * 1e-6) / 1e9)


def stage_prefill(W, torch):
    log("[bench] staging the 65,536-token prefill chunk (two input sets)")
    sets = [W.prefill_65536(variant=v) for v in range(2)]
    devs = [W.to_device(wl) for wl in sets]
    torch.cuda.synchronize()
    return sets, devs


def bench_prefill(msa, W, torch, iters, warmup, warm_ms, staged, unfused_iters=0):
    """`warmup` launches, then more back to back until at least `warm_ms` of device time has run (the
    engine clock settles only after tens of milliseconds of load), then `iters` timed launches."""
    sets, devs = staged
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warm_launches, warm_elapsed = 0, 0.0
    e0.record(s)
    while warm_launches < warmup or warm_elapsed < warm_ms:
        for _ in range(50):
            call(msa, sets[warm_launches % 2], devs[warm_launches % 2])
            warm_launches += 1
        e1.record(s)
        e1.synchronize()
        warm_elapsed = e0.elapsed_time(e1)
    log(f"[bench] prefill warm: {warm_launches} launches, {warm_elapsed:.1f} ms")
    e0.record(s)
    for i in range(iters):
        call(msa, sets[i % 2], devs[i % 2])
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    b = sets[0].algorithmic_bytes()
    us = ms * 1000 / iters
    gbs = b / (us * 1e-6) / 1e9
    out = dict(us_per_call=us, bytes=b, gbs=gbs, launches=iters, warm_launches=warm_launches, warm_ms=warm_elapsed)
    if unfused_iters:
        # the same chunk through the unfused path (slots from the fused calls above)
        ws = torch.empty(msa.msa_produce_unfused_workspace_size(sets[0].T, sets[0].hkv, sets[0].hik),
                         dtype=torch.uint8, device="cuda")
        for i in range(10):
            unfused_call(msa, sets[i % 2], devs[i % 2], devs[i % 2].slots, ws)
        torch.cuda.synchronize()
        e0.record(s)
        for i in range(unfused_iters):
            unfused_call(msa, sets[i % 2], devs[i % 2], devs[i % 2].slots, ws)
        e1.record(s)
        torch.cuda.synchronize()
        out["unfused_us_per_call"] = e0.elapsed_time(e1) * 1000 / unfused_iters
        out["unfused_launches_per_call"] = unfused_launches(sets[0])
        del ws
    del devs
    torch.cuda.empty_cache()
    return out


def _indexer_graph_us(msa, torch, score, topk, reps, per_graph=20):
    """us per (score + top-k) call: `per_graph` calls captured in one graph, `reps` replays timed
    after 5 warm ones."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        score()
        topk()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for _ in range(per_graph):
                score()
                topk()
        for _ in range(5):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000 / (reps * per_graph)


def _indexer_inputs(msa, W, torch, np, wl):
    fill = W.index_cache_fill(wl)
    iq = torch.from_numpy(W.index_queries(wl.T, wl.hiq).view(np.int16)).cuda()
    nb = W.index_blocks(wl)
    c = wl.caches[2]
    store = torch.from_numpy(fill).cuda()
    view = store.as_strided((wl.num_pages, c.heads, wl.page_size, 128), (*c.strides, 1))
    scale = torch.tensor([c.scale], dtype=torch.float32, device="cuda")
    pos = torch.from_numpy(wl.positions).cuda()
    seq = torch.from_numpy(wl.seq_idx).cuda()
    pt = torch.from_numpy(np.ascontiguousarray(wl.page_table)).cuda()
    bs = torch.empty((wl.hiq, wl.T, nb), dtype=torch.float64, device="cuda")
    ids = torch.empty((wl.hiq, wl.T, 16), dtype=torch.int32, device="cuda")
    cnt = torch.empty((wl.hiq, wl.T), dtype=torch.int32, device="cuda")
    return dict(store=store, iq=iq, nb=nb, view=view, scale=scale, pos=pos, seq=seq, pt=pt, bs=bs, ids=ids, cnt=cnt)


def bench_indexer(msa, W, torch, np, reps):
    """Indexer at decode batch 64 (positions 7000..9199, about 8k keys per sequence in a pre-populated
    fp8 index-K cache): msa_index_scores + msa_index_topk (top 16 of 128-token blocks), 20 calls per
    captured graph, `reps` graph replays timed after 5 warm ones."""
    wl = W.decode_batch64()
    d = _indexer_inputs(msa, W, torch, np, wl)
    nb = d["nb"]
    us = _indexer_graph_us(
        msa, torch,
        lambda: msa.msa_index_scores(d["iq"], d["pos"], d["seq"], d["pt"], d["view"], d["bs"], ik_scale=d["scale"],
                                     num_pages=wl.num_pages),
        lambda: msa.msa_index_topk(d["bs"], d["ids"], d["cnt"]), reps)
    keys = int((wl.positions.astype(np.int64) + 1).sum())
    # keys (128 B each, shared by both index-Q heads) + index-Q rows + token metadata + one page-table
    # entry per 64 keys + the block-score table written and read back + the selected ids
    b = (keys * 128 + wl.T * wl.hiq * 256 + wl.T * 8 + keys // 64 * 4 + 2 * wl.hiq * wl.T * nb * 8
         + wl.hiq * wl.T * (16 * 4 + 4))
    gbs = b / (us * 1e-6) / 1e9
    return dict(workload=f"decode batch 64 indexer: {keys} visible fp8 index-K keys, 2 index-Q heads, "
                         f"{nb} blocks of 128 tokens, top 16",
                us_per_call=us, algorithmic_bytes_per_call=b,
                roofline=dict(bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s", frac=gbs / HBM_PEAK_GBS,
                              traffic=counter_traffic("decode_64_indexer_call", INDEX_COUNTERS, INDEX_SRCS),
                              kernel="index_scores_rs_kernel<2, false> + index_topk_rank_kernel"))


def bench_indexer_verify(msa, W, torch, np, reps, draft_len=3):
    """Indexer on speculative-decoding verify windows (64 sequences x (1 + draft_len) consecutive
    tokens, positions 7000..9200): msa_index_scores (keys loaded per token) against
    msa_index_scores_grouped with one window per group (keys loaded once per window), each followed by
    msa_index_topk, 20 calls per captured graph."""
    wl = W.verify_window(draft_len=draft_len)
    L = 1 + draft_len
    d = _indexer_inputs(msa, W, torch, np, wl)
    nb = d["nb"]
    out = {"workload": f"verify windows: 64 sequences x {L} tokens, 2 index-Q heads, {nb} blocks of 128 tokens, "
                       f"top 16", "tokens": wl.T}
    topk = lambda: msa.msa_index_topk(d["bs"], d["ids"], d["cnt"])
    for name, group in (("per_token", 1), ("grouped", L)):
        out[name + "_us_per_call"] = _indexer_graph_us(
            msa, torch,
            lambda g=group: msa.msa_index_scores(d["iq"], d["pos"], d["seq"], d["pt"], d["view"], d["bs"],
                                                 ik_scale=d["scale"], num_pages=wl.num_pages, group_tokens=g),
            topk, reps)
    # keys visible to the window's last token, read once per window: the grouped call's algorithmic bytes
    last = wl.positions.reshape(-1, L)[:, -1].astype(np.int64)
    keys = int((last + 1).sum())
    b = (keys * 128 + wl.T * wl.hiq * 256 + wl.T * 8 + keys // 64 * 4 + 2 * wl.hiq * wl.T * nb * 8
         + wl.hiq * wl.T * (16 * 4 + 4))
    gbs = b / (out["grouped_us_per_call"] * 1e-6) / 1e9
    out["algorithmic_bytes_per_call"] = b
    out["roofline"] = dict(bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s", frac=gbs / HBM_PEAK_GBS,
                           traffic=None, kernel="index_scores_group_kernel<2, false> + index_topk_rank_kernel")
    return out


MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_projection(msa, W, torch, np, layers, steps, warmup):
    """The packed projection x = bf16(h w^T) (hidden 3072, 2,944 packed columns) alone and with the
    producer as its epilogue, against the same projection through torch.mm (hipBLASLt) followed by
    msa_produce.  Prefill: the 65,536-token chunk, eager launches timed with HIP events.  Decode
    batch 64: `layers` layers per step captured in one HIP graph (RoPE table and slots once per
    step for the fused path)."""
    def dev16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()

    def timed(fn, n, warm, stream=None):
        s = stream or torch.cuda.current_stream()
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(n):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000 / n

    out = {"hidden": W.PROJECTION_HIDDEN, "inputs": "h ~ N(0, 1), w ~ N(0, 1/hidden), bf16"}
    # ---- prefill
    wl = W.prefill_65536()
    d = W.to_device(wl)
    h, w = W.with_projection(wl, seed=1)
    hd, wd = dev16(h), dev16(w)
    T, K = h.shape
    x = torch.empty((T, wl.W), dtype=torch.int16, device="cuda")
    cos = torch.empty((T, 64), dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    msa.msa_rope_table(d.positions, cos, sin, wl.theta)
    msa.msa_slots(d.positions, d.seq_idx, d.page_table, d.slots, page_size=wl.page_size, num_pages=wl.num_pages)
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")   # prefill: the tiled kernel uses none

    def produce():
        call(msa, wl, d)

    def fused():
        msa.msa_project_produce(hd, wd, cos, sin, d.slots, *d.weights, d.q_out, d.iq_out, d.caches[0], d.caches[1],
                                d.caches[2], workspace=ws, k_scale=d.scales[0], v_scale=d.scales[1],
                                ik_scale=d.scales[2], num_pages=wl.num_pages, rms_eps=wl.eps)

    d.x = x                                                   # produce() reads the projected row
    # The GEMMs run power-limited, so the four compositions are timed in interleaved rounds (each
    # round times every one, n launches after 2 warm ones) and each reports its median round: none
    # is favoured by running first, on a cooler chip.
    n, rounds = max(steps // 20, 5), 7
    fns = {"gemm": lambda: msa.msa_project(hd, wd, x, workspace=ws),
           "torch": lambda: torch.mm(hd.view(torch.bfloat16), wd.view(torch.bfloat16).t(), out=x.view(torch.bfloat16)),
           "prod": produce, "fused": fused}
    for f in fns.values():
        timed(f, 1, max(warmup // 60, 3))
    per = {k: [] for k in fns}
    for _ in range(rounds):
        for k, f in fns.items():
            per[k].append(timed(f, n, 2))
    gemm_us, torch_us, prod_us, fused_us = (float(np.median(per[k])) for k in ("gemm", "torch", "prod", "fused"))
    flops = 2.0 * T * wl.W * K
    tf = flops / (gemm_us * 1e-6) / 1e12
    out["prefill"] = {
        "tokens": T, "timing": f"median of {rounds} interleaved rounds of {n} launches each",
        "fused_us": fused_us, "msa_project_us": gemm_us, "msa_produce_us": prod_us,
        "msa_project_plus_produce_us": gemm_us + prod_us, "torch_mm_us": torch_us,
        "torch_mm_plus_produce_us": torch_us + prod_us,
        "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "project_tile_kernel<false> (msa_project, 65,536 x 3,072 x 2,944)"},
    }
    log(f"[bench] projection prefill: fused {fused_us:.1f} us, msa_project {gemm_us:.1f} us ({tf:.0f} TFLOP/s), "
        f"torch.mm {torch_us:.1f} us, msa_produce {prod_us:.1f} us")
    del d, x, hd, wd
    torch.cuda.empty_cache()
    # ---- decode batch 64, one graph per composition
    wls = [W.decode_batch64(layer=i) for i in range(layers)]
    devs = [W.to_device(x) for x in wls]
    for dd in devs[1:]:
        dd.positions, dd.seq_idx, dd.page_table = devs[0].positions, devs[0].seq_idx, devs[0].page_table
    hws = [W.with_projection(x, seed=10 + i) for i, x in enumerate(wls)]
    hds = [(dev16(a), dev16(b)) for a, b in hws]
    d0, wl0 = devs[0], wls[0]
    Tt = wl0.T
    cos = torch.empty((Tt, 64), dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    ws = torch.zeros(msa.msa_project_workspace_size(Tt, K, wl0.W // 128), dtype=torch.uint8, device="cuda")
    xs = torch.empty((Tt, wl0.W), dtype=torch.int16, device="cuda")

    def step_fused():
        msa.msa_rope_table(d0.positions, cos, sin, wl0.theta)
        msa.msa_slots(d0.positions, d0.seq_idx, d0.page_table, d0.slots, page_size=wl0.page_size,
                      num_pages=wl0.num_pages)
        for wl_, dd, (a_, b_) in zip(wls, devs, hds):
            msa.msa_project_produce(a_, b_, cos, sin, d0.slots, *dd.weights, dd.q_out, dd.iq_out, dd.caches[0],
                                    dd.caches[1], dd.caches[2], workspace=ws, k_scale=dd.scales[0],
                                    v_scale=dd.scales[1], ik_scale=dd.scales[2], num_pages=wl_.num_pages)

    def step_ours():
        for wl_, dd, (a_, b_) in zip(wls, devs, hds):
            msa.msa_project(a_, b_, xs, workspace=ws)
            dd.x = xs
            call(msa, wl_, dd)

    def step_torch():
        for wl_, dd, (a_, b_) in zip(wls, devs, hds):
            torch.mm(a_.view(torch.bfloat16), b_.view(torch.bfloat16).t(), out=xs.view(torch.bfloat16))
            dd.x = xs
            call(msa, wl_, dd)

    res = {"layers": layers, "tokens": Tt}
    for name, fn in (("fused", step_fused), ("msa_project_plus_produce", step_ours),
                     ("torch_mm_plus_produce", step_torch)):
        s_ = torch.cuda.Stream()
        s_.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s_):
            fn()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s_):
                fn()
        torch.cuda.synchronize()
        with torch.cuda.stream(s_):
            us = timed(g.replay, 50, 10, stream=s_)
        res[name + "_us_per_step"] = us
        res[name + "_us_per_layer"] = us / layers
    # Algorithmic bytes of one fused layer call: the packed weight and the hidden rows, each token's RoPE
    # coefficients (2 x 64 binary32) and slot, and the producer's outputs (its bytes minus the packed
    # row it no longer reads and its per-token metadata).
    ab = (wl0.W * K * 2 + Tt * K * 2 + Tt * (2 * 64 * 4 + 8)
          + wl0.algorithmic_bytes() - Tt * wl0.W * 2 - Tt * 12)
    gbs = ab / (res["fused_us_per_layer"] * 1e-6) / 1e9
    res["algorithmic_bytes_per_layer_call"] = ab
    res["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                       "traffic": None, "kernel": "project_split_kernel<true> (msa_project_produce, 64 x 3,072 x 2,944)"}
    out["decode"] = res
    log(f"[bench] projection decode-64: fused {res['fused_us_per_layer']:.2f} us/layer, "
        f"msa_project + produce {res['msa_project_plus_produce_us_per_layer']:.2f}, "
        f"torch.mm + produce {res['torch_mm_plus_produce_us_per_layer']:.2f}")
    del devs, hds
    torch.cuda.empty_cache()
    return out


def host_threads():
    """(threads the CPU oracle runs on, cores this process may use): one GPU's share of the host is 16
    threads, so at most 16 of the usable cores."""
    cores = len(os.sched_getaffinity(0))
    return min(16, cores), cores


def cpu_baseline(W, seconds: float):
    """The CPU oracle as it stands, on leading slices of the prefill workload for about `seconds`."""
    import oracle
    threads, cores = host_threads()
    wl = W.prefill_65536()
    rows = 4096
    args = (wl.x, wl.x_stride, rows, wl.head_dim, wl.hq, wl.hkv, wl.hiq, wl.hik, wl.positions[:rows],
            wl.seq_idx[:rows], wl.page_table, wl.max_pages, wl.num_seqs, wl.max_pages, wl.page_size, wl.num_pages,
            *wl.weights, wl.eps, wl.theta)
    kw = dict(dtypes=[c.dtype for c in wl.caches], scales=[c.scale for c in wl.caches], num_threads=threads)
    oracle.produce_rows(*args, **kw)
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.produce_rows(*args, **kw)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_call = el / n
    bytes_per_call = wl.algorithmic_bytes() * rows / wl.T
    return dict(value=bytes_per_call / per_call / 1e9, unit="GB/s", cores=threads, host_cores=cores, kind="oracle",
                sample=f"{n} oracle calls on the first {rows} tokens of the 65,536-token prefill (all heads, fp8 "
                       f"cache codes in the dense per-token form), {threads} OpenMP threads (one GPU's share of "
                       f"the host; {cores} cores usable by this process), {el:.1f} s: "
                       f"{per_call * 1e3:.1f} ms per {rows} tokens")


def cpu_detail(W, seconds: float):
    """The CPU oracle with one thread and with every host thread (at most 16), on the decode batch of
    64 tokens and on the first 4,096 tokens of the prefill workload: about `seconds` per figure."""
    import oracle
    out = []
    for name, wl, rows in (("decode batch 64", W.decode_batch64(), 64), ("prefill, first 4,096 tokens", W.prefill_65536(), 4096)):
        args = (wl.x, wl.x_stride, rows, wl.head_dim, wl.hq, wl.hkv, wl.hiq, wl.hik, wl.positions[:rows],
                wl.seq_idx[:rows], wl.page_table, wl.max_pages, wl.num_seqs, wl.max_pages, wl.page_size,
                wl.num_pages, *wl.weights, wl.eps, wl.theta)
        for threads in (1, host_threads()[0]):
            kw = dict(dtypes=[c.dtype for c in wl.caches], scales=[c.scale for c in wl.caches], num_threads=threads)
            oracle.produce_rows(*args, **kw)
            n, t0 = 0, time.perf_counter()
            while True:
                oracle.produce_rows(*args, **kw)
                n += 1
                el = time.perf_counter() - t0
                if el >= seconds:
                    break
            per_call = el / n
            gbs = wl.algorithmic_bytes() * rows / wl.T / per_call / 1e9
            out.append({"workload": name, "threads": threads, "calls": n, "ms_per_call": per_call * 1e3,
                        "GB_per_s": gbs})
            log(f"[bench] oracle {name}, {threads} threads: {per_call * 1e3:.3f} ms per call, {gbs:.2f} GB/s")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed prefill launches")
    ap.add_argument("--warmup", type=int, default=300, help="untimed prefill launches first (at least)")
    ap.add_argument("--warm-ms", type=float, default=300.0,
                    help="untimed prefill launches continue until this much device time has run: the engine "
                         "clock takes tens of ms of load to settle")
    ap.add_argument("--layers", type=int, default=60)
    ap.add_argument("--decode-steps", type=int, default=200, help="timed 60-layer decode graph replays")
    ap.add_argument("--decode-warmup", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-indexer", action="store_true", help="skip the indexer measurement")
    ap.add_argument("--no-unfused", action="store_true", help="skip the unfused-path comparison")
    ap.add_argument("--no-verify", action="store_true", help="skip the verify-window decode measurement")
    ap.add_argument("--no-projection", action="store_true", help="skip the projection (GEMM + producer) measurement")
    ap.add_argument("--cpu-detail", action="store_true",
                    help="only time the CPU oracle (one thread and every host thread, decode batch 64 and a "
                         "4,096-token prefill slice), print one JSON line and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run three plain 1 GiB device-to-device copies (the reference kernel that "
                         "scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the producer runs on one tensor-parallel rank's local heads "
              f"and never communicates; --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    if args.cpu_detail:
        from paged_kv_cache_msa_amd import workloads as W
        threads, cores = host_threads()
        print(json.dumps({"cpu_oracle": cpu_detail(W, args.cpu_seconds / 4), "threads": threads,
                          "host_cores": cores}), flush=True)
        return

    import torch
    import paged_kv_cache_msa_amd as msa
    from paged_kv_cache_msa_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    msa.lib()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each": src.numel() * 4, "copies": 3}), flush=True)
        return

    # The prefill runs first, on input staged before any device work, so that nothing but its own
    # warm phase precedes its timed launches.
    pre = bench_prefill(msa, W, torch, args.steps, args.warmup, args.warm_ms, stage_prefill(W, torch),
                        0 if args.no_unfused else 50)
    torch.cuda.empty_cache()
    cref = copy_reference(torch, pre["bytes"])
    dec = bench_decode(msa, W, torch, args.layers, args.decode_steps, args.decode_warmup)
    us_step = dec["ms_per_step"] * 1000
    us_call = us_step / args.layers
    launch_us = dec["ms_total"] * 1000 / dec["launches"]
    launch_gbs = dec["bytes_per_call"] / (launch_us * 1e-6) / 1e9
    ver = None if args.no_verify else bench_verify(msa, W, torch, __import__("numpy"), dec["wls"], dec["devs"],
                                                   args.decode_steps, args.decode_warmup)
    unf = None
    if not args.no_unfused:
        unf = bench_decode_unfused(msa, torch, dec["wls"], dec["devs"], args.decode_steps, args.decode_warmup)
    del dec["devs"]
    torch.cuda.empty_cache()

    import numpy as np
    idx = None if args.no_indexer else bench_indexer(msa, W, torch, np, 50)
    torch.cuda.empty_cache()
    idx_ver = None if args.no_indexer or args.no_verify else bench_indexer_verify(msa, W, torch, np, 50)
    torch.cuda.empty_cache()
    if idx_ver:
        log(f"[bench] indexer on verify windows ({idx_ver['tokens']} tokens): per token "
            f"{idx_ver['per_token_us_per_call']:.2f} us, grouped {idx_ver['grouped_us_per_call']:.2f} us per call")
    proj = None if args.no_projection else bench_projection(msa, W, torch, np, args.layers, args.steps, args.warmup)
    torch.cuda.empty_cache()
    cpu = None if args.no_cpu_baseline else cpu_baseline(W, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": pre["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["us_per_call"] / 1000,
        "pct_of_hbm_peak": 100.0 * pre["gbs"] / HBM_PEAK_GBS,
        "us_per_layer_call": us_call,
        "us_per_decode_step": us_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "prefill chunk: 8 seqs x 8192 tokens (65,536 rows) at positions 0..8191, local heads Q=16 "
                        "KV=2 index-Q=2 index-K=1, head_dim 128, fp8 e4m3 HND caches, 12,000-page pool; one "
                        "msa_produce launch per step.  us_per_layer_call: decode batch 64 (64 seqs x 1 token at "
                        f"positions 7000..9199), {args.layers} layer calls per step in one HIP graph",
            "tokens": 65536,
            "algorithmic_bytes_per_step": pre["bytes"],
            "decode_tokens": 64,
            "decode_layers": args.layers,
            "decode_algorithmic_bytes_per_layer_call": dec["bytes_per_call"],
            "parallelism": "single GPU (one tensor-parallel rank's local heads)",
        },
        "roofline": {
            "bound": "hbm", "achieved": pre["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": pre["gbs"] / HBM_PEAK_GBS, "traffic": counter_traffic("prefill_65536"),
            "kernel": "produce_kernel<3, 16, 2, 2, 1> (prefill)", "avg_launch_us": pre["us_per_call"],
            "warm_launches": pre["warm_launches"], "warm_ms": pre["warm_ms"],
            "reference_copy": {"what": "torch device-to-device copy moving the same bytes (half read, half written)",
                               "us": cref["us"], "gbs": cref["gbs"], "frac_of_peak": cref["gbs"] / HBM_PEAK_GBS},
        },
        "decode": {
            "steps": args.decode_steps, "warmup": args.decode_warmup, "layers": args.layers,
            "step": "positions advanced by one in place (one elementwise node), then one producer launch per "
                    "layer; every replay writes new slots",
            "us_per_layer_call": us_call, "us_per_step": us_step,
            "roofline": {
                "bound": "hbm", "achieved": launch_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": launch_gbs / HBM_PEAK_GBS, "traffic": counter_traffic("decode_64"),
                "kernel": "produce_kernel<1, 16, 2, 2, 1> (decode batch 64)", "avg_launch_us": launch_us,
            },
        },
        "unfused": None if unf is None else {
            "path": "msa_slots once per step, then per layer: main and index norm/RoPE producers, and division, "
                    "remainder, index cast and scatter for each of K, V and index-K (identical output bytes)",
            "decode": dict(unf, fused_launches_per_step=args.layers, fused_us_per_step=us_step),
            "prefill": {"us_per_call": pre.get("unfused_us_per_call"),
                        "launches_per_call": pre.get("unfused_launches_per_call"),
                        "fused_us_per_call": pre["us_per_call"]},
        },
        "verify": ver,
        "projection": proj,
        "indexer": idx,
        "indexer_verify": idx_ver,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
