"""Seeded synthetic inputs for the MSA fused producer.

This module only draws inputs; it contains none of the producer's arithmetic.
Both the HIP path (tests, benchmark) and the CPU oracle consume what it returns.

The workloads stand in for the serving workload the pages measure on (random
prompts of about 8k input and 1k output tokens at concurrency 32/64 in "Fuse
MiniMax-M3 MSA per-layer KV-cache writes into one kernel", "Measured impact";
8K input / 1K output at concurrency 256 in "Fuse MiniMax-M3 QKV and index
projection", "Performance"):
decode positions around 8k context, batches of 64 and 256, 8192-token prefill
chunks, and a mixed prefill+decode batch whose cache pool needs 64-bit offsets.

Every array is plain numpy on the host:
  x            uint16 [T, row_stride] (bf16 bits); the producer reads the first W columns
  positions    int32 [T]
  seq_idx      int32 [T] (-1 marks a padded token)
  page_table   int32 [num_seqs, max_pages]
  weights      4 x uint16 [D] (bf16 bits) for Q, K, index-Q, index-K (None when that stream has no heads)
  caches       3 x CacheSpec for K, V, index-K
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

FP8_E4M3 = 0
BF16 = 1
SENTINEL_BYTE = 0x7F
HEAD_DIM = 128
PAGE_SIZE = 64


@dataclasses.dataclass
class CacheSpec:
    """A paged HND cache view [num_pages, heads, page_size, head_dim] over a flat storage.

    storage_shape is the full allocation (may be larger than the view, e.g. a padded token dim);
    strides are the view's element strides (page, head, token); the dim stride is 1.
    """
    heads: int
    dtype: int
    scale: float
    storage_shape: tuple
    strides: tuple

    @property
    def elem_size(self) -> int:
        return 1 if self.dtype == FP8_E4M3 else 2

    @property
    def storage_elems(self) -> int:
        return int(np.prod(self.storage_shape)) if self.heads > 0 else 0


@dataclasses.dataclass
class Workload:
    name: str
    hq: int
    hkv: int
    hiq: int
    hik: int
    head_dim: int
    page_size: int
    num_pages: int
    x: np.ndarray
    positions: np.ndarray
    seq_idx: np.ndarray
    page_table: np.ndarray
    weights: List[Optional[np.ndarray]]
    caches: List[CacheSpec]
    eps: float = 1e-6
    theta: float = 1e4
    n_invalid: int = 0

    @property
    def T(self) -> int:
        return int(self.positions.shape[0])

    @property
    def W(self) -> int:
        return (self.hq + 2 * self.hkv + self.hiq + self.hik) * self.head_dim

    @property
    def x_stride(self) -> int:
        return int(self.x.shape[1])

    @property
    def num_seqs(self) -> int:
        return int(self.page_table.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    def algorithmic_bytes(self) -> int:
        """Bytes the producer must move per call: the W-column input row, Q and index-Q in bf16,
        the three cache rows of every token that has a cache slot, and 12 bytes of per-token
        metadata (position, sequence index, one page-table entry)."""
        T, D = self.T, self.head_dim
        rd = T * self.W * 2 + T * 12
        wr = T * (self.hq + self.hiq) * D * 2
        for c in self.caches:
            wr += self.n_written * c.heads * D * c.elem_size
        return rd + wr

    @property
    def n_written(self) -> int:
        """Tokens that own a cache slot, as drawn: all tokens minus those made padded or
        pointed past the pool on purpose."""
        return self.T - self.n_invalid


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bits (torch's round-to-nearest-even cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _normal_bf16(rng, shape, sigma):
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma))


def _weights(rng, hq, hkv, hiq, hik, D):
    out = []
    for h in (hq, hkv, hiq, hik):
        out.append(to_bf16_bits(rng.uniform(0.5, 1.5, D).astype(np.float32)) if h > 0 else None)
    return out


def _hnd_cache(num_pages, heads, dtype, scale, page_size=PAGE_SIZE, D=HEAD_DIM, token_pad=0):
    tp = page_size + token_pad
    shape = (num_pages, heads, tp, D)
    strides = (heads * tp * D, tp * D, D)
    return CacheSpec(heads=heads, dtype=dtype, scale=float(scale), storage_shape=shape, strides=strides)


# Head geometry of one tensor-parallel rank: Q=16, KV=2, index-Q=2, index-K=1 (W = 23 * 128 = 2944).
DECODE_HEADS = (16, 2, 2, 1)


def tiny_decode(seed: int = 0) -> Workload:
    """Tiny decode: 4 sequences x 1 token, positions U{0..511}, heads 4/1/1/1 (W = 1024),
    16-page pool, page table [4, 8] from permutations of the pool, fp8 caches with scale 1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    hq, hkv, hiq, hik = 4, 1, 1, 1
    return _tiny(rng, "tiny-decode-4 (heads 4/1/1/1, W=1024)", hq, hkv, hiq, hik)


def tiny_decode_no_index_k(seed: int = 10) -> Workload:
    """Tiny decode without index-K: heads 4/1/1/0 (W = 896)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _tiny(rng, "tiny-decode-4 no index-K (heads 4/1/1/0, W=896)", 4, 1, 1, 0)


def _tiny(rng, name, hq, hkv, hiq, hik):
    T = S = 4
    D, P, num_pages, max_pages = HEAD_DIM, PAGE_SIZE, 16, 8
    W = (hq + 2 * hkv + hiq + hik) * D
    x = _normal_bf16(rng, (T, W), 1.0)
    pos = rng.integers(0, 512, T).astype(np.int32)
    seq = np.arange(T, dtype=np.int32)
    while True:
        pt = np.concatenate([rng.permutation(num_pages), rng.permutation(num_pages)]).astype(np.int32).reshape(S, max_pages)
        written = pt[seq, pos // P]
        if len(set(written.tolist())) == T:
            break
    w = _weights(rng, hq, hkv, hiq, hik, D)
    caches = [_hnd_cache(num_pages, h, FP8_E4M3, 1.0) for h in (hkv, hkv, hik)]
    return Workload(name, hq, hkv, hiq, hik, D, P, num_pages, x, pos, seq, pt, w, caches)


def decode_batch64(seed: int = 1, layer: int = 0, meta_only: bool = False) -> Workload:
    """Decode batch 64: 64 sequences x 1 token at positions U{7000..9199}, heads 16/2/2/1,
    page table = permutation(10240) as [64, 160], fp8 caches [10240, H, 64, 128], scales U(0.5, 2).
    `layer` draws a distinct input row, weights and scales per layer over shared metadata."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T = S = 64
    D, P, max_pages = HEAD_DIM, PAGE_SIZE, 160
    num_pages = S * max_pages
    hq, hkv, hiq, hik = DECODE_HEADS
    pos = rng.integers(7000, 9200, T).astype(np.int32)
    seq = np.arange(T, dtype=np.int32)
    pt = rng.permutation(num_pages).astype(np.int32).reshape(S, max_pages)
    lrng = np.random.Generator(np.random.PCG64([seed, 1000 + layer]))
    W = (hq + 2 * hkv + hiq + hik) * D
    x = np.zeros((T, W), np.uint16) if meta_only else _normal_bf16(lrng, (T, W), 1.0)
    w = _weights(lrng, hq, hkv, hiq, hik, D)
    scales = lrng.uniform(0.5, 2.0, 3)
    caches = [_hnd_cache(num_pages, h, FP8_E4M3, s) for h, s in zip((hkv, hkv, hik), scales)]
    return Workload(f"decode-64 x 1 token, heads 16/2/2/1, fp8 (layer {layer})", hq, hkv, hiq, hik, D, P,
                    num_pages, x, pos, seq, pt, w, caches)


def decode_batch256_padded(seed: int = 2) -> Workload:
    """Decode batch 256 with padding: 26 tokens (10%) padded (seq = -1), 5 tokens (2%) whose page-table
    entry points past the pool; x is columns [0, 2944) of a [256, 3072] buffer; caches are the
    [:, :, :64, :] view of storage [40960, H, 65, 128] (padded token dimension)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T = S = 256
    D, P, max_pages = HEAD_DIM, PAGE_SIZE, 160
    num_pages = S * max_pages
    hq, hkv, hiq, hik = DECODE_HEADS
    pos = rng.integers(7000, 9200, T).astype(np.int32)
    seq = np.arange(T, dtype=np.int32)
    pt = rng.permutation(num_pages).astype(np.int32).reshape(S, max_pages)
    order = rng.permutation(T)
    padded, oob = order[:26], order[26:31]
    seq[padded] = -1
    for k, t in enumerate(oob):
        pt[t, pos[t] // P] = num_pages + int(rng.integers(0, 1000))
    x = _normal_bf16(rng, (T, 3072), 1.0)
    w = _weights(rng, hq, hkv, hiq, hik, D)
    scales = rng.uniform(0.5, 2.0, 3)
    caches = [_hnd_cache(num_pages, h, FP8_E4M3, s, token_pad=1) for h, s in zip((hkv, hkv, hik), scales)]
    return Workload("decode-256 padded, strided input [256,3072], padded-head-stride fp8 caches",
                    hq, hkv, hiq, hik, D, P, num_pages, x, pos, seq, pt, w, caches,
                    n_invalid=len(padded) + len(oob))


def prefill_65536(seed: int = 3, variant: int = 0) -> Workload:
    """Prefill chunk: 8 sequences x 8192 tokens (65,536 rows) at positions 0..8191, heads 16/2/2/1,
    x ~ N(0, 1.5^2), page table [8, 128] = 1,024 distinct pages of a permuted 12,000-page pool,
    fp8 caches, scales U(0.5, 2).  `variant` redraws the values (not the shapes)."""
    rng = np.random.Generator(np.random.PCG64([seed, variant]))
    S, L = 8, 8192
    T = S * L
    D, P = HEAD_DIM, PAGE_SIZE
    max_pages, num_pages = L // P, 12000
    hq, hkv, hiq, hik = DECODE_HEADS
    t = np.arange(T, dtype=np.int64)
    pos = (t % L).astype(np.int32)
    seq = (t // L).astype(np.int32)
    pt = rng.permutation(num_pages)[: S * max_pages].astype(np.int32).reshape(S, max_pages)
    W = (hq + 2 * hkv + hiq + hik) * D
    x = _normal_bf16(rng, (T, W), 1.5)
    w = _weights(rng, hq, hkv, hiq, hik, D)
    scales = rng.uniform(0.5, 2.0, 3)
    caches = [_hnd_cache(num_pages, h, FP8_E4M3, s) for h, s in zip((hkv, hkv, hik), scales)]
    return Workload("prefill 8 x 8192 tokens (65,536 rows), heads 16/2/2/1, fp8", hq, hkv, hiq, hik, D, P,
                    num_pages, x, pos, seq, pt, w, caches)


def mixed_batch_64bit(cache_dtype: int = BF16, seed: int = 4) -> Workload:
    """Mixed batch with 64-bit offsets: 4 prefill chunks of 2048 tokens (chunk start U{1..30720})
    followed by 192 decode tokens (positions U{1..32767}); T = 8384; page table [196, 512];
    270,000-page pool so that index-K holds 2.21e9 > 2^31 elements; at least a quarter of the written
    pages have ids >= 262,144 so K and index-K offsets exceed 32 bits."""
    rng = np.random.Generator(np.random.PCG64(seed))
    D, P, max_pages, num_pages = HEAD_DIM, PAGE_SIZE, 512, 270_000
    hq, hkv, hiq, hik = DECODE_HEADS
    n_chunks, chunk, n_dec = 4, 2048, 192
    S = n_chunks + n_dec
    starts = rng.integers(1, 30721, n_chunks)
    pos = np.concatenate([s + np.arange(chunk) for s in starts] + [rng.integers(1, 32768, n_dec)]).astype(np.int32)
    seq = np.concatenate([np.full(chunk, i) for i in range(n_chunks)] + [np.arange(n_chunks, S)]).astype(np.int32)
    T = pos.shape[0]
    # logical pages actually written, per sequence
    needed = sorted({(int(s), int(p) // P) for s, p in zip(seq, pos)})
    n_high = (len(needed) + 3) // 4
    high = rng.choice(np.arange(262_144, num_pages), n_high, replace=False)
    low = rng.choice(262_144, len(needed) - n_high, replace=False)
    phys = rng.permutation(np.concatenate([high, low]))
    pt = rng.integers(0, num_pages, (S, max_pages)).astype(np.int32)
    for (s, lp), pg in zip(needed, phys):
        pt[s, lp] = pg
    W = (hq + 2 * hkv + hiq + hik) * D
    x = _normal_bf16(rng, (T, W), 1.0)
    w = _weights(rng, hq, hkv, hiq, hik, D)
    scales = rng.uniform(0.5, 2.0, 3)
    caches = [_hnd_cache(num_pages, h, cache_dtype, s) for h, s in zip((hkv, hkv, hik), scales)]
    dn = "bf16" if cache_dtype == BF16 else "fp8"
    return Workload(f"mixed 4x2048 prefill + 192 decode, 270,000-page pool (64-bit offsets), {dn}",
                    hq, hkv, hiq, hik, D, P, num_pages, x, pos, seq, pt, w, caches)


def ragged(T: int, seed: int = 7, heads=DECODE_HEADS, cache_dtypes=(FP8_E4M3, FP8_E4M3, FP8_E4M3),
           pad_frac: float = 0.1, sigma: float = 1.0, row_pad: int = 0, page_size: int = PAGE_SIZE) -> Workload:
    """Arbitrary token count (ragged tails of the launch grid): T single-token sequences with
    positions U{0..4095}, some padded, distinct pages, caches with mixed dtypes if asked, pages of
    `page_size` tokens (any size; 4096 / page_size pages per sequence)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    hq, hkv, hiq, hik = heads
    D, P = HEAD_DIM, page_size
    max_pages = -(-4096 // P)
    S = max(T, 1)
    num_pages = S * 2 + 7
    pos = rng.integers(0, 4096, T).astype(np.int32)
    seq = np.arange(T, dtype=np.int32)
    if T:
        seq[rng.random(T) < pad_frac] = -1
    pt = rng.integers(0, num_pages, (S, max_pages)).astype(np.int32)
    distinct = rng.permutation(num_pages)[:T]
    for t in range(T):
        pt[t, pos[t] // P] = distinct[t]
    W = (hq + 2 * hkv + hiq + hik) * D
    x = _normal_bf16(rng, (T, W + row_pad), sigma)
    w = _weights(rng, hq, hkv, hiq, hik, D)
    scales = rng.uniform(0.5, 2.0, 3)
    caches = [_hnd_cache(num_pages, h, dt, s, page_size=P) for h, dt, s in zip((hkv, hkv, hik), cache_dtypes, scales)]
    return Workload(f"ragged T={T}" + ("" if P == PAGE_SIZE else f", page size {P}"), hq, hkv, hiq, hik, D, P,
                    num_pages, x, pos, seq, pt, w, caches,
                    n_invalid=int(np.count_nonzero(seq < 0)))


@dataclasses.dataclass
class DeviceWorkload:
    """A workload staged in device memory: inputs, zero-initialised outputs and sentinel-filled
    caches.  `storages` are the flat cache allocations; `caches` the 4-D views handed to the
    producer (over the first num_pages * ... elements of each storage)."""
    x: torch.Tensor
    positions: torch.Tensor
    seq_idx: torch.Tensor
    page_table: torch.Tensor
    weights: list
    q_out: torch.Tensor
    iq_out: torch.Tensor
    storages: list
    caches: list
    scales: list
    slots: torch.Tensor


def to_device(wl: Workload, device="cuda", sentinel: int = SENTINEL_BYTE) -> DeviceWorkload:
    T, D = wl.T, wl.head_dim
    x_full = torch.from_numpy(wl.x.view(np.int16)).to(device)
    x = x_full[:, : wl.W]
    pos = torch.from_numpy(wl.positions).to(device)
    seq = torch.from_numpy(wl.seq_idx).to(device)
    pt = torch.from_numpy(np.ascontiguousarray(wl.page_table)).to(device)
    ws = [None if w is None else torch.from_numpy(w.view(np.int16)).to(device) for w in wl.weights]
    q = torch.zeros((T, wl.hq, D), dtype=torch.int16, device=device)
    iq = torch.zeros((T, wl.hiq, D), dtype=torch.int16, device=device)
    storages, views, scales = [], [], []
    for c in wl.caches:
        if c.heads == 0:
            storages.append(None)
            views.append(None)
            scales.append(None)
            continue
        if c.dtype == FP8_E4M3:
            s = torch.full((c.storage_elems,), sentinel, dtype=torch.uint8, device=device)
        else:
            s = torch.full((c.storage_elems,), sentinel * 0x0101, dtype=torch.int16, device=device)
        storages.append(s)
        views.append(s.as_strided((wl.num_pages, c.heads, wl.page_size, D), (*c.strides, 1)))
        scales.append(torch.tensor([c.scale], dtype=torch.float32, device=device))
    slots = torch.full((T,), -7, dtype=torch.int64, device=device)
    return DeviceWorkload(x, pos, seq, pt, ws, q, iq, storages, views, scales, slots)


def verify_window(draft_len: int = 3, seqs: int = 64, seed: int = 5, cache_dtype: int = FP8_E4M3,
                  num_pages: int = 10240, max_pages: int = 160, pos_lo: int = 7000, pos_hi: int = 9200,
                  layer: int = 0) -> Workload:
    """Speculative-decoding verify rows: every sequence brings 1 + draft_len consecutive tokens (the
    uniform verify window of one-model Eagle3 decoding in "Wire in custom decode kernels for
    MinimaxM3", conflict-resolution notes), so windows cross page boundaries.  Each sequence's
    page table holds distinct pages for every logical page its window touches; `num_pages` and
    `max_pages` set the pool geometry (a draft model uses its own)."""
    rng = np.random.Generator(np.random.PCG64([seed, layer]))
    D, P = HEAD_DIM, PAGE_SIZE
    hq, hkv, hiq, hik = DECODE_HEADS
    L = 1 + draft_len
    base = rng.integers(pos_lo, pos_hi, seqs)
    # force some windows to straddle a page boundary
    straddle = rng.random(seqs) < 0.25
    base = np.where(straddle, (base // P + 1) * P - rng.integers(1, L, seqs), base)
    pos = (base[:, None] + np.arange(L)[None, :]).reshape(-1).astype(np.int32)
    seq = np.repeat(np.arange(seqs), L).astype(np.int32)
    assert int(pos.max()) // P < max_pages
    pt = rng.integers(0, num_pages, (seqs, max_pages)).astype(np.int32)
    touched = sorted({(int(s), int(p_) // P) for s, p_ in zip(seq, pos)})
    for (s, lp), pg in zip(touched, rng.permutation(num_pages)[: len(touched)]):
        pt[s, lp] = pg
    W_ = (hq + 2 * hkv + hiq + hik) * D
    x = _normal_bf16(rng, (seqs * L, W_), 1.0)
    w = _weights(rng, hq, hkv, hiq, hik, D)
    scales = rng.uniform(0.5, 2.0, 3)
    caches = [_hnd_cache(num_pages, h, cache_dtype, s) for h, s in zip((hkv, hkv, hik), scales)]
    return Workload(f"verify window {seqs} seqs x (1 + {draft_len}) tokens, {num_pages}-page pool", hq, hkv, hiq, hik,
                    D, P, num_pages, x, pos, seq, pt, w, caches)


def index_cache_fill(wl: Workload, seed: int = 99) -> np.ndarray:
    """Pre-populated index-K cache storage (the keys of earlier tokens): random finite codes over the
    whole storage (fp8: every byte except the NaN codes 0x7F / 0xFF; bf16: N(0, 1) values)."""
    c = wl.caches[2]
    rng = np.random.Generator(np.random.PCG64([seed, 7]))
    if c.dtype == FP8_E4M3:
        codes = rng.integers(0, 254, c.storage_elems, dtype=np.uint16).astype(np.uint8)
        codes[codes >= 0x7F] += 1            # 0..253 -> every code but 0x7F and 0xFF
        return codes
    return to_bf16_bits(rng.standard_normal(c.storage_elems, dtype=np.float32))


def index_queries(T: int, hiq: int, seed: int = 98) -> np.ndarray:
    """Index-Q rows [T, hiq, 128] as bf16 bits, N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64([seed, 8]))
    return to_bf16_bits(rng.standard_normal((T, hiq, HEAD_DIM), dtype=np.float32))


def index_blocks(wl: Workload, block_tokens: int = 128) -> int:
    """Row length of the block-score table: enough blocks for the largest position."""
    return int(wl.positions.max()) // block_tokens + 1 if wl.T else 0


# ------------------------------------------------------------------ projection inputs

PROJECTION_HIDDEN = 3072   # hidden size of the projection workloads (the pages do not state one)


def projection_inputs(T: int, hidden: int = PROJECTION_HIDDEN, n_cols: int = 2944, seed: int = 0,
                      dyadic: bool = False):
    """Hidden states h [T, hidden] and a packed projection weight w [n_cols, hidden], bf16 bits.

    Default: h ~ N(0, 1) and w ~ N(0, 1/hidden), so the packed row x = h w^T is about N(0, 1) like
    the producer workloads' rows.  dyadic=True draws h from {k/16 : |k| <= 64} and w from
    {k/64 : |k| <= 32}: every product is a multiple of 2^-10 and every partial sum stays below
    2^14 in magnitude for hidden <= 8192, so a binary32 accumulation in any order is exact and the
    projection has one correct answer bit for bit."""
    rng = np.random.Generator(np.random.PCG64([seed, 4242]))
    if dyadic:
        h = rng.integers(-64, 65, (T, hidden)).astype(np.float32) / np.float32(16)
        w = rng.integers(-32, 33, (n_cols, hidden)).astype(np.float32) / np.float32(64)
    else:
        h = rng.standard_normal((T, hidden), dtype=np.float32)
        w = rng.standard_normal((n_cols, hidden), dtype=np.float32) * np.float32(1.0 / np.sqrt(hidden))
    return to_bf16_bits(h), to_bf16_bits(w)


def with_projection(wl: Workload, hidden: int = PROJECTION_HIDDEN, seed: int = 0, dyadic: bool = False):
    """(h, w) for a producer workload: the packed row of wl becomes bf16(h w^T); wl.x is left as is
    (the caller replaces it with the oracle's projection where a row is needed)."""
    return projection_inputs(wl.T, hidden, wl.W, seed=seed, dyadic=dyadic)
