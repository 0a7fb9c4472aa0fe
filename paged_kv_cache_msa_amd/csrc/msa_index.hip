// MSA indexer for CDNA4 (gfx950): block scores of index-Q against the paged index-K cache, max-pooled
// over fixed token blocks, and the top-k blocks per (index-Q head, token).  Operation: page "Fuse
// MiniMax-M3 MSA per-layer KV-cache writes into one kernel", "Where this PR targets at", step 4;
// page "Fuse MiniMax-M3 QKV and index projection", BEFORE/AFTER figures (score visible index-K,
// max-pool by block, select top-k block IDs).  The reading is documented in include/msa_index.h.
//
// Scoring streams the visible keys (128 B of fp8 per key).  Each key meets only the few index-Q
// heads of its own token (decode tokens share no keys), so there is no reuse for the matrix cores
// to exploit, and the scores are exact binary64 dot products: it runs on the vector ALUs, where the
// binary64 conversions and multiply-adds (about 3.5 vector instructions per key byte with two
// heads) cost about as much time as the key bytes take to arrive, so the kernels are built to keep
// both busy at once.  8 lanes per key (16 elements each), 8 keys per step.  Products of bf16 and
// e4m3/bf16 values are exact in binary64 and so are their sums, so the block scores do not depend
// on the summation order.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "msa_common.h"
#include "msa_index.h"

namespace {

using msa_internal::aligned;
using msa_internal::CacheDev;
using msa_internal::check_cache;
using msa_internal::check_operands;
using msa_internal::kHeadDim;
using msa_internal::nbytes;
using msa_internal::row_bytes;
using msa_internal::Span;

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kLanesPerKey = 8;
constexpr int kKeysPerStep = kWave / kLanesPerKey;
constexpr int kElemsPerLane = kHeadDim / kLanesPerKey;   // 16
constexpr int kMaxHeadsPerLaunch = 2;
constexpr int kParts = 2;                  // waves per (token, block), each scoring a contiguous part
constexpr int kMaxTopK = 64;
constexpr int kMaxRowBlocks = 4096;
constexpr int kRankRowBlocks = 512;     // rows of up to this many blocks are ranked in LDS
constexpr int kRankThreads = 512;       // threads of the ranking work-group

struct ScoreArgs {
    const uint16_t* iq;
    const int32_t* pos;
    const int32_t* seq;
    const int32_t* pt;
    int64_t pt_stride;
    int64_t num_pages;
    int32_t T, S, max_pages, page_size, page_shift;
    int32_t hiq, group, head0, block_tokens, max_blocks;
    CacheDev ik;
    double* out;
};

template <int Ctrl>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, Ctrl, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), Ctrl, 0xf, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Sum over the 8 lanes of a key group; every lane of the group ends with the same value.
__device__ __forceinline__ double sum8(double v)
{
    v += dpp_f64<0xb1>(v);    // quad_perm [1,0,3,2]
    v += dpp_f64<0x4e>(v);    // quad_perm [2,3,0,1]
    v += dpp_f64<0x141>(v);   // row_half_mirror
    return v;
}

__device__ __forceinline__ double shfl_xor_f64(double v, int m)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __shfl_xor((int)(uint32_t)u, m), hi = __shfl_xor((int)(uint32_t)(u >> 32), m);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// max that never lets a NaN in: a NaN candidate loses against anything.
__device__ __forceinline__ double max_no_nan(double best, double cand) { return cand > best ? cand : best; }

// Cache slot of a position, or -1 (same rule as the producer's).
__device__ __forceinline__ int64_t page_of(const ScoreArgs& a, int32_t sq, int32_t p, int32_t* off)
{
    if (sq < 0 || sq >= a.S || p < 0) return -1;
    const int32_t lp = a.page_shift >= 0 ? p >> a.page_shift : p / a.page_size;
    if (lp >= a.max_pages) return -1;
    const int64_t pg = a.pt[(int64_t)sq * a.pt_stride + lp];
    if (pg < 0 || pg >= a.num_pages) return -1;
    *off = p - lp * a.page_size;
    return pg;
}

// This lane's 16 elements of one key, raw: fp8 keys take 16 bytes (two 8-byte loads; cache strides
// are multiples of 8 elements, so an fp8 row share is 8-byte but not always 16-byte aligned), bf16
// keys 32 bytes.
template <bool kBf16>
struct KeyRaw {
    uint32_t w[kBf16 ? 8 : 4];
};

template <bool kBf16>
__device__ __forceinline__ KeyRaw<kBf16> load_key_at(const uint8_t* p)
{
    KeyRaw<kBf16> r;
    if (kBf16) {
        const uint4* src = reinterpret_cast<const uint4*>(p);
        const uint4 lo = src[0], hi = src[1];
        r.w[0] = lo.x; r.w[1] = lo.y; r.w[2] = lo.z; r.w[3] = lo.w;
        r.w[kBf16 ? 4 : 0] = hi.x; r.w[kBf16 ? 5 : 1] = hi.y; r.w[kBf16 ? 6 : 2] = hi.z; r.w[kBf16 ? 7 : 3] = hi.w;
    } else {
        const uint2 v0 = reinterpret_cast<const uint2*>(p)[0];
        const uint2 v1 = reinterpret_cast<const uint2*>(p)[1];
        r.w[0] = v0.x; r.w[1] = v0.y; r.w[2] = v1.x; r.w[3] = v1.y;
    }
    return r;
}

template <bool kBf16>
__device__ __forceinline__ KeyRaw<kBf16> load_key(const CacheDev& c, int64_t e)
{
    return load_key_at<kBf16>(c.data + e * (kBf16 ? 2 : 1));
}

// Decode to binary64 (e4m3 and bf16 values are exact in binary32, hence in binary64).
template <bool kBf16>
__device__ __forceinline__ void decode_key(const KeyRaw<kBf16>& r, double* k)
{
    if (kBf16) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            k[2 * i] = (double)__uint_as_float(r.w[i] << 16);
            k[2 * i + 1] = (double)__uint_as_float(r.w[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)r.w[i], false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)r.w[i], true);
            k[4 * i] = (double)lo[0];
            k[4 * i + 1] = (double)lo[1];
            k[4 * i + 2] = (double)hi[0];
            k[4 * i + 3] = (double)hi[1];
        }
    }
}

// One wavefront per (token, block); heads [head0, head0 + NH).  The keys of a block are fetched in
// batches of BATCH steps (8 keys per step): every page-table entry of a batch first, then every
// key, then the arithmetic, so a wave waits on two memory round trips per batch, not two per step.
// kStepInPage: page_size and block_tokens are multiples of 8, so the 8 keys of a step always share
// one page: the page lookup and the 64-bit page base are then wave-uniform (scalar) per step.
// Four waves per SIMD (at most 128 registers, no spills): batches of 3 steps with two fp8 heads, 4
// with one, 2 with bf16 keys (whose raw rows are twice as wide) are the deepest that fit.  This
// kernel serves the layouts the batch-in-page kernel below does not take (page sizes or selection
// blocks that are not multiples of 64 tokens).
template <int NH, bool kBf16, bool kStepInPage>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void index_scores_kernel(const ScoreArgs a)
{
    constexpr int BATCH = kBf16 ? 2 : NH == 2 ? 3 : 4;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // kParts waves per (token, block), each scoring a contiguous part of the block's keys; their
    // maxima meet in LDS.  Part-block waves keep the work left after the first round of resident
    // waves short (two parts measured 5% faster than whole blocks per wave, four parts 7% slower).
    // Block-major order: waves are dispatched in item order, so the high blocks, which only the
    // tokens at the longest positions can see (the others exit at once), come last.
    const uint32_t item = blockIdx.x * (kWavesPerBlock / kParts) + (uint32_t)(wave / kParts);
    const int part = wave % kParts;
    const bool item_ok = item < (uint32_t)a.T * (uint32_t)a.max_blocks;   // wave-uniform
    const int32_t b = item_ok ? (int32_t)(item / (uint32_t)a.T) : 0;
    const int32_t t = item_ok ? (int32_t)(item - (uint32_t)b * (uint32_t)a.T) : 0;
    const int ks = lane / kLanesPerKey;    // key slot of a step
    const int sub = lane % kLanesPerKey;   // element group within the key

    const int32_t pos = a.pos[t];
    const int32_t sq = a.seq[t];
    int32_t own_off;
    const bool token_ok = item_ok && page_of(a, sq, pos, &own_off) >= 0;
    // Each part but the last takes hb positions (a multiple of 8, so that steps of 8 keys stay within
    // a page when the block does), the last one the rest.
    const int64_t hb = ((int64_t)a.block_tokens + kParts * kKeysPerStep - 1) / (kParts * kKeysPerStep) * kKeysPerStep;
    const int64_t blk0 = (int64_t)b * a.block_tokens;
    const int64_t p0_64 = blk0 + part * hb;
    const int64_t p_lim = part == kParts - 1 ? blk0 + a.block_tokens : min(blk0 + (part + 1) * hb, blk0 + (int64_t)a.block_tokens);
    const int32_t p0 = (int32_t)min(p0_64, (int64_t)INT32_MAX);   // exact whenever the part is scored
    double best[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) best[h] = -INFINITY;

    if (token_ok && p0_64 <= pos && p0_64 < p_lim) {
        // This lane's 16 elements of every head's query, as binary64.
        double q[NH][kElemsPerLane];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const uint16_t* qp = a.iq + ((int64_t)t * a.hiq + a.head0 + h) * kHeadDim + sub * kElemsPerLane;
            const uint4 lo = reinterpret_cast<const uint4*>(qp)[0], hi = reinterpret_cast<const uint4*>(qp)[1];
            const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                q[h][2 * i] = (double)__uint_as_float(w[i] << 16);
                q[h][2 * i + 1] = (double)__uint_as_float(w[i] & 0xffff0000u);
            }
        }
        const double scale = kBf16 ? 1.0 : (double)*a.ik.scale;
        const int32_t p_end = (int32_t)min(p_lim, (int64_t)pos + 1);
        const int64_t head_off = (int64_t)(a.head0 / a.group) * a.ik.sh;   // NH heads share one index-K head
        // kStepInPage: the page-table entries of up to 64 steps are fetched at once, step j of the
        // chunk by lane j, and each step reads its entry back with a lane read: one memory round
        // trip per 64 steps (512 keys) instead of a dependent lookup per step.
        int32_t step_pg = -1;      // lane j: page of step chunk0 + j, or -1
        int32_t chunk0 = 0;        // first step (counted from p0) of the fetched chunk
        bool fetched = false;
        for (int32_t pb = p0; pb < p_end; pb += BATCH * kKeysPerStep) {
            const int32_t step0 = (pb - p0) / kKeysPerStep;
            if (kStepInPage && (!fetched || step0 + BATCH > chunk0 + kWave)) {   // wave-uniform
                chunk0 = step0;
                fetched = true;
                const int64_t ps_l = (int64_t)pb + (int64_t)lane * kKeysPerStep;
                int32_t unused;
                step_pg = ps_l < p_end ? (int32_t)page_of(a, sq, (int32_t)ps_l, &unused) : -1;
            }
            int64_t e[BATCH];
            uint32_t live = 0;                     // bit i: key of step i exists and has a page
#pragma unroll
            for (int i = 0; i < BATCH; ++i) {
                const int32_t p = pb + i * kKeysPerStep + ks;
                int64_t pg;
                int32_t off = 0;
                if (kStepInPage) {
                    // the step's first position decides the page for all 8 keys (wave-uniform)
                    const int32_t ps = pb + i * kKeysPerStep;
                    const int32_t pe = __builtin_amdgcn_readlane(step_pg, step0 + i - chunk0);
                    const int32_t lps = a.page_shift >= 0 ? ps >> a.page_shift : ps / a.page_size;
                    pg = p < p_end ? (int64_t)pe : -1;   // pe is -1 for a step past p_end
                    off = ps - lps * a.page_size + ks;
                } else {
                    pg = p < p_end ? page_of(a, sq, p, &off) : -1;
                }
                // A key outside the block or without a valid page reads the pool's first row (a
                // valid address) and is discarded.
                e[i] = pg >= 0 ? pg * a.ik.sp + head_off + (int64_t)off * a.ik.st : 0;
                live |= (pg >= 0 ? 1u : 0u) << i;
            }
            KeyRaw<kBf16> raw[BATCH];
#pragma unroll
            for (int i = 0; i < BATCH; ++i) raw[i] = load_key<kBf16>(a.ik, e[i] + sub * kElemsPerLane);
#pragma unroll
            for (int i = 0; i < BATCH; ++i) {
                double k[kElemsPerLane];
                decode_key<kBf16>(raw[i], k);
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    double acc = 0.0;
#pragma unroll
                    for (int j = 0; j < kElemsPerLane; ++j) acc = __builtin_fma(q[h][j], k[j], acc);
                    const double dot = sum8(acc);
                    if (live >> i & 1u) best[h] = max_no_nan(best[h], dot * scale);
                }
            }
        }
    }
    // Max over the 8 key slots (lanes sub, sub + 8, ..., sub + 56).
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        best[h] = max_no_nan(best[h], shfl_xor_f64(best[h], 8));
        best[h] = max_no_nan(best[h], shfl_xor_f64(best[h], 16));
        best[h] = max_no_nan(best[h], shfl_xor_f64(best[h], 32));
    }
    __shared__ double part_best[kWavesPerBlock][NH];
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < NH; ++h) part_best[wave][h] = best[h];
    }
    __syncthreads();
    if (lane == 0 && part == 0 && item_ok) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            double m = best[h];
#pragma unroll
            for (int k = 1; k < kParts; ++k) m = max_no_nan(m, part_best[wave + k][h]);
            a.out[((int64_t)(a.head0 + h) * a.T + t) * a.max_blocks + b] = m;
        }
    }
}

// ------------------------------------------------------------------ batch-in-page score kernel

// The common layout (pages of a multiple of 64 tokens, selection blocks of a multiple of 64 tokens
// and at most 64 batches): one wave per (token, block), scoring the block in batches of 8
// (step, head) items per lane: NH heads x 8 / NH steps of 8 keys, i.e. 32 or 64 consecutive
// positions, which never cross a page, so one page-table entry and one scalar row base serve a
// batch.  Two batches' loads are in flight at a time.
//
// The 8 lanes of a key each hold a partial dot product of every item.  Instead of summing each item
// over the 8 lanes (three exchange-and-add steps per item), the items are summed with a
// reduce-scatter: three steps that halve the number of values a lane carries (4 + 2 + 1 exchanges
// and additions for 8 items instead of 24), after which lane L of the group holds the full dot
// product of one item.  For that, lane L keeps item s ^ g(L) in register slot s, where g is the
// XOR-linear map with g(1) = 1, g(2) = 2, g(4) = 7: the partners of the three steps are lanes L ^ 1,
// L ^ 2 and L ^ 7 (the last being the DPP half-row mirror), and each step adds one of the lane's
// slots to the partner's other slot, which holds the same item, with no selects.  The per-lane slot
// order costs nothing: lane L loads the key of step i ^ (g(L) >> 1) (NH = 2; i ^ g(L) for NH = 1)
// into batch slot i, and the query of head h ^ (g(L) & 1) into query slot h.  Each item is still an
// exact binary64 dot product, so the block scores are those of the other kernel, bit for bit.
__device__ __forceinline__ int slot_map(int sub) { return (sub & 3) ^ ((sub & 4) ? 7 : 0); }

template <bool kBf16, int BATCH>
struct Batch {
    KeyRaw<kBf16> raw[BATCH];
    int32_t pg;
};

// Three waves per SIMD: the queries (binary64) and two batches of raw keys fit 168 registers
// without spilling; measured 15% faster than the per-key-reduction kernel at four waves per SIMD.
template <int NH, bool kBf16>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3, 3)))
void index_scores_rs_kernel(const ScoreArgs a)
{
    constexpr int BATCH = 8 / NH;                          // steps per batch
    constexpr int kBatchPos = BATCH * kKeysPerStep;        // 32 or 64 positions
    // One bf16 head's batch holds 64 raw registers: two of them would not fit.
    constexpr bool kPairs = !(kBf16 && NH == 1);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // Block-major item order, as in the other kernel.
    const uint32_t item = blockIdx.x * kWavesPerBlock + (uint32_t)wave;
    if (item >= (uint32_t)a.T * (uint32_t)a.max_blocks) return;          // wave-uniform
    const int32_t b = (int32_t)(item / (uint32_t)a.T);
    const int32_t t = (int32_t)(item - (uint32_t)b * (uint32_t)a.T);
    const int ks = lane / kLanesPerKey;
    const int sub = lane % kLanesPerKey;
    const int g = slot_map(sub);
    const int g_head = NH == 2 ? (g & 1) : 0;
    const int g_step = NH == 2 ? (g >> 1) : g;

    // The query rows go out first (their address needs only t), then the token metadata.
    uint4 qraw[NH][2];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const uint16_t* qp = a.iq + ((int64_t)t * a.hiq + a.head0 + (h ^ g_head)) * kHeadDim + sub * kElemsPerLane;
        qraw[h][0] = reinterpret_cast<const uint4*>(qp)[0];
        qraw[h][1] = reinterpret_cast<const uint4*>(qp)[1];
    }
    const int32_t pos = a.pos[t];
    const int32_t sq = a.seq[t];
    const int64_t p0_64 = (int64_t)b * a.block_tokens;
    const int32_t p0 = (int32_t)min(p0_64, (int64_t)INT32_MAX);   // exact whenever the block is scored
    const int32_t p_end = (int32_t)min(p0_64 + a.block_tokens, (int64_t)pos + 1);
    // Own slot and the page-table entries of the block's batches (lane j: batch j), requested together.
    int32_t own_off, unused;
    const int64_t own_pg = page_of(a, sq, pos, &own_off);
    int32_t batch_pg = -1;
    {
        const int64_t ps = p0_64 + (int64_t)lane * kBatchPos;
        if (ps < p_end) batch_pg = (int32_t)page_of(a, sq, (int32_t)ps, &unused);
    }
    double best = -INFINITY;      // lane L: head g(L) & 1 (NH = 2)

    if (own_pg >= 0 && p0_64 <= pos) {
        const double scale = kBf16 ? 1.0 : (double)*a.ik.scale;
        const int64_t head_off = (int64_t)(a.head0 / a.group) * a.ik.sh;
        const int64_t st = a.ik.st;
        const int32_t n_batches = (p_end - p0 + kBatchPos - 1) / kBatchPos;
        // Loads of batch j.  Past the last batch, and for a batch without a page, the pool's first
        // row is read (a valid address) and discarded.
        auto fetch = [&](int32_t j) {
            Batch<kBf16, BATCH> bt;
            const int32_t pb = p0 + j * kBatchPos;
            bt.pg = j < n_batches ? __builtin_amdgcn_readlane(batch_pg, j & (kWave - 1)) : -1;
            const int32_t lp = a.page_shift >= 0 ? pb >> a.page_shift : pb / a.page_size;
            const int32_t off0 = pb - lp * a.page_size;
            // A wave-uniform batch base plus the lane's 32-bit offset within the batch (the host checks
            // that a batch spans less than 2 GiB): the loads take the base from scalar registers.
            constexpr int kEs = kBf16 ? 2 : 1;
            const int64_t base = bt.pg >= 0 ? (int64_t)bt.pg * a.ik.sp + head_off + (int64_t)off0 * st : 0;
            const uint8_t* sb = a.ik.data + base * kEs;
            const uint32_t st_b = bt.pg >= 0 ? (uint32_t)st * kEs : 0u;
#pragma unroll
            for (int i = 0; i < BATCH; ++i) {
                const uint32_t key = (uint32_t)((i ^ g_step) * kKeysPerStep + ks);       // within the batch
                const uint8_t* src = sb + (key * st_b + (uint32_t)(sub * kElemsPerLane * kEs));
                bt.raw[i] = load_key_at<kBf16>(src);
            }
            return bt;
        };
        double qs[NH][kElemsPerLane];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const uint32_t w[8] = {qraw[h][0].x, qraw[h][0].y, qraw[h][0].z, qraw[h][0].w,
                                   qraw[h][1].x, qraw[h][1].y, qraw[h][1].z, qraw[h][1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                qs[h][2 * i] = (double)__uint_as_float(w[i] << 16);
                qs[h][2 * i + 1] = (double)__uint_as_float(w[i] & 0xffff0000u);
            }
        }
        // Sums batch j (its loads in bt) into this lane's running maximum.
        auto consume = [&](const Batch<kBf16, BATCH>& bt, int32_t j) {
            double acc[BATCH][NH];
#pragma unroll
            for (int i = 0; i < BATCH; ++i)
#pragma unroll
                for (int h = 0; h < NH; ++h) acc[i][h] = 0.0;
#pragma unroll
            for (int i = 0; i < BATCH; ++i) {
                // four elements at a time (keeps the decoded values few)
#pragma unroll
                for (int e4 = 0; e4 < kElemsPerLane / 4; ++e4) {
                    double k[4];
                    if (kBf16) {
                        const uint32_t w0 = bt.raw[i].w[2 * e4], w1 = bt.raw[i].w[2 * e4 + 1];
                        k[0] = (double)__uint_as_float(w0 << 16);
                        k[1] = (double)__uint_as_float(w0 & 0xffff0000u);
                        k[2] = (double)__uint_as_float(w1 << 16);
                        k[3] = (double)__uint_as_float(w1 & 0xffff0000u);
                    } else {
                        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)bt.raw[i].w[e4], false);
                        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)bt.raw[i].w[e4], true);
                        k[0] = (double)lo[0];
                        k[1] = (double)lo[1];
                        k[2] = (double)hi[0];
                        k[3] = (double)hi[1];
                    }
#pragma unroll
                    for (int h = 0; h < NH; ++h)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[i][h] = __builtin_fma(qs[h][4 * e4 + e], k[e], acc[i][h]);
                }
            }
            // Slot s = NH * i + h.  Reduce-scatter over the 8 lanes of the key.
            double v8[8];
#pragma unroll
            for (int i = 0; i < BATCH; ++i)
#pragma unroll
                for (int h = 0; h < NH; ++h) v8[NH * i + h] = acc[i][h];
            double v4[4], v2[2];
#pragma unroll
            for (int m = 0; m < 4; ++m) v4[m] = v8[2 * m] + dpp_f64<0xb1>(v8[2 * m + 1]);     // partner L ^ 1
#pragma unroll
            for (int m = 0; m < 2; ++m) v2[m] = v4[2 * m] + dpp_f64<0x4e>(v4[2 * m + 1]);     // partner L ^ 2
            const double dot = v2[0] + dpp_f64<0x141>(v2[1]);                                 // partner L ^ 7
            const int32_t p = p0 + j * kBatchPos + g_step * kKeysPerStep + ks;   // this lane's key
            if (bt.pg >= 0 && p < p_end) best = max_no_nan(best, dot * scale);
        };
        if (kPairs) {
            // Two batches' loads in flight together; past the last batch the second reads a
            // discarded row.
            for (int32_t j = 0; j < n_batches; j += 2) {
                const Batch<kBf16, BATCH> A = fetch(j);
                const Batch<kBf16, BATCH> B = fetch(j + 1);
                consume(A, j);
                consume(B, j + 1);
            }
        } else {
            for (int32_t j = 0; j < n_batches; ++j) consume(fetch(j), j);
        }
    }
    // Max over the lanes that hold the same head: the 8 key slots (lanes ^ 8, 16, 32) and, within a
    // key's lanes, those with the same g & 1 (NH = 2: L, L ^ 2, L ^ 5, L ^ 7; NH = 1: all 8).
    best = max_no_nan(best, shfl_xor_f64(best, 8));
    best = max_no_nan(best, shfl_xor_f64(best, 16));
    best = max_no_nan(best, shfl_xor_f64(best, 32));
    if (NH == 2) {
        best = max_no_nan(best, shfl_xor_f64(best, 2));
        best = max_no_nan(best, shfl_xor_f64(best, 5));
    } else {
        best = max_no_nan(best, shfl_xor_f64(best, 1));
        best = max_no_nan(best, shfl_xor_f64(best, 2));
        best = max_no_nan(best, shfl_xor_f64(best, 4));
    }
    // Lane h (h < NH) now holds head h's maximum: g(0) = 0, g(1) = 1.
    if (lane < NH) a.out[((int64_t)(a.head0 + lane) * a.T + t) * a.max_blocks + b] = best;
}

// ------------------------------------------------------------------ grouped score kernel

// Tokens that read the same keys (a verify window: the 1 + draft_len consecutive positions of one
// sequence) are scored together: one wave per (group of G consecutive tokens, block) computes the
// dot products of every (token, head) query of the group (G x NH <= 8 items) with each key it loads,
// so a key is loaded and decoded once per group instead of once per token.
//
// 16 lanes per key (8 elements each), 4 keys per step.  Every lane holds all 8 queries' 8 elements
// in binary64 (128 registers) and forms the 8 partial dot products of its key; the items are summed
// over the key's 16 lanes with the reduce-scatter of the batch kernel extended by one step: lane L
// keeps item s ^ g(L & 7) in slot s (queries loaded in that order), three exchanges within each
// 8-lane half (partners L ^ 1, L ^ 2, L ^ 7) leave lane L with item g(L & 7) summed over its half,
// and a fourth (partner L ^ 8, the DPP row rotation by 8) adds the other half, which holds the same
// item.  Each dot product is still the exact binary64 sum, so the block scores equal the per-token
// kernels' bit for bit.
//
// The keys a pass loads are those of one sequence; the group's tokens of that sequence are scored in
// the pass (a key counts for token i only up to its own position), the others in later passes, so
// any grouping of tokens gives the per-token result; a verify window takes one pass.
constexpr int kGLanes = 16;                       // lanes per key
constexpr int kGKeys = kWave / kGLanes;           // keys per step
constexpr int kGElems = kHeadDim / kGLanes;       // elements per lane
constexpr int kGItems = 8;                        // (token, head) queries per wave
constexpr int kGSteps = 8;                        // steps per batch
constexpr int kGBatchPos = kGSteps * kGKeys;      // 32 positions, never across a page
constexpr int kMaxGroupTokens = 8;

template <bool kBf16>
struct GKeyRaw {
    uint32_t w[kBf16 ? 4 : 2];
};

template <bool kBf16>
struct GBatch {
    GKeyRaw<kBf16> raw[kGSteps];
    int32_t pg;
};

template <int NH, bool kBf16>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2, 2)))
void index_scores_group_kernel(const ScoreArgs a, int32_t group, int32_t n_groups)
{
    // Single-head bf16 batches hold 32 raw registers each; two would not fit beside the queries.
    constexpr bool kPairs = !kBf16;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t item = blockIdx.x * kWavesPerBlock + (uint32_t)wave;   // block-major, as the others
    if (item >= (uint32_t)n_groups * (uint32_t)a.max_blocks) return;      // wave-uniform
    const int32_t b = (int32_t)(item / (uint32_t)n_groups);
    const int32_t t0 = (int32_t)(item - (uint32_t)b * (uint32_t)n_groups) * group;
    const int ks = lane / kGLanes;
    const int sub = lane % kGLanes;
    const int g = slot_map(sub & 7);                  // this lane's item after the reduce-scatter
    const int n_items = group * NH;                   // <= kGItems

    // Queries first: slot s holds item s ^ g (token (s ^ g) / NH, head (s ^ g) % NH); slots past the
    // group's items (or past T) read token t0's first head and are never counted.
    uint4 qraw[kGItems];
#pragma unroll
    for (int s = 0; s < kGItems; ++s) {
        const int j = s ^ g;
        const int ti = j < n_items ? j / NH : 0;
        const int h = j < n_items ? j % NH : 0;
        const int32_t t = min(t0 + ti, a.T - 1);
        qraw[s] = *reinterpret_cast<const uint4*>(a.iq + ((int64_t)t * a.hiq + a.head0 + h) * kHeadDim + sub * kGElems);
    }
    // The group's token metadata, lane i for token t0 + i; then wave-uniform copies.
    int32_t m_pos = -1, m_seq = -1, m_ok = 0;
    if (lane < group && t0 + lane < a.T) {
        m_pos = a.pos[t0 + lane];
        m_seq = a.seq[t0 + lane];
        int32_t unused;
        m_ok = page_of(a, m_seq, m_pos, &unused) >= 0 ? 1 : 0;
    }
    uint32_t valid = 0;                               // bit i: token t0 + i has a slot of its own
    int32_t tpos[kMaxGroupTokens], tseq[kMaxGroupTokens];
#pragma unroll
    for (int i = 0; i < kMaxGroupTokens; ++i) {
        tpos[i] = __builtin_amdgcn_readlane(m_pos, i);
        tseq[i] = __builtin_amdgcn_readlane(m_seq, i);
        valid |= (uint32_t)(__builtin_amdgcn_readlane(m_ok, i) & (i < group ? 1 : 0)) << i;
    }
    // This lane's item: its token and position (selected by value, no indexed registers).
    const int my_tok = g < n_items ? g / NH : kMaxGroupTokens;
    int32_t my_pos = -1;
#pragma unroll
    for (int i = 0; i < kMaxGroupTokens; ++i) my_pos = my_tok == i ? tpos[i] : my_pos;

    double qs[kGItems][kGElems];
#pragma unroll
    for (int s = 0; s < kGItems; ++s) {
        const uint32_t w[4] = {qraw[s].x, qraw[s].y, qraw[s].z, qraw[s].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qs[s][2 * i] = (double)__uint_as_float(w[i] << 16);
            qs[s][2 * i + 1] = (double)__uint_as_float(w[i] & 0xffff0000u);
        }
    }
    const double scale = kBf16 ? 1.0 : (double)*a.ik.scale;
    const int64_t head_off = (int64_t)(a.head0 / a.group) * a.ik.sh;
    const int64_t p0_64 = (int64_t)b * a.block_tokens;
    const int32_t p0 = (int32_t)min(p0_64, (int64_t)INT32_MAX);   // exact whenever the block is scored
    double best = -INFINITY;                          // item g of this lane

    uint32_t done = 0;
    for (int pass = 0; pass < kMaxGroupTokens; ++pass) {                   // wave-uniform
        const uint32_t left = valid & ~done;
        if (!left) break;
        const int lead = __builtin_ctz(left);
        int32_t pass_seq = tseq[0];
#pragma unroll
        for (int i = 1; i < kMaxGroupTokens; ++i) pass_seq = lead == i ? tseq[i] : pass_seq;
        uint32_t act = 0;
        int32_t max_pos = -1;
#pragma unroll
        for (int i = 0; i < kMaxGroupTokens; ++i) {
            const bool in = (left >> i & 1u) && tseq[i] == pass_seq;
            act |= (in ? 1u : 0u) << i;
            max_pos = in && tpos[i] > max_pos ? tpos[i] : max_pos;
        }
        done |= act;
        const bool mine = my_tok < kMaxGroupTokens && (act >> my_tok & 1u);   // this lane's item scored now
        const int32_t p_end = (int32_t)min(p0_64 + a.block_tokens, (int64_t)max_pos + 1);
        if (p0_64 >= p_end) continue;
        // Page-table entries of the pass's batches (lane j: batch j), one request.
        int32_t batch_pg = -1;
        {
            const int64_t ps = p0_64 + (int64_t)lane * kGBatchPos;
            int32_t unused;
            if (ps < p_end) batch_pg = (int32_t)page_of(a, pass_seq, (int32_t)ps, &unused);
        }
        const int32_t n_batches = (p_end - p0 + kGBatchPos - 1) / kGBatchPos;
        auto fetch = [&](int32_t j) {
            GBatch<kBf16> bt;
            const int32_t pb = p0 + j * kGBatchPos;
            bt.pg = j < n_batches ? __builtin_amdgcn_readlane(batch_pg, j & (kWave - 1)) : -1;
            const int32_t lp = a.page_shift >= 0 ? pb >> a.page_shift : pb / a.page_size;
            const int32_t off0 = pb - lp * a.page_size;
            constexpr int kEs = kBf16 ? 2 : 1;
            const int64_t base = bt.pg >= 0 ? (int64_t)bt.pg * a.ik.sp + head_off + (int64_t)off0 * a.ik.st : 0;
            const uint8_t* sb = a.ik.data + base * kEs;
            const uint32_t st_b = bt.pg >= 0 ? (uint32_t)a.ik.st * kEs : 0u;
#pragma unroll
            for (int i = 0; i < kGSteps; ++i) {
                const uint32_t key = (uint32_t)(i * kGKeys + ks);
                const uint8_t* src = sb + (key * st_b + (uint32_t)(sub * kGElems * kEs));
                if (kBf16) {
                    const uint4 v = *reinterpret_cast<const uint4*>(src);
                    bt.raw[i].w[0] = v.x; bt.raw[i].w[kBf16 ? 1 : 0] = v.y;
                    bt.raw[i].w[kBf16 ? 2 : 0] = v.z; bt.raw[i].w[kBf16 ? 3 : 0] = v.w;
                } else {
                    const uint2 v = *reinterpret_cast<const uint2*>(src);
                    bt.raw[i].w[0] = v.x; bt.raw[i].w[1] = v.y;
                }
            }
            return bt;
        };
        auto consume = [&](const GBatch<kBf16>& bt, int32_t j) {
#pragma unroll
            for (int i = 0; i < kGSteps; ++i) {
                double k[kGElems];
                if (kBf16) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        k[2 * e] = (double)__uint_as_float(bt.raw[i].w[e] << 16);
                        k[2 * e + 1] = (double)__uint_as_float(bt.raw[i].w[e] & 0xffff0000u);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)bt.raw[i].w[e], false);
                        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)bt.raw[i].w[e], true);
                        k[4 * e] = (double)lo[0];
                        k[4 * e + 1] = (double)lo[1];
                        k[4 * e + 2] = (double)hi[0];
                        k[4 * e + 3] = (double)hi[1];
                    }
                }
                double v8[kGItems];
#pragma unroll
                for (int s = 0; s < kGItems; ++s) {
                    double acc = 0.0;
#pragma unroll
                    for (int e = 0; e < kGElems; ++e) acc = __builtin_fma(qs[s][e], k[e], acc);
                    v8[s] = acc;
                }
                double v4[4], v2[2];
#pragma unroll
                for (int m = 0; m < 4; ++m) v4[m] = v8[2 * m] + dpp_f64<0xb1>(v8[2 * m + 1]);   // partner L ^ 1
#pragma unroll
                for (int m = 0; m < 2; ++m) v2[m] = v4[2 * m] + dpp_f64<0x4e>(v4[2 * m + 1]);   // partner L ^ 2
                const double half = v2[0] + dpp_f64<0x141>(v2[1]);                             // partner L ^ 7
                const double dot = half + dpp_f64<0x128>(half);                                // partner L ^ 8
                const int32_t p = p0 + j * kGBatchPos + i * kGKeys + ks;                       // this lane's key
                if (mine && bt.pg >= 0 && p < p_end && p <= my_pos) best = max_no_nan(best, dot * scale);
            }
        };
        if (kPairs) {
            for (int32_t j = 0; j < n_batches; j += 2) {
                const GBatch<kBf16> A = fetch(j);
                const GBatch<kBf16> B = fetch(j + 1);
                consume(A, j);
                consume(B, j + 1);
            }
        } else {
            for (int32_t j = 0; j < n_batches; ++j) consume(fetch(j), j);
        }
    }
    // Max over the lanes that hold the same item: the other half of the key's lanes and the other key
    // slots.  Lane L < 8 then holds item g(L)'s maximum.
    best = max_no_nan(best, shfl_xor_f64(best, 8));
    best = max_no_nan(best, shfl_xor_f64(best, 16));
    best = max_no_nan(best, shfl_xor_f64(best, 32));
    if (lane < 8 && g < n_items) {
        const int32_t t = t0 + g / NH;
        if (t < a.T) a.out[((int64_t)(a.head0 + g % NH) * a.T + t) * a.max_blocks + b] = best;
    }
}

// (score, index) order of the selection: higher score first, then lower index.
__device__ __forceinline__ bool before(double s1, int32_t i1, double s2, int32_t i2)
{
    return s1 > s2 || (s1 == s2 && i1 < i2);
}

// Rows of up to kRankRowBlocks blocks: one 512-thread work-group per row stages the row in LDS
// (padded with -inf) and computes the rank of every candidate (how many candidates are ordered
// before it); a candidate of rank r < top_k is the r-th pick, with no serial rounds.  S threads share
// a candidate (S = 4 up to 128 blocks, 2 up to 256, else 1), each comparing it against every S-th
// pair of entries, and their counts are summed over the S lanes.
template <int S>
__global__ __launch_bounds__(kRankThreads) void index_topk_rank_kernel(const double* scores, int32_t rows, int32_t nb,
                                                                        int32_t top_k, int32_t* ids, int32_t* counts)
{
    static_assert(S == 1 || S == 2 || S == 4, "1, 2 or 4 threads per candidate");
    constexpr int kCands = kRankThreads / S;            // candidates per pass
    __shared__ __attribute__((aligned(16))) double row_lds[kRankRowBlocks + 2 * S];
    __shared__ int32_t n_lds[kRankThreads / kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int32_t r = (int32_t)blockIdx.x;
    if (r >= rows) return;   // uniform over the work-group
    const double* row = scores + (int64_t)r * nb;
    const int32_t npad = (nb + 2 * S - 1) / (2 * S) * (2 * S);   // whole pairs for every thread of a candidate
    int n_local = 0;
    for (int32_t i0 = 0; i0 < npad; i0 += kRankThreads) {
        const int32_t i = i0 + tid;
        const double v = i < nb ? row[i] : -INFINITY;
        const bool cand = v > -INFINITY;              // -inf and NaN are never picked
        if (i < npad) row_lds[i] = cand ? v : -INFINITY;
        n_local += __popcll(__ballot(cand));          // the wave's candidates, counted once per wave
    }
    if (lane == 0) n_lds[wave] = n_local;
    __syncthreads();
    int32_t n = 0;
#pragma unroll
    for (int w = 0; w < kRankThreads / kWave; ++w) n += n_lds[w];
    const int32_t picked = n < top_k ? n : top_k;
    int32_t* out = ids + (int64_t)r * top_k;
    for (int32_t k = picked + tid; k < top_k; k += kRankThreads) out[k] = -1;
    const int part = tid % S;
    const int32_t n_pairs = npad / (2 * S);           // pairs per thread
    const double2* rp = reinterpret_cast<const double2*>(row_lds) + part;
    for (int32_t c0 = 0; c0 < nb; c0 += kCands) {     // uniform over the work-group
        const int32_t i = c0 + tid / S;
        const double si = i < nb ? row_lds[i] : -INFINITY;
        int32_t rank = 0;
#pragma unroll 8
        for (int32_t m = 0; m < n_pairs; ++m) {       // -inf entries never count
            const double2 sj = rp[S * m];
            const int32_t j = 2 * (S * m + part);
            rank += (sj.x > si || (sj.x == si && j < i)) ? 1 : 0;
            rank += (sj.y > si || (sj.y == si && j + 1 < i)) ? 1 : 0;
        }
        if (S >= 2) rank += __shfl_xor(rank, 1);
        if (S >= 4) rank += __shfl_xor(rank, 2);
        if (part == 0 && si > -INFINITY && rank < top_k) out[rank] = i;
    }
    if (counts && tid == 0) counts[r] = picked;
}

// Longer rows: one wavefront per row, top_k rounds of a wave-wide arg-max over the candidates ranked
// after the previous pick (so no pick repeats and no membership list is needed).
__global__ __launch_bounds__(kBlock) void index_topk_kernel(const double* scores, int32_t rows, int32_t nb,
                                                            int32_t top_k, int32_t* ids, int32_t* counts)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int32_t r = (int32_t)(blockIdx.x * kWavesPerBlock + wave);
    if (r >= rows) return;   // wave-uniform
    const double* row = scores + (int64_t)r * nb;
    double last_s = INFINITY;
    int32_t last_i = -1;
    int32_t my_id = -1;   // lane k keeps the k-th pick
    int32_t n = 0;
    for (int32_t k = 0; k < top_k; ++k) {
        double bs = -INFINITY;
        int32_t bi = -1;
        for (int32_t i = lane; i < nb; i += kWave) {
            const double s = row[i];
            if (!(s > -INFINITY)) continue;                       // -inf and NaN are never picked
            if (!before(last_s, last_i, s, i)) continue;          // already picked (ranked before the last)
            if (bi < 0 || before(s, i, bs, bi)) { bs = s; bi = i; }
        }
#pragma unroll
        for (int m = 1; m < kWave; m <<= 1) {
            const double os = shfl_xor_f64(bs, m);
            const int32_t oi = __shfl_xor(bi, m);
            if (oi >= 0 && (bi < 0 || before(os, oi, bs, bi))) { bs = os; bi = oi; }
        }
        if (bi < 0) break;                                        // wave-uniform after the reduction
        if (lane == k) my_id = bi;
        last_s = bs;
        last_i = bi;
        ++n;
    }
    if (lane < top_k) ids[(int64_t)r * top_k + lane] = my_id;
    if (counts && lane == 0) counts[r] = n;
}

msa_status launch_topk(const double* block_scores, int32_t rows, int32_t max_blocks, int32_t top_k,
                       int32_t* block_ids, int32_t* counts, hipStream_t stream)
{
    const bool rank = max_blocks <= kRankRowBlocks;
    const dim3 grid(rank ? (unsigned)rows : (unsigned)(((int64_t)rows + kWavesPerBlock - 1) / kWavesPerBlock));
    void* args[] = {const_cast<double**>(&block_scores), &rows, &max_blocks, &top_k, &block_ids, &counts};
    const void* fn = !rank ? reinterpret_cast<const void*>(&index_topk_kernel)
                     : max_blocks <= kRankThreads / 4 ? reinterpret_cast<const void*>(&index_topk_rank_kernel<4>)
                     : max_blocks <= kRankThreads / 2 ? reinterpret_cast<const void*>(&index_topk_rank_kernel<2>)
                                                      : reinterpret_cast<const void*>(&index_topk_rank_kernel<1>);
    const hipError_t e = hipLaunchKernel(fn, grid, dim3(rank ? kRankThreads : kBlock), args, 0, stream);
    return e == hipSuccess ? MSA_OK : MSA_ERR_LAUNCH;
}

// Every check of a score call, then its kernel arguments and layout (items == 0: nothing to launch).
struct ScorePlan {
    ScoreArgs a;
    int64_t items;
    bool batch_in_page;   // pages and blocks of multiples of 64 tokens, blocks of at most 2,048
    bool in_page;         // pages and blocks of multiples of 8 tokens
};

msa_status prepare_scores(const uint16_t* iq, int32_t num_tokens, int32_t head_dim, int32_t num_iq_heads,
                          const int32_t* positions, const int32_t* seq_idx,
                          const int32_t* page_table, int64_t page_table_stride, int32_t num_seqs,
                          int32_t max_pages_per_seq, int32_t page_size, int64_t num_pages,
                          const msa_cache_view* ik_cache, int32_t block_tokens, int32_t max_blocks,
                          double* block_scores, hipStream_t s, ScorePlan* plan)
{
    if (head_dim != kHeadDim) return MSA_ERR_UNSUPPORTED;
    if (num_tokens < 0 || num_iq_heads < 1 || num_iq_heads > 4096 || block_tokens <= 0 || max_blocks < 0)
        return MSA_ERR_SHAPE;
    if (page_size <= 0 || num_seqs < 0 || max_pages_per_seq < 0 || num_pages < 0) return MSA_ERR_SHAPE;
    if (num_seqs > 0 && page_table_stride < max_pages_per_seq) return MSA_ERR_STRIDE;
    if (!ik_cache) return MSA_ERR_NULL_POINTER;
    const int32_t hik = ik_cache->num_heads;
    if (hik < 1 || num_iq_heads % hik) return MSA_ERR_SHAPE;
    CacheDev ik;
    uint64_t ik_span;
    const msa_status st = check_cache(ik_cache, hik, page_size, num_pages, &ik, true, &ik_span);
    if (st != MSA_OK) return st;
    if (num_tokens > 0 && max_blocks > 0) {
        if (!iq || !positions || !seq_idx || !block_scores) return MSA_ERR_NULL_POINTER;
        if (num_seqs > 0 && max_pages_per_seq > 0 && !page_table) return MSA_ERR_NULL_POINTER;
    }
    if (!aligned(iq, 16) || !aligned(positions, 4) || !aligned(seq_idx, 4) || !aligned(page_table, 4) ||
        !aligned(block_scores, 8))
        return MSA_ERR_ALIGNMENT;
    if ((int64_t)max_blocks * block_tokens > 0x80000000LL) return MSA_ERR_SHAPE;   // block starts fit in int32
    int64_t items, tmp;
    if (__builtin_mul_overflow((int64_t)num_tokens, (int64_t)max_blocks, &items) || items + kWavesPerBlock > 0x7fffffffLL)
        return MSA_ERR_SHAPE;
    if (num_seqs > 0 && __builtin_mul_overflow((int64_t)num_seqs, page_table_stride, &tmp)) return MSA_ERR_OVERFLOW;
    plan->items = items;
    if (items == 0) return MSA_OK;

    ScoreArgs& a = plan->a;
    std::memset(&a, 0, sizeof(a));
    a.iq = iq;
    a.pos = positions;
    a.seq = seq_idx;
    a.pt = page_table;
    a.pt_stride = page_table_stride;
    a.num_pages = num_pages;
    a.T = num_tokens;
    a.S = num_seqs;
    a.max_pages = max_pages_per_seq;
    a.page_size = page_size;
    a.page_shift = (page_size & (page_size - 1)) == 0 ? __builtin_ctz((unsigned)page_size) : -1;
    a.hiq = num_iq_heads;
    a.group = num_iq_heads / hik;
    a.block_tokens = block_tokens;
    a.max_blocks = max_blocks;
    a.ik = ik;
    a.out = block_scores;
    // Batches of 32 / 64 positions never cross a page, and the parts start on batch boundaries.
    plan->batch_in_page = page_size % 64 == 0 && block_tokens % 64 == 0 && block_tokens <= 64 * 32 &&
                          (int64_t)64 * ik.st * (ik.is_bf16 ? 2 : 1) + 256 <= 0x7fffffffLL;
    plan->in_page = page_size % kKeysPerStep == 0 && block_tokens % kKeysPerStep == 0;
    const Span spans[] = {
        {iq, nbytes((int64_t)num_tokens * num_iq_heads * kHeadDim, 2)},
        {positions, nbytes(num_tokens, 4)},
        {seq_idx, nbytes(num_tokens, 4)},
        {page_table, num_seqs > 0 ? row_bytes(num_seqs, page_table_stride, max_pages_per_seq, 4) : 0},
        {ik.data, ik_span},
        {ik.scale, 4},
        {block_scores, nbytes((int64_t)num_iq_heads * items, 8)},
    };
    return check_operands(spans, sizeof(spans) / sizeof(spans[0]), s);
}

// Per-token kernels: one launch per pair of index-Q heads that read the same index-K head (two heads'
// queries fit the registers at once).
msa_status launch_scores(ScorePlan& p, hipStream_t s)
{
    ScoreArgs& a = p.a;
    const int items_per_group = p.batch_in_page ? kWavesPerBlock : kWavesPerBlock / kParts;
    const dim3 grid((unsigned)((p.items + items_per_group - 1) / items_per_group));
    const bool bf = a.ik.is_bf16;
    for (int32_t h0 = 0; h0 < a.hiq;) {
        const int32_t group_end = (h0 / a.group + 1) * a.group;
        const int nh = (group_end - h0 >= kMaxHeadsPerLaunch) ? kMaxHeadsPerLaunch : 1;
        a.head0 = h0;
        void* args[] = {&a};
        const void* fn;
        if (p.batch_in_page)
            fn = bf ? (nh == 2 ? reinterpret_cast<const void*>(&index_scores_rs_kernel<2, true>)
                               : reinterpret_cast<const void*>(&index_scores_rs_kernel<1, true>))
                    : (nh == 2 ? reinterpret_cast<const void*>(&index_scores_rs_kernel<2, false>)
                               : reinterpret_cast<const void*>(&index_scores_rs_kernel<1, false>));
        else if (p.in_page)
            fn = bf ? (nh == 2 ? reinterpret_cast<const void*>(&index_scores_kernel<2, true, true>)
                               : reinterpret_cast<const void*>(&index_scores_kernel<1, true, true>))
                    : (nh == 2 ? reinterpret_cast<const void*>(&index_scores_kernel<2, false, true>)
                               : reinterpret_cast<const void*>(&index_scores_kernel<1, false, true>));
        else
            fn = bf ? (nh == 2 ? reinterpret_cast<const void*>(&index_scores_kernel<2, true, false>)
                               : reinterpret_cast<const void*>(&index_scores_kernel<1, true, false>))
                    : (nh == 2 ? reinterpret_cast<const void*>(&index_scores_kernel<2, false, false>)
                               : reinterpret_cast<const void*>(&index_scores_kernel<1, false, false>));
        const hipError_t e = hipLaunchKernel(fn, grid, dim3(kBlock), args, 0, s);
        if (e != hipSuccess) return MSA_ERR_LAUNCH;
        h0 += nh;
    }
    return MSA_OK;
}

// Grouped kernel: groups of `group` tokens, two index-Q heads per launch where the group and the
// head grouping allow it (group x heads <= 8 items), else one.
msa_status launch_scores_grouped(ScorePlan& p, int32_t group, hipStream_t s)
{
    ScoreArgs& a = p.a;
    const int32_t n_groups = (a.T + group - 1) / group;
    const int64_t waves = (int64_t)n_groups * a.max_blocks;
    const dim3 grid((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock));
    const bool bf = a.ik.is_bf16;
    for (int32_t h0 = 0; h0 < a.hiq;) {
        const int32_t group_end = (h0 / a.group + 1) * a.group;
        const int nh = (group_end - h0 >= 2 && 2 * group <= kGItems) ? 2 : 1;
        a.head0 = h0;
        void* args[] = {&a, &group, const_cast<int32_t*>(&n_groups)};
        const void* fn = bf ? (nh == 2 ? reinterpret_cast<const void*>(&index_scores_group_kernel<2, true>)
                                       : reinterpret_cast<const void*>(&index_scores_group_kernel<1, true>))
                            : (nh == 2 ? reinterpret_cast<const void*>(&index_scores_group_kernel<2, false>)
                                       : reinterpret_cast<const void*>(&index_scores_group_kernel<1, false>));
        const hipError_t e = hipLaunchKernel(fn, grid, dim3(kBlock), args, 0, s);
        if (e != hipSuccess) return MSA_ERR_LAUNCH;
        h0 += nh;
    }
    return MSA_OK;
}

}  // namespace

extern "C" {

msa_status msa_index_scores(const uint16_t* iq, int32_t num_tokens, int32_t head_dim, int32_t num_iq_heads,
                            const int32_t* positions, const int32_t* seq_idx,
                            const int32_t* page_table, int64_t page_table_stride, int32_t num_seqs,
                            int32_t max_pages_per_seq, int32_t page_size, int64_t num_pages,
                            const msa_cache_view* ik_cache, int32_t block_tokens, int32_t max_blocks,
                            double* block_scores, void* stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    ScorePlan p;
    const msa_status st = prepare_scores(iq, num_tokens, head_dim, num_iq_heads, positions, seq_idx, page_table,
                                         page_table_stride, num_seqs, max_pages_per_seq, page_size, num_pages,
                                         ik_cache, block_tokens, max_blocks, block_scores, s, &p);
    if (st != MSA_OK || p.items == 0) return st;
    return launch_scores(p, s);
}

msa_status msa_index_scores_grouped(const uint16_t* iq, int32_t num_tokens, int32_t head_dim, int32_t num_iq_heads,
                                    const int32_t* positions, const int32_t* seq_idx,
                                    const int32_t* page_table, int64_t page_table_stride, int32_t num_seqs,
                                    int32_t max_pages_per_seq, int32_t page_size, int64_t num_pages,
                                    const msa_cache_view* ik_cache, int32_t block_tokens, int32_t max_blocks,
                                    int32_t group_tokens, double* block_scores, void* stream)
{
    if (group_tokens < 1 || group_tokens > kMaxGroupTokens) return MSA_ERR_SHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    ScorePlan p;
    const msa_status st = prepare_scores(iq, num_tokens, head_dim, num_iq_heads, positions, seq_idx, page_table,
                                         page_table_stride, num_seqs, max_pages_per_seq, page_size, num_pages,
                                         ik_cache, block_tokens, max_blocks, block_scores, s, &p);
    if (st != MSA_OK || p.items == 0) return st;
    // One token per group, or a layout the grouped kernel does not take: the per-token kernels.
    if (group_tokens == 1 || !p.batch_in_page) return launch_scores(p, s);
    return launch_scores_grouped(p, group_tokens, s);
}

msa_status msa_index_topk(const double* block_scores, int32_t rows, int32_t max_blocks, int32_t top_k,
                          int32_t* block_ids, int32_t* counts, void* stream)
{
    if (rows < 0 || max_blocks < 0 || max_blocks > kMaxRowBlocks || top_k < 1 || top_k > kMaxTopK)
        return MSA_ERR_SHAPE;
    if (rows == 0) return MSA_OK;
    if (!block_ids || (max_blocks > 0 && !block_scores)) return MSA_ERR_NULL_POINTER;
    if (!aligned(block_scores, 8) || !aligned(block_ids, 4) || !aligned(counts, 4)) return MSA_ERR_ALIGNMENT;
    const Span spans[] = {{block_scores, nbytes((int64_t)rows * max_blocks, 8)},
                          {block_ids, nbytes((int64_t)rows * top_k, 4)},
                          {counts, nbytes(rows, 4)}};
    const msa_status st = check_operands(spans, 3, static_cast<hipStream_t>(stream));
    if (st != MSA_OK) return st;
    return launch_topk(block_scores, rows, max_blocks, top_k, block_ids, counts, static_cast<hipStream_t>(stream));
}

}  // extern "C"
