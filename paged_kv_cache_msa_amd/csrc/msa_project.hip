// The packed projection x = bf16(h w^T) on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16), alone or
// with the producer as its epilogue.  Operation: page "Fuse MiniMax-M3 QKV and index projection"
// (AFTER figure: one wider GEMM produces the row [Q | K | V | index-Q | index-K] that the fused
// producer consumes); the epilogue is the producer of msa_produce.hip, on the row while it is still
// in registers.
//
// Orientation.  The matrix cores compute C^T = w h^T: MFMA rows are output columns (features),
// MFMA columns are tokens.  In a 32 x 32 result block lane l holds token l % 32 and the 16 features
// 8 (i / 4) + 4 (l / 32) + i % 4, i < 16.  A wave that owns one head (4 row blocks of 32 features)
// for a block of 32 tokens therefore holds half of each token's head row in each of lanes l and
// l ^ 32: the RMSNorm sum of squares is an in-lane sum plus one exchange with lane l ^ 32, and the
// rotate-half partners (f, f + 64) sit in the same lane (row blocks b and b + 2, same register).
//
// Kernels.
//   project_splitk_kernel  up to 1,024 tokens: one work-group per (head, 64-token chunk, K slice);
//                          each wave owns 32 of the head's features for the chunk and streams its
//                          slice of w and h straight from memory into MFMA operands.  Partial sums go
//                          to the workspace; the last slice to finish for a (head, chunk) (a counter
//                          per pair) adds the slices in slice order and runs the epilogue.
//   project_tile_kernel    larger batches: 256 features (2 heads) x 256 tokens per work-group, four
//                          waves of one head x 128 tokens each, 64-wide K steps double-buffered
//                          through LDS (row pitch 144 bytes: conflict-free 16-byte fragment reads),
//                          the tile order chosen so that the work-groups of one XCD walk the feature
//                          tiles of the same token rows (their h panel stays in that XCD's L2).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "msa_common.h"
#include "msa_device.h"
#include "msa_project.h"

namespace {

using namespace msa_internal;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kSplitMaxTokens = 1024;
constexpr int kChunk = 64;                 // tokens per split-K work-group (two MFMA token blocks)
constexpr int kPartFloats = 4 * 2 * 64 * 16;   // one work-group's partial sums: [wave][tb][lane][16]
constexpr int kTile = 256;                 // tiled kernel: features and tokens per work-group
constexpr int kBK = 64;                    // K per pipeline stage
constexpr int kPitch = 72;                 // LDS row pitch in bf16 elements (144 B)
constexpr uint64_t kAlign = 256;

enum Stream { kQ = 0, kK = 1, kV = 2, kIQ = 3, kIK = 4 };

__device__ __forceinline__ f32x16_t mfma(const uint4& a, const uint4& b, const f32x16_t& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                    c, 0, 0, 0);
}

// Everything the epilogue needs.  Plain mode uses x_out / x_stride; produce mode the rest.
struct Epi {
    uint16_t* x_out;
    int64_t x_stride;
    const float* cos;          // [T, 64]
    const float* sin;
    const int64_t* slots;
    int64_t num_pages;
    const uint16_t* w[4];      // norm weights of Q, K, index-Q, index-K
    uint16_t* q_out;
    uint16_t* iq_out;
    CacheDev cache[3];         // K, V, index-K
    int32_t page_size;
    int32_t hq, hkv, hiq, hik;
    int32_t T;
    float eps;
};

// One head's row for one token per lane pair: a[b][i] is feature 32 b + 8 (i / 4) + 4 hh + i % 4
// (hh = lane / 32) of `head`, token t.  Rounds the row to bf16 (the packed row's values), then
// either stores it (plain) or runs the producer arithmetic on it.
template <bool kProduce>
__device__ __forceinline__ void epilogue(const Epi& e, int head, int32_t t, float (&a)[4][16])
{
    const int lane = threadIdx.x & 63;
    const int hh = lane >> 5;
    const bool tok = t < e.T;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t w = bf16x2(a[b][2 * j], a[b][2 * j + 1]);
            a[b][2 * j] = bf16_lo(w);
            a[b][2 * j + 1] = bf16_hi(w);
        }
    if (!kProduce) {
        if (!tok) return;
        uint16_t* dst = e.x_out + (int64_t)t * e.x_stride + head * kHeadDim + 4 * hh;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<uint2*>(dst + 32 * b + 8 * g) =
                    make_uint2(bf16x2(a[b][4 * g], a[b][4 * g + 1]), bf16x2(a[b][4 * g + 2], a[b][4 * g + 3]));
        return;
    }

    const int h_k = e.hq, h_v = e.hq + e.hkv, h_iq = e.hq + 2 * e.hkv, h_ik = h_iq + e.hiq;
    const int st = head < h_k ? kQ : head < h_v ? kK : head < h_iq ? kV : head < h_ik ? kIQ : kIK;
    if (st != kV) {
        // RMSNorm: binary64 sum of squares over the lane's 64 features plus the partner lane's.
        double ss = 0.0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) ss = __builtin_fma((double)a[b][i], (double)a[b][i], ss);
        ss += __shfl_xor(ss, 32);
        const float r = rms_from_ss(ss, e.eps);
        const uint16_t* wp = e.w[st == kQ ? 0 : st == kK ? 1 : st == kIQ ? 2 : 3] + 4 * hh;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint2 wv = *reinterpret_cast<const uint2*>(wp + 32 * b + 8 * g);
                const float w4[4] = {bf16_lo(wv.x), bf16_hi(wv.x), bf16_lo(wv.y), bf16_hi(wv.y)};
#pragma unroll
                for (int q = 0; q < 4; ++q) a[b][4 * g + q] = (a[b][4 * g + q] * r) * w4[q];
            }
        // RoPE, neox rotate-half: frequency f < 64 pairs feature f (block b) with f + 64 (block b + 2).
        const int32_t tl = tok ? t : e.T - 1;
        const float* cp = e.cos + (int64_t)tl * kHalf + 4 * hh;
        const float* sp = e.sin + (int64_t)tl * kHalf + 4 * hh;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 c4 = *reinterpret_cast<const float4*>(cp + 32 * b + 8 * g);
                const float4 s4 = *reinterpret_cast<const float4*>(sp + 32 * b + 8 * g);
                const float c[4] = {c4.x, c4.y, c4.z, c4.w}, s[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float y0 = a[b][4 * g + q], y1 = a[b + 2][4 * g + q];
                    a[b][4 * g + q] = y0 * c[q] - y1 * s[q];
                    a[b + 2][4 * g + q] = y1 * c[q] + y0 * s[q];
                }
            }
    }
    if (!tok) return;
    if (st == kQ || st == kIQ) {
        uint16_t* dst = (st == kQ ? e.q_out + ((int64_t)t * e.hq + head) * kHeadDim
                                  : e.iq_out + ((int64_t)t * e.hiq + (head - h_iq)) * kHeadDim) + 4 * hh;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<uint2*>(dst + 32 * b + 8 * g) =
                    make_uint2(bf16x2(a[b][4 * g], a[b][4 * g + 1]), bf16x2(a[b][4 * g + 2], a[b][4 * g + 3]));
        return;
    }
    const int64_t slot = e.slots[t];
    if (slot < 0) return;
    const int64_t page = slot / e.page_size;
    if (page >= e.num_pages) return;
    const int64_t off = slot - page * e.page_size;
    const int ci = st == kK ? 0 : st == kV ? 1 : 2;
    const int hl = st == kK ? head - h_k : st == kV ? head - h_v : head - h_ik;
    const CacheDev& cd = e.cache[ci];
    const int64_t base = page * cd.sp + off * cd.st + (int64_t)hl * cd.sh + 4 * hh;
    if (cd.is_bf16) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(cd.data) + base;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<uint2*>(dst + 32 * b + 8 * g) =
                    make_uint2(bf16x2(a[b][4 * g], a[b][4 * g + 1]), bf16x2(a[b][4 * g + 2], a[b][4 * g + 3]));
    } else {
        const float m = inv_scale_of(cd.scale);
        uint8_t* dst = cd.data + base;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<uint32_t*>(dst + 32 * b + 8 * g) =
                    e4m3x4(a[b][4 * g] * m, a[b][4 * g + 1] * m, a[b][4 * g + 2] * m, a[b][4 * g + 3] * m);
    }
}

// ------------------------------------------------------------------ split-K kernel (<= 1,024 tokens)

struct SplitArgs {
    const uint16_t* h;
    int64_t h_stride;
    const uint16_t* w;
    int64_t w_stride;
    float* part;               // [head][chunk][slice] x kPartFloats
    uint32_t* counters;        // [head][chunk]
    int32_t K, kc, splits, n_tc;
    Epi e;
};

template <bool kProduce>
__global__ __launch_bounds__(256) void project_splitk_kernel(const SplitArgs a)
{
    __shared__ int s_last;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // 32-feature block of the head
    const int hh = lane >> 5;
    const int split = (int)(blockIdx.x % (uint32_t)a.splits);
    const int pair = (int)(blockIdx.x / (uint32_t)a.splits);         // head * n_tc + chunk
    const int tc = pair % a.n_tc;
    const int head = pair / a.n_tc;
    const int k_begin = split * a.kc;
    const int k_end = min(a.K, k_begin + a.kc);

    const uint16_t* ap = a.w + (int64_t)(head * kHeadDim + wave * 32 + (lane & 31)) * a.w_stride + 8 * hh;
    const int32_t t0 = min(tc * kChunk + (lane & 31), a.e.T - 1);           // rows past T: read row T-1, unused
    const int32_t t1 = min(tc * kChunk + 32 + (lane & 31), a.e.T - 1);
    const uint16_t* bp0 = a.h + (int64_t)t0 * a.h_stride + 8 * hh;
    const uint16_t* bp1 = a.h + (int64_t)t1 * a.h_stride + 8 * hh;

    f32x16_t c0 = {}, c1 = {};
    uint4 av[4], b0[4], b1[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        av[s] = *reinterpret_cast<const uint4*>(ap + k_begin + 16 * s);
        b0[s] = *reinterpret_cast<const uint4*>(bp0 + k_begin + 16 * s);
        b1[s] = *reinterpret_cast<const uint4*>(bp1 + k_begin + 16 * s);
    }
    for (int k = k_begin; k < k_end; k += kBK) {
        uint4 na[4], n0[4], n1[4];
        const bool more = k + kBK < k_end;
        if (more) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                na[s] = *reinterpret_cast<const uint4*>(ap + k + kBK + 16 * s);
                n0[s] = *reinterpret_cast<const uint4*>(bp0 + k + kBK + 16 * s);
                n1[s] = *reinterpret_cast<const uint4*>(bp1 + k + kBK + 16 * s);
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            c0 = mfma(av[s], b0[s], c0);
            c1 = mfma(av[s], b1[s], c1);
        }
        if (more) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                av[s] = na[s];
                b0[s] = n0[s];
                b1[s] = n1[s];
            }
        }
    }

    float* pp = a.part + (int64_t)blockIdx.x * kPartFloats;
    float4* p0 = reinterpret_cast<float4*>(pp + ((wave * 2 + 0) * 64 + lane) * 16);
    float4* p1 = reinterpret_cast<float4*>(pp + ((wave * 2 + 1) * 64 + lane) * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        p0[q] = make_float4(c0[4 * q], c0[4 * q + 1], c0[4 * q + 2], c0[4 * q + 3]);
        p1[q] = make_float4(c1[4 * q], c1[4 * q + 1], c1[4 * q + 2], c1[4 * q + 3]);
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = atomicAdd(&a.counters[pair], 1u);
        const int last = prev == (uint32_t)(a.splits - 1);
        if (last) atomicExch(&a.counters[pair], 0u);     // ready for the next call
        s_last = last;
    }
    __syncthreads();
    if (!s_last || wave >= 2) return;
    __threadfence();

    // Last slice of this (head, chunk): waves 0 and 1 each take one 32-token block, add the slices'
    // partial sums in slice order and run the epilogue.
    const int tb = wave;
    const float* base = a.part + (int64_t)pair * a.splits * kPartFloats;
    float acc[4][16];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const float4* src = reinterpret_cast<const float4*>(base + ((b * 2 + tb) * 64 + lane) * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = src[q];
            acc[b][4 * q] = v.x; acc[b][4 * q + 1] = v.y; acc[b][4 * q + 2] = v.z; acc[b][4 * q + 3] = v.w;
        }
    }
    for (int s = 1; s < a.splits; ++s) {
        const float* ps = base + (int64_t)s * kPartFloats;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float4* src = reinterpret_cast<const float4*>(ps + ((b * 2 + tb) * 64 + lane) * 16);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = src[q];
                acc[b][4 * q] += v.x; acc[b][4 * q + 1] += v.y; acc[b][4 * q + 2] += v.z; acc[b][4 * q + 3] += v.w;
            }
        }
    }
    epilogue<kProduce>(a.e, head, tc * kChunk + tb * 32 + (lane & 31), acc);
}

// ------------------------------------------------------------------ tiled kernel (prefill)

struct TileArgs {
    const uint16_t* h;
    int64_t h_stride;
    const uint16_t* w;
    int64_t w_stride;
    int32_t K, N, heads, n_tt, n_tf;
    Epi e;
};

// Block index -> linear tile index such that each XCD (blocks are dealt to the 8 XCDs round-robin)
// receives a contiguous range of tiles; tiles are numbered feature-tile fastest.
__device__ __forceinline__ uint32_t xcd_tile(uint32_t bid, uint32_t total)
{
    const uint32_t x = bid & 7u;
    uint32_t prefix = 0;
    for (uint32_t i = 0; i < x; ++i) prefix += (total - i + 7u) >> 3;
    return prefix + (bid >> 3);
}

template <bool kProduce>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void project_tile_kernel(const TileArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kTile][kPitch];   // [stage][w | h][row][k]
    const uint32_t L = xcd_tile(blockIdx.x, (uint32_t)(a.n_tt * a.n_tf));
    const int tile_t = (int)(L / (uint32_t)a.n_tf);
    const int tile_f = (int)(L - (uint32_t)tile_t * (uint32_t)a.n_tf);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wf = wave & 1, wt = wave >> 1;
    const int hh = lane >> 5;
    const int f_base = tile_f * kTile, t_base = tile_t * kTile;

    // Global -> LDS: thread `tid` moves 16 B (8 k) at column 8 (tid & 7) of rows (tid >> 3) + 32 j.
    const int r0 = tid >> 3, c8 = (tid & 7) * 8;
    const uint16_t* ga[8];
    const uint16_t* gb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        ga[j] = a.w + (int64_t)min(f_base + r0 + 32 * j, a.N - 1) * a.w_stride + c8;
        gb[j] = a.h + (int64_t)min(t_base + r0 + 32 * j, a.e.T - 1) * a.h_stride + c8;
    }
    f32x16_t acc[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[b][tb] = f32x16_t{};

    const int nk = a.K / kBK;
    {
        uint4 ra[8], rb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            ra[j] = *reinterpret_cast<const uint4*>(ga[j]);
            rb[j] = *reinterpret_cast<const uint4*>(gb[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            *reinterpret_cast<uint4*>(&lds[0][0][r0 + 32 * j][c8]) = ra[j];
            *reinterpret_cast<uint4*>(&lds[0][1][r0 + 32 * j][c8]) = rb[j];
        }
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int s = kt & 1;
        // Next stage's slice, in flight during this stage's MFMAs (the last step re-reads its own
        // slice, unused, so the loads stay unconditional).
        const int kn = (kt + 1 < nk ? kt + 1 : kt) * kBK;
        uint4 ra[8], rb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            ra[j] = *reinterpret_cast<const uint4*>(ga[j] + kn);
            rb[j] = *reinterpret_cast<const uint4*>(gb[j] + kn);
        }
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            uint4 af[4], bf[4];
#pragma unroll
            for (int b = 0; b < 4; ++b)
                af[b] = *reinterpret_cast<const uint4*>(&lds[s][0][wf * 128 + b * 32 + (lane & 31)][ks * 16 + 8 * hh]);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                bf[tb] = *reinterpret_cast<const uint4*>(&lds[s][1][wt * 128 + tb * 32 + (lane & 31)][ks * 16 + 8 * hh]);
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) acc[b][tb] = mfma(af[b], bf[tb], acc[b][tb]);
        }
        if (kt + 1 < nk) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                *reinterpret_cast<uint4*>(&lds[s ^ 1][0][r0 + 32 * j][c8]) = ra[j];
                *reinterpret_cast<uint4*>(&lds[s ^ 1][1][r0 + 32 * j][c8]) = rb[j];
            }
        }
        __syncthreads();
    }

    const int head = tile_f * 2 + wf;
    if (head >= a.heads) return;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        float v[4][16];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[b][i] = acc[b][tb][i];
        epilogue<kProduce>(a.e, head, t_base + wt * 128 + tb * 32 + (lane & 31), v);
    }
}

// ------------------------------------------------------------------ host side

uint64_t round_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct SplitPlan {
    int32_t splits, kc, n_tc;
    uint64_t counter_bytes, bytes;
};

// K slices per (head, chunk): enough work-groups to cover the chip about once, at most 8 slices
// (the last slice reads every slice's partials through one compute unit), each slice a multiple
// of 64.
SplitPlan split_plan(int32_t T, int32_t K, int32_t heads)
{
    SplitPlan p;
    p.n_tc = (T + kChunk - 1) / kChunk;
    const int64_t groups = (int64_t)heads * p.n_tc;
    int64_t want = (256 + groups - 1) / groups;
    const int64_t steps = K / kBK;
    if (want > 8) want = 8;
    if (want > steps) want = steps;
    if (want < 1) want = 1;
    p.kc = (int32_t)(((steps + want - 1) / want) * kBK);
    p.splits = (K + p.kc - 1) / p.kc;
    p.counter_bytes = round_up((uint64_t)groups * sizeof(uint32_t));
    p.bytes = p.counter_bytes + (uint64_t)groups * p.splits * kPartFloats * sizeof(float);
    return p;
}

msa_status check_gemm(const uint16_t* h, int64_t h_row_stride, int32_t T, int32_t K, const uint16_t* w,
                      int64_t w_row_stride, int64_t N)
{
    if (T < 0 || K <= 0 || K % kBK || N <= 0 || N % kHeadDim || N > (int64_t)4096 * kHeadDim) return MSA_ERR_SHAPE;
    if (h_row_stride < K || h_row_stride % 8 || w_row_stride < K || w_row_stride % 8) return MSA_ERR_STRIDE;
    if (T > 0 && (!h || !w)) return MSA_ERR_NULL_POINTER;
    if (!aligned(h, 16) || !aligned(w, 16)) return MSA_ERR_ALIGNMENT;
    int64_t tmp;
    if (__builtin_mul_overflow((int64_t)T, h_row_stride, &tmp) || __builtin_mul_overflow(N, w_row_stride, &tmp))
        return MSA_ERR_OVERFLOW;
    const int64_t tiles = ((int64_t)T + kTile - 1) / kTile * ((N / kHeadDim + 1) / 2);
    if (tiles > 0x7fffffffLL) return MSA_ERR_SHAPE;      // grid size of the tiled kernel
    return MSA_OK;
}

template <bool kProduce>
msa_status launch_projection(const uint16_t* h, int64_t h_row_stride, int32_t T, int32_t K, const uint16_t* w,
                             int64_t w_row_stride, int32_t heads, const Epi& e, void* workspace,
                             uint64_t workspace_bytes, hipStream_t s)
{
    hipError_t err;
    if (T <= kSplitMaxTokens) {
        const SplitPlan p = split_plan(T, K, heads);
        if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < p.bytes) return MSA_ERR_WORKSPACE;
        SplitArgs a;
        a.h = h;
        a.h_stride = h_row_stride;
        a.w = w;
        a.w_stride = w_row_stride;
        a.counters = static_cast<uint32_t*>(workspace);
        a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + p.counter_bytes);
        a.K = K;
        a.kc = p.kc;
        a.splits = p.splits;
        a.n_tc = p.n_tc;
        a.e = e;
        void* args[] = {&a};
        const dim3 grid((unsigned)((int64_t)heads * p.n_tc * p.splits));
        err = hipLaunchKernel(reinterpret_cast<const void*>(&project_splitk_kernel<kProduce>), grid, dim3(256), args,
                              0, s);
    } else {
        TileArgs a;
        a.h = h;
        a.h_stride = h_row_stride;
        a.w = w;
        a.w_stride = w_row_stride;
        a.K = K;
        a.N = heads * kHeadDim;
        a.heads = heads;
        a.n_tt = (T + kTile - 1) / kTile;
        a.n_tf = (heads + 1) / 2;
        a.e = e;
        void* args[] = {&a};
        const dim3 grid((unsigned)((int64_t)a.n_tt * a.n_tf));
        err = hipLaunchKernel(reinterpret_cast<const void*>(&project_tile_kernel<kProduce>), grid, dim3(256), args, 0,
                              s);
    }
    return err == hipSuccess ? MSA_OK : MSA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

msa_status msa_project_workspace_size(int32_t num_tokens, int32_t hidden, int32_t num_heads, uint64_t* bytes)
{
    if (!bytes) return MSA_ERR_NULL_POINTER;
    if (num_tokens < 0 || hidden <= 0 || hidden % kBK || num_heads <= 0 || num_heads > 4096) return MSA_ERR_SHAPE;
    *bytes = num_tokens == 0 || num_tokens > kSplitMaxTokens ? 0 : split_plan(num_tokens, hidden, num_heads).bytes;
    return MSA_OK;
}

msa_status msa_project(const uint16_t* h, int64_t h_row_stride, int32_t num_tokens, int32_t hidden,
                       const uint16_t* w, int64_t w_row_stride, int32_t num_cols,
                       uint16_t* x_out, int64_t x_row_stride,
                       void* workspace, uint64_t workspace_bytes, void* stream)
{
    msa_status st = check_gemm(h, h_row_stride, num_tokens, hidden, w, w_row_stride, num_cols);
    if (st != MSA_OK) return st;
    if (x_row_stride < num_cols || x_row_stride % 8) return MSA_ERR_STRIDE;
    if (num_tokens > 0 && !x_out) return MSA_ERR_NULL_POINTER;
    if (!aligned(x_out, 16)) return MSA_ERR_ALIGNMENT;
    int64_t tmp;
    if (__builtin_mul_overflow((int64_t)num_tokens, x_row_stride, &tmp)) return MSA_ERR_OVERFLOW;
    if (num_tokens == 0) return MSA_OK;
    Epi e;
    std::memset(&e, 0, sizeof(e));
    e.x_out = x_out;
    e.x_stride = x_row_stride;
    e.T = num_tokens;
    return launch_projection<false>(h, h_row_stride, num_tokens, hidden, w, w_row_stride, num_cols / kHeadDim, e,
                                    workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

msa_status msa_project_produce(const uint16_t* h, int64_t h_row_stride, int32_t num_tokens, int32_t hidden,
                               const uint16_t* w, int64_t w_row_stride, int32_t head_dim,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t num_iq_heads,
                               int32_t num_ik_heads, const float* rope_cos, const float* rope_sin,
                               const int64_t* slots, int32_t page_size, int64_t num_pages,
                               const uint16_t* q_norm_weight, const uint16_t* k_norm_weight,
                               const uint16_t* iq_norm_weight, const uint16_t* ik_norm_weight,
                               float rms_eps, uint16_t* q_out, uint16_t* iq_out,
                               const msa_cache_view* k_cache, const msa_cache_view* v_cache,
                               const msa_cache_view* ik_cache,
                               void* workspace, uint64_t workspace_bytes, void* stream)
{
    if (head_dim != kHeadDim) return MSA_ERR_UNSUPPORTED;
    if (num_tokens < 0 || num_q_heads < 0 || num_kv_heads < 0 || num_iq_heads < 0 || num_ik_heads < 0)
        return MSA_ERR_SHAPE;
    const int64_t heads = (int64_t)num_q_heads + 2 * (int64_t)num_kv_heads + num_iq_heads + num_ik_heads;
    if (heads < 1 || heads > 4096) return MSA_ERR_SHAPE;
    if (page_size <= 0 || num_pages < 0 || !(rms_eps >= 0.0f)) return MSA_ERR_SHAPE;
    msa_status st = check_gemm(h, h_row_stride, num_tokens, hidden, w, w_row_stride, heads * kHeadDim);
    if (st != MSA_OK) return st;
    if (num_tokens > 0) {
        if (!rope_cos || !rope_sin || !slots) return MSA_ERR_NULL_POINTER;
        if ((num_q_heads > 0 && !q_out) || (num_iq_heads > 0 && !iq_out)) return MSA_ERR_NULL_POINTER;
    }
    if ((num_q_heads > 0 && !q_norm_weight) || (num_kv_heads > 0 && !k_norm_weight) ||
        (num_iq_heads > 0 && !iq_norm_weight) || (num_ik_heads > 0 && !ik_norm_weight))
        return MSA_ERR_NULL_POINTER;
    if (!aligned(rope_cos, 16) || !aligned(rope_sin, 16) || !aligned(slots, 8) || !aligned(q_out, 16) ||
        !aligned(iq_out, 16) || !aligned(q_norm_weight, 16) || !aligned(k_norm_weight, 16) ||
        !aligned(iq_norm_weight, 16) || !aligned(ik_norm_weight, 16))
        return MSA_ERR_ALIGNMENT;
    Epi e;
    std::memset(&e, 0, sizeof(e));
    if ((st = check_cache(k_cache, num_kv_heads, page_size, num_pages, &e.cache[0])) != MSA_OK) return st;
    if ((st = check_cache(v_cache, num_kv_heads, page_size, num_pages, &e.cache[1])) != MSA_OK) return st;
    if ((st = check_cache(ik_cache, num_ik_heads, page_size, num_pages, &e.cache[2])) != MSA_OK) return st;
    int64_t tmp;
    if (__builtin_mul_overflow(num_pages, (int64_t)page_size, &tmp)) return MSA_ERR_OVERFLOW;
    if (num_tokens == 0) return MSA_OK;
    e.cos = rope_cos;
    e.sin = rope_sin;
    e.slots = slots;
    e.num_pages = num_pages;
    e.w[0] = q_norm_weight;
    e.w[1] = k_norm_weight;
    e.w[2] = iq_norm_weight;
    e.w[3] = ik_norm_weight;
    e.q_out = q_out;
    e.iq_out = iq_out;
    e.page_size = page_size;
    e.hq = num_q_heads;
    e.hkv = num_kv_heads;
    e.hiq = num_iq_heads;
    e.hik = num_ik_heads;
    e.T = num_tokens;
    e.eps = rms_eps;
    return launch_projection<true>(h, h_row_stride, num_tokens, hidden, w, w_row_stride, (int32_t)heads, e, workspace,
                                   workspace_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
