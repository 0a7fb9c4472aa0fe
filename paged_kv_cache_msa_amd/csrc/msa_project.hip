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
//   project_split_kernel   up to 1,024 tokens, one launch: one work-group of eight waves per (head,
//                          64-token chunk, K slice of at most 384 columns).  The slice of w (128
//                          rows) and h (64 rows) is requested into LDS at once with direct global ->
//                          LDS loads (products start on its first half while the second lands);
//                          each wave multiplies a 32-feature block of the head against 32 tokens.
//                          The partial sums go to the workspace; the work-group of slice q then
//                          adds token group q (8 tokens) over all slices in a fixed order and runs
//                          the producer's arithmetic on the bf16-rounded sums in msa_produce's row
//                          layout (8 lanes per head row).  Work-groups on different XCDs exchange
//                          the partial sums with agent-scope coherent stores and polled loads, no
//                          cache-wide fence (see the kernel's comment).
//   project_tile_kernel    larger batches: 256 features (2 heads) x 256 tokens per work-group, four
//                          waves (one per SIMD) of one head x 128 tokens each (16 products per
//                          16-column step, 256 accumulator registers), 64-column K stages through
//                          two LDS buffers filled by direct global -> LDS loads, fragments read one
//                          step ahead of the products, and every load, copy and wait in a fixed
//                          slot between the products.  The output rows leave through LDS so that
//                          each store writes whole rows, and the tile order is chosen so that the
//                          work-groups of one XCD walk the feature tiles of the same token rows
//                          (their h panel stays in that XCD's L2).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "msa_common.h"
#include "msa_device.h"
#include "msa_project.h"

namespace {

using namespace msa_internal;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSplitMaxTokens = 1024;
constexpr int kChunk = 64;                 // tokens per split-K work-group (two MFMA token blocks)
constexpr int kPartFloats = 4 * 2 * 4 * 64 * 4;   // one work-group's partial sums: [wave][tb][q][lane][4]
constexpr int kTile = 256;                 // tiled kernel: features and tokens per work-group
constexpr int kBK = 64;                    // K per pipeline stage
constexpr uint64_t kAlign = 256;
constexpr int64_t kMaxTiledStride = 1 << 22;   // tiled kernel: 256 rows stay under 2 GiB
constexpr int kSliceMax = 384;             // split-K: K per slice at most (LDS: (128 + 64) rows x 384 bf16)
constexpr int kSplitLds = (128 + kChunk) * kSliceMax * 2;

enum Stream { kQ = 0, kK = 1, kV = 2, kIQ = 3, kIK = 4 };

// One 16-byte LDS read, issued as written: the compiler neither reorders it nor makes it wait for
// the direct global -> LDS loads in flight (it cannot see which LDS bytes an inline read touches).
// Completion is awaited explicitly with lgkm_wait below.
__device__ __forceinline__ u32x4_t lds_read16(uint32_t addr)
{
    u32x4_t v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}

// Waits until at most N LDS reads are in flight; the fragments passed are tied to the wait so that
// no use of them is scheduled above it.
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4_t (&a)[4], u32x4_t (&b)[2])
{
    asm volatile("s_waitcnt lgkmcnt(%6)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1])
                 : "n"(N));
}

template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4_t (&a)[4], u32x4_t (&b)[4])
{
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3])
                 : "n"(N));
}

// One 16-byte LDS read at an immediate offset from addr (see lds_read16).
template <int O>
__device__ __forceinline__ u32x4_t lds_read16o(uint32_t addr)
{
    u32x4_t v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(O));
    return v;
}

// Waits until at most N LDS reads are in flight, tied to eight fragments (see lgkm_wait).
template <int N>
__device__ __forceinline__ void lgkm_wait8(u32x4_t (&a)[8])
{
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
                 : "n"(N));
}

__device__ __forceinline__ f32x16_t mfma4(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c)
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

// The epilogue's per-lane inputs for one (head, token): the head's norm weights at this lane's 64
// features (bf16 pairs as loaded: w[b][g] holds features 32 b + 8 g + 4 hh .. + 3), where the
// token's RoPE coefficients sit in LDS (cs: its 512-byte row, 16 chunks of cos then 16 of sin,
// logical chunk c at position c ^ sw), and its cache slot.
struct EpiIn {
    uint2 w[4][4];
    uint32_t cs;
    int sw;
    int64_t slot;
    float scale;               // fp8 cache rows: the dequantisation scale (1 otherwise)
};

__device__ __forceinline__ int stream_of(const Epi& e, int head)
{
    const int h_k = e.hq, h_v = e.hq + e.hkv, h_iq = e.hq + 2 * e.hkv, h_ik = h_iq + e.hiq;
    return head < h_k ? kQ : head < h_v ? kK : head < h_iq ? kV : head < h_ik ? kIQ : kIK;
}

// Where one token's head row goes: dst == nullptr means nowhere (a token past T, or a cache row
// without a valid slot); fp8 rows are 128 bytes (e4m3 of value * m), the others 256 bytes of bf16.
struct RowOut {
    uint8_t* dst;
    bool fp8;
    float m;
};

// One head's row for one token per lane pair: a[b][i] is feature 32 b + 8 (i / 4) + 4 hh + i % 4
// (hh = lane / 32) of `head`, token t.  Rounds the row to bf16 (the packed row's values), then, in
// produce mode, runs the producer arithmetic on it with the norm weights, RoPE coefficients, slot
// and scale in `in` (fetched ahead by the caller); returns the row's destination.
template <bool kProduce>
__device__ __forceinline__ RowOut epilogue_math(const Epi& e, int head, int32_t t, float (&a)[4][16], const EpiIn& in)
{
    const int hh = (threadIdx.x & 63) >> 5;
    const bool tok = t < e.T;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t w = bf16x2(a[b][2 * j], a[b][2 * j + 1]);
            a[b][2 * j] = bf16_lo(w);
            a[b][2 * j + 1] = bf16_hi(w);
        }
    RowOut o{nullptr, false, 1.0f};
    if (!kProduce) {
        if (tok) o.dst = reinterpret_cast<uint8_t*>(e.x_out + (int64_t)t * e.x_stride + head * kHeadDim);
        return o;
    }

    const int h_k = e.hq, h_v = e.hq + e.hkv, h_iq = e.hq + 2 * e.hkv, h_ik = h_iq + e.hiq;
    const int st = stream_of(e, head);
    const bool cache_row = st == kK || st == kV || st == kIK;
    const CacheDev& cd = e.cache[st == kK ? 0 : st == kV ? 1 : 2];
    // The row format depends on the head only, so it is uniform over the wave (the row stores
    // rely on it), whatever the token.
    o.fp8 = cache_row && !cd.is_bf16;
    if (st != kV) {
        // RMSNorm: binary64 sum of squares over the lane's 64 features (two chains of 32, for the
        // latency) plus the partner lane's.  The squares of bf16 values are exact in binary64, and
        // so is every partial sum while the largest square is within about 2^30 of the smallest
        // nonzero one; past that the order of the additions moves only the last bits of the
        // binary64 sum, far below the binary32 scale taken from it.
        double ss0 = 0.0, ss1 = 0.0;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                ss0 = __builtin_fma((double)a[b][i], (double)a[b][i], ss0);
                ss1 = __builtin_fma((double)a[b + 2][i], (double)a[b + 2][i], ss1);
            }
        double ss = ss0 + ss1;
        ss += __shfl_xor(ss, 32);
        const float r = rms_from_ss(ss, e.eps);
        // This lane's 32 frequencies 32 b + 8 g + 4 hh .. + 3 (b < 2) of cos and sin, read while the
        // norm runs.
        u32x4_t cv[8], sv[8];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int cc = 8 * b + 2 * g + hh;
                cv[4 * b + g] = lds_read16(in.cs + (uint32_t)((cc ^ in.sw) * 16));
                sv[4 * b + g] = lds_read16(in.cs + (uint32_t)(((16 + cc) ^ in.sw) * 16));
            }
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 wv = in.w[b][g];
                // (Opaque per token block: otherwise the unpacked weights are shared by the four
                // blocks and stay live across them, 64 registers where 32 suffice.)
                asm volatile("" : "+v"(wv.x), "+v"(wv.y));
                const float w4[4] = {bf16_lo(wv.x), bf16_hi(wv.x), bf16_lo(wv.y), bf16_hi(wv.y)};
#pragma unroll
                for (int q = 0; q < 4; ++q) a[b][4 * g + q] = (a[b][4 * g + q] * r) * w4[q];
            }
        // RoPE, neox rotate-half: frequency f < 64 pairs feature f (block b) with f + 64 (block b + 2).
        lgkm_wait8<0>(cv);
        lgkm_wait8<0>(sv);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4_t c = __builtin_bit_cast(f32x4_t, cv[4 * b + g]);
                const f32x4_t sn = __builtin_bit_cast(f32x4_t, sv[4 * b + g]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i = 4 * g + q;
                    const float y0 = a[b][i], y1 = a[b + 2][i];
                    a[b][i] = y0 * c[q] - y1 * sn[q];
                    a[b + 2][i] = y1 * c[q] + y0 * sn[q];
                }
            }
    }
    if (!tok) return o;
    if (st == kQ || st == kIQ) {
        o.dst = reinterpret_cast<uint8_t*>(st == kQ ? e.q_out + ((int64_t)t * e.hq + head) * kHeadDim
                                                    : e.iq_out + ((int64_t)t * e.hiq + (head - h_iq)) * kHeadDim);
        return o;
    }
    const int64_t slot = in.slot;
    if (slot < 0) return o;
    const int64_t page = slot / e.page_size;
    if (page >= e.num_pages) return o;
    const int64_t off = slot - page * e.page_size;
    const int hl = st == kK ? head - h_k : st == kV ? head - h_v : head - h_ik;
    const int64_t elem = page * cd.sp + off * cd.st + (int64_t)hl * cd.sh;
    o.dst = cd.data + (o.fp8 ? elem : 2 * elem);
    if (o.fp8) o.m = inv_scale(in.scale);
    return o;
}

// Stores the bf16 rows of a 32-token block (lane l holds part of token l % 32's row, as above)
// through this wave's 8 KiB of LDS: every lane first writes its pieces into the row-major block,
// then each lane stores 16 contiguous bytes of one row, so that a store instruction writes whole
// rows.  In the staging block the 16-byte chunk c of row r sits at position c ^ (r & 15).
__device__ __forceinline__ void row_store_staged(const RowOut& o, const float (&a)[4][16], uint8_t* stage)
{
    const int lane = threadIdx.x & 63;
    const uint32_t st0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)stage;
    const int hh = lane >> 5, r = lane & 31;
    const uint32_t dlo = (uint32_t)reinterpret_cast<uintptr_t>(o.dst);
    const uint32_t dhi = (uint32_t)(reinterpret_cast<uintptr_t>(o.dst) >> 32);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *reinterpret_cast<uint2*>(stage + r * 256 + (((4 * b + g) ^ (r & 15)) * 16) + 8 * hh) =
                make_uint2(bf16x2(a[b][4 * g], a[b][4 * g + 1]), bf16x2(a[b][4 * g + 2], a[b][4 * g + 3]));
    __builtin_amdgcn_wave_barrier();
    // All reads and row addresses first, then the stores: no wait between the stores.
    u32x4_t v[8];
    uintptr_t d[8];
    const int c = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int rr = 4 * i + (lane >> 4);
        v[i] = lds_read16(st0 + (uint32_t)(rr * 256 + ((c ^ (rr & 15)) * 16)));
        d[i] = ((uintptr_t)(uint32_t)__shfl((int)dhi, rr) << 32) | (uint32_t)__shfl((int)dlo, rr);
    }
    lgkm_wait8<0>(v);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (d[i] != 0) *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint8_t*>(d[i]) + c * 16) = v[i];
    __builtin_amdgcn_wave_barrier();
}

// Stores the bf16 rows of a 32-token block (lane l holds part of token l % 32's row, as above)
// straight from the registers: the two lanes of a token swap halves of their pieces
// (v_permlane32_swap) so that each lane holds 16 contiguous bytes, features 32 b + 8 g .. + 7 for
// g = 2 p + hh, and stores them at its own token's row (o.dst; nullptr: no store).  A store
// instruction writes 32 bytes of 32 rows; the eight of a block complete every row.
__device__ __forceinline__ void row_store_bf16_direct(const RowOut& o, const float (&a)[4][16])
{
    const int hh = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            uint32_t ax = bf16x2(a[b][8 * p], a[b][8 * p + 1]), ay = bf16x2(a[b][8 * p + 2], a[b][8 * p + 3]);
            uint32_t bx = bf16x2(a[b][8 * p + 4], a[b][8 * p + 5]), by = bf16x2(a[b][8 * p + 6], a[b][8 * p + 7]);
            // lanes 0-31 keep a and take the partner's a as b; lanes 32-63 take the partner's b as a
            const auto sx = __builtin_amdgcn_permlane32_swap(ax, bx, false, false);
            const auto sy = __builtin_amdgcn_permlane32_swap(ay, by, false, false);
            if (o.dst != nullptr) {
                u32x4_t v = {sx[0], sy[0], sx[1], sy[1]};
                *reinterpret_cast<u32x4_t*>(o.dst + (32 * b + 8 * (2 * p + hh)) * 2) = v;
            }
        }
}

// Stores the fp8 rows of a 32-token block straight from the registers: encodes the lane's 64
// values (e4m3 of value * o.m), then the two lanes of a token exchange words (v_permlane32_swap)
// so that for each 32-feature block b lane hh holds the 16 contiguous bytes 32 b + 16 hh .. + 15,
// stored at its own token's row (o.dst; nullptr: no store).  A store instruction writes 32 bytes
// of 32 rows; the four of a block complete every row.
__device__ __forceinline__ void row_store_fp8_direct(const RowOut& o, const float (&a)[4][16])
{
    uint32_t q[4][4], nan_bytes = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            q[b][g] = e4m3x4_rne(a[b][4 * g] * o.m, a[b][4 * g + 1] * o.m, a[b][4 * g + 2] * o.m, a[b][4 * g + 3] * o.m);
            nan_bytes |= e4m3_nan_bytes(q[b][g]);
        }
    if (__builtin_amdgcn_ballot_w64(nan_bytes != 0) != 0) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                q[b][g] = e4m3x4(a[b][4 * g] * o.m, a[b][4 * g + 1] * o.m, a[b][4 * g + 2] * o.m, a[b][4 * g + 3] * o.m);
    }
    const int hh = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        // q[b][g] holds features 32 b + 8 g + 4 hh .. + 3.  Lanes 0-31 end with (own g0, partner's g0,
        // own g1, partner's g1) = features 32 b .. + 15; lanes 32-63 with (partner's g2, own g2,
        // partner's g3, own g3) = features 32 b + 16 .. + 31.
        const auto s0 = __builtin_amdgcn_permlane32_swap(q[b][0], q[b][2], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(q[b][1], q[b][3], false, false);
        if (o.dst != nullptr) {
            u32x4_t v = {s0[0], s0[1], s1[0], s1[1]};
            *reinterpret_cast<u32x4_t*>(o.dst + 32 * b + 16 * hh) = v;
        }
    }
}

// ------------------------------------------------------------------ split-K kernel (<= 1,024 tokens)

// Workspace of the split-K kernel: a 256-byte header (word 1: error bits), then the partial sums.
// A partial sum is stored as the bitwise complement of its binary32 bits, so that a zero word means
// "not written yet": no sum these kernels compute has all 32 bits set (a NaN comes either from the
// bf16 inputs, whose low 16 bits are zero, or is the default NaN).  Every word is consumed once per
// launch and zeroed again by the work-group that read it, so a launch that completes leaves the
// workspace all zero, as it must be before its first use.
constexpr int kHeaderBytes = 256;
constexpr int kMaxSplits = 63;
constexpr int kCoherent = 16;             // buffer cache policy sc1: agent-scope coherent load / store
constexpr int kPollLimit = 1 << 16;       // polls of a partial-sum fragment before a wave gives up
constexpr int kPollPolicy = (int)(16u | 0x80000000u);   // sc1 and the compiler's volatile bit
constexpr uint32_t kErrWait = 1u;

struct SplitArgs {
    const uint16_t* h;
    int64_t h_stride;
    const uint16_t* w;
    int64_t w_stride;
    uint32_t* err;             // error bits
    uint32_t* part;            // [pair][slice] x kPartFloats complemented binary32, pair = head * n_tc + chunk
    int32_t K, base, extra, splits, n_tc;      // slice s: base + (s < extra) planes of 64 columns
    Epi e;
};

typedef __attribute__((address_space(3))) void lds_void;

// LDS image of a K slice: 64-column planes (one per 64 columns of the slice), each holding every
// row's 128 bytes as 8 chunks of 16 bytes, chunk c of row r at position c ^ (r & 7): the 8 rows read
// by 8 consecutive lanes at one chunk fall in 8 different bank groups.
__device__ __forceinline__ int plane_slot(int rows, int plane, int row, int chunk)
{
    return (plane * rows + row) * 8 + (chunk ^ (row & 7));
}

// Moves plane g (64 columns) of rows [0, rows) of a K slice (row r at src_row(r)) into LDS at `dst`
// with the direct global -> LDS path: each lane of each wave fills one 16-byte slot per instruction
// (64 consecutive slots per wave).  rows is 64 or 128: rows / 64 instructions per wave (8 waves).
template <typename RowPtr>
__device__ __forceinline__ void plane_to_lds(uint8_t* dst, int rows, int g, RowPtr src_row)
{
    const int tid = threadIdx.x, wave = tid >> 6;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (j * 512 >= rows * 8) break;
        const int p = j * 512 + tid;                               // slot within the plane
        const int row = p >> 3;
        const int chunk = (p & 7) ^ (row & 7);                     // logical chunk stored at this slot
        const uint16_t* gsrc = src_row(row) + g * 64 + chunk * 8;
        uint8_t* l = dst + ((size_t)(g * rows * 8 + j * 512 + wave * 64)) * 16;
        __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)l, 16, 0, 0);
    }
}

// The epilogue of one token's head row in the producer's row layout: lane (ts = lane / 8, sub =
// lane % 8) of a wave holds features [8 sub, 8 sub + 8) and [64 + 8 sub, 64 + 8 sub + 8) of token
// 8 g + ts, so both rotate-half partners sit in one lane and a head's sum of squares is an 8-lane
// reduction, as in msa_produce (the same operations in the same order: the fused outputs equal
// msa_produce applied to msa_project's row, bit for bit).  RowIn holds what the epilogue reads
// besides the sums (norm weights, RoPE coefficients, slot, fp8 scale), fetched ahead.
struct RowIn {
    uint4 wa, wb;
    float4 c4[2], s4[2];
    int64_t slot;              // as loaded; meaningful where use_slot
    float scale;               // as loaded; meaningful where use_scale
    bool use_slot, use_scale;
};

// One binary32 read through the vector memory path (a raw buffer load), so that it is counted with
// the wave's other vector loads and no scalar-load wait stands between it and them.
__device__ __forceinline__ float vload_f32(const float* p)
{
    // 0x00020000: the gfx9-family word 3 of a raw (untyped, dword) buffer resource.
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, 4, 0x00020000);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0));
}

// Every load is unconditional: a stream without norm weights, a padded token and a cache without
// scale read valid stand-ins (the RoPE table, the last token's slot) whose values are then
// discarded, so no load has to complete at a branch join before the slice's loads are issued.
template <bool kProduce>
__device__ __forceinline__ RowIn row_inputs(const Epi& e, int head, int32_t t, int sub)
{
    RowIn in;
    in.wa = in.wb = make_uint4(0, 0, 0, 0);
    in.slot = -1;
    in.scale = 1.0f;
    in.use_slot = in.use_scale = false;
    if (!kProduce) return in;
    const bool tok = t < e.T;
    const int32_t tl = tok ? t : e.T - 1;
    const int st = stream_of(e, head);
    const uint16_t* w = st == kV ? reinterpret_cast<const uint16_t*>(e.cos)
                                 : e.w[st == kQ ? 0 : st == kK ? 1 : st == kIQ ? 2 : 3];
    in.wa = *reinterpret_cast<const uint4*>(w + sub * 8);
    in.wb = *reinterpret_cast<const uint4*>(w + kHalf + sub * 8);
    const float4* cp = reinterpret_cast<const float4*>(e.cos + (int64_t)tl * kHalf + sub * 8);
    const float4* sp = reinterpret_cast<const float4*>(e.sin + (int64_t)tl * kHalf + sub * 8);
    in.c4[0] = cp[0]; in.c4[1] = cp[1];
    in.s4[0] = sp[0]; in.s4[1] = sp[1];
    const bool cache_row = st == kK || st == kV || st == kIK;
    in.slot = e.slots[tl];
    in.use_slot = cache_row && tok;
    const CacheDev& cd = e.cache[st == kK ? 0 : st == kV ? 1 : 2];
    in.use_scale = cache_row && !cd.is_bf16;
    in.scale = vload_f32(in.use_scale ? cd.scale : e.cos);
    return in;
}

// v: the lane's 16 features' sums (binary32) of token t.
template <bool kProduce>
__device__ __forceinline__ void row_epilogue(const Epi& e, int head, int32_t t, int sub, const RowIn& in,
                                             const float (&v)[16])
{
    const bool tok = t < e.T;
    // The packed row's values: the sums rounded to bf16.
    uint4 ra = make_uint4(bf16x2(v[0], v[1]), bf16x2(v[2], v[3]), bf16x2(v[4], v[5]), bf16x2(v[6], v[7]));
    uint4 rb = make_uint4(bf16x2(v[8], v[9]), bf16x2(v[10], v[11]), bf16x2(v[12], v[13]), bf16x2(v[14], v[15]));
    if (!kProduce) {
        if (tok) {
            uint16_t* dst = e.x_out + (int64_t)t * e.x_stride + head * kHeadDim + sub * 8;
            *reinterpret_cast<uint4*>(dst) = ra;
            *reinterpret_cast<uint4*>(dst + kHalf) = rb;
        }
        return;
    }
    const int st = stream_of(e, head);
    float x[16];
    unpack8(ra, x);
    unpack8(rb, x + 8);
    float o[16];
    if (st == kV) {
#pragma unroll
        for (int j = 0; j < 16; ++j) o[j] = x[j];
    } else {
        double acc = 0.0;
#pragma unroll
        for (int j = 0; j < 16; ++j) acc = __builtin_fma((double)x[j], (double)x[j], acc);
        const float r = rms_from_ss(head_sum8(acc), e.eps);
        float wv[16];
        unpack8(in.wa, wv);
        unpack8(in.wb, wv + 8);
        const float cf[8] = {in.c4[0].x, in.c4[0].y, in.c4[0].z, in.c4[0].w, in.c4[1].x, in.c4[1].y, in.c4[1].z, in.c4[1].w};
        const float sf[8] = {in.s4[0].x, in.s4[0].y, in.s4[0].z, in.s4[0].w, in.s4[1].x, in.s4[1].y, in.s4[1].z, in.s4[1].w};
        float y[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) y[j] = (x[j] * r) * wv[j];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            o[j] = y[j] * cf[j] - y[j + 8] * sf[j];
            o[j + 8] = y[j + 8] * cf[j] + y[j] * sf[j];
        }
    }
    if (!tok) return;
    const int h_k = e.hq, h_v = e.hq + e.hkv, h_iq = e.hq + 2 * e.hkv, h_ik = h_iq + e.hiq;
    if (st == kQ || st == kIQ) {
        uint16_t* dst = (st == kQ ? e.q_out + ((int64_t)t * e.hq + head) * kHeadDim
                                  : e.iq_out + ((int64_t)t * e.hiq + (head - h_iq)) * kHeadDim) + sub * 8;
        *reinterpret_cast<uint4*>(dst) = bf16x8(o);
        *reinterpret_cast<uint4*>(dst + kHalf) = bf16x8(o + 8);
        return;
    }
    const int64_t slot = in.use_slot ? in.slot : -1;
    if (slot < 0) return;
    const int64_t page = slot / e.page_size;
    if (page >= e.num_pages) return;
    const int64_t off = slot - page * e.page_size;
    const CacheDev& cd = e.cache[st == kK ? 0 : st == kV ? 1 : 2];
    const int hl = st == kK ? head - h_k : st == kV ? head - h_v : head - h_ik;
    const int64_t elem = page * cd.sp + off * cd.st + (int64_t)hl * cd.sh + sub * 8;
    if (cd.is_bf16) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(cd.data) + elem;
        *reinterpret_cast<uint4*>(dst) = bf16x8(o);
        *reinterpret_cast<uint4*>(dst + kHalf) = bf16x8(o + 8);
    } else {
        uint2 lo, hi;
        e4m3x16(o, inv_scale(in.use_scale ? in.scale : 1.0f), lo, hi);
        uint8_t* dst = cd.data + elem;
        *reinterpret_cast<uint2*>(dst) = lo;
        *reinterpret_cast<uint2*>(dst + kHalf) = hi;
    }
}

// One launch for up to 1,024 tokens: one work-group of eight waves per (head, 64-token chunk, K
// slice), block index = (head * n_tc + chunk) * S + slice.
//   1. The slice of w (128 rows) and h (64 rows) is requested into LDS at once (its memory latency
//      paid once), in two plane groups; wave (b, tb) multiplies the head's 32-feature block b
//      against token block tb of the chunk with two MFMA chains, starting on the first group while
//      the second is still arriving.
//   2. The partial sums go to the workspace, complemented, with agent-scope coherent stores
//      (written through, so a work-group on another XCD reads them without a cache-wide
//      write-back).  Nothing waits for them here.
//   3. Token group q (8 tokens) of the chunk is reduced by the work-group of slice q mod S: its wave
//      j reads slices j, j + 8, ... of that token group, polling each fragment until every word of
//      it has been written (nonzero), adds them in that order, zeroes the words it read, and hands
//      its sum to wave 0 through LDS; wave 0 adds the eight waves' sums in wave order (for S <= 8,
//      slice order) and runs the epilogue (row_epilogue).  The order is fixed, so every call gives
//      the same bits.
// A work-group polls only for the other S - 1 slices of its own (head, chunk), which hold the
// adjacent block indices.  Work-groups start in block order as compute units free up, and each one
// holds a compute unit only until its token group is reduced, so the polls end as long as S work-
// groups of this kernel fit on the device at once (S <= 63; at most 8 at hidden sizes up to 3,072).
// A wave that still finds unwritten words after kPollLimit polls (only possible if that does not
// hold, or if the workspace was not zero on entry) sets an error bit and leaves its token group
// unwritten: no state of the device or the workspace can make a launch hang.
template <bool kProduce>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void project_split_kernel(const SplitArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSplitLds];
    __shared__ uint32_t s_ok;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int fb = wave & 3, tb = wave >> 2;                         // 32-feature block, 32-token block
    const int hh = lane >> 5;
    const int split = (int)(blockIdx.x % (uint32_t)a.splits);
    const int pair = (int)(blockIdx.x / (uint32_t)a.splits);         // head * n_tc + chunk
    const int tc = pair % a.n_tc;
    const int head = pair / a.n_tc;
    const int k_begin = kBK * (split * a.base + min(split, a.extra));
    const int planes = a.base + (split < a.extra ? 1 : 0);

    // Epilogue inputs of this work-group's first token group, fetched by wave 0 (which runs the
    // epilogue) before the slice, so that they are not behind it in the wave's in-order load counter.
    // (Fetched by every wave, the same addresses eight times over, a decode call took 0.5 us longer.)
    const int t_first = tc * kChunk, t_last = a.e.T - 1;
    const int ts = lane / 8, sub = lane % 8;
    RowIn in;
    if (wave == 0) in = row_inputs<kProduce>(a.e, head, t_first + 8 * split + ts, sub);

    // The whole slice of w (128 rows) and h (64 rows) in flight at once, in plane order: each wave
    // issues 3 loads per plane (2 of w, 1 of h).
    uint8_t* lds_a = smem;
    uint8_t* lds_b = smem + (size_t)128 * planes * 8 * 16;
    const uint16_t* wrow = a.w + (int64_t)head * kHeadDim * a.w_stride + k_begin;
    const int64_t ws = a.w_stride, hs = a.h_stride;
    const uint16_t* hrow = a.h + k_begin;
    for (int g = 0; g < planes; ++g) {
        plane_to_lds(lds_a, 128, g, [&](int r) { return wrow + r * ws; });
        plane_to_lds(lds_b, kChunk, g, [&](int r) { return hrow + (int64_t)min(t_first + r, t_last) * hs; });
    }

    // Two independent accumulation chains (even / odd 16-column steps), over the planes in two
    // groups: the first group's products run while the second group's planes are still arriving.
    f32x16_t c = {}, d = {};
    const int ra = fb * 32 + (lane & 31), rb = tb * 32 + (lane & 31);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
    const uint32_t lds_b0 = lds0 + (uint32_t)(128 * planes * 8 * 16);
    auto products = [&](int g0, int g1) {
        for (int g = g0; g < g1; ++g) {
            u32x4_t av[4], bv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ch = 2 * q + hh;
                av[q] = lds_read16(lds0 + (uint32_t)plane_slot(128, g, ra, ch) * 16);
                bv[q] = lds_read16(lds_b0 + (uint32_t)plane_slot(kChunk, g, rb, ch) * 16);
            }
            lgkm_wait<0>(av, bv);
            c = mfma4(av[0], bv[0], c);
            d = mfma4(av[1], bv[1], d);
            c = mfma4(av[2], bv[2], c);
            d = mfma4(av[3], bv[3], d);
        }
    };
    const int first = planes - planes / 2;                          // planes of the first group
    // vmcnt(3 x the second group's planes): this wave's loads of the first group have landed (its
    // loads retire in issue order; anything issued later only makes the wait longer).
    switch (planes / 2) {
    case 0: __builtin_amdgcn_s_waitcnt(0x3f70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x3f73); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x3f76); break;
    default: __builtin_amdgcn_s_waitcnt(0x3f79); break;
    }
    // Bare barriers: __syncthreads' fence would wait for every direct-to-LDS load still in flight.
    // The waits above order this wave's loads; after the barrier every wave's are in LDS.
    __builtin_amdgcn_s_barrier();
    products(0, first);
    __builtin_amdgcn_s_waitcnt(0x3f70);                              // vmcnt(0): every slot landed
    __builtin_amdgcn_s_barrier();
    products(first, planes);
    c += d;

    // Partial sums of this slice, complemented: [pair][slice][b][tb][q][lane] x 4 words.
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        a.part + (int64_t)pair * a.splits * kPartFloats, (short)0, a.splits * kPartFloats * (int)sizeof(float),
        0x00020000);
    constexpr int kSliceBytes = kPartFloats * 4;
    const int wbase = split * kSliceBytes + (((fb * 2 + tb) * 4) * 64 + lane) * 16;   // q = 0
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x4_t enc = __builtin_bit_cast(
            f32x4_t, ~__builtin_bit_cast(u32x4_t, f32x4_t{c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]}));
        __builtin_amdgcn_raw_buffer_store_b128(enc, rs, wbase + q * 1024, 0, kCoherent);
    }

    // Reduction of token groups q = split, split + S, ... (one per work-group when S >= 8).
    f32x4_t* red = reinterpret_cast<f32x4_t*>(smem);                // [wave][4][lane] x 4 sums
    for (int q = split; q < kChunk / 8; q += a.splits) {
        __syncthreads();                                             // LDS free: products / last group done
        if (q != split && wave == 0) in = row_inputs<kProduce>(a.e, head, t_first + 8 * q + ts, sub);
        // Byte offsets (within a slice) of this lane's four fragments: token t64 = 8 q + ts, feature
        // blocks sub / 4 and 2 + sub / 4, fragment row sub % 4, lane halves 0 and 1.
        const int t64 = 8 * q + ts, ftb = t64 / 32, t32 = t64 % 32;
        auto at = [&](int w, int h2) { return ((((w * 2 + ftb) * 4 + (sub % 4)) * 64) + t32 + 32 * h2) * 16; };
        const int off[4] = {at(sub / 4, 0), at(sub / 4, 1), at(2 + sub / 4, 0), at(2 + sub / 4, 1)};
        float v[16];
        bool ok = true;
        for (int sl = wave; sl < a.splits; sl += 8) {
            const int sb = sl * kSliceBytes;
            u32x4_t x[4];
            for (int polls = 0;; ++polls) {
                // Volatile loads: the words change under this loop (the compiler keeps every load and
                // every word's test inside it; volatile makes them system-scope coherent).
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    x[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, sb + off[i], 0, kPollPolicy));
                int full = 1;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) full &= x[i][j] != 0u ? 1 : 0;
                if (__all(full)) break;
                if (polls == kPollLimit) {
                    ok = false;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            if (!ok) break;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // Written through like the partial sums: plain stores would leave these lines dirty
                // for the kernel's end to write back (1.6 us per decode call, measured).
                __builtin_amdgcn_raw_buffer_store_b128(f32x4_t{0.f, 0.f, 0.f, 0.f}, rs, sb + off[i], 0, kCoherent);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float y = __builtin_bit_cast(float, ~x[i][j]);
                    v[4 * i + j] = sl == wave ? y : v[4 * i + j] + y;
                }
            }
        }
        if (!ok && lane == 0) atomicOr(a.err, kErrWait);
        if (wave < a.splits) {
#pragma unroll
            for (int i = 0; i < 4; ++i) red[(wave * 4 + i) * 64 + lane] = f32x4_t{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
        }
        if (tid == 0) s_ok = 1;
        __syncthreads();
        if (!ok) s_ok = 0;
        __syncthreads();
        if (wave == 0 && s_ok) {
            float sum[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4_t r = red[i * 64 + lane];
                sum[4 * i] = r[0]; sum[4 * i + 1] = r[1]; sum[4 * i + 2] = r[2]; sum[4 * i + 3] = r[3];
            }
            for (int w = 1; w < min(a.splits, 8); ++w)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4_t r = red[(w * 4 + i) * 64 + lane];
                    sum[4 * i] += r[0]; sum[4 * i + 1] += r[1]; sum[4 * i + 2] += r[2]; sum[4 * i + 3] += r[3];
                }
            row_epilogue<kProduce>(a.e, head, t_first + 8 * q + ts, sub, in, sum);
        }
    }
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
// receives a contiguous range of tiles.
__device__ __forceinline__ uint32_t xcd_tile(uint32_t bid, uint32_t total)
{
    const uint32_t x = bid & 7u;
    uint32_t prefix = 0;
    for (uint32_t i = 0; i < x; ++i) prefix += (total - i + 7u) >> 3;
    return prefix + (bid >> 3);
}

// Linear tile index -> (token tile, feature tile): blocks of four token tiles by every feature
// tile, token tile fastest within a block.  The 32 work-groups an XCD runs at once then cover
// 4 token tiles x 8 feature tiles of the 2,944-column projection, 12 distinct operand tiles per
// stage for its L2, where numbering feature tiles fastest covers about 2.7 x 12, 14.7 of them
// (measured 2% faster; blocks of two or eight token tiles were in between).  A bijection for any
// tile counts (the last block may hold fewer token tiles).
__device__ __forceinline__ void tile_of(uint32_t L, int n_tt, int n_tf, int& tile_t, int& tile_f)
{
    constexpr int kBlockT = 4;
    const int per = kBlockT * n_tf;
    const int blk = (int)L / per, rr = (int)L - blk * per;
    const int t0 = kBlockT * blk, nt = min(kBlockT, n_tt - t0);
    tile_t = t0 + rr % nt;
    tile_f = rr / nt;
}

template <bool kProduce>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void project_tile_kernel(const TileArgs a)
{
    // Two stages, each [w | h] x 256 rows x 64 columns: 128-byte rows, chunk c of row r at position
    // c ^ ((r >> 1) & 7) (fragment reads of 32 rows at one chunk are free of bank conflicts;
    // measured).  After the last step the output rows are staged in the first 32 KiB (plain mode);
    // in produce mode the stages then hold RoPE coefficients and the rows go out from the registers.
    constexpr int kOp = kTile * 128;
    constexpr int kStage = 2 * kOp;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];
    int tile_t, tile_f;
    tile_of(xcd_tile(blockIdx.x, (uint32_t)(a.n_tt * a.n_tf)), a.n_tt, a.n_tf, tile_t, tile_f);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, r = lane & 31;
    const int wf = wave & 1, wt = wave >> 1;            // head of the tile, 128-token half
    const int f_base = tile_f * kTile, t_base = tile_t * kTile;

    // Stage copy instruction i (0..15) of a thread: i < 8 copies w, else h; it fills slot
    // (i & 7) * 256 + tid of that operand, which holds row 32 (i & 7) + (tid >> 3) and, at position
    // tid & 7, logical chunk (tid & 7) ^ ((row >> 1) & 7).  Rows past the matrix read its last row.
    // The copies are buffer loads from the tile's first row: 32-bit row offsets (the host keeps
    // 256 rows under 2 GiB), the column offset in the scalar offset, no per-copy address arithmetic
    // (measured 1-2% faster than global loads with 64-bit addresses).
    const int prow = tid >> 3;
    const int pchunk = (tid & 7) ^ ((tid >> 4) & 7);
    const int wrows = min(kTile, a.N - f_base), hrows = min(kTile, a.e.T - t_base);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.w + (int64_t)f_base * a.w_stride), 0, (int)(wrows * a.w_stride * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.h + (int64_t)t_base * a.h_stride), 0, (int)(hrows * a.h_stride * 2), 0x00020000);
    int woff[8], hoff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        woff[j] = (min(j * 32 + prow, wrows - 1) * (int)a.w_stride + pchunk * 8) * 2;
        hoff[j] = (min(j * 32 + prow, hrows - 1) * (int)a.h_stride + pchunk * 8) * 2;
    }
    auto copy = [&](int buf, int k0, int i) {
        const int j = i & 7;
        lds_void* dst = (lds_void*)(&lds[buf * kStage + (i >> 3) * kOp + (j * 256 + wave * 64) * 16]);
        if (i < 8) __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, dst, 16, woff[j], k0 * 2, 0, 0);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(hr, dst, 16, hoff[j], k0 * 2, 0, 0);
    };
    const int nk = a.K / kBK;
    // Produce mode: the epilogue's RoPE coefficients, for the tile's 256 tokens, are copied into the
    // stage buffers in place of the two stages past the last one: "stage" nk + h holds tokens
    // 128 h .. 128 h + 127 (token u's 512-byte row: 16 chunks of cos, then 16 of sin, logical chunk
    // c at position c ^ (u & 15), so that the 32 tokens of a fragment read spread over the banks).
    // One copy per token for both heads, in whole rows, and started while the last products run.
    // Tiles of V heads only skip them; the plain kernel copies nothing past the last stage.
    const bool rope = kProduce && (stream_of(a.e, tile_f * 2) != kV ||
                                   (tile_f * 2 + 1 < a.heads && stream_of(a.e, tile_f * 2 + 1) != kV));
    // (The table pointers are copied out of the argument block first: selected per lane straight
    // from it, each copy would load the pointer from memory and wait for it.)
    const float* const cos_t = a.e.cos;
    const float* const sin_t = a.e.sin;
    const int32_t t_last = a.e.T - 1;
    auto rope_copy = [&](int h, int i) {     // copy i (0..15) of the coefficients of tokens 128 h ..
        if (!rope) return;
        const int u = 128 * h + 2 * (i * 4 + wave) + (lane >> 5);
        const int c = (lane & 31) ^ (u & 15);
        const int32_t tl = min(t_base + u, t_last);
        const float* src = (c < 16 ? cos_t : sin_t) + (int64_t)tl * kHalf + (c & 15) * 4;
        __builtin_amdgcn_global_load_lds(src, (lds_void*)(&lds[((nk + h) & 1) * kStage + (i * 4 + wave) * 1024]), 16, 0, 0);
    };
    // Fragment f of 16-column step ks: f < 4 is the head's 32-feature block f, else 32-token block f - 4.
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)&lds[0];
    const int sw = (r >> 1) & 7;
    uint32_t fa[4], fb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        fa[ks] = lds0 + (uint32_t)((wf * 128 + r) * 128 + (((2 * ks + hh) ^ sw) * 16));
        fb[ks] = lds0 + (uint32_t)(kOp + (wt * 128 + r) * 128 + (((2 * ks + hh) ^ sw) * 16));
    }
    auto frag = [&](int buf, int ks, int f) -> u32x4_t {
        const uint32_t pa = fa[ks] + (uint32_t)(buf * kStage), pb = fb[ks] + (uint32_t)(buf * kStage);
        switch (f) {
        case 0: return lds_read16o<0>(pa);
        case 1: return lds_read16o<4096>(pa);
        case 2: return lds_read16o<8192>(pa);
        case 3: return lds_read16o<12288>(pa);
        case 4: return lds_read16o<0>(pb);
        case 5: return lds_read16o<4096>(pb);
        case 6: return lds_read16o<8192>(pb);
        default: return lds_read16o<12288>(pb);
        }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[b][tb] = f32x16_t{};
#pragma unroll
    for (int i = 0; i < 16; ++i) copy(0, 0, i);
    __builtin_amdgcn_s_waitcnt(0x3f70);                          // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    if (nk > 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) copy(1, kBK, i);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) rope_copy(0, i);
    }
    u32x4_t F0[8], F1[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) F0[f] = frag(0, 0, f);
    // Stage kt is in buffer kt & 1.  Each step issues its 16 products one per slot, and the other
    // instructions sit in fixed slots between them (sched_barrier keeps the order):
    //   steps 0-2, slots 0-7: the next step's fragments;
    //   step 0, even slots: the last eight copy instructions of stage kt + 1;
    //   step 3, slot 3: wait for this wave's copies of stage kt + 1, then the barrier (every
    //     wave's copies landed, every wave's reads of stage kt done);
    //   step 3, slots 4-11: stage kt + 1's first fragments and the first eight copy
    //     instructions of stage kt + 2, into the buffer the barrier released.
    // Past the last stage nothing is copied, or the RoPE coefficients (above).  A stage's copies
    // so go out three to four steps before the wait for them (issued at the top of the stage
    // before, two and a half steps ahead, the kernel was 6% slower; all sixteen after the
    // barrier, 3%; twelve after the barrier and four in step 0's first slots, 1.5%: the copies
    // bunched in one step hold up the vector-memory issue).
    // The loop body for stage kt: M = 0 while stage kt + 2 exists, 1 for kt = nk - 2, 2 for the last
    // stage (the copies past the last stage are the RoPE coefficients' or none, without a branch
    // among the products).
    auto stage = [&](int kt, auto M) {
        constexpr int m = decltype(M)::value;
        const int buf = kt & 1, nb = buf ^ 1;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            u32x4_t (&C)[8] = (ks & 1) ? F1 : F0;
            u32x4_t (&N)[8] = (ks & 1) ? F0 : F1;
            lgkm_wait8<0>(C);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                acc[i >> 2][i & 3] = mfma4(C[i >> 2], C[4 + (i & 3)], acc[i >> 2][i & 3]);
                if (ks < 3) {
                    if (i < 8) N[i] = frag(buf, ks + 1, i);
                    if (ks == 0 && (i & 1) == 0) {
                        if (m < 2) copy(nb, (kt + 1) * kBK, 8 + i / 2);
                        else rope_copy(0, 8 + i / 2);
                    }
                } else {
                    if (i == 3) {
                        __builtin_amdgcn_s_waitcnt(0x3f70);      // vmcnt(0)
                        __builtin_amdgcn_s_barrier();
                    }
                    if (i >= 4 && i < 12) {
                        N[i - 4] = frag(nb, 0, i - 4);
                        if (m == 0) copy(buf, (kt + 2) * kBK, i - 4);
                        if (m == 1) rope_copy(0, i - 4);
                    }
                    if (m == 2 && i >= 4) rope_copy(1, i - 4);  // all sixteen: no stage follows
                    if (m == 2 && i >= 12) rope_copy(1, i);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    for (int kt = 0; kt < nk - 2; ++kt) stage(kt, std::integral_constant<int, 0>{});
    if (nk > 1) stage(nk - 2, std::integral_constant<int, 1>{});
    // Produce mode: the epilogue's norm weights (this lane's 64 features of the head, as bf16 pairs)
    // and the cache slots of its four 32-token blocks are loaded before the last stage, whose
    // products cover their latency.
    const int head = tile_f * 2 + wf;
    const int st = kProduce ? stream_of(a.e, min(head, a.heads - 1)) : kQ;
    const bool cache_row = st == kK || st == kV || st == kIK;
    EpiIn in;
    int64_t slot4[4];
    if constexpr (kProduce) {
        const Epi& e = a.e;
        in.scale = 1.0f;
        if (cache_row) {
            const CacheDev& cd = e.cache[st == kK ? 0 : st == kV ? 1 : 2];
            if (!cd.is_bf16) in.scale = *cd.scale;
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int32_t t = t_base + wt * 128 + tb * 32 + r;
            slot4[tb] = cache_row && t < e.T ? e.slots[t] : -1;
        }
    }
    stage(nk - 1, std::integral_constant<int, 2>{});
    __builtin_amdgcn_s_waitcnt(0x3f70);                          // vmcnt(0): every copy landed
    lgkm_wait8<0>(F0);
    __syncthreads();
    // The accumulators stay in the accumulator registers up to here: left free, the register
    // allocator pulls some towards the epilogue's vector registers and then moves them inside the
    // loop.
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) asm volatile("" : "+a"(acc[b][tb]));

    if constexpr (kProduce) {
        const Epi& e = a.e;
        if (st != kV) {
            const uint16_t* wp = e.w[st == kQ ? 0 : st == kK ? 1 : st == kIQ ? 2 : 3] + 4 * hh;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int g = 0; g < 4; ++g) in.w[b][g] = *reinterpret_cast<const uint2*>(wp + 32 * b + 8 * g);
        }
        __builtin_amdgcn_s_waitcnt(0x3f70);                      // vmcnt(0): this wave's coefficient copies
        __syncthreads();                                         // everyone's
        if (head >= a.heads) return;
        const uint32_t lds0e = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)&lds[0];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            float v[4][16];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                // (Ordered after the block before: read early, the blocks' values would all be
                // live at once.)
                asm volatile("" : "+a"(acc[b][tb]));
#pragma unroll
                for (int i = 0; i < 16; ++i) v[b][i] = acc[b][tb][i];
            }
            const int u = wt * 128 + tb * 32 + r;
            const int32_t t = t_base + u;
            in.cs = lds0e + (uint32_t)(((nk + wt) & 1) * kStage + (u & 127) * 512);
            in.sw = u & 15;
            in.slot = slot4[tb];
            const RowOut o = epilogue_math<true>(e, head, t, v, in);
            // Rows from the registers: no LDS round trip and no exchange of row addresses (bf16
            // rows: 1% faster than staging them).
            if (o.fp8) row_store_fp8_direct(o, v);
            else row_store_bf16_direct(o, v);
        }
    } else {
        if (head >= a.heads) return;
        uint8_t* stage = &lds[0] + wave * 8192;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            float v[4][16];
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) v[b][i] = acc[b][tb][i];
            const int32_t t = t_base + wt * 128 + tb * 32 + r;
            const RowOut o = epilogue_math<false>(a.e, head, t, v, in);
            // (Staged: stored straight from the registers, 32 bytes of 32 rows per instruction,
            // the plain kernel's output bursts were 2% slower.)
            row_store_staged(o, v, stage);
        }
    }
}

// ------------------------------------------------------------------ host side

uint64_t round_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct SplitPlan {
    int32_t splits, base, extra, n_tc;
    uint64_t ctl_bytes, bytes;
};

// K slices per (head, chunk): as few as the LDS allows (a slice of at most kSliceMax columns of w
// and h is staged whole).  Slices are whole 64-column planes, the first `extra` of them one plane
// longer.  (More, smaller slices, to occupy more of the 256 compute units, measured slower: the
// decode batch's 23 heads at 8 slices take 12.2 us per layer, at 11 slices 12.5, at 12 slices, more
// work-groups than compute units, 17.8.)
SplitPlan split_plan(int32_t T, int32_t K, int32_t heads)
{
    SplitPlan p;
    p.n_tc = (T + kChunk - 1) / kChunk;
    const int64_t groups = (int64_t)heads * p.n_tc;
    const int64_t steps = K / kBK;
    int64_t splits = (K + kSliceMax - 1) / kSliceMax;
#ifdef PROJECT_FORCE_SPLITS
    splits = PROJECT_FORCE_SPLITS;
#endif
    if (splits > steps) splits = steps;
    p.splits = (int32_t)splits;
    p.base = (int32_t)(steps / splits);
    p.extra = (int32_t)(steps % splits);
    p.ctl_bytes = kHeaderBytes;
    p.bytes = p.ctl_bytes + round_up((uint64_t)groups * p.splits * kPartFloats * sizeof(float));
    return p;
}

// Workspace bytes a projection of T tokens uses (none for the tiled path).
uint64_t workspace_need(int32_t T, int32_t K, int32_t heads)
{
    return T <= 0 || T > kSplitMaxTokens ? 0 : split_plan(T, K, heads).bytes;
}

msa_status check_gemm(const uint16_t* h, int64_t h_row_stride, int32_t T, int32_t K, const uint16_t* w,
                      int64_t w_row_stride, int64_t N)
{
    if (T < 0 || K <= 0 || K % kBK || N <= 0 || N % kHeadDim || N > (int64_t)4096 * kHeadDim) return MSA_ERR_SHAPE;
    if (T <= kSplitMaxTokens && K > kMaxSplits * kSliceMax) return MSA_ERR_SHAPE;   // split-K slices per item
    if (h_row_stride < K || h_row_stride % 8 || w_row_stride < K || w_row_stride % 8) return MSA_ERR_STRIDE;
    if (T > 0 && (!h || !w)) return MSA_ERR_NULL_POINTER;
    if (!aligned(h, 16) || !aligned(w, 16)) return MSA_ERR_ALIGNMENT;
    int64_t tmp;
    if (__builtin_mul_overflow((int64_t)T, h_row_stride, &tmp) || __builtin_mul_overflow(N, w_row_stride, &tmp))
        return MSA_ERR_OVERFLOW;
    const int64_t tiles = ((int64_t)T + kTile - 1) / kTile * ((N / kHeadDim + 1) / 2);
    if (tiles > 0x7fffffffLL) return MSA_ERR_SHAPE;      // grid size of the tiled kernel
    if (T > kSplitMaxTokens && (h_row_stride >= kMaxTiledStride || w_row_stride >= kMaxTiledStride))
        return MSA_ERR_STRIDE;                           // the tiled kernel's 32-bit row offsets
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
        a.err = static_cast<uint32_t*>(workspace) + 1;
        a.part = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) + p.ctl_bytes);
        a.K = K;
        a.base = p.base;
        a.extra = p.extra;
        a.splits = p.splits;
        a.n_tc = p.n_tc;
        a.e = e;
        void* args[] = {&a};
        const int64_t items = (int64_t)heads * p.n_tc * p.splits;
        err = hipLaunchKernel(reinterpret_cast<const void*>(&project_split_kernel<kProduce>), dim3((unsigned)items),
                              dim3(512), args, 0, s);
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

// msa_project_produce's checks and launches.  `own_scratch`: the workspace is the library's static
// scratch array (its residency is not queried: the runtime places the code object's arrays itself).
msa_status project_produce(const uint16_t* h, int64_t h_row_stride, int32_t num_tokens, int32_t hidden,
                           const uint16_t* w, int64_t w_row_stride, int32_t head_dim,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t num_iq_heads,
                           int32_t num_ik_heads, const float* rope_cos, const float* rope_sin,
                           const int64_t* slots, int32_t page_size, int64_t num_pages,
                           const uint16_t* q_norm_weight, const uint16_t* k_norm_weight,
                           const uint16_t* iq_norm_weight, const uint16_t* ik_norm_weight,
                           float rms_eps, uint16_t* q_out, uint16_t* iq_out,
                           const msa_cache_view* k_cache, const msa_cache_view* v_cache,
                           const msa_cache_view* ik_cache,
                           void* workspace, uint64_t workspace_bytes, hipStream_t stream, bool own_scratch)
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
    uint64_t cache_span[3];
    if ((st = check_cache(k_cache, num_kv_heads, page_size, num_pages, &e.cache[0], true, &cache_span[0])) != MSA_OK)
        return st;
    if ((st = check_cache(v_cache, num_kv_heads, page_size, num_pages, &e.cache[1], true, &cache_span[1])) != MSA_OK)
        return st;
    if ((st = check_cache(ik_cache, num_ik_heads, page_size, num_pages, &e.cache[2], true, &cache_span[2])) != MSA_OK)
        return st;
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
    const uint64_t need = workspace_need(num_tokens, hidden, (int32_t)heads);
    if (need > 0 && (!workspace || !aligned(workspace, kAlign) || workspace_bytes < need)) return MSA_ERR_WORKSPACE;
    const Span spans[] = {
        {h, row_bytes(num_tokens, h_row_stride, hidden, 2)},
        {w, row_bytes(heads * kHeadDim, w_row_stride, hidden, 2)},
        {rope_cos, nbytes((int64_t)num_tokens * (kHeadDim / 2), 4)},
        {rope_sin, nbytes((int64_t)num_tokens * (kHeadDim / 2), 4)},
        {slots, nbytes(num_tokens, 8)},
        {q_norm_weight, 2 * kHeadDim}, {k_norm_weight, 2 * kHeadDim},
        {iq_norm_weight, 2 * kHeadDim}, {ik_norm_weight, 2 * kHeadDim},
        {q_out, nbytes((int64_t)num_tokens * num_q_heads * kHeadDim, 2)},
        {iq_out, nbytes((int64_t)num_tokens * num_iq_heads * kHeadDim, 2)},
        {e.cache[0].data, cache_span[0]}, {e.cache[1].data, cache_span[1]}, {e.cache[2].data, cache_span[2]},
        {e.cache[0].scale, 4}, {e.cache[1].scale, 4}, {e.cache[2].scale, 4},
        {own_scratch ? nullptr : workspace, need},
    };
    if ((st = check_operands(spans, sizeof(spans) / sizeof(spans[0]), stream)) != MSA_OK) return st;
    return launch_projection<true>(h, h_row_stride, num_tokens, hidden, w, w_row_stride, (int32_t)heads, e, workspace,
                                   workspace_bytes, stream);
}


// ------------------------------------------------------------------ the library's own scratch

// Split-K partial sums of msa_project_produce_noalloc: one array per device, resident from the
// code object's load until the process ends; it starts zero (static storage), the state every call
// needs on entry and leaves behind.  32 MiB holds the partial sums of 23 heads x 3,072 hidden
// columns for up to 256 tokens (64 tokens: 5.9 MB).  Host code never names `scratch` where
// it needs the memory: the name is a host-side stand-in, and each device's address comes from the
// runtime (scratch_address).
constexpr uint64_t kScratchBytes = 32ull << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_dev_ptr[kMaxDevices];

// The current device's copy of `scratch`, looked up once per device (with that device current) and
// kept.
msa_status scratch_address(void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return MSA_ERR_LAUNCH;
    }
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_dev_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return MSA_ERR_LAUNCH;
        }
        scratch_dev_ptr[dev] = p;
    }
    *out = scratch_dev_ptr[dev];
    return MSA_OK;
}

}  // namespace

extern "C" {

msa_status msa_project_workspace_size(int32_t num_tokens, int32_t hidden, int32_t num_heads, uint64_t* bytes)
{
    if (!bytes) return MSA_ERR_NULL_POINTER;
    if (num_tokens < 0 || hidden <= 0 || hidden % kBK || num_heads <= 0 || num_heads > 4096) return MSA_ERR_SHAPE;
    if (num_tokens > 0 && num_tokens <= kSplitMaxTokens && hidden > kMaxSplits * kSliceMax) return MSA_ERR_SHAPE;
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
    const uint64_t need = workspace_need(num_tokens, hidden, num_cols / kHeadDim);
    if (need > 0 && (!workspace || !aligned(workspace, kAlign) || workspace_bytes < need)) return MSA_ERR_WORKSPACE;
    const Span spans[] = {
        {h, row_bytes(num_tokens, h_row_stride, hidden, 2)},
        {w, row_bytes(num_cols, w_row_stride, hidden, 2)},
        {x_out, row_bytes(num_tokens, x_row_stride, num_cols, 2)},
        {workspace, need},
    };
    if ((st = check_operands(spans, 4, static_cast<hipStream_t>(stream))) != MSA_OK) return st;
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
    return project_produce(h, h_row_stride, num_tokens, hidden, w, w_row_stride, head_dim, num_q_heads, num_kv_heads,
                           num_iq_heads, num_ik_heads, rope_cos, rope_sin, slots, page_size, num_pages, q_norm_weight,
                           k_norm_weight, iq_norm_weight, ik_norm_weight, rms_eps, q_out, iq_out, k_cache, v_cache,
                           ik_cache, workspace, workspace_bytes, static_cast<hipStream_t>(stream), false);
}

msa_status msa_project_produce_noalloc(const uint16_t* h, int64_t h_row_stride, int32_t num_tokens, int32_t hidden,
                                       const uint16_t* w, int64_t w_row_stride, int32_t head_dim,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t num_iq_heads,
                                       int32_t num_ik_heads, const float* rope_cos, const float* rope_sin,
                                       const int64_t* slots, int32_t page_size, int64_t num_pages,
                                       const uint16_t* q_norm_weight, const uint16_t* k_norm_weight,
                                       const uint16_t* iq_norm_weight, const uint16_t* ik_norm_weight,
                                       float rms_eps, uint16_t* q_out, uint16_t* iq_out,
                                       const msa_cache_view* k_cache, const msa_cache_view* v_cache,
                                       const msa_cache_view* ik_cache, void* stream)
{
    // Sizes first (nothing touches the device for a call that cannot fit).
    const int64_t heads = (int64_t)num_q_heads + 2 * (int64_t)num_kv_heads + num_iq_heads + num_ik_heads;
    if (num_tokens < 0 || heads < 1 || heads > 4096 || hidden <= 0 || hidden % kBK) return MSA_ERR_SHAPE;
    if (workspace_need(num_tokens, hidden, (int32_t)heads) > kScratchBytes) return MSA_ERR_WORKSPACE;
    void* scratch_dev = nullptr;
    if (num_tokens > 0) {
        const msa_status st = scratch_address(&scratch_dev);
        if (st != MSA_OK) return st;
    }
    return project_produce(h, h_row_stride, num_tokens, hidden, w, w_row_stride, head_dim, num_q_heads, num_kv_heads,
                           num_iq_heads, num_ik_heads, rope_cos, rope_sin, slots, page_size, num_pages, q_norm_weight,
                           k_norm_weight, iq_norm_weight, ik_norm_weight, rms_eps, q_out, iq_out, k_cache, v_cache,
                           ik_cache, scratch_dev, kScratchBytes, static_cast<hipStream_t>(stream), true);
}

}  // extern "C"
