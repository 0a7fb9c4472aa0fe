// The unfused producer path for CDNA4 (gfx950): the write path as it ran before the fusion, kept
// as the route for cache layouts the fused kernel does not take and as the other side of the
// launch-count comparison.  Structure: page "Fuse MiniMax-M3 MSA per-layer KV-cache writes into
// one kernel" ("The problem": division, remainder, index cast and an indexed scatter for each of
// K, V and index-K; summary: layouts the fused kernel cannot take use the per-cache writes);
// page "Wire in custom decode kernels for MinimaxM3" (commit notes of the ported fusion: before it,
// every cache tensor recomputed its slot's page and offset and converted the index on its own
// before its indexed store); page "Fuse MiniMax-M3 QKV and index projection" (BEFORE figure:
// separate main and index producers).
//
// Every rounding comes from the device arithmetic the fused kernel uses, in the same order, so
// both paths write the same bytes: the producers hold each head as 8 lanes x (8 + 8) elements
// exactly as the fused kernel does, and the normalised K / index-K rows travel through binary32,
// which the fused kernel also holds them in before the cast.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "msa_common.h"
#include "msa_device.h"
#include "msa_unfused.h"

namespace {

using namespace msa_internal;

constexpr int kWave = 64;
constexpr int kLanesPerHead = 8;
constexpr int kHeadsPerPass = kWave / kLanesPerHead;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr uint64_t kRegionAlign = 256;

// ------------------------------------------------------------------ step metadata

struct SlotArgs {
    const int32_t* pos;
    const int32_t* seq;
    const int32_t* pt;
    int64_t pt_stride;
    int64_t num_pages;
    int64_t* slots;
    int32_t T, S, max_pages, page_size;
};

__global__ __launch_bounds__(256) void slots_kernel(const SlotArgs a)
{
    const int32_t t = (int32_t)(blockIdx.x * 256 + threadIdx.x);
    if (t >= a.T) return;
    const int32_t pos = a.pos[t];
    const int32_t sq = a.seq[t];
    int64_t slot = -1;
    if (sq >= 0 && sq < a.S && pos >= 0) {
        const int32_t lp = pos / a.page_size;
        if (lp < a.max_pages) {
            const int64_t pg = a.pt[(int64_t)sq * a.pt_stride + lp];
            if (pg >= 0 && pg < a.num_pages) slot = pg * a.page_size + (pos - lp * a.page_size);
        }
    }
    a.slots[t] = slot;
}

// ------------------------------------------------------------------ norm + RoPE producers

// One producer over two consecutive head streams of the row: A (Q or index-Q; bf16 output) and
// B (K or index-K; binary32 output).  One wave per (token, group of 8 heads).
struct NormRopeArgs {
    const uint16_t* x;
    int64_t x_stride;
    const int32_t* pos;
    const uint16_t* w_a;
    const uint16_t* w_b;
    uint16_t* out_a;           // [T, ha, 128] bf16
    float* out_b;              // [T, hb, 128] binary32
    int32_t T, col0, ha, hb, npass;
    float eps;
    double inv_freq[kHalf];
};

__global__ __launch_bounds__(kBlock) void norm_rope_kernel(const NormRopeArgs a)
{
    __shared__ __attribute__((aligned(16))) float cs_lds[kWavesPerBlock][2 * kHalf];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t item = blockIdx.x * kWavesPerBlock + wave;
    if (item >= (uint32_t)a.T * (uint32_t)a.npass) return;   // wave-uniform
    const int32_t t = (int32_t)(item / (uint32_t)a.npass);
    const int pass = (int)(item - (uint32_t)t * (uint32_t)a.npass);
    const int hs = lane / kLanesPerHead;
    const int sub = lane % kLanesPerHead;
    const int total = a.ha + a.hb;
    const int h = pass * kHeadsPerPass + hs;
    const int hc = h < total ? h : total - 1;   // idle slots compute the last head, store nothing

    const uint16_t* hp = a.x + (int64_t)t * a.x_stride + a.col0 + (int64_t)hc * kHeadDim + sub * 8;
    const uint4 xa = *reinterpret_cast<const uint4*>(hp);
    const uint4 xb = *reinterpret_cast<const uint4*>(hp + kHalf);
    const uint16_t* w = (hc < a.ha ? a.w_a : a.w_b) + sub * 8;
    const uint4 wa = *reinterpret_cast<const uint4*>(w);
    const uint4 wb = *reinterpret_cast<const uint4*>(w + kHalf);

    {
        float c, s;
        rope_coeff(a.pos[t], a.inv_freq[lane], &c, &s);
        cs_lds[wave][lane] = c;
        cs_lds[wave][kHalf + lane] = s;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    float u[16], wv[16];
    unpack8(xa, u);
    unpack8(xb, u + 8);
    unpack8(wa, wv);
    unpack8(wb, wv + 8);
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc = __builtin_fma((double)u[j], (double)u[j], acc);
    const float r = rms_from_ss(head_sum8(acc), a.eps);

    float cf[8], sf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        cf[j] = cs_lds[wave][sub * 8 + j];
        sf[j] = cs_lds[wave][kHalf + sub * 8 + j];
    }
    float y[16], o[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) y[j] = (u[j] * r) * wv[j];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        o[j] = y[j] * cf[j] - y[j + 8] * sf[j];
        o[j + 8] = y[j + 8] * cf[j] + y[j] * sf[j];
    }
    if (h >= total) return;
    if (h < a.ha) {
        uint16_t* dst = a.out_a + ((int64_t)t * a.ha + h) * kHeadDim + sub * 8;
        *reinterpret_cast<uint4*>(dst) = bf16x8(o);
        *reinterpret_cast<uint4*>(dst + kHalf) = bf16x8(o + 8);
    } else {
        float* dst = a.out_b + ((int64_t)t * a.hb + (h - a.ha)) * kHeadDim + sub * 8;
        reinterpret_cast<float4*>(dst)[0] = make_float4(o[0], o[1], o[2], o[3]);
        reinterpret_cast<float4*>(dst)[1] = make_float4(o[4], o[5], o[6], o[7]);
        reinterpret_cast<float4*>(dst + kHalf)[0] = make_float4(o[8], o[9], o[10], o[11]);
        reinterpret_cast<float4*>(dst + kHalf)[1] = make_float4(o[12], o[13], o[14], o[15]);
    }
}

// ------------------------------------------------------------------ per-cache write kernels

__global__ __launch_bounds__(256) void slot_div_kernel(const int64_t* slots, int32_t T, int32_t page_size,
                                                       int64_t* page)
{
    const int32_t t = (int32_t)(blockIdx.x * 256 + threadIdx.x);
    if (t < T) page[t] = slots[t] >= 0 ? slots[t] / page_size : -1;
}

__global__ __launch_bounds__(256) void slot_rem_kernel(const int64_t* slots, int32_t T, int32_t page_size,
                                                       int64_t* off)
{
    const int32_t t = (int32_t)(blockIdx.x * 256 + threadIdx.x);
    if (t < T) off[t] = slots[t] >= 0 ? slots[t] % page_size : -1;
}

// (page, offset) -> element index of (page, head 0, offset, dim 0), or -1.  A page outside the
// pool is contained here; the element index of a page inside it fits in int64 (checked on the
// host against the view's largest offset).
__global__ __launch_bounds__(256) void index_cast_kernel(const int64_t* page, const int64_t* off, int32_t T,
                                                         int64_t num_pages, int64_t stride_page,
                                                         int64_t stride_token, int64_t* index)
{
    const int32_t t = (int32_t)(blockIdx.x * 256 + threadIdx.x);
    if (t >= T) return;
    const int64_t p = page[t];
    index[t] = p >= 0 && p < num_pages ? p * stride_page + off[t] * stride_token : -1;
}

// Source rows: binary32 compact [T, heads, 128] (normalised K / index-K) or bf16 rows of the
// packed input (V, raw).
struct ScatterArgs {
    const void* src;
    int64_t src_stride;        // elements between tokens
    const int64_t* index;
    CacheDev c;
    int32_t T, heads, src_bf16;
};

// VW elements per thread: 8 when the cache layout allows 8-element stores (16-byte aligned base,
// strides multiples of 8 elements), else 1.
template <int VW>
__global__ __launch_bounds__(256) void scatter_kernel(const ScatterArgs a)
{
    constexpr int kPerRow = kHeadDim / VW;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = i / kPerRow;
    if (row >= (int64_t)a.T * a.heads) return;
    const int d = (int)(i - row * kPerRow) * VW;
    const int32_t t = (int32_t)(row / a.heads);
    const int32_t h = (int32_t)(row - (int64_t)t * a.heads);
    const int64_t base = a.index[t];
    if (base < 0) return;

    float v[VW];
    if (a.src_bf16) {
        const uint16_t* s = static_cast<const uint16_t*>(a.src) + (int64_t)t * a.src_stride + h * kHeadDim + d;
        if (VW == 8) {
            unpack8(*reinterpret_cast<const uint4*>(s), v);
        } else {
#pragma unroll
            for (int j = 0; j < VW; ++j) v[j] = __uint_as_float((uint32_t)s[j] << 16);
        }
    } else {
        const float* s = static_cast<const float*>(a.src) + (int64_t)t * a.src_stride + h * kHeadDim + d;
#pragma unroll
        for (int j = 0; j < VW; ++j) v[j] = s[j];
    }
    const int64_t e = base + (int64_t)h * a.c.sh + d;
    if (a.c.is_bf16) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(a.c.data) + e;
        if (VW == 8) {
            *reinterpret_cast<uint4*>(dst) = bf16x8(v);
        } else {
#pragma unroll
            for (int j = 0; j < VW; ++j) dst[j] = (uint16_t)bf16x2(v[j], 0.0f);
        }
    } else {
        const float m = inv_scale_of(a.c.scale);
        uint8_t* dst = a.c.data + e;
        if (VW == 8) {
            const uint32_t lo = e4m3x4(v[0] * m, v[1] * m, v[2] * m, v[3] * m);
            const uint32_t hi = e4m3x4(v[4] * m, v[5] * m, v[6] * m, v[7] * m);
            *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
        } else {
#pragma unroll
            for (int j = 0; j < VW; ++j) dst[j] = (uint8_t)e4m3x4(v[j] * m, 0.0f, 0.0f, 0.0f);
        }
    }
}

// ------------------------------------------------------------------ host side

hipError_t launch(const void* fn, int64_t threads, void** args, hipStream_t s)
{
    const dim3 grid((unsigned)((threads + 255) / 256));
    return hipLaunchKernel(fn, grid, dim3(256), args, 0, s);
}

struct Workspace {
    uint64_t k_f32, ik_f32, page[3], off[3], index[3], total;
};

uint64_t round_up(uint64_t v) { return (v + kRegionAlign - 1) / kRegionAlign * kRegionAlign; }

Workspace layout(int32_t T, int32_t hkv, int32_t hik)
{
    Workspace w;
    uint64_t o = 0;
    w.k_f32 = o;
    o += round_up((uint64_t)T * hkv * kHeadDim * sizeof(float));
    w.ik_f32 = o;
    o += round_up((uint64_t)T * hik * kHeadDim * sizeof(float));
    for (int c = 0; c < 3; ++c) {
        w.page[c] = o;
        o += round_up((uint64_t)T * sizeof(int64_t));
        w.off[c] = o;
        o += round_up((uint64_t)T * sizeof(int64_t));
        w.index[c] = o;
        o += round_up((uint64_t)T * sizeof(int64_t));
    }
    w.total = o;
    return w;
}

// Whether a validated cache takes the 8-element stores.
bool vector_layout(const CacheDev& c)
{
    return aligned(c.data, 16) && c.sp % 8 == 0 && c.sh % 8 == 0 && c.st % 8 == 0;
}

}  // namespace

extern "C" {

msa_status msa_slots(const int32_t* positions, const int32_t* seq_idx, int32_t num_tokens,
                     const int32_t* page_table, int64_t page_table_stride, int32_t num_seqs,
                     int32_t max_pages_per_seq, int32_t page_size, int64_t num_pages,
                     int64_t* slots_out, void* stream)
{
    if (num_tokens < 0 || page_size <= 0 || num_seqs < 0 || max_pages_per_seq < 0 || num_pages < 0)
        return MSA_ERR_SHAPE;
    if (num_seqs > 0 && page_table_stride < max_pages_per_seq) return MSA_ERR_STRIDE;
    int64_t tmp;
    if (__builtin_mul_overflow(num_pages, (int64_t)page_size, &tmp)) return MSA_ERR_OVERFLOW;
    if (num_seqs > 0 && __builtin_mul_overflow((int64_t)num_seqs, page_table_stride, &tmp)) return MSA_ERR_OVERFLOW;
    if (num_tokens == 0) return MSA_OK;
    if (!positions || !seq_idx || !slots_out) return MSA_ERR_NULL_POINTER;
    if (num_seqs > 0 && max_pages_per_seq > 0 && !page_table) return MSA_ERR_NULL_POINTER;
    if (!aligned(positions, 4) || !aligned(seq_idx, 4) || !aligned(page_table, 4) || !aligned(slots_out, 8))
        return MSA_ERR_ALIGNMENT;
    SlotArgs a;
    a.pos = positions;
    a.seq = seq_idx;
    a.pt = page_table;
    a.pt_stride = page_table_stride;
    a.num_pages = num_pages;
    a.slots = slots_out;
    a.T = num_tokens;
    a.S = num_seqs;
    a.max_pages = max_pages_per_seq;
    a.page_size = page_size;
    const Span spans[] = {{positions, nbytes(num_tokens, 4)}, {seq_idx, nbytes(num_tokens, 4)},
                          {page_table, num_seqs > 0 ? row_bytes(num_seqs, page_table_stride, max_pages_per_seq, 4) : 0},
                          {slots_out, nbytes(num_tokens, 8)}};
    const msa_status st = check_operands(spans, 4, static_cast<hipStream_t>(stream));
    if (st != MSA_OK) return st;
    void* args[] = {&a};
    const hipError_t e = launch(reinterpret_cast<const void*>(&slots_kernel), num_tokens, args,
                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MSA_OK : MSA_ERR_LAUNCH;
}

msa_status msa_produce_unfused_workspace_size(int32_t num_tokens, int32_t num_kv_heads, int32_t num_ik_heads,
                                              uint64_t* bytes)
{
    if (!bytes) return MSA_ERR_NULL_POINTER;
    if (num_tokens < 0 || num_kv_heads < 0 || num_ik_heads < 0 || num_kv_heads > 4096 || num_ik_heads > 4096)
        return MSA_ERR_SHAPE;
    *bytes = layout(num_tokens, num_kv_heads, num_ik_heads).total;
    return MSA_OK;
}

msa_status msa_produce_unfused(const uint16_t* x, int64_t x_row_stride, int32_t num_tokens, int32_t head_dim,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t num_iq_heads,
                               int32_t num_ik_heads, const int32_t* positions, const int64_t* slots,
                               int32_t page_size, int64_t num_pages,
                               const uint16_t* q_norm_weight, const uint16_t* k_norm_weight,
                               const uint16_t* iq_norm_weight, const uint16_t* ik_norm_weight,
                               float rms_eps, double rope_theta,
                               uint16_t* q_out, uint16_t* iq_out,
                               const msa_cache_view* k_cache, const msa_cache_view* v_cache,
                               const msa_cache_view* ik_cache,
                               void* workspace, uint64_t workspace_bytes, void* stream)
{
    if (head_dim != kHeadDim) return MSA_ERR_UNSUPPORTED;
    if (num_tokens < 0 || num_q_heads < 0 || num_kv_heads < 0 || num_iq_heads < 0 || num_ik_heads < 0)
        return MSA_ERR_SHAPE;
    const int64_t heads_total = (int64_t)num_q_heads + 2 * (int64_t)num_kv_heads + num_iq_heads + num_ik_heads;
    if (heads_total < 1 || heads_total > 4096) return MSA_ERR_SHAPE;
    if (page_size <= 0 || num_pages < 0) return MSA_ERR_SHAPE;
    if (!(rms_eps >= 0.0f) || !(rope_theta > 0.0) || !std::isfinite(rope_theta)) return MSA_ERR_SHAPE;
    if (x_row_stride < heads_total * kHeadDim || x_row_stride % 8) return MSA_ERR_STRIDE;
    if (num_tokens > 0) {
        if (!x || !positions || !slots) return MSA_ERR_NULL_POINTER;
        if ((num_q_heads > 0 && !q_out) || (num_iq_heads > 0 && !iq_out)) return MSA_ERR_NULL_POINTER;
    }
    if ((num_q_heads > 0 && !q_norm_weight) || (num_kv_heads > 0 && !k_norm_weight) ||
        (num_iq_heads > 0 && !iq_norm_weight) || (num_ik_heads > 0 && !ik_norm_weight))
        return MSA_ERR_NULL_POINTER;
    if (!aligned(x, 16) || !aligned(q_out, 16) || !aligned(iq_out, 16) || !aligned(positions, 4) ||
        !aligned(slots, 8) || !aligned(q_norm_weight, 16) || !aligned(k_norm_weight, 16) ||
        !aligned(iq_norm_weight, 16) || !aligned(ik_norm_weight, 16))
        return MSA_ERR_ALIGNMENT;
    int64_t tmp;
    if (__builtin_mul_overflow((int64_t)num_tokens, x_row_stride, &tmp)) return MSA_ERR_OVERFLOW;
    CacheDev cache[3];
    uint64_t cache_span[3];
    msa_status st;
    for (int c = 0; c < 3; ++c) {
        const msa_cache_view* v = c == 0 ? k_cache : c == 1 ? v_cache : ik_cache;
        if ((st = check_cache(v, c == 2 ? num_ik_heads : num_kv_heads, page_size, num_pages, &cache[c], false,
                              &cache_span[c])) != MSA_OK)
            return st;
    }
    if (__builtin_mul_overflow(num_pages, (int64_t)page_size, &tmp)) return MSA_ERR_OVERFLOW;
    const Workspace ws = layout(num_tokens, num_kv_heads, num_ik_heads);
    if (num_tokens == 0) return MSA_OK;
    if (!workspace || !aligned(workspace, kRegionAlign) || workspace_bytes < ws.total) return MSA_ERR_WORKSPACE;
    if ((int64_t)num_tokens * heads_total > ((int64_t)1 << 31)) return MSA_ERR_SHAPE;   // grid sizes

    hipStream_t s = static_cast<hipStream_t>(stream);
    {
        const Span spans[] = {
            {x, row_bytes(num_tokens, x_row_stride, heads_total * kHeadDim, 2)},
            {positions, nbytes(num_tokens, 4)},
            {slots, nbytes(num_tokens, 8)},
            {q_norm_weight, 2 * kHeadDim}, {k_norm_weight, 2 * kHeadDim},
            {iq_norm_weight, 2 * kHeadDim}, {ik_norm_weight, 2 * kHeadDim},
            {q_out, nbytes((int64_t)num_tokens * num_q_heads * kHeadDim, 2)},
            {iq_out, nbytes((int64_t)num_tokens * num_iq_heads * kHeadDim, 2)},
            {cache[0].data, cache_span[0]}, {cache[1].data, cache_span[1]}, {cache[2].data, cache_span[2]},
            {cache[0].scale, 4}, {cache[1].scale, 4}, {cache[2].scale, 4},
            {workspace, ws.total},
        };
        if ((st = check_operands(spans, sizeof(spans) / sizeof(spans[0]), s)) != MSA_OK) return st;
    }
    uint8_t* w = static_cast<uint8_t*>(workspace);
    float* k_f32 = reinterpret_cast<float*>(w + ws.k_f32);
    float* ik_f32 = reinterpret_cast<float*>(w + ws.ik_f32);
    double inv_freq[kHalf];
    fill_inv_freq(rope_theta, inv_freq);

    // Main producer (Q, K), then index producer (index-Q, index-K).
    const int32_t col_iq = (int32_t)((num_q_heads + 2 * num_kv_heads) * kHeadDim);
    const struct {
        int32_t col0, ha, hb;
        const uint16_t *wa, *wb;
        uint16_t* oa;
        float* ob;
    } prod[2] = {{0, num_q_heads, num_kv_heads, q_norm_weight, k_norm_weight, q_out, k_f32},
                 {col_iq, num_iq_heads, num_ik_heads, iq_norm_weight, ik_norm_weight, iq_out, ik_f32}};
    for (const auto& p : prod) {
        if (p.ha + p.hb == 0) continue;
        NormRopeArgs a;
        std::memset(&a, 0, sizeof(a));
        a.x = x;
        a.x_stride = x_row_stride;
        a.pos = positions;
        a.w_a = p.ha ? p.wa : p.wb;    // a stream without heads reads the other's weights, unused
        a.w_b = p.hb ? p.wb : p.wa;
        a.out_a = p.oa;
        a.out_b = p.ob;
        a.T = num_tokens;
        a.col0 = p.col0;
        a.ha = p.ha;
        a.hb = p.hb;
        a.npass = (p.ha + p.hb + kHeadsPerPass - 1) / kHeadsPerPass;
        a.eps = rms_eps;
        std::memcpy(a.inv_freq, inv_freq, sizeof(inv_freq));
        const int64_t waves = (int64_t)num_tokens * a.npass;
        if (waves + kWavesPerBlock > 0x7fffffffLL) return MSA_ERR_SHAPE;
        void* args[] = {&a};
        const dim3 grid((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock));
        if (hipLaunchKernel(reinterpret_cast<const void*>(&norm_rope_kernel), grid, dim3(kBlock), args, 0, s) !=
            hipSuccess)
            return MSA_ERR_LAUNCH;
    }

    // The three cache writes, four launches each.
    const struct {
        const void* src;
        int64_t src_stride;
        int32_t heads, src_bf16;
    } srcs[3] = {{k_f32, (int64_t)num_kv_heads * kHeadDim, num_kv_heads, 0},
                 {x + (int64_t)(num_q_heads + num_kv_heads) * kHeadDim, x_row_stride, num_kv_heads, 1},
                 {ik_f32, (int64_t)num_ik_heads * kHeadDim, num_ik_heads, 0}};
    for (int c = 0; c < 3; ++c) {
        if (srcs[c].heads == 0) continue;
        int64_t* page = reinterpret_cast<int64_t*>(w + ws.page[c]);
        int64_t* off = reinterpret_cast<int64_t*>(w + ws.off[c]);
        int64_t* index = reinterpret_cast<int64_t*>(w + ws.index[c]);
        int32_t T = num_tokens, P = page_size;
        int64_t np = num_pages, sp = cache[c].sp, stt = cache[c].st;
        void* a_div[] = {const_cast<int64_t**>(&slots), &T, &P, &page};
        void* a_rem[] = {const_cast<int64_t**>(&slots), &T, &P, &off};
        void* a_idx[] = {&page, &off, &T, &np, &sp, &stt, &index};
        ScatterArgs sa;
        sa.src = srcs[c].src;
        sa.src_stride = srcs[c].src_stride;
        sa.index = index;
        sa.c = cache[c];
        sa.T = num_tokens;
        sa.heads = srcs[c].heads;
        sa.src_bf16 = srcs[c].src_bf16;
        void* a_sc[] = {&sa};
        const bool vec = vector_layout(cache[c]);
        const int64_t rows = (int64_t)num_tokens * srcs[c].heads;
        if (launch(reinterpret_cast<const void*>(&slot_div_kernel), num_tokens, a_div, s) != hipSuccess ||
            launch(reinterpret_cast<const void*>(&slot_rem_kernel), num_tokens, a_rem, s) != hipSuccess ||
            launch(reinterpret_cast<const void*>(&index_cast_kernel), num_tokens, a_idx, s) != hipSuccess)
            return MSA_ERR_LAUNCH;
        const hipError_t e = vec ? launch(reinterpret_cast<const void*>(&scatter_kernel<8>), rows * (kHeadDim / 8), a_sc, s)
                                 : launch(reinterpret_cast<const void*>(&scatter_kernel<1>), rows * kHeadDim, a_sc, s);
        if (e != hipSuccess) return MSA_ERR_LAUNCH;
    }
    return MSA_OK;
}

}  // extern "C"
