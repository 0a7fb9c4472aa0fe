// MiniMax-M3 MSA fused producer for CDNA4 (gfx950): per-head RMSNorm + neox RoPE on the Q, K,
// index-Q and index-K heads of one packed projection row per token, compact bf16 Q / index-Q,
// and K / V / index-K scattered into paged HND caches (OCP FP8 E4M3 or bf16), one launch per
// layer.  Operation: page "Fuse MiniMax-M3 QKV and index projection" (AFTER figure, change
// list); page/offset computed once per token and the three cache writes fused: page "Fuse
// MiniMax-M3 MSA per-layer KV-cache writes into one kernel" ("The problem", "The fix", "Nsys
// trace"); slots derived from the page table: page "Wire in custom decode kernels for
// MinimaxM3" (conflict-resolution commit notes).  The arithmetic reading is documented in
// include/msa_produce.h.
//
// Work decomposition.  head_dim is 128 = 8 lanes x (8 first-half + 8 second-half elements):
// lane `sub` of a head holds elements [8 sub, 8 sub + 8) and [64 + 8 sub, 64 + 8 sub + 8), so
// both members of every rotate-half pair (i, i + 64) sit in the same lane and RoPE needs no
// cross-lane exchange.  A wavefront (64 lanes) covers 8 heads per pass with two 16-byte loads
// per lane (1 KiB contiguous per head-row pair); 23 heads take 3 passes.  The per-head sum of
// squares is reduced over the 8 lanes of a head with three DPP steps in binary64.  Each wave
// computes its token's 64 RoPE coefficient pairs once (one binary64 sincos per lane) and
// broadcasts them through LDS.  Token metadata (position, sequence, page-table entry) is
// wave-uniform and read once per wave; cache offsets are 64-bit.  Large batches run one wave per
// token (all passes); small batches split a token's passes over several waves to spread the
// latency.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "msa_common.h"
#include "msa_device.h"
#include "msa_produce.h"

namespace {

using namespace msa_internal;

constexpr int kWave = 64;
constexpr int kLanesPerHead = 8;
constexpr int kHeadsPerPass = kWave / kLanesPerHead;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kMaxPassesPerWave = 4;

enum Stream { kQ = 0, kK = 1, kV = 2, kIQ = 3, kIK = 4 };

struct ProduceArgs {
    const uint16_t* x;
    int64_t x_stride;
    const int32_t* pos;
    const int32_t* seq;
    const int32_t* pt;
    int64_t pt_stride;
    int64_t num_pages;
    int32_t T, S, max_pages, page_size, page_shift;   // page_shift = log2(page_size), or -1
    int32_t hq, hkv, hiq, hik, heads_total, npass, waves_per_token;
    float eps;
    const uint16_t* w[4];      // norm weights of Q, K, index-Q, index-K
    uint16_t* q_out;
    uint16_t* iq_out;
    CacheDev cache[3];         // K, V, index-K
    int64_t* slots_out;
    double inv_freq[kHalf];
};

struct FreqArgs {
    double inv_freq[kHalf];
};

// One float through a buffer load of a 4-byte range: always a vector memory instruction, even at a
// wave-uniform address.  Vector loads retire in issue order, so a later wait for an earlier load
// does not wait for this one, whereas a scalar load would join the next wait for the (scalar) token
// metadata.  The range check returns 0 outside the 4 bytes and cannot fault.
__device__ __forceinline__ float vector_load_f32(const float* p)
{
    // 0x00020000: the gfx9-family word 3 of a raw (untyped, dword) buffer resource.
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, 4, 0x00020000);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0));
}

// Stream of head slot h (h < heads_total) in the packed row order Q, K, V, index-Q, index-K.
__device__ __forceinline__ int stream_of(int h, int h_k, int h_v, int h_iq, int h_ik)
{
    return h < h_k ? kQ : h < h_v ? kK : h < h_iq ? kV : h < h_ik ? kIQ : kIK;
}

// One of three wave-uniform values, chosen per lane.
template <typename V>
__device__ __forceinline__ V sel3(int i, V v0, V v1, V v2) { return i == 0 ? v0 : i == 1 ? v1 : v2; }

// One producer launch.  PPW = passes (groups of 8 heads) per wave.  HQ..HIK fix the head
// geometry at compile time (the stream of every head slot then folds to constants); all four
// negative selects the generic build that reads the geometry from the arguments.
template <int PPW, int HQ, int HKV, int HIQ, int HIK>
__global__ __launch_bounds__(kBlock) void produce_kernel(const ProduceArgs a)
{
    constexpr bool kFixed = HQ >= 0;
    constexpr int kTotal = HQ + 2 * HKV + HIQ + HIK;
    constexpr int kNpass = kFixed ? (kTotal + kHeadsPerPass - 1) / kHeadsPerPass : -1;
    // With a fixed geometry whose passes all fit one wave, every wave starts at pass 0.
    constexpr bool kWholeToken = kFixed && kNpass <= PPW;
    // Several passes per wave (large batches): stage the norm weights in LDS (one copy per wave, so
    // waves never wait on each other), and stream the input rows and the outputs (nontemporal loads
    // and stores: 1% and 7% faster on the 65,536-token prefill, measured).
    constexpr bool kStageW = PPW > 1;
    constexpr bool kStream = PPW > 1;

    const int hq = kFixed ? HQ : a.hq;
    const int hkv = kFixed ? HKV : a.hkv;
    const int hiq = kFixed ? HIQ : a.hiq;
    const int heads_total = kFixed ? kTotal : a.heads_total;
    const int npass = kFixed ? kNpass : a.npass;
    const int h_k = hq, h_v = hq + hkv, h_iq = hq + 2 * hkv, h_ik = h_iq + hiq;

    __shared__ __attribute__((aligned(16))) float w_lds[kStageW ? kWavesPerBlock : 1][kStageW ? 4 : 1][kHeadDim];
    __shared__ __attribute__((aligned(16))) float cs_lds[kWavesPerBlock][2 * kHalf];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t item = blockIdx.x * kWavesPerBlock + wave;
    const bool live = item < (uint32_t)a.T * (uint32_t)a.waves_per_token;   // wave-uniform
    int32_t t, chunk;
    if (kWholeToken || a.waves_per_token == 1) {
        t = (int32_t)item;
        chunk = 0;
    } else {
        t = (int32_t)(item / (uint32_t)a.waves_per_token);
        chunk = (int32_t)(item - (uint32_t)t * (uint32_t)a.waves_per_token);
    }
    const int pass0 = kWholeToken ? 0 : chunk * PPW;

    const int hs = lane / kLanesPerHead;   // head slot within a pass
    const int sub = lane % kLanesPerHead;  // element group within the head

    // Loads that do not depend on the token metadata go out first, so that their memory round
    // trips overlap one another instead of following the arithmetic (on the decode critical path):
    // this lane's RoPE frequency, the fp8 dequantisation scales, a one-pass wave's norm weights,
    // then the rows.  A V head (no norm) reads its "weights" from the input row instead, a valid
    // address, and discards them.
    const double freq = a.inv_freq[lane];
    // Waves with several passes (large batches, bound by bandwidth) read the scales at the cast
    // instead, which keeps three registers free.
    float scale_v[3] = {1.0f, 1.0f, 1.0f};
    if (PPW == 1) {
#pragma unroll
        for (int c = 0; c < 3; ++c)   // no scale (bf16 cache, or no heads): read the row instead, unused
            scale_v[c] = vector_load_f32(a.cache[c].scale ? a.cache[c].scale : reinterpret_cast<const float*>(a.x));
    }
    uint4 wa = make_uint4(0, 0, 0, 0), wb = make_uint4(0, 0, 0, 0);
    if (!kStageW) {
        const int h = pass0 * kHeadsPerPass + hs;
        const int st = stream_of(h < heads_total ? h : heads_total - 1, h_k, h_v, h_iq, h_ik);
        // all four pointers first, then a per-lane choice by value (no branch per stream)
        const uint16_t* const w0 = a.w[0] ? a.w[0] : a.x;
        const uint16_t* const w1 = a.w[1] ? a.w[1] : a.x;
        const uint16_t* const w2 = a.w[2] ? a.w[2] : a.x;
        const uint16_t* const w3 = a.w[3] ? a.w[3] : a.x;
        const uint16_t* const w = st == kQ ? w0 : st == kK ? w1 : st == kIQ ? w2 : st == kIK ? w3 : a.x;
        wa = *reinterpret_cast<const uint4*>(w + sub * 8);
        wb = *reinterpret_cast<const uint4*>(w + kHalf + sub * 8);
    }

    // Row loads of every pass of this wave.  Slots past the last head (and waves past the last
    // token) read the token's first head instead, a valid address, and discard it.
    const int32_t t_ld = live ? t : 0;
    const uint16_t* row = a.x + (int64_t)t_ld * a.x_stride + sub * 8;
    uint4 xa[PPW], xb[PPW];
#pragma unroll
    for (int k = 0; k < PPW; ++k) {
        const int h = (pass0 + k) * kHeadsPerPass + hs;
        const uint16_t* hp = row + (h < heads_total ? h : 0) * kHeadDim;
        xa[k] = load16<kStream>(hp);
        xb[k] = load16<kStream>(hp + kHalf);
    }

    if (kStageW) {
        // Each wave stages its own copy (no block barrier): lane L converts weights [8L, 8L + 8) of
        // the 512 (stream L / 16).
        const uint16_t* w = a.w[lane / 16];
        float* dst = &w_lds[wave][lane / 16][(lane % 16) * 8];
        if (w) {
            float f[8];
            unpack8(*reinterpret_cast<const uint4*>(w + (lane % 16) * 8), f);
            reinterpret_cast<float4*>(dst)[0] = make_float4(f[0], f[1], f[2], f[3]);
            reinterpret_cast<float4*>(dst)[1] = make_float4(f[4], f[5], f[6], f[7]);
        } else {
            reinterpret_cast<float4*>(dst)[0] = make_float4(0.f, 0.f, 0.f, 0.f);
            reinterpret_cast<float4*>(dst)[1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }

    // Token metadata, once per wave (wave-uniform).  The page-table entry is read without a
    // branch (an invalid slot reads the position array instead, a valid address) so that the
    // RoPE coefficients are computed while the entry is in flight.
    const int32_t pos = a.pos[t_ld];
    const int32_t sq = a.seq[t_ld];
    const bool seq_ok = live && sq >= 0 && sq < a.S && pos >= 0;
    const int32_t lp = a.page_shift >= 0 ? pos >> a.page_shift : pos / a.page_size;
    const bool lp_ok = seq_ok && lp < a.max_pages;
    const int32_t* pte = lp_ok ? a.pt + ((int64_t)sq * a.pt_stride + lp) : a.pos;
    const int64_t pg = *pte;
    {
        // RoPE coefficients of this token: lane i computes frequency i.
        float c, s;
        rope_coeff(pos, freq, &c, &s);
        cs_lds[wave][lane] = c;
        cs_lds[wave][kHalf + lane] = s;
    }
    const bool valid = lp_ok && pg >= 0 && pg < a.num_pages;
    const int64_t page = valid ? pg : -1;
    const int32_t off = valid ? pos - lp * a.page_size : 0;
    if (!live) return;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // One-pass waves: this token's row in each cache (head 0, element 0) as a byte address, and the
    // head stride in bytes, wave-uniform and once per wave; lanes then pick their cache by value
    // (indexing the descriptors by a per-lane cache number would load them from the argument
    // segment with vector loads, one more memory round trip before the stores).
    uint8_t* row_base[3] = {nullptr, nullptr, nullptr};
    int64_t head_bytes[3] = {0, 0, 0};
    bool c_bf16[3] = {false, false, false};
#pragma unroll
    for (int c = 0; c < (PPW == 1 ? 3 : 0); ++c) {
        const CacheDev& cd = a.cache[c];
        c_bf16[c] = cd.is_bf16 != 0;
        const int64_t esz = c_bf16[c] ? 2 : 1;
        // Only used when the slot is valid and the cache has heads; formed unconditionally (a guard
        // here made the compiler wait for the page-table entry early: 5% slower per decode call).
        row_base[c] = cd.data + (page * cd.sp + (int64_t)off * cd.st) * esz;
        head_bytes[c] = cd.sh * esz;
    }

    float cf[8], sf[8];
    {
        const float4* cp = reinterpret_cast<const float4*>(&cs_lds[wave][sub * 8]);
        const float4* sp = reinterpret_cast<const float4*>(&cs_lds[wave][kHalf + sub * 8]);
        const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
        cf[0] = c0.x; cf[1] = c0.y; cf[2] = c0.z; cf[3] = c0.w; cf[4] = c1.x; cf[5] = c1.y; cf[6] = c1.z; cf[7] = c1.w;
        sf[0] = s0.x; sf[1] = s0.y; sf[2] = s0.z; sf[3] = s0.w; sf[4] = s1.x; sf[5] = s1.y; sf[6] = s1.z; sf[7] = s1.w;
    }

    // Sums of squares of every pass in binary64 (each square exact), reduced over the 8 lanes of
    // each head.  Rows stay packed between this phase and the per-pass work below, which unpacks
    // them again: that keeps the register footprint at five waves per SIMD.
    double ss[PPW];
#pragma unroll
    for (int k = 0; k < PPW; ++k) {
        float u[16];
        unpack8(xa[k], u);
        unpack8(xb[k], u + 8);
        double acc = 0.0;
#pragma unroll
        for (int j = 0; j < 16; ++j) acc = __builtin_fma((double)u[j], (double)u[j], acc);
        ss[k] = head_sum8(acc);
    }
    // RMSNorm scales: with several passes, lane `sub` of a head group computes the scale of pass
    // `sub` once and the group reads it back.
    float r[PPW];
    if (PPW == 1) {
        r[0] = rms_from_ss(ss[0], a.eps);
    } else {
        double mine = ss[0];
#pragma unroll
        for (int k = 1; k < PPW; ++k)
            if (sub == k) mine = ss[k];
        const float rm = rms_from_ss(mine, a.eps);
#pragma unroll
        for (int k = 0; k < PPW; ++k) r[k] = __shfl(rm, hs * kLanesPerHead + k);
    }

#pragma unroll
    for (int k = 0; k < PPW; ++k) {
        const int pass = pass0 + k;
        if (pass >= npass) break;                   // wave-uniform
        const int h = pass * kHeadsPerPass + hs;
        // Slots past the last head compute as the last head (its stream has heads, so its weight
        // pointer is valid) and store nothing.
        const int hc = h < heads_total ? h : heads_total - 1;
        const int st = stream_of(hc, h_k, h_v, h_iq, h_ik);

        // Keep each pass's temporaries from being hoisted into the previous pass (register footprint).
        __builtin_amdgcn_sched_barrier(0);
        float v[1][16];
        unpack8(xa[k], v[0]);
        unpack8(xb[k], v[0] + 8);
        float o[16];
        if (st == kV) {
#pragma unroll
            for (int j = 0; j < 16; ++j) o[j] = v[0][j];
        } else {
            const int ws = st == kQ ? 0 : st == kK ? 1 : st == kIQ ? 2 : 3;
            float wv[16];
            if (kStageW) {
                const float4* wp = reinterpret_cast<const float4*>(&w_lds[wave][ws][sub * 8]);
                const float4* wq = reinterpret_cast<const float4*>(&w_lds[wave][ws][kHalf + sub * 8]);
                const float4 w0 = wp[0], w1 = wp[1], w2 = wq[0], w3 = wq[1];
                wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w; wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
                wv[8] = w2.x; wv[9] = w2.y; wv[10] = w2.z; wv[11] = w2.w; wv[12] = w3.x; wv[13] = w3.y; wv[14] = w3.z; wv[15] = w3.w;
            } else {
                unpack8(wa, wv);         // one pass per wave: loaded at the top
                unpack8(wb, wv + 8);
            }
            float y[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) y[j] = (v[0][j] * r[k]) * wv[j];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                o[j] = y[j] * cf[j] - y[j + 8] * sf[j];
                o[j + 8] = y[j + 8] * cf[j] + y[j] * sf[j];
            }
        }
        if (h >= heads_total) continue;

        if (st == kQ || st == kIQ) {
            uint16_t* dst = st == kQ ? a.q_out + ((int64_t)t * hq + h) * kHeadDim
                                     : a.iq_out + ((int64_t)t * hiq + (h - h_iq)) * kHeadDim;
            dst += sub * 8;
            store16<kStream>(dst, bf16x8(o));
            store16<kStream>(dst + kHalf, bf16x8(o + 8));
        } else if (valid) {
            const int ci = st == kK ? 0 : st == kV ? 1 : 2;
            const int hl = st == kK ? h - h_k : st == kV ? h - h_v : h - h_ik;
            uint8_t* head_row;   // byte address of (token, head hl, element 0) in the cache
            bool is_bf16;
            float m = 1.0f;      // fp8 quantisation multiplier
            if (PPW == 1) {
                head_row = sel3(ci, row_base[0], row_base[1], row_base[2])
                         + (int64_t)hl * sel3(ci, head_bytes[0], head_bytes[1], head_bytes[2]);
                is_bf16 = sel3(ci, c_bf16[0], c_bf16[1], c_bf16[2]);
                if (!is_bf16) m = inv_scale(sel3(ci, scale_v[0], scale_v[1], scale_v[2]));
            } else {
                const CacheDev& cd = a.cache[ci];
                is_bf16 = cd.is_bf16 != 0;
                head_row = cd.data + (page * cd.sp + (int64_t)off * cd.st + (int64_t)hl * cd.sh) * (is_bf16 ? 2 : 1);
                if (!is_bf16) m = inv_scale_of(cd.scale);
            }
            if (is_bf16) {
                uint16_t* dst = reinterpret_cast<uint16_t*>(head_row) + sub * 8;
                store16<kStream>(dst, bf16x8(o));
                store16<kStream>(dst + kHalf, bf16x8(o + 8));
            } else {
                uint2 lo, hi;
                e4m3x16(o, m, lo, hi);
                uint8_t* dst = head_row + sub * 8;
                store8<kStream>(dst, lo);
                store8<kStream>(dst + kHalf, hi);
            }
        }
    }
    // Last: a store issued early would make the waits for the rows also wait for it.
    if (chunk == 0 && lane == 0 && a.slots_out) a.slots_out[t] = valid ? page * a.page_size + off : -1;
}

// ------------------------------------------------------------------ step-level kernels

__global__ __launch_bounds__(256) void rope_table_kernel(const int32_t* pos, int64_t n, float* cos_out,
                                                         float* sin_out, const FreqArgs f)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n * kHalf) return;
    const int64_t t = i / kHalf;
    const int k = (int)(i - t * kHalf);
    float c, s;
    rope_coeff(pos[t], f.inv_freq[k], &c, &s);
    cos_out[i] = c;
    sin_out[i] = s;
}

__global__ __launch_bounds__(256) void quantize_kernel(const float* v, int64_t n, int32_t is_bf16,
                                                       const float* scale, void* out)
{
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= n) return;
    float x[4];
    for (int j = 0; j < 4; ++j) x[j] = i + j < n ? v[i + j] : 0.0f;
    if (is_bf16) {
        const uint32_t w0 = bf16x2(x[0], x[1]), w1 = bf16x2(x[2], x[3]);
        uint16_t* o = reinterpret_cast<uint16_t*>(out) + i;
        const uint16_t h[4] = {(uint16_t)w0, (uint16_t)(w0 >> 16), (uint16_t)w1, (uint16_t)(w1 >> 16)};
        for (int j = 0; j < 4; ++j)
            if (i + j < n) o[j] = h[j];
    } else {
        const float m = inv_scale_of(scale);
        const uint32_t w = e4m3x4(x[0] * m, x[1] * m, x[2] * m, x[3] * m);
        uint8_t* o = reinterpret_cast<uint8_t*>(out) + i;
        for (int j = 0; j < 4; ++j)
            if (i + j < n) o[j] = (uint8_t)(w >> (8 * j));
    }
}

__global__ __launch_bounds__(256) void rms_scale_kernel(const double* ss, int64_t n, float eps, float* r)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) r[i] = rms_from_ss(ss[i], eps);
}

// ------------------------------------------------------------------ host side

template <int PPW, int HQ, int HKV, int HIQ, int HIK>
hipError_t launch_produce(const ProduceArgs& a, hipStream_t stream)
{
    const int64_t waves = (int64_t)a.T * a.waves_per_token;
    const dim3 grid((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock));
    void* args[] = {const_cast<ProduceArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&produce_kernel<PPW, HQ, HKV, HIQ, HIK>), grid, dim3(kBlock),
                           args, 0, stream);
}

}  // namespace

extern "C" {

msa_status msa_produce(const uint16_t* x, int64_t x_row_stride, int32_t num_tokens, int32_t head_dim,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t num_iq_heads, int32_t num_ik_heads,
                       const int32_t* positions, const int32_t* seq_idx,
                       const int32_t* page_table, int64_t page_table_stride, int32_t num_seqs,
                       int32_t max_pages_per_seq, int32_t page_size, int64_t num_pages,
                       const uint16_t* q_norm_weight, const uint16_t* k_norm_weight,
                       const uint16_t* iq_norm_weight, const uint16_t* ik_norm_weight,
                       float rms_eps, double rope_theta,
                       uint16_t* q_out, uint16_t* iq_out,
                       const msa_cache_view* k_cache, const msa_cache_view* v_cache,
                       const msa_cache_view* ik_cache,
                       int64_t* slots_out, void* stream)
{
    if (head_dim != kHeadDim) return MSA_ERR_UNSUPPORTED;
    if (num_tokens < 0 || num_q_heads < 0 || num_kv_heads < 0 || num_iq_heads < 0 || num_ik_heads < 0)
        return MSA_ERR_SHAPE;
    const int64_t heads_total = (int64_t)num_q_heads + 2 * (int64_t)num_kv_heads + num_iq_heads + num_ik_heads;
    if (heads_total < 1 || heads_total > 4096) return MSA_ERR_SHAPE;
    if (page_size <= 0 || num_seqs < 0 || max_pages_per_seq < 0 || num_pages < 0) return MSA_ERR_SHAPE;
    if (!(rms_eps >= 0.0f) || !(rope_theta > 0.0) || !std::isfinite(rope_theta)) return MSA_ERR_SHAPE;
    if (x_row_stride < heads_total * kHeadDim) return MSA_ERR_STRIDE;
    if (x_row_stride % 8) return MSA_ERR_STRIDE;
    if (num_seqs > 0 && page_table_stride < max_pages_per_seq) return MSA_ERR_STRIDE;
    if (num_tokens > 0) {
        if (!x || !positions || !seq_idx) return MSA_ERR_NULL_POINTER;
        if (num_seqs > 0 && max_pages_per_seq > 0 && !page_table) return MSA_ERR_NULL_POINTER;
        if ((num_q_heads > 0 && !q_out) || (num_iq_heads > 0 && !iq_out)) return MSA_ERR_NULL_POINTER;
    }
    if ((num_q_heads > 0 && !q_norm_weight) || (num_kv_heads > 0 && !k_norm_weight) ||
        (num_iq_heads > 0 && !iq_norm_weight) || (num_ik_heads > 0 && !ik_norm_weight))
        return MSA_ERR_NULL_POINTER;
    if (!aligned(x, 16) || !aligned(q_out, 16) || !aligned(iq_out, 16) || !aligned(positions, 4) ||
        !aligned(seq_idx, 4) || !aligned(page_table, 4) || !aligned(slots_out, 8) ||
        !aligned(q_norm_weight, 16) || !aligned(k_norm_weight, 16) || !aligned(iq_norm_weight, 16) ||
        !aligned(ik_norm_weight, 16))
        return MSA_ERR_ALIGNMENT;
    // Row offsets of the largest token must fit in int64.
    int64_t row_end;
    if (__builtin_mul_overflow((int64_t)num_tokens, x_row_stride, &row_end)) return MSA_ERR_OVERFLOW;
    if (num_seqs > 0 && __builtin_mul_overflow((int64_t)num_seqs, page_table_stride, &row_end)) return MSA_ERR_OVERFLOW;

    ProduceArgs a;
    std::memset(&a, 0, sizeof(a));
    msa_status st;
    uint64_t cache_span[3];
    if ((st = check_cache(k_cache, num_kv_heads, page_size, num_pages, &a.cache[0], true, &cache_span[0])) != MSA_OK)
        return st;
    if ((st = check_cache(v_cache, num_kv_heads, page_size, num_pages, &a.cache[1], true, &cache_span[1])) != MSA_OK)
        return st;
    if ((st = check_cache(ik_cache, num_ik_heads, page_size, num_pages, &a.cache[2], true, &cache_span[2])) != MSA_OK)
        return st;
    int64_t slot_max;
    if (__builtin_mul_overflow(num_pages, (int64_t)page_size, &slot_max)) return MSA_ERR_OVERFLOW;
    if (num_tokens == 0) return MSA_OK;

    a.x = x;
    a.x_stride = x_row_stride;
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
    a.hq = num_q_heads;
    a.hkv = num_kv_heads;
    a.hiq = num_iq_heads;
    a.hik = num_ik_heads;
    a.heads_total = (int32_t)heads_total;
    a.npass = (int32_t)((heads_total + kHeadsPerPass - 1) / kHeadsPerPass);
    a.eps = rms_eps;
    a.w[0] = q_norm_weight;
    a.w[1] = k_norm_weight;
    a.w[2] = iq_norm_weight;
    a.w[3] = ik_norm_weight;
    a.q_out = q_out;
    a.iq_out = iq_out;
    a.slots_out = slots_out;
    fill_inv_freq(rope_theta, a.inv_freq);

    // Small batches: one wave per (token, pass) to spread latency over more waves; large
    // batches: one wave per token so the token's RoPE coefficients are computed once.
    int ppw;
    if ((int64_t)num_tokens * a.npass <= 16384) ppw = 1;
    else ppw = a.npass < kMaxPassesPerWave ? a.npass : kMaxPassesPerWave;
    a.waves_per_token = (a.npass + ppw - 1) / ppw;
    if ((int64_t)num_tokens * a.waves_per_token + kWavesPerBlock > 0x7fffffffLL) return MSA_ERR_SHAPE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    {
        const Span spans[] = {
            {x, row_bytes(num_tokens, x_row_stride, heads_total * kHeadDim, 2)},
            {positions, nbytes(num_tokens, 4)},
            {seq_idx, nbytes(num_tokens, 4)},
            {page_table, num_seqs > 0 ? row_bytes(num_seqs, page_table_stride, max_pages_per_seq, 4) : 0},
            {q_norm_weight, 2 * kHeadDim}, {k_norm_weight, 2 * kHeadDim},
            {iq_norm_weight, 2 * kHeadDim}, {ik_norm_weight, 2 * kHeadDim},
            {q_out, nbytes((int64_t)num_tokens * num_q_heads * kHeadDim, 2)},
            {iq_out, nbytes((int64_t)num_tokens * num_iq_heads * kHeadDim, 2)},
            {a.cache[0].data, cache_span[0]}, {a.cache[1].data, cache_span[1]}, {a.cache[2].data, cache_span[2]},
            {a.cache[0].scale, 4}, {a.cache[1].scale, 4}, {a.cache[2].scale, 4},
            {slots_out, nbytes(num_tokens, 8)},
        };
        if ((st = check_operands(spans, sizeof(spans) / sizeof(spans[0]), s)) != MSA_OK) return st;
    }
    hipError_t e;
    // Builds specialised for the head geometry of one tensor-parallel rank (16/2/2/1); any other
    // geometry runs the generic build.
    const bool rank_geom = num_q_heads == 16 && num_kv_heads == 2 && num_iq_heads == 2 && num_ik_heads == 1;
    if (rank_geom && ppw == 1) e = launch_produce<1, 16, 2, 2, 1>(a, s);
    else if (rank_geom && ppw == 3) e = launch_produce<3, 16, 2, 2, 1>(a, s);
    else switch (ppw) {
        case 1: e = launch_produce<1, -1, -1, -1, -1>(a, s); break;
        case 2: e = launch_produce<2, -1, -1, -1, -1>(a, s); break;
        case 3: e = launch_produce<3, -1, -1, -1, -1>(a, s); break;
        default: e = launch_produce<4, -1, -1, -1, -1>(a, s); break;
    }
    return e == hipSuccess ? MSA_OK : MSA_ERR_LAUNCH;
}

msa_status msa_rope_table(const int32_t* positions, int64_t n, double rope_theta, int32_t head_dim,
                          float* cos_out, float* sin_out, void* stream)
{
    if (head_dim != kHeadDim) return MSA_ERR_UNSUPPORTED;
    if (n < 0 || !(rope_theta > 0.0) || !std::isfinite(rope_theta) || n > ((int64_t)1 << 40)) return MSA_ERR_SHAPE;
    if (n == 0) return MSA_OK;
    if (!positions || !cos_out || !sin_out) return MSA_ERR_NULL_POINTER;
    if (!aligned(positions, 4) || !aligned(cos_out, 4) || !aligned(sin_out, 4)) return MSA_ERR_ALIGNMENT;
    FreqArgs f;
    fill_inv_freq(rope_theta, f.inv_freq);
    const int64_t total = n * kHalf;
    const dim3 grid((unsigned)((total + 255) / 256));
    if ((total + 255) / 256 > 0x7fffffffLL) return MSA_ERR_SHAPE;
    const Span spans[] = {{positions, nbytes(n, 4)}, {cos_out, nbytes(total, 4)}, {sin_out, nbytes(total, 4)}};
    const msa_status st = check_operands(spans, 3, static_cast<hipStream_t>(stream));
    if (st != MSA_OK) return st;
    void* args[] = {const_cast<int32_t**>(&positions), &n, &cos_out, &sin_out, &f};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&rope_table_kernel), grid, dim3(256), args, 0,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MSA_OK : MSA_ERR_LAUNCH;
}

msa_status msa_quantize(const float* values, int64_t n, int32_t dtype, const float* scale, void* codes_out,
                        void* stream)
{
    if (dtype != MSA_CACHE_FP8_E4M3 && dtype != MSA_CACHE_BF16) return MSA_ERR_DTYPE;
    if (n < 0 || n > ((int64_t)1 << 40)) return MSA_ERR_SHAPE;
    if (n == 0) return MSA_OK;
    if (!values || !codes_out) return MSA_ERR_NULL_POINTER;
    if (dtype == MSA_CACHE_FP8_E4M3 && !scale) return MSA_ERR_DTYPE;
    if (!aligned(values, 4) || !aligned(scale, 4) || (dtype == MSA_CACHE_BF16 && !aligned(codes_out, 2)))
        return MSA_ERR_ALIGNMENT;
    int32_t is_bf16 = dtype == MSA_CACHE_BF16;
    const Span spans[] = {{values, nbytes(n, 4)}, {is_bf16 ? nullptr : scale, 4}, {codes_out, nbytes(n, is_bf16 ? 2 : 1)}};
    const msa_status st = check_operands(spans, 3, static_cast<hipStream_t>(stream));
    if (st != MSA_OK) return st;
    const int64_t threads = (n + 3) / 4;
    const dim3 grid((unsigned)((threads + 255) / 256));
    void* args[] = {const_cast<float**>(&values), &n, &is_bf16, const_cast<float**>(&scale), &codes_out};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&quantize_kernel), grid, dim3(256), args, 0,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MSA_OK : MSA_ERR_LAUNCH;
}

msa_status msa_rms_scale(const double* sum_sq, int64_t n, int32_t head_dim, float rms_eps, float* r_out,
                         void* stream)
{
    if (head_dim != kHeadDim) return MSA_ERR_UNSUPPORTED;
    if (n < 0 || n > ((int64_t)1 << 40) || !(rms_eps >= 0.0f)) return MSA_ERR_SHAPE;
    if (n == 0) return MSA_OK;
    if (!sum_sq || !r_out) return MSA_ERR_NULL_POINTER;
    if (!aligned(sum_sq, 8) || !aligned(r_out, 4)) return MSA_ERR_ALIGNMENT;
    const Span spans[] = {{sum_sq, nbytes(n, 8)}, {r_out, nbytes(n, 4)}};
    const msa_status st = check_operands(spans, 2, static_cast<hipStream_t>(stream));
    if (st != MSA_OK) return st;
    const dim3 grid((unsigned)((n + 255) / 256));
    void* args[] = {const_cast<double**>(&sum_sq), &n, &rms_eps, &r_out};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&rms_scale_kernel), grid, dim3(256), args, 0,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MSA_OK : MSA_ERR_LAUNCH;
}

msa_status msa_check_device_pointers(const void* const* ptrs, const uint64_t* bytes, int32_t n, int32_t* first_bad)
{
    if (first_bad) *first_bad = -1;
    if (n < 0) return MSA_ERR_SHAPE;
    if (n == 0) return MSA_OK;
    if (!ptrs) return MSA_ERR_NULL_POINTER;
    int32_t bad = -1;
    msa_status st = MSA_OK;
    for (int32_t i = 0; i < n && st == MSA_OK; ++i) {
        const Span sp{ptrs[i], bytes ? bytes[i] : 1};
        if ((st = spans_resident(&sp, 1, nullptr)) != MSA_OK) bad = i;
    }
    if (first_bad) *first_bad = bad;
    return st;
}

const char* msa_status_str(msa_status s) { return msa_status_string(s); }

const char* msa_status_string(msa_status s)
{
    switch (s) {
        case MSA_OK: return "ok";
        case MSA_ERR_NULL_POINTER: return "a required pointer is NULL";
        case MSA_ERR_UNSUPPORTED: return "unsupported head_dim (only 128 is built)";
        case MSA_ERR_SHAPE: return "invalid count or geometry";
        case MSA_ERR_STRIDE: return "invalid stride (too small, overlapping, or not a multiple of 8 elements)";
        case MSA_ERR_ALIGNMENT: return "misaligned pointer";
        case MSA_ERR_DTYPE: return "invalid cache dtype or missing fp8 scale";
        case MSA_ERR_OVERFLOW: return "element offset overflows int64";
        case MSA_ERR_LAUNCH: return "kernel launch failed";
        case MSA_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
        case MSA_ERR_NOT_DEVICE: return "an operand is not accessible from the current device or runs past its allocation";
    }
    return "unknown status";
}

}  // extern "C"
