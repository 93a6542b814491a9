// santa_kernels.h -- device building blocks shared by the gfx950 kernel
// translation units of libsanta (prop, flash, exact): block-wide scans, tile
// maxima, exp weights, V row loads, the per-tile merge kernel and the
// dispatch macros.
#pragma once

#include <hip/hip_ext.h>

#include "santa_launch.h"
#include "santa_score.h"

namespace santa {

#ifndef SANTA_SAMPLE_MANY_HEADS
#define SANTA_SAMPLE_MANY_HEADS 512
#endif
// above this many heads the systematic sampling kernel runs 8 waves per head,
// above kSampleVeryManyHeads 4 (every head of a batch of 64 resident at once)
constexpr int kSampleManyHeads = SANTA_SAMPLE_MANY_HEADS;
constexpr int kSampleVeryManyHeads = 1024;
// the same for the list generators, whose 16-wave workgroups take a whole
// compute unit each (more registers)
constexpr int kSampleListManyHeads = 256;
constexpr int kMergeBlock = 1024;                  // threads of the per-head merge block
constexpr int kMergeParts = kMergeBlock / kHeadDim;

// -------------------------------------------------------------------
// block-wide scans (fixed order, deterministic)
// -------------------------------------------------------------------
template <typename V>
__device__ __forceinline__ V block_incl_sum(V v, V *sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    V x = wave_incl_scan(v, lane);
    if (lane == 63) sh[w] = x;
    __syncthreads();
    V off = 0;
    for (int i = 0; i < w; ++i) off += sh[i];
    __syncthreads();
    return x + off;
}

__device__ __forceinline__ float block_max(float v, float *sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_max(v);
    if (lane == 0) sh[w] = v;
    __syncthreads();
    float m = sh[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = fmaxf(m, sh[i]);
    __syncthreads();
    return m;
}

// exp-weight e = exp(scale (x - m)) of an unscaled score x, tile max m
// (tile, request, KV head) of this workgroup in the per-tile kernels.
// Contiguous K: tile fastest, so consecutive blocks stream adjacent pieces of
// one KV head (64 KiB each for T = 256).  Paged K ([pages, Hkv, 16, d]): KV
// head fastest, so consecutive blocks read the heads' adjacent 4 KiB pieces
// of the same pages; tile-fastest order would have them all read one head's
// pieces at the Hkv * 4 KiB page stride (16% slower on pages held in order).
template <bool PAGED>
__device__ __forceinline__ void tile_of_block(const KVLayout &L, int max_nt, int &tile, int &b, int &g) {
    const int id = blockIdx.x;
    if (PAGED) {
        g = id % L.num_kv_heads;
        const int rest = id / L.num_kv_heads;
        tile = rest % max_nt;
        b = rest / max_nt;
    } else {
        tile = id % max_nt;
        const int bg = id / max_nt;
        b = bg / L.num_kv_heads;
        g = bg - b * L.num_kv_heads;
    }
}

template <typename acc_t>
__device__ __forceinline__ float exp_weight(acc_t x, float m, acc_t c2) {
    return exp2f((float)((x - (acc_t)m) * c2));
}

// ===================================================================
// V row loads (8 consecutive elements of a row per lane)
// ===================================================================
template <typename KV>
__device__ __forceinline__ void load_v8(const KV *p, float (&v)[8]);

template <>
__device__ __forceinline__ void load_v8<uint16_t>(const uint16_t *p, float (&v)[8]) {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(p);
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x);
    v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z);
    v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
}
template <>
__device__ __forceinline__ void load_v8<uint8_t>(const uint8_t *p, float (&v)[8]) {
    const uint2 a = *reinterpret_cast<const uint2 *>(p);
    e4m3x4_to_f32(a.x, v);
    e4m3x4_to_f32(a.y, v + 4);
}
template <>
__device__ __forceinline__ void load_v8<float>(const float *p, float (&v)[8]) {
    const u32x4 a = reinterpret_cast<const u32x4 *>(p)[0];
    const u32x4 c = reinterpret_cast<const u32x4 *>(p)[1];
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(c.x); v[5] = __uint_as_float(c.y);
    v[6] = __uint_as_float(c.z); v[7] = __uint_as_float(c.w);
}

// 8 consecutive elements of a V row kept in storage form (so that many
// loads can be in flight in few registers), widened to fp32 at use
template <typename KV> struct Raw8;
template <> struct Raw8<uint16_t> { u32x4 x[1]; };
template <> struct Raw8<float> { u32x4 x[2]; };
template <> struct Raw8<uint8_t> { uint2 x; };

template <typename KV>
__device__ __forceinline__ Raw8<KV> load_raw8(const KV *p) {
    Raw8<KV> r;
    if constexpr (sizeof(KV) == 1) {
        r.x = *reinterpret_cast<const uint2 *>(p);
    } else {
#pragma unroll
        for (int i = 0; i < (int)(sizeof(r.x) / sizeof(u32x4)); ++i) r.x[i] = reinterpret_cast<const u32x4 *>(p)[i];
    }
    return r;
}
__device__ __forceinline__ void widen8(const Raw8<uint8_t> &r, float (&v)[8]) {
    e4m3x4_to_f32(r.x.x, v);
    e4m3x4_to_f32(r.x.y, v + 4);
}
__device__ __forceinline__ void widen8(const Raw8<uint16_t> &r, float (&v)[8]) {
    const u32x4 a = r.x[0];
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x);
    v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z);
    v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
}
__device__ __forceinline__ void widen8(const Raw8<float> &r, float (&v)[8]) {
    v[0] = __uint_as_float(r.x[0].x); v[1] = __uint_as_float(r.x[0].y);
    v[2] = __uint_as_float(r.x[0].z); v[3] = __uint_as_float(r.x[0].w);
    v[4] = __uint_as_float(r.x[1].x); v[5] = __uint_as_float(r.x[1].y);
    v[6] = __uint_as_float(r.x[1].z); v[7] = __uint_as_float(r.x[1].w);
}

// ===================================================================
// Merge of per-tile (m_t, l_t, o_t): out = sum_t w_t o_t / norm with
// w_t = e^{scale (m_t - M)} * coef_t.  Flash: coef_t = Z_t (the tile's true
// mass), o_t are tile means, norm = sum_t w_t.  Exact: coef_t = 1, o_t are
// unnormalised sums, norm = sum_t w_t l_t.
// grid: B * Hq blocks of 1024 threads: thread (part p, element d) sums the
// tiles t = p, p + 8, ...; the 8 parts are added in order.
// ===================================================================
static __global__ __launch_bounds__(kMergeBlock) void merge_tiles_kernel(
    const float *__restrict__ part_m, const float *__restrict__ part_l, const float *__restrict__ part_o,
    const int *__restrict__ seq_lens, int max_seq_len, int T, int nt_stride, int batch, int num_q_heads,
    int num_kv_heads, int flash, float scale, float *__restrict__ out) {
    // block = head-in-group * B*Hkv + bg: the XCD that ran this KV head's tiles
    const int BG = batch * num_kv_heads, G = num_q_heads / num_kv_heads;
    const int bg = blockIdx.x % BG, hl = blockIdx.x / BG;
    const int b = bg / num_kv_heads, g = bg - b * num_kv_heads;
    const int bh = b * num_q_heads + g * G + hl;
    const int tid = threadIdx.x;
    const int n = seq_len_of(seq_lens, max_seq_len, b);
    const int nt = (n + T - 1) / T;
    extern __shared__ double wts[];     // [nt_stride]
    __shared__ double shd[kMergeBlock / 64];
    __shared__ float shf[kMergeBlock / 64];
    __shared__ float red[kMergeParts][kHeadDim];
    if (nt == 0) {
        if (tid < kHeadDim) out[(size_t)bh * kHeadDim + tid] = 0.f;
        return;
    }
    const float *pm = part_m + (size_t)bh * nt_stride;
    const float *pl = part_l + (size_t)bh * nt_stride;
    // nt <= kMergeBlock (checked on the host): thread t owns tile t
    const float mt = tid < nt ? pm[tid] : -INFINITY;
    const float lt = tid < nt ? pl[tid] : 0.f;
    const double M = (double)block_max(mt, shf);
    double nl = 0.0;
    if (tid < nt) {
        const double f = (double)exp2f((mt - (float)M) * (scale * 1.4426950408889634f));
        const double wt = flash ? f * (double)lt : f;
        nl = flash ? wt : wt * (double)lt;
        wts[tid] = wt;
    }
    const double norm_incl = block_incl_sum<double>(nl, shd);
    if (tid == kMergeBlock - 1) shd[0] = norm_incl;
    __syncthreads();
    const double inv = 1.0 / shd[0];
    const int d = tid & (kHeadDim - 1), p = tid / kHeadDim;
    const float *po = part_o + (size_t)bh * nt_stride * kHeadDim + d;
    double acc = 0.0;
#pragma unroll 8
    for (int tt = p; tt < nt; tt += kMergeParts) acc += wts[tt] * (double)po[(size_t)tt * kHeadDim];
    red[p][d] = (float)(acc * inv);
    __syncthreads();
    if (tid < kHeadDim) {
        float s = 0.f;
#pragma unroll
        for (int pp = 0; pp < kMergeParts; ++pp) s += red[pp][tid];
        out[(size_t)bh * kHeadDim + tid] = s;
    }
}

// ===================================================================
// launch helpers
// ===================================================================
inline KVLayout layout_of(const LaunchArgs &a) {
    return KVLayout{a.num_kv_heads, a.max_seq_len, a.page_size, a.page_table, a.max_pages};
}

// dispatch over (group, tile length, layout) for one storage type
#define SANTA_P_CASES(KV, G, T, FN) \
    return a.page_size ? FN<KV, G, T, true>(a, hook) : FN<KV, G, T, false>(a, hook);
#define SANTA_T_CASES(KV, G, FN)                        \
    switch (a.tile_len) {                               \
        case 64: SANTA_P_CASES(KV, G, 64, FN)           \
        case 128: SANTA_P_CASES(KV, G, 128, FN)         \
        case 256: SANTA_P_CASES(KV, G, 256, FN)         \
        case 512: SANTA_P_CASES(KV, G, 512, FN)         \
        case 1024: SANTA_P_CASES(KV, G, 1024, FN)       \
        default: return hipErrorInvalidValue;           \
    }
#define SANTA_G_CASES(KV, FN)                           \
    switch (a.group) {                                  \
        case 1: SANTA_T_CASES(KV, 1, FN)                \
        case 2: SANTA_T_CASES(KV, 2, FN)                \
        case 4: SANTA_T_CASES(KV, 4, FN)                \
        case 8: SANTA_T_CASES(KV, 8, FN)                \
        default: return hipErrorInvalidValue;           \
    }
// explicit instantiation of a per-type launcher for this compilation's KV
// storage type (all three when SANTA_KV is not given)
#ifdef SANTA_KV
#define SANTA_INSTANTIATE(F) template hipError_t F<SANTA_KV>(const LaunchArgs &, const TimingHook &);
#else
#define SANTA_INSTANTIATE(F)                                                      \
    template hipError_t F<uint16_t>(const LaunchArgs &, const TimingHook &);      \
    template hipError_t F<uint8_t>(const LaunchArgs &, const TimingHook &);       \
    template hipError_t F<float>(const LaunchArgs &, const TimingHook &);
#endif

}  // namespace santa
