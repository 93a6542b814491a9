// santa_score.h -- streaming the K tile of one (request, KV head) and scoring
// it for every query head of the group.
//
// A 256-thread workgroup scores a tile of T rows (T % 64 == 0): wave w,
// step s (0..T/64-1) covers the 16 consecutive tile rows 64 s + 16 w + 0..15,
// so the 4 waves of one step read 64 consecutive rows.  Two lane layouts:
//
//  * MFMA (bf16 K): the group's queries are the A operand of
//    v_mfma_f32_16x16x32_bf16 (16 rows = heads, padded with zeros), 16 K rows
//    are the B operand (16 columns = tokens), 4 MFMAs cover d = 128.  Lane l
//    takes 16 bytes of token l%16 at d = 32 kb + 8 (l/16) for kb = 0..3 and
//    receives the scores of heads 4 (l/16) + v, v = 0..3, for that token.
//    K is loaded as whole 256-byte rows and transposed through LDS.
//  * VALU (fp32 K, fp64 accumulation; also bf16 when SANTA_BF16_VALU is
//    defined, for comparison): 4 lanes per row, each holding 16-byte chunks
//    c, c+4, ... of the row; partial dots for every head, a quad sum, then
//    lane c keeps heads c + 4 v.
//
// Scores are kept UNSCALED (x = <q, k>); the softmax scale is applied after
// the max subtraction, which keeps large planted-key logits accurate to the
// accumulation error.  bf16 products are exact in fp32; fp32 inputs use fp64.
#pragma once

#include "santa_device.h"

// 64-row steps of a bf16 tile whose K loads are issued together: all four
// of a 256-row tile (64 KiB per workgroup in flight at once; 92 VGPRs, so
// 4 workgroups per CU still fit, as many as the 32k batch-1 grid places)
#ifndef SANTA_BF16_STEPS_IN_FLIGHT
#define SANTA_BF16_STEPS_IN_FLIGHT 4
#endif

namespace santa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// partial dot of one 16-byte chunk pair
__device__ __forceinline__ float chunk_dot(const u32x4 &a, const u32x4 &b, float acc) {
    acc = dot2_bf16(a.x, b.x, acc);
    acc = dot2_bf16(a.y, b.y, acc);
    acc = dot2_bf16(a.z, b.z, acc);
    acc = dot2_bf16(a.w, b.w, acc);
    return acc;
}
__device__ __forceinline__ double chunk_dot(const u32x4 &a, const u32x4 &b, double acc) {
    acc = fma((double)__uint_as_float(a.x), (double)__uint_as_float(b.x), acc);
    acc = fma((double)__uint_as_float(a.y), (double)__uint_as_float(b.y), acc);
    acc = fma((double)__uint_as_float(a.z), (double)__uint_as_float(b.z), acc);
    acc = fma((double)__uint_as_float(a.w), (double)__uint_as_float(b.w), acc);
    return acc;
}

// wave-uniform element offset of the 16-row block starting at row j0; a
// block starting at or past n (end of the request) is replaced by the
// tile's first block, which is valid since t0 < n, so every load stays in
// bounds without a branch (scores of such rows are masked by the caller)
template <bool PAGED>
__device__ __forceinline__ size_t block_base(const KVLayout &L, int b, int g, int j0, int n, int t0) {
    const int jb = j0 < n ? j0 : t0;
    if (PAGED) {
        const int page = L.page_table[(size_t)b * L.max_pages + jb / L.page_size];
        return (((size_t)page * L.num_kv_heads + g) * L.page_size + (jb % L.page_size)) * kHeadDim;
    }
    return (((size_t)b * L.num_kv_heads + g) * L.max_seq_len + jb) * kHeadDim;
}

// ------------------------------------------------------------------ MFMA
// KV: uint16_t (bf16 rows of 256 bytes) or uint8_t (e4m3 rows of 128 bytes,
// widened to bf16 on their way into LDS)
template <typename KV, int G, int T, bool PAGED>
struct ScorerMfma {
    typedef float acc_t;
    static constexpr int NS = T / 64;
    static constexpr int NV = 4;
    // steps whose K loads are in flight together: e4m3 rows are half as long,
    // so twice as many steps keep the same bytes in flight
    static constexpr int CH_MAX = sizeof(KV) == 1 ? 4 : SANTA_BF16_STEPS_IN_FLIGHT;
    static constexpr int CH = NS < CH_MAX ? NS : CH_MAX;
    static constexpr int kStageVec = kWavesPerBlock * 256;   // LDS staging, 16-byte units (4 KiB per wave)
    bf16x8_t qa[4];
    acc_t x[NS][NV];

    __device__ __forceinline__ static int head(int lane, int v) { return 4 * (lane >> 4) + v; }
    __device__ __forceinline__ static int row(int lane, int w, int s) { return 64 * s + 16 * w + (lane & 15); }
    __device__ __forceinline__ static bool writer(int lane) { return (lane & 15) == 0; }
    __device__ __forceinline__ static float reduce_max(float v) { return row16_max(v); }
    __device__ __forceinline__ static float reduce_sum(float v) { return row16_sum(v); }

    __device__ __forceinline__ void load_q(const uint16_t *q_group) {
        const int lane = threadIdx.x & 63;
        const int hrow = lane & 15, kq = lane >> 4;
        // rows >= G repeat row G-1: their MFMA outputs are never used, and the
        // load stays unconditional (no branch, so no early wait on it)
        const int hsrc = hrow < G ? hrow : G - 1;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            qa[kb] = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const u32x4 *>(q_group + hsrc * kHeadDim + 32 * kb + 8 * kq));
    }

    // K is read as whole rows: bf16, 4 rows (4 x 256 bytes) per load
    // instruction, lane l holding 16-byte piece l%16 of row 4 kb + l/16 of the
    // wave's 16-row block; e4m3, 8 rows (8 x 128 bytes) per instruction, lane
    // l holding bytes 16 (l%8) .. 16 (l%8) + 15 of row 8 i + l/8, which widen
    // to bf16 pieces 2 (l%8) and 2 (l%8) + 1.  The block then goes through
    // the wave's 4 KiB of `stage` as bf16 (piece p of row r at slot p ^ r,
    // so that both the row-wise writes and the token-wise reads touch every
    // bank once) into the MFMA layout: lane l reads piece 4 kb + l/16 of
    // token l%16.
    static constexpr bool kFp8 = sizeof(KV) == 1;
    static constexpr int kLoads = kFp8 ? 2 : 4;     // 16-byte loads per lane per 16-row block

    __device__ __forceinline__ void score(const KV *__restrict__ k, const KVLayout &L, int b, int g,
                                          int t0, int n, u32x4 *stage) {
        const int lane = threadIdx.x & 63;
        // paged: the wave index in a scalar register, so that the page
        // lookups are scalar loads, and every block's lookup issued first, so
        // that they overlap instead of preceding each chunk's K loads
        const int w = PAGED ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : (int)(threadIdx.x >> 6);
        const int tok = lane & 15, kq = lane >> 4;
        u32x4 *wst = stage + w * 256;
        size_t base_all[PAGED ? NS : 1];
        if constexpr (PAGED) {
#pragma unroll
            for (int s = 0; s < NS; ++s) base_all[s] = block_base<PAGED>(L, b, g, t0 + 64 * s + 16 * w, n, t0);
        }
#pragma unroll
        for (int s0 = 0; s0 < NS; s0 += CH) {
            size_t base[CH];
#pragma unroll
            for (int ii = 0; ii < CH; ++ii)
                base[ii] = PAGED ? base_all[PAGED ? s0 + ii : 0]
                                 : block_base<PAGED>(L, b, g, t0 + 64 * (s0 + ii) + 16 * w, n, t0);
            u32x4 kv[CH][kLoads];
#pragma unroll
            for (int ii = 0; ii < CH; ++ii) {
#pragma unroll
                for (int li = 0; li < kLoads; ++li) {
                    // rows past the end read the block's row 0 (always a valid
                    // row of the tile); their scores are masked below
                    const int r = kFp8 ? 8 * li + (lane >> 3) : 4 * li + kq;
                    const int piece = kFp8 ? (lane & 7) : tok;
                    const bool valid = t0 + 64 * (s0 + ii) + 16 * w + r < n;
                    const u32x4 *rowp =
                        reinterpret_cast<const u32x4 *>(k + base[ii] + (size_t)(valid ? r : 0) * kHeadDim) + piece;
                    kv[ii][li] = __builtin_nontemporal_load(rowp);
                }
            }
#pragma unroll
            for (int ii = 0; ii < CH; ++ii) {
#pragma unroll
                for (int li = 0; li < kLoads; ++li) {
                    if constexpr (kFp8) {
                        const int r = 8 * li + (lane >> 3), p8 = lane & 7;
                        const u32x4 raw = kv[ii][li];
                        const u32x4 lo = {e4m3x2_to_bf16<false>(raw.x), e4m3x2_to_bf16<true>(raw.x),
                                          e4m3x2_to_bf16<false>(raw.y), e4m3x2_to_bf16<true>(raw.y)};
                        const u32x4 hi = {e4m3x2_to_bf16<false>(raw.z), e4m3x2_to_bf16<true>(raw.z),
                                          e4m3x2_to_bf16<false>(raw.w), e4m3x2_to_bf16<true>(raw.w)};
                        wst[r * 16 + ((2 * p8) ^ r)] = lo;
                        wst[r * 16 + ((2 * p8 + 1) ^ r)] = hi;
                    } else {
                        const int r = 4 * li + kq;
                        wst[r * 16 + (tok ^ r)] = kv[ii][li];
                    }
                }
                wave_sync_lds();
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const u32x4 kt = wst[tok * 16 + ((4 * kb + kq) ^ tok)];
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kb], __builtin_bit_cast(bf16x8_t, kt), acc, 0, 0, 0);
                }
                wave_sync_lds();
                const bool valid = t0 + 64 * (s0 + ii) + 16 * w + tok < n;
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    x[s0 + ii][v] = (valid && head(lane, v) < G) ? acc[v] : -INFINITY;
            }
        }
    }
};

// ------------------------------------------------------------------ VALU
template <typename KV> struct KVTraits;
template <> struct KVTraits<uint16_t> {       // bf16 storage
    typedef float acc_t;
    static constexpr int kChunks = kHeadDim * 2 / 64;   // 16-byte chunks per lane per row
};
template <> struct KVTraits<float> {
    typedef double acc_t;
    static constexpr int kChunks = kHeadDim * 4 / 64;
};

template <typename KV, int G, int T, bool PAGED>
struct ScorerValu {
    typedef typename KVTraits<KV>::acc_t acc_t;
    static constexpr int NC = KVTraits<KV>::kChunks;
    static constexpr int NS = T / 64;
    static constexpr int NV = (G + 3) / 4;            // heads per lane
    // steps whose K loads are in flight together (keeps G >= 4 under 128 VGPRs)
    static constexpr int CHMAX = G <= 2 ? 4 : 2;
    static constexpr int CH = NS < CHMAX ? NS : CHMAX;
    static constexpr int ROW_VEC = kHeadDim * (int)sizeof(KV) / 16;
    static constexpr int kStageVec = 0;                       // no LDS staging
    u32x4 qv[G][NC];
    acc_t x[NS][NV];

    __device__ __forceinline__ static int head(int lane, int v) { return (lane & 3) + 4 * v; }
    __device__ __forceinline__ static int row(int lane, int w, int s) { return 64 * s + 16 * w + (lane >> 2); }
    __device__ __forceinline__ static bool writer(int lane) { return lane < 4; }
    __device__ __forceinline__ static float reduce_max(float v) { return max_stride4(v); }
    __device__ __forceinline__ static float reduce_sum(float v) { return sum_stride4(v); }

    __device__ __forceinline__ void load_q(const KV *q_group) {
        const int c = threadIdx.x & 3;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(q_group);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int j = 0; j < NC; ++j) qv[h][j] = src[h * ROW_VEC + c + 4 * j];
    }

    __device__ __forceinline__ void score(const KV *__restrict__ k, const KVLayout &L, int b, int g, int t0,
                                          int n, u32x4 * /*stage: unused*/) {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        const int c = lane & 3, r = lane >> 2;
#pragma unroll
        for (int s0 = 0; s0 < NS; s0 += CH) {
            size_t base[CH];
#pragma unroll
            for (int ii = 0; ii < CH; ++ii) base[ii] = block_base<PAGED>(L, b, g, t0 + 64 * (s0 + ii) + 16 * w, n, t0);
            u32x4 kv[CH][NC];
#pragma unroll
            for (int ii = 0; ii < CH; ++ii) {
                const bool valid = t0 + 64 * (s0 + ii) + 16 * w + r < n;
                const u32x4 *rowp = reinterpret_cast<const u32x4 *>(k + base[ii]) + (valid ? r : 0) * ROW_VEC;
#pragma unroll
                for (int jj = 0; jj < NC; ++jj) kv[ii][jj] = __builtin_nontemporal_load(rowp + c + 4 * jj);
            }
#pragma unroll
            for (int ii = 0; ii < CH; ++ii) {
                const bool valid = t0 + 64 * (s0 + ii) + 16 * w + r < n;
                acc_t part[G];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    acc_t a = 0;
#pragma unroll
                    for (int jj = 0; jj < NC; ++jj) a = chunk_dot(qv[h][jj], kv[ii][jj], a);
                    part[h] = quad_sum(a);
                }
#pragma unroll
                for (int hh = 0; hh < NV; ++hh) {
                    acc_t s = part[hh * 4 < G ? hh * 4 : 0];
#pragma unroll
                    for (int h = hh * 4 + 1; h < G && h < hh * 4 + 4; ++h)
                        if (c == h - hh * 4) s = part[h];
                    x[s0 + ii][hh] = (valid && head(lane, hh) < G) ? s : (acc_t)(-INFINITY);
                }
            }
        }
    }
};

// scorer used for a storage type: MFMA for bf16 and e4m3, VALU/fp64 for fp32
template <typename KV, int G, int T, bool PAGED> struct ScorerFor;
template <int G, int T, bool PAGED> struct ScorerFor<float, G, T, PAGED> {
    typedef ScorerValu<float, G, T, PAGED> type;
};
#ifdef SANTA_BF16_VALU
template <int G, int T, bool PAGED> struct ScorerFor<uint16_t, G, T, PAGED> {
    typedef ScorerValu<uint16_t, G, T, PAGED> type;
};
#else
template <int G, int T, bool PAGED> struct ScorerFor<uint16_t, G, T, PAGED> {
    typedef ScorerMfma<uint16_t, G, T, PAGED> type;
};
#endif
template <int G, int T, bool PAGED> struct ScorerFor<uint8_t, G, T, PAGED> {
    typedef ScorerMfma<uint8_t, G, T, PAGED> type;
};

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Per-head tile maximum of the unscaled scores: red_m[w][head] holds each
// wave's maximum, mt[v] the tile maximum of this lane's v-th head.
template <class SC>
__device__ __forceinline__ void tile_max(const SC &sc, float (&red_m)[kWavesPerBlock][16],
                                         float (&mt)[SC::NV]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int v = 0; v < SC::NV; ++v) {
        typename SC::acc_t m = sc.x[0][v];
#pragma unroll
        for (int s = 1; s < SC::NS; ++s) m = sc.x[s][v] > m ? sc.x[s][v] : m;
        const float mf = SC::reduce_max((float)m);
        const int h = SC::head(lane, v);
        if (SC::writer(lane) && h < 16) red_m[w][h] = mf;
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < SC::NV; ++v) {
        const int h = SC::head(lane, v) & 15;
        float m = red_m[0][h];
#pragma unroll
        for (int ww = 1; ww < kWavesPerBlock; ++ww) m = fmaxf(m, red_m[ww][h]);
        mt[v] = m;
    }
}

}  // namespace santa
