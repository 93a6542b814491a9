// santa_score.h -- streaming the K tile of one (request, KV head) and scoring
// it for every query head of the group.
//
// Thread layout of a 256-thread workgroup over a tile of T rows (T % 64 == 0):
//   wave w (0..3), lane l; quad position c = l & 3, row slot r = l >> 2 (0..15)
//   step i (0..T/64-1) covers tile rows 64*i + 16*w + r, so the 4 waves of one
//   step read 64 consecutive rows (16 KiB of bf16 K).  Within a row the 4
//   lanes of a quad each read 16-byte chunks c, c+4, c+8, ... (coalesced
//   64-byte pieces; 4 per bf16 row, 8 per fp32 row).
//   Every lane forms partial dot products over its part of the row for all
//   G heads; a quad sum completes them.  Lane c then keeps heads c, c+4, ...
//
// Scores are kept UNSCALED (x = <q, k>); the softmax scale is applied after
// the max subtraction, which keeps the large planted-key logits exact to the
// accumulation error only.  bf16 inputs accumulate in fp32 (bf16 products
// are exact in fp32); fp32 inputs accumulate in fp64.
#pragma once

#include "santa_device.h"

namespace santa {

template <typename KV> struct KVTraits;

template <> struct KVTraits<uint16_t> {       // bf16 storage
    typedef float acc_t;
    static constexpr int kChunks = kHeadDim * 2 / 64;   // 16-byte chunks per lane per row
};
template <> struct KVTraits<float> {
    typedef double acc_t;
    static constexpr int kChunks = kHeadDim * 4 / 64;
};

template <int G> struct HeadsPerLane { static constexpr int value = (G + 3) / 4; };

// q fragment of one lane: the elements of its row chunks, for all G heads
template <typename KV, int G>
struct QFrag {
    u32x4 v[G][KVTraits<KV>::kChunks];
};

template <typename KV, int G>
__device__ __forceinline__ void load_qfrag(QFrag<KV, G> &f, const KV *q_group, int c) {
    constexpr int NC = KVTraits<KV>::kChunks;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(q_group);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < NC; ++j)
            f.v[h][j] = src[h * (kHeadDim * sizeof(KV) / 16) + c + 4 * j];
}

// partial dot of one chunk pair (16 bytes of q and 16 bytes of k)
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

// Score the tile rows [t0, t0 + T) of (b, g), rows >= n are invalid.
// x[i][hh]: unscaled score of row t0 + 64 i + 16 w + r for head c + 4 hh,
// or -inf when the row is invalid or the head index is >= G.
template <typename KV, int G, int T>
__device__ __forceinline__ void score_tile(
    const KV *__restrict__ k, const KVLayout &L, int b, int g, int t0, int n,
    const QFrag<KV, G> &qf, typename KVTraits<KV>::acc_t (&x)[T / 64][HeadsPerLane<G>::value]) {
    typedef typename KVTraits<KV>::acc_t acc_t;
    constexpr int NC = KVTraits<KV>::kChunks;
    constexpr int HPL = HeadsPerLane<G>::value;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = lane & 3, r = lane >> 2;
#pragma unroll
    for (int i = 0; i < T / 64; ++i) {
        const int j0 = t0 + 64 * i + 16 * w;          // first row of this wave's block
        const bool valid = (j0 + r) < n;
        u32x4 kv[NC];
        if (j0 < n) {
            const u32x4 *row = reinterpret_cast<const u32x4 *>(k + block16_offset(L, b, g, j0)) +
                               (size_t)r * (kHeadDim * sizeof(KV) / 16);
#pragma unroll
            for (int jj = 0; jj < NC; ++jj)
                kv[jj] = valid ? __builtin_nontemporal_load(row + c + 4 * jj) : u32x4{0u, 0u, 0u, 0u};
        } else {
#pragma unroll
            for (int jj = 0; jj < NC; ++jj) kv[jj] = u32x4{0u, 0u, 0u, 0u};
        }
        acc_t part[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            acc_t a = 0;
#pragma unroll
            for (int jj = 0; jj < NC; ++jj) a = chunk_dot(qf.v[h][jj], kv[jj], a);
            part[h] = quad_sum(a);
        }
#pragma unroll
        for (int hh = 0; hh < HPL; ++hh) {
            acc_t s = part[hh * 4 < G ? hh * 4 : 0];
#pragma unroll
            for (int h = hh * 4 + 1; h < G && h < hh * 4 + 4; ++h)
                if (c == h - hh * 4) s = part[h];
            const bool head_ok = (c + 4 * hh) < G;
            x[i][hh] = (valid && head_ok) ? s : (acc_t)(-INFINITY);
        }
    }
}

}  // namespace santa
