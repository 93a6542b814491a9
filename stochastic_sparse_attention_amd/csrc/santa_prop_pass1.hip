// santa_prop_pass1.hip -- S2ANTA-prop, pass 1: scores, tile max, tile
// partition function and the exponentiated-score stash (its own translation
// unit; the reducer and pass 2 are in santa_prop.hip, and santa_dispatch.cpp
// launches the step).
//
// The method follows the web page "Stochastic Sparse Attention for
// Memory-Bound Inference" (ICML 2026 paper notes on SANTA), key design 2:
// pass 1 scores every tile and stashes its exp-scores with the tile
// partition function.
#include "santa_kernels.h"

namespace santa {

// ===================================================================
// S2ANTA-prop, pass 1: scores, tile max, tile partition function, stash
// ===================================================================
// grid: B * Hkv * max_nt workgroups (tile fastest); block: 256 threads.
// stash [B, Hq, max_nt * T] fp32 (rows padded to whole tiles):
// e_j = exp(scale * (x_j - m_t))
// stats [B, Hq, max_nt] float2: (m_t unscaled tile max, Z_t = sum_j e_j)
template <typename KV, int G, int T, bool PAGED>
__global__ __launch_bounds__(kBlock) void prop_pass1_kernel(
    const typename QOf<KV>::type *__restrict__ q, const KV *__restrict__ k, KVLayout L, const int *__restrict__ seq_lens,
    int num_q_heads, int max_nt, float scale, float *__restrict__ stash, float2 *__restrict__ stats) {
    typedef typename ScorerFor<KV, G, T, PAGED>::type SC;
    typedef typename SC::acc_t acc_t;
    int tile, b, g;
    tile_of_block<PAGED>(L, max_nt, tile, b, g);
    const int n = seq_len_of(seq_lens, L.max_seq_len, b);
    const int t0 = tile * T;
    if (t0 >= n) return;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;

    // LDS: the scorer's staging area, then (after the barrier in tile_max)
    // the tile's stash rows E[G][T], staged for wide stores
    __shared__ __align__(16) unsigned char lds[cmax(SC::kStageVec * 16, G * T * 4)];
    __shared__ float red_m[kWavesPerBlock][16];
    __shared__ float red_z[kWavesPerBlock][16];
    float (*E)[T] = reinterpret_cast<float (*)[T]>(lds);

    SC sc;
    sc.load_q(q + ((size_t)b * num_q_heads + (size_t)g * G) * kHeadDim);
    sc.score(k, L, b, g, t0, n, reinterpret_cast<u32x4 *>(lds));

    float mt[SC::NV];
    tile_max(sc, red_m, mt);

    const acc_t c2 = (acc_t)scale * (acc_t)1.4426950408889634;   // scale * log2(e)
#pragma unroll
    for (int v = 0; v < SC::NV; ++v) {
        const int hl = SC::head(lane, v);                 // head within the group
        float zsum = 0.f;
        if (hl < G) {
#pragma unroll
            for (int s = 0; s < SC::NS; ++s) {
                const int row = SC::row(lane, w, s);
                const float e = (t0 + row < n) ? exp_weight(sc.x[s][v], mt[v], c2) : 0.f;
                E[hl][row] = e;
                zsum += e;
            }
        }
        zsum = SC::reduce_sum(zsum);
        if (SC::writer(lane) && hl < 16) red_z[w][hl] = zsum;
    }
    __syncthreads();
    // stash: wave w writes head rows w, w+4, ...; each store instruction
    // covers 64 lanes x 16 bytes = 256 consecutive tokens.  The whole tile
    // is written, so positions past the sequence end hold 0 and pass 2
    // reads them unmasked.
    for (int hl = w; hl < G; hl += kWavesPerBlock) {
        float *srow = stash + ((size_t)b * num_q_heads + (size_t)g * G + hl) * ((size_t)max_nt * T) + t0;
#pragma unroll
        for (int j4 = 4 * lane; j4 < T; j4 += 256)
            *reinterpret_cast<float4 *>(srow + j4) = *reinterpret_cast<const float4 *>(&E[hl][j4]);
    }
    if (threadIdx.x < G) {
        const int hl = threadIdx.x;
        float z = red_z[0][hl], m = red_m[0][hl];
#pragma unroll
        for (int ww = 1; ww < kWavesPerBlock; ++ww) {
            z += red_z[ww][hl];
            m = fmaxf(m, red_m[ww][hl]);
        }
        stats[((size_t)b * num_q_heads + (size_t)g * G + hl) * max_nt + tile] = make_float2(m, z);
    }
}

template <typename KV, int G, int T, bool PAGED>
static hipError_t launch_pass1_t(const LaunchArgs &a, const TimingHook &hook) {
    const int max_nt = a.max_nt;
    hipStream_t st = (hipStream_t)a.stream;
    float *stash = (float *)a.ws.stash;
    float2 *stats = (float2 *)a.ws.stats;
    const KVLayout L = layout_of(a);
    // with a timing hook the dispatch itself records the two events, so
    // they bracket the kernel's execution and nothing else
    if (hook.begin)
        hipExtLaunchKernelGGL((prop_pass1_kernel<KV, G, T, PAGED>), dim3((unsigned)(a.batch * a.num_kv_heads * max_nt)), dim3(kBlock), 0, st, (hipEvent_t)hook.begin, (hipEvent_t)hook.end, 0,
                       (const typename QOf<KV>::type *)a.q, (const KV *)a.k, L, a.seq_lens, a.num_q_heads, max_nt, a.scale,
                       stash, stats);
    else
        hipLaunchKernelGGL((prop_pass1_kernel<KV, G, T, PAGED>), dim3((unsigned)(a.batch * a.num_kv_heads * max_nt)), dim3(kBlock), 0, st,
                       (const typename QOf<KV>::type *)a.q, (const KV *)a.k, L, a.seq_lens, a.num_q_heads, max_nt, a.scale,
                       stash, stats);
    return hipGetLastError();
}

template <typename KV>
hipError_t launch_prop_pass1_kv(const LaunchArgs &a, const TimingHook &hook) { SANTA_G_CASES(KV, launch_pass1_t) }
SANTA_INSTANTIATE(launch_prop_pass1_kv)

}  // namespace santa
