// santa_exact.hip -- exact split-KV decode kernel and launcher (the baseline).
//
// The method follows the web page "Stochastic Sparse Attention for
// Memory-Bound Inference" (ICML 2026 paper notes on SANTA):
//   key design 1  systematic sampling: one offset U in [0,1/S), thresholds
//                 U + m/S, selected index = inverse CDF at each threshold
//   key design 2  S2ANTA-prop: pass 1 scores and stashes exp-scores with the
//                 tile partition function, a reducer turns the n_t tile
//                 masses into per-tile budgets, pass 2 samples and gathers V
//   key design 3  S2ANTA-flash: S/n_t local samples per tile, partial means
//                 rescaled by the true tile mass when merged
// The exact split-KV decode is the FlashDecoding-style baseline the pages
// compare against.
//
// Precision: scores are accumulated unscaled as in prop (bf16 products are
// exact in fp32; fp32 inputs use fp64), the tile max is subtracted before the
// scale is applied, each tile's weights and weighted V sums are fp32, and
// the merge of the tiles works in fp64.
#include "santa_kernels.h"

namespace santa {

// ===================================================================
// Exact split-KV decode: per tile (m_t, l_t, o_t = sum_j p_j V_j)
// ===================================================================
template <typename KV, int G, int T, bool PAGED>
__global__ __launch_bounds__(kBlock) void exact_partial_kernel(
    const typename QOf<KV>::type *__restrict__ q, const KV *__restrict__ k, const KV *__restrict__ v, KVLayout L,
    const int *__restrict__ seq_lens, int num_q_heads, int max_nt, float scale,
    float *__restrict__ part_m, float *__restrict__ part_l, float *__restrict__ part_o) {
    typedef typename ScorerFor<KV, G, T, PAGED>::type SC;
    typedef typename SC::acc_t acc_t;
    int tile, b, g;
    tile_of_block<PAGED>(L, max_nt, tile, b, g);
    const int n = seq_len_of(seq_lens, L.max_seq_len, b);
    const int t0 = tile * T;
    if (t0 >= n) return;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;

    // LDS: the scorer's staging area, then (after the barrier in tile_max)
    // the tile's weights Pw[T][G] (a row's G weights in one LDS read) and the
    // per-wave V sums red_o
    constexpr int kPwBytes = G * T * 4, kRedBytes = kWavesPerBlock * G * kHeadDim * 4;
    __shared__ __align__(16) unsigned char lds[cmax(SC::kStageVec * 16, kPwBytes + kRedBytes)];
    __shared__ float red_m[kWavesPerBlock][16];
    __shared__ float red_l[kWavesPerBlock][16];
    float *Pw = reinterpret_cast<float *>(lds);   // [T][G]
    float (*red_o)[G][kHeadDim] = reinterpret_cast<float (*)[G][kHeadDim]>(lds + kPwBytes);

    SC sc;
    sc.load_q(q + ((size_t)b * num_q_heads + (size_t)g * G) * kHeadDim);
    sc.score(k, L, b, g, t0, n, reinterpret_cast<u32x4 *>(lds));

    float mt[SC::NV];
    tile_max(sc, red_m, mt);
    const acc_t c2 = (acc_t)scale * (acc_t)1.4426950408889634;
#pragma unroll
    for (int v = 0; v < SC::NV; ++v) {
        const int hl = SC::head(lane, v);
        float lsum = 0.f;
        if (hl < G) {
#pragma unroll
            for (int s = 0; s < SC::NS; ++s) {
                const int row = SC::row(lane, w, s);
                const float p = (t0 + row < n) ? exp_weight(sc.x[s][v], mt[v], c2) : 0.f;
                Pw[row * G + hl] = p;
                lsum += p;
            }
        }
        lsum = SC::reduce_sum(lsum);
        if (SC::writer(lane) && hl < 16) red_l[w][hl] = lsum;
    }
    __syncthreads();

    // V pass: wave w takes the 16-row blocks 64 s + 16 w of the tile (as the
    // scorer does), 16 lanes per row (8 elements each), 4 rows per load
    // instruction; the loads of VCH blocks are in flight together and rows
    // past the end read the block's row 0 with weight 0 (Pw is 0 there)
    constexpr int NSV = T / 64;
    constexpr int VCH_MAX = sizeof(KV) == 1 ? 4 : 2;     // e4m3 rows: twice the blocks in flight
    constexpr int VCH = NSV < VCH_MAX ? NSV : VCH_MAX;
    const int slot = lane >> 4, chunk = lane & 15;
    float acc[G][8];
#pragma unroll
    for (int hl = 0; hl < G; ++hl)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hl][e] = 0.f;
#pragma unroll
    for (int s0 = 0; s0 < NSV; s0 += VCH) {
        Raw8<KV> vv[VCH][4];
#pragma unroll
        for (int ii = 0; ii < VCH; ++ii) {
            const int j0 = t0 + 64 * (s0 + ii) + 16 * w;
            const size_t vb = block_base<PAGED>(L, b, g, j0, n, t0);
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int r = 4 * r4 + slot;
                const bool valid = j0 + r < n;
                vv[ii][r4] = load_raw8<KV>(v + vb + (size_t)(valid ? r : 0) * kHeadDim + 8 * chunk);
            }
        }
#pragma unroll
        for (int ii = 0; ii < VCH; ++ii)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int row = 64 * (s0 + ii) + 16 * w + 4 * r4 + slot;
                float xv[8];
                widen8(vv[ii][r4], xv);
#pragma unroll
                for (int hl = 0; hl < G; ++hl) {
                    const float p = Pw[row * G + hl];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[hl][e] = fmaf(p, xv[e], acc[hl][e]);
                }
            }
    }
#pragma unroll
    for (int hl = 0; hl < G; ++hl)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[hl][e] += __shfl_xor(acc[hl][e], 16);
            acc[hl][e] += __shfl_xor(acc[hl][e], 32);
        }
    if (lane < 16) {
#pragma unroll
        for (int hl = 0; hl < G; ++hl)
#pragma unroll
            for (int e = 0; e < 8; ++e) red_o[w][hl][8 * chunk + e] = acc[hl][e];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kBlock) {
        const int hl = idx / kHeadDim, d = idx - hl * kHeadDim;
        float s = red_o[0][hl][d];
#pragma unroll
        for (int ww = 1; ww < kWavesPerBlock; ++ww) s += red_o[ww][hl][d];
        const size_t bh = (size_t)b * num_q_heads + (size_t)g * G + hl;
        part_o[(bh * max_nt + tile) * kHeadDim + d] = s;
    }
    if (threadIdx.x < G) {
        const int hl = threadIdx.x;
        float m = red_m[0][hl], l = red_l[0][hl];
#pragma unroll
        for (int ww = 1; ww < kWavesPerBlock; ++ww) {
            m = fmaxf(m, red_m[ww][hl]);
            l += red_l[ww][hl];
        }
        const size_t bh = (size_t)b * num_q_heads + (size_t)g * G + hl;
        part_m[bh * max_nt + tile] = m;
        part_l[bh * max_nt + tile] = l;
    }
}

// ===================================================================
// launchers
// ===================================================================
template <typename KV, int G, int T, bool PAGED>
static hipError_t launch_exact_t(const LaunchArgs &a, const TimingHook &hook) {
    hipStream_t st = (hipStream_t)a.stream;
    const KVLayout L = layout_of(a);
    const int max_nt = a.max_nt;
    // with a timing hook the dispatch itself records the two events, so
    // they bracket the kernel's execution and nothing else
    if (hook.begin)
        hipExtLaunchKernelGGL((exact_partial_kernel<KV, G, T, PAGED>), dim3((unsigned)(a.batch * a.num_kv_heads * max_nt)), dim3(kBlock), 0, st, (hipEvent_t)hook.begin, (hipEvent_t)hook.end, 0,
                       (const typename QOf<KV>::type *)a.q, (const KV *)a.k, (const KV *)a.v, L, a.seq_lens, a.num_q_heads,
                       max_nt, a.scale, (float *)a.ws.part_m, (float *)a.ws.part_l, (float *)a.ws.part_o);
    else
        hipLaunchKernelGGL((exact_partial_kernel<KV, G, T, PAGED>), dim3((unsigned)(a.batch * a.num_kv_heads * max_nt)), dim3(kBlock), 0, st,
                       (const typename QOf<KV>::type *)a.q, (const KV *)a.k, (const KV *)a.v, L, a.seq_lens, a.num_q_heads,
                       max_nt, a.scale, (float *)a.ws.part_m, (float *)a.ws.part_l, (float *)a.ws.part_o);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(merge_tiles_kernel, dim3((unsigned)(a.batch * a.num_q_heads)), dim3(kMergeBlock),
                       sizeof(double) * (size_t)max_nt, st, (const float *)a.ws.part_m,
                       (const float *)a.ws.part_l, (const float *)a.ws.part_o, a.seq_lens, a.max_seq_len, T,
                       max_nt, a.batch, a.num_q_heads, a.num_kv_heads, 0, a.scale, a.out);
    return hipGetLastError();
}

template <typename KV>
hipError_t launch_exact_kv(const LaunchArgs &a, const TimingHook &hook) { SANTA_G_CASES(KV, launch_exact_t) }
SANTA_INSTANTIATE(launch_exact_kv)

}  // namespace santa
