// santa_flash.hip -- S2ANTA-flash tile kernel and launcher.
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
// Precision plan (why index parity with an fp64 oracle holds): scores are
// accumulated unscaled (bf16 products are exact in fp32; fp32 inputs use
// fp64), the tile max is subtracted before the scale is applied, and the
// local CDF positions P_j / Z_t are fp32 with thresholds formed in fp64.
#include "santa_kernels.h"

namespace santa {

// c[i] = #{m < len : th[m] < F[i]} for a nondecreasing fp32 list, the N searches
// in lockstep (binary lifting: c grows by each power of two, largest first,
// while th[c + step - 1] < F), so that their LDS reads are in flight together
template <int N>
__device__ __forceinline__ void count_below_f(const float *th, int len, const float (&F)[N], int (&c)[N]) {
    int step = 1;
    while (2 * step <= len) step <<= 1;
#pragma unroll
    for (int i = 0; i < N; ++i) c[i] = 0;
    for (; step > 0; step >>= 1) {
        float o[N];
#pragma unroll
        for (int i = 0; i < N; ++i) o[i] = th[min(c[i] + step, len) - 1];
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (c[i] + step <= len && o[i] < F[i]) c[i] += step;
    }
}

// ===================================================================
// S2ANTA-flash: tile kernel (score, local softmax, S_f local samples,
// gather) -- merge below
// ===================================================================
// part_m / part_z [B, Hq, nt] (unscaled tile max, local partition function)
// part_o [B, Hq, nt, d]: mean of the tile's S_f sampled V rows
//
// Local sampling per head (one wave): inclusive scan of the tile's weights,
// local thresholds on the local CDF P_j / Z_t, and the same per-element count
// rule as pass 2 of prop (counts of thresholds below each position, monotone,
// forced to S_f from the last nonzero weight on).  Systematic thresholds
// u_f + m/S_f (u_f = U * n_t) have closed-form counts.  With LIST: the
// stratified thresholds (m + u_m)/S_f go to an LDS list read by a
// three-comparison closed form; i.i.d. counts of up to 64 uniforms are taken
// across the wave from registers (the count does not depend on the order),
// longer lists are sorted in LDS and searched in lockstep.
template <typename KV, int G, int T, bool PAGED, bool LIST>
__global__ __launch_bounds__(kBlock) void flash_tile_kernel(
    const typename QOf<KV>::type *__restrict__ q, const KV *__restrict__ k, const KV *__restrict__ v, KVLayout L,
    int num_q_heads, int nt, int Sf, int S, int sampler, float scale, const float *__restrict__ u,
    float *__restrict__ part_m, float *__restrict__ part_z, float *__restrict__ part_o,
    int *__restrict__ sample_idx) {
    typedef typename ScorerFor<KV, G, T, PAGED>::type SC;
    typedef typename SC::acc_t acc_t;
    constexpr int EPL = T / 64;
    int tile, b, g;
    tile_of_block<PAGED>(L, nt, tile, b, g);
    const int n = L.max_seq_len;
    const int t0 = tile * T;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;

    // LDS: the scorer's staging area, then (after the barrier in tile_max)
    // the tile's exp-weights E[G][T] and, with LIST, the heads' local
    // threshold lists TH[G][S_f <= T]
    __shared__ __align__(16) unsigned char lds[cmax(SC::kStageVec * 16, (LIST ? 2 : 1) * G * T * 4)];
    __shared__ float red_m[kWavesPerBlock][16];
    float (*E)[T] = reinterpret_cast<float (*)[T]>(lds);
    float (*TH)[T] = reinterpret_cast<float (*)[T]>(lds + (LIST ? G * T * 4 : 0));

    // list generators: a head's uniforms for this tile (tile-major: this
    // tile's at t*S_f ..), outside [0,1) clamped into it (NaN and -0 as +0).
    // (Loading them before K was measured: the registers held through the
    // scorer cost a wave per SIMD, more than the overlap gained.)
    constexpr int RMAX = T / 64;                         // S_f <= T: uniforms per lane
    auto load_uniforms = [&](int hl, float (&uvo)[RMAX]) {
        const float kBelowOne = 1.0f - 0x1p-24f;
        const float *ub = u + ((size_t)b * num_q_heads + (size_t)g * G + hl) * S + (size_t)tile * Sf;
#pragma unroll
        for (int r = 0; r < RMAX; ++r) {
            const int m = lane + 64 * r;
            float x = m < Sf ? ub[m] : 0.f;
            x = x > 0.f ? x : 0.f;
            uvo[r] = x < kBelowOne ? x : kBelowOne;
        }
    };

    SC sc;
    sc.load_q(q + ((size_t)b * num_q_heads + (size_t)g * G) * kHeadDim);
    sc.score(k, L, b, g, t0, n, reinterpret_cast<u32x4 *>(lds));

    float mt[SC::NV];
    tile_max(sc, red_m, mt);
    const acc_t c2 = (acc_t)scale * (acc_t)1.4426950408889634;
#pragma unroll
    for (int v = 0; v < SC::NV; ++v) {
        const int hl = SC::head(lane, v);
        if (hl < G) {
#pragma unroll
            for (int s = 0; s < SC::NS; ++s) {
                const int row = SC::row(lane, w, s);
                E[hl][row] = (t0 + row < n) ? exp_weight(sc.x[s][v], mt[v], c2) : 0.f;
            }
        }
    }
    __syncthreads();

    for (int hl = w; hl < G; hl += kWavesPerBlock) {
        const int bh = b * num_q_heads + g * G + hl;
        float e[EPL];
        int lz = -1;
        float run = 0.f;
#pragma unroll
        for (int qq = 0; qq < EPL; ++qq) {
            e[qq] = E[hl][lane * EPL + qq];
            if (e[qq] > 0.f) lz = lane * EPL + qq;
            run += e[qq];
            e[qq] = run;
        }
        lz = wave_max(lz);
        const float lincl = wave_incl_scan(run, lane);
        float excl = __shfl_up(lincl, 1);
        if (lane == 0) excl = 0.f;
        const float Zt = __shfl(lincl, 63);
        int cj[EPL];
        int lmax = 0;
        if constexpr (!LIST) {
            const double uf = clamp_offset(u[bh], S) * (double)nt;
            // per-element local threshold counts #{m : u_f + m/S_f < P_j / Z_t}
            //   = ceil(P_j * a + b), a = S_f / Z_t, b = -u_f S_f (fp32; the
            //   rounding moves a threshold by ~1e-7 of the tile's mass)
            const float a = (float)((double)Sf / (double)Zt), bb = (float)(-uf * (double)Sf);
            const float fSf = (float)Sf;
#pragma unroll
            for (int qq = 0; qq < EPL; ++qq) {
                const int j = lane * EPL + qq;
                const int cc = (int)fminf(fmaxf(ceilf(fmaf(excl + e[qq], a, bb)), 0.f), fSf);
                lmax = max(lmax, j < lz ? cc : Sf);
                cj[qq] = lmax;
            }
        } else {
            // the tile's thresholds (uniforms tile-major: this tile's at
            // t*S_f ..; outside [0,1) clamped into it, NaN as 0)
            float *th = TH[hl];
            float uv[RMAX];
            load_uniforms(hl, uv);
            // local CDF positions P_j / Z_t
            const float invZt = 1.0f / Zt;
            float F[EPL];
            int cc[EPL];
#pragma unroll
            for (int qq = 0; qq < EPL; ++qq) F[qq] = (excl + e[qq]) * invZt;
            // counts c = #{thresholds < F}, with no chain of dependent LDS
            // reads: LDS is shared with the other workgroups' K staging, so
            // each dependent read waits long
            if (sampler == kSamplerIid && Sf <= 64) {
                // i.i.d., short list: the count does not depend on the order,
                // so lane m keeps u_m and every lane compares its positions
                // with each u_m in turn (read across the wave); no sort
#pragma unroll
                for (int qq = 0; qq < EPL; ++qq) cc[qq] = 0;
                const int ub = __float_as_int(uv[0]);
                for (int m = 0; m < Sf; ++m) {
                    const float t = __int_as_float(__builtin_amdgcn_readlane(ub, m));
#pragma unroll
                    for (int qq = 0; qq < EPL; ++qq) cc[qq] += (int)(t < F[qq]);
                }
            } else {
                if (sampler == kSamplerStrat) {
                    // (m + u_m)/S_f, formed in fp64, already in increasing order
#pragma unroll
                    for (int r = 0; r < RMAX; ++r) {
                        const int m = lane + 64 * r;
                        if (m < Sf) th[m] = (float)(((double)m + (double)uv[r]) / (double)Sf);
                    }
                } else {
                    // i.i.d.: rank of each uniform (ties by index), then placed
#pragma unroll
                    for (int r = 0; r < RMAX; ++r)
                        if (lane + 64 * r < Sf) th[lane + 64 * r] = uv[r];
                    wave_sync_lds();
                    // rank: the number of keys (bits of u_k, k) below (bits
                    // of u_m, m) as unsigned 64-bit integers (nonnegative
                    // floats order as their bits); 8 reads in flight
                    int rank[RMAX];
                    unsigned long long km[RMAX];
#pragma unroll
                    for (int r = 0; r < RMAX; ++r) {
                        rank[r] = 0;
                        km[r] = ((unsigned long long)__float_as_uint(uv[r]) << 32) | (unsigned)(lane + 64 * r);
                    }
                    for (int k0 = 0; k0 < Sf; k0 += 8) {
                        float o[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) o[i] = th[min(k0 + i, Sf - 1)];
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const unsigned long long ko = ((unsigned long long)__float_as_uint(o[i]) << 32) | (unsigned)(k0 + i);
#pragma unroll
                            for (int r = 0; r < RMAX; ++r) rank[r] += (int)((k0 + i < Sf) & (ko < km[r]));
                        }
                    }
                    wave_sync_lds();
#pragma unroll
                    for (int r = 0; r < RMAX; ++r)
                        if (lane + 64 * r < Sf) th[rank[r]] = uv[r];
                }
                wave_sync_lds();
                if (sampler == kSamplerStrat) {
                    // thresholds (m + u_m)/S_f lie in [m/S_f, (m+1)/S_f]:
                    // every m <= k-2 is below F and every m >= k+2 is not,
                    // with k = floor(F S_f) (a margin of 1/S_f, far above the
                    // rounding), so three comparisons give the exact count
#pragma unroll
                    for (int qq = 0; qq < EPL; ++qq) {
                        const int k = (int)fminf(fmaxf(floorf(F[qq] * (float)Sf), 0.f), (float)Sf);
                        const float a0 = th[max(k - 1, 0)], a1 = th[min(k, Sf - 1)], a2 = th[min(k + 1, Sf - 1)];
                        cc[qq] = max(k - 1, 0) + (int)(k >= 1 && a0 < F[qq]) + (int)(k < Sf && a1 < F[qq]) +
                                 (int)(k + 1 < Sf && a2 < F[qq]);
                    }
                } else {
                    count_below_f(th, Sf, F, cc);   // i.i.d., long list: sorted, searched in lockstep
                }
            }
#pragma unroll
            for (int qq = 0; qq < EPL; ++qq) {
                const int j = lane * EPL + qq;
                lmax = max(lmax, j < lz ? cc[qq] : Sf);
                cj[qq] = lmax;
            }
        }
        const int lmax_incl = wave_incl_max_scan(lmax, lane);
        int pmax = __shfl_up(lmax_incl, 1);
        if (lane == 0) pmax = 0;
        // selected rows of this head go to an LDS list that reuses E[hl]
        // (S_f <= T is checked on the host), after every lane has read it
        wave_sync_lds();
        int *sel = reinterpret_cast<int *>(&E[hl][0]);
        int prev = pmax;
#pragma unroll
        for (int qq = 0; qq < EPL; ++qq) {
            const int cc = max(cj[qq], pmax);
            for (int m = prev; m < cc; ++m) sel[m] = t0 + lane * EPL + qq;
            prev = cc;
        }
        wave_sync_lds();
        if (sample_idx)
            for (int m = lane; m < Sf; m += 64) sample_idx[(size_t)bh * S + (size_t)tile * Sf + m] = sel[m];
        // gather S_f rows: 16 lanes per row, 4 rows per instruction
        const int slot = lane >> 4, chunk = lane & 15;
        float acc[8];
#pragma unroll
        for (int ee = 0; ee < 8; ++ee) acc[ee] = 0.f;
#pragma unroll 4
        for (int m = slot; m < Sf; m += 4) {
            float xv[8];
            load_v8<KV>(v + row_offset<PAGED>(L, b, g, sel[m]) + 8 * chunk, xv);
#pragma unroll
            for (int ee = 0; ee < 8; ++ee) acc[ee] += xv[ee];
        }
#pragma unroll
        for (int ee = 0; ee < 8; ++ee) {
            acc[ee] += __shfl_xor(acc[ee], 16);
            acc[ee] += __shfl_xor(acc[ee], 32);
        }
        const bool pow2 = (Sf & (Sf - 1)) == 0;
        if (lane < 16) {
            float *dst = part_o + ((size_t)bh * nt + tile) * kHeadDim + 8 * lane;
#pragma unroll
            for (int ee = 0; ee < 8; ++ee) dst[ee] = pow2 ? acc[ee] * (1.0f / (float)Sf) : acc[ee] / (float)Sf;
        }
        if (lane == 0) {
            float m = red_m[0][hl];
#pragma unroll
            for (int ww = 1; ww < kWavesPerBlock; ++ww) m = fmaxf(m, red_m[ww][hl]);
            part_m[(size_t)bh * nt + tile] = m;
            part_z[(size_t)bh * nt + tile] = Zt;
        }
    }
}

// ===================================================================
// launchers
// ===================================================================
template <typename KV, int G, int T, bool PAGED>
static hipError_t launch_flash_t(const LaunchArgs &a, const TimingHook &hook) {
    hipStream_t st = (hipStream_t)a.stream;
    const KVLayout L = layout_of(a);
    const int nt = a.max_nt;
    // with a timing hook the dispatch itself records the two events, so
    // they bracket the kernel's execution and nothing else
    auto launch = [&](auto kernel) {
        if (hook.begin)
            hipExtLaunchKernelGGL(kernel, dim3((unsigned)(a.batch * a.num_kv_heads * nt)), dim3(kBlock), 0, st,
                                  (hipEvent_t)hook.begin, (hipEvent_t)hook.end, 0,
                                  (const typename QOf<KV>::type *)a.q, (const KV *)a.k, (const KV *)a.v, L,
                                  a.num_q_heads, nt, a.S / nt, a.S, a.sampler, a.scale, a.u, (float *)a.ws.part_m,
                                  (float *)a.ws.part_l, (float *)a.ws.part_o, a.sample_idx);
        else
            hipLaunchKernelGGL(kernel, dim3((unsigned)(a.batch * a.num_kv_heads * nt)), dim3(kBlock), 0, st,
                               (const typename QOf<KV>::type *)a.q, (const KV *)a.k, (const KV *)a.v, L,
                               a.num_q_heads, nt, a.S / nt, a.S, a.sampler, a.scale, a.u, (float *)a.ws.part_m,
                               (float *)a.ws.part_l, (float *)a.ws.part_o, a.sample_idx);
    };
    if (a.sampler == kSamplerSys) launch(flash_tile_kernel<KV, G, T, PAGED, false>);
    else launch(flash_tile_kernel<KV, G, T, PAGED, true>);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(merge_tiles_kernel, dim3((unsigned)(a.batch * a.num_q_heads)), dim3(kMergeBlock),
                       sizeof(double) * (size_t)nt, st, (const float *)a.ws.part_m,
                       (const float *)a.ws.part_l, (const float *)a.ws.part_o, (const int *)nullptr,
                       a.max_seq_len, T, nt, a.batch, a.num_q_heads, a.num_kv_heads, 1, a.scale, a.out);
    return hipGetLastError();
}

template <typename KV>
hipError_t launch_flash_kv(const LaunchArgs &a, const TimingHook &hook) { SANTA_G_CASES(KV, launch_flash_t) }
SANTA_INSTANTIATE(launch_flash_kv)

}  // namespace santa
