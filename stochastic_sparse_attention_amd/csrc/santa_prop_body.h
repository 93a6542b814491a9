// santa_prop_body.h -- the two halves of S2ANTA-prop as device functions:
// pass 1 of one tile (scores, tile max, tile partition function, stash) and
// the reducer + pass 2 of one head.  santa_prop_pass1.hip and santa_prop.hip
// wrap them in the two kernels of santa_decode_prop; santa_prop_fused.hip
// runs both in one launch.
//
// The method follows the web page "Stochastic Sparse Attention for
// Memory-Bound Inference" (ICML 2026 paper notes on SANTA):
//   key design 1  systematic sampling: one offset U in [0,1/S), thresholds
//                 U + m/S, selected index = inverse CDF at each threshold
//   key design 2  S2ANTA-prop: pass 1 scores and stashes exp-scores with the
//                 tile partition function, a reducer turns the n_t tile
//                 masses into per-tile budgets, pass 2 samples and gathers V
//
// Precision plan (why index parity with an fp64 oracle holds): scores are
// accumulated unscaled (bf16 products are exact in fp32; fp32 inputs use
// fp64), the tile max is subtracted before the scale is applied, the reducer
// works in fp64, and pass 2 evaluates each CDF position as one fp32 fma
// whose coefficients were formed in fp64.
#pragma once

#include "santa_kernels.h"

namespace santa {

// ===================================================================
// S2ANTA-prop, pass 1: scores, tile max, tile partition function, stash
// ===================================================================
// grid: B * Hkv * max_nt workgroups (tile fastest); block: 256 threads.
// stash [B, Hq, max_nt * T] fp32 (rows padded to whole tiles):
// e_j = exp(scale * (x_j - m_t))
// stats [B, Hq, max_nt] float2: (m_t unscaled tile max, Z_t = sum_j e_j)
// Scores, tile max, partition function and stash of tile `tile` of KV group
// (b, g), by one workgroup of kBlock threads (t0 < n).
template <typename KV, int G, int T, bool PAGED>
__device__ __forceinline__ void pass1_tile(
    const typename QOf<KV>::type *__restrict__ q, const KV *__restrict__ k, KVLayout L, int n,
    int num_q_heads, int max_nt, float scale, float *__restrict__ stash, float2 *__restrict__ stats,
    int tile, int b, int g) {
    typedef typename ScorerFor<KV, G, T, PAGED>::type SC;
    typedef typename SC::acc_t acc_t;
    const int t0 = tile * T;
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

// ===================================================================
// S2ANTA-prop, reducer + pass 2: one workgroup per (request, q head), of
// 16 waves (8 or 4 with many heads), or two (part 0 and 1 of nparts = 2)
// when heads are few.  Both parts run the reducer; their waves take
// alternate groups of visited tiles, and each adds its share of the output
// onto the row that pass 1 zeroed (two addends onto zero: the same sum in
// either order).  Nothing else passes between workgroups.
// ===================================================================
// Reducer (wave 0; lane l owns tiles [l CH, l CH + CH), CH = ceil(n_t/64),
// n_t <= 1024): global max M of the tile maxima, tile masses
// z_t = Z_t e^{scale (m_t - M)}, Z = sum z_t, tile CDF C_t (fp64,
// C_{n_t-1} := 1), threshold counts cnt_t = #{thresholds < C_t} made
// monotone, budgets S_t = cnt_t - cnt_{t-1}; tiles with S_t > 0 go to an LDS
// visit list in tile order.
// Pass 2 (LPT lanes per visited tile, EPL consecutive tokens per lane):
// inclusive scan of the tile's stash P_j, then the count c_j of thresholds
// below the CDF position of token j, clamped to the tile's threshold range
// (see VisitRec).  Token j takes thresholds c_{j-1} .. c_j - 1, so only the
// tokens where the count steps are recorded: a marker (row j, multiplicity
// c_j - c_{j-1}) at LDS position c_{j-1}.  If the fp32 tile total falls short
// of the tile's last threshold, the remaining ones go to the last token of
// nonzero weight, as a marker at the short count.  Every threshold position
// holds the marker of its token or lies after it in the same tile, so a
// running max over positions gives the index list.
// Gather: each wave reads the V rows of its own tiles' markers right away
// (16 lanes per row, 4 rows per wave instruction) and accumulates
// multiplicity * row; the waves' sums are added in a fixed order and
// divided by S.
// Visit record of a tile with S_t > 0: its thresholds are first .. first+cnt-1.
// Systematic thresholds: the number of thresholds below the CDF position of
// its element j is ceil(P_j * a + b), with P_j the stash prefix,
// a = S e^{scale(m_t-M)}/Z and b = S (C_{t-1} - U).  Stratified and i.i.d.
// thresholds: P_j * a + b is that CDF position itself (a = e^{scale(m_t-M)}/Z,
// b = C_{t-1}).  Both are formed in fp64 and rounded to fp32; the rounding
// moves a threshold by ~1e-7 in CDF units.
struct VisitRec {
    int t, first, cnt;
    float a, b;
};

constexpr int kRegisterTiles = 256;  // up to this many tiles the reducer keeps them in registers
constexpr int kStepSlots = 16;       // stepping lanes a wave stages in LDS at a time (systematic pass 2)
constexpr int kGatherRounds = 4;     // V rows per lane slot in flight together in the gather

// EPL consecutive floats from a 16-byte aligned address (EPL = T/64)
template <int EPL>
__device__ __forceinline__ void load_stash(const float *p, float (&e)[EPL]) {
    if constexpr (EPL >= 4) {
#pragma unroll
        for (int i = 0; i < EPL; i += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(p + i);
            e[i] = v.x; e[i + 1] = v.y; e[i + 2] = v.z; e[i + 3] = v.w;
        }
    } else if constexpr (EPL == 2) {
        const float2 v = *reinterpret_cast<const float2 *>(p);
        e[0] = v.x; e[1] = v.y;
    } else {
        e[0] = p[0];
    }
}

// Threshold counts: the number of thresholds strictly below a CDF position.
// Systematic thresholds U + m/S have the closed form; the stratified and
// i.i.d. generators give a sorted list in LDS, searched by bisection.
struct SysCount {
    double U;
    int S;
    __device__ __forceinline__ int operator()(double C) const { return thresholds_below(C, U, S); }
    // visit record: count below the position of token j = ceil(P_j a + b)
    __device__ __forceinline__ void rec_ab(double f, double invZ, double cprev, float &a, float &b) const {
        a = (float)((double)S * f * invZ);
        b = (float)((double)S * (cprev - U));
    }
};
struct ListCount {
    const double *thr;    // [S], nondecreasing, in [0, 1)
    int S;
    bool strat;           // thr[m] = (m + u_m)/S, i.e. thr[m] in [m/S, (m+1)/S)
    __device__ __forceinline__ int operator()(double C) const {
        if (strat) {
            // every threshold m <= k-2 is below C and every m >= k+2 is not,
            // with k = floor(C S) (a margin of 1/S, far above the rounding
            // of C S and of thr), so three comparisons give the exact count;
            // the three reads are unconditional (clamped indices), so they
            // are in flight together
            const int k = (int)fmin(fmax(floor(C * (double)S), 0.0), (double)S);
            const double a0 = thr[max(k - 1, 0)], a1 = thr[min(k, S - 1)], a2 = thr[min(k + 1, S - 1)];
            return max(k - 1, 0) + (int)(k >= 1 && a0 < C) + (int)(k < S && a1 < C) + (int)(k + 1 < S && a2 < C);
        }
        int lo = 0, hi = S;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (thr[mid] < C) lo = mid + 1;
            else hi = mid;
        }
        return lo;
    }
    // visit record: CDF position of token j = P_j a + b
    __device__ __forceinline__ void rec_ab(double f, double invZ, double cprev, float &a, float &b) const {
        a = (float)(f * invZ);
        b = (float)cprev;
    }
};

// Reducer of one head on one wave, with each lane's tiles (at most CHR of
// them: lane l owns tiles [l*CH, l*CH + CH), CH = ceil(n_t/64)) held in
// registers.  Writes the visit list, its length and the optional budgets.
// The arithmetic and its order are those of the LDS variant below.
constexpr int kStatRegs = kRegisterTiles / 64;   // tiles per reducer lane held in registers

// the reducer lane's tile statistics (m_t, Z_t) for the register reducer,
// (-inf, 0) past the lane's tiles (nt >= 1).  Every load is issued
// unconditionally, from a clamped index, and masked afterwards: under a
// per-lane condition each load became a branch, and the last one waited
// for all of them on the spot
__device__ __forceinline__ void load_lane_stats(const float2 *__restrict__ stp, int nt, int lane,
                                                float2 (&st)[kStatRegs]) {
    const int CH = (nt + 63) / 64;
    const int tb = lane * CH;
    float2 raw[kStatRegs];
#pragma unroll
    for (int i = 0; i < kStatRegs; ++i) raw[i] = stp[min(tb + i, nt - 1)];
#pragma unroll
    for (int i = 0; i < kStatRegs; ++i) {
        const bool ok = i < CH && tb + i < nt;
        st[i] = ok ? raw[i] : make_float2(-INFINITY, 0.f);
    }
}

template <int CHR, class CNT>
__device__ __forceinline__ void reduce_in_registers(const float2 (&st)[kStatRegs], int nt, int lane, const CNT &count,
                                                    float scale, int kcap, VisitRec *vis,
                                                    int *__restrict__ budget, int max_nt, int &nvis_out) {
    const int CH = (nt + 63) / 64;
    const int tb = lane * CH;
    float lmaxv = -INFINITY;
#pragma unroll
    for (int i = 0; i < CHR; ++i) lmaxv = fmaxf(lmaxv, st[i].x);
    const float Mf = wave_max(lmaxv);
    // tile weight e^{scale (m_t - M)} in fp32: its rounding moves a tile's
    // CDF interval by ~1e-7 of the tile's own mass, and the same value is
    // used for C_t and for the pass-2 mapping, so the two stay consistent
    const float c2 = scale * 1.4426950408889634f;
    double f[CHR];
    double lsum = 0.0;
#pragma unroll
    for (int i = 0; i < CHR; ++i) {
        const bool ok = i < CH && tb + i < nt;
        f[i] = ok ? (double)exp2f((st[i].x - Mf) * c2) : 0.0;
        if (ok) lsum += (double)st[i].y * f[i];
    }
    const double incl = wave_incl_scan(lsum, lane);
    double excl = __shfl_up(incl, 1);
    if (lane == 0) excl = 0.0;
    const double Z = __shfl(incl, 63);
    const double invZ = 1.0 / Z;
    double C[CHR];
    int c[CHR];
    bool okv[CHR];
    double lrun = 0.0, clast = 0.0;
    int lcnt = 0;
#pragma unroll
    for (int i = 0; i < CHR; ++i) {
        okv[i] = i < CH && tb + i < nt;
        if (okv[i]) lrun += (double)st[i].y * f[i];
        C[i] = (tb + i == nt - 1) ? 1.0 : (excl + lrun) * invZ;
    }
#pragma unroll
    for (int i = 0; i < CHR; ++i) c[i] = okv[i] ? count(C[i]) : 0;
#pragma unroll
    for (int i = 0; i < CHR; ++i) {
        if (okv[i]) {
            lcnt = max(lcnt, c[i]);
            clast = C[i];
        }
    }
    const int cmax = wave_incl_max_scan(lcnt, lane);
    int cpred = __shfl_up(cmax, 1);
    double Cpred = __shfl_up(clast, 1);      // C of the previous lane's last tile
    if (lane == 0) {
        cpred = 0;
        Cpred = 0.0;
    }
    int nvl = 0;
    {
        int cp = cpred;
#pragma unroll
        for (int i = 0; i < CHR; ++i) {
            if (i < CH && tb + i < nt) {
                const int cnt = max(cp, c[i]);
                nvl += cnt > cp;
                cp = cnt;
            }
        }
    }
    const int vincl = wave_incl_scan(nvl, lane);
    int vpos = vincl - nvl;
    if (lane == 63) nvis_out = vincl;
    int cp = cpred;
    double cprev = Cpred;
#pragma unroll
    for (int i = 0; i < CHR; ++i) {
        const int t = tb + i;
        if (i < CH && t < nt) {
            const int cnt = max(cp, c[i]);
            const int St = cnt - cp;
            if (budget) budget[t] = St;
            if (St > 0 && vpos < kcap) {
                VisitRec rec;
                rec.t = t;
                rec.first = cp;
                rec.cnt = St;
                count.rec_ab(f[i], invZ, cprev, rec.a, rec.b);
                vis[vpos] = rec;
                ++vpos;
            }
            cp = cnt;
            cprev = C[i];
        }
    }
    if (budget)
        for (int t = nt + lane; t < max_nt; t += 64) budget[t] = 0;
}

// Per-tile arrays of the LDS reducer (more than 4 tiles per lane).
struct ReducerLds {
    float2 *tstat;    // (m_t, Z_t)
    double *tf;       // e^{scale (m_t - M)}
    double *tC;       // tile CDF C_t
    int *tcn;         // thresholds below C_t
};

template <class CNT>
__device__ __forceinline__ void reduce_with_lds(const float2 *__restrict__ stp, int nt, int lane, const CNT &count,
                                                float scale, int kcap, VisitRec *vis, int *__restrict__ budget,
                                                int max_nt, int &nvis_out, const ReducerLds &R) {
    const int CH = (nt + 63) / 64;
    const int tb = lane * CH, te = min(nt, tb + CH);
    float lmaxv = -INFINITY;
    for (int t = tb; t < te; ++t) {
        const float2 v2 = stp[t];
        R.tstat[t] = v2;
        lmaxv = fmaxf(lmaxv, v2.x);
    }
    const float Mf = wave_max(lmaxv);
    const float c2 = scale * 1.4426950408889634f;
    double lsum = 0.0;
    for (int t = tb; t < te; ++t) {
        const float2 v2 = R.tstat[t];
        const double f = (double)exp2f((v2.x - Mf) * c2);
        R.tf[t] = f;
        lsum += (double)v2.y * f;
    }
    const double incl = wave_incl_scan(lsum, lane);
    double excl = __shfl_up(incl, 1);
    if (lane == 0) excl = 0.0;
    const double Z = __shfl(incl, 63);
    const double invZ = 1.0 / Z;
    // C_t = (excl + lane-local running sum) / Z, C_{n_t-1} := 1, and the
    // count of thresholds below each C_t (once per tile; the counts are
    // made monotone across lanes below)
    double lrun = 0.0;
    int lcnt = 0;
    for (int t = tb; t < te; ++t) {
        lrun += (double)R.tstat[t].y * R.tf[t];
        const double C = (t == nt - 1) ? 1.0 : (excl + lrun) * invZ;
        R.tC[t] = C;
        const int c = count(C);
        R.tcn[t] = c;
        lcnt = max(lcnt, c);
    }
    const int cmax = wave_incl_max_scan(lcnt, lane);
    int cpred = __shfl_up(cmax, 1);
    double Cpred = __shfl_up(te > tb ? R.tC[te - 1] : 0.0, 1);      // C of the previous lane's last tile
    if (lane == 0) {
        cpred = 0;
        Cpred = 0.0;
    }
    // visited tiles of this lane, then their positions in the visit list
    int nvl = 0;
    {
        int cp = cpred;
        for (int t = tb; t < te; ++t) {
            const int cnt = max(cp, R.tcn[t]);
            nvl += cnt > cp;
            cp = cnt;
        }
    }
    const int vincl = wave_incl_scan(nvl, lane);
    int vpos = vincl - nvl;
    if (lane == 63) nvis_out = vincl;
    int cp = cpred;
    double cprev = Cpred;
    for (int t = tb; t < te; ++t) {
        const int cnt = max(cp, R.tcn[t]);
        const int St = cnt - cp;
        if (budget) budget[t] = St;
        if (St > 0 && vpos < kcap) {
            VisitRec rec;
            rec.t = t;
            rec.first = cp;
            rec.cnt = St;
            count.rec_ab(R.tf[t], invZ, cprev, rec.a, rec.b);
            vis[vpos] = rec;
            ++vpos;
        }
        cp = cnt;
        cprev = R.tC[t];
    }
    if (budget)
        for (int t = nt + lane; t < max_nt; t += 64) budget[t] = 0;
}

// st: the lane's statistics from load_lane_stats when nt <= kRegisterTiles
template <class CNT>
__device__ __forceinline__ void reduce_head(const float2 *__restrict__ stp, const float2 (&st)[kStatRegs], int nt,
                                            int lane, const CNT &count, float scale, int kcap, VisitRec *vis,
                                            int *__restrict__ budget, int max_nt, int &nvis_out,
                                            const ReducerLds &R) {
    static_assert(kStatRegs == 4, "register reducer variants");
    if (nt <= 64)
        reduce_in_registers<1>(st, nt, lane, count, scale, kcap, vis, budget, max_nt, nvis_out);
    else if (nt <= 128)
        reduce_in_registers<2>(st, nt, lane, count, scale, kcap, vis, budget, max_nt, nvis_out);
    else if (__builtin_expect(nt <= kRegisterTiles, 1))
        reduce_in_registers<4>(st, nt, lane, count, scale, kcap, vis, budget, max_nt, nvis_out);
    else
        reduce_with_lds(stp, nt, lane, count, scale, kcap, vis, budget, max_nt, nvis_out, R);
}

// #{m in [0, len) : thr[m] < F} for a nondecreasing list
__device__ __forceinline__ int count_below(const double *thr, int len, double F) {
    int lo = 0, hi = len;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (thr[mid] < F) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// #{m : thr[m] < F} clamped to [lo, hi], for the sorted list of S
// thresholds; equal to lo + #{m in [lo, hi) : thr[m] < F} because the
// thresholds below F form a prefix.  Stratified: the closed form of
// ListCount; i.i.d.: a bisection over [lo, hi).
__device__ __forceinline__ int count_in_range(const ListCount &lc, double F, int lo, int hi) {
    if (lc.strat) return min(max(lc(F), lo), hi);
    return lo + count_below(lc.thr + lo, hi - lo, F);
}

// the largest float at or below x, for x >= 0: the nearest float, one step
// down if it lies above x (it is then > 0)
__device__ __forceinline__ float float_at_or_below(double x) {
    const float r = (float)x;
    return (double)r > x ? __uint_as_float(__float_as_uint(r) - 1u) : r;
}


// Reducer and pass 2 of head hl of KV group (b, g), run by one workgroup of
// NW waves (its own kernel below, or the last workgroup of a group in the
// single-launch variant).  LIST: stratified / i.i.d. thresholds (a sorted
// list in LDS); else the systematic closed form
// NW: waves per workgroup (16; 8 or 4 for many heads: more heads per CU)
// Registers: systematic, at most 64 VGPRs (8 waves per SIMD), so that two
// 16-wave or four 8-wave workgroups share a compute unit; list generators,
// at most 128 (4 waves per SIMD): one 16-wave or two 8-wave workgroups.
template <typename KV, int T, bool PAGED, bool LIST, int NW>
__device__ __forceinline__ void sample_head(
    const KV *__restrict__ v, KVLayout L, const int *__restrict__ seq_lens, int num_q_heads,
    int G, int S, int max_nt, int kcap, int sampler, const float *__restrict__ u, float scale,
    const float *__restrict__ stash, const float2 *__restrict__ stats, float *__restrict__ out,
    int *__restrict__ sample_idx, int *__restrict__ tile_budget, int stash_shift, int b, int g, int hl,
    int part, int nparts) {
    constexpr int SB = NW * kWave;                  // threads per workgroup
    extern __shared__ __align__(16) unsigned char smem[];
    // stratified / i.i.d.: the sorted thresholds first (padded to a power of
    // two for the sort), then the visit list and the marker arrays
    constexpr bool list = LIST;
    const int np = list ? threshold_slots(S, sampler) : 0;
    double *thr = reinterpret_cast<double *>(smem);                                     // [np]
    VisitRec *vis = reinterpret_cast<VisitRec *>(smem + (size_t)np * sizeof(double));   // [kcap]
    int *jsel = reinterpret_cast<int *>(smem + (size_t)np * sizeof(double) + (size_t)kcap * sizeof(VisitRec));   // [S] marker rows, -1 elsewhere
    int *jmul = jsel + S;                                                  // [S] marker multiplicities
    // per-tile arrays of the LDS reducer (more than 256 tiles; sized only
    // when max_nt needs them): (m_t, Z_t), e^{scale (m_t - M)}, C_t, counts
    unsigned char *rbase = reinterpret_cast<unsigned char *>(jmul + S);
    rbase += (8 - ((uintptr_t)rbase & 7)) & 7;
    const int rn = max_nt > kRegisterTiles ? max_nt : 0;
    double *tf = reinterpret_cast<double *>(rbase);
    double *tC = tf + rn;
    float2 *tstat = reinterpret_cast<float2 *>(tC + rn);
    int *tcn = reinterpret_cast<int *>(tstat + rn);
    __shared__ float red[NW][kHeadDim];
    __shared__ int nvis_sh;
    __shared__ int wrow[NW][kWave];        // per-wave compacted marker rows
    __shared__ float wmul[NW][kWave];      // and their multiplicities
    // per-wave slots of the lanes whose count steps (systematic thresholds):
    // their in-lane prefixes, (b_lane, a, hi, prev) and first token row
    __shared__ __align__(16) float stepP[NW][kStepSlots][16];
    __shared__ float4 stepM[NW][kStepSlots];
    __shared__ int stepRow[NW][kStepSlots];

    const int bh = b * num_q_heads + g * G + hl;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = seq_len_of(seq_lens, L.max_seq_len, b);
    const int nt = (n + T - 1) / T;

    // rare branches are marked unlikely: the compiler then places their
    // code after the hot path, which spans fewer instruction-cache lines
    if (__builtin_expect(nt == 0, 0)) {             // empty request
        if (tile_budget)
            for (int t = tid; t < max_nt; t += SB) tile_budget[(size_t)bh * max_nt + t] = 0;
        if (sample_idx)
            for (int m = tid; m < S; m += SB) sample_idx[(size_t)bh * S + m] = -1;
        if (tid < kHeadDim) out[(size_t)bh * kHeadDim + tid] = 0.f;
        return;
    }
    // the reducer's inputs, issued first and together: the systematic
    // offset and the tile statistics (their latency overlaps the threshold
    // loads below)
    const float2 *stp = stats + (size_t)bh * max_nt;
    float2 st[kStatRegs];
    float u_sys = 0.f;
    if (w == 0) {
        if constexpr (!LIST) u_sys = u[bh];
        if (nt <= kRegisterTiles) load_lane_stats(stp, nt, lane, st);
    }

    // ---------------- thresholds of the stratified and i.i.d. generators:
    // (m + u_m)/S, or the uniforms sorted, in fp64 (uniforms outside [0,1)
    // are clamped into it; NaN counts as 0)
    if constexpr (LIST) {
        const float *ub = u + (size_t)bh * S;
        const double kBelowOne = 1.0 - 0x1p-53;
        const double kUniformMax = 1.0 - 0x1p-24;      // the largest float below 1
        // i.i.d. up to SB thresholds: the clamped uniforms are exact fp32
        // values, ranked as fp32 keys held in the marker array (free until
        // the reducer) and then placed into thr
        const bool rank_sort = sampler == kSamplerIid && S <= SB;
        float *keyf = reinterpret_cast<float *>(jsel);
        for (int m = tid; m < np; m += SB) {
            double x = INFINITY;                        // sort padding
            if (m < S) {
                x = (double)ub[m];
                x = x > 0.0 ? x : 0.0;                  // NaN and -0 become +0
                x = x < kUniformMax ? x : kUniformMax;
                if (sampler == kSamplerStrat) x = ((double)m + x) / (double)S;
                x = x < kBelowOne ? x : kBelowOne;
            }
            if (rank_sort) {
                if (m < S) keyf[m] = (float)x;
            } else {
                thr[m] = x;
            }
        }
        __syncthreads();
        if (rank_sort) {
            // rank sort: threshold m goes to position #{j : x_j < x_m} +
            // #{j < m : x_j == x_m}, i.e. the number of keys (bits of x_j,
            // j) below (bits of x_m, m) as unsigned 64-bit integers (the
            // order of nonnegative floats is that of their bits); P = SB/S
            // (a power of two, at most 64) consecutive lanes share one
            // threshold's comparisons
            int P = 1;
            while (P < 64 && 2 * P * S <= SB) P <<= 1;
            const int m = tid / P, pp = tid % P;
            float x = 0.f;
            int rank = 0;
            if (m < S) {
                x = keyf[m];
                const unsigned long long km = ((unsigned long long)__float_as_uint(x) << 32) | (unsigned)m;
                // 8 reads in flight per batch (indices clamped, the extra
                // ones masked out of the count), no branch per element
                for (int j0 = pp; j0 < S; j0 += 8 * P) {
                    float y[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) y[i] = keyf[min(j0 + i * P, S - 1)];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int j = j0 + i * P;
                        const unsigned long long kj = ((unsigned long long)__float_as_uint(y[i]) << 32) | (unsigned)j;
                        rank += (int)((j < S) & (kj < km));
                    }
                }
            }
            for (int o = 1; o < P; o <<= 1) rank += __shfl_xor(rank, o);
            // the keys are only read above and thr only written below
            if (m < S && pp == 0) thr[rank] = (double)x;
            __syncthreads();
        } else if (sampler == kSamplerIid) {
            // bitonic sort of the np slots, ascending
            for (int k2 = 2; k2 <= np; k2 <<= 1) {
                for (int j2 = k2 >> 1; j2 > 0; j2 >>= 1) {
                    for (int i = tid; i < np; i += SB) {
                        const int p = i ^ j2;
                        if (p > i) {
                            const double a = thr[i], c = thr[p];
                            const bool up = (i & k2) == 0;
                            if ((a > c) == up) {
                                thr[i] = c;
                                thr[p] = a;
                            }
                        }
                    }
                    __syncthreads();
                }
            }
        }
    }

    // ---------------- reducer: wave 0, lane l owns tiles [l*CH, l*CH + CH);
    // the other waves clear the marker positions meanwhile
    if (w != 0) {
        for (int m = tid - kWave; m < S; m += SB - kWave) jsel[m] = -1;
    } else {
        int *budget = tile_budget && part == 0 ? tile_budget + (size_t)bh * max_nt : nullptr;
        const ReducerLds R{tstat, tf, tC, tcn};
        if constexpr (!LIST)
            reduce_head(stp, st, nt, lane, SysCount{clamp_offset(u_sys, S), S}, scale, kcap, vis, budget, max_nt, nvis_sh, R);
        else
            reduce_head(stp, st, nt, lane, ListCount{thr, S, sampler == kSamplerStrat}, scale, kcap, vis, budget,
                        max_nt, nvis_sh, R);
    }
    __syncthreads();
    const int nvis = min(nvis_sh, kcap);

    // ---------------- pass 2 + gather, per wave: TPW visited tiles at once,
    // LPT lanes per tile, EPL2 consecutive stash values per lane
    constexpr int LPT = T >= 1024 ? 64 : (T >= 512 ? 32 : 16);
    constexpr int TPW = 64 / LPT;
    constexpr int EPL2 = T / LPT;
    static_assert(EPL2 <= 32, "a lane's tokens fit one 32-bit mask");
    const int sub = lane / LPT, gl = lane % LPT;          // tile slot in the wave, lane in group
    const int slot = lane >> 4, chunk = lane & 15;        // gather: row slot, 8-element chunk
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // V sums of the wave's 4 row slots
    // gather of the markers at positions [m_lo, m_hi), 64 at a time: they
    // are compacted into the wave's LDS list, then read 4 rows per wave
    // instruction with every load of a round in flight together; each row
    // is weighed by its multiplicity
    auto gather_range = [&](int m_lo, int m_hi) {
        for (int c = m_lo; c < m_hi; c += kWave) {
            const int m = c + lane;
            const int r = (m < m_hi) ? jsel[m] : -1;
            const unsigned long long bal = __ballot(r >= 0);
            const int nm = __popcll(bal);
            if (r >= 0) {
                const int pos = __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
                wrow[w][pos] = r;
                wmul[w][pos] = (float)jmul[m];
            }
            wave_sync_lds();
            for (int i0 = 0; i0 < nm; i0 += 4 * kGatherRounds) {
                int rows[kGatherRounds];
                float mul[kGatherRounds];
#pragma unroll
                for (int u = 0; u < kGatherRounds; ++u) {
                    // slots past the list re-read its first row with weight 0
                    const int idx = i0 + slot + 4 * u;
                    rows[u] = wrow[w][idx < nm ? idx : 0];
                    mul[u] = idx < nm ? wmul[w][idx] : 0.f;
                }
                // every load of the batch in flight as raw storage, each
                // widened only when it is added
                Raw8<KV> raw[kGatherRounds];
#pragma unroll
                for (int u = 0; u < kGatherRounds; ++u)
                    raw[u] = load_raw8<KV>(v + row_offset<PAGED>(L, b, g, rows[u]) + 8 * chunk);
#pragma unroll
                for (int u = 0; u < kGatherRounds; ++u) {
                    float xv[8];
                    widen8(raw[u], xv);
#pragma unroll
                    for (int e2 = 0; e2 < 8; ++e2) acc[e2] = fmaf(mul[u], xv[e2], acc[e2]);
                }
            }
            wave_sync_lds();
        }
    };
    // with two workgroups per head (nparts = 2, part 0 or 1), the TPW-tile
    // groups alternate between them: wave w of workgroup p takes groups
    // 2 w + p, 2 w + p + 2 NW, ..., so each compute unit serves half of the
    // head's stash and V loads even when one round would cover every tile
    const bool multi = nvis > TPW * NW * nparts;   // some wave takes more than one round of tiles
    for (int k0 = (w * nparts + part) * TPW; k0 < nvis; k0 += TPW * NW * nparts) {
        const int kv = k0 + sub;
        const bool active = kv < nvis;
        const VisitRec rec = vis[active ? kv : k0];
        const int start = rec.t * T;
        float e[EPL2];
        // whole slice, unconditionally: pass 1 writes every tile in full,
        // with 0 past the sequence end
        load_stash<EPL2>(stash + (size_t)((bh >> stash_shift) << stash_shift) * max_nt * T + start + gl * EPL2, e);
        float run = 0.f;
#pragma unroll
        for (int qq = 0; qq < EPL2; ++qq) {
            run += e[qq];
            e[qq] = run;                                   // in-lane inclusive prefix
        }
        const float gincl = group_incl_scan<LPT>(run);
        float excl = dpp_f<kWaveShr1, 0xF>(0.f, gincl);   // sum of the earlier lanes of the group
        if (gl == 0) excl = 0.f;
        // x_j = P_j a + b for the lane's tokens: e_j a + (excl a + b), monotone
        // in the lane; across lanes a running max keeps the counts monotone
        const float bl = fmaf(excl, rec.a, rec.b);
        const int lo = rec.first, hi = rec.first + rec.cnt;
        const float fhi = (float)hi;
        // count reached at the lane's last token: systematic, the closed
        // form; stratified / i.i.d., a bisection over the tile's thresholds
        // at the CDF position P a + b
        const ListCount lcnt{thr, S, sampler == kSamplerStrat};
        const int yl = list ? count_in_range(lcnt, (double)fmaf(e[EPL2 - 1], rec.a, bl), lo, hi)
                            : max((int)fminf(ceilf(fmaf(e[EPL2 - 1], rec.a, bl)), fhi), lo);
        const int gmax = group_incl_max<LPT>(yl);
        int prev = dpp_i<kWaveShr1, 0xF>(0, gmax);        // count reached by the earlier lanes
        if (gl == 0) prev = lo;
        // Thresholds prev .. yl-1 fall on the lane's tokens.  A step can fall
        // on a token of zero weight only through fp32 rounding across lanes
        // (a threshold within ~1e-7 of that token's CDF position); past the
        // sequence end such a token is replaced by the last one, so every
        // row read is inside the request.
        if constexpr (!LIST) {
            // Systematic: y_q = min(ceil(P_q a + b), hi) is nondecreasing
            // along the lane (P_q is a prefix of nonnegative weights, a >= 0,
            // and fma, ceil and min are monotone), so token q steps exactly
            // when y_q > z_q = max(prev, y_{q-1}) (z_0 = prev), and its
            // marker sits at z_q with multiplicity y_q - z_q.  The lanes
            // that step (a few per tile) put their prefixes into the wave's
            // LDS slots; the wave then evaluates SPP such lanes per pass, one
            // token per thread, instead of every lane walking its EPL2
            // tokens.
            constexpr int SPP = kWave / EPL2;
            const bool steps = active && yl > prev;
            const unsigned long long smask = __ballot(steps);
            const int nstep = __popcll(smask);
            const int rank = __builtin_amdgcn_mbcnt_hi((unsigned)(smask >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((unsigned)smask, 0u));
            const int q = lane % EPL2;
            for (int base = 0; base < nstep; base += kStepSlots) {
                const int sl = rank - base;
                if (steps && sl >= 0 && sl < kStepSlots) {
#pragma unroll
                    for (int q4 = 0; q4 < EPL2; q4 += 4)
                        *reinterpret_cast<float4 *>(&stepP[w][sl][q4]) = make_float4(e[q4], e[q4 + 1], e[q4 + 2], e[q4 + 3]);
                    stepM[w][sl] = make_float4(bl, rec.a, fhi, __int_as_float(prev));
                    stepRow[w][sl] = start + gl * EPL2;
                }
                wave_sync_lds();
                const int cnt = min(nstep - base, kStepSlots);
                for (int p0 = 0; p0 < cnt; p0 += SPP) {
                    const int s2 = p0 + lane / EPL2;
                    const int sc = s2 < cnt ? s2 : 0;
                    const float4 m = stepM[w][sc];
                    const int y = (int)fminf(ceilf(fmaf(stepP[w][sc][q], m.y, m.x)), m.z);
                    const int pv = __float_as_int(m.w);
                    const int ym1 = dpp_i<kRowShr1, 0xF>(0, y);  // y_{q-1}: same slot for q >= 1
                    const int z = q == 0 ? pv : max(pv, ym1);
                    if (s2 < cnt && y > z) {
                        jsel[z] = min(stepRow[w][sc] + q, n - 1);
                        jmul[z] = y - z;
                    }
                }
                wave_sync_lds();
            }
        } else if (active && yl > prev) {
            // stratified / i.i.d.: merge of the lane's tokens with its
            // thresholds.  The next threshold is kept in a register as the
            // largest float at or below it: for a float F, thr < F exactly
            // when that float is < F, so the test is the fp64 one.  A token
            // past it reaches clamp(#{thr < F}, yp + 1, yl): one closed-form
            // count (stratified) or one bisection (i.i.d.) per token that
            // holds thresholds, however many it holds.
            int yp = prev;
            float nxt = float_at_or_below(thr[yp]);         // yp < yl <= S here
#pragma unroll
            for (int qq = 0; qq < EPL2; ++qq) {
                const float Fq = fmaf(e[qq], rec.a, bl);
                if (nxt < Fq) {
                    const int y = count_in_range(lcnt, (double)Fq, yp + 1, yl);
                    jsel[yp] = min(start + gl * EPL2 + qq, n - 1);
                    jmul[yp] = y - yp;
                    yp = y;
                    nxt = yp < yl ? float_at_or_below(thr[yp]) : INFINITY;
                }
            }
        }
        // rare: the fp32 tile total is short of the tile's last threshold
        // (the count at the group's last lane, gmax there, is below hi);
        // thresholds gmax .. hi-1 go to the last token whose weight moved P
        const bool short_tile = active && gl == LPT - 1 && gmax < hi;
        if (__builtin_expect(__ballot(short_tile) != 0, 0)) {
            // the lane's tokens that moved P, as bits: one
            // register, where per-token candidate indices were hoisted out
            // of the tile loop by the compiler and spilled
            unsigned moved = 0;
#pragma unroll
            for (int qq = 0; qq < EPL2; ++qq) moved |= (e[qq] > (qq ? e[qq - 1] : 0.f) ? 1u : 0u) << qq;
            int lz = moved ? gl * EPL2 + 31 - __clz(moved) : -1;
            lz = group_incl_max<LPT>(lz);
            if (short_tile) {
                jsel[gmax] = start + max(lz, 0);
                jmul[gmax] = hi - gmax;
            }
        }
        // the wave's threshold range [m0, m1): from its first tile's first
        // threshold to its last active tile's end
        const int m0 = __shfl(lo, 0);
        const int m1 = wave_max(active ? hi : 0);
        wave_sync_lds();
        if (sample_idx) {
            // each position takes the row of the nearest marker at or before
            // it (a running max over marker positions; m0 always holds one)
            int carry = m0;
            for (int c = m0; c < m1; c += kWave) {
                const int m = c + lane;
                int pm = (m < m1 && jsel[m] >= 0) ? m : -1;
                pm = max(wave_incl_max_scan(pm, lane), carry);
                if (m < m1) sample_idx[(size_t)bh * S + m] = jsel[pm];
                carry = __builtin_amdgcn_readlane(pm, 63);
            }
        }
        if (!multi) gather_range(m0, m1);
    }
    if (multi) {
        // more than one round of tiles per wave: the gather waits for every
        // marker and then reads all of them in one round, 64 positions per
        // wave at a time, instead of one V round trip per round of tiles
        __syncthreads();
        for (int c = w * kWave; c < S; c += NW * kWave) gather_range(c, min(c + kWave, S));
    }
    // One workgroup per head, or one tile group in all (the second
    // workgroup then has none): the first stores the head's output.
    // Otherwise both add their halves into the output row that pass 1
    // zeroed: two addends onto zero give the same sum in either order.
    const bool alone = nparts == 1 || nvis <= TPW;
    if (!alone || part == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[e] += __shfl_xor(acc[e], 16);
            acc[e] += __shfl_xor(acc[e], 32);
        }
        if (lane < 16) {
#pragma unroll
            for (int e = 0; e < 8; ++e) red[w][8 * chunk + e] = acc[e];
        }
        __syncthreads();
        if (tid < kHeadDim) {
            float sum = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) sum += red[ww][tid];
            // divide by S: for a power of two this is an exact exponent shift
            const bool pow2 = (S & (S - 1)) == 0;
            const float r = pow2 ? sum * (1.0f / (float)S) : sum / (float)S;
            if (alone) out[(size_t)bh * kHeadDim + tid] = r;
            else atomicAdd(out + (size_t)bh * kHeadDim + tid, r);
        }
    }
}

// dynamic LDS of sample_head: the threshold list (list generators), the
// visit list, the marker arrays and, above kRegisterTiles tiles, the LDS
// reducer's per-tile arrays
inline size_t prop_sample_lds_bytes(int kcap, int S, int sampler, int max_nt) {
    const size_t thr = sampler == kSamplerSys ? 0 : (size_t)threshold_slots(S, sampler) * sizeof(double);
    const size_t red = max_nt > kRegisterTiles ? 8 + (size_t)max_nt * (2 * sizeof(double) + sizeof(float2) + sizeof(int)) : 0;
    return thr + (size_t)kcap * sizeof(VisitRec) + 2 * (size_t)S * sizeof(int) + red;
}

}  // namespace santa
