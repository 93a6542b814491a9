// santa_kernels.hip -- gfx950 kernels of libsanta and their launchers.
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
// Precision plan (why the index parity with an fp64 oracle holds): scores
// are accumulated unscaled (bf16 products are exact in fp32; fp32 inputs use
// fp64), the tile max is subtracted before the scale is applied, the reducer
// works in fp64, and the local CDF targets of pass 2 are formed in fp64.
#include "santa_launch.h"
#include "santa_score.h"

namespace santa {

// ===================================================================
// S2ANTA-prop, pass 1: scores, tile max, tile partition function, stash
// ===================================================================
// grid: B * Hkv * max_nt workgroups (tile fastest); block: 256 threads.
// stash [B, Hq, max_seq_len] fp32: e_j = exp(scale * (x_j - m_t))
// stats [B, Hq, max_nt] float2: (m_t unscaled tile max, Z_t = sum_j e_j)
template <typename KV, int G, int T>
__global__ __launch_bounds__(kBlock) void prop_pass1_kernel(
    const KV *__restrict__ q, const KV *__restrict__ k, KVLayout L, const int *__restrict__ seq_lens,
    int num_q_heads, int max_nt, float scale, float *__restrict__ stash, float2 *__restrict__ stats) {
    typedef typename KVTraits<KV>::acc_t acc_t;
    constexpr int HPL = HeadsPerLane<G>::value;
    constexpr int NI = T / 64;
    const int tile = blockIdx.x % max_nt;
    const int bg = blockIdx.x / max_nt;
    const int b = bg / L.num_kv_heads, g = bg - b * L.num_kv_heads;
    const int n = seq_len_of(seq_lens, L.max_seq_len, b);
    const int t0 = tile * T;
    if (t0 >= n) return;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = lane & 3, r = lane >> 2;

    QFrag<KV, G> qf;
    load_qfrag<KV, G>(qf, q + ((size_t)b * num_q_heads + (size_t)g * G) * kHeadDim, c);
    acc_t x[NI][HPL];
    score_tile<KV, G, T>(k, L, b, g, t0, n, qf, x);

    __shared__ float red_m[kWavesPerBlock][4 * HPL];
    __shared__ float red_z[kWavesPerBlock][4 * HPL];
    float mt[HPL];
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) {
        acc_t m = x[0][hh];
#pragma unroll
        for (int i = 1; i < NI; ++i) m = x[i][hh] > m ? x[i][hh] : m;
        float mf = max_stride4((float)m);
        if (r == 0) red_m[w][c + 4 * hh] = mf;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) {
        float m = red_m[0][c + 4 * hh];
#pragma unroll
        for (int ww = 1; ww < kWavesPerBlock; ++ww) m = fmaxf(m, red_m[ww][c + 4 * hh]);
        mt[hh] = m;
    }

    const acc_t c2 = (acc_t)scale * (acc_t)1.4426950408889634;   // scale * log2(e)
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) {
        const int hl = c + 4 * hh;                      // head within the group
        const bool head_ok = hl < G;
        float zsum = 0.f;
        float *srow = stash + ((size_t)b * num_q_heads + (size_t)g * G + (head_ok ? hl : 0)) *
                                  (size_t)L.max_seq_len;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row = t0 + 64 * i + 16 * w + r;
            float e = 0.f;
            if (head_ok && row < n) {
                e = exp2f((float)((x[i][hh] - (acc_t)mt[hh]) * c2));
                srow[row] = e;
            }
            zsum += e;
        }
        zsum = sum_stride4(zsum);
        if (r == 0) red_z[w][c + 4 * hh] = zsum;
    }
    __syncthreads();
    if (threadIdx.x < 4 * HPL) {
        const int hl = threadIdx.x;                      // c + 4 hh with r == 0, w == 0
        if (hl < G) {
            float z = red_z[0][hl];
#pragma unroll
            for (int ww = 1; ww < kWavesPerBlock; ++ww) z += red_z[ww][hl];
            const int hh = hl >> 2;
            (void)hh;
            float m = red_m[0][hl];
#pragma unroll
            for (int ww = 1; ww < kWavesPerBlock; ++ww) m = fmaxf(m, red_m[ww][hl]);
            stats[((size_t)b * num_q_heads + (size_t)g * G + hl) * max_nt + tile] = make_float2(m, z);
        }
    }
}

// ===================================================================
// S2ANTA-prop, reducer: one wave per (request, q head)
// ===================================================================
// From the n_t tile statistics it forms the global max M, the tile masses
// z_t = Z_t e^{scale (m_t - M)}, Z = sum z_t, the tile CDF C_t (fp64,
// C_{n_t-1} := 1) and the number of thresholds below each C_t,
//   cnt_t = #{m : U + m/S < C_t},  S_t = cnt_t - cnt_{t-1}.
// Tiles with S_t > 0 are written, in tile order, to a compact visit list
// with what pass 2 needs: first threshold index, S_t, C_{t-1} and the factor
// r_t = e^{scale (m_t - M)} / Z that maps the tile's stash prefix to CDF units.
struct VisitRec {
    int t, first, cnt, pad;
    double cprev, r;
};

__global__ __launch_bounds__(64) void prop_reduce_kernel(
    const float2 *__restrict__ stats, const int *__restrict__ seq_lens, int max_seq_len, int T,
    int max_nt, int kmax, int S, const float *__restrict__ u, float scale, VisitRec *__restrict__ vis,
    int *__restrict__ vis_count, int *__restrict__ tile_budget, int *__restrict__ counters,
    int *__restrict__ sample_idx, int num_q_heads) {
    const int bh = blockIdx.x;
    const int b = bh / num_q_heads;
    const int lane = threadIdx.x;
    const int n = seq_len_of(seq_lens, max_seq_len, b);
    const int nt = (n + T - 1) / T;
    if (lane == 0) counters[bh] = 0;
    if (nt == 0) {
        if (lane == 0) vis_count[bh] = 0;
        if (tile_budget)
            for (int t = lane; t < max_nt; t += 64) tile_budget[(size_t)bh * max_nt + t] = 0;
        if (sample_idx)
            for (int m = lane; m < S; m += 64) sample_idx[(size_t)bh * S + m] = -1;
        return;
    }
    const float2 *st = stats + (size_t)bh * max_nt;
    const int CH = (nt + 63) / 64;
    const int tb = lane * CH, te = min(nt, tb + CH);
    const double U = (double)u[bh];
    const double dscale = (double)scale;

    // global max of the (unscaled) tile maxima
    float Mf = -INFINITY;
    for (int t = tb; t < te; ++t) Mf = fmaxf(Mf, st[t].x);
    Mf = wave_max(Mf);
    const double M = (double)Mf;

    // phase A: lane totals of z_t, wave scan -> exclusive offsets, Z
    double lsum = 0.0;
    for (int t = tb; t < te; ++t) {
        const float2 s = st[t];
        lsum += (double)s.y * exp(((double)s.x - M) * dscale);
    }
    const double incl = wave_incl_scan(lsum, lane);
    double excl = __shfl_up(incl, 1);
    if (lane == 0) excl = 0.0;
    const double Z = __shfl(incl, 63);
    const double invZ = 1.0 / Z;

    // phase B: C at each lane's last tile; monotone threshold counts
    double c_last = (excl + lsum) / Z;
    if (te == nt && tb < te) c_last = 1.0;
    const int cnt_last_raw = (tb < te) ? thresholds_below(c_last, U, S) : 0;
    const int cnt_last_incl = wave_incl_max_scan(cnt_last_raw, lane);
    int cnt_pred = __shfl_up(cnt_last_incl, 1);
    double c_pred = __shfl_up(c_last, 1);
    if (lane == 0) {
        cnt_pred = 0;
        c_pred = 0.0;
    }

    // phase C: visited tiles per lane
    // (C is always formed as (excl + lane-local running sum) / Z, the same
    //  expression as c_last, so neighbouring lanes agree on shared edges)
    int nvis = 0;
    {
        double lrun = 0.0;
        int cp = cnt_pred;
        for (int t = tb; t < te; ++t) {
            const float2 s = st[t];
            lrun += (double)s.y * exp(((double)s.x - M) * dscale);
            const double C = (t == nt - 1) ? 1.0 : (excl + lrun) / Z;
            const int cnt = max(cp, thresholds_below(C, U, S));
            nvis += (cnt > cp);
            cp = cnt;
        }
    }
    const int vincl = wave_incl_scan(nvis, lane);
    int vpos = vincl - nvis;
    if (lane == 63) vis_count[bh] = vincl;

    // phase D: write visit records and budgets
    {
        double lrun = 0.0;
        double cprev = c_pred;
        int cp = cnt_pred;
        for (int t = tb; t < te; ++t) {
            const float2 s = st[t];
            const double f = exp(((double)s.x - M) * dscale);
            lrun += (double)s.y * f;
            const double C = (t == nt - 1) ? 1.0 : (excl + lrun) / Z;
            const int cnt = max(cp, thresholds_below(C, U, S));
            const int St = cnt - cp;
            if (tile_budget) tile_budget[(size_t)bh * max_nt + t] = St;
            if (St > 0 && vpos < kmax) {
                VisitRec rec;
                rec.t = t;
                rec.first = cp;
                rec.cnt = St;
                rec.pad = 0;
                rec.cprev = cprev;
                rec.r = f * invZ;
                vis[(size_t)bh * kmax + vpos] = rec;
                ++vpos;
            }
            cp = cnt;
            cprev = C;
        }
    }
    if (tile_budget)
        for (int t = nt + lane; t < max_nt; t += 64) tile_budget[(size_t)bh * max_nt + t] = 0;
}

// ===================================================================
// S2ANTA-prop, pass 2: per visited tile, scan the stash, invert the CDF at
// the tile's thresholds, gather and sum those V rows; merge per head.
// ===================================================================
// grid: B * Hq * nwg workgroups of 4 waves; the 4*nwg waves of a head take
// the visited tiles round-robin.  Each wave keeps its running V sum in
// registers (16 lanes per row, 8 elements per lane, 4 row slots), writes it
// to `part`, and the last workgroup of the head to finish adds the wave
// partials in wave order and scales by 1/S.
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
__device__ __forceinline__ void load_v8<float>(const float *p, float (&v)[8]) {
    const u32x4 a = reinterpret_cast<const u32x4 *>(p)[0];
    const u32x4 c = reinterpret_cast<const u32x4 *>(p)[1];
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(c.x); v[5] = __uint_as_float(c.y);
    v[6] = __uint_as_float(c.z); v[7] = __uint_as_float(c.w);
}

// first j in [0, len) with P[j] > tau, or len
__device__ __forceinline__ int upper_index(const float *P, int len, double tau) {
    int lo = 0, hi = len;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((double)P[mid] > tau) hi = mid;
        else lo = mid + 1;
    }
    return lo;
}

// Scan the tile's values e[0..len) held EPL per lane (lane-major) into P
// (inclusive prefix, fp32) in LDS; returns the last index with e > 0.
template <int T>
__device__ __forceinline__ int scan_tile_to_lds(float (&e)[T / 64], int len, float *P, int lane) {
    constexpr int EPL = T / 64;
    int lz = -1;
    float run = 0.f;
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
        const int j = lane * EPL + q;
        if (j < len && e[q] > 0.f) lz = j;
        run += e[q];
        e[q] = run;
    }
    const float incl = wave_incl_scan(run, lane);
    float excl = __shfl_up(incl, 1);
    if (lane == 0) excl = 0.f;
#pragma unroll
    for (int q = 0; q < EPL; ++q) P[lane * EPL + q] = excl + e[q];
    wave_sync_lds();
    return wave_max(lz);
}

// Gather-and-add the V rows J (one per active lane, nact <= 64 lanes) of
// (b, g), tile base `start`, into acc (16 lanes per row, 4 row slots).
template <typename KV>
__device__ __forceinline__ void gather_rows(const KV *__restrict__ v, const KVLayout &L, int b, int g,
                                            int start, int J, int nact, int lane, float (&acc)[8]) {
    const int slot = lane >> 4, chunk = lane & 15;
#pragma unroll 4
    for (int rr = 0; rr < 16; ++rr) {
        const int src = 4 * rr + slot;
        const int Jr = __shfl(J, src);
        if (4 * rr >= nact) break;
        if (src < nact) {
            float x[8];
            load_v8<KV>(v + row_offset(L, b, g, start + Jr) + 8 * chunk, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += x[e];
        }
    }
}

template <typename KV, int T>
__global__ __launch_bounds__(kBlock) void prop_pass2_kernel(
    const KV *__restrict__ v, KVLayout L, const int *__restrict__ seq_lens, int num_q_heads, int G,
    int S, const float *__restrict__ u, const float *__restrict__ stash,
    const VisitRec *__restrict__ vis, const int *__restrict__ vis_count, int kmax, int nwg,
    float *__restrict__ part, int *__restrict__ counters, float *__restrict__ out,
    int *__restrict__ sample_idx) {
    constexpr int EPL = T / 64;
    const int bh = blockIdx.x / nwg;
    const int s = blockIdx.x - bh * nwg;
    const int b = bh / num_q_heads, h = bh - b * num_q_heads, g = h / G;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int NW = nwg * kWavesPerBlock;
    const int wh = s * kWavesPerBlock + w;
    const int n = seq_len_of(seq_lens, L.max_seq_len, b);
    const int count = vis_count[bh];
    const double U = (double)u[bh];
    const double dS = (double)S;

    __shared__ float P[kWavesPerBlock][T];
    __shared__ int ticket;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;

    for (int kv = wh; kv < count; kv += NW) {
        const VisitRec rec = vis[(size_t)bh * kmax + kv];
        const int start = rec.t * T;
        const int len = min(T, n - start);
        const float *st = stash + (size_t)bh * L.max_seq_len + start;
        float e[EPL];
#pragma unroll
        for (int qq = 0; qq < EPL; ++qq) {
            const int j = lane * EPL + qq;
            e[qq] = j < len ? st[j] : 0.f;
        }
        const int lz = scan_tile_to_lds<T>(e, len, P[w], lane);
        for (int base = 0; base < rec.cnt; base += 64) {
            const int kk = base + lane;
            const int nact = min(64, rec.cnt - base);
            int J = 0;
            if (kk < rec.cnt) {
                const int m = rec.first + kk;
                const double tm = U + (double)m / dS;
                const double tau = (tm - rec.cprev) / rec.r;
                J = upper_index(P[w], len, tau);
                if (J >= len) J = lz;
                J = J < 0 ? 0 : J;
                if (sample_idx) sample_idx[(size_t)bh * S + m] = start + J;
            }
            gather_rows<KV>(v, L, b, g, start, J, nact, lane, acc);
        }
        wave_sync_lds();
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        acc[e] += __shfl_xor(acc[e], 16);
        acc[e] += __shfl_xor(acc[e], 32);
    }
    if (lane < 16) {
        float *dst = part + ((size_t)bh * NW + wh) * kHeadDim + 8 * lane;
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = acc[e];
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) ticket = atomicAdd(&counters[bh], 1);
    __syncthreads();
    if (ticket != nwg - 1) return;
    __threadfence();
    if (threadIdx.x < kHeadDim) {
        const float *src = part + (size_t)bh * NW * kHeadDim + threadIdx.x;
        float sum = 0.f;
        for (int ww = 0; ww < NW; ++ww) sum += __builtin_nontemporal_load(src + (size_t)ww * kHeadDim);
        // divide by S: for a power of two this is an exact exponent shift
        const bool pow2 = (S & (S - 1)) == 0;
        out[(size_t)bh * kHeadDim + threadIdx.x] = pow2 ? sum * (1.0f / (float)S) : sum / (float)S;
    }
}

// ===================================================================
// S2ANTA-flash: tile kernel (score, local softmax, S_f local samples,
// gather) and merge
// ===================================================================
// part_m / part_z [B, Hq, nt] (unscaled tile max, local partition function)
// part_o [B, Hq, nt, d]: mean of the tile's S_f sampled V rows
template <typename KV, int G, int T>
__global__ __launch_bounds__(kBlock) void flash_tile_kernel(
    const KV *__restrict__ q, const KV *__restrict__ k, const KV *__restrict__ v, KVLayout L,
    int num_q_heads, int nt, int Sf, int S, float scale, const float *__restrict__ u,
    float *__restrict__ part_m, float *__restrict__ part_z, float *__restrict__ part_o,
    int *__restrict__ sample_idx) {
    typedef typename KVTraits<KV>::acc_t acc_t;
    constexpr int HPL = HeadsPerLane<G>::value;
    constexpr int NI = T / 64;
    constexpr int EPL = T / 64;
    const int tile = blockIdx.x % nt;
    const int bg = blockIdx.x / nt;
    const int b = bg / L.num_kv_heads, g = bg - b * L.num_kv_heads;
    const int n = L.max_seq_len;
    const int t0 = tile * T;
    const int len = min(T, n - t0);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = lane & 3, r = lane >> 2;

    QFrag<KV, G> qf;
    load_qfrag<KV, G>(qf, q + ((size_t)b * num_q_heads + (size_t)g * G) * kHeadDim, c);
    acc_t x[NI][HPL];
    score_tile<KV, G, T>(k, L, b, g, t0, n, qf, x);

    __shared__ float red_m[kWavesPerBlock][4 * HPL];
    __shared__ float E[G][T];
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) {
        acc_t m = x[0][hh];
#pragma unroll
        for (int i = 1; i < NI; ++i) m = x[i][hh] > m ? x[i][hh] : m;
        float mf = max_stride4((float)m);
        if (r == 0) red_m[w][c + 4 * hh] = mf;
    }
    __syncthreads();
    const acc_t c2 = (acc_t)scale * (acc_t)1.4426950408889634;
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) {
        const int hl = c + 4 * hh;
        if (hl < G) {
            float m = red_m[0][hl];
#pragma unroll
            for (int ww = 1; ww < kWavesPerBlock; ++ww) m = fmaxf(m, red_m[ww][hl]);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int row = 64 * i + 16 * w + r;
                E[hl][row] = (t0 + row < n) ? exp2f((float)((x[i][hh] - (acc_t)m) * c2)) : 0.f;
            }
        }
    }
    __syncthreads();

    const double dSf = (double)Sf;
    for (int hl = w; hl < G; hl += kWavesPerBlock) {
        const int bh = b * num_q_heads + g * G + hl;
        float e[EPL];
#pragma unroll
        for (int qq = 0; qq < EPL; ++qq) e[qq] = E[hl][lane * EPL + qq];
        wave_sync_lds();
        const int lz = scan_tile_to_lds<T>(e, len, E[hl], lane);
        const float Zt = E[hl][len - 1];
        const double uf = (double)u[bh] * (double)nt;
        float acc[8];
#pragma unroll
        for (int ee = 0; ee < 8; ++ee) acc[ee] = 0.f;
        for (int base = 0; base < Sf; base += 64) {
            const int kk = base + lane;
            const int nact = min(64, Sf - base);
            int J = 0;
            if (kk < Sf) {
                const double tau = (uf + (double)kk / dSf) * (double)Zt;
                J = upper_index(E[hl], len, tau);
                if (J >= len) J = lz;
                J = J < 0 ? 0 : J;
                if (sample_idx) sample_idx[(size_t)bh * S + (size_t)tile * Sf + kk] = t0 + J;
            }
            gather_rows<KV>(v, L, b, g, t0, J, nact, lane, acc);
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

// Merge of per-tile (m_t, mass_t, o_t) triples: out = sum_t w_t o_t / norm,
// w_t = e^{scale (m_t - M)} * coef_t.  For flash coef_t = Z_t and norm =
// sum_t w_t (weights by true tile mass); for the exact decode coef_t = 1,
// o_t holds unnormalised sums and norm = sum_t w_t l_t.
// grid: B * Hq blocks of 128 threads (one output element each); dynamic
// shared memory holds the nt fp64 weights.
__global__ __launch_bounds__(128) void merge_tiles_kernel(
    const float *__restrict__ part_m, const float *__restrict__ part_l, const float *__restrict__ part_o,
    const int *__restrict__ seq_lens, int max_seq_len, int T, int nt_stride, int num_q_heads,
    int flash, float scale, float *__restrict__ out) {
    const int bh = blockIdx.x;
    const int b = bh / num_q_heads;
    const int tid = threadIdx.x;
    const int n = seq_len_of(seq_lens, max_seq_len, b);
    const int nt = (n + T - 1) / T;
    extern __shared__ double wts[];     // [nt_stride]
    __shared__ double sh[2];
    const float *pm = part_m + (size_t)bh * nt_stride;
    const float *pl = part_l + (size_t)bh * nt_stride;
    if (nt == 0) {
        out[(size_t)bh * kHeadDim + tid] = 0.f;
        return;
    }
    // global max
    float mloc = -INFINITY;
    for (int t = tid; t < nt; t += 128) mloc = fmaxf(mloc, pm[t]);
    mloc = wave_max(mloc);
    __shared__ float wm[2];
    if ((tid & 63) == 0) wm[tid >> 6] = mloc;
    __syncthreads();
    const double M = (double)fmaxf(wm[0], wm[1]);
    const double dscale = (double)scale;
    double nloc = 0.0;
    for (int t = tid; t < nt; t += 128) {
        const double f = exp(((double)pm[t] - M) * dscale);
        const double wt = flash ? f * (double)pl[t] : f;
        wts[t] = wt;
        nloc += flash ? wt : wt * (double)pl[t];
    }
    // fixed-order block reduction of the normaliser
    for (int o = 1; o < 64; o <<= 1) nloc += __shfl_xor(nloc, o);
    if ((tid & 63) == 0) sh[tid >> 6] = nloc;
    __syncthreads();
    const double norm = sh[0] + sh[1];
    const double inv = 1.0 / norm;
    double acc = 0.0;
    const float *po = part_o + (size_t)bh * nt_stride * kHeadDim + tid;
    for (int t = 0; t < nt; ++t) acc += wts[t] * (double)po[(size_t)t * kHeadDim];
    out[(size_t)bh * kHeadDim + tid] = (float)(acc * inv);
}

// ===================================================================
// Exact split-KV decode: per tile (m_t, l_t, o_t = sum_j p_j V_j)
// ===================================================================
template <typename KV, int G, int T>
__global__ __launch_bounds__(kBlock) void exact_partial_kernel(
    const KV *__restrict__ q, const KV *__restrict__ k, const KV *__restrict__ v, KVLayout L,
    const int *__restrict__ seq_lens, int num_q_heads, int max_nt, float scale,
    float *__restrict__ part_m, float *__restrict__ part_l, float *__restrict__ part_o) {
    typedef typename KVTraits<KV>::acc_t acc_t;
    constexpr int HPL = HeadsPerLane<G>::value;
    constexpr int NI = T / 64;
    const int tile = blockIdx.x % max_nt;
    const int bg = blockIdx.x / max_nt;
    const int b = bg / L.num_kv_heads, g = bg - b * L.num_kv_heads;
    const int n = seq_len_of(seq_lens, L.max_seq_len, b);
    const int t0 = tile * T;
    if (t0 >= n) return;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = lane & 3, r = lane >> 2;

    QFrag<KV, G> qf;
    load_qfrag<KV, G>(qf, q + ((size_t)b * num_q_heads + (size_t)g * G) * kHeadDim, c);
    acc_t x[NI][HPL];
    score_tile<KV, G, T>(k, L, b, g, t0, n, qf, x);

    __shared__ float red_m[kWavesPerBlock][4 * HPL];
    __shared__ float red_l[kWavesPerBlock][4 * HPL];
    __shared__ float Pw[G][T];
    __shared__ float red_o[kWavesPerBlock][G][kHeadDim];
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) {
        acc_t m = x[0][hh];
#pragma unroll
        for (int i = 1; i < NI; ++i) m = x[i][hh] > m ? x[i][hh] : m;
        float mf = max_stride4((float)m);
        if (r == 0) red_m[w][c + 4 * hh] = mf;
    }
    __syncthreads();
    const acc_t c2 = (acc_t)scale * (acc_t)1.4426950408889634;
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) {
        const int hl = c + 4 * hh;
        float lsum = 0.f;
        if (hl < G) {
            float m = red_m[0][hl];
#pragma unroll
            for (int ww = 1; ww < kWavesPerBlock; ++ww) m = fmaxf(m, red_m[ww][hl]);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int row = 64 * i + 16 * w + r;
                const float p = (t0 + row < n) ? exp2f((float)((x[i][hh] - (acc_t)m) * c2)) : 0.f;
                Pw[hl][row] = p;
                lsum += p;
            }
        }
        lsum = sum_stride4(lsum);
        if (r == 0) red_l[w][c + 4 * hh] = lsum;
    }
    __syncthreads();

    // V pass: 16 lanes per row (8 elements each), 4 rows per wave step,
    // 16 consecutive rows per block step
    const int slot = lane >> 4, chunk = lane & 15;
    float acc[G][8];
#pragma unroll
    for (int hl = 0; hl < G; ++hl)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hl][e] = 0.f;
#pragma unroll 4
    for (int i2 = 0; i2 < T / 16; ++i2) {
        const int row = 16 * i2 + 4 * w + slot;
        if (t0 + row < n) {
            float xv[8];
            load_v8<KV>(v + row_offset(L, b, g, t0 + row) + 8 * chunk, xv);
#pragma unroll
            for (int hl = 0; hl < G; ++hl) {
                const float p = Pw[hl][row];
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
template <typename KV, int G, int T>
static hipError_t launch_prop_t(const LaunchArgs &a, const TimingHook &hook) {
    const int max_nt = a.max_nt;
    hipStream_t st = (hipStream_t)a.stream;
    float *stash = (float *)a.ws.stash;
    float2 *stats = (float2 *)a.ws.stats;
    const KVLayout L{a.num_kv_heads, a.max_seq_len, a.page_size, a.page_table, a.max_pages};
    if (hook.begin) hipEventRecord((hipEvent_t)hook.begin, st);
    hipLaunchKernelGGL((prop_pass1_kernel<KV, G, T>), dim3((unsigned)(a.batch * a.num_kv_heads * max_nt)),
                       dim3(kBlock), 0, st, (const KV *)a.q, (const KV *)a.k, L, a.seq_lens,
                       a.num_q_heads, max_nt, a.scale, stash, stats);
    if (hook.end) hipEventRecord((hipEvent_t)hook.end, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int BH = a.batch * a.num_q_heads;
    hipLaunchKernelGGL(prop_reduce_kernel, dim3((unsigned)BH), dim3(64), 0, st, stats, a.seq_lens,
                       a.max_seq_len, T, max_nt, a.kmax, a.S, a.u, a.scale, (VisitRec *)a.ws.vis,
                       (int *)a.ws.vis_count, a.tile_budget, (int *)a.ws.counters, a.sample_idx,
                       a.num_q_heads);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prop_pass2_kernel<KV, T>), dim3((unsigned)(BH * a.nwg)), dim3(kBlock), 0, st,
                       (const KV *)a.v, L, a.seq_lens, a.num_q_heads, G, a.S, a.u, stash,
                       (const VisitRec *)a.ws.vis, (const int *)a.ws.vis_count, a.kmax, a.nwg,
                       (float *)a.ws.part, (int *)a.ws.counters, a.out, a.sample_idx);
    return hipGetLastError();
}

template <typename KV, int G, int T>
static hipError_t launch_flash_t(const LaunchArgs &a, const TimingHook &hook) {
    hipStream_t st = (hipStream_t)a.stream;
    const KVLayout L{a.num_kv_heads, a.max_seq_len, a.page_size, a.page_table, a.max_pages};
    const int nt = a.max_nt;
    if (hook.begin) hipEventRecord((hipEvent_t)hook.begin, st);
    hipLaunchKernelGGL((flash_tile_kernel<KV, G, T>), dim3((unsigned)(a.batch * a.num_kv_heads * nt)),
                       dim3(kBlock), 0, st, (const KV *)a.q, (const KV *)a.k, (const KV *)a.v, L,
                       a.num_q_heads, nt, a.S / nt, a.S, a.scale, a.u, (float *)a.ws.part_m,
                       (float *)a.ws.part_l, (float *)a.ws.part_o, a.sample_idx);
    if (hook.end) hipEventRecord((hipEvent_t)hook.end, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(merge_tiles_kernel, dim3((unsigned)(a.batch * a.num_q_heads)), dim3(128),
                       sizeof(double) * (size_t)nt, st, (const float *)a.ws.part_m,
                       (const float *)a.ws.part_l, (const float *)a.ws.part_o, (const int *)nullptr,
                       a.max_seq_len, T, nt, a.num_q_heads, 1, a.scale, a.out);
    return hipGetLastError();
}

template <typename KV, int G, int T>
static hipError_t launch_exact_t(const LaunchArgs &a, const TimingHook &hook) {
    hipStream_t st = (hipStream_t)a.stream;
    const KVLayout L{a.num_kv_heads, a.max_seq_len, a.page_size, a.page_table, a.max_pages};
    const int max_nt = a.max_nt;
    if (hook.begin) hipEventRecord((hipEvent_t)hook.begin, st);
    hipLaunchKernelGGL((exact_partial_kernel<KV, G, T>),
                       dim3((unsigned)(a.batch * a.num_kv_heads * max_nt)), dim3(kBlock), 0, st,
                       (const KV *)a.q, (const KV *)a.k, (const KV *)a.v, L, a.seq_lens, a.num_q_heads,
                       max_nt, a.scale, (float *)a.ws.part_m, (float *)a.ws.part_l, (float *)a.ws.part_o);
    if (hook.end) hipEventRecord((hipEvent_t)hook.end, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(merge_tiles_kernel, dim3((unsigned)(a.batch * a.num_q_heads)), dim3(128),
                       sizeof(double) * (size_t)max_nt, st, (const float *)a.ws.part_m,
                       (const float *)a.ws.part_l, (const float *)a.ws.part_o, a.seq_lens,
                       a.max_seq_len, T, max_nt, a.num_q_heads, 0, a.scale, a.out);
    return hipGetLastError();
}

// dispatch over (dtype, group, tile length)
#define SANTA_T_CASES(KV, G, FN)                        \
    switch (a.tile_len) {                               \
        case 64: return FN<KV, G, 64>(a, hook);         \
        case 128: return FN<KV, G, 128>(a, hook);       \
        case 256: return FN<KV, G, 256>(a, hook);       \
        case 512: return FN<KV, G, 512>(a, hook);       \
        case 1024: return FN<KV, G, 1024>(a, hook);     \
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
#define SANTA_DISPATCH(FN)                                          \
    if (a.bf16) { SANTA_G_CASES(uint16_t, FN) }                     \
    else { SANTA_G_CASES(float, FN) }

hipError_t launch_prop(const LaunchArgs &a, const TimingHook &hook) { SANTA_DISPATCH(launch_prop_t) }
hipError_t launch_flash(const LaunchArgs &a, const TimingHook &hook) { SANTA_DISPATCH(launch_flash_t) }
hipError_t launch_exact(const LaunchArgs &a, const TimingHook &hook) { SANTA_DISPATCH(launch_exact_t) }

size_t visit_record_bytes() { return sizeof(VisitRec); }

}  // namespace santa
