// santa_bernoulli.hip -- Bernoulli qK^T scoring as pass 1 of S2ANTA-prop.
//
// The method follows the web page "Stochastic Sparse Attention for
// Memory-Bound Inference" (ICML 2026 paper notes on SANTA), key design 4 and
// the ablation table's mean group query.  The query is scaled into [-1, 1] by
// a = max_i |q_i|; each of `draws` ternary draws keeps feature i with
// probability |q_i| / a and the sign of q_i (kept when fl32(u * a) < |q_i|);
// with c_i the sum of the draws, (a / draws) * sum_i c_i K_{j,i} estimates
// <q, K_j> without bias.  Only features with c_i != 0 are read, so K is taken
// feature-major, [B, Hkv, d, max_seq_len] (bf16, or OCP e4m3 with bf16
// queries): a kept feature of a tile is one contiguous run of T values, and a
// dropped one costs no HBM traffic.
//
// The kernel writes the stash and the tile statistics in exactly the format
// of the exact-score pass 1 (stash e_j = exp(scale * (x_j - m_t)), stats
// (m_t, Z_t) with x unscaled), so the reducer and pass 2 run unchanged; with
// the mean query the G equal stash rows of a group are written once.
#include "santa_kernels.h"

namespace santa {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// wave-wide sum in a fixed order, returned to every lane
__device__ __forceinline__ float wave_total(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_incl_scan(v, 0)), 63));
}

// 4 consecutive keys of one feature: 8 bytes of bf16 or 4 of e4m3
template <typename KV> struct Chunk4;
template <> struct Chunk4<uint16_t> { typedef u32x2 type; };
template <> struct Chunk4<uint8_t> { typedef uint32_t type; };

__device__ __forceinline__ void widen4(u32x2 r, float (&k)[4]) {
    k[0] = bf16_lo(r.x); k[1] = bf16_hi(r.x); k[2] = bf16_lo(r.y); k[3] = bf16_hi(r.y);
}
__device__ __forceinline__ void widen4(uint32_t r, float (&k)[4]) { e4m3x4_to_f32(r, k); }

// grid: B * Hkv * max_nt workgroups (tile fastest); block: 256 threads.
//   q   [B, Hq, d] bf16;  kf  [B, Hkv, d, max_seq_len] KV (max_seq_len % 4 == 0)
//   ub  [owners, draws, d] fp32 uniforms, owners = B*Hq (a query per head) or
//       B*Hkv (MEAN: one mean query per group)
//   features_read [B*Hkv] (optional): kept features of the group, written by
//       the tile-0 workgroup (also for an empty request)
template <typename KV, int G, int T, bool MEAN>
__global__ __launch_bounds__(kBlock) void bernoulli_pass1_kernel(
    const uint16_t *__restrict__ q, const KV *__restrict__ kf, int num_kv_heads, int max_seq_len,
    const int *__restrict__ seq_lens, int num_q_heads, int max_nt, float scale, int draws,
    const float *__restrict__ ub, float *__restrict__ stash, float2 *__restrict__ stats,
    int *__restrict__ features_read, float *__restrict__ zero_out) {
    constexpr int NQ = MEAN ? 1 : G;           // ternary queries of the group
    constexpr int CH = T / 4;                  // 4-token chunks in a tile's feature run
    constexpr int FP = kBlock / CH;            // feature slots working side by side
    constexpr int NE = (NQ * kHeadDim + kBlock - 1) / kBlock;   // query entries per thread
    static_assert(CH <= kBlock && kBlock % CH == 0, "tile length");

    const int tile = blockIdx.x % max_nt;
    const int bg = blockIdx.x / max_nt;
    const int b = bg / num_kv_heads, g = bg - b * num_kv_heads;
    const int n = seq_len_of(seq_lens, max_seq_len, b);
    const int t0 = tile * T;
    if (t0 >= n && tile != 0) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

    // thread (slot fs, chunk): 4 consecutive keys of the features the slot
    // streams.  Per head, the group's queries keep nearly every feature
    // between them, so each slot's first U features in natural order
    // (fs, fs + FP, ..., all below U * FP <= d) are requested before the
    // queries are known; a feature that no query keeps then has coefficient
    // 0.  With the mean query a third of the features are dropped, and none
    // is read before the list is known.
    constexpr int U = 8;                         // features in flight per thread
    constexpr bool SPEC = !MEAN;
    static_assert(U * FP <= kHeadDim, "speculative features");
    const int chunk = tid % CH, fs = tid / CH;
    const int j = t0 + 4 * chunk;
    const bool jin = j < max_seq_len;            // whole chunk in the row (max_seq_len % 4 == 0)
    const KV *kbase = kf + ((size_t)b * num_kv_heads + g) * kHeadDim * (size_t)max_seq_len + (jin ? j : 0);
    typedef typename Chunk4<KV>::type chunk_t;

    __shared__ float cq[kHeadDim][NQ];           // c_i of each query, feature-major
    __shared__ float amax[NQ][2];                // max |q_i| over each half of d
    __shared__ float red_m[NQ], red_z[NQ];
    __shared__ unsigned long long kept[2];
    __shared__ int flist[kHeadDim];              // kept features, ascending
    __shared__ __align__(16) float part[FP][NQ][T];   // per-slot partial dots, then x and e

    // ---- the ternary queries: a, then c_i = sign(q_i) * #{r : fl(u a) < |q_i|}
    // (the first RP draws' uniforms load together with the query: they do
    // not depend on a)
    // Every load is issued unconditionally, from indices clamped into range,
    // and selected afterwards, so that all of them are in flight together
    // (a load under a per-lane condition becomes a branch that waits for it).
    float qv[NE];
    constexpr int RP = 8;                        // draws whose uniforms load with the query
    constexpr int QL = MEAN ? G : 1;             // query rows read per entry
    float upre[NE][RP];
    uint16_t qraw[NE][QL];
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const int e = min(tid + k * kBlock, NQ * kHeadDim - 1);
        const int qh = e / kHeadDim, i = e % kHeadDim;
        const size_t owner = MEAN ? (size_t)b * num_kv_heads + g : (size_t)b * num_q_heads + (size_t)g * G + qh;
        const float *u = ub + owner * (size_t)draws * kHeadDim + i;
#pragma unroll
        for (int r = 0; r < RP; ++r) upre[k][r] = u[(size_t)min(r, draws - 1) * kHeadDim];
        const uint16_t *qrow = q + ((size_t)b * num_q_heads + (size_t)g * G) * kHeadDim + i;
#pragma unroll
        for (int hh = 0; hh < QL; ++hh) qraw[k][hh] = qrow[(size_t)(MEAN ? hh : qh) * kHeadDim];
    }
    // the speculative K loads go behind the query and uniforms, which the
    // prologue waits for first
    chunk_t spec[SPEC ? U : 1];
    if constexpr (SPEC) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            spec[u] = __builtin_nontemporal_load(
                reinterpret_cast<const chunk_t *>(kbase + (size_t)(fs + u * FP) * max_seq_len));
    }
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const int e = tid + k * kBlock;
        const bool ok = e < NQ * kHeadDim;
        float qf;
        if (MEAN) {
            float s = bf16_lo(qraw[k][0]);
#pragma unroll
            for (int hh = 1; hh < QL; ++hh) s = s + bf16_lo(qraw[k][hh]);
            qf = s * (1.0f / (float)G);
        } else {
            qf = bf16_lo(qraw[k][0]);
        }
        qv[k] = ok ? qf : 0.f;
#pragma unroll
        // masked with bits, not a select: a select let the compiler sink a
        // load into a branch behind the K loads, whose wait then drained them
        for (int r = 0; r < RP; ++r)
            upre[k][r] = __int_as_float(__float_as_int(upre[k][r]) & -(int)(ok && r < draws));
        // 64 consecutive entries lie in one half of one query
        const float m = wave_max(fabsf(qv[k]));
        if (lane == 0 && ok) amax[e / kHeadDim][(e % kHeadDim) / 64] = m;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const int e = tid + k * kBlock;
        if (e < NQ * kHeadDim) {
            const int qh = e / kHeadDim, i = e % kHeadDim;
            const float a = fmaxf(amax[qh][0], amax[qh][1]);
            const size_t owner = MEAN ? (size_t)b * num_kv_heads + g
                                      : (size_t)b * num_q_heads + (size_t)g * G + qh;
            const float *u = ub + owner * (size_t)draws * kHeadDim + i;
            const float mag = fabsf(qv[k]);
            int kept_draws = 0;
#pragma unroll
            for (int r = 0; r < RP; ++r)
                if (r < draws) kept_draws += (upre[k][r] * a < mag) ? 1 : 0;
            for (int r = RP; r < draws; ++r) kept_draws += (u[(size_t)r * kHeadDim] * a < mag) ? 1 : 0;
            const int c = qv[k] > 0.f ? kept_draws : (qv[k] < 0.f ? -kept_draws : 0);
            cq[i][qh] = (float)c;
        }
    }
    __syncthreads();
    // the group's read set: features kept by any of its queries, compacted
    if (w < 2) {
        const int i = tid;
        bool any = false;
#pragma unroll
        for (int qh = 0; qh < NQ; ++qh) any |= cq[i][qh] != 0.f;
        const unsigned long long mask = __ballot(any);
        if (lane == 0) kept[w] = mask;
    }
    __syncthreads();
    const unsigned long long k0 = kept[0], k1 = kept[1];
    const int m = __popcll(k0) + __popcll(k1);
    if (w < 2) {
        const unsigned long long mine = w == 0 ? k0 : k1;
        if ((mine >> lane) & 1ull) {
            const int pos = (w == 0 ? 0 : __popcll(k0)) + __popcll(mine & ((1ull << lane) - 1ull));
            flist[pos] = tid;
        }
    }
    if (tile == 0 && tid == 0 && features_read) features_read[(size_t)b * num_kv_heads + g] = m;
    __syncthreads();
    if (t0 >= n) return;   // empty request: only its read count is written

    // ---- stream the kept features: slot fs takes list entries fs, fs+FP, ...
    float acc[NQ][4];
#pragma unroll
    for (int qh = 0; qh < NQ; ++qh)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[qh][e] = 0.f;
    int kstart = 0;                              // list entries already added
    if constexpr (SPEC) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int f = fs + u * FP;
            float kv[4];
            widen4(jin ? spec[u] : chunk_t{}, kv);
#pragma unroll
            for (int qh = 0; qh < NQ; ++qh) {
                const float c = cq[f][qh];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[qh][e] = fmaf(c, kv[e], acc[qh][e]);
            }
        }
        // the list then continues with the kept features from U * FP on
        constexpr int NF = U * FP;
        if constexpr (NF >= 128) kstart = m;
        else if constexpr (NF > 64) kstart = __popcll(k0) + __popcll(k1 & ((1ull << (NF - 64)) - 1ull));
        else if constexpr (NF == 64) kstart = __popcll(k0);
        else kstart = __popcll(k0 & ((1ull << NF) - 1ull));
    }
    for (int kk = kstart + fs; kk < m; kk += U * FP) {
        chunk_t raw[U];
        int fi[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = kk + u * FP;
            fi[u] = k < m ? flist[k] : -1;
            raw[u] = chunk_t{};
            if (fi[u] >= 0 && jin)
                raw[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const chunk_t *>(kbase + (size_t)fi[u] * max_seq_len));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (fi[u] < 0) continue;
            float kv[4];
            widen4(raw[u], kv);
#pragma unroll
            for (int qh = 0; qh < NQ; ++qh) {
                const float c = cq[fi[u]][qh];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[qh][e] = fmaf(c, kv[e], acc[qh][e]);
            }
        }
    }
#pragma unroll
    for (int qh = 0; qh < NQ; ++qh)
        *reinterpret_cast<float4 *>(&part[fs][qh][4 * chunk]) =
            make_float4(acc[qh][0], acc[qh][1], acc[qh][2], acc[qh][3]);
    __syncthreads();

    // ---- scores x = (a / draws) * sum over slots (fixed order); -inf past the end
    for (int e = tid; e < NQ * T; e += kBlock) {
        const int qh = e / T, jj = e % T;
        float s = part[0][qh][jj];
#pragma unroll
        for (int f = 1; f < FP; ++f) s += part[f][qh][jj];
        const float a = fmaxf(amax[qh][0], amax[qh][1]);
        part[0][qh][jj] = (t0 + jj < n) ? (a / (float)draws) * s : -INFINITY;
    }
    __syncthreads();
    // tile max and partition function of each query: one wave per query
    const float c2 = scale * 1.4426950408889634f;   // scale * log2(e)
    for (int qh = w; qh < NQ; qh += kWavesPerBlock) {
        float mx = -INFINITY;
        for (int jj = lane; jj < T; jj += 64) mx = fmaxf(mx, part[0][qh][jj]);
        mx = wave_max(mx);
        float z = 0.f;
        for (int jj = lane; jj < T; jj += 64) {
            const float x = part[0][qh][jj];
            const float ev = (t0 + jj < n) ? exp_weight(x, mx, c2) : 0.f;
            part[0][qh][jj] = ev;
            z += ev;
        }
        z = wave_total(z);
        if (lane == 0) {
            red_m[qh] = mx;
            red_z[qh] = z;
        }
    }
    __syncthreads();
    // stash rows: one per head, or with the mean query one per group (the
    // group's first head's row, which the sampler reads for all its heads);
    // stats for every head
    for (int hl = w; hl < (MEAN ? 1 : G); hl += kWavesPerBlock) {
        const int qh = MEAN ? 0 : hl;
        float *srow = stash + ((size_t)b * num_q_heads + (size_t)g * G + hl) * ((size_t)max_nt * T) + t0;
        for (int j4 = 4 * lane; j4 < T; j4 += 256)
            *reinterpret_cast<float4 *>(srow + j4) = *reinterpret_cast<const float4 *>(&part[0][qh][j4]);
    }
    if (tid < G) {
        const int qh = MEAN ? 0 : tid;
        stats[((size_t)b * num_q_heads + (size_t)g * G + tid) * max_nt + tile] = make_float2(red_m[qh], red_z[qh]);
    }
    // when the sampling kernel adds two workgroups' halves into out, the
    // group's tile-0 workgroup zeroes the group's output rows (last, off the
    // path of its loads; an empty request's rows are written by the sampler)
    if (zero_out && tile == 0)
        for (int i = tid; i < G * kHeadDim; i += kBlock)
            zero_out[((size_t)b * num_q_heads + (size_t)g * G) * kHeadDim + i] = 0.f;
}

template <typename KV, int G, int T, bool MEAN>
static hipError_t launch_bern_t(const LaunchArgs &a, const TimingHook &hook) {
    hipStream_t st = (hipStream_t)a.stream;
    const dim3 grid((unsigned)(a.batch * a.num_kv_heads * a.max_nt));
    if (hook.begin)
        hipExtLaunchKernelGGL((bernoulli_pass1_kernel<KV, G, T, MEAN>), grid, dim3(kBlock), 0, st,
                              (hipEvent_t)hook.begin, (hipEvent_t)hook.end, 0, (const uint16_t *)a.q,
                              (const KV *)a.k, a.num_kv_heads, a.max_seq_len, a.seq_lens, a.num_q_heads,
                              a.max_nt, a.scale, a.draws, a.u_bern, (float *)a.ws.stash, (float2 *)a.ws.stats,
                              a.features_read, a.sample_parts > 1 ? a.out : nullptr);
    else
        hipLaunchKernelGGL((bernoulli_pass1_kernel<KV, G, T, MEAN>), grid, dim3(kBlock), 0, st, (const uint16_t *)a.q,
                           (const KV *)a.k, a.num_kv_heads, a.max_seq_len, a.seq_lens, a.num_q_heads,
                           a.max_nt, a.scale, a.draws, a.u_bern, (float *)a.ws.stash, (float2 *)a.ws.stats,
                           a.features_read, a.sample_parts > 1 ? a.out : nullptr);
    return hipGetLastError();
}

template <typename KV, int G, int T>
static hipError_t launch_bern_m(const LaunchArgs &a, const TimingHook &hook) {
    return a.group_mean ? launch_bern_t<KV, G, T, true>(a, hook) : launch_bern_t<KV, G, T, false>(a, hook);
}

template <typename KV, int G>
static hipError_t launch_bern_g(const LaunchArgs &a, const TimingHook &hook) {
    switch (a.tile_len) {
        case 64: return launch_bern_m<KV, G, 64>(a, hook);
        case 128: return launch_bern_m<KV, G, 128>(a, hook);
        case 256: return launch_bern_m<KV, G, 256>(a, hook);
        case 512: return launch_bern_m<KV, G, 512>(a, hook);
        case 1024: return launch_bern_m<KV, G, 1024>(a, hook);
        default: return hipErrorInvalidValue;
    }
}

template <typename KV>
static hipError_t launch_bern_kv(const LaunchArgs &a, const TimingHook &hook) {
    switch (a.group) {
        case 1: return launch_bern_g<KV, 1>(a, hook);
        case 2: return launch_bern_g<KV, 2>(a, hook);
        case 4: return launch_bern_g<KV, 4>(a, hook);
        case 8: return launch_bern_g<KV, 8>(a, hook);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bernoulli_pass1(const LaunchArgs &a, const TimingHook &hook) {
    switch (a.kv_dtype) {
        case kKvBf16: return launch_bern_kv<uint16_t>(a, hook);
        case kKvFp8: return launch_bern_kv<uint8_t>(a, hook);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace santa
