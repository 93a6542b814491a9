// santa_prop_fused.hip -- S2ANTA-prop in a single launch: every workgroup runs
// pass 1 of its tile, and the last workgroup of each KV group to finish runs
// the reducer and pass 2 of the group's heads (the bodies are those of the
// two-launch path, santa_prop_body.h).
//
// The method follows the web page "Stochastic Sparse Attention for
// Memory-Bound Inference" (ICML 2026 paper notes on SANTA), key design 2: the
// only step between the passes is a global reduction over the n_t tile
// statistics.  Here it is a per-group arrival count instead of a kernel
// boundary: each workgroup publishes its stash and statistics with an
// agent-scope release and increments the group's counter; the one that
// brings it to n_t acquires, resets the counter to 0 for the next call, and
// samples.  No workgroup waits for another, so the grid needs no
// co-residency.
//
// The counters live in the workspace's first SANTA_SYNC_BYTES; they must be
// zero before the first call and every call leaves them zero.
#include "santa_prop_body.h"

namespace santa {

template <typename KV, int G, int T, bool PAGED>
__global__ __launch_bounds__(kBlock) void prop_fused_kernel(
    const typename QOf<KV>::type *__restrict__ q, const KV *__restrict__ k, const KV *__restrict__ v, KVLayout L,
    const int *__restrict__ seq_lens, int num_q_heads, int max_nt, float scale, int S, int kcap,
    const float *__restrict__ u, float *__restrict__ stash, float2 *__restrict__ stats, float *__restrict__ out,
    int *__restrict__ sample_idx, int *__restrict__ tile_budget, unsigned *__restrict__ counters) {
    int tile, b, g;
    tile_of_block<PAGED>(L, max_nt, tile, b, g);
    const int n = seq_len_of(seq_lens, L.max_seq_len, b);
    const int nt = (n + T - 1) / T;
    if (nt == 0) {
        // an empty request has no tile to count: its tile-0 workgroup writes
        // the group's empty results (output 0, indices -1, budgets 0)
        if (tile == 0)
            for (int hl = 0; hl < G; ++hl)
                sample_head<KV, T, PAGED, false, kWavesPerBlock>(v, L, seq_lens, num_q_heads, G, S, max_nt, kcap,
                                                                 kSamplerSys, u, scale, stash, stats, out,
                                                                 sample_idx, tile_budget, 0, b, g, hl, 0, 1);
        return;
    }
    if (tile >= nt) return;
    pass1_tile<KV, G, T, PAGED>(q, k, L, n, num_q_heads, max_nt, scale, stash, stats, tile, b, g);

    // arrival: every thread's stash and statistics stores are ordered before
    // thread 0's release by the barrier; the release makes them visible on
    // every XCD before the count does
    __shared__ int last;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned *c = counters + (size_t)(b * L.num_kv_heads + g) * kSyncStride;
        const unsigned old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        last = old == (unsigned)nt - 1;
        if (last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last) return;
    // the group's last tile: acquire what the other workgroups published,
    // then the reducer and pass 2 of each head of the group in turn
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    for (int hl = 0; hl < G; ++hl) {
        if (hl) __syncthreads();
        sample_head<KV, T, PAGED, false, kWavesPerBlock>(v, L, seq_lens, num_q_heads, G, S, max_nt, kcap,
                                                         kSamplerSys, u, scale, stash, stats, out, sample_idx,
                                                         tile_budget, 0, b, g, hl, 0, 1);
    }
}

template <typename KV, int G, int T, bool PAGED>
static hipError_t launch_fused_t(const LaunchArgs &a, const TimingHook &hook) {
    hipStream_t st = (hipStream_t)a.stream;
    const KVLayout L = layout_of(a);
    const size_t lds = prop_sample_lds_bytes(a.kmax, a.S, kSamplerSys, a.max_nt);
    const auto kernel = prop_fused_kernel<KV, G, T, PAGED>;
    if (lds > 64 * 1024) {
        const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (ea != hipSuccess) return ea;
    }
    const dim3 grid((unsigned)(a.batch * a.num_kv_heads * a.max_nt));
    if (hook.begin)
        hipExtLaunchKernelGGL(kernel, grid, dim3(kBlock), lds, st, (hipEvent_t)hook.begin, (hipEvent_t)hook.end, 0,
                              (const typename QOf<KV>::type *)a.q, (const KV *)a.k, (const KV *)a.v, L, a.seq_lens,
                              a.num_q_heads, a.max_nt, a.scale, a.S, a.kmax, a.u, (float *)a.ws.stash,
                              (float2 *)a.ws.stats, a.out, a.sample_idx, a.tile_budget, (unsigned *)a.ws.sync);
    else
        hipLaunchKernelGGL(kernel, grid, dim3(kBlock), lds, st, (const typename QOf<KV>::type *)a.q, (const KV *)a.k,
                           (const KV *)a.v, L, a.seq_lens, a.num_q_heads, a.max_nt, a.scale, a.S, a.kmax, a.u,
                           (float *)a.ws.stash, (float2 *)a.ws.stats, a.out, a.sample_idx, a.tile_budget,
                           (unsigned *)a.ws.sync);
    return hipGetLastError();
}

template <typename KV>
hipError_t launch_prop_fused_kv(const LaunchArgs &a, const TimingHook &hook) { SANTA_G_CASES(KV, launch_fused_t) }
SANTA_INSTANTIATE(launch_prop_fused_kv)

}  // namespace santa
