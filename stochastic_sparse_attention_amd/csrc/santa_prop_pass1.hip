// santa_prop_pass1.hip -- S2ANTA-prop, pass 1: scores, tile max, tile
// partition function and the exponentiated-score stash (the kernel; its body
// is in santa_prop_body.h, the reducer and pass 2 in santa_prop.hip, and
// santa_dispatch.cpp launches the step).
//
// The method follows the web page "Stochastic Sparse Attention for
// Memory-Bound Inference" (ICML 2026 paper notes on SANTA), key design 2:
// pass 1 scores every tile and stashes its exp-scores with the tile
// partition function.
#include "santa_prop_body.h"

namespace santa {

template <typename KV, int G, int T, bool PAGED>
__global__ __launch_bounds__(kBlock) void prop_pass1_kernel(
    const typename QOf<KV>::type *__restrict__ q, const KV *__restrict__ k, KVLayout L, const int *__restrict__ seq_lens,
    int num_q_heads, int max_nt, float scale, float *__restrict__ stash, float2 *__restrict__ stats,
    float *__restrict__ zero_out) {
    int tile, b, g;
    tile_of_block<PAGED>(L, max_nt, tile, b, g);
    const int n = seq_len_of(seq_lens, L.max_seq_len, b);
    if (tile * T >= n) return;
    pass1_tile<KV, G, T, PAGED>(q, k, L, n, num_q_heads, max_nt, scale, stash, stats, tile, b, g);
    // when the sampling kernel adds two workgroups' halves into out, the
    // group's tile-0 workgroup zeroes the group's output rows (last, off the
    // path of its loads; an empty request's rows are written by the sampler)
    if (zero_out && tile == 0)
        for (int i = threadIdx.x; i < G * kHeadDim; i += kBlock)
            zero_out[((size_t)b * num_q_heads + (size_t)g * G) * kHeadDim + i] = 0.f;
}

template <typename KV, int G, int T, bool PAGED>
static hipError_t launch_pass1_t(const LaunchArgs &a, const TimingHook &hook) {
    const int max_nt = a.max_nt;
    hipStream_t st = (hipStream_t)a.stream;
    float *stash = (float *)a.ws.stash;
    float2 *stats = (float2 *)a.ws.stats;
    const KVLayout L = layout_of(a);
    float *zero_out = a.sample_parts > 1 ? a.out : nullptr;
    // with a timing hook the dispatch itself records the two events, so
    // they bracket the kernel's execution and nothing else
    if (hook.begin)
        hipExtLaunchKernelGGL((prop_pass1_kernel<KV, G, T, PAGED>), dim3((unsigned)(a.batch * a.num_kv_heads * max_nt)), dim3(kBlock), 0, st, (hipEvent_t)hook.begin, (hipEvent_t)hook.end, 0,
                       (const typename QOf<KV>::type *)a.q, (const KV *)a.k, L, a.seq_lens, a.num_q_heads, max_nt, a.scale,
                       stash, stats, zero_out);
    else
        hipLaunchKernelGGL((prop_pass1_kernel<KV, G, T, PAGED>), dim3((unsigned)(a.batch * a.num_kv_heads * max_nt)), dim3(kBlock), 0, st,
                       (const typename QOf<KV>::type *)a.q, (const KV *)a.k, L, a.seq_lens, a.num_q_heads, max_nt, a.scale,
                       stash, stats, zero_out);
    return hipGetLastError();
}

template <typename KV>
hipError_t launch_prop_pass1_kv(const LaunchArgs &a, const TimingHook &hook) { SANTA_G_CASES(KV, launch_pass1_t) }
SANTA_INSTANTIATE(launch_prop_pass1_kv)

}  // namespace santa
