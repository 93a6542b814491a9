// santa_prop.hip -- S2ANTA-prop: the per-head sampling kernel (reducer + pass
// 2, whose body is in santa_prop_body.h) and its launcher.  Pass 1 is in
// santa_prop_pass1.hip; santa_dispatch.cpp launches the two in order.
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
// fp64), the tile max is subtracted before the scale is applied, the reducer
// works in fp64, and pass 2 evaluates each CDF position as one fp32 fma
// whose coefficients were formed in fp64.
#include "santa_prop_body.h"

namespace santa {

// One workgroup per (request, q head), or two (nparts = 2): block
// part * B*Hq + bg + i * B*Hkv takes head i of the group of (request, KV
// head) bg.
template <typename KV, int T, bool PAGED, bool LIST, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(LIST ? 4 : 8))) void prop_sample_kernel(
    const KV *__restrict__ v, KVLayout L, const int *__restrict__ seq_lens, int batch, int num_q_heads,
    int G, int S, int max_nt, int kcap, int sampler, const float *__restrict__ u, float scale,
    const float *__restrict__ stash, const float2 *__restrict__ stats, float *__restrict__ out,
    int *__restrict__ sample_idx, int *__restrict__ tile_budget, int stash_shift, int nparts) {
    const int BG = batch * L.num_kv_heads, BH = batch * num_q_heads;
    const int part = blockIdx.x / BH, hb = blockIdx.x - part * BH;
    const int bg = hb % BG, hl = hb / BG;
    const int b = bg / L.num_kv_heads, g = bg - b * L.num_kv_heads;
    sample_head<KV, T, PAGED, LIST, NW>(v, L, seq_lens, num_q_heads, G, S, max_nt, kcap, sampler, u, scale, stash,
                                        stats, out, sample_idx, tile_budget, stash_shift, b, g, hl, part, nparts);
}

// ===================================================================
// launchers
// ===================================================================

template <typename KV, int G, int T, bool PAGED>
static hipError_t launch_sample_t(const LaunchArgs &a, const TimingHook &) {
    const int max_nt = a.max_nt;
    hipStream_t st = (hipStream_t)a.stream;
    float *stash = (float *)a.ws.stash;
    float2 *stats = (float2 *)a.ws.stats;
    const KVLayout L = layout_of(a);
    const int BH = a.batch * a.num_q_heads;
    const int nparts = a.sample_parts > 1 ? 2 : 1;
    const size_t lds = prop_sample_lds_bytes(a.kmax, a.S, a.sampler, max_nt);
    // few heads: 16 waves per head; many heads: 8, so that more heads (and
    // their dependent memory round trips) share each compute unit
    const bool many = BH > (a.sampler == kSamplerSys ? kSampleManyHeads : kSampleListManyHeads);
    auto launch = [&](auto kernel, int nw) -> hipError_t {
        if (lds > 64 * 1024) {
            const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (ea != hipSuccess) return ea;
        }
        hipLaunchKernelGGL(kernel, dim3((unsigned)(BH * nparts)), dim3(nw * kWave), lds, st, (const KV *)a.v, L,
                           a.seq_lens, a.batch, a.num_q_heads, G, a.S, max_nt, a.kmax, a.sampler, a.u, a.scale,
                           (const float *)stash, (const float2 *)stats, a.out, a.sample_idx, a.tile_budget,
                           a.stash_shift, nparts);
        return hipGetLastError();
    };
    if (a.sampler != kSamplerSys)
        return many ? launch(prop_sample_kernel<KV, T, PAGED, true, 8>, 8)
                    : launch(prop_sample_kernel<KV, T, PAGED, true, 16>, 16);
    if (BH > kSampleVeryManyHeads) return launch(prop_sample_kernel<KV, T, PAGED, false, 4>, 4);
    if (many) return launch(prop_sample_kernel<KV, T, PAGED, false, 8>, 8);
    return launch(prop_sample_kernel<KV, T, PAGED, false, 16>, 16);
}

template <typename KV>
hipError_t launch_prop_sample_kv(const LaunchArgs &a, const TimingHook &hook) { SANTA_G_CASES(KV, launch_sample_t) }
SANTA_INSTANTIATE(launch_prop_sample_kv)


}  // namespace santa
