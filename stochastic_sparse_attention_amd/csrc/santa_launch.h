// santa_launch.h -- host-side interface between the C ABI (santa_api.cpp)
// and the kernel launchers (santa_prop.hip, santa_flash.hip, santa_exact.hip).
// Internal to libsanta.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace santa {

// KV storage types (the values of santa_dtype)
constexpr int kKvF32 = 0, kKvBf16 = 1, kKvFp8 = 2;

// threshold generators of prop (the values of santa_sampler)
constexpr int kSamplerSys = 0, kSamplerStrat = 1, kSamplerIid = 2;

// LDS slots of a head's threshold list: S, or the next power of two for
// the i.i.d. generator, whose uniforms are sorted with a bitonic network
__host__ __device__ inline int threshold_slots(int S, int sampler) {
    if (sampler != kSamplerIid) return S;
    int p = 1;
    while (p < S) p <<= 1;
    return p;
}

// Arrival counters of the single-launch prop: the first kSyncBytes of every
// workspace, one counter per (request, KV group) every kSyncStride words;
// zero before the first call, and every call leaves them zero.
constexpr int kSyncStride = 16;                        // 64 bytes apart
constexpr size_t kSyncBytes = 64 * 1024;
constexpr int kMaxSyncGroups = (int)(kSyncBytes / (kSyncStride * 4));

// Carved workspace regions (device pointers; unused ones are null).
struct Workspace {
    void *sync;       // every variant: [kMaxSyncGroups * kSyncStride] uint32 (the single-launch prop's counters)
    void *stash;      // prop: [B, Hq, max_nt * T] fp32
    void *stats;      // prop: [B, Hq, max_nt] float2
    void *part_m;     // flash/exact: [B, Hq, max_nt] fp32
    void *part_l;     // flash/exact: [B, Hq, max_nt] fp32
    void *part_o;     // flash/exact: [B, Hq, max_nt, d] fp32
};

struct LaunchArgs {
    int batch, num_q_heads, num_kv_heads, group;
    int max_seq_len, max_nt, tile_len;
    const int *seq_lens;
    int page_size;
    const int *page_table;
    int max_pages;
    int kv_dtype;   // kKvF32 / kKvBf16 / kKvFp8 (q is bf16 for fp8 KV)
    float scale;
    const void *q, *k, *v;
    int S;
    const float *u;
    float *out;
    int *sample_idx;
    int *tile_budget;
    int kmax;   // prop: visit-list capacity per head
    int sampler;   // prop: kSamplerSys / kSamplerStrat / kSamplerIid
    // prop on Bernoulli scores: k is feature-major [B, Hkv, d, max_seq_len]
    int draws;            // ternary draws per query
    int group_mean;       // 1: one mean query per KV group
    const float *u_bern;  // [B*Hq or B*Hkv, draws, d] uniforms
    int *features_read;   // [B*Hkv] or null
    int stash_shift;      // prop: 1 << stash_shift consecutive heads share one stash row
    int sample_parts;     // prop: workgroups per head in the sampling kernel (0 or 1: one;
                          // 2: two, and pass 1 zeroes out, which both add into)
    Workspace ws;
    void *stream;
};

struct TimingHook {
    void *begin;
    void *end;
};

// Up to this many q heads per call, prop's sampling kernel gives each head
// two workgroups: systematic thresholds, at most two 16-wave workgroups per
// compute unit (they fit together); stratified and i.i.d. thresholds, whose
// workgroups take a whole compute unit, at most one.  The output of a head
// can differ in its last bits between calls above and below this count
// (the two halves are added in another order).
constexpr int kSampleSplitHeads = 256;
constexpr int kSampleListSplitHeads = 128;

// One decode call: the launches for a.kv_dtype (santa_dispatch.cpp).
hipError_t launch_prop(const LaunchArgs &a, const TimingHook &hook);
hipError_t launch_flash(const LaunchArgs &a, const TimingHook &hook);
hipError_t launch_exact(const LaunchArgs &a, const TimingHook &hook);
// prop with Bernoulli qK^T scores (bf16, contiguous): its pass 1, then the
// same reducer + pass 2 as launch_prop
hipError_t launch_prop_bernoulli(const LaunchArgs &a, const TimingHook &hook);
// prop in one launch (pass 1, then the reducer and pass 2 in each group's
// last workgroup)
hipError_t launch_prop_fused(const LaunchArgs &a, const TimingHook &hook);
hipError_t launch_bernoulli_pass1(const LaunchArgs &a, const TimingHook &hook);

// The launchers per KV storage type (uint16_t bf16, uint8_t e4m3, float).
// Each kernel source is compiled once per type, and every compilation
// instantiates only its own (SANTA_KV), so that they build in parallel.
template <typename KV> hipError_t launch_prop_pass1_kv(const LaunchArgs &a, const TimingHook &hook);
template <typename KV> hipError_t launch_prop_sample_kv(const LaunchArgs &a, const TimingHook &hook);
template <typename KV> hipError_t launch_flash_kv(const LaunchArgs &a, const TimingHook &hook);
template <typename KV> hipError_t launch_exact_kv(const LaunchArgs &a, const TimingHook &hook);
template <typename KV> hipError_t launch_prop_fused_kv(const LaunchArgs &a, const TimingHook &hook);

}  // namespace santa
