// santa_dispatch.cpp -- the launches of one decode call, by KV storage type
// (the per-type launchers are compiled separately from the kernel sources).
#include "santa_launch.h"

namespace santa {

#define SANTA_KV_SWITCH(F)                                         \
    switch (a.kv_dtype) {                                          \
        case kKvBf16: return F<uint16_t>(a, hook);                 \
        case kKvFp8: return F<uint8_t>(a, hook);                   \
        case kKvF32: return F<float>(a, hook);                     \
        default: return hipErrorInvalidValue;                      \
    }

static hipError_t launch_pass1(const LaunchArgs &a, const TimingHook &hook) { SANTA_KV_SWITCH(launch_prop_pass1_kv) }
static hipError_t launch_sample(const LaunchArgs &a, const TimingHook &hook) { SANTA_KV_SWITCH(launch_prop_sample_kv) }

// prop: pass 1, then the per-head reducer + pass 2.  With few heads each
// head's pass 2 is split over two workgroups,
// so that a head with more visited tiles than one round of 16 waves takes
// them in one round on two compute units; pass 1 then zeroes the output rows
// that the two add into.
hipError_t launch_prop(const LaunchArgs &a0, const TimingHook &hook) {
    LaunchArgs a = a0;
    const int split_heads = a.sampler == kSamplerSys ? kSampleSplitHeads : kSampleListSplitHeads;
    a.sample_parts = a.batch * a.num_q_heads <= split_heads ? 2 : 1;
    const hipError_t e = launch_pass1(a, hook);
    if (e != hipSuccess) return e;
    return launch_sample(a, hook);
}

hipError_t launch_prop_bernoulli(const LaunchArgs &a0, const TimingHook &hook) {
    LaunchArgs a = a0;
    a.sample_parts = a.batch * a.num_q_heads <= kSampleSplitHeads ? 2 : 1;
    const hipError_t e = launch_bernoulli_pass1(a, hook);
    if (e != hipSuccess) return e;
    return launch_sample(a, hook);
}

hipError_t launch_prop_fused(const LaunchArgs &a, const TimingHook &hook) { SANTA_KV_SWITCH(launch_prop_fused_kv) }
hipError_t launch_flash(const LaunchArgs &a, const TimingHook &hook) { SANTA_KV_SWITCH(launch_flash_kv) }
hipError_t launch_exact(const LaunchArgs &a, const TimingHook &hook) { SANTA_KV_SWITCH(launch_exact_kv) }

}  // namespace santa
