// santa_static.hip -- santa_decode_prop_static: S2ANTA-prop for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  It is santa_decode_prop with its
// workspace (the exp-score stash and the tile statistics) taken from a
// file-scope device array instead of the caller.
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends.  Host code never passes the array's name
// to a kernel or a copy: the name is a host-side stand-in, and only the
// per-device address from hipGetSymbolAddress is a device pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/santa.h"

namespace {
constexpr size_t kScratchBytes = (size_t)SANTA_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
}  // namespace

// the workspace of every santa_decode_prop_static call on this GPU
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::once_flag g_once[kMaxDevices];
void *g_scratch[kMaxDevices];          // device address of `scratch`, per device
hipError_t g_status[kMaxDevices];

// the array's address on the current device, looked up once per device
// with that device current
int scratch_of_current_device(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SANTA_ERR_HIP;
    std::call_once(g_once[dev], [dev] {
        void *p = nullptr;
        g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch[dev] = p;
    });
    if (g_status[dev] != hipSuccess || !g_scratch[dev]) return SANTA_ERR_HIP;
    *ptr = g_scratch[dev];
    return SANTA_OK;
}
}  // namespace

extern "C" {

int santa_decode_prop_static(const santa_problem *p, const void *q, const void *k, const void *v, int32_t S,
                             const float *u, float *out, int32_t *sample_idx, int32_t *tile_budget,
                             void *stream) {
    size_t need = 0;
    const int st = santa_workspace_size(p, SANTA_VARIANT_PROP, S, &need);
    if (st != SANTA_OK) return st;
    if (need > kScratchBytes) return SANTA_ERR_TOO_LARGE;     // nothing launched
    void *ws = nullptr;
    const int sc = scratch_of_current_device(&ws);
    if (sc != SANTA_OK) return sc;
    // prop writes every stash and statistics entry it reads, so nothing in
    // the array has to start at zero, whatever an earlier call left there
    return santa_decode_prop(p, q, k, v, S, u, out, sample_idx, tile_budget, ws, kScratchBytes, stream);
}

}  // extern "C"
