// santa_device.h -- device helpers shared by the gfx950 kernels of libsanta.
//
// Wave64 throughout.  Cross-lane traffic inside a 4-lane quad uses DPP
// quad permutes; wider exchanges use ds_bpermute (__shfl*).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace santa {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kHeadDim = 128;         // the only head dimension built
constexpr int kBlock = 256;           // threads per workgroup of the streaming kernels
constexpr int kWavesPerBlock = kBlock / kWave;

// ---------------------------------------------------------------- layouts
// Where row j of request b / KV head g lives, for contiguous and paged caches.
struct KVLayout {
    int num_kv_heads;
    int max_seq_len;
    int page_size;           // 0: contiguous
    const int *page_table;   // [B, max_pages]
    int max_pages;
};

// Element offset of the first element of a 16-row block starting at row j0
// (j0 % 16 == 0); rows j0..j0+15 are contiguous in both layouts.
__device__ __forceinline__ size_t block16_offset(const KVLayout &L, int b, int g, int j0) {
    if (L.page_size == 0)
        return ((size_t)(b * L.num_kv_heads + g) * L.max_seq_len + j0) * kHeadDim;
    int page = L.page_table[(size_t)b * L.max_pages + j0 / L.page_size];
    return ((size_t)(page * L.num_kv_heads + g) * L.page_size + (j0 % L.page_size)) * kHeadDim;
}

__device__ __forceinline__ size_t row_offset(const KVLayout &L, int b, int g, int j) {
    int j0 = j & ~15;
    return block16_offset(L, b, g, j0) + (size_t)(j - j0) * kHeadDim;
}

__device__ __forceinline__ int seq_len_of(const int *seq_lens, int max_seq_len, int b) {
    if (!seq_lens) return max_seq_len;
    int n = seq_lens[b];
    return n < 0 ? 0 : (n > max_seq_len ? max_seq_len : n);
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + a.lo*b.lo + a.hi*b.hi  (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// ---------------------------------------------------------------- DPP
// quad_perm control words
constexpr int kQuadXor1 = 0xB1;   // [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // [2,3,0,1]

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// sum over the 4 lanes of a quad; every lane of the quad gets the result
__device__ __forceinline__ float quad_sum(float v) {
    v += dpp_f<kQuadXor1>(v);
    v += dpp_f<kQuadXor2>(v);
    return v;
}

__device__ __forceinline__ double quad_sum(double v) {
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    return v;
}

// ---------------------------------------------------------------- reductions
// Reductions over the 16 lanes that share (lane & 3): strides 4..32.
__device__ __forceinline__ float sum_stride4(float v) {
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}
__device__ __forceinline__ float max_stride4(float v) {
    v = fmaxf(v, __shfl_xor(v, 4));
    v = fmaxf(v, __shfl_xor(v, 8));
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

// Inclusive prefix sum over the wave (Hillis-Steele, fixed order).
__device__ __forceinline__ float wave_incl_scan(float v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        float t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}
__device__ __forceinline__ double wave_incl_scan(double v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        double t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}
__device__ __forceinline__ int wave_incl_max_scan(int v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int t = __shfl_up(v, o);
        if (lane >= o) v = max(v, t);
    }
    return v;
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// count of thresholds t_m = U + m/S (m = 0..S-1) strictly below x
__device__ __forceinline__ int thresholds_below(double x, double U, int S) {
    double c = ceil((x - U) * (double)S);
    if (!(c > 0.0)) return 0;
    if (c > (double)S) return S;
    return (int)c;
}

}  // namespace santa
