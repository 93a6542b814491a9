// santa_device.h -- device helpers shared by the gfx950 kernels of libsanta.
//
// Wave64 throughout.  Cross-lane traffic inside a 4-lane quad uses DPP
// quad permutes; wider exchanges use ds_bpermute (__shfl*).
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
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

// Element offset of row j of request b / KV head g.  PAGED (the layout of
// the kernel's instantiation, page_size != 0): row j % page_size of page
// page_table[b][j / page_size]; else the contiguous [B, Hkv, max_seq_len, d]
// cache.  A compile-time choice, so that a kernel carries only its own
// layout's address code.
template <bool PAGED>
__device__ __forceinline__ size_t row_offset(const KVLayout &L, int b, int g, int j) {
    if constexpr (PAGED) {
        const int page = L.page_table[(size_t)b * L.max_pages + j / L.page_size];
        return (((size_t)page * L.num_kv_heads + g) * L.page_size + (j % L.page_size)) * kHeadDim;
    } else {
        return (((size_t)b * L.num_kv_heads + g) * L.max_seq_len + j) * kHeadDim;
    }
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

// ---------------------------------------------------------------- fp8
// OCP e4m3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
// infinities).  The gfx950 conversion decodes it exactly, and every e4m3
// value is exact in bf16, so widening to bf16 keeps the value.
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// bf16 pair (lo, hi) from two exactly representable floats: their high halves
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
// two e4m3 bytes (the low or the high half of w) -> a bf16 pair
template <bool HIGH>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16(uint32_t w) {
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HIGH);
    return pack_bf16_exact(a.x, a.y);
}
// four e4m3 bytes -> four floats
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float *f) {
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
}

// storage type of the query for a KV storage type: fp8 KV keeps bf16 queries
template <typename KV> struct QOf { typedef KV type; };
template <> struct QOf<uint8_t> { typedef uint16_t type; };

// ---------------------------------------------------------------- DPP
// quad_perm control words
constexpr int kQuadXor1 = 0xB1;   // [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // [2,3,0,1]

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// row_ror:n rotates within each row of 16 lanes
template <int N>
__device__ __forceinline__ float row_ror(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}
// sum / max over the 16 lanes of a DPP row; every lane of the row gets it
__device__ __forceinline__ float row16_sum(float v) {
    v += row_ror<8>(v);
    v += row_ror<4>(v);
    v += row_ror<2>(v);
    v += row_ror<1>(v);
    return v;
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, row_ror<8>(v));
    v = fmaxf(v, row_ror<4>(v));
    v = fmaxf(v, row_ror<2>(v));
    v = fmaxf(v, row_ror<1>(v));
    return v;
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
// Reductions over the 16 lanes that share (lane & 3): strides 4 and 8
// inside a row by DPP rotation, then across the 4 rows.
__device__ __forceinline__ float sum_stride4(float v) {
    v += row_ror<8>(v);
    v += row_ror<4>(v);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}
__device__ __forceinline__ float max_stride4(float v) {
    v = fmaxf(v, row_ror<8>(v));
    v = fmaxf(v, row_ror<4>(v));
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// ---------------------------------------------------------------- DPP wave scans
// Inclusive scans over the 64 lanes with DPP only (no LDS round trips):
// row_shr 1, 2, 4, 8 scan each row of 16 lanes, then row_bcast:15 (rows 1
// and 3 add the total of the row before) and row_bcast:31 (rows 2 and 3
// add the total of rows 0-1).  Lanes with no DPP source keep the identity.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp_i(int ident, int v) {
    return __builtin_amdgcn_update_dpp(ident, v, CTRL, ROWMASK, 0xF, false);
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_f(float ident, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(ident), __float_as_int(v), CTRL, ROWMASK,
                                                      0xF, false));
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_d(double ident, double v) {
    const long long iv = __double_as_longlong(v), ii = __double_as_longlong(ident);
    const int lo = __builtin_amdgcn_update_dpp((int)ii, (int)iv, CTRL, ROWMASK, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(ii >> 32), (int)(iv >> 32), CTRL, ROWMASK, 0xF, false);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
// whole-wave shift by one lane (lane l reads lane l-1; lane 0 keeps the
// identity): a DPP control the GFX9-family parts, gfx950 among them, keep
constexpr int kWaveShr1 = 0x138;

__device__ __forceinline__ float wave_incl_scan(float v, int /*lane*/) {
    v += dpp_f<kRowShr1, 0xF>(0.f, v);
    v += dpp_f<kRowShr2, 0xF>(0.f, v);
    v += dpp_f<kRowShr4, 0xF>(0.f, v);
    v += dpp_f<kRowShr8, 0xF>(0.f, v);
    v += dpp_f<kRowBcast15, 0xA>(0.f, v);
    v += dpp_f<kRowBcast31, 0xC>(0.f, v);
    return v;
}
__device__ __forceinline__ double wave_incl_scan(double v, int /*lane*/) {
    v += dpp_d<kRowShr1, 0xF>(0.0, v);
    v += dpp_d<kRowShr2, 0xF>(0.0, v);
    v += dpp_d<kRowShr4, 0xF>(0.0, v);
    v += dpp_d<kRowShr8, 0xF>(0.0, v);
    v += dpp_d<kRowBcast15, 0xA>(0.0, v);
    v += dpp_d<kRowBcast31, 0xC>(0.0, v);
    return v;
}
__device__ __forceinline__ int wave_incl_scan(int v, int /*lane*/) {
    v += dpp_i<kRowShr1, 0xF>(0, v);
    v += dpp_i<kRowShr2, 0xF>(0, v);
    v += dpp_i<kRowShr4, 0xF>(0, v);
    v += dpp_i<kRowShr8, 0xF>(0, v);
    v += dpp_i<kRowBcast15, 0xA>(0, v);
    v += dpp_i<kRowBcast31, 0xC>(0, v);
    return v;
}
// running maximum of ints >= 0 (identity 0 ... callers pass non-negative values)
__device__ __forceinline__ int wave_incl_max_scan(int v, int /*lane*/) {
    v = max(v, dpp_i<kRowShr1, 0xF>(INT_MIN, v));
    v = max(v, dpp_i<kRowShr2, 0xF>(INT_MIN, v));
    v = max(v, dpp_i<kRowShr4, 0xF>(INT_MIN, v));
    v = max(v, dpp_i<kRowShr8, 0xF>(INT_MIN, v));
    v = max(v, dpp_i<kRowBcast15, 0xA>(INT_MIN, v));
    v = max(v, dpp_i<kRowBcast31, 0xC>(INT_MIN, v));
    return v;
}
__device__ __forceinline__ float wave_incl_max_scan(float v) {
    v = fmaxf(v, dpp_f<kRowShr1, 0xF>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kRowShr2, 0xF>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kRowShr4, 0xF>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kRowShr8, 0xF>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kRowBcast15, 0xA>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kRowBcast31, 0xC>(-INFINITY, v));
    return v;
}

// Inclusive scans over groups of LPT consecutive lanes (LPT = 16, 32 or 64):
// the row steps, then the row_bcast steps that stay inside a group.
template <int LPT>
__device__ __forceinline__ float group_incl_scan(float v) {
    v += dpp_f<kRowShr1, 0xF>(0.f, v);
    v += dpp_f<kRowShr2, 0xF>(0.f, v);
    v += dpp_f<kRowShr4, 0xF>(0.f, v);
    v += dpp_f<kRowShr8, 0xF>(0.f, v);
    if (LPT >= 32) v += dpp_f<kRowBcast15, 0xA>(0.f, v);
    if (LPT >= 64) v += dpp_f<kRowBcast31, 0xC>(0.f, v);
    return v;
}
template <int LPT>
__device__ __forceinline__ int group_incl_max(int v) {
    v = max(v, dpp_i<kRowShr1, 0xF>(INT_MIN, v));
    v = max(v, dpp_i<kRowShr2, 0xF>(INT_MIN, v));
    v = max(v, dpp_i<kRowShr4, 0xF>(INT_MIN, v));
    v = max(v, dpp_i<kRowShr8, 0xF>(INT_MIN, v));
    if (LPT >= 32) v = max(v, dpp_i<kRowBcast15, 0xA>(INT_MIN, v));
    if (LPT >= 64) v = max(v, dpp_i<kRowBcast31, 0xC>(INT_MIN, v));
    return v;
}

// wave-wide maximum, returned to every lane (lane 63 of the scan holds it)
__device__ __forceinline__ float wave_max(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_incl_max_scan(v)), 63));
}
__device__ __forceinline__ int wave_max(int v) {
    return __builtin_amdgcn_readlane(wave_incl_max_scan(v, 0), 63);
}


__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The systematic offset U is meant to lie in [0, 1/S).  Any other value is
// clamped into [0, u_max], u_max the largest float below 1/S (NaN and -0
// become +0), so that threshold m stays in [m/S, (m+1)/S) and all S
// thresholds lie below 1: every position of the index list is written and
// the budgets sum to S whatever the caller passes.
__device__ __forceinline__ double clamp_offset(float U, int S) {
    const double inv = 1.0 / (double)S;
    float umax = (float)inv;                      // nearest float to 1/S
    if ((double)umax >= inv) umax = __uint_as_float(__float_as_uint(umax) - 1u);
    float x = U > 0.f ? U : 0.f;
    x = x < umax ? x : umax;
    return (double)x;
}

// count of thresholds t_m = U + m/S (m = 0..S-1) strictly below x:
// #{m >= 0 : m < (x - U) S} = ceil((x - U) S), clamped to [0, S]
// (branch-free; a NaN position counts as 0)
__device__ __forceinline__ int thresholds_below(double x, double U, int S) {
    const double c = ceil((x - U) * (double)S);
    return (int)fmin(fmax(c, 0.0), (double)S);
}

}  // namespace santa
