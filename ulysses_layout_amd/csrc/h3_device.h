// h3_device.h -- device-side pieces shared by the kernel translation units:
// vector types, bf16 packing, the swizzled LDS tile layout of the attention
// kernels, the transposing LDS read and the reductions across the two 32-lane
// halves of a wave.  Not part of the C ABI.
#pragma once

#include "h3_internal.h"

namespace h3 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kD = H3_HEAD_DIM;            // 128 channels per head
constexpr int kBufferWord3 = 0x00020000;   // buffer resource word 3 for raw 32-bit data on gfx9-class parts
constexpr int kSchedMfma = 0x008;          // sched_group_barrier class masks
constexpr int kSchedValu = 0x002;
constexpr int kSchedDsRead = 0x100;

// Round two floats to bf16 (nearest even) and pack them, element 0 in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 f = {lo, hi};
    bf16x2 b = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// The two bf16 values of a packed word, widened exactly to float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// LDS tiles of 128-channel bf16 rows: 16-byte chunk c of row r sits at chunk
// c ^ f(r), f(r) = 4*(r%4) + (r/4)%4, so that 16 consecutive rows read at one
// logical chunk, and the 4 rows x 4 chunks a 32-lane half reads through the
// transposing load, both hit 16 distinct chunk positions.
__device__ __forceinline__ int swz_f(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// element offset of (row r, 16-byte chunk c) inside a swizzled tile
__device__ __forceinline__ int swz(int r, int c) { return r * kD + ((c ^ swz_f(r)) << 3); }

// LDS tiles of 128-channel bf16 rows read as 16x16x32 MFMA fragments: chunk c
// of row r sits at chunk c ^ g(r), g(r) = 2*(r%8) + (r/8)%2.  The 16 rows a
// 16-lane group reads at one logical chunk, and the 8 rows x 2 chunks a
// 32-lane half reads through the transposing load, then hit distinct bank
// groups; g depends on r%16 only, so row blocks of 16 are immediate offsets.
__device__ __forceinline__ int tile16_f(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int tile16_off(int r, int c) { return r * kD + ((c ^ tile16_f(r)) << 3); }

// gfx950's transposing LDS read: per 16-lane group a 4-row x 16-channel
// block becomes one channel x 4 rows per lane
__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t *p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(lds_void *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// reductions across the two 32-lane halves (lane l and lane l ^ 32)
__device__ __forceinline__ float half_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace h3
