// Device-side helpers shared by the gfx950 kernels: bf16 vector types, the MFMA wrapper and the
// operand-row permutation used by the attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace pkd {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16) on the matrix cores.
// Operand layout per lane l of the wave: A row (l % 32), k = 8*(l/32) .. +7;
// B column (l % 32), same k; D column (l % 32), register r holds row 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row permutation (swap bits 2 and 3 of the row index inside a 32-row block).  Feeding the first
// operand of a product whose result is reused as the k operand of a second product in this
// order makes each lane's 8 k values of the second product consecutive rows, so that operand
// can be read from LDS with one 16-byte load.
__device__ __forceinline__ int row_perm(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Row of 32x32 result register r for a lane in half hb (before any permutation).
__device__ __forceinline__ int acc_row(int r, int hb) { return 8 * (r >> 2) + 4 * hb + (r & 3); }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    bf16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
    return z;
}

__device__ __forceinline__ f32x16 zero_f32x16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16 *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

__device__ __forceinline__ void store_bf16x8(bf16 *p, bf16x8 v) {
    *reinterpret_cast<bf16x8 *>(p) = v;
}

__device__ __forceinline__ uint32_t pack_bf16x2(bf16 lo, bf16 hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

}  // namespace pkd
