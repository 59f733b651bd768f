// Device-side helpers shared by the gfx950 kernels: vector types, the MFMA wrapper and the
// operand-row permutation used by the attention kernels.
//
// Number formats: tensors cross the ABI as bfloat16 (q, k, v, out, dout) or float32; inside the
// kernels every matrix-core operand is IEEE half (fp16) and every accumulator float32.  The
// bf16 inputs convert to fp16 exactly over fp16's normal range, and the values formed inside the
// kernels (RoPE-rotated q/k, softmax probabilities, dS) keep 3 more mantissa bits than bf16
// would give them, at the same v_mfma rate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace pkd {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, fp32) += A(32x16, fp16) * B(16x32, fp16) on the matrix cores (v_mfma_f32_32x32x16_f16).
// Operand layout per lane l of the wave: A row (l % 32), k = 8*(l/32) .. +7;
// B column (l % 32), same k; D column (l % 32), register r holds row 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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

__device__ __forceinline__ f16x8 zero_f16x8() {
    f16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (f16)0.0f;
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

__device__ __forceinline__ f16x8 load_f16x8(const f16 *p) {
    return *reinterpret_cast<const f16x8 *>(p);
}

__device__ __forceinline__ void store_f16x8(f16 *p, f16x8 v) {
    *reinterpret_cast<f16x8 *>(p) = v;
}

// bf16 -> fp16 through fp32 (exact over fp16's normal range), with an optional scale.
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(bf16x8 x, float scale = 1.0f) {
    f16x8 y;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = (f16)((float)x[i] * scale);
    return y;
}

__device__ __forceinline__ uint32_t pack_f16x2(f16 lo, f16 hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(bf16 lo, bf16 hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

}  // namespace pkd
