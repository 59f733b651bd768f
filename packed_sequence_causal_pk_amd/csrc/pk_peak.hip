// Measured roofline of the device: the dense fp16 matrix-core rate and the HBM read, write and
// copy bandwidths the attention kernels are measured against.  Measurement aids only; nothing on
// the attention path calls them.
//
//   k_peak_mfma  every wave runs 4 independent chains of v_mfma_f32_32x32x16_f16 (the product
//                shape of the attention kernels) on register operands, so the matrix cores never
//                wait on memory; 32 * 32 * 16 * 2 flops per instruction.  One value per wave is
//                written so the chains cannot be dropped.
//   k_peak_read  reads a buffer with 16-byte loads, four in flight per thread.
//   k_peak_write fills a buffer with 16-byte stores.
//   k_peak_copy  copies with 16-byte loads and stores.
#include "pk_internal.h"
#include "pk_device.h"

namespace {

using namespace pkd;

__global__ __launch_bounds__(256) void k_peak_mfma(float *__restrict__ sink, int iters, float seed) {
    f16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (f16)(seed * (float)(threadIdx.x % 7 + e));
        b[e] = (f16)(seed * (float)(threadIdx.x % 5 - e));
    }
    f32x16 c0 = zero_f32x16(), c1 = zero_f32x16(), c2 = zero_f32x16(), c3 = zero_f32x16();
    for (int it = 0; it < iters; ++it) {
        c0 = mfma32(a, b, c0);
        c1 = mfma32(b, a, c1);
        c2 = mfma32(a, a, c2);
        c3 = mfma32(b, b, c3);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = s;
}

// Each workgroup moves one 16 KiB span: thread x takes 16-byte chunks x, x + 256, x + 512,
// x + 768, so every wave instruction covers 1 KiB of contiguous memory and each thread keeps four
// accesses in flight (the access pattern of the path's streaming kernels).
constexpr int kSpan16 = 1024;   // 16-byte chunks per workgroup

__global__ __launch_bounds__(256) void k_peak_read(const uint4 *__restrict__ src, int64_t n16,
                                                   float *__restrict__ sink) {
    const int64_t base = (int64_t)blockIdx.x * kSpan16 + threadIdx.x;
    uint32_t acc = 0;
    uint4 x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = base + 256 * k < n16 ? src[base + 256 * k] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= x[k].x ^ x[k].y ^ x[k].z ^ x[k].w;
    if (acc == 0x9e3779b9u) sink[0] = 1.f;   // practically never true; keeps the loads
}

__global__ __launch_bounds__(256) void k_peak_write(uint4 *__restrict__ dst, int64_t n16) {
    const int64_t base = (int64_t)blockIdx.x * kSpan16 + threadIdx.x;
    const uint4 v = make_uint4(threadIdx.x, blockIdx.x, 0u, 0u);
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (base + 256 * k < n16) dst[base + 256 * k] = v;
}

__global__ __launch_bounds__(256) void k_peak_copy(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                   int64_t n16) {
    const int64_t base = (int64_t)blockIdx.x * kSpan16 + threadIdx.x;
    uint4 x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (base + 256 * k < n16) x[k] = src[base + 256 * k];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (base + 256 * k < n16) dst[base + 256 * k] = x[k];
}

}  // namespace

extern "C" {

pk_status pk_peak_mfma(float *sink, int32_t workgroups, int32_t iters, void *hip_stream) {
    if (!sink || workgroups < 1 || iters < 1) return PK_ERR_INVALID;
    k_peak_mfma<<<workgroups, 256, 0, static_cast<hipStream_t>(hip_stream)>>>(sink, iters, 0.001f);
    return hipGetLastError() == hipSuccess ? PK_OK : PK_ERR_HIP;
}

pk_status pk_peak_hbm(int32_t mode, const void *src, void *dst, size_t bytes, float *sink,
                      void *hip_stream) {
    if (bytes == 0 || bytes % 16 || mode < 0 || mode > 2) return PK_ERR_INVALID;
    if ((mode != 1 && !src) || (mode != 0 && !dst) || (mode == 0 && !sink)) return PK_ERR_INVALID;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) return PK_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const int64_t n16 = (int64_t)(bytes / 16);
    const unsigned workgroups = (unsigned)((n16 + kSpan16 - 1) / kSpan16);
    if (mode == 0)
        k_peak_read<<<workgroups, 256, 0, s>>>((const uint4 *)src, n16, sink);
    else if (mode == 1)
        k_peak_write<<<workgroups, 256, 0, s>>>((uint4 *)dst, n16);
    else
        k_peak_copy<<<workgroups, 256, 0, s>>>((const uint4 *)src, (uint4 *)dst, n16);
    return hipGetLastError() == hipSuccess ? PK_OK : PK_ERR_HIP;
}

}  // extern "C"
