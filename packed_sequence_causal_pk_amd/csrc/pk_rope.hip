// Prologue passes of the attention calls: the RoPE rotation table, rotated K (and Q for the
// backward), rowsum(dout * out) and the dout scale.
//
// Rotate-half RoPE ([UN-2023] "Introducing Unsloth：LLM 训练提速 30 倍", "OpenAI Triton kernels"):
// with x1 the first half of a head vector and x2 the second half,
//     R(x) = [x1 cos - x2 sin, x2 cos + x1 sin],
// and its backward is the transpose, sin -> -sin.  The angle of pair i at position p is
// p * base^(-2i/d); p restarts at 0 in every packed sequence ([UN-2026] §1: positions come from
// the pack's metadata).  The factors are computed once per call into a [T, d/2] table of
// (cos, sin), the "rotation factors served from a precomputed table" idea of
// [MV] "UnSloth极速微调：底层CUDA优化带来的变革", and read by the attention kernels instead of
// evaluating sin/cos in their loops.
//
// Rotated q and k, v, and the scaled dout are written as fp16, the matrix-core operand format of
// the attention kernels, so those can copy tiles straight into LDS.  The backward prologue first
// reduces max|dout| and max|v| per block (k_bwd_pre, whose other blocks write the (cos, sin)
// table).  k_bwd_rows then turns the maxima into powers of two sigma and tau with
// max|dout| * sigma and max|v| * tau in [1, 2) (each workgroup reduces the maxima itself, which
// costs less than a launch of its own), so the backward's fp16 operands (sigma dout, tau v, and
// dS scaled by sigma tau, all unscaled exactly at the end) stay inside fp16's range whatever the
// magnitude of the incoming gradient and of v (the bound is derived at k_bwd_rows), and writes
// the rotated Q (times scale * log2(e)) and K, tau V and sigma * dout in fp16,
// -sigma * tau * rowsum(dout * out) and -lse * log2(e).  Values the prologues round to fp16
// without a scale (rotated q and k; v in the forward) are range-checked against 65504: one out of
// range sets PK_META_FP16_RANGE in the meta's range word.
//
// The table: inverse frequencies base^(-2i/d) in double precision (once per workgroup, in LDS),
// each angle p * f in double, reduced modulo 2 pi in double, and its cosine and sine taken in
// float.  Thread layout: k_fwd_prep has one thread per (token, KV head, group c of 4 rotation
// pairs), the table blocks of k_bwd_pre one per (token, c); a thread owns elements d in
// [4c, 4c+4) and their partners d + D/2, so each rotation stays inside one thread and a token's
// threads read each half-row contiguously.
#include <algorithm>

#include "pk_internal.h"
#include "pk_device.h"

namespace {

using pkd::zero_bf16x8;

// Inverse frequencies base^(-2i/D) of the D/2 rotation pairs, in double precision, into the
// workgroup's LDS (every thread of the workgroup must call this before any returns).
template <int D>
__device__ __forceinline__ void rope_inv_freq(float base, double *s_inv) {
    if (threadIdx.x < D / 2) s_inv[threadIdx.x] = exp2(-(2.0 * threadIdx.x / D) * log2((double)base));
    __syncthreads();
}

// cos and sin of the angles of pairs [4c, 4c + 4) of token t: p * f formed in double, reduced
// modulo 2 pi in double (a two-part 2 pi), then sine and cosine of the reduced angle in float
// (the fp32 table needs no more).  Written to the table when `write`.
template <int D>
__device__ __forceinline__ void rope_factors(const int32_t *__restrict__ pos, int64_t t, int c,
                                             const double *s_inv, float2 *__restrict__ table,
                                             bool write, float cs[4], float sn[4]) {
    constexpr double kTwoPiHi = 6.283185307179586, kTwoPiLo = 2.4492935982947064e-16;
    constexpr double kInvTwoPi = 0.15915494309189535;
    const double p = (double)pos[t];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const double a = p * s_inv[4 * c + k];
        const double n = rint(a * kInvTwoPi);
        const double r = fma(-n, kTwoPiLo, fma(-n, kTwoPiHi, a));
        sincosf((float)r, &sn[k], &cs[k]);
    }
    if (write) {
        float4 *dst = reinterpret_cast<float4 *>(table + t * (D / 2) + 4 * c);
        dst[0] = make_float4(cs[0], sn[0], cs[1], sn[1]);
        dst[1] = make_float4(cs[2], sn[2], cs[3], sn[3]);
    }
}

// Largest magnitude an fp16 operand may take: the kernels round these values to fp16, which
// overflows past it.  A value above it (or not finite) sets PK_META_FP16_RANGE in the meta's
// range word; the results of that call are then not meaningful.
constexpr float kF16Max = 65504.f;

__device__ __forceinline__ void flag_range(bool bad, int32_t *flags) {
    if (__builtin_expect(bad, 0)) atomicOr(flags, PK_META_FP16_RANGE);
}

__device__ __forceinline__ float amax4(const float x[4]) {
    return fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
}

__device__ __forceinline__ void load4(const bf16 *p, float x[4]) {
    const uint2 raw = *reinterpret_cast<const uint2 *>(p);
    const bf16 *b = reinterpret_cast<const bf16 *>(&raw);
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = (float)b[k];
}

__device__ __forceinline__ void store4(f16 *p, const float x[4]) {
    uint2 raw;
    raw.x = pkd::pack_f16x2((f16)x[0], (f16)x[1]);
    raw.y = pkd::pack_f16x2((f16)x[2], (f16)x[3]);
    *reinterpret_cast<uint2 *>(p) = raw;
}

// Copy 4 + 4 elements of one head row as fp16 (no rotation); returns their largest magnitude.
template <int D>
__device__ __forceinline__ float convert_row(const bf16 *__restrict__ src, f16 *__restrict__ dst, int c) {
    float x1[4], x2[4];
    load4(src + 4 * c, x1);
    load4(src + D / 2 + 4 * c, x2);
    store4(dst + 4 * c, x1);
    store4(dst + D / 2 + 4 * c, x2);
    return fmaxf(amax4(x1), amax4(x2));
}

// Rotate 4 pairs of one head row (row points at the head's element 0); returns the largest
// magnitude of the rotated values.
template <int D>
__device__ __forceinline__ float rotate_row(const bf16 *__restrict__ src, f16 *__restrict__ dst,
                                            int c, const float cs[4], const float sn[4]) {
    float x1[4], x2[4], y1[4], y2[4];
    load4(src + 4 * c, x1);
    load4(src + D / 2 + 4 * c, x2);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        y1[k] = x1[k] * cs[k] - x2[k] * sn[k];
        y2[k] = x2[k] * cs[k] + x1[k] * sn[k];
    }
    store4(dst + 4 * c, y1);
    store4(dst + D / 2 + 4 * c, y2);
    return fmaxf(amax4(y1), amax4(y2));
}

// One thread per (token t, KV head h, group c of 4 rotation pairs), c fastest so that a wave's
// loads and stores are contiguous; the threads of head 0 also write the table.
template <int D>
__global__ __launch_bounds__(256) void k_fwd_prep(const int32_t *__restrict__ pos, int64_t T,
                                                  int hkv, float base,
                                                  const bf16 *__restrict__ k,
                                                  const bf16 *__restrict__ v,
                                                  f16 *__restrict__ krot,
                                                  f16 *__restrict__ vh,
                                                  float2 *__restrict__ table,
                                                  int32_t *__restrict__ flags) {
    constexpr int G = D / 8;
    __shared__ double s_inv[D / 2];
    rope_inv_freq<D>(base, s_inv);
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int c = (int)(gid % G);
    const int64_t rest = gid / G;
    const int h = (int)(rest % hkv);
    const int64_t t = rest / hkv;
    if (t >= T) return;
    float cs[4], sn[4];
    rope_factors<D>(pos, t, c, s_inv, table, h == 0, cs, sn);
    const int64_t off = (t * hkv + h) * D;
    const float m = fmaxf(rotate_row<D>(k + off, krot + off, c, cs, sn), convert_row<D>(v + off, vh + off, c));
    flag_range(!(m <= kF16Max), flags);
}

// max|x| per block over a flattened bf16 tensor of n8 groups of 8 elements (dout, v), 8 elements
// per thread step; block b of nb.
__device__ __forceinline__ void bwd_amax_block(const bf16 *__restrict__ dout, int64_t n8,
                                               float *__restrict__ blockmax, int b, int nb) {
    __shared__ float s_max[4];
    float amax = 0.f;
    auto fold = [&](const uint4 &raw) {
        const bf16 *b = reinterpret_cast<const bf16 *>(&raw);
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf((float)b[k]));
    };
    const int64_t stride = (int64_t)nb * 256;
    int64_t c = (int64_t)b * 256 + threadIdx.x;
    // four independent 16-byte loads in flight per thread, then the remainder one at a time
    for (; c + 3 * stride < n8; c += 4 * stride) {
        uint4 raw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) raw[k] = *reinterpret_cast<const uint4 *>(dout + 8 * (c + k * stride));
#pragma unroll
        for (int k = 0; k < 4; ++k) fold(raw[k]);
    }
    for (; c < n8; c += stride) fold(*reinterpret_cast<const uint4 *>(dout + 8 * c));
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = amax;
    __syncthreads();
    if (threadIdx.x == 0)
        blockmax[b] = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
}

// Store 4 floats as fp16 after scaling.
__device__ __forceinline__ void store4s(f16 *p, const float x[4], float scale) {
    const float y[4] = {x[0] * scale, x[1] * scale, x[2] * scale, x[3] * scale};
    store4(p, y);
}

// The (cos, sin) table alone: one thread per (token, group of 4 rotation pairs).
template <int D>
__device__ __forceinline__ void rope_table_block(const int32_t *__restrict__ pos, int64_t T, float base,
                                                 float2 *__restrict__ table, int b) {
    constexpr int G = D / 8;
    __shared__ double s_inv[D / 2];
    rope_inv_freq<D>(base, s_inv);
    const int64_t gid = (int64_t)b * 256 + threadIdx.x;
    const int64_t t = gid / G;
    if (t >= T) return;
    float cs[4], sn[4];
    rope_factors<D>(pos, t, (int)(gid % G), s_inv, table, true, cs, sn);
}

// First launch of the backward prologue, three independent jobs in one grid (fewer launches,
// which small packs feel): blocks [0, nb) reduce max|dout| per block, blocks [nb, nb + nbv)
// max|v| per block (into blockmax[nb ..]), the rest write the RoPE table (one thread per token
// and group of 4 rotation pairs).  Block 0 also clears the work counters.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_pre(const bf16 *__restrict__ dout, int64_t n8,
                                                 const bf16 *__restrict__ v, int64_t n8v,
                                                 float *__restrict__ blockmax, int nb, int nbv,
                                                 const int32_t *__restrict__ pos, int64_t T,
                                                 float base, float2 *__restrict__ table,
                                                 int32_t *__restrict__ sched) {
    const int b = (int)blockIdx.x;
    if (b == 0 && threadIdx.x < pk::kSchedInts) sched[threadIdx.x] = 0;
    if (b < nb)
        bwd_amax_block(dout, n8, blockmax, b, nb);
    else if (b < nb + nbv)
        bwd_amax_block(v, n8v, blockmax + nb, b - nb, nbv);
    else
        rope_table_block<D>(pos, T, base, table, b - nb - nbv);
}

// Rotation factors of pairs [8c, 8c + 8) of token t from the table.
template <int D>
__device__ __forceinline__ void table8(const float2 *__restrict__ table, int64_t t, int c,
                                       float cs[8], float sn[8]) {
    const float4 *f = reinterpret_cast<const float4 *>(table + t * (D / 2) + 8 * c);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float4 x = f[k];
        cs[2 * k] = x.x;
        sn[2 * k] = x.y;
        cs[2 * k + 1] = x.z;
        sn[2 * k + 1] = x.w;
    }
}

// A power-of-two scale computed by every workgroup that needs it from per-block maxima (at most
// 1024 floats, an L2-resident read): 2^e with max * 2^e in [1, 2) (1 when the maximum is 0; 1
// and a range flag when it is not finite).  Used for sigma (from max|dout|) and tau (from
// max|v|).  Every thread of the workgroup must call it; all get the same value.
__device__ __forceinline__ float block_pow2_scale(const float *__restrict__ blockmax, int nb,
                                                  int32_t *__restrict__ flags) {
    __shared__ float s_max[4];
    __syncthreads();   // s_max may still be read by a previous call
    float m = 0.f;
    for (int i = threadIdx.x; i < nb; i += 256) m = fmaxf(m, blockmax[i]);
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    float scale = 1.f;
    if (m > 0.f && m <= 3.0e38f) {
        int ex = 0;
        (void)frexpf(m, &ex);           // m = f * 2^ex, f in [0.5, 1)
        ex = min(max(1 - ex, -100), 100);
        scale = ldexpf(1.f, ex);
    }
    if (threadIdx.x == 0) flag_range(!(m <= 3.0e38f), flags);
    return scale;
}

// Per-row work of the backward prologue, one thread per (row, group c of 8 rotation pairs): the
// thread owns elements [8c, 8c + 8) of a head row and their partners + D/2, read and written as
// 16-byte vectors.  Rows [0, T * hkv) are K rows (rotated) with their V rows (converted, times
// tau); rows [T * hkv, T * (hkv + hq)) are query-head rows: Q rotated and multiplied by qscale
// (the softmax scale times log2(e), so that the backward's score products come out in the exp2
// domain), sigma * dout, and the row values -sigma * tau * sum(dout * out) and -lse * log2(e),
// stored negated because the backward's products start from them.
//
// sigma and tau are powers of two from the maxima k_bwd_pre reduced: max|sigma dout| and
// max|tau v| lie in [1, 2).  With them every fp16 operand of the backward has a bound that holds
// for any finite dout and v:  |sigma dout| < 2, |tau v| < 2, P <= 1, and
//     |sigma tau dS_ij| = P_ij |sigma tau (dout_i . v_j - D_i)| < 2 d * 2 + 2 d * 2 = 8 d
// (|dout_i . v_j| <= |dout_i|_1 max|v|, and |D_i| <= |dout_i|_1 max|out_i| <= |dout_i|_1 max|v|
// because out_i is a convex combination of v rows), i.e. < 1024 for d = 128.  The remaining
// inputs are range-checked here: |R(q)| * qscale and |R(k)| above 65504 (or not finite) set the
// range flag.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_rows(int64_t T, int hq, int hkv,
                                                  const float2 *__restrict__ table,
                                                  const bf16 *__restrict__ q,
                                                  const bf16 *__restrict__ k,
                                                  const bf16 *__restrict__ v,
                                                  const bf16 *__restrict__ out,
                                                  const bf16 *__restrict__ dout,
                                                  const float *__restrict__ lse,
                                                  const float *__restrict__ blockmax, int nb, int nbv,
                                                  float *__restrict__ dscale,
                                                  f16 *__restrict__ qrot,
                                                  f16 *__restrict__ krot,
                                                  f16 *__restrict__ vh,
                                                  f16 *__restrict__ dout16,
                                                  float *__restrict__ dsum,
                                                  float *__restrict__ lse2, float qscale,
                                                  int32_t *__restrict__ flags) {
    constexpr int G = D / 16;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int c = (int)(gid % G);
    int64_t row = gid / G;
    const int64_t nkv = T * hkv;
    // tau in every workgroup (its V rows or its dsum rows need it); sigma in the workgroups that
    // hold query rows (a workgroup-uniform test); the first of them also stores
    // {sigma, 1/sigma, tau, 1/(sigma tau)} for the attention kernels
    const float tau = block_pow2_scale(blockmax + nb, nbv, flags);
    float sigma = 1.f;
    const int64_t first_q_block = nkv * G / 256;
    if ((int64_t)blockIdx.x >= first_q_block) {
        sigma = block_pow2_scale(blockmax, nb, flags);
        if ((int64_t)blockIdx.x == first_q_block && threadIdx.x == 0) {
            dscale[0] = sigma;
            dscale[1] = 1.f / sigma;
            dscale[2] = tau;
            dscale[3] = 1.f / (sigma * tau);
        }
    }
    float cs[8], sn[8];
    // rotate 8 pairs, scale, store as fp16; returns the largest magnitude stored
    auto rotate = [&](const bf16 *src, f16 *dst, float mult) {
        const bf16x8 x1 = pkd::load_bf16x8(src + 8 * c), x2 = pkd::load_bf16x8(src + D / 2 + 8 * c);
        f16x8 y1, y2;
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float a1 = (float)x1[e], a2 = (float)x2[e];
            const float b1 = (a1 * cs[e] - a2 * sn[e]) * mult, b2 = (a2 * cs[e] + a1 * sn[e]) * mult;
            m = fmaxf(m, fmaxf(fabsf(b1), fabsf(b2)));
            y1[e] = (f16)b1;
            y2[e] = (f16)b2;
        }
        pkd::store_f16x8(dst + 8 * c, y1);
        pkd::store_f16x8(dst + D / 2 + 8 * c, y2);
        return m;
    };
    if (row < nkv) {
        table8<D>(table, row / hkv, c, cs, sn);
        const int64_t off = row * D;
        flag_range(!(rotate(k + off, krot + off, 1.0f) <= kF16Max), flags);
        pkd::store_f16x8(vh + off + 8 * c, pkd::bf16x8_to_f16x8(pkd::load_bf16x8(v + off + 8 * c), tau));
        pkd::store_f16x8(vh + off + D / 2 + 8 * c,
                         pkd::bf16x8_to_f16x8(pkd::load_bf16x8(v + off + D / 2 + 8 * c), tau));
        return;
    }
    row -= nkv;
    // The G threads of a row are consecutive lanes of one wave and exit together, so the
    // shuffle reduction below only mixes lanes of one row.
    if (row >= T * hq) return;
    const int64_t t = row / hq;
    const int h = (int)(row % hq);
    table8<D>(table, t, c, cs, sn);
    const int64_t off = row * D;
    flag_range(!(rotate(q + off, qrot + off, qscale) <= kF16Max), flags);
    const bf16x8 o1 = pkd::load_bf16x8(out + off + 8 * c), o2 = pkd::load_bf16x8(out + off + D / 2 + 8 * c);
    const bf16x8 g1 = pkd::load_bf16x8(dout + off + 8 * c), g2 = pkd::load_bf16x8(dout + off + D / 2 + 8 * c);
    pkd::store_f16x8(dout16 + off + 8 * c, pkd::bf16x8_to_f16x8(g1, sigma));
    pkd::store_f16x8(dout16 + off + D / 2 + 8 * c, pkd::bf16x8_to_f16x8(g2, sigma));
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) part += (float)o1[e] * (float)g1[e] + (float)o2[e] * (float)g2[e];
#pragma unroll
    for (int sh = G / 2; sh > 0; sh >>= 1) part += __shfl_xor(part, sh, 64);
    if (c == 0) {
        // stored negated: the dP products start from it
        dsum[(int64_t)h * T + t] = -part * (sigma * tau);
        lse2[(int64_t)h * T + t] = -lse[(int64_t)h * T + t] * pkd::kLog2e;
    }
}

}  // namespace

namespace pk {

unsigned prep_blocks(int64_t T, int d) { return (unsigned)((T * (d / 8) + 255) / 256); }

unsigned dmax_blocks(int64_t T, int hq, int d) {
    const int64_t n8 = T * hq * d / 8;
    return (unsigned)std::max<int64_t>(1, std::min<int64_t>(1024, (n8 + 255) / 256));
}

unsigned vmax_blocks(int64_t T, int hkv, int d) {
    const int64_t n8 = T * hkv * d / 8;
    return (unsigned)std::max<int64_t>(1, std::min<int64_t>(256, (n8 + 1023) / 1024));
}

hipError_t launch_fwd_prep(const RopeArgs &r, const void *k, const void *v, void *krot, void *vh,
                           void *rope, int32_t *flags, hipStream_t s) {
    const unsigned g = (unsigned)((r.T * r.hkv * (r.d / 8) + 255) / 256);
    if (r.d == 128)
        k_fwd_prep<128><<<g, 256, 0, s>>>(r.pos, r.T, r.hkv, r.rope_base, (const bf16 *)k,
                                           (const bf16 *)v, (f16 *)krot, (f16 *)vh, (float2 *)rope,
                                           flags);
    else
        k_fwd_prep<64><<<g, 256, 0, s>>>(r.pos, r.T, r.hkv, r.rope_base, (const bf16 *)k,
                                          (const bf16 *)v, (f16 *)krot, (f16 *)vh, (float2 *)rope,
                                          flags);
    return hipGetLastError();
}

hipError_t launch_bwd_prep(const RopeArgs &r, const void *q, const void *k, const void *v,
                           const void *out, const void *dout, const float *lse, void *qrot,
                           void *krot, void *vh, void *dout16, void *rope, float *dsum,
                           float *lse2, float *blockmax, float *scale, float qscale,
                           int32_t *flags, int32_t *sched, hipStream_t s) {
    const int64_t n8 = r.T * r.hq * r.d / 8, n8v = r.T * r.hkv * r.d / 8;
    const unsigned nb = dmax_blocks(r.T, r.hq, r.d), nbv = vmax_blocks(r.T, r.hkv, r.d);
    const unsigned gt = prep_blocks(r.T, r.d);
    const unsigned gr = (unsigned)((r.T * (r.hq + r.hkv) * (r.d / 16) + 255) / 256);
    if (r.d == 128)
        k_bwd_pre<128><<<nb + nbv + gt, 256, 0, s>>>((const bf16 *)dout, n8, (const bf16 *)v, n8v,
                                                     blockmax, (int)nb, (int)nbv, r.pos, r.T,
                                                     r.rope_base, (float2 *)rope, sched);
    else
        k_bwd_pre<64><<<nb + nbv + gt, 256, 0, s>>>((const bf16 *)dout, n8, (const bf16 *)v, n8v,
                                                    blockmax, (int)nb, (int)nbv, r.pos, r.T,
                                                    r.rope_base, (float2 *)rope, sched);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (r.d == 128) {
        k_bwd_rows<128><<<gr, 256, 0, s>>>(r.T, r.hq, r.hkv, (const float2 *)rope, (const bf16 *)q,
                                            (const bf16 *)k, (const bf16 *)v, (const bf16 *)out,
                                            (const bf16 *)dout, lse, blockmax, (int)nb, (int)nbv,
                                            scale, (f16 *)qrot, (f16 *)krot, (f16 *)vh,
                                            (f16 *)dout16, dsum, lse2, qscale, flags);
    } else {
        k_bwd_rows<64><<<gr, 256, 0, s>>>(r.T, r.hq, r.hkv, (const float2 *)rope, (const bf16 *)q,
                                           (const bf16 *)k, (const bf16 *)v, (const bf16 *)out,
                                           (const bf16 *)dout, lse, blockmax, (int)nb, (int)nbv,
                                           scale, (f16 *)qrot, (f16 *)krot, (f16 *)vh,
                                           (f16 *)dout16, dsum, lse2, qscale, flags);
    }
    return hipGetLastError();
}

}  // namespace pk
