// Two steps around the attention path, each usable on its own:
//
//  * k_dense_mask -- the materialised T x T keep pattern of a pack, the structure the pages'
//    uncached path rebuilds for every layer ([UN-2026] "如何用 Unsloth 和 NVIDIA 让 LLM 训练更快"
//    §1 "快速合理性验证": the packed SDPA mask rebuild dominates the repeated per-layer cost).
//    The attention kernels never read it; it exists to measure that baseline on this device.
//    Key j is visible to query i iff cu[seq(i)] <= j <= i, i.e. j in [i - pos[i], i], so a row is
//    one run of ones and the kernel is a pure HBM write stream.
//
//  * k_rope_apply -- rotate-half RoPE of a [T, H, d] bfloat16 tensor at each token's position
//    inside its packed sequence ([UN-2023] "Introducing Unsloth：LLM 训练提速 30 倍",
//    "OpenAI Triton kernels": out1 = x1 cos - x2 sin, out2 = x2 cos + x1 sin over the two halves
//    of the head dim; the backward flag applies the transpose, sin -> -sin).  Angle of pair i at
//    position p: p * base^(-2i/d), evaluated in double precision and rounded to float for the
//    rotation, once per (token, pair) and reused over the heads.
#include "pk_internal.h"
#include "pk_device.h"

namespace {

// One thread per 16 consecutive bytes of the row-major [T, T] mask (T*T bytes in all).  A
// 16-byte run may cross into the next row (T not a multiple of 16, or T < 16).
__global__ __launch_bounds__(256) void k_dense_mask(const int32_t *__restrict__ hdr,
                                                    const int32_t *__restrict__ pos, int64_t T,
                                                    uint8_t *__restrict__ mask) {
    const int64_t TT = T * T;
    const int64_t b0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
    if (b0 >= TT) return;
    const bool valid = hdr[0] == 0;
    int64_t i = b0 / T, j = b0 - i * T;
    int64_t lo = valid ? i - pos[i] : T;   // an invalid pack gets an all-zero mask
    uint8_t v[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
        v[x] = (uint8_t)(j >= lo && j <= i);
        if (++j == T) {
            j = 0;
            ++i;
            lo = (valid && i < T) ? i - pos[i] : T;
        }
    }
    if (b0 + 16 <= TT) {
        uint4 w;
        w.x = v[0] | (v[1] << 8) | (v[2] << 16) | ((uint32_t)v[3] << 24);
        w.y = v[4] | (v[5] << 8) | (v[6] << 16) | ((uint32_t)v[7] << 24);
        w.z = v[8] | (v[9] << 8) | (v[10] << 16) | ((uint32_t)v[11] << 24);
        w.w = v[12] | (v[13] << 8) | (v[14] << 16) | ((uint32_t)v[15] << 24);
        *reinterpret_cast<uint4 *>(mask + b0) = w;
    } else {
        for (int x = 0; x < 16 && b0 + x < TT; ++x) mask[b0 + x] = v[x];
    }
}

// One thread per (token t, group c of 8 rotation pairs): it owns elements [8c, 8c + 8) and
// their partners + D/2 of every head of token t, read and written as 16-byte vectors.  x and out
// may be the same buffer: every element is read before the thread that owns it writes it.
template <int D>
__global__ __launch_bounds__(256) void k_rope_apply(const int32_t *__restrict__ hdr,
                                                    const int32_t *__restrict__ pos, int64_t T,
                                                    int H, float base, int inverse,
                                                    const bf16 *x, bf16 *out) {
    constexpr int G = D / 16;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t t = gid / G;
    const int c = (int)(gid % G);
    if (t >= T) return;
    const bool valid = hdr[0] == 0;
    float cs[8], sn[8];
    const double p = valid ? (double)pos[t] : 0.0;
    const double lb = log2((double)base);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int i = 8 * c + k;
        double s, co;
        sincos(p * exp2(-(2.0 * i / D) * lb), &s, &co);
        cs[k] = (float)co;
        sn[k] = inverse ? -(float)s : (float)s;
    }
    for (int h = 0; h < H; ++h) {
        const int64_t off = (t * H + h) * D + 8 * c;
        bf16x8 y1 = pkd::zero_bf16x8(), y2 = pkd::zero_bf16x8();
        if (valid) {
            const bf16x8 x1 = pkd::load_bf16x8(x + off), x2 = pkd::load_bf16x8(x + off + D / 2);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a1 = (float)x1[e], a2 = (float)x2[e];
                y1[e] = (bf16)(a1 * cs[e] - a2 * sn[e]);
                y2[e] = (bf16)(a2 * cs[e] + a1 * sn[e]);
            }
        }
        pkd::store_bf16x8(out + off, y1);
        pkd::store_bf16x8(out + off + D / 2, y2);
    }
}

}  // namespace

namespace pk {

hipError_t launch_dense_mask(const pk_meta_s &m, uint8_t *mask, hipStream_t s) {
    const int64_t T = m.total_tokens;
    const int64_t chunks = (T * T + 15) / 16;
    if (chunks == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((chunks + 255) / 256);
    k_dense_mask<<<blocks, 256, 0, s>>>(m.hdr, m.pos, T, mask);
    return hipGetLastError();
}

hipError_t launch_rope_apply(const pk_meta_s &m, const void *x, int H, int d, float base,
                             int inverse, void *out, hipStream_t s) {
    const int64_t T = m.total_tokens;
    if (T == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((T * (d / 16) + 255) / 256);
    if (d == 128)
        k_rope_apply<128><<<blocks, 256, 0, s>>>(m.hdr, m.pos, T, H, base, inverse, (const bf16 *)x,
                                                 (bf16 *)out);
    else
        k_rope_apply<64><<<blocks, 256, 0, s>>>(m.hdr, m.pos, T, H, base, inverse, (const bf16 *)x,
                                                (bf16 *)out);
    return hipGetLastError();
}

}  // namespace pk
