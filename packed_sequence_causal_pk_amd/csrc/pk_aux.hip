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
//    position p: p * base^(-2i/d), formed and reduced modulo 2 pi in double precision, its sine
//    and cosine taken in float, once per (token, pair, group of heads).
#include <algorithm>

#include "pk_internal.h"
#include "pk_device.h"

namespace {

constexpr int kMaskChunks = 4;   // 16-byte chunks per thread in the row-wise mask kernel

// Row-wise form, used when T is a multiple of 16: workgroup (bx, by) writes columns
// [bx * 16 KiB, +16 KiB) of rows by, by + gridDim.y, ...; thread x writes 16-byte chunks
// x, x + 256, x + 512, x + 768 of that span, so every store instruction of a wave covers 1 KiB
// of one row.  The row's first visible key lo = i - pos[i] is one scalar load per row.
__global__ __launch_bounds__(256) void k_dense_mask_rows(const int32_t *__restrict__ hdr,
                                                         const int32_t *__restrict__ pos, int T,
                                                         uint8_t *__restrict__ mask) {
    const bool valid = hdr[0] == 0;
    for (int i = blockIdx.y; i < T; i += gridDim.y) {
        const int lo = valid ? i - pos[i] : T;   // an invalid pack gets an all-zero mask
        const int hi = valid ? i : -1;
        uint8_t *row = mask + (int64_t)i * T;
#pragma unroll
        for (int k = 0; k < kMaskChunks; ++k) {
            const int j0 = 16 * ((blockIdx.x * kMaskChunks + k) * 256 + threadIdx.x);
            if (j0 >= T) break;
            uint32_t wv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t word = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int j = j0 + 4 * q + b;
                    word |= (uint32_t)(j >= lo && j <= hi) << (8 * b);
                }
                wv[q] = word;
            }
            *reinterpret_cast<uint4 *>(row + j0) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
    }
}

// General form (any T < 65536, so T * T < 2^32): one thread per 16 consecutive bytes of the
// flattened mask; a 16-byte run may cross into the next row (T not a multiple of 16, or T < 16).
__global__ __launch_bounds__(256) void k_dense_mask_flat(const int32_t *__restrict__ hdr,
                                                         const int32_t *__restrict__ pos, uint32_t T,
                                                         uint8_t *__restrict__ mask) {
    const uint32_t TT = T * T;
    const uint64_t b0 = ((uint64_t)blockIdx.x * 256 + threadIdx.x) * 16;
    if (b0 >= TT) return;
    const bool valid = hdr[0] == 0;
    uint32_t i = (uint32_t)b0 / T, j = (uint32_t)b0 - i * T;
    int64_t lo = valid ? (int64_t)i - pos[i] : T;
    uint8_t v[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
        v[x] = (uint8_t)((int64_t)j >= lo && j <= i);
        if (++j == T) {
            j = 0;
            ++i;
            lo = (valid && i < T) ? (int64_t)i - pos[i] : T;
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

constexpr int kRopeHeads = 4;   // heads per thread in the RoPE kernel

// One thread per (token t, group of kRopeHeads heads, group c of 8 rotation pairs): it owns
// elements [8c, 8c + 8) and their partners + D/2 of those heads, read and written as 16-byte
// vectors, all loads issued before any store.  x and out may be the same buffer: every element
// is read before the thread that owns it writes it, and no other thread touches it.
// The angles: inverse frequencies base^(-2i/D) in double precision (once per workgroup, in LDS),
// the angle p * f in double, reduced modulo 2 pi in double (a two-part 2 pi), then sin and cos
// of the reduced angle in float.
template <int D>
__global__ __launch_bounds__(256) void k_rope_apply(const int32_t *__restrict__ hdr,
                                                    const int32_t *__restrict__ pos, int64_t T,
                                                    int H, float base, int inverse,
                                                    const bf16 *x, bf16 *out) {
    constexpr int G = D / 16;
    __shared__ double s_inv[D / 2];
    if (threadIdx.x < D / 2) s_inv[threadIdx.x] = exp2(-(2.0 * threadIdx.x / D) * log2((double)base));
    __syncthreads();
    // T * ceil(H / kRopeHeads) * G < 2^32 for every accepted size, so 32-bit index arithmetic
    const uint32_t HG = (uint32_t)(H + kRopeHeads - 1) / kRopeHeads;
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    const int c = (int)(gid % G);
    const uint32_t rest = gid / G;
    const int hg = (int)(rest % HG);
    const int64_t t = rest / HG;
    if (t >= T) return;
    const bool valid = hdr[0] == 0;
    constexpr double kTwoPiHi = 6.283185307179586, kTwoPiLo = 2.4492935982947064e-16;
    constexpr double kInvTwoPi = 0.15915494309189535;
    const double p = valid ? (double)pos[t] : 0.0;
    float cs[8], sn[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const double a = p * s_inv[8 * c + k];
        const double n = rint(a * kInvTwoPi);
        const double r = fma(-n, kTwoPiLo, fma(-n, kTwoPiHi, a));
        float sf, cf;
        sincosf((float)r, &sf, &cf);
        cs[k] = cf;
        sn[k] = inverse ? -sf : sf;
    }
    const int h0 = hg * kRopeHeads;
    bf16x8 x1[kRopeHeads], x2[kRopeHeads];
#pragma unroll
    for (int u = 0; u < kRopeHeads; ++u) {
        if (h0 + u < H) {
            const int64_t off = (t * H + h0 + u) * D + 8 * c;
            x1[u] = pkd::load_bf16x8(x + off);
            x2[u] = pkd::load_bf16x8(x + off + D / 2);
        }
    }
#pragma unroll
    for (int u = 0; u < kRopeHeads; ++u) {
        if (h0 + u >= H) break;
        bf16x8 y1 = pkd::zero_bf16x8(), y2 = pkd::zero_bf16x8();
        if (valid) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a1 = (float)x1[u][e], a2 = (float)x2[u][e];
                y1[e] = (bf16)(a1 * cs[e] - a2 * sn[e]);
                y2[e] = (bf16)(a2 * cs[e] + a1 * sn[e]);
            }
        }
        const int64_t off = (t * H + h0 + u) * D + 8 * c;
        pkd::store_bf16x8(out + off, y1);
        pkd::store_bf16x8(out + off + D / 2, y2);
    }
}

}  // namespace

namespace pk {

hipError_t launch_dense_mask(const pk_meta_s &m, uint8_t *mask, hipStream_t s) {
    const int64_t T = m.total_tokens;
    if (T == 0) return hipSuccess;
    if (T % 16 == 0) {
        const unsigned bx = (unsigned)((T / 16 + 256 * kMaskChunks - 1) / (256 * kMaskChunks));
        const dim3 grid(bx, (unsigned)std::min<int64_t>(T, 65535));
        k_dense_mask_rows<<<grid, 256, 0, s>>>(m.hdr, m.pos, (int)T, mask);
    } else {
        const int64_t chunks = (T * T + 15) / 16;
        k_dense_mask_flat<<<(unsigned)((chunks + 255) / 256), 256, 0, s>>>(m.hdr, m.pos, (uint32_t)T, mask);
    }
    return hipGetLastError();
}

hipError_t launch_rope_apply(const pk_meta_s &m, const void *x, int H, int d, float base,
                             int inverse, void *out, hipStream_t s) {
    const int64_t T = m.total_tokens;
    if (T == 0) return hipSuccess;
    const int64_t hg = (H + kRopeHeads - 1) / kRopeHeads;
    const unsigned blocks = (unsigned)((T * hg * (d / 16) + 255) / 256);
    if (d == 128)
        k_rope_apply<128><<<blocks, 256, 0, s>>>(m.hdr, m.pos, T, H, base, inverse, (const bf16 *)x,
                                                 (bf16 *)out);
    else
        k_rope_apply<64><<<blocks, 256, 0, s>>>(m.hdr, m.pos, T, H, base, inverse, (const bf16 *)x,
                                                (bf16 *)out);
    return hipGetLastError();
}

}  // namespace pk
