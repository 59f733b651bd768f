// LoRA-adapted QKV projection, the producer of the attention path's q, k, v
// ("Introducing Unsloth：LLM 训练提速 30 倍", "手动 Autograd": Q = X (W_q + A_q B_q), and the
// same for K and V).  With the three projections stacked along the output dimension:
//     Y [T, N] = X [T, K] (W + s A B),   W [K, N], A [K, r], B [r, N],
// computed without forming W + s A B:  Y = X W + U B with U = s X A (T x r, small).
//
// Storage (the weight layout of a linear layer, out x in): wt = W^T [N, K], at = A^T [r, K],
// bt = B^T [N, r]; x, y row-major; all bfloat16, fp32 accumulation on the matrix cores
// (v_mfma_f32_32x32x16_bf16).
//
// Three launches:
//   k_lora_pad   A^T and B^T copied into rank-64 zero-padded buffers (so the adapter term is one
//                more full 64-wide step of the same product);
//   k_gemm_nt (64 columns)   U = s X A (T x 64, columns >= r are zero), bf16;
//   k_gemm_nt (128 columns)  Y = X W + U B: one product over K + 64 reduction steps, the last
//                64 from (U, B), so the adapter costs one extra step instead of a pass over Y.
//
// k_gemm_nt computes C [M, N] = alpha (A1 B1^T + A2 B2^T) for row-major A* [M, K*] and B* [N, K*]
// (K* multiples of 64; the second pair optional).  Workgroup: BM rows of C x BN columns, 4
// waves; 64-wide K slices of both operands stream through double-buffered swizzled LDS tiles by
// asynchronous global->LDS copies (the attention kernels' tile format, 64 halves per row).  The
// product is taken transposed, C^T = B A^T, so each lane's accumulator holds 4 consecutive output
// columns of one row and the epilogue stores 8 bytes at a time.
#include "pk_internal.h"
#include "pk_device.h"


namespace {

using namespace pkd;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma32_bf16(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int kBK = 64;    // K slice per LDS tile (64 halves per tile row)
constexpr int kRank = 64;  // padded adapter rank

struct GemmArgs {
    const f16 *a1, *b1;    // [M, k1], [N, k1] (bf16 bits)
    const f16 *a2, *b2;    // [M, k2], [N, k2] or null
    f16 *c;                // [M, N] bf16 bits
    int64_t M;
    int N, k1, k2;
    float alpha;
};

// 4 waves as WN x WM over a BM x BN tile of C; each wave computes (BM / WM) rows x (BN / WN)
// columns.  The larger the wave's tile, the fewer LDS bytes per product (each operand chunk read
// from LDS feeds MBW or NBW products).
template <int BM, int BN, int WN, int MINWG>
__global__ __launch_bounds__(256, MINWG) void k_gemm_nt(GemmArgs g) {
    constexpr int kBM = BM;
    constexpr int WM = 4 / WN;
    constexpr int NBW = BN / WN / 32;          // 32-column blocks per wave
    constexpr int MBW = kBM / WM / 32;         // 32-row blocks per wave
    __shared__ __attribute__((aligned(16))) f16 lds_a[2][kBM * kBK];
    __shared__ __attribute__((aligned(16))) f16 lds_b[2][BN * kBK];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = w % WN, wm = w / WN;
    const int ntiles = g.N / BN;
    const int nt = blockIdx.x % ntiles;
    const int64_t m0 = (int64_t)(blockIdx.x / ntiles) * kBM;
    const int n0 = nt * BN;
    const bool full_m = m0 + kBM <= g.M;
    const int steps1 = g.k1 / kBK, steps = steps1 + g.k2 / kBK;
    const uint32_t off1a = tile_copy_lane_off<kBK, 4>(g.k1), off1b = off1a;
    const uint32_t off2 = tile_copy_lane_off<kBK, 4>(g.k2 > 0 ? g.k2 : kBK);

    // copy K slice s of both operands into buffer buf
    auto issue = [&](int s, int buf) {
        const bool first = s < steps1;
        const int kk = first ? s * kBK : (s - steps1) * kBK;
        const int ld = first ? g.k1 : g.k2;
        const f16 *ab = first ? g.a1 : g.a2;
        const f16 *bb = first ? g.b1 : g.b2;
        const uint32_t off = first ? off1a : off2;
        if (full_m) {
            tile_copy_async_whole<kBK, kBM, 4>(lds_a[buf], ab + m0 * ld + kk, ld, off);
        } else {
            // the last row tile: rows past M read row M - 1 (finite data, never stored)
            tile_copy_async<kBK, kBM>(lds_a[buf], 4, [&](int row) {
                return ab + min64(m0 + row, g.M - 1) * ld + kk;
            });
        }
        tile_copy_async_whole<kBK, BN, 4>(lds_b[buf], bb + (int64_t)n0 * ld + kk, ld,
                                          first ? off1b : off2);
    };

    // per-lane LDS offsets (bytes) of the 16-byte operand chunks: row (lane % 32) of each 32-row
    // block, k = 16 ks + 8 (lane / 32)
    uint32_t aoff[MBW][4], boff[NBW][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int j = 0; j < MBW; ++j)
            aoff[j][ks] = 2 * tile_off<kBK>(wm * (kBM / WM) + 32 * j + (lane & 31), 16 * ks + 8 * (lane >> 5));
#pragma unroll
        for (int i = 0; i < NBW; ++i)
            boff[i][ks] = 2 * tile_off<kBK>(wn * (BN / WN) + 32 * i + (lane & 31), 16 * ks + 8 * (lane >> 5));
    }

    f32x16 acc[NBW][MBW];
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < MBW; ++j) acc[i][j] = zero_f32x16();

    auto compute = [&](auto bufc) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        const char *ta = reinterpret_cast<const char *>(lds_a[BUF]);
        const char *tb = reinterpret_cast<const char *>(lds_b[BUF]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            f16x8 bf[NBW], af[MBW];
#pragma unroll
            for (int i = 0; i < NBW; ++i) bf[i] = *reinterpret_cast<const f16x8 *>(tb + boff[i][ks]);
#pragma unroll
            for (int j = 0; j < MBW; ++j) af[j] = *reinterpret_cast<const f16x8 *>(ta + aoff[j][ks]);
#pragma unroll
            for (int i = 0; i < NBW; ++i)
#pragma unroll
                for (int j = 0; j < MBW; ++j) acc[i][j] = mfma32_bf16(bf[i], af[j], acc[i][j]);
        }
    };
    auto step = [&](auto bufc, int s) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        lds_copy_wait();
        __syncthreads();
        if (s + 1 < steps) issue(s + 1, BUF ^ 1);
        compute(bufc);
    };
    issue(0, 0);
    for (int s = 0; s < steps; s += 2) {
        step(std::integral_constant<int, 0>(), s);
        if (s + 1 < steps) step(std::integral_constant<int, 1>(), s + 1);
    }

    // epilogue: acc[i][j] is C^T for columns n = n0 + wn*BN/WN + 32 i + 8 (r / 4) + 4 (lane / 32)
    // + r % 4 and row m = m0 + wm*kBM/WM + 32 j + lane % 32
#pragma unroll
    for (int j = 0; j < MBW; ++j) {
        const int64_t m = m0 + wm * (kBM / WM) + 32 * j + (lane & 31);
        if (m >= g.M) continue;
        f16 *crow = g.c + m * g.N;
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * (BN / WN) + 32 * i + 8 * q + 4 * (lane >> 5);
                uint2 raw;
                raw.x = pack_bf16x2((bf16)(acc[i][j][4 * q + 0] * g.alpha), (bf16)(acc[i][j][4 * q + 1] * g.alpha));
                raw.y = pack_bf16x2((bf16)(acc[i][j][4 * q + 2] * g.alpha), (bf16)(acc[i][j][4 * q + 3] * g.alpha));
                *reinterpret_cast<uint2 *>(crow + n) = raw;
            }
        }
    }
}

// Zero-padded copies of the adapter: apad [64, K] = A^T rows (zero for rows >= r),
// bpad [N, 64] = B^T columns (zero for columns >= r).  One thread per element of the outputs.
__global__ __launch_bounds__(256) void k_lora_pad(const f16 *__restrict__ at, const f16 *__restrict__ bt,
                                                  int r, int K, int N, f16 *__restrict__ apad,
                                                  f16 *__restrict__ bpad) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t na = (int64_t)kRank * K;
    if (gid < na) {
        const int j = (int)(gid / K);
        apad[gid] = j < r ? at[gid] : (f16)0.0f;
        return;
    }
    const int64_t e = gid - na;
    if (e >= (int64_t)N * kRank) return;
    const int64_t n = e / kRank;
    const int j = (int)(e % kRank);
    bpad[e] = j < r ? bt[n * r + j] : (f16)0.0f;
}

}  // namespace

namespace pk {

LoraWorkspace lora_workspace(int64_t T, int K, int N) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    LoraWorkspace w;
    size_t off = 0;
    w.u = off; off += al((size_t)T * kRank * 2);
    w.apad = off; off += al((size_t)kRank * K * 2);
    w.bpad = off; off += al((size_t)N * kRank * 2);
    w.total = off;
    return w;
}

hipError_t launch_lora_qkv(const void *x, const void *wt, const void *at, const void *bt,
                           int64_t T, int K, int N, int r, float scale, void *y, void *ws,
                           hipStream_t s) {
    const LoraWorkspace W = lora_workspace(T, K, N);
    char *base = static_cast<char *>(ws);
    f16 *u = reinterpret_cast<f16 *>(base + W.u);
    f16 *apad = reinterpret_cast<f16 *>(base + W.apad);
    f16 *bpad = reinterpret_cast<f16 *>(base + W.bpad);
    const int64_t npad = (int64_t)kRank * K + (int64_t)N * kRank;
    k_lora_pad<<<(unsigned)((npad + 255) / 256), 256, 0, s>>>((const f16 *)at, (const f16 *)bt, r, K, N,
                                                              apad, bpad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || T == 0) return e;
    GemmArgs g1{(const f16 *)x, apad, nullptr, nullptr, u, T, kRank, K, 0, scale};
    k_gemm_nt<128, 64, 1, 2><<<(unsigned)((T + 127) / 128), 256, 0, s>>>(g1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GemmArgs g2{(const f16 *)x, (const f16 *)wt, u, bpad, (f16 *)y, T, N, K, kRank, 1.0f};
    // 128 x 128 tiles, 64 KB of LDS, two workgroups per compute unit (measured on the
    // Qwen3-14B-shaped projection: 879 TFLOP/s; 256 x 128 tiles, whose 96 KB leave one workgroup
    // per compute unit, 683 TFLOP/s)
    k_gemm_nt<128, 128, 2, 2><<<(unsigned)((T + 127) / 128) * (unsigned)(N / 128), 256, 0, s>>>(g2);
    return hipGetLastError();
}

}  // namespace pk
