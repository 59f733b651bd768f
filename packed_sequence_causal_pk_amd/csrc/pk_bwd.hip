// Backward attention over a packed batch on gfx950 matrix cores.
//
// For the loss sum(out * dout) of the forward in pk_fwd.hip, with P the masked softmax,
// D_i = sum_d dout_i * out_i (computed in the prologue pass), and scores on the rotated Q, K:
//     dV_j     = sum over the group's heads and queries i of P_ij dout_i
//     dS_ij    = P_ij (dout_i . v_j - D_i)
//     dK_rot_j = scale * sum_i dS_ij q_rot_i          dQ_rot_i = scale * sum_j dS_ij k_rot_j
// and dK, dQ are the inverse rotations of dK_rot, dQ_rot.  This is the softmax calculus of the
// formula in [UN-2023] "Introducing Unsloth：LLM 训练提速 30 倍", "手动 Autograd" (which derives
// its gradients by hand), applied to A = softmax(Q K^T / sqrt(d) + M) V.
//
// Layout for CDNA4 (one workgroup = one backward work item, i.e. 128 keys, x one KV head):
//   * the 4 waves own 32 keys each; K_rot and V of those keys sit in registers as the k operand
//     of S = Q K^T and dP = dO V^T (v_mfma_f32_32x32x16_f16), so each lane owns one key column;
//   * dK^T and dV^T accumulate in registers over every query block AND every query head of the
//     GQA group, so the group sum costs nothing and dK, dV are written once;
//   * query blocks of 64 rows are staged in LDS row-major (for S, dP) and transposed (for the
//     dV^T += dO^T P and dK^T += Q^T dS products); query rows of S and dP are fed in row_perm
//     order so the transposed operands are single 16-byte LDS reads;
//   * dS goes to LDS once per block, and dQ_rot += dS K_rot is computed by all four waves from
//     LDS and accumulated into the float32 dq buffer with hardware float atomics (the inverse
//     RoPE of dq runs in the epilogue pass once all atomics are done);
//   * the mask is applied element-wise only on blocks that straddle a sequence boundary or the
//     diagonal; blocks fully outside the wave's visible range skip their products;
//   * operands are fp16 with fp32 accumulation.  dout enters scaled by the power of two sigma
//     the prologue chose (max|dout| * sigma in [1, 2)), so dP and dS are sigma-scaled too; the
//     results are unscaled exactly by 1/sigma when dQ, dK and dV are written.
#include "pk_internal.h"
#include "pk_device.h"

namespace {

using namespace pkd;

struct BwdArgs {
    const f16 *qrot;      // [T, hq, D] fp16
    const f16 *krot;      // [T, hkv, D] fp16
    const bf16 *v;        // [T, hkv, D]
    const bf16 *dout;     // [T, hq, D]
    const float *lse;     // [hq, T]
    const float *dsum;    // [hq, T]
    const float *dscale;  // {sigma, 1/sigma}
    const float2 *rope;   // [T, D/2]
    const int32_t *items; // [n_items, 8] longest first
    const int32_t *pos;   // [T]
    const int32_t *hdr;
    float *dq;            // [T, hq, D]  (accumulator, zeroed by the prologue pass)
    float *dk;            // [T, hkv, D]
    float *dv;            // [T, hkv, D]
    int64_t T;
    int hq, hkv, group;
    float scale;
};

template <int D>
struct BwdSmem {
    static constexpr int BQ = 64;        // query rows per block
    static constexpr int BKV = 128;      // keys per workgroup
    static constexpr int QP = D + 8;     // row-major Q / dO pitch
    static constexpr int TP = BQ + 8;    // transposed Q / dO pitch
    static constexpr int SP = BKV + 8;   // dS pitch
    static constexpr int KTP = BKV + 8;  // transposed K pitch
    f16 q[BQ * QP];
    f16 dO[BQ * QP];
    f16 qt[D * TP];
    f16 dOt[D * TP];
    f16 ds[BQ * SP];
    f16 kt[D * KTP];
    float lse[BQ];   // lse * log2(e); +inf for rows past the item
    float dd[BQ];    // D_i * sigma
    int lo[BQ];      // first key of the row's sequence; INT_MAX past the item
};

template <int D>
__device__ void bwd_zero_tile(const BwdArgs &a, int tile, int kvh) {
    const int64_t r0 = (int64_t)tile * PK_TILE_ROWS;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int e = threadIdx.x; e < PK_TILE_ROWS * (D / 4); e += blockDim.x) {
        const int64_t j = r0 + e / (D / 4);
        if (j < a.T) {
            const int64_t off = (j * a.hkv + kvh) * D + (e % (D / 4)) * 4;
            *reinterpret_cast<float4 *>(a.dk + off) = z;
            *reinterpret_cast<float4 *>(a.dv + off) = z;
        }
    }
}

__device__ __forceinline__ f16x8 load_as_f16x8(const f16 *p, float) { return load_f16x8(p); }
__device__ __forceinline__ f16x8 load_as_f16x8(const bf16 *p, float scale) {
    return bf16x8_to_f16x8(load_bf16x8(p), scale);
}

// Stage rows [qb, qb+BQ) of one head of a [T, H, D] tensor (fp16, or bf16 times `scale`) into
// LDS as fp16, row-major and transposed.  Each thread moves a pair of rows x 8 columns; rows at
// or past `q_end` are zero.
template <int D, typename Src>
__device__ __forceinline__ void stage_rows(const Src *__restrict__ src, float scale, int H, int h,
                                           int qb, int q_end, f16 *rowmaj, f16 *trans) {
    using S = BwdSmem<D>;
    for (int e = threadIdx.x; e < (S::BQ / 2) * (D / 8); e += 256) {
        const int rp = e % (S::BQ / 2), ch = e / (S::BQ / 2);
        const int i0 = qb + 2 * rp;
        const f16x8 x0 = i0 < q_end ? load_as_f16x8(src + ((int64_t)i0 * H + h) * D + ch * 8, scale) : zero_f16x8();
        const f16x8 x1 = i0 + 1 < q_end ? load_as_f16x8(src + ((int64_t)(i0 + 1) * H + h) * D + ch * 8, scale) : zero_f16x8();
        store_f16x8(rowmaj + (2 * rp) * S::QP + ch * 8, x0);
        store_f16x8(rowmaj + (2 * rp + 1) * S::QP + ch * 8, x1);
#pragma unroll
        for (int s = 0; s < 8; ++s)
            *reinterpret_cast<uint32_t *>(trans + (ch * 8 + s) * S::TP + 2 * rp) = pack_f16x2(x0[s], x1[s]);
    }
}

template <int D>
__global__ __launch_bounds__(256, 1) void k_attn_bwd(BwdArgs a) {
    using S = BwdSmem<D>;
    constexpr int BQ = S::BQ, BKV = S::BKV;
    constexpr int NKK = D / 16, NDB = D / 32;
    constexpr int NQB = 2 * NDB;          // 32x32 blocks of one dQ block (2 query x NDB d)
    constexpr int QB_PER_WAVE = NQB / 4;  // 2 for D = 128, 1 for D = 64
    __shared__ __attribute__((aligned(16))) S sm;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n32 = lane & 31, hb = lane >> 5;
    const int r = blockIdx.x / a.hkv, kvh = blockIdx.x % a.hkv;
    const int32_t *it = a.items + (int64_t)r * PK_ITEM_FIELDS;
    if (a.hdr[0] != 0) {
        bwd_zero_tile<D>(a, it[7], kvh);
        return;
    }
    const int kv_start = it[0], kv_end = it[1], q_start = it[2], q_end = it[3];
    const int64_t T = a.T;
    const float sigma = a.dscale[0], inv_sigma = a.dscale[1];

    const int j = kv_start + 32 * w + n32;  // this lane's key
    const bool kvalid = j < kv_end;
    const int wk0 = kv_start + 32 * w;
    const bool wave_active = wk0 < kv_end;
    const int wk_last = min(wk0 + 31, kv_end - 1);
    const int blk_last = kv_end - 1;

    // K_rot and V of this lane's key, as k operands (d in [16kk + 8hb, +8))
    f16x8 kf[NKK], vf[NKK];
    {
        const int64_t row = ((int64_t)(kvalid ? j : kv_start) * a.hkv + kvh) * D + 8 * hb;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            kf[kk] = kvalid ? load_f16x8(a.krot + row + 16 * kk) : zero_f16x8();
            vf[kk] = kvalid ? bf16x8_to_f16x8(load_bf16x8(a.v + row + 16 * kk)) : zero_f16x8();
        }
    }
    // K_rot^T of the workgroup's 128 keys -> LDS, for dQ
    for (int e = tid; e < (BKV / 2) * (D / 8); e += 256) {
        const int kp = e % (BKV / 2), ch = e / (BKV / 2);
        const int j0 = kv_start + 2 * kp;
        const f16x8 x0 = j0 < kv_end ? load_f16x8(a.krot + ((int64_t)j0 * a.hkv + kvh) * D + ch * 8) : zero_f16x8();
        const f16x8 x1 = j0 + 1 < kv_end ? load_f16x8(a.krot + ((int64_t)(j0 + 1) * a.hkv + kvh) * D + ch * 8) : zero_f16x8();
#pragma unroll
        for (int s = 0; s < 8; ++s)
            *reinterpret_cast<uint32_t *>(sm.kt + (ch * 8 + s) * S::KTP + 2 * kp) = pack_f16x2(x0[s], x1[s]);
    }

    f32x16 dka[NDB], dva[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        dka[db] = zero_f32x16();
        dva[db] = zero_f32x16();
    }

    for (int hh = 0; hh < a.group; ++hh) {
        const int h = kvh * a.group + hh;
        for (int qb = q_start; qb < q_end; qb += BQ) {
            __syncthreads();
            stage_rows<D>(a.qrot, 1.f, a.hq, h, qb, q_end, sm.q, sm.qt);
            stage_rows<D>(a.dout, sigma, a.hq, h, qb, q_end, sm.dO, sm.dOt);
            if (tid < BQ) {
                const int i = qb + tid;
                const bool ok = i < q_end;
                sm.lse[tid] = ok ? a.lse[(int64_t)h * T + i] * kLog2e : INFINITY;
                sm.dd[tid] = ok ? a.dsum[(int64_t)h * T + i] * sigma : 0.f;
                sm.lo[tid] = ok ? i - a.pos[i] : INT_MAX;
            }
            __syncthreads();
            const int nrows = min(BQ, q_end - qb);
            const int lo_first = sm.lo[0], lo_last = sm.lo[nrows - 1];
            // is any (query, key) pair of this block visible?
            if (qb + nrows - 1 < kv_start || lo_first > blk_last) continue;

            const bool active = wave_active && !(qb + nrows - 1 < wk0) && !(lo_first > wk_last);
            if (active) {
                const bool need_mask = !(qb >= wk0 + 31 && lo_last <= wk0);
                f32x16 sp[2], dp[2];
#pragma unroll
                for (int qm = 0; qm < 2; ++qm) {
                    sp[qm] = zero_f32x16();
                    dp[qm] = zero_f32x16();
                    const int row = 32 * qm + row_perm(n32);
                    const f16 *qrow = sm.q + row * S::QP + 8 * hb;
                    const f16 *grow = sm.dO + row * S::QP + 8 * hb;
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) {
                        sp[qm] = mfma32(load_f16x8(qrow + 16 * kk), kf[kk], sp[qm]);
                        dp[qm] = mfma32(load_f16x8(grow + 16 * kk), vf[kk], dp[qm]);
                    }
                }
                const float sl2 = a.scale * kLog2e;
#pragma unroll
                for (int qm = 0; qm < 2; ++qm) {
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) {
                        const int row = 32 * qm + row_perm(acc_row(rr, hb));
                        float p = exp2f(sp[qm][rr] * sl2 - sm.lse[row]);
                        if (need_mask) {
                            const int i = qb + row;
                            p = (j >= sm.lo[row] && j <= i) ? p : 0.f;
                        }
                        sp[qm][rr] = p;
                        dp[qm][rr] = p * (dp[qm][rr] - sm.dd[row]);
                    }
                }
                // dV^T += dO^T P,  dK^T += Q^T dS  (queries are the k dimension)
#pragma unroll
                for (int qm = 0; qm < 2; ++qm) {
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        f16x8 pb, sb;
#pragma unroll
                        for (int x = 0; x < 8; ++x) {
                            pb[x] = (f16)sp[qm][8 * e + x];
                            sb[x] = (f16)dp[qm][8 * e + x];
                        }
                        const int col = 32 * qm + 16 * e + 8 * hb;
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const int drow = 32 * db + n32;
                            dva[db] = mfma32(load_f16x8(sm.dOt + drow * S::TP + col), pb, dva[db]);
                            dka[db] = mfma32(load_f16x8(sm.qt + drow * S::TP + col), sb, dka[db]);
                        }
                    }
                }
                // dS -> LDS [query][key]
#pragma unroll
                for (int qm = 0; qm < 2; ++qm)
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr)
                        sm.ds[(32 * qm + row_perm(acc_row(rr, hb))) * S::SP + 32 * w + n32] = (f16)dp[qm][rr];
            } else {
                for (int row = hb; row < BQ; row += 2) sm.ds[row * S::SP + 32 * w + n32] = (f16)0.f;
            }
            __syncthreads();
            // dQ_rot[qb .. qb+64) += scale * dS K_rot, split in 32x32 blocks over the 4 waves
#pragma unroll
            for (int u = 0; u < QB_PER_WAVE; ++u) {
                const int pidx = w * QB_PER_WAVE + u;
                const int qm = pidx / NDB, db = pidx % NDB;
                f32x16 c = zero_f32x16();
                const f16 *arow = sm.ds + (32 * qm + n32) * S::SP + 8 * hb;
                const f16 *brow = sm.kt + (32 * db + n32) * S::KTP + 8 * hb;
#pragma unroll
                for (int ks = 0; ks < BKV / 16; ++ks)
                    c = mfma32(load_f16x8(arow + 16 * ks), load_f16x8(brow + 16 * ks), c);
                const float cscale = a.scale * inv_sigma;
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int i = qb + 32 * qm + acc_row(rr, hb);
                    if (i < q_end)
                        unsafeAtomicAdd(a.dq + ((int64_t)i * a.hq + h) * D + 32 * db + n32, c[rr] * cscale);
                }
            }
        }
    }

    // epilogue: dV as is; dK = R(-theta) (scale * dK_rot)
    if (kvalid) {
        float *dvrow = a.dv + ((int64_t)j * a.hkv + kvh) * D;
        float *dkrow = a.dk + ((int64_t)j * a.hkv + kvh) * D;
        const float2 *cs = a.rope + (int64_t)j * (D / 2);
        const float kscale = a.scale * inv_sigma;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = 32 * db + 8 * g4 + 4 * hb;
                *reinterpret_cast<float4 *>(dvrow + d) =
                    make_float4(dva[db][4 * g4] * inv_sigma, dva[db][4 * g4 + 1] * inv_sigma,
                                dva[db][4 * g4 + 2] * inv_sigma, dva[db][4 * g4 + 3] * inv_sigma);
            }
#pragma unroll
        for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = 32 * db + 8 * g4 + 4 * hb;  // first half; partner d + D/2
                float y1[4], y2[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float2 f = cs[d + x];
                    const float x1 = dka[db][4 * g4 + x] * kscale;
                    const float x2 = dka[db + NDB / 2][4 * g4 + x] * kscale;
                    y1[x] = x1 * f.x + x2 * f.y;
                    y2[x] = x2 * f.x - x1 * f.y;
                }
                *reinterpret_cast<float4 *>(dkrow + d) = make_float4(y1[0], y1[1], y1[2], y1[3]);
                *reinterpret_cast<float4 *>(dkrow + d + D / 2) = make_float4(y2[0], y2[1], y2[2], y2[3]);
            }
    }
}

}  // namespace

namespace pk {

hipError_t launch_bwd(const AttnShape &sh, const pk_meta_s &m, const void *qrot,
                      const void *krot, const void *v, const void *dout, const float *lse,
                      const float *dsum, const float *scale, const void *rope, float *dq,
                      float *dk, float *dv, hipStream_t s) {
    BwdArgs a;
    a.qrot = (const f16 *)qrot;
    a.krot = (const f16 *)krot;
    a.dscale = scale;
    a.v = (const bf16 *)v;
    a.dout = (const bf16 *)dout;
    a.lse = lse;
    a.dsum = dsum;
    a.rope = (const float2 *)rope;
    a.items = m.bwd_items;
    a.pos = m.pos;
    a.hdr = m.hdr;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.T = sh.T;
    a.hq = sh.hq;
    a.hkv = sh.hkv;
    a.group = sh.hq / sh.hkv;
    a.scale = sh.scale;
    const unsigned grid = (unsigned)sh.n_items * (unsigned)sh.hkv;
    if (sh.d == 128)
        k_attn_bwd<128><<<grid, 256, 0, s>>>(a);
    else
        k_attn_bwd<64><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace pk
