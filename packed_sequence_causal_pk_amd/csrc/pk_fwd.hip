// Forward attention over a packed batch on gfx950 matrix cores.
//
// Computes, for every query row i and query head h ([UN-2023] "Introducing Unsloth：LLM 训练提速
// 30 倍", "手动 Autograd", read with the scale 1/sqrt(d)):
//     out[i, h] = sum_j softmax_j(scale * <R q_i, R k_j> + M_ij) v_j,   lse[h, i] = log sum_j exp(.)
// with M_ij = 0 when j lies in i's packed sequence and j <= i, else -inf.  M is never formed:
// the forward work list gives each 128-query tile the key range [start of its first sequence,
// end of the tile], and inside that range only tiles that straddle a sequence boundary or the
// diagonal are masked, element by element, from each query's sequence start lo_i = i - pos_i.
//
// Design ([N1N-2026] "利用 Unsloth 和 NVIDIA 硬件加速 LLM 训练", §2 "FlashAttention-2 的深度集成":
// tiles stay on chip, softmax is fused with the two products, no N x N matrix is stored),
// laid out for CDNA4:
//   * one workgroup = one work item (128 queries) x one query head; 4 waves of 32 queries;
//     items are taken in the work list's longest-first order, heads fastest;
//   * the scores are computed transposed, S^T = K_rot Q_rot^T, with v_mfma_f32_32x32x16_f16,
//     so each lane of a wave owns one query: the row max needs one cross-half exchange and the
//     O^T accumulator is rescaled with a per-lane factor;
//   * P^T stays in registers and is the k operand of O^T += V^T P^T; key rows of the first
//     product are fed in row_perm order so each lane's 8 keys of the V^T operand are
//     consecutive, read with two transposing LDS loads (ds_read_b64_tr_b16);
//   * K_rot and V tiles of 32 keys (64 on small packs; both fp16, written by the prologue pass)
//     stream into double-buffered swizzled row-major LDS tiles (no padding, no transposed copy;
//     32 KB per workgroup, so three workgroups share a compute unit) with asynchronous
//     global->LDS copies, so the next tile loads while the current one is computed and no
//     registers are spent on staging;
//   * online softmax in the exp2 domain with scale * log2(e) folded into the scores; the row
//     sum adds the same fp16-rounded weights that multiply V (v_dot2_f32_f16, two per op);
//   * LDS operands are issued a few products ahead of the products that take them;
//   * Q is rotated in the prologue from the per-call (cos, sin) table; K comes pre-rotated;
//   * operands are fp16 (the bf16 inputs convert exactly; rotated values, P keep 3 more bits
//     than bf16), accumulators and the softmax state fp32.
#include <type_traits>

#include "pk_internal.h"
#include "pk_device.h"

namespace {

using namespace pkd;

struct FwdArgs {
    const bf16 *q;        // [T, hq, D]
    const f16 *krot;      // [T, hkv, D] fp16
    const f16 *v;         // [T, hkv, D] fp16 copy of v
    const float2 *rope;   // [T, D/2] (cos, sin)
    const int32_t *items; // [n_items, 8] longest first
    const int32_t *pos;   // [T]
    const int32_t *hdr;   // status, max_seqlen
    int32_t *flags;       // the meta's operand-range word
    bf16 *out;            // [T, hq, D]
    float *lse;           // [hq, T]
    int64_t T;
    int hq, hkv, group;
    float scale_log2;     // softmax scale * log2(e)
    float inv_scale_log2; // its reciprocal (the rescale threshold is a heuristic: a rounding of
                          // it only moves which tile rescales)
};

template <int D>
__device__ void fwd_zero_tile(const FwdArgs &a, int tile, int h) {
    const int64_t r0 = (int64_t)tile * PK_TILE_ROWS;
    for (int e = threadIdx.x; e < PK_TILE_ROWS * (D / 8); e += blockDim.x) {
        const int64_t i = r0 + e / (D / 8);
        if (i < a.T) store_bf16x8(a.out + (i * a.hq + h) * D + (e % (D / 8)) * 8, zero_bf16x8());
    }
    for (int e = threadIdx.x; e < PK_TILE_ROWS; e += blockDim.x)
        if (r0 + e < a.T) a.lse[(int64_t)h * a.T + r0 + e] = 0.f;
}

// BK keys per LDS tile: 32 (32 KB of tiles per workgroup, three workgroups per compute unit) on
// packs with many (item, head) workgroups; 64 (64 KB, two per compute unit, half the barriers
// and tile copies per key) on small packs, whose time goes to latency rather than throughput
// (measured: 64-key tiles are 4-6% slower on the Qwen3-14B-shaped pack and 6-7% faster on the
// Llama- and Qwen3-0.6B-shaped ones).
template <int D, int BK>
__global__ __launch_bounds__(256, 2) void k_attn_fwd(FwdArgs a) {
    static_assert(BK == 32 || BK == 64, "tiles of 32 or 64 keys");
    constexpr int NKK = D / 16;   // k-steps of the score product
    constexpr int NDB = D / 32;   // 32-row blocks of O^T
    constexpr int NMB = BK / 32;  // 32-key blocks per tile
    __shared__ __attribute__((aligned(16))) f16 lds_k[2][BK * D];   // double-buffered tiles
    __shared__ __attribute__((aligned(16))) f16 lds_v[2][BK * D];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: lets bounds live in SGPRs
    const int n32 = lane & 31, hb = lane >> 5;
    int r, h;
    item_head_of_block(blockIdx.x, a.hq, a.hkv, r, h);
    const int kvh = h / a.group;
    const int32_t *it = a.items + (int64_t)r * PK_ITEM_FIELDS;
    if (a.hdr[0] != 0) {
        fwd_zero_tile<D>(a, it[7], h);
        return;
    }
    const int q_start = it[0], q_end = it[1], kv_start = it[2];
    const int64_t T = a.T;

    // this lane's query and its wave's query range
    const int i = q_start + 32 * w + n32;
    const bool qvalid = i < q_end;
    const int lo_i = qvalid ? i - a.pos[i] : 0;
    const int wq0 = q_start + 32 * w;
    const bool wave_active = wq0 < q_end;
    const int wq_last = min(wq0 + 31, q_end - 1);
    const int wlo_min = __builtin_amdgcn_readfirstlane(wave_active ? wq0 - a.pos[wq0] : 0);
    const int wlo_max = __builtin_amdgcn_readfirstlane(wave_active ? wq_last - a.pos[wq_last] : 0);

    // Q fragments (k operand of S^T = K Q^T), rotated in registers.  Chunk kk holds
    // d in [16kk + 8hb, +8); chunk kk + NKK/2 holds the RoPE partners d + D/2.  A rotated value
    // beyond fp16's range (|q| above 65504 / sqrt(2) can give one) sets the range flag.
    f16x8 qf[NKK];
    {
        float qmax = 0.f;
        const bf16 *qrow = a.q + ((int64_t)(qvalid ? i : q_start) * a.hq + h) * D;
        const float2 *cs = a.rope + (int64_t)(qvalid ? i : q_start) * (D / 2);
#pragma unroll
        for (int kk = 0; kk < NKK / 2; ++kk) {
            const int d0 = 16 * kk + 8 * hb;
            const bf16x8 x1 = load_bf16x8(qrow + d0);
            const bf16x8 x2 = load_bf16x8(qrow + d0 + D / 2);
            f16x8 y1, y2;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const float2 f = cs[d0 + s];
                const float a1 = (float)x1[s], a2 = (float)x2[s];
                const float b1 = qvalid ? a1 * f.x - a2 * f.y : 0.f, b2 = qvalid ? a2 * f.x + a1 * f.y : 0.f;
                qmax = fmaxf(qmax, fmaxf(fabsf(b1), fabsf(b2)));
                y1[s] = (f16)b1;
                y2[s] = (f16)b2;
            }
            qf[kk] = y1;
            qf[kk + NKK / 2] = y2;
        }
        if (__builtin_expect(!(qmax <= 65504.f), 0)) atomicOr(a.flags, PK_META_FP16_RANGE);
    }

    float mref = -INFINITY;  // reference max of this query's scaled scores (log2 domain)
    float neg_m = 0.f;       // -mref, or 0 while mref is -inf (the exponent offset of p)
    float thr = -INFINITY;   // (mref + 8) / c: a raw score above it moves the reference
    float l = 0.f;           // running sum of exp2(s*c - mref) over this lane's half of the keys
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = zero_f32x16();

    const int kb_hi = ((q_end - 1) / BK) * BK;
    const int kb_lo = (kv_start / BK) * BK;

    // Per-lane LDS byte offsets, fixed for the kernel, so that every tile read in the loop is a
    // register plus an immediate: aoff[kk] is the 16-byte chunk of key row row_perm(n32) for
    // d in [16kk + 8hb, +8) (rows 32.. add 64 D bytes); toff are the transposed V^T reads.
    uint32_t aoff[NKK], toff[NDB][2];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) aoff[kk] = 2 * tile_off<D>(row_perm(n32), 16 * kk + 8 * hb);
    tile_tr_offsets<D>(toff);
    const uint32_t loff = tile_copy_lane_off<D>((int64_t)a.hkv * D);

    // K_rot / V tiles stream into double-buffered swizzled LDS tiles with asynchronous
    // global->LDS copies: tile t+1 is in flight while tile t is computed, one barrier per tile.
    // Rows past T are clamped to row T-1 (finite data; the causal mask zeroes their weight).
    // Whole tiles (every tile but possibly the first, the one holding row T - 1) are addressed
    // from running pointers that step back one tile per issue, so an issue costs a 64-bit
    // subtraction instead of a multiply.
    const int64_t tstride = (int64_t)BK * a.hkv * D;
    const int T32 = (int)T;   // (T <= PK_MAX_TOKENS: a 32-bit test is a scalar compare, a 64-bit
                              // signed one takes vector instructions on this target)
    const f16 *kp = a.krot + ((int64_t)kb_hi * a.hkv + kvh) * D;
    const f16 *vp = a.v + ((int64_t)kb_hi * a.hkv + kvh) * D;
    auto issue_tile = [&](int k0, int buf) {
        if (k0 + BK <= T32) {
            tile_copy_async_whole<D, BK, 4>(lds_k[buf], kp, (int64_t)a.hkv * D, loff);
            tile_copy_async_whole<D, BK, 4>(lds_v[buf], vp, (int64_t)a.hkv * D, loff);
        } else {
            tile_issue<D, BK>(lds_k[buf], a.krot, a.hkv, kvh, k0, T, loff);
            tile_issue<D, BK>(lds_v[buf], a.v, a.hkv, kvh, k0, T, loff);
        }
        kp -= tstride;
        vp -= tstride;
    };

    auto tile = [&](auto bufc, int k0) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        const char *tk = reinterpret_cast<const char *>(lds_k[BUF]);
        const char *tv = reinterpret_cast<const char *>(lds_v[BUF]);
        if (k0 > wq_last) return;            // every key is after every query of the wave
        if (k0 + BK - 1 < wlo_min) return;   // every key is before the wave's first sequence
        const bool need_mask = !(k0 + BK - 1 <= wq0 && k0 >= wlo_max);

        // S^T (keys x queries), key rows in row_perm order
        f32x16 s[NMB];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) s[mb] = zero_f32x16();
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
                s[mb] = mfma32(*reinterpret_cast<const f16x8 *>(tk + aoff[kk] + 64 * D * mb), qf[kk], s[mb]);
        // K operands issued four products ahead of their use
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int m = 0; m < NKK * NMB - 4; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        // Online softmax in the exp2 domain.  The running max is kept on the raw scores; the
        // scale * log2(e) factor is folded into one FMA per score: p = exp2(s*c - m*c).
        // Masking runs only on tiles that straddle a boundary or the diagonal (a uniform branch).
        if (need_mask) {
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int j = k0 + 32 * mb + row_perm(acc_row(rr, hb));
                    const bool keep = qvalid & (j >= lo_i) & (j <= i);
                    s[mb][rr] = keep ? s[mb][rr] : -INFINITY;
                }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) tmax = fmaxf(tmax, s[mb][rr]);
        tmax = half_swap_max(tmax);
        // Lazy rescaling: the reference max mref (log2 domain) only moves when a row's max
        // exceeds it by more than 8, so p = exp2(s*c - mref) <= 256 (exact enough in fp32 and
        // fp16) and the O rescale is skipped for the whole wave on most tiles.  The test is made
        // on the raw maximum against a threshold kept with mref, so a tile that does not move it
        // spends one compare.
        const bool bump = tmax > thr;
        if (__builtin_amdgcn_ballot_w64(bump)) {
            const float mnew = bump ? tmax * a.scale_log2 : mref;
            const float alpha = fast_exp2(mref - mnew);   // mref = -inf gives 0
            l *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] *= alpha;
            mref = mnew;
            neg_m = mref == -INFINITY ? 0.f : -mref;
            thr = (mref + 8.f) * a.inv_scale_log2;
        }
        // P in fp16 (the k operand of the second product); l sums the same fp16 weights, two at
        // a time with v_dot2_f32_f16 against (1, 1)
        f16x8 pb[NMB][2];
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        const f16x2 ones = {(f16)1.0f, (f16)1.0f};
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int x = 0; x < 8; ++x)
                    pb[mb][e][x] = (f16)fast_exp2(fmaf(s[mb][8 * e + x], a.scale_log2, neg_m));
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const f16x2 pair = {pb[mb][e][2 * x], pb[mb][e][2 * x + 1]};
                    l = __builtin_amdgcn_fdot2(pair, ones, l, false);
                }

        // O^T (d x queries) += V^T (d x keys) * P^T (keys x queries); V^T read transposed
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    o[db] = mfma32(tile_tr_at(tv, toff[db], 2 * D * (32 * mb + 16 * e)), pb[mb][e], o[db]);
            }
        }
        // V^T operands issued two products ahead of their use
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int m = 0; m < 2 * NMB * NDB - 2; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    };

    // the loop is unrolled by two so that the buffer of each step is a compile-time constant
    auto step = [&](auto bufc, int k0) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        lds_copy_wait();
        __syncthreads();
        if (k0 - BK >= kb_lo) issue_tile(k0 - BK, BUF ^ 1);
        if (wave_active) tile(bufc, k0);
    };
    issue_tile(kb_hi, 0);
    for (int k0 = kb_hi; k0 >= kb_lo; k0 -= 2 * BK) {
        step(std::integral_constant<int, 0>(), k0);
        if (k0 - BK >= kb_lo) step(std::integral_constant<int, 1>(), k0 - BK);
    }

    // epilogue: O = O^T / l, lse = ln(sum) of the scaled scores
    const float l_tot = half_swap_sum(l);
    if (qvalid) {
        const float inv = 1.f / l_tot;
        bf16 *orow = a.out + ((int64_t)i * a.hq + h) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = 32 * db + 8 * g4 + 4 * hb;
                uint2 raw;
                raw.x = pack_bf16x2((bf16)(o[db][4 * g4 + 0] * inv), (bf16)(o[db][4 * g4 + 1] * inv));
                raw.y = pack_bf16x2((bf16)(o[db][4 * g4 + 2] * inv), (bf16)(o[db][4 * g4 + 3] * inv));
                *reinterpret_cast<uint2 *>(orow + d) = raw;
            }
        }
        if (hb == 0) a.lse[(int64_t)h * T + i] = (mref + log2f(l_tot)) * kLn2;
    }
}

}  // namespace

namespace pk {

hipError_t launch_fwd(const AttnShape &sh, const pk_meta_s &m, const void *q, const void *krot,
                      const void *v, const void *rope, void *out, float *lse, hipStream_t s) {
    FwdArgs a;
    a.q = (const bf16 *)q;
    a.krot = (const f16 *)krot;
    a.v = (const f16 *)v;
    a.rope = (const float2 *)rope;
    a.items = m.fwd_items;
    a.pos = m.pos;
    a.hdr = m.hdr;
    a.flags = m.hdr + 2;
    a.out = (bf16 *)out;
    a.lse = lse;
    a.T = sh.T;
    a.hq = sh.hq;
    a.hkv = sh.hkv;
    a.group = sh.hq / sh.hkv;
    a.scale_log2 = sh.scale * pkd::kLog2e;
    a.inv_scale_log2 = (float)(1.0 / ((double)sh.scale * 1.4426950408889634));
    const unsigned grid = (unsigned)sh.n_items * (unsigned)sh.hq;
    const bool small = grid <= 2048;   // a few rounds of workgroups on a 256-CU device
    if (sh.d == 128) {
        if (small)
            k_attn_fwd<128, 64><<<grid, 256, 0, s>>>(a);
        else
            k_attn_fwd<128, 32><<<grid, 256, 0, s>>>(a);
    } else {
        if (small)
            k_attn_fwd<64, 64><<<grid, 256, 0, s>>>(a);
        else
            k_attn_fwd<64, 32><<<grid, 256, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace pk
