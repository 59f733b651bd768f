// Backward attention over a packed batch on gfx950 matrix cores: what the two kernels share.
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
// Two kernels, neither with atomics on the results (the only atomics are a persistent launch's
// work counters), so every gradient is written exactly once (and, when the caller's workspace
// holds it, a dS store that hands dS from the first kernel to the second):
//   k_attn_bwd_kv  one workgroup per backward work item (128 keys) x KV head (on packs with more
//                  of these units than the device holds workgroups at once, a persistent grid that
//                  takes them from per-XCD work counters, pk_device.h), 8 waves split by
//                  role over four 32-key sub-tiles; K_rot and V of a sub-tile's keys are the k
//                  operands of S = Q K^T and dP = dO V^T (v_mfma_f32_32x32x16_f16), dK^T and dV^T
//                  accumulate in registers over every query block AND every query head of the
//                  GQA group (so the group sum is free), and dK, dV are written once.  Query blocks of 64 rows stream
//                  into double-buffered swizzled LDS tiles by asynchronous global->LDS copies;
//                  the transposed operands of dV^T += dO^T P and dK^T += Q^T dS are read with
//                  ds_read_b64_tr_b16 from the same row-major tiles.
//   k_attn_bwd_q   one workgroup per forward work item (128 queries) x query head, laid out like
//                  the forward: S^T = K Q^T and dP^T = V dO^T give each lane one query, so its
//                  lse and D are per-lane scalars; dQ^T += K^T dS^T accumulates in registers and
//                  dQ is rotated back by R(-theta) and written once.
// dQ needs dS summed over keys, while k_attn_bwd_kv holds it laid out for sums over queries.
// With a dS store, k_attn_bwd_kv writes its fp16 dS^T blocks and k_attn_bwd_q computes
// dQ^T = K^T dS^T from them (one product, streaming dS from HBM; ds_read_b64_tr_b16 does the
// transpose on the way out of LDS).  Without one, k_attn_bwd_q recomputes S and dP (two extra
// products).  Either replaces float atomics on dQ (whose throughput, about 2.6 TB/s on this
// part, made them slower than the recompute), a zero-fill of dq and a separate inverse-rotation
// pass.
//
// Common to both: the mask is applied element-wise only on tiles that straddle a sequence
// boundary or the diagonal, and tiles outside a wave's visible range skip their products;
// operands are fp16 with fp32 accumulation; dout and v enter scaled by the powers of two sigma
// and tau the prologue chose (max|dout| * sigma and max|v| * tau in [1, 2)), so dP and dS are
// scaled by sigma tau (|sigma tau dS| < 8 d, inside fp16 for any finite input), dV by sigma, and
// the results are unscaled exactly when written.  Q_rot is stored times scale * log2(e) (one fp16
// rounding of the scaled value, as precise as rounding Q_rot itself), and the score and dP
// products start from the per-row values -lse * log2(e) and -sigma D, so they end as the
// exponent of P and as sigma (dP - D) with no further arithmetic.
//
// k_attn_bwd_kv lives in pk_bwd_kv.hip and k_attn_bwd_q in pk_bwd_q.hip (separate sources so
// each can be built with the machine scheduler that suits it).
#pragma once

#include "pk_internal.h"
#include "pk_device.h"

namespace pkb {

using namespace pkd;

struct BwdArgs {
    const f16 *qrot;      // [T, hq, D] fp16, R(q) * scale * log2(e)
    const f16 *krot;      // [T, hkv, D] fp16
    const f16 *v;         // [T, hkv, D] tau * v, fp16
    const f16 *dout16;    // [T, hq, D] sigma * dout, fp16
    const float *lse2;    // [hq, T] -lse * log2(e)
    const float *dsum;    // [hq, T] -sigma * tau * rowsum(dout * out)
    const float *dscale;  // {sigma, 1/sigma, tau, 1/(sigma tau)}
    const float2 *rope;   // [T, D/2]
    const int32_t *items; // [n_items, 8] longest first (backward list for _kv, forward for _q)
    const int32_t *pos;   // [T]
    const int32_t *hdr;   // [3] = blocks of the pack's dS store
    f16 *ds;              // the dS store (null: none), see PK_DS_BLOCK_ROWS
    const int32_t *ds_off;// [n_items + 1] first block of each key tile (tile order)
    int64_t ds_cap;       // blocks (of all hq heads) the store can hold
    float *dq;            // [T, hq, D]
    float *dk;            // [T, hkv, D]
    float *dv;            // [T, hkv, D]
    int32_t *sched;       // per-launch work counters of a persistent launch
    int64_t T;
    int hq, hkv, group, n_items;
    float scale;
};

inline BwdArgs make_bwd_args(const pk::AttnShape &sh, const pk_meta_s &m, const void *qrot,
                             const void *krot, const void *v, const void *dout16,
                             const float *lse2, const float *dsum, const float *scale,
                             const void *rope, float *dq, float *dk, float *dv) {
    BwdArgs a;
    a.qrot = (const f16 *)qrot;
    a.krot = (const f16 *)krot;
    a.v = (const f16 *)v;
    a.dout16 = (const f16 *)dout16;
    a.lse2 = lse2;
    a.dsum = dsum;
    a.dscale = scale;
    a.rope = (const float2 *)rope;
    a.items = nullptr;
    a.pos = m.pos;
    a.hdr = m.hdr;
    a.ds = nullptr;
    a.ds_off = m.ds_off;
    a.ds_cap = 0;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.sched = nullptr;
    a.T = sh.T;
    a.hq = sh.hq;
    a.hkv = sh.hkv;
    a.group = sh.hq / sh.hkv;
    a.n_items = sh.n_items;
    a.scale = sh.scale;
    return a;
}

// Layout of one stored block (128 keys x 64 queries, fp16, 16 KB): 16 chunks of 1 KB, chunk
// c = 4 s + 2 hf + e for the 32-key sub-tile s, the 32-query half hf and e; inside a chunk,
// lane l = n + 32 b holds the 8 queries 32 hf + 16 e + 8 b .. + 7 of key 32 s + n (16 bytes at
// 16 l).  That is the order in which the dK/dV kernel's dS waves hold dS (one 1 KB store per
// (hf, e)); the dQ kernel gathers the 16-byte pieces into a row-major [key][query] LDS tile.
__device__ __forceinline__ int ds_piece_offset(int key, int qchunk) {   // halves, in a block
    const int s = key >> 5, n = key & 31, hf = qchunk >> 2, e = (qchunk >> 1) & 1, b = qchunk & 1;
    return ((4 * s + 2 * hf + e) * 64 + n + 32 * b) * 8;
}

// The dS store is used when the caller gave one that holds the pack's blocks (a wave-uniform
// test on the meta's block total; both kernels reach the same decision).
__device__ __forceinline__ bool ds_stored(const BwdArgs &a) {
    return a.ds != nullptr && (int64_t)a.hdr[3] <= a.ds_cap;
}

}  // namespace pkb
