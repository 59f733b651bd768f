// dQ of the packed attention backward (query-tile outer, from the dS store or recomputing S and
// dP); the math and the conventions shared with the dK/dV kernel are described in pk_bwd.h.
#include <type_traits>

#include "pk_bwd.h"

namespace {

using namespace pkd;
using pkb::BwdArgs;

// ------------------------------------------------------------------------------------------
// dQ: query-tile outer
// ------------------------------------------------------------------------------------------
template <int D>
__device__ void q_zero_tile(const BwdArgs &a, int tile, int h) {
    const int64_t r0 = (int64_t)tile * PK_TILE_ROWS;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int e = threadIdx.x; e < PK_TILE_ROWS * (D / 4); e += blockDim.x) {
        const int64_t i = r0 + e / (D / 4);
        if (i < a.T) *reinterpret_cast<float4 *>(a.dq + (i * a.hq + h) * D + (e % (D / 4)) * 4) = z;
    }
}

// dQ = R(-theta) (scale / (sigma tau) * dQ_rot) of this lane's query, written once; acc holds
// dQ_rot^T (rows d, this lane's query column).
template <int D>
__device__ __forceinline__ void q_epilogue(const BwdArgs &a, int i, int h, const f32x16 (&acc)[D / 32]) {
    constexpr int NDB = D / 32;
    const int hb = (threadIdx.x & 63) >> 5;
    float *row = a.dq + ((int64_t)i * a.hq + h) * D;
    const float2 *cs = a.rope + (int64_t)i * (D / 2);
    const float qscale = a.scale * a.dscale[3];   // dS carries sigma * tau
#pragma unroll
    for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int d = 32 * db + 8 * g4 + 4 * hb;  // first half; partner d + D/2
            float y1[4], y2[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float2 f = cs[d + x];
                const float x1 = acc[db][4 * g4 + x] * qscale;
                const float x2 = acc[db + NDB / 2][4 * g4 + x] * qscale;
                y1[x] = x1 * f.x + x2 * f.y;
                y2[x] = x2 * f.x - x1 * f.y;
            }
            *reinterpret_cast<float4 *>(row + d) = make_float4(y1[0], y1[1], y1[2], y1[3]);
            *reinterpret_cast<float4 *>(row + d + D / 2) = make_float4(y2[0], y2[1], y2[2], y2[3]);
        }
}

// dQ from the dS store.  Per step of 64 keys (from the diagonal down), the K_rot tile
// [64 keys][D] and, for each of the item's two 64-query blocks, the dS^T tile [64 keys][64
// queries] of key tile u = k0 / 128 are copied into LDS (global_load_lds: the dS pieces are
// gathered from the stored register order into row-major swizzled tiles); each wave takes the
// tile of its own 32 queries and accumulates dQ^T += K^T dS^T, both operands read transposed
// (ds_read_b64_tr_b16).  dS streams from HBM and is read once, so its copies run two steps ahead
// in three LDS buffers (K, an L2 hit, one step ahead in two): vmcnt counts the copies in issue
// order, and each step's K copies are issued before the dS copies of two steps later, so waiting
// for one step's K leaves the later dS in flight.  The store already holds the mask (masked
// pairs have P = 0, so dS = 0), and a wave skips the keys none of its queries sees exactly as
// the recomputing path does, so it only reads blocks the dK/dV kernel wrote; a block the tile
// pair does not have is replaced by an in-bounds dummy copy into a tile no wave reads.
template <int D>
__device__ __forceinline__ void q_from_store(const BwdArgs &a, char *lds, const int32_t *it, int h,
                                             int kvh) {
    constexpr int BK = 64, BQ = PK_DS_BLOCK_ROWS, NDB = D / 32;
    constexpr int BLK = PK_TILE_ROWS * BQ;   // halves per stored block
    constexpr int NSB = 3;                   // dS buffers (copies two steps ahead)
    f16 *lds_k = reinterpret_cast<f16 *>(lds);                       // [2][BK * D]
    f16 *lds_s = reinterpret_cast<f16 *>(lds + 2 * BK * D * 2);      // [NSB][2][BK * BQ]
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n32 = lane & 31;
    const int q_start = it[0], q_end = it[1], kv_start = it[2];
    const int t = q_start / PK_TILE_ROWS;
    const int64_t T = a.T;
    const int i = q_start + 32 * w + n32;
    const bool qvalid = i < q_end;
    const int wq0 = q_start + 32 * w;
    const bool wave_active = wq0 < q_end;
    const int wq_last = min(wq0 + 31, q_end - 1);
    const int wlo_min = __builtin_amdgcn_readfirstlane(wave_active ? wq0 - a.pos[wq0] : 0);

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = zero_f32x16();

    const int kb_hi = ((q_end - 1) / BK) * BK;
    const int kb_lo = (kv_start / BK) * BK;
    const int n_steps = (kb_hi - kb_lo) / BK + 1;
    uint32_t toff[NDB][2], soff[BQ / 32][2];
    tile_tr_offsets<D>(toff);
    tile_tr_offsets<BQ>(soff);
    const uint32_t loff = tile_copy_lane_off<D>((int64_t)a.hkv * D);
    // gather offsets of the dS tiles: LDS run R (rows 8R .. 8R + 7 of a [64 keys][64 queries]
    // swizzled tile) is filled by wave R % 4; lane l takes physical chunk l % 8 of row 8R + l / 8,
    // i.e. query chunk (l % 8) ^ swz(row), from the stored block's register order.  Runs R and
    // R + 4 are 32 keys (one sub-tile, 2048 halves) apart with the same swizzle.
    uint32_t loff_s;
    {
        const int row = 8 * w + lane / 8;
        loff_s = 2u * (uint32_t)pkb::ds_piece_offset(row, (lane % 8) ^ swz<BQ>(row));
    }
    const int64_t tstride = (int64_t)BK * a.hkv * D;
    const f16 *kp = a.krot + ((int64_t)kb_hi * a.hkv + kvh) * D;
    auto issue_k = [&](int sidx, int buf) {
        const int k0 = kb_hi - BK * sidx;
        if (k0 + BK <= (int)T)
            tile_copy_async_whole<D, BK, 4>(lds_k + buf * BK * D, kp, (int64_t)a.hkv * D, loff);
        else
            tile_issue<D, BK>(lds_k + buf * BK * D, a.krot, a.hkv, kvh, k0, T, loff);
        kp -= tstride;
    };
    // the two dS^T tiles of step sidx: blocks m0, m0 + 1 of key tile u that exist in the store
    // (the tile's offsets come from scalar loads: constant address space)
    auto issue_s = [&](int sidx, int buf) {
        const int k0 = kb_hi - BK * sidx;
        const int u = __builtin_amdgcn_readfirstlane(k0 / PK_TILE_ROWS);
        const __attribute__((address_space(4))) int32_t *offs =
            (const __attribute__((address_space(4))) int32_t *)a.ds_off;
        const int off_u = offs[u], nb = offs[u + 1] - off_u;
        const int m0 = 2 * (t - u);
        // key half (k0 % 128) / 64 = sub-tiles 2, 3 of the block: chunks from 4096 halves on.
        // Every step issues exactly 4 copies per wave (the waits count on it): a block the tile
        // pair does not have is replaced by block 0 of the store, into a tile no wave reads.
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int64_t b = (m0 + x < nb) ? (int64_t)(off_u + m0 + x) * a.hq + h : 0;
            const f16 *bs = a.ds + b * BLK + (k0 % PK_TILE_ROWS) * 64;
            const uint32_t dst = lds_addr(lds_s + (2 * buf + x) * BK * BQ) + 1024u * w;
            lds_dma_s<16>(bs, loff_s, dst);
            lds_dma_s<16>(bs + 2048, loff_s, dst + 4096u);
        }
    };
    auto tile = [&](auto kbufc, auto sbufc, int k0) __attribute__((always_inline)) {
        constexpr int KB = decltype(kbufc)::value, SB = decltype(sbufc)::value;
        if (k0 > wq_last) return;            // every key is after every query of the wave
        if (k0 + BK - 1 < wlo_min) return;   // every key is before the wave's first sequence
        const char *tk = reinterpret_cast<const char *>(lds_k + KB * BK * D);
        const char *ts = reinterpret_cast<const char *>(lds_s + (2 * SB + (w >> 1)) * BK * BQ);
#pragma unroll
        for (int kq = 0; kq < BK / 16; ++kq) {
            const f16x8 sb = tile_tr_at(ts, soff[w & 1], 2 * BQ * 16 * kq);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                acc[db] = mfma32(tile_tr_at(tk, toff[db], 2 * D * 16 * kq), sb, acc[db]);
        }
        // operands (one dS^T and NDB K^T reads per 16 keys, two instructions each) issued a few
        // products ahead of their use
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int m = 0; m < (BK / 16) * NDB; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        }
    };
    // step sidx (buffers: K sidx % 2, dS sidx % 3, compile-time through the unrolled loop):
    // in flight at its start are K(sidx) and dS(sidx), dS(sidx + 1), issued in the order
    // dS(sidx), K(sidx), dS(sidx + 1); waiting until only dS(sidx + 1)'s copies (4 per wave,
    // when issued) remain completes the first two.
    auto step = [&](auto stepc, int sidx) __attribute__((always_inline)) {
        constexpr int J = decltype(stepc)::value;   // sidx % 6
        if (sidx + 1 < n_steps)
            lds_copy_wait_keep<4>();
        else
            lds_copy_wait();
        __syncthreads();
        if (sidx + 1 < n_steps) issue_k(sidx + 1, (J + 1) % 2);
        if (sidx + 2 < n_steps) issue_s(sidx + 2, (J + 2) % NSB);
        if (wave_active)
            tile(std::integral_constant<int, J % 2>(), std::integral_constant<int, J % NSB>(), kb_hi - BK * sidx);
    };
    issue_s(0, 0);
    issue_k(0, 0);
    if (1 < n_steps) issue_s(1, 1);
    for (int sidx = 0; sidx < n_steps; sidx += 6) {
        step(std::integral_constant<int, 0>(), sidx);
        if (sidx + 1 < n_steps) step(std::integral_constant<int, 1>(), sidx + 1);
        if (sidx + 2 < n_steps) step(std::integral_constant<int, 2>(), sidx + 2);
        if (sidx + 3 < n_steps) step(std::integral_constant<int, 3>(), sidx + 3);
        if (sidx + 4 < n_steps) step(std::integral_constant<int, 4>(), sidx + 4);
        if (sidx + 5 < n_steps) step(std::integral_constant<int, 5>(), sidx + 5);
    }
    if (qvalid) q_epilogue<D>(a, i, h, acc);
}

// LDS of the dQ kernel: the recomputing path's K and V tiles, or the stored path's K and dS
// tiles, in one buffer.
template <int D>
constexpr int q_lds_bytes() {
    constexpr int recompute = 2 * 2 * 64 * D * 2, stored = 2 * 64 * D * 2 + 3 * 2 * 64 * PK_DS_BLOCK_ROWS * 2;
    return recompute > stored ? recompute : stored;
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_attn_bwd_q(BwdArgs a) {
    constexpr int BK = 64;        // keys per LDS tile
    constexpr int NKK = D / 16, NDB = D / 32, NMB = BK / 32;
    __shared__ __attribute__((aligned(16))) char lds_raw[q_lds_bytes<D>()];
    f16 (*lds_k)[BK * D] = reinterpret_cast<f16 (*)[BK * D]>(lds_raw);                   // [2][BK * D]
    f16 (*lds_v)[BK * D] = reinterpret_cast<f16 (*)[BK * D]>(lds_raw + 2 * BK * D * 2);  // [2][BK * D]

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: lets bounds live in SGPRs
    const int n32 = lane & 31, hb = lane >> 5;
    int r, h;
    item_head_of_block(blockIdx.x, a.hq, a.hkv, r, h);
    const int kvh = h / a.group;
    const int32_t *it = a.items + (int64_t)r * PK_ITEM_FIELDS;
    if (a.hdr[0] != 0) {
        q_zero_tile<D>(a, it[7], h);
        return;
    }
    if (pkb::ds_stored(a)) {
        q_from_store<D>(a, lds_raw, it, h, kvh);
        return;
    }
    const int q_start = it[0], q_end = it[1], kv_start = it[2];
    const int64_t T = a.T;

    // this lane's query and its wave's query range
    const int i = q_start + 32 * w + n32;
    const bool qvalid = i < q_end;
    const int ii = qvalid ? i : q_start;
    const int lo_i = qvalid ? i - a.pos[i] : 0;
    const int wq0 = q_start + 32 * w;
    const bool wave_active = wq0 < q_end;
    const int wq_last = min(wq0 + 31, q_end - 1);
    const int wlo_min = __builtin_amdgcn_readfirstlane(wave_active ? wq0 - a.pos[wq0] : 0);
    const int wlo_max = __builtin_amdgcn_readfirstlane(wave_active ? wq_last - a.pos[wq_last] : 0);
    const float nlse2 = qvalid ? a.lse2[(int64_t)h * T + i] : -INFINITY;   // -lse * log2(e)
    const float dd = qvalid ? a.dsum[(int64_t)h * T + i] : 0.f;

    // Q_rot and sigma * dout of this lane's query as k operands (d in [16kk + 8hb, +8))
    f16x8 qf[NKK], gf[NKK];
    {
        const int64_t row = ((int64_t)ii * a.hq + h) * D + 8 * hb;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            qf[kk] = qvalid ? load_f16x8(a.qrot + row + 16 * kk) : zero_f16x8();
            gf[kk] = qvalid ? load_f16x8(a.dout16 + row + 16 * kk) : zero_f16x8();
        }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            settle(qf[kk]);
            settle(gf[kk]);
        }
        settle(nlse2);
        settle(dd);
        settle(lo_i);
    }
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = zero_f32x16();
    // -sigma D (as stored) in every result register: the dP product starts from it, so it
    // yields sigma (dP - D) directly
    // and -lse * log2(e) likewise for the score product: with Q_rot carrying scale * log2(e) it
    // ends as the exponent of P
    f32x16 ndd, nls;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        ndd[r] = dd;
        nls[r] = nlse2;
    }

    const int kb_hi = ((q_end - 1) / BK) * BK;
    const int kb_lo = (kv_start / BK) * BK;

    // Per-lane LDS byte offsets, fixed for the kernel: aoff[kk] is the 16-byte chunk of key row
    // row_perm(n32) for d in [16kk + 8hb, +8) (rows 32.. add 64 D bytes); toff the K^T reads.
    uint32_t aoff[NKK], toff[NDB][2];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) aoff[kk] = 2 * tile_off<D>(row_perm(n32), 16 * kk + 8 * hb);
    tile_tr_offsets<D>(toff);
    const uint32_t loff = tile_copy_lane_off<D>((int64_t)a.hkv * D);

    // K_rot / V tiles stream into double-buffered swizzled LDS tiles with asynchronous
    // global->LDS copies (rows past T clamped to T-1; their weight is masked to zero)
    // Whole tiles (every tile but possibly the first, the one holding row T - 1) are addressed
    // from running pointers that step back one tile per issue.
    const int64_t tstride = (int64_t)BK * a.hkv * D;
    const f16 *kp = a.krot + ((int64_t)kb_hi * a.hkv + kvh) * D;
    const f16 *vp = a.v + ((int64_t)kb_hi * a.hkv + kvh) * D;
    auto issue_tile = [&](int k0, int buf) {
        if (k0 + BK <= (int)T) {
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
        if (k0 > wq_last) return;            // every key is after every query of the wave
        if (k0 + BK - 1 < wlo_min) return;   // every key is before the wave's first sequence
        const bool need_mask = !(k0 + BK - 1 <= wq0 && k0 >= wlo_max);
        const char *tk = reinterpret_cast<const char *>(lds_k[BUF]);
        const char *tv = reinterpret_cast<const char *>(lds_v[BUF]);

        // per 32-key block mb: S^T = K Q^T and dP^T = V dO^T, dS^T, then dQ^T += K^T dS^T
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            f32x16 sc = nls, dp = ndd;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                sc = mfma32(*reinterpret_cast<const f16x8 *>(tk + aoff[kk] + 64 * D * mb), qf[kk], sc);
                dp = mfma32(*reinterpret_cast<const f16x8 *>(tv + aoff[kk] + 64 * D * mb), gf[kk], dp);
            }
            // K and V operands issued 2 products ahead of their use
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int m = 0; m < 2 * NKK - 2; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (need_mask) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int jj = k0 + 32 * mb + row_perm(acc_row(rr, hb));
                    const bool keep = qvalid & (jj >= lo_i) & (jj <= i);
                    sc[rr] = keep ? sc[rr] : -INFINITY;
                }
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                f16x8 sb;
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const float p = fast_exp2(sc[8 * e + x]);
                    sb[x] = (f16)(p * dp[8 * e + x]);
                }
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    acc[db] = mfma32(tile_tr_at(tk, toff[db], 2 * D * (32 * mb + 16 * e)), sb, acc[db]);
            }
            // K^T operands issued two products ahead of their use
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int m = 0; m < 2 * NDB - 2; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
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

    if (qvalid) q_epilogue<D>(a, i, h, acc);
}

}  // namespace

namespace pk {

hipError_t launch_bwd_q(const AttnShape &sh, const pk_meta_s &m, const void *qrot,
                        const void *krot, const void *v, const void *dout16, const float *lse2,
                        const float *dsum, const float *scale, const void *rope, float *dq,
                        const DsStore &ds, hipStream_t s) {
    BwdArgs a = pkb::make_bwd_args(sh, m, qrot, krot, v, dout16, lse2, dsum, scale, rope, dq,
                                   nullptr, nullptr);
    a.items = m.fwd_items;
    a.ds = (f16 *)ds.ptr;
    a.ds_cap = ds.cap_blocks;
    const unsigned grid = (unsigned)sh.n_items * (unsigned)sh.hq;
    if (sh.d == 128)
        k_attn_bwd_q<128><<<grid, 256, 0, s>>>(a);
    else
        k_attn_bwd_q<64><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace pk
