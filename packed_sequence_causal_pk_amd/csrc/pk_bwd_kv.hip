// dK and dV of the packed attention backward (key-tile outer); the math and the conventions
// shared with the dQ kernel are described in pk_bwd.h.
#include <type_traits>

#include "pk_bwd.h"

namespace {

using namespace pkd;
using pkb::BwdArgs;

// ------------------------------------------------------------------------------------------
// dK, dV: key-tile outer
// ------------------------------------------------------------------------------------------
template <int D>
struct KvSmem {
    static constexpr int BQ = 64;        // query rows per block
    float lse2[2][BQ];   // -lse * log2(e) of the block's rows (double-buffered like the tiles)
    float dd[2][BQ];     // -sigma * D_i
    int pos[2][BQ];      // position of each row inside its sequence
    f16 q[2][BQ * D];    // swizzled row-major Q_rot blocks
    f16 dO[2][BQ * D];   // swizzled row-major sigma * dout blocks
    // P of the current block handed from the P waves to the dS waves: [key wave][half][chunk c]
    // [lane][4] holds result registers 4c..4c+3 of that lane (conflict-free 16-byte accesses)
    float xp[4][2][4][64][4];
};

template <int D>
__device__ void kv_zero_tile(const BwdArgs &a, int tile, int kvh) {
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

// Start the asynchronous copy of one query block (rows [qb, qb + BQ) of head h) into buffer
// `buf` by the workgroup's 8 waves: Q_rot and sigma * dout tiles, and the per-row lse2, dd and
// pos.  A block whose rows all exist is addressed by scalar bases and the precomputed lane offset
// `loff`; the last block of a pack clamps its rows to T - 1 lane by lane (their weights are
// masked to zero).
template <int D>
__device__ __forceinline__ void kv_issue_block(const BwdArgs &a, KvSmem<D> &sm, int buf, int h,
                                               int qb, uint32_t loff) {
    using S = KvSmem<D>;
    const int tid = opaque_tid(), lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    tile_issue<D, S::BQ, 8>(sm.q[buf], a.qrot, a.hq, h, qb, a.T, loff);
    tile_issue<D, S::BQ, 8>(sm.dO[buf], a.dout16, a.hq, h, qb, a.T, loff);
    if (w == 0) {  // one wave: 64 rows x 4 bytes per array
        if (qb + S::BQ <= (int)a.T) {   // T <= PK_MAX_TOKENS; a 32-bit test stays scalar
            lds_dma_s<4>(a.lse2 + (int64_t)h * a.T + qb, 4u * lane, lds_addr(sm.lse2[buf]));
            lds_dma_s<4>(a.dsum + (int64_t)h * a.T + qb, 4u * lane, lds_addr(sm.dd[buf]));
            lds_dma_s<4>(a.pos + qb, 4u * lane, lds_addr(sm.pos[buf]));
        } else {
            const int64_t i = min((int64_t)(qb + lane), a.T - 1);
            lds_dma<4>(a.lse2 + (int64_t)h * a.T + i, lds_addr(sm.lse2[buf]));
            lds_dma<4>(a.dsum + (int64_t)h * a.T + i, lds_addr(sm.dd[buf]));
            lds_dma<4>(a.pos + i, lds_addr(sm.pos[buf]));
        }
    }
}

// 8 consecutive floats (or ints) of a per-row LDS array as two 16-byte reads.
template <typename T>
__device__ __forceinline__ void lds_row8(const T *p, T (&out)[8]) {
    typedef T v4 __attribute__((ext_vector_type(4)));
    const v4 x = reinterpret_cast<const v4 *>(p)[0], y = reinterpret_cast<const v4 *>(p)[1];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        out[c] = x[c];
        out[4 + c] = y[c];
    }
}

// Writes one row of dK taken back through the rotation, y = R(-theta) (s * acc).  The lane holds dims 32 db + 8 g4 + 4 hb .. + 3 of the first half in acc[db] and their partners
// (+ D/2) in acc[db + D/64].  Every cos/sin pair is loaded before the first store: the row and
// the table may alias as far as the compiler knows, so a load placed after a store is kept
// there, and its wait (vmcnt counts stores as well as loads) then also waits for the store --
// one memory round trip per 16 bytes written instead of one for the row.
template <int D>
__device__ __forceinline__ void store_rotated_back(float *row, const float2 *cs, float s, int hb,
                                                   const f32x16 (&acc)[D / 32]) {
    constexpr int NH = D / 64;   // 32-dim blocks per half
    float4 c[NH][4][2];
#pragma unroll
    for (int db = 0; db < NH; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const float4 *p = reinterpret_cast<const float4 *>(cs + 32 * db + 8 * g4 + 4 * hb);
            c[db][g4][0] = p[0];
            c[db][g4][1] = p[1];
        }
#pragma unroll
    for (int db = 0; db < NH; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int d = 32 * db + 8 * g4 + 4 * hb;
            const float cx[4] = {c[db][g4][0].x, c[db][g4][0].z, c[db][g4][1].x, c[db][g4][1].z};
            const float sx[4] = {c[db][g4][0].y, c[db][g4][0].w, c[db][g4][1].y, c[db][g4][1].w};
            float y1[4], y2[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float x1 = acc[db][4 * g4 + x] * s;
                const float x2 = acc[db + NH][4 * g4 + x] * s;
                y1[x] = x1 * cx[x] + x2 * sx[x];
                y2[x] = x2 * cx[x] - x1 * sx[x];
            }
            *reinterpret_cast<float4 *>(row + d) = make_float4(y1[0], y1[1], y1[2], y1[3]);
            *reinterpret_cast<float4 *>(row + d + D / 2) = make_float4(y2[0], y2[1], y2[2], y2[3]);
        }
}

// The work of one (key tile, KV head) item is split by role over 8 waves; waves w and w + 4 own
// the same 32 keys and share a SIMD:
//   P waves (0..3)   S = Q K^T, the mask, P = exp2(S scale log2e - lse2), hand P over in LDS,
//                    dV^T += dO^T P;
//   dS waves (4..7)  dP = dO V^T, dS = P (dP - D) with P from LDS, dK^T += Q^T dS.
// Each role holds one operand (K_rot or V) and one accumulator (dV or dK), so a wave needs
// about half the registers of doing both, two waves fit on every SIMD, and every product
// accumulates in ordinary VGPRs.  Per 64-row block the waves meet at two barriers:
//   B0: block data in LDS  ->  S, P (P waves) | dP (dS waves)  ->  B1: P in LDS  ->
//   dV (P waves) | dS, dK (dS waves)
// so each SIMD runs one wave's products while the other does its element-wise work.
//
// NS = 2 splits every item over two workgroups of 64 keys each, for packs whose grid of items x
// KV heads would leave compute units idle: a workgroup's 8 waves are then two 32-key sub-tiles
// x two roles x the two 32-row halves of each query block, each wave doing one half, and the
// two halves' partial dK, dV are summed through LDS at the end.  Each block costs a wave half
// the products, so the longest workgroup (which sets the time of a small pack) takes about half
// as long.
//
// One unit: backward item r (key tile), key half kh (NS = 2) and KV head kvh.  claim() is called
// as the last query block starts (persistent launches, pk_device.h).
template <int D, int NS, typename Claim>
__device__ __forceinline__ void kv_unit(const BwdArgs &a, KvSmem<D> &sm, int r, int kh, int kvh,
                                        Claim &&claim) {
    static_assert(NS == 1 || NS == 2, "an item on one or two workgroups");
    using S = KvSmem<D>;
    constexpr int BQ = S::BQ;
    constexpr int NKK = D / 16, NDB = D / 32;
    constexpr uint32_t HALF = 32 * D * 2;    // bytes from row 0 to row 32 of a tile

    const int tid = opaque_tid(), lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: lets bounds live in SGPRs
    const int w = wv & 3;              // P hand-off slot; with NS = 1 also the key sub-tile
    const bool p_role = wv < 4;
    const int n32 = lane & 31, hb = lane >> 5;
    const int sub = NS == 1 ? w : (w & 1);       // 32-key sub-tile of this wave
    const int hf_own = NS == 1 ? -1 : (w >> 1);  // with NS = 2: the query-block half of this wave
    const int32_t *it = a.items + (int64_t)r * PK_ITEM_FIELDS;
    if (a.hdr[0] != 0) {
        if (kh == 0) kv_zero_tile<D>(a, it[7], kvh);
        return;
    }
    const int kv_start = it[0], kv_end = it[1], q_end = it[3];
    const int key_base = kv_start + 64 * kh;     // first key of this workgroup
    if (key_base >= kv_end) return;              // (NS = 2) an item of 64 keys or fewer
    // Query blocks start at the first key of the workgroup: earlier rows see none of its keys.
    const int q_start = NS == 1 ? it[2] : it[2] + 64 * kh;
    const float inv_sigma = a.dscale[1];        // dV unscale
    const float inv_sigma_tau = a.dscale[3];    // dK unscale (dS carries sigma * tau)

    const int j = key_base + 32 * sub + n32;  // this lane's key
    const bool kvalid = j < kv_end;
    const int wk0 = key_base + 32 * sub;
    const bool wave_active = wk0 < kv_end;
    const int wk_last = min(wk0 + 31, kv_end - 1);

    const int nqb = (q_end - q_start + BQ - 1) / BQ;
    const int n_iter = a.group * nqb;
    // dS store: block (key tile u, query block m, head h) sits at block index
    // (ds_off[u] + m) * hq + h and holds dS of 128 keys x 64 queries in the register order of the
    // dS waves (layout in pk_bwd.h), so each store instruction writes 1 KB contiguous
    static_assert(BQ == PK_DS_BLOCK_ROWS, "dS store blocks are the kernel's query blocks");
    const bool store = pkb::ds_stored(a);
    f16 *ds_tile = store ? a.ds + (int64_t)a.ds_off[it[7]] * a.hq * (PK_TILE_ROWS * BQ) : nullptr;
    const int ds_sub = (j - kv_start) >> 5;           // 32-key sub-tile of the 128-key tile
    const int ds_lane = ds_sub * 2048 + 8 * lane;     // halves, inside a block
    const uint32_t loff = tile_copy_lane_off<D, 8>((int64_t)a.hq * D);
    // iteration itn: head (itn / nqb) of the group, query block (itn % nqb)
    auto iter_row = [&](int itn) { return q_start + (itn % nqb) * BQ; };
    auto iter_head = [&](int itn) { return kvh * a.group + itn / nqb; };
    kv_issue_block<D>(a, sm, 0, iter_head(0), iter_row(0), loff);

    // this role's operand of this lane's key: K_rot (P waves) or V (dS waves), as k operands
    // (d in [16kk + 8hb, +8))
    f16x8 kvf[NKK];
    {
        const f16 *src = p_role ? a.krot : a.v;
        const int64_t row = ((int64_t)(kvalid ? j : kv_start) * a.hkv + kvh) * D + 8 * hb;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) kvf[kk] = kvalid ? load_f16x8(src + row + 16 * kk) : zero_f16x8();
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) settle(kvf[kk]);
    }

    // Per-lane byte offsets inside a tile, fixed for the whole kernel so that every LDS read in
    // the loop is a register plus an immediate:
    //   aoff[kk]     row operand chunk of tile row row_perm(n32) (rows 32.. add HALF)
    //   toff[db][x]  the two ds_read_b64_tr_b16 of the transposed operand of columns 32 db ..
    uint32_t aoff[NKK], toff[NDB][2];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) aoff[kk] = 2 * tile_off<D>(row_perm(n32), 16 * kk + 8 * hb);
    tile_tr_offsets<D>(toff);

    f32x16 acc[NDB];   // dV^T (P waves) or dK_rot^T (dS waves): d rows x this wave's 32 keys
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = zero_f32x16();

    // The main loop, instantiated once per role so that each role's code and registers are
    // its own.
    auto main_loop = [&](auto rolec) __attribute__((always_inline)) {
    constexpr bool p_role = decltype(rolec)::value;
    // One 64-row block in buffer BUF.  Result register rr of the 32x32 products of half hf
    // belongs to block row 32 hf + 8 hb + (rr % 8) + 16 (rr / 8) (the row_perm order of the row
    // operand), so each lane's per-row values are two runs of 8 consecutive rows.
    auto block = [&](auto bufc, int qb, int itn) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        const char *cq = reinterpret_cast<const char *>(sm.q[BUF]);
        const char *cg = reinterpret_cast<const char *>(sm.dO[BUF]);
        const int nrows = min(BQ, q_end - qb);
        auto row_op = [&](const char *t, int kk, int hf) {
            return *reinterpret_cast<const f16x8 *>(t + aoff[kk] + hf * HALF);
        };
        // Per-half visibility (uniform): a half is skipped when it has no item rows or sees none
        // of this wave's keys, and masked element-wise unless all 32 rows see all 32 keys.  Both
        // roles of a key sub-tile reach the same decisions from the same LDS data.
        // (The four position reads are issued together and the tests combined without short
        // circuits, so the decision costs one LDS round trip and no branches.)
        bool run[2], masked[2];
        int pfirst[2], plast[2], rlast[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            rlast[hf] = 32 * hf + max(min(32, nrows - 32 * hf), 1) - 1;
            pfirst[hf] = sm.pos[BUF][32 * hf];
            plast[hf] = sm.pos[BUF][rlast[hf]];
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int r0 = 32 * hf, rl = rlast[hf];
            const int hrows = min(32, nrows - r0);
            const int lo_first = __builtin_amdgcn_readfirstlane(qb + r0 - pfirst[hf]);
            const int lo_last = __builtin_amdgcn_readfirstlane(qb + rl - plast[hf]);
            run[hf] = wave_active & (hrows > 0) & (qb + rl >= wk0) & (lo_first <= wk_last) &
                      (NS == 1 || hf == hf_own);
            masked[hf] = !((hrows == 32) & (qb + r0 >= wk0 + 31) & (lo_last <= wk0));
        }

        f32x16 sp[2];       // P waves: S then P; dS waves: dP
        f16x8 pb[2][2];     // fp16 k operands of the second products: P (P waves) or dS (dS waves)
        // the first product of half hf: S = Q K^T (P waves) or dP = dO V^T (dS waves).  Each
        // starts from a per-row value stored negated: the P waves from -lse * log2(e), so with
        // Q_rot carrying scale * log2(e) the product ends as the exponent of P; the dS waves from
        // -sigma D, so it ends as sigma (dP - D), the factor that multiplies P in dS.
        auto init_scores = [&](int hf) __attribute__((always_inline)) {
            const float *init = p_role ? sm.lse2[BUF] : sm.dd[BUF];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                float iv[8];
                lds_row8(&init[32 * hf + 16 * e + 8 * hb], iv);
#pragma unroll
                for (int x = 0; x < 8; ++x) sp[hf][8 * e + x] = iv[x];
            }
        };
        auto scores = [&](int hf) __attribute__((always_inline)) {
            const char *t = p_role ? cq : cg;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) sp[hf] = mfma32(row_op(t, kk, hf), kvf[kk], sp[hf]);
        };
        // P waves: P = exp2(S scale log2e - lse log2e) (masked when asked), stored for the dS
        // waves
        auto softmax = [&](int hf, bool msk) __attribute__((always_inline)) {
            float4 *xp = reinterpret_cast<float4 *>(&sm.xp[w][hf][0][lane][0]);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r8 = 32 * hf + 16 * e + 8 * hb;   // first row of this lane's 8
                int p8[8];
                if (msk) lds_row8(&sm.pos[BUF][r8], p8);
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    float sv = sp[hf][8 * e + x];
                    if (msk) {
                        const int i = qb + r8 + x;
                        const bool keep = (r8 + x < nrows) & (j >= i - p8[x]) & (j <= i);  // no short circuit
                        sv = keep ? sv : -INFINITY;
                    }
                    sp[hf][8 * e + x] = fast_exp2(sv);
                }
                xp[(2 * e) * 64] = make_float4(sp[hf][8 * e], sp[hf][8 * e + 1], sp[hf][8 * e + 2], sp[hf][8 * e + 3]);
                xp[(2 * e + 1) * 64] = make_float4(sp[hf][8 * e + 4], sp[hf][8 * e + 5], sp[hf][8 * e + 6], sp[hf][8 * e + 7]);
            }
        };
        // dS waves: dS = P (dP - D) with P from the P waves, as fp16 operands
        auto dscore = [&](int hf) __attribute__((always_inline)) {
            const float4 *xp = reinterpret_cast<const float4 *>(&sm.xp[w][hf][0][lane][0]);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float4 p0 = xp[(2 * e) * 64], p1 = xp[(2 * e + 1) * 64];
                const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
                for (int x = 0; x < 8; ++x) pb[hf][e][x] = (f16)(pv[x] * sp[hf][8 * e + x]);
            }
        };
        auto pconv = [&](int hf) __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int x = 0; x < 8; ++x) pb[hf][e][x] = (f16)sp[hf][8 * e + x];
        };
        // dS waves with a store: write dS^T of half hf (zeros when `zero`) to block (u, m) of head
        // h, m = (qb - first query row of the item) / BQ
        auto store_ds = [&](int hf, bool zero) __attribute__((always_inline)) {
            const int m = (qb - q_start) / BQ + (NS == 1 ? 0 : kh);   // block of the key tile
            f16 *dst = ds_tile + ((int64_t)m * a.hq + iter_head(itn)) * (PK_TILE_ROWS * BQ) +
                       ds_lane + 1024 * hf;
            // streaming stores: the store is read once, by the dQ kernel, and left in the caches
            // it would evict the query blocks other workgroups are about to re-read
#pragma unroll
            for (int e = 0; e < 2; ++e)
                __builtin_nontemporal_store(zero ? zero_f16x8() : pb[hf][e], reinterpret_cast<f16x8 *>(dst + 512 * e));
        };
        // the second product of half hf: dV^T += dO^T P (P waves) or dK^T += Q^T dS (dS waves);
        // queries are the k dimension and the transposed operand comes straight from the tile
        auto grads = [&](int hf) __attribute__((always_inline)) {
            const char *t = p_role ? cg : cq;
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    acc[db] = mfma32(tile_tr_at(t, toff[db], 2 * D * (32 * hf + 16 * e)), pb[hf][e], acc[db]);
        };

        // Blocks where both halves run (and, for the P waves, need no mask) take straight-line
        // code whose LDS reads are issued ahead of their products; the rest go half by half.
        const bool both = run[0] & run[1];
        const bool fast = both & (!p_role | (!masked[0] & !masked[1]));
        if (fast) {
            // the row values first, in a region of their own, so that the operand reads below
            // keep their distance ahead of the products
            init_scores(0);
            init_scores(1);
            __builtin_amdgcn_sched_barrier(0);
            scores(0);
            scores(1);
            __builtin_amdgcn_sched_group_barrier(0x100, NKK, 0);       // one half's operands ahead
#pragma unroll
            for (int m = 0; m < NKK; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NKK, 0);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (p_role) {
                softmax(0, false);
                softmax(1, false);
            }
        } else {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                if (!run[hf]) continue;
                init_scores(hf);
                scores(hf);
                if constexpr (p_role) softmax(hf, masked[hf]);
            }
        }
        __syncthreads();   // B1: P of both halves is in LDS
        if constexpr (NS == 1) {
            // One path for every block that runs at all: a half that does not run gets a zero
            // operand instead of a branch, so the accumulators keep their registers from block
            // to block (separate whole-block and per-half paths made the register allocator copy
            // them at every join).
            if (run[0] | run[1]) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    if (run[hf]) {
                        if constexpr (!p_role)
                            dscore(hf);
                        else
                            pconv(hf);
                    } else {
                        pb[hf][0] = zero_f16x8();
                        pb[hf][1] = zero_f16x8();
                    }
                }
                if constexpr (!p_role) {
                    if (store) {
                        store_ds(0, false);
                        store_ds(1, false);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                grads(0);
                grads(1);
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);     // 4 transposed operands ahead
#pragma unroll
                for (int m = 0; m < 4 * NDB - 4; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            } else if constexpr (!p_role) {
                // no row of the block sees these keys: their part of the store is zero
                if (store) {
                    store_ds(0, true);
                    store_ds(1, true);
                }
            }
        } else {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                if (!run[hf]) continue;
                if (!p_role)
                    dscore(hf);
                else
                    pconv(hf);
                if constexpr (!p_role) {
                    if (store) store_ds(hf, false);
                }
                grads(hf);
            }
            if constexpr (!p_role) {
                if (store && !run[hf_own]) store_ds(hf_own, true);
            }
        }
    };

    // the loop is unrolled by two so that the buffer of each step is a compile-time constant
    auto step = [&](auto bufc, int itn) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        const int qb = iter_row(itn);
        // wait for this block's copies; a dS wave's stores of the previous block (issued after
        // those copies, and counted by vmcnt in order with them) may stay in flight
        if constexpr (!p_role) {
            if (store && itn > 0)
                lds_copy_wait_keep<NS == 1 ? 4 : 2>();
            else
                lds_copy_wait();
        } else {
            lds_copy_wait();
        }
        __syncthreads();   // B0: this block is in LDS; every wave is done with the other buffer
        if (itn + 1 == n_iter) claim();
        if (itn + 1 < n_iter) kv_issue_block<D>(a, sm, BUF ^ 1, iter_head(itn + 1), iter_row(itn + 1), loff);
        block(bufc, qb, itn);
    };
    for (int itn = 0; itn < n_iter; itn += 2) {
        step(std::integral_constant<int, 0>(), itn);
        if (itn + 1 < n_iter) step(std::integral_constant<int, 1>(), itn + 1);
    }

    };
    if (wv < 4)
        main_loop(std::true_type());
    else
        main_loop(std::false_type());

    if constexpr (NS == 2) {
        // the second-half waves hand their partial sums over in the (now free) block tiles, the
        // first-half waves add them and write
        __syncthreads();   // every wave is done with the last block's tiles
        float *red = reinterpret_cast<float *>(&sm.q[0][0]);   // spans sm.q and sm.dO
        static_assert(sizeof(sm.q) + sizeof(sm.dO) >= 4 * NDB * 16 * 64 * sizeof(float),
                      "room for four waves' accumulators");
        const int slot = (p_role ? 0 : 2) + sub;
        if (hf_own == 1) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) red[((slot * NDB + db) * 16 + rr) * 64 + lane] = acc[db][rr];
        }
        __syncthreads();
        if (hf_own == 1) return;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) acc[db][rr] += red[((slot * NDB + db) * 16 + rr) * 64 + lane];
    }

    // epilogue: P waves write dV (unscaled by 1/sigma); dS waves write
    // dK = R(-theta) (scale * dK_rot) (unscaled by 1/(sigma tau))
    if (kvalid) {
        const int64_t rowoff = ((int64_t)j * a.hkv + kvh) * D;
        if (p_role) {
            float *dvrow = a.dv + rowoff;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = 32 * db + 8 * g4 + 4 * hb;
                    *reinterpret_cast<float4 *>(dvrow + d) =
                        make_float4(acc[db][4 * g4] * inv_sigma, acc[db][4 * g4 + 1] * inv_sigma,
                                    acc[db][4 * g4 + 2] * inv_sigma, acc[db][4 * g4 + 3] * inv_sigma);
                }
        } else {
            // Q_rot carries scale * log2(e), so scale * dK_rot = ln(2) * acc
            store_rotated_back<D>(a.dk + rowoff, a.rope + (int64_t)j * (D / 2),
                                       kLn2 * inv_sigma_tau, hb, acc);
        }
    }
}

// One workgroup per unit, or (PERSIST, NS = 1) a persistent grid of fewer workgroups that take
// the units from per-XCD counters (pk_device.h).  Units are (item, KV head), heads fastest.
template <int D, int NS, bool PERSIST>
__global__ __launch_bounds__(512, 1) void k_attn_bwd_kv(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) KvSmem<D> sm;
    if constexpr (PERSIST) {
        static_assert(NS == 1, "persistent launches take whole items");
        __shared__ int s_next[2];
        persistent_units(a.sched, a.hkv * a.n_items, s_next,
                         [&](int b, auto &claim) __attribute__((always_inline)) {
                             const BwdArgs u = reload_args<BwdArgs>();
                             kv_unit<D, 1>(u, sm, b / u.hkv, 0, b % u.hkv, claim);
                         });
    } else {
        kv_unit<D, NS>(a, sm, blockIdx.x / (a.hkv * NS), (blockIdx.x / a.hkv) % NS, blockIdx.x % a.hkv,
                       NoClaim());
    }
}

}  // namespace

namespace pk {

// Items x KV heads up to which an item is split over two workgroups (NS = 2).
constexpr unsigned kSplitGrid = 256;

hipError_t launch_bwd_kv(const AttnShape &sh, const pk_meta_s &m, const void *qrot,
                         const void *krot, const void *v, const void *dout16, const float *lse2,
                         const float *dsum, const float *scale, const void *rope, float *dk,
                         float *dv, const DsStore &ds, int32_t *sched, hipStream_t s) {
    BwdArgs a = pkb::make_bwd_args(sh, m, qrot, krot, v, dout16, lse2, dsum, scale, rope, nullptr,
                                   dk, dv);
    a.items = m.bwd_items;
    a.ds = (f16 *)ds.ptr;
    a.ds_cap = ds.cap_blocks;
    a.sched = sched;
    const unsigned units = (unsigned)sh.n_items * (unsigned)sh.hkv;
    auto go = [&](auto kernel, auto split, auto persistent) {
        // more units than resident workgroups: a persistent grid of the resident workgroups
        const unsigned slots = persistent_grid((const void *)persistent, 512);
        if (units <= kSplitGrid)
            split<<<2 * units, 512, 0, s>>>(a);
        else if (slots && units > slots)
            persistent<<<slots, 512, 0, s>>>(a);
        else
            kernel<<<units, 512, 0, s>>>(a);
    };
    if (sh.d == 128)
        go(k_attn_bwd_kv<128, 1, false>, k_attn_bwd_kv<128, 2, false>, k_attn_bwd_kv<128, 1, true>);
    else
        go(k_attn_bwd_kv<64, 1, false>, k_attn_bwd_kv<64, 2, false>, k_attn_bwd_kv<64, 1, true>);
    return hipGetLastError();
}

}  // namespace pk
