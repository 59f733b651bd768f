// Device-side helpers shared by the gfx950 kernels: vector types, the MFMA wrapper and the
// operand-row permutation used by the attention kernels.
//
// Number formats: tensors cross the ABI as bfloat16 (q, k, v, out, dout) or float32; inside the
// kernels every matrix-core operand is IEEE half (fp16) and every accumulator float32.  The
// bf16 inputs convert to fp16 exactly over fp16's normal range, and the values formed inside the
// kernels (RoPE-rotated q/k, softmax probabilities, dS) keep 3 more mantissa bits than bf16
// would give them, at the same v_mfma rate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace pkd {

// 64-bit minimum (the device min() overloads take int: int64_t arguments would be truncated).
__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, fp32) += A(32x16, fp16) * B(16x32, fp16) on the matrix cores (v_mfma_f32_32x32x16_f16).
// Operand layout per lane l of the wave: A row (l % 32), k = 8*(l/32) .. +7;
// B column (l % 32), same k; D column (l % 32), register r holds row 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Values of lanes l and l ^ 32 combined with one v_permlane32_swap: the swap leaves, in every
// lane, the pair {x[l], x[l ^ 32]} in its two results, so a symmetric op of the two is the
// cross-half reduction (no LDS permute and no address arithmetic).
__device__ __forceinline__ float half_swap_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x with the bare v_exp_f32 (results below 2^-126 flush to zero, which a softmax weight can
// afford); exp2f would add a denormal-range fix-up of four more instructions per call.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row permutation (swap bits 2 and 3 of the row index inside a 32-row block).  Feeding the first
// operand of a product whose result is reused as the k operand of a second product in this
// order makes each lane's 8 k values of the second product consecutive rows, so that operand
// can be read from LDS with one 16-byte load.
__device__ __forceinline__ int row_perm(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Row of 32x32 result register r for a lane in half hb (before any permutation).
__device__ __forceinline__ int acc_row(int r, int hb) { return 8 * (r >> 2) + 4 * hb + (r & 3); }

// Workgroup b of a grid of n_items x hq -> (work item r, query head h).  Workgroups are handed
// to the 8 XCDs round-robin (b runs on XCD b % 8), each XCD with its own L2.  When the KV heads
// split evenly over the XCDs, the query heads that share a KV head get consecutive slots of one
// XCD, so the K/V tiles they all read are fetched into that L2 once; items keep their
// longest-first order.  Otherwise the plain item-major, head-minor order is used.
__device__ __forceinline__ void item_head_of_block(int b, int hq, int hkv, int &r, int &h) {
    constexpr int NX = 8;
    if (hkv % NX == 0) {
        const int group = hq / hkv, per = hq / NX;   // query heads per XCD per item
        const int x = b % NX, m = b / NX;
        r = m / per;
        const int t = m % per;
        h = (x + NX * (t / group)) * group + t % group;
    } else {
        r = b / hq;
        h = b % hq;
    }
}

// threadIdx.x as a value the optimiser cannot hoist: in a persistent workgroup's loop over units
// (below), the per-lane offsets a unit derives from it are recomputed per unit instead of being
// held in registers across the whole loop.
__device__ __forceinline__ int opaque_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// ---- Persistent workgroups -------------------------------------------------------------------
// A persistent launch has G workgroups (a multiple of 8, as many as the device holds at once) for
// more units than that.  Workgroup g serves the units b = 8 m + g % 8, the units a plain launch
// would run on XCD g % 8 (workgroups go to the XCDs round-robin, so g itself runs there): first
// m = g / 8, then, as it nears the end of each unit, m = G / 8 + the value it takes from the
// class's counter sched[g % 8] (an atomic add).  So the workgroup that finishes first takes the
// longest unit left in its class (the greedy longest-first rule), and starts it at once instead
// of waiting for the dispatcher to start a new workgroup on the freed slot.  The unit calls
// claim() as its last block of work starts, which hides the add's latency behind that block;
// claiming earlier would reserve units for workgroups still busy with long ones.  (A unit that
// never calls claim() gets its next unit claimed when it ends.)  sched[8 + x] counts
// the workgroups of class x that have left: the last one sets both counters back to zero, so every
// launch finds them cleared (the prologue kernels also clear them, for a workspace's first use).
// `unit(b, claim)` runs one unit with the whole workgroup; s_next is two LDS ints.
template <typename F>
__device__ __forceinline__ void persistent_units(int32_t *sched, int n_units, int *s_next, F &&unit) {
    const int x = blockIdx.x & 7, wgs = gridDim.x >> 3;
    const int count = n_units > x ? (n_units - x + 7) >> 3 : 0;   // units of class x
    int m = blockIdx.x >> 3, par = 0;
    while (m < count) {
        int nxt = -1;   // (thread 0) the claimed next unit
        auto claim = [&]() __attribute__((always_inline)) {
            if (threadIdx.x == 0) nxt = wgs + atomicAdd(sched + x, 1);
        };
        unit(8 * m + x, claim);
        if (threadIdx.x == 0) s_next[par] = nxt >= 0 ? nxt : wgs + atomicAdd(sched + x, 1);
        __syncthreads();   // also: every wave is done with the unit's LDS
        m = __builtin_amdgcn_readfirstlane(s_next[par]);
        par ^= 1;
    }
    if (threadIdx.x == 0 && atomicAdd(sched + 8 + x, 1) == wgs - 1) {
        atomicExch(sched + x, 0);
        atomicExch(sched + 8 + x, 0);
    }
}

// The claim() of a unit that is not part of a persistent launch.
struct NoClaim {
    __device__ void operator()() const {}
};

// The kernel's arguments, when they are its only parameter (so they sit at the start of the
// kernel-argument segment), read afresh from that constant segment: a persistent loop that passes
// this copy to its units reloads the fields each unit (a few scalar loads) instead of holding all
// of them in scalar registers across the loop.
template <typename Args>
__device__ __forceinline__ Args reload_args() {
    typedef __attribute__((address_space(4))) const Args *cptr;
    cptr p = (cptr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    return *(const Args *)p;
}

// ---- Swizzled row-major fp16 LDS tiles ------------------------------------------------------
// A tile holds rows of D halves with no padding; the 16-byte chunk c of row r is stored at chunk
// position c ^ swz(r).  Two read patterns are conflict-free on the 64 LDS banks:
//   * ds_read_b128 of one chunk by 16 lanes on 16 different rows (operand rows);
//   * ds_read_b64_tr_b16 by 32 lanes on 4 consecutive rows x 64 bytes (transposed operands).
// D = 128 (256-byte rows): swz(r) = 4*(r%4) + (r/4)%4.
// D = 64 (128-byte rows, two per bank sweep): swz(r) = 4*((r/2)%2) + (r/4)%4.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Offset in halves of element (r, col) of a swizzled tile (col any multiple of 4).
template <int D>
__device__ __forceinline__ int tile_off(int r, int col) {
    return r * D + 8 * ((col >> 3) ^ swz<D>(r)) + (col & 7);
}

// 8 halves (one 16-byte chunk, col multiple of 8) of row r.
template <int D>
__device__ __forceinline__ f16x8 tile_row8(const f16 *tile, int r, int col) {
    return *reinterpret_cast<const f16x8 *>(tile + tile_off<D>(r, col));
}

template <int D>
__device__ __forceinline__ void tile_store8(f16 *tile, int r, int col, f16x8 v) {
    *reinterpret_cast<f16x8 *>(tile + tile_off<D>(r, col)) = v;
}

// A operand (32 rows m x 16 k) of mfma32 taken transposed from a swizzled tile X:
// A[m][k] = X[k0 + k][m0 + m] (k0 multiple of 4, m0 multiple of 32).  Two ds_read_b64_tr_b16:
// within each 16-lane group, source lane j addresses the 4 halves X[kb + j/4][mb + 4(j%4) ..],
// and lane i receives element i%4 of the halves read by source lanes i/4 + 4t (t = 0..3),
// i.e. the 4 consecutive k of its own column m.
template <int D>
__device__ __forceinline__ f16x8 tile_a_tr(const f16 *tile, int k0, int m0) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
    const int r = k0 + 8 * (g >> 1) + (j >> 2);
    const int col = m0 + 16 * (g & 1) + 4 * (j & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(tile + tile_off<D>(r, col)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(tile + tile_off<D>(r + 4, col)));
    return __builtin_bit_cast(f16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One global_load_lds per lane: `BYTES` (4 or 16) bytes from global address g land in LDS at
// byte lds + BYTES * lane (lds is the wave-uniform LDS offset, passed through M0).  The load is
// written as inline assembly on purpose: the compiler cannot tell which LDS bytes the builtin form
// writes, so after it it makes the first LDS read of ANY buffer wait for every outstanding copy,
// which would serialise a double-buffered prefetch with the compute on the other buffer.  The
// copies stay counted by vmcnt; lds_copy_wait() followed by a barrier publishes them.
template <int BYTES>
__device__ __forceinline__ void lds_dma(const void *g, uint32_t lds) {
    static_assert(BYTES == 4 || BYTES == 16, "global_load_lds moves 4 or 16 bytes per lane");
    if constexpr (BYTES == 16)
        asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
    else
        asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

// LDS byte offset of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// Asynchronous copy of one row-major [rows x D] fp16 tile from global memory into a swizzled LDS
// tile with global_load_lds_dwordx4: each instruction moves 64 lanes x 16 bytes to a contiguous
// 1 KB run of LDS (lane l at byte 16 l), so the swizzle is applied on the global side by choosing
// which chunk each lane fetches.  `src(row)` returns the global address of element 0 of a tile
// row; rows are clamped by the caller.  The copy is tracked by vmcnt; wait with
// lds_copy_wait() before a barrier.  Waves split the tile's 1 KB runs: wave w issues runs
// w, w + nwaves, ...
template <int D, int ROWS, typename RowPtr>
__device__ __forceinline__ void tile_copy_async(f16 *tile, int nwaves, RowPtr src) {
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int RUNS = ROWS * CPR / 64;      // 1 KB runs per tile
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t base = lds_addr(tile);
    for (int run = w; run < RUNS; run += nwaves) {
        const int c = run * 64 + lane;         // physical chunk index in the tile
        const int row = c / CPR;
        const int logical = (c % CPR) ^ swz<D>(row);
        lds_dma<16>(src(row) + 8 * logical, base + 1024u * run);
    }
}

// Same load with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte offset (the
// saddr form), so a caller can advance the base with scalar arithmetic only.
template <int BYTES>
__device__ __forceinline__ void lds_dma_s(const void *base, uint32_t lane_off, uint32_t lds) {
    static_assert(BYTES == 4 || BYTES == 16, "global_load_lds moves 4 or 16 bytes per lane");
    if constexpr (BYTES == 16)
        asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(lane_off), "s"(base), "{m0}"(lds) : "memory");
    else
        asm volatile("global_load_lds_dword %0, %1" ::"v"(lane_off), "s"(base), "{m0}"(lds) : "memory");
}

// Copies by NW waves with every tile row present: lane offset (bytes, from element 0 of the tile's
// first row) of the 16 bytes this lane fetches in its wave's first 1 KB run, for rows that are
// `row_stride` halves apart.  Wave w issues runs w, w + NW, ...; run w + NW t starts
// NW t * (64 / (D/8)) rows further down, a multiple of 16 rows, so the swizzled chunk of the lane
// is the same in every run and only the wave-uniform base moves.
template <int D, int NW = 4>
__device__ __forceinline__ uint32_t tile_copy_lane_off(int64_t row_stride) {
    constexpr int CPR = D / 8, RPR = 64 / CPR;
    static_assert((NW * RPR) % 16 == 0, "swizzle period");
    const int lane = threadIdx.x & 63, w = (threadIdx.x >> 6) % NW;
    const int row = w * RPR + lane / CPR;
    const int chunk = (lane % CPR) ^ swz<D>(row);
    return (uint32_t)(((int64_t)row * row_stride + 8 * chunk) * 2);
}

template <int D, int ROWS, int NW = 4>
__device__ __forceinline__ void tile_copy_async_whole(f16 *tile, const f16 *base, int64_t row_stride,
                                                      uint32_t lane_off) {
    constexpr int CPR = D / 8, RPR = 64 / CPR, RUNS = ROWS * CPR / 64;
    static_assert(RUNS % NW == 0, "runs are split evenly over the waves");
    const int w = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) % NW);
    const uint32_t lds = lds_addr(tile) + 1024u * w;
#pragma unroll
    for (int t = 0; t < RUNS / NW; ++t)
        lds_dma_s<16>(base + (int64_t)(NW * RPR * t) * row_stride, lane_off, lds + 1024u * NW * t);
}

// Asynchronous copy of rows [row0, row0 + ROWS) of head h of a [T, H, D] fp16 tensor into a
// swizzled LDS tile by NW waves.  Tiles whose rows all exist take the scalar-addressed path
// (lane_off from tile_copy_lane_off<D, NW>(H * D)); a tile that runs past T clamps its rows to
// T - 1 lane by lane, and the caller masks those rows.
template <int D, int ROWS, int NW = 4>
__device__ __forceinline__ void tile_issue(f16 *tile, const f16 *x, int H, int h, int row0, int64_t T,
                                           uint32_t lane_off) {
    const int64_t stride = (int64_t)H * D;
    if (row0 + ROWS <= (int)T) {   // T <= PK_MAX_TOKENS; a 32-bit test stays scalar
        tile_copy_async_whole<D, ROWS, NW>(tile, x + (int64_t)row0 * stride + (int64_t)h * D, stride, lane_off);
    } else {
        tile_copy_async<D, ROWS>(tile, NW, [&](int row) {
            return x + min64((int64_t)row0 + row, T - 1) * stride + (int64_t)h * D;
        });
    }
}

// Per-lane byte offsets of the two ds_read_b64_tr_b16 that make up the transposed operand of
// columns [32 db, +32) and tile rows [0, 16) (the layout of tile_a_tr with k0 = 0, m0 = 32 db):
// rows k0 + 16 t add 32 D t bytes, the swizzle being periodic in 16 rows.
template <int D>
__device__ __forceinline__ void tile_tr_offsets(uint32_t (&off)[D / 32][2]) {
    const int lane = threadIdx.x & 63, jj = lane & 15, g = lane >> 4;
    const int r = 8 * (g >> 1) + (jj >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        const int col = 32 * db + 16 * (g & 1) + 4 * (jj & 3);
        off[db][0] = 2 * tile_off<D>(r, col);
        off[db][1] = 2 * tile_off<D>(r + 4, col);
    }
}

// Transposed operand from a tile at LDS bytes `t`, rows k0.. (k0 multiple of 16), columns of
// the offsets `off` (from tile_tr_offsets).
__device__ __forceinline__ f16x8 tile_tr_at(const char *t, const uint32_t (&off)[2], int byte_k0) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(t + off[0] + byte_k0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(t + off[1] + byte_k0));
    return __builtin_bit_cast(f16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ void lds_copy_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait for every vector memory operation of the wave but the last N (vmcnt counts them in
// issue order): lets N global stores issued after the copies being waited for stay in flight.
template <int N>
__device__ __forceinline__ void lds_copy_wait_keep() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Make the compiler complete the pending global load of x here.  Used on values loaded before a
// loop that keeps asynchronous LDS copies in flight: left alone, the compiler's wait for such a
// value sits inside the loop, where a full vmcnt wait would also drain those copies.
template <typename T>
__device__ __forceinline__ void settle(const T &x) { asm volatile("" ::"v"(x)); }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    bf16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
    return z;
}

__device__ __forceinline__ f16x8 zero_f16x8() {
    f16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (f16)0.0f;
    return z;
}

__device__ __forceinline__ f32x16 zero_f32x16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16 *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

__device__ __forceinline__ void store_bf16x8(bf16 *p, bf16x8 v) {
    *reinterpret_cast<bf16x8 *>(p) = v;
}

__device__ __forceinline__ f16x8 load_f16x8(const f16 *p) {
    return *reinterpret_cast<const f16x8 *>(p);
}

__device__ __forceinline__ void store_f16x8(f16 *p, f16x8 v) {
    *reinterpret_cast<f16x8 *>(p) = v;
}

// bf16 -> fp16 through fp32 (exact over fp16's normal range), with an optional scale.
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(bf16x8 x, float scale = 1.0f) {
    f16x8 y;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = (f16)((float)x[i] * scale);
    return y;
}

__device__ __forceinline__ uint32_t pack_f16x2(f16 lo, f16 hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(bf16 lo, bf16 hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

}  // namespace pkd
