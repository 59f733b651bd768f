// Internal interface between the C-ABI layer (pk_api.cpp) and the HIP kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pk.h"

// The host object behind pk_meta_t: pointers into the caller's meta buffer plus the sizes the
// host already knows (so no launch ever needs a device read to size its grid).
struct pk_meta_s {
    int32_t *hdr;        // [0] = status bits, [1] = max_seqlen, [2] = operand-range flags
    int32_t *cu;         // [n_seqs + 1]
    int32_t *seq_id;     // [T]
    int32_t *pos;        // [T]
    int32_t *fwd_items;  // [n_items * 8], longest first
    int32_t *bwd_items;  // [n_items * 8], longest first
    int32_t *fwd_raw;    // [n_items * 8], tile order (build scratch)
    int32_t *bwd_raw;    // [n_items * 8], tile order (build scratch)
    int32_t *ds_off;     // [n_items + 1], tile order: first dS block of each key tile; [n] = total
    int32_t n_seqs;
    int32_t n_items;
    int64_t total_tokens;
    int32_t device;
};

namespace pk {

// Byte layout of the meta buffer; every region starts on a 256-byte boundary.
struct MetaLayout {
    size_t hdr, cu, seq_id, pos, fwd_items, bwd_items, fwd_raw, bwd_raw, ds_off, total;
};

// The backward's dS store: the dK/dV kernel writes, for each key tile u and each block of
// PK_DS_BLOCK_ROWS query rows in its backward item's range, and for each query head, the fp16
// block dS^T [128 keys][64 queries] (16 KB); block (u, m) of head h sits at block index
// (ds_off[u] + m) * hq + h.  The dQ kernel reads them back instead of recomputing S and dP.
constexpr size_t kDsBlockBytes = (size_t)PK_TILE_ROWS * PK_DS_BLOCK_ROWS * 2;
MetaLayout meta_layout(int32_t n_seqs, int64_t total_tokens);

// Byte layout of the attention workspaces.
struct FwdWorkspace {
    size_t krot, vh, rope, total;
};
struct BwdWorkspace {
    size_t qrot, krot, vh, dout16, rope, dsum, lse2, blockmax, scale, sched, total;
};
// Work counters of the persistent dK/dV launch (int32, in the backward workspace), cleared by the
// backward prologue.
constexpr int kSchedInts = 16;
// Workgroups of `kernel` (with `threads` threads each) the current device holds at once, rounded
// down to a multiple of 8; 0 when the runtime cannot say.  Cached per device and kernel.
unsigned persistent_grid(const void *kernel, int threads);
FwdWorkspace fwd_workspace(int64_t T, int hq, int hkv, int d);
BwdWorkspace bwd_workspace(int64_t T, int hq, int hkv, int d);
// Upper bound on the dS store's blocks (per head) for a pack of T tokens whose sequences are at
// most max_seqlen_bound long (<= 0: no bound, i.e. T).
int64_t ds_bound_blocks(int64_t T, int64_t max_seqlen_bound);

inline int64_t n_tiles(int64_t T) { return (T + PK_TILE_ROWS - 1) / PK_TILE_ROWS; }

// Launchers.  Each enqueues its kernels on `stream` and returns the launch status.
hipError_t launch_meta(const int32_t *lengths, const pk_meta_s &m, hipStream_t stream);

struct RopeArgs {
    const int32_t *pos;
    int64_t T;
    int hq, hkv, d;
    float rope_base;
};
// `flags` (the meta's range word) receives PK_META_FP16_RANGE when an operand the kernels round
// to fp16 lies outside its range.
hipError_t launch_fwd_prep(const RopeArgs &r, const void *k, const void *v, void *krot, void *vh,
                           void *rope, int32_t *flags, hipStream_t s);
// Blocks of the per-token prologue/epilogue kernels (one thread per token and 4 rotation pairs).
unsigned prep_blocks(int64_t T, int d);
// Blocks of the max|dout| (at most 1024) and max|v| (at most 256) reductions.
unsigned dmax_blocks(int64_t T, int hq, int d);
unsigned vmax_blocks(int64_t T, int hkv, int d);
hipError_t launch_bwd_prep(const RopeArgs &r, const void *q, const void *k, const void *v,
                           const void *out, const void *dout, const float *lse, void *qrot,
                           void *krot, void *vh, void *dout16, void *rope, float *dsum,
                           float *lse2, float *blockmax, float *scale, float qscale,
                           int32_t *flags, int32_t *sched, hipStream_t s);   // also clears sched

struct AttnShape {
    int64_t T;
    int hq, hkv, d, n_items;
    float scale;
};
hipError_t launch_fwd(const AttnShape &sh, const pk_meta_s &m, const void *q, const void *krot,
                      const void *v, const void *rope, void *out, float *lse, hipStream_t s);
// qrot = R(q) * softmax_scale * log2(e) (fp16), v16 = tau * v (fp16), dout16 = sigma * dout (fp16),
// dsum = -sigma * tau * rowsum(dout * out), lse2 = -lse * log2(e),
// scale = {sigma, 1/sigma, tau, 1/(sigma tau)}.
// launch_bwd_kv writes dk and dv, launch_bwd_q writes dq.
// The dS store region of a backward workspace: `cap_blocks` blocks of kDsBlockBytes for each of
// the hq heads (null / 0: none).
struct DsStore {
    void *ptr;
    int64_t cap_blocks;
};
hipError_t launch_bwd_kv(const AttnShape &sh, const pk_meta_s &m, const void *qrot,
                         const void *krot, const void *v, const void *dout16, const float *lse2,
                         const float *dsum, const float *scale, const void *rope, float *dk,
                         float *dv, const DsStore &ds, int32_t *sched, hipStream_t s);
hipError_t launch_bwd_q(const AttnShape &sh, const pk_meta_s &m, const void *qrot,
                        const void *krot, const void *v, const void *dout16, const float *lse2,
                        const float *dsum, const float *scale, const void *rope, float *dq,
                        const DsStore &ds, hipStream_t s);

// Steps around the attention path (pk_aux.hip, pk_moe.hip).
hipError_t launch_dense_mask(const pk_meta_s &m, uint8_t *mask, hipStream_t s);
hipError_t launch_rope_apply(const pk_meta_s &m, const void *x, int H, int d, float base,
                             int inverse, void *out, hipStream_t s);
#define PK_MOE_CHUNK 1024   // assignments per workgroup of the grouping kernels
int moe_chunks(int64_t M);
// chunk_counts: [n_experts][moe_chunks(M)] int32, chunk_bad: [moe_chunks(M)] int32 (workspace)
hipError_t launch_moe_group(const int32_t *idx, int64_t M, int E, int32_t *counts,
                            int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *status,
                            int32_t *chunk_counts, int32_t *chunk_bad, hipStream_t s);

// LoRA-adapted QKV projection (pk_lora.hip).
struct LoraWorkspace {
    size_t u, apad, bpad, total;
};
LoraWorkspace lora_workspace(int64_t T, int K, int N);
hipError_t launch_lora_qkv(const void *x, const void *wt, const void *at, const void *bt,
                           int64_t T, int K, int N, int r, float scale, void *y, void *ws,
                           hipStream_t s);

}  // namespace pk
