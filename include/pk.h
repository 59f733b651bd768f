/*
 * pk.h -- packed-sequence causal attention for AMD Instinct MI355X (gfx950), C ABI.
 *
 * Sources, cited by page title and section:
 *   [UN-2026] "如何用 Unsloth 和 NVIDIA 让 LLM 训练更快" (Unsloth x NVIDIA, dbyun.net/tutorial/10079),
 *             §1 "缓存 Packed-Sequence 元数据": short samples are concatenated with no padding; the
 *             boundaries travel as metadata B = {lengths, cu_seqlens, max_seqlen, mask structure};
 *             every layer consumes the same B, so it is built once and used L times, and no
 *             per-layer device-to-host synchronisation is allowed on the path.
 *             §3 (MoE routing): group once with a stable sort + counts instead of one dynamic
 *             query per group -- the pattern the work-list build follows, and pk_moe_group.
 *             §2 "用双缓冲检查点重载隐藏延迟": two device buffers so that copying activations back
 *             from pinned host memory overlaps the backward -- pk_reload_*.
 *   [UN-2023] "Introducing Unsloth：LLM 训练提速 30 倍" (dbyun.net/tutorial/10038),
 *             "手动 Autograd": A(X) = softmax(Q K^T / sqrt(d) + M) V;
 *             "OpenAI Triton kernels": rotate-half RoPE on the two halves of the head dim.
 *   [N1N-2026] "利用 Unsloth 和 NVIDIA 硬件加速 LLM 训练：技术深度解析" (explore.n1n.ai),
 *             §2 "FlashAttention-2 的深度集成": tiles kept on chip, softmax fused with the
 *             products, no N x N matrix stored.
 *   [MV] "UnSloth极速微调：底层CUDA优化带来的变革" (maplevalley.com.cn), RoPE paragraph:
 *             positions' rotation factors served from a precomputed table.
 *
 * Conventions for every entry point:
 *   - Device pointers point to memory the caller allocated on the current HIP device and owns.
 *     The library allocates no device memory.  Host pointers are marked "host".
 *   - Every call that takes `hip_stream` (a hipStream_t, NULL = the default stream) only enqueues
 *     work on that stream and returns; none of them synchronises or reads device memory, except
 *     pk_meta_check, a debugging aid.
 *   - Argument errors are detected on the host before anything is launched: the call returns a
 *     negative pk_status and enqueues nothing.  Errors reported by the HIP runtime at launch
 *     return PK_ERR_HIP.  No exceptions cross the ABI.
 *   - Tensor layouts are contiguous "token-major" packs:
 *       q, out, dout, dq : [T, hq, d]      k, v, dk, dv : [T, hkv, d]      lse : [hq, T]
 *     q/k/v/out/dout are bfloat16, lse/dq/dk/dv are float32.
 *   - Supported shapes: d in {64, 128}; hq % hkv == 0; 1 <= hkv <= hq <= 256;
 *     0 <= T <= PK_MAX_TOKENS; 0 <= n_seqs <= T (n_seqs may be 0 only when T == 0).
 */
#ifndef PK_H
#define PK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PK_TILE_ROWS 128          /* tokens per work item (rule W granularity) */
#define PK_ITEM_FIELDS 8          /* int32 fields per work item */
#define PK_MAX_TOKENS (1 << 20)   /* largest pack the library accepts */

typedef enum pk_status {
    PK_OK = 0,
    PK_ERR_INVALID = -1,      /* null pointer, negative size, size mismatch, wrong device */
    PK_ERR_UNSUPPORTED = -2,  /* head_dim, head counts or token count outside the supported set */
    PK_ERR_CAPACITY = -3,     /* a caller buffer (meta buffer, workspace) is too small */
    PK_ERR_HIP = -4,          /* the HIP runtime reported an error */
    PK_ERR_DEVICE = -5        /* pk_meta_check only: the device-side status word is non-zero */
} pk_status;

/* Device-side status word bits, set by pk_build_meta for data only the device can see. */
#define PK_META_BAD_LENGTH 1      /* some length < 1 */
#define PK_META_BAD_TOTAL 2       /* the lengths do not sum to total_tokens */
/* Operand-range flag, kept in a word of its own next to the status word: cleared by
 * pk_build_meta, set (atomically, so concurrent calls may share the meta) by an attention call
 * that meets an input its fp16 matrix operands cannot hold; the results of that call are then not
 * meaningful.  Attention calls keep running on a meta with this flag set (it is not a pack error);
 * pk_meta_check reports it together with the status bits.  The matrix-core operands are fp16
 * with fp32 accumulation; the bounds that hold for every fp16 operand are:
 *   forward:  |q|, |k| <= 65504 / sqrt(2) (a rotated element is at most sqrt(2) max|x|),
 *             |v| <= 65504; P <= 256 (the online softmax's reference maximum moves when a score
 *             exceeds it by 8 in the exp2 domain);
 *   backward: dout and v enter scaled by powers of two sigma, tau with max|sigma dout| and
 *             max|tau v| in [1, 2), so |sigma dout| < 2, |tau v| < 2, P <= 1 and
 *             |sigma tau dS| < 8 d for any finite dout and v (dS = P (dout.v - D), where
 *             |dout_i . v_j| and |D_i| are both at most |dout_i|_1 max|v|); the remaining inputs
 *             need |R(q)| * softmax_scale * log2(e) <= 65504 and |R(k)| <= 65504.
 * Inputs outside these bounds, or not finite, set the flag. */
#define PK_META_FP16_RANGE 4

/* Opaque handle: a small host object that points into the caller's meta buffer.  It is
 * immutable after pk_build_meta returns, so several streams may read it concurrently. */
typedef struct pk_meta_s *pk_meta_t;

/* Device pointers into the meta buffer (all int32), for callers and tests that read B. */
typedef struct pk_meta_view {
    const int32_t *cu_seqlens;    /* [n_seqs + 1]: cu[0] = 0, cu[s+1] = cu[s] + lengths[s] */
    const int32_t *max_seqlen;    /* [1] */
    const int32_t *status;        /* [1]: PK_META_* bits, 0 when the pack is valid */
    const int32_t *seq_id;        /* [T]: sequence of each token */
    const int32_t *pos;           /* [T]: position of each token inside its sequence */
    const int32_t *fwd_items;     /* [n_items][8]: {q_start, q_end, kv_start, kv_end, seq_first,
                                     seq_last, cost, tile}, longest first */
    const int32_t *bwd_items;     /* [n_items][8]: {kv_start, kv_end, q_start, q_end, seq_first,
                                     seq_last, cost, tile}, longest first */
    int32_t n_seqs;
    int32_t n_items;              /* ceil(T / PK_TILE_ROWS) */
    int64_t total_tokens;
    int32_t device;               /* HIP device the meta was built on */
    const int32_t *ds_off;        /* [n_items + 1], tile order: ds_off[u] = sum over key tiles
                                     u' < u of ceil((q_end - q_start) / PK_DS_BLOCK_ROWS) of their
                                     backward items (the first block of tile u in the backward's
                                     dS store); ds_off[n_items] = the total */
} pk_meta_view_t;

/* Work-list granularity (PK_TILE_ROWS), exported for bindings. */
int32_t pk_tile_rows(void);

/* Bytes of device memory pk_build_meta needs for a pack of n_seqs sequences and T tokens.
 * Returns 0 for unsupported sizes. */
size_t pk_meta_bytes(int32_t n_seqs, int64_t total_tokens);

/* Build B for one pack ([UN-2026] §1): cu_seqlens by an on-device prefix sum of `lengths`,
 * max_seqlen, per-token seq_id and pos, the forward (query-tile) and backward (key-tile) work
 * lists sorted longest-first, and a status word.  `lengths_dev` is int32 [n_seqs] on the device
 * and must stay valid until the enqueued work has run.  `meta_buf_dev` (>= pk_meta_bytes bytes,
 * 256-byte aligned) holds B and must outlive the handle.  On success *out receives a new handle;
 * release it with pk_meta_destroy.  T and n_seqs come from the host, so nothing is read back:
 * invalid lengths are only visible in the device status word, and attention calls given such a
 * meta write zeros. */
pk_status pk_build_meta(const int32_t *lengths_dev, int32_t n_seqs, int64_t total_tokens,
                        void *meta_buf_dev, size_t meta_buf_bytes, void *hip_stream,
                        pk_meta_t *out /* host */);

/* Fill *view (host) with the device pointers and sizes of a meta. */
pk_status pk_meta_view(pk_meta_t meta, pk_meta_view_t *view /* host */);

/* DEBUGGING AID, SYNCHRONISES `hip_stream`: copy the status word (OR-ed with the operand-range
 * flag PK_META_FP16_RANGE) and max_seqlen to the host.  Returns PK_ERR_DEVICE when that word is
 * non-zero.  Either output pointer may be NULL. */
pk_status pk_meta_check(pk_meta_t meta, void *hip_stream, int32_t *status_host,
                        int32_t *max_seqlen_host);

/* Free the handle (host memory only; the caller's meta buffer is untouched). */
pk_status pk_meta_destroy(pk_meta_t meta);

/* Workspace bytes pk_attn_fwd needs: the rotated K and V as fp16, and the RoPE cos/sin table. */
size_t pk_attn_fwd_workspace_bytes(pk_meta_t meta, int32_t hq, int32_t hkv, int32_t d);

/* Forward ([UN-2023] "手动 Autograd", [N1N-2026] §2):
 *   out = softmax(scale * R(q) R(k)^T + M) v,   lse = log-sum-exp of the scaled masked scores,
 * with M the block-diagonal causal mask of the pack (key j visible to query i iff both are in
 * the same sequence and j <= i), R the rotate-half RoPE ([UN-2023] "OpenAI Triton kernels") at
 * the token's position inside its sequence with angle pos * rope_base^(-2i/d), and q head h
 * reading KV head h / (hq / hkv).  No T x T mask is formed: the work list bounds each tile.
 * `ws` is device memory of at least pk_attn_fwd_workspace_bytes bytes (256-byte aligned). */
pk_status pk_attn_fwd(pk_meta_t meta, const void *q, const void *k, const void *v,
                      int32_t hq, int32_t hkv, int32_t d, float softmax_scale, float rope_base,
                      void *out, float *lse, void *ws, size_t ws_bytes, void *hip_stream);

/* Largest workspace pk_attn_fwd_noalloc can use: 128 MiB, i.e. T * hkv * d * 4 + T * d * 4 bytes
 * (plus 256-byte alignment of each part) up to this size -- e.g. T = 16384 tokens with 8 KV heads
 * of d = 128 (76 MiB), or T = 32768 with 4 KV heads of d = 128 (80 MiB). */
#define PK_NOALLOC_SCRATCH_BYTES (128u << 20)

/* pk_attn_fwd for callers that cannot allocate device memory (code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid allocation): the same computation and the
 * same kernels, with the workspace taken from a fixed array of PK_NOALLOC_SCRATCH_BYTES that the
 * library holds on each device it runs on (from its load until the process ends) instead of from
 * the caller.  It allocates nothing (no hipMalloc, no allocating library call); the caller still
 * passes q, k, v, out and lse.  Returns PK_ERR_CAPACITY, enqueueing nothing, when
 * pk_attn_fwd_workspace_bytes(meta, hq, hkv, d) exceeds PK_NOALLOC_SCRATCH_BYTES.  Every call
 * on one device shares that device's array and overwrites it before reading it: calls that may
 * overlap on one device (other streams, other host threads) race and must be ordered by the
 * caller; the array keeps the last call's contents. */
pk_status pk_attn_fwd_noalloc(pk_meta_t meta, const void *q, const void *k, const void *v,
                              int32_t hq, int32_t hkv, int32_t d, float softmax_scale,
                              float rope_base, void *out, float *lse, void *hip_stream);

/* Workspace bytes pk_attn_bwd needs: the fp16 operands (rotated Q and K, V, scaled dout), the
 * RoPE table, per-row values (rowsum(dout * out), lse), the dout and v scales with their
 * per-block maxima, and the work counters of the dK/dV kernel's persistent launch (which the
 * prologue clears and the launch leaves at zero; calls that overlap on one workspace race). */
size_t pk_attn_bwd_workspace_bytes(pk_meta_t meta, int32_t hq, int32_t hkv, int32_t d);

/* Query rows per block of the backward's dS store. */
#define PK_DS_BLOCK_ROWS 64

/* Workspace bytes for pk_attn_bwd with a dS store sized for packs whose sequences are at most
 * `max_seqlen_bound` tokens long (<= 0: no bound, sized for one sequence of T tokens): the
 * bytes pk_attn_bwd_workspace_bytes gives, followed by room for
 *   hq * sum over key tiles u of min(ceil((T - 128 u) / 64), ceil((max_seqlen_bound + 127) / 64))
 * blocks of 128 x 64 fp16 (16 KiB) -- a tile's backward item spans at most the rest of the last
 * sequence that starts inside the tile.  (The Qwen3-14B-shaped pack, 16384 tokens, 40 query
 * heads, longest sequence 3523: 4.6 GiB.)  0 for unsupported arguments. */
size_t pk_attn_bwd_workspace_bytes_ds(pk_meta_t meta, int32_t hq, int32_t hkv, int32_t d,
                                      int64_t max_seqlen_bound);

/* Backward of pk_attn_fwd for the loss sum(out * dout): float32 dq [T,hq,d], dk and dv
 * [T,hkv,d] (dk, dv summed over the query heads of each KV group).  `out` and `lse` are the
 * forward's outputs for the same inputs (D = rowsum(dout * out) is formed from the given out).
 * dq, dk and dv are fully overwritten.
 * The first pk_attn_bwd_workspace_bytes bytes of `ws` hold the backward's operands; whatever
 * `ws_bytes` leaves after them is a dS store.  When the store holds the pack's blocks
 * (hq * ds_off[n_items] blocks of 16 KiB, a test made on the device, so nothing is read back),
 * the dK/dV kernel writes its fp16 dS there and the dQ kernel computes dQ = dS K from it; else
 * the dQ kernel recomputes S and dP (two more products).  Both give dq within the same rounding.
 * Without a store, on packs too small to fill the device, the dQ kernel runs on a library-owned
 * stream of the same device (default priority, created on first use), forked from and joined
 * back into `hip_stream` with events, so every result is ordered on `hip_stream` as if it ran
 * there. */
pk_status pk_attn_bwd(pk_meta_t meta, const void *q, const void *k, const void *v,
                      const void *out, const float *lse, const void *dout,
                      int32_t hq, int32_t hkv, int32_t d, float softmax_scale, float rope_base,
                      float *dq, float *dk, float *dv, void *ws, size_t ws_bytes,
                      void *hip_stream);

/* pk_attn_bwd in two halves, for callers that overlap one layer's prologue with another
 * layer's attention kernels (the prologue streams HBM while the attention kernels keep the
 * matrix cores busy).  pk_attn_bwd_prep reads q, k, v, out, lse, dout and writes the backward's
 * operands into `ws`; pk_attn_bwd_main reads only `ws` (same size as pk_attn_bwd's) and writes
 * dq, dk, dv.  pk_attn_bwd = prep then main on one stream.  Between the two halves the caller
 * orders the streams (e.g. with events); two layers in flight need two workspaces.
 * pk_attn_bwd_main may run again on the same prologue (it leaves `ws`'s operands unchanged). */
pk_status pk_attn_bwd_prep(pk_meta_t meta, const void *q, const void *k, const void *v,
                           const void *out, const float *lse, const void *dout, int32_t hq,
                           int32_t hkv, int32_t d, float softmax_scale, float rope_base, void *ws,
                           size_t ws_bytes, void *hip_stream);
pk_status pk_attn_bwd_main(pk_meta_t meta, int32_t hq, int32_t hkv, int32_t d,
                           float softmax_scale, float *dq, float *dk, float *dv, void *ws,
                           size_t ws_bytes, void *hip_stream);

/* ---- Steps around the attention path, each usable on its own -------------------------- */

#define PK_MASK_MAX_TOKENS 65536  /* largest pack pk_dense_mask accepts (a 4 GiB mask) */

/* Materialised keep pattern of the pack: mask[i * T + j] = 1 when key j is visible to query i
 * (same packed sequence and j <= i), else 0; T = the meta's token count.  This is the T x T
 * structure the pages' uncached path rebuilds for every layer ([UN-2026] §1 "快速合理性验证":
 * the packed SDPA mask rebuild is the dominant repeated cost) -- the attention calls above never
 * form or read it; it serves as the baseline that caching B removes.  Byte layout = torch.bool.
 * `mask` is device memory of at least T * T bytes, 16-byte aligned; T <= PK_MASK_MAX_TOKENS
 * (else PK_ERR_UNSUPPORTED).  A meta whose status word is set yields an all-zero mask. */
pk_status pk_dense_mask(pk_meta_t meta, uint8_t *mask, size_t mask_bytes, void *hip_stream);

/* Rotate-half RoPE of one bfloat16 tensor x [T, h, d] at each token's position inside its
 * packed sequence ([UN-2023] "OpenAI Triton kernels": out1 = x1 cos - x2 sin,
 * out2 = x2 cos + x1 sin over the halves of the head dim; the angle of pair i at position p is
 * p * rope_base^(-2i/d)).  inverse != 0 applies the transpose rotation (sin -> -sin), the
 * backward of the forward rotation.  Arithmetic in float32 from double-precision angles, result
 * rounded to bfloat16 (nearest even).  `out` [T, h, d] bfloat16 may be `x` itself (in place).
 * d in {64, 128}, 1 <= h <= 1024.  A meta whose status word is set yields zeros. */
pk_status pk_rope_apply(pk_meta_t meta, const void *x, int32_t h, int32_t d, float rope_base,
                        int32_t inverse, void *out, void *hip_stream);

#define PK_MOE_MAX_EXPERTS 1024    /* largest expert count pk_moe_group accepts */
#define PK_MOE_MAX_ASSIGN (1 << 26) /* largest n_tokens * top_k */
#define PK_MOE_BAD_EXPERT 1        /* status bit: some router index lies outside [0, n_experts) */

/* Workspace bytes of pk_moe_group (per-chunk counts), 0 for unsupported sizes. */
size_t pk_moe_group_workspace_bytes(int64_t n_assign, int32_t n_experts);

/* Group MoE routing assignments by expert in one pass ([UN-2026] §3: flatten the router's
 * [n_tokens, top_k] indices, sort them stably by expert, count per expert, offsets from the
 * counts, split) with no host round trip.  With M = n_tokens * top_k and f = token * top_k + slot:
 *   counts  [n_experts]     assignments per expert
 *   offsets [n_experts + 1] start of each expert's group; offsets[n_experts] = M when all valid
 *   perm    [M]             flat assignment at each grouped position (inside a group: ascending f)
 *   inv     [M]             grouped position of each flat assignment (-1 for an invalid index)
 *   status  [1]             0, or PK_MOE_BAD_EXPERT when an index lies outside [0, n_experts);
 *                           then the other outputs hold the grouping of the valid assignments.
 * All int32 device buffers written in full (perm and inv may be NULL when M = 0); `ws` holds at
 * least pk_moe_group_workspace_bytes bytes, 256-byte aligned.  Results are deterministic.
 * 1 <= n_experts <= PK_MOE_MAX_EXPERTS, top_k >= 1, M <= PK_MOE_MAX_ASSIGN. */
pk_status pk_moe_group(const int32_t *router_indices, int64_t n_tokens, int32_t top_k,
                       int32_t n_experts, int32_t *counts, int32_t *offsets, int32_t *perm,
                       int32_t *inv, int32_t *status, void *ws, size_t ws_bytes,
                       void *hip_stream);

/* ---- LoRA-adapted QKV projection (the producer of q, k, v) ----------------------------
 * "Introducing Unsloth：LLM 训练提速 30 倍", "手动 Autograd": Q = X (W_q + A_q B_q), likewise K
 * and V.  With the three projections stacked along the output dimension (N = (hq + 2 hkv) d;
 * columns [0, hq d) are q, then k, then v, so y viewed as [T, N] splits into the [T, h, d]
 * tensors pk_attn_fwd takes):
 *     y [T, N] = x [T, K] (W + scale A B),   W [K, N], A [K, r], B [r, N],
 * computed as x W + (scale x A) B without forming W + scale A B.  Storage is the weight layout
 * of a linear layer (out x in): wt = W^T [N, K], at = A^T [r, K], bt = B^T [N, r]; x, y
 * row-major.  All bfloat16, fp32 accumulation; scale x A is rounded to bf16 before it meets B.
 * K % 64 == 0 (64..65536), N % 128 == 0 (128..65536), 1 <= r <= PK_LORA_MAX_RANK,
 * T <= PK_MAX_TOKENS; device pointers 16-byte aligned, `ws` (>= pk_lora_qkv_workspace_bytes,
 * 256-byte aligned) holds scale x A and zero-padded copies of the adapter. */
#define PK_LORA_MAX_RANK 64
size_t pk_lora_qkv_workspace_bytes(int64_t T, int32_t K, int32_t N, int32_t r);
pk_status pk_lora_qkv(const void *x, const void *wt, const void *at, const void *bt, int64_t T,
                      int32_t K, int32_t N, int32_t r, float scale, void *y, void *ws,
                      size_t ws_bytes, void *hip_stream);

/* ---- Double-buffered reload of activations from pinned host memory --------------------
 * [UN-2026] §2 "用双缓冲检查点重载隐藏延迟": activations offloaded to pinned host memory are
 * copied back for the backward; with one device buffer the copy and the backward that consumes it
 * alternate (T ~ L (c + g)), with two the copy of the next layer overlaps the current layer's
 * compute (T ~ c + (L - 1) max(c, g) + g).  A pipeline owns a copy stream (default priority) and
 * two slots; the caller owns the device buffers of each slot and the pinned host memory (allocate
 * it pinned, e.g. hipHostMalloc; pageable memory works but is not overlapped).  Ordering is by
 * events only -- no call blocks the host except pk_reload_destroy, which waits for pending
 * copies.  Typical loop over layers l = L-1 .. 0 with slot s = (L-1-l) % 2:
 *     fetch(s0, layer L-1); for each l: fetch(1-s, layer l-1); acquire(s, stream);
 *     backward(l) on stream; release(s, stream).
 * One pipeline is used from one device; calls on it are serialised internally. */
typedef struct pk_reload_s *pk_reload_t;

/* Create a pipeline on the current device.  *out receives the handle. */
pk_status pk_reload_create(pk_reload_t *out /* host */);

/* Enqueue on the pipeline's copy stream a copy of `bytes` from host memory `src_host` to device
 * memory `dst` (a buffer of slot `slot`, 0 or 1), after the compute work that the last
 * pk_reload_release(slot) marked (the first fetch after a release makes the copy stream wait for
 * it; the copy stream runs in order, so the slot's later fetches follow).  Several fetches may
 * fill one slot.  `src_host` should be
 * page-locked (hipHostMalloc) memory: from pageable memory the runtime stages the copy through
 * the host and it no longer overlaps the compute (the Python binding requires pinned memory). */
pk_status pk_reload_fetch(pk_reload_t r, int32_t slot, void *dst, const void *src_host,
                          size_t bytes);

/* Make `hip_stream` wait until every fetch issued so far into `slot` has landed. */
pk_status pk_reload_acquire(pk_reload_t r, int32_t slot, void *hip_stream);

/* Mark the work enqueued so far on `hip_stream` as the last use of `slot`'s buffers: the next
 * fetch into the slot waits for it. */
pk_status pk_reload_release(pk_reload_t r, int32_t slot, void *hip_stream);

/* Wait for pending copies, then free the stream and events. */
pk_status pk_reload_destroy(pk_reload_t r);

/* ---- Measured roofline (measurement aids; nothing on the attention path calls them) -----
 * pk_peak_mfma: `workgroups` workgroups of 4 waves, each wave running 4 independent chains of
 * `iters` v_mfma_f32_32x32x16_f16 on register operands (32 * 32 * 16 * 2 flops each), so
 * flops = workgroups * 4 * 4 * iters * 32768; `sink` (device, >= 4 * workgroups floats) receives
 * one value per wave.  pk_peak_hbm: mode 0 reads `bytes` of `src` (sink: device, >= 1 float),
 * mode 1 writes `bytes` to `dst`, mode 2 copies; 16-byte aligned buffers, bytes % 16 == 0.
 * Both only enqueue on `hip_stream`; time them with events on that stream. */
pk_status pk_peak_mfma(float *sink, int32_t workgroups, int32_t iters, void *hip_stream);
pk_status pk_peak_hbm(int32_t mode, const void *src, void *dst, size_t bytes, float *sink,
                      void *hip_stream);

/* Human-readable name of a status code (static storage). */
const char *pk_status_str(pk_status status);

/* ---- Kernel timing (for benchmarks; off by default) -------------------------------------
 * pk_prof_enable(kinds) takes a bit mask of kernel kinds (bit k = kind k, PK_PROF_ALL for all,
 * 0 to stop; other values: PK_ERR_INVALID).  While a kind is enabled, each of its launches
 * records a pair of HIP events around it on its stream (no synchronisation; each record costs
 * a few microseconds of GPU time, so enable only the kinds to be timed).  pk_prof_query
 * synchronises on the recorded events and returns the total milliseconds and launch count of
 * one kernel kind since the last reset.  The records are process-wide and guarded by a lock, so
 * several host threads may launch while timing is on.  The events belong to the device that was
 * current at the first pk_prof_enable; launches on other devices are not recorded. */
typedef enum pk_kernel_kind {
    PK_K_META = 0,        /* all metadata-build kernels of one pk_build_meta */
    PK_K_FWD_PREP = 1,    /* forward prologue: RoPE table + rotated K */
    PK_K_FWD = 2,         /* forward attention */
    PK_K_BWD_PREP = 3,    /* backward prologue: RoPE table, rotated Q/K, rowsum(dout*out), dout scale */
    PK_K_BWD = 4,         /* backward attention, key-tile outer: dK, dV */
    PK_K_BWD_DQ = 5,      /* backward attention, query-tile outer: dQ */
    PK_K_MASK = 6,        /* pk_dense_mask */
    PK_K_ROPE = 7,        /* pk_rope_apply */
    PK_K_MOE = 8,         /* all kernels of one pk_moe_group */
    PK_K_LORA = 9,        /* all kernels of one pk_lora_qkv */
    PK_K_COUNT = 10
} pk_kernel_kind;
#define PK_PROF_ALL ((1 << PK_K_COUNT) - 1)

pk_status pk_prof_enable(int32_t kinds);
pk_status pk_prof_reset(void);
pk_status pk_prof_query(int32_t kind, double *total_ms /* host */, int64_t *launches /* host */);

#ifdef __cplusplus
}
#endif

#endif /* PK_H */
