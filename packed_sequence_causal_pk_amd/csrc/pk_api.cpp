// C-ABI layer of libpk: argument validation, buffer carving, launches, optional kernel timing.
// Every check here runs on the host before anything is enqueued; nothing here waits on the
// device except pk_meta_check and pk_prof_query, which say so in pk.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <new>
#include <vector>

#include "pk_internal.h"

// ------------------------------------------------------------------ allocation-free workspace
// The workspace of pk_attn_fwd_noalloc: a file-scope device array, one copy per device, held
// from the library's load until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory, so it is never passed anywhere: its device address is looked up
// once per device (with that device current, scratch_address below) and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[PK_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned256(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 255) == 0; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool shape_supported(int hq, int hkv, int d) {
    if (d != 64 && d != 128) return false;
    if (hkv < 1 || hq < hkv || hq > 256) return false;
    return hq % hkv == 0;
}

// ------------------------------------------------------------------ kernel timing (optional)
// The records live in one process-wide table guarded by g_prof_mu, so calls from several host
// threads may record at once.  A scope keeps its own copy of its stop event (the pool is never
// freed), so a reset while a launch is being recorded leaves nothing dangling.
struct ProfRecord {
    int kind;
    hipEvent_t start, stop;
};
struct Prof {
    uint32_t mask = 0;              // bit k: record launches of kernel kind k
    std::vector<hipEvent_t> pool;   // created once, reused after a reset
    std::vector<ProfRecord> recs;
    size_t used = 0;
};
Prof g_prof;
std::mutex g_prof_mu;
constexpr size_t kProfCapacity = 16384;  // event pairs

struct ProfScope {
    hipEvent_t stop = nullptr;
    hipStream_t stream;
    ProfScope(int kind, hipStream_t s) : stream(s) {
        std::lock_guard<std::mutex> lock(g_prof_mu);
        if (!((g_prof.mask >> kind) & 1u) || g_prof.used >= kProfCapacity) return;
        ProfRecord r;
        r.kind = kind;
        r.start = g_prof.pool[2 * g_prof.used];
        r.stop = g_prof.pool[2 * g_prof.used + 1];
        if (hipEventRecord(r.start, s) != hipSuccess) return;
        g_prof.recs.push_back(r);
        stop = r.stop;
        ++g_prof.used;
    }
    ~ProfScope() {
        if (stop) (void)hipEventRecord(stop, stream);
    }
};

pk_status hip_status(hipError_t e) { return e == hipSuccess ? PK_OK : PK_ERR_HIP; }

// ------------------------------------------------------------------ side stream of the backward
// The dK/dV and dQ kernels of one backward call are independent once the prologue has run.  When
// the dK/dV grid (one workgroup of 512 threads per item and KV head, one per compute unit) is
// too small to fill the device twice over (but not so small that the whole backward is a few
// microseconds, where the fork and join cost more than they save), the dQ kernel runs on a second stream of the same
// device (default priority), forked from and joined back into the caller's stream with events,
// and takes the compute units the dK/dV kernel leaves idle (measured: -7% backward time on the
// Llama-shaped pack, -2% on the Qwen3-0.6B-shaped one; on the Qwen3-14B-shaped pack, whose
// grid is four times the device, running the two side by side was 3-5% slower, so it stays on
// one stream).  One side stream per device, created on first use and kept for the life of the
// process; calls that use it are serialised by a mutex so the fork/join events are never
// recorded by two calls at once.
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    int cus = 0;   // compute units of the device
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];
std::mutex g_side_mu;

SideStream *side_stream(int dev) {  // caller holds g_side_mu
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    SideStream &ss = g_side[dev];
    if (!ss.cus && hipDeviceGetAttribute(&ss.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return nullptr;
    if (!ss.stream) {
        hipStream_t st = nullptr;
        hipEvent_t a = nullptr, b = nullptr;
        if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
        if (hipEventCreateWithFlags(&a, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&b, hipEventDisableTiming) != hipSuccess) {
            if (a) (void)hipEventDestroy(a);
            (void)hipStreamDestroy(st);
            return nullptr;
        }
        ss.stream = st;
        ss.fork = a;
        ss.join = b;
    }
    return &ss;
}

bool on_meta_device(const pk_meta_s *m) {
    int dev = -1;
    return hipGetDevice(&dev) == hipSuccess && dev == m->device;
}

void *g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on device `dev` (the current device), or null on a HIP error.
void *scratch_address(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

namespace pk {

FwdWorkspace fwd_workspace(int64_t T, int hq, int hkv, int d) {
    (void)hq;
    FwdWorkspace w;
    size_t off = 0;
    w.krot = off; off += align256((size_t)T * hkv * d * 2);
    w.vh = off; off += align256((size_t)T * hkv * d * 2);
    w.rope = off; off += align256((size_t)T * (d / 2) * 8);
    w.total = off;
    return w;
}

BwdWorkspace bwd_workspace(int64_t T, int hq, int hkv, int d) {
    BwdWorkspace w;
    size_t off = 0;
    w.qrot = off; off += align256((size_t)T * hq * d * 2);
    w.krot = off; off += align256((size_t)T * hkv * d * 2);
    w.vh = off; off += align256((size_t)T * hkv * d * 2);
    w.dout16 = off; off += align256((size_t)T * hq * d * 2);
    w.rope = off; off += align256((size_t)T * (d / 2) * 8);
    w.dsum = off; off += align256((size_t)T * hq * 4);
    w.lse2 = off; off += align256((size_t)T * hq * 4);
    w.blockmax = off; off += align256((size_t)(dmax_blocks(T, hq, d) + vmax_blocks(T, hkv, d)) * 4);
    w.scale = off; off += align256(4 * 4);
    w.sched = off; off += align256(kSchedInts * 4);
    w.total = off;
    return w;
}

int64_t ds_bound_blocks(int64_t T, int64_t max_seqlen_bound) {
    // A key tile u's backward item spans the queries from its first row to the end of the last
    // sequence it touches; that sequence starts inside the tile, so the span is at most
    // min(T - 128 u, max_seqlen + 127) rows.
    const int64_t L = (max_seqlen_bound > 0 && max_seqlen_bound < T) ? max_seqlen_bound : T;
    const int64_t per_item = (L + PK_TILE_ROWS - 1 + PK_DS_BLOCK_ROWS - 1) / PK_DS_BLOCK_ROWS;
    int64_t total = 0;
    for (int64_t u = 0; u * PK_TILE_ROWS < T; ++u)
        total += std::min<int64_t>((T - PK_TILE_ROWS * u + PK_DS_BLOCK_ROWS - 1) / PK_DS_BLOCK_ROWS, per_item);
    return total;
}

unsigned persistent_grid(const void *kernel, int threads) {
    struct Entry {
        int dev;
        const void *kernel;
        unsigned grid;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry &e : cache)
        if (e.dev == dev && e.kernel == kernel) return e.grid;
    int cus = 0, per_cu = 0;
    unsigned grid = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) == hipSuccess &&
        cus > 0 && per_cu > 0)
        grid = (unsigned)(cus * per_cu) & ~7u;
    cache.push_back({dev, kernel, grid});
    return grid;
}

}  // namespace pk

extern "C" {

int32_t pk_tile_rows(void) { return PK_TILE_ROWS; }

size_t pk_meta_bytes(int32_t n_seqs, int64_t total_tokens) {
    if (n_seqs < 0 || total_tokens < 0 || total_tokens > PK_MAX_TOKENS || n_seqs > total_tokens) return 0;
    return pk::meta_layout(n_seqs, total_tokens).total;
}

pk_status pk_build_meta(const int32_t *lengths_dev, int32_t n_seqs, int64_t total_tokens,
                        void *meta_buf_dev, size_t meta_buf_bytes, void *hip_stream,
                        pk_meta_t *out) {
    if (!out) return PK_ERR_INVALID;
    *out = nullptr;
    if (n_seqs < 0 || total_tokens < 0 || n_seqs > total_tokens) return PK_ERR_INVALID;
    if (total_tokens > PK_MAX_TOKENS) return PK_ERR_UNSUPPORTED;
    if (n_seqs > 0 && !lengths_dev) return PK_ERR_INVALID;
    if (!meta_buf_dev || !aligned256(meta_buf_dev)) return PK_ERR_INVALID;
    const pk::MetaLayout L = pk::meta_layout(n_seqs, total_tokens);
    if (meta_buf_bytes < L.total) return PK_ERR_CAPACITY;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return PK_ERR_HIP;

    pk_meta_s *m = new (std::nothrow) pk_meta_s;
    if (!m) return PK_ERR_INVALID;
    char *base = static_cast<char *>(meta_buf_dev);
    m->hdr = reinterpret_cast<int32_t *>(base + L.hdr);
    m->cu = reinterpret_cast<int32_t *>(base + L.cu);
    m->seq_id = reinterpret_cast<int32_t *>(base + L.seq_id);
    m->pos = reinterpret_cast<int32_t *>(base + L.pos);
    m->fwd_items = reinterpret_cast<int32_t *>(base + L.fwd_items);
    m->bwd_items = reinterpret_cast<int32_t *>(base + L.bwd_items);
    m->fwd_raw = reinterpret_cast<int32_t *>(base + L.fwd_raw);
    m->bwd_raw = reinterpret_cast<int32_t *>(base + L.bwd_raw);
    m->ds_off = reinterpret_cast<int32_t *>(base + L.ds_off);
    m->n_seqs = n_seqs;
    m->total_tokens = total_tokens;
    m->n_items = (int32_t)pk::n_tiles(total_tokens);
    m->device = dev;

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e;
    {
        ProfScope ps(PK_K_META, s);
        e = pk::launch_meta(lengths_dev, *m, s);
    }
    if (e != hipSuccess) {
        delete m;
        return PK_ERR_HIP;
    }
    *out = m;
    return PK_OK;
}

pk_status pk_meta_view(pk_meta_t meta, pk_meta_view_t *view) {
    if (!meta || !view) return PK_ERR_INVALID;
    view->cu_seqlens = meta->cu;
    view->max_seqlen = meta->hdr + 1;
    view->status = meta->hdr;
    view->seq_id = meta->seq_id;
    view->pos = meta->pos;
    view->fwd_items = meta->fwd_items;
    view->bwd_items = meta->bwd_items;
    view->n_seqs = meta->n_seqs;
    view->n_items = meta->n_items;
    view->total_tokens = meta->total_tokens;
    view->device = meta->device;
    view->ds_off = meta->ds_off;
    return PK_OK;
}

pk_status pk_meta_check(pk_meta_t meta, void *hip_stream, int32_t *status_host,
                        int32_t *max_seqlen_host) {
    if (!meta) return PK_ERR_INVALID;
    if (!on_meta_device(meta)) return PK_ERR_INVALID;
    int32_t hdr[3] = {0, 0, 0};
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (hipMemcpyAsync(hdr, meta->hdr, sizeof(hdr), hipMemcpyDeviceToHost, s) != hipSuccess) return PK_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return PK_ERR_HIP;
    const int32_t status = hdr[0] | hdr[2];   // build status bits | operand-range flags
    if (status_host) *status_host = status;
    if (max_seqlen_host) *max_seqlen_host = hdr[1];
    return status ? PK_ERR_DEVICE : PK_OK;
}

pk_status pk_meta_destroy(pk_meta_t meta) {
    if (!meta) return PK_ERR_INVALID;
    delete meta;
    return PK_OK;
}

size_t pk_attn_fwd_workspace_bytes(pk_meta_t meta, int32_t hq, int32_t hkv, int32_t d) {
    if (!meta || !shape_supported(hq, hkv, d)) return 0;
    return pk::fwd_workspace(meta->total_tokens, hq, hkv, d).total;
}

size_t pk_attn_bwd_workspace_bytes(pk_meta_t meta, int32_t hq, int32_t hkv, int32_t d) {
    if (!meta || !shape_supported(hq, hkv, d)) return 0;
    return pk::bwd_workspace(meta->total_tokens, hq, hkv, d).total;
}

size_t pk_attn_bwd_workspace_bytes_ds(pk_meta_t meta, int32_t hq, int32_t hkv, int32_t d,
                                      int64_t max_seqlen_bound) {
    if (!meta || !shape_supported(hq, hkv, d)) return 0;
    const int64_t T = meta->total_tokens;
    const size_t blocks = (size_t)pk::ds_bound_blocks(T, max_seqlen_bound);
    return pk::bwd_workspace(T, hq, hkv, d).total + align256(blocks * (size_t)hq * pk::kDsBlockBytes);
}

// The forward on a workspace `w` the caller has checked for size and alignment.
static pk_status attn_fwd_on(pk_meta_t meta, const void *q, const void *k, const void *v, int32_t hq,
                             int32_t hkv, int32_t d, float softmax_scale, float rope_base, void *out,
                             float *lse, char *w, hipStream_t s) {
    const int64_t T = meta->total_tokens;
    const pk::FwdWorkspace W = pk::fwd_workspace(T, hq, hkv, d);
    pk::RopeArgs ra{meta->pos, T, hq, hkv, d, rope_base};
    hipError_t e;
    {
        ProfScope ps(PK_K_FWD_PREP, s);
        e = pk::launch_fwd_prep(ra, k, v, w + W.krot, w + W.vh, w + W.rope, meta->hdr + 2, s);
    }
    if (e != hipSuccess) return PK_ERR_HIP;
    pk::AttnShape sh{T, hq, hkv, d, meta->n_items, softmax_scale};
    {
        ProfScope ps(PK_K_FWD, s);
        e = pk::launch_fwd(sh, *meta, q, w + W.krot, w + W.vh, w + W.rope, out, lse, s);
    }
    return hip_status(e);
}

pk_status pk_attn_fwd(pk_meta_t meta, const void *q, const void *k, const void *v, int32_t hq,
                      int32_t hkv, int32_t d, float softmax_scale, float rope_base, void *out,
                      float *lse, void *ws, size_t ws_bytes, void *hip_stream) {
    if (!meta) return PK_ERR_INVALID;
    if (!shape_supported(hq, hkv, d)) return PK_ERR_UNSUPPORTED;
    if (!(softmax_scale > 0.f) || !(rope_base > 0.f)) return PK_ERR_INVALID;
    const int64_t T = meta->total_tokens;
    if (T == 0) return PK_OK;
    if (!q || !k || !v || !out || !lse || !ws || !aligned256(ws)) return PK_ERR_INVALID;
    if (ws_bytes < pk::fwd_workspace(T, hq, hkv, d).total) return PK_ERR_CAPACITY;
    if (!on_meta_device(meta)) return PK_ERR_INVALID;
    return attn_fwd_on(meta, q, k, v, hq, hkv, d, softmax_scale, rope_base, out, lse,
                       static_cast<char *>(ws), static_cast<hipStream_t>(hip_stream));
}

pk_status pk_attn_fwd_noalloc(pk_meta_t meta, const void *q, const void *k, const void *v,
                              int32_t hq, int32_t hkv, int32_t d, float softmax_scale,
                              float rope_base, void *out, float *lse, void *hip_stream) {
    if (!meta) return PK_ERR_INVALID;
    if (!shape_supported(hq, hkv, d)) return PK_ERR_UNSUPPORTED;
    if (!(softmax_scale > 0.f) || !(rope_base > 0.f)) return PK_ERR_INVALID;
    const int64_t T = meta->total_tokens;
    if (T == 0) return PK_OK;
    if (!q || !k || !v || !out || !lse) return PK_ERR_INVALID;
    if (pk::fwd_workspace(T, hq, hkv, d).total > (size_t)PK_NOALLOC_SCRATCH_BYTES) return PK_ERR_CAPACITY;
    if (!on_meta_device(meta)) return PK_ERR_INVALID;
    char *w = static_cast<char *>(scratch_address(meta->device));
    if (!w) return PK_ERR_HIP;
    return attn_fwd_on(meta, q, k, v, hq, hkv, d, softmax_scale, rope_base, out, lse, w,
                       static_cast<hipStream_t>(hip_stream));
}

pk_status pk_attn_bwd_prep(pk_meta_t meta, const void *q, const void *k, const void *v,
                           const void *out, const float *lse, const void *dout, int32_t hq,
                           int32_t hkv, int32_t d, float softmax_scale, float rope_base, void *ws,
                           size_t ws_bytes, void *hip_stream) {
    if (!meta) return PK_ERR_INVALID;
    if (!shape_supported(hq, hkv, d)) return PK_ERR_UNSUPPORTED;
    if (!(softmax_scale > 0.f) || !(rope_base > 0.f)) return PK_ERR_INVALID;
    const int64_t T = meta->total_tokens;
    if (T == 0) return PK_OK;
    if (!q || !k || !v || !out || !lse || !dout || !ws || !aligned256(ws)) return PK_ERR_INVALID;
    const pk::BwdWorkspace W = pk::bwd_workspace(T, hq, hkv, d);
    if (ws_bytes < W.total) return PK_ERR_CAPACITY;
    if (!on_meta_device(meta)) return PK_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    char *w = static_cast<char *>(ws);
    pk::RopeArgs ra{meta->pos, T, hq, hkv, d, rope_base};
    ProfScope ps(PK_K_BWD_PREP, s);
    return hip_status(pk::launch_bwd_prep(
        ra, q, k, v, out, dout, lse, w + W.qrot, w + W.krot, w + W.vh, w + W.dout16, w + W.rope,
        reinterpret_cast<float *>(w + W.dsum), reinterpret_cast<float *>(w + W.lse2),
        reinterpret_cast<float *>(w + W.blockmax), reinterpret_cast<float *>(w + W.scale),
        softmax_scale * 1.4426950408889634f, meta->hdr + 2, reinterpret_cast<int32_t *>(w + W.sched),
        s));
}

pk_status pk_attn_bwd_main(pk_meta_t meta, int32_t hq, int32_t hkv, int32_t d,
                           float softmax_scale, float *dq, float *dk, float *dv, void *ws,
                           size_t ws_bytes, void *hip_stream) {
    if (!meta) return PK_ERR_INVALID;
    if (!shape_supported(hq, hkv, d)) return PK_ERR_UNSUPPORTED;
    if (!(softmax_scale > 0.f)) return PK_ERR_INVALID;
    const int64_t T = meta->total_tokens;
    if (T == 0) return PK_OK;
    if (!dq || !dk || !dv || !ws || !aligned256(ws)) return PK_ERR_INVALID;
    const pk::BwdWorkspace W = pk::bwd_workspace(T, hq, hkv, d);
    if (ws_bytes < W.total) return PK_ERR_CAPACITY;
    if (!on_meta_device(meta)) return PK_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    char *w = static_cast<char *>(ws);
    const float *dsum = reinterpret_cast<const float *>(w + W.dsum);
    const float *lse2 = reinterpret_cast<const float *>(w + W.lse2);
    const float *scale = reinterpret_cast<const float *>(w + W.scale);
    pk::AttnShape sh{T, hq, hkv, d, meta->n_items, softmax_scale};
    // the rest of the workspace, if any, is the dS store
    pk::DsStore ds{nullptr, 0};
    if (ws_bytes > W.total) {
        ds.cap_blocks = (int64_t)((ws_bytes - W.total) / ((size_t)hq * pk::kDsBlockBytes));
        if (ds.cap_blocks > 0) ds.ptr = w + W.total;
    }
    if (ds.ptr) {
        // dK/dV first (it writes the store when the pack's blocks fit), then dQ on the same
        // stream; the device falls back to the recomputing dQ when they do not
        hipError_t e;
        {
            ProfScope ps(PK_K_BWD, s);
            e = pk::launch_bwd_kv(sh, *meta, w + W.qrot, w + W.krot, w + W.vh, w + W.dout16, lse2,
                                  dsum, scale, w + W.rope, dk, dv, ds,
                                  reinterpret_cast<int32_t *>(w + W.sched), s);
        }
        if (e != hipSuccess) return PK_ERR_HIP;
        ProfScope ps(PK_K_BWD_DQ, s);
        return hip_status(pk::launch_bwd_q(sh, *meta, w + W.qrot, w + W.krot, w + W.vh, w + W.dout16,
                                           lse2, dsum, scale, w + W.rope, dq, ds, s));
    }
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream *side = side_stream(meta->device);
    hipStream_t sq = s;   // stream of the dQ kernel
    const int64_t kv_grid = (int64_t)meta->n_items * hkv;
    if (side && kv_grid >= 64 && kv_grid <= 2 * (int64_t)side->cus && hipEventRecord(side->fork, s) == hipSuccess &&
        hipStreamWaitEvent(side->stream, side->fork, 0) == hipSuccess)
        sq = side->stream;
    hipError_t e;
    {
        ProfScope ps(PK_K_BWD_DQ, sq);
        e = pk::launch_bwd_q(sh, *meta, w + W.qrot, w + W.krot, w + W.vh, w + W.dout16, lse2, dsum,
                             scale, w + W.rope, dq, ds, sq);
    }
    hipError_t e2;
    {
        ProfScope ps(PK_K_BWD, s);
        e2 = pk::launch_bwd_kv(sh, *meta, w + W.qrot, w + W.krot, w + W.vh, w + W.dout16, lse2, dsum,
                               scale, w + W.rope, dk, dv, ds, reinterpret_cast<int32_t *>(w + W.sched),
                               s);
    }
    if (sq != s) {
        // join: the caller's stream continues only after the dQ kernel
        if (hipEventRecord(side->join, sq) != hipSuccess || hipStreamWaitEvent(s, side->join, 0) != hipSuccess)
            return PK_ERR_HIP;
    }
    if (e != hipSuccess) return PK_ERR_HIP;
    return hip_status(e2);
}

pk_status pk_attn_bwd(pk_meta_t meta, const void *q, const void *k, const void *v,
                      const void *out, const float *lse, const void *dout, int32_t hq,
                      int32_t hkv, int32_t d, float softmax_scale, float rope_base, float *dq,
                      float *dk, float *dv, void *ws, size_t ws_bytes, void *hip_stream) {
    if (meta && meta->total_tokens > 0 && (!dq || !dk || !dv)) return PK_ERR_INVALID;
    const pk_status st = pk_attn_bwd_prep(meta, q, k, v, out, lse, dout, hq, hkv, d, softmax_scale,
                                          rope_base, ws, ws_bytes, hip_stream);
    if (st != PK_OK) return st;
    return pk_attn_bwd_main(meta, hq, hkv, d, softmax_scale, dq, dk, dv, ws, ws_bytes, hip_stream);
}

pk_status pk_dense_mask(pk_meta_t meta, uint8_t *mask, size_t mask_bytes, void *hip_stream) {
    if (!meta) return PK_ERR_INVALID;
    const int64_t T = meta->total_tokens;
    if (T > PK_MASK_MAX_TOKENS) return PK_ERR_UNSUPPORTED;
    if (T == 0) return PK_OK;
    if (!mask || (reinterpret_cast<uintptr_t>(mask) & 15)) return PK_ERR_INVALID;
    if (mask_bytes < (size_t)(T * T)) return PK_ERR_CAPACITY;
    if (!on_meta_device(meta)) return PK_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    ProfScope ps(PK_K_MASK, s);
    return hip_status(pk::launch_dense_mask(*meta, mask, s));
}

pk_status pk_rope_apply(pk_meta_t meta, const void *x, int32_t h, int32_t d, float rope_base,
                        int32_t inverse, void *out, void *hip_stream) {
    if (!meta) return PK_ERR_INVALID;
    if ((d != 64 && d != 128) || h < 1 || h > 1024) return PK_ERR_UNSUPPORTED;
    if (!(rope_base > 0.f)) return PK_ERR_INVALID;
    if (meta->total_tokens == 0) return PK_OK;
    if (!x || !out || (reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(out) & 15))
        return PK_ERR_INVALID;
    if (!on_meta_device(meta)) return PK_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    ProfScope ps(PK_K_ROPE, s);
    return hip_status(pk::launch_rope_apply(*meta, x, h, d, rope_base, inverse ? 1 : 0, out, s));
}

size_t pk_moe_group_workspace_bytes(int64_t n_assign, int32_t n_experts) {
    if (n_assign < 0 || n_assign > PK_MOE_MAX_ASSIGN || n_experts < 1 || n_experts > PK_MOE_MAX_EXPERTS)
        return 0;
    const size_t nc = (size_t)pk::moe_chunks(n_assign);
    return align256(nc * (size_t)n_experts * 4) + align256(nc * 4);
}

pk_status pk_moe_group(const int32_t *router_indices, int64_t n_tokens, int32_t top_k,
                       int32_t n_experts, int32_t *counts, int32_t *offsets, int32_t *perm,
                       int32_t *inv, int32_t *status, void *ws, size_t ws_bytes,
                       void *hip_stream) {
    if (n_tokens < 0 || top_k < 1) return PK_ERR_INVALID;
    if (n_experts < 1 || n_experts > PK_MOE_MAX_EXPERTS) return PK_ERR_UNSUPPORTED;
    if (n_tokens > PK_MOE_MAX_ASSIGN / top_k) return PK_ERR_UNSUPPORTED;
    const int64_t M = n_tokens * top_k;
    if (!counts || !offsets || !status || !ws || !aligned256(ws)) return PK_ERR_INVALID;
    if (M > 0 && (!router_indices || !perm || !inv)) return PK_ERR_INVALID;
    if (ws_bytes < pk_moe_group_workspace_bytes(M, n_experts)) return PK_ERR_CAPACITY;
    const size_t nc = (size_t)pk::moe_chunks(M);
    char *w = static_cast<char *>(ws);
    int32_t *chunk_counts = reinterpret_cast<int32_t *>(w);
    int32_t *chunk_bad = reinterpret_cast<int32_t *>(w + align256(nc * (size_t)n_experts * 4));
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    ProfScope ps(PK_K_MOE, s);
    return hip_status(pk::launch_moe_group(router_indices, M, n_experts, counts, offsets, perm, inv,
                                           status, chunk_counts, chunk_bad, s));
}

static bool lora_shape_ok(int64_t T, int32_t K, int32_t N, int32_t r) {
    return T >= 0 && T <= PK_MAX_TOKENS && K >= 64 && K % 64 == 0 && K <= 65536 && N >= 128 &&
           N % 128 == 0 && N <= 65536 && r >= 1 && r <= PK_LORA_MAX_RANK;
}

size_t pk_lora_qkv_workspace_bytes(int64_t T, int32_t K, int32_t N, int32_t r) {
    if (!lora_shape_ok(T, K, N, r)) return 0;
    return pk::lora_workspace(T, K, N).total;
}

pk_status pk_lora_qkv(const void *x, const void *wt, const void *at, const void *bt, int64_t T,
                      int32_t K, int32_t N, int32_t r, float scale, void *y, void *ws,
                      size_t ws_bytes, void *hip_stream) {
    if (!lora_shape_ok(T, K, N, r)) return PK_ERR_UNSUPPORTED;
    if (!(scale == scale)) return PK_ERR_INVALID;
    if (!wt || !at || !bt || !ws || !aligned256(ws)) return PK_ERR_INVALID;
    if (T > 0 && (!x || !y)) return PK_ERR_INVALID;
    const uintptr_t align = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(wt) |
                            reinterpret_cast<uintptr_t>(at) | reinterpret_cast<uintptr_t>(bt) |
                            reinterpret_cast<uintptr_t>(y);
    if (align & 15) return PK_ERR_INVALID;
    if (ws_bytes < pk::lora_workspace(T, K, N).total) return PK_ERR_CAPACITY;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    ProfScope ps(PK_K_LORA, s);
    return hip_status(pk::launch_lora_qkv(x, wt, at, bt, T, K, N, r, scale, y, ws, s));
}

const char *pk_status_str(pk_status status) {
    switch (status) {
        case PK_OK: return "ok";
        case PK_ERR_INVALID: return "invalid argument";
        case PK_ERR_UNSUPPORTED: return "unsupported shape";
        case PK_ERR_CAPACITY: return "buffer too small";
        case PK_ERR_HIP: return "HIP runtime error";
        case PK_ERR_DEVICE: return "device status word set (invalid pack lengths)";
    }
    return "unknown status";
}

pk_status pk_prof_enable(int32_t kinds) {
    if (kinds < 0 || kinds > PK_PROF_ALL) return PK_ERR_INVALID;
    std::lock_guard<std::mutex> lock(g_prof_mu);
    if (kinds && g_prof.pool.empty()) {
        std::vector<hipEvent_t> pool(2 * kProfCapacity, nullptr);
        for (size_t e = 0; e < pool.size(); ++e)
            if (hipEventCreate(&pool[e]) != hipSuccess) {
                for (size_t x = 0; x < e; ++x) (void)hipEventDestroy(pool[x]);
                return PK_ERR_HIP;
            }
        g_prof.pool.swap(pool);
        g_prof.recs.reserve(kProfCapacity);
    }
    g_prof.mask = (uint32_t)kinds;
    return PK_OK;
}

pk_status pk_prof_reset(void) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof.recs.clear();
    g_prof.used = 0;
    return PK_OK;
}

pk_status pk_prof_query(int32_t kind, double *total_ms, int64_t *launches) {
    if (!total_ms || !launches || kind < 0 || kind >= PK_K_COUNT) return PK_ERR_INVALID;
    std::vector<ProfRecord> recs;
    {
        std::lock_guard<std::mutex> lock(g_prof_mu);
        for (const ProfRecord &r : g_prof.recs)
            if (r.kind == kind) recs.push_back(r);
    }
    double sum = 0.0;
    for (const ProfRecord &r : recs) {
        if (hipEventSynchronize(r.stop) != hipSuccess) return PK_ERR_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return PK_ERR_HIP;
        sum += ms;
    }
    *total_ms = sum;
    *launches = (int64_t)recs.size();
    return PK_OK;
}

}  // extern "C"
