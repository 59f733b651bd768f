// Packed-batch metadata B, built once per pack on the device with no host round trip.
//
// [UN-2026] ("如何用 Unsloth 和 NVIDIA 让 LLM 训练更快", §1 "缓存 Packed-Sequence 元数据"):
// a packed batch is described by B = {lengths, cu_seqlens, max_seqlen, mask structure}; every
// layer reads the same B, so it is built once and reused, and building it must not force a
// device-to-host synchronisation.  Here the mask structure is carried by per-token sequence ids
// and positions plus two tile work lists; no T x T mask exists anywhere.
//
// Four launches, all stream-ordered:
//   k_meta_scan    one workgroup: exclusive prefix sum of the lengths (cu_seqlens), max, and the
//                  status word (a length < 1, or lengths that do not sum to T)
//   k_meta_tokens  one thread per token: its sequence (binary search in cu_seqlens) and position
//   k_meta_items   one thread per 128-token tile: the forward item (query tile -> key range) and
//                  the backward item (key tile -> query range)
//   k_meta_rank    one thread per tile: rank = #items with larger cost + #earlier items with the
//                  same cost, i.e. a stable sort by cost, largest first -- the same "group once,
//                  then use the offsets" idea as the routing change in [UN-2026] §3 -- and the
//                  offsets of each key tile's blocks in the backward's dS store.
#include "pk_internal.h"
#include "pk_device.h"

namespace {

constexpr int kScanThreads = 1024;
constexpr int kWaves = kScanThreads / 64;

__global__ __launch_bounds__(kScanThreads) void k_meta_scan(const int32_t *__restrict__ lengths,
                                                            int32_t n, int64_t T,
                                                            int32_t *__restrict__ cu,
                                                            int32_t *__restrict__ hdr) {
    __shared__ long long s_sum[kWaves];
    __shared__ int s_max[kWaves];
    __shared__ int s_bad[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (n + kScanThreads - 1) / kScanThreads;
    const int a = min(n, tid * per), b = min(n, a + per);
    long long sum = 0;
    int mx = 0, bad = 0;
    for (int i = a; i < b; ++i) {
        const int x = lengths[i];
        sum += x;
        mx = max(mx, x);
        bad |= (x < 1);
    }
    // inclusive scan of the per-thread sums inside the wave
    long long inc = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const long long y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
    }
    int wmx = mx, wbad = bad;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        wmx = max(wmx, __shfl_xor(wmx, off, 64));
        wbad |= __shfl_xor(wbad, off, 64);
    }
    if (lane == 63) s_sum[wave] = inc;
    if (lane == 0) {
        s_max[wave] = wmx;
        s_bad[wave] = wbad;
    }
    __syncthreads();
    long long wave_base = 0;
    long long total = 0;
    int gmax = 0, gbad = 0;
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave) wave_base += s_sum[w];
        total += s_sum[w];
        gmax = max(gmax, s_max[w]);
        gbad |= s_bad[w];
    }
    long long run = wave_base + inc - sum;  // exclusive prefix of this thread's chunk
    if (tid == 0) cu[0] = 0;
    for (int i = a; i < b; ++i) {
        run += lengths[i];
        cu[i + 1] = (int32_t)run;
    }
    if (tid == 0) {
        int status = 0;
        if (gbad) status |= PK_META_BAD_LENGTH;
        if (total != T) status |= PK_META_BAD_TOTAL;
        hdr[0] = status;
        hdr[1] = gmax;
        hdr[2] = 0;   // operand-range flags, set later by attention calls that see one
        hdr[3] = 0;
    }
}

__global__ __launch_bounds__(256) void k_meta_tokens(const int32_t *__restrict__ cu, int32_t n,
                                                     int64_t T, const int32_t *__restrict__ hdr,
                                                     int32_t *__restrict__ seq_id,
                                                     int32_t *__restrict__ pos) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    if (hdr[0] != 0) {
        seq_id[t] = 0;
        pos[t] = 0;
        return;
    }
    // largest s with cu[s] <= t (cu is strictly increasing when the status word is clear)
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    seq_id[t] = lo;
    pos[t] = (int32_t)(t - cu[lo]);
}

__global__ __launch_bounds__(256) void k_meta_items(const int32_t *__restrict__ cu,
                                                    const int32_t *__restrict__ seq_id, int64_t T,
                                                    int32_t n_items,
                                                    const int32_t *__restrict__ hdr,
                                                    int32_t *__restrict__ fwd_raw,
                                                    int32_t *__restrict__ bwd_raw) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_items) return;
    int32_t f[PK_ITEM_FIELDS] = {0, 0, 0, 0, 0, 0, 0, t};
    int32_t g[PK_ITEM_FIELDS] = {0, 0, 0, 0, 0, 0, 0, t};
    if (hdr[0] == 0) {
        const int R = PK_TILE_ROWS;
        const int lo = R * t;
        const int hi = (int)min((int64_t)R * (t + 1), T);
        const int sf = seq_id[lo], sl = seq_id[hi - 1];
        const int ks = cu[sf];
        f[0] = lo; f[1] = hi; f[2] = ks; f[3] = hi; f[4] = sf; f[5] = sl;
        f[6] = (hi - ks + R - 1) / R;
        const int qe = cu[sl + 1];
        g[0] = lo; g[1] = hi; g[2] = lo; g[3] = qe; g[4] = sf; g[5] = sl;
        g[6] = (qe - lo + R - 1) / R;
    }
#pragma unroll
    for (int i = 0; i < PK_ITEM_FIELDS; ++i) {
        fwd_raw[t * PK_ITEM_FIELDS + i] = f[i];
        bwd_raw[t * PK_ITEM_FIELDS + i] = g[i];
    }
}

// Query blocks of PK_DS_BLOCK_ROWS rows a backward item spans: ceil((q_end - q_start) / 64).
__device__ __forceinline__ int item_query_blocks(const int32_t *item) {
    return (item[3] - item[2] + PK_DS_BLOCK_ROWS - 1) / PK_DS_BLOCK_ROWS;
}

// Also, per key tile u (tile order), the offset of its first block in the backward's dS store:
// ds_off[u] = sum over tiles u' < u of their query blocks, and ds_off[n_items] = the total, copied
// to hdr[3] (an exclusive prefix sum formed in the same pass over the items as the ranks).
__global__ __launch_bounds__(256) void k_meta_rank(const int32_t *__restrict__ fwd_raw,
                                                   const int32_t *__restrict__ bwd_raw,
                                                   int32_t n_items, int32_t *__restrict__ fwd,
                                                   int32_t *__restrict__ bwd,
                                                   int32_t *__restrict__ ds_off,
                                                   int32_t *__restrict__ hdr) {
    __shared__ int s_cf[256];
    __shared__ int s_cb[256];
    __shared__ int s_nb[256];
    const int tid = threadIdx.x;
    const int i = blockIdx.x * blockDim.x + tid;
    const int my_f = i < n_items ? fwd_raw[i * PK_ITEM_FIELDS + 6] : 0;
    const int my_b = i < n_items ? bwd_raw[i * PK_ITEM_FIELDS + 6] : 0;
    int rank_f = 0, rank_b = 0, off = 0;
    for (int base = 0; base < n_items; base += 256) {
        __syncthreads();
        const int j = base + tid;
        s_cf[tid] = j < n_items ? fwd_raw[j * PK_ITEM_FIELDS + 6] : 0;
        s_cb[tid] = j < n_items ? bwd_raw[j * PK_ITEM_FIELDS + 6] : 0;
        s_nb[tid] = j < n_items ? item_query_blocks(bwd_raw + j * PK_ITEM_FIELDS) : 0;
        __syncthreads();
        const int m = min(256, n_items - base);
        for (int x = 0; x < m; ++x) {
            const int jj = base + x;
            const int cf = s_cf[x], cb = s_cb[x];
            rank_f += (cf > my_f) | ((cf == my_f) & (jj < i));
            rank_b += (cb > my_b) | ((cb == my_b) & (jj < i));
            off += (jj < i) ? s_nb[x] : 0;
        }
    }
    if (i < n_items) {
#pragma unroll
        for (int k = 0; k < PK_ITEM_FIELDS; ++k) {
            fwd[rank_f * PK_ITEM_FIELDS + k] = fwd_raw[i * PK_ITEM_FIELDS + k];
            bwd[rank_b * PK_ITEM_FIELDS + k] = bwd_raw[i * PK_ITEM_FIELDS + k];
        }
        ds_off[i] = off;
        if (i == n_items - 1) {
            const int total = off + item_query_blocks(bwd_raw + i * PK_ITEM_FIELDS);
            ds_off[n_items] = total;
            hdr[3] = total;
        }
    }
}

}  // namespace

namespace pk {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

MetaLayout meta_layout(int32_t n_seqs, int64_t T) {
    MetaLayout L;
    const size_t items = (size_t)n_tiles(T) * PK_ITEM_FIELDS * sizeof(int32_t);
    size_t off = 0;
    L.hdr = off; off += align256(4 * sizeof(int32_t));
    L.cu = off; off += align256((size_t)(n_seqs + 1) * sizeof(int32_t));
    L.seq_id = off; off += align256((size_t)T * sizeof(int32_t));
    L.pos = off; off += align256((size_t)T * sizeof(int32_t));
    L.fwd_items = off; off += align256(items);
    L.bwd_items = off; off += align256(items);
    L.fwd_raw = off; off += align256(items);
    L.bwd_raw = off; off += align256(items);
    L.ds_off = off; off += align256((size_t)(n_tiles(T) + 1) * sizeof(int32_t));
    L.total = off;
    return L;
}

hipError_t launch_meta(const int32_t *lengths, const pk_meta_s &m, hipStream_t stream) {
    const int64_t T = m.total_tokens;
    k_meta_scan<<<1, kScanThreads, 0, stream>>>(lengths, m.n_seqs, T, m.cu, m.hdr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || T == 0) return e;
    k_meta_tokens<<<(unsigned)((T + 255) / 256), 256, 0, stream>>>(m.cu, m.n_seqs, T, m.hdr,
                                                                   m.seq_id, m.pos);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const unsigned g = (unsigned)((m.n_items + 255) / 256);
    k_meta_items<<<g, 256, 0, stream>>>(m.cu, m.seq_id, T, m.n_items, m.hdr, m.fwd_raw, m.bwd_raw);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_meta_rank<<<g, 256, 0, stream>>>(m.fwd_raw, m.bwd_raw, m.n_items, m.fwd_items, m.bwd_items,
                                       m.ds_off, m.hdr);
    return hipGetLastError();
}

}  // namespace pk
