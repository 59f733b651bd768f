// MoE routing grouped by expert in one pass over the assignments, with no host round trip
// ([UN-2026] "如何用 Unsloth 和 NVIDIA 让 LLM 训练更快" §3 "一个更小但实用的 MoE 优化": instead
// of asking once per expert which tokens chose it -- a data-dependent query each time -- flatten
// the [n_tokens, top_k] router indices, sort them stably by expert, count per expert, build
// offsets from the counts and split the grouped list).
//
// The stable sort is a counting sort, which is what "stable sort by expert + bincount" amounts
// to when the keys are small integers:
//   k_moe_hist    one workgroup per chunk of 1024 assignments: per-expert counts of the chunk
//                 (LDS atomics), written expert-major [E][n_chunks]; ids outside [0, E) are
//                 counted per chunk as bad.
//   k_moe_scan    one workgroup per expert: exclusive scan of that expert's chunk counts, in
//                 place, and the expert's total.
//   k_moe_scatter one workgroup per chunk: the offsets (exclusive scan of the totals), then the
//                 chunk's assignments in order, 256 at a time; an assignment's grouped position
//                 is its expert's offset + the counts of that expert in earlier chunks, earlier
//                 rounds, earlier waves of this round, and earlier lanes of its wave.  The last
//                 term comes from ballots: lanes holding the same expert are found bit by bit of
//                 the expert id (ceil(log2 E) ballots), and a lane's rank is the number of such
//                 lanes below it.  That keeps ascending flat order inside every group (stable).
// Workgroup 0 of the scatter also writes offsets[0..E] and the status word, so nothing needs
// clearing beforehand.  An assignment with a bad id is not placed (its inv entry is -1), so
// every write stays inside [0, M).
#include <algorithm>

#include "pk_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Exclusive scan of one value per thread over the workgroup; returns the thread's prefix and
// the workgroup total in *total.  s_tmp holds kWaves ints.
__device__ __forceinline__ int block_excl_scan(int v, int *s_tmp, int *total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const int y = __shfl_up(x, s, 64);
        if (lane >= s) x += y;
    }
    if (lane == 63) s_tmp[w] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
        const int c = s_tmp[k];
        before += k < w ? c : 0;
        all += c;
    }
    __syncthreads();
    *total = all;
    return before + x - v;
}

__global__ __launch_bounds__(kThreads) void k_moe_hist(const int32_t *__restrict__ idx, int64_t M,
                                                       int E, int n_chunks,
                                                       int32_t *__restrict__ chunk_counts,
                                                       int32_t *__restrict__ chunk_bad) {
    __shared__ int s_hist[PK_MOE_MAX_EXPERTS];
    __shared__ int s_bad;
    for (int e = threadIdx.x; e < E; e += kThreads) s_hist[e] = 0;
    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    const int b = blockIdx.x;
    int bad = 0;
    for (int r = 0; r < PK_MOE_CHUNK / kThreads; ++r) {
        const int64_t f = (int64_t)b * PK_MOE_CHUNK + r * kThreads + threadIdx.x;
        if (f >= M) break;
        const int e = idx[f];
        if (e >= 0 && e < E)
            atomicAdd(&s_hist[e], 1);
        else
            ++bad;
    }
    if (bad) atomicAdd(&s_bad, bad);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads) chunk_counts[(int64_t)e * n_chunks + b] = s_hist[e];
    if (threadIdx.x == 0) chunk_bad[b] = s_bad;
}

__global__ __launch_bounds__(kThreads) void k_moe_scan(int n_chunks, int32_t *__restrict__ chunk_counts,
                                                       int32_t *__restrict__ counts) {
    __shared__ int s_tmp[kWaves];
    const int e = blockIdx.x;
    int32_t *row = chunk_counts + (int64_t)e * n_chunks;
    // each thread takes a run of consecutive chunks, so the scan is one pass per workgroup
    const int per = (n_chunks + kThreads - 1) / kThreads;
    const int lo = min(n_chunks, (int)threadIdx.x * per), hi = min(n_chunks, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += row[i];
    int total;
    int run = block_excl_scan(sum, s_tmp, &total);
    for (int i = lo; i < hi; ++i) {
        const int c = row[i];
        row[i] = run;
        run += c;
    }
    if (threadIdx.x == 0) counts[e] = total;
}

__global__ __launch_bounds__(kThreads) void k_moe_scatter(const int32_t *__restrict__ idx, int64_t M,
                                                          int E, int id_bits, int n_chunks,
                                                          const int32_t *__restrict__ chunk_base,
                                                          const int32_t *__restrict__ chunk_bad,
                                                          const int32_t *__restrict__ counts,
                                                          int32_t *__restrict__ offsets,
                                                          int32_t *__restrict__ perm,
                                                          int32_t *__restrict__ inv,
                                                          int32_t *__restrict__ status) {
    __shared__ int s_run[PK_MOE_MAX_EXPERTS];             // next grouped position per expert
    __shared__ int s_wave[kWaves][PK_MOE_MAX_EXPERTS];    // per-wave counts of the current round
    __shared__ int s_tmp[kWaves];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;

    // offsets = exclusive scan of the per-expert totals (E <= 4 * kThreads)
    constexpr int PER = PK_MOE_MAX_EXPERTS / kThreads;
    int c[PER], sum = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int e = PER * threadIdx.x + k;
        c[k] = e < E ? counts[e] : 0;
        sum += c[k];
    }
    int total;
    int run = block_excl_scan(sum, s_tmp, &total);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int e = PER * threadIdx.x + k;
        if (e < E) {
            s_run[e] = run + chunk_base[(int64_t)e * n_chunks + b];
            if (b == 0) offsets[e] = run;
            for (int ww = 0; ww < kWaves; ++ww) s_wave[ww][e] = 0;
        }
        run += c[k];
    }
    if (b == 0) {   // uniform over the workgroup
        int bad = 0;
        for (int i = threadIdx.x; i < n_chunks; i += kThreads) bad |= chunk_bad[i];
        bad = __syncthreads_or(bad);
        if (threadIdx.x == 0) {
            offsets[E] = total;
            status[0] = bad ? PK_MOE_BAD_EXPERT : 0;
        }
    }
    __syncthreads();

    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int r = 0; r < PK_MOE_CHUNK / kThreads; ++r) {
        const int64_t base = (int64_t)b * PK_MOE_CHUNK + r * kThreads;
        if (base >= M) break;                      // uniform over the workgroup
        const int64_t f = base + threadIdx.x;
        const int e = f < M ? idx[f] : -1;
        const bool ok = e >= 0 && e < E;
        uint64_t peers = __ballot(ok);
        for (int bit = 0; bit < id_bits; ++bit) {
            const bool one = ok && ((e >> bit) & 1);
            const uint64_t m1 = __ballot(one);
            peers &= one ? m1 : ~m1;
        }
        const int rank = __popcll(peers & below);
        if (ok && rank == 0) s_wave[w][e] = __popcll(peers);
        __syncthreads();
        if (ok) {
            int p = s_run[e] + rank;
            for (int ww = 0; ww < w; ++ww) p += s_wave[ww][e];
            perm[p] = (int32_t)f;
            inv[f] = p;
        } else if (f < M) {
            inv[f] = -1;
        }
        __syncthreads();
        for (int x = threadIdx.x; x < E; x += kThreads) {
            int add = 0;
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) {
                add += s_wave[ww][x];
                s_wave[ww][x] = 0;
            }
            s_run[x] += add;
        }
        __syncthreads();
    }
}

}  // namespace

namespace pk {

int moe_chunks(int64_t M) { return (int)std::max<int64_t>(1, (M + PK_MOE_CHUNK - 1) / PK_MOE_CHUNK); }

hipError_t launch_moe_group(const int32_t *idx, int64_t M, int E, int32_t *counts,
                            int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *status,
                            int32_t *chunk_counts, int32_t *chunk_bad, hipStream_t s) {
    const int nc = moe_chunks(M);
    int id_bits = 0;
    while ((1 << id_bits) < E) ++id_bits;
    k_moe_hist<<<nc, kThreads, 0, s>>>(idx, M, E, nc, chunk_counts, chunk_bad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_moe_scan<<<E, kThreads, 0, s>>>(nc, chunk_counts, counts);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_moe_scatter<<<nc, kThreads, 0, s>>>(idx, M, E, id_bits, nc, chunk_counts, chunk_bad, counts,
                                          offsets, perm, inv, status);
    return hipGetLastError();
}

}  // namespace pk
