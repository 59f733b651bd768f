// Two-slot reload pipeline for activations kept in pinned host memory
// ([UN-2026] "如何用 Unsloth 和 NVIDIA 让 LLM 训练更快" §2 "用双缓冲检查点重载隐藏延迟": with one
// device buffer the copy back and the backward that consumes it alternate, T ~ L (c + g); with
// two, the copy of the next layer's activations runs while the current layer computes,
// T ~ c + (L - 1) max(c, g) + g).
//
// The pipeline owns one copy stream (default priority) and two events per slot:
//   landed[s] recorded on the copy stream after the last fetch into slot s;
//   freed[s]  recorded on the compute stream after the last use of slot s.
// The first fetch into s after a release makes the copy stream wait on freed[s] (later fetches
// into s are behind that wait already: the copy stream runs in order, and each cross-queue wait
// costs the copy engine time -- measured, about 50 us per wait); an acquire makes the compute
// stream wait on landed[s].  Everything is stream-ordered: no call blocks the host.
#include <hip/hip_runtime.h>

#include <mutex>
#include <new>

#include "pk_internal.h"

struct pk_reload_s {
    int device;
    hipStream_t copy;
    hipEvent_t landed[2], freed[2];
    bool wait_pending[2];     // freed[s] was recorded and the copy stream has not waited on it
    std::mutex mu;            // fetch/release on one pipeline from several host threads
};

namespace {

void destroy_events(pk_reload_s *r) {
    for (int s = 0; s < 2; ++s) {
        if (r->landed[s]) (void)hipEventDestroy(r->landed[s]);
        if (r->freed[s]) (void)hipEventDestroy(r->freed[s]);
    }
}

bool on_device(const pk_reload_s *r) {
    int dev = -1;
    return hipGetDevice(&dev) == hipSuccess && dev == r->device;
}

}  // namespace

extern "C" {

pk_status pk_reload_create(pk_reload_t *out) {
    if (!out) return PK_ERR_INVALID;
    *out = nullptr;
    pk_reload_s *r = new (std::nothrow) pk_reload_s;
    if (!r) return PK_ERR_INVALID;
    r->copy = nullptr;
    for (int s = 0; s < 2; ++s) {
        r->landed[s] = r->freed[s] = nullptr;
        r->wait_pending[s] = false;
    }
    bool ok = hipGetDevice(&r->device) == hipSuccess &&
              hipStreamCreateWithFlags(&r->copy, hipStreamNonBlocking) == hipSuccess;
    for (int s = 0; ok && s < 2; ++s)
        ok = hipEventCreateWithFlags(&r->landed[s], hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&r->freed[s], hipEventDisableTiming) == hipSuccess;
    if (!ok) {
        destroy_events(r);
        if (r->copy) (void)hipStreamDestroy(r->copy);
        delete r;
        return PK_ERR_HIP;
    }
    *out = r;
    return PK_OK;
}

pk_status pk_reload_fetch(pk_reload_t r, int32_t slot, void *dst, const void *src_host, size_t bytes) {
    if (!r || slot < 0 || slot > 1) return PK_ERR_INVALID;
    if (bytes == 0) return PK_OK;
    if (!dst || !src_host) return PK_ERR_INVALID;
    if (!on_device(r)) return PK_ERR_INVALID;
    std::lock_guard<std::mutex> lock(r->mu);
    if (r->wait_pending[slot]) {
        if (hipStreamWaitEvent(r->copy, r->freed[slot], 0) != hipSuccess) return PK_ERR_HIP;
        r->wait_pending[slot] = false;
    }
    if (hipMemcpyAsync(dst, src_host, bytes, hipMemcpyHostToDevice, r->copy) != hipSuccess)
        return PK_ERR_HIP;
    return hipEventRecord(r->landed[slot], r->copy) == hipSuccess ? PK_OK : PK_ERR_HIP;
}

pk_status pk_reload_acquire(pk_reload_t r, int32_t slot, void *hip_stream) {
    if (!r || slot < 0 || slot > 1) return PK_ERR_INVALID;
    if (!on_device(r)) return PK_ERR_INVALID;
    std::lock_guard<std::mutex> lock(r->mu);
    return hipStreamWaitEvent(static_cast<hipStream_t>(hip_stream), r->landed[slot], 0) == hipSuccess
               ? PK_OK : PK_ERR_HIP;
}

pk_status pk_reload_release(pk_reload_t r, int32_t slot, void *hip_stream) {
    if (!r || slot < 0 || slot > 1) return PK_ERR_INVALID;
    if (!on_device(r)) return PK_ERR_INVALID;
    std::lock_guard<std::mutex> lock(r->mu);
    if (hipEventRecord(r->freed[slot], static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return PK_ERR_HIP;
    r->wait_pending[slot] = true;
    return PK_OK;
}

pk_status pk_reload_destroy(pk_reload_t r) {
    if (!r) return PK_ERR_INVALID;
    // pending copies finish before the stream goes away
    (void)hipStreamSynchronize(r->copy);
    destroy_events(r);
    (void)hipStreamDestroy(r->copy);
    delete r;
    return PK_OK;
}

}  // extern "C"
