// Host-side argument handling of every libpk entry point, built with AddressSanitizer on the host
// code (device code unchanged) and run without a GPU: each call here must return its status
// before touching the device, with no invalid host memory access.  Driven by
// tests/test_abi_asan.py; prints OK and exits 0 when every status is the expected one.
#include <cstdio>
#include <cstring>

#include "pk.h"

static int g_bad = 0;

static void expect(long got, long want, const char *what) {
    if (got != want) {
        std::printf("FAIL %s: got %ld, want %ld\n", what, got, want);
        ++g_bad;
    }
}

int main() {
    void *fake = reinterpret_cast<void *>(0x10000);   // never dereferenced
    void *unaligned = reinterpret_cast<void *>(0x10004);
    pk_meta_t h = nullptr;
    const int32_t *lens = static_cast<const int32_t *>(fake);

    // sizes and constants
    expect(pk_tile_rows(), PK_TILE_ROWS, "tile rows");
    expect(pk_meta_bytes(4, 256) > 0, 1, "meta bytes");
    expect((long)pk_meta_bytes(-1, 10), 0, "meta bytes negative");
    expect((long)pk_meta_bytes(5, 4), 0, "meta bytes n > T");
    expect((long)pk_meta_bytes(1, PK_MAX_TOKENS + 1), 0, "meta bytes too large");
    for (int s = 0; s >= -5; --s) expect(std::strlen(pk_status_str((pk_status)s)) > 0, 1, "status str");
    expect(std::strcmp(pk_status_str((pk_status)-99), "unknown status") == 0, 1, "unknown status");

    // metadata build
    expect(pk_build_meta(lens, 4, 256, fake, 1 << 20, nullptr, nullptr), PK_ERR_INVALID, "build: null out");
    expect(pk_build_meta(lens, -1, 256, fake, 1 << 20, nullptr, &h), PK_ERR_INVALID, "build: n < 0");
    expect(pk_build_meta(lens, 4, (int64_t)PK_MAX_TOKENS * 2, fake, 1 << 30, nullptr, &h), PK_ERR_UNSUPPORTED, "build: T");
    expect(pk_build_meta(nullptr, 4, 256, fake, 1 << 20, nullptr, &h), PK_ERR_INVALID, "build: lengths");
    expect(pk_build_meta(lens, 4, 256, nullptr, 1 << 20, nullptr, &h), PK_ERR_INVALID, "build: buffer");
    expect(pk_build_meta(lens, 4, 256, unaligned, 1 << 20, nullptr, &h), PK_ERR_INVALID, "build: alignment");
    expect(pk_build_meta(lens, 4, 256, fake, 16, nullptr, &h), PK_ERR_CAPACITY, "build: capacity");
    expect(pk_build_meta(lens, 300, 256, fake, 1 << 20, nullptr, &h), PK_ERR_INVALID, "build: n > T");
    expect(h == nullptr, 1, "no handle on failure");
    expect(pk_meta_view(nullptr, nullptr), PK_ERR_INVALID, "view");
    expect(pk_meta_check(nullptr, nullptr, nullptr, nullptr), PK_ERR_INVALID, "check");
    expect(pk_meta_destroy(nullptr), PK_ERR_INVALID, "destroy");

    // attention
    expect((long)pk_attn_fwd_workspace_bytes(nullptr, 2, 1, 64), 0, "fwd ws");
    expect((long)pk_attn_bwd_workspace_bytes(nullptr, 2, 1, 64), 0, "bwd ws");
    expect(pk_attn_fwd(nullptr, fake, fake, fake, 2, 1, 64, 0.125f, 1e4f, fake, (float *)fake, fake, 1 << 20,
                       nullptr), PK_ERR_INVALID, "fwd");
    expect(pk_attn_fwd_noalloc(nullptr, fake, fake, fake, 2, 1, 64, 0.125f, 1e4f, fake, (float *)fake, nullptr),
           PK_ERR_INVALID, "fwd noalloc");
    expect(pk_attn_bwd(nullptr, fake, fake, fake, fake, (const float *)fake, fake, 2, 1, 64, 0.125f, 1e4f,
                       (float *)fake, (float *)fake, (float *)fake, fake, 1 << 20, nullptr), PK_ERR_INVALID, "bwd");
    expect(pk_attn_bwd_prep(nullptr, fake, fake, fake, fake, (const float *)fake, fake, 2, 1, 64, 0.125f, 1e4f,
                            fake, 1 << 20, nullptr), PK_ERR_INVALID, "bwd prep");
    expect(pk_attn_bwd_main(nullptr, 2, 1, 64, 0.125f, (float *)fake, (float *)fake, (float *)fake, fake,
                            1 << 20, nullptr), PK_ERR_INVALID, "bwd main");

    // steps around the path
    expect(pk_dense_mask(nullptr, (uint8_t *)fake, 1 << 20, nullptr), PK_ERR_INVALID, "mask");
    expect(pk_rope_apply(nullptr, fake, 2, 64, 1e4f, 0, fake, nullptr), PK_ERR_INVALID, "rope");
    expect((long)pk_moe_group_workspace_bytes(-1, 8), 0, "moe ws");
    expect((long)pk_moe_group_workspace_bytes(16, PK_MOE_MAX_EXPERTS + 1), 0, "moe ws experts");
    const size_t mws = pk_moe_group_workspace_bytes(64, 8);
    int32_t *i32 = static_cast<int32_t *>(fake);
    expect(pk_moe_group(i32, -1, 4, 8, i32, i32, i32, i32, i32, fake, mws, nullptr), PK_ERR_INVALID, "moe n");
    expect(pk_moe_group(i32, 16, 4, 0, i32, i32, i32, i32, i32, fake, mws, nullptr), PK_ERR_UNSUPPORTED, "moe E");
    expect(pk_moe_group(i32, 16, 4, 8, i32, i32, i32, i32, i32, unaligned, mws, nullptr), PK_ERR_INVALID, "moe ws align");
    expect(pk_moe_group(i32, 16, 4, 8, i32, i32, i32, i32, i32, fake, mws - 1, nullptr), PK_ERR_CAPACITY, "moe ws size");
    expect((long)pk_lora_qkv_workspace_bytes(16, 63, 128, 4), 0, "lora ws K");
    expect((long)pk_lora_qkv_workspace_bytes(16, 64, 100, 4), 0, "lora ws N");
    expect((long)pk_lora_qkv_workspace_bytes(16, 64, 128, PK_LORA_MAX_RANK + 1), 0, "lora ws r");
    const size_t lws = pk_lora_qkv_workspace_bytes(16, 64, 128, 4);
    expect(pk_lora_qkv(fake, fake, fake, fake, 16, 64, 128, 0, 1.f, fake, fake, lws, nullptr), PK_ERR_UNSUPPORTED, "lora r");
    expect(pk_lora_qkv(fake, nullptr, fake, fake, 16, 64, 128, 4, 1.f, fake, fake, lws, nullptr), PK_ERR_INVALID, "lora w");
    expect(pk_lora_qkv(fake, fake, fake, fake, 16, 64, 128, 4, 1.f, unaligned, fake, lws, nullptr), PK_ERR_INVALID, "lora y");
    expect(pk_lora_qkv(fake, fake, fake, fake, 16, 64, 128, 4, 1.f, fake, fake, lws - 1, nullptr), PK_ERR_CAPACITY, "lora ws");
    expect(pk_reload_create(nullptr), PK_ERR_INVALID, "reload create");
    expect(pk_reload_fetch(nullptr, 0, fake, fake, 16), PK_ERR_INVALID, "reload fetch");
    expect(pk_reload_acquire(nullptr, 0, nullptr), PK_ERR_INVALID, "reload acquire");
    expect(pk_reload_release(nullptr, 0, nullptr), PK_ERR_INVALID, "reload release");
    expect(pk_reload_destroy(nullptr), PK_ERR_INVALID, "reload destroy");
    expect(pk_peak_mfma(nullptr, 1, 1, nullptr), PK_ERR_INVALID, "peak mfma");
    expect(pk_peak_hbm(0, fake, fake, 1000, (float *)fake, nullptr), PK_ERR_INVALID, "peak hbm");

    // kernel timing bookkeeping (no events are created while disabled)
    double ms = 1.0;
    int64_t n = 1;
    expect(pk_prof_enable(-1), PK_ERR_INVALID, "prof enable");
    expect(pk_prof_enable(0), PK_OK, "prof disable");
    expect(pk_prof_reset(), PK_OK, "prof reset");
    expect(pk_prof_query(PK_K_FWD, &ms, &n), PK_OK, "prof query");
    expect(n == 0 && ms == 0.0, 1, "prof empty");
    expect(pk_prof_query(99, &ms, &n), PK_ERR_INVALID, "prof kind");

    std::printf(g_bad ? "FAILED\n" : "OK\n");
    return g_bad ? 1 : 0;
}
