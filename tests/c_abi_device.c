/* A plain C99 user of kvstream.h on the GPU: device memory from the HIP
 * runtime's C API, every buffer handed to the library as a bare pointer.
 * It fills a small cache on the host, then runs through the C ABI a ragged
 * multi-token pack, a move of the packed block to another device buffer,
 * the pack's unpack, a staged swap-out to pinned host memory, and a staging
 * ring (push, flush, restore), and writes the caches it made and every
 * result to <dir>/<name>.bin for tests/test_gpu_c_abi.py to check against
 * the oracle.  Prints "<call> <status>" per library call and "done"
 * at the end; exits non-zero at the first failure. */
#include "kvstream.h"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define L_ 3
#define B_ 3
#define H_ 2
#define D_ 64
#define S_ 100
#define STEPS 5
#define RING_R 2

static const char *g_dir;

static int hip_ok(hipError_t e, const char *what)
{
    if (e != hipSuccess) {
        printf("%s failed: %s\n", what, hipGetErrorString(e));
        return 0;
    }
    return 1;
}

static int lib_ok(int st, const char *what)
{
    printf("%s %d\n", what, st);
    if (st != KV_OK)
        printf("  error: %s\n", kv_last_error());
    return st == KV_OK;
}

static int save(const char *name, const void *p, size_t bytes)
{
    char path[1024];
    snprintf(path, sizeof path, "%s/%s.bin", g_dir, name);
    FILE *f = fopen(path, "wb");
    if (!f)
        return 0;
    const size_t n = fwrite(p, 1, bytes, f);
    fclose(f);
    return n == bytes;
}

/* device -> host copy of `bytes`, then save */
static int save_dev(const char *name, const void *dev, size_t bytes)
{
    void *h = malloc(bytes);
    int ok = h && hip_ok(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost), "hipMemcpy d2h") &&
             save(name, h, bytes);
    free(h);
    return ok;
}

int main(int argc, char **argv)
{
    if (argc != 2) {
        printf("usage: c_abi_device <output dir>\n");
        return 2;
    }
    g_dir = argv[1];
    kv_layout lay;
    if (!lib_ok(kv_layout_init(&lay, L_, B_, H_, D_, S_, KV_F16), "kv_layout_init"))
        return 1;
    const size_t elems = (size_t)L_ * B_ * H_ * D_ * S_;
    const size_t cache_bytes = elems * 2;
    uint16_t *k = malloc(cache_bytes), *v = malloc(cache_bytes);
    if (!k || !v)
        return 1;
    /* any 16-bit patterns will do: the library moves bits */
    uint32_t x = 12345u;
    for (size_t i = 0; i < elems; ++i) {
        x = x * 1664525u + 1013904223u;
        k[i] = (uint16_t)(x >> 16);
        x = x * 1664525u + 1013904223u;
        v[i] = (uint16_t)(x >> 16);
    }
    if (!save("k", k, cache_bytes) || !save("v", v, cache_bytes))
        return 1;

    void *dk, *dv, *zk, *zv;
    hipStream_t s, copy;
    if (!hip_ok(hipMalloc(&dk, cache_bytes), "hipMalloc") ||
        !hip_ok(hipMalloc(&dv, cache_bytes), "hipMalloc") ||
        !hip_ok(hipMalloc(&zk, cache_bytes), "hipMalloc") ||
        !hip_ok(hipMalloc(&zv, cache_bytes), "hipMalloc") ||
        !hip_ok(hipMemcpy(dk, k, cache_bytes, hipMemcpyHostToDevice), "hipMemcpy h2d") ||
        !hip_ok(hipMemcpy(dv, v, cache_bytes, hipMemcpyHostToDevice), "hipMemcpy h2d") ||
        !hip_ok(hipStreamCreate(&s), "hipStreamCreate") ||
        !hip_ok(hipStreamCreate(&copy), "hipStreamCreate"))
        return 1;

    /* ragged multi-token pack of every layer, then its unpack into a zeroed cache */
    const int32_t start[B_] = {0, 10, 99};
    const int32_t count[B_] = {100, 45, 1};
    const int64_t need = kv_pack_bytes(&lay, L_, count, 0);
    void *stage;
    if (need <= 0 || !hip_ok(hipMalloc(&stage, (size_t)need), "hipMalloc"))
        return 1;
    if (!lib_ok(kv_pack_tokens(&lay, dk, dv, 0, L_, start, count, stage, need, s),
                "kv_pack_tokens") ||
        !hip_ok(hipStreamSynchronize(s), "hipStreamSynchronize") ||
        !save_dev("pack", stage, (size_t)need))
        return 1;
    /* the packed block moved to a second device buffer */
    void *stage2;
    if (!hip_ok(hipMalloc(&stage2, (size_t)need), "hipMalloc") ||
        !lib_ok(kv_copy_packed(stage2, stage, need, s), "kv_copy_packed") ||
        !hip_ok(hipStreamSynchronize(s), "hipStreamSynchronize") ||
        !save_dev("copy", stage2, (size_t)need))
        return 1;
    (void)hipFree(stage2);
    if (!hip_ok(hipMemset(zk, 0, cache_bytes), "hipMemset") ||
        !hip_ok(hipMemset(zv, 0, cache_bytes), "hipMemset") ||
        !lib_ok(kv_unpack_tokens(&lay, zk, zv, 0, L_, start, count, stage, need, s),
                "kv_unpack_tokens") ||
        !hip_ok(hipStreamSynchronize(s), "hipStreamSynchronize") ||
        !save_dev("unpack_k", zk, cache_bytes) || !save_dev("unpack_v", zv, cache_bytes))
        return 1;

    /* staged swap-out through two one-layer banks to pinned host memory */
    const int64_t layer_bytes = kv_pack_bytes(&lay, 1, count, 0);
    void *bank0, *bank1, *host;
    kv_swap *e = NULL;
    hipEvent_t done;
    if (!hip_ok(hipMalloc(&bank0, (size_t)layer_bytes), "hipMalloc") ||
        !hip_ok(hipMalloc(&bank1, (size_t)layer_bytes), "hipMalloc") ||
        !hip_ok(hipHostMalloc(&host, (size_t)need, hipHostMallocDefault), "hipHostMalloc") ||
        !hip_ok(hipEventCreate(&done), "hipEventCreate"))
        return 1;
    memset(host, 0, (size_t)need);
    if (!lib_ok(kv_swap_create(&e, &lay, bank0, bank1, layer_bytes, copy, KV_XFER_AUTO),
                "kv_swap_create") ||
        !lib_ok(kv_swap_out(e, dk, dv, 0, L_, start, count, host, need, s, done), "kv_swap_out") ||
        !hip_ok(hipEventSynchronize(done), "hipEventSynchronize") || !save("swap", host, (size_t)need) ||
        !lib_ok(kv_swap_destroy(e), "kv_swap_destroy"))
        return 1;

    /* staging ring of two slots per bank: five decode steps, flush, restore */
    const int64_t slot = kv_pack_bytes(&lay, L_, NULL, 1);
    void *rb0, *rb1, *rhost;
    kv_ring *r = NULL;
    if (!hip_ok(hipMalloc(&rb0, (size_t)(RING_R * slot)), "hipMalloc") ||
        !hip_ok(hipMalloc(&rb1, (size_t)(RING_R * slot)), "hipMalloc") ||
        !hip_ok(hipHostMalloc(&rhost, (size_t)(STEPS * slot), hipHostMallocDefault),
                "hipHostMalloc"))
        return 1;
    if (!lib_ok(kv_ring_create(&r, &lay, RING_R, rb0, rb1, RING_R * slot, rhost, STEPS * slot,
                               copy, KV_XFER_AUTO),
                "kv_ring_create"))
        return 1;
    int32_t pos[STEPS][B_];
    for (int j = 0; j < STEPS; ++j) {
        pos[j][0] = 50 + j;
        pos[j][1] = 60 + j;
        pos[j][2] = 7 * j;
        if (!lib_ok(kv_ring_push(r, dk, dv, pos[j], s), "kv_ring_push"))
            return 1;
    }
    if (!save("ring_pos", pos, sizeof pos) ||
        !lib_ok(kv_ring_flush(r, s, NULL), "kv_ring_flush") ||
        !hip_ok(hipMemset(zk, 0, cache_bytes), "hipMemset") ||
        !hip_ok(hipMemset(zv, 0, cache_bytes), "hipMemset") ||
        !lib_ok(kv_ring_restore(r, zk, zv, s, NULL), "kv_ring_restore") ||
        !hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize") ||
        !save("ring", rhost, (size_t)(STEPS * slot)) ||
        !save_dev("restore_k", zk, cache_bytes) || !save_dev("restore_v", zv, cache_bytes) ||
        !lib_ok(kv_ring_destroy(r), "kv_ring_destroy"))
        return 1;

    (void)hipHostFree(host);
    (void)hipHostFree(rhost);
    (void)hipFree(stage);
    (void)hipFree(bank0);
    (void)hipFree(bank1);
    (void)hipFree(rb0);
    (void)hipFree(rb1);
    (void)hipFree(dk);
    (void)hipFree(dv);
    (void)hipFree(zk);
    (void)hipFree(zv);
    (void)hipEventDestroy(done);
    (void)hipStreamDestroy(s);
    (void)hipStreamDestroy(copy);
    free(k);
    free(v);
    printf("done\n");
    return 0;
}
