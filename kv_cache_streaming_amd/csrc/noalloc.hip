// Swap-out that allocates nothing, for callers that cannot allocate memory
// (code under graph capture, serving loops, harnesses that forbid it).
//
// Same host bytes as kv_swap_out: the selected region is packed chunk by
// chunk into a staging buffer and each chunk is copied to the pinned host
// image by the link-copy kernel.  Here the staging buffer is the library's
// own static device array `scratch` rather than caller-provided banks, and
// every step runs on the one stream the caller passes, in stream order (the
// pack of chunk i+1 follows the copy of chunk i), so no event and no handle
// is needed.
#include "chunks.h"
#include "kvs_internal.h"

#include <mutex>

namespace {

constexpr int64_t kScratchBytes = KV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

}  // namespace

// The staging buffer, one copy per GPU that loads the library, held until the
// process ends.  In host code this name is a host-side stand-in, not the
// device address: host code uses the address from hipGetSymbolAddress below.
static __device__ __align__(256) uint4 scratch[kScratchBytes / 16];

namespace {

std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` on each device

// Device address of the current device's `scratch`, looked up once per device.
int scratch_address(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return kvs::hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return kvs::set_error(KV_EINVAL, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return kvs::hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (p == nullptr)
            return kvs::set_error(KV_EHIP, "no device address for the scratch buffer");
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return KV_OK;
}

}  // namespace

extern "C" int kv_swap_out_noalloc(const kv_layout *lay, const void *k, const void *v,
                                   int32_t layer_begin, int32_t layer_count,
                                   const int32_t *start, const int32_t *count, void *host,
                                   int64_t host_bytes, hipStream_t s)
{
    using namespace kvs;
    int st = check_layout(lay);
    if (st)
        return st;
    if ((st = check_layers(*lay, layer_begin, layer_count)))
        return st;
    RowTable rt;
    int32_t mx;
    if ((st = build_rows(*lay, start, count, &rt, &mx)))
        return st;
    const int64_t need = packed_bytes(*lay, layer_count, rt.off[lay->B]);
    if (host_bytes < need)
        return set_error(KV_ESIZE, "host holds %lld bytes, %lld needed", (long long)host_bytes,
                         (long long)need);
    if ((st = check_pinned_host(host, need, "host")))
        return st;
    void *host_dev = nullptr;
    if (need > 0 && (st = host_device_address(host, need, &host_dev)))
        return st;
    if ((st = check_device_buffer(k, lay->k_bytes, "key cache")) ||
        (st = check_device_buffer(v, lay->v_bytes, "value cache")))
        return st;
    // every (layer, row) block must fit the scratch buffer: a dry run of the
    // chunking rejects the call before anything is enqueued
    if ((st = for_each_chunk(*lay, layer_begin, layer_count, rt, kScratchBytes,
                             [](const Chunk &) { return KV_OK; }))) {
        if (st == KV_ESIZE)
            return set_error(KV_ESIZE,
                             "one layer of one row exceeds the %lld-byte scratch buffer of "
                             "kv_swap_out_noalloc; use kv_swap_out with larger banks",
                             (long long)kScratchBytes);
        return st;
    }
    if (need == 0)
        return KV_OK;
    void *buf = nullptr;
    if ((st = scratch_address(&buf)))
        return st;
    const kv_layout &L = *lay;
    return for_each_chunk(L, layer_begin, layer_count, rt, kScratchBytes, [&](const Chunk &c) {
        RowTable sub;
        int32_t cmx;
        chunk_rows(L, rt, c, &sub, &cmx);
        int rc = enqueue_copy(true, L, k, v, c.l0, c.nl, sub, cmx, buf, s);
        for (int p = 0; rc == KV_OK && p < c.pieces; ++p)
            rc = launch_link_copy((char *)host_dev + c.host_off[p], (char *)buf + c.bank_off[p],
                                  c.bytes[p], true, s);
        return rc;
    });
}
