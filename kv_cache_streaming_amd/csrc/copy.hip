// Device-to-device move of a packed block ("DejaVu: KV-Cache Streaming ...",
// Method details, Fast prompt KV transfer; DejaVuLib primitives, Table 1):
// when the worker that packs and the worker that unpacks share a GPU, the
// packed buffer moves as a plain copy.
//
// One 16-byte vector per thread, 256 threads per workgroup, one workgroup
// per 4 KiB, non-temporal loads and stores: on MI355X this moves a 2 GiB
// buffer at 6.46 TB/s (read + write), against 6.08 TB/s with ordinary loads
// and stores and 5.4-5.9 TB/s with two to eight vectors per thread.
#include "kvs_internal.h"

#include <algorithm>

namespace kvs {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void copy_packed_kernel(const v4u *__restrict__ src,
                                                                   v4u *__restrict__ dst,
                                                                   int64_t nvec)
{
    const int64_t i = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x;
    if (i < nvec)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace
}  // namespace kvs

using namespace kvs;

extern "C" int kv_copy_packed(void *dst, const void *src, int64_t bytes, hipStream_t s)
{
    if (dst == nullptr || src == nullptr)
        return set_error(KV_EINVAL, "kv_copy_packed: NULL buffer");
    if (bytes < 0)
        return set_error(KV_ESIZE, "kv_copy_packed: negative size %lld", (long long)bytes);
    if (bytes % 16 != 0)
        return set_error(KV_EINVAL, "kv_copy_packed: %lld bytes is not a whole number of 16-byte "
                         "vectors", (long long)bytes);
    if (bytes == 0)
        return KV_OK;
    int st;
    if ((st = check_device_buffer(src, bytes, "source")) ||
        (st = check_device_buffer(dst, bytes, "destination")))
        return st;
    if (overlaps(dst, bytes, src, bytes))
        return set_error(KV_EINVAL, "kv_copy_packed: source and destination overlap");
    // launches of at most 2^31 - 1 workgroups (8 TiB each)
    constexpr int64_t kMaxBlocks = 0x7fffffffLL;
    const int64_t nvec = bytes / 16;
    for (int64_t done = 0; done < nvec; done += kMaxBlocks * kCopyThreads) {
        const int64_t n = std::min<int64_t>(nvec - done, kMaxBlocks * kCopyThreads);
        const v4u *from = (const v4u *)src + done;
        v4u *to = (v4u *)dst + done;
        int64_t count = n;
        void *args[] = {(void *)&from, (void *)&to, (void *)&count};
        const dim3 grid((unsigned)((n + kCopyThreads - 1) / kCopyThreads)), block(kCopyThreads);
        const LaunchTimer t = profile_take();
        const hipError_t e =
            t.start ? hipExtLaunchKernel((const void *)copy_packed_kernel, grid, block, args, 0, s,
                                         t.start, t.stop, 0)
                    : hipLaunchKernel((const void *)copy_packed_kernel, grid, block, args, 0, s);
        profile_commit(t, "copy_packed", 2 * n * 16, e == hipSuccess);
        if (e != hipSuccess)
            return hip_fail(e, "kv_copy_packed");
    }
    return KV_OK;
}
