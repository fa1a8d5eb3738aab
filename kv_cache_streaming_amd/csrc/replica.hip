// Acknowledgement log of replicated decode steps and the restart point after a
// failure ("DejaVu: KV-Cache Streaming ...", Method details, Failure
// detection and recovery, Fig 10).  Host-only.
#include "kvs_internal.h"

#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

using namespace kvs;

struct kv_acklog {
    int32_t workers, microbatches;
    std::vector<int64_t> last;   // [x * microbatches + j]: last acknowledged step, -1 if none
};

extern "C" {

int kv_acklog_create(kv_acklog **out, int32_t workers, int32_t microbatches)
{
    if (out == nullptr)
        return set_error(KV_EINVAL, "output handle pointer is NULL");
    *out = nullptr;
    if (workers < 1 || microbatches < 1)
        return set_error(KV_EINVAL, "workers=%d and microbatches=%d must be positive", workers,
                         microbatches);
    kv_acklog *a = new (std::nothrow) kv_acklog();
    if (!a)
        return set_error(KV_EINVAL, "out of host memory for the handle");
    a->workers = workers;
    a->microbatches = microbatches;
    a->last.assign((size_t)workers * microbatches, -1);
    *out = a;
    return KV_OK;
}

int kv_acklog_destroy(kv_acklog *a)
{
    delete a;
    return KV_OK;
}

int kv_ack(kv_acklog *a, int32_t x, int32_t j, int64_t t)
{
    if (!a)
        return set_error(KV_EINVAL, "ack log handle is NULL");
    if (x < 0 || x >= a->workers || j < 0 || j >= a->microbatches || t < 0)
        return set_error(KV_ERANGE, "ack (%d, %d, %lld) outside %d workers x %d microbatches", x,
                         j, (long long)t, a->workers, a->microbatches);
    int64_t &slot = a->last[(size_t)x * a->microbatches + j];
    if (t > slot)
        slot = t;
    return KV_OK;
}

int kv_ack_restart_point(const kv_acklog *a, int32_t *j_out, int64_t *t_out)
{
    if (!a || !j_out || !t_out)
        return set_error(KV_EINVAL, "NULL argument");
    int32_t best_j = 0;
    int64_t best_t = -1;
    for (int32_t j = 0; j < a->microbatches; ++j) {
        int64_t replicated = INT64_MAX;            // last step every worker holds
        for (int32_t x = 0; x < a->workers; ++x)
            replicated = std::min(replicated, a->last[(size_t)x * a->microbatches + j]);
        const int64_t next = replicated + 1;       // first step of j to run again
        if (best_t < 0 || next < best_t) {         // earliest in (step, microbatch) order
            best_t = next;
            best_j = j;
        }
    }
    *j_out = best_j;
    *t_out = best_t;
    return KV_OK;
}

}  // extern "C"
