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

// ---------------------------------------------------------------------------
// Microbatch swapping on two device slots ("DejaVu: KV-Cache Streaming ...",
// Method details, Microbatch swapping workflow, Fig 9) and the break-even
// test of its Appendix E.

struct kv_mbswap {
    kv_layout lay;
    int32_t n;
    void *k[2], *v[2];
    kv_swap *in;
    std::vector<kv_ring *> rings;
    std::vector<void *> prompt_host;
    std::vector<int64_t> prompt_bytes;
    std::vector<int32_t> prompt_len;   // n * B
    hipStream_t swap;
    hipEvent_t read_done;              // the push of the leaving microbatch has read its slot
    hipEvent_t loaded[2];              // slot s holds its microbatch
    int64_t round;
    bool started;
};

namespace {

int mb_event(hipEvent_t *e)
{
    const hipError_t r = hipEventCreateWithFlags(e, hipEventDisableTiming);
    return r == hipSuccess ? KV_OK : hip_fail(r, "hipEventCreateWithFlags");
}

// Swap microbatch x into slot s on the swap stream: prompt image, then steps.
int mb_swap_in(kv_mbswap *m, int32_t x, int s)
{
    const int32_t B = m->lay.B;
    std::vector<int32_t> zero(B, 0);
    int st = kv_swap_in(m->in, m->k[s], m->v[s], 0, m->lay.L, zero.data(),
                        &m->prompt_len[(size_t)x * B], m->prompt_host[x], m->prompt_bytes[x],
                        m->swap, nullptr);
    if (st)
        return st;
    if ((st = kv_ring_restore(m->rings[x], m->k[s], m->v[s], m->swap, nullptr)))
        return st;
    const hipError_t r = hipEventRecord(m->loaded[s], m->swap);
    return r == hipSuccess ? KV_OK : hip_fail(r, "mbswap loaded");
}

}  // namespace

extern "C" {

int kv_mbswap_create(kv_mbswap **out, const kv_layout *lay, int32_t microbatches,
                     void *slot0_k, void *slot0_v, void *slot1_k, void *slot1_v,
                     kv_swap *in, kv_ring *const *rings, void *const *prompt_host,
                     const int64_t *prompt_bytes, const int32_t *prompt_len,
                     hipStream_t swap_stream)
{
    if (out == nullptr)
        return set_error(KV_EINVAL, "output handle pointer is NULL");
    *out = nullptr;
    int st = check_layout(lay);
    if (st)
        return st;
    if (microbatches < 2)
        return set_error(KV_EINVAL, "microbatches=%d must be at least 2", microbatches);
    if (!in || !rings || !prompt_host || !prompt_bytes || !prompt_len)
        return set_error(KV_EINVAL, "NULL engine, ring, prompt or length array");
    void *slots[4] = {slot0_k, slot0_v, slot1_k, slot1_v};
    for (int i = 0; i < 4; ++i) {
        const int64_t bytes = (i % 2 == 0) ? lay->k_bytes : lay->v_bytes;
        if ((st = check_device_buffer(slots[i], bytes, "slot cache")))
            return st;
        for (int j = 0; j < i; ++j) {
            const int64_t jb = (j % 2 == 0) ? lay->k_bytes : lay->v_bytes;
            if (overlaps(slots[i], bytes, slots[j], jb))
                return set_error(KV_EINVAL, "slot caches overlap");
        }
    }
    for (int32_t x = 0; x < microbatches; ++x) {
        if (!rings[x])
            return set_error(KV_EINVAL, "ring %d is NULL", x);
        for (int32_t b = 0; b < lay->B; ++b) {
            const int32_t len = prompt_len[(size_t)x * lay->B + b];
            if (len < 0 || len > lay->Smax)
                return set_error(KV_ERANGE, "microbatch %d row %d: prompt length %d", x, b, len);
        }
    }
    kv_mbswap *m = new (std::nothrow) kv_mbswap();
    if (!m)
        return set_error(KV_EINVAL, "out of host memory for the handle");
    m->lay = *lay;
    m->n = microbatches;
    m->k[0] = slot0_k;
    m->v[0] = slot0_v;
    m->k[1] = slot1_k;
    m->v[1] = slot1_v;
    m->in = in;
    m->rings.assign(rings, rings + microbatches);
    m->prompt_host.assign(prompt_host, prompt_host + microbatches);
    m->prompt_bytes.assign(prompt_bytes, prompt_bytes + microbatches);
    m->prompt_len.assign(prompt_len, prompt_len + (size_t)microbatches * lay->B);
    m->swap = swap_stream;
    m->round = 0;
    m->started = false;
    m->read_done = m->loaded[0] = m->loaded[1] = nullptr;
    if ((st = mb_event(&m->read_done)) || (st = mb_event(&m->loaded[0])) ||
        (st = mb_event(&m->loaded[1]))) {
        kv_mbswap_destroy(m);
        return st;
    }
    *out = m;
    return KV_OK;
}

int kv_mbswap_destroy(kv_mbswap *m)
{
    if (!m)
        return KV_OK;
    for (hipEvent_t e : {m->read_done, m->loaded[0], m->loaded[1]})
        if (e)
            (void)hipEventDestroy(e);
    delete m;
    return KV_OK;
}

int kv_mbswap_start(kv_mbswap *m, hipStream_t compute)
{
    if (!m)
        return set_error(KV_EINVAL, "mbswap handle is NULL");
    if (m->started)
        return set_error(KV_EBUSY, "already started");
    int st;
    if ((st = mb_swap_in(m, 0, 0)) || (st = mb_swap_in(m, 1, 1)))
        return st;
    const hipError_t r = hipStreamWaitEvent(compute, m->loaded[0], 0);
    if (r != hipSuccess)
        return hip_fail(r, "mbswap start wait");
    m->started = true;
    return KV_OK;
}

int kv_mbswap_current(const kv_mbswap *m, int32_t *x, void **k, void **v)
{
    if (!m || !x || !k || !v)
        return set_error(KV_EINVAL, "NULL argument");
    const int s = (int)(m->round & 1);
    *x = (int32_t)(m->round % m->n);
    *k = m->k[s];
    *v = m->v[s];
    return KV_OK;
}

int kv_mbswap_round(kv_mbswap *m, const int32_t *pos, hipStream_t compute)
{
    if (!m)
        return set_error(KV_EINVAL, "mbswap handle is NULL");
    if (!m->started)
        return set_error(KV_EBUSY, "call kv_mbswap_start first");
    const int s = (int)(m->round & 1);
    const int32_t x = (int32_t)(m->round % m->n);
    // incremental swap-out of the step's update
    int st = kv_ring_push(m->rings[x], m->k[s], m->v[s], pos, compute);
    if (st)
        return st;
    if ((st = kv_ring_flush(m->rings[x], compute, nullptr)))
        return st;
    // microbatch x+2 moves into the slot x leaves, once the push has read it
    if (m->n > 2) {
        hipError_t r = hipEventRecord(m->read_done, compute);
        if (r == hipSuccess)
            r = hipStreamWaitEvent(m->swap, m->read_done, 0);
        if (r != hipSuccess)
            return hip_fail(r, "mbswap hand-over");
        if ((st = mb_swap_in(m, (x + 2) % m->n, s)))
            return st;
    }
    m->round += 1;
    const hipError_t r = hipStreamWaitEvent(compute, m->loaded[m->round & 1], 0);
    return r == hipSuccess ? KV_OK : hip_fail(r, "mbswap next wait");
}

int kv_swap_pays(int64_t N, double t, int64_t p, int64_t B, double C, double bw, double *lhs,
                 double *rhs)
{
    if (!lhs || !rhs)
        return set_error(KV_EINVAL, "NULL output");
    if (N < 0 || p < 0 || B < 1 || !(t >= 0) || !(C >= 0) || !(bw > 0))
        return set_error(KV_EINVAL, "bad argument (N=%lld p=%lld B=%lld t=%g C=%g bw=%g)",
                         (long long)N, (long long)p, (long long)B, t, C, bw);
    double sum = 0;
    for (int64_t i = p; i <= N + p; ++i)
        sum += std::max(t, (double)i * (double)B * C / bw);
    *lhs = 2.0 * (double)N * t;
    *rhs = sum;
    return *lhs >= *rhs ? 1 : 0;
}

}  // extern "C"
