// Device-to-host copies on one chosen DMA engine, ordered with HIP streams.
//
// "DejaVu: KV-Cache Streaming ...", Method details, Token computation and
// streaming parallelization (Fig 7c): the copy of a filled buffer to the host
// runs beside the next step's compute.  The default transport moves that leg
// with the library's link-copy kernel; its host stores cost co-running HBM
// kernels about a third of their speed, where a DMA engine's do not.  HIP
// lets the runtime pick the engine of a hipMemcpyAsync, and on MI355X only
// engines 0-3 write host memory at full speed (4-15 reach 7-12 GB/s).  This
// copier names the engine through the HSA runtime instead.
//
// Ordering.  At the call, the copy is submitted to the engine with one
// dependency, a signal `gate` that reads 1; on the stream follow an event
// `ready` (its default system-scope release writes the bank back from every
// L2), a write of 0 to `gate` (the engine starts the copy once the stream
// gets there), a wait until the copy's completion signal reads 0, and an
// event `reused` that says the stream is past that wait.  Copies reach the
// engine in the order they are enqueued, and everything a copy waits for was
// enqueued before it, so a copy that sits ahead of another on an engine --
// ours or the runtime's -- never waits for that other one.
#include "kvs_internal.h"

#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include <atomic>
#include <chrono>
#include <cstring>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

namespace kvs {

namespace {

struct HsaAgents {
    bool ok = false;
    int device = -1;
    hsa_agent_t cpu{}, gpu{};
    char why[160] = "";
};

struct FindArgs {
    uint32_t bdf;
    uint32_t domain;
    HsaAgents *a;
    bool cpu_found, gpu_found;
};

hsa_status_t visit_agent(hsa_agent_t agent, void *data)
{
    auto *f = (FindArgs *)data;
    hsa_device_type_t type;
    if (hsa_agent_get_info(agent, HSA_AGENT_INFO_DEVICE, &type) != HSA_STATUS_SUCCESS)
        return HSA_STATUS_SUCCESS;
    if (type == HSA_DEVICE_TYPE_CPU && !f->cpu_found) {
        f->a->cpu = agent;
        f->cpu_found = true;
    } else if (type == HSA_DEVICE_TYPE_GPU && !f->gpu_found) {
        uint32_t bdf = 0, domain = 0;
        if (hsa_agent_get_info(agent, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_BDFID, &bdf) ==
                HSA_STATUS_SUCCESS &&
            hsa_agent_get_info(agent, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_DOMAIN, &domain) ==
                HSA_STATUS_SUCCESS &&
            bdf == f->bdf && domain == f->domain) {
            f->a->gpu = agent;
            f->gpu_found = true;
        }
    }
    return HSA_STATUS_SUCCESS;
}

// The CPU agent and the GPU agent of the current HIP device (HSA is already
// running under HIP; hsa_init only takes a reference).
int agents_for_current_device(HsaAgents *out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    static std::mutex mu;
    static std::vector<HsaAgents> cache;
    std::lock_guard<std::mutex> g(mu);
    for (const HsaAgents &a : cache)
        if (a.device == dev) {
            *out = a;
            return a.ok ? KV_OK : set_error(KV_EINVAL, "%s", a.why);
        }
    HsaAgents a;
    a.device = dev;
    int bus = 0, slot = 0, domain = 0, can_wait = 0;
    if ((e = hipDeviceGetAttribute(&bus, hipDeviceAttributePciBusId, dev)) != hipSuccess ||
        (e = hipDeviceGetAttribute(&slot, hipDeviceAttributePciDeviceId, dev)) != hipSuccess ||
        (e = hipDeviceGetAttribute(&domain, hipDeviceAttributePciDomainId, dev)) != hipSuccess ||
        (e = hipDeviceGetAttribute(&can_wait, hipDeviceAttributeCanUseStreamWaitValue, dev)) !=
            hipSuccess)
        return hip_fail(e, "hipDeviceGetAttribute");
    if (!can_wait) {
        std::snprintf(a.why, sizeof a.why, "device %d cannot wait on memory values in a stream",
                      dev);
    } else if (hsa_init() != HSA_STATUS_SUCCESS) {
        std::snprintf(a.why, sizeof a.why, "the HSA runtime did not initialise");
    } else {
        FindArgs f{(uint32_t)((bus << 8) | (slot << 3)), (uint32_t)domain, &a, false, false};
        hsa_iterate_agents(visit_agent, &f);
        if (!f.cpu_found || !f.gpu_found)
            std::snprintf(a.why, sizeof a.why, "no HSA %s agent for device %d",
                          f.gpu_found ? "CPU" : "GPU", dev);
        else
            a.ok = true;
    }
    cache.push_back(a);
    *out = a;
    return a.ok ? KV_OK : set_error(KV_EINVAL, "%s", a.why);
}

std::atomic<uint32_t> g_next_engine{0};

struct Slot {
    hipEvent_t ready = nullptr;        // release point before the copy starts
    hipEvent_t reused = nullptr;       // the stream is past its wait for the copy
    hsa_signal_t gate{};               // 1 until the stream reaches the copy
    hsa_signal_t done{};               // 1 until the engine finishes the copy
    volatile hsa_signal_value_t *gate_value = nullptr;
    volatile hsa_signal_value_t *done_value = nullptr;
    bool recorded = false;             // `reused` has been recorded at least once
    bool retired = false;              // a failed call left the signals in use
};

}  // namespace

struct EngineCopier {
    HsaAgents agents;
    uint32_t engine = 0;
    bool pinned = false;           // always `engine`, never another idle one
    std::vector<Slot *> slots;
};

// Engines whose host writes run at full speed on MI355X.  (Splitting a copy
// over two of them was measured and dropped: it slowed the steps by 2-10%.)
constexpr uint32_t kFastEngines[] = {HSA_AMD_SDMA_ENGINE_0, HSA_AMD_SDMA_ENGINE_1,
                                     HSA_AMD_SDMA_ENGINE_2, HSA_AMD_SDMA_ENGINE_3};

int engine_copier_create(EngineCopier **out)
{
    *out = nullptr;
    if (serialized_dispatch())
        return set_error(KV_EINVAL,
                         "KV_XFER_ENGINE needs concurrent dispatch: with AMD_SERIALIZE_KERNEL or "
                         "counter collection (ROCPROF_COUNTER_COLLECTION) its stream waits on a "
                         "DMA copy never finish; use another transport");
    HsaAgents a;
    int st = agents_for_current_device(&a);
    if (st)
        return st;
    auto *c = new (std::nothrow) EngineCopier();
    if (!c)
        return set_error(KV_EINVAL, "out of host memory for the copier");
    c->agents = a;
    // spread copiers over the fast engines, preferring one the runtime reports free
    uint32_t mask = 0;
    if (hsa_amd_memory_copy_engine_status(a.cpu, a.gpu, &mask) != HSA_STATUS_SUCCESS)
        mask = 0;
    const uint32_t first = g_next_engine.fetch_add(1);
    for (uint32_t i = 0; i < 4 && !c->engine; ++i) {
        const uint32_t e = kFastEngines[(first + i) % 4];
        if (mask & e)
            c->engine = e;
    }
    if (!c->engine)   // the status is a snapshot of busy engines: use the next one anyway
        c->engine = kFastEngines[first % 4];
    *out = c;
    return KV_OK;
}

void engine_copier_pin(EngineCopier *c, int32_t engine)
{
    if (!c)
        return;
    c->pinned = engine >= 0 && engine < 4;
    if (c->pinned)
        c->engine = kFastEngines[engine];
}

int engine_copier_destroy(EngineCopier *c)
{
    if (!c)
        return KV_OK;
    int abandoned = 0;
    // the signals must outlive every copy and every stream wait on them
    bool retired = false;
    for (Slot *s : c->slots)
        retired |= s->retired;
    if (retired)
        (void)hipDeviceSynchronize();
    for (Slot *s : c->slots) {
        if (s->recorded)
            (void)hipEventSynchronize(s->reused);
        // a released copy still running: give it up to ten seconds, then
        // leave its signals alive rather than free them under the engine
        const auto t0 = std::chrono::steady_clock::now();
        bool busy = false;
        while (hsa_signal_load_scacquire(s->done) > 0 && hsa_signal_load_scacquire(s->gate) == 0) {
            if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(10)) {
                busy = true;
                break;
            }
            std::this_thread::yield();
        }
        if (busy) {
            ++abandoned;
            continue;
        }
        (void)hipEventDestroy(s->ready);
        (void)hipEventDestroy(s->reused);
        hsa_signal_destroy(s->gate);
        hsa_signal_destroy(s->done);
        delete s;
    }
    delete c;
    if (abandoned)
        return set_error(KV_EHIP,
                         "%d DMA copies were still running ten seconds into destroy; their "
                         "signals are left allocated", abandoned);
    return KV_OK;
}

namespace {

int gpu_signal(hsa_signal_t *sig, volatile hsa_signal_value_t **value)
{
    if (hsa_amd_signal_create(1, 0, nullptr, HSA_AMD_SIGNAL_AMD_GPU_ONLY, sig) !=
        HSA_STATUS_SUCCESS)
        return set_error(KV_EHIP, "could not create an HSA signal for a DMA copy");
    if (hsa_amd_signal_value_pointer(*sig, value) != HSA_STATUS_SUCCESS) {
        hsa_signal_destroy(*sig);
        return set_error(KV_EHIP, "no value address for an HSA signal");
    }
    return KV_OK;
}

int take_slot(EngineCopier *c, Slot **out)
{
    for (Slot *s : c->slots) {
        if (s->retired)
            continue;
        if (s->recorded) {
            const hipError_t q = hipEventQuery(s->reused);
            if (q == hipErrorNotReady)
                continue;
            if (q != hipSuccess)
                return hip_fail(q, "hipEventQuery");
        }
        *out = s;
        return KV_OK;
    }
    auto *s = new (std::nothrow) Slot();
    if (!s)
        return set_error(KV_EINVAL, "out of host memory for a copy slot");
    hipError_t e = hipEventCreateWithFlags(&s->ready, hipEventDisableTiming);
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&s->reused, hipEventDisableTiming);
    if (e != hipSuccess) {
        if (s->ready)
            (void)hipEventDestroy(s->ready);
        delete s;
        return hip_fail(e, "hipEventCreateWithFlags");
    }
    int st = gpu_signal(&s->gate, &s->gate_value);
    if (st == KV_OK && (st = gpu_signal(&s->done, &s->done_value)) != KV_OK)
        hsa_signal_destroy(s->gate);
    if (st != KV_OK) {
        (void)hipEventDestroy(s->ready);
        (void)hipEventDestroy(s->reused);
        delete s;
        return st;
    }
    c->slots.push_back(s);
    *out = s;
    return KV_OK;
}

}  // namespace

int engine_copy_to_host(EngineCopier *c, void *dst_host, const void *src_dev, int64_t bytes,
                        hipStream_t s)
{
    if (bytes <= 0)
        return KV_OK;
    Slot *slot = nullptr;
    int st = take_slot(c, &slot);
    if (st)
        return st;
    hsa_signal_store_relaxed(slot->gate, 1);
    hsa_signal_store_relaxed(slot->done, 1);
    hipError_t e = hipEventRecord(slot->ready, s);
    if (e != hipSuccess)
        return hip_fail(e, "hipEventRecord");
    // an engine with nothing queued, if one of the four is: a copy queued
    // behind others (the runtime's host->device copies, gated on their own
    // banks) would wait for all of them.  Consecutive copies of a stream may
    // use different engines: each starts only after the stream is past the
    // one before.
    uint32_t idle = 0;
    if (hsa_amd_memory_copy_engine_status(c->agents.cpu, c->agents.gpu, &idle) !=
        HSA_STATUS_SUCCESS)
        idle = 0;
    if (!c->pinned && !(idle & c->engine))
        for (uint32_t e : kFastEngines)
            if (idle & e) {
                c->engine = e;
                break;
            }
    if (hsa_amd_memory_async_copy_on_engine(dst_host, c->agents.cpu, src_dev, c->agents.gpu,
                                            (size_t)bytes, 1, &slot->gate, slot->done,
                                            (hsa_amd_sdma_engine_id_t)c->engine, false) !=
        HSA_STATUS_SUCCESS)
        return set_error(KV_EHIP, "DMA engine %#x refused a copy of %lld bytes", c->engine,
                         (long long)bytes);
    // from here the engine holds the copy: every failure path must release it
    e = hipStreamWriteValue64(s, (void *)slot->gate_value, 0, 0);
    if (e != hipSuccess) {
        hsa_signal_store_screlease(slot->gate, 0);   // let the engine move on
        slot->retired = true;
        return hip_fail(e, "hipStreamWriteValue64");
    }
    e = hipStreamWaitValue64(s, (void *)slot->done_value, 0, hipStreamWaitValueEq, ~0ull);
    if (e == hipSuccess)
        e = hipEventRecord(slot->reused, s);
    if (e != hipSuccess) {
        slot->retired = true;
        return hip_fail(e, "hipStreamWaitValue64");
    }
    slot->recorded = true;
    return KV_OK;
}

}  // namespace kvs
