// Staged transfers between the cache and pinned host memory: the swap engine
// (microbatch swap-out/in and the layer-by-layer prompt streamer) and the
// decode-step staging ring with its flush policy and restore.
//
// "DejaVu: KV-Cache Streaming ...", Method details: Buffered copies (Fig 7a:
// fill a reusable device buffer, copy it out once filled), Layer-by-layer
// prompt cache streaming (Fig 7b), Token computation and streaming
// parallelization (Fig 7c: streaming overlaps the next step's compute on a
// separate stream), Microbatch swapping workflow (Fig 9), Failure detection
// and recovery (Fig 10: the replica is copied back to a fresh worker).
//
// Ordering is carried entirely by hipEvents between the caller's compute
// stream and the engine's copy stream; no call waits on the host.  Each of
// the two banks has a "free" event (after it, the bank may be overwritten)
// and a "filled" event (after it, the bank holds the data the other stream
// needs).
#include "kvs_internal.h"
#include "chunks.h"

#include <algorithm>
#include <cstring>
#include <deque>
#include <new>
#include <utility>
#include <vector>

using namespace kvs;

namespace {

// Chunking of one swap into a vector (see for_each_chunk).
int plan_chunks(const kv_layout &lay, int32_t l0, int32_t nl, const RowTable &rt,
                int64_t bank_bytes, std::vector<Chunk> *out)
{
    out->clear();
    return for_each_chunk(lay, l0, nl, rt, bank_bytes, [out](const Chunk &c) {
        out->push_back(c);
        return KV_OK;
    });
}

int check_banks_apart(void *const bank[2], int64_t bank_bytes, const kv_layout &lay,
                      const void *k, const void *v)
{
    for (int b = 0; b < 2; ++b)
        if (overlaps(bank[b], bank_bytes, k, lay.k_bytes) || overlaps(bank[b], bank_bytes, v, lay.v_bytes))
            return set_error(KV_EINVAL, "bank%d overlaps a cache", b);
    return KV_OK;
}

int record(hipEvent_t e, hipStream_t s, const char *what)
{
    const hipError_t r = hipEventRecord(e, s);
    return r == hipSuccess ? KV_OK : hip_fail(r, what);
}

int wait(hipStream_t s, hipEvent_t e, const char *what)
{
    const hipError_t r = hipStreamWaitEvent(s, e, 0);
    return r == hipSuccess ? KV_OK : hip_fail(r, what);
}

int create_events(hipEvent_t *ev, int n)
{
    for (int i = 0; i < n; ++i) {
        const hipError_t r = hipEventCreateWithFlags(&ev[i], hipEventDisableTiming);
        if (r != hipSuccess) {
            for (int j = 0; j < i; ++j)
                (void)hipEventDestroy(ev[j]);
            return hip_fail(r, "hipEventCreateWithFlags");
        }
    }
    return KV_OK;
}

// One contiguous transfer between a bank and pinned host memory on `s`, with
// the engine's transport.  `host_dev` is the device-visible address of the
// host side (used by the link-copy kernel).
int transfer(int32_t transport, EngineCopier *copier, int32_t link_blocks, void *bank, void *host,
             void *host_dev, int64_t bytes, bool to_host, hipStream_t s)
{
    if (bytes <= 0)
        return KV_OK;
    if (transport == KV_XFER_ENGINE && to_host)
        return engine_copy_to_host(copier, host, bank, bytes, s);
    const bool kernel = transport == KV_XFER_KERNEL || (transport == KV_XFER_AUTO && to_host);
    if (kernel)
        return to_host ? launch_link_copy(host_dev, bank, bytes, true, s, link_blocks)
                       : launch_link_copy(bank, host_dev, bytes, false, s);
    hipError_t r;
    if (transport == KV_XFER_DMA || (transport == KV_XFER_DMA_OUT && to_host))
        r = to_host ? hipMemcpyAsync(host_dev, bank, (size_t)bytes, hipMemcpyDeviceToDeviceNoCU, s)
                    : hipMemcpyAsync(bank, host_dev, (size_t)bytes, hipMemcpyDeviceToDeviceNoCU, s);
    else
        r = to_host ? hipMemcpyAsync(host, bank, (size_t)bytes, hipMemcpyDeviceToHost, s)
                    : hipMemcpyAsync(bank, host, (size_t)bytes, hipMemcpyHostToDevice, s);
    return r == hipSuccess ? KV_OK : hip_fail(r, "hipMemcpyAsync");
}

int check_transport(int32_t transport)
{
    if (transport < KV_XFER_AUTO || transport > KV_XFER_ENGINE)
        return set_error(KV_EINVAL, "transport %d is not a kv_transport", transport);
    if (transport == KV_XFER_ENGINE && serialized_dispatch())
        return set_error(KV_EINVAL,
                         "KV_XFER_ENGINE needs concurrent dispatch: with AMD_SERIALIZE_KERNEL or "
                         "counter collection (ROCPROF_COUNTER_COLLECTION) its stream waits on a "
                         "DMA copy never finish; use another transport");
    return KV_OK;
}

}  // namespace

struct kv_swap {
    kv_layout lay;
    void *bank[2];
    int64_t bank_bytes;
    hipStream_t copy;
    int32_t transport;
    EngineCopier *copier;        // KV_XFER_ENGINE: the device->host DMA engine
    int32_t link_blocks;         // link-copy kernel workgroups, device->host (0: default)
    hipEvent_t ev[4];            // free0, free1, filled0, filled1
    bool free_valid[2];
    int next;
    hipEvent_t free_ev(int b) const { return ev[b]; }
    hipEvent_t filled_ev(int b) const { return ev[2 + b]; }
};

struct kv_ring {
    kv_layout lay;
    int32_t R;
    void *bank[2];
    int64_t bank_bytes;
    void *host;
    int64_t host_bytes;
    void *host_dev;              // device-visible address of `host`
    hipStream_t copy;
    int32_t transport;
    EngineCopier *copier;        // KV_XFER_ENGINE: the device->host DMA engine
    int32_t link_blocks;         // link-copy kernel workgroups, device->host (0: default)
    int64_t slot_bytes;
    int64_t steps, flushed;
    std::vector<int32_t> pos;    // steps * B positions, in step order
    hipEvent_t ev[5];            // free0, free1, filled0, filled1, sync
    // compute streams of the packs (gather per step) into the bank of the
    // unflushed steps: the copy stream orders itself after each of them
    // before it reads (flush) or overwrites (restore) that bank
    std::vector<hipStream_t> pack_streams;
    bool wait_needed[2];         // a push must wait on free_ev before writing the bank
    bool free_valid[2];          // free_ev has been recorded at least once
    // flush copies not yet known complete: (event after the copy, steps held once it lands)
    std::deque<std::pair<hipEvent_t, int64_t>> landing;
    std::vector<hipEvent_t> spare;   // recycled landing events
    int64_t durable;             // steps known to be in the host image
    int32_t gather;              // KV_RING_GATHER_EACH_STEP or KV_RING_GATHER_AT_FLUSH
    // caches of the steps [flushed, steps) not yet gathered (gather at flush)
    std::vector<std::pair<const void *, const void *>> pend;
    hipEvent_t free_ev(int b) const { return ev[b]; }
    hipEvent_t filled_ev(int b) const { return ev[2 + b]; }
    hipEvent_t sync_ev() const { return ev[4]; }
};

namespace {

int swap_out_rows(kv_swap *e, const void *k, const void *v, int32_t l0, int32_t nl,
                  const RowTable &rt, void *host, int64_t host_bytes, hipStream_t compute,
                  hipEvent_t done)
{
    const kv_layout &lay = e->lay;
    const int64_t need = packed_bytes(lay, nl, rt.off[lay.B]);
    int st;
    if (host_bytes < need)
        return set_error(KV_ESIZE, "host holds %lld bytes, %lld needed", (long long)host_bytes,
                         (long long)need);
    if ((st = check_pinned_host(host, need, "host")))
        return st;
    void *host_dev = nullptr;
    if (need > 0 && (st = host_device_address(host, need, &host_dev)))
        return st;
    if ((st = check_device_buffer(k, lay.k_bytes, "key cache")))
        return st;
    if ((st = check_device_buffer(v, lay.v_bytes, "value cache")))
        return st;
    if ((st = check_banks_apart(e->bank, e->bank_bytes, lay, k, v)))
        return st;
    std::vector<Chunk> chunks;
    if ((st = plan_chunks(lay, l0, nl, rt, e->bank_bytes, &chunks)))
        return st;
    for (const Chunk &c : chunks) {
        const int bk = e->next;
        e->next ^= 1;
        if (e->free_valid[bk] && (st = wait(compute, e->free_ev(bk), "swap-out bank wait")))
            return st;
        RowTable sub;
        int32_t mx;
        chunk_rows(lay, rt, c, &sub, &mx);
        if ((st = enqueue_copy(true, lay, k, v, c.l0, c.nl, sub, mx, e->bank[bk], compute)))
            return st;
        if ((st = record(e->filled_ev(bk), compute, "swap-out packed")) ||
            (st = wait(e->copy, e->filled_ev(bk), "swap-out copy wait")))
            return st;
        for (int p = 0; p < c.pieces; ++p)
            if ((st = transfer(e->transport, e->copier, e->link_blocks, (char *)e->bank[bk] + c.bank_off[p],
                               (char *)host + c.host_off[p], (char *)host_dev + c.host_off[p],
                               c.bytes[p], true, e->copy)))
                return st;
        if ((st = record(e->free_ev(bk), e->copy, "swap-out copied")))
            return st;
        e->free_valid[bk] = true;
    }
    if (done && (st = record(done, e->copy, "swap-out done")))
        return st;
    return KV_OK;
}

}  // namespace

extern "C" {

int kv_swap_create(kv_swap **out, const kv_layout *lay, void *bank0, void *bank1,
                   int64_t bank_bytes, hipStream_t copy, int32_t transport)
{
    if (out == nullptr)
        return set_error(KV_EINVAL, "output handle pointer is NULL");
    *out = nullptr;
    int st = check_layout(lay);
    if (st)
        return st;
    if ((st = check_transport(transport)))
        return st;
    if (bank_bytes <= 0)
        return set_error(KV_ESIZE, "bank_bytes %lld must be positive", (long long)bank_bytes);
    if ((st = check_device_buffer(bank0, bank_bytes, "bank0")) ||
        (st = check_device_buffer(bank1, bank_bytes, "bank1")))
        return st;
    if (overlaps(bank0, bank_bytes, bank1, bank_bytes))
        return set_error(KV_EINVAL, "the two banks overlap");
    kv_swap *e = new (std::nothrow) kv_swap();
    if (!e)
        return set_error(KV_EINVAL, "out of host memory for the handle");
    e->lay = *lay;
    e->bank[0] = bank0;
    e->bank[1] = bank1;
    e->bank_bytes = bank_bytes;
    e->copy = copy;
    e->transport = transport;
    e->free_valid[0] = e->free_valid[1] = false;
    e->next = 0;
    e->copier = nullptr;
    e->link_blocks = 0;
    if ((st = create_events(e->ev, 4))) {
        delete e;
        return st;
    }
    if (transport == KV_XFER_ENGINE && (st = engine_copier_create(&e->copier))) {
        for (hipEvent_t ev : e->ev)
            (void)hipEventDestroy(ev);
        delete e;
        return st;
    }
    *out = e;
    return KV_OK;
}

int kv_swap_destroy(kv_swap *e)
{
    if (!e)
        return KV_OK;
    const int st = engine_copier_destroy(e->copier);
    for (hipEvent_t ev : e->ev)
        (void)hipEventDestroy(ev);
    delete e;
    return st;
}

int kv_swap_out(kv_swap *e, const void *k, const void *v, int32_t layer_begin,
                int32_t layer_count, const int32_t *start, const int32_t *count, void *host,
                int64_t host_bytes, hipStream_t compute, hipEvent_t done)
{
    if (!e)
        return set_error(KV_EINVAL, "swap handle is NULL");
    int st;
    if ((st = check_layers(e->lay, layer_begin, layer_count)))
        return st;
    RowTable rt;
    int32_t mx;
    if ((st = build_rows(e->lay, start, count, &rt, &mx)))
        return st;
    return swap_out_rows(e, k, v, layer_begin, layer_count, rt, host, host_bytes, compute, done);
}

int kv_stream_prompt_layer(kv_swap *e, const void *k, const void *v, int32_t layer,
                           int32_t tok_begin, int32_t tok_count, const int32_t *row_len,
                           void *host, int64_t host_bytes, hipStream_t compute, hipEvent_t done)
{
    if (!e)
        return set_error(KV_EINVAL, "swap handle is NULL");
    const kv_layout &lay = e->lay;
    int st;
    if ((st = check_layers(lay, layer, 1)))
        return st;
    int32_t start[KV_MAX_ROWS], count[KV_MAX_ROWS];
    if ((st = prompt_rows(lay, tok_begin, tok_count, row_len, start, count)))
        return st;
    RowTable rt;
    int32_t mx;
    if ((st = build_rows(lay, start, count, &rt, &mx)))
        return st;
    return swap_out_rows(e, k, v, layer, 1, rt, host, host_bytes, compute, done);
}

int kv_swap_in(kv_swap *e, void *k, void *v, int32_t layer_begin, int32_t layer_count,
               const int32_t *start, const int32_t *count, const void *host, int64_t host_bytes,
               hipStream_t compute, hipEvent_t done)
{
    if (!e)
        return set_error(KV_EINVAL, "swap handle is NULL");
    const kv_layout &lay = e->lay;
    int st;
    if ((st = check_layers(lay, layer_begin, layer_count)))
        return st;
    RowTable rt;
    int32_t mx;
    if ((st = build_rows(lay, start, count, &rt, &mx)))
        return st;
    const int64_t need = packed_bytes(lay, layer_count, rt.off[lay.B]);
    if (host_bytes < need)
        return set_error(KV_ESIZE, "host holds %lld bytes, %lld needed", (long long)host_bytes,
                         (long long)need);
    if ((st = check_pinned_host(host, need, "host")))
        return st;
    void *host_dev = nullptr;
    if (need > 0 && (st = host_device_address(host, need, &host_dev)))
        return st;
    if ((st = check_device_buffer(k, lay.k_bytes, "key cache")) ||
        (st = check_device_buffer(v, lay.v_bytes, "value cache")))
        return st;
    if ((st = check_banks_apart(e->bank, e->bank_bytes, lay, k, v)))
        return st;
    std::vector<Chunk> chunks;
    if ((st = plan_chunks(lay, layer_begin, layer_count, rt, e->bank_bytes, &chunks)))
        return st;
    for (const Chunk &c : chunks) {
        const int bk = e->next;
        e->next ^= 1;
        if (e->free_valid[bk] && (st = wait(e->copy, e->free_ev(bk), "swap-in bank wait")))
            return st;
        for (int p = 0; p < c.pieces; ++p)
            if ((st = transfer(e->transport, e->copier, e->link_blocks, (char *)e->bank[bk] + c.bank_off[p],
                               (char *)host + c.host_off[p], (char *)host_dev + c.host_off[p],
                               c.bytes[p], false, e->copy)))
                return st;
        if ((st = record(e->filled_ev(bk), e->copy, "swap-in loaded")) ||
            (st = wait(compute, e->filled_ev(bk), "swap-in unpack wait")))
            return st;
        RowTable sub;
        int32_t cmx;
        chunk_rows(lay, rt, c, &sub, &cmx);
        if ((st = enqueue_copy(false, lay, k, v, c.l0, c.nl, sub, cmx, e->bank[bk], compute)))
            return st;
        if ((st = record(e->free_ev(bk), compute, "swap-in unpacked")))
            return st;
        e->free_valid[bk] = true;
    }
    if (done && (st = record(done, compute, "swap-in done")))
        return st;
    return KV_OK;
}

int64_t kv_swap_plan(const kv_layout *lay, int32_t layer_begin, int32_t layer_count,
                     const int32_t *start, const int32_t *count, int64_t bank_bytes,
                     kv_chunk *out, int64_t max_chunks)
{
    int st = check_layout(lay);
    if (st)
        return st;
    if ((st = check_layers(*lay, layer_begin, layer_count)))
        return st;
    if (bank_bytes <= 0)
        return set_error(KV_ESIZE, "bank_bytes must be positive");
    RowTable rt;
    int32_t mx;
    if ((st = build_rows(*lay, start, count, &rt, &mx)))
        return st;
    std::vector<Chunk> chunks;
    if ((st = plan_chunks(*lay, layer_begin, layer_count, rt, bank_bytes, &chunks)))
        return st;
    for (int64_t i = 0; out && i < max_chunks && i < (int64_t)chunks.size(); ++i) {
        const Chunk &c = chunks[i];
        kv_chunk &o = out[i];
        std::memset(&o, 0, sizeof o);
        o.layer_begin = c.l0;
        o.layer_count = c.nl;
        o.row_begin = c.b0;
        o.row_end = c.b1;
        o.staged_bytes = c.staged;
        o.pieces = c.pieces;
        for (int p = 0; p < 2; ++p) {
            o.host_off[p] = c.host_off[p];
            o.bank_off[p] = c.bank_off[p];
            o.bytes[p] = c.bytes[p];
        }
    }
    return (int64_t)chunks.size();
}

// ---------------------------------------------------------------------------
// staging ring

int kv_ring_create(kv_ring **out, const kv_layout *lay, int32_t R, void *bank0, void *bank1,
                   int64_t bank_bytes, void *host, int64_t host_bytes, hipStream_t copy,
                   int32_t transport)
{
    if (out == nullptr)
        return set_error(KV_EINVAL, "output handle pointer is NULL");
    *out = nullptr;
    int st = check_layout(lay);
    if (st)
        return st;
    if ((st = check_transport(transport)))
        return st;
    if (R <= 0)
        return set_error(KV_EINVAL, "R=%d must be positive", R);
    const int64_t slot = packed_bytes(*lay, lay->L, lay->B);
    if (bank_bytes < (int64_t)R * slot)
        return set_error(KV_ESIZE, "banks hold %lld bytes; %d slots need %lld",
                         (long long)bank_bytes, R, (long long)R * slot);
    if (host_bytes < 0)
        return set_error(KV_ESIZE, "host_bytes is negative");
    if ((st = check_device_buffer(bank0, (int64_t)R * slot, "bank0")) ||
        (st = check_device_buffer(bank1, (int64_t)R * slot, "bank1")))
        return st;
    if (overlaps(bank0, (int64_t)R * slot, bank1, (int64_t)R * slot))
        return set_error(KV_EINVAL, "the two banks overlap");
    if ((st = check_pinned_host(host, host_bytes, "host")))
        return st;
    void *host_dev = nullptr;
    if (host_bytes > 0 && (st = host_device_address(host, host_bytes, &host_dev)))
        return st;
    kv_ring *r = new (std::nothrow) kv_ring();
    if (!r)
        return set_error(KV_EINVAL, "out of host memory for the handle");
    r->lay = *lay;
    r->R = R;
    r->bank[0] = bank0;
    r->bank[1] = bank1;
    r->bank_bytes = bank_bytes;
    r->host = host;
    r->host_bytes = host_bytes;
    r->host_dev = host_dev;
    r->copy = copy;
    r->transport = transport;
    r->slot_bytes = slot;
    r->steps = r->flushed = 0;
    r->durable = 0;
    r->gather = KV_RING_GATHER_EACH_STEP;
    r->wait_needed[0] = r->wait_needed[1] = false;
    r->free_valid[0] = r->free_valid[1] = false;
    r->copier = nullptr;
    r->link_blocks = 0;
    if ((st = create_events(r->ev, 5))) {
        delete r;
        return st;
    }
    if (transport == KV_XFER_ENGINE && (st = engine_copier_create(&r->copier))) {
        for (hipEvent_t ev : r->ev)
            (void)hipEventDestroy(ev);
        delete r;
        return st;
    }
    *out = r;
    return KV_OK;
}

int kv_ring_destroy(kv_ring *r)
{
    if (!r)
        return KV_OK;
    const int st = engine_copier_destroy(r->copier);
    for (hipEvent_t ev : r->ev)
        (void)hipEventDestroy(ev);
    for (auto &p : r->landing)
        (void)hipEventDestroy(p.first);
    for (hipEvent_t ev : r->spare)
        (void)hipEventDestroy(ev);
    delete r;
    return st;
}

namespace {

// Step j's positions are step j-1's plus one on every row.
bool follows(const kv_ring *r, int64_t j)
{
    const int32_t B = r->lay.B;
    const int32_t *p = &r->pos[(size_t)j * B];
    for (int32_t b = 0; b < B; ++b)
        if (p[b] != p[b - B] + 1)
            return false;
    return true;
}

// Pack (or unpack) steps [j0, j0+n) between caches and their slots at
// `slots` (step j0's slot first), one pass per run of steps whose positions
// advance by one per row, else one pack per step.  The caches are (k, v) for
// every step, or caches[i] for step j0+i when `caches` is given (a run then
// also needs the same caches).
int ring_copy_steps(kv_ring *r, bool pack, const void *k, const void *v, int64_t j0, int64_t n,
                    void *slots, hipStream_t compute,
                    const std::pair<const void *, const void *> *caches)
{
    const kv_layout &lay = r->lay;
    int st;
    for (int64_t a = 0; a < n;) {
        int64_t e = a + 1;
        while (e < n && (!caches || caches[e] == caches[a]) && follows(r, j0 + e))
            ++e;
        const void *ka = caches ? caches[a].first : k;
        const void *va = caches ? caches[a].second : v;
        void *slot = (char *)slots + a * r->slot_bytes;
        const int32_t *p = &r->pos[(size_t)(j0 + a) * lay.B];
        if (e - a >= 2) {
            if ((st = enqueue_steps(pack, lay, ka, va, p, (int32_t)(e - a), slot, r->slot_bytes,
                                    compute)))
                return st;
        } else {
            RowTable rt;
            int32_t mx;
            if ((st = build_rows(lay, p, nullptr, &rt, &mx)) ||
                (st = enqueue_copy(pack, lay, ka, va, 0, lay.L, rt, mx, slot, compute)))
                return st;
        }
        a = e;
    }
    return KV_OK;
}

// Gather the steps pushed since the last flush (gather-at-flush mode).
int ring_gather(kv_ring *r, hipStream_t compute)
{
    if (r->pend.empty())
        return KV_OK;
    const int64_t j0 = r->flushed;
    const int bk = (int)((j0 / r->R) & 1);
    int st;
    if (r->wait_needed[bk]) {
        if ((st = wait(compute, r->free_ev(bk), "ring bank wait")))
            return st;
        r->wait_needed[bk] = false;
    }
    st = ring_copy_steps(r, true, nullptr, nullptr, j0, (int64_t)r->pend.size(),
                         (char *)r->bank[bk] + (j0 % r->R) * r->slot_bytes, compute,
                         r->pend.data());
    r->pend.clear();
    return st;
}

// Make the copy stream wait for every pack of an unflushed step, except
// those on `covered` when `skip` (the stream whose own event the copy waits on
// anyway).  One event serves them all: a stream wait takes the event's state
// at the time of the wait.
int ring_order_packs(kv_ring *r, bool skip, hipStream_t covered)
{
    int st;
    for (hipStream_t s : r->pack_streams)
        if (!(skip && s == covered) &&
            ((st = record(r->sync_ev(), s, "ring pack order")) ||
             (st = wait(r->copy, r->sync_ev(), "ring pack order wait"))))
            return st;
    return KV_OK;
}

// Copy steps [first, first+n) -- all in one bank -- to the host image.
int ring_flush_range(kv_ring *r, int64_t first, int64_t n, hipStream_t compute)
{
    const int bk = (int)((first / r->R) & 1);
    const int64_t off = (first % r->R) * r->slot_bytes;
    int st;
    if ((st = record(r->filled_ev(bk), compute, "ring filled")) ||
        (st = wait(r->copy, r->filled_ev(bk), "ring flush wait")) ||
        (st = ring_order_packs(r, true, compute)))
        return st;
    r->pack_streams.clear();
    if ((st = transfer(r->transport, r->copier, r->link_blocks, (char *)r->bank[bk] + off,
                       (char *)r->host + first * r->slot_bytes,
                       (char *)r->host_dev + first * r->slot_bytes, n * r->slot_bytes, true,
                       r->copy)))
        return st;
    if ((st = record(r->free_ev(bk), r->copy, "ring flushed")))
        return st;
    r->wait_needed[bk] = true;
    r->free_valid[bk] = true;
    r->flushed = first + n;
    hipEvent_t landed = nullptr;
    if (!r->spare.empty()) {
        landed = r->spare.back();
        r->spare.pop_back();
    } else if ((st = create_events(&landed, 1))) {
        return st;
    }
    if ((st = record(landed, r->copy, "ring landed"))) {
        r->spare.push_back(landed);
        return st;
    }
    r->landing.emplace_back(landed, r->flushed);
    return KV_OK;
}

}  // namespace

int kv_ring_push(kv_ring *r, const void *k, const void *v, const int32_t *pos,
                 hipStream_t compute)
{
    if (!r)
        return set_error(KV_EINVAL, "ring handle is NULL");
    const kv_layout &lay = r->lay;
    if (pos == nullptr)
        return set_error(KV_EINVAL, "pos is NULL");
    for (int32_t b = 0; b < lay.B; ++b)
        if (pos[b] < 0 || pos[b] >= lay.Smax)
            return set_error(KV_ERANGE, "row %d: position %d outside [0, %d)", b, pos[b],
                             lay.Smax);
    if ((r->steps + 1) * r->slot_bytes > r->host_bytes)
        return set_error(KV_ESIZE, "host image full after %lld steps", (long long)r->steps);
    int st;
    if ((st = check_device_buffer(k, lay.k_bytes, "key cache")) ||
        (st = check_device_buffer(v, lay.v_bytes, "value cache")))
        return st;
    if ((st = check_banks_apart(r->bank, r->bank_bytes, lay, k, v)))
        return st;
    RowTable rt;
    int32_t mx;
    if ((st = build_rows(lay, pos, nullptr, &rt, &mx)))
        return st;
    const int64_t j = r->steps;
    if (r->gather == KV_RING_GATHER_AT_FLUSH) {
        r->pend.emplace_back(k, v);
    } else {
        const int bk = (int)((j / r->R) & 1);
        if (r->wait_needed[bk]) {
            if ((st = wait(compute, r->free_ev(bk), "ring bank wait")))
                return st;
            r->wait_needed[bk] = false;
        }
        void *slot = (char *)r->bank[bk] + (j % r->R) * r->slot_bytes;
        if ((st = enqueue_copy(true, lay, k, v, 0, lay.L, rt, mx, slot, compute)))
            return st;
        if (std::find(r->pack_streams.begin(), r->pack_streams.end(), compute) ==
            r->pack_streams.end())
            r->pack_streams.push_back(compute);
    }
    r->pos.insert(r->pos.end(), pos, pos + lay.B);
    r->steps = j + 1;
    if (r->steps % r->R == 0) {
        if ((st = ring_gather(r, compute)))
            return st;
        return ring_flush_range(r, r->flushed, r->steps - r->flushed, compute);
    }
    return KV_OK;
}

int kv_ring_set_gather(kv_ring *r, int32_t mode)
{
    if (!r)
        return set_error(KV_EINVAL, "ring handle is NULL");
    if (mode != KV_RING_GATHER_EACH_STEP && mode != KV_RING_GATHER_AT_FLUSH)
        return set_error(KV_EINVAL, "gather mode %d is not a kv_ring_gather", mode);
    if (r->steps != r->flushed)
        return set_error(KV_EBUSY, "unflushed steps; flush before changing the gather mode");
    r->gather = mode;
    return KV_OK;
}

int kv_ring_flush(kv_ring *r, hipStream_t compute, hipEvent_t done)
{
    if (!r)
        return set_error(KV_EINVAL, "ring handle is NULL");
    int st;
    if ((st = ring_gather(r, compute)))
        return st;
    if (r->steps > r->flushed &&
        (st = ring_flush_range(r, r->flushed, r->steps - r->flushed, compute)))
        return st;
    if (done && (st = record(done, r->copy, "ring flush done")))
        return st;
    return KV_OK;
}

namespace {

// Unpack steps [0, n) of the host image into (k, v) in ascending step order.
int ring_restore_n(kv_ring *r, void *k, void *v, int64_t n_steps, hipStream_t compute,
                   hipEvent_t done)
{
    const kv_layout &lay = r->lay;
    int st;
    if ((st = check_device_buffer(k, lay.k_bytes, "key cache")) ||
        (st = check_device_buffer(v, lay.v_bytes, "value cache")))
        return st;
    if ((st = check_banks_apart(r->bank, r->bank_bytes, lay, k, v)))
        return st;
    // steps pushed after the last flush may still be packing into a bank
    // the loads below overwrite
    if ((st = ring_order_packs(r, false, nullptr)))
        return st;
    for (int64_t j0 = 0, g = 0; j0 < n_steps; j0 += r->R, ++g) {
        const int64_t n = std::min<int64_t>(r->R, n_steps - j0);
        const int bk = (int)(g & 1);
        if (r->free_valid[bk] && (st = wait(r->copy, r->free_ev(bk), "ring restore bank wait")))
            return st;
        if ((st = transfer(r->transport, r->copier, r->link_blocks, r->bank[bk], (char *)r->host + j0 * r->slot_bytes,
                           (char *)r->host_dev + j0 * r->slot_bytes, n * r->slot_bytes, false,
                           r->copy)))
            return st;
        if ((st = record(r->filled_ev(bk), r->copy, "ring restore loaded")) ||
            (st = wait(compute, r->filled_ev(bk), "ring restore unpack wait")))
            return st;
        // ascending steps; a run of positions advancing by one holds no
        // position twice, so one pass per run keeps the later-step-wins order
        if ((st = ring_copy_steps(r, false, k, v, j0, n, r->bank[bk], compute, nullptr)))
            return st;
        if ((st = record(r->free_ev(bk), compute, "ring restore unpacked")))
            return st;
        r->wait_needed[bk] = true;
        r->free_valid[bk] = true;
    }
    if (done && (st = record(done, compute, "ring restore done")))
        return st;
    return KV_OK;
}

}  // namespace

int kv_ring_restore(kv_ring *r, void *k, void *v, hipStream_t compute, hipEvent_t done)
{
    if (!r)
        return set_error(KV_EINVAL, "ring handle is NULL");
    if (r->flushed != r->steps)
        return set_error(KV_EBUSY, "%lld of %lld steps are not flushed; call kv_ring_flush",
                         (long long)(r->steps - r->flushed), (long long)r->steps);
    return ring_restore_n(r, k, v, r->steps, compute, done);
}

int kv_ring_restore_steps(kv_ring *r, void *k, void *v, int64_t n, hipStream_t compute,
                          hipEvent_t done)
{
    if (!r)
        return set_error(KV_EINVAL, "ring handle is NULL");
    if (n < 0 || n > r->flushed)
        return set_error(KV_ERANGE, "restore of %lld steps; %lld are flushed", (long long)n,
                         (long long)r->flushed);
    const int st = ring_restore_n(r, k, v, n, compute, done);
    if (st != KV_OK)
        return st;
    // the ring now continues from step n: later steps are gone
    if (n < r->steps) {
        r->steps = r->flushed = n;
        r->pend.clear();
        r->pack_streams.clear();
        r->pos.resize((size_t)n * r->lay.B);
        r->durable = std::min(r->durable, n);
        std::deque<std::pair<hipEvent_t, int64_t>> keep;
        for (auto &p : r->landing) {
            if (p.second <= n)
                keep.push_back(p);
            else
                r->spare.push_back(p.first);
        }
        r->landing.swap(keep);
    }
    return KV_OK;
}

int64_t kv_ring_durable_steps(kv_ring *r)
{
    if (!r)
        return set_error(KV_EINVAL, "ring handle is NULL");
    while (!r->landing.empty()) {
        const hipError_t q = hipEventQuery(r->landing.front().first);
        if (q == hipErrorNotReady) {
            (void)hipGetLastError();
            break;
        }
        if (q != hipSuccess)
            return hip_fail(q, "kv_ring_durable_steps");
        r->durable = r->landing.front().second;
        r->spare.push_back(r->landing.front().first);
        r->landing.pop_front();
    }
    return r->durable;
}

int64_t kv_ring_steps(const kv_ring *r)
{
    if (!r)
        return set_error(KV_EINVAL, "ring handle is NULL");
    return r->steps;
}

int kv_ring_reset(kv_ring *r)
{
    if (!r)
        return set_error(KV_EINVAL, "ring handle is NULL");
    if (r->steps > r->flushed)
        return set_error(KV_EBUSY, "unflushed steps; flush before reset");
    r->steps = r->flushed = 0;
    r->durable = 0;
    for (auto &p : r->landing)
        r->spare.push_back(p.first);
    r->landing.clear();
    r->pos.clear();
    r->pend.clear();
    return KV_OK;
}

namespace {

int set_option(int32_t transport, EngineCopier *copier, int32_t *link_blocks, int32_t option,
               int64_t value)
{
    switch (option) {
    case KV_OPT_DMA_ENGINE:
        if (transport != KV_XFER_ENGINE)
            return set_error(KV_EINVAL, "KV_OPT_DMA_ENGINE applies to KV_XFER_ENGINE handles");
        if (value < -1 || value > 3)
            return set_error(KV_EINVAL, "DMA engine %lld is not -1 or 0..3", (long long)value);
        engine_copier_pin(copier, (int32_t)value);
        return KV_OK;
    case KV_OPT_LINK_BLOCKS:
        if (value < 0 || value > kLinkBlocksMax)
            return set_error(KV_EINVAL, "link-copy workgroups %lld outside [0, %d]",
                             (long long)value, kLinkBlocksMax);
        *link_blocks = (int32_t)value;
        return KV_OK;
    default:
        return set_error(KV_EINVAL, "option %d is not a kv_option", option);
    }
}

}  // namespace

int kv_swap_set_option(kv_swap *e, int32_t option, int64_t value)
{
    if (!e)
        return set_error(KV_EINVAL, "swap handle is NULL");
    return set_option(e->transport, e->copier, &e->link_blocks, option, value);
}

int kv_ring_set_option(kv_ring *r, int32_t option, int64_t value)
{
    if (!r)
        return set_error(KV_EINVAL, "ring handle is NULL");
    return set_option(r->transport, r->copier, &r->link_blocks, option, value);
}

}  // extern "C"

