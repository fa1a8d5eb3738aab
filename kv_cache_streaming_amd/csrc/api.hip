// C-ABI entry points: layout descriptor, pack/unpack, errors, live timing.
#include "kvs_internal.h"

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <strings.h>
#include <utility>
#include <vector>

namespace kvs {

namespace {
thread_local char g_error[512] = "no error";
}

int set_error(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return status;
}

int hip_fail(hipError_t e, const char *what)
{
    return set_error(KV_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

int check_layout(const kv_layout *lay)
{
    if (lay == nullptr)
        return set_error(KV_EINVAL, "layout is NULL");
    if (lay->magic != kLayoutMagic)
        return set_error(KV_EINVAL, "layout was not filled by kv_layout_init");
    return KV_OK;
}

bool overlaps(const void *a, int64_t an, const void *b, int64_t bn)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return an > 0 && bn > 0 && x < y + (uintptr_t)bn && y < x + (uintptr_t)an;
}

namespace {

// Memory type of one address, or -1 when HIP does not know it (pageable host
// memory, garbage).  Clears the sticky error HIP may leave behind.
int memory_type(const void *p)
{
    hipPointerAttribute_t a;
    std::memset(&a, 0, sizeof a);
    const hipError_t e = hipPointerGetAttributes(&a, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return (int)a.type;
}

}  // namespace

int check_device_buffer(const void *p, int64_t bytes, const char *name)
{
    if (p == nullptr)
        return set_error(KV_EINVAL, "%s is NULL", name);
    if (((uintptr_t)p & 15u) != 0)
        return set_error(KV_EINVAL, "%s is not 16-byte aligned", name);
    if (bytes <= 0)
        return KV_OK;
    const char *end = (const char *)p + (bytes - 1);
    const int t0 = memory_type(p), t1 = memory_type(end);
    if (t0 != hipMemoryTypeDevice || t1 != hipMemoryTypeDevice)
        return set_error(KV_EINVAL, "%s [%p, +%lld) is not device memory", name, p,
                         (long long)bytes);
    // the whole range must lie in the one allocation that holds its first byte
    // (two adjacent allocations would pass the check of both ends)
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) == hipSuccess && base) {
        const uintptr_t b = (uintptr_t)base, x = (uintptr_t)p;
        if (x < b || (uint64_t)(x - b) + (uint64_t)bytes > (uint64_t)size)
            return set_error(KV_EINVAL,
                             "%s [%p, +%lld) runs past the end of its allocation [%p, +%zu)",
                             name, p, (long long)bytes, base, size);
    } else {
        (void)hipGetLastError();   // memory the runtime cannot size: the end checks stand
    }
    return KV_OK;
}

bool serialized_dispatch()
{
    // HIP's own serialisation switch, and the environment rocprofv3 sets for
    // hardware counter collection (which runs one dispatch at a time)
    auto on = [](const char *name) {
        const char *v = std::getenv(name);
        return v && *v && std::strcmp(v, "0") != 0 && strcasecmp(v, "false") != 0;
    };
    return on("AMD_SERIALIZE_KERNEL") || on("ROCPROF_COUNTER_COLLECTION");
}

int check_pinned_host(const void *p, int64_t bytes, const char *name)
{
    if (p == nullptr)
        return set_error(KV_EINVAL, "%s is NULL", name);
    if (((uintptr_t)p & 15u) != 0)
        return set_error(KV_EINVAL, "%s is not 16-byte aligned", name);
    if (bytes <= 0)
        return KV_OK;
    const char *end = (const char *)p + (bytes - 1);
    const int t0 = memory_type(p), t1 = memory_type(end);
    if (t0 != hipMemoryTypeHost || t1 != hipMemoryTypeHost)
        return set_error(KV_EINVAL, "%s [%p, +%lld) is not pinned host memory", name, p,
                         (long long)bytes);
    return KV_OK;
}

int host_device_address(const void *host, int64_t bytes, void **dev)
{
    hipPointerAttribute_t a;
    std::memset(&a, 0, sizeof a);
    if (hipPointerGetAttributes(&a, host) != hipSuccess || a.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return set_error(KV_EINVAL, "%p is not pinned host memory", host);
    }
    if (a.devicePointer == nullptr || a.hostPointer == nullptr)
        return set_error(KV_EINVAL, "pinned host memory at %p is not mapped for the GPU", host);
    char *d = (char *)a.devicePointer + ((const char *)host - (const char *)a.hostPointer);
    if (bytes > 0) {
        // the whole range must map with the same offset (one allocation)
        hipPointerAttribute_t b;
        std::memset(&b, 0, sizeof b);
        const char *end = (const char *)host + (bytes - 1);
        if (hipPointerGetAttributes(&b, end) != hipSuccess || b.devicePointer == nullptr ||
            (char *)b.devicePointer + (end - (const char *)b.hostPointer) != d + (bytes - 1)) {
            (void)hipGetLastError();
            return set_error(KV_EINVAL, "pinned host range at %p does not map contiguously", host);
        }
    }
    *dev = d;
    return KV_OK;
}

int check_layers(const kv_layout &lay, int32_t layer_begin, int32_t layer_count)
{
    if (layer_count < 0 || layer_begin < 0 || layer_begin > lay.L ||
        (int64_t)layer_begin + layer_count > lay.L)
        return set_error(KV_ERANGE, "layers [%d, +%d) outside [0, %d)", layer_begin,
                         layer_count, lay.L);
    return KV_OK;
}

int64_t packed_bytes(const kv_layout &lay, int32_t nl, int64_t tokens)
{
    return 2 * (int64_t)nl * lay.H * lay.D * lay.elem_bytes * tokens;
}

int build_rows(const kv_layout &lay, const int32_t *start, const int32_t *count, RowTable *rt,
               int32_t *max_count)
{
    if (start == nullptr)
        return set_error(KV_EINVAL, "start is NULL");
    int64_t off = 0;
    int32_t mx = 0;
    for (int32_t b = 0; b < lay.B; ++b) {
        const int32_t s = start[b];
        const int32_t c = count ? count[b] : 1;
        if (c < 0)
            return set_error(KV_ERANGE, "row %d: negative count %d", b, c);
        if (c > 0 && (s < 0 || (int64_t)s + c > lay.Smax))
            return set_error(KV_ERANGE, "row %d: tokens [%d, +%d) outside [0, %d)", b, s, c,
                             lay.Smax);
        rt->start[b] = c > 0 ? s : 0;
        rt->off[b] = (int32_t)off;
        off += c;
        mx = std::max(mx, c);
    }
    rt->off[lay.B] = (int32_t)off;   // B * Smax <= 256 * 2^31: checked at init
    *max_count = mx;
    return KV_OK;
}

int enqueue_copy(bool pack, const kv_layout &lay, const void *k, const void *v, int32_t l0,
                 int32_t nl, const RowTable &rt, int32_t max_count, void *stage, hipStream_t s,
                 int32_t h0, int32_t nh)
{
    Geometry g;
    g.k = (uint4 *)k;
    g.v = (uint4 *)v;
    g.stage = (uint4 *)stage;
    g.B = lay.B;
    g.H = lay.H;
    g.C = lay.D / 8;
    g.Smax = lay.Smax;
    g.l0 = l0;
    g.nl = nl;
    g.h0 = nh < 0 ? 0 : h0;
    g.nh = nh < 0 ? lay.H : nh;
    g.tiles_per_row = 0;
    g.tile_tokens = 0;
    g.layer_wgs = 0;
    g.T = rt.off[lay.B];
    return launch_copy(pack, g, rt, max_count, s);
}

int enqueue_steps(bool pack, const kv_layout &lay, const void *k, const void *v,
                  const int32_t *pos0, int32_t n, void *stage, int64_t slot_bytes,
                  hipStream_t s)
{
    RowTable rt;
    for (int32_t b = 0; b < lay.B; ++b) {
        if (pos0[b] < 0 || (int64_t)pos0[b] + n > lay.Smax)
            return set_error(KV_ERANGE, "row %d: steps at [%d, +%d) outside [0, %d)", b, pos0[b],
                             n, lay.Smax);
        rt.start[b] = pos0[b];
        rt.off[b] = b;
    }
    rt.off[lay.B] = lay.B;
    Geometry g;
    g.k = (uint4 *)k;
    g.v = (uint4 *)v;
    g.stage = (uint4 *)stage;
    g.B = lay.B;
    g.H = lay.H;
    g.C = lay.D / 8;
    g.Smax = lay.Smax;
    g.l0 = 0;
    g.nl = lay.L;
    g.h0 = 0;
    g.nh = lay.H;
    g.tiles_per_row = 0;
    g.tile_tokens = 0;
    g.layer_wgs = 0;
    g.T = lay.B;
    return launch_steps(pack, g, rt, n, slot_bytes / 16, s);
}

int prompt_rows(const kv_layout &lay, int32_t tok_begin, int32_t tok_count,
                const int32_t *row_len, int32_t *start, int32_t *count)
{
    if (tok_begin < 0 || tok_count < 0 || (int64_t)tok_begin + tok_count > lay.Smax)
        return set_error(KV_ERANGE, "prompt tokens [%d, +%d) outside [0, %d)", tok_begin,
                         tok_count, lay.Smax);
    for (int32_t b = 0; b < lay.B; ++b) {
        int32_t end = tok_begin + tok_count;
        if (row_len) {
            if (row_len[b] < 0 || row_len[b] > lay.Smax)
                return set_error(KV_ERANGE, "row %d: length %d outside [0, %d]", b, row_len[b],
                                 lay.Smax);
            end = std::min(end, row_len[b]);
        }
        start[b] = tok_begin;
        count[b] = std::max(0, end - tok_begin);
    }
    return KV_OK;
}


// ---------------------------------------------------------------------------
// live kernel timing
namespace {

struct Pending {
    hipEvent_t a, b;
    std::string name;
    int64_t bytes;
};

struct ProfileState {
    std::mutex mu;
    bool on = false;
    std::vector<Pending> pending;
    std::vector<hipEvent_t> pool;
    kv_profile_window last{};
};

// Length of the union of [start, end) intervals (sorted in place).
double union_ms(std::vector<std::pair<double, double>> &iv)
{
    std::sort(iv.begin(), iv.end());
    double total = 0.0, lo = 0.0, hi = 0.0;
    bool open = false;
    for (const auto &x : iv) {
        if (open && x.first <= hi) {
            hi = std::max(hi, x.second);
            continue;
        }
        if (open)
            total += hi - lo;
        lo = x.first;
        hi = x.second;
        open = true;
    }
    if (open)
        total += hi - lo;
    return total;
}

ProfileState &prof()
{
    static ProfileState *p = new ProfileState();  // never destroyed: events may outlive static dtors
    return *p;
}

hipEvent_t take_event(ProfileState &ps)
{
    if (!ps.pool.empty()) {
        hipEvent_t e = ps.pool.back();
        ps.pool.pop_back();
        return e;
    }
    // Timing only: these events are bound to dispatches and never order
    // streams, so they are made without the system-scope fence (a recorded
    // default event writes back and invalidates the caches).
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    return e;
}

}  // namespace

LaunchTimer profile_take()
{
    ProfileState &ps = prof();
    std::lock_guard<std::mutex> g(ps.mu);
    LaunchTimer t;
    if (!ps.on)
        return t;
    hipEvent_t a = take_event(ps);
    hipEvent_t b = take_event(ps);
    if (!a || !b) {
        if (a) ps.pool.push_back(a);
        if (b) ps.pool.push_back(b);
        return t;
    }
    t.start = a;
    t.stop = b;
    return t;
}

void profile_commit(const LaunchTimer &t, const char *name, int64_t bytes, bool launched)
{
    if (!t.start)
        return;
    ProfileState &ps = prof();
    std::lock_guard<std::mutex> g(ps.mu);
    if (launched) {
        ps.pending.push_back(Pending{t.start, t.stop, std::string(name), bytes});
    } else {
        ps.pool.push_back(t.start);
        ps.pool.push_back(t.stop);
    }
}

}  // namespace kvs

using namespace kvs;

extern "C" {

int kv_version(void) { return KV_VERSION; }

const char *kv_last_error(void) { return kvs::g_error; }

int kv_layout_init(kv_layout *out, int32_t L, int32_t B, int32_t H, int32_t D, int32_t Smax,
                   int32_t dtype)
{
    if (out == nullptr)
        return set_error(KV_EINVAL, "layout output is NULL");
    std::memset(out, 0, sizeof *out);
    if (L <= 0 || B <= 0 || H <= 0 || D <= 0 || Smax <= 0)
        return set_error(KV_EINVAL, "dims must be positive (L=%d B=%d H=%d D=%d Smax=%d)", L, B,
                         H, D, Smax);
    if (D % 8 != 0 || D > KV_MAX_HEAD_DIM)
        return set_error(KV_EINVAL, "D=%d must be a multiple of 8 and at most %d", D,
                         KV_MAX_HEAD_DIM);
    if (B > KV_MAX_ROWS)
        return set_error(KV_EINVAL, "B=%d exceeds %d rows", B, KV_MAX_ROWS);
    if (dtype != KV_F16 && dtype != KV_BF16)
        return set_error(KV_EINVAL, "dtype %d is neither KV_F16 nor KV_BF16", dtype);
    // bytes = L*B*H*D*Smax*2 must fit int64 (and every intermediate of it)
    __int128 n = (__int128)L * B * H * D * Smax * 2;
    if (n > (__int128)INT64_MAX / 2)
        return set_error(KV_EINVAL, "cache of %d x %d x %d x %d x %d is too large", L, B, H, D,
                         Smax);
    // one head's key (or value) region, in 16-byte vectors, must fit int32:
    // per-token offsets inside a head are 32-bit in the kernels
    if ((int64_t)Smax * (D / 8) > INT32_MAX)
        return set_error(KV_EINVAL, "Smax * D/8 = %lld exceeds int32", (long long)Smax * (D / 8));
    // total packed tokens of one call must fit int32 (row offsets travel as int32)
    if ((int64_t)B * Smax > INT32_MAX)
        return set_error(KV_EINVAL, "B * Smax = %lld exceeds int32", (long long)B * Smax);
    out->L = L;
    out->B = B;
    out->H = H;
    out->D = D;
    out->Smax = Smax;
    out->dtype = dtype;
    out->elem_bytes = 2;
    out->vec_elems = 8;
    // K [L,B,H,D/8,Smax,8]
    out->k_strides[5] = 1;
    out->k_strides[4] = 8;
    out->k_strides[3] = 8 * (int64_t)Smax;
    out->k_strides[2] = out->k_strides[3] * (D / 8);
    out->k_strides[1] = out->k_strides[2] * H;
    out->k_strides[0] = out->k_strides[1] * B;
    // V [L,B,H,Smax,D]
    out->v_strides[4] = 1;
    out->v_strides[3] = D;
    out->v_strides[2] = (int64_t)D * Smax;
    out->v_strides[1] = out->v_strides[2] * H;
    out->v_strides[0] = out->v_strides[1] * B;
    out->k_bytes = out->k_strides[0] * L * 2;
    out->v_bytes = out->v_strides[0] * L * 2;
    out->magic = kLayoutMagic;
    return KV_OK;
}

int64_t kv_pack_bytes(const kv_layout *lay, int32_t layer_count, const int32_t *count,
                      int32_t uniform_count)
{
    int st = check_layout(lay);
    if (st)
        return st;
    if (layer_count < 0 || layer_count > lay->L)
        return set_error(KV_ERANGE, "layer_count %d outside [0, %d]", layer_count, lay->L);
    int64_t tokens = 0;
    for (int32_t b = 0; b < lay->B; ++b) {
        const int32_t c = count ? count[b] : uniform_count;
        if (c < 0 || c > lay->Smax)
            return set_error(KV_ERANGE, "row %d: count %d outside [0, %d]", b, c, lay->Smax);
        tokens += c;
    }
    return packed_bytes(*lay, layer_count, tokens);
}

namespace {

int copy_entry(bool pack, const kv_layout *lay, const void *k, const void *v, int32_t l0,
               int32_t nl, const int32_t *start, const int32_t *count, const void *staging,
               int64_t staging_bytes, hipStream_t s)
{
    int st = check_layout(lay);
    if (st)
        return st;
    if ((st = check_layers(*lay, l0, nl)))
        return st;
    RowTable rt;
    int32_t max_count = 0;
    if ((st = build_rows(*lay, start, count, &rt, &max_count)))
        return st;
    const int64_t need = packed_bytes(*lay, nl, rt.off[lay->B]);
    if (staging_bytes < need)
        return set_error(KV_ESIZE, "staging holds %lld bytes, %lld needed",
                         (long long)staging_bytes, (long long)need);
    if ((st = check_device_buffer(k, lay->k_bytes, "key cache")))
        return st;
    if ((st = check_device_buffer(v, lay->v_bytes, "value cache")))
        return st;
    if ((st = check_device_buffer(staging, need, "staging")))
        return st;
    if (overlaps(staging, need, k, lay->k_bytes) || overlaps(staging, need, v, lay->v_bytes))
        return set_error(KV_EINVAL, "staging overlaps a cache");
    if (need == 0)
        return KV_OK;
    return enqueue_copy(pack, *lay, k, v, l0, nl, rt, max_count, (void *)staging, s);
}

}  // namespace

int kv_pack_tokens(const kv_layout *lay, const void *k, const void *v, int32_t layer_begin,
                   int32_t layer_count, const int32_t *start, const int32_t *count,
                   void *staging, int64_t staging_bytes, hipStream_t s)
{
    return copy_entry(true, lay, k, v, layer_begin, layer_count, start, count, staging,
                      staging_bytes, s);
}

int kv_unpack_tokens(const kv_layout *lay, void *k, void *v, int32_t layer_begin,
                     int32_t layer_count, const int32_t *start, const int32_t *count,
                     const void *staging, int64_t staging_bytes, hipStream_t s)
{
    return copy_entry(false, lay, k, v, layer_begin, layer_count, start, count, staging,
                      staging_bytes, s);
}

int kv_pack_prompt_layer(const kv_layout *lay, const void *k, const void *v, int32_t layer,
                         int32_t tok_begin, int32_t tok_count, const int32_t *row_len,
                         void *staging, int64_t staging_bytes, hipStream_t s)
{
    int st = check_layout(lay);
    if (st)
        return st;
    int32_t start[KV_MAX_ROWS], count[KV_MAX_ROWS];
    if ((st = prompt_rows(*lay, tok_begin, tok_count, row_len, start, count)))
        return st;
    return copy_entry(true, lay, k, v, layer, 1, start, count, staging, staging_bytes, s);
}

int kv_unpack_prompt_layer(const kv_layout *lay, void *k, void *v, int32_t layer,
                           int32_t tok_begin, int32_t tok_count, const int32_t *row_len,
                           const void *staging, int64_t staging_bytes, hipStream_t s)
{
    int st = check_layout(lay);
    if (st)
        return st;
    int32_t start[KV_MAX_ROWS], count[KV_MAX_ROWS];
    if ((st = prompt_rows(*lay, tok_begin, tok_count, row_len, start, count)))
        return st;
    return copy_entry(false, lay, k, v, layer, 1, start, count, staging, staging_bytes, s);
}

int kv_profile_begin(void)
{
    ProfileState &ps = prof();
    std::lock_guard<std::mutex> g(ps.mu);
    for (auto &p : ps.pending) {
        ps.pool.push_back(p.a);
        ps.pool.push_back(p.b);
    }
    ps.pending.clear();
    ps.on = true;
    return KV_OK;
}

int kv_profile_end(kv_kernel_stat *out, int32_t max)
{
    ProfileState &ps = prof();
    std::lock_guard<std::mutex> g(ps.mu);
    ps.on = false;
    std::vector<kv_kernel_stat> stats;
    int status = KV_OK;
    // every timed kernel's interval, as offsets from the first one's start
    std::vector<std::pair<double, double>> hbm_iv, link_iv;
    kv_profile_window win{};
    double first = 0.0, last = 0.0;
    for (auto &p : ps.pending) {
        float ms = 0.f, t0 = 0.f;
        hipError_t e = hipEventSynchronize(p.b);
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms, p.a, p.b);
        if (e == hipSuccess)
            e = hipEventElapsedTime(&t0, ps.pending.front().a, p.a);
        if (e != hipSuccess) {
            status = hip_fail(e, "kv_profile_end");
            (void)hipGetLastError();
        }
        const bool link = p.name.compare(0, 9, "link_copy") == 0;
        (link ? link_iv : hbm_iv).emplace_back((double)t0, (double)t0 + ms);
        if (link) {
            win.link_bytes += p.bytes;
            win.link_launches += 1;
        } else {
            win.hbm_bytes += p.bytes;
            win.hbm_launches += 1;
        }
        first = std::min(first, (double)t0);
        last = std::max(last, (double)t0 + ms);
        auto it = std::find_if(stats.begin(), stats.end(), [&](const kv_kernel_stat &s) {
            return p.name == s.name;
        });
        if (it == stats.end()) {
            kv_kernel_stat s;
            std::memset(&s, 0, sizeof s);
            std::snprintf(s.name, sizeof s.name, "%s", p.name.c_str());
            stats.push_back(s);
            it = stats.end() - 1;
        }
        it->launches += 1;
        it->ms += ms;
        it->bytes += p.bytes;
        ps.pool.push_back(p.a);
        ps.pool.push_back(p.b);
    }
    if (!ps.pending.empty()) {
        win.span_ms = last - first;
        win.hbm_busy_ms = union_ms(hbm_iv);
        win.link_busy_ms = union_ms(link_iv);
    }
    ps.last = win;
    ps.pending.clear();
    if (status != KV_OK)
        return status;
    for (int32_t i = 0; out && i < max && i < (int32_t)stats.size(); ++i)
        out[i] = stats[i];
    return (int)stats.size();
}

int kv_profile_last_window(kv_profile_window *out)
{
    if (!out)
        return set_error(KV_EINVAL, "output pointer is NULL");
    ProfileState &ps = prof();
    std::lock_guard<std::mutex> g(ps.mu);
    *out = ps.last;
    return KV_OK;
}

}  // extern "C"
