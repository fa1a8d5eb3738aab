// stream_out / stream_in between workers that split the model differently
// ("DejaVu: KV-Cache Streaming ...", DejaVuLib primitives, Table 1; Fast
// prompt KV transfer): the piece two partitions share is a layer range, a
// head range and a row range of each side's cache, moved with the same
// pack/unpack kernels restricted to those heads.
#include "kvs_internal.h"

#include <algorithm>
#include <climits>

namespace kvs {
namespace {

struct Range {
    int32_t lo, hi;   // [lo, hi), hi >= lo
    int32_t n() const { return hi - lo; }
};

Range meet(int32_t a0, int32_t an, int32_t b0, int32_t bn)
{
    const int32_t lo = std::max(a0, b0);
    const int32_t hi = std::min(a0 + an, b0 + bn);
    return {lo, std::max(lo, hi)};
}

int check_part(const kv_part *p, const char *name)
{
    if (p == nullptr)
        return set_error(KV_EINVAL, "%s partition is NULL", name);
    if (p->layer0 < 0 || p->head0 < 0 || p->row0 < 0 || p->layers <= 0 || p->heads <= 0 ||
        p->rows <= 0)
        return set_error(KV_EINVAL, "%s partition {%d,%d,%d,%d,%d,%d}: offsets must be >= 0 "
                         "and sizes > 0", name, p->layer0, p->layers, p->head0, p->heads,
                         p->row0, p->rows);
    if ((int64_t)p->layer0 + p->layers > INT_MAX || (int64_t)p->head0 + p->heads > INT_MAX ||
        (int64_t)p->row0 + p->rows > INT_MAX)
        return set_error(KV_EINVAL, "%s partition ends past INT_MAX", name);
    return KV_OK;
}

// The shared ranges of `self` (whose cache `lay` describes) and `peer`, and the
// row table of self's local rows with rows outside the meet masked out.
struct Piece {
    Range layers, heads, rows;
    RowTable rt;
    int32_t max_count;
    int64_t bytes;
};

int plan_piece(const kv_layout *lay, const kv_part *self, const kv_part *peer,
               const int32_t *start, const int32_t *count, Piece *pc)
{
    int st = check_layout(lay);
    if (st)
        return st;
    if ((st = check_part(self, "own")) || (st = check_part(peer, "peer")))
        return st;
    if (lay->L != self->layers || lay->H != self->heads || lay->B != self->rows)
        return set_error(KV_EINVAL, "layout (L=%d, B=%d, H=%d) does not hold the partition "
                         "(%d layers, %d rows, %d heads)", lay->L, lay->B, lay->H, self->layers,
                         self->rows, self->heads);
    pc->layers = meet(self->layer0, self->layers, peer->layer0, peer->layers);
    pc->heads = meet(self->head0, self->heads, peer->head0, peer->heads);
    pc->rows = meet(self->row0, self->rows, peer->row0, peer->rows);
    // every local row's range is checked; rows outside the meet then move nothing
    int32_t s_in[KV_MAX_ROWS], c_in[KV_MAX_ROWS];
    for (int32_t b = 0; b < lay->B; ++b) {
        const int32_t g = self->row0 + b;
        const bool shared = g >= pc->rows.lo && g < pc->rows.hi && pc->layers.n() > 0 &&
                            pc->heads.n() > 0;
        s_in[b] = start ? start[b] : 0;
        c_in[b] = count ? count[b] : 1;
        if (c_in[b] < 0)
            return set_error(KV_ERANGE, "row %d: negative count %d", b, c_in[b]);
        if (c_in[b] > 0 && (s_in[b] < 0 || (int64_t)s_in[b] + c_in[b] > lay->Smax))
            return set_error(KV_ERANGE, "row %d: tokens [%d, +%d) outside [0, %d)", b, s_in[b],
                             c_in[b], lay->Smax);
        if (!shared)
            s_in[b] = c_in[b] = 0;
    }
    if ((st = build_rows(*lay, s_in, c_in, &pc->rt, &pc->max_count)))
        return st;
    pc->bytes = 2 * (int64_t)pc->layers.n() * pc->heads.n() * lay->D * lay->elem_bytes *
                (int64_t)pc->rt.off[lay->B];
    return KV_OK;
}

int stream_copy(bool out, const kv_layout *lay, const kv_part *self, const void *k,
                const void *v, const kv_part *peer, const int32_t *start,
                const int32_t *count, const void *staging, int64_t staging_bytes, hipStream_t s)
{
    if (start == nullptr)
        return set_error(KV_EINVAL, "start is NULL");
    Piece pc;
    int st = plan_piece(lay, self, peer, start, count, &pc);
    if (st)
        return st;
    if (staging_bytes < pc.bytes)
        return set_error(KV_ESIZE, "staging holds %lld bytes, the piece needs %lld",
                         (long long)staging_bytes, (long long)pc.bytes);
    if ((st = check_device_buffer(k, lay->k_bytes, "key cache")) ||
        (st = check_device_buffer(v, lay->v_bytes, "value cache")))
        return st;
    if (pc.bytes == 0)
        return KV_OK;
    if ((st = check_device_buffer(staging, pc.bytes, "staging")))
        return st;
    if (overlaps(staging, pc.bytes, k, lay->k_bytes) || overlaps(staging, pc.bytes, v, lay->v_bytes))
        return set_error(KV_EINVAL, "staging overlaps a cache");
    return enqueue_copy(out, *lay, k, v, pc.layers.lo - self->layer0, pc.layers.n(), pc.rt,
                        pc.max_count, (void *)staging, s, pc.heads.lo - self->head0,
                        pc.heads.n());
}

}  // namespace
}  // namespace kvs

using namespace kvs;

extern "C" {

int64_t kv_stream_bytes(const kv_layout *lay, const kv_part *self, const kv_part *peer,
                        const int32_t *count)
{
    // the byte count depends on counts only; a zero start row stands in
    static const int32_t zeros[KV_MAX_ROWS] = {};
    Piece pc;
    const int st = plan_piece(lay, self, peer, zeros, count, &pc);
    return st ? st : pc.bytes;
}

int kv_stream_out(const kv_layout *lay, const kv_part *src, const void *k, const void *v,
                  const kv_part *dst, const int32_t *start, const int32_t *count,
                  void *staging, int64_t staging_bytes, hipStream_t s)
{
    return stream_copy(true, lay, src, k, v, dst, start, count, staging, staging_bytes, s);
}

int kv_stream_in(const kv_layout *lay, const kv_part *dst, void *k, void *v,
                 const kv_part *src, const int32_t *start, const int32_t *count,
                 const void *staging, int64_t staging_bytes, hipStream_t s)
{
    return stream_copy(false, lay, dst, k, v, src, start, count, staging, staging_bytes, s);
}

}  // extern "C"
