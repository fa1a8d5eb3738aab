// Gather/scatter between a paged KV pool and the packed format.  The pages
// name vLLM's paged memory and Mooncake's chunks; the pool layout is the
// contiguous one with (row, Smax) replaced by (block, block_tokens), and a
// per-row block table maps logical tokens to blocks.
#include "kvs_internal.h"

#include <algorithm>
#include <climits>
#include <cstring>

namespace kvs {
namespace {

constexpr uint32_t kPagedMagic = 0x4b565047u;  // "KVPG"

int check_paged(const kv_paged *pg)
{
    if (pg == nullptr)
        return set_error(KV_EINVAL, "pool descriptor is NULL");
    if (pg->magic != kPagedMagic)
        return set_error(KV_EINVAL, "pool descriptor not initialised by kv_paged_init");
    return KV_OK;
}

// Validates B, the row ranges against the table's logical capacity, and fills
// the row table.
int paged_rows(const kv_paged &pg, int32_t B, int32_t table_stride, const int32_t *start,
               const int32_t *count, RowTable *rt, int32_t *max_count)
{
    if (B <= 0 || B > KV_MAX_ROWS)
        return set_error(KV_EINVAL, "B=%d outside [1, %d]", B, KV_MAX_ROWS);
    if (table_stride <= 0)
        return set_error(KV_EINVAL, "table_stride=%d must be positive", table_stride);
    if (start == nullptr)
        return set_error(KV_EINVAL, "start is NULL");
    const int64_t cap = (int64_t)table_stride * pg.block_tokens;
    if (cap > INT32_MAX)
        return set_error(KV_EINVAL, "table_stride * block_tokens = %lld exceeds int32",
                         (long long)cap);
    int64_t off = 0;
    int32_t mx = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t s = start[b];
        const int32_t c = count ? count[b] : 1;
        if (c < 0)
            return set_error(KV_ERANGE, "row %d: negative count %d", b, c);
        if (c > 0 && (s < 0 || (int64_t)s + c > cap))
            return set_error(KV_ERANGE, "row %d: tokens [%d, +%d) outside the table's [0, %lld)",
                             b, s, c, (long long)cap);
        rt->start[b] = c > 0 ? s : 0;
        rt->off[b] = (int32_t)off;
        off += c;
        mx = std::max(mx, c);
    }
    if (off > INT32_MAX)
        return set_error(KV_ERANGE, "%lld tokens in one call exceed int32", (long long)off);
    rt->off[B] = (int32_t)off;
    *max_count = mx;
    return KV_OK;
}

int paged_entry(bool pack, const kv_paged *pg, const void *k, const void *v, int32_t l0,
                int32_t nl, int32_t B, const int32_t *table, int32_t table_stride,
                const int32_t *start, const int32_t *count, const void *staging,
                int64_t staging_bytes, hipStream_t s)
{
    int st = check_paged(pg);
    if (st)
        return st;
    if (l0 < 0 || nl < 0 || (int64_t)l0 + nl > pg->L)
        return set_error(KV_ERANGE, "layers [%d, +%d) outside [0, %d)", l0, nl, pg->L);
    RowTable rt;
    int32_t max_count = 0;
    if ((st = paged_rows(*pg, B, table_stride, start, count, &rt, &max_count)))
        return st;
    const int64_t need = 2 * (int64_t)nl * pg->H * pg->D * pg->elem_bytes * rt.off[B];
    if (staging_bytes < need)
        return set_error(KV_ESIZE, "staging holds %lld bytes, %lld needed",
                         (long long)staging_bytes, (long long)need);
    if ((st = check_device_buffer(k, pg->k_bytes, "key pool")) ||
        (st = check_device_buffer(v, pg->v_bytes, "value pool")))
        return st;
    const int64_t table_bytes = (int64_t)B * table_stride * 4;
    if (table == nullptr || ((uintptr_t)table & 3u) != 0)
        return set_error(KV_EINVAL, "block table is NULL or not 4-byte aligned");
    if ((st = check_device_buffer((const void *)((uintptr_t)table & ~(uintptr_t)15),
                                  table_bytes + ((uintptr_t)table & 15u), "block table")))
        return st;
    if (need == 0)
        return KV_OK;
    if ((st = check_device_buffer(staging, need, "staging")))
        return st;
    if (overlaps(staging, need, k, pg->k_bytes) || overlaps(staging, need, v, pg->v_bytes) ||
        overlaps(staging, need, table, table_bytes))
        return set_error(KV_EINVAL, "staging overlaps a pool or the block table");
    if (!pack && (overlaps(table, table_bytes, k, pg->k_bytes) ||
                  overlaps(table, table_bytes, v, pg->v_bytes)))
        return set_error(KV_EINVAL, "block table overlaps a pool");
    PagedGeometry g;
    g.k = (uint4 *)k;
    g.v = (uint4 *)v;
    g.stage = (uint4 *)staging;
    g.table = table;
    g.table_stride = table_stride;
    g.NB = pg->blocks;
    g.H = pg->H;
    g.C = pg->D / 8;
    g.P = pg->block_tokens;
    g.p_shift = -1;
    if ((g.P & (g.P - 1)) == 0) {
        g.p_shift = 0;
        while ((1 << g.p_shift) < g.P)
            ++g.p_shift;
    }
    g.B = B;
    g.l0 = l0;
    g.nl = nl;
    g.tiles_per_row = 0;
    g.tile_tokens = 0;
    g.T = rt.off[B];
    return launch_paged_copy(pack, g, rt, max_count, s);
}

}  // namespace
}  // namespace kvs

using namespace kvs;

extern "C" {

int kv_paged_init(kv_paged *out, int32_t L, int32_t blocks, int32_t H, int32_t D,
                  int32_t block_tokens, int32_t dtype)
{
    if (out == nullptr)
        return set_error(KV_EINVAL, "pool descriptor output is NULL");
    std::memset(out, 0, sizeof *out);
    if (L <= 0 || blocks <= 0 || H <= 0 || D <= 0 || block_tokens <= 0)
        return set_error(KV_EINVAL, "dims must be positive (L=%d blocks=%d H=%d D=%d P=%d)", L,
                         blocks, H, D, block_tokens);
    if (D % 8 != 0 || D > KV_MAX_HEAD_DIM)
        return set_error(KV_EINVAL, "D=%d must be a multiple of 8 and at most %d", D,
                         KV_MAX_HEAD_DIM);
    if (dtype != KV_F16 && dtype != KV_BF16)
        return set_error(KV_EINVAL, "dtype %d is neither KV_F16 nor KV_BF16", dtype);
    const __int128 n = (__int128)L * blocks * H * D * block_tokens * 2;
    if (n > (__int128)INT64_MAX / 2)
        return set_error(KV_EINVAL, "pool of %d x %d x %d x %d x %d is too large", L, blocks, H,
                         D, block_tokens);
    if ((int64_t)block_tokens * (D / 8) > INT32_MAX)
        return set_error(KV_EINVAL, "block_tokens * D/8 exceeds int32");
    out->L = L;
    out->blocks = blocks;
    out->H = H;
    out->D = D;
    out->block_tokens = block_tokens;
    out->dtype = dtype;
    out->elem_bytes = 2;
    out->vec_elems = 8;
    out->k_strides[5] = 1;
    out->k_strides[4] = 8;
    out->k_strides[3] = 8 * (int64_t)block_tokens;
    out->k_strides[2] = out->k_strides[3] * (D / 8);
    out->k_strides[1] = out->k_strides[2] * H;
    out->k_strides[0] = out->k_strides[1] * blocks;
    out->v_strides[4] = 1;
    out->v_strides[3] = D;
    out->v_strides[2] = (int64_t)D * block_tokens;
    out->v_strides[1] = out->v_strides[2] * H;
    out->v_strides[0] = out->v_strides[1] * blocks;
    out->k_bytes = out->k_strides[0] * L * 2;
    out->v_bytes = out->v_strides[0] * L * 2;
    out->magic = kPagedMagic;
    return KV_OK;
}

int64_t kv_paged_pack_bytes(const kv_paged *pg, int32_t layer_count, int32_t B,
                            const int32_t *count)
{
    int st = check_paged(pg);
    if (st)
        return st;
    if (layer_count < 0 || layer_count > pg->L)
        return set_error(KV_ERANGE, "layer_count %d outside [0, %d]", layer_count, pg->L);
    if (B <= 0 || B > KV_MAX_ROWS)
        return set_error(KV_EINVAL, "B=%d outside [1, %d]", B, KV_MAX_ROWS);
    int64_t tokens = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t c = count ? count[b] : 1;
        if (c < 0)
            return set_error(KV_ERANGE, "row %d: negative count %d", b, c);
        tokens += c;
    }
    return 2 * (int64_t)layer_count * pg->H * pg->D * pg->elem_bytes * tokens;
}

int kv_pack_paged(const kv_paged *pg, const void *k, const void *v, int32_t layer_begin,
                  int32_t layer_count, int32_t B, const int32_t *table, int32_t table_stride,
                  const int32_t *start, const int32_t *count, void *staging,
                  int64_t staging_bytes, hipStream_t s)
{
    return paged_entry(true, pg, k, v, layer_begin, layer_count, B, table, table_stride, start,
                       count, staging, staging_bytes, s);
}

int kv_unpack_paged(const kv_paged *pg, void *k, void *v, int32_t layer_begin,
                    int32_t layer_count, int32_t B, const int32_t *table, int32_t table_stride,
                    const int32_t *start, const int32_t *count, const void *staging,
                    int64_t staging_bytes, hipStream_t s)
{
    return paged_entry(false, pg, k, v, layer_begin, layer_count, B, table, table_stride, start,
                       count, staging, staging_bytes, s);
}

int kv_paged_check_table(const kv_paged *pg, int32_t B, const int32_t *table,
                         int32_t table_stride, const int32_t *start, const int32_t *count)
{
    int st = check_paged(pg);
    if (st)
        return st;
    RowTable rt;
    int32_t mx;
    if ((st = paged_rows(*pg, B, table_stride, start, count, &rt, &mx)))
        return st;
    if (table == nullptr)
        return set_error(KV_EINVAL, "block table is NULL");
    for (int32_t b = 0; b < B; ++b) {
        const int32_t c = rt.off[b + 1] - rt.off[b];
        if (c == 0)
            continue;
        const int32_t q0 = rt.start[b] / pg->block_tokens;
        const int32_t q1 = (rt.start[b] + c - 1) / pg->block_tokens;
        for (int32_t q = q0; q <= q1; ++q) {
            const int32_t id = table[(int64_t)b * table_stride + q];
            if (id < 0 || id >= pg->blocks)
                return set_error(KV_ERANGE, "row %d block %d: id %d outside [0, %d)", b, q, id,
                                 pg->blocks);
        }
    }
    return KV_OK;
}

}  // extern "C"
