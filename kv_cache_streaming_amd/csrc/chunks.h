// Chunking of a staged transfer between a cache and pinned host memory:
// the pieces a swap moves through a device bank of a given size, in order.
// Shared by the swap engine and the single-stream swap-out.
#pragma once

#include <algorithm>

#include "kvs_internal.h"

namespace kvs {

struct Chunk {
    int32_t l0, nl, b0, b1;
    int64_t staged;
    int32_t pieces;
    int64_t host_off[2], bank_off[2], bytes[2];
};

// Calls f(chunk) for each chunk of a transfer of layers [l0, l0+nl) and the
// rows of `rt`: whole layers (as many as fit a bank) when a layer fits,
// otherwise row groups of one layer (whose K part and V part are then two
// contiguous pieces of the host image).  Stops at the first non-zero return
// of f and returns it; KV_ESIZE when one (layer, row) block exceeds the bank
// (before any call of f); KV_OK otherwise.  Allocates nothing.
template <class F>
int for_each_chunk(const kv_layout &lay, int32_t l0, int32_t nl, const RowTable &rt,
                   int64_t bank_bytes, F &&f)
{
    const int64_t T = rt.off[lay.B];
    const int64_t per_tok = (int64_t)lay.H * lay.D * lay.elem_bytes;   // one K (or V) token of a row
    const int64_t layer_bytes = 2 * per_tok * T;
    if (nl == 0 || T == 0)
        return KV_OK;
    int st;
    if (layer_bytes <= bank_bytes) {
        const int32_t per = (int32_t)std::min<int64_t>(nl, bank_bytes / layer_bytes);
        for (int32_t l = 0; l < nl; l += per) {
            Chunk c;
            c.l0 = l0 + l;
            c.nl = std::min(per, nl - l);
            c.b0 = 0;
            c.b1 = lay.B;
            c.staged = c.nl * layer_bytes;
            c.pieces = 1;
            c.host_off[0] = l * layer_bytes;
            c.bank_off[0] = 0;
            c.bytes[0] = c.staged;
            c.host_off[1] = c.bank_off[1] = c.bytes[1] = 0;
            if ((st = f(c)))
                return st;
        }
        return KV_OK;
    }
    for (int32_t b = 0; b < lay.B; ++b) {
        const int64_t rb = 2 * per_tok * (rt.off[b + 1] - rt.off[b]);
        if (rb > bank_bytes)
            return set_error(KV_ESIZE, "row %d of one layer needs %lld bytes; banks hold %lld", b,
                             (long long)rb, (long long)bank_bytes);
    }
    for (int32_t l = 0; l < nl; ++l) {
        int32_t b0 = 0;
        while (b0 < lay.B) {
            int32_t b1 = b0;
            while (b1 < lay.B &&
                   2 * per_tok * (rt.off[b1 + 1] - rt.off[b0]) <= bank_bytes)
                ++b1;
            const int64_t tok = rt.off[b1] - rt.off[b0];
            if (tok > 0) {
                Chunk c;
                c.l0 = l0 + l;
                c.nl = 1;
                c.b0 = b0;
                c.b1 = b1;
                c.staged = 2 * per_tok * tok;
                c.pieces = 2;
                c.host_off[0] = l * layer_bytes + per_tok * rt.off[b0];
                c.host_off[1] = l * layer_bytes + per_tok * T + per_tok * rt.off[b0];
                c.bank_off[0] = 0;
                c.bank_off[1] = per_tok * tok;
                c.bytes[0] = c.bytes[1] = per_tok * tok;
                if ((st = f(c)))
                    return st;
            }
            b0 = b1;
        }
    }
    return KV_OK;
}

// Row table of one chunk: rows outside [b0, b1) move nothing.
inline void chunk_rows(const kv_layout &lay, const RowTable &rt, const Chunk &c, RowTable *sub,
                       int32_t *max_count)
{
    int32_t off = 0, mx = 0;
    for (int32_t b = 0; b < lay.B; ++b) {
        const int32_t n = (b >= c.b0 && b < c.b1) ? rt.off[b + 1] - rt.off[b] : 0;
        sub->start[b] = n ? rt.start[b] : 0;
        sub->off[b] = off;
        off += n;
        mx = std::max(mx, n);
    }
    sub->off[lay.B] = off;
    *max_count = mx;
}

}  // namespace kvs
