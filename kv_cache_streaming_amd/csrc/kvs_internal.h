// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvstream.h"

namespace kvs {

constexpr uint32_t kLayoutMagic = 0x4b565354u;  // "KVST"
constexpr int kMaxRows = KV_MAX_ROWS;

// Per-call row metadata, passed by value in the kernel arguments so that it
// is captured at launch and needs no device allocation.
struct RowTable {
    int32_t start[kMaxRows];    // first cache position of row b's range
    int32_t off[kMaxRows + 1];  // prefix sums of the counts: row b's tokens are [off[b], off[b+1])
};

// Geometry of one pack/unpack launch, in 16-byte vectors.
struct Geometry {
    uint4 *k;        // key cache base
    uint4 *v;        // value cache base
    uint4 *stage;    // packed buffer base
    int32_t B, H, C, Smax;  // C = D/8 vectors per head row; H = heads of the cache
    int32_t l0, nl;         // layer range
    int32_t h0, nh;         // head range [h0, h0 + nh) moved; the packed format has nh heads
    int32_t tiles_per_row;  // tile kernel: tiles per (row, head) of a dense grid (the longest
                            // row's), or 0 for a grid of the rows' own tiles (RowTiles)
    int32_t tile_tokens;    // tile kernel: tokens per tile
    int32_t k_tiles;        // dense split tile grid: the first k_tiles tiles of a row move K, the rest V
    int32_t layer_wgs;      // grid of the rows' own tiles: workgroups per layer
    int32_t b0, nb;         // pack/unpack grids cover rows [b0, b0 + nb) (set by the launcher)
    int64_t T;              // sum of counts
};

// Workgroups of the rows [b0, b0 + nb) of one layer in a grid that holds
// only the tiles each row has: row b0 + i owns workgroups [pre[i], pre[i + 1])
// of the layer, head after head, each head's K tiles first and then its V
// runs.
struct RowTiles {
    int32_t pre[kMaxRows + 1];
};

// Geometry of one launch on a paged pool: key [L, NB, H, D/8, P, 8], value
// [L, NB, H, P, D]; row b's token s is in block table[b*table_stride + s/P]
// at slot s%P.  Block ids outside [0, NB) are skipped by the kernels.
struct PagedGeometry {
    uint4 *k;
    uint4 *v;
    uint4 *stage;
    const int32_t *table;   // device memory, int32[B * table_stride]
    int32_t table_stride;
    int32_t NB, H, C, P;    // physical blocks, heads, D/8, tokens per block
    int32_t p_shift;        // log2(P) when P is a power of two, else -1
    int32_t B, l0, nl;
    int32_t tiles_per_row, tile_tokens;
    int32_t k_tiles;        // split tile kernel: the first k_tiles tiles of a row move K, the rest V
    int32_t b0, nb;         // grids cover rows [b0, b0 + nb) (set by the launcher)
    int64_t T;              // sum of counts
};

// ---- errors (api.hip) ----
int set_error(int status, const char *fmt, ...);
int hip_fail(hipError_t e, const char *what);

// ---- validation helpers (api.hip) ----
int check_layout(const kv_layout *lay);
int check_device_buffer(const void *p, int64_t bytes, const char *name);
int check_pinned_host(const void *p, int64_t bytes, const char *name);
bool overlaps(const void *a, int64_t an, const void *b, int64_t bn);
// True when the environment asks for kernel dispatches one at a time
// (AMD_SERIALIZE_KERNEL, or rocprofv3's counter collection): a copy that a
// stream waits on through a memory value then never starts.
bool serialized_dispatch();
// Validates per-row ranges and fills `rt`; returns KV_OK or an error.  `count`
// NULL means one token per row.
int build_rows(const kv_layout &lay, const int32_t *start, const int32_t *count, RowTable *rt,
               int32_t *max_count);
int check_layers(const kv_layout &lay, int32_t layer_begin, int32_t layer_count);
int64_t packed_bytes(const kv_layout &lay, int32_t nl, int64_t tokens);
// Per-row ranges of a prompt-layer call: [tok_begin, tok_begin+tok_count)
// clipped to [0, row_len_b) (row_len NULL: no clip).
int prompt_rows(const kv_layout &lay, int32_t tok_begin, int32_t tok_count,
                const int32_t *row_len, int32_t *start, int32_t *count);

// Validated pack/unpack of a whole call (used by the public entry points and
// the engines).  Buffers are assumed checked by the caller.
// Heads [h0, h0 + nh) only when nh >= 0 (default: all heads).
int enqueue_copy(bool pack, const kv_layout &lay, const void *k, const void *v, int32_t l0,
                 int32_t nl, const RowTable &rt, int32_t max_count, void *stage, hipStream_t s,
                 int32_t h0 = 0, int32_t nh = -1);

// n consecutive decode steps of a ring: step t of row b at pos0[b] + t, its
// slot at stage + t * slot_bytes.  All L layers and H heads.
int enqueue_steps(bool pack, const kv_layout &lay, const void *k, const void *v,
                  const int32_t *pos0, int32_t n, void *stage, int64_t slot_bytes,
                  hipStream_t s);

// ---- kernels (kernels.hip) ----
// Launches the pack (or unpack) kernels for one call; returns KV_OK or KV_EHIP.
int launch_copy(bool pack, const Geometry &g, const RowTable &rt, int32_t max_count,
                hipStream_t s);

// n decode steps at once: step t of row b at position rt.start[b] + t, its
// one-token-per-row packed block at g.stage + t * slot_vecs (16-byte vectors).
// Uses g.k, g.v, g.stage, B, H, C, Smax, l0, nl.
int launch_steps(bool pack, const Geometry &g, const RowTable &rt, int32_t n,
                 int64_t slot_vecs, hipStream_t s);

// Paged counterpart of launch_copy.
int launch_paged_copy(bool pack, const PagedGeometry &g, const RowTable &rt, int32_t max_count,
                      hipStream_t s);

// Copies `bytes` (a multiple of 16) between a device buffer and pinned host
// memory with the link-copy kernel, from `blocks` workgroups (0: the
// default for the direction, kLinkBlocksToHost for device->host).
// `dst`/`src` are device-visible addresses (see host_device_address).
constexpr int32_t kLinkBlocksToHost = 8;
constexpr int32_t kLinkBlocksMax = 1024;
int launch_link_copy(void *dst, const void *src, int64_t bytes, bool to_host, hipStream_t s,
                     int32_t blocks = 0);

// Device-visible address of pinned host memory [host, host+bytes); returns
// KV_OK or KV_EINVAL.
int host_device_address(const void *host, int64_t bytes, void **dev);

// ---- device->host copies on a chosen DMA engine (engine_copy.hip) ----
struct EngineCopier;
// A copier on one of the DMA engines that write host memory at full speed,
// for the current device; KV_EINVAL when the device or runtime cannot.
int engine_copier_create(EngineCopier **out);
// Waits until every copy is submitted and every stream is past it.  Returns
// KV_EHIP (with kv_last_error set) when a copy was still running after ten
// seconds: its signals are then left allocated rather than freed under the
// engine.
int engine_copier_destroy(EngineCopier *c);
// Pin the copier to one of the four fast engines (0-3), or let it take, at
// each copy, one the runtime reports idle (-1, the default).
void engine_copier_pin(EngineCopier *c, int32_t engine);
// Enqueue on `s` a copy of `bytes` from device memory to pinned host memory
// that starts once everything enqueued on `s` so far has run, and that later
// work on `s` waits for.
int engine_copy_to_host(EngineCopier *c, void *dst_host, const void *src_dev, int64_t bytes,
                        hipStream_t s);

// ---- profiling (api.hip) ----
// Two events that a timed launch binds to its dispatch (hipExtLaunchKernel):
// they then hold the kernel's own begin and end timestamps.  Both null when
// profiling is off.
struct LaunchTimer {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchTimer profile_take();
// Record the launch timed by `t` (moving `bytes`), or give its events back
// when the launch failed.  No-op for a null timer.
void profile_commit(const LaunchTimer &t, const char *name, int64_t bytes, bool launched);

}  // namespace kvs
