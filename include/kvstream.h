/*
 * kvstream.h -- C ABI of the MI355X KV-cache buffered-copy library.
 *
 * The library moves slices of a preallocated, maximum-length, strided K/V
 * cache into a contiguous HBM staging buffer and back ("buffered copies"),
 * and streams staged blocks to and from pinned host memory, layer by layer,
 * for microbatch swapping, prompt-cache streaming and replication.
 *
 * Sources (cited by page title and section):
 *   [DV]  "DejaVu: KV-Cache Streaming for Fast, Fault-Tolerant Generative LLM
 *         Serving" (papercache.org summary), section "Method details":
 *         DejaVuLib implementation (Fig 6), Buffered copies (Fig 7a),
 *         Layer-by-layer prompt cache streaming (Fig 7b), Token computation
 *         and streaming parallelization (Fig 7c), DejaVuLib primitives
 *         (Table 1), Fast prompt KV transfer, Microbatch swapping workflow
 *         (Fig 9), Failure detection and recovery (Fig 10).
 *   [KV]  lsln.cn article on decode-only inference, section "KV Cache
 *         capacity": KV bytes = 2 x B x S x H x D x P x N.
 *
 * ---------------------------------------------------------------------------
 * Cache layouts (16-bit elements, fp16 or bf16, moved as raw bits):
 *   key   K[L][B][H][D/8][Smax][8]   element (l,b,h,s,d) at
 *         ((((l*B + b)*H + h)*(D/8) + d/8)*Smax + s)*8 + d%8
 *   value V[L][B][H][Smax][D]        element (l,b,h,s,d) at
 *         (((l*B + b)*H + h)*Smax + s)*D + d
 * Both are preallocated at the maximum sequence length [DV, Fig 6].  In the
 * key layout a token's D values of one head are D/8 separate 16-byte vectors
 * Smax*16 bytes apart, which is why a decode step touches a small,
 * non-contiguous part of the key cache [DV, Fig 6].
 *
 * Packed (staging) format -- the layout of every staging buffer and host
 * image this library writes or reads.  For a layer range [l0, l0+nl) and
 * per-row token ranges [start_b, start_b + count_b), let T = sum_b count_b
 * and rowoff_b = sum_{b'<b} count_b'.  Element (l, kv, b, h, t, d), kv = 0
 * for K and 1 for V, t in [0, count_b), comes from cache position
 * s = start_b + t and sits at staging element
 *     ((l - l0)*2 + kv)*(H*T*D) + (H*rowoff_b + h*count_b + t)*D + d.
 * That is: layer-major; within a layer the K block then the V block; each
 * block [b][h][t][d] with d contiguous.  Its size is
 *     2 * nl * H * D * P * T bytes,
 * which for uniform rows (T = B*S) is the closed form 2 x B x S x H x D x P x N
 * of [KV].  The pages print no staged buffer; this order is the reading this
 * library fixes.
 *
 * ---------------------------------------------------------------------------
 * Conventions for every call:
 *   - The caller owns all memory: caches, staging banks, pinned host buffers,
 *     streams and events.  The library allocates only its handle structs
 *     and the hipEvents inside them; it never allocates data memory.
 *   - Device pointers (caches, staging, banks) must be device memory and
 *     16-byte aligned; host images must be pinned host memory (e.g. from
 *     hipHostMalloc).  Staging must not overlap either cache.
 *   - Per-row arrays (start, count, pos, row_len) are host int32[B], read
 *     during the call only.  B <= KV_MAX_ROWS.
 *   - Every call validates its arguments synchronously.  A call rejected by
 *     these checks returns a negative kv_status, enqueues nothing, and sets
 *     the thread-local kv_last_error().  A call that enqueues several
 *     launches or copies and then meets a HIP runtime failure (KV_EHIP)
 *     leaves the part before the failure enqueued; destroy the handle then.
 *   - On success it returns once the work is enqueued (asynchronous).  Buffers
 *     must stay alive until the stream (or the `done` event) passes them.
 *   - No C++ exception crosses this ABI.  Device faults surface at the
 *     caller's next synchronisation.
 *   - Handles are not thread-safe; distinct handles may be used concurrently.
 */
#ifndef KVSTREAM_H
#define KVSTREAM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KV_VERSION 1
#define KV_MAX_ROWS 256          /* rows per call: per-row ranges travel in kernel arguments */
#define KV_MAX_HEAD_DIM 1024

typedef enum kv_status {
    KV_OK = 0,
    KV_EINVAL = -1,   /* bad argument: dims, dtype, NULL, misaligned, not device / not pinned, overlap */
    KV_ERANGE = -2,   /* layer outside [0,L) or a token range outside [0,Smax) */
    KV_ESIZE = -3,    /* a destination or bank smaller than required */
    KV_EHIP = -4,     /* a HIP runtime call failed; detail in kv_last_error() */
    KV_EBUSY = -5     /* handle state does not allow the call (e.g. restore before flush) */
} kv_status;

typedef enum kv_dtype { KV_F16 = 0, KV_BF16 = 1 } kv_dtype;

/* Cache-layout descriptor, filled by kv_layout_init [DV, Fig 6]. */
typedef struct kv_layout {
    int32_t L, B, H, D, Smax, dtype;
    int32_t elem_bytes;        /* P = 2 */
    int32_t vec_elems;         /* x = 8 elements per 16-byte key vector */
    int64_t k_strides[6];      /* element strides of K [L,B,H,D/8,Smax,8] */
    int64_t v_strides[5];      /* element strides of V [L,B,H,Smax,D] */
    int64_t k_bytes, v_bytes;  /* bytes of each cache tensor */
    uint32_t magic;            /* set by kv_layout_init; checked by every call */
    uint32_t reserved;
} kv_layout;

/* Layout descriptor of a cache preallocated at the maximum sequence length
 * [DV, Fig 6].  Pure host call.  Requires L, B, H, D, Smax > 0, D % 8 == 0,
 * D <= KV_MAX_HEAD_DIM, B <= KV_MAX_ROWS, dtype a kv_dtype, byte sizes
 * that fit int64, and B * Smax and Smax * D/8 below 2^31.  Returns KV_OK or
 * KV_EINVAL. */
int kv_layout_init(kv_layout *out, int32_t L, int32_t B, int32_t H, int32_t D,
                   int32_t Smax, int32_t dtype);

/* Bytes of one packed block over `layer_count` layers:
 * 2 * layer_count * H * D * P * sum_b count_b -- the closed form
 * 2 x B x S x H x D x P x N of [KV] for uniform rows.  `count` NULL means
 * every row moves `uniform_count` tokens.  Pure host call; returns the byte
 * count, or a negative kv_status on bad arguments. */
int64_t kv_pack_bytes(const kv_layout *lay, int32_t layer_count,
                      const int32_t *count, int32_t uniform_count);

/* Gather ("buffered copy", [DV, Buffered copies, Fig 7a]; gather in Table 1):
 * copy, for layers [layer_begin, layer_begin+layer_count) and each row b,
 * tokens [start_b, start_b + count_b) of both caches into `staging` in the
 * packed format.  `count` NULL means one token per row (a decode step,
 * [DV, Fig 6]).  count_b = 0 skips a row.  Requires start_b >= 0 and
 * start_b + count_b <= Smax (else KV_ERANGE), staging_bytes >=
 * kv_pack_bytes (else KV_ESIZE).  Reads the caches, writes exactly
 * kv_pack_bytes bytes of staging, on stream `s`. */
int kv_pack_tokens(const kv_layout *lay, const void *k, const void *v,
                   int32_t layer_begin, int32_t layer_count,
                   const int32_t *start, const int32_t *count,
                   void *staging, int64_t staging_bytes, hipStream_t s);

/* Scatter (the destination side of a buffered copy, [DV, Fig 7a]; scatter in
 * Table 1): the exact inverse of kv_pack_tokens.  Writes each packed element
 * of `staging` to its cache position and writes no other cache element.
 * Same arguments, checks and errors as kv_pack_tokens. */
int kv_unpack_tokens(const kv_layout *lay, void *k, void *v,
                     int32_t layer_begin, int32_t layer_count,
                     const int32_t *start, const int32_t *count,
                     const void *staging, int64_t staging_bytes, hipStream_t s);

/* One prompt layer ([DV, Layer-by-layer prompt cache streaming, Fig 7b]):
 * layer `layer`, every row, tokens [tok_begin, tok_begin + tok_count) clipped
 * to [0, row_len_b) (`row_len` NULL: no clip).  Same packed format as
 * kv_pack_tokens with layer_count = 1.  A chunked prompt (fixed-size token
 * chunks) is a sequence of calls with advancing tok_begin.  Requires
 * 0 <= tok_begin, tok_count >= 0, tok_begin + tok_count <= Smax and
 * 0 <= row_len_b <= Smax (else KV_ERANGE). */
int kv_pack_prompt_layer(const kv_layout *lay, const void *k, const void *v,
                         int32_t layer, int32_t tok_begin, int32_t tok_count,
                         const int32_t *row_len, void *staging, int64_t staging_bytes,
                         hipStream_t s);

/* Inverse of kv_pack_prompt_layer (loading a streamed prompt layer into the
 * token-side cache, [DV, Fast prompt KV transfer]). */
int kv_unpack_prompt_layer(const kv_layout *lay, void *k, void *v,
                           int32_t layer, int32_t tok_begin, int32_t tok_count,
                           const int32_t *row_len, const void *staging, int64_t staging_bytes,
                           hipStream_t s);

/* ---------------------------------------------------------------------------
 * Paged pools.  The pages name vLLM's paged KV memory and Mooncake's
 * chunk-organised KV ([DV, Related work]; [KV, KV Cache transfer: Mooncake,
 * KV Cache Pool]) without giving a layout; the one taken here is the
 * contiguous layout with (row, Smax)
 * replaced by (physical block, block_tokens P): key
 * [L, blocks, H, D/8, P, 8], value [L, blocks, H, P, D].  A row's tokens
 * live in the blocks its table names: token s of row b is slot s % P of
 * block table[b * table_stride + s / P].  Packing from a pool writes the same
 * packed format as kv_pack_tokens, so everything downstream (rings, swap,
 * streaming) is shared.
 */
typedef struct kv_paged {
    int32_t L, blocks, H, D, block_tokens, dtype;
    int32_t elem_bytes;        /* P = 2 */
    int32_t vec_elems;         /* 8 elements per 16-byte key vector */
    int64_t k_strides[6];      /* element strides of K [L,blocks,H,D/8,block_tokens,8] */
    int64_t v_strides[5];      /* element strides of V [L,blocks,H,block_tokens,D] */
    int64_t k_bytes, v_bytes;
    uint32_t magic;
    uint32_t reserved;
} kv_paged;

/* Pool descriptor.  Requires all dims > 0, D % 8 == 0, D <= KV_MAX_HEAD_DIM,
 * dtype a kv_dtype, byte sizes that fit int64 and block_tokens * D/8 below
 * 2^31 (else KV_EINVAL).  Pure host call. */
int kv_paged_init(kv_paged *out, int32_t L, int32_t blocks, int32_t H, int32_t D,
                  int32_t block_tokens, int32_t dtype);

/* Bytes a pack of B rows over `layer_count` layers moves:
 * 2 * layer_count * H * D * P * sum_b count_b (count NULL: one per row). */
int64_t kv_paged_pack_bytes(const kv_paged *pg, int32_t layer_count, int32_t B,
                            const int32_t *count);

/* Gather from a pool: rows b < B (B <= KV_MAX_ROWS), tokens
 * [start_b, start_b + count_b) (count NULL: one per row), layers
 * [layer_begin, layer_begin + layer_count), into `staging` in the packed
 * format of kv_pack_tokens.  `table`: device memory, int32[B * table_stride],
 * caller-owned.  Requires start_b + count_b <= table_stride * block_tokens
 * (else KV_ERANGE) and the usual buffer checks.  Block ids are read on the
 * GPU: a token whose id lies outside [0, blocks) is skipped (its packed
 * words are not written); kv_paged_check_table validates a host copy. */
int kv_pack_paged(const kv_paged *pg, const void *k, const void *v, int32_t layer_begin,
                  int32_t layer_count, int32_t B, const int32_t *table, int32_t table_stride,
                  const int32_t *start, const int32_t *count, void *staging,
                  int64_t staging_bytes, hipStream_t s);

/* Scatter into a pool: the inverse of kv_pack_paged; writes exactly the
 * selected slots (tokens of skipped blocks are not written).  The selected
 * tokens must map to distinct slots. */
int kv_unpack_paged(const kv_paged *pg, void *k, void *v, int32_t layer_begin,
                    int32_t layer_count, int32_t B, const int32_t *table, int32_t table_stride,
                    const int32_t *start, const int32_t *count, const void *staging,
                    int64_t staging_bytes, hipStream_t s);

/* Host check of a block table (host memory, same shape): KV_ERANGE if a
 * selected token's block id lies outside [0, blocks), else KV_OK. */
int kv_paged_check_table(const kv_paged *pg, int32_t B, const int32_t *table,
                         int32_t table_stride, const int32_t *start, const int32_t *count);

/* ---------------------------------------------------------------------------
 * stream_out / stream_in between partitions ([DV, DejaVuLib primitives,
 * Table 1]; Fast prompt KV transfer): the source and destination workers may
 * split the model differently (pipeline depth: layer ranges; tensor
 * parallelism: head ranges; batch size: request ranges).  A worker's cache
 * holds one partition, stored at local indices from 0.  The piece a source
 * sends a destination is the intersection of the two partitions, packed in
 * the order of kv_pack_tokens over the shared layers, rows and heads (global
 * order); the source splits its cache into one piece per destination, the
 * destination merges the pieces of all its sources.
 */
typedef struct kv_part {
    int32_t layer0, layers;  /* global layers [layer0, layer0 + layers) = local layers [0, layers) */
    int32_t head0, heads;    /* global heads [head0, head0 + heads) = local heads [0, heads) */
    int32_t row0, rows;      /* global requests [row0, row0 + rows) = local rows [0, rows) */
} kv_part;

/* Bytes of the piece `self` and `peer` share: 2 * (shared layers) *
 * (shared heads) * D * P * (sum of count_b over the shared rows), count
 * being int32[self->rows] (NULL: one token per row).  0 when they do not
 * meet.  `lay` must describe self's cache (L = layers, B = rows, H = heads),
 * else KV_EINVAL.  Pure host call; negative kv_status on error. */
int64_t kv_stream_bytes(const kv_layout *lay, const kv_part *self, const kv_part *peer,
                        const int32_t *count);

/* stream_out: pack the piece of src's cache (k, v; layout `lay`) that `dst`
 * holds into `staging` (device memory).  start/count: int32[src->rows], the
 * token range [start_b, start_b + count_b) of each local row (count NULL:
 * one token per row).  Every row's range is checked (KV_ERANGE); only the
 * rows dst holds are moved.  Errors as kv_pack_tokens; an empty intersection
 * enqueues nothing (staging may then be NULL). */
int kv_stream_out(const kv_layout *lay, const kv_part *src, const void *k, const void *v,
                  const kv_part *dst, const int32_t *start, const int32_t *count,
                  void *staging, int64_t staging_bytes, hipStream_t s);

/* stream_in: merge the piece `src` sent (staging, as kv_stream_out wrote
 * it) into dst's cache (k, v; layout `lay`).  start/count: int32[dst->rows]
 * in dst's local rows; the shared rows' counts must equal the source's
 * (staging_bytes must cover the piece as these counts size it, else
 * KV_ESIZE).  Writes exactly the piece's elements. */
int kv_stream_in(const kv_layout *lay, const kv_part *dst, void *k, void *v,
                 const kv_part *src, const int32_t *start, const int32_t *count,
                 const void *staging, int64_t staging_bytes, hipStream_t s);

/* Move a packed block from one device buffer to another on the same GPU
 * ([DV, Fast prompt KV transfer]: the prompt worker's packed KV goes to the
 * token worker's buffer; Table 1: stream_out's pieces reach the workers
 * that merge them).  When both workers share a GPU the move is a plain
 * device-to-device copy: `bytes` (a multiple of 16) from `src` to `dst`, both
 * 16-byte aligned device memory inside one allocation each, not
 * overlapping (else KV_EINVAL; negative bytes KV_ESIZE; 0 bytes enqueues
 * nothing).  Enqueued on `s`; every byte is read once and written once with
 * the non-temporal hint, one 16-byte vector per thread -- the fastest plain
 * copy measured on MI355X, so its rate is also the practical HBM ceiling
 * the pack and unpack kernels are compared with. */
int kv_copy_packed(void *dst, const void *src, int64_t bytes, hipStream_t s);

/* ---------------------------------------------------------------------------
 * Swap engine: staged, layer-pipelined transfers between a cache and pinned
 * host memory ([DV, Microbatch swapping workflow, Fig 9]; flush/fetch in
 * Table 1, local leg).  Two caller-owned device banks alternate: the pack of
 * chunk i+1 overlaps the device-to-host copy of chunk i; a bank is reused
 * only after the copy that read it (or the unpack that read it) completes,
 * enforced with events on the GPU, never by host waits.  Chunks are whole
 * layers when a layer fits a bank (several layers per chunk when they fit),
 * otherwise row ranges of one layer (the K part and the V part of a row
 * range are then two copies).  A single (layer, row) block must fit a bank
 * (else KV_ESIZE).  Copies run on the caller's `copy` stream.
 */
typedef struct kv_swap kv_swap;

/* How a bank reaches pinned host memory (flush/fetch, local leg, Table 1).
 *   KV_XFER_AUTO    -- device->host by the link-copy kernel, host->device by
 *                      hipMemcpyAsync (DMA).  The default.
 *   KV_XFER_KERNEL  -- both directions by the library's link-copy kernel on
 *                      the copy stream: the host buffer is mapped into the
 *                      GPU's address space and the GPU's load/store units move
 *                      16-byte vectors across the host link.
 *   KV_XFER_RUNTIME -- both directions by hipMemcpyAsync with the ordinary
 *                      host<->device kinds (the runtime picks the engine).
 *   KV_XFER_DMA     -- both directions by hipMemcpyAsync between the bank and
 *                      the host buffer's device-visible address with
 *                      hipMemcpyDeviceToDeviceNoCU, which asks the runtime
 *                      for the DMA engines (it may still run a copy as its
 *                      own copy kernel, and it picks the engine).
 *   KV_XFER_DMA_OUT -- device->host as KV_XFER_DMA, host->device as
 *                      KV_XFER_RUNTIME.
 *   KV_XFER_ENGINE  -- device->host on a named DMA engine through the HSA
 *                      runtime: one of engines 0-3 (the ones that write host
 *                      memory at full speed), for each copy one the runtime
 *                      reports idle.  The copy is submitted when the call is
 *                      made, gated on a signal that the copy stream clears
 *                      once it reaches the copy; the stream then waits on the
 *                      copy's completion signal.  host->device as
 *                      KV_XFER_RUNTIME.  Needs stream memory waits
 *                      (KV_EINVAL at create time otherwise).  Destroying the
 *                      handle waits until its copies are done.  These copies
 *                      cannot be captured into a graph, and a profiler that
 *                      runs one dispatch at a time (hardware counter
 *                      collection) cannot order them: create then refuses
 *                      the transport (collect counters with another one).
 * Measured on MI355X: DMA copies in both directions at once run at full
 * duplex when one direction moves large (bank-sized) chunks, but fall to
 * about one direction's rate when both move small dependent chunks (one
 * layer each), and device->host DMA copies can drop to a fraction of the
 * link for the rest of the process; GPU-initiated reads of host memory keep
 * the two directions from running at once.  GPU-initiated writes (the
 * link-copy kernel) and DMA reads overlap in every pattern -- hence AUTO.
 * All transports produce identical bytes. */
typedef enum kv_transport {
    KV_XFER_AUTO = 0,
    KV_XFER_KERNEL = 1,
    KV_XFER_RUNTIME = 2,
    KV_XFER_DMA = 3,
    KV_XFER_DMA_OUT = 4,
    KV_XFER_ENGINE = 5
} kv_transport;

/* bank0/bank1: caller-owned device banks of bank_bytes each; `copy`: the
 * stream that carries the transfers; `transport`: a kv_transport.
 * Returns KV_EINVAL for KV_XFER_ENGINE when kernel dispatches are
 * serialised (AMD_SERIALIZE_KERNEL set, or ROCPROF_COUNTER_COLLECTION as
 * rocprofv3 sets it for hardware counters): the stream's wait on a DMA
 * copy would then never end. */
int kv_swap_create(kv_swap **out, const kv_layout *lay, void *bank0, void *bank1,
                   int64_t bank_bytes, hipStream_t copy, int32_t transport);
/* Waits until the handle's DMA copies are done; KV_EHIP if one was still
 * running after ten seconds (its signals are then left allocated). */
int kv_swap_destroy(kv_swap *e);

/* Per-handle settings of the link leg, for swap engines and rings; they
 * apply to copies enqueued after the call.
 *   KV_OPT_DMA_ENGINE  -- KV_XFER_ENGINE handles only: -1 (the default)
 *                         takes, at each copy, one of the four fast engines
 *                         the runtime reports idle; 0..3 always uses that
 *                         engine.  On MI355X the engines differ in what
 *                         they leave to co-running kernels: with the
 *                         100K-context step's prompt streaming on engine 0
 *                         its pack kernels kept 0.64 of HBM peak, on
 *                         engines 2 or 3 0.50-0.53 (on engine 1 the step
 *                         ran 25% slower).
 *   KV_OPT_LINK_BLOCKS -- workgroups of the link-copy kernel's
 *                         device->host copies (KV_XFER_AUTO, KV_XFER_KERNEL);
 *                         0 (the default) means 8, at most 1024.  More
 *                         workgroups move the copy faster when it shares
 *                         the link with DMA copies; fewer leave co-running
 *                         kernels more of HBM.
 * KV_EINVAL for an unknown option, a value out of range, or an engine
 * setting on a handle of another transport. */
typedef enum kv_option {
    KV_OPT_DMA_ENGINE = 1,
    KV_OPT_LINK_BLOCKS = 2
} kv_option;
int kv_swap_set_option(kv_swap *e, int32_t option, int64_t value);

/* Swap-out: pack the selected region (kernels on `compute`, so they see the
 * cache as of the call) and copy it to `host` (pinned) on the copy stream.
 * The host bytes are identical to one kv_pack_tokens over the whole layer
 * range.  `done` (nullable) is recorded on the copy stream after the last
 * copy: the host image is valid once it completes.  Later work on `compute`
 * may overwrite the cache as soon as it runs: the packs precede it there. */
int kv_swap_out(kv_swap *e, const void *k, const void *v,
                int32_t layer_begin, int32_t layer_count,
                const int32_t *start, const int32_t *count,
                void *host, int64_t host_bytes, hipStream_t compute, hipEvent_t done);

/* Swap-in: copy `host` (pinned, packed format) to the banks on the copy
 * stream and unpack it into the caches on `compute`.  The copies wait only for
 * the bank they overwrite to be free; the host image must already be complete
 * when they run -- order its producer before the call on the copy stream (for
 * instance hipStreamWaitEvent(copy, done of the swap-out that wrote it)) or on
 * the host.  `done` (nullable) is recorded on `compute` after the last unpack;
 * later work on `compute` sees the restored cache. */
int kv_swap_in(kv_swap *e, void *k, void *v,
               int32_t layer_begin, int32_t layer_count,
               const int32_t *start, const int32_t *count,
               const void *host, int64_t host_bytes, hipStream_t compute, hipEvent_t done);

/* Swap-out that allocates nothing, for callers that cannot allocate memory:
 * code under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same host bytes as kv_swap_out over the same region, without a
 * handle or banks: each chunk of the region (whole layers, or row groups of
 * one layer, that fit KV_NOALLOC_SCRATCH_BYTES) is packed on `s` into a
 * static device buffer of the library and then copied to `host` (pinned) by
 * the link-copy kernel on `s`, chunk after chunk in stream order.  The host
 * image is valid once `s` has passed the call.  The library holds that
 * buffer (KV_NOALLOC_SCRATCH_BYTES) on every GPU it runs on until the process
 * ends; the call itself calls no hipMalloc, hipFree or other allocating
 * routine.  All calls on one GPU share the buffer and nothing in it needs to
 * start at any value: calls on one stream follow one another, but calls that
 * overlap in time on one GPU (other streams, other threads) race on it and
 * must be ordered by the caller.  KV_ESIZE when one layer of one row needs
 * more than KV_NOALLOC_SCRATCH_BYTES; other errors as kv_swap_out. */
#define KV_NOALLOC_SCRATCH_BYTES (128ll << 20)
int kv_swap_out_noalloc(const kv_layout *lay, const void *k, const void *v,
                        int32_t layer_begin, int32_t layer_count,
                        const int32_t *start, const int32_t *count,
                        void *host, int64_t host_bytes, hipStream_t s);

/* Layer-by-layer prompt streaming ([DV, Fig 7b; Fast prompt KV transfer]):
 * pack one prompt layer (as kv_pack_prompt_layer) into the next bank on
 * `compute` and copy it to `host` on the copy stream, so that streaming layer
 * l overlaps the computation of layer l+1.  `done` as in kv_swap_out. */
int kv_stream_prompt_layer(kv_swap *e, const void *k, const void *v,
                           int32_t layer, int32_t tok_begin, int32_t tok_count,
                           const int32_t *row_len, void *host, int64_t host_bytes,
                           hipStream_t compute, hipEvent_t done);

/* Host-only view of the swap engine's chunking, for inspection and tests.
 * Fills up to `max_chunks` entries and returns the number of chunks (may
 * exceed max_chunks), or a negative kv_status. */
typedef struct kv_chunk {
    int32_t layer_begin, layer_count;  /* layers of this chunk */
    int32_t row_begin, row_end;        /* rows [row_begin, row_end) */
    int64_t staged_bytes;              /* bytes packed into the bank */
    int32_t pieces;                    /* contiguous copies: 1 or 2 */
    int32_t reserved;
    int64_t host_off[2], bank_off[2], bytes[2];
} kv_chunk;

int64_t kv_swap_plan(const kv_layout *lay, int32_t layer_begin, int32_t layer_count,
                     const int32_t *start, const int32_t *count, int64_t bank_bytes,
                     kv_chunk *out, int64_t max_chunks);

/* ---------------------------------------------------------------------------
 * Staging ring for decode steps ([DV, Buffered copies, Fig 7a; Token
 * computation and streaming parallelization, Fig 7c]).  Step j (0-based)
 * packs one token per row, at pos[b], of all L layers into slot j mod R of
 * bank (j / R) mod 2.  When a bank's R slots are filled the bank is copied
 * to host offset j0 * slot_bytes (j0 = its first unflushed step) in one
 * contiguous copy on the copy stream; the host image therefore holds the
 * slots in step order.  A push that reuses a bank waits, on the GPU, for
 * that bank's previous copy.  slot_bytes = 2 * L * H * D * P * B.
 */
typedef struct kv_ring kv_ring;

/* bank_bytes must hold R slots; host_bytes bounds the steps that can be
 * pushed (steps * slot_bytes); `transport` as for kv_swap_create. */
int kv_ring_create(kv_ring **out, const kv_layout *lay, int32_t R,
                   void *bank0, void *bank1, int64_t bank_bytes,
                   void *host, int64_t host_bytes, hipStream_t copy, int32_t transport);
/* As kv_swap_destroy. */
int kv_ring_destroy(kv_ring *r);
/* As kv_swap_set_option. */
int kv_ring_set_option(kv_ring *r, int32_t option, int64_t value);

/* One decode step: pos is int32[B], every pos_b in [0, Smax).  The step is
 * packed from (k, v) on `compute` at this call, or, in gather-at-flush mode,
 * when its bank fills or kv_ring_flush runs (see kv_ring_set_gather). */
int kv_ring_push(kv_ring *r, const void *k, const void *v, const int32_t *pos,
                 hipStream_t compute);

/* When a ring reads the cache.  KV_RING_GATHER_EACH_STEP (the default): every
 * push packs its step at once.  KV_RING_GATHER_AT_FLUSH: a push only records
 * the step; the steps of a bank are packed together just before the bank is
 * copied out (on the compute stream of the push or flush that triggers it),
 * so the pushed positions must keep their contents until then -- true of a
 * decode loop, where each step writes a new position.  Steps whose positions
 * advance by one on every row (and share the caches) are packed in one pass
 * that reads whole cache lines; a single-step pack reads one 16-byte key
 * vector per line.  The bytes produced are identical.  Changing the mode
 * requires every pushed step flushed (else KV_EBUSY). */
enum kv_ring_gather {
    KV_RING_GATHER_EACH_STEP = 0,
    KV_RING_GATHER_AT_FLUSH = 1
};
int kv_ring_set_gather(kv_ring *r, int32_t mode);

/* Copy the filled but unflushed slots (a final partial bank) to the host.
 * `done` (nullable) is recorded on the copy stream after every copy so far:
 * the whole host image is valid once it completes. */
int kv_ring_flush(kv_ring *r, hipStream_t compute, hipEvent_t done);

/* Restore ([DV, Failure detection and recovery, Fig 10], data leg): copy the
 * host image back through the banks and unpack every step into (k, v) in
 * ascending step order (a later step wins where two name the same position;
 * runs of steps whose positions advance by one are unpacked in one pass).
 * Requires every pushed step flushed (else KV_EBUSY).  The copies follow the
 * ring's own flushes on the copy stream.  `done` (nullable) is recorded on
 * `compute` after the last unpack. */
int kv_ring_restore(kv_ring *r, void *k, void *v, hipStream_t compute, hipEvent_t done);

/* Restore only steps [0, n) (n <= steps flushed so far; else KV_ERANGE), as
 * after a failure when only the replicated prefix survives.  The ring then
 * continues from step n: later steps are dropped, and the next push is step
 * n (its slot overwrites the host image from there on). */
int kv_ring_restore_steps(kv_ring *r, void *k, void *v, int64_t n, hipStream_t compute,
                          hipEvent_t done);

/* Steps pushed so far, or a negative kv_status. */
int64_t kv_ring_steps(const kv_ring *r);

/* Steps whose flush copy to the host has completed, so that the host image
 * (the replica) holds steps [0, n): a non-blocking query of the ring's flush
 * events ([DV, Failure detection and recovery]: a worker acknowledges a
 * step once its update has reached the replica).  Negative kv_status on
 * error. */
int64_t kv_ring_durable_steps(kv_ring *r);

/* Forget all steps (the host image and banks are reused from step 0). */
int kv_ring_reset(kv_ring *r);

/* ---------------------------------------------------------------------------
 * Microbatch swapping on two device slots ([DV, Microbatch swapping workflow,
 * Fig 9]): N microbatches share two device caches; while microbatch x is
 * processed in one slot, x+1 is being swapped into the other.  Microbatch x's
 * KV lives on the host as its prompt image (packed tokens [0, prompt_len) of
 * every layer) plus the host image of rings[x], one slot per generated step:
 * the incremental swap-out of a step is a ring push (flushed at once when the
 * ring has R = 1), and a full swap-in is the prompt image followed by the
 * ring's steps.  The library orders everything with events: no host waits.
 */
typedef struct kv_mbswap kv_mbswap;

/* microbatches >= 2.  Slots: two full caches of `lay` (device, 16-byte
 * aligned).  `in`: the swap engine used for prompt swap-ins.  rings[x]: one
 * ring per microbatch.  prompt_host[x] / prompt_bytes[x]: pinned prompt
 * images, complete before kv_mbswap_start; prompt_len: int32[microbatches*B].
 * `swap_stream`: the stream that runs the swap-in unpacks, so that they
 * overlap the compute stream's work.  The overlap needs the compute stream,
 * `swap_stream` and the engine's and rings' copy streams on distinct hardware
 * queues: HIP maps streams onto GPU_MAX_HW_QUEUES queues per process, and
 * streams that share a queue run one after the other (a round then costs
 * compute plus transfer instead of the larger of the two).  The handle keeps
 * the pointers; the caller keeps the memory and the other handles alive. */
int kv_mbswap_create(kv_mbswap **out, const kv_layout *lay, int32_t microbatches,
                     void *slot0_k, void *slot0_v, void *slot1_k, void *slot1_v,
                     kv_swap *in, kv_ring *const *rings, void *const *prompt_host,
                     const int64_t *prompt_bytes, const int32_t *prompt_len,
                     hipStream_t swap_stream);
int kv_mbswap_destroy(kv_mbswap *m);

/* Swap microbatches 0 and 1 into slots 0 and 1; `compute` waits for slot 0. */
int kv_mbswap_start(kv_mbswap *m, hipStream_t compute);

/* The microbatch of the current round and the slot (k, v) that holds it. */
int kv_mbswap_current(const kv_mbswap *m, int32_t *x, void **k, void **v);

/* End the current round after the caller's step wrote one token per row at
 * pos[b] (int32[B]) on `compute`: swap out that update (rings[x] push), swap
 * microbatch (x+2) % N into the slot x leaves (after the push has read it),
 * advance to x+1 and make `compute` wait until x+1's slot is loaded. */
int kv_mbswap_round(kv_mbswap *m, const int32_t *pos, hipStream_t compute);

/* Appendix E of [DV]: with swapping the batch doubles from B to 2B, and
 * swapping pays iff 2 * N * t >= sum_{i=p}^{N+p} max(t, transf_i) with
 * transf_i = i * B * C / bw, the time to bring back the cache of B requests
 * holding i tokens.  N: tokens generated; t: seconds per decode step; p:
 * prompt length; C: KV bytes per token per request (2 * L * H * D * P for
 * the layers one GPU holds); bw: host-link bytes per second.  Writes both
 * sides and returns 1 if swapping pays, 0 if not, or a negative kv_status. */
int kv_swap_pays(int64_t N, double t, int64_t p, int64_t B, double C, double bw,
                 double *lhs, double *rhs);

/* ---------------------------------------------------------------------------
 * Acknowledgement log and restart point ([DV, Failure detection and
 * recovery, Fig 10]).  Worker x acknowledges (x, j, t) once the replica holds
 * microbatch j's KV up to and including step t.  After a failure the pipeline
 * restarts at one (microbatch j, step t).  Reading taken here: a
 * (microbatch, step) pair is replicated when every worker has acknowledged
 * it; steps run in (step, microbatch) order -- every microbatch's step t
 * before any microbatch's step t+1 -- and the restart point is the earliest
 * pair in that order that is not replicated, i.e. the smallest
 * (t_j + 1, j) with t_j = min over workers of the last step acknowledged for
 * microbatch j (-1 when none).  Host-only.
 */
typedef struct kv_acklog kv_acklog;

/* workers >= 1, microbatches >= 1 (else KV_EINVAL). */
int kv_acklog_create(kv_acklog **out, int32_t workers, int32_t microbatches);
int kv_acklog_destroy(kv_acklog *a);

/* Record (x, j, t); x in [0, workers), j in [0, microbatches), t >= 0 (else
 * KV_ERANGE).  Acks may arrive out of order: an ack for an earlier step than
 * one already recorded for (x, j) changes nothing. */
int kv_ack(kv_acklog *a, int32_t x, int32_t j, int64_t t);

/* The restart point (j, t) under the rule above. */
int kv_ack_restart_point(const kv_acklog *a, int32_t *j, int64_t *t);

/* ---------------------------------------------------------------------------
 * Live kernel timing.  Between kv_profile_begin and kv_profile_end every
 * kernel the library launches is timed by two hipEvents bound to its
 * dispatch (hipExtLaunchKernel's start and stop events), which take the
 * kernel's own begin and end timestamps: no extra packets on the stream,
 * and no launch latency in the interval.  kv_profile_end waits for those
 * events, fills up to `max` per-kernel entries and returns the number of
 * distinct kernels.  `bytes` is the algorithmic HBM traffic: payload read
 * plus payload written (for the link-copy kernels: bytes over the link).
 */
typedef struct kv_kernel_stat {
    char name[40];
    int64_t launches;
    double ms;          /* summed kernel duration */
    int64_t bytes;      /* summed algorithmic bytes (read + write) */
} kv_kernel_stat;

int kv_profile_begin(void);
int kv_profile_end(kv_kernel_stat *out, int32_t max);

/* The window kv_profile_end last closed, all streams together.  Kernels of
 * different streams run at the same time, so per-kernel durations do not
 * add up to the GPU time the path took; these are the unions of the
 * timed intervals instead: `hbm_busy_ms` is the time during which at
 * least one pack or unpack kernel ran and `hbm_bytes` the algorithmic bytes
 * those kernels moved (their rate together is hbm_bytes / hbm_busy_ms);
 * `link_*` the same for the link-copy kernels (bytes crossing the host
 * link).  `span_ms` runs from the first timed kernel's start to the last
 * one's end.  All zero when nothing was timed.  KV_EINVAL for a NULL `out`. */
typedef struct kv_profile_window {
    double span_ms;
    double hbm_busy_ms;
    int64_t hbm_bytes;
    int64_t hbm_launches;
    double link_busy_ms;
    int64_t link_bytes;
    int64_t link_launches;
} kv_profile_window;

int kv_profile_last_window(kv_profile_window *out);

/* Thread-local text of the last error; never NULL. */
const char *kv_last_error(void);
int kv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVSTREAM_H */
