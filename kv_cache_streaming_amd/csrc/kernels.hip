// Pack (gather) and unpack (scatter) kernels for gfx950.
//
// Pure data movement: 16-byte vectors (one key vector of 8 elements, or 8
// value elements) are the unit everywhere, loaded and stored as uint4 and
// never converted.  No MFMA, no arithmetic on the data.
//
// Buffered copies ("DejaVu: KV-Cache Streaming ...", Method details, Fig 7a)
// gather the many small non-contiguous cache pieces of a step into one
// contiguous buffer; these kernels are that gather and its inverse.
//
// Two kernels:
//  * copy_rows_small -- few tokens per row (decode steps, Fig 6): one thread
//    per (layer, row, head, key vector c); it moves K vector c and V vector c
//    of each of the row's tokens.  A wave covers 64/C heads, so every store
//    instruction writes contiguous runs of C*16 bytes of the packed buffer.
//  * copy_split -- many tokens per row (prompt layers, chunks, swaps):
//    256-thread workgroups, each either a K tile or a V run of one (layer,
//    row, head).  A V workgroup is a straight contiguous copy.  K's token
//    range is D/8 rows ("chunks") of 16-byte vectors, which the packed format
//    wants token-major; a K tile is loaded chunk-major (each wave reads
//    contiguous runs of one chunk row), transposed at 16-byte granularity
//    through LDS, and stored token-major (contiguous).  Unpack is the mirror
//    image.  The LDS index is XOR-swizzled so that both the chunk-major
//    writes and the token-major reads spread a wave's 16-byte accesses over
//    all banks.
#include "kvs_internal.h"

#include <algorithm>
#include <cstdlib>
#include <tuple>

namespace kvs {
namespace {

constexpr int kThreads = 256;
constexpr int kSmallMaxTokens = 8;        // rows with at most this many tokens use copy_rows_small


template <bool kPack>
__global__ __launch_bounds__(kThreads) void copy_rows_small(Geometry g, RowTable rt)
{
    // flat thread id over (layer, row, head, vector); the launcher keeps it < 2^31
    const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
    const uint32_t C = (uint32_t)g.C;
    uint32_t r = gid / C;
    const uint32_t c = gid - r * C;
    const uint32_t h = r % (uint32_t)g.nh;     // head within the moved range
    r /= (uint32_t)g.nh;
    const uint32_t b = (uint32_t)g.b0 + r % (uint32_t)g.nb;
    r /= (uint32_t)g.nb;
    if (r >= (uint32_t)g.nl)
        return;
    const int32_t li = (int32_t)r;
    const int32_t off = rt.off[b];
    const int32_t cnt = rt.off[b + 1] - off;
    if (cnt <= 0)
        return;
    const int32_t s0 = rt.start[b];
    const int64_t unit = ((int64_t)(g.l0 + li) * g.B + b) * g.H + g.h0 + h;
    uint4 *kc = g.k + (unit * C + c) * g.Smax + s0;       // token t: kc[t]
    uint4 *vc = g.v + (unit * g.Smax + s0) * C + c;       // token t: vc[t*C]
    const int64_t blk = (int64_t)g.nh * g.T * C;          // one (layer, K|V) block
    uint4 *ks = g.stage + 2 * (int64_t)li * blk + ((int64_t)g.nh * off + (int64_t)h * cnt) * C + c;
    uint4 *vs = ks + blk;                                 // token t: ks[t*C], vs[t*C]

    int32_t t = 0;
    for (; t + 2 <= cnt; t += 2) {
        if (kPack) {
            const uint4 a0 = kc[t], a1 = kc[t + 1];
            const uint4 d0 = vc[t * C], d1 = vc[(t + 1) * C];
            ks[t * C] = a0;
            ks[(t + 1) * C] = a1;
            vs[t * C] = d0;
            vs[(t + 1) * C] = d1;
        } else {
            const uint4 a0 = ks[t * C], a1 = ks[(t + 1) * C];
            const uint4 d0 = vs[t * C], d1 = vs[(t + 1) * C];
            kc[t] = a0;
            kc[t + 1] = a1;
            vc[t * C] = d0;
            vc[(t + 1) * C] = d1;
        }
    }
    if (t < cnt) {
        if (kPack) {
            const uint4 a = kc[t];
            const uint4 d = vc[t * C];
            ks[t * C] = a;
            vs[t * C] = d;
        } else {
            const uint4 a = ks[t * C];
            const uint4 d = vs[t * C];
            kc[t] = a;
            vc[t * C] = d;
        }
    }
}

// Several decode steps in one pass (a ring bank): step t of every row sits at
// position start_b + t, and its one-token-per-row packed block is at
// stage + t * slot_vecs.  One thread per (layer, row, head, key vector c)
// walks the n positions: its n key vectors are contiguous in the cache, so
// whole cache lines are read or written, where a single-step pack touches one
// 16-byte vector per line.
template <bool kPack>
__global__ __launch_bounds__(kThreads) void copy_steps(Geometry g, RowTable rt, int32_t n,
                                                       int64_t slot_vecs)
{
    const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
    const uint32_t C = (uint32_t)g.C;
    uint32_t r = gid / C;
    const uint32_t c = gid - r * C;
    const uint32_t h = r % (uint32_t)g.H;
    r /= (uint32_t)g.H;
    const uint32_t b = r % (uint32_t)g.B;
    r /= (uint32_t)g.B;
    if (r >= (uint32_t)g.nl)
        return;
    const int32_t li = (int32_t)r;
    const int32_t s0 = rt.start[b];
    const int64_t unit = ((int64_t)(g.l0 + li) * g.B + b) * g.H + h;
    uint4 *kc = g.k + (unit * C + c) * g.Smax + s0;        // step t: kc[t]
    uint4 *vc = g.v + (unit * g.Smax + s0) * C + c;        // step t: vc[t*C]
    const int64_t blk = (int64_t)g.H * g.B * C;            // one (layer, K|V) block of a slot
    uint4 *ks = g.stage + 2 * (int64_t)li * blk + ((int64_t)g.H * b + h) * C + c;
    uint4 *vs = ks + blk;                                  // step t: ks[t*slot_vecs], vs[...]
    int32_t t = 0;
    for (; t + 4 <= n; t += 4) {
        if (kPack) {
            const uint4 a0 = kc[t], a1 = kc[t + 1], a2 = kc[t + 2], a3 = kc[t + 3];
            const uint4 d0 = vc[t * C], d1 = vc[(t + 1) * C], d2 = vc[(t + 2) * C],
                        d3 = vc[(t + 3) * C];
            ks[t * slot_vecs] = a0;
            ks[(t + 1) * slot_vecs] = a1;
            ks[(t + 2) * slot_vecs] = a2;
            ks[(t + 3) * slot_vecs] = a3;
            vs[t * slot_vecs] = d0;
            vs[(t + 1) * slot_vecs] = d1;
            vs[(t + 2) * slot_vecs] = d2;
            vs[(t + 3) * slot_vecs] = d3;
        } else {
            const uint4 a0 = ks[t * slot_vecs], a1 = ks[(t + 1) * slot_vecs],
                        a2 = ks[(t + 2) * slot_vecs], a3 = ks[(t + 3) * slot_vecs];
            const uint4 d0 = vs[t * slot_vecs], d1 = vs[(t + 1) * slot_vecs],
                        d2 = vs[(t + 2) * slot_vecs], d3 = vs[(t + 3) * slot_vecs];
            kc[t] = a0;
            kc[t + 1] = a1;
            kc[t + 2] = a2;
            kc[t + 3] = a3;
            vc[t * C] = d0;
            vc[(t + 1) * C] = d1;
            vc[(t + 2) * C] = d2;
            vc[(t + 3) * C] = d3;
        }
    }
    for (; t < n; ++t) {
        if (kPack) {
            const uint4 a = kc[t], d = vc[t * C];
            ks[t * slot_vecs] = a;
            vs[t * slot_vecs] = d;
        } else {
            const uint4 a = ks[t * slot_vecs], d = vs[t * slot_vecs];
            kc[t] = a;
            vc[t * C] = d;
        }
    }
}

// LDS slot of (token i, chunk c) in a tile stored token-major.  For a
// power-of-two CT the chunk index is XOR-ed with a function of the row so
// that 16 consecutive tokens of one chunk (chunk-major access) land in 16
// distinct 16-byte bank groups of a 256-byte window, while the C chunks of
// one token (token-major access) stay a permutation of one row.
template <int CT>
__device__ __forceinline__ int lds_slot(int i, int c, int C)
{
    if constexpr (CT == 0) {
        return i * C + c;
    } else if constexpr (CT >= 16) {
        return i * CT + (c ^ (i & 15));
    } else {
        constexpr int kRowsPer256 = 16 / CT;
        return i * CT + (c ^ ((i / kRowsPer256) & (CT - 1)));
    }
}

// Registers are a native 4 x 32-bit vector type: arrays of it stay in VGPRs
// (arrays of the uint4 struct end up in scratch).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Packed-buffer stores of the tile pack kernels (contiguous and paged) go
// out write-through (sc0 sc1): each line leaves the L2 as it is written
// instead of sitting there dirty until the kernel's end-of-launch
// write-back.  Measured on one GPT-2-1.5B layer packed alone (102 MB read +
// write): 17.9 us instead of 20.4 us; 16-token paged packs 6% faster.
// The ring's step gather stores ordinarily: write-through gained nothing
// there, or lost 3-8%.  The split-role tile kernel (copy_split) also loads
// with the non-temporal hint in both directions and stores to the caches
// (unpack) with it: every byte is touched once, so nothing is worth keeping
// in the caches on the way.  Measured alone on cold data (median of 20):
// 48 GPT-2-1.5B layers in one call 0.78/0.76 -> 0.79/0.80 of HBM peak
// (pack/unpack), a BLOOM-176B layer 0.72/0.73 -> 0.75/0.78, a 100K-context
// row layer 0.75/0.75 -> 0.77/0.78; inside the 100K-context step its packs
// 0.62-0.63 -> 0.66, inside the BLOOM step 0.72 -> 0.75 (unpacks 0.60 ->
// 0.62), step times unchanged.  Non-temporal packed-buffer stores in place
// of write-through raised the isolated packs a little more (0.80, 0.76,
// 0.77) but cost the 100K step's in-step packs (0.63).  A plain streaming
// copy kernel (one 16-byte vector per thread, 256 threads per workgroup,
// 2 GiB) moves 6.08 TB/s (read + write) with ordinary and 6.46 TB/s with
// non-temporal loads and stores on this GPU: the practical copy ceiling.
// The paged kernels take the same hints (pool reads of the pack, packed
// reads and pool writes of the unpack): 48 GPT-2-1.5B layers from 16-token
// pages 0.68 -> 0.76 of peak packed, 0.70 -> 0.71 unpacked; 256-token
// chunks 0.67 -> 0.69 and 0.71 -> 0.72.  The ring's step gather loads the
// cache non-temporally when it packs: in the OPT-66B ring step its packs
// run at 0.49 of peak beside the flushes instead of 0.38, though 24
// GPT-2-1.5B steps packed alone take 0.90 us per step instead of 0.84.  It
// keeps ordinary accesses when it unpacks (non-temporal there: OPT-66B
// in-step unpacks 0.37 -> 0.33).
constexpr int kWriteThrough = 1 | 16;   // sc0 | sc1

// Buffer resource over `bytes` (< 2^31) of packed buffer from `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stage_rsrc(void *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void stage_store(u32x4 v, __amdgpu_buffer_rsrc_t r, int32_t vec)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, vec * 16, 0, kWriteThrough);
}

// The same R steps, one wave per (layer, row, head) unit, through LDS: a
// wave reads the unit's key chunk rows (R contiguous vectors each) and its
// value run (R*C contiguous vectors), transposes the key through its own LDS
// region, and writes step t's C key vectors and C value vectors (contiguous)
// into slot t, four vectors in flight per lane.  Used when a unit's R*C
// vectors fit the wave's LDS region.
constexpr int kStepWaves = 4;                 // waves (units) per workgroup
constexpr int kStepMaxVecs = 1024;            // R*C limit: 16 KiB of LDS per wave

__device__ __forceinline__ int step_slot(int t, int c, int C)
{
    // token-major with the chunk XOR-ed by the token when C is a power of two,
    // so the chunk-major writes of consecutive tokens spread over the banks
    return (C & (C - 1)) == 0 ? t * C + (c ^ (t & (C - 1))) : t * C + c;
}

template <bool kPack>
__global__ __launch_bounds__(kThreads) void copy_steps_lds(Geometry g, RowTable rt, int32_t n,
                                                           int64_t slot_vecs, int64_t units)
{
    extern __shared__ u32x4 step_lds[];
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int32_t C = g.C;
    const int32_t nv = n * C;                                   // vectors of K (and of V) per unit
    u32x4 *lds = step_lds + wave * nv;
    const int64_t u = (int64_t)blockIdx.x * kStepWaves + wave;
    const bool active = u < units;
    // unit u = ((li * B) + b) * H + h
    const int32_t h = active ? (int32_t)(u % g.H) : 0;
    const int32_t b = active ? (int32_t)((u / g.H) % g.B) : 0;
    const int32_t li = active ? (int32_t)(u / ((int64_t)g.H * g.B)) : 0;
    const int32_t s0 = rt.start[b];
    const int64_t unit = ((int64_t)(g.l0 + li) * g.B + b) * g.H + h;
    u32x4 *kc = (u32x4 *)(g.k + unit * C * g.Smax + s0);       // chunk c, step t: kc[c*Smax + t]
    u32x4 *vc = (u32x4 *)(g.v + (unit * g.Smax + s0) * C);     // step t, chunk c: vc[t*C + c]
    const int64_t blk = (int64_t)g.H * g.B * C;
    u32x4 *ks = (u32x4 *)(g.stage + 2 * (int64_t)li * blk + ((int64_t)g.H * b + h) * C);
    u32x4 *vs = ks + blk;                                       // step t, chunk c: ks[t*slot + c]
    constexpr int kB = 4;                                       // vectors in flight per lane
    if (kPack) {
        if (active) {
            for (int32_t e0 = lane; e0 < nv; e0 += 64 * kB) {   // key, chunk-major reads
                u32x4 r[kB];
#pragma unroll
                for (int j = 0; j < kB; ++j) {
                    const int32_t e = e0 + 64 * j, c = e / n, t = e - c * n;
                    if (e < nv)
                        r[j] = __builtin_nontemporal_load(kc + (int64_t)c * g.Smax + t);
                }
#pragma unroll
                for (int j = 0; j < kB; ++j) {
                    const int32_t e = e0 + 64 * j, c = e / n, t = e - c * n;
                    if (e < nv)
                        lds[step_slot(t, c, C)] = r[j];
                }
            }
            for (int32_t e0 = lane; e0 < nv; e0 += 64 * kB) {   // value: straight, per step
                u32x4 r[kB];
#pragma unroll
                for (int j = 0; j < kB; ++j)
                    if (e0 + 64 * j < nv)
                        r[j] = __builtin_nontemporal_load(vc + e0 + 64 * j);
#pragma unroll
                for (int j = 0; j < kB; ++j) {
                    const int32_t e = e0 + 64 * j, t = e / C, c = e - t * C;
                    if (e < nv)
                        vs[t * slot_vecs + c] = r[j];
                }
            }
        }
        __syncthreads();
        if (active)
            for (int32_t e = lane; e < nv; e += 64) {           // key, token-major writes
                const int32_t t = e / C, c = e - t * C;
                ks[t * slot_vecs + c] = lds[step_slot(t, c, C)];
            }
    } else {
        if (active) {
            for (int32_t e0 = lane; e0 < nv; e0 += 64 * kB) {
                u32x4 a[kB], d[kB];
#pragma unroll
                for (int j = 0; j < kB; ++j) {
                    const int32_t e = e0 + 64 * j, t = e / C, c = e - t * C;
                    if (e < nv) {
                        a[j] = ks[t * slot_vecs + c];
                        d[j] = vs[t * slot_vecs + c];
                    }
                }
#pragma unroll
                for (int j = 0; j < kB; ++j) {
                    const int32_t e = e0 + 64 * j, t = e / C, c = e - t * C;
                    if (e < nv) {
                        lds[step_slot(t, c, C)] = a[j];
                        vc[e] = d[j];
                    }
                }
            }
        }
        __syncthreads();
        if (active)
            for (int32_t e = lane; e < nv; e += 64) {
                const int32_t c = e / n, t = e - c * n;
                kc[(int64_t)c * g.Smax + t] = lds[step_slot(t, c, C)];
            }
    }
}

// The row owning workgroup q of a layer in a grid of the rows' own tiles:
// the last i in [0, nb) with pre[i] <= q.  A row without tokens owns no
// workgroups, so it is never the one found.  q is uniform across the
// workgroup: the search runs on scalar loads of the kernel arguments.
__device__ __forceinline__ int32_t tile_row(const RowTiles &rtl, int32_t nb, int32_t q)
{
    int32_t lo = 0, hi = nb;
    while (hi - lo > 1) {
        const int32_t mid = (lo + hi) >> 1;
        if (rtl.pre[mid] <= q)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

// The tile kernel (many tokens per row: prompt layers, chunks, swaps).  Split
// roles: a row's first g.k_tiles workgroups move K only -- a tile of TTK =
// 256 * KPER / C tokens of every chunk row, loaded chunk-major (each wave
// reads contiguous runs of one chunk row), transposed through LDS and
// stored token-major -- and the others move V only, a straight contiguous
// copy of 256 * VPER vectors with every load issued before the first store.
// Against the former tile kernel, whose workgroups moved a K tile and the
// matching V run together (one vector per thread each for heads of up to 16
// vectors), measured alone on cold data, median of 20: a BLOOM-176B layer
// 0.69-0.70 -> 0.73-0.74 of HBM peak packed and 0.69-0.75 -> 0.71-0.72
// unpacked, a 99,000-token 100K-context row layer 0.71 -> 0.74-0.76 both
// ways, 48 GPT-2-1.5B layers in one call 0.75 -> 0.78 and 0.73-0.77 ->
// 0.76-0.77.  Larger tiles (2 or 4 vectors per thread for K, V or both)
// were slower on 8- and 16-vector heads.  Loads, and the cache stores of
// unpack, carry the non-temporal hint (the cache policy note above).
template <int CT, int KPER, int VPER, bool kPack>
__global__ __launch_bounds__(kThreads) void copy_split(Geometry g, RowTable rt, RowTiles rtl)
{
    constexpr int TVK = kThreads * KPER;
    constexpr int TVV = kThreads * VPER;
    __shared__ u32x4 lds[TVK];
    const int32_t C = CT ? CT : g.C;
    const int32_t TTK = CT ? TVK / (CT ? CT : 1) : g.tile_tokens;

    // block -> (layer, row, head, tile); within a layer rows, then heads, then
    // tiles, as the cache and the packed buffer lay them out
    int32_t b, h, tile, li, k_tiles;
    if (g.tiles_per_row > 0) {
        // dense: every row of the span has the longest row's tiles (those
        // past a short row's end exit at once)
        int32_t bid = blockIdx.x;
        tile = bid % g.tiles_per_row;
        bid /= g.tiles_per_row;
        h = bid % g.nh;               // head within the moved range
        bid /= g.nh;
        b = g.b0 + bid % g.nb;
        li = bid / g.nb;
        k_tiles = g.k_tiles;
    } else {
        // the rows' own tiles only
        const int32_t q = (int32_t)blockIdx.x % g.layer_wgs;
        li = (int32_t)blockIdx.x / g.layer_wgs;
        const int32_t row = tile_row(rtl, g.nb, q);
        b = g.b0 + row;
        const int32_t n = rt.off[b + 1] - rt.off[b];
        k_tiles = (n + TTK - 1) / TTK;
        const int32_t row_tiles = k_tiles + (n * C + TVV - 1) / TVV;
        const int32_t r = q - rtl.pre[row];
        h = r / row_tiles;
        tile = r - h * row_tiles;
    }

    const int32_t off = rt.off[b];
    const int32_t cnt = rt.off[b + 1] - off;
    const int64_t unit = ((int64_t)(g.l0 + li) * g.B + b) * g.H + g.h0 + h;
    const int64_t blk = (int64_t)g.nh * g.T * C;          // one (layer, K|V) block
    u32x4 *ks_unit = (u32x4 *)(g.stage + 2 * (int64_t)li * blk +
                               ((int64_t)g.nh * off + (int64_t)h * cnt) * C);
    const int tid = threadIdx.x;

    if (tile >= k_tiles) {
        const int32_t v0 = (tile - k_tiles) * TVV;
        const int32_t nv = cnt * C;
        if (v0 >= nv)
            return;
        const int32_t n = min(TVV, nv - v0);
        u32x4 *vc = (u32x4 *)(g.v + (unit * g.Smax + rt.start[b]) * C) + v0;
        u32x4 *vs = ks_unit + blk + v0;
        u32x4 r[VPER];
        if (kPack) {
            const __amdgpu_buffer_rsrc_t rs = stage_rsrc(vs, (int64_t)n * 16);
#pragma unroll
            for (int p = 0; p < VPER; ++p) {
                const int e = tid + p * kThreads;
                if (e < n)
                    r[p] = __builtin_nontemporal_load(vc + e);
            }
#pragma unroll
            for (int p = 0; p < VPER; ++p) {
                const int e = tid + p * kThreads;
                if (e < n)
                    stage_store(r[p], rs, e);
            }
        } else {
#pragma unroll
            for (int p = 0; p < VPER; ++p) {
                const int e = tid + p * kThreads;
                if (e < n)
                    r[p] = __builtin_nontemporal_load(vs + e);
            }
#pragma unroll
            for (int p = 0; p < VPER; ++p) {
                const int e = tid + p * kThreads;
                if (e < n)
                    __builtin_nontemporal_store(r[p], vc + e);
            }
        }
        return;
    }

    const int32_t t0 = tile * TTK;
    if (t0 >= cnt)
        return;
    const int32_t nt = min(TTK, cnt - t0);
    const int32_t nvec = nt * C;
    u32x4 *kc = (u32x4 *)(g.k + unit * C * g.Smax + rt.start[b] + t0);  // chunk c, token i: kc[c*Smax + i]
    u32x4 *ks = ks_unit + (int64_t)t0 * C;                              // nvec contiguous vectors
    u32x4 kr[KPER];
    if (kPack) {
        const __amdgpu_buffer_rsrc_t krs = stage_rsrc(ks, (int64_t)nvec * 16);
#pragma unroll
        for (int p = 0; p < KPER; ++p) {
            const int e = tid + p * kThreads, c = e / TTK, i = e % TTK;
            if (c < C && i < nt)
                kr[p] = __builtin_nontemporal_load(kc + (int64_t)c * g.Smax + i);
        }
#pragma unroll
        for (int p = 0; p < KPER; ++p) {
            const int e = tid + p * kThreads, c = e / TTK, i = e % TTK;
            if (c < C && i < nt)
                lds[lds_slot<CT>(i, c, C)] = kr[p];
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < KPER; ++p) {
            const int e = tid + p * kThreads;
            if (e < nvec)
                stage_store(lds[lds_slot<CT>(e / C, e % C, C)], krs, e);
        }
    } else {
#pragma unroll
        for (int p = 0; p < KPER; ++p) {
            const int e = tid + p * kThreads;
            if (e < nvec)
                kr[p] = __builtin_nontemporal_load(ks + e);
        }
#pragma unroll
        for (int p = 0; p < KPER; ++p) {
            const int e = tid + p * kThreads;
            if (e < nvec)
                lds[lds_slot<CT>(e / C, e % C, C)] = kr[p];
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < KPER; ++p) {
            const int e = tid + p * kThreads, c = e / TTK, i = e % TTK;
            if (c < C && i < nt)
                __builtin_nontemporal_store(lds[lds_slot<CT>(i, c, C)], kc + (int64_t)c * g.Smax + i);
        }
    }
}

// Vectors per thread of the split-role kernel for K and for V: one each for
// heads of up to 32 vectors; four K vectors per thread for wider heads, so
// that a K tile still spans 8 or more tokens.  Measured alone on 256-, 512-
// and 1024-dim heads (4000 tokens, cold data): one vector per thread reached
// 0.76/0.75 of peak (pack/unpack) at 256 dims but 0.65/0.67 at 512 and
// 0.44/0.42 at 1024 (2-token K tiles); four K vectors 0.74/0.71, 0.72/0.71
// and 0.72/0.71; four for both 0.67-0.69; the former joint K+V tiles of
// 1024 vectors 0.70/0.68, 0.70/0.68-0.69, 0.69-0.70/0.68.
struct SplitMode {
    int kper, vper;
};

SplitMode split_mode(int32_t C)
{
    return C <= 32 ? SplitMode{1, 1} : SplitMode{4, 1};
}

// ---- paged pool --------------------------------------------------------------
// Token s of a row -> (index of its block in the row's table, slot in the block).
__device__ __forceinline__ void paged_split(const PagedGeometry &g, uint32_t s, uint32_t &q,
                                            uint32_t &slot)
{
    if (g.p_shift >= 0) {
        q = s >> g.p_shift;
        slot = s & (uint32_t)(g.P - 1);
    } else {
        q = s / (uint32_t)g.P;
        slot = s - q * (uint32_t)g.P;
    }
}

// Decode-sized ranges on a pool: one thread per (layer, row, head, vector c),
// as copy_rows_small, with each token's block looked up in the row's table.
template <bool kPack>
__global__ __launch_bounds__(kThreads) void copy_paged_small(PagedGeometry g, RowTable rt)
{
    const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
    const uint32_t C = (uint32_t)g.C;
    uint32_t r = gid / C;
    const uint32_t c = gid - r * C;
    const uint32_t h = r % (uint32_t)g.H;
    r /= (uint32_t)g.H;
    const uint32_t b = (uint32_t)g.b0 + r % (uint32_t)g.nb;
    r /= (uint32_t)g.nb;
    if (r >= (uint32_t)g.nl)
        return;
    const int32_t li = (int32_t)r;
    const int32_t off = rt.off[b];
    const int32_t cnt = rt.off[b + 1] - off;
    const int32_t s0 = rt.start[b];
    const int64_t layer = g.l0 + li;
    const int32_t *trow = g.table + (int64_t)b * g.table_stride;
    const int64_t blk = (int64_t)g.H * g.T * C;
    uint4 *ks = g.stage + 2 * (int64_t)li * blk + ((int64_t)g.H * off + (int64_t)h * cnt) * C + c;
    uint4 *vs = ks + blk;
    for (int32_t t = 0; t < cnt; ++t) {
        uint32_t q, slot;
        paged_split(g, (uint32_t)(s0 + t), q, slot);
        const int32_t id = trow[q];
        if (id < 0 || id >= g.NB)
            continue;
        const int64_t unit = (layer * g.NB + id) * g.H + h;
        uint4 *kc = g.k + (unit * C + c) * g.P + slot;
        uint4 *vc = g.v + (unit * g.P + slot) * C + c;
        if (kPack) {
            const uint4 a = *kc, d = *vc;
            ks[t * C] = a;
            vs[t * C] = d;
        } else {
            const uint4 a = ks[t * C], d = vs[t * C];
            *kc = a;
            *vc = d;
        }
    }
}

// Many tokens per row on a pool: the joint K+V tile scheme (K loaded
// chunk-major, transposed through LDS, stored token-major), with the tile's
// block ids staged in LDS first.  Within a block a key chunk row is P*16
// contiguous bytes, so chunk-major loads stay contiguous per block.
template <int CT, int PER, bool kPack>
__global__ __launch_bounds__(kThreads) void copy_paged_tiles(PagedGeometry g, RowTable rt)
{
    constexpr int TV = kThreads * PER;
    __shared__ u32x4 lds[TV];
    __shared__ int32_t ids[TV + 1];       // blocks touched by the tile (at most its tokens + 1)
    const int32_t C = CT ? CT : g.C;
    const int32_t TT = CT ? TV / CT : g.tile_tokens;

    int32_t bid = blockIdx.x;
    const int32_t tile = bid % g.tiles_per_row;
    bid /= g.tiles_per_row;
    const int32_t h = bid % g.H;
    bid /= g.H;
    const int32_t b = g.b0 + bid % g.nb;
    const int32_t li = bid / g.nb;

    const int32_t off = rt.off[b];
    const int32_t cnt = rt.off[b + 1] - off;
    const int32_t t0 = tile * TT;
    if (t0 >= cnt)
        return;
    const int32_t nt = min(TT, cnt - t0);
    const int32_t nvec = nt * C;
    const uint32_t s0 = (uint32_t)(rt.start[b] + t0);
    uint32_t q0, o0, q1, o1;
    paged_split(g, s0, q0, o0);
    paged_split(g, s0 + (uint32_t)nt - 1u, q1, o1);
    const int32_t nblk = (int32_t)(q1 - q0) + 1;
    const int32_t *trow = g.table + (int64_t)b * g.table_stride + q0;
    const int tid = threadIdx.x;
    for (int j = tid; j < nblk; j += kThreads) {
        const int32_t id = trow[j];
        ids[j] = (id >= 0 && id < g.NB) ? id : -1;
    }
    __syncthreads();

    const int64_t layer = g.l0 + li;
    const int64_t CP = (int64_t)C * g.P;          // vectors of one (block, head) unit
    const int64_t blk = (int64_t)g.H * g.T * C;
    u32x4 *ks = (u32x4 *)(g.stage + 2 * (int64_t)li * blk +
                          ((int64_t)g.H * off + (int64_t)h * cnt + t0) * C);
    u32x4 *vs = ks + blk;
    const u32x4 *kpool = (const u32x4 *)g.k;
    const u32x4 *vpool = (const u32x4 *)g.v;
    // unit base (in vectors) of tile token i, or -1 for a skipped block
    auto unit_of = [&](int32_t i, uint32_t &slot) -> int64_t {
        uint32_t q;
        paged_split(g, o0 + (uint32_t)i, q, slot);
        const int32_t id = ids[q];
        return id < 0 ? -1 : ((layer * g.NB + id) * g.H + h) * CP;
    };
    u32x4 kr[PER], vr[PER];

    if (kPack) {
        const __amdgpu_buffer_rsrc_t krs = stage_rsrc(ks, nvec * 16), vrs = stage_rsrc(vs, nvec * 16);
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = tid + p * kThreads, c = e / TT, i = e % TT;
            if (c < C && i < nt) {
                uint32_t slot;
                const int64_t u = unit_of(i, slot);
                if (u >= 0)
                    kr[p] = __builtin_nontemporal_load(kpool + u + (int64_t)c * g.P + slot);
            }
            if (e < nvec) {
                uint32_t slot;
                const int64_t u = unit_of(e / C, slot);
                if (u >= 0)
                    vr[p] = __builtin_nontemporal_load(vpool + u + (int64_t)slot * C + e % C);
            }
        }
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = tid + p * kThreads, c = e / TT, i = e % TT;
            if (c < C && i < nt)
                lds[lds_slot<CT>(i, c, C)] = kr[p];
            if (e < nvec) {
                uint32_t slot;
                if (unit_of(e / C, slot) >= 0)
                    stage_store(vr[p], vrs, e);
            }
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = tid + p * kThreads;
            if (e < nvec) {
                uint32_t slot;
                if (unit_of(e / C, slot) >= 0)
                    stage_store(lds[lds_slot<CT>(e / C, e % C, C)], krs, e);
            }
        }
    } else {
        u32x4 *kw = (u32x4 *)g.k;
        u32x4 *vw = (u32x4 *)g.v;
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = tid + p * kThreads;
            if (e < nvec) {
                kr[p] = ks[e];
                vr[p] = vs[e];
            }
        }
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = tid + p * kThreads;
            if (e < nvec) {
                lds[lds_slot<CT>(e / C, e % C, C)] = kr[p];
                uint32_t slot;
                const int64_t u = unit_of(e / C, slot);
                if (u >= 0)
                    vw[u + (int64_t)slot * C + e % C] = vr[p];
            }
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = tid + p * kThreads, c = e / TT, i = e % TT;
            if (c < C && i < nt) {
                uint32_t slot;
                const int64_t u = unit_of(i, slot);
                if (u >= 0)
                    kw[u + (int64_t)c * g.P + slot] = lds[lds_slot<CT>(i, c, C)];
            }
        }
    }
}

// Launch kernel `k` on `s`.  With a timer, the timer's two events take the
// dispatch's own begin and end timestamps, so a timed launch costs no extra
// packets on the stream and its interval is the kernel's alone.
template <typename... P, typename... A>
hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                  const LaunchTimer &t, A... a)
{
    std::tuple<P...> vals(a...);
    void *ptrs[sizeof...(P)];
    std::apply([&ptrs](auto &...v) {
        size_t i = 0;
        ((ptrs[i++] = (void *)&v), ...);
    }, vals);
    if (t.start)
        return hipExtLaunchKernel((const void *)k, grid, block, ptrs, lds, s, t.start, t.stop, 0);
    return hipLaunchKernel((const void *)k, grid, block, ptrs, lds, s);
}

// Unpack of many tokens per row into a pool, split roles as copy_split: K
// workgroups stage the block ids of their tile in LDS and scatter the tile
// through LDS; V workgroups move 256 * VPER vectors of the row's token range
// (token-major, contiguous in the packed buffer), each to the slot its
// token's block gives.  Tokens of skipped blocks are not written.
template <int CT, int KPER, int VPER>
__global__ __launch_bounds__(kThreads) void unpack_paged_split(PagedGeometry g, RowTable rt)
{
    constexpr int TVK = kThreads * KPER;
    constexpr int TVV = kThreads * VPER;
    __shared__ u32x4 lds[TVK];
    __shared__ int32_t ids[TVK + 1];      // blocks touched by a K tile (at most its tokens + 1)
    const int32_t C = CT ? CT : g.C;
    const int32_t TTK = CT ? TVK / (CT ? CT : 1) : g.tile_tokens;

    int32_t bid = blockIdx.x;
    const int32_t tile = bid % g.tiles_per_row;
    bid /= g.tiles_per_row;
    const int32_t h = bid % g.H;
    bid /= g.H;
    const int32_t b = g.b0 + bid % g.nb;
    const int32_t li = bid / g.nb;

    const int32_t off = rt.off[b];
    const int32_t cnt = rt.off[b + 1] - off;
    const int64_t layer = g.l0 + li;
    const int64_t CP = (int64_t)C * g.P;          // vectors of one (block, head) unit
    const int64_t blk = (int64_t)g.H * g.T * C;
    const u32x4 *ks_unit = (const u32x4 *)(g.stage + 2 * (int64_t)li * blk +
                                           ((int64_t)g.H * off + (int64_t)h * cnt) * C);
    const int32_t *trow = g.table + (int64_t)b * g.table_stride;
    const int tid = threadIdx.x;

    if (tile >= g.k_tiles) {
        const int32_t v0 = (tile - g.k_tiles) * TVV;
        const int32_t nv = cnt * C;
        if (v0 >= nv)
            return;
        const int32_t n = min(TVV, nv - v0);
        const u32x4 *vs = ks_unit + blk + v0;
        u32x4 *vpool = (u32x4 *)g.v;
        u32x4 r[VPER];
#pragma unroll
        for (int p = 0; p < VPER; ++p) {
            const int e = tid + p * kThreads;
            if (e < n)
                r[p] = __builtin_nontemporal_load(vs + e);
        }
#pragma unroll
        for (int p = 0; p < VPER; ++p) {
            const int e = tid + p * kThreads;
            if (e < n) {
                const int32_t tok = (v0 + e) / C, c = v0 + e - tok * C;
                uint32_t q, slot;
                paged_split(g, (uint32_t)(rt.start[b] + tok), q, slot);
                const int32_t id = trow[q];
                if (id >= 0 && id < g.NB)
                    __builtin_nontemporal_store(r[p], vpool + ((layer * g.NB + id) * g.H + h) * CP + (int64_t)slot * C + c);
            }
        }
        return;
    }

    const int32_t t0 = tile * TTK;
    if (t0 >= cnt)
        return;
    const int32_t nt = min(TTK, cnt - t0);
    const int32_t nvec = nt * C;
    const uint32_t s0 = (uint32_t)(rt.start[b] + t0);
    uint32_t q0, o0, q1, o1;
    paged_split(g, s0, q0, o0);
    paged_split(g, s0 + (uint32_t)nt - 1u, q1, o1);
    const int32_t nblk = (int32_t)(q1 - q0) + 1;
    for (int j = tid; j < nblk; j += kThreads) {
        const int32_t id = trow[q0 + j];
        ids[j] = (id >= 0 && id < g.NB) ? id : -1;
    }
    const u32x4 *ks = ks_unit + (int64_t)t0 * C;
    u32x4 kr[KPER];
#pragma unroll
    for (int p = 0; p < KPER; ++p) {
        const int e = tid + p * kThreads;
        if (e < nvec)
            kr[p] = __builtin_nontemporal_load(ks + e);
    }
#pragma unroll
    for (int p = 0; p < KPER; ++p) {
        const int e = tid + p * kThreads;
        if (e < nvec)
            lds[lds_slot<CT>(e / C, e % C, C)] = kr[p];
    }
    __syncthreads();     // the tile in LDS and the block ids
    u32x4 *kw = (u32x4 *)g.k;
#pragma unroll
    for (int p = 0; p < KPER; ++p) {
        const int e = tid + p * kThreads, c = e / TTK, i = e % TTK;
        if (c < C && i < nt) {
            uint32_t q, slot;
            paged_split(g, o0 + (uint32_t)i, q, slot);
            const int32_t id = ids[q];
            if (id >= 0)
                __builtin_nontemporal_store(lds[lds_slot<CT>(i, c, C)],
                    kw + ((layer * g.NB + id) * g.H + h) * CP + (int64_t)c * g.P + slot);
        }
    }
}

template <int CT>
hipError_t launch_unpack_paged_split_c(const SplitMode &m, const PagedGeometry &g,
                                       const RowTable &rt, dim3 grid, hipStream_t s,
                                       const LaunchTimer &t)
{
    const dim3 block(kThreads);
    if constexpr (CT == 0 || CT <= 32)
        if (m.kper == 1 && m.vper == 1)
            return launch(unpack_paged_split<CT, 1, 1>, grid, block, 0, s, t, g, rt);
    if constexpr (CT == 0 || CT > 32)
        if (m.kper == 4 && m.vper == 1)
            return launch(unpack_paged_split<CT, 4, 1>, grid, block, 0, s, t, g, rt);
    return hipErrorInvalidValue;
}

hipError_t launch_unpack_paged_split(const SplitMode &m, const PagedGeometry &g,
                                     const RowTable &rt, int64_t blocks, hipStream_t s,
                                     const LaunchTimer &t)
{
    const dim3 grid((unsigned)blocks);
    switch (g.C) {
    case 1: return launch_unpack_paged_split_c<1>(m, g, rt, grid, s, t);
    case 2: return launch_unpack_paged_split_c<2>(m, g, rt, grid, s, t);
    case 4: return launch_unpack_paged_split_c<4>(m, g, rt, grid, s, t);
    case 8: return launch_unpack_paged_split_c<8>(m, g, rt, grid, s, t);
    case 16: return launch_unpack_paged_split_c<16>(m, g, rt, grid, s, t);
    case 32: return launch_unpack_paged_split_c<32>(m, g, rt, grid, s, t);
    case 64: return launch_unpack_paged_split_c<64>(m, g, rt, grid, s, t);
    case 128: return launch_unpack_paged_split_c<128>(m, g, rt, grid, s, t);
    default: return launch_unpack_paged_split_c<0>(m, g, rt, grid, s, t);
    }
}

// Which tile kernel a paged pack or unpack uses.  Measured alone on a
// GPT-2-1.5B pool (48 layers x 8 rows x 1000 tokens, 2.46 GB), two runs:
// split roles unpack 16-token pages at 0.68 of HBM peak and 256-token pages
// at 0.69 (joint tiles 0.67 and 0.67), but pack them at 0.66 and 0.66-0.67
// (joint 0.68 and 0.67).  (A split V workgroup of a pack looks up each
// vector's block in the table before it can load from the pool; one of an
// unpack loads the packed buffer first.)  So: joint tiles pack, split roles
// unpack.

// Vectors per thread of the paged tile kernel: 256-vector tiles for heads of
// up to 16 vectors (measured 4-5% faster packs and 1.5-3% faster unpacks
// than 512-vector tiles on a GPT-2-1.5B pool), 1024-vector tiles for wider
// ones.
constexpr int paged_per_thread(int32_t C) { return C <= 16 ? 1 : 4; }

template <bool kPack>
hipError_t launch_paged_tiles(const PagedGeometry &g, const RowTable &rt, int64_t blocks,
                              hipStream_t s, const LaunchTimer &t)
{
    const dim3 grid((unsigned)blocks), block(kThreads);
    hipError_t e;
    switch (g.C) {
    case 1: e = launch(copy_paged_tiles<1, 1, kPack>, grid, block, 0, s, t, g, rt); break;
    case 2: e = launch(copy_paged_tiles<2, 1, kPack>, grid, block, 0, s, t, g, rt); break;
    case 4: e = launch(copy_paged_tiles<4, 1, kPack>, grid, block, 0, s, t, g, rt); break;
    case 8: e = launch(copy_paged_tiles<8, 1, kPack>, grid, block, 0, s, t, g, rt); break;
    case 16: e = launch(copy_paged_tiles<16, 1, kPack>, grid, block, 0, s, t, g, rt); break;
    case 32: e = launch(copy_paged_tiles<32, 4, kPack>, grid, block, 0, s, t, g, rt); break;
    case 64: e = launch(copy_paged_tiles<64, 4, kPack>, grid, block, 0, s, t, g, rt); break;
    case 128: e = launch(copy_paged_tiles<128, 4, kPack>, grid, block, 0, s, t, g, rt); break;
    default:
        if (paged_per_thread(g.C) == 1)
            e = launch(copy_paged_tiles<0, 1, kPack>, grid, block, 0, s, t, g, rt);
        else
            e = launch(copy_paged_tiles<0, 4, kPack>, grid, block, 0, s, t, g, rt);
        break;
    }
    return e;
}

template <int CT, bool kPack>
hipError_t launch_split_c(const SplitMode &m, const Geometry &g, const RowTable &rt,
                          const RowTiles &rtl, dim3 grid, hipStream_t s, const LaunchTimer &t)
{
    const dim3 block(kThreads);
    if constexpr (CT == 0 || CT <= 32)
        if (m.kper == 1 && m.vper == 1)
            return launch(copy_split<CT, 1, 1, kPack>, grid, block, 0, s, t, g, rt, rtl);
    if constexpr (CT == 0 || CT > 32)
        if (m.kper == 4 && m.vper == 1)
            return launch(copy_split<CT, 4, 1, kPack>, grid, block, 0, s, t, g, rt, rtl);
    return hipErrorInvalidValue;
}

template <bool kPack>
hipError_t launch_split(const SplitMode &m, const Geometry &g, const RowTable &rt,
                        const RowTiles &rtl, int64_t blocks, hipStream_t s, const LaunchTimer &t)
{
    const dim3 grid((unsigned)blocks);
    switch (g.C) {
    case 1: return launch_split_c<1, kPack>(m, g, rt, rtl, grid, s, t);
    case 2: return launch_split_c<2, kPack>(m, g, rt, rtl, grid, s, t);
    case 4: return launch_split_c<4, kPack>(m, g, rt, rtl, grid, s, t);
    case 8: return launch_split_c<8, kPack>(m, g, rt, rtl, grid, s, t);
    case 16: return launch_split_c<16, kPack>(m, g, rt, rtl, grid, s, t);
    case 32: return launch_split_c<32, kPack>(m, g, rt, rtl, grid, s, t);
    case 64: return launch_split_c<64, kPack>(m, g, rt, rtl, grid, s, t);
    case 128: return launch_split_c<128, kPack>(m, g, rt, rtl, grid, s, t);
    default: return launch_split_c<0, kPack>(m, g, rt, rtl, grid, s, t);
    }
}

// Tokens per tile of a kernel whose threads move `per` vectors each.
int tile_tokens_for(int32_t C, int per)
{
    const int tv = kThreads * per;
    return C >= tv ? 1 : tv / C;
}

// Transfer between a staging bank in HBM and pinned host memory, run by the
// GPU's own load/store units instead of a DMA engine (the host buffer is
// mapped into the GPU's address space).  Each thread keeps four 16-byte
// vectors in flight.
//
// Device->host stores go through a bounds-checked buffer resource with the
// system-coherent, non-temporal cache policy (sc0 sc1 nt), from a small grid
// (8 workgroups by default).  Measured on MI355X: that keeps the host link at
// ~56 GB/s while co-running HBM kernels lose about a third of their speed;
// ordinary stores to host memory, or many workgroups, hold up other kernels'
// HBM traffic several-fold.  Host->device reads use non-temporal loads.
constexpr int kHostStorePolicy = 1 | 2 | 16;   // sc0 | nt | sc1

template <bool kToHost>
__global__ __launch_bounds__(kThreads) void link_copy(const u32x4 *__restrict__ src,
                                                      u32x4 *__restrict__ dst, int32_t nvec)
{
    const int32_t stride = (int32_t)gridDim.x * kThreads;
    int32_t i = (int32_t)blockIdx.x * kThreads + threadIdx.x;
    if (kToHost) {
        // num_records = nvec * 16 bytes (< 2^31 per launch): out-of-range stores are dropped
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(dst, 0, nvec * 16, 0x00020000);
        for (; i + 3 * stride < nvec; i += 4 * stride) {
            const u32x4 a = src[i], b = src[i + stride];
            const u32x4 c = src[i + 2 * stride], d = src[i + 3 * stride];
            __builtin_amdgcn_raw_buffer_store_b128(a, r, i * 16, 0, kHostStorePolicy);
            __builtin_amdgcn_raw_buffer_store_b128(b, r, (i + stride) * 16, 0, kHostStorePolicy);
            __builtin_amdgcn_raw_buffer_store_b128(c, r, (i + 2 * stride) * 16, 0, kHostStorePolicy);
            __builtin_amdgcn_raw_buffer_store_b128(d, r, (i + 3 * stride) * 16, 0, kHostStorePolicy);
        }
        for (; i < nvec; i += stride)
            __builtin_amdgcn_raw_buffer_store_b128(src[i], r, i * 16, 0, kHostStorePolicy);
        __threadfence_system();   // host-visible before the kernel completes
    } else {
        for (; i + 3 * stride < nvec; i += 4 * stride) {
            const u32x4 a = __builtin_nontemporal_load(src + i);
            const u32x4 b = __builtin_nontemporal_load(src + i + stride);
            const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
            const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
            dst[i] = a;
            dst[i + stride] = b;
            dst[i + 2 * stride] = c;
            dst[i + 3 * stride] = d;
        }
        for (; i < nvec; i += stride)
            dst[i] = __builtin_nontemporal_load(src + i);
    }
}

// Workgroups of one link copy: `blocks` when positive, else the default
// (8 for device->host, 128 for host->device).
int link_blocks(bool to_host, int32_t blocks)
{
    if (blocks > 0)
        return blocks;
    return to_host ? kLinkBlocksToHost : 128;
}

// The span [b0, b0 + nb) from the first to the last row that moves a token:
// the grids cover it alone, since a workgroup of an empty row still has to be
// dispatched (measured: a 3-row group of a 16-row layer took 126 us in a grid
// over all rows against 97 us over the three).  False when no row moves one.
bool row_span(const RowTable &rt, int32_t B, int32_t *b0, int32_t *nb)
{
    int32_t lo = 0, hi = B;
    while (lo < hi && rt.off[lo + 1] == rt.off[lo])
        ++lo;
    while (hi > lo && rt.off[hi] == rt.off[hi - 1])
        --hi;
    *b0 = lo;
    *nb = hi - lo;
    return hi > lo;
}

// Prefix of the workgroups of rows [b0, b0 + nb) of one layer into
// rtl->pre: each of the nh heads of row b has ceil(count_b / ttk) K tiles
// and ceil(count_b * C / tvv) V runs.  Returns the layer's total, or -1
// when it does not fit a grid.
int64_t row_tile_prefix(const RowTable &rt, int32_t b0, int32_t nb, int32_t nh, int32_t ttk,
                        int32_t C, int32_t tvv, RowTiles *rtl)
{
    int64_t total = 0;
    rtl->pre[0] = 0;
    for (int32_t i = 0; i < nb; ++i) {
        const int64_t cnt = rt.off[b0 + i + 1] - rt.off[b0 + i];
        total += nh * ((cnt + ttk - 1) / ttk + (cnt * C + tvv - 1) / tvv);
        if (total > 0x7fffffffLL)
            return -1;
        rtl->pre[i + 1] = (int32_t)total;
    }
    return total;
}

}  // namespace

int launch_copy(bool pack, const Geometry &g0, const RowTable &rt, int32_t max_count,
                hipStream_t s)
{
    if (max_count <= 0 || g0.nl <= 0 || g0.T <= 0)
        return KV_OK;
    const bool small = max_count <= kSmallMaxTokens;
    Geometry g = g0;
    if (!row_span(rt, g.B, &g.b0, &g.nb))
        return KV_OK;
    int64_t per_layer;
    RowTiles rtl{};
    if (small) {
        per_layer = ((int64_t)g.nb * g.nh * g.C + kThreads - 1) / kThreads;
    } else {
        const SplitMode m = split_mode(g.C);
        g.tile_tokens = tile_tokens_for(g.C, m.kper);
        g.k_tiles = (max_count + g.tile_tokens - 1) / g.tile_tokens;
        const int32_t tvv = kThreads * m.vper;
        g.tiles_per_row = g.k_tiles + (int32_t)(((int64_t)max_count * g.C + tvv - 1) / tvv);
        per_layer = (int64_t)g.nb * g.nh * g.tiles_per_row;
        // ragged rows: a grid of the rows' own tiles when the dense one would
        // be a fifth or more empty workgroups (finding its row costs a
        // workgroup a few dependent loads before its first access, which
        // lost 7% on uniform 4 KiB tiles)
        const int64_t own = row_tile_prefix(rt, g.b0, g.nb, g.nh, g.tile_tokens, g.C, tvv, &rtl);
        if (own >= 0 && own * 5 <= per_layer * 4) {
            g.tiles_per_row = 0;
            g.layer_wgs = (int32_t)own;
            per_layer = own;
        }
    }
    // A launch covers whole layers.  Keep every grid within 2^31-1 blocks and,
    // for the small kernel, its flat thread id within 2^31.
    const int64_t max_blocks = small ? 0x7fffffffLL / kThreads : 0x7fffffffLL;
    const int32_t layers_per_launch =
        (int32_t)std::max<int64_t>(1, std::min<int64_t>(g.nl, max_blocks / per_layer));
    const char *name = small ? (pack ? "pack_rows_small" : "unpack_rows_small")
                             : (pack ? "pack_tiles" : "unpack_tiles");
    const int64_t blk = (int64_t)g.nh * g.T * g.C;  // vectors per (layer, K|V) block

    for (int32_t done = 0; done < g0.nl; done += layers_per_launch) {
        Geometry gl = g;
        gl.l0 = g0.l0 + done;
        gl.nl = std::min<int32_t>(layers_per_launch, g0.nl - done);
        gl.stage = g0.stage + 2 * (int64_t)done * blk;
        const int64_t payload = 2 * (int64_t)gl.nl * blk * 16;
        const LaunchTimer t = profile_take();
        hipError_t e;
        if (small) {
            const int64_t threads = (int64_t)gl.nl * gl.nb * gl.nh * gl.C;
            const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads)), block(kThreads);
            if (pack)
                e = launch(copy_rows_small<true>, grid, block, 0, s, t, gl, rt);
            else
                e = launch(copy_rows_small<false>, grid, block, 0, s, t, gl, rt);
        } else {
            const int64_t blocks = (int64_t)gl.nl * per_layer;
            const SplitMode m = split_mode(g.C);
            e = pack ? launch_split<true>(m, gl, rt, rtl, blocks, s, t)
                     : launch_split<false>(m, gl, rt, rtl, blocks, s, t);
        }
        profile_commit(t, name, 2 * payload, e == hipSuccess);
        if (e != hipSuccess)
            return hip_fail(e, name);
    }
    return KV_OK;
}

int launch_steps(bool pack, const Geometry &g0, const RowTable &rt, int32_t n,
                 int64_t slot_vecs, hipStream_t s)
{
    if (n <= 0 || g0.nl <= 0)
        return KV_OK;
    const int64_t per_layer = (int64_t)g0.B * g0.H * g0.C;       // threads
    const int32_t layers_per_launch = (int32_t)std::max<int64_t>(
        1, std::min<int64_t>(g0.nl, (0x7fffffffLL / kThreads) * kThreads / per_layer));
    const int64_t blk = (int64_t)g0.H * g0.B * g0.C;
    const char *name = pack ? "pack_steps" : "unpack_steps";
    for (int32_t done = 0; done < g0.nl; done += layers_per_launch) {
        Geometry gl = g0;
        gl.l0 = g0.l0 + done;
        gl.nl = std::min<int32_t>(layers_per_launch, g0.nl - done);
        gl.stage = g0.stage + 2 * (int64_t)done * blk;
        const int64_t payload = 2 * (int64_t)gl.nl * blk * 16 * n;
        const int64_t threads = (int64_t)gl.nl * per_layer;
        const LaunchTimer t = profile_take();
        hipError_t e;
        if ((int64_t)n * g0.C <= kStepMaxVecs) {
            const int64_t units = (int64_t)gl.nl * g0.B * g0.H;
            const dim3 grid((unsigned)((units + kStepWaves - 1) / kStepWaves)), block(kThreads);
            const size_t lds = (size_t)kStepWaves * n * g0.C * sizeof(u32x4);
            if (pack)
                e = launch(copy_steps_lds<true>, grid, block, lds, s, t, gl, rt, n, slot_vecs, units);
            else
                e = launch(copy_steps_lds<false>, grid, block, lds, s, t, gl, rt, n, slot_vecs, units);
        } else {
            const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads)), block(kThreads);
            if (pack)
                e = launch(copy_steps<true>, grid, block, 0, s, t, gl, rt, n, slot_vecs);
            else
                e = launch(copy_steps<false>, grid, block, 0, s, t, gl, rt, n, slot_vecs);
        }
        profile_commit(t, name, 2 * payload, e == hipSuccess);
        if (e != hipSuccess)
            return hip_fail(e, name);
    }
    return KV_OK;
}

int launch_paged_copy(bool pack, const PagedGeometry &g0, const RowTable &rt, int32_t max_count,
                      hipStream_t s)
{
    if (max_count <= 0 || g0.nl <= 0 || g0.T <= 0)
        return KV_OK;
    const bool small = max_count <= kSmallMaxTokens;
    PagedGeometry g = g0;
    if (!row_span(rt, g.B, &g.b0, &g.nb))
        return KV_OK;
    int64_t per_layer;
    if (small) {
        per_layer = ((int64_t)g.nb * g.H * g.C + kThreads - 1) / kThreads;
    } else if (pack) {
        g.tile_tokens = tile_tokens_for(g.C, paged_per_thread(g.C));
        g.tiles_per_row = (max_count + g.tile_tokens - 1) / g.tile_tokens;
        per_layer = (int64_t)g.nb * g.H * g.tiles_per_row;
    } else {
        const SplitMode m = split_mode(g.C);
        g.tile_tokens = tile_tokens_for(g.C, m.kper);
        g.k_tiles = (max_count + g.tile_tokens - 1) / g.tile_tokens;
        const int32_t tvv = kThreads * m.vper;
        g.tiles_per_row = g.k_tiles + (int32_t)(((int64_t)max_count * g.C + tvv - 1) / tvv);
        per_layer = (int64_t)g.nb * g.H * g.tiles_per_row;
    }
    const int64_t max_blocks = small ? 0x7fffffffLL / kThreads : 0x7fffffffLL;
    const int32_t layers_per_launch =
        (int32_t)std::max<int64_t>(1, std::min<int64_t>(g.nl, max_blocks / per_layer));
    const char *name = small ? (pack ? "pack_paged_small" : "unpack_paged_small")
                             : (pack ? "pack_paged_tiles" : "unpack_paged_tiles");
    const int64_t blk = (int64_t)g.H * g.T * g.C;
    for (int32_t done = 0; done < g0.nl; done += layers_per_launch) {
        PagedGeometry gl = g;
        gl.l0 = g0.l0 + done;
        gl.nl = std::min<int32_t>(layers_per_launch, g0.nl - done);
        gl.stage = g0.stage + 2 * (int64_t)done * blk;
        const int64_t payload = 2 * (int64_t)gl.nl * blk * 16;
        const LaunchTimer t = profile_take();
        hipError_t e;
        if (small) {
            const int64_t threads = (int64_t)gl.nl * gl.nb * gl.H * gl.C;
            const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads)), block(kThreads);
            if (pack)
                e = launch(copy_paged_small<true>, grid, block, 0, s, t, gl, rt);
            else
                e = launch(copy_paged_small<false>, grid, block, 0, s, t, gl, rt);
        } else {
            const int64_t blocks = (int64_t)gl.nl * per_layer;
            e = pack ? launch_paged_tiles<true>(gl, rt, blocks, s, t)
                     : launch_unpack_paged_split(split_mode(g.C), gl, rt, blocks, s, t);
        }
        profile_commit(t, name, 2 * payload, e == hipSuccess);
        if (e != hipSuccess)
            return hip_fail(e, name);
    }
    return KV_OK;
}

int launch_link_copy(void *dst, const void *src, int64_t bytes, bool to_host, hipStream_t s,
                     int32_t blocks_wanted)
{
    if (bytes <= 0)
        return KV_OK;
    if (bytes % 16 != 0 || ((uintptr_t)dst | (uintptr_t)src) % 16 != 0)
        return set_error(KV_EINVAL, "link copy of %lld bytes is not in whole 16-byte vectors",
                         (long long)bytes);
    const char *name = to_host ? "link_copy_d2h" : "link_copy_h2d";
    // one launch per piece of at most 1 GiB: 32-bit offsets inside a launch
    constexpr int64_t kPiece = int64_t(1) << 30;
    for (int64_t done = 0; done < bytes; done += kPiece) {
        const int64_t n = std::min(kPiece, bytes - done);
        const int32_t nvec = (int32_t)(n / 16);
        const int64_t blocks =
            std::min<int64_t>(link_blocks(to_host, blocks_wanted), (nvec + kThreads - 1) / kThreads);
        const u32x4 *from = (const u32x4 *)((const char *)src + done);
        u32x4 *to = (u32x4 *)((char *)dst + done);
        const LaunchTimer t = profile_take();
        const dim3 grid((unsigned)blocks), block(kThreads);
        hipError_t e;
        if (to_host)
            e = launch(link_copy<true>, grid, block, 0, s, t, from, to, nvec);
        else
            e = launch(link_copy<false>, grid, block, 0, s, t, from, to, nvec);
        profile_commit(t, name, n, e == hipSuccess);
        if (e != hipSuccess)
            return hip_fail(e, name);
    }
    return KV_OK;
}

}  // namespace kvs
