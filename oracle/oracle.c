/*
 * oracle.c -- the oracle for the KV-cache buffered-copy path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library: every index below is written out here from the
 * definitions, in plain scalar loops, one 16-bit element at a time.
 *
 * What it computes (sources are the pages this project follows):
 *
 *  - "DejaVu: KV-Cache Streaming for Fast, Fault-Tolerant Generative LLM
 *    Serving" (papercache.org summary), section "Method details":
 *      * DejaVuLib implementation, Fig 6 -- the KV cache is preallocated at
 *        the maximum sequence length, and each generated token updates a
 *        small, non-contiguous part of the key cache;
 *      * Buffered copies, Fig 7a -- the small updates are aggregated into one
 *        contiguous temporary buffer in GPU memory, which is then copied out
 *        once it is filled;
 *      * Layer-by-layer prompt cache streaming, Fig 7b -- prompt KV is moved
 *        one layer at a time;
 *      * Table 1 -- scatter/gather break a non-contiguous KV region into
 *        contiguous transfers;
 *      * Microbatch swapping workflow, Fig 9 -- swap-out moves cache contents
 *        to CPU memory and swap-in brings them back.
 *  - lsln.cn article on decode-only inference, section "KV Cache capacity":
 *    the KV bytes of B rows, S tokens, H heads of D dims, P bytes per element
 *    and N layers are 2 x B x S x H x D x P x N.
 *
 * Readings taken where the pages are silent:
 *  - Cache layouts: key [L,B,H,D/8,Smax,8], value [L,B,H,Smax,D]; an element
 *    is 16 bits (fp16 or bf16, moved as raw bits, never converted).
 *  - Packed (staging) order: the selected elements in lexicographic order of
 *    (layer, K before V, row b, head h, token t, dim d).  With
 *    T = sum_b count_b and rowoff_b = sum_{b'<b} count_b', element
 *    (l, kv, b, h, t, d) sits at
 *        ((l-l0)*2 + kv)*(H*T*D) + (H*rowoff_b + h*count_b + t)*D + d.
 *    The pages print no staged buffer, so this order is a reading; what pins
 *    the oracle is this definition (brute-force coordinate decoding, numpy
 *    transposes, the size closed form and round-trip identity in the tests).
 *  - Prompt-layer range: row b moves tokens [tok_begin, tok_begin+tok_count)
 *    clipped to [0, row_len_b).
 *  - Ring restore: slots are unpacked in ascending step order, so a later
 *    step wins when two steps name the same position.
 *  - Appendix E (microbatch swapping benefit): the inequality
 *    2 N t >= sum_{i=p}^{N+p} max(t, i B C / bw), bounds inclusive as printed.
 *  - Restart point after a failure ("Failure detection and recovery",
 *    Fig 10): a (microbatch, step) pair counts as replicated once every worker
 *    has acknowledged it; steps run in (step, microbatch) order; the pipeline
 *    restarts at the first pair in that order that is not replicated.
 *  - Paged pool (vLLM's paging and Mooncake's chunks are named in the pages;
 *    neither layout is given): the contiguous layouts with (row, Smax)
 *    replaced by (physical block, block_tokens P) -- key
 *    [L, NB, H, D/8, P, 8], value [L, NB, H, P, D] -- and a block table per
 *    row: row b's token s lives in block table[b*stride + s/P] at slot s%P.
 *    A paged pack writes the same packed format as a contiguous pack.
 *  - stream_out / stream_in (Table 1, Fast prompt KV transfer): a worker's
 *    cache holds one partition of the model's KV -- a global layer range, a
 *    global head range and a global request (row) range, stored at local
 *    indices from 0.  The piece a source sends a destination is the
 *    intersection of the two partitions, in the packed order above taken over
 *    global (layer, K/V, row, head, token, dim); the destination merges each
 *    piece it receives at its own local indices.
 *
 * Every function here is plain C99, single-threaded.
 */
#include <stdint.h>
#include <stddef.h>

/* Element offset of K(l,b,h,s,d) in the key layout [L,B,H,D/8,Smax,8]. */
int64_t oracle_key_offset(int64_t L, int64_t B, int64_t H, int64_t D, int64_t Smax,
                          int64_t l, int64_t b, int64_t h, int64_t s, int64_t d)
{
    (void)L;
    int64_t chunk = d / 8;   /* which 8-element (16-byte) vector of the head */
    int64_t lane = d % 8;    /* element inside that vector */
    return ((((l * B + b) * H + h) * (D / 8) + chunk) * Smax + s) * 8 + lane;
}

/* Element offset of V(l,b,h,s,d) in the value layout [L,B,H,Smax,D]. */
int64_t oracle_value_offset(int64_t L, int64_t B, int64_t H, int64_t D, int64_t Smax,
                            int64_t l, int64_t b, int64_t h, int64_t s, int64_t d)
{
    (void)L;
    return (((l * B + b) * H + h) * Smax + s) * D + d;
}

/* Number of 16-bit elements moved by one pack over `layer_count` layers:
 * 2 (K and V) * layer_count * H * D * sum_b count_b. */
int64_t oracle_pack_elems(int64_t H, int64_t D, int64_t layer_count,
                          int64_t B, const int32_t *count)
{
    int64_t tokens = 0;
    for (int64_t b = 0; b < B; ++b)
        tokens += count[b];
    return 2 * layer_count * H * D * tokens;
}

/* Gather (pack): copy the selected region of both caches into `out` in the
 * packed order.  Rows with count 0 contribute nothing. */
void oracle_pack(int64_t L, int64_t B, int64_t H, int64_t D, int64_t Smax,
                 const uint16_t *key, const uint16_t *value,
                 int64_t layer_begin, int64_t layer_count,
                 const int32_t *start, const int32_t *count,
                 uint16_t *out)
{
    int64_t o = 0;
    for (int64_t l = layer_begin; l < layer_begin + layer_count; ++l)
        for (int kv = 0; kv < 2; ++kv)
            for (int64_t b = 0; b < B; ++b)
                for (int64_t h = 0; h < H; ++h)
                    for (int64_t t = 0; t < count[b]; ++t)
                        for (int64_t d = 0; d < D; ++d) {
                            int64_t s = start[b] + t;
                            if (kv == 0)
                                out[o] = key[oracle_key_offset(L, B, H, D, Smax, l, b, h, s, d)];
                            else
                                out[o] = value[oracle_value_offset(L, B, H, D, Smax, l, b, h, s, d)];
                            ++o;
                        }
}

/* Scatter (unpack): the inverse of oracle_pack.  Writes exactly the selected
 * elements of the caches from `in`; every other element is left as it was. */
void oracle_unpack(int64_t L, int64_t B, int64_t H, int64_t D, int64_t Smax,
                   uint16_t *key, uint16_t *value,
                   int64_t layer_begin, int64_t layer_count,
                   const int32_t *start, const int32_t *count,
                   const uint16_t *in)
{
    int64_t o = 0;
    for (int64_t l = layer_begin; l < layer_begin + layer_count; ++l)
        for (int kv = 0; kv < 2; ++kv)
            for (int64_t b = 0; b < B; ++b)
                for (int64_t h = 0; h < H; ++h)
                    for (int64_t t = 0; t < count[b]; ++t)
                        for (int64_t d = 0; d < D; ++d) {
                            int64_t s = start[b] + t;
                            if (kv == 0)
                                key[oracle_key_offset(L, B, H, D, Smax, l, b, h, s, d)] = in[o];
                            else
                                value[oracle_value_offset(L, B, H, D, Smax, l, b, h, s, d)] = in[o];
                            ++o;
                        }
}

/* Per-row token ranges of one prompt-layer pack: tokens
 * [tok_begin, tok_begin + tok_count) clipped to [0, row_len_b).  A NULL
 * row_len means no clipping. */
void oracle_prompt_ranges(int64_t B, int32_t tok_begin, int32_t tok_count,
                          const int32_t *row_len, int32_t *start, int32_t *count)
{
    for (int64_t b = 0; b < B; ++b) {
        int32_t end = tok_begin + tok_count;
        if (row_len != NULL && row_len[b] < end)
            end = row_len[b];
        start[b] = tok_begin;
        count[b] = end > tok_begin ? end - tok_begin : 0;
    }
}

/* Ring restore: `steps` slots, each one single-token pack of all L layers
 * (one token per row at positions pos[j*B + b]), stored back to back in
 * step order `slot_elems` apart.  They are unpacked in ascending step order,
 * so the later of two steps that name the same position wins. */
void oracle_ring_restore(int64_t L, int64_t B, int64_t H, int64_t D, int64_t Smax,
                         uint16_t *key, uint16_t *value,
                         int64_t steps, const int32_t *pos, int64_t slot_elems,
                         const uint16_t *host)
{
    int32_t one[B > 0 ? B : 1];
    for (int64_t b = 0; b < B; ++b)
        one[b] = 1;
    for (int64_t j = 0; j < steps; ++j)
        oracle_unpack(L, B, H, D, Smax, key, value, 0, L, pos + j * B, one,
                      host + j * slot_elems);
}

/* Restart point after a failure, from acknowledgements (x, j, t): worker x's
 * replica holds microbatch j up to and including step t.  Walk the pairs in
 * processing order -- step 0 of microbatches 0..M-1, then step 1, ... -- and
 * return the first pair some worker has not acknowledged (an ack for step t
 * covers every earlier step of that microbatch).  `max_step` bounds the walk. */
void oracle_restart_point(int64_t workers, int64_t microbatches, int64_t n_acks,
                          const int64_t *ack_x, const int64_t *ack_j, const int64_t *ack_t,
                          int64_t max_step, int64_t *j_out, int64_t *t_out)
{
    for (int64_t t = 0; t <= max_step; ++t)
        for (int64_t j = 0; j < microbatches; ++j)
            for (int64_t x = 0; x < workers; ++x) {
                int covered = 0;
                for (int64_t a = 0; a < n_acks; ++a)
                    if (ack_x[a] == x && ack_j[a] == j && ack_t[a] >= t)
                        covered = 1;
                if (!covered) {
                    *j_out = j;
                    *t_out = t;
                    return;
                }
            }
    *j_out = 0;
    *t_out = max_step + 1;
}

/* Appendix E of the DejaVu summary: doubling the batch from B to 2B by
 * swapping pays when 2*N*t (two batches of B without swapping, N decode steps
 * of t each) is at least the swapped run, in which the step that holds i
 * tokens lasts max(t, i*B*C/bw) -- the compute time or the time to bring the
 * other batch's cache back -- summed for i = p .. N+p.  Returns 1 if it pays. */
int oracle_swap_pays(int64_t N, double t, int64_t p, int64_t B, double C, double bw,
                     double *lhs, double *rhs)
{
    double sum = 0.0;
    for (int64_t i = p; i <= N + p; ++i) {
        double transfer = (double)i * (double)B * C / bw;
        sum += transfer > t ? transfer : t;
    }
    *lhs = 2.0 * (double)N * t;
    *rhs = sum;
    return *lhs >= *rhs;
}

/* ---- stream_out / stream_in between partitions ---------------------------
 * A partition is six integers: {layer0, layers, head0, heads, row0, rows}.
 * The worker's cache has L = layers, H = heads, B = rows, and its local
 * (l, b, h) is the global (layer0 + l, row0 + b, head0 + h). */

/* Intersection [*lo, *hi) of [a0, a0 + an) and [b0, b0 + bn). */
static void oracle_meet(int64_t a0, int64_t an, int64_t b0, int64_t bn, int64_t *lo, int64_t *hi)
{
    *lo = a0 > b0 ? a0 : b0;
    *hi = (a0 + an) < (b0 + bn) ? (a0 + an) : (b0 + bn);
    if (*hi < *lo)
        *hi = *lo;
}

/* 16-bit elements of the piece `src` sends `dst`: 2 * layers * heads * D *
 * (sum of the source's counts over the shared rows).  `count` is per source row. */
int64_t oracle_stream_elems(const int64_t *src, const int64_t *dst, int64_t D,
                            const int32_t *count)
{
    int64_t l_lo, l_hi, h_lo, h_hi, r_lo, r_hi;
    oracle_meet(src[0], src[1], dst[0], dst[1], &l_lo, &l_hi);
    oracle_meet(src[2], src[3], dst[2], dst[3], &h_lo, &h_hi);
    oracle_meet(src[4], src[5], dst[4], dst[5], &r_lo, &r_hi);
    int64_t tokens = 0;
    for (int64_t r = r_lo; r < r_hi; ++r)
        tokens += count[r - src[4]];
    return 2 * (l_hi - l_lo) * (h_hi - h_lo) * D * tokens;
}

/* stream_out: the piece of the source cache that the destination holds, in
 * the packed order over global indices.  start/count: per source row. */
void oracle_stream_out(int64_t D, int64_t Smax, const int64_t *src, const int64_t *dst,
                       const uint16_t *key, const uint16_t *value,
                       const int32_t *start, const int32_t *count, uint16_t *out)
{
    const int64_t L = src[1], H = src[3], B = src[5];
    int64_t l_lo, l_hi, h_lo, h_hi, r_lo, r_hi;
    oracle_meet(src[0], src[1], dst[0], dst[1], &l_lo, &l_hi);
    oracle_meet(src[2], src[3], dst[2], dst[3], &h_lo, &h_hi);
    oracle_meet(src[4], src[5], dst[4], dst[5], &r_lo, &r_hi);
    int64_t o = 0;
    for (int64_t gl = l_lo; gl < l_hi; ++gl)
        for (int kv = 0; kv < 2; ++kv)
            for (int64_t gr = r_lo; gr < r_hi; ++gr)
                for (int64_t gh = h_lo; gh < h_hi; ++gh) {
                    const int64_t l = gl - src[0], b = gr - src[4], h = gh - src[2];
                    for (int64_t t = 0; t < count[b]; ++t)
                        for (int64_t d = 0; d < D; ++d) {
                            const int64_t s = start[b] + t;
                            if (kv == 0)
                                out[o] = key[oracle_key_offset(L, B, H, D, Smax, l, b, h, s, d)];
                            else
                                out[o] = value[oracle_value_offset(L, B, H, D, Smax, l, b, h, s, d)];
                            ++o;
                        }
                }
}

/* stream_in: merge the piece `src` sent into the destination cache at the
 * destination's local indices.  start/count: per destination row. */
void oracle_stream_in(int64_t D, int64_t Smax, const int64_t *dst, const int64_t *src,
                      uint16_t *key, uint16_t *value,
                      const int32_t *start, const int32_t *count, const uint16_t *in)
{
    const int64_t L = dst[1], H = dst[3], B = dst[5];
    int64_t l_lo, l_hi, h_lo, h_hi, r_lo, r_hi;
    oracle_meet(src[0], src[1], dst[0], dst[1], &l_lo, &l_hi);
    oracle_meet(src[2], src[3], dst[2], dst[3], &h_lo, &h_hi);
    oracle_meet(src[4], src[5], dst[4], dst[5], &r_lo, &r_hi);
    int64_t o = 0;
    for (int64_t gl = l_lo; gl < l_hi; ++gl)
        for (int kv = 0; kv < 2; ++kv)
            for (int64_t gr = r_lo; gr < r_hi; ++gr)
                for (int64_t gh = h_lo; gh < h_hi; ++gh) {
                    const int64_t l = gl - dst[0], b = gr - dst[4], h = gh - dst[2];
                    for (int64_t t = 0; t < count[b]; ++t)
                        for (int64_t d = 0; d < D; ++d) {
                            const int64_t s = start[b] + t;
                            if (kv == 0)
                                key[oracle_key_offset(L, B, H, D, Smax, l, b, h, s, d)] = in[o];
                            else
                                value[oracle_value_offset(L, B, H, D, Smax, l, b, h, s, d)] = in[o];
                            ++o;
                        }
                }
}

/* ---- paged pool ----------------------------------------------------------- */

/* Element offset of K(l, block, h, slot o, d) in the pool [L, NB, H, D/8, P, 8]. */
int64_t oracle_paged_key_offset(int64_t NB, int64_t H, int64_t D, int64_t P,
                                int64_t l, int64_t blk, int64_t h, int64_t o, int64_t d)
{
    return ((((l * NB + blk) * H + h) * (D / 8) + d / 8) * P + o) * 8 + d % 8;
}

/* Element offset of V(l, block, h, slot o, d) in the pool [L, NB, H, P, D]. */
int64_t oracle_paged_value_offset(int64_t NB, int64_t H, int64_t D, int64_t P,
                                  int64_t l, int64_t blk, int64_t h, int64_t o, int64_t d)
{
    return (((l * NB + blk) * H + h) * P + o) * D + d;
}

/* Gather from the pool: the packed format of oracle_pack, for rows whose
 * tokens are found through their block tables. */
void oracle_pack_paged(int64_t NB, int64_t H, int64_t D, int64_t P,
                       const uint16_t *key, const uint16_t *value,
                       int64_t layer_begin, int64_t layer_count, int64_t B,
                       const int32_t *table, int64_t stride,
                       const int32_t *start, const int32_t *count, uint16_t *out)
{
    int64_t o = 0;
    for (int64_t l = layer_begin; l < layer_begin + layer_count; ++l)
        for (int kv = 0; kv < 2; ++kv)
            for (int64_t b = 0; b < B; ++b)
                for (int64_t h = 0; h < H; ++h)
                    for (int64_t t = 0; t < count[b]; ++t) {
                        const int64_t s = start[b] + t;
                        const int64_t blk = table[b * stride + s / P];
                        const int64_t slot = s % P;
                        for (int64_t d = 0; d < D; ++d) {
                            if (kv == 0)
                                out[o] = key[oracle_paged_key_offset(NB, H, D, P, l, blk, h, slot, d)];
                            else
                                out[o] = value[oracle_paged_value_offset(NB, H, D, P, l, blk, h, slot, d)];
                            ++o;
                        }
                    }
}

/* Scatter into the pool: the inverse of oracle_pack_paged. */
void oracle_unpack_paged(int64_t NB, int64_t H, int64_t D, int64_t P,
                         uint16_t *key, uint16_t *value,
                         int64_t layer_begin, int64_t layer_count, int64_t B,
                         const int32_t *table, int64_t stride,
                         const int32_t *start, const int32_t *count, const uint16_t *in)
{
    int64_t o = 0;
    for (int64_t l = layer_begin; l < layer_begin + layer_count; ++l)
        for (int kv = 0; kv < 2; ++kv)
            for (int64_t b = 0; b < B; ++b)
                for (int64_t h = 0; h < H; ++h)
                    for (int64_t t = 0; t < count[b]; ++t) {
                        const int64_t s = start[b] + t;
                        const int64_t blk = table[b * stride + s / P];
                        const int64_t slot = s % P;
                        for (int64_t d = 0; d < D; ++d) {
                            if (kv == 0)
                                key[oracle_paged_key_offset(NB, H, D, P, l, blk, h, slot, d)] = in[o];
                            else
                                value[oracle_paged_value_offset(NB, H, D, P, l, blk, h, slot, d)] = in[o];
                            ++o;
                        }
                    }
}
