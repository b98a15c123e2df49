/*
 * dsa.h -- C ABI of the MI355X (gfx950) DSA decode hot path.
 *
 * The path has three steps, each one entry point, plus one entry point that
 * runs all three for every row of a call (and, beside them, the cache write
 * that feeds the path, dsa_cache_write):
 *
 *   dsa_index_scores  lightning-indexer score of every cached token
 *   dsa_topk_select   exact per-row top-k over [0, L_r)
 *   dsa_mla_decode    NoPE MLA attention of a latent-absorbed query over the
 *                     selected rows of an FP8 paged 512-wide latent cache
 *   dsa_decode_k      index -> select -> attend for S sequences x K rows
 *   dsa_topk_select_pooled  the same selection over pools of kp tokens,
 *                     expanded back to token ids
 *
 * Sources: the pages describing the GLM-5.3 DSA layer of the spark_model
 * crate -- the "spark_model/layers/glm5next_dsa/layer.rs" source page (cited
 * below as layer.rs) and the rustdoc page "Struct Glm5NextDsaLayer".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Rows are sequence-major: R = num_seqs * rows_per_seq and row r belongs to
 *   sequence s = r / rows_per_seq (rustdoc of Glm5NextDsaLayer,
 *   `decode_verify_multi`). The rows of one sequence share that sequence's
 *   key cache and block-table row (layer.rs, `decode_k`, the note on the
 *   block-table row stride of zero for the rows of one sequence).
 * - L_r = seq_lens[r] is the number of tokens row r sees, positions
 *   [0, L_r); it counts the row's own token (layer.rs, `decode_k`: the
 *   sequence length handed to the gather is the position plus one).
 *   Contract: 0 <= seq_lens[r] <= shape->max_len. Kernels clamp to that
 *   range, so a value outside it cannot fault, but its results are
 *   unspecified.
 * - Every pointer argument is a DEVICE pointer owned by the caller, 16-byte
 *   aligned, to a C-contiguous array of the stated layout. The library keeps
 *   no state between calls except a thread-local error string.
 * - A call validates its arguments on the host, enqueues its kernels on
 *   `stream` (a hipStream_t; NULL is the default stream) and returns. It never
 *   allocates, frees, synchronises or copies between host and device
 *   (layer.rs: doc of the persistent `bt` workspace buffer and the five
 *   blocking host-to-device copies that `decode_k` removed), so it may be
 *   captured into a HIP graph.
 * - Return value: DSA_OK, or a negative code. On a negative code nothing was
 *   enqueued (except DSA_ELAUNCH, reported after an enqueue failed) and
 *   dsa_last_error() describes the refusal. Refusing before any launch
 *   follows layer.rs `decode_k` (lockstep, row-count and metadata checks
 *   that bail out before touching the device) and `indexer_forward`
 *   (room is checked before any write).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_OK 0
#define DSA_EINVAL (-1)       /* null or misaligned pointer, non-positive size   */
#define DSA_EUNSUPPORTED (-2) /* a shape this build has no kernel for             */
#define DSA_ERANGE (-3)       /* sizes that do not fit one another                */
#define DSA_EWORKSPACE (-4)   /* workspace null or smaller than dsa_workspace_bytes */
#define DSA_ELAUNCH (-5)      /* the HIP runtime refused a launch                 */
#define DSA_EMETADATA (-6)    /* dsa_check_metadata found out-of-contract values  */

/* `where` argument of dsa_check_metadata */
#define DSA_META_DEVICE 0     /* the arrays are device memory                     */
#define DSA_META_HOST 1       /* the arrays are host memory                       */

/*
 * Problem shape. Names follow the layer's config (layer.rs: the
 * Glm5NextDsaConfig fields kv_lora_rank, local_heads, index_heads,
 * index_head_dim, index_topk; DsaDecodePaging: num_seqs, max_blocks_per_seq,
 * block_size).
 */
typedef struct dsa_shape {
    int32_t num_seqs;           /* S >= 1                                          */
    int32_t rows_per_seq;       /* K in [1, 16]: 1 = decode, 2..8 = K-token        */
                                /* verify, up to 16 = a row group of one sequence  */
                                /* scored together (layer.rs: the prefill          */
                                /* row-group selector, groups of up to 16 rows)    */
    int32_t num_heads;          /* H in [1, 128], attention heads (one KV head)    */
    int32_t latent_dim;         /* kv_lora_rank; must be 512                       */
    int32_t index_heads;        /* Hi in [1, 32]                                   */
    int32_t index_dim;          /* D in {64, 128}                                  */
    int32_t top_k;              /* index_topk in [1, 16384]                        */
    int32_t page_size;          /* tokens per page of the latent cache, >= 1       */
    int32_t max_len;            /* ceiling on every seq_lens[r], in [1, 1<<22];    */
                                /* sizes grids and the score row stride            */
    int32_t k_capacity;         /* key-cache rows per sequence, >= max_len         */
    int32_t max_blocks_per_seq; /* block-table row stride (entries);               */
                                /* max_blocks_per_seq * page_size >= max_len       */
    int32_t num_pages;          /* physical pages in the latent cache, >= 1        */
} dsa_shape;

/*
 * Bytes of caller-owned device workspace that dsa_topk_select, dsa_mla_decode
 * and dsa_decode_k need for `shape` (selection candidates and bitmaps past
 * their on-chip capacity, per-chunk attention partials). Its contents need no initialisation: every
 * call writes each part before reading it. Calls that share one workspace
 * must not overlap.
 * Returns 0 for a shape that dsa_decode_k would refuse.
 */
size_t dsa_workspace_bytes(const dsa_shape *shape);

/*
 * Index scores (layer.rs module header: the head weights carry
 * index_heads^-0.5 and the scorer adds no scale; `select_row` and
 * `indexer_forward`: q_idx and head weights per query row, the key cache read
 * as k[raw * D + d] over the whole context):
 *
 *   scores[r, t] = sum_{h < Hi} w[r, h] * max(0, sum_{d < D} q_idx[r, h, d] * k_normed[s, t, d])
 *
 * for t in [0, L_r), s = r / K. bf16 products are accumulated in fp32 on the
 * matrix cores; the ReLU, the weights and the head sum are fp32.
 *   q_idx    [R, Hi, D] bf16
 *   w        [R, Hi]    fp32
 *   k_normed [S, k_capacity, D] bf16, token-major (D * 2 bytes per token)
 *   seq_lens [R] int32
 *   scores   [R, dsa_score_stride(shape)] fp32 (output; the row stride is
 *            max_len rounded up to a multiple of 64, so rows are 256-byte
 *            aligned; entries t >= L_r are not written)
 */
int dsa_index_scores(const dsa_shape *shape, const void *q_idx, const float *w,
                     const void *k_normed, const int32_t *seq_lens, float *scores,
                     void *stream);

/*
 * Top-k selection (layer.rs: `select_row`, top-k over [0, len); the doc of the
 * prefill row-group selector that precedes `batch_select_enabled`, which
 * orders candidates by score descending and then index ascending, a total
 * order with a unique top-k prefix). Read per token: row r selects the
 * n_r = min(top_k, L_r) tokens of [0, L_r) that come first under (score
 * descending, index ascending), with -0.0 equal to +0.0.
 *   scores   [R, dsa_score_stride(shape)] fp32 (only [0, L_r) of each row is
 *            read; NaN scores are ordered by their bit pattern and are out of
 *            contract)
 *   seq_lens [R] int32
 *   sel      [R, top_k] int32 (output): the n_r selected ids in ascending
 *            order, then -1 in every slot past n_r
 *   ws       workspace of at least dsa_workspace_bytes(shape) bytes
 * With max_len at most DSA_SELECT_DIRECT_MAX the selection is one kernel
 * that holds whole rows; longer rows take a threshold filter and a finish
 * (two kernels). The result is the same unique top-k either way.
 */
#define DSA_SELECT_DIRECT_MAX 24576
int dsa_topk_select(const dsa_shape *shape, const float *scores, const int32_t *seq_lens,
                    int32_t *sel, void *ws, size_t ws_bytes, void *stream);

/*
 * Gather-attend (layer.rs: module header, fourth trap -- Q arrives absorbed
 * into the 512-wide latent space; `attend_rows` -- one launch for every row,
 * each with its own selection row, length and block-table row; the `v_cache`
 * argument -- keys and values are the same latent; the `kv_scale` field --
 * one FP8 scale shared by reads and writes; `decode_k` -- the page of token t
 * is block_table[t / page_size], its slot t % page_size, the page stride
 * page_size * latent_dim bytes):
 *
 *   c_j = kv_scale * e4m3(latent row of token sel[r, j]),  j < n_r
 *   z_j = sm_scale * (q[r, h, :] . c_j),  p = softmax(z),  out[r, h, :] = sum_j p_j c_j
 *
 * n_r = min(top_k, L_r); a row with n_r = 0 gets a zero output.
 *   q            [R, H, 512] bf16
 *   kv_cache     [num_pages, page_size, 512] OCP E4M3 (FN) bytes
 *   block_tables [S, max_blocks_per_seq] int32 physical page ids
 *   seq_lens     [R] int32
 *   sel          [R, top_k] int32 as written by dsa_topk_select; an id outside
 *                [0, L_r) or one whose page id is outside [0, num_pages) is
 *                skipped (out of contract; never read from memory)
 *   out          [R, H, 512] bf16 (output)
 * QK and PV run as bf16 matrix-core products with fp32 accumulation; the
 * softmax is online in fp32, P is rounded to bf16 for PV. Every row's
 * arithmetic is a function of that row alone (never of R, of the other rows
 * or of scheduling), so outputs are bit-reproducible.
 */
int dsa_mla_decode(const dsa_shape *shape, const void *q, const uint8_t *kv_cache,
                   const int32_t *block_tables, const int32_t *seq_lens, const int32_t *sel,
                   float kv_scale, float sm_scale, void *out, void *ws, size_t ws_bytes,
                   void *stream);

/*
 * The whole step for S sequences x K rows (layer.rs `decode_k`: K tokens of
 * one sequence, selection per row over that row's own [0, L_r), one
 * gather-attend launch for every row; bit-identical to K serial
 * single-row calls). Runs dsa_index_scores, dsa_topk_select and
 * dsa_mla_decode with the arguments above (the selection histogram is fused
 * into the scoring pass). Row r's scores, sel and out are byte-identical to
 * those of a call with rows_per_seq = 1 that holds row r, whatever K and S.
 */
int dsa_decode_k(const dsa_shape *shape, const void *q_idx, const float *w,
                 const void *k_normed, const void *q, const uint8_t *kv_cache,
                 const int32_t *block_tables, const int32_t *seq_lens, float kv_scale,
                 float sm_scale, float *scores, int32_t *sel, void *out, void *ws,
                 size_t ws_bytes, void *stream);

/*
 * dsa_decode_k for measurement: the same kernels on the same stream, each
 * launched with hipExtLaunchKernel and a start/stop pair of caller-created
 * HIP events (hipEvent_t, created with timing), so that the span of a pair
 * is that kernel's own run. events[0..9] are the pairs of the index pass,
 * the selection's filter, its finish, the attention and the chunk merge.
 * A stage without a kernel has its two events recorded back to back in
 * stream order (their span is no kernel's): the merge when no row has more
 * than one chunk, the filter when the selection is one kernel (max_len at
 * most DSA_SELECT_DIRECT_MAX; the finish's pair then times that kernel).
 * Results are those of dsa_decode_k. Refusals as dsa_decode_k, and
 * DSA_EINVAL for a NULL event.
 */
int dsa_decode_k_timed(const dsa_shape *shape, const void *q_idx, const float *w,
                       const void *k_normed, const void *q, const uint8_t *kv_cache,
                       const int32_t *block_tables, const int32_t *seq_lens, float kv_scale,
                       float sm_scale, float *scores, int32_t *sel, void *out, void *ws,
                       size_t ws_bytes, void *stream, void *const *events);

/*
 * dsa_decode_k for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * same kernels and results as dsa_decode_k (byte for byte), with the
 * workspace taken from an array the library holds on each device instead of
 * from the caller: DSA_NOALLOC_SCRATCH_BYTES bytes per device, claimed when
 * the library's code first loads on that device and kept until the process
 * ends. The call allocates nothing. A shape whose dsa_workspace_bytes exceeds
 * the array is refused with DSA_EWORKSPACE before anything is enqueued. All
 * calls on one device share its array, so calls that may overlap on one
 * device (other streams, other threads) race and must be serialised by the
 * caller; the array needs no clearing between calls (each call writes every
 * part it reads). The first call on a device looks the array's address up
 * (hipGetSymbolAddress) with that device current.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (64u << 20)
int dsa_decode_k_noalloc(const dsa_shape *shape, const void *q_idx, const float *w,
                         const void *k_normed, const void *q, const uint8_t *kv_cache,
                         const int32_t *block_tables, const int32_t *seq_lens, float kv_scale,
                         float sm_scale, float *scores, int32_t *sel, void *out, void *stream);

/*
 * Pooled selection (the selector of the pages' own layer, on pools of kp
 * consecutive tokens) and its expansion back to token ids. layer.rs, doc of
 * the prefill row-group selector: a pool is a candidate of row r only when it
 * is complete and its last token is visible to the row's query, so the row
 * sees pools [0, L_r / kp); it takes row_select_k = min(top_k, L_r / kp)
 * pools under the total order (score descending, pool index ascending); the
 * selected pools expand to their kp tokens, and the row's visible tail (the
 * incomplete pool, tokens L_r / kp * kp .. L_r - 1) goes from slot
 * row_select_k * kp on. With kp = 1 this is dsa_topk_select.
 *   shape->top_k   pools to select (select_k); shape->max_len the token ceiling
 *   kp             tokens per pool, in [1, 1024]
 *   pool_scores    [R, dsa_pool_score_stride(shape, kp)] fp32, entries
 *                  [0, L_r / kp) read. How the pages form pool scores (their
 *                  gate and positional terms) is not on the pages: the
 *                  caller supplies them.
 *   pool_valid     [S, dsa_pool_score_stride(shape, kp)] uint8, or NULL (every
 *                  visible pool complete): the second term of the pages'
 *                  candidacy test (pool_valid[p] && end_c <= q_pos[r]); a
 *                  pool of sequence s marked 0 is no candidate of its rows.
 *                  A row then takes its top min(row_select_k, candidates)
 *                  pools; their tokens come first, the places of the pools
 *                  it could not fill are -1, and the tail still starts at
 *                  slot row_select_k * kp.
 *   seq_lens       [R] int32
 *   sel            [R, top_k * kp + kp - 1] int32 (output): the selected
 *                  pools' tokens in ascending pool order, then the tail, then
 *                  -1
 *   ws             >= dsa_pooled_workspace_bytes(shape, kp) bytes
 * Refusals: as dsa_topk_select; kp outside [1, 1024] is EUNSUPPORTED. The
 * helpers return 0 for a refused shape or kp.
 */
size_t dsa_pooled_workspace_bytes(const dsa_shape *shape, int32_t kp);
size_t dsa_pool_score_stride(const dsa_shape *shape, int32_t kp);
int dsa_topk_select_pooled(const dsa_shape *shape, int32_t kp, const float *pool_scores,
                           const uint8_t *pool_valid, const int32_t *seq_lens, int32_t *sel,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * The cache-write side that feeds the path (the step before it): row r
 * stores its token at pos = seq_lens[r] - 1 in both caches.
 *   latent: the plain RMSNorm y = x * w / sqrt(mean(x^2) + eps) of kv_a[r]
 *     (layer.rs module header, first trap: the vanilla form, no 1 + w),
 *     times 1 / kv_scale (the `kv_scale` field: the write takes 1/scale),
 *     saturated to +-448, encoded to OCP E4M3 with round-to-nearest-even and
 *     written to kv_cache[page * page_size + pos % page_size] with page =
 *     block_tables[s][pos / page_size] (the `latent_write` kernel handle;
 *     `decode_k` slot arithmetic). A page outside [0, num_pages) skips it.
 *   key: the LayerNorm with bias y = (x - mean) / sqrt(var + eps) * k_w +
 *     k_b of k_proj[r] (module header, second trap), var the population
 *     variance, stored as bf16 (nearest-even) at k_normed[s][pos]
 *     (`indexer_forward`).
 *   validity mark: valid[s][pos] = 1, written with the key row (the same
 *     condition), when valid is not NULL (`indexer_forward`: placement and
 *     the mark both from the device position, so a captured graph does not
 *     freeze the address).
 * Norm sums run in fp32. Rows with seq_lens[r] outside [1, max_len] write
 * nothing; two rows of one sequence must not name the same position.
 *   kv_a     [R, latent_dim] bf16     latent_w [latent_dim] bf16
 *   k_proj   [R, index_dim] bf16      k_w, k_b [index_dim] bf16
 *   seq_lens [R] int32                block_tables [S, max_blocks_per_seq] int32
 *   kv_cache [num_pages, page_size, latent_dim] E4M3 bytes (updated in place)
 *   k_normed [S, k_capacity, index_dim] bf16 (updated in place)
 *   valid    [S, k_capacity] uint8 (updated in place) or NULL
 * eps >= 0 and finite; kv_scale > 0 and finite.
 */
int dsa_cache_write(const dsa_shape *shape, const void *kv_a, const void *latent_w,
                    const void *k_proj, const void *k_w, const void *k_b,
                    const int32_t *seq_lens, const int32_t *block_tables, float eps,
                    float kv_scale, uint8_t *kv_cache, void *k_normed, uint8_t *valid,
                    void *stream);

/*
 * Row stride, in floats, of every scores buffer for `shape`: max_len rounded
 * up to a multiple of 64. Returns 0 for a shape the entry points refuse.
 */
size_t dsa_score_stride(const dsa_shape *shape);

/*
 * Block-table entries a paged gather can touch for k query rows starting at
 * seq_len, plus one entry of slack; block_size 0 counts as 1 (layer.rs,
 * `bt_entries_needed` and its bt_trim_tests module). Host-only helper.
 */
size_t dsa_bt_entries_needed(size_t seq_len, size_t k, size_t block_size);

/*
 * Check of the device-resident metadata that the step entry points read
 * without checking it (they cannot without a synchronisation): a test and
 * debugging aid, never on the timed path. It is the counterpart of the
 * pages' refusals before any launch (layer.rs `decode_k`: the row-count and
 * metadata checks that bail out before touching the device, and the refusal
 * of a block-table row too short for the positions it must cover).
 * Checks, for the rows and sequences of `shape`:
 *   - 0 <= seq_lens[r] <= max_len;
 *   - every block-table entry a row can reach, block_tables[s][b] for
 *     b < ceil(max_j L_{s,j} / page_size), lies in [0, num_pages);
 *   - if sel is not NULL: the first n_r = min(top_k, L_r) ids of sel[r] lie
 *     in [0, L_r) and are distinct (a selection is a set), and every slot
 *     past n_r holds -1 (the padding dsa_topk_select writes).
 * where = DSA_META_DEVICE: the arrays are device memory; they are copied to
 * the host in the order of `stream` (so they reflect the work enqueued
 * before), which this call then synchronises. where = DSA_META_HOST: the
 * arrays are host memory and nothing touches the device. Unlike the step
 * entry points this call synchronises and allocates host memory.
 * Returns DSA_OK, a refusal code for bad arguments, or DSA_EMETADATA with
 * dsa_last_error() naming the first violation and the number found.
 */
int dsa_check_metadata(const dsa_shape *shape, const int32_t *seq_lens,
                       const int32_t *block_tables, const int32_t *sel, int where,
                       void *stream);

/* Message for the last non-zero return on this thread ("" if none). */
const char *dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
