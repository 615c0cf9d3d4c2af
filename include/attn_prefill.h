/*
 * attn_prefill.h -- C ABI of the MI355X (gfx950) fused causal grouped-query
 * flash-attention prefill library (libattn_prefill.so).
 *
 * The operation.  For each sequence b, q head h (reading KV head
 * h / (h_q / h_kv)), and chunk row q in [0, sq_b) at absolute position
 * past_len[b] + q:
 *
 *   keep key k  iff  k <= past_len + q  and  (window <= 0 or
 *                                             k >= past_len + q - window + 1)
 *   s_k   = scale * <q_row, k_k>                      (kept keys only)
 *   out   = sum_k exp(s_k - m) v_k / ( sum_k exp(s_k - m) + exp(sink_h - m) )
 *
 * with m the row maximum; a row without sink drops the exp(sink_h - m) term.
 * Sources: "perf(gqa): support sliding windows in the fused flash prefill
 * kernel" (ROCm/hip-ep pull request 622), commit "window in v5" for the
 * per-row window lower bound and the KV-loop start tile, commit "fold sink
 * into v5 epilogue" for the sink in the softmax denominator and the clamped
 * denominator of fully masked rows, and the "Why" section of its body for
 * chunked prefill over a cached prefix; sgl-project/sglang pull request
 * 34468, commit "bound the stage-1 prefix loop", for the tile floor over a
 * full (unbounded) cached prefix.
 *
 * Common conventions for every entry point:
 *  - Device pointers are caller-owned HIP device allocations on the current
 *    device; the library never allocates, frees or copies device memory on
 *    this path and never copies device-to-host.
 *  - All tensors are dense row-major with the innermost dimension contiguous,
 *    and every tensor base pointer must be 16-byte aligned:
 *      q, out            [tokens, h_q, d]        tokens = sum of chunk lengths
 *      k_cache, v_cache  [batch, h_kv, s_cap, d]
 *    The caller has already written the chunk's own keys/values at cache
 *    positions [past_len[b], past_len[b] + sq_b).  A call computes from the
 *    cache positions [0, past_len[b] + sq_b) of sequence b only; apart from
 *    the tuning sweep below, it reads no other position (positions up to
 *    s_cap may hold anything, NaN included).
 *  - head_sink: device float32 [h_q] sink logits in the units of the scaled
 *    scores, or NULL for no sink.  An entry of -INFINITY disables the sink
 *    for that head.
 *  - scale multiplies q.k (typically 1/sqrt(d)).
 *  - window <= 0 means no window; window = 1 keeps only the diagonal key.
 *  - stream is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    on it and the call returns without synchronising, except the first call
 *    for a new tuning key, which runs a synchronous tuning sweep on that
 *    stream (see attn_tune_stats).
 *  - The tuning sweep (first call of a new key only; none when
 *    ATTN_PREFILL_TUNE=0 or a configuration is forced) times every kernel
 *    configuration on the caller's own buffers before the real launch.  To
 *    time a depth that stands for the deeper calls the key will also serve,
 *    it runs each sequence of a dense cache over positions
 *    [0, max(past_len[b] + sq_b, min(s_cap, 16384))) -- still inside the
 *    caller's allocation, whatever those positions hold -- while token-pool
 *    calls read only their listed keys.  It writes out (and lse and the split
 *    workspace) several times, without the sink; the real launch then
 *    overwrites them, so a successful call returns exactly the result of the
 *    call as specified.  If the sweep fails (ATTN_EHIP), out, lse and the
 *    workspace may hold a sweep's values.  Nothing outside the caller's
 *    buffers is touched and nothing is allocated.
 *  - Return codes: ATTN_OK; ATTN_DECLINED (-1): the request is valid but not
 *    supported (d not 64/128/256, dtype not f16/bf16, out dtype neither the input
 *    dtype nor f32, misaligned pointers, device not gfx950, fp16 inputs with
 *    |scale| > ln 2: fp16 q is pre-scaled by scale * log2 e in fp16, which
 *    stays finite for every fp16 q only up to that scale) -- nothing is
 *    launched and out is untouched, so the caller can fall back; ATTN_EINVAL
 *    (-2): invalid arguments (null pointers, non-positive sizes, h_q not a
 *    multiple of h_kv, past_len < 0, past_len + sq > s_cap, cu_seqlens not
 *    starting at 0 or decreasing, tile log too small); ATTN_EHIP (-3): a HIP
 *    runtime error.  attn_last_error() describes the last non-zero return of
 *    the calling thread.  No C++ exception crosses this interface.
 *  - Thread safety: calls may come from several threads; the tuning cache is
 *    guarded by a mutex.
 */
#ifndef ATTN_PREFILL_H
#define ATTN_PREFILL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ATTN_OK = 0, ATTN_DECLINED = -1, ATTN_EINVAL = -2, ATTN_EHIP = -3 };
enum { ATTN_F16 = 1, ATTN_BF16 = 2, ATTN_F32 = 3 };
enum { ATTN_FLAG_NONCAUSAL = 1 };  /* attn_prefill_split / attn_prefill_paged flags */

/* Fields of one visited-tile record (int32 each).  Every number in fields
 * 5..7 and in the per-wave fields is observed: each wave notes the tiles whose
 * scores its softmax actually consumed, and the record's union is formed from
 * those notes after the loop (never from the floor / ceiling formula). */
enum {
  ATTN_LOG_B = 0,        /* sequence index                                   */
  ATTN_LOG_H_FIRST = 1,  /* first q head of the work item                    */
  ATTN_LOG_N_HEADS = 2,  /* q heads the work item covers (h_first ...); the
                            Q tile's rows are (position, head) pairs, row r =
                            position q_first + r / n_heads, head
                            h_first + r % n_heads                            */
  ATTN_LOG_Q_FIRST = 3,  /* first chunk row of the Q tile                    */
  ATTN_LOG_Q_LAST = 4,   /* last chunk row of the Q tile (inclusive)         */
  ATTN_LOG_T_FIRST = 5,  /* lowest KV tile any wave used (-1: none)          */
  ATTN_LOG_T_LAST = 6,   /* highest KV tile any wave used (-1: none)         */
  ATTN_LOG_N_VISITED = 7,/* distinct KV tiles some wave used                 */
  ATTN_LOG_N_WAVES = 8,  /* waves reported below (<= ATTN_LOG_MAX_WAVES)      */
  ATTN_LOG_N_SPLITS = 9, /* waves per row group: wave w serves Q-tile rows
                            [W (w % R), W (w % R) + W - 1], W = rows per
                            wave, R = n_waves / n_splits, and takes the tiles
                            t of its range with
                            (t - range_first) % n_splits == w / R            */
  ATTN_LOG_PART = 10,    /* KV part of this record (attn_prefill_split)       */
  ATTN_LOG_N_PARTS = 11, /* KV parts per Q tile (n_split; 1 otherwise)       */
  ATTN_LOG_ROWS_PER_WAVE = 12, /* W above (32 or 64)                          */
  /* 13..15 reserved (0) */
  ATTN_LOG_WAVES = 16,   /* wave w: fields 16 + 3w: first tile it used (-1:
                            none), + 1: last tile it used (-1: none), + 2: how
                            many tiles it used                               */
  ATTN_LOG_MAX_WAVES = 8,
  ATTN_LOG_FIELDS = 40
};

/*
 * Optional record of the KV tiles each work item's loop visited, for
 * checking the tile floor ("window in v5": the loop starts at the first tile
 * the Q tile's first row can reach; the causal ceiling is the tile holding
 * the last row's own key).  KV tile t holds keys [t * bkv, (t + 1) * bkv) of
 * its sequence.
 *   records   device int32 [capacity * ATTN_LOG_FIELDS], caller-owned
 *   capacity  records available; tokens * h_q always suffices
 *   n_records out: records written (one per work item and KV part, in no
 *             set order)
 *   bkv       out: keys per KV tile
 *   q_rows    out: chunk rows per Q tile
 */
typedef struct attn_tile_log {
  int32_t* records;
  int64_t capacity;
  int64_t n_records;
  int32_t bkv;
  int32_t q_rows;
} attn_tile_log;

/*
 * One sequence: a chunk of sq query rows after past_len cached keys.
 *   q        [sq, h_q, d]            dtype
 *   k_cache  [1, h_kv, s_cap, d]     dtype   (keys [0, past_len + sq) valid)
 *   v_cache  [1, h_kv, s_cap, d]     dtype
 *   out      [sq, h_q, d]            out_dtype (dtype or ATTN_F32)
 * sq = 0 is a valid no-op.
 */
int attn_prefill(const void* q, const void* k_cache, const void* v_cache,
                 int32_t past_len, int32_t window, const float* head_sink, float scale,
                 void* out,
                 int32_t sq, int32_t h_q, int32_t h_kv, int32_t d, int32_t s_cap,
                 int32_t dtype, int32_t out_dtype, void* stream);

/*
 * Ragged batch: sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 * of q/out and cache slot b, with past_len[b] cached keys before its chunk.
 *   cu_seqlens_q  HOST int32 [batch + 1], cu_seqlens_q[0] = 0, non-decreasing
 *   past_len      HOST int32 [batch]
 *   tile_log      NULL, or a record to fill (see attn_tile_log)
 * Chunks of length 0 are allowed; batch = 0 is a no-op.  The metadata stays
 * on the host: nothing is copied to or from the device for it.
 */
int attn_prefill_varlen(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* cu_seqlens_q, const int32_t* past_len, int32_t batch,
                        int32_t window, const float* head_sink, float scale, void* out,
                        int32_t h_q, int32_t h_kv, int32_t d, int32_t s_cap,
                        int32_t dtype, int32_t out_dtype,
                        attn_tile_log* tile_log, void* stream);

/*
 * Ragged batch with a log-sum-exp side output and KV splits across
 * workgroups (sglang pull request 34468 names the per-row "lse_extend" output
 * that partial results over disjoint key ranges are merged with; cutting a Q
 * tile's KV range over several workgroups raises the number of workgroups
 * when a call has few Q tiles, e.g. one 512-row chunk at a tensor-parallel
 * rank's 16 q / 2 KV heads).
 *   arguments as attn_prefill_varlen, plus:
 *   lse          NULL, or DEVICE float [tokens, h_q]: per row the natural-log
 *                log-sum-exp of its kept scaled scores, log(sum_k exp(s_k)),
 *                sink EXCLUDED; -inf for a row that keeps no key.  With
 *                head_sink = NULL, (out, lse) is the standard pair that
 *                partial attentions over disjoint key sets merge by.
 *   n_split      1..64.  1: one workgroup per Q tile walks the whole KV range
 *                (workspace unused).  > 1: the KV tiles of every Q tile are
 *                cut into n_split contiguous parts (some may be empty), each
 *                run by its own workgroup; a second kernel merges the parts,
 *                folds in the sink and writes out (and lse).
 *   workspace    DEVICE buffer, 16-byte aligned, of at least
 *                attn_split_workspace_bytes(tokens, h_q, d, n_split) bytes when
 *                n_split > 1 (caller-owned; the call overwrites it; calls that
 *                share one workspace must be ordered on one stream).
 *   flags        0, or ATTN_FLAG_NONCAUSAL: every row keeps every key of its
 *                sequence, k < past_len + sq, still above the window's floor
 *                when window > 0 (sglang pull request 34468 tests its kernel
 *                "causal and non-causal"; reading: the window's lower bound is
 *                a mask of its own).  The KV loop then ends at the sequence's
 *                last key's tile for every Q tile.
 *   tile_log     records per (work item, split): the split's own tile range.
 * Errors as attn_prefill_varlen; -2 also for n_split outside 1..64 or a
 * missing / too small workspace, -1 for a misaligned workspace.
 */
int attn_prefill_split(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* cu_seqlens_q, const int32_t* past_len, int32_t batch,
                       int32_t window, const float* head_sink, float scale, void* out,
                       float* lse, int32_t h_q, int32_t h_kv, int32_t d, int32_t s_cap,
                       int32_t dtype, int32_t out_dtype, int32_t n_split, int32_t flags,
                       void* workspace, int64_t workspace_bytes, attn_tile_log* tile_log,
                       void* stream);

/*
 * attn_prefill_split without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results and errors are those
 * of attn_prefill_split (without workspace / workspace_bytes).  Differences:
 *  - The KV-split partials live in the library's own device scratch, a
 *    file-scope array of ATTN_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, held
 *    until the process ends; a call whose partials,
 *    attn_split_workspace_bytes(tokens, h_q, d, n_split), exceed it returns
 *    ATTN_EINVAL before anything is launched.
 *  - Nothing is allocated or freed, and no tuning sweep runs: the call uses
 *    the configuration its tuning key already holds, else the default one.
 *  - All calls on one GPU share that GPU's scratch: calls that may overlap
 *    in time on one GPU (different streams, different threads) race and must
 *    be ordered by the caller.  Nothing in the scratch needs to start at
 *    zero (each call writes every partial it then reads).
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((int64_t)32 << 20)
int attn_prefill_split_noalloc(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* cu_seqlens_q, const int32_t* past_len,
                               int32_t batch, int32_t window, const float* head_sink, float scale,
                               void* out, float* lse, int32_t h_q, int32_t h_kv, int32_t d,
                               int32_t s_cap, int32_t dtype, int32_t out_dtype, int32_t n_split,
                               int32_t flags, attn_tile_log* tile_log, void* stream);

/*
 * Ragged batch over a token-pool KV layout (sglang pull request 34468,
 * "Commit 1": the extend kernel reads the cached prefix through kv_indptr /
 * kv_indices into a pool of token slots, and its window-bounded variant
 * through window_kv_indptr / window_kv_indices).  Key k of sequence b -- the
 * cached prefix and the chunk's own keys alike, k < past_len[b] + sq_b -- is
 * pool row kv_indices[kv_indptr[b] + k].  A window-bounded list is the same
 * call with past_len[b] = the number of prefix keys the list keeps: both mask
 * bounds compare a key with its own row's position, so dropping prefix keys
 * no row keeps and shifting positions changes nothing.
 *   q, out       as attn_prefill_varlen ([tokens, h_q, d])
 *   k_pool, v_pool  DEVICE [n_pool, h_kv, d] (q dtype), 16-byte aligned; the
 *                caller has written the chunk's own keys / values into the
 *                rows its list names.  n_pool * h_kv * d * 2 must be at most
 *                4 GiB - 1 (else -1: pool offsets travel as 32-bit offsets).
 *   kv_indices   DEVICE int32: pool rows.  An entry outside [0, n_pool) is
 *                clamped into the pool (the read stays in bounds; the result
 *                for that key is then another row's).
 *   kv_indptr    HOST int32 [batch + 1], non-decreasing, kv_indptr[0] >= 0;
 *                sequence b needs kv_indptr[b + 1] - kv_indptr[b] >=
 *                past_len[b] + sq_b (extra entries are never read).
 *   lse, flags   as attn_prefill_split (NULL / 0 for none); no KV splits.
 * The kernels, their tile floor / ceiling and the tile log are those of the
 * dense call; only the address of each key row differs.  Errors as
 * attn_prefill_varlen, with the cache-length check replaced by the index-list
 * length check; -2 also for null kv_indptr / kv_indices or n_pool < 1.
 */
int attn_prefill_paged(const void* q, const void* k_pool, const void* v_pool, int64_t n_pool,
                       const int32_t* kv_indices, const int32_t* kv_indptr,
                       const int32_t* cu_seqlens_q, const int32_t* past_len, int32_t batch,
                       int32_t window, const float* head_sink, float scale, void* out,
                       float* lse, int32_t h_q, int32_t h_kv, int32_t d, int32_t dtype,
                       int32_t out_dtype, int32_t flags, attn_tile_log* tile_log,
                       void* stream);

/* Bytes of workspace attn_prefill_split needs (0 for n_split = 1; -1 for
 * invalid sizes): n_split * q_tokens * h_q * (d + 1) * 4. */
int64_t attn_split_workspace_bytes(int64_t q_tokens, int32_t h_q, int32_t d, int32_t n_split);

/* Text describing the last non-zero return on the calling thread ("" if none). */
const char* attn_last_error(void);

/*
 * Tuning cache ("tuning key" commit of hip-ep pull request 622: keyed on
 * (d, sq, H_q, G) rather than the growing KV length, plus the window, which
 * caps the tiles a block walks).  Here the key is (d, dtype, out dtype, q
 * tokens of the call, h_q, group size, window, batch).  The first call for a
 * key times every kernel configuration (a synchronous sweep on the caller's
 * stream, without the sink: three interleaved passes, each timing a
 * configuration over at least ~150 us of back-to-back launches, ranked by
 * the median) and keeps the fastest; later calls with the same key reuse
 * it.  Since the key leaves out the KV depth, the sweep
 * times every sequence at depth max(past_len, min(s_cap, 16384) - sq) of the
 * caller's cache (see "The tuning sweep" above), so that the choice made on a
 * shallow first chunk holds for the deep ones.  Environment: ATTN_PREFILL_TUNE=0 skips sweeps and uses the
 * default configuration; ATTN_PREFILL_CONFIG=<name> forces one.
 * Some configurations run only some calls: the streaming window one
 * ("swin_r128_kv32") needs a causal call with window > 0, one KV part, d 64
 * or 128, and a window short enough for its ring of 32-key blocks to hold
 * the keys of four consecutive Q tiles plus one window
 * ((4 q_rows + window - 2) / 32 + 2 <= 9, q_rows = 128 / gcd(group, 32)).
 * A sweep skips a configuration that does not run its call, and a call
 * forced onto one runs the default configuration instead (its tile log
 * reports that configuration's bkv and q_rows).
 */
int attn_tune_stats(int64_t* sweeps, int64_t* tuning_launches, int64_t* cached_keys);
void attn_tune_reset(void);
/* The configuration index the tuning cache holds for the key of an unsplit
 * call (its arguments; q_tokens = rows of q), or -1 if that key has not been
 * swept.  Split calls (attn_prefill_split, n_split > 1) have keys of their own. */
int32_t attn_tuned_config(int32_t d, int32_t dtype, int32_t out_dtype, int64_t q_tokens,
                          int32_t h_q, int32_t h_kv, int32_t window, int32_t batch);

/* Kernel configurations: count, name of index i (NULL if out of range), and
 * forcing one for all later calls of this process (index -1 clears). */
int32_t attn_config_count(void);
const char* attn_config_name(int32_t i);
int attn_force_config(int32_t i);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PREFILL_H */
