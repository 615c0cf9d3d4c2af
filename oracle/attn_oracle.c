/*
 * attn_oracle.c -- CPU oracle for causal grouped-query attention prefill with
 * a sliding-window lower bound and a per-head sink logit.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * GPU library is compared against.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code, header, table or constant with the GPU library.
 *
 * Everything is computed in IEEE double precision from double copies of the
 * (exactly representable) fp16/bf16 inputs.  There is no tiling, no online
 * rescaling and no reordering: every score row is materialised over all keys
 * of the sequence, the mask is applied element by element, and the softmax
 * uses the exact row maximum and natural exp().
 *
 * Sources (web pages; cited by title and section):
 *   [hip-ep #622]  "perf(gqa): support sliding windows in the fused flash
 *                  prefill kernel", ROCm/hip-ep pull request 622: commits
 *                  "fold sink into v5 epilogue", "harness: sink cases",
 *                  "window in v5", "harness: window cases", and the PR body
 *                  sections "Why", "A NaN the window introduces", "Notes".
 *   [sglang #34468] "bound the stage-1 prefix loop" / "same floor in
 *                  _fwd_kernel_unified", sgl-project/sglang pull request
 *                  34468, commit messages and the "Commit 1" body section.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - a query row q of a chunk sits at absolute position past_len + q and the
 *     sequence's valid keys are [0, past_len + sq);
 *   - window <= 0 means no window; a row keeps key k iff k <= past_len + q
 *     and (window <= 0 or k >= past_len + q - window + 1)  [hip-ep #622,
 *     "window in v5": the lower bound k < past_len + q - window + 1 is masked];
 *   - q head h reads KV head h / (H_q / H_kv) (contiguous groups);
 *   - the sink is a logit in the units of the scaled scores, one per q head;
 *     it enters the softmax denominator only  [hip-ep #622, "fold sink into
 *     v5 epilogue": exp(sink - m) is added to the denominator];
 *   - a row with no kept key outputs 0: its numerator is 0 and the
 *     denominator is clamped to a positive floor, the sink is not added
 *     [same commit: fully masked rows keep the clamped floor].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <float.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Positive floor for the softmax denominator.  Its value is unobservable:
 * a row with no kept key has numerator exactly 0, and any other row has a
 * denominator >= 1 because its maximum term is exp(0). */
#define ORACLE_DENOM_FLOOR DBL_MIN

/* ---------------------------------------------------------------------------
 * The mask.  [hip-ep #622, commit "window in v5" and PR body "Why"]: causal
 * keeps k <= past_len + q; the window adds the lower bound
 * k >= past_len + q - window + 1, so a row sees `window` keys including
 * itself and window = 1 keeps only the diagonal key ("harness: window
 * cases").  window <= 0 disables the lower bound.
 * ------------------------------------------------------------------------- */
static int kept_ex(int64_t past_len, int64_t q, int64_t k, int64_t window, int causal)
{
    int64_t pos = past_len + q;
    if (k < 0) return 0;
    if (causal && k > pos) return 0;
    if (window > 0 && k < pos - window + 1) return 0;
    return 1;
}

static int kept(int64_t past_len, int64_t q, int64_t k, int64_t window)
{
    return kept_ex(past_len, q, k, window, 1);
}

int oracle_kept(int64_t past_len, int64_t q, int64_t k, int64_t window)
{
    return kept(past_len, q, k, window);
}

/* Non-causal attention (sglang pull request 34468 tests its kernel "causal
 * and non-causal"): the row no longer stops at its own position; it keeps
 * every key of its sequence, k < past_len + sq, still above the window's
 * lower bound when a window is given (reading: the window's lower bound is
 * a mask of its own, independent of causality, as in the page's kernel,
 * whose window mask keeps q <= kv + SLIDING_WINDOW_SIZE alongside the
 * optional causal mask).  The key range k < skv is the caller's loop bound. */

/* ---------------------------------------------------------------------------
 * One output row.  Softmax over the kept scores and the sink logit, with
 * the sink's value vector taken as zero ([hip-ep #622, "fold sink into v5
 * epilogue"]: the sink adds exp(sink - m) to the denominator and nothing to
 * the numerator).
 *   q_row   : [d]            the query row
 *   k_head  : [s_cap, d]     keys of the KV head this q head reads
 *   v_head  : [s_cap, d]     values of that KV head
 *   skv     : number of valid keys (past_len + sq)
 *   sink    : the head's sink logit, or -INFINITY for none
 *   score   : scratch [skv]
 *   out     : [d]
 * ------------------------------------------------------------------------- */
static void attend_row(const double* q_row, const double* k_head, const double* v_head,
                       int64_t d, int64_t skv, int64_t past_len, int64_t q, int64_t window,
                       int causal, double sink, double scale, double* score, double* out,
                       double* lse)
{
    int64_t j, t;
    int any = 0;
    double m = -INFINITY, l = 0.0;

    /* 1. the full score row S[j] = scale * <q, k_j>, masked entries -inf */
    for (j = 0; j < skv; ++j) {
        if (!kept_ex(past_len, q, j, window, causal)) { score[j] = -INFINITY; continue; }
        double dot = 0.0;
        for (t = 0; t < d; ++t) dot += q_row[t] * k_head[j * d + t];
        score[j] = scale * dot;
        any = 1;
    }
    for (t = 0; t < d; ++t) out[t] = 0.0;
    /* 1b. optional log-sum-exp of the kept scores, natural log, sink left
     *     out: lse = log(sum_j exp(S_j)) over kept j, written as
     *     max + log(sum_j exp(S_j - max)); -inf for a row with no kept key.
     *     This is the quantity partial results over disjoint key ranges are
     *     merged with (sglang's "lse_extend" side output). */
    if (lse) {
        double mk = -INFINITY, sum = 0.0;
        for (j = 0; j < skv; ++j) if (score[j] > mk) mk = score[j];
        if (mk == -INFINITY) {
            *lse = -INFINITY;
        } else {
            for (j = 0; j < skv; ++j)
                if (score[j] != -INFINITY) sum += exp(score[j] - mk);
            *lse = mk + log(sum);
        }
    }
    /* 2. a row with no kept key: output 0, sink not added */
    if (!any) return;

    /* 3. exact maximum over the kept scores and the sink */
    for (j = 0; j < skv; ++j) if (score[j] > m) m = score[j];
    if (sink > m) m = sink;

    /* 4. p_j = exp(S_j - m); numerator sum_j p_j v_j; denominator
     *    sum_j p_j + exp(sink - m)                                         */
    for (j = 0; j < skv; ++j) {
        if (score[j] == -INFINITY) continue;
        double p = exp(score[j] - m);
        l += p;
        for (t = 0; t < d; ++t) out[t] += p * v_head[j * d + t];
    }
    if (sink != -INFINITY) l += exp(sink - m);
    if (l < ORACLE_DENOM_FLOOR) l = ORACLE_DENOM_FLOOR;
    for (t = 0; t < d; ++t) out[t] /= l;
}

static int check_batch(int32_t batch, const int32_t* cu_seqlens_q, const int32_t* past_len,
                       int32_t h_q, int32_t h_kv, int32_t d, int32_t s_cap)
{
    int32_t b;
    if (batch < 0 || h_q <= 0 || h_kv <= 0 || d <= 0 || s_cap < 0) return -2;
    if (h_q % h_kv != 0) return -2;
    if (batch > 0 && (!cu_seqlens_q || !past_len)) return -2;
    if (batch > 0 && cu_seqlens_q[0] != 0) return -2;
    for (b = 0; b < batch; ++b) {
        int64_t sq = (int64_t)cu_seqlens_q[b + 1] - cu_seqlens_q[b];
        if (sq < 0 || past_len[b] < 0) return -2;
        if ((int64_t)past_len[b] + sq > s_cap) return -2;
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Ragged batch of chunked prefills.
 *   q, out       : [tokens, h_q, d], tokens = cu_seqlens_q[batch]; sequence b
 *                  owns rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *   k, v         : [batch, h_kv, s_cap, d]; keys [0, past_len[b] + sq_b) valid
 *   sink         : [h_q] logits, or NULL for no sink
 *   nthreads     : OpenMP threads (<= 0: the runtime default)
 * Returns 0, or -2 on an invalid argument.
 * ------------------------------------------------------------------------- */
int oracle_attn_prefill_varlen_ex(const double* q, const double* k, const double* v,
                                  int32_t batch, const int32_t* cu_seqlens_q,
                                  const int32_t* past_len, int32_t h_q, int32_t h_kv, int32_t d,
                                  int32_t s_cap, int32_t window, int32_t causal,
                                  const double* sink, double scale, double* out, double* lse,
                                  int32_t nthreads)
{
    int64_t n_units, u;
    int32_t group;
    if (check_batch(batch, cu_seqlens_q, past_len, h_q, h_kv, d, s_cap)) return -2;
    if (batch == 0) return 0;
    if (!q || !k || !v || !out) return -2;
    group = h_q / h_kv;
    n_units = (int64_t)batch * h_q;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (u = 0; u < n_units; ++u) {
        int32_t b = (int32_t)(u / h_q), h = (int32_t)(u % h_q), g = h / group;
        int64_t sq = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
        int64_t skv = (int64_t)past_len[b] + sq;
        const double* kh = k + (((int64_t)b * h_kv + g) * s_cap) * d;
        const double* vh = v + (((int64_t)b * h_kv + g) * s_cap) * d;
        double s = sink ? sink[h] : -INFINITY;
        double* score = (double*)malloc(sizeof(double) * (size_t)(skv > 0 ? skv : 1));
        int64_t i;
        for (i = 0; i < sq; ++i) {
            int64_t tok = cu_seqlens_q[b] + i;
            attend_row(q + (tok * h_q + h) * d, kh, vh, d, skv, past_len[b], i, window,
                       causal != 0, s, scale, score, out + (tok * h_q + h) * d,
                       lse ? lse + tok * h_q + h : NULL);
        }
        free(score);
    }
    (void)nthreads;
    return 0;
}

/* Causal, with the log-sum-exp output. */
int oracle_attn_prefill_varlen_lse(const double* q, const double* k, const double* v,
                                   int32_t batch, const int32_t* cu_seqlens_q,
                                   const int32_t* past_len, int32_t h_q, int32_t h_kv, int32_t d,
                                   int32_t s_cap, int32_t window, const double* sink,
                                   double scale, double* out, double* lse, int32_t nthreads)
{
    return oracle_attn_prefill_varlen_ex(q, k, v, batch, cu_seqlens_q, past_len, h_q, h_kv, d,
                                         s_cap, window, 1, sink, scale, out, lse, nthreads);
}

/* The same without the log-sum-exp output. */
int oracle_attn_prefill_varlen(const double* q, const double* k, const double* v,
                               int32_t batch, const int32_t* cu_seqlens_q, const int32_t* past_len,
                               int32_t h_q, int32_t h_kv, int32_t d, int32_t s_cap,
                               int32_t window, const double* sink, double scale,
                               double* out, int32_t nthreads)
{
    return oracle_attn_prefill_varlen_lse(q, k, v, batch, cu_seqlens_q, past_len, h_q, h_kv, d,
                                          s_cap, window, sink, scale, out, NULL, nthreads);
}

/* ---------------------------------------------------------------------------
 * Selected rows only, for spot checks at sizes where the full oracle is too
 * slow.  Row r is (token row_tok[r], q head row_head[r]); its output goes to
 * out_rows[r * d .. r * d + d).  The arithmetic is the same attend_row().
 * ------------------------------------------------------------------------- */
int oracle_attn_rows_lse(const double* q, const double* k, const double* v,
                         int32_t batch, const int32_t* cu_seqlens_q, const int32_t* past_len,
                         int32_t h_q, int32_t h_kv, int32_t d, int32_t s_cap,
                         int32_t window, const double* sink, double scale,
                         int64_t n_rows, const int64_t* row_tok, const int32_t* row_head,
                         double* out_rows, double* lse_rows, int32_t nthreads)
{
    int64_t r, tokens;
    int32_t group;
    if (check_batch(batch, cu_seqlens_q, past_len, h_q, h_kv, d, s_cap)) return -2;
    if (n_rows == 0) return 0;
    if (!q || !k || !v || !out_rows || !row_tok || !row_head || batch == 0) return -2;
    tokens = cu_seqlens_q[batch];
    for (r = 0; r < n_rows; ++r)
        if (row_tok[r] < 0 || row_tok[r] >= tokens || row_head[r] < 0 || row_head[r] >= h_q)
            return -2;
    group = h_q / h_kv;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (r = 0; r < n_rows; ++r) {
        int64_t tok = row_tok[r];
        int32_t h = row_head[r], g = h / group, b = 0;
        while (cu_seqlens_q[b + 1] <= tok) ++b;   /* the sequence owning tok */
        {
            int64_t i = tok - cu_seqlens_q[b];
            int64_t skv = (int64_t)past_len[b] + (cu_seqlens_q[b + 1] - cu_seqlens_q[b]);
            const double* kh = k + (((int64_t)b * h_kv + g) * s_cap) * d;
            const double* vh = v + (((int64_t)b * h_kv + g) * s_cap) * d;
            double* score = (double*)malloc(sizeof(double) * (size_t)(skv > 0 ? skv : 1));
            attend_row(q + (tok * h_q + h) * d, kh, vh, d, skv, past_len[b], i, window, 1,
                       sink ? sink[h] : -INFINITY, scale, score, out_rows + r * d,
                       lse_rows ? lse_rows + r : NULL);
            free(score);
        }
    }
    (void)nthreads;
    return 0;
}

int oracle_attn_rows(const double* q, const double* k, const double* v,
                     int32_t batch, const int32_t* cu_seqlens_q, const int32_t* past_len,
                     int32_t h_q, int32_t h_kv, int32_t d, int32_t s_cap,
                     int32_t window, const double* sink, double scale,
                     int64_t n_rows, const int64_t* row_tok, const int32_t* row_head,
                     double* out_rows, int32_t nthreads)
{
    return oracle_attn_rows_lse(q, k, v, batch, cu_seqlens_q, past_len, h_q, h_kv, d, s_cap,
                                window, sink, scale, n_rows, row_tok, row_head, out_rows, NULL,
                                nthreads);
}

/* ---------------------------------------------------------------------------
 * One head under an explicit boolean mask (mask[i * skv + j] != 0 keeps key j
 * for row i).  Used to pin the fully-masked-row behaviour, which valid calls
 * of the attention entry points never produce (window >= 1 always keeps the
 * diagonal key).  [hip-ep #622, "fold sink into v5 epilogue": a row whose
 * maximum stays -inf skips the sink and keeps the clamped floor.]
 *   q [sq, d], k/v [skv, d], out [sq, d]; sink = -INFINITY for none.
 * ------------------------------------------------------------------------- */
int oracle_attn_masked(const double* q, const double* k, const double* v,
                       int32_t sq, int32_t skv, int32_t d, const uint8_t* mask,
                       double sink, double scale, double* out)
{
    int64_t i, j, t;
    if (sq < 0 || skv < 0 || d <= 0) return -2;
    if (sq == 0) return 0;
    if (!q || !out || (skv > 0 && (!k || !v || !mask))) return -2;
    for (i = 0; i < sq; ++i) {
        double m = -INFINITY, l = 0.0;
        int any = 0;
        double* o = out + i * d;
        for (t = 0; t < d; ++t) o[t] = 0.0;
        for (j = 0; j < skv; ++j) if (mask[i * skv + j]) any = 1;
        if (!any) continue;                 /* numerator 0, sink skipped */
        for (j = 0; j < skv; ++j) {
            double dot = 0.0;
            if (!mask[i * skv + j]) continue;
            for (t = 0; t < d; ++t) dot += q[i * d + t] * k[j * d + t];
            if (scale * dot > m) m = scale * dot;
        }
        if (sink > m) m = sink;
        for (j = 0; j < skv; ++j) {
            double dot = 0.0, p;
            if (!mask[i * skv + j]) continue;
            for (t = 0; t < d; ++t) dot += q[i * d + t] * k[j * d + t];
            p = exp(scale * dot - m);
            l += p;
            for (t = 0; t < d; ++t) o[t] += p * v[j * d + t];
        }
        if (sink != -INFINITY) l += exp(sink - m);
        if (l < ORACLE_DENOM_FLOOR) l = ORACLE_DENOM_FLOOR;
        for (t = 0; t < d; ++t) o[t] /= l;
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * KV tiles a Q tile must visit.  A Q tile holds the chunk rows
 * [q_first, q_last] of one sequence; KV tile t holds keys
 * [t * bkv, (t + 1) * bkv), aligned to the sequence's key 0.
 *
 * Floor  [hip-ep #622, "window in v5"; sglang #34468, "bound the stage-1
 * prefix loop"]: lower bounds are non-decreasing in q, so the first tile any
 * row can reach is the one holding the first row's lowest kept key,
 * A = past_len + q_first - window + 1, i.e. tile floor(A / bkv), clamped to 0
 * when A < 0.  With no window the floor is tile 0.
 * Ceiling: causal keys end at the last row's own position past_len + q_last,
 * so the last tile is floor((past_len + q_last) / bkv).
 * The visited set is every tile in [t_lo, t_hi].
 * ------------------------------------------------------------------------- */
void oracle_tile_range(int64_t past_len, int64_t q_first, int64_t q_last, int64_t window,
                       int64_t bkv, int64_t* t_lo, int64_t* t_hi)
{
    int64_t lo_key = 0;
    if (window > 0) {
        lo_key = past_len + q_first - window + 1;
        if (lo_key < 0) lo_key = 0;
    }
    *t_lo = lo_key / bkv;
    *t_hi = (past_len + q_last) / bkv;
}

/* Brute force: does KV tile t hold at least one key that some row of the Q
 * tile [q_first, q_last] keeps?  Scans the mask predicate as written,
 * restricted to the sequence's valid keys [0, past_len + sq). */
int oracle_tile_has_kept(int64_t past_len, int64_t sq, int64_t q_first, int64_t q_last,
                         int64_t window, int64_t bkv, int64_t t)
{
    int64_t q, kk, skv = past_len + sq;
    for (q = q_first; q <= q_last; ++q)
        for (kk = t * bkv; kk < (t + 1) * bkv && kk < skv; ++kk)
            if (kept(past_len, q, kk, window)) return 1;
    return 0;
}

/* Number of (row, key) pairs the mask keeps for a chunk of sq rows after
 * past_len cached keys.  Useful work is 4 * d flops per kept pair per head
 * (two multiply-adds per element of q.k and of p.v). */
int64_t oracle_kept_pairs(int64_t past_len, int64_t sq, int64_t window)
{
    int64_t q, total = 0;
    for (q = 0; q < sq; ++q) {
        int64_t pos = past_len + q;
        int64_t lo = (window > 0 && pos - window + 1 > 0) ? pos - window + 1 : 0;
        total += pos - lo + 1;
    }
    return total;
}
