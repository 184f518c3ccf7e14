/*
 * oracle.c -- plain, slow fp64 reference for grouped-query attention with
 * per-head attention sinks.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU baseline
 * of the benchmark use it.  It shares no code, header or table with the HIP
 * library.
 *
 * What it computes (the definition, written out directly -- no tiling, no
 * online rescaling, no fusion):
 *
 *   "GPT-OSS on Day 0" (perplexity.ai), section "Attention: GQA with
 *   Attention Sinks": every attention head owns one pre-trained sink value
 *   that takes part in the softmax; query heads are grouped so that several
 *   of them read the same key/value head.
 *
 *   Same page, section "Kernels for GPT-OSS / Sink Attention": the sink is an
 *   extra bias term that enters the softmax next to the Q.K^T products.  The
 *   formula itself is lost from the extracted text; the reading used here is
 *   that the sink is one extra logit, in the same (natural-log) units as the
 *   scaled products sm_scale * q.k, that is NOT multiplied by sm_scale, and
 *   that has no value row.  For one query row with visible keys j < n:
 *
 *       x_j = sm_scale * sum_d q[d] * k_j[d]
 *       z   = [x_0, ..., x_{n-1}, s_h]            (append the sink logit)
 *       w   = softmax(z)                           (max-subtracted, fp64)
 *       out = sum_{j<n} w_j * v_j                  (sink column dropped)
 *
 *   Query head h reads key/value head h / G (G = group size); consecutive
 *   query heads share a key/value head.
 *
 *   Same section, split along the key length: when the key range is cut into
 *   blocks, only the first block (lowest key positions) carries the sink.  A
 *   block's state is (m, d, o): m = max of its logits (and of the sink for
 *   block 0), d = sum of exp(z - m), o = sum of exp(x_j - m) * v_j.  Blocks
 *   combine with M = max m_c, D = sum d_c exp(m_c - M),
 *   O = sum o_c exp(m_c - M), out = O / D.
 *
 *   "Fast embeddings on GPUs" (perplexity blog), section "ROSE": attention
 *   over ragged batches (no padding; sequences packed back to back and
 *   located by cumulative offsets) and over a paged key/value cache.
 *
 * Conventions (readings where the pages are silent):
 *   - causal masking is bottom-right aligned: row i of a sequence with Lq
 *     queries and Lkv keys sees keys j <= i + (Lkv - Lq);
 *   - a row with no visible key and sink = -inf has output 0 (the softmax is
 *     empty); with a finite sink the sink takes all the weight and the
 *     output is 0 too;
 *   - sink = +inf is outside the domain (result unspecified);
 *   - paged cache: K page = [Hkv][P][D] (token-major rows), V page =
 *     [Hkv][D][P] (dim-major rows); page_table[b][p] is the physical page
 *     holding tokens p*P .. p*P+P-1 of sequence b;
 *   - split-KV chunks are page aligned: with np = ceil(L/P) pages and S
 *     splits, ppc = ceil(np/S) pages per chunk, chunk c covers tokens
 *     [c*ppc*P, min((c+1)*ppc*P, L)).  An empty chunk c > 0 has state
 *     (-inf, 0, 0); an empty chunk 0 has (s, 1, 0) (or (-inf, 0, 0) when
 *     s = -inf).  Split prefill cuts each sequence's key range by the same
 *     rule (16-key units when the keys are not paged); a row's chunk then
 *     holds only the keys of the chunk that the row can see;
 *   - paged prefill (several new query tokens per sequence against the
 *     cache): kv_lens[b] counts every key in the cache, the new tokens'
 *     included, and the Lq queries are the last Lq positions, which the
 *     bottom-right causal rule above expresses.
 *
 * Element types accepted for inputs: 0 = fp32, 1 = bf16 (raw 16-bit
 * patterns, widened exactly to fp32 then fp64), 2 = fp64.  Outputs are fp64.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int thread_id(void)
{
#ifdef _OPENMP
    return omp_get_thread_num();
#else
    return 0;
#endif
}

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };

static double elem(const void *p, int dt, int64_t i)
{
    if (dt == ORC_F32)
        return (double)((const float *)p)[i];
    if (dt == ORC_BF16) {
        /* bf16 is the upper half of an IEEE binary32 pattern */
        uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return ((const double *)p)[i];
}

/*
 * Softmax over [x_0 .. x_{n-1}, sink] with the sink column dropped, then the
 * weighted sum of value rows.  vrow(j, d) addresses value element d of key j.
 */
typedef double (*value_fn)(const void *ctx, int j, int d);

static void sink_softmax_row(int n, const double *x, double sink, int dim,
                             value_fn vrow, const void *ctx, double *out)
{
    double mx = sink;
    for (int j = 0; j < n; ++j)
        if (x[j] > mx)
            mx = x[j];
    for (int d = 0; d < dim; ++d)
        out[d] = 0.0;
    if (mx == -INFINITY)            /* empty softmax: no key, sink = -inf */
        return;
    double den = exp(sink - mx);    /* the sink's share of the denominator */
    for (int j = 0; j < n; ++j)
        den += exp(x[j] - mx);
    for (int j = 0; j < n; ++j) {
        double w = exp(x[j] - mx) / den;
        for (int d = 0; d < dim; ++d)
            out[d] += w * vrow(ctx, j, d);
    }
}

/*
 * State (m, d, o) of the keys [t0, t1) of one row (logits x), the block
 * representation of the split along the key length: m = max of the block's
 * logits, and of the sink when the block carries it; d = sum of exp(z - m)
 * over the block's logits (and the sink); o = sum of exp(x_j - m) * v_j.
 * A block with nothing in it (no key, and no finite sink) is (-inf, 0, 0).
 */
static void block_state(const double *x, int64_t t0, int64_t t1, int with_sink,
                        double sink, int dim, value_fn vrow, const void *ctx,
                        double *m_out, double *d_out, double *o)
{
    double m = with_sink ? sink : -INFINITY;
    for (int64_t t = t0; t < t1; ++t)
        if (x[t] > m)
            m = x[t];
    for (int d = 0; d < dim; ++d)
        o[d] = 0.0;
    double den = 0.0;
    if (m != -INFINITY) {
        if (with_sink)
            den = exp(sink - m);
        for (int64_t t = t0; t < t1; ++t) {
            double e = exp(x[t] - m);
            den += e;
            for (int d = 0; d < dim; ++d)
                o[d] += e * vrow(ctx, (int)t, d);
        }
    }
    *m_out = m;
    *d_out = den;
}

/* Chunk c of S over a key range of length L, in units of `unit` tokens:
 * ppc = ceil(ceil(L / unit) / S) units per chunk; [t0, t1) clipped to L. */
static void chunk_range(int64_t L, int unit, int splits, int c, int64_t *t0,
                        int64_t *t1)
{
    const int64_t nu = (L + unit - 1) / unit;
    const int64_t ppc = (nu + splits - 1) / splits;
    int64_t a = (int64_t)c * ppc * unit, e = a + ppc * unit;
    *t0 = a > L ? L : a;
    *t1 = e > L ? L : e;
}

/* Sequence holding packed query token tok (cu_q prefix offsets), or -1. */
static int seq_of(const int32_t *cu_q, int batch, int64_t tok)
{
    for (int i = 0; i < batch; ++i)
        if (tok >= cu_q[i] && tok < cu_q[i + 1])
            return i;
    return -1;
}

/* Keys visible to row i of a sequence with lq queries and lkv keys. */
static int64_t visible_keys(int64_t i, int64_t lq, int64_t lkv, int causal)
{
    if (!causal)
        return lkv;
    int64_t n = i + (lkv - lq) + 1;          /* bottom-right alignment */
    return n < 0 ? 0 : (n > lkv ? lkv : n);
}

/* ---------------------------------------------------------------- prefill */

struct ragged_v {
    const void *v;
    int dt;
    int64_t row0;       /* first token of the sequence in the packed array */
    int64_t stride;     /* elements between consecutive tokens: Hkv * D    */
    int64_t head_off;   /* kv_head * D                                     */
};

static double ragged_v_at(const void *ctx, int j, int d)
{
    const struct ragged_v *c = (const struct ragged_v *)ctx;
    return elem(c->v, c->dt, (c->row0 + j) * c->stride + c->head_off + d);
}

/* One (token, head) row of ragged prefill.  Returns 0, or -1 if the token
 * does not belong to any sequence. */
static int prefill_one(const void *q, const void *k, const void *v, int dt,
                       const double *sinks, const int32_t *cu_q,
                       const int32_t *cu_kv, int batch, int hkv, int group,
                       int dim, double scale, int causal, int64_t tok, int h,
                       double *x, double *out)
{
    const int b = seq_of(cu_q, batch, tok);
    if (b < 0)
        return -1;
    const int hq = hkv * group;
    const int g = h / group;                 /* GQA: query head -> kv head */
    const int64_t lq = cu_q[b + 1] - cu_q[b];
    const int64_t lkv = cu_kv[b + 1] - cu_kv[b];
    const int64_t n = visible_keys(tok - cu_q[b], lq, lkv, causal);
    for (int64_t j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int d = 0; d < dim; ++d)
            acc += elem(q, dt, (tok * hq + h) * (int64_t)dim + d) *
                   elem(k, dt, ((cu_kv[b] + j) * hkv + g) * (int64_t)dim + d);
        x[j] = scale * acc;
    }
    struct ragged_v ctx = {v, dt, cu_kv[b], (int64_t)hkv * dim,
                           (int64_t)g * dim};
    sink_softmax_row((int)n, x, sinks[h], dim, ragged_v_at, &ctx, out);
    return 0;
}

/*
 * Selected rows of ragged prefill.
 *   q   [total_q, Hkv*G, D], k/v [total_kv, Hkv, D], element type dt
 *   sinks [Hkv*G] fp64; cu_q / cu_kv [batch+1] int32 prefix offsets
 *   rows: n_rows pairs (token index into q, query head); out [n_rows, D]
 *   max_kv: upper bound on any sequence's key count (scratch sizing)
 * Returns 0 or -1 on a bad row.
 */
int oracle_prefill_rows(const void *q, const void *k, const void *v, int dt,
                        const double *sinks, const int32_t *cu_q,
                        const int32_t *cu_kv, int batch, int hkv, int group,
                        int dim, double scale, int causal, int max_kv,
                        int64_t n_rows, const int64_t *row_tok,
                        const int32_t *row_head, double *out, double *scratch)
{
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        double *x = scratch + (int64_t)thread_id() * (max_kv > 0 ? max_kv : 1);
        if (prefill_one(q, k, v, dt, sinks, cu_q, cu_kv, batch, hkv, group,
                        dim, scale, causal, row_tok[r], row_head[r], x,
                        out + r * (int64_t)dim))
            bad = 1;
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------ paged decode */

struct paged_v {
    const void *v;
    int dt;
    const int32_t *pages;   /* this sequence's row of the page table */
    int64_t j0;             /* first token of the key range             */
    int hkv, g, dim, psz;
};

/* V page layout [Hkv][D][P]: element d of token t lives at
 * ((page*Hkv + g)*D + d)*P + t%P */
static double paged_v_at(const void *ctx, int j, int d)
{
    const struct paged_v *c = (const struct paged_v *)ctx;
    int64_t t = c->j0 + j;
    int64_t page = c->pages[t / c->psz];
    return elem(c->v, c->dt,
                ((page * c->hkv + c->g) * c->dim + d) * (int64_t)c->psz +
                    t % c->psz);
}

/* K page layout [Hkv][P][D]: logit of token t of this sequence */
static double paged_logit(const void *q, const void *k, int dt,
                          const int32_t *pages, int64_t t, int64_t qoff, int g,
                          int hkv, int dim, int psz, double scale)
{
    int64_t page = pages[t / psz];
    int64_t base = ((page * hkv + g) * psz + t % psz) * (int64_t)dim;
    double acc = 0.0;
    for (int d = 0; d < dim; ++d)
        acc += elem(q, dt, qoff + d) * elem(k, dt, base + d);
    return scale * acc;
}

/*
 * Paged decode, one query token per sequence, whole key range, for selected
 * (sequence, query head) rows.
 *   q [batch, Hkv*G, D]; k_cache [num_pages, Hkv, P, D];
 *   v_cache [num_pages, Hkv, D, P]; page_table [batch, max_pages];
 *   kv_lens [batch]; rows: n_rows pairs (row_b, row_h); out [n_rows, D].
 *   scratch: oracle_max_threads() * max_len doubles.
 */
int oracle_decode_paged_rows(const void *q, const void *kc, const void *vc,
                             int dt, const int32_t *page_table,
                             const int32_t *kv_lens, const double *sinks,
                             int batch, int max_pages, int hkv, int group,
                             int dim, int psz, double scale, int max_len,
                             int64_t n_rows, const int32_t *row_b,
                             const int32_t *row_h, double *out,
                             double *scratch)
{
    const int hq = hkv * group;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int b = row_b[r], h = row_h[r];
        if (b < 0 || b >= batch || h < 0 || h >= hq || kv_lens[b] > max_len) {
            bad = 1;
            continue;
        }
        double *x = scratch + (int64_t)thread_id() * (max_len > 0 ? max_len : 1);
        const int32_t *pages = page_table + (int64_t)b * max_pages;
        const int g = h / group;            /* GQA: query head -> kv head */
        const int64_t L = kv_lens[b];
        const int64_t qoff = ((int64_t)b * hq + h) * dim;
        for (int64_t t = 0; t < L; ++t)
            x[t] = paged_logit(q, kc, dt, pages, t, qoff, g, hkv, dim, psz,
                               scale);
        struct paged_v ctx = {vc, dt, pages, 0, hkv, g, dim, psz};
        sink_softmax_row((int)L, x, sinks[h], dim, paged_v_at, &ctx,
                         out + r * (int64_t)dim);
    }
    return bad ? -1 : 0;
}

/*
 * Split-KV partial states of paged decode for selected rows; only the first
 * block carries the sink.  Outputs m, d [n_rows, S] and o [n_rows, S, D], fp64,
 * m in natural-log units, o unnormalised (relative to m).
 *   scratch: oracle_max_threads() * max_len doubles.
 */
int oracle_decode_partials_rows(const void *q, const void *kc, const void *vc,
                                int dt, const int32_t *page_table,
                                const int32_t *kv_lens, const double *sinks,
                                int batch, int max_pages, int hkv, int group,
                                int dim, int psz, double scale, int splits,
                                int max_len, int64_t n_rows,
                                const int32_t *row_b, const int32_t *row_h,
                                double *m_out, double *d_out, double *o_out,
                                double *scratch)
{
    const int hq = hkv * group;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int b = row_b[r], h = row_h[r];
        if (b < 0 || b >= batch || h < 0 || h >= hq || kv_lens[b] > max_len) {
            bad = 1;
            continue;
        }
        double *x = scratch + (int64_t)thread_id() * (max_len > 0 ? max_len : 1);
        const int32_t *pages = page_table + (int64_t)b * max_pages;
        const int g = h / group;
        const int64_t L = kv_lens[b];
        const int64_t qoff = ((int64_t)b * hq + h) * dim;
        for (int64_t t = 0; t < L; ++t)
            x[t] = paged_logit(q, kc, dt, pages, t, qoff, g, hkv, dim, psz,
                               scale);
        /* page-aligned chunks: ppc = ceil(ceil(L/P) / S) pages each; only
         * chunk 0 carries the sink */
        struct paged_v ctx = {vc, dt, pages, 0, hkv, g, dim, psz};
        for (int c = 0; c < splits; ++c) {
            int64_t t0, t1;
            chunk_range(L, psz, splits, c, &t0, &t1);
            const int64_t st = r * splits + c;
            block_state(x, t0, t1, c == 0, sinks[h], dim, paged_v_at, &ctx,
                        m_out + st, d_out + st, o_out + st * dim);
        }
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------- split prefill, paged prefill */

/*
 * Split-KV partial states of ragged prefill for selected (token, head) rows.
 * The key range of each sequence is cut by the chunk rule above (units of
 * `unit` keys, ppc = ceil(ceil(Lkv / unit) / S)); a row's chunk c holds the
 * chunk's keys that the row can see, and only chunk 0 carries the sink.
 * Layouts as in oracle_prefill_rows; m, d [n_rows, S], o [n_rows, S, D].
 */
int oracle_prefill_partials_rows(const void *q, const void *k, const void *v,
                                 int dt, const double *sinks,
                                 const int32_t *cu_q, const int32_t *cu_kv,
                                 int batch, int hkv, int group, int dim,
                                 double scale, int causal, int unit, int splits,
                                 int max_kv, int64_t n_rows,
                                 const int64_t *row_tok, const int32_t *row_head,
                                 double *m_out, double *d_out, double *o_out,
                                 double *scratch)
{
    const int hq = hkv * group;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t tok = row_tok[r];
        const int h = row_head[r];
        const int b = seq_of(cu_q, batch, tok);
        if (b < 0 || h < 0 || h >= hq) {
            bad = 1;
            continue;
        }
        double *x = scratch + (int64_t)thread_id() * (max_kv > 0 ? max_kv : 1);
        const int g = h / group;
        const int64_t lkv = cu_kv[b + 1] - cu_kv[b];
        const int64_t n = visible_keys(tok - cu_q[b], cu_q[b + 1] - cu_q[b], lkv,
                                       causal);
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int d = 0; d < dim; ++d)
                acc += elem(q, dt, (tok * hq + h) * (int64_t)dim + d) *
                       elem(k, dt, ((cu_kv[b] + j) * hkv + g) * (int64_t)dim + d);
            x[j] = scale * acc;
        }
        struct ragged_v ctx = {v, dt, cu_kv[b], (int64_t)hkv * dim,
                               (int64_t)g * dim};
        for (int c = 0; c < splits; ++c) {
            int64_t t0, t1;
            chunk_range(lkv, unit, splits, c, &t0, &t1);
            if (t1 > n)
                t1 = n;             /* keys past the row's causal limit */
            if (t0 > t1)
                t0 = t1;
            const int64_t st = r * splits + c;
            block_state(x, t0, t1, c == 0, sinks[h], dim, ragged_v_at, &ctx,
                        m_out + st, d_out + st, o_out + st * dim);
        }
    }
    return bad ? -1 : 0;
}

/*
 * Paged prefill: several query tokens per sequence against the paged cache
 * (chunked prefill; "Fast embeddings on GPUs", section "ROSE").  Sequence b
 * has Lq = cu_q[b+1] - cu_q[b] query tokens and Lkv = kv_lens[b] keys in the
 * cache, the queries being the last Lq positions for the causal mask.
 *   q [total_q, Hkv*G, D]; k_cache [num_pages, Hkv, P, D];
 *   v_cache [num_pages, Hkv, D, P]; page_table [batch, max_pages].
 * splits == 0: full result into out [n_rows, D].  splits >= 1: partial
 * states into m, d [n_rows, S] and o [n_rows, S, D], chunks of whole pages
 * as in oracle_decode_partials_rows, clipped to each row's visible keys.
 *   scratch: oracle_max_threads() * max_len doubles.
 */
int oracle_prefill_paged_rows(const void *q, const void *kc, const void *vc,
                              int dt, const int32_t *page_table,
                              const int32_t *cu_q, const int32_t *kv_lens,
                              const double *sinks, int batch, int max_pages,
                              int hkv, int group, int dim, int psz, double scale,
                              int causal, int splits, int max_len,
                              int64_t n_rows, const int64_t *row_tok,
                              const int32_t *row_head, double *out,
                              double *m_out, double *d_out, double *o_out,
                              double *scratch)
{
    const int hq = hkv * group;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t tok = row_tok[r];
        const int h = row_head[r];
        const int b = seq_of(cu_q, batch, tok);
        if (b < 0 || h < 0 || h >= hq || kv_lens[b] > max_len ||
            kv_lens[b] > (int64_t)max_pages * psz) {
            bad = 1;
            continue;
        }
        double *x = scratch + (int64_t)thread_id() * (max_len > 0 ? max_len : 1);
        const int32_t *pages = page_table + (int64_t)b * max_pages;
        const int g = h / group;
        const int64_t lkv = kv_lens[b];
        const int64_t n = visible_keys(tok - cu_q[b], cu_q[b + 1] - cu_q[b], lkv,
                                       causal);
        const int64_t qoff = (tok * hq + h) * (int64_t)dim;
        for (int64_t t = 0; t < n; ++t)
            x[t] = paged_logit(q, kc, dt, pages, t, qoff, g, hkv, dim, psz,
                               scale);
        struct paged_v ctx = {vc, dt, pages, 0, hkv, g, dim, psz};
        if (splits == 0) {
            sink_softmax_row((int)n, x, sinks[h], dim, paged_v_at, &ctx,
                             out + r * (int64_t)dim);
            continue;
        }
        for (int c = 0; c < splits; ++c) {
            int64_t t0, t1;
            chunk_range(lkv, psz, splits, c, &t0, &t1);
            if (t1 > n)
                t1 = n;
            if (t0 > t1)
                t0 = t1;
            const int64_t st = r * splits + c;
            block_state(x, t0, t1, c == 0, sinks[h], dim, paged_v_at, &ctx,
                        m_out + st, d_out + st, o_out + st * dim);
        }
    }
    return bad ? -1 : 0;
}

/*
 * Merge of split-KV partial states: rows x splits states of (m, d, o[D]).
 * out [rows, D] fp64.  A row whose states all have m = -inf gets 0.
 */
int oracle_merge(const double *m, const double *d, const double *o, int64_t rows,
                 int splits, int dim, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double M = -INFINITY;
        for (int c = 0; c < splits; ++c)
            if (m[r * splits + c] > M)
                M = m[r * splits + c];
        double *y = out + r * dim;
        for (int k = 0; k < dim; ++k)
            y[k] = 0.0;
        if (M == -INFINITY)
            continue;
        double D = 0.0;
        for (int c = 0; c < splits; ++c) {
            double mc = m[r * splits + c];
            if (mc == -INFINITY)
                continue;
            double w = exp(mc - M);
            D += d[r * splits + c] * w;
            for (int k = 0; k < dim; ++k)
                y[k] += o[(r * splits + c) * dim + k] * w;
        }
        for (int k = 0; k < dim; ++k)
            y[k] /= D;
    }
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
