/*
 * hwkv_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU model of the per-head windowed KV
 * cache.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no code, header or table with the HIP library; the
 * two meet only through seeded inputs generated elsewhere.
 *
 * Everything floating point is accumulated in double precision over the exact
 * input values (fp32, or bf16 widened exactly).  No blocking, no fusion, no
 * reordering: each function states the definition it follows.
 *
 * Sources (web pages, cited by title and section):
 *  [HW]  "HeadWiseKV: budgeted per-head KV cache residency for hybrid
 *        long-context language models" (KnoAI write-up), sections
 *        摘要 (abstract: static per-head history windows, exact pre-serve
 *        demand, policy materialised as real per-head residency) and
 *        核心技术 2 "Grouped-Cache Runtime" (no masking of a full cache; each
 *        head's BlockTable holds ceil(window_size / block_size) blocks).
 *  [HW-M] same page, 背景动机 (full-cache memory grows as
 *        seq_len x num_heads x head_dim x 2).
 *  [P1]  "KV Cache Management in Hybrid Attention LLMs", section 2.2, item
 *        "SWA window" (only the most recent KV within a fixed window is kept).
 *  [P2]  "KV Cache Consistency Practices for Long-Context Model Inference",
 *        "Five Heterogeneous Cache Object Forms", item "SWA Window" (the
 *        window position shifts as the sequence advances).
 *
 * Readings where the pages are silent (each is also listed with the design
 * notes):
 *  - the window of a head at context L is the last w tokens [max(0,L-w), L),
 *    including the token appended last;
 *  - a head's ring holds C = ceil(w/bs)*bs token slots (whole blocks); token t
 *    lives in ring block (t div bs) mod nblocks, row t mod bs;
 *  - GQA: query head i reads kv head i div G (contiguous groups);
 *  - in a chunked prefill, keys t < P come from the cache history and keys
 *    t >= P from the chunk itself; a query row p sees [max(0,p-w+1), p].
 *
 * Return codes: 0 = ok, -1 = invalid argument, -2 = history does not cover a
 * window that a requested output needs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ELEM_F32 0
#define ELEM_BF16 1
#define ELEM_F16 2

/* IEEE-754 binary16 to double, from the format's definition: 1 sign bit, 5
 * exponent bits (bias 15), 10 fraction bits; exponent 0 holds zero and the
 * subnormals (fraction * 2^-24), exponent 31 infinities and NaNs.  Every
 * binary16 value is exact in double. */
static double f16_to_double(uint16_t h)
{
    const int sign = h >> 15, ex = (h >> 10) & 0x1f, fr = h & 0x3ff;
    double mag;
    if (ex == 0)
        mag = ldexp((double)fr, -24);
    else if (ex == 31)
        mag = fr ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + fr), ex - 25);
    return sign ? -mag : mag;
}

/* Widen one stored element to double.  bf16 is the top half of an IEEE-754
 * binary32, so widening is exact; so is binary16. */
static double load_elem(const void *base, int64_t idx, int elem)
{
    if (elem == ELEM_F32)
        return (double)((const float *)base)[idx];
    if (elem == ELEM_F16)
        return f16_to_double(((const uint16_t *)base)[idx]);
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* The widening above, exported so that it can be checked on its own. */
void hwkvref_widen(const void *src, int64_t n, int elem, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = load_elem(src, i, elem);
}

static int elem_size(int elem) { return elem == ELEM_F32 ? 4 : 2; }

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* [HW] 核心技术 2: blocks per head = ceil(window_size / block_size). */
int64_t hwkvref_blocks(int64_t window, int64_t block_size)
{
    return ceil_div(window, block_size);
}

/* Per-head block counts and, layer-major, the offset of each head's block
 * table inside one sequence's table row.  Returns blocks per sequence, or -1.
 * head_off has n_layers*n_kv_heads+1 entries. */
int64_t hwkvref_layout(int n_layers, int n_kv_heads, const int32_t *windows,
                       int block_size, int32_t *nblocks, int64_t *head_off)
{
    if (n_layers < 1 || n_kv_heads < 1 || block_size < 1)
        return -1;
    int64_t acc = 0;
    for (int64_t i = 0; i < (int64_t)n_layers * n_kv_heads; i++) {
        if (windows[i] < 1)
            return -1;
        int64_t nb = hwkvref_blocks(windows[i], block_size);
        if (nblocks)
            nblocks[i] = (int32_t)nb;
        if (head_off)
            head_off[i] = acc;
        acc += nb;
    }
    if (head_off)
        head_off[(int64_t)n_layers * n_kv_heads] = acc;
    return acc;
}

/* [HW] 摘要 + 核心技术 2: with static per-head windows the pool size is known
 * exactly before serving: n_seqs * sum over heads of
 * ceil(w/bs) * bs * head_dim * 2 (K and V) * bytes per element. */
uint64_t hwkvref_mem_estimate(int n_layers, int n_kv_heads,
                              const int32_t *windows, int block_size,
                              int head_dim, int elem_bytes, int64_t n_seqs)
{
    uint64_t per_seq = 0;
    for (int64_t i = 0; i < (int64_t)n_layers * n_kv_heads; i++) {
        uint64_t nb = (uint64_t)hwkvref_blocks(windows[i], block_size);
        per_seq += nb * (uint64_t)block_size * (uint64_t)head_dim * 2u *
                   (uint64_t)elem_bytes;
    }
    return per_seq * (uint64_t)n_seqs;
}

/* Default allocation: sequence row s of the table gets the consecutive block
 * ids [s*bps, (s+1)*bps). */
void hwkvref_default_table(int64_t n_seqs, int64_t blocks_per_seq,
                           int32_t *block_ids)
{
    for (int64_t s = 0; s < n_seqs; s++)
        for (int64_t j = 0; j < blocks_per_seq; j++)
            block_ids[s * blocks_per_seq + j] = (int32_t)(s * blocks_per_seq + j);
}

/* Ring placement of absolute token position t in a head with nblocks blocks:
 * ring block index (t div bs) mod nblocks, row t mod bs. */
void hwkvref_ring_slot(int64_t t, int block_size, int nblocks, int32_t *ring_block,
                       int32_t *row)
{
    *ring_block = (int32_t)((t / block_size) % nblocks);
    *row = (int32_t)(t % block_size);
}

/* Byte offset of element 0 of row `row` of the K (kv=0) or V (kv=1) half of
 * physical block `block`.  A block is [K rows][V rows], each bs x head_dim. */
static uint64_t pool_row_offset(int64_t block, int kv, int row, int block_size,
                                int head_dim, int eb)
{
    return ((((uint64_t)block * 2u + (uint64_t)kv) * (uint64_t)block_size +
             (uint64_t)row) *
            (uint64_t)head_dim) *
           (uint64_t)eb;
}

/* Append n_new tokens at positions [pos0[b], pos0[b]+n_new) for layers
 * [layer_begin, layer_begin+n_layers) of every sequence b.  k and v are
 * [n_layers][n_seqs][n_new][n_kv_heads][head_dim] raw elements.  For each head
 * with ring capacity C only the newest C of the new tokens are stored (an
 * older one would be overwritten by a newer one with the same residue within
 * this call); every other byte of the pool is left as it was.  Pure byte
 * copies: no arithmetic on values. */
int hwkvref_append(uint8_t *pool, uint64_t pool_bytes, const int32_t *block_ids,
                   int64_t table_rows, const int32_t *windows, int n_layers_total,
                   int n_kv_heads, int block_size, int head_dim, int elem,
                   int layer_begin, int n_layers, int n_seqs,
                   const int32_t *seq_slots, const int64_t *pos0, int n_new,
                   const uint8_t *k, const uint8_t *v)
{
    const int eb = elem_size(elem);
    if (layer_begin < 0 || n_layers < 0 || layer_begin + n_layers > n_layers_total)
        return -1;
    const int64_t n_heads = (int64_t)n_layers_total * n_kv_heads;
    if (n_heads < 1)
        return -1;
    int32_t *nblocks = (int32_t *)malloc((size_t)n_heads * sizeof(int32_t));
    int64_t *head_off = (int64_t *)malloc((size_t)(n_heads + 1) * sizeof(int64_t));
    int64_t bps = (nblocks && head_off)
                      ? hwkvref_layout(n_layers_total, n_kv_heads, windows,
                                       block_size, nblocks, head_off)
                      : -1;
    int rc = bps < 0 ? -1 : 0;
    const uint64_t row_bytes = (uint64_t)head_dim * (uint64_t)eb;
    for (int li = 0; li < n_layers && rc == 0; li++) {
        int layer = layer_begin + li;
        for (int b = 0; b < n_seqs && rc == 0; b++) {
            int64_t slot = seq_slots ? seq_slots[b] : b;
            if (slot < 0 || slot >= table_rows) {
                rc = -1;
                break;
            }
            int64_t P = pos0[b];
            for (int h = 0; h < n_kv_heads && rc == 0; h++) {
                int64_t hi = (int64_t)layer * n_kv_heads + h;
                int64_t C = (int64_t)nblocks[hi] * block_size;
                int64_t first = P + n_new - C;
                if (first < P)
                    first = P;
                for (int64_t t = first; t < P + n_new && rc == 0; t++) {
                    int32_t rb, row;
                    hwkvref_ring_slot(t, block_size, nblocks[hi], &rb, &row);
                    int64_t block = block_ids[slot * bps + head_off[hi] + rb];
                    uint64_t src = (((((uint64_t)li * n_seqs + b) * n_new +
                                      (uint64_t)(t - P)) *
                                     n_kv_heads) +
                                    h) *
                                   row_bytes;
                    for (int kv = 0; kv < 2; kv++) {
                        uint64_t dst = pool_row_offset(block, kv, row, block_size,
                                                       head_dim, eb);
                        if (dst + row_bytes > pool_bytes) {
                            rc = -1;
                            break;
                        }
                        memcpy(pool + dst, (kv == 0 ? k : v) + src, row_bytes);
                    }
                }
            }
        }
    }
    free(nblocks);
    free(head_off);
    return rc;
}

/* softmax(scale * q.k_t) weighted sum of v_t over a set of positions, all in
 * double.  `pos_ok(t)` is expressed by the [t_lo, t_hi) range and an optional
 * mask range: positions outside [m_lo, m_hi) get score -inf (weight 0). */
static void attend(const double *qv, int d, double scale, int64_t t_lo,
                   int64_t t_hi, int64_t m_lo, int64_t m_hi,
                   const void *ksrc, const void *vsrc, int elem,
                   int64_t (*row_index)(const void *ctx, int64_t t),
                   const void *ctx, double *out, double *scores)
{
    double mx = -INFINITY;
    for (int64_t t = t_lo; t < t_hi; t++) {
        double s;
        if (t < m_lo || t >= m_hi) {
            s = -INFINITY;
        } else {
            int64_t r = row_index(ctx, t);
            s = 0.0;
            for (int i = 0; i < d; i++)
                s += qv[i] * load_elem(ksrc, r * d + i, elem);
            s *= scale;
        }
        scores[t - t_lo] = s;
        if (s > mx)
            mx = s;
    }
    double den = 0.0;
    for (int i = 0; i < d; i++)
        out[i] = 0.0;
    for (int64_t t = t_lo; t < t_hi; t++) {
        double s = scores[t - t_lo];
        if (s == -INFINITY)
            continue;
        double p = exp(s - mx);
        den += p;
        int64_t r = row_index(ctx, t);
        for (int i = 0; i < d; i++)
            out[i] += p * load_elem(vsrc, r * d + i, elem);
    }
    for (int i = 0; i < d; i++)
        out[i] /= den;
}

/* Row of the logical history [base, base+T) of one (layer, seq, kv head): the
 * history is stored [T][n_kv_heads][d]; row index counts d-element rows. */
typedef struct {
    int64_t base, head, n_kv_heads, seq_off_rows;
} hist_ctx;

static int64_t hist_row(const void *c, int64_t t)
{
    const hist_ctx *h = (const hist_ctx *)c;
    return h->seq_off_rows + (t - h->base) * h->n_kv_heads + h->head;
}

static int decode_common(int masked, int n_layers, int n_seqs, int n_kv_heads,
                         int group, int head_dim, int elem, const int32_t *windows,
                         const int64_t *ctx_len, const void *q, const void *k_hist,
                         const void *v_hist, const int64_t *hist_base, int64_t T,
                         double scale, double *out)
{
    if (n_layers < 1 || n_seqs < 1 || n_kv_heads < 1 || group < 1 || head_dim < 1)
        return -1;
    const int n_q = n_kv_heads * group;
    /* validate coverage first, so that nothing is computed on bad input */
    for (int l = 0; l < n_layers; l++)
        for (int b = 0; b < n_seqs; b++)
            for (int h = 0; h < n_kv_heads; h++) {
                int64_t L = ctx_len[b], w = windows[l * n_kv_heads + h];
                int64_t lo = L - w > 0 ? L - w : 0;
                if (L < 1 || w < 1)
                    return -1;
                if (masked) {
                    if (hist_base[b] != 0 || T < L)
                        return -2;
                } else if (hist_base[b] > lo || hist_base[b] + T < L) {
                    return -2;
                }
            }
    int rc = 0;
    const int64_t n_items = (int64_t)n_layers * n_seqs * n_q;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t it = 0; it < n_items; it++) {
        int l = (int)(it / ((int64_t)n_seqs * n_q));
        int b = (int)((it / n_q) % n_seqs);
        int i = (int)(it % n_q);
        int h = i / group; /* GQA: contiguous groups */
        int64_t L = ctx_len[b], w = windows[l * n_kv_heads + h];
        int64_t lo = L - w > 0 ? L - w : 0; /* the last w tokens, [lo, L) */
        double qv[1024];
        double *scores = NULL;
        int64_t span = masked ? L : (L - lo);
        /* scratch for the scores of one row */
        double stack_scores[4096];
        double *heap = NULL;
        if (span <= 4096) {
            scores = stack_scores;
        } else {
            heap = (double *)malloc((size_t)span * sizeof(double));
            scores = heap;
        }
        if (!scores || head_dim > 1024) {
            rc = -1;
            free(heap);
            continue;
        }
        int64_t qoff = (((int64_t)l * n_seqs + b) * n_q + i) * head_dim;
        for (int e = 0; e < head_dim; e++)
            qv[e] = load_elem(q, qoff + e, elem);
        hist_ctx hc;
        hc.base = hist_base[b];
        hc.head = h;
        hc.n_kv_heads = n_kv_heads;
        hc.seq_off_rows = ((int64_t)l * n_seqs + b) * T * n_kv_heads;
        double *o = out + qoff;
        if (masked) /* O8: all of [0, L), keys outside the window masked */
            attend(qv, head_dim, scale, 0, L, lo, L, k_hist, v_hist, elem,
                   hist_row, &hc, o, scores);
        else /* O6: materialise only the window [lo, L) */
            attend(qv, head_dim, scale, lo, L, lo, L, k_hist, v_hist, elem,
                   hist_row, &hc, o, scores);
        free(heap);
    }
    return rc;
}

/* Decode attention at context length ctx_len[b] (the newest token, at
 * position ctx_len[b]-1, already appended).  For query head i of layer l and
 * sequence b, with kv head h = i div group and window w = windows[l][h]:
 *   o = sum_{t in [max(0,L-w), L)} softmax_t(scale * q_i . k_t) v_t.
 * q: [n_layers][n_seqs][n_kv_heads*group][head_dim]; k_hist, v_hist:
 * [n_layers][n_seqs][T][n_kv_heads][head_dim] holding positions
 * [hist_base[b], hist_base[b]+T); out: double, same shape as q. */
int hwkvref_decode(int n_layers, int n_seqs, int n_kv_heads, int group,
                   int head_dim, int elem, const int32_t *windows,
                   const int64_t *ctx_len, const void *q, const void *k_hist,
                   const void *v_hist, const int64_t *hist_base, int64_t T,
                   double scale, double *out)
{
    return decode_common(0, n_layers, n_seqs, n_kv_heads, group, head_dim, elem,
                         windows, ctx_len, q, k_hist, v_hist, hist_base, T, scale,
                         out);
}

/* The masked twin: attention over the whole history [0, L) with the scores
 * of positions before L-w set to -inf.  Requires hist_base == 0, T >= L. */
int hwkvref_decode_masked(int n_layers, int n_seqs, int n_kv_heads, int group,
                          int head_dim, int elem, const int32_t *windows,
                          const int64_t *ctx_len, const void *q,
                          const void *k_hist, const void *v_hist,
                          const int64_t *hist_base, int64_t T, double scale,
                          double *out)
{
    return decode_common(1, n_layers, n_seqs, n_kv_heads, group, head_dim, elem,
                         windows, ctx_len, q, k_hist, v_hist, hist_base, T, scale,
                         out);
}

/* Key/value row source for a prefill query: positions < P come from the
 * cache history [hist_base, hist_base+T), positions >= P from the chunk. */
typedef struct {
    int64_t P, base, T, head, n_kv_heads, seq, n_chunk;
} pf_ctx;

static int64_t pf_hist_row(const void *c, int64_t t)
{
    const pf_ctx *p = (const pf_ctx *)c;
    return (p->seq * p->T + (t - p->base)) * p->n_kv_heads + p->head;
}

static int64_t pf_chunk_row(const void *c, int64_t t)
{
    const pf_ctx *p = (const pf_ctx *)c;
    return (p->seq * p->n_chunk + (t - p->P)) * p->n_kv_heads + p->head;
}

/* Chunked prefill for one layer.  Sequence b has history [0, P) with
 * P = pos0[b] and receives n_chunk new tokens at [P, P+n_chunk).  Query row
 * r (position p = P + r) of query head i attends to kv head h = i div group
 * over [max(0, p-w+1), p], causal and windowed.  Only the rows listed in
 * rows[0..n_rows) are computed.
 * q: [n_seqs][n_chunk][n_q][d]; k_chunk, v_chunk: [n_seqs][n_chunk][n_kv][d];
 * k_hist, v_hist: [n_seqs][T][n_kv][d] for positions [hist_base[b], +T);
 * out: double [n_seqs][n_rows][n_q][d]. */
int hwkvref_prefill(int n_seqs, int n_kv_heads, int group, int head_dim,
                    int elem, const int32_t *windows, const int64_t *pos0,
                    int n_chunk, const void *q, const void *k_chunk,
                    const void *v_chunk, const void *k_hist, const void *v_hist,
                    const int64_t *hist_base, int64_t T, int n_rows,
                    const int32_t *rows, double scale, double *out)
{
    if (n_seqs < 1 || n_kv_heads < 1 || group < 1 || head_dim < 1 ||
        head_dim > 1024 || n_chunk < 1 || n_rows < 0)
        return -1;
    const int n_q = n_kv_heads * group;
    for (int b = 0; b < n_seqs; b++)
        for (int r = 0; r < n_rows; r++) {
            if (rows[r] < 0 || rows[r] >= n_chunk)
                return -1;
            for (int h = 0; h < n_kv_heads; h++) {
                int64_t P = pos0[b], p = P + rows[r], w = windows[h];
                int64_t lo = p - w + 1 > 0 ? p - w + 1 : 0;
                if (P < 0 || w < 1)
                    return -1;
                if (lo < P && (hist_base[b] > lo || hist_base[b] + T < P))
                    return -2;
            }
        }
    int rc = 0;
    const int64_t n_items = (int64_t)n_seqs * n_rows * n_q;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t it = 0; it < n_items; it++) {
        int b = (int)(it / ((int64_t)n_rows * n_q));
        int r = (int)((it / n_q) % n_rows);
        int i = (int)(it % n_q);
        int h = i / group;
        int64_t P = pos0[b], p = P + rows[r], w = windows[h];
        int64_t lo = p - w + 1 > 0 ? p - w + 1 : 0; /* window [lo, p] */
        int64_t span = p + 1 - lo;
        double *scores = (double *)malloc((size_t)span * sizeof(double));
        if (!scores) {
            rc = -1;
            continue;
        }
        double qv[1024];
        int64_t qoff = (((int64_t)b * n_chunk + rows[r]) * n_q + i) * head_dim;
        for (int e = 0; e < head_dim; e++)
            qv[e] = load_elem(q, qoff + e, elem);
        pf_ctx pc = {P, hist_base[b], T, h, n_kv_heads, b, n_chunk};
        double *o = out + (((int64_t)b * n_rows + r) * n_q + i) * head_dim;
        /* Two sources: attend over the union by hand, in double.  First the
         * scores of every position, then one softmax over all of them. */
        double mx = -INFINITY;
        for (int64_t t = lo; t <= p; t++) {
            const void *ks = t < P ? k_hist : k_chunk;
            int64_t row = t < P ? pf_hist_row(&pc, t) : pf_chunk_row(&pc, t);
            double s = 0.0;
            for (int e = 0; e < head_dim; e++)
                s += qv[e] * load_elem(ks, row * head_dim + e, elem);
            s *= scale;
            scores[t - lo] = s;
            if (s > mx)
                mx = s;
        }
        double den = 0.0;
        for (int e = 0; e < head_dim; e++)
            o[e] = 0.0;
        for (int64_t t = lo; t <= p; t++) {
            const void *vs = t < P ? v_hist : v_chunk;
            int64_t row = t < P ? pf_hist_row(&pc, t) : pf_chunk_row(&pc, t);
            double pw = exp(scores[t - lo] - mx);
            den += pw;
            for (int e = 0; e < head_dim; e++)
                o[e] += pw * load_elem(vs, row * head_dim + e, elem);
        }
        for (int e = 0; e < head_dim; e++)
            o[e] /= den;
        free(scores);
    }
    return rc;
}

/* Number of OpenMP threads the oracle runs on (1 without OpenMP). */
int hwkvref_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void hwkvref_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
