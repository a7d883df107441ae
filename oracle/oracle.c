/*
 * oracle.c -- plain, slow, fp64 CPU reference for the DFlash2 block-drafting
 * hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls anything here, and nothing here is shared with it.
 *
 * Every floating-point quantity is a double.  bf16 and fp32 inputs are
 * converted to double by the caller (exact).  No blocking, fusion or online
 * softmax: each function writes out the definition it cites, step by step.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "Speculative decoding" (Reflection developer docs), "How it works".
 *   [P2] "Beam 1.0 DFlash2" model card, "Model" and "Evaluation".
 *   [P3] "DFlash vs DFlash 2" (blog), sections "The problem: one expensive
 *        token at a time", "DFlash: generate the block all at once",
 *        "Conditioning on the target model", "Training with anchors".
 *
 * Readings where the pages are silent are listed next to each function.
 *
 * Return codes: 0 ok, -2 bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as   */
/* easy as 1, 2, 3", SC'11).  Written from the paper's definition: a         */
/* 4-word, 64-bit counter, a 2-word key, ten rounds of the Philox S-box with */
/* a Weyl-sequence key schedule.                                              */
/* ------------------------------------------------------------------------ */
static void mul_hi_lo_64(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo)
{
    unsigned __int128 p = (unsigned __int128)a * (unsigned __int128)b;
    *hi = (uint64_t)(p >> 64);
    *lo = (uint64_t)p;
}

void orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4])
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
    uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += W0; k1 += W1; }
        uint64_t hi0, lo0, hi1, lo1;
        mul_hi_lo_64(M0, x0, &hi0, &lo0);
        mul_hi_lo_64(M1, x2, &hi1, &lo1);
        uint64_t y0 = hi1 ^ x1 ^ k0;
        uint64_t y1 = lo1;
        uint64_t y2 = hi0 ^ x3 ^ k1;
        uint64_t y3 = lo0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* One uniform in [0,1) per (sequence seed, step, sequence, block row,
 * purpose): key = (seed, 0), counter = (step, b, row, purpose); the top 53
 * bits of the first output word, times 2^-53.  Purposes: 0 = draft draw,
 * 1 = accept test, 2 = correction or bonus draw.  (Reading: the pages name no
 * generator; this layout is this project's choice.) */
double orc_uniform(uint64_t seed, uint64_t step, uint64_t b, uint64_t row, uint64_t purpose)
{
    uint64_t ctr[4] = {step, b, row, purpose};
    uint64_t key[2] = {seed, 0};
    uint64_t out[4];
    orc_philox4x64_10(ctr, key, out);
    return (double)(out[0] >> 11) * 0x1.0p-53;
}

/* ------------------------------------------------------------------------ */
/* Block-draft attention.                                                     */
/* [P3] "DFlash: generate the block all at once": one non-causal masked pass  */
/*      over the block (anchor + masks).                                      */
/* [P3] "Conditioning on the target model", equation for Q_i, K_i, V_i:       */
/*      queries come from the draft block only; keys and values are the      */
/*      target-context rows followed by the draft-block rows; in-block        */
/*      attention is non-causal.                                              */
/* [P1] "How it works" / [P2] "Model": the context is a 4,096-token sliding  */
/*      window; [P2] "Model": 40 query heads, 8 KV heads, dimension 128.     */
/* Readings: scale is an argument (1/sqrt(d) in practice); query head h uses */
/* KV head floor(h / (HQ/HKV)); the ring holds the most recent min(len, W)   */
/* context rows in slots [0, min(len, W)) in any order (a set); Q and K are  */
/* pre-projected, so there is no position encoding inside the operation.     */
/*                                                                            */
/* q     [B, G, HQ, D]      k_blk, v_blk [B, G, HKV, D]                        */
/* k_ring, v_ring [B, HKV, W, D]        ctx_len [B]                           */
/* out   [B, G, HQ, D]      lse [B, G, HQ] (natural log, of scaled scores;    */
/*                                          may be NULL)                      */
/* ------------------------------------------------------------------------ */
int orc_block_attn(const double* q, const double* k_blk, const double* v_blk,
                   const double* k_ring, const double* v_ring, const int64_t* ctx_len,
                   double scale, int B, int G, int HQ, int HKV, int D, int W,
                   double* out, double* lse)
{
    if (B < 0 || G < 1 || HQ < 1 || HKV < 1 || D < 1 || W < 0 || HQ % HKV != 0) return -2;
    for (int b = 0; b < B; ++b) if (ctx_len[b] < 0) return -2;
    const int group = HQ / HKV;
    const int64_t units = (int64_t)B * G * HQ;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
        const int h = (int)(u % HQ);
        const int g = (int)((u / HQ) % G);
        const int b = (int)(u / ((int64_t)HQ * G));
        const int kvh = h / group;
        const int64_t n = ctx_len[b] < W ? ctx_len[b] : W;
        const int64_t nkeys = n + G;
        const double* qv = q + (((int64_t)b * G + g) * HQ + h) * D;
        double* s = (double*)malloc(sizeof(double) * (size_t)nkeys);
        if (!s) { bad = 1; continue; }
        /* scores: context rows first, then the block rows */
        for (int64_t j = 0; j < nkeys; ++j) {
            const double* kv;
            if (j < n) kv = k_ring + (((int64_t)b * HKV + kvh) * W + j) * D;
            else       kv = k_blk + (((int64_t)b * G + (j - n)) * HKV + kvh) * D;
            double acc = 0.0;
            for (int d = 0; d < D; ++d) acc += qv[d] * kv[d];
            s[j] = scale * acc;
        }
        /* softmax by its definition: max, exponentials, sum, normalise */
        double m = -INFINITY;
        for (int64_t j = 0; j < nkeys; ++j) if (s[j] > m) m = s[j];
        double sum = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) { s[j] = exp(s[j] - m); sum += s[j]; }
        double* o = out + (((int64_t)b * G + g) * HQ + h) * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) {
            const double* vv;
            if (j < n) vv = v_ring + (((int64_t)b * HKV + kvh) * W + j) * D;
            else       vv = v_blk + (((int64_t)b * G + (j - n)) * HKV + kvh) * D;
            const double p = s[j] / sum;
            for (int d = 0; d < D; ++d) o[d] += p * vv[d];
        }
        if (lse) lse[((int64_t)b * G + g) * HQ + h] = m + log(sum);
        free(s);
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Per-position top-k candidates.                                             */
/* [P3] "The candidate selector": keep the top k candidates of each          */
/* position's draft logits.  Reading: order by raw logit, descending; equal  */
/* logits ordered by lower vocabulary index.  A library sort is the step.    */
/* ------------------------------------------------------------------------ */
typedef struct { double z; int64_t i; } zi_t;

static int cmp_desc_then_index(const void* a, const void* b)
{
    const zi_t* x = (const zi_t*)a;
    const zi_t* y = (const zi_t*)b;
    if (x->z > y->z) return -1;
    if (x->z < y->z) return 1;
    return (x->i > y->i) - (x->i < y->i);
}

/* z [rows, V] -> idx, val [rows, k] */
int orc_topk(const double* z, int64_t rows, int64_t V, int k, int64_t* idx, double* val)
{
    if (rows < 0 || V < 1 || k < 1 || k > V) return -2;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        zi_t* t = (zi_t*)malloc(sizeof(zi_t) * (size_t)V);
        if (!t) { bad = 1; continue; }
        for (int64_t v = 0; v < V; ++v) { t[v].z = z[r * V + v]; t[v].i = v; }
        qsort(t, (size_t)V, sizeof(zi_t), cmp_desc_then_index);
        for (int j = 0; j < k; ++j) { idx[r * k + j] = t[j].i; val[r * k + j] = t[j].z; }
        free(t);
    }
    return bad ? -2 : 0;
}

/* argmax with the lowest index among equal maxima */
int64_t orc_argmax(const double* z, int64_t V)
{
    int64_t best = 0;
    for (int64_t v = 1; v < V; ++v) if (z[v] > z[best]) best = v;
    return best;
}

/* log sum_v exp(z_v / T) = m + log sum_v exp(z_v/T - m), m = max_v z_v/T */
double orc_logsumexp(const double* z, int64_t V, double T)
{
    double m = -INFINITY;
    for (int64_t v = 0; v < V; ++v) { double x = z[v] / T; if (x > m) m = x; }
    double s = 0.0;
    for (int64_t v = 0; v < V; ++v) s += exp(z[v] / T - m);
    return m + log(s);
}

/* Inverse-CDF categorical draw: the smallest index i whose running sum of the
 * non-negative weights (ascending index order) exceeds u * sum(w).  If
 * rounding leaves no such index, the last index with positive weight.
 * Reading: the pages say "samples"; inverse CDF with one uniform is the
 * plainest sampler that two implementations can reproduce exactly. */
int64_t orc_categorical(const double* w, int64_t V, double u)
{
    double total = 0.0;
    for (int64_t v = 0; v < V; ++v) total += w[v];
    const double target = u * total;
    double run = 0.0;
    int64_t last_pos = -1;
    for (int64_t v = 0; v < V; ++v) {
        run += w[v];
        if (w[v] > 0.0) last_pos = v;
        if (run > target && w[v] > 0.0) return v;
    }
    return last_pos;
}

/* Drafter-side step for each drafter row: top-k candidates, the row's
 * log-normaliser at temperature T, and the drafted token.  T == 0: the draft
 * is the argmax.  T > 0: the draft is drawn from softmax(z/T) with the
 * purpose-0 uniform of (seed[b], step, b, row).
 * [P3] "The problem: one expensive token at a time": the drafter proposes a
 * token y from its distribution q.
 * z [B, G, V] -> idx, val [B, G, k], lse [B, G] (T > 0 only), draft [B, G]. */
int orc_draft_rows(const double* z, int B, int G, int64_t V, int k, double T,
                   const uint64_t* seeds, uint64_t step,
                   int64_t* idx, double* val, double* lse, int64_t* draft)
{
    if (B < 0 || G < 1 || V < 1 || k < 1 || k > V || T < 0.0) return -2;
    if (T > 0.0 && !seeds) return -2;
    int rc = orc_topk(z, (int64_t)B * G, V, k, idx, val);
    if (rc) return rc;
    const int64_t rows = (int64_t)B * G;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        const double* zr = z + r * V;
        const int b = (int)(r / G), g = (int)(r % G);
        if (T == 0.0) {
            if (lse) lse[r] = NAN;
            draft[r] = orc_argmax(zr, V);
            continue;
        }
        const double L = orc_logsumexp(zr, V, T);
        if (lse) lse[r] = L;
        double* w = (double*)malloc(sizeof(double) * (size_t)V);
        if (!w) { bad = 1; continue; }
        for (int64_t v = 0; v < V; ++v) w[v] = exp(zr[v] / T - L);
        draft[r] = orc_categorical(w, V, orc_uniform(seeds[b], step, (uint64_t)b, (uint64_t)g, 0));
        free(w);
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Drafter LM head: logits, top-k, row log-normaliser and the draft draw.    */
/* [P2] "Model" and [P1] "How it works": the drafter reuses the target's    */
/* frozen LM head over the 151,936-entry vocabulary (hidden size 5,120).     */
/* [P3] "Conditioning on the target model" (diagram): the draft layers'     */
/* output goes through the target LM head.  [P3] "The candidate selector":  */
/* top-k candidates of each position; the full-vocabulary LM-head pass is   */
/* the costly part.  [P3] "The problem: one expensive token at a time": the  */
/* drafter proposes y ~ q = softmax(z / T).                                  */
/*                                                                            */
/* z = h W^T, W stored one row per vocabulary entry.  Everything computed    */
/* from z is orc_draft_rows' definition, unchanged: top-k, the              */
/* log-normaliser, and the draft (T == 0 the argmax; T > 0 one inverse-CDF   */
/* draw from softmax(z / T) over the whole row, in increasing vocabulary    */
/* order, with the row's purpose-0 uniform).  The same seeds give the same  */
/* draft as orc_draft_rows on the same logits.                               */
/*                                                                            */
/* h [n, d] and w [V, d] are bf16 bit patterns (converted exactly to double  */
/* here); row_id [n] is each row's global index r (sequence b = r / G,       */
/* block row g = r % G; NULL = 0..n-1).  -> idx, val [n, k]; lse [n] (NaN at */
/* T == 0; may be NULL); draft [n] (may be NULL); z_out [n, V] (may be NULL).*/
/* ------------------------------------------------------------------------ */
static double bf16_bits_to_double(uint16_t bits)
{
    const uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int orc_lm_head_topk(const uint16_t* h, const uint16_t* w, const int64_t* row_id, int n, int G,
                     int64_t V, int d, int k, double T, const uint64_t* seeds, uint64_t step,
                     int64_t* idx, double* val, double* lse, int64_t* draft, double* z_out)
{
    if (n < 0 || G < 1 || V < 1 || d < 1 || k < 1 || k > V || T < 0.0) return -2;
    if (T > 0.0 && draft && !seeds) return -2;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n; ++i) {
        const int64_t r = row_id ? row_id[i] : i;
        const int64_t b = r / G, g = r % G;
        double* hr = (double*)malloc(sizeof(double) * (size_t)d);
        double* z = (double*)malloc(sizeof(double) * (size_t)V);
        double* wv = (double*)malloc(sizeof(double) * (size_t)V);
        if (!hr || !z || !wv) { bad = 1; free(hr); free(z); free(wv); continue; }
        for (int j = 0; j < d; ++j) hr[j] = bf16_bits_to_double(h[(int64_t)i * d + j]);
        /* logits: one dot product per vocabulary entry */
        for (int64_t v = 0; v < V; ++v) {
            const uint16_t* wr = w + v * d;
            double acc = 0.0;
            for (int j = 0; j < d; ++j) acc += hr[j] * bf16_bits_to_double(wr[j]);
            z[v] = acc;
        }
        if (z_out) memcpy(z_out + (int64_t)i * V, z, sizeof(double) * (size_t)V);
        if (orc_topk(z, 1, V, k, idx + (int64_t)i * k, val + (int64_t)i * k)) bad = 1;
        if (T == 0.0) {
            if (lse) lse[i] = NAN;
            if (draft) draft[i] = orc_argmax(z, V);
        } else {
            const double L = orc_logsumexp(z, V, T);
            if (lse) lse[i] = L;
            if (draft) {
                for (int64_t v = 0; v < V; ++v) wv[v] = exp(z[v] / T - L);
                draft[i] = orc_categorical(wv, V, orc_uniform(seeds[b], step, (uint64_t)b,
                                                              (uint64_t)g, 0));
            }
        }
        free(hr); free(z); free(wv);
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Top-p (nucleus) truncation of a logits row.                               */
/* [P2] "Evaluation": sampled runs use temperature 0.7 and top-p 0.99.       */
/* [P3] "The problem: one expensive token at a time": verification keeps    */
/* the output distribution equal to the target's, so with top-p the target  */
/* distribution is the truncated one, and so is the drafter's proposal.     */
/* Reading: the nucleus of softmax(z/T) is the shortest prefix, in the order */
/* (logit descending, index ascending), whose probability reaches top_p;   */
/* the truncated distribution renormalises it.  Masking the logits outside  */
/* the nucleus to -inf gives exactly that distribution under softmax(z/T),  */
/* so the unchanged draws and verification run on the masked rows.          */
/* top_p >= 1 keeps every entry.                                              */
/* z [rows, V] -> z_out [rows, V] (may equal z); kept [rows] (may be NULL):  */
/* the nucleus size.                                                          */
/* ------------------------------------------------------------------------ */
int orc_top_p_mask(const double* z, int64_t rows, int64_t V, double T, double top_p,
                   double* z_out, int64_t* kept)
{
    if (rows < 0 || V < 1 || !(T > 0.0) || !(top_p > 0.0)) return -2;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        const double* zr = z + r * V;
        double* out = z_out + r * V;
        zi_t* t = (zi_t*)malloc(sizeof(zi_t) * (size_t)V);
        if (!t) { bad = 1; continue; }
        double m = -INFINITY;
        for (int64_t v = 0; v < V; ++v) if (zr[v] / T > m) m = zr[v] / T;
        /* probabilities by definition: exponentials, then the total */
        double S = 0.0;
        for (int64_t v = 0; v < V; ++v) S += exp(zr[v] / T - m);
        for (int64_t v = 0; v < V; ++v) { t[v].z = zr[v]; t[v].i = v; }
        qsort(t, (size_t)V, sizeof(zi_t), cmp_desc_then_index);
        int64_t K = V;
        if (top_p < 1.0) {
            double c = 0.0;
            for (int64_t j = 0; j < V; ++j) {
                c += exp(t[j].z / T - m) / S;
                if (c >= top_p) { K = j + 1; break; }
            }
        }
        if (kept) kept[r] = K;
        /* copy first (z_out may alias z), then mask the entries ranked after K */
        for (int64_t v = 0; v < V; ++v) out[v] = zr[v];
        for (int64_t j = K; j < V; ++j) out[t[j].i] = -INFINITY;
        free(t);
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Verification.                                                              */
/* [P3] "The problem: one expensive token at a time": the target scores the  */
/* whole block in one pass, keeps the longest valid prefix and corrects the  */
/* first rejection.  Greedy: a draft survives while it equals the target's   */
/* choice.  Sampling: accept y with probability min(1, p(y)/q(y)); on reject */
/* draw a correction from the residual proportional to [p - q]_+; when every */
/* draft survives, one bonus token from the target's next distribution.      */
/* [P2] "Evaluation": a block of 8 verifies 7 drafted tokens.                */
/*                                                                            */
/* Rows of a block (G rows): target row r (0-based) is the target's          */
/* distribution for the token after anchor + drafts[0..r-1]; rows 0..G-2     */
/* verify drafts[0..G-2], row G-1 gives the bonus.  Drafter row r is q for   */
/* drafts[r].  accept_len = j in [0, G-1]; out_tokens = drafts[0..j-1] then  */
/* one target token, the rest -1; tau = j + 1.                               */
/* ------------------------------------------------------------------------ */

/* One sequence, greedy.  zp [G, V]; drafts [G-1]. */
int orc_greedy_verify_seq(const double* zp, const int64_t* drafts, int G, int64_t V,
                          int32_t* accept_len, int64_t* out_tokens, uint8_t* accepted)
{
    if (G < 1 || V < 1) return -2;
    int j = 0;
    int leading = 1;
    for (int r = 0; r < G - 1; ++r) {
        const int ok = drafts[r] == orc_argmax(zp + (int64_t)r * V, V);
        if (accepted) accepted[r] = (uint8_t)ok;
        if (leading && ok) ++j; else leading = 0;
    }
    for (int r = 0; r < G; ++r) out_tokens[r] = -1;
    for (int r = 0; r < j; ++r) out_tokens[r] = drafts[r];
    out_tokens[j] = orc_argmax(zp + (int64_t)j * V, V);
    *accept_len = j;
    return 0;
}

/* One sequence, sampled, with the uniforms given explicitly:
 * u_acc [G-1] for the accept tests (accept iff u < min(1, r)); u_draw [G],
 * where u_draw[r] is used if the correction or bonus is drawn from row r.
 * ratio [G-1] (may be NULL) receives r = p(d)/q(d) at each draft, computed as
 * exp((zp[d] - zq[d])/T - LSE_p + LSE_q).  Reading: p and q are both at
 * temperature T; when the residual has no mass, the correction is drawn
 * from p.
 * zq == NULL: the drafts are deterministic (chosen by the candidate selector,
 * "The candidate selector"), so q is the point mass at each draft: the draft
 * is accepted with probability p(d) and the residual [p - q]_+ is p with d
 * removed. */
int orc_sampled_verify_seq_u(const double* zp, const double* zq, const int64_t* drafts,
                             int G, int64_t V, double T,
                             const double* u_acc, const double* u_draw,
                             int32_t* accept_len, int64_t* out_tokens, uint8_t* accepted,
                             double* ratio)
{
    if (G < 1 || V < 1 || !(T > 0.0)) return -2;
    int j = 0, leading = 1;
    for (int r = 0; r < G - 1; ++r) {
        const int64_t d = drafts[r];
        if (d < 0 || d >= V) return -2;
        const double Lp = orc_logsumexp(zp + (int64_t)r * V, V, T);
        double rk;
        if (zq) {
            const double Lq = orc_logsumexp(zq + (int64_t)r * V, V, T);
            rk = exp((zp[(int64_t)r * V + d] - zq[(int64_t)r * V + d]) / T - Lp + Lq);
        } else {
            rk = exp(zp[(int64_t)r * V + d] / T - Lp);  /* p(d) / 1 */
        }
        if (ratio) ratio[r] = rk;
        /* accept iff u < min(1, r).  When p(d) and q(d) are both zero, r is
         * 0/0 (NaN): the target gives d no probability, so it is rejected
         * (committing it would leave the target's distribution). */
        const int ok = rk >= 1.0 || u_acc[r] < rk;
        if (accepted) accepted[r] = (uint8_t)ok;
        if (leading && ok) ++j; else leading = 0;
    }
    double* w = (double*)malloc(sizeof(double) * (size_t)V);
    if (!w) return -2;
    const double* zpj = zp + (int64_t)j * V;
    const double Lp = orc_logsumexp(zpj, V, T);
    if (j < G - 1) {
        /* correction from the residual [p - q]_+ of the first rejected row */
        double mass = 0.0;
        if (zq) {
            const double* zqj = zq + (int64_t)j * V;
            const double Lq = orc_logsumexp(zqj, V, T);
            for (int64_t v = 0; v < V; ++v) {
                const double diff = exp(zpj[v] / T - Lp) - exp(zqj[v] / T - Lq);
                w[v] = diff > 0.0 ? diff : 0.0;
                mass += w[v];
            }
        } else {
            for (int64_t v = 0; v < V; ++v) {
                w[v] = v == drafts[j] ? 0.0 : exp(zpj[v] / T - Lp);
                mass += w[v];
            }
        }
        if (!(mass > 0.0))
            for (int64_t v = 0; v < V; ++v) w[v] = exp(zpj[v] / T - Lp);
    } else {
        /* bonus from the target's distribution after the last draft */
        for (int64_t v = 0; v < V; ++v) w[v] = exp(zpj[v] / T - Lp);
    }
    const int64_t tok = orc_categorical(w, V, u_draw[j]);
    free(w);
    for (int r = 0; r < G; ++r) out_tokens[r] = -1;
    for (int r = 0; r < j; ++r) out_tokens[r] = drafts[r];
    out_tokens[j] = tok;
    *accept_len = j;
    return 0;
}

/* Batched verify.  T == 0: greedy (zq unused, may be NULL).  T > 0: sampled
 * with the uniforms of (seeds[b], step, b, row): purpose 1 for the accept
 * test of row r, purpose 2 for a correction or bonus drawn from row r;
 * zq == NULL means deterministic drafts (point-mass q, see above).
 * zp, zq [B, G, V]; drafts [B, G-1]; accept_len [B]; out_tokens [B, G];
 * accepted [B, G-1] (may be NULL); ratio [B, G-1] (may be NULL, T > 0). */
int orc_spec_verify(const double* zp, const double* zq, const int64_t* drafts,
                    int B, int G, int64_t V, double T, const uint64_t* seeds, uint64_t step,
                    int32_t* accept_len, int64_t* out_tokens, uint8_t* accepted, double* ratio)
{
    if (B < 0 || G < 1 || V < 1 || T < 0.0) return -2;
    if (T > 0.0 && !seeds) return -2;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        const double* zpb = zp + (int64_t)b * G * V;
        const int64_t* db = drafts + (int64_t)b * (G - 1);
        uint8_t* ab = accepted ? accepted + (int64_t)b * (G - 1) : NULL;
        int rc;
        if (T == 0.0) {
            rc = orc_greedy_verify_seq(zpb, db, G, V, accept_len + b, out_tokens + (int64_t)b * G, ab);
        } else {
            double* ua = (double*)malloc(sizeof(double) * (size_t)(G > 1 ? G - 1 : 1));
            double* ud = (double*)malloc(sizeof(double) * (size_t)G);
            if (!ua || !ud) { free(ua); free(ud); bad = 1; continue; }
            for (int r = 0; r < G - 1; ++r) ua[r] = orc_uniform(seeds[b], step, (uint64_t)b, (uint64_t)r, 1);
            for (int r = 0; r < G; ++r) ud[r] = orc_uniform(seeds[b], step, (uint64_t)b, (uint64_t)r, 2);
            rc = orc_sampled_verify_seq_u(zpb, zq ? zq + (int64_t)b * G * V : NULL, db, G, V, T, ua, ud,
                                          accept_len + b, out_tokens + (int64_t)b * G, ab,
                                          ratio ? ratio + (int64_t)b * (G - 1) : NULL);
            free(ua);
            free(ud);
        }
        if (rc) bad = 1;
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Candidate selector.                                                         */
/* [P3] "The candidate selector": each block position keeps the top-k draft   */
/* candidates; a transition from candidate a at the preceding position to     */
/* candidate b at position t scores                                           */
/*     S_t(a, b) = U_t(b) + sum_i A(a)_i H(h_t)_i B(b)_i,                     */
/* and one path is walked from the anchor.  Readings: U_t(b) is the drafter's */
/* logit of b at position t (a per-position constant shift would not change   */
/* the walk); A, B are token-embedding tables [V, r] and H(h_t) is given as   */
/* its output gate vector g_t [r]; the walk is greedy ("a is the token        */
/* selected at the preceding position"): position 0 follows the anchor, each  */
/* later position follows the token just chosen; ties go to the candidate     */
/* listed first.                                                              */
/*                                                                            */
/* cand [B, G, k] token ids   score [B, G, k] = U   emb_a, emb_b [V, r]       */
/* gate [B, G, r]   anchor [B]   ->   path [B, G], path_score [B, G] (may be   */
/* NULL) = S_t(prev, chosen).                                                 */
/* ------------------------------------------------------------------------ */
int orc_select_path(const int64_t* cand, const double* score, const double* emb_a,
                    const double* emb_b, const double* gate, const int64_t* anchor,
                    int B, int G, int k, int64_t V, int r, int64_t* path, double* path_score)
{
    if (B < 0 || G < 1 || k < 1 || V < 1 || r < 1) return -2;
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (int b = 0; b < B; ++b) {
        int64_t prev = anchor[b];
        if (prev < 0 || prev >= V) { bad = 1; continue; }
        for (int t = 0; t < G; ++t) {
            const int64_t* ct = cand + ((int64_t)b * G + t) * k;
            const double* ut = score + ((int64_t)b * G + t) * k;
            const double* gt = gate + ((int64_t)b * G + t) * r;
            const double* ea = emb_a + prev * r;
            int best = -1;
            double best_s = 0.0;
            for (int j = 0; j < k; ++j) {
                const int64_t c = ct[j];
                if (c < 0 || c >= V) { bad = 1; break; }
                const double* eb = emb_b + c * r;
                double s = ut[j];
                for (int i = 0; i < r; ++i) s += ea[i] * gt[i] * eb[i];
                if (best < 0 || s > best_s) { best = j; best_s = s; }
            }
            if (best < 0) { bad = 1; break; }
            path[(int64_t)b * G + t] = ct[best];
            if (path_score) path_score[(int64_t)b * G + t] = best_s;
            prev = ct[best];
        }
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Two-tap dynamic convolution.                                               */
/* [P3] "The two-tap dynamic convolution": Conv_k(x)_t = k_{t,0} * x_t +      */
/* k_{t,1} * x_{t-1}, depthwise, with a content-dependent kernel shared by a  */
/* group of channels; it never crosses a block boundary and position 1 reads  */
/* from the verified anchor.  Readings: block row 0 is the anchor's position, */
/* so row t >= 1 reads row t - 1 and row 0 has no predecessor (zero); channel */
/* c uses group c / (D / n_groups); the kernel values are an input (the small */
/* network producing them from the content is outside the path).             */
/*                                                                            */
/* x [B, G, D]   kern [B, G, 2, n_groups]   ->   y [B, G, D]                   */
/* ------------------------------------------------------------------------ */
int orc_two_tap_conv(const double* x, const double* kern, int B, int G, int D, int n_groups,
                     double* y)
{
    if (B < 0 || G < 1 || D < 1 || n_groups < 1 || D % n_groups) return -2;
    const int gs = D / n_groups;
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < G; ++t) {
            const double* xt = x + ((int64_t)b * G + t) * D;
            const double* kt = kern + ((int64_t)b * G + t) * 2 * n_groups;
            double* yt = y + ((int64_t)b * G + t) * D;
            for (int c = 0; c < D; ++c) {
                const int grp = c / gs;
                const double prev = t > 0 ? xt[c - D] : 0.0;
                yt[c] = kt[grp] * xt[c] + kt[n_groups + grp] * prev;
            }
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Context fusion and context K/V injection.                                  */
/* [P3] "Conditioning on the target model", equation for H_t: hidden states  */
/* of five target layers are concatenated, projected by W_c and RMS-         */
/* normalised; equation for K_i, V_i: the context half of each draft layer's */
/* keys and values is W_i^K H_t and W_i^V H_t.                               */
/* [P2] "Model": target layers 4, 16, 28, 40 and 46 are read.               */
/* Readings: RMSNorm(y) = y / sqrt(mean(y^2) + eps) * g with a learnable     */
/* gain g; no bias and no position encoding on the projections; the K/V     */
/* rows of all draft layers come from one stacked projection whose output   */
/* column is ((layer*2 + kv)*NKV + head)*DH + d (kv 0 = K, 1 = V); a row at */
/* absolute position pos of sequence s goes to ring slot pos mod W.         */
/*                                                                            */
/* x [rows, KX] (KX = taps*d_target)   wc [DM, KX]   g [DM]                   */
/* wkv [NL*2*NKV*DH, DM]   row_seq [rows]   row_pos [rows]                    */
/* h_out [rows, DM] (may be NULL)   ring [NL, 2, B, NKV, W, DH] (in/out)     */
/* ------------------------------------------------------------------------ */
int orc_context_fuse(const double* x, const double* wc, const double* g, double eps,
                     const double* wkv, const int32_t* row_seq, const int64_t* row_pos,
                     int rows, int KX, int DM, int NL, int NKV, int DH, int W, int B,
                     double* h_out, double* ring)
{
    if (rows < 0 || KX < 1 || DM < 1 || NL < 1 || NKV < 1 || DH < 1 || W < 1 || B < 1 || eps < 0.0)
        return -2;
    for (int r = 0; r < rows; ++r)
        if (row_seq[r] < 0 || row_seq[r] >= B || row_pos[r] < 0) return -2;
    const int NKVC = NL * 2 * NKV * DH;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; ++r) {
        double* y = (double*)malloc(sizeof(double) * (size_t)DM);
        if (!y) { bad = 1; continue; }
        const double* xr = x + (int64_t)r * KX;
        /* Y = W_c [H^(l1); ...; H^(l5)] */
        for (int n = 0; n < DM; ++n) {
            const double* wr = wc + (int64_t)n * KX;
            double acc = 0.0;
            for (int k = 0; k < KX; ++k) acc += xr[k] * wr[k];
            y[n] = acc;
        }
        /* RMSNorm */
        double ss = 0.0;
        for (int n = 0; n < DM; ++n) ss += y[n] * y[n];
        const double inv = 1.0 / sqrt(ss / DM + eps);
        for (int n = 0; n < DM; ++n) y[n] = y[n] * inv * g[n];
        if (h_out) for (int n = 0; n < DM; ++n) h_out[(int64_t)r * DM + n] = y[n];
        /* context K/V of every draft layer, written to the ring slot */
        const int s = row_seq[r];
        const int64_t slot = row_pos[r] % W;
        for (int c = 0; c < NKVC; ++c) {
            const double* wr = wkv + (int64_t)c * DM;
            double acc = 0.0;
            for (int n = 0; n < DM; ++n) acc += y[n] * wr[n];
            const int d = c % DH;
            const int h = (c / DH) % NKV;
            const int kv = (c / (DH * NKV)) % 2;
            const int layer = c / (DH * NKV * 2);
            ring[(((((int64_t)layer * 2 + kv) * B + s) * NKV + h) * W + slot) * DH + d] = acc;
        }
        free(y);
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Position weights of the training loss.                                    */
/* [P3] "Training with anchors", equation for w_k: w_k = exp(-(k-1)/gamma)  */
/* for position k = 1..gamma of a block of size gamma.                       */
/* ------------------------------------------------------------------------ */
int orc_position_weights(int G, double* w)
{
    if (G < 1) return -2;
    for (int k = 1; k <= G; ++k) w[k - 1] = exp(-(double)(k - 1) / (double)G);
    return 0;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
