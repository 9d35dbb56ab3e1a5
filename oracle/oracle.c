/*
 * oracle.c -- plain, slow, fp64 CPU oracle of BLASST block-skipping attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or helper with the HIP
 * library: the two meet only in the input tensors they are handed.
 *
 * What it computes (sources, cited by page title and section):
 *  - "BLASST: Dynamic BLocked Attention Sparsity via Softmax Thresholding"
 *    (gist.science/pt/paper/2512.12087), section 2 "Metodologia: BLASST":
 *    blockwise online softmax keeps a running row max m_i; for every block
 *    S_j the block-local row max m~_i is formed, and the block is skipped when
 *    m~_i - m_i < ln(lambda).  A skipped block does no exponential, no V load
 *    and no P.V product.  The same statement is in the Hindi explainer
 *    (gist.science/hi/paper/2512.12087), section 2, "core insight".
 *  - BLASST reading notes (papers.lqhl.me/papers/BLASST-MLSys26), section
 *    "核心方法" (core method): Algorithm 1 modifies the FlashAttention forward
 *    pass so that each block first updates the running max, then tests and
 *    skips; section "设计取舍" (design trade-offs): the decision is taken per
 *    block, not per token.
 *  - The FlashAttention blockwise forward itself is only named on the pages
 *    ("online softmax", "running max"); it is written here in its textbook
 *    form: m' = max(m, m~), alpha = exp(m - m'), P = exp(S - m'),
 *    l = alpha*l + rowsum(P), acc = alpha*acc + P V, O = acc / l.
 *
 * Readings taken where the pages are silent (each is listed with its reason in
 * the design notes of this repository):
 *  - key blocks are visited in ascending order;
 *  - a query tile skips a key block only if EVERY valid row of the tile meets
 *    the test, i.e. g = max_r (m~_r - m_r) < ln(lambda), strict '<';
 *  - a row with no unmasked key in the block has d_r = -inf; a row whose
 *    running max is still -inf (first block) has d_r = +inf, so a unit's first
 *    visited block is always executed;
 *  - lambda in [0,1); lambda = 0 gives ln(lambda) = -inf, i.e. never skip;
 *  - a (unit, block) pair is "visited" when at least one (row, key) entry of
 *    it is unmasked; unvisited pairs are marked 255 in the skip map and -inf
 *    in the gap map and change nothing;
 *  - decode: the rows of a unit are the G query heads that share one KV head;
 *    split s of a sequence with nkb key blocks covers the contiguous run
 *    [s*ceil(nkb/S), min(nkb, (s+1)*ceil(nkb/S))) and starts from m = -inf;
 *    the per-split partials (acc, m, l) are merged by the log-sum-exp rule
 *    O = sum_s e^{m_s-M} acc_s / sum_s e^{m_s-M} l_s with M = max_s m_s;
 *  - sliding window W (the BLASST reading notes, "问题与动机", list sliding
 *    window among the supported attention forms and give no further detail):
 *    a query at position i sees keys c with i - W < c <= i; blocks with no
 *    visible key are not visited, and the skip test runs unchanged on the
 *    rest.  In decode the query is at position len-1, so it sees the last W
 *    keys, and the splits cut the blocks from the first block that holds a
 *    visible key: split s covers [j0 + s*ceil((nkb - j0)/S), ...), j0 =
 *    max(0, len - W) div block_k;
 *  - sink-seeded splits (optional, decode): split s >= 1 starts its running
 *    max from the row maxima of the sequence's first visible block (block j0,
 *    the sink block 0 without a window) instead of -inf.  This borrows the
 *    pseudo-maximum of the FFD summary (gist.science/pt/paper/2609.00097,
 *    section 2 "A Estratégia de Seleção Top-δ"), estimated there from sink
 *    and local tokens; here from the sink block alone.  The seed is a real score of a
 *    visible key, so the running max stays below the true row max and the
 *    skip test keeps its meaning; a split may then skip every block (l = 0)
 *    and the merge ignores it.  Split 0 is unseeded (its first block is
 *    always executed).
 *
 * Arithmetic is IEEE fp64 with libm exp/log, loops in the order written.
 * Inputs are fp64 arrays (the tests pass the exact bf16 values the GPU reads).
 *
 * Non-finite inputs (the pages say nothing about them; this is the reading
 * both sides implement):
 *  - a block max, the running max and the max over a tile's row gaps ignore
 *    NaN (a NaN score is not greater than anything); a row gap that is NaN
 *    (inf - inf) therefore never keeps a block from being skipped;
 *  - in an executed block every key that some row of the unit sees
 *    contributes p * V to every row's accumulator and p to its sum, with
 *    p = 0 for a row that does not see the key; 0 * inf and 0 * NaN are NaN,
 *    so a non-finite V value reaches every row of a unit that executes its
 *    block.  Keys that no row of the unit sees contribute nothing;
 *  - O = acc / l when l != 0 (a NaN l gives NaN), and exactly 0 when l = 0
 *    (the row saw no key);
 *  - the split merge takes every split with l != 0 (NaN included) and the
 *    max of their running maxima.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

static double oracle_ln_lambda(double lambda)
{
    /* ln(0) = -inf: the test g < -inf is never true, so nothing is skipped. */
    return lambda == 0.0 ? -INFINITY : log(lambda);
}

/*
 * One unit of the method: R query rows against one key/value sequence,
 * visiting key blocks j_begin .. j_end-1 (block size bc) in ascending order.
 *
 *   q      : row r at q + r*q_stride (d values)
 *   qpos   : position of row r (key c visible iff c <= qpos[r]), or NULL
 *   window : > 0: key c also needs c > qpos[r] - window (sliding window)
 *   k, v   : [klen_alloc][d] and [klen_alloc][dv], contiguous
 *   klen   : keys with index >= klen are masked
 *   seed   : initial running max per row, or NULL for -inf
 *   m,l,acc: outputs, the unit's final running max, sum and accumulator
 *   skip   : per visited block 0 executed / 1 skipped / 255 not visited
 *   gap    : per block g(unit, j), -inf when not visited
 *   S      : scratch [R][bc]
 */
static void oracle_unit(int64_t R, int64_t d, int64_t dv,
                        const double *q, int64_t q_stride, const int64_t *qpos, int64_t window,
                        const double *k, const double *v, int64_t klen,
                        int64_t j_begin, int64_t j_end, int64_t bc,
                        double scale, double lnlam, const double *seed,
                        double *m, double *l, double *acc,
                        uint8_t *skip, double *gap, double *S, double *mt,
                        int64_t *visited_out, int64_t *skipped_out)
{
    int64_t visited = 0, skipped = 0;
    for (int64_t r = 0; r < R; ++r) {
        m[r] = seed ? seed[r] : -INFINITY;
        l[r] = 0.0;
        for (int64_t x = 0; x < dv; ++x)
            acc[r * dv + x] = 0.0;
    }
    uint8_t seen[bc]; /* key c of the block is seen by some row of the unit */
    for (int64_t j = j_begin; j < j_end; ++j) {
        int64_t c0 = j * bc;
        int any = 0;
        memset(seen, 0, (size_t)bc);
        /* Scores of the block and the block-local row max m~ (BLASST summary, section 2). */
        for (int64_t r = 0; r < R; ++r) {
            const double *qr = q + r * q_stride;
            mt[r] = -INFINITY;
            for (int64_t c = 0; c < bc; ++c) {
                int64_t key = c0 + c;
                int visible = key < klen &&
                              (qpos == NULL || (key <= qpos[r] && (window <= 0 || key > qpos[r] - window)));
                if (!visible) {
                    S[r * bc + c] = -INFINITY;
                    continue;
                }
                const double *kc = k + key * d;
                double dot = 0.0;
                for (int64_t x = 0; x < d; ++x)
                    dot += qr[x] * kc[x];
                double s = scale * dot;
                S[r * bc + c] = s;
                if (s > mt[r]) /* a NaN score never raises the max */
                    mt[r] = s;
                seen[c] = 1;
                any = 1;
            }
        }
        int64_t jj = j - j_begin;
        if (!any) {
            skip[jj] = 255;
            gap[jj] = -INFINITY;
            continue;
        }
        ++visited;
        /* Tile gap g = max over rows of m~_r - m_r, with the infinity rules. */
        double g = -INFINITY;
        for (int64_t r = 0; r < R; ++r) {
            double dr;
            if (mt[r] == -INFINITY)
                dr = -INFINITY;
            else if (m[r] == -INFINITY)
                dr = INFINITY;
            else
                dr = mt[r] - m[r];
            if (dr > g)
                g = dr;
        }
        gap[jj] = g;
        /* Skip test (BLASST summary, section 2; Hindi explainer, section 2): m~ - m < ln(lambda). */
        if (g < lnlam) {
            skip[jj] = 1;
            ++skipped;
            continue; /* no exp, no V read, no P.V, no change to m, l, acc */
        }
        skip[jj] = 0;
        /* Textbook online-softmax update of the executed block.  Every key
         * that some row of the unit sees enters every row, with p = 0 where the
         * row does not see it (a row that has seen no key yet keeps m = -inf
         * and l = 0 and only gathers 0 * V). */
        for (int64_t r = 0; r < R; ++r) {
            double mp = m[r] > mt[r] ? m[r] : mt[r];
            double alpha = (m[r] == -INFINITY) ? 0.0 : exp(m[r] - mp);
            double *ar = acc + r * dv;
            double rowsum = 0.0;
            for (int64_t x = 0; x < dv; ++x)
                ar[x] *= alpha;
            for (int64_t c = 0; c < bc; ++c) {
                if (!seen[c])
                    continue; /* no row of the unit sees this key */
                double s = S[r * bc + c];
                double p = (s == -INFINITY) ? 0.0 : exp(s - mp);
                rowsum += p;
                const double *vc = v + (c0 + c) * dv;
                for (int64_t x = 0; x < dv; ++x)
                    ar[x] += p * vc[x];
            }
            l[r] = alpha * l[r] + rowsum;
            m[r] = mp;
        }
    }
    *visited_out = visited;
    *skipped_out = skipped;
}

/*
 * Prefill (causal or not), Lq = Lk = L, one query tile = tile_q consecutive
 * positions of one query head; query head h reads KV head h / (Hq/Hkv).
 * window > 0 (causal only): query i sees keys i - window < c <= i.
 *
 *   q [B][Hq][L][d], k [B][Hkv][L][d], v [B][Hkv][L][dv]  (contiguous fp64)
 *   unit_mask [B][Hq][nQT] or NULL: compute only units whose byte is nonzero
 *   o [B][Hq][L][dv], skip_map / gap_map [B][Hq][nQT][nKB] (may be NULL)
 *   counters [2] = {visited, skipped} summed over computed units (may be NULL)
 */
int oracle_prefill(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d, int64_t dv,
                   const double *q, const double *k, const double *v,
                   int causal, int64_t window, double scale, double lambda,
                   int64_t tile_q, int64_t block_k, const uint8_t *unit_mask,
                   double *o, uint8_t *skip_map, double *gap_map,
                   int64_t *counters, int nthreads)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || L < 0 || d <= 0 || dv <= 0 || tile_q <= 0 ||
        block_k <= 0 || Hq % Hkv != 0 || !(lambda >= 0.0 && lambda < 1.0) || window < 0 ||
        (window > 0 && !causal))
        return ORACLE_EINVAL;
    const int64_t G = Hq / Hkv;
    const int64_t nqt = (L + tile_q - 1) / tile_q;
    const int64_t nkb = (L + block_k - 1) / block_k;
    const int64_t units = B * Hq * nqt;
    const double lnlam = oracle_ln_lambda(lambda);
    int64_t tot_visited = 0, tot_skipped = 0;
    int err = ORACLE_OK;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();

#pragma omp parallel num_threads(nthreads) reduction(+ : tot_visited, tot_skipped)
    {
        double *S = malloc(sizeof(double) * tile_q * block_k);
        double *mt = malloc(sizeof(double) * tile_q);
        double *m = malloc(sizeof(double) * tile_q);
        double *l = malloc(sizeof(double) * tile_q);
        double *acc = malloc(sizeof(double) * tile_q * dv);
        int64_t *qpos = malloc(sizeof(int64_t) * tile_q);
        uint8_t *sk = malloc(nkb > 0 ? nkb : 1);
        double *gp = malloc(sizeof(double) * (nkb > 0 ? nkb : 1));
        if (!S || !mt || !m || !l || !acc || !qpos || !sk || !gp) {
#pragma omp atomic write
            err = ORACLE_ENOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < units; ++u) {
                if (unit_mask && !unit_mask[u])
                    continue;
                int64_t t = u % nqt, h = (u / nqt) % Hq, b = u / (nqt * Hq);
                int64_t hk = h / G;
                int64_t r0 = t * tile_q;
                int64_t R = (L - r0) < tile_q ? (L - r0) : tile_q; /* rows >= L do not exist */
                for (int64_t r = 0; r < R; ++r)
                    qpos[r] = r0 + r;
                const double *qb = q + ((b * Hq + h) * L + r0) * d;
                const double *kb = k + (b * Hkv + hk) * L * d;
                const double *vb = v + (b * Hkv + hk) * L * dv;
                int64_t vis = 0, skp = 0;
                oracle_unit(R, d, dv, qb, d, causal ? qpos : NULL, window, kb, vb, L, 0, nkb, block_k,
                            scale, lnlam, NULL, m, l, acc, sk, gp, S, mt, &vis, &skp);
                tot_visited += vis;
                tot_skipped += skp;
                double *ob = o + ((b * Hq + h) * L + r0) * dv;
                for (int64_t r = 0; r < R; ++r)
                    for (int64_t x = 0; x < dv; ++x)
                        ob[r * dv + x] = l[r] != 0.0 ? acc[r * dv + x] / l[r] : 0.0;
                if (skip_map)
                    memcpy(skip_map + u * nkb, sk, nkb);
                if (gap_map)
                    memcpy(gap_map + u * nkb, gp, sizeof(double) * nkb);
            }
        }
        free(S); free(mt); free(m); free(l); free(acc); free(qpos); free(sk); free(gp);
    }
    if (counters) {
        counters[0] = tot_visited;
        counters[1] = tot_skipped;
    }
    return err;
}

/*
 * Decode: one query token per sequence.  Unit = (sequence b, KV head g); its
 * rows are the G = Hq/Hkv query heads g*G .. g*G+G-1 (GQA; MQA when Hkv = 1,
 * MHA when G = 1; the MLA absorbed form is GQA with Hkv = 1 and a V that the
 * caller takes as the first dv columns of the latent cache).
 *
 *   q [B][Hq][dqk], k [B][Hkv][Lmax][dqk], v [B][Hkv][Lmax][dv]
 *   seq_lens [B] in 1..Lmax; keys >= seq_lens[b] are masked
 *   num_splits >= 1: contiguous block runs, each from m = -inf, merged by LSE
 *   window > 0: the query (position len-1) sees the last `window` keys only
 *   sink_seed != 0: splits s >= 1 start from the row maxima of block j0
 *   unit_mask [B][Hkv] or NULL
 *   o [B][Hq][dv]; skip_map / gap_map [B][Hkv][nKB], nKB = ceil(Lmax/block_k)
 */
int oracle_decode(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t dqk, int64_t dv,
                  const double *q, const double *k, const double *v, const int32_t *seq_lens,
                  double scale, double lambda, int64_t block_k, int64_t num_splits, int64_t window,
                  int sink_seed, const uint8_t *unit_mask, double *o, uint8_t *skip_map, double *gap_map,
                  int64_t *counters, int nthreads)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Lmax <= 0 || dqk <= 0 || dv <= 0 || block_k <= 0 ||
        num_splits <= 0 || Hq % Hkv != 0 || !(lambda >= 0.0 && lambda < 1.0) || window < 0)
        return ORACLE_EINVAL;
    for (int64_t b = 0; b < B; ++b)
        if (seq_lens[b] < 1 || seq_lens[b] > Lmax)
            return ORACLE_EINVAL;
    const int64_t G = Hq / Hkv;
    const int64_t nkb = (Lmax + block_k - 1) / block_k;
    const int64_t units = B * Hkv;
    const double lnlam = oracle_ln_lambda(lambda);
    int64_t tot_visited = 0, tot_skipped = 0;
    int err = ORACLE_OK;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();

#pragma omp parallel num_threads(nthreads) reduction(+ : tot_visited, tot_skipped)
    {
        double *S = malloc(sizeof(double) * G * block_k);
        double *mt = malloc(sizeof(double) * G);
        double *ms = malloc(sizeof(double) * G * num_splits);
        double *ls = malloc(sizeof(double) * G * num_splits);
        double *accs = malloc(sizeof(double) * G * dv * num_splits);
        uint8_t *sk = malloc(nkb);
        double *gp = malloc(sizeof(double) * nkb);
        int64_t *qpos = malloc(sizeof(int64_t) * G);
        double *seed = malloc(sizeof(double) * G);
        if (!S || !mt || !ms || !ls || !accs || !sk || !gp || !qpos || !seed) {
#pragma omp atomic write
            err = ORACLE_ENOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < units; ++u) {
                if (unit_mask && !unit_mask[u])
                    continue;
                int64_t g = u % Hkv, b = u / Hkv;
                int64_t len = seq_lens[b];
                int64_t nkb_b = (len + block_k - 1) / block_k;
                int64_t j0 = (window > 0 && len > window) ? (len - window) / block_k : 0;
                int64_t per = (nkb_b - j0 + num_splits - 1) / num_splits;
                for (int64_t r = 0; r < G; ++r)
                    qpos[r] = len - 1; /* the query token is the sequence's last position */
                const double *qb = q + (b * Hq + g * G) * dqk;
                const double *kb = k + (b * Hkv + g) * Lmax * dqk;
                const double *vb = v + (b * Hkv + g) * Lmax * dv;
                for (int64_t j = 0; j < nkb; ++j) {
                    sk[j] = 255;
                    gp[j] = -INFINITY;
                }
                /* Seed: row max of the scaled scores over the visible keys of block j0. */
                for (int64_t r = 0; r < G; ++r) {
                    seed[r] = -INFINITY;
                    for (int64_t key = j0 * block_k; key < (j0 + 1) * block_k && key < len; ++key) {
                        if (window > 0 && key <= len - 1 - window)
                            continue;
                        double dot = 0.0;
                        for (int64_t x = 0; x < dqk; ++x)
                            dot += qb[r * dqk + x] * kb[key * dqk + x];
                        if (scale * dot > seed[r])
                            seed[r] = scale * dot;
                    }
                }
                for (int64_t s = 0; s < num_splits; ++s) {
                    int64_t jb = j0 + s * per, je = j0 + (s + 1) * per;
                    if (je > nkb_b)
                        je = nkb_b;
                    double *m = ms + s * G, *l = ls + s * G, *acc = accs + s * G * dv;
                    if (jb >= je) { /* empty split: contributes nothing */
                        for (int64_t r = 0; r < G; ++r) {
                            m[r] = -INFINITY;
                            l[r] = 0.0;
                        }
                        continue;
                    }
                    int64_t vis = 0, skp = 0;
                    oracle_unit(G, dqk, dv, qb, dqk, window > 0 ? qpos : NULL, window, kb, vb, len, jb, je, block_k, scale,
                                lnlam, (sink_seed && s > 0) ? seed : NULL, m, l, acc, sk + jb, gp + jb, S, mt, &vis, &skp);
                    tot_visited += vis;
                    tot_skipped += skp;
                }
                /* Log-sum-exp merge of the split partials, per head row. */
                for (int64_t r = 0; r < G; ++r) {
                    double M = -INFINITY;
                    for (int64_t s = 0; s < num_splits; ++s)
                        if (ls[s * G + r] != 0.0 && ms[s * G + r] > M) /* splits that saw keys (NaN l too) */
                            M = ms[s * G + r];
                    double den = 0.0;
                    double *orow = o + (b * Hq + g * G + r) * dv;
                    for (int64_t x = 0; x < dv; ++x)
                        orow[x] = 0.0;
                    for (int64_t s = 0; s < num_splits; ++s) {
                        if (ls[s * G + r] == 0.0)
                            continue; /* saw no key, or skipped every block */
                        double w = exp(ms[s * G + r] - M);
                        den += w * ls[s * G + r];
                        const double *ar = accs + (s * G + r) * dv;
                        for (int64_t x = 0; x < dv; ++x)
                            orow[x] += w * ar[x];
                    }
                    for (int64_t x = 0; x < dv; ++x)
                        orow[x] = den != 0.0 ? orow[x] / den : 0.0;
                }
                if (skip_map)
                    memcpy(skip_map + u * nkb, sk, nkb);
                if (gap_map)
                    memcpy(gap_map + u * nkb, gp, sizeof(double) * nkb);
            }
        }
        free(S); free(mt); free(ms); free(ls); free(accs); free(sk); free(gp); free(qpos); free(seed);
    }
    if (counters) {
        counters[0] = tot_visited;
        counters[1] = tot_skipped;
    }
    return err;
}

/*
 * Threshold calibration (BLASST summary, section 2 "Calibração Automática";
 * BLASST reading notes, "关键观察" observation 2 and "核心方法"): lambda = a / L, with a fitted per
 * target sparsity on calibration data.
 *
 * oracle_lambda_for_target: given the gaps g of the visited (unit, block)
 * pairs at one context length, the sparsity reached at lambda is the fraction
 * of gaps below ln(lambda) (decisions depend on the gaps alone, because the
 * running max ignores the decisions).  To skip k = ceil(target*N) pairs, take
 * ln(lambda) halfway between the k-th and (k+1)-th smallest gap.  Returns the
 * lambda; *reached gets the fraction of gaps strictly below ln(lambda).
 * lambda is clamped below 1 (ln(lambda) < 0): an unreachable target reports
 * the sparsity actually reached.
 */
static int oracle_cmp_double(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x > y) - (x < y);
}

double oracle_lambda_for_target(const double *gaps, int64_t n, double target, double *reached)
{
    double *s = malloc(sizeof(double) * (n > 0 ? n : 1));
    if (!s || n <= 0) {
        free(s);
        if (reached)
            *reached = 0.0;
        return 0.0;
    }
    memcpy(s, gaps, sizeof(double) * n);
    qsort(s, n, sizeof(double), oracle_cmp_double);
    int64_t kk = (int64_t)ceil(target * (double)n);
    if (kk < 0)
        kk = 0;
    if (kk > n)
        kk = n;
    double lnl;
    if (kk == 0)
        lnl = -INFINITY; /* lambda = 0: skip nothing */
    else if (kk == n || isinf(s[kk]))
        lnl = s[kk - 1] + 1.0;
    else
        lnl = 0.5 * (s[kk - 1] + s[kk]);
    /* largest double below 0 keeps lambda < 1 */
    if (!(lnl < 0.0))
        lnl = -0x1p-40;
    double lam = exp(lnl);
    int64_t below = 0;
    for (int64_t i = 0; i < n; ++i)
        if (gaps[i] < lnl)
            ++below;
    if (reached)
        *reached = (double)below / (double)n;
    free(s);
    return lam;
}

/* a from lambdas measured at several lengths: ln a = mean_L ln(lambda_L * L). */
double oracle_fit_a(const double *lambda_at_L, const int64_t *L, int64_t n)
{
    double sum = 0.0;
    for (int64_t i = 0; i < n; ++i)
        sum += log(lambda_at_L[i] * (double)L[i]);
    return exp(sum / (double)n);
}

/* lambda = a(target) / L with ln a linear in the target between table rows. */
double oracle_lambda_from_table(const double *targets, const double *a, int64_t n,
                                double target, int64_t L)
{
    double lna;
    if (target <= targets[0])
        lna = log(a[0]);
    else if (target >= targets[n - 1])
        lna = log(a[n - 1]);
    else {
        int64_t i = 0;
        while (!(target >= targets[i] && target <= targets[i + 1]))
            ++i;
        double w = (target - targets[i]) / (targets[i + 1] - targets[i]);
        lna = (1.0 - w) * log(a[i]) + w * log(a[i + 1]);
    }
    return exp(lna) / (double)L;
}
