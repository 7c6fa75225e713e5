/*
 * oracle.c -- plain, slow, fp64 CPU reference for speculative-decoding
 * verification over the vocabulary.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * source, header or constant with the GPU library and must never serve as a
 * fallback for it.
 *
 * Sources (page titles; sections/equations/figures on those pages):
 *  [SD]  "Speculative decoding verifies draft tokens without changing the
 *        target sampling distribution" -- sections "Acceptance depends on both
 *        target and draft probabilities" (ratio test min(1, p(x)/q(x)), left
 *        to right, stop at the first rejection), "Rejection uses a residual
 *        distribution" (correction drawn from max(0, p - q) normalised), "A
 *        fully accepted block yields more than one committed token" (bonus
 *        token drawn from p after the last draft position), "Logit processing
 *        must be consistent across verification" (one temperature for p and q;
 *        masked tokens are impossible).
 *  [J++] "JetSpec++: Foresight Parallel Drafting with Self Refinements" --
 *        Appendix F.1 (worked example, Proposition 1: independent fresh draw
 *        per test, rejection ends the block, bonus from p_{gamma+1}).
 *  [JN]  "JetSpec reading notes" (page 3) -- Eq. 1 (acceptance probability),
 *        Eq. 16-17 (per-branch Bernoulli tests, accepted prefix length),
 *        section "Tree verification" with Fig. 5 and the greedy note (at T=0 a
 *        node is accepted iff its token is the target argmax after its
 *        parent's path), Algorithm 1 (parent pointers, node 0 is the root).
 *
 * Readings where the pages leave a step open (each also listed with the
 * design notes of the repository):
 *  - uniforms: u[b][i] drives the test at draft position i (i < gamma),
 *    u[b][gamma] drives the final draw; accept iff u < r (u uniform on [0,1)
 *    then accepts with probability exactly r);
 *  - ratio r = min(1, p(x)/q(x)) evaluated as exp(log p(x) - log q(x)); by
 *    convention r = 0 when p(x) = 0 and r = 1 when q(x) = 0 < p(x);
 *  - the final draw maps u to a token by inverse CDF in ascending token id:
 *    the smallest v with sum_{t<=v} w(t) > u * W; if rounding leaves no such
 *    v, the last v with w(v) > 0.  The pages fix the law of the draw but not
 *    the order in which the CDF is walked; this order is the textbook
 *    inverse-transform sampler's, and the tests pin the map against NumPy's
 *    Generator.choice, which samples the same way;
 *  - a residual with W = 0 (impossible in exact arithmetic after a
 *    rejection) falls back to sampling from p at that position; the block is
 *    flagged and its final margin is 0;
 *  - argmax ties go to the lowest token id; among accepted tree nodes of
 *    maximal depth the lowest node index wins;
 *  - invalid input (a draft token outside [0, V), a NaN or +inf logit, a row
 *    with no finite logit, a malformed parent array) makes that block
 *    invalid: accept_len = -1 and all its output tokens -1.  Every other
 *    input, however large its logits or small its temperature, is evaluated
 *    by the definitions below in double precision.
 *
 * Every allocation is checked; an entry point that cannot get its memory
 * frees what it holds and returns -2.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* Exact decoding: fp32 as stored; bf16 by placing its 16 bits on top of a
 * 32-bit float.  Both then widen exactly to double. */
static double logit_at(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORC_F32)
        return (double)((const float *)base)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Temperature softmax of one row, by definition: m = max z over the row,
 * S = sum_v exp((z_v - m)/T), p(v) = exp((z_v - m)/T) / S.  Returns 0 and
 * fills (m, S) for a valid row; -1 if the row holds NaN or +inf or no finite
 * logit at all.  ([SD] "Logit processing must be consistent": p and q are
 * both taken at the same temperature T.) */
static int row_softmax_stats(const void *base, int dtype, int64_t off, int V, double T,
                             double *m_out, double *S_out)
{
    double m = -INFINITY;
    for (int v = 0; v < V; ++v) {
        double z = logit_at(base, dtype, off + v);
        if (isnan(z) || z == INFINITY)
            return -1;
        if (z > m)
            m = z;
    }
    if (m == -INFINITY)
        return -1;
    double S = 0.0;
    for (int v = 0; v < V; ++v) {
        double z = logit_at(base, dtype, off + v);
        S += exp((z - m) / T);
    }
    *m_out = m;
    *S_out = S;
    return 0;
}

static double prob_at(const void *base, int dtype, int64_t off, int v, double T, double m,
                      double S)
{
    return exp((logit_at(base, dtype, off + v) - m) / T) / S;
}

static double logprob_at(const void *base, int dtype, int64_t off, int v, double T, double m,
                         double S)
{
    double z = logit_at(base, dtype, off + v);
    if (z == -INFINITY)
        return -INFINITY;
    return (z - m) / T - log(S);
}

typedef struct {
    const void *target, *draft;
    int dtype;
    const int32_t *draft_tokens;
    const double *uniforms; /* [B][gamma+1] as doubles */
    int B, gamma, V;
    double T;
    int32_t *accept_len, *out_tokens;
    double *final_dist; /* nullable [B][V] */
    double *margin;     /* nullable [B]: smallest decision margin on the path */
    double *ratios;     /* nullable [B][gamma]: r_i at every position */
    int32_t *fallback;  /* nullable [B]: 1 if the W = 0 fallback was taken */
    double *work;       /* [nthreads][V] scratch for w(v) */
    double *rowstats;   /* [nthreads][4 (gamma+1)] scratch for (m, S) of p and q */
    int nthreads;
} chain_job;

/* One chain block, following [SD] and [J++] F.1 step by step.  w holds V
 * doubles and st 4 (gamma+1) doubles of the calling thread's scratch. */
static void chain_block(const chain_job *J, int b, double *w, double *st)
{
    const int g = J->gamma, V = J->V, dt = J->dtype;
    const double T = J->T;
    const double *u = J->uniforms + (int64_t)b * (g + 1);
    int32_t *out = J->out_tokens + (int64_t)b * (g + 1);
    const int32_t *d = J->draft_tokens + (int64_t)b * g;
    const int64_t trow = (int64_t)V, tblk = (int64_t)(g + 1) * V, dblk = (int64_t)g * V;

    for (int i = 0; i <= g; ++i)
        out[i] = -1;
    J->accept_len[b] = -1;
    if (J->margin)
        J->margin[b] = 0.0;
    if (J->fallback)
        J->fallback[b] = 0;
    if (J->final_dist)
        for (int v = 0; v < V; ++v)
            J->final_dist[(int64_t)b * V + v] = 0.0;
    if (J->ratios)
        for (int i = 0; i < g; ++i)
            J->ratios[(int64_t)b * g + i] = NAN;

    /* Validate the whole block first: every draft token in range and every
     * row a proper distribution. */
    for (int i = 0; i < g; ++i)
        if (d[i] < 0 || d[i] >= V)
            return;
    double *mp = st, *Sp = st + (g + 1), *mq = st + 2 * (g + 1), *Sq = st + 3 * (g + 1);
    int bad = 0;
    for (int j = 0; j <= g && !bad; ++j)
        bad |= row_softmax_stats(J->target, dt, b * tblk + j * trow, V, T, &mp[j], &Sp[j]);
    for (int j = 0; j < g && !bad; ++j)
        bad |= row_softmax_stats(J->draft, dt, b * dblk + j * trow, V, T, &mq[j], &Sq[j]);
    if (bad)
        return;

    /* Ratio r_i = min(1, p_i(x)/q_i(x)) at every draft position ([SD]
     * "Acceptance depends on ..."; [JN] Eq. 1). */
    double margin = INFINITY;
    int k = g;
    int decided = 0;
    for (int i = 0; i < g; ++i) {
        double lp = logprob_at(J->target, dt, b * tblk + i * trow, d[i], T, mp[i], Sp[i]);
        double lq = logprob_at(J->draft, dt, b * dblk + i * trow, d[i], T, mq[i], Sq[i]);
        double r;
        if (lp == -INFINITY)
            r = 0.0;
        else if (lq == -INFINITY)
            r = 1.0;
        else
            r = fmin(1.0, exp(lp - lq));
        if (J->ratios)
            J->ratios[(int64_t)b * g + i] = r;
        if (!decided) {
            /* Left to right; a fresh uniform per test; the first failure ends
             * the block ([SD]; [J++] F.1; [JN] Eq. 17). */
            margin = fmin(margin, fabs(u[i] - r));
            if (!(u[i] < r)) {
                k = i;
                decided = 1;
            }
        }
    }

    /* Final draw: residual max(0, p_k - q_k) after a rejection, or p_gamma
     * (the bonus row) after a fully accepted block ([SD] "Rejection uses a
     * residual distribution", "A fully accepted block ..."; [J++] F.1). */
    const int64_t prow = b * tblk + (int64_t)k * trow;
    double W = 0.0;
    if (k < g) {
        const int64_t qrow = b * dblk + (int64_t)k * trow;
        for (int v = 0; v < V; ++v) {
            double pv = prob_at(J->target, dt, prow, v, T, mp[k], Sp[k]);
            double qv = prob_at(J->draft, dt, qrow, v, T, mq[k], Sq[k]);
            w[v] = fmax(0.0, pv - qv);
            W += w[v];
        }
    }
    int fell_back = 0;
    if (k == g || !(W > 0.0)) {
        fell_back = (k < g);
        W = 0.0;
        for (int v = 0; v < V; ++v) {
            w[v] = prob_at(J->target, dt, prow, v, T, mp[k], Sp[k]);
            W += w[v];
        }
    }
    /* Inverse CDF in ascending token id. */
    const double t = u[g] * W;
    double C = 0.0, Cprev = 0.0;
    int tok = -1;
    for (int v = 0; v < V; ++v) {
        Cprev = C;
        C += w[v];
        if (C > t) {
            tok = v;
            break;
        }
    }
    double mf;
    if (tok < 0) {
        for (int v = V - 1; v >= 0; --v)
            if (w[v] > 0.0) {
                tok = v;
                break;
            }
        mf = 0.0;
    } else {
        mf = fmin(t - Cprev, C - t) / W;
    }
    margin = fmin(margin, mf);
    if (fell_back)
        margin = 0.0;

    J->accept_len[b] = k;
    for (int i = 0; i < k; ++i)
        out[i] = d[i];
    out[k] = tok;
    if (J->margin)
        J->margin[b] = margin;
    if (J->fallback)
        J->fallback[b] = fell_back;
    if (J->final_dist)
        for (int v = 0; v < V; ++v)
            J->final_dist[(int64_t)b * V + v] = w[v] / W;
}

typedef struct {
    const chain_job *J;
    int tid;
    void (*block)(const chain_job *, int, double *, double *);
} chain_arg;

static void *chain_worker(void *p)
{
    const chain_arg *a = (const chain_arg *)p;
    const chain_job *J = a->J;
    double *w = J->work + (int64_t)a->tid * J->V;
    double *st = J->rowstats + (int64_t)a->tid * 4 * (J->gamma + 1);
    for (int b = a->tid; b < J->B; b += J->nthreads)
        a->block(J, b, w, st);
    return NULL;
}

/* Runs fn(arg_i) for i < n on up to n threads; a thread that cannot be
 * started has its share run on the calling thread instead. */
static void run_parallel(void *(*fn)(void *), void *args, size_t arg_size, int n)
{
    pthread_t *th = n > 1 ? malloc(sizeof(pthread_t) * (size_t)n) : NULL;
    char *started = n > 1 ? calloc((size_t)n, 1) : NULL;
    for (int i = 0; i < n; ++i) {
        void *ai = (char *)args + (size_t)i * arg_size;
        if (th && started && pthread_create(&th[i], NULL, fn, ai) == 0)
            started[i] = 1;
        else
            fn(ai);
    }
    for (int i = 0; i < n; ++i)
        if (th && started && started[i])
            pthread_join(th[i], NULL);
    free(th);
    free(started);
}

static int run_chain(chain_job *J, void (*block)(const chain_job *, int, double *, double *))
{
    int nt = J->nthreads < 1 ? 1 : J->nthreads;
    if (nt > J->B)
        nt = J->B;
    J->nthreads = nt;
    J->work = malloc(sizeof(double) * (size_t)nt * (size_t)J->V);
    J->rowstats = malloc(sizeof(double) * (size_t)nt * 4 * (size_t)(J->gamma + 1));
    chain_arg *args = malloc(sizeof(chain_arg) * (size_t)nt);
    if (!J->work || !J->rowstats || !args) {
        free(J->work);
        free(J->rowstats);
        free(args);
        return -2;
    }
    for (int i = 0; i < nt; ++i) {
        args[i].J = J;
        args[i].tid = i;
        args[i].block = block;
    }
    run_parallel(chain_worker, args, sizeof(chain_arg), nt);
    free(args);
    free(J->work);
    free(J->rowstats);
    return 0;
}

/* Chain verification with double-precision uniforms (the exact-enumeration
 * tests drive the decision function with continuous u). */
int oracle_chain_du(const void *target, const void *draft, int dtype,
                    const int32_t *draft_tokens, const double *uniforms, int B, int gamma,
                    int V, double T, int32_t *accept_len, int32_t *out_tokens,
                    double *final_dist, double *margin, double *ratios, int32_t *fallback,
                    int nthreads)
{
    if (!target || !draft || !draft_tokens || !uniforms || !accept_len || !out_tokens)
        return -1;
    if (B < 1 || gamma < 1 || V < 1 || !(T > 0.0) || !isfinite(T))
        return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16)
        return -1;
    chain_job J = {target, draft, dtype, draft_tokens, uniforms, B, gamma, V, T, accept_len,
                   out_tokens, final_dist, margin, ratios, fallback, NULL, NULL, nthreads};
    return run_chain(&J, chain_block);
}

/* Chain verification with the float32 uniforms of the library interface;
 * each uniform widens exactly to double. */
int oracle_chain(const void *target, const void *draft, int dtype, const int32_t *draft_tokens,
                 const float *uniforms, int B, int gamma, int V, double T,
                 int32_t *accept_len, int32_t *out_tokens, double *final_dist, double *margin,
                 double *ratios, int32_t *fallback, int nthreads)
{
    if (!uniforms || B < 1 || gamma < 1)
        return -1;
    size_t nu = (size_t)B * (size_t)(gamma + 1);
    double *ud = malloc(sizeof(double) * nu);
    if (!ud)
        return -2;
    for (size_t i = 0; i < nu; ++i)
        ud[i] = (double)uniforms[i];
    int rc = oracle_chain_du(target, draft, dtype, draft_tokens, ud, B, gamma, V, T, accept_len,
                             out_tokens, final_dist, margin, ratios, fallback, nthreads);
    free(ud);
    return rc;
}

/* ------------------------------------------------------- point mass -- */

/* Point-mass ("exact-match") chain verification of one block ([J++]
 * Appendix F.3 and Proposition 1; the worked example of Appendix F.1).  The
 * draft proposes x_i with certainty, so the test at position i accepts with
 * probability p_i(x_i): accept iff u_i < p_i(x_i), left to right, the first
 * failure k ending the block.  After a rejection at k the extra token is
 * drawn from p_k with x_k removed and the remainder renormalised (the
 * residual max(0, p_k - q_k) for q_k = delta_{x_k}); after a fully accepted
 * block it is drawn from the bonus row p_gamma.  Same readings as the chain:
 * u[i] drives test i, u[gamma] the final draw by inverse CDF in ascending
 * token id; an empty residual falls back to p_k (flagged, margin 0). */
static void pointmass_block(const chain_job *J, int b, double *w, double *st)
{
    const int g = J->gamma, V = J->V, dt = J->dtype;
    const double T = J->T;
    const double *u = J->uniforms + (int64_t)b * (g + 1);
    int32_t *out = J->out_tokens + (int64_t)b * (g + 1);
    const int32_t *d = J->draft_tokens + (int64_t)b * g;
    const int64_t trow = (int64_t)V, tblk = (int64_t)(g + 1) * V;

    for (int i = 0; i <= g; ++i)
        out[i] = -1;
    J->accept_len[b] = -1;
    if (J->margin)
        J->margin[b] = 0.0;
    if (J->fallback)
        J->fallback[b] = 0;
    if (J->final_dist)
        for (int v = 0; v < V; ++v)
            J->final_dist[(int64_t)b * V + v] = 0.0;
    if (J->ratios)
        for (int i = 0; i < g; ++i)
            J->ratios[(int64_t)b * g + i] = NAN;

    for (int i = 0; i < g; ++i)
        if (d[i] < 0 || d[i] >= V)
            return;
    double *mp = st, *Sp = st + (g + 1);
    int bad = 0;
    for (int j = 0; j <= g && !bad; ++j)
        bad |= row_softmax_stats(J->target, dt, b * tblk + j * trow, V, T, &mp[j], &Sp[j]);
    if (bad)
        return;

    /* Tests: r_i = p_i(x_i). */
    double margin = INFINITY;
    int k = g, decided = 0;
    for (int i = 0; i < g; ++i) {
        const double r = prob_at(J->target, dt, b * tblk + i * trow, d[i], T, mp[i], Sp[i]);
        if (J->ratios)
            J->ratios[(int64_t)b * g + i] = r;
        if (!decided) {
            margin = fmin(margin, fabs(u[i] - r));
            if (!(u[i] < r)) {
                k = i;
                decided = 1;
            }
        }
    }

    /* Final draw: p_k without x_k after a rejection, p_gamma after none. */
    const int64_t prow = b * tblk + (int64_t)k * trow;
    double W = 0.0;
    for (int v = 0; v < V; ++v) {
        w[v] = (k < g && v == d[k]) ? 0.0 : prob_at(J->target, dt, prow, v, T, mp[k], Sp[k]);
        W += w[v];
    }
    int fell_back = 0;
    if (!(W > 0.0)) {
        fell_back = 1;
        W = 0.0;
        for (int v = 0; v < V; ++v) {
            w[v] = prob_at(J->target, dt, prow, v, T, mp[k], Sp[k]);
            W += w[v];
        }
    }
    const double t = u[g] * W;
    double C = 0.0, Cprev = 0.0;
    int tok = -1;
    for (int v = 0; v < V; ++v) {
        Cprev = C;
        C += w[v];
        if (C > t) {
            tok = v;
            break;
        }
    }
    double mf;
    if (tok < 0) {
        for (int v = V - 1; v >= 0; --v)
            if (w[v] > 0.0) {
                tok = v;
                break;
            }
        mf = 0.0;
    } else {
        mf = fmin(t - Cprev, C - t) / W;
    }
    margin = fmin(margin, mf);
    if (fell_back)
        margin = 0.0;

    J->accept_len[b] = k;
    for (int i = 0; i < k; ++i)
        out[i] = d[i];
    out[k] = tok;
    if (J->margin)
        J->margin[b] = margin;
    if (J->fallback)
        J->fallback[b] = fell_back;
    if (J->final_dist)
        for (int v = 0; v < V; ++v)
            J->final_dist[(int64_t)b * V + v] = w[v] / W;
}

/* Point-mass chain verification over B blocks: target [B][gamma+1][V],
 * draft tokens [B][gamma], double uniforms [B][gamma+1]; outputs as
 * oracle_chain_du (ratios hold p_i(x_i)). */
int oracle_chain_pointmass_du(const void *target, int dtype, const int32_t *draft_tokens,
                              const double *uniforms, int B, int gamma, int V, double T,
                              int32_t *accept_len, int32_t *out_tokens, double *final_dist,
                              double *margin, double *ratios, int32_t *fallback, int nthreads)
{
    if (!target || !draft_tokens || !uniforms || !accept_len || !out_tokens)
        return -1;
    if (B < 1 || gamma < 1 || V < 1 || !(T > 0.0) || !isfinite(T))
        return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16)
        return -1;
    chain_job J = {target, NULL, dtype, draft_tokens, uniforms, B, gamma, V, T, accept_len,
                   out_tokens, final_dist, margin, ratios, fallback, NULL, NULL, nthreads};
    return run_chain(&J, pointmass_block);
}

/* The same with the float32 uniforms of the library interface. */
int oracle_chain_pointmass(const void *target, int dtype, const int32_t *draft_tokens,
                           const float *uniforms, int B, int gamma, int V, double T,
                           int32_t *accept_len, int32_t *out_tokens, double *final_dist,
                           double *margin, double *ratios, int32_t *fallback, int nthreads)
{
    if (!uniforms || B < 1 || gamma < 1)
        return -1;
    size_t nu = (size_t)B * (size_t)(gamma + 1);
    double *ud = malloc(sizeof(double) * nu);
    if (!ud)
        return -2;
    for (size_t i = 0; i < nu; ++i)
        ud[i] = (double)uniforms[i];
    int rc = oracle_chain_pointmass_du(target, dtype, draft_tokens, ud, B, gamma, V, T,
                                       accept_len, out_tokens, final_dist, margin, ratios,
                                       fallback, nthreads);
    free(ud);
    return rc;
}

/* ------------------------------------------------- outcome scoring -- */

typedef struct {
    double p;
    int k, a;
} outcome;

/* Descending probability; among equal probabilities the smaller k, then the
 * smaller token id, comes first. */
static int outcome_cmp(const void *x, const void *y)
{
    const outcome *a = (const outcome *)x, *b = (const outcome *)y;
    if (a->p != b->p)
        return a->p > b->p ? -1 : 1;
    if (a->k != b->k)
        return a->k < b->k ? -1 : 1;
    return a->a < b->a ? -1 : (a->a > b->a);
}

/* Outcome scores and cache selection for R requests ([J++] Section 4.2,
 * "Outcome Selection"; Appendix F.1 and Proposition 1).  Row j of a request
 * (j = 0..gamma) holds logits that stand for the target's distribution of the
 * token following the anchor and draft tokens x_0..x_{j-1}; its softmax at
 * temperature T is p_j.  With p_j(x_j) the probability row j gives draft token x_j:
 *   P(k, a) = prod_{i<k} p_i(x_i) * p_k(a)   for k < gamma and a != x_k,
 *   P(gamma, a) = prod_{i<gamma} p_i(x_i) * p_gamma(a),
 * the probability that verification of the block ends with k accepted tokens
 * and extra token a.  The cache keeps the ncache most probable outcomes
 * (ties: smaller k, then smaller a; outcomes of probability 0 are never
 * kept, their slots hold k = a = -1 and probability 0); the hit probability
 * is the sum of the kept probabilities.  An invalid request (a token outside
 * [0, V), a NaN or +inf logit, a row without a finite logit) gets
 * k = a = -1 everywhere and hit probability -1.  all_scores
 * (nullable, [R][gamma+1][V]) receives every P(k, a), 0 where a = x_k. */
int oracle_outcome_topk(const void *logits, int dtype, const int32_t *draft_tokens, int R,
                        int gamma, int V, double T, int ncache, int32_t *out_k, int32_t *out_a,
                        double *out_p, double *hit, double *all_scores)
{
    if (!logits || !draft_tokens || !out_k || !out_a || !out_p || !hit)
        return -1;
    if (R < 1 || gamma < 1 || V < 1 || ncache < 1 || !(T > 0.0) || !isfinite(T))
        return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16)
        return -1;
    const int rows = gamma + 1;
    const int64_t n = (int64_t)rows * V;
    outcome *cand = malloc(sizeof(outcome) * (size_t)n);
    double *m = malloc(sizeof(double) * (size_t)rows);
    double *S = malloc(sizeof(double) * (size_t)rows);
    if (!cand || !m || !S) {
        free(cand);
        free(m);
        free(S);
        return -2;
    }
    for (int r = 0; r < R; ++r) {
        const int32_t *x = draft_tokens + (int64_t)r * gamma;
        const int64_t base = (int64_t)r * n;
        for (int c = 0; c < ncache; ++c) {
            out_k[(int64_t)r * ncache + c] = -1;
            out_a[(int64_t)r * ncache + c] = -1;
            out_p[(int64_t)r * ncache + c] = 0.0;
        }
        hit[r] = -1.0;
        if (all_scores)
            for (int64_t i = 0; i < n; ++i)
                all_scores[base + i] = 0.0;
        int bad = 0;
        for (int i = 0; i < gamma; ++i)
            bad |= (x[i] < 0 || x[i] >= V);
        for (int j = 0; j < rows && !bad; ++j)
            bad |= row_softmax_stats(logits, dtype, base + (int64_t)j * V, V, T, &m[j], &S[j]);
        if (bad)
            continue;
        double prefix = 1.0; /* prod_{i<k} p_i(x_i) */
        int64_t nc = 0;
        for (int k = 0; k < rows; ++k) {
            const int64_t row = base + (int64_t)k * V;
            for (int a = 0; a < V; ++a) {
                if (k < gamma && a == x[k])
                    continue;
                const double P = prefix * prob_at(logits, dtype, row, a, T, m[k], S[k]);
                if (all_scores)
                    all_scores[row + a] = P;
                if (P > 0.0) {
                    cand[nc].p = P;
                    cand[nc].k = k;
                    cand[nc].a = a;
                    ++nc;
                }
            }
            if (k < gamma)
                prefix *= prob_at(logits, dtype, row, x[k], T, m[k], S[k]);
        }
        qsort(cand, (size_t)nc, sizeof(outcome), outcome_cmp);
        double h = 0.0;
        for (int c = 0; c < ncache && c < nc; ++c) {
            out_k[(int64_t)r * ncache + c] = cand[c].k;
            out_a[(int64_t)r * ncache + c] = cand[c].a;
            out_p[(int64_t)r * ncache + c] = cand[c].p;
            h += cand[c].p;
        }
        hit[r] = h;
    }
    free(cand);
    free(m);
    free(S);
    return 0;
}

/* Per-position acceptance probability alpha_i = sum_v min(p_i(v), q_i(v)),
 * the probability that the test at position i passes when x ~ q_i
 * ([SD] "Rejection uses a residual distribution": accepted and residual
 * parts recombine to p).  Invalid rows give NaN.  Blocks are shared out over
 * up to nthreads threads. */
typedef struct {
    const void *target, *draft;
    int dtype, B, gamma, V, nthreads, tid;
    double T;
    double *alpha;
} alpha_arg;

static void *alpha_worker(void *p)
{
    const alpha_arg *A = (const alpha_arg *)p;
    const int gamma = A->gamma, V = A->V, dtype = A->dtype;
    for (int b = A->tid; b < A->B; b += A->nthreads)
        for (int i = 0; i < gamma; ++i) {
            int64_t pr = (int64_t)b * (gamma + 1) * V + (int64_t)i * V;
            int64_t qr = (int64_t)b * gamma * V + (int64_t)i * V;
            double mp, Sp, mq, Sq, a = 0.0;
            if (row_softmax_stats(A->target, dtype, pr, V, A->T, &mp, &Sp) ||
                row_softmax_stats(A->draft, dtype, qr, V, A->T, &mq, &Sq)) {
                A->alpha[(int64_t)b * gamma + i] = NAN;
                continue;
            }
            for (int v = 0; v < V; ++v)
                a += fmin(prob_at(A->target, dtype, pr, v, A->T, mp, Sp),
                          prob_at(A->draft, dtype, qr, v, A->T, mq, Sq));
            A->alpha[(int64_t)b * gamma + i] = a;
        }
    return NULL;
}

int oracle_chain_alpha(const void *target, const void *draft, int dtype, int B, int gamma, int V,
                       double T, double *alpha, int nthreads)
{
    if (!target || !draft || !alpha || B < 1 || gamma < 1 || V < 1 || !(T > 0.0))
        return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16)
        return -1;
    int nt = nthreads < 1 ? 1 : (nthreads > B ? B : nthreads);
    alpha_arg *args = malloc(sizeof(alpha_arg) * (size_t)nt);
    if (!args)
        return -2;
    for (int t = 0; t < nt; ++t) {
        alpha_arg a = {target, draft, dtype, B, gamma, V, nt, t, T, alpha};
        args[t] = a;
    }
    run_parallel(alpha_worker, args, sizeof(alpha_arg), nt);
    free(args);
    return 0;
}

/* ---------------------------------------------------------------- tree -- */

typedef struct {
    const void *target;
    int dtype;
    const int32_t *parents, *tokens;
    int B, n, V;
    int32_t *accept_len, *accept_node, *out_tokens, *amax_out;
    int32_t *scratch; /* [nthreads][3 n] */
    int nthreads;
} tree_job;

/* Greedy tree verification of one request ([JN] "Tree verification",
 * Fig. 5 and the greedy note; Eq. 17 for the accepted length). */
static void tree_request(const tree_job *J, int b, int32_t *scratch)
{
    const int n = J->n, V = J->V;
    const int32_t *par = J->parents + (int64_t)b * n;
    const int32_t *tok = J->tokens + (int64_t)b * n;
    int32_t *out = J->out_tokens + (int64_t)b * n;
    for (int j = 0; j < n; ++j)
        out[j] = -1;
    J->accept_len[b] = -1;
    J->accept_node[b] = -1;
    if (J->amax_out)
        for (int j = 0; j < n; ++j)
            J->amax_out[(int64_t)b * n + j] = -1;

    /* Parent array: node 0 is the root; every other node's parent precedes
     * it (Algorithm 1 adds a child only under an existing node). */
    if (par[0] != -1)
        return;
    for (int j = 1; j < n; ++j)
        if (par[j] < 0 || par[j] >= j || tok[j] < 0 || tok[j] >= V)
            return;

    /* Target argmax of every node row, lowest token id on ties. */
    int32_t *amax = scratch, *acc = scratch + n, *depth = scratch + 2 * n;
    for (int j = 0; j < n; ++j) {
        int64_t off = ((int64_t)b * n + j) * V;
        double best = -INFINITY;
        int arg = -1;
        for (int v = 0; v < V; ++v) {
            double z = logit_at(J->target, J->dtype, off + v);
            if (isnan(z) || z == INFINITY)
                return;
            if (z > best) {
                best = z;
                arg = v;
            }
        }
        if (arg < 0)
            return; /* no finite logit in this row */
        amax[j] = arg;
    }
    if (J->amax_out)
        for (int j = 0; j < n; ++j)
            J->amax_out[(int64_t)b * n + j] = amax[j];

    /* A node is accepted iff its parent is and its token equals the target
     * argmax after the parent's path.  Parents precede children, so one
     * pass in index order suffices. */
    acc[0] = 1;
    depth[0] = 0;
    for (int j = 1; j < n; ++j) {
        acc[j] = acc[par[j]] && tok[j] == amax[par[j]];
        depth[j] = depth[par[j]] + 1;
    }
    int best = 0;
    for (int j = 1; j < n; ++j)
        if (acc[j] && depth[j] > depth[best])
            best = j;
    /* Emit the accepted path root->best (root excluded), then the target
     * argmax after it (the bonus token). */
    for (int j = best; j != 0; j = par[j])
        out[depth[j] - 1] = tok[j];
    out[depth[best]] = amax[best];
    J->accept_len[b] = depth[best];
    J->accept_node[b] = best;
}

typedef struct {
    const tree_job *J;
    int tid;
} tree_arg;

static void *tree_worker(void *p)
{
    const tree_arg *a = (const tree_arg *)p;
    int32_t *scratch = a->J->scratch + (int64_t)a->tid * 3 * a->J->n;
    for (int b = a->tid; b < a->J->B; b += a->J->nthreads)
        tree_request(a->J, b, scratch);
    return NULL;
}

int oracle_tree_greedy(const void *target, int dtype, const int32_t *parents,
                       const int32_t *tokens, int B, int n, int V, int32_t *accept_len,
                       int32_t *accept_node, int32_t *out_tokens, int32_t *amax_out,
                       int nthreads)
{
    if (!target || !parents || !tokens || !accept_len || !accept_node || !out_tokens)
        return -1;
    if (B < 1 || n < 1 || V < 1 || (dtype != ORC_F32 && dtype != ORC_BF16))
        return -1;
    tree_job J = {target, dtype, parents, tokens, B, n, V, accept_len, accept_node, out_tokens,
                  amax_out, NULL, nthreads < 1 ? 1 : nthreads};
    if (J.nthreads > B)
        J.nthreads = B;
    J.scratch = malloc(sizeof(int32_t) * 3 * (size_t)n * (size_t)J.nthreads);
    tree_arg *args = malloc(sizeof(tree_arg) * (size_t)J.nthreads);
    if (!J.scratch || !args) {
        free(J.scratch);
        free(args);
        return -2;
    }
    for (int i = 0; i < J.nthreads; ++i) {
        args[i].J = &J;
        args[i].tid = i;
    }
    run_parallel(tree_worker, args, sizeof(tree_arg), J.nthreads);
    free(args);
    free(J.scratch);
    return 0;
}

/* ----------------------------------------------------------------------
 * Tree construction by best-first search ([JN] Algorithm 1, with the branch
 * score of Eq. 15).
 *
 * Each request has M rows of draft logits, one per potential node: row m is
 * the draft distribution q_m (softmax at temperature T) of the token that
 * follows potential node m's path, and row 0 belongs to the root (the
 * verified prefix).  The pages have the draft head produce these rows in one
 * pass before the search starts.  C(v), the candidate children of a node
 * whose row is m, are the W most probable tokens of q_m (ties: the smaller
 * token id; tokens of probability 0 are not candidates).  The child reached
 * through the j-th of them has row child_row[m][j] (-1: it has no row and is
 * never expanded).  With child_row NULL the potential nodes are numbered
 * breadth first in a complete W-ary tree: child j of row m has row
 * m*W + 1 + j if that is below M, else none.
 *
 * The search: the tree starts as the root alone (node 0, depth 0, score 0)
 * and the queue holds the root.  While the tree has fewer than `budget` nodes
 * and the queue is not empty, the node with the highest score leaves the
 * queue (ties: the smaller node index, i.e. the one added first).  A node at
 * depth N or without a row is not expanded.  Otherwise each candidate child y
 * in turn is added to the tree -- next node index, parent v, token y, score
 * s_v + ln q_m(y), the sum of the draft log probabilities along the path
 * ([JN] Eq. 15) -- and enters the queue, until the tree holds `budget` nodes.
 *
 * Outputs per request ([R][budget]): parents (root -1), tokens (root -1),
 * node_row (-1 for none), score (natural log; -inf past the end), and
 * n_nodes [R]; past the end parents, tokens and node_row are -1.  An invalid
 * request (a NaN or +inf logit, or a row without a finite logit, in any of
 * its M rows) gets n_nodes = -1 and every node output
 * -1 / -inf; a child_row entry outside [-1, M) makes every request invalid.
 * min_gap (nullable, [R]) receives, over the pops that expand a node, the
 * smallest difference between the popped score and the score of any other
 * expandable node in the queue, leaving out exact ties between siblings
 * (equal logits in one row tie exactly in any arithmetic); +inf if there is
 * none.  A small gap marks an order that rounding elsewhere may swap.
 */
int oracle_tree_build(const void *logits, int dtype, int R, int M, int V, double T, int W, int N,
                      int budget, const int32_t *child_row, int32_t *parents, int32_t *tokens,
                      int32_t *node_row, double *score, int32_t *n_nodes, double *min_gap)
{
    if (!logits || !parents || !tokens || !node_row || !score || !n_nodes)
        return -1;
    if (R < 1 || M < 1 || V < 1 || W < 1 || N < 1 || budget < 1 || !(T > 0.0) || !isfinite(T))
        return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16)
        return -1;
    int map_ok = 1;
    if (child_row)
        for (int64_t i = 0; i < (int64_t)M * W; ++i)
            map_ok &= (child_row[i] >= -1 && child_row[i] < M);
    double *m = malloc(sizeof(double) * (size_t)M);
    double *S = malloc(sizeof(double) * (size_t)M);
    int *depth = malloc(sizeof(int) * (size_t)budget);
    char *inq = malloc((size_t)budget);
    int *ctok = malloc(sizeof(int) * (size_t)W);
    char *taken = malloc((size_t)V);
    if (!m || !S || !depth || !inq || !ctok || !taken) {
        free(m);
        free(S);
        free(depth);
        free(inq);
        free(ctok);
        free(taken);
        return -2;
    }
    for (int r = 0; r < R; ++r) {
        const int64_t o = (int64_t)r * budget;
        int32_t *par = parents + o, *tok = tokens + o, *row = node_row + o;
        double *sc = score + o;
        for (int i = 0; i < budget; ++i) {
            par[i] = tok[i] = row[i] = -1;
            sc[i] = -INFINITY;
        }
        n_nodes[r] = -1;
        if (min_gap)
            min_gap[r] = INFINITY;
        const int64_t base = (int64_t)r * M * V;
        int bad = !map_ok;
        for (int j = 0; j < M && !bad; ++j)
            bad |= row_softmax_stats(logits, dtype, base + (int64_t)j * V, V, T, &m[j], &S[j]);
        if (bad)
            continue;
        int n = 1;
        row[0] = 0;
        sc[0] = 0.0;
        depth[0] = 0;
        inq[0] = 1;
        double gap = INFINITY;
        while (n < budget) {
            int v = -1;
            for (int u = 0; u < n; ++u)
                if (inq[u] && (v < 0 || sc[u] > sc[v]))
                    v = u;
            if (v < 0)
                break;
            inq[v] = 0;
            if (depth[v] >= N || row[v] < 0)
                continue;
            for (int u = 0; u < n; ++u) {
                if (!inq[u] || depth[u] >= N || row[u] < 0)
                    continue;
                if (par[u] == par[v] && sc[u] == sc[v])
                    continue;
                if (sc[v] - sc[u] < gap)
                    gap = sc[v] - sc[u];
            }
            /* C(v): the W most probable tokens of the row, by selection */
            const int64_t off = base + (int64_t)row[v] * V;
            memset(taken, 0, (size_t)V);
            int nc = 0;
            for (int j = 0; j < W; ++j) {
                int best = -1;
                double bz = -INFINITY;
                for (int y = 0; y < V; ++y) {
                    const double z = logit_at(logits, dtype, off + y);
                    if (!taken[y] && z > bz) {
                        bz = z;
                        best = y;
                    }
                }
                if (best < 0)
                    break; /* only probability-0 tokens are left */
                taken[best] = 1;
                ctok[nc++] = best;
            }
            for (int j = 0; j < nc && n < budget; ++j) {
                const int u = n++;
                const int mr = row[v];
                par[u] = v;
                tok[u] = ctok[j];
                if (child_row)
                    row[u] = child_row[(int64_t)mr * W + j];
                else
                    row[u] = ((int64_t)mr * W + 1 + j < M) ? mr * W + 1 + j : -1;
                depth[u] = depth[v] + 1;
                sc[u] = sc[v] + logprob_at(logits, dtype, off, ctok[j], T, m[mr], S[mr]);
                inq[u] = 1;
            }
        }
        n_nodes[r] = n;
        if (min_gap)
            min_gap[r] = gap;
    }
    free(m);
    free(S);
    free(depth);
    free(inq);
    free(ctok);
    free(taken);
    return 0;
}

/* Scores of a given tree under the draft rows ([JN] Eq. 15: a node's score
 * is the sum of the draft log probabilities ln q(token) along its path, each
 * token taken in the row of its parent).  For each request r with
 * n = n_nodes[r] nodes (parents[r][0] = -1, 0 <= parents[r][j] < j, every
 * parent with a child having a row in [0, M), tokens in [0, V)): score[r][0]
 * = 0 and score[r][j] = score[r][parents[j]] + ln q_{row(parents[j])}(
 * tokens[j]); -inf past the last node.  A request whose tree breaks those
 * conditions, or one with a NaN, +inf or all -inf row among the rows it uses,
 * gets NaN scores.  (Tests use it to score a tree built elsewhere.) */
int oracle_tree_score(const void *logits, int dtype, int R, int M, int V, double T, int budget,
                      const int32_t *parents, const int32_t *tokens, const int32_t *node_row,
                      const int32_t *n_nodes, double *score)
{
    if (!logits || !parents || !tokens || !node_row || !n_nodes || !score)
        return -1;
    if (R < 1 || M < 1 || V < 1 || budget < 1 || !(T > 0.0) || !isfinite(T))
        return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16)
        return -1;
    for (int r = 0; r < R; ++r) {
        const int64_t o = (int64_t)r * budget;
        const int32_t *par = parents + o, *tok = tokens + o, *row = node_row + o;
        double *sc = score + o;
        const int n = n_nodes[r];
        for (int j = 0; j < budget; ++j)
            sc[j] = -INFINITY;
        int bad = n < 1 || n > budget || par[0] != -1;
        for (int j = 1; j < n && !bad; ++j)
            bad |= par[j] < 0 || par[j] >= j || tok[j] < 0 || tok[j] >= V ||
                   row[par[j]] < 0 || row[par[j]] >= M;
        if (!bad) {
            sc[0] = 0.0;
            for (int j = 1; j < n && !bad; ++j) {
                const int64_t off = ((int64_t)r * M + row[par[j]]) * V;
                double m, S;
                if (row_softmax_stats(logits, dtype, off, V, T, &m, &S)) {
                    bad = 1;
                    break;
                }
                sc[j] = sc[par[j]] + logprob_at(logits, dtype, off, tok[j], T, m, S);
            }
        }
        if (bad)
            for (int j = 0; j < budget; ++j)
                sc[j] = NAN;
    }
    return 0;
}

/* ----------------------------------------------------------------------
 * Stochastic tree verification ([JN] section "Tree verification", Eq. 16-17
 * and Fig. 5).
 *
 * Request b holds a candidate tree of n nodes: parents[b][0] = -1 (node 0 is
 * the root, the verified prefix), 0 <= parents[b][j] < j, tokens[b][j] the
 * token of node j (node 0's is not used).  Target row j and draft row j are
 * the target's and the draft's next-token logits after node j's path; p_j
 * and q_j are their softmax at temperature T.
 *  - Every node j >= 1 takes one Bernoulli test (Eq. 16) with probability
 *    alpha_j = min(1, p_par(y_j) / q_par(y_j)), par = parents[j], y_j its
 *    token: accepted iff u[b][j] < alpha_j (a node shared by several
 *    branches is tested once).  As in the chain rule, alpha = 0 when
 *    p_par(y) = 0 and alpha = 1 when q_par(y) = 0 < p_par(y).
 *  - A branch keeps its longest prefix of accepted tokens (Eq. 17): node j
 *    counts as accepted iff its parent does and its own test passes; the
 *    root counts as accepted.
 *  - The best branch ends at the deepest accepted node v* (the lowest index
 *    among equally deep ones); its tokens are committed.
 *  - The correction token is drawn from p_{v*}, the target distribution
 *    after the accepted path (as Fig. 5 shows), by inverse CDF in ascending
 *    token id with u[b][0]: the smallest v with sum_{t<=v} p(t) > u * W
 *    (W the total), else the last v of positive probability.  The pages give
 *    no residual rule for a branch rejected below v*, so none is applied.
 * Outputs as for greedy tree verification: accept_len[b] = depth of v*,
 * accept_node[b] = v*, out_tokens[b][0..n) the path root -> v* (root
 * excluded), the drawn token, then -1.  final_dist (nullable, [B][V])
 * receives p_{v*}; margin (nullable, [B]) the smallest |u_j - alpha_j| over
 * the nodes whose parent is accepted, and the draw's distance to the nearest
 * CDF breakpoint relative to W; alpha (nullable, [B][n]) every node's test
 * probability alpha_j (NaN for the root and for an invalid request).  An
 * invalid request (a malformed parent array, a token outside [0, V), a NaN
 * or +inf logit or a row without a finite logit in any target or draft row)
 * gets accept_len = accept_node = -1 and all tokens -1.
 * oracle_tree_stochastic_du takes double uniforms (the exact-enumeration
 * tests drive it with continuous u); oracle_tree_stochastic takes the
 * float32 uniforms of the library interface, each widened exactly.
 */
int oracle_tree_stochastic_du(const void *target, const void *draft, int dtype,
                              const int32_t *parents, const int32_t *tokens,
                              const double *uniforms, int B, int n, int V, double T,
                              int32_t *accept_len, int32_t *accept_node, int32_t *out_tokens,
                              double *final_dist, double *margin, double *alpha_out)
{
    if (!target || !draft || !parents || !tokens || !uniforms || !accept_len || !accept_node ||
        !out_tokens)
        return -1;
    if (B < 1 || n < 1 || V < 1 || !(T > 0.0) || !isfinite(T))
        return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16)
        return -1;
    double *mp = malloc(sizeof(double) * (size_t)n), *Sp = malloc(sizeof(double) * (size_t)n);
    double *mq = malloc(sizeof(double) * (size_t)n), *Sq = malloc(sizeof(double) * (size_t)n);
    int *acc = malloc(sizeof(int) * (size_t)n), *depth = malloc(sizeof(int) * (size_t)n);
    double *w = malloc(sizeof(double) * (size_t)V);
    int rc = 0;
    if (!mp || !Sp || !mq || !Sq || !acc || !depth || !w) {
        rc = -2;
        goto out;
    }
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parents + (int64_t)b * n, *tok = tokens + (int64_t)b * n;
        const double *u = uniforms + (int64_t)b * n;
        int32_t *out = out_tokens + (int64_t)b * n;
        const int64_t base = (int64_t)b * n * V;
        for (int j = 0; j < n; ++j)
            out[j] = -1;
        accept_len[b] = accept_node[b] = -1;
        if (margin)
            margin[b] = 0.0;
        if (alpha_out)
            for (int j = 0; j < n; ++j)
                alpha_out[(int64_t)b * n + j] = NAN;
        if (final_dist)
            for (int v = 0; v < V; ++v)
                final_dist[(int64_t)b * V + v] = 0.0;
        int bad = par[0] != -1;
        for (int j = 1; j < n && !bad; ++j)
            bad |= (par[j] < 0 || par[j] >= j || tok[j] < 0 || tok[j] >= V);
        for (int j = 0; j < n && !bad; ++j) {
            bad |= row_softmax_stats(target, dtype, base + (int64_t)j * V, V, T, &mp[j], &Sp[j]);
            if (!bad)
                bad |= row_softmax_stats(draft, dtype, base + (int64_t)j * V, V, T, &mq[j], &Sq[j]);
        }
        if (bad)
            continue;
        /* per-node tests, in index order (parents precede children) */
        double mg = INFINITY;
        acc[0] = 1;
        depth[0] = 0;
        for (int j = 1; j < n; ++j) {
            const int p = par[j];
            const double lp = logprob_at(target, dtype, base + (int64_t)p * V, tok[j], T, mp[p], Sp[p]);
            const double lq = logprob_at(draft, dtype, base + (int64_t)p * V, tok[j], T, mq[p], Sq[p]);
            double alpha;
            if (lp == -INFINITY)
                alpha = 0.0;
            else if (lq == -INFINITY)
                alpha = 1.0;
            else
                alpha = fmin(1.0, exp(lp - lq));
            if (alpha_out)
                alpha_out[(int64_t)b * n + j] = alpha;
            acc[j] = acc[p] && u[j] < alpha;
            depth[j] = depth[p] + 1;
            if (acc[p])
                mg = fmin(mg, fabs(u[j] - alpha));
        }
        int best = 0;
        for (int j = 1; j < n; ++j)
            if (acc[j] && depth[j] > depth[best])
                best = j;
        /* the correction from p at the deepest accepted node */
        const int64_t prow = base + (int64_t)best * V;
        double W = 0.0;
        for (int v = 0; v < V; ++v) {
            w[v] = prob_at(target, dtype, prow, v, T, mp[best], Sp[best]);
            W += w[v];
        }
        const double t = u[0] * W;
        double C = 0.0, Cprev = 0.0;
        int drawn = -1;
        for (int v = 0; v < V; ++v) {
            Cprev = C;
            C += w[v];
            if (C > t) {
                drawn = v;
                break;
            }
        }
        double mf;
        if (drawn < 0) {
            for (int v = V - 1; v >= 0; --v)
                if (w[v] > 0.0) {
                    drawn = v;
                    break;
                }
            mf = 0.0;
        } else {
            mf = fmin(t - Cprev, C - t) / W;
        }
        for (int j = best; j != 0; j = par[j])
            out[depth[j] - 1] = tok[j];
        out[depth[best]] = drawn;
        accept_len[b] = depth[best];
        accept_node[b] = best;
        if (margin)
            margin[b] = fmin(mg, mf);
        if (final_dist)
            for (int v = 0; v < V; ++v)
                final_dist[(int64_t)b * V + v] = w[v] / W;
    }
out:
    free(mp);
    free(Sp);
    free(mq);
    free(Sq);
    free(acc);
    free(depth);
    free(w);
    return rc;
}

int oracle_tree_stochastic(const void *target, const void *draft, int dtype,
                           const int32_t *parents, const int32_t *tokens, const float *uniforms,
                           int B, int n, int V, double T, int32_t *accept_len,
                           int32_t *accept_node, int32_t *out_tokens, double *final_dist,
                           double *margin, double *alpha_out)
{
    if (!uniforms || B < 1 || n < 1)
        return -1;
    const size_t nu = (size_t)B * (size_t)n;
    double *ud = malloc(sizeof(double) * nu);
    if (!ud)
        return -2;
    for (size_t i = 0; i < nu; ++i)
        ud[i] = (double)uniforms[i];
    const int rc = oracle_tree_stochastic_du(target, draft, dtype, parents, tokens, ud, B, n, V,
                                             T, accept_len, accept_node, out_tokens, final_dist,
                                             margin, alpha_out);
    free(ud);
    return rc;
}
