/*
 * specverify_oracle.c -- plain, slow, double-precision CPU oracle of the
 * speculative-sampling verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or constant table with the HIP
 * library: every step below is written out again from the method's definition.
 *
 * Sources (cited by page title and section):
 *  - "Kangaroo: Self-Speculative Decoding via Shallow Sub-Networks",
 *    section "3. Lossless Speculative Verification": accept draft token x_i
 *    when a uniform r satisfies r <= min(1, p_i/q_i); at the first rejection
 *    emit a sample of max(0, p_i - q_i) normalised over the vocabulary and
 *    stop.  Its simulation listing counts one guaranteed extra (bonus) token.
 *  - glossary "speculative decoding llm", sections "How Speculative Decoding
 *    Works" and "Why It Produces Identical Outputs": same accept rule and
 *    residual; the output law equals the target's.
 *  - "Speculative Speculative Decoding", sections "Key claims" and "Method":
 *    the bonus token comes from the residual max(p_t - p_d, 0); Saguaro
 *    down-weights the most likely draft probabilities by a factor beta.
 *  - "LayerSkip Guide: Early Exit & Self-Speculative Decoding", section
 *    "2. The Drafting and Single-Pass Verification Pipeline": greedy mode
 *    accepts drafts while they equal the target argmax, then emits the
 *    target argmax.
 *  - Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers:
 *    As Easy as 1, 2, 3", SC'11 (a published counter-based generator; the
 *    pages only ask for reproducible uniforms).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - accept iff u <= ratio (inclusive); u in (0,1] with 2^-24 resolution;
 *  - the bonus after acceptance of all K drafts is drawn from target row K;
 *  - the residual is clamped at zero; if its mass is exactly zero the bonus
 *    is drawn from the target row of that position instead;
 *  - inverse CDF in ascending token id: smallest v with C(v) >= u * Z;
 *  - greedy ties go to the lowest token id;
 *  - both softmaxes use the same per-sequence temperature T; T == 0 is greedy;
 *  - beta multiplies the probabilities of the 4 largest draft logits (ties by
 *    lower token id) and the draft law is renormalised; beta == 1 is off;
 *  - a draft token outside [0, V) is rejected (ratio 0) and flagged;
 *  - ragged draft lengths (Kangaroo's second early exit stops drafting once
 *    the draft's confidence falls below a threshold, so a round carries
 *    K_b <= K drafts): sequence b verifies positions 0..K_b-1 and draws the
 *    bonus from target row K_b after K_b acceptances, with the uniforms keyed
 *    exactly as for K = K_b; rows past K_b are never read;
 *  - the draft confidence of position i is max_v p_d(v) of draft row i at the
 *    sequence temperature, before the beta re-weighting (NaN for greedy
 *    sequences, whose draft rows are not read);
 *  - the verification-outcome distribution ("Speculative Speculative
 *    Decoding", "Method") is taken over drafts drawn from the (beta-weighted)
 *    draft law the verify step assumes, for all K positions whatever was
 *    drafted; "the most likely bonus tokens" of a position are ranked by the
 *    clamped residual mass max(p - q', 0) (target mass at position K), ties
 *    to the lower token id; greedy sequences have no outcome law (NaN);
 *  - tree verification (named on the pages without a rule) follows the
 *    published recursive rejection sampling: children of a context are tried
 *    in node order against the current law, which a rejection replaces by
 *    its normalised residual; node j's test uses u(b, j, 0), the bonus
 *    u(b, d, 1) with d the accepted depth, so a chain is the verify step.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F32 0
#define OR_BF16 1

#define OR_ACCEPT 0u
#define OR_BONUS 1u

#define OR_ERR_TOKEN 1       /* a draft token outside [0, V)              */
#define OR_ERR_TEMPERATURE 2 /* T < 0, NaN or infinite                    */
#define OR_ERR_ROW 4         /* a row whose maximum logit is not finite   */
#define OR_ERR_DRAFT_MASS 8  /* beta re-weighting left zero draft mass    */
#define OR_ERR_NO_DRAFT 16   /* T > 0 and K > 0 but no draft logits given */
#define OR_ERR_DRAFT_LEN 32  /* a ragged draft length outside [0, K]       */
#define OR_ERR_TREE 64       /* a tree parent outside [-1, i-1]           */

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (SC'11): 10 rounds of a multiply/xor S-box; the 2-word key
 * advances by the Weyl constants before every round after the first.       */

static void or_philox_round(uint32_t c[4], const uint32_t k[2])
{
    uint64_t prod0 = (uint64_t)0xD2511F53u * (uint64_t)c[0];
    uint64_t prod1 = (uint64_t)0xCD9E8D57u * (uint64_t)c[2];
    uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
    uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
    uint32_t n0 = hi1 ^ c[1] ^ k[0];
    uint32_t n2 = hi0 ^ c[3] ^ k[1];
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
}

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k[0] += 0x9E3779B9u;
            k[1] += 0xBB67AE85u;
        }
        or_philox_round(c, k);
    }
    out[0] = c[0];
    out[1] = c[1];
    out[2] = c[2];
    out[3] = c[3];
}

/* Uniform keyed by (seed, sequence, position, purpose): key = seed split into
 * low/high words, counter = (b, pos, purpose, 0), first output word mapped to
 * ((w >> 8) + 1) * 2^-24, which lies in (0, 1] and is exact in float.      */
double oracle_uniform(uint64_t seed, uint32_t b, uint32_t pos, uint32_t purpose)
{
    uint32_t ctr[4] = {b, pos, purpose, 0u};
    uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return (double)((out[0] >> 8) + 1u) * (1.0 / 16777216.0);
}

/* ------------------------------------------------------------------ */
/* Reading logits: bf16 and fp32 both convert to double exactly.             */

static double or_logit(const void *base, int dtype, size_t idx)
{
    if (dtype == OR_F32) {
        return (double)((const float *)base)[idx];
    }
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Largest logit of a row (plain scan). */
double oracle_row_max(const void *row, int dtype, int32_t V)
{
    double m = -INFINITY;
    for (int32_t v = 0; v < V; ++v) {
        double z = or_logit(row, dtype, (size_t)v);
        if (z > m) m = z;
    }
    return m;
}

/* Index of the largest logit, lowest index on ties. */
int32_t oracle_row_argmax(const void *row, int dtype, int32_t V)
{
    int32_t best = 0;
    double bestz = or_logit(row, dtype, 0);
    for (int32_t v = 1; v < V; ++v) {
        double z = or_logit(row, dtype, (size_t)v);
        if (z > bestz) {
            bestz = z;
            best = v;
        }
    }
    return best;
}

/* L = log sum_v exp(z_v / T): the normaliser of softmax(z / T).
 * ln p(v) = z_v / T - L.                                                     */
double oracle_row_lognorm(const void *row, int dtype, int32_t V, double T)
{
    double m = -INFINITY;
    for (int32_t v = 0; v < V; ++v) {
        double a = or_logit(row, dtype, (size_t)v) / T;
        if (a > m) m = a;
    }
    double s = 0.0;
    for (int32_t v = 0; v < V; ++v) {
        double a = or_logit(row, dtype, (size_t)v) / T;
        s += exp(a - m);
    }
    return m + log(s);
}

/* The min(4, V) largest logits of a row, ordered by (logit descending,
 * index ascending).  Plain repeated selection.                              */
int32_t oracle_row_top4(const void *row, int dtype, int32_t V, int32_t idx[4])
{
    int32_t count = V < 4 ? V : 4;
    for (int32_t j = 0; j < count; ++j) {
        int32_t best = -1;
        double bestz = 0.0;
        for (int32_t v = 0; v < V; ++v) {
            int taken = 0;
            for (int32_t q = 0; q < j; ++q)
                if (idx[q] == v) taken = 1;
            if (taken) continue;
            double z = or_logit(row, dtype, (size_t)v);
            if (best < 0 || z > bestz) {
                best = v;
                bestz = z;
            }
        }
        idx[j] = best;
    }
    for (int32_t j = count; j < 4; ++j) idx[j] = -1;
    return count;
}

/* A prepared row: its normaliser and, for a beta-weighted draft row, the
 * down-weighted tokens and the renormalisation log N.                       */
typedef struct {
    const void *z;
    int dtype;
    int32_t V;
    double T;
    double L;          /* log sum exp(z / T)                                  */
    int weighted;      /* beta re-weighting active                            */
    double beta;
    int32_t top[4];    /* down-weighted tokens                                */
    int32_t ntop;
    double logN;       /* log sum_v w(v) p(v)                                 */
} or_row;

static double or_weight(const or_row *r, int32_t v)
{
    if (!r->weighted) return 1.0;
    for (int32_t j = 0; j < r->ntop; ++j)
        if (r->top[j] == v) return r->beta;
    return 1.0;
}

/* ln p(v) for a prepared row; for a weighted draft row this is
 * ln w(v) + ln p(v) - ln N  (w(v) = beta on the top tokens, 1 elsewhere).   */
static double or_logprob(const or_row *r, int32_t v)
{
    double lp = or_logit(r->z, r->dtype, (size_t)v) / r->T - r->L;
    if (r->weighted) {
        double w = or_weight(r, v);
        lp += log(w) - r->logN; /* log(0) = -inf for beta == 0 */
    }
    return lp;
}

static int or_prepare(or_row *r, const void *z, int dtype, int32_t V, double T, int weighted,
                      double beta)
{
    r->z = z;
    r->dtype = dtype;
    r->V = V;
    r->T = T;
    r->weighted = weighted;
    r->beta = beta;
    r->ntop = 0;
    r->logN = 0.0;
    double m = oracle_row_max(z, dtype, V);
    if (!isfinite(m)) return OR_ERR_ROW;
    r->L = oracle_row_lognorm(z, dtype, V, T);
    if (weighted) {
        r->ntop = oracle_row_top4(z, dtype, V, r->top);
        /* N = sum_v w(v) p(v), summed over the whole vocabulary. */
        double N = 0.0;
        for (int32_t v = 0; v < V; ++v) {
            double p = exp(or_logit(z, dtype, (size_t)v) / T - r->L);
            N += or_weight(r, v) * p;
        }
        if (!(N > 0.0)) return OR_ERR_DRAFT_MASS;
        r->logN = log(N);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Full verify step for one sequence.                                        */

typedef struct {
    const void *target;   /* [B, K+1, V] */
    const void *draft;    /* [B, K, V] (may be NULL when every T == 0) */
    const int32_t *tokens;/* [B, K] */
    int32_t B, K, V;
    int dtype;
    uint64_t seed;
    const float *temperature; /* [B] */
    double beta;
    int32_t *accepted_len;    /* [B] */
    int32_t *out_tokens;      /* [B, K+1] */
    double *p_target;         /* [B, K]   or NULL */
    double *p_draft;          /* [B, K]   or NULL */
    double *residual_mass;    /* [B]      or NULL */
    double *margin_accept;    /* [B, K]   or NULL */
    double *margin_bonus;     /* [B]      or NULL */
    int32_t *seq_error;       /* [B]      or NULL */
    const int32_t *seq_ids;   /* [B] global sequence index used by the uniforms, or NULL */
    const int32_t *draft_len; /* [B] drafts of each sequence (K_b <= K), or NULL for K */
    double *draft_conf;       /* [B, K]   or NULL */
    const uint8_t *force;     /* [B, K] nonzero: that accept test takes the other outcome, or NULL */
} or_call;

static const void *or_row_ptr(const void *base, int dtype, size_t row, int32_t V)
{
    size_t elt = dtype == OR_F32 ? 4u : 2u;
    return (const char *)base + row * (size_t)V * elt;
}

/* A sequence that cannot be verified: no accepted drafts, every output
 * token -1 and every diagnostic NaN. */
static void or_fail_sequence(const or_call *c, int32_t b)
{
    c->accepted_len[b] = 0;
    for (int32_t j = 0; j <= c->K; ++j) c->out_tokens[(size_t)b * (c->K + 1) + j] = -1;
    for (int32_t i = 0; i < c->K; ++i) {
        if (c->p_target) c->p_target[(size_t)b * c->K + i] = NAN;
        if (c->p_draft) c->p_draft[(size_t)b * c->K + i] = NAN;
        if (c->margin_accept) c->margin_accept[(size_t)b * c->K + i] = NAN;
        if (c->draft_conf) c->draft_conf[(size_t)b * c->K + i] = NAN;
    }
    if (c->residual_mass) c->residual_mass[b] = NAN;
    if (c->margin_bonus) c->margin_bonus[b] = NAN;
}

static int or_verify_sequence(const or_call *c, int32_t b)
{
    const int32_t Kr = c->K, V = c->V; /* row layout: K + 1 target rows, K draft rows */
    int err = 0;
    int32_t *out = c->out_tokens + (size_t)b * (Kr + 1);
    const int32_t *x = c->tokens + (size_t)b * Kr;
    const uint32_t gb = c->seq_ids ? (uint32_t)c->seq_ids[b] : (uint32_t)b;
    const double nan = NAN;

    for (int32_t j = 0; j <= Kr; ++j) out[j] = -1;
    for (int32_t i = 0; i < Kr; ++i) {
        if (c->p_target) c->p_target[(size_t)b * Kr + i] = nan;
        if (c->p_draft) c->p_draft[(size_t)b * Kr + i] = nan;
        if (c->margin_accept) c->margin_accept[(size_t)b * Kr + i] = nan;
        if (c->draft_conf) c->draft_conf[(size_t)b * Kr + i] = nan;
    }
    if (c->residual_mass) c->residual_mass[b] = nan;
    if (c->margin_bonus) c->margin_bonus[b] = nan;

    /* this sequence's drafts: positions 0..K-1 are verified, row K is the bonus row */
    const int32_t K = c->draft_len ? c->draft_len[b] : Kr;
    if (K < 0 || K > Kr) {
        or_fail_sequence(c, b);
        return OR_ERR_DRAFT_LEN;
    }

    double T = (double)c->temperature[b];
    if (!(T >= 0.0) || isinf(T)) {
        or_fail_sequence(c, b);
        return OR_ERR_TEMPERATURE;
    }

    if (T == 0.0) {
        /* Greedy: accept while the draft equals the target argmax; the first
         * mismatch (or position K) emits the target argmax.                 */
        int32_t n = K;
        for (int32_t i = 0; i <= K; ++i) {
            const void *row = or_row_ptr(c->target, c->dtype, (size_t)b * (Kr + 1) + i, V);
            if (!isfinite(oracle_row_max(row, c->dtype, V))) {
                or_fail_sequence(c, b);
                return err | OR_ERR_ROW;
            }
            int32_t a = oracle_row_argmax(row, c->dtype, V);
            if (i < K && x[i] == a) {
                out[i] = x[i];
                continue;
            }
            if (i < K && (x[i] < 0 || x[i] >= V)) err |= OR_ERR_TOKEN;
            out[i] = a;
            n = i;
            break;
        }
        c->accepted_len[b] = n;
        return err;
    }

    if (K > 0 && c->draft == NULL) {
        or_fail_sequence(c, b);
        return OR_ERR_NO_DRAFT;
    }

    /* Draft confidence of each drafted position: max_v p_d(v) = exp(m/T - L),
     * before any beta re-weighting (every drafted row, reached or not). */
    if (c->draft_conf)
        for (int32_t i = 0; i < K; ++i) {
            const void *row = or_row_ptr(c->draft, c->dtype, (size_t)b * Kr + i, V);
            double m = oracle_row_max(row, c->dtype, V);
            c->draft_conf[(size_t)b * Kr + i] =
                isfinite(m) ? exp(m / T - oracle_row_lognorm(row, c->dtype, V, T)) : nan;
        }

    /* Sampling: accept x_i iff u_i <= ratio_i = p_t(x_i) / p_d'(x_i). */
    int weighted = c->beta < 1.0;
    int32_t n = K;
    or_row rt, rd;
    for (int32_t i = 0; i < K; ++i) {
        int e = or_prepare(&rt, or_row_ptr(c->target, c->dtype, (size_t)b * (Kr + 1) + i, V),
                           c->dtype, V, T, 0, 1.0);
        e |= or_prepare(&rd, or_row_ptr(c->draft, c->dtype, (size_t)b * Kr + i, V), c->dtype, V,
                        T, weighted, c->beta);
        if (e) {
            or_fail_sequence(c, b);
            return err | e;
        }
        double ratio;
        if (x[i] < 0 || x[i] >= V) {
            err |= OR_ERR_TOKEN;
            ratio = 0.0;
        } else {
            double lpt = or_logprob(&rt, x[i]);
            double lpd = or_logprob(&rd, x[i]);
            if (c->p_target) c->p_target[(size_t)b * Kr + i] = exp(lpt);
            if (c->p_draft) c->p_draft[(size_t)b * Kr + i] = exp(lpd);
            /* a draft token the draft law gives zero mass cannot be rejected */
            ratio = (lpd == -INFINITY) ? INFINITY : exp(lpt - lpd);
        }
        double u = oracle_uniform(c->seed, gb, (uint32_t)i, OR_ACCEPT);
        if (c->margin_accept) c->margin_accept[(size_t)b * Kr + i] = fabs(u - ratio);
        int accept = u <= ratio;
        /* parity checks only: a decision another finite-precision path took
         * the other way (its margin being within rounding) is replayed so
         * that the rest of the sequence can still be compared */
        if (c->force && c->force[(size_t)b * Kr + i]) accept = !accept;
        if (accept) {
            out[i] = x[i];
            continue;
        }
        n = i;
        break;
    }

    /* Residual law at position n: max(p_t - p_d', 0) after a rejection,
     * the target row K itself after K acceptances.                        */
    int e = or_prepare(&rt, or_row_ptr(c->target, c->dtype, (size_t)b * (Kr + 1) + n, V), c->dtype,
                       V, T, 0, 1.0);
    if (n < K)
        e |= or_prepare(&rd, or_row_ptr(c->draft, c->dtype, (size_t)b * Kr + n, V), c->dtype, V, T,
                        weighted, c->beta);
    if (e) {
        or_fail_sequence(c, b);
        return err | e;
    }
    double *r = (double *)malloc(sizeof(double) * (size_t)V);
    double Z = 0.0;
    for (int32_t v = 0; v < V; ++v) {
        double pt = exp(or_logprob(&rt, v));
        r[v] = pt;
        if (n < K) {
            double d = pt - exp(or_logprob(&rd, v));
            r[v] = d > 0.0 ? d : 0.0;
        }
        Z += r[v];
    }
    if (Z == 0.0) {
        /* zero residual mass can only come from rounding: use p_t instead */
        Z = 0.0;
        for (int32_t v = 0; v < V; ++v) {
            r[v] = exp(or_logprob(&rt, v));
            Z += r[v];
        }
    }
    /* Inverse CDF over ascending token ids: smallest v with C(v) >= u Z.
     * C is the same running sum that produced Z, so C(V-1) == Z.          */
    double uB = oracle_uniform(c->seed, gb, (uint32_t)n, OR_BONUS);
    double thr = uB * Z;
    double C = 0.0, Cprev = 0.0;
    int32_t bonus = -1;
    for (int32_t v = 0; v < V; ++v) {
        Cprev = C;
        C += r[v];
        if (C >= thr) {
            bonus = v;
            break;
        }
    }
    if (bonus < 0) { /* unreachable: C(V-1) == Z >= u Z */
        for (int32_t v = V - 1; v >= 0; --v)
            if (r[v] > 0.0) {
                bonus = v;
                break;
            }
        C = Z;
    }
    free(r);
    out[n] = bonus;
    c->accepted_len[b] = n;
    if (c->residual_mass) c->residual_mass[b] = Z;
    if (c->margin_bonus) {
        double m1 = fabs(uB - Cprev / Z), m2 = fabs(uB - C / Z);
        c->margin_bonus[b] = m1 < m2 ? m1 : m2;
    }
    return err;
}

/* Verify every sequence of a batch.  Returns the OR of the error bits.
 * nthreads <= 0 uses the OpenMP default; sequences are independent, so the
 * result does not depend on the thread count.  force [B, K] (or NULL) names
 * accept tests whose outcome is reversed: a parity check replays a decision
 * that sat within rounding of its threshold the way the other implementation
 * took it, and compares the rest of the sequence.                           */
int32_t oracle_spec_verify_ragged(const void *target, const void *draft, const int32_t *tokens,
                                  const int32_t *draft_len, int32_t B, int32_t K, int32_t V,
                                  int32_t dtype, uint64_t seed, const float *temperature,
                                  double beta, int32_t *accepted_len, int32_t *out_tokens,
                                  double *p_target, double *p_draft, double *residual_mass,
                                  double *margin_accept, double *margin_bonus, int32_t *seq_error,
                                  double *draft_conf, const int32_t *seq_ids, const uint8_t *force,
                                  int32_t nthreads)
{
    or_call c = {target, draft, tokens, B, K, V, dtype, seed, temperature, beta,
                 accepted_len, out_tokens, p_target, p_draft, residual_mass,
                 margin_accept, margin_bonus, seq_error, seq_ids, draft_len, draft_conf, force};
    int32_t all_err = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : all_err)
#endif
    for (int32_t b = 0; b < B; ++b) {
        int e = or_verify_sequence(&c, b);
        if (seq_error) seq_error[b] = e;
        all_err |= e;
    }
    return all_err;
}

/* ------------------------------------------------------------------ */
/* Verification-outcome distribution ("Speculative Speculative Decoding",
 * "Method": a verification outcome is the accepted prefix length plus the
 * bonus token's identity; the speculator prepares the likeliest ones).
 * Over drafts drawn from the draft law, position j accepts with probability
 * alpha_j = sum_v min(p_j(v), q'_j(v)) and, on a rejection, emits v with
 * probability r_j(v) / (1 - alpha_j), r_j = max(p_j - q'_j, 0); so
 *   P(n = k) = (prod_{j<k} alpha_j) (1 - alpha_k),  P(n = K) = prod alpha_j,
 *   P(n = k, bonus = v) = (prod_{j<k} alpha_j) r_k(v)   (k < K),
 *   P(n = K, bonus = v) = (prod_j alpha_j) p_K(v).
 * Per sampling sequence: accept_rate [K] = alpha, p_len [K+1] = P(n = k),
 * and for each position k <= K the F tokens of largest r_k (p_K at k = K)
 * by (mass desc, token asc), with those masses (token -1, mass 0 past the
 * positive ones).  Optionally draft_top_mass [K]: the residual mass r_k on
 * the 4 largest logits of draft row k (the tokens beta down-weights), so
 * that P(bonus among them | n = k) = draft_top_mass_k / (1 - alpha_k)
 * ("Key claims": Saguaro sampling concentrates the residual on the draft's
 * likeliest tokens, raising the speculation cache's hit rate).  Greedy sequences (whose outcome their drafts fix) and
 * failed ones get NaN, -1 and 0; a failed sequence reports the failures of
 * all its rows.                                                               */
static int or_outcome_sequence(const void *target, const void *draft, int32_t b, int32_t K,
                               int32_t V, int dtype, double T, double beta, int32_t F,
                               double *alpha, double *p_len, int32_t *top_tok, double *top_mass,
                               double *d4_mass)
{
    for (int32_t j = 0; j < K; ++j) alpha[j] = NAN;
    if (d4_mass)
        for (int32_t j = 0; j < K; ++j) d4_mass[j] = NAN;
    for (int32_t k = 0; k <= K; ++k) {
        p_len[k] = NAN;
        for (int32_t f = 0; f < F; ++f) {
            top_tok[(size_t)k * F + f] = -1;
            top_mass[(size_t)k * F + f] = 0.0;
        }
    }
    if (!(T >= 0.0) || isinf(T)) return OR_ERR_TEMPERATURE;
    if (T == 0.0) return 0;
    if (K > 0 && draft == NULL) return OR_ERR_NO_DRAFT;
    int weighted = beta < 1.0;
    double *r = (double *)malloc(sizeof(double) * (size_t)V);
    int err = 0; /* the failures of every row of the sequence, OR-ed */
    for (int32_t k = 0; k <= K; ++k) {
        or_row rt, rd;
        int e = or_prepare(&rt, or_row_ptr(target, dtype, (size_t)b * (K + 1) + k, V), dtype, V, T, 0, 1.0);
        if (k < K)
            e |= or_prepare(&rd, or_row_ptr(draft, dtype, (size_t)b * K + k, V), dtype, V, T, weighted,
                            beta);
        err |= e;
        if (err) continue;
        double amin = 0.0;
        for (int32_t v = 0; v < V; ++v) {
            double pt = exp(or_logprob(&rt, v));
            if (k < K) {
                double q = exp(or_logprob(&rd, v));
                amin += pt < q ? pt : q;
                r[v] = pt > q ? pt - q : 0.0;
            } else {
                r[v] = pt;
            }
        }
        if (k < K) alpha[k] = amin;
        if (k < K && d4_mass) { /* residual mass on the draft row's top-4 */
            int32_t t4[4];
            int32_t n4 = oracle_row_top4(or_row_ptr(draft, dtype, (size_t)b * K + k, V), dtype, V, t4);
            double m4 = 0.0;
            for (int32_t q = 0; q < n4; ++q) m4 += r[t4[q]];
            d4_mass[k] = m4;
        }
        /* the F largest masses, ties to the lower token: F passes over V */
        for (int32_t f = 0; f < F; ++f) {
            int32_t best = -1;
            for (int32_t v = 0; v < V; ++v) {
                if (!(r[v] > 0.0)) continue;
                int taken = 0;
                for (int32_t g = 0; g < f; ++g)
                    if (top_tok[(size_t)k * F + g] == v) taken = 1;
                if (taken) continue;
                if (best < 0 || r[v] > r[best]) best = v;
            }
            if (best < 0) break;
            top_tok[(size_t)k * F + f] = best;
            top_mass[(size_t)k * F + f] = r[best];
        }
    }
    free(r);
    if (err) {
        for (int32_t j = 0; j < K; ++j) alpha[j] = NAN;
        if (d4_mass)
            for (int32_t j = 0; j < K; ++j) d4_mass[j] = NAN;
        for (int32_t k = 0; k <= K; ++k)
            for (int32_t f = 0; f < F; ++f) {
                top_tok[(size_t)k * F + f] = -1;
                top_mass[(size_t)k * F + f] = 0.0;
            }
        return err;
    }
    double reach = 1.0; /* prod_{j<k} alpha_j */
    for (int32_t k = 0; k < K; ++k) {
        p_len[k] = reach * (1.0 - alpha[k]);
        reach *= alpha[k];
    }
    p_len[K] = reach;
    return 0;
}

int32_t oracle_spec_verify_outcomes(const void *target, const void *draft, int32_t B, int32_t K,
                                    int32_t V, int32_t dtype, const float *temperature, double beta,
                                    int32_t F, double *accept_rate, double *p_len, int32_t *top_tokens,
                                    double *top_mass, double *draft_top_mass, int32_t *seq_error,
                                    int32_t nthreads)
{
    int32_t all_err = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : all_err)
#endif
    for (int32_t b = 0; b < B; ++b) {
        int e = or_outcome_sequence(target, draft, b, K, V, dtype, (double)temperature[b], beta, F,
                                    accept_rate + (size_t)b * K, p_len + (size_t)b * (K + 1),
                                    top_tokens + (size_t)b * (K + 1) * F,
                                    top_mass + (size_t)b * (K + 1) * F,
                                    draft_top_mass ? draft_top_mass + (size_t)b * K : NULL);
        if (seq_error) seq_error[b] = e;
        all_err |= e;
    }
    return all_err;
}

/* ------------------------------------------------------------------ */
/* Tree (multi-draft) verification.  The pages name tree-based speculative
 * decoding ("Speculative Speculative Decoding", Key claims: SSD composes with
 * Medusa-style trees) but give no verify rule for it; this is the published
 * recursive rejection sampling over a token tree (Miao et al., "SpecInfer",
 * ASPLOS'24, multi-step speculative sampling), which keeps the output law
 * the target's when the children of a context are drawn i.i.d. from its
 * draft law.
 *  - Node i in [0, N) has parent[i] in [-1, i-1] (-1: the root) and token x_i.
 *    Context 0 is the root and context i + 1 is node i: target row c holds
 *    the target logits after context c (N + 1 rows), draft row c (c < N) the
 *    draft logits the children of context c were drawn from.
 *  - At the current context the law is r = p_t (its target row).  Its
 *    children are tried in ascending node index: child j with token x is
 *    accepted iff u(b, j, 0) <= r(x) / q(x); on a rejection
 *    r <- max(r - q, 0) / sum_v max(r - q, 0) (kept as it is if that sum is
 *    zero).  An accepted child becomes the current context.  When no child
 *    is left (none, or all rejected) the bonus is the smallest v with
 *    C(v) >= u(b, d, 1) C(V-1), C the running sum of r in token order, d the
 *    number of accepted nodes.
 *  - Greedy (T == 0): the first child whose token is the target argmax is
 *    accepted; the bonus is the final context's argmax.
 * The law after L rejections that left mass is computed in closed form:
 * with z_i the mass of the i-th residual, r_{i+1} = max(r_i - q, 0) / z_i
 * unrolls to r_L = max(p - q A, 0) / P, A = sum_{k<L} prod_{i<k} z_i,
 * P = prod_{i<L} z_i (A = 0, P = 1 for p itself; once p - q A_i <= 0 at a
 * token it stays so, as A only grows), and a rejection's residual is
 * max(p - q (A + P), 0) / P.  Each element is formed as
 * p(v) max(-expm1(s(v)), 0), s(v) = ln(q(v) A / p(v)) = (z_d(v) - z_t(v)) / T
 * + ln(S_t / S_d) + ln A with S the rows' sums relative to their maxima, so
 * that repeated rejections, whose residual masses multiply, keep the law's
 * shape: the iterated subtraction r - q leaves each element a rounding error
 * of ~1e-16 of p, which is the whole of r once P falls that low.
 * A chain (parent[i] = i - 1) is the verify step with K = N, uniforms
 * included.  Outputs: accepted_len[b] = d, out_tokens[b, 0..d-1] the accepted
 * tokens and out_tokens[b, d] the bonus (-1 after), path[b, 0..d-1] the
 * accepted nodes (-1 after); for parity checks node_margin[b, j] = |u - ratio|
 * of node j's accept test (NaN for nodes not tested) and bonus_margin[b] the
 * distance of u from the ends of the bonus token's CDF interval.  force[b, j]
 * (or NULL) reverses the outcome of node j's test, so that a near-tie another
 * implementation decided the other way can be replayed.  probe[b] (or NULL):
 * a token whose CDF interval [C(t-1), C(t)] / C(V-1) under the final law is
 * written to probe_cdf[b, 0..1] (parity checks of a bonus another
 * implementation drew).  Only the rows the walk visits are checked for
 * finite maxima.                                                             */
/* Max and sum of exp((z - max) / T) of a row. */
static double or_row_sum(const void *row, int dtype, int32_t V, double T, double *m_out)
{
    double m = -INFINITY;
    for (int32_t v = 0; v < V; ++v) {
        double a = or_logit(row, dtype, (size_t)v) / T;
        if (a > m) m = a;
    }
    double s = 0.0;
    for (int32_t v = 0; v < V; ++v) s += exp(or_logit(row, dtype, (size_t)v) / T - m);
    *m_out = m;
    return s;
}

/* Element v of max(p - q A, 0) (A > 0) as p(v) max(-expm1(s), 0), with
 * lnR = ln(S_t / S_d) + ln A. */
static double or_tree_resid(const or_row *rt, const void *dz, double lnR, int32_t v)
{
    const double pv = exp(or_logprob(rt, v));
    if (pv == 0.0) return 0.0;
    const double zt = or_logit(rt->z, rt->dtype, (size_t)v), zd = or_logit(dz, rt->dtype, (size_t)v);
    const double sv = (zd - zt) / rt->T + lnR; /* -inf where the draft gives v no mass */
    const double f = -expm1(sv);
    return f > 0.0 ? pv * f : 0.0;
}

static int or_tree_sequence(const void *target, const void *draft, const int32_t *parent,
                            const int32_t *tokens, int32_t N, int32_t V, int dtype, uint64_t seed,
                            uint32_t gb, double T, int32_t *acc, int32_t *out, int32_t *path,
                            double *node_margin, double *bonus_margin, const uint8_t *force,
                            int32_t probe, double *probe_cdf)
{
    *acc = 0;
    for (int32_t j = 0; j <= N; ++j) out[j] = -1;
    for (int32_t j = 0; j < N; ++j) path[j] = -1;
    for (int32_t j = 0; j < N; ++j) node_margin[j] = NAN;
    *bonus_margin = NAN;
    for (int32_t i = 0; i < N; ++i)
        if (parent[i] < -1 || parent[i] >= i) return OR_ERR_TREE;
    if (!(T >= 0.0) || isinf(T)) return OR_ERR_TEMPERATURE;
    int err = 0;
    int32_t cur = -1, d = 0;
    if (T == 0.0) {
        for (;;) {
            const void *row = or_row_ptr(target, dtype, (size_t)(cur + 1), V);
            if (!isfinite(oracle_row_max(row, dtype, V))) {
                for (int32_t j = 0; j <= N; ++j) out[j] = -1;
                for (int32_t j = 0; j < N; ++j) path[j] = -1;
                *acc = 0;
                return err | OR_ERR_ROW;
            }
            const int32_t a = oracle_row_argmax(row, dtype, V);
            int32_t next = -1;
            for (int32_t j = cur + 1; j < N && next < 0; ++j) {
                if (parent[j] != cur) continue;
                if (tokens[j] < 0 || tokens[j] >= V) err |= OR_ERR_TOKEN;
                if (tokens[j] == a) next = j;
            }
            if (next < 0) {
                out[d] = a;
                *acc = d;
                return err;
            }
            out[d] = a;
            path[d] = next;
            ++d;
            cur = next;
        }
    }
    if (N > 0 && draft == NULL) return OR_ERR_NO_DRAFT;
    or_row rt, rd;
    for (;;) {
        const void *trow = or_row_ptr(target, dtype, (size_t)(cur + 1), V);
        const void *drow = draft ? or_row_ptr(draft, dtype, (size_t)(cur + 1), V) : NULL;
        int e = or_prepare(&rt, trow, dtype, V, T, 0, 1.0);
        int have_child = 0;
        for (int32_t j = cur + 1; j < N; ++j) have_child |= parent[j] == cur;
        if (!e && have_child) e = or_prepare(&rd, drow, dtype, V, T, 0, 1.0);
        if (e) {
            for (int32_t j = 0; j <= N; ++j) out[j] = -1;
            for (int32_t j = 0; j < N; ++j) path[j] = -1;
            for (int32_t j = 0; j < N; ++j) node_margin[j] = NAN;
            *acc = 0;
            return err | e;
        }
        /* ln(S_t / S_d) from the rows' sums relative to their maxima */
        double lnST = 0.0;
        if (have_child) {
            double mt, md;
            const double st = or_row_sum(trow, dtype, V, T, &mt), sd = or_row_sum(drow, dtype, V, T, &md);
            lnST = (mt - md) + log(st / sd);
        }
        double A = 0.0, P = 1.0; /* the current law r = max(p - q A, 0) / P */
        int32_t next = -1;
        for (int32_t j = cur + 1; j < N && next < 0; ++j) {
            if (parent[j] != cur) continue;
            const int32_t x = tokens[j];
            double ratio;
            if (x < 0 || x >= V) {
                err |= OR_ERR_TOKEN;
                ratio = 0.0;
            } else {
                const double lq = or_logprob(&rd, x);
                /* r(x) / q(x) = max(p(x) / q(x) - A, 0) / P */
                const double pq = exp(or_logprob(&rt, x) - lq);
                ratio = (lq == -INFINITY) ? INFINITY : (A == 0.0 ? pq : fmax(pq - A, 0.0) / P);
            }
            const double u = oracle_uniform(seed, gb, (uint32_t)j, OR_ACCEPT);
            node_margin[j] = fabs(u - ratio);
            int accept = u <= ratio;
            if (force && force[j]) accept = !accept;
            if (accept) {
                next = j;
                break;
            }
            /* the law after this rejection: max(r - q, 0) = max(p - q (A + P), 0) / P */
            const double lnR = lnST + log(A + P);
            double sw = 0.0;
            for (int32_t v = 0; v < V; ++v) sw += or_tree_resid(&rt, drow, lnR, v);
            if (sw > 0.0) { /* else the law stays as it is */
                A = A + P;
                P = sw;
            }
        }
        if (next >= 0) {
            out[d] = tokens[next];
            path[d] = next;
            ++d;
            cur = next;
            continue;
        }
        /* bonus from the current law */
        double *w = (double *)malloc(sizeof(double) * (size_t)V);
        const double lnR = A > 0.0 ? lnST + log(A) : 0.0;
        double S = 0.0;
        for (int32_t v = 0; v < V; ++v) {
            w[v] = A > 0.0 ? or_tree_resid(&rt, drow, lnR, v) : exp(or_logprob(&rt, v));
            S += w[v];
        }
        const double uB = oracle_uniform(seed, gb, (uint32_t)d, OR_BONUS);
        const double thr = uB * S;
        double C = 0.0, Cprev = 0.0;
        int32_t bonus = -1;
        for (int32_t v = 0; v < V; ++v) {
            Cprev = C;
            C += w[v];
            if (C >= thr) {
                bonus = v;
                break;
            }
        }
        if (bonus < 0) {
            for (int32_t v = V - 1; v >= 0; --v)
                if (w[v] > 0.0) {
                    bonus = v;
                    break;
                }
            C = S;
        }
        const double m1 = fabs(uB - Cprev / S), m2 = fabs(uB - C / S);
        if (probe_cdf) {
            probe_cdf[0] = probe_cdf[1] = NAN;
            if (probe >= 0 && probe < V) {
                double cp = 0.0;
                for (int32_t v = 0; v < probe; ++v) cp += w[v];
                probe_cdf[0] = cp / S;
                probe_cdf[1] = (cp + w[probe]) / S;
            }
        }
        free(w);
        out[d] = bonus;
        *acc = d;
        *bonus_margin = m1 < m2 ? m1 : m2;
        return err;
    }
}

int32_t oracle_spec_verify_tree(const void *target, const void *draft, const int32_t *parent,
                                const int32_t *tokens, int32_t B, int32_t N, int32_t V, int32_t dtype,
                                uint64_t seed, const float *temperature, int32_t *accepted_len,
                                int32_t *out_tokens, int32_t *path, double *node_margin,
                                double *bonus_margin, int32_t *seq_error, const int32_t *seq_ids,
                                const uint8_t *force, const int32_t *probe, double *probe_cdf,
                                int32_t nthreads)
{
    int32_t all_err = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : all_err)
#endif
    for (int32_t b = 0; b < B; ++b) {
        const size_t tr = (size_t)b * (N + 1), dr = (size_t)b * N;
        int e = or_tree_sequence(or_row_ptr(target, dtype, tr, V),
                                 draft ? or_row_ptr(draft, dtype, dr, V) : NULL,
                                 parent + (size_t)b * N, tokens + (size_t)b * N, N, V, dtype, seed,
                                 seq_ids ? (uint32_t)seq_ids[b] : (uint32_t)b,
                                 (double)temperature[b], accepted_len + b, out_tokens + (size_t)b * (N + 1),
                                 path + (size_t)b * N, node_margin + (size_t)b * N, bonus_margin + b,
                                 force ? force + (size_t)b * N : NULL, probe ? probe[b] : -1,
                                 probe_cdf ? probe_cdf + (size_t)b * 2 : NULL);
        if (seq_error) seq_error[b] = e;
        all_err |= e;
    }
    return all_err;
}

/* The batch with every sequence drafting K tokens. */
int32_t oracle_spec_verify(const void *target, const void *draft, const int32_t *tokens,
                           int32_t B, int32_t K, int32_t V, int32_t dtype, uint64_t seed,
                           const float *temperature, double beta, int32_t *accepted_len,
                           int32_t *out_tokens, double *p_target, double *p_draft,
                           double *residual_mass, double *margin_accept, double *margin_bonus,
                           int32_t *seq_error, const int32_t *seq_ids, int32_t nthreads)
{
    return oracle_spec_verify_ragged(target, draft, tokens, NULL, B, K, V, dtype, seed, temperature,
                                     beta, accepted_len, out_tokens, p_target, p_draft,
                                     residual_mass, margin_accept, margin_bonus, seq_error, NULL,
                                     seq_ids, NULL, nthreads);
}

/* Full draft log-law ln p_d'(v) of one row (for invariant checks). */
int32_t oracle_draft_logprobs(const void *row, int32_t dtype, int32_t V, double T, double beta,
                              double *out)
{
    or_row r;
    int e = or_prepare(&r, row, dtype, V, T, beta < 1.0, beta);
    if (e) return e;
    for (int32_t v = 0; v < V; ++v) out[v] = or_logprob(&r, v);
    return 0;
}

/* u(seed, b, pos, purpose) for b < B, pos < P, purpose in {0, 1}, laid out
 * [B, P, 2]. */
void oracle_uniforms(uint64_t seed, int32_t B, int32_t P, double *out)
{
    for (int32_t b = 0; b < B; ++b)
        for (int32_t pos = 0; pos < P; ++pos)
            for (uint32_t purpose = 0; purpose < 2; ++purpose)
                out[((size_t)b * P + pos) * 2 + purpose] =
                    oracle_uniform(seed, (uint32_t)b, (uint32_t)pos, purpose);
}

/* Number of threads an OpenMP parallel region would use by default. */
int32_t oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
