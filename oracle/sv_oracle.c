/*
 * CPU ORACLE for batched draft verification -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The product path (the HIP library) never calls it and
 * shares no code, header, table or helper with it.
 *
 * It is the plain definition of one verification step, in fp64, one sequence
 * at a time, in the order the pages describe it:
 *
 *  - The draft proposes a block; the target scores the whole block in one pass;
 *    the prefix the target agrees with is kept, plus one token the target
 *    generates itself; the rest is discarded.
 *      (umans.ai blog "DeepSeek V4 Pro DSpark: the model isn't ready, the
 *       architecture is", section "Speculative decoding, briefly";
 *       zhichai.net article, section "Why LLMs speak so slowly": generation
 *       restarts from the first error.)
 *  - The acceptance rule is rejection sampling on the ratio of target to draft
 *    probability, built so that the emitted tokens follow the target's
 *    distribution exactly; a rejected token is replaced by one the target
 *    would have produced.
 *      (umans.ai blog, "Speculative decoding, briefly"; zhichai.net, "Why LLMs
 *       speak so slowly".)  The construction that meets this statement is the
 *    standard one: accept x with probability min(1, p(x)/q(x)); on rejection
 *    draw the replacement from max(0, p - q) normalised.
 *  - A confidence per draft position is the probability that the token
 *    survives given that everything before it survived; multiplying along the
 *    block gives the survival of each prefix; the verify length follows from
 *    these survivals and the load.
 *      (umans.ai blog, section "2. Verify smarter: a throttle that costs the
 *       user nothing"; zhichai.net, section "Under the hood".)  The rule used
 *    here: S_0 = 1, S_j = S_{j-1} c_j, L = max({0} U {j : S_j >= tau}).
 *
 * Readings where the pages are silent (the GPU path takes the same ones):
 *  - K+1 target rows per sequence; row K+1 is the distribution of the bonus
 *    token after the whole block.
 *  - One temperature T for target and draft: p = softmax(l_t / T),
 *    q = softmax(l_d / T).  T == 0 means greedy: target token = argmax of the
 *    raw target row (lowest index on ties), accept while the draft equals it.
 *  - Uniforms u[b][0..K-1] serve the accept tests of positions 1..K; u[b][K]
 *    serves the final draw (replacement or bonus).  Accept iff u < p/q.
 *  - Inverse CDF in ascending token id: y = min{v : C_v > w}, C the running
 *    sum.  If rounding leaves w >= C_{V-1}, y = the largest v with mass > 0.
 *    If the residual mass Z is not positive, the replacement is drawn from p.
 *  - c_j = max_v q_j(v) when no confidence is given.
 *  - A drafted id outside [0, V) at a position that is tested, or a given
 *    verify length outside [0, K], marks the sequence bad: accepted length 0,
 *    no token (-1).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { SVO_F32 = 0, SVO_BF16 = 1 };
enum { SVO_LEN_FIXED = 0, SVO_LEN_TAU = 1 };
enum { SVO_FINAL_RESIDUAL = 0, SVO_FINAL_BONUS = 1, SVO_FINAL_GREEDY = 2, SVO_FINAL_BAD_INPUT = 3 };
enum { SVO_MARGIN_ACCEPT = 1, SVO_MARGIN_CDF = 2, SVO_MARGIN_SURVIVAL = 4 };
/* Draft distribution.  PROBS: q_j = softmax(draft logits / T).  ONEHOT: the
 * drafter picked its tokens greedily, so q_j is the point mass at x_j (the
 * `draft_sample_method: greedy` option of vLLM's DSpark support in the
 * techvisionai blog, Chapter 7); no draft logits are read, the derived
 * confidence max_v q_j(v) is 1, and lse of the draft rows is not reported. */
enum { SVO_DRAFT_PROBS = 0, SVO_DRAFT_ONEHOT = 1 };

/* Margin of the bit-exact comparison: |u - p/q| at a tested position, and the
 * final draw's CDF gap (distance of w to the nearest step of the running sum)
 * relative to the draw's total mass Z (1 for a bonus draw). */
#define SVO_MARGIN 1e-6

typedef struct {
    int32_t B, K, V;
    int32_t dtype;
    const void* target;              /* [B][K+1][V] via the strides below (elements) */
    int64_t target_batch_stride, target_row_stride;
    const void* draft;               /* [B][K][V]; NULL allowed when T == 0 */
    int64_t draft_batch_stride, draft_row_stride;
    const int32_t* tokens;           /* [B][K] */
    const float* uniforms;           /* [B][K+1] */
    float temperature;
    int32_t length_mode;
    const int32_t* verify_len_in;    /* fixed mode: [B] or NULL (=> K) */
    const float* confidence;         /* tau mode: [B][K] or NULL (=> max draft prob) */
    const float* tau;                /* tau mode: [B] */
    const int32_t* seq_index;        /* sequences to evaluate, or NULL => 0..n_seq-1 */
    int32_t n_seq;
    int32_t all_rows;                /* 1: report lse of every row, not only the rows the step reads */
    int32_t n_threads;               /* <= 0: library default */
    int32_t draft_mode;              /* SVO_DRAFT_PROBS, or SVO_DRAFT_ONEHOT: q_j is the point mass at x_j */
} svo_problem;

typedef struct {                     /* indexed by i in 0..n_seq-1 */
    int32_t* accepted_len;           /* [n] */
    int32_t* out_tokens;             /* [n][K+1], -1 padded */
    int32_t* verify_len;             /* [n] */
    double* lse_target;              /* [n][K+1], NaN where not evaluated */
    double* lse_draft;               /* [n][K],   NaN where not evaluated */
    double* survival;                /* [n][K],   NaN where not evaluated */
    double* residual_mass;           /* [n] Z of the replacement draw, 1 for a bonus draw */
    double* sampled_prob;            /* [n] probability of the final token under its draw */
    int32_t* final_kind;             /* [n] SVO_FINAL_* */
    int32_t* margin;                 /* [n] SVO_MARGIN_* bits */
    double* accept_gap;              /* [n] min |u_j - ratio_j| over tested positions (inf if none) */
    double* cdf_gap;                 /* [n] normalised distance of w to the nearest CDF step (inf if greedy) */
    int32_t* alt_token;              /* [n] the token across the nearest CDF step, -1 if none */
} svo_result;

/* Element v of a row as fp64 (bf16 is the upper half of an fp32 pattern). */
static inline double load_logit(const void* base, int dtype, int64_t idx)
{
    if (dtype == SVO_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
        float f;
        memcpy(&f, &bits, 4);
        return (double)f;
    }
    return (double)((const float*)base)[idx];
}

/* softmax of z = l / T over one row, kept as (m, s): m = max z,
 * s = sum exp(z - m), so that softmax(z)_v = exp(z_v - m) / s and
 * lse = m + ln s.  Probabilities are formed against m, never against lse:
 * z_v - lse in fp64 loses ln s once |z| is large (1e30 and ln 20000 round to
 * the same double), while z_v - m is exact there. */
typedef struct { double m, s; } svo_softmax;

static svo_softmax row_softmax(const void* base, int dtype, int64_t off, int32_t V, double T)
{
    svo_softmax r = {-INFINITY, 0.0};
    for (int32_t v = 0; v < V; ++v) {
        double z = load_logit(base, dtype, off + v) / T;
        if (z > r.m) r.m = z;
    }
    for (int32_t v = 0; v < V; ++v) r.s += exp(load_logit(base, dtype, off + v) / T - r.m);
    return r;
}

static inline double softmax_at(svo_softmax r, const void* base, int dtype, int64_t idx, double T)
{
    return exp(load_logit(base, dtype, idx) / T - r.m) / r.s;
}

/* Argmax of the raw row, lowest index on ties. */
static int32_t row_argmax(const void* base, int dtype, int64_t off, int32_t V)
{
    int32_t best = 0;
    double bv = load_logit(base, dtype, off);
    for (int32_t v = 1; v < V; ++v) {
        double x = load_logit(base, dtype, off + v);
        if (x > bv) { bv = x; best = v; }
    }
    return best;
}

/* Inverse-CDF draw over masses r[0..V-1] in ascending id: y = min{v : C_v > w}
 * with C the running sum.  If no step passes w (rounding), y = the largest v
 * with r_v > 0.  *gap = distance of w to the nearest of C_{y-1}, C_y divided by
 * norm; *alt = the token across that step (-1 if none). */
static int32_t inverse_cdf(const double* r, int32_t V, double w, double norm, double* gap, int32_t* alt)
{
    double C = 0.0, C_prev = 0.0;
    int32_t y = -1, prev_pos = -1;
    for (int32_t v = 0; v < V; ++v) {
        C_prev = C;
        C += r[v];
        if (C > w) { y = v; break; }
        if (r[v] > 0.0) prev_pos = v;
    }
    if (y < 0) {
        for (int32_t v = V - 1; v >= 0; --v)
            if (r[v] > 0.0) { y = v; break; }
        *gap = 0.0;
        *alt = -1;
        return y;
    }
    const double below = fabs(w - C_prev), above = fabs(C - w);
    if (below <= above) {
        *gap = below / norm;
        *alt = prev_pos;
    } else {
        *gap = above / norm;
        *alt = -1;
        for (int32_t v = y + 1; v < V; ++v)
            if (r[v] > 0.0) { *alt = v; break; }
    }
    return y;
}

static void verify_one(const svo_problem* P, int32_t b, int32_t i, const svo_result* R, double* r)
{
    const int32_t K = P->K, V = P->V;
    const double T = (double)P->temperature;
    const int greedy = !(T > 0.0);
    const int onehot = P->draft_mode == SVO_DRAFT_ONEHOT;
    const int64_t tb = (int64_t)b * P->target_batch_stride;
    const int64_t db = (int64_t)b * P->draft_batch_stride;
    const int32_t* x = P->tokens + (int64_t)b * K;
    const float* u = P->uniforms ? P->uniforms + (int64_t)b * (K + 1) : NULL;
    int32_t* out = R->out_tokens + (int64_t)i * (K + 1);
    double* lse_t = R->lse_target + (int64_t)i * (K + 1);
    double* lse_d = R->lse_draft + (int64_t)i * K;
    double* surv = R->survival + (int64_t)i * K;

    for (int32_t j = 0; j <= K; ++j) { out[j] = -1; lse_t[j] = NAN; }
    for (int32_t j = 0; j < K; ++j) { lse_d[j] = NAN; surv[j] = NAN; }
    /* softmax of every row the step reads, computed once (lse_* NaN = not yet) */
    svo_softmax sm_t[K + 1], sm_d[K > 0 ? K : 1];
#define NEED_T(j) do { if (isnan(lse_t[(j) - 1])) { \
        sm_t[(j) - 1] = row_softmax(P->target, P->dtype, tb + (int64_t)((j) - 1) * P->target_row_stride, V, T); \
        lse_t[(j) - 1] = sm_t[(j) - 1].m + log(sm_t[(j) - 1].s); } } while (0)
#define NEED_D(j) do { if (isnan(lse_d[(j) - 1])) { \
        sm_d[(j) - 1] = row_softmax(P->draft, P->dtype, db + (int64_t)((j) - 1) * P->draft_row_stride, V, T); \
        lse_d[(j) - 1] = sm_d[(j) - 1].m + log(sm_d[(j) - 1].s); } } while (0)
    int32_t margin = 0;
    double accept_gap = INFINITY, cdf_gap = INFINITY;
    int32_t alt = -1;

    /* ---- verify length ---- */
    int32_t L;
    if (P->length_mode == SVO_LEN_FIXED) {
        L = P->verify_len_in ? P->verify_len_in[b] : K;
        if (L < 0 || L > K) {
            /* outside the block: the sequence is marked bad, nothing is emitted */
            R->accepted_len[i] = 0;
            R->verify_len[i] = L;
            R->residual_mass[i] = NAN;
            R->sampled_prob[i] = NAN;
            R->final_kind[i] = SVO_FINAL_BAD_INPUT;
            R->margin[i] = 0;
            R->accept_gap[i] = INFINITY;
            R->cdf_gap[i] = INFINITY;
            R->alt_token[i] = -1;
            return;
        }
    } else {
        const double tau = (double)P->tau[b];
        double S = 1.0;
        L = 0;
        for (int32_t j = 1; j <= K; ++j) {
            double c;
            if (P->confidence) {
                c = (double)P->confidence[(int64_t)b * K + (j - 1)];
            } else if (P->draft_mode == SVO_DRAFT_ONEHOT) {
                c = 1.0; /* max of a point mass */
            } else {
                NEED_D(j);
                c = 1.0 / sm_d[j - 1].s; /* max_v q_j(v) = exp(m - m) / s */
            }
            S *= c;
            surv[j - 1] = S;
            if (S >= tau) L = j;
        }
        /* margin on the survivals the step has to look at */
        for (int32_t j = 1; j <= K && j <= L + 1; ++j) {
            double scale = tau > 1e-30 ? tau : 1e-30;
            if (fabs(surv[j - 1] - tau) < SVO_MARGIN * scale) margin |= SVO_MARGIN_SURVIVAL;
        }
    }

    int32_t a = 0, y = -1, kind;
    double Z = 1.0, py = NAN;

    if (greedy) {
        /* ---- greedy: accept while the drafted id equals the target argmax ---- */
        kind = SVO_FINAL_GREEDY;
        int bad = 0;
        for (int32_t j = 1; j <= L; ++j) {
            if (x[j - 1] < 0 || x[j - 1] >= V) { bad = 1; break; }
            const int32_t g = row_argmax(P->target, P->dtype, tb + (int64_t)(j - 1) * P->target_row_stride, V);
            if (x[j - 1] != g) break;
            a = j;
        }
        if (bad) {
            kind = SVO_FINAL_BAD_INPUT; a = 0; y = -1;
        } else {
            y = row_argmax(P->target, P->dtype, tb + (int64_t)a * P->target_row_stride, V);
        }
    } else {
        /* ---- rejection sampling along the block, stop at the first rejection ---- */
        int bad = 0, rejected = 0;
        for (int32_t j = 1; j <= L; ++j) {
            const int64_t toff = tb + (int64_t)(j - 1) * P->target_row_stride;
            const int64_t doff = db + (int64_t)(j - 1) * P->draft_row_stride;
            NEED_T(j);
            if (!onehot) NEED_D(j);
            const int32_t xj = x[j - 1];
            if (xj < 0 || xj >= V) { bad = 1; break; }
            const double p = softmax_at(sm_t[j - 1], P->target, P->dtype, toff + xj, T);
            const double q = onehot ? 1.0 : softmax_at(sm_d[j - 1], P->draft, P->dtype, doff + xj, T);
            const double ratio = q > 0.0 ? p / q : INFINITY;
            const double uj = (double)u[j - 1];
            const double gap = fabs(uj - ratio);
            if (gap < accept_gap) accept_gap = gap;
            if (gap < SVO_MARGIN) margin |= SVO_MARGIN_ACCEPT;
            if (uj < ratio) {
                a = j;
            } else {
                rejected = 1;
                break;
            }
        }
        if (bad) {
            kind = SVO_FINAL_BAD_INPUT; a = 0; y = -1; Z = 1.0;
        } else {
            const int32_t js = a + 1; /* the row of the final draw (1-based) */
            const int64_t toff = tb + (int64_t)(js - 1) * P->target_row_stride;
            NEED_T(js);
            const double uf = (double)u[K];
            int use_p = !rejected;
            if (rejected) {
                /* replacement from max(0, p - q), normalised: w = u * Z */
                const int64_t doff = db + (int64_t)(js - 1) * P->draft_row_stride;
                double Zr = 0.0;
                for (int32_t v = 0; v < V; ++v) {
                    const double p = softmax_at(sm_t[js - 1], P->target, P->dtype, toff + v, T);
                    const double q = onehot ? (v == x[js - 1] ? 1.0 : 0.0)
                                            : softmax_at(sm_d[js - 1], P->draft, P->dtype, doff + v, T);
                    r[v] = p > q ? p - q : 0.0;
                    Zr += r[v];
                }
                kind = SVO_FINAL_RESIDUAL;
                if (Zr > 0.0) {
                    y = inverse_cdf(r, V, uf * Zr, Zr, &cdf_gap, &alt);
                    Z = Zr;
                    py = r[y] / Zr;
                } else {
                    use_p = 1; /* cannot happen in exact arithmetic after a rejection */
                    Z = 0.0;
                }
            } else {
                kind = SVO_FINAL_BONUS;
                Z = 1.0;
            }
            if (use_p) {
                /* bonus (or the degenerate replacement): draw from p of that row, w = u */
                for (int32_t v = 0; v < V; ++v)
                    r[v] = softmax_at(sm_t[js - 1], P->target, P->dtype, toff + v, T);
                y = inverse_cdf(r, V, uf, 1.0, &cdf_gap, &alt);
                py = r[y];
            }
            if (cdf_gap < SVO_MARGIN) margin |= SVO_MARGIN_CDF;
        }
    }

    if (P->all_rows && !greedy) {
        for (int32_t j = 1; j <= K + 1; ++j) NEED_T(j);
        if (P->draft && !onehot)
            for (int32_t j = 1; j <= K; ++j) NEED_D(j);
    }

    /* ---- emit: accepted prefix, then the final token ---- */
    if (y >= 0) {
        for (int32_t j = 0; j < a; ++j) out[j] = x[j];
        out[a] = y;
    }
    R->accepted_len[i] = a;
    R->verify_len[i] = L;
    R->residual_mass[i] = greedy ? NAN : Z;
    R->sampled_prob[i] = py;
    R->final_kind[i] = kind;
    R->margin[i] = margin;
    R->accept_gap[i] = accept_gap;
    R->cdf_gap[i] = cdf_gap;
    R->alt_token[i] = alt;
#undef NEED_T
#undef NEED_D
}

/* Returns 0, or -1 for arguments the definition does not cover. */
int svo_verify(const svo_problem* P, const svo_result* R)
{
    if (!P || !R || P->B < 0 || P->K < 1 || P->V < 1 || P->n_seq < 0) return -1;
    const int greedy = !(P->temperature > 0.0f);
    if (P->draft_mode != SVO_DRAFT_PROBS && P->draft_mode != SVO_DRAFT_ONEHOT) return -1;
    if (!greedy && ((!P->draft && P->draft_mode == SVO_DRAFT_PROBS) || !P->uniforms)) return -1;
    if (P->length_mode == SVO_LEN_TAU && !P->tau) return -1;
    if (P->length_mode == SVO_LEN_TAU && greedy && !P->confidence) return -1;
    if (P->temperature < 0.0f || isnan(P->temperature)) return -1;
#ifdef _OPENMP
    if (P->n_threads > 0) omp_set_num_threads(P->n_threads);
#endif
    int err = 0;
    #pragma omp parallel reduction(| : err)
    {
        double* r = (double*)malloc(sizeof(double) * (size_t)P->V);
        if (!r) err = 1;
        #pragma omp for schedule(dynamic, 4)
        for (int32_t i = 0; i < P->n_seq; ++i) {
            if (!r) continue;
            const int32_t b = P->seq_index ? P->seq_index[i] : i;
            verify_one(P, b, i, R, r);
        }
        free(r);
    }
    return err ? -1 : 0;
}

int svo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ======================================================================
 * Load-aware admission: how many drafted positions each sequence verifies.
 *
 * umans.ai blog, section "2. Verify smarter: a throttle that costs the user
 * nothing": the engine's step rate is profiled against batch size once; each
 * step the expected system throughput is the expected number of accepted
 * tokens times the step rate at that batch size; every candidate token of
 * every request is ranked by its survival probability and admitted one at a
 * time until that product stops rising.  zhichai.net article, section "Under
 * the hood": each request's verified prefix is chosen to maximise accepted
 * tokens times verification speed.
 *
 * Readings where the pages leave the scheduler open:
 *  - a candidate is drafted position j of sequence b, with survival
 *    S_bj = prod_{i<=j} c_bi (fp64, left to right);
 *  - confidences outside [0, 1] (NaN included) are clamped into it (NaN -> 0)
 *    and reported as bad input;
 *  - the verify batch of m admitted candidates holds B + m tokens (every
 *    sequence also scores its own next position); the expected number of
 *    emitted tokens is B + the sum of the admitted survivals;
 *  - ranking: S descending, then b ascending, then j ascending (with c in
 *    [0, 1], S does not increase along a sequence, so every sequence's
 *    admitted positions are a prefix 1..L_b);
 *  - T(m) = (B + sum of the m best survivals) * speed[B + m]; admission stops
 *    at the first m with T(m + 1) <= T(m) ("stops rising"), m = N if never.
 * ====================================================================== */

typedef struct {
    int32_t B, K;
    const float* confidence;  /* [B][K] */
    const double* speed;      /* [n_speed] steps per second at a batch of n tokens */
    int32_t n_speed;          /* >= B (K + 1) + 1 */
} svo_sched_problem;

typedef struct {
    int32_t* verify_len;      /* [B] */
    double* survival;         /* [B][K] */
    int32_t* admitted;        /* [1] m */
    double* tau;              /* [1] smallest admitted survival, NaN if none */
    double* expected;         /* [1] T(m) */
    int32_t* margin;          /* [1] 1 if a stop decision at or before m was within 1e-9 (relative) */
    int32_t* bad;             /* [1] 1 if a confidence was outside [0, 1] */
} svo_sched_result;

typedef struct { double s; int32_t b, j; } svo_cand;

static int svo_cand_cmp(const void* x, const void* y)
{
    const svo_cand* a = (const svo_cand*)x;
    const svo_cand* c = (const svo_cand*)y;
    if (a->s > c->s) return -1;
    if (a->s < c->s) return 1;
    if (a->b != c->b) return a->b < c->b ? -1 : 1;
    return a->j < c->j ? -1 : (a->j > c->j);
}

int svo_schedule(const svo_sched_problem* P, const svo_sched_result* R)
{
    const int32_t B = P->B, K = P->K;
    const int64_t N = (int64_t)B * K;
    if (B < 0 || K < 1 || P->n_speed < (int64_t)B * (K + 1) + 1) return -1;
    int bad = 0;
    svo_cand* cand = (svo_cand*)malloc(sizeof(svo_cand) * (size_t)(N > 0 ? N : 1));
    if (!cand) return -2;
    /* survivals */
    for (int32_t b = 0; b < B; ++b) {
        double S = 1.0;
        for (int32_t j = 0; j < K; ++j) {
            double c = (double)P->confidence[(int64_t)b * K + j];
            if (!(c >= 0.0 && c <= 1.0)) {
                bad = 1;
                c = c > 1.0 ? 1.0 : 0.0; /* NaN and negatives -> 0 */
            }
            S *= c;
            R->survival[(int64_t)b * K + j] = S;
            cand[(int64_t)b * K + j].s = S;
            cand[(int64_t)b * K + j].b = b;
            cand[(int64_t)b * K + j].j = j;
        }
    }
    /* rank every candidate by survival */
    qsort(cand, (size_t)N, sizeof(svo_cand), svo_cand_cmp);
    /* admit one at a time while the expected throughput rises */
    double P_m = 0.0;                     /* sum of the m best survivals */
    int64_t m = 0;
    int margin = 0;
    for (;;) {
        const double T_m = ((double)B + P_m) * P->speed[B + m];
        if (m == N) break;
        const double T_next = ((double)B + P_m + cand[m].s) * P->speed[B + m + 1];
        const double scale = fmax(fabs(T_m), fabs(T_next));
        if (fabs(T_next - T_m) <= 1e-9 * scale) margin = 1;
        if (T_next <= T_m) break;         /* the product stops rising */
        P_m += cand[m].s;
        ++m;
    }
    for (int32_t b = 0; b < B; ++b) R->verify_len[b] = 0;
    for (int64_t i = 0; i < m; ++i) R->verify_len[cand[i].b]++;
    *R->admitted = (int32_t)m;
    *R->tau = m > 0 ? cand[m - 1].s : NAN;
    *R->expected = ((double)B + P_m) * P->speed[B + m];
    *R->margin = margin;
    *R->bad = bad;
    free(cand);
    return 0;
}
