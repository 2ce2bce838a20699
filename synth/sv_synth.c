/*
 * Seeded synthetic inputs for batched draft verification.
 *
 * This module only makes inputs: target and draft logit rows, drafted tokens,
 * the uniforms the verifier consumes, and per-sequence thresholds.  It holds
 * none of the verifier's arithmetic (no log-sum-exp, no acceptance ratio, no
 * residual distribution).  Drafted tokens are drawn with the Gumbel-max trick,
 * which samples from softmax(d/T) without normalising the row.
 *
 * Random numbers: Philox4x32-10, the counter-based generator of
 *   J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
 *   "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11, section 3.
 * Ten rounds; each round multiplies counter words 0 and 2 by the two Philox
 * multipliers, and the key is advanced by the two Weyl increments between
 * rounds.
 *
 * Streams.  Every random word is addressed by a counter (c0, row, stream, 0)
 * under a key (seed, 0), so any row can be regenerated on its own.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

enum {
    STREAM_TARGET = 1, /* target-row normals */
    STREAM_DRAFT = 2,  /* draft-noise normals */
    STREAM_PERM = 3,   /* per-row rank permutation */
    STREAM_PLANT = 4,  /* planted-maximum position */
    STREAM_GUMBEL = 5, /* Gumbel noise for drawing a drafted token */
    STREAM_COIN = 6,   /* match / random-token coin for greedy drafts */
    STREAM_TAU = 7     /* per-sequence threshold choice */
};

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline void philox_block(uint32_t c0, uint32_t row, uint32_t stream, uint32_t seed, uint32_t w[4])
{
    uint32_t ctr[4] = {c0, row, stream, 0u};
    uint32_t key[2] = {seed, 0u};
    synth_philox4x32_10(ctr, key, w);
}

/* Open-interval uniform from one 32-bit word: (w + 1/2) * 2^-32. */
static inline double u32_open(uint32_t w) { return ((double)w + 0.5) * 2.3283064365386963e-10; }

/* Four standard normals from one Philox block (two Box-Muller pairs, fp64). */
static inline void normals4(uint32_t c0, uint32_t row, uint32_t stream, uint32_t seed, double z[4])
{
    uint32_t w[4];
    philox_block(c0, row, stream, seed, w);
    const double two_pi = 6.283185307179586476925286766559;
    for (int p = 0; p < 2; ++p) {
        double u1 = u32_open(w[2 * p]);
        double u2 = u32_open(w[2 * p + 1]);
        double r = sqrt(-2.0 * log(u1));
        z[2 * p] = r * cos(two_pi * u2);
        z[2 * p + 1] = r * sin(two_pi * u2);
    }
}

/* fp64 -> fp32 (round to nearest even, by the C conversion) -> bf16 (round to
 * nearest even on the upper 16 bits).  Inputs are finite or -inf. */
static inline uint16_t f32_to_bf16_rne(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, 4);
    if ((bits & 0x7F800000u) == 0x7F800000u) return (uint16_t)(bits >> 16); /* inf */
    uint32_t bias = 0x7FFFu + ((bits >> 16) & 1u);
    return (uint16_t)((bits + bias) >> 16);
}

static inline double bf16_to_double(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* Round a fp64 value to the storage dtype and return the stored value as fp64. */
static inline double store_value(void* base, int64_t idx, int dtype, double x)
{
    float f = (float)x;
    if (dtype == 1) {
        uint16_t h = f32_to_bf16_rne(f);
        ((uint16_t*)base)[idx] = h;
        return bf16_to_double(h);
    }
    ((float*)base)[idx] = f;
    return (double)f;
}

/* Uniforms for the verifier: u_i = (2k+1) * 2^-24 with k = w_i >> 9, where w_i
 * is word (i mod 4) of Philox((i div 4, 0, 0, 0), (seed, 0)).  Exact in fp32
 * and strictly inside (0, 1). */
void synth_uniforms(uint32_t seed, int64_t n, float* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < (n + 3) / 4; ++blk) {
        uint32_t ctr[4] = {(uint32_t)blk, 0u, 0u, 0u};
        uint32_t key[2] = {seed, 0u};
        uint32_t w[4];
        synth_philox4x32_10(ctr, key, w);
        for (int q = 0; q < 4; ++q) {
            int64_t i = blk * 4 + q;
            if (i < n) out[i] = (float)((2.0 * (double)(w[q] >> 9) + 1.0) * 5.9604644775390625e-08);
        }
    }
}

/* A problem recipe.  Rows are laid out [B][K+1][V] (target) and [B][K][V]
 * (draft), V contiguous, in fp32 (dtype 0) or bf16 (dtype 1). */
typedef struct {
    int32_t B, K, V, dtype;
    int32_t target_kind;     /* 0: scale * N(0,1); 1: -zipf_s * ln(rank) + jitter * N(0,1) */
    double target_scale;
    double zipf_s, zipf_jitter;
    int32_t plant;           /* 1: overwrite one seeded position per target row with plant_value */
    double plant_value;
    int32_t make_draft;      /* 1: draft row j = target row j (fp64) + sigma_j * N(0,1) */
    double sigma_first, sigma_last; /* sigma_j linear in j from first to last position */
    int32_t token_mode;      /* 0: x_j ~ softmax(d_j / T) (Gumbel-max); 1: planted max w.p. p_match else uniform id;
                                2: the draft row's largest value (a greedy drafter) */
    double temperature, p_match;
    uint32_t seed_target, seed_draft, seed_tokens, seed_aux;
} synth_spec;

/* Planted position of target row r (Lemire's multiply-shift onto [0, V)). */
static inline int32_t planted_index(const synth_spec* s, uint32_t row)
{
    uint32_t w[4];
    philox_block(0u, row, STREAM_PLANT, s->seed_aux, w);
    return (int32_t)(((uint64_t)w[0] * (uint64_t)s->V) >> 32);
}

/* One target row in fp64, before rounding.  perm is scratch of V int32. */
static void target_row_f64(const synth_spec* s, uint32_t row, double* out, int32_t* perm)
{
    const int32_t V = s->V;
    for (int32_t v = 0; v < V; v += 4) {
        double z[4];
        normals4((uint32_t)(v >> 2), row, STREAM_TARGET, s->seed_target, z);
        for (int q = 0; q < 4 && v + q < V; ++q) out[v + q] = z[q];
    }
    if (s->target_kind == 0) {
        for (int32_t v = 0; v < V; ++v) out[v] *= s->target_scale;
    } else {
        /* ranks 1..V in a seeded Fisher-Yates order */
        for (int32_t v = 0; v < V; ++v) perm[v] = v + 1;
        for (int32_t i = V - 1; i >= 1; --i) {
            uint32_t w[4];
            philox_block((uint32_t)i, row, STREAM_PERM, s->seed_aux, w);
            int32_t j = (int32_t)(((uint64_t)w[0] * (uint64_t)(i + 1)) >> 32);
            int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
        }
        for (int32_t v = 0; v < V; ++v)
            out[v] = -s->zipf_s * log((double)perm[v]) + s->zipf_jitter * out[v];
    }
    if (s->plant) out[planted_index(s, row)] = s->plant_value;
}

/* Gumbel-max draw from softmax(stored / T): argmax_v stored_v / T + G_v with
 * G_v = -ln(-ln U_v).  Lowest index wins an exact tie. */
static int32_t gumbel_max_token(const synth_spec* s, uint32_t row, const double* stored)
{
    const int32_t V = s->V;
    int32_t best = 0;
    double best_key = -INFINITY;
    for (int32_t v = 0; v < V; v += 4) {
        uint32_t w[4];
        philox_block((uint32_t)(v >> 2), row, STREAM_GUMBEL, s->seed_tokens, w);
        for (int q = 0; q < 4 && v + q < V; ++q) {
            double key = stored[v + q] / s->temperature - log(-log(u32_open(w[q])));
            if (key > best_key) { best_key = key; best = v + q; }
        }
    }
    return best;
}

/*
 * Fill target [B][K+1][V], draft [B][K][V] (may be NULL when make_draft == 0)
 * and tokens [B][K].  Returns 0, or -1 when a planted maximum is not unique.
 */
int synth_make_problem(const synth_spec* s, void* target, void* draft, int32_t* tokens)
{
    const int32_t B = s->B, K = s->K, V = s->V;
    int bad = 0;
    #pragma omp parallel reduction(| : bad)
    {
        double* trow = (double*)malloc(sizeof(double) * (size_t)V);
        double* stored = (double*)malloc(sizeof(double) * (size_t)V);
        int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)V);
        #pragma omp for schedule(dynamic, 1)
        for (int64_t bj = 0; bj < (int64_t)B * (K + 1); ++bj) {
            const int32_t b = (int32_t)(bj / (K + 1)), j = (int32_t)(bj % (K + 1));
            const uint32_t trow_id = (uint32_t)bj;
            target_row_f64(s, trow_id, trow, perm);
            const int64_t tbase = bj * (int64_t)V;
            for (int32_t v = 0; v < V; ++v) stored[v] = store_value(target, tbase + v, s->dtype, trow[v]);
            if (s->plant) {
                const int32_t pi = planted_index(s, trow_id);
                for (int32_t v = 0; v < V; ++v)
                    if (v != pi && stored[v] >= stored[pi]) bad = 1;
            }
            if (j == K) continue; /* bonus row: no draft, no token */
            const uint32_t drow_id = (uint32_t)((int64_t)b * K + j);
            if (s->make_draft && draft) {
                const double sigma = (K > 1) ? s->sigma_first + (s->sigma_last - s->sigma_first) * (double)j / (double)(K - 1)
                                             : s->sigma_first;
                const int64_t dbase = (int64_t)drow_id * V;
                for (int32_t v = 0; v < V; v += 4) {
                    double z[4];
                    normals4((uint32_t)(v >> 2), drow_id, STREAM_DRAFT, s->seed_draft, z);
                    for (int q = 0; q < 4 && v + q < V; ++q)
                        stored[v + q] = store_value(draft, dbase + v + q, s->dtype, trow[v + q] + sigma * z[q]);
                }
            }
            if (s->token_mode == 0) {
                tokens[drow_id] = gumbel_max_token(s, drow_id, stored);
            } else if (s->token_mode == 2) {
                /* a drafter that picks greedily: the first id holding the
                 * largest stored draft value */
                int32_t best = 0;
                for (int32_t v = 1; v < V; ++v)
                    if (stored[v] > stored[best]) best = v;
                tokens[drow_id] = best;
            } else {
                uint32_t w[4];
                philox_block(0u, drow_id, STREAM_COIN, s->seed_tokens, w);
                if (u32_open(w[0]) < s->p_match)
                    tokens[drow_id] = planted_index(s, trow_id);
                else
                    tokens[drow_id] = (int32_t)(((uint64_t)w[1] * (uint64_t)V) >> 32);
            }
        }
        free(trow);
        free(stored);
        free(perm);
    }
    return bad ? -1 : 0;
}

/* Per-sequence threshold chosen by seed from a list of n_choices values. */
void synth_choose_tau(uint32_t seed, int32_t B, const float* choices, int32_t n_choices, float* out)
{
    for (int32_t b = 0; b < B; ++b) {
        uint32_t w[4];
        philox_block((uint32_t)b, 0u, STREAM_TAU, seed, w);
        out[b] = choices[w[0] % (uint32_t)n_choices];
    }
}

/* Raw Philox words (for tests of the stream layout). */
void synth_philox_words(uint32_t seed, uint32_t row, uint32_t stream, uint32_t n_blocks, uint32_t* out)
{
    for (uint32_t c = 0; c < n_blocks; ++c) philox_block(c, row, stream, seed, out + 4 * (size_t)c);
}
