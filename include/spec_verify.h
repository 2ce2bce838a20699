/*
 * spec_verify -- batched verification of drafted tokens on one AMD Instinct
 * MI355X (gfx950).  C ABI; plain pointers and sizes only.
 *
 * The operation (one verification step for B sequences at once):
 *   A draft model proposes K tokens per sequence; the target model scores the
 *   whole block in one pass; the verifier keeps the longest prefix the target
 *   accepts and appends one token the target generates itself; everything after
 *   the first rejection is discarded.
 *     - umans.ai blog "DeepSeek V4 Pro DSpark: the model isn't ready, the
 *       architecture is", section "Speculative decoding, briefly";
 *     - zhichai.net article on DSpark, section "Why LLMs speak so slowly"
 *       (generation restarts from the first error).
 *   Acceptance is rejection sampling on the target/draft probability ratio so
 *   that emitted tokens follow the target distribution exactly (same two
 *   sections).  Concretely, with p = softmax(target_logits / T) and
 *   q = softmax(draft_logits / T) at position j:
 *     accept x_j  iff  u_j < p_j(x_j) / q_j(x_j)      (probability min(1, p/q));
 *     after the first rejection at j*, the replacement is drawn from
 *     max(0, p_j* - q_j*) normalised, by inverse CDF in ascending token id;
 *     when every verified position is accepted, the bonus token is drawn from
 *     p of the next row by inverse CDF.
 *   T == 0 selects greedy verification: the target token is the argmax of the
 *   raw target row (lowest id on ties); x_j is accepted iff it equals it.
 *   With draft_mode SV_DRAFT_ONEHOT, q_j is the point mass at x_j (see the
 *   field's comment below).
 *
 *   Verify length (confidence scheduling): each draft position carries a
 *   confidence c_j, the probability that it survives given that all earlier
 *   positions survived; the survival of a prefix is the product along the
 *   block; how many positions to verify depends on these survivals and the
 *   load.
 *     - umans.ai blog, section "2. Verify smarter: a throttle that costs the
 *       user nothing"; zhichai.net article, section "Under the hood".
 *   This library's rule:  S_0 = 1,  S_j = S_{j-1} * c_j,
 *                         L = max({0} U {j in 1..K : S_j >= tau}),
 *   with tau given per sequence (the load-dependent threshold) and c either
 *   given by the caller or c_j = max_v q_j(v).  Only positions 1..L are tested.
 *
 * Layout (all device memory, row-major, vocabulary contiguous):
 *   target_logits  element (b, j, v), j = 0..K (row K is the bonus row),
 *                  at target_logits + b*target_batch_stride + j*target_row_stride + v
 *   draft_logits   element (b, j, v), j = 0..K-1, same scheme with draft strides
 *   both tensors share one element type (SV_F32 or SV_BF16, set at create).
 *   Strides are in elements; a batch stride of 0 shares one set of rows among
 *   all sequences.  Row strides must be >= V.
 *   draft_tokens   int32 [B][K]
 *   uniforms       float [B][K+1]: column j < K is the accept test of position
 *                  j+1; column K is the final (replacement or bonus) draw.
 *                  Values in (0, 1).
 *
 * Outputs (device, caller-allocated):
 *   accepted_len   int32 [B]      a_b, number of accepted drafted tokens
 *   out_tokens     int32 [B][K+1] x_1..x_a, then the final token, then -1
 *   verify_len_out int32 [B]      L_b
 *   optional (NULL = skip; entries the step does not evaluate are left untouched):
 *   lse_target     float [B][K+1] log-sum-exp of target_logits/T for rows 1..a+1
 *   lse_draft      float [B][K]   same for the draft rows the step reads
 *   survival       float [B][K]   S_j (tau mode; with derived c, for the
 *                                 positions whose draft row was read)
 *   residual_mass  float [B]      Z = sum max(0, p - q) of the replacement draw;
 *                                 1 for a bonus draw; 0 if a rejection met Z <= 0
 *                                 (then the draw falls back to p); NaN for greedy
 *   sampled_prob   float [B]      probability of the final token under its draw
 *   rows_read      int32 [B]      logit rows (target + draft) of which the step
 *                                 streamed at least one split for the sequence;
 *                                 rows of positions dispatched before an earlier
 *                                 rejection was known count
 *   bytes_read     int64 [B]      logit bytes streamed for the sequence (each
 *                                 streamed split of a row once)
 *   device_status  int32 [1]      0, or SV_STATUS_* bits (see below)
 *
 * Ownership: the caller owns every buffer and keeps it alive until the work
 * queued on the stream has finished.  The handle owns its workspace, allocated
 * once by spec_verify_create; spec_verify_run allocates nothing.
 *
 * Streams and threads: spec_verify_run only enqueues work on the given HIP
 * stream (NULL = the default stream) and never synchronises the host.  One
 * handle serves one stream at a time; calls that overlap on one handle race.
 * Separate handles are independent.
 *
 * Errors: argument checks run on the host before anything is enqueued and
 * return SV_EINVAL / SV_EUNSUPPORTED with outputs untouched.  A failed launch
 * returns SV_EDEVICE.  Drafted ids outside [0, V) at a tested position, or a
 * given verify length outside [0, K], are found on the device: that sequence
 * gets a = 0 and no token (-1), and SV_STATUS_BAD_INPUT is set.
 *
 * Determinism: for identical inputs the outputs are bitwise identical from run
 * to run, and a sequence's outputs do not depend on its batch position or on B.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spec_verify spec_verify_t; /* opaque handle */

enum { SV_OK = 0, SV_EINVAL = -1, SV_ENOMEM = -2, SV_EDEVICE = -3, SV_EUNSUPPORTED = -4 };
enum { SV_F32 = 0, SV_BF16 = 1 };
enum { SV_LEN_FIXED = 0, SV_LEN_TAU = 1 };
enum { SV_DRAFT_PROBS = 0, SV_DRAFT_ONEHOT = 1 };
/* device_status bits.  SV_STATUS_INCOMPLETE: a sequence's verify-length walk
 * did not finish on the device (an internal consistency check; the sequence is
 * reported like a bad one).  No valid input raises it. */
enum { SV_STATUS_BAD_INPUT = 1, SV_STATUS_INCOMPLETE = 2 };

/* Limits checked by spec_verify_create.  Besides these, the largest launch of
 * a configuration must stay within 2^32 - 1 work-items: max_batch *
 * 2 * min(32, max_draft + 1) * ceil(vocab / 16384) workgroups of 256 (and
 * max_batch * ceil(vocab / 16384) * 2 of them); larger configurations return
 * SV_EUNSUPPORTED. */
#define SV_MAX_VOCAB 1048576
#define SV_MAX_BATCH 1048575
#define SV_MAX_DRAFT 256

typedef struct {
    int32_t max_batch; /* 1..SV_MAX_BATCH; workspace is sized from these three */
    int32_t max_draft; /* 1..SV_MAX_DRAFT */
    int32_t vocab;     /* V, 1..SV_MAX_VOCAB */
    int32_t dtype;     /* SV_F32 | SV_BF16, for both logit tensors */
    int32_t device;    /* HIP device ordinal */
} spec_verify_config;

typedef struct {
    int32_t B, K;                  /* 0 <= B <= max_batch; 1 <= K <= max_draft */
    const void* target_logits;     /* see layout above */
    int64_t target_batch_stride, target_row_stride;
    const void* draft_logits;      /* NULL allowed iff temperature == 0 */
    int64_t draft_batch_stride, draft_row_stride;
    const int32_t* draft_tokens;   /* [B][K] */
    const float* uniforms;         /* [B][K+1]; NULL allowed iff temperature == 0 */
    float temperature;             /* > 0 rejection sampling; == 0 greedy */
    int32_t length_mode;           /* SV_LEN_FIXED | SV_LEN_TAU */
    const int32_t* verify_len_in;  /* FIXED: [B] in [0, K], or NULL => L = K */
    const float* confidence;       /* TAU: [B][K] in [0, 1], or NULL => c_j = max_v q_j(v) (needs T > 0) */
    const float* tau;              /* TAU: [B] */
    int32_t* accepted_len;         /* [B] */
    int32_t* out_tokens;           /* [B][K+1] */
    int32_t* verify_len_out;       /* [B] */
    float* lse_target;             /* optional [B][K+1] */
    float* lse_draft;              /* optional [B][K] */
    float* survival;               /* optional [B][K] */
    float* residual_mass;          /* optional [B] */
    float* sampled_prob;           /* optional [B] */
    int32_t* rows_read;            /* optional [B] */
    int32_t* device_status;        /* optional [1] */
    int32_t draft_mode;            /* SV_DRAFT_PROBS (0): q = softmax(draft_logits / T).
                                      SV_DRAFT_ONEHOT: the drafter chose greedily, so q_j is the
                                      point mass at x_j (techvisionai blog, Chapter 7: vLLM's
                                      draft_sample_method greedy).  Acceptance has probability
                                      p_j(x_j); the replacement is p_j without x_j, renormalised;
                                      derived c_j = 1.  draft_logits is not read (may be NULL);
                                      lse_draft is not written; no draft row is streamed. */
    const int64_t* target_row_offsets; /* optional device [B+1]: packed rows ("pruned, not padded":
                                      zhichai.net article, "Under the hood", on variable-length
                                      verification in SGLang).  Target row j (0-based) of sequence b
                                      is row target_row_offsets[b] + j of a [total rows][V] tensor at
                                      target_logits (row stride as above; batch stride unused); the
                                      sequence brings L_b + 1 rows, so L_b is their count minus 1
                                      (SV_LEN_FIXED, verify_len_in must be NULL).  A count outside
                                      [1, K+1] marks the sequence bad.  NULL = the dense layout. */
    const int64_t* draft_row_offsets;  /* packed draft rows, [B+1] likewise (L_b rows per sequence;
                                      a different count marks the sequence bad).  Required with
                                      target_row_offsets when T > 0 and SV_DRAFT_PROBS. */
    int64_t* bytes_read;           /* optional [B] */
    int32_t max_verify_len;        /* 0 = no bound.  SV_LEN_FIXED only (dense or packed), 1..K: the
                                      caller's promise that every L_b <= max_verify_len, as an
                                      engine knows once it has built the verify batch (the packed
                                      layout's row counts, or admission's lengths).  The step then
                                      launches no work for positions past max_verify_len + 1, so
                                      short verify batches do not pay for K + 1 positions.  A
                                      sequence whose L_b exceeds the bound is marked bad (a = 0, no
                                      token, SV_STATUS_BAD_INPUT); the others' outputs are those
                                      of the unbounded call, bit for bit. */
} spec_verify_args;

/* Allocate a handle and its workspace on cfg->device.  *out is set only on SV_OK. */
int spec_verify_create(const spec_verify_config* cfg, spec_verify_t** out);

/* Host-only argument check of one call against a configuration; touches no
 * device state.  Returns SV_OK, SV_EINVAL or SV_EUNSUPPORTED. */
int spec_verify_check(const spec_verify_config* cfg, const spec_verify_args* a);

/* Enqueue one verification step on hip_stream (a hipStream_t, or NULL).  The
 * step is kernel launches on that stream only (no allocation, copy, memset or
 * synchronisation), so it may be captured in a HIP graph; a captured step
 * reads the pointers and sizes of the args it was captured with. */
int spec_verify_run(spec_verify_t* h, const spec_verify_args* a, void* hip_stream);

/* For callers that cannot allocate device memory at all (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): one
 * verification step without a handle, identical in its outputs to
 * spec_verify_run.  Its workspace is a static device array of
 * SV_NOALLOC_SCRATCH_BYTES on cfg->device, loaded with the library and held
 * until the process ends; the call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine) and only launches kernels on hip_stream.
 *
 * cfg gives the vocabulary, dtype and device, and the limits a->B and a->K are
 * checked against (as for spec_verify_check).  The workspace the call needs
 * grows with a->B, a->K and vocab: about 15 KB per sequence at K = 16 and
 * V = 129280, so up to 1024 such sequences fit.  A call that needs more than
 * the array returns SV_EUNSUPPORTED before any device work; other errors as
 * for spec_verify_run (devices numbered 64 and above: SV_EUNSUPPORTED).
 *
 * The array is shared by every call on one device and keeps the last call's
 * contents; each call's first kernel clears what must start at zero.  Calls
 * that overlap on one device (other streams, other threads) race and give
 * undefined results: serialise them. */
#define SV_NOALLOC_SCRATCH_BYTES 16777216
int spec_verify_run_noalloc(const spec_verify_config* cfg, const spec_verify_args* a, void* hip_stream);

/* Free the handle.  The caller synchronises the stream first.  NULL is a no-op. */
int spec_verify_destroy(spec_verify_t* h);

/* Static description of a status code. */
const char* spec_verify_status_string(int status);

/* Per-kernel timing with HIP events, for benchmarks.  After
 * spec_verify_timing_begin(h, max_calls), the next max_calls runs launch each
 * kernel with a start and a stop event attached to its dispatch
 * (hipExtLaunchKernelGGL), which time the kernel's execution itself; a kernel
 * the step does not launch records nothing.  Outputs are unchanged.
 * spec_verify_timing_end synchronises those events, writes the summed
 * milliseconds of kernel k to ms[k] (k < n_kernels, see
 * spec_verify_kernel_name), the number of timed runs to *n_runs, and frees
 * the events. */
int spec_verify_timing_begin(spec_verify_t* h, int32_t max_calls);
int spec_verify_timing_end(spec_verify_t* h, double* ms, int32_t n_kernels, int32_t* n_runs);

/* Number of kernels a run launches, and the name of kernel k (static string). */
int32_t spec_verify_kernel_count(void);
const char* spec_verify_kernel_name(int32_t k);

/*
 * Load-aware admission: how many drafted positions each sequence verifies.
 *
 *   umans.ai blog, section "2. Verify smarter: a throttle that costs the user
 *   nothing": the engine's step rate is profiled once against batch size;
 *   every step, expected throughput is expected accepted tokens times the rate
 *   at that batch size; every candidate token of every request is ranked by
 *   survival probability and admitted one at a time until that product stops
 *   rising.  zhichai.net article, section "Under the hood": the verified
 *   prefix of each request maximises accepted tokens x verification speed.
 *
 * This library's rule (the oracle follows the same words):
 *   S_bj = prod_{i<=j} c_bi (fp64, left to right); every drafted position
 *   (b, j) is ranked by S descending, then b, then j ascending; admitting the
 *   first m gives a verify batch of B + m tokens and
 *     T(m) = (B + sum of the m best survivals) * speed[B + m];
 *   m is the first value with T(m + 1) <= T(m) (m = B K if none);
 *   L_b = number of admitted positions of sequence b (always positions 1..L_b).
 * Feed L_b to spec_verify_run as verify_len_in with SV_LEN_FIXED.
 *
 * Layout: confidence float [B][K] (device), speed double [n_speed] (device):
 * steps per second of a verify batch of n tokens, finite and >= 0, n_speed >=
 * B (K + 1) + 1.  Outputs (device, caller-allocated): verify_len_out int32 [B];
 * optional survival float [B][K], admitted int32 [1] (m), tau float [1]
 * (smallest admitted survival, NaN if m = 0), expected_rate double [1] (T(m)),
 * device_status int32 [1] (SV_STATUS_BAD_INPUT if a confidence was outside
 * [0, 1]; such values are clamped into it, NaN to 0).
 * Limits: B <= min(max_batch, SV_MAX_SCHED_BATCH), K <= max_draft,
 * B K <= SV_MAX_SCHED_CANDIDATES.  Errors as for spec_verify_run: host checks
 * first (SV_EINVAL / SV_EUNSUPPORTED, nothing enqueued), SV_EDEVICE on a
 * failed launch.  Uses the handle's workspace: calls on one handle must not
 * overlap with each other or with spec_verify_run.  Deterministic: a
 * fixed-order prefix, no floating-point atomics.
 */
#define SV_MAX_SCHED_BATCH 4096
#define SV_MAX_SCHED_CANDIDATES 65536

typedef struct {
    int32_t B, K;
    const float* confidence;      /* [B][K] */
    const double* speed;          /* [n_speed] */
    int32_t n_speed;
    int32_t* verify_len_out;      /* [B] */
    float* survival;              /* optional [B][K] */
    int32_t* admitted;            /* optional [1] */
    float* tau;                   /* optional [1] */
    double* expected_rate;        /* optional [1] */
    int32_t* device_status;       /* optional [1] */
} spec_verify_sched_args;

/*
 * Calibrated, causally delayed confidences (the input of the two calls above).
 *
 *   umans.ai blog, section "2. Verify smarter": raw confidence is calibrated
 *   with a per-position temperature fitted on held-out data, and the
 *   production version sizes the truncation from confidence measured two
 *   steps earlier, a causal barrier between the decision and the tokens it
 *   could otherwise peek at.  zhichai.net article, section "Under the hood":
 *   Sequential Temperature Scaling.
 *
 * Each call takes this step's raw confidence logits z [B][K] (slot b, drafted
 * position j) and per-position temperatures T [K]:
 *   conf_now[b][j] = sigmoid(z_bj / T_j)   (fp64, rounded to fp32; a temperature
 *                    that is not finite and positive gives 0 and raises
 *                    SV_STATUS_BAD_INPUT),
 *   conf_out[b][j] = the conf_now of slot b, position j from `delay` calls
 *                    earlier, or c_default while the slot has recorded fewer
 *                    than `delay` calls since its last reset (delay 0: conf_now).
 * The handle keeps the last SV_MAX_CONF_DELAY calls of every slot (zero from
 * create on).  reset[b] != 0 says slot b holds a new sequence from this call on:
 * its history is dropped first.  Keep K fixed while a slot's history is in use.
 * conf_out feeds spec_verify_schedule (confidence) or spec_verify_run (tau mode).
 * Fitting the temperatures is not part of the library.
 * Limits: B <= max_batch, K <= max_draft, max_batch * max_draft <=
 * SV_MAX_SCHED_CANDIDATES (the history is sized at create).  Host checks as for
 * the other calls; calls on one handle must not overlap.
 */
#define SV_MAX_CONF_DELAY 4

typedef struct {
    int32_t B, K;
    const float* conf_logits;     /* device [B][K] */
    const float* temperature;     /* device [K] */
    const int32_t* reset;         /* optional device [B] */
    int32_t delay;                /* 0 .. SV_MAX_CONF_DELAY */
    float c_default;
    float* conf_now;              /* optional device [B][K] */
    float* conf_out;              /* device [B][K] */
    int32_t* device_status;       /* optional device [1] */
} spec_verify_conf_args;

int spec_verify_conf_check(const spec_verify_config* cfg, const spec_verify_conf_args* a);
int spec_verify_confidence(spec_verify_t* h, const spec_verify_conf_args* a, void* hip_stream);

/* Host-only check of a spec_verify_schedule call.  Returns SV_OK, SV_EINVAL or
 * SV_EUNSUPPORTED. */
int spec_verify_sched_check(const spec_verify_config* cfg, const spec_verify_sched_args* a);

/* Enqueue the admission decision on hip_stream (a hipStream_t, or NULL). */
int spec_verify_schedule(spec_verify_t* h, const spec_verify_sched_args* a, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
