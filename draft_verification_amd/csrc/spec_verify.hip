// Batched draft verification for AMD Instinct MI355X (gfx950, CDNA4).
//
// What one call computes is stated in include/spec_verify.h (with the passages
// of the pages it follows).  This file holds the kernels and the C ABI.
//
// Shape of the work.  Every verified position j of sequence b needs the
// log-sum-exp of its target row (and, when T > 0, of its draft row): a pure
// streaming reduction over V ~ 128K logits per row, bound by HBM bandwidth.
// Nothing here is a dense contraction, so there is no MFMA; the kernels are
// built around 16-byte coalesced loads, wavefront shuffles and small LDS
// reductions.
//
// Pipeline of one call (four launches on the caller's stream):
//   sv_plan     per-sequence set-up: verify length where it is known without
//               reading logits, work-queue initialisation.
//   sv_stream   persistent, queue-driven.  A queue entry is "position j of
//               sequence b"; its items are fixed 16384-element splits of the
//               target row and of the draft row.  Each item reduces its split
//               to (max, sum exp) and the last item of an entry to finish merges
//               the splits and takes the per-position decision: survival and
//               verify length, the acceptance test u < p/q (or the greedy
//               match), and what comes next.  Only then is position j+1 of that
//               sequence put on the queue, so rows after the first rejection
//               (and draft rows past the verify length) are never read.  The
//               pages say generation restarts from the first error; nothing
//               after it can change the output.
//   sv_resid    per (rejecting sequence, split): sum of max(0, p - q) over the
//               split of the rejected row pair.
//   sv_draw     per sequence: inverse-CDF draw (replacement or bonus) by split
//               prefix in fp64, then one 16384-element split re-read and scanned
//               in token order; writes all outputs.
//
// Numerics.  bf16 and fp32 inputs are exact in fp32.  Per element the kernel
// forms a = (l - m) * log2(e)/T with the constant split in two fp32 parts (so
// the scale carries no systematic rounding bias) and takes v_exp_f32.  Sums run
// in fp32 over 8 elements and in fp64 beyond, so a row sum carries ~1e-8
// relative error.  Decisions (acceptance ratio, survival product, CDF prefix)
// are taken in fp64.  The final draw evaluates large masses (> 2^-12) in fp64.
//
// Determinism.  Split boundaries depend only on V, every reduction has a fixed
// order and there are no floating-point atomics, so outputs are bitwise
// reproducible and independent of a sequence's batch position and of B.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;              // 4 wavefronts of 64
constexpr int kWaves = kThreads / 64;
constexpr int kSplit = 16384;              // elements per split (fixed for batch invariance)
constexpr int kPerLane = kSplit / kThreads; // 64 elements per lane per split
constexpr int kMaxSplits = SV_MAX_VOCAB / kSplit; // 64
constexpr uint32_t kNeedT = 1u << 30;
constexpr uint32_t kNeedD = 1u << 31;
constexpr unsigned long long kTimeoutTicks = 400000000ull; // 4 s of the 100 MHz real-time counter

enum { CTL_HEAD = 0, CTL_TAIL = 1, CTL_FINISHED = 2, CTL_STATUS = 3, CTL_WORDS = 64 };
enum { FL_ACC = 1, FL_LEN = 2 };
enum { KIND_NONE = -1, KIND_RESID = 0, KIND_BONUS = 1, KIND_GREEDY = 2, KIND_BAD = 3 };
enum { K_PLAN = 0, K_STREAM = 1, K_RESID = 2, K_DRAW = 3, K_COUNT = 4 };

struct SeqState {
    double S;      // survival product S_j of the positions evaluated so far
    double St, Sd; // sums of exp2((l - M) c) of the rows of the final draw
    float Mt, Md;  // maxima of those rows
    int L;         // verify length, -1 while undetermined
    int a;         // accepted positions so far
    int flags;     // FL_ACC: acceptance walk open; FL_LEN: verify length open
    int kind;      // KIND_*
    int js;        // 1-based row of the final draw
    int y;         // token chosen in sv_stream (greedy)
    int e_final;   // queue entry that holds the final target row's split partials
    int pad;
};

struct Work {
    int* ctl;
    uint32_t* queue;  // [entries] packed (b, j, need target, need draft), 0 = not yet published
    int* cnt;         // [entries] finished items per entry
    float* part_m;    // [entries][2][nsplit] split maxima (target, draft)
    double* part_s;   // [entries][2][nsplit] split sums
    int* part_i;      // [entries][nsplit] split argmax (greedy)
    SeqState* st;     // [max_batch]
    double* rsum;     // [max_batch][nsplit] residual mass per split
};

struct Params {
    int B, K, V, nsplit, ipe;  // ipe: items per queue entry
    int greedy, derived;       // derived: tau mode with c = max draft probability
    int len_mode;
    const void* t;
    long long tbs, trs;
    const void* d;
    long long dbs, drs;
    const int* tok;
    const float* u;
    const int* vl_in;
    const float* conf;
    const float* tau;
    double invT64, c64;        // 1/T and log2(e)/T in fp64
    float c_hi, c_lo;          // c64 = c_hi + c_lo, c_hi rounded toward zero, c_lo > 0
    int* acc_out;
    int* out_tok;
    int* vl_out;
    float* lse_t;
    float* lse_d;
    float* surv;
    float* zmass;
    float* pys;
    int* status_out;
};

// ---------------------------------------------------------------- memory model

__device__ __forceinline__ int ld_relaxed(const int* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ uint32_t ld_relaxed_u(const uint32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_relaxed_u(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ int add_relaxed(int* p, int v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ int add_acq_rel(int* p, int v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void or_relaxed(int* p, int v) { __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }

__device__ __forceinline__ uint32_t enc_word(int b, int j, bool nt, bool nd)
{
    return (uint32_t)b | ((uint32_t)j << 20) | (nt ? kNeedT : 0u) | (nd ? kNeedD : 0u);
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// (value, index) maximum with the lower index on ties
__device__ __forceinline__ void wave_argmax(float& v, int& i)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float ov = __shfl_xor(v, o);
        int oi = __shfl_xor(i, o);
        if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
    }
}

__device__ __forceinline__ float block_max(float v, float* red)
{
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return r;
}

__device__ __forceinline__ double block_sum(double v, double* red)
{
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    double r = ((red[0] + red[1]) + red[2]) + red[3];
    __syncthreads();
    return r;
}

__device__ __forceinline__ void block_argmax(float& v, int& i, float* redf, int* redi)
{
    wave_argmax(v, i);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { redf[w] = v; redi[w] = i; }
    __syncthreads();
    v = redf[0];
    i = redi[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k)
        if (redf[k] > v || (redf[k] == v && redi[k] < i)) { v = redf[k]; i = redi[k]; }
    __syncthreads();
}

// ---------------------------------------------------------------- split loads
//
// A split is 16384 consecutive elements of one row.  Lane l holds 64 of them.
// bf16: 8 loads of 16 bytes; element e of the lane is split_base +
//       (e/8)*2048 + l*8 + e%8.
// fp32: 16 loads of 16 bytes; element e is split_base + (e/4)*1024 + l*4 + e%4.
// Every load instruction of a wavefront covers 1 KB contiguous.  Elements past
// V read as -inf.  With VEC the row start is 16-byte aligned and V is a whole
// number of vectors, so a vector is either fully inside the row or fully out.

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int DT>
struct Chunk;

template <>
struct Chunk<SV_BF16> {
    uint32_t w[kPerLane / 2];
    __device__ __forceinline__ float get(int e) const { return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]); }
    __device__ __forceinline__ static int index(int base, int lane, int e) { return base + (e >> 3) * 2048 + lane * 8 + (e & 7); }
    template <bool VEC>
    __device__ __forceinline__ void load(const void* row, int base, int V, int lane)
    {
        const uint16_t* r = (const uint16_t*)row;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i0 = base + k * 2048 + lane * 8;
            if (VEC) {
                if (i0 < V) {
                    const uint4 q = *(const uint4*)(r + i0);
                    w[4 * k] = q.x; w[4 * k + 1] = q.y; w[4 * k + 2] = q.z; w[4 * k + 3] = q.w;
                } else {
                    w[4 * k] = w[4 * k + 1] = w[4 * k + 2] = w[4 * k + 3] = 0xFF80FF80u;
                }
            } else {
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const int i = i0 + 2 * h;
                    const uint32_t lo = i < V ? (uint32_t)r[i] : 0xFF80u;
                    const uint32_t hi = i + 1 < V ? (uint32_t)r[i + 1] : 0xFF80u;
                    w[4 * k + h] = lo | (hi << 16);
                }
            }
        }
    }
};

template <>
struct Chunk<SV_F32> {
    float w[kPerLane];
    __device__ __forceinline__ float get(int e) const { return w[e]; }
    __device__ __forceinline__ static int index(int base, int lane, int e) { return base + (e >> 2) * 1024 + lane * 4 + (e & 3); }
    template <bool VEC>
    __device__ __forceinline__ void load(const void* row, int base, int V, int lane)
    {
        const float* r = (const float*)row;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int i0 = base + k * 1024 + lane * 4;
            if (VEC) {
                if (i0 < V) {
                    const float4 q = *(const float4*)(r + i0);
                    w[4 * k] = q.x; w[4 * k + 1] = q.y; w[4 * k + 2] = q.z; w[4 * k + 3] = q.w;
                } else {
                    w[4 * k] = w[4 * k + 1] = w[4 * k + 2] = w[4 * k + 3] = -INFINITY;
                }
            } else {
#pragma unroll
                for (int h = 0; h < 4; ++h) w[4 * k + h] = (i0 + h < V) ? r[i0 + h] : -INFINITY;
            }
        }
    }
};

template <int DT>
__device__ __forceinline__ float load_one(const void* row, int i)
{
    if (DT == SV_BF16) return bf16_lo((uint32_t)((const uint16_t*)row)[i]);
    return ((const float*)row)[i];
}

template <int DT>
__device__ __forceinline__ const void* row_ptr(const void* base, long long bs, long long rs, int b, int j)
{
    const long long off = (long long)b * bs + (long long)j * rs;
    return (const void*)((const char*)base + off * (DT == SV_BF16 ? 2 : 4));
}

// exp2((l - m) * c) with c = c_hi + c_lo; exact subtraction for bf16 inputs,
// no bias from rounding c.  l = -inf gives 0 (c_lo > 0 keeps the product -inf).
__device__ __forceinline__ float scaled_exp2(float l, float m, float c_hi, float c_lo)
{
    const float t = l - m;
    return __builtin_amdgcn_exp2f(fmaf(t, c_hi, t * c_lo));
}

// (max, sum exp) of one split: sum in fp32 over runs of 8 elements, fp64 beyond.
template <int DT, bool VEC>
__device__ void split_stats(const void* row, int V, int split, float c_hi, float c_lo, float& M, double& S,
                            float* redf, double* redd)
{
    Chunk<DT> c;
    c.template load<VEC>(row, split * kSplit, V, threadIdx.x);
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) m = fmaxf(m, c.get(e));
    m = block_max(m, redf);
    double acc = 0.0;
    if (m != -INFINITY) {
#pragma unroll
        for (int r = 0; r < kPerLane / 8; ++r) {
            float run = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) run += scaled_exp2(c.get(8 * r + i), m, c_hi, c_lo);
            acc += (double)run;
        }
    }
    S = block_sum(acc, redd);
    M = m;
}

// (max, lowest index of the max) of one split of the raw row.
template <int DT, bool VEC>
__device__ void split_argmax(const void* row, int V, int split, float& M, int& I, float* redf, int* redi)
{
    Chunk<DT> c;
    c.template load<VEC>(row, split * kSplit, V, threadIdx.x);
    float best = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
        const float v = c.get(e);
        const int idx = Chunk<DT>::index(split * kSplit, threadIdx.x, e);
        if (idx < V && (v > best || bi == 0x7fffffff)) { best = v; bi = idx; }
    }
    block_argmax(best, bi, redf, redi);
    M = best;
    I = bi;
}

// ---------------------------------------------------------------- sv_plan

__global__ __launch_bounds__(kThreads) void sv_plan_kernel(Params p, Work w)
{
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long ne = (long long)p.B * (p.K + 1);
    if (i == 0) {
        w.ctl[CTL_HEAD] = 0;
        w.ctl[CTL_TAIL] = p.B;
        w.ctl[CTL_FINISHED] = 0;
        w.ctl[CTL_STATUS] = 0;
    }
    if (i < ne) {
        w.cnt[i] = 0;
        if (i >= p.B) w.queue[i] = 0u;
    }
    if (i >= p.B) return;
    const int b = (int)i, K = p.K;
    SeqState st;
    st.S = 1.0;
    st.St = st.Sd = 0.0;
    st.Mt = st.Md = 0.0f;
    st.a = 0;
    st.kind = KIND_NONE;
    st.js = 0;
    st.y = -1;
    st.e_final = -1;
    st.pad = 0;
    bool bad = false, len_open = false;
    int L;
    if (p.len_mode == SV_LEN_FIXED) {
        L = p.vl_in ? p.vl_in[b] : K;
        if (L < 0 || L > K) bad = true;
    } else if (p.conf) {
        // given confidences: S_j = S_{j-1} c_j, L = max({0} U {j : S_j >= tau})
        const double tau = (double)p.tau[b];
        double S = 1.0;
        L = 0;
        for (int j = 1; j <= K; ++j) {
            S *= (double)p.conf[(long long)b * K + (j - 1)];
            if (p.surv) p.surv[(long long)b * K + (j - 1)] = (float)S;
            if (S >= tau) L = j;
        }
    } else {
        // c_j = max_v q_j(v) lies in (0, 1], so tau <= 0 passes every position and
        // tau > 1 (or NaN) none; otherwise the walk along the block decides.
        const float tau = p.tau[b];
        if (!(tau <= 1.0f)) L = 0;
        else if (tau <= 0.0f) L = K;
        else { L = -1; len_open = true; }
    }
    st.L = L;
    if (bad) {
        st.kind = KIND_BAD;
        st.flags = 0;
        or_relaxed(&w.ctl[CTL_STATUS], SV_STATUS_BAD_INPUT);
    } else {
        st.flags = FL_ACC | (len_open ? FL_LEN : 0);
    }
    w.st[b] = st;
    const bool nt = !bad;
    const bool nd = !bad && !p.greedy && (len_open || L >= 1);
    w.queue[b] = enc_word(b, 1, nt, nd);
}

// ---------------------------------------------------------------- sv_stream
//
// Per-position decision, run by the workgroup that finishes the last item of
// queue entry e = (b, j).  Wave 0 merges the split partials; thread 0 updates
// the sequence state and publishes (b, j+1) or retires the sequence.

template <int DT, bool GREEDY>
__device__ void decide(const Params& p, const Work& w, int e, int b, int j, bool nt, bool nd)
{
    __shared__ float s_Mt, s_Md;
    __shared__ double s_St, s_Sd;
    __shared__ int s_g;
    const int lane = threadIdx.x;
    if (lane < 64) {
        const bool has = lane < p.nsplit;
        if (nt) {
            const long long pb = ((long long)e * 2 + 0) * p.nsplit + lane;
            if (GREEDY) {
                float v = has ? w.part_m[pb] : -INFINITY;
                int ix = has ? w.part_i[(long long)e * p.nsplit + lane] : 0x7fffffff;
                wave_argmax(v, ix);
                if (lane == 0) { s_Mt = v; s_g = ix; }
            } else {
                const float m = has ? w.part_m[pb] : -INFINITY;
                const float M = wave_max(m);
                double s = 0.0;
                if (has && m != -INFINITY) s = w.part_s[pb] * exp2(((double)m - (double)M) * p.c64);
                s = wave_sum(s);
                if (lane == 0) { s_Mt = M; s_St = s; }
            }
        }
        if (!GREEDY && nd) {
            const long long pb = ((long long)e * 2 + 1) * p.nsplit + lane;
            const float m = has ? w.part_m[pb] : -INFINITY;
            const float M = wave_max(m);
            double s = 0.0;
            if (has && m != -INFINITY) s = w.part_s[pb] * exp2(((double)m - (double)M) * p.c64);
            s = wave_sum(s);
            if (lane == 0) { s_Md = M; s_Sd = s; }
        }
    }
    __syncthreads();
    if (threadIdx.x != 0) return;

    SeqState st = w.st[b];
    bool acc = (st.flags & FL_ACC) != 0;
    bool len = (st.flags & FL_LEN) != 0;
    const int K = p.K;
    const float Mt = s_Mt, Md = s_Md;
    const double St = s_St, Sd = s_Sd;

    if (!GREEDY) {
        if (nt && p.lse_t) p.lse_t[(long long)b * (K + 1) + (j - 1)] = (float)((double)Mt * p.invT64 + log(St));
        if (nd && p.lse_d) p.lse_d[(long long)b * K + (j - 1)] = (float)((double)Md * p.invT64 + log(Sd));
        if (nd && p.derived) {
            // c_j = max_v q_j(v) = 1 / Sd; S_j = S_{j-1} c_j
            const double S = st.S / Sd;
            st.S = S;
            if (p.surv) p.surv[(long long)b * K + (j - 1)] = (float)S;
            if (len) {
                if (S >= (double)p.tau[b]) {
                    if (j == K) { st.L = K; len = false; }
                } else {
                    st.L = j - 1;
                    len = false;
                }
            }
        }
    }

    if (acc && nt) {
        const bool verify = len || st.L >= j; // open walk means S_j >= tau, so L >= j
        if (verify) {
            const int x = p.tok[(long long)b * K + (j - 1)];
            if (x < 0 || x >= p.V) {
                st.kind = KIND_BAD;
                st.a = 0;
                acc = false;
                or_relaxed(&w.ctl[CTL_STATUS], SV_STATUS_BAD_INPUT);
            } else if (GREEDY) {
                if (x == s_g) {
                    st.a = j;
                } else {
                    st.kind = KIND_GREEDY;
                    st.y = s_g;
                    acc = false;
                }
            } else {
                const float lt = load_one<DT>(row_ptr<DT>(p.t, p.tbs, p.trs, b, j - 1), x);
                const float ld = load_one<DT>(row_ptr<DT>(p.d, p.dbs, p.drs, b, j - 1), x);
                double ratio;
                if (ld == -INFINITY) {
                    ratio = INFINITY; // q(x) = 0
                } else {
                    const double dlt = (double)lt - (double)Mt, dld = (double)ld - (double)Md;
                    ratio = exp2((dlt - dld) * p.c64) * (Sd / St);
                }
                const double uj = (double)p.u[(long long)b * (K + 1) + (j - 1)];
                if (uj < ratio) {
                    st.a = j;
                } else {
                    st.kind = KIND_RESID;
                    st.js = j;
                    st.Mt = Mt; st.St = St; st.Md = Md; st.Sd = Sd;
                    st.e_final = e;
                    acc = false;
                }
            }
        } else {
            // L == j - 1: the final token comes from target row j
            if (GREEDY) {
                st.kind = KIND_GREEDY;
                st.y = s_g;
            } else {
                st.kind = KIND_BONUS;
                st.js = j;
                st.Mt = Mt; st.St = St;
                st.e_final = e;
            }
            acc = false;
        }
    }

    st.flags = (acc ? FL_ACC : 0) | (len ? FL_LEN : 0);
    w.st[b] = st;
    if (acc || len) {
        const int jn = j + 1;
        const bool ntn = acc;
        const bool ndn = !GREEDY && jn <= K && (len || (acc && st.L >= jn));
        const int slot = add_relaxed(&w.ctl[CTL_TAIL], 1);
        fence_release(); // the state above before the queue word
        st_relaxed_u(&w.queue[slot], enc_word(b, jn, ntn, ndn));
    } else {
        fence_release();
        add_relaxed(&w.ctl[CTL_FINISHED], 1);
    }
}

template <int DT, bool VEC, bool GREEDY>
__global__ __launch_bounds__(kThreads) void sv_stream_kernel(Params p, Work w)
{
    __shared__ float redf[kWaves];
    __shared__ double redd[kWaves];
    __shared__ int redi[kWaves];
    __shared__ int s_cmd, s_sub, s_e, s_last;
    __shared__ uint32_t s_word;
    const long long entries = (long long)p.B * (p.K + 1);

    for (;;) {
        if (threadIdx.x == 0) {
            const int item = add_relaxed(&w.ctl[CTL_HEAD], 1);
            const long long e = item / p.ipe;
            int cmd = 0;
            uint32_t word = 0;
            if (e >= entries) {
                cmd = 1;
            } else {
                const unsigned long long t0 = wall_clock64();
                for (;;) {
                    word = ld_relaxed_u(&w.queue[e]);
                    if (word) break;
                    if (ld_relaxed(&w.ctl[CTL_FINISHED]) >= p.B) { cmd = 1; break; }
                    if (wall_clock64() - t0 > kTimeoutTicks) {
                        or_relaxed(&w.ctl[CTL_STATUS], SV_STATUS_TIMEOUT);
                        cmd = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(4);
                }
                if (!cmd) fence_acquire();
            }
            s_cmd = cmd;
            s_word = word;
            s_sub = item % p.ipe;
            s_e = (int)e;
        }
        __syncthreads();
        if (s_cmd) return;
        const uint32_t word = s_word;
        const int sub = s_sub, e = s_e;
        __syncthreads();

        const int b = (int)(word & 0xFFFFFu);
        const int j = (int)((word >> 20) & 0x3FFu);
        const bool nt = (word & kNeedT) != 0, nd = (word & kNeedD) != 0;
        const int kind = GREEDY ? 0 : sub / p.nsplit;
        const int split = GREEDY ? sub : sub % p.nsplit;
        if (kind == 0 ? nt : nd) {
            if (GREEDY) {
                float M;
                int I;
                split_argmax<DT, VEC>(row_ptr<DT>(p.t, p.tbs, p.trs, b, j - 1), p.V, split, M, I, redf, redi);
                if (threadIdx.x == 0) {
                    w.part_m[((long long)e * 2) * p.nsplit + split] = M;
                    w.part_i[(long long)e * p.nsplit + split] = I;
                }
            } else {
                const void* row = kind == 0 ? row_ptr<DT>(p.t, p.tbs, p.trs, b, j - 1)
                                            : row_ptr<DT>(p.d, p.dbs, p.drs, b, j - 1);
                float M;
                double S;
                split_stats<DT, VEC>(row, p.V, split, p.c_hi, p.c_lo, M, S, redf, redd);
                if (threadIdx.x == 0) {
                    const long long pi = ((long long)e * 2 + kind) * p.nsplit + split;
                    w.part_m[pi] = M;
                    w.part_s[pi] = S;
                }
            }
        }
        if (threadIdx.x == 0) {
            const int old = add_acq_rel(&w.cnt[e], 1); // releases this item's partial
            s_last = (old == p.ipe - 1);
        }
        __syncthreads();
        if (s_last) {
            fence_acquire();
            decide<DT, GREEDY>(p, w, e, b, j, nt, nd);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- final draw

struct DrawCtx {
    float Mt, Md, invSt, invSd, c_hi, c_lo;
    double St, Sd, c64;
    bool resid;
};

__device__ __noinline__ double draw_mass_f64(float lt, float ld, const DrawCtx& c)
{
    const double pd = exp2(((double)lt - (double)c.Mt) * c.c64) / c.St;
    const double qd = c.resid ? exp2(((double)ld - (double)c.Md) * c.c64) / c.Sd : 0.0;
    return pd > qd ? pd - qd : 0.0;
}

// Mass of one token under the final draw: max(0, p - q) for a replacement,
// p for a bonus.  fp32 first; masses above 2^-12 are recomputed in fp64.
__device__ __forceinline__ double draw_mass(float lt, float ld, const DrawCtx& c)
{
    const float pf = scaled_exp2(lt, c.Mt, c.c_hi, c.c_lo) * c.invSt;
    const float qf = c.resid ? scaled_exp2(ld, c.Md, c.c_hi, c.c_lo) * c.invSd : 0.0f;
    if (fmaxf(pf, qf) > 0x1p-12f) return draw_mass_f64(lt, ld, c);
    return pf > qf ? (double)(pf - qf) : 0.0;
}

__device__ __forceinline__ DrawCtx make_ctx(const SeqState& st, const Params& p, bool resid)
{
    DrawCtx c;
    c.Mt = st.Mt;
    c.Md = st.Md;
    c.St = st.St;
    c.Sd = st.Sd;
    c.invSt = (float)(1.0 / st.St);
    c.invSd = resid ? (float)(1.0 / st.Sd) : 0.0f;
    c.c_hi = p.c_hi;
    c.c_lo = p.c_lo;
    c.c64 = p.c64;
    c.resid = resid;
    return c;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void sv_resid_kernel(Params p, Work w)
{
    __shared__ double redd[kWaves];
    const int b = (int)(blockIdx.x / p.nsplit);
    const int split = (int)(blockIdx.x % p.nsplit);
    const SeqState st = w.st[b];
    if (st.kind != KIND_RESID) return;
    const DrawCtx c = make_ctx(st, p, true);
    Chunk<DT> tc, dc;
    tc.template load<VEC>(row_ptr<DT>(p.t, p.tbs, p.trs, b, st.js - 1), split * kSplit, p.V, threadIdx.x);
    dc.template load<VEC>(row_ptr<DT>(p.d, p.dbs, p.drs, b, st.js - 1), split * kSplit, p.V, threadIdx.x);
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) acc += draw_mass(tc.get(e), dc.get(e), c);
    acc = block_sum(acc, redd);
    if (threadIdx.x == 0) w.rsum[(long long)b * p.nsplit + split] = acc;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void sv_draw_kernel(Params p, Work w)
{
    __shared__ double s_mass[kMaxSplits];
    __shared__ double s_tsum[kThreads];
    __shared__ double s_wrel, s_prefix, s_Z, s_my;
    __shared__ int s_split, s_tstar, s_resid, s_y;
    const int b = blockIdx.x;
    const int K = p.K;
    const SeqState st = w.st[b];
    int kind = st.kind;
    int a = st.a;
    int y = -1;
    float zrep = NAN, py = NAN;

    if (kind == KIND_RESID || kind == KIND_BONUS) {
        if (threadIdx.x == 0) {
            bool resid = kind == KIND_RESID;
            double Z = 0.0;
            if (resid) {
                for (int k = 0; k < p.nsplit; ++k) {
                    s_mass[k] = w.rsum[(long long)b * p.nsplit + k];
                    Z += s_mass[k];
                }
                if (!(Z > 0.0)) resid = false; // cannot happen in exact arithmetic after a rejection
            }
            if (!resid) {
                // masses of p per split from the stream pass: s_k 2^((m_k - M) c) / S
                const long long pb = ((long long)st.e_final * 2) * p.nsplit;
                for (int k = 0; k < p.nsplit; ++k) {
                    const float m = w.part_m[pb + k];
                    s_mass[k] = m == -INFINITY ? 0.0 : w.part_s[pb + k] * exp2(((double)m - (double)st.Mt) * p.c64) / st.St;
                }
            }
            const double uf = (double)p.u[(long long)b * (K + 1) + K];
            const double target = resid ? uf * Z : uf;
            double C = 0.0, wrel = INFINITY;
            int ks = -1;
            for (int k = 0; k < p.nsplit; ++k) {
                const double Cn = C + s_mass[k];
                if (Cn > target) { ks = k; wrel = target - C; break; }
                C = Cn;
            }
            if (ks < 0) { // rounding: take the last token with mass
                for (int k = p.nsplit - 1; k >= 0; --k)
                    if (s_mass[k] > 0.0) { ks = k; break; }
                if (ks < 0) ks = 0;
                wrel = INFINITY;
            }
            s_split = ks;
            s_wrel = wrel;
            s_resid = resid ? 1 : 0;
            s_Z = kind == KIND_RESID ? (resid ? Z : 0.0) : 1.0;
        }
        __syncthreads();
        const bool resid = s_resid != 0;
        const DrawCtx c = make_ctx(st, p, resid);
        const void* trow = row_ptr<DT>(p.t, p.tbs, p.trs, b, st.js - 1);
        const void* drow = resid ? row_ptr<DT>(p.d, p.dbs, p.drs, b, st.js - 1) : nullptr;
        const int base = s_split * kSplit + threadIdx.x * kPerLane;
        const int end = min(base + kPerLane, p.V);
        double s = 0.0;
        int last_pos = -1;
        for (int i = base; i < end; ++i) {
            const double m = draw_mass(load_one<DT>(trow, i), resid ? load_one<DT>(drow, i) : 0.0f, c);
            s += m;
            if (m > 0.0) last_pos = i;
        }
        s_tsum[threadIdx.x] = s;
        __syncthreads();
        if (threadIdx.x == 0) {
            double P = 0.0, wrel = s_wrel;
            int ts = -1;
            for (int t = 0; t < kThreads; ++t) {
                if (P + s_tsum[t] > wrel) { ts = t; break; }
                P += s_tsum[t];
            }
            if (ts < 0) {
                wrel = INFINITY;
                P = 0.0;
                for (int t = kThreads - 1; t >= 0; --t)
                    if (s_tsum[t] > 0.0) { ts = t; break; }
                if (ts < 0) ts = 0;
                for (int t = 0; t < ts; ++t) P += s_tsum[t];
            }
            s_tstar = ts;
            s_prefix = P;
            s_wrel = wrel;
        }
        __syncthreads();
        if ((int)threadIdx.x == s_tstar) {
            const double P = s_prefix, wrel = s_wrel;
            double cl = 0.0, my;
            int yy = -1;
            if (wrel != INFINITY) {
                for (int i = base; i < end; ++i) {
                    const double m = draw_mass(load_one<DT>(trow, i), resid ? load_one<DT>(drow, i) : 0.0f, c);
                    cl += m;
                    if (P + cl > wrel) { yy = i; break; }
                }
            }
            if (yy < 0) yy = last_pos >= 0 ? last_pos : base;
            // the reported probability of the chosen token is always evaluated in fp64
            my = draw_mass_f64(load_one<DT>(trow, yy), resid ? load_one<DT>(drow, yy) : 0.0f, c);
            s_y = yy;
            s_my = my;
        }
        __syncthreads();
        y = s_y;
        zrep = (float)s_Z;
        py = (float)(kind == KIND_RESID && resid ? s_my / s_Z : s_my);
    } else if (kind == KIND_GREEDY) {
        y = st.y;
    } else {
        kind = KIND_BAD;
        a = 0;
        y = -1;
    }

    for (int jj = threadIdx.x; jj <= K; jj += kThreads) {
        int v = -1;
        if (y >= 0) v = jj < a ? p.tok[(long long)b * K + jj] : (jj == a ? y : -1);
        p.out_tok[(long long)b * (K + 1) + jj] = v;
    }
    if (threadIdx.x == 0) {
        p.acc_out[b] = a;
        p.vl_out[b] = st.L;
        if (p.zmass) p.zmass[b] = zrep;
        if (p.pys) p.pys[b] = py;
        if (b == 0 && p.status_out) *p.status_out = w.ctl[CTL_STATUS];
    }
}

// ---------------------------------------------------------------- host side

const char* const kKernelNames[K_COUNT] = {"sv_plan", "sv_stream", "sv_resid", "sv_draw"};

template <int DT, bool VEC, bool G>
const void* stream_fn() { return (const void*)sv_stream_kernel<DT, VEC, G>; }

} // namespace

struct spec_verify {
    spec_verify_config cfg;
    int nsplit;
    int cus;
    int occ[2][2];        // [vec][greedy] resident workgroups per CU of sv_stream
    void* ws;
    Work w;
    int timing_max, timing_n;
    hipEvent_t* ev;       // [timing_max][K_COUNT][2]
};

namespace {

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

int nsplit_of(int V) { return (V + kSplit - 1) / kSplit; }

bool args_vec_ok(const spec_verify_config* cfg, const spec_verify_args* a)
{
    const int es = cfg->dtype == SV_BF16 ? 2 : 4;
    const int per = 16 / es;
    if (cfg->vocab % per) return false;
    if ((uintptr_t)a->target_logits % 16) return false;
    if ((a->target_batch_stride * es) % 16 || (a->target_row_stride * es) % 16) return false;
    if (a->temperature > 0.0f) {
        if ((uintptr_t)a->draft_logits % 16) return false;
        if ((a->draft_batch_stride * es) % 16 || (a->draft_row_stride * es) % 16) return false;
    }
    return true;
}

struct DeviceGuard {
    int old = -1;
    explicit DeviceGuard(int dev)
    {
        if (hipGetDevice(&old) != hipSuccess) old = -1;
        if (old != dev) (void)hipSetDevice(dev);
    }
    ~DeviceGuard()
    {
        int cur = -1;
        if (old >= 0 && hipGetDevice(&cur) == hipSuccess && cur != old) (void)hipSetDevice(old);
    }
};

} // namespace

extern "C" {

const char* spec_verify_status_string(int status)
{
    switch (status) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument";
    case SV_ENOMEM: return "out of device memory";
    case SV_EDEVICE: return "HIP device or launch error";
    case SV_EUNSUPPORTED: return "unsupported configuration";
    default: return "unknown status";
    }
}

int32_t spec_verify_kernel_count(void) { return K_COUNT; }

const char* spec_verify_kernel_name(int32_t k) { return (k >= 0 && k < K_COUNT) ? kKernelNames[k] : ""; }

static int check_config(const spec_verify_config* cfg)
{
    if (!cfg) return SV_EINVAL;
    if (cfg->max_batch < 1 || cfg->max_batch > SV_MAX_BATCH) return SV_EINVAL;
    if (cfg->max_draft < 1 || cfg->max_draft > SV_MAX_DRAFT) return SV_EINVAL;
    if (cfg->vocab < 1 || cfg->vocab > SV_MAX_VOCAB) return SV_EINVAL;
    if (cfg->dtype != SV_F32 && cfg->dtype != SV_BF16) return SV_EUNSUPPORTED;
    if (cfg->device < 0) return SV_EINVAL;
    const long long items = (long long)cfg->max_batch * (cfg->max_draft + 1) * 2 * nsplit_of(cfg->vocab);
    if (items > (1ll << 30)) return SV_EUNSUPPORTED;
    return SV_OK;
}

int spec_verify_check(const spec_verify_config* cfg, const spec_verify_args* a)
{
    int rc = check_config(cfg);
    if (rc != SV_OK) return rc;
    if (!a) return SV_EINVAL;
    if (a->B < 0 || a->B > cfg->max_batch) return SV_EINVAL;
    if (a->K < 1 || a->K > cfg->max_draft) return SV_EINVAL;
    const float T = a->temperature;
    if (!(T >= 0.0f) || isinf(T)) return SV_EINVAL;
    if (a->length_mode != SV_LEN_FIXED && a->length_mode != SV_LEN_TAU) return SV_EINVAL;
    if (a->B == 0) return SV_OK;
    const int V = cfg->vocab;
    if (!a->target_logits || a->target_row_stride < V || a->target_batch_stride < 0) return SV_EINVAL;
    if (!a->draft_tokens) return SV_EINVAL;
    if (T > 0.0f) {
        if (!a->draft_logits || !a->uniforms) return SV_EINVAL;
        if (a->draft_row_stride < V || a->draft_batch_stride < 0) return SV_EINVAL;
    }
    if (a->length_mode == SV_LEN_TAU) {
        if (!a->tau) return SV_EINVAL;
        if (!a->confidence && !(T > 0.0f)) return SV_EINVAL; // max draft prob needs a draft distribution
    }
    if (!a->accepted_len || !a->out_tokens || !a->verify_len_out) return SV_EINVAL;
    return SV_OK;
}

int spec_verify_create(const spec_verify_config* cfg, spec_verify_t** out)
{
    if (!out) return SV_EINVAL;
    int rc = check_config(cfg);
    if (rc != SV_OK) return rc;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device >= ndev) return SV_EDEVICE;
    DeviceGuard guard(cfg->device);

    spec_verify* h = (spec_verify*)calloc(1, sizeof(spec_verify));
    if (!h) return SV_ENOMEM;
    h->cfg = *cfg;
    h->nsplit = nsplit_of(cfg->vocab);
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, cfg->device) != hipSuccess) { free(h); return SV_EDEVICE; }
    h->cus = prop.multiProcessorCount;
    for (int v = 0; v < 2; ++v)
        for (int g = 0; g < 2; ++g) {
            const void* fn;
            if (cfg->dtype == SV_BF16)
                fn = v ? (g ? stream_fn<SV_BF16, true, true>() : stream_fn<SV_BF16, true, false>())
                       : (g ? stream_fn<SV_BF16, false, true>() : stream_fn<SV_BF16, false, false>());
            else
                fn = v ? (g ? stream_fn<SV_F32, true, true>() : stream_fn<SV_F32, true, false>())
                       : (g ? stream_fn<SV_F32, false, true>() : stream_fn<SV_F32, false, false>());
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, 0) != hipSuccess || n < 1) n = 1;
            h->occ[v][g] = n;
        }

    const long long ne = (long long)cfg->max_batch * (cfg->max_draft + 1);
    const size_t ns = (size_t)h->nsplit;
    size_t off = 0;
    const size_t o_ctl = off; off = align_up(off + CTL_WORDS * sizeof(int));
    const size_t o_q = off; off = align_up(off + ne * sizeof(uint32_t));
    const size_t o_cnt = off; off = align_up(off + ne * sizeof(int));
    const size_t o_pm = off; off = align_up(off + ne * 2 * ns * sizeof(float));
    const size_t o_ps = off; off = align_up(off + ne * 2 * ns * sizeof(double));
    const size_t o_pi = off; off = align_up(off + ne * ns * sizeof(int));
    const size_t o_st = off; off = align_up(off + (size_t)cfg->max_batch * sizeof(SeqState));
    const size_t o_rs = off; off = align_up(off + (size_t)cfg->max_batch * ns * sizeof(double));
    if (hipMalloc(&h->ws, off) != hipSuccess) { free(h); return SV_ENOMEM; }
    char* base = (char*)h->ws;
    h->w.ctl = (int*)(base + o_ctl);
    h->w.queue = (uint32_t*)(base + o_q);
    h->w.cnt = (int*)(base + o_cnt);
    h->w.part_m = (float*)(base + o_pm);
    h->w.part_s = (double*)(base + o_ps);
    h->w.part_i = (int*)(base + o_pi);
    h->w.st = (SeqState*)(base + o_st);
    h->w.rsum = (double*)(base + o_rs);
    *out = h;
    return SV_OK;
}

int spec_verify_destroy(spec_verify_t* h)
{
    if (!h) return SV_OK;
    DeviceGuard guard(h->cfg.device);
    if (h->ev) {
        for (int i = 0; i < h->timing_max * K_COUNT * 2; ++i) (void)hipEventDestroy(h->ev[i]);
        free(h->ev);
    }
    int rc = hipFree(h->ws) == hipSuccess ? SV_OK : SV_EDEVICE;
    free(h);
    return rc;
}

int spec_verify_timing_begin(spec_verify_t* h, int32_t max_calls)
{
    if (!h || max_calls < 1 || max_calls > 100000 || h->ev) return SV_EINVAL;
    DeviceGuard guard(h->cfg.device);
    const int n = max_calls * K_COUNT * 2;
    h->ev = (hipEvent_t*)calloc((size_t)n, sizeof(hipEvent_t));
    if (!h->ev) return SV_ENOMEM;
    for (int i = 0; i < n; ++i)
        if (hipEventCreate(&h->ev[i]) != hipSuccess) {
            for (int k = 0; k < i; ++k) (void)hipEventDestroy(h->ev[k]);
            free(h->ev);
            h->ev = nullptr;
            return SV_EDEVICE;
        }
    h->timing_max = max_calls;
    h->timing_n = 0;
    return SV_OK;
}

int spec_verify_timing_end(spec_verify_t* h, double* ms, int32_t n_kernels, int32_t* n_runs)
{
    if (!h || !h->ev || !ms || n_kernels < 1) return SV_EINVAL;
    DeviceGuard guard(h->cfg.device);
    int rc = SV_OK;
    for (int k = 0; k < n_kernels; ++k) ms[k] = 0.0;
    for (int c = 0; c < h->timing_n; ++c)
        for (int k = 0; k < K_COUNT && k < n_kernels; ++k) {
            hipEvent_t e0 = h->ev[(c * K_COUNT + k) * 2], e1 = h->ev[(c * K_COUNT + k) * 2 + 1];
            float t = 0.0f;
            if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&t, e0, e1) != hipSuccess) {
                rc = SV_EDEVICE;
                continue;
            }
            ms[k] += t;
        }
    if (n_runs) *n_runs = h->timing_n;
    for (int i = 0; i < h->timing_max * K_COUNT * 2; ++i) (void)hipEventDestroy(h->ev[i]);
    free(h->ev);
    h->ev = nullptr;
    h->timing_max = h->timing_n = 0;
    return rc;
}

int spec_verify_run(spec_verify_t* h, const spec_verify_args* a, void* hip_stream)
{
    if (!h) return SV_EINVAL;
    int rc = spec_verify_check(&h->cfg, a);
    if (rc != SV_OK) return rc;
    if (a->B == 0) return SV_OK;
    DeviceGuard guard(h->cfg.device);
    hipStream_t s = (hipStream_t)hip_stream;

    const bool greedy = !(a->temperature > 0.0f);
    const bool vec = args_vec_ok(&h->cfg, a);
    Params p;
    memset(&p, 0, sizeof(p));
    p.B = a->B;
    p.K = a->K;
    p.V = h->cfg.vocab;
    p.nsplit = h->nsplit;
    p.ipe = greedy ? h->nsplit : 2 * h->nsplit;
    p.greedy = greedy;
    p.len_mode = a->length_mode;
    p.derived = (a->length_mode == SV_LEN_TAU && !a->confidence) ? 1 : 0;
    p.t = a->target_logits;
    p.tbs = a->target_batch_stride;
    p.trs = a->target_row_stride;
    p.d = a->draft_logits;
    p.dbs = a->draft_batch_stride;
    p.drs = a->draft_row_stride;
    p.tok = a->draft_tokens;
    p.u = a->uniforms;
    p.vl_in = a->length_mode == SV_LEN_FIXED ? a->verify_len_in : nullptr;
    p.conf = a->length_mode == SV_LEN_TAU ? a->confidence : nullptr;
    p.tau = a->length_mode == SV_LEN_TAU ? a->tau : nullptr;
    if (!greedy) {
        p.invT64 = 1.0 / (double)a->temperature;
        p.c64 = 1.4426950408889634073599246810019 / (double)a->temperature;
        float hi = (float)p.c64;
        if ((double)hi > p.c64) hi = nextafterf(hi, 0.0f);
        float lo = (float)(p.c64 - (double)hi);
        if (!(lo > 1e-37f)) lo = 1e-37f;
        p.c_hi = hi;
        p.c_lo = lo;
    }
    p.acc_out = a->accepted_len;
    p.out_tok = a->out_tokens;
    p.vl_out = a->verify_len_out;
    p.lse_t = a->lse_target;
    p.lse_d = a->lse_draft;
    p.surv = a->survival;
    p.zmass = a->residual_mass;
    p.pys = a->sampled_prob;
    p.status_out = a->device_status;

    const bool timing = h->ev && h->timing_n < h->timing_max;
    auto mark = [&](int k, int which) {
        if (timing) (void)hipEventRecord(h->ev[(h->timing_n * K_COUNT + k) * 2 + which], s);
    };

    const long long ne = (long long)p.B * (p.K + 1);
    const long long items = ne * p.ipe;
    const int bf = h->cfg.dtype == SV_BF16;

    mark(K_PLAN, 0);
    hipLaunchKernelGGL(sv_plan_kernel, dim3((unsigned)((ne + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, p, h->w);
    mark(K_PLAN, 1);

    long long grid = (long long)h->occ[vec][greedy] * h->cus;
    if (grid > items) grid = items;
    if (grid < 1) grid = 1;
    mark(K_STREAM, 0);
#define SV_STREAM(DT, VEC, G) hipLaunchKernelGGL((sv_stream_kernel<DT, VEC, G>), dim3((unsigned)grid), dim3(kThreads), 0, s, p, h->w)
    if (bf) {
        if (vec) { if (greedy) SV_STREAM(SV_BF16, true, true); else SV_STREAM(SV_BF16, true, false); }
        else { if (greedy) SV_STREAM(SV_BF16, false, true); else SV_STREAM(SV_BF16, false, false); }
    } else {
        if (vec) { if (greedy) SV_STREAM(SV_F32, true, true); else SV_STREAM(SV_F32, true, false); }
        else { if (greedy) SV_STREAM(SV_F32, false, true); else SV_STREAM(SV_F32, false, false); }
    }
#undef SV_STREAM
    mark(K_STREAM, 1);

    mark(K_RESID, 0);
    if (!greedy) {
        const dim3 g((unsigned)((long long)p.B * p.nsplit));
        if (bf) {
            if (vec) hipLaunchKernelGGL((sv_resid_kernel<SV_BF16, true>), g, dim3(kThreads), 0, s, p, h->w);
            else hipLaunchKernelGGL((sv_resid_kernel<SV_BF16, false>), g, dim3(kThreads), 0, s, p, h->w);
        } else {
            if (vec) hipLaunchKernelGGL((sv_resid_kernel<SV_F32, true>), g, dim3(kThreads), 0, s, p, h->w);
            else hipLaunchKernelGGL((sv_resid_kernel<SV_F32, false>), g, dim3(kThreads), 0, s, p, h->w);
        }
    }
    mark(K_RESID, 1);

    mark(K_DRAW, 0);
    if (bf) hipLaunchKernelGGL((sv_draw_kernel<SV_BF16>), dim3((unsigned)p.B), dim3(kThreads), 0, s, p, h->w);
    else hipLaunchKernelGGL((sv_draw_kernel<SV_F32>), dim3((unsigned)p.B), dim3(kThreads), 0, s, p, h->w);
    mark(K_DRAW, 1);
    if (timing) h->timing_n++;

    return hipGetLastError() == hipSuccess ? SV_OK : SV_EDEVICE;
}

} // extern "C"
