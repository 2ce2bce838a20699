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
// Early exit.  The pages say generation restarts from the first error, so no
// row after the first rejection can change the output.  Positions are walked
// in groups (sizes 3, 3, 4, 8, 16, ... along the block); each group is two
// plain launches:
//   sv_rows    one workgroup per 16384-element split of every row the group
//              needs (target and draft rows of sequences still open), reduced
//              to (max, sum exp2) or (max, argmax) partials.  No atomics and no
//              fences: the kernel boundary publishes the partials.  The last
//              group from the fourth on, where few sequences are still open,
//              runs as sv_rows_late (eight candidate rows per workgroup).
//   sv_decide  one workgroup per open sequence: merges the partials of the
//              group's positions in fp64 and walks them in order -- survival
//              and verify length, the acceptance test u < p/q (or the greedy
//              match) -- until the first rejection, the bonus row, or the end of
//              the group.
// Rows inside a group past a rejection are read speculatively (they lie within
// the verify window).  Synchronising only at kernel boundaries keeps every
// launch a pure stream: an agent-scope fence costs ~130 ns, serialised, on
// this chip, so work is never handed between workgroups inside a launch.
//
// When the step samples with draft probabilities, the last group has no
// sv_decide launch: sv_resid takes those decisions at its start.
//
// After the last group:
//   sv_resid   per (sequence, split, half split): the last group's decisions
//              (every workgroup of a sequence derives them; one writes them),
//              then for a rejecting sequence the segment sums of
//              max(0, p - q) over the rejected row pair.  (One-hot drafts have
//              no residual pass: sv_draw forms p without x itself.)
//   sv_draw    per sequence: inverse-CDF draw (replacement or bonus) by split
//              and segment prefix in fp64, then one segment's tokens scanned
//              in token order; writes the outputs.
// sv_plan (first) sets up per-sequence state and the verify length where it
// is known without reading logits.
//
// Numerics.  bf16 and fp32 inputs are exact in fp32.  The row statistics take
// one fma per element, l*c - round(m*c) with c = log2(e)/T in fp32, and keep
// the exact rounding error of m*c beside the split sum for the fp64 merges;
// the final draw forms a = (l - m) * log2(e)/T with the constant split in two
// fp32 parts and scales by the rows' 1/S in two fp32 parts (no systematic scale
// bias, which would not cancel in p - q).  v_exp_f32 measured on MI355X:
// < 0.8 ulp for arguments >= -12.  Sums run in fp32 over 8 elements and in
// fp64 beyond, so a row sum carries ~1e-8 relative error.
// Decisions (acceptance ratio, survival product, CDF prefix) are taken in fp64.
// The final draw evaluates large masses (> 2^-9) in fp64.
//
// Determinism.  Split boundaries depend only on V, every reduction has a fixed
// order and there are no floating-point atomics, so outputs are bitwise
// reproducible and independent of a sequence's batch position and of B.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;                     // 4 wavefronts of 64
constexpr int kWaves = kThreads / 64;
constexpr int kSplit = 16384;                     // elements per split (fixed for batch invariance)
constexpr int kPerLane = kSplit / kThreads;       // 64 elements per lane per split
constexpr int kMaxGroup = 16;                     // positions per group
constexpr int kMaxGroups = 64;                    // groups per step (K + 1 <= 2 + 2 + 4 + 8 + 16 * 59)

enum { CTL_STATUS = 0, CTL_SCHED_STATUS = 1, CTL_CONF_STATUS = 2, CTL_WORDS = 64 };
enum { FL_ACC = 1, FL_LEN = 2 };
// Compile-time variants of the step kernels: MODE_ONEHOT (q is the point mass
// at the drafted token; never with greedy verification) and MODE_PACKED (rows
// addressed through per-sequence offsets).
enum { MODE_ONEHOT = 1, MODE_PACKED = 2 };
enum { KIND_NONE = -1, KIND_RESID = 0, KIND_BONUS = 1, KIND_GREEDY = 2, KIND_BAD = 3 };
enum { K_PLAN = 0, K_ROWS = 1, K_DECIDE = 2, K_RESID = 3, K_DRAW = 4, K_COUNT = 5 };

struct SeqState {
    double S;      // survival product S_j of the positions evaluated so far
    double St, Sd; // sums of exp2((l - M) c) of the rows of the final draw
    float Mt, Md;  // maxima of those rows
    int L;         // verify length, -1 while undetermined
    int a;         // accepted positions so far
    int flags;     // FL_ACC: acceptance walk open; FL_LEN: verify-length walk open
    int kind;      // KIND_*
    int js;        // 1-based row of the final draw
    int y;         // token chosen by the walk (greedy)
    int rows;      // logit rows streamed for this sequence
    int pad;
};

struct Work {
    int* ctl;
    float* part_m;    // [B][2K+1][nsplit] split maxima; row j-1 target, K+j draft (j 1-based)
    double* part_s;   // same layout, split sums of exp2((l - m) c + d)
    float* part_d;    // same layout, the d of that sum (the true split sum is part_s * 2^-d)
    int* part_i;      // same layout, split argmax (greedy)
    SeqState* st;     // [max_batch]
    SeqState* fin;    // [max_batch] state after the last group, stored by sv_resid (which takes its decisions)
    int* live;        // [max_batch] (L + 1) << 2 | flags, the part of st that sv_rows reads
    double* seg;      // [max_batch][nsplit][64] residual mass per segment of a split
    float* xlog;      // [max_batch][2K+1] logit of the drafted token in each row
};

// Workspace of the admission and confidence calls (kept out of Work so that the
// verify kernels' arguments stay small).
struct AuxWork {
    int* ctl;
    double* sched_s;      // [B][K] survivals of the admission scheduler
    int* sched_rank;      // [B][K] rank of each drafted position by survival
    double* sched_sorted; // [B K] survivals in rank order
    float* conf_ring;     // [max_batch][SV_MAX_CONF_DELAY][max_draft] calibrated confidences of past calls
    int* conf_head;       // [max_batch] ring slot of the next call
    int* conf_count;      // [max_batch] calls recorded since the slot's reset (capped)
    int conf_K;           // max_draft: the ring's row length
};

struct Params {
    int B, K, V, nsplit, seg_w;   // seg_w: the power of two >= nsplit
    int greedy, derived;       // derived: tau mode with c = max draft probability
    int onehot;                // q_j is the point mass at x_j; no draft row is streamed
    const long long* toff;     // packed rows: target rows of sequence b start at row toff[b] (NULL: dense)
    const long long* doff;     // packed rows: draft rows of sequence b start at row doff[b]
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
    float c32;                 // c64 rounded to nearest
    int* acc_out;
    int* out_tok;
    int* vl_out;
    float* lse_t;
    float* lse_d;
    float* surv;
    float* zmass;
    float* pys;
    int* rows_out;
    int* status_out;
};

__device__ __forceinline__ void or_status(int* p, int v) { __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

__device__ __forceinline__ long long part_index(const Params& p, int b, int row)
{
    return ((long long)b * (2 * p.K + 1) + row) * p.nsplit;
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

// Workgroup barrier that orders LDS only: global loads issued before it may
// stay in flight (so the next split can be prefetched across a reduction).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup reductions over kThreads threads; t is the thread's index.
__device__ __forceinline__ float block_max(float v, float* red, int t = threadIdx.x)
{
    v = wave_max(v);
    const int w = t >> 6;
    if ((t & 63) == 0) red[w] = v;
    lds_barrier();
    float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    lds_barrier();
    return r;
}

__device__ __forceinline__ double block_sum(double v, double* red, int t = threadIdx.x)
{
    v = wave_sum(v);
    const int w = t >> 6;
    if ((t & 63) == 0) red[w] = v;
    lds_barrier();
    double r = ((red[0] + red[1]) + red[2]) + red[3];
    lds_barrier();
    return r;
}

__device__ __forceinline__ void block_argmax(float& v, int& i, float* redf, int* redi, int t = threadIdx.x)
{
    wave_argmax(v, i);
    const int w = t >> 6;
    if ((t & 63) == 0) { redf[w] = v; redi[w] = i; }
    lds_barrier();
    v = redf[0];
    i = redi[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k)
        if (redf[k] > v || (redf[k] == v && redi[k] < i)) { v = redf[k]; i = redi[k]; }
    lds_barrier();
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

// 16-byte load of streamed logits, marked non-temporal: the row statistics read
// each row once per step and the residual pass reads the rejected row pairs
// once, so their lines are not kept in the caches (measured: 23 us less per
// verify step at B=256 K=16 V=129280 bf16, the row statistics at 5.5 TB/s
// instead of 4.9).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 load16_stream(const void* p) { return __builtin_nontemporal_load((const u32x4*)p); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int DT>
struct Chunk;

template <>
struct Chunk<SV_BF16> {
    uint32_t w[kPerLane / 2];
    __device__ __forceinline__ float get(int e) const { return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]); }
    __device__ __forceinline__ static int index(int base, int lane, int e) { return base + (e >> 3) * 2048 + lane * 8 + (e & 7); }
    // lane and element holding offset off (0 <= off < kSplit) of the split
    __device__ __forceinline__ static void owner(int off, int& lane, int& e) { lane = (off >> 3) & 255; e = (off >> 11) * 8 + (off & 7); }
    // the one-hot draft row: -inf everywhere, 0 at element e of this lane (e < 0: none)
    __device__ __forceinline__ void one_hot(int e)
    {
#pragma unroll
        for (int k = 0; k < kPerLane / 2; ++k) {
            const uint32_t lo = 2 * k == e ? 0x0000u : 0xFF80u, hi = 2 * k + 1 == e ? 0x0000u : 0xFF80u;
            w[k] = lo | (hi << 16);
        }
    }
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
    // Same data as load(), with every vector load issued unconditionally (the
    // address of a vector past V is clamped to the row's last vector) so that
    // the number of loads in flight is fixed and a later chunk's loads need not
    // be waited for; fix_tail() then sets the vectors past V to -inf.
    template <bool VEC>
    __device__ __forceinline__ void issue(const void* row, int base, int V, int lane)
    {
        if (!VEC) {
            load<false>(row, base, V, lane);
            return;
        }
        const uint16_t* r = (const uint16_t*)row;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i0 = base + k * 2048 + lane * 8;
            const u32x4 q = load16_stream(r + (i0 < V ? i0 : V - 8));
            w[4 * k] = q.x; w[4 * k + 1] = q.y; w[4 * k + 2] = q.z; w[4 * k + 3] = q.w;
        }
    }
    template <bool VEC>
    __device__ __forceinline__ void fix_tail(int base, int V, int lane)
    {
        if (!VEC || base + kSplit <= V) return;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (base + k * 2048 + lane * 8 >= V) w[4 * k] = w[4 * k + 1] = w[4 * k + 2] = w[4 * k + 3] = 0xFF80FF80u;
    }
};

template <>
struct Chunk<SV_F32> {
    float w[kPerLane];
    __device__ __forceinline__ float get(int e) const { return w[e]; }
    __device__ __forceinline__ static int index(int base, int lane, int e) { return base + (e >> 2) * 1024 + lane * 4 + (e & 3); }
    __device__ __forceinline__ static void owner(int off, int& lane, int& e) { lane = (off >> 2) & 255; e = (off >> 10) * 4 + (off & 3); }
    __device__ __forceinline__ void one_hot(int e)
    {
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) w[k] = k == e ? 0.0f : -INFINITY;
    }
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
    template <bool VEC>
    __device__ __forceinline__ void issue(const void* row, int base, int V, int lane)
    {
        if (!VEC) {
            load<false>(row, base, V, lane);
            return;
        }
        const float* r = (const float*)row;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int i0 = base + k * 1024 + lane * 4;
            const u32x4 q = load16_stream(r + (i0 < V ? i0 : V - 4));
            w[4 * k] = __uint_as_float(q.x); w[4 * k + 1] = __uint_as_float(q.y);
            w[4 * k + 2] = __uint_as_float(q.z); w[4 * k + 3] = __uint_as_float(q.w);
        }
    }
    template <bool VEC>
    __device__ __forceinline__ void fix_tail(int base, int V, int lane)
    {
        if (!VEC || base + kSplit <= V) return;
#pragma unroll
        for (int k = 0; k < 16; ++k)
            if (base + k * 1024 + lane * 4 >= V) w[4 * k] = w[4 * k + 1] = w[4 * k + 2] = w[4 * k + 3] = -INFINITY;
    }
};

// A part of a split (one of kParts): loads q NL .. q NL + NL - 1 of the
// split layout above, kPerLane / kParts elements per lane.  Element e of the
// part is element q PER + e of the lane's split elements.
constexpr int kParts = 2;

template <int DT>
struct Part;

template <>
struct Part<SV_BF16> {
    static constexpr int NL = 8 / kParts, PER = 8 * NL;
    uint32_t w[PER / 2];
    __device__ __forceinline__ float get(int e) const { return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]); }
    template <bool VEC>
    __device__ __forceinline__ void load(const void* row, int base, int V, int lane, int q)
    {
        const uint16_t* r = (const uint16_t*)row;
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int i0 = base + (q * NL + k) * 2048 + lane * 8;
            if (VEC) {
                if (i0 < V) {
                    const u32x4 v = load16_stream(r + i0);
                    w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
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
struct Part<SV_F32> {
    static constexpr int NL = 16 / kParts, PER = 4 * NL;
    float w[PER];
    __device__ __forceinline__ float get(int e) const { return w[e]; }
    template <bool VEC>
    __device__ __forceinline__ void load(const void* row, int base, int V, int lane, int q)
    {
        const float* r = (const float*)row;
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int i0 = base + (q * NL + k) * 1024 + lane * 4;
            if (VEC) {
                if (i0 < V) {
                    const u32x4 v = load16_stream(r + i0);
                    w[4 * k] = __uint_as_float(v.x); w[4 * k + 1] = __uint_as_float(v.y);
                    w[4 * k + 2] = __uint_as_float(v.z); w[4 * k + 3] = __uint_as_float(v.w);
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

// Row j (0-based) of sequence b, dense ([B][rows][V] by strides) or packed
// (the sequence's rows start at row off[b] of a [sum of rows][V] tensor).
template <int DT, bool PK>
__device__ __forceinline__ const void* seq_row(const void* base, const long long* off, long long bs, long long rs, int b,
                                               int j)
{
    if (PK) {
        typedef const __attribute__((address_space(4))) long long* cptr;
        const long long r = ((cptr)off)[b] + j; // uniform: a scalar load
        return (const void*)((const char*)base + r * rs * (DT == SV_BF16 ? 2 : 4));
    }
    return row_ptr<DT>(base, bs, rs, b, j);
}

// exp2((l - m) * c) with c = c_hi + c_lo; exact subtraction for bf16 inputs,
// no bias from rounding c.  l = -inf gives 0 (c_lo > 0 keeps the product -inf).
__device__ __forceinline__ float scaled_exp2(float l, float m, float c_hi, float c_lo)
{
    const float t = l - m;
    return __builtin_amdgcn_exp2f(fmaf(t, c_hi, t * c_lo));
}

// 2^a in fp64: a = n + f with n = rint(a), |f| <= 1/2, and e^(f ln 2) from its
// Taylor series to the x^11 term (|x| <= 0.347, truncation below 1e-14
// relative), scaled by 2^n.  -inf and very negative a give 0; NaN passes.
__device__ __forceinline__ double exp2_f64(double a)
{
    if (!(a > -1100.0)) return a != a ? a : 0.0;
    if (a > 1100.0) return INFINITY;
    const double n = rint(a);
    const double x = (a - n) * 0.69314718055994530942;
    double r = 2.505210838544171877505e-08;    // 1/11!
    r = fma(r, x, 2.755731922398589065256e-07); // 1/10!
    r = fma(r, x, 2.755731922398589065256e-06); // 1/9!
    r = fma(r, x, 2.480158730158730158730e-05); // 1/8!
    r = fma(r, x, 1.984126984126984126984e-04); // 1/7!
    r = fma(r, x, 1.388888888888888888889e-03); // 1/6!
    r = fma(r, x, 8.333333333333333333333e-03); // 1/5!
    r = fma(r, x, 4.166666666666666666667e-02); // 1/4!
    r = fma(r, x, 1.666666666666666666667e-01); // 1/3!
    r = fma(r, x, 0.5);
    r = fma(r, x, 1.0);
    r = fma(r, x, 1.0);
    return ldexp(r, (int)n);
}

// (max, sum exp) of one loaded split: sum in fp32 over runs of 8 elements, fp64 beyond.
// The exponent of each term is one fma, l*c - mc with mc = m*c rounded; the
// rounding error d = m*c - mc is exact in fp32, every term carries the factor
// 2^d (|d| <= 2^-5), and d is returned beside the sum for the consumers to take
// out in fp64.  The only bias left is that of c rounded to fp32 (relative
// 2^-24 of the exponent).  Rows with |m*c| >= 2^20 take the exact-difference
// form (d = 0).
//
// bf16: the sum pass widens the packed words again with byte permutes rather
// than reusing the max pass's shifts, so the 64 widened values are never live
// at once (registers are what bound the loads in flight).
__device__ __forceinline__ float bf16_lo_perm(uint32_t w) { return __uint_as_float(__builtin_amdgcn_perm(w, 0u, 0x05040c0cu)); }
__device__ __forceinline__ float bf16_hi_perm(uint32_t w) { return __uint_as_float(__builtin_amdgcn_perm(w, 0u, 0x07060c0cu)); }

template <int DT>
__device__ __forceinline__ float chunk_elem_sum(const Chunk<DT>& c, int e)
{
    if (DT == SV_BF16) return (e & 1) ? bf16_hi_perm(((const uint32_t*)&c)[e >> 1]) : bf16_lo_perm(((const uint32_t*)&c)[e >> 1]);
    return c.get(e);
}

template <int DT>
__device__ __forceinline__ void chunk_stats(const Chunk<DT>& c, float c32, float c_hi, float c_lo, float& M,
                                            double& S, float& D, float* redf, double* redd, int t)
{
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) m = fmaxf(m, c.get(e));
    m = block_max(m, redf, t);
    double acc = 0.0;
    float d = 0.0f;
    if (m != -INFINITY) {
        const float mc = m * c32;
        if (fabsf(mc) < 0x1p20f) {
            d = fmaf(m, c32, -mc);
#pragma unroll
            for (int r = 0; r < kPerLane / 8; ++r) {
                float run = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) run += __builtin_amdgcn_exp2f(fmaf(chunk_elem_sum<DT>(c, 8 * r + i), c32, -mc));
                acc += (double)run;
                __builtin_amdgcn_sched_barrier(0); // widen one run at a time
            }
        } else {
#pragma unroll
            for (int r = 0; r < kPerLane / 8; ++r) {
                float run = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) run += scaled_exp2(chunk_elem_sum<DT>(c, 8 * r + i), m, c_hi, c_lo);
                acc += (double)run;
            }
        }
    }
    S = block_sum(acc, redd, t);
    D = d;
    M = m;
}

// (max, lowest index of the max) of one loaded split of the raw row.
template <int DT>
__device__ __forceinline__ void chunk_argmax(const Chunk<DT>& c, int V, int split, float& M, int& I, float* redf,
                                             int* redi, int t)
{
    float best = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
        const float v = c.get(e);
        const int idx = Chunk<DT>::index(split * kSplit, t, e);
        if (idx < V && (v > best || bi == 0x7fffffff)) { best = v; bi = idx; }
    }
    block_argmax(best, bi, redf, redi, t);
    M = best;
    I = bi;
}

// ---------------------------------------------------------------- sv_plan

__global__ __launch_bounds__(kThreads) void sv_plan_kernel(Params p, Work w)
{
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
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
    st.rows = 0;
    st.pad = 0;
    bool bad = false, len_open = false;
    int L;
    if (p.toff) {
        // packed rows: the sequence brings L + 1 target rows (and L draft rows)
        const long long nt = p.toff[b + 1] - p.toff[b];
        L = (int)(nt - 1);
        if (nt < 1 || nt > K + 1) bad = true;
        if (p.doff && p.doff[b + 1] - p.doff[b] != nt - 1) bad = true;
    } else if (p.len_mode == SV_LEN_FIXED) {
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
        else if (tau <= 0.0f || p.onehot) L = K; // one-hot drafts: c_j = 1
        else { L = -1; len_open = true; }
        if (p.onehot && p.surv)
            for (int j = 0; j < K; ++j) p.surv[(long long)b * K + j] = 1.0f;
    }
    st.L = L;
    if (bad) {
        st.kind = KIND_BAD;
        st.flags = 0;
        or_status(&w.ctl[CTL_STATUS], SV_STATUS_BAD_INPUT);
    } else {
        st.flags = FL_ACC | (len_open ? FL_LEN : 0);
    }
    w.st[b] = st;
    w.live[b] = st.flags ? (((st.L + 1) << 2) | st.flags) : 0;
}

// ---------------------------------------------------------------- sv_rows
//
// Which rows of a group are streamed, from the state at the start of the group:
//   target row j  iff the acceptance walk is open and (L unknown or j <= L+1)
//   draft row j   iff j <= K and (the length walk is open, or the acceptance
//                 walk is open and j <= L)
// sv_decide uses the same state, so every row its walk touches was streamed.

__device__ __forceinline__ bool target_row_needed(int flags, int L, int j, int K)
{
    return (flags & FL_ACC) && j <= K + 1 && (L < 0 || j <= L + 1);
}

__device__ __forceinline__ bool draft_row_needed(int flags, int L, int j, int K)
{
    return j <= K && ((flags & FL_LEN) || ((flags & FL_ACC) && j <= L));
}

// One split of one needed row: (max, sum exp2) or (max, argmax) partials, and
// the drafted token's logit when the split holds it.
struct RowRef {
    const void* row;
    int b, j, prow, split;
};

template <int DT, bool PK>
__device__ __forceinline__ RowRef row_ref(const Params& p, int b, int j, bool draft, int split)
{
    RowRef r;
    r.row = draft ? seq_row<DT, PK>(p.d, p.doff, p.dbs, p.drs, b, j - 1)
                  : seq_row<DT, PK>(p.t, p.toff, p.tbs, p.trs, b, j - 1);
    r.b = b;
    r.j = j;
    r.prow = draft ? p.K + j : j - 1;
    r.split = split;
    return r;
}

// t: thread index inside the workgroup.
template <int DT, bool GREEDY>
__device__ __forceinline__ void rows_finish(const Params& p, const Work& w, const Chunk<DT>& c, const RowRef& r,
                                            float* redf, double* redd, int* redi, int t)
{
    const long long pi = part_index(p, r.b, r.prow) + r.split;
    if (GREEDY) {
        float M;
        int I;
        chunk_argmax<DT>(c, p.V, r.split, M, I, redf, redi, t);
        if (t == 0) {
            w.part_m[pi] = M;
            w.part_i[pi] = I;
        }
    } else {
        // the drafted token of this position and its logit in this row, when
        // the split holds it: r.b, r.j and x are uniform, so both come through
        // scalar loads (the token ids and logits are never written here)
        if (r.j <= p.K) {
            typedef const __attribute__((address_space(4))) uint32_t* cptr;
            const int x = (int)((cptr)p.tok)[(long long)r.b * p.K + (r.j - 1)];
            const int off = x - r.split * kSplit;
            if (x >= 0 && x < p.V && off >= 0 && off < kSplit) {
                float xl;
                if (DT == SV_BF16) {
                    // the aligned word holding element x lies in the same page
                    const uintptr_t a = (uintptr_t)r.row + 2 * (uintptr_t)x;
                    const uint32_t word = *(cptr)(a & ~(uintptr_t)3);
                    xl = (a & 2) ? bf16_hi(word) : bf16_lo(word);
                } else {
                    xl = __uint_as_float(((cptr)r.row)[x]);
                }
                if (t == 0) w.xlog[(long long)r.b * (2 * p.K + 1) + r.prow] = xl;
            }
        }
        float M, D;
        double S;
        chunk_stats<DT>(c, p.c32, p.c_hi, p.c_lo, M, S, D, redf, redd, t);
        if (t == 0) {
            w.part_m[pi] = M;
            w.part_s[pi] = S;
            w.part_d[pi] = D;
        }
    }
}

// One workgroup per (sequence, row slot, split), split fastest, so that
// consecutive workgroups stream consecutive 32 KB pieces of a row (HBM keeps
// its rate on long contiguous runs).  A workgroup of a row the walk does not
// need exits after one scalar load.
template <int DT, bool VEC, bool GREEDY, int MODE>
__global__ __launch_bounds__(kThreads, (DT == SV_BF16 && VEC) ? 8 : 1) void sv_rows_kernel(Params p, Work w, int j0,
                                                                                           int G)
{
    constexpr bool OH = (MODE & MODE_ONEHOT) != 0, PK = (MODE & MODE_PACKED) != 0;
    __shared__ float redf[kWaves];
    __shared__ double redd[kWaves];
    __shared__ int redi[kWaves];
    const int t = (int)threadIdx.x;
    const int split = (int)(blockIdx.x % (unsigned)p.nsplit);
    const int rest = (int)(blockIdx.x / (unsigned)p.nsplit);
    const int slots = (GREEDY || OH) ? G : 2 * G; // one-hot drafts: target rows only
    const int slot = rest % slots;
    const int b = rest / slots;
    const bool draft = !GREEDY && slot >= G;
    const int j = j0 + (draft ? slot - G : slot);
    typedef const __attribute__((address_space(4))) int* cptr;
    const int lv = ((cptr)w.live)[b];
    const int flags = lv & 3, L = (lv >> 2) - 1;
    const bool need = draft ? draft_row_needed(flags, L, j, p.K) : target_row_needed(flags, L, j, p.K);
    if (!need) return;
    const RowRef r = row_ref<DT, PK>(p, b, j, draft, split);
    Chunk<DT> c;
    c.template issue<VEC>(r.row, split * kSplit, p.V, t);
    c.template fix_tail<VEC>(split * kSplit, p.V, t);
    rows_finish<DT, GREEDY>(p, w, c, r, redf, redd, redi, t);
}

// The same statistics for the last position group from the fourth group on,
// where the walks of most sequences have ended (typically a few in a hundred
// are still open) and one workgroup per row would mostly start only to find
// its row unneeded.  The group's rows (sequence, row slot) are dealt to nw =
// gridDim.x / nsplit workgroup columns: column c takes rows c, c + nw, ...,
// kRowsLate of them.  Lanes 0 .. kRowsLate-1 read those sequences' states at
// once, and the workgroup streams the needed ones in turn.  Each turn is a
// separate straight-line copy of the row code (a schedule barrier between
// copies, the thread index re-derived in each) so that the copies neither
// share registers nor overlap: registers bound the loads in flight.
// (8 measured best for the last group at 4% of sequences open; 2 or 4 rows per
// workgroup lost on a group with a quarter of them open, as one row per
// workgroup then keeps more rows in flight.)
constexpr int kRowsLate = 8;

template <int DT, bool VEC, bool GREEDY, int MODE>
__global__ __launch_bounds__(kThreads, (DT == SV_BF16 && VEC) ? 8 : 1) void sv_rows_late_kernel(Params p, Work w,
                                                                                                int j0, int G)
{
    constexpr bool OH = (MODE & MODE_ONEHOT) != 0, PK = (MODE & MODE_PACKED) != 0;
    __shared__ float redf[kWaves];
    __shared__ double redd[kWaves];
    __shared__ int redi[kWaves];
    const int t = (int)threadIdx.x, lane = t & 63;
    const int split = (int)(blockIdx.x % (unsigned)p.nsplit);
    const int col = (int)(blockIdx.x / (unsigned)p.nsplit);
    const int nw = (int)(gridDim.x / (unsigned)p.nsplit);
    const int slots = (GREEDY || OH) ? G : 2 * G;
    const int nrow = p.B * slots;
    bool need = false;
    if (lane < kRowsLate) {
        const int i = col + lane * nw;
        if (i < nrow) {
            const int b = i / slots, slot = i % slots;
            const int lv = w.live[b];
            const int flags = lv & 3, L = (lv >> 2) - 1;
            const bool draft = !GREEDY && slot >= G;
            const int j = j0 + (draft ? slot - G : slot);
            need = draft ? draft_row_needed(flags, L, j, p.K) : target_row_needed(flags, L, j, p.K);
        }
    }
    const unsigned long long mask = __ballot(need); // the same in every wavefront
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
#pragma unroll
    for (int k = 0; k < kRowsLate; ++k) {
        __builtin_amdgcn_sched_barrier(0);
        if ((mask >> k) & 1) {
            const int i = col + k * nw;
            const int b = i / slots, slot = i % slots;
            const bool draft = !GREEDY && slot >= G;
            const int j = j0 + (draft ? slot - G : slot);
            int z = 0;
            asm volatile("" : "+v"(z)); // opaque: the index below is computed afresh in this copy
            const int tl = (wv << 6) | (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, (unsigned)z));
            const RowRef r = row_ref<DT, PK>(p, b, j, draft, split);
            Chunk<DT> c;
            c.template issue<VEC>(r.row, split * kSplit, p.V, tl);
            c.template fix_tail<VEC>(split * kSplit, p.V, tl);
            rows_finish<DT, GREEDY>(p, w, c, r, redf, redd, redi, tl);
        }
    }
}

// ---------------------------------------------------------------- sv_decide
//
// One workgroup per sequence.  Threads take (position, row, split) triples and
// merge the split partials with fixed-order shuffles inside groups of sw lanes
// (sw = the power of two >= nsplit), so every partial of the group is loaded in
// one round trip; other threads gather the drafted tokens' logits.  Thread 0
// then walks the positions in order.

__device__ __forceinline__ float seg_max(float v, int sw)
{
    for (int o = sw >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ double seg_sum(double v, int sw)
{
    for (int o = sw >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ void seg_argmax(float& v, int& i, int sw)
{
    for (int o = sw >> 1; o > 0; o >>= 1) {
        const float ov = __shfl_xor(v, o);
        const int oi = __shfl_xor(i, o);
        if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
    }
}

struct DecideSmem {
    float sMt[kMaxGroup], sMd[kMaxGroup], sLt[kMaxGroup], sLd[kMaxGroup];
    double sSt[kMaxGroup], sSd[kMaxGroup];
    int sG[kMaxGroup];
    double sRatio[kMaxGroup];
    float sLseT[kMaxGroup], sLseD[kMaxGroup];
    int sTok[kMaxGroup];
    float sU[kMaxGroup];
    SeqState st;
};

// The decisions of sequence b over positions j0 .. j0+G-1, from the state
// before the group (w.st); every thread of the workgroup calls it and gets the
// state after the group, which the caller stores.  writer: this workgroup
// writes the decisions' outputs (lse and survival rows, status bits); other
// callers only learn the result.
template <int DT, bool GREEDY, int MODE>
__device__ SeqState decide_group(const Params& p, const Work& w, int b, int j0, int G, bool writer, DecideSmem& sm)
{
    constexpr bool OH = (MODE & MODE_ONEHOT) != 0;
    float* const sMt = sm.sMt;
    float* const sMd = sm.sMd;
    float* const sLt = sm.sLt;
    float* const sLd = sm.sLd;
    double* const sSt = sm.sSt;
    double* const sSd = sm.sSd;
    int* const sG = sm.sG;
    double* const sRatio = sm.sRatio;
    float* const sLseT = sm.sLseT;
    float* const sLseD = sm.sLseD;
    int* const sTok = sm.sTok;
    float* const sU = sm.sU;
    const int tid = threadIdx.x, K = p.K;
    const int n = min(j0 + G - 1, K + 1) - j0 + 1;
    const int sw = p.seg_w;
    const int per = 2 * n * sw;
    // Everything the group's decisions read is requested at once: the state,
    // the split partials of every row of the group, the drafted tokens' logits,
    // tokens and uniforms.  Their addresses depend on the group only (rows that
    // were not streamed are loaded too and masked below), so one round trip
    // serves them all.
    const SeqState st0 = w.st[b];
    float pm = -INFINITY, pd = 0.0f;
    double ps = 0.0;
    int pix = 0x7fffffff;
    if (tid < per && per <= kThreads) {
        const int pk = tid / sw, k = tid % sw, q = pk >> 1, kind = pk & 1, j = j0 + q;
        if (k < p.nsplit && (kind == 0 || (!GREEDY && !OH && j <= K))) {
            const long long pi = part_index(p, b, kind ? K + j : j - 1) + k;
            pm = w.part_m[pi];
            if (GREEDY) {
                pix = w.part_i[pi];
            } else {
                ps = w.part_s[pi];
                pd = w.part_d[pi];
            }
        }
    }
    float xl = 0.0f;
    {
        const int q = tid & 63, kind = tid >> 6, j = j0 + q;
        if (!GREEDY && kind < 2 && q < n && j <= K && !(kind && OH))
            xl = w.xlog[(long long)b * (2 * K + 1) + (kind ? K + j : j - 1)];
        if (kind == 2 && q < n && j <= K) {
            sTok[q] = p.tok[(long long)b * K + (j - 1)];
            if (!GREEDY) sU[q] = p.u[(long long)b * (K + 1) + (j - 1)];
        }
    }
    const float tau_b = (!GREEDY && p.derived) ? p.tau[b] : 0.0f;
    const int flags0 = st0.flags, L0 = st0.L;
    if (!(flags0 & (FL_ACC | FL_LEN))) return st0; // (the same in every thread)
    for (int base = 0; base < per; base += kThreads) {
        const int t = base + tid;
        const int pk = t / sw, k = t % sw;
        const int q = pk >> 1, kind = pk & 1, j = j0 + q;
        const bool read = t < per && (kind ? (!GREEDY && !OH && draft_row_needed(flags0, L0, j, K))
                                           : target_row_needed(flags0, L0, j, K));
        const bool has = read && k < p.nsplit;
        if (per > kThreads) {
            // groups wider than one workgroup's threads (very large vocabularies)
            const long long pi = has ? part_index(p, b, kind ? K + j : j - 1) + k : 0;
            pm = has ? w.part_m[pi] : -INFINITY;
            if (GREEDY) pix = has ? w.part_i[pi] : 0x7fffffff;
            else {
                ps = has ? w.part_s[pi] : 0.0;
                pd = has ? w.part_d[pi] : 0.0f;
            }
        }
        if (GREEDY) {
            float v = has ? pm : -INFINITY;
            int ix = has ? pix : 0x7fffffff;
            seg_argmax(v, ix, sw);
            if (read && k == 0) { sMt[q] = v; sG[q] = ix; }
        } else {
            const float m = has ? pm : -INFINITY;
            const float M = seg_max(m, sw);
            double v = (has && m != -INFINITY) ? ps * exp2_f64(((double)m - (double)M) * p.c64 - (double)pd) : 0.0;
            v = seg_sum(v, sw);
            if (read && k == 0) {
                if (kind) { sMd[q] = M; sSd[q] = v; }
                else { sMt[q] = M; sSt[q] = v; }
            }
        }
    }
    if (!GREEDY) {
        // logits of the drafted tokens, kept by sv_rows: threads 0..n-1 target rows, 64..64+n-1 draft rows
        const int q = tid & 63, kind = tid >> 6, j = j0 + q;
        if (kind < 2 && q < n && j <= K) {
            const bool read = kind ? draft_row_needed(flags0, L0, j, K) : target_row_needed(flags0, L0, j, K);
            if (read) {
                if (kind && OH) {
                    // the one-hot draft row: logit 0 at x, -inf elsewhere (max 0, sum 1)
                    sLd[q] = 0.0f;
                    sMd[q] = 0.0f;
                    sSd[q] = 1.0;
                } else if (kind) {
                    sLd[q] = xl;
                } else {
                    sLt[q] = xl;
                }
            }
        }
    }
    __syncthreads();
    if (!GREEDY) {
        // per-position quantities in parallel: the acceptance ratio p(x)/q(x), and the
        // rows' log-sum-exp when asked for (thread q handles position j0 + q)
        const int q = tid, j = j0 + q;
        if (q < n) {
            const bool tread = target_row_needed(flags0, L0, j, K);
            const bool dread = draft_row_needed(flags0, L0, j, K);
            if (tread && dread) {
                const float ld = sLd[q];
                double ratio = INFINITY; // q(x) = 0
                if (ld != -INFINITY) {
                    const double dlt = (double)sLt[q] - (double)sMt[q], dld = (double)ld - (double)sMd[q];
                    ratio = exp2_f64((dlt - dld) * p.c64) * (sSd[q] / sSt[q]);
                }
                sRatio[q] = ratio;
            }
            if (tread && p.lse_t) sLseT[q] = (float)((double)sMt[q] * p.invT64 + log(sSt[q]));
            if (dread && p.lse_d && !OH) sLseD[q] = (float)((double)sMd[q] * p.invT64 + log(sSd[q]));
        }
    }
    __syncthreads();
    if (tid == 0) {
    SeqState st = st0;
    bool acc = (flags0 & FL_ACC) != 0;
    bool len = (flags0 & FL_LEN) != 0;
    for (int q = 0; q < n; ++q) {
        const int j = j0 + q;
        const bool dread = !GREEDY && draft_row_needed(flags0, L0, j, K);
        st.rows += (target_row_needed(flags0, L0, j, K) ? 1 : 0) + ((dread && !OH) ? 1 : 0);
        if (!acc && !len) continue; // rows of this group past the stop were still streamed
        if (!GREEDY) {
            if (writer && acc && p.lse_t) p.lse_t[(long long)b * (K + 1) + (j - 1)] = sLseT[q];
            if (writer && dread && p.lse_d && !OH) p.lse_d[(long long)b * K + (j - 1)] = sLseD[q];
            if (dread && p.derived && !OH) {
                // c_j = max_v q_j(v) = 1 / Sd; S_j = S_{j-1} c_j
                const double S = st.S / sSd[q];
                st.S = S;
                if (writer && p.surv) p.surv[(long long)b * K + (j - 1)] = (float)S;
                if (len) {
                    if (S >= (double)tau_b) {
                        if (j == K) { st.L = K; len = false; }
                    } else {
                        st.L = j - 1;
                        len = false;
                    }
                }
            }
        }
        if (!acc) continue;
        const bool verify = len || st.L >= j; // open length walk means S_j >= tau, so L >= j
        if (verify) {
            const int x = sTok[q];
            if (x < 0 || x >= p.V) {
                st.kind = KIND_BAD;
                st.a = 0;
                acc = false;
                if (writer) or_status(&w.ctl[CTL_STATUS], SV_STATUS_BAD_INPUT);
            } else if (GREEDY) {
                if (x == sG[q]) {
                    st.a = j;
                } else {
                    st.kind = KIND_GREEDY;
                    st.y = sG[q];
                    acc = false;
                }
            } else {
                const double ratio = sRatio[q];
                const double uj = (double)sU[q];
                if (uj < ratio) {
                    st.a = j;
                } else {
                    st.kind = KIND_RESID;
                    st.js = j;
                    st.Mt = sMt[q]; st.St = sSt[q]; st.Md = sMd[q]; st.Sd = sSd[q];
                    acc = false;
                }
            }
        } else {
            // L == j - 1: the final token comes from target row j
            if (GREEDY) {
                st.kind = KIND_GREEDY;
                st.y = sG[q];
            } else {
                st.kind = KIND_BONUS;
                st.js = j;
                st.Mt = sMt[q]; st.St = sSt[q];
            }
            acc = false;
        }
    }
    st.flags = (acc ? FL_ACC : 0) | (len ? FL_LEN : 0);
    sm.st = st;
    }
    __syncthreads();
    return sm.st;
}

// One workgroup per sequence.
template <int DT, bool GREEDY, int MODE>
__global__ __launch_bounds__(kThreads) void sv_decide_kernel(Params p, Work w, int j0, int G)
{
    __shared__ DecideSmem sm;
    const int b = (int)blockIdx.x;
    const SeqState st = decide_group<DT, GREEDY, MODE>(p, w, b, j0, G, true, sm);
    if (threadIdx.x == 0) {
        w.st[b] = st;
        w.live[b] = st.flags ? (((st.L + 1) << 2) | st.flags) : 0;
    }
}

// ---------------------------------------------------------------- final draw
//
// Token order inside a split.  With the split layout above, load k of lane
// (64 w + l) covers RUN consecutive tokens at split_base + (4k + w) SEG + l RUN,
// where RUN = 8 (bf16) or 4 (fp32) and SEG = 64 RUN.  So the split is 4 NLOAD
// consecutive segments of SEG tokens, segment g = 4k + w, and inside a segment
// lane l holds tokens l RUN .. l RUN + RUN - 1.  The draw locates its token
// split -> segment -> lane -> token, each level by a fixed-order prefix.

template <int DT>
struct Seg {
    static constexpr int RUN = DT == SV_BF16 ? 8 : 4;
    static constexpr int NLOAD = kPerLane / RUN;
    static constexpr int SEGS = NLOAD * kWaves; // 32 (bf16) or 64 (fp32)
    static constexpr int SEGLEN = 64 * RUN;
};
constexpr int kSegStride = 64; // segment sums stored per split

// The rows' 1/S enter the fp32 masses as two fp32 parts (hi + lo, ~2^-48
// relative): a single fp32 rounding would scale every p (or q) of the row by the
// same factor, an error that does not cancel in p - q and is large relative to
// the residual mass when the rows are nearly equal.
struct DrawCtx {
    float Mt, Md, iSt_hi, iSt_lo, iSd_hi, iSd_lo, c_hi, c_lo;
    double iSt, iSd, c64;
};

__device__ __forceinline__ float scale2(float e, float hi, float lo) { return fmaf(e, hi, e * lo); }

__device__ __forceinline__ DrawCtx make_ctx(const SeqState& st, const Params& p)
{
    DrawCtx c;
    c.Mt = st.Mt;
    c.Md = st.Md;
    c.iSt = 1.0 / st.St;
    c.iSd = st.Sd > 0.0 ? 1.0 / st.Sd : 0.0;
    c.iSt_hi = (float)c.iSt;
    c.iSt_lo = (float)(c.iSt - (double)c.iSt_hi);
    c.iSd_hi = (float)c.iSd;
    c.iSd_lo = (float)(c.iSd - (double)c.iSd_hi);
    c.c_hi = p.c_hi;
    c.c_lo = p.c_lo;
    c.c64 = p.c64;
    return c;
}

__device__ __forceinline__ float uniform_f32(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }

__device__ __forceinline__ double uniform_f64(double v)
{
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)u);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(u >> 32));
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// The context of a workgroup-uniform state, held in scalar registers.
__device__ __forceinline__ DrawCtx uniform_ctx(const DrawCtx& c)
{
    DrawCtx u;
    u.Mt = uniform_f32(c.Mt); u.Md = uniform_f32(c.Md);
    u.iSt_hi = uniform_f32(c.iSt_hi); u.iSt_lo = uniform_f32(c.iSt_lo);
    u.iSd_hi = uniform_f32(c.iSd_hi); u.iSd_lo = uniform_f32(c.iSd_lo);
    u.c_hi = uniform_f32(c.c_hi); u.c_lo = uniform_f32(c.c_lo);
    u.iSt = uniform_f64(c.iSt); u.iSd = uniform_f64(c.iSd); u.c64 = uniform_f64(c.c64);
    return u;
}

__device__ __forceinline__ double mass_f64(float lt, float ld, const DrawCtx& c, bool resid)
{
    const double pd = exp2_f64(((double)lt - (double)c.Mt) * c.c64) * c.iSt;
    const double qd = resid ? exp2_f64(((double)ld - (double)c.Md) * c.c64) * c.iSd : 0.0;
    return pd > qd ? pd - qd : 0.0;
}

// Mass of one token under the final draw: max(0, p - q) for a replacement,
// p for a bonus.  fp32 first; masses whose p or q exceeds 2^-9 are evaluated
// in fp64 (at most 2^10 tokens of a row pair qualify).  Below that, the fp32
// value carries a few 1e-8 relative error, independent from token to token.
__device__ __forceinline__ double draw_mass(float lt, float ld, const DrawCtx& c, bool resid)
{
    const float pf = scale2(scaled_exp2(lt, c.Mt, c.c_hi, c.c_lo), c.iSt_hi, c.iSt_lo);
    const float qf = resid ? scale2(scaled_exp2(ld, c.Md, c.c_hi, c.c_lo), c.iSd_hi, c.iSd_lo) : 0.0f;
    if (fmaxf(pf, qf) > 0x1p-9f) return mass_f64(lt, ld, c, resid);
    return (double)fmaxf(pf - qf, 0.0f);
}

// Inclusive prefix sum over the 64 lanes of a wavefront (fixed order).
__device__ __forceinline__ double wave_incl_scan(double v, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double n = __shfl_up(v, o);
        if (lane >= o) v += n;
    }
    return v;
}

// Mass of a run of RUN consecutive tokens, in token order.  The fast path is
// branch-free fp32 per token, summed in fp64; a run that holds a token whose p
// or q exceeds 2^-9 is summed again with draw_mass (fp64 for those tokens).
// Both kernels that need a run's mass call this, so the sums agree bit for bit.
template <int RUN>
__device__ __forceinline__ double run_mass(const float (&lt)[RUN], const float (&ld)[RUN], const DrawCtx& c, bool resid,
                                           bool& slow)
{
    // fmaxf(pf - qf, 0) equals (pf > qf ? pf - qf : 0) for these finite
    // values; the run is tested once, on its largest p or q
    double acc = 0.0;
    float big = 0.0f;
#pragma unroll
    for (int i = 0; i < RUN; ++i) {
        const float pf = scale2(scaled_exp2(lt[i], c.Mt, c.c_hi, c.c_lo), c.iSt_hi, c.iSt_lo);
        const float qf = resid ? scale2(scaled_exp2(ld[i], c.Md, c.c_hi, c.c_lo), c.iSd_hi, c.iSd_lo) : 0.0f;
        big = fmaxf(big, fmaxf(pf, qf));
        acc += (double)fmaxf(pf - qf, 0.0f);
    }
    slow = big > 0x1p-9f;
    return acc;
}

template <int RUN>
__device__ __forceinline__ double run_mass_exact(const float (&lt)[RUN], const float (&ld)[RUN], const DrawCtx& c,
                                                 bool resid)
{
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < RUN; ++i) acc += draw_mass(lt[i], ld[i], c, resid);
    return acc;
}

// Segment sums of one split (all 256 threads): lane run sums of RUN tokens,
// scanned across each wavefront; lane 63 holds the segment total.
template <int DT>
__device__ __forceinline__ void split_segments(const Chunk<DT>& tc, const Chunk<DT>& dc, const DrawCtx& c, bool resid,
                                               double* seg_out)
{
    using S = Seg<DT>;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < S::NLOAD; ++k) {
        float lt[S::RUN], ld[S::RUN];
#pragma unroll
        for (int i = 0; i < S::RUN; ++i) {
            lt[i] = tc.get(k * S::RUN + i);
            ld[i] = resid ? dc.get(k * S::RUN + i) : 0.0f;
        }
        bool slow;
        double r = run_mass<S::RUN>(lt, ld, c, resid, slow);
        if (slow) r = run_mass_exact<S::RUN>(lt, ld, c, resid); // rare: a large p or q in the run
        const double incl = wave_incl_scan(r, lane);
        if (lane == 63) seg_out[k * kWaves + wv] = incl;
    }
}

// One workgroup per (sequence, split, half of the split): first the decisions
// of the last position group (positions j0 .. j0+G-1), taken by each of the
// sequence's workgroups from the group's partials (the one of split 0, half 0
// writes the outputs and w.fin), then, if they end in a rejection, the
// residual mass of each of the half's segments (w.seg).  Taking the last
// decisions here saves a launch and its drain.  Halves (32 tokens per lane) keep
// the workgroups short and balance the compute-bound pass (two exponentials
// per token) better than whole splits; quarters and eighths measured slower.
template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void sv_resid_kernel(Params p, Work w, int j0, int G)
{
    static_assert((MODE & MODE_ONEHOT) == 0, "one-hot drafts have no residual pass");
    constexpr bool PK = (MODE & MODE_PACKED) != 0;
    using S = Seg<DT>;
    constexpr int NL = Part<DT>::NL, QSEG = NL * kWaves;
    __shared__ double s_seg[QSEG];
    __shared__ DecideSmem sm;
    const int q = (int)(blockIdx.x % kParts);
    const int split = (int)((blockIdx.x / kParts) % p.nsplit);
    const int b = (int)(blockIdx.x / kParts / p.nsplit);
    const bool writer = split == 0 && q == 0;
    const SeqState st = decide_group<DT, false, 0>(p, w, b, j0, G, writer, sm);
    if (writer && threadIdx.x == 0) w.fin[b] = st;
    if (st.kind != KIND_RESID) return;
    const DrawCtx c = uniform_ctx(make_ctx(st, p));
    const int t = (int)threadIdx.x, lane = t & 63, wv = t >> 6;
    Part<DT> tc, dc;
    tc.template load<VEC>(seq_row<DT, PK>(p.t, p.toff, p.tbs, p.trs, b, st.js - 1), split * kSplit, p.V, t, q);
    dc.template load<VEC>(seq_row<DT, PK>(p.d, p.doff, p.dbs, p.drs, b, st.js - 1), split * kSplit, p.V, t, q);
#pragma unroll
    for (int k = 0; k < NL; ++k) {
        float lt[S::RUN], ld[S::RUN];
#pragma unroll
        for (int i = 0; i < S::RUN; ++i) {
            lt[i] = tc.get(k * S::RUN + i);
            ld[i] = dc.get(k * S::RUN + i);
        }
        bool slow;
        double r = run_mass<S::RUN>(lt, ld, c, true, slow);
        if (slow) r = run_mass_exact<S::RUN>(lt, ld, c, true); // rare: a large p or q in the run
        const double incl = wave_incl_scan(r, lane);
        if (lane == 63) s_seg[k * kWaves + wv] = incl;
    }
    __syncthreads();
    if (t < QSEG) w.seg[((long long)b * p.nsplit + split) * kSegStride + q * QSEG + t] = s_seg[t];
}

// First lane whose inclusive prefix exceeds w (lanes < n), as (lane, w minus
// the exclusive prefix of that lane); lane -1 if none.  All lanes take part.
__device__ __forceinline__ int wave_select(double v, int n, double target, double& rel)
{
    const int lane = threadIdx.x & 63;
    const double incl = wave_incl_scan(v, lane);
    const double up = __shfl_up(incl, 1); // every lane takes part in the shuffle
    const double excl = lane == 0 ? 0.0 : up;
    const unsigned long long pass = __ballot(lane < n && incl > target);
    if (!pass) { rel = INFINITY; return -1; }
    const int f = __ffsll(pass) - 1;
    rel = target - __shfl(excl, f);
    return f;
}

// Last lane (< n) with v > 0, or -1.
__device__ __forceinline__ int wave_last_positive(double v, int n)
{
    const int lane = threadIdx.x & 63;
    const unsigned long long pos = __ballot(lane < n && v > 0.0);
    return pos ? 63 - __clzll(pos) : -1;
}

// sts: the states after the last group (w.fin when sv_resid took the last
// decisions, else w.st).
template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void sv_draw_kernel(Params p, Work w, const SeqState* __restrict__ sts)
{
    constexpr bool OH = (MODE & MODE_ONEHOT) != 0, PK = (MODE & MODE_PACKED) != 0;
    using S = Seg<DT>;
    extern __shared__ double s_all[];  // [nsplit][SEGS] residual segment sums of the sequence
    __shared__ double s_bonus[S::SEGS]; // segment sums of the bonus draw's split
    __shared__ double s_wrel, s_Z, s_my;
    __shared__ int s_split, s_resid, s_y;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int K = p.K;
    // requested together with the state: the final draw's uniform and the
    // drafted tokens this thread copies to the output
    const float uf32 = (p.u == nullptr) ? 0.0f : p.u[(long long)b * (K + 1) + K];
    const int tok0 = tid < K ? p.tok[(long long)b * K + tid] : -1;
    const SeqState st = sts[b];
    int kind = st.kind;
    int a = st.a;
    int y = -1;
    float zrep = NAN, py = NAN;

    if (kind == KIND_RESID || kind == KIND_BONUS) {
        if (kind == KIND_RESID && !OH) {
            // every segment sum of the sequence at once (one round trip): the
            // split totals and the search inside the chosen split both read LDS
            const double* sg = w.seg + (long long)b * p.nsplit * kSegStride;
            for (int i = tid; i < p.nsplit * S::SEGS; i += kThreads)
                s_all[i] = sg[(i / S::SEGS) * kSegStride + i % S::SEGS];
            __syncthreads();
        }
        // 1. the split holding the draw point (wave 0, lane k = split k)
        if (tid < 64) {
            bool resid = kind == KIND_RESID;
            double m = 0.0;
            if (resid && !OH && lane < p.nsplit) {
                // residual mass of split `lane`: its segments summed in order
#pragma unroll 8
                for (int g = 0; g < S::SEGS; ++g) m += s_all[lane * S::SEGS + g];
            }
            if (resid && OH) {
                // one-hot drafts (no residual pass): the residual is p without
                // x, so split `lane` carries its mass of p, less p(x) in the
                // split holding x
                const int x = p.tok[(long long)b * K + (st.js - 1)];
                const void* trow = seq_row<DT, PK>(p.t, p.toff, p.tbs, p.trs, b, st.js - 1);
                const double px =
                    exp2_f64(((double)load_one<DT>(trow, x) - (double)st.Mt) * p.c64) / st.St;
                if (lane < p.nsplit) {
                    const long long pb = part_index(p, b, st.js - 1) + lane;
                    const float mk = w.part_m[pb];
                    if (mk != -INFINITY)
                        m = w.part_s[pb] * exp2_f64(((double)mk - (double)st.Mt) * p.c64 - (double)w.part_d[pb]) / st.St;
                    if (x / kSplit == lane) m = fmax(m - px, 0.0);
                }
            }
            const double Z = __shfl(wave_incl_scan(m, lane), p.nsplit - 1);
            if (resid && !(Z > 0.0)) resid = false; // cannot happen in exact arithmetic after a rejection
            if (!resid) {
                m = 0.0;
                if (lane < p.nsplit) {
                    const long long pb = part_index(p, b, st.js - 1) + lane;
                    const float mk = w.part_m[pb];
                    if (mk != -INFINITY)
                        m = w.part_s[pb] * exp2_f64(((double)mk - (double)st.Mt) * p.c64 - (double)w.part_d[pb]) / st.St;
                }
            }
            const double uf = (double)uf32;
            double wrel;
            int ks = wave_select(m, p.nsplit, resid ? uf * Z : uf, wrel);
            if (ks < 0) { // rounding: the last split with mass, its last token
                ks = max(wave_last_positive(m, p.nsplit), 0);
                wrel = INFINITY;
            }
            if (lane == 0) {
                s_split = ks;
                s_wrel = wrel;
                s_resid = resid ? 1 : 0;
                s_Z = kind == KIND_RESID ? (resid ? Z : 0.0) : 1.0;
            }
        }
        __syncthreads();
        const bool resid = s_resid != 0;
        const int ks = s_split;
        const DrawCtx c = make_ctx(st, p);
        const void* trow = seq_row<DT, PK>(p.t, p.toff, p.tbs, p.trs, b, st.js - 1);
        const void* drow = (resid && !OH) ? seq_row<DT, PK>(p.d, p.doff, p.dbs, p.drs, b, st.js - 1) : nullptr;
        const int xone = (resid && OH) ? p.tok[(long long)b * K + (st.js - 1)] : -1; // one-hot draft token

        // 2. segment sums of that split: stored by sv_resid for a replacement
        //    (already in LDS), computed here for a bonus draw and for a
        //    one-hot replacement (the draft row built in registers)
        const double* s_seg = (resid && !OH) ? s_all + ks * S::SEGS : s_bonus;
        if (!resid || OH) {
            Chunk<DT> tc;
            tc.template load<VEC>(trow, ks * kSplit, p.V, tid);
            if (resid) {
                const int off = xone - ks * kSplit;
                int e = -1;
                if (off >= 0 && off < kSplit) {
                    int ol, oe;
                    Chunk<DT>::owner(off, ol, oe);
                    if (tid == ol) e = oe;
                }
                Chunk<DT> dc;
                dc.one_hot(e);
                split_segments<DT>(tc, dc, c, true, s_bonus);
            } else {
                split_segments<DT>(tc, tc, c, false, s_bonus);
            }
            __syncthreads();
        }

        // 3. segment, lane and token (wave 0)
        if (tid < 64) {
            const double wrel = s_wrel;
            double wseg = INFINITY;
            int g = wrel == INFINITY ? -1 : wave_select(lane < S::SEGS ? s_seg[lane] : 0.0, S::SEGS, wrel, wseg);
            if (g < 0) {
                g = max(wave_last_positive(lane < S::SEGS ? s_seg[lane] : 0.0, S::SEGS), 0);
                wseg = INFINITY;
            }
            const int i0 = ks * kSplit + g * S::SEGLEN + lane * S::RUN;
            float lt[S::RUN], ld[S::RUN];
#pragma unroll
            for (int i = 0; i < S::RUN; ++i) {
                lt[i] = i0 + i < p.V ? load_one<DT>(trow, i0 + i) : -INFINITY;
                ld[i] = (resid && i0 + i < p.V)
                            ? (OH ? (i0 + i == xone ? 0.0f : -INFINITY) : load_one<DT>(drow, i0 + i))
                            : -INFINITY;
            }
            bool slow;
            double r = run_mass<S::RUN>(lt, ld, c, resid, slow);
            if (slow) r = run_mass_exact<S::RUN>(lt, ld, c, resid);
            // per-token masses with the same arithmetic as the run sum, for the walk
            double m[S::RUN];
            int lastpos = -1;
#pragma unroll
            for (int i = 0; i < S::RUN; ++i) {
                if (slow) {
                    m[i] = draw_mass(lt[i], ld[i], c, resid);
                } else {
                    const float pf = scale2(scaled_exp2(lt[i], c.Mt, c.c_hi, c.c_lo), c.iSt_hi, c.iSt_lo);
                    const float qf =
                        resid ? scale2(scaled_exp2(ld[i], c.Md, c.c_hi, c.c_lo), c.iSd_hi, c.iSd_lo) : 0.0f;
                    m[i] = (double)fmaxf(pf - qf, 0.0f);
                }
                if (m[i] > 0.0) lastpos = i0 + i;
            }
            double wl;
            int l = wseg == INFINITY ? -1 : wave_select(r, 64, wseg, wl);
            bool walk = l >= 0;
            if (!walk) l = max(wave_last_positive(r, 64), 0);
            if (lane == l) {
                int yy = -1;
                if (walk) {
                    double cl = 0.0;
#pragma unroll
                    for (int i = 0; i < S::RUN; ++i) {
                        cl += m[i];
                        if (yy < 0 && cl > wl) yy = i0 + i;
                    }
                }
                if (yy < 0) yy = lastpos >= 0 ? lastpos : i0; // rounding: last token with mass
                s_y = yy;
                // the reported probability of the chosen token is evaluated in
                // fp64, from the logits this lane holds (yy lies in its run)
                float lty = lt[0], ldy = ld[0];
#pragma unroll
                for (int i = 1; i < S::RUN; ++i)
                    if (i0 + i == yy) { lty = lt[i]; ldy = ld[i]; }
                s_my = mass_f64(lty, resid ? ldy : 0.0f, c, resid);
            }
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

    for (int jj = tid; jj <= K; jj += kThreads) {
        int v = -1;
        if (y >= 0) v = jj < a ? (jj == tid ? tok0 : p.tok[(long long)b * K + jj]) : (jj == a ? y : -1);
        p.out_tok[(long long)b * (K + 1) + jj] = v;
    }
    if (tid == 0) {
        p.acc_out[b] = a;
        p.vl_out[b] = st.L;
        if (p.zmass) p.zmass[b] = zrep;
        if (p.pys) p.pys[b] = py;
        if (p.rows_out) p.rows_out[b] = st.rows;
        if (b == 0) {
            // every kernel that can raise a status bit has finished; the word
            // starts the next call at zero (it is zero from create on)
            if (p.status_out) *p.status_out = w.ctl[CTL_STATUS];
            w.ctl[CTL_STATUS] = 0;
        }
    }
}

// ---------------------------------------------------------------- admission
//
// Load-aware admission (umans.ai blog, "2. Verify smarter: a throttle that
// costs the user nothing"; zhichai.net article, "Under the hood"): every
// drafted position of every sequence is ranked by its survival S_bj =
// prod_{i<=j} c_bi and admitted one at a time while
//   T(m) = (B + sum of the m best survivals) * speed[B + m]
// rises (a verify batch of m admitted positions holds B + m tokens).  Ties
// rank by sequence, then position, so each sequence's admitted positions are
// its first L_b.  Confidences outside [0, 1] are clamped (NaN -> 0) and raise
// SV_STATUS_BAD_INPUT.

struct SchedParams {
    int B, K, n_speed;
    const float* conf;
    const double* speed;
    int* vl_out;
    float* surv;
    int* admitted;
    float* tau;
    double* expected;
    int* status_out;
};

// survivals, left to right in fp64, one thread per sequence
__global__ __launch_bounds__(kThreads) void sv_sched_surv_kernel(SchedParams q, AuxWork w)
{
    const int b = (int)(blockIdx.x * kThreads + threadIdx.x);
    if (b >= q.B) return;
    double S = 1.0;
    bool bad = false;
    for (int j = 0; j < q.K; ++j) {
        const long long i = (long long)b * q.K + j;
        double c = (double)q.conf[i];
        if (!(c >= 0.0 && c <= 1.0)) {
            bad = true;
            c = c > 1.0 ? 1.0 : 0.0;
        }
        S *= c;
        w.sched_s[i] = S;
        if (q.surv) q.surv[i] = (float)S;
    }
    if (bad) or_status(&w.ctl[CTL_SCHED_STATUS], SV_STATUS_BAD_INPUT);
}

// Rank of each drafted position in the descending order.  Every sequence's
// survivals are already non-increasing, so the rank of (b, j) is j plus, for
// every other sequence b', the number of its survivals that rank before S_bj:
// those > S_bj, and for b' < b also those equal to it (one binary search per
// sequence).  One workgroup per position, threads over sequences.
__global__ __launch_bounds__(kThreads) void sv_sched_rank_kernel(SchedParams q, AuxWork w)
{
    __shared__ double red[kWaves];
    const int i = blockIdx.x;
    const int b = i / q.K, j = i % q.K;
    const double x = w.sched_s[i];
    double cnt = 0.0; // counts are small integers: exact in fp64
    for (int bb = threadIdx.x; bb < q.B; bb += kThreads) {
        if (bb == b) continue;
        const double* s = w.sched_s + (long long)bb * q.K;
        const bool ge = bb < b; // count equal survivals too
        int lo = 0, hi = q.K;   // first index whose survival ranks after x
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            const bool before = ge ? s[mid] >= x : s[mid] > x;
            if (before) lo = mid + 1;
            else hi = mid;
        }
        cnt += (double)lo;
    }
    const long long rank = (long long)j + (long long)block_sum(cnt, red);
    if (threadIdx.x == 0) {
        w.sched_rank[i] = (int)rank;
        w.sched_sorted[rank] = x;
    }
}

// One workgroup of 1024 threads: prefix sums of the ranked survivals (each
// thread sums a run of consecutive ranks, then the run totals are scanned in a
// fixed order), the first m at which T stops rising, and the outputs.
constexpr int kSchedThreads = 1024;

__global__ __launch_bounds__(kSchedThreads) void sv_sched_pick_kernel(SchedParams q, AuxWork w)
{
    __shared__ double s_scan[kSchedThreads];
    __shared__ int s_first[kSchedThreads / 64];
    __shared__ int s_m;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int N = q.B * q.K;
    const int per = (N + kSchedThreads - 1) / kSchedThreads;
    const int m0 = tid * per, m1 = min(N, m0 + per);
    double run = 0.0;
    for (int m = m0; m < m1; ++m) run += w.sched_sorted[m];
    s_scan[tid] = run;
    __syncthreads();
    for (int o = 1; o < kSchedThreads; o <<= 1) { // inclusive scan, fixed order
        const double v = tid >= o ? s_scan[tid - o] : 0.0;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
    }
    const double base = (tid > 0 ? s_scan[tid - 1] : 0.0) + (double)q.B; // B + P(m0)
    // first m in this thread's run with T(m+1) <= T(m)
    int first = 0x7fffffff;
    double Pm = base;
    for (int m = m0; m < m1; ++m) {
        const double s = w.sched_sorted[m];
        const double Tm = Pm * q.speed[q.B + m];
        const double Tn = (Pm + s) * q.speed[q.B + m + 1];
        if (Tn <= Tm) { first = m; break; }
        Pm += s;
    }
    for (int o = 32; o > 0; o >>= 1) first = min(first, __shfl_xor(first, o));
    if (lane == 0) s_first[wv] = first;
    __syncthreads();
    if (tid == 0) {
        int f = 0x7fffffff;
        for (int k = 0; k < kSchedThreads / 64; ++k) f = min(f, s_first[k]);
        s_m = f == 0x7fffffff ? N : f;
    }
    __syncthreads();
    const int M = s_m;
    // the thread whose run holds M (the last non-empty run when M = N) reports T(M)
    const bool owner = M < N ? (M >= m0 && M < m1) : (m0 < m1 && m1 == N);
    if (owner) {
        double P = base;
        for (int m = m0; m < M; ++m) P += w.sched_sorted[m];
        if (q.expected) *q.expected = P * q.speed[q.B + M];
        if (q.admitted) *q.admitted = M;
        if (q.tau) *q.tau = M > 0 ? (float)w.sched_sorted[M - 1] : NAN;
    }
    for (int b = tid; b < q.B; b += kSchedThreads) {
        int L = 0;
        for (int j = 0; j < q.K; ++j) L += w.sched_rank[(long long)b * q.K + j] < M ? 1 : 0;
        q.vl_out[b] = L;
    }
    if (tid == 0) {
        if (q.status_out) *q.status_out = w.ctl[CTL_SCHED_STATUS];
        w.ctl[CTL_SCHED_STATUS] = 0;
    }
}

// ---------------------------------------------------------------- confidences
//
// Calibrated, causally delayed confidences (umans.ai blog, "2. Verify
// smarter"; zhichai.net article, "Under the hood"): sigmoid(z / T_j) per
// position, handed over `delay` calls later from a per-slot ring.

struct ConfParams {
    int B, K, delay;
    float c_default;
    const float* z;
    const float* temp;
    const int* reset;
    float* now_out;
    float* out;
    int* status_out;
};

// one workgroup per slot, one thread per position
__global__ __launch_bounds__(kThreads) void sv_conf_kernel(ConfParams q, AuxWork w)
{
    __shared__ int s_h, s_n;
    const int b = blockIdx.x;
    if (threadIdx.x == 0) {
        const bool fresh = q.reset && q.reset[b] != 0;
        s_h = w.conf_head[b];
        s_n = fresh ? 0 : w.conf_count[b];
    }
    __syncthreads();
    const int h = s_h, n = s_n;
    float* ring = w.conf_ring + (long long)b * SV_MAX_CONF_DELAY * w.conf_K;
    for (int j = threadIdx.x; j < q.K; j += kThreads) {
        const long long i = (long long)b * q.K + j;
        const double T = (double)q.temp[j];
        float now;
        if (!(T > 0.0 && T < INFINITY)) {
            now = 0.0f;
            or_status(&w.ctl[CTL_CONF_STATUS], SV_STATUS_BAD_INPUT);
        } else {
            // 1 / (1 + e^{-z/T}); e^{-x} = 2^{-x log2 e} with this library's fp64 exp2
            const double x = (double)q.z[i] / T;
            now = (float)(1.0 / (1.0 + exp2_f64(-x * 1.4426950408889634073599246810019)));
        }
        float out;
        if (q.delay == 0) out = now;
        else if (n >= q.delay) out = ring[((h - q.delay + SV_MAX_CONF_DELAY) % SV_MAX_CONF_DELAY) * w.conf_K + j];
        else out = q.c_default;
        ring[h * w.conf_K + j] = now; // after the read: delay SV_MAX_CONF_DELAY reads this entry
        q.out[i] = out;
        if (q.now_out) q.now_out[i] = now;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        w.conf_head[b] = (h + 1) % SV_MAX_CONF_DELAY;
        w.conf_count[b] = min(n + 1, SV_MAX_CONF_DELAY);
    }
}

__global__ void sv_conf_status_kernel(ConfParams q, AuxWork w)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        if (q.status_out) *q.status_out = w.ctl[CTL_CONF_STATUS];
        w.ctl[CTL_CONF_STATUS] = 0;
    }
}

// ---------------------------------------------------------------- host side


const char* const kKernelNames[K_COUNT] = {"sv_plan", "sv_rows", "sv_decide", "sv_resid", "sv_draw"};
constexpr int kMaxSlots = 64; // timed launches per run

} // namespace

struct spec_verify {
    spec_verify_config cfg;
    int nsplit;
    void* ws;
    Work w;
    AuxWork aux;
    int timing_max, timing_n;
    hipEvent_t* ev;       // [timing_max][kMaxSlots][2]
    int* ev_kernel;       // [timing_max][kMaxSlots] kernel id of each timed launch, -1 unused
};

namespace {

// Launches one kernel of a step (256 threads per workgroup) on stream s.  While
// per-kernel timing is on, the start and stop events are attached to the
// dispatch itself (hipExtLaunchKernelGGL), so they time the kernel's execution
// and not the queue around it.
struct StepLauncher {
    const spec_verify* h;
    hipStream_t s;
    bool timing;
    int slot;
    template <typename F, typename... Args>
    void operator()(int k, F kernel, dim3 grid, uint32_t shmem, Args... args)
    {
        if (timing && slot < kMaxSlots) {
            const int idx = h->timing_n * kMaxSlots + slot;
            hipExtLaunchKernelGGL(kernel, grid, dim3(kThreads), shmem, s, h->ev[idx * 2], h->ev[idx * 2 + 1], 0,
                                  args...);
            h->ev_kernel[idx] = k;
            ++slot;
        } else {
            hipLaunchKernelGGL(kernel, grid, dim3(kThreads), shmem, s, args...);
        }
    }
};

// One verification step on stream s: plan, then per position group the row
// statistics and the decisions (those of the last group inside the residual
// pass when there is one), then the residual masses and the final draw.
// Groups hold 3, 3, 4, 8, 16, 16, ... positions (a remainder of one position
// joins the previous group).  Early groups are small because most sequences
// stop early; each group costs a fixed few microseconds (the launches' ramp and
// drain and the decisions), rows past a rejection inside a group are read for
// nothing.  At B = 256, K = 16 with about 3.8 accepted positions per sequence
// this schedule (3, 3, 4, 7) measured 4.5 us per step less than 2, 2, 4, 9.
template <int DT, bool VEC, bool GR, int MODE, typename Launch>
void enqueue_step(const spec_verify* h, const Params& p, hipStream_t s, Launch& launch)
{
    constexpr bool OH = (MODE & MODE_ONEHOT) != 0;
    const unsigned B = (unsigned)p.B;
    int gj[kMaxGroups], gn[kMaxGroups], ng = 0;
    const int npos = p.K + 1;
    static const int kFirst[] = {3, 3, 4, 8};
    const int nfirst = (int)(sizeof(kFirst) / sizeof(kFirst[0]));
    for (int j0 = 1; j0 <= npos; ++ng) {
        int G = ng < nfirst ? kFirst[ng] : min(kFirst[nfirst - 1] << (ng - nfirst + 1), kMaxGroup);
        if (npos - (j0 + G - 1) <= 1) G = npos - j0 + 1;
        if (G > kMaxGroup) G = kMaxGroup;
        gj[ng] = j0;
        gn[ng] = G;
        j0 += G;
    }
    auto slots = [&](int g) { return (GR || OH) ? gn[g] : 2 * gn[g]; };
    launch(K_PLAN, sv_plan_kernel, dim3((B + kThreads - 1) / kThreads), 0, p, h->w);
    // With a residual pass (sampling with draft probabilities) that pass takes
    // the last group's decisions; otherwise each group has its own launch.
    constexpr bool FUSED_LAST = !GR && !OH;
    for (int g = 0; g < ng; ++g) {
        const long long nrow = (long long)B * slots(g);
        if (VEC && g >= 3 && g + 1 == ng) // (the unaligned path keeps one row per workgroup)
            launch(K_ROWS, sv_rows_late_kernel<DT, true, GR, MODE>,
                   dim3((unsigned)((nrow + kRowsLate - 1) / kRowsLate * p.nsplit)), 0, p, h->w, gj[g], gn[g]);
        else
            launch(K_ROWS, sv_rows_kernel<DT, VEC, GR, MODE>, dim3((unsigned)(nrow * p.nsplit)), 0, p, h->w, gj[g],
                   gn[g]);
        if (FUSED_LAST && g + 1 == ng) break;
        launch(K_DECIDE, sv_decide_kernel<DT, GR, MODE & MODE_ONEHOT>, dim3(B), 0, p, h->w, gj[g], gn[g]);
    }
    if constexpr (FUSED_LAST) // (one-hot drafts: the final draw forms p without x itself)
        launch(K_RESID, sv_resid_kernel<DT, VEC, MODE>, dim3(B * (unsigned)p.nsplit * kParts), 0, p, h->w, gj[ng - 1],
               gn[ng - 1]);
    launch(K_DRAW, sv_draw_kernel<DT, VEC, MODE>, dim3(B), (uint32_t)(p.nsplit * Seg<DT>::SEGS * sizeof(double)), p,
           h->w, (const SeqState*)(FUSED_LAST ? h->w.fin : h->w.st));
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

int nsplit_of(int V) { return (V + kSplit - 1) / kSplit; }

bool args_vec_ok(const spec_verify_config* cfg, const spec_verify_args* a)
{
    const int es = cfg->dtype == SV_BF16 ? 2 : 4;
    const int per = 16 / es;
    if (cfg->vocab % per) return false;
    if ((uintptr_t)a->target_logits % 16) return false;
    if ((a->target_batch_stride * es) % 16 || (a->target_row_stride * es) % 16) return false;
    if (a->temperature > 0.0f && a->draft_mode == SV_DRAFT_PROBS) {
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
    // A launch's work-item count must fit in 32 bits.  The largest launches:
    // sv_rows over the widest position group (at most min(kMaxGroup, K + 1)
    // positions, a target and a draft row each) and sv_resid.
    const long long ns = nsplit_of(cfg->vocab);
    const long long gmax = std::min(kMaxGroup, cfg->max_draft + 1);
    const long long rows_wg = (long long)cfg->max_batch * 2 * gmax * ns;
    const long long resid_wg = (long long)cfg->max_batch * ns * kParts;
    if (std::max(rows_wg, resid_wg) * kThreads > 0xffffffffll) return SV_EUNSUPPORTED;
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
    if (a->draft_mode != SV_DRAFT_PROBS && a->draft_mode != SV_DRAFT_ONEHOT) return SV_EINVAL;
    if (a->draft_row_offsets && !a->target_row_offsets) return SV_EINVAL;
    if (a->target_row_offsets) {
        // packed rows: the row counts give L, so the length is fixed and not passed
        if (a->length_mode != SV_LEN_FIXED || a->verify_len_in) return SV_EINVAL;
        if (T > 0.0f && a->draft_mode == SV_DRAFT_PROBS && !a->draft_row_offsets) return SV_EINVAL;
    }
    if (T > 0.0f) {
        if (!a->uniforms) return SV_EINVAL;
        if (a->draft_mode == SV_DRAFT_PROBS) {
            if (!a->draft_logits) return SV_EINVAL;
            if (a->draft_row_stride < V || a->draft_batch_stride < 0) return SV_EINVAL;
        }
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
    const long long nrow = (long long)cfg->max_batch * (2 * cfg->max_draft + 1);
    const size_t ns = (size_t)h->nsplit;
    size_t off = 0;
    const size_t o_ctl = off; off = align_up(off + CTL_WORDS * sizeof(int));
    const size_t o_pm = off; off = align_up(off + nrow * ns * sizeof(float));
    const size_t o_ps = off; off = align_up(off + nrow * ns * sizeof(double));
    const size_t o_pi = off; off = align_up(off + nrow * ns * sizeof(int));
    const size_t o_pd = off; off = align_up(off + nrow * ns * sizeof(float));
    const size_t o_st = off; off = align_up(off + (size_t)cfg->max_batch * sizeof(SeqState));
    const size_t o_fi = off; off = align_up(off + (size_t)cfg->max_batch * sizeof(SeqState));
    const size_t o_lv = off; off = align_up(off + (size_t)cfg->max_batch * sizeof(int));
    const size_t o_sg = off; off = align_up(off + (size_t)cfg->max_batch * ns * kSegStride * sizeof(double));
    const size_t o_xl = off; off = align_up(off + nrow * sizeof(float));
    const long long ncand = std::min((long long)cfg->max_batch * cfg->max_draft, (long long)SV_MAX_SCHED_CANDIDATES);
    const size_t o_ss = off; off = align_up(off + (size_t)ncand * sizeof(double));
    const size_t o_sr = off; off = align_up(off + (size_t)ncand * sizeof(int));
    const size_t o_so = off; off = align_up(off + (size_t)ncand * sizeof(double));
    const bool conf_ok = (long long)cfg->max_batch * cfg->max_draft <= SV_MAX_SCHED_CANDIDATES;
    const size_t o_cr = off; off = align_up(off + (conf_ok ? (size_t)ncand * SV_MAX_CONF_DELAY * sizeof(float) : 0));
    const size_t o_ch = off; off = align_up(off + (conf_ok ? (size_t)cfg->max_batch * sizeof(int) : 0));
    const size_t o_cc = off; off = align_up(off + (conf_ok ? (size_t)cfg->max_batch * sizeof(int) : 0));
    if (hipMalloc(&h->ws, off) != hipSuccess) { free(h); return SV_ENOMEM; }
    char* base = (char*)h->ws;
    h->w.ctl = (int*)(base + o_ctl);
    h->w.part_m = (float*)(base + o_pm);
    h->w.part_s = (double*)(base + o_ps);
    h->w.part_d = (float*)(base + o_pd);
    h->w.part_i = (int*)(base + o_pi);
    h->w.st = (SeqState*)(base + o_st);
    h->w.fin = (SeqState*)(base + o_fi);
    h->w.live = (int*)(base + o_lv);
    h->w.seg = (double*)(base + o_sg);
    h->w.xlog = (float*)(base + o_xl);
    h->aux.ctl = h->w.ctl;
    h->aux.sched_s = (double*)(base + o_ss);
    h->aux.sched_rank = (int*)(base + o_sr);
    h->aux.sched_sorted = (double*)(base + o_so);
    h->aux.conf_ring = conf_ok ? (float*)(base + o_cr) : nullptr;
    h->aux.conf_head = conf_ok ? (int*)(base + o_ch) : nullptr;
    h->aux.conf_count = conf_ok ? (int*)(base + o_cc) : nullptr;
    h->aux.conf_K = cfg->max_draft;
    // control words (status bits) start at zero; each call clears what it reports;
    // the confidence history starts empty
    bool zero_ok = hipMemset(h->w.ctl, 0, CTL_WORDS * sizeof(int)) == hipSuccess;
    if (conf_ok) {
        zero_ok = zero_ok && hipMemset(base + o_cr, 0, o_cc + (size_t)cfg->max_batch * sizeof(int) - o_cr) == hipSuccess;
    }
    if (!zero_ok || hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(h->ws);
        free(h);
        return SV_EDEVICE;
    }
    *out = h;
    return SV_OK;
}

int spec_verify_destroy(spec_verify_t* h)
{
    if (!h) return SV_OK;
    DeviceGuard guard(h->cfg.device);
    if (h->ev) {
        for (int i = 0; i < h->timing_max * kMaxSlots * 2; ++i) (void)hipEventDestroy(h->ev[i]);
        free(h->ev);
        free(h->ev_kernel);
    }
    int rc = hipFree(h->ws) == hipSuccess ? SV_OK : SV_EDEVICE;
    free(h);
    return rc;
}

int spec_verify_timing_begin(spec_verify_t* h, int32_t max_calls)
{
    if (!h || max_calls < 1 || max_calls > 10000 || h->ev) return SV_EINVAL;
    DeviceGuard guard(h->cfg.device);
    const int n = max_calls * kMaxSlots * 2;
    h->ev = (hipEvent_t*)calloc((size_t)n, sizeof(hipEvent_t));
    h->ev_kernel = (int*)malloc(sizeof(int) * (size_t)max_calls * kMaxSlots);
    if (!h->ev || !h->ev_kernel) {
        free(h->ev);
        free(h->ev_kernel);
        h->ev = nullptr;
        h->ev_kernel = nullptr;
        return SV_ENOMEM;
    }
    for (int i = 0; i < max_calls * kMaxSlots; ++i) h->ev_kernel[i] = -1;
    for (int i = 0; i < n; ++i)
        if (hipEventCreate(&h->ev[i]) != hipSuccess) {
            for (int k = 0; k < i; ++k) (void)hipEventDestroy(h->ev[k]);
            free(h->ev);
            free(h->ev_kernel);
            h->ev = nullptr;
            h->ev_kernel = nullptr;
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
        for (int s = 0; s < kMaxSlots; ++s) {
            const int k = h->ev_kernel[c * kMaxSlots + s];
            if (k < 0) break;
            hipEvent_t e0 = h->ev[(c * kMaxSlots + s) * 2], e1 = h->ev[(c * kMaxSlots + s) * 2 + 1];
            float t = 0.0f;
            if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&t, e0, e1) != hipSuccess) {
                rc = SV_EDEVICE;
                continue;
            }
            if (k < n_kernels) ms[k] += t;
        }
    if (n_runs) *n_runs = h->timing_n;
    for (int i = 0; i < h->timing_max * kMaxSlots * 2; ++i) (void)hipEventDestroy(h->ev[i]);
    free(h->ev);
    free(h->ev_kernel);
    h->ev = nullptr;
    h->ev_kernel = nullptr;
    h->timing_max = h->timing_n = 0;
    return rc;
}

int spec_verify_conf_check(const spec_verify_config* cfg, const spec_verify_conf_args* a)
{
    int rc = check_config(cfg);
    if (rc != SV_OK) return rc;
    if (!a) return SV_EINVAL;
    if (a->B < 0 || a->B > cfg->max_batch || a->K < 1 || a->K > cfg->max_draft) return SV_EINVAL;
    if (a->delay < 0 || a->delay > SV_MAX_CONF_DELAY) return SV_EINVAL;
    if ((long long)cfg->max_batch * cfg->max_draft > SV_MAX_SCHED_CANDIDATES) return SV_EUNSUPPORTED;
    if (a->B == 0) return SV_OK;
    if (!a->conf_logits || !a->temperature || !a->conf_out) return SV_EINVAL;
    return SV_OK;
}

int spec_verify_confidence(spec_verify_t* h, const spec_verify_conf_args* a, void* hip_stream)
{
    if (!h) return SV_EINVAL;
    int rc = spec_verify_conf_check(&h->cfg, a);
    if (rc != SV_OK) return rc;
    if (a->B == 0) return SV_OK;
    DeviceGuard guard(h->cfg.device);
    hipStream_t s = (hipStream_t)hip_stream;
    ConfParams q;
    q.B = a->B;
    q.K = a->K;
    q.delay = a->delay;
    q.c_default = a->c_default;
    q.z = a->conf_logits;
    q.temp = a->temperature;
    q.reset = a->reset;
    q.now_out = a->conf_now;
    q.out = a->conf_out;
    q.status_out = a->device_status;
    hipLaunchKernelGGL(sv_conf_kernel, dim3(a->B), dim3(kThreads), 0, s, q, h->aux);
    hipLaunchKernelGGL(sv_conf_status_kernel, dim3(1), dim3(64), 0, s, q, h->aux);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EDEVICE;
}

int spec_verify_sched_check(const spec_verify_config* cfg, const spec_verify_sched_args* a)
{
    int rc = check_config(cfg);
    if (rc != SV_OK) return rc;
    if (!a) return SV_EINVAL;
    if (a->B < 0 || a->B > cfg->max_batch || a->K < 1 || a->K > cfg->max_draft) return SV_EINVAL;
    if (a->B > SV_MAX_SCHED_BATCH || (long long)a->B * a->K > SV_MAX_SCHED_CANDIDATES) return SV_EUNSUPPORTED;
    if (a->B == 0) return SV_OK;
    if (!a->confidence || !a->speed || !a->verify_len_out) return SV_EINVAL;
    if ((long long)a->n_speed < (long long)a->B * (a->K + 1) + 1) return SV_EINVAL;
    return SV_OK;
}

int spec_verify_schedule(spec_verify_t* h, const spec_verify_sched_args* a, void* hip_stream)
{
    if (!h) return SV_EINVAL;
    int rc = spec_verify_sched_check(&h->cfg, a);
    if (rc != SV_OK) return rc;
    if (a->B == 0) return SV_OK;
    DeviceGuard guard(h->cfg.device);
    hipStream_t s = (hipStream_t)hip_stream;
    SchedParams q;
    q.B = a->B;
    q.K = a->K;
    q.n_speed = a->n_speed;
    q.conf = a->confidence;
    q.speed = a->speed;
    q.vl_out = a->verify_len_out;
    q.surv = a->survival;
    q.admitted = a->admitted;
    q.tau = a->tau;
    q.expected = a->expected_rate;
    q.status_out = a->device_status;
    const unsigned N = (unsigned)(a->B * a->K);
    hipLaunchKernelGGL(sv_sched_surv_kernel, dim3((a->B + kThreads - 1) / kThreads), dim3(kThreads), 0, s, q, h->aux);
    hipLaunchKernelGGL(sv_sched_rank_kernel, dim3(N), dim3(kThreads), 0, s, q, h->aux);
    hipLaunchKernelGGL(sv_sched_pick_kernel, dim3(1), dim3(kSchedThreads), 0, s, q, h->aux);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EDEVICE;
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
    p.seg_w = 1;
    while (p.seg_w < p.nsplit) p.seg_w <<= 1;
    p.greedy = greedy;
    p.len_mode = a->length_mode;
    p.derived = (a->length_mode == SV_LEN_TAU && !a->confidence) ? 1 : 0;
    p.onehot = (!greedy && a->draft_mode == SV_DRAFT_ONEHOT) ? 1 : 0;
    p.toff = (const long long*)a->target_row_offsets;
    p.doff = (greedy || p.onehot) ? nullptr : (const long long*)a->draft_row_offsets;
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
        p.c32 = (float)p.c64;
    }
    p.acc_out = a->accepted_len;
    p.out_tok = a->out_tokens;
    p.vl_out = a->verify_len_out;
    p.lse_t = a->lse_target;
    p.lse_d = a->lse_draft;
    p.surv = a->survival;
    p.zmass = a->residual_mass;
    p.pys = a->sampled_prob;
    p.rows_out = a->rows_read;
    p.status_out = a->device_status;

    const bool timing = h->ev && h->timing_n < h->timing_max;
    StepLauncher launch{h, s, timing, 0};
    const int bf = h->cfg.dtype == SV_BF16;
    const int mode = (p.onehot ? MODE_ONEHOT : 0) | (p.toff ? MODE_PACKED : 0);
    // runtime choices -> kernel variants (greedy steps never take the one-hot variant)
#define SV_STEP(DT, VEC, GR, M) enqueue_step<DT, VEC, GR, M>(h, p, s, launch)
#define SV_STEP_M(DT, VEC, GR) do { switch (GR ? (mode & MODE_PACKED) : mode) { \
        case 0: SV_STEP(DT, VEC, GR, 0); break; case 1: SV_STEP(DT, VEC, GR, 1); break; \
        case 2: SV_STEP(DT, VEC, GR, 2); break; default: SV_STEP(DT, VEC, GR, 3); break; } } while (0)
    if (bf) {
        if (vec) { if (greedy) SV_STEP_M(SV_BF16, true, true); else SV_STEP_M(SV_BF16, true, false); }
        else { if (greedy) SV_STEP_M(SV_BF16, false, true); else SV_STEP_M(SV_BF16, false, false); }
    } else {
        if (vec) { if (greedy) SV_STEP_M(SV_F32, true, true); else SV_STEP_M(SV_F32, true, false); }
        else { if (greedy) SV_STEP_M(SV_F32, false, true); else SV_STEP_M(SV_F32, false, false); }
    }
#undef SV_STEP_M
#undef SV_STEP
    if (timing) h->timing_n++;

    return hipGetLastError() == hipSuccess ? SV_OK : SV_EDEVICE;
}

} // extern "C"
