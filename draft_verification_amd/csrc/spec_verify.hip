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
// Early exit inside one launch.  The pages say generation restarts from the
// first error, so no row after the first rejection can change the output.
// A step is four launches:
//   sv_plan    per sequence: the verify length where it is known without
//              logits, and the control words of the step.
//   sv_stream  one workgroup per 16384-element split of every row the step may
//              need, ordered position by position (all sequences' position 1,
//              then position 2, ...).  A workgroup first reads its sequence's
//              control word and exits if an earlier position has already been
//              rejected (or the verify length excludes its row); otherwise it
//              reduces its split to (max, sum exp2) or (max, argmax) partials.
//              The last of a row's split workgroups to finish (an arrival
//              counter) merges the row in fp64; the second of a position's two
//              rows to finish takes the acceptance test u < p/q and, on a
//              rejection, lowers the sequence's "first rejection" word, which
//              later workgroups of the same launch read.  Rows of positions
//              dispatched before the rejection was known are read anyway (they
//              lie inside the verify window).  With a derived confidence and an
//              open length walk, each merged draft row also advances the
//              sequence's survival product S_j = S_{j-1} c_j as far as the
//              merged rows allow, and closes the walk (fixes L) at the first
//              S_j < tau.
//   sv_resid   per (sequence, split, half split), for a sequence whose walk
//              ended in a rejection: the segment sums of max(0, p - q) over the
//              rejected row pair.  (One-hot drafts have no residual pass:
//              sv_draw forms p without x itself.)
//   sv_draw    per sequence: inverse-CDF draw (replacement or bonus) by split
//              and segment prefix in fp64, then one segment's tokens scanned in
//              token order; writes the outputs.
//
// Workgroups of one launch exchange records only through agent-scope stores
// and loads (coherent across the chip's eight L2 caches) and arrival counters:
// a writer waits for its stores to complete before the atomic that hands them
// over, so no L2 write-back fence is needed (that fence costs ~130 ns per
// workgroup, serialised).  A workgroup that is not last at a counter simply
// exits; the only wait is that of a workgroup of an open length walk for the
// walk to reach its position, a bounded poll of rows dispatched before it.
//
// Numerics.  bf16 and fp32 inputs are exact in fp32.  The row statistics take
// one fma per element, l*c - round(m*c) with c = log2(e)/T in fp32, and keep
// the exact rounding error of m*c beside the split sum for the fp64 merges.
// v_exp_f32 measured on MI355X: < 0.8 ulp for arguments >= -12.  Sums run in
// fp32 over 8 elements and in fp64 beyond.  Decisions (acceptance ratio,
// survival product, CDF prefix) are taken in fp64.  The residual mass of a
// token is p (1 - 2^-D) with D = log2(p/q) formed from the exact logit
// difference, so it keeps its relative accuracy when p and q nearly agree.
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

#include <algorithm>
#include <mutex>
#include <tuple>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;                     // 4 wavefronts of 64
constexpr int kWaves = kThreads / 64;
constexpr int kSplit = 16384;                     // elements per split (fixed for batch invariance)
constexpr int kPerLane = kSplit / kThreads;       // 64 elements per lane per split
constexpr int kChunkPos = 32;                     // positions per sv_stream launch
constexpr int kOpenPolls = 2000;                  // bound on an open walk's wait in sv_stream (about 2 ms)

enum { CTL_SCHED_STATUS = 2, CTL_CONF_STATUS = 3, CTL_WORDS = 64 };
enum { SEQ_BAD = 1, SEQ_OPEN = 2 };               // plan-time flags of a sequence
enum { DEC_REJECT = 2, DEC_BAD = 3 };             // decision of a position (written on rejection only)
// Compile-time variants of the step kernels: MODE_ONEHOT (q is the point mass
// at the drafted token; never with greedy verification) and MODE_PACKED (rows
// addressed through per-sequence offsets).
enum { MODE_ONEHOT = 1, MODE_PACKED = 2 };
enum { KIND_RESID = 0, KIND_BONUS = 1, KIND_GREEDY = 2, KIND_BAD = 3 };
enum { K_PLAN = 0, K_STREAM = 1, K_RESID = 2, K_DRAW = 3, K_COUNT = 4 };
constexpr unsigned kUnread = 0x7fbadbadu;         // part_m bits of a split no workgroup streamed

// Control word of a sequence.  dead: the first rejected (or bad) position
// known so far, K + 2 while none (0 for a sequence marked bad at plan time);
// lowered with atomic min.  lw: (L + 1) << 16 |
// f, where L + 1 == 0 while the verify length is still open and f is the number
// of survivals S_1..S_f the open walk has formed; moved with compare-and-swap.
// Each sequence's word has a 128-byte line to itself (every workgroup of the
// step reads its word with a coherent load, and the decisions update it with
// atomics): with 16-byte words eight sequences shared a line, and sv_stream
// took 40.3 us instead of 37.2 at B = 64, K = 8.
struct SeqCtl {
    int dead;
    int lw;
    int flags;  // SEQ_*
    int Lout;   // verify length as given (reported for a sequence marked bad)
    int pad[28];
};
static_assert(sizeof(SeqCtl) == 128, "one control word per 128-byte line");

struct Work {
    int* ctl;
    SeqCtl* seq;      // [B]
    int* rcnt;        // [B][2K+1] split arrivals per row (+1 once an open walk's draft row is stored)
    int* pcnt;        // [B][K+2] arrivals per position (1 .. K+1): split workgroups of its rows (verify
                      //   length known at plan time), or merged rows (open length walk)
    int* dec;         // [B][K+1] DEC_* of a rejected or bad position
    float* part_m;    // [B][2K+1][nsplit] split maxima; row j-1 target, K+j draft (j 1-based)
    double* part_s;   // same layout, split sums of exp2((l - m) c + d)
    float* part_d;    // same layout, the d of that sum (the true split sum is part_s * 2^-d)
    int* part_i;      // same layout, split argmax (greedy)
    float* row_m;     // [B][2K+1] row maximum
    double* row_s;    // [B][2K+1] row sum of exp2((l - row_m) c)
    int* row_g;       // [B][2K+1] row argmax (greedy)
    float* xlog;      // [B][2K+1] logit of the drafted token in each row
    double* srec;     // [B][K] survivals S_j of an open length walk
    double* seg;      // [B][nsplit][64] residual mass per segment of a split
    double* segq;     // [B][nsplit][64] q on the residual's support per segment (nearly equal rows)
    double* kp;       // [B][nsplit][2][4] renormalisation sums per half split (nearly equal rows)
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
    int B, K, V, nsplit;
    int greedy, derived;       // derived: tau mode with c = max draft probability
    int onehot;                // q_j is the point mass at x_j; no draft row is streamed
    int count;                 // mark streamed splits (rows_read / bytes_read asked for)
    const long long* toff;     // packed rows: target rows of sequence b start at row toff[b] (NULL: dense)
    const long long* doff;     // packed rows: draft rows of sequence b start at row doff[b]
    int len_mode;
    int lbound;                // fixed lengths: every L_b <= lbound (0: no bound); positions past lbound + 1 are not launched
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
    long long* bytes_out;
    int* status_out;
};

__device__ __forceinline__ void or_status(int* p, int v) { __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Records handed between workgroups of one launch: agent-scope (coherent)
// stores and loads, and the wait for a workgroup's own stores to complete
// (s_waitcnt vmcnt(0)) before the atomic that publishes them.
template <typename T>
__device__ __forceinline__ T ld_ag(const T* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename T>
__device__ __forceinline__ void st_ag(T* p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void stores_done() { __builtin_amdgcn_s_waitcnt(0x0F70); } // vmcnt(0)
__device__ __forceinline__ int add_ag(int* p, int v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void min_ag(int* p, int v) { (void)__hip_atomic_fetch_min(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ bool cas_ag(int* p, int expect, int desired)
{
    return __hip_atomic_compare_exchange_strong(p, &expect, desired, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ long long part_index(const Params& p, int b, int row)
{
    return ((long long)b * (2 * p.K + 1) + row) * p.nsplit;
}

__device__ __forceinline__ long long row_index(const Params& p, int b, int row)
{
    return (long long)b * (2 * p.K + 1) + row;
}

// Arrival counter of position j (1 .. K + 1) of sequence b.
__device__ __forceinline__ long long pos_index(const Params& p, int b, int j)
{
    return (long long)b * (p.K + 2) + j;
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
// once, so their lines are not kept in the caches (measured: the row
// statistics at 5.5 TB/s instead of 4.9 at B=256 K=16 V=129280 bf16).
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
    // the number of loads in flight is fixed; fix_tail() then sets the vectors
    // past V to -inf.
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
// An fp64 constant held in scalar registers (an fma takes one scalar operand):
// inside loops the compiler would otherwise keep every coefficient below in a
// pair of vector registers for the whole loop.
__device__ __forceinline__ double sk(double c)
{
    asm("" : "+s"(c));
    return c;
}

__device__ __forceinline__ double exp2_f64(double a)
{
    if (!(a > -1100.0)) return a != a ? a : 0.0;
    if (a > 1100.0) return INFINITY;
    const double n = rint(a);
    const double x = (a - n) * sk(0.69314718055994530942);
    double r = sk(2.505210838544171877505e-08);     // 1/11!
    r = fma(r, x, sk(2.755731922398589065256e-07)); // 1/10!
    r = fma(r, x, sk(2.755731922398589065256e-06)); // 1/9!
    r = fma(r, x, sk(2.480158730158730158730e-05)); // 1/8!
    r = fma(r, x, sk(1.984126984126984126984e-04)); // 1/7!
    r = fma(r, x, sk(1.388888888888888888889e-03)); // 1/6!
    r = fma(r, x, sk(8.333333333333333333333e-03)); // 1/5!
    r = fma(r, x, sk(4.166666666666666666667e-02)); // 1/4!
    r = fma(r, x, sk(1.666666666666666666667e-01)); // 1/3!
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
__device__ __forceinline__ float bf16_perm(uint32_t w, uint32_t sel) { return __uint_as_float(__builtin_amdgcn_perm(w, 0u, sel)); }

// Element e of a loaded split for the sum pass; sel_lo and sel_hi are the byte
// selectors of the low and high bf16 half, passed in opaquely per run so that
// no widening is moved out of its run.
template <int DT>
__device__ __forceinline__ float chunk_elem_sum(const Chunk<DT>& c, int e, uint32_t sel_lo, uint32_t sel_hi)
{
    if (DT == SV_BF16) return bf16_perm(((const uint32_t*)&c)[e >> 1], (e & 1) ? sel_hi : sel_lo);
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
                uint32_t lo = 0x05040c0cu, hi = 0x07060c0cu;
                asm volatile("" : "+s"(lo), "+s"(hi)); // widen one run at a time
                float run = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) run += __builtin_amdgcn_exp2f(fmaf(chunk_elem_sum<DT>(c, 8 * r + i, lo, hi), c32, -mc));
                acc += (double)run;
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int r = 0; r < kPerLane / 8; ++r) {
                uint32_t lo = 0x05040c0cu, hi = 0x07060c0cu;
                asm volatile("" : "+s"(lo), "+s"(hi));
                float run = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) run += scaled_exp2(chunk_elem_sum<DT>(c, 8 * r + i, lo, hi), m, c_hi, c_lo);
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
//
// One thread per (sequence, row): clears the row's arrival counter (and the
// position's), marks the row's splits unread when the caller counts streamed
// bytes; the thread of row 0 sets the sequence's control word.

__global__ __launch_bounds__(kThreads) void sv_plan_kernel(Params p, Work w)
{
    const long long R = 2LL * p.K + 1;
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (long long)p.B * R) return;
    const int b = (int)(i / R), r = (int)(i % R), K = p.K;
    w.rcnt[i] = 0;
    if (r <= K + 1) w.pcnt[pos_index(p, b, r)] = 0; // positions 1 .. K + 1 (R = 2K + 1 >= K + 2)
    if (p.count)
        for (int k = 0; k < p.nsplit; ++k) w.part_m[i * p.nsplit + k] = __uint_as_float(kUnread);
    if (i == 0 && p.status_out) *p.status_out = 0; // sv_draw raises this call's bits
    if (r != 0) return;
    bool bad = false, open = false;
    int L;
    if (p.toff) {
        // packed rows: the sequence brings L + 1 target rows (and L draft rows)
        const long long nt = p.toff[b + 1] - p.toff[b];
        L = (int)(nt - 1);
        if (nt < 1 || nt > K + 1) bad = true;
        if (p.doff && p.doff[b + 1] - p.doff[b] != nt - 1) bad = true;
        if (p.lbound && L > p.lbound) bad = true; // its later rows are not launched
    } else if (p.len_mode == SV_LEN_FIXED) {
        L = p.vl_in ? p.vl_in[b] : K;
        if (L < 0 || L > K || (p.lbound && L > p.lbound)) bad = true;
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
        else { L = -1; open = true; }
        if (p.onehot && p.surv)
            for (int j = 0; j < K; ++j) p.surv[(long long)b * K + j] = 1.0f;
    }
    // a bad sequence needs no row: dead = 0 and a closed length (L + 1 = 1),
    // since an unknown length would ask for every draft row
    SeqCtl* c = &w.seq[b];
    c->dead = bad ? 0 : K + 2;
    c->lw = bad ? (1 << 16) : (open ? 0 : ((L + 1) << 16));
    c->flags = (bad ? SEQ_BAD : 0) | (open ? SEQ_OPEN : 0);
    c->Lout = L;
}

// ---------------------------------------------------------------- sv_stream
//
// Which rows a workgroup streams, from its sequence's control word when it
// starts (dead = first known rejection, L = verify length or unknown):
//   target row j  iff j <= dead and (L unknown or j <= L + 1)
//   draft row j   iff j <= K and (L unknown, or j <= min(dead, L))
// With L unknown (an open length walk) every draft row feeds the survival
// product; once the walk closes, only the tested positions' draft rows are read.

// Survival walk of an open verify length (derived confidence c_j = 1/Sd_j):
// advances S_f -> S_{f+1} = S_f c_{f+1} while the next draft row's statistics
// are stored, and closes the walk at the first S_j < tau (L = j - 1) or at K.
// Any thread that finds the next row ready may take the step (compare-and-swap
// on the control word; a racing thread computes the same value); a thread that
// finds it not ready leaves, and the thread that stores that row continues.
// Bounded: every failed swap means another thread advanced the walk.
__device__ void advance_survival(const Params& p, const Work& w, int b)
{
    const double tau = (double)p.tau[b];
    const int K = p.K, ns = p.nsplit;
    int* lwp = &w.seq[b].lw;
    for (int it = 0; it <= 2 * K + 2; ++it) {
        const int lw = ld_ag(lwp);
        if (lw >> 16) return;          // closed
        const int f = lw & 0xffff;     // S_1 .. S_f formed
        if (f >= K) return;
        if (ld_ag(&w.rcnt[row_index(p, b, K + f + 1)]) != ns + 1) return; // c_{f+1} not stored yet
        const double Sd = ld_ag(&w.row_s[row_index(p, b, K + f + 1)]);
        const double Sp = f ? ld_ag(&w.srec[(long long)b * K + f - 1]) : 1.0;
        const double S = Sp / Sd;      // c = max_v q(v) = 1 / Sd
        st_ag(&w.srec[(long long)b * K + f], S);
        stores_done();
        int nw;
        if (S < tau) nw = ((f + 1) << 16) | (f + 1);   // L = f
        else if (f + 1 == K) nw = ((K + 1) << 16) | K; // L = K
        else nw = f + 1;
        (void)cas_ag(lwp, lw, nw);
    }
}

// Merge of one row's split partials in fp64, fixed order (wave 0; lane k
// holds split k's partials, other lanes hold (-inf, 0)).
__device__ __forceinline__ void merge_stats(const Params& p, float pm, double ps, float pd, int lane, float& M, double& S)
{
    M = wave_max(pm);
    const double v = (lane < p.nsplit && pm != -INFINITY) ? ps * exp2_f64(((double)pm - (double)M) * p.c64 - (double)pd) : 0.0;
    S = wave_sum(v);
}

// Acceptance test of position j: accept the drafted token iff u_j <
// p_j(x_j) / q_j(x_j), the ratio from exact logit differences and the fp64 row
// sums (q(x) = 0 accepts).  Returns 0 (accept) or DEC_REJECT.
__device__ __forceinline__ int accept_test(const Params& p, float u, float xt, float Mt, double St, float xd, float Md,
                                           double Sd)
{
    double ratio = INFINITY;
    if (xd != -INFINITY) ratio = exp2_f64((((double)xt - (double)Mt) - ((double)xd - (double)Md)) * p.c64) * (Sd / St);
    return ((double)u < ratio) ? 0 : DEC_REJECT;
}

__device__ __forceinline__ void record_rejection(const Work& w, const Params& p, int b, int j, int dec)
{
    st_ag(&w.dec[(long long)b * (p.K + 1) + j], dec);
    min_ag(&w.seq[b].dead, j);
}

// Verify length known at plan time: the last split workgroup of position j
// (wave 0 only) merges the position's rows -- the target row, and the draft
// row when j <= L -- stores their records and takes the decision of a tested
// position (j <= L): the greedy match, or u < p(x)/q(x) (q(x) = 1 for a
// one-hot draft).  x and u are the drafted token and its uniform.
template <bool GREEDY, int MODE>
__device__ void position_complete(const Params& p, const Work& w, int b, int j, int L, int lane, int x, float u)
{
    constexpr bool OH = (MODE & MODE_ONEHOT) != 0;
    const int K = p.K, ns = p.nsplit;
    const bool two = !GREEDY && !OH && j <= L;
    const long long pt = part_index(p, b, j - 1), pd_ = part_index(p, b, K + j);
    // every partial of the position in one round trip
    float mt = -INFINITY, md = -INFINITY, dt = 0.0f, dd = 0.0f, xt = 0.0f, xd = 0.0f;
    double st = 0.0, sd = 0.0;
    int it = 0x7fffffff;
    if (lane < ns) {
        mt = ld_ag(&w.part_m[pt + lane]);
        if (GREEDY) {
            it = ld_ag(&w.part_i[pt + lane]);
        } else {
            st = ld_ag(&w.part_s[pt + lane]);
            dt = ld_ag(&w.part_d[pt + lane]);
        }
        if (two) {
            md = ld_ag(&w.part_m[pd_ + lane]);
            sd = ld_ag(&w.part_s[pd_ + lane]);
            dd = ld_ag(&w.part_d[pd_ + lane]);
        }
    }
    const bool tested = j <= K && j <= L && x >= 0 && x < p.V;
    if (!GREEDY && tested && lane == 0) {
        xt = ld_ag(&w.xlog[row_index(p, b, j - 1)]);
        if (two) xd = ld_ag(&w.xlog[row_index(p, b, K + j)]);
    }
    float Mt, Md = 0.0f;
    double St = 0.0, Sd = 1.0;
    int G = 0;
    if (GREEDY) {
        float v = mt;
        int ix = it;
        wave_argmax(v, ix);
        Mt = v;
        G = ix;
    } else {
        merge_stats(p, mt, st, dt, lane, Mt, St);
        if (two) merge_stats(p, md, sd, dd, lane, Md, Sd);
    }
    if (lane != 0) return;
    const long long rt = row_index(p, b, j - 1);
    w.row_m[rt] = Mt;
    if (GREEDY) w.row_g[rt] = G;
    else w.row_s[rt] = St;
    if (two) {
        w.row_m[row_index(p, b, K + j)] = Md;
        w.row_s[row_index(p, b, K + j)] = Sd;
    }
    if (j > K || j > L) return; // the bonus row: no test
    int dec;
    if (x < 0 || x >= p.V) dec = DEC_BAD;
    else if (GREEDY) dec = x == G ? 0 : DEC_REJECT;
    else if (OH) dec = accept_test(p, u, xt, Mt, St, 0.0f, 0.0f, 1.0); // one-hot draft row: max 0, sum 1
    else dec = accept_test(p, u, xt, Mt, St, xd, Md, Sd);
    if (dec) record_rejection(w, p, b, j, dec);
}

// Open length walk (derived confidence, 0 < tau <= 1): the last split
// workgroup of a row (wave 0 only) merges that row and publishes its record.
// A draft row then advances the survival walk; the second of a position's two
// rows takes the acceptance test (a test past the L the walk settles on is
// ignored by the final state).
__device__ void row_complete_open(const Params& p, const Work& w, int b, int j, bool draft, int prow, int lane, int x,
                                  float u)
{
    const int K = p.K, ns = p.nsplit;
    const long long pb = part_index(p, b, prow), ri = row_index(p, b, prow);
    float pm = -INFINITY, pd = 0.0f;
    double ps = 0.0;
    if (lane < ns) {
        pm = ld_ag(&w.part_m[pb + lane]);
        ps = ld_ag(&w.part_s[pb + lane]);
        pd = ld_ag(&w.part_d[pb + lane]);
    }
    float M;
    double S;
    merge_stats(p, pm, ps, pd, lane, M, S);
    if (lane != 0) return;
    st_ag(&w.row_m[ri], M);
    st_ag(&w.row_s[ri], S);
    stores_done();
    if (draft) {
        (void)add_ag(&w.rcnt[ri], 1); // the row's statistics are stored: ns + 1
        advance_survival(p, w, b);
    }
    if (j > K || add_ag(&w.pcnt[pos_index(p, b, j)], 1) != 1) return;
    int dec;
    if (x < 0 || x >= p.V) {
        dec = DEC_BAD;
    } else {
        const long long rt = row_index(p, b, j - 1), rd = row_index(p, b, K + j);
        const float Mt = ld_ag(&w.row_m[rt]), Md = ld_ag(&w.row_m[rd]);
        const double St = ld_ag(&w.row_s[rt]), Sd = ld_ag(&w.row_s[rd]);
        dec = accept_test(p, u, ld_ag(&w.xlog[rt]), Mt, St, ld_ag(&w.xlog[rd]), Md, Sd);
    }
    if (dec) record_rejection(w, p, b, j, dec);
}

// Streams split `split` of row (b, j, draft), which the sequence needs, and
// hands its partials over.  Returns true in wave 0 when this was the last
// arrival at the position's (or, in an open length walk, the row's) counter:
// then the caller completes it (complete_row) with the drafted token x and its
// uniform u returned here.  flags and L1 = L + 1 (0 while unknown) come from
// the sequence's control word.  t: the thread index (re-derived by each caller
// copy).
template <int DT, bool VEC, bool GREEDY, int MODE>
__device__ __forceinline__ bool stream_row(const Params& p, const Work& w, int b, int j, bool draft, int split,
                                           int flags, int L1, float* redf, double* redd, int* redi, int t, int& x_out,
                                           float& u_out)
{
    constexpr bool OH = (MODE & MODE_ONEHOT) != 0, PK = (MODE & MODE_PACKED) != 0;
    constexpr int SLOTS = (GREEDY || OH) ? 1 : 2;
    const int K = p.K;
    const int prow = draft ? K + j : j - 1;
    const void* row = draft ? seq_row<DT, PK>(p.d, p.doff, p.dbs, p.drs, b, j - 1)
                            : seq_row<DT, PK>(p.t, p.toff, p.tbs, p.trs, b, j - 1);
    Chunk<DT> c;
    c.template issue<VEC>(row, split * kSplit, p.V, t);
    c.template fix_tail<VEC>(split * kSplit, p.V, t);
    // the drafted token of this position, its uniform, and its logit in this
    // row when the split holds it: b, j and x are uniform, so all come through
    // scalar loads (the token ids, uniforms and logits are never written here)
    typedef const __attribute__((address_space(4))) uint32_t* cptr;
    int x = -1;
    float u = 0.0f, xl = 0.0f;
    bool hasx = false;
    if (j <= K) {
        x = (int)((cptr)p.tok)[(long long)b * K + (j - 1)];
        if (!GREEDY) u = __uint_as_float(((cptr)p.u)[(long long)b * (K + 1) + (j - 1)]);
        const int off = x - split * kSplit;
        if (!GREEDY && x >= 0 && x < p.V && off >= 0 && off < kSplit) {
            if (DT == SV_BF16) {
                // the aligned word holding element x lies in the same page
                const uintptr_t a = (uintptr_t)row + 2 * (uintptr_t)x;
                const uint32_t word = *(cptr)(a & ~(uintptr_t)3);
                xl = (a & 2) ? bf16_hi(word) : bf16_lo(word);
            } else {
                xl = __uint_as_float(((cptr)row)[x]);
            }
            hasx = true;
        }
    }
    const long long pi = part_index(p, b, prow) + split;
    float M, D = 0.0f;
    double S = 0.0;
    int I = 0;
    if (GREEDY) chunk_argmax<DT>(c, p.V, split, M, I, redf, redi, t);
    else chunk_stats<DT>(c, p.c32, p.c_hi, p.c_lo, M, S, D, redf, redd, t);
    x_out = x;
    u_out = u;
    if (t >= 64) return false; // wave 0 hands the partials over
    const bool open = (flags & SEQ_OPEN) != 0;
    int* ctr = open ? &w.rcnt[row_index(p, b, prow)] : &w.pcnt[pos_index(p, b, j)];
    const int expect = p.nsplit * ((!open && SLOTS == 2 && j <= L1 - 1) ? 2 : 1);
    int old = 0;
    if (t == 0) {
        st_ag(&w.part_m[pi], M);
        if (GREEDY) {
            st_ag(&w.part_i[pi], I);
        } else {
            st_ag(&w.part_s[pi], S);
            st_ag(&w.part_d[pi], D);
        }
        if (hasx) st_ag(&w.xlog[row_index(p, b, prow)], xl);
        stores_done();
        old = add_ag(ctr, 1);
    }
    old = __builtin_amdgcn_readfirstlane(old);
    return old == expect - 1;
}

// Completion of the last arrival (wave 0; lane = thread index).
template <bool GREEDY, int MODE>
__device__ __forceinline__ void complete_row(const Params& p, const Work& w, int b, int j, bool draft, int flags, int L1,
                                             int lane, int x, float u)
{
    constexpr bool OH = (MODE & MODE_ONEHOT) != 0;
    if constexpr (!GREEDY && !OH) {
        if (flags & SEQ_OPEN) {
            row_complete_open(p, w, b, j, draft, draft ? p.K + j : j - 1, lane, x, u);
            return;
        }
    }
    position_complete<GREEDY, MODE>(p, w, b, j, L1 - 1, lane, x, u);
}


// A sequence's control word (dead, lw) as read now, one agent-scope load
// shared through LDS so that all waves of the workgroup see the same value.
__device__ __forceinline__ unsigned long long control_word(const Work& w, int b, int t)
{
    __shared__ unsigned long long s_cw;
    if (t == 0) s_cw = ld_ag((const unsigned long long*)&w.seq[b]);
    __syncthreads();
    const unsigned long long cw = s_cw;
    __syncthreads(); // (the next read may overwrite it)
    return cw;
}

// Whether a sequence needs row (j, draft) given its control word as read now
// (dead = first known rejection, L1 = L + 1 or 0 while unknown):
//   target row j  iff j <= dead and (L unknown or j <= L + 1)
//   draft row j   iff j <= K and (L unknown, or j <= min(dead, L))
// With L unknown (an open length walk) every draft row feeds the survival
// product; once the walk closes, only the tested positions' draft rows are read.
__device__ __forceinline__ bool row_needed(int K, int j, bool draft, int dead, int L1)
{
    return draft ? (j <= K && (L1 == 0 || j <= min(dead, L1 - 1))) : (j <= dead && (L1 == 0 || j <= L1));
}

// The row statistics with in-launch decisions, over positions j0 .. j0 +
// gridDim.x / (B rows ns) - 1: one workgroup per (position, sequence, row,
// split), split fastest, then the sequence's rows, then sequences, then
// positions.  Consecutive workgroups stream consecutive 32 KB pieces of a row,
// and a sequence's next position is a whole position block later, by when its
// previous position is usually decided.  A workgroup whose row is no longer
// needed exits after reading its sequence's control word.  Measured
// alternatives, all slower at B=256 K=16 V=129280: dealing several rows to one
// workgroup (one control-word load for several rows, but their decisions come
// later, so more rows are read past a rejection: +40 us); a resident grid that
// strides through the same task order and skips stopped sequences without a
// dispatch each (it runs ahead of the decisions: 1.05 GB read instead of
// 0.75, +100 us); walkers that stream one (sequence, row, split) from
// position to position (each sequence's work serialised: +50 us).
template <int DT, bool VEC, bool GREEDY, int MODE>
__global__ __launch_bounds__(kThreads, (DT == SV_BF16 && VEC) ? 8 : 1) void sv_stream_kernel(Params p, Work w, int j0)
{
    constexpr bool OH = (MODE & MODE_ONEHOT) != 0;
    constexpr int SLOTS = (GREEDY || OH) ? 1 : 2; // one-hot drafts: target rows only
    __shared__ float redf[kWaves];
    __shared__ double redd[kWaves];
    __shared__ int redi[kWaves];
    const int t = (int)threadIdx.x;
    const unsigned ns = (unsigned)p.nsplit;
    const int split = (int)(blockIdx.x % ns);
    unsigned rest = blockIdx.x / ns;
    const bool draft = SLOTS == 2 && (rest & 1);
    rest /= SLOTS;
    const int b = (int)(rest % (unsigned)p.B);
    const int j = j0 + (int)(rest / (unsigned)p.B);
    // the sequence's control word as this workgroup starts: dead and lw in one
    // load (a sequence marked bad at plan time has dead = 0), read once and
    // shared so that every wave takes the same decision
    unsigned long long cw = control_word(w, b, t);
    int dead = (int)(unsigned)cw, L1 = (int)(cw >> 48);
    if (!row_needed(p.K, j, draft, dead, L1)) return;
    const int flags = w.seq[b].flags; // set by sv_plan
    if constexpr (!GREEDY && !OH) {
        // An open length walk needs the rows of position j >= 2 only if it
        // passes j - 1 (S_{j-1} >= tau).  Rather than stream them before that
        // is known, wait until the walk has formed S_{j-1} or closed, or the
        // sequence was rejected before j: every row the walk waits for was
        // dispatched earlier and waits for nothing later.  The wait is bounded
        // (kOpenPolls control-word reads); past it the rows are streamed.
        if ((flags & SEQ_OPEN) && j >= 2) {
#pragma clang loop unroll(disable)
            for (int it = 0; it < kOpenPolls && L1 == 0 && dead >= j && (int)((cw >> 32) & 0xffff) < j - 1; ++it) {
                __builtin_amdgcn_s_sleep(8);
                cw = control_word(w, b, t);
                dead = (int)(unsigned)cw;
                L1 = (int)(cw >> 48);
            }
            if (!row_needed(p.K, j, draft, dead, L1)) return;
        }
    }
    int x;
    float u;
    if (stream_row<DT, VEC, GREEDY, MODE>(p, w, b, j, draft, split, flags, L1, redf, redd, redi, t, x, u))
        complete_row<GREEDY, MODE>(p, w, b, j, draft, flags, L1, t, x, u);
}

// ---------------------------------------------------------------- final state
//
// The outcome of a sequence's walk, from its control word after the stream:
// the first rejection r (if r <= L) ends the walk with a replacement draw from
// row pair r (greedy: the target's token of row r), otherwise every verified
// position was accepted and the bonus token comes from target row L + 1.

struct Final {
    int kind, a, L, js, y;
    bool bad_dec;  // marked bad by a drafted id outside [0, V) at a tested position
};

__device__ __forceinline__ Final final_state(const Params& p, const Work& w, int b, bool greedy)
{
    const SeqCtl& c = w.seq[b];
    const int K = p.K;
    Final f;
    f.y = -1;
    f.js = 0;
    f.a = 0;
    f.bad_dec = false;
    if (c.flags & SEQ_BAD) {
        f.kind = KIND_BAD;
        f.L = c.Lout;
        return f;
    }
    const int L1 = c.lw >> 16;
    if (L1 == 0) { // the survival walk did not close: cannot happen (reported as SV_STATUS_INCOMPLETE)
        f.kind = KIND_BAD;
        f.L = -1;
        return f;
    }
    f.L = L1 - 1;
    const int r = c.dead;
    if (r <= f.L) {
        if (w.dec[(long long)b * (K + 1) + r] == DEC_BAD) {
            f.kind = KIND_BAD;
            f.bad_dec = true;
            return f;
        }
        f.a = r - 1;
        f.js = r;
        f.kind = greedy ? KIND_GREEDY : KIND_RESID;
    } else {
        f.a = f.L;
        f.js = f.L + 1;
        f.kind = greedy ? KIND_GREEDY : KIND_BONUS;
    }
    if (greedy) f.y = w.row_g[row_index(p, b, f.js - 1)];
    return f;
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

// Token masses of the final draw.  p_v = 2^((l_v - Mt) c) / St: per token in
// fp32 without the 1/St, which scales each run's fp32 sum once it is widened
// to fp64; a replacement takes r_v = max(0, p_v - q_v) as
// p_v (1 - 2^-D_v) with D_v = log2(p_v / q_v) = c ((lt_v - ld_v) - (Mt - Md)) +
// log2(Sd / St): the logit difference is exact (a two-sum for fp32 logits;
// bf16 logits differ exactly in fp32), Mt - Md and log2(Sd / St) come from fp64
// in two fp32 parts, and 1 - 2^-D comes from a polynomial in D when |D| < 1/4
// (one_minus_exp2_neg), so r_v keeps its relative accuracy when p and q nearly
// agree (no cancellation of two separately rounded masses).
struct DrawCtx {
    float Mt, c_hi, c_lo;
    float dM_hi, dM_lo, k_hi, k_lo, c32;
    double Mt64, iSt64, dM64, k64, c64;
};


__device__ __forceinline__ DrawCtx make_ctx(float Mt, double St, float Md, double Sd, bool resid, const Params& p)
{
    DrawCtx c;
    c.Mt = Mt;
    c.Mt64 = (double)Mt;
    c.iSt64 = 1.0 / St;
    c.c_hi = p.c_hi;
    c.c_lo = p.c_lo;
    c.c32 = p.c32;
    c.c64 = p.c64;
    c.dM64 = resid ? (double)Mt - (double)Md : 0.0;
    c.k64 = resid ? log2(Sd / St) : 0.0;
    c.dM_hi = (float)c.dM64;
    c.dM_lo = (float)(c.dM64 - (double)c.dM_hi);
    c.k_hi = (float)c.k64;
    c.k_lo = (float)(c.k64 - (double)c.k_hi);
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
    u.Mt = uniform_f32(c.Mt); u.c_hi = uniform_f32(c.c_hi); u.c_lo = uniform_f32(c.c_lo);
    u.dM_hi = uniform_f32(c.dM_hi); u.dM_lo = uniform_f32(c.dM_lo);
    u.k_hi = uniform_f32(c.k_hi); u.k_lo = uniform_f32(c.k_lo); u.c32 = uniform_f32(c.c32);
    u.Mt64 = uniform_f64(c.Mt64); u.iSt64 = uniform_f64(c.iSt64); u.dM64 = uniform_f64(c.dM64);
    u.k64 = uniform_f64(c.k64); u.c64 = uniform_f64(c.c64);
    return u;
}

// St p_v in fp32 (the target mass before the 1/St).
__device__ __forceinline__ float p_mass32(float lt, const DrawCtx& c)
{
    return scaled_exp2(lt, c.Mt, c.c_hi, c.c_lo);
}

// 1 - 2^-D: for |D| < 1/4 as D times a degree-4 polynomial in D fitted to
// (1 - 2^-D) / D on [-1/4, 1/4] (near-minimax in relative error, by
// iteratively reweighted least squares; with these fp32 coefficients the
// polynomial is within 2.0e-8 relative, checked on the host by
// tests/test_kernel_constants.py), else 1 - v_exp_f32(-D) (the difference is
// then at least 0.159, so exp's ulp costs < 4e-7 relative).
__device__ __forceinline__ float one_minus_exp2_neg(float D)
{
    // coefficients of D^4 .. D^0 (kernel-constant: one_minus_exp2_neg)
    float s = fmaf(D, 1.333353342e-03f, -9.630151093e-03f);
    s = fmaf(s, D, 5.550416559e-02f);
    s = fmaf(s, D, -2.402263135e-01f);
    s = fmaf(s, D, 6.931471825e-01f);
    return fabsf(D) < 0.25f ? s * D : 1.0f - __builtin_amdgcn_exp2f(-D);
}

// Residual mass of one token in fp32, times St (see DrawCtx).  -inf logits: q_v = 0
// gives D = +inf and r_v = p_v; p_v = 0 gives 0 (a NaN D is dropped by fmaxf).
template <int DT, bool LO = true>
__device__ __forceinline__ float resid_mass32(float lt, float ld, const DrawCtx& c)
{
    const float pf = p_mass32(lt, c);
    float u;
    if (DT == SV_BF16) {
        u = (lt - ld) - c.dM_hi;
        if (LO) u -= c.dM_lo;
    } else {
        const float lq = fmaxf(ld, -0x1p127f); // keeps the two-sum finite when q_v = 0
        const float s = lt - lq;
        const float bb = s - lt;
        const float e = (lt - (s - bb)) - (lq + bb);
        u = ((s - c.dM_hi) + e) - c.dM_lo;
    }
    const float D = fmaf(u, c.c32, c.k_hi) + c.k_lo;
    return pf * fmaxf(one_minus_exp2_neg(D), 0.0f);
}

template <int DT, bool LO = true>
__device__ __forceinline__ float draw_mass32(float lt, float ld, const DrawCtx& c, bool resid)
{
    return resid ? resid_mass32<DT, LO>(lt, ld, c) : p_mass32(lt, c);
}

// The residual mass of one token with the two sums that renormalise the draft
// row against the target row (see the renormalisation at sv_draw), all times
// St: qa = q_v
// on the residual's support (where p > q) and kap = p_v - q_v (signed, over
// every token), both as p_v times a factor of 2^-D.  bad: the token's q_v
// exceeds p_v by more than 2^120 (a target logit of -inf where the draft has
// mass), where kap cannot be formed this way.
template <int DT>
__device__ __forceinline__ void resid_parts32(float lt, float ld, const DrawCtx& c, float& r, float& qa, float& kap,
                                              float& pp, bool& bad)
{
    const float pf = p_mass32(lt, c);
    float u;
    if (DT == SV_BF16) {
        u = ((lt - ld) - c.dM_hi) - c.dM_lo;
    } else {
        const float lq = fmaxf(ld, -0x1p127f);
        const float s = lt - lq;
        const float bb = s - lt;
        const float e = (lt - (s - bb)) - (lq + bb);
        u = ((s - c.dM_hi) + e) - c.dM_lo;
    }
    const float D = fmaf(u, c.c32, c.k_hi) + c.k_lo;
    const bool ok = D >= -120.0f;
    const float om = one_minus_exp2_neg(ok ? D : -120.0f);
    r = pf * fmaxf(om, 0.0f);
    qa = om > 0.0f ? pf - r : 0.0f;
    kap = ok ? pf * om : 0.0f;
    pp = pf;
    bad = !ok && ld > -INFINITY;
}

// The same mass in fp64 (the reported probability of the drawn token); qa:
// q_v where the residual is positive, else 0.
__device__ __forceinline__ double draw_mass64(float lt, float ld, const DrawCtx& c, bool resid, double& qa)
{
    const double pd = exp2_f64(((double)lt - c.Mt64) * c.c64) * c.iSt64;
    qa = 0.0;
    if (!resid || !(ld > -INFINITY)) return pd;
    const double D = (((double)lt - (double)ld) - c.dM64) * c.c64 + c.k64;
    double om;
    if (fabs(D) < 0.0625) {
        // 1 - e^-x = x sum_{m=0}^{8} (-x)^m / (m+1)!, |x| < 0.044: truncation below 1e-18
        const double x = D * 0.69314718055994530942, y = -x;
        double h = 1.0 / 362880.0;
        h = fma(h, y, 1.0 / 40320.0);
        h = fma(h, y, 1.0 / 5040.0);
        h = fma(h, y, 1.0 / 720.0);
        h = fma(h, y, 1.0 / 120.0);
        h = fma(h, y, 1.0 / 24.0);
        h = fma(h, y, 1.0 / 6.0);
        h = fma(h, y, 0.5);
        h = fma(h, y, 1.0);
        om = x * h;
    } else {
        om = 1.0 - exp2_f64(-D);
    }
    if (om > 0.0) qa = pd * (1.0 - om);
    return pd * fmax(om, 0.0);
}

// v of the lane CTRL selects (a DPP row shift or row broadcast), 0 where that
// lane is out of the row or the row is masked off; both halves of the double.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v)
{
    const long long x = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(x >> 32), CTRL, ROWS, 0xf, false);
    return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

// Inclusive prefix sum over the 64 lanes of a wavefront (fixed order): a scan
// inside each row of 16 lanes (shifts by 1, 2, 4, 8), then row 0's total
// added to row 1 and row 2's to row 3, then rows 0-1's total to rows 2 and 3.
// Every kernel that needs lane prefixes calls this, so they agree bit for bit.
__device__ __forceinline__ double wave_incl_scan(double v, int)
{
    v += dpp_f64<0x111, 0xf>(v); // row_shr:1
    v += dpp_f64<0x112, 0xf>(v); // row_shr:2
    v += dpp_f64<0x114, 0xf>(v); // row_shr:4
    v += dpp_f64<0x118, 0xf>(v); // row_shr:8
    v += dpp_f64<0x142, 0xa>(v); // row_bcast:15 into rows 1 and 3
    v += dpp_f64<0x143, 0xc>(v); // row_bcast:31 into rows 2 and 3
    return v;
}

// Mass of a run of RUN consecutive tokens: per-token fp32 masses (times St)
// summed pairwise in fp32 (at most 3 roundings deep), then widened and scaled
// by 1/St.  Every kernel that needs a run's mass calls this, so the sums agree
// bit for bit.
template <int DT, int RUN, bool LO = true>
__device__ __forceinline__ double run_mass(const float (&lt)[RUN], const float (&ld)[RUN], const DrawCtx& c, bool resid)
{
    float m[RUN];
#pragma unroll
    for (int i = 0; i < RUN; ++i) m[i] = draw_mass32<DT, LO>(lt[i], ld[i], c, resid);
#pragma unroll
    for (int w = 1; w < RUN; w <<= 1)
#pragma unroll
        for (int i = 0; i + w < RUN; i += 2 * w) m[i] += m[i + w];
    return (double)m[0] * c.iSt64;
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
        const double r = run_mass<DT, S::RUN>(lt, ld, c, resid);
        const double incl = wave_incl_scan(r, lane);
        if (lane == 63) seg_out[k * kWaves + wv] = incl;
    }
}

// ---------------------------------------------------------------- sv_resid
//
// Renormalisation of nearly equal rows.  Every token's residual uses the log
// ratio of the two row sums, log2(Sd / St), from the row statistics; their
// errors (a few 1e-8, from fp32 exponents and run sums) are independent, so
// the ratio is off by a few 1e-8 and every r_v = p_v (1 - 2^-D_v) by about
// q_v times that -- negligible against Z unless the rows nearly agree (Z ~
// 1e-3 and below).  For such a row pair the residual pass also sums
// kap = sum_v (p_v - q_v) over all tokens and P = sum_v p_v, each term formed
// from the exact logit difference (so kap's error is ~1e-7 of sum |p - q| =
// 2Z, not of 1), and qa = q_v over the residual's support per segment.  Then
// q is rescaled to the same total as p: q_v -> q_v F, F = P / (P - kap), and
// to first order r_v -> r_v - (F - 1) q_v on the support, Z -> (Z - (F - 1)
// QA) / P.  Which row pairs: those whose rejected token has p(x)/q(x) within
// 1/8 of 1 (nearly equal rows give ratios near 1 for every token); the test
// reads only stored records, so both kernels take it identically.
constexpr int kKpStride = 4; // (kap, P, bad, -) per half split

__device__ __forceinline__ bool near_equal_rows(const Params& p, const Work& w, int b, int js)
{
    const long long rt = row_index(p, b, js - 1), rd = row_index(p, b, p.K + js);
    const float xd = w.xlog[rd];
    if (xd == -INFINITY) return false;
    const double ratio =
        exp2_f64((((double)w.xlog[rt] - (double)w.row_m[rt]) - ((double)xd - (double)w.row_m[rd])) * p.c64) *
        (w.row_s[rd] / w.row_s[rt]);
    return fabs(ratio - 1.0) < 0.125;
}

// One workgroup per (sequence, split, half of the split): if the sequence's
// walk ended in a rejection at position js, the residual mass of each of the
// half's segments of row pair js (w.seg), and for nearly equal rows the
// renormalisation sums (w.segq, w.kp).  Halves (32 tokens per lane) keep the
// workgroups short and balance the compute-bound pass (two exponentials per
// token) better than whole splits.
template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void sv_resid_kernel(Params p, Work w)
{
    static_assert((MODE & MODE_ONEHOT) == 0, "one-hot drafts have no residual pass");
    constexpr bool PK = (MODE & MODE_PACKED) != 0;
    using S = Seg<DT>;
    constexpr int NL = Part<DT>::NL, QSEG = NL * kWaves;
    __shared__ double s_seg[QSEG], s_segq[QSEG];
    __shared__ double s_red[kWaves];
    const int q = (int)(blockIdx.x % kParts);
    const int split = (int)((blockIdx.x / kParts) % p.nsplit);
    const int b = (int)(blockIdx.x / kParts / p.nsplit);
    const Final f = final_state(p, w, b, false);
    if (f.kind != KIND_RESID) return;
    const int K = p.K;
    const long long rt = row_index(p, b, f.js - 1), rd = row_index(p, b, K + f.js);
    const DrawCtx c = uniform_ctx(make_ctx(w.row_m[rt], w.row_s[rt], w.row_m[rd], w.row_s[rd], true, p));
    const bool fine = near_equal_rows(p, w, b, f.js);
    const int t = (int)threadIdx.x, lane = t & 63, wv = t >> 6;
    Part<DT> tc, dc;
    tc.template load<VEC>(seq_row<DT, PK>(p.t, p.toff, p.tbs, p.trs, b, f.js - 1), split * kSplit, p.V, t, q);
    dc.template load<VEC>(seq_row<DT, PK>(p.d, p.doff, p.dbs, p.drs, b, f.js - 1), split * kSplit, p.V, t, q);
    const long long so = ((long long)b * p.nsplit + split) * kSegStride + q * QSEG;
    if (!fine) {
        // bf16 maxima differ exactly in fp32 (the low part of Mt - Md is then
        // 0 and subtracting it changes no bit): one instruction less per token
        if (DT == SV_BF16 && c.dM_lo == 0.0f) {
#pragma unroll
            for (int k = 0; k < NL; ++k) {
                float lt[S::RUN], ld[S::RUN];
#pragma unroll
                for (int i = 0; i < S::RUN; ++i) {
                    lt[i] = tc.get(k * S::RUN + i);
                    ld[i] = dc.get(k * S::RUN + i);
                }
                const double r = run_mass<DT, S::RUN, false>(lt, ld, c, true);
                const double incl = wave_incl_scan(r, lane);
                if (lane == 63) s_seg[k * kWaves + wv] = incl;
            }
        } else {
#pragma unroll
            for (int k = 0; k < NL; ++k) {
                float lt[S::RUN], ld[S::RUN];
#pragma unroll
                for (int i = 0; i < S::RUN; ++i) {
                    lt[i] = tc.get(k * S::RUN + i);
                    ld[i] = dc.get(k * S::RUN + i);
                }
                const double r = run_mass<DT, S::RUN>(lt, ld, c, true);
                const double incl = wave_incl_scan(r, lane);
                if (lane == 63) s_seg[k * kWaves + wv] = incl;
            }
        }
        __syncthreads();
        if (t < QSEG) w.seg[so + t] = s_seg[t];
        return;
    }
    double kap = 0.0, pp = 0.0;
    bool bad = false;
#pragma unroll
    for (int k = 0; k < NL; ++k) {
        float r[S::RUN], qa[S::RUN];
        float ks = 0.0f, ps = 0.0f; // kap and P of the run, in token order
#pragma unroll
        for (int i = 0; i < S::RUN; ++i) {
            bool bi;
            float kk, pv;
            resid_parts32<DT>(tc.get(k * S::RUN + i), dc.get(k * S::RUN + i), c, r[i], qa[i], kk, pv, bi);
            ks += kk;
            ps += pv;
            bad |= bi;
        }
        // pairwise in fp32 (the residual in the same order as run_mass, which
        // the draw repeats token by token)
#pragma unroll
        for (int h = 1; h < S::RUN; h <<= 1)
#pragma unroll
            for (int i = 0; i + h < S::RUN; i += 2 * h) {
                r[i] += r[i + h];
                qa[i] += qa[i + h];
            }
        kap += (double)ks * c.iSt64;
        pp += (double)ps * c.iSt64;
        const double incl = wave_incl_scan((double)r[0] * c.iSt64, lane);
        const double inclq = wave_incl_scan((double)qa[0] * c.iSt64, lane);
        if (lane == 63) {
            s_seg[k * kWaves + wv] = incl;
            s_segq[k * kWaves + wv] = inclq;
        }
        __builtin_amdgcn_sched_barrier(0); // one run at a time (registers)
    }
    const bool anybad = __syncthreads_or(bad);
    kap = block_sum(kap, s_red, t);
    pp = block_sum(pp, s_red, t);
    if (t < QSEG) {
        w.seg[so + t] = s_seg[t];
        w.segq[so + t] = s_segq[t];
    }
    if (t == 0) {
        double* kq = w.kp + (((long long)b * p.nsplit + split) * kParts + q) * kKpStride;
        kq[0] = kap;
        kq[1] = pp;
        kq[2] = anybad ? 1.0 : 0.0;
    }
}

// ---------------------------------------------------------------- sv_draw

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

// Mass of split k of target row js under p, from the row statistics' partials.
__device__ __forceinline__ double split_p_mass(const Params& p, const Work& w, int b, int js, int k, float Mt, double St)
{
    const long long pb = part_index(p, b, js - 1) + k;
    const float mk = w.part_m[pb];
    if (mk == -INFINITY) return 0.0;
    return w.part_s[pb] * exp2_f64(((double)mk - (double)Mt) * p.c64 - (double)w.part_d[pb]) / St;
}

// One workgroup per sequence: the final draw, the emitted block and the
// diagnostics.  The last workgroup to finish reports the call's status bits.
template <int DT, bool VEC, bool GREEDY, int MODE>
__global__ __launch_bounds__(kThreads) void sv_draw_kernel(Params p, Work w)
{
    constexpr bool OH = (MODE & MODE_ONEHOT) != 0, PK = (MODE & MODE_PACKED) != 0;
    using S = Seg<DT>;
    extern __shared__ double s_all[];  // [nsplit][SEGS] residual segment sums of the sequence
    __shared__ double s_bonus[S::SEGS]; // segment sums of the bonus draw's split
    __shared__ double s_wrel, s_Z, s_my, s_F1, s_P;
    __shared__ int s_split, s_resid, s_y;
    __shared__ double s_cnt[kWaves];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int K = p.K;
    const long long R = 2LL * K + 1, rb = (long long)b * R;
    // requested together with the state: the final draw's uniform and the
    // drafted tokens this thread copies to the output
    const float uf32 = (p.u == nullptr) ? 0.0f : p.u[(long long)b * (K + 1) + K];
    const int tok0 = tid < K ? p.tok[(long long)b * K + tid] : -1;
    // the segment sums a replacement draw needs, requested before the state is
    // known (one value per thread at V = 129280; unused for other draws)
    constexpr int kSegPre = 2;
    double segv[kSegPre];
    const double* sg = w.seg + (long long)b * p.nsplit * kSegStride;
    const int nseg = GREEDY || OH ? 0 : p.nsplit * S::SEGS;
#pragma unroll
    for (int k = 0; k < kSegPre; ++k) {
        const int i = tid + k * kThreads;
        segv[k] = i < nseg ? sg[(i / S::SEGS) * kSegStride + i % S::SEGS] : 0.0;
    }
    const Final f = final_state(p, w, b, GREEDY);
    int kind = f.kind;
    const int a = f.a;
    int y = -1;
    float zrep = NAN, py = NAN;

    if (kind == KIND_RESID || kind == KIND_BONUS) {
        const int js = f.js;
        const float Mt = w.row_m[rb + js - 1];
        const double St = w.row_s[rb + js - 1];
        float Md = 0.0f;
        double Sd = 1.0; // one-hot draft row: max 0, sum 1
        // nearly equal rows: the residual is renormalised (see sv_resid)
        const bool fine = kind == KIND_RESID && !OH && near_equal_rows(p, w, b, js);
        if (kind == KIND_RESID && !OH) {
            Md = w.row_m[rb + K + js];
            Sd = w.row_s[rb + K + js];
            // every segment sum of the sequence in LDS: the split totals and
            // the search inside the chosen split both read them
#pragma unroll
            for (int k = 0; k < kSegPre; ++k)
                if (tid + k * kThreads < nseg) s_all[tid + k * kThreads] = segv[k];
            for (int i = tid + kSegPre * kThreads; i < nseg; i += kThreads)
                s_all[i] = sg[(i / S::SEGS) * kSegStride + i % S::SEGS];
            __syncthreads();
        }
        // 1. the split holding the draw point (wave 0, lane k = split k)
        if (tid < 64) {
            bool resid = kind == KIND_RESID;
            double m = 0.0, F1 = 0.0, P = 1.0;
            if (fine) {
                // F - 1 = kap / (P - kap) from the half splits' sums (fixed order)
                const double* kq = w.kp + (long long)b * p.nsplit * kParts * kKpStride;
                double kv = 0.0, pv = 0.0;
                bool bad = false;
                for (int i = lane; i < p.nsplit * kParts; i += 64) {
                    kv += kq[i * kKpStride];
                    pv += kq[i * kKpStride + 1];
                    bad |= kq[i * kKpStride + 2] != 0.0;
                }
                const double kap = wave_sum(kv);
                P = wave_sum(pv);
                F1 = (__ballot(bad) || !(P > kap)) ? 0.0 : kap / (P - kap);
            }
            if (resid && !OH && lane < p.nsplit) {
                // residual mass of split `lane`: its segments summed in order
#pragma unroll 8
                for (int g = 0; g < S::SEGS; ++g) m += s_all[lane * S::SEGS + g];
                if (fine) {
                    const double* sq = w.segq + ((long long)b * p.nsplit + lane) * kSegStride;
                    double mq = 0.0;
#pragma unroll 8
                    for (int g = 0; g < S::SEGS; ++g) mq += sq[g];
                    m = fmax(m - F1 * mq, 0.0);
                }
            }
            if (resid && OH) {
                // one-hot drafts (no residual pass): the residual is p without
                // x, so split `lane` carries its mass of p, less p(x) in the
                // split holding x
                const int x = p.tok[(long long)b * K + (js - 1)];
                const void* trow = seq_row<DT, PK>(p.t, p.toff, p.tbs, p.trs, b, js - 1);
                const double px = exp2_f64(((double)load_one<DT>(trow, x) - (double)Mt) * p.c64) / St;
                if (lane < p.nsplit) {
                    m = split_p_mass(p, w, b, js, lane, Mt, St);
                    if (x / kSplit == lane) m = fmax(m - px, 0.0);
                }
            }
            const double Z = __shfl(wave_incl_scan(m, lane), p.nsplit - 1);
            if (resid && !(Z > 0.0)) resid = false; // cannot happen in exact arithmetic after a rejection
            if (!resid) {
                m = lane < p.nsplit ? split_p_mass(p, w, b, js, lane, Mt, St) : 0.0;
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
                s_F1 = resid ? F1 : 0.0;
                s_P = (fine && resid) ? P : 1.0; // the target row's own total
            }
        }
        __syncthreads();
        const bool resid = s_resid != 0;
        const int ks = s_split;
        const DrawCtx c = make_ctx(Mt, St, Md, Sd, resid, p);
        const void* trow = seq_row<DT, PK>(p.t, p.toff, p.tbs, p.trs, b, js - 1);
        const void* drow = (resid && !OH) ? seq_row<DT, PK>(p.d, p.doff, p.dbs, p.drs, b, js - 1) : nullptr;
        const int xone = (resid && OH) ? p.tok[(long long)b * K + (js - 1)] : -1; // one-hot draft token

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
            const double wrel = s_wrel, F1 = s_F1;
            const bool corr = fine && resid;
            double sv = lane < S::SEGS ? s_seg[lane] : 0.0;
            if (corr && lane < S::SEGS)
                sv = fmax(sv - F1 * w.segq[((long long)b * p.nsplit + ks) * kSegStride + lane], 0.0);
            double wseg = INFINITY;
            int g = wrel == INFINITY ? -1 : wave_select(sv, S::SEGS, wrel, wseg);
            if (g < 0) {
                g = max(wave_last_positive(sv, S::SEGS), 0);
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
            double r;
            // per-token masses with the same arithmetic as the run sum, for the walk
            double m[S::RUN];
            int lastpos = -1;
            if (corr) {
                float rr[S::RUN], qq[S::RUN], kk, pp;
                bool bb;
#pragma unroll
                for (int i = 0; i < S::RUN; ++i) resid_parts32<DT>(lt[i], ld[i], c, rr[i], qq[i], kk, pp, bb);
#pragma unroll
                for (int i = 0; i < S::RUN; ++i)
                    m[i] = fmax((double)rr[i] * c.iSt64 - F1 * ((double)qq[i] * c.iSt64), 0.0);
#pragma unroll
                for (int h = 1; h < S::RUN; h <<= 1)
#pragma unroll
                    for (int i = 0; i + h < S::RUN; i += 2 * h) {
                        rr[i] += rr[i + h];
                        qq[i] += qq[i + h];
                    }
                r = fmax((double)rr[0] * c.iSt64 - F1 * ((double)qq[0] * c.iSt64), 0.0);
            } else {
                r = run_mass<DT, S::RUN>(lt, ld, c, resid);
#pragma unroll
                for (int i = 0; i < S::RUN; ++i) m[i] = (double)draw_mass32<DT>(lt[i], ld[i], c, resid) * c.iSt64;
            }
#pragma unroll
            for (int i = 0; i < S::RUN; ++i)
                if (m[i] > 0.0) lastpos = i0 + i;
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
                double qy;
                s_my = draw_mass64(lty, ldy, c, resid, qy);
                if (corr) s_my = fmax(s_my - F1 * qy, 0.0);
            }
        }
        __syncthreads();
        y = s_y;
        // Z relative to the target row's computed total; r_y / Z in one unit
        zrep = (float)(s_Z / s_P);
        py = (float)(kind == KIND_RESID && resid ? s_my / s_Z : s_my);
    } else if (kind == KIND_GREEDY) {
        y = f.y;
    } else {
        kind = KIND_BAD;
        y = -1;
    }
    const int a_out = kind == KIND_BAD ? 0 : a;

    for (int jj = tid; jj <= K; jj += kThreads) {
        int v = -1;
        if (y >= 0) v = jj < a_out ? (jj == tid ? tok0 : p.tok[(long long)b * K + jj]) : (jj == a_out ? y : -1);
        p.out_tok[(long long)b * (K + 1) + jj] = v;
    }
    // diagnostics of the rows the walk evaluated: lse of target rows 1..a+1,
    // of the draft rows read (the tested positions, and with an open length
    // walk every position up to L + 1), and the survivals
    if (!GREEDY && kind != KIND_BAD) {
        const int L = f.L;
        const bool open = (w.seq[b].flags & SEQ_OPEN) != 0;
        const int nd = OH ? 0 : (open ? min(L + 1, K) : min(a + 1, L));
        for (int jj = tid; jj <= K; jj += kThreads) {
            if (p.lse_t && jj <= a) p.lse_t[(long long)b * (K + 1) + jj] = (float)((double)w.row_m[rb + jj] * p.invT64 + log(w.row_s[rb + jj]));
            if (p.lse_d && jj < nd) p.lse_d[(long long)b * K + jj] = (float)((double)w.row_m[rb + K + 1 + jj] * p.invT64 + log(w.row_s[rb + K + 1 + jj]));
            if (p.surv && p.derived && !OH && open && jj < nd) p.surv[(long long)b * K + jj] = (float)w.srec[(long long)b * K + jj];
        }
        if (p.surv && p.derived && !OH && !open && tid == 0) {
            // verify length fixed at plan time (tau <= 0): S_j over the draft rows read
            double Sv = 1.0;
            for (int jj = 0; jj < nd; ++jj) {
                Sv = Sv / w.row_s[rb + K + 1 + jj];
                p.surv[(long long)b * K + jj] = (float)Sv;
            }
        }
    }
    // rows and bytes streamed for this sequence (splits marked by sv_plan)
    if (p.count) {
        double rows = 0.0, elems = 0.0;
        for (long long r = tid; r < R; r += kThreads) {
            int any = 0;
            for (int k = 0; k < p.nsplit; ++k)
                if (__float_as_uint(w.part_m[(rb + r) * p.nsplit + k]) != kUnread) {
                    any = 1;
                    elems += (double)min(kSplit, p.V - k * kSplit);
                }
            rows += any;
        }
        rows = block_sum(rows, s_cnt);
        elems = block_sum(elems, s_cnt);
        if (tid == 0) {
            if (p.rows_out) p.rows_out[b] = (int)rows;
            if (p.bytes_out) p.bytes_out[b] = (long long)elems * (DT == SV_BF16 ? 2 : 4);
        }
    }
    if (tid == 0) {
        p.acc_out[b] = a_out;
        p.vl_out[b] = f.L;
        if (p.zmass) p.zmass[b] = zrep;
        if (p.pys) p.pys[b] = py;
        int bits = 0;
        if (kind == KIND_BAD) bits |= (f.L < 0 && !(w.seq[b].flags & SEQ_BAD)) ? SV_STATUS_INCOMPLETE : SV_STATUS_BAD_INPUT;
        if (bits && p.status_out) or_status(p.status_out, bits);
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

const char* const kKernelNames[K_COUNT] = {"sv_plan", "sv_stream", "sv_resid", "sv_draw"};
constexpr int kMaxSlots = 64; // timed launches per run

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

int nsplit_of(int V) { return (V + kSplit - 1) / kSplit; }

// Carves the verify step's workspace for up to B sequences of up to K drafted
// positions over a vocabulary of ns splits out of base (NULL: sizes only).
// Returns the bytes it needs.
size_t carve_work(char* base, long long B, int K, int ns, Work* w)
{
    const long long R = 2LL * K + 1;
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        const size_t o = off;
        off = align_up(off + bytes);
        return base ? base + o : nullptr;
    };
    w->ctl = (int*)take(CTL_WORDS * sizeof(int));
    w->seq = (SeqCtl*)take((size_t)B * sizeof(SeqCtl));
    w->rcnt = (int*)take((size_t)(B * R) * sizeof(int));
    w->pcnt = (int*)take((size_t)(B * (K + 2)) * sizeof(int));
    w->dec = (int*)take((size_t)(B * (K + 1)) * sizeof(int));
    w->part_m = (float*)take((size_t)(B * R * ns) * sizeof(float));
    w->part_s = (double*)take((size_t)(B * R * ns) * sizeof(double));
    w->part_d = (float*)take((size_t)(B * R * ns) * sizeof(float));
    w->part_i = (int*)take((size_t)(B * R * ns) * sizeof(int));
    w->row_m = (float*)take((size_t)(B * R) * sizeof(float));
    w->row_s = (double*)take((size_t)(B * R) * sizeof(double));
    w->row_g = (int*)take((size_t)(B * R) * sizeof(int));
    w->xlog = (float*)take((size_t)(B * R) * sizeof(float));
    w->srec = (double*)take((size_t)(B * K) * sizeof(double));
    w->seg = (double*)take((size_t)(B * ns * kSegStride) * sizeof(double));
    w->segq = (double*)take((size_t)(B * ns * kSegStride) * sizeof(double));
    w->kp = (double*)take((size_t)(B * ns * kParts * kKpStride) * sizeof(double));
    return off;
}

} // namespace

// Workspace of spec_verify_run_noalloc: one copy per device, loaded with the
// code object and held until the process ends.  Host code never passes this
// name to a kernel or a copy (on the host it is only a stand-in for the
// symbol): it uses the device address hipGetSymbolAddress returns for the
// current device.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

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

// Launches kernel on stream s with block threads per workgroup and returns the
// launch's own status.  With start and stop events the events are attached to
// the dispatch itself (hipExtLaunchKernel), so they time the kernel's
// execution and not the queue around it.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, hipEvent_t e0,
                         hipEvent_t e1, Args... args)
{
    std::tuple<KArgs...> t(args...);
    void* a[sizeof...(KArgs)];
    std::apply([&](auto&... x) {
        int i = 0;
        ((a[i++] = (void*)&x), ...);
    }, t);
    if (e0) return hipExtLaunchKernel((const void*)kernel, grid, block, a, shmem, s, e0, e1, 0);
    return hipLaunchKernel((const void*)kernel, grid, block, a, shmem, s);
}

// Launches the kernels of a step; while per-kernel timing is on, each launch
// carries its own start and stop events.  Keeps the first failing status.
struct StepLauncher {
    const spec_verify* h;
    hipStream_t s;
    bool timing;
    int slot;
    hipError_t err;
    template <typename F, typename... Args>
    void operator()(int k, F kernel, dim3 grid, uint32_t shmem, Args... args)
    {
        if (err != hipSuccess) return;
        hipEvent_t e0 = nullptr, e1 = nullptr;
        if (timing && slot < kMaxSlots) {
            const int idx = h->timing_n * kMaxSlots + slot;
            e0 = h->ev[idx * 2];
            e1 = h->ev[idx * 2 + 1];
            h->ev_kernel[idx] = k;
            ++slot;
        }
        err = launch_kernel(kernel, grid, dim3(kThreads), shmem, s, e0, e1, args...);
    }
};

// One verification step on stream s: plan, the row statistics with in-launch
// decisions (one launch per kChunkPos positions), the residual masses, and the
// final draw.
template <int DT, bool VEC, bool GR, int MODE, typename Launch>
void enqueue_step(const Params& p, const Work& w, hipStream_t s, Launch& launch)
{
    constexpr bool OH = (MODE & MODE_ONEHOT) != 0;
    constexpr unsigned SLOTS = (GR || OH) ? 1u : 2u;
    const unsigned B = (unsigned)p.B, ns = (unsigned)p.nsplit;
    const unsigned long long R = 2ull * p.K + 1;
    launch(K_PLAN, sv_plan_kernel, dim3((unsigned)((B * R + kThreads - 1) / kThreads)), 0, p, w);
    // positions 1 .. Lmax + 1: a bounded call's later positions need no row
    const int Lmax = p.lbound ? p.lbound : p.K;
    for (int j0 = 1; j0 <= Lmax + 1; j0 += kChunkPos) {
        const unsigned np = (unsigned)std::min(kChunkPos, Lmax + 2 - j0);
        launch(K_STREAM, sv_stream_kernel<DT, VEC, GR, MODE>, dim3(np * B * SLOTS * ns), 0, p, w, j0);
    }
    if constexpr (!GR && !OH)
        launch(K_RESID, sv_resid_kernel<DT, VEC, MODE>, dim3(B * ns * kParts), 0, p, w);
    launch(K_DRAW, sv_draw_kernel<DT, VEC, GR, MODE>, dim3(B), (uint32_t)(ns * Seg<DT>::SEGS * sizeof(double)), p, w);
}

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

int check_config(const spec_verify_config* cfg)
{
    if (!cfg) return SV_EINVAL;
    if (cfg->max_batch < 1 || cfg->max_batch > SV_MAX_BATCH) return SV_EINVAL;
    if (cfg->max_draft < 1 || cfg->max_draft > SV_MAX_DRAFT) return SV_EINVAL;
    if (cfg->vocab < 1 || cfg->vocab > SV_MAX_VOCAB) return SV_EINVAL;
    if (cfg->dtype != SV_F32 && cfg->dtype != SV_BF16) return SV_EUNSUPPORTED;
    if (cfg->device < 0) return SV_EINVAL;
    // A launch's work-item count must fit in 32 bits.  The largest launches:
    // sv_stream over a chunk of positions (at most min(kChunkPos, K + 1), a
    // target and a draft row each), sv_resid and sv_plan.
    const long long ns = nsplit_of(cfg->vocab);
    const long long gmax = std::min(kChunkPos, cfg->max_draft + 1);
    const long long rows_wg = (long long)cfg->max_batch * 2 * gmax * ns;
    const long long resid_wg = (long long)cfg->max_batch * ns * kParts;
    if (std::max(rows_wg, resid_wg) * kThreads > 0xffffffffll) return SV_EUNSUPPORTED;
    return SV_OK;
}

// Fills the kernels' parameters of one call (after spec_verify_check).
Params make_params(const spec_verify_config* cfg, const spec_verify_args* a)
{
    const bool greedy = !(a->temperature > 0.0f);
    Params p;
    memset(&p, 0, sizeof(p));
    p.B = a->B;
    p.K = a->K;
    p.V = cfg->vocab;
    p.nsplit = nsplit_of(cfg->vocab);
    p.greedy = greedy;
    p.len_mode = a->length_mode;
    p.lbound = a->max_verify_len;
    p.derived = (a->length_mode == SV_LEN_TAU && !a->confidence) ? 1 : 0;
    p.onehot = (!greedy && a->draft_mode == SV_DRAFT_ONEHOT) ? 1 : 0;
    p.count = (a->rows_read || a->bytes_read) ? 1 : 0;
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
    p.bytes_out = (long long*)a->bytes_read;
    p.status_out = a->device_status;
    return p;
}

// Enqueues one checked call's kernels with workspace w.
template <typename Launch>
void enqueue_call(const spec_verify_config* cfg, const spec_verify_args* a, const Work& w, hipStream_t s,
                  Launch& launch)
{
    const Params p = make_params(cfg, a);
    const bool vec = args_vec_ok(cfg, a);
    const int mode = (p.onehot ? MODE_ONEHOT : 0) | (p.toff ? MODE_PACKED : 0);
    // runtime choices -> kernel variants (greedy steps never take the one-hot variant)
#define SV_STEP(DT, VEC, GR, M) enqueue_step<DT, VEC, GR, M>(p, w, s, launch)
#define SV_STEP_M(DT, VEC, GR) do { switch (GR ? (mode & MODE_PACKED) : mode) { \
        case 0: SV_STEP(DT, VEC, GR, 0); break; case 1: SV_STEP(DT, VEC, GR, 1); break; \
        case 2: SV_STEP(DT, VEC, GR, 2); break; default: SV_STEP(DT, VEC, GR, 3); break; } } while (0)
    if (cfg->dtype == SV_BF16) {
        if (vec) { if (p.greedy) SV_STEP_M(SV_BF16, true, true); else SV_STEP_M(SV_BF16, true, false); }
        else { if (p.greedy) SV_STEP_M(SV_BF16, false, true); else SV_STEP_M(SV_BF16, false, false); }
    } else {
        if (vec) { if (p.greedy) SV_STEP_M(SV_F32, true, true); else SV_STEP_M(SV_F32, true, false); }
        else { if (p.greedy) SV_STEP_M(SV_F32, false, true); else SV_STEP_M(SV_F32, false, false); }
    }
#undef SV_STEP_M
#undef SV_STEP
}

// Device address of the scratch array on device dev (the current device),
// looked up on the first call for that device and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices) return SV_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SV_EDEVICE;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SV_OK;
}

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
    if (a->max_verify_len < 0 || a->max_verify_len > a->K) return SV_EINVAL;
    if (a->max_verify_len && a->length_mode != SV_LEN_FIXED) return SV_EINVAL;
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
    const size_t verify_bytes = carve_work(nullptr, cfg->max_batch, cfg->max_draft, h->nsplit, &h->w);
    size_t off = align_up(verify_bytes);
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
    carve_work(base, cfg->max_batch, cfg->max_draft, h->nsplit, &h->w);
    h->aux.ctl = h->w.ctl;
    h->aux.sched_s = (double*)(base + o_ss);
    h->aux.sched_rank = (int*)(base + o_sr);
    h->aux.sched_sorted = (double*)(base + o_so);
    h->aux.conf_ring = conf_ok ? (float*)(base + o_cr) : nullptr;
    h->aux.conf_head = conf_ok ? (int*)(base + o_ch) : nullptr;
    h->aux.conf_count = conf_ok ? (int*)(base + o_cc) : nullptr;
    h->aux.conf_K = cfg->max_draft;
    // control words (status bits of the admission and confidence calls) start at
    // zero; each call clears what it reports; the confidence history starts empty
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
    hipError_t e = launch_kernel(sv_conf_kernel, dim3(a->B), dim3(kThreads), 0, s, nullptr, nullptr, q, h->aux);
    if (e == hipSuccess) e = launch_kernel(sv_conf_status_kernel, dim3(1), dim3(64), 0, s, nullptr, nullptr, q, h->aux);
    return e == hipSuccess ? SV_OK : SV_EDEVICE;
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
    hipError_t e = launch_kernel(sv_sched_surv_kernel, dim3((a->B + kThreads - 1) / kThreads), dim3(kThreads), 0, s,
                                 nullptr, nullptr, q, h->aux);
    if (e == hipSuccess) e = launch_kernel(sv_sched_rank_kernel, dim3(N), dim3(kThreads), 0, s, nullptr, nullptr, q, h->aux);
    if (e == hipSuccess)
        e = launch_kernel(sv_sched_pick_kernel, dim3(1), dim3(kSchedThreads), 0, s, nullptr, nullptr, q, h->aux);
    return e == hipSuccess ? SV_OK : SV_EDEVICE;
}

int spec_verify_run(spec_verify_t* h, const spec_verify_args* a, void* hip_stream)
{
    if (!h) return SV_EINVAL;
    int rc = spec_verify_check(&h->cfg, a);
    if (rc != SV_OK) return rc;
    if (a->B == 0) return SV_OK;
    DeviceGuard guard(h->cfg.device);
    const bool timing = h->ev && h->timing_n < h->timing_max;
    StepLauncher launch{h, (hipStream_t)hip_stream, timing, 0, hipSuccess};
    enqueue_call(&h->cfg, a, h->w, (hipStream_t)hip_stream, launch);
    if (timing) h->timing_n++;
    return launch.err == hipSuccess ? SV_OK : SV_EDEVICE;
}

int spec_verify_run_noalloc(const spec_verify_config* cfg, const spec_verify_args* a, void* hip_stream)
{
    int rc = spec_verify_check(cfg, a);
    if (rc != SV_OK) return rc;
    if (a->B == 0) return SV_OK;
    // the workspace of this call's B, K and vocabulary, carved from the array
    const int ns = nsplit_of(cfg->vocab);
    Work w;
    if (carve_work(nullptr, a->B, a->K, ns, &w) > (size_t)SV_NOALLOC_SCRATCH_BYTES) return SV_EUNSUPPORTED;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device >= ndev) return SV_EDEVICE;
    DeviceGuard guard(cfg->device);
    void* base = nullptr;
    rc = scratch_address(cfg->device, &base);
    if (rc != SV_OK) return rc;
    carve_work((char*)base, a->B, a->K, ns, &w);
    // sv_plan clears the counters and status words the step needs at zero
    // (a kernel, not a memset); nothing else is read before it is written
    StepLauncher launch{nullptr, (hipStream_t)hip_stream, false, 0, hipSuccess};
    enqueue_call(cfg, a, w, (hipStream_t)hip_stream, launch);
    return launch.err == hipSuccess ? SV_OK : SV_EDEVICE;
}

} // extern "C"
