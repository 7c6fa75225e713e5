// Device-side building blocks shared by the verification kernels (gfx950).
//
// Layout conventions: a logit row is V contiguous elements (float32, or
// bfloat16 bit patterns).  A workgroup of kThreads threads streams an element
// range of one row with 16-byte vector loads (4 fp32 or 8 bf16 elements per
// load; consecutive threads read consecutive 16-byte vectors, so every wave
// load instruction moves one contiguous KiB).  Elements before the first
// 16-byte boundary and after the last one are read one at a time.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cfloat>
#include <cmath>

#include "sv_kernels.hpp"

namespace sv {

constexpr int kThreads = 256;          // threads per workgroup (4 wave64s)
constexpr int kWaves = kThreads / 64;  // waves per workgroup

// Element traits: storage type and unpacking of one 16-byte vector.
struct F32 {
    using storage = float;
    static constexpr int kPerVec = 4;
    __device__ static inline float one(const storage* p) { return *p; }
    __device__ static inline void unpack(const uint4& v, float* x) {
        x[0] = __uint_as_float(v.x);
        x[1] = __uint_as_float(v.y);
        x[2] = __uint_as_float(v.z);
        x[3] = __uint_as_float(v.w);
    }
};

struct BF16 {
    using storage = uint16_t;
    static constexpr int kPerVec = 8;
    __device__ static inline float one(const storage* p) {
        return __uint_as_float(static_cast<uint32_t>(*p) << 16);
    }
    // A bf16 value is the top half of a float32; the lower address holds the
    // lower 16 bits of each 32-bit word (little endian).
    __device__ static inline void unpack(const uint4& v, float* x) {
        x[0] = __uint_as_float(v.x << 16);
        x[1] = __uint_as_float(v.x & 0xffff0000u);
        x[2] = __uint_as_float(v.y << 16);
        x[3] = __uint_as_float(v.y & 0xffff0000u);
        x[4] = __uint_as_float(v.z << 16);
        x[5] = __uint_as_float(v.z & 0xffff0000u);
        x[6] = __uint_as_float(v.w << 16);
        x[7] = __uint_as_float(v.w & 0xffff0000u);
    }
};

// Split of an element range [e0, e1) of a row into a scalar head, a body of
// whole 16-byte vectors and a scalar tail, from the actual addresses.
template <class E>
struct RangeSplit {
    int head_begin, head_end;  // scalar elements [head_begin, head_end)
    int body_begin;            // first element of the vector body
    int nvec;                  // number of 16-byte vectors in the body
    int tail_begin, tail_end;  // scalar elements [tail_begin, tail_end)
};

template <class E>
__device__ inline RangeSplit<E> split_range(const typename E::storage* row, int e0, int e1) {
    using S = typename E::storage;
    RangeSplit<E> r;
    const uintptr_t a = reinterpret_cast<uintptr_t>(row + e0);
    int head = static_cast<int>(((16u - (a & 15u)) & 15u) / sizeof(S));
    const int len = e1 - e0;
    if (head > len) head = len;
    r.head_begin = e0;
    r.head_end = e0 + head;
    r.body_begin = e0 + head;
    r.nvec = (len - head) / E::kPerVec;
    r.tail_begin = r.body_begin + r.nvec * E::kPerVec;
    r.tail_end = e1;
    return r;
}

// Plain 16-byte load that the compiler may schedule freely.
__device__ inline uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming 16-byte load: the logits are read exactly once, so the load is
// marked non-temporal and does not displace reusable lines in the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline uint4 load16_stream(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Streams the 16-byte vectors [0, nvec) of `body` through f.  Batches of U
// vectors per thread (kThreads*U per workgroup) are software-pipelined: the
// loads of batch t+1 are issued before batch t is folded, and every load is
// unconditional, so the only wait before a fold is for that batch's own
// loads.  The fewer than kThreads*U vectors left after the whole batches are
// loaded before the last whole batch is folded (a thread whose index falls
// past the end re-reads the final vector and discards it).
//
// f.template batch<N>(const uint4* v, int v0) folds N vectors; vector u of
// the call is body vector v0 + u*kThreads.
template <int U, class F>
__device__ inline void stream_vectors(const char* body, int nvec, F& f) {
    if (nvec <= 0) return;
    const int tid = threadIdx.x;
    constexpr int kBatch = kThreads * U;
    const int nb = nvec / kBatch;
    const int rest0 = nb * kBatch;
    uint4 rest[U];
    if (nb > 0) {
        uint4 cur[U];
#pragma unroll
        for (int u = 0; u < U; ++u) cur[u] = load16_stream(body + static_cast<size_t>(u * kThreads + tid) * 16);
        for (int t = 0; t + 1 < nb; ++t) {
            uint4 nxt[U];
            const char* nbp = body + static_cast<size_t>(t + 1) * kBatch * 16;
#pragma unroll
            for (int u = 0; u < U; ++u) nxt[u] = load16_stream(nbp + static_cast<size_t>(u * kThreads + tid) * 16);
            f.template batch<U>(cur, t * kBatch + tid);
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = min(rest0 + u * kThreads + tid, nvec - 1);
            rest[u] = load16_stream(body + static_cast<size_t>(v) * 16);
        }
        f.template batch<U>(cur, (nb - 1) * kBatch + tid);
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = min(u * kThreads + tid, nvec - 1);
            rest[u] = load16_stream(body + static_cast<size_t>(v) * 16);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int v = rest0 + u * kThreads + tid;
        if (v < nvec) f.template batch<1>(&rest[u], v);
    }
}

// ---------------------------------------------------------------------------
// Row statistics of a temperature softmax, kept as (m, R, S):
//   m  the largest logit seen (for the domain check),
//   R  an integer-valued float with R >= (approximately) max z*c,
//   S  sum over the seen elements of 2^(z*c - R), in fp64,
// where c = log2(e)/T is carried as c_hi + c_lo (two floats, so z*c is
// effectively exact).  Because R is an integer, moving S to a larger R' is an
// exact multiplication by 2^(R - R'), so partial sums from different lanes,
// waves and workgroups merge without rounding in the rescale.  The row's
// log2-sum-exp is then R + log2(S) in units of log2, i.e.
//   log2 p(v) = z_v*c - (R + log2 S).
__device__ inline Stat stat_empty() { return Stat{-INFINITY, -FLT_MAX, 0.0}; }

__device__ inline int rescale_exponent(float from, float to) {
    // from <= to; clamp so that the conversion is defined even when "from" is
    // the -FLT_MAX start value (the scaled sum is then 0 anyway).
    float d = fmaxf(from - to, -2000.0f);
    return static_cast<int>(d);
}

__device__ inline Stat stat_merge(const Stat& a, const Stat& b) {
    Stat r;
    r.m = fmaxf(a.m, b.m);
    r.R = fmaxf(a.R, b.R);
    r.S = ldexp(a.S, rescale_exponent(a.R, r.R)) + ldexp(b.S, rescale_exponent(b.R, r.R));
    return r;
}

// Pairwise sum of N floats, to keep the fp32 rounding of one batch at
// ceil(log2 N) steps: each step adds element i + ceil(n/2) to element i of
// the n still to be summed (for N a power of two, element i + n/2; an odd
// count carries its middle element to the next step).
template <int N>
__device__ inline float pairwise_sum(float* v) {
#pragma unroll
    for (int n = N; n > 1; n = (n + 1) / 2) {
        const int off = (n + 1) / 2;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) v[i] = v[i] + v[i + off];
    }
    return v[0];
}

// Fold a batch of N logits into the running statistics.  One max per
// element, one integer-aligned reference update per batch, then for each
// element t = z*c_hi - R + z*c_lo (two fused multiply-adds, the subtraction
// of R exact inside the first) and 2^t on the hardware exp2 unit; the batch
// sum is pairwise in fp32 and accumulated in fp64.
// stat_fold_max takes the batch maximum lm from the caller.
template <int N>
__device__ inline void stat_fold_max(Stat& s, const float* x, float lm, float c_hi, float c_lo) {
    const float Rn = fmaxf(s.R, ceilf(lm * c_hi));
    s.S = ldexp(s.S, rescale_exponent(s.R, Rn));
    s.R = Rn;
    s.m = fmaxf(s.m, lm);
    float e[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float t = fmaf(x[i], c_hi, -Rn);
        t = fmaf(x[i], c_lo, t);
        e[i] = __builtin_amdgcn_exp2f(t);
    }
    s.S += static_cast<double>(pairwise_sum<N>(e));
}

template <int N>
__device__ inline void stat_fold(Stat& s, const float* x, float c_hi, float c_lo) {
    float lm = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) lm = fmaxf(lm, x[i]);
    stat_fold_max<N>(s, x, lm, c_hi, c_lo);
}

// ---------------------------------------------------------------------------
// Wave64 and workgroup reductions.

template <class T>
__device__ inline T wave_xor(T v, int mask) {
    return __shfl_xor(v, mask, 64);
}

// DPP lane moves (the move is one VALU operand modifier, no LDS round trip).
// Lanes the move leaves out (rows outside ROWS, or a source past the row's
// edge when BOUND is set) receive `old`.
template <int CTRL, int ROWS, bool BOUND>
__device__ inline double dpp_f64(double x, double old) {
    const int lo = __builtin_amdgcn_update_dpp(__double2loint(old), __double2loint(x), CTRL, ROWS,
                                               0xf, BOUND);
    const int hi = __builtin_amdgcn_update_dpp(__double2hiint(old), __double2hiint(x), CTRL, ROWS,
                                               0xf, BOUND);
    return __hiloint2double(hi, lo);
}
template <int CTRL, int ROWS, bool BOUND>
__device__ inline float dpp_f32(float x, float old) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL,
                                                      ROWS, 0xf, BOUND));
}
__device__ inline double readlane_f64(double x, int l) {
    const int lo = __builtin_amdgcn_readlane(__double2loint(x), l);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(x), l);
    return __hiloint2double(hi, lo);
}

// One combining step of a wave-wide reduction: quad swaps, then half-row and
// row mirrors leave every lane with its row's total; the row broadcasts
// (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3) carry the
// totals up to lane 63.
template <int CTRL, int ROWS>
__device__ inline Stat dpp_stat(const Stat& s) {
    Stat o;
    o.m = dpp_f32<CTRL, ROWS, false>(s.m, -INFINITY);  // (the empty statistic elsewhere)
    o.R = dpp_f32<CTRL, ROWS, false>(s.R, -FLT_MAX);
    o.S = dpp_f64<CTRL, ROWS, false>(s.S, 0.0);
    return o;
}

// The merge of the wave's statistics; every lane gets it.
__device__ inline Stat wave_reduce_stat(Stat s) {
    s = stat_merge(s, dpp_stat<0xb1, 0xf>(s));   // quad_perm [1,0,3,2]
    s = stat_merge(s, dpp_stat<0x4e, 0xf>(s));   // quad_perm [2,3,0,1]
    s = stat_merge(s, dpp_stat<0x141, 0xf>(s));  // row_half_mirror
    s = stat_merge(s, dpp_stat<0x140, 0xf>(s));  // row_mirror
    s = stat_merge(s, dpp_stat<0x142, 0xa>(s));  // row_bcast:15
    s = stat_merge(s, dpp_stat<0x143, 0xc>(s));  // row_bcast:31
    Stat r;
    r.m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s.m), 63));
    r.R = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s.R), 63));
    r.S = readlane_f64(s.S, 63);
    return r;
}

// A DPP move whose lanes outside ROWS are left undefined (no old value to
// initialise), for reductions that read only lanes the pattern defines.
template <int CTRL, int ROWS>
__device__ inline double dpp_f64_any(double x) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(x), CTRL, ROWS, 0xf, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(x), CTRL, ROWS, 0xf, false);
    return __hiloint2double(hi, lo);
}

// The sum of the wave's values; every lane gets it.  Only lane 63's partial
// is read: after the row steps every lane holds its row's sum, the two
// broadcasts leave row 3 with rows 0-3 (rows 0-2 hold values nobody reads,
// so the lanes the broadcasts skip need no defined old value).
__device__ inline double wave_sum(double v) {
    v += dpp_f64_any<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
    v += dpp_f64_any<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
    v += dpp_f64_any<0x141, 0xf>(v);  // row_half_mirror
    v += dpp_f64_any<0x140, 0xf>(v);  // row_mirror
    v += dpp_f64_any<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_f64_any<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return readlane_f64(v, 63);
}

// Workgroup-wide merge of one Stat per thread; every thread gets the result.
// Uses kWaves Stats of LDS and is safe to call repeatedly (it synchronises
// before reusing the LDS slots).
__device__ inline Stat block_reduce_stat(Stat st, Stat* lds_waves) {
    st = wave_reduce_stat(st);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) lds_waves[wave] = st;
    __syncthreads();
    Stat r = lds_waves[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = stat_merge(r, lds_waves[w]);
    return r;
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele within
// each row of 16 lanes (row_shr by 1, 2, 4, 8, zero past the row's start),
// then the row broadcasts add the earlier rows' totals.
__device__ inline double wave_inclusive_scan(double v) {
    v += dpp_f64<0x111, 0xf, true>(v, 0.0);  // row_shr:1
    v += dpp_f64<0x112, 0xf, true>(v, 0.0);  // row_shr:2
    v += dpp_f64<0x114, 0xf, true>(v, 0.0);  // row_shr:4
    v += dpp_f64<0x118, 0xf, true>(v, 0.0);  // row_shr:8
    v += dpp_f64<0x142, 0xa, false>(v, 0.0); // row_bcast:15 into rows 1 and 3
    v += dpp_f64<0x143, 0xc, false>(v, 0.0); // row_bcast:31 into rows 2 and 3
    return v;
}

// Workgroup-wide exclusive prefix sum of one double per thread, in thread
// order; also returns the total.  Uses kWaves doubles of LDS.
__device__ inline double block_exclusive_scan(double v, double* lds_waves, double* total) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    double incl = wave_inclusive_scan(v);
    __syncthreads();
    if (lane == 63) lds_waves[wave] = incl;
    __syncthreads();
    double base = 0.0, all = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        double t = lds_waves[w];
        if (w < wave) base += t;
        all += t;
    }
    *total = all;
    return base + incl - v;
}

__device__ inline double block_sum(double v, double* lds_waves) {
    double t;
    block_exclusive_scan(v, lds_waves, &t);
    return t;
}

// Workgroup-wide min / max of one int per thread (every thread gets it).
__device__ inline int block_min_int(int v, int* lds) {
    __syncthreads();
    if (threadIdx.x == 0) *lds = INT32_MAX;
    __syncthreads();
    atomicMin(lds, v);
    __syncthreads();
    return *lds;
}

__device__ inline int block_max_int(int v, int* lds) {
    __syncthreads();
    if (threadIdx.x == 0) *lds = INT32_MIN;
    __syncthreads();
    atomicMax(lds, v);
    __syncthreads();
    return *lds;
}

// Launch of a kernel on `s`, optionally bracketed by events that the launch
// itself records at the kernel's start and end.
template <class K, class... Args>
inline hipError_t launch_timed(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                               hipEvent_t ev_start, hipEvent_t ev_stop, Args... args) {
    if (ev_start && ev_stop)
        hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(lds), s, ev_start, ev_stop,
                              0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Candidate keys and wave-wide maxima (outcome scoring, tree construction).

// Candidate keys: unsigned 64-bit integers ordered like the candidates
// (value descending, then index ascending).  The high word maps the float
// value monotonically (-0 counts as +0, as in a float comparison), the low
// word is 0xffffffff - index.  Key 0 is below every real key and means none.
__device__ inline uint32_t value_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_value(uint64_t k) {
    const uint32_t u = static_cast<uint32_t>(k >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u ^ 0x80000000u) : ~u);
}
__device__ inline uint64_t make_key(float v, uint32_t idx) {
    return (static_cast<uint64_t>(value_key(v)) << 32) | (0xffffffffu - idx);
}
__device__ inline uint32_t key_index(uint64_t k) { return 0xffffffffu - static_cast<uint32_t>(k); }

__device__ inline uint64_t readlane64(uint64_t x, int l) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(x), l);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(x >> 32), l);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ inline uint64_t uniform64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<int>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<int>(x >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// (score desc, index asc) order of scored candidates with distinct indices.
__device__ inline bool cand_ahead(double s1, int i1, double s2, int i2) {
    return s1 > s2 || (s1 == s2 && s1 > -INFINITY && i1 < i2);
}

// One step of a wave-wide maximum over DPP lane moves (lanes outside the
// move keep their own value).
template <int CTRL, int ROWS>
__device__ inline void dpp_max_step(double& s, int& i) {
    const int lo = __double2loint(s), hi = __double2hiint(s);
    const int olo = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xf, false);
    const int ohi = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xf, false);
    const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, ROWS, 0xf, false);
    const double os = __hiloint2double(ohi, olo);
    const bool take = (os > s) | ((os == s) & (os > -INFINITY) & (oi < i));  // as cand_ahead
    s = take ? os : s;
    i = take ? oi : i;
}

// The wave's best (score, i); every lane gets it.  Quad swaps, half-row and
// row mirrors leave each row of 16 lanes with its best, the two row
// broadcasts carry it to lane 63.
__device__ inline void wave_best(double& s, int& i) {
    dpp_max_step<0xb1, 0xf>(s, i);   // quad_perm [1,0,3,2]
    dpp_max_step<0x4e, 0xf>(s, i);   // quad_perm [2,3,0,1]
    dpp_max_step<0x141, 0xf>(s, i);  // row_half_mirror
    dpp_max_step<0x140, 0xf>(s, i);  // row_mirror
    dpp_max_step<0x142, 0xa>(s, i);  // row_bcast:15 into rows 1 and 3
    dpp_max_step<0x143, 0xc>(s, i);  // row_bcast:31 into rows 2 and 3
    const int lo = __builtin_amdgcn_readlane(__double2loint(s), 63);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(s), 63);
    i = __builtin_amdgcn_readlane(i, 63);
    s = __hiloint2double(hi, lo);
}

// The largest 64-bit key over the wave (same lane moves as wave_best).
template <int CTRL, int ROWS>
__device__ inline void dpp_max_step_u64(uint64_t& x) {
    const int lo = static_cast<int>(x), hi = static_cast<int>(x >> 32);
    const uint32_t olo = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xf, false);
    const uint32_t ohi = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xf, false);
    const uint64_t o = (static_cast<uint64_t>(ohi) << 32) | olo;
    x = o > x ? o : x;
}
__device__ inline uint64_t wave_max_u64(uint64_t x) {
    dpp_max_step_u64<0xb1, 0xf>(x);
    dpp_max_step_u64<0x4e, 0xf>(x);
    dpp_max_step_u64<0x141, 0xf>(x);
    dpp_max_step_u64<0x140, 0xf>(x);
    dpp_max_step_u64<0x142, 0xa>(x);
    dpp_max_step_u64<0x143, 0xc>(x);
    return readlane64(x, 63);
}


// ---------------------------------------------------------------------------
// Tree paths by pointer jumping (greedy and stochastic tree verification).
// On entry, for every node j < n: s_anc[j] its parent (root: 0), s_dep[j] = 1
// (root: 0), s_ok[j] whether the edge into j passes its test (root: 1), and
// *s_key = -1.  After ceil(log2 n) rounds s_anc[j] is the root, s_dep[j] the
// depth and s_ok[j] whether every edge on the path passed; *s_key then holds
// (depth << 11) | (2047 - index) of the deepest such node, the lowest index
// among equally deep ones.  All threads of the workgroup call it (n <= 1024,
// at most kMaxTreeNodes / kThreads nodes per thread).
__device__ inline void deepest_accepted(int n, int* s_anc, int* s_dep, unsigned char* s_ok,
                                        int* s_key) {
    constexpr int kPer = kMaxTreeNodes / kThreads;
    const int tid = threadIdx.x;
    for (int span = 1; span < n; span <<= 1) {
        int nanc[kPer], ndep[kPer];
        unsigned char nok[kPer];
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int j = tid + m * kThreads;
            if (j < n) {
                const int up = s_anc[j];
                nok[m] = s_ok[j] & s_ok[up];
                ndep[m] = s_dep[j] + s_dep[up];
                nanc[m] = s_anc[up];
            }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int j = tid + m * kThreads;
            if (j < n) {
                s_ok[j] = nok[m];
                s_dep[j] = ndep[m];
                s_anc[j] = nanc[m];
            }
        }
        __syncthreads();
    }
    for (int j = tid; j < n; j += kThreads)
        if (s_ok[j]) atomicMax(s_key, (s_dep[j] << 11) | (2047 - j));
    __syncthreads();
}

}  // namespace sv
