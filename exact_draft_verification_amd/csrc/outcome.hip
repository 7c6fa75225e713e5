// Outcome scoring and cache selection for gfx950.
//
// What is computed ("JetSpec++", Section 4.2 "Outcome Selection", and
// Appendix F.1 with Proposition 1): row j (j = 0..gamma) of a request is the
// decoder's next-token logits after the block's first j draft tokens; with
// p_j = softmax(row_j / T) and x_j the draft tokens, the outcome (k, a) --
// k accepted tokens, then extra token a -- has probability
//   P(k, a) = prod_{i<k} p_i(x_i) * p_k(a)   (k < gamma, a != x_k),
//   P(gamma, a) = prod_{i<gamma} p_i(x_i) * p_gamma(a).
// The cache keeps the ncache most probable outcomes (ties: smaller k, then
// smaller a); its hit probability is the sum of their probabilities.
//
// Within a row the order of P(k, .) is the order of the logits, so the
// candidates are found in the same single pass over the logits that takes
// the softmax statistics:
//  1. outcome_stats: one workgroup per (request, row, segment) folds (m, R, S)
//     as the chain statistics do and keeps the KB largest logits of the
//     segment (lowest token id first among equal ones), the row's draft token
//     excluded.  Each thread holds an exact sorted list of its own KB best; a
//     workgroup-wide threshold in LDS -- the largest of the threads' KB-th
//     values, a lower bound of the workgroup's KB-th best -- filters the
//     stream so that insertions stay rare.  The lists are merged by KB
//     rounds of a workgroup-wide maximum.
//  2. outcome_select: one workgroup per request merges the row statistics,
//     forms A_k = sum_{i<k} log2 p_i(x_i) by a prefix sum, scores every
//     candidate in fp64 as log2 P = A_k + z*c - L_k and keeps the ncache best.
#include "sv_device.hpp"

namespace sv {

namespace {

constexpr double kDomain = 268435456.0;  // |m| / T limit (2^28)
constexpr float kNegInf = -INFINITY;

// Total order of floats as signed ints (larger float, larger key).
__device__ inline int order_key(float f) {
    const int i = __float_as_int(f);
    return i >= 0 ? i : i ^ 0x7fffffff;
}
__device__ inline float key_float(int k) { return __int_as_float(k >= 0 ? k : k ^ 0x7fffffff); }

// (value desc, index asc): is (v, i) ahead of (w, j)?
__device__ inline bool ahead(float v, int i, float w, int j) { return v > w || (v == w && i < j); }

template <class E, int KB>
struct TopFolder {
    Stat s;
    float c_hi, c_lo;
    float val[KB];
    int id[KB];
    int excl;          // the row's draft token (not an outcome), or -1
    int body_begin;    // element index of body vector 0
    int* s_theta;      // workgroup threshold (order key)

    // Insert (z, e) into the sorted list; the caller has checked that it
    // beats the KB-th entry (elements reach a thread in increasing index, so
    // an equal value never displaces an earlier one).
    __device__ inline void insert(float z, int e) {
        float v = z;
        int ix = e;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            const bool b = ahead(v, ix, val[j], id[j]);
            const float tv = b ? val[j] : v;
            const int ti = b ? id[j] : ix;
            val[j] = b ? v : val[j];
            id[j] = b ? ix : id[j];
            v = tv;
            ix = ti;
        }
    }

    __device__ inline void offer(float z, int e, float theta) {
        if (z > val[KB - 1] && z >= theta && e != excl) insert(z, e);
    }

    template <int N>
    __device__ inline void batch(const uint4* v, int v0) {
        float x[N * E::kPerVec];
#pragma unroll
        for (int u = 0; u < N; ++u) E::unpack(v[u], x + u * E::kPerVec);
        stat_fold<N * E::kPerVec>(s, x, c_hi, c_lo);
        const float theta = key_float(*s_theta);
        // the batch max is cheap to test before any per-element work
        float bm = x[0];
#pragma unroll
        for (int i = 1; i < N * E::kPerVec; ++i) bm = fmaxf(bm, x[i]);
        if (bm > val[KB - 1] && bm >= theta) {
#pragma unroll
            for (int u = 0; u < N; ++u)
#pragma unroll
                for (int w = 0; w < E::kPerVec; ++w)
                    offer(x[u * E::kPerVec + w], body_begin + (v0 + u * kThreads) * E::kPerVec + w,
                          theta);
            if (val[KB - 1] > kNegInf) atomicMax(s_theta, order_key(val[KB - 1]));
        }
    }
};

template <class E, int U, int KB>
__global__ __launch_bounds__(kThreads) void outcome_stats_kernel(OutcomeArgs a) {
    __shared__ Stat s_w[kWaves];
    __shared__ int s_theta;
    __shared__ float s_bv[kWaves];
    __shared__ int s_bi[kWaves];
    const int rows = a.gamma + 1;
    const int unit = blockIdx.x;
    const int seg = unit % a.nseg;
    const int rr = unit / a.nseg;  // r * rows + k
    const int k = rr % rows;
    const int r = rr / rows;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    using S = typename E::storage;
    const S* row = static_cast<const S*>(a.logits) + static_cast<int64_t>(rr) * a.V;
    const int e0 = seg * a.seg_len;
    const int e1 = min(a.V, e0 + a.seg_len);
    if (tid == 0) s_theta = order_key(kNegInf);
    int excl = -1;
    if (k < a.gamma) excl = a.tokens[static_cast<int64_t>(r) * a.gamma + k];
    // the draft token's logit, if this segment holds it
    float zx = 0.0f;
    const bool have_zx = tid == 0 && excl >= e0 && excl < e1;
    if (have_zx) zx = E::one(row + excl);
    __syncthreads();

    TopFolder<E, KB> f;
    f.s = stat_empty();
    f.c_hi = a.c_hi;
    f.c_lo = a.c_lo;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
        f.val[j] = kNegInf;
        f.id[j] = INT32_MAX;
    }
    f.excl = excl;
    f.s_theta = &s_theta;
    if (e0 < e1) {
        const RangeSplit<E> sp = split_range<E>(row, e0, e1);
        f.body_begin = sp.body_begin;
        for (int e = sp.head_begin + tid; e < sp.head_end; e += kThreads) {
            const float x = E::one(row + e);
            stat_fold<1>(f.s, &x, a.c_hi, a.c_lo);
            f.offer(x, e, kNegInf);
        }
        stream_vectors<U>(reinterpret_cast<const char*>(row + sp.body_begin), sp.nvec, f);
        for (int e = sp.tail_begin + tid; e < sp.tail_end; e += kThreads) {
            const float x = E::one(row + e);
            stat_fold<1>(f.s, &x, a.c_hi, a.c_lo);
            f.offer(x, e, kNegInf);
        }
    }
    const Stat st = block_reduce_stat(f.s, s_w);
    // KB rounds of a workgroup-wide maximum over the threads' list heads
    OutcomeCand* out = a.cand + static_cast<int64_t>(unit) * KB;
    for (int round = 0; round < KB; ++round) {
        float bv = f.val[0];
        int bi = f.id[0];
#pragma unroll
        for (int mask = 32; mask >= 1; mask >>= 1) {
            const float ov = __shfl_xor(bv, mask, 64);
            const int oi = __shfl_xor(bi, mask, 64);
            if (ahead(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        __syncthreads();
        if (lane == 0) {
            s_bv[wave] = bv;
            s_bi[wave] = bi;
        }
        __syncthreads();
        float wv = s_bv[0];
        int wi = s_bi[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            if (ahead(s_bv[w], s_bi[w], wv, wi)) {
                wv = s_bv[w];
                wi = s_bi[w];
            }
        if (tid == 0) out[round] = OutcomeCand{wv, wi};
        // the owner of the winning head pops it (token ids are unique)
        if (wi != INT32_MAX && f.id[0] == wi) {
#pragma unroll
            for (int j = 0; j + 1 < KB; ++j) {
                f.val[j] = f.val[j + 1];
                f.id[j] = f.id[j + 1];
            }
            f.val[KB - 1] = kNegInf;
            f.id[KB - 1] = INT32_MAX;
        }
    }
    if (tid == 0) {
        a.part[unit] = st;
        if (have_zx) a.zx[rr] = zx;
    }
}

// Per-request merge: row statistics, prefix of accepted-token log2
// probabilities, candidate scores and the ncache best outcomes.
__global__ __launch_bounds__(kThreads) void outcome_select_kernel(OutcomeArgs a) {
    extern __shared__ unsigned char s_dyn[];
    __shared__ double s_L[kMaxGamma + 1];
    __shared__ double s_A[kMaxGamma + 1];
    __shared__ double s_waves[kWaves];
    __shared__ int s_bad;
    __shared__ double s_bv[kWaves];
    __shared__ int s_bk[kWaves], s_ba[kWaves], s_bj[kWaves];
    const int r = blockIdx.x;
    const int g = a.gamma, rows = g + 1, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ncand = rows * a.nseg * a.kb;  // candidates of this request
    const int per_row = a.nseg * a.kb;                              // candidates per row
    double* c_score = reinterpret_cast<double*>(s_dyn);             // [ncand]
    int* c_tok = reinterpret_cast<int*>(c_score + ncand);           // [ncand]
    if (tid == 0) s_bad = 0;
    __syncthreads();
    // row statistics (one thread per row, its segments merged in order)
    for (int k = tid; k < rows; k += kThreads) {
        const Stat* p = a.part + (static_cast<int64_t>(r) * rows + k) * a.nseg;
        Stat t = p[0];
        for (int s = 1; s < a.nseg; ++s) t = stat_merge(t, p[s]);
        const bool ok = isfinite(t.S) && t.S > 0.0 && fabs(static_cast<double>(t.m) / a.T) <= kDomain;
        if (!ok) atomicOr(&s_bad, 1);
        s_L[k] = static_cast<double>(t.R) + log2(t.S);
        if (k < g) {
            const int x = a.tokens[static_cast<int64_t>(r) * g + k];
            if (x < 0 || x >= a.V) atomicOr(&s_bad, 1);
        }
    }
    __syncthreads();
    // A_k = sum_{i<k} log2 p_i(x_i): exclusive prefix over the rows
    double term = 0.0;
    if (tid < g) {
        const float zx = a.zx[static_cast<int64_t>(r) * rows + tid];
        term = zx == kNegInf ? -INFINITY : static_cast<double>(zx) * a.c_d - s_L[tid];
    }
    // a -inf term (a masked draft token) makes every later prefix -inf
    const bool neg = term == -INFINITY;
    double total;
    const double excl_sum = block_exclusive_scan(neg ? 0.0 : term, s_waves, &total);
    __syncthreads();
    // the first position whose draft token is masked, via the LDS minimum
    __shared__ int s_firstneg;
    if (tid == 0) s_firstneg = INT32_MAX;
    __syncthreads();
    if (neg) atomicMin(&s_firstneg, tid);
    __syncthreads();
    if (tid < rows) s_A[tid] = tid > s_firstneg ? -INFINITY : excl_sum;
    __syncthreads();
    // scores of every candidate (log2 P), -inf for empty slots
    for (int i = tid; i < ncand; i += kThreads) {
        const int k = i / per_row;
        const OutcomeCand c = a.cand[static_cast<int64_t>(r) * ncand + i];
        double sc = -INFINITY;
        if (c.idx != INT32_MAX && c.val != kNegInf && !s_bad)
            sc = s_A[k] + (static_cast<double>(c.val) * a.c_d - s_L[k]);
        c_score[i] = sc;
        c_tok[i] = c.idx;
    }
    __syncthreads();
    // ncache rounds of a workgroup-wide maximum (ties: smaller k, then token)
    int32_t* ok_ = a.out_k + static_cast<int64_t>(r) * a.ncache;
    int32_t* oa_ = a.out_a + static_cast<int64_t>(r) * a.ncache;
    double* op_ = a.out_p + static_cast<int64_t>(r) * a.ncache;
    double hit = 0.0;
    for (int c = 0; c < a.ncache; ++c) {
        double bv = -INFINITY;
        int bk = INT32_MAX, ba = INT32_MAX, bj = -1;
        for (int i = tid; i < ncand; i += kThreads) {
            const double v = c_score[i];
            const int k = i / per_row, t = c_tok[i];
            if (v > bv || (v == bv && v > -INFINITY && (k < bk || (k == bk && t < ba)))) {
                bv = v;
                bk = k;
                ba = t;
                bj = i;
            }
        }
#pragma unroll
        for (int mask = 32; mask >= 1; mask >>= 1) {
            const double ov = __shfl_xor(bv, mask, 64);
            const int ok = __shfl_xor(bk, mask, 64), oa = __shfl_xor(ba, mask, 64);
            const int oj = __shfl_xor(bj, mask, 64);
            if (ov > bv || (ov == bv && ov > -INFINITY && (ok < bk || (ok == bk && oa < ba)))) {
                bv = ov;
                bk = ok;
                ba = oa;
                bj = oj;
            }
        }
        if (lane == 0) {
            s_bv[wave] = bv;
            s_bk[wave] = bk;
            s_ba[wave] = ba;
            s_bj[wave] = bj;
        }
        __syncthreads();
        double wv = s_bv[0];
        int wk = s_bk[0], wa = s_ba[0], wj = s_bj[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            const double ov = s_bv[w];
            if (ov > wv || (ov == wv && ov > -INFINITY && (s_bk[w] < wk || (s_bk[w] == wk && s_ba[w] < wa)))) {
                wv = ov;
                wk = s_bk[w];
                wa = s_ba[w];
                wj = s_bj[w];
            }
        }
        __syncthreads();
        if (wv > -INFINITY) {
            const double P = exp2(wv);
            hit += P;
            if (tid == 0) {
                ok_[c] = wk;
                oa_[c] = wa;
                op_[c] = P;
                c_score[wj] = -INFINITY;  // taken
            }
        } else if (tid == 0) {
            ok_[c] = -1;
            oa_[c] = -1;
            op_[c] = 0.0;
        }
        __syncthreads();
    }
    if (tid == 0) {
        if (s_bad) {
            for (int c = 0; c < a.ncache; ++c) {
                ok_[c] = -1;
                oa_[c] = -1;
                op_[c] = 0.0;
            }
            a.hit[r] = -1.0;
        } else {
            a.hit[r] = hit;
        }
    }
}

}  // namespace

hipError_t launch_outcome_stats(const OutcomeArgs& a, int dtype, hipStream_t s,
                                hipEvent_t ev_start, hipEvent_t ev_stop) {
    const dim3 grid(a.R * (a.gamma + 1) * a.nseg);
    const dim3 block(kThreads);
    if (dtype == 0) {
        if (a.kb == 4) return launch_timed(outcome_stats_kernel<F32, 4, 4>, grid, block, 0, s, ev_start, ev_stop, a);
        if (a.kb == 8) return launch_timed(outcome_stats_kernel<F32, 4, 8>, grid, block, 0, s, ev_start, ev_stop, a);
        return launch_timed(outcome_stats_kernel<F32, 4, 16>, grid, block, 0, s, ev_start, ev_stop, a);
    }
    if (a.kb == 4) return launch_timed(outcome_stats_kernel<BF16, 4, 4>, grid, block, 0, s, ev_start, ev_stop, a);
    if (a.kb == 8) return launch_timed(outcome_stats_kernel<BF16, 4, 8>, grid, block, 0, s, ev_start, ev_stop, a);
    return launch_timed(outcome_stats_kernel<BF16, 4, 16>, grid, block, 0, s, ev_start, ev_stop, a);
}

hipError_t launch_outcome_select(const OutcomeArgs& a, hipStream_t s) {
    const size_t ncand = static_cast<size_t>(a.gamma + 1) * a.nseg * a.kb;
    const size_t lds = ncand * (sizeof(double) + sizeof(int));
    hipLaunchKernelGGL(outcome_select_kernel, dim3(a.R), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace sv
