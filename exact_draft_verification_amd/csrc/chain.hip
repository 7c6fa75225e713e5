// Chain verification kernels for gfx950.
//
// What is computed (speculative sampling over the vocabulary): for each block
// b and draft position i, p_i = softmax(target_i / T) and
// q_i = softmax(draft_i / T); the draft token x_i passes iff
// u_i < min(1, p_i(x_i)/q_i(x_i)), scanning left to right and stopping at the
// first failure k ("Speculative decoding verifies draft tokens without
// changing the target sampling distribution", sections "Acceptance depends on
// both target and draft probabilities" and "Rejection uses a residual
// distribution"; "JetSpec reading notes", Eq. 1 and Eq. 17).  The extra token
// is the inverse-CDF draw with u_gamma from max(0, p_k - q_k) if k < gamma, or
// from the bonus row p_gamma if every test passed ("A fully accepted block
// yields more than one committed token"; "JetSpec++", Appendix F.1).
//
// Point-mass mode ("JetSpec++", Appendix F.3 and Proposition 1): no draft
// logits; position i passes iff u_i < p_i(x_i), and after a rejection at k
// the draw is from p_k without x_k.
//
// Kernels, in stream order (data crosses workgroups only at kernel
// boundaries, so no workgroup ever waits on another):
//  1. chain_stats: one workgroup per (block, row, segment) streams its share
//     of the block's rows once, folds it into (m, R, S) statistics and writes
//     them as one partial; the workgroup whose segment holds a row's draft
//     token also records that token's logit.
//  2. chain_chunks: one workgroup per (block, chunk of the vocabulary) merges
//     the block's partials (staged in LDS), evaluates every ratio of the block
//     in fp64, finds the first rejection k, and writes the draw-weight sum of
//     every quarter (64 16-byte vectors) of its chunk of the final row
//     (residual row k, p_k without x_k, or the bonus row).
//  3. chain_select: one wave per block scans the quarter sums, finds the
//     quarter holding u_gamma * W and resolves the token inside it with a
//     second wave scan in token order.
//  4. chain_dist (only when final_dist is requested): writes the normalised
//     draw distribution.
// Stochastic tree verification (treestoch.hip) reuses 1-4: its statistics
// pass covers n target and n draft rows per request (draft_rows = n, no
// per-row draft token), and with `given` set the chunk kernel reads the
// decision an earlier kernel wrote (row v*, a plain p draw) and the select
// kernel writes only the drawn token, after the accepted path.
//
// Numerics.  Ratios are evaluated in the log2 domain in fp64 from the row
// statistics, so they are accurate to about 1e-8 whatever the dynamic range.
// The residual weight is formed as p(v) * (1 - 2^-D(v)) with
// D(v) = log2 p(v) - log2 q(v) taken from the exact logit difference (float
// pairs for bf16, fp64 for fp32), so neither the subtraction p - q nor a
// constant offset between the target and draft logits costs precision;
// weights are fp32, sums and prefix sums fp64.
#include "sv_device.hpp"

namespace sv {

namespace {

constexpr double kDomain = 268435456.0;  // |m| / T limit (2^28)

template <class E>
__device__ inline const typename E::storage* chain_row(const ChainArgs& a, int b, int rho) {
    using S = typename E::storage;
    if (rho <= a.gamma)
        return static_cast<const S*>(a.target) + (static_cast<int64_t>(b) * (a.gamma + 1) + rho) *
                                                     static_cast<int64_t>(a.V);
    return static_cast<const S*>(a.draft) +
           (static_cast<int64_t>(b) * a.draft_rows + (rho - a.gamma - 1)) * static_cast<int64_t>(a.V);
}

template <class E>
struct StatFolder {
    Stat s;
    float c_hi, c_lo;
    template <int N>
    __device__ inline void batch(const uint4* v, int) {
        float x[N * E::kPerVec];
#pragma unroll
        for (int u = 0; u < N; ++u) E::unpack(v[u], x + u * E::kPerVec);
        stat_fold<N * E::kPerVec>(s, x, c_hi, c_lo);
    }
};

// Statistics of elements [e0, e1) of one row, folded by the whole workgroup
// (one partial per thread); U 16-byte vectors per thread per batch.
template <class E, int U>
__device__ inline Stat row_range_stats(const typename E::storage* row, int e0, int e1, float c_hi,
                                       float c_lo) {
    StatFolder<E> f{stat_empty(), c_hi, c_lo};
    if (e0 >= e1) return f.s;
    const int tid = threadIdx.x;
    const RangeSplit<E> sp = split_range<E>(row, e0, e1);
    for (int e = sp.head_begin + tid; e < sp.head_end; e += kThreads) {
        float x = E::one(row + e);
        stat_fold<1>(f.s, &x, c_hi, c_lo);
    }
    stream_vectors<U>(reinterpret_cast<const char*>(row + sp.body_begin), sp.nvec, f);
    for (int e = sp.tail_begin + tid; e < sp.tail_end; e += kThreads) {
        float x = E::one(row + e);
        stat_fold<1>(f.s, &x, c_hi, c_lo);
    }
    return f.s;
}

template <class E, int U>
__global__ __launch_bounds__(kThreads) void chain_stats_kernel(ChainArgs a) {
    __shared__ Stat s_w[kWaves];
    const int rows = a.rows;
    const int unit = blockIdx.x;
    const int seg = unit % a.nseg;
    const int rr = unit / a.nseg;  // b * rows + rho
    const int rho = rr % rows;
    const int b = rr / rows;
    const int tid = threadIdx.x;
    const auto* row = chain_row<E>(a, b, rho);
    const int e0 = seg * a.seg_len;
    const int e1 = min(a.V, e0 + a.seg_len);
    // The logit of this row's draft token, if it lies in this segment (the
    // load is issued before the stream so its latency is hidden).  Rows
    // i < gamma (target) and gamma+1+i (draft) belong to draft position i.
    float zx = 0.0f;
    bool have_zx = false;
    if (tid == 0 && a.tokens) {  // (tree rows have no per-row draft token)
        const int i = rho < a.gamma ? rho : (rho > a.gamma ? rho - a.gamma - 1 : -1);
        if (i >= 0) {
            const int x = a.tokens[static_cast<int64_t>(b) * a.gamma + i];
            if (x >= e0 && x < e1) {
                zx = E::one(row + x);
                have_zx = true;
            }
        }
    }
    Stat st = row_range_stats<E, U>(row, e0, e1, a.c_hi, a.c_lo);
    st = block_reduce_stat(st, s_w);
    if (tid == 0) {
        a.part[unit] = st;
        if (have_zx) a.zx[rr] = zx;
    }
}

// Ratio tests of block b, taken by every workgroup of the block's final-draw
// kernel for itself (cheaper than a launch of its own): every input (the
// block's row partials, the draft tokens, their logits and the uniforms) is
// requested in one round of loads; the partials are merged per row in LDS;
// then for each draft position i, r_i = min(1, p_i(x_i)/q_i(x_i)) is
// evaluated in the log2 domain in fp64 and the first i with u_i >= r_i kept.
template <class E, int NT = kThreads>
__device__ ChainDecision chain_decide(const ChainArgs& a, int b, Stat* s_part) {
    __shared__ double s_L[2 * kMaxGamma + 1];
    __shared__ double s_S[kMaxGamma + 1];
    __shared__ float s_R[2 * kMaxGamma + 1];
    __shared__ int s_x[kMaxGamma];
    __shared__ int s_bad, s_k;
    constexpr int kPer = kMaxBlockParts / NT;
    const int g = a.gamma, rows = a.rows, tid = threadIdx.x;
    const int np = rows * a.nseg;
    // per-position inputs (gamma <= 255 < NT: one position per thread)
    int x = 0;
    float zp = 0.0f, zq = 0.0f, u = 0.0f;
    if (tid < g) {
        x = a.tokens[static_cast<int64_t>(b) * g + tid];
        zp = a.zx[static_cast<int64_t>(b) * rows + tid];
        if (!a.pointmass) zq = a.zx[static_cast<int64_t>(b) * rows + g + 1 + tid];
        u = a.uniforms[static_cast<int64_t>(b) * (g + 1) + tid];
        s_x[tid] = x;
    }
    {
        // every load issued before any LDS store; a Stat is one 16-byte
        // vector (indices past the end re-read the last partial, unstored)
        static_assert(sizeof(Stat) == 16, "Stat is staged as one 16-byte vector");
        const uint4* src = reinterpret_cast<const uint4*>(a.part + static_cast<int64_t>(b) * np);
        uint4* dst = reinterpret_cast<uint4*>(s_part);
        uint4 t[kPer];
#pragma unroll
        for (int m = 0; m < kPer; ++m)
            t[m] = m * NT < np ? src[min(tid + m * NT, np - 1)] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int m = 0; m < kPer; ++m)
            if (tid + m * NT < np) dst[tid + m * NT] = t[m];
    }
    if (tid == 0) {
        s_bad = 0;
        s_k = g;
    }
    __syncthreads();
    for (int r = tid; r < rows; r += NT) {
        // four independent merge chains (the merge is a short dependent
        // sequence, so one chain over many segments is latency-bound)
        const Stat* p = s_part + r * a.nseg;
        Stat t0 = p[0], t1 = stat_empty(), t2 = stat_empty(), t3 = stat_empty();
        int s = 1;
        for (; s + 3 < a.nseg; s += 4) {
            t0 = stat_merge(t0, p[s]);
            t1 = stat_merge(t1, p[s + 1]);
            t2 = stat_merge(t2, p[s + 2]);
            t3 = stat_merge(t3, p[s + 3]);
        }
        for (; s < a.nseg; ++s) t0 = stat_merge(t0, p[s]);
        const Stat t = stat_merge(stat_merge(t0, t1), stat_merge(t2, t3));
        const bool ok = isfinite(t.S) && t.S > 0.0 && fabs(static_cast<double>(t.m) / a.T) <= kDomain;
        if (!ok) atomicOr(&s_bad, 1);
        s_L[r] = static_cast<double>(t.R) + log2(t.S);
        s_R[r] = t.R;
        if (r <= g) s_S[r] = t.S;
    }
    __syncthreads();
    if (tid < g) {
        if (x < 0 || x >= a.V) {
            atomicOr(&s_bad, 1);
        } else {
            double r;
            if (zp == -INFINITY) {
                r = 0.0;
            } else if (a.pointmass) {
                // the draft proposes x with certainty: r = p(x) = 2^(log2 p(x))
                const double d = static_cast<double>(zp) * a.c_d - s_L[tid];
                r = d >= 0.0 ? 1.0 : exp2(d);
            } else if (zq == -INFINITY) {
                r = 1.0;
            } else {
                // log2 p(x) - log2 q(x), both rows' log2-sum-exp in fp64
                const double d = (static_cast<double>(zp) * a.c_d - s_L[tid]) -
                                 (static_cast<double>(zq) * a.c_d - s_L[g + 1 + tid]);
                r = d >= 0.0 ? 1.0 : exp2(d);
            }
            if (!(static_cast<double>(u) < r)) atomicMin(&s_k, tid);
        }
    }
    __syncthreads();
    ChainDecision d;
    d.pad = 0;
    if (s_bad) {
        d.k = -1;
        d.Rp = 0.0f;
        d.dL = 0.0;
        d.excl = -1;
        d.Sp = 0.0;
    } else {
        const int k = s_k;
        d.k = k;
        d.Rp = s_R[k];
        d.Sp = s_S[k];
        // ratio test: the residual needs the row pair's log-normaliser gap;
        // point mass: the residual is p_k without the rejected token
        d.dL = (k < g && !a.pointmass) ? s_L[k] - s_L[g + 1 + k] : 0.0;
        d.excl = (k < g && a.pointmass) ? s_x[k] : -1;
    }
    return d;
}

// ---------------------------------------------------------------------------
// Final draw.
//
// The final row (residual row k, or the bonus row) is cut into tiles of
// kThreads 16-byte vectors; thread t of a workgroup owns vector t of a tile,
// i.e. the kPerVec consecutive tokens starting at tile + t*kPerVec, and wave w
// owns the "quarter" of 64 vectors [64w, 64w+64).  Each lane sums its kPerVec
// weights in token order in fp32; lanes and quarters are summed in fp64.  The
// chunk kernel writes one weight sum per quarter; the select kernel (one wave
// per block) scans the quarter sums for the quarter holding u * W, then scans
// that quarter's 64 lanes in token order.

struct DrawRow {
    float Rp, c_hi, c_lo;
    float dL_hi, dL_lo;  // dL as a float pair
    float A_hi;          // Rp - dL rounded to float (a screen for negligible draft weights)
    double c_d, dL;
    double A;            // Rp - dL: log2 Q'(v) = z_q(v) c - A
    bool resid;  // residual of p_k and q_k (else p_k itself, unnormalised)
    int excl;    // a token whose weight is 0 (point mass: the rejected one), or -1
};

// D(v) = log2 p_k(v) - log2 q_k(v) = (z_p - z_q) c - dL.  bf16 logits: the
// difference of two bf16 values is exact in fp32, and with c and dL carried
// as float pairs the two fused multiply-adds round once each, at the scale of
// D itself, so a constant offset between the rows cancels exactly.  fp32
// logits: the difference is taken in fp64.
__device__ inline float log_ratio(float zp, float zq, const DrawRow& r, BF16) {
    const float dz = zp - zq;
    return fmaf(dz, r.c_hi, -r.dL_hi) + fmaf(dz, r.c_lo, -r.dL_lo);
}
__device__ inline float log_ratio(float zp, float zq, const DrawRow& r, F32) {
    return static_cast<float>(fma(static_cast<double>(zp) - static_cast<double>(zq), r.c_d, -r.dL));
}

// 1 - 2^-D for 0 <= D < 1, to within 2e-7 relative: x * g(x) with
// x = D ln 2 and g(x) = (1 - e^-x)/x approximated on [0, ln 2] by a degree-5
// polynomial (coefficients fitted here to minimise the relative error: at
// most 1.83e-8 with these fp32 coefficients in exact arithmetic, 1.55e-7
// once x, each step and x * g are rounded to fp32).  From 1 up the callers
// use 1 - 2^-D with the hardware exp2, where 2^-D <= 1/2 keeps the
// subtraction well conditioned.
__device__ inline float one_minus_exp2_neg_small(float D) {
    const float x = D * 0.693147180559945309f;
    float g = -1.033136854e-03f;
    g = fmaf(g, x, 8.067236282e-03f);
    g = fmaf(g, x, -4.157199338e-02f);
    g = fmaf(g, x, 1.666511893e-01f);
    g = fmaf(g, x, -4.999990761e-01f);
    g = fmaf(g, x, 1.0f);
    return x * g;
}

// t = z_p c - R_p of a token (its target weight is 2^t).
__device__ inline float target_t(float zp, const DrawRow& r) {
    const float t = fmaf(zp, r.c_hi, -r.Rp);
    return fmaf(zp, r.c_lo, t);
}

// The terms of a token whose target weight is not negligible (t > -60).
template <class E>
__device__ inline void resid_main(float zp, float zq, float t, const DrawRow& r, float& w,
                                  float& d, float& pz) {
    const float D = log_ratio(zp, zq, r, E{});
    const float aD = fabsf(D);
    const float sm = one_minus_exp2_neg_small(aD);
    const float e = __builtin_amdgcn_exp2f(-D);
    const bool small = aD < 1.0f;
    const bool pos = D > 0.0f;
    const float f = pos ? (small ? sm : 1.0f - e) : -(small ? sm * e : e - 1.0f);
    const float P = __builtin_amdgcn_exp2f(t);
    d = P * f;
    w = fmaxf(d, 0.0f);
    pz = pos ? P : 0.0f;
}

// A token of negligible target weight: whether its draft weight Q' is not
// negligible as well, and then d = -Q' (log2 Q' = z_q c - A in double, then
// 2^(hi + lo) = 2^hi (1 + lo ln 2)).
__device__ inline bool draft_weight_counts(float zq, const DrawRow& r) {
    return fmaf(zq, r.c_hi, -r.A_hi) > -62.0f;
}
__device__ inline float minus_draft_weight(float zq, const DrawRow& r) {
    const double tq = static_cast<double>(zq) * r.c_d - r.A;
    const float hi = static_cast<float>(tq);
    const double lo = tq - static_cast<double>(hi);
    return -static_cast<float>(static_cast<double>(__builtin_amdgcn_exp2f(hi)) *
                               (1.0 + lo * 0.69314718055994530942));
}

// Residual terms of one token of the residual draw (ratio test, k < gamma).
// With P = 2^(z_p c - R_p) (p's weight) and D = log2 p - log2 q, where q uses
// the dL in hand, let Q' = P 2^-D (q's weight in P's units):
//   d  = P - Q' = P (1 - 2^-D), signed,
//   w  = max(d, 0), the residual weight,
//   pz = P where D > 0, else 0.
// If the dL in hand is off by delta (its error from the row statistics, up to
// about 2e-7), the sum of d over the row is S_p (1 - 2^delta), so the select
// kernel recovers delta from it, and w + kappa (pz - w) with kappa =
// delta ln 2 is the weight at the exact dL to first order (dw/d(dL) =
// -ln 2 (pz - w)).  Without it the residual mass W would carry a relative
// error of about delta ln 2 q(D > 0) / W, large when p and q nearly agree.
// So d must be accurate relative to itself, whatever its sign: for |D| < 1
// it is formed from s = 1 - 2^-|D| (the polynomial) as P s (D > 0) or
// -P s 2^|D| (D < 0), beyond that from 2^-D.  A token of negligible target
// weight (as in the draw weights, t <= -60) has d = -Q', taken from its draft
// logit in double precision when Q' is not negligible as well.
template <class E>
__device__ inline void resid_terms(float zp, float zq, const DrawRow& r, float& w, float& d,
                                   float& pz) {
    const float t = target_t(zp, r);
    w = 0.0f;
    d = 0.0f;
    pz = 0.0f;
    if (t > -60.0f)
        resid_main<E>(zp, zq, t, r, w, d, pz);
    else if (draft_weight_counts(zq, r))
        d = minus_draft_weight(zq, r);
}

// The lane's kPerVec residual terms in token order: weights w[i] and
// pz[i], and the fp32 sums of w, d and pz in that order (the select kernel's
// view of one quarter).
template <class E>
__device__ inline void lane_resid(const float* zp, const float* zq, const DrawRow& r, float* w,
                                  float* pz, float& sw, float& sd, float& sp) {
    sw = 0.0f;
    sd = 0.0f;
    sp = 0.0f;
#pragma unroll
    for (int i = 0; i < E::kPerVec; ++i) {
        float d;
        resid_terms<E>(zp[i], zq[i], r, w[i], d, pz[i]);
        sw += w[i];
        sd += d;
        sp += pz[i];
    }
}

// The same three fp32 sums without the terms themselves (the chunk kernel's
// view).  A token adds only its nonzero terms: adding +0 or -0 to these sums
// is exact (a running sum of them is never -0), so the sums are bit for bit
// those of lane_resid, and a token whose terms are all zero (most tokens of a
// peaked row) costs only its tests.
template <class E>
__device__ inline void lane_resid_sums(const float* zp, const float* zq, const DrawRow& r,
                                       float& sw, float& sd, float& sp) {
    sw = 0.0f;
    sd = 0.0f;
    sp = 0.0f;
#pragma unroll
    for (int i = 0; i < E::kPerVec; ++i) {
        const float t = target_t(zp[i], r);
        if (t > -60.0f) {
            float w, d, pz;
            resid_main<E>(zp[i], zq[i], t, r, w, d, pz);
            sw += w;
            sd += d;
            sp += pz;
        } else if (draft_weight_counts(zq[i], r)) {
            sd += minus_draft_weight(zq[i], r);
        }
    }
}

// Unnormalised draw weight of token v for a draw from p_k itself (the bonus
// row, point mass, a stochastic tree, or the fallback of an empty residual):
// w = P(v) = 2^(z_p c - R_p), 0 for a masked token (-inf logit).  The
// residual draw uses resid_terms instead.
template <class E>
__device__ inline float draw_weight(float zp, float, const DrawRow& r) {
    float t = fmaf(zp, r.c_hi, -r.Rp);
    t = fmaf(zp, r.c_lo, t);
    return __builtin_amdgcn_exp2f(t);
}

template <class E>
struct FinalRows {
    const typename E::storage* p;
    const typename E::storage* q;  // nullptr unless k < gamma
    bool vec_ok;                   // both rows 16-byte aligned
};

template <class E>
__device__ inline FinalRows<E> final_rows(const ChainArgs& a, int b, int k) {
    using S = typename E::storage;
    FinalRows<E> f;
    f.p = static_cast<const S*>(a.target) + (static_cast<int64_t>(b) * (a.gamma + 1) + k) * a.V;
    f.q = (k < a.gamma && !a.pointmass)
              ? static_cast<const S*>(a.draft) + (static_cast<int64_t>(b) * a.gamma + k) * a.V
              : nullptr;
    f.vec_ok = (reinterpret_cast<uintptr_t>(f.p) & 15u) == 0 &&
               (f.q == nullptr || (reinterpret_cast<uintptr_t>(f.q) & 15u) == 0);
    return f;
}

// The draw of block b: the residual of p_k and q_k after a rejection under
// the ratio test; p_k without the rejected token under point mass; p_gamma
// after a fully accepted block.
__device__ inline DrawRow draw_row(const ChainArgs& a, const ChainDecision& d) {
    const float dL_hi = static_cast<float>(d.dL);
    const float dL_lo = static_cast<float>(d.dL - static_cast<double>(dL_hi));
    const bool resid = d.k < a.gamma && !a.pointmass;
    const double A = static_cast<double>(d.Rp) - d.dL;
    return DrawRow{d.Rp,  a.c_hi, a.c_lo, dL_hi, dL_lo, static_cast<float>(A),
                   a.c_d, d.dL,   A,      resid, d.excl};
}

// The kPerVec tokens [e, e + kPerVec) of the final row(s) as floats: one
// 16-byte load when the whole vector is in range and aligned, else one load
// per in-range token; tokens at or past V read as -inf (weight 0).
template <class E>
__device__ inline void load_tokens(const FinalRows<E>& rows, bool resid, int e, int V, float* zp,
                                   float* zq) {
    if (rows.vec_ok && e + E::kPerVec <= V) {
        E::unpack(load16_stream(rows.p + e), zp);
        if (resid) E::unpack(load16_stream(rows.q + e), zq);
    } else {
#pragma unroll
        for (int i = 0; i < E::kPerVec; ++i) {
            zp[i] = e + i < V ? E::one(rows.p + e + i) : -INFINITY;
            if (resid) zq[i] = e + i < V ? E::one(rows.q + e + i) : -INFINITY;
        }
    }
    if (!resid) {
#pragma unroll
        for (int i = 0; i < E::kPerVec; ++i) zq[i] = 0.0f;
    }
}

// Weights of the lane's kPerVec tokens [e, e + kPerVec) for a draw from p_k
// itself (r.resid false) and their sum, accumulated in token order in fp32
// (the select kernel repeats exactly this order, so its running prefix ends
// on the very value the quarter sums were built from; lane_resid keeps the
// same order for the residual draw).
template <class E>
__device__ inline float lane_weights(const float* zp, const float* zq, const DrawRow& r, int e,
                                     float* w) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < E::kPerVec; ++i) {
        w[i] = draw_weight<E>(zp[i], zq[i], r);
        s += w[i];
    }
    // only a point-mass draw excludes a token: the one lane that holds it
    // zeroes its weight and sums again, in the same order
    if (static_cast<unsigned>(r.excl - e) < static_cast<unsigned>(E::kPerVec)) {
        s = 0.0f;
#pragma unroll
        for (int i = 0; i < E::kPerVec; ++i) {
            w[i] = e + i == r.excl ? 0.0f : w[i];
            s += w[i];
        }
    }
    return s;
}


// Exclusive prefix sum over the lanes of a wave, plus the wave total.
__device__ inline double wave_exclusive_scan(double v, double* total) {
    const double incl = wave_inclusive_scan(v);
    *total = readlane_f64(incl, 63);
    return incl - v;
}

// Outputs of block b: accept length k, then x_0 .. x_{k-1}, the drawn token
// and -1 padding (all -1 for an invalid block).  Any block size.
template <class E>
__device__ void write_outputs(const ChainArgs& a, int b, int k, int token, int first, int stride) {
    const int g = a.gamma;
    int32_t* out = a.out_tokens + static_cast<int64_t>(b) * (g + 1);
    for (int i = first; i <= g; i += stride) {
        int32_t v = -1;
        if (k >= 0) {
            if (i < k)
                v = a.tokens[static_cast<int64_t>(b) * g + i];
            else if (i == k)
                v = token;
        }
        out[i] = v;
    }
    if (first == 0) a.accept_len[b] = k;
}

// The decision of block b as written by the chunk kernel.  k is clamped to
// the invalid marker unless it lies in [0, gamma], so no row pointer is ever
// formed from an out-of-range value.
__device__ inline ChainDecision load_decision(const ChainArgs& a, int b) {
    ChainDecision d = a.dec[b];
    if (d.k < 0 || d.k > a.gamma) d.k = -1;
    return d;
}

// Raw 16-byte vectors of one group of G tiles of the final row(s), tiles
// [t, t + G): this thread's vector of each tile.  Every load is issued
// unconditionally (so the group's count of loads in flight is fixed): a tile
// at or past t1 re-reads tile t1 - 1, and a vector not wholly inside the row
// re-reads the row's last whole vector; group_sums discards both.  Needs
// 16-byte aligned rows of at least one whole vector.
template <class E, int G, bool RESID, int NT = kThreads>
__device__ inline void issue_group(const FinalRows<E>& rows, int t, int t1, int vlast, uint4* p,
                                   uint4* q) {
    constexpr int kTile = NT * E::kPerVec;
#pragma unroll
    for (int m = 0; m < G; ++m) {
        const int e = min(min(t + m, t1 - 1) * kTile + static_cast<int>(threadIdx.x) * E::kPerVec, vlast);
        p[m] = load16_stream(rows.p + e);
        if constexpr (RESID) q[m] = load16_stream(rows.q + e);
    }
}

// Quarter sums of the group of tiles [t, min(t + G, t1)) from its raw
// vectors; a vector that straddles the row's end is read token by token,
// one past it is all -inf (weight 0).
template <class E, int G, bool RESID, int NT = kThreads>
__device__ inline void group_sums(const FinalRows<E>& rows, const DrawRow& r, int t, int t1, int V,
                                  const uint4* p, const uint4* q, double* qs, double* qp,
                                  int nquart, double& dacc) {
    constexpr int kTile = NT * E::kPerVec;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int m = 0; m < G; ++m) {
        const int j = t + m;
        if (j >= t1) break;  // (uniform)
        const int e = j * kTile + static_cast<int>(threadIdx.x) * E::kPerVec;
        float zp[E::kPerVec], zq[E::kPerVec], w[E::kPerVec];
        if (e + E::kPerVec <= V) {
            E::unpack(p[m], zp);
            if constexpr (RESID) {
                E::unpack(q[m], zq);
            } else {
#pragma unroll
                for (int i = 0; i < E::kPerVec; ++i) zq[i] = 0.0f;
            }
        } else {
            load_tokens<E>(rows, RESID, e, V, zp, zq);
        }
        const int qi = j * (NT / 64) + wave;
        if constexpr (RESID) {
            float lw, ld, lp;
            lane_resid_sums<E>(zp, zq, r, lw, ld, lp);
            dacc += static_cast<double>(ld);
            const double sw = wave_sum(static_cast<double>(lw));
            const double sp = wave_sum(static_cast<double>(lp));
            if (lane == 0 && qi < nquart) {
                qs[qi] = sw;
                qp[qi] = sp;
            }
        } else {
            const double sw =
                wave_sum(static_cast<double>(lane_weights<E>(zp, zq, r, e, w)));
            if (lane == 0 && qi < nquart) qs[qi] = sw;
        }
    }
}

// The chunk's tiles [t0, t1) in groups of G, software-pipelined: the next
// group's loads are in flight while the current group's weights are formed.
template <class E, int G, bool RESID, int NT = kThreads>
__device__ inline void stream_tiles(const FinalRows<E>& rows, const DrawRow& r, int t0, int t1,
                                    int V, double* qs, double* qp, int nquart, double& dacc) {
    const int vlast = (V / E::kPerVec - 1) * E::kPerVec;  // the row's last whole vector
    const int ngroup = (t1 - t0 + G - 1) / G;
    uint4 cp[G], cq[G];
    issue_group<E, G, RESID, NT>(rows, t0, t1, vlast, cp, cq);
    for (int gi = 0; gi + 1 < ngroup; ++gi) {
        uint4 np[G], nq[G];
        issue_group<E, G, RESID, NT>(rows, t0 + (gi + 1) * G, t1, vlast, np, nq);
        group_sums<E, G, RESID, NT>(rows, r, t0 + gi * G, t1, V, cp, cq, qs, qp, nquart, dacc);
#pragma unroll
        for (int m = 0; m < G; ++m) {
            cp[m] = np[m];
            if constexpr (RESID) cq[m] = nq[m];
        }
    }
    group_sums<E, G, RESID, NT>(rows, r, t0 + (ngroup - 1) * G, t1, V, cp, cq, qs, qp, nquart, dacc);
}

// Chunk workgroup: the block's decision, then the chunk's tiles of the final
// row, a run of chunk_tiles consecutive tiles streamed in groups of G.
template <class E, int G>
__global__ __launch_bounds__(kThreads) void chain_chunks_kernel(ChainArgs a) {
    extern __shared__ Stat s_part[];  // [2*gamma+1][nseg]
    constexpr int kTile = kThreads * E::kPerVec;
    const int b = blockIdx.x / a.nchunk;
    const int c = blockIdx.x % a.nchunk;
    ChainDecision d;
    if (a.given) {
        d = load_decision(a, b);
    } else {
        d = chain_decide<E>(a, b, s_part);
        if (c == 0 && threadIdx.x == 0) a.dec[b] = d;
    }
    if (d.k < 0) return;  // invalid block: the select kernel writes -1s
    const FinalRows<E> rows = final_rows<E>(a, b, d.k);
    const DrawRow r = draw_row(a, d);
    const int ntile = (a.V + kTile - 1) / kTile;
    const int t0 = c * a.chunk_tiles, t1 = min(ntile, t0 + a.chunk_tiles);
    double* qs = a.qsum + static_cast<int64_t>(b) * a.nquart;
    double* qp = a.qpos + static_cast<int64_t>(b) * a.nquart;
    double dacc = 0.0;  // residual draw: this thread's share of sum (P - Q') over the chunk
    if (rows.vec_ok && a.V >= E::kPerVec) {
        if (r.resid)
            stream_tiles<E, G, true>(rows, r, t0, t1, a.V, qs, qp, a.nquart, dacc);
        else
            stream_tiles<E, G, false>(rows, r, t0, t1, a.V, qs, qp, a.nquart, dacc);
    } else {
        // rows not 16-byte aligned (or shorter than a vector): token by token
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        for (int j = t0; j < t1; ++j) {
            float zp[E::kPerVec], zq[E::kPerVec], w[E::kPerVec];
            const int e = j * kTile + static_cast<int>(threadIdx.x) * E::kPerVec;
            load_tokens<E>(rows, r.resid, e, a.V, zp, zq);
            const int qi = j * kWaves + wave;
            if (r.resid) {
                float lw, ld, lp;
                lane_resid_sums<E>(zp, zq, r, lw, ld, lp);
                dacc += static_cast<double>(ld);
                const double sw = wave_sum(static_cast<double>(lw));
                const double sp = wave_sum(static_cast<double>(lp));
                if (lane == 0 && qi < a.nquart) {
                    qs[qi] = sw;
                    qp[qi] = sp;
                }
            } else {
                const double sw = wave_sum(static_cast<double>(lane_weights<E>(zp, zq, r, e, w)));
                if (lane == 0 && qi < a.nquart) qs[qi] = sw;
            }
        }
    }
    if (r.resid) {
        // the chunk's sum of P - Q'
        __shared__ double s_d[kWaves];
        const double wd = wave_sum(dacc);
        if ((threadIdx.x & 63) == 0) s_d[threadIdx.x >> 6] = wd;
        __syncthreads();
        if (threadIdx.x == 0) {
            double t = 0.0;
#pragma unroll
            for (int i = 0; i < kWaves; ++i) t += s_d[i];
            a.cdiff[static_cast<int64_t>(b) * a.nchunk + c] = t;
        }
    }
}

// Token selection for block b, by one wave.
//
// The draw is the smallest token v whose inclusive prefix sum of weights
// exceeds u * W (W the total).  Lane l takes a contiguous run of quarters;
// one wave scan of the runs' sums and a walk inside the crossing lane's run
// give the quarter; lane l of that quarter holds the kPerVec consecutive
// tokens starting at quarter + l*kPerVec, so a second wave scan gives the
// token.  If rounding leaves no crossing, the last token of positive weight
// is taken.  A residual that sums to zero (possible only through rounding
// after a rejection) falls back to p_k: the wave then recomputes the quarter
// sums from p_k itself (slow, but never on a normal path).
//
// select_block is that selection for one wave (all 64 of its lanes, lane =
// this lane's index): qs and qp are the block's quarter sums (global memory,
// or LDS when the whole draw runs in one workgroup).  The residual draw's sum
// of P - Q' over the row comes from the chunks' partial sums cd[0 .. nchunk)
// when cd is given, else it is rowd.  dk: the block's decision if the caller
// holds it, else it is loaded here.
template <class E>
__device__ void select_block(const ChainArgs& a, int b, int lane, double* qs, const double* qp,
                             const double* cd, double rowd, const ChainDecision* dk) {
    constexpr int kQuart = 64 * E::kPerVec;
    const int g = a.gamma;
    const int per = (a.nquart + 63) / 64;
    const int q0 = min(a.nquart, lane * per), q1 = min(a.nquart, q0 + per);
    // this lane's run of quarter sums, requested together with the decision
    // and the uniform (runs of up to kRun in registers, longer ones looped)
    constexpr int kRun = 16;
    double run_v[kRun], run_p[kRun];
#pragma unroll
    for (int j = 0; j < kRun; ++j) run_v[j] = q0 + j < q1 ? qs[q0 + j] : 0.0;
    const ChainDecision d = dk ? *dk : load_decision(a, b);
    // residual draw: the quarters' sums of P where D > 0, and the chunks'
    // sums of P - Q' (written only for a residual draw; read only then)
    const bool resid_draw = d.k >= 0 && d.k < g && !a.pointmass;
    double dpart = 0.0;
    if (resid_draw) {
#pragma unroll
        for (int j = 0; j < kRun; ++j) run_p[j] = q0 + j < q1 ? qp[q0 + j] : 0.0;
        if (cd) {
            for (int c = lane; c < a.nchunk; c += 64) dpart += cd[c];
        } else if (lane == 0) {
            dpart = rowd;
        }
    }
    const double u =
        static_cast<double>(a.uniforms[static_cast<int64_t>(b) * (g + 1) + (a.given ? 0 : g)]);
    // the block's draft tokens for its output row, requested now (one per
    // lane; a block of 64 or more positions loads them when writing)
    const bool lane_out = !a.given && g < 64;
    const int xtok = lane_out && lane < g ? a.tokens[static_cast<int64_t>(b) * g + lane] : -1;
    if (d.k < 0) {
        if (!a.given) write_outputs<E>(a, b, -1, -1, lane, 64);  // (a given decision wrote its own)
        return;
    }
    const FinalRows<E> rows = final_rows<E>(a, b, d.k);
    double mine = 0.0;
#pragma unroll
    for (int j = 0; j < kRun; ++j) mine += run_v[j];
    for (int q = q0 + kRun; q < q1; ++q) mine += qs[q];
    int fallback = 0;
    DrawRow r = draw_row(a, d);
    // residual draw: kappa = delta ln 2 from the row's sum of P - Q' (see
    // resid_terms); every weight below is taken as w + kappa (pz - w)
    double kappa = 0.0;
    if (resid_draw) kappa = log1p(-wave_sum(dpart) / d.Sp);
    if ((r.resid || r.excl >= 0) && !(wave_sum(mine) > 0.0)) {
        fallback = 1;
        r.resid = false;
        r.excl = -1;
        // quarter sums of p_k, each by one lane, in the chunk kernel's order
        kappa = 0.0;
        mine = 0.0;
        for (int q = q0; q < q1; ++q) {
            double sq = 0.0;
            for (int l = 0; l < 64; ++l) {
                float zp[E::kPerVec], zq[E::kPerVec], w[E::kPerVec];
                const int e = q * kQuart + l * E::kPerVec;
                load_tokens<E>(rows, false, e, a.V, zp, zq);
                sq += static_cast<double>(lane_weights<E>(zp, zq, r, e, w));
            }
            qs[q] = sq;
            mine += sq;
        }
    }
    const bool corr = r.resid;  // (after a fallback the draw is from p_k itself)
    if (corr) {
        double mp = 0.0;
#pragma unroll
        for (int j = 0; j < kRun; ++j) mp += run_p[j];
        for (int q = q0 + kRun; q < q1; ++q) mp += qp[q];
        mine += kappa * (mp - mine);
    }
    double W;
    const double excl = wave_exclusive_scan(mine, &W);
    const double target = u * W;
    // the lane whose run holds the crossing, then the quarter inside it
    const unsigned long long hit = __ballot(mine > 0.0 && excl + mine > target);
    bool last_positive = false;
    int src;
    if (hit) {
        src = __ffsll(static_cast<long long>(hit)) - 1;
    } else {
        // no crossing (rounding): the last quarter of positive weight
        const unsigned long long pos = __ballot(mine > 0.0);
        src = pos ? 63 - __clzll(static_cast<long long>(pos)) : 0;
        last_positive = true;
    }
    // the quarter inside the crossing lane's run: lane j takes the run's
    // j-th quarter (runs of up to 64 quarters; longer runs are walked by
    // their own lane), one more wave scan finds the crossing
    // (src, jj and the like are wave-uniform: broadcasts are lane reads)
    const int sq0 = __builtin_amdgcn_readlane(q0, src), sq1 = __builtin_amdgcn_readlane(q1, src);
    const double sbase = readlane_f64(excl, src);
    int qstar;
    double base;
    if (sq1 - sq0 <= 64) {
        const int q = sq0 + lane;
        double x;
        if (per <= kRun && !fallback) {
            // the run is in the crossing lane's registers (the fallback
            // rewrote the sums in memory only): lane j takes its j-th entry
            // by shuffle
            x = 0.0;
            double xp = 0.0;
#pragma unroll
            for (int j = 0; j < kRun; ++j) {
                const double v = readlane_f64(run_v[j], src);
                if (lane == j) x = v;
                if (corr) {
                    const double vp = readlane_f64(run_p[j], src);
                    if (lane == j) xp = vp;
                }
            }
            if (corr) x += kappa * (xp - x);
        } else {
            x = q < sq1 ? qs[q] : 0.0;
            if (corr && q < sq1) x += kappa * (qp[q] - x);
        }
        double xt;
        const double xe = wave_exclusive_scan(x, &xt);
        const unsigned long long hq = __ballot(!last_positive && x > 0.0 && sbase + xe + x > target);
        const unsigned long long pq = __ballot(x > 0.0);
        int jj;
        if (hq) {
            jj = __ffsll(static_cast<long long>(hq)) - 1;
        } else {
            // rounding: the run's last positive quarter
            jj = pq ? 63 - __clzll(static_cast<long long>(pq)) : 0;
        }
        qstar = sq0 + jj;
        base = sbase + readlane_f64(xe, jj);
    } else {
        int qfound = q0;
        double b0 = excl;
        if (lane == src) {
            double run = excl, run_last = excl;
            int lastq = -1;
            qfound = -1;
            for (int q = q0; q < q1; ++q) {
                const double sqv = corr ? qs[q] + kappa * (qp[q] - qs[q]) : qs[q];
                if (sqv > 0.0) {
                    lastq = q;
                    run_last = run;
                    if (!last_positive && run + sqv > target) {
                        qfound = q;
                        b0 = run;
                        break;
                    }
                }
                run += sqv;
            }
            if (qfound < 0) {
                qfound = lastq >= 0 ? lastq : q0;
                b0 = run_last;
            }
        }
        qstar = __builtin_amdgcn_readlane(qfound, src);
        base = readlane_f64(b0, src);
    }
    // tokens of the chosen quarter, kPerVec per lane in token order
    const int e0 = qstar * kQuart + lane * E::kPerVec;
    float zp[E::kPerVec], zq[E::kPerVec], w[E::kPerVec], pz[E::kPerVec];
    load_tokens<E>(rows, r.resid, e0, a.V, zp, zq);
    double lval;
    if (corr) {
        float lw, ld, lp;
        lane_resid<E>(zp, zq, r, w, pz, lw, ld, lp);
        lval = static_cast<double>(lw) + kappa * (static_cast<double>(lp) - static_cast<double>(lw));
    } else {
        lval = static_cast<double>(lane_weights<E>(zp, zq, r, e0, w));
#pragma unroll
        for (int i = 0; i < E::kPerVec; ++i) pz[i] = 0.0f;
    }
    double qtot;
    const double lbase = base + wave_exclusive_scan(lval, &qtot);
    int found = INT32_MAX, lastpos = -1;
    float pre = 0.0f, prep = 0.0f;
#pragma unroll
    for (int i = 0; i < E::kPerVec; ++i) {
        pre += w[i];
        prep += pz[i];
        if (w[i] > 0.0f) {
            lastpos = e0 + i;
            const double at = static_cast<double>(pre) +
                              kappa * (static_cast<double>(prep) - static_cast<double>(pre));
            if (!last_positive && found == INT32_MAX && lbase + at > target) found = e0 + i;
        }
    }
    const unsigned long long fl = __ballot(found != INT32_MAX);
    int token;
    if (fl) {
        token = __builtin_amdgcn_readlane(found, __ffsll(static_cast<long long>(fl)) - 1);
    } else {
        const unsigned long long pl = __ballot(lastpos >= 0);
        token = pl ? __builtin_amdgcn_readlane(lastpos, 63 - __clzll(static_cast<long long>(pl)))
                   : min(qstar * kQuart, a.V - 1);
    }
    if (a.given) {
        if (lane == 0) a.out_tokens[static_cast<int64_t>(b) * (g + 1) + d.pad] = token;
    } else if (lane_out) {
        // x_0 .. x_{k-1}, the drawn token, -1 padding: one entry per lane
        if (lane <= g)
            a.out_tokens[static_cast<int64_t>(b) * (g + 1) + lane] =
                lane < d.k ? xtok : (lane == d.k ? token : -1);
        if (lane == 0) a.accept_len[b] = d.k;
    } else {
        write_outputs<E>(a, b, d.k, token, lane, 64);
    }
    if (lane == 0 && a.final_dist) a.fin[b] = FinalState{W, kappa, fallback, 0};
}

template <class E>
__global__ __launch_bounds__(64) void chain_select_kernel(ChainArgs a) {
    const int b = blockIdx.x;
    select_block<E>(a, b, threadIdx.x, a.qsum + static_cast<int64_t>(b) * a.nquart,
                    a.qpos + static_cast<int64_t>(b) * a.nquart,
                    a.cdiff + static_cast<int64_t>(b) * a.nchunk, 0.0, nullptr);
}

// ---------------------------------------------------------------------------
// The whole final draw of a block in one workgroup of kBlockThreads threads,
// for batches with at least one block per compute unit (the launcher uses it
// for point-mass drafts): the decision once instead of once per chunk, the
// final row (and q_k for a residual) streamed with the quarter sums kept in
// LDS, then the selection on the first wave, reading the sums from LDS, with
// no selection launch and no quarter sums in HBM.  A
// quarter is the same 64 vectors as in the chunk kernel (wave w of tile j
// owns quarter 16j + w), its sum the same fp64 wave sum of the same lanes'
// fp32 sums, so the selection is the select kernel's; only the row's sum of
// P - Q' (the residual correction's input) is added in another order.
constexpr int kBlockThreads = 1024;
constexpr size_t kBlockDrawLds = 48 * 1024;  // its dynamic LDS at most

template <class E, int G>
__global__ __launch_bounds__(kBlockThreads) void chain_block_draw_kernel(ChainArgs a) {
    constexpr int NT = kBlockThreads, NW = NT / 64;
    constexpr int kTile = NT * E::kPerVec;
    extern __shared__ double s_dyn[];
    double* s_qs = s_dyn;                                      // [nquart] weight sums
    double* s_qp = s_qs + a.nquart;                            // [nquart] sums of P, D > 0
    Stat* s_part = reinterpret_cast<Stat*>(s_qp + a.nquart);  // [rows][nseg]
    __shared__ double s_d[NW];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const ChainDecision d = chain_decide<E, NT>(a, b, s_part);
    if (tid == 0) a.dec[b] = d;  // (the final_dist kernel reads it)
    const DrawRow r = draw_row(a, d);
    const bool resid = d.k >= 0 && r.resid;
    double dacc = 0.0;  // residual draw: this thread's share of sum (P - Q') over the row
    if (d.k >= 0) {
        const FinalRows<E> rows = final_rows<E>(a, b, d.k);
        const int ntile = (a.V + kTile - 1) / kTile;
        if (rows.vec_ok && a.V >= E::kPerVec) {
            if (r.resid)
                stream_tiles<E, G, true, NT>(rows, r, 0, ntile, a.V, s_qs, s_qp, a.nquart, dacc);
            else
                stream_tiles<E, G, false, NT>(rows, r, 0, ntile, a.V, s_qs, s_qp, a.nquart, dacc);
        } else {
            // rows not 16-byte aligned (or shorter than a vector): token by token
            for (int j = 0; j < ntile; ++j) {
                float zp[E::kPerVec], zq[E::kPerVec], w[E::kPerVec];
                const int e = j * kTile + tid * E::kPerVec;
                load_tokens<E>(rows, r.resid, e, a.V, zp, zq);
                const int qi = j * NW + wave;
                if (r.resid) {
                    float lw, ld, lp;
                    lane_resid_sums<E>(zp, zq, r, lw, ld, lp);
                    dacc += static_cast<double>(ld);
                    const double sw = wave_sum(static_cast<double>(lw));
                    const double sp = wave_sum(static_cast<double>(lp));
                    if (lane == 0 && qi < a.nquart) {
                        s_qs[qi] = sw;
                        s_qp[qi] = sp;
                    }
                } else {
                    const double sw =
                        wave_sum(static_cast<double>(lane_weights<E>(zp, zq, r, e, w)));
                    if (lane == 0 && qi < a.nquart) s_qs[qi] = sw;
                }
            }
        }
    }
    if (resid) {
        const double wd = wave_sum(dacc);
        if (lane == 0) s_d[wave] = wd;
    }
    __syncthreads();  // the quarter sums and the waves' sums are in LDS
    if (wave != 0) return;
    double rowd = 0.0;
    if (resid) {
#pragma unroll
        for (int i = 0; i < NW; ++i) rowd += s_d[i];
    }
    select_block<E>(a, b, lane, s_qs, s_qp, nullptr, rowd, &d);
}

template <class E>
__global__ __launch_bounds__(kThreads) void chain_dist_kernel(ChainArgs a) {
    const int b = blockIdx.x;
    const ChainDecision d = load_decision(a, b);
    float* out = a.final_dist + static_cast<int64_t>(b) * a.V;
    if (d.k < 0) {
        for (int e = threadIdx.x; e < a.V; e += kThreads) out[e] = 0.0f;
        return;
    }
    const FinalState f = a.fin[b];
    const FinalRows<E> rows = final_rows<E>(a, b, d.k);
    DrawRow r = draw_row(a, d);
    if (f.fallback) {
        r.resid = false;
        r.excl = -1;
    }
    const double inv = 1.0 / f.W;
    for (int e = threadIdx.x; e < a.V; e += kThreads) {
        const float zp = E::one(rows.p + e);
        double w;
        if (r.resid) {
            float wf, df, pzf;
            resid_terms<E>(zp, E::one(rows.q + e), r, wf, df, pzf);
            w = static_cast<double>(wf) +
                f.kappa * (static_cast<double>(pzf) - static_cast<double>(wf));
        } else {
            w = e == r.excl ? 0.0 : static_cast<double>(draw_weight<E>(zp, 0.0f, r));
        }
        out[e] = static_cast<float>(w * inv);
    }
}

}  // namespace

hipError_t launch_chain_stats(const ChainArgs& a, int dtype, hipStream_t s, hipEvent_t ev_start,
                              hipEvent_t ev_stop) {
    const dim3 grid(a.B * a.rows * a.nseg);
    // 8 vectors per thread per batch once a segment holds two such batches,
    // else 4 (a short segment would mostly re-read its last vector)
    const bool deep = a.seg_len / (kThreads * (dtype == 0 ? 4 : 8)) >= 16;
    if (dtype == 0)
        return deep ? launch_timed(chain_stats_kernel<F32, 8>, grid, dim3(kThreads), 0, s, ev_start, ev_stop, a)
                    : launch_timed(chain_stats_kernel<F32, 4>, grid, dim3(kThreads), 0, s, ev_start, ev_stop, a);
    return deep ? launch_timed(chain_stats_kernel<BF16, 8>, grid, dim3(kThreads), 0, s, ev_start, ev_stop, a)
                : launch_timed(chain_stats_kernel<BF16, 4>, grid, dim3(kThreads), 0, s, ev_start, ev_stop, a);
}

hipError_t launch_chain_chunks(const ChainArgs& a, int dtype, hipStream_t s) {
    const dim3 grid(a.B * a.nchunk);
    const size_t lds = a.given ? 0 : sizeof(Stat) * static_cast<size_t>(a.rows) * a.nseg;
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(kThreads), lds, s, a);
        return hipGetLastError();
    };
    if (dtype == 0) {
        if (a.chunk_tiles == 1) return go(chain_chunks_kernel<F32, 1>);
        if (a.chunk_tiles == 2) return go(chain_chunks_kernel<F32, 2>);
        return go(chain_chunks_kernel<F32, 4>);
    }
    // bf16 runs of more than two tiles stream in groups of two: at 8 tokens
    // per 16-byte vector the residual arithmetic per group is large enough,
    // and the smaller register footprint (under 80 VGPRs against over 100
    // with groups of four) keeps more waves per SIMD
    if (a.chunk_tiles == 1) return go(chain_chunks_kernel<BF16, 1>);
    return go(chain_chunks_kernel<BF16, 2>);
}

// LDS of chain_block_draw_kernel beyond its static arrays: the quarter sums
// and their sums of P, and the block's partials for the decision.
static size_t block_draw_lds(const ChainArgs& a) {
    return 2 * sizeof(double) * static_cast<size_t>(a.nquart) +
           sizeof(Stat) * static_cast<size_t>(a.rows) * a.nseg;
}

// Compute units of the current device, found once (every device this
// library runs on is the same part); 0 if the runtime cannot say.
static int device_cus() {
    static const int cus = [] {
        int dev = 0, n = 0;
        return (hipGetDevice(&dev) == hipSuccess &&
                hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
                   ? n
                   : 0;
    }();
    return cus;
}

hipError_t launch_chain_draw(const ChainArgs& a, int dtype, hipStream_t s) {
    // A point-mass draft's draw (one row, little arithmetic per token) runs
    // in one workgroup per block when the blocks cover the compute units,
    // the logits' rows are 16-byte aligned and the quarter sums fit in LDS.
    // A residual draw reads two rows and does more arithmetic per token; it
    // needs the chunk kernel's greater number of waves per compute unit to
    // hide its latencies (at B = 256 the single workgroup per block was
    // slower than chunks and selection), so ratio-test chains keep those.
    const size_t eb = dtype == 0 ? 4 : 2;
    const bool aligned = (reinterpret_cast<uintptr_t>(a.target) & 15u) == 0 &&
                         (static_cast<size_t>(a.V) * eb) % 16 == 0;
    const int cus = device_cus();
    if (a.pointmass && !a.given && aligned && cus > 0 && a.B >= cus &&
        block_draw_lds(a) <= kBlockDrawLds) {
        const size_t lds = block_draw_lds(a);
        if (dtype == 0)
            hipLaunchKernelGGL((chain_block_draw_kernel<F32, 2>), dim3(a.B), dim3(kBlockThreads), lds, s, a);
        else
            hipLaunchKernelGGL((chain_block_draw_kernel<BF16, 2>), dim3(a.B), dim3(kBlockThreads), lds, s, a);
        return hipGetLastError();
    }
    const hipError_t e = launch_chain_chunks(a, dtype, s);
    if (e != hipSuccess) return e;
    return launch_chain_select(a, dtype, s);
}

hipError_t launch_chain_select(const ChainArgs& a, int dtype, hipStream_t s) {
    if (dtype == 0)
        hipLaunchKernelGGL(chain_select_kernel<F32>, dim3(a.B), dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL(chain_select_kernel<BF16>, dim3(a.B), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_chain_dist(const ChainArgs& a, int dtype, hipStream_t s) {
    if (dtype == 0)
        hipLaunchKernelGGL(chain_dist_kernel<F32>, dim3(a.B), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(chain_dist_kernel<BF16>, dim3(a.B), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace sv
