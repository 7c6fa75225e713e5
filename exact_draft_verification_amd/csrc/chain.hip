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
// Kernels, in stream order (data crosses workgroups only at kernel
// boundaries, so no workgroup ever waits on another):
//  1. chain_stats: one workgroup per (block, row, segment) streams its share
//     of the 2*gamma+1 rows once, folds it into (m, R, S) statistics and
//     writes them as one partial; the workgroup whose segment holds a row's
//     draft token also records that token's logit.
//  2. chain_chunks: one workgroup per (block, chunk of the vocabulary) merges
//     the block's partials (staged in LDS), evaluates every ratio of the block
//     in fp64, finds the first rejection k, and sums the draw weights of its
//     chunk of the final row (residual row k, or the bonus row).
//  3. chain_select: one workgroup per block scans the chunk sums, finds the
//     chunk holding u_gamma * W and resolves the token inside it with one
//     workgroup-wide prefix sum in token order.
//  4. chain_dist (only when final_dist is requested): writes the normalised
//     draw distribution.
//
// Numerics.  Ratios are evaluated in the log2 domain in fp64 from the row
// statistics, so they are accurate to about 1e-8 whatever the dynamic range.
// The residual weight is formed as p(v) * (1 - 2^-D(v)) with
// D(v) = log2 p(v) - log2 q(v) computed in fp64 from the logit difference, so
// neither the subtraction p - q nor a constant offset between the target and
// draft logits costs precision; weights are fp32, sums and prefix sums fp64.
#include "sv_device.hpp"

namespace sv {

namespace {

constexpr double kDomain = 268435456.0;  // |m| / T limit (2^28)
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kStreamU = 4;              // 16-byte vectors per thread per batch

template <class E>
__device__ inline const typename E::storage* chain_row(const ChainArgs& a, int b, int rho) {
    using S = typename E::storage;
    if (rho <= a.gamma)
        return static_cast<const S*>(a.target) + (static_cast<int64_t>(b) * (a.gamma + 1) + rho) *
                                                     static_cast<int64_t>(a.V);
    return static_cast<const S*>(a.draft) +
           (static_cast<int64_t>(b) * a.gamma + (rho - a.gamma - 1)) * static_cast<int64_t>(a.V);
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
// (one partial per thread).
template <class E>
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
    stream_vectors<kStreamU>(reinterpret_cast<const char*>(row + sp.body_begin), sp.nvec, f);
    for (int e = sp.tail_begin + tid; e < sp.tail_end; e += kThreads) {
        float x = E::one(row + e);
        stat_fold<1>(f.s, &x, c_hi, c_lo);
    }
    return f.s;
}

template <class E>
__global__ __launch_bounds__(kThreads) void chain_stats_kernel(ChainArgs a) {
    __shared__ Stat s_w[kWaves];
    const int rows = 2 * a.gamma + 1;
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
    if (tid == 0) {
        const int i = rho < a.gamma ? rho : (rho > a.gamma ? rho - a.gamma - 1 : -1);
        if (i >= 0) {
            const int x = a.tokens[static_cast<int64_t>(b) * a.gamma + i];
            if (x >= e0 && x < e1) {
                zx = E::one(row + x);
                have_zx = true;
            }
        }
    }
    Stat st = row_range_stats<E>(row, e0, e1, a.c_hi, a.c_lo);
    st = block_reduce_stat(st, s_w);
    if (tid == 0) {
        a.part[unit] = st;
        if (have_zx) a.zx[rr] = zx;
    }
}

// Ratio tests of block b (every workgroup of the block's final draw takes
// them for itself): merges the block's row partials, staged in LDS, then for
// each draft position i evaluates r_i = min(1, p_i(x_i)/q_i(x_i)) in the
// log2 domain in fp64 and keeps the first i with u_i >= r_i.
template <class E>
__device__ ChainDecision chain_decide(const ChainArgs& a, int b, Stat* s_part) {
    __shared__ double s_L[2 * kMaxGamma + 1];
    __shared__ float s_R[2 * kMaxGamma + 1];
    __shared__ int s_bad, s_k;
    constexpr int kPer = kMaxBlockParts / kThreads;
    const int g = a.gamma, rows = 2 * g + 1, tid = threadIdx.x;
    const int np = rows * a.nseg;
    const Stat* src = a.part + static_cast<int64_t>(b) * np;
    {
        // every load issued before any LDS store (indices past the end
        // re-read the last partial and are not stored)
        Stat t[kPer];
#pragma unroll
        for (int m = 0; m < kPer; ++m) t[m] = src[min(tid + m * kThreads, np - 1)];
#pragma unroll
        for (int m = 0; m < kPer; ++m)
            if (tid + m * kThreads < np) s_part[tid + m * kThreads] = t[m];
    }
    if (tid == 0) {
        s_bad = 0;
        s_k = g;
    }
    __syncthreads();
    for (int r = tid; r < rows; r += kThreads) {
        const Stat* p = s_part + r * a.nseg;
        Stat t = p[0];
        for (int s = 1; s < a.nseg; ++s) t = stat_merge(t, p[s]);
        const bool ok = isfinite(t.S) && t.S > 0.0 && fabs(static_cast<double>(t.m) / a.T) <= kDomain;
        if (!ok) atomicOr(&s_bad, 1);
        s_L[r] = static_cast<double>(t.R) + log2(t.S);
        s_R[r] = t.R;
    }
    __syncthreads();
    const float* zx = a.zx + static_cast<int64_t>(b) * rows;
    for (int i = tid; i < g; i += kThreads) {
        const int x = a.tokens[static_cast<int64_t>(b) * g + i];
        if (x < 0 || x >= a.V) {
            atomicOr(&s_bad, 1);
            continue;
        }
        const float zp = zx[i];
        const float zq = zx[g + 1 + i];
        double r;
        if (zp == -INFINITY) {
            r = 0.0;
        } else if (zq == -INFINITY) {
            r = 1.0;
        } else {
            // log2 p(x) - log2 q(x), both rows' log2-sum-exp in fp64
            const double d = (static_cast<double>(zp) * a.c_d - s_L[i]) -
                             (static_cast<double>(zq) * a.c_d - s_L[g + 1 + i]);
            r = d >= 0.0 ? 1.0 : exp2(d);
        }
        const double u = static_cast<double>(a.uniforms[static_cast<int64_t>(b) * (g + 1) + i]);
        if (!(u < r)) atomicMin(&s_k, i);
    }
    __syncthreads();
    ChainDecision d;
    if (s_bad) {
        d.k = -1;
        d.Rp = 0.0f;
        d.dL = 0.0;
    } else {
        const int k = s_k;
        d.k = k;
        d.Rp = s_R[k];
        d.dL = k < g ? s_L[k] - s_L[g + 1 + k] : 0.0;
    }
    return d;
}

// ---------------------------------------------------------------------------
// Final draw.

struct DrawRow {
    float Rp, c_hi, c_lo;
    double c_d, dL;
    bool resid;  // residual of p_k and q_k (else p_k itself, unnormalised)
};

// Unnormalised draw weight of token v.  With P(v) = 2^(z_p c - R_p)
// (proportional to p_k(v)): residual  w = P(v) * (1 - 2^-D(v)) for D > 0,
// D(v) = log2 p_k(v) - log2 q_k(v) = (z_p - z_q) c - dL; bonus/fallback w = P(v).
__device__ inline float draw_weight(float zp, float zq, const DrawRow& r) {
    if (zp == -INFINITY) return 0.0f;
    float t = fmaf(zp, r.c_hi, -r.Rp);
    t = fmaf(zp, r.c_lo, t);
    const float P = __builtin_amdgcn_exp2f(t);
    if (!r.resid || zq == -INFINITY) return P;
    const double D = fma(static_cast<double>(zp) - static_cast<double>(zq), r.c_d, -r.dL);
    if (!(D > 0.0)) return 0.0f;
    return P * (-expm1f(static_cast<float>(-D) * kLn2));
}

template <class E>
struct FinalRows {
    const typename E::storage* p;
    const typename E::storage* q;  // nullptr unless resid
};

// Sum of draw weights over elements [e0, e1) by the whole workgroup (per
// thread partial, fp64).
template <class E>
__device__ inline double range_weight_sum(const FinalRows<E>& rows, int e0, int e1,
                                          const DrawRow& r) {
    const int tid = threadIdx.x;
    double acc = 0.0;
    if (e0 >= e1) return acc;
    const auto* p = rows.p;
    const auto* q = rows.q;
    const bool same_align =
        !r.resid || ((reinterpret_cast<uintptr_t>(q) - reinterpret_cast<uintptr_t>(p)) & 15u) == 0;
    if (!same_align) {
        for (int e = e0 + tid; e < e1; e += kThreads)
            acc += static_cast<double>(draw_weight(E::one(p + e), E::one(q + e), r));
        return acc;
    }
    const RangeSplit<E> sp = split_range<E>(p, e0, e1);
    for (int e = sp.head_begin + tid; e < sp.head_end; e += kThreads)
        acc += static_cast<double>(draw_weight(E::one(p + e), r.resid ? E::one(q + e) : 0.0f, r));
    const char* pb = reinterpret_cast<const char*>(p + sp.body_begin);
    const char* qb = r.resid ? reinterpret_cast<const char*>(q + sp.body_begin) : nullptr;
    for (int v = tid; v < sp.nvec; v += kThreads) {
        float xp[E::kPerVec], xq[E::kPerVec];
        E::unpack(load16_stream(pb + static_cast<size_t>(v) * 16), xp);
        if (r.resid) {
            E::unpack(load16_stream(qb + static_cast<size_t>(v) * 16), xq);
        } else {
#pragma unroll
            for (int i = 0; i < E::kPerVec; ++i) xq[i] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < E::kPerVec; ++i) acc += static_cast<double>(draw_weight(xp[i], xq[i], r));
    }
    for (int e = sp.tail_begin + tid; e < sp.tail_end; e += kThreads)
        acc += static_cast<double>(draw_weight(E::one(p + e), r.resid ? E::one(q + e) : 0.0f, r));
    return acc;
}

template <class E>
__device__ inline float weight_at(const FinalRows<E>& rows, int e, const DrawRow& r) {
    return draw_weight(E::one(rows.p + e), r.resid ? E::one(rows.q + e) : 0.0f, r);
}

template <class E>
__device__ void write_outputs(const ChainArgs& a, int b, int k, int token) {
    const int g = a.gamma;
    int32_t* out = a.out_tokens + static_cast<int64_t>(b) * (g + 1);
    for (int i = threadIdx.x; i <= g; i += kThreads) {
        int32_t v = -1;
        if (k >= 0) {
            if (i < k)
                v = a.tokens[static_cast<int64_t>(b) * g + i];
            else if (i == k)
                v = token;
        }
        out[i] = v;
    }
    if (threadIdx.x == 0) a.accept_len[b] = k;
}

// Token selection for block b (one workgroup), from the chunk sums of the
// chunk kernel.
//
// The draw is the smallest token v whose inclusive prefix sum of weights
// exceeds u * W (W the total).  The chunk holding that crossing is found from
// the chunk sums (one per thread, one workgroup-wide scan); inside the chunk,
// tile by tile, thread t holds the kPerVec consecutive tokens starting at
// tile + t*kPerVec, so one more workgroup scan of the per-thread sums puts
// every token's prefix in token order.  If rounding leaves no crossing, the
// last token of positive weight is taken.
template <class E>
__device__ void chain_select(const ChainArgs& a, int b, const ChainDecision& d,
                             const FinalRows<E>& rows, DrawRow r) {
    __shared__ double s_waves[kWaves];
    __shared__ double s_base;
    __shared__ int s_int;
    constexpr int kTile = kThreads * E::kPerVec;
    const int tid = threadIdx.x;
    const int g = a.gamma;
    double wc = 0.0;
    if (tid < a.nchunk) wc = a.chunk_sum[static_cast<int64_t>(b) * a.nchunk + tid];
    double total;
    double excl = block_exclusive_scan(wc, s_waves, &total);
    int fallback = 0;
    if (!(total > 0.0)) {
        // An empty residual (possible only through rounding after a
        // rejection): sample from p_k instead.
        fallback = 1;
        r.resid = false;
        double mine = 0.0;
        for (int c = 0; c < a.nchunk; ++c) {
            const int e0 = c * a.chunk_len, e1 = min(a.V, e0 + a.chunk_len);
            const double s = block_sum(range_weight_sum<E>(rows, e0, e1, r), s_waves);
            if (tid == c) mine = s;
        }
        wc = mine;
        excl = block_exclusive_scan(wc, s_waves, &total);
    }
    const double target =
        static_cast<double>(a.uniforms[static_cast<int64_t>(b) * (g + 1) + g]) * total;
    // first chunk whose inclusive prefix exceeds the target
    const int cand = (tid < a.nchunk && wc > 0.0 && excl + wc > target) ? tid : INT32_MAX;
    int cstar = block_min_int(cand, &s_int);
    bool last_positive = false;
    if (cstar == INT32_MAX) {
        // no crossing (rounding): the last token of positive weight
        cstar = block_max_int((tid < a.nchunk && wc > 0.0) ? tid : -1, &s_int);
        last_positive = true;
        if (cstar < 0) cstar = 0;  // no positive weight at all: keep every read in range
    }
    if (tid == cstar) s_base = excl;
    __syncthreads();
    double base = s_base;
    const int e0 = cstar * a.chunk_len, e1 = min(a.V, e0 + a.chunk_len);
    int token = -1, lastpos = -1;
    for (int t0 = e0; t0 < e1; t0 += kTile) {
        float w[E::kPerVec];
        double mine = 0.0;
        const int my0 = t0 + tid * E::kPerVec;
#pragma unroll
        for (int i = 0; i < E::kPerVec; ++i) {
            const int e = my0 + i;
            w[i] = e < e1 ? weight_at<E>(rows, e, r) : 0.0f;
            mine += static_cast<double>(w[i]);
        }
        double tile_total;
        const double my_excl = block_exclusive_scan(mine, s_waves, &tile_total);
        int found = INT32_MAX, lp = -1;
        double run = base + my_excl;
#pragma unroll
        for (int i = 0; i < E::kPerVec; ++i) {
            run += static_cast<double>(w[i]);
            if (w[i] > 0.0f) {
                lp = my0 + i;
                if (!last_positive && found == INT32_MAX && run > target) found = my0 + i;
            }
        }
        found = block_min_int(found, &s_int);
        lp = block_max_int(lp, &s_int);
        if (lp >= 0) lastpos = lp;
        if (found != INT32_MAX) {
            token = found;
            break;
        }
        base += tile_total;
    }
    if (token < 0) token = lastpos >= 0 ? lastpos : e0;
    write_outputs<E>(a, b, d.k, token);
    if (tid == 0 && a.final_dist) a.fin[b] = FinalState{total, fallback, 0};
}

template <class E>
__device__ inline FinalRows<E> final_rows(const ChainArgs& a, int b, int k) {
    using S = typename E::storage;
    FinalRows<E> f;
    f.p = static_cast<const S*>(a.target) + (static_cast<int64_t>(b) * (a.gamma + 1) + k) * a.V;
    f.q = k < a.gamma
              ? static_cast<const S*>(a.draft) + (static_cast<int64_t>(b) * a.gamma + k) * a.V
              : nullptr;
    return f;
}

__device__ inline DrawRow draw_row(const ChainArgs& a, const ChainDecision& d, bool resid) {
    return DrawRow{d.Rp, a.c_hi, a.c_lo, a.c_d, d.dL, resid};
}

// The decision of block b as written by the chunk kernel.  k is clamped to
// the invalid marker unless it lies in [0, gamma], so no row pointer is ever
// formed from an out-of-range value.
__device__ inline ChainDecision load_decision(const ChainArgs& a, int b) {
    ChainDecision d = a.dec[b];
    if (d.k < 0 || d.k > a.gamma) d.k = -1;
    return d;
}

template <class E>
__global__ __launch_bounds__(kThreads) void chain_chunks_kernel(ChainArgs a) {
    extern __shared__ Stat s_part[];  // [2*gamma+1][nseg]
    __shared__ double s_waves[kWaves];
    const int b = blockIdx.x / a.nchunk;
    const int c = blockIdx.x % a.nchunk;
    const ChainDecision d = chain_decide<E>(a, b, s_part);
    const bool valid = d.k >= 0;
    const FinalRows<E> rows = final_rows<E>(a, b, valid ? d.k : 0);
    const DrawRow r = draw_row(a, d, valid && d.k < a.gamma);
    const int e0 = c * a.chunk_len, e1 = min(a.V, e0 + a.chunk_len);
    const double s = valid ? block_sum(range_weight_sum<E>(rows, e0, e1, r), s_waves) : 0.0;
    if (threadIdx.x == 0) {
        a.chunk_sum[static_cast<int64_t>(b) * a.nchunk + c] = s;
        if (c == 0) a.dec[b] = d;
    }
}

template <class E>
__global__ __launch_bounds__(kThreads) void chain_select_kernel(ChainArgs a) {
    const int b = blockIdx.x;
    const ChainDecision d = load_decision(a, b);
    if (d.k < 0) {
        write_outputs<E>(a, b, -1, -1);
        return;
    }
    const FinalRows<E> rows = final_rows<E>(a, b, d.k);
    chain_select<E>(a, b, d, rows, draw_row(a, d, d.k < a.gamma));
}

template <class E>
__global__ __launch_bounds__(kThreads) void chain_dist_kernel(ChainArgs a) {
    const int b = blockIdx.x / a.nchunk;
    const int c = blockIdx.x % a.nchunk;
    const ChainDecision d = load_decision(a, b);
    const int e0 = c * a.chunk_len, e1 = min(a.V, e0 + a.chunk_len);
    float* out = a.final_dist + static_cast<int64_t>(b) * a.V;
    if (d.k < 0) {
        for (int e = e0 + threadIdx.x; e < e1; e += kThreads) out[e] = 0.0f;
        return;
    }
    const FinalState f = a.fin[b];
    const FinalRows<E> rows = final_rows<E>(a, b, d.k);
    const DrawRow r = draw_row(a, d, d.k < a.gamma && !f.fallback);
    const double inv = 1.0 / f.W;
    for (int e = e0 + threadIdx.x; e < e1; e += kThreads)
        out[e] = static_cast<float>(static_cast<double>(weight_at<E>(rows, e, r)) * inv);
}

}  // namespace

hipError_t launch_chain_stats(const ChainArgs& a, int dtype, hipStream_t s) {
    const int grid = a.B * (2 * a.gamma + 1) * a.nseg;
    if (dtype == 0)
        hipLaunchKernelGGL(chain_stats_kernel<F32>, dim3(grid), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(chain_stats_kernel<BF16>, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_chain_chunks(const ChainArgs& a, int dtype, hipStream_t s) {
    const int grid = a.B * a.nchunk;
    const size_t lds = sizeof(Stat) * static_cast<size_t>(2 * a.gamma + 1) * a.nseg;
    if (dtype == 0)
        hipLaunchKernelGGL(chain_chunks_kernel<F32>, dim3(grid), dim3(kThreads), lds, s, a);
    else
        hipLaunchKernelGGL(chain_chunks_kernel<BF16>, dim3(grid), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_chain_select(const ChainArgs& a, int dtype, hipStream_t s) {
    if (dtype == 0)
        hipLaunchKernelGGL(chain_select_kernel<F32>, dim3(a.B), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(chain_select_kernel<BF16>, dim3(a.B), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_chain_dist(const ChainArgs& a, int dtype, hipStream_t s) {
    const int grid = a.B * a.nchunk;
    if (dtype == 0)
        hipLaunchKernelGGL(chain_dist_kernel<F32>, dim3(grid), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(chain_dist_kernel<BF16>, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace sv
