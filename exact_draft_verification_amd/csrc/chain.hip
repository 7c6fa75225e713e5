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
// Kernels, in stream order:
//  1. chain_stats: one workgroup per (block, row, segment) streams its share
//     of the 2*gamma+1 rows once and folds it into (m, R, S) statistics; the
//     last workgroup to finish a block (arrival counter) merges the block's
//     statistics, evaluates every ratio in fp64 and finds k.
//  2. chain_final: one workgroup per (block, chunk of the final row) sums the
//     draw weights of its chunk; the last workgroup of a block scans the chunk
//     sums, finds the chunk holding u_gamma * W and rescans that chunk alone
//     in token order to pick the token.
//  3. chain_dist (only when final_dist is requested): writes the normalised
//     draw distribution.
//
// Numerics.  Ratios are evaluated in the log2 domain in fp64 from the row
// statistics, so they are accurate to about 1e-8 whatever the dynamic range.
// The residual weight is formed as p(v) * (1 - 2^-D(v)) with
// D(v) = log2 p(v) - log2 q(v) computed from the logit difference, which
// avoids the cancellation of p - q when the two rows are close; weights are
// fp32, sums and prefix sums fp64.
#include "sv_device.hpp"

namespace sv {

namespace {

constexpr double kDomain = 268435456.0;  // |m| / T limit (2^28)
constexpr float kLn2 = 0.693147180559945309f;

template <class E>
__device__ inline const typename E::storage* chain_row(const ChainArgs& a, int b, int rho) {
    using S = typename E::storage;
    if (rho <= a.gamma)
        return static_cast<const S*>(a.target) + (static_cast<int64_t>(b) * (a.gamma + 1) + rho) *
                                                     static_cast<int64_t>(a.V);
    return static_cast<const S*>(a.draft) +
           (static_cast<int64_t>(b) * a.gamma + (rho - a.gamma - 1)) * static_cast<int64_t>(a.V);
}

// Statistics of elements [e0, e1) of one row, folded by the whole workgroup.
template <class E>
__device__ inline Stat row_range_stats(const typename E::storage* row, int e0, int e1, float c_hi,
                                       float c_lo) {
    constexpr int U = 4;                 // 16-byte vectors per thread per batch
    constexpr int NB = U * E::kPerVec;   // elements per thread per batch
    constexpr int kBatchVec = kThreads * U;
    const int tid = threadIdx.x;
    Stat st = stat_empty();
    if (e0 >= e1) return st;
    const RangeSplit<E> sp = split_range<E>(row, e0, e1);
    for (int e = sp.head_begin + tid; e < sp.head_end; e += kThreads) {
        float x = E::one(row + e);
        stat_fold<1>(st, &x, c_hi, c_lo);
    }
    const char* body = reinterpret_cast<const char*>(row + sp.body_begin);
    const int nfull = sp.nvec / kBatchVec;
    if (nfull > 0) {
        // Two register buffers alternate so that the loads of batch t+1 are in
        // flight while batch t is folded.
        uint4 A[U], Bv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) A[u] = load16(body + static_cast<size_t>(u * kThreads + tid) * 16);
        for (int t = 0; t < nfull; t += 2) {
            const bool has1 = t + 1 < nfull;
            if (has1) {
                const char* nb = body + static_cast<size_t>(t + 1) * kBatchVec * 16;
#pragma unroll
                for (int u = 0; u < U; ++u) Bv[u] = load16(nb + static_cast<size_t>(u * kThreads + tid) * 16);
            }
            {
                float x[NB];
#pragma unroll
                for (int u = 0; u < U; ++u) E::unpack(A[u], x + u * E::kPerVec);
                if (t + 2 < nfull) {
                    const char* nb = body + static_cast<size_t>(t + 2) * kBatchVec * 16;
#pragma unroll
                    for (int u = 0; u < U; ++u) A[u] = load16(nb + static_cast<size_t>(u * kThreads + tid) * 16);
                }
                stat_fold<NB>(st, x, c_hi, c_lo);
            }
            if (has1) {
                float x[NB];
#pragma unroll
                for (int u = 0; u < U; ++u) E::unpack(Bv[u], x + u * E::kPerVec);
                stat_fold<NB>(st, x, c_hi, c_lo);
            }
        }
    }
    for (int v = nfull * kBatchVec + tid; v < sp.nvec; v += kThreads) {
        float x[E::kPerVec];
        E::unpack(load16(body + static_cast<size_t>(v) * 16), x);
        stat_fold<E::kPerVec>(st, x, c_hi, c_lo);
    }
    for (int e = sp.tail_begin + tid; e < sp.tail_end; e += kThreads) {
        float x = E::one(row + e);
        stat_fold<1>(st, &x, c_hi, c_lo);
    }
    return st;
}

__device__ inline Stat block_reduce_stat(Stat st) {
    __shared__ Stat s_w[kWaves];
    st = wave_reduce_stat(st);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) s_w[wave] = st;
    __syncthreads();
    Stat r = s_w[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = stat_merge(r, s_w[w]);
    return r;
}

// Ratio tests of block b: runs in the last statistics workgroup of the block.
template <class E>
__device__ void chain_decide(const ChainArgs& a, int b) {
    using S = typename E::storage;
    __shared__ double s_L[2 * kMaxGamma + 1];
    __shared__ float s_R[2 * kMaxGamma + 1];
    __shared__ int s_bad, s_k;
    const int g = a.gamma, rows = 2 * g + 1, tid = threadIdx.x;
    if (tid == 0) {
        s_bad = 0;
        s_k = g;
    }
    __syncthreads();
    for (int r = tid; r < rows; r += kThreads) {
        Stat* p = a.part + (static_cast<int64_t>(b) * rows + r) * a.nseg;
        Stat t = p[0];
        for (int s = 1; s < a.nseg; ++s) t = stat_merge(t, p[s]);
        for (int s = 0; s < a.nseg; ++s) p[s] = Stat{0.0f, 0.0f, 0.0};  // this call's last reader
        const bool ok = isfinite(t.S) && t.S > 0.0 && fabs(static_cast<double>(t.m) / a.T) <= kDomain;
        if (!ok) atomicOr(&s_bad, 1);
        s_L[r] = static_cast<double>(t.R) + log2(t.S);
        s_R[r] = t.R;
    }
    __syncthreads();
    const S* tg = static_cast<const S*>(a.target) + static_cast<int64_t>(b) * (g + 1) * a.V;
    const S* dr = static_cast<const S*>(a.draft) + static_cast<int64_t>(b) * g * a.V;
    for (int i = tid; i < g; i += kThreads) {
        const int x = a.tokens[static_cast<int64_t>(b) * g + i];
        if (x < 0 || x >= a.V) {
            atomicOr(&s_bad, 1);
            continue;
        }
        const float zp = E::one(tg + static_cast<int64_t>(i) * a.V + x);
        const float zq = E::one(dr + static_cast<int64_t>(i) * a.V + x);
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
    if (tid == 0) {
        ChainDecision d;
        if (s_bad) {
            d.k = -1;
            d.Rp = d.Rq = d.dL = 0.0f;
        } else {
            const int k = s_k;
            d.k = k;
            d.Rp = s_R[k];
            if (k < g) {
                d.Rq = s_R[g + 1 + k];
                d.dL = static_cast<float>(s_L[k] - s_L[g + 1 + k]);
            } else {
                d.Rq = 0.0f;
                d.dL = 0.0f;
            }
        }
        a.dec[b] = d;
        a.cnt_stats[b] = 0u;  // leave the counter ready for the next call
    }
}

template <class E>
__global__ __launch_bounds__(kThreads) void chain_stats_kernel(ChainArgs a) {
    const int rows = 2 * a.gamma + 1;
    const int unit = blockIdx.x;
    const int seg = unit % a.nseg;
    const int rr = unit / a.nseg;
    const int rho = rr % rows;
    const int b = rr / rows;
    const auto* row = chain_row<E>(a, b, rho);
    const int e0 = seg * a.seg_len;
    const int e1 = min(a.V, e0 + a.seg_len);
    Stat st = row_range_stats<E>(row, e0, e1, a.c_hi, a.c_lo);
    st = block_reduce_stat(st);
    __shared__ int s_last;
    if (threadIdx.x == 0) {
        a.part[unit] = st;
        const unsigned prev = arrive(&a.cnt_stats[b]);
        s_last = (prev == static_cast<unsigned>(rows * a.nseg - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    chain_decide<E>(a, b);
}

// ---------------------------------------------------------------------------
// Final draw.

struct DrawRow {
    float Rp, Rq, dL, c_hi, c_lo;
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
    const float dz = zp - zq;
    const float D = fmaf(dz, r.c_hi, fmaf(dz, r.c_lo, -r.dL));
    if (!(D > 0.0f)) return 0.0f;
    return P * (-expm1f(-D * kLn2));
}

template <class E>
struct FinalRows {
    const typename E::storage* p;
    const typename E::storage* q;  // nullptr unless resid
};

// Sum of draw weights over elements [e0, e1) by the whole workgroup (per
// thread partial, fp64).
template <class E>
__device__ inline double range_weight_sum(const FinalRows<E>& rows, int e0, int e1, const DrawRow& r) {
    const int tid = threadIdx.x;
    double acc = 0.0;
    if (e0 >= e1) return acc;
    const auto* p = rows.p;
    const auto* q = rows.q;
    const bool same_align =
        !r.resid || ((reinterpret_cast<uintptr_t>(q) - reinterpret_cast<uintptr_t>(p)) & 15u) == 0;
    if (!same_align) {
        for (int e = e0 + tid; e < e1; e += kThreads)
            acc += draw_weight(E::one(p + e), E::one(q + e), r);
        return acc;
    }
    const RangeSplit<E> sp = split_range<E>(p, e0, e1);
    for (int e = sp.head_begin + tid; e < sp.head_end; e += kThreads)
        acc += draw_weight(E::one(p + e), r.resid ? E::one(q + e) : 0.0f, r);
    const char* pb = reinterpret_cast<const char*>(p + sp.body_begin);
    const char* qb = r.resid ? reinterpret_cast<const char*>(q + sp.body_begin) : nullptr;
    for (int v = tid; v < sp.nvec; v += kThreads) {
        float xp[E::kPerVec], xq[E::kPerVec];
        E::unpack(load16(pb + static_cast<size_t>(v) * 16), xp);
        if (r.resid) {
            E::unpack(load16(qb + static_cast<size_t>(v) * 16), xq);
        } else {
#pragma unroll
            for (int i = 0; i < E::kPerVec; ++i) xq[i] = 0.0f;
        }
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < E::kPerVec; ++i) s += draw_weight(xp[i], xq[i], r);
        acc += static_cast<double>(s);
    }
    for (int e = sp.tail_begin + tid; e < sp.tail_end; e += kThreads)
        acc += draw_weight(E::one(p + e), r.resid ? E::one(q + e) : 0.0f, r);
    return acc;
}

template <class E>
__device__ inline float weight_at(const FinalRows<E>& rows, int e, const DrawRow& r) {
    return draw_weight(E::one(rows.p + e), r.resid ? E::one(rows.q + e) : 0.0f, r);
}

__device__ inline int block_min_int(int v, int* lds) {
    if (threadIdx.x == 0) *lds = INT32_MAX;
    __syncthreads();
    atomicMin(lds, v);
    __syncthreads();
    const int r = *lds;
    __syncthreads();
    return r;
}

__device__ inline int block_max_int(int v, int* lds) {
    if (threadIdx.x == 0) *lds = INT32_MIN;
    __syncthreads();
    atomicMax(lds, v);
    __syncthreads();
    const int r = *lds;
    __syncthreads();
    return r;
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

// Token selection for block b: runs in the last final-draw workgroup, after
// every chunk sum of the block is in.  Clears the chunk sums it read.
template <class E>
__device__ void chain_select(const ChainArgs& a, int b, const ChainDecision& d, FinalRows<E> rows,
                             DrawRow r) {
    __shared__ double s_waves[kWaves];
    __shared__ double s_chunk[kMaxChunks];
    __shared__ double s_excl;
    __shared__ int s_int;
    const int tid = threadIdx.x;
    const int g = a.gamma;
    double wc = 0.0;
    if (tid < a.nchunk) {
        double* slot = a.chunk_sum + static_cast<int64_t>(b) * a.nchunk + tid;
        wc = *slot;
        *slot = 0.0;
    }
    double total;
    double excl = block_exclusive_scan(wc, s_waves, &total);
    int fallback = 0;
    if (!(total > 0.0)) {
        // An empty residual (possible only through rounding after a
        // rejection): sample from p_k instead.
        fallback = 1;
        r.resid = false;
        for (int c = 0; c < a.nchunk; ++c) {
            const int e0 = c * a.chunk_len, e1 = min(a.V, e0 + a.chunk_len);
            const double s = block_sum(range_weight_sum<E>(rows, e0, e1, r), s_waves);
            if (tid == 0) s_chunk[c] = s;
        }
        __syncthreads();
        wc = tid < a.nchunk ? s_chunk[tid] : 0.0;
        excl = block_exclusive_scan(wc, s_waves, &total);
    }
    const double target = static_cast<double>(a.uniforms[static_cast<int64_t>(b) * (g + 1) + g]) * total;
    // first chunk whose inclusive prefix exceeds the target
    int cand = (tid < a.nchunk && wc > 0.0 && excl + wc > target) ? tid : INT32_MAX;
    int cstar = block_min_int(cand, &s_int);
    bool last_positive = false;
    if (cstar == INT32_MAX) {
        // no crossing (rounding, or u >= 1): last token of positive weight
        cstar = block_max_int((tid < a.nchunk && wc > 0.0) ? tid : -1, &s_int);
        last_positive = true;
        if (cstar < 0) cstar = 0;  // no positive weight at all: keep every read in range
    }
    if (tid == 0) s_excl = 0.0;
    __syncthreads();
    if (tid == cstar) s_excl = excl;
    __syncthreads();
    const double base = s_excl;
    const int e0 = cstar * a.chunk_len, e1 = min(a.V, e0 + a.chunk_len);
    const int len = e1 - e0;
    const int per = (len + kThreads - 1) / kThreads;
    const int m0 = min(e1, e0 + tid * per), m1 = min(e1, m0 + per);
    double mine = 0.0;
    for (int e = m0; e < m1; ++e) mine += static_cast<double>(weight_at<E>(rows, e, r));
    double tot2;
    const double my_excl = block_exclusive_scan(mine, s_waves, &tot2);
    int found = INT32_MAX;
    if (!last_positive) {
        double run = base + my_excl;
        for (int e = m0; e < m1; ++e) {
            run += static_cast<double>(weight_at<E>(rows, e, r));
            if (run > target) {
                found = e;
                break;
            }
        }
    }
    int token = block_min_int(found, &s_int);
    if (token == INT32_MAX) {
        int lastpos = -1;
        for (int e = m0; e < m1; ++e)
            if (weight_at<E>(rows, e, r) > 0.0f) lastpos = e;
        token = block_max_int(lastpos, &s_int);
    }
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
    return DrawRow{d.Rp, d.Rq, d.dL, a.c_hi, a.c_lo, resid};
}

// The decision of block b as written by the statistics kernel.  k is clamped
// to the invalid marker unless it lies in [0, gamma], so no row pointer is
// ever formed from an out-of-range value.
__device__ inline ChainDecision load_decision(const ChainArgs& a, int b) {
    ChainDecision d = a.dec[b];
    if (d.k < 0 || d.k > a.gamma) d.k = -1;
    return d;
}

template <class E>
__global__ __launch_bounds__(kThreads) void chain_final_kernel(ChainArgs a) {
    __shared__ double s_waves[kWaves];
    __shared__ int s_last;
    const int b = blockIdx.x / a.nchunk;
    const int c = blockIdx.x % a.nchunk;
    const ChainDecision d = load_decision(a, b);
    const bool valid = d.k >= 0;
    const FinalRows<E> rows = final_rows<E>(a, b, valid ? d.k : 0);
    const DrawRow r = draw_row(a, d, valid && d.k < a.gamma);
    const int e0 = c * a.chunk_len, e1 = min(a.V, e0 + a.chunk_len);
    const double s = valid ? block_sum(range_weight_sum<E>(rows, e0, e1, r), s_waves) : 0.0;
    if (threadIdx.x == 0) {
        a.chunk_sum[static_cast<int64_t>(b) * a.nchunk + c] = s;
        const unsigned prev = arrive(&a.cnt_final[b]);
        s_last = (prev == static_cast<unsigned>(a.nchunk - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (valid) {
        chain_select<E>(a, b, d, rows, r);
    } else {
        for (int i = threadIdx.x; i < a.nchunk; i += kThreads)
            a.chunk_sum[static_cast<int64_t>(b) * a.nchunk + i] = 0.0;
        write_outputs<E>(a, b, -1, -1);
    }
    if (threadIdx.x == 0) {
        // every workgroup of this block has read the decision by now; the
        // final_dist pass, when requested, still needs it (and clears it)
        if (!a.final_dist) a.dec[b] = ChainDecision{0, 0.0f, 0.0f, 0.0f};
        a.cnt_final[b] = 0u;
    }
}

template <class E>
__global__ __launch_bounds__(kThreads) void chain_dist_kernel(ChainArgs a) {
    __shared__ int s_last;
    const int b = blockIdx.x / a.nchunk;
    const int c = blockIdx.x % a.nchunk;
    const ChainDecision d = load_decision(a, b);
    const FinalState f = a.fin[b];
    const int e0 = c * a.chunk_len, e1 = min(a.V, e0 + a.chunk_len);
    float* out = a.final_dist + static_cast<int64_t>(b) * a.V;
    if (d.k < 0) {
        for (int e = e0 + threadIdx.x; e < e1; e += kThreads) out[e] = 0.0f;
    } else {
        const FinalRows<E> rows = final_rows<E>(a, b, d.k);
        const DrawRow r = draw_row(a, d, d.k < a.gamma && !f.fallback);
        const double inv = 1.0 / f.W;
        for (int e = e0 + threadIdx.x; e < e1; e += kThreads)
            out[e] = static_cast<float>(static_cast<double>(weight_at<E>(rows, e, r)) * inv);
    }
    __syncthreads();  // every thread of this workgroup has read dec[b] and fin[b]
    if (threadIdx.x == 0) {
        const unsigned prev = arrive(&a.cnt_dist[b]);
        s_last = (prev == static_cast<unsigned>(a.nchunk - 1));
    }
    __syncthreads();
    if (s_last && threadIdx.x == 0) {
        a.dec[b] = ChainDecision{0, 0.0f, 0.0f, 0.0f};
        a.fin[b] = FinalState{0.0, 0, 0};
        a.cnt_dist[b] = 0u;
    }
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

hipError_t launch_chain_final(const ChainArgs& a, int dtype, hipStream_t s) {
    const int grid = a.B * a.nchunk;
    if (dtype == 0)
        hipLaunchKernelGGL(chain_final_kernel<F32>, dim3(grid), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(chain_final_kernel<BF16>, dim3(grid), dim3(kThreads), 0, s, a);
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
