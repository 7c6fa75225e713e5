// Greedy tree verification kernel for gfx950.
//
// The rule ("JetSpec reading notes", section "Tree verification", Fig. 5 and
// the greedy note; parent pointers as built by Algorithm 1): node j of a draft
// tree is accepted iff its parent is accepted and its token equals the target
// argmax after the parent's path; the deepest accepted node v* is kept (the
// lowest node index among equally deep ones), its path is committed and the
// target argmax after v* is emitted as the extra token.
//
// Two launches (data crosses workgroups only at the kernel boundary):
//  1. tree_argmax: one workgroup per segment of one node row finds the largest
//     logit and the lowest index holding it (plus a NaN flag) and writes it as
//     one partial.
//  2. tree_resolve: one workgroup per request merges its rows' partials
//     (staged in LDS), validates the parent array and resolves every node's
//     acceptance and depth by pointer jumping in LDS (ceil(log2 n) rounds),
//     then writes the path.
#include "sv_device.hpp"

namespace sv {

namespace {

struct Best {
    float v;
    int idx;
};

// Keep the larger value; on equal values the lower index.
__device__ inline Best best_merge(Best a, Best b) {
    if (b.v > a.v || (b.v == a.v && b.idx < a.idx)) return b;
    return a;
}

// Fold a batch of N elements whose token ids are idx_of(i), increasing in i.
template <int N, class IdxFn>
__device__ inline void argmax_fold(Best& best, const float* x, IdxFn idx_of) {
    float bm = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) bm = fmaxf(bm, x[i]);
    if (bm > best.v) {
        int first = N - 1;
#pragma unroll
        for (int i = N - 1; i >= 0; --i)
            if (x[i] == bm) first = i;
        best.v = bm;
        best.idx = idx_of(first);
    }
}

// NaN flag for one 16-byte vector, from the raw bits.
__device__ inline uint32_t nan_bits(const uint4& v, F32) {
    // (|x| bits) + 0x007fffff has bit 31 set iff |x| > +inf, i.e. NaN
    return ((v.x & 0x7fffffffu) + 0x007fffffu) | ((v.y & 0x7fffffffu) + 0x007fffffu) |
           ((v.z & 0x7fffffffu) + 0x007fffffu) | ((v.w & 0x7fffffffu) + 0x007fffffu);
}
__device__ inline uint32_t nan_bits(const uint4& v, BF16) {
    // per 16-bit half: (|x| bits) + 0x007f sets the half's top bit iff NaN
    constexpr uint32_t M = 0x7fff7fffu, A = 0x007f007fu;
    return ((v.x & M) + A) | ((v.y & M) + A) | ((v.z & M) + A) | ((v.w & M) + A);
}
__device__ inline uint32_t nan_mask(F32) { return 0x80000000u; }
__device__ inline uint32_t nan_mask(BF16) { return 0x80008000u; }

template <class E>
struct ArgmaxFolder {
    Best best;
    uint32_t nanacc;
    int body_begin;
    template <int N>
    __device__ inline void batch(const uint4* v, int v0) {
        float x[N * E::kPerVec];
#pragma unroll
        for (int u = 0; u < N; ++u) {
            E::unpack(v[u], x + u * E::kPerVec);
            nanacc |= nan_bits(v[u], E{});
        }
        // element i of the batch is element w of vector v0 + u*kThreads
        argmax_fold<N * E::kPerVec>(best, x, [&](int i) {
            const int u = i / E::kPerVec, w = i % E::kPerVec;
            return body_begin + (v0 + u * kThreads) * E::kPerVec + w;
        });
    }
};

template <class E, int U>
__device__ inline void range_argmax(const typename E::storage* row, int e0, int e1, Best& best,
                                    uint32_t& nanacc, bool& nan_scalar) {
    const int tid = threadIdx.x;
    if (e0 >= e1) return;
    const RangeSplit<E> sp = split_range<E>(row, e0, e1);
    for (int e = sp.head_begin + tid; e < sp.head_end; e += kThreads) {
        const float x = E::one(row + e);
        nan_scalar |= isnan(x);
        argmax_fold<1>(best, &x, [&](int) { return e; });
    }
    ArgmaxFolder<E> f{best, nanacc, sp.body_begin};
    stream_vectors<U>(reinterpret_cast<const char*>(row + sp.body_begin), sp.nvec, f);
    best = f.best;
    nanacc = f.nanacc;
    for (int e = sp.tail_begin + tid; e < sp.tail_end; e += kThreads) {
        const float x = E::one(row + e);
        nan_scalar |= isnan(x);
        argmax_fold<1>(best, &x, [&](int) { return e; });
    }
}

// Path resolution for request b (one workgroup).
__device__ void tree_resolve(const TreeArgs& a, int b, ArgmaxPart* s_part) {
    __shared__ int s_par[kMaxTreeNodes];
    __shared__ int s_tok[kMaxTreeNodes];
    __shared__ int s_anc[kMaxTreeNodes];
    __shared__ int s_dep[kMaxTreeNodes];
    __shared__ int s_amax[kMaxTreeNodes];
    __shared__ unsigned char s_ok[kMaxTreeNodes];
    __shared__ int s_bad, s_key;
    constexpr int kStage = kMaxBlockParts / kThreads;
    constexpr int kNodes = kMaxTreeNodes / kThreads;
    const int n = a.n, tid = threadIdx.x;
    const int32_t* par = a.parents + static_cast<int64_t>(b) * n;
    const int32_t* tok = a.tokens + static_cast<int64_t>(b) * n;
    int32_t* out = a.out_tokens + static_cast<int64_t>(b) * n;
    {
        // stage the request's n*nseg row partials and every node's parent
        // and token: all loads issued before any LDS store (partial indices
        // past the end re-read the last partial and are not stored)
        static_assert(sizeof(ArgmaxPart) == 16, "ArgmaxPart is staged as one 16-byte vector");
        const int np = n * a.nseg;
        const uint4* src = reinterpret_cast<const uint4*>(a.part + static_cast<int64_t>(b) * np);
        uint4* dst = reinterpret_cast<uint4*>(s_part);
        uint4 t[kStage];
        int pv[kNodes], tv[kNodes];
#pragma unroll
        for (int m = 0; m < kStage; ++m)
            t[m] = m * kThreads < np ? src[min(tid + m * kThreads, np - 1)] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int q = 0; q < kNodes; ++q) {
            const int j = tid + q * kThreads;
            pv[q] = j < n ? par[j] : 0;
            tv[q] = j < n ? tok[j] : 0;
        }
#pragma unroll
        for (int m = 0; m < kStage; ++m)
            if (tid + m * kThreads < np) dst[tid + m * kThreads] = t[m];
#pragma unroll
        for (int q = 0; q < kNodes; ++q) {
            const int j = tid + q * kThreads;
            if (j < n) {
                s_par[j] = pv[q];
                s_tok[j] = tv[q];
            }
        }
    }
    if (tid == 0) {
        s_bad = 0;
        s_key = -1;
    }
    __syncthreads();
    for (int j = tid; j < n; j += kThreads) {
        const ArgmaxPart* p = s_part + j * a.nseg;
        Best best{p[0].best, p[0].idx};
        uint32_t bad = p[0].bad;
        for (int s = 1; s < a.nseg; ++s) {
            best = best_merge(best, Best{p[s].best, p[s].idx});
            bad |= p[s].bad;
        }
        // a valid row has no NaN, no +inf and at least one finite logit
        if (bad || !(best.v > -INFINITY) || best.v == INFINITY) s_bad = 1;
        s_amax[j] = best.idx;
        const int pj = s_par[j];
        if (j == 0) {
            if (pj != -1) s_bad = 1;
        } else if (pj < 0 || pj >= j || s_tok[j] < 0 || s_tok[j] >= a.V) {
            s_bad = 1;
        }
    }
    __syncthreads();
    if (s_bad) {
        for (int j = tid; j < n; j += kThreads) out[j] = -1;
        if (tid == 0) {
            a.accept_len[b] = -1;
            a.accept_node[b] = -1;
        }
        return;
    }
    // acceptance of the edge into each node, then pointer jumping: after each
    // round s_anc[j] is 2^r levels up (or the root), s_dep[j] the distance to
    // it and s_ok[j] whether every edge in between matched.
    for (int j = tid; j < n; j += kThreads) {
        if (j == 0) {
            s_anc[0] = 0;
            s_dep[0] = 0;
            s_ok[0] = 1;
        } else {
            s_anc[j] = s_par[j];
            s_dep[j] = 1;
            s_ok[j] = s_tok[j] == s_amax[s_par[j]];
        }
    }
    __syncthreads();
    deepest_accepted(n, s_anc, s_dep, s_ok, &s_key);
    const int key = s_key;
    const int depth = key >> 11;
    const int vstar = 2047 - (key & 2047);
    for (int j = depth + 1 + tid; j < n; j += kThreads) out[j] = -1;
    if (tid == 0) {
        int v = vstar;
        for (int d = depth; d >= 1; --d) {
            out[d - 1] = s_tok[v];
            v = s_par[v];
        }
        out[depth] = s_amax[vstar];
        a.accept_len[b] = depth;
        a.accept_node[b] = vstar;
    }
}

// Merge of one ArgmaxPart per thread across the workgroup (every thread
// gets the result; safe to call repeatedly).
__device__ inline ArgmaxPart block_reduce_argmax(Best best, uint32_t bad, ArgmaxPart* lds_waves) {
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) {
        Best o{__shfl_xor(best.v, mask, 64), __shfl_xor(best.idx, mask, 64)};
        best = best_merge(best, o);
        bad |= __shfl_xor(bad, mask, 64);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) lds_waves[wave] = ArgmaxPart{best.v, best.idx, bad, 0u};
    __syncthreads();
    Best r{lds_waves[0].best, lds_waves[0].idx};
    uint32_t rb = lds_waves[0].bad;
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        r = best_merge(r, Best{lds_waves[w].best, lds_waves[w].idx});
        rb |= lds_waves[w].bad;
    }
    return ArgmaxPart{r.v, r.idx, rb, 0u};
}

template <class E, int U>
__global__ __launch_bounds__(kThreads) void tree_argmax_kernel(TreeArgs a) {
    __shared__ ArgmaxPart s_w[kWaves];
    const int unit = blockIdx.x;
    const int seg = unit % a.nseg;
    const int rr = unit / a.nseg;  // = b * n + j
    using S = typename E::storage;
    const S* row = static_cast<const S*>(a.target) + static_cast<int64_t>(rr) * a.V;
    const int e0 = seg * a.seg_len;
    const int e1 = min(a.V, e0 + a.seg_len);
    Best best{-INFINITY, INT32_MAX};
    uint32_t nanacc = 0;
    bool nan_scalar = false;
    range_argmax<E, U>(row, e0, e1, best, nanacc, nan_scalar);
    const uint32_t bad = ((nanacc & nan_mask(E{})) != 0u || nan_scalar) ? 1u : 0u;
    const ArgmaxPart res = block_reduce_argmax(best, bad, s_w);
    if (threadIdx.x == 0) a.part[unit] = res;
}

__global__ __launch_bounds__(kThreads) void tree_resolve_kernel(TreeArgs a) {
    extern __shared__ ArgmaxPart s_part[];  // [n][nseg]
    tree_resolve(a, blockIdx.x, s_part);
}

}  // namespace

hipError_t launch_tree_argmax(const TreeArgs& a, int dtype, hipStream_t s, hipEvent_t ev_start,
                              hipEvent_t ev_stop) {
    // 4 vectors per thread per batch (measured faster than 8 for the argmax
    // fold, which keeps more live registers than the softmax fold)
    const dim3 grid(a.B * a.n * a.nseg);
    if (dtype == 0)
        return launch_timed(tree_argmax_kernel<F32, 4>, grid, dim3(kThreads), 0, s, ev_start, ev_stop, a);
    return launch_timed(tree_argmax_kernel<BF16, 4>, grid, dim3(kThreads), 0, s, ev_start, ev_stop, a);
}

hipError_t launch_tree_resolve(const TreeArgs& a, hipStream_t s) {
    const size_t lds = sizeof(ArgmaxPart) * static_cast<size_t>(a.n) * a.nseg;
    hipLaunchKernelGGL(tree_resolve_kernel, dim3(a.B), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace sv
