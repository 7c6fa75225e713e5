// Stochastic tree verification for gfx950.
//
// What is computed ("JetSpec" reading notes, section "Tree verification",
// Eq. 16-17 and Fig. 5): request b's candidate tree has n nodes (node 0 the
// root, parents preceding children); target row j and draft row j are the
// next-token logits after node j's path.  Every node j >= 1 takes one
// Bernoulli test, accepted iff u[b][j] < min(1, p_par(y_j) / q_par(y_j)); a
// node counts as accepted iff its whole path passed; the deepest accepted
// node v* (lowest index among equally deep ones) ends the best branch, and
// the correction token is drawn from p_{v*} with u[b][0].
//
// Kernels:
//  1. chain_stats_kernel over 2n rows per request (n target rows, then n
//     draft rows): the softmax statistics, once per logit.
//  2. tree_stoch_decide_kernel (here), one workgroup per request: merges the
//     row statistics, gathers each node's token logits from its parent's
//     rows, takes the tests in fp64, finds v* by pointer jumping, writes the
//     path and the decision of the draw.
//  3. chain_chunks_kernel and chain_select_kernel with the decision given:
//     the draw from p_{v*} by inverse CDF, as for a chain's bonus token.
#include "sv_device.hpp"

namespace sv {

namespace {

constexpr double kDomain = 268435456.0;  // |m| / T limit (2^28)

__global__ __launch_bounds__(kThreads) void tree_stoch_decide_kernel(TreeStochArgs t) {
    extern __shared__ unsigned char s_dyn[];  // row partials, then the path arrays
    __shared__ double s_L[2 * kMaxTreeNodes];
    __shared__ float s_Rp[kMaxTreeNodes];
    __shared__ int s_par[kMaxTreeNodes];
    __shared__ int s_tok[kMaxTreeNodes];
    __shared__ int s_bad, s_key;
    constexpr int kStage = kMaxBlockParts / kThreads;
    constexpr int kNodes = kMaxTreeNodes / kThreads;
    const ChainArgs& a = t.ch;
    const int b = blockIdx.x, tid = threadIdx.x, n = t.n, rows = 2 * n;
    const int32_t* par = t.parents + static_cast<int64_t>(b) * n;
    const int32_t* tok = t.node_tokens + static_cast<int64_t>(b) * n;
    const float* uu = a.uniforms + static_cast<int64_t>(b) * n;
    int32_t* out = a.out_tokens + static_cast<int64_t>(b) * n;
    // node j = tid + q*kThreads: parent, token and uniform, in registers
    int pv[kNodes], tv[kNodes];
    float uv[kNodes];
    {
        // stage the request's 2n*nseg row partials, and load every node's
        // inputs: all loads issued before any LDS store (partial indices past
        // the end re-read the last one, unstored)
        const int np = rows * a.nseg;
        const uint4* src = reinterpret_cast<const uint4*>(a.part + static_cast<int64_t>(b) * np);
        uint4* dst = reinterpret_cast<uint4*>(s_dyn);
        uint4 v[kStage];
#pragma unroll
        for (int m = 0; m < kStage; ++m)
            v[m] = m * kThreads < np ? src[min(tid + m * kThreads, np - 1)] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int q = 0; q < kNodes; ++q) {
            const int j = tid + q * kThreads;
            pv[q] = j < n ? par[j] : 0;
            tv[q] = j < n ? tok[j] : 0;
            uv[q] = j < n ? uu[j] : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < kStage; ++m)
            if (tid + m * kThreads < np) dst[tid + m * kThreads] = v[m];
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
    const Stat* s_part = reinterpret_cast<const Stat*>(s_dyn);
    for (int r = tid; r < rows; r += kThreads) {
        const Stat* p = s_part + r * a.nseg;
        Stat st = p[0];
        for (int sg = 1; sg < a.nseg; ++sg) st = stat_merge(st, p[sg]);
        const bool ok = isfinite(st.S) && st.S > 0.0 &&
                        fabs(static_cast<double>(st.m) / a.T) <= kDomain;
        if (!ok) atomicOr(&s_bad, 1);
        s_L[r] = static_cast<double>(st.R) + log2(st.S);
        if (r < n) s_Rp[r] = st.R;
    }
#pragma unroll
    for (int q = 0; q < kNodes; ++q) {
        const int j = tid + q * kThreads, pj = pv[q];
        if (j >= n) break;
        if (j == 0) {
            if (pj != -1) atomicOr(&s_bad, 1);
        } else if (pj < 0 || pj >= j || tv[q] < 0 || tv[q] >= a.V) {
            atomicOr(&s_bad, 1);
        }
    }
    __syncthreads();  // (the partials are dead from here: their LDS is reused)
    if (s_bad) {
        for (int j = tid; j < n; j += kThreads) out[j] = -1;
        if (tid == 0) {
            a.accept_len[b] = -1;
            t.accept_node[b] = -1;
            a.dec[b] = ChainDecision{-1, 0.0f, 0.0, -1, 0, 0.0};
        }
        return;
    }
    int* s_anc = reinterpret_cast<int*>(s_dyn);
    int* s_dep = s_anc + kMaxTreeNodes;
    unsigned char* s_ok = reinterpret_cast<unsigned char*>(s_dep + kMaxTreeNodes);
    using S16 = uint16_t;
    // the token logits after each node's parent path, target and draft: all
    // gathers issued before any is used
    float zp[kNodes], zq[kNodes];
#pragma unroll
    for (int q = 0; q < kNodes; ++q) {
        const int j = tid + q * kThreads;
        zp[q] = 0.0f;
        zq[q] = 0.0f;
        if (j >= 1 && j < n) {
            const int64_t off = (static_cast<int64_t>(b) * n + pv[q]) * a.V + tv[q];
            if (t.dtype == 0) {
                zp[q] = static_cast<const float*>(a.target)[off];
                zq[q] = static_cast<const float*>(a.draft)[off];
            } else {
                zp[q] = __uint_as_float(static_cast<uint32_t>(static_cast<const S16*>(a.target)[off]) << 16);
                zq[q] = __uint_as_float(static_cast<uint32_t>(static_cast<const S16*>(a.draft)[off]) << 16);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < kNodes; ++q) {
        const int j = tid + q * kThreads;
        if (j >= n) break;
        if (j == 0) {
            s_anc[0] = 0;
            s_dep[0] = 0;
            s_ok[0] = 1;
            continue;
        }
        const int p = pv[q];
        // alpha = min(1, p/q) in the log2 domain, both rows' normalisers in
        // fp64; p = 0 rejects, q = 0 < p accepts
        double alpha;
        if (zp[q] == -INFINITY) {
            alpha = 0.0;
        } else if (zq[q] == -INFINITY) {
            alpha = 1.0;
        } else {
            const double d = (static_cast<double>(zp[q]) * a.c_d - s_L[p]) -
                             (static_cast<double>(zq[q]) * a.c_d - s_L[n + p]);
            alpha = d >= 0.0 ? 1.0 : exp2(d);
        }
        s_anc[j] = p;
        s_dep[j] = 1;
        s_ok[j] = static_cast<double>(uv[q]) < alpha;
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
        a.accept_len[b] = depth;
        t.accept_node[b] = vstar;
        // the draw: p at v* (the chain kernels' bonus draw), token at `depth`
        a.dec[b] = ChainDecision{vstar, s_Rp[vstar], 0.0, -1, depth, 0.0};
    }
}

}  // namespace

hipError_t launch_tree_stoch_decide(const TreeStochArgs& t, hipStream_t s) {
    // the row partials, and later the path arrays, share the dynamic LDS
    const size_t part = sizeof(Stat) * static_cast<size_t>(2 * t.n) * t.ch.nseg;
    const size_t path = 2 * sizeof(int) * kMaxTreeNodes + kMaxTreeNodes;
    hipLaunchKernelGGL(tree_stoch_decide_kernel, dim3(t.ch.B), dim3(kThreads),
                       part > path ? part : path, s, t);
    return hipGetLastError();
}

}  // namespace sv
