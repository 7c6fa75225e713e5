// Draft-tree construction by best-first search for gfx950.
//
// What is computed ("JetSpec" reading notes, Algorithm 1 with the branch
// score of Eq. 15): the draft head has produced, in one pass, a row of
// logits for each potential node -- row m is the draft distribution q_m of
// the token after potential node m's path, row 0 the root's.  A node whose
// row is m has as candidate children the W most probable tokens of q_m (ties:
// smaller token id; zero-probability tokens are not candidates); the child
// through the j-th of them has row child_row[m][j] (or, with no map, the
// complete W-ary breadth-first numbering m*W + 1 + j when below M).  Starting
// from the root, the queued node of highest score (ties: the one added first)
// is expanded -- all its candidate children are added in order, each with
// score s_parent + ln q_m(token) -- until the tree holds `budget` nodes;
// nodes at depth N or without a row are never expanded.
//
// Three kernels:
//  1. outcome_stats_kernel (outcome.hip), without draft tokens: one pass over
//     every row keeps the softmax statistics and each segment's best logits.
//  2. tree_rows_kernel: one wave per row merges the segment statistics and,
//     by a tournament over the segments' sorted lists, takes the row's W best
//     tokens with their ln q.
//  3. tree_search_kernel: one wave per request stages every row's children in
//     LDS and runs the search.  The queue never holds a node that cannot be
//     expanded (popping it would change nothing), and it is kept as the union
//     of the expanded nodes' child lists: children of one node have
//     consecutive indices and non-increasing scores, so each list is sorted
//     and a pop is one wave-wide maximum over the lists' heads (each lane owns
//     every 64th list), after which only the popped list advances.
#include "sv_device.hpp"

namespace sv {

namespace {

constexpr double kDomain = 268435456.0;  // |m| / T limit (2^28)
constexpr double kLn2 = 0.69314718055994530942;

__global__ __launch_bounds__(kThreads) void tree_rows_kernel(TreeBuildArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);  // r*M + m
    if (row >= static_cast<int64_t>(a.st.R) * a.M) return;  // the whole wave leaves together
    const int nseg = a.st.nseg, kb = a.st.kb;
    Stat t = stat_empty();
    if (lane < nseg) t = a.st.part[row * nseg + lane];
    t = wave_reduce_stat(t);
    const bool ok = isfinite(t.S) && t.S > 0.0 && fabs(static_cast<double>(t.m) / a.st.T) <= kDomain;
    const double L = static_cast<double>(t.R) + log2(t.S);
    // lane s walks segment s's candidate list (sorted by value, then token)
    const OutcomeCand* list = a.st.cand + (row * nseg + lane) * kb;
    int pos = 0;
    auto head = [&]() -> uint64_t {
        if (lane >= nseg || pos >= kb) return 0;
        const OutcomeCand c = list[pos];
        if (c.idx == INT32_MAX || c.val == -INFINITY) return 0;  // empty or probability 0
        return make_key(c.val, static_cast<uint32_t>(c.idx));
    };
    uint64_t h = head();
    int32_t* tok = a.rt_tok + row * a.W;
    float* lq = a.rt_lq + row * a.W;
    int j = 0;
    for (; j < a.W; ++j) {
        const uint64_t w = wave_max_u64(h);
        if (w == 0) break;  // fewer than W tokens of positive probability
        if (lane == 0) {
            tok[j] = static_cast<int32_t>(key_index(w));
            lq[j] = static_cast<float>((static_cast<double>(key_value(w)) * a.st.c_d - L) * kLn2);
        }
        if (h == w) {
            ++pos;
            h = head();
        }
    }
    if (lane == 0) {
        for (; j < a.W; ++j) {
            tok[j] = -1;
            lq[j] = -INFINITY;
        }
        a.rt_ok[row] = ok ? 1 : 0;
    }
}

__global__ __launch_bounds__(64) void tree_search_kernel(TreeBuildArgs a) {
    extern __shared__ unsigned char s_dyn[];
    const int r = blockIdx.x, lane = threadIdx.x;
    const int M = a.M, W = a.W, B = a.budget, N = a.max_depth;
    const int slots = M * W;
    double* n_score = reinterpret_cast<double*>(s_dyn);  // [B] node scores
    float* c_lq = reinterpret_cast<float*>(n_score + B);  // [slots] children per row
    int* c_tok = reinterpret_cast<int*>(c_lq + slots);    // [slots]
    int* c_row = c_tok + slots;                            // [slots]
    int* n_row = c_row + slots;                            // [B]
    int* n_depth = n_row + B;                              // [B]
    int* l_head = n_depth + B;                             // [B] list heads
    int* l_end = l_head + B;                               // [B] list ends
    const int64_t rb = static_cast<int64_t>(r) * M;
    const int64_t ob = static_cast<int64_t>(r) * B;
    int32_t* o_par = a.parents + ob;
    int32_t* o_tok = a.tokens + ob;
    int32_t* o_row = a.node_row + ob;
    double* o_sc = a.score + ob;

    // stage every row's children and the child map; check the rows
    int bad = 0;
    for (int i = lane; i < slots; i += 64) {
        c_tok[i] = a.rt_tok[rb * W + i];
        c_lq[i] = a.rt_lq[rb * W + i];
        int cr;
        if (a.child_row) {
            cr = a.child_row[i];
            bad |= (cr < -1 || cr >= M);
        } else {
            const int m = i / W;
            const int64_t c = static_cast<int64_t>(m) * W + 1 + (i - m * W);
            cr = c < M ? static_cast<int>(c) : -1;
        }
        c_row[i] = cr;
    }
    for (int m = lane; m < M; m += 64) bad |= (a.rt_ok[rb + m] == 0);
    if (__ballot(bad) != 0) {
        for (int i = lane; i < B; i += 64) {
            o_par[i] = -1;
            o_tok[i] = -1;
            o_row[i] = -1;
            o_sc[i] = -INFINITY;
        }
        if (lane == 0) a.n_nodes[r] = -1;
        return;
    }
    if (lane == 0) {
        n_score[0] = 0.0;
        n_row[0] = 0;
        n_depth[0] = 0;
        o_par[0] = -1;
        o_tok[0] = -1;
        o_row[0] = 0;
        o_sc[0] = 0.0;
    }
    __syncthreads();

    int n = 1, nlists = 0;
    // this lane's best list head: score, node, list
    double bs = -INFINITY;
    int bn = INT32_MAX, bl = -1;
    auto consider = [&](int l) {
        const int h = l_head[l];
        if (h < l_end[l] && cand_ahead(n_score[h], h, bs, bn)) {
            bs = n_score[h];
            bn = h;
            bl = l;
        }
    };
    // adds the candidate children of node v (all lanes, v uniform)
    auto expand = [&](int v) {
        const int rv = n_row[v], dv = n_depth[v];
        const double sv = n_score[v];
        int cnt = 0;
        for (int j = 0; j < W; ++j) cnt += c_tok[rv * W + j] >= 0;  // children form a prefix
        cnt = min(cnt, B - n);
        if (lane < cnt) {
            const int u = n + lane, i = rv * W + lane;
            const double s = sv + static_cast<double>(c_lq[i]);
            n_score[u] = s;
            n_row[u] = c_row[i];
            n_depth[u] = dv + 1;
            o_par[u] = v;
            o_tok[u] = c_tok[i];
            o_row[u] = c_row[i];
            o_sc[u] = s;
        }
        __syncthreads();
        if (dv + 1 < N && cnt > 0) {
            const int l = nlists++;
            if (lane == (l & 63)) {
                int h = n;
                while (h < n + cnt && n_row[h] < 0) ++h;  // only nodes with a row are queued
                l_head[l] = h;
                l_end[l] = n + cnt;
                consider(l);
            }
        }
        n += cnt;
    };
    expand(0);  // the root is the only queued node at first
    while (n < B) {
        double ws = bs;
        int wn = bn;
        wave_best(ws, wn);
        if (wn == INT32_MAX) break;  // nothing left to expand
        if (bn == wn) {              // the owner advances the popped list
            int h = wn + 1;
            const int e = l_end[bl];
            while (h < e && n_row[h] < 0) ++h;
            l_head[bl] = h;
            bs = -INFINITY;
            bn = INT32_MAX;
            bl = -1;
            for (int l = lane; l < nlists; l += 64) consider(l);
        }
        expand(wn);
    }
    for (int i = n + lane; i < B; i += 64) {
        o_par[i] = -1;
        o_tok[i] = -1;
        o_row[i] = -1;
        o_sc[i] = -INFINITY;
    }
    if (lane == 0) a.n_nodes[r] = n;
}

}  // namespace

hipError_t launch_tree_rows(const TreeBuildArgs& a, hipStream_t s) {
    const int64_t rows = static_cast<int64_t>(a.st.R) * a.M;
    hipLaunchKernelGGL(tree_rows_kernel, dim3(static_cast<unsigned>((rows + kWaves - 1) / kWaves)),
                       dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

size_t tree_search_lds_bytes(int M, int W, int budget) {
    const size_t slots = static_cast<size_t>(M) * W;
    return static_cast<size_t>(budget) * (sizeof(double) + 4 * sizeof(int)) +
           slots * (sizeof(float) + 2 * sizeof(int));
}

hipError_t launch_tree_search(const TreeBuildArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(tree_search_kernel, dim3(a.st.R), dim3(64),
                       tree_search_lds_bytes(a.M, a.W, a.budget), s, a);
    return hipGetLastError();
}

}  // namespace sv
