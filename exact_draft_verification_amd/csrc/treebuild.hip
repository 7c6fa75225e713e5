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
// Two kernels:
//  1. outcome_stats_kernel (outcome.hip), without draft tokens: one pass over
//     every row keeps the softmax statistics and each segment's best logits.
//  2. tree_search_kernel: one workgroup per request merges each row's
//     segments into the row's W best tokens with their ln q, in LDS (one row
//     per thread), and then its first wave runs the search.  The queue never holds a node that cannot be
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

// Order-preserving image of a score (finite or -inf) as an unsigned key:
// a larger score gives a larger key, and -0 counts as +0.
__device__ inline uint64_t score_key(double s) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(s + 0.0));
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

template <int CTRL, int ROWS>
__device__ inline void dpp_min_step(int& x) {
    x = min(x, __builtin_amdgcn_update_dpp(x, x, CTRL, ROWS, 0xf, false));
}

// Wave-wide best of (score desc, node asc) over the lanes' (s, i), carrying
// the node's packed row and depth along; every lane gets the winner.  The
// maximum is taken over the scores' integer keys; equal best scores on
// several lanes (rare) are settled by a minimum over their nodes.
__device__ inline void wave_best_rd(double& s, int& i, int& rd) {
    const uint64_t k = score_key(s);
    const uint64_t km = wave_max_u64(k);
    const bool at_max = k == km;
    const uint64_t tied = __ballot(at_max);
    int src = __builtin_ctzll(tied);
    if (__popcll(tied) > 1) {
        int c = at_max ? i : INT32_MAX;
        dpp_min_step<0xb1, 0xf>(c);
        dpp_min_step<0x4e, 0xf>(c);
        dpp_min_step<0x141, 0xf>(c);
        dpp_min_step<0x140, 0xf>(c);
        dpp_min_step<0x142, 0xa>(c);
        dpp_min_step<0x143, 0xc>(c);
        const int cm = __builtin_amdgcn_readlane(c, 63);
        src = __builtin_ctzll(__ballot(at_max & (i == cm)));
    }
    s = readlane_f64(s, src);
    i = __builtin_amdgcn_readlane(i, src);
    rd = __builtin_amdgcn_readlane(rd, src);
}

// A node's row (>= 0) and depth in one int (rows < 2^20, depths < 2^10).
__device__ inline int pack_rd(int row, int depth) { return (row << 10) | depth; }

__global__ __launch_bounds__(kThreads) void tree_search_kernel(TreeBuildArgs a) {
    extern __shared__ unsigned char s_dyn[];
    const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int M = a.M, W = a.W, B = a.budget, N = a.max_depth;
    const int slots = M * W;
    const int nseg = a.st.nseg, kb = a.st.kb;
    double* n_score = reinterpret_cast<double*>(s_dyn);  // [B] node scores
    double* l_hs = n_score + B;                          // [B] list head scores
    double* c_lq = l_hs + B;                             // [slots] children's ln q per row
    int* c_tok = reinterpret_cast<int*>(c_lq + slots);   // [slots]
    int* c_row = c_tok + slots;                          // [slots]
    int* n_row = c_row + slots;                          // [B]
    int* l_head = n_row + B;                             // [B] list heads
    int* l_end = l_head + B;                             // [B] list ends
    int* l_hrd = l_end + B;                              // [B] head's packed row and depth
    const int64_t rb = static_cast<int64_t>(r) * M;
    const int64_t ob = static_cast<int64_t>(r) * B;
    int32_t* o_par = a.parents + ob;
    int32_t* o_tok = a.tokens + ob;
    int32_t* o_row = a.node_row + ob;
    double* o_sc = a.score + ob;

    // every row's W children, one row per thread of the workgroup: its
    // segment statistics merged, and the W best of its segments' sorted
    // candidate lists
    int bad = 0;
    for (int m = tid; m < M; m += kThreads) {
        const Stat* pp = a.st.part + (rb + m) * nseg;
        const OutcomeCand* cc = a.st.cand + (rb + m) * nseg * kb;
        if (nseg == 1) {
            // one sorted list: its first W entries, loaded together
            OutcomeCand c[kMaxTreeWidth];
#pragma unroll
            for (int q = 0; q < kMaxTreeWidth; ++q)
                if (q < W) c[q] = cc[q];
            const Stat t = pp[0];
            bad |= !(isfinite(t.S) && t.S > 0.0 &&
                     fabs(static_cast<double>(t.m) / a.st.T) <= kDomain);
            const double L = static_cast<double>(t.R) + log2(t.S);
#pragma unroll
            for (int q = 0; q < kMaxTreeWidth; ++q) {
                if (q < W) {
                    const bool ok = c[q].idx != INT32_MAX && c[q].val != -INFINITY;  // a prefix
                    c_tok[m * W + q] = ok ? c[q].idx : -1;
                    c_lq[m * W + q] =
                        ok ? (static_cast<double>(c[q].val) * a.st.c_d - L) * kLn2 : -INFINITY;
                }
            }
            continue;
        }
        Stat t = pp[0];
        for (int sg = 1; sg < nseg; ++sg) t = stat_merge(t, pp[sg]);
        bad |= !(isfinite(t.S) && t.S > 0.0 &&
                 fabs(static_cast<double>(t.m) / a.st.T) <= kDomain);
        const double L = static_cast<double>(t.R) + log2(t.S);
        // pass j takes the best key below the one taken by pass j-1 (keys are
        // distinct); a segment contributes at most W
        const int depth_k = min(kb, W);
        uint64_t prev = ~0ull;
        int j = 0;
        for (; j < W; ++j) {
            uint64_t best = 0;
            for (int sg = 0; sg < nseg; ++sg) {
                for (int p = 0; p < depth_k; ++p) {
                    const OutcomeCand c = cc[sg * kb + p];
                    if (c.idx == INT32_MAX || c.val == -INFINITY) break;  // the rest is empty
                    const uint64_t k = make_key(c.val, static_cast<uint32_t>(c.idx));
                    if (k < prev) {  // the segment's best not yet taken
                        best = k > best ? k : best;
                        break;
                    }
                }
            }
            if (best == 0) break;  // fewer than W tokens of positive probability
            c_tok[m * W + j] = static_cast<int>(key_index(best));
            c_lq[m * W + j] = (static_cast<double>(key_value(best)) * a.st.c_d - L) * kLn2;
            prev = best;
        }
        for (; j < W; ++j) {
            c_tok[m * W + j] = -1;
            c_lq[m * W + j] = -INFINITY;
        }
    }
    // the child map, in chunks whose loads are all issued before use
    constexpr int kChunk = 8;
    for (int base = 0; base < slots; base += kThreads * kChunk) {
        int cr[kChunk];
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
            const int i = base + c * kThreads + tid;
            if (i < slots) {
                if (a.child_row) {
                    cr[c] = a.child_row[i];
                } else {
                    const int m = i / W;
                    const int64_t ch = static_cast<int64_t>(m) * W + 1 + (i - m * W);
                    cr[c] = ch < M ? static_cast<int>(ch) : -1;
                }
            }
        }
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
            const int i = base + c * kThreads + tid;
            if (i < slots) {
                c_row[i] = cr[c];
                bad |= (cr[c] < -1 || cr[c] >= M);
            }
        }
    }
    if (__syncthreads_or(bad)) {
        for (int i = tid; i < B; i += kThreads) {
            o_par[i] = -1;
            o_tok[i] = -1;
            o_row[i] = -1;
            o_sc[i] = -INFINITY;
        }
        if (tid == 0) a.n_nodes[r] = -1;
        return;
    }
    if (tid >= 64) return;  // the search runs on the first wave alone
    if (lane == 0) {
        n_score[0] = 0.0;
        n_row[0] = 0;
        o_par[0] = -1;
        o_tok[0] = -1;
        o_row[0] = 0;
        o_sc[0] = 0.0;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    int n = 1, nlists = 0;
    // this lane's best list head: score, node, packed row/depth, list
    double bs = -INFINITY;
    int bn = INT32_MAX, brd = 0, bl = -1;
    auto consider = [&](int l) {
        const int h = l_head[l];
        const double hs = l_hs[l];
        if (h < l_end[l] && cand_ahead(hs, h, bs, bn)) {
            bs = hs;
            bn = h;
            brd = l_hrd[l];
            bl = l;
        }
    };
    // the candidate children of row rv: lane j < W gets child j's token,
    // ln q and row (static tables, so the read may precede the list update)
    struct Children {
        int tk, cr;
        double q;
    };
    auto children = [&](int rv) {
        Children c{-1, -1, 0.0};
        if (lane < W) {
            c.tk = c_tok[rv * W + lane];
            c.q = c_lq[rv * W + lane];
            c.cr = c_row[rv * W + lane];
        }
        return c;
    };
    // adds the candidate children c of node v (all lanes; arguments uniform)
    auto expand = [&](int v, int dv, double sv, const Children& c) {
        const int cnt = min(__popcll(__ballot(c.tk >= 0)), B - n);  // the children form a prefix
        const double s = sv + c.q;
        if (lane < cnt) {
            const int u = n + lane;
            n_score[u] = s;
            n_row[u] = c.cr;
            o_par[u] = v;
            o_tok[u] = c.tk;
            o_row[u] = c.cr;
            o_sc[u] = s;
        }
        // only children with a row are ever expanded
        const uint64_t expandable = __ballot(lane < cnt && c.cr >= 0);
        if (dv + 1 < N && expandable != 0) {
            const int f = __builtin_ctzll(expandable);
            const int l = nlists++;
            const double hs = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(s), f),
                                               __builtin_amdgcn_readlane(__double2loint(s), f));
            const int hrd = pack_rd(__builtin_amdgcn_readlane(c.cr, f), dv + 1);
            if (lane == (l & 63)) {
                l_head[l] = n + f;
                l_end[l] = n + cnt;
                l_hs[l] = hs;
                l_hrd[l] = hrd;
                if (cand_ahead(hs, n + f, bs, bn)) {
                    bs = hs;
                    bn = n + f;
                    brd = hrd;
                    bl = l;
                }
            }
        }
        n += cnt;
        // the workgroup is this one wave: order its LDS writes before later
        // reads without waiting for the global stores
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    };
    expand(0, 0, 0.0, children(0));  // the root is the only queued node at first
    while (n < B) {
        double ws = bs;
        int wn = bn, wrd = brd;
        wave_best_rd(ws, wn, wrd);
        if (wn == INT32_MAX) break;  // nothing left to expand
        const Children c = children(wrd >> 10);
        if (bn == wn) {  // the owner advances the popped list
            const int e = l_end[bl];
            int h = wn + 1;
            while (h < e && n_row[h] < 0) ++h;
            l_head[bl] = h;
            bs = -INFINITY;
            bn = INT32_MAX;
            if (h < e) {
                const double hs = n_score[h];
                const int hrd = pack_rd(n_row[h], wrd & 1023);
                l_hs[bl] = hs;
                l_hrd[bl] = hrd;
                if (nlists <= 64) {
                    // the lane owns this one list: its head is the lane's best
                    bs = hs;
                    bn = h;
                    brd = hrd;
                }
            }
            if (nlists > 64) {
                bl = -1;
                for (int l = lane; l < nlists; l += 64) consider(l);
            } else if (h >= e) {
                bl = -1;
            }
        }
        expand(wn, wrd & 1023, ws, c);
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

size_t tree_search_lds_bytes(int M, int W, int budget) {
    const size_t slots = static_cast<size_t>(M) * W;
    return static_cast<size_t>(budget) * (2 * sizeof(double) + 4 * sizeof(int)) +
           slots * (sizeof(double) + 2 * sizeof(int));
}

hipError_t launch_tree_search(const TreeBuildArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(tree_search_kernel, dim3(a.st.R), dim3(kThreads),
                       tree_search_lds_bytes(a.M, a.W, a.budget), s, a);
    return hipGetLastError();
}

}  // namespace sv
