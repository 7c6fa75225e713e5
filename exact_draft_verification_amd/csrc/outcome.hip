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
//     as the chain statistics do and finds the KB largest logits of the
//     segment (lowest token id first among equal ones), the row's draft token
//     excluded.  Candidates are ordered by a 64-bit key (value, then index).
//     The stream itself only takes the maximum of every 16-byte vector: the
//     KB best elements lie in the KB+1 best vectors by (maximum, vector
//     index) -- a vector outside them is behind KB+1 vector maxima, at most
//     one of which is the excluded token -- so each wave keeps a sorted list
//     of its best vector keys spread over its lanes, and a vector is offered
//     to it only when its maximum passes a threshold shared through LDS (the
//     largest of the waves' (KB+1)-th keys).  At the end the KB+1 best
//     vectors of the workgroup are re-read and their elements, with the
//     unaligned head and tail elements, ranked exactly.
//  2. outcome_select: one workgroup per request merges the row statistics,
//     forms A_k = sum_{i<k} log2 p_i(x_i) by a prefix sum, scores every
//     candidate in fp64 as log2 P = A_k + z*c - L_k and keeps the ncache best.
#include "sv_device.hpp"

namespace sv {

namespace {

constexpr double kDomain = 268435456.0;  // |m| / T limit (2^28)
constexpr float kNegInf = -INFINITY;

// 64-bit cross-lane moves.  dpp64: a DPP pattern (lanes whose source lies
// outside the wave are left undefined).  xor_lanes<J>: the key of lane (lane ^ J);
// within a row it is one or two DPP moves (x ^ 7 is the half-row mirror,
// x ^ 15 the row mirror, x ^ 3 a quad permute), across rows a swizzle (16)
// or a permute through LDS (32).
template <int CTRL>
__device__ inline uint64_t dpp64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_mov_dpp(static_cast<uint32_t>(x), CTRL, 0xf, 0xf, false);
    const uint32_t hi = __builtin_amdgcn_mov_dpp(static_cast<uint32_t>(x >> 32), CTRL, 0xf, 0xf, false);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}
template <int J>
__device__ inline uint64_t xor_lanes(uint64_t x) {
    if constexpr (J == 1) {
        return dpp64<0xb1>(x);  // quad_perm [1,0,3,2]
    } else if constexpr (J == 2) {
        return dpp64<0x4e>(x);  // quad_perm [2,3,0,1]
    } else if constexpr (J == 4) {
        return dpp64<0x1b>(dpp64<0x141>(x));  // half-row mirror, then quad_perm [3,2,1,0]
    } else if constexpr (J == 8) {
        return dpp64<0x141>(dpp64<0x140>(x));  // row mirror, then half-row mirror
    } else if constexpr (J == 16) {
        const uint32_t lo = __builtin_amdgcn_ds_swizzle(static_cast<int>(static_cast<uint32_t>(x)), 0x401f);
        const uint32_t hi = __builtin_amdgcn_ds_swizzle(static_cast<int>(static_cast<uint32_t>(x >> 32)), 0x401f);
        return (static_cast<uint64_t>(hi) << 32) | lo;
    } else {
        return __shfl_xor(x, J, 64);
    }
}

// One compare-exchange step of a bitonic sort (partner lane ^ J, stage K).
template <int J, int K>
__device__ inline uint64_t bitonic_step(uint64_t x, int lane) {
    const uint64_t o = xor_lanes<J>(x);
    const bool keep_max = ((lane & J) == 0) == ((lane & K) == 0);
    return keep_max ? (o > x ? o : x) : (o < x ? o : x);
}

// Descending bitonic sort of one key per lane over the 64 lanes of a wave.
__device__ inline uint64_t wave_sort_desc(uint64_t x) {
    const int lane = threadIdx.x & 63;
    x = bitonic_step<1, 2>(x, lane);
    x = bitonic_step<2, 4>(x, lane);
    x = bitonic_step<1, 4>(x, lane);
    x = bitonic_step<4, 8>(x, lane);
    x = bitonic_step<2, 8>(x, lane);
    x = bitonic_step<1, 8>(x, lane);
    x = bitonic_step<8, 16>(x, lane);
    x = bitonic_step<4, 16>(x, lane);
    x = bitonic_step<2, 16>(x, lane);
    x = bitonic_step<1, 16>(x, lane);
    x = bitonic_step<16, 32>(x, lane);
    x = bitonic_step<8, 32>(x, lane);
    x = bitonic_step<4, 32>(x, lane);
    x = bitonic_step<2, 32>(x, lane);
    x = bitonic_step<1, 32>(x, lane);
    x = bitonic_step<32, 64>(x, lane);
    x = bitonic_step<16, 64>(x, lane);
    x = bitonic_step<8, 64>(x, lane);
    x = bitonic_step<4, 64>(x, lane);
    x = bitonic_step<2, 64>(x, lane);
    x = bitonic_step<1, 64>(x, lane);
    return x;
}

// Statistics plus the per-wave list of the best vector keys.  Every member
// function that uses ballots or cross-lane moves is called by all 64 lanes.
template <class E, int KB>
struct TopVectorFolder {
    static constexpr int L = KB + 1;  // vectors that hold the KB best elements
    Stat s;
    float c_hi, c_lo;
    uint64_t lst;     // sorted (descending) over the wave's lanes; lanes < L matter
    uint64_t th;      // wave-uniform: a vector whose key is not above it cannot
                      // be among the workgroup's L best
    float th_val;     // the value part of th; -inf while th is 0
    bool seeded;      // the list holds the first batch
    unsigned long long* s_th;  // workgroup threshold in LDS

    __device__ inline void set_th(uint64_t t) {
        th = t;
        th_val = t == 0 ? kNegInf : key_value(t);
    }
    // the wave's L-th best key is a valid threshold for the whole workgroup
    __device__ inline void publish() {
        const uint64_t w = readlane64(lst, L - 1);
        if (w > th) {
            set_th(w);
            if ((threadIdx.x & 63) == 0) atomicMax(s_th, static_cast<unsigned long long>(w));
        }
    }
    __device__ inline void refresh() {
        const uint64_t t =
            uniform64(__hip_atomic_load(s_th, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (t > th) set_th(t);
    }
    // ck > th (so it lands in lanes < L); keeps the lanes sorted
    __device__ inline void insert(uint64_t ck) {
        const int lane = threadIdx.x & 63;
        const int pos = __popcll(__ballot(lst > ck));
        const uint64_t up = dpp64<0x138>(lst);  // wave_shr:1 (lane 0's value is not used)
        lst = lane < pos ? lst : (lane == pos ? ck : up);
        publish();
    }
    // The vectors of a batch after the first: a vector is offered when its
    // maximum is not below the threshold's value (a float test that passes
    // every vector whose key is above th, equal values and NaN included);
    // its key is then formed from the lane's value and index and tested
    // exactly.  Lanes are taken in increasing order and each is tested
    // against th as it stands, as offer() does.
    template <int N, bool FULL>
    __device__ inline void offer_maxima(const float* vm, int v0, int nvec) {
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const int vi = v0 + u * kThreads;
            uint64_t m = __ballot((FULL || vi < nvec) && !(vm[u] < th_val));
            while (m) {
                const int l = __builtin_ctzll(m);
                m &= m - 1;
                const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vm[u]), l));
                const uint32_t i = static_cast<uint32_t>(__builtin_amdgcn_readlane(vi, l));
                const uint64_t ck = make_key(v, i);
                if (ck > th) insert(ck);
            }
        }
    }
    template <int N>
    __device__ inline void offer(const uint64_t* key) {
#pragma unroll
        for (int u = 0; u < N; ++u) {
            uint64_t m = __ballot(key[u] > th);
            while (m) {
                const int l = __builtin_ctzll(m);
                insert(readlane64(key[u], l));
                m &= ~(1ull << l);
                m &= __ballot(key[u] > th);
            }
        }
    }

    // N vectors per thread; vector u is body vector v0 + u*kThreads, present
    // when FULL or when that index is below nvec.
    template <int N, bool FULL>
    __device__ inline void batch(const uint4* v, int v0, int nvec) {
        constexpr int P = E::kPerVec;
        float x[N * P];
#pragma unroll
        for (int u = 0; u < N; ++u) E::unpack(v[u], x + u * P);
        float vm[N];
#pragma unroll
        for (int u = 0; u < N; ++u) {
            vm[u] = x[u * P];
#pragma unroll
            for (int i = 1; i < P; ++i) vm[u] = fmaxf(vm[u], x[u * P + i]);
        }
        float bm;
        if (FULL) {
            bm = vm[0];
#pragma unroll
            for (int u = 1; u < N; ++u) bm = fmaxf(bm, vm[u]);
            stat_fold_max<N * P>(s, x, bm, c_hi, c_lo);
        } else {
            bm = kNegInf;
#pragma unroll
            for (int u = 0; u < N; ++u) {
                if (v0 + u * kThreads < nvec) {
                    stat_fold_max<P>(s, x + u * P, vm[u], c_hi, c_lo);
                    bm = fmaxf(bm, vm[u]);
                }
            }
        }
        if (seeded) {
            refresh();
            // cheap test first: can any lane's batch reach the threshold?
            if (!__ballot(!(bm < th_val))) return;
            offer_maxima<N, FULL>(vm, v0, nvec);
            return;
        }
        // the first batch: the list starts as the sorted best vectors of
        // each lane's batch; the lanes' other vectors are offered as usual
        uint64_t key[N];
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const int vi = v0 + u * kThreads;
            key[u] = (FULL || vi < nvec) ? make_key(vm[u], static_cast<uint32_t>(vi)) : 0;
        }
        uint64_t best = key[0];
#pragma unroll
        for (int u = 1; u < N; ++u) best = key[u] > best ? key[u] : best;
        lst = wave_sort_desc(best);
#pragma unroll
        for (int u = 0; u < N; ++u) key[u] = key[u] == best ? 0 : key[u];
        seeded = true;
        publish();
        refresh();
        offer<N>(key);
    }
};

// Streams the 16-byte vectors [0, nvec) of `body` through f as
// stream_vectors does, except that the partial batch at the end is also
// folded by every thread (f.batch<U, false> skips the vectors past the end),
// so the wave-wide list operations always run with all 64 lanes.
template <int U, class F>
__device__ inline void stream_all_lanes(const char* body, int nvec, F& f) {
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
            f.template batch<U, true>(cur, t * kBatch + tid, nvec);
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = min(rest0 + u * kThreads + tid, nvec - 1);
            rest[u] = load16_stream(body + static_cast<size_t>(v) * 16);
        }
        f.template batch<U, true>(cur, (nb - 1) * kBatch + tid, nvec);
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = min(u * kThreads + tid, nvec - 1);
            rest[u] = load16_stream(body + static_cast<size_t>(v) * 16);
        }
    }
    if (rest0 < nvec) f.template batch<U, false>(rest, rest0 + tid, nvec);
}

template <class E, int U, int KB>
__global__ __launch_bounds__(kThreads) void outcome_stats_kernel(OutcomeArgs a) {
    constexpr int L = KB + 1;
    constexpr int P = E::kPerVec;
    constexpr int kMaxCand = L * P + 2 * (P - 1);  // vector elements + head + tail
    static_assert(kWaves * L <= kThreads && kMaxCand <= kThreads, "one key per thread");
    __shared__ Stat s_w[kWaves];
    __shared__ unsigned long long s_th;
    __shared__ unsigned long long s_lst[kWaves * L];
    __shared__ unsigned long long s_ck[kMaxCand];
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
    if (tid == 0) s_th = 0;
    if (tid < L * P) s_ck[tid] = 0;
    int excl = -1;
    if (k < a.gamma && a.tokens) excl = a.tokens[static_cast<int64_t>(r) * a.gamma + k];
    // the draft token's logit, if this segment holds it
    float zx = 0.0f;
    const bool have_zx = tid == 0 && excl >= e0 && excl < e1;
    if (have_zx) zx = E::one(row + excl);
    __syncthreads();

    TopVectorFolder<E, KB> f;
    f.s = stat_empty();
    f.c_hi = a.c_hi;
    f.c_lo = a.c_lo;
    f.lst = 0;
    f.set_th(0);
    f.seeded = false;
    f.s_th = &s_th;
    RangeSplit<E> sp{e0, e0, e0, 0, e0, e0};
    if (e0 < e1) sp = split_range<E>(row, e0, e1);
    // candidate slots: [0, L*P) the elements of the workgroup's L best
    // vectors, in rank order, then the head and the tail elements
    const int nh = sp.head_end - sp.head_begin;
    const int nc = L * P + nh + (sp.tail_end - sp.tail_begin);
    for (int e = sp.head_begin + tid; e < sp.head_end; e += kThreads) {
        const float x = E::one(row + e);
        stat_fold<1>(f.s, &x, a.c_hi, a.c_lo);
        s_ck[L * P + (e - sp.head_begin)] = e != excl ? make_key(x, static_cast<uint32_t>(e)) : 0;
    }
    stream_all_lanes<U>(reinterpret_cast<const char*>(row + sp.body_begin), sp.nvec, f);
    for (int e = sp.tail_begin + tid; e < sp.tail_end; e += kThreads) {
        const float x = E::one(row + e);
        stat_fold<1>(f.s, &x, a.c_hi, a.c_lo);
        s_ck[L * P + nh + (e - sp.tail_begin)] = e != excl ? make_key(x, static_cast<uint32_t>(e)) : 0;
    }
    // re-read the wave's L best vectors while the statistics are reduced
    const bool listed = lane < L && f.lst != 0;
    const int vbeg = sp.body_begin + static_cast<int>(key_index(f.lst)) * P;
    uint4 raw = make_uint4(0u, 0u, 0u, 0u);
    if (listed) raw = load16(row + vbeg);
    if (lane < L) s_lst[wave * L + lane] = f.lst;
    const Stat st = block_reduce_stat(f.s, s_w);  // synchronises the workgroup

    // a listed vector among the workgroup's L best (by rank over the waves'
    // lists; nonzero keys are distinct) scatters its element keys
    if (listed) {
        int rank = 0;
        for (int j = 0; j < kWaves * L; ++j) rank += s_lst[j] > f.lst;
        if (rank < L) {
            float x[P];
            E::unpack(raw, x);
#pragma unroll
            for (int i = 0; i < P; ++i)
                s_ck[rank * P + i] = vbeg + i != excl ? make_key(x[i], static_cast<uint32_t>(vbeg + i)) : 0;
        }
    }
    __syncthreads();
    // exact ranks: nonzero keys are distinct, so a key's rank is the number
    // of keys above it; empty keys (0) follow them in position order
    OutcomeCand* out = a.cand + static_cast<int64_t>(unit) * KB;
    if (tid < nc) {
        const uint64_t ck = s_ck[tid];
        int rank = 0;
#pragma unroll 4
        for (int j = 0; j < nc; ++j) rank += s_ck[j] > ck;
        if (ck == 0)
            for (int j = 0; j < tid; ++j) rank += s_ck[j] == 0;
        if (rank < KB)
            out[rank] = ck != 0 ? OutcomeCand{key_value(ck), static_cast<int32_t>(key_index(ck))}
                                : OutcomeCand{kNegInf, INT32_MAX};
    }
    if (tid == 0) {
        a.part[unit] = st;
        if (have_zx) a.zx[rr] = zx;
    }
}

// Per-request merge: row statistics, prefix of accepted-token log2
// probabilities, candidate scores and the ncache best outcomes.
//
// Candidate i of a request sits at ((k * nseg + segment) * kb + position);
// each segment's list is sorted by (logit desc, token asc) and the segments
// of a row cover increasing token ranges, so among equal scores the
// required order (smaller k, then smaller token) is the order of i.  The
// best outcomes are therefore found by a tournament over the list heads on
// one wave: each lane owns some lists, one wave-wide maximum of
// (score desc, i asc) per kept outcome, after which only the winning list
// advances.
__global__ __launch_bounds__(kThreads) void outcome_select_kernel(OutcomeArgs a) {
    extern __shared__ unsigned char s_dyn[];
    __shared__ double s_L[kMaxGamma + 1];
    __shared__ double s_A[kMaxGamma + 1];
    __shared__ double s_waves[kWaves];
    __shared__ int s_bad;
    __shared__ int s_firstneg;
    constexpr int kPre = 2;  // candidates per thread loaded up front
    const int r = blockIdx.x;
    const int g = a.gamma, rows = g + 1, tid = threadIdx.x, lane = tid & 63;
    const int kb = a.kb;
    const int nlists = rows * a.nseg;  // one sorted list per (row, segment)
    const int ncand = nlists * kb;     // candidates of this request
    const int per_row = a.nseg * kb;   // candidates per row
    double* c_score = reinterpret_cast<double*>(s_dyn);  // [ncand]
    int* c_tok = reinterpret_cast<int*>(c_score + ncand);  // [ncand]
    int* l_pos = c_tok + ncand;                            // [nlists] next entry
    const OutcomeCand* cand = a.cand + static_cast<int64_t>(r) * ncand;
    // every global read of the request is issued before the first wait
    OutcomeCand pre[kPre];
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
        const int i = tid + j * kThreads;
        pre[j] = i < ncand ? cand[i] : OutcomeCand{kNegInf, INT32_MAX};
    }
    int x_tok = 0;
    float zx = 0.0f;
    if (tid < g) {
        x_tok = a.tokens[static_cast<int64_t>(r) * g + tid];
        zx = a.zx[static_cast<int64_t>(r) * rows + tid];
    }
    Stat t = stat_empty();
    if (tid < rows) {
        const Stat* p = a.part + (static_cast<int64_t>(r) * rows + tid) * a.nseg;
        t = p[0];
        for (int s = 1; s < a.nseg; ++s) t = stat_merge(t, p[s]);
    }
    if (tid == 0) {
        s_bad = 0;
        s_firstneg = INT32_MAX;
    }
    for (int l = tid; l < nlists; l += kThreads) l_pos[l] = 0;
    __syncthreads();
    // row statistics (one thread per row; rows <= kThreads)
    if (tid < rows) {
        const bool ok = isfinite(t.S) && t.S > 0.0 && fabs(static_cast<double>(t.m) / a.T) <= kDomain;
        if (!ok) atomicOr(&s_bad, 1);
        s_L[tid] = static_cast<double>(t.R) + log2(t.S);
        if (tid < g && (x_tok < 0 || x_tok >= a.V)) atomicOr(&s_bad, 1);
    }
    __syncthreads();
    // A_k = sum_{i<k} log2 p_i(x_i): exclusive prefix over the rows
    double term = 0.0;
    if (tid < g) term = zx == kNegInf ? -INFINITY : static_cast<double>(zx) * a.c_d - s_L[tid];
    // a -inf term (a masked draft token) makes every later prefix -inf
    const bool neg = term == -INFINITY;
    double total;
    const double excl_sum = block_exclusive_scan(neg ? 0.0 : term, s_waves, &total);
    if (neg) atomicMin(&s_firstneg, tid);
    __syncthreads();
    if (tid < rows) s_A[tid] = tid > s_firstneg ? -INFINITY : excl_sum;
    __syncthreads();
    // scores of every candidate (log2 P), -inf for empty slots
    const bool bad = s_bad != 0;
    auto score = [&](int i, const OutcomeCand& c) {
        const int k = i / per_row;
        double sc = -INFINITY;
        if (c.idx != INT32_MAX && c.val != kNegInf && !bad)
            sc = s_A[k] + (static_cast<double>(c.val) * a.c_d - s_L[k]);
        c_score[i] = sc;
        c_tok[i] = c.idx;
    };
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
        const int i = tid + j * kThreads;
        if (i < ncand) score(i, pre[j]);
    }
    for (int i = tid + kPre * kThreads; i < ncand; i += kThreads) score(i, cand[i]);
    __syncthreads();
    if (tid >= 64) return;  // the tournament runs on the first wave alone

    int32_t* ok_ = a.out_k + static_cast<int64_t>(r) * a.ncache;
    int32_t* oa_ = a.out_a + static_cast<int64_t>(r) * a.ncache;
    double* op_ = a.out_p + static_cast<int64_t>(r) * a.ncache;
    // this lane's best list head
    double bs = -INFINITY;
    int bi = INT32_MAX, bl = -1;
    auto rescan = [&]() {
        bs = -INFINITY;
        bi = INT32_MAX;
        bl = -1;
        for (int l = lane; l < nlists; l += 64) {
            const int p = l_pos[l];
            if (p >= kb) continue;
            const int i = l * kb + p;
            const double sc = c_score[i];
            if (cand_ahead(sc, i, bs, bi)) {
                bs = sc;
                bi = i;
                bl = l;
            }
        }
    };
    rescan();
    double won = -INFINITY;  // lane c: log2 P of the outcome kept in round c
    int c = 0;
    for (; c < a.ncache; ++c) {
        double ws = bs;
        int wi = bi;
        wave_best(ws, wi);
        if (!(ws > -INFINITY)) break;  // no outcome with positive probability left
        if (lane == c) won = ws;
        if (lane == 0) {
            ok_[c] = wi / per_row;
            oa_[c] = c_tok[wi];
        }
        if (bi == wi) {  // the owner of the winning list advances it
            l_pos[bl] += 1;
            rescan();
        }
    }
    // the kept outcomes' probabilities, one per lane off the rounds' critical
    // path, and the hit probability summed in round order
    const double P = lane < c ? exp2(won) : 0.0;
    if (lane < c) op_[lane] = P;
    double hit = 0.0;
    for (int j = 0; j < c; ++j) hit += readlane_f64(P, j);
    if (lane == 0) {
        for (; c < a.ncache; ++c) {
            ok_[c] = -1;
            oa_[c] = -1;
            op_[c] = 0.0;
        }
        a.hit[r] = bad ? -1.0 : hit;
    }
}

// One thread per request: the verified outcome against the request's cache.
__global__ __launch_bounds__(kThreads) void cache_lookup_kernel(const int32_t* accept_len,
                                                                 const int32_t* out_tokens, int R,
                                                                 int gamma, const int32_t* cache_k,
                                                                 const int32_t* cache_a, int ncache,
                                                                 int32_t* slot) {
    const int r = blockIdx.x * kThreads + threadIdx.x;
    if (r >= R) return;
    const int k = accept_len[r];
    int found = -1;
    if (k >= 0 && k <= gamma) {
        const int a = out_tokens[static_cast<int64_t>(r) * (gamma + 1) + k];
        const int32_t* ck = cache_k + static_cast<int64_t>(r) * ncache;
        const int32_t* ca = cache_a + static_cast<int64_t>(r) * ncache;
        for (int c = 0; c < ncache; ++c) {
            if (ck[c] == k && ca[c] == a) {
                found = c;
                break;
            }
        }
    }
    slot[r] = found;
}

}  // namespace

hipError_t launch_cache_lookup(const int32_t* accept_len, const int32_t* out_tokens, int R,
                               int gamma, const int32_t* cache_k, const int32_t* cache_a,
                               int ncache, int32_t* slot, hipStream_t s) {
    hipLaunchKernelGGL(cache_lookup_kernel, dim3((R + kThreads - 1) / kThreads), dim3(kThreads),
                       0, s, accept_len, out_tokens, R, gamma, cache_k, cache_a, ncache, slot);
    return hipGetLastError();
}

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
    const size_t nlists = static_cast<size_t>(a.gamma + 1) * a.nseg;
    const size_t lds = nlists * a.kb * (sizeof(double) + sizeof(int)) + nlists * sizeof(int);
    hipLaunchKernelGGL(outcome_select_kernel, dim3(a.R), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace sv
