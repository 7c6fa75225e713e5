// Host side of libspecverify.so: argument validation, workspace layout and
// launch sequencing on the caller's stream.  See include/spec_verify.h for the
// contract of every entry point.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "spec_verify.h"
#include "spec_verify_timing.h"
#include "sv_kernels.hpp"

namespace sv {
namespace {

constexpr int kThreadsHost = 256;
constexpr int64_t kChainUnits = 4096;   // chain statistics workgroups to aim for
constexpr int64_t kTreeUnits = 8192;    // tree argmax workgroups to aim for
constexpr int64_t kOutcomeUnits = 1024; // outcome-scoring workgroups to aim for
constexpr int64_t kChunkUnits = 1024;   // final-draw chunk workgroups to aim for
constexpr int kResidualChunkTiles = 4;   // tiles per chunk at most where the draw can be residual

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int elem_bytes(int32_t dtype) { return dtype == SV_DTYPE_F32 ? 4 : 2; }
bool dtype_ok(int32_t dtype) { return dtype == SV_DTYPE_F32 || dtype == SV_DTYPE_BF16; }

// Segments of a row for the streaming kernels: enough workgroups to fill the
// chip several times over, each with at least min_vec_per_thread 16-byte
// vectors per thread; segment lengths are whole 16-byte vectors.
void plan_segments(int64_t rows_total, int V, int epv, int64_t target, int min_vec_per_thread,
                   int max_seg, int* nseg, int* seg_len) {
    const int64_t nvec = ceil_div(V, epv);
    int64_t cap = nvec / (static_cast<int64_t>(kThreadsHost) * min_vec_per_thread);
    if (cap < 1) cap = 1;
    if (cap > max_seg) cap = max_seg;
    int64_t s = ceil_div(target, rows_total);
    if (s < 1) s = 1;
    if (s > cap) s = cap;
    int64_t len = ceil_div(ceil_div(V, s), epv) * epv;
    *seg_len = static_cast<int>(len);
    *nseg = static_cast<int>(ceil_div(V, len));
}

struct ChainPlan {
    int rows, nseg, seg_len, nchunk, chunk_tiles, nquart;
    size_t off_part, off_zx, off_dec, off_qsum, off_qpos, off_cdiff, off_fin, bytes;
};

// Carves `n` objects of `size` bytes out of the workspace at *off (256-byte
// aligned regions); returns the region's offset.
size_t carve(size_t* off, size_t size, size_t n) {
    const size_t at = *off;
    *off = align_up(at + size * n, 256);
    return at;
}

// Plan of a chain call: rows per block are 2*gamma+1 (target and draft
// logits) for the ratio test, gamma+1 (target only) for a point-mass draft.
// Statistics segments, final-draw chunks and workspace for B blocks of `rows`
// logit rows each (chains; stochastic trees, whose blocks are requests).
int32_t block_plan(int32_t B, int64_t rows, int32_t V, int32_t dtype, int max_tiles, ChainPlan* p) {
    const int E = elem_bytes(dtype), epv = 16 / E;
    const int64_t rows_total = static_cast<int64_t>(B) * rows;
    // every element index and byte offset must fit comfortably in int64, and
    // grid sizes in int32
    if (static_cast<double>(rows_total) * V * E > 9.0e18) return SV_ERR_SHAPE;
    p->rows = static_cast<int>(rows);
    // a block's rows*nseg partials are staged in LDS by the kernel that takes
    // its decision; fewer, longer segments keep them few
    plan_segments(rows_total, V, epv, kChainUnits, 4,
                  static_cast<int>(kMaxBlockParts / rows), &p->nseg, &p->seg_len);
    if (rows_total * p->nseg > INT32_MAX) return SV_ERR_SHAPE;
    // final draw: tiles of one 16-byte vector per thread, sums kept per
    // quarter tile (64 vectors); a chunk workgroup takes the block's decision
    // once and then streams a run of tiles, so a large batch gets a few long
    // chunks per block (about kChunkUnits workgroups in all) and a small one
    // many single-tile chunks.  A residual draw reads two rows and takes more
    // arithmetic per token, which overlaps its loads better with more waves:
    // its runs are capped at max_tiles tiles.
    const int64_t tile = static_cast<int64_t>(kThreadsHost) * epv;
    const int64_t ntile = ceil_div(V, tile);
    int64_t nchunk = ceil_div(kChunkUnits, B);
    if (max_tiles > 0 && nchunk < ceil_div(ntile, max_tiles)) nchunk = ceil_div(ntile, max_tiles);
    if (nchunk > ntile) nchunk = ntile;
    p->chunk_tiles = static_cast<int>(ceil_div(ntile, nchunk));
    p->nchunk = static_cast<int>(ceil_div(ntile, p->chunk_tiles));
    p->nquart = static_cast<int>(ceil_div(V, 64 * static_cast<int64_t>(epv)));
    if (static_cast<int64_t>(B) * p->nchunk > INT32_MAX) return SV_ERR_SHAPE;
    const size_t nb = static_cast<size_t>(B), nr = static_cast<size_t>(rows_total);
    size_t off = 0;
    p->off_part = carve(&off, sizeof(Stat), nr * p->nseg);
    p->off_zx = carve(&off, sizeof(float), nr);
    p->off_dec = carve(&off, sizeof(ChainDecision), nb);
    p->off_qsum = carve(&off, sizeof(double), nb * p->nquart);
    p->off_qpos = carve(&off, sizeof(double), nb * p->nquart);
    p->off_cdiff = carve(&off, sizeof(double), nb * p->nchunk);
    p->off_fin = carve(&off, sizeof(FinalState), nb);
    p->bytes = off;
    return SV_OK;
}

int32_t chain_plan(int32_t B, int32_t gamma, int32_t V, int32_t dtype, bool pointmass,
                   ChainPlan* p) {
    if (!dtype_ok(dtype)) return SV_ERR_DTYPE;
    if (B < 1 || gamma < 1 || V < 1 || V > kMaxVocab || gamma > kMaxGamma) return SV_ERR_SHAPE;
    return block_plan(B, (pointmass ? 1 : 2) * static_cast<int64_t>(gamma) + 1, V, dtype,
                      pointmass ? 0 : kResidualChunkTiles, p);
}

// Stochastic tree verification: n target rows and n draft rows per request.
int32_t tree_stoch_plan(int32_t B, int32_t n, int32_t V, int32_t dtype, ChainPlan* p) {
    if (!dtype_ok(dtype)) return SV_ERR_DTYPE;
    if (B < 1 || n < 1 || V < 1 || V > kMaxVocab || n > kMaxTreeNodes) return SV_ERR_SHAPE;
    return block_plan(B, 2 * static_cast<int64_t>(n), V, dtype, 0, p);
}

struct TreePlan {
    int nseg, seg_len;
    size_t off_part, bytes;
};

int32_t tree_plan(int32_t B, int32_t n, int32_t V, int32_t dtype, TreePlan* p) {
    if (!dtype_ok(dtype)) return SV_ERR_DTYPE;
    if (B < 1 || n < 1 || V < 1 || V > kMaxVocab || n > kMaxTreeNodes) return SV_ERR_SHAPE;
    const int E = elem_bytes(dtype), epv = 16 / E;
    const int64_t rows_total = static_cast<int64_t>(B) * n;
    if (static_cast<double>(rows_total) * V * E > 9.0e18) return SV_ERR_SHAPE;
    // a request's n*nseg partials are staged in LDS by the resolve kernel
    plan_segments(rows_total, V, epv, kTreeUnits, 4, kMaxBlockParts / n, &p->nseg,
                  &p->seg_len);
    if (rows_total * p->nseg > INT32_MAX) return SV_ERR_SHAPE;
    size_t off = 0;
    p->off_part = carve(&off, sizeof(ArgmaxPart), static_cast<size_t>(rows_total) * p->nseg);
    p->bytes = off;
    return SV_OK;
}

struct OutcomePlan {
    int nseg, seg_len, kb;
    size_t off_part, off_cand, off_zx, bytes;
};

int32_t outcome_plan(int32_t R, int32_t gamma, int32_t V, int32_t dtype, int32_t ncache,
                     OutcomePlan* p) {
    if (!dtype_ok(dtype)) return SV_ERR_DTYPE;
    if (R < 1 || gamma < 1 || V < 1 || V > kMaxVocab || gamma > kMaxGamma || ncache < 1 ||
        ncache > kMaxCache)
        return SV_ERR_SHAPE;
    const int E = elem_bytes(dtype), epv = 16 / E;
    const int64_t rows = static_cast<int64_t>(gamma) + 1;
    const int64_t rows_total = static_cast<int64_t>(R) * rows;
    if (static_cast<double>(rows_total) * V * E > 9.0e18) return SV_ERR_SHAPE;
    p->kb = ncache <= 4 ? 4 : (ncache <= 8 ? 8 : 16);
    // a request's rows*nseg*kb candidates are staged in LDS by the select
    // kernel (12 bytes each, at most 4096 of them: 48 KiB)
    const int64_t max_seg = 4096 / (rows * p->kb);
    // long segments (few workgroups, at least 16 vectors per thread): the
    // workgroup threshold that keeps top-list insertions rare only becomes
    // selective after a thread has seen many logits
    plan_segments(rows_total, V, epv, kOutcomeUnits, 16,
                  static_cast<int>(max_seg < 1 ? 1 : max_seg), &p->nseg, &p->seg_len);
    if (rows_total * p->nseg > INT32_MAX) return SV_ERR_SHAPE;
    const size_t nr = static_cast<size_t>(rows_total);
    size_t off = 0;
    p->off_part = carve(&off, sizeof(Stat), nr * p->nseg);
    p->off_cand = carve(&off, sizeof(OutcomeCand), nr * p->nseg * p->kb);
    p->off_zx = carve(&off, sizeof(float), nr);
    p->bytes = off;
    return SV_OK;
}

struct TreeBuildPlan {
    int nseg, seg_len, kb;
    size_t off_part, off_cand, bytes;
};

int32_t tree_build_plan(int32_t R, int32_t M, int32_t V, int32_t dtype, int32_t W,
                        int32_t max_depth, int32_t budget, TreeBuildPlan* p) {
    if (!dtype_ok(dtype)) return SV_ERR_DTYPE;
    if (R < 1 || M < 1 || V < 1 || V > kMaxVocab || W < 1 || W > kMaxTreeWidth ||
        max_depth < 1 || budget < 1 || budget > kMaxTreeNodes ||
        static_cast<int64_t>(M) * W > kMaxTreeSlots)
        return SV_ERR_SHAPE;
    const int E = elem_bytes(dtype), epv = 16 / E;
    const int64_t rows_total = static_cast<int64_t>(R) * M;
    if (static_cast<double>(rows_total) * V * E > 9.0e18) return SV_ERR_SHAPE;
    p->kb = W <= 4 ? 4 : (W <= 8 ? 8 : 16);
    // a row's segments are merged by one lane
    plan_segments(rows_total, V, epv, kOutcomeUnits, 16, kMaxTreeSegs, &p->nseg, &p->seg_len);
    if (rows_total * p->nseg > INT32_MAX) return SV_ERR_SHAPE;
    const size_t nr = static_cast<size_t>(rows_total);
    size_t off = 0;
    p->off_part = carve(&off, sizeof(Stat), nr * p->nseg);
    p->off_cand = carve(&off, sizeof(OutcomeCand), nr * p->nseg * p->kb);
    p->bytes = off;
    return SV_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hipEvent_t event_at(void* const* ev, int i) {
    return ev ? static_cast<hipEvent_t>(ev[i]) : nullptr;
}

int32_t record(void* const* ev, int i, hipStream_t s) {
    if (!ev) return SV_OK;
    return hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace
}  // namespace sv

using namespace sv;

extern "C" const char* spec_verify_status_string(int32_t status) {
    switch (status) {
        case SV_OK: return "ok";
        case SV_ERR_NULL: return "a required pointer is null";
        case SV_ERR_SHAPE: return "a size is out of range";
        case SV_ERR_TEMPERATURE: return "temperature must be finite and in [1e-6, 1e6]";
        case SV_ERR_DTYPE: return "unknown logit dtype";
        case SV_ERR_WORKSPACE: return "workspace too small or not 16-byte aligned";
        case SV_ERR_HIP: return "HIP runtime error";
        case SV_ERR_ALIGN: return "a pointer is not aligned to its element size";
        case SV_ERR_SCRATCH:
            return "the sizes need more scratch than the allocation-free entry point holds";
        default: return "unknown status";
    }
}

extern "C" size_t spec_verify_chain_workspace_bytes(int32_t B, int32_t gamma, int32_t V,
                                                    int32_t dtype) {
    ChainPlan p;
    return chain_plan(B, gamma, V, dtype, false, &p) == SV_OK ? p.bytes : 0;
}

extern "C" size_t spec_verify_chain_pointmass_workspace_bytes(int32_t B, int32_t gamma, int32_t V,
                                                              int32_t dtype) {
    ChainPlan p;
    return chain_plan(B, gamma, V, dtype, true, &p) == SV_OK ? p.bytes : 0;
}

extern "C" size_t spec_verify_tree_greedy_workspace_bytes(int32_t B, int32_t n, int32_t V,
                                                          int32_t dtype) {
    TreePlan p;
    return tree_plan(B, n, V, dtype, &p) == SV_OK ? p.bytes : 0;
}

namespace sv {
namespace {

// The host checks of a chain call other than the workspace's: sizes, null
// pointers, temperature and alignment; fills the plan.
int32_t chain_check(const void* target_logits, const void* draft_logits, bool pointmass,
                    int32_t dtype, const int32_t* draft_tokens, const float* uniforms, int32_t B,
                    int32_t gamma, int32_t V, double temperature, const int32_t* accept_len,
                    const int32_t* out_tokens, const float* final_dist, ChainPlan* p) {
    int32_t st = chain_plan(B, gamma, V, dtype, pointmass, p);
    if (st != SV_OK) return st;
    if (!target_logits || (!pointmass && !draft_logits) || !draft_tokens || !uniforms ||
        !accept_len || !out_tokens)
        return SV_ERR_NULL;
    if (!std::isfinite(temperature) || temperature < 1e-6 || temperature > 1e6)
        return SV_ERR_TEMPERATURE;
    const size_t E = static_cast<size_t>(elem_bytes(dtype));
    if (!aligned(target_logits, E) || (!pointmass && !aligned(draft_logits, E)) ||
        !aligned(draft_tokens, 4) ||
        !aligned(uniforms, 4) || !aligned(accept_len, 4) || !aligned(out_tokens, 4) ||
        (final_dist && !aligned(final_dist, 4)))
        return SV_ERR_ALIGN;
    return SV_OK;
}

// Both chain entry points: validation, workspace layout and the launches.
// draft_logits is null exactly when `pointmass`.
int32_t chain_call(const void* target_logits, const void* draft_logits, bool pointmass,
                   int32_t dtype, const int32_t* draft_tokens, const float* uniforms, int32_t B,
                   int32_t gamma, int32_t V, double temperature, int32_t* accept_len,
                   int32_t* out_tokens, float* final_dist, void* workspace,
                   size_t workspace_bytes, void* stream, void* const* phase_events) {
    ChainPlan p;
    const int32_t st = chain_check(target_logits, draft_logits, pointmass, dtype, draft_tokens,
                                   uniforms, B, gamma, V, temperature, accept_len, out_tokens,
                                   final_dist, &p);
    if (st != SV_OK) return st;
    if (!workspace) return SV_ERR_NULL;
    if (!aligned(workspace, 16) || workspace_bytes < p.bytes) return SV_ERR_WORKSPACE;

    ChainArgs a;
    a.target = target_logits;
    a.draft = draft_logits;
    a.tokens = draft_tokens;
    a.uniforms = uniforms;
    a.B = B;
    a.gamma = gamma;
    a.V = V;
    a.pointmass = pointmass ? 1 : 0;
    a.rows = p.rows;
    a.draft_rows = gamma;
    a.given = 0;
    // log2(e)/T as c_hi + c_lo with c_hi the largest float strictly below c,
    // so c_lo > 0: a -inf logit then scales to -inf in both parts and never
    // meets +inf (which would give NaN) when the two products are added.
    const double c = 1.4426950408889634074 / temperature;
    float c_hi = static_cast<float>(c);
    if (static_cast<double>(c_hi) >= c) c_hi = std::nextafter(c_hi, 0.0f);
    a.c_hi = c_hi;
    a.c_lo = static_cast<float>(c - static_cast<double>(c_hi));
    a.c_d = static_cast<double>(a.c_hi) + static_cast<double>(a.c_lo);
    a.T = temperature;
    a.nseg = p.nseg;
    a.seg_len = p.seg_len;
    a.nchunk = p.nchunk;
    a.chunk_tiles = p.chunk_tiles;
    a.nquart = p.nquart;
    char* ws = static_cast<char*>(workspace);
    a.part = reinterpret_cast<Stat*>(ws + p.off_part);
    a.zx = reinterpret_cast<float*>(ws + p.off_zx);
    a.dec = reinterpret_cast<ChainDecision*>(ws + p.off_dec);
    a.qsum = reinterpret_cast<double*>(ws + p.off_qsum);
    a.qpos = reinterpret_cast<double*>(ws + p.off_qpos);
    a.cdiff = reinterpret_cast<double*>(ws + p.off_cdiff);
    a.fin = reinterpret_cast<FinalState*>(ws + p.off_fin);
    a.accept_len = accept_len;
    a.out_tokens = out_tokens;
    a.final_dist = final_dist;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_chain_stats(a, dtype, s, event_at(phase_events, 0), event_at(phase_events, 1)) !=
        hipSuccess)
        return SV_ERR_HIP;
    if (launch_chain_draw(a, dtype, s) != hipSuccess) return SV_ERR_HIP;
    if (record(phase_events, 2, s) != SV_OK) return SV_ERR_HIP;
    if (final_dist && launch_chain_dist(a, dtype, s) != hipSuccess) return SV_ERR_HIP;
    return SV_OK;
}

}  // namespace
}  // namespace sv

extern "C" int32_t spec_verify_chain(const void* target_logits, const void* draft_logits,
                                     int32_t dtype, const int32_t* draft_tokens,
                                     const float* uniforms, int32_t B, int32_t gamma, int32_t V,
                                     double temperature, int32_t* accept_len,
                                     int32_t* out_tokens, float* final_dist, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    return chain_call(target_logits, draft_logits, false, dtype, draft_tokens, uniforms, B, gamma,
                      V, temperature, accept_len, out_tokens, final_dist, workspace,
                      workspace_bytes, stream, nullptr);
}

extern "C" int32_t spec_verify_chain_timed(const void* target_logits, const void* draft_logits,
                                           int32_t dtype, const int32_t* draft_tokens,
                                           const float* uniforms, int32_t B, int32_t gamma,
                                           int32_t V, double temperature, int32_t* accept_len,
                                           int32_t* out_tokens, float* final_dist,
                                           void* workspace, size_t workspace_bytes, void* stream,
                                           void* const* phase_events) {
    return chain_call(target_logits, draft_logits, false, dtype, draft_tokens, uniforms, B, gamma,
                      V, temperature, accept_len, out_tokens, final_dist, workspace,
                      workspace_bytes, stream, phase_events);
}

extern "C" int32_t spec_verify_chain_pointmass(const void* target_logits, int32_t dtype,
                                               const int32_t* draft_tokens,
                                               const float* uniforms, int32_t B, int32_t gamma,
                                               int32_t V, double temperature,
                                               int32_t* accept_len, int32_t* out_tokens,
                                               float* final_dist, void* workspace,
                                               size_t workspace_bytes, void* stream) {
    return chain_call(target_logits, nullptr, true, dtype, draft_tokens, uniforms, B, gamma, V,
                      temperature, accept_len, out_tokens, final_dist, workspace,
                      workspace_bytes, stream, nullptr);
}

extern "C" int32_t spec_verify_chain_pointmass_timed(
    const void* target_logits, int32_t dtype, const int32_t* draft_tokens, const float* uniforms,
    int32_t B, int32_t gamma, int32_t V, double temperature, int32_t* accept_len,
    int32_t* out_tokens, float* final_dist, void* workspace, size_t workspace_bytes, void* stream,
    void* const* phase_events) {
    return chain_call(target_logits, nullptr, true, dtype, draft_tokens, uniforms, B, gamma, V,
                      temperature, accept_len, out_tokens, final_dist, workspace,
                      workspace_bytes, stream, phase_events);
}

// ---------------------------------------------------------------------------
// Allocation-free chain verification.  Its scratch is a file-scope device
// array, one copy per GPU, held until the process ends.  On the host the name
// `scratch` is only a stand-in for the device symbol, never an address: each
// GPU's copy is found once with hipGetSymbolAddress (with that GPU current)
// and its address kept in scratch_dev, which is what the kernels are given.

namespace sv {
namespace {

__device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];  // per device: the address of its copy, or null

// The address of `scratch` on the device that runs `stream` (the current
// device for the null stream), looked up on the first call there.
int32_t scratch_for(hipStream_t stream, void** out) {
    int dev = -1;
    if (stream) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return SV_ERR_HIP;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return SV_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return SV_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return SV_ERR_HIP;
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return SV_ERR_HIP;
        if (e != hipSuccess || !ptr) return SV_ERR_HIP;
        scratch_dev[dev] = ptr;
    }
    *out = scratch_dev[dev];
    return SV_OK;
}

}  // namespace
}  // namespace sv

extern "C" int32_t spec_verify_chain_noalloc(const void* target_logits, const void* draft_logits,
                                             int32_t dtype, const int32_t* draft_tokens,
                                             const float* uniforms, int32_t B, int32_t gamma,
                                             int32_t V, double temperature, int32_t* accept_len,
                                             int32_t* out_tokens, float* final_dist,
                                             void* stream) {
    ChainPlan p;
    int32_t st = chain_check(target_logits, draft_logits, false, dtype, draft_tokens, uniforms, B,
                             gamma, V, temperature, accept_len, out_tokens, final_dist, &p);
    if (st != SV_OK) return st;
    if (p.bytes > SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_SCRATCH;
    void* ws = nullptr;
    st = scratch_for(static_cast<hipStream_t>(stream), &ws);
    if (st != SV_OK) return st;
    // every byte of the workspace is written before it is read within one
    // call, so the previous call's contents need no clearing
    return chain_call(target_logits, draft_logits, false, dtype, draft_tokens, uniforms, B, gamma,
                      V, temperature, accept_len, out_tokens, final_dist, ws,
                      SV_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

extern "C" size_t spec_outcome_topk_workspace_bytes(int32_t R, int32_t gamma, int32_t V,
                                                    int32_t dtype, int32_t ncache) {
    OutcomePlan p;
    return outcome_plan(R, gamma, V, dtype, ncache, &p) == SV_OK ? p.bytes : 0;
}

static int32_t outcome_topk_call(const void* logits, int32_t dtype, const int32_t* draft_tokens,
                                 int32_t R, int32_t gamma, int32_t V, double temperature,
                                 int32_t ncache, int32_t* out_k, int32_t* out_a, double* out_p,
                                 double* hit, void* workspace, size_t workspace_bytes,
                                 void* stream, void* const* phase_events) {
    OutcomePlan p;
    int32_t st = outcome_plan(R, gamma, V, dtype, ncache, &p);
    if (st != SV_OK) return st;
    if (!logits || !draft_tokens || !out_k || !out_a || !out_p || !hit || !workspace)
        return SV_ERR_NULL;
    if (!std::isfinite(temperature) || temperature < 1e-6 || temperature > 1e6)
        return SV_ERR_TEMPERATURE;
    const size_t E = static_cast<size_t>(elem_bytes(dtype));
    if (!aligned(logits, E) || !aligned(draft_tokens, 4) || !aligned(out_k, 4) ||
        !aligned(out_a, 4) || !aligned(out_p, 8) || !aligned(hit, 8))
        return SV_ERR_ALIGN;
    if (!aligned(workspace, 16) || workspace_bytes < p.bytes) return SV_ERR_WORKSPACE;
    OutcomeArgs a;
    a.logits = logits;
    a.tokens = draft_tokens;
    a.R = R;
    a.gamma = gamma;
    a.V = V;
    const double c = 1.4426950408889634074 / temperature;
    float c_hi = static_cast<float>(c);
    if (static_cast<double>(c_hi) >= c) c_hi = std::nextafter(c_hi, 0.0f);
    a.c_hi = c_hi;
    a.c_lo = static_cast<float>(c - static_cast<double>(c_hi));
    a.c_d = static_cast<double>(a.c_hi) + static_cast<double>(a.c_lo);
    a.T = temperature;
    a.nseg = p.nseg;
    a.seg_len = p.seg_len;
    a.ncache = ncache;
    a.kb = p.kb;
    char* ws = static_cast<char*>(workspace);
    a.part = reinterpret_cast<Stat*>(ws + p.off_part);
    a.cand = reinterpret_cast<OutcomeCand*>(ws + p.off_cand);
    a.zx = reinterpret_cast<float*>(ws + p.off_zx);
    a.out_k = out_k;
    a.out_a = out_a;
    a.out_p = out_p;
    a.hit = hit;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_outcome_stats(a, dtype, s, event_at(phase_events, 0), event_at(phase_events, 1)) !=
        hipSuccess)
        return SV_ERR_HIP;
    if (launch_outcome_select(a, s) != hipSuccess) return SV_ERR_HIP;
    return SV_OK;
}

extern "C" int32_t spec_outcome_topk(const void* logits, int32_t dtype,
                                     const int32_t* draft_tokens, int32_t R, int32_t gamma,
                                     int32_t V, double temperature, int32_t ncache,
                                     int32_t* out_k, int32_t* out_a, double* out_p, double* hit,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    return outcome_topk_call(logits, dtype, draft_tokens, R, gamma, V, temperature, ncache, out_k,
                             out_a, out_p, hit, workspace, workspace_bytes, stream, nullptr);
}

extern "C" int32_t spec_outcome_topk_timed(const void* logits, int32_t dtype,
                                           const int32_t* draft_tokens, int32_t R, int32_t gamma,
                                           int32_t V, double temperature, int32_t ncache,
                                           int32_t* out_k, int32_t* out_a, double* out_p,
                                           double* hit, void* workspace, size_t workspace_bytes,
                                           void* stream, void* const* phase_events) {
    return outcome_topk_call(logits, dtype, draft_tokens, R, gamma, V, temperature, ncache, out_k,
                             out_a, out_p, hit, workspace, workspace_bytes, stream, phase_events);
}

extern "C" size_t spec_tree_build_workspace_bytes(int32_t R, int32_t M, int32_t V, int32_t dtype,
                                                  int32_t W, int32_t max_depth, int32_t budget) {
    TreeBuildPlan p;
    return tree_build_plan(R, M, V, dtype, W, max_depth, budget, &p) == SV_OK ? p.bytes : 0;
}

static int32_t tree_build_call(const void* draft_logits, int32_t dtype, const int32_t* child_row,
                               int32_t R, int32_t M, int32_t V, double temperature, int32_t W,
                               int32_t max_depth, int32_t budget, int32_t* parents,
                               int32_t* tokens, int32_t* node_row, double* score,
                               int32_t* n_nodes, void* workspace, size_t workspace_bytes,
                               void* stream, void* const* phase_events) {
    TreeBuildPlan p;
    int32_t st = tree_build_plan(R, M, V, dtype, W, max_depth, budget, &p);
    if (st != SV_OK) return st;
    if (!draft_logits || !parents || !tokens || !node_row || !score || !n_nodes || !workspace)
        return SV_ERR_NULL;
    if (!std::isfinite(temperature) || temperature < 1e-6 || temperature > 1e6)
        return SV_ERR_TEMPERATURE;
    const size_t E = static_cast<size_t>(elem_bytes(dtype));
    if (!aligned(draft_logits, E) || (child_row && !aligned(child_row, 4)) ||
        !aligned(parents, 4) || !aligned(tokens, 4) || !aligned(node_row, 4) ||
        !aligned(score, 8) || !aligned(n_nodes, 4))
        return SV_ERR_ALIGN;
    if (!aligned(workspace, 16) || workspace_bytes < p.bytes) return SV_ERR_WORKSPACE;
    TreeBuildArgs a;
    OutcomeArgs& o = a.st;
    o = OutcomeArgs{};
    o.logits = draft_logits;
    o.tokens = nullptr;  // no token is excluded from a row's candidates
    o.R = R;
    o.gamma = M - 1;  // M rows per request
    o.V = V;
    const double c = 1.4426950408889634074 / temperature;
    float c_hi = static_cast<float>(c);
    if (static_cast<double>(c_hi) >= c) c_hi = std::nextafter(c_hi, 0.0f);
    o.c_hi = c_hi;
    o.c_lo = static_cast<float>(c - static_cast<double>(c_hi));
    o.c_d = static_cast<double>(o.c_hi) + static_cast<double>(o.c_lo);
    o.T = temperature;
    o.nseg = p.nseg;
    o.seg_len = p.seg_len;
    o.ncache = W;
    o.kb = p.kb;
    char* ws = static_cast<char*>(workspace);
    o.part = reinterpret_cast<Stat*>(ws + p.off_part);
    o.cand = reinterpret_cast<OutcomeCand*>(ws + p.off_cand);
    o.zx = nullptr;  // written only for rows with a draft token
    a.child_row = child_row;
    a.M = M;
    a.W = W;
    a.max_depth = max_depth;
    a.budget = budget;
    a.parents = parents;
    a.tokens = tokens;
    a.node_row = node_row;
    a.score = score;
    a.n_nodes = n_nodes;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_outcome_stats(o, dtype, s, event_at(phase_events, 0), event_at(phase_events, 1)) !=
        hipSuccess)
        return SV_ERR_HIP;
    if (launch_tree_search(a, s) != hipSuccess) return SV_ERR_HIP;
    return SV_OK;
}

extern "C" int32_t spec_tree_build(const void* draft_logits, int32_t dtype,
                                   const int32_t* child_row, int32_t R, int32_t M, int32_t V,
                                   double temperature, int32_t W, int32_t max_depth,
                                   int32_t budget, int32_t* parents, int32_t* tokens,
                                   int32_t* node_row, double* score, int32_t* n_nodes,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    return tree_build_call(draft_logits, dtype, child_row, R, M, V, temperature, W, max_depth,
                           budget, parents, tokens, node_row, score, n_nodes, workspace,
                           workspace_bytes, stream, nullptr);
}

extern "C" int32_t spec_tree_build_timed(const void* draft_logits, int32_t dtype,
                                         const int32_t* child_row, int32_t R, int32_t M, int32_t V,
                                         double temperature, int32_t W, int32_t max_depth,
                                         int32_t budget, int32_t* parents, int32_t* tokens,
                                         int32_t* node_row, double* score, int32_t* n_nodes,
                                         void* workspace, size_t workspace_bytes, void* stream,
                                         void* const* phase_events) {
    return tree_build_call(draft_logits, dtype, child_row, R, M, V, temperature, W, max_depth,
                           budget, parents, tokens, node_row, score, n_nodes, workspace,
                           workspace_bytes, stream, phase_events);
}

extern "C" size_t spec_verify_tree_stochastic_workspace_bytes(int32_t B, int32_t n, int32_t V,
                                                              int32_t dtype) {
    ChainPlan p;
    return tree_stoch_plan(B, n, V, dtype, &p) == SV_OK ? p.bytes : 0;
}

static int32_t tree_stochastic_call(
    const void* target_logits, const void* draft_logits, int32_t dtype, const int32_t* parents,
    const int32_t* tokens, const float* uniforms, int32_t B, int32_t n, int32_t V,
    double temperature, int32_t* accept_len, int32_t* accept_node, int32_t* out_tokens,
    float* final_dist, void* workspace, size_t workspace_bytes, void* stream,
    void* const* phase_events) {
    ChainPlan p;
    const int32_t st = tree_stoch_plan(B, n, V, dtype, &p);
    if (st != SV_OK) return st;
    if (!target_logits || !draft_logits || !parents || !tokens || !uniforms || !accept_len ||
        !accept_node || !out_tokens || !workspace)
        return SV_ERR_NULL;
    if (!std::isfinite(temperature) || temperature < 1e-6 || temperature > 1e6)
        return SV_ERR_TEMPERATURE;
    const size_t E = static_cast<size_t>(elem_bytes(dtype));
    if (!aligned(target_logits, E) || !aligned(draft_logits, E) || !aligned(parents, 4) ||
        !aligned(tokens, 4) || !aligned(uniforms, 4) || !aligned(accept_len, 4) ||
        !aligned(accept_node, 4) || !aligned(out_tokens, 4) ||
        (final_dist && !aligned(final_dist, 4)))
        return SV_ERR_ALIGN;
    if (!aligned(workspace, 16) || workspace_bytes < p.bytes) return SV_ERR_WORKSPACE;
    TreeStochArgs t;
    ChainArgs& a = t.ch;
    a = ChainArgs{};
    a.target = target_logits;
    a.draft = draft_logits;
    a.tokens = nullptr;  // the statistics pass gathers nothing; the decision does
    a.uniforms = uniforms;
    a.B = B;
    a.gamma = n - 1;     // n target rows per request
    a.V = V;
    a.pointmass = 1;     // the draw is from p itself, no residual
    a.rows = p.rows;     // 2n
    a.draft_rows = n;
    a.given = 1;
    const double c = 1.4426950408889634074 / temperature;
    float c_hi = static_cast<float>(c);
    if (static_cast<double>(c_hi) >= c) c_hi = std::nextafter(c_hi, 0.0f);
    a.c_hi = c_hi;
    a.c_lo = static_cast<float>(c - static_cast<double>(c_hi));
    a.c_d = static_cast<double>(a.c_hi) + static_cast<double>(a.c_lo);
    a.T = temperature;
    a.nseg = p.nseg;
    a.seg_len = p.seg_len;
    a.nchunk = p.nchunk;
    a.chunk_tiles = p.chunk_tiles;
    a.nquart = p.nquart;
    char* ws = static_cast<char*>(workspace);
    a.part = reinterpret_cast<Stat*>(ws + p.off_part);
    a.zx = nullptr;
    a.dec = reinterpret_cast<ChainDecision*>(ws + p.off_dec);
    a.qsum = reinterpret_cast<double*>(ws + p.off_qsum);
    a.qpos = reinterpret_cast<double*>(ws + p.off_qpos);
    a.cdiff = reinterpret_cast<double*>(ws + p.off_cdiff);
    a.fin = reinterpret_cast<FinalState*>(ws + p.off_fin);
    a.accept_len = accept_len;
    a.out_tokens = out_tokens;
    a.final_dist = final_dist;
    t.parents = parents;
    t.node_tokens = tokens;
    t.n = n;
    t.dtype = dtype;
    t.accept_node = accept_node;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_chain_stats(a, dtype, s, event_at(phase_events, 0), event_at(phase_events, 1)) !=
        hipSuccess)
        return SV_ERR_HIP;
    if (launch_tree_stoch_decide(t, s) != hipSuccess) return SV_ERR_HIP;
    if (launch_chain_chunks(a, dtype, s) != hipSuccess) return SV_ERR_HIP;
    if (launch_chain_select(a, dtype, s) != hipSuccess) return SV_ERR_HIP;
    if (record(phase_events, 2, s) != SV_OK) return SV_ERR_HIP;
    if (final_dist && launch_chain_dist(a, dtype, s) != hipSuccess) return SV_ERR_HIP;
    return SV_OK;
}

extern "C" int32_t spec_verify_tree_stochastic(
    const void* target_logits, const void* draft_logits, int32_t dtype, const int32_t* parents,
    const int32_t* tokens, const float* uniforms, int32_t B, int32_t n, int32_t V,
    double temperature, int32_t* accept_len, int32_t* accept_node, int32_t* out_tokens,
    float* final_dist, void* workspace, size_t workspace_bytes, void* stream) {
    return tree_stochastic_call(target_logits, draft_logits, dtype, parents, tokens, uniforms, B,
                                n, V, temperature, accept_len, accept_node, out_tokens,
                                final_dist, workspace, workspace_bytes, stream, nullptr);
}

extern "C" int32_t spec_verify_tree_stochastic_timed(
    const void* target_logits, const void* draft_logits, int32_t dtype, const int32_t* parents,
    const int32_t* tokens, const float* uniforms, int32_t B, int32_t n, int32_t V,
    double temperature, int32_t* accept_len, int32_t* accept_node, int32_t* out_tokens,
    float* final_dist, void* workspace, size_t workspace_bytes, void* stream,
    void* const* phase_events) {
    return tree_stochastic_call(target_logits, draft_logits, dtype, parents, tokens, uniforms, B,
                                n, V, temperature, accept_len, accept_node, out_tokens,
                                final_dist, workspace, workspace_bytes, stream, phase_events);
}

extern "C" int32_t spec_cache_lookup(const int32_t* accept_len, const int32_t* out_tokens,
                                     int32_t R, int32_t gamma, const int32_t* cache_k,
                                     const int32_t* cache_a, int32_t ncache, int32_t* slot,
                                     void* stream) {
    if (R < 1 || gamma < 1 || gamma > kMaxGamma || ncache < 1 || ncache > kMaxCache)
        return SV_ERR_SHAPE;
    if (!accept_len || !out_tokens || !cache_k || !cache_a || !slot) return SV_ERR_NULL;
    if (!aligned(accept_len, 4) || !aligned(out_tokens, 4) || !aligned(cache_k, 4) ||
        !aligned(cache_a, 4) || !aligned(slot, 4))
        return SV_ERR_ALIGN;
    return launch_cache_lookup(accept_len, out_tokens, R, gamma, cache_k, cache_a, ncache, slot,
                               static_cast<hipStream_t>(stream)) == hipSuccess
               ? SV_OK
               : SV_ERR_HIP;
}

static int32_t tree_greedy_call(const void* target_logits, int32_t dtype, const int32_t* parents,
                                const int32_t* tokens, int32_t B, int32_t n, int32_t V,
                                int32_t* accept_len, int32_t* accept_node, int32_t* out_tokens,
                                void* workspace, size_t workspace_bytes, void* stream,
                                void* const* phase_events) {
    TreePlan p;
    int32_t st = tree_plan(B, n, V, dtype, &p);
    if (st != SV_OK) return st;
    if (!target_logits || !parents || !tokens || !accept_len || !accept_node || !out_tokens ||
        !workspace)
        return SV_ERR_NULL;
    const size_t E = static_cast<size_t>(elem_bytes(dtype));
    if (!aligned(target_logits, E) || !aligned(parents, 4) || !aligned(tokens, 4) ||
        !aligned(accept_len, 4) || !aligned(accept_node, 4) || !aligned(out_tokens, 4))
        return SV_ERR_ALIGN;
    if (!aligned(workspace, 16) || workspace_bytes < p.bytes) return SV_ERR_WORKSPACE;
    TreeArgs a;
    a.target = target_logits;
    a.parents = parents;
    a.tokens = tokens;
    a.B = B;
    a.n = n;
    a.V = V;
    a.nseg = p.nseg;
    a.seg_len = p.seg_len;
    char* ws = static_cast<char*>(workspace);
    a.part = reinterpret_cast<ArgmaxPart*>(ws + p.off_part);
    a.accept_len = accept_len;
    a.accept_node = accept_node;
    a.out_tokens = out_tokens;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_tree_argmax(a, dtype, s, event_at(phase_events, 0), event_at(phase_events, 1)) !=
        hipSuccess)
        return SV_ERR_HIP;
    if (launch_tree_resolve(a, s) != hipSuccess) return SV_ERR_HIP;
    return SV_OK;
}

extern "C" int32_t spec_verify_tree_greedy(const void* target_logits, int32_t dtype,
                                           const int32_t* parents, const int32_t* tokens,
                                           int32_t B, int32_t n, int32_t V, int32_t* accept_len,
                                           int32_t* accept_node, int32_t* out_tokens,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream) {
    return tree_greedy_call(target_logits, dtype, parents, tokens, B, n, V, accept_len,
                            accept_node, out_tokens, workspace, workspace_bytes, stream, nullptr);
}

extern "C" int32_t spec_verify_tree_greedy_timed(const void* target_logits, int32_t dtype,
                                                 const int32_t* parents, const int32_t* tokens,
                                                 int32_t B, int32_t n, int32_t V,
                                                 int32_t* accept_len, int32_t* accept_node,
                                                 int32_t* out_tokens, void* workspace,
                                                 size_t workspace_bytes, void* stream,
                                                 void* const* phase_events) {
    return tree_greedy_call(target_logits, dtype, parents, tokens, B, n, V, accept_len,
                            accept_node, out_tokens, workspace, workspace_bytes, stream,
                            phase_events);
}
