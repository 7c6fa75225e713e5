// Kernel argument blocks and launch entry points shared by the host API
// (api.hip) and the kernel translation units (chain.hip, tree.hip).
//
// Data moves between workgroups only across kernel boundaries: a kernel writes
// per-workgroup partial results to the workspace and the next kernel on the
// stream reads them.  No kernel waits on, or publishes to, another workgroup
// of the same launch, so no device-scope fence (which on gfx950 writes back and
// invalidates a whole L2) is ever issued per workgroup, and the workspace
// needs no initialisation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kMaxGamma = 255;        // draft positions per chain block
constexpr int kMaxTreeNodes = 1024;   // nodes per tree, root included
constexpr int kMaxVocab = 1 << 29;    // vocabulary size V (element indices, and sums of
                                       // them with a tile or segment, stay far inside int32)
constexpr int kMaxBlockParts = 2048;  // row partials of one block / request (staged in LDS)

// Row statistics of a temperature softmax (see stat_fold in sv_device.hpp):
// m = largest logit, R = integer-valued reference, S = sum 2^(z*c - R).
struct Stat {
    float m;
    float R;
    double S;
};

// Outcome of the ratio tests of one chain block.
struct ChainDecision {
    int32_t k;     // first rejected position, gamma if none, -1 if the block is invalid
    float Rp;      // integer reference R of target row k
    double dL;     // (R_p + log2 S_p) - (R_q + log2 S_q) at row k (ratio test, k < gamma), else 0
    int32_t excl;  // point mass, k < gamma: the rejected draft token (weight 0 in the draw); else -1
    int32_t pad;   // tree verification: accept length (where the drawn token goes); else 0
    double Sp;     // S of target row k (sum of 2^(z c - Rp) over the row)
};

// Normaliser of the final draw of one block, kept for the final_dist pass.
struct FinalState {
    double W;          // sum of the (corrected, unnormalised) draw weights over the row
    double kappa;      // residual draw: first-order correction of the weights for the error
                       // of dL (w + kappa * (P[D > 0] - w)); 0 otherwise
    int32_t fallback;  // 1 if an empty residual fell back to p_k
    int32_t pad;
};

struct ChainArgs {
    const void* target;
    const void* draft;
    const int32_t* tokens;
    const float* uniforms;
    int B, gamma, V;
    int pointmass;     // 1: the draft proposes each token with certainty (no draft logits)
    int rows;          // logit rows per block: 2*gamma+1 (target and draft), or gamma+1
    int draft_rows;    // draft rows per block (the draft array's block stride): gamma, or
                       // gamma+1 for tree rows
    int given;         // 1: dec[b] was written by an earlier kernel (tree verification);
                       // the draw takes uniforms[b][0] and writes only its token, at
                       // out_tokens[b][dec.pad]
    float c_hi, c_lo;  // log2(e)/T as a float pair
    double c_d;        // c_hi + c_lo exactly
    double T;
    int nseg, seg_len;      // statistics: segments per row, elements per segment
    int nchunk;             // final draw: chunk workgroups per row
    int chunk_tiles;        // final draw: tiles (one 16-byte vector per thread) per chunk
                            // workgroup, streamed in groups of 1, 2 or 4
    int nquart;             // final draw: quarters (64 16-byte vectors) per row
    Stat* part;             // [B][rows][nseg]
    float* zx;              // [B][rows]: logit of the draft token in rows i < gamma
                            // (target) and gamma+1+i (draft); other entries unused
    ChainDecision* dec;     // [B]
    double* qsum;           // [B][nquart]: draw-weight sum per quarter
    double* qpos;           // [B][nquart]: residual draw: sum of P over the quarter's tokens
                            // with D > 0 (the weights' derivative in dL, see chain.hip)
    double* cdiff;          // [B][nchunk]: residual draw: sum of P - Q' (signed) per chunk
    FinalState* fin;        // [B]
    int32_t* accept_len;
    int32_t* out_tokens;
    float* final_dist;
};

struct ArgmaxPart {
    float best;     // largest logit seen (-inf if none)
    int32_t idx;    // lowest index holding it (INT32_MAX if none)
    uint32_t bad;   // nonzero if a NaN was seen
    uint32_t pad;
};

struct TreeArgs {
    const void* target;
    const int32_t* parents;
    const int32_t* tokens;
    int B, n, V;
    int nseg, seg_len;
    ArgmaxPart* part;  // [B][n][nseg]
    int32_t* accept_len;
    int32_t* accept_node;
    int32_t* out_tokens;
};

// Outcome scoring: one candidate (logit, token id) of a row segment.
struct OutcomeCand {
    float val;    // logit (-inf for an empty slot)
    int32_t idx;  // token id (INT32_MAX for an empty slot)
};

constexpr int kMaxCache = 16;  // cache entries per request

struct OutcomeArgs {
    const void* logits;      // [R][gamma+1][V]
    const int32_t* tokens;   // [R][gamma]; null: no token is excluded
    int R, gamma, V;
    float c_hi, c_lo;
    double c_d;
    double T;
    int nseg, seg_len;
    int ncache;              // 1..kMaxCache
    int kb;                  // candidates kept per row segment: 4, 8 or 16 (>= ncache)
    Stat* part;              // [R][gamma+1][nseg]
    OutcomeCand* cand;       // [R][gamma+1][nseg][kb]
    float* zx;               // [R][gamma+1]: logit of row k's draft token (k < gamma)
    int32_t* out_k;          // [R][ncache]
    int32_t* out_a;          // [R][ncache]
    double* out_p;           // [R][ncache]
    double* hit;             // [R]
};

// Draft-tree construction: per-potential-node draft logits, the W best
// children of every row, then a best-first search per request.
constexpr int kMaxTreeWidth = 16;     // children per node
constexpr int kMaxTreeSlots = 2048;   // M * W (the search stages every row's children)
constexpr int kMaxTreeSegs = 64;      // segments per row

struct TreeBuildArgs {
    OutcomeArgs st;          // statistics pass over the rows (no draft tokens)
    const int32_t* child_row;  // [M][W] or null (complete W-ary numbering)
    int M, W, max_depth, budget;
    int32_t* parents;        // [R][budget]
    int32_t* tokens;         // [R][budget]
    int32_t* node_row;       // [R][budget]
    double* score;           // [R][budget]
    int32_t* n_nodes;        // [R]
};

// Stochastic tree verification: the chain statistics over n target and n
// draft rows per request, a per-request decision, then the chain draw.
struct TreeStochArgs {
    ChainArgs ch;               // gamma = n-1, rows = 2n, draft_rows = n, given = 1
    const int32_t* parents;     // [B][n]
    const int32_t* node_tokens; // [B][n]
    int n;
    int dtype;                  // 0 f32, 1 bf16
    int32_t* accept_node;       // [B]
};

// Launchers (return the hipError_t of the launch).
// The streaming launchers take an optional pair of events (both null, or
// both valid): when given, the launch itself records them at the kernel's
// start and end (hipExtLaunchKernel), so their interval is the kernel's own
// execution time.
hipError_t launch_chain_stats(const ChainArgs& a, int dtype, hipStream_t s, hipEvent_t ev_start,
                              hipEvent_t ev_stop);
hipError_t launch_chain_chunks(const ChainArgs& a, int dtype, hipStream_t s);
hipError_t launch_chain_select(const ChainArgs& a, int dtype, hipStream_t s);
hipError_t launch_chain_dist(const ChainArgs& a, int dtype, hipStream_t s);
// The final draw of a chain (chunk and select kernels, or one workgroup per
// block for a large batch of point-mass blocks).
hipError_t launch_chain_draw(const ChainArgs& a, int dtype, hipStream_t s);
hipError_t launch_tree_argmax(const TreeArgs& a, int dtype, hipStream_t s, hipEvent_t ev_start,
                              hipEvent_t ev_stop);
hipError_t launch_tree_resolve(const TreeArgs& a, hipStream_t s);
hipError_t launch_outcome_stats(const OutcomeArgs& a, int dtype, hipStream_t s,
                                hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_outcome_select(const OutcomeArgs& a, hipStream_t s);
hipError_t launch_tree_search(const TreeBuildArgs& a, hipStream_t s);
hipError_t launch_tree_stoch_decide(const TreeStochArgs& t, hipStream_t s);
hipError_t launch_cache_lookup(const int32_t* accept_len, const int32_t* out_tokens, int R,
                               int gamma, const int32_t* cache_k, const int32_t* cache_a,
                               int ncache, int32_t* slot, hipStream_t s);

}  // namespace sv
