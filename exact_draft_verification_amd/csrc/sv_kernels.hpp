// Kernel argument blocks and launch entry points shared by the host API
// (api.hip) and the kernel translation units (chain.hip, tree.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kMaxGamma = 255;       // draft positions per chain block
constexpr int kMaxTreeNodes = 1024;  // nodes per tree, root included
constexpr int kMaxChunks = 256;      // final-draw chunks per row (one per thread)

// Row statistics of a temperature softmax (see stat_fold in sv_device.hpp):
// m = largest logit, R = integer-valued reference, S = sum 2^(z*c - R).
struct Stat {
    float m;
    float R;
    double S;
};

// Outcome of the ratio tests of one chain block, written by the last
// statistics workgroup of that block.
struct ChainDecision {
    int32_t k;   // first rejected position, gamma if none, -1 if the block is invalid
    float Rp;    // integer reference R of target row k
    float Rq;    // integer reference R of draft row k (k < gamma)
    float dL;    // (R_p + log2 S_p) - (R_q + log2 S_q) at row k, rounded to fp32
};

// Normaliser of the final draw of one block, kept for the final_dist pass.
struct FinalState {
    double W;          // sum of the (unnormalised) draw weights over the row
    int32_t fallback;  // 1 if an empty residual fell back to p_k
    int32_t pad;
};

struct ChainArgs {
    const void* target;
    const void* draft;
    const int32_t* tokens;
    const float* uniforms;
    int B, gamma, V;
    float c_hi, c_lo;  // log2(e)/T as a float pair
    double c_d;        // c_hi + c_lo exactly
    double T;
    int nseg, seg_len;      // statistics: segments per row, elements per segment
    int nchunk, chunk_len;  // final draw: chunks per row, elements per chunk
    Stat* part;             // [B][2*gamma+1][nseg]
    ChainDecision* dec;     // [B]
    double* chunk_sum;      // [B][nchunk]
    FinalState* fin;        // [B]
    // Arrival counters, one per block and kernel.  Every call leaves every
    // workspace byte it used at zero: the last reader of each region clears it.
    unsigned* cnt_stats;    // [B]
    unsigned* cnt_final;    // [B]
    unsigned* cnt_dist;     // [B]
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
    unsigned* cnt;     // [B]
    int32_t* accept_len;
    int32_t* accept_node;
    int32_t* out_tokens;
};

// Launchers (return the hipError_t of the launch).
hipError_t launch_chain_stats(const ChainArgs& a, int dtype, hipStream_t s);
hipError_t launch_chain_final(const ChainArgs& a, int dtype, hipStream_t s);
hipError_t launch_chain_dist(const ChainArgs& a, int dtype, hipStream_t s);
hipError_t launch_tree(const TreeArgs& a, int dtype, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace sv
