// Internal definitions shared by the HIP translation units of libdt.so.
// gfx950 only: wave64, 256-thread workgroups, LDS-resident tree state.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dt.h"

namespace dt {

constexpr int kMaxK = 32;
constexpr int kMaxW = 64;
constexpr int kMaxD = 32;
constexpr int kMaxBudget = 1024;
constexpr int kMaxCandidates = 1024;   // W * k
constexpr int kMaxV = 1 << 26;         // token ids fit the 26-bit field of the tie key
constexpr int kThreads = 256;          // sweep and merge kernels: four wave64s
constexpr int kWaves = kThreads / 64;
constexpr int kTreeThreads = 1024;     // tree kernel: sixteen wave64s per request
constexpr int kTreeWaves = kTreeThreads / 64;
constexpr int kMergeWaves = 8;         // tree-kernel waves that merge the sweep partials
constexpr int kMiscInts = 32;          // tree-kernel counters (0..3) and scan scratch (16..31)
constexpr int kTreeLdsLimit = 64 * 1024;
constexpr int kMergeKeysPerRow = 256;  // C * 4 * k bound: per-wave merge scratch in the tree kernel
constexpr int kSweepVecsPerThread = 4; // 16-byte vectors each thread holds per batch
constexpr int kSweepCap = 128;         // per-wave candidate buffer of the sweep

// ---------------------------------------------------------------------------
// Top-k keys.  A candidate (value x, token id) is packed as
//   key = ord(x) << 32 | ~id
// where ord maps fp32 bit patterns to unsigned integers in the order of the
// values (-0 is first canonicalised to +0).  Larger key = larger value, and
// for equal values the lower id: the (value desc, id asc) order the top-k
// is defined with.  Key 0 never occurs for a real entry and marks "empty".
// ---------------------------------------------------------------------------
__host__ __device__ inline uint32_t ord_bits(uint32_t u) {
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__host__ __device__ inline uint32_t unord_bits(uint32_t o) {
    return (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
}

// ---------------------------------------------------------------------------
// Launch plan of the vocabulary sweep: every row (b, i) is cut into C chunks
// of `chunk` elements (a multiple of 8, so 16-byte vectors never straddle a
// chunk boundary inside a row).  One 256-thread workgroup per chunk.
// ---------------------------------------------------------------------------
struct SweepPlan {
    int C;
    int chunk;
    int64_t rows;
};

// Workspace: per (row, chunk, sweep wave) partial results of the sweep.
//   part_m    float  [rows][C*4]      running max of the wave's elements
//   part_s    double [rows][C*4]      sum exp(x - part_m) over them
//   part_keys uint64 [rows][C*4][k]   their top-k keys, descending; 0 pads
struct WorkspacePlan {
    size_t off_m, off_s, off_keys, total;
};

// Shared-memory plan of the tree kernel (byte offsets into dynamic LDS).
struct TreePlan {
    int n_ctx;          // continuity contexts looked up before the depth loop
    int max_nodes;      // d * W
    int max_cand;       // W * k
    int off_lse;        // double [d]
    int off_ttok;       // int    [d][k]   top-k ids per position
    int off_tx;         // float  [d][k]   their logits
    int off_ctxbase;    // int    [d + 2]  first context of each depth
    int off_vmask;      // uint32 [n_ctx]  admissible children (bit j = T[t-1][j])
    int off_g;          // double [d][k][k] parent-conditioned terms (DARTree)
    int off_nodes;      // node arrays (aliased by the merge scratch)
    int off_n_tok, off_n_par, off_n_dep, off_n_tidx, off_n_cctx, off_n_new, off_n_out;
    int off_n_rk, off_n_s;
    int off_merge;      // uint64 [kMergeWaves][kMergeKeysPerRow] (aliases the node arrays)
    int off_sv_key;     // 16-byte survivor keys [W*k] of the depth loop
    int off_sv_s;       // double [W*k] their cumulative scores
    int off_misc;       // int counters
    int total;
};

struct SweepArgs {
    const void* logits;
    int V;
    int C;
    int chunk;
    int k;
    float* part_m;
    double* part_s;
    unsigned long long* part_keys;
};

struct TreeArgs {
    int B, V, d, k, W, budget, mode, C, R, mask_words;
    const int32_t* ctx;
    const float* part_m;
    const double* part_s;
    const unsigned long long* part_keys;
    int ng_kind;
    float min_logp;
    const float* dense;
    const int32_t* row_ptr;
    const int32_t* col;
    const float* csr_logp;
    const unsigned long long* keys;
    const int32_t* succ;
    const float* hash_logp;
    long long cap;
    int S;
    const float* E;
    const float* F;
    int32_t* n_nodes;
    int32_t* tokens;
    int32_t* parents;
    int32_t* depths;
    float* scores;
    uint32_t* mask;
    TreePlan plan;
};

struct MergeArgs {
    int rows, C, k;
    const float* part_m;
    const double* part_s;
    const unsigned long long* part_keys;
    double* lse;
    int32_t* tok;
    float* val;
};

// host-side planning (api.hip)
SweepPlan plan_sweep(const dt_params* p);
WorkspacePlan plan_workspace(const dt_params* p, const SweepPlan& s);
TreePlan plan_tree(const dt_params* p, int ngram_kind);

// launchers (sweep.hip, tree.hip)
hipError_t launch_sweep(const SweepArgs& a, int64_t rows, int dtype, hipStream_t stream);
hipError_t launch_tree(const TreeArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

}  // namespace dt
