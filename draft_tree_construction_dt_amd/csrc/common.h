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
constexpr int kTreeThreads = 256;      // tree kernel: four wave64s per request
constexpr int kTreeWaves = kTreeThreads / 64;
constexpr int kPrepRows = 3;           // rows a prep workgroup merges: children, parents, grandparents
constexpr int kPrepContexts = 64;      // trigram contexts per prep workgroup (one per lane quad)
constexpr int kMiscInts = 32;          // tree-kernel counters (0..3) and scan scratch (16..31)
constexpr int kTreeLdsLimit = 160 * 1024;
// Calls on several streams: while one call's sweep fills every compute unit
// with two workgroups, the next call's sweep should wait for them to retire
// instead of splitting the memory bandwidth with it, so that the calls stay
// staggered (one call's sweep beside the previous call's prep and tree work)
// rather than sweeping together and then all sitting in their latency-bound
// tails at once.  A sweep workgroup that holds more than a third of a
// compute unit's 160 KB of LDS leaves room for no third one; the prep and
// tree workgroups still fit beside two when their LDS fits in the rest.
// Only a sweep of more than one and at most two workgroups per compute unit
// (256 of them on MI355X) takes turns: a smaller one leaves room for another
// call's beside it either way, and a larger one fills the compute units by
// itself (four of its workgroups fit on one) and would only run in more
// rounds (B=128 on one stream: 52.9 -> 53.7 us per sweep).
constexpr int kSweepLdsTurn = 56 * 1024;
constexpr int64_t kSweepTurnMinGrid = 256 + 1;
constexpr int64_t kSweepTurnMaxGrid = 2 * 256;
constexpr int kPrepLds = 8 * 1024 + 256;      // prep_kernel's static LDS (an upper bound)
constexpr int kMergeKeysPerRow = 256;  // C * 4 * k bound: per-wave merge scratch
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
    int lists;          // partial lists per chunk: kWaves (one per wave) or 1 (merged in the workgroup)
    int64_t rows;
};

// Workspace: per (row, chunk[, sweep wave]) partial results of the sweep, then
// what the prep kernel derives from them for the tree kernel.
//   part_m    float  [rows][C*L]      running max of the list's elements (L = lists per chunk)
//   part_s    double [rows][C*L]      sum exp(x - part_m) over them
//   part_keys uint64 [rows][C*L][k]   their top-k keys, descending; 0 pads
//   lse       double [rows]           log-softmax normaliser of each row
//   ttok      int32  [rows][k]        top-k token ids (T_i), value desc, id asc
//   tx        float  [rows][k]        their logits
//   vmask     uint32 [B][n_ctx_cap]   admissible children of every context
//   g         double [rows][k][k]     parent-conditioned terms (DARTree only)
//   full-vocabulary DARTree mode only:
//   f_tok, f_rk, f_s, f_node  [B][W]     the current frontier: token, Rk, S, node index
//   f_n, n_tree               [B]        frontier size, candidate-tree size
//   nd_tok, nd_par, nd_dep    [B][d*W]   candidate-tree nodes in BFS order
//   nd_s                      [B][d*W]   their cumulative log-scores
//   part                      [B][C2][W] each vocabulary chunk's top-W (VocabEntry)
//   fnorm                     [V]        |F_v|, the screen's rounding bound
//   seed                      [B]        a lower bound for the depth's W-th key
struct WorkspacePlan {
    size_t off_m, off_s, off_keys, off_lse, off_ttok, off_tx, off_vmask, off_g;
    size_t off_f_tok, off_f_rk, off_f_s, off_f_node, off_f_n, off_n_tree;
    size_t off_nd_tok, off_nd_par, off_nd_dep, off_nd_s, off_part, off_fnorm, off_fbf, off_seed, off_cmp_n, off_cmp;
    size_t total;
    int n_ctx_cap;      // contexts per request the vmask area holds (the trigram count)
    int vchunk, C2;     // full-vocabulary mode: columns per chunk and chunk count
};

// Shared-memory plan of the tree kernel (byte offsets into dynamic LDS).
struct TreePlan {
    int n_ctx;          // continuity contexts of the table kind
    int max_nodes;      // d * W
    int max_cand;       // W * k
    int off_lse;        // double [d]
    int off_ttok;       // int    [d][k]   top-k ids per position
    int off_tx;         // float  [d][k]   their logits
    int off_vmask;      // uint32 [n_ctx]  admissible children (bit j = T[t-1][j])
    int off_g;          // double [d][k][k] parent-conditioned terms (DARTree)
    int off_n_tok, off_n_par, off_n_dep, off_n_new, off_n_out, off_n_s;
    int off_n_rec;      // 32-byte frontier records [d*W] read by the next depth
    int off_sv_key;     // 16-byte survivor keys [W*k + 32] of the depth loop
    int off_sv_s;       // 16-byte survivor records [W*k + 32]: score and children's mask
    int off_misc;       // int counters
    int total;
};

struct SweepArgs {
    const void* logits;
    int V;
    int C;
    int chunk;
    int lists;
    int k;
    float* part_m;
    double* part_s;
    unsigned long long* part_keys;
};

// the N-gram table as the kernels see it
struct NGramArgs {
    int kind;
    int V;
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
};

struct PrepArgs {
    int B, d, k, L, mode, R, n_ctx, nsplit;
    const int32_t* ctx;
    const float* part_m;
    const double* part_s;
    const unsigned long long* part_keys;
    NGramArgs ng;
    const float* E;
    const float* F;
    double* lse;
    int32_t* ttok;
    float* tx;
    uint32_t* vmask;
    double* g;
};

struct TreeArgs {
    int B, d, k, W, budget, mode, mask_words, ng_kind, n_ctx;
    const double* lse;
    const int32_t* ttok;
    const float* tx;
    const uint32_t* vmask;
    const double* g;
    int32_t* n_nodes;
    int32_t* tokens;
    int32_t* parents;
    int32_t* depths;
    float* scores;
    uint32_t* mask;
    TreePlan plan;
};

struct NGramUpdateArgs {
    int B, L, S;
    long long cap;
    float new_logp;
    const int32_t* ctx;
    const int32_t* tokens;
    const int32_t* lengths;
    unsigned long long* keys;
    int32_t* succ;
    float* hash_logp;
    int* counts;
};

// ---------------------------------------------------------------------------
// Full-vocabulary DARTree mode: per depth, every frontier node scores every
// token v by Rk = (Rk_parent + x[v]) + E[parent_tok] . F[v].
// ---------------------------------------------------------------------------
constexpr int kVocabReqPerWave = 2;                       // requests a wave owns
constexpr int kVocabReqPerGroup = kVocabReqPerWave * kWaves;
constexpr int kVocabCap = 320;                            // per-(wave, request) candidate buffer
constexpr int kVocabGroupBlocks = 10;                     // 16-token blocks whose logits load together
constexpr int kVocabChunk = 128;                          // least vocabulary columns per workgroup
constexpr int kVocabGroups = 768;                         // workgroups a depth aims for (three per CU)
constexpr int kFullMaxW = 16;                             // one 16-row MFMA tile per request
constexpr int kMaxVocabChunks = 1024;                     // chunks per depth (at most kVocabGroups)

// one entry of a chunk's top-W list: exact key, the parent-conditioned term,
// the logit and the tie key token * 64 + parent rank (smaller wins)
struct VocabEntry {
    double rk;
    double g;
    float x;
    uint32_t tie;
    uint32_t pad[2];
};

// Each request's non-empty chunk lists of a depth, appended by the
// vocabulary kernel (count cmp_n[b], entries cmp[b][0 .. kFrontCap)), so the
// frontier kernel reads what was found in one round instead of every list
constexpr int kFrontCap = 1024;

struct VocabArgs {
    int B, V, d, W, R, t, dtype;
    int vchunk, C2;
    const void* logits;
    const float* E;
    const float* F;
    const float* fnorm;            // |F_v| (slightly rounded up), [V]
    const uint16_t* Fbf;           // F rounded to bf16 (nearest even), [V][R]
    const int32_t* ctx;
    const int32_t* f_tok;
    const double* f_rk;
    const int32_t* f_n;
    const double* seed;            // [B] a lower bound for this depth's W-th key (-inf = none)
    VocabEntry* part;
    int32_t* cmp_n;                // [B] entries appended this depth
    VocabEntry* cmp;               // [B][kFrontCap]
};

struct FrontierArgs {
    int B, V, d, W, t, C2, k, R;
    const VocabEntry* part;
    int32_t* cmp_n;                // [B] read, then cleared for the next depth
    const VocabEntry* cmp;         // [B][kFrontCap]
    const double* lse;
    const int32_t* ttok;           // [B*d][k] each row's top-k tokens
    const float* tx;               // [B*d][k] their logits
    const float* E;
    const float* F;
    const float* fnorm;            // [V] |F_v|
    double* seed;                  // [B] a lower bound for the next depth's W-th key
    int32_t* f_tok;
    double* f_rk;
    double* f_s;
    int32_t* f_node;
    int32_t* f_n;
    int32_t* n_tree;
    int32_t* nd_tok;
    int32_t* nd_par;
    int32_t* nd_dep;
    double* nd_s;
};

struct FinishArgs {
    int B, d, W, budget, mask_words;
    const int32_t* n_tree;
    const int32_t* nd_tok;
    const int32_t* nd_par;
    const int32_t* nd_dep;
    const double* nd_s;
    int32_t* n_nodes;
    int32_t* tokens;
    int32_t* parents;
    int32_t* depths;
    float* scores;
    uint32_t* mask;
};

struct VerifyArgs {
    int B, budget;
    double cost_fixed, cost_per_token;
    const int32_t* n_nodes;
    const int32_t* parents;
    const int32_t* depths;
    const float* scores;
    int32_t* n_verify;
    int32_t* rank;
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
int n_contexts(int ngram_kind, int d, int k);

// launchers (sweep.hip, tree.hip)
hipError_t launch_sweep(const SweepArgs& a, int64_t rows, int dtype, bool take_turns, hipStream_t stream);
hipError_t launch_prep(const PrepArgs& a, hipStream_t stream);
hipError_t launch_tree(const TreeArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_ngram_update(const NGramUpdateArgs& a, hipStream_t stream);
hipError_t launch_vocab(const VocabArgs& a, hipStream_t stream);
hipError_t launch_fnorm(const float* F, int V, int R, float* out, uint16_t* fbf, hipStream_t stream);
hipError_t launch_frontier(const FrontierArgs& a, hipStream_t stream);
hipError_t launch_seed1(const FrontierArgs& a, const int32_t* ctx, hipStream_t stream);
hipError_t launch_finish(const FinishArgs& a, hipStream_t stream);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);


}  // namespace dt
