/*
 * dt.h -- C ABI of libdt.so: draft-tree construction on AMD Instinct MI355X
 * (gfx950) for diffusion-style speculative decoding.
 *
 * The operation (one call = one batch of B independent requests):
 *
 *   d per-position draft logit rows  --->  pruned draft token tree + mask
 *
 * as the pages define it:
 *   - DART (arXiv 2601.19278), Fig. 3 caption ("Continuity-Aware Tree
 *     Pruning"): the drafter's d logits come from one forward with d-1 mask
 *     tokens ("shifted logits prediction"), the first from the last prefix
 *     position; candidate tokens of each depth are taken from that
 *     position's own logit; an N-gram model keeps only expansions that stay
 *     continuous; the pruned tree is verified with tree attention.
 *   - DARTree (llmdb page, "Tree Construction" and its P_AR equation;
 *     scholarbro abstract): a fixed-width candidate tree of depth K and
 *     width W, every candidate of a depth scored in one batch with a
 *     path-conditioned score, the top-W kept across the whole frontier after
 *     each depth, then best-first pruning selects the verification tree.
 *
 * Concretely, for request b:
 *   1. lse_i = log sum_v exp(logits[b][i][v]) and T_i = the k largest
 *      logits of row i, ordered (value desc, token id asc), i = 0..d-1.
 *   2. The root is the last committed token ctx[b][1] (context ctx[b][0],
 *      ctx[b][1]).  For depth t = 1..d every frontier node p of depth t-1
 *      is paired with every child c in T_{t-1}.  The pair is kept iff
 *      logits[b][t-1][c] > -inf and the N-gram admits c after p's context
 *      (bigram: p's token; trigram: (p's parent's token, p's token), the
 *      root using ctx[b][0]); an admitted entry needs logp > min_logp
 *      (strict), and min_logp = -INFINITY tests membership only.
 *   3. Each kept child gets Rk = (Rk_p + x) + g and S = (S_p + (x - lse)) + g
 *      in double precision, x = its logit, g = E[tok_p] . F[c] in DARTREE
 *      mode (the low-rank parent-conditioned term), g = 0 in DART mode.
 *      The frontier of depth t is the first min(W, #kept) candidates in the
 *      order (Rk desc, token asc, parent's frontier rank asc).  Growth stops
 *      at the first empty frontier.
 *   4. If the candidate tree has more than `budget` nodes, best-first
 *      selection repeatedly takes the available node (parent already taken,
 *      or depth 1) with the best (S desc, depth asc, BFS index asc) until
 *      `budget` nodes are taken.
 *   5. Output in BFS order (depth asc, then frontier rank).
 *
 * DARTREE_FULL mode (DARTree page, "Tree Construction": the drafter proposes
 * W candidate tokens per frontier node): instead of the position's shared
 * top-k, every frontier node p proposes its own W best tokens of the whole
 * vocabulary under its parent-conditioned distribution x[v] + E[tok_p].F[v]
 * (order: Rk desc, token asc), and the frontier is the top-W of all
 * proposals, ranked as in step 3.  This equals the top-W over every
 * (node, token) pair.  k is not used for proposals; the N-gram table must
 * be of kind NONE; W <= 16 and R in {16, 32, 64}.  Keys are exact fp64 (the
 * dense product runs on bf16 matrix cores only to discard tokens that
 * provably cannot be selected).  Best-first selection is replayed literally
 * (g may be positive, so S can rise along a path).
 *
 * Output tree (caller-allocated device memory, n_max = budget,
 * mask_words = ceil(budget / 32)):
 *   n_nodes [B]                     int32, number of draft nodes (0..budget)
 *   tokens  [B][n_max]              int32, token id, -1 in padding rows
 *   parents [B][n_max]              int32, parent node index, -1 = the root
 *   depths  [B][n_max]              int32, 1..d, 0 in padding rows
 *   scores  [B][n_max]              float, S rounded to fp32, -inf padding
 *   mask    [B][n_max][mask_words]  uint32, row i has bit j (word j >> 5,
 *                                   bit j & 31, LSB first) set iff node j
 *                                   is node i or one of its ancestors; the
 *                                   root and prefix are implicit; padding
 *                                   rows are zero.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers unless stated otherwise; the
 *     structs themselves are host memory read during the call only.
 *   - The caller owns every buffer, including the workspace.  The library
 *     never allocates, frees or synchronises, and keeps no state between
 *     calls (dt_build_tree_noalloc aside: it holds its scratch array per
 *     GPU).  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and the call returns without waiting.  Calls on different
 *     streams need different workspaces.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     an error nothing is enqueued and no output is touched.  A launch
 *     failure returns DT_ERR_HIP.  Faults during execution surface at the
 *     caller's next synchronisation of `stream`.
 *   - Logits are finite or -inf.  NaN or +inf logits give unspecified
 *     (but memory-safe) results.  ctx ids must lie in [0, V); other values
 *     admit no children under bigram tables and add no parent term.  Table
 *     contents (row_ptr ranges, successor ids) are trusted as given.
 *   - Limits: B >= 0; 1 <= d <= 32; 1 <= k <= 32 and k <= V; 1 <= W <= 64;
 *     W * k <= 1024; 1 <= budget <= 1024; 1 <= V < 2^26; the logits
 *     pointer 16-byte aligned; and the tree kernel's shared-memory plan
 *     (which grows with d, k, W, the N-gram kind and the mode) must fit in
 *     the 160 KiB of LDS a gfx950 workgroup may use, else
 *     DT_ERR_UNSUPPORTED.  DARTREE mode needs E and F 16-byte
 *     aligned with R a multiple of 4, 4 <= R <= 256.  A trigram table's
 *     keys array must be 16-byte aligned.
 */
#ifndef DT_H
#define DT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dt_status {
    DT_OK = 0,
    DT_ERR_INVALID_ARG = 1,   /* a null pointer, a value out of range, a misaligned buffer */
    DT_ERR_UNSUPPORTED = 2,   /* valid but outside the library's limits (see above) */
    DT_ERR_WORKSPACE = 3,     /* workspace missing or smaller than dt_workspace_size() */
    DT_ERR_HIP = 4            /* the HIP runtime refused a launch */
} dt_status;

typedef enum dt_dtype { DT_DTYPE_F32 = 0, DT_DTYPE_BF16 = 1 } dt_dtype;

typedef enum dt_mode {
    DT_MODE_DART = 0,      /* score = cumulative draft log-probability */
    DT_MODE_DARTREE = 1,   /* + parent-conditioned term E[parent] . F[child] */
    DT_MODE_DARTREE_FULL = 2  /* DARTREE with per-node proposals over the whole vocabulary */
} dt_mode;

typedef enum dt_ngram_kind {
    DT_NGRAM_NONE = 0,          /* every expansion is continuous */
    DT_NGRAM_DENSE_BIGRAM = 1,  /* logp[V][V] indexed [parent token][child] */
    DT_NGRAM_CSR_BIGRAM = 2,    /* successors of a token, ascending ids */
    DT_NGRAM_HASH_TRIGRAM = 3   /* open-addressing table keyed by (t_-2, t_-1) */
} dt_ngram_kind;

/* N-gram continuity table (device arrays; unused fields may be NULL).
 *  dense:  dense_logp[V][V] float.
 *  CSR:    row_ptr[V+1] int32, col[nnz] int32 ascending within a row,
 *          csr_logp[nnz] float (may be NULL when min_logp = -INFINITY);
 *          col and csr_logp may be NULL when nnz = 0 (every row empty).
 *  hash:   keys[cap] uint64 with key = (uint64)t_-2 << 32 | (uint32)t_-1 and
 *          0xFFFFFFFFFFFFFFFF marking a free slot; a key lives in the first
 *          free slot at or after splitmix64(key) & (cap - 1) (the SplitMix64
 *          output function of Steele, Lea and Flood), probing linearly with
 *          wrap-around; succ[cap][S] int32 successor ids, -1 = none;
 *          hash_logp[cap][S] float (may be NULL when min_logp = -INFINITY).
 *          cap is a power of two with at least one free slot, 1 <= S <= 64. */
typedef struct dt_ngram_table {
    int32_t kind;              /* dt_ngram_kind */
    float min_logp;            /* keep iff logp > min_logp; -INFINITY = membership */
    const float* dense_logp;
    const int32_t* row_ptr;
    const int32_t* col;
    const float* csr_logp;
    int64_t nnz;
    const uint64_t* keys;
    const int32_t* succ;
    const float* hash_logp;
    int64_t cap;
    int32_t S;
} dt_ngram_table;

typedef struct dt_params {
    int32_t B;                 /* requests in the batch */
    int32_t V;                 /* vocabulary size (row length) */
    int32_t d;                 /* draft positions = tree depth (K in DARTree) */
    int32_t k;                 /* candidates taken from each position's logit */
    int32_t W;                 /* frontier width kept per depth */
    int32_t budget;            /* verification budget = n_max rows of the output */
    int32_t dtype;             /* dt_dtype of the logits */
    int32_t mode;              /* dt_mode */
    const int32_t* ctx;        /* [B][2] device: (t_-2, t_-1), t_-1 is the root */
    const float* E;            /* [V][R] device, DARTREE only (else may be NULL) */
    const float* F;            /* [V][R] device, DARTREE only */
    int32_t R;                 /* rank of E and F */
    int32_t sweep_chunks;      /* 0 = automatic; else split each row into this many chunks */
    void* workspace;           /* device scratch of at least dt_workspace_size() bytes */
    size_t workspace_bytes;
    void* stream;              /* hipStream_t */
    void* prof_event_start;    /* optional hipEvent_t recorded on `stream` right before */
    void* prof_event_stop;     /* ... and right after the vocabulary-sweep kernel */
} dt_params;

typedef struct dt_tree_out {
    int32_t* n_nodes;          /* [B] */
    int32_t* tokens;           /* [B][budget] */
    int32_t* parents;          /* [B][budget] */
    int32_t* depths;           /* [B][budget] */
    float* scores;             /* [B][budget] */
    uint32_t* mask;            /* [B][budget][ceil(budget/32)] */
} dt_tree_out;

/* The whole path (steps 1-5 above) for B requests.
 * logits: device [B][d][V] of dtype, rows contiguous, 16-byte aligned.
 * Calls on different streams overlap: a sweep of 257 to 512 workgroups
 * (one to two per compute unit, e.g. B=64 at V=151936, d=8) holds 56 KiB
 * of LDS per workgroup when the call's
 * prep and tree workgroups still fit beside two of them, so two calls'
 * sweeps take turns instead of sharing the memory bandwidth, and one call's
 * (latency-bound, raised-priority) prep and tree kernels run beside the next
 * call's sweep. */
dt_status dt_build_tree(const void* logits, const dt_ngram_table* ngram,
                        const dt_params* params, const dt_tree_out* out);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation as dt_build_tree, same arguments except that params->workspace
 * and params->workspace_bytes are ignored.  The workspace is instead a
 * scratch array of DT_NOALLOC_SCRATCH_BYTES bytes inside the library, one
 * copy per GPU (the device of params->stream, or the current device for
 * the null stream), held from the first call on that GPU until the process
 * ends.  The call allocates nothing and calls no allocating routine; its
 * first call on a GPU looks the array's address up (hipGetSymbolAddress).
 * Every call on one GPU shares that GPU's array: calls whose executions
 * overlap on the same GPU (different streams, or different host threads)
 * race and give undefined trees, so serialise them (one stream, or events).
 * Errors: as dt_build_tree, and DT_ERR_WORKSPACE when dt_workspace_size()
 * of the parameters exceeds DT_NOALLOC_SCRATCH_BYTES; DT_ERR_HIP when the
 * device or the array's address cannot be obtained. */
#define DT_NOALLOC_SCRATCH_BYTES (32u << 20)
dt_status dt_build_tree_noalloc(const void* logits, const dt_ngram_table* ngram,
                                const dt_params* params, const dt_tree_out* out);

/* Bytes of workspace dt_build_tree / dt_position_topk need for these
 * parameters (depends on B, V, d, k, mode, dtype and sweep_chunks only, and
 * on W and R in DARTREE_FULL mode; the N-gram area is sized for the largest
 * table kind); 0 if the parameters are invalid.  The workspace holds the
 * sweep's per-chunk partials and the per-row normalisers, top-k lists,
 * continuity masks (and DARTree terms) the tree step reads; in DARTREE_FULL
 * mode also the frontier, the candidate tree, the column norms and a bf16
 * copy of F (V * R * 2 bytes) for the matrix-core screen, and every
 * vocabulary chunk's top-W.  Its contents are meaningless between calls. */
size_t dt_workspace_size(const dt_params* params);

/* Static, human-readable name of a status code. */
const char* dt_status_string(dt_status s);

/* Step 1 alone (DART Fig. 3: each position's own logit proposes the tokens
 * of its depth): per row (b, i) the log-softmax normaliser and the top-k.
 * lse: device [B][d] double; topk_tok: device [B][d][k] int32 in order
 * (value desc, id asc); topk_val: device [B][d][k] float (the logits).
 * Uses B, V, d, k, dtype, sweep_chunks, workspace and stream of params. */
dt_status dt_position_topk(const void* logits, const dt_params* params,
                           double* lse, int32_t* topk_tok, float* topk_val);

/* The step after verification: keep a trigram table current with the tokens
 * the target accepted (the N-gram model that keeps DART's expansions
 * continuous, DART Fig. 3).  For request b the stream ctx[b][0], ctx[b][1],
 * tokens[b][0 .. lengths[b]-1] contributes, for every accepted token s_i,
 * the trigram (s_{i-2}, s_{i-1}) -> s_i:
 *   - a missing key takes the first free slot of its probe sequence (the
 *     layout dt_build_tree reads: first free slot at or after
 *     splitmix64(key) & (cap - 1), linear probing); its row starts empty,
 *     so rows of free slots must hold -1 in every entry;
 *   - a missing successor takes the first -1 entry of the key's row and,
 *     when table->hash_logp is not NULL, the log-probability new_logp;
 *   - a trigram whose row is full, whose probe sequence has no free slot, or
 *     whose key equals the free-slot marker is dropped.
 * The trigrams of one call are applied concurrently: the resulting keys and
 * successor sets are those of applying them one by one in any order as long
 * as no row fills up and the table keeps free slots; the slot a new key lands
 * in, and which successors an overflowing row keeps, may vary between runs.
 * table: kind DT_NGRAM_HASH_TRIGRAM; its keys, succ and (if not NULL)
 *   hash_logp arrays are written in place (keys 8-byte, succ and hash_logp
 *   4-byte aligned).
 * ctx: device [B][2] int32; tokens: device [B][L] int32; lengths: device [B]
 *   int32 (entries past lengths[b], or past L, are ignored).
 * counts: device int32[3] or NULL; atomically incremented by keys added,
 *   successors added and trigrams dropped (the caller zeroes it).
 * Must not run concurrently with a dt_build_tree reading the same table.
 * Errors: DT_ERR_INVALID_ARG for a non-trigram table, null or misaligned
 *   arrays, cap not a power of two >= 2, B or L < 0 or a NaN new_logp;
 *   DT_ERR_UNSUPPORTED for S outside 1..64; DT_ERR_HIP if the launch fails. */
dt_status dt_ngram_update(const dt_ngram_table* table, const int32_t* ctx, const int32_t* tokens,
                          const int32_t* lengths, int32_t B, int32_t L, float new_logp,
                          int32_t* counts, void* stream);

/* How many nodes of each built tree to send to verification (LibraSpec,
 * scholarbro listing abstract: the speculative length is chosen for expected
 * speedup and extended only while the acceptance gain outweighs the added
 * verification cost, judged from the drafter's confidence).  Candidate
 * verification sets are the prefixes of the tree's best-first order (a node
 * is available once its parent is taken; the best available by score desc,
 * depth asc, index asc is taken next; every prefix is closed under parents).
 * Node n of that order has confidence c_n = exp(score_n); with
 * A(n) = 1 + sum_{i<n} c_i expected tokens per round and
 * T(n) = cost_fixed + cost_per_token * n its cost (any time unit), node n is
 * added while c_n * T(n) > cost_per_token * A(n), i.e. while A/T strictly
 * grows; n_verify[b] is where that stops (0..n_nodes).  rank[b][i] receives
 * node i's best-first position, -1 for rows i >= n_nodes: verify the nodes
 * with rank < n_verify.
 * tree: the arrays dt_build_tree wrote ([B][budget]; tokens and mask unused).
 * n_verify: device [B] int32; rank: device [B][budget] int32.
 * Errors: DT_ERR_INVALID_ARG for null arrays, B < 0, budget < 1, or a cost
 *   that is not finite, cost_fixed <= 0 or cost_per_token < 0;
 *   DT_ERR_UNSUPPORTED for budget > 1024; DT_ERR_HIP if the launch fails. */
dt_status dt_verify_length(const dt_tree_out* tree, int32_t B, int32_t budget, double cost_fixed,
                           double cost_per_token, int32_t* n_verify, int32_t* rank, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DT_H */
