/*
 * Plain CPU oracle for draft-tree construction.  TEST INFRASTRUCTURE ONLY:
 * it exists so the tests, the smoke check and the CPU-baseline leg of the
 * benchmark can check and time the HIP library against an obviously correct
 * implementation.  The product path never calls it.
 *
 * What it computes, in the order the method states it:
 *  - DART (arXiv 2601.19278), Fig. 3 caption: the d logits of one drafter
 *    forward each propose the token of one tree depth ("candidate tokens are
 *    selected from the corresponding position's predicted logit"), an N-gram
 *    model keeps only continuations that stay continuous, and the pruned tree
 *    is verified with tree attention.
 *  - DARTree (llmdb page, "Tree Construction" and its equation; scholarbro
 *    abstract): a fixed-width candidate tree of depth K and width W, all
 *    candidates of a depth scored in one batch with a path-conditioned score,
 *    the top-W across the whole frontier kept after every depth, then
 *    best-first pruning selects the verification tree.
 *
 * Readings where the pages are silent:
 *  - the N-gram is a hard filter, keep iff logp > min_logp (strict); with
 *    min_logp = -INFINITY sparse tables test membership only;
 *  - continuity is checked at every depth, depth 1 against the committed
 *    context ctx[b] = (t_-2, t_-1);
 *  - the ranked score is the cumulative path log-probability
 *    S = sum(x - lse) (+ g in DARTree mode), g = E[parent_tok] . F[child_tok];
 *    within a depth the lse-free key Rk = sum(x) (+ g) orders candidates
 *    identically and is what is sorted;
 *  - ties: top-k by (x desc, id asc); frontier by (Rk desc, token asc,
 *    parent rank asc); budget by (S desc, depth asc, BFS index asc);
 *  - children with x = -inf (probability zero) are never expanded;
 *  - the budget counts draft nodes (root excluded);
 *  - full-vocabulary DARTree mode (ORACLE_MODE_DARTREE_FULL): the drafter
 *    proposes W tokens for every frontier node (DARTree page, "Tree
 *    Construction": W proposals per frontier node) from that
 *    node's own parent-conditioned distribution over the whole vocabulary,
 *    x[v] + E[parent_tok] . F[v]; a node's proposals are its W best tokens
 *    under the candidate order (Rk desc, token asc), and the frontier is then
 *    the top-W of all proposals as in the other modes.  k is not used.
 *
 * All arithmetic is double precision.  Logits are read exactly (bf16 widened
 * by a 16-bit shift).  NaN logits are undefined.
 */
#ifndef DT_ORACLE_H
#define DT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_NGRAM_NONE 0
#define ORACLE_NGRAM_DENSE_BIGRAM 1
#define ORACLE_NGRAM_CSR_BIGRAM 2
#define ORACLE_NGRAM_HASH_TRIGRAM 3

#define ORACLE_MODE_DART 0
#define ORACLE_MODE_DARTREE 1
#define ORACLE_MODE_DARTREE_FULL 2

typedef struct oracle_ngram {
    int32_t kind;
    float min_logp;
    const float* dense_logp;    /* [V][V] */
    const int32_t* row_ptr;     /* [V+1] */
    const int32_t* col;         /* [nnz] */
    const float* csr_logp;      /* [nnz] */
    const uint64_t* keys;       /* [cap], 0xFFFF..FF = empty */
    const int32_t* succ;        /* [cap][S], -1 = none */
    const float* hash_logp;     /* [cap][S] */
    int64_t cap;
    int32_t S;
} oracle_ngram;

/* log-softmax normaliser of one row: m + log(sum exp(x - m)), -inf if every
 * entry is -inf. */
double oracle_row_lse(const void* row, int is_bf16, int64_t V);

/* The k largest entries of one row by (value desc, id asc): ids and values. */
void oracle_row_topk(const void* row, int is_bf16, int64_t V, int k,
                     int32_t* tok, double* val);

/* Does the N-gram admit child token c after context (t2, t1)?  (t2 is only
 * used by the trigram.) */
int oracle_continuity(const oracle_ngram* ng, int64_t V, int32_t t2, int32_t t1, int32_t c);

/* The whole path for B requests.  Outputs are [B][budget] (mask
 * [B][budget][ceil(budget/32)]); rows past n_nodes hold token -1,
 * parent -1, depth 0, score -inf and a zero mask row.  lookups (optional,
 * [B]) receives the number of N-gram lookups made (one per expanded node).
 * Returns 0, or -1 on invalid arguments. */
int oracle_build_tree(const void* logits, int is_bf16, int B, int64_t V, int d, int k,
                      int W, int budget, int mode, const int32_t* ctx,
                      const float* E, const float* F, int R, const oracle_ngram* ng,
                      int32_t* n_nodes, int32_t* tokens, int32_t* parents,
                      int32_t* depths, float* scores, uint32_t* mask, int64_t* lookups);

/* Keep a trigram table current after verification (the step after the
 * path: "an N-gram model" that the DART pages pair with the drafter, kept
 * from the tokens the target accepted).  For every request b, in order, the
 * stream ctx[b][0], ctx[b][1], tokens[b][0 .. lengths[b]-1] contributes, for
 * each accepted token s_i, the trigram (s_{i-2}, s_{i-1}) -> s_i, applied in
 * stream order: a missing key takes the first free slot of its linear probe
 * sequence (its successor row starts empty); a missing successor takes the
 * first free (-1) entry of the key's row and, when the table has a logp
 * array, the log-probability new_logp.  A trigram whose row is full, whose
 * key finds no free slot, or whose key equals the free-slot marker is
 * dropped.  The arrays are updated in place; counts[3] receives keys added,
 * successors added and trigrams dropped.  Returns 0, or -1 on invalid
 * arguments. */
int oracle_ngram_update(uint64_t* keys, int32_t* succ, float* hash_logp, int64_t cap, int32_t S,
                        const int32_t* ctx, const int32_t* tokens, const int32_t* lengths,
                        int B, int L, float new_logp, int64_t* counts);

/* How many nodes of a built tree to verify (LibraSpec, scholarbro listing
 * abstract: the speculative length is chosen by expected speedup, extending
 * only while the acceptance gain outweighs the extra verification cost,
 * judged from the drafter's confidence).  For each request, in best-first
 * order over its tree (a node is available once its parent is taken; the
 * best available by (score desc, depth asc, index asc) is taken next), node
 * n has confidence c_n = exp(score_n), the drafter's probability that its
 * whole path is accepted.  With A(n) = 1 + sum_{i<n} c_i expected tokens per
 * round and T(n) = cost_fixed + cost_per_token * n the round's cost, node n
 * is added while c_n * T(n) > cost_per_token * A(n), i.e. while A/T strictly
 * grows; the first n where it does not is n_verify.  rank[b][i] receives the
 * best-first position of node i (-1 for rows past n_nodes).  Inputs are the
 * tree arrays as dt_build_tree writes them (host memory here).  Returns 0,
 * or -1 on invalid arguments (cost_fixed <= 0, cost_per_token < 0). */
int oracle_verify_length(const int32_t* n_nodes, const int32_t* parents, const int32_t* depths,
                         const float* scores, int B, int budget, double cost_fixed, double cost_per_token,
                         int32_t* n_verify, int32_t* rank);

#ifdef __cplusplus
}
#endif
#endif
