/*
 * Plain CPU oracle for draft-tree construction.  TEST INFRASTRUCTURE ONLY
 * (tests, the smoke check and the benchmark's CPU-baseline leg); see
 * oracle.h for what is computed and the readings taken.  Scalar loops,
 * double precision, full sorts: slow and meant to be checked by eye.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- reading the inputs ------------------------------------------------ */

static double logit_at(const void* base, int is_bf16, int64_t i) {
    if (is_bf16) {
        uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16; /* bf16 -> fp32 is exact */
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float*)base)[i];
}

/* ---- per-position normaliser and top-k (DART Fig. 3: each position's own
 *      logit proposes the tokens of its depth) ----------------------------- */

double oracle_row_lse(const void* row, int is_bf16, int64_t V) {
    double m = -INFINITY;
    for (int64_t v = 0; v < V; ++v) {
        double x = logit_at(row, is_bf16, v);
        if (x > m) m = x;
    }
    if (m == -INFINITY) return -INFINITY;
    double s = 0.0;
    for (int64_t v = 0; v < V; ++v) s += exp(logit_at(row, is_bf16, v) - m);
    return m + log(s);
}

typedef struct {
    double x;
    int32_t id;
} entry;

static int by_value_desc_id_asc(const void* a, const void* b) {
    const entry* p = (const entry*)a;
    const entry* q = (const entry*)b;
    if (p->x > q->x) return -1;
    if (p->x < q->x) return 1;
    return (p->id > q->id) - (p->id < q->id);
}

void oracle_row_topk(const void* row, int is_bf16, int64_t V, int k, int32_t* tok, double* val) {
    entry* all = (entry*)malloc((size_t)V * sizeof(entry));
    for (int64_t v = 0; v < V; ++v) {
        all[v].x = logit_at(row, is_bf16, v);
        all[v].id = (int32_t)v;
    }
    qsort(all, (size_t)V, sizeof(entry), by_value_desc_id_asc);
    for (int i = 0; i < k; ++i) {
        tok[i] = all[i].id;
        val[i] = all[i].x;
    }
    free(all);
}

/* ---- N-gram continuity (DART Fig. 3: "a N-gram model ensures that the
 *      expanded tokens maintain continuity") -------------------------------- */

static uint64_t splitmix64_mix(uint64_t z) {
    /* SplitMix64 output function (Steele, Lea, Flood; Vigna's public-domain
     * reference implementation). */
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static int keeps(const oracle_ngram* ng, double logp) {
    return logp > (double)ng->min_logp;
}

int oracle_continuity(const oracle_ngram* ng, int64_t V, int32_t t2, int32_t t1, int32_t c) {
    switch (ng->kind) {
    case ORACLE_NGRAM_NONE:
        return 1;
    case ORACLE_NGRAM_DENSE_BIGRAM:
        return keeps(ng, (double)ng->dense_logp[(int64_t)t1 * V + c]);
    case ORACLE_NGRAM_CSR_BIGRAM:
        for (int32_t e = ng->row_ptr[t1]; e < ng->row_ptr[t1 + 1]; ++e) {
            if (ng->col[e] == c)
                return ng->min_logp == -INFINITY || ng->csr_logp == NULL ||
                       keeps(ng, (double)ng->csr_logp[e]);
        }
        return 0;
    case ORACLE_NGRAM_HASH_TRIGRAM: {
        uint64_t key = ((uint64_t)(uint32_t)t2 << 32) | (uint32_t)t1;
        uint64_t slot = splitmix64_mix(key) & (uint64_t)(ng->cap - 1);
        for (int64_t probe = 0; probe < ng->cap; ++probe) {
            uint64_t here = ng->keys[slot];
            if (here == ~0ULL) return 0;        /* empty slot: key absent */
            if (here == key) {
                for (int32_t s = 0; s < ng->S; ++s) {
                    int64_t e = (int64_t)slot * ng->S + s;
                    if (ng->succ[e] == c)
                        return ng->min_logp == -INFINITY || ng->hash_logp == NULL ||
                               keeps(ng, (double)ng->hash_logp[e]);
                }
                return 0;
            }
            slot = (slot + 1) & (uint64_t)(ng->cap - 1);
        }
        return 0;
    }
    default:
        return 0;
    }
}

/* ---- the tree ----------------------------------------------------------- */

typedef struct {
    int32_t tok;      /* drafted token */
    int32_t parent;   /* index of the parent in the candidate tree, -1 = root */
    int32_t depth;    /* 1..d */
    int32_t rank;     /* rank within its depth's frontier */
    double rk;        /* sum of raw logits (+ g) along the path: within-depth key */
    double s;         /* cumulative log-score sum(x - lse) (+ g) */
} node;

typedef struct {
    double rk, s;
    int32_t tok, parent_rank, parent;
} cand;

static int cand_order(const void* a, const void* b) {
    const cand* p = (const cand*)a;
    const cand* q = (const cand*)b;
    if (p->rk > q->rk) return -1;
    if (p->rk < q->rk) return 1;
    if (p->tok != q->tok) return p->tok < q->tok ? -1 : 1;
    return (p->parent_rank > q->parent_rank) - (p->parent_rank < q->parent_rank);
}

/* best-first order for the verification budget: (S desc, depth asc, index asc) */
static int better_for_budget(const node* nodes, int a, int b) {
    if (nodes[a].s != nodes[b].s) return nodes[a].s > nodes[b].s;
    if (nodes[a].depth != nodes[b].depth) return nodes[a].depth < nodes[b].depth;
    return a < b;
}

static double dot_fp64(const float* e, const float* f, int R) {
    double acc = 0.0;
    for (int j = 0; j < R; ++j) acc += (double)e[j] * (double)f[j];
    return acc;
}

int oracle_build_tree(const void* logits, int is_bf16, int B, int64_t V, int d, int k,
                      int W, int budget, int mode, const int32_t* ctx,
                      const float* E, const float* F, int R, const oracle_ngram* ng,
                      int32_t* n_nodes, int32_t* tokens, int32_t* parents,
                      int32_t* depths, float* scores, uint32_t* mask, int64_t* lookups) {
    if (B < 0 || V < 1 || d < 1 || k < 1 || k > V || W < 1 || budget < 1) return -1;
    if (mode != ORACLE_MODE_DART && mode != ORACLE_MODE_DARTREE && mode != ORACLE_MODE_DARTREE_FULL) return -1;
    if (mode != ORACLE_MODE_DART && (E == NULL || F == NULL || R < 1)) return -1;
    const int full = mode == ORACLE_MODE_DARTREE_FULL;
    const int words = (budget + 31) / 32;
    const size_t esize = is_bf16 ? 2 : 4;

    double* lse = (double*)malloc((size_t)d * sizeof(double));
    int32_t* top_tok = (int32_t*)malloc((size_t)d * k * sizeof(int32_t));
    double* top_x = (double*)malloc((size_t)d * k * sizeof(double));
    node* nodes = (node*)malloc((size_t)d * W * sizeof(node));
    /* full-vocabulary mode: W proposals per frontier node, chosen from all V */
    cand* cands = (cand*)malloc((size_t)W * (full ? W : k) * sizeof(cand));
    cand* pool = full ? (cand*)malloc((size_t)V * sizeof(cand)) : NULL;
    int* frontier = (int*)malloc((size_t)W * sizeof(int));
    int* next = (int*)malloc((size_t)W * sizeof(int));
    char* taken = (char*)malloc((size_t)d * W);
    int32_t* new_index = (int32_t*)malloc((size_t)d * W * sizeof(int32_t));

    for (int b = 0; b < B; ++b) {
        const char* req = (const char*)logits + (size_t)b * d * V * esize;
        const int32_t ctx2 = ctx[2 * b + 0], ctx1 = ctx[2 * b + 1];
        int64_t nlook = 0;

        /* 1-2. per position: normaliser and top-k of its own logit row */
        for (int i = 0; i < d; ++i) {
            const char* row = req + (size_t)i * V * esize;
            lse[i] = oracle_row_lse(row, is_bf16, V);
            if (!full) oracle_row_topk(row, is_bf16, V, k, top_tok + (size_t)i * k, top_x + (size_t)i * k);
        }

        /* 3-4. depth loop: expand every frontier node with its depth's
         * candidates, keep the top-W across the whole frontier */
        int n_tree = 0;        /* nodes in the candidate tree so far (BFS order) */
        int n_front = 1;       /* the root is the only frontier node of depth 0 */
        frontier[0] = -1;
        for (int t = 1; t <= d; ++t) {
            const int pos = t - 1; /* logit row proposing depth t */
            int nc = 0;
            for (int r = 0; r < n_front; ++r) {
                const int p = frontier[r];
                const int32_t ptok = p < 0 ? ctx1 : nodes[p].tok;
                const int32_t pprev = p < 0 ? ctx2 : (nodes[p].parent < 0 ? ctx1 : nodes[nodes[p].parent].tok);
                const double prk = p < 0 ? 0.0 : nodes[p].rk;
                const double ps = p < 0 ? 0.0 : nodes[p].s;
                if (ng->kind != ORACLE_NGRAM_NONE) ++nlook;
                if (full) {
                    /* this node's own proposals: score every token of the
                     * vocabulary under the node's path, keep its W best */
                    const char* row = req + (size_t)pos * V * esize;
                    int np = 0;
                    for (int64_t v = 0; v < V; ++v) {
                        const double x = logit_at(row, is_bf16, v);
                        if (x == -INFINITY) continue;
                        if (!oracle_continuity(ng, V, pprev, ptok, (int32_t)v)) continue;
                        const double g = dot_fp64(E + (size_t)ptok * R, F + (size_t)v * R, R);
                        cand* cd = &pool[np++];
                        cd->rk = (prk + x) + g;
                        cd->s = (ps + (x - lse[pos])) + g;
                        cd->tok = (int32_t)v;
                        cd->parent_rank = r;
                        cd->parent = p;
                    }
                    qsort(pool, (size_t)np, sizeof(cand), cand_order);
                    const int take = np < W ? np : W;
                    memcpy(cands + nc, pool, (size_t)take * sizeof(cand));
                    nc += take;
                    continue;
                }
                for (int j = 0; j < k; ++j) {
                    const int32_t c = top_tok[(size_t)pos * k + j];
                    const double x = top_x[(size_t)pos * k + j];
                    if (x == -INFINITY) continue;                       /* probability zero */
                    if (!oracle_continuity(ng, V, pprev, ptok, c)) continue;
                    double g = 0.0;
                    if (mode == ORACLE_MODE_DARTREE)
                        g = dot_fp64(E + (size_t)ptok * R, F + (size_t)c * R, R);
                    cand* cd = &cands[nc++];
                    cd->rk = (prk + x) + g;
                    cd->s = (ps + (x - lse[pos])) + g;
                    cd->tok = c;
                    cd->parent_rank = r;
                    cd->parent = p;
                }
            }
            if (nc == 0) break;
            qsort(cands, (size_t)nc, sizeof(cand), cand_order);
            const int keep = nc < W ? nc : W;
            for (int r = 0; r < keep; ++r) {
                node* nd = &nodes[n_tree];
                nd->tok = cands[r].tok;
                nd->parent = cands[r].parent;
                nd->depth = t;
                nd->rank = r;
                nd->rk = cands[r].rk;
                nd->s = cands[r].s;
                next[r] = n_tree++;
            }
            memcpy(frontier, next, (size_t)keep * sizeof(int));
            n_front = keep;
        }

        /* 6. verification budget: best-first over the candidate tree, a node
         * becomes available once its parent is taken */
        if (n_tree <= budget) {
            memset(taken, 1, (size_t)n_tree);
        } else {
            memset(taken, 0, (size_t)n_tree);
            for (int step = 0; step < budget; ++step) {
                int best = -1;
                for (int i = 0; i < n_tree; ++i) {
                    if (taken[i]) continue;
                    if (nodes[i].parent >= 0 && !taken[nodes[i].parent]) continue;
                    if (best < 0 || better_for_budget(nodes, i, best)) best = i;
                }
                taken[best] = 1;
            }
        }

        /* 7-8. compact in BFS order, remap parents, pack the ancestor mask */
        int n_out = 0;
        for (int i = 0; i < n_tree; ++i) new_index[i] = taken[i] ? n_out++ : -1;
        int32_t* o_tok = tokens + (size_t)b * budget;
        int32_t* o_par = parents + (size_t)b * budget;
        int32_t* o_dep = depths + (size_t)b * budget;
        float* o_sc = scores + (size_t)b * budget;
        uint32_t* o_mask = mask + (size_t)b * budget * words;
        for (int i = 0; i < budget; ++i) {
            o_tok[i] = -1;
            o_par[i] = -1;
            o_dep[i] = 0;
            o_sc[i] = -INFINITY;
        }
        memset(o_mask, 0, (size_t)budget * words * sizeof(uint32_t));
        for (int i = 0; i < n_tree; ++i) {
            const int o = new_index[i];
            if (o < 0) continue;
            const int po = nodes[i].parent < 0 ? -1 : new_index[nodes[i].parent];
            o_tok[o] = nodes[i].tok;
            o_par[o] = po;
            o_dep[o] = nodes[i].depth;
            o_sc[o] = (float)nodes[i].s;
            /* row(o) = row(parent) | bit(o): every node attends to its ancestors and itself */
            if (po >= 0) memcpy(o_mask + (size_t)o * words, o_mask + (size_t)po * words, words * sizeof(uint32_t));
            o_mask[(size_t)o * words + (o >> 5)] |= 1u << (o & 31);
        }
        n_nodes[b] = n_out;
        if (lookups) lookups[b] = nlook;
    }

    free(lse);
    free(top_tok);
    free(top_x);
    free(nodes);
    free(cands);
    free(pool);
    free(frontier);
    free(next);
    free(taken);
    free(new_index);
    return 0;
}

/* ---- keeping the trigram table current ---------------------------------- */

int oracle_ngram_update(uint64_t* keys, int32_t* succ, float* hash_logp, int64_t cap, int32_t S,
                        const int32_t* ctx, const int32_t* tokens, const int32_t* lengths,
                        int B, int L, float new_logp, int64_t* counts) {
    if (!keys || !succ || !ctx || !tokens || !lengths || !counts || cap < 2 || (cap & (cap - 1)) ||
        S < 1 || B < 0 || L < 0)
        return -1;
    counts[0] = counts[1] = counts[2] = 0;
    for (int b = 0; b < B; ++b) {
        int32_t prev2 = ctx[2 * b], prev1 = ctx[2 * b + 1];
        const int n = lengths[b] < L ? lengths[b] : L;
        for (int i = 0; i < n; ++i) {
            const int32_t c = tokens[(int64_t)b * L + i];
            const uint64_t key = ((uint64_t)(uint32_t)prev2 << 32) | (uint32_t)prev1;
            prev2 = prev1;
            prev1 = c;
            if (key == ~0ULL) {                   /* indistinguishable from a free slot */
                ++counts[2];
                continue;
            }
            /* find the key, or the first free slot of its probe sequence */
            int64_t slot = -1;
            uint64_t pos = splitmix64_mix(key) & (uint64_t)(cap - 1);
            for (int64_t probe = 0; probe < cap; ++probe) {
                if (keys[pos] == key) {
                    slot = (int64_t)pos;
                    break;
                }
                if (keys[pos] == ~0ULL) {
                    keys[pos] = key;
                    ++counts[0];
                    slot = (int64_t)pos;
                    break;
                }
                pos = (pos + 1) & (uint64_t)(cap - 1);
            }
            if (slot < 0) {                       /* no free slot on the way */
                ++counts[2];
                continue;
            }
            /* the successor: present already, or the first free entry */
            int placed = 0;
            for (int32_t e = 0; e < S; ++e) {
                int32_t* here = &succ[slot * S + e];
                if (*here == c) {
                    placed = 1;
                    break;
                }
                if (*here == -1) {
                    *here = c;
                    if (hash_logp) hash_logp[slot * S + e] = new_logp;
                    ++counts[1];
                    placed = 1;
                    break;
                }
            }
            if (!placed) ++counts[2];             /* row full */
        }
    }
    return 0;
}

/* ---- how many nodes to verify ------------------------------------------- */

int oracle_verify_length(const int32_t* n_nodes, const int32_t* parents, const int32_t* depths,
                         const float* scores, int B, int budget, double cost_fixed, double cost_per_token,
                         int32_t* n_verify, int32_t* rank) {
    if (B < 0 || budget < 1 || !(cost_fixed > 0.0) || !(cost_per_token >= 0.0)) return -1;
    char* taken = (char*)malloc((size_t)budget);
    int32_t* order = (int32_t*)malloc((size_t)budget * sizeof(int32_t));
    for (int b = 0; b < B; ++b) {
        const int n = n_nodes[b];
        const int32_t* par = parents + (size_t)b * budget;
        const int32_t* dep = depths + (size_t)b * budget;
        const float* sc = scores + (size_t)b * budget;
        int32_t* rk = rank + (size_t)b * budget;
        for (int i = 0; i < budget; ++i) rk[i] = -1;
        memset(taken, 0, (size_t)budget);
        /* best-first order over the tree */
        for (int step = 0; step < n; ++step) {
            int best = -1;
            for (int i = 0; i < n; ++i) {
                if (taken[i] || (par[i] >= 0 && !taken[par[i]])) continue;
                if (best < 0 || sc[i] > sc[best] || (sc[i] == sc[best] && dep[i] < dep[best])) best = i;
            }
            taken[best] = 1;
            rk[best] = step;
            order[step] = best;
        }
        /* extend while the expected tokens per unit cost strictly grow */
        double A = 1.0, T = cost_fixed;
        int m = 0;
        while (m < n) {
            const double c = exp((double)sc[order[m]]);
            if (!(c * T > cost_per_token * A)) break;
            A += c;
            T += cost_per_token;
            ++m;
        }
        n_verify[b] = m;
    }
    free(taken);
    free(order);
    return 0;
}
