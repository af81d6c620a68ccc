// Tree construction: one 256-thread workgroup per request, all state in LDS.
//
//  1. Merge the sweep's per-chunk partials of the request's d rows into the
//     log-softmax normaliser (fp64 merge and log) and the exact top-k list
//     T_i of every position (DART, arXiv 2601.19278, Fig. 3: a position's
//     own logit proposes the tokens of its depth).
//  2. Look up N-gram continuity for every context a frontier node can have
//     before the depth loop starts.  A depth-t parent carries a token of
//     T_{t-2} (and, for the trigram, its parent a token of T_{t-3}), so at
//     most 1 + k + (d-2) k^2 trigram contexts (1 + (d-1) k bigram contexts)
//     exist; all lookups are issued in parallel and the result is one
//     admissibility bit per (context, child of T_{t-1}).  In DARTree mode the
//     parent-conditioned terms E[parent].F[child] for every (T_{t-2}, T_{t-1})
//     pair come from fp64 MFMA tiles (DARTree "Tree Construction": all
//     candidates of a depth are scored in one batch).
//  3. Depth loop: candidates = frontier x T_{t-1}, scored with the lse-free
//     key Rk and the cumulative log-score S in fp64; the top-W across the
//     whole frontier by (Rk desc, token asc, parent rank asc) become the next
//     frontier (DARTree: "selects the top-W scored nodes across the entire
//     frontier").  No global memory is touched inside the loop.
//  4. Budget: best-first selection of the verification tree (DARTree
//     abstract).  In DART mode S never increases along a path, so the
//     best-first set equals the top-`budget` nodes by (S desc, BFS index);
//     DARTree mode replays best-first literally.
//  5. Compact in BFS order, remap parents and pack the ancestor mask used by
//     tree-attention verification.
#include "common.h"

namespace dt {
namespace {

typedef double v4d __attribute__((ext_vector_type(4)));
constexpr unsigned long long kEmptyKey = 0xFFFFFFFFFFFFFFFFull;

__device__ __forceinline__ float key_value(unsigned long long key) {
    return __uint_as_float(unord_bits((uint32_t)(key >> 32)));
}
__device__ __forceinline__ uint32_t key_id(unsigned long long key) { return ~(uint32_t)key; }

__device__ __forceinline__ int lanes_below(unsigned long long mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ unsigned long long mix64(unsigned long long z) {
    // SplitMix64 output function (Steele, Lea, Flood).
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const unsigned long long o = __shfl_xor(v, off);
        v = o > v ? o : v;
    }
    return v;
}

// ---------------------------------------------------------------------------
// 1. one wave merges the C partials of one row
// ---------------------------------------------------------------------------
__device__ void merge_row(const float* __restrict__ part_m, const double* __restrict__ part_s,
                          const unsigned long long* __restrict__ part_keys, int64_t row, int C, int k,
                          unsigned long long* scratch, int lane, double* lse_out, int* tok_out,
                          float* val_out) {
    const float* pm = part_m + row * C;
    const double* ps = part_s + row * C;
    float mc = -INFINITY;
    for (int c = lane; c < C; c += 64) mc = fmaxf(mc, pm[c]);
    const float M = wave_max_f(mc);
    double sum = 0.0;
    if (M != -INFINITY)
        for (int c = lane; c < C; c += 64) {
            const float m = pm[c];
            if (m != -INFINITY) sum += ps[c] * exp((double)m - (double)M);
        }
    sum = wave_sum_d(sum);
    if (lane == 0) {
        // the true normaliser is >= the row max; clamp the rounding of a sum
        // whose largest term is 1 so that every log-probability stays <= 0
        double l = log(sum);
        *lse_out = (M == -INFINITY) ? -INFINITY : (double)M + (l > 0.0 ? l : 0.0);
    }

    // top-k: every chunk list is sorted; the k-th key of any full list is a
    // lower bound for the row's k-th key, so only keys >= the largest such
    // bound can be in the row's top-k
    const unsigned long long* keys = part_keys + row * (int64_t)C * k;
    const int n = C * k;
    unsigned long long th = 0ull;
    for (int c = lane; c < C; c += 64) {
        const unsigned long long v = keys[(int64_t)c * k + k - 1];
        th = v > th ? v : th;
    }
    th = wave_max_u64(th);
    int ns = 0;
    for (int base = 0; base < n; base += 64) {
        const int e = base + lane;
        const unsigned long long v = e < n ? keys[e] : 0ull;
        const bool keep = v != 0ull && v >= th;
        const unsigned long long bal = __ballot(keep);
        if (keep) scratch[ns + lanes_below(bal)] = v;
        ns += __popcll(bal);
    }
    __builtin_amdgcn_wave_barrier();
    for (int base = 0; base < ns; base += 64) {
        const int e = base + lane;
        const unsigned long long v = e < ns ? scratch[e] : 0ull;
        int r = 0;
        for (int j = 0; j < ns; ++j) r += scratch[j] > v;
        if (e < ns && r < k) {
            tok_out[r] = (int)key_id(v);
            val_out[r] = key_value(v);
        }
    }
    __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// 2. continuity
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool logp_keeps(const TreeArgs& a, const float* lp, int64_t e) {
    return a.min_logp == -INFINITY || lp == nullptr || lp[e] > a.min_logp;
}

// Bit j set iff child T_{t-1}[j] (finite logit) is admitted after (a2, a1).
__device__ uint32_t admitted_children(const TreeArgs& a, int a2, int a1, const int* ch, const float* cx) {
    const int k = a.k;
    uint32_t live = 0;
    for (int j = 0; j < k; ++j)
        if (cx[j] != -INFINITY) live |= 1u << j;
    if (live == 0) return 0;
    // context ids come from the caller's ctx for the first depths: ids outside
    // [0, V) index no table row and admit nothing
    const bool bigram = a.ng_kind == DT_NGRAM_DENSE_BIGRAM || a.ng_kind == DT_NGRAM_CSR_BIGRAM;
    if (bigram && (a1 < 0 || a1 >= a.V)) return 0;
    uint32_t m = 0;
    if (a.ng_kind == DT_NGRAM_DENSE_BIGRAM) {
        const float* row = a.dense + (int64_t)a1 * a.V;
        for (int j = 0; j < k; ++j)
            if (row[ch[j]] > a.min_logp) m |= 1u << j;
    } else if (a.ng_kind == DT_NGRAM_CSR_BIGRAM) {
        const int lo = a.row_ptr[a1], hi = a.row_ptr[a1 + 1];
        if (hi - lo <= 64) {
            for (int e = lo; e < hi; ++e) {
                const int c = a.col[e];
                for (int j = 0; j < k; ++j)
                    if (ch[j] == c && logp_keeps(a, a.csr_logp, e)) m |= 1u << j;
            }
        } else {
            for (int j = 0; j < k; ++j) {       // rows are ascending: binary search
                int l = lo, h = hi;
                while (l < h) {
                    const int mid = (l + h) >> 1;
                    if (a.col[mid] < ch[j]) l = mid + 1; else h = mid;
                }
                if (l < hi && a.col[l] == ch[j] && logp_keeps(a, a.csr_logp, l)) m |= 1u << j;
            }
        }
    } else if (a.ng_kind == DT_NGRAM_HASH_TRIGRAM) {
        const unsigned long long key = ((unsigned long long)(uint32_t)a2 << 32) | (uint32_t)a1;
        const unsigned long long cm = (unsigned long long)a.cap - 1ull;
        unsigned long long slot = mix64(key) & cm;
        bool found = false;
        for (long long probe = 0; probe < a.cap; ++probe) {
            const unsigned long long here = a.keys[slot];
            if (here == key) { found = true; break; }
            if (here == kEmptyKey) break;
            slot = (slot + 1ull) & cm;
        }
        if (!found) return 0;
        const int* succ = a.succ + (int64_t)slot * a.S;
        for (int s = 0; s < a.S; ++s) {
            const int c = succ[s];
            if (c < 0) continue;
            for (int j = 0; j < k; ++j)
                if (ch[j] == c && logp_keeps(a, a.hash_logp, (int64_t)slot * a.S + s)) m |= 1u << j;
        }
    } else {
        m = live;
    }
    return m & live;
}

// Index of a continuity context.  Depth t's contexts: bigram -> parent token
// (t = 1: the root; t >= 2: T_{t-2}[i1]); trigram -> (grandparent, parent)
// (t = 1: (ctx0, ctx1); t = 2: (ctx1, T_0[i1]); t >= 3: (T_{t-3}[i2], T_{t-2}[i1])).
__device__ __forceinline__ int ctx_index(int kind, int k, int t, int i2, int i1) {
    if (t == 1) return 0;
    if (kind == DT_NGRAM_HASH_TRIGRAM) {
        if (t == 2) return 1 + i1;
        return 1 + k + (t - 3) * k * k + i2 * k + i1;
    }
    return 1 + (t - 2) * k + i1;
}

// ---------------------------------------------------------------------------
// ordering keys
// ---------------------------------------------------------------------------
// frontier: (Rk desc, token asc, parent rank asc); tie = token << 6 | rank
__device__ __forceinline__ bool cand_before(double rk_a, uint32_t tie_a, double rk_b, uint32_t tie_b) {
    return rk_a > rk_b || (rk_a == rk_b && tie_a < tie_b);
}
// budget: (S desc, depth asc, BFS index asc); BFS index order implies depth order
__device__ __forceinline__ bool node_before(double s_a, int i_a, double s_b, int i_b) {
    return s_a > s_b || (s_a == s_b && i_a < i_b);
}

template <typename T>
__device__ __forceinline__ T* lds_at(unsigned char* base, int off) {
    return reinterpret_cast<T*>(base + off);
}

// exclusive prefix sum over the workgroup (one value per thread)
__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) tmp[wave] = x;
    __syncthreads();
    int before = 0, all = 0;
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave) before += tmp[w];
        all += tmp[w];
    }
    __syncthreads();
    *total = all;
    return before + x - v;
}

__global__ void __launch_bounds__(kThreads) tree_kernel(TreeArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const TreePlan& P = a.plan;
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int d = a.d, k = a.k, W = a.W, budget = a.budget;
    const int kind = a.ng_kind;
    const bool dartree = a.mode == DT_MODE_DARTREE;

    double* s_lse = lds_at<double>(lds, P.off_lse);
    int* s_ttok = lds_at<int>(lds, P.off_ttok);
    float* s_tx = lds_at<float>(lds, P.off_tx);
    uint32_t* s_vmask = lds_at<uint32_t>(lds, P.off_vmask);
    double* s_g = lds_at<double>(lds, P.off_g);
    int* n_tok = lds_at<int>(lds, P.off_n_tok);
    int* n_par = lds_at<int>(lds, P.off_n_par);
    int* n_dep = lds_at<int>(lds, P.off_n_dep);
    int* n_tidx = lds_at<int>(lds, P.off_n_tidx);
    int* n_cctx = lds_at<int>(lds, P.off_n_cctx);
    int* n_new = lds_at<int>(lds, P.off_n_new);
    int* n_out = lds_at<int>(lds, P.off_n_out);
    double* n_rk = lds_at<double>(lds, P.off_n_rk);
    double* n_s = lds_at<double>(lds, P.off_n_s);
    double* c_rk = lds_at<double>(lds, P.off_c_rk);
    double* c_s = lds_at<double>(lds, P.off_c_s);
    uint32_t* c_tie = lds_at<uint32_t>(lds, P.off_c_tie);
    int* c_surv = lds_at<int>(lds, P.off_c_surv);
    double* rowmax = lds_at<double>(lds, P.off_rowmax);
    int* misc = lds_at<int>(lds, P.off_misc);
    unsigned long long* merge = lds_at<unsigned long long>(lds, P.off_merge) + wave * kMergeKeysPerRow;

    const int ctx0 = a.ctx[2 * b], ctx1 = a.ctx[2 * b + 1];

    // ---- 1. normalisers and top-k lists of the d positions
    for (int i = wave; i < d; i += kWaves)
        merge_row(a.part_m, a.part_s, a.part_keys, (int64_t)b * d + i, a.C, k, merge, lane,
                  &s_lse[i], &s_ttok[i * k], &s_tx[i * k]);
    __syncthreads();

    // ---- 2a. continuity of every context a parent can have
    for (int ci = tid; ci < P.n_ctx; ci += kThreads) {
        int t, a2, a1;
        if (ci == 0) {
            t = 1; a2 = ctx0; a1 = ctx1;
        } else if (kind == DT_NGRAM_HASH_TRIGRAM) {
            if (ci < 1 + k) {
                t = 2; a2 = ctx1; a1 = s_ttok[ci - 1];
            } else {
                int r = ci - 1 - k;
                t = 3 + r / (k * k);
                r -= (t - 3) * k * k;
                a2 = s_ttok[(t - 3) * k + r / k];
                a1 = s_ttok[(t - 2) * k + r % k];
            }
        } else {
            t = 2 + (ci - 1) / k;
            a2 = 0;
            a1 = s_ttok[(t - 2) * k + (ci - 1) % k];
        }
        s_vmask[ci] = admitted_children(a, a2, a1, s_ttok + (t - 1) * k, s_tx + (t - 1) * k);
    }

    // ---- 2b. DARTree parent-conditioned terms G_t[i][j] = E[par_i] . F[T_{t-1}[j]]
    //          with par = root token (t = 1) or T_{t-2}; fp64 MFMA 16x16x4 tiles
    if (dartree) {
        const int tk = (k + 15) >> 4;
        const int tiles = d * tk * tk;
        for (int tile = wave; tile < tiles; tile += kWaves) {
            const int t = 1 + tile / (tk * tk);
            const int r = tile - (t - 1) * tk * tk;
            const int ti = r / tk, tj = r - ti * tk;
            const int kp = t == 1 ? 1 : k;
            if (ti * 16 >= kp) continue;                      // wave-uniform
            const int i = ti * 16 + (lane & 15), j = tj * 16 + (lane & 15), kk = lane >> 4;
            int ptok = i < kp ? (t == 1 ? ctx1 : s_ttok[(t - 2) * k + i]) : -1;
            if (ptok >= a.V) ptok = -1;                           // out-of-range root id: no term
            const int ctok = j < k ? s_ttok[(t - 1) * k + j] : -1;
            const float* er = ptok >= 0 ? a.E + (int64_t)ptok * a.R : nullptr;
            const float* fr = ctok >= 0 ? a.F + (int64_t)ctok * a.R : nullptr;
            v4d acc = {0.0, 0.0, 0.0, 0.0};
            for (int s = 0; s < a.R; s += 4) {
                const double av = er ? (double)er[s + kk] : 0.0;   // A[i][kk]
                const double bv = fr ? (double)fr[s + kk] : 0.0;   // B[kk][j]
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {                          // D[lane/16 + 4q][lane%16]
                const int ii = ti * 16 + (lane >> 4) + 4 * q, jj = tj * 16 + (lane & 15);
                if (ii < kp && jj < k) s_g[((t - 1) * k + ii) * k + jj] = acc[q];
            }
        }
    }
    if (tid < 4) misc[tid] = 0;
    __syncthreads();

    // ---- 3. depth loop
    int f = 1;        // frontier size (depth 0: the root)
    int fbase = 0;    // BFS index of the first frontier node
    int nb = 0;       // nodes in the candidate tree
    for (int t = 1; t <= d; ++t) {
        int* cnt = &misc[t & 1];
        const int m = f * k;                 // candidate slots, slot = p * k + j
        const double lse_t = s_lse[t - 1];
        int mine = 0;
        for (int ci = tid; ci < m; ci += kThreads) {
            const int p = ci / k, j = ci - p * k;
            const float x = s_tx[(t - 1) * k + j];
            bool ok = x != -INFINITY;
            double prk = 0.0, ps = 0.0;
            int cidx = 0, gp = 0;
            if (t > 1) {
                const int nd = fbase + p;
                prk = n_rk[nd];
                ps = n_s[nd];
                cidx = n_cctx[nd];
                gp = n_tidx[nd];
            }
            if (ok && kind != DT_NGRAM_NONE) ok = (s_vmask[cidx] >> j) & 1u;
            double rk = -INFINITY, sc = -INFINITY;
            if (ok) {
                const double g = dartree ? s_g[((t - 1) * k + gp) * k + j] : 0.0;
                rk = (prk + (double)x) + g;
                sc = (ps + ((double)x - lse_t)) + g;
                ++mine;
            }
            c_rk[ci] = rk;
            c_s[ci] = sc;
            c_tie[ci] = ((uint32_t)s_ttok[(t - 1) * k + j] << 6) | (uint32_t)p;
        }
        if (mine) atomicAdd(cnt, mine);
        if (tid == 0) {
            misc[(t + 1) & 1] = 0;
            misc[2] = 0;
        }
        __syncthreads();
        const int n = *(volatile int*)cnt;
        if (n == 0) break;
        const int keep = n < W ? n : W;

        // candidates to rank: all slots, or, when the frontier is full and the
        // slots are many, only those whose key reaches the smallest row maximum
        // (the W row maxima are W candidates at or above it)
        const bool filter = f == W && m > 128;
        int ns = m;
        if (filter) {
            for (int p = tid; p < f; p += kThreads) {
                double best = -INFINITY;
                for (int j = 0; j < k; ++j) best = fmax(best, c_rk[p * k + j]);
                rowmax[p] = best;
            }
            __syncthreads();
            double lb = INFINITY;
            for (int p = 0; p < f; ++p) lb = fmin(lb, rowmax[p]);
            for (int ci = tid; ci < m; ci += kThreads) {
                const bool in = c_rk[ci] != -INFINITY && c_rk[ci] >= lb;
                const unsigned long long bal = __ballot(in);
                int base = 0;
                if (lane == 0 && bal) base = atomicAdd(&misc[2], __popcll(bal));
                base = __shfl(base, 0);
                if (in) c_surv[base + lanes_below(bal)] = ci;
            }
            __syncthreads();
            ns = *(volatile int*)&misc[2];
        }

        // rank by counting; tpc threads share one candidate's comparisons
        int tpc = 1;
        while (tpc < 8 && 2 * tpc * ns <= kThreads) tpc <<= 1;
        for (int base = 0; base < ns * tpc; base += kThreads) {
            const int e = base + tid;
            const int c = e / tpc, part = e - c * tpc;
            int r = 0;
            int slot = -1;
            bool live = false;
            if (c < ns) {
                slot = filter ? c_surv[c] : c;
                const double my = c_rk[slot];
                const uint32_t mt = c_tie[slot];
                live = my != -INFINITY;
                if (live) {
                    for (int q = part; q < ns; q += tpc) {
                        const int o = filter ? c_surv[q] : q;
                        r += cand_before(c_rk[o], c_tie[o], my, mt);
                    }
                }
            }
            for (int off = 1; off < tpc; off <<= 1) r += __shfl_xor(r, off);
            if (live && part == 0 && r < keep) {
                const int p = slot / k, j = slot - p * k;
                const int nd = nb + r;
                n_tok[nd] = s_ttok[(t - 1) * k + j];
                n_par[nd] = t == 1 ? -1 : fbase + p;
                n_dep[nd] = t;
                n_tidx[nd] = j;
                const int pj = t == 1 ? 0 : n_tidx[fbase + p];
                n_cctx[nd] = t < d ? ctx_index(kind, k, t + 1, pj, j) : 0;
                n_rk[nd] = c_rk[slot];
                n_s[nd] = c_s[slot];
            }
        }
        __syncthreads();
        fbase = nb;
        nb += keep;
        f = keep;
    }

    // ---- 4. verification budget
    int n_sel = nb;
    if (nb <= budget) {
        for (int i = tid; i < nb; i += kThreads) {
            n_new[i] = i;
            n_out[i] = i;
        }
        __syncthreads();
    } else if (!dartree) {
        // parent-closed top-budget by (S desc, BFS index asc)
        const int per = (nb + kThreads - 1) / kThreads;
        int flags = 0, cntl = 0;
        for (int q = 0; q < per; ++q) {
            const int i = tid * per + q;
            if (i < nb) {
                int r = 0;
                const double si = n_s[i];
                for (int j = 0; j < nb; ++j) r += node_before(n_s[j], j, si, i);
                if (r < budget) {
                    flags |= 1 << q;
                    ++cntl;
                }
            }
        }
        int total;
        int pos = block_exclusive_scan(cntl, misc + 4, &total);
        for (int q = 0; q < per; ++q) {
            const int i = tid * per + q;
            if (i < nb) {
                if (flags >> q & 1) {
                    n_new[i] = pos;
                    n_out[pos] = i;
                    ++pos;
                } else {
                    n_new[i] = -1;
                }
            }
        }
        n_sel = total;
        __syncthreads();
    } else {
        // best-first, literally: take the best available node budget times
        for (int i = tid; i < nb; i += kThreads) n_new[i] = (n_par[i] < 0) ? -2 : -3;  // -2 available, -3 waiting
        __syncthreads();
        if (wave == 0) {
            for (int step = 0; step < budget; ++step) {
                double bs = -INFINITY;
                int bi = -1;
                for (int i = lane; i < nb; i += 64)
                    if (n_new[i] == -2 && (bi < 0 || node_before(n_s[i], i, bs, bi))) {
                        bs = n_s[i];
                        bi = i;
                    }
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) {
                    const double os = __shfl_xor(bs, off);
                    const int oi = __shfl_xor(bi, off);
                    if (oi >= 0 && (bi < 0 || node_before(os, oi, bs, bi))) {
                        bs = os;
                        bi = oi;
                    }
                }
                if (bi < 0) break;                                // cannot happen: nb > budget
                __builtin_amdgcn_wave_barrier();
                if (lane == 0) n_new[bi] = -1;                    // taken (index assigned below)
                __builtin_amdgcn_wave_barrier();
                for (int i = lane; i < nb; i += 64)
                    if (n_par[i] == bi) n_new[i] = -2;
                __builtin_amdgcn_wave_barrier();
            }
        }
        __syncthreads();
        // taken nodes keep BFS order
        const int per = (nb + kThreads - 1) / kThreads;
        int cntl = 0;
        for (int q = 0; q < per; ++q) {
            const int i = tid * per + q;
            if (i < nb && n_new[i] == -1) ++cntl;
        }
        int total;
        int pos = block_exclusive_scan(cntl, misc + 4, &total);
        __syncthreads();
        for (int q = 0; q < per; ++q) {
            const int i = tid * per + q;
            if (i < nb) {
                if (n_new[i] == -1) {
                    n_new[i] = pos;
                    n_out[pos] = i;
                    ++pos;
                } else {
                    n_new[i] = -1;
                }
            }
        }
        n_sel = total;
        __syncthreads();
    }

    // ---- 5. outputs in BFS order, parents remapped, ancestor mask
    const int64_t ob = (int64_t)b * budget;
    for (int o = tid; o < budget; o += kThreads) {
        if (o < n_sel) {
            const int i = n_out[o];
            a.tokens[ob + o] = n_tok[i];
            a.parents[ob + o] = n_par[i] < 0 ? -1 : n_new[n_par[i]];
            a.depths[ob + o] = n_dep[i];
            a.scores[ob + o] = (float)n_s[i];
        } else {
            a.tokens[ob + o] = -1;
            a.parents[ob + o] = -1;
            a.depths[ob + o] = 0;
            a.scores[ob + o] = -INFINITY;
        }
    }
    const int words = a.mask_words;
    for (int e = tid; e < budget * words; e += kThreads) {
        const int o = e / words, w = e - o * words;
        uint32_t bits = 0;
        if (o < n_sel) {
            for (int i = n_out[o]; i >= 0; i = n_par[i]) {
                const int ni = n_new[i];
                if ((ni >> 5) == w) bits |= 1u << (ni & 31);
            }
        }
        a.mask[ob * words + e] = bits;
    }
    if (tid == 0) a.n_nodes[b] = n_sel;
}

// one wave per row: per-position normaliser and top-k only
__global__ void __launch_bounds__(kThreads) merge_kernel(MergeArgs a) {
    __shared__ unsigned long long scratch[kWaves][kMergeKeysPerRow];
    __shared__ int s_tok[kWaves][kMaxK];
    __shared__ float s_val[kWaves][kMaxK];
    __shared__ double s_lse[kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
    if (row >= a.rows) return;                                  // wave-uniform; no block barrier below
    merge_row(a.part_m, a.part_s, a.part_keys, row, a.C, a.k, scratch[wave], lane, &s_lse[wave],
              s_tok[wave], s_val[wave]);
    if (lane < a.k) {
        a.tok[row * a.k + lane] = s_tok[wave][lane];
        a.val[row * a.k + lane] = s_val[wave][lane];
    }
    if (lane == 0) a.lse[row] = s_lse[wave];
}

}  // namespace

hipError_t launch_tree(const TreeArgs& a, hipStream_t stream) {
    if (a.B <= 0) return hipSuccess;
    hipLaunchKernelGGL(tree_kernel, dim3((unsigned)a.B), dim3(kThreads), (size_t)a.plan.total, stream, a);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((a.rows + kWaves - 1) / kWaves);
    hipLaunchKernelGGL(merge_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dt
