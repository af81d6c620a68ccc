// Tree construction: two kernels after the vocabulary sweep.
//
// prep_kernel -- one 256-thread workgroup per (request, depth t) [and slice
// of that depth's contexts], so the latency-bound random reads of the N-gram
// table and of E/F are spread over many compute units instead of queueing in
// one:
//  1. Up to three waves merge the sweep's per-chunk partials of rows t-1 (the
//     children of depth t), t-2 and t-3 (the tokens a depth-t parent and its
//     own parent carry) into the log-softmax normaliser (fp64 merge and log)
//     and the exact top-k list T_i of each row (DART, arXiv 2601.19278,
//     Fig. 3: a position's own logit proposes the tokens of its depth).  Row
//     t-1 is written out for the tree kernel.
//  2. N-gram continuity of every context a depth-t parent can have: a
//     depth-t parent carries a token of T_{t-2} (and, for the trigram, its
//     parent a token of T_{t-3}), so depth t has 1, k or k^2 contexts; each
//     thread looks one up and stores one admissibility bit per child of
//     T_{t-1}.
//  3. DARTree: the parent-conditioned terms E[parent].F[child] of depth t
//     for every (T_{t-2}, T_{t-1}) pair from fp64 MFMA tiles (DARTree "Tree
//     Construction": all candidates of a depth are scored in one batch).
//
// tree_kernel -- one 256-thread workgroup per request, all state in LDS:
//  4. Depth loop: candidates = frontier x T_{t-1}, scored with the lse-free
//     key Rk and the cumulative log-score S in fp64; the top-W across the
//     whole frontier by (Rk desc, token asc, parent rank asc) become the next
//     frontier (DARTree: "selects the top-W scored nodes across the entire
//     frontier").  Keys live in registers, ranks come from one wave, and no
//     global memory is touched inside the loop.
//  5. Budget: best-first selection of the verification tree (DARTree
//     abstract).  In DART mode S never increases along a path, so the
//     best-first set equals the top-`budget` nodes by (S desc, BFS index);
//     DARTree mode replays best-first literally.
//  6. Compact in BFS order, remap parents and pack the ancestor mask used by
//     tree-attention verification.
#include "tree_dev.h"

namespace dt {
namespace {
using namespace treedev;

// ---------------------------------------------------------------------------
// prep: rows, continuity and parent-conditioned terms of one depth
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) prep_kernel(PrepArgs a) {
    // latency-bound work: with another call's sweep on the same compute
    // unit, its waves go first when both are ready to issue
    __builtin_amdgcn_s_setprio(3);
    __shared__ unsigned long long s_scratch[kPrepRows][kMergeKeysPerRow + 8];
    __shared__ int s_tok[kPrepRows][kMaxK];
    __shared__ float s_x[kPrepRows][kMaxK];
    __shared__ double s_lse[kPrepRows];
    __shared__ int s_ctok[kChildSlots];
    __shared__ int s_cj[kChildSlots];
    // (the sweep's turn-taking test counts on this bound)
    static_assert(sizeof(s_scratch) + sizeof(s_tok) + sizeof(s_x) + sizeof(s_lse) + sizeof(s_ctok) +
                      sizeof(s_cj) <= kPrepLds, "prep LDS above kPrepLds");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int d = a.d, k = a.k;
    const int split = blockIdx.x % a.nsplit;
    const int bt = blockIdx.x / a.nsplit;
    const int b = bt / d, t = bt - b * d + 1;                  // depth t = 1..d
    const int kind = a.ng.kind;
    const bool dartree = a.mode == DT_MODE_DARTREE;
    const bool trigram = kind == DT_NGRAM_HASH_TRIGRAM;
    const int ctx0 = a.ctx[2 * b], ctx1 = a.ctx[2 * b + 1];

    // ---- 1. wave w merges row t-1-w: the children (w = 0), the parents'
    //         tokens (w = 1) and, for the trigram, the grandparents' (w = 2)
    const int rows = 1 + ((t >= 2 && (kind != DT_NGRAM_NONE || dartree)) ? 1 : 0) + ((t >= 3 && trigram) ? 1 : 0);
    if (wave < rows) {
        const int64_t row = (int64_t)b * d + (t - 1 - wave);
        merge_row(a.part_m, a.part_s, a.part_keys, row, a.L, k, s_scratch[wave], lane, &s_lse[wave],
                  s_tok[wave], s_x[wave]);
        if (wave == 0 && split == 0) {                       // row t-1 is written once
            if (lane < k) {
                a.ttok[row * k + lane] = s_tok[0][lane];
                a.tx[row * k + lane] = s_x[0][lane];
            }
            if (lane == 0) a.lse[row] = s_lse[0];
        }
    }
    __syncthreads();

    // ---- 2. continuity of depth t's contexts against the children T_{t-1}
    if (kind != DT_NGRAM_NONE) {
        int n_t, base;                                       // contexts of depth t, index of the first
        if (t == 1) {
            n_t = 1;
            base = 0;
        } else if (trigram) {
            n_t = t == 2 ? k : k * k;
            base = t == 2 ? 1 : 1 + k + (t - 3) * k * k;
        } else {
            n_t = k;
            base = 1 + (t - 2) * k;
        }
        const int per = (n_t + a.nsplit - 1) / a.nsplit;
        const int lo = split * per, hi = lo + per < n_t ? lo + per : n_t;
        // children of depth t by token (the trigram and CSR rows list
        // successors by token), then one lane quad per context
        if (kind != DT_NGRAM_DENSE_BIGRAM) {
            for (int i = tid; i < kChildSlots; i += kThreads) s_ctok[i] = -1;
            __syncthreads();
            if (tid < k) {
                const int tok = s_tok[0][tid];
                uint32_t pos = child_hash(tok);
                while (true) {                               // <= 32 keys in 128 slots
                    if (atomicCAS(&s_ctok[pos], -1, tok) == -1) {
                        s_cj[pos] = tid;
                        break;
                    }
                    pos = (pos + 1) & (kChildSlots - 1);
                }
            }
            __syncthreads();
        }
        uint32_t live = 0;
        for (int j = 0; j < k; ++j) live |= (uint32_t)(s_x[0][j] != -INFINITY) << j;
        const int g = tid & 3;
        for (int c0 = lo; c0 < hi; c0 += kThreads / 4) {
            const int c = c0 + (tid >> 2);
            const bool active = c < hi;
            uint32_t m;
            if (trigram) {
                int a2 = 0, a1 = 0;
                if (active) {
                    if (t == 1) {
                        a2 = ctx0;
                        a1 = ctx1;
                    } else {
                        a2 = t == 2 ? ctx1 : s_tok[2][c / k];
                        a1 = t == 2 ? s_tok[1][c] : s_tok[1][c % k];
                    }
                }
                m = quad_admitted(a.ng, a2, a1, active, g, s_ctok, s_cj, live);
            } else {
                const int a1 = !active ? 0 : (t == 1 ? ctx1 : s_tok[1][c]);
                m = quad_admitted_bigram(a.ng, a1, active, g, s_tok[0], s_ctok, s_cj, live, k);
            }
            if (active && g == 0) a.vmask[(int64_t)b * a.n_ctx + base + c] = m;
        }
    }

    // ---- 3. DARTree: G_t[i][j] = E[par_i] . F[T_{t-1}[j]], par = root token
    //         (t = 1) or T_{t-2}; fp64 MFMA 16x16x4 tiles, one per wave
    if (dartree && split == 0) {
        const int tk = (k + 15) >> 4;
        const int kp = t == 1 ? 1 : k;
        const int tiles = ((kp + 15) >> 4) * tk;
        for (int tile = wave; tile < tiles; tile += kThreads / 64) {
            const int ti = tile / tk, tj = tile - ti * tk;
            const int i = ti * 16 + (lane & 15), j = tj * 16 + (lane & 15), grp = lane >> 4;
            int ptok = i < kp ? (t == 1 ? ctx1 : s_tok[1][i]) : -1;
            if (ptok >= a.ng.V) ptok = -1;                         // out-of-range root id: no term
            const int ctok = j < k ? s_tok[0][j] : -1;
            const float* er = ptok >= 0 ? a.E + (int64_t)ptok * a.R : nullptr;
            const float* fr = ctok >= 0 ? a.F + (int64_t)ctok * a.R : nullptr;
            // The dot product is a sum over the rank index; step q of a block of
            // 4*per columns takes column grp*per + q from lane group grp, so each
            // lane reads `per` contiguous floats of its row (16-byte loads).
            v4d acc = {0.0, 0.0, 0.0, 0.0};
            for (int r0 = 0; r0 < a.R; r0 += 64) {
                const int per = (a.R - r0 < 64 ? a.R - r0 : 64) >> 2;
                float ea[16], fb[16];
                if (per == 16) {
                    typedef float f4 __attribute__((ext_vector_type(4)));
                    const f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const f4 x = er ? reinterpret_cast<const f4*>(er + r0 + grp * 16)[v] : z;
                        const f4 y = fr ? reinterpret_cast<const f4*>(fr + r0 + grp * 16)[v] : z;
                        ea[4 * v] = x.x; ea[4 * v + 1] = x.y; ea[4 * v + 2] = x.z; ea[4 * v + 3] = x.w;
                        fb[4 * v] = y.x; fb[4 * v + 1] = y.y; fb[4 * v + 2] = y.z; fb[4 * v + 3] = y.w;
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        ea[q] = (er && q < per) ? er[r0 + grp * per + q] : 0.f;
                        fb[q] = (fr && q < per) ? fr[r0 + grp * per + q] : 0.f;
                    }
                }
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (q < per) acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)ea[q], (double)fb[q], acc, 0, 0, 0);
            }
            double* gt = a.g + ((int64_t)b * d + (t - 1)) * k * k;
#pragma unroll
            for (int q = 0; q < 4; ++q) {                          // D[lane/16 + 4q][lane%16]
                const int ii = ti * 16 + (lane >> 4) + 4 * q, jj = tj * 16 + (lane & 15);
                if (ii < kp && jj < k) gt[ii * k + jj] = acc[q];
            }
        }
    }
}

template <int RM, bool DTREE, bool NG>
__global__ void __launch_bounds__(kTreeThreads) tree_kernel(TreeArgs a) {
    // latency-bound work: with another call's sweep on the same compute
    // unit, its waves go first when both are ready to issue
    __builtin_amdgcn_s_setprio(3);
    extern __shared__ __align__(16) unsigned char lds[];
    const TreePlan& P = a.plan;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int d = a.d, k = a.k, W = a.W, budget = a.budget;
    const int kind = a.ng_kind;
    constexpr bool dartree = DTREE;

    double* s_lse = lds_at<double>(lds, P.off_lse);
    int* s_ttok = lds_at<int>(lds, P.off_ttok);
    float* s_tx = lds_at<float>(lds, P.off_tx);
    uint32_t* s_vmask = lds_at<uint32_t>(lds, P.off_vmask);
    double* s_g = lds_at<double>(lds, P.off_g);
    int* n_tok = lds_at<int>(lds, P.off_n_tok);
    int* n_par = lds_at<int>(lds, P.off_n_par);
    int* n_dep = lds_at<int>(lds, P.off_n_dep);
    int* n_new = lds_at<int>(lds, P.off_n_new);
    int* n_out = lds_at<int>(lds, P.off_n_out);
    double* n_s = lds_at<double>(lds, P.off_n_s);
    int* misc = lds_at<int>(lds, P.off_misc);
    // ---- load what the prep kernel derived for this request (contiguous)
    {
        const int64_t r0 = (int64_t)b * d;
        const int dk = d * k, nc = P.n_ctx;
        // The first round of every array (up to four entries per thread:
        // all of them at the usual sizes) is loaded before anything is
        // stored, so the loads share one memory round trip; the indices are
        // clamped so that every load is issued unconditionally.
        constexpr int U4 = 4;
        const double l_lse = a.lse[r0 + (tid < d ? tid : 0)];
        int l_tok[U4];
        float l_tx[U4];
        uint32_t l_vm[U4];
#pragma unroll
        for (int u = 0; u < U4; ++u) {
            const int i = tid + u * kTreeThreads, ic = i < dk ? i : 0;
            l_tok[u] = a.ttok[r0 * k + ic];
            l_tx[u] = a.tx[r0 * k + ic];
        }
        if (nc > 0) {
#pragma unroll
            for (int u = 0; u < U4; ++u) {
                const int i = tid + u * kTreeThreads, ic = i < nc ? i : 0;
                l_vm[u] = a.vmask[(int64_t)b * a.n_ctx + ic];
            }
        }
        typedef double d2 __attribute__((ext_vector_type(2)));
        const double* gsrc = a.g + r0 * k * k;
        const int ng = dartree ? d * k * k : 0;
        const bool gvec = (((uintptr_t)gsrc | (uintptr_t)s_g) & 15u) == 0 && (ng & 1) == 0;
        const int nv = ng >> 1;
        constexpr int UG = 8;
        d2 l_g[UG];
        if (dartree && gvec) {
            const d2* src = reinterpret_cast<const d2*>(gsrc);
#pragma unroll
            for (int u = 0; u < UG; ++u) {
                const int i = tid + u * kTreeThreads;
                l_g[u] = src[i < nv ? i : 0];
            }
        }
        if (tid < d) s_lse[tid] = l_lse;
#pragma unroll
        for (int u = 0; u < U4; ++u) {
            const int i = tid + u * kTreeThreads;
            if (i < dk) {
                s_ttok[i] = l_tok[u];
                s_tx[i] = l_tx[u];
            }
        }
        if (nc > 0) {
#pragma unroll
            for (int u = 0; u < U4; ++u) {
                const int i = tid + u * kTreeThreads;
                if (i < nc) s_vmask[i] = l_vm[u];
            }
        }
        // the rest, rarely any (d < 256 always)
        for (int i = tid + U4 * kTreeThreads; i < dk; i += kTreeThreads) {
            s_ttok[i] = a.ttok[r0 * k + i];
            s_tx[i] = a.tx[r0 * k + i];
        }
        for (int i = tid + U4 * kTreeThreads; i < nc; i += kTreeThreads) s_vmask[i] = a.vmask[(int64_t)b * a.n_ctx + i];
        if (dartree) {
            if (gvec) {
                const d2* src = reinterpret_cast<const d2*>(gsrc);
                d2* dst = reinterpret_cast<d2*>(s_g);
#pragma unroll
                for (int u = 0; u < UG; ++u) {
                    const int i = tid + u * kTreeThreads;
                    if (i < nv) dst[i] = l_g[u];
                }
                for (int base = UG * kTreeThreads; base < nv; base += 4 * kTreeThreads) {
                    d2 v0, v1, v2, v3;
                    const int i0 = base + tid, i1 = i0 + kTreeThreads, i2 = i1 + kTreeThreads, i3 = i2 + kTreeThreads;
                    if (i0 < nv) v0 = src[i0];
                    if (i1 < nv) v1 = src[i1];
                    if (i2 < nv) v2 = src[i2];
                    if (i3 < nv) v3 = src[i3];
                    if (i0 < nv) dst[i0] = v0;
                    if (i1 < nv) dst[i1] = v1;
                    if (i2 < nv) dst[i2] = v2;
                    if (i3 < nv) dst[i3] = v3;
                }
            } else {
                for (int i = tid; i < ng; i += kTreeThreads) s_g[i] = gsrc[i];
            }
        }
    }
    __syncthreads();

    const int nb = depth_loop<RM, DTREE, NG>(P, lds, d, k, W, kind == DT_NGRAM_HASH_TRIGRAM);
    budget_and_emit(nb, dartree, b, n_tok, n_par, n_dep, n_s, n_new, n_out, misc,
                    EmitOut{a.n_nodes, a.tokens, a.parents, a.depths, a.scores, a.mask, budget, a.mask_words});
}

// Full-vocabulary DARTree mode: the candidate tree the frontier kernels built
// (workspace, BFS order) goes through the same budget and output stages.
__global__ void __launch_bounds__(kTreeThreads) finish_kernel(FinishArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int nmax = a.d * a.W;
    double* n_s = reinterpret_cast<double*>(lds);
    int* n_tok = reinterpret_cast<int*>(n_s + nmax);
    int* n_par = n_tok + nmax;
    int* n_dep = n_par + nmax;
    int* n_new = n_dep + nmax;
    int* n_out = n_new + nmax;
    int* misc = n_out + nmax;
    const int nb = a.n_tree[b];
    const int64_t src = (int64_t)b * nmax;
    for (int i = tid; i < nb; i += kTreeThreads) {
        n_s[i] = a.nd_s[src + i];
        n_tok[i] = a.nd_tok[src + i];
        n_par[i] = a.nd_par[src + i];
        n_dep[i] = a.nd_dep[src + i];
    }
    __syncthreads();
    budget_and_emit(nb, true, b, n_tok, n_par, n_dep, n_s, n_new, n_out, misc,
                    EmitOut{a.n_nodes, a.tokens, a.parents, a.depths, a.scores, a.mask, a.budget, a.mask_words});
}

// one wave per row: per-position normaliser and top-k only
__global__ void __launch_bounds__(kThreads) merge_kernel(MergeArgs a) {
    __shared__ unsigned long long scratch[kWaves][kMergeKeysPerRow + 8];
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

hipError_t launch_prep(const PrepArgs& a, hipStream_t stream) {
    if (a.B <= 0) return hipSuccess;
    const int64_t grid = (int64_t)a.B * a.d * a.nsplit;
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <int RM>
static void launch_tree_rm(const TreeArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.B), block(kTreeThreads);
    const size_t lds = (size_t)a.plan.total;
    const bool dtree = a.mode == DT_MODE_DARTREE, ng = a.ng_kind != DT_NGRAM_NONE;
    if (dtree && ng)
        hipLaunchKernelGGL((tree_kernel<RM, true, true>), grid, block, lds, stream, a);
    else if (dtree)
        hipLaunchKernelGGL((tree_kernel<RM, true, false>), grid, block, lds, stream, a);
    else if (ng)
        hipLaunchKernelGGL((tree_kernel<RM, false, true>), grid, block, lds, stream, a);
    else
        hipLaunchKernelGGL((tree_kernel<RM, false, false>), grid, block, lds, stream, a);
}

hipError_t launch_tree(const TreeArgs& a, hipStream_t stream) {
    if (a.B <= 0) return hipSuccess;
    const int m = a.W * a.k;
    if (m <= 128)
        launch_tree_rm<2>(a, stream);
    else if (m <= 256)
        launch_tree_rm<4>(a, stream);
    else
        launch_tree_rm<16>(a, stream);
    return hipGetLastError();
}

static size_t finish_lds_bytes(int d, int W) { return (size_t)d * W * (8 + 5 * 4) + kMiscInts * 4; }

hipError_t launch_finish(const FinishArgs& a, hipStream_t stream) {
    if (a.B <= 0) return hipSuccess;
    hipLaunchKernelGGL(finish_kernel, dim3((unsigned)a.B), dim3(kTreeThreads), finish_lds_bytes(a.d, a.W), stream, a);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((a.rows + kWaves - 1) / kWaves);
    hipLaunchKernelGGL(merge_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dt
