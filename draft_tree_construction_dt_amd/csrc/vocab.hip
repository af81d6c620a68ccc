// Full-vocabulary DARTree mode (DARTree page, "Tree Construction": at every
// depth the drafter proposes W candidate tokens for each frontier node, all
// candidates are scored with the path-conditioned head in one batch, and the
// top-W across the whole frontier survive).  Here a node's proposals come
// from its own parent-conditioned distribution over the whole vocabulary,
// x[v] + E[tok_p] . F[v], and its W proposals are its W best tokens under the
// candidate order.  Since no parent places more than W candidates in the
// frontier's top-W, the frontier is also the top-W of ALL (node, token)
// pairs by
//     Rk(p, v) = (Rk_p + x[v]) + g(p, v),   g(p, v) = E[tok_p] . F[v]
// (ties: token asc, parent rank asc), which is what these kernels compute.
//
// Per depth t, two kernels:
//  vocab_kernel    - one workgroup per (vocabulary chunk, group of 8 requests),
//                    a wave per 2 requests.  The dense part, G = E_frontier .
//                    F_chunk^T for 16 frontier rows x 16 tokens per step, runs
//                    on fp32 MFMA (v_mfma_f32_16x16x4f32).  fp32 decides
//                    nothing: every candidate carries an interval around its
//                    fp64 key, ak +- e with e = 2^-17 |E_p| |F_v| + |ak| 2^-44
//                    (a product meets at most 1 + 3 + R/4 <= 20 roundings of
//                    2^-24 on its way into an MFMA output, and
//                    sum |E_k F_k| <= |E_p| |F_v|), so a candidate is
//                    dropped only when its upper end is below the W-th largest
//                    lower end seen.  What survives is rescored exactly, in
//                    fp64 summed k = 0..R-1 (fp32 x fp32 products are exact in
//                    fp64, so the sum is the oracle's bit for bit), and the
//                    chunk's exact top-W is written out.
//  frontier_kernel - one workgroup per request: merges the chunks' sorted
//                    lists (the largest W-th entry of any list bounds the
//                    frontier's W-th key from below, so only entries above it
//                    are ranked), appends the new nodes with their cumulative
//                    log-scores S = (S_p + (x - lse)) + g, and makes them the
//                    next frontier.
// The budget and the outputs are then the tree kernel's (finish_kernel).
#include "common.h"

namespace dt {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned long long ord64(double x) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(x);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ double unord64(unsigned long long o) {
    const unsigned long long u = (o >> 63) ? (o & 0x7FFFFFFFFFFFFFFFull) : ~o;
    return __longlong_as_double((long long)u);
}

template <int DT>
__device__ __forceinline__ float load_logit(const void* base, int64_t i) {
    if (DT == DT_DTYPE_BF16) return __uint_as_float((uint32_t)((const uint16_t*)base)[i] << 16);
    return ((const float*)base)[i];
}

__device__ __forceinline__ double shfl_d(double v, int src) {
    const long long u = __double_as_longlong(v);
    const int lo = __shfl((int)(u & 0xFFFFFFFFll), src), hi = __shfl((int)(u >> 32), src);
    return __longlong_as_double(((long long)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ int lanes_below(unsigned long long m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// the kth largest of the wave's 4 x 64 keys (key 0 = no candidate): the
// largest T with at least kth keys >= T, found bit by bit from the top
__device__ unsigned long long wave_kth_key(const unsigned long long (&key)[4], int kth) {
    unsigned long long T = 0;
    for (int bit = 63; bit >= 0; --bit) {
        const unsigned long long c = T | (1ull << bit);
        int n = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) n += __popcll(__ballot(key[i] >= c));
        if (n >= kth) T = c;
    }
    return T;
}

// exact key of one candidate, summed like the oracle: k = 0 .. R-1
__device__ __forceinline__ double exact_g(const float* __restrict__ E, const float* __restrict__ F, int R,
                                          int tok, int v) {
    const float4* e4 = reinterpret_cast<const float4*>(E + (int64_t)tok * R);
    const float4* f4 = reinterpret_cast<const float4*>(F + (int64_t)v * R);
    double g = 0.0;
    for (int q = 0; q < (R >> 2); ++q) {
        const float4 e = e4[q], f = f4[q];
        g += (double)e.x * (double)f.x;
        g += (double)e.y * (double)f.y;
        g += (double)e.z * (double)f.z;
        g += (double)e.w * (double)f.w;
    }
    return g;
}

constexpr int kOwn = (kVocabCap + 63) / 64;                  // buffer entries per lane

struct VocabLds {
    double ak[kVocabReqPerGroup][kVocabCap];   // key estimate (exact once rescored)
    float e[kVocabReqPerGroup][kVocabCap];     // half-width of its interval (0 = exact)
    uint32_t id[kVocabReqPerGroup][kVocabCap]; // token << 4 | parent row
    double rk[kVocabReqPerGroup][16];          // the parents' Rk
    int tok[kVocabReqPerGroup][16];            // the parents' tokens
};

// Drop every entry whose interval lies below the W-th largest lower end; the
// new bound is returned (it never decreases).
__device__ double compact(VocabLds& L, int slot, int& cnt, double lam, int W, int lane) {
    const int n = cnt;
    double l_own[kOwn], ak_own[kOwn];
    float e_own[kOwn];
    uint32_t id_own[kOwn];
    double found = -INFINITY;
#pragma unroll
    for (int r = 0; r < kOwn; ++r) {
        const int q = lane + 64 * r;
        ak_own[r] = q < n ? L.ak[slot][q] : -INFINITY;
        e_own[r] = q < n ? L.e[slot][q] : 0.f;
        id_own[r] = q < n ? L.id[slot][q] : 0u;
        l_own[r] = ak_own[r] - (double)e_own[r];
    }
    if (n >= W) {
#pragma unroll
        for (int r = 0; r < kOwn; ++r) {
            const int q = lane + 64 * r;
            int rank = 0;
            if (q < n) {
                for (int j = 0; j < n; ++j) {
                    const double lj = L.ak[slot][j] - (double)L.e[slot][j];
                    rank += (lj > l_own[r]) | ((lj == l_own[r]) & (j < q));
                }
                if (rank == W - 1) found = l_own[r];
            }
        }
        found = wave_max_d(found);
        lam = fmax(lam, found);
    }
    __builtin_amdgcn_wave_barrier();
    int base = 0;
#pragma unroll
    for (int r = 0; r < kOwn; ++r) {
        const int q = lane + 64 * r;
        const bool keep = q < n && ak_own[r] + (double)e_own[r] >= lam;
        const unsigned long long m = __ballot(keep);
        if (keep) {
            const int pos = base + lanes_below(m);
            L.ak[slot][pos] = ak_own[r];
            L.e[slot][pos] = e_own[r];
            L.id[slot][pos] = id_own[r];
        }
        base += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
    cnt = base;
    return lam;
}

// Rescore every entry exactly and keep the exact top-W, sorted.  With `out`
// set, the list is also written there (W entries, empties padded).
template <int DT>
__device__ double finalize(VocabLds& L, int slot, int& cnt, int W, int lane, const VocabArgs& a, int b,
                           VocabEntry* out) {
    const int n = cnt;
    double K[kOwn], G[kOwn];
    float X[kOwn];
    uint32_t I[kOwn];
    const int64_t row = ((int64_t)b * a.d + (a.t - 1)) * a.V;
#pragma unroll
    for (int r = 0; r < kOwn; ++r) {
        const int q = lane + 64 * r;
        K[r] = -INFINITY;
        G[r] = 0.0;
        X[r] = 0.f;
        I[r] = 0xFFFFFFFFu;
        if (q < n) {
            const uint32_t id = L.id[slot][q];
            const int v = (int)(id >> 4), p = (int)(id & 15u);
            const float x = load_logit<DT>(a.logits, row + v);
            const int ptok = L.tok[slot][p];
            const double g = ptok >= 0 ? exact_g(a.E, a.F, a.R, ptok, v) : 0.0;
            K[r] = (L.rk[slot][p] + (double)x) + g;
            G[r] = g;
            X[r] = x;
            I[r] = id;
        }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int r = 0; r < kOwn; ++r) {
        const int q = lane + 64 * r;
        if (q < n) L.ak[slot][q] = K[r];
    }
    __builtin_amdgcn_wave_barrier();
    int rank[kOwn];
#pragma unroll
    for (int r = 0; r < kOwn; ++r) {
        const int q = lane + 64 * r;
        rank[r] = kVocabCap;
        if (q < n) {
            int c = 0;
            for (int j = 0; j < n; ++j) {
                const double kj = L.ak[slot][j];
                const uint32_t ij = L.id[slot][j];
                c += (kj > K[r]) | ((kj == K[r]) & (ij < I[r]));
            }
            rank[r] = c;
        }
    }
    __builtin_amdgcn_wave_barrier();
    double lam = -INFINITY;
#pragma unroll
    for (int r = 0; r < kOwn; ++r) {
        if (rank[r] < W) {
            L.ak[slot][rank[r]] = K[r];
            L.e[slot][rank[r]] = 0.f;
            L.id[slot][rank[r]] = I[r];
            if (out) {
                VocabEntry ve;
                ve.rk = K[r];
                ve.g = G[r];
                ve.x = X[r];
                ve.tie = (I[r] >> 4) * 64u + (I[r] & 15u);
                ve.pad[0] = ve.pad[1] = 0u;
                out[rank[r]] = ve;
            }
            if (rank[r] == W - 1) lam = K[r];
        }
    }
    const int kept = n < W ? n : W;
    if (out && lane >= kept && lane < W) {
        VocabEntry ve;
        ve.rk = -INFINITY;
        ve.g = 0.0;
        ve.x = 0.f;
        ve.tie = 0xFFFFFFFFu;
        ve.pad[0] = ve.pad[1] = 0u;
        out[lane] = ve;
    }
    __builtin_amdgcn_wave_barrier();
    cnt = kept;
    return wave_max_d(lam);
}

template <int DT, int KS>
__global__ void __launch_bounds__(kThreads) vocab_kernel(VocabArgs a) {
    __shared__ VocabLds L;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ng = (a.B + kVocabReqPerGroup - 1) / kVocabReqPerGroup;
    const int c = blockIdx.x / ng, rg = blockIdx.x - c * ng;
    const int col0 = c * a.vchunk;
    const int ncol = min(a.vchunk, a.V - col0);
    const int W = a.W;
    constexpr int R = 4 * KS;
    const int m = lane & 15, kq = lane >> 4;

    // ---- the frontier rows of the wave's requests: A operands, Rk, |E_p|
    float A[kVocabReqPerWave][KS];
    double rk[kVocabReqPerWave][4];
    float eb[kVocabReqPerWave][4];
    int nf[kVocabReqPerWave], bq[kVocabReqPerWave];
#pragma unroll
    for (int j = 0; j < kVocabReqPerWave; ++j) {
        const int slot = wave * kVocabReqPerWave + j;
        const int b = rg * kVocabReqPerGroup + wave + kWaves * j;
        bq[j] = b;
        int n = 0;
        if (b < a.B) n = a.t == 1 ? 1 : a.f_n[b];
        nf[j] = __builtin_amdgcn_readfirstlane(n);
        int tokm = -1;
        double rkm = 0.0;
        if (m < nf[j]) {
            tokm = a.t == 1 ? a.ctx[2 * b + 1] : a.f_tok[(int64_t)b * W + m];
            rkm = a.t == 1 ? 0.0 : a.f_rk[(int64_t)b * W + m];
        }
        // a root token outside the vocabulary adds no parent term (E row 0)
        const bool has_e = (unsigned)tokm < (unsigned)a.V;
        if (kq == 0) {
            L.tok[slot][m] = has_e ? tokm : -1;
            L.rk[slot][m] = rkm;
        }
        const float4* er = reinterpret_cast<const float4*>(a.E + (int64_t)(has_e ? tokm : 0) * R + kq * KS);
#pragma unroll
        for (int s4 = 0; s4 < KS / 4; ++s4) {
            const float4 e = has_e ? er[s4] : make_float4(0.f, 0.f, 0.f, 0.f);
            A[j][4 * s4 + 0] = e.x;
            A[j][4 * s4 + 1] = e.y;
            A[j][4 * s4 + 2] = e.z;
            A[j][4 * s4 + 3] = e.w;
        }
        float ne = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) ne += A[j][s] * A[j][s];
        ne += __shfl_xor(ne, 16);
        ne += __shfl_xor(ne, 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * kq + i;
            eb[j][i] = 0x1p-17f * sqrtf(__shfl(ne, r));
            rk[j][i] = shfl_d(rkm, r);
        }
    }
    __builtin_amdgcn_wave_barrier();

    double lam[kVocabReqPerWave];
    int cnt[kVocabReqPerWave];
#pragma unroll
    for (int j = 0; j < kVocabReqPerWave; ++j) {
        lam[j] = -INFINITY;
        cnt[j] = 0;
    }
    const int64_t rowoff = (int64_t)(a.t - 1) * a.V;
    const int nblk = (ncol + 15) >> 4;
    for (int cb = 0; cb < nblk; ++cb) {
        const int cl = cb * 16 + m;
        const bool vv = cl < ncol;
        const int v = col0 + (vv ? cl : 0);
        float f[KS];
        const float4* fr = reinterpret_cast<const float4*>(a.F + (int64_t)v * R + kq * KS);
#pragma unroll
        for (int s4 = 0; s4 < KS / 4; ++s4) {
            const float4 q = vv ? fr[s4] : make_float4(0.f, 0.f, 0.f, 0.f);
            f[4 * s4 + 0] = q.x;
            f[4 * s4 + 1] = q.y;
            f[4 * s4 + 2] = q.z;
            f[4 * s4 + 3] = q.w;
        }
        float nfv = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) nfv += f[s] * f[s];
        nfv += __shfl_xor(nfv, 16);
        nfv += __shfl_xor(nfv, 32);
        nfv = sqrtf(nfv);
#pragma unroll
        for (int j = 0; j < kVocabReqPerWave; ++j) {
            if (nf[j] == 0) continue;                                   // wave-uniform
            const int slot = wave * kVocabReqPerWave + j;
            const float x = vv ? load_logit<DT>(a.logits, (int64_t)bq[j] * a.d * a.V + rowoff + v) : -INFINITY;
            v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[j][s], f[s], acc, 0, 0, 0);
            double ak[4];
            float e[4];
            bool ok[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ok[i] = (4 * kq + i < nf[j]) && x != -INFINITY;
                ak[i] = (rk[j][i] + (double)x) + (double)acc[i];
                e[i] = eb[j][i] * nfv + fabsf((float)ak[i]) * 0x1p-44f + 0x1p-100f;
            }
            if (lam[j] == -INFINITY) {
                // seed the bound with the W-th largest lower end of this tile
                unsigned long long key[4];
                int nv = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    key[i] = ok[i] ? ord64(ak[i] - (double)e[i]) : 0ull;
                    nv += __popcll(__ballot(ok[i]));
                }
                if (nv >= W) lam[j] = unord64(wave_kth_key(key, W));
            }
            int base = cnt[j];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool pass = ok[i] && ak[i] + (double)e[i] >= lam[j];
                const unsigned long long bm = __ballot(pass);
                if (pass) {
                    const int pos = base + lanes_below(bm);
                    L.ak[slot][pos] = ak[i];
                    L.e[slot][pos] = e[i];
                    L.id[slot][pos] = ((uint32_t)v << 4) | (uint32_t)(4 * kq + i);
                }
                base += __popcll(bm);
            }
            __builtin_amdgcn_wave_barrier();
            cnt[j] = base;
            if (cnt[j] > kVocabCap - 256) {
                // room for the next tile: tighten, and if intervals still
                // overlap too much (ties), settle the order exactly
                lam[j] = compact(L, slot, cnt[j], lam[j], W, lane);
                if (cnt[j] > kVocabCap - 256)
                    lam[j] = finalize<DT>(L, slot, cnt[j], W, lane, a, bq[j], nullptr);
            }
        }
    }

    // ---- the chunk's exact top-W per request
#pragma unroll
    for (int j = 0; j < kVocabReqPerWave; ++j) {
        const int b = bq[j];
        if (b >= a.B) continue;                                         // wave-uniform
        const int slot = wave * kVocabReqPerWave + j;
        VocabEntry* out = a.part + ((int64_t)b * a.C2 + c) * W;
        if (cnt[j] > W) lam[j] = compact(L, slot, cnt[j], lam[j], W, lane);
        finalize<DT>(L, slot, cnt[j], W, lane, a, b, out);
    }
}

// ---------------------------------------------------------------------------
// frontier merge: one workgroup per request
// ---------------------------------------------------------------------------
constexpr int kFrontCap = 1024;

__device__ __forceinline__ bool entry_before(double ka, uint32_t ta, double kb, uint32_t tb) {
    return ka > kb || (ka == kb && ta < tb);
}

__global__ void __launch_bounds__(kThreads) frontier_kernel(FrontierArgs a) {
    __shared__ double s_k[kFrontCap];
    __shared__ uint32_t s_t[kFrontCap];
    __shared__ int s_src[kFrontCap];
    __shared__ double s_red_k[kWaves];
    __shared__ uint32_t s_red_t[kWaves];
    __shared__ int s_cnt;
    __shared__ int s_win[kFullMaxW];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int W = a.W, C2 = a.C2;
    const VocabEntry* lists = a.part + (int64_t)b * C2 * W;

    // 1. a lower bound for the frontier's W-th key: the best W-th entry of any list
    double hk = -INFINITY;
    uint32_t ht = 0xFFFFFFFFu;
    for (int c = tid; c < C2; c += kThreads) {
        const VocabEntry& e = lists[(int64_t)c * W + (W - 1)];
        if (e.rk != -INFINITY && entry_before(e.rk, e.tie, hk, ht)) {
            hk = e.rk;
            ht = e.tie;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const double ok = __shfl_xor(hk, off);
        const uint32_t ot = __shfl_xor(ht, off);
        if (entry_before(ok, ot, hk, ht)) {
            hk = ok;
            ht = ot;
        }
    }
    if (lane == 0) {
        s_red_k[wave] = hk;
        s_red_t[wave] = ht;
    }
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    hk = s_red_k[0];
    ht = s_red_t[0];
    for (int w = 1; w < kWaves; ++w)
        if (entry_before(s_red_k[w], s_red_t[w], hk, ht)) {
            hk = s_red_k[w];
            ht = s_red_t[w];
        }

    // 2. every entry at or above the bound (lists are sorted)
    for (int c = tid; c < C2; c += kThreads) {
        for (int r = 0; r < W; ++r) {
            const int64_t idx = (int64_t)c * W + r;
            const VocabEntry& e = lists[idx];
            if (e.rk == -INFINITY) break;
            if (hk != -INFINITY && entry_before(hk, ht, e.rk, e.tie)) break;
            const int pos = atomicAdd(&s_cnt, 1);
            if (pos < kFrontCap) {
                s_k[pos] = e.rk;
                s_t[pos] = e.tie;
                s_src[pos] = (int)idx;
            }
        }
    }
    __syncthreads();
    const int n = s_cnt;
    const int nsel = n < W ? n : W;
    if (n <= kFrontCap) {
        for (int q = tid; q < n; q += kThreads) {
            int r = 0;
            for (int j = 0; j < n; ++j) r += entry_before(s_k[j], s_t[j], s_k[q], s_t[q]);
            if (r < W) s_win[r] = s_src[q];
        }
    } else {
        // many exact ties at the bound: take the best W one at a time
        double pk = INFINITY;
        uint32_t pt = 0u;
        for (int r = 0; r < W; ++r) {
            double bk = -INFINITY;
            uint32_t bt = 0xFFFFFFFFu;
            int bi = -1;
            for (int64_t idx = tid; idx < (int64_t)C2 * W; idx += kThreads) {
                const VocabEntry& e = lists[idx];
                if (e.rk == -INFINITY || !entry_before(pk, pt, e.rk, e.tie)) continue;
                if (bi < 0 || entry_before(e.rk, e.tie, bk, bt)) {
                    bk = e.rk;
                    bt = e.tie;
                    bi = (int)idx;
                }
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const double ok = __shfl_xor(bk, off);
                const uint32_t ot = __shfl_xor(bt, off);
                const int oi = __shfl_xor(bi, off);
                if (oi >= 0 && (bi < 0 || entry_before(ok, ot, bk, bt))) {
                    bk = ok;
                    bt = ot;
                    bi = oi;
                }
            }
            __syncthreads();
            if (lane == 0) {
                s_red_k[wave] = bk;
                s_red_t[wave] = bt;
                s_src[wave] = bi;
            }
            __syncthreads();
            bk = -INFINITY;
            bt = 0xFFFFFFFFu;
            bi = -1;
            for (int w = 0; w < kWaves; ++w)
                if (s_src[w] >= 0 && (bi < 0 || entry_before(s_red_k[w], s_red_t[w], bk, bt))) {
                    bk = s_red_k[w];
                    bt = s_red_t[w];
                    bi = s_src[w];
                }
            if (tid == 0) s_win[r] = bi;
            pk = bk;
            pt = bt;
        }
    }
    __syncthreads();

    // 3. the new nodes and the next frontier (parents read before any write)
    const int base = a.t == 1 ? 0 : a.n_tree[b];
    const int64_t fb = (int64_t)b * W;
    int tok = 0, pnode = -1;
    double rkv = 0.0, s = 0.0;
    if (tid < nsel) {
        const VocabEntry& e = lists[s_win[tid]];
        tok = (int)(e.tie >> 6);
        const int pr = (int)(e.tie & 63u);
        const double ps = a.t == 1 ? 0.0 : a.f_s[fb + pr];
        pnode = a.t == 1 ? -1 : a.f_node[fb + pr];
        rkv = e.rk;
        s = (ps + ((double)e.x - a.lse[(int64_t)b * a.d + (a.t - 1)])) + e.g;
    }
    __syncthreads();
    if (tid < nsel) {
        const int node = base + tid;
        const int64_t nb = (int64_t)b * a.d * W + node;
        a.nd_tok[nb] = tok;
        a.nd_par[nb] = pnode;
        a.nd_dep[nb] = a.t;
        a.nd_s[nb] = s;
        a.f_tok[fb + tid] = tok;
        a.f_rk[fb + tid] = rkv;
        a.f_s[fb + tid] = s;
        a.f_node[fb + tid] = node;
    }
    if (tid == 0) {
        a.f_n[b] = nsel;
        a.n_tree[b] = base + nsel;
    }
}

}  // namespace

hipError_t launch_vocab(const VocabArgs& a, hipStream_t stream) {
    if (a.B <= 0) return hipSuccess;
    const int ng = (a.B + kVocabReqPerGroup - 1) / kVocabReqPerGroup;
    const dim3 grid((unsigned)(a.C2 * ng)), block(kThreads);
    const bool bf = a.dtype == DT_DTYPE_BF16;
    switch (a.R) {
    case 16:
        if (bf) hipLaunchKernelGGL((vocab_kernel<DT_DTYPE_BF16, 4>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((vocab_kernel<DT_DTYPE_F32, 4>), grid, block, 0, stream, a);
        break;
    case 32:
        if (bf) hipLaunchKernelGGL((vocab_kernel<DT_DTYPE_BF16, 8>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((vocab_kernel<DT_DTYPE_F32, 8>), grid, block, 0, stream, a);
        break;
    case 64:
        if (bf) hipLaunchKernelGGL((vocab_kernel<DT_DTYPE_BF16, 16>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((vocab_kernel<DT_DTYPE_F32, 16>), grid, block, 0, stream, a);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_frontier(const FrontierArgs& a, hipStream_t stream) {
    if (a.B <= 0) return hipSuccess;
    hipLaunchKernelGGL(frontier_kernel, dim3((unsigned)a.B), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dt
