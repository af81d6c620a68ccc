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
//                    on bf16 MFMA (v_mfma_f32_16x16x32_bf16; F is rounded to
//                    bf16 once per call, E rows when they are loaded).  The
//                    matrix cores decide nothing: every candidate carries an
//                    interval around its fp64 key, ak +- e with
//                    e = 1.125 * 2^-7 |E_p| |F_v| + |ak| 2^-44 (rounding both
//                    operands to bf16 moves each product by at most
//                    (2^-7 + 2^-16) |E_k F_k|, the fp32 accumulation adds at
//                    most about 2^-18 of the sum, and
//                    sum |E_k F_k| <= |E_p| |F_v|), so a candidate is
//                    dropped only when its upper end is below the W-th largest
//                    lower end seen.  What survives is rescored exactly, in
//                    fp64 summed k = 0..R-1 over the fp32 E and F (fp32 x
//                    fp32 products are exact in fp64, so the sum is the
//                    oracle's bit for bit), and the chunk's exact top-W is
//                    written out.  Before any product, a block of 16 tokens
//                    is skipped when no token in it can reach the bound
//                    even with the largest parent term Cauchy-Schwarz
//                    allows (|g(p, v)| <= |E_p| |F_v|); the logits and F
//                    norms this test needs are loaded for many blocks at
//                    once, and only the blocks that pass load F rows.
//  frontier_kernel - one workgroup per request: merges the chunks' sorted
//                    lists (the largest W-th entry of any list bounds the
//                    frontier's W-th key from below, so only entries above it
//                    are ranked), appends the new nodes with their cumulative
//                    log-scores S = (S_p + (x - lse)) + g, and makes them the
//                    next frontier.
// The budget and the outputs are then the tree kernel's (finish_kernel).
#include "common.h"
#include "wave.h"

namespace dt {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef short s4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

// two floats rounded to bf16 (nearest, ties to even; finite inputs), packed
// low element first
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
    auto rne = [](float f) {
        const uint32_t u = __float_as_uint(f);
        return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    };
    return rne(lo) | (rne(hi) << 16);
}

// one 16 x 16 tile of the screen's product on bf16 matrix cores: lane
// (m, kq) holds KS consecutive features kq*KS .. kq*KS+KS-1 of its A row
// (frontier node m) and B column (token m), two per word; the products are
// exact in fp32 and accumulated in fp32
template <int KS>
__device__ __forceinline__ v4f mfma_bf16(const uint32_t (&a)[KS / 2], const uint32_t (&b)[KS / 2], v4f acc) {
    if constexpr (KS == 4) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4v, u2v{a[0], a[1]}),
                                                         __builtin_bit_cast(s4v, u2v{b[0], b[1]}), acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int h = 0; h < KS / 8; ++h)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf8v, u4v{a[4 * h], a[4 * h + 1], a[4 * h + 2], a[4 * h + 3]}),
                __builtin_bit_cast(bf8v, u4v{b[4 * h], b[4 * h + 1], b[4 * h + 2], b[4 * h + 3]}), acc, 0, 0, 0);
        return acc;
    }
}

// lane (m, kq)'s KS bf16 features of token v's F row
template <int KS>
__device__ __forceinline__ void load_fbf(const uint16_t* __restrict__ Fbf, int64_t v, int kq, uint32_t (&f)[KS / 2]) {
    const uint16_t* src = Fbf + v * (4 * KS) + kq * KS;
    if constexpr (KS == 4) {
        const uint2 q = *reinterpret_cast<const uint2*>(src);
        f[0] = q.x;
        f[1] = q.y;
    } else {
#pragma unroll
        for (int h = 0; h < KS / 8; ++h) {
            const uint4 q = reinterpret_cast<const uint4*>(src)[h];
            f[4 * h] = q.x;
            f[4 * h + 1] = q.y;
            f[4 * h + 2] = q.z;
            f[4 * h + 3] = q.w;
        }
    }
}

// raw logit bits (bf16 zero-extended, or fp32), widened only where used, so
// that a prefetch is not waited for at the load
template <int DT>
__device__ __forceinline__ uint32_t load_raw(const void* base, int64_t i) {
    if (DT == DT_DTYPE_BF16) return (uint32_t)((const uint16_t*)base)[i];
    return __float_as_uint(((const float*)base)[i]);
}

template <int DT>
__device__ __forceinline__ float raw_logit(uint32_t u) {
    return DT == DT_DTYPE_BF16 ? __uint_as_float(u << 16) : __uint_as_float(u);
}

template <int DT>
__device__ __forceinline__ float load_logit(const void* base, int64_t i) {
    if (DT == DT_DTYPE_BF16) return __uint_as_float((uint32_t)((const uint16_t*)base)[i] << 16);
    return ((const float*)base)[i];
}

__device__ __forceinline__ double wave_max_d(double v) { return wave_max_f64(v); }

__device__ __forceinline__ int lanes_below(unsigned long long m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// the kth largest of the wave's 4 x 64 32-bit keys (key 0 = no candidate)
__device__ uint32_t wave_kth_key32(const uint32_t (&key)[4], int kth) {
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = T | (1u << bit);
        int n = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) n += __popcll(__ballot(key[i] >= c));
        if (n >= kth) T = c;
    }
    return T;
}

// fp32 screen thresholds of the four output rows a lane holds: a candidate
// whose fp64 interval reaches lam has (x + acc) + e32 >= thr; the slack
// covers the fp64 roundings of the key (the screen may only pass more).
// Rows past the frontier get +inf, so nothing passes there; the screen
// takes a missing or -inf logit as NaN, which passes nothing either.
__device__ __forceinline__ void row_thresholds(float (&thr)[4], double lam, const double* rk, int nrow, int kq) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        thr[i] = 4 * kq + i >= nrow ? INFINITY
                 : lam == -INFINITY ? -INFINITY
                                    : __double2float_rd((lam - rk[i]) - 0x1p-40 * (fabs(lam) + fabs(rk[i])));
}

// Block skip.  |g(p, v)| <= |E_p| |F_v| (Cauchy-Schwarz), so no frontier
// node gives token v a key above rkmax + x_v + Emax |F_v|; a block of tokens
// none of which reaches lam that way holds no candidate and is skipped
// before its products.  The fp32 test x + Emax' |F_v| >= ts takes Emax' a
// little above the largest |E_p| (covering the fp32 norms) and ts rounded
// down with room for the fp64 roundings of the keys and of the test.
__device__ __forceinline__ float skip_threshold(double lam, double rkmax) {
    return lam == -INFINITY ? -INFINITY
                            : __double2float_rd((lam - rkmax) - 0x1p-30 * (fabs(lam) + fabs(rkmax)) - 0x1p-100);
}

// exact key of one candidate, summed like the oracle: k = 0 .. R-1 (the rows
// are loaded in groups of four vectors ahead of the serial sum)
template <int R>
__device__ __forceinline__ double exact_g(const float* __restrict__ E, const float* __restrict__ F, int tok, int v) {
    const float4* e4 = reinterpret_cast<const float4*>(E + (int64_t)tok * R);
    const float4* f4 = reinterpret_cast<const float4*>(F + (int64_t)v * R);
    double g = 0.0;
#pragma unroll
    for (int q0 = 0; q0 < R / 4; q0 += 4) {
        float4 e[4], f[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            e[u] = e4[q0 + u];
            f[u] = f4[q0 + u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            g += (double)e[u].x * (double)f[u].x;
            g += (double)e[u].y * (double)f[u].y;
            g += (double)e[u].z * (double)f[u].z;
            g += (double)e[u].w * (double)f[u].w;
        }
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

// Drop every entry whose interval lies below the bound.
__device__ void compact(VocabLds& L, int slot, int& cnt, double lam, int lane) {
    const int n = cnt;
    double ak_own[kOwn];
    float e_own[kOwn];
    uint32_t id_own[kOwn];
#pragma unroll
    for (int r = 0; r < kOwn; ++r) {
        const int q = lane + 64 * r;
        ak_own[r] = q < n ? L.ak[slot][q] : -INFINITY;
        e_own[r] = q < n ? L.e[slot][q] : 0.f;
        id_own[r] = q < n ? L.id[slot][q] : 0u;
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
}

// The W largest lower ends inserted so far, descending, in lanes 0..W-1
// (-inf where fewer); the bound is the W-th.
__device__ __forceinline__ void top_insert(double& lst, double y, int W, int lane) {
    const int pos = __popcll(__ballot(lane < W && lst >= y));
    if (pos >= W) return;                                               // wave-uniform
    const long long u = __double_as_longlong(lst);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(u & 0xFFFFFFFFll), 0x111, 0xF, 0xF, false);  // row_shr:1
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), 0x111, 0xF, 0xF, false);
    const double up = __longlong_as_double(((long long)hi << 32) | (uint32_t)lo);
    lst = lane < pos ? lst : (lane == pos ? y : up);
}

__device__ __forceinline__ double readlane_d(double v, int l) {
    const long long u = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(u & 0xFFFFFFFFll), l);
    const int hi = __builtin_amdgcn_readlane((int)(u >> 32), l);
    return __longlong_as_double(((long long)hi << 32) | (uint32_t)lo);
}

// Rescore every entry exactly and keep the exact top-W, sorted.  With `out`
// set, the list is also written there (W entries, empties padded).
template <int DT, int R>
__device__ double finalize(VocabLds& L, int slot, int& cnt, int W, int lane, const VocabArgs& a, int b,
                           VocabEntry* out, VocabEntry* out2 = nullptr) {
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
            const double g = ptok >= 0 ? exact_g<R>(a.E, a.F, ptok, v) : 0.0;
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
                ve.pad[0] = rank[r] == 0 ? (uint32_t)(n < W ? n : W) : 0u;   // entry 0: the list's length
                ve.pad[1] = 0u;
                out[rank[r]] = ve;
                if (out2) out2[rank[r]] = ve;
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
__global__ void __launch_bounds__(kThreads, 3) vocab_kernel(VocabArgs a) {
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

    // ---- the frontier rows of the wave's requests: A operands (bf16), Rk, |E_p|
    float A[kVocabReqPerWave][KS];
    uint32_t Ab[kVocabReqPerWave][KS / 2];
    float eb[kVocabReqPerWave][4];
    float emax[kVocabReqPerWave];   // a little above the largest |E_p| of the frontier
    int nf[kVocabReqPerWave], bq[kVocabReqPerWave];
    // The first group of logits and F norms (they do not depend on the
    // frontier), then every frontier read of both requests, are issued
    // before anything waits on them; indices are clamped so each read is in
    // bounds.
    const int64_t rowoff = (int64_t)(a.t - 1) * a.V;
    int64_t xrow[kVocabReqPerWave];
#pragma unroll
    for (int j = 0; j < kVocabReqPerWave; ++j) {
        bq[j] = rg * kVocabReqPerGroup + wave + kWaves * j;
        xrow[j] = (int64_t)(bq[j] < a.B ? bq[j] : 0) * a.d * a.V + rowoff;
    }
    constexpr int G = kVocabGroupBlocks;
    float gn[G];
    uint32_t gx[G][kVocabReqPerWave];
#pragma unroll
    for (int q = 0; q < G; ++q) {
        const int cl = q * 16 + m;
        const int v = col0 + (cl < ncol ? cl : ncol - 1);
        gn[q] = a.fnorm[v];
#pragma unroll
        for (int j = 0; j < kVocabReqPerWave; ++j) gx[q][j] = load_raw<DT>(a.logits, xrow[j] + v);
    }
    int nraw[kVocabReqPerWave], traw[kVocabReqPerWave];
    double rraw[kVocabReqPerWave], seedv[kVocabReqPerWave];
#pragma unroll
    for (int j = 0; j < kVocabReqPerWave; ++j) {
        const int bc = bq[j] < a.B ? bq[j] : 0;
        const int64_t fi = (int64_t)bc * W + (m < W ? m : 0);
        nraw[j] = a.t == 1 ? 1 : a.f_n[bc];
        traw[j] = a.t == 1 ? a.ctx[2 * bc + 1] : a.f_tok[fi];
        rraw[j] = a.t == 1 ? 0.0 : a.f_rk[fi];
        seedv[j] = a.seed[bc];
    }
#pragma unroll
    for (int j = 0; j < kVocabReqPerWave; ++j) {
        const int slot = wave * kVocabReqPerWave + j;
        const int b = bq[j];
        nf[j] = __builtin_amdgcn_readfirstlane(b < a.B ? nraw[j] : 0);
        const int tokm = m < nf[j] ? traw[j] : -1;
        const double rkm = m < nf[j] ? rraw[j] : 0.0;
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
#pragma unroll
        for (int s = 0; s < KS / 2; ++s) Ab[j][s] = bf16_pair(A[j][2 * s], A[j][2 * s + 1]);
        ne += __shfl_xor(ne, 16);
        ne += __shfl_xor(ne, 32);
        // |g32 - g| <= (2 * 2^-8 + 2^-16) sum_k |E_k F_k| from rounding both
        // operands to bf16, plus about 2^-18 of it from the fp32
        // accumulation (at most R <= 64 roundings of 2^-24), and
        // sum_k |E_k F_k| <= |E_p| |F_v|: under 1.003 * 2^-7 |E_p| |F_v|,
        // with room to spare at 1.125 * 2^-7
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * kq + i;
            eb[j][i] = 0x1.2p-7f * sqrtf(__shfl(ne, r));
        }
        emax[j] = sqrtf(wave_max_f32_all(ne)) * (1.0f + 0x1p-14f);
    }
    __builtin_amdgcn_wave_barrier();
    double rkmax[kVocabReqPerWave];
#pragma unroll
    for (int j = 0; j < kVocabReqPerWave; ++j) {
        const int slot = wave * kVocabReqPerWave + j;
        rkmax[j] = wave_max_f64(m < nf[j] ? L.rk[slot][m] : -INFINITY);
    }

    double lam[kVocabReqPerWave], lst[kVocabReqPerWave];
    int cnt[kVocabReqPerWave];
    float thr[kVocabReqPerWave][4], ts[kVocabReqPerWave];
#pragma unroll
    for (int j = 0; j < kVocabReqPerWave; ++j) {
        lam[j] = nf[j] > 0 ? seedv[j] : -INFINITY;                     // exact keys of real candidates
        lst[j] = -INFINITY;
        cnt[j] = 0;
        row_thresholds(thr[j], lam[j], &L.rk[wave * kVocabReqPerWave + j][4 * kq], nf[j], kq);
        ts[j] = skip_threshold(lam[j], rkmax[j]);
    }
    const int nblk = (ncol + 15) >> 4;

    // The blocks' logits and F norms are loaded a group of kVocabGroupBlocks
    // blocks at a time (one memory round trip per group) and the bound above
    // marks the blocks that can hold a candidate of each request; only those
    // load their F rows and run the products and the screen.  Every load
    // reads a valid address (the last column for the padding of a ragged
    // chunk) and validity is applied where the block is used.
    for (int g0 = 0; g0 < nblk; g0 += G) {
        if (g0 > 0) {                                                   // (the first group is loaded)
#pragma unroll
            for (int q = 0; q < G; ++q) {
                const int cl = (g0 + q) * 16 + m;
                const int v = col0 + (cl < ncol ? cl : ncol - 1);
                gn[q] = a.fnorm[v];
#pragma unroll
                for (int j = 0; j < kVocabReqPerWave; ++j) gx[q][j] = load_raw<DT>(a.logits, xrow[j] + v);
            }
        }
        uint32_t livem[kVocabReqPerWave], anyl = 0u;      // bit q: block g0 + q (wave-uniform)
#pragma unroll
        for (int j = 0; j < kVocabReqPerWave; ++j) {
            livem[j] = 0u;
#pragma unroll
            for (int q = 0; q < G; ++q) {
                const int cl = (g0 + q) * 16 + m;
                const float xr = raw_logit<DT>(gx[q][j]);
                const float x = (cl < ncol && xr != -INFINITY) ? xr : __builtin_nanf("");
                const float w = fmaf(emax[j], gn[q], x);
                const bool hit = __ballot(w + fabsf(w) * 0x1p-20f >= ts[j]) != 0ull;
                livem[j] |= (hit && g0 + q < nblk && nf[j] > 0) ? 1u << q : 0u;
            }
            anyl |= livem[j];
        }
        while (anyl != 0u) {
            const int q = __builtin_ctz(anyl);
            anyl &= anyl - 1u;
            const int cb = g0 + q;
            const int cl = cb * 16 + m;
            const bool vv = cl < ncol;
            const int v = col0 + (vv ? cl : ncol - 1);
            uint32_t fc[KS / 2];
            load_fbf<KS>(a.Fbf, v, kq, fc);
            const float nfv = a.fnorm[v];
            float xs[kVocabReqPerWave];
            bool live[kVocabReqPerWave];
#pragma unroll
            for (int j = 0; j < kVocabReqPerWave; ++j) {
                const float xr = raw_logit<DT>(load_raw<DT>(a.logits, xrow[j] + v));
                xs[j] = (vv && xr != -INFINITY) ? xr : __builtin_nanf("");
                live[j] = (livem[j] >> q) & 1u;
            }
            v4f acc[kVocabReqPerWave];
#pragma unroll
            for (int j = 0; j < kVocabReqPerWave; ++j) {
                acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
                if (live[j]) acc[j] = mfma_bf16<KS>(Ab[j], fc, acc[j]);
            }
#pragma unroll
            for (int j = 0; j < kVocabReqPerWave; ++j) {
                if (!live[j]) continue;                                     // wave-uniform
                const int slot = wave * kVocabReqPerWave + j;
                const float x = xs[j];
                // (branch-free: the thresholds reject rows past the frontier, and
                // a NaN logit every comparison)
                bool pf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float sx = x + acc[j][i];
                    const float e32 = fmaf(eb[j][i], nfv, fmaf(fabsf(sx), 0x1p-22f, 0x1p-100f));
                    pf[i] = sx + e32 >= thr[j][i];
                }
                const bool anyp = (pf[0] | pf[1]) | (pf[2] | pf[3]);
                if (lam[j] == -INFINITY) {
                    bool ok[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) ok[i] = (4 * kq + i < nf[j]) && x == x;
                    // seed the bound: the W-th largest lower end of this tile,
                    // rounded down to fp32
                    uint32_t key[4];
                    int nv = 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const double ak = (L.rk[slot][4 * kq + i] + (double)x) + (double)acc[j][i];
                        const float e = eb[j][i] * nfv + fabsf((float)ak) * 0x1p-44f + 0x1p-100f;
                        key[i] = ok[i] ? ord_bits(__float_as_uint(__double2float_rd(ak - (double)e))) : 0u;
                        nv += __popcll(__ballot(ok[i]));
                    }
                    if (nv >= W) {
                        lam[j] = (double)__uint_as_float(unord_bits(wave_kth_key32(key, W)));
                        row_thresholds(thr[j], lam[j], &L.rk[wave * kVocabReqPerWave + j][4 * kq], nf[j], kq);
                        ts[j] = skip_threshold(lam[j], rkmax[j]);
                    }
                }
                if (__ballot(anyp) == 0) continue;                          // nothing reaches the bound
                int base = cnt[j];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const double ak = (L.rk[slot][4 * kq + i] + (double)x) + (double)acc[j][i];
                    const float e = eb[j][i] * nfv + fabsf((float)ak) * 0x1p-44f + 0x1p-100f;
                    const bool pass = pf[i] && ak + (double)e >= lam[j];
                    unsigned long long bm = __ballot(pass);
                    if (pass) {
                        const int pos = base + lanes_below(bm);
                        L.ak[slot][pos] = ak;
                        L.e[slot][pos] = e;
                        L.id[slot][pos] = ((uint32_t)v << 4) | (uint32_t)(4 * kq + i);
                    }
                    base += __popcll(bm);
                    // the bound follows the W-th largest lower end inserted
                    const double lo = ak - (double)e;
                    while (bm) {
                        const int src = __builtin_ctzll(bm);
                        bm &= bm - 1;
                        top_insert(lst[j], readlane_d(lo, src), W, lane);
                    }
                }
                __builtin_amdgcn_wave_barrier();
                cnt[j] = base;
                const double lw = readlane_d(lst[j], W - 1);
                if (lw > lam[j]) lam[j] = lw;
                if (cnt[j] > kVocabCap - 256) {
                    // room for the next tile; if intervals still overlap too much
                    // (ties), settle the order exactly
                    compact(L, slot, cnt[j], lam[j], lane);
                    if (cnt[j] > kVocabCap - 256) {
                        lam[j] = fmax(lam[j], finalize<DT, R>(L, slot, cnt[j], W, lane, a, bq[j], nullptr));
                        lst[j] = lane < cnt[j] ? L.ak[slot][lane < kVocabCap ? lane : 0] : -INFINITY;
                    }
                }
                row_thresholds(thr[j], lam[j], &L.rk[wave * kVocabReqPerWave + j][4 * kq], nf[j], kq);
                ts[j] = skip_threshold(lam[j], rkmax[j]);
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
        if (cnt[j] > W) compact(L, slot, cnt[j], lam[j], lane);
        // a non-empty list is also appended to the request's compact list
        // (a slot range taken with one atomic; past the capacity the frontier
        // kernel falls back to the per-chunk lists)
        const int kept = cnt[j] < W ? cnt[j] : W;
        VocabEntry* out2 = nullptr;
        if (kept > 0) {
            int pos = 0;
            if (lane == 0) pos = atomicAdd(&a.cmp_n[b], kept);
            pos = __builtin_amdgcn_readfirstlane(pos);
            if (pos + kept <= kFrontCap) out2 = a.cmp + (int64_t)b * kFrontCap + pos;
        }
        finalize<DT, R>(L, slot, cnt[j], W, lane, a, b, out, out2);
    }
}

// ---------------------------------------------------------------------------
// A lower bound for a depth's W-th key before it is searched: the pairs
// (frontier node, one of the row's top-k tokens) are real candidates of the
// depth, so the W-th largest of their keys' lower ends bounds the W-th key of
// all candidates from below.  g is small next to the spread of the logits,
// so the bound is close, and the vocabulary scan then keeps little but the
// winners.  The pairs' g come from one 16 x 16 fp32 MFMA tile per 16 tokens,
// with the scan's interval (ak - e is below the exact key).  One wave.
// ---------------------------------------------------------------------------
// the token side of the pairs: the row's first 32 top-k tokens, their logits,
// F rows and norms (independent of the frontier, so loaded early)
template <int KS>
struct SeedSide {
    float f[2][KS];
    float x[2];
    float nf[2];
    bool ok[2];
};

template <int KS>
__device__ __forceinline__ void seed_side(const FrontierArgs& a, int row, int lane, SeedSide<KS>& sd) {
    constexpr int R = 4 * KS;
    const int m = lane & 15, kq = lane >> 4;
    const int k = a.k;
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
        const int col = tile * 16 + m;
        const bool cv = col < k;
        const int64_t o = (int64_t)row * k + (cv ? col : 0);
        const int v = cv ? a.ttok[o] : 0;
        const float x = cv ? a.tx[o] : -INFINITY;
        const bool vv = cv && x != -INFINITY && v >= 0 && v < a.V;
        const int vs = vv ? v : 0;
        const float4* fr = reinterpret_cast<const float4*>(a.F + (int64_t)vs * R + kq * KS);
#pragma unroll
        for (int s4 = 0; s4 < KS / 4; ++s4) {
            const float4 q = fr[s4];
            sd.f[tile][4 * s4 + 0] = q.x;
            sd.f[tile][4 * s4 + 1] = q.y;
            sd.f[tile][4 * s4 + 2] = q.z;
            sd.f[tile][4 * s4 + 3] = q.w;
        }
        sd.nf[tile] = a.fnorm[vs];
        sd.x[tile] = x;
        sd.ok[tile] = vv;
    }
}

// the frontier side: lane (m, kq) holds quarter kq of E[tok] for frontier
// node m (zeros when tok < 0)
template <int KS>
__device__ __forceinline__ void load_erow(const FrontierArgs& a, int tok, int kq, float (&A)[KS]) {
    constexpr int R = 4 * KS;
    const float4* er = reinterpret_cast<const float4*>(a.E + (int64_t)(tok >= 0 ? tok : 0) * R + kq * KS);
#pragma unroll
    for (int s4 = 0; s4 < KS / 4; ++s4) {
        const float4 e = tok >= 0 ? er[s4] : make_float4(0.f, 0.f, 0.f, 0.f);
        A[4 * s4 + 0] = e.x;
        A[4 * s4 + 1] = e.y;
        A[4 * s4 + 2] = e.z;
        A[4 * s4 + 3] = e.w;
    }
}

// the bound: one 16 x 16 fp32 MFMA tile per 16 tokens, each pair's lower end
// ak - e (below its exact key), the W-th largest of them
template <int KS>
__device__ double seed_bound(const FrontierArgs& a, const SeedSide<KS>& sd, int nfr, const float (&A)[KS],
                             const double* frk, int lane) {
    const int kq = lane >> 4;
    const int W = a.W;
    float ne = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) ne += A[s] * A[s];
    ne += __shfl_xor(ne, 16);
    ne += __shfl_xor(ne, 32);
    float eb[4];
    double rr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * kq + i;
        eb[i] = 0x1p-17f * sqrtf(__shfl(ne, r)) * (1.f + 0x1p-20f);
        rr[i] = frk[r < nfr ? r : 0];
    }
    double lo[2][4];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[s], sd.f[tile][s], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = sd.ok[tile] && 4 * kq + i < nfr;
            const double ak = (rr[i] + (double)sd.x[tile]) + (double)acc[i];
            const float e = eb[i] * sd.nf[tile] + fabsf((float)ak) * 0x1p-44f + 0x1p-100f;
            lo[tile][i] = ok ? ak - (double)e : -INFINITY;
        }
    }
    // the W-th largest of the lanes' two best lower ends, each rounded down
    // to fp32 (still below the exact keys; W distinct pairs reach it): the
    // largest T with at least W of those values >= T, bit by bit
    double b1 = -INFINITY, b2 = -INFINITY;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const double v = lo[q >> 2][q & 3];
        b2 = fmax(b2, fmin(b1, v));
        b1 = fmax(b1, v);
    }
    const bool ok1 = b1 != -INFINITY, ok2 = b2 != -INFINITY;
    if (__popcll(__ballot(ok1)) + __popcll(__ballot(ok2)) < W) return -INFINITY;   // fewer than W pairs
    const uint32_t k1 = ok1 ? ord_bits(__float_as_uint(__double2float_rd(b1))) : 0u;
    const uint32_t k2 = ok2 ? ord_bits(__float_as_uint(__double2float_rd(b2))) : 0u;
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = T | (1u << bit);
        if (__popcll(__ballot(k1 >= c)) + __popcll(__ballot(k2 >= c)) >= W) T = c;
    }
    return (double)__uint_as_float(unord_bits(T));
}

// depth 1: the root is the only frontier node
template <int KS>
__global__ void __launch_bounds__(64) seed1_kernel(FrontierArgs a, const int32_t* __restrict__ ctx) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const int root = ctx[2 * b + 1];
    const int tok = (unsigned)root < (unsigned)a.V ? root : -1;      // outside the vocabulary: no parent term
    const double rk0 = 0.0;
    SeedSide<KS> sd;
    seed_side<KS>(a, b * a.d + 0, lane, sd);
    float A[KS];
    load_erow<KS>(a, (lane & 15) < 1 ? tok : -1, lane >> 4, A);
    const double s = seed_bound<KS>(a, sd, 1, A, &rk0, lane);
    if (lane == 0) {
        a.seed[b] = s;
        a.cmp_n[b] = 0;                                            // depth 1's compact list starts empty
    }
}

// ---------------------------------------------------------------------------
// frontier merge: one workgroup per request
// ---------------------------------------------------------------------------
constexpr int kHeadsPerLane = kMaxVocabChunks / 64;

__device__ __forceinline__ bool entry_before(double ka, uint32_t ta, double kb, uint32_t tb) {
    return ka > kb || (ka == kb && ta < tb);
}

// One wave per request.  The chunk lists are sorted, so the W-th largest of
// their heads bounds the frontier's W-th key from below (W distinct entries
// reach it) and only entries at or above it can be selected; they are ranked
// exactly by (Rk desc, tie asc).
template <int KS>
__global__ void __launch_bounds__(64) frontier_kernel(FrontierArgs a) {
    __shared__ double s_k[kFrontCap];
    __shared__ uint32_t s_t[kFrontCap];
    __shared__ int s_src[kFrontCap];
    __shared__ double s_g[kFrontCap];
    __shared__ float s_x[kFrontCap];
    __shared__ int s_q[kMaxVocabChunks];
    __shared__ int s_win[kFullMaxW];
    __shared__ double s_ps[kFullMaxW];
    __shared__ int s_pn[kFullMaxW];
    __shared__ int s_ftok[kFullMaxW];
    __shared__ double s_frk[kFullMaxW];
    const int b = blockIdx.x, lane = threadIdx.x;
    const int W = a.W, C2 = a.C2;
    const VocabEntry* lists = a.part + (int64_t)b * C2 * W;
    const int64_t fb = (int64_t)b * W;

    // 0. loads that need nothing from this kernel: the previous frontier's
    //    scores and node ids, and the token side of the next depth's bound
    if (a.t > 1 && lane < W) {
        s_ps[lane] = a.f_s[fb + lane];
        s_pn[lane] = a.f_node[fb + lane];
    }
    SeedSide<KS> sd;
    if (a.t < a.d) seed_side<KS>(a, b * a.d + a.t, lane, sd);
    const double lse_t = a.lse[(int64_t)b * a.d + (a.t - 1)];

    // 1. the compact list of this depth's entries (its count and the first 64
    //    entries in one round), then the count cleared for the next depth
    const int ncmp = __builtin_amdgcn_readfirstlane(a.cmp_n[b]);
    const VocabEntry* cl = a.cmp + (int64_t)b * kFrontCap;
    const VocabEntry e0 = cl[lane];                                      // (in bounds: kFrontCap >= 64)
    if (lane == 0 && ncmp >= 0) a.cmp_n[b] = 0;                        // (after the read: depends on it)

    int n = 0;
    double hk[kHeadsPerLane];
    if (ncmp <= kFrontCap) {
        // 2a. every entry found (usually a few dozen)
        if (lane < ncmp) {
            s_k[lane] = e0.rk;
            s_t[lane] = e0.tie;
            s_g[lane] = e0.g;
            s_x[lane] = e0.x;
            s_src[lane] = lane;
        }
        for (int it = 64 + lane; it < ncmp; it += 64) {
            const VocabEntry e = cl[it];
            s_k[it] = e.rk;
            s_t[it] = e.tie;
            s_g[it] = e.g;
            s_x[it] = e.x;
            s_src[it] = it;
        }
        n = ncmp;
    } else {
        // 2b. more entries than the compact list holds: the W-th largest of
        //     the chunk lists' heads bounds the frontier's W-th key from below
        //     (W distinct entries reach it); read the entries of the lists
        //     whose head reaches it
#pragma unroll
        for (int q = 0; q < kHeadsPerLane; ++q) {
            const int c = lane + 64 * q;
            hk[q] = c < C2 ? lists[(int64_t)c * W].rk : -INFINITY;
        }
        uint32_t taken = 0;
        double bound = -INFINITY;
        int found = 0;
        for (int r = 0; r < W; ++r) {
            double lb = -INFINITY;
            int lq = -1;
#pragma unroll
            for (int q = 0; q < kHeadsPerLane; ++q)
                if (!((taken >> q) & 1u) && hk[q] != -INFINITY && (lq < 0 || hk[q] > lb)) {
                    lb = hk[q];
                    lq = q;
                }
            const double wb = wave_max_d(lq >= 0 ? lb : -INFINITY);
            if (wb == -INFINITY) break;
            const int wl = __builtin_ctzll(__ballot(lq >= 0 && lb == wb));
            if (lane == wl) taken |= 1u << lq;
            bound = wb;
            ++found;
        }
        if (found < W) bound = -INFINITY;
        int nq = 0;
#pragma unroll
        for (int q = 0; q < kHeadsPerLane; ++q) {
            const int c = lane + 64 * q;
            const bool qual = c < C2 && hk[q] != -INFINITY && hk[q] >= bound;
            const unsigned long long mq = __ballot(qual);
            if (qual) s_q[nq + lanes_below(mq)] = c;
            nq += __popcll(mq);
        }
        __syncthreads();
        const int items = nq * W;
        for (int it0 = 0; it0 < items; it0 += 64) {
            const int it = it0 + lane;
            double k = -INFINITY;
            uint32_t t = 0xFFFFFFFFu;
            int idx = 0;
            if (it < items) {
                const int qi = it / W, r = it - qi * W;
                idx = s_q[qi] * W + r;
                k = lists[idx].rk;
                t = lists[idx].tie;
            }
            const bool take = k != -INFINITY && k >= bound;
            const unsigned long long m = __ballot(take);
            if (take) {
                const int pos = n + lanes_below(m);
                if (pos < kFrontCap) {
                    s_k[pos] = k;
                    s_t[pos] = t;
                    s_g[pos] = lists[idx].g;
                    s_x[pos] = lists[idx].x;
                    s_src[pos] = pos;
                }
            }
            n += __popcll(m);
        }
    }
    __syncthreads();
    const int nsel = n < W ? n : W;
    if (n <= 256) {
        // each candidate's rank by (Rk desc, tie asc): a count over the
        // others, sixteen broadcast reads at a time
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = lane + 64 * q;
            if (64 * q < n) {
                const int ic = i < n ? i : 0;
                const double ki = s_k[ic];
                const uint32_t ti = s_t[ic];
                int r = 0;
                for (int j0 = 0; j0 < n; j0 += 16) {
                    double kj[16];
                    uint32_t tj[16];
#pragma unroll
                    for (int u = 0; u < 16; ++u) {
                        const int j = j0 + u < n ? j0 + u : ic;          // itself: never before itself
                        kj[u] = s_k[j];
                        tj[u] = s_t[j];
                    }
#pragma unroll
                    for (int u = 0; u < 16; ++u) r += entry_before(kj[u], tj[u], ki, ti);
                }
                if (i < n && r < W) s_win[r] = s_src[i];
            }
        }
    } else if (n <= kFrontCap) {
        // W extractions over the candidates, 16 per lane in registers
        double ck[kFrontCap / 64];
        uint32_t ct[kFrontCap / 64];
#pragma unroll
        for (int q = 0; q < kFrontCap / 64; ++q) {
            const int pos = lane + 64 * q;
            ck[q] = pos < n ? s_k[pos] : -INFINITY;
            ct[q] = pos < n ? s_t[pos] : 0xFFFFFFFFu;
        }
        uint32_t used = 0;
        for (int r = 0; r < nsel; ++r) {
            double bk = -INFINITY;
            uint32_t bt = 0xFFFFFFFFu;
            int bq = -1;
#pragma unroll
            for (int q = 0; q < kFrontCap / 64; ++q)
                if (lane + 64 * q < n && !((used >> q) & 1u) && (bq < 0 || entry_before(ck[q], ct[q], bk, bt))) {
                    bk = ck[q];
                    bt = ct[q];
                    bq = q;
                }
            const double mk = wave_max_d(bq >= 0 ? bk : -INFINITY);
            const bool atk = bq >= 0 && bk == mk;
            const unsigned long long mt = wave_min_u64(atk ? (unsigned long long)bt : ~0ull);
            const int bl = __builtin_ctzll(__ballot(atk && (unsigned long long)bt == mt));
            if (lane == bl) {
                used |= 1u << bq;
                s_win[r] = s_src[lane + 64 * bq];
            }
        }
    } else {
        // many exact ties at the bound: take the best W one at a time
        double pk = INFINITY;
        uint32_t pt = 0u;
        for (int r = 0; r < W; ++r) {
            double bk = -INFINITY;
            uint32_t bt = 0xFFFFFFFFu;
            int bi = -1;
            for (int64_t idx = lane; idx < (int64_t)C2 * W; idx += 64) {
                const double k = lists[idx].rk;
                const uint32_t t = lists[idx].tie;
                if (k == -INFINITY || !entry_before(pk, pt, k, t)) continue;
                if (bi < 0 || entry_before(k, t, bk, bt)) {
                    bk = k;
                    bt = t;
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
            if (lane == 0) s_win[r] = -1 - bi;                          // a list index, not a slot
            pk = bk;
            pt = bt;
        }
    }
    __syncthreads();

    // 3. the new nodes and the next frontier
    const int base = a.t == 1 ? 0 : a.n_tree[b];
    int tok = 0, pnode = -1;
    double rkv = 0.0, sc = 0.0;
    if (lane < nsel) {
        const int w = s_win[lane];
        double ek, eg;
        float ex;
        uint32_t et;
        if (w >= 0) {                                                   // a candidate slot in LDS
            ek = s_k[w];
            et = s_t[w];
            eg = s_g[w];
            ex = s_x[w];
        } else {
            const VocabEntry& e = lists[-1 - w];
            ek = e.rk;
            et = e.tie;
            eg = e.g;
            ex = e.x;
        }
        tok = (int)(et >> 6);
        const int pr = (int)(et & 63u);
        const double ps = a.t == 1 ? 0.0 : s_ps[pr];
        pnode = a.t == 1 ? -1 : s_pn[pr];
        rkv = ek;
        sc = (ps + ((double)ex - lse_t)) + eg;
    }
    if (lane < nsel) {
        const int node = base + lane;
        const int64_t nb = (int64_t)b * a.d * W + node;
        a.nd_tok[nb] = tok;
        a.nd_par[nb] = pnode;
        a.nd_dep[nb] = a.t;
        a.nd_s[nb] = sc;
        a.f_tok[fb + lane] = tok;
        a.f_rk[fb + lane] = rkv;
        a.f_s[fb + lane] = sc;
        a.f_node[fb + lane] = node;
        s_ftok[lane] = tok;
        s_frk[lane] = rkv;
    }
    if (lane == 0) {
        a.f_n[b] = nsel;
        a.n_tree[b] = base + nsel;
    }
    // 4. a lower bound for the next depth's W-th key
    if (a.t < a.d) {
        __syncthreads();
        const int m = lane & 15, kq = lane >> 4;
        float A[KS];
        load_erow<KS>(a, m < nsel ? s_ftok[m] : -1, kq, A);
        const double bnd = nsel > 0 ? seed_bound<KS>(a, sd, nsel, A, s_frk, lane) : -INFINITY;
        if (lane == 0) a.seed[b] = bnd;
    }
}

// |F_v| for every token (the rounding bound of the screen) and F rounded
// to bf16 (the screen's matrix operand), once per call
// (R/4 lanes per row, one 16-byte vector each, so a wave reads and writes
// contiguous memory; the row's sum of squares is reduced across its lanes)
template <int R>
__global__ void __launch_bounds__(kThreads) fnorm_kernel(const float* __restrict__ F, int V, float* __restrict__ out,
                                                         uint16_t* __restrict__ fbf) {
    constexpr int LPR = R / 4;
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t v = gid / LPR;
    const int sub = (int)(gid - v * LPR);
    const bool in = v < V;
    const float4 f = in ? reinterpret_cast<const float4*>(F + v * R)[sub] : make_float4(0.f, 0.f, 0.f, 0.f);
    float s = f.x * f.x + f.y * f.y + f.z * f.z + f.w * f.w;
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) s += __shfl_xor(s, o);
    if (in) {
        reinterpret_cast<uint2*>(fbf + v * R)[sub] = make_uint2(bf16_pair(f.x, f.y), bf16_pair(f.z, f.w));
        if (sub == 0) out[v] = sqrtf(s) * (1.f + 0x1p-20f);
    }
}

}  // namespace

hipError_t launch_fnorm(const float* F, int V, int R, float* out, uint16_t* fbf, hipStream_t stream) {
    const int64_t threads = (int64_t)V * (R / 4);
    const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads)), block(kThreads);
    if (R == 16) hipLaunchKernelGGL(fnorm_kernel<16>, grid, block, 0, stream, F, V, out, fbf);
    else if (R == 32) hipLaunchKernelGGL(fnorm_kernel<32>, grid, block, 0, stream, F, V, out, fbf);
    else if (R == 64) hipLaunchKernelGGL(fnorm_kernel<64>, grid, block, 0, stream, F, V, out, fbf);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

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

hipError_t launch_seed1(const FrontierArgs& a, const int32_t* ctx, hipStream_t stream) {
    if (a.B <= 0) return hipSuccess;
    const dim3 grid((unsigned)a.B), block(64);
    if (a.R == 16) hipLaunchKernelGGL(seed1_kernel<4>, grid, block, 0, stream, a, ctx);
    else if (a.R == 32) hipLaunchKernelGGL(seed1_kernel<8>, grid, block, 0, stream, a, ctx);
    else if (a.R == 64) hipLaunchKernelGGL(seed1_kernel<16>, grid, block, 0, stream, a, ctx);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_frontier(const FrontierArgs& a, hipStream_t stream) {
    if (a.B <= 0) return hipSuccess;
    const dim3 grid((unsigned)a.B), block(64);
    if (a.R == 16) hipLaunchKernelGGL(frontier_kernel<4>, grid, block, 0, stream, a);
    else if (a.R == 32) hipLaunchKernelGGL(frontier_kernel<8>, grid, block, 0, stream, a);
    else if (a.R == 64) hipLaunchKernelGGL(frontier_kernel<16>, grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace dt
