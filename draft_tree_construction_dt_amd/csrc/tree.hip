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
#include "common.h"
#include "wave.h"

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

// ---------------------------------------------------------------------------
// one wave merges the L partial lists of one row
// ---------------------------------------------------------------------------
__device__ void merge_row(const float* __restrict__ part_m, const double* __restrict__ part_s,
                          const unsigned long long* __restrict__ part_keys, int64_t row, int L, int k,
                          unsigned long long* scratch, int lane, double* lse_out, int* tok_out,
                          float* val_out) {
    const float* pm = part_m + row * L;
    const double* ps = part_s + row * L;
    const unsigned long long* keys = part_keys + row * (int64_t)L * k;
    const int n = L * k;
    // all loads of the row are independent: issue them together
    float mc[4];
    double sc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = lane + 64 * q;
        mc[q] = c < L ? pm[c] : -INFINITY;
        sc[q] = c < L ? ps[c] : 0.0;
    }
    unsigned long long kv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        kv[q] = e < n ? keys[e] : 0ull;
    }

    // normaliser: max and rescaled sum over the lists, log in fp64
    const float M = wave_max_f32(fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3])));
    double sum = 0.0;
    if (M != -INFINITY) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (mc[q] != -INFINITY) sum += sc[q] * (double)__builtin_amdgcn_exp2f((mc[q] - M) * 1.4426950408889634f);
    }
    sum = wave_add_f64(sum);
    if (lane == 0) {
        // the true normaliser is >= the row max; clamp the rounding of a sum
        // whose largest term is 1 so that every log-probability stays <= 0
        const double l = log(sum);
        *lse_out = (M == -INFINITY) ? -INFINITY : (double)M + (l > 0.0 ? l : 0.0);
    }

    // top-k.  Lower bounds for the row's k-th key, both from k distinct keys:
    // the k-th key of any full list, and the q-th key of every list holding
    // q = ceil(k/L) keys when there are enough such lists.
    const int q = (k + L - 1) / L;
    unsigned long long bk = 0ull, bq = ~0ull;
    int nq = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int e = lane + 64 * r;
        if (e < n) {
            const int i = e % k;
            if (i == k - 1) bk = kv[r] > bk ? kv[r] : bk;
            if (i == q - 1 && kv[r] != 0ull) {
                bq = kv[r] < bq ? kv[r] : bq;
                ++nq;
            }
        }
    }
    bk = wave_max_u64(bk);
    bq = wave_min_u64(bq);
    nq = wave_add_i32(nq);
    unsigned long long th = bk;
    if (nq * q >= k && bq > th) th = bq;
    int ns = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool keep = kv[r] != 0ull && kv[r] >= th;
        const unsigned long long bal = __ballot(keep);
        if (keep) scratch[ns + lanes_below(bal)] = kv[r];
        ns += __popcll(bal);
    }
    // pad to a multiple of eight with empty keys (0 is below every key)
    const int ns8 = (ns + 7) & ~7;
    if (lane < ns8 - ns) scratch[ns + lane] = 0ull;
    __builtin_amdgcn_wave_barrier();
    // rank: lane e holds survivor e (blocks of 64) and streams past all of
    // them, eight independent broadcast reads per step (keys are unique)
    for (int e0 = 0; e0 < ns; e0 += 64) {
        const int e = e0 + lane;
        const unsigned long long v = e < ns ? scratch[e] : ~0ull;
        int rank = 0;
        for (int j = 0; j < ns8; j += 8) {
            unsigned long long o[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) o[u] = scratch[j + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) rank += o[u] > v;
        }
        if (e < ns && rank < k) {
            tok_out[rank] = (int)key_id(v);
            val_out[rank] = key_value(v);
        }
    }
    __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// continuity
// ---------------------------------------------------------------------------
// Children of one depth by token: an open-addressing table in LDS
// (kChildSlots slots, load <= 1/4) maps a token to its index in T_{t-1}.
constexpr int kChildSlots = 128;
__device__ __forceinline__ uint32_t child_hash(int tok) { return ((uint32_t)tok * 2654435761u) >> 25; }

// Index in T_{t-1} of token s, or -1.
__device__ __forceinline__ int child_index(const int* ctok, const int* cj, int s) {
    if (s < 0) return -1;
    uint32_t pos = child_hash(s);
    for (int probe = 0; probe < kChildSlots; ++probe) {
        const int t = ctok[pos];
        if (t == s) return cj[pos];
        if (t == -1) return -1;
        pos = (pos + 1) & (kChildSlots - 1);
    }
    return -1;
}

// OR over the four lanes of a quad (DPP quad permutations, no LDS traffic)
__device__ __forceinline__ uint32_t quad_or(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    return v;
}

// Successors 4g .. 4g+3 of a 16-wide chunk of a row (-1 past its end):
// one 16-byte load when the row allows it.
__device__ __forceinline__ void load_succ4(int (&r)[4], const int* row, int from, int n) {
    typedef int i4 __attribute__((ext_vector_type(4)));
    const int* p = row + from;
    if (from + 4 <= n && ((uintptr_t)p & 15u) == 0) {
        const i4 x = *reinterpret_cast<const i4*>(p);
        r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) r[u] = from + u < n ? p[u] : -1;
    }
}

// Admissible children of the trigram context (a2, a1), computed by the four
// lanes of a quad together (g = lane & 3): lane g probes slots 2g and 2g+1 of
// every window of 8 probe positions and holds successors 4g..4g+3 of every 16
// of the row, and each successor is mapped to its child index through the
// LDS table.  The first window and the home slot's row are read at once, so a
// key found in its home slot costs one memory round trip.  Inactive quads
// (`active` false in all four lanes) read in bounds and return 0.  The
// result is the same in all four lanes.
__device__ uint32_t quad_admitted(const NGramArgs& a, int a2, int a1, bool active, int g,
                                  const int* ctok, const int* cj, uint32_t live) {
    const unsigned long long key = ((unsigned long long)(uint32_t)a2 << 32) | (uint32_t)a1;
    const long long cm = a.cap - 1;
    const long long home = active ? (long long)(mix64(key) & (unsigned long long)cm) : 0;
    const int S = a.S;
    // trip 1: probe window 0 and the first 16 successors of the home slot
    unsigned long long k0 = a.keys[(home + 2 * g) & cm], k1 = a.keys[(home + 2 * g + 1) & cm];
    int spec[4];
    load_succ4(spec, a.succ + home * S, 4 * g, S);
    long long slot = -1;
    bool done = !active;
    for (long long w0 = 0; !done; w0 += 8) {
        if (w0 > 0) {
            k0 = a.keys[(home + w0 + 2 * g) & cm];
            k1 = a.keys[(home + w0 + 2 * g + 1) & cm];
        }
        // probe order within the window: slot 2g + e of lane g
        const uint32_t hitm = (uint32_t)(k0 == key) | ((uint32_t)(k1 == key) << 1);
        const uint32_t endm = hitm | (uint32_t)(k0 == kEmptyKey) | ((uint32_t)(k1 == kEmptyKey) << 1);
        const uint32_t F = quad_or(endm << (2 * g)), M = quad_or(hitm << (2 * g));
        if (F != 0u) {
            const int idx = __builtin_ctz(F);
            if ((M >> idx) & 1u) slot = (home + w0 + idx) & cm;
            done = true;
        } else if (w0 + 8 >= a.cap) {
            done = true;                                      // every slot seen: absent
        }
    }
    if (slot < 0) return 0u;
    const bool membership = a.min_logp == -INFINITY || a.hash_logp == nullptr;
    const int* row = a.succ + slot * S;
    uint32_t hit = 0;
    for (int c0 = 0; c0 < S; c0 += 16) {
        int sv[4];
        if (c0 == 0 && slot == home) {
#pragma unroll
            for (int u = 0; u < 4; ++u) sv[u] = spec[u];
        } else {
            load_succ4(sv, row, c0 + 4 * g, S);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = child_index(ctok, cj, sv[u]);
            if (j >= 0 && (membership || a.hash_logp[slot * S + c0 + 4 * g + u] > a.min_logp)) hit |= 1u << j;
        }
    }
    return quad_or(hit) & live;
}

// Admissible children after the bigram context a1, by the four lanes of a
// quad (g = lane & 3): a dense row is read at the children's columns (lane g
// takes children g, g+4, ...); a CSR row is read 64 successors per round
// trip (lane g takes 4g..4g+3 of every 16), each mapped to its child index
// through the LDS token table.  Inactive quads and ids outside [0, V) admit
// nothing.  The result is the same in all four lanes.
__device__ uint32_t quad_admitted_bigram(const NGramArgs& a, int a1, bool active, int g, const int* ch,
                                         const int* ctok, const int* cj, uint32_t live, int k) {
    if (!active || a1 < 0 || a1 >= a.V) return 0u;               // the same in the whole quad
    uint32_t hit = 0;
    if (a.kind == DT_NGRAM_DENSE_BIGRAM) {
        const float* row = a.dense + (int64_t)a1 * a.V;
        float v[kMaxK / 4];
#pragma unroll
        for (int u = 0; u < kMaxK / 4; ++u) {
            const int j = g + 4 * u;
            v[u] = j < k ? row[ch[j]] : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < kMaxK / 4; ++u) {
            const int j = g + 4 * u;
            if (j < k && v[u] > a.min_logp) hit |= 1u << j;
        }
    } else {
        const int lo = a.row_ptr[a1], hi = a.row_ptr[a1 + 1];
        const bool membership = a.min_logp == -INFINITY || a.csr_logp == nullptr;
        for (int e0 = lo; e0 < hi; e0 += 64) {
            int sv[16];
            float lp[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int e = e0 + 16 * (u >> 2) + 4 * g + (u & 3);
                sv[u] = e < hi ? a.col[e] : -1;
                lp[u] = (!membership && e < hi) ? a.csr_logp[e] : INFINITY;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int j = child_index(ctok, cj, sv[u]);
                if (j >= 0 && (membership || lp[u] > a.min_logp)) hit |= 1u << j;
            }
        }
    }
    return quad_or(hit) & live;
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
// budget: (S desc, depth asc, BFS index asc); BFS index order implies depth order
__device__ __forceinline__ bool node_before(double s_a, int i_a, double s_b, int i_b) {
    return s_a > s_b || (s_a == s_b && i_a < i_b);
}

__device__ __forceinline__ double readlane_d(double v, int l) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFFll), l);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// a ranked candidate of the depth loop: key (Rk, tie) and its slot
struct __align__(16) SurvKey {
    double rk;
    uint32_t tie;
    uint32_t j;           // index of the child in T_{t-1}
};
// what a winner needs besides its key: cumulative score and the continuity
// mask of its own children's context
struct __align__(16) SurvAux {
    double s;
    uint32_t cm;
    uint32_t pad;
};
// a frontier node as the next depth reads it: key, score, the continuity
// mask of its children's context and its index in its own T list
struct __align__(16) NodeRec {
    double rk;
    double s;
    uint32_t cm;
    uint32_t tidx;
};

template <typename T>
__device__ __forceinline__ T* lds_at(unsigned char* base, int off) {
    return reinterpret_cast<T*>(base + off);
}

// exclusive prefix sum over the workgroup (one value per thread); tmp holds kTreeWaves ints
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
    for (int w = 0; w < kTreeWaves; ++w) {
        if (w < wave) before += tmp[w];
        all += tmp[w];
    }
    __syncthreads();
    *total = all;
    return before + x - v;
}

// ---------------------------------------------------------------------------
// prep: rows, continuity and parent-conditioned terms of one depth
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) prep_kernel(PrepArgs a) {
    __shared__ unsigned long long s_scratch[kPrepRows][kMergeKeysPerRow + 8];
    __shared__ int s_tok[kPrepRows][kMaxK];
    __shared__ float s_x[kPrepRows][kMaxK];
    __shared__ double s_lse[kPrepRows];
    __shared__ int s_ctok[kChildSlots];
    __shared__ int s_cj[kChildSlots];
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

// Steps 5 and 6 on a candidate tree of nb nodes held in LDS in BFS order
// (tokens, parents as node indices, depths, cumulative scores).  `literal`
// replays best-first one node at a time (scores may rise along a path);
// otherwise S never rises along a path and the top-budget nodes by (S desc,
// BFS index asc) are already closed under parents.
struct EmitOut {
    int32_t* n_nodes;
    int32_t* tokens;
    int32_t* parents;
    int32_t* depths;
    float* scores;
    uint32_t* mask;
    int budget;
    int mask_words;
};

__device__ __forceinline__ void budget_and_emit(int nb, bool literal, int b, const int* n_tok, const int* n_par,
                                                const int* n_dep, const double* n_s, int* n_new, int* n_out,
                                                int* misc, const EmitOut& eo) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int budget = eo.budget;
    // ---- 5. verification budget
    int n_sel = nb;
    if (nb <= budget) {
        for (int i = tid; i < nb; i += kTreeThreads) {
            n_new[i] = i;
            n_out[i] = i;
        }
        __syncthreads();
    } else if (!literal) {
        // parent-closed top-budget by (S desc, BFS index asc)
        const int per = (nb + kTreeThreads - 1) / kTreeThreads;
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
        int pos = block_exclusive_scan(cntl, misc + 16, &total);
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
        for (int i = tid; i < nb; i += kTreeThreads) n_new[i] = (n_par[i] < 0) ? -2 : -3;  // -2 available, -3 waiting
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
        const int per = (nb + kTreeThreads - 1) / kTreeThreads;
        int cntl = 0;
        for (int q = 0; q < per; ++q) {
            const int i = tid * per + q;
            if (i < nb && n_new[i] == -1) ++cntl;
        }
        int total;
        int pos = block_exclusive_scan(cntl, misc + 16, &total);
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

    // ---- 6. outputs in BFS order, parents remapped, ancestor mask
    const int64_t ob = (int64_t)b * budget;
    for (int o = tid; o < budget; o += kTreeThreads) {
        if (o < n_sel) {
            const int i = n_out[o];
            eo.tokens[ob + o] = n_tok[i];
            eo.parents[ob + o] = n_par[i] < 0 ? -1 : n_new[n_par[i]];
            eo.depths[ob + o] = n_dep[i];
            eo.scores[ob + o] = (float)n_s[i];
        } else {
            eo.tokens[ob + o] = -1;
            eo.parents[ob + o] = -1;
            eo.depths[ob + o] = 0;
            eo.scores[ob + o] = -INFINITY;
        }
    }
    const int words = eo.mask_words;
    if (budget * words > kTreeThreads && words <= 8) {
        // more (node, word) pairs than threads: one thread per node walks its
        // ancestors once and sets their bits in all its words
        for (int o = tid; o < budget; o += kTreeThreads) {
            uint32_t a0 = 0, a1 = 0, a2 = 0, a3 = 0, a4 = 0, a5 = 0, a6 = 0, a7 = 0;
            if (o < n_sel) {
                for (int i = n_out[o]; i >= 0; i = n_par[i]) {
                    const int ni = n_new[i];
                    const uint32_t bit = 1u << (ni & 31), wd = (uint32_t)ni >> 5;
                    a0 |= wd == 0 ? bit : 0u;
                    a1 |= wd == 1 ? bit : 0u;
                    a2 |= wd == 2 ? bit : 0u;
                    a3 |= wd == 3 ? bit : 0u;
                    a4 |= wd == 4 ? bit : 0u;
                    a5 |= wd == 5 ? bit : 0u;
                    a6 |= wd == 6 ? bit : 0u;
                    a7 |= wd == 7 ? bit : 0u;
                }
            }
            uint32_t* row = eo.mask + (ob + o) * words;
            row[0] = a0;
            if (words > 1) row[1] = a1;
            if (words > 2) row[2] = a2;
            if (words > 3) row[3] = a3;
            if (words > 4) row[4] = a4;
            if (words > 5) row[5] = a5;
            if (words > 6) row[6] = a6;
            if (words > 7) row[7] = a7;
        }
    } else {
        for (int e = tid; e < budget * words; e += kTreeThreads) {
            const int o = e / words, w = e - o * words;
            uint32_t bits = 0;
            if (o < n_sel) {
                for (int i = n_out[o]; i >= 0; i = n_par[i]) {
                    const int ni = n_new[i];
                    if ((ni >> 5) == w) bits |= 1u << (ni & 31);
                }
            }
            eo.mask[ob * words + e] = bits;
        }
    }
    if (tid == 0) eo.n_nodes[b] = n_sel;
}

template <int RM>
__global__ void __launch_bounds__(kTreeThreads) tree_kernel(TreeArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const TreePlan& P = a.plan;
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
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
    NodeRec* n_rec = lds_at<NodeRec>(lds, P.off_n_rec);
    SurvKey* sv_key = lds_at<SurvKey>(lds, P.off_sv_key);
    SurvAux* sv_aux = lds_at<SurvAux>(lds, P.off_sv_s);
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

    // ---- 4. depth loop, run by wave 0 alone (wave-synchronous, no barriers).
    //      Candidate slot r*64 + lane = parent_rank * k + child.  Every phase
    //      issues its LDS reads together, so a depth costs a few LDS round
    //      trips: (a) the candidates read the child's logit and token and
    //      the parent's 32-byte frontier record; (b) the candidates that can
    //      still win fetch the continuity mask of their own children's
    //      context and are packed (with a full frontier only keys that reach
    //      the smallest "first valid child" key of the W parents can be among
    //      the top W: those W candidates are distinct); (c) ranks among the
    //      survivors: up to 32 of them are compared all-pairs, each lane
    //      taking a few rotations of a replicated copy and the replicas'
    //      counts summed with lane shuffles; more are streamed sixteen at a
    //      time.  Winners write their records in parallel.
    int nb = 0;       // nodes in the candidate tree
    if (wave == 0) {
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        int f = 1;        // frontier size (depth 0: the root)
        int fbase = 0;    // BFS index of the first frontier node
        const uint32_t root_mask = kind == DT_NGRAM_NONE ? 0xFFFFFFFFu : s_vmask[0];
        const float inv_k = 1.0f / (float)k;
        // per-depth constants, lane t-1 holding depth t's: normaliser and the
        // mask of children with a finite logit
        const double lse_l = lane < d ? s_lse[lane] : 0.0;
        uint32_t live_l = 0;
        if (lane < d)
            for (int j = 0; j < k; ++j) live_l |= (uint32_t)(s_tx[lane * k + j] != -INFINITY) << j;
        // a lane's candidate slots have fixed (parent rank, child) pairs
        int cj[RM], cp[RM];
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            const int slot = r * 64 + lane;
            const int sl = slot < kMaxCandidates ? slot : 0;
            cp[r] = (int)(((float)sl + 0.5f) * inv_k);         // exact: slot < 2^11
            cj[r] = sl - cp[r] * k;
        }
        for (int t = 1; t <= d; ++t) {
            const int tk = (t - 1) * k;
            const int m = f * k;
            const double lse_t = readlane_d(lse_l, t - 1);
            const uint32_t live = (uint32_t)__builtin_amdgcn_readlane((int)live_l, t - 1);
            const bool next_ctx = kind != DT_NGRAM_NONE && t < d;
            // (a) one batch of LDS reads for all rounds; indices are clamped so
            //     every read is in bounds and no read waits on a branch
            int ctok[RM];
            float cx[RM];
            u4 crec[RM];
            u2 crec2[RM];
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                const int nd = (t > 1 && r * 64 + lane < m) ? fbase + cp[r] : 0;
                cx[r] = s_tx[tk + cj[r]];
                ctok[r] = s_ttok[tk + cj[r]];
                crec[r] = *reinterpret_cast<const u4*>(&n_rec[nd]);
                crec2[r] = *reinterpret_cast<const u2*>(&n_rec[nd].cm);
            }
            double krk[RM], ksc[RM];
            uint32_t ktie[RM];
            bool kok[RM];
            int kgp[RM];
            int nvalid = 0, nfirst = 0;
            double firstmin = INFINITY;
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                const int slot = r * 64 + lane;
                const int j = cj[r];
                const bool root = t == 1;
                const double prk = root ? 0.0 : __longlong_as_double(((long long)crec[r].y << 32) | crec[r].x);
                const double ps = root ? 0.0 : __longlong_as_double(((long long)crec[r].w << 32) | crec[r].z);
                const uint32_t cm = root ? root_mask : crec2[r].x;
                kgp[r] = root ? 0 : (int)crec2[r].y;
                const uint32_t rowv = cm & live;
                const bool ok = slot < m && ((rowv >> j) & 1u);
                const bool first = ok && j == __builtin_ctz(rowv);
                const double g = (dartree && ok) ? s_g[(tk + kgp[r]) * k + j] : 0.0;
                krk[r] = ok ? (prk + (double)cx[r]) + g : -INFINITY;
                ksc[r] = ok ? (ps + ((double)cx[r] - lse_t)) + g : -INFINITY;
                ktie[r] = ok ? (((uint32_t)ctok[r] << 6) | (uint32_t)cp[r]) : 0xFFFFFFFFu;
                if (first) firstmin = fmin(firstmin, krk[r]);
                kok[r] = ok;
                nvalid += __popcll(__ballot(ok));
                nfirst += __popcll(__ballot(first));
            }
            if (nvalid == 0) break;
            const int keep = nvalid < W ? nvalid : W;
            // (b) survivors, each with the continuity mask of its children's
            //     context (read before the reduction, so the two overlap)
            uint32_t kcm[RM];
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                kcm[r] = 0xFFFFFFFFu;
                if (next_ctx) {
                    const int ci = kok[r] ? ctx_index(kind, k, t + 1, t == 1 ? 0 : kgp[r], cj[r]) : 0;
                    kcm[r] = s_vmask[ci];
                }
            }
            double lb = nfirst >= W ? wave_min_f64(firstmin) : -INFINITY;
            // With many candidates above that bound (no continuity filter, or
            // a parent term that reorders a parent's children), tighten it:
            // the W-th largest of the lanes' best keys, each rounded down to
            // fp32, is reached by W distinct candidates, so it bounds the
            // depth's W-th key from below too.  Found bit by bit with ballots
            // over the order-preserving bits of the rounded values.
            int nin = 0;
#pragma unroll
            for (int r = 0; r < RM; ++r) nin += __popcll(__ballot(kok[r] && krk[r] >= lb));
            if (nin > 32) {
                double lm = -INFINITY;
#pragma unroll
                for (int r = 0; r < RM; ++r)
                    if (kok[r]) lm = fmax(lm, krk[r]);
                const uint32_t u = ord_bits(__float_as_uint(__double2float_rd(lm) + 0.0f));
                uint32_t th = 0;
                for (int bit = 31; bit >= 0; --bit) {
                    const uint32_t c = th | (1u << bit);
                    if (__popcll(__ballot(u >= c)) >= W) th = c;
                }
                lb = fmax(lb, (double)__uint_as_float(unord_bits(th)));
            }
            int ns = 0;
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                const bool in = kok[r] && krk[r] >= lb;
                const unsigned long long bal = __ballot(in);
                if (in) {
                    const int e = ns + lanes_below(bal);
                    sv_key[e] = SurvKey{krk[r], ktie[r], (uint32_t)cj[r]};
                    sv_aux[e] = SurvAux{ksc[r], kcm[r], 0u};
                }
                ns += __popcll(bal);
            }
            // sentinels (Rk = -inf beats nothing) round the list up to a
            // multiple of 32
            const int ns32 = (ns + 31) & ~31;
            if (lane < ns32 - ns) sv_key[ns + lane] = SurvKey{-INFINITY, 0xFFFFFFFFu, 0u};
            __builtin_amdgcn_wave_barrier();
            // (c) ranks
            if (ns <= 32) {
                // G lanes per replica, 64/G replicas; lane (rep, i) compares
                // survivor i with survivors i+s (mod G), s = 1 + rep + u*64/G
                const int G = ns <= 16 ? 16 : 32;
                const int F = 64 / G;
                const int i = lane & (G - 1), rep = lane / G;
                const SurvKey me = sv_key[i];
                const SurvAux ax = sv_aux[i];
                int part = 0;
                for (int s0 = 1 + rep; s0 < G; s0 += 4 * F) {
                    u4 o[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int sh = s0 + u * F;
                        o[u] = *reinterpret_cast<const u4*>(&sv_key[(i + (sh < G ? sh : 0)) & (G - 1)]);
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int sh = s0 + u * F;
                        const double ork = __longlong_as_double(((long long)o[u].y << 32) | o[u].x);
                        part += (sh < G) & ((ork > me.rk) | ((ork == me.rk) & (o[u].z < me.tie)));
                    }
                }
                if (G == 16) part += __shfl_xor(part, 16);
                part += __shfl_xor(part, 32);
                if (rep == 0 && i < ns && part < keep) {
                    const int nd = nb + part;
                    n_tok[nd] = (int)(me.tie >> 6);
                    n_par[nd] = t == 1 ? -1 : fbase + (int)(me.tie & 63u);
                    n_dep[nd] = t;
                    n_s[nd] = ax.s;
                    n_rec[nd] = NodeRec{me.rk, ax.s, ax.cm, me.j};
                }
            } else {
                // lane e holds survivor e (blocks of 64) and streams past all
                for (int e0 = 0; e0 < ns; e0 += 64) {
                    const int e = e0 + lane;
                    const int ec = e < ns ? e : 0;
                    const SurvKey me = sv_key[ec];
                    const SurvAux ax = sv_aux[ec];
                    int rank = 0;
                    for (int q = 0; q < ns32; q += 16) {
                        u4 o[16];
#pragma unroll
                        for (int u = 0; u < 16; ++u) o[u] = *reinterpret_cast<const u4*>(&sv_key[q + u]);
#pragma unroll
                        for (int u = 0; u < 16; ++u) {
                            const double ork = __longlong_as_double(((long long)o[u].y << 32) | o[u].x);
                            rank += (ork > me.rk) | ((ork == me.rk) & (o[u].z < me.tie));
                        }
                    }
                    if (e < ns && rank < keep) {
                        const int nd = nb + rank;
                        n_tok[nd] = (int)(me.tie >> 6);
                        n_par[nd] = t == 1 ? -1 : fbase + (int)(me.tie & 63u);
                        n_dep[nd] = t;
                        n_s[nd] = ax.s;
                        n_rec[nd] = NodeRec{me.rk, ax.s, ax.cm, me.j};
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
            fbase = nb;
            nb += keep;
            f = keep;
        }
        if (lane == 0) misc[0] = nb;
    }
    __syncthreads();
    nb = misc[0];                                            // ordered by the barrier

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

hipError_t launch_tree(const TreeArgs& a, hipStream_t stream) {
    if (a.B <= 0) return hipSuccess;
    const int m = a.W * a.k;
    if (m <= 128)
        hipLaunchKernelGGL(tree_kernel<2>, dim3((unsigned)a.B), dim3(kTreeThreads), (size_t)a.plan.total, stream, a);
    else if (m <= 256)
        hipLaunchKernelGGL(tree_kernel<4>, dim3((unsigned)a.B), dim3(kTreeThreads), (size_t)a.plan.total, stream, a);
    else
        hipLaunchKernelGGL(tree_kernel<16>, dim3((unsigned)a.B), dim3(kTreeThreads), (size_t)a.plan.total, stream, a);
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
