// Device code of the tree step (the prep, tree and merge kernels of
// tree.hip): the row merge, the N-gram continuity lookups, the depth loop
// (frontier-wide top-W), the verification budget and the output stage.  The
// algorithm is described at the top of tree.hip.
#pragma once

#include "common.h"
#include "wave.h"

namespace dt {
namespace treedev {
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
__device__ __forceinline__ void merge_row(const float* __restrict__ part_m, const double* __restrict__ part_s,
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
    const float M = wave_max_f32_all(max_f(max_f(mc[0], mc[1]), max_f(mc[2], mc[3])));
    double sum = 0.0;
    if (M != -INFINITY) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (mc[q] != -INFINITY) sum += sc[q] * (double)__builtin_amdgcn_exp2f((mc[q] - M) * 1.4426950408889634f);
    }
    sum = wave_add_f64_all(sum);
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
    bk = wave_max_u64_all(bk);
    bq = wave_min_u64_all(bq);
    nq = wave_add_i32_all(nq);
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
__device__ __forceinline__ uint32_t quad_admitted(const NGramArgs& a, int a2, int a1, bool active, int g,
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
__device__ __forceinline__ uint32_t quad_admitted_bigram(const NGramArgs& a, int a1, bool active, int g, const int* ch,
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
// a node of the candidate tree: the next depth reads its key, score, the
// continuity mask of its children's context and its index in its own T list
// (the first 24 bytes); the output stage reads its token, parent and depth
struct __align__(16) NodeRec {
    double rk;
    double s;
    uint32_t cm;
    uint32_t tj;          // index in its own T list | depth << 8
    int32_t tok;
    int32_t par;          // BFS index of the parent, -1 at depth 1
};

// High word of the order-preserving 64-bit image of a double (sign bit
// flipped for values >= +0, all bits inverted below): monotone in the
// value, so the double whose image is (o, 0) is at most every value whose
// high word is >= o.
__device__ __forceinline__ uint32_t ord_hi(double x) {
    const uint32_t h = (uint32_t)((uint64_t)__double_as_longlong(x) >> 32);
    return h ^ ((uint32_t)((int32_t)h >> 31) | 0x80000000u);
}
__device__ __forceinline__ double ord_hi_floor(uint32_t o) {
    const uint32_t h = (o & 0x80000000u) ? (o ^ 0x80000000u) : ~o;
    const uint32_t l = (o & 0x80000000u) ? 0u : 0xFFFFFFFFu;
    return __longlong_as_double((long long)(((uint64_t)h << 32) | l));
}

template <typename T>
__device__ __forceinline__ T* lds_at(unsigned char* base, int off) {
    return reinterpret_cast<T*>(base + off);
}

// exclusive prefix sum over the workgroup (one value per thread); tmp holds kTreeWaves ints
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
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

// The largest t with its bits below LOW clear such that at least W lanes
// hold u >= t, found bit by bit with ballots (fully unrolled).
template <int LOW>
__device__ __forceinline__ uint32_t wave_kth_high(uint32_t u, int W) {
    uint32_t th = 0;
#pragma unroll
    for (int bit = 31; bit >= LOW; --bit) {
        const uint32_t c = th | (1u << bit);
        if (__popcll(__ballot(u >= c)) >= W) th = c;
    }
    return th;
}

// 1 if the survivor held SH lanes away within the 16-lane row (DPP
// row_ror:SH of the (key low, key high, tie) words) ranks before (rk, tie).
template <int SH>
__device__ __forceinline__ int beats_rotated(uint32_t lo, uint32_t hi, uint32_t tie, double rk, uint32_t mytie) {
    // (a rotation inside the row reads a lane of the row for every lane, so
    // the moves need no initial value)
    const uint32_t l = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo, 0x120 + SH, 0xF, 0xF, false);
    const uint32_t h = (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, 0x120 + SH, 0xF, 0xF, false);
    const uint32_t t = (uint32_t)__builtin_amdgcn_mov_dpp((int)tie, 0x120 + SH, 0xF, 0xF, false);
    const double ork = __longlong_as_double((long long)(((uint64_t)h << 32) | l));
    return (ork > rk) | ((ork == rk) & (t < mytie));
}

// Step 4 for one request whose per-row data (normalisers, top-k lists,
// continuity masks and, in DARTree mode, parent-conditioned terms) are in
// shared memory at plan P: the depth loop, run by wave 0 alone, leaving the
// candidate tree (n_tok, n_par, n_dep, n_s in BFS order) in shared memory.
// DTREE: the parent-conditioned term is added; NG: continuity masks apply
// (trigram contexts when `trigram`, else bigram).  Every thread of the
// workgroup must call it; returns the number of nodes.
template <int RM, bool DTREE, bool NG>
__device__ __forceinline__ int depth_loop(const TreePlan& P, unsigned char* lds, int d, int k, int W,
                                          bool trigram) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const double* s_lse = lds_at<double>(lds, P.off_lse);
    const int* s_ttok = lds_at<int>(lds, P.off_ttok);
    const float* s_tx = lds_at<float>(lds, P.off_tx);
    const uint32_t* s_vmask = lds_at<uint32_t>(lds, P.off_vmask);
    const double* s_g = lds_at<double>(lds, P.off_g);
    int* n_tok = lds_at<int>(lds, P.off_n_tok);
    int* n_par = lds_at<int>(lds, P.off_n_par);
    int* n_dep = lds_at<int>(lds, P.off_n_dep);
    NodeRec* n_rec = lds_at<NodeRec>(lds, P.off_n_rec);
    SurvKey* sv_key = lds_at<SurvKey>(lds, P.off_sv_key);
    SurvAux* sv_aux = lds_at<SurvAux>(lds, P.off_sv_s);
    double* n_s = lds_at<double>(lds, P.off_n_s);
    int* misc = lds_at<int>(lds, P.off_misc);
    const int nn = P.max_nodes;                  // the root's record sits at n_rec[nn]
    // ---- 4. depth loop, run by wave 0 alone (wave-synchronous, no barriers).
    //      Candidate slot r*64 + lane = parent_rank * k + child.  A depth
    //      costs a few rounds of shared-memory reads: (a) every candidate
    //      reads the child's logit and token and the parent's record, then
    //      what depends on the parent's T index (the parent-conditioned term,
    //      the continuity mask of its own children's context); (b) with a
    //      full frontier only keys that reach the smallest "first valid
    //      child" key of the W parents can be among the top W (those W
    //      candidates are distinct), and those survivors are packed; (c) ranks
    //      among the survivors: up to 32 of them are compared all-pairs, each
    //      lane taking a few rotations of a replicated copy and the replicas'
    //      counts summed with lane permutes; more are streamed sixteen at a
    //      time.  Winners write their 32-byte records in parallel.
    int nb = 0;       // nodes in the candidate tree
    if (wave == 0) {
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        if (lane == 0) n_rec[nn] = NodeRec{0.0, 0.0, NG ? s_vmask[0] : 0xFFFFFFFFu, 0u, -1, -1};
        int f = 1;        // frontier size (depth 0: the root)
        int fbase = 0;    // BFS index of the first frontier node
        const float inv_k = 1.0f / (float)k;
        // per-depth constants, lane t-1 holding depth t's: normaliser and the
        // mask of children with a finite logit
        const double lse_l = lane < d ? s_lse[lane] : 0.0;
        uint32_t live_l = 0;
        if (lane < d)
            for (int j = 0; j < k; ++j) live_l |= (uint32_t)(s_tx[lane * k + j] != -INFINITY) << j;
        // a lane's candidate slots have fixed (parent rank, child) pairs
        int cj[RM], cp[RM];
        uint32_t below[RM];   // the children ranked before cj in T
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            const int slot = r * 64 + lane;
            const int sl = slot < kMaxCandidates ? slot : 0;
            cp[r] = (int)(((float)sl + 0.5f) * inv_k);         // exact: slot < 2^11
            cj[r] = sl - cp[r] * k;
            below[r] = (1u << cj[r]) - 1u;                     // cj < 32
        }
        __builtin_amdgcn_wave_barrier();
        // where a depth's candidates' own children's contexts start, stepped
        // instead of recomputed
        int cbase = 1;
        const int kk = k * k;
        for (int t = 1; t <= d; ++t) {
            const int tk = (t - 1) * k;
            const int m = f * k;
            const int rb = t == 1 ? nn : fbase;          // the parents' records
            const int pbase = t == 1 ? -1 : fbase;       // parent index = pbase + parent rank
            const double lse_t = readlane_d(lse_l, t - 1);
            const uint32_t live = (uint32_t)__builtin_amdgcn_readlane((int)live_l, t - 1);
            // context of a depth-t candidate's own children (depth t + 1):
            // cbase + (parent's T index) * cstride + child index
            const bool next_ctx = NG && t < d;
            const int cstride = (trigram && t > 1) ? k : 0;
            // (a) one batch of reads for all rounds, then the reads that
            //     depend on the parent's T index; indices are clamped so every
            //     read is in bounds and none waits on a branch
            int ctok[RM];
            float cx[RM];
            u4 crec[RM];
            u2 crec2[RM];
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                const int nd = r * 64 + lane < m ? rb + cp[r] : rb;
                cx[r] = s_tx[tk + cj[r]];
                ctok[r] = s_ttok[tk + cj[r]];
                crec[r] = *reinterpret_cast<const u4*>(&n_rec[nd]);
                crec2[r] = *reinterpret_cast<const u2*>(&n_rec[nd].cm);
            }
            double gv[RM];
            uint32_t kcm[RM];
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                const int kgp = (int)(crec2[r].y & 0xFFu);
                gv[r] = DTREE ? s_g[(tk + kgp) * k + cj[r]] : 0.0;
                if (NG) {
                    // (operands below 2^8: the 24-bit multiply is exact and full rate)
                    const int ci = cbase + (int)__umul24((uint32_t)kgp, (uint32_t)cstride) + cj[r];
                    const uint32_t v = s_vmask[next_ctx ? ci : 0];
                    kcm[r] = next_ctx ? v : 0xFFFFFFFFu;
                } else {
                    kcm[r] = 0xFFFFFFFFu;
                }
            }
            double krk[RM], ksc[RM];
            uint32_t ktie[RM];
            int nvalid = 0, nfirst = 0;
            uint32_t fmin = 0xFFFFFFFFu;    // smallest ordered high word of a first-valid key
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                const double prk = __longlong_as_double(((long long)crec[r].y << 32) | crec[r].x);
                const double ps = __longlong_as_double(((long long)crec[r].w << 32) | crec[r].z);
                const uint32_t rowv = NG ? (crec2[r].x & live) : live;
                // single comparisons, so each ballot is one compare's mask:
                // sel = the child's bit for a slot of a real parent, else 0
                const uint32_t sel = r * 64 + lane < m ? 1u << cj[r] : 0u;
                const bool ok = (rowv & sel) != 0u;
                const bool first = (rowv & (sel | below[r])) == (sel ? sel : 0xFFFFFFFFu);
                double kr = prk + (double)cx[r];
                double ks = ps + ((double)cx[r] - lse_t);
                if (DTREE) {
                    kr += gv[r];
                    ks += gv[r];
                }
                krk[r] = ok ? kr : -INFINITY;
                ksc[r] = ok ? ks : -INFINITY;
                ktie[r] = ok ? (((uint32_t)ctok[r] << 6) | (uint32_t)cp[r]) : 0xFFFFFFFFu;
                const uint32_t o = ord_hi(kr);
                if (first && o < fmin) fmin = o;
                nvalid += __popcll(__ballot(ok));
                nfirst += __popcll(__ballot(first));
            }
            if (nvalid == 0) break;
            const int keep = nvalid < W ? nvalid : W;
            // (b) the bound: the W first-valid keys are distinct candidates,
            //     so the depth's W-th key is at least the smallest of them
            //     (taken on the high words of their ordered images)
            // (every valid key is finite, so a bound of -DBL_MAX admits all of
            // them and no invalid one)
            double lb = -1.7976931348623157e308;
            if (nfirst >= W) lb = ord_hi_floor(wave_min_u32(fmin));
            // With many candidates above that bound (no continuity filter, or
            // a parent term that reorders a parent's children), tighten it:
            // the W-th largest of the lanes' best keys, taken on the same high
            // words, is reached by W distinct candidates, so it bounds the
            // depth's W-th key from below too.  Found bit by bit with ballots.
            int nin = 0;
#pragma unroll
            for (int r = 0; r < RM; ++r) nin += __popcll(__ballot(krk[r] >= lb));
            // (up to 16 survivors take the register-only ranking below; with
            // W above 12 the tightened bound rarely gets there, so it is
            // tried only past 32)
            if (nin > (W <= 12 ? 16 : 32)) {
                // (a lane without a valid candidate has -inf, whose high word
                // 0x000FFFFF is below every finite key's; a threshold that low
                // maps to a NaN, which leaves lb as it is)
                double lm = krk[0];
#pragma unroll
                for (int r = 1; r < RM; ++r) lm = max_d(lm, krk[r]);
                const uint32_t u = ord_hi(lm);
                // (every prefix of the search is such a bound too, only
                // coarser; it stops once the bits left rarely change which
                // candidates survive: at bit 12, or bit 8 when W > 12, whose
                // wider frontiers fall into the longer ranking paths sooner)
                const uint32_t th = W <= 12 ? wave_kth_high<12>(u, W) : wave_kth_high<8>(u, W);
                lb = max_d(lb, ord_hi_floor(th));
            }
            int ns = 0;
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                const bool in = krk[r] >= lb;
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
            const uint32_t tdep = (uint32_t)t << 8;
            // (c) ranks
            if (ns <= 16) {
                // Four replicas of the survivor list, one per 16-lane row:
                // lane (row r, i) holds survivor i and survivor (i + 4r) mod 16,
                // rotates the latter by 1..4 lanes within the row (DPP
                // row_ror), so the four rows together compare survivor i with
                // every other one; the rows' counts are summed with the
                // row-swapping permutes.  One round of shared-memory reads.
                const int i = lane & 15, rep = lane >> 4;
                const SurvKey me = sv_key[i];
                const SurvKey ot = sv_key[(i + 4 * rep) & 15];
                const SurvAux ax = sv_aux[i];
                // (keeps the winners' fields in the same round of reads
                // instead of a second one after the ranks)
                asm volatile("" ::"v"(ax.s), "v"(ax.cm), "v"(me.j));
                const uint32_t ot_lo = (uint32_t)__double_as_longlong(ot.rk);
                const uint32_t ot_hi = (uint32_t)((uint64_t)__double_as_longlong(ot.rk) >> 32);
                const int part = beats_rotated<1>(ot_lo, ot_hi, ot.tie, me.rk, me.tie) +
                                 beats_rotated<2>(ot_lo, ot_hi, ot.tie, me.rk, me.tie) +
                                 beats_rotated<3>(ot_lo, ot_hi, ot.tie, me.rk, me.tie) +
                                 beats_rotated<4>(ot_lo, ot_hi, ot.tie, me.rk, me.tie);
                const auto q16 = __builtin_amdgcn_permlane16_swap((uint32_t)part, (uint32_t)part, false, false);
                const uint32_t pair = q16[0] + q16[1];                  // rows 0+1 | 2+3
                const auto q32 = __builtin_amdgcn_permlane32_swap(pair, pair, false, false);
                const int rank = (int)(q32[0] + q32[1]);
                if (rep == 0 && i < ns && rank < keep)
                    n_rec[nb + rank] = NodeRec{me.rk, ax.s, ax.cm, me.j | tdep, (int)(me.tie >> 6),
                                               pbase + (int)(me.tie & 63u)};
            } else if (ns <= 32) {
                // 32 lanes per replica, two replicas; lane (rep, i) compares
                // survivor i with survivors i+s (mod 32), s = 1 + rep + 2u
                constexpr int G = 32, F = 2;
                const int i = lane & (G - 1), rep = lane / G;
                const SurvKey me = sv_key[i];
                const SurvAux ax = sv_aux[i];
                // all sixteen reads in the same round as the lane's own
                u4 o[G / F];
#pragma unroll
                for (int u = 0; u < G / F; ++u) {
                    const int sh = 1 + rep + u * F;
                    o[u] = *reinterpret_cast<const u4*>(&sv_key[(i + (sh < G ? sh : 0)) & (G - 1)]);
                }
                asm volatile("" ::"v"(ax.s), "v"(ax.cm), "v"(me.j));
                int part = 0;
#pragma unroll
                for (int u = 0; u < G / F; ++u) {
                    const int sh = 1 + rep + u * F;
                    const double ork = __longlong_as_double(((long long)o[u].y << 32) | o[u].x);
                    part += (sh < G) & ((ork > me.rk) | ((ork == me.rk) & (o[u].z < me.tie)));
                }
                const auto q32 = __builtin_amdgcn_permlane32_swap((uint32_t)part, (uint32_t)part, false, false);
                part = (int)(q32[0] + q32[1]);
                if (rep == 0 && i < ns && part < keep)
                    n_rec[nb + part] = NodeRec{me.rk, ax.s, ax.cm, me.j | tdep, (int)(me.tie >> 6),
                                               pbase + (int)(me.tie & 63u)};
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
                    if (e < ns && rank < keep)
                        n_rec[nb + rank] = NodeRec{me.rk, ax.s, ax.cm, me.j | tdep, (int)(me.tie >> 6),
                                                   pbase + (int)(me.tie & 63u)};
                }
            }
            __builtin_amdgcn_wave_barrier();
            fbase = nb;
            nb += keep;
            f = keep;
            cbase += (!trigram || t == 1) ? k : kk;
        }
        if (lane == 0) misc[0] = nb;
    }
    __syncthreads();
    nb = misc[0];                                            // ordered by the barrier
    // the output stage's per-node arrays
    for (int i = tid; i < nb; i += kTreeThreads) {
        const NodeRec rec = n_rec[i];
        n_tok[i] = rec.tok;
        n_par[i] = rec.par;
        n_dep[i] = (int)(rec.tj >> 8);
        n_s[i] = rec.s;
    }
    __syncthreads();
    return nb;
}

}  // namespace treedev
}  // namespace dt
