// Keeping the trigram table current after verification: every accepted
// token s_i of a request adds the trigram (s_{i-2}, s_{i-1}) -> s_i, where
// the stream starts with the request's committed context (DART, arXiv
// 2601.19278, Fig. 3: the N-gram model that keeps expansions continuous; its
// contents come from text the target model produced).
//
// One thread per accepted token; all of a call's trigrams are applied
// concurrently with 64- and 32-bit compare-and-swap:
//  - the key: probing linearly from splitmix64(key), a slot holding the key
//    is used as is; a free slot is claimed by CAS (free -> key); a CAS that
//    loses to the same key uses the slot, one that loses to another key goes
//    on probing.  Slots never become free again, so every key stays at or
//    after its home slot with no free slot in between, which is what a lookup
//    relies on;
//  - the successor: the first entry equal to it ends the search; a free entry
//    (-1) is claimed by CAS, and a lost CAS continues with the next entry.
// The keys and successor sets that result are those of applying the trigrams
// one by one in any order, as long as no row fills up and no probe sequence
// runs out of free slots; which slot a key added in the same call lands in,
// and which successors survive a row that overflows, depend on timing.
//
// Latency, not bandwidth, bounds this kernel (a few hundred trigrams per
// call, each a chain of dependent memory round trips), so each round trip
// covers eight slots or entries: plain loads of an aligned group, then the
// scan in registers.  A plain load may return an entry's old value while
// another workgroup (on another XCD's L2) is claiming it; since an entry only
// ever goes from free to a value, the stale value can only be "free", and
// the CAS that follows returns the real one.  The counters are summed per
// wave before one atomic add each.
#include "common.h"

namespace dt {
namespace {

constexpr unsigned long long kFree = 0xFFFFFFFFFFFFFFFFull;

__device__ __forceinline__ unsigned long long mix64(unsigned long long z) {
    // SplitMix64 output function (Steele, Lea, Flood).
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Find or claim the slot of `key`: its index, or -1 if the whole probe
// sequence is taken by other keys.  *added is set when this thread claimed it.
__device__ __forceinline__ long long find_or_claim(unsigned long long* keys, long long cap,
                                                   unsigned long long key, int* added) {
    const unsigned long long cm = (unsigned long long)cap - 1ull;
    const int G = cap < 8 ? (int)cap : 8;                   // cap is a power of two
    const unsigned long long pos = mix64(key) & cm;
    unsigned long long g0 = pos & ~(unsigned long long)(G - 1);
    int off = (int)(pos - g0);
    long long slot = -1;
    for (long long seen = 0; seen < cap && slot < 0; seen += G - off, off = 0, g0 = (g0 + G) & cm) {
        unsigned long long v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = j < G ? keys[g0 + j] : 0ull;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (slot >= 0 || j < off || j >= G) continue;
            if (v[j] == key) {
                slot = (long long)(g0 + j);
            } else if (v[j] == kFree) {
                const unsigned long long cur = atomicCAS(keys + g0 + j, kFree, key);
                if (cur == kFree) *added = 1;
                if (cur == kFree || cur == key) slot = (long long)(g0 + j);
            }
        }
    }
    return slot;
}

// Add successor c to a row of S entries.  1 = added at entry *at, 0 = present
// already, -1 = the row is full of other successors.  A row whose slot this
// thread has just claimed starts empty, so its first group is taken as free
// without a load: the CAS returns what other threads may have put there.
__device__ __forceinline__ int add_successor(int32_t* row, int S, int32_t c, int* at, bool fresh) {
    for (int e0 = 0; e0 < S; e0 += 8) {
        int32_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = e0 + j >= S ? 0 : (fresh && e0 == 0) ? -1 : row[e0 + j];
        int res = -1;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (res >= 0 || e0 + j >= S) continue;
            if (v[j] == c) {
                res = 0;
            } else if (v[j] == -1) {
                const int32_t cur = atomicCAS(row + e0 + j, -1, c);
                if (cur == -1) {
                    res = 1;
                    *at = e0 + j;
                } else if (cur == c) {
                    res = 0;
                }
            }
        }
        if (res >= 0) return res;
    }
    return -1;
}

__global__ void __launch_bounds__(kThreads) ngram_update_kernel(NGramUpdateArgs a) {
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    int key_added = 0, succ_added = 0, dropped = 0;
    bool active = t < (int64_t)a.B * a.L;
    unsigned long long key = 0;
    int32_t c = 0;
    if (active) {
        // the length and the three tokens are independent loads, all in bounds
        const int b = (int)(t / a.L), i = (int)(t - (int64_t)b * a.L);
        const int32_t* tok = a.tokens + (int64_t)b * a.L;
        const int len = a.lengths[b];
        c = tok[i];
        const int32_t t2 = i >= 2 ? tok[i - 2] : (i == 1 ? a.ctx[2 * b + 1] : a.ctx[2 * b]);
        const int32_t t1 = i >= 1 ? tok[i - 1] : a.ctx[2 * b + 1];
        key = ((unsigned long long)(uint32_t)t2 << 32) | (uint32_t)t1;
        active = i < len;
    }
    if (active) {
        const long long slot = key == kFree ? -1 : find_or_claim(a.keys, a.cap, key, &key_added);
        if (slot < 0) {                                       // the free marker, or no free slot on the way
            dropped = 1;
        } else {
            int at = 0;
            const int r = add_successor(a.succ + slot * a.S, a.S, c, &at, key_added != 0);
            if (r > 0 && a.hash_logp) a.hash_logp[slot * a.S + at] = a.new_logp;
            succ_added = r > 0;
            dropped = r < 0;
        }
    }
    if (a.counts) {
        const unsigned long long m0 = __ballot(key_added), m1 = __ballot(succ_added), m2 = __ballot(dropped);
        if ((threadIdx.x & 63) == 0) {
            if (m0) atomicAdd(&a.counts[0], __popcll(m0));
            if (m1) atomicAdd(&a.counts[1], __popcll(m1));
            if (m2) atomicAdd(&a.counts[2], __popcll(m2));
        }
    }
}

}  // namespace

hipError_t launch_ngram_update(const NGramUpdateArgs& a, hipStream_t stream) {
    const int64_t n = (int64_t)a.B * a.L;
    if (n <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((n + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(ngram_update_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dt
