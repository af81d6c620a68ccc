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
// Reads of entries other threads may claim use device-scope atomic loads.
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

__global__ void __launch_bounds__(kThreads) ngram_update_kernel(NGramUpdateArgs a) {
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= (int64_t)a.B * a.L) return;
    const int b = (int)(t / a.L), i = (int)(t - (int64_t)b * a.L);
    const int n = a.lengths[b] < a.L ? a.lengths[b] : a.L;
    if (i >= n) return;
    const int32_t* tok = a.tokens + (int64_t)b * a.L;
    const int32_t c = tok[i];
    const int32_t t2 = i >= 2 ? tok[i - 2] : (i == 1 ? a.ctx[2 * b + 1] : a.ctx[2 * b]);
    const int32_t t1 = i >= 1 ? tok[i - 1] : a.ctx[2 * b + 1];
    const unsigned long long key = ((unsigned long long)(uint32_t)t2 << 32) | (uint32_t)t1;
    int* counts = a.counts;
    if (key == kFree) {                                       // indistinguishable from a free slot
        if (counts) atomicAdd(&counts[2], 1);
        return;
    }
    const unsigned long long cm = (unsigned long long)a.cap - 1ull;
    unsigned long long pos = mix64(key) & cm;
    long long slot = -1;
    for (long long probe = 0; probe < a.cap; ++probe) {
        unsigned long long* kp = a.keys + pos;
        unsigned long long cur = __hip_atomic_load(kp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (cur == kFree) {
            cur = atomicCAS(kp, kFree, key);
            if (cur == kFree) {
                if (counts) atomicAdd(&counts[0], 1);
                slot = (long long)pos;
                break;
            }
        }
        if (cur == key) {
            slot = (long long)pos;
            break;
        }
        pos = (pos + 1ull) & cm;
    }
    if (slot < 0) {                                           // no free slot on the way
        if (counts) atomicAdd(&counts[2], 1);
        return;
    }
    int32_t* row = a.succ + slot * a.S;
    for (int e = 0; e < a.S; ++e) {
        int32_t cur = __hip_atomic_load(row + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (cur == -1) {
            cur = atomicCAS(row + e, -1, c);
            if (cur == -1) {
                if (a.hash_logp) a.hash_logp[slot * a.S + e] = a.new_logp;
                if (counts) atomicAdd(&counts[1], 1);
                return;
            }
        }
        if (cur == c) return;                                 // present already
    }
    if (counts) atomicAdd(&counts[2], 1);                     // row full
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
