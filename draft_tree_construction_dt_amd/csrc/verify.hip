// How many nodes of a built tree to send to verification (LibraSpec,
// scholarbro listing abstract: the speculative length is chosen for expected
// speedup, and extended only while the acceptance gain outweighs the added
// verification cost, judged from the drafter's confidence).  For a tree the
// candidate verification sets are the prefixes of its best-first order (each
// is closed under parents).  Node n of that order has confidence
// c_n = exp(S_n), the drafter's probability that its whole path is accepted;
// with A(n) = 1 + sum_{i<n} c_i expected tokens per round and
// T(n) = cost_fixed + cost_per_token * n the round's cost, node n is added
// while c_n * T(n) > cost_per_token * A(n), i.e. while A/T strictly grows.
//
// One wave per request, up to 16 nodes per lane in registers.  The
// best-first order is replayed: at each step the best available node (parent
// taken) by (score desc, depth asc, index asc) is found with wavefront
// reductions; lane 0 then applies the rule in that order, summing like the
// sequential definition.
#include <math.h>

#include "common.h"
#include "wave.h"

namespace dt {
namespace {


constexpr int kPerLane = kMaxBudget / 64;
constexpr int kNone = 0x7FFFFFFF;

__global__ void __launch_bounds__(64) verify_kernel(VerifyArgs a) {
    __shared__ int s_order[kMaxBudget];
    __shared__ float s_sc[kMaxBudget];
    __shared__ int s_dep[kMaxBudget];
    const int b = blockIdx.x, lane = threadIdx.x;
    const int budget = a.budget;
    const int64_t base = (int64_t)b * budget;
    int n = a.n_nodes[b];
    n = n < 0 ? 0 : (n > budget ? budget : n);
    float sc[kPerLane];
    int dep[kPerLane], par[kPerLane], rk[kPerLane];
    uint32_t avail = 0, taken = 0;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
        const int i = lane + 64 * q;
        const bool valid = i < n;
        sc[q] = valid ? a.scores[base + i] : -INFINITY;
        dep[q] = valid ? a.depths[base + i] : 0;
        par[q] = valid ? a.parents[base + i] : -2;
        rk[q] = -1;
        if (valid) {
            s_sc[i] = sc[q];
            s_dep[i] = dep[q];
            if (par[q] < 0) avail |= 1u << q;
        }
    }
    // When no score rises along an edge (always in DART mode: x - lse <= 0,
    // and fp32 rounding keeps the order), every parent comes before its
    // children in the order (score desc, depth asc, index asc), so that order
    // IS the best-first order: each node's position is a count.
    bool mono = true;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
        const int i = lane + 64 * q;
        if (i < n && par[q] >= 0 && par[q] < n) mono &= a.scores[base + par[q]] >= sc[q];
        if (i < n && (par[q] >= i || par[q] < -1)) mono = false;       // not a tree in BFS order: replay
    }
    if (__ballot(!mono) == 0) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kPerLane; ++q) {
            const int i = lane + 64 * q;
            if (i < n) {
                int r = 0;
                for (int j = 0; j < n; ++j) {
                    const float sj = s_sc[j];
                    const int dj = s_dep[j];
                    r += (sj > sc[q]) | ((sj == sc[q]) & ((dj < dep[q]) | ((dj == dep[q]) & (j < i))));
                }
                rk[q] = r;
                s_order[r] = i;
            }
        }
    } else {
    for (int step = 0; step < n; ++step) {
        float bs = -INFINITY;
        int bd = kNone, bi = kNone;
#pragma unroll
        for (int q = 0; q < kPerLane; ++q) {
            const int i = lane + 64 * q;
            if (((avail & ~taken) >> q) & 1u) {
                if (bi == kNone || sc[q] > bs || (sc[q] == bs && (dep[q] < bd || (dep[q] == bd && i < bi)))) {
                    bs = sc[q];
                    bd = dep[q];
                    bi = i;
                }
            }
        }
        const float ms = wave_max_f32(bi != kNone ? bs : -INFINITY);
        const bool m1 = bi != kNone && bs == ms;
        const int md = wave_min_i32(m1 ? bd : kNone);
        const bool m2 = m1 && bd == md;
        const int mi = wave_min_i32(m2 ? bi : kNone);
        if (mi == kNone) {                                              // only a malformed tree (a parent
            n = step;                                                   // not among its nodes) gets here
            break;
        }
#pragma unroll
        for (int q = 0; q < kPerLane; ++q) {
            if (lane + 64 * q == mi) {
                taken |= 1u << q;
                rk[q] = step;
            }
            if (par[q] == mi) avail |= 1u << q;
        }
        if (lane == 0) s_order[step] = mi;
    }
    }
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
        const int i = lane + 64 * q;
        if (i < budget) a.rank[base + i] = rk[q];
    }
    __syncthreads();
    if (lane == 0) {
        double A = 1.0, T = a.cost_fixed;
        int m = 0;
        while (m < n) {
            const double c = exp((double)s_sc[s_order[m]]);
            if (!(c * T > a.cost_per_token * A)) break;
            A += c;
            T += a.cost_per_token;
            ++m;
        }
        a.n_verify[b] = m;
    }
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
    if (a.B <= 0) return hipSuccess;
    hipLaunchKernelGGL(verify_kernel, dim3((unsigned)a.B), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dt
