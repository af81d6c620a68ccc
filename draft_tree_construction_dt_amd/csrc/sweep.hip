// Vocabulary sweep: per (row, chunk) the running max, the sum of exp(x - max)
// and the exact top-k keys of the chunk.  DART (arXiv 2601.19278), Fig. 3:
// every draft position's own logit row proposes the tokens of its depth, so
// each of the B*d rows needs its log-softmax normaliser and its k best
// tokens.  This pass reads every logit exactly once and carries nearly all
// of the path's HBM traffic.
//
// Layout: a 256-thread workgroup owns one chunk of one row; each of its four
// waves streams a quarter of every batch and emits its own partial list (no
// barriers, no shared state between waves).  Each thread
// keeps kSweepVecsPerThread 16-byte vectors (8 bf16 or 4 fp32) per batch, the
// 64 lanes of a wave reading 1 KiB contiguous per load; loads are
// non-temporal (streamed once) and the next batch is loaded before the
// current one is reduced.  Per lane: online max and sum in the exp2 domain
// (v_exp_f32), batch sums in fp32 folded into an fp64 accumulator.  Per
// wave: an exact top-k by threshold filtering -- an element enters the
// wave's LDS buffer only if its key beats the current k-th key -- with the
// threshold seeded from the k-th largest of the 64 lane maxima of the first
// batch and raised by selections of the buffer.
#include "common.h"

namespace dt {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

extern "C" __device__ float __ockl_wfred_max_f32(float);      // DPP wavefront reductions (ROCm ockl)
extern "C" __device__ double __ockl_wfred_add_f64(double);
constexpr int U = kSweepVecsPerThread;
typedef uint32_t vec4 __attribute__((ext_vector_type(4)));
constexpr int CAP = kSweepCap;

__device__ __forceinline__ unsigned long long make_key(float x, uint32_t id) {
    return ((unsigned long long)ord_bits(__float_as_uint(x + 0.0f)) << 32) | (uint32_t)(~id);
}
__device__ __forceinline__ float key_value(unsigned long long key) {
    return __uint_as_float(unord_bits((uint32_t)(key >> 32)));
}
__device__ __forceinline__ uint32_t key_id(unsigned long long key) { return ~(uint32_t)key; }

__device__ __forceinline__ int lanes_below(unsigned long long mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// k-th largest of one float per lane (bitonic sort across the wave, descending).
__device__ __forceinline__ float wave_kth_largest(float v, int k, int lane) {
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const float o = __shfl_xor(v, stride);
            const bool desc = (lane & size) == 0;
            const bool lower = (lane & stride) == 0;
            v = (desc == lower) ? fmaxf(v, o) : fminf(v, o);
        }
    }
    return __shfl(v, k - 1);
}

struct WaveState {
    float m;          // lane: running max
    double s;         // lane: sum exp(x - m)
    int cnt;          // wave: entries in the buffer
    float thv;        // wave: threshold value (k-th key so far)
    uint32_t thid;    //       and its id
    bool fresh;       // wave: no batch seen yet
};

// Keep the k largest keys of buf[0..cnt), sorted descending, and raise the
// threshold to the k-th.  Rank by counting: every entry counts the entries
// with a larger key (keys are unique: ids differ).
__device__ __forceinline__ void wave_select(unsigned long long* buf, WaveState& st, int k, int lane) {
    const int n = st.cnt;
    const unsigned long long a = lane < n ? buf[lane] : 0ull;
    const unsigned long long b = lane + 64 < n ? buf[lane + 64] : 0ull;
    int ra = 0, rb = 0;
    for (int j = 0; j < n; ++j) {
        const unsigned long long v = buf[j];
        ra += v > a;
        rb += v > b;
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < n && ra < k) buf[ra] = a;
    if (lane + 64 < n && rb < k) buf[rb] = b;
    __builtin_amdgcn_wave_barrier();
    st.cnt = n < k ? n : k;
    if (st.cnt == k) {
        const unsigned long long t = buf[k - 1];
        st.thv = key_value(t);
        st.thid = key_id(t);
    }
}

// Fold NE elements per lane into the lane's softmax state and the wave's
// top-k buffer.  id0[u] is the row index of element u*EPV, vok[u] whether
// vector u exists (padding elements are -inf and never enter the top-k).
template <int NE, int EPV>
__device__ __forceinline__ void consume(const float (&xs)[NE], const int (&id0)[NE / EPV],
                                        const bool (&vok)[NE / EPV], WaveState& st,
                                        unsigned long long* buf, int k, int trig, int lane) {
    float bm = xs[0];
#pragma unroll
    for (int e = 1; e < NE; ++e) bm = fmaxf(bm, xs[e]);

    if (bm > st.m) {
        st.s *= (double)__builtin_amdgcn_exp2f((st.m - bm) * kLog2e);
        st.m = bm;
    }
    if (st.m != -INFINITY) {
        const float mL = st.m * kLog2e;
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc += __builtin_amdgcn_exp2f(fmaf(xs[e], kLog2e, -mL));
        st.s += (double)acc;
    }

    if (st.fresh) {
        st.thv = wave_kth_largest(bm, k, lane);   // k lanes hold an element >= this value
        st.thid = 0xFFFFFFFFu;
        st.fresh = false;
    }
    if (__ballot(bm >= st.thv) == 0ull) return;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const float x = xs[e];
        if (__ballot(x >= st.thv) == 0ull) continue;
        const int u = e / EPV;
        const uint32_t id = (uint32_t)(id0[u] + (e % EPV));
        bool q = vok[u] && (x > st.thv || (x == st.thv && id < st.thid));
        unsigned long long bal = __ballot(q);
        if (bal == 0ull) continue;
        if (st.cnt + 64 > CAP) {
            wave_select(buf, st, k, lane);
            q = q && (x > st.thv || (x == st.thv && id < st.thid));
            bal = __ballot(q);
        }
        if (q) buf[st.cnt + lanes_below(bal)] = make_key(x, id);
        st.cnt += __popcll(bal);
    }
    if (st.cnt >= trig) wave_select(buf, st, k, lane);
}

template <bool BF16>
__device__ __forceinline__ void unpack(const vec4& r, float* out) {
    if constexpr (BF16) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        out[0] = __uint_as_float(r.x);
        out[1] = __uint_as_float(r.y);
        out[2] = __uint_as_float(r.z);
        out[3] = __uint_as_float(r.w);
    }
}

template <bool BF16>
__device__ __forceinline__ void load_batch(vec4 (&r)[U], const vec4* vbase, int64_t q, int64_t v_hi) {
    constexpr uint32_t NEG = BF16 ? 0xFF80FF80u : 0xFF800000u;   // -inf patterns
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t qu = q + (int64_t)u * kThreads;
        r[u] = qu < v_hi ? __builtin_nontemporal_load(vbase + qu) : vec4{NEG, NEG, NEG, NEG};
    }
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads) sweep_kernel(SweepArgs a) {
    constexpr int EPV = BF16 ? 8 : 4;
    constexpr int NE = U * EPV;

    __shared__ unsigned long long s_buf[kWaves][CAP];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t row = blockIdx.x / a.C;
    const int chunk = blockIdx.x - (int)(row * a.C);
    const int k = a.k;
    const int trig = k * 2 < 32 ? 32 : (k * 2 > 64 ? 64 : k * 2);
    const int lo = chunk * a.chunk;
    const int hi = lo + a.chunk < a.V ? lo + a.chunk : a.V;
    const int64_t row0 = row * (int64_t)a.V;                       // global index of element 0
    const int64_t g_lo = row0 + lo, g_hi = row0 + hi;
    // aligned vectors [v_lo, v_hi) inside the chunk, and up to two scalar
    // stretches [s1_lo, s1_hi), [s2_lo, s2_hi) at unaligned row ends
    int64_t v_lo = (g_lo + EPV - 1) / EPV, v_hi = g_hi / EPV;
    int64_t s1_lo, s1_hi, s2_lo, s2_hi;
    if (v_lo <= v_hi) {
        s1_lo = g_lo; s1_hi = v_lo * EPV;
        s2_lo = v_hi * EPV; s2_hi = g_hi;
    } else {                                   // the chunk lies inside one vector
        v_lo = v_hi = 0;
        s1_lo = g_lo; s1_hi = g_hi;
        s2_lo = s2_hi = 0;
    }
    const vec4* vbase = reinterpret_cast<const vec4*>(a.logits);
    unsigned long long* buf = s_buf[wave];

    WaveState st;
    st.m = -INFINITY;
    st.s = 0.0;
    st.cnt = 0;
    st.thv = -INFINITY;
    st.thid = 0xFFFFFFFFu;
    st.fresh = true;

    // ---- batches of kThreads*U vectors, software pipelined: the next batch
    //      (the last one guarded) is loaded before the current one is reduced
    const int64_t per_batch = (int64_t)kThreads * U;
    const int64_t nvec = v_hi - v_lo;
    const int64_t nbat = (nvec + per_batch - 1) / per_batch;
    if (nbat > 0) {
        vec4 cur[U];
        load_batch<BF16>(cur, vbase, v_lo + tid, v_hi);
        for (int64_t bi = 0; bi < nbat; ++bi) {
            const int64_t q0 = v_lo + bi * per_batch + tid;
            vec4 nxt[U];
            if (bi + 1 < nbat) load_batch<BF16>(nxt, vbase, q0 + per_batch, v_hi);
            float xs[NE];
            int id0[U];
            bool vok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t q = q0 + (int64_t)u * kThreads;
                unpack<BF16>(cur[u], xs + u * EPV);
                id0[u] = (int)(q * EPV - row0);
                vok[u] = q < v_hi;
            }
            consume<NE, EPV>(xs, id0, vok, st, buf, k, trig, lane);
            if (bi + 1 < nbat) {
#pragma unroll
                for (int u = 0; u < U; ++u) cur[u] = nxt[u];
            }
        }
    }
    // ---- elements outside the aligned vectors (row ends that are not 16-byte aligned)
    {
        const int64_t n1 = s1_hi - s1_lo, n2 = s2_hi - s2_lo;       // each < EPV
        if (n1 + n2 > 0) {
            float xs[1];
            int id0[1];
            bool vok[1];
            const int64_t g = tid < n1 ? s1_lo + tid : s2_lo + (tid - n1);
            vok[0] = tid < n1 + n2;
            float x = -INFINITY;
            if (vok[0]) {
                if constexpr (BF16) {
                    x = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(a.logits)[g] << 16);
                } else {
                    x = reinterpret_cast<const float*>(a.logits)[g];
                }
            }
            xs[0] = x;
            id0[0] = vok[0] ? (int)(g - row0) : 0;
            consume<1, 1>(xs, id0, vok, st, buf, k, trig, lane);
        }
    }

    // ---- this wave's partial: its top-k sorted, and (max, sum exp(x - max));
    //      every wave writes its own list, so waves never wait for each other
    wave_select(buf, st, k, lane);
    const float M = __ockl_wfred_max_f32(st.m);
    const double sl = (st.m == -INFINITY) ? 0.0 : st.s * (double)__builtin_amdgcn_exp2f((st.m - M) * kLog2e);
    const double S = __ockl_wfred_add_f64(sl);
    const int64_t list = (row * a.C + chunk) * kWaves + wave;
    unsigned long long* out = a.part_keys + list * k;
    if (lane < k) out[lane] = lane < st.cnt ? buf[lane] : 0ull;
    if (lane == 0) {
        a.part_m[list] = M;
        a.part_s[list] = S;
    }
}

}  // namespace

hipError_t launch_sweep(const SweepArgs& a, int64_t rows, int dtype, hipStream_t stream) {
    const int64_t grid = rows * a.C;
    if (grid <= 0) return hipSuccess;
    if (dtype == DT_DTYPE_BF16)
        hipLaunchKernelGGL(sweep_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(sweep_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dt
