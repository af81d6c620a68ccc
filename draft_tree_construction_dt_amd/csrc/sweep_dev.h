// Vocabulary sweep (device code of sweep_kernel): per (row, chunk) the running max, the sum of exp(x - max)
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
// non-temporal (streamed once) and the next batch is loaded into the other
// of two register sets before the current one is reduced (no copies, and no
// branch around the loads, so the compiler waits only for the batch it
// needs).  Per lane: online max and sum in the exp2 domain
// (v_exp_f32), batch sums in fp32 folded into an fp64 accumulator.  Per
// wave: an exact top-k by threshold filtering -- an element enters the
// wave's LDS buffer only if its key beats the current k-th key -- with the
// threshold seeded from the k-th largest of the 64 lane maxima of the first
// batch (a ballot radix selection, no data exchange between lanes) and raised
// by selections of the buffer.
#pragma once

#include "common.h"
#include "wave.h"

namespace dt {
namespace sweepdev {

constexpr float kLog2e = 1.4426950408889634f;

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

// A threshold below which no element can be among the wave's k largest:
// the largest value t with ord(t) a multiple of 2^16 such that at least k
// lanes hold a value >= t, found bit by bit with ballots (the 16 high bits of
// ord; exact for bf16 data, whose low 16 bits are zero).  Lanes' padding
// values are -inf, so the result is never below -inf.
__device__ __forceinline__ float wave_threshold(float v, int k) {
    const uint32_t u = ord_bits(__float_as_uint(v + 0.0f));
    uint32_t t = 0;
#pragma unroll
    for (int b = 31; b >= 16; --b) {
        const uint32_t c = t | (1u << b);
        if (__popcll(__ballot(u >= c)) >= k) t = c;
    }
    const uint32_t floor_ord = ord_bits(0xFF800000u);              // -inf
    return t <= floor_ord ? -INFINITY : __uint_as_float(unord_bits(t));
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
    const int n8 = (n + 7) & ~7;
    // pad to a multiple of eight with empty keys (0 beats nothing); a wave's
    // LDS accesses complete in order, so the reads below see these writes
    if (lane < n8 - n) buf[n + lane] = 0ull;
    const unsigned long long a = lane < n ? buf[lane] : 0ull;
    const unsigned long long b = lane + 64 < n ? buf[lane + 64] : 0ull;
    int ra = 0, rb = 0;
    for (int j = 0; j < n8; j += 8) {            // eight independent broadcast reads per step
        unsigned long long v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = buf[j + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            ra += v[u] > a;
            rb += v[u] > b;
        }
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

// Rare path of consume: some lane's batch holds an element that reaches the
// threshold.  The lane's elements are staged in LDS (element-major, so the
// 64 lanes hit 64 different banks) and visited by a compact runtime loop, one
// round per candidate of the lane that holds the most; the common path thus
// stays a short straight loop.  Element e of the batch is vector e / EPV,
// lane element e % EPV; its row index is id0 + (e / EPV) * id_step + e % EPV.
template <int NE, int EPV>
__device__ __forceinline__ void insert_candidates(const float (&xs)[NE], int id0, int id_step,
                                                  const bool (&vok)[NE / EPV], WaveState& st,
                                                  unsigned long long* buf, float* stage, int k,
                                                  int trig, int lane) {
    static_assert(NE <= 32, "one pass mask bit per element");
    uint32_t pm = 0;
#pragma unroll
    for (int e = 0; e < NE; ++e) pm |= (uint32_t)(vok[e / EPV] && xs[e] >= st.thv) << e;
    if (pm) {
#pragma unroll
        for (int e = 0; e < NE; ++e) stage[e * 64 + lane] = xs[e];
    }
    while (__ballot(pm != 0u) != 0ull) {
        const bool has = pm != 0u;
        const int e = has ? __builtin_ctz(pm) : 0;
        pm &= pm - 1u;
        const float x = has ? stage[e * 64 + lane] : -INFINITY;
        const uint32_t id = (uint32_t)(id0 + (e / EPV) * id_step + (e % EPV));
        bool q = has && (x > st.thv || (x == st.thv && id < st.thid));
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

// Fold NE elements per lane into the lane's softmax state and the wave's
// top-k buffer.  Element e is vector e / EPV (vok: whether it exists; padding
// elements are -inf), lane element e % EPV, row index
// id0 + (e / EPV) * id_step + e % EPV.
template <int NE, int EPV>
__device__ __forceinline__ void consume(const float (&xs)[NE], int id0, int id_step,
                                        const bool (&vok)[NE / EPV], WaveState& st,
                                        unsigned long long* buf, float* stage, float* seeds,
                                        int k, int trig, int lane, int wave) {
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
        // Every wave seeds a threshold from its first batch: k of its lanes
        // hold an element >= the seed.  Any k elements of the row bound the
        // row's k-th largest from below, so no element under the largest of
        // the four seeds can be among the row's top k, and every wave filters
        // with that one.  (All waves of the workgroup take their first batch
        // in the same call, so the barrier is reached by all of them.)
        // A second seed: if every wave has q = ceil(k/4) lanes at or above
        // some value, the four waves together hold k elements there.
        const float t = wave_threshold(bm, k);
        const float tq = wave_threshold(bm, (k + kWaves - 1) / kWaves);
        if (lane == 0) {
            seeds[wave] = t;
            seeds[kWaves + wave] = tq;
        }
        __syncthreads();
        float tm = seeds[0], qm = seeds[kWaves];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            tm = fmaxf(tm, seeds[w]);
            qm = fminf(qm, seeds[kWaves + w]);
        }
        st.thv = fmaxf(tm, qm);
        st.thid = 0xFFFFFFFFu;
        st.fresh = false;
    }
    if (__ballot(bm >= st.thv) == 0ull) return;
    insert_candidates<NE, EPV>(xs, id0, id_step, vok, st, buf, stage, k, trig, lane);
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

// Unguarded loads: a vector past the chunk's end reads the chunk's last
// vector instead (a valid address; the batch that holds it masks it out), so
// every load is issued and the compiler can count the loads in flight.
template <bool BF16>
__device__ __forceinline__ void load_clamped(vec4 (&r)[U], const vec4* vbase, int64_t q, int64_t v_hi) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t qu = q + (int64_t)u * kThreads;
        r[u] = __builtin_nontemporal_load(vbase + (qu < v_hi ? qu : v_hi - 1));
    }
}

// One batch of vectors q0 + u * kThreads: vectors past the chunk's end (only
// in a partial last batch) become -inf, then the batch is folded in.  FULL:
// the batch is known to lie inside the chunk.
template <bool BF16, int NE, int EPV, bool FULL>
__device__ __forceinline__ void eat_batch(vec4 (&r)[U], int64_t q0, int64_t v_hi, bool partial, int64_t row0,
                                          WaveState& st, unsigned long long* buf, float* stage, float* seeds,
                                          int k, int trig, int lane, int wave) {
    constexpr uint32_t NEG = BF16 ? 0xFF80FF80u : 0xFF800000u;   // -inf patterns
    bool vok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) vok[u] = FULL || q0 + (int64_t)u * kThreads < v_hi;
    if (!FULL && partial) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (!vok[u]) r[u] = vec4{NEG, NEG, NEG, NEG};
    }
    float xs[NE];
#pragma unroll
    for (int u = 0; u < U; ++u) unpack<BF16>(r[u], xs + u * EPV);
    consume<NE, EPV>(xs, (int)(q0 * EPV - row0), kThreads * EPV, vok, st, buf, stage, seeds, k, trig, lane, wave);
}


// Shared-memory layout of one sweep workgroup (byte offsets from a 16-byte
// aligned base): the per-wave candidate buffers, the rare-path staging of a
// batch, the waves' first-batch seeds and the buffers of the workgroup merge.
template <bool BF16>
struct SweepLds {
    static constexpr int NE = U * (BF16 ? 8 : 4);
    static constexpr int off_buf = 0;                                            // u64 [kWaves][CAP]
    static constexpr int off_stage = off_buf + kWaves * CAP * 8;                 // float [kWaves][NE*64]
    static constexpr int off_all = off_stage + kWaves * NE * 64 * 4;             // u64 [kWaves*kMaxK + 8]
    static constexpr int off_ws = off_all + (kWaves * kMaxK + 8) * 8;            // double [kWaves]
    static constexpr int off_seeds = off_ws + kWaves * 8;                        // float [2*kWaves]
    static constexpr int off_wm = off_seeds + 2 * kWaves * 4;                    // float [kWaves]
    static constexpr int bytes = off_wm + kWaves * 4;
};

// Where a chunk's result goes: every wave's own list to the partial arrays
// (no barrier after the seed exchange), the workgroup's merged list to the
// partial arrays, or the merged list kept in shared memory (wave 0's buffer,
// descending keys, 0 pads) with its (max, sum) for the caller.
enum SweepOut { kOutWaveLists = 0, kOutMergedList = 1, kOutMergedLds = 2 };

struct MergedRow {
    float M;
    double S;
    const unsigned long long* keys;   // k keys in shared memory, descending
};

// One chunk of one row, swept by the whole workgroup (256 threads).
template <bool BF16>
__device__ __forceinline__ MergedRow sweep_chunk(const SweepArgs& a, int64_t row, int chunk, int out_mode,
                                                 unsigned char* lds) {
    constexpr int EPV = BF16 ? 8 : 4;
    constexpr int NE = U * EPV;
    using L = SweepLds<BF16>;
    unsigned long long (*s_buf)[CAP] = reinterpret_cast<unsigned long long (*)[CAP]>(lds + L::off_buf);
    float (*s_stage)[NE * 64] = reinterpret_cast<float (*)[NE * 64]>(lds + L::off_stage);
    float* s_seeds = reinterpret_cast<float*>(lds + L::off_seeds);
    unsigned long long* s_all = reinterpret_cast<unsigned long long*>(lds + L::off_all);
    float* s_wm = reinterpret_cast<float*>(lds + L::off_wm);
    double* s_ws = reinterpret_cast<double*>(lds + L::off_ws);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    float* stage = s_stage[wave];

    WaveState st;
    st.m = -INFINITY;
    st.s = 0.0;
    st.cnt = 0;
    st.thv = -INFINITY;
    st.thid = 0xFFFFFFFFu;
    st.fresh = true;

    // ---- batches of kThreads*U vectors, software pipelined over two
    //      register sets: the next batch is loaded before the current one is
    //      reduced, with no copies between the sets and every load issued
    //      unconditionally in the steady state (only the last batch can be
    //      partial)
    const int64_t per_batch = (int64_t)kThreads * U;
    const int64_t nvec = v_hi - v_lo;
    const int64_t nbat = (nvec + per_batch - 1) / per_batch;
    if (nbat > 0) {
        vec4 ra[U], rb[U];
        load_clamped<BF16>(ra, vbase, v_lo + tid, v_hi);
        int64_t bi = 0;
        for (; bi + 2 < nbat; bi += 2) {                 // batches bi and bi+1 are full
            const int64_t q0 = v_lo + bi * per_batch + tid;
            load_clamped<BF16>(rb, vbase, q0 + per_batch, v_hi);
            eat_batch<BF16, NE, EPV, true>(ra, q0, v_hi, false, row0, st, buf, stage, s_seeds, k, trig, lane, wave);
            load_clamped<BF16>(ra, vbase, q0 + 2 * per_batch, v_hi);
            eat_batch<BF16, NE, EPV, true>(rb, q0 + per_batch, v_hi, false, row0, st, buf, stage, s_seeds, k, trig,
                                           lane, wave);
        }
        const int64_t q0 = v_lo + bi * per_batch + tid;
        if (bi + 1 < nbat) {                             // two left: bi full, bi+1 the last
            load_clamped<BF16>(rb, vbase, q0 + per_batch, v_hi);
            eat_batch<BF16, NE, EPV, true>(ra, q0, v_hi, false, row0, st, buf, stage, s_seeds, k, trig, lane, wave);
            eat_batch<BF16, NE, EPV, false>(rb, q0 + per_batch, v_hi, (bi + 2) * per_batch > nvec, row0, st, buf,
                                            stage, s_seeds, k, trig, lane, wave);
        } else {                                         // one left: the last
            eat_batch<BF16, NE, EPV, false>(ra, q0, v_hi, (bi + 1) * per_batch > nvec, row0, st, buf, stage, s_seeds,
                                            k, trig, lane, wave);
        }
    }
    // ---- elements outside the aligned vectors (row ends that are not 16-byte aligned)
    {
        const int64_t n1 = s1_hi - s1_lo, n2 = s2_hi - s2_lo;       // each < EPV
        if (n1 + n2 > 0) {
            float xs[1];
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
            consume<1, 1>(xs, vok[0] ? (int)(g - row0) : 0, 0, vok, st, buf, stage, s_seeds, k, trig, lane, wave);
        }
    }

    // ---- this wave's partial: its top-k sorted, and (max, sum exp(x - max))
    wave_select(buf, st, k, lane);
    const float M = wave_max_f32(st.m);
    const double sl = (st.m == -INFINITY) ? 0.0 : st.s * (double)__builtin_amdgcn_exp2f((st.m - M) * kLog2e);
    const double S = wave_add_f64(sl);
    if (out_mode == kOutWaveLists) {
        // every wave writes its own list, so waves never wait for each other
        const int64_t list = (row * a.C + chunk) * kWaves + wave;
        unsigned long long* out = a.part_keys + list * k;
        if (lane < k) out[lane] = lane < st.cnt ? buf[lane] : 0ull;
        if (lane == 0) {
            a.part_m[list] = M;
            a.part_s[list] = S;
        }
        return MergedRow{M, S, nullptr};
    }
    // one list per workgroup: wave 0 merges the four wave partials
    if (lane < k) s_all[wave * k + lane] = lane < st.cnt ? buf[lane] : 0ull;
    if (lane == 0) {
        s_wm[wave] = M;
        s_ws[wave] = S;
    }
    __syncthreads();
    if (wave != 0) return MergedRow{0.f, 0.0, nullptr};
    const int n = kWaves * k, n8 = (n + 7) & ~7;
    if (lane < n8 - n) s_all[n + lane] = 0ull;          // pad: 0 beats nothing
    const float mw = lane < kWaves ? s_wm[lane] : -INFINITY;
    const float Mall = wave_max_f32(mw);
    const double sw = (lane < kWaves && mw != -INFINITY)
                          ? s_ws[lane] * (double)__builtin_amdgcn_exp2f((mw - Mall) * kLog2e) : 0.0;
    const double Sall = wave_add_f64(sw);
    const unsigned long long ka = lane < n ? s_all[lane] : 0ull;
    const unsigned long long kb = lane + 64 < n ? s_all[lane + 64] : 0ull;
    int ra = 0, rb = 0;
    for (int j = 0; j < n8; j += 8) {
        unsigned long long v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = s_all[j + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            ra += v[u] > ka;
            rb += v[u] > kb;
        }
    }
    __builtin_amdgcn_wave_barrier();
    // ranks of the nonzero keys are 0..(count-1) (keys are unique); slots
    // past the count keep the zero written first
    unsigned long long* sel = buf;                       // wave 0's buffer is free now
    if (lane < k) sel[lane] = 0ull;
    __builtin_amdgcn_wave_barrier();
    if (ka != 0ull && ra < k) sel[ra] = ka;
    if (kb != 0ull && rb < k) sel[rb] = kb;
    __builtin_amdgcn_wave_barrier();
    if (out_mode == kOutMergedLds) return MergedRow{Mall, Sall, sel};
    const int64_t list = row * a.C + chunk;
    if (lane < k) a.part_keys[list * k + lane] = sel[lane];
    if (lane == 0) {
        a.part_m[list] = Mall;
        a.part_s[list] = Sall;
    }
    return MergedRow{Mall, Sall, sel};
}

}  // namespace sweepdev
}  // namespace dt
