// C entry points of libdt.so (declared and documented in include/dt.h):
// host-side validation, launch planning and the two kernel launches.
// Nothing here allocates, synchronises or keeps state between calls.
#include <math.h>
#include <string.h>

#include <mutex>

#include "common.h"

namespace dt {

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t round_up(int64_t a, int64_t m) { return ceil_div(a, m) * m; }

SweepPlan plan_sweep(const dt_params* p) {
    SweepPlan s{};
    s.rows = (int64_t)p->B * p->d;
    const int V = p->V;
    int C;
    int lists = kWaves;
    const int64_t by_merge4 = kMergeKeysPerRow / (p->k * kWaves);     // chunks with one list per wave
    const int64_t by_merge1 = kMergeKeysPerRow / p->k;                // chunks with one list per chunk
    if (p->sweep_chunks > 0) {
        C = p->sweep_chunks;
        if (C > by_merge4) lists = 1;
    } else {
        // at least ~two 256-thread workgroups per CU (256 CUs) and chunks of
        // >= 4096 elements; a row merges at most kMergeKeysPerRow keys, so
        // short chunks (small batches) merge their four wave lists in the
        // workgroup first
        const int64_t target = 512;
        int64_t c = s.rows >= target ? 1 : ceil_div(target, s.rows > 0 ? s.rows : 1);
        const int64_t by_len = V / 4096 > 1 ? V / 4096 : 1;
        if (c > by_len) c = by_len;
        if (c > by_merge4) {
            lists = 1;
            if (c > by_merge1) c = by_merge1;
        }
        C = (int)(c < 1 ? 1 : c);
    }
    if (C > V) C = V;
    s.chunk = (int)round_up(ceil_div(V, C), 8);
    s.C = (int)ceil_div(V, s.chunk);
    s.lists = lists;
    return s;
}

int n_contexts(int kind, int d, int k) {
    if (kind == DT_NGRAM_NONE) return 0;
    if (kind == DT_NGRAM_HASH_TRIGRAM) return d == 1 ? 1 : 1 + k + (d - 2) * k * k;
    return 1 + (d - 1) * k;
}

WorkspacePlan plan_workspace(const dt_params* p, const SweepPlan& s) {
    WorkspacePlan w{};
    const int64_t n = s.rows * s.C * s.lists;    // partial lists
    const int64_t rows = s.rows, k = p->k;
    w.n_ctx_cap = n_contexts(DT_NGRAM_HASH_TRIGRAM, p->d, p->k);   // the largest kind
    int64_t off = 0;
    auto take = [&](int64_t bytes) {
        const int64_t o = round_up(off, 256);
        off = o + bytes;
        return (size_t)o;
    };
    w.off_m = take(n * 4);
    w.off_s = take(n * 8);
    w.off_keys = take(n * k * 8);
    w.off_lse = take(rows * 8);
    w.off_ttok = take(rows * k * 4);
    w.off_tx = take(rows * k * 4);
    w.off_vmask = take((int64_t)p->B * w.n_ctx_cap * 4);
    w.off_g = take(p->mode == DT_MODE_DARTREE ? rows * k * k * 8 : 0);
    const bool full = p->mode == DT_MODE_DARTREE_FULL;
    const int64_t B = p->B, fw = full ? (int64_t)p->B * p->W : 0, nn = full ? fw * p->d : 0;
    // chunks of at least kVocabChunk tokens, about kVocabGroups workgroups
    // per depth over all request groups
    const int64_t ngroups = ceil_div(p->B > 0 ? p->B : 1, kVocabReqPerGroup);
    const int64_t want = kVocabGroups / ngroups > 1 ? kVocabGroups / ngroups : 1;
    const int64_t vc = round_up(ceil_div(p->V, want), 16);
    w.vchunk = (int)(vc > kVocabChunk ? vc : kVocabChunk);
    w.C2 = full ? (int)ceil_div(p->V, w.vchunk) : 0;
    w.off_f_tok = take(fw * 4);
    w.off_f_rk = take(fw * 8);
    w.off_f_s = take(fw * 8);
    w.off_f_node = take(fw * 4);
    w.off_f_n = take(full ? B * 4 : 0);
    w.off_n_tree = take(full ? B * 4 : 0);
    w.off_nd_tok = take(nn * 4);
    w.off_nd_par = take(nn * 4);
    w.off_nd_dep = take(nn * 4);
    w.off_nd_s = take(nn * 8);
    w.off_part = take(fw * w.C2 * (int64_t)sizeof(VocabEntry));
    w.off_fnorm = take(full ? (int64_t)p->V * 4 : 0);
    w.off_fbf = take(full ? (int64_t)p->V * p->R * 2 : 0);
    w.off_seed = take(full ? B * 8 : 0);
    w.off_cmp_n = take(full ? B * 4 : 0);
    w.off_cmp = take(full ? B * kFrontCap * (int64_t)sizeof(VocabEntry) : 0);
    w.total = (size_t)round_up(off, 256);
    return w;
}

TreePlan plan_tree(const dt_params* p, int kind) {
    TreePlan P{};
    const int d = p->d, k = p->k, W = p->W;
    P.n_ctx = n_contexts(kind, d, k);
    P.max_nodes = d * W;
    P.max_cand = W * k;
    int off = 0;
    auto take = [&](int bytes, int align) {
        off = (int)round_up(off, align);
        const int o = off;
        off += bytes;
        return o;
    };
    P.off_lse = take(d * 8, 8);
    P.off_g = take(p->mode == DT_MODE_DARTREE ? d * k * k * 8 : 0, 16);
    P.off_ttok = take(d * k * 4, 4);
    P.off_tx = take(d * k * 4, 4);
    P.off_vmask = take(P.n_ctx * 4, 4);
    P.off_misc = take(kMiscInts * 4, 4);
    P.off_sv_key = take((P.max_cand + 32) * 16, 16);  // + a block of sentinels
    P.off_sv_s = take((P.max_cand + 32) * 16, 16);
    const int nn = P.max_nodes;
    P.off_n_rec = take((nn + 1) * 32, 16);      // + the root's record
    P.off_n_s = take(nn * 8, 8);
    P.off_n_tok = take(nn * 4, 4);
    P.off_n_par = take(nn * 4, 4);
    P.off_n_dep = take(nn * 4, 4);
    P.off_n_new = take(nn * 4, 4);
    P.off_n_out = take(nn * 4, 4);
    P.total = (int)round_up(off, 16);
    return P;
}

// ---------------------------------------------------------------------------
// validation (host only; no HIP call)
// ---------------------------------------------------------------------------
static dt_status check_shape(const dt_params* p) {
    if (!p) return DT_ERR_INVALID_ARG;
    if (p->B < 0 || p->d < 1 || p->k < 1 || p->V < 1 || p->W < 1 || p->budget < 1)
        return DT_ERR_INVALID_ARG;
    if (p->k > p->V) return DT_ERR_INVALID_ARG;
    if (p->dtype != DT_DTYPE_F32 && p->dtype != DT_DTYPE_BF16) return DT_ERR_INVALID_ARG;
    if (p->mode != DT_MODE_DART && p->mode != DT_MODE_DARTREE && p->mode != DT_MODE_DARTREE_FULL)
        return DT_ERR_INVALID_ARG;
    if (p->sweep_chunks < 0) return DT_ERR_INVALID_ARG;
    if (p->d > kMaxD || p->k > kMaxK || p->W > kMaxW || p->budget > kMaxBudget ||
        p->W * p->k > kMaxCandidates || p->V >= kMaxV)
        return DT_ERR_UNSUPPORTED;
    const SweepPlan s = plan_sweep(p);
    if ((int64_t)s.C * s.lists * p->k > kMergeKeysPerRow || (int64_t)s.C * s.lists > 256) return DT_ERR_UNSUPPORTED;
    return DT_OK;
}

static dt_status check_workspace(const dt_params* p) {
    const WorkspacePlan w = plan_workspace(p, plan_sweep(p));
    if (w.total == 0) return DT_OK;
    if (!p->workspace || ((uintptr_t)p->workspace & 15u) || p->workspace_bytes < w.total)
        return DT_ERR_WORKSPACE;
    return DT_OK;
}

static dt_status check_ngram(const dt_ngram_table* g) {
    if (!g) return DT_ERR_INVALID_ARG;
    const bool finite = !(isinf(g->min_logp) && g->min_logp < 0);
    if (isnan(g->min_logp)) return DT_ERR_INVALID_ARG;
    switch (g->kind) {
    case DT_NGRAM_NONE:
        return DT_OK;
    case DT_NGRAM_DENSE_BIGRAM:
        return g->dense_logp ? DT_OK : DT_ERR_INVALID_ARG;
    case DT_NGRAM_CSR_BIGRAM:
        // an empty table (nnz = 0) needs no successor arrays
        if (!g->row_ptr || g->nnz < 0) return DT_ERR_INVALID_ARG;
        if (g->nnz > 0 && (!g->col || (finite && !g->csr_logp))) return DT_ERR_INVALID_ARG;
        return DT_OK;
    case DT_NGRAM_HASH_TRIGRAM:
        if (!g->keys || !g->succ || (finite && !g->hash_logp)) return DT_ERR_INVALID_ARG;
        if (g->cap < 2 || (g->cap & (g->cap - 1)) != 0) return DT_ERR_INVALID_ARG;
        if (g->S < 1 || g->S > 64) return DT_ERR_UNSUPPORTED;
        if (((uintptr_t)g->keys & 15u) != 0) return DT_ERR_INVALID_ARG;
        return DT_OK;
    default:
        return DT_ERR_INVALID_ARG;
    }
}

}  // namespace dt

using namespace dt;

extern "C" const char* dt_status_string(dt_status s) {
    // any int may arrive from C: read the bits without loading an
    // out-of-range enumeration value
    int v;
    memcpy(&v, &s, sizeof v);
    switch (v) {
    case DT_OK: return "DT_OK";
    case DT_ERR_INVALID_ARG: return "DT_ERR_INVALID_ARG: null pointer, value out of range or misaligned buffer";
    case DT_ERR_UNSUPPORTED: return "DT_ERR_UNSUPPORTED: outside the library's limits";
    case DT_ERR_WORKSPACE: return "DT_ERR_WORKSPACE: workspace missing, misaligned or smaller than dt_workspace_size()";
    case DT_ERR_HIP: return "DT_ERR_HIP: the HIP runtime refused a launch";
    default: return "unknown dt_status";
    }
}

extern "C" size_t dt_workspace_size(const dt_params* p) {
    if (check_shape(p) != DT_OK) return 0;
    return plan_workspace(p, plan_sweep(p)).total;
}

static dt_status launch_sweep_for(const void* logits, const dt_params* p, const SweepPlan& s,
                                  const WorkspacePlan& w, bool take_turns) {
    hipStream_t stream = (hipStream_t)p->stream;
    char* ws = (char*)p->workspace;
    SweepArgs sa{};
    sa.logits = logits;
    sa.V = p->V;
    sa.C = s.C;
    sa.chunk = s.chunk;
    sa.lists = s.lists;
    sa.k = p->k;
    sa.part_m = (float*)(ws + w.off_m);
    sa.part_s = (double*)(ws + w.off_s);
    sa.part_keys = (unsigned long long*)(ws + w.off_keys);
    if (p->prof_event_start && hipEventRecord((hipEvent_t)p->prof_event_start, stream) != hipSuccess)
        return DT_ERR_HIP;
    if (launch_sweep(sa, s.rows, p->dtype, take_turns, stream) != hipSuccess) return DT_ERR_HIP;
    if (p->prof_event_stop && hipEventRecord((hipEvent_t)p->prof_event_stop, stream) != hipSuccess)
        return DT_ERR_HIP;
    return DT_OK;
}

// Full-vocabulary DARTree mode: the sweep and the row merge give lse; then
// per depth the vocabulary kernel and the frontier merge; then the budget
// and the outputs.  The profiling events (if given) bracket the depth loop.
static dt_status build_full(const void* logits, const dt_params* p, const SweepPlan& s, const WorkspacePlan& w,
                            const dt_tree_out* out) {
    hipStream_t stream = (hipStream_t)p->stream;
    char* ws = (char*)p->workspace;
    SweepArgs sa{};
    sa.logits = logits;
    sa.V = p->V;
    sa.C = s.C;
    sa.chunk = s.chunk;
    sa.lists = s.lists;
    sa.k = p->k;
    sa.part_m = (float*)(ws + w.off_m);
    sa.part_s = (double*)(ws + w.off_s);
    sa.part_keys = (unsigned long long*)(ws + w.off_keys);
    if (launch_sweep(sa, s.rows, p->dtype, false, stream) != hipSuccess) return DT_ERR_HIP;
    MergeArgs ma{};
    ma.rows = (int)s.rows;
    ma.C = s.C * s.lists;
    ma.k = p->k;
    ma.part_m = sa.part_m;
    ma.part_s = sa.part_s;
    ma.part_keys = sa.part_keys;
    ma.lse = (double*)(ws + w.off_lse);
    ma.tok = (int32_t*)(ws + w.off_ttok);
    ma.val = (float*)(ws + w.off_tx);
    if (launch_merge(ma, stream) != hipSuccess) return DT_ERR_HIP;

    VocabArgs va{};
    va.B = p->B;
    va.V = p->V;
    va.d = p->d;
    va.W = p->W;
    va.R = p->R;
    va.dtype = p->dtype;
    va.vchunk = w.vchunk;
    va.C2 = w.C2;
    va.logits = logits;
    va.E = p->E;
    va.F = p->F;
    va.fnorm = (const float*)(ws + w.off_fnorm);
    va.Fbf = (const uint16_t*)(ws + w.off_fbf);
    va.ctx = p->ctx;
    va.f_tok = (const int32_t*)(ws + w.off_f_tok);
    va.f_rk = (const double*)(ws + w.off_f_rk);
    va.f_n = (const int32_t*)(ws + w.off_f_n);
    va.part = (VocabEntry*)(ws + w.off_part);
    va.seed = (const double*)(ws + w.off_seed);
    va.cmp_n = (int32_t*)(ws + w.off_cmp_n);
    va.cmp = (VocabEntry*)(ws + w.off_cmp);
    FrontierArgs fa{};
    fa.B = p->B;
    fa.d = p->d;
    fa.W = p->W;
    fa.C2 = w.C2;
    fa.part = va.part;
    fa.cmp_n = va.cmp_n;
    fa.cmp = va.cmp;
    fa.lse = ma.lse;
    fa.f_tok = (int32_t*)(ws + w.off_f_tok);
    fa.f_rk = (double*)(ws + w.off_f_rk);
    fa.f_s = (double*)(ws + w.off_f_s);
    fa.f_node = (int32_t*)(ws + w.off_f_node);
    fa.f_n = (int32_t*)(ws + w.off_f_n);
    fa.n_tree = (int32_t*)(ws + w.off_n_tree);
    fa.nd_tok = (int32_t*)(ws + w.off_nd_tok);
    fa.nd_par = (int32_t*)(ws + w.off_nd_par);
    fa.nd_dep = (int32_t*)(ws + w.off_nd_dep);
    fa.nd_s = (double*)(ws + w.off_nd_s);
    fa.V = p->V;
    fa.k = p->k;
    fa.R = p->R;
    fa.ttok = ma.tok;
    fa.tx = ma.val;
    fa.E = p->E;
    fa.F = p->F;
    fa.seed = (double*)(ws + w.off_seed);
    fa.fnorm = va.fnorm;
    if (launch_fnorm(p->F, p->V, p->R, (float*)(ws + w.off_fnorm), (uint16_t*)(ws + w.off_fbf), stream) != hipSuccess)
        return DT_ERR_HIP;
    fa.t = 0;
    if (launch_seed1(fa, p->ctx, stream) != hipSuccess) return DT_ERR_HIP;
    if (p->prof_event_start && hipEventRecord((hipEvent_t)p->prof_event_start, stream) != hipSuccess)
        return DT_ERR_HIP;
    for (int t = 1; t <= p->d; ++t) {
        va.t = t;
        fa.t = t;
        if (launch_vocab(va, stream) != hipSuccess) return DT_ERR_HIP;
        if (launch_frontier(fa, stream) != hipSuccess) return DT_ERR_HIP;
    }
    if (p->prof_event_stop && hipEventRecord((hipEvent_t)p->prof_event_stop, stream) != hipSuccess)
        return DT_ERR_HIP;
    FinishArgs na{};
    na.B = p->B;
    na.d = p->d;
    na.W = p->W;
    na.budget = p->budget;
    na.mask_words = (p->budget + 31) / 32;
    na.n_tree = fa.n_tree;
    na.nd_tok = fa.nd_tok;
    na.nd_par = fa.nd_par;
    na.nd_dep = fa.nd_dep;
    na.nd_s = fa.nd_s;
    na.n_nodes = out->n_nodes;
    na.tokens = out->tokens;
    na.parents = out->parents;
    na.depths = out->depths;
    na.scores = out->scores;
    na.mask = out->mask;
    if (launch_finish(na, stream) != hipSuccess) return DT_ERR_HIP;
    return DT_OK;
}

static dt_status enqueue_build(const void* logits, const dt_ngram_table* ngram, const dt_params* p,
                               const dt_tree_out* out);

// Every argument check of dt_build_tree except the workspace's; host only.
// DT_OK with *nothing = true means a valid call with nothing to enqueue (B = 0).
static dt_status check_build(const void* logits, const dt_ngram_table* ngram, const dt_params* p,
                             const dt_tree_out* out, bool* nothing) {
    *nothing = false;
    dt_status st = check_shape(p);
    if (st != DT_OK) return st;
    if ((st = check_ngram(ngram)) != DT_OK) return st;
    if (!out) return DT_ERR_INVALID_ARG;
    if (p->mode == DT_MODE_DARTREE) {
        if (!p->E || !p->F) return DT_ERR_INVALID_ARG;
        if (p->R < 4 || p->R > 256 || p->R % 4 != 0) return DT_ERR_UNSUPPORTED;
        if (((uintptr_t)p->E & 15u) || ((uintptr_t)p->F & 15u)) return DT_ERR_INVALID_ARG;
    }
    if (p->mode == DT_MODE_DARTREE_FULL) {
        if (!p->E || !p->F) return DT_ERR_INVALID_ARG;
        if (((uintptr_t)p->E & 15u) || ((uintptr_t)p->F & 15u)) return DT_ERR_INVALID_ARG;
        if (p->R != 16 && p->R != 32 && p->R != 64) return DT_ERR_UNSUPPORTED;
        if (p->W > kFullMaxW || ngram->kind != DT_NGRAM_NONE) return DT_ERR_UNSUPPORTED;
    }
    const TreePlan plan = plan_tree(p, ngram->kind);
    if (plan.total > kTreeLdsLimit) return DT_ERR_UNSUPPORTED;
    if (p->B == 0) {
        *nothing = true;
        return DT_OK;
    }
    if (!logits || ((uintptr_t)logits & 15u) || !p->ctx) return DT_ERR_INVALID_ARG;
    if (!out->n_nodes || !out->tokens || !out->parents || !out->depths || !out->scores || !out->mask)
        return DT_ERR_INVALID_ARG;
    return DT_OK;
}

extern "C" dt_status dt_build_tree(const void* logits, const dt_ngram_table* ngram,
                                   const dt_params* p, const dt_tree_out* out) {
    bool nothing;
    dt_status st = check_build(logits, ngram, p, out, &nothing);
    if (st != DT_OK || nothing) return st;
    if ((st = check_workspace(p)) != DT_OK) return st;
    return enqueue_build(logits, ngram, p, out);
}

// The scratch buffer of dt_build_tree_noalloc: a device array of fixed size
// in this library's code object, one copy per GPU, held until the process
// ends.  Host code never passes the array's own name to a kernel (on the
// host it is only a stand-in for the symbol): the device address of each
// GPU's copy comes from hipGetSymbolAddress, looked up once per device on
// the first call there and kept below.
static __device__ __align__(256) unsigned char scratch[DT_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

static dt_status scratch_of(hipStream_t stream, void** ptr_out) {
    int dev = 0;
    if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess) return DT_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return DT_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return DT_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return DT_ERR_HIP;
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return DT_ERR_HIP;
        if (e != hipSuccess || !ptr) return DT_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *ptr_out = g_scratch_ptr[dev];
    return DT_OK;
}

extern "C" dt_status dt_build_tree_noalloc(const void* logits, const dt_ngram_table* ngram,
                                           const dt_params* p, const dt_tree_out* out) {
    bool nothing;
    dt_status st = check_build(logits, ngram, p, out, &nothing);
    if (st != DT_OK || nothing) return st;
    if (plan_workspace(p, plan_sweep(p)).total > (size_t)DT_NOALLOC_SCRATCH_BYTES) return DT_ERR_WORKSPACE;
    dt_params q = *p;
    if ((st = scratch_of((hipStream_t)p->stream, &q.workspace)) != DT_OK) return st;
    q.workspace_bytes = DT_NOALLOC_SCRATCH_BYTES;
    return enqueue_build(logits, ngram, &q, out);
}

// Launches of the whole path for validated arguments and a large enough workspace.
static dt_status enqueue_build(const void* logits, const dt_ngram_table* ngram, const dt_params* p,
                               const dt_tree_out* out) {
    dt_status st;
    const TreePlan plan = plan_tree(p, ngram->kind);
    const SweepPlan s = plan_sweep(p);
    const WorkspacePlan w = plan_workspace(p, s);
    if (p->mode == DT_MODE_DARTREE_FULL) {
        if (w.C2 > kMaxVocabChunks) return DT_ERR_UNSUPPORTED;   // cannot happen: chunks adapt to V
        return build_full(logits, p, s, w, out);
    }
    char* ws = (char*)p->workspace;
    const bool take_turns = s.rows * s.C >= kSweepTurnMinGrid && s.rows * s.C <= kSweepTurnMaxGrid &&
                            plan.total + kPrepLds <= kTreeLdsLimit - 2 * kSweepLdsTurn;
    if ((st = launch_sweep_for(logits, p, s, w, take_turns)) != DT_OK) return st;
    PrepArgs pa{};
    pa.B = p->B;
    pa.d = p->d;
    pa.k = p->k;
    pa.L = s.C * s.lists;                         // partial lists per row
    pa.mode = p->mode;
    pa.R = p->R;
    pa.n_ctx = w.n_ctx_cap;
    pa.ctx = p->ctx;
    pa.part_m = (const float*)(ws + w.off_m);
    pa.part_s = (const double*)(ws + w.off_s);
    pa.part_keys = (const unsigned long long*)(ws + w.off_keys);
    pa.ng.kind = ngram->kind;
    pa.ng.V = p->V;
    pa.ng.min_logp = ngram->min_logp;
    pa.ng.dense = ngram->dense_logp;
    pa.ng.row_ptr = ngram->row_ptr;
    pa.ng.col = ngram->col;
    pa.ng.csr_logp = ngram->csr_logp;
    pa.ng.keys = (const unsigned long long*)ngram->keys;
    pa.ng.succ = ngram->succ;
    pa.ng.hash_logp = ngram->hash_logp;
    pa.ng.cap = ngram->cap;
    pa.ng.S = ngram->S;
    pa.E = p->E;
    pa.F = p->F;
    pa.lse = (double*)(ws + w.off_lse);
    pa.ttok = (int32_t*)(ws + w.off_ttok);
    pa.tx = (float*)(ws + w.off_tx);
    pa.vmask = (uint32_t*)(ws + w.off_vmask);
    pa.g = (double*)(ws + w.off_g);
    // the k^2 trigram contexts of a depth are split over workgroups of
    // kPrepContexts lookups
    pa.nsplit = ngram->kind == DT_NGRAM_HASH_TRIGRAM ? (int)ceil_div((int64_t)p->k * p->k, kPrepContexts) : 1;
    if (launch_prep(pa, (hipStream_t)p->stream) != hipSuccess) return DT_ERR_HIP;

    TreeArgs ta{};
    ta.B = p->B;
    ta.d = p->d;
    ta.k = p->k;
    ta.W = p->W;
    ta.budget = p->budget;
    ta.mode = p->mode;
    ta.mask_words = (p->budget + 31) / 32;
    ta.ng_kind = ngram->kind;
    ta.n_ctx = w.n_ctx_cap;                       // per-request stride of vmask
    ta.lse = pa.lse;
    ta.ttok = pa.ttok;
    ta.tx = pa.tx;
    ta.vmask = pa.vmask;
    ta.g = pa.g;
    ta.n_nodes = out->n_nodes;
    ta.tokens = out->tokens;
    ta.parents = out->parents;
    ta.depths = out->depths;
    ta.scores = out->scores;
    ta.mask = out->mask;
    ta.plan = plan;
    if (launch_tree(ta, (hipStream_t)p->stream) != hipSuccess) return DT_ERR_HIP;
    return DT_OK;
}

extern "C" dt_status dt_position_topk(const void* logits, const dt_params* p, double* lse,
                                      int32_t* topk_tok, float* topk_val) {
    dt_status st = check_shape(p);
    if (st != DT_OK) return st;
    if (p->B == 0) return DT_OK;
    if (!logits || ((uintptr_t)logits & 15u) || !lse || !topk_tok || !topk_val) return DT_ERR_INVALID_ARG;
    if ((st = check_workspace(p)) != DT_OK) return st;
    const SweepPlan s = plan_sweep(p);
    const WorkspacePlan w = plan_workspace(p, s);
    if ((st = launch_sweep_for(logits, p, s, w, false)) != DT_OK) return st;
    char* ws = (char*)p->workspace;
    MergeArgs ma{};
    ma.rows = (int)s.rows;
    ma.C = s.C * s.lists;
    ma.k = p->k;
    ma.part_m = (const float*)(ws + w.off_m);
    ma.part_s = (const double*)(ws + w.off_s);
    ma.part_keys = (const unsigned long long*)(ws + w.off_keys);
    ma.lse = lse;
    ma.tok = topk_tok;
    ma.val = topk_val;
    if (launch_merge(ma, (hipStream_t)p->stream) != hipSuccess) return DT_ERR_HIP;
    return DT_OK;
}

extern "C" dt_status dt_ngram_update(const dt_ngram_table* table, const int32_t* ctx, const int32_t* tokens,
                                     const int32_t* lengths, int32_t B, int32_t L, float new_logp,
                                     int32_t* counts, void* stream) {
    if (!table || table->kind != DT_NGRAM_HASH_TRIGRAM) return DT_ERR_INVALID_ARG;
    if (B < 0 || L < 0 || isnan(new_logp)) return DT_ERR_INVALID_ARG;
    if (!table->keys || !table->succ || table->cap < 2 || (table->cap & (table->cap - 1)) != 0)
        return DT_ERR_INVALID_ARG;
    if (((uintptr_t)table->keys & 7u) != 0 || ((uintptr_t)table->succ & 3u) != 0 ||
        ((uintptr_t)table->hash_logp & 3u) != 0)
        return DT_ERR_INVALID_ARG;
    if (table->S < 1 || table->S > 64) return DT_ERR_UNSUPPORTED;
    if ((int64_t)B * L == 0) return DT_OK;
    if (!ctx || !tokens || !lengths) return DT_ERR_INVALID_ARG;
    NGramUpdateArgs a{};
    a.B = B;
    a.L = L;
    a.S = table->S;
    a.cap = table->cap;
    a.new_logp = new_logp;
    a.ctx = ctx;
    a.tokens = tokens;
    a.lengths = lengths;
    a.keys = (unsigned long long*)table->keys;           // the update writes the table in place
    a.succ = (int32_t*)table->succ;
    a.hash_logp = (float*)table->hash_logp;
    a.counts = counts;
    if (launch_ngram_update(a, (hipStream_t)stream) != hipSuccess) return DT_ERR_HIP;
    return DT_OK;
}

extern "C" dt_status dt_verify_length(const dt_tree_out* tree, int32_t B, int32_t budget, double cost_fixed,
                                      double cost_per_token, int32_t* n_verify, int32_t* rank, void* stream) {
    if (!tree || B < 0 || budget < 1) return DT_ERR_INVALID_ARG;
    if (!(cost_fixed > 0.0) || !isfinite(cost_fixed) || !(cost_per_token >= 0.0) || !isfinite(cost_per_token))
        return DT_ERR_INVALID_ARG;
    if (budget > kMaxBudget) return DT_ERR_UNSUPPORTED;
    if (B == 0) return DT_OK;
    if (!tree->n_nodes || !tree->parents || !tree->depths || !tree->scores || !n_verify || !rank)
        return DT_ERR_INVALID_ARG;
    VerifyArgs a{};
    a.B = B;
    a.budget = budget;
    a.cost_fixed = cost_fixed;
    a.cost_per_token = cost_per_token;
    a.n_nodes = tree->n_nodes;
    a.parents = tree->parents;
    a.depths = tree->depths;
    a.scores = tree->scores;
    a.n_verify = n_verify;
    a.rank = rank;
    if (launch_verify(a, (hipStream_t)stream) != hipSuccess) return DT_ERR_HIP;
    return DT_OK;
}
