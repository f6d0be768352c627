// C ABI of the attention library: argument checks, the chunk planner and the executor.
//
// The executor runs a plan as Q chunks x KV chunks.  Each (Q chunk, KV chunk) pair is one launch
// of the forward kernel over the query rows that can see the chunk; chunks entirely above the
// causal diagonal are never scheduled.  Partials are merged exactly by log-sum-exp, either by the
// forward kernel's epilogue (fused) or by the merge kernel, and a final pass normalises.  Operands
// in pinned host memory are copied chunk by chunk on a side stream into two device buffers that
// alternate (double buffering), with events ordering each copy after the compute that last read
// its buffer and each compute after its copy (the two-stream pattern of block-streamer 0.1.0,
// README section "Streams, residency, and memory budget").  Output bound for host memory leaves
// on a third stream.
//
// A second schedule runs the cyclic quorum-set decomposition of the Stream-CQSA pages (depth 1):
// c parts, subproblem i holding parts (i + s) mod c for s in the interest set, each (query part, key
// part) pair computed once by its owner subproblem and folded into a device accumulator.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "cqsa.h"
#include "cqsa_internal.h"

using namespace cqsa;

namespace {

thread_local std::string g_err;

cqsa_status fail(cqsa_status s, const char* fmt, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

#define CQSA_HIP(expr)                                                                                     \
    do {                                                                                                   \
        hipError_t e_ = (expr);                                                                            \
        if (e_ != hipSuccess) return fail(CQSA_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));   \
    } while (0)

#define CQSA_TRY(expr)                        \
    do {                                      \
        cqsa_status s_ = (expr);              \
        if (s_ != CQSA_OK) return s_;         \
    } while (0)

constexpr double kSafety = 0.85;           // fraction of the budget the planner fills
constexpr int64_t kRowGrain = 256;         // chunk sizes are multiples of this (then clipped)
constexpr int64_t kKvCap = 262144;         // largest automatic KV chunk (keys)
constexpr int64_t kKvMinStream = 4096;     // smallest automatic KV chunk worth streaming
// Device-resident inputs whose key range exceeds kLongKeys, with query tiles for several rounds of
// workgroups, run one launch per KV chunk of kKvResident keys (folded by the kernel epilogue), not one
// pass: workgroups that start their sweeps of millions of keys at different times lose the cache reuse
// that every workgroup sweeping the same 128K-key chunk keeps (4M causal keys, H=8, D=64: 20.4 s one
// pass, 17.3 s in 128K chunks)
constexpr int64_t kLongKeys = 524288;
constexpr int64_t kKvResident = 131072;

int esize_of(int dt) { return dt == CQSA_F32 ? 4 : 2; }

// ---------------------------------------------------------------------------------------------
// operand views

struct View {
    char* data = nullptr;
    int dtype = 0;
    int es = 2;
    bool host = false;
    int64_t B = 0, H = 0, N = 0, D = 0;
    int64_t sb = 0, sh = 0, sn = 0;
};

cqsa_status locate(const cqsa_tensor* t, const char* name, bool allow_null, bool* host) {
    if (!t->data) {
        if (!allow_null) return fail(CQSA_ERR_INVALID, "%s: data is NULL", name);
        if (t->where == CQSA_WHERE_DEVICE || t->where == CQSA_WHERE_HOST) {
            *host = t->where == CQSA_WHERE_HOST;
            return CQSA_OK;
        }
        return fail(CQSA_ERR_INVALID, "%s: NULL data needs where = DEVICE or HOST", name);
    }
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof attr);
    hipError_t e = hipPointerGetAttributes(&attr, t->data);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky error a foreign pointer leaves
        return fail(CQSA_ERR_INVALID,
                    "%s: pageable host memory (or an unknown pointer); host operands must be pinned "
                    "(hipHostMalloc / pin_memory)",
                    name);
    }
    if (attr.type == hipMemoryTypeHost) {
        *host = true;
    } else if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) {
        *host = false;
    } else {
        return fail(CQSA_ERR_INVALID, "%s: pageable host memory; host operands must be pinned (hipHostMalloc)",
                    name);
    }
    return CQSA_OK;
}

cqsa_status make_view(const cqsa_tensor* t, const char* name, bool allow_null, bool detect, View* v) {
    if (!t) return fail(CQSA_ERR_INVALID, "%s: descriptor is NULL", name);
    if (t->dtype != CQSA_F16 && t->dtype != CQSA_BF16 && t->dtype != CQSA_F32)
        return fail(CQSA_ERR_UNSUPPORTED, "%s: dtype %d is not fp16/bf16/fp32", name, t->dtype);
    for (int i = 0; i < 4; ++i) {
        if (t->shape[i] < 0) return fail(CQSA_ERR_INVALID, "%s: negative shape", name);
        if (t->stride[i] < 0) return fail(CQSA_ERR_INVALID, "%s: negative stride", name);
    }
    if (t->stride[3] != 1) return fail(CQSA_ERR_INVALID, "%s: the head-dim stride must be 1", name);
    v->data = static_cast<char*>(t->data);
    v->dtype = t->dtype;
    v->es = esize_of(t->dtype);
    v->B = t->shape[0];
    v->H = t->shape[1];
    v->N = t->shape[2];
    v->D = t->shape[3];
    v->sb = t->stride[0];
    v->sh = t->stride[1];
    v->sn = t->stride[2];
    v->host = false;
    if (detect) {
        const bool empty = v->B == 0 || v->H == 0 || v->N == 0 || v->D == 0;
        if (t->data || !empty) {
            cqsa_status s = locate(t, name, allow_null, &v->host);
            if (s != CQSA_OK) return s;
        }
    } else {
        v->host = t->where == CQSA_WHERE_HOST;
    }
    return CQSA_OK;
}

struct Problem {
    View q, k, v, out;
    float* lse = nullptr;
    bool lse_host = false;
    bool want_lse = false;
    int64_t B = 0, Hq = 0, Hkv = 0, Nq = 0, Nk = 0, D = 0;
    int dtype = 0;
    bool causal = false;
    float scale = 0.f;
    bool empty = false;
    bool streamed = false;
    int p_split = 0;   // precision 1: split-P PV product
    bool one_pass = false;   // the caller runs single-pass plans only (the no-allocation entry point)
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

cqsa_status check_problem(Problem* P, int is_causal, float scale) {
    const View &q = P->q, &k = P->k, &v = P->v, &o = P->out;
    if (q.dtype != k.dtype || q.dtype != v.dtype)
        return fail(CQSA_ERR_INVALID, "q, k, v must share one dtype");
    if (q.dtype == CQSA_F32) return fail(CQSA_ERR_UNSUPPORTED, "inputs must be fp16 or bf16 (got fp32)");
    if (k.B != q.B || v.B != q.B || o.B != q.B) return fail(CQSA_ERR_INVALID, "batch sizes differ");
    if (k.H != v.H || k.N != v.N || k.D != v.D) return fail(CQSA_ERR_INVALID, "k and v shapes differ");
    if (k.D != q.D || o.D != q.D) return fail(CQSA_ERR_INVALID, "head dims differ");
    if (o.H != q.H || o.N != q.N) return fail(CQSA_ERR_INVALID, "out shape must equal q's shape");
    if (k.H == 0 && q.H != 0) return fail(CQSA_ERR_INVALID, "k has no heads");
    if (k.H != 0 && q.H % k.H != 0)
        return fail(CQSA_ERR_INVALID, "query heads (%lld) must be a multiple of key/value heads (%lld)",
                    (long long)q.H, (long long)k.H);
    P->B = q.B;
    P->Hq = q.H;
    P->Hkv = k.H;
    P->Nq = q.N;
    P->Nk = k.N;
    P->D = q.D;
    P->dtype = q.dtype;
    P->causal = is_causal != 0;
    P->empty = P->B == 0 || P->Hq == 0 || P->Nq == 0;
    if (P->D != 64 && P->D != 128)
        return fail(CQSA_ERR_UNSUPPORTED, "head dim %lld is not supported (64 or 128)", (long long)P->D);
    if (P->empty) return CQSA_OK;
    if (P->Nk == 0) return fail(CQSA_ERR_INVALID, "no keys: every query row would have nothing to attend to");
    if (P->causal && P->Nq > P->Nk)
        return fail(CQSA_ERR_INVALID,
                    "causal with Nq (%lld) > Nk (%lld): the first rows would see no key (bottom-right alignment)",
                    (long long)P->Nq, (long long)P->Nk);
    // vector loads of 8 elements, vector stores of 4
    for (const View* t : {&q, &k, &v}) {
        if (t->data && (!aligned16(t->data) || t->sn % 8 || t->sh % 8 || t->sb % 8))
            return fail(CQSA_ERR_UNSUPPORTED, "q/k/v data and row/head/batch strides must be 16-byte aligned");
    }
    if (o.data && ((reinterpret_cast<uintptr_t>(o.data) % (4 * o.es)) || o.sn % 4 || o.sh % 4 || o.sb % 4))
        return fail(CQSA_ERR_UNSUPPORTED, "out data and strides must be aligned to 4 elements");
    if (!(scale > 0.f) || !std::isfinite(scale)) scale = 1.0f / std::sqrt((float)P->D);
    P->scale = scale;
    P->streamed = q.host || k.host || v.host || o.host || (P->want_lse && P->lse_host);
    return CQSA_OK;
}

// ---------------------------------------------------------------------------------------------
// planner

struct Plan {
    cqsa_plan_info info;
    int bm = 256;
    int64_t q_chunk = 0, kv_chunk = 0, n_q = 0, n_kv = 0;
    int kv_splits = 1;
    int merge = 0;  // 0 single pass, CQSA_MERGE_KERNEL, CQSA_MERGE_FUSED
    bool chunked = false;
    // workspace layout (byte offsets); 0-size pieces are unused
    uint64_t off_q = 0, off_k[2] = {0, 0}, off_v[2] = {0, 0};
    uint64_t off_acc_o = 0, off_acc_ml = 0, off_part_o = 0, off_part_ml = 0, off_out = 0, off_lse = 0;
    uint64_t total = 0;
    // cyclic quorum-set schedule
    bool cqs = false;
    int cqs_c = 0;
    int cqs_nbuf = 0;                      // staging sets (1 or 2)
    std::vector<int> cqs_owner;            // owner[a * c + b]
    uint64_t off_stage[2] = {0, 0}, stage_bytes = 0;
    int64_t out_rows = 0;                  // query rows per finalize chunk (host output)
    struct CqsLaunch {
        std::vector<std::pair<int, int>> pairs;   // (query part, key part), sorted
    };
    struct CqsWave {
        std::vector<int> subs;                     // subproblems with pairs in the wave
        std::vector<std::pair<int, int>> pairs;    // (query part, key part) pairs the wave computes
        std::vector<char> qp, kp;                  // query / key parts it stages and reads
        uint64_t stage = 0;                        // staging bytes (host operands)
        std::vector<CqsLaunch> launches;           // at most kWaveCap query and key parts each
    };
    std::vector<CqsWave> cqs_waves;
    int64_t wave_tokens = 0;                       // the packed-row budget the waves were cut to
};

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Device bytes of a chunked plan with Q chunks of qc rows and KV chunks of kc keys.
uint64_t chunk_bytes(const Problem& P, int64_t qc, int64_t kc, int merge, bool layout, Plan* pl) {
    uint64_t off = 0;
    auto take = [&](uint64_t bytes) {
        uint64_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    const uint64_t rows = (uint64_t)P.B * P.Hq * qc;
    const uint64_t kvrows = (uint64_t)P.B * P.Hkv * kc;
    uint64_t o_q = P.q.host ? take(rows * P.D * 2) : 0;
    uint64_t o_k0 = P.k.host ? take(kvrows * P.D * 2) : 0;
    uint64_t o_k1 = P.k.host ? take(kvrows * P.D * 2) : 0;
    uint64_t o_v0 = P.v.host ? take(kvrows * P.D * 2) : 0;
    uint64_t o_v1 = P.v.host ? take(kvrows * P.D * 2) : 0;
    const bool multi = kc < P.Nk;
    uint64_t o_ao = multi ? take(rows * P.D * 4) : 0;
    uint64_t o_aml = multi ? take(rows * 8) : 0;
    uint64_t o_po = (multi && merge == CQSA_MERGE_KERNEL) ? take(rows * P.D * 4) : 0;
    uint64_t o_pml = (multi && merge == CQSA_MERGE_KERNEL) ? take(rows * 8) : 0;
    uint64_t o_out = P.out.host ? take(rows * P.D * P.out.es) : 0;
    uint64_t o_lse = (P.want_lse && P.lse_host) ? take(rows * 4) : 0;
    if (layout) {
        pl->off_q = o_q;
        pl->off_k[0] = o_k0;
        pl->off_k[1] = o_k1;
        pl->off_v[0] = o_v0;
        pl->off_v[1] = o_v1;
        pl->off_acc_o = o_ao;
        pl->off_acc_ml = o_aml;
        pl->off_part_o = o_po;
        pl->off_part_ml = o_pml;
        pl->off_out = o_out;
        pl->off_lse = o_lse;
        pl->total = off;
    }
    return off;
}

// Count launches / merges / pairs of a chunked plan (causal chunks above the diagonal are skipped).
void count_chunked(const Problem& P, Plan* pl) {
    int64_t pairs = 0, merges = 0, launches = 0;
    uint64_t h2d = 0, d2h = 0;
    int64_t max_kv = 0;
    for (int64_t qa = 0; qa < P.Nq; qa += pl->q_chunk) {
        const int64_t qn = std::min(pl->q_chunk, P.Nq - qa);
        const int64_t last = P.Nk - P.Nq + qa + qn - 1;
        const int64_t kv_end = P.causal ? std::min(P.Nk, last + 1) : P.Nk;
        const int64_t nkv = ceil_div(kv_end, pl->kv_chunk);
        max_kv = std::max(max_kv, nkv);
        pairs += nkv;
        launches += nkv;
        if (nkv > 1) {
            merges += nkv - 1;
            if (pl->merge == CQSA_MERGE_KERNEL) launches += nkv - 1;
            launches += 1;  // finalize
        }
        if (P.q.host) h2d += (uint64_t)P.B * P.Hq * qn * P.D * 2;
        if (P.k.host) h2d += (uint64_t)P.B * P.Hkv * kv_end * P.D * 2;
        if (P.v.host) h2d += (uint64_t)P.B * P.Hkv * kv_end * P.D * 2;
        if (P.out.host) d2h += (uint64_t)P.B * P.Hq * qn * P.D * P.out.es;
        if (P.want_lse && P.lse_host) d2h += (uint64_t)P.B * P.Hq * qn * 4;
    }
    pl->info.chunk_pairs = pairs;
    pl->info.merges = merges;
    pl->info.kernel_launches = launches;
    pl->info.h2d_bytes = h2d;
    pl->info.d2h_bytes = d2h;
    pl->info.n_kv_chunks = ceil_div(P.Nk, pl->kv_chunk);
    (void)max_kv;
}


// ---------------------------------------------------------------------------------------------
// cyclic quorum-set schedule

// Perfect difference sets (every nonzero residue mod c is exactly one difference of two elements).
struct QuorumSet {
    int c, l;
    int s[8];
};
constexpr QuorumSet kQuorumSets[] = {
    {3, 2, {0, 1}}, {7, 3, {0, 1, 3}}, {13, 4, {0, 1, 3, 9}}, {21, 5, {0, 1, 4, 14, 16}}, {31, 6, {0, 1, 3, 8, 12, 18}}};

int default_quorum_set(int c, int* out, int max_l) {
    for (const QuorumSet& q : kQuorumSets)
        if (q.c == c) {
            for (int i = 0; i < q.l && i < max_l; ++i) out[i] = q.s[i];
            return q.l;
        }
    return 0;
}

// Validates the set and fills owner[a * c + b]: the smallest subproblem i whose parts
// {(i + s) mod c} contain both a and b.
cqsa_status quorum_owner(int c, const int* set, int l, std::vector<int>* owner) {
    if (c < 1 || c > 4096) return fail(CQSA_ERR_INVALID, "cqs: c = %d is outside [1, 4096]", c);
    if (l < 1 || l > c) return fail(CQSA_ERR_INVALID, "cqs: interest set size %d is outside [1, c = %d]", l, c);
    if (!set) return fail(CQSA_ERR_INVALID, "cqs: interest set is NULL");
    std::vector<char> in(c, 0);
    for (int u = 0; u < l; ++u) {
        if (set[u] < 0 || set[u] >= c) return fail(CQSA_ERR_INVALID, "cqs: set element %d is outside [0, %d)", set[u], c);
        if (in[set[u]]) return fail(CQSA_ERR_INVALID, "cqs: set element %d is repeated", set[u]);
        in[set[u]] = 1;
    }
    owner->assign((size_t)c * c, -1);
    for (int a = 0; a < c; ++a)
        for (int u = 0; u < l; ++u) {
            const int i = ((a - set[u]) % c + c) % c;       // a is in subproblem i
            for (int v = 0; v < l; ++v) {
                const int b = (i + set[v]) % c;             // so is b
                int& o = (*owner)[(size_t)a * c + b];
                if (o < 0 || i < o) o = i;
            }
        }
    for (int a = 0; a < c; ++a)
        for (int b = 0; b < c; ++b)
            if ((*owner)[(size_t)a * c + b] < 0)
                return fail(CQSA_ERR_INVALID, "cqs: parts %d and %d share no subproblem (not a quorum set mod %d)", a, b, c);
    return CQSA_OK;
}

// Depth itr: the sequence is cut into C = c^itr parts, part p having base-c digits p_1 .. p_itr (p_1 the
// most significant, so that the parts with one p_1 form part p_1 of the depth-1 cut).  Subproblem
// I = (i_1 .. i_itr), also read base c, holds the parts whose every digit p_k is in {(i_k + s) mod c}:
// the cyclic quorum set applied again inside each part of the level above.  Two parts a and b meet in
// subproblem I exactly when a_k and b_k meet in i_k at every level, so the lexicographically smallest
// such I, the owner, takes the depth-1 owner of (a_k, b_k) digit by digit.  Fills owner[a * C + b].
cqsa_status quorum_owner_itr(int c, const int* set, int l, int itr, std::vector<int>* owner) {
    std::vector<int> own1;
    CQSA_TRY(quorum_owner(c, set, l, &own1));
    int64_t C = 1;
    for (int k = 0; k < itr; ++k) {
        C *= c;
        if (C > 4096) return fail(CQSA_ERR_INVALID, "cqs: c^itr = %d^%d parts exceed 4096", c, itr);
    }
    owner->assign((size_t)(C * C), 0);
    for (int64_t a = 0; a < C; ++a)
        for (int64_t b = 0; b < C; ++b) {
            int64_t o = 0, x = a, y = b, w = 1;
            for (int k = 0; k < itr; ++k) {   // least significant digit first
                o += own1[(size_t)(x % c) * c + (size_t)(y % c)] * w;
                x /= c;
                y /= c;
                w *= c;
            }
            (*owner)[(size_t)(a * C + b)] = (int)o;
        }
    return CQSA_OK;
}

int64_t part_lo(int64_t n, int c, int p) { return n * p / c; }

// Does any key of key part b lie at or before the last row of query part a (causal)?
bool pair_visible(const Problem& P, int c, int a, int b) {
    const int64_t qa = part_lo(P.Nq, c, a), qe = part_lo(P.Nq, c, a + 1);
    const int64_t ka = part_lo(P.Nk, c, b), ke = part_lo(P.Nk, c, b + 1);
    if (qe <= qa || ke <= ka) return false;
    if (!P.causal) return true;
    return ka <= (P.Nk - P.Nq) + qe - 1;
}

cqsa_status make_plan_cqs(const Problem& P, uint64_t budget, const cqsa_options& opt, Plan* pl) {
    const int c0 = opt.cqs_c, itr = std::max(1, opt.cqs_itr);
    int dflt[8];
    const int* set = opt.cqs_set;
    int l = opt.cqs_l;
    if (!set) {
        l = default_quorum_set(c0, dflt, 8);
        if (l == 0) return fail(CQSA_ERR_INVALID, "cqs: no built-in interest set for c = %d; pass cqs_set", c0);
        set = dflt;
    }
    CQSA_TRY(quorum_owner_itr(c0, set, l, itr, &pl->cqs_owner));
    int c = 1;   // from here on: the number of parts (and of subproblems), c0^itr
    for (int k = 0; k < itr; ++k) c *= c0;
    if (opt.q_chunk > 0 || opt.kv_chunk > 0 || opt.kv_splits > 1)
        return fail(CQSA_ERR_INVALID, "cqs: q_chunk, kv_chunk and kv_splits do not apply to the quorum-set schedule");
    pl->cqs = true;
    pl->chunked = true;
    pl->cqs_c = c;
    pl->merge = CQSA_MERGE_FUSED;
    pl->kv_splits = 1;
    // subproblems that own at least one non-empty pair, in index order
    const uint64_t qrow = (uint64_t)P.B * P.Hq * P.D * 2, kvrow = (uint64_t)P.B * P.Hkv * P.D * 2;
    auto qlen = [&](int a) { return part_lo(P.Nq, c, a + 1) - part_lo(P.Nq, c, a); };
    auto klen = [&](int b) { return part_lo(P.Nk, c, b + 1) - part_lo(P.Nk, c, b); };
    std::vector<std::pair<int, std::vector<std::pair<int, int>>>> subs;
    int64_t pairs = 0, max_q = 0, max_k = 0;
    for (int a = 0; a < c; ++a) max_q = std::max(max_q, qlen(a));
    for (int b = 0; b < c; ++b) max_k = std::max(max_k, klen(b));
    {
        std::vector<std::vector<std::pair<int, int>>> by(c);
        for (int a = 0; a < c; ++a)
            for (int b = 0; b < c; ++b)
                if (pair_visible(P, c, a, b)) by[pl->cqs_owner[(size_t)a * c + b]].emplace_back(a, b);
        for (int i = 0; i < c; ++i)
            if (!by[i].empty()) {
                pairs += (int64_t)by[i].size();
                subs.emplace_back(i, std::move(by[i]));
            }
    }
    // Waves: consecutive units (whole subproblems, or a subproblem's pairs of one query part when whole
    // subproblems stage too much for two staging sets) whose staged rows (query rows of the union of
    // their query parts plus key rows of the union of their key parts) stay within the packed-row
    // budget W; a wave runs as one launch per kWaveCap query and key parts.
    using Units = std::vector<std::pair<int, std::vector<std::pair<int, int>>>>;
    Units by_part;
    for (const auto& sp : subs) {
        size_t i = 0;
        while (i < sp.second.size()) {   // the pairs are in query-part order
            size_t j = i;
            while (j < sp.second.size() && sp.second[j].first == sp.second[i].first) ++j;
            by_part.emplace_back(sp.first, std::vector<std::pair<int, int>>(sp.second.begin() + i, sp.second.begin() + j));
            i = j;
        }
    }
    auto cut = [&](int64_t W, const Units& units) {
        std::vector<Plan::CqsWave> ws;
        Plan::CqsWave cur;
        int64_t tok = 0;
        auto fresh = [&]() {
            cur = Plan::CqsWave();
            cur.qp.assign(c, 0);
            cur.kp.assign(c, 0);
            tok = 0;
        };
        fresh();
        std::vector<char> nq(c), nk(c);
        auto added = [&](const std::vector<std::pair<int, int>>& prs) {   // rows the subproblem adds to cur
            std::fill(nq.begin(), nq.end(), 0);
            std::fill(nk.begin(), nk.end(), 0);
            int64_t add = 0;
            for (const auto& pr : prs) {
                if (!cur.qp[pr.first] && !nq[pr.first]) {
                    nq[pr.first] = 1;
                    add += qlen(pr.first);
                }
                if (!cur.kp[pr.second] && !nk[pr.second]) {
                    nk[pr.second] = 1;
                    add += klen(pr.second);
                }
            }
            return add;
        };
        for (const auto& sp : units) {
            int64_t add = added(sp.second);
            if (!cur.pairs.empty() && tok + add > W) {
                ws.push_back(std::move(cur));
                fresh();
                add = added(sp.second);
            }
            if (cur.subs.empty() || cur.subs.back() != sp.first) cur.subs.push_back(sp.first);
            cur.pairs.insert(cur.pairs.end(), sp.second.begin(), sp.second.end());
            for (int p = 0; p < c; ++p) {
                cur.qp[p] |= nq[p];
                cur.kp[p] |= nk[p];
            }
            tok += add;
        }
        if (!cur.pairs.empty()) ws.push_back(std::move(cur));
        for (auto& wv : ws) {
            uint64_t bytes = 0;
            for (int a = 0; a < c; ++a)
                if (wv.qp[a] && P.q.host) bytes = align_up(bytes + (uint64_t)qlen(a) * qrow, 256);
            for (int b = 0; b < c; ++b) {
                if (wv.kp[b] && P.k.host) bytes = align_up(bytes + (uint64_t)klen(b) * kvrow, 256);
                if (wv.kp[b] && P.v.host) bytes = align_up(bytes + (uint64_t)klen(b) * kvrow, 256);
            }
            wv.stage = bytes;
        }
        return ws;
    };
    const uint64_t rows = (uint64_t)P.B * P.Hq * P.Nq;
    const uint64_t orows = (uint64_t)P.B * P.Hq * max_q;
    uint64_t off = 0;
    auto take = [&](uint64_t b) {
        const uint64_t at = off;
        off = align_up(off + b, 256);
        return at;
    };
    pl->off_acc_o = take(rows * P.D * 4);
    pl->off_acc_ml = take(rows * 8);
    pl->out_rows = max_q;
    pl->off_out = P.out.host ? take(orows * P.D * P.out.es) : 0;
    pl->off_lse = (P.want_lse && P.lse_host) ? take(orows * 4) : 0;
    const uint64_t base = off;
    int64_t W = opt.wave_tokens > 0 ? opt.wave_tokens
                                    : std::min<int64_t>(int64_t(1) << 22, std::max<int64_t>(int64_t(1) << 20, P.Nq + P.Nk));
    // The largest budget (halving from W) whose waves fit two staging sets, so that the copy of a wave
    // overlaps the compute of the one before; whole subproblems are tried before per-query-part units
    // (smaller units copy a key part once per unit instead of once per subproblem).  When no budget
    // gives two sets, the largest one that fits one set.
    std::vector<Plan::CqsWave> waves;
    uint64_t stage = 0;
    int nbuf = 0;
    auto stage_of = [](const std::vector<Plan::CqsWave>& ws) {
        uint64_t m = 0;
        for (const auto& wv : ws) m = std::max(m, wv.stage);
        return m;
    };
    bool found = false;
    for (int64_t w2 = W;; w2 = std::max<int64_t>(1, w2 / 2)) {
        for (const Units* u : {&subs, &by_part}) {
            std::vector<Plan::CqsWave> ws = cut(w2, *u);
            const uint64_t st = stage_of(ws);
            if (st == 0 || base + 2 * align_up(st, 256) <= budget) {
                waves = std::move(ws);
                stage = st;
                nbuf = st == 0 ? 0 : 2;
                W = w2;
                found = true;
                break;
            }
        }
        if (found || w2 <= 1) break;
    }
    for (int64_t w1 = W; !found; w1 = std::max<int64_t>(1, w1 / 2)) {
        for (const Units* u : {&subs, &by_part}) {
            std::vector<Plan::CqsWave> ws = cut(w1, *u);
            const uint64_t st = stage_of(ws);
            if (base + align_up(st, 256) <= budget || (w1 <= 1 && u == &by_part)) {
                waves = std::move(ws);
                stage = st;
                nbuf = 1;
                W = w1;
                found = true;
                break;
            }
        }
    }
    pl->wave_tokens = W;
    uint64_t h2d = 0;
    int64_t launches = 0, folds = 0;
    for (auto& wv : waves) {
        for (int a = 0; a < c; ++a)
            if (wv.qp[a] && P.q.host) h2d += (uint64_t)qlen(a) * qrow;
        for (int b = 0; b < c; ++b)
            if (wv.kp[b]) h2d += (uint64_t)klen(b) * kvrow * ((P.k.host ? 1 : 0) + (P.v.host ? 1 : 0));
        std::vector<std::pair<int, int>> prs = wv.pairs;
        std::sort(prs.begin(), prs.end());
        // launches: blocks of kWaveCap query parts x kWaveCap key parts of the wave's parts (in order)
        std::vector<int> qrank(c, -1), krank(c, -1);
        int nqw = 0, nkw = 0;
        for (int a = 0; a < c; ++a)
            if (wv.qp[a]) qrank[a] = nqw++;
        for (int b = 0; b < c; ++b)
            if (wv.kp[b]) krank[b] = nkw++;
        const int nkb = (nkw + kWaveCap - 1) / kWaveCap;
        std::vector<Plan::CqsLaunch> blocks((size_t)((nqw + kWaveCap - 1) / kWaveCap) * nkb);
        for (const auto& pr : prs)
            blocks[(size_t)(qrank[pr.first] / kWaveCap) * nkb + krank[pr.second] / kWaveCap].pairs.push_back(pr);
        for (auto& L : blocks)
            if (!L.pairs.empty()) wv.launches.push_back(std::move(L));
        launches += (int64_t)wv.launches.size();
        for (const auto& L : wv.launches) {
            std::vector<int> qd;
            for (const auto& pr : L.pairs)
                if (qd.empty() || qd.back() != pr.first) qd.push_back(pr.first);
            folds += (int64_t)qd.size();
        }
    }
    pl->cqs_waves = std::move(waves);
    pl->stage_bytes = stage;
    pl->cqs_nbuf = nbuf;
    for (int i = 0; i < nbuf; ++i) pl->off_stage[i] = take(stage);
    pl->total = off;
    if (pl->total > budget)
        return fail(CQSA_ERR_BUDGET,
                    "mem_budget too small for the quorum-set schedule over %d parts: needs %llu bytes "
                    "(x 1/0.85 = %llu)", c, (unsigned long long)pl->total,
                    (unsigned long long)(pl->total / kSafety) + 1);
    cqsa_plan_info& in = pl->info;
    in.merge_mode = CQSA_MERGE_FUSED;
    in.q_chunk = max_q;
    in.kv_chunk = max_k;
    in.n_q_chunks = c;
    in.n_kv_chunks = c;
    in.kv_splits = 1;
    in.chunk_pairs = pairs;
    in.merges = folds;
    // wave launches, the accumulator fill, and the finalize: one per query part when out or lse is
    // shipped to the host in query-part pieces, else one
    const bool host_out = P.out.host || (P.want_lse && P.lse_host);
    in.kernel_launches = launches + 1 + (host_out ? c : 1);
    in.workspace_bytes = pl->total;
    in.h2d_bytes = h2d;
    in.d2h_bytes = (P.out.host ? rows * P.D * P.out.es : 0) + ((P.want_lse && P.lse_host) ? rows * 4 : 0);
    in.cqs_c = c0;
    in.cqs_subproblems = (int32_t)subs.size();
    in.cqs_waves = (int32_t)pl->cqs_waves.size();
    in.wave_tokens = pl->wave_tokens;
    return CQSA_OK;
}

cqsa_status make_plan(const Problem& P, uint64_t budget, const cqsa_options& opt, int num_cus, Plan* pl) {
    std::memset(&pl->info, 0, sizeof pl->info);
    pl->bm = fwd_block_m((int)P.D, P.p_split);
    pl->info.block_m = pl->bm;
    pl->info.budget_bytes = budget;
    pl->info.streamed = P.streamed ? 1 : 0;
    if (P.empty) {
        pl->info.q_chunk = 0;
        return CQSA_OK;
    }
    if (opt.cqs_c < 0) return fail(CQSA_ERR_INVALID, "cqs_c %d is negative", opt.cqs_c);
    if (opt.cqs_itr < 0) return fail(CQSA_ERR_INVALID, "cqs_itr %d is negative", opt.cqs_itr);
    if (opt.cqs_itr > 1 && opt.cqs_c <= 0)
        return fail(CQSA_ERR_INVALID, "cqs_itr applies to the quorum-set schedule only (cqs_c > 0)");
    if (opt.wave_tokens < 0) return fail(CQSA_ERR_INVALID, "wave_tokens %lld is negative", (long long)opt.wave_tokens);
    if (opt.wave_tokens > 0 && opt.cqs_c <= 0)
        return fail(CQSA_ERR_INVALID, "wave_tokens applies to the quorum-set schedule only (cqs_c > 0)");
    if (opt.cqs_c > 0) return make_plan_cqs(P, budget, opt, pl);
    const int req_merge = opt.merge_mode;
    if (req_merge < 0 || req_merge > 2) return fail(CQSA_ERR_INVALID, "merge_mode %d is not 0, 1 or 2", req_merge);
    if (opt.q_chunk < 0 || opt.kv_chunk < 0 || opt.kv_splits < 0)
        return fail(CQSA_ERR_INVALID, "negative chunk option");
    const bool forced = opt.q_chunk > 0 || opt.kv_chunk > 0;
    // workgroups of one pass, and how many the CUs hold at once
    const int64_t wgs_one_pass = P.B * P.Hq * ceil_div(P.Nq, pl->bm);
    const int64_t wgs_target = (int64_t)fwd_wgs_per_cu((int)P.D, P.p_split) * std::max(num_cus, 1);
    // long key ranges on the device: KV chunks of kKvResident keys when their accumulator fits and the
    // query tiles make several rounds of workgroups, whose sweeps drift apart (a 2,048-query prompt over
    // 1M keys, one round, measured 1% faster in one pass; with few tiles side-by-side splits fill the CUs)
    bool long_keys = false;
    if (!P.streamed && !P.one_pass && !forced && opt.kv_splits == 0 && P.Nk > kLongKeys &&
        wgs_one_pass >= 4 * wgs_target)
        long_keys = chunk_bytes(P, P.Nq, kKvResident, req_merge == 0 ? CQSA_MERGE_FUSED : req_merge, false, pl) <= budget;

    if (!P.streamed && !forced && !long_keys) {
        // one pass over all keys; optional side-by-side KV splits to fill the GPU: up to as many
        // workgroups as the CUs hold at once (more only add merges: the 2,048-query prompt at 32K keys
        // and D=128, 256 workgroups of one per CU, measured 2.5% slower in two splits)
        const int64_t wgs = wgs_one_pass;
        int splits = opt.kv_splits;
        if (splits == 0) {
            splits = 1;
            const int64_t target = wgs_target;
            const int64_t min_keys = P.causal ? (P.Nk - P.Nq + 1) : P.Nk;  // fewest keys a row sees
            if (wgs < target && min_keys >= 16384) {
                splits = (int)std::min<int64_t>({ceil_div(target, wgs), min_keys / 8192, 16});
                splits = std::max(splits, 1);
            }
        }
        splits = std::min<int>(std::max(splits, 1), kMaxMergeParts);
        splits = (int)std::min<int64_t>(splits, ceil_div(P.Nk, 64));
        const uint64_t rows = (uint64_t)P.B * P.Hq * P.Nq;
        while (splits > 1 && (uint64_t)splits * rows * (P.D + 2) * 4 + 512 > budget) splits = splits / 2;
        pl->kv_splits = std::max(splits, 1);
        pl->q_chunk = P.Nq;
        pl->kv_chunk = P.Nk;
        pl->n_q = 1;
        pl->n_kv = 1;
        pl->merge = pl->kv_splits > 1 ? CQSA_MERGE_KERNEL : 0;
        pl->chunked = false;
        if (pl->kv_splits > 1) {
            pl->off_part_o = 0;
            pl->off_part_ml = align_up((uint64_t)pl->kv_splits * rows * P.D * 4, 256);
            pl->total = align_up(pl->off_part_ml + (uint64_t)pl->kv_splits * rows * 8, 256);
        } else {
            pl->total = 0;
        }
        pl->info.q_chunk = pl->q_chunk;
        pl->info.kv_chunk = pl->kv_chunk;
        pl->info.n_q_chunks = 1;
        pl->info.n_kv_chunks = 1;
        pl->info.kv_splits = pl->kv_splits;
        pl->info.merge_mode = pl->merge;
        pl->info.chunk_pairs = 1;
        pl->info.merges = pl->kv_splits > 1 ? pl->kv_splits - 1 : 0;
        pl->info.kernel_launches = pl->kv_splits > 1 ? 2 : 1;
        pl->info.workspace_bytes = pl->total;
        return CQSA_OK;
    }

    // chunked plan
    pl->chunked = true;
    pl->kv_splits = 1;
    // the planner's choice is the fused fold: the same formula with no partial written and read back (the
    // full-size softmax-stress case, 16 KV chunks: 1028 ms with the merge kernel, 1004 ms fused)
    pl->merge = req_merge == 0 ? CQSA_MERGE_FUSED : req_merge;
    int64_t qc = opt.q_chunk > 0 ? std::min(opt.q_chunk, P.Nq) : 0;
    int64_t kc = opt.kv_chunk > 0 ? std::min(opt.kv_chunk, P.Nk) : 0;
    if (long_keys) {
        qc = P.Nq;
        kc = kKvResident;
    } else if (qc > 0 && kc > 0) {
        // both forced
    } else if (!P.streamed) {
        if (qc == 0) qc = P.Nq;
        if (kc == 0) kc = P.Nk;
    } else {
        // streamed: smallest number of Q chunks that leaves room for KV chunks of at least kKvMinStream
        // keys; when even that does not fit, the smallest chunk grain
        int64_t best_q = 0, best_k = 0;
        const int64_t floors[2] = {std::min<int64_t>(kKvMinStream, P.Nk), std::min<int64_t>(kRowGrain, P.Nk)};
        for (int f = 0; f < 2 && best_q == 0; ++f) {
            // KV chunk candidates: multiples of the grain, clipped to Nk
            auto kv_of = [&](int64_t g) { return std::min<int64_t>(P.Nk, g * kRowGrain); };
            const int64_t g_lo = kc > 0 ? 0 : ceil_div(floors[f], kRowGrain);
            const int64_t g_hi = kc > 0 ? 0 : std::max<int64_t>(g_lo, ceil_div(std::min<int64_t>(kKvCap, P.Nk), kRowGrain));
            const int64_t k_first = kc > 0 ? kc : kv_of(g_lo);
            for (int64_t nq = 1;; ++nq) {
                const int64_t cand =
                    qc > 0 ? qc
                           : std::min<int64_t>(P.Nq, (int64_t)align_up((uint64_t)ceil_div(P.Nq, nq), kRowGrain));
                if (chunk_bytes(P, cand, k_first, pl->merge, false, pl) <= budget) {
                    int64_t best = k_first;
                    if (kc == 0) {
                        // bisection for the largest feasible grain multiple: bytes grow with the chunk
                        int64_t lo = g_lo, hi = g_hi;
                        while (lo < hi) {
                            const int64_t mid = lo + (hi - lo + 1) / 2;
                            if (chunk_bytes(P, cand, kv_of(mid), pl->merge, false, pl) <= budget)
                                lo = mid;
                            else
                                hi = mid - 1;
                        }
                        best = kv_of(lo);
                    }
                    best_q = cand;
                    best_k = best;
                    break;
                }
                if (qc > 0 || cand <= kRowGrain) break;
            }
        }
        if (best_q == 0) {
            const uint64_t need = chunk_bytes(P, std::min<int64_t>(P.Nq, qc > 0 ? qc : kRowGrain),
                                              kc > 0 ? kc : floors[1], pl->merge, false, pl);
            return fail(CQSA_ERR_BUDGET, "mem_budget too small: the smallest plan needs %llu bytes (x 1/0.85 = %llu)",
                        (unsigned long long)need, (unsigned long long)(need / kSafety) + 1);
        }
        qc = best_q;
        kc = best_k;
    }
    pl->q_chunk = qc;
    pl->kv_chunk = kc;
    pl->n_q = ceil_div(P.Nq, qc);
    pl->n_kv = ceil_div(P.Nk, kc);
    const uint64_t need = chunk_bytes(P, qc, kc, pl->merge, true, pl);
    if (need > budget)
        return fail(CQSA_ERR_BUDGET, "mem_budget too small for q_chunk %lld, kv_chunk %lld: needs %llu bytes (x 1/0.85 = %llu)",
                    (long long)qc, (long long)kc, (unsigned long long)need,
                    (unsigned long long)(need / kSafety) + 1);
    if (pl->n_kv == 1) pl->merge = 0;
    pl->info.q_chunk = qc;
    pl->info.kv_chunk = kc;
    pl->info.n_q_chunks = pl->n_q;
    pl->info.kv_splits = 1;
    pl->info.merge_mode = pl->merge;
    pl->info.workspace_bytes = pl->total;
    count_chunked(P, pl);
    return CQSA_OK;
}

// ---------------------------------------------------------------------------------------------
// device resources

struct DeviceRes {
    bool init = false;
    int num_cus = 0;
    hipStream_t h2d = nullptr;
    hipStream_t d2h = nullptr;
};
std::mutex g_res_mu;
DeviceRes g_res[64];

cqsa_status device_res(DeviceRes** out) {
    int dev = 0;
    CQSA_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64) return fail(CQSA_ERR_HIP, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_res_mu);
    DeviceRes& r = g_res[dev];
    if (!r.init) {
        CQSA_HIP(hipDeviceGetAttribute(&r.num_cus, hipDeviceAttributeMultiprocessorCount, dev));
        r.init = true;
    }
    *out = &r;
    return CQSA_OK;
}

cqsa_status side_streams(DeviceRes* r) {
    std::lock_guard<std::mutex> lk(g_res_mu);
    if (!r->h2d) CQSA_HIP(hipStreamCreateWithFlags(&r->h2d, hipStreamNonBlocking));
    if (!r->d2h) CQSA_HIP(hipStreamCreateWithFlags(&r->d2h, hipStreamNonBlocking));
    return CQSA_OK;
}

// After a failed call: wait for every stream the call may have issued work on (the caller's stream and
// the library's copy streams), so that no copy or kernel of the failed call still reads or writes
// caller memory (inputs, outputs, workspace) once the error is returned.  Errors met while waiting are
// cleared; the call's first error is the one reported.
void drain_after_failure(hipStream_t st, DeviceRes* r) {
    hipStream_t side[2] = {nullptr, nullptr};
    if (r) {
        std::lock_guard<std::mutex> lk(g_res_mu);
        side[0] = r->h2d;
        side[1] = r->d2h;
    }
    (void)hipStreamSynchronize(st);
    for (hipStream_t s : side)
        if (s) (void)hipStreamSynchronize(s);
    (void)hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Schedule recording (cqsa_schedule_trace): the executors issue every copy, launch, event record and
// event wait through the x_* wrappers below.  With a recorder installed on the calling thread they
// append one line per operation instead of calling HIP (no GPU is touched):
//   copy <stream> R:<lo>:<hi> | W:<lo>:<hi>        a device range the copy reads (D2H) or writes (H2D)
//   kernel <stream> <name> R:<lo>:<hi> ... W:<lo>:<hi> ...   byte ranges (hulls) a launch reads / writes
//   record <stream> <event>,  wait <stream> <event>,  sync <stream>
// Streams and events are numbered in order of first use.

struct Recorder {
    std::string text;
    std::vector<const void*> streams, events;
    uintptr_t next_event = 0x1000;
    int id(std::vector<const void*>& v, const void* p) {
        for (size_t i = 0; i < v.size(); ++i)
            if (v[i] == p) return (int)i;
        v.push_back(p);
        return (int)v.size() - 1;
    }
    void line(const std::string& l) { text += l + "\n"; }
    std::string st(hipStream_t s) { return "s" + std::to_string(id(streams, s)); }
    std::string ev(hipEvent_t e) { return "e" + std::to_string(id(events, e)); }
};
thread_local Recorder* g_rec = nullptr;

std::string rng(char kind, const void* lo, const void* hi) {
    return std::string(1, kind) + ":" + std::to_string((unsigned long long)(uintptr_t)lo) + ":" +
           std::to_string((unsigned long long)(uintptr_t)hi);
}

hipError_t x_record(hipEvent_t e, hipStream_t s) {
    if (g_rec) {
        g_rec->line("record " + g_rec->st(s) + " " + g_rec->ev(e));
        return hipSuccess;
    }
    return hipEventRecord(e, s);
}
hipError_t x_wait(hipStream_t s, hipEvent_t e) {
    if (g_rec) {
        g_rec->line("wait " + g_rec->st(s) + " " + g_rec->ev(e));
        return hipSuccess;
    }
    return hipStreamWaitEvent(s, e, 0);
}
hipError_t x_sync(hipStream_t s) {
    if (g_rec) {
        g_rec->line("sync " + g_rec->st(s));
        return hipSuccess;
    }
    return hipStreamSynchronize(s);
}
hipError_t x_elapsed(float* ms, hipEvent_t a, hipEvent_t b) {
    if (g_rec) {
        *ms = 0.f;
        return hipSuccess;
    }
    return hipEventElapsedTime(ms, a, b);
}
// a 2D copy of height rows of width bytes; the device side's rows are pitch bytes apart
hipError_t x_copy2d(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height,
                    hipMemcpyKind kind, hipStream_t s) {
    if (g_rec) {
        const bool h2d = kind == hipMemcpyHostToDevice;
        const char* dev = static_cast<const char*>(h2d ? dst : src);
        const size_t pitch = h2d ? dpitch : spitch;
        const size_t extent = height == 0 ? 0 : (height - 1) * pitch + width;
        g_rec->line("copy " + g_rec->st(s) + " " + rng(h2d ? 'W' : 'R', dev, dev + extent));
        return hipSuccess;
    }
    return hipMemcpy2DAsync(dst, dpitch, src, spitch, width, height, kind, s);
}
hipError_t x_copy(void* dst, const void* src, size_t bytes, hipMemcpyKind kind, hipStream_t s) {
    if (g_rec) return x_copy2d(dst, bytes, src, bytes, bytes, 1, kind, s);
    return hipMemcpyAsync(dst, src, bytes, kind, s);
}

// the byte hull of rows [r0, r1) of a [B, H, *, D] view with element strides (sb, sh, sn)
std::string view_hull(char kind, const void* base, int64_t es, int64_t B, int64_t H, int64_t sb, int64_t sh,
                      int64_t sn, int64_t r0, int64_t r1, int64_t D) {
    const char* p = static_cast<const char*>(base);
    if (r1 <= r0 || B <= 0 || H <= 0) return "";
    return rng(kind, p + r0 * sn * es, p + ((B - 1) * sb + (H - 1) * sh + (r1 - 1) * sn + D) * es);
}

// ---------------------------------------------------------------------------------------------
// chunk copies between a [B, H, N, D] tensor (any strides) and a compact device buffer

struct Compact {
    int64_t sb, sh, sn;
};

// Device layout for rows [ra, ra + rn) of t: keeps the host's order of heads and rows, so that a
// token-major host tensor moves in one contiguous block per batch entry.
Compact compact_for(const View& t, int64_t rn) {
    const bool token_major = t.H > 1 && t.sh < t.sn;
    if (token_major) return Compact{rn * t.H * t.D, t.D, t.H * t.D};
    return Compact{t.H * rn * t.D, rn * t.D, t.D};
}

// Copy rows [ra, ra + rn) of host/device tensor t to or from the compact device buffer dev.
cqsa_status copy_rows(const View& t, int64_t ra, int64_t rn, char* dev, bool to_device, hipStream_t st) {
    if (rn <= 0) return CQSA_OK;
    const Compact c = compact_for(t, rn);
    const hipMemcpyKind kind = to_device ? hipMemcpyHostToDevice : hipMemcpyDeviceToHost;
    const size_t es = (size_t)t.es;
    const bool token_major = t.H > 1 && t.sh < t.sn;
    for (int64_t b = 0; b < t.B; ++b) {
        char* hb = t.data + (size_t)(b * t.sb + ra * t.sn) * es;
        char* db = dev + (size_t)(b * c.sb) * es;
        if (token_major && t.sh == t.D && t.sn == t.H * t.D) {
            const size_t bytes = (size_t)rn * t.H * t.D * es;
            if (to_device)
                CQSA_HIP(x_copy(db, hb, bytes, kind, st));
            else
                CQSA_HIP(x_copy(hb, db, bytes, kind, st));
        } else if (!token_major && t.sn == t.D && t.sh >= rn * t.D) {
            // each head: rn * D contiguous elements; heads at stride sh
            const size_t width = (size_t)rn * t.D * es;
            if (to_device)
                CQSA_HIP(x_copy2d(db, (size_t)c.sh * es, hb, (size_t)t.sh * es, width, (size_t)t.H, kind, st));
            else
                CQSA_HIP(x_copy2d(hb, (size_t)t.sh * es, db, (size_t)c.sh * es, width, (size_t)t.H, kind, st));
        } else {
            for (int64_t h = 0; h < t.H; ++h) {
                char* hh = hb + (size_t)(h * t.sh) * es;
                char* dh = db + (size_t)(h * c.sh) * es;
                const size_t width = (size_t)t.D * es;
                if (to_device)
                    CQSA_HIP(x_copy2d(dh, (size_t)c.sn * es, hh, (size_t)t.sn * es, width, (size_t)rn, kind, st));
                else
                    CQSA_HIP(x_copy2d(hh, (size_t)t.sn * es, dh, (size_t)c.sn * es, width, (size_t)rn, kind, st));
            }
        }
    }
    return CQSA_OK;
}

// lse rows [ra, ra + rn) of a [B, Hq, Nq] fp32 array <-> compact [B, Hq, rn]
cqsa_status copy_lse_rows(float* host, const float* dev, int64_t B, int64_t Hq, int64_t Nq, int64_t ra, int64_t rn,
                          hipStream_t st) {
    if (rn <= 0) return CQSA_OK;
    CQSA_HIP(x_copy2d(host + ra, (size_t)Nq * 4, dev, (size_t)rn * 4, (size_t)rn * 4, (size_t)(B * Hq),
                      hipMemcpyDeviceToHost, st));
    return CQSA_OK;
}

// ---------------------------------------------------------------------------------------------
// kernel argument helpers

FwdArgs base_args(const Problem& P) {
    FwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.B = (int32_t)P.B;
    a.Hq = (int32_t)P.Hq;
    a.Hkv = (int32_t)P.Hkv;
    a.group = (int32_t)(P.Hq / P.Hkv);
    a.causal = P.causal ? 1 : 0;
    a.scale_log2 = P.scale * 1.44269504088896340736f;
    a.n_splits = 1;
    a.p_split = P.p_split;
    return a;
}

void set_q(FwdArgs& a, const char* data, int64_t sb, int64_t sh, int64_t sn) {
    a.q = reinterpret_cast<const uint16_t*>(data);
    a.q_sb = sb;
    a.q_sh = sh;
    a.q_sn = sn;
}
void set_k(FwdArgs& a, const char* data, int64_t sb, int64_t sh, int64_t sn) {
    a.k = reinterpret_cast<const uint16_t*>(data);
    a.k_sb = sb;
    a.k_sh = sh;
    a.k_sn = sn;
}
void set_v(FwdArgs& a, const char* data, int64_t sb, int64_t sh, int64_t sn) {
    a.v = reinterpret_cast<const uint16_t*>(data);
    a.v_sb = sb;
    a.v_sh = sh;
    a.v_sn = sn;
}

// Failure injection for the error-path tests (cqsa_set_test_controls): with a limit n >= 0, every
// forward launch of a call after its first n fails as a launch error would, once the call's earlier
// copies and launches have been issued.  The count restarts at each public call; -1 = off.
std::atomic<int64_t> g_fail_after{-1};
thread_local int64_t g_fwd_launches = 0;

bool injected_launch_failure() {
    const int64_t n = g_fail_after.load(std::memory_order_relaxed);
    return n >= 0 && g_fwd_launches++ >= n;
}

cqsa_status run_fwd(const Problem& P, FwdArgs& a, hipStream_t st) {
    const int bm = fwd_block_m((int)P.D, P.p_split);
    const int64_t rows = a.r1 - a.r0;
    if (rows <= 0) return CQSA_OK;
    const int64_t n_qt = ceil_div(rows, bm);
    if (n_qt > 0x7FFFFFFF) return fail(CQSA_ERR_UNSUPPORTED, "too many query tiles");
    a.n_qt = (int32_t)n_qt;
    if (g_rec) {
        const int64_t D = P.D;
        std::string l = "kernel " + g_rec->st(st) + " fwd";
        l += " " + view_hull('R', a.q, 2, a.B, a.Hq, a.q_sb, a.q_sh, a.q_sn, a.r0, a.r1, D);
        l += " " + view_hull('R', a.k, 2, a.B, a.Hkv, a.k_sb, a.k_sh, a.k_sn, a.k_lo, a.k_hi, D);
        l += " " + view_hull('R', a.v, 2, a.B, a.Hkv, a.v_sb, a.v_sh, a.v_sn, a.k_lo, a.k_hi, D);
        if (a.mode == FWD_FINAL) {
            const int64_t es = a.out_dtype == ET_F32 ? 4 : 2;
            l += " " + view_hull('W', a.out, es, a.B, a.Hq, a.o_sb, a.o_sh, a.o_sn, a.r0, a.r1, D);
            if (a.lse) l += " " + view_hull('W', a.lse, 4, a.B, a.Hq, a.l_sb, a.l_sh, 1, a.r0, a.r1, 1);
        } else {
            // accumulator rows ((split B + b) Hq + h) acc_rows + i, i in [r0, r1)
            const int64_t heads = (int64_t)a.n_splits * a.B * a.Hq;
            const std::string o = view_hull('W', a.acc_o, 4, 1, heads, 0, a.acc_rows * D, D, a.r0, a.r1, D);
            const std::string ml = view_hull('W', a.acc_ml, 4, 1, heads, 0, a.acc_rows * 2, 2, a.r0, a.r1, 2);
            l += " " + o + " " + ml;
            if (a.mode == FWD_ACCUM) l += " R" + o.substr(1) + " R" + ml.substr(1);
        }
        g_rec->line(l);
        return CQSA_OK;
    }
    if (injected_launch_failure()) return fail(CQSA_ERR_HIP, "forward kernel launch failed: injected (cqsa_set_test_controls)");
    const hipError_t e = launch_fwd(a, (int)P.D, P.dtype == CQSA_F16 ? ET_F16 : ET_BF16, st);
    if (e != hipSuccess) return fail(CQSA_ERR_HIP, "forward kernel launch failed: %s", hipGetErrorString(e));
    return CQSA_OK;
}

cqsa_status run_merge(MergeArgs& m, hipStream_t st) {
    if (g_rec) {
        const int64_t D = m.D, heads = (int64_t)m.B * m.Hq;
        std::string l = "kernel " + g_rec->st(st) + " merge";
        for (int p = 0; p < m.n_parts; ++p) {
            l += " " + view_hull('R', m.part_o[p], 4, 1, heads, 0, m.rows_per_head * D, D, m.i_lo, m.i_hi, D);
            l += " " + view_hull('R', m.part_ml[p], 4, 1, heads, 0, m.rows_per_head * 2, 2, m.i_lo, m.i_hi, 2);
        }
        if (m.final_out) {
            const int64_t es = m.out_dtype == ET_F32 ? 4 : 2;
            l += " " + view_hull('W', m.out, es, m.B, m.Hq, m.o_sb, m.o_sh, m.o_sn, 0, m.i_hi - m.i_lo, D);
            if (m.lse) l += " " + view_hull('W', m.lse, 4, m.B, m.Hq, m.l_sb, m.l_sh, 1, 0, m.i_hi - m.i_lo, 1);
        } else {
            l += " " + view_hull('W', m.o_out, 4, 1, heads, 0, m.rows_per_head * D, D, m.i_lo, m.i_hi, D);
            l += " " + view_hull('W', m.ml_out, 4, 1, heads, 0, m.rows_per_head * 2, 2, m.i_lo, m.i_hi, 2);
        }
        g_rec->line(l);
        return CQSA_OK;
    }
    const hipError_t e = launch_merge(m, st);
    if (e != hipSuccess) return fail(CQSA_ERR_HIP, "merge kernel launch failed: %s", hipGetErrorString(e));
    return CQSA_OK;
}

int elem_type(int dt) { return dt == CQSA_F16 ? ET_F16 : (dt == CQSA_BF16 ? ET_BF16 : ET_F32); }

// ---------------------------------------------------------------------------------------------
// executors

// Every operand on the device, no forced chunking: one pass over all keys, optionally as side-by-side
// KV splits merged by one merge-and-normalise pass.
cqsa_status exec_single(const Problem& P, const Plan& pl, char* ws, hipStream_t st) {
    FwdArgs a = base_args(P);
    set_q(a, P.q.data, P.q.sb, P.q.sh, P.q.sn);
    set_k(a, P.k.data, P.k.sb, P.k.sh, P.k.sn);
    set_v(a, P.v.data, P.v.sb, P.v.sh, P.v.sn);
    a.r0 = 0;
    a.r1 = P.Nq;
    a.k_lo = 0;
    a.k_hi = P.Nk;
    a.causal_delta = P.Nk - P.Nq;
    if (pl.kv_splits <= 1) {
        a.split_len = P.Nk;
        a.mode = FWD_FINAL;
        a.out = P.out.data;
        a.out_dtype = elem_type(P.out.dtype);
        a.o_sb = P.out.sb;
        a.o_sh = P.out.sh;
        a.o_sn = P.out.sn;
        a.lse = P.want_lse ? P.lse : nullptr;
        a.l_sb = P.Hq * P.Nq;
        a.l_sh = P.Nq;
        return run_fwd(P, a, st);
    }
    const int S = pl.kv_splits;
    a.n_splits = S;
    a.split_len = align_up(ceil_div(P.Nk, S), 64);
    a.mode = FWD_PARTIAL;
    a.acc_o = reinterpret_cast<float*>(ws + pl.off_part_o);
    a.acc_ml = reinterpret_cast<float*>(ws + pl.off_part_ml);
    a.acc_rows = P.Nq;
    cqsa_status s = run_fwd(P, a, st);
    if (s != CQSA_OK) return s;
    MergeArgs m;
    std::memset(&m, 0, sizeof m);
    const uint64_t rows = (uint64_t)P.B * P.Hq * P.Nq;
    for (int p = 0; p < S; ++p) {
        m.part_o[p] = a.acc_o + (uint64_t)p * rows * P.D;
        m.part_ml[p] = a.acc_ml + (uint64_t)p * rows * 2;
    }
    m.n_parts = S;
    m.D = (int32_t)P.D;
    m.B = (int32_t)P.B;
    m.Hq = (int32_t)P.Hq;
    m.rows_per_head = P.Nq;
    m.i_lo = 0;
    m.i_hi = P.Nq;
    m.final_out = 1;
    m.out_dtype = elem_type(P.out.dtype);
    m.out = P.out.data;
    m.o_sb = P.out.sb;
    m.o_sh = P.out.sh;
    m.o_sn = P.out.sn;
    m.lse = P.want_lse ? P.lse : nullptr;
    m.l_sb = P.Hq * P.Nq;
    m.l_sh = P.Nq;
    return run_merge(m, st);
}

struct EventSet {
    std::vector<hipEvent_t> evs;
    ~EventSet() {
        for (hipEvent_t e : evs) (void)hipEventDestroy(e);
    }
    cqsa_status make(hipEvent_t* e, bool timing) {
        if (g_rec) {   // a distinct handle that no HIP call ever sees
            *e = reinterpret_cast<hipEvent_t>(g_rec->next_event += 0x10);
            return CQSA_OK;
        }
        hipError_t r = hipEventCreateWithFlags(e, timing ? hipEventDefault : hipEventDisableTiming);
        if (r != hipSuccess) return fail(CQSA_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(r));
        evs.push_back(*e);
        return CQSA_OK;
    }
};

struct TimedCopy {
    hipEvent_t start, stop;
};


// Q chunks x KV chunks; operands may live in pinned host memory.
cqsa_status exec_chunked(const Problem& P, const Plan& pl, char* ws, hipStream_t st, DeviceRes* res,
                         cqsa_plan_info* info) {
    // out and lse of a Q chunk are staged in the workspace when they live on the host; the next Q chunk
    // writes the same staging, so it waits for the D2H copy of either one
    const bool host_out = P.out.host || (P.want_lse && P.lse_host);
    const bool need_side = P.q.host || P.k.host || P.v.host || host_out;
    hipStream_t h2d = st, d2h = st;
    if (need_side) {
        CQSA_TRY(side_streams(res));
        h2d = res->h2d;
        d2h = res->d2h;
    }
    EventSet es;
    hipEvent_t ev_start, ev_qcopy, ev_qfree, ev_fin, ev_d2h, ev_copy[2], ev_comp[2];
    CQSA_TRY(es.make(&ev_start, false));
    CQSA_TRY(es.make(&ev_qcopy, false));
    CQSA_TRY(es.make(&ev_qfree, false));
    CQSA_TRY(es.make(&ev_fin, false));
    CQSA_TRY(es.make(&ev_d2h, false));
    for (int i = 0; i < 2; ++i) {
        CQSA_TRY(es.make(&ev_copy[i], false));
        CQSA_TRY(es.make(&ev_comp[i], false));
    }
    std::vector<TimedCopy> h2d_t, d2h_t;
    auto timed = [&](std::vector<TimedCopy>& v, TimedCopy* tc) -> cqsa_status {
        CQSA_TRY(es.make(&tc->start, true));
        CQSA_TRY(es.make(&tc->stop, true));
        v.push_back(*tc);
        return CQSA_OK;
    };
    // side streams start after the work already queued on the compute stream
    CQSA_HIP(x_record(ev_start, st));
    if (need_side) {
        CQSA_HIP(x_wait(h2d, ev_start));
        CQSA_HIP(x_wait(d2h, ev_start));
    }
    bool qfree_recorded = false, d2h_recorded = false;
    bool comp_recorded[2] = {false, false};
    int64_t pair = 0;

    float* acc_o = reinterpret_cast<float*>(ws + pl.off_acc_o);
    float* acc_ml = reinterpret_cast<float*>(ws + pl.off_acc_ml);
    float* part_o = reinterpret_cast<float*>(ws + pl.off_part_o);
    float* part_ml = reinterpret_cast<float*>(ws + pl.off_part_ml);

    for (int64_t qa = 0; qa < P.Nq; qa += pl.q_chunk) {
        const int64_t qn = std::min(pl.q_chunk, P.Nq - qa);
        FwdArgs a = base_args(P);
        // ---- Q view
        if (P.q.host) {
            if (qfree_recorded) CQSA_HIP(x_wait(h2d, ev_qfree));
            TimedCopy tc;
            CQSA_TRY(timed(h2d_t, &tc));
            CQSA_HIP(x_record(tc.start, h2d));
            CQSA_TRY(copy_rows(P.q, qa, qn, ws + pl.off_q, true, h2d));
            CQSA_HIP(x_record(tc.stop, h2d));
            CQSA_HIP(x_record(ev_qcopy, h2d));
            CQSA_HIP(x_wait(st, ev_qcopy));
            const Compact c = compact_for(P.q, qn);
            set_q(a, ws + pl.off_q, c.sb, c.sh, c.sn);
        } else {
            set_q(a, P.q.data + (size_t)(qa * P.q.sn) * 2, P.q.sb, P.q.sh, P.q.sn);
        }
        // ---- output view for this chunk
        char* out_base;
        int64_t o_sb, o_sh, o_sn;
        if (P.out.host) {
            const Compact c = compact_for(P.out, qn);
            out_base = ws + pl.off_out;
            o_sb = c.sb;
            o_sh = c.sh;
            o_sn = c.sn;
        } else {
            out_base = P.out.data + (size_t)(qa * P.out.sn) * P.out.es;
            o_sb = P.out.sb;
            o_sh = P.out.sh;
            o_sn = P.out.sn;
        }
        float* lse_base = nullptr;
        int64_t l_sb = 0, l_sh = 0;
        if (P.want_lse) {
            if (P.lse_host) {
                lse_base = reinterpret_cast<float*>(ws + pl.off_lse);
                l_sb = P.Hq * qn;
                l_sh = qn;
            } else {
                lse_base = P.lse + qa;
                l_sb = P.Hq * P.Nq;
                l_sh = P.Nq;
            }
        }
        const int64_t pos0 = P.Nk - P.Nq + qa;  // key position of local query row 0
        const int64_t kv_end = P.causal ? std::min(P.Nk, pos0 + qn) : P.Nk;
        const int64_t nkv = ceil_div(kv_end, pl.kv_chunk);
        const bool single = nkv == 1;

        for (int64_t kc = 0; kc < nkv; ++kc) {
            const int64_t ka = kc * pl.kv_chunk;
            const int64_t kn = std::min(pl.kv_chunk, kv_end - ka);
            const int buf = (int)(pair & 1);
            // ---- K/V views (copy into buffer `buf` after the compute that last read it)
            if (P.k.host || P.v.host) {
                if (comp_recorded[buf]) CQSA_HIP(x_wait(h2d, ev_comp[buf]));
                TimedCopy tc;
                CQSA_TRY(timed(h2d_t, &tc));
                CQSA_HIP(x_record(tc.start, h2d));
                if (P.k.host) CQSA_TRY(copy_rows(P.k, ka, kn, ws + pl.off_k[buf], true, h2d));
                if (P.v.host) CQSA_TRY(copy_rows(P.v, ka, kn, ws + pl.off_v[buf], true, h2d));
                CQSA_HIP(x_record(tc.stop, h2d));
                CQSA_HIP(x_record(ev_copy[buf], h2d));
                CQSA_HIP(x_wait(st, ev_copy[buf]));
            }
            if (P.k.host) {
                const Compact c = compact_for(P.k, kn);
                set_k(a, ws + pl.off_k[buf], c.sb, c.sh, c.sn);
            } else {
                set_k(a, P.k.data + (size_t)(ka * P.k.sn) * 2, P.k.sb, P.k.sh, P.k.sn);
            }
            if (P.v.host) {
                const Compact c = compact_for(P.v, kn);
                set_v(a, ws + pl.off_v[buf], c.sb, c.sh, c.sn);
            } else {
                set_v(a, P.v.data + (size_t)(ka * P.v.sn) * 2, P.v.sb, P.v.sh, P.v.sn);
            }
            a.k_lo = 0;
            a.k_hi = kn;
            a.split_len = kn;
            a.causal_delta = pos0 - ka;
            a.r0 = P.causal ? std::max<int64_t>(0, ka - pos0) : 0;
            a.r1 = qn;
            a.acc_rows = qn;
            if (single) {
                if (host_out && d2h_recorded) CQSA_HIP(x_wait(st, ev_d2h));
                a.mode = FWD_FINAL;
                a.out = out_base;
                a.out_dtype = elem_type(P.out.dtype);
                a.o_sb = o_sb;
                a.o_sh = o_sh;
                a.o_sn = o_sn;
                a.lse = lse_base;
                a.l_sb = l_sb;
                a.l_sh = l_sh;
                CQSA_TRY(run_fwd(P, a, st));
            } else if (kc == 0 || pl.merge == CQSA_MERGE_FUSED) {
                a.mode = kc == 0 ? FWD_PARTIAL : FWD_ACCUM;
                a.acc_o = acc_o;
                a.acc_ml = acc_ml;
                CQSA_TRY(run_fwd(P, a, st));
            } else {
                a.mode = FWD_PARTIAL;
                a.acc_o = part_o;
                a.acc_ml = part_ml;
                CQSA_TRY(run_fwd(P, a, st));
                MergeArgs m;
                std::memset(&m, 0, sizeof m);
                m.part_o[0] = acc_o;
                m.part_ml[0] = acc_ml;
                m.part_o[1] = part_o;
                m.part_ml[1] = part_ml;
                m.n_parts = 2;
                m.D = (int32_t)P.D;
                m.B = (int32_t)P.B;
                m.Hq = (int32_t)P.Hq;
                m.rows_per_head = qn;
                m.i_lo = a.r0;
                m.i_hi = qn;
                m.o_out = acc_o;
                m.ml_out = acc_ml;
                CQSA_TRY(run_merge(m, st));
            }
            CQSA_HIP(x_record(ev_comp[buf], st));
            comp_recorded[buf] = true;
            ++pair;
        }
        if (!single) {
            if (host_out && d2h_recorded) CQSA_HIP(x_wait(st, ev_d2h));
            MergeArgs m;
            std::memset(&m, 0, sizeof m);
            m.part_o[0] = acc_o;
            m.part_ml[0] = acc_ml;
            m.n_parts = 1;
            m.D = (int32_t)P.D;
            m.B = (int32_t)P.B;
            m.Hq = (int32_t)P.Hq;
            m.rows_per_head = qn;
            m.i_lo = 0;
            m.i_hi = qn;
            m.final_out = 1;
            m.out_dtype = elem_type(P.out.dtype);
            m.out = out_base;
            m.o_sb = o_sb;
            m.o_sh = o_sh;
            m.o_sn = o_sn;
            m.lse = lse_base;
            m.l_sb = l_sb;
            m.l_sh = l_sh;
            CQSA_TRY(run_merge(m, st));
        }
        CQSA_HIP(x_record(ev_qfree, st));
        qfree_recorded = true;
        if (host_out) {
            CQSA_HIP(x_record(ev_fin, st));
            CQSA_HIP(x_wait(d2h, ev_fin));
            TimedCopy tc;
            CQSA_TRY(timed(d2h_t, &tc));
            CQSA_HIP(x_record(tc.start, d2h));
            if (P.out.host) CQSA_TRY(copy_rows(P.out, qa, qn, ws + pl.off_out, false, d2h));
            if (P.want_lse && P.lse_host)
                CQSA_TRY(copy_lse_rows(P.lse, reinterpret_cast<float*>(ws + pl.off_lse), P.B, P.Hq, P.Nq, qa, qn, d2h));
            CQSA_HIP(x_record(tc.stop, d2h));
            CQSA_HIP(x_record(ev_d2h, d2h));
            d2h_recorded = true;
        }
    }
    // join the side streams back into the compute stream
    if (need_side) {
        hipEvent_t j1, j2;
        CQSA_TRY(es.make(&j1, false));
        CQSA_TRY(es.make(&j2, false));
        CQSA_HIP(x_record(j1, h2d));
        CQSA_HIP(x_record(j2, d2h));
        CQSA_HIP(x_wait(st, j1));
        CQSA_HIP(x_wait(st, j2));
        CQSA_HIP(x_sync(st));
        double h = 0, d = 0;
        for (auto& t : h2d_t) {
            float ms = 0;
            CQSA_HIP(x_elapsed(&ms, t.start, t.stop));
            h += ms;
        }
        for (auto& t : d2h_t) {
            float ms = 0;
            CQSA_HIP(x_elapsed(&ms, t.start, t.stop));
            d += ms;
        }
        if (info) {
            info->h2d_ms = h;
            info->d2h_ms = d;
        }
    }
    return CQSA_OK;
}

// The quorum-set schedule (make_plan_cqs): the accumulator for every query row starts as the
// identity (0, -inf, 0); each subproblem stages the parts of its owned non-empty pairs (host
// operands, into one of two staging sets that alternate) and folds one forward launch per pair into
// the accumulator rows of the pair's query part; a last pass normalises (and ships host output in
// query-part-sized pieces).
cqsa_status exec_cqs(const Problem& P, const Plan& pl, char* ws, hipStream_t st, DeviceRes* res,
                     cqsa_plan_info* info) {
    const int c = pl.cqs_c;
    const bool host_in = P.q.host || P.k.host || P.v.host;
    const bool host_out = P.out.host || (P.want_lse && P.lse_host);
    hipStream_t h2d = st, d2h = st;
    if (host_in || host_out) {
        CQSA_TRY(side_streams(res));
        h2d = res->h2d;
        d2h = res->d2h;
    }
    EventSet es;
    hipEvent_t ev_start, ev_fin, ev_d2h, ev_copy[2], ev_comp[2];
    CQSA_TRY(es.make(&ev_start, false));
    CQSA_TRY(es.make(&ev_fin, false));
    CQSA_TRY(es.make(&ev_d2h, false));
    for (int i = 0; i < 2; ++i) {
        CQSA_TRY(es.make(&ev_copy[i], false));
        CQSA_TRY(es.make(&ev_comp[i], false));
    }
    std::vector<TimedCopy> h2d_t, d2h_t;
    auto timed = [&](std::vector<TimedCopy>& v, TimedCopy* tc) -> cqsa_status {
        CQSA_TRY(es.make(&tc->start, true));
        CQSA_TRY(es.make(&tc->stop, true));
        v.push_back(*tc);
        return CQSA_OK;
    };
    CQSA_HIP(x_record(ev_start, st));
    if (host_in || host_out) {
        CQSA_HIP(x_wait(h2d, ev_start));
        CQSA_HIP(x_wait(d2h, ev_start));
    }
    float* acc_o = reinterpret_cast<float*>(ws + pl.off_acc_o);
    float* acc_ml = reinterpret_cast<float*>(ws + pl.off_acc_ml);
    {
        MergeArgs m;   // no parts: writes the identity triple
        std::memset(&m, 0, sizeof m);
        m.n_parts = 0;
        m.D = (int32_t)P.D;
        m.B = (int32_t)P.B;
        m.Hq = (int32_t)P.Hq;
        m.rows_per_head = P.Nq;
        m.i_lo = 0;
        m.i_hi = P.Nq;
        m.o_out = acc_o;
        m.ml_out = acc_ml;
        CQSA_TRY(run_merge(m, st));
    }
    const uint64_t qrow = (uint64_t)P.B * P.Hq * P.D * 2, kvrow = (uint64_t)P.B * P.Hkv * P.D * 2;
    const int bm = wave_block_m((int)P.D, P.p_split);
    const int dt = P.dtype == CQSA_F16 ? ET_F16 : ET_BF16;
    bool comp_recorded[2] = {false, false};
    int run = 0;
    std::vector<uint64_t> qoff(c), koff(c), voff(c);
    for (const Plan::CqsWave& wv : pl.cqs_waves) {
        const int buf = pl.cqs_nbuf == 2 ? (run & 1) : 0;
        char* stg = ws + pl.off_stage[buf];
        if (host_in) {
            if (comp_recorded[buf]) CQSA_HIP(x_wait(h2d, ev_comp[buf]));
            TimedCopy tc;
            CQSA_TRY(timed(h2d_t, &tc));
            CQSA_HIP(x_record(tc.start, h2d));
            uint64_t o = 0;
            for (int a = 0; a < c; ++a)
                if (wv.qp[a] && P.q.host) {
                    const int64_t lo = part_lo(P.Nq, c, a), n = part_lo(P.Nq, c, a + 1) - lo;
                    qoff[a] = o;
                    CQSA_TRY(copy_rows(P.q, lo, n, stg + o, true, h2d));
                    o = align_up(o + (uint64_t)n * qrow, 256);
                }
            for (int b = 0; b < c; ++b)
                if (wv.kp[b]) {
                    const int64_t lo = part_lo(P.Nk, c, b), n = part_lo(P.Nk, c, b + 1) - lo;
                    if (P.k.host) {
                        koff[b] = o;
                        CQSA_TRY(copy_rows(P.k, lo, n, stg + o, true, h2d));
                        o = align_up(o + (uint64_t)n * kvrow, 256);
                    }
                    if (P.v.host) {
                        voff[b] = o;
                        CQSA_TRY(copy_rows(P.v, lo, n, stg + o, true, h2d));
                        o = align_up(o + (uint64_t)n * kvrow, 256);
                    }
                }
            CQSA_HIP(x_record(tc.stop, h2d));
            CQSA_HIP(x_record(ev_copy[buf], h2d));
            CQSA_HIP(x_wait(st, ev_copy[buf]));
        }
        for (const Plan::CqsLaunch& L : wv.launches) {
            // the launch's key parts (ascending) and query parts with their key masks
            std::vector<int> ks, qs;
            for (const auto& pr : L.pairs) {
                if (std::find(ks.begin(), ks.end(), pr.second) == ks.end()) ks.push_back(pr.second);
                if (qs.empty() || qs.back() != pr.first) qs.push_back(pr.first);
            }
            std::sort(ks.begin(), ks.end());
            if (ks.size() > 32 || qs.size() > 32)   // the planner's blocks hold at most 32 of each
                return fail(CQSA_ERR_INVALID, "internal: a wave launch with %zu query and %zu key parts", qs.size(),
                            ks.size());
            WaveTable t;
            std::memset(&t, 0, sizeof t);
            t.n_k = (int32_t)ks.size();
            t.n_q = (int32_t)qs.size();
            t.q_layout = P.q.host ? (P.q.H > 1 && P.q.sh < P.q.sn ? WAVE_COMPACT_TOKEN : WAVE_COMPACT_HEAD) : WAVE_STRIDED;
            t.k_layout = P.k.host ? (P.k.H > 1 && P.k.sh < P.k.sn ? WAVE_COMPACT_TOKEN : WAVE_COMPACT_HEAD) : WAVE_STRIDED;
            t.v_layout = P.v.host ? (P.v.H > 1 && P.v.sh < P.v.sn ? WAVE_COMPACT_TOKEN : WAVE_COMPACT_HEAD) : WAVE_STRIDED;
            t.H_q = (int32_t)P.Hq;
            t.H_kv = (int32_t)P.Hkv;
            for (int u = 0; u < t.n_k; ++u) {
                const int b = ks[u];
                const int64_t lo = part_lo(P.Nk, c, b);
                WaveK& K = t.ki[u];
                K.k = reinterpret_cast<const uint16_t*>(P.k.host ? stg + koff[b] : P.k.data + (size_t)(lo * P.k.sn) * 2);
                K.v = reinterpret_cast<const uint16_t*>(P.v.host ? stg + voff[b] : P.v.data + (size_t)(lo * P.v.sn) * 2);
                K.lo = lo;
                K.n = (int32_t)(part_lo(P.Nk, c, b + 1) - lo);
            }
            // query parts, the ones with the most key rows first (they finish last)
            std::vector<std::pair<int64_t, int>> order;
            std::vector<uint32_t> mask(c, 0u);
            for (const auto& pr : L.pairs) {
                const int u = (int)(std::find(ks.begin(), ks.end(), pr.second) - ks.begin());
                mask[pr.first] |= 1u << u;
            }
            for (int a : qs) {
                int64_t keys = 0;
                for (int u = 0; u < t.n_k; ++u)
                    if ((mask[a] >> u) & 1u) keys += t.ki[u].n;
                order.emplace_back(-keys, a);
            }
            std::sort(order.begin(), order.end());
            int64_t tiles = 0;
            for (int u = 0; u < t.n_q; ++u) {
                const int a = order[u].second;
                const int64_t lo = part_lo(P.Nq, c, a), n = part_lo(P.Nq, c, a + 1) - lo;
                WaveQ& Q = t.qi[u];
                Q.q = reinterpret_cast<const uint16_t*>(P.q.host ? stg + qoff[a] : P.q.data + (size_t)(lo * P.q.sn) * 2);
                Q.lo = lo;
                Q.n = (int32_t)n;
                Q.kmask = mask[a];
                Q.n_qt = (int32_t)ceil_div(n, bm);
                Q.t0 = (int32_t)tiles;
                tiles += Q.n_qt;
            }
            const int64_t blocks = (int64_t)P.B * P.Hq * tiles;
            if (blocks > 0x7FFFFFFF) return fail(CQSA_ERR_UNSUPPORTED, "too many workgroups in one wave launch");
            t.n_tiles = (int32_t)tiles;
            FwdArgs fa = base_args(P);
            if (!P.q.host) set_q(fa, P.q.data, P.q.sb, P.q.sh, P.q.sn);
            if (!P.k.host) set_k(fa, P.k.data, P.k.sb, P.k.sh, P.k.sn);
            if (!P.v.host) set_v(fa, P.v.data, P.v.sb, P.v.sh, P.v.sn);
            fa.causal_delta = P.Nk - P.Nq;
            fa.mode = FWD_ACCUM;
            fa.acc_o = acc_o;
            fa.acc_ml = acc_ml;
            fa.acc_rows = P.Nq;
            if (g_rec) {
                const int64_t D = P.D;
                std::string l = "kernel " + g_rec->st(st) + " wave";
                auto part = [&](char kind, const uint16_t* p0, int layout, int64_t n, int64_t H, int64_t sb, int64_t sh,
                                int64_t sn) {
                    const Compact cc = layout == WAVE_COMPACT_TOKEN ? Compact{n * H * D, D, H * D}
                                       : layout == WAVE_COMPACT_HEAD ? Compact{H * n * D, n * D, D}
                                                                     : Compact{sb, sh, sn};
                    return view_hull(kind, p0, 2, P.B, H, cc.sb, cc.sh, cc.sn, 0, n, D);
                };
                for (int u = 0; u < t.n_q; ++u) {
                    const WaveQ& Q = t.qi[u];
                    l += " " + part('R', Q.q, t.q_layout, Q.n, P.Hq, P.q.sb, P.q.sh, P.q.sn);
                    const std::string o = view_hull('W', fa.acc_o, 4, 1, P.B * P.Hq, 0, P.Nq * D, D, Q.lo, Q.lo + Q.n, D);
                    const std::string ml = view_hull('W', fa.acc_ml, 4, 1, P.B * P.Hq, 0, P.Nq * 2, 2, Q.lo, Q.lo + Q.n, 2);
                    l += " " + o + " " + ml + " R" + o.substr(1) + " R" + ml.substr(1);
                }
                for (int u = 0; u < t.n_k; ++u) {
                    const WaveK& K = t.ki[u];
                    l += " " + part('R', K.k, t.k_layout, K.n, P.Hkv, P.k.sb, P.k.sh, P.k.sn);
                    l += " " + part('R', K.v, t.v_layout, K.n, P.Hkv, P.v.sb, P.v.sh, P.v.sn);
                }
                g_rec->line(l);
            } else {
                const hipError_t e = launch_wave(fa, t, (int)blocks, (int)P.D, dt, st);
                if (e != hipSuccess) return fail(CQSA_ERR_HIP, "wave launch: %s", hipGetErrorString(e));
            }
        }
        CQSA_HIP(x_record(ev_comp[buf], st));
        comp_recorded[buf] = true;
        ++run;
    }
    // normalise
    MergeArgs m;
    std::memset(&m, 0, sizeof m);
    m.part_o[0] = acc_o;
    m.part_ml[0] = acc_ml;
    m.n_parts = 1;
    m.D = (int32_t)P.D;
    m.B = (int32_t)P.B;
    m.Hq = (int32_t)P.Hq;
    m.rows_per_head = P.Nq;
    m.final_out = 1;
    m.out_dtype = elem_type(P.out.dtype);
    const bool lse_host = P.want_lse && P.lse_host;
    const int64_t step = host_out ? std::max<int64_t>(pl.out_rows, 1) : P.Nq;
    bool d2h_recorded = false;
    for (int64_t qa = 0; qa < P.Nq; qa += step) {
        const int64_t qn = std::min(step, P.Nq - qa);
        m.i_lo = qa;
        m.i_hi = qa + qn;
        if (P.out.host) {
            const Compact co = compact_for(P.out, qn);
            m.out = ws + pl.off_out;
            m.o_sb = co.sb;
            m.o_sh = co.sh;
            m.o_sn = co.sn;
        } else {
            m.out = P.out.data + (size_t)(qa * P.out.sn) * P.out.es;
            m.o_sb = P.out.sb;
            m.o_sh = P.out.sh;
            m.o_sn = P.out.sn;
        }
        m.lse = nullptr;
        if (P.want_lse) {
            if (lse_host) {
                m.lse = reinterpret_cast<float*>(ws + pl.off_lse);
                m.l_sb = P.Hq * qn;
                m.l_sh = qn;
            } else {
                m.lse = P.lse + qa;
                m.l_sb = P.Hq * P.Nq;
                m.l_sh = P.Nq;
            }
        }
        if (host_out && d2h_recorded) CQSA_HIP(x_wait(st, ev_d2h));
        CQSA_TRY(run_merge(m, st));
        if (host_out) {
            CQSA_HIP(x_record(ev_fin, st));
            CQSA_HIP(x_wait(d2h, ev_fin));
            TimedCopy tc;
            CQSA_TRY(timed(d2h_t, &tc));
            CQSA_HIP(x_record(tc.start, d2h));
            if (P.out.host) CQSA_TRY(copy_rows(P.out, qa, qn, ws + pl.off_out, false, d2h));
            if (lse_host)
                CQSA_TRY(copy_lse_rows(P.lse, reinterpret_cast<float*>(ws + pl.off_lse), P.B, P.Hq, P.Nq, qa, qn, d2h));
            CQSA_HIP(x_record(tc.stop, d2h));
            CQSA_HIP(x_record(ev_d2h, d2h));
            d2h_recorded = true;
        }
    }
    if (host_in || host_out) {
        hipEvent_t j1, j2;
        CQSA_TRY(es.make(&j1, false));
        CQSA_TRY(es.make(&j2, false));
        CQSA_HIP(x_record(j1, h2d));
        CQSA_HIP(x_record(j2, d2h));
        CQSA_HIP(x_wait(st, j1));
        CQSA_HIP(x_wait(st, j2));
        CQSA_HIP(x_sync(st));
        double h = 0, d = 0;
        for (auto& t : h2d_t) {
            float ms = 0;
            CQSA_HIP(x_elapsed(&ms, t.start, t.stop));
            h += ms;
        }
        for (auto& t : d2h_t) {
            float ms = 0;
            CQSA_HIP(x_elapsed(&ms, t.start, t.stop));
            d += ms;
        }
        if (info) {
            info->h2d_ms = h;
            info->d2h_ms = d;
        }
    }
    return CQSA_OK;
}

cqsa_status build_problem(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v, int is_causal,
                          float scale, const cqsa_tensor* out, float* lse, int want_lse, bool detect, bool allow_null,
                          Problem* P) {
    CQSA_TRY(make_view(q, "q", allow_null, detect, &P->q));
    CQSA_TRY(make_view(k, "k", allow_null, detect, &P->k));
    CQSA_TRY(make_view(v, "v", allow_null, detect, &P->v));
    CQSA_TRY(make_view(out, "out", allow_null, detect, &P->out));
    P->want_lse = want_lse != 0;
    P->lse = lse;
    P->lse_host = false;
    if (P->want_lse && lse && detect) {
        cqsa_tensor lt;
        std::memset(&lt, 0, sizeof lt);
        lt.data = lse;
        lt.dtype = CQSA_F32;
        lt.shape[0] = 1;
        lt.shape[1] = 1;
        lt.shape[2] = 1;
        lt.shape[3] = 1;
        lt.stride[3] = 1;
        CQSA_TRY(locate(&lt, "lse", false, &P->lse_host));
    }
    return check_problem(P, is_causal, scale);
}

// want_lse of cqsa_plan and cqsa_schedule_trace: CQSA_LSE_NONE, _WITH_OUT, _DEVICE or _HOST
cqsa_status check_lse_where(int want_lse) {
    if (want_lse < CQSA_LSE_NONE || want_lse > CQSA_LSE_HOST)
        return fail(CQSA_ERR_INVALID, "want_lse %d is not one of CQSA_LSE_NONE/WITH_OUT/DEVICE/HOST", want_lse);
    return CQSA_OK;
}

bool lse_on_host(int want_lse, bool out_host) {
    return want_lse == CQSA_LSE_HOST || (want_lse == CQSA_LSE_WITH_OUT && out_host);
}

cqsa_status set_precision(const cqsa_options& o, Problem* P) {
    if (o.precision != 0 && o.precision != 1)
        return fail(CQSA_ERR_INVALID, "precision %d is not 0 (operand-rounded P) or 1 (split P)", o.precision);
    P->p_split = o.precision;
    return CQSA_OK;
}

cqsa_status resolve_budget(uint64_t mem_budget, uint64_t* budget) {
    if (mem_budget > 0) {
        *budget = (uint64_t)((double)mem_budget * kSafety);
        return CQSA_OK;
    }
    size_t free_b = 0, total_b = 0;
    CQSA_HIP(hipMemGetInfo(&free_b, &total_b));
    *budget = (uint64_t)((double)free_b * kSafety);
    return CQSA_OK;
}

bool log_enabled() {
    static int v = -1;
    if (v < 0) {
        const char* e = std::getenv("CQSA_LOG");
        v = (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
    }
    return v == 1;
}

}  // namespace

// =============================================================================================
// C ABI

extern "C" {

const char* cqsa_last_error(void) { return g_err.c_str(); }

int32_t cqsa_version(void) { return CQSA_ABI_VERSION; }

cqsa_status cqsa_set_test_controls(int32_t fwd_variant, int64_t fail_after_launches) {
    g_err.clear();
    if (fwd_variant < 0 || fwd_variant >= fwd_variant_count())
        return fail(CQSA_ERR_INVALID, "fwd_variant %d is not in 0..%d", fwd_variant, fwd_variant_count() - 1);
    if (fail_after_launches < -1)
        return fail(CQSA_ERR_INVALID, "fail_after_launches %lld is below -1", (long long)fail_after_launches);
    set_fwd_variant(fwd_variant);
    g_fail_after.store(fail_after_launches, std::memory_order_relaxed);
    return CQSA_OK;
}

uint64_t cqsa_struct_size(int32_t which) {
    switch (which) {
        case 0: return sizeof(cqsa_tensor);
        case 1: return sizeof(cqsa_options);
        case 2: return sizeof(cqsa_plan_info);
        case 3: return sizeof(cqsa_probe_result);
        default: return 0;
    }
}

cqsa_status cqsa_cqs_assign(int32_t c, const int32_t* interest_set, int32_t l, int32_t* owner) {
    g_err.clear();
    if (!owner) return fail(CQSA_ERR_INVALID, "owner is NULL");
    std::vector<int> set(interest_set ? interest_set : nullptr, interest_set ? interest_set + std::max(l, 0) : nullptr);
    std::vector<int> own;
    CQSA_TRY(quorum_owner(c, interest_set ? set.data() : nullptr, l, &own));
    for (size_t i = 0; i < own.size(); ++i) owner[i] = own[i];
    return CQSA_OK;
}

cqsa_status cqsa_cqs_assign_itr(int32_t c, const int32_t* interest_set, int32_t l, int32_t itr, int32_t* owner) {
    g_err.clear();
    if (!owner) return fail(CQSA_ERR_INVALID, "owner is NULL");
    if (itr < 1) return fail(CQSA_ERR_INVALID, "cqs: itr = %d is below 1", itr);
    std::vector<int> set(interest_set ? interest_set : nullptr, interest_set ? interest_set + std::max(l, 0) : nullptr);
    std::vector<int> own;
    CQSA_TRY(quorum_owner_itr(c, interest_set ? set.data() : nullptr, l, itr, &own));
    for (size_t i = 0; i < own.size(); ++i) owner[i] = own[i];
    return CQSA_OK;
}

int32_t cqsa_cqs_default_set(int32_t c, int32_t* set, int32_t max_l) {
    int tmp[8];
    const int l = default_quorum_set(c, tmp, 8);
    if (set)
        for (int i = 0; i < l && i < max_l; ++i) set[i] = tmp[i];
    return l;
}

const char* cqsa_fwd_kernel_name(int64_t head_dim, int32_t precision) {
    return (head_dim == 64 || head_dim == 128) ? fwd_kernel_name((int)head_dim, precision == 1 ? 1 : 0) : "";
}

cqsa_status cqsa_plan(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v, int is_causal,
                      uint64_t mem_budget, const cqsa_tensor* out, int want_lse, const cqsa_options* opt,
                      cqsa_plan_info* info) {
    g_err.clear();
    cqsa_options o;
    std::memset(&o, 0, sizeof o);
    if (opt) o = *opt;
    // detect locations only for tensors whose `where` is DETECT
    Problem P;
    const bool detect = (q && q->where == CQSA_WHERE_DETECT) || (k && k->where == CQSA_WHERE_DETECT) ||
                        (v && v->where == CQSA_WHERE_DETECT) || (out && out->where == CQSA_WHERE_DETECT);
    CQSA_TRY(check_lse_where(want_lse));
    CQSA_TRY(build_problem(q, k, v, is_causal, 0.f, out, nullptr, want_lse, detect, true, &P));
    CQSA_TRY(set_precision(o, &P));
    P.lse_host = lse_on_host(want_lse, P.out.host);
    P.streamed = P.q.host || P.k.host || P.v.host || P.out.host || (P.want_lse && P.lse_host);
    uint64_t budget = 0;
    CQSA_TRY(resolve_budget(mem_budget, &budget));
    int cus = o.num_cus;
    if (cus <= 0) {
        DeviceRes* r = nullptr;
        CQSA_TRY(device_res(&r));
        cus = r->num_cus;
    }
    Plan pl;
    CQSA_TRY(make_plan(P, budget, o, cus, &pl));
    if (info) *info = pl.info;
    return CQSA_OK;
}

cqsa_status cqsa_schedule_trace(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v, int is_causal,
                                uint64_t mem_budget, const cqsa_tensor* out, int want_lse, const cqsa_options* opt,
                                char* buf, uint64_t buf_len, uint64_t* needed) {
    g_err.clear();
    if (!q || !k || !v || !out) return fail(CQSA_ERR_INVALID, "schedule trace: q, k, v and out are required");
    for (const cqsa_tensor* t : {q, k, v, out})
        if (t->where != CQSA_WHERE_HOST && t->where != CQSA_WHERE_DEVICE)
            return fail(CQSA_ERR_INVALID, "schedule trace: every tensor needs where = HOST or DEVICE");
    if (mem_budget == 0) return fail(CQSA_ERR_INVALID, "schedule trace: mem_budget must be given");
    cqsa_options o;
    std::memset(&o, 0, sizeof o);
    if (opt) o = *opt;
    Problem P;
    CQSA_TRY(check_lse_where(want_lse));
    CQSA_TRY(build_problem(q, k, v, is_causal, 0.f, out, nullptr, want_lse, false, true, &P));
    CQSA_TRY(set_precision(o, &P));
    P.lse_host = lse_on_host(want_lse, P.out.host);
    P.streamed = P.q.host || P.k.host || P.v.host || P.out.host || (P.want_lse && P.lse_host);
    Recorder rec;
    if (P.want_lse) {   // the lse array: a distinct stand-in range 2^40 bytes past out
        P.lse = reinterpret_cast<float*>(out->data ? static_cast<char*>(out->data) + ((uint64_t)1 << 40) : nullptr);
    }
    if (!P.empty) {
        uint64_t budget = 0;
        CQSA_TRY(resolve_budget(mem_budget, &budget));
        Plan pl;
        CQSA_TRY(make_plan(P, budget, o, o.num_cus > 0 ? o.num_cus : 256, &pl));
        // stand-ins that no HIP call sees: the workspace base and the three streams
        char* ws = static_cast<char*>(o.workspace ? o.workspace : reinterpret_cast<void*>((uintptr_t)1 << 46));
        hipStream_t st = o.stream ? static_cast<hipStream_t>(o.stream) : reinterpret_cast<hipStream_t>((uintptr_t)0x10);
        DeviceRes res;
        res.init = true;
        res.num_cus = 256;
        res.h2d = reinterpret_cast<hipStream_t>((uintptr_t)0x20);
        res.d2h = reinterpret_cast<hipStream_t>((uintptr_t)0x30);
        rec.id(rec.streams, st);
        rec.line("workspace " + rng('W', ws, ws + pl.total));
        g_rec = &rec;
        cqsa_status s;
        if (pl.cqs)
            s = exec_cqs(P, pl, ws, st, &res, &pl.info);
        else if (!pl.chunked)
            s = exec_single(P, pl, ws, st);
        else
            s = exec_chunked(P, pl, ws, st, &res, &pl.info);
        g_rec = nullptr;
        CQSA_TRY(s);
        if (P.streamed) rec.line("sync " + rec.st(st));
    }
    if (needed) *needed = rec.text.size() + 1;
    if (buf && buf_len > 0) {
        const size_t n = std::min<size_t>(rec.text.size(), buf_len - 1);
        std::memcpy(buf, rec.text.data(), n);
        buf[n] = 0;
        if (n < rec.text.size()) return fail(CQSA_ERR_INVALID, "schedule trace: buffer of %llu bytes is too small",
                                             (unsigned long long)buf_len);
    }
    return CQSA_OK;
}

cqsa_status cqsa_attention_ex(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v, int is_causal,
                              float scale, uint64_t mem_budget, cqsa_tensor* out, float* lse,
                              const cqsa_options* opt, cqsa_plan_info* info) {
    g_err.clear();
    g_fwd_launches = 0;
    const auto t0 = std::chrono::steady_clock::now();
    cqsa_options o;
    std::memset(&o, 0, sizeof o);
    if (opt) o = *opt;
    Problem P;
    CQSA_TRY(build_problem(q, k, v, is_causal, scale, out, lse, lse != nullptr, true, false, &P));
    CQSA_TRY(set_precision(o, &P));
    if (P.empty) {
        if (info) std::memset(info, 0, sizeof *info);
        return CQSA_OK;
    }
    DeviceRes* res = nullptr;
    CQSA_TRY(device_res(&res));
    uint64_t budget = 0;
    CQSA_TRY(resolve_budget(mem_budget, &budget));
    Plan pl;
    CQSA_TRY(make_plan(P, budget, o, res->num_cus, &pl));
    hipStream_t st = static_cast<hipStream_t>(o.stream);

    char* ws = nullptr;
    bool owned = false;
    if (pl.total > 0) {
        if (o.workspace && o.workspace_bytes >= pl.total) {
            ws = static_cast<char*>(o.workspace);
        } else {
            hipError_t e = hipMalloc(reinterpret_cast<void**>(&ws), pl.total);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                return fail(CQSA_ERR_OOM, "hipMalloc of %llu workspace bytes failed: %s",
                            (unsigned long long)pl.total, hipGetErrorString(e));
            }
            owned = true;
        }
    }
    cqsa_status s;
    if (pl.cqs)
        s = exec_cqs(P, pl, ws, st, res, &pl.info);
    else if (!pl.chunked)
        s = exec_single(P, pl, ws, st);
    else
        s = exec_chunked(P, pl, ws, st, res, &pl.info);
    const bool sync = owned || P.streamed;
    if (sync && s == CQSA_OK) {
        hipError_t e = hipStreamSynchronize(st);
        if (e != hipSuccess) s = fail(CQSA_ERR_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
    }
    if (s != CQSA_OK) drain_after_failure(st, res);
    if (owned) (void)hipFree(ws);
    if (s != CQSA_OK) return s;
    if (sync) pl.info.wall_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    if (info) *info = pl.info;
    if (log_enabled()) {
        std::fprintf(stderr,
                     "cqsa: B=%lld Hq=%lld Hkv=%lld Nq=%lld Nk=%lld D=%lld causal=%d | %s q_chunk=%lld kv_chunk=%lld "
                     "splits=%d merge=%d pairs=%lld launches=%lld ws=%llu h2d=%llu d2h=%llu\n",
                     (long long)P.B, (long long)P.Hq, (long long)P.Hkv, (long long)P.Nq, (long long)P.Nk,
                     (long long)P.D, (int)P.causal, P.streamed ? "streamed" : "resident",
                     (long long)pl.info.q_chunk, (long long)pl.info.kv_chunk, pl.info.kv_splits,
                     pl.info.merge_mode, (long long)pl.info.chunk_pairs, (long long)pl.info.kernel_launches,
                     (unsigned long long)pl.info.workspace_bytes, (unsigned long long)pl.info.h2d_bytes,
                     (unsigned long long)pl.info.d2h_bytes);
    }
    return CQSA_OK;
}

cqsa_status cqsa_attention(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v, int is_causal,
                           float scale, uint64_t mem_budget, cqsa_tensor* out, float* lse) {
    return cqsa_attention_ex(q, k, v, is_causal, scale, mem_budget, out, lse, nullptr, nullptr);
}

cqsa_status cqsa_attention_noalloc(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v, int is_causal,
                                   float scale, cqsa_tensor* out, float* lse, int32_t kv_splits, void* stream,
                                   cqsa_plan_info* info) {
    static_assert(kNoAllocScratchBytes == CQSA_NOALLOC_SCRATCH_BYTES, "one size on both sides of the ABI");
    g_err.clear();
    g_fwd_launches = 0;
    if (kv_splits < 0) return fail(CQSA_ERR_INVALID, "kv_splits %d is negative", kv_splits);
    Problem P;
    CQSA_TRY(build_problem(q, k, v, is_causal, scale, out, lse, lse != nullptr, true, false, &P));
    if (P.streamed)
        return fail(CQSA_ERR_UNSUPPORTED, "cqsa_attention_noalloc takes device memory only (host operands need "
                                          "staging): use cqsa_attention_ex");
    if (P.empty) {
        if (info) std::memset(info, 0, sizeof *info);
        return CQSA_OK;
    }
    P.one_pass = true;
    // a forced split: its partial triples must fit the fixed array as asked, not halved to fit
    const uint64_t rows = (uint64_t)P.B * P.Hq * P.Nq;
    if (kv_splits > 1) {
        const int64_t s = std::min<int64_t>({kv_splits, kMaxMergeParts, ceil_div(P.Nk, 64)});
        const uint64_t need = (uint64_t)s * rows * (P.D + 2) * 4 + 512;
        if (need > kNoAllocScratchBytes)
            return fail(CQSA_ERR_BUDGET, "kv_splits=%d needs %llu bytes of partials; the no-allocation entry point "
                        "holds %llu bytes (CQSA_NOALLOC_SCRATCH_BYTES)", kv_splits, (unsigned long long)need,
                        (unsigned long long)kNoAllocScratchBytes);
    }
    DeviceRes* res = nullptr;
    CQSA_TRY(device_res(&res));
    cqsa_options o;
    std::memset(&o, 0, sizeof o);
    o.kv_splits = kv_splits;
    o.stream = stream;
    Plan pl;
    CQSA_TRY(make_plan(P, kNoAllocScratchBytes, o, res->num_cus, &pl));
    if (pl.cqs || pl.chunked || pl.total > kNoAllocScratchBytes)
        return fail(CQSA_ERR_BUDGET, "the plan needs %llu bytes; the no-allocation entry point holds %llu",
                    (unsigned long long)pl.total, (unsigned long long)kNoAllocScratchBytes);
    char* ws = nullptr;
    if (pl.total > 0) {
        void* p = nullptr;
        const hipError_t e = noalloc_scratch(&p);
        if (e != hipSuccess)
            return fail(CQSA_ERR_HIP, "address of the no-allocation scratch array: %s", hipGetErrorString(e));
        ws = static_cast<char*>(p);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const cqsa_status s = exec_single(P, pl, ws, st);
    if (s != CQSA_OK) {
        drain_after_failure(st, res);
        return s;
    }
    if (info) *info = pl.info;
    return CQSA_OK;
}

// The backward's operands, validated: q, k, v, out (Problem), dout, the gradients and lse.
struct BwdProblem {
    Problem P;
    View dout, dq, dk, dv;
    const float* lse = nullptr;
    bool lse_host = false;
};

// detect: find each operand's placement with HIP; otherwise take it from `where` (lse_where for lse).
cqsa_status bwd_problem(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v, const cqsa_tensor* out,
                        const cqsa_tensor* dout, const float* lse, int is_causal, float scale, cqsa_tensor* dq,
                        cqsa_tensor* dk, cqsa_tensor* dv, BwdProblem* bp, bool detect = true,
                        int lse_where = CQSA_WHERE_DETECT) {
    Problem& P = bp->P;
    CQSA_TRY(build_problem(q, k, v, is_causal, scale, out, nullptr, 0, detect, false, &P));
    View &vdo = bp->dout, &vdq = bp->dq, &vdk = bp->dk, &vdv = bp->dv;
    CQSA_TRY(make_view(dout, "dout", false, detect, &vdo));
    CQSA_TRY(make_view(dq, "dq", false, detect, &vdq));
    CQSA_TRY(make_view(dk, "dk", false, detect, &vdk));
    CQSA_TRY(make_view(dv, "dv", false, detect, &vdv));
    if (vdo.dtype != P.dtype) return fail(CQSA_ERR_INVALID, "dout must have q's dtype");
    if (vdo.B != P.B || vdo.H != P.Hq || vdo.N != P.Nq || vdo.D != P.D) return fail(CQSA_ERR_INVALID, "dout must have q's shape");
    if (vdq.B != P.B || vdq.H != P.Hq || vdq.N != P.Nq || vdq.D != P.D) return fail(CQSA_ERR_INVALID, "dq must have q's shape");
    for (const View* g : {&vdk, &vdv})
        if (g->B != P.B || g->H != P.Hkv || g->N != P.Nk || g->D != P.D)
            return fail(CQSA_ERR_INVALID, "dk and dv must have k's shape");
    if (vdk.dtype != vdq.dtype || vdv.dtype != vdq.dtype) return fail(CQSA_ERR_INVALID, "dq, dk, dv must share one dtype");
    if (P.empty || P.Nk == 0) return CQSA_OK;
    if (!lse) return fail(CQSA_ERR_INVALID, "lse is NULL");
    bp->lse = lse;
    if (!detect) {
        bp->lse_host = lse_where == CQSA_WHERE_HOST;
    } else {
        cqsa_tensor lt;
        std::memset(&lt, 0, sizeof lt);
        lt.data = const_cast<float*>(lse);
        lt.dtype = CQSA_F32;
        lt.shape[0] = 1; lt.shape[1] = 1; lt.shape[2] = 1; lt.shape[3] = 1;
        lt.stride[3] = 1;
        CQSA_TRY(locate(&lt, "lse", false, &bp->lse_host));
    }
    if (!aligned16(vdo.data) || vdo.sn % 8 || vdo.sh % 8 || vdo.sb % 8)
        return fail(CQSA_ERR_UNSUPPORTED, "dout data and strides must be 16-byte aligned");
    for (const View* g : {&vdq, &vdk, &vdv})
        if ((reinterpret_cast<uintptr_t>(g->data) % (4 * g->es)) || g->sn % 4 || g->sh % 4 || g->sb % 4)
            return fail(CQSA_ERR_UNSUPPORTED, "gradient data and strides must be aligned to 4 elements");
    if (P.out.dtype == CQSA_F32 ? (!aligned16(P.out.data) || P.out.sn % 4 || P.out.sh % 4 || P.out.sb % 4)
                                : (!aligned16(P.out.data) || P.out.sn % 8 || P.out.sh % 8 || P.out.sb % 8))
        return fail(CQSA_ERR_UNSUPPORTED, "out data and strides must be 16-byte aligned for the backward");
    return CQSA_OK;
}

// Arguments common to every backward launch of a problem (pointers and extents are set per launch).
BwdArgs bwd_base(const BwdProblem& bp) {
    const Problem& P = bp.P;
    BwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.B = (int32_t)P.B;
    a.Hq = (int32_t)P.Hq;
    a.Hkv = (int32_t)P.Hkv;
    a.group = (int32_t)(P.Hq / P.Hkv);
    a.causal = P.causal ? 1 : 0;
    a.out_dtype = elem_type(P.out.dtype);
    a.grad_dtype = elem_type(bp.dq.dtype);
    a.scale = P.scale;
    a.scale_log2 = P.scale * 1.44269504088896340736f;
    return a;
}

cqsa_status run_bwd_pass(const Problem& P, const BwdArgs& a, int pass, hipStream_t st) {
    if (g_rec) {
        const int64_t D = P.D, oes = a.out_dtype == ET_F32 ? 4 : 2, ges = a.grad_dtype == ET_F32 ? 4 : 2;
        std::string l = "kernel " + g_rec->st(st) + (pass == BWD_STATS ? " bwd_stats" : pass == BWD_DQ ? " bwd_dq" : " bwd_dkdv");
        const std::string stats_rows =
            view_hull('X', a.stats, 4, 1, a.B * a.Hq, 0, a.stats_rows * 2, 2, 0, a.Nq, 2).substr(1);
        if (pass == BWD_STATS) {
            l += " " + view_hull('R', a.out, oes, a.B, a.Hq, a.o_sb, a.o_sh, a.o_sn, 0, a.Nq, D);
            l += " " + view_hull('R', a.dout, 2, a.B, a.Hq, a.do_sb, a.do_sh, a.do_sn, 0, a.Nq, D);
            l += " " + view_hull('R', a.lse, 4, a.B, a.Hq, a.l_sb, a.l_sh, 1, 0, a.Nq, 1);
            l += " W" + stats_rows;
        } else {
            l += " " + view_hull('R', a.q, 2, a.B, a.Hq, a.q_sb, a.q_sh, a.q_sn, 0, a.Nq, D);
            l += " " + view_hull('R', a.dout, 2, a.B, a.Hq, a.do_sb, a.do_sh, a.do_sn, 0, a.Nq, D);
            l += " " + view_hull('R', a.k, 2, a.B, a.Hkv, a.k_sb, a.k_sh, a.k_sn, 0, a.Nk, D);
            l += " " + view_hull('R', a.v, 2, a.B, a.Hkv, a.v_sb, a.v_sh, a.v_sn, 0, a.Nk, D);
            l += " R" + stats_rows;
            auto grad = [&](const void* g, int64_t H, int64_t sb, int64_t sh, int64_t sn, int64_t n) {
                const std::string w = view_hull('W', g, ges, a.B, H, sb, sh, sn, 0, n, D);
                return a.accumulate ? w + " R" + w.substr(1) : w;
            };
            if (pass == BWD_DQ) l += " " + grad(a.dq, a.Hq, a.dq_sb, a.dq_sh, a.dq_sn, a.Nq);
            else l += " " + grad(a.dk, a.Hkv, a.dk_sb, a.dk_sh, a.dk_sn, a.Nk) + " " + grad(a.dv, a.Hkv, a.dv_sb, a.dv_sh, a.dv_sn, a.Nk);
        }
        g_rec->line(l);
        return CQSA_OK;
    }
    const hipError_t e = launch_bwd_pass(a, (int)P.D, P.dtype == CQSA_F16 ? ET_F16 : ET_BF16, pass, st);
    if (e != hipSuccess) return fail(CQSA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
    return CQSA_OK;
}

cqsa_status run_cast(const float* src, int64_t B, int64_t H, int64_t n, int64_t D, void* dst, int dtype, int64_t sb,
                     int64_t sh, int64_t sn, hipStream_t st) {
    if (g_rec) {
        const int64_t es = dtype == ET_F32 ? 4 : 2;
        g_rec->line("kernel " + g_rec->st(st) + " cast " + view_hull('R', src, 4, B, H, H * n * D, n * D, D, 0, n, D) + " " +
                    view_hull('W', dst, es, B, H, sb, sh, sn, 0, n, D));
        return CQSA_OK;
    }
    const hipError_t e = launch_cast(src, B, H, n, D, dst, dtype, sb, sh, sn, st);
    if (e != hipSuccess) return fail(CQSA_ERR_HIP, "cast launch failed: %s", hipGetErrorString(e));
    return CQSA_OK;
}

// lse rows [ra, ra + rn) of a [B, Hq, Nq] fp32 host array -> compact device [B, Hq, rn]
cqsa_status copy_lse_rows_in(float* dev, const float* host, int64_t B, int64_t Hq, int64_t Nq, int64_t ra, int64_t rn,
                             hipStream_t st) {
    if (rn <= 0) return CQSA_OK;
    CQSA_HIP(x_copy2d(dev, (size_t)rn * 4, host + ra, (size_t)Nq * 4, (size_t)rn * 4, (size_t)(B * Hq),
                      hipMemcpyHostToDevice, st));
    return CQSA_OK;
}

// The chunked backward plan: query chunks of qc rows, key chunks of kc keys, and the workspace layout.
struct BwdPlan {
    int64_t qc = 0, kc = 0;
    uint64_t off_stats = 0, off_dq = 0, off_dk = 0, off_dv = 0;
    uint64_t off_q[2] = {0, 0}, off_do[2] = {0, 0}, off_lse[2] = {0, 0}, off_o = 0;
    uint64_t off_k[2] = {0, 0}, off_v[2] = {0, 0};
    uint64_t off_gq = 0, off_gk = 0, off_gv = 0;   // gradient staging for host gradients
    uint64_t total = 0;
};

uint64_t bwd_layout(const BwdProblem& bp, int64_t qc, int64_t kc, BwdPlan* pl) {
    const Problem& P = bp.P;
    uint64_t off = 0;
    auto take = [&](uint64_t bytes) {
        const uint64_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    const uint64_t qrow = (uint64_t)P.B * P.Hq * P.D, krow = (uint64_t)P.B * P.Hkv * P.D;
    const uint64_t ges = (uint64_t)bp.dq.es;
    pl->qc = qc;
    pl->kc = kc;
    pl->off_stats = take((uint64_t)P.B * P.Hq * P.Nq * 8);
    pl->off_dq = take(qrow * P.Nq * 4);
    pl->off_dk = take(krow * kc * 4);
    pl->off_dv = take(krow * kc * 4);
    for (int i = 0; i < 2; ++i) {
        pl->off_q[i] = P.q.host ? take(qrow * qc * 2) : 0;
        pl->off_do[i] = bp.dout.host ? take(qrow * qc * 2) : 0;
        pl->off_lse[i] = bp.lse_host ? take((uint64_t)P.B * P.Hq * qc * 4) : 0;
        pl->off_k[i] = P.k.host ? take(krow * kc * 2) : 0;
        pl->off_v[i] = P.v.host ? take(krow * kc * 2) : 0;
    }
    pl->off_o = P.out.host ? take(qrow * qc * P.out.es) : 0;
    pl->off_gq = bp.dq.host ? take(qrow * qc * ges) : 0;
    pl->off_gk = bp.dk.host ? take(krow * kc * ges) : 0;
    pl->off_gv = bp.dv.host ? take(krow * kc * ges) : 0;
    pl->total = off;
    return off;
}

cqsa_status bwd_plan(const BwdProblem& bp, uint64_t budget, const cqsa_options& o, BwdPlan* pl) {
    const Problem& P = bp.P;
    int64_t qc = o.q_chunk > 0 ? std::min(o.q_chunk, P.Nq) : std::min<int64_t>(P.Nq, kKvCap);
    int64_t kc = o.kv_chunk > 0 ? std::min(o.kv_chunk, P.Nk) : std::min<int64_t>(P.Nk, kKvCap);
    for (;;) {
        if (bwd_layout(bp, qc, kc, pl) <= budget) return CQSA_OK;
        const bool can_q = o.q_chunk <= 0 && qc > kRowGrain, can_k = o.kv_chunk <= 0 && kc > kRowGrain;
        if (!can_q && !can_k) break;
        if (can_k && (kc >= qc || !can_q)) kc = std::max<int64_t>(kRowGrain, (kc / 2 + kRowGrain - 1) / kRowGrain * kRowGrain);
        else qc = std::max<int64_t>(kRowGrain, (qc / 2 + kRowGrain - 1) / kRowGrain * kRowGrain);
    }
    return fail(CQSA_ERR_BUDGET,
                "mem_budget too small for the chunked backward: needs %llu bytes at %lld-row query chunks and "
                "%lld-key chunks (the fp32 dq accumulator alone is %llu bytes)",
                (unsigned long long)pl->total, (long long)qc, (long long)kc,
                (unsigned long long)((uint64_t)P.B * P.Hq * P.Nq * P.D * 4));
}

// Key chunks outermost.  Pass 1: the row statistics of every query chunk (out, dout and lse staged when
// on the host).  Pass 2: for each key chunk (K, V staged), every query chunk that sees it (Q, dout
// staged): dQ accumulates in an fp32 array for all query rows, dK and dV in fp32 arrays for the key
// chunk, which are rounded into the caller's gradients (through staging and a D2H copy when those live
// on the host) when the chunk is done.  dQ is rounded last.  Staging alternates between two buffers
// per operand, ordered by events like the forward's chunked schedule.
cqsa_status exec_bwd_chunked(const BwdProblem& bp, const BwdPlan& pl, char* ws, hipStream_t st, DeviceRes* res,
                             cqsa_plan_info* info) {
    const Problem& P = bp.P;
    const bool any_in = P.q.host || P.k.host || P.v.host || P.out.host || bp.dout.host || bp.lse_host;
    const bool any_out = bp.dq.host || bp.dk.host || bp.dv.host;
    hipStream_t h2d = st, d2h = st;
    if (any_in || any_out) {
        CQSA_TRY(side_streams(res));
        h2d = res->h2d;
        d2h = res->d2h;
    }
    EventSet es;
    hipEvent_t ev_start, ev_qcopy[2], ev_qcomp[2], ev_kvcopy[2], ev_kvcomp[2], ev_ocopy, ev_ocomp, ev_cast, ev_d2h;
    CQSA_TRY(es.make(&ev_start, false));
    CQSA_TRY(es.make(&ev_ocopy, false));
    CQSA_TRY(es.make(&ev_ocomp, false));
    CQSA_TRY(es.make(&ev_cast, false));
    CQSA_TRY(es.make(&ev_d2h, false));
    for (int i = 0; i < 2; ++i) {
        CQSA_TRY(es.make(&ev_qcopy[i], false));
        CQSA_TRY(es.make(&ev_qcomp[i], false));
        CQSA_TRY(es.make(&ev_kvcopy[i], false));
        CQSA_TRY(es.make(&ev_kvcomp[i], false));
    }
    bool qcomp_rec[2] = {false, false}, kvcomp_rec[2] = {false, false}, ocomp_rec = false, d2h_rec = false;
    std::vector<TimedCopy> h2d_t, d2h_t;
    auto timed = [&](std::vector<TimedCopy>& v, TimedCopy* tc) -> cqsa_status {
        CQSA_TRY(es.make(&tc->start, true));
        CQSA_TRY(es.make(&tc->stop, true));
        v.push_back(*tc);
        return CQSA_OK;
    };
    CQSA_HIP(x_record(ev_start, st));
    if (any_in || any_out) {
        CQSA_HIP(x_wait(h2d, ev_start));
        CQSA_HIP(x_wait(d2h, ev_start));
    }
    const int64_t D = P.D, Nq = P.Nq, Nk = P.Nk, qc = pl.qc, kc = pl.kc;
    const int64_t n_q = ceil_div(Nq, qc), n_k = ceil_div(Nk, kc);
    float* stats = reinterpret_cast<float*>(ws + pl.off_stats);
    float* dq_acc = reinterpret_cast<float*>(ws + pl.off_dq);
    float* dk_acc = reinterpret_cast<float*>(ws + pl.off_dk);
    float* dv_acc = reinterpret_cast<float*>(ws + pl.off_dv);
    const BwdArgs base = bwd_base(bp);
    int64_t pairs = 0, launches = 0;
    int qturn = 0;   // alternates the query-side staging buffers across both passes

    // stage (or point at) rows [qa, qa + qn) of a query-side operand
    auto qside = [&](const View& t, int64_t qa, int64_t qn, uint64_t off, bool host, const char** p, int64_t* sb,
                     int64_t* sh, int64_t* sn) -> cqsa_status {
        if (host) {
            CQSA_TRY(copy_rows(t, qa, qn, ws + off, true, h2d));
            const Compact c = compact_for(t, qn);
            *p = ws + off;
            *sb = c.sb;
            *sh = c.sh;
            *sn = c.sn;
        } else {
            *p = t.data + (size_t)(qa * t.sn) * t.es;
            *sb = t.sb;
            *sh = t.sh;
            *sn = t.sn;
        }
        return CQSA_OK;
    };

    // pass 1: row statistics
    for (int64_t r = 0; r < n_q; ++r) {
        const int64_t qa = r * qc, qn = std::min(qc, Nq - qa);
        const int qb = qturn++ & 1;
        BwdArgs a = base;
        const char *po = nullptr, *pd = nullptr;
        if (P.out.host || bp.dout.host || bp.lse_host) {
            if (qcomp_rec[qb]) CQSA_HIP(x_wait(h2d, ev_qcomp[qb]));
            if (P.out.host && ocomp_rec) CQSA_HIP(x_wait(h2d, ev_ocomp));
            TimedCopy tc;
            CQSA_TRY(timed(h2d_t, &tc));
            CQSA_HIP(x_record(tc.start, h2d));
        }
        CQSA_TRY(qside(P.out, qa, qn, pl.off_o, P.out.host, &po, &a.o_sb, &a.o_sh, &a.o_sn));
        CQSA_TRY(qside(bp.dout, qa, qn, pl.off_do[qb], bp.dout.host, &pd, &a.do_sb, &a.do_sh, &a.do_sn));
        if (bp.lse_host) {
            float* dl = reinterpret_cast<float*>(ws + pl.off_lse[qb]);
            CQSA_TRY(copy_lse_rows_in(dl, bp.lse, P.B, P.Hq, Nq, qa, qn, h2d));
            a.lse = dl;
            a.l_sb = P.Hq * qn;
            a.l_sh = qn;
        } else {
            a.lse = bp.lse + qa;
            a.l_sb = P.Hq * Nq;
            a.l_sh = Nq;
        }
        if (P.out.host || bp.dout.host || bp.lse_host) {
            CQSA_HIP(x_record(h2d_t.back().stop, h2d));
            CQSA_HIP(x_record(ev_qcopy[qb], h2d));
            CQSA_HIP(x_wait(st, ev_qcopy[qb]));
        }
        a.out = po;
        a.dout = reinterpret_cast<const uint16_t*>(pd);
        a.stats = stats + 2 * qa;
        a.stats_rows = Nq;
        a.Nq = qn;
        a.Nk = Nk;
        CQSA_TRY(run_bwd_pass(P, a, BWD_STATS, st));
        ++launches;
        CQSA_HIP(x_record(ev_qcomp[qb], st));
        qcomp_rec[qb] = true;
        if (P.out.host) {
            CQSA_HIP(x_record(ev_ocomp, st));
            ocomp_rec = true;
        }
    }

    // pass 2: key chunks outermost
    for (int64_t c = 0; c < n_k; ++c) {
        const int64_t ka = c * kc, kn = std::min(kc, Nk - ka);
        const int kb = (int)(c & 1);
        const char *pk = nullptr, *pv = nullptr;
        int64_t k_sb, k_sh, k_sn, v_sb, v_sh, v_sn;
        if (P.k.host || P.v.host) {
            if (kvcomp_rec[kb]) CQSA_HIP(x_wait(h2d, ev_kvcomp[kb]));
            TimedCopy tc;
            CQSA_TRY(timed(h2d_t, &tc));
            CQSA_HIP(x_record(tc.start, h2d));
        }
        CQSA_TRY(qside(P.k, ka, kn, pl.off_k[kb], P.k.host, &pk, &k_sb, &k_sh, &k_sn));
        CQSA_TRY(qside(P.v, ka, kn, pl.off_v[kb], P.v.host, &pv, &v_sb, &v_sh, &v_sn));
        if (P.k.host || P.v.host) {
            CQSA_HIP(x_record(h2d_t.back().stop, h2d));
            CQSA_HIP(x_record(ev_kvcopy[kb], h2d));
            CQSA_HIP(x_wait(st, ev_kvcopy[kb]));
        }
        bool first = true;
        for (int64_t r = 0; r < n_q; ++r) {
            const int64_t qa = r * qc, qn = std::min(qc, Nq - qa);
            if (P.causal && ka > qa + qn - 1 + (Nk - Nq)) continue;   // no row of the chunk sees these keys
            const int qb = qturn++ & 1;
            BwdArgs a = base;
            const char *pq = nullptr, *pd = nullptr;
            if (P.q.host || bp.dout.host) {
                if (qcomp_rec[qb]) CQSA_HIP(x_wait(h2d, ev_qcomp[qb]));
                TimedCopy tc;
                CQSA_TRY(timed(h2d_t, &tc));
                CQSA_HIP(x_record(tc.start, h2d));
            }
            CQSA_TRY(qside(P.q, qa, qn, pl.off_q[qb], P.q.host, &pq, &a.q_sb, &a.q_sh, &a.q_sn));
            CQSA_TRY(qside(bp.dout, qa, qn, pl.off_do[qb], bp.dout.host, &pd, &a.do_sb, &a.do_sh, &a.do_sn));
            if (P.q.host || bp.dout.host) {
                CQSA_HIP(x_record(h2d_t.back().stop, h2d));
                CQSA_HIP(x_record(ev_qcopy[qb], h2d));
                CQSA_HIP(x_wait(st, ev_qcopy[qb]));
            }
            a.q = reinterpret_cast<const uint16_t*>(pq);
            a.dout = reinterpret_cast<const uint16_t*>(pd);
            a.k = reinterpret_cast<const uint16_t*>(pk);
            a.v = reinterpret_cast<const uint16_t*>(pv);
            a.k_sb = k_sb; a.k_sh = k_sh; a.k_sn = k_sn;
            a.v_sb = v_sb; a.v_sh = v_sh; a.v_sn = v_sn;
            a.stats = stats + 2 * qa;
            a.stats_rows = Nq;
            a.Nq = qn;
            a.Nk = kn;
            a.causal_delta = qa - ka + (Nk - Nq);
            a.grad_dtype = ET_F32;
            // dQ rows of the chunk in the all-rows accumulator; key chunk 0 is seen by every row, so it
            // starts each row's sum
            a.dq = dq_acc + qa * D;
            a.dq_sb = P.Hq * Nq * D; a.dq_sh = Nq * D; a.dq_sn = D;
            a.accumulate = c > 0 ? 1 : 0;
            CQSA_TRY(run_bwd_pass(P, a, BWD_DQ, st));
            a.dk = dk_acc;
            a.dv = dv_acc;
            a.dk_sb = a.dv_sb = P.Hkv * kn * D; a.dk_sh = a.dv_sh = kn * D; a.dk_sn = a.dv_sn = D;
            a.accumulate = first ? 0 : 1;
            CQSA_TRY(run_bwd_pass(P, a, BWD_DKDV, st));
            launches += P.D == 128 ? 3 : 2;   // the dK/dV pass is two launches at D = 128
            ++pairs;
            first = false;
            CQSA_HIP(x_record(ev_qcomp[qb], st));
            qcomp_rec[qb] = true;
        }
        CQSA_HIP(x_record(ev_kvcomp[kb], st));
        kvcomp_rec[kb] = true;
        // deliver dK and dV of the chunk
        const int gdt = elem_type(bp.dq.dtype);
        for (int g = 0; g < 2; ++g) {
            const View& t = g == 0 ? bp.dk : bp.dv;
            const float* acc = g == 0 ? dk_acc : dv_acc;
            if (!t.host) {
                CQSA_TRY(run_cast(acc, P.B, P.Hkv, kn, D, t.data + (size_t)(ka * t.sn) * t.es, gdt, t.sb, t.sh, t.sn, st));
            } else {
                if (d2h_rec) CQSA_HIP(x_wait(st, ev_d2h));
                char* stg = ws + (g == 0 ? pl.off_gk : pl.off_gv);
                const Compact cc = compact_for(t, kn);
                CQSA_TRY(run_cast(acc, P.B, P.Hkv, kn, D, stg, gdt, cc.sb, cc.sh, cc.sn, st));
                CQSA_HIP(x_record(ev_cast, st));
                CQSA_HIP(x_wait(d2h, ev_cast));
                TimedCopy tc;
                CQSA_TRY(timed(d2h_t, &tc));
                CQSA_HIP(x_record(tc.start, d2h));
                CQSA_TRY(copy_rows(t, ka, kn, stg, false, d2h));
                CQSA_HIP(x_record(tc.stop, d2h));
                CQSA_HIP(x_record(ev_d2h, d2h));
                d2h_rec = true;
            }
            ++launches;
        }
    }
    // deliver dQ
    {
        const View& t = bp.dq;
        const int gdt = elem_type(t.dtype);
        if (!t.host) {
            CQSA_TRY(run_cast(dq_acc, P.B, P.Hq, Nq, D, t.data, gdt, t.sb, t.sh, t.sn, st));
            ++launches;
        } else {
            for (int64_t r = 0; r < n_q; ++r) {
                const int64_t qa = r * qc, qn = std::min(qc, Nq - qa);
                if (d2h_rec) CQSA_HIP(x_wait(st, ev_d2h));
                const Compact cc = compact_for(t, qn);
                // rows [qa, qa + qn) of every head: a [B Hq][qn] slice of the accumulator with head
                // stride Nq D, rounded into the compact staging
                for (int64_t bh = 0; bh < P.B * P.Hq; ++bh) {
                    const int64_t b = bh / P.Hq, h = bh % P.Hq;
                    CQSA_TRY(run_cast(dq_acc + (bh * Nq + qa) * D, 1, 1, qn, D,
                                      ws + pl.off_gq + (size_t)(b * cc.sb + h * cc.sh) * t.es, gdt, 0, 0, cc.sn, st));
                    ++launches;
                }
                CQSA_HIP(x_record(ev_cast, st));
                CQSA_HIP(x_wait(d2h, ev_cast));
                TimedCopy tc;
                CQSA_TRY(timed(d2h_t, &tc));
                CQSA_HIP(x_record(tc.start, d2h));
                CQSA_TRY(copy_rows(t, qa, qn, ws + pl.off_gq, false, d2h));
                CQSA_HIP(x_record(tc.stop, d2h));
                CQSA_HIP(x_record(ev_d2h, d2h));
                d2h_rec = true;
            }
        }
    }
    if (any_in || any_out) {
        hipEvent_t j1, j2;
        CQSA_TRY(es.make(&j1, false));
        CQSA_TRY(es.make(&j2, false));
        CQSA_HIP(x_record(j1, h2d));
        CQSA_HIP(x_record(j2, d2h));
        CQSA_HIP(x_wait(st, j1));
        CQSA_HIP(x_wait(st, j2));
        CQSA_HIP(x_sync(st));
        double h = 0, d = 0;
        for (auto& t : h2d_t) {
            float ms = 0;
            CQSA_HIP(x_elapsed(&ms, t.start, t.stop));
            h += ms;
        }
        for (auto& t : d2h_t) {
            float ms = 0;
            CQSA_HIP(x_elapsed(&ms, t.start, t.stop));
            d += ms;
        }
        if (info) {
            info->h2d_ms = h;
            info->d2h_ms = d;
        }
    }
    if (info) {
        info->chunk_pairs = pairs;
        info->kernel_launches = launches;
    }
    return CQSA_OK;
}

cqsa_status cqsa_attention_backward(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v,
                                    const cqsa_tensor* out, const cqsa_tensor* dout, const float* lse, int is_causal,
                                    float scale, cqsa_tensor* dq, cqsa_tensor* dk, cqsa_tensor* dv, float* stats_ws,
                                    void* stream) {
    g_err.clear();
    BwdProblem bp;
    CQSA_TRY(bwd_problem(q, k, v, out, dout, lse, is_causal, scale, dq, dk, dv, &bp));
    const Problem& P = bp.P;
    if (P.empty || P.Nk == 0) return CQSA_OK;
    if (P.streamed || bp.dout.host || bp.dq.host || bp.dk.host || bp.dv.host || bp.lse_host)
        return fail(CQSA_ERR_UNSUPPORTED,
                    "cqsa_attention_backward needs every operand in device memory (cqsa_attention_backward_ex "
                    "streams host operands)");
    hipStream_t st = static_cast<hipStream_t>(stream);
    float* stats = stats_ws;
    bool owned = false;
    if (!stats) {
        const size_t bytes = (size_t)P.B * P.Hq * P.Nq * 2 * sizeof(float);
        hipError_t e = hipMalloc(reinterpret_cast<void**>(&stats), bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(CQSA_ERR_OOM, "hipMalloc of %llu bytes for the row statistics failed: %s",
                        (unsigned long long)bytes, hipGetErrorString(e));
        }
        owned = true;
    }
    BwdArgs a = bwd_base(bp);
    a.q = reinterpret_cast<const uint16_t*>(P.q.data);
    a.k = reinterpret_cast<const uint16_t*>(P.k.data);
    a.v = reinterpret_cast<const uint16_t*>(P.v.data);
    a.dout = reinterpret_cast<const uint16_t*>(bp.dout.data);
    a.out = P.out.data;
    a.lse = bp.lse;
    a.q_sb = P.q.sb; a.q_sh = P.q.sh; a.q_sn = P.q.sn;
    a.k_sb = P.k.sb; a.k_sh = P.k.sh; a.k_sn = P.k.sn;
    a.v_sb = P.v.sb; a.v_sh = P.v.sh; a.v_sn = P.v.sn;
    a.do_sb = bp.dout.sb; a.do_sh = bp.dout.sh; a.do_sn = bp.dout.sn;
    a.o_sb = P.out.sb; a.o_sh = P.out.sh; a.o_sn = P.out.sn;
    a.l_sb = P.Hq * P.Nq;
    a.l_sh = P.Nq;
    a.stats = stats;
    a.dq = bp.dq.data; a.dk = bp.dk.data; a.dv = bp.dv.data;
    a.dq_sb = bp.dq.sb; a.dq_sh = bp.dq.sh; a.dq_sn = bp.dq.sn;
    a.dk_sb = bp.dk.sb; a.dk_sh = bp.dk.sh; a.dk_sn = bp.dk.sn;
    a.dv_sb = bp.dv.sb; a.dv_sh = bp.dv.sh; a.dv_sn = bp.dv.sn;
    a.Nq = P.Nq;
    a.Nk = P.Nk;
    a.causal_delta = P.Nk - P.Nq;
    a.stats_rows = P.Nq;
    a.accumulate = 0;
    hipError_t e = launch_bwd(a, (int)P.D, P.dtype == CQSA_F16 ? ET_F16 : ET_BF16, st);
    cqsa_status s = CQSA_OK;
    if (e != hipSuccess) s = fail(CQSA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
    if (owned) {
        (void)hipStreamSynchronize(st);
        (void)hipFree(stats);
    }
    return s;
}

cqsa_status cqsa_backward_schedule_trace(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v,
                                         const cqsa_tensor* out, const cqsa_tensor* dout, const float* lse,
                                         int32_t lse_where, int is_causal, uint64_t mem_budget, const cqsa_tensor* dq,
                                         const cqsa_tensor* dk, const cqsa_tensor* dv, const cqsa_options* opt,
                                         char* buf, uint64_t buf_len, uint64_t* needed) {
    g_err.clear();
    for (const cqsa_tensor* t : {q, k, v, out, dout, dq, dk, dv})
        if (!t || (t->where != CQSA_WHERE_HOST && t->where != CQSA_WHERE_DEVICE))
            return fail(CQSA_ERR_INVALID, "schedule trace: every tensor needs where = HOST or DEVICE");
    if (lse_where != CQSA_WHERE_HOST && lse_where != CQSA_WHERE_DEVICE)
        return fail(CQSA_ERR_INVALID, "schedule trace: lse_where must be HOST or DEVICE");
    if (mem_budget == 0) return fail(CQSA_ERR_INVALID, "schedule trace: mem_budget must be given");
    cqsa_options o;
    std::memset(&o, 0, sizeof o);
    if (opt) o = *opt;
    BwdProblem bp;
    CQSA_TRY(bwd_problem(q, k, v, out, dout, lse, is_causal, 0.f, const_cast<cqsa_tensor*>(dq),
                         const_cast<cqsa_tensor*>(dk), const_cast<cqsa_tensor*>(dv), &bp, false, lse_where));
    Recorder rec;
    if (!bp.P.empty && bp.P.Nk > 0) {
        uint64_t budget = 0;
        CQSA_TRY(resolve_budget(mem_budget, &budget));
        BwdPlan pl;
        CQSA_TRY(bwd_plan(bp, budget, o, &pl));
        char* ws = static_cast<char*>(o.workspace ? o.workspace : reinterpret_cast<void*>((uintptr_t)1 << 46));
        hipStream_t st = o.stream ? static_cast<hipStream_t>(o.stream) : reinterpret_cast<hipStream_t>((uintptr_t)0x10);
        DeviceRes res;
        res.init = true;
        res.num_cus = 256;
        res.h2d = reinterpret_cast<hipStream_t>((uintptr_t)0x20);
        res.d2h = reinterpret_cast<hipStream_t>((uintptr_t)0x30);
        rec.id(rec.streams, st);
        rec.line("workspace " + rng('W', ws, ws + pl.total));
        g_rec = &rec;
        const cqsa_status s = exec_bwd_chunked(bp, pl, ws, st, &res, nullptr);
        g_rec = nullptr;
        CQSA_TRY(s);
        rec.line("sync " + rec.st(st));
    }
    if (needed) *needed = rec.text.size() + 1;
    if (buf && buf_len > 0) {
        const size_t n = std::min<size_t>(rec.text.size(), buf_len - 1);
        std::memcpy(buf, rec.text.data(), n);
        buf[n] = 0;
        if (n < rec.text.size())
            return fail(CQSA_ERR_INVALID, "schedule trace: buffer of %llu bytes is too small", (unsigned long long)buf_len);
    }
    return CQSA_OK;
}

cqsa_status cqsa_attention_backward_ex(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v,
                                       const cqsa_tensor* out, const cqsa_tensor* dout, const float* lse, int is_causal,
                                       float scale, uint64_t mem_budget, cqsa_tensor* dq, cqsa_tensor* dk, cqsa_tensor* dv,
                                       const cqsa_options* opt, cqsa_plan_info* info) {
    g_err.clear();
    const auto t0 = std::chrono::steady_clock::now();
    cqsa_options o;
    std::memset(&o, 0, sizeof o);
    if (opt) o = *opt;
    if (info) std::memset(info, 0, sizeof *info);
    if (o.q_chunk < 0 || o.kv_chunk < 0) return fail(CQSA_ERR_INVALID, "negative chunk option");
    BwdProblem bp;
    CQSA_TRY(bwd_problem(q, k, v, out, dout, lse, is_causal, scale, dq, dk, dv, &bp));
    const Problem& P = bp.P;
    if (P.empty || P.Nk == 0) return CQSA_OK;
    const bool host = P.streamed || bp.dout.host || bp.dq.host || bp.dk.host || bp.dv.host || bp.lse_host;
    if (!host && o.q_chunk == 0 && o.kv_chunk == 0) {
        float* stats = nullptr;
        const uint64_t bytes = (uint64_t)P.B * P.Hq * P.Nq * 8;
        if (o.workspace && o.workspace_bytes >= bytes) stats = static_cast<float*>(o.workspace);
        CQSA_TRY(cqsa_attention_backward(q, k, v, out, dout, lse, is_causal, scale, dq, dk, dv, stats, o.stream));
        if (info) {
            info->workspace_bytes = bytes;
            info->chunk_pairs = 1;
            info->kernel_launches = P.D == 128 ? 4 : 3;
        }
        return CQSA_OK;
    }
    DeviceRes* res = nullptr;
    CQSA_TRY(device_res(&res));
    uint64_t budget = 0;
    CQSA_TRY(resolve_budget(mem_budget, &budget));
    BwdPlan pl;
    CQSA_TRY(bwd_plan(bp, budget, o, &pl));
    hipStream_t st = static_cast<hipStream_t>(o.stream);
    char* ws = nullptr;
    bool owned = false;
    if (o.workspace && o.workspace_bytes >= pl.total) {
        ws = static_cast<char*>(o.workspace);
    } else {
        hipError_t e = hipMalloc(reinterpret_cast<void**>(&ws), pl.total);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(CQSA_ERR_OOM, "hipMalloc of %llu workspace bytes failed: %s", (unsigned long long)pl.total,
                        hipGetErrorString(e));
        }
        owned = true;
    }
    cqsa_plan_info in;
    std::memset(&in, 0, sizeof in);
    cqsa_status s = exec_bwd_chunked(bp, pl, ws, st, res, &in);
    if (s == CQSA_OK && (owned || host)) {
        const hipError_t e = hipStreamSynchronize(st);
        if (e != hipSuccess) s = fail(CQSA_ERR_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
    }
    if (s != CQSA_OK) drain_after_failure(st, res);
    if (owned) (void)hipFree(ws);
    if (s != CQSA_OK) return s;
    if (info) {
        *info = in;
        info->streamed = host ? 1 : 0;
        info->q_chunk = pl.qc;
        info->kv_chunk = pl.kc;
        info->n_q_chunks = ceil_div(P.Nq, pl.qc);
        info->n_kv_chunks = ceil_div(P.Nk, pl.kc);
        info->workspace_bytes = pl.total;
        info->budget_bytes = budget;
        const uint64_t qb = (uint64_t)P.B * P.Hq * P.D, kb = (uint64_t)P.B * P.Hkv * P.D;
        uint64_t h2d_b = 0;
        if (P.out.host) h2d_b += qb * P.Nq * P.out.es;
        if (bp.lse_host) h2d_b += (uint64_t)P.B * P.Hq * P.Nq * 4;
        if (P.k.host) h2d_b += kb * P.Nk * 2;
        if (P.v.host) h2d_b += kb * P.Nk * 2;
        // Q and dout travel once per (query chunk, key chunk) pair, dout once more for the statistics
        if (bp.dout.host) h2d_b += qb * P.Nq * 2;
        for (int64_t c = 0; c < info->n_kv_chunks; ++c)
            for (int64_t r = 0; r < info->n_q_chunks; ++r) {
                const int64_t qa = r * pl.qc, qn = std::min(pl.qc, P.Nq - qa), ka = c * pl.kc;
                if (P.causal && ka > qa + qn - 1 + (P.Nk - P.Nq)) continue;
                h2d_b += qb * qn * 2 * ((P.q.host ? 1 : 0) + (bp.dout.host ? 1 : 0));
            }
        info->h2d_bytes = h2d_b;
        info->d2h_bytes = (uint64_t)bp.dq.es * (qb * P.Nq * (bp.dq.host ? 1 : 0) + kb * P.Nk * ((bp.dk.host ? 1 : 0) + (bp.dv.host ? 1 : 0)));
        if (owned || host)
            info->wall_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    }
    return CQSA_OK;
}

cqsa_status cqsa_fwd_partial(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v, int is_causal,
                             float scale, int64_t kv_begin, int64_t kv_end, float* o_part, float* ml_part,
                             void* stream) {
    g_err.clear();
    Problem P;
    // out has q's shape; describe it with q's descriptor (it is not written)
    CQSA_TRY(build_problem(q, k, v, is_causal, scale, q, nullptr, 0, true, false, &P));
    if (P.q.host || P.k.host || P.v.host) return fail(CQSA_ERR_INVALID, "cqsa_fwd_partial takes device tensors");
    if (P.empty) return CQSA_OK;
    if (kv_begin < 0 || kv_end < kv_begin || kv_end > P.Nk)
        return fail(CQSA_ERR_INVALID, "key range [%lld, %lld) outside [0, %lld]", (long long)kv_begin,
                    (long long)kv_end, (long long)P.Nk);
    if (!o_part || !ml_part) return fail(CQSA_ERR_INVALID, "o_part / ml_part is NULL");
    FwdArgs a = base_args(P);
    set_q(a, P.q.data, P.q.sb, P.q.sh, P.q.sn);
    set_k(a, P.k.data, P.k.sb, P.k.sh, P.k.sn);
    set_v(a, P.v.data, P.v.sb, P.v.sh, P.v.sn);
    a.r0 = 0;
    a.r1 = P.Nq;
    a.k_lo = kv_begin;
    a.k_hi = kv_end;
    a.split_len = std::max<int64_t>(kv_end - kv_begin, 1);
    a.causal_delta = P.Nk - P.Nq;
    a.mode = FWD_PARTIAL;
    a.acc_o = o_part;
    a.acc_ml = ml_part;
    a.acc_rows = P.Nq;
    return run_fwd(P, a, static_cast<hipStream_t>(stream));
}

cqsa_status cqsa_lse_merge(const float* const* o_parts, const float* const* ml_parts, int32_t num_parts,
                           int64_t rows, int64_t D, float* o_out, float* ml_out, void* stream) {
    g_err.clear();
    if (num_parts < 1 || num_parts > kMaxMergeParts)
        return fail(CQSA_ERR_INVALID, "num_parts %d outside [1, %d]", num_parts, kMaxMergeParts);
    if (D != 64 && D != 128) return fail(CQSA_ERR_UNSUPPORTED, "D %lld is not 64 or 128", (long long)D);
    if (rows < 0) return fail(CQSA_ERR_INVALID, "negative rows");
    if (!o_parts || !ml_parts || !o_out || !ml_out) return fail(CQSA_ERR_INVALID, "NULL pointer");
    MergeArgs m;
    std::memset(&m, 0, sizeof m);
    for (int p = 0; p < num_parts; ++p) {
        if (!o_parts[p] || !ml_parts[p]) return fail(CQSA_ERR_INVALID, "part %d is NULL", p);
        if (!aligned16(o_parts[p])) return fail(CQSA_ERR_UNSUPPORTED, "part %d is not 16-byte aligned", p);
        m.part_o[p] = o_parts[p];
        m.part_ml[p] = ml_parts[p];
    }
    if (!aligned16(o_out)) return fail(CQSA_ERR_UNSUPPORTED, "o_out is not 16-byte aligned");
    m.n_parts = num_parts;
    m.D = (int32_t)D;
    m.B = 1;
    m.Hq = 1;
    m.rows_per_head = rows;
    m.i_lo = 0;
    m.i_hi = rows;
    m.o_out = o_out;
    m.ml_out = ml_out;
    return run_merge(m, static_cast<hipStream_t>(stream));
}

cqsa_status cqsa_finalize(const float* o, const float* ml, cqsa_tensor* out, float* lse, void* stream) {
    g_err.clear();
    View ov;
    CQSA_TRY(make_view(out, "out", false, true, &ov));
    if (ov.host) return fail(CQSA_ERR_INVALID, "cqsa_finalize writes device memory only");
    if (ov.D != 64 && ov.D != 128) return fail(CQSA_ERR_UNSUPPORTED, "D %lld is not 64 or 128", (long long)ov.D);
    if (!o || !ml) return fail(CQSA_ERR_INVALID, "NULL pointer");
    if ((reinterpret_cast<uintptr_t>(ov.data) % (4 * ov.es)) || ov.sn % 4 || ov.sh % 4 || ov.sb % 4)
        return fail(CQSA_ERR_UNSUPPORTED, "out data and strides must be aligned to 4 elements");
    MergeArgs m;
    std::memset(&m, 0, sizeof m);
    m.part_o[0] = o;
    m.part_ml[0] = ml;
    m.n_parts = 1;
    m.D = (int32_t)ov.D;
    m.B = (int32_t)ov.B;
    m.Hq = (int32_t)ov.H;
    m.rows_per_head = ov.N;
    m.i_lo = 0;
    m.i_hi = ov.N;
    m.final_out = 1;
    m.out_dtype = elem_type(ov.dtype);
    m.out = ov.data;
    m.o_sb = ov.sb;
    m.o_sh = ov.sh;
    m.o_sn = ov.sn;
    m.lse = lse;
    m.l_sb = ov.H * ov.N;
    m.l_sh = ov.N;
    return run_merge(m, static_cast<hipStream_t>(stream));
}

cqsa_status cqsa_probe_device(uint64_t copy_bytes, int32_t repeats, cqsa_probe_result* out) {
    g_err.clear();
    if (!out) return fail(CQSA_ERR_INVALID, "out is NULL");
    if (repeats < 1 || repeats > 100) return fail(CQSA_ERR_INVALID, "repeats (%d) must be in [1, 100]", repeats);
    if (copy_bytes < (1ull << 20) || copy_bytes > (1ull << 34) || copy_bytes % 16)
        return fail(CQSA_ERR_INVALID, "copy_bytes (%llu) must be a multiple of 16 in [2^20, 2^34]",
                    (unsigned long long)copy_bytes);
    *out = cqsa_probe_result{};
    int dev = 0, cus = 0, wall_khz = 0;
    CQSA_HIP(hipGetDevice(&dev));
    CQSA_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    CQSA_HIP(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev));
    if (cus < 1 || wall_khz < 1) return fail(CQSA_ERR_HIP, "device reports %d compute units, wall clock %d kHz", cus, wall_khz);
    // 4-wave workgroups: eight per compute unit for the matrix cores (not all resident at once; the
    // rate is taken over the whole launch), two for LDS (32 KiB each)
    const int mfma_blocks = 8 * cus, lds_blocks = 2 * cus;
    const int waves = 4 * mfma_blocks;             // the larger of the two launches
    constexpr int kMfmaIters = 4096, kLdsIters = 32768;

    struct Res {   // everything the probe holds, released on every return
        void *sink = nullptr, *src = nullptr, *dst = nullptr;
        uint64_t* clk = nullptr;
        hipEvent_t e0 = nullptr, e1 = nullptr;
        ~Res() {
            if (e0) (void)hipEventDestroy(e0);
            if (e1) (void)hipEventDestroy(e1);
            for (void* p : {sink, src, dst, static_cast<void*>(clk)})
                if (p) (void)hipFree(p);
        }
    } r;
    auto alloc = [](void** p, size_t bytes) -> cqsa_status {
        const hipError_t e = hipMalloc(p, bytes);
        if (e == hipSuccess) return CQSA_OK;
        (void)hipGetLastError();
        *p = nullptr;
        return fail(e == hipErrorOutOfMemory ? CQSA_ERR_OOM : CQSA_ERR_HIP, "hipMalloc of %zu bytes failed: %s", bytes,
                    hipGetErrorString(e));
    };
    CQSA_TRY(alloc(&r.sink, (size_t)mfma_blocks * 256 * 4));
    CQSA_TRY(alloc(reinterpret_cast<void**>(&r.clk), (size_t)waves * 2 * sizeof(uint64_t)));
    CQSA_TRY(alloc(&r.src, copy_bytes));
    CQSA_TRY(alloc(&r.dst, copy_bytes));
    CQSA_HIP(hipMemset(r.src, 0x3c, copy_bytes));
    CQSA_HIP(hipEventCreate(&r.e0));
    CQSA_HIP(hipEventCreate(&r.e1));
    std::vector<uint64_t> clk((size_t)waves * 2);

    // one untimed launch, then `repeats` timed ones: the fastest time, and the clock of that launch
    // averaged over its first clocked_waves waves (0 when the kernel records no clock)
    auto run = [&](auto&& launch, int clocked_waves, double* secs, double* hz) -> cqsa_status {
        CQSA_HIP(launch());
        CQSA_HIP(hipDeviceSynchronize());
        double best = 0.0, best_hz = 0.0;
        for (int i = 0; i < repeats; ++i) {
            CQSA_HIP(hipEventRecord(r.e0, nullptr));
            CQSA_HIP(launch());
            CQSA_HIP(hipEventRecord(r.e1, nullptr));
            CQSA_HIP(hipEventSynchronize(r.e1));
            float ms = 0.f;
            CQSA_HIP(hipEventElapsedTime(&ms, r.e0, r.e1));
            double f = 0.0;
            if (clocked_waves > 0) {
                CQSA_HIP(hipMemcpy(clk.data(), r.clk, (size_t)clocked_waves * 2 * sizeof(uint64_t),
                                   hipMemcpyDeviceToHost));
                int n = 0;
                for (int w = 0; w < clocked_waves; ++w)
                    if (clk[2 * w + 1] > 0) {
                        f += (double)clk[2 * w] / (double)clk[2 * w + 1];
                        ++n;
                    }
                f = n ? f / n * wall_khz * 1e3 : 0.0;
            }
            if (i == 0 || ms * 1e-3 < best) {
                best = ms * 1e-3;
                best_hz = f;
            }
        }
        *secs = best;
        if (hz) *hz = best_hz;
        return CQSA_OK;
    };
    CQSA_TRY(run([&] { return launch_probe_mfma(mfma_blocks, static_cast<float*>(r.sink), r.clk, kMfmaIters, nullptr); },
                 4 * mfma_blocks, &out->mfma_seconds, &out->mfma_clock_hz));
    CQSA_TRY(run([&] { return launch_probe_lds(lds_blocks, static_cast<uint32_t*>(r.sink), r.clk, kLdsIters, nullptr); },
                 4 * lds_blocks, &out->lds_seconds, &out->lds_clock_hz));
    // the copy: four workgroups per compute unit, which measured fastest (5.7 TB/s for 1 GiB, against
    // 4.6-4.8 with 8 to 64, and 5.2 for the runtime's own device copy)
    CQSA_TRY(run([&] { return launch_probe_copy(4 * cus, r.src, r.dst, (int64_t)copy_bytes, nullptr); }, 0,
                 &out->copy_seconds, nullptr));
    out->mfma_f16_flop_per_s = 4.0 * mfma_blocks * kMfmaIters * 4 * 32768.0 / out->mfma_seconds;
    out->lds_read_bytes_per_s = 4.0 * lds_blocks * kLdsIters * 8 * 1024.0 / out->lds_seconds;
    out->hbm_copy_bytes_per_s = 2.0 * (double)copy_bytes / out->copy_seconds;
    out->compute_units = cus;
    out->wall_clock_khz = wall_khz;
    return CQSA_OK;
}

}  // extern "C"
