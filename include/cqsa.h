/*
 * cqsa.h -- exact scaled-dot-product attention for AMD Instinct MI355X (gfx950).
 *
 * The attention softmax(scale * Q K^T [+ causal mask]) V is computed as query
 * chunks x key/value chunks.  Each (query rows, key range) piece yields an
 * unnormalised partial triple (O, m, l): O = sum_j exp(s_j - m) v_j, m = the
 * largest scaled logit, l = sum_j exp(s_j - m).  Partials are merged exactly by
 * the log-sum-exp rule, so a context that does not fit in device memory can be
 * streamed from pinned host memory and still give the monolithic answer.  This
 * is the method of the Stream-CQSA pages (exact attention for contexts past
 * device memory: stream-cqsa 2.2.2 -> 2.2.3 diff, README.md section "Use", and
 * the attention() docstring in stream_cqsa/api.py of the 2.2.0 -> 2.2.2 diff).
 *
 * Conventions shared by every entry point
 *   - Tensors are described by cqsa_tensor: shape [B, H, N, D] and element
 *     strides; stride[3] (head dim) must be 1.  Any batch/head/row strides work,
 *     so both [B,H,N,D] and token-major [B,N,H,D] storage are accepted.
 *   - q is [B, Hq, Nq, D]; k and v are [B, Hkv, Nk, D] with Hq % Hkv == 0.
 *     Query head h reads key/value head h / (Hq / Hkv) (grouped-query attention,
 *     the repeat-interleave mapping of PyTorch SDPA's enable_gqa).
 *   - q, k, v are all CQSA_F16 or all CQSA_BF16; D is 64 or 128.  Products run
 *     on the matrix cores in that type with fp32 accumulation; softmax is fp32.
 *   - Causal masking is bottom-right aligned: query row i sits at key position
 *     i + Nk - Nq and sees keys j <= i + Nk - Nq.  With Nq == Nk this is the
 *     ordinary lower-triangular mask.  Causal calls need Nq <= Nk (every row must
 *     see at least one key).  (PyTorch aligns Nq != Nk top-left; the Stream-CQSA
 *     pages only ever use square calls.)
 *   - scale <= 0 (or NaN) selects the SDPA default 1/sqrt(D).  The scale is used
 *     as the given fp32 value.
 *   - lse, when requested, is fp32 [B, Hq, Nq] contiguous: m + ln(l), natural log
 *     of the sum of exp(scaled logits).
 *   - Memory: device pointers or pinned host pointers (hipHostMalloc / torch
 *     pin_memory).  Pageable host memory is rejected with CQSA_ERR_INVALID before
 *     any work (block-streamer 0.1.0, README section "Streams, residency, and
 *     memory budget": an unpinned transfer source must fail loudly).
 *   - All buffers are caller-owned; the library keeps no pointer after return.
 *   - The calls run on the current HIP device.  Errors never throw: every call
 *     returns a cqsa_status, and cqsa_last_error() returns a message for the
 *     calling thread.  Arguments are validated before any device work starts.
 *     A call that fails after it has issued device work (a failed launch or
 *     copy) returns only once its stream and the library's copy streams have
 *     drained: nothing of the failed call still reads or writes caller memory.
 *     Its outputs are then unspecified.
 */
#ifndef CQSA_H
#define CQSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CQSA_ABI_VERSION 5

typedef enum {
    CQSA_OK = 0,
    CQSA_ERR_INVALID = -1,     /* bad argument: shape, stride, dtype mix, pageable host memory, no visible key */
    CQSA_ERR_UNSUPPORTED = -2, /* head dim not 64/128, input dtype not fp16/bf16, misaligned data or rows */
    CQSA_ERR_BUDGET = -3,      /* mem_budget below the smallest plan; the message names the bytes needed */
    CQSA_ERR_OOM = -4,         /* hipMalloc failed (no retry: re-planning is the caller's choice) */
    CQSA_ERR_HIP = -5          /* a HIP runtime call failed; the message carries hipGetErrorString */
} cqsa_status;

typedef enum { CQSA_F16 = 0, CQSA_BF16 = 1, CQSA_F32 = 2 } cqsa_dtype;

/* Where a tensor lives.  DETECT asks hipPointerGetAttributes. */
typedef enum { CQSA_WHERE_DETECT = 0, CQSA_WHERE_DEVICE = 1, CQSA_WHERE_HOST = 2 } cqsa_where;

typedef struct {
    void* data;         /* first element; may be NULL only for cqsa_plan or an empty tensor */
    int32_t dtype;      /* cqsa_dtype */
    int32_t where;      /* cqsa_where */
    int64_t shape[4];   /* [B, H, N, D] */
    int64_t stride[4];  /* element strides; stride[3] == 1 */
} cqsa_tensor;

/* Merge strategies for multi-chunk plans.  The request applies to chunked plans (KV chunks run one
 * after another); side-by-side KV splits (kv_splits > 1) run at the same time, so their partials always
 * go through the merge kernel, whatever is requested. */
typedef enum {
    CQSA_MERGE_AUTO = 0,   /* the planner's choice: CQSA_MERGE_FUSED for chunked plans, the merge kernel
                              for side-by-side KV splits */
    CQSA_MERGE_KERNEL = 1, /* each KV chunk writes a partial; a separate LSE-merge kernel folds it in */
    CQSA_MERGE_FUSED = 2   /* the forward kernel folds its partial into the running triple in its epilogue */
} cqsa_merge_mode;

typedef struct {
    int64_t q_chunk;          /* query rows per Q chunk; 0 = planner */
    int64_t kv_chunk;         /* keys per KV chunk; 0 = planner; > 0 forces this split */
    int32_t kv_splits;        /* single-chunk device calls: KV splits run side by side and merged
                                 (fills the GPU when there are few query tiles); 0 = planner, 1 = off */
    int32_t merge_mode;       /* cqsa_merge_mode */
    void* workspace;          /* device memory the call may use instead of allocating; NULL = allocate */
    uint64_t workspace_bytes; /* its size */
    void* stream;             /* hipStream_t carrying the compute; NULL = the null stream */
    int32_t num_cus;          /* cqsa_plan only: compute units to plan for; 0 = ask the device */
    int32_t cqs_c;            /* > 0: run the cyclic quorum-set schedule over cqs_c parts (below);
                                 0 = the Q-chunk x KV-chunk grid */
    int32_t cqs_l;            /* size of the interest set cqs_set */
    int32_t precision;        /* 0: P is rounded to the input dtype for the PV product (the default);
                                 1: split P: the PV product takes P as an fp16/bf16 hi part plus the
                                 rounded residual as a lo part, in two accumulator chains summed in
                                 fp32 at the end (the hi/lo split with separate chains of Strata pull
                                 request #800); about twice the PV work, error near the fp32 class */
    const int32_t* cqs_set;   /* the interest set: cqs_l distinct part offsets in [0, cqs_c);
                                 NULL = the built-in set for cqs_c (see cqsa_cqs_default_set) */
    int64_t wave_tokens;      /* quorum-set schedule: packed-row budget of a wave, the consecutive
                                 subproblems that share one launch (query rows of the wave's query
                                 parts plus key rows of its key parts); 0 = min(2^22, max(2^20,
                                 Nq + Nk)); 1 = one subproblem (or one query part's pairs of a
                                 subproblem, see below) per wave.  With host operands the
                                 planner halves it until two waves' staging fits the memory budget
                                 (copy of one wave under the compute of the other), cutting waves
                                 per query part of a subproblem when whole subproblems are too large;
                                 failing that, until one wave's staging fits. */
    int32_t cqs_itr;          /* depth of the quorum-set decomposition: 0 or 1 = one level (c parts);
                                 itr > 1 = the set applied again inside each part, itr levels deep
                                 (c^itr parts and subproblems, at most 4096; see below) */
} cqsa_options;

/* What a plan does (filled by cqsa_plan and cqsa_attention_ex). */
typedef struct {
    int32_t streamed;          /* 1 when an operand lives in host memory and is copied in chunks */
    int32_t merge_mode;        /* as planned: 0 single pass, CQSA_MERGE_KERNEL, CQSA_MERGE_FUSED */
    int64_t q_chunk;           /* query rows per Q chunk */
    int64_t kv_chunk;          /* keys per KV chunk */
    int64_t n_q_chunks;
    int64_t n_kv_chunks;       /* KV chunks of the whole key range */
    int32_t kv_splits;         /* side-by-side KV splits of a single-chunk call (1 = none) */
    int32_t block_m;           /* query rows per workgroup of the forward kernel */
    int64_t chunk_pairs;       /* (Q chunk, KV chunk) pairs that run; causal skipping applied */
    int64_t merges;            /* log-sum-exp merges (merge-kernel launches or fused epilogues) */
    int64_t kernel_launches;
    uint64_t workspace_bytes;  /* device bytes the plan uses (allocated unless a workspace is given) */
    uint64_t budget_bytes;     /* the byte limit planned against: mem_budget x 0.85 */
    uint64_t h2d_bytes;        /* host-to-device bytes the plan copies */
    uint64_t d2h_bytes;        /* device-to-host bytes */
    double h2d_ms;             /* summed duration of the H2D copies (HIP events; streamed calls) */
    double d2h_ms;             /* summed duration of the D2H copies */
    double wall_ms;            /* host wall time of a synchronising call */
    int32_t cqs_c;             /* parts of a quorum-set schedule (0 = grid schedule) */
    int32_t cqs_subproblems;   /* subproblems that run (those owning at least one non-empty part pair) */
    int32_t cqs_waves;         /* waves of the quorum-set schedule */
    int32_t reserved0;
    int64_t wave_tokens;       /* the packed-row budget the waves were cut to */
} cqsa_plan_info;

/*
 * cqsa_attention: out = softmax(scale * q k^T [+ causal mask]) v, exactly.
 *
 *   q, k, v     inputs, as described above; device or pinned host memory.
 *   is_causal   nonzero for the bottom-right causal mask.
 *   scale       logit scale; <= 0 selects 1/sqrt(D).
 *   mem_budget  most device bytes the call may use for its own buffers
 *               (staging, accumulators, partials); the planner keeps to 85% of it,
 *               the safety margin of the Stream-CQSA planner (stream-cqsa
 *               2.2.0 -> 2.2.2 diff, stream_cqsa/autoconfig.py, plan(), safety=0.85).
 *               0 = the free device memory (hipMemGetInfo) x 0.85.
 *   out         [B, Hq, Nq, D], CQSA_F16, CQSA_BF16 or CQSA_F32 (results are rounded
 *               to nearest even from fp32); device or pinned host memory.
 *   lse         NULL, or fp32 [B, Hq, Nq] (device or pinned host).
 * With every operand on the device and no allocation needed, the call is
 * ordered on the null stream and returns without waiting; otherwise it returns
 * after the work is done.
 */
cqsa_status cqsa_attention(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v, int is_causal,
                           float scale, uint64_t mem_budget, cqsa_tensor* out, float* lse);

/*
 * cqsa_attention_ex: cqsa_attention with options and a report.
 *   opt   NULL = defaults.  opt->stream carries the compute; with a workspace of
 *         sufficient size the library allocates nothing.  Forced chunk sizes
 *         (kv_chunk, q_chunk) run the decomposed schedule even when everything fits.
 *   info  NULL, or filled with the plan and, for synchronising calls, timings.
 */
cqsa_status cqsa_attention_ex(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v, int is_causal,
                              float scale, uint64_t mem_budget, cqsa_tensor* out, float* lse,
                              const cqsa_options* opt, cqsa_plan_info* info);

/* want_lse of cqsa_plan and cqsa_schedule_trace: whether the call returns lse, and where the lse
 * array lives (host lse is staged in the workspace and copied back, like host out). */
#define CQSA_LSE_NONE 0      /* no lse */
#define CQSA_LSE_WITH_OUT 1  /* lse lives where out lives */
#define CQSA_LSE_DEVICE 2    /* lse in device memory */
#define CQSA_LSE_HOST 3      /* lse in pinned host memory */

/*
 * cqsa_attention_noalloc: cqsa_attention for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  It makes no hipMalloc,
 * hipFree or other allocating call.  The only buffer its kernels need beyond q, k, v, out and lse,
 * the partial triples of a key range split across the GPU, lives in a fixed device array inside the
 * library: CQSA_NOALLOC_SCRATCH_BYTES per device, held by every device the library runs on from the
 * loading of its code until the process ends.
 *   q, k, v, out, lse  as for cqsa_attention, all in device memory (host operands: CQSA_ERR_UNSUPPORTED).
 *   kv_splits          0 = the planner's split (within the array), 1 = one pass, n > 1 = n side-by-side
 *                      splits merged by log-sum-exp; a split whose partials exceed the array gives
 *                      CQSA_ERR_BUDGET (with the bytes it needs) before any device work.
 *   stream             hipStream_t (NULL = the null stream); the call is stream-ordered and returns
 *                      without waiting.
 *   info               NULL, or the plan that ran.
 * Every call on one device uses that device's one array and leaves its last contents there (nothing
 * in it needs to start at zero): calls that may overlap on one device (on different streams, or from
 * several threads) race on it and must be ordered by the caller.  The first call on each device looks
 * up the array's address (hipGetSymbolAddress, no allocation); a caller that captures calls into a
 * graph makes one call on that device before capturing.
 */
#define CQSA_NOALLOC_SCRATCH_BYTES (128ull << 20)

cqsa_status cqsa_attention_noalloc(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v, int is_causal,
                                   float scale, cqsa_tensor* out, float* lse, int32_t kv_splits, void* stream,
                                   cqsa_plan_info* info);

/*
 * cqsa_plan: the plan cqsa_attention_ex would run, without running it or
 * allocating (the dry run of the pages' estimate(): stream-cqsa 2.2.2 -> 2.2.3
 * diff, README.md section "Use").  Tensor data may be NULL; then each tensor's
 * `where` must say DEVICE or HOST.  want_lse is one of the CQSA_LSE_ values
 * (CQSA_ERR_INVALID otherwise).  With mem_budget > 0, explicit `where` values
 * and opt->num_cus > 0 the call makes no HIP call at all.
 */
cqsa_status cqsa_plan(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v, int is_causal,
                      uint64_t mem_budget, const cqsa_tensor* out, int want_lse, const cqsa_options* opt,
                      cqsa_plan_info* info);

/*
 * cqsa_schedule_trace: the operations cqsa_attention_ex would issue for this problem, recorded instead
 * of issued (no HIP call is made, no memory is allocated or touched): one line per copy, kernel
 * launch, event record, event wait and stream synchronisation, in host issue order, with the device
 * byte ranges each copy and kernel reads (R:lo:hi) and writes (W:lo:hi):
 *     workspace W:lo:hi | copy sN R|W:lo:hi | kernel sN fwd|merge|wave R:..|W:.. ... |
 *     record sN eM | wait sN eM | sync sN
 * Streams (sN) and events (eM) are numbered by first use; s0 is the caller's stream.  It exists to
 * check the executors' stream and event ordering on a machine without a GPU (any two operations that
 * touch one device byte, one of them writing, must be ordered by their streams and events).
 * The tensors' data pointers are used as given (stand-in addresses are fine; they are never
 * dereferenced); every `where` must be DEVICE or HOST and mem_budget must be > 0; opt->workspace and
 * opt->stream, when set, stand in for the workspace base and the caller's stream.  want_lse (a
 * CQSA_LSE_ value, which also says where lse lives) records the lse writes at a stand-in address
 * 2^40 bytes past out.  The text (NUL-terminated) goes to buf;
 * *needed (may be NULL) receives the size it needs.  CQSA_ERR_INVALID when buf_len is too small (buf
 * then holds the truncated text), or an argument error of cqsa_plan.
 */
cqsa_status cqsa_schedule_trace(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v, int is_causal,
                                uint64_t mem_budget, const cqsa_tensor* out, int want_lse, const cqsa_options* opt,
                                char* buf, uint64_t buf_len, uint64_t* needed);

/* The chunked backward's operations (cqsa_attention_backward_ex with host operands or forced chunks),
 * recorded the same way: every tensor's `where` must be HOST or DEVICE, lse_where says where lse
 * lives, and the stand-in addresses are never dereferenced.  Kernel lines name bwd_stats, bwd_dq,
 * bwd_dkdv and cast. */
cqsa_status cqsa_backward_schedule_trace(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v,
                                         const cqsa_tensor* out, const cqsa_tensor* dout, const float* lse,
                                         int32_t lse_where, int is_causal, uint64_t mem_budget, const cqsa_tensor* dq,
                                         const cqsa_tensor* dk, const cqsa_tensor* dv, const cqsa_options* opt,
                                         char* buf, uint64_t buf_len, uint64_t* needed);

/*
 * cqsa_fwd_partial: the partial triple of one KV chunk, for every query row.  This is one
 * subproblem's forward pass of the method, the FlashAttention-2 online softmax of the pages' CQS
 * forward kernel (stream-cqsa 2.2.0 -> 2.2.2 diff, README.md, kernel table) run over one key range
 * and stopped before the normalisation, so that the ranges can be merged afterwards (stream-cqsa
 * 2.2.2 -> 2.2.3 diff, README.md section "Use": the decomposed call still gives the monolithic
 * answer).
 *   q, k, v            device tensors as above.
 *   kv_begin, kv_end   the key range [kv_begin, kv_end) of the chunk (0 <= begin <= end <= Nk).
 *   o_part             fp32 [B, Hq, Nq, D] contiguous: sum over visible keys in the range of
 *                      exp(s - m) v (unnormalised).
 *   ml_part            fp32 [B, Hq, Nq, 2] contiguous: (m, l), m in natural-log units of the
 *                      scaled logits.  A row with no visible key in the range gets the identity
 *                      (O = 0, m = -inf, l = 0).
 *   stream             hipStream_t or NULL.  Stream-ordered; returns without waiting.
 */
cqsa_status cqsa_fwd_partial(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v, int is_causal,
                             float scale, int64_t kv_begin, int64_t kv_end, float* o_part, float* ml_part,
                             void* stream);

/*
 * cqsa_lse_merge: exact log-sum-exp merge of num_parts partial triples, row by row (the merge of
 * per-subproblem partial outputs that the pages' wave engine performs on the host, here on the
 * device: stream-cqsa 2.2.0 -> 2.2.2 diff, README.md, the paragraph on peak memory and the wave
 * budget, where each packed token keeps one fp32 partial output until its wave is merged):
 *   m = max_p m_p,  w_p = exp(m_p - m) (0 when m_p = -inf),  l = sum_p w_p l_p,
 *   O = sum_p w_p O_p.  Empty partials (m = -inf) are identities and never give NaN.
 *   o_parts[p]   device fp32 [rows, D];  ml_parts[p]  device fp32 [rows, 2] (m, l).
 *                The two pointer arrays themselves are host arrays of num_parts entries
 *                (1 <= num_parts <= 64).
 *   o_out, ml_out  device fp32 [rows, D] / [rows, 2]; may be the same memory as part 0.
 *   D            64 or 128.
 * Stream-ordered; returns without waiting.
 */
cqsa_status cqsa_lse_merge(const float* const* o_parts, const float* const* ml_parts, int32_t num_parts,
                           int64_t rows, int64_t D, float* o_out, float* ml_out, void* stream);

/*
 * cqsa_finalize: deliver a merged triple: out = O / l rounded to out's dtype, and
 * lse = m + ln(l).  This is the last step of the pages' attention() call, which leaves the fp32
 * result in the accumulator and then casts it to the input dtype and moves it to the caller
 * (stream-cqsa 2.2.0 -> 2.2.2 diff, stream_cqsa/api.py, _attention() and _deliver()), with the
 * softmax normaliser applied once at the end as in the FlashAttention-2 recurrence of the forward
 * kernel (the same diff, README.md, kernel table).
 *   o     device fp32 [B, Hq, Nq, D] contiguous (B, Hq, Nq, D taken from out's shape).
 *   ml    device fp32 [B, Hq, Nq, 2] contiguous.
 *   out   device tensor, any strides (stride[3] == 1); lse NULL or device fp32 [B, Hq, Nq].
 * A row with l = 0 (no visible key) gets out = 0 and lse = -inf.
 */
cqsa_status cqsa_finalize(const float* o, const float* ml, cqsa_tensor* out, float* lse, void* stream);

/*
 * cqsa_attention_backward: the gradients of out = softmax(scale q k^T [+ causal mask]) v for an
 * upstream gradient dout, by the derivative of the same expression (P = exp(s - lse),
 * dV = P^T dO, dS = P (dO V^T - rowsum(dO * out)), dQ = scale dS K, dK = scale dS^T Q): the
 * backward the Stream-CQSA pages ship beside the forward (stream-cqsa 2.2.0 -> 2.2.2 diff, README.md,
 * kernel table).  Device memory only.
 *
 *   q, k, v     the forward's inputs (fp16 or bf16, D 64 or 128, causal bottom-right as above).
 *   out, lse    the forward's output (any dtype) and fp32 lse [B, Hq, Nq] contiguous (device).
 *   dout        [B, Hq, Nq, D] in q's dtype; rows 16-byte aligned.
 *   dq          [B, Hq, Nq, D]; dk, dv [B, Hkv, Nk, D] (with GQA, summed over each key/value
 *               head's query heads); one dtype among fp16, bf16, fp32.  Written, not accumulated.
 *   stats_ws    device scratch of 2 B Hq Nq floats (row statistics), or NULL: the library then
 *               allocates it and the call returns after the work is done.
 *   stream      hipStream_t (NULL = null stream); with stats_ws the call is stream-ordered and
 *               returns without waiting.
 * Deterministic (every gradient element is summed by one wave in a fixed order).  Host-resident
 * operands give CQSA_ERR_UNSUPPORTED.
 */
cqsa_status cqsa_attention_backward(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v,
                                    const cqsa_tensor* out, const cqsa_tensor* dout, const float* lse, int is_causal,
                                    float scale, cqsa_tensor* dq, cqsa_tensor* dk, cqsa_tensor* dv, float* stats_ws,
                                    void* stream);

/*
 * cqsa_attention_backward_ex: the same gradients, with every operand (q, k, v, out, dout, lse and the
 * gradients) in device memory or in pinned host memory, under a device-memory budget.  When every
 * operand is on the device and opt forces no chunking it is cqsa_attention_backward (opt->workspace,
 * when large enough, holds the statistics).  Otherwise the problem runs in query chunks x key chunks,
 * key chunks outermost: the row statistics of every query chunk first, then for each key chunk (K, V
 * staged) every query chunk that sees it (Q, dout staged); dQ accumulates in fp32 for all query rows
 * and dK, dV in fp32 for the key chunk, rounded into the caller's gradients when complete.  Host
 * operands move on two side streams with double-buffered staging; the call then returns after
 * completion.  Device bytes: the fp32 dQ accumulator (B Hq Nq D 4) and statistics (B Hq Nq 8) plus
 * the chunks' accumulators and staging; the chunks are halved until that fits mem_budget x 0.85
 * (0 = free memory x 0.85), else CQSA_ERR_BUDGET.  opt: q_chunk, kv_chunk (> 0 forces the size),
 * workspace (used when large enough, else hipMalloc), stream.  info (may be NULL): chunk sizes and
 * counts, pairs, launches, workspace, H2D/D2H bytes and times.
 */
cqsa_status cqsa_attention_backward_ex(const cqsa_tensor* q, const cqsa_tensor* k, const cqsa_tensor* v,
                                       const cqsa_tensor* out, const cqsa_tensor* dout, const float* lse, int is_causal,
                                       float scale, uint64_t mem_budget, cqsa_tensor* dq, cqsa_tensor* dk, cqsa_tensor* dv,
                                       const cqsa_options* opt, cqsa_plan_info* info);

/* Message describing the last failure on the calling thread ("" if none). */
const char* cqsa_last_error(void);

/* CQSA_ABI_VERSION of the built library. */
int32_t cqsa_version(void);

/* sizeof of the ABI structs, for bindings to check their layout:
 * 0 = cqsa_tensor, 1 = cqsa_options, 2 = cqsa_plan_info, 3 = cqsa_probe_result; 0 for other values. */
uint64_t cqsa_struct_size(int32_t which);

/*
 * Cyclic quorum-set (CQS) schedule.  The method decomposes one attention call into c^itr
 * subproblems over c parts of the sequence, each subproblem holding an interest set of l parts,
 * with work factor (l^2/c)^itr (stream-cqsa 2.2.0 -> 2.2.2 diff, stream_cqsa/autoconfig.py, plan()
 * docstring; the default set (0, 1, 3) for c = 7 in stream_cqsa/api.py).  At depth itr = 1 the query
 * rows and the keys are each split into c contiguous parts (part p covers [floor(p n / c),
 * floor((p + 1) n / c))), and subproblem i holds the parts (i + s) mod c for s in the set.  The set
 * must be a cyclic quorum set: every pair of parts meets in some subproblem, i.e. every d in 1..c-1 is
 * a difference of two set elements mod c.  The pair (query part a, key part b) is computed by exactly
 * one subproblem, its owner: the smallest i whose parts contain both a and b.  At depth itr > 1
 * (cqsa_options.cqs_itr) the same set is applied inside each part of the level above: there are
 * C = c^itr contiguous parts, part p with base-c digits p_1 .. p_itr (p_1 the most significant, the
 * depth-1 part it lies in); subproblem I = (i_1 .. i_itr) holds the parts whose digit p_k is in
 * {(i_k + s) mod c} at every level k, i.e. l^itr of the C parts, and the owner of a pair is the
 * smallest such I (digit by digit the depth-1 owner).  Every pair of parts is still computed once.
 * Subproblems run in waves (the wave engine of the same pages: README.md, the paragraph on peak
 * memory and the wave budget; stream_cqsa/api.py, _pick_wave): consecutive subproblems are packed
 * into one wave while the rows it stages (query rows of its query parts plus key rows of its key
 * parts, each part counted once) stay within cqsa_options.wave_tokens.  A wave stages the union of
 * its parts once (from pinned host memory when the inputs live there) and runs as one batched launch
 * per 32 query and 32 key parts: every query part of the launch attends, in one online-softmax pass,
 * to all the key parts it owns pairs with in the wave, and the launch folds the result into a device
 * accumulator for all query rows by the log-sum-exp rule (on the device, in the kernel epilogue).
 * Waves run one after another, the staging of wave w + 1 overlapping the compute of wave w; the
 * accumulator is normalised at the end.  Causal pairs with no visible key are skipped.  Needs budget
 * for the fp32 accumulator (B Hq Nq (D + 2) 4 bytes) plus the staging of one query part's pairs of a
 * subproblem (two waves' staging when it fits, for the overlap); CQSA_ERR_BUDGET otherwise.
 */

/* owner[a * c + b] = the subproblem that computes the pair (query part a, key part b), for a valid
 * cyclic quorum set; CQSA_ERR_INVALID (with a message) when c < 1, l < 1, l > c, an element is
 * outside [0, c) or repeated, or some pair of parts shares no subproblem.  Host-only. */
cqsa_status cqsa_cqs_assign(int32_t c, const int32_t* interest_set, int32_t l, int32_t* owner);

/* The owner table of the depth-itr schedule (itr >= 1; itr = 1 is cqsa_cqs_assign): owner[a * C + b]
 * for the C = c^itr parts, C at most 4096.  Errors as cqsa_cqs_assign, and CQSA_ERR_INVALID for
 * itr < 1 or C > 4096.  Host-only. */
cqsa_status cqsa_cqs_assign_itr(int32_t c, const int32_t* interest_set, int32_t l, int32_t itr, int32_t* owner);

/* The built-in interest set for c parts (perfect difference sets: c = 3, 7, 13, 21, 31): writes up to
 * max_l elements to set and returns its size, or 0 when there is none for c. */
int32_t cqsa_cqs_default_set(int32_t c, int32_t* set, int32_t max_l);

/* Name and shape of the forward kernel a call with this head dim (64 or 128) and precision (see
 * cqsa_options) launches, e.g. "fwd_dma_kernel waves=4 keys_per_tile=64 rows_per_wave=32"; "" for
 * another head dim.  With precision 0 the choice follows cqsa_set_test_controls (fwd_variant 0 =
 * the default kernel).  The string is static; no HIP call is made. */
const char* cqsa_fwd_kernel_name(int64_t head_dim, int32_t precision);

/*
 * Test and measurement controls, process-wide (not part of the attention contract; every call
 * runs with the defaults, 0 and -1, unless a test or a measurement sets them):
 *   fwd_variant          0 = the default forward kernel of each head dim (the ping-pong DMA
 *                        kernel); 1..7 = the alternative kernels and shapes (6 = the DMA kernel's
 *                        best shape), so that tests can run every kernel and measurements can
 *                        compare them (cqsa_fwd_kernel_name names the choice).
 *   fail_after_launches  -1 = off; n >= 0 makes every forward launch of a call after its first n
 *                        fail from the host, as a failed launch would (CQSA_ERR_HIP), so that tests
 *                        can exercise the error path of a streamed call with no kernel fault.
 * CQSA_ERR_INVALID for values outside these ranges (nothing is changed then).  Host-only; no HIP
 * call.  Calls in flight on other threads see the change at their next launch.
 */
cqsa_status cqsa_set_test_controls(int32_t fwd_variant, int64_t fail_after_launches);

/*
 * Device probe: the rates the kernels are measured against, measured on the current device, each with
 * the shader clock it ran at.  Three kernels, each launched once untimed and then `repeats` times
 * between hip events on the null stream (the fastest launch is reported):
 *  - matrix cores: back-to-back v_mfma_f32_32x32x16_f16 with operands in registers, four independent
 *    accumulator chains per wave, eight 4-wave workgroups per compute unit;
 *  - LDS: ds_read_b128 at bank-conflict-free addresses (consecutive lanes on consecutive 16-byte
 *    granules), two 4-wave workgroups per compute unit;
 *  - HBM: a copy kernel over copy_bytes (the rate counts the bytes read plus the bytes written).
 * The clock is the mean over the waves of the launch of (shader cycles / wall-clock ticks) across
 * the wave's loop, times the wall-clock rate (hipDeviceAttributeWallClockRate).
 * copy_bytes: a multiple of 16 in [2^20, 2^34]; repeats in [1, 100].  Allocates 2 copy_bytes plus a
 * few KiB of device memory and frees them before returning (CQSA_ERR_OOM if that fails); synchronous.
 * CQSA_ERR_INVALID for bad arguments or a NULL result (checked before any HIP call), CQSA_ERR_HIP for
 * a failing HIP call.  Not part of the attention path: bench and profile tooling use it to state the
 * peak each figure is a fraction of.
 */
typedef struct {
    double mfma_f16_flop_per_s;    /* dense fp16 matrix-core FLOP/s */
    double mfma_clock_hz;          /* shader clock during that launch */
    double lds_read_bytes_per_s;   /* LDS bytes read per second, all compute units */
    double lds_clock_hz;
    double hbm_copy_bytes_per_s;   /* (read + written) bytes per second */
    double mfma_seconds, lds_seconds, copy_seconds;   /* the timed launches (fastest of `repeats`) */
    int32_t compute_units;
    int32_t wall_clock_khz;
} cqsa_probe_result;

cqsa_status cqsa_probe_device(uint64_t copy_bytes, int32_t repeats, cqsa_probe_result* out);

#ifdef __cplusplus
}
#endif

#endif /* CQSA_H */
