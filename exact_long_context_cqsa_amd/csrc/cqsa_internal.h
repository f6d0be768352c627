// Internal interface between the runtime (cqsa_api.cpp) and the gfx950 kernels
// (cqsa_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace cqsa {

// Epilogue of the forward kernel.
enum FwdMode : int32_t {
    FWD_FINAL = 0,    // write O / l in the output dtype and lse = m + ln l
    FWD_PARTIAL = 1,  // write the unnormalised triple (O, m, l) to the partial buffers
    FWD_ACCUM = 2     // merge the triple into the running (O, m, l) buffers in place
};

enum ElemType : int32_t { ET_F16 = 0, ET_BF16 = 1, ET_F32 = 2 };

// One forward launch: query rows [r0, r1) of the q view against keys [k_lo, k_hi)
// of the k/v views, optionally split into n_splits key ranges of split_len keys.
// Row and key indices are local to the views; the causal rule is
// key j visible to row i  <=>  j <= i + causal_delta.
struct FwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    int64_t q_sb, q_sh, q_sn;  // element strides
    int64_t k_sb, k_sh, k_sn;
    int64_t v_sb, v_sh, v_sn;
    int64_t r0, r1;
    int64_t k_lo, k_hi;
    int64_t split_len;
    int64_t causal_delta;
    int32_t B, Hq, Hkv, group;
    int32_t n_qt, n_splits;
    int32_t causal, mode;
    int32_t out_dtype;
    float scale_log2;          // scale * log2(e)
    // FWD_FINAL
    void* out;
    int64_t o_sb, o_sh, o_sn;
    float* lse;                // [b * l_sb + h * l_sh + i], may be null
    int64_t l_sb, l_sh;
    // FWD_PARTIAL / FWD_ACCUM: row (split, b, h, i) at ((split * B + b) * Hq + h) * acc_rows + i
    float* acc_o;              // [..][D]
    float* acc_ml;             // [..][2]
    int64_t acc_rows;
    int32_t p_split;           // 1: P enters the PV product as an fp16/bf16 hi part plus a lo residual
};

// One launch of the wave engine (the quorum-set schedule): several query parts, each against the
// union of its key parts that the launch's subproblems own, in one online-softmax pass per query row
// that folds into the running accumulator (FWD_ACCUM).  Parts are contiguous row ranges of the whole
// problem; a part's rows sit either in the caller's tensor (layout STRIDED: the FwdArgs strides) or in a
// compact staging copy of just that part (COMPACT_HEAD: [B][H][n][D], COMPACT_TOKEN: [B][n][H][D]).
enum WaveLayout : int32_t { WAVE_STRIDED = 0, WAVE_COMPACT_HEAD = 1, WAVE_COMPACT_TOKEN = 2 };

constexpr int kWaveCap = 32;   // query parts and key parts per launch

struct WaveQ {
    const uint16_t* q;   // element (b, h, 0, 0) of the part at q + b * sb + h * sh
    int64_t lo;          // first query row of the part (accumulator row)
    int32_t n;           // rows of the part
    uint32_t kmask;      // key parts (bits over WaveTable::ki) this part attends to in the launch
    int32_t t0;          // first query tile of the part in a head's tile list
    int32_t n_qt;        // query tiles of the part
};

struct WaveK {
    const uint16_t* k;   // element (b, h, 0, 0) of the part (layout k_layout / v_layout)
    const uint16_t* v;
    int64_t lo;          // first key of the part
    int32_t n;           // keys of the part
    int32_t pad;
};

struct WaveTable {
    WaveQ qi[kWaveCap];
    WaveK ki[kWaveCap];
    int32_t n_q, n_k;
    int32_t q_layout, k_layout, v_layout;
    int32_t H_q, H_kv;   // heads of the compact layouts (Hq for q, Hkv for k and v)
    int32_t n_tiles;     // query tiles of all parts per (b, query head); workgroups = B * Hq * n_tiles
};

constexpr int kMaxMergeParts = 64;

// Log-sum-exp merge of n_parts triples for rows (b, h, i), i in [i_lo, i_hi), laid out
// at (b * Hq + h) * rows_per_head + i.  With final_out set, writes out = O / l and lse
// instead of the merged triple.
struct MergeArgs {
    const float* part_o[kMaxMergeParts];
    const float* part_ml[kMaxMergeParts];
    int32_t n_parts;
    int32_t D;
    int32_t B, Hq;
    int64_t rows_per_head;
    int64_t i_lo, i_hi;
    float* o_out;
    float* ml_out;
    int32_t final_out;
    int32_t out_dtype;
    void* out;                 // element (b, h, i - i_lo + out_row0 ...) see below
    int64_t o_sb, o_sh, o_sn;  // out row for local row i is (i - i_lo)
    float* lse;
    int64_t l_sb, l_sh;
};

// Backward: gradients of out = softmax(scale q k^T [+ causal]) v for an upstream gradient dout, over
// Nq query rows and Nk keys (the whole problem, or one query chunk against one key chunk).  stats is
// an fp32 array of (lse * log2 e, -Delta) pairs, Delta = rowsum(dout * out): row i of head (b, h) at
// 2 ((b Hq + h) stats_rows + i), written by the first pass and read by the two gradient kernels.  The
// causal rule is key j visible to row i iff j <= i + causal_delta (Nk - Nq for a whole, bottom-right
// aligned problem).  dq is [B, Hq, Nq, D]; dk, dv are [B, Hkv, Nk, D] and sum over the query heads of
// their group.  With accumulate set the gradients are fp32 and each kernel adds to what they hold.
struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dout;
    const void* out;
    const float* lse;
    int64_t q_sb, q_sh, q_sn;
    int64_t k_sb, k_sh, k_sn;
    int64_t v_sb, v_sh, v_sn;
    int64_t do_sb, do_sh, do_sn;
    int64_t o_sb, o_sh, o_sn;
    int64_t l_sb, l_sh;
    float* stats;
    void* dq;
    void* dk;
    void* dv;
    int64_t dq_sb, dq_sh, dq_sn;
    int64_t dk_sb, dk_sh, dk_sn;
    int64_t dv_sb, dv_sh, dv_sn;
    int64_t Nq, Nk;
    int32_t B, Hq, Hkv, group;
    int32_t causal;
    int32_t out_dtype;   // ElemType of out
    int32_t grad_dtype;  // ElemType of dq, dk, dv
    float scale;
    float scale_log2;
    int64_t causal_delta;
    int64_t stats_rows;
    int32_t accumulate;
    int32_t pad;
};

hipError_t launch_bwd(const BwdArgs& a, int D, int dtype, hipStream_t stream);

// One pass of the backward: BWD_STATS (the row statistics), BWD_DQ or BWD_DKDV.
enum BwdPass : int32_t { BWD_STATS = 0, BWD_DQ = 1, BWD_DKDV = 2 };
hipError_t launch_bwd_pass(const BwdArgs& a, int D, int dtype, int pass, hipStream_t stream);

// fp32 rows of a compact [B][H][n][D] buffer, rounded (RNE) into element (b, h, i) of a strided
// [B, H, n, D] tensor of ElemType dtype.
hipError_t launch_cast(const float* src, int64_t B, int64_t H, int64_t n, int64_t D, void* dst, int dtype,
                       int64_t sb, int64_t sh, int64_t sn, hipStream_t stream);

// Which forward kernel shape the launches take (0 = the default); set by cqsa_set_test_controls.
void set_fwd_variant(int v);
int fwd_variant_count();

// Bytes of the fixed device array behind cqsa_attention_noalloc (CQSA_NOALLOC_SCRATCH_BYTES).
constexpr uint64_t kNoAllocScratchBytes = 128ull << 20;

// The device address of that array on the current device, resolved once per device
// (hipGetSymbolAddress) and kept; the error of the first resolution is returned.
hipError_t noalloc_scratch(void** ptr);

// Query rows per workgroup of the forward kernel for a head dim (and the split-P mode).
int fwd_block_m(int D, int p_split);
// Workgroups of the forward kernel (the default or the split-P shape) that one CU holds at once.
int fwd_wgs_per_cu(int D, int p_split);

// Name and shape of the forward kernel launched for a head dim ("" if none).
const char* fwd_kernel_name(int D, int p_split);

// Launchers (return the launch status).
hipError_t launch_fwd(const FwdArgs& a, int D, int dtype, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

// The wave engine's launch: a carries the problem-wide fields (strides of STRIDED views, B, Hq, Hkv,
// group, causal with causal_delta = Nk - Nq, scale, p_split, FWD_ACCUM with the accumulator base and
// acc_rows = Nq); blocks = B * Hq * t.n_tiles.
hipError_t launch_wave(const FwdArgs& a, const WaveTable& t, int blocks, int D, int dtype, hipStream_t stream);

// Query rows per workgroup of the wave kernel.
int wave_block_m(int D, int p_split);

// Rate probes (cqsa_probe.hip), 256-thread workgroups of four waves.  The matrix and LDS probes
// write one float / uint32 per thread to sink (blocks * 256 of them) and, per wave w, the shader
// cycles and wall-clock ticks of its loop to clk[2 w], clk[2 w + 1] (blocks * 8 uint64 in all).
hipError_t launch_probe_mfma(int blocks, float* sink, uint64_t* clk, int iters, hipStream_t stream);
hipError_t launch_probe_lds(int blocks, uint32_t* sink, uint64_t* clk, int iters, hipStream_t stream);
// dst = src over bytes (a multiple of 16; both 16-byte aligned).
hipError_t launch_probe_copy(int blocks, const void* src, void* dst, int64_t bytes, hipStream_t stream);

}  // namespace cqsa
