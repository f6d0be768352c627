// gfx950 (CDNA4) kernels for exact attention by Q-tiles x KV-chunks with a log-sum-exp merge.
//
// Forward kernels: one workgroup = BM query rows of one (batch, query head) against one key range.
// The online softmax (the FlashAttention-2 recurrence that the pages' CQS forward kernel builds on:
// stream-cqsa 2.2.0 -> 2.2.2 diff, README.md) produces the partial triple (O, m, l) of the range;
// the epilogue normalises it, stores it, or folds it into a running triple.
//   fwd_dma_kernel  K/V tiles staged into LDS by buffer-load DMA, V read with transpose loads
//                   (the default);
//   fwd_kernel      K/V tiles staged through registers, V written to LDS transposed;
//   fwd_pp_kernel   as fwd_kernel, with the two halves of the workgroup half a tile apart.
// merge_kernel      the exact log-sum-exp merge of partial triples, optionally normalising (finalize).
//
// Matrix-core layout (v_mfma_f32_32x32x16_{f16,bf16}; wave64; lane = 32*hi + l32):
//   A operand: lane holds A[row l32][k = 8*hi .. 8*hi+7]
//   B operand: lane holds B[k = 8*hi .. 8*hi+7][col l32]
//   C/D:       lane holds C[row = 8*(r/4) + 4*hi + r%4][col l32], r = 0..15
// Scores are computed transposed, S^T = K Q^T (A = 32 keys from LDS, B = 32 query rows kept in
// registers), so each lane owns one query column and 16 of its keys: the row max needs one exchange
// with lane ^ 32, the row sum stays per lane until the end, and the fp32 scores, once turned into
// probabilities and rounded to fp16/bf16, are already the B operand of O^T = V^T P^T.  That product
// contracts over keys in the order the score accumulator holds them, so V must reach the matrix
// cores as V^T[d][key slot] with each group of 16 keys permuted to match: fwd_kernel writes it into
// LDS that way, fwd_dma_kernel assembles it from row-major tiles with transpose loads.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <math.h>
#include <mutex>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "cqsa_internal.h"

namespace cqsa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.44269504088896340736f;

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mfma32<ET_F16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
}

template <>
__device__ __forceinline__ f32x16 mfma32<ET_BF16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// Eight fp32 probabilities -> eight fp16/bf16 (round to nearest even), packed as an MFMA operand.
template <int DT>
__device__ __forceinline__ u32x4 pack8(f32x8 x);

template <>
__device__ __forceinline__ u32x4 pack8<ET_F16>(f32x8 x) {
    return __builtin_bit_cast(u32x4, __builtin_convertvector(x, f16x8));
}

template <>
__device__ __forceinline__ u32x4 pack8<ET_BF16>(f32x8 x) {
    return __builtin_bit_cast(u32x4, __builtin_convertvector(x, bf16x8));
}

__device__ __forceinline__ void store4(void* base, int64_t off, int dt, f32x4 v) {
    if (dt == ET_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(base) + off) = v;
    } else if (dt == ET_F16) {
        *reinterpret_cast<f16x4*>(static_cast<_Float16*>(base) + off) = __builtin_convertvector(v, f16x4);
    } else {
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(base) + off) = __builtin_convertvector(v, bf16x4);
    }
}

// Blocks are dispatched round-robin over the 8 XCDs (block i -> XCD i % 8).  Renumber them so
// that each XCD receives a contiguous range of work items: items that share a K/V head then share
// that XCD's L2.  A bijection on [0, G) for any G.
__device__ __forceinline__ int xcd_remap(int bid, int G) {
    const int q = G >> 3, r = G & 7;
    const int xcd = bid & 7, slot = bid >> 3;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
}

// Position of key offset o (0..15) inside its 16-key group of the V^T tile.  Score accumulator
// register 8u+s of a lane in half hi holds key 16u + 8*(s/4) + 4*hi + s%4 of the 32-key block; the
// PV product's k index 8*hi + s must address that key, so key offset o is stored at slot
// 8*((o/4)%2) + o%4 + 4*(o/8).  The map swaps the middle two groups of four and is its own inverse;
// keys 2p and 2p+1 stay adjacent.
__device__ __forceinline__ int vslot(int j) {
    const int o = j & 15;
    return (j & ~15) + (((o >> 2) & 1) << 3) + (o & 3) + ((o >> 3) << 2);
}

// Row maximum of a lane's NKB x 16 score registers with 8 independent partial chains, so the
// reduction is not one long dependency chain (two waves per SIMD cannot hide its latency).
template <int NKB>
__device__ __forceinline__ float lane_max(const f32x16 (&s)[NKB]) {
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m[(kb * 16 + r) & 7] = fmaxf(m[(kb * 16 + r) & 7], s[kb][r]);
    return fmaxf(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3])), fmaxf(fmaxf(m[4], m[5]), fmaxf(m[6], m[7])));
}

constexpr float kLazyBound = 256.f;

// Whether the predicate holds in some lane of the wave: the compare's lane mask tested on the scalar
// unit (no VALU lane-count work).
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// max(x[lane], x[lane ^ 32]) in every lane: v_permlane32_swap leaves the pair {x[lane], x[lane ^ 32]}
// in its two results (one VALU instruction, no LDS round trip).
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Key masking of one tile's transposed scores: register r of block kb holds key offset
// kb * 32 + (r & 3) + 4 * hi + 8 * (r >> 2); offsets at or past lim become -inf.  The lane's part
// 4 * hi is taken out of lim once, so every compare is against a constant.
template <int NKB>
__device__ __forceinline__ void mask_keys(f32x16 (&s)[NKB], int lim, int hi) {
    const int lh = lim - 4 * hi;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (kb * 32 + (r & 3) + 8 * (r >> 2) >= lh) s[kb][r] = -INFINITY;
}

// fp16/bf16 operand -> the eight fp32 values it holds (exact).
template <int DT>
__device__ __forceinline__ f32x8 unpack8(u32x4 u);

template <>
__device__ __forceinline__ f32x8 unpack8<ET_F16>(u32x4 u) {
    return __builtin_convertvector(__builtin_bit_cast(f16x8, u), f32x8);
}

template <>
__device__ __forceinline__ f32x8 unpack8<ET_BF16>(u32x4 u) {
    return __builtin_convertvector(__builtin_bit_cast(bf16x8, u), f32x8);
}

// Fast half of the online-softmax step: p = 2^(s c - m) with the running shift m unchanged, rounded
// into the PV operand pf; returns the lane's sum of the fp32 p (4 partial chains).  With SPLIT, plo
// receives the rounding residual p - pf, rounded again: pf + plo carries p to about twice the
// operand precision (the hi / lo split of P for the PV product).
template <int NKB, int DT, bool SPLIT>
__device__ __forceinline__ float softmax_fast(const f32x16 (&s)[NKB], u32x4 (&pf)[2 * NKB], u32x4 (&plo)[2 * NKB],
                                              float m, float c) {
    // One 32-key block (the pipelined kernel): the four partial sums start from the first four
    // probabilities rather than from 0, since the compiler keeps 0 + p as an add (signed zeros); for
    // p >= 0 (or NaN) the sums are the same.  Measured 0.8% faster at D=64; with two blocks (D=128)
    // the same change measured 1% slower, so there the sums start from 0.
    float acc[4];
    if constexpr (NKB > 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < 2 * NKB; ++t) {
        const int kb = t >> 1, u = t & 1;
        f32x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * u + e], c, -m));
            x[e] = p;
            if (NKB == 1 && t == 0 && e < 4)
                acc[e] = p;
            else
                acc[e & 3] += p;
        }
        pf[t] = pack8<DT>(x);
        if constexpr (SPLIT) plo[t] = pack8<DT>(x - unpack8<DT>(pf[t]));
    }
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Exact half, taken by the whole wave when some lane's fast sum is not <= 2^8: the tile's row maximum
// (exchanged with lane ^ 32) becomes the new shift, p and its sum rs are recomputed, and l and O
// (both accumulator chains with SPLIT) are rescaled by 2^(m_old - m_new) (0 when m_old = -inf; a row
// with no visible key so far keeps m = -inf and gets p = 0, with no (-inf) - (-inf) ever kept).
template <int NKB, int NDB, int DT, bool SPLIT, bool LEAN = false>
__device__ __forceinline__ void softmax_exact(const f32x16 (&s)[NKB], u32x4 (&pf)[2 * NKB], u32x4 (&plo)[2 * NKB],
                                              float& m, float& l, f32x16 (&o)[NDB], f32x16 (&olo)[NDB], float c,
                                              float& rs) {
    const float mx = max_halves(lane_max<NKB>(s));
    const float mnew = fmaxf(m, mx * c);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m - muse);   // m = -inf gives 0
    rs = softmax_fast<NKB, DT, SPLIT>(s, pf, plo, muse, c);
    l *= alpha;
    if (LEAN ? wave_any(alpha != 1.f) : __any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            o[db] *= alpha;
            if constexpr (SPLIT) olo[db] *= alpha;
        }
    }
    m = mnew;
}

// Online softmax of one key tile for one 32-row query block (lane = one row, NKB x 16 of its keys).
// The running shift m (base 2) is kept while no probability of the tile exceeds 2^8: then
// p = 2^(s c - m) needs no max at all.  The exact result does not depend on which m is used, only
// on using the same m for p, l and O; the bound keeps p within fp16 range and its rounding
// relative.  When some lane's partial sum exceeds 2^8 (which also catches the first tile, where
// m = -inf, and any overflow), the wave takes the exact path.  Probabilities are rounded to fp16/bf16
// into the PV operand pf (plus the residual plo with SPLIT); the row sum l accumulates the fp32
// probabilities.
template <int NKB, int NDB, int DT, bool SPLIT, bool LEAN = false>
__device__ __forceinline__ void softmax_tile(const f32x16 (&s)[NKB], u32x4 (&pf)[2 * NKB], u32x4 (&plo)[2 * NKB],
                                             float& m, float& l, f32x16 (&o)[NDB], f32x16 (&olo)[NDB], float c) {
    float rs = softmax_fast<NKB, DT, SPLIT>(s, pf, plo, m, c);
    if (LEAN ? wave_any(!(rs <= kLazyBound)) : __any(!(rs <= kLazyBound)))
        softmax_exact<NKB, NDB, DT, SPLIT, LEAN>(s, pf, plo, m, l, o, olo, c, rs);
    l += rs;
}

template <int NKB, int NDB, int DT>
__device__ __forceinline__ void softmax_tile(const f32x16 (&s)[NKB], u32x4 (&pf)[2 * NKB], float& m, float& l,
                                             f32x16 (&o)[NDB], float c) {
    u32x4 unused_lo[2 * NKB];
    softmax_tile<NKB, NDB, DT, false>(s, pf, unused_lo, m, l, o, o, c);
}

// Transposed scores of one key tile, S^T = K Q^T: NKB blocks of 32 keys, each accumulated over the
// NDK 16-dim steps of the head.  The NKB accumulation chains alternate, so no MFMA waits on the one
// before it.
template <int D, int NKB, int NDK, int DT>
__device__ __forceinline__ void scores(const uint16_t* st, const int (&kread)[NDK], const u32x4 (&qf)[NDK],
                                       f32x16 (&sacc)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int t = 0; t < NDK; ++t)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            sacc[kb] = mfma32<DT>(*reinterpret_cast<const u32x4*>(st + kread[t] + kb * 32 * D), qf[t], sacc[kb]);
}

// PV product of the 16-key group t of the tile in stage st: O^T += V^T P^T for every 32-dim block.
// The V^T operand comes from the row-major V tile by two transposing reads whose lane addresses
// pick the key order of the packed probabilities (vslot).
template <int D, int NDB, int DT, bool SPLIT>
__device__ __forceinline__ void pv_group(const uint16_t* st, const int (&vread)[NDB], int t, u32x4 pf, u32x4 plo,
                                         f32x16 (&o)[NDB], f32x16 (&olo)[NDB]) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(st + vread[db] + (16 * t) * D));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(st + vread[db] + (16 * t + 8) * D));
        u32x4 vf;
        vf[0] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 0, 1));
        vf[1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 2, 3));
        vf[2] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 0, 1));
        vf[3] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 2, 3));
        o[db] = mfma32<DT>(vf, pf, o[db]);
        if constexpr (SPLIT) olo[db] = mfma32<DT>(vf, plo, olo[db]);
    }
}

// Online softmax and PV products of one key tile (scores s: NKB blocks of 32 keys).  Without PIPE
// the softmax of the whole tile (and its lazy-shift check) runs first, then every PV product.  With
// PIPE the softmax runs per 32-key block and the block's PV products are issued before the softmax
// of the next block, so inside one wave the matrix core works on block kb while the VALU computes
// block kb + 1.  Each accumulator still sums the key groups in ascending order; only the points at
// which the shift may move differ (any shift gives the same exact result).
template <int D, int NKB, int NDB, int DT, bool SPLIT, bool PIPE, bool LEAN = false>
__device__ __forceinline__ void softmax_pv(const f32x16 (&s)[NKB], const uint16_t* st, const int (&vread)[NDB],
                                           float& m, float& l, f32x16 (&o)[NDB], f32x16 (&olo)[NDB], float c) {
    if constexpr (PIPE) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            u32x4 pf[2], plo[2];
            softmax_tile<1, NDB, DT, SPLIT, LEAN>(reinterpret_cast<const f32x16(&)[1]>(s[kb]), pf, plo, m, l, o, olo, c);
            pv_group<D, NDB, DT, SPLIT>(st, vread, 2 * kb, pf[0], plo[0], o, olo);
            pv_group<D, NDB, DT, SPLIT>(st, vread, 2 * kb + 1, pf[1], plo[1], o, olo);
        }
    } else {
        u32x4 pf[2 * NKB], plo[2 * NKB];
        softmax_tile<NKB, NDB, DT, SPLIT, LEAN>(s, pf, plo, m, l, o, olo, c);
#pragma unroll
        for (int t = 0; t < 2 * NKB; ++t) pv_group<D, NDB, DT, SPLIT>(st, vread, t, pf[t], plo[t], o, olo);
    }
}

// Buffer resource word 3 for raw (untyped) buffer loads on gfx9-family parts: 32-bit data format,
// no swizzle.  Loads at or past num_records bytes return zero.
constexpr int kRsrcWord3 = 0x00020000;

// A buffer resource covering rows [j0, j0 + nvalid) of a K or V view with row stride sn (elements):
// rows at or past nvalid read as zero, so the ragged end of a key range needs no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base, int64_t sn, int64_t j0,
                                                            int64_t nvalid, int D) {
    const uint16_t* p = base + j0 * sn;
    const uint32_t bytes = nvalid > 0 ? (uint32_t)((nvalid - 1) * sn * 2 + (int64_t)D * 2) : 0u;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), (short)0, (int)bytes, kRsrcWord3);
}

// One wave's share of the DMA of one K or V tile: rows [j0, j0 + nvalid) of the view at base (row
// stride sn) into LDS at st, 1 KiB per instruction, lane byte offsets off (swizzle included).  Rows at
// or past nvalid read as zero.  Compiled in the device pass only (the host pass cannot type the LDS-DMA builtin, and a failure there
// silently drops the kernel's host launch stub).
template <int NW, int BPW, int D>
__device__ __forceinline__ void dma_rows(uint16_t* st, const uint16_t* base, int64_t sn, int64_t j0, int64_t nvalid,
                                         const int (&off)[BPW], int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t r = rows_rsrc(base, sn, j0, nvalid, D);
#pragma unroll
    for (int i = 0; i < BPW; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(st + (wave + i * NW) * 512),
                                                 16, off[i], 0, 0, 0);
#endif
}

// The same DMA in the form the lean forward loop uses: rows [0, nvalid) of the view starting at row0
// (row stride sn_bytes), with the wave index a scalar, so that the LDS destinations, the row count and
// the resource are all formed on the scalar unit.  Device pass only, like dma_rows.
template <int NW, int BPW, int D>
__device__ __forceinline__ void dma_rows_s(uint16_t* st, const uint16_t* row0, int sn_bytes, int nvalid,
                                           const int (&off)[BPW], int wave_s) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int bytes = nvalid > 0 ? (nvalid - 1) * sn_bytes + D * 2 : 0;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(row0), (short)0, bytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < BPW; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(st + (wave_s + i * NW) * 512), 16, off[i], 0, 0, 0);
#endif
}

// The row statistics of a query tile into LDS by buffer-load DMA, rearranged on the way: HBM holds
// (lse2, -Delta) pairs per row, LDS receives the tile's lse2 values and then its -Delta values, so that
// the 4 rows of a score register group load as one f32x4 of each.  Lane l of instruction i writes LDS
// word 64 i + l from the byte offset off[i] (pair word 2 j for lse2 word j, 2 j + 1 for -Delta word j);
// rows at or past nrows read as zero.  Device pass only, like dma_rows.
template <int NSI>
__device__ __forceinline__ void dma_stats(float* st, const float* base, int nrows, const int (&off)[NSI]) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, nrows > 0 ? nrows * 8 : 0, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < NSI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(st + 64 * i), 4, off[i],
                                                 0, 0, 0);
#endif
}

// Epilogue shared by the forward kernels: the lane pair (l32, l32 + 32) holds one query row's
// unnormalised O^T column (NDB x 16 dims each), its base-2 shift m and half of its sum l.
//   FWD_FINAL:   O / l in the output dtype, lse = (m + log2 l) ln 2 (natural log of the scaled logits)
//   FWD_PARTIAL: the raw triple (O, m ln 2, l) into the fp32 accumulator slot of this split
//   FWD_ACCUM:   the exact log-sum-exp fold of the triple into the accumulator slot.
template <int NDB>
__device__ __forceinline__ void fwd_epilogue(const FwdArgs& a, const f32x16 (&oacc)[NDB], float mrun, float lrun, int b,
                                             int hq, int split, int64_t row, bool valid, int hi) {
    constexpr int D = NDB * 32;
    const float ltot = lrun + __shfl_xor(lrun, 32);
    if (!valid) return;
    const float mnat = ltot > 0.f ? mrun * kLn2 : -INFINITY;
    if (a.mode == FWD_FINAL) {
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        const int64_t ob = (int64_t)b * a.o_sb + (int64_t)hq * a.o_sh + row * a.o_sn;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 x = {oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
                store4(a.out, ob + db * 32 + 8 * g + 4 * hi, a.out_dtype, x * inv);
            }
        if (a.lse && hi == 0)
            a.lse[(int64_t)b * a.l_sb + (int64_t)hq * a.l_sh + row] =
                ltot > 0.f ? (mrun + __log2f(ltot)) * kLn2 : -INFINITY;
        return;
    }
    const int64_t ridx = (((int64_t)split * a.B + b) * a.Hq + hq) * a.acc_rows + row;
    float* op = a.acc_o + ridx * D;
    float* mlp = a.acc_ml + ridx * 2;
    if (a.mode == FWD_PARTIAL) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 x = {oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
                *reinterpret_cast<f32x4*>(op + db * 32 + 8 * g + 4 * hi) = x;
            }
        if (hi == 0) {
            mlp[0] = mnat;
            mlp[1] = ltot;
        }
        return;
    }
    const float ma = mlp[0], la = mlp[1];
    const float mm = fmaxf(ma, mnat);
    const float wa = ma == -INFINITY ? 0.f : exp2f((ma - mm) * kLog2e);
    const float wb = mnat == -INFINITY ? 0.f : exp2f((mnat - mm) * kLog2e);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float* dst = op + db * 32 + 8 * g + 4 * hi;
            const f32x4 old = *reinterpret_cast<const f32x4*>(dst);
            f32x4 x = {oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
            *reinterpret_cast<f32x4*>(dst) = old * wa + x * wb;
        }
    if (hi == 0) {
        mlp[0] = mm;
        mlp[1] = wa * la + wb * ltot;
    }
}

// D: head dim; DT: fp16/bf16; QB: 32-row query blocks per wave; NW: waves per workgroup;
// KT: keys per LDS tile.
template <int D, int DT, int QB, int NW, int KT>
__global__ void __launch_bounds__(NW * 64) fwd_kernel(const FwdArgs a) {
    constexpr int NT = NW * 64;
    constexpr int QW = 32 * QB;                            // query rows per wave
    constexpr int BM = NW * QW;                            // query rows per workgroup
    constexpr int KS = D + 8;                              // K tile row stride (elements): 16 B pad
    constexpr int VS = KT + 8;                             // V^T tile row stride (elements): 16 B pad
    constexpr int KTILE = KT * KS;
    constexpr int STAGE = KTILE + D * VS;
    constexpr int KITEMS = KT * (D / 8);                   // 16-byte K pieces per tile
    constexpr int VITEMS = (KT / 2) * (D / 8);             // (key pair x 8 dims) V pieces per tile
    constexpr int KCH = (KITEMS + NT - 1) / NT;
    constexpr int VCH = (VITEMS + NT - 1) / NT;
    constexpr int NKB = KT / 32;                           // 32-key score blocks per tile
    constexpr int NPK = KT / 16;                           // 16-key steps of the PV product
    constexpr int NDB = D / 32;
    constexpr int NDK = D / 16;

    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    // ---- which work item: (b, kv head, split, head in group, query tile), longest tiles first
    int w = xcd_remap(blockIdx.x, gridDim.x);
    const int qt_idx = w % a.n_qt;
    w /= a.n_qt;
    const int gi = w % a.group;
    w /= a.group;
    const int split = w % a.n_splits;
    w /= a.n_splits;
    const int hkv = w % a.Hkv;
    const int b = w / a.Hkv;
    const int hq = hkv * a.group + gi;
    const int qt = a.n_qt - 1 - qt_idx;

    const int64_t i0 = a.r0 + (int64_t)qt * BM;
    const int64_t i_end = min(i0 + (int64_t)BM, a.r1);
    const int64_t iw0 = i0 + (int64_t)wave * QW;
    const int64_t iw_end = min(iw0 + (int64_t)QW, i_end);

    const int64_t klo = a.k_lo + (int64_t)split * a.split_len;
    int64_t khi = min(a.k_hi, klo + a.split_len);
    if (a.causal) khi = min(khi, i_end + a.causal_delta);  // the last row sees keys <= i_end - 1 + delta
    const int ntiles = khi > klo ? (int)((khi - klo + KT - 1) / KT) : 0;

    const uint16_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh;
    const uint16_t* kp = a.k + (int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh;
    const uint16_t* vp = a.v + (int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh;
    const int64_t k_sn = a.k_sn, v_sn = a.v_sn;

    // ---- Q fragments, the B operand of S^T = K Q^T
    u32x4 qf[QB][NDK];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int64_t row = iw0 + qb * 32 + l32;
        const bool ok = row < i_end;
        const uint16_t* p = qp + (ok ? row : 0) * a.q_sn + 8 * hi;
#pragma unroll
        for (int t = 0; t < NDK; ++t) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(p + 16 * t);
            qf[qb][t] = ok ? x : u32x4{0u, 0u, 0u, 0u};
        }
    }

    f32x16 oacc[QB][NDB];
    float mrun[QB], lrun[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        mrun[qb] = -INFINITY;
        lrun[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[qb][db] = f32x16{};
    }

    // ---- tile staging: global -> registers (next tile) -> LDS (double buffered)
    u32x4 kreg[KCH];
    u32x4 vreg[VCH][2];
    auto load_tile = [&](int64_t j0) {
        const int64_t nvalid = min(khi - j0, (int64_t)KT);
        const __amdgpu_buffer_rsrc_t kr = rows_rsrc(kp, k_sn, j0, nvalid, D);
        const __amdgpu_buffer_rsrc_t vr = rows_rsrc(vp, v_sn, j0, nvalid, D);
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int idx = tid + c * NT;
            if (KITEMS % NT == 0 || idx < KITEMS) {
                const int row = idx / (D / 8), col8 = idx % (D / 8);
                kreg[c] = __builtin_amdgcn_raw_buffer_load_b128(kr, (int)((row * k_sn + col8 * 8) * 2), 0, 0);
            }
        }
#pragma unroll
        for (int c = 0; c < VCH; ++c) {
            const int idx = tid + c * NT;
            if (VITEMS % NT == 0 || idx < VITEMS) {
                const int pr = idx % (KT / 2), col8 = idx / (KT / 2);
                const int off = (int)((2 * pr * v_sn + col8 * 8) * 2);
                vreg[c][0] = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0);
                vreg[c][1] = __builtin_amdgcn_raw_buffer_load_b128(vr, off + (int)(v_sn * 2), 0, 0);
            }
        }
    };
    auto store_tile = [&](int s) {
        uint16_t* ks = lds + s * STAGE;
        uint16_t* vs = ks + KTILE;
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int idx = tid + c * NT;
            if (KITEMS % NT == 0 || idx < KITEMS) {
                const int row = idx / (D / 8), col8 = idx % (D / 8);
                *reinterpret_cast<u32x4*>(ks + row * KS + col8 * 8) = kreg[c];
            }
        }
#pragma unroll
        for (int c = 0; c < VCH; ++c) {
            const int idx = tid + c * NT;
            if (VITEMS % NT == 0 || idx < VITEMS) {
                const int pr = idx % (KT / 2), col8 = idx / (KT / 2);
                const int slot = vslot(2 * pr);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t w0 = vreg[c][0][e >> 1], w1 = vreg[c][1][e >> 1];
                    const uint32_t word =
                        (e & 1) ? ((w0 >> 16) | (w1 & 0xFFFF0000u)) : ((w0 & 0xFFFFu) | (w1 << 16));
                    *reinterpret_cast<uint32_t*>(vs + (col8 * 8 + e) * VS + slot) = word;
                }
            }
        }
    };

    if (ntiles > 0) {
        load_tile(klo);
        store_tile(0);
    }
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int s = it & 1;
        const int64_t j0 = klo + (int64_t)it * KT;
        if (it + 1 < ntiles) load_tile(j0 + KT);

        const bool active = iw0 < i_end && (!a.causal || j0 <= iw_end - 1 + a.causal_delta);
        if (active) {
            const uint16_t* ks = lds + s * STAGE;
            const uint16_t* vs = ks + KTILE;

            // S^T for KT keys x QW queries
            f32x16 sacc[NKB][QB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = f32x16{};
#pragma unroll
            for (int t = 0; t < NDK; ++t) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const u32x4 af = *reinterpret_cast<const u32x4*>(ks + (kb * 32 + l32) * KS + 16 * t + 8 * hi);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = mfma32<DT>(af, qf[qb][t], sacc[kb][qb]);
                }
            }

            // mask keys past the range end and, on diagonal tiles, keys after the query:
            // key offset t in the tile is visible to this lane's row iff t < lim
            const bool need_mask = (j0 + KT > khi) || (a.causal && (j0 + KT - 1 > iw0 + a.causal_delta));
            if (need_mask) {
                const int lim_range = (int)min(khi - j0, (int64_t)KT);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    int lim = lim_range;
                    if (a.causal) {
                        const int64_t row = iw0 + qb * 32 + l32;
                        const int64_t c = row + a.causal_delta - j0 + 1;
                        lim = min(lim, (int)max(min(c, (int64_t)KT), (int64_t)0));
                    }
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int t = kb * 32 + (r & 3) + 4 * hi + 8 * (r >> 2);
                            if (t >= lim) sacc[kb][qb][r] = -INFINITY;
                        }
                }
            }

            // online softmax (base 2: scale * log2(e) folded into one multiply-add)
            u32x4 pf[QB][NPK];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                f32x16 sq[NKB];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) sq[kb] = sacc[kb][qb];
                softmax_tile<NKB, NDB, DT>(sq, pf[qb], mrun[qb], lrun[qb], oacc[qb], a.scale_log2);
            }

            // O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int t = 0; t < NPK; ++t) {
                    const u32x4 vf = *reinterpret_cast<const u32x4*>(vs + (db * 32 + l32) * VS + 16 * t + 8 * hi);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = mfma32<DT>(vf, pf[qb][t], oacc[qb][db]);
                }
            }
        }

        if (it + 1 < ntiles) store_tile(s ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int64_t row = iw0 + qb * 32 + l32;
        fwd_epilogue<NDB>(a, oacc[qb], mrun[qb], lrun[qb], b, hq, split, row, row < i_end, hi);
    }
}

// Ping-pong forward kernel: 8 waves, each with 32 query rows.  Waves 0-3 (group A) and 4-7 (group B)
// share the four SIMDs and run half an iteration apart: while one group issues the matrix-core work
// of its iteration (PV of the previous tile, then S of the current tile) the other group runs the
// softmax of its tile on the vector ALU, so the two units overlap instead of taking turns.
// Two barriers per iteration keep the groups in alternating phases; group B enters the loop one
// phase late and group A leaves one phase late, so both execute the same number of barriers.
// LDS holds two K tiles and two V^T tiles.  With phases numbered from 0, K_j is read in phases
// 2j (A) and 2j+1 (B) and V_j in phases 2j+2 (A) and 2j+3 (B); group A writes K_{j} during its
// softmax phase 2j-1 and group B writes V_{j} during its softmax phase 2j, each into the buffer
// whose previous tile was last read before that phase.  Global loads are issued one iteration
// before their LDS write.
template <int D, int DT, int KT>
__global__ void __launch_bounds__(512) fwd_pp_kernel(const FwdArgs a) {
    constexpr int NT = 512;
    constexpr int GT = 256;                                // threads per group
    constexpr int BM = 256;                                // query rows per workgroup
    constexpr int KS = D + 8;
    constexpr int VS = KT + 8;
    constexpr int KTILE = KT * KS;
    constexpr int VTILE = D * VS;
    constexpr int KITEMS = KT * (D / 8);
    constexpr int VITEMS = (KT / 2) * (D / 8);
    constexpr int KCH = KITEMS / GT;
    constexpr int VCH = VITEMS / GT;
    constexpr int NREG = KCH > 2 * VCH ? KCH : 2 * VCH;
    constexpr int NKB = KT / 32;
    constexpr int NPK = KT / 16;
    constexpr int NDB = D / 32;
    constexpr int NDK = D / 16;
    static_assert(KITEMS % GT == 0 && VITEMS % GT == 0, "tile split");
    (void)NT;

    __shared__ __attribute__((aligned(16))) uint16_t kls[2 * KTILE];
    __shared__ __attribute__((aligned(16))) uint16_t vls[2 * VTILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int grp = wave >> 2;
    const int gtid = tid & (GT - 1);

    int w = xcd_remap(blockIdx.x, gridDim.x);
    const int qt_idx = w % a.n_qt;
    w /= a.n_qt;
    const int gi = w % a.group;
    w /= a.group;
    const int split = w % a.n_splits;
    w /= a.n_splits;
    const int hkv = w % a.Hkv;
    const int b = w / a.Hkv;
    const int hq = hkv * a.group + gi;
    const int qt = a.n_qt - 1 - qt_idx;

    const int64_t i0 = a.r0 + (int64_t)qt * BM;
    const int64_t i_end = min(i0 + (int64_t)BM, a.r1);
    const int64_t iw0 = i0 + (int64_t)wave * 32;
    const int64_t iw_end = min(iw0 + 32, i_end);

    const int64_t klo = a.k_lo + (int64_t)split * a.split_len;
    int64_t khi = min(a.k_hi, klo + a.split_len);
    if (a.causal) khi = min(khi, i_end + a.causal_delta);
    const int ntiles = khi > klo ? (int)((khi - klo + KT - 1) / KT) : 0;

    const uint16_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh;
    const uint16_t* kp = a.k + (int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh;
    const uint16_t* vp = a.v + (int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh;
    const int64_t k_sn = a.k_sn, v_sn = a.v_sn;

    u32x4 qf[NDK];
    {
        const int64_t row = iw0 + l32;
        const bool ok = row < i_end;
        const uint16_t* p = qp + (ok ? row : 0) * a.q_sn + 8 * hi;
#pragma unroll
        for (int t = 0; t < NDK; ++t) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(p + 16 * t);
            qf[t] = ok ? x : u32x4{0u, 0u, 0u, 0u};
        }
    }

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    float mrun = -INFINITY, lrun = 0.f;

    // group A stages K tiles, group B stages V tiles, through the same registers
    u32x4 sreg[NREG];
    auto issue_k = [&](int j) {
        if (j >= ntiles) return;
        const int64_t j0 = klo + (int64_t)j * KT;
        const __amdgpu_buffer_rsrc_t kr = rows_rsrc(kp, k_sn, j0, min(khi - j0, (int64_t)KT), D);
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int idx = gtid + c * GT;
            const int row = idx / (D / 8), col8 = idx % (D / 8);
            sreg[c] = __builtin_amdgcn_raw_buffer_load_b128(kr, (int)((row * k_sn + col8 * 8) * 2), 0, 0);
        }
    };
    auto write_k = [&](int j) {
        if (j >= ntiles) return;
        uint16_t* ks = kls + (j & 1) * KTILE;
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int idx = gtid + c * GT;
            const int row = idx / (D / 8), col8 = idx % (D / 8);
            *reinterpret_cast<u32x4*>(ks + row * KS + col8 * 8) = sreg[c];
        }
    };
    auto issue_v = [&](int j) {
        if (j >= ntiles) return;
        const int64_t j0 = klo + (int64_t)j * KT;
        const __amdgpu_buffer_rsrc_t vr = rows_rsrc(vp, v_sn, j0, min(khi - j0, (int64_t)KT), D);
#pragma unroll
        for (int c = 0; c < VCH; ++c) {
            const int idx = gtid + c * GT;
            const int pr = idx % (KT / 2), col8 = idx / (KT / 2);
            const int off = (int)((2 * pr * v_sn + col8 * 8) * 2);
            sreg[2 * c] = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0);
            sreg[2 * c + 1] = __builtin_amdgcn_raw_buffer_load_b128(vr, off + (int)(v_sn * 2), 0, 0);
        }
    };
    auto write_v = [&](int j) {
        if (j >= ntiles) return;
        uint16_t* vs = vls + (j & 1) * VTILE;
#pragma unroll
        for (int c = 0; c < VCH; ++c) {
            const int idx = gtid + c * GT;
            const int pr = idx % (KT / 2), col8 = idx / (KT / 2);
            const int slot = vslot(2 * pr);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t w0 = sreg[2 * c][e >> 1], w1 = sreg[2 * c + 1][e >> 1];
                const uint32_t word = (e & 1) ? ((w0 >> 16) | (w1 & 0xFFFF0000u)) : ((w0 & 0xFFFFu) | (w1 << 16));
                *reinterpret_cast<uint32_t*>(vs + (col8 * 8 + e) * VS + slot) = word;
            }
        }
    };

    // prologue: tile 0 into buffer 0, and tile 1 in flight in registers
    if (grp == 0) {
        issue_k(0);
        write_k(0);
        issue_k(1);
    } else {
        issue_v(0);
        write_v(0);
        issue_v(1);
    }
    __syncthreads();

    f32x16 sacc[NKB];
    u32x4 pf[NPK];
    bool pv_pending = false;
    if (grp == 1) __syncthreads();  // group B runs one phase behind
    for (int it = 0; it <= ntiles; ++it) {
        const int64_t j0 = klo + (int64_t)it * KT;
        const bool active = it < ntiles && iw0 < i_end && (!a.causal || j0 <= iw_end - 1 + a.causal_delta);
        // ---- matrix-core phase: PV of the previous tile, then S of this tile
        if (pv_pending) {
            const uint16_t* vs = vls + ((it - 1) & 1) * VTILE;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int t = 0; t < NPK; ++t) {
                    const u32x4 vf = *reinterpret_cast<const u32x4*>(vs + (db * 32 + l32) * VS + 16 * t + 8 * hi);
                    oacc[db] = mfma32<DT>(vf, pf[t], oacc[db]);
                }
        }
        if (active) {
            const uint16_t* ks = kls + (it & 1) * KTILE;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
            for (int t = 0; t < NDK; ++t)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const u32x4 af = *reinterpret_cast<const u32x4*>(ks + (kb * 32 + l32) * KS + 16 * t + 8 * hi);
                    sacc[kb] = mfma32<DT>(af, qf[t], sacc[kb]);
                }
        }
        __syncthreads();
        // ---- vector phase: softmax of this tile, then stage a later tile
        pv_pending = active;
        if (active) {
            const bool need_mask = (j0 + KT > khi) || (a.causal && (j0 + KT - 1 > iw0 + a.causal_delta));
            if (need_mask) {
                int lim = (int)min(khi - j0, (int64_t)KT);
                if (a.causal) {
                    const int64_t c = iw0 + l32 + a.causal_delta - j0 + 1;
                    lim = min(lim, (int)max(min(c, (int64_t)KT), (int64_t)0));
                }
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int t = kb * 32 + (r & 3) + 4 * hi + 8 * (r >> 2);
                        if (t >= lim) sacc[kb][r] = -INFINITY;
                    }
            }
            softmax_tile<NKB, NDB, DT>(sacc, pf, mrun, lrun, oacc, a.scale_log2);
        }
        if (it < ntiles) {
            if (grp == 0) {
                write_k(it + 1);
                issue_k(it + 2);
            } else {
                write_v(it + 1);
                issue_v(it + 2);
            }
        }
        __syncthreads();
    }
    if (grp == 0) __syncthreads();  // group A leaves one phase late

    const int64_t row = iw0 + l32;
    fwd_epilogue<NDB>(a, oacc, mrun, lrun, b, hq, split, row, row < i_end, hi);
}

// DMA forward kernel: 8 waves x 32 query rows, K and V tiles copied from global memory straight into
// LDS by the buffer unit (buffer_load ... lds: no registers, no vector-ALU work), one tile ahead.
// Both tiles keep the natural row-major [key][dim] layout with the 16-byte granules of each row
// permuted by an XOR with a per-row mask, which spreads the matrix-operand reads over all LDS banks:
//   K: granule g of row r sits at g ^ fk(r); fk = (r >> 1) & 7 (D = 64) or r & 15 (D = 128), so the
//      32 key rows x 16 bytes of one S operand read are conflict free.
//   V: granule g of row r sits at g ^ fv(r); fv = 4 ((r >> 1) & 1) (D = 64) or 4 (r & 3) (D = 128).
// The PV product needs V^T (each lane: 8 keys of one dim).  ds_read_b64_tr_b16 provides it from the
// row-major tile: within each 16-lane group, output lane i receives element i % 4 of the 8-byte reads
// made by source lanes i / 4 + 4 j (j = 0..3).  Source lane s therefore reads 4 consecutive dims of key
// row kbase + s / 4, and every lane ends up with 4 keys of its own dim; two such reads fill one MFMA
// operand (8 key slots), in the key order the score accumulator holds them.
template <int D>
__device__ __forceinline__ int kswz(int r) {
    return D == 64 ? ((r >> 1) & 7) : (r & 15);
}
template <int D>
__device__ __forceinline__ int vswz(int r) {
    return D == 64 ? (4 * ((r >> 1) & 1)) : (4 * (r & 3));
}

// NW waves per workgroup (32 query rows each); WPE asks the compiler for registers that leave room for
// WPE waves per SIMD (several small workgroups per CU drift out of phase, so one's softmax overlaps
// another's matrix products).
// LEAN: the per-tile bounds of the loop are scalars computed once per wave (tiles this wave computes,
// first tile it masks) and the lazy-shift test reads the compare's lane mask; the arithmetic on the
// tiles is unchanged.
template <int D, int DT, int KT, int NW, int WPE, bool SPLIT, bool PIPE, bool LEAN = false>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
fwd_dma_kernel(const FwdArgs a) {
    constexpr int BM = NW * 32;
    constexpr int TILE = KT * D;                           // elements of one K (or V) tile
    constexpr int STAGE = 2 * TILE;                        // K then V
    constexpr int GPR = D / 8;                             // 16-byte granules per row
    constexpr int RPI = 64 / GPR;                          // rows per DMA instruction (1 KiB)
    constexpr int NBLK = KT / RPI;                         // DMA instructions per tensor and tile
    constexpr int BPW = (NBLK + NW - 1) / NW;              // per wave
    constexpr int NKB = KT / 32;
    constexpr int NDB = D / 32;
    constexpr int NDK = D / 16;
    static_assert(NBLK % NW == 0, "tile split");

    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    int w = xcd_remap(blockIdx.x, gridDim.x);
    const int qt_idx = w % a.n_qt;
    w /= a.n_qt;
    const int gi = w % a.group;
    w /= a.group;
    const int split = w % a.n_splits;
    w /= a.n_splits;
    const int hkv = w % a.Hkv;
    const int b = w / a.Hkv;
    const int hq = hkv * a.group + gi;
    const int qt = a.n_qt - 1 - qt_idx;

    const int64_t i0 = a.r0 + (int64_t)qt * BM;
    const int64_t i_end = min(i0 + (int64_t)BM, a.r1);
    const int64_t iw0 = i0 + (int64_t)wave * 32;
    const int64_t iw_end = min(iw0 + 32, i_end);

    const int64_t klo = a.k_lo + (int64_t)split * a.split_len;
    int64_t khi = min(a.k_hi, klo + a.split_len);
    if (a.causal) khi = min(khi, i_end + a.causal_delta);
    const int ntiles = khi > klo ? (int)((khi - klo + KT - 1) / KT) : 0;

    const uint16_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh;
    const uint16_t* kp = a.k + (int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh;
    const uint16_t* vp = a.v + (int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh;
    const int64_t k_sn = a.k_sn, v_sn = a.v_sn;

    u32x4 qf[NDK];
    {
        const int64_t row = iw0 + l32;
        const bool ok = row < i_end;
        const uint16_t* p = qp + (ok ? row : 0) * a.q_sn + 8 * hi;
#pragma unroll
        for (int t = 0; t < NDK; ++t) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(p + 16 * t);
            qf[t] = ok ? x : u32x4{0u, 0u, 0u, 0u};
        }
    }

    // per-lane byte offsets of this wave's DMA blocks within a tile (same for every tile)
    int koff[BPW], voff[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
        const int n = wave + i * NW;
        const int r = n * RPI + lane / GPR;
        const int pg = lane % GPR;
        koff[i] = (int)((r * k_sn + ((pg ^ kswz<D>(r)) * 8)) * 2);
        voff[i] = (int)((r * v_sn + ((pg ^ vswz<D>(r)) * 8)) * 2);
    }
    // issue the DMA of key tile j into LDS stage j & 1
#define CQSA_ISSUE_TILE(j)                                                                                  \
    do {                                                                                                  \
        const int64_t j0_ = klo + (int64_t)(j) * KT;                                                      \
        const int64_t nv_ = min(khi - j0_, (int64_t)KT);                                                  \
        uint16_t* st_ = lds + ((j) & 1) * STAGE;                                                           \
        dma_rows<NW, BPW, D>(st_, kp, k_sn, j0_, nv_, koff, wave);                                         \
        dma_rows<NW, BPW, D>(st_ + TILE, vp, v_sn, j0_, nv_, voff, wave);                                  \
    } while (0)

    // per-lane LDS element offsets of the matrix-operand reads (relative to a stage)
    int kread[NDK];
#pragma unroll
    for (int t = 0; t < NDK; ++t) kread[t] = l32 * D + (((2 * t + hi) ^ kswz<D>(l32)) * 8);
    int vread[NDB];
    {
        const int src = lane & 15;
        const int row = 4 * hi + src / 4;                       // + 16 t + 8 r at use
        const int sub = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            vread[db] = TILE + row * D + (((db * 4 + sub) ^ vswz<D>(row)) * 8) + 4 * (lane & 1);
    }

    f32x16 oacc[NDB], olo[NDB];   // olo: the lo chain of the split-P product (SPLIT only)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        oacc[db] = f32x16{};
        if constexpr (SPLIT) olo[db] = f32x16{};
    }
    float mrun = -INFINITY, lrun = 0.f;

    if constexpr (LEAN) {
        // per-wave bounds, wave-uniform, taken to scalar registers once
        const int64_t span = iw_end - 1 + a.causal_delta - klo;        // last key offset of the wave's rows
        int wt = iw0 < i_end ? ntiles : 0;
        if (a.causal) wt = span < 0 ? 0 : min(wt, (int)(span / KT) + 1);
        int mf = (khi - klo) % KT != 0 ? ntiles - 1 : ntiles;           // a ragged last tile
        if (a.causal) {
            const int64_t x = iw0 + a.causal_delta - klo - KT + 1;      // tile it masks iff it KT > x
            const int64_t first = x < 0 ? 0 : x / KT + 1;
            mf = (int)min((int64_t)mf, first);
        }
        const int wtiles = __builtin_amdgcn_readfirstlane(wt);
        const int mask_from = __builtin_amdgcn_readfirstlane(mf);
        const int wave_s = __builtin_amdgcn_readfirstlane(wave);
        const int nkeys = (int)(khi - klo);                             // keys of the range (< 2^31)
        const uint16_t* k0 = kp + klo * k_sn;
        const uint16_t* v0 = vp + klo * v_sn;
        const int ksb = (int)(k_sn * 2), vsb = (int)(v_sn * 2);
        auto tile = [&](int it, int S) {
            __syncthreads();   // tile it is in LDS; every wave is done with tile it - 1
            if (it + 1 < ntiles) {
                const int rem = nkeys - (it + 1) * KT;
                const int nvn = rem < KT ? rem : KT;
                const int64_t jn = (int64_t)(it + 1) * KT;
                dma_rows_s<NW, BPW, D>(lds + (1 - S) * STAGE, k0 + jn * k_sn, ksb, nvn, koff, wave_s);
                dma_rows_s<NW, BPW, D>(lds + (1 - S) * STAGE + TILE, v0 + jn * v_sn, vsb, nvn, voff, wave_s);
            }
            if (it >= wtiles) return;
            const int64_t j0 = klo + (int64_t)it * KT;
            const uint16_t* st = lds + S * STAGE;
            f32x16 sacc[NKB];
            scores<D, NKB, NDK, DT>(st, kread, qf, sacc);
            if (it >= mask_from) {
                int lim = (int)min(khi - j0, (int64_t)KT);
                if (a.causal) {
                    const int64_t c = iw0 + l32 + a.causal_delta - j0 + 1;
                    lim = min(lim, (int)max(min(c, (int64_t)KT), (int64_t)0));
                }
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int t = kb * 32 + (r & 3) + 4 * hi + 8 * (r >> 2);
                        if (t >= lim) sacc[kb][r] = -INFINITY;
                    }
            }
            softmax_pv<D, NKB, NDB, DT, SPLIT, PIPE, true>(sacc, st, vread, mrun, lrun, oacc, olo, a.scale_log2);
        };
        if (ntiles > 0) CQSA_ISSUE_TILE(0);
        for (int it = 0; it < ntiles; ++it) tile(it, it & 1);
    } else {
        if (ntiles > 0) CQSA_ISSUE_TILE(0);
        for (int it = 0; it < ntiles; ++it) {
            __syncthreads();   // tile it is in LDS; every wave is done with tile it - 1
            if (it + 1 < ntiles) CQSA_ISSUE_TILE(it + 1);
            const int64_t j0 = klo + (int64_t)it * KT;
            const bool active = iw0 < i_end && (!a.causal || j0 <= iw_end - 1 + a.causal_delta);
            if (!active) continue;
            const uint16_t* st = lds + (it & 1) * STAGE;

            f32x16 sacc[NKB];
            scores<D, NKB, NDK, DT>(st, kread, qf, sacc);

            const bool need_mask = (j0 + KT > khi) || (a.causal && (j0 + KT - 1 > iw0 + a.causal_delta));
            if (need_mask) {
                int lim = (int)min(khi - j0, (int64_t)KT);
                if (a.causal) {
                    const int64_t c = iw0 + l32 + a.causal_delta - j0 + 1;
                    lim = min(lim, (int)max(min(c, (int64_t)KT), (int64_t)0));
                }
    #pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int t = kb * 32 + (r & 3) + 4 * hi + 8 * (r >> 2);
                        if (t >= lim) sacc[kb][r] = -INFINITY;
                    }
            }

            softmax_pv<D, NKB, NDB, DT, SPLIT, PIPE>(sacc, st, vread, mrun, lrun, oacc, olo, a.scale_log2);
        }
    }

#undef CQSA_ISSUE_TILE

    // the two chains of the split product meet in one fp32 add
    if constexpr (SPLIT) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] += olo[db];
    }
    const int64_t row = iw0 + l32;
    fwd_epilogue<NDB>(a, oacc, mrun, lrun, b, hq, split, row, row < i_end, hi);
}

// Barrier that waits only for this wave's LDS operations, not for its buffer loads, so LDS-DMA
// issued in the phase before may still be in flight (the caller proves that no wave reads the
// buffers those loads write until a later barrier that waits for them).  The memory clobber keeps
// the compiler from moving loads or stores across it.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Workgroup barrier for tile loops with two LDS stages: each wave first waits for all of its buffer loads,
// LDS DMA included, and its LDS operations, then meets the others.  A tile's DMA is split over the
// waves, so only a wait before the barrier makes every wave's rows visible to all.  (The compiler's own
// waits cannot be relied on here: the stages are separate LDS arrays, and it sees that the DMA in
// flight writes the stage not being read.)
__device__ __forceinline__ void barrier_dma() {
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) expcnt(7) lgkmcnt(0), a wait the compiler accounts for
    __syncthreads();
}

// Instruction order for NM matrix products that each take RPM LDS operand reads, issued by one wave:
// the reads of the first PD products, then one product and the reads PD products ahead, so that PD
// products' worth of reads are always in flight behind the matrix core.
template <int NM, int RPM, int PD>
__device__ __forceinline__ void mfma_read_pipeline() {
    __builtin_amdgcn_sched_group_barrier(0x100, PD * RPM, 0);
#pragma unroll
    for (int i = 0; i < NM - PD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PD, 0);
}

// Ping-pong DMA forward kernel: 8 waves of 32 query rows in two groups, A = waves 0-3 and B = waves
// 4-7, so that wave w of A and wave w of B share a SIMD.  Each group alternates a matrix phase (the
// PV products of the previous tile, then the scores of the current tile) and a vector phase (the
// online softmax of the current tile); B runs one phase behind A.  Every phase ends with a barrier, so
// in each phase one wave of every SIMD keeps the matrix core busy while the other uses the VALU,
// instead of both taking turns.
// K and V tiles reach LDS by buffer-load DMA into the two stages of the DMA kernel's layout.  Only
// group A issues it, at the end of its matrix phase 2i (after its operand reads): K(i+1) and V(i).
// The barrier ending phase 2i + 1 waits for them (vmcnt(0)); the one ending phase 2i waits for LDS
// operations only.  K(i) is read in phases 2i (A) and 2i+1 (B), V(i) in phases 2i+2 (A) and 2i+3
// (B), so each DMA writes a buffer whose last reader finished before the phase it is issued in, and
// is read only after the barrier that waited for it.
template <int D, int DT, int KT, int WPE>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(WPE)))
fwd_pp_dma_kernel(const FwdArgs a) {
    // matrix-phase order: the scores first at D=128, the PV products first at D=64 (each measured
    // about 1% faster than the other order at its head dim); three products' reads in flight
    constexpr bool SFIRST = D == 128;
    constexpr int PD = 3;
    // the softmax block by block at D=64, where the whole-tile form spills at four waves per SIMD;
    // over the whole tile at D=128
    constexpr bool PERBLOCK = D == 64;
    // D=64 holds one DMA offset per tensor and one K and one V^T read address, and forms the others
    // from them each tile (an add or an XOR): the shape runs at four waves per SIMD, where every VGPR
    // freed is one the register allocator need not spill
    constexpr bool DERIVE = D == 64;
    constexpr int NW = 8;
    constexpr int BM = NW * 32;
    constexpr int TILE = KT * D;
    constexpr int STAGE = 2 * TILE;
    constexpr int GPR = D / 8;
    constexpr int RPI = 64 / GPR;
    constexpr int NBLK = KT / RPI;                         // DMA instructions per tensor and tile
    constexpr int NA = 4;                                  // the waves of group A issue them
    constexpr int BPW = NBLK / NA;
    constexpr int NKB = KT / 32;
    constexpr int NDB = D / 32;
    constexpr int NDK = D / 16;
    static_assert(NBLK % NA == 0, "tile split");

    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    int w = xcd_remap(blockIdx.x, gridDim.x);
    const int qt_idx = w % a.n_qt;
    w /= a.n_qt;
    const int gi = w % a.group;
    w /= a.group;
    const int split = w % a.n_splits;
    w /= a.n_splits;
    const int hkv = w % a.Hkv;
    const int b = w / a.Hkv;
    const int hq = hkv * a.group + gi;
    const int qt = a.n_qt - 1 - qt_idx;

    const int64_t i0 = a.r0 + (int64_t)qt * BM;
    const int64_t i_end = min(i0 + (int64_t)BM, a.r1);
    const int64_t iw0 = i0 + (int64_t)wave * 32;
    const int64_t iw_end = min(iw0 + 32, i_end);

    const int64_t klo = a.k_lo + (int64_t)split * a.split_len;
    int64_t khi = min(a.k_hi, klo + a.split_len);
    if (a.causal) khi = min(khi, i_end + a.causal_delta);
    const int ntiles = khi > klo ? (int)((khi - klo + KT - 1) / KT) : 0;

    const uint16_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh;
    const uint16_t* kp = a.k + (int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh;
    const uint16_t* vp = a.v + (int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh;
    const int64_t k_sn = a.k_sn, v_sn = a.v_sn;

    u32x4 qf[NDK];
    {
        const int64_t row = iw0 + l32;
        const bool ok = row < i_end;
        const uint16_t* p = qp + (ok ? row : 0) * a.q_sn + 8 * hi;
#pragma unroll
        for (int t = 0; t < NDK; ++t) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(p + 16 * t);
            qf[t] = ok ? x : u32x4{0u, 0u, 0u, 0u};
        }
    }

    // DMA lane offsets for the waves of group A (the same for every tile)
    int koff[BPW], voff[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
        const int n = (wave & 3) + i * NA;
        const int r = n * RPI + lane / GPR;
        const int pg = lane % GPR;
        koff[i] = (int)((r * k_sn + ((pg ^ kswz<D>(r)) * 8)) * 2);
        voff[i] = (int)((r * v_sn + ((pg ^ vswz<D>(r)) * 8)) * 2);
    }
    int kread[NDK];
#pragma unroll
    for (int t = 0; t < NDK; ++t) kread[t] = l32 * D + (((2 * t + hi) ^ kswz<D>(l32)) * 8);
    int vread[NDB];
    {
        const int src = lane & 15;
        const int row = 4 * hi + src / 4;
        const int sub = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            vread[db] = TILE + row * D + (((db * 4 + sub) ^ vswz<D>(row)) * 8) + 4 * (lane & 1);
    }

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    float mrun = -INFINITY, lrun = 0.f;

    // per-wave bounds, wave-uniform scalars: tiles this wave computes and the first one it masks
    const int64_t span = iw_end - 1 + a.causal_delta - klo;
    int wt = iw0 < i_end ? ntiles : 0;
    if (a.causal) wt = span < 0 ? 0 : min(wt, (int)(span / KT) + 1);
    int mf = (khi - klo) % KT != 0 ? ntiles - 1 : ntiles;
    if (a.causal) {
        const int64_t x = iw0 + a.causal_delta - klo - KT + 1;
        const int64_t first = x < 0 ? 0 : x / KT + 1;
        mf = (int)min((int64_t)mf, first);
    }
    const int wtiles = __builtin_amdgcn_readfirstlane(wt);
    const int mask_from = __builtin_amdgcn_readfirstlane(mf);
    const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);
    const int wave_a = __builtin_amdgcn_readfirstlane(wave & 3);
    const int nkeys = (int)(khi - klo);
    // causal: this lane's row sees the keys klo + j for j < vis_end (32 bits, clamped to the range)
    const int vis_end = (int)max(min(iw0 + l32 + a.causal_delta - klo + 1, (int64_t)nkeys + KT), (int64_t)-KT);
    const uint16_t* k0 = kp + klo * k_sn;
    const uint16_t* v0 = vp + klo * v_sn;
    const int ksb = (int)(k_sn * 2), vsb = (int)(v_sn * 2);

    if (grp == 0 && ntiles > 0) dma_rows_s<NA, BPW, D>(lds, k0, ksb, min(nkeys, KT), koff, wave_a);
    __syncthreads();

    f32x16 sacc[NKB];
    u32x4 pf[2 * NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int t = 0; t < 2 * NKB; ++t) pf[t] = u32x4{0u, 0u, 0u, 0u};

    typedef short s16x4 __attribute__((ext_vector_type(4)));
    // matrix phase of tile i: the PV products of tile i - 1 (P is zero where this wave had no keys),
    // then the scores of tile i; with DMA (group A), the K(i + 1) and V(i) copies after the reads
    auto mphase = [&](int i, int S, bool dma) __attribute__((always_inline)) {   // S = i & 1, a constant at every call
        auto pv = [&]() __attribute__((always_inline)) {
            if (i >= 1) {
                const uint16_t* sv = lds + (S ^ 1) * STAGE;
                int vr[NDB];
                if constexpr (DERIVE) {
                    int v0r = vread[0];
                    asm volatile("" : "+v"(v0r));   // formed here each tile, not kept in registers
#pragma unroll
                    for (int db = 0; db < NDB; ++db) vr[db] = v0r ^ (32 * db);
                } else {
#pragma unroll
                    for (int db = 0; db < NDB; ++db) vr[db] = vread[db];
                }
                s16x4 vt[2 * NKB][NDB][2];
#pragma unroll
                for (int t = 0; t < 2 * NKB; ++t)
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int r = 0; r < 2; ++r)
                            vt[t][db][r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (__attribute__((address_space(3))) s16x4*)(sv + vr[db] + (16 * t + 8 * r) * D));
#pragma unroll
                for (int t = 0; t < 2 * NKB; ++t)
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        u32x4 vf;
                        vf[0] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(vt[t][db][0], vt[t][db][0], 0, 1));
                        vf[1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(vt[t][db][0], vt[t][db][0], 2, 3));
                        vf[2] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(vt[t][db][1], vt[t][db][1], 0, 1));
                        vf[3] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(vt[t][db][1], vt[t][db][1], 2, 3));
                        oacc[db] = mfma32<DT>(vf, pf[t], oacc[db]);
                    }
                mfma_read_pipeline<2 * NKB * NDB, 2, PD>();
            }
        };
        auto sc = [&]() __attribute__((always_inline)) {
            if (i < ntiles) {
                int kr[NDK];
                if constexpr (DERIVE) {
                    int k0r = kread[0];
                    asm volatile("" : "+v"(k0r));
#pragma unroll
                    for (int t = 0; t < NDK; ++t) kr[t] = k0r ^ (16 * t);
                } else {
#pragma unroll
                    for (int t = 0; t < NDK; ++t) kr[t] = kread[t];
                }
                scores<D, NKB, NDK, DT>(lds + S * STAGE, kr, qf, sacc);
                mfma_read_pipeline<NDK * NKB, 1, PD>();
            }
        };
        if constexpr (SFIRST) {
            sc();
            pv();
        } else {
            pv();
            sc();
        }
        if (dma) {
            __builtin_amdgcn_sched_barrier(0);
            int ko[BPW], vo[BPW];
            if constexpr (DERIVE) {
                int k0o = koff[0], v0o = voff[0];
                asm volatile("" : "+v"(k0o), "+v"(v0o));
#pragma unroll
                for (int j = 0; j < BPW; ++j) {
                    ko[j] = k0o + j * (NA * RPI) * ksb;   // the swizzles repeat every NA * RPI rows
                    vo[j] = v0o + j * (NA * RPI) * vsb;
                }
            } else {
#pragma unroll
                for (int j = 0; j < BPW; ++j) {
                    ko[j] = koff[j];
                    vo[j] = voff[j];
                }
            }
            if (i + 1 < ntiles) {
                const int rem = nkeys - (i + 1) * KT;
                dma_rows_s<NA, BPW, D>(lds + (S ^ 1) * STAGE, k0 + (int64_t)(i + 1) * KT * k_sn, ksb,
                                       rem < KT ? rem : KT, ko, wave_a);
            }
            if (i < ntiles) {
                const int rem = nkeys - i * KT;
                dma_rows_s<NA, BPW, D>(lds + S * STAGE + TILE, v0 + (int64_t)i * KT * v_sn, vsb,
                                       rem < KT ? rem : KT, vo, wave_a);
            }
        }
    };
    // vector phase of tile i: masks, online softmax, P into pf for the next matrix phase (zero for a
    // tile past this wave's last key)
    auto vphase = [&](int i) __attribute__((always_inline)) {
        if (i >= wtiles) {
#pragma unroll
            for (int t = 0; t < 2 * NKB; ++t) pf[t] = u32x4{0u, 0u, 0u, 0u};
            return;
        }
        if (i >= mask_from) {
            const int rem = nkeys - i * KT;
            int lim = rem < KT ? rem : KT;
            if (a.causal) lim = min(lim, max(min(vis_end - i * KT, KT), 0));
            mask_keys<NKB>(sacc, lim, hi);
        }
        if constexpr (PERBLOCK) {
            // block by block (fewer registers live); every block's P waits for the next matrix phase,
            // so when a later block moves the shift, the earlier blocks' P are formed again at the
            // final shift (l and O were rescaled by the exact path; only P is stale)
            float m_first = mrun;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                softmax_tile<1, NDB, DT, false, true>(reinterpret_cast<const f32x16(&)[1]>(sacc[kb]),
                                                      reinterpret_cast<u32x4(&)[2]>(pf[2 * kb]),
                                                      reinterpret_cast<u32x4(&)[2]>(pf[2 * kb]), mrun, lrun, oacc,
                                                      oacc, a.scale_log2);
                if (kb == 0) m_first = mrun;
            }
            if (wave_any(mrun != m_first)) {
                const float muse = mrun == -INFINITY ? 0.f : mrun;
#pragma unroll
                for (int kb = 0; kb + 1 < NKB; ++kb)
                    (void)softmax_fast<1, DT, false>(reinterpret_cast<const f32x16(&)[1]>(sacc[kb]),
                                                     reinterpret_cast<u32x4(&)[2]>(pf[2 * kb]),
                                                     reinterpret_cast<u32x4(&)[2]>(pf[2 * kb]), muse, a.scale_log2);
            }
        } else {
            // one shift for the whole tile
            softmax_tile<NKB, NDB, DT, false, true>(sacc, pf, pf, mrun, lrun, oacc, oacc, a.scale_log2);
        }
    };
    // phase 2i: A in the matrix phase of tile i, B in the vector phase of tile i - 1;
    // phase 2i + 1: A in the vector phase of tile i, B in the matrix phase of tile i.
    // One loop per group, so each keeps its accumulators in place; both pass the same barriers.  Each
    // trip covers two tiles, so the LDS stage of every operand read is a constant.
    if (grp == 0) {
        auto step = [&](int i, int S) __attribute__((always_inline)) {
            mphase(i, S, true);
            barrier_lds();
            if (i < ntiles) vphase(i);
            barrier_dma();   // the DMA issued in phase 2i is in LDS
        };
        for (int i = 0; i <= ntiles; i += 2) {
            step(i, 0);
            if (i + 1 <= ntiles) step(i + 1, 1);
        }
    } else {
        auto step = [&](int i, int S) __attribute__((always_inline)) {
            if (i >= 1) vphase(i - 1);
            barrier_lds();
            mphase(i, S, false);
            __syncthreads();   // group B issues no DMA: a plain barrier
        };
        for (int i = 0; i <= ntiles; i += 2) {
            step(i, 0);
            if (i + 1 <= ntiles) step(i + 1, 1);
        }
    }

    const int64_t row = iw0 + l32;
    fwd_epilogue<NDB>(a, oacc, mrun, lrun, b, hq, split, row, row < i_end, hi);
}

// The wave engine's kernel: the DMA kernel's tile loop walked over a list of key parts (segments).
// A workgroup takes BM rows of one query part of the table and one (b, query head); its key loop
// runs over the key parts in the part's mask in ascending order, each cut at the causal limit of the
// workgroup's last row, with one online softmax across all of them, and the epilogue folds the result
// into the accumulator rows of the part (FWD_ACCUM).  Tiles are counted across segments, so the LDS
// double buffer and the DMA of tile it + 1 run on without a break at a segment boundary.
__device__ __forceinline__ void wave_strides(int layout, int64_t n, int H, int D, int64_t sb, int64_t sh, int64_t sn,
                                             int64_t& osb, int64_t& osh, int64_t& osn) {
    if (layout == WAVE_COMPACT_HEAD) {
        osb = (int64_t)H * n * D;
        osh = n * D;
        osn = D;
    } else if (layout == WAVE_COMPACT_TOKEN) {
        osb = n * H * D;
        osh = D;
        osn = (int64_t)H * D;
    } else {
        osb = sb;
        osh = sh;
        osn = sn;
    }
}

template <int D, int DT, int KT, int NW, int WPE, bool SPLIT, bool PIPE>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
fwd_wave_kernel(const FwdArgs a, const WaveTable t) {
    constexpr int BM = NW * 32;
    constexpr int TILE = KT * D;
    constexpr int STAGE = 2 * TILE;
    constexpr int GPR = D / 8;
    constexpr int RPI = 64 / GPR;
    constexpr int NBLK = KT / RPI;
    constexpr int BPW = (NBLK + NW - 1) / NW;
    constexpr int NKB = KT / 32;
    constexpr int NDB = D / 32;
    constexpr int NDK = D / 16;
    static_assert(NBLK % NW == 0, "tile split");

    // two stages, each its own LDS array named at compile time by every read and DMA, so the next
    // tile's DMA costs no wait inside the current tile
    __shared__ __attribute__((aligned(16))) uint16_t lds0[STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t lds1[STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    // Workgroups are ordered (b, kv head, head in group, query part, query tile): every (b, head) holds
    // the same work, so the contiguous ranges the XCD remap hands each XCD stay balanced, and a
    // head's K/V stays in one XCD's L2.  Within a head the parts come longest-first.
    int w = xcd_remap(blockIdx.x, gridDim.x);
    const int r = w % t.n_tiles;
    w /= t.n_tiles;
    int item = 0;
    while (item + 1 < t.n_q && r >= t.qi[item + 1].t0) ++item;
    const WaveQ& Q = t.qi[item];
    const int qt_idx = r - Q.t0;
    const int gi = w % a.group;
    w /= a.group;
    const int hkv = w % a.Hkv;
    const int b = w / a.Hkv;
    const int hq = hkv * a.group + gi;
    const int qt = Q.n_qt - 1 - qt_idx;

    const int64_t i0 = (int64_t)qt * BM;               // rows local to the query part
    const int64_t i_end = min(i0 + (int64_t)BM, (int64_t)Q.n);
    const int64_t iw0 = i0 + (int64_t)wave * 32;
    const int64_t iw_end = min(iw0 + 32, i_end);
    const int64_t pos0 = Q.lo + a.causal_delta;        // key position of the part's row 0

    int64_t sb, sh, sn;
    wave_strides(t.q_layout, Q.n, t.H_q, D, a.q_sb, a.q_sh, a.q_sn, sb, sh, sn);
    u32x4 qf[NDK];
    {
        const uint16_t* qp = Q.q + (int64_t)b * sb + (int64_t)hq * sh;
        const int64_t row = iw0 + l32;
        const bool ok = row < i_end;
        const uint16_t* p = qp + (ok ? row : 0) * sn + 8 * hi;
#pragma unroll
        for (int u = 0; u < NDK; ++u) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(p + 16 * u);
            qf[u] = ok ? x : u32x4{0u, 0u, 0u, 0u};
        }
    }

    // keys of segment s this workgroup visits (causal: up to the position of its last row)
    auto seg_len = [&](int s) -> int {
        int64_t n = t.ki[s].n;
        if (a.causal) n = min(n, pos0 + i_end - t.ki[s].lo);
        return (int)max(n, (int64_t)0);
    };
    auto next_seg = [&](int s) -> int {   // next segment after s with keys to visit, or -1
        for (++s; s < t.n_k; ++s)
            if (((Q.kmask >> s) & 1u) && seg_len(s) > 0) return s;
        return -1;
    };

    // The row strides of K and V do not depend on a part's length in any layout, so the lane offsets
    // of the DMA are fixed for the whole loop; a segment changes only the base pointers.
    int64_t ksb, ksh, ksn, vsb, vsh, vsn;
    wave_strides(t.k_layout, 1, t.H_kv, D, a.k_sb, a.k_sh, a.k_sn, ksb, ksh, ksn);
    wave_strides(t.v_layout, 1, t.H_kv, D, a.v_sb, a.v_sh, a.v_sn, vsb, vsh, vsn);
    int koff[BPW], voff[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
        const int n = wave + i * NW;
        const int r = n * RPI + lane / GPR;
        const int pg = lane % GPR;
        koff[i] = (int)((r * ksn + ((pg ^ kswz<D>(r)) * 8)) * 2);
        voff[i] = (int)((r * vsn + ((pg ^ vswz<D>(r)) * 8)) * 2);
    }
    // the (b, kv head) rows of segment s
    auto seg_k = [&](int s) -> const uint16_t* {
        int64_t sb_, sh_, sn_;
        wave_strides(t.k_layout, t.ki[s].n, t.H_kv, D, a.k_sb, a.k_sh, a.k_sn, sb_, sh_, sn_);
        return t.ki[s].k + (int64_t)b * sb_ + (int64_t)hkv * sh_;
    };
    auto seg_v = [&](int s) -> const uint16_t* {
        int64_t sb_, sh_, sn_;
        wave_strides(t.v_layout, t.ki[s].n, t.H_kv, D, a.v_sb, a.v_sh, a.v_sn, sb_, sh_, sn_);
        return t.ki[s].v + (int64_t)b * sb_ + (int64_t)hkv * sh_;
    };

    // LDS read offsets (relative to a stage) of the matrix operands, as in the DMA kernel
    int kread[NDK];
#pragma unroll
    for (int u = 0; u < NDK; ++u) kread[u] = l32 * D + (((2 * u + hi) ^ kswz<D>(l32)) * 8);
    int vread[NDB];
    {
        const int src = lane & 15;
        const int row = 4 * hi + src / 4;
        const int sub = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            vread[db] = TILE + row * D + (((db * 4 + sub) ^ vswz<D>(row)) * 8) + 4 * (lane & 1);
    }

    f32x16 oacc[NDB], olo[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        oacc[db] = f32x16{};
        if constexpr (SPLIT) olo[db] = f32x16{};
    }
    float mrun = -INFINITY, lrun = 0.f;

    // fetch cursor (tile fj of segment fs) and compute cursor (tile cj of segment cs), each with the
    // state of its segment; the fetch cursor runs one tile ahead
    int fs = next_seg(-1);
    if (fs < 0) {
        const int64_t row = iw0 + l32;
        fwd_epilogue<NDB>(a, oacc, mrun, lrun, b, hq, 0, Q.lo + row, row < i_end, hi);
        return;
    }
    int fj0 = 0, flen = seg_len(fs);
    const uint16_t* fk = seg_k(fs);
    const uint16_t* fv = seg_v(fs);
    int cj0 = 0, clen = flen;
    int64_t cdelta = pos0 - t.ki[fs].lo;
    int cs = fs;
    dma_rows<NW, BPW, D>(lds0, fk, ksn, 0, min(flen, KT), koff, wave);
    dma_rows<NW, BPW, D>(lds0 + TILE, fv, vsn, 0, min(flen, KT), voff, wave);
    // one tile: computes from stage st, prefetches the next tile into stage nst; false once the
    // compute cursor has passed the last segment
    auto tile = [&](const uint16_t* st, uint16_t* nst) __attribute__((always_inline)) -> bool {
        barrier_dma();   // this tile is in LDS; every wave is done with the previous one
        if (fs >= 0) {
            fj0 += KT;
            if (fj0 >= flen) {
                fs = next_seg(fs);
                if (fs >= 0) {
                    fj0 = 0;
                    flen = seg_len(fs);
                    fk = seg_k(fs);
                    fv = seg_v(fs);
                }
            }
            if (fs >= 0) {
                const int nv = min(flen - fj0, KT);
                dma_rows<NW, BPW, D>(nst, fk, ksn, fj0, nv, koff, wave);
                dma_rows<NW, BPW, D>(nst + TILE, fv, vsn, fj0, nv, voff, wave);
            }
        }

        const int j0 = cj0;   // first key of the tile, local to the segment
        const bool active = iw0 < i_end && (!a.causal || j0 <= iw_end - 1 + cdelta);
        if (active) {
            f32x16 sacc[NKB];
            scores<D, NKB, NDK, DT>(st, kread, qf, sacc);
            const bool need_mask = (j0 + KT > clen) || (a.causal && (j0 + KT - 1 > iw0 + cdelta));
            if (need_mask) {
                int lim = min(clen - j0, KT);
                if (a.causal) {
                    const int64_t c = iw0 + l32 + cdelta - j0 + 1;
                    lim = min(lim, (int)max(min(c, (int64_t)KT), (int64_t)0));
                }
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int tt = kb * 32 + (r & 3) + 4 * hi + 8 * (r >> 2);
                        if (tt >= lim) sacc[kb][r] = -INFINITY;
                    }
            }
            softmax_pv<D, NKB, NDB, DT, SPLIT, PIPE>(sacc, st, vread, mrun, lrun, oacc, olo, a.scale_log2);
        }
        // advance the compute cursor
        cj0 += KT;
        if (cj0 >= clen) {
            cs = next_seg(cs);
            if (cs < 0) return false;
            cj0 = 0;
            clen = seg_len(cs);
            cdelta = pos0 - t.ki[cs].lo;
        }
        return true;
    };
    while (tile(lds0, lds1) && tile(lds1, lds0)) {
    }

    if constexpr (SPLIT) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] += olo[db];
    }
    const int64_t row = iw0 + l32;
    fwd_epilogue<NDB>(a, oacc, mrun, lrun, b, hq, 0, Q.lo + row, row < i_end, hi);
}

// =============================================================================================
// Backward.  Three launches: bwd_stats_kernel (-Delta_i = -dO_i . O_i and the base-2 lse per row),
// bwd_dq_kernel (per query tile, over key tiles: dQ^T += K^T dS^T) and bwd_dkdv_kernel (per key
// tile, over the group's query heads and query tiles: dV^T += dO^T P, dK^T += Q^T dS).  Each
// gradient element is accumulated by one wave in a fixed order: no atomics, deterministic.  The
// derivative itself: P = exp(s - lse), dP = dO V^T, dS = P (dP - Delta), dQ = scale dS K,
// dK = scale dS^T Q, dV = P^T dO.  Every staged tile is read both ways: row reads (ds_read_b128, A
// operand = rows of the tile) and transposed reads (ds_read_b64_tr_b16, A operand = the tile
// transposed, in the key-slot order of the packed B operand).  The tiles therefore use their own
// swizzle, bswz: granule g of row r sits at g ^ bswz(r).  LDS has 64 banks of 4 bytes; a row read is
// served 16 lanes (16 rows) at a time and bswz gives those 16 rows 16 distinct 16-byte bank groups; a
// transposed read is served 32 lanes (4 rows, 64 bytes each) at a time and bswz puts those 4 row
// pieces on disjoint banks.  (The forward's kswz suits only the first pattern and vswz only the
// second: with vswz a row read takes 4 times its conflict-free cycles.)

template <int D>
__device__ __forceinline__ int bswz(int r) {
    return D == 64 ? ((4 * ((r >> 1) & 1)) | ((r >> 2) & 3)) : ((4 * (r & 3)) | ((r >> 2) & 3));
}

template <int D>
__device__ __forceinline__ int rows_read(int l32, int t, int hi) {
    return l32 * D + (((2 * t + hi) ^ bswz<D>(l32)) * 8);
}

// Element offset of this lane's transposed read of dim block db, rows 8 sec .. 8 sec + 7 of a 16-row
// group (the group's offset, 16 t D, is added by the caller: bswz ignores row bits 4 and up).
template <int D>
__device__ __forceinline__ int tr_read(int lane, int db, int sec) {
    const int hi = lane >> 5;
    const int src = lane & 15;
    const int row = 8 * sec + 4 * hi + src / 4;
    const int sub = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    return row * D + (((db * 4 + sub) ^ bswz<D>(row)) * 8) + 4 * (lane & 1);
}

// Offset from the first to the second read of tr_operand.  Rows r and r + 8 (r < 8) differ in bswz
// by 2, so the granule moves by +-2 according to bit 1 of (sub ^ bswz(r)) = bit 1 of sub: the offset
// depends on the lane but not on db.
template <int D>
__device__ __forceinline__ int tr_second(int lane) {
    return 8 * D + (((lane >> 4) & 1) ? -16 : 16);
}

// The transposed operand of one 16-slot group: p = tile + tr_read(lane, db, 0) + 16 t D, p2 its
// tr_second offset.
template <int D>
__device__ __forceinline__ u32x4 tr_operand(const uint16_t* p, int p2) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p + p2));
    u32x4 x;
    x[0] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 0, 1));
    x[1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 2, 3));
    x[2] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 0, 1));
    x[3] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 2, 3));
    return x;
}

template <int DT>
__device__ __forceinline__ f32x8 load8(const void* base, int64_t off, int dt) {
    if (dt == ET_F32) {
        const float* p = static_cast<const float*>(base) + off;
        const f32x4 x = *reinterpret_cast<const f32x4*>(p), y = *reinterpret_cast<const f32x4*>(p + 4);
        return f32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    }
    const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off);
    return dt == ET_F16 ? unpack8<ET_F16>(u) : unpack8<ET_BF16>(u);
}


// A gradient store: four values at element off of base, in dtype dt; with accumulate (fp32 only)
// added to what the four elements hold.
__device__ __forceinline__ void store_grad(void* base, int64_t off, int dt, int accumulate, f32x4 v) {
    if (accumulate) {
        f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(base) + off);
        *p = *p + v;
    } else {
        store4(base, off, dt, v);
    }
}

// Rounds fp32 rows of a compact [B][H][n][D] buffer into a strided tensor (4 values per thread).
__global__ void __launch_bounds__(256) cast_kernel(const float* src, int64_t B, int64_t H, int64_t n, int64_t D,
                                                   void* dst, int dtype, int64_t sb, int64_t sh, int64_t sn) {
    const int64_t per_row = D / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= B * H * n * per_row) return;
    const int64_t d0 = (idx % per_row) * 4;
    const int64_t r = idx / per_row;             // (b H + h) n + i
    const int64_t i = r % n, bh = r / n;
    const int64_t b = bh / H, h = bh % H;
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + r * D + d0);
    store4(dst, b * sb + h * sh + i * sn + d0, dtype, v);
}

// stats[row] = (lse * log2 e, -sum_d dO O) = (lse2, -Delta); D / 8 threads per row, 8 dims each.
template <int D, int DT>
__global__ void __launch_bounds__(256) bwd_stats_kernel(const BwdArgs a) {
    constexpr int TPR = D / 8;
    constexpr int RPB = 256 / TPR;
    const int64_t total = (int64_t)a.B * a.Hq * a.Nq;
    const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int d0 = (threadIdx.x % TPR) * 8;
    float acc = 0.f;
    int64_t b = 0, h = 0, i = 0;
    if (r < total) {
        i = r % a.Nq;
        h = (r / a.Nq) % a.Hq;
        b = r / (a.Nq * a.Hq);
        const f32x8 dov = unpack8<DT>(*reinterpret_cast<const u32x4*>(a.dout + b * a.do_sb + h * a.do_sh + i * a.do_sn + d0));
        const f32x8 ov = load8<DT>(a.out, b * a.o_sb + h * a.o_sh + i * a.o_sn + d0, a.out_dtype);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(dov[e], ov[e], acc);
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (r < total && d0 == 0) {
        const float l = a.lse[b * a.l_sb + h * a.l_sh + i];
        const int64_t sr = (b * a.Hq + h) * a.stats_rows + i;
        a.stats[2 * sr] = l == -INFINITY ? INFINITY : l * kLog2e;   // no visible key: P = 0
        a.stats[2 * sr + 1] = -acc;
    }
}

// dQ for BM = 32 NW query rows of one (b, query head): the forward's tiling with dS^T in place of P^T.
template <int D, int DT, int KT, int NW, int WPE>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE))) bwd_dq_kernel(const BwdArgs a, int n_qt) {
    constexpr int BM = NW * 32;
    constexpr int TILE = KT * D;
    constexpr int STAGE = 2 * TILE;
    constexpr int GPR = D / 8, RPI = 64 / GPR, NBLK = KT / RPI, BPW = NBLK / NW;
    constexpr int NKB = KT / 32, NPK = KT / 16, NDB = D / 32, NDK = D / 16;
    static_assert(NBLK % NW == 0, "tile split");

    // two stages, each its own LDS array, named at compile time by every read and DMA (so the next
    // tile's DMA costs no wait inside the current tile)
    __shared__ __attribute__((aligned(16))) uint16_t lds0[STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t lds1[STAGE];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    int w = xcd_remap(blockIdx.x, gridDim.x);
    const int qt_idx = w % n_qt;
    w /= n_qt;
    const int hq = w % a.Hq;
    const int b = w / a.Hq;
    const int hkv = hq / a.group;
    const int qt = n_qt - 1 - qt_idx;
    const int64_t delta_c = a.causal_delta;

    const int64_t i0 = (int64_t)qt * BM;
    const int64_t i_end = min(i0 + (int64_t)BM, a.Nq);
    const int64_t iw0 = i0 + (int64_t)wave * 32;
    const int64_t iw_end = min(iw0 + 32, i_end);
    int64_t khi = a.Nk;
    if (a.causal) khi = min(khi, i_end + delta_c);
    const int ntiles = khi > 0 ? (int)((khi + KT - 1) / KT) : 0;

    const uint16_t* kp = a.k + (int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh;
    const uint16_t* vp = a.v + (int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh;

    // B operands: this lane's query row of q and of dO; its (lse2, -Delta)
    const int64_t row = iw0 + l32;
    const bool row_ok = row < i_end;
    u32x4 qf[NDK], dof[NDK];
    {
        const uint16_t* qr = a.q + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh + (row_ok ? row : 0) * a.q_sn + 8 * hi;
        const uint16_t* dr = a.dout + (int64_t)b * a.do_sb + (int64_t)hq * a.do_sh + (row_ok ? row : 0) * a.do_sn + 8 * hi;
#pragma unroll
        for (int t = 0; t < NDK; ++t) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(qr + 16 * t);
            const u32x4 y = *reinterpret_cast<const u32x4*>(dr + 16 * t);
            qf[t] = row_ok ? x : u32x4{0u, 0u, 0u, 0u};
            dof[t] = row_ok ? y : u32x4{0u, 0u, 0u, 0u};
        }
    }
    float lse2 = INFINITY, ndlt = 0.f;
    if (row_ok) {
        const float* sp = a.stats + 2 * (((int64_t)b * a.Hq + hq) * a.stats_rows + row);
        lse2 = sp[0];
        ndlt = sp[1];
    }
    f32x16 dpinit;   // the dP^T accumulators start from the row's -Delta, so dS = P dP
#pragma unroll
    for (int r = 0; r < 16; ++r) dpinit[r] = ndlt;

    int koff[BPW], voff[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
        const int r = (wave + i * NW) * RPI + lane / GPR;
        const int pg = lane % GPR;
        koff[i] = (int)((r * a.k_sn + ((pg ^ bswz<D>(r)) * 8)) * 2);
        voff[i] = (int)((r * a.v_sn + ((pg ^ bswz<D>(r)) * 8)) * 2);
    }
    int rread[NDK], tread[NDB];
#pragma unroll
    for (int t = 0; t < NDK; ++t) rread[t] = rows_read<D>(l32, t, hi);
#pragma unroll
    for (int db = 0; db < NDB; ++db) tread[db] = tr_read<D>(lane, db, 0);
    const int tsec = tr_second<D>(lane);

    f32x16 dqacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};

    // per-wave bounds, wave-uniform and taken to scalar registers once: the tiles this wave computes
    // (its last row sees keys <= iw_end - 1 + delta) and the first tile it masks (the causal diagonal,
    // or a ragged last tile); the DMA of a tile is formed on the scalar unit too
    int wt = iw0 < i_end ? ntiles : 0;
    if (a.causal) {
        const int64_t span = iw_end - 1 + delta_c;
        wt = span < 0 ? 0 : min(wt, (int)(span / KT) + 1);
    }
    int mf = khi % KT != 0 ? ntiles - 1 : ntiles;
    if (a.causal) {
        const int64_t x = iw0 + delta_c - KT + 1;                      // tile it masks iff it KT > x
        mf = (int)min((int64_t)mf, x < 0 ? (int64_t)0 : x / KT + 1);
    }
    const int wtiles = __builtin_amdgcn_readfirstlane(wt);
    const int mask_from = __builtin_amdgcn_readfirstlane(mf);
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int nkeys = (int)khi;
    const int ksb = (int)(a.k_sn * 2), vsb = (int)(a.v_sn * 2);
    auto issue = [&](int j, uint16_t* st_) __attribute__((always_inline)) {
        const int rem = nkeys - j * KT;
        const int nv = rem < KT ? rem : KT;
        dma_rows_s<NW, BPW, D>(st_, kp + (int64_t)j * KT * a.k_sn, ksb, nv, koff, wave_s);
        dma_rows_s<NW, BPW, D>(st_ + TILE, vp + (int64_t)j * KT * a.v_sn, vsb, nv, voff, wave_s);
    };

    // tile it: reads stage st, issues tile it + 1 into stage nst
    auto tile = [&](int it, const uint16_t* st, uint16_t* nst) __attribute__((always_inline)) {
        barrier_dma();
        if (it + 1 < ntiles) issue(it + 1, nst);
        const int64_t j0 = (int64_t)it * KT;
        if (it >= wtiles) return;

        f32x16 sacc[NKB], dpacc[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            sacc[kb] = f32x16{};
            dpacc[kb] = dpinit;
        }
#pragma unroll
        for (int t = 0; t < NDK; ++t)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const u32x4 kf = *reinterpret_cast<const u32x4*>(st + rread[t] + kb * 32 * D);
                const u32x4 vf = *reinterpret_cast<const u32x4*>(st + TILE + rread[t] + kb * 32 * D);
                sacc[kb] = mfma32<DT>(kf, qf[t], sacc[kb]);
                dpacc[kb] = mfma32<DT>(vf, dof[t], dpacc[kb]);
            }
        if (it >= mask_from) {
            int lim = (int)min(khi - j0, (int64_t)KT);
            if (a.causal) {
                const int64_t cl = row + delta_c - j0 + 1;
                lim = min(lim, (int)max(min(cl, (int64_t)KT), (int64_t)0));
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int t = kb * 32 + (r & 3) + 4 * hi + 8 * (r >> 2);
                    if (t >= lim) sacc[kb][r] = -INFINITY;
                }
        }
        u32x4 pf[NPK];
#pragma unroll
        for (int t = 0; t < NPK; ++t) {
            const int kb = t >> 1, u = t & 1;
            f32x8 x;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * u + e], a.scale_log2, -lse2));
                x[e] = p * dpacc[kb][8 * u + e];
            }
            pf[t] = pack8<DT>(x);
        }
#pragma unroll
        for (int t = 0; t < NPK; ++t)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                dqacc[db] = mfma32<DT>(tr_operand<D>(st + tread[db] + 16 * t * D, tsec), pf[t], dqacc[db]);
    };
    if (ntiles > 0) issue(0, lds0);
    for (int it = 0; it < ntiles; it += 2) {
        tile(it, lds0, lds1);
        if (it + 1 < ntiles) tile(it + 1, lds1, lds0);
    }

    if (!row_ok) return;
    const int64_t ob = (int64_t)b * a.dq_sb + (int64_t)hq * a.dq_sh + row * a.dq_sn;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 x = {dqacc[db][4 * g], dqacc[db][4 * g + 1], dqacc[db][4 * g + 2], dqacc[db][4 * g + 3]};
            store_grad(a.dq, ob + db * 32 + 8 * g + 4 * hi, a.grad_dtype, a.accumulate, x * a.scale);
        }
}

// dK and dV for BN = 32 NW keys of one (b, key/value head), summed over the group's query heads:
// each wave keeps 32 keys (and their values) as B operands and streams query tiles of QT rows.
// PART 0 computes both; PART 1 only dV (S -> P -> dV, no dP) and PART 2 only dK (S, dP -> dS -> dK):
// at D = 128 the two accumulators and both operand sets of PART 0 need more than the 256 VGPRs of
// two waves per SIMD, so dV and dK run as two launches that each recompute S (10 D FLOP per visible
// pair instead of 8) at twice the occupancy.
// Per tile: the dP accumulator starts from the rows' -Delta (so dS = P dP needs no subtraction); the
// operand reads of the S and dP products run three products ahead of the matrix core; a tile that
// reaches the causal diagonal or a ragged end masks by one compare pair per score against the lane's
// visible row range; the next tile's DMA addresses are running scalar pointers.
template <int D, int DT, int QT, int NW, int WPE, int PART>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE))) bwd_dkdv_kernel(const BwdArgs a, int n_kt) {
    constexpr int BN = NW * 32;
    constexpr int TILE = QT * D;
    constexpr int STAGE = 2 * TILE;                    // Q tile, then dO tile
    constexpr int GPR = D / 8, RPI = 64 / GPR, NBLK = QT / RPI, BPW = NBLK / NW;
    constexpr int NQB = QT / 32, NPQ = QT / 16, NDB = D / 32, NDK = D / 16;
    constexpr int NSI = 2 * QT / 64;                   // stats DMA instructions per tile
    static_assert(NBLK % NW == 0, "tile split");
    static_assert(2 * QT % 64 == 0, "the row statistics of a tile are whole 64-lane DMA instructions");

    // two stages, each its own LDS array (tiles, then the rows' lse2 and -Delta): every read and every
    // DMA below names its array at compile time, so the compiler can tell that the next tile's DMA does
    // not write what the current tile reads and inserts no wait for it inside the tile
    __shared__ __attribute__((aligned(16))) uint16_t lds0[STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t lds1[STAGE];
    __shared__ __attribute__((aligned(16))) float stl0[2 * QT];
    __shared__ __attribute__((aligned(16))) float stl1[2 * QT];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    int w = xcd_remap(blockIdx.x, gridDim.x);
    const int kt = w % n_kt;                          // low key tiles (most query rows) first
    w /= n_kt;
    const int hkv = w % a.Hkv;
    const int b = w / a.Hkv;
    const int64_t delta_c = a.causal_delta;

    const int64_t jw0 = (int64_t)kt * BN + (int64_t)wave * 32;
    const int64_t key = jw0 + l32;
    const bool key_ok = key < a.Nk;
    constexpr bool WANT_DV = PART != 2, WANT_DK = PART != 1;
    u32x4 kf[NDK], vf[NDK];
    {
        const uint16_t* kr = a.k + (int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh + (key_ok ? key : 0) * a.k_sn + 8 * hi;
        const uint16_t* vr = a.v + (int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh + (key_ok ? key : 0) * a.v_sn + 8 * hi;
#pragma unroll
        for (int t = 0; t < NDK; ++t) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(kr + 16 * t);
            kf[t] = key_ok ? x : u32x4{0u, 0u, 0u, 0u};
            if constexpr (WANT_DK) {
                const u32x4 y = *reinterpret_cast<const u32x4*>(vr + 16 * t);
                vf[t] = key_ok ? y : u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    // query rows that see a key of this workgroup: i >= first key - delta (causal)
    const int64_t kb0 = (int64_t)kt * BN;
    const int64_t i_start = a.causal ? max((int64_t)0, kb0 - delta_c) : 0;
    const int nqt = i_start < a.Nq ? (int)((a.Nq - i_start + QT - 1) / QT) : 0;
    const int total = nqt * a.group;

    int qoff[BPW], doff[BPW], soff[NSI];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
        const int r = (wave + i * NW) * RPI + lane / GPR;
        const int pg = lane % GPR;
        qoff[i] = (int)((r * a.q_sn + ((pg ^ bswz<D>(r)) * 8)) * 2);
        doff[i] = (int)((r * a.do_sn + ((pg ^ bswz<D>(r)) * 8)) * 2);
    }
#pragma unroll
    for (int i = 0; i < NSI; ++i) {
        const int j = 64 * i + lane;
        soff[i] = 4 * (j < QT ? 2 * j : 2 * (j - QT) + 1);
    }
    int rread[NDK], tread[NDB];
#pragma unroll
    for (int t = 0; t < NDK; ++t) rread[t] = rows_read<D>(l32, t, hi);
#pragma unroll
    for (int db = 0; db < NDB; ++db) tread[db] = tr_read<D>(lane, db, 0);
    const int tsec = tr_second<D>(lane);

    f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        dkacc[db] = f32x16{};
        dvacc[db] = f32x16{};
    }

    // Tiles run head-major over (query head th of the group, query tile tq from row i_start).  The next
    // tile's Q, dO and statistics are addressed by running scalar pointers (stepped by a tile, or reset
    // to the next head's row i_start), its row count by a running remainder; the wave index is a scalar
    // too, so the whole DMA issue stays on the scalar unit.
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const uint16_t* qh = a.q + (int64_t)b * a.q_sb + (int64_t)hkv * a.group * a.q_sh + i_start * a.q_sn;
    const uint16_t* dh = a.dout + (int64_t)b * a.do_sb + (int64_t)hkv * a.group * a.do_sh + i_start * a.do_sn;
    const float* sh = a.stats + 2 * (((int64_t)b * a.Hq + (int64_t)hkv * a.group) * a.stats_rows + i_start);
    const int rows_left = (int)(a.Nq - i_start);
    const int qsb = (int)(a.q_sn * 2), dsb = (int)(a.do_sn * 2);
    const uint16_t* qn = qh;
    const uint16_t* dn = dh;
    const float* sn = sh;
    int rem = rows_left;
    auto issue_next = [&](uint16_t* st_, float* sl_) __attribute__((always_inline)) {
        const int nv_ = rem < QT ? rem : QT;
        dma_rows_s<NW, BPW, D>(st_, qn, qsb, nv_, qoff, wave_s);
        dma_rows_s<NW, BPW, D>(st_ + TILE, dn, dsb, nv_, doff, wave_s);
        if (wave_s == NW - 1) dma_stats<NSI>(sl_, sn, nv_, soff);
    };
    // per-wave bounds on the query tile index, wave-uniform and taken to scalar registers once:
    //   the wave works on tile tq when some row of it sees some valid key of the wave (tq >= tq_first),
    //   and masks when the tile reaches the causal diagonal (tq < tq_diag), the end of the rows (the
    //   last tile of a ragged row range) or the wave's keys reach the end of the key range
    const int64_t jw = jw0;
    int64_t first = 0, diag = 0;
    if (a.causal) {
        const int64_t x = jw - delta_c - QT + 1 - i_start;      // tile tq active iff tq QT >= x
        first = x <= 0 ? 0 : (x + QT - 1) / QT;
        const int64_t y = jw + 31 - delta_c - i_start;          // tile tq masks iff tq QT < y
        diag = y <= 0 ? 0 : (y + QT - 1) / QT;
    }
    const int tq_first = __builtin_amdgcn_readfirstlane((int)min(first, (int64_t)nqt));
    const int tq_diag = __builtin_amdgcn_readfirstlane((int)min(diag, (int64_t)nqt));
    const int wave_live = __builtin_amdgcn_readfirstlane(jw < a.Nk ? 1 : 0);
    const int key_ragged = __builtin_amdgcn_readfirstlane(jw + 32 > a.Nk ? 1 : 0);
    const int row_ragged = (a.Nq - i_start) % QT != 0 ? 1 : 0;
    // the lane's key sees tile rows t >= key - delta - (i_start + tq QT) (causal), all rows when not
    // causal, none when the key does not exist; kept relative to row i_start and clamped
    const int64_t vis0 = !key_ok ? (int64_t)a.Nq : (a.causal ? max(key - delta_c - i_start, (int64_t)0) : (int64_t)0);
    const int vis_row = (int)min(vis0, (int64_t)rows_left + QT);

    int tq = 0;                             // query tile of tile it
    int nq = 0;                             // query tile of the next tile to issue
    auto advance = [&]() __attribute__((always_inline)) {
        if (++nq == nqt) {
            nq = 0;
            qh += a.q_sh;
            dh += a.do_sh;
            sh += 2 * a.stats_rows;
            qn = qh;
            dn = dh;
            sn = sh;
            rem = rows_left;
        } else {
            qn += (int64_t)QT * a.q_sn;
            dn += (int64_t)QT * a.do_sn;
            sn += 2 * QT;
            rem -= QT;
        }
    };
    // tile it: reads stage st / sl, issues tile it + 1 into stage nst / nsl
    auto tile = [&](int it, const uint16_t* st, const float* sl, uint16_t* nst, float* nsl)
                    __attribute__((always_inline)) {
        barrier_dma();
        const int cur_q = tq;
        tq = nq;
        if (it + 1 < total) {
            issue_next(nst, nsl);
            advance();
        }
        if (!wave_live || cur_q < tq_first) return;
        const bool need_mask = key_ragged || (a.causal && cur_q < tq_diag) || (row_ragged && cur_q == nqt - 1);
        // visible rows [mlo, mhi) of this tile for the lane's key, less the lane's row offset 4 hi
        const int mlo = vis_row - cur_q * QT - 4 * hi;
        const int mhi = rows_left - cur_q * QT - 4 * hi;

        u32x4 pp[NPQ], ps[NPQ];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            // register r of the lane holds query row qb 32 + 8 (r / 4) + 4 hi + r % 4 of the tile
            f32x16 sacc = f32x16{}, dpacc = f32x16{};
            if constexpr (WANT_DK) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(sl + QT + qb * 32 + 8 * g + 4 * hi);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dpacc[4 * g + e] = d4[e];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < NDK; ++t) {
                const u32x4 qa = *reinterpret_cast<const u32x4*>(st + rread[t] + qb * 32 * D);
                sacc = mfma32<DT>(qa, kf[t], sacc);
                if constexpr (WANT_DK) {
                    const u32x4 da = *reinterpret_cast<const u32x4*>(st + TILE + rread[t] + qb * 32 * D);
                    dpacc = mfma32<DT>(da, vf[t], dpacc);
                }
            }
            mfma_read_pipeline<(WANT_DK ? 2 : 1) * NDK, 1, 3>();
            f32x4 l4[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) l4[g] = *reinterpret_cast<const f32x4*>(sl + qb * 32 + 8 * g + 4 * hi);
            if (need_mask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int c = qb * 32 + 8 * (r >> 2) + (r & 3);
                    if (c < mlo || c >= mhi) sacc[r] = -INFINITY;
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                f32x8 xp, xs;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = 8 * u + e;
                    const float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], a.scale_log2, -l4[r >> 2][r & 3]));
                    xp[e] = p;
                    if constexpr (WANT_DK) xs[e] = p * dpacc[r];
                }
                if constexpr (WANT_DV) pp[2 * qb + u] = pack8<DT>(xp);
                if constexpr (WANT_DK) ps[2 * qb + u] = pack8<DT>(xs);
            }
        }
#pragma unroll
        for (int t = 0; t < NPQ; ++t)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                if constexpr (WANT_DV)
                    dvacc[db] = mfma32<DT>(tr_operand<D>(st + TILE + tread[db] + 16 * t * D, tsec), pp[t], dvacc[db]);
                if constexpr (WANT_DK)
                    dkacc[db] = mfma32<DT>(tr_operand<D>(st + tread[db] + 16 * t * D, tsec), ps[t], dkacc[db]);
            }
    };
    if (total > 0) {
        issue_next(lds0, stl0);
        advance();
    }
    for (int it = 0; it < total; it += 2) {
        tile(it, lds0, stl0, lds1, stl1);
        if (it + 1 < total) tile(it + 1, lds1, stl1, lds0, stl0);
    }

    if (!key_ok) return;
    const int64_t kbase = (int64_t)b * a.dk_sb + (int64_t)hkv * a.dk_sh + key * a.dk_sn;
    const int64_t vbase = (int64_t)b * a.dv_sb + (int64_t)hkv * a.dv_sh + key * a.dv_sn;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 x = {dkacc[db][4 * g], dkacc[db][4 * g + 1], dkacc[db][4 * g + 2], dkacc[db][4 * g + 3]};
            const f32x4 y = {dvacc[db][4 * g], dvacc[db][4 * g + 1], dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]};
            if constexpr (WANT_DK) store_grad(a.dk, kbase + db * 32 + 8 * g + 4 * hi, a.grad_dtype, a.accumulate, x * a.scale);
            if constexpr (WANT_DV) store_grad(a.dv, vbase + db * 32 + 8 * g + 4 * hi, a.grad_dtype, a.accumulate, y);
        }
}

// Log-sum-exp merge: TPR threads per row, four output dims per thread.  The threads of one row
// sit in one wave, so in-place operation (output == part 0) reads every input before it writes.
template <int D>
__global__ void __launch_bounds__(256) merge_kernel(const MergeArgs a) {
    constexpr int TPR = D / 4;
    constexpr int RPB = 256 / TPR;
    const int64_t nloc = a.i_hi - a.i_lo;
    const int64_t total = (int64_t)a.B * a.Hq * nloc;
    const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    if (r >= total) return;
    const int d0 = (threadIdx.x % TPR) * 4;
    const int64_t bh = r / nloc;
    const int64_t i = a.i_lo + r % nloc;
    const int64_t ridx = bh * a.rows_per_head + i;

    float mm = -INFINITY;
    for (int p = 0; p < a.n_parts; ++p) mm = fmaxf(mm, a.part_ml[p][2 * ridx]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
    for (int p = 0; p < a.n_parts; ++p) {
        const float mp = a.part_ml[p][2 * ridx];
        const float wgt = mp == -INFINITY ? 0.f : exp2f((mp - mm) * kLog2e);
        l += wgt * a.part_ml[p][2 * ridx + 1];
        acc += wgt * *reinterpret_cast<const f32x4*>(a.part_o[p] + ridx * D + d0);
    }
    if (a.final_out) {
        const int64_t b = bh / a.Hq, h = bh % a.Hq;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        store4(a.out, b * a.o_sb + h * a.o_sh + (i - a.i_lo) * a.o_sn + d0, a.out_dtype, acc * inv);
        if (a.lse && d0 == 0) a.lse[b * a.l_sb + h * a.l_sh + (i - a.i_lo)] = l > 0.f ? mm + logf(l) : -INFINITY;
    } else {
        *reinterpret_cast<f32x4*>(a.o_out + ridx * D + d0) = acc;
        if (d0 == 0) {
            a.ml_out[2 * ridx] = l > 0.f ? mm : -INFINITY;
            a.ml_out[2 * ridx + 1] = l;
        }
    }
}

template <int D, int DT, int KT, int NW, int WPE, bool SPLIT = false, bool PIPE = false, bool LEAN = false>
hipError_t launch_dma_t(const FwdArgs& a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.n_splits * a.B * a.Hq * a.n_qt;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_dma_kernel<D, DT, KT, NW, WPE, SPLIT, PIPE, LEAN>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                       stream, a);
    return hipGetLastError();
}

template <int D, int DT, int KT>
hipError_t launch_pp_t(const FwdArgs& a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.n_splits * a.B * a.Hq * a.n_qt;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_pp_kernel<D, DT, KT>), dim3((unsigned)blocks), dim3(512), 0, stream, a);
    return hipGetLastError();
}

template <int D, int DT, int KT, int WPE>
hipError_t launch_ppdma_t(const FwdArgs& a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.n_splits * a.B * a.Hq * a.n_qt;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_pp_dma_kernel<D, DT, KT, WPE>), dim3((unsigned)blocks), dim3(512), 0, stream, a);
    return hipGetLastError();
}

template <int D, int DT, int QB, int NW, int KT>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.n_splits * a.B * a.Hq * a.n_qt;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_kernel<D, DT, QB, NW, KT>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

// Kernel choice per head dim: kind 3 the ping-pong DMA kernel (8 waves in two groups, wpe waves per
// SIMD asked of the register allocator), kind 2 the DMA kernel (nw waves, kt keys per tile, pipe:
// softmax and PV products interleaved per 32-key block, lean: scalar tile bounds), kind 1 the
// register-staged kernel, kind 0 the register-staged ping-pong kernel.
// Entry 0 is the default: the ping-pong DMA kernel, which measured faster than every DMA-kernel shape
// at both head dims.  Entry 6 is the DMA kernel's best shape (pipelined and lean at D=64, plain at
// D=128), entries 4 and 5 its other pipelining and lean choices, entry 7 the ping-pong DMA kernel with
// 32-key tiles (level with 64-key tiles at D=64, 17% slower at D=128).  cqsa_set_test_controls selects another entry for the whole process, for
// measurement and for the tests that cover every kernel.
struct Shape {
    int kind, nw, kt, wpe, pipe, lean;
};
constexpr Shape kShapes64[] = {{3, 8, 64, 4, 0, 0}, {2, 8, 128, 2, 0, 0}, {1, 8, 128, 2, 0, 0}, {0, 8, 128, 2, 0, 0},
                               {2, 4, 64, 3, 0, 0}, {2, 4, 64, 3, 1, 0}, {2, 4, 64, 4, 1, 1}, {3, 8, 32, 4, 0, 0}};
constexpr Shape kShapes128[] = {{3, 8, 64, 2, 0, 0}, {2, 8, 32, 2, 0, 0}, {1, 8, 64, 2, 0, 0}, {0, 8, 64, 2, 0, 0},
                                {2, 8, 64, 2, 1, 0}, {2, 8, 64, 2, 0, 1}, {2, 8, 64, 2, 0, 0}, {3, 8, 32, 2, 0, 0}};
constexpr int kNumShapes = 8;

std::atomic<int> g_variant{0};

int variant() { return g_variant.load(std::memory_order_relaxed); }

// The split-P product (two PV chains) runs on the DMA kernel in one shape per head dim; pipelined at
// D=64 (measured 11% faster than 8 waves in the plain order, though it spills three VGPRs).
constexpr Shape kSplit64 = {2, 4, 64, 3, 1, 0};
constexpr Shape kSplit128 = {2, 8, 32, 2, 0, 0};

Shape shape_of(int D, int p_split) {
    if (p_split) return D == 64 ? kSplit64 : kSplit128;
    return (D == 64 ? kShapes64 : kShapes128)[variant()];
}

template <int D, int DT>
hipError_t launch_d(const FwdArgs& a, hipStream_t st) {
    if (a.p_split) {
        if constexpr (D == 64)
            return launch_dma_t<D, DT, kSplit64.kt, kSplit64.nw, kSplit64.wpe, true, (kSplit64.pipe != 0)>(a, st);
        else
            return launch_dma_t<D, DT, kSplit128.kt, kSplit128.nw, kSplit128.wpe, true, (kSplit128.pipe != 0)>(a, st);
    }
    const Shape sh = (D == 64 ? kShapes64 : kShapes128)[variant()];
    if (sh.kind == 2) {
#define CQSA_DMA_CASE(NW_, KT_, WPE_, PIPE_, LEAN_)                                                        \
    if (sh.nw == NW_ && sh.kt == KT_ && sh.wpe == WPE_ && sh.pipe == PIPE_ && sh.lean == LEAN_)          \
        return launch_dma_t<D, DT, KT_, NW_, WPE_, false, (PIPE_ != 0), (LEAN_ != 0)>(a, st);
        if constexpr (D == 64) {
            CQSA_DMA_CASE(4, 64, 3, 1, 0)
            CQSA_DMA_CASE(4, 64, 3, 0, 0)
            CQSA_DMA_CASE(8, 128, 2, 0, 0)
            CQSA_DMA_CASE(4, 64, 4, 1, 1)
        } else {
            CQSA_DMA_CASE(8, 64, 2, 0, 0)
            CQSA_DMA_CASE(8, 32, 2, 0, 0)
            CQSA_DMA_CASE(8, 64, 2, 1, 0)
            CQSA_DMA_CASE(8, 64, 2, 0, 1)
        }
#undef CQSA_DMA_CASE
        return hipErrorInvalidValue;
    }
    if (sh.kind == 3) {
        if constexpr (D == 64) {
            if (sh.kt == 64 && sh.wpe == 4) return launch_ppdma_t<D, DT, 64, 4>(a, st);
            if (sh.kt == 32 && sh.wpe == 4) return launch_ppdma_t<D, DT, 32, 4>(a, st);
        } else {
            if (sh.kt == 64) return launch_ppdma_t<D, DT, 64, 2>(a, st);
            if (sh.kt == 32) return launch_ppdma_t<D, DT, 32, 2>(a, st);
        }
        return hipErrorInvalidValue;
    }
    if (sh.kind == 0) {
        if (sh.kt == 64) return launch_pp_t<D, DT, 64>(a, st);
        if constexpr (D == 64)
            if (sh.kt == 128) return launch_pp_t<D, DT, 128>(a, st);
        return hipErrorInvalidValue;
    }
    if (sh.kt == 64) return launch_fwd_t<D, DT, 1, 8, 64>(a, st);
    if constexpr (D == 64)
        if (sh.kt == 128) return launch_fwd_t<D, DT, 1, 8, 128>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace

void set_fwd_variant(int v) { g_variant.store((v < 0 || v >= kNumShapes) ? 0 : v, std::memory_order_relaxed); }

int fwd_variant_count() { return kNumShapes; }

namespace {

// The device memory of the no-allocation entry point: one fixed array, which every device holds from
// the loading of this code object until the process ends.  In host code the name stands in for the
// array and is not a device address; host code passes kernels the address hipGetSymbolAddress gives
// for the current device (noalloc_scratch), never the name.
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

int fwd_block_m(int D, int p_split) { return shape_of(D, p_split).nw * 32; }

int fwd_wgs_per_cu(int D, int p_split) {
    const Shape sh = shape_of(D, p_split);
    return std::max(1, 4 * sh.wpe / sh.nw);   // 4 SIMDs, wpe waves each, nw waves per workgroup
}

const char* fwd_kernel_name(int D, int p_split) {
    static char names[2][kNumShapes + 1][112];
    if (D != 64 && D != 128) return "";
    const int v = p_split ? kNumShapes : variant();
    const Shape sh = shape_of(D, p_split);
    static const char* const kind[4] = {"fwd_pp_kernel", "fwd_kernel", "fwd_dma_kernel", "fwd_pp_dma_kernel"};
    char* out = names[D == 64 ? 0 : 1][v];
    snprintf(out, sizeof names[0][0], "%s waves=%d keys_per_tile=%d rows_per_wave=32%s%s%s", kind[sh.kind], sh.nw,
             sh.kt, sh.pipe ? " pipelined" : "", sh.lean ? " lean" : "", p_split ? " split_p" : "");
    return out;
}

hipError_t launch_fwd(const FwdArgs& a, int D, int dtype, hipStream_t stream) {
    if (D == 64 && dtype == ET_F16) return launch_d<64, ET_F16>(a, stream);
    if (D == 64 && dtype == ET_BF16) return launch_d<64, ET_BF16>(a, stream);
    if (D == 128 && dtype == ET_F16) return launch_d<128, ET_F16>(a, stream);
    if (D == 128 && dtype == ET_BF16) return launch_d<128, ET_BF16>(a, stream);
    return hipErrorInvalidValue;
}

namespace {

// The wave kernel runs the DMA kernel's pipelined D=64 shape and plain D=128 shape (the split-P
// shape with p_split); its loop has its own bookkeeping, so the lean flag does not apply.
constexpr Shape kWave64 = kShapes64[5];
constexpr Shape kWave128 = kShapes128[6];
static_assert(kWave64.kind == 2 && kWave128.kind == 2, "the wave kernel is the DMA kernel's loop");
static_assert(sizeof(FwdArgs) + sizeof(WaveTable) <= 4096, "the wave kernel's arguments fit the 4 KiB kernel-argument segment");

Shape wave_shape(int D, int p_split) {
    if (p_split) return D == 64 ? kSplit64 : kSplit128;
    return D == 64 ? kWave64 : kWave128;
}

template <int D, int DT>
hipError_t launch_wave_d(const FwdArgs& a, const WaveTable& t, int blocks, hipStream_t st) {
    if (a.p_split) {
        if constexpr (D == 64)
            hipLaunchKernelGGL((fwd_wave_kernel<D, DT, kSplit64.kt, kSplit64.nw, kSplit64.wpe, true, (kSplit64.pipe != 0)>), dim3((unsigned)blocks),
                               dim3(kSplit64.nw * 64), 0, st, a, t);
        else
            hipLaunchKernelGGL((fwd_wave_kernel<D, DT, kSplit128.kt, kSplit128.nw, kSplit128.wpe, true, (kSplit128.pipe != 0)>),
                               dim3((unsigned)blocks), dim3(kSplit128.nw * 64), 0, st, a, t);
    } else {
        if constexpr (D == 64)
            hipLaunchKernelGGL((fwd_wave_kernel<D, DT, kWave64.kt, kWave64.nw, kWave64.wpe, false, (kWave64.pipe != 0)>), dim3((unsigned)blocks),
                               dim3(kWave64.nw * 64), 0, st, a, t);
        else
            hipLaunchKernelGGL((fwd_wave_kernel<D, DT, kWave128.kt, kWave128.nw, kWave128.wpe, false, (kWave128.pipe != 0)>),
                               dim3((unsigned)blocks), dim3(kWave128.nw * 64), 0, st, a, t);
    }
    return hipGetLastError();
}

}  // namespace

int wave_block_m(int D, int p_split) { return wave_shape(D, p_split).nw * 32; }

hipError_t launch_wave(const FwdArgs& a, const WaveTable& t, int blocks, int D, int dtype, hipStream_t stream) {
    if (blocks <= 0) return hipSuccess;
    if (t.n_q < 1 || t.n_q > kWaveCap || t.n_k < 0 || t.n_k > kWaveCap || t.n_tiles < 1) return hipErrorInvalidValue;
    if (D == 64 && dtype == ET_F16) return launch_wave_d<64, ET_F16>(a, t, blocks, stream);
    if (D == 64 && dtype == ET_BF16) return launch_wave_d<64, ET_BF16>(a, t, blocks, stream);
    if (D == 128 && dtype == ET_F16) return launch_wave_d<128, ET_F16>(a, t, blocks, stream);
    if (D == 128 && dtype == ET_BF16) return launch_wave_d<128, ET_BF16>(a, t, blocks, stream);
    return hipErrorInvalidValue;
}

namespace {

template <int D, int DT>
hipError_t launch_bwd_d(const BwdArgs& a, int pass, hipStream_t st) {
    const int64_t rows = (int64_t)a.B * a.Hq * a.Nq;
    if (rows <= 0) return hipSuccess;
    if (pass == BWD_STATS) {
        constexpr int RPB = 256 / (D / 8);
        const int64_t blocks = (rows + RPB - 1) / RPB;
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((bwd_stats_kernel<D, DT>), dim3((unsigned)blocks), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    constexpr int DQ_NW = D == 64 ? 8 : 4, DQ_KT = D == 64 ? 64 : 32, DQ_WPE = 2;
    // D=64: dK and dV in one pass at three waves per SIMD; D=128: a dV pass at three waves, then a dK
    // pass at two (its 224 registers)
    constexpr int KV_NW = 4, KV_QT = 32;
    if (pass == BWD_DQ) {
        const int64_t n_qt = (a.Nq + DQ_NW * 32 - 1) / (DQ_NW * 32);
        const int64_t blocks = (int64_t)a.B * a.Hq * n_qt;
        if (blocks > 0x7FFFFFFF || n_qt > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        if (blocks > 0)
            hipLaunchKernelGGL((bwd_dq_kernel<D, DT, DQ_KT, DQ_NW, DQ_WPE>), dim3((unsigned)blocks), dim3(DQ_NW * 64), 0, st, a,
                               (int)n_qt);
        return hipGetLastError();
    }
    if (pass != BWD_DKDV) return hipErrorInvalidValue;
    const int64_t n_kt = (a.Nk + KV_NW * 32 - 1) / (KV_NW * 32);
    const int64_t blocks = (int64_t)a.B * a.Hkv * n_kt;
    if (blocks > 0x7FFFFFFF || n_kt > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (blocks > 0) {
        if constexpr (D == 64) {
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, DT, KV_QT, KV_NW, 3, 0>), dim3((unsigned)blocks),
                               dim3(KV_NW * 64), 0, st, a, (int)n_kt);
        } else {
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, DT, KV_QT, KV_NW, 3, 1>), dim3((unsigned)blocks), dim3(KV_NW * 64), 0,
                               st, a, (int)n_kt);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, DT, KV_QT, KV_NW, 2, 2>), dim3((unsigned)blocks), dim3(KV_NW * 64), 0,
                               st, a, (int)n_kt);
        }
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_pass(const BwdArgs& a, int D, int dtype, int pass, hipStream_t stream) {
    if (D == 64 && dtype == ET_F16) return launch_bwd_d<64, ET_F16>(a, pass, stream);
    if (D == 64 && dtype == ET_BF16) return launch_bwd_d<64, ET_BF16>(a, pass, stream);
    if (D == 128 && dtype == ET_F16) return launch_bwd_d<128, ET_F16>(a, pass, stream);
    if (D == 128 && dtype == ET_BF16) return launch_bwd_d<128, ET_BF16>(a, pass, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs& a, int D, int dtype, hipStream_t stream) {
    for (int pass : {BWD_STATS, BWD_DQ, BWD_DKDV}) {
        const hipError_t e = launch_bwd_pass(a, D, dtype, pass, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_cast(const float* src, int64_t B, int64_t H, int64_t n, int64_t D, void* dst, int dtype,
                       int64_t sb, int64_t sh, int64_t sn, hipStream_t stream) {
    const int64_t threads = B * H * n * (D / 4);
    if (threads <= 0) return hipSuccess;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFF || D % 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL(cast_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, B, H, n, D, dst, dtype, sb, sh, sn);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
    const int64_t total = (int64_t)a.B * a.Hq * (a.i_hi - a.i_lo);
    if (total <= 0) return hipSuccess;
    const int rpb = 256 / (a.D / 4);
    const int64_t blocks = (total + rpb - 1) / rpb;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (a.D == 64) {
        hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    } else if (a.D == 128) {
        hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cqsa
