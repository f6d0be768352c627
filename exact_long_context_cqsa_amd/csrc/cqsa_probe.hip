// Rate probes for gfx950: the matrix-core, LDS-read and HBM-copy rates the attention kernels are
// measured against, each with the shader clock the run held.  Every wave of the matrix and LDS
// probes reads the shader cycle counter (s_memtime) and the constant-rate wall clock
// (s_memrealtime) before and after its loop; the host turns the pair into a clock frequency.
//
// Workgroups are 256 threads (four waves).  The host launches the matrix probe with eight workgroups
// per compute unit and the LDS probe with two (32 KiB of LDS each), which measured the highest rates:
// 4018 FLOP and 256 bytes per clock per compute unit on MI355X.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "cqsa_internal.h"

namespace cqsa {
namespace {

typedef _Float16 probe_f16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;      // waves per workgroup
constexpr int kChains = 4;     // independent accumulator chains per wave (covers the MFMA latency)
constexpr int kLdsRows = 8;    // 1 KiB rows per wave in the LDS probe

__device__ __forceinline__ void put_clock(uint64_t* clk, uint64_t c0, uint64_t w0) {
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), w1 = __builtin_amdgcn_s_memrealtime();
    const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if ((threadIdx.x & 63) == 0) {
        clk[2 * wave] = c1 - c0;
        clk[2 * wave + 1] = w1 - w0;
    }
}

// kChains chains of v_mfma_f32_32x32x16_f16 per wave, operands in registers: iters * kChains * 32768
// FLOP per wave.  sink receives one float per thread so that nothing is eliminated.
__global__ void __launch_bounds__(256) probe_mfma_kernel(float* sink, uint64_t* clk, int iters) {
    const int lane = threadIdx.x & 63;
    probe_f16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)((float)((lane * 8 + i) % 17 - 8) * 0.0625f);
        b[i] = (_Float16)((float)((lane * 5 + i) % 13 - 6) * 0.0625f);
    }
    probe_f32x16 c[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = probe_f32x16{};
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), w0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[j], 0, 0, 0);
    }
    put_clock(clk, c0, w0);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += c[j][r];
    sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Each wave reads its own kLdsRows x 1 KiB of LDS with ds_read_b128, lane l at bytes 16 l .. 16 l + 15
// of each row (consecutive lanes on consecutive 16-byte granules: no bank conflict): iters * kLdsRows
// KiB per wave.  The reads are written out (a volatile block with its own wait) so that they are
// neither hoisted out of the loop nor narrowed, and only one dword of each is folded into the
// result, which keeps the VALU work per read small next to the LDS time.
__global__ void __launch_bounds__(256) probe_lds_kernel(uint32_t* sink, uint64_t* clk, int iters) {
    __shared__ __attribute__((aligned(16))) uint32_t buf[kWaves][kLdsRows * 256];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int i = lane; i < kLdsRows * 256; i += 64) buf[w][i] = (uint32_t)i * 2654435761u + (uint32_t)w;
    __syncthreads();
    // LDS byte address of this lane's granule in row 0 (the low half of the flat address of an LDS
    // variable is its LDS offset); rows 1..7 are reached by the instruction offsets below, all inside
    // buf[w] (at most 7168 + 1008 + 16 = 8192 bytes past its start).
    const uint32_t addr = (uint32_t)reinterpret_cast<uintptr_t>(&buf[w][lane * 4]);
    uint32_t acc = 0u;
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), w0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        probe_u32x4 r0, r1, r2, r3, r4, r5, r6, r7;
        asm volatile(
            "ds_read_b128 %0, %8\n\t"
            "ds_read_b128 %1, %8 offset:1024\n\t"
            "ds_read_b128 %2, %8 offset:2048\n\t"
            "ds_read_b128 %3, %8 offset:3072\n\t"
            "ds_read_b128 %4, %8 offset:4096\n\t"
            "ds_read_b128 %5, %8 offset:5120\n\t"
            "ds_read_b128 %6, %8 offset:6144\n\t"
            "ds_read_b128 %7, %8 offset:7168\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
            : "v"(addr)
            : "memory");
        acc ^= r0[0] ^ r1[1] ^ r2[2] ^ r3[3] ^ r4[0] ^ r5[1] ^ r6[2] ^ r7[3];
    }
    put_clock(clk, c0, w0);
    sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// dst[i] = src[i] over n16 16-byte elements, grid-stride.
__global__ void __launch_bounds__(256) probe_copy_kernel(const probe_u32x4* __restrict__ src,
                                                         probe_u32x4* __restrict__ dst, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

hipError_t launch_probe_mfma(int blocks, float* sink, uint64_t* clk, int iters, hipStream_t stream) {
    if (blocks < 1 || iters < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(64 * kWaves), 0, stream, sink, clk, iters);
    return hipGetLastError();
}

hipError_t launch_probe_lds(int blocks, uint32_t* sink, uint64_t* clk, int iters, hipStream_t stream) {
    if (blocks < 1 || iters < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_lds_kernel, dim3(blocks), dim3(64 * kWaves), 0, stream, sink, clk, iters);
    return hipGetLastError();
}

hipError_t launch_probe_copy(int blocks, const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    if (blocks < 1 || bytes < 0 || bytes % 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_copy_kernel, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const probe_u32x4*>(src), static_cast<probe_u32x4*>(dst), bytes / 16);
    return hipGetLastError();
}

}  // namespace cqsa
