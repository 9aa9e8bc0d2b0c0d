// fa_probe.hip -- measurement probes for the benchmark (libfa_probe.so).
//
// Not part of the attention library: these kernels calibrate what the chip
// delivers, so that measured rates can be set against a measured ceiling as
// well as against the published peaks.
//   * fa_probe_mfma: a register-only loop of v_mfma_f32_32x32x16_bf16 on four
//     independent accumulators at two waves per SIMD, on random operands or on
//     constant ones, optionally with one v_exp_f32 per product (the forward's
//     ratio of exponentials to products); or of the e4m3 product
//     v_mfma_scale_f32_32x32x64_f8f6f4 on random codes.  Each workgroup records the
//     shader-clock cycles (s_memtime) and the constant 100 MHz reference
//     (s_memrealtime) it took, which gives the clock the chip ran at.
//   * fa_probe_stream_read: a streaming read of a large buffer (16-byte
//     non-temporal loads), the practical HBM read ceiling.
//   * fa_probe_fwd_clock: the library's own bf16 forward kernel (d = 128,
//     causal, bf16 O), instantiated with its per-workgroup clock record on.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_kernel.hpp"

namespace fa {

namespace {

constexpr int PROBE_THREADS = 256;

typedef int i32x8 __attribute__((ext_vector_type(8)));

// MODE 0: random operands; 1: random operands and one exp per product;
// 2: constant operands (all bf16); 3: random e4m3 codes on the fp8 product
// (unit block scales).  ops holds 8 16-byte operand vectors per lane
// (a0..a3, b0..b3; an fp8 operand takes two of them).
template <int MODE>
__global__ void __launch_bounds__(PROBE_THREADS) __attribute__((amdgpu_waves_per_eu(2)))
mfma_probe_kernel(const uint4* __restrict__ ops, int iters, float* __restrict__ sink,
                  unsigned long long* __restrict__ clk) {
    unsigned long long t0 = 0, r0 = 0;
    if (threadIdx.x == 0) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    const size_t base = ((size_t)blockIdx.x * PROBE_THREADS + threadIdx.x) * 8;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a[j] = as_bf16x8(ops[base + j]);
        b[j] = as_bf16x8(ops[base + 4 + j]);
    }
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = zero16();
    float x[4] = {0.1f, 0.2f, 0.3f, 0.4f};
    if constexpr (MODE == 3) {
        i32x8 fa8[2], fb8[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint4 lo = ops[base + 2 * j], hi = ops[base + 2 * j + 1];
            const uint4 blo = ops[base + 4 + 2 * j], bhi = ops[base + 5 + 2 * j];
            fa8[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            fb8[j] = i32x8{(int)blo.x, (int)blo.y, (int)blo.z, (int)blo.w, (int)bhi.x, (int)bhi.y, (int)bhi.z, (int)bhi.w};
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa8[j & 1], fb8[(j >> 1) & 1], acc[j],
                                                                         0, 0, 0, 127, 0, 127);
        }
    } else {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[j] = mfma_bf16(a[j], b[j], acc[j]);
                if constexpr (MODE == 1) x[j] = exp2_fast(fmaf(x[j], -0.37f, 0.6f));
            }
        }
    }
    float s = x[0] + x[1] + x[2] + x[3];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    sink[(size_t)blockIdx.x * PROBE_THREADS + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - t0;
        clk[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - r0;
    }
}

__global__ void __launch_bounds__(PROBE_THREADS)
stream_read_kernel(const uint4* __restrict__ p, size_t n16, uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * PROBE_THREADS;
    uint32_t acc = 0;
    for (size_t i = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x; i < n16; i += stride) {
        const uint4 v = load_stream16(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(size_t)blockIdx.x * PROBE_THREADS + threadIdx.x] = acc;
}

}  // namespace

}  // namespace fa

extern "C" {

// mode 0..3 (see mfma_probe_kernel); ops: grid * 256 * 8 16-byte operand
// vectors; sink: grid * 256 floats; clk: 2 * grid values.  Returns a
// hipError_t code.
int fa_probe_mfma(int mode, const void* ops, int iters, int grid, float* sink, unsigned long long* clk,
                  void* stream) {
    if (!ops || !sink || !clk || iters < 1 || grid < 1 || mode < 0 || mode > 3) return (int)hipErrorInvalidValue;
    const dim3 g((unsigned)grid), b(fa::PROBE_THREADS);
    hipStream_t st = (hipStream_t)stream;
    const uint4* o = (const uint4*)ops;
    if (mode == 0) hipLaunchKernelGGL((fa::mfma_probe_kernel<0>), g, b, 0, st, o, iters, sink, clk);
    else if (mode == 1) hipLaunchKernelGGL((fa::mfma_probe_kernel<1>), g, b, 0, st, o, iters, sink, clk);
    else if (mode == 2) hipLaunchKernelGGL((fa::mfma_probe_kernel<2>), g, b, 0, st, o, iters, sink, clk);
    else hipLaunchKernelGGL((fa::mfma_probe_kernel<3>), g, b, 0, st, o, iters, sink, clk);
    return (int)hipGetLastError();
}

// buf: bytes (a multiple of 16) of device memory; sink: grid * 256 words.
int fa_probe_stream_read(const void* buf, size_t bytes, int grid, uint32_t* sink, void* stream) {
    if (!buf || !sink || grid < 1 || bytes % 16) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(fa::stream_read_kernel, dim3((unsigned)grid), dim3(fa::PROBE_THREADS), 0, (hipStream_t)stream,
                       (const uint4*)buf, bytes / 16, sink);
    return (int)hipGetLastError();
}

// The bf16 forward (d = 128, causal, bf16 O) with the clock record on.  q, k,
// v, o: [B,H,N,128] bf16; lse: [B,H,N] fp32; clk: 2 * ceil(N/128) * B * H
// values.  Returns a hipError_t code.
int fa_probe_fwd_clock(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                       float scale, unsigned long long* clk, void* stream) {
    if (!q || !k || !v || !o || !lse || !clk || B < 1 || H < 1 || N < 1) return (int)hipErrorInvalidValue;
    const int BH = B * H, nqt = (N + fa::FWD_BR - 1) / fa::FWD_BR;
    hipLaunchKernelGGL((fa::fwd_bf16_kernel<128, true, true, true>), dim3((unsigned)(nqt * BH)),
                       dim3(fa::FWD_THREADS), 0, (hipStream_t)stream, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, o, lse, BH, 1, N, nqt, scale * fa::kLog2e, clk);
    return (int)hipGetLastError();
}

}  // extern "C"
