// Measurement probe, not part of the attention path: the dense bf16 MFMA
// rate and the shader clock this chip sustains under an all-MFMA load, so
// that rooflines can be stated against a measured peak as well as against the
// data-sheet figure (2.5 PFLOP/s at 2.4 GHz for MI355X).
//
// Every wave of 8 per workgroup (two per SIMD) runs `iters` rounds of four
// independent 32x32x16 bf16 MFMA chains from registers (no memory traffic in
// the loop) and records its elapsed shader cycles (s_memtime) and reference
// ticks (s_memrealtime, 100 MHz), from which the caller derives the clock.
#include <hip/hip_runtime.h>

#include "../../include/mla_peak.h"
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

__global__ __launch_bounds__(512, 1) void mfma_peak_kernel(int iters, unsigned long long *clocks, float *sink) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(lane * 0.01f + i);
    b[i] = static_cast<__bf16>(i * 0.5f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(a, b, c1);
    c2 = mfma32(a, b, c2);
    c3 = mfma32(a, b, c3);
  }
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc += c0[r] + c1[r] + c2[r] + c3[r];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * 512 + threadIdx.x] = acc;   // keeps the chains live
  if (lane == 0) {
    clocks[(blockIdx.x * 8 + wave) * 2] = t1 - t0;
    clocks[(blockIdx.x * 8 + wave) * 2 + 1] = r1 - r0;
  }
}

}  // namespace
}  // namespace mla

extern "C" int mla_peak_mfma_bf16(int blocks, int iters, unsigned long long *clocks, float *sink, void *stream) {
  if (blocks < 1 || iters < 1 || clocks == nullptr || sink == nullptr) return -1;
  hipLaunchKernelGGL(mla::mfma_peak_kernel, dim3(blocks), dim3(512), 0, static_cast<hipStream_t>(stream), iters, clocks,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
