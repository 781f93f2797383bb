// Rotary embedding of the RoPE band, in place (hyper-parallel
// mla_context_parallel.py, `apply_mla_rope`): the half-band rotation
// [a | b] -> [a cos - b sin | b cos + a sin], or adjacent pairs rotated and
// stored as real then imaginary half-bands. One thread per band row: the
// interleaved form writes positions other threads would read, so a row is read
// whole before any of it is written. HBM-bound (the band, the two tables of
// its token, the band again); rows of 16-byte multiples move as 16-byte chunks.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_common.cuh"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kRopeThreads = 256;

struct RopeArgs {
  unsigned char *x;
  const unsigned char *cos, *sin;
  int64_t rows, st, sh, cst;   // byte strides
  int heads, R;
};

template <bool BF16>
__device__ __forceinline__ float elem(const u32x4 (&v)[32], int i) {
  if constexpr (BF16) {
    const uint32_t w = v[i >> 3][(i >> 1) & 3];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  } else {
    return __uint_as_float(v[i >> 2][i & 3]);
  }
}

// R known at compile time, rows and tables 16-byte aligned: registers only
template <bool BF16, int R, bool INTERLEAVED>
__global__ __launch_bounds__(kRopeThreads) void rope_vec_kernel(RopeArgs a) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int CH = R * EB / 16;     // 16-byte chunks per row
  constexpr int H = R / 2;
  static_assert(CH * 16 == R * EB && CH <= 32, "row of whole 16-byte chunks");
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRopeThreads + threadIdx.x;
  if (row >= a.rows) return;
  const int64_t t = row / a.heads, h = row - t * a.heads;
  u32x4 *xp = reinterpret_cast<u32x4 *>(a.x + t * a.st + h * a.sh);
  const u32x4 *cp = reinterpret_cast<const u32x4 *>(a.cos + t * a.cst);
  const u32x4 *sp = reinterpret_cast<const u32x4 *>(a.sin + t * a.cst);
  u32x4 xv[32], cv[32], sv[32];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    xv[i] = xp[i];
    cv[i] = cp[i];
    sv[i] = sp[i];
  }
  float out[R];
#pragma unroll
  for (int i = 0; i < H; ++i) {
    if constexpr (INTERLEAVED) {
      const float re = elem<BF16>(xv, 2 * i), im = elem<BF16>(xv, 2 * i + 1);
      const float c = elem<BF16>(cv, i), s = elem<BF16>(sv, i);
      out[i] = re * c - im * s;
      out[H + i] = im * c + re * s;
    } else {
      const float x0 = elem<BF16>(xv, i), x1 = elem<BF16>(xv, H + i);
      out[i] = x0 * elem<BF16>(cv, i) - x1 * elem<BF16>(sv, i);
      out[H + i] = x1 * elem<BF16>(cv, H + i) + x0 * elem<BF16>(sv, H + i);
    }
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    u32x4 w;
    if constexpr (BF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(out[8 * i + 2 * e], out[8 * i + 2 * e + 1]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(out[4 * i + e]);
    }
    xp[i] = w;
  }
}

// any even R <= 256, any element-aligned layout
template <bool BF16>
__global__ __launch_bounds__(kRopeThreads) void rope_generic_kernel(RopeArgs a, int interleaved) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRopeThreads + threadIdx.x;
  if (row >= a.rows) return;
  const int64_t t = row / a.heads, h = row - t * a.heads;
  unsigned char *xp = a.x + t * a.st + h * a.sh;
  const unsigned char *cp = a.cos + t * a.cst, *sp = a.sin + t * a.cst;
  auto ld = [&](const unsigned char *p, int i) {
    if constexpr (BF16)
      return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t *>(p)[i]) << 16);
    else
      return reinterpret_cast<const float *>(p)[i];
  };
  const int R = a.R, H = R / 2;
  float out[256];
  for (int i = 0; i < H; ++i) {
    if (interleaved) {
      const float re = ld(xp, 2 * i), im = ld(xp, 2 * i + 1), c = ld(cp, i), s = ld(sp, i);
      out[i] = re * c - im * s;
      out[H + i] = im * c + re * s;
    } else {
      const float x0 = ld(xp, i), x1 = ld(xp, H + i);
      out[i] = x0 * ld(cp, i) - x1 * ld(sp, i);
      out[H + i] = x1 * ld(cp, H + i) + x0 * ld(sp, H + i);
    }
  }
  for (int i = 0; i < R; ++i) {
    if constexpr (BF16) {
      const uint32_t w = pack_bf16x2(out[i], 0.f);
      reinterpret_cast<uint16_t *>(xp)[i] = static_cast<uint16_t>(w & 0xffffu);
    } else {
      reinterpret_cast<float *>(xp)[i] = out[i];
    }
  }
}

template <bool BF16, int R>
hipError_t launch_vec(const RopeArgs &a, bool inter, dim3 grid, hipStream_t s) {
  if (inter)
    hipLaunchKernelGGL((rope_vec_kernel<BF16, R, true>), grid, dim3(kRopeThreads), 0, s, a);
  else
    hipLaunchKernelGGL((rope_vec_kernel<BF16, R, false>), grid, dim3(kRopeThreads), 0, s, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t dispatch(const RopeArgs &a, const RopePlan &p, dim3 grid, hipStream_t s) {
  constexpr int EB = BF16 ? 2 : 4;
  const uintptr_t al = reinterpret_cast<uintptr_t>(p.x) | reinterpret_cast<uintptr_t>(p.cos) |
                       reinterpret_cast<uintptr_t>(p.sin) | static_cast<uintptr_t>(a.st) |
                       static_cast<uintptr_t>(a.sh) | static_cast<uintptr_t>(a.cst);
  const bool vec = al % 16 == 0 && (p.R * EB) % 16 == 0;
  const bool inter = p.interleaved != 0;
  if (vec && p.R == 64) return launch_vec<BF16, 64>(a, inter, grid, s);
  if (vec && p.R == 32) return launch_vec<BF16, 32>(a, inter, grid, s);
  if (vec && p.R == 128) return launch_vec<BF16, 128>(a, inter, grid, s);
  hipLaunchKernelGGL((rope_generic_kernel<BF16>), grid, dim3(kRopeThreads), 0, s, a, p.interleaved);
  return hipGetLastError();
}

}  // namespace

int launch_rope(const RopePlan &p, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t eb = p.bf16 ? 2 : 4;
  RopeArgs a;
  a.x = static_cast<unsigned char *>(p.x);
  a.cos = static_cast<const unsigned char *>(p.cos);
  a.sin = static_cast<const unsigned char *>(p.sin);
  a.rows = p.tokens * p.heads;
  a.st = p.stride_t * eb;
  a.sh = p.stride_h * eb;
  a.cst = p.cs_stride * eb;
  a.heads = p.heads;
  a.R = p.R;
  const int64_t blocks = (a.rows + kRopeThreads - 1) / kRopeThreads;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  return p.bf16 ? dispatch<true>(a, p, grid, s) : dispatch<false>(a, p, grid, s);
}

}  // namespace mla
