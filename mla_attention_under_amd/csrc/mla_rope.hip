// Rotary embedding of the RoPE band, in place (hyper-parallel
// mla_context_parallel.py, `apply_mla_rope`): the half-band rotation
// [a | b] -> [a cos - b sin | b cos + a sin], or adjacent pairs rotated and
// stored as real then imaginary half-bands. A row is read whole (its chunks
// spread over a group of lanes, or one thread's registers) before any of it is
// written, since the interleaved form writes positions other chunks are read
// from. HBM-bound: the band, the two tables of its token, the band again.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_common.h"
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

// Rows of CH 16-byte chunks (CH dividing 64), rows and tables 16-byte aligned:
// a row is handled by CH consecutive lanes, lane c holding chunk c, so every
// load and store instruction covers whole rows. Half-band: the partner half of
// chunk c is chunk c ^ CH/2 (one exchange). Interleaved: output chunk c takes
// the real (c < CH/2) or imaginary parts of the pairs in input chunks
// 2c mod CH and 2c+1 mod CH (two exchanges); its angles are table chunk
// c mod CH/2.
template <bool BF16, bool INTERLEAVED>
__global__ __launch_bounds__(kRopeThreads) void rope_vec_kernel(RopeArgs a, int ch) {
  constexpr int E = BF16 ? 8 : 4;   // elements per chunk
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kRopeThreads + threadIdx.x;
  const int64_t row = gid / ch;
  if (row >= a.rows) return;        // whole rows leave together: ch divides the block
  const int c = static_cast<int>(gid - row * ch);
  const int lane = threadIdx.x & 63, base = lane - c;
  const int64_t t = row / a.heads, h = row - t * a.heads;
  u32x4 *xp = reinterpret_cast<u32x4 *>(a.x + t * a.st + h * a.sh);
  const u32x4 *cp = reinterpret_cast<const u32x4 *>(a.cos + t * a.cst);
  const u32x4 *sp = reinterpret_cast<const u32x4 *>(a.sin + t * a.cst);
  const int half = ch / 2;
  const bool upper = c >= half;
  auto get = [&](const u32x4 &v, int e) {
    if constexpr (BF16) {
      const uint32_t w = v[e >> 1];
      return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
      return __uint_as_float(v[e]);
    }
  };
  auto shfl4 = [&](const u32x4 &v, int src) {
    return u32x4{static_cast<uint32_t>(__shfl(static_cast<int>(v[0]), src)),
                 static_cast<uint32_t>(__shfl(static_cast<int>(v[1]), src)),
                 static_cast<uint32_t>(__shfl(static_cast<int>(v[2]), src)),
                 static_cast<uint32_t>(__shfl(static_cast<int>(v[3]), src))};
  };
  const u32x4 xv = xp[c];
  float out[E];
  if constexpr (!INTERLEAVED) {
    const u32x4 cv = cp[c], sv = sp[c];
    const u32x4 pv = shfl4(xv, base + (c ^ half));
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float x0 = get(xv, e), xp_ = get(pv, e), cs = get(cv, e), sn = get(sv, e);
      out[e] = upper ? rope_im(xp_, x0, cs, sn) : rope_re(x0, xp_, cs, sn);
    }
  } else {
    const int tc = upper ? c - half : c;   // table chunk of this output chunk's pairs
    const u32x4 cv = cp[tc], sv = sp[tc];
    const int src0 = base + ((2 * c) & (ch - 1));
    const u32x4 in0 = shfl4(xv, src0), in1 = shfl4(xv, src0 + 1);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      // pair tc*E + e: elements 2e, 2e+1 of input chunk 2tc (e < E/2) or 2tc+1
      const u32x4 &iv = e < E / 2 ? in0 : in1;
      const int k = 2 * (e % (E / 2));
      const float re = get(iv, k), im = get(iv, k + 1), cs = get(cv, e), sn = get(sv, e);
      out[e] = upper ? rope_im(re, im, cs, sn) : rope_re(re, im, cs, sn);
    }
  }
  u32x4 w;
  if constexpr (BF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(out[2 * e], out[2 * e + 1]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(out[e]);
  }
  xp[c] = w;
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
      out[i] = rope_re(re, im, c, s);
      out[H + i] = rope_im(re, im, c, s);
    } else {
      const float x0 = ld(xp, i), x1 = ld(xp, H + i);
      out[i] = rope_re(x0, x1, ld(cp, i), ld(sp, i));
      out[H + i] = rope_im(x0, x1, ld(cp, H + i), ld(sp, H + i));
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

template <bool BF16>
hipError_t dispatch(const RopeArgs &a, const RopePlan &p, hipStream_t s) {
  constexpr int EB = BF16 ? 2 : 4;
  const uintptr_t al = reinterpret_cast<uintptr_t>(p.x) | reinterpret_cast<uintptr_t>(p.cos) |
                       reinterpret_cast<uintptr_t>(p.sin) | static_cast<uintptr_t>(a.st) |
                       static_cast<uintptr_t>(a.sh) | static_cast<uintptr_t>(a.cst);
  const int ch = (p.R * EB) % 16 == 0 ? p.R * EB / 16 : 0;
  const bool vec = al % 16 == 0 && ch >= 2 && ch <= 64 && (ch & (ch - 1)) == 0;
  if (vec) {
    const int64_t blocks = (a.rows * ch + kRopeThreads - 1) / kRopeThreads;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (p.interleaved)
      hipLaunchKernelGGL((rope_vec_kernel<BF16, true>), grid, dim3(kRopeThreads), 0, s, a, ch);
    else
      hipLaunchKernelGGL((rope_vec_kernel<BF16, false>), grid, dim3(kRopeThreads), 0, s, a, ch);
    return hipGetLastError();
  }
  const int64_t blocks = (a.rows + kRopeThreads - 1) / kRopeThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((rope_generic_kernel<BF16>), dim3(static_cast<unsigned>(blocks)), dim3(kRopeThreads), 0, s, a,
                     p.interleaved);
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
  if (a.rows == 0) return hipSuccess;
  return p.bf16 ? dispatch<true>(a, p, s) : dispatch<false>(a, p, s);
}

}  // namespace mla
