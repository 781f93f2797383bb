// Device helpers shared by the gfx950 kernels: bf16 vector types, the bf16
// MFMA wrappers, and fp32 <-> bf16 conversion.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// D[32x32] += A[32x16] * B[16x32] in fp32. Lane l holds A row (l%32), k = 8*(l/32)..+7
// and B column (l%32), k = 8*(l/32)..+7; D[i][j] sits in lane j + 32*((i/4)%2),
// register 4*(i/8) + i%4.
__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D[16x16] += A[16x32] * B[32x16]. Lane l holds A row (l%16), k = 8*(l/16)..+7 and
// B column (l%16), k = 8*(l/16)..+7; D[i][j] sits in lane j + 16*(i/4), register i%4.
__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(const bf16x8 &v) { return __builtin_bit_cast(u32x4, v); }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
}
// Round-to-nearest-even fp32 -> bf16 (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two fp32 -> two bf16 packed in one dword (low = a), one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// One rotated element of a RoPE pair (the real part when `second` is false,
// the imaginary part when it is true): first*c - second_in*s and
// second_in*c + first*s, evaluated as one product and one fused multiply-add
// so that every kernel rotating a band rounds identically.
__device__ __forceinline__ float rope_re(float re, float im, float c, float s) {
  return __builtin_fmaf(re, c, -(im * s));
}
__device__ __forceinline__ float rope_im(float re, float im, float c, float s) {
  return __builtin_fmaf(im, c, re * s);
}
// bf16 element e of a 16-byte chunk, widened
__device__ __forceinline__ float bf16_elem(const u32x4 &v, int e) {
  const uint32_t w = v[e >> 1];
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

// Interleave the 16-bit halves of two dwords: lo16(a)|lo16(b)<<16 and hi16(a)|hi16(b)<<16.
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// Buffer resource over [base, base + bytes): loads past the end return zero
// (hardware range check), so tile loaders need no clamps or branches.
constexpr int kBufferDword3 = 0x00020000;   // raw 32-bit data format (gfx9 family)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), kBufferDword3);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(byte_off), 0, 0));
}

// ---- LDS helpers -----------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Buffer resource (base, byte range) as four scalar dwords, for dma16.
__device__ __forceinline__ u32x4 dma_rsrc(const void *base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(b), hi = static_cast<uint32_t>(b >> 32) & 0xffffu;
  return u32x4{static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(lo)),
               static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(hi)),
               static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(bytes)), static_cast<uint32_t>(kBufferDword3)};
}

// One 1 KB global->LDS transfer of a wave: lane l copies the 16 bytes at byte
// voff of the buffer (zero outside its range) to lds_dst + 16 l. Written as
// inline assembly so that the compiler does not track it: completion is
// awaited explicitly with vmcnt before the barrier that publishes the tile.
// (Tracked, its alias analysis loses the buffers apart in an unrolled ring
// and waits for every transfer in flight before reading any tile.)
__device__ __forceinline__ void dma16(const u32x4 &r, uint32_t lds_dst, uint32_t voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(lds_dst));
}

// LDS byte address of a shared-memory pointer (uniform)
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
      static_cast<int>(reinterpret_cast<uintptr_t>((lds_void *)(p)))));
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): lane i of each 16-lane
// group receives column i of the 4x16 block of bf16 whose rows its lanes
// address (each lane addresses 4 consecutive elements of one row).
__device__ __forceinline__ s16x4 read_tr(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}

template <typename T>
__device__ __forceinline__ float load_f32(const T *p, int64_t i);
template <>
__device__ __forceinline__ float load_f32<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_f32<uint16_t>(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename T>
__device__ __forceinline__ void store_f32(T *p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_f32<float>(float *p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_f32<uint16_t>(uint16_t *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }

}  // namespace mla
