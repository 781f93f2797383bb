// Latent up-projection through wkv_b for a contiguous head range:
//   out[t][n] = sum_l latent[t][l] * w[l][col0 + n],   n < ncols = heads*(N+V)
// (torchtitan "MLA CP optimization", sections "K/V all-gather CP" and "Ulysses CP";
// hyper-parallel `_head_projection_request` selects the rows of the head range,
// here the column block [col0, col0 + ncols) of the [L][heads_total*(N+V)] weight).
// The weight may also come as torch.nn.Linear stores it, [heads_total*(N+V)][L]
// (k-contiguous, the layout hyper-parallel `_validate_up_projections` checks):
// then its tile is staged like the latent's and read with plain 16-byte reads,
// and the products and their k order are the same, so both layouts give the same
// bits.
//
// bf16 path: one 128x128 output tile per 256-thread workgroup (4 waves of
// 64x64), two workgroups per CU (64 KB of LDS and 138 registers each), K
// streamed in 64-wide slices through two LDS buffers per operand. Tiles move
// global->LDS with buffer_load ... lds (no staging registers; rows past the
// matrix read zero through the buffer range check), one slice ahead of the
// one being multiplied; the two independent workgroups of a CU cover each
// other's transfer waits and barriers (measured 10 % faster than one 256x128
// workgroup of 8 waves with a three-slice ring). The latent is
// k-contiguous and feeds the MFMA straight from LDS; the weight is
// n-contiguous, and ds_read_b64_tr_b16 delivers its k-contiguous operand from
// the row-major tile. Each wave computes out^T = W^T latent^T with 32x32x16
// MFMAs, so a lane owns one output row and 4-wide column runs; the tile leaves
// through XOR-swizzled LDS as 16-byte row-contiguous stores.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int GM = 128, GN = 128, GK = 64;
constexpr int NWAVES = 4;
constexpr int A_E = GM * GK, B_E = GK * GN;       // elements per buffer
constexpr int A_I = A_E / 8 / (64 * NWAVES);      // 1 KB transfers per wave per slice (A)
constexpr int B_I = B_E / 8 / (64 * NWAVES);      // (B)
constexpr int kDmaPerSlice = A_I + B_I;
static_assert(A_I * 64 * NWAVES * 8 == A_E && B_I * 64 * NWAVES * 8 == B_E, "transfer split");
static_assert(kDmaPerSlice < 16, "vmcnt field");
static_assert(GM / 2 * GN <= A_E, "half the output tile fits one A buffer");
constexpr uint32_t kOob = 0x80000000u;            // a byte offset past every buffer range

__device__ __forceinline__ int a_swz(int m) { return (m ^ (m >> 3)) & 7; }            // 8 chunks per row
__device__ __forceinline__ int b_swz(int k) { return (k & 2) | ((k & 1) * 5); }       // 8 segments per row

// Slab-layout output (the projection written straight into the token->head
// pack): column n of the projection is element n % P of head n / P's block;
// head h (0-based within the projected range) belongs to the rank whose slab
// starts at head off[h] and holds qr[h] heads. Its row for token m is
//   send[T*off*F + (m*qr + h - off)*F + col_off + n % P].
// Columns [rope_off, rope_off + R) of each block are rotated (RoPE) in fp32
// from the accumulators, so the band is rounded to bf16 once; R = 64 at a
// multiple of 64 in a block whose width is a multiple of 64 (checked on the
// host), so a head's band is exactly one wave's 64-column group.
struct SlabOut {
  uint16_t *send;
  const uint16_t *cos, *sin;
  int64_t tokens, cs_stride;
  int P, F, col_off, rope_off, R, interleaved;
  int16_t off[kMaxSlabHeads], qr[kMaxSlabHeads];
};

// WT: the weight is [ncols-block rows][ldw] k-contiguous (element (k, n) at
// W[(col0 + n) * ldw + k]) instead of [K][ldw] n-contiguous.
template <bool SLAB, bool WT>
__global__ __launch_bounds__(256, 2) void up_proj_bf16_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W, uint16_t *__restrict__ C,
    int M, int K, int64_t ldw, int64_t col0, int ncols, int tiles_m, int tiles_n, SlabOut so) {
  __shared__ __attribute__((aligned(1024))) uint16_t a0[A_E];
  __shared__ __attribute__((aligned(1024))) uint16_t a1[A_E];
  __shared__ __attribute__((aligned(1024))) uint16_t b0[B_E];
  __shared__ __attribute__((aligned(1024))) uint16_t b1[B_E];

  // Consecutive workgroups land on different XCDs (round robin over 8); give
  // each XCD a contiguous run of tiles so tiles sharing weight columns share an L2.
  const int nt = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  const int base = nt / 8 * 8;
  const int tile = bid < base ? (bid % 8) * (nt / 8) + bid / 8 : bid;
  const int m0 = __builtin_amdgcn_readfirstlane((tile % tiles_m) * GM);
  const int n0 = __builtin_amdgcn_readfirstlane((tile / tiles_m) * GN);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int half = lane >> 5, lrow = lane & 31, grp = lane >> 4, gl = lane & 15;

  // Transfer plan: wave w fills A chunks [64*(A_I w + i), +64) and B chunks
  // [64*(B_I w + i), +64); lane l loads the global chunk the swizzle puts there.
  uint32_t a_off[A_I], b_off[B_I];
  int a_k[A_I], b_k[B_I];
#pragma unroll
  for (int i = 0; i < A_I; ++i) {
    const int p = 64 * (A_I * wave + i) + lane;
    const int m = p >> 3, c = (p & 7) ^ a_swz(m);
    a_k[i] = 8 * c;
    a_off[i] = static_cast<uint32_t>((m * K + 8 * c) * 2);
  }
#pragma unroll
  for (int i = 0; i < B_I; ++i) {
    const int p = 64 * (B_I * wave + i) + lane;
    if constexpr (WT) {   // [GN rows n][GK] like the latent's tile
      const int n = p >> 3, c = (p & 7) ^ a_swz(n);
      b_k[i] = 8 * c;
      b_off[i] = static_cast<uint32_t>((n * ldw + 8 * c) * 2);
    } else {              // [GK rows k][GN], 32-byte segments swizzled per row
      const int k = p >> 4, cp = p & 15;
      const int c = 2 * ((cp >> 1) ^ b_swz(k)) + (cp & 1);
      b_k[i] = 0;
      b_off[i] = static_cast<uint32_t>((k * ldw + 8 * c) * 2);
    }
  }
  const u32x4 ra = dma_rsrc(A + static_cast<int64_t>(m0) * K, static_cast<uint32_t>(min(M - m0, GM) * K * 2));
  // k-contiguous weight: rows [col0 + n0, + min(ncols - n0, GN)) of the transposed weight
  const u32x4 rbt = WT ? dma_rsrc(W + (col0 + n0) * ldw, static_cast<uint32_t>(min(ncols - n0, GN) * ldw * 2))
                       : u32x4{0, 0, 0, 0};
  auto issue = [&](uint16_t *as, uint16_t *bs, int k0) {
    const uint32_t la = lds_addr(as), lb = lds_addr(bs);
#pragma unroll
    for (int i = 0; i < A_I; ++i)
      dma16(ra, la + 1024 * (A_I * wave + i), k0 + a_k[i] < K ? a_off[i] + 2 * k0 : kOob);
    if constexpr (WT) {
#pragma unroll
      for (int i = 0; i < B_I; ++i)
        dma16(rbt, lb + 1024 * (B_I * wave + i), k0 + b_k[i] < K ? b_off[i] + 2 * k0 : kOob);
    } else {
      const u32x4 rb = dma_rsrc(W + static_cast<int64_t>(k0) * ldw + col0 + n0,
                                static_cast<uint32_t>(min(K - k0, GK) * ldw * 2));
#pragma unroll
      for (int i = 0; i < B_I; ++i) dma16(rb, lb + 1024 * (B_I * wave + i), b_off[i]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // one 64-wide k slice from buffers (as, bs): weight^T via transposing
  // reads (or direct, k-contiguous weight), latent^T direct
  auto slice = [&](const uint16_t *As, const uint16_t *Bs) __attribute__((always_inline)) {
    bf16x8 wf[GK / 16][2], lf[GK / 16][2];
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (WT) {
          const int n = 64 * wn + 32 * i + lrow;
          wf[ks][i] = *reinterpret_cast<const bf16x8 *>(Bs + n * GK + 8 * ((2 * ks + half) ^ a_swz(n)));
          continue;
        }
        const int n = 64 * wn + 32 * i + 16 * (grp & 1) + 4 * (gl & 3);
        // lanes of half h take k = 16ks + 8h + 0..7 in natural order (the latent operand's order)
        const int k0r = 16 * ks + 8 * (grp >> 1) + (gl >> 2), k1r = k0r + 4;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)(Bs + k0r * GN + 16 * ((n >> 4) ^ b_swz(k0r)) + (n & 15)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)(Bs + k1r * GN + 16 * ((n >> 4) ^ b_swz(k1r)) + (n & 15)));
        wf[ks][i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = 64 * wm + 32 * j + lrow;
        lf[ks][j] = *reinterpret_cast<const bf16x8 *>(As + m * GK + 8 * ((2 * ks + half) ^ a_swz(m)));
      }
    }
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(wf[ks][i], lf[ks][j], acc[i][j]);
  };

  // slice s lives in buffer s % 2; during slice s the transfers of slice s+1
  // go into the buffer slice s-1 used, and each wave waits for them before the
  // barrier that ends the slice (two workgroups per CU cover each other's waits)
  const int nk = (K + GK - 1) / GK;
  auto step = [&](int s, const uint16_t *as, const uint16_t *bs, uint16_t *an, uint16_t *bn)
      __attribute__((always_inline)) {
    if (s + 1 < nk) issue(an, bn, (s + 1) * GK);
    slice(as, bs);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  issue(a0, b0, 0);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  int s = 0;
  for (; s + 1 < nk; s += 2) {
    step(s, a0, b0, a1, b1);
    step(s + 1, a1, b1, a0, b0);
  }
  if (s < nk) step(s, a0, b0, a1, b1);

  // epilogue: registers -> LDS (rows [0,128) in a0, [128,256) in a1, each
  // [128][128] bf16 with 16-byte chunks XOR-swizzled by row) -> 16-byte row stores
  __syncthreads();
  if constexpr (SLAB) {
    // RoPE of the band on the fp32 accumulators. The waves whose 64-column
    // group is a band hold all of it: lane (lrow, half) has columns
    // 32 i + 8 g + 4 half + e of rows 32 j + lrow. A half-band pair (c, c + 32)
    // is acc[0] / acc[1] of one lane; an interleaved pair (2p, 2p + 1) comes
    // through the wave's own 16 KB of LDS (the stage buffers are free here).
    const int g0 = n0 + 64 * wn;
    const bool band = so.R > 0 && g0 < ncols && g0 % so.P == so.rope_off;   // uniform per wave
    float *xs = reinterpret_cast<float *>(wave == 0 ? a0 : wave == 1 ? a1 : wave == 2 ? b0 : b1);
    // 16-byte chunk c4 (of 16) of row r of the wave's [64][64] fp32 block, XOR-swizzled by row
    auto xchunk = [&](int r, int c4) { return reinterpret_cast<f32x4 *>(xs + 64 * r + 4 * (c4 ^ (r & 15))); };
    auto tab = [&](const u32x2 &v, int e) {
      const uint32_t w = v[e >> 1];
      return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    };
    if (band && so.interleaved) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *xchunk(32 * j + lrow, 8 * i + 2 * g + half) =
                f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
    }
    __syncthreads();
    if (band) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t mt = min(m0 + 64 * wm + 32 * j + lrow, M - 1);   // rows past the end are not stored
        const uint16_t *cr = so.cos + mt * so.cs_stride, *sr = so.sin + mt * so.cs_stride;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c0 = 8 * g + 4 * half;
          if (!so.interleaved) {
            // out[c] = x[c] cos[c] - x[c+32] sin[c], out[c+32] = x[c+32] cos[c+32] + x[c] sin[c+32]
            const u32x2 ca = *reinterpret_cast<const u32x2 *>(cr + c0), sa = *reinterpret_cast<const u32x2 *>(sr + c0);
            const u32x2 cb = *reinterpret_cast<const u32x2 *>(cr + c0 + 32),
                        sb = *reinterpret_cast<const u32x2 *>(sr + c0 + 32);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float lo = acc[0][j][4 * g + e], hi = acc[1][j][4 * g + e];
              acc[0][j][4 * g + e] = rope_re(lo, hi, tab(ca, e), tab(sa, e));
              acc[1][j][4 * g + e] = rope_im(lo, hi, tab(cb, e), tab(sb, e));
            }
          } else {
            // pair p = c0 + e is (x[2p], x[2p+1]): its real part goes to column p, its imaginary part to p + 32
            const u32x2 ca = *reinterpret_cast<const u32x2 *>(cr + c0), sa = *reinterpret_cast<const u32x2 *>(sr + c0);
            const f32x4 in0 = *xchunk(32 * j + lrow, 4 * g + 2 * half), in1 = *xchunk(32 * j + lrow, 4 * g + 2 * half + 1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float re = e < 2 ? in0[2 * e] : in1[2 * e - 4], im = e < 2 ? in0[2 * e + 1] : in1[2 * e - 3];
              acc[0][j][4 * g + e] = rope_re(re, im, tab(ca, e), tab(sa, e));
              acc[1][j][4 * g + e] = rope_im(re, im, tab(ca, e), tab(sa, e));
            }
          }
        }
      }
    }
    __syncthreads();
  }
  uint16_t *Cs = wm == 0 ? a0 : a1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m = 32 * j + lrow;
        const int n = 64 * wn + 32 * i + 8 * g + 4 * half;
        const u32x2 v{pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                      pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
        *reinterpret_cast<u32x2 *>(Cs + m * GN + 8 * ((n >> 3) ^ (m & 15)) + (n & 7)) = v;
      }
  __syncthreads();
  if constexpr (SLAB) {
#pragma unroll 4
    for (int u = 0; u < GM * GN / 8 / 256; ++u) {
      const int c = tid + 256 * u;
      const int row = c >> 4, nc = c & 15;
      const int m = m0 + row, n = n0 + 8 * nc;
      if (m >= M || n >= ncols) continue;
      const uint16_t *rowp = (row < GM / 2 ? a0 : a1) + (row & (GM / 2 - 1)) * GN;
      auto chunk_at = [&](int col) { return *reinterpret_cast<const u32x4 *>(rowp + 8 * ((col >> 3) ^ (row & 15))); };
      const u32x4 v = chunk_at(8 * nc);
      const int hh = n / so.P, f = n - hh * so.P;
      const int ro = so.off[hh], qr = so.qr[hh];
      uint16_t *dst = so.send + (so.tokens * ro + static_cast<int64_t>(m) * qr + (hh - ro)) * so.F + so.col_off + f;
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < GM * GN / 8 / 256; ++u) {
    const int c = tid + 256 * u;
    const int row = c >> 4, nc = c & 15;
    const int m = m0 + row, n = n0 + 8 * nc;
    const uint16_t *src = (row < GM / 2 ? a0 : a1) + (row & (GM / 2 - 1)) * GN + 8 * (nc ^ (row & 15));
    if (m < M && n < ncols)
      // streamed past L2: whole 128-byte lines, and no dirty lines left for
      // the end-of-kernel write-back (measured 15.1 -> 13.7 us on the rank shard)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(src),
                                  reinterpret_cast<u32x4 *>(C + static_cast<int64_t>(m) * ncols + n));
  }
}

// Plain per-element kernel for fp32 (and any shape the tiled kernel does not take).
template <typename T, bool WT>
__global__ __launch_bounds__(256) void up_proj_generic_kernel(const T *__restrict__ A, const T *__restrict__ W,
                                                              T *__restrict__ C, int64_t M, int K, int64_t ldw,
                                                              int64_t col0, int64_t ncols) {
  const int64_t total = M * ncols;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t m = idx / ncols, n = idx % ncols;
    float acc = 0.f;
    for (int k = 0; k < K; ++k)
      acc += load_f32(A, m * K + k) * load_f32(W, WT ? (col0 + n) * ldw + k : k * ldw + col0 + n);
    store_f32(C, idx, acc);
  }
}

}  // namespace

int launch_up_proj(const UpProjPlan &p, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.T == 0) return hipSuccess;
  const uintptr_t al = reinterpret_cast<uintptr_t>(p.latent) | reinterpret_cast<uintptr_t>(p.w) |
                       reinterpret_cast<uintptr_t>(p.out);
  // (k-contiguous weight: every row starts 16-byte aligned when ldw % 8 == 0,
  // whatever col0.) A tile's transfers address its rows by 32-bit byte
  // offsets: the latent's GM rows, the k-contiguous weight's GN rows or the
  // row-major weight's GK rows must fit 4 GiB, and the grid 2^31 workgroups.
  const int64_t tm64 = (p.T + GM - 1) / GM, tn64 = (p.ncols + GN - 1) / GN;
  const bool tiled = p.bf16 && p.L % 8 == 0 && p.ldw % 8 == 0 && (p.w_kmajor || p.col0 % 8 == 0) &&
                     p.ncols % 8 == 0 && al % 16 == 0 && p.T < (1LL << 31) && p.ncols < (1LL << 31) &&
                     static_cast<int64_t>(GM) * p.L * 2 < (1LL << 32) &&
                     static_cast<int64_t>(p.w_kmajor ? GN : GK) * p.ldw * 2 < (1LL << 32) &&
                     tm64 * tn64 < (1LL << 31);
  if (tiled) {
    const int tm = static_cast<int>(tm64);
    const int tn = static_cast<int>(tn64);
    SlabOut none{};
    if (p.w_kmajor)
      hipLaunchKernelGGL((up_proj_bf16_kernel<false, true>), dim3(tm * tn), dim3(256), 0, s,
                         static_cast<const uint16_t *>(p.latent), static_cast<const uint16_t *>(p.w),
                         static_cast<uint16_t *>(p.out), static_cast<int>(p.T), p.L, p.ldw, p.col0,
                         static_cast<int>(p.ncols), tm, tn, none);
    else
      hipLaunchKernelGGL((up_proj_bf16_kernel<false, false>), dim3(tm * tn), dim3(256), 0, s,
                         static_cast<const uint16_t *>(p.latent), static_cast<const uint16_t *>(p.w),
                         static_cast<uint16_t *>(p.out), static_cast<int>(p.T), p.L, p.ldw, p.col0,
                         static_cast<int>(p.ncols), tm, tn, none);
    return hipGetLastError();
  }
  const int64_t total = p.T * p.ncols;
  const int blocks = static_cast<int>(std::min<int64_t>((total + 255) / 256, 65536));
  auto generic = [&](auto zero) {
    using T = decltype(zero);
    if (p.w_kmajor)
      hipLaunchKernelGGL((up_proj_generic_kernel<T, true>), dim3(blocks), dim3(256), 0, s,
                         static_cast<const T *>(p.latent), static_cast<const T *>(p.w), static_cast<T *>(p.out), p.T,
                         p.L, p.ldw, p.col0, p.ncols);
    else
      hipLaunchKernelGGL((up_proj_generic_kernel<T, false>), dim3(blocks), dim3(256), 0, s,
                         static_cast<const T *>(p.latent), static_cast<const T *>(p.w), static_cast<T *>(p.out), p.T,
                         p.L, p.ldw, p.col0, p.ncols);
  };
  if (p.bf16)
    generic(uint16_t{0});
  else
    generic(0.f);
  return hipGetLastError();
}

int launch_project_pack(const ProjectPackPlan &p, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.T == 0) return hipSuccess;
  SlabOut so;
  so.send = static_cast<uint16_t *>(p.send);
  so.cos = static_cast<const uint16_t *>(p.cos);
  so.sin = static_cast<const uint16_t *>(p.sin);
  so.tokens = p.T;
  so.cs_stride = p.cs_stride;
  so.P = p.P;
  so.F = p.F;
  so.col_off = p.col_off;
  so.rope_off = p.R > 0 ? p.rope_off : p.P;   // no band: no column qualifies
  so.R = p.R;
  so.interleaved = p.interleaved;
  for (int h = 0; h < p.heads; ++h) {
    so.off[h] = static_cast<int16_t>(p.off[h]);
    so.qr[h] = static_cast<int16_t>(p.qr[h]);
  }
  const int64_t ncols = static_cast<int64_t>(p.heads) * p.P;
  const int tm = static_cast<int>((p.T + GM - 1) / GM);
  const int tn = static_cast<int>((ncols + GN - 1) / GN);
  hipLaunchKernelGGL((up_proj_bf16_kernel<true, false>), dim3(tm * tn), dim3(256), 0, s,
                     static_cast<const uint16_t *>(p.latent), static_cast<const uint16_t *>(p.w), nullptr,
                     static_cast<int>(p.T), p.L, p.ldw, p.col0, static_cast<int>(ncols), tm, tn, so);
  return hipGetLastError();
}

}  // namespace mla
