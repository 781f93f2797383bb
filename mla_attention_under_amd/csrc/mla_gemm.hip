// Latent up-projection through wkv_b for a contiguous head range:
//   out[t][n] = sum_l latent[t][l] * w[l][col0 + n],   n < ncols = heads*(N+V)
// (torchtitan "MLA CP optimization", sections "K/V all-gather CP" and "Ulysses CP";
// hyper-parallel `_head_projection_request` selects the rows of the head range,
// here the column block [col0, col0 + ncols) of the [L][heads_total*(N+V)] weight).
//
// bf16 path: one 128x128 output tile per 256-thread workgroup (4 waves of
// 64x64, two workgroups per CU), K streamed in 64-wide slices. Tiles move global->LDS with
// buffer_load ... lds into double-buffered, XOR-swizzled LDS (no staging
// registers; rows past the matrix read zero through the buffer range check).
// The latent is k-contiguous and feeds the MFMA straight from LDS; the weight
// is n-contiguous, and ds_read_b64_tr_b16 delivers its k-contiguous operand
// from the row-major tile. Each wave computes out^T = W^T latent^T with
// 32x32x16 MFMAs, so a lane owns one output row and 4-wide column runs; the
// tile leaves through LDS as 16-byte row-contiguous stores.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "mla_common.cuh"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int GM = 128, GN = 128, GK = 64;
constexpr int A_E = GM * GK, B_E = GK * GN;       // elements per stage
constexpr int CP = GN + 8;                        // LDS pitch of the output tile [m][n]
constexpr int SMEM_E = 2 * (A_E + B_E) > GM * CP ? 2 * (A_E + B_E) : GM * CP;
constexpr uint32_t kOob = 0x80000000u;            // a byte offset past every buffer range

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ int a_swz(int m) { return (m ^ (m >> 3)) & 7; }            // 8 chunks per row
__device__ __forceinline__ int b_swz(int k) { return (k & 2) | ((k & 1) * 5); }       // 8 segments per row

__global__ __launch_bounds__(256, 2) void up_proj_bf16_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W, uint16_t *__restrict__ C,
    int M, int K, int64_t ldw, int64_t col0, int ncols, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM_E];
  uint16_t *const st0 = smem, *const st1 = smem + (A_E + B_E);

  // Consecutive workgroups land on different XCDs (round robin over 8); give
  // each XCD a contiguous run of tiles so tiles sharing weight columns share an L2.
  const int nt = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int base = nt / 8 * 8;
  const int tile = b < base ? (b % 8) * (nt / 8) + b / 8 : b;
  const int m0 = __builtin_amdgcn_readfirstlane((tile % tiles_m) * GM);
  const int n0 = __builtin_amdgcn_readfirstlane((tile / tiles_m) * GN);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int half = lane >> 5, lrow = lane & 31, grp = lane >> 4, gl = lane & 15;

  // DMA plan: wave w fills A chunks [64*(4w+i), +64) and B chunks [64*(4w+i), +64)
  uint32_t a_off[4], b_off[4];
  int a_k[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = 64 * (4 * wave + i) + lane;
    const int m = p >> 3, c = (p & 7) ^ a_swz(m);
    a_k[i] = 8 * c;
    a_off[i] = static_cast<uint32_t>((m * K + 8 * c) * 2);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = 64 * (4 * wave + i) + lane;
    const int k = p >> 4, cp = p & 15;
    const int c = 2 * ((cp >> 1) ^ b_swz(k)) + (cp & 1);
    b_off[i] = static_cast<uint32_t>((k * ldw + 8 * c) * 2);
  }
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(A + static_cast<int64_t>(m0) * K, static_cast<uint32_t>(min(M - m0, GM) * K * 2));
  auto issue = [&](uint16_t *st, int k0) {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(W + static_cast<int64_t>(k0) * ldw + col0 + n0,
                                                static_cast<uint32_t>(min(K - k0, GK) * ldw * 2));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(st + 512 * (4 * wave + i)), 16,
                                               static_cast<int>(k0 + a_k[i] < K ? a_off[i] + 2 * k0 : kOob),
                                               0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(st + A_E + 512 * (4 * wave + i)), 16,
                                               static_cast<int>(b_off[i]), 0, 0, 0);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Operand fragments of one 64-wide k slice: weight^T via transposing reads,
  // latent^T direct. All of a slice's fragments are read before the next
  // slice's transfers are issued, so no LDS read waits on transfers in flight.
  bf16x8 wf[GK / 16][2], lf[GK / 16][2];
  auto read = [&](const uint16_t *st) {
    const uint16_t *As = st, *Bs = st + A_E;
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
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
  };
  auto mma = [&]() {
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(wf[ks][i], lf[ks][j], acc[i][j]);
  };

  const int nk = (K + GK - 1) / GK;
  issue(st0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    read(st0);
    if (kt + 1 < nk) issue(st1, (kt + 1) * GK);
    mma();
    __builtin_amdgcn_sched_barrier(0);   // keep the MFMAs ahead of the wait
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (kt + 1 < nk) {
      read(st1);
      if (kt + 2 < nk) issue(st0, (kt + 2) * GK);
      mma();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
    }
  }

  // epilogue: registers -> LDS tile [m][n] (bf16) -> 16-byte row stores
  uint16_t *Cs = smem;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m = 64 * wm + 32 * j + lrow;
        const int n = 64 * wn + 32 * i + 8 * g + 4 * half;
        const u32x2 v{pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                      pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
        *reinterpret_cast<u32x2 *>(Cs + m * CP + n) = v;
      }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < GM * GN / 8 / 256; ++u) {
    const int c = tid + 256 * u;
    const int row = c >> 4, nc = c & 15;
    const int m = m0 + row, n = n0 + 8 * nc;
    if (m < M && n < ncols)
      *reinterpret_cast<u32x4 *>(C + static_cast<int64_t>(m) * ncols + n) =
          *reinterpret_cast<const u32x4 *>(Cs + row * CP + 8 * nc);
  }
}

// Plain per-element kernel for fp32 (and any shape the tiled kernel does not take).
template <typename T>
__global__ __launch_bounds__(256) void up_proj_generic_kernel(const T *__restrict__ A, const T *__restrict__ W,
                                                              T *__restrict__ C, int64_t M, int K, int64_t ldw,
                                                              int64_t col0, int64_t ncols) {
  const int64_t total = M * ncols;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t m = idx / ncols, n = idx % ncols;
    float acc = 0.f;
    for (int k = 0; k < K; ++k) acc += load_f32(A, m * K + k) * load_f32(W, k * ldw + col0 + n);
    store_f32(C, idx, acc);
  }
}

}  // namespace

int launch_up_proj(const UpProjPlan &p, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.T == 0) return hipSuccess;
  const uintptr_t al = reinterpret_cast<uintptr_t>(p.latent) | reinterpret_cast<uintptr_t>(p.w) |
                       reinterpret_cast<uintptr_t>(p.out);
  const bool tiled = p.bf16 && p.L % 8 == 0 && p.ldw % 8 == 0 && p.col0 % 8 == 0 && p.ncols % 8 == 0 &&
                     al % 16 == 0 && p.T < (1LL << 31) && p.ncols < (1LL << 31);
  if (tiled) {
    const int tm = static_cast<int>((p.T + GM - 1) / GM);
    const int tn = static_cast<int>((p.ncols + GN - 1) / GN);
    hipLaunchKernelGGL(up_proj_bf16_kernel, dim3(tm * tn), dim3(256), 0, s,
                       static_cast<const uint16_t *>(p.latent), static_cast<const uint16_t *>(p.w),
                       static_cast<uint16_t *>(p.out), static_cast<int>(p.T), p.L, p.ldw, p.col0,
                       static_cast<int>(p.ncols), tm, tn);
    return hipGetLastError();
  }
  const int64_t total = p.T * p.ncols;
  const int blocks = static_cast<int>(std::min<int64_t>((total + 255) / 256, 65536));
  if (p.bf16)
    hipLaunchKernelGGL(up_proj_generic_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint16_t *>(p.latent), static_cast<const uint16_t *>(p.w),
                       static_cast<uint16_t *>(p.out), p.T, p.L, p.ldw, p.col0, p.ncols);
  else
    hipLaunchKernelGGL(up_proj_generic_kernel<float>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const float *>(p.latent), static_cast<const float *>(p.w),
                       static_cast<float *>(p.out), p.T, p.L, p.ldw, p.col0, p.ncols);
  return hipGetLastError();
}

}  // namespace mla
