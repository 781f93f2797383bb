// Latent up-projection through wkv_b for a contiguous head range:
//   out[t][n] = sum_l latent[t][l] * w[l][col0 + n],   n < ncols = heads*(N+V)
// (torchtitan "MLA CP optimization", sections "K/V all-gather CP" and "Ulysses CP";
// hyper-parallel `_head_projection_request` selects the rows of the head range,
// here the column block [col0, col0 + ncols) of the [L][heads_total*(N+V)] weight).
//
// bf16 path: one 128x128 output tile per 256-thread workgroup, K streamed in
// 64-wide slices through double-buffered LDS with global->register prefetch.
// Both MFMA operands want 8 consecutive k per lane; the latent is k-contiguous
// already, the weight is n-contiguous, so each thread transposes a 4(k) x 8(n)
// block of it in registers before writing it to LDS as [n][k]. Each wave
// computes a 64x64 sub-tile as out^T = W^T * latent^T with 32x32x16 MFMAs, so
// a lane owns one output row and 4-wide runs of columns; the tile leaves
// through LDS as 16-byte row-contiguous stores.
#include <hip/hip_runtime.h>

#include "mla_common.cuh"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int GM = 128, GN = 128, GK = 64;
constexpr int AP = GK + 8;   // LDS pitch (elements) of latent rows [m][k]
constexpr int BP = GK + 8;   // LDS pitch of transposed weight rows [n][k]
constexpr int CP = GN + 8;   // LDS pitch of the output tile [m][n]
constexpr int kStage = GM * AP + GN * BP;
static_assert(2 * kStage >= GM * CP, "epilogue tile must fit in the staging buffers");

__global__ __launch_bounds__(256) void up_proj_bf16_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W, uint16_t *__restrict__ C,
    int M, int K, int64_t ldw, int64_t col0, int ncols, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStage];

  // Consecutive workgroups land on different XCDs (round robin over 8); give
  // each XCD a contiguous run of tiles so tiles sharing weight columns share an L2.
  const int nt = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int base = nt / 8 * 8;
  const int tile = b < base ? (b % 8) * (nt / 8) + b / 8 : b;
  const int m0 = (tile % tiles_m) * GM;
  const int n0 = (tile / tiles_m) * GN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // global -> register staging
  u32x4 ra[4];
  u32x4 rb[4];
  const int kq = tid & 15, nq = tid >> 4;   // weight block: k rows 4kq..4kq+3, n cols 8nq..8nq+7
  const bool n_ok = n0 + 8 * nq < ncols;

  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u;
      const int row = c >> 3, kc = c & 7;
      const int m = m0 + row, k = k0 + 8 * kc;
      ra[u] = (m < M && k < K) ? *reinterpret_cast<const u32x4 *>(A + static_cast<int64_t>(m) * K + k)
                               : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = k0 + 4 * kq + r;
      rb[r] = (n_ok && k < K)
                  ? *reinterpret_cast<const u32x4 *>(W + static_cast<int64_t>(k) * ldw + col0 + n0 + 8 * nq)
                  : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&](int buf) {
    uint16_t *As = smem + buf * kStage;
    uint16_t *Bs = As + GM * AP;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u;
      *reinterpret_cast<u32x4 *>(As + (c >> 3) * AP + 8 * (c & 7)) = ra[u];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const u32x2 lo{lo_halves(rb[0][m], rb[1][m]), lo_halves(rb[2][m], rb[3][m])};
      const u32x2 hi{hi_halves(rb[0][m], rb[1][m]), hi_halves(rb[2][m], rb[3][m])};
      *reinterpret_cast<u32x2 *>(Bs + (8 * nq + 2 * m) * BP + 4 * kq) = lo;
      *reinterpret_cast<u32x2 *>(Bs + (8 * nq + 2 * m + 1) * BP + 4 * kq) = hi;
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + GK - 1) / GK;
  load(0);
  store(0);
  __syncthreads();
  const int lrow = lane & 31, lk = 8 * (lane >> 5);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load((kt + 1) * GK);
    const uint16_t *As = smem + (kt & 1) * kStage;
    const uint16_t *Bs = As + GM * AP;
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks) {
      bf16x8 a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(Bs + (64 * wn + 32 * i + lrow) * BP + 16 * ks + lk);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bb[j] = *reinterpret_cast<const bf16x8 *>(As + (64 * wm + 32 * j + lrow) * AP + 16 * ks + lk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], bb[j], acc[i][j]);
    }
    if (kt + 1 < nk) store((kt + 1) & 1);
    __syncthreads();
  }

  // epilogue: registers -> LDS tile [m][n] (bf16) -> 16-byte row stores
  uint16_t *Cs = smem;
  const int half = lane >> 5;
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
  for (int u = 0; u < 8; ++u) {
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
