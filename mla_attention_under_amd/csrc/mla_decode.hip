// Latent-cache decode with a split-KV online-softmax reduction (DeepSpeed PR
// #8602, "Components": decode attention with KV split-K and an online softmax;
// the keys/values are the latent-first up-projection of the cache, torchtitan
// "MLA CP optimization", section "K/V all-gather CP").
//
// The rank's heads all project from ONE cached latent row per position, so the
// up-projection can move from the cache to the query without changing the
// result (associativity of the sums):
//   q_nope . (c_j W_k[h]) = (W_k[h] q_nope) . c_j        (W_k[h]: the k_nope columns of head h)
//   sum_j p_j (c_j W_v[h]) = (sum_j p_j c_j) W_v[h]      (W_v[h]: the v columns of head h)
// Three kernels:
//   1. absorb   : q_abs[b][h] = [W_k[h] q_nope[b][h] | q_rope[b][h]]   (bf16, L+R wide)
//   2. split    : per (sequence, chunk): scores of all heads against the
//                 chunk's [latent | rope] rows with 16x16x32 MFMAs (heads are
//                 the MFMA N dimension), online softmax over 64-key tiles, and
//                 o_c = sum_j p_j c_j / l_c in the latent space; writes m_c, l_c, o_c.
//   3. combine  : m = max m_c, l = sum l_c 2^(m_c - m), o_lat = sum l_c 2^(m_c-m) o_c / l,
//                 out[b][h] = o_lat W_v[h], lse = (m + log2 l) ln 2.
// The cache is read exactly once, so the step is bound by HBM bandwidth on
// the cache; the weight is read once per head.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "mla_common.cuh"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int DL = 512;          // latent width the split kernel is built for
constexpr int DR = 64;           // rope width
constexpr int DK = DL + DR;      // score width (576)
constexpr int DH = 16;           // heads per MFMA column block
constexpr int DT = 64;           // keys per tile
constexpr int CKP = DK + 8;      // LDS pitch of key-major rows [key][dim]
constexpr int CTP = DT + 8;      // LDS pitch of dim-major rows [dim][key]
constexpr int PSP = DT + 8;      // LDS pitch of P rows [head][key]
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeWs {
  size_t qabs, m, l, o, bytes;
};
DecodeWs decode_ws(int B, int H, int L, int R, int splits) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  DecodeWs w;
  const size_t bh = static_cast<size_t>(B) * H;
  w.qabs = 0;
  w.m = up(bh * (L + R) * 2);
  w.l = w.m + up(bh * splits * 4);
  w.o = w.l + up(bh * splits * 4);
  w.bytes = w.o + up(bh * splits * L * 4);
  return w;
}

// ---- 1. absorb: one workgroup per (head, group of sequences); thread per latent column
__global__ __launch_bounds__(512) void decode_absorb_kernel(const uint16_t *__restrict__ q,
                                                            const uint16_t *__restrict__ w, uint16_t *__restrict__ qabs,
                                                            int B, int H, int L, int N, int V, int R, int64_t ldw,
                                                            int64_t col0, int bpb) {
  extern __shared__ float qs[];   // q_nope of the current sequence, [N]
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * bpb;
  const int64_t kcol = col0 + static_cast<int64_t>(h) * (N + V);   // first k_nope column of head h
  for (int b = b0; b < min(B, b0 + bpb); ++b) {
    const uint16_t *qp = q + (static_cast<int64_t>(b) * H + h) * (N + R);
    __syncthreads();
    for (int n = threadIdx.x; n < N; n += blockDim.x) qs[n] = bf16_to_f32(qp[n]);
    __syncthreads();
    uint16_t *out = qabs + (static_cast<int64_t>(b) * H + h) * (L + R);
    for (int l = threadIdx.x; l < L; l += blockDim.x) {
      const uint16_t *wr = w + static_cast<int64_t>(l) * ldw + kcol;
      float acc = 0.f;
      for (int n = 0; n < N; ++n) acc += bf16_to_f32(wr[n]) * qs[n];
      out[l] = f32_to_bf16(acc);
    }
    for (int r = threadIdx.x; r < R; r += blockDim.x) out[L + r] = qp[N + r];
  }
}

// ---- 2. split-KV over the latent cache
struct SplitArgs {
  const uint16_t *qabs;   // [B][H][DK]
  const uint16_t *c;      // [B][S][DL]
  const uint16_t *kr;     // [B][S][DR]
  float *m, *l, *o;       // [B][H][splits], [B][H][splits], [B][H][splits][DL]
  int64_t S;
  int H, splits;
  float scale_log2;
};

// dim-major V^T layout: 8-key column groups are XOR-swizzled by (row/8)%8 so the
// transposing stores of 64 lanes spread over the banks
__device__ __forceinline__ int ct_col(int row, int col) { return col ^ (((row >> 3) & 7) << 3); }

__global__ __launch_bounds__(256) void decode_split_kernel(SplitArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ck[DT * CKP];
  __shared__ __attribute__((aligned(16))) uint16_t Ct[DL * CTP];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[DH * PSP];
  __shared__ float red[4][DH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int b = blockIdx.x / a.splits, cidx = blockIdx.x % a.splits;
  const int64_t chunk = (a.S + a.splits - 1) / a.splits;
  const int64_t k_lo = std::min<int64_t>(a.S, cidx * chunk);
  const int64_t k_hi = std::min<int64_t>(a.S, k_lo + chunk);
  const int n_tiles = static_cast<int>((k_hi - k_lo + DT - 1) / DT);

  // Q^T fragments (B operand): head l16, dims 32*ks + 8*g4 .. +7
  bf16x8 qf[DK / 32];
  {
    const bool hv = l16 < a.H;
    const uint16_t *qp = a.qabs + (static_cast<int64_t>(b) * a.H + (hv ? l16 : 0)) * DK;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks)
      qf[ks] = as_bf16x8(hv ? *reinterpret_cast<const u32x4 *>(qp + 32 * ks + 8 * g4) : u32x4{0, 0, 0, 0});
  }

  const uint16_t *cb = a.c + static_cast<int64_t>(b) * a.S * DL;
  const uint16_t *kb = a.kr + static_cast<int64_t>(b) * a.S * DR;
  u32x4 rc[4][4];
  u32x4 rr[2];
  auto load = [&](int64_t j0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = tid + 256 * u;
      const int dq = g & 63, kq = g >> 6;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t j = j0 + 4 * kq + r;
        rc[u][r] = j < k_hi ? *reinterpret_cast<const u32x4 *>(cb + j * DL + 8 * dq) : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cc = tid + 256 * u;
      const int64_t j = j0 + (cc >> 3);
      rr[u] = j < k_hi ? *reinterpret_cast<const u32x4 *>(kb + j * DR + 8 * (cc & 7)) : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = tid + 256 * u;
      const int dq = g & 63, kq = g >> 6;
#pragma unroll
      for (int r = 0; r < 4; ++r) *reinterpret_cast<u32x4 *>(Ck + (4 * kq + r) * CKP + 8 * dq) = rc[u][r];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int row0 = 8 * dq + 2 * m;
        const u32x2 lo{lo_halves(rc[u][0][m], rc[u][1][m]), lo_halves(rc[u][2][m], rc[u][3][m])};
        const u32x2 hi{hi_halves(rc[u][0][m], rc[u][1][m]), hi_halves(rc[u][2][m], rc[u][3][m])};
        *reinterpret_cast<u32x2 *>(Ct + row0 * CTP + ct_col(row0, 4 * kq)) = lo;
        *reinterpret_cast<u32x2 *>(Ct + (row0 + 1) * CTP + ct_col(row0 + 1, 4 * kq)) = hi;
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cc = tid + 256 * u;
      *reinterpret_cast<u32x4 *>(Ck + (cc >> 3) * CKP + DL + 8 * (cc & 7)) = rr[u];
    }
  };

  f32x4 o[8];   // O^T for dims 128*wave + 16*db + 4*g4 + r, head l16
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -1.0e30f, l_run = 0.f;
  const float cs = a.scale_log2;

  if (n_tiles > 0) {
    load(k_lo);
    store();
  }
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int64_t j0 = k_lo + static_cast<int64_t>(t) * DT;
    if (t + 1 < n_tiles) load(j0 + DT);
    // S^T for keys 16*wave .. +15, all heads
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(Ck + (16 * wave + l16) * CKP + 32 * ks + 8 * g4);
      s = mfma16(kf, qf[ks], s);
    }
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t j = j0 + 16 * wave + 4 * g4 + r;
      s[r] = j < k_hi ? s[r] * cs : -INFINITY;
      mt = fmaxf(mt, s[r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    if (g4 == 0) red[wave][l16] = mt;
    __syncthreads();
    mt = fmaxf(fmaxf(red[0][l16], red[1][l16]), fmaxf(red[2][l16], red[3][l16]));
    const float mn = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
    m_run = mn;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(s[r] - mn);
    l_run = l_run * alpha + (p[0] + p[1]) + (p[2] + p[3]);
    *reinterpret_cast<u32x2 *>(Ps + l16 * PSP + 16 * wave + 4 * g4) = u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] *= alpha;
    __syncthreads();
    // O^T[dims][heads] += C^T[dims][keys] P^T[keys][heads]
#pragma unroll
    for (int ks = 0; ks < DT / 32; ++ks) {
      const bf16x8 pf = *reinterpret_cast<const bf16x8 *>(Ps + l16 * PSP + 32 * ks + 8 * g4);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const int row = 128 * wave + 16 * d + l16;
        const bf16x8 cf = *reinterpret_cast<const bf16x8 *>(Ct + row * CTP + ct_col(row, 32 * ks + 8 * g4));
        o[d] = mfma16(cf, pf, o[d]);
      }
    }
    __syncthreads();
    if (t + 1 < n_tiles) {
      store();
      __syncthreads();
    }
  }

  // chunk partials: row sum over all lanes and waves of each head
  float lsum = l_run + __shfl_xor(l_run, 16);
  lsum += __shfl_xor(lsum, 32);
  __syncthreads();
  if (g4 == 0) red[wave][l16] = lsum;
  __syncthreads();
  const float l_c = (red[0][l16] + red[1][l16]) + (red[2][l16] + red[3][l16]);
  if (l16 >= a.H) return;
  const int64_t bh = static_cast<int64_t>(b) * a.H + l16;
  const float inv = l_c > 0.f ? 1.f / l_c : 0.f;
  float *op = a.o + (bh * a.splits + cidx) * DL;
#pragma unroll
  for (int d = 0; d < 8; ++d)
    *reinterpret_cast<f32x4 *>(op + 128 * wave + 16 * d + 4 * g4) = o[d] * inv;
  if (wave == 0 && g4 == 0) {
    a.m[bh * a.splits + cidx] = n_tiles > 0 ? m_run : -INFINITY;
    a.l[bh * a.splits + cidx] = l_c;
  }
}

// ---- 3. combine chunks and project the latent output through W_v
__global__ __launch_bounds__(256) void decode_combine_kernel(const float *__restrict__ m, const float *__restrict__ l,
                                                             const float *__restrict__ o,
                                                             const uint16_t *__restrict__ w, uint16_t *__restrict__ out,
                                                             float *__restrict__ lse, int H, int splits, int L, int N,
                                                             int V, int64_t ldw, int64_t col0) {
  extern __shared__ float ol[];   // [L]
  const int bh = blockIdx.x;
  const int h = bh % H;
  const float *mp = m + static_cast<int64_t>(bh) * splits;
  const float *lp = l + static_cast<int64_t>(bh) * splits;
  float mx = -INFINITY;
  for (int c = 0; c < splits; ++c) mx = fmaxf(mx, mp[c]);
  float den = 0.f;
  for (int c = 0; c < splits; ++c) den += lp[c] * __builtin_amdgcn_exp2f(mp[c] - mx);
  const float inv = den > 0.f ? 1.f / den : 0.f;
  for (int d = threadIdx.x; d < L; d += blockDim.x) {
    float acc = 0.f;
    for (int c = 0; c < splits; ++c) {
      const float wgt = lp[c] * __builtin_amdgcn_exp2f(mp[c] - mx);
      acc += wgt * o[(static_cast<int64_t>(bh) * splits + c) * L + d];
    }
    ol[d] = acc * inv;
  }
  __syncthreads();
  const int64_t vcol = col0 + static_cast<int64_t>(h) * (N + V) + N;
  for (int v = threadIdx.x; v < V; v += blockDim.x) {
    float acc = 0.f;
    for (int d = 0; d < L; ++d) acc += ol[d] * bf16_to_f32(w[static_cast<int64_t>(d) * ldw + vcol + v]);
    out[static_cast<int64_t>(bh) * V + v] = f32_to_bf16(acc);
  }
  if (lse != nullptr && threadIdx.x == 0) lse[bh] = (mx + __builtin_amdgcn_logf(den)) * 0.6931471805599453f;
}

}  // namespace

bool decode_supported(int L, int N, int R, int V) { return L == DL && R == DR && N >= 1 && V >= 1; }

size_t decode_workspace_bytes(int B, int H, int L, int N, int R, int V, int splits) {
  (void)N;
  (void)V;
  return decode_ws(B, H, L, R, splits).bytes;
}

int launch_decode(const DecodePlan &p, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.H > DH) return hipErrorInvalidValue;
  const DecodeWs w = decode_ws(p.B, p.H, p.L, p.R, p.splits);
  char *ws = static_cast<char *>(p.ws);
  uint16_t *qabs = reinterpret_cast<uint16_t *>(ws + w.qabs);
  float *wm = reinterpret_cast<float *>(ws + w.m);
  float *wl = reinterpret_cast<float *>(ws + w.l);
  float *wo = reinterpret_cast<float *>(ws + w.o);
  const int bpb = 8;
  hipLaunchKernelGGL(decode_absorb_kernel, dim3(p.H, (p.B + bpb - 1) / bpb), dim3(512), p.N * sizeof(float), s,
                     static_cast<const uint16_t *>(p.q), static_cast<const uint16_t *>(p.w), qabs, p.B, p.H, p.L,
                     p.N, p.V, p.R, p.ldw, p.col0, bpb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SplitArgs a;
  a.qabs = qabs;
  a.c = static_cast<const uint16_t *>(p.c);
  a.kr = static_cast<const uint16_t *>(p.kr);
  a.m = wm;
  a.l = wl;
  a.o = wo;
  a.S = p.S;
  a.H = p.H;
  a.splits = p.splits;
  a.scale_log2 = p.scale * kLog2e;
  hipLaunchKernelGGL(decode_split_kernel, dim3(p.B * p.splits), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(p.B * p.H), dim3(256), p.L * sizeof(float), s, wm, wl, wo,
                     static_cast<const uint16_t *>(p.w), static_cast<uint16_t *>(p.out), p.lse, p.H, p.splits, p.L,
                     p.N, p.V, p.ldw, p.col0);
  return hipGetLastError();
}

}  // namespace mla
