// Backward of the shard's attention with the head-shared RoPE key band
// (torchtitan "MLA CP optimization", section "Numerical comparison": the
// method is trained, so the shard is differentiated; hyper-parallel
// `_assemble_key_value`: the band is one tensor repeated over the heads, so
// its gradient is the sum of every head's band gradient).
//
// Per head, with p the probabilities recomputed from the forward's
// log-sum-exp, the row term D_t = sum_v dout[t][v] out[t][v], and k the key
// [k_nope | k_rope]:
//   dv = p^T dout, dp = dout v^T, ds = p (dp - D), dq = scale ds k,
//   dk = scale ds^T q; dk_rope = sum over heads of dk[..., N:].
//
// Three launches, all on blocks of 32 keys by 32 queries with the score block
// kept transposed (keys are rows, queries are the lanes' columns, so a lane's
// log-sum-exp and row term are one register each):
//   row_term_kernel   D[h][t] from out and dout;
//   attn_bwd_kernel   one workgroup (two waves) per (block b, head), two
//                     phases: dk, dv of key block b accumulated over the query
//                     blocks that see it (the band part of dk goes to a
//                     per-head slice of the workspace), then dq of query block
//                     b accumulated over the key blocks it sees (scores
//                     recomputed rather than reduced across workgroups, so no
//                     atomics and a fixed summation order). Under the causal
//                     mask key block b is seen by nb - b query blocks and query
//                     block b sees b + 1 key blocks, so every workgroup carries
//                     the same nb + 1 block steps and the grid drains evenly;
//   band_sum_kernel   dk_rope[t] = sum over heads of the band slices, in head
//                     order.
// Then the latent up-projection's backward (dlatent_kernel, dw_kernel): the
// gradients of the latent and of the head range's weight columns.
// The five products per block are bf16 MFMAs (v_mfma_f32_32x32x16_bf16) with
// fp32 accumulation; p and ds are rounded to bf16 as MFMA operands.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int BB = 32;          // keys or queries per block
constexpr int TP = BB + 8;      // pitch of the 32x32 p / ds blocks in LDS, in bf16
constexpr float kLog2e = 1.4426950408889634f;

struct BwdArgs {
  const uint16_t *q, *kv, *kr, *out, *dout;
  int64_t q_st, q_sh, kv_st, kv_sh, kr_st, o_st, o_sh, do_st, do_sh;   // in elements
  const float *lse;     // [H][T], natural log
  float *dq, *dkv;      // [T][H][N+R], [T][H][N+V]
  float *dkr;           // [T][R]
  float *Dws;           // [H][T] row terms
  float *band;          // [H][T][R] per-head band gradients
  const int32_t *cu;
  int n_seq;
  int T, H;
  float scale;
  int causal;
};

// document [lo, hi) holding token t (one document of T tokens without cu);
// the bounds are clamped to [0, T], so malformed offsets give wrong documents,
// never an access outside the buffers
__device__ __forceinline__ void doc_of(const BwdArgs &a, int t, int &lo, int &hi) {
  if (a.cu == nullptr) {
    lo = 0;
    hi = a.T;
    return;
  }
  int l = 0, r = a.n_seq;   // largest d with cu[d] <= t lies in [l, r)
  while (r - l > 1) {
    const int m = (l + r) >> 1;
    if (a.cu[m] <= t) l = m;
    else r = m;
  }
  lo = min(max(a.cu[l], 0), a.T);
  hi = min(max(a.cu[l + 1], lo), a.T);
}

// MFMA operands straight from memory: fragment s of lane l is row r0 + l%32
// (zero at or past lim), elements 16s + 8*(l/32) .. +7 of that row; the
// fragments of W columns are one 16-byte load each.
template <int W>
__device__ __forceinline__ void load_frags(const uint16_t *src, int64_t st, int r0, int lim, bf16x8 *f, int lane) {
  const int r = r0 + (lane & 31);
  const bool ok = r >= 0 && r < lim;
  const uint16_t *row = src + static_cast<int64_t>(ok ? r : 0) * st + 8 * (lane >> 5);
#pragma unroll
  for (int s = 0; s < W / 16; ++s)
    f[s] = ok ? *reinterpret_cast<const bf16x8 *>(row + 16 * s) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
}

// Fragments (see load_frags) to a row-major LDS block of pitch P: one 16-byte
// store each.
template <int W>
__device__ __forceinline__ void store_rows(const bf16x8 *f, uint16_t *dst, int P, int lane) {
#pragma unroll
  for (int s = 0; s < W / 16; ++s)
    *reinterpret_cast<bf16x8 *>(dst + (lane & 31) * P + 16 * s + 8 * (lane >> 5)) = f[s];
}

// Transposing LDS reads (gfx950 ds_read_b64_tr_b16): lane i of each 16-lane
// group receives column i of the 4x16 block whose rows its lanes address.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ s16x4 read_tr(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}

// MFMA operand of contraction step b (rows 16b .. 16b+15 of a row-major
// [row][column] LDS block of pitch P) for the 32 columns 32d + l%32, read
// transposed. Element m of lane l comes from row 16b + 8(m/4) + 4(l/32) + m%4:
// the other operand of the product must list its contraction index in the
// same order (perm_frag).
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t *tile, int P, int b, int d, int lane) {
  const int grp = lane >> 4, gl = lane & 15;
  const int col = 32 * d + 16 * (grp & 1) + 4 * (gl & 3);
  const int r0 = 4 * (grp >> 1) + (gl >> 2) + 16 * b;
  const s16x4 lo = read_tr(tile + r0 * P + col), hi = read_tr(tile + (r0 + 8) * P + col);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// The matching operand from a row-major [i][k] LDS block of pitch P: row l%32,
// elements 16b + 4(l/32) .. +3 and 16b + 8 + 4(l/32) .. +3 (tr_frag's order).
__device__ __forceinline__ bf16x8 perm_frag(const uint16_t *m, int P, int b, int lane) {
  const uint16_t *row = m + (lane & 31) * P + 16 * b + 4 * (lane >> 5);
  const u32x2 lo = *reinterpret_cast<const u32x2 *>(row), hi = *reinterpret_cast<const u32x2 *>(row + 8);
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// row i of the block held in register r of lane l (column l%32)
__device__ __forceinline__ int row_of(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// p^T and ds^T of one block, from the transposed scores and dp^T:
//   p = exp(scale*s - lse_j), ds = p (dp - D_j), zero where key i is not
// visible to query j (another document, past the diagonal, past T).
__device__ __forceinline__ void probs_t(const BwdArgs &a, f32x16 &st, f32x16 &dp, int k0, int q, int qlo, int qhi,
                                        float lse2, float Dq, int lane) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = k0 + row_of(r, lane);
    const bool vis = key >= qlo && key < qhi && (!a.causal || key <= q);
    const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], a.scale * kLog2e, -lse2)) : 0.f;
    st[r] = p;
    dp[r] = p * (dp[r] - Dq);
  }
}

// block values (C layout) to a row-major bf16 LDS block [i][j], or its transpose
__device__ __forceinline__ void store_block(const f32x16 &v, uint16_t *m, bool transpose, int lane) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = row_of(r, lane), j = lane & 31;
    m[transpose ? j * TP + i : i * TP + j] = f32_to_bf16(v[r]);
  }
}

__global__ __launch_bounds__(256) void row_term_kernel(BwdArgs a, int V) {
  // 16 lanes per (t, h) row, 8 elements each per pass
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = gid >> 4;
  const int c = static_cast<int>(gid & 15);
  const bool live = row < static_cast<int64_t>(a.T) * a.H;
  const int t = live ? static_cast<int>(row / a.H) : 0, h = live ? static_cast<int>(row % a.H) : 0;
  float acc = 0.f;
  if (live) {
    const uint16_t *o = a.out + t * a.o_st + h * a.o_sh;
    const uint16_t *g = a.dout + t * a.do_st + h * a.do_sh;
    for (int k = 8 * c; k < V; k += 128) {
      const u32x4 ov = *reinterpret_cast<const u32x4 *>(o + k);
      const u32x4 gv = *reinterpret_cast<const u32x4 *>(g + k);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(bf16_elem(ov, e), bf16_elem(gv, e), acc);
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (live && c == 0) a.Dws[static_cast<int64_t>(h) * a.T + t] = acc;
}

// LDS of a workgroup: the dk/dv phase's q, dout (row-major, read back
// transposed), p^T and ds^T blocks, or the dq phase's k and ds blocks; rows
// padded by 8 elements
template <int K, int V>
constexpr int kBwdLds = BB * (K + 8) + BB * (V + 8) + 2 * BB * TP;

// Two waves per (block b, head), each under 256 VGPRs so that two waves share
// a SIMD and cover each other's barriers and LDS round trips. Wave 0 holds the
// key (or query) side of the scores: it computes s, then p and ds, and the
// first KS column tiles of dk (or dq); wave 1 holds the value side: dp, which
// it hands over through LDS in its own register layout, then dv and the last
// column tiles of dk (or dq). Each wave runs its own loop; the two meet at the
// same three barriers per block step:
//   (1) the previous step's readers are done; row-major copies and the s / dp
//       products, the next block's loads issued;
//   (2) dp is in LDS; wave 0 forms p and ds into LDS;
//   (3) the second-stage products of both waves.
// Workgroups are dealt to the 8 XCDs round robin by launch order; when the
// grid divides evenly, launch slot i is remapped so that each XCD runs a
// contiguous run of (head, block) pairs, i.e. whole heads, whose q, k, v and
// dout then stay in that XCD's L2 instead of every XCD streaming every head.
template <int N, int R, int V>
__global__ __launch_bounds__(128, 2) void attn_bwd_kernel(BwdArgs a) {
  constexpr int K = N + R;
  constexpr int KS = 4;   // dk / dq column tiles of wave 0 (the rest go to wave 1)
  static_assert(K / 32 > KS, "both waves own dk columns");
  __shared__ __attribute__((aligned(16))) uint16_t lds[kBwdLds<K, V>];
  __shared__ __attribute__((aligned(16))) float dps[16 * 64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nb = gridDim.x, G = nb * gridDim.y;
  int lin = blockIdx.x + nb * blockIdx.y;
  if (G % 8 == 0) lin = (lin % 8) * (G / 8) + lin / 8;
  const int h = lin / nb, b0 = (lin % nb) * BB;
  const int b1 = min(b0 + BB, a.T) - 1;
  int lo0, hi0, lo1, hi1;
  doc_of(a, b0, lo0, hi0);
  doc_of(a, b1, lo1, hi1);

  // ---- phase 1: dk, dv of key block b0
  {
    constexpr int KP = K + 8, VP = V + 8;
    uint16_t *const Qs = lds, *const Os = Qs + BB * KP, *const Ps = Os + BB * VP, *const Ss = Ps + BB * TP;
    const int qbeg = __builtin_amdgcn_readfirstlane(a.causal ? b0 : lo0);
    const int qend = __builtin_amdgcn_readfirstlane(hi1);
    if (wave == 0) {
      bf16x8 kf[K / 16], qf[K / 16];
      float lse_n = 0.f, D_n = 0.f;
      auto rows_terms = [&](int q0) {
        const int q = q0 + (lane & 31);
        const int64_t i = static_cast<int64_t>(h) * a.T + (q < a.T ? q : 0);
        lse_n = a.lse[i];
        D_n = a.Dws[i];
      };
      load_frags<N>(a.kv + h * a.kv_sh, a.kv_st, b0, a.T, kf, lane);
      if constexpr (R > 0) load_frags<R>(a.kr, a.kr_st, b0, a.T, kf + N / 16, lane);
      if (qbeg < qend) {
        load_frags<K>(a.q + h * a.q_sh, a.q_st, qbeg, a.T, qf, lane);
        rows_terms(qbeg);
      }
      f32x16 dk[KS] = {};
      for (int q0 = qbeg; q0 < qend; q0 += BB) {
        const int q = q0 + (lane & 31);
        int qlo = 1, qhi = 0;
        if (q < a.T) doc_of(a, q, qlo, qhi);
        const float lse2 = lse_n * kLog2e, Dq = D_n;
        __syncthreads();                                   // (1)
        store_rows<K>(qf, Qs, KP, lane);
        f32x16 st = {};
#pragma unroll
        for (int s = 0; s < K / 16; ++s) st = mfma32(kf[s], qf[s], st);
        if (q0 + BB < qend) {
          load_frags<K>(a.q + h * a.q_sh, a.q_st, q0 + BB, a.T, qf, lane);
          rows_terms(q0 + BB);
        }
        __syncthreads();                                   // (2)
        f32x16 dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = dps[r * 64 + lane];
        probs_t(a, st, dp, b0, q, qlo, qhi, lse2, Dq, lane);
        store_block(st, Ps, false, lane);   // p^T [key][query]
        store_block(dp, Ss, false, lane);   // ds^T [key][query]
        __syncthreads();                                   // (3)
#pragma unroll
        for (int s = 0; s < BB / 16; ++s) {
          const bf16x8 sa = perm_frag(Ss, TP, s, lane);
#pragma unroll
          for (int kt = 0; kt < KS; ++kt) dk[kt] = mfma32(sa, tr_frag(Qs, KP, s, kt, lane), dk[kt]);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = b0 + row_of(r, lane);
        if (key >= a.T) continue;
        float *row = a.dkv + (static_cast<int64_t>(key) * a.H + h) * (N + V);
        float *brow = a.band + (static_cast<int64_t>(h) * a.T + key) * R;
#pragma unroll
        for (int kt = 0; kt < KS; ++kt) {
          const int c = 32 * kt + (lane & 31);
          const float g = a.scale * dk[kt][r];
          if (c < N) row[c] = g;
          else brow[c - N] = g;
        }
      }
    } else {
      bf16x8 vf[V / 16], gf[V / 16];
      load_frags<V>(a.kv + h * a.kv_sh + N, a.kv_st, b0, a.T, vf, lane);
      if (qbeg < qend) load_frags<V>(a.dout + h * a.do_sh, a.do_st, qbeg, a.T, gf, lane);
      f32x16 dv[V / 32] = {}, dk[K / 32 - KS] = {};
      for (int q0 = qbeg; q0 < qend; q0 += BB) {
        __syncthreads();                                   // (1)
        store_rows<V>(gf, Os, VP, lane);
        f32x16 dp = {};
#pragma unroll
        for (int s = 0; s < V / 16; ++s) dp = mfma32(vf[s], gf[s], dp);
        if (q0 + BB < qend) load_frags<V>(a.dout + h * a.do_sh, a.do_st, q0 + BB, a.T, gf, lane);
#pragma unroll
        for (int r = 0; r < 16; ++r) dps[r * 64 + lane] = dp[r];
        __syncthreads();                                   // (2)
        __syncthreads();                                   // (3)
#pragma unroll
        for (int s = 0; s < BB / 16; ++s) {
          const bf16x8 pa = perm_frag(Ps, TP, s, lane), sa = perm_frag(Ss, TP, s, lane);
#pragma unroll
          for (int vt = 0; vt < V / 32; ++vt) dv[vt] = mfma32(pa, tr_frag(Os, VP, s, vt, lane), dv[vt]);
#pragma unroll
          for (int kt = KS; kt < K / 32; ++kt)
            dk[kt - KS] = mfma32(sa, tr_frag(Qs, KP, s, kt, lane), dk[kt - KS]);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = b0 + row_of(r, lane);
        if (key >= a.T) continue;
        float *row = a.dkv + (static_cast<int64_t>(key) * a.H + h) * (N + V);
        float *brow = a.band + (static_cast<int64_t>(h) * a.T + key) * R;
#pragma unroll
        for (int kt = KS; kt < K / 32; ++kt) {
          const int c = 32 * kt + (lane & 31);
          const float g = a.scale * dk[kt - KS][r];
          if (c < N) row[c] = g;
          else brow[c - N] = g;
        }
#pragma unroll
        for (int vt = 0; vt < V / 32; ++vt) row[N + 32 * vt + (lane & 31)] = dv[vt][r];
      }
    }
  }
  __syncthreads();   // phase 1's readers are done with the LDS

  // ---- phase 2: dq of query block b0
  {
    constexpr int KP = K + 8;
    uint16_t *const Ks = lds, *const Ss = Ks + BB * KP;
    const int kbeg = __builtin_amdgcn_readfirstlane(lo0);
    const int kend = __builtin_amdgcn_readfirstlane(a.causal ? b1 + 1 : hi1);
    if (wave == 0) {
      bf16x8 kf[K / 16], qf[K / 16];
      load_frags<K>(a.q + h * a.q_sh, a.q_st, b0, a.T, qf, lane);
      auto load_k = [&](int k0) {
        load_frags<N>(a.kv + h * a.kv_sh, a.kv_st, k0, a.T, kf, lane);
        if constexpr (R > 0) load_frags<R>(a.kr, a.kr_st, k0, a.T, kf + N / 16, lane);
      };
      if (kbeg < kend) load_k(kbeg);
      const int q = b0 + (lane & 31);
      int qlo = 1, qhi = 0;
      float lse2 = 0.f, Dq = 0.f;
      if (q < a.T) {
        doc_of(a, q, qlo, qhi);
        lse2 = a.lse[static_cast<int64_t>(h) * a.T + q] * kLog2e;
        Dq = a.Dws[static_cast<int64_t>(h) * a.T + q];
      }
      f32x16 dq[KS] = {};
      for (int k0 = kbeg; k0 < kend; k0 += BB) {
        __syncthreads();                                   // (1)
        store_rows<K>(kf, Ks, KP, lane);
        f32x16 st = {};
#pragma unroll
        for (int s = 0; s < K / 16; ++s) st = mfma32(kf[s], qf[s], st);
        if (k0 + BB < kend) load_k(k0 + BB);
        __syncthreads();                                   // (2)
        f32x16 dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = dps[r * 64 + lane];
        probs_t(a, st, dp, k0, q, qlo, qhi, lse2, Dq, lane);
        store_block(dp, Ss, true, lane);   // ds [query][key]
        __syncthreads();                                   // (3)
#pragma unroll
        for (int s = 0; s < BB / 16; ++s) {
          const bf16x8 sa = perm_frag(Ss, TP, s, lane);
#pragma unroll
          for (int kt = 0; kt < KS; ++kt) dq[kt] = mfma32(sa, tr_frag(Ks, KP, s, kt, lane), dq[kt]);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = b0 + row_of(r, lane);
        if (t >= a.T) continue;
        float *row = a.dq + (static_cast<int64_t>(t) * a.H + h) * K;
#pragma unroll
        for (int kt = 0; kt < KS; ++kt) row[32 * kt + (lane & 31)] = a.scale * dq[kt][r];
      }
    } else {
      bf16x8 vf[V / 16], gf[V / 16];
      load_frags<V>(a.dout + h * a.do_sh, a.do_st, b0, a.T, gf, lane);
      if (kbeg < kend) load_frags<V>(a.kv + h * a.kv_sh + N, a.kv_st, kbeg, a.T, vf, lane);
      f32x16 dq[K / 32 - KS] = {};
      for (int k0 = kbeg; k0 < kend; k0 += BB) {
        __syncthreads();                                   // (1)
        f32x16 dp = {};
#pragma unroll
        for (int s = 0; s < V / 16; ++s) dp = mfma32(vf[s], gf[s], dp);
        if (k0 + BB < kend) load_frags<V>(a.kv + h * a.kv_sh + N, a.kv_st, k0 + BB, a.T, vf, lane);
#pragma unroll
        for (int r = 0; r < 16; ++r) dps[r * 64 + lane] = dp[r];
        __syncthreads();                                   // (2)
        __syncthreads();                                   // (3)
#pragma unroll
        for (int s = 0; s < BB / 16; ++s) {
          const bf16x8 sa = perm_frag(Ss, TP, s, lane);
#pragma unroll
          for (int kt = KS; kt < K / 32; ++kt)
            dq[kt - KS] = mfma32(sa, tr_frag(Ks, KP, s, kt, lane), dq[kt - KS]);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = b0 + row_of(r, lane);
        if (t >= a.T) continue;
        float *row = a.dq + (static_cast<int64_t>(t) * a.H + h) * K;
#pragma unroll
        for (int kt = KS; kt < K / 32; ++kt) row[32 * kt + (lane & 31)] = a.scale * dq[kt - KS][r];
      }
    }
  }
}

// four consecutive band elements per thread (R is a multiple of 4), the heads
// added in order, four heads' loads in flight at a time
__global__ __launch_bounds__(256) void band_sum_kernel(BwdArgs a, int R) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = static_cast<int64_t>(a.T) * R / 4, stride = static_cast<int64_t>(a.T) * R / 4;
  if (i >= n) return;
  const f32x4 *src = reinterpret_cast<const f32x4 *>(a.band) + i;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int h = 0;
  for (; h + 4 <= a.H; h += 4) {
    const f32x4 x0 = src[h * stride], x1 = src[(h + 1) * stride], x2 = src[(h + 2) * stride], x3 = src[(h + 3) * stride];
    acc += x0;
    acc += x1;
    acc += x2;
    acc += x3;
  }
  for (; h < a.H; ++h) acc += src[h * stride];
  reinterpret_cast<f32x4 *>(a.dkr)[i] = acc;
}

// ---- backward of the latent up-projection -------------------------------
// kv[t][c] = sum_l latent[t][l] w[l][col0 + c] over the head range's columns c,
// so d_latent = dkv w_cols^T and dw_cols = latent^T dkv. dkv arrives in fp32
// and is rounded to bf16 as an MFMA operand; both products accumulate in fp32.

struct UpBwdArgs {
  const uint16_t *latent, *w;
  const float *dkv;
  float *dl, *dw;
  int T, L, C;         // C = heads*(N+V)
  int64_t ldw, col0;   // w row length and the range's first column
};

// eight fp32 values -> one bf16 operand fragment (round to nearest even)
__device__ __forceinline__ bf16x8 f32x8_to_bf16(const f32x4 &lo, const f32x4 &hi) {
  return as_bf16x8(u32x4{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                         pack_bf16x2(hi[2], hi[3])});
}


// d_latent[t][l] = sum_c dkv[t][c] w[l][col0 + c]: both operands are
// contiguous along the contraction c. A 4-wave workgroup owns 64 tokens x 64
// latent columns (32 x 32 per wave); each 128-column stage of dkv (rounded to
// bf16) and of the weight rows is stored row-major to LDS, double-buffered,
// and read back as ordinary row fragments, the next stage's global loads in
// flight during the current stage's products.
constexpr int kDlM = 64, kDlN = 64, kDlK = 128, kDlP = kDlK + 8;  // rows, columns, stage, LDS pitch
constexpr int kDlJ = kDlN / 64;                                     // 32-column tiles per wave
__global__ __launch_bounds__(256) void dlatent_kernel(UpBwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kDlM * kDlP], Bs[2][kDlN * kDlP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.x * kDlM, l0 = blockIdx.y * kDlN;
  // thread unit u = tid + 256 i covers row u / kCH, columns 8 (u % kCH) .. +7 of a stage
  constexpr int kCH = kDlK / 8, kAU = kDlM * kCH / 256;   // 16-byte chunks per row, dkv chunks per thread
  f32x4 areg[kAU][2];
  constexpr int kBU = kDlN * kCH / 256;   // weight chunks per thread
  u32x4 breg[kBU];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kAU; ++i) {
      const int u = tid + 256 * i, r = u / kCH, c8 = (u % kCH) * 8, t = t0 + r;
      const bool ok = t < a.T && k0 + c8 < a.C;
      const float *g = a.dkv + static_cast<int64_t>(ok ? t : 0) * a.C + k0 + c8;
      areg[i][0] = ok ? *reinterpret_cast<const f32x4 *>(g) : f32x4{};
      areg[i][1] = ok ? *reinterpret_cast<const f32x4 *>(g + 4) : f32x4{};
    }
#pragma unroll
    for (int i = 0; i < kBU; ++i) {
      const int u = tid + 256 * i, r = u / kCH, c8 = (u % kCH) * 8, l = l0 + r;
      const bool ok = l < a.L && k0 + c8 < a.C;
      breg[i] = ok ? *reinterpret_cast<const u32x4 *>(a.w + static_cast<int64_t>(l) * a.ldw + a.col0 + k0 + c8)
                   : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kAU; ++i) {
      const int u = tid + 256 * i, r = u / kCH, c8 = (u % kCH) * 8;
      *reinterpret_cast<u32x4 *>(As[buf] + r * kDlP + c8) = as_u32x4(f32x8_to_bf16(areg[i][0], areg[i][1]));
    }
#pragma unroll
    for (int i = 0; i < kBU; ++i) {
      const int u = tid + 256 * i, r = u / kCH, c8 = (u % kCH) * 8;
      *reinterpret_cast<u32x4 *>(Bs[buf] + r * kDlP + c8) = breg[i];
    }
  };
  // row fragment of contraction step s: row rbase + l%32, elements 16s + 8(l/32) .. +7
  auto rfrag = [&](const uint16_t *m, int rbase, int s) {
    return *reinterpret_cast<const bf16x8 *>(m + (rbase + (lane & 31)) * kDlP + 16 * s + 8 * (lane >> 5));
  };
  f32x16 acc[kDlJ] = {};
  const int nst = (a.C + kDlK - 1) / kDlK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) gload((st + 1) * kDlK);
#pragma unroll
    for (int s = 0; s < kDlK / 16; ++s) {
      const bf16x8 af = rfrag(As[buf], 32 * wm, s);
#pragma unroll
      for (int j = 0; j < kDlJ; ++j) acc[j] = mfma32(af, rfrag(Bs[buf], (kDlN / 2) * wn + 32 * j, s), acc[j]);
    }
    // the other buffer's readers finished before the previous stage's barrier
    if (st + 1 < nst) lstore(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = t0 + 32 * wm + row_of(r, lane);
    if (t >= a.T) continue;
#pragma unroll
    for (int j = 0; j < kDlJ; ++j) {
      const int l = l0 + (kDlN / 2) * wn + 32 * j + (lane & 31);
      if (l < a.L) a.dl[static_cast<int64_t>(t) * a.L + l] = acc[j][r];
    }
  }
}

// dw tiles: [64 tokens][128 columns] bf16, row-major with the 16-element
// blocks of row r XOR-permuted by tr_swz(r) (spreads the transposing reads
// over the banks)
constexpr int kDwM = 64, kDwN = 128, kDwT = 64;   // latent columns (the first kDwM of a 128-wide tile), dkv columns, tokens
constexpr int kDwU = kDwT * 16 / 256;   // 16-byte chunks of each tile per thread and stage
__device__ __forceinline__ int tr_swz(int r) { return (r & 2) | ((r & 1) * 5); }
__device__ __forceinline__ int tr_pos(int r, int c) { return r * 128 + 16 * ((c >> 4) ^ tr_swz(r)) + (c & 15); }

// MFMA operand of 16 tokens (b) by 32 columns (d) from a [token][column] tile:
// lane l takes column 32d + l%32; both operands of dw use the same read, so
// their token orders match.
__device__ __forceinline__ bf16x8 dw_frag(const uint16_t *tile, int b, int d, int lane) {
  const int grp = lane >> 4, gl = lane & 15;
  const int col = 32 * d + 16 * (grp & 1) + 4 * (gl & 3);
  const int r0 = 4 * (grp >> 1) + (gl >> 2) + 16 * b, r1 = r0 + 8;
  const s16x4 lo = read_tr(tile + tr_pos(r0, col)), hi = read_tr(tile + tr_pos(r1, col));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// dw[l][c] = sum_t latent[t][l] dkv[t][c]: the contraction runs over tokens,
// the row index of both operands. A 4-wave workgroup owns 64 x 128 outputs
// (32 x 64 per wave); each 64-token stage of latent and dkv (the latter
// rounded to bf16) is stored row-major to LDS and read back transposed, the
// next stage's global loads in flight during the current stage's products.
__global__ __launch_bounds__(256) void dw_kernel(UpBwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Lt[2][kDwT * 128], Gt[2][kDwT * kDwN];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int c0 = blockIdx.x * kDwN, l0 = blockIdx.y * kDwM;
  u32x4 lreg[kDwU];
  f32x4 greg[kDwU][2];
  // thread unit u = tid + 256 i: tile row u / 16, columns 8 (u % 16) .. +7
  auto gload = [&](int t0) {
#pragma unroll
    for (int i = 0; i < kDwU; ++i) {
      const int u = tid + 256 * i, r = u >> 4, c8 = (u & 15) * 8, t = t0 + r;
      const bool lt = t < a.T && c8 < kDwM && l0 + c8 < a.L, ct = t < a.T && c0 + c8 < a.C;
      lreg[i] = lt ? *reinterpret_cast<const u32x4 *>(a.latent + static_cast<int64_t>(t) * a.L + l0 + c8)
                   : u32x4{0u, 0u, 0u, 0u};
      const float *g = a.dkv + static_cast<int64_t>(ct ? t : 0) * a.C + c0 + c8;
      greg[i][0] = ct ? *reinterpret_cast<const f32x4 *>(g) : f32x4{};
      greg[i][1] = ct ? *reinterpret_cast<const f32x4 *>(g + 4) : f32x4{};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kDwU; ++i) {
      const int u = tid + 256 * i, r = u >> 4, c8 = (u & 15) * 8;
      *reinterpret_cast<u32x4 *>(Lt[buf] + tr_pos(r, c8)) = lreg[i];
      *reinterpret_cast<u32x4 *>(Gt[buf] + tr_pos(r, c8)) = as_u32x4(f32x8_to_bf16(greg[i][0], greg[i][1]));
    }
  };
  f32x16 acc[2] = {};
  const int nst = (a.T + kDwT - 1) / kDwT;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) gload((st + 1) * kDwT);
#pragma unroll
    for (int b = 0; b < kDwT / 16; ++b) {
      const bf16x8 af = dw_frag(Lt[buf], b, wm, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[j] = mfma32(af, dw_frag(Gt[buf], b, 2 * wn + j, lane), acc[j]);
    }
    // the other buffer's readers finished before the previous stage's barrier
    if (st + 1 < nst) lstore(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int l = l0 + 32 * wm + row_of(r, lane);
    if (l >= a.L) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = c0 + 32 * (2 * wn + j) + (lane & 31);
      if (c < a.C) a.dw[static_cast<int64_t>(l) * a.C + c] = acc[j][r];
    }
  }
}

// ---- split contraction for whole tiles -------------------------------------
// With T, L and C multiples of 128 and a workspace, both products run as
// 128x128 output tiles whose contraction is cut into 2S parts of nks 64-wide
// slices. One 8-wave workgroup per CU holds two groups of 4 waves (64x64 each,
// 32x32x16 MFMA); group g of split s multiplies part 2s + g, the second group's
// sums join the first group's through LDS, and the first group writes the fp32
// partial tile of split s (streaming stores: no dirty lines left in L2 for the
// end-of-kernel write-back). split_sum_kernel adds the S partials in split
// order, so the summation order is fixed and the result does not depend on
// scheduling. Each wave issues 16 MFMAs per 64-wide slice against 8 fragment
// reads, where the single-pass kernels above issue one MFMA per two reads.
// Operands move global -> registers -> LDS (bf16, XOR-swizzled), two register
// sets deep and one LDS buffer ahead of the slice being multiplied.
//   d_latent: out[t][l], contraction over c; dkv [t][c] and w [l][col0 + c]
//             are both contiguous along c, stored [row][64] and read as
//             ordinary row fragments;
//   dw:       out[l][c], contraction over t; latent [t][l] and dkv [t][c] are
//             contiguous along the output index, stored [64 t][128] and read
//             back transposed (ds_read_b64_tr_b16).
constexpr int kSM = 128, kSN = 128, kSK = 64;
struct SplitArgs {
  const float *dkv;
  const uint16_t *latent, *w;
  float *out;             // partials [S][M][N], or the output itself when S == 1
  int M, N;               // output rows, columns
  int nks;                // 64-wide slices per split
  int tiles_m, tiles_n;
  int64_t L, C, ldw, col0;
};

__device__ __forceinline__ int rs_swz(int m) { return (m ^ (m >> 3)) & 7; }              // [row][64]: 8 chunks
__device__ __forceinline__ int ts_swz(int k) { return (k & 2) | ((k & 1) * 5); }         // [64][128]: 8 segments
__device__ __forceinline__ int rs_pos(int m, int c8) { return m * kSK + 8 * ((c8 >> 3) ^ rs_swz(m)); }
__device__ __forceinline__ int ts_pos(int k, int c) { return k * kSN + 16 * ((c >> 4) ^ ts_swz(k)) + (c & 15); }

template <bool DW>
__global__ __launch_bounds__(512, 1) void up_bwd_split_kernel(SplitArgs a) {
  // two groups of 4 waves, each with its own double-buffered slices
  __shared__ __attribute__((aligned(1024))) uint16_t lds_all[2 * 2 * (kSM * kSK + kSK * kSN)];
  // consecutive workgroups go to different XCDs (round robin over 8): give
  // each XCD a contiguous run of (split, tile) pairs, so the tiles of one
  // split, which read the same contraction slices, share an L2
  const int G = gridDim.x, bid = blockIdx.x;
  const int lin = G % 8 == 0 ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int tiles = a.tiles_m * a.tiles_n;
  const int split = lin / tiles, tile = lin % tiles;
  const int m0 = (tile % a.tiles_m) * kSM, n0 = (tile / a.tiles_m) * kSN;
  const int grp2 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);   // contraction part 2 split + grp2
  const int kbeg = (2 * split + grp2) * a.nks * kSK;
  uint16_t (*As)[kSM * kSK] = reinterpret_cast<uint16_t (*)[kSM * kSK]>(lds_all + grp2 * 2 * (kSM * kSK + kSK * kSN));
  uint16_t (*Bs)[kSK * kSN] = reinterpret_cast<uint16_t (*)[kSK * kSN]>(lds_all + grp2 * 2 * (kSM * kSK + kSK * kSN) +
                                                                        2 * kSM * kSK);

  const int tid = threadIdx.x & 255, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int half = lane >> 5, lrow = lane & 31, grp = lane >> 4, gl = lane & 15;

  // staging: thread unit u = tid + 256 i holds 8 consecutive elements of
  // one operand row (fp32 dkv as two f32x4, rounded to bf16 on the way to LDS);
  // two register sets, so a slice's loads are issued two slices before it is
  // multiplied
  f32x4 dreg[2][4][2];
  u32x4 hreg[2][4];
  auto gload = [&](int set, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + 256 * i;
      if constexpr (!DW) {   // dkv rows m0.., columns k0..k0+63; w rows n0.., same columns
        const int r = u >> 3, c8 = (u & 7) * 8;
        const float *g = a.dkv + (m0 + r) * a.C + k0 + c8;
        dreg[set][i][0] = *reinterpret_cast<const f32x4 *>(g);
        dreg[set][i][1] = *reinterpret_cast<const f32x4 *>(g + 4);
        hreg[set][i] = *reinterpret_cast<const u32x4 *>(a.w + (n0 + r) * a.ldw + a.col0 + k0 + c8);
      } else {               // tokens k0 + r: latent columns m0.., dkv columns n0..
        const int r = u >> 4, c8 = (u & 15) * 8;
        const int64_t t = k0 + r;
        hreg[set][i] = *reinterpret_cast<const u32x4 *>(a.latent + t * a.L + m0 + c8);
        const float *g = a.dkv + t * a.C + n0 + c8;
        dreg[set][i][0] = *reinterpret_cast<const f32x4 *>(g);
        dreg[set][i][1] = *reinterpret_cast<const f32x4 *>(g + 4);
      }
    }
  };
  auto lstore = [&](int buf, int set) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + 256 * i;
      const u32x4 d = as_u32x4(f32x8_to_bf16(dreg[set][i][0], dreg[set][i][1]));
      if constexpr (!DW) {
        const int r = u >> 3, c8 = (u & 7) * 8;
        *reinterpret_cast<u32x4 *>(As[buf] + rs_pos(r, c8)) = d;
        *reinterpret_cast<u32x4 *>(Bs[buf] + rs_pos(r, c8)) = hreg[set][i];
      } else {
        const int r = u >> 4, c8 = (u & 15) * 8;
        *reinterpret_cast<u32x4 *>(As[buf] + ts_pos(r, c8)) = hreg[set][i];
        *reinterpret_cast<u32x4 *>(Bs[buf] + ts_pos(r, c8)) = d;
      }
    }
  };
  // operand fragment of contraction step ks for the 32 output rows (A) or
  // columns (B) starting at x0: lane l takes index x0 + l%32 and contraction
  // elements 16ks + 8(l/32) .. +7 in natural order (both forms)
  auto frag = [&](const uint16_t *t, int x0, int ks) __attribute__((always_inline)) {
    if constexpr (!DW) {
      const int m = x0 + lrow;
      return *reinterpret_cast<const bf16x8 *>(t + rs_pos(m, 16 * ks + 8 * half));
    } else {
      const int x = x0 + 16 * (grp & 1) + 4 * (gl & 3);
      const int k0r = 16 * ks + 8 * (grp >> 1) + (gl >> 2), k1r = k0r + 4;
      const s16x4 lo = read_tr(t + ts_pos(k0r, x)), hi = read_tr(t + ts_pos(k1r, x));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // slice st: LDS buffer st % 2, register set st % 2
  gload(0, kbeg);
  if (a.nks > 1) gload(1, kbeg + kSK);
  lstore(0, 0);
  __syncthreads();
  auto slice = [&](int st, auto set_c) __attribute__((always_inline)) {
    constexpr int set = decltype(set_c)::value;
    const int buf = st & 1;
    // set `set` went to LDS before this slice: refill it with slice st + 2
    if (st + 2 < a.nks) gload(set, kbeg + (st + 2) * kSK);
    bf16x8 af[kSK / 16][2], bf[kSK / 16][2];
#pragma unroll
    for (int ks = 0; ks < kSK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[ks][i] = frag(As[buf], 64 * wm + 32 * i, ks);
        bf[ks][i] = frag(Bs[buf], 64 * wn + 32 * i, ks);
      }
#pragma unroll
    for (int ks = 0; ks < kSK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[ks][i], bf[ks][j], acc[i][j]);
    // the other buffer's readers finished before the previous slice's barrier
    if (st + 1 < a.nks) lstore(buf ^ 1, set ^ 1);
    __syncthreads();
  };
  for (int st = 0; st < a.nks; st += 2) {
    slice(st, std::integral_constant<int, 0>());
    if (st + 1 < a.nks) slice(st + 1, std::integral_constant<int, 1>());
  }
  // the second group's sums meet the first group's through LDS (first + second)
  float *red = reinterpret_cast<float *>(lds_all);
  if (grp2 == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((wave * 4 + i * 2 + j) * 16 + r) * 64 + lane] = acc[i][j][r];
  }
  __syncthreads();
  if (grp2 == 1) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] += red[((wave * 4 + i * 2 + j) * 16 + r) * 64 + lane];
  float *out = a.out + static_cast<int64_t>(split) * a.M * a.N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + 64 * wm + 32 * i + row_of(r, lane);
        __builtin_nontemporal_store(acc[i][j][r], out + m * a.N + n0 + 64 * wn + 32 * j + lrow);
      }
}

// out[i] = sum over s of part[s][i], s = 0, 1, ..., S-1 in that order
__global__ __launch_bounds__(256) void split_sum_kernel(const float *part, float *out, int64_t n4, int S) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4 *p = reinterpret_cast<const f32x4 *>(part) + i;
  f32x4 v = p[0];
  for (int s = 1; s < S; ++s) {
    const f32x4 w = p[s * n4];
    v[0] += w[0];
    v[1] += w[1];
    v[2] += w[2];
    v[3] += w[3];
  }
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(out) + i);
}

__global__ __launch_bounds__(256) void zero_kernel(float *x, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

template <int N, int R, int V>
int run(const BwdArgs &a, hipStream_t s) {
  static_assert(R % 4 == 0, "the band sum moves four elements per thread");
  const unsigned rows = static_cast<unsigned>((static_cast<int64_t>(a.T) * a.H * 16 + 255) / 256);
  row_term_kernel<<<rows, 256, 0, s>>>(a, V);
  const dim3 grid(static_cast<unsigned>((a.T + BB - 1) / BB), static_cast<unsigned>(a.H));
  attn_bwd_kernel<N, R, V><<<grid, 128, 0, s>>>(a);
  const unsigned sums = static_cast<unsigned>((static_cast<int64_t>(a.T) * R / 4 + 255) / 256);
  if (R > 0) band_sum_kernel<<<sums, 256, 0, s>>>(a, R);
  return hipGetLastError();
}

}  // namespace

bool attn_bwd_supported(int N, int R, int V) { return N == 128 && R == 64 && V == 128; }

size_t attn_bwd_workspace_bytes(int64_t T, int H, int R) {
  const size_t d = (static_cast<size_t>(T) * H * 4 + 255) / 256 * 256;
  const size_t b = (static_cast<size_t>(T) * H * R * 4 + 255) / 256 * 256;
  return d + b;
}

int launch_attention_bwd(const AttnBwdPlan &p, void *stream) {
  BwdArgs a;
  a.q = static_cast<const uint16_t *>(p.q);
  a.kv = static_cast<const uint16_t *>(p.kv);
  a.kr = static_cast<const uint16_t *>(p.kr);
  a.out = static_cast<const uint16_t *>(p.out);
  a.dout = static_cast<const uint16_t *>(p.dout);
  a.q_st = p.q_st;
  a.q_sh = p.q_sh;
  a.kv_st = p.kv_st;
  a.kv_sh = p.kv_sh;
  a.kr_st = p.kr_st;
  a.o_st = p.o_st;
  a.o_sh = p.o_sh;
  a.do_st = p.do_st;
  a.do_sh = p.do_sh;
  a.lse = p.lse;
  a.dq = p.dq;
  a.dkv = p.dkv;
  a.dkr = p.dkr;
  a.Dws = static_cast<float *>(p.ws);
  a.band = reinterpret_cast<float *>(static_cast<char *>(p.ws) + (static_cast<size_t>(p.T) * p.H * 4 + 255) / 256 * 256);
  a.cu = p.cu;
  a.n_seq = p.n_seq;
  a.T = static_cast<int>(p.T);
  a.H = p.H;
  a.scale = p.scale;
  a.causal = p.causal;
  if (p.T == 0) return hipSuccess;
  return run<128, 64, 128>(a, static_cast<hipStream_t>(stream));
}

int launch_up_proj_bwd(const UpProjBwdPlan &p, void *stream) {
  UpBwdArgs a;
  a.latent = static_cast<const uint16_t *>(p.latent);
  a.w = static_cast<const uint16_t *>(p.w);
  a.dkv = p.dkv;
  a.dl = p.d_latent;
  a.dw = p.dw;
  a.T = static_cast<int>(p.T);
  a.L = p.L;
  a.C = p.C;
  a.ldw = p.ldw;
  a.col0 = p.col0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.T == 0) {   // no tokens: the weight gradient is zero
    const int64_t n = static_cast<int64_t>(p.L) * p.C;
    zero_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(p.dw, n);
    return hipGetLastError();
  }
  const UpBwdSplits sp = up_bwd_splits(p.T, p.L, p.C);
  if (sp.aligned && p.ws != nullptr && p.ws_bytes >= sp.ws_bytes) {
    SplitArgs g;
    g.dkv = p.dkv;
    g.latent = a.latent;
    g.w = a.w;
    g.L = p.L;
    g.C = p.C;
    g.ldw = p.ldw;
    g.col0 = p.col0;
    float *ws = static_cast<float *>(p.ws);
    // d_latent [T][L]: contraction over the C columns
    g.M = a.T;
    g.N = p.L;
    g.tiles_m = a.T / kSM;
    g.tiles_n = p.L / kSN;
    g.nks = p.C / kSK / (2 * sp.s_dl);
    g.out = sp.s_dl > 1 ? ws : p.d_latent;
    up_bwd_split_kernel<false><<<g.tiles_m * g.tiles_n * sp.s_dl, 512, 0, s>>>(g);
    const int64_t n_dl = static_cast<int64_t>(a.T) * p.L / 4;
    if (sp.s_dl > 1)
      split_sum_kernel<<<static_cast<unsigned>((n_dl + 255) / 256), 256, 0, s>>>(ws, p.d_latent, n_dl, sp.s_dl);
    // dw [L][C]: contraction over the T tokens (the workspace is free again:
    // the sum above runs first on the stream)
    g.M = p.L;
    g.N = p.C;
    g.tiles_m = p.L / kSM;
    g.tiles_n = p.C / kSN;
    g.nks = a.T / kSK / (2 * sp.s_dw);
    g.out = sp.s_dw > 1 ? ws : p.dw;
    up_bwd_split_kernel<true><<<g.tiles_m * g.tiles_n * sp.s_dw, 512, 0, s>>>(g);
    const int64_t n_dw = static_cast<int64_t>(p.L) * p.C / 4;
    if (sp.s_dw > 1)
      split_sum_kernel<<<static_cast<unsigned>((n_dw + 255) / 256), 256, 0, s>>>(ws, p.dw, n_dw, sp.s_dw);
    return hipGetLastError();
  }
  // token blocks run fastest: the column tiles of one token block are 8k
  // launch slots apart and so share an XCD (and its L2 copy of their dkv rows)
  dlatent_kernel<<<dim3((a.T + kDlM - 1) / kDlM, (a.L + kDlN - 1) / kDlN), 256, 0, s>>>(a);
  dw_kernel<<<dim3((a.C + kDwN - 1) / kDwN, (a.L + kDwM - 1) / kDwM), 256, 0, s>>>(a);
  return hipGetLastError();
}

// Split counts: the largest power of two (at most 8) that keeps a launch
// within 256 workgroups (one per CU) with 2S equal parts of whole 64-wide
// slices; the workspace holds one product's partials at a time.
UpBwdSplits up_bwd_splits(int64_t T, int L, int C) {
  UpBwdSplits r;
  r.aligned = T > 0 && T % kSM == 0 && L % kSM == 0 && C % kSN == 0 && T <= (1LL << 24) && L <= (1 << 20) &&
              C <= (1 << 24);   // grid sizes stay below 2^31
  if (!r.aligned) return r;
  auto pick = [](int64_t tiles, int64_t slices) {
    int s = 1;
    while (s < 8 && tiles * s * 2 <= 256 && slices % (s * 4) == 0) s *= 2;
    return s;
  };
  r.s_dl = pick(T / kSM * (L / kSN), C / kSK);
  r.s_dw = pick(static_cast<int64_t>(L / kSM) * (C / kSN), T / kSK);
  const size_t dl = r.s_dl > 1 ? static_cast<size_t>(r.s_dl) * T * L * 4 : 0;
  const size_t dw = r.s_dw > 1 ? static_cast<size_t>(r.s_dw) * L * C * 4 : 0;
  r.ws_bytes = dl > dw ? dl : dw;
  return r;
}

}  // namespace mla
