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
//   2. split    : per (sequence, split): the split's 64-key tiles of [latent |
//                 rope] rows (every splits-th tile of the sequence) stream from
//                 HBM into registers; each wave scores its 16 keys against all
//                 heads with 16x16x32 MFMAs straight from those registers (heads
//                 are the MFMA N dimension), the waves agree on the online-softmax
//                 maximum, and each accumulates o_c = sum_j p_j c_j for its
//                 quarter of the latent dims from the tile's latent rows in LDS
//                 (transposing reads); writes m_c, l_c, o_c / l_c.
//   3. merge    : m = max m_c, l = sum l_c 2^(m_c - m), o_lat = sum l_c 2^(m_c-m) o_c / l,
//                 lse = (m + log2 l) ln 2;
//      project  : out[b][h] = o_lat W_v[h].
// The cache is read exactly once, so the step is bound by HBM bandwidth on
// the cache; the weight is read once per head.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int DL = 512;          // latent width the split kernel is built for
constexpr int DR = 64;           // rope width
constexpr int DK = DL + DR;      // score width (576)
constexpr int DH = 16;           // heads per MFMA column block
constexpr int DT = 64;           // keys per tile
constexpr int SPLIT_WAVES = 4;   // wave w scores keys [16w, 16w+16) of a tile and owns latent dims [128w, 128w+128)
constexpr int SPLIT_THREADS = 64 * SPLIT_WAVES;
constexpr int KS = DK / 32;      // k-steps of the score product (16 latent + 2 rope)
constexpr int LKS = DL / 32;     // latent k-steps
constexpr int NSLOT = 2;         // latent tiles in LDS
constexpr int DEPTH = 2;         // tiles in flight in registers per wave
constexpr int PT_LD = DT + 8;    // row of the P^T buffer (bf16), padded against bank conflicts
constexpr float kLog2e = 1.4426950408889634f;
static_assert(DT == 16 * SPLIT_WAVES && DL == 128 * SPLIT_WAVES, "split work division");
static_assert(KS * (DEPTH - 1) < 64, "vmcnt field");

// Latent rows in LDS are unpadded 1 KB rows of 64 sixteen-byte chunks; chunk
// c of row r sits at c ^ kswz(r). The writes (one chunk of 16 rows per lane
// group) and the transposing reads (two neighbouring chunks of four
// consecutive rows) both land on distinct banks.
__device__ __forceinline__ int kswz(int key) { return ((key & 3) << 1) | ((key >> 2) & 1); }

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

// ---- 1. absorb: q_abs[b][h][l] = sum_n W[l][k-col(h) + n] q_nope[b][h][n]
// One workgroup per (head, 64 latent rows); thread (row, sequence group of
// SPW) reads its weight row once and forms SPW dot products.
constexpr int ABS_ROWS = 64, ABS_GROUPS = 4, ABS_SEQ = 64;   // sequences per workgroup slice
__global__ __launch_bounds__(ABS_ROWS * ABS_GROUPS) void decode_absorb_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ w, uint16_t *__restrict__ qabs, int B_all, int H,
    int L, int N, int V, int R, int64_t ldw, int64_t col0) {
  extern __shared__ float qs[];   // q_nope of this slice's sequences of this head, [B][N]
  const int h = blockIdx.x, l = blockIdx.y * ABS_ROWS + (threadIdx.x % ABS_ROWS);
  const int grp = threadIdx.x / ABS_ROWS;
  const int bz = blockIdx.z * ABS_SEQ;
  const int B = min(ABS_SEQ, B_all - bz);
  q += static_cast<int64_t>(bz) * H * (N + R);
  qabs += static_cast<int64_t>(bz) * H * (L + R);
  for (int i = threadIdx.x; i < B * N; i += blockDim.x)
    qs[i] = bf16_to_f32(q[(static_cast<int64_t>(i / N) * H + h) * (N + R) + i % N]);
  __syncthreads();
  const int64_t kcol = col0 + static_cast<int64_t>(h) * (N + V);   // first k_nope column of head h
  // rope band copies through unchanged
  if (blockIdx.y == 0)
    for (int i = threadIdx.x; i < B * R; i += blockDim.x)
      qabs[(static_cast<int64_t>(i / R) * H + h) * (L + R) + L + i % R] =
          q[(static_cast<int64_t>(i / R) * H + h) * (N + R) + N + i % R];
  if (l >= L) return;
  const uint16_t *wr = w + static_cast<int64_t>(l) * ldw + kcol;
  const bool vec = N % 8 == 0 && (reinterpret_cast<uintptr_t>(wr) & 15) == 0;
  for (int b0 = grp; b0 < B; b0 += 8 * ABS_GROUPS) {
    float acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = 0.f;
    if (vec) {
      for (int n = 0; n < N; n += 8) {
        const u32x4 wv = *reinterpret_cast<const u32x4 *>(wr + n);
        float wf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wf[2 * e] = __uint_as_float(wv[e] << 16);
          wf[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int b = b0 + u * ABS_GROUPS;
          if (b < B)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[u] += wf[e] * qs[b * N + n + e];
        }
      }
    } else {
      for (int n = 0; n < N; ++n) {
        const float wv = bf16_to_f32(wr[n]);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int b = b0 + u * ABS_GROUPS;
          if (b < B) acc[u] += wv * qs[b * N + n];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int b = b0 + u * ABS_GROUPS;
      if (b < B) qabs[(static_cast<int64_t>(b) * H + h) * (L + R) + l] = f32_to_bf16(acc[u]);
    }
  }
}

// MFMA form of the absorb (N a multiple of 16, 16-byte aligned rows): per
// head, q_abs^T[l][b] = W_k[l][:] . q_nope[b][:] as 32x32x16 MFMAs whose two
// operands are both contiguous in n, so they load straight from global
// memory. One wave per 32 latent rows x 32 sequences.
__global__ __launch_bounds__(256) void decode_absorb_mfma_kernel(const uint16_t *__restrict__ q,
                                                                 const uint16_t *__restrict__ w,
                                                                 uint16_t *__restrict__ qabs, int B, int H, int L,
                                                                 int N, int V, int R, int64_t ldw, int64_t col0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.x, l0 = blockIdx.y * 128 + 32 * wave, b0 = blockIdx.z * 32;
  const int i = lane & 31, g = lane >> 5;
  const int64_t kcol = col0 + static_cast<int64_t>(h) * (N + V);
  const int l = l0 + i, b = b0 + i;
  const uint16_t *wr = w + static_cast<int64_t>(l < L ? l : 0) * ldw + kcol;
  const uint16_t *qr = q + (static_cast<int64_t>(b < B ? b : 0) * H + h) * (N + R);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int n0 = 0; n0 < N; n0 += 128) {   // all eight k-steps' loads in flight before the products
    u32x4 av[8], bv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int n = n0 + 16 * u;
      av[u] = l < L && n < N ? *reinterpret_cast<const u32x4 *>(wr + n + 8 * g) : u32x4{0, 0, 0, 0};
      bv[u] = b < B && n < N ? *reinterpret_cast<const u32x4 *>(qr + n + 8 * g) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = mfma32(as_bf16x8(av[u]), as_bf16x8(bv[u]), acc);
  }
  // D[row = latent l0 + ri][col = sequence b0 + i]: lane holds rows 8*(r/4) + 4*g + r%4
  if (b < B) {
    uint16_t *out = qabs + (static_cast<int64_t>(b) * H + h) * (L + R);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int lr = l0 + 8 * rb + 4 * g;
      if (lr + 3 < L)
        *reinterpret_cast<u32x2 *>(out + lr) =
            u32x2{pack_bf16x2(acc[4 * rb], acc[4 * rb + 1]), pack_bf16x2(acc[4 * rb + 2], acc[4 * rb + 3])};
      else
        for (int e = 0; e < 4 && lr + e < L; ++e) out[lr + e] = f32_to_bf16(acc[4 * rb + e]);
    }
  }
  if (blockIdx.y == 0) {   // the rope band copies through unchanged, 16 bytes per thread
    const int rc = R / 8;
    for (int i = threadIdx.x; i < 32 * rc; i += blockDim.x) {
      const int bb = b0 + i / rc, c = i % rc;
      if (bb < B)
        *reinterpret_cast<u32x4 *>(qabs + (static_cast<int64_t>(bb) * H + h) * (L + R) + L + 8 * c) =
            *reinterpret_cast<const u32x4 *>(q + (static_cast<int64_t>(bb) * H + h) * (N + R) + N + 8 * c);
    }
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

// Tile t of a split holds keys [j0, j0 + 64). Wave w loads the [latent | rope]
// rows of keys j0 + 16w .. +15 straight into the register layout of the
// 16x16x32 MFMA A operand (lane (l16, g4): key l16, dims 32 ks + 8 g4 .. +7),
// scores them against all heads from registers, and stores the latent part
// into the LDS slot of the tile. The four waves then agree on the tile's
// row maximum, publish bf16 P^T, and each accumulates o_c^T for its 128
// latent dims over all 64 keys from transposing LDS reads. The next DEPTH
// tiles are in flight in registers meanwhile.
__global__ __launch_bounds__(SPLIT_THREADS, 1) void decode_split_kernel(SplitArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t lat_ring[NSLOT * DT * DL];   // [slot][key][dim], swizzled
  __shared__ __attribute__((aligned(16))) uint16_t pt[DH * PT_LD];                // P^T: [head][key] bf16
  __shared__ float wmax[SPLIT_WAVES][DH];
  __shared__ float wsum[SPLIT_WAVES][DH];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  // Split cidx of sequence b takes the tiles cidx, cidx + splits, cidx +
  // 2 splits, ... of the sequence: all splits of a sequence sweep its cache
  // together, front to back. The online softmax and the merge accept any
  // partition of the keys.
  const int b = blockIdx.x / a.splits, cidx = blockIdx.x % a.splits;
  const int64_t all_tiles = (a.S + DT - 1) / DT;
  const int n_tiles = cidx < all_tiles ? static_cast<int>((all_tiles - cidx + a.splits - 1) / a.splits) : 0;

  // Q^T fragments (B operand of S^T = K Q^T): head l16, dims 32 ks + 8 g4 .. +7
  bf16x8 qf[KS];
  {
    const bool hv = l16 < a.H;
    const uint16_t *qp = a.qabs + (static_cast<int64_t>(b) * a.H + (hv ? l16 : 0)) * DK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = as_bf16x8(hv ? *reinterpret_cast<const u32x4 *>(qp + 32 * ks + 8 * g4) : u32x4{0, 0, 0, 0});
  }

  auto tile_j0 = [&](int t) { return (static_cast<int64_t>(cidx) + static_cast<int64_t>(t) * a.splits) * DT; };
  // the sequence's rows as buffer ranges: rows at or past S read as zero
  const __amdgpu_buffer_rsrc_t rl =
      make_rsrc(a.c + static_cast<int64_t>(b) * a.S * DL, static_cast<uint32_t>(a.S * DL * 2));
  const __amdgpu_buffer_rsrc_t rr =
      make_rsrc(a.kr + static_cast<int64_t>(b) * a.S * DR, static_cast<uint32_t>(a.S * DR * 2));
  const int key = 16 * wave + l16;   // this lane's key within a tile
  auto load = [&](u32x4 (&r)[KS], int t) __attribute__((always_inline)) {
    const uint32_t row = static_cast<uint32_t>(std::min<int64_t>(tile_j0(t), a.S)) + key;
#pragma unroll
    for (int ks = 0; ks < LKS; ++ks) r[ks] = buffer_load16(rl, row * (DL * 2) + 64 * ks + 16 * g4);
#pragma unroll
    for (int ks = LKS; ks < KS; ++ks) r[ks] = buffer_load16(rr, row * (DR * 2) + 64 * (ks - LKS) + 16 * g4);
  };

  f32x4 o[8];   // O^T for dims 128 wave + 16 d + 4 g4 + r, head l16
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -1.0e30f, l_part = 0.f;   // l_part: this lane's keys only
  const float cs = a.scale_log2;

  auto step = [&](int t, u32x4 (&cur)[KS]) __attribute__((always_inline)) {
    // tile t's rows are the older of the two register sets in flight
    __builtin_amdgcn_s_waitcnt(0x0F70 | (KS * (DEPTH - 1) & 15) | ((KS * (DEPTH - 1) >> 4) << 14));
    // S^T[key][head] for this wave's 16 keys, two interleaved accumulation chains
    f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
      sa = mfma16(as_bf16x8(cur[ks]), qf[ks], sa);
      sb = mfma16(as_bf16x8(cur[ks + 1]), qf[ks + 1], sb);
    }
    uint16_t *slot = lat_ring + (t & 1) * (DT * DL);
#pragma unroll
    for (int ks = 0; ks < LKS; ++ks)
      *reinterpret_cast<u32x4 *>(slot + key * DL + 8 * ((4 * ks + g4) ^ kswz(key))) = cur[ks];
    load(cur, t + DEPTH);
    // lane holds keys j0 + 16 wave + 4 g4 + r of head l16
    const int64_t jb = tile_j0(t) + 16 * wave + 4 * g4;
    float sv[4], mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = sa[r] + sb[r];
      sv[r] = jb + r < a.S ? x * cs : -INFINITY;
      mt = fmaxf(mt, sv[r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    if (g4 == 0) wmax[wave][l16] = mt;
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): latent rows and maxima are in LDS
    __builtin_amdgcn_s_barrier();
    const float tm = fmaxf(fmaxf(wmax[0][l16], wmax[1][l16]), fmaxf(wmax[2][l16], wmax[3][l16]));
    const float mn = fmaxf(m_run, tm);
    const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
    m_run = mn;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sv[r] - mn);
    l_part = l_part * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    *reinterpret_cast<u32x2 *>(pt + l16 * PT_LD + 16 * wave + 4 * g4) = u32x2{pack_bf16x2(p[0], p[1]),
                                                                               pack_bf16x2(p[2], p[3])};
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    // O^T[dims][heads] = alpha O^T + C^T[dims][keys] P^T[keys][heads], keys in natural order
    bf16x8 pb[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) pb[kk] = *reinterpret_cast<const bf16x8 *>(pt + l16 * PT_LD + 32 * kk + 8 * g4);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int dcol = 128 * wave + 16 * d + 4 * (l16 & 3);
      f32x4 acc = o[d] * alpha;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int k0 = 32 * kk + 8 * g4 + (l16 >> 2), k1 = k0 + 4;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)(slot + k0 * DL + 8 * ((dcol >> 3) ^ kswz(k0)) + (dcol & 7)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)(slot + k1 * DL + 8 * ((dcol >> 3) ^ kswz(k1)) + (dcol & 7)));
        acc = mfma16(__builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)), pb[kk], acc);
      }
      o[d] = acc;
    }
  };

  // Slot reuse: tile t+2 overwrites slot t&1 only after both barriers of
  // tile t+1, which every wave passes after finishing tile t's products; the
  // P^T and maxima buffers are rewritten one barrier after their last read.
  u32x4 st0[KS], st1[KS];
  load(st0, 0);
  load(st1, 1);
  int t = 0;
  for (; t + 2 <= n_tiles; t += 2) {   // whole rounds: the loads in flight are the same on entry and back edge
    step(t, st0);
    step(t + 1, st1);
  }
  if (t < n_tiles) step(t, st0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // no load outlives the loop

  // partials: every wave holds the same m; l sums over the lanes of a head and the waves
  float ls = l_part + __shfl_xor(l_part, 16);
  ls += __shfl_xor(ls, 32);
  if (g4 == 0) wsum[wave][l16] = ls;
  __syncthreads();
  const float lsum = (wsum[0][l16] + wsum[1][l16]) + (wsum[2][l16] + wsum[3][l16]);
  if (l16 >= a.H) return;
  const int64_t bh = static_cast<int64_t>(b) * a.H + l16;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  float *op = a.o + (bh * a.splits + cidx) * DL;
  // streamed past L2: no dirty lines left for the end-of-kernel write-back
  // (the whole call 72.2 -> 72.0 us with a cold cache)
#pragma unroll
  for (int d = 0; d < 8; ++d)
    __builtin_nontemporal_store(o[d] * inv, reinterpret_cast<f32x4 *>(op + 128 * wave + 16 * d + 4 * g4));
  if (wave == 0 && g4 == 0) {
    a.m[bh * a.splits + cidx] = n_tiles > 0 ? m_run : -INFINITY;
    a.l[bh * a.splits + cidx] = lsum;
  }
}

// ---- 3a. merge the chunk partials of each (sequence, head):
// o_lat = sum_c l_c 2^(m_c - m) o_c / l (bf16, into the query buffer, which is
// free by now), lse = (m + log2 l) ln 2.
__global__ __launch_bounds__(256) void decode_merge_kernel(const float *__restrict__ m, const float *__restrict__ l,
                                                           const float *__restrict__ o, uint16_t *__restrict__ olat,
                                                           float *__restrict__ lse, int splits, int L) {
  const int64_t bh = blockIdx.x;
  const float *mp = m + bh * splits, *lp = l + bh * splits, *ob = o + bh * splits * L;
  for (int d = 2 * threadIdx.x; d < L; d += 2 * blockDim.x) {
    // the splits combine online, eight at a time with all their loads in
    // flight together: running max mx (finite start, so empty splits with
    // m_c = -inf weigh zero), denominator den and the two output sums
    float mx = -1.0e30f, den = 0.f, a0 = 0.f, a1 = 0.f;
    for (int c0 = 0; c0 < splits; c0 += 8) {
      f32x2_t v[8];
      float mc[8], lc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in = c0 + u < splits;
        v[u] = in ? *reinterpret_cast<const f32x2_t *>(ob + static_cast<int64_t>(c0 + u) * L + d) : f32x2_t{0.f, 0.f};
        mc[u] = in ? mp[c0 + u] : -INFINITY;
        lc[u] = in ? lp[c0 + u] : 0.f;
      }
      float cm = mx;
#pragma unroll
      for (int u = 0; u < 8; ++u) cm = fmaxf(cm, mc[u]);
      const float sc = __builtin_amdgcn_exp2f(mx - cm);
      den *= sc;
      a0 *= sc;
      a1 *= sc;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wu = lc[u] * __builtin_amdgcn_exp2f(mc[u] - cm);
        den += wu;
        a0 += wu * v[u].x;
        a1 += wu * v[u].y;
      }
      mx = cm;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    *reinterpret_cast<uint32_t *>(olat + bh * L + d) = pack_bf16x2(a0 * inv, a1 * inv);
    if (lse != nullptr && d == 0) lse[bh] = (mx + __builtin_amdgcn_logf(den)) * 0.6931471805599453f;
  }
}

// ---- 3b. out[b][h][v] = sum_d o_lat[b][h][d] W[d][v-col(h) + v]. One
// workgroup per (head, 16 value columns), eight waves; wave w contracts the
// latent rows [64w, 64w+64): its [64][16] weight block is staged in LDS and
// read transposed (ds_read_b64_tr_b16) as the B operand of 16x16x32 MFMAs,
// o_lat rows are the A operand straight from global memory. The eight
// partial sums meet in LDS, 64 sequences at a time.
constexpr int PV_COLS = 16, PV_WAVES = 8, PV_ROWS = DL / PV_WAVES, PV_SEQ = 64;
__global__ __launch_bounds__(PV_WAVES * 64) void decode_project_kernel(const uint16_t *__restrict__ olat,
                                                                      const uint16_t *__restrict__ w,
                                                                      uint16_t *__restrict__ out, int B, int H, int L,
                                                                      int N, int V, int64_t ldw, int64_t col0) {
  __shared__ __attribute__((aligned(16))) uint16_t ws[DL * PV_COLS];          // [d][v], 32-byte rows
  __shared__ __attribute__((aligned(16))) float red[PV_WAVES][PV_SEQ][PV_COLS];
  if (L != DL) return;
  const int h = blockIdx.x, v0 = blockIdx.y * PV_COLS;
  const int nv = min(PV_COLS, V - v0);
  const int64_t vcol = col0 + static_cast<int64_t>(h) * (N + V) + N + v0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool vec = nv == PV_COLS && ldw % 8 == 0 && ((reinterpret_cast<uintptr_t>(w + vcol)) & 15) == 0;
  const int l16 = lane & 15, g4 = lane >> 4;
  // A operands (o_lat rows: sequence bs + 16 mb + l16, this wave's dims) of
  // one 64-sequence chunk; the first chunk is in flight with the weight
  u32x4 av[PV_SEQ / 16][PV_ROWS / 32];
  auto load_a = [&](int bs) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < PV_SEQ / 16; ++mb) {
      const int ba = bs + 16 * mb + l16;
      const uint16_t *ar = olat + (static_cast<int64_t>(ba < B ? ba : 0) * H + h) * DL + PV_ROWS * wave + 8 * g4;
#pragma unroll
      for (int ks = 0; ks < PV_ROWS / 32; ++ks)
        av[mb][ks] = ba < B ? *reinterpret_cast<const u32x4 *>(ar + 32 * ks) : u32x4{0, 0, 0, 0};
    }
  };
  load_a(0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {   // 64 rows x two 16-byte chunks per wave
    const int p = lane + 64 * i, d = PV_ROWS * wave + (p >> 1), c = p & 1;
    const uint16_t *src = w + static_cast<int64_t>(d) * ldw + vcol + 8 * c;
    u32x4 v;
    if (vec) {
      v = *reinterpret_cast<const u32x4 *>(src);
    } else {
      uint16_t e[8];
      for (int k = 0; k < 8; ++k) e[k] = 8 * c + k < nv ? src[k] : 0;
      v = u32x4{e[0] | (static_cast<uint32_t>(e[1]) << 16), e[2] | (static_cast<uint32_t>(e[3]) << 16),
                e[4] | (static_cast<uint32_t>(e[5]) << 16), e[6] | (static_cast<uint32_t>(e[7]) << 16)};
    }
    *reinterpret_cast<u32x4 *>(ws + d * PV_COLS + 8 * c) = v;
  }
  __syncthreads();
  bf16x8 bw[PV_ROWS / 32];
#pragma unroll
  for (int ks = 0; ks < PV_ROWS / 32; ++ks) {
    const int d0 = PV_ROWS * wave + 32 * ks + 8 * g4 + (l16 >> 2), d1 = d0 + 4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(ws + d0 * PV_COLS + 4 * (l16 & 3)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(ws + d1 * PV_COLS + 4 * (l16 & 3)));
    bw[ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  for (int bs = 0; bs < B; bs += PV_SEQ) {
#pragma unroll
    for (int mb = 0; mb < PV_SEQ / 16; ++mb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < PV_ROWS / 32; ++ks) acc = mfma16(as_bf16x8(av[mb][ks]), bw[ks], acc);
      // D[row = sequence 16 mb + 4 g4 + r][col = value column l16]
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][16 * mb + 4 * g4 + r][l16] = acc[r];
    }
    if (bs + PV_SEQ < B) load_a(bs + PV_SEQ);
    __syncthreads();
    for (int i = threadIdx.x; i < PV_SEQ * PV_COLS; i += PV_WAVES * 64) {
      const int bq = i / PV_COLS, v = i % PV_COLS;
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < PV_WAVES; ++k) sum += red[k][bq][v];
      if (bs + bq < B && v < nv) out[(static_cast<int64_t>(bs + bq) * H + h) * V + v0 + v] = f32_to_bf16(sum);
    }
    __syncthreads();
  }
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
  const bool abs_mfma = p.N % 16 == 0 && p.R % 8 == 0 && p.ldw % 8 == 0 && p.col0 % 8 == 0 &&
                        (p.N + p.V) % 8 == 0 && p.L % 8 == 0;
  if (abs_mfma) {
    hipLaunchKernelGGL(decode_absorb_mfma_kernel, dim3(p.H, (p.L + 127) / 128, (p.B + 31) / 32), dim3(256), 0, s,
                       static_cast<const uint16_t *>(p.q), static_cast<const uint16_t *>(p.w), qabs, p.B, p.H, p.L,
                       p.N, p.V, p.R, p.ldw, p.col0);
  } else {
  const size_t abs_lds = static_cast<size_t>(std::min(p.B, ABS_SEQ)) * p.N * sizeof(float);
  if (abs_lds > 64 * 1024) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(decode_absorb_kernel,
                     dim3(p.H, (p.L + ABS_ROWS - 1) / ABS_ROWS, (p.B + ABS_SEQ - 1) / ABS_SEQ),
                     dim3(ABS_ROWS * ABS_GROUPS), abs_lds, s, static_cast<const uint16_t *>(p.q), static_cast<const uint16_t *>(p.w), qabs, p.B,
                     p.H, p.L, p.N, p.V, p.R, p.ldw, p.col0);
  }
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
  hipLaunchKernelGGL(decode_split_kernel, dim3(p.B * p.splits), dim3(SPLIT_THREADS), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint16_t *olat = qabs;   // [B][H][L] bf16; the query buffer is no longer read
  hipLaunchKernelGGL(decode_merge_kernel, dim3(p.B * p.H), dim3(256), 0, s, wm, wl, wo, olat, p.lse, p.splits, p.L);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_project_kernel, dim3(p.H, (p.V + PV_COLS - 1) / PV_COLS), dim3(PV_WAVES * 64), 0, s, olat, static_cast<const uint16_t *>(p.w), static_cast<uint16_t *>(p.out), p.B, p.H,
                     p.L, p.N, p.V, p.ldw, p.col0);
  return hipGetLastError();
}

}  // namespace mla
