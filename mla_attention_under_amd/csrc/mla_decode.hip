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
//   2. split    : per (sequence, split): the split's 32-key tiles of [latent |
//                 rope] rows (every splits-th tile of the sequence) stream through
//                 registers into a two-slot LDS ring; every wave scores all heads
//                 against the whole tile with
//                 16x16x32 MFMAs (heads are the MFMA N dimension), keeps the online
//                 softmax, and accumulates o_c = sum_j p_j c_j for its quarter of
//                 the latent dims through transposing LDS reads; writes m_c, l_c,
//                 o_c / l_c.
//   3. merge    : m = max m_c, l = sum l_c 2^(m_c - m), o_lat = sum l_c 2^(m_c-m) o_c / l,
//                 lse = (m + log2 l) ln 2;
//      project  : out[b][h] = o_lat W_v[h].
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
constexpr int DT = 32;           // keys per tile
constexpr int LAT_E = DT * DL, ROPE_E = DT * DR, ST_E = LAT_E + ROPE_E;   // elements per ring slot
constexpr int SPLIT_THREADS = 256;
constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// rows of the ring are unpadded; 16-byte chunks are XOR-swizzled by key within
// groups of eight so the row-parallel operand reads spread over the banks
__device__ __forceinline__ int kswz(int key) { return key & 7; }

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
  for (int n = 0; n < N; n += 16) {
    const u32x4 av = l < L ? *reinterpret_cast<const u32x4 *>(wr + n + 8 * g) : u32x4{0, 0, 0, 0};
    const u32x4 bv = b < B ? *reinterpret_cast<const u32x4 *>(qr + n + 8 * g) : u32x4{0, 0, 0, 0};
    acc = mfma32(as_bf16x8(av), as_bf16x8(bv), acc);
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
    if (blockIdx.y == 0 && wave == 0)   // the rope band copies through unchanged
      for (int r = g; r < R; r += 2) out[L + r] = qr[N + r];
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

// Tiles travel global -> registers -> LDS: the cache streams from HBM, and
// plain vector loads keep more bytes in flight per CU (DEPTH tiles per thread)
// than global->LDS transfers do.
constexpr int NSLOT = 2;                                       // LDS slots
constexpr int DEPTH = 4;                                       // tiles in flight in registers
constexpr int LAT_PT = LAT_E / 8 / SPLIT_THREADS;              // 16-byte latent chunks per thread per tile
constexpr int ROPE_PT = ROPE_E / 8 / SPLIT_THREADS;            // rope chunks per thread per tile
constexpr int PT = LAT_PT + ROPE_PT;
static_assert(LAT_PT * 8 * SPLIT_THREADS == LAT_E && ROPE_PT * 8 * SPLIT_THREADS == ROPE_E, "tile load split");
static_assert(PT * (DEPTH - 1) < 64, "vmcnt field");

__global__ __launch_bounds__(SPLIT_THREADS, 1) void decode_split_kernel(SplitArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t ring[NSLOT * ST_E];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  // Split cidx of sequence b takes the 32-key tiles cidx, cidx + splits,
  // cidx + 2 splits, ... of the sequence: all splits of a sequence sweep its
  // cache together, front to back, which streams from HBM far faster than
  // one contiguous chunk per split (their aligned starts collide in the
  // memory channels). The online softmax and the merge accept any partition.
  const int b = blockIdx.x / a.splits, cidx = blockIdx.x % a.splits;
  const int64_t k_hi = a.S;
  const int64_t all_tiles = (a.S + DT - 1) / DT;
  const int n_tiles = cidx < all_tiles ? static_cast<int>((all_tiles - cidx + a.splits - 1) / a.splits) : 0;

  // Q^T fragments (B operand of S^T = K Q^T): head l16, dims 32*ks + 8*g4 .. +7
  bf16x8 qf[DK / 32];
  {
    const bool hv = l16 < a.H;
    const uint16_t *qp = a.qabs + (static_cast<int64_t>(b) * a.H + (hv ? l16 : 0)) * DK;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks)
      qf[ks] = as_bf16x8(hv ? *reinterpret_cast<const u32x4 *>(qp + 32 * ks + 8 * g4) : u32x4{0, 0, 0, 0});
  }

  // first key of this split's t-th tile (t >= n_tiles: past the cache)
  auto tile_j0 = [&](int t) { return (static_cast<int64_t>(cidx) + static_cast<int64_t>(t) * a.splits) * DT; };
  // the sequence's rows as buffer ranges: rows past its end read zero
  const uint16_t *cb = a.c + static_cast<int64_t>(b) * a.S * DL;
  const uint16_t *rb = a.kr + static_cast<int64_t>(b) * a.S * DR;
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(cb, static_cast<uint32_t>(a.S * DL * 2));
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(rb, static_cast<uint32_t>(a.S * DR * 2));
  // this thread's chunks of a tile: source byte offsets and swizzled LDS element offsets
  uint32_t lsrc[LAT_PT], ldst[LAT_PT], rsrc_off, rdst;
#pragma unroll
  for (int i = 0; i < LAT_PT; ++i) {
    const int q = tid + SPLIT_THREADS * i, key = q >> 6, c = q & 63;
    lsrc[i] = static_cast<uint32_t>(key * DL * 2 + 16 * c);
    ldst[i] = static_cast<uint32_t>(key * DL + 8 * (c ^ kswz(key)));
  }
  {
    const int key = tid >> 3, c = tid & 7;
    rsrc_off = static_cast<uint32_t>(key * DR * 2 + 16 * c);
    rdst = static_cast<uint32_t>(LAT_E + key * DR + 8 * (c ^ kswz(key)));
  }
  u32x4 stage[DEPTH][PT];
  auto load = [&](u32x4 (&r)[PT], int t) {
    const uint32_t kl = static_cast<uint32_t>(std::min<int64_t>(tile_j0(t), a.S));
#pragma unroll
    for (int i = 0; i < LAT_PT; ++i) r[i] = buffer_load16(rl, kl * DL * 2 + lsrc[i]);
    r[LAT_PT] = buffer_load16(rr, kl * DR * 2 + rsrc_off);
  };
  auto put = [&](const u32x4 (&r)[PT], int slot) {
    uint16_t *st = ring + slot * ST_E;
#pragma unroll
    for (int i = 0; i < LAT_PT; ++i) *reinterpret_cast<u32x4 *>(st + ldst[i]) = r[i];
    *reinterpret_cast<u32x4 *>(st + rdst) = r[LAT_PT];
  };

  f32x4 o[8];   // O^T for dims 128*wave + 16*db + 4*g4 + r, head l16
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -1.0e30f, l_run = 0.f;
  const float cs = a.scale_log2;

  auto compute = [&](int t) __attribute__((always_inline)) {
    const uint16_t *lat = ring + (t % NSLOT) * ST_E, *rope = lat + LAT_E;
    const int64_t j0 = tile_j0(t);
    // S^T for both 16-key blocks of the tile, all heads
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int key = 16 * kb + l16;
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const int c = 4 * (ks & 15) + g4;
        const uint16_t *src = ks < 16 ? lat + key * DL + 8 * (c ^ kswz(key)) : rope + key * DR + 8 * (c ^ kswz(key));
        s[kb] = mfma16(*reinterpret_cast<const bf16x8 *>(src), qf[ks], s[kb]);
      }
    }
    // online softmax (every wave holds the whole tile's scores)
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t j = j0 + 16 * kb + 4 * g4 + r;
        s[kb][r] = j < k_hi ? s[kb][r] * cs : -INFINITY;
        mt = fmaxf(mt, s[kb][r]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
    m_run = mn;
    float p[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) p[4 * kb + r] = __builtin_amdgcn_exp2f(s[kb][r] - mn);
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    // P^T (B operand): k slot e < 4 is key 4*g4 + e of block 0, e >= 4 key 4*g4 + e-4 of block 1
    const bf16x8 pf = as_bf16x8(u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                      pack_bf16x2(p[6], p[7])});
    // O^T[dims][heads] = alpha O^T + C^T[dims][keys] P^T[keys][heads]; C^T via
    // transposing reads in the same key order (rows 4*g4 + i/4 and 16 + ...)
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int dbase = 128 * wave + 16 * d;
      const int dcol = dbase + 4 * (l16 & 3);
      const int k0 = 4 * g4 + (l16 >> 2), k1 = k0 + 16;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4 *)(lat + k0 * DL + 8 * ((dcol >> 3) ^ kswz(k0)) + (dcol & 7)));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4 *)(lat + k1 * DL + 8 * ((dcol >> 3) ^ kswz(k1)) + (dcol & 7)));
      o[d] = mfma16(__builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)), pf, o[d] * alpha);
    }
  };
  // iteration t: tile t is in LDS slot t % 2 and tiles t+1 .. t+DEPTH are in
  // flight in register set (t+i) % DEPTH; tile t+1 goes to LDS, its set
  // fetches tile t+1+DEPTH, then tile t is consumed
  auto step = [&](int t, u32x4 (&next)[PT]) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | (PT * (DEPTH - 1) & 15) | ((PT * (DEPTH - 1) >> 4) << 14));   // tile t+1 arrived
    put(next, (t + 1) % NSLOT);
    load(next, t + 1 + DEPTH);
    compute(t);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this thread's LDS writes are done
    __builtin_amdgcn_s_barrier();
  };
  // vmcnt leaves the newer tiles in flight; the barriers pass no memory fence
  // (a fence would wait for every load in flight)
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) load(stage[i], i);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (PT * (DEPTH - 1) & 15) | ((PT * (DEPTH - 1) >> 4) << 14));   // tile 0 arrived
  put(stage[0], 0);
  load(stage[0], DEPTH);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  for (int t = 0; t < n_tiles; t += DEPTH) {
    step(t, stage[1]);
    if (t + 1 < n_tiles) step(t + 1, stage[2]);
    if (t + 2 < n_tiles) step(t + 2, stage[3]);
    if (t + 3 < n_tiles) step(t + 3, stage[0]);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // no load outlives the loop

  // chunk partials: every wave holds the same m and l; row sums over the four lane groups
  float lsum = l_run + __shfl_xor(l_run, 16);
  lsum += __shfl_xor(lsum, 32);
  if (l16 >= a.H) return;
  const int64_t bh = static_cast<int64_t>(b) * a.H + l16;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  float *op = a.o + (bh * a.splits + cidx) * DL;
#pragma unroll
  for (int d = 0; d < 8; ++d)
    *reinterpret_cast<f32x4 *>(op + 128 * wave + 16 * d + 4 * g4) = o[d] * inv;
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
  __shared__ float wt[kDecodeMaxSplits];
  const int64_t bh = blockIdx.x;
  const float *mp = m + bh * splits, *lp = l + bh * splits;
  float mx = -INFINITY;
  for (int c = 0; c < splits; ++c) mx = fmaxf(mx, mp[c]);
  float den = 0.f;
  for (int c = 0; c < splits; ++c) den += lp[c] * __builtin_amdgcn_exp2f(mp[c] - mx);
  const float inv = den > 0.f ? 1.f / den : 0.f;
  for (int c = threadIdx.x; c < splits; c += blockDim.x) wt[c] = lp[c] * __builtin_amdgcn_exp2f(mp[c] - mx) * inv;
  __syncthreads();
  const float *ob = o + bh * splits * L;
  for (int d = 2 * threadIdx.x; d < L; d += 2 * blockDim.x) {
    float a0 = 0.f, a1 = 0.f;
    for (int c = 0; c < splits; ++c) {
      const f32x2_t v = *reinterpret_cast<const f32x2_t *>(ob + static_cast<int64_t>(c) * L + d);
      a0 += wt[c] * v.x;
      a1 += wt[c] * v.y;
    }
    *reinterpret_cast<uint32_t *>(olat + bh * L + d) = pack_bf16x2(a0, a1);
  }
  if (lse != nullptr && threadIdx.x == 0) lse[bh] = (mx + __builtin_amdgcn_logf(den)) * 0.6931471805599453f;
}

// ---- 3b. out[b][h][v] = sum_d o_lat[b][h][d] W[d][v-col(h) + v]. One
// workgroup per (head, 64 value columns); the weight slice [L][64] is staged
// in LDS (16-byte chunks XOR-swizzled by row) and read transposed
// (ds_read_b64_tr_b16) as the B operand of 16x16x32 MFMAs; o_lat rows are
// the A operand straight from global memory. Wave w owns columns 16w..16w+15
// for every sequence.
constexpr int PV_COLS = 64;
__global__ __launch_bounds__(256) void decode_project_kernel(const uint16_t *__restrict__ olat,
                                                             const uint16_t *__restrict__ w, uint16_t *__restrict__ out,
                                                             int B, int H, int L, int N, int V, int64_t ldw,
                                                             int64_t col0) {
  __shared__ __attribute__((aligned(16))) uint16_t ws[DL * PV_COLS];   // [d][v], chunk c of row d at c ^ (d & 7)
  if (L != DL) return;
  const int h = blockIdx.x, v0 = blockIdx.y * PV_COLS;
  const int nv = min(PV_COLS, V - v0);
  const int64_t vcol = col0 + static_cast<int64_t>(h) * (N + V) + N + v0;
  constexpr int CPR = PV_COLS / 8;   // 16-byte chunks per weight row
  const bool vec = nv == PV_COLS && ldw % 8 == 0 && ((reinterpret_cast<uintptr_t>(w + vcol)) & 15) == 0;
  for (int i = threadIdx.x; i < DL * CPR; i += blockDim.x) {
    const int d = i / CPR, c = i % CPR;
    u32x4 v;
    if (vec) {
      v = *reinterpret_cast<const u32x4 *>(w + static_cast<int64_t>(d) * ldw + vcol + 8 * c);
    } else {
      uint16_t e[8];
      for (int k = 0; k < 8; ++k) e[k] = 8 * c + k < nv ? w[static_cast<int64_t>(d) * ldw + vcol + 8 * c + k] : 0;
      v = u32x4{e[0] | (static_cast<uint32_t>(e[1]) << 16), e[2] | (static_cast<uint32_t>(e[3]) << 16),
                e[4] | (static_cast<uint32_t>(e[5]) << 16), e[6] | (static_cast<uint32_t>(e[7]) << 16)};
    }
    *reinterpret_cast<u32x4 *>(ws + d * PV_COLS + 8 * (c ^ (d & 7))) = v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int vc = 16 * wave + 4 * (l16 & 3);   // this lane's column group for the transposing read
  for (int bb = 0; bb < B; bb += 16) {
    const int ba = bb + l16;                  // A row: sequence
    const uint16_t *ar = olat + (static_cast<int64_t>(ba < B ? ba : 0) * H + h) * DL;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int ks = 0; ks < DL / 32; ++ks) {
      const u32x4 av = ba < B ? *reinterpret_cast<const u32x4 *>(ar + 32 * ks + 8 * g4) : u32x4{0, 0, 0, 0};
      const int d0 = 32 * ks + 8 * g4 + (l16 >> 2), d1 = d0 + 4;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4 *)(ws + d0 * PV_COLS + 8 * ((vc >> 3) ^ (d0 & 7)) + (vc & 7)));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4 *)(ws + d1 * PV_COLS + 8 * ((vc >> 3) ^ (d1 & 7)) + (vc & 7)));
      acc = mfma16(as_bf16x8(av), __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)),
                   acc);
    }
    // D[row = sequence bb + 4*g4 + r][col = value column 16*wave + l16]
    const int v = 16 * wave + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int bo = bb + 4 * g4 + r;
      if (bo < B && v < nv) out[(static_cast<int64_t>(bo) * H + h) * V + v0 + v] = f32_to_bf16(acc[r]);
    }
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
  const bool abs_mfma = p.N % 16 == 0 && (p.N + p.R) % 8 == 0 && p.ldw % 8 == 0 && p.col0 % 8 == 0 &&
                        (p.N + p.V) % 8 == 0 && p.L % 4 == 0;
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
  hipLaunchKernelGGL(decode_project_kernel, dim3(p.H, (p.V + PV_COLS - 1) / PV_COLS), dim3(256), 0, s, olat, static_cast<const uint16_t *>(p.w), static_cast<uint16_t *>(p.out), p.B, p.H,
                     p.L, p.N, p.V, p.ldw, p.col0);
  return hipGetLastError();
}

}  // namespace mla
