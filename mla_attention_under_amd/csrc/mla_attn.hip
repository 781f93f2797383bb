// Causal / packed-document softmax attention of one rank's heads with a
// head-shared RoPE key band (torchtitan "MLA CP optimization", section
// "Ulysses CP": k_THK = concat(k_nope_THN, expand_per_head(k_shared_TR)), then
// attention; hyper-parallel `_assemble_key_value`, `MLAContextParallel.__call__`
// with no look-ahead for causal, `_causal_partition` for document-local keys).
//
// gfx950 design (bf16 in, fp32 accumulate):
//  * One workgroup = 4 waves = 64 queries of one head: 2 query blocks of 32 x
//    2 key halves. A 64-key tile is split between the halves (32 keys each);
//    the two partial softmax states of a query block are merged through LDS
//    at the end. Two workgroups fit a CU (80 KB LDS, <= 256 registers), so
//    every SIMD runs two waves and one wave's softmax overlaps the other's MFMAs.
//  * Tiles move global->LDS with buffer_load ... lds (no staging registers),
//    double-buffered, one barrier per tile. The key tile is assembled from two
//    sources: k_nope from this head's projected kv rows and the shared k_rope
//    row (one copy for all heads), so the expanded key never exists in HBM.
//    Loads past the visible keys fall outside the buffer range and read zero.
//  * LDS rows are unpadded and XOR-swizzled per row, so MFMA operand reads and
//    the transposing reads do not conflict on banks.
//  * Scores are computed transposed, S^T = K Q^T (32x32x16 MFMA), so lane l
//    holds 16 keys of query (l % 32) and lane l^32 the other 16: row max and
//    sum take one cross-lane step. P^T stays in registers as the B operand of
//    O^T = V^T P^T (MFMA k order permuted to match); V^T comes straight from
//    the row-major V tile with ds_read_b64_tr_b16.
//  * Online softmax in the exp2 domain (one fma + one exp per score); the
//    running output is rescaled only when a row max grows by more than 2^8
//    (exact: any reference max gives the same quotient).
//  * Work order: dense causal tiles are dealt heaviest-first, then lightest-
//    first, so co-resident workgroups carry complementary causal work; packed
//    documents use a device-built schedule sorted by key-tile count.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>

#include "mla_common.cuh"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int BM = 64;       // queries per workgroup (2 blocks of 32)
constexpr int BN = 64;       // keys per tile (2 halves of 32)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.0f;   // log2 growth of a row max that forces a rescale
constexpr float kNegBig = -1.0e30f;

struct AttnArgs {
  const uint16_t *q;
  const uint16_t *kv;
  const uint16_t *kr;
  uint16_t *out;
  float *lse;
  int64_t q_st, q_sh, kv_st, kv_sh, kr_st, o_st, o_sh;
  const int32_t *cu;      // nullptr: one document [0, T)
  const int2 *tasks;      // packed documents: (query start, document) per task, sorted
  const int *task_count;
  int n_qtiles;           // dense: query tiles per head
  int order;              // dense tile order: 0 heaviest first, 1 heavy half then light half
  int T, H;
  float scale_log2;       // scale * log2(e)
  int causal;
};

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// per-row XOR swizzles of the unpadded LDS tiles (16-byte chunks / 32-byte segments)
__device__ __forceinline__ int kn_swz(int key) { return key & 15; }
__device__ __forceinline__ int kr_swz(int key) { return (key ^ (key >> 3)) & 7; }
__device__ __forceinline__ int v_swz(int key) { return (key & 2) | ((key & 1) * 5); }

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const uint16_t *lds_dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(lds_dst), 16, static_cast<int>(voff), 0, 0, 0);
}

// 4 bf16 of V^T from a row-major V tile: ds_read_b64_tr_b16 hands lane i of
// each 16-lane group column i of the 4x16 block whose rows its lanes address.
__device__ __forceinline__ s16x4 read_tr(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}

template <int N, int R, int V>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int KD = N + R;          // score width
  constexpr int NCH = N / 8;         // 16-byte chunks per k_nope row
  constexpr int RCH = R / 8;         // per k_rope row
  constexpr int VCH = V / 8;         // per V row
  constexpr int KSTEPS = KD / 16;
  constexpr int NSTEPS = N / 16;
  constexpr int DBLK = V / 32;
  constexpr int KN_E = BN * N, KR_E = BN * R, V_E = BN * V;   // elements per stage
  constexpr int KN_I = BN * NCH / 256, KR_I = BN * RCH / 256, V_I = BN * VCH / 256;   // DMA instrs per wave
  static_assert(N == 128 && R == 64 && V == 128, "swizzles and DMA splits are laid out for 128/64/128");
  static_assert(KN_I * 256 == BN * NCH && KR_I * 256 == BN * RCH && V_I * 256 == BN * VCH, "tile DMA split");
  __shared__ __attribute__((aligned(1024))) uint16_t st0[KN_E + KR_E + V_E];
  __shared__ __attribute__((aligned(1024))) uint16_t st1[KN_E + KR_E + V_E];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qb = wave & 1, kh = wave >> 1;          // query block, key half
  const int half = lane >> 5, lrow = lane & 31;
  const int grp = lane >> 4, gl = lane & 15;        // 16-lane groups for the transposing read

  // ---- which (head, query tile)
  int h, q0, doc_lo, doc_hi;
  if (a.tasks == nullptr) {
    const int b = blockIdx.x, H = a.H, n = a.n_qtiles;
    int qt;
    if (a.order == 1 && a.causal) {
      const int heavy = ((n + 1) / 2) * H;
      if (b < heavy) {
        h = b % H;
        qt = n - 1 - b / H;
      } else {
        h = (b - heavy) % H;
        qt = (b - heavy) / H;
      }
    } else {
      h = b % H;
      qt = n - 1 - b / H;
    }
    q0 = qt * BM;
    doc_lo = 0;
    doc_hi = a.T;
  } else {
    const int t = static_cast<int>(blockIdx.x) / a.H;
    if (t >= *a.task_count) return;
    h = blockIdx.x % a.H;
    const int2 task = a.tasks[t];
    q0 = task.x;
    doc_lo = min(max(a.cu[task.y], 0), a.T);          // the same clamping as the schedule
    doc_hi = min(max(a.cu[task.y + 1], doc_lo), a.T);
  }
  h = __builtin_amdgcn_readfirstlane(h);
  q0 = __builtin_amdgcn_readfirstlane(q0);
  doc_lo = __builtin_amdgcn_readfirstlane(doc_lo);
  doc_hi = __builtin_amdgcn_readfirstlane(doc_hi);
  const int q_end = min(q0 + BM, doc_hi);
  const int kv_hi = a.causal ? q_end : doc_hi;
  const int n_tiles = (kv_hi - doc_lo + BN - 1) / BN;
  if (n_tiles <= 0) return;   // uniform: an empty task

  // ---- zero both stages once: loads past the buffer range may leave LDS untouched
  {
    u32x4 z{0, 0, 0, 0};
    for (int i = tid; i < (KN_E + KR_E + V_E) / 8; i += 256) {
      reinterpret_cast<u32x4 *>(st0)[i] = z;
      reinterpret_cast<u32x4 *>(st1)[i] = z;
    }
  }

  // ---- this lane's query and its Q fragment (B operand of S^T = K Q^T)
  const int qi = q0 + 32 * qb + lrow;
  const bool q_ok = qi < q_end;
  const int wq_first = q0 + 32 * qb;
  const int wq_last = min(q0 + 32 * qb + 31, q_end - 1);
  const bool wave_has_q = wq_first < q_end;
  bf16x8 qf[KSTEPS];
  {
    const uint16_t *qp = a.q + static_cast<int64_t>(min(qi, q_end - 1)) * a.q_st + static_cast<int64_t>(h) * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(qp + 16 * ks + 8 * half));
  }

  // ---- DMA plan: every wave issues KN_I + KR_I + V_I 1 KB transfers per tile.
  // Transfer i of wave w fills LDS chunks [64*(w*I + i), +64); lane l loads the
  // global chunk that the swizzle places at chunk 64*(w*I + i) + l.
  const uint16_t *kv_h = a.kv + static_cast<int64_t>(h) * a.kv_sh;
  uint32_t kn_off[KN_I], kr_off[KR_I], v_off[V_I];
#pragma unroll
  for (int i = 0; i < KN_I; ++i) {
    const int p = 64 * (wave * KN_I + i) + lane;
    const int key = p / NCH, c = (p % NCH) ^ kn_swz(key);
    kn_off[i] = static_cast<uint32_t>((key * a.kv_st + 8 * c) * 2);
  }
#pragma unroll
  for (int i = 0; i < KR_I; ++i) {
    const int p = 64 * (wave * KR_I + i) + lane;
    const int key = p / RCH, c = (p % RCH) ^ kr_swz(key);
    kr_off[i] = static_cast<uint32_t>((key * a.kr_st + 8 * c) * 2);
  }
#pragma unroll
  for (int i = 0; i < V_I; ++i) {
    const int p = 64 * (wave * V_I + i) + lane;
    const int key = p / VCH, cp = p % VCH;
    const int c = 2 * ((cp >> 1) ^ v_swz(key)) + (cp & 1);
    v_off[i] = static_cast<uint32_t>((key * a.kv_st + N + 8 * c) * 2);
  }
  auto issue = [&](uint16_t *st, int j0) {
    const int rows = min(kv_hi - j0, BN);
    const __amdgpu_buffer_rsrc_t rkv =
        make_rsrc(kv_h + static_cast<int64_t>(j0) * a.kv_st, static_cast<uint32_t>(rows * a.kv_st * 2));
    const __amdgpu_buffer_rsrc_t rkr =
        make_rsrc(a.kr + static_cast<int64_t>(j0) * a.kr_st, static_cast<uint32_t>(rows * a.kr_st * 2));
#pragma unroll
    for (int i = 0; i < KN_I; ++i) dma16(rkv, st + 512 * (wave * KN_I + i), kn_off[i]);
#pragma unroll
    for (int i = 0; i < KR_I; ++i) dma16(rkr, st + KN_E + 512 * (wave * KR_I + i), kr_off[i]);
#pragma unroll
    for (int i = 0; i < V_I; ++i) dma16(rkv, st + KN_E + KR_E + 512 * (wave * V_I + i), v_off[i]);
  };

  // ---- LDS read addresses (elements), loop-invariant
  // K: key 32*kh + lrow, chunk 2*ks + half
  const int kkey = 32 * kh + lrow;
  // V^T: for 16-key step b and read r, rows 32kh + 16b + 8r + 4*(grp>>1) + (gl>>2), d = 32db + 16*(grp&1) + 4*(gl&3)
  const int vrow0 = 32 * kh + 4 * (grp >> 1) + (gl >> 2);

  // ---- running state (per lane: one query; m in log2 units, partial row sum)
  f32x16 o[DBLK];
#pragma unroll
  for (int d = 0; d < DBLK; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
  float m_run = kNegBig, l_run = 0.f;
  const float c = a.scale_log2;

  // V^T operand fragments of this wave's 32-key half: [16-key step b][d block]
  auto active_for = [&](int j0) {
    const int jh = j0 + 32 * kh;
    return wave_has_q && jh < kv_hi && !(a.causal && jh > wq_last);
  };
  auto read_v = [&](const uint16_t *st, bf16x8 (&vf)[2][DBLK]) {
    const uint16_t *Vs = st + KN_E + KR_E;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int d = 0; d < DBLK; ++d) {
        const int dcol = 32 * d + 16 * (grp & 1) + 4 * (gl & 3);
        const int r0 = vrow0 + 16 * b, r1 = r0 + 8;
        const s16x4 lo = read_tr(Vs + r0 * V + 16 * ((dcol >> 4) ^ v_swz(r0)) + (dcol & 15));
        const s16x4 hi = read_tr(Vs + r1 * V + 16 * ((dcol >> 4) ^ v_swz(r1)) + (dcol & 15));
        vf[b][d] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
  };
  auto compute = [&](const uint16_t *st, int j0, const bf16x8 (&vf)[2][DBLK]) {
    const uint16_t *Kn = st, *Kr = st + KN_E;
    const int jh = j0 + 32 * kh;                     // first key of this wave's half
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int cidx = 2 * ks + half;
      const uint16_t *src = ks < NSTEPS ? Kn + kkey * N + 8 * (cidx ^ kn_swz(kkey))
                                        : Kr + kkey * R + 8 * ((cidx - 2 * NSTEPS) ^ kr_swz(kkey));
      s = mfma32(*reinterpret_cast<const bf16x8 *>(src), qf[ks], s);
    }
    // mask keys past the diagonal / the visible end (uniform test)
    if (jh + 31 >= kv_hi || (a.causal && jh + 31 > wq_first)) {
      const int lim = a.causal ? min(qi, kv_hi - 1) : kv_hi - 1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = jh + 8 * (r >> 2) + 4 * half + (r & 3);
        s[r] = j > lim ? -INFINITY : s[r];
      }
    }
    float mt = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32)) * c;
    if (__any(mt > m_run + kRescale)) {
      const float mn = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
    }
    bf16x8 pf[2];
    float lsum = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * b + 2 * e], c, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * b + 2 * e + 1], c, -m_run));
        lsum += p0 + p1;
        w[e] = pack_bf16x2(p0, p1);
      }
      pf[b] = as_bf16x8(w);
    }
    l_run += lsum;
    // O^T += V^T P^T
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int d = 0; d < DBLK; ++d) o[d] = mfma32(vf[b][d], pf[b], o[d]);
  };

  // One barrier per tile. A tile's V^T fragments are read into registers
  // before the next tile's transfers are issued, so no LDS read of the tile
  // being computed waits on the transfers in flight into the other stage.
  __syncthreads();                 // stages zeroed before the first transfer lands
  issue(st0, doc_lo);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's transfers have landed
  __syncthreads();
  for (int kt = 0; kt < n_tiles; kt += 2) {
    const int j0 = doc_lo + kt * BN;
    {
      const bool act = active_for(j0);
      bf16x8 vf[2][DBLK];
      if (act) read_v(st0, vf);
      if (kt + 1 < n_tiles) issue(st1, j0 + BN);
      if (act) compute(st0, j0, vf);
      __builtin_amdgcn_sched_barrier(0);   // keep the tile's MFMAs ahead of the wait
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
    }
    if (kt + 1 < n_tiles) {
      const bool act = active_for(j0 + BN);
      bf16x8 vf[2][DBLK];
      if (act) read_v(st1, vf);
      if (kt + 2 < n_tiles) issue(st0, j0 + 2 * BN);
      if (act) compute(st1, j0 + BN, vf);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
    }
  }

  // ---- merge the two key halves of each query block through LDS (stage 0 is free)
  float *xo = reinterpret_cast<float *>(st0) + qb * (DBLK * 16 + 2) * 64;
  if (kh == 1) {
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(d * 16 + r) * 64 + lane] = o[d][r];
    xo[(DBLK * 16) * 64 + lane] = m_run;
    xo[(DBLK * 16 + 1) * 64 + lane] = l_run;
  }
  __syncthreads();
  if (kh == 1 || !wave_has_q) return;
  {
    const float m1 = xo[(DBLK * 16) * 64 + lane];
    const float l1 = xo[(DBLK * 16 + 1) * 64 + lane];
    const float mn = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - mn), a1 = __builtin_amdgcn_exp2f(m1 - mn);
    l_run = l_run * a0 + l1 * a1;
    m_run = mn;
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] = o[d][r] * a0 + xo[(d * 16 + r) * 64 + lane] * a1;
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!q_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t *op = a.out + static_cast<int64_t>(qi) * a.o_st + static_cast<int64_t>(h) * a.o_sh;
#pragma unroll
  for (int d = 0; d < DBLK; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 v{pack_bf16x2(o[d][4 * g] * inv, o[d][4 * g + 1] * inv),
                    pack_bf16x2(o[d][4 * g + 2] * inv, o[d][4 * g + 3] * inv)};
      *reinterpret_cast<u32x2 *>(op + 32 * d + 8 * g + 4 * half) = v;
    }
  if (a.lse != nullptr && half == 0)
    a.lse[static_cast<int64_t>(h) * a.T + qi] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.6931471805599453f;
}

// ---- packed-document schedule: all (document, query tile) tasks, heaviest first
// Single workgroup. Writes tasks[] sorted by descending key-tile count and *count.
constexpr int kSchedThreads = 1024;
constexpr int kSchedBins = 4096;

// Document bounds are clamped to [0, T] with end >= start, so malformed offsets
// yield wrong documents but never an out-of-range access; at most max_tasks
// tasks are written.
__global__ __launch_bounds__(kSchedThreads) void attn_schedule_kernel(const int32_t *__restrict__ cu, int n_seq,
                                                                      int T, int causal, int max_tasks,
                                                                      int2 *__restrict__ tasks,
                                                                      int *__restrict__ count,
                                                                      int *__restrict__ doc_first) {
  __shared__ int hist[kSchedBins];
  __shared__ int scan_carry;
  const int tid = threadIdx.x;
  for (int i = tid; i < kSchedBins; i += kSchedThreads) hist[i] = 0;
  if (tid == 0) scan_carry = 0;
  __syncthreads();
  auto lo_of = [&](int d) { return min(max(cu[d], 0), T); };
  auto hi_of = [&](int d) { return min(max(cu[d + 1], lo_of(d)), T); };
  auto tiles_of = [&](int d) { return (hi_of(d) - lo_of(d) + BM - 1) / BM; };
  auto work_of = [&](int d, int t) {
    const int lo = lo_of(d), hi = hi_of(d);
    const int kv = causal ? min(lo + (t + 1) * BM, hi) - lo : hi - lo;
    return min((kv + BN - 1) / BN, kSchedBins - 1);
  };
  // exclusive prefix sum of tiles per document, in chunks of kSchedThreads
  __shared__ int part[kSchedThreads];
  for (int base = 0; base < n_seq; base += kSchedThreads) {
    const int d = base + tid;
    const int v = d < n_seq ? tiles_of(d) : 0;
    part[tid] = v;
    __syncthreads();
    for (int off = 1; off < kSchedThreads; off <<= 1) {
      const int add = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    if (d < n_seq) doc_first[d] = scan_carry + part[tid] - v;
    __syncthreads();
    if (tid == kSchedThreads - 1) scan_carry += part[tid];
    __syncthreads();
  }
  const int total = scan_carry;
  // histogram of work per task
  for (int d = 0; d < n_seq; ++d) {
    const int nt = tiles_of(d);
    for (int t = tid; t < nt; t += kSchedThreads) atomicAdd(&hist[work_of(d, t)], 1);
  }
  __syncthreads();
  // descending-bin exclusive offsets (serial over bins; 4096 bins, one thread)
  if (tid == 0) {
    int acc = 0;
    for (int b = kSchedBins - 1; b >= 0; --b) {
      const int v = hist[b];
      hist[b] = acc;
      acc += v;
    }
    *count = min(total, max_tasks);
  }
  __syncthreads();
  for (int d = 0; d < n_seq; ++d) {
    const int nt = tiles_of(d);
    for (int t = tid; t < nt; t += kSchedThreads) {
      const int slot = atomicAdd(&hist[work_of(d, t)], 1);
      if (slot < max_tasks) tasks[slot] = make_int2(lo_of(d) + t * BM, d);
    }
  }
}

// ---- generic kernel: one thread per (query, head); fp32 or any head widths
template <typename T>
__global__ __launch_bounds__(256) void attn_generic_kernel(AttnPlan p) {
  const T *q = static_cast<const T *>(p.q);
  const T *kv = static_cast<const T *>(p.kv);
  const T *kr = static_cast<const T *>(p.kr);
  T *out = static_cast<T *>(p.out);
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= p.T * p.H) return;
  const int64_t t = idx / p.H;
  const int h = static_cast<int>(idx % p.H);
  int64_t lo = 0, hi = p.T;
  if (p.cu != nullptr) {
    int d = 0;
    while (d + 1 < p.n_seq && p.cu[d + 1] <= t) ++d;
    lo = min(max<int64_t>(p.cu[d], 0), p.T);
    hi = min(max<int64_t>(p.cu[d + 1], lo), p.T);
  }
  const int64_t kend = p.causal ? min(t + 1, hi) : hi;
  const T *qp = q + t * p.q_st + h * p.q_sh;
  auto score = [&](int64_t j) {
    const T *kp = kv + j * p.kv_st + h * p.kv_sh;
    const T *rp = kr + j * p.kr_st;
    float acc = 0.f;
    for (int d = 0; d < p.N; ++d) acc += load_f32(qp, d) * load_f32(kp, d);
    for (int d = 0; d < p.R; ++d) acc += load_f32(qp, p.N + d) * load_f32(rp, d);
    return acc * p.scale;
  };
  float m = -INFINITY;
  for (int64_t j = lo; j < kend; ++j) m = fmaxf(m, score(j));
  float l = 0.f;
  for (int64_t j = lo; j < kend; ++j) l += expf(score(j) - m);
  T *op = out + t * p.o_st + h * p.o_sh;
  constexpr int CH = 16;
  for (int v0 = 0; v0 < p.V; v0 += CH) {
    float acc[CH];
    for (int i = 0; i < CH; ++i) acc[i] = 0.f;
    for (int64_t j = lo; j < kend; ++j) {
      const float w = expf(score(j) - m) / l;
      const T *vp = kv + j * p.kv_st + h * p.kv_sh + p.N;
      for (int i = 0; i < CH && v0 + i < p.V; ++i) acc[i] += w * load_f32(vp, v0 + i);
    }
    for (int i = 0; i < CH && v0 + i < p.V; ++i) store_f32(op, v0 + i, acc[i]);
  }
  if (p.lse != nullptr) p.lse[static_cast<int64_t>(h) * p.T + t] = m + logf(l);
}

struct WsLayout {
  size_t count_off, tasks_off, first_off, bytes;
};
WsLayout ws_layout(int64_t T, int n_seq) {
  WsLayout w;
  const size_t max_tasks = static_cast<size_t>((T + BM - 1) / BM + n_seq);
  w.count_off = 0;
  w.tasks_off = 256;
  w.first_off = w.tasks_off + ((max_tasks * sizeof(int2) + 255) / 256) * 256;
  w.bytes = w.first_off + ((static_cast<size_t>(n_seq) * sizeof(int) + 255) / 256) * 256;
  return w;
}

// Dense causal work order. 1 (default): the heavier half of the query tiles
// heaviest-first, then the lighter half lightest-first, so the workgroups that
// share a CU carry complementary causal work. 0: heaviest-first throughout.
// MLA_ATTN_ORDER overrides it (for measurement).
int attn_order() {
  static const int order = [] {
    const char *e = getenv("MLA_ATTN_ORDER");
    return e ? atoi(e) : 1;
  }();
  return order;
}

}  // namespace

bool attn_fast_path(int N, int R, int V, int bf16) { return bf16 && N == 128 && R == 64 && V == 128; }

size_t attn_workspace_bytes(int64_t T, int n_seq, int has_cu, int N, int R, int V, int bf16) {
  if (!has_cu || !attn_fast_path(N, R, V, bf16)) return 0;
  return ws_layout(T, n_seq).bytes;
}

int launch_attention(const AttnPlan &p, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.T == 0) return hipSuccess;
  if (!attn_fast_path(p.N, p.R, p.V, p.bf16)) {
    const int64_t n = p.T * p.H;
    const int blocks = static_cast<int>((n + 255) / 256);
    if (p.bf16)
      hipLaunchKernelGGL(attn_generic_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(attn_generic_kernel<float>, dim3(blocks), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  AttnArgs a;
  a.q = static_cast<const uint16_t *>(p.q);
  a.kv = static_cast<const uint16_t *>(p.kv);
  a.kr = static_cast<const uint16_t *>(p.kr);
  a.out = static_cast<uint16_t *>(p.out);
  a.lse = p.lse;
  a.q_st = p.q_st;
  a.q_sh = p.q_sh;
  a.kv_st = p.kv_st;
  a.kv_sh = p.kv_sh;
  a.kr_st = p.kr_st;
  a.o_st = p.o_st;
  a.o_sh = p.o_sh;
  a.T = static_cast<int>(p.T);
  a.H = p.H;
  a.scale_log2 = p.scale * kLog2e;
  a.causal = p.causal;
  a.cu = p.cu;
  int64_t tasks;
  if (p.cu == nullptr) {
    a.tasks = nullptr;
    a.task_count = nullptr;
    a.n_qtiles = static_cast<int>((p.T + BM - 1) / BM);
    a.order = attn_order();
    tasks = a.n_qtiles;
  } else {
    const WsLayout w = ws_layout(p.T, p.n_seq);
    char *ws = static_cast<char *>(p.ws);
    int *count = reinterpret_cast<int *>(ws + w.count_off);
    int2 *task_arr = reinterpret_cast<int2 *>(ws + w.tasks_off);
    int *first = reinterpret_cast<int *>(ws + w.first_off);
    const int max_tasks = static_cast<int>((p.T + BM - 1) / BM + p.n_seq);
    hipLaunchKernelGGL(attn_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, s, p.cu, p.n_seq,
                       static_cast<int>(p.T), p.causal, max_tasks, task_arr, count, first);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.tasks = task_arr;
    a.task_count = count;
    a.n_qtiles = 0;
    a.order = 0;
    tasks = (p.T + BM - 1) / BM + p.n_seq;
  }
  const int64_t blocks = tasks * p.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_kernel<128, 64, 128>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
