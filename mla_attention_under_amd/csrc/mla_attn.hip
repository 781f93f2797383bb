// Causal / packed-document softmax attention of one rank's heads with a
// head-shared RoPE key band (torchtitan "MLA CP optimization", section
// "Ulysses CP": k_THK = concat(k_nope_THN, expand_per_head(k_shared_TR)), then
// attention; hyper-parallel `_assemble_key_value`, `MLAContextParallel.__call__`
// with no look-ahead for causal, `_causal_partition` for document-local keys).
//
// gfx950 design (bf16 in, fp32 accumulate):
//  * One workgroup = 4 waves = one (head, 128-query tile); each wave owns 32
//    queries for the whole key loop, its Q fragment resident in VGPRs.
//  * Keys stream in 64-key tiles through double-buffered LDS with
//    global->register prefetch of the next tile. The K tile is assembled from
//    two sources per key: k_nope from the projected kv rows (per head) and the
//    shared k_rope row (the same row for every head), so the expanded key is
//    never materialised in HBM.
//  * Scores are computed transposed, S^T = K Q^T (32x32x16 MFMA), so lane l
//    holds 16 keys of query (l % 32) and lane l^32 the other 16: the row max
//    and row sum need one cross-lane step. P^T leaves the accumulator already
//    in the B-operand layout of O^T = V^T P^T (the MFMA k order is permuted to
//    match), so P never goes through LDS; V is written to LDS transposed
//    (V^T[d][key], keys permuted to the same k order) by a 4x8 register
//    transpose in the loader.
//  * Online softmax in the exp2 domain (scale*log2(e) folded into one multiply),
//    with the running output rescaled only when a row max grows by more than
//    2^8 (exact: any reference max gives the same quotient).
//  * Causal tiles past a wave's last query are skipped per wave; masks are
//    applied only on tiles that cross the diagonal or the document end.
//  * Work order: heaviest query tiles first (dense: from the end of the
//    sequence; packed documents: a device-built schedule sorted by key-tile
//    count, held in the caller's workspace).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "mla_common.cuh"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int BM = 128;      // queries per workgroup
constexpr int BN = 64;       // keys per tile
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
  int n_qtiles;           // dense: query tiles
  int T, H;
  float scale_log2;       // scale * log2(e)
  int causal;
};

// Position of key (kq*4 .. kq*4+3) inside its 16-key group in the permuted k order
// the P^T operand uses: lanes 0-31 hold keys {0-3, 8-11}, lanes 32-63 {4-7, 12-15}.
__device__ __forceinline__ int vt_pos(int kq) {
  const int q4 = kq & 3;
  return 16 * (kq >> 2) + ((q4 & 1) << 3) + ((q4 >> 1) << 2);
}

template <int N, int R, int V>
__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnArgs a) {
  constexpr int KD = N + R;            // score width
  constexpr int KP = KD + 8;           // LDS pitch of K rows [key][d]
  constexpr int VP = BN + 8;           // LDS pitch of V^T rows [d][key]
  constexpr int KCH = KD / 8;          // 16-byte chunks per key row
  constexpr int NCH = N / 8;
  constexpr int KLOADS = BN * KCH / 256;
  constexpr int VGROUPS = (BN / 4) * (V / 8);
  constexpr int VLOADS = VGROUPS / 256;
  constexpr int KSTEPS = KD / 16;
  constexpr int DBLK = V / 32;
  constexpr int KT_ELEMS = BN * KP, VT_ELEMS = V * VP;
  static_assert(KD % 16 == 0 && N % 8 == 0 && V % 32 == 0, "head widths");
  static_assert((BN * KCH) % 256 == 0 && VGROUPS % 256 == 0, "tile loads must split evenly");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (KT_ELEMS + VT_ELEMS)];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, lrow = lane & 31;

  // ---- which (head, query tile)
  int h, q0, doc_lo, doc_hi;
  if (a.tasks == nullptr) {
    h = blockIdx.x % a.H;
    q0 = (a.n_qtiles - 1 - static_cast<int>(blockIdx.x) / a.H) * BM;
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
  const int q_end = min(q0 + BM, doc_hi);
  const int kv_hi = a.causal ? q_end : doc_hi;
  const int n_tiles = (kv_hi - doc_lo + BN - 1) / BN;

  // ---- this lane's query and its Q fragment (B operand of S^T = K Q^T)
  const int qi = q0 + 32 * wave + lrow;
  const bool q_ok = qi < q_end;
  const int wave_q_first = q0 + 32 * wave;
  const int wave_q_last = min(q0 + 32 * wave + 31, q_end - 1);
  bf16x8 qf[KSTEPS];
  {
    const uint16_t *qp = a.q + static_cast<int64_t>(q_ok ? qi : q0) * a.q_st + static_cast<int64_t>(h) * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const u32x4 v = q_ok ? *reinterpret_cast<const u32x4 *>(qp + 16 * ks + 8 * half) : u32x4{0, 0, 0, 0};
      qf[ks] = as_bf16x8(v);
    }
  }

  // ---- tile loaders
  u32x4 rk[KLOADS];
  u32x4 rv[VLOADS][4];
  const uint16_t *kv_h = a.kv + static_cast<int64_t>(h) * a.kv_sh;
  auto load = [&](int j0) {
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int c = tid + 256 * u;
      const int key = c / KCH, part = c % KCH;
      const int j = j0 + key;
      u32x4 v{0, 0, 0, 0};
      if (j < kv_hi) {
        const uint16_t *src = part < NCH ? kv_h + static_cast<int64_t>(j) * a.kv_st + 8 * part
                                         : a.kr + static_cast<int64_t>(j) * a.kr_st + 8 * (part - NCH);
        v = *reinterpret_cast<const u32x4 *>(src);
      }
      rk[u] = v;
    }
#pragma unroll
    for (int u = 0; u < VLOADS; ++u) {
      const int g = tid + 256 * u;
      const int kq = g % (BN / 4), dq = g / (BN / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 4 * kq + r;
        rv[u][r] = j < kv_hi ? *reinterpret_cast<const u32x4 *>(kv_h + static_cast<int64_t>(j) * a.kv_st + N + 8 * dq)
                             : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store = [&](int buf) {
    uint16_t *Ks = smem + buf * (KT_ELEMS + VT_ELEMS);
    uint16_t *Vt = Ks + KT_ELEMS;
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int c = tid + 256 * u;
      *reinterpret_cast<u32x4 *>(Ks + (c / KCH) * KP + 8 * (c % KCH)) = rk[u];
    }
#pragma unroll
    for (int u = 0; u < VLOADS; ++u) {
      const int g = tid + 256 * u;
      const int kq = g % (BN / 4), dq = g / (BN / 4);
      const int pos = vt_pos(kq);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const u32x2 lo{lo_halves(rv[u][0][m], rv[u][1][m]), lo_halves(rv[u][2][m], rv[u][3][m])};
        const u32x2 hi{hi_halves(rv[u][0][m], rv[u][1][m]), hi_halves(rv[u][2][m], rv[u][3][m])};
        *reinterpret_cast<u32x2 *>(Vt + (8 * dq + 2 * m) * VP + pos) = lo;
        *reinterpret_cast<u32x2 *>(Vt + (8 * dq + 2 * m + 1) * VP + pos) = hi;
      }
    }
  };

  // ---- running state (per lane: one query, partial row sum over its keys)
  f32x16 o[DBLK];
#pragma unroll
  for (int d = 0; d < DBLK; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
  float m_run = kNegBig, l_run = 0.f;
  const float c = a.scale_log2;

  if (n_tiles > 0) {
    load(doc_lo);
    store(0);
  }
  __syncthreads();
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int j0 = doc_lo + kt * BN;
    if (kt + 1 < n_tiles) load(j0 + BN);
    const uint16_t *Ks = smem + (kt & 1) * (KT_ELEMS + VT_ELEMS);
    const uint16_t *Vt = Ks + KT_ELEMS;
    const bool wave_active = !(a.causal && j0 > wave_q_last) && wave_q_first < q_end;
    if (wave_active) {
      // S^T = K Q^T : two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[jb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(Ks + (32 * jb + lrow) * KP + 16 * ks + 8 * half);
          s[jb] = mfma32(kf, qf[ks], s[jb]);
        }
      }
      // scale into the log2 domain and mask
      const bool need_mask = (j0 + BN > kv_hi) || (a.causal && j0 + BN - 1 > wave_q_first);
      float mt = kNegBig;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[jb][r] * c;
          if (need_mask) {
            const int j = j0 + 32 * jb + 8 * (r >> 2) + 4 * half + (r & 3);
            if (j >= kv_hi || (a.causal && j > qi)) x = -INFINITY;
          }
          s[jb][r] = x;
          mt = fmaxf(mt, x);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
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
      // P^T in the B-operand layout of the PV MFMA: 16-key step b = registers 8*(b%2).. of block b/2
      bf16x8 pf[BN / 16];
      float lsum = 0.f;
#pragma unroll
      for (int b = 0; b < BN / 16; ++b) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(s[b >> 1][8 * (b & 1) + 2 * e] - m_run);
          const float p1 = __builtin_amdgcn_exp2f(s[b >> 1][8 * (b & 1) + 2 * e + 1] - m_run);
          lsum += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pf[b] = as_bf16x8(w);
      }
      l_run += lsum;
      // O^T += V^T P^T
#pragma unroll
      for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int b = 0; b < BN / 16; ++b) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(Vt + (32 * d + lrow) * VP + 16 * b + 8 * half);
          o[d] = mfma32(vf, pf[b], o[d]);
        }
    }
    if (kt + 1 < n_tiles) store((kt + 1) & 1);
    __syncthreads();
  }

  // ---- finish: full row sum, normalise, store
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
    tasks = (p.T + BM - 1) / BM + p.n_seq;
  }
  const int64_t blocks = tasks * p.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_kernel<128, 64, 128>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
