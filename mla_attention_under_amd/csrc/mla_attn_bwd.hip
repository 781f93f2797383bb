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
// Three launches:
//   row_term_kernel   D[h][t] from out and dout;
//   attn_bwd8_kernel  one workgroup (eight waves) per (block b of 128 tokens,
//                     head), two phases: dk, dv of key block b accumulated over
//                     the query steps that see it (the band part of dk goes to
//                     a per-head slice of the workspace), then dq of query
//                     block b accumulated over the key steps it sees (scores
//                     recomputed rather than reduced across workgroups, so no
//                     atomics and a fixed summation order);
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

// row i of the block held in register r of lane l (column l%32)
__device__ __forceinline__ int row_of(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

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

// ---- eight-wave form ---------------------------------------------------------
// One workgroup of eight waves (two per SIMD) per (block b of 128 tokens, head).
// Phase 1 accumulates dk and dv of key block b over 32-query steps, phase 2 dq
// of query block b over 32-key steps. Under the causal mask the two phases
// together take (T + 128) / 32 steps for every b, so the grid drains evenly.
// The four 32-token groups g of the block each have two waves, g and g + 4,
// which share a SIMD and split the group's products between them:
//   phase 1 (keys own0 = 128b + 32g): wave g computes s = q k^T and p, writes
//     p to LDS and accumulates dv = p^T dout; wave g + 4 computes dp = dout v^T,
//     reads p, forms ds = p (dp - D) and accumulates dk = ds^T q;
//   phase 2 (queries own0): wave g computes s^T = k q^T and p^T, wave g + 4
//     dp^T = v dout^T; they swap p^T and dp^T through LDS, both form ds, and
//     each accumulates three of the six 32-column tiles of dq = ds k.
// Each wave keeps only its own operand as register fragments (k or v, q or
// dout), so no product is computed twice; a step has two barriers (stage
// ready; the exchange written).
//
// The streamed block of each step (q, dout, lse, D in phase 1; k, v in phase
// 2) goes to one of kStages LDS stages by buffer_load ... lds, kStages - 1
// steps ahead. The scores come out with a lane per owned token: phase 1 s and
// dp have lane = key, registers = queries; phase 2 s^T and dp^T lane = query,
// registers = keys. Registers 8s .. 8s+7 of such a block, packed to bf16, are
// directly the A operand of the next product over the 16 streamed tokens
// 16s + 8(m/4) + 4(l/32) + m%4 (m = element), and the B operand comes from
// the stage through the transposing read, whose element order is the same
// (st_tr).
constexpr int kWB = 128;   // tokens per workgroup block
constexpr int kSB = 32;    // streamed tokens per step
constexpr int kStages = 3;
// A stage: three bf16 parts of kSB rows (CH 16-byte chunks per row), then lse
// and D (phase 1). A part is stored in fragment order: the 16 columns of k step
// f form one 1 KB block whose 16-byte slot l holds row l%32, columns
// 16f + 8(l/32) .. +7, with the slots of the upper half-wave swapped in pairs
// of 64 bytes (slot l ^ 4 for l >= 32). A row fragment is then one
// lane-contiguous 16-byte read, and the four rows x two half-chunks that a
// transposing read's 16 lanes address fall on distinct banks. Measured with
// eight waves per CU: 180 B/clk for the row reads and 117 for the transposing
// reads, against 128 and 102 for row-major rows with an XOR chunk swizzle.
template <int N, int R, int V>
struct Stage {
  static constexpr int kN = kSB * N, kR = kSB * R, kV = kSB * V;   // elements of the parts
  static constexpr int kLse = kN + kR + kV;                        // element offset of lse (fp32 x 32), then D
  static constexpr int kElems = kLse + 2 * kSB * 2;
};

// element (r, col) of a stage part with CH chunks per row
__device__ __forceinline__ int frag_slot(int l) { return l ^ ((l >> 5) << 2); }   // its own inverse
template <int CH>
__device__ __forceinline__ int st_elem(int r, int col) {
  return (col >> 4) * 512 + frag_slot(r + 32 * ((col & 15) >> 3)) * 8 + (col & 7);
}
// row fragment of k step s (lane l: row l%32, columns 16s + 8(l/32) .. +7)
template <int CH>
__device__ __forceinline__ bf16x8 st_row(const uint16_t *part, int s, int lane) {
  return *reinterpret_cast<const bf16x8 *>(part + 512 * s + 8 * frag_slot(lane));
}
// Transposed fragment of contraction step b for the columns 32d + l%32:
// element m of lane l comes from row 16b + 8(m/4) + 4(l/32) + m%4, the order
// in which registers 8b .. 8b+7 of a score block hold their rows (row_of).
template <int CH>
__device__ __forceinline__ bf16x8 st_tr(const uint16_t *part, int b, int d, int lane) {
  const int grp = lane >> 4, gl = lane & 15;
  const int col = 32 * d + 16 * (grp & 1) + 4 * (gl & 3);
  const int r0 = 4 * (grp >> 1) + (gl >> 2) + 16 * b;
  const s16x4 lo = read_tr(part + st_elem<CH>(r0, col)), hi = read_tr(part + st_elem<CH>(r0 + 8, col));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// the A operand of k step s from registers 8s .. 8s+7 of a score block
__device__ __forceinline__ bf16x8 pack_frag(const f32x16 &v, int s) {
  return as_bf16x8(u32x4{pack_bf16x2(v[8 * s], v[8 * s + 1]), pack_bf16x2(v[8 * s + 2], v[8 * s + 3]),
                         pack_bf16x2(v[8 * s + 4], v[8 * s + 5]), pack_bf16x2(v[8 * s + 6], v[8 * s + 7])});
}
// a score block through LDS: register 4j + e of lane l at f32x4 j*64 + l, element e
__device__ __forceinline__ void xch_put(float *buf, const f32x16 &v, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    reinterpret_cast<f32x4 *>(buf)[64 * j + lane] = f32x4{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
}
__device__ __forceinline__ f32x16 xch_get(const float *buf, int lane) {
  f32x16 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 x = reinterpret_cast<const f32x4 *>(buf)[64 * j + lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * j + e] = x[e];
  }
  return v;
}

// Transfers of one part of kSB rows x CH chunks into a stage by the waves
// ws = 0 .. NW-1 of a set, one 1 KB fragment block per transfer: slot l of
// block f holds row l'%32, chunk 2f + l'/32 (l' = frag_slot(l)), read from
// byte row * row_bytes + col_bytes + 16 chunk of the buffer (rows past its
// range read zero).
template <int CH, int NW>
__device__ __forceinline__ void stage_part(const u32x4 &rsrc, uint32_t lds, int64_t row_bytes, int col_bytes,
                                           int ws, int lane) {
  constexpr int I = CH / 2 / NW;   // fragment blocks per wave
  static_assert(I * 2 * NW == CH && kSB == 32, "whole fragment blocks per wave");
  const int l = frag_slot(lane), r = l & 31;
#pragma unroll
  for (int i = 0; i < I; ++i) {
    const int f = I * ws + i;
    dma16(rsrc, lds + 1024 * f, static_cast<uint32_t>(r * row_bytes + col_bytes + 16 * (2 * f + (l >> 5))));
  }
}

template <int N, int R, int V>
__global__ __launch_bounds__(512, 1) void attn_bwd8_kernel(BwdArgs a) {
  static_assert(N == 128 && R == 64 && V == 128, "stage layout, transfer split and fragment counts");
  constexpr int K = N + R;
  using St = Stage<N, R, V>;
  constexpr int CN = N / 8, CR = R / 8, CV = V / 8;
  __shared__ __attribute__((aligned(1024))) uint16_t stages[kStages][St::kElems];
  __shared__ __attribute__((aligned(1024))) float xch[2][4][16 * 64];   // [p, dp][group] score blocks
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g4 = wave & 3, second = wave >> 2;   // token group, which of its two waves
  const int nb = gridDim.x, G = nb * gridDim.y;
  int lin = blockIdx.x + nb * blockIdx.y;
  if (G % 8 == 0) lin = (lin % 8) * (G / 8) + lin / 8;   // each XCD runs whole heads
  const int h = lin / nb, b0 = (lin % nb) * kWB;
  const int b_end = min(b0 + kWB, a.T);
  const int own0 = b0 + 32 * g4;                          // the group's 32 owned tokens
  const int own = own0 + (lane & 31);
  const float c2 = a.scale * kLog2e;
  const bool nocausal = !a.causal;
  int lo0, hi0, lo1, hi1;
  doc_of(a, b0, lo0, hi0);
  doc_of(a, b_end - 1, lo1, hi1);

  // Issue order of a product block, pinned (the scheduler would otherwise put
  // each LDS read right before its MFMA and wait for it there): `ahead` reads
  // first, then one MFMA per `per` reads, then the last MFMAs.
  constexpr int kMfma = 0x008, kDsRead = 0x100;
  auto pin = [&](auto n_mfma, auto per, auto ahead) __attribute__((always_inline)) {
    constexpr int M = decltype(n_mfma)::value, P = decltype(per)::value, A = decltype(ahead)::value;
    __builtin_amdgcn_sched_group_barrier(kDsRead, A, 0);
#pragma unroll
    for (int i = 0; i < M - A / P; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kDsRead, P, 0);
    }
#pragma unroll
    for (int i = 0; i < A / P; ++i) __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  auto settle = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
  };
  auto sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // The second waves issue all transfers, kBatch per wave and step (steps
  // past the end issue empty ones), in the time they would otherwise wait for
  // p. When step t starts, the batches of steps t+1 .. t+kStages-2 are the
  // only ones issued after its own: waiting until at most that many transfers
  // are pending means step t's have landed (the first waves have none pending).
  constexpr int kBatch = 6;
  using Pend1 = std::integral_constant<int, kBatch * (kStages - 2)>;
  auto wait_stage = [&](auto pend_c) __attribute__((always_inline)) {
    constexpr int P = decltype(pend_c)::value;   // this wave's transfers of the later batches
    static_assert(P < 64, "vmcnt field");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((P & 15) | ((P >> 4) << 14) | (7 << 4) | (15 << 8));
    __builtin_amdgcn_s_barrier();         // every wave's transfers landed; stage (t-1) % kStages is free
    __builtin_amdgcn_sched_barrier(0);
  };
  // the empty transfer that evens out a wave's batch in phase 2 (it writes
  // zeros over the stage's lse / D slots, which phase 2 does not read)
  auto pad_transfer = [&](uint32_t base) __attribute__((always_inline)) {
    const u32x4 r0 = dma_rsrc(a.kr, 0);
    if (lane < 16) dma16(r0, base + 2 * St::kLse, static_cast<uint32_t>(16 * lane));
  };

  // ---- phase 1: dv (first waves) and dk (second waves) of keys own0 .. own0+31
  {
    const int qbeg = __builtin_amdgcn_readfirstlane(a.causal ? b0 : lo0);
    const int qend = __builtin_amdgcn_readfirstlane(hi1);
    // six transfers per second wave: the q rows and band (part 0), the dout
    // rows, lse and D (part 1); rows at or past qend are never visible and
    // read zero
    auto issue_part = [&](int part, int stg, int q0) __attribute__((always_inline)) {
      const int ws = wave - 4;
      const uint32_t rows = static_cast<uint32_t>(max(0, min(kSB, qend - q0)));
      const uint32_t base = lds_addr(stages[stg]);
      if (part == 0) {
        const uint16_t *qrow = a.q + static_cast<int64_t>(q0) * a.q_st + static_cast<int64_t>(h) * a.q_sh;
        const u32x4 rq = dma_rsrc(qrow, rows * static_cast<uint32_t>(a.q_st) * 2);
        stage_part<CN, 4>(rq, base, a.q_st * 2, 0, ws, lane);
        stage_part<CR, 4>(rq, base + 2 * St::kN, a.q_st * 2, 2 * N, ws, lane);
      } else {
        const uint16_t *grow = a.dout + static_cast<int64_t>(q0) * a.do_st + static_cast<int64_t>(h) * a.do_sh;
        const u32x4 rg = dma_rsrc(grow, rows * static_cast<uint32_t>(a.do_st) * 2);
        stage_part<CV, 4>(rg, base + 2 * (St::kN + St::kR), a.do_st * 2, 0, ws, lane);
        // lse (waves 4, 6) and D (waves 5, 7): the two copies write the same bytes
        const int which = ws & 1;
        const float *src = (which == 0 ? a.lse : a.Dws) + static_cast<int64_t>(h) * a.T + min(q0, a.T);
        const u32x4 rl = dma_rsrc(src, rows * 4);
        if (lane < 8) dma16(rl, base + 2 * St::kLse + 128 * which, static_cast<uint32_t>(16 * lane));
      }
    };
    auto issue = [&](int stg, int q0) __attribute__((always_inline)) {
      issue_part(0, stg, q0);
      issue_part(1, stg, q0);
    };
    int klo = 1, khi = 0;   // the owned key's document (empty past T)
    if (own < a.T) doc_of(a, own, klo, khi);
    const int nst = (qend - qbeg + kSB - 1) / kSB;
    // The two waves of a group run their own loops (so each holds only its
    // own registers) with the same barriers in the same order.
    auto run1 = [&](auto second_c) __attribute__((always_inline)) {
      constexpr bool SECOND = decltype(second_c)::value;
      constexpr int NF = SECOND ? V / 16 : K / 16, NT = SECOND ? K / 32 : V / 32;
      bf16x8 of[NF];   // the owned operand: k (first wave) or v (second wave)
      if constexpr (!SECOND) {
        load_frags<N>(a.kv + h * a.kv_sh, a.kv_st, own0, a.T, of, lane);
        load_frags<R>(a.kr, a.kr_st, own0, a.T, of + N / 16, lane);
      } else {
        load_frags<V>(a.kv + h * a.kv_sh + N, a.kv_st, own0, a.T, of, lane);
      }
      f32x16 acc[NT] = {};   // dv (first wave) or dk (second wave)
      // nothing the compiler tracks may be pending inside the loop (its wait
      // for one would also drain every transfer in flight)
      settle();
      if constexpr (SECOND)
        if (nst > 0)
#pragma unroll
          for (int i = 0; i < kStages - 1; ++i) issue(i, qbeg + kSB * i);
      // every query of a step lies in every owned key's document when it lies in
      // the last key's document start and the first key's document end
      const int vis_lo = __builtin_amdgcn_readlane(klo, 31), vis_hi = __builtin_amdgcn_readlane(khi, 0);
      for (int t = 0; t < nst; ++t) {
        const int q0 = qbeg + kSB * t;
        wait_stage(Pend1());
        const uint16_t *sg = stages[t % kStages];
        const uint16_t *Qn = sg, *Qr = sg + St::kN, *Gv = sg + St::kN + St::kR;
        const float *Ls = reinterpret_cast<const float *>(sg + St::kLse), *Ds = Ls + kSB;
        // nothing visible when the group's keys all follow the step's queries or lie past T
        const bool idle = own0 >= a.T || (a.causal && q0 + kSB - 1 < own0);
        // everything visible: no mask to apply
        const bool full = q0 >= vis_lo && q0 + kSB <= vis_hi && (nocausal || q0 >= own0 + kSB - 1);
        (void)full;
        f32x16 s = {};
        if constexpr (!SECOND) {   // s = q k^T, then p; dv += p^T dout
          if (!idle) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < N / 16; ++k) s = mfma32(st_row<CN>(Qn, k, lane), of[k], s);
#pragma unroll
            for (int k = 0; k < R / 16; ++k) s = mfma32(st_row<CR>(Qr, k, lane), of[N / 16 + k], s);
            pin(std::integral_constant<int, K / 16>(), I1(), I4());
            // registers 4j .. 4j+3 hold queries q0 + 8j + 4(l/32) + 0..3
            if (full) {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const f32x4 l4 = *reinterpret_cast<const f32x4 *>(Ls + 8 * j + 4 * (lane >> 5));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  s[4 * j + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * j + e], c2, -l4[e] * kLog2e));
              }
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int qi = 8 * j + 4 * (lane >> 5);
                const f32x4 l4 = *reinterpret_cast<const f32x4 *>(Ls + qi);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int q = q0 + qi + e;
                  const bool vis = (q >= klo) & (q < khi) & (nocausal | (q >= own));   // no short circuit: no branches
                  // exp2(-inf) = 0: the mask is a select, not a branch around the exponential
                  s[4 * j + e] = __builtin_amdgcn_exp2f(vis ? __builtin_fmaf(s[4 * j + e], c2, -l4[e] * kLog2e)
                                                            : -__builtin_inff());
                }
              }
            }
            xch_put(xch[0][g4], s, lane);
          }
          sync();   // p is in LDS
          if (!idle) {
            const bf16x8 pa0 = pack_frag(s, 0), pa1 = pack_frag(s, 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int d = 0; d < V / 32; ++d) acc[d] = mfma32(pa0, st_tr<CV>(Gv, 0, d, lane), acc[d]);
#pragma unroll
            for (int d = 0; d < V / 32; ++d) acc[d] = mfma32(pa1, st_tr<CV>(Gv, 1, d, lane), acc[d]);
            pin(std::integral_constant<int, (kSB / 16) * V / 32>(), I2(), I8());
          }
        } else {                   // dp = dout v^T; ds = p (dp - D); dk += ds^T q
          // half of the step's transfers before the dp products (the first
          // wave's score products keep the matrix pipe busy meanwhile), half
          // after them (while the first wave exponentiates)
          issue_part(0, (t + kStages - 1) % kStages, q0 + kSB * (kStages - 1));
          if (!idle) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < V / 16; ++k) s = mfma32(st_row<CV>(Gv, k, lane), of[k], s);
            pin(std::integral_constant<int, V / 16>(), I1(), I4());
          }
          issue_part(1, (t + kStages - 1) % kStages, q0 + kSB * (kStages - 1));
          sync();   // p is in LDS
          if (!idle) {
            const f32x4 *pb = reinterpret_cast<const f32x4 *>(xch[0][g4]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const f32x4 p4 = pb[64 * j + lane];
              const f32x4 d4 = *reinterpret_cast<const f32x4 *>(Ds + 8 * j + 4 * (lane >> 5));
#pragma unroll
              for (int e = 0; e < 4; ++e) s[4 * j + e] = p4[e] * (s[4 * j + e] - d4[e]);
            }
            const bf16x8 sa0 = pack_frag(s, 0), sa1 = pack_frag(s, 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < kSB / 16; ++k) {
              const bf16x8 sa = k == 0 ? sa0 : sa1;
#pragma unroll
              for (int d = 0; d < N / 32; ++d) acc[d] = mfma32(sa, st_tr<CN>(Qn, k, d, lane), acc[d]);
#pragma unroll
              for (int d = 0; d < R / 32; ++d)
                acc[N / 32 + d] = mfma32(sa, st_tr<CR>(Qr, k, d, lane), acc[N / 32 + d]);
            }
            pin(std::integral_constant<int, (kSB / 16) * K / 32>(), I2(), I8());
          }
        }
      }
      // register r holds key own0 + row_of(r), lane l%32 the column: dv, or dk
      // scaled (its band part to this head's slice). dk and dv are final
      // outputs and stream past L2 (no dirty lines for the end-of-kernel
      // write-back: kernel about 2 us faster); the band slices stay in the
      // caches for the band sum that reads them next.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = own0 + row_of(r, lane);
        if (key >= a.T) continue;
        float *row = a.dkv + (static_cast<int64_t>(key) * a.H + h) * (N + V);
        if constexpr (SECOND) {
          float *brow = a.band + (static_cast<int64_t>(h) * a.T + key) * R;
#pragma unroll
          for (int d = 0; d < N / 32; ++d)
            __builtin_nontemporal_store(a.scale * acc[d][r], row + 32 * d + (lane & 31));
#pragma unroll
          for (int d = 0; d < R / 32; ++d) brow[32 * d + (lane & 31)] = a.scale * acc[N / 32 + d][r];
        } else {
#pragma unroll
          for (int d = 0; d < V / 32; ++d)
            __builtin_nontemporal_store(acc[d][r], row + N + 32 * d + (lane & 31));
        }
      }
    };
    if (second) run1(std::true_type());
    else run1(std::false_type());
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // the trailing (empty) transfers landed
  __syncthreads();                      // and every wave is done with the stages

  // ---- phase 2: dq of queries own0 .. own0+31, tiles 0-2 (first wave) and 3-5 (second)
  {
    const int kbeg = __builtin_amdgcn_readfirstlane(lo0);
    const int kend = __builtin_amdgcn_readfirstlane(a.causal ? b_end : hi1);
    // the second waves move the k and v rows (four transfers each), the first
    // waves the band and an empty transfer (two each), in the time each would
    // otherwise wait for the other's half of the pair
    // part 0: the k rows (second waves) or the band (first waves); part 1:
    // the v rows or the empty transfer
    auto issue_part = [&](int part, int stg, int k0) __attribute__((always_inline)) {
      const int ws = wave & 3;
      const uint32_t rows = static_cast<uint32_t>(max(0, min(kSB, kend - k0)));
      const uint32_t base = lds_addr(stages[stg]);
      if (second) {
        const uint16_t *krow = a.kv + static_cast<int64_t>(k0) * a.kv_st + static_cast<int64_t>(h) * a.kv_sh;
        const u32x4 rk = dma_rsrc(krow, rows * static_cast<uint32_t>(a.kv_st) * 2);
        if (part == 0)
          stage_part<CN, 4>(rk, base, a.kv_st * 2, 0, ws, lane);
        else
          stage_part<CV, 4>(rk, base + 2 * (St::kN + St::kR), a.kv_st * 2, 2 * N, ws, lane);
      } else if (part == 0) {
        const u32x4 rr =
            dma_rsrc(a.kr + static_cast<int64_t>(k0) * a.kr_st, rows * static_cast<uint32_t>(a.kr_st) * 2);
        stage_part<CR, 4>(rr, base + 2 * St::kN, a.kr_st * 2, 0, ws, lane);
      } else {
        pad_transfer(base);
      }
    };
    auto issue = [&](int stg, int k0) __attribute__((always_inline)) {
      issue_part(0, stg, k0);
      issue_part(1, stg, k0);
    };
    int qlo = 1, qhi = 0;
    float lse2 = 0.f, Dq = 0.f;
    if (own < a.T) {
      doc_of(a, own, qlo, qhi);
      lse2 = a.lse[static_cast<int64_t>(h) * a.T + own] * kLog2e;
      Dq = a.Dws[static_cast<int64_t>(h) * a.T + own];
    }
    const int nst = (kend - kbeg + kSB - 1) / kSB;
    auto run2 = [&](auto second_c) __attribute__((always_inline)) {
      constexpr bool SECOND = decltype(second_c)::value;
      constexpr int NF = SECOND ? V / 16 : K / 16;
      bf16x8 of[NF];   // the owned operand: q (first wave) or dout (second wave)
      if constexpr (!SECOND) load_frags<K>(a.q + h * a.q_sh, a.q_st, own0, a.T, of, lane);
      else load_frags<V>(a.dout + h * a.do_sh, a.do_st, own0, a.T, of, lane);
      f32x16 dq[3] = {};   // dq tiles 0-2 (first wave) or 3-5 (second wave)
      settle();
      if (nst > 0)
#pragma unroll
        for (int i = 0; i < kStages - 1; ++i) issue(i, kbeg + kSB * i);
      using Pend2 = std::integral_constant<int, (SECOND ? 4 : 2) * (kStages - 2)>;
      // every key of a step lies in every owned query's document (see phase 1)
      const int vis_lo = __builtin_amdgcn_readlane(qlo, 31), vis_hi = __builtin_amdgcn_readlane(qhi, 0);
      for (int t = 0; t < nst; ++t) {
        const int k0 = kbeg + kSB * t;
        wait_stage(Pend2());
        const uint16_t *sg = stages[t % kStages];
        const uint16_t *Kn = sg, *Kr = sg + St::kN, *Vv = sg + St::kN + St::kR;
        // nothing visible when the step's keys all follow the group's queries or the queries lie past T
        const bool idle = own0 >= a.T || (a.causal && k0 > own0 + 31);
        const bool full = k0 >= vis_lo && k0 + kSB <= vis_hi && (nocausal || k0 + kSB - 1 <= own0);
        f32x16 s = {};
        // half of the step's transfers before the products, half after them
        issue_part(0, (t + kStages - 1) % kStages, k0 + kSB * (kStages - 1));
        if (!idle) {
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (!SECOND) {   // s^T = k q^T, then p^T
#pragma unroll
            for (int k = 0; k < N / 16; ++k) s = mfma32(st_row<CN>(Kn, k, lane), of[k], s);
#pragma unroll
            for (int k = 0; k < R / 16; ++k) s = mfma32(st_row<CR>(Kr, k, lane), of[N / 16 + k], s);
            pin(std::integral_constant<int, K / 16>(), I1(), I4());
            if (full) {
#pragma unroll
              for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c2, -lse2));
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = k0 + row_of(r, lane);
                const bool vis = (key >= qlo) & (key < qhi) & (nocausal | (key <= own));
                s[r] = __builtin_amdgcn_exp2f(vis ? __builtin_fmaf(s[r], c2, -lse2) : -__builtin_inff());
              }
            }
          } else {                   // dp^T = v dout^T
#pragma unroll
            for (int k = 0; k < V / 16; ++k) s = mfma32(st_row<CV>(Vv, k, lane), of[k], s);
            pin(std::integral_constant<int, V / 16>(), I1(), I4());
          }
          xch_put(xch[SECOND ? 1 : 0][g4], s, lane);
        }
        issue_part(1, (t + kStages - 1) % kStages, k0 + kSB * (kStages - 1));
        sync();   // p^T and dp^T are in LDS
        if (!idle) {
          // ds = p (dp - D), with the other wave's half of the pair
          const f32x4 *ob = reinterpret_cast<const f32x4 *>(xch[SECOND ? 0 : 1][g4]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 o4 = ob[64 * j + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * j + e;
              s[r] = SECOND ? o4[e] * (s[r] - Dq) : s[r] * (o4[e] - Dq);
            }
          }
          const bf16x8 sa0 = pack_frag(s, 0), sa1 = pack_frag(s, 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int k = 0; k < kSB / 16; ++k) {
            const bf16x8 sa = k == 0 ? sa0 : sa1;
            if constexpr (!SECOND) {
#pragma unroll
              for (int d = 0; d < 3; ++d) dq[d] = mfma32(sa, st_tr<CN>(Kn, k, d, lane), dq[d]);
            } else {
              dq[0] = mfma32(sa, st_tr<CN>(Kn, k, 3, lane), dq[0]);
#pragma unroll
              for (int d = 0; d < R / 32; ++d) dq[1 + d] = mfma32(sa, st_tr<CR>(Kr, k, d, lane), dq[1 + d]);
            }
          }
          pin(std::integral_constant<int, (kSB / 16) * 3>(), I2(), I8());
        }
      }
      // the trailing (empty) transfers land before the workgroup gives up its LDS
      __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = own0 + row_of(r, lane);
        if (t >= a.T) continue;
        float *row = a.dq + (static_cast<int64_t>(t) * a.H + h) * K + (SECOND ? 96 : 0);
#pragma unroll
        for (int d = 0; d < 3; ++d) __builtin_nontemporal_store(a.scale * dq[d][r], row + 32 * d + (lane & 31));
      }
    };
    if (second) run2(std::true_type());
    else run2(std::false_type());
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
  const dim3 grid(static_cast<unsigned>((a.T + kWB - 1) / kWB), static_cast<unsigned>(a.H));
  attn_bwd8_kernel<N, R, V><<<grid, 512, 0, s>>>(a);
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
