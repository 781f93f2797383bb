// Causal / packed-document softmax attention of one rank's heads with a
// head-shared RoPE key band (torchtitan "MLA CP optimization", section
// "Ulysses CP": k_THK = concat(k_nope_THN, expand_per_head(k_shared_TR)), then
// attention; hyper-parallel `_assemble_key_value`, `MLAContextParallel.__call__`
// with no look-ahead for causal, `_causal_partition` for document-local keys).
//
// gfx950 design (bf16 in, fp32 accumulate):
//  * One workgroup = 8 waves = 128 queries of one head: 4 query blocks of 32 x
//    2 key halves. A 64-key tile is split between the halves (32 keys each);
//    the two partial softmax states of a query block are merged through LDS
//    at the end, after which each of the two waves keeps half of the output
//    columns. Every SIMD runs two waves (<= 256 registers each) half a tile
//    apart, so one wave's softmax overlaps the other's MFMAs, and each K/V
//    tile brought into LDS serves 128 queries.
//  * Tiles move global->LDS with buffer_load ... lds (no staging registers)
//    into rings of three K and three V buffers (120 KB), two tiles ahead, with
//    two barriers per tile. The key tile is assembled from two sources: k_nope
//    from this head's projected kv rows and the shared k_rope row (one copy
//    for all heads), so the expanded key never exists in HBM. Loads past the
//    visible keys fall outside the buffer range and read zero.
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
//  * Work order: dense causal query tiles are paired (i, n-1-i) and every pair
//    is split into two workgroups of nearly equal key-tile count; the tile
//    that straddles both is merged by whichever arrives second (see
//    arrive_swap). Packed documents use a device-built schedule sorted by
//    key-tile count.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int BM = 128;      // queries per workgroup (4 blocks of 32)
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
  int64_t o_sc;           // output chunk stride (queries in chunks of o_chunk rows)
  int o_chunk;            // queries per output chunk, 0: one chunk
  const int32_t *cu;      // query offsets; nullptr: one document [0, T)
  const int32_t *cu_k;    // key offsets of the same documents (nullptr with cu == nullptr: [0, T_k))
  const int2 *tasks;      // packed documents: (query start, document) per task, sorted
  const int *task_count;
  int n_qtiles;           // dense: query tiles per head
  int order;              // dense causal: 1 pairs tiles and splits the work evenly, 0 heaviest first
  float *part;            // dense causal pairing: two softmax-state records per pair
  unsigned long long *flags;   // dense causal pairing: one arrival flag per pair
  unsigned long long epoch;    // this call's flag tag (see arrive)
  int T, T_k, H;           // query rows, key rows, heads
  float scale_log2;       // scale * log2(e)
  int causal;
};

// per-row XOR swizzles of the unpadded LDS tiles (16-byte chunks / 32-byte segments)
__device__ __forceinline__ int kn_swz(int key) { return key & 15; }
__device__ __forceinline__ int kr_swz(int key) { return (key ^ (key >> 3)) & 7; }
__device__ __forceinline__ int v_swz(int key) { return (key & 2) | ((key & 1) * 5); }


// Causal pairing of query tiles (dense, one sequence). Query tiles i and
// n-1-i of a head together hold U = u(i) + u(n-1-i) key tiles, nearly the
// same for every i; two workgroups share the pair, about U/2 key tiles each
// (the one that runs two segments a few less). The
// first takes the first x key tiles of the heavier tile j = n-1-i and then all
// of tile i; the second takes the remaining key tiles of tile j. Both write
// their partial softmax state of tile j to the workspace and the later of the
// two merges them (see arrive). With an odd tile count the middle tile is one
// workgroup alone.
//
// Key tiles the two-segment workgroup gives up to the other: its second
// segment's first transfers, its publish and its arrival cost several key
// tiles more than the other workgroup's tail (which usually finds the pair
// already arrived and merges without publishing). Measured on the 2048-token
// causal shard, kernel trace and whole step, shifts 2..5: 3 is best.
constexpr int kPairShift = 3;

struct PairPlan {
  int qt;        // query tile of the first segment
  int t0, t1;    // its key-tile range
  int part;      // 1: the first segment is a partial of a split tile
  int qt2;       // second segment (full tile), -1 if none
  int slot;      // split-tile slot in the workspace, -1 if none
};

// Key tiles a dense causal query tile needs: its last query, min((qt+1)BM, T) - 1,
// sees the keys up to itself shifted by T_k - T (the sequence's last query lines
// up with its last key).
__device__ __forceinline__ int key_tiles_of(int qt, int T, int T_k) {
  const int hi = min(max(min((qt + 1) * BM, T) + (T_k - T), 0), T_k);
  return (hi + BN - 1) / BN;
}

__device__ __forceinline__ PairPlan pair_plan(int k, int h, int n, int T, int T_k, int shift) {
  PairPlan pp;
  const int pairs = n / 2;
  pp.qt2 = -1;
  pp.slot = -1;
  pp.part = 0;
  if (k >= 2 * pairs) {                      // middle tile
    pp.qt = pairs;
    pp.t0 = 0;
    pp.t1 = key_tiles_of(pairs, T, T_k);
    return pp;
  }
  const int i = k >> 1, j = n - 1 - i;
  const int ui = key_tiles_of(i, T, T_k), uj = key_tiles_of(j, T, T_k);
  // key tiles of j done by the first workgroup: half the pair's work, less
  // the shift for the second segment's fixed cost
  const int x = max(0, (ui + uj + 1) / 2 - ui - shift);
  if ((k & 1) == 0) {
    if (x > 0) {
      pp.qt = j;
      pp.t0 = 0;
      pp.t1 = x;
      pp.part = 1;
      pp.qt2 = i;
    } else {
      pp.qt = i;
      pp.t0 = 0;
      pp.t1 = ui;
    }
  } else {
    pp.qt = j;
    pp.t0 = x;
    pp.t1 = uj;
    pp.part = x > 0;
  }
  if (pp.part) pp.slot = h * pairs + i;
  return pp;
}

// Softmax state of one query block as a wave holds it after the key halves
// are merged: o[d] is the 32x32 block d of O^T (dims x queries, MFMA output
// layout), m is the running max (log2 domain, equal on lanes l and l^32) and
// l the partial denominator of this lane's keys.
constexpr int kRecFloats = 4 * (4 * 16 + 2) * 64;   // 4 query blocks x (64 O + m + l) x 64 lanes

// element offset of query row qi's output rows: in chunks of o_chunk queries
// when o_chunk > 0 (e.g. sequence ranks' queries written straight into the
// token-major layout that follows the head->token exchange)
__device__ __forceinline__ int64_t out_row(const AttnArgs &a, int qi) {
  if (a.o_chunk == 0) return static_cast<int64_t>(qi) * a.o_st;
  const unsigned c = static_cast<unsigned>(qi) / static_cast<unsigned>(a.o_chunk);
  const unsigned r = static_cast<unsigned>(qi) - c * static_cast<unsigned>(a.o_chunk);
  return static_cast<int64_t>(c) * a.o_sc + static_cast<int64_t>(r) * a.o_st;
}

// normalise the state of query block qb of the tile starting at q0 and store
// its columns [col0, col0 + 32 NDB) from o[0 .. NDB). The lane layout (a lane
// holds 8-byte pieces of one query row) goes through the wave's own free
// stage region xs, so every query row leaves as whole 16-byte chunks, streamed
// past L2 with nontemporal stores (no dirty lines left for the end-of-kernel
// write-back). The wave of key half 0 also writes the row's log-sum-exp.
template <int NDB, int DBLK>
__device__ __forceinline__ void store_rows(const AttnArgs &a, const f32x16 (&o)[DBLK], float m_run, float l_run,
                                           int h, int q0, int q_end, int qb, int lane, uint16_t *xs, int col0,
                                           bool write_lse) {
  constexpr int XLD = 32 * NDB + 8;   // padded row of xs (bf16)
  const int half = lane >> 5, row = lane & 31;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<u32x2 *>(xs + row * XLD + 32 * d + 8 * g + 4 * half) =
          u32x2{pack_bf16x2(o[d][4 * g] * inv, o[d][4 * g + 1] * inv),
                pack_bf16x2(o[d][4 * g + 2] * inv, o[d][4 * g + 3] * inv)};
  // one wave writes and reads xs, and its LDS accesses complete in order
  constexpr int CPR = 32 * NDB / 8;   // 16-byte chunks per stored row piece
  const int rsub = lane / CPR, c = lane % CPR;
#pragma unroll
  for (int i = 0; i < 32 * CPR / 64; ++i) {
    const int rr = rsub + (64 / CPR) * i;
    const int qi = q0 + 32 * qb + rr;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(xs + rr * XLD + 8 * c);
    if (qi < q_end)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(a.out + out_row(a, qi) +
                                                               static_cast<int64_t>(h) * a.o_sh + col0 + 8 * c));
  }
  const int qi = q0 + 32 * qb + row;
  if (write_lse && a.lse != nullptr && half == 0 && qi < q_end)
    a.lse[static_cast<int64_t>(h) * a.T + qi] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.6931471805599453f;
}

// Split tiles of the causal pairing: each of the two workgroups that share
// tile j stores its partial softmax state (O^T, m, l per lane, fp32) with
// agent-scope stores, waits for them to complete and then arrives at the
// pair's flag; the one that arrives second reads both records with
// agent-scope loads, combines them, m = max(m0, m1), l = l0 2^(m0-m) +
// l1 2^(m1-m), o = o0 2^(m0-m) + o1 2^(m1-m), and stores the rows. Nothing
// ever waits for the other workgroup, and no cache maintenance is needed (an
// agent-scope fence would write back and invalidate the L2 that the other
// workgroups of the XCD are reading their K/V tiles from).
//
// An arrival is one atomic exchange that leaves (epoch << 1) | 1 ("first
// arrival of this call") in the flag; the workgroup that gets that value back
// is second. Any other old value (an earlier call, memory never used, or
// epoch << 1, "merged") means first. The epoch is a 62-bit per-call tag
// (next_call_tag), so the workspace needs no clearing. The second arrival
// marks the pair merged (epoch << 1), and so does the one-segment
// workgroup's early merge, so every call leaves every split-tile flag at
// epoch << 1 and a captured launch replayed with the same epoch finds every
// flag at "nobody yet" again. The exchange's result is needed only when the
// arriving workgroup is done with its own segments, so the two-segment
// workgroup issues it without waiting for it.
__device__ __forceinline__ unsigned long long arrive_swap(unsigned long long *flag, unsigned long long epoch) {
  return __hip_atomic_exchange(flag, (epoch << 1) | 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void mark_merged(unsigned long long *flag, unsigned long long epoch) {
  __hip_atomic_store(flag, epoch << 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int N, int R, int V>
__global__ __launch_bounds__(512, 1) void attn_fwd_kernel(AttnArgs a) {
  constexpr int KD = N + R;          // score width
  constexpr int NCH = N / 8;         // 16-byte chunks per k_nope row
  constexpr int RCH = R / 8;         // per k_rope row
  constexpr int VCH = V / 8;         // per V row
  constexpr int KSTEPS = KD / 16;
  constexpr int NSTEPS = N / 16;
  constexpr int DBLK = V / 32;
  constexpr int KN_E = BN * N, KR_E = BN * R, V_E = BN * V;   // elements per stage
  constexpr int NW = 8;              // waves per workgroup
  constexpr int KN_I = BN * NCH / (64 * NW), KR_I = BN * RCH / (64 * NW), V_I = BN * VCH / (64 * NW);   // DMA instrs per wave
  constexpr int REC = DBLK * 16 + 2; // floats per lane of a wave's softmax state: O, m, l
  static_assert(N == 128 && R == 64 && V == 128, "swizzles and DMA splits are laid out for 128/64/128");
  static_assert(4 * REC * 64 == kRecFloats, "workspace record size");
  static_assert(REC * 64 * 4 <= (KN_E + KR_E) * 2, "a query block's state fits one K buffer");
  static_assert(KN_I * 64 * NW == BN * NCH && KR_I * 64 * NW == BN * RCH && V_I * 64 * NW == BN * VCH, "tile DMA split");
  // K (k_nope | k_rope) and V tiles in rings of three buffers each. Separate
  // arrays let the compiler tell transfers in flight from tiles being read.
  __shared__ __attribute__((aligned(1024))) uint16_t kb0[KN_E + KR_E];
  __shared__ __attribute__((aligned(1024))) uint16_t kb1[KN_E + KR_E];
  __shared__ __attribute__((aligned(1024))) uint16_t kb2[KN_E + KR_E];
  __shared__ __attribute__((aligned(1024))) uint16_t vb0[V_E];
  __shared__ __attribute__((aligned(1024))) uint16_t vb1[V_E];
  __shared__ __attribute__((aligned(1024))) uint16_t vb2[V_E];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qb = wave & 3, kh = wave >> 2;          // query block, key half
  const int half = lane >> 5, lrow = lane & 31;
  const int grp = lane >> 4, gl = lane & 15;        // 16-lane groups for the transposing read
  // the stage buffer this query block's waves use for the key-half merge and the output transpose
  uint16_t *const xs_own = qb == 0 ? kb0 : qb == 1 ? kb1 : qb == 2 ? kb2 : vb0;

  // ---- which head, document and segments. Queries of the document are
  // [doc_lo, doc_hi), its keys [kdoc_lo, kdoc_hi); when causal, query t sees
  // the keys j <= t + kshift (the document's last query lines up with its last
  // key; kshift = 0 for equal lengths).
  int h, doc_lo, doc_hi, kdoc_lo, kdoc_hi;
  PairPlan pp;
  if (a.tasks == nullptr) {
    const int b = blockIdx.x, H = a.H, n = a.n_qtiles;
    h = b % H;
    doc_lo = 0;
    doc_hi = a.T;
    kdoc_lo = 0;
    kdoc_hi = a.T_k;
    if (a.causal && a.order == 1) {
      pp = pair_plan(b / H, h, n, a.T, a.T_k, kPairShift);
    } else {                                  // heaviest first
      pp.qt = n - 1 - b / H;
      pp.t0 = 0;
      pp.t1 = a.causal ? key_tiles_of(pp.qt, a.T, a.T_k) : (a.T_k + BN - 1) / BN;
      pp.part = 0;
      pp.qt2 = -1;
      pp.slot = -1;
    }
  } else {
    const int t = static_cast<int>(blockIdx.x) / a.H;
    if (t >= *a.task_count) return;
    h = blockIdx.x % a.H;
    const int2 task = a.tasks[t];
    doc_lo = min(max(a.cu[task.y], 0), a.T);          // the same clamping as the schedule
    doc_hi = min(max(a.cu[task.y + 1], doc_lo), a.T);
    kdoc_lo = min(max(a.cu_k[task.y], 0), a.T_k);
    kdoc_hi = min(max(a.cu_k[task.y + 1], kdoc_lo), a.T_k);
    pp.qt = (task.x - doc_lo) / BM;
    const int q_end = min(task.x + BM, doc_hi);
    const int k_end = a.causal ? min(max(q_end + (kdoc_hi - doc_hi), kdoc_lo), kdoc_hi) : kdoc_hi;
    pp.t0 = 0;
    pp.t1 = (k_end - kdoc_lo + BN - 1) / BN;
    pp.part = 0;
    pp.qt2 = -1;
    pp.slot = -1;
  }
  h = __builtin_amdgcn_readfirstlane(h);
  doc_lo = __builtin_amdgcn_readfirstlane(doc_lo);
  doc_hi = __builtin_amdgcn_readfirstlane(doc_hi);
  kdoc_lo = __builtin_amdgcn_readfirstlane(kdoc_lo);
  kdoc_hi = __builtin_amdgcn_readfirstlane(kdoc_hi);
  const int kshift = kdoc_hi - doc_hi;

  // ---- zero the stages once: loads past the buffer range may leave LDS
  // untouched, and a masked key's zero probability must not meet a stale
  // NaN. Only a partial key tile reads past the range: with dense tiles, T_k
  // a multiple of the key tile and (causal) T_k - T too, every tile is whole
  // (a query tile's causal key range ends at a multiple of BM plus T_k - T, or
  // at T_k).
  // The stage buffers are untouched until the first segment's transfers
  // unless they are zeroed here: then every wave's zeroing must be done
  // before any wave's transfers land (see segment).
  bool stages_busy = false;
  if (a.tasks != nullptr || a.T_k % BN != 0 || (a.causal && (a.T_k - a.T) % BN != 0)) {
    stages_busy = true;
    u32x4 z{0, 0, 0, 0};
    for (int i = tid; i < (KN_E + KR_E) / 8; i += 64 * NW) {
      reinterpret_cast<u32x4 *>(kb0)[i] = z;
      reinterpret_cast<u32x4 *>(kb1)[i] = z;
      reinterpret_cast<u32x4 *>(kb2)[i] = z;
    }
    for (int i = tid; i < V_E / 8; i += 64 * NW) {
      reinterpret_cast<u32x4 *>(vb0)[i] = z;
      reinterpret_cast<u32x4 *>(vb1)[i] = z;
      reinterpret_cast<u32x4 *>(vb2)[i] = z;
    }
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
  const uint32_t kv_row_bytes = static_cast<uint32_t>(a.kv_st) * 2, kr_row_bytes = static_cast<uint32_t>(a.kr_st) * 2;
  const int kkey = 32 * kh + lrow;                      // K rows this lane reads
  // byte offset, within a K buffer, of the 16 bytes this lane feeds to score step ks
  uint32_t koff[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const int cidx = 2 * ks + half;
    koff[ks] = static_cast<uint32_t>(ks < NSTEPS ? 2 * (kkey * N + 8 * (cidx ^ kn_swz(kkey)))
                                                 : 2 * (KN_E + kkey * R + 8 * ((cidx - 2 * NSTEPS) ^ kr_swz(kkey))));
  }
  const int vrow0 = 32 * kh + 4 * (grp >> 1) + (gl >> 2);   // first V row of the transposing reads
  // Register block d of the output (o[d]) holds column block dblk_of(d): the
  // wave of key half 1 runs the blocks rotated by half, so that after the key
  // halves merge every wave keeps o[0 .. DBLK/2) (its columns) and hands
  // o[DBLK/2 ..) to its partner with compile-time register indices only (a
  // run-time index into o would move o to scratch memory).
  auto dblk_of = [&](int d) { return (d + (DBLK / 2) * kh) % DBLK; };
  const float c = a.scale_log2;

  f32x16 o[DBLK];
  float m_run, l_run;
  bf16x8 qf[KSTEPS];   // Q^T fragments of the current segment's query block
  // ---- a split tile's partial state, stored past this XCD's L2. A lane's
  // DBLK*8+1 float pairs (O^T pieces, then (m, l)) leave as 8-byte
  // agent-scope stores; pair i of lane l sits at float 128 i + 2 l of its
  // query block's record. After the key halves merge, the wave of key half kh
  // keeps column blocks 2 kh and 2 kh + 1 of its query block (in o[0], o[1]):
  // it stores, publishes and reads pairs [OWN kh, OWN kh + OWN) and (m, l).
  constexpr int DOWN = DBLK / 2;          // column blocks a wave keeps
  constexpr int OWN = DOWN * 8;           // their float pairs
  constexpr int ML = DBLK * 8;            // the (m, l) pair
  static_assert(DBLK % 2 == 0, "column blocks split between the key halves");
  auto rec_of = [&](int slot, int role) {
    return reinterpret_cast<unsigned long long *>(a.part + static_cast<int64_t>(slot) * (2 * kRecFloats) +
                                                  role * kRecFloats + qb * REC * 64) + lane;
  };
  // The workgroup without a second segment usually finishes the split tile
  // long after the other one has arrived. It reads the pair's flag during
  // its last key step (the step's closing barrier publishes what it saw); if
  // the other workgroup has arrived (flag = first arrival of this call), it is
  // certainly second: it skips publishing and arriving, and its waves start
  // loading the other record before the key halves merge.
  __shared__ int early_second;
  unsigned long long arrive_old = 0;   // the two-segment workgroup's arrival (its exchange's old value)
  unsigned long long other[OWN + 1];   // this wave's pairs of the other record, then (m, l)
  // this wave's pairs of a record: its own column blocks, then (m, l)
  auto load_own = [&](const unsigned long long *rec, unsigned long long (&v)[OWN + 1]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < OWN; ++i)
      v[i] = __hip_atomic_load(rec + 64 * (OWN * kh + i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    v[OWN] = __hip_atomic_load(rec + 64 * ML, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // the stage region this wave stores its rows through (its half of its query
  // block's merge buffer, which only it reads after the merge)
  uint16_t *const xs_wave = xs_own + kh * (DOWN * 4 * 64 * 8);
  bool early = false;

  // ---- one segment: query tile qt over key tiles [t0, t1); leaves the merged
  // (both key halves) softmax state with each wave of a query block holding
  // its half of the columns in o[0 .. DBLK/2) and the common (m, l).
  //
  // Per tile t a wave does M_t = {O += V_{t-1}^T P_{t-1}^T, S_t = K_t Q^T} on
  // the matrix cores and then X_t = softmax(S_t) -> P_t on the vector ALUs.
  // The two waves of a SIMD (same query block, key halves 0 and 1) run these
  // half a tile apart, so while one does M the other does X:
  //     step t, first half:   kh 0: M_t   kh 1: X_{t-1}
  //     step t, second half:  kh 0: X_t   kh 1: M_t
  // Every wave starts its share of the transfers of K_{t+2} and V_{t+1}
  // (five 1 KB transfers) in step t, into the buffers that held K_{t-1} and
  // V_{t-2}, which no wave reads after step t-1: the three K transfers at
  // the start of its vector half-phase, the two V transfers at the end of its
  // matrix half-phase, once its MFMAs are issued. A step ends with each wave
  // waiting only for its transfers of the previous step, then a barrier.
  // probe: the pair flag to read for an early second arrival (nullptr: none);
  // its record is other_rec. mode 0 runs the whole segment; mode 1 only
  // starts its first transfers (Q, K_0) and leaves the softmax
  // state alone; mode 2 runs a segment whose first transfers mode 1 started.
  auto segment = [&](int qt, int t0, int t1, const unsigned long long *probe, const unsigned long long *other_rec,
                     int mode, unsigned long long *arrive_flag) __attribute__((always_inline)) {
    const int q0 = doc_lo + qt * BM;
    const int q_end = min(q0 + BM, doc_hi);
    const int kv_hi = a.causal ? min(max(q_end + kshift, kdoc_lo), kdoc_hi) : kdoc_hi;   // keys end (exclusive)
    const int qi = q0 + 32 * qb + lrow;
    const int wq_first = q0 + 32 * qb;
    const int nt = t1 - t0;
    unsigned long long flag_seen = 0;
    // Q arrives with the segment's first transfers: query block b's 32 rows
    // go to a stage buffer the first step does not read (kb2: blocks 0 and
    // 1, vb1: block 2, vb2: block 3), one 1 KB region per 16-wide k step,
    // lane-major, so each lane reads back exactly its own MFMA fragment; the
    // two waves of a block fetch six steps each
    uint16_t *const qbuf = qb == 0 ? kb2 : qb == 1 ? kb2 + 32 * KD : qb == 2 ? vb1 : vb2;
    auto issue_q = [&]() __attribute__((always_inline)) {
      const int rows = __builtin_amdgcn_readfirstlane(max(0, min(32, q_end - (q0 + 32 * qb))));
      const u32x4 rq = dma_rsrc(a.q + static_cast<int64_t>(q0 + 32 * qb) * a.q_st + static_cast<int64_t>(h) * a.q_sh,
                                static_cast<uint32_t>(rows * a.q_st * 2));
      const uint32_t base = lds_addr(qbuf);
#pragma unroll
      for (int i = 0; i < KSTEPS / 2; ++i) {
        const int ks = (KSTEPS / 2) * kh + i;
        dma16(rq, base + 1024 * ks, static_cast<uint32_t>((lrow * a.q_st + 16 * ks + 8 * half) * 2));
      }
    };
    if (mode != 1) {
#pragma unroll
      for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
      m_run = kNegBig;
      l_run = 0.f;
    }

    auto j0_of = [&](int t) { return kdoc_lo + (t0 + t) * BN; };
    // rows past the visible keys (a whole tile past the end included) lie
    // outside the buffer range: nothing is read for them
    // rows of the tile at key j0 that are visible, 0..BN (uniform)
    // visible rows of tile t (uniform): BN before the last tile, the remainder
    // in it, none past it
    const int last_rows = __builtin_amdgcn_readfirstlane(kv_hi - j0_of(nt - 1));
    auto tile_rows = [&](int t) {
      return static_cast<uint32_t>(t < nt - 1 ? BN : t == nt - 1 ? last_rows : 0);
    };
    auto issue_k = [&](uint16_t *kb, int t) {
      const int j0 = j0_of(t);
      const uint32_t rows = tile_rows(t);
      const u32x4 rkv = dma_rsrc(kv_h + static_cast<int64_t>(j0) * a.kv_st, rows * kv_row_bytes);
      const u32x4 rkr = dma_rsrc(a.kr + static_cast<int64_t>(j0) * a.kr_st, rows * kr_row_bytes);
      const uint32_t base = lds_addr(kb);
#pragma unroll
      for (int i = 0; i < KN_I; ++i) dma16(rkv, base + 1024 * (wave * KN_I + i), kn_off[i]);
#pragma unroll
      for (int i = 0; i < KR_I; ++i) dma16(rkr, base + 2 * KN_E + 1024 * (wave * KR_I + i), kr_off[i]);
    };
    auto issue_v = [&](uint16_t *vb, int t) {
      const int j0 = j0_of(t);
      const uint32_t rows = tile_rows(t);
      const u32x4 rkv = dma_rsrc(kv_h + static_cast<int64_t>(j0) * a.kv_st, rows * kv_row_bytes);
      const uint32_t base = lds_addr(vb);
#pragma unroll
      for (int i = 0; i < V_I; ++i) dma16(rkv, base + 1024 * (wave * V_I + i), v_off[i]);
    };
    f32x16 sc;           // S_t awaiting its softmax
    bf16x8 pf[2];        // P_t awaiting its PV product

    // Matrix half-phase: PV of the previous tile (from vprev and pf) and/or
    // S = K Q^T of this tile (from kb). Straight-line code: every LDS read is
    // issued well ahead of the MFMA that consumes it, since no other wave's
    // MFMAs cover the LDS latency while this one runs.
    constexpr int KAHEAD = 4;   // K fragment reads in flight during the S chain
    auto M = [&](auto pv, auto sv, const uint16_t *kb, const uint16_t *vprev) __attribute__((always_inline)) {
      constexpr bool DO_PV = decltype(pv)::value, DO_S = decltype(sv)::value;
      auto kread = [&](int ks) {
        return *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(kb) + koff[ks]);
      };
      auto vread = [&](int b, int d) {
        const int dcol = 32 * dblk_of(d) + 16 * (grp & 1) + 4 * (gl & 3);
        const int r0 = vrow0 + 16 * b, r1 = r0 + 8;
        const s16x4 lo = read_tr(vprev + r0 * V + 16 * ((dcol >> 4) ^ v_swz(r0)) + (dcol & 15));
        const s16x4 hi = read_tr(vprev + r1 * V + 16 * ((dcol >> 4) ^ v_swz(r1)) + (dcol & 15));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 vf[2][DBLK];
      bf16x8 kf[KAHEAD];
      if constexpr (DO_PV) {
#pragma unroll
        for (int d = 0; d < DBLK; ++d) vf[0][d] = vread(0, d);
      }
      if constexpr (DO_S) {
#pragma unroll
        for (int i = 0; i < KAHEAD; ++i) kf[i] = kread(i);
      }
      if constexpr (DO_PV) {
#pragma unroll
        for (int d = 0; d < DBLK; ++d) vf[1][d] = vread(1, d);
        // O^T += V^T P^T
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int d = 0; d < DBLK; ++d) o[d] = mfma32(vf[b][d], pf[b], o[d]);
      }
      if constexpr (DO_S) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          sc = mfma32(kf[ks % KAHEAD], qf[ks], sc);
          if (ks + KAHEAD < KSTEPS) kf[ks % KAHEAD] = kread(ks + KAHEAD);
        }
      }
      // Pin the issue order (the scheduler would otherwise sink each read next
      // to its MFMA): first reads up front, then one MFMA per read.
      constexpr int kMfma = 0x008, kDsRead = 0x100;
      auto mfma_one = [&]() { __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0); };
      if constexpr (DO_PV) __builtin_amdgcn_sched_group_barrier(kDsRead, 2 * DBLK, 0);
      if constexpr (DO_S) __builtin_amdgcn_sched_group_barrier(kDsRead, KAHEAD, 0);
      if constexpr (DO_PV) {
#pragma unroll
        for (int d = 0; d < DBLK; ++d) {
          __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
        }
#pragma unroll
        for (int d = 0; d < DBLK; ++d) mfma_one();
      }
      if constexpr (DO_S) {
#pragma unroll
        for (int ks = 0; ks + KAHEAD < KSTEPS; ++ks) {
          mfma_one();
          __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < KAHEAD; ++i) mfma_one();
      }
    };

    auto X = [&](int t) __attribute__((always_inline)) {
      const int jh = j0_of(t) + 32 * kh;               // first key of this wave's half
      // mask keys past the diagonal / the visible end (uniform test)
      if (jh + 31 >= kv_hi || (a.causal && jh + 31 > wq_first + kshift)) {
        const int lim = a.causal ? min(qi + kshift, kv_hi - 1) : kv_hi - 1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = jh + 8 * (r >> 2) + 4 * half + (r & 3);
          sc[r] = j > lim ? -INFINITY : sc[r];
        }
      }
      float mt = sc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
      {
        // lanes l and l^32 hold the two key halves of one query row. (The swap's
        // results are copied to scalars first: bit-casting a vector element in
        // place reads element 0.)
        const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, mt),
                                                         __builtin_bit_cast(unsigned, mt), false, false);
        const unsigned own = sw[0], other = sw[1];
        mt = fmaxf(__uint_as_float(own), __uint_as_float(other)) * c;
      }
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
      // P^T in bf16 (the row sum stays in fp32 adds: the bf16 dot instructions
      // share the matrix pipe and would stall behind the other wave's MFMAs)
      float ps[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) ps[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], c, -m_run));
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(ps[8 * b + 2 * e], ps[8 * b + 2 * e + 1]);
        pf[b] = as_bf16x8(w);
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) ps[r] += ps[r + 8];
#pragma unroll
      for (int r = 0; r < 4; ++r) ps[r] += ps[r + 4];
      l_run += (ps[0] + ps[2]) + (ps[1] + ps[3]);
    };

    // Step t (0 <= t <= nt): K_t in kcur, V_{t-1} in vprev; K_{t+2} goes to
    // kdst and V_{t+1} to vdst. pv / sv / dma: whether the matrix half-phase
    // has a PV product (t >= 1), a score product (t < nt) and transfers.
    constexpr int kDmaPerStep = KN_I + KR_I + V_I;
    static_assert(kDmaPerStep < 16, "vmcnt field");
    auto step = [&](auto pv, auto sv, auto dma, int t, const uint16_t *kcur, const uint16_t *vprev,
                    uint16_t *kdst, uint16_t *vdst) __attribute__((always_inline)) {
      const int jk = t + 2, jv = t + 1;
      // Issuing a transfer stalls the wave while the CU's memory queue is
      // full. The vector half-phase (softmax) is the longer half, so it starts
      // only the K transfers; the matrix wave starts the V transfers after its
      // last MFMA is issued, in time it would otherwise wait at the barrier
      // (the three K transfers there as well made the step slower).
      auto transfers_k = [&]() __attribute__((always_inline)) {
        if constexpr (decltype(dma)::value) issue_k(kdst, jk);
      };
      auto transfers_v = [&]() __attribute__((always_inline)) {
        if constexpr (decltype(dma)::value) {
          __builtin_amdgcn_sched_barrier(0);
          issue_v(vdst, jv);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (kh == 0) {
        M(pv, sv, kcur, vprev);
        transfers_v();
      }
      if (kh == 1) {
        transfers_k();
        if (t >= 1) X(t - 1);
      }
      // Phase alignment only: both half-phases read buffers that landed before
      // this step, so no memory fence (which would wait for the transfers just
      // started) is needed at either barrier. Each wave waits for its own
      // transfers of the previous step before the second one, which makes
      // them visible to all waves after it.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (kh == 1) {
        M(pv, sv, kcur, vprev);
        transfers_v();
      }
      if (kh == 0) {
        transfers_k();
        if (t < nt) X(t);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(dma)::value) {
        __builtin_amdgcn_s_waitcnt(0x0F70 | kDmaPerStep);   // vmcnt(5): this step's transfers may stay in flight
      } else {
        // the segment's last step: vmcnt(0), which includes the pair-flag
        // probe, so the early-merge decision is published by this barrier
        __builtin_amdgcn_s_waitcnt(0x0F70);
        if (probe != nullptr && tid == 0) early_second = flag_seen == ((a.epoch << 1) | 1ull);
        __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0)
      }
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    const std::true_type yes;
    const std::false_type no;

    if (mode != 2) {
      // the previous segment's LDS readers (and the stage zeroing) are done
      // with the buffers; its global stores may stay in flight. A first
      // segment over stages nobody has touched skips the barrier, so each
      // wave starts its transfers as soon as it is running (the prologue's
      // own wait and barrier come before any stage is read).
      if (stages_busy) {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
      }
      stages_busy = true;
      if (nt > 0) {
        // K_t lives in kb[t % 3], V_t in vb[t % 3]
        issue_q();
        issue_k(kb0, 0);
      }
      if (mode == 1) return;
    }
    if (nt > 0) {
      // Q and K_0 are the only transfers step 0 needs: wait for them alone.
      // V_0 and K_1 follow once this wave has read its Q (issuing a transfer
      // stalls the wave while the CU's memory queue is full, and the first
      // transfers of all workgroups arrive at once); step 0's closing wait
      // covers them.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // every wave's older memory operations are complete here (the counter
      // retires in issue order), the previous segment's record stores
      // included: the arrival of the two-segment workgroup
      if (arrive_flag != nullptr && tid == 0) arrive_old = arrive_swap(arrive_flag, a.epoch);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8 *>(qbuf + 512 * ks + 8 * lane);
      __builtin_amdgcn_sched_barrier(0);
      issue_v(vb0, 0);
      issue_k(kb1, 1);
      __builtin_amdgcn_sched_barrier(0);
      // every wave holds its Q before step 0's transfers reuse kb2 and vb1
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      step(no, yes, yes, 0, kb0, vb2, kb2, vb1);
      int t = 1;
      for (; t + 2 < nt; t += 3) {                    // whole rounds of the ring
        step(yes, yes, yes, t, kb1, vb0, kb0, vb2);
        step(yes, yes, yes, t + 1, kb2, vb1, kb1, vb0);
        step(yes, yes, yes, t + 2, kb0, vb2, kb2, vb1);
      }
      if (t < nt) {
        step(yes, yes, yes, t, kb1, vb0, kb0, vb2);
        ++t;
      }
      if (t < nt) {
        step(yes, yes, yes, t, kb2, vb1, kb1, vb0);
        ++t;
      }
      if (probe != nullptr && tid == 0) flag_seen = __hip_atomic_load(probe, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int rl = (nt - 1) % 3;                     // t == nt: the last PV product
      step(yes, no, no, nt, kb0, rl == 0 ? vb0 : rl == 1 ? vb1 : vb2, kb0, vb0);
      // an early merge starts loading the other record now, so that the
      // loads are in flight while the key halves merge
      if (probe != nullptr) {
        early = __builtin_amdgcn_readfirstlane(early_second) != 0;
        if (early) load_own(other_rec, other);
      }
    }

    // merge the two key halves of each query block through LDS in one round
    // (every stage buffer is free). The wave of key half kh keeps column
    // blocks 2 kh, 2 kh + 1 and hands the other two to its partner: query
    // block b's O^T pieces in 16-byte pieces in kb0 / kb1 / kb2 / vb0 (blocks
    // 0-1 in the first 8 KB, 2-3 in the next), the (m, l) pairs in vb1. Both
    // waves form the same (m, l), key half 0's term first. The next segment's
    // first barrier keeps its transfers off these buffers until the reads are
    // done.
    {
      f32x4 *xo = reinterpret_cast<f32x4 *>(xs_own);
      f32x2_t *xml = reinterpret_cast<f32x2_t *>(vb1) + 128 * qb;
      // o[DOWN ..] hold the partner's column blocks (see dblk_of)
      const int dx = DOWN * (1 - kh);   // first column block handed over
#pragma unroll
      for (int d = 0; d < DOWN; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          xo[(4 * (dx + d) + g) * 64 + lane] =
              f32x4{o[DOWN + d][4 * g], o[DOWN + d][4 * g + 1], o[DOWN + d][4 * g + 2], o[DOWN + d][4 * g + 3]};
      xml[64 * kh + lane] = f32x2_t{m_run, l_run};
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_s_barrier();
      const f32x2_t ml = xml[64 * (1 - kh) + lane];
      const float m0 = kh == 0 ? m_run : ml.x, l0 = kh == 0 ? l_run : ml.y;   // key half 0
      const float m1 = kh == 0 ? ml.x : m_run, l1 = kh == 0 ? ml.y : l_run;   // key half 1
      const float mn = fmaxf(m0, m1);
      const float a0 = __builtin_amdgcn_exp2f(m0 - mn), a1 = __builtin_amdgcn_exp2f(m1 - mn);
      const float a_own = kh == 0 ? a0 : a1, a_oth = kh == 0 ? a1 : a0;
      l_run = l0 * a0 + l1 * a1;
      m_run = mn;
#pragma unroll
      for (int d = 0; d < DOWN; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = xo[(4 * (DOWN * kh + d) + g) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[d][4 * g + e] = o[d][4 * g + e] * a_own + v[e] * a_oth;
        }
    }
  };

  auto publish = [&](int slot, int role) {
    unsigned long long *rec = rec_of(slot, role);
    auto put = [&](int i, float x, float y) {
      __hip_atomic_store(rec + 64 * i, (static_cast<unsigned long long>(__float_as_uint(y)) << 32) | __float_as_uint(x),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
#pragma unroll
    for (int d = 0; d < DOWN; ++d)
#pragma unroll
      for (int r = 0; r < 16; r += 2) put(OWN * kh + d * 8 + r / 2, o[d][r], o[d][r + 1]);
    if (kh == 0) put(ML, m_run, l_run);
  };
  // ---- every wave combines its own state with its pairs of the other record
  // (its column blocks' pairs, then (m, l), in v) and stores its columns of
  // the rows of split tile qt
  auto combine_store = [&](const unsigned long long (&v)[OWN + 1], int qt) __attribute__((always_inline)) {
    const float m1 = __uint_as_float(static_cast<unsigned>(v[OWN]));
    const float l1 = __uint_as_float(static_cast<unsigned>(v[OWN] >> 32));
    const float mn = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - mn), a1 = __builtin_amdgcn_exp2f(m1 - mn);
#pragma unroll
    for (int d = 0; d < DOWN; ++d)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const unsigned long long x = v[d * 8 + r / 2];
        o[d][r] = o[d][r] * a0 + __uint_as_float(static_cast<unsigned>(x)) * a1;
        o[d][r + 1] = o[d][r + 1] * a0 + __uint_as_float(static_cast<unsigned>(x >> 32)) * a1;
      }
    store_rows<DOWN>(a, o, mn, l_run * a0 + l1 * a1, h, doc_lo + qt * BM, doc_hi, qb, lane, xs_wave, 32 * DOWN * kh,
                     kh == 0);
  };
  // ---- the one-segment workgroup, after publishing: arrive at the pair's
  // flag once its record stores are complete; a second arrival combines its
  // own state (still in registers) with the other workgroup's record of split
  // tile qt and stores the rows
  __shared__ int second_arrival;
  const unsigned long long first_mark = (a.epoch << 1) | 1ull;
  auto arrive_and_merge = [&](int slot, int role, int qt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (tid == 0) {
      const bool sec = arrive_swap(a.flags + slot, a.epoch) == first_mark;
      if (sec) mark_merged(a.flags + slot, a.epoch);
      second_arrival = sec;
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(second_arrival) == 0) return;
    load_own(rec_of(slot, 1 - role), other);
    combine_store(other, qt);
  };
  // ---- the two-segment workgroup arriving second: both records of split
  // tile qt (its own is role 0) are combined and stored after its second
  // segment
  auto merge_records = [&](int slot, int qt) __attribute__((always_inline)) {
    unsigned long long mine[OWN + 1];
    load_own(rec_of(slot, 0), mine);
    load_own(rec_of(slot, 1), other);
#pragma unroll
    for (int d = 0; d < DOWN; ++d)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const unsigned long long x = mine[d * 8 + r / 2];
        o[d][r] = __uint_as_float(static_cast<unsigned>(x));
        o[d][r + 1] = __uint_as_float(static_cast<unsigned>(x >> 32));
      }
    m_run = __uint_as_float(static_cast<unsigned>(mine[OWN]));
    l_run = __uint_as_float(static_cast<unsigned>(mine[OWN] >> 32));
    combine_store(other, qt);
  };

  const int qt1 = __builtin_amdgcn_readfirstlane(pp.qt);
  const int qt2 = __builtin_amdgcn_readfirstlane(pp.qt2);
  {
    const bool probe = pp.part && qt2 < 0;
    const int slot = __builtin_amdgcn_readfirstlane(pp.slot);
    segment(qt1, __builtin_amdgcn_readfirstlane(pp.t0), __builtin_amdgcn_readfirstlane(pp.t1),
            probe ? a.flags + slot : nullptr, probe ? rec_of(slot, 0) : nullptr, 0, nullptr);
  }
  const int role = qt2 >= 0 ? 0 : 1;
  // a workgroup with a split tile and a second segment starts the second
  // segment's first transfers right after its record stores and arrives at
  // that segment's first barrier (see segment)
  const bool pre = pp.part && qt2 >= 0;
  const int tiles2 = qt2 >= 0 ? key_tiles_of(qt2, a.T, a.T_k) : 0;
  if (early) {
    // the other workgroup arrived first in this call and never looks at the
    // flag again: mark the pair done, so that every call leaves every flag at
    // epoch << 1 and a replay of the same launch (same epoch) starts from
    // "nobody yet" on every pair
    if (tid == 0) mark_merged(a.flags + __builtin_amdgcn_readfirstlane(pp.slot), a.epoch);
    combine_store(other, qt1);
  } else if (pp.part) {
    publish(pp.slot, role);
    if (pre) segment(qt2, 0, tiles2, nullptr, nullptr, 1, nullptr);
  } else {
    store_rows<DOWN>(a, o, m_run, l_run, h, doc_lo + qt1 * BM, doc_hi, qb, lane, xs_wave, 32 * DOWN * kh, kh == 0);
  }
  // The workgroup with a second segment arrives early in it, so that usually
  // the other workgroup of the pair, which has no second segment, finds it
  // arrived and merges the split tile (early); if it arrives second after
  // all, it merges after its second segment.
  if (pp.part && !early && !pre) arrive_and_merge(__builtin_amdgcn_readfirstlane(pp.slot), role, qt1);
  if (qt2 >= 0) {
    unsigned long long *const flag = pre ? a.flags + __builtin_amdgcn_readfirstlane(pp.slot) : nullptr;
    segment(qt2, 0, tiles2, nullptr, nullptr, pre ? 2 : 0, flag);
    if (pre && tiles2 == 0) {   // no first barrier in the segment: arrive here
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (tid == 0) arrive_old = arrive_swap(flag, a.epoch);
    }
    store_rows<DOWN>(a, o, m_run, l_run, h, doc_lo + qt2 * BM, doc_hi, qb, lane, xs_wave, 32 * DOWN * kh, kh == 0);
  }
  if (pre) {
    if (tid == 0) {
      const bool sec = arrive_old == first_mark;
      if (sec) mark_merged(a.flags + __builtin_amdgcn_readfirstlane(pp.slot), a.epoch);
      second_arrival = sec;
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(second_arrival) != 0) merge_records(__builtin_amdgcn_readfirstlane(pp.slot), qt1);
  }
}

// ---- packed-document schedule: all (document, query tile) tasks, heaviest first
// Single workgroup. Writes tasks[] sorted by descending key-tile count and *count.
constexpr int kSchedThreads = 1024;
constexpr int kSchedBins = 4096;

// Document bounds are clamped to [0, T] with end >= start, so malformed offsets
// yield wrong documents but never an out-of-range access; at most max_tasks
// tasks are written.
__global__ __launch_bounds__(kSchedThreads) void attn_schedule_kernel(const int32_t *__restrict__ cu,
                                                                      const int32_t *__restrict__ cu_k, int n_seq,
                                                                      int T, int T_k, int causal, int max_tasks,
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
  auto klen_of = [&](int d) {
    const int klo = min(max(cu_k[d], 0), T_k);
    return min(max(cu_k[d + 1], klo), T_k) - klo;
  };
  auto tiles_of = [&](int d) { return (hi_of(d) - lo_of(d) + BM - 1) / BM; };
  // key tiles of query tile t of document d (causal: the document's last
  // query lines up with its last key)
  auto work_of = [&](int d, int t) {
    const int lo = lo_of(d), hi = hi_of(d), nk = klen_of(d);
    const int kv = causal ? min(max(min(lo + (t + 1) * BM, hi) - lo + (nk - (hi - lo)), 0), nk) : nk;
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
  // descending-bin exclusive offsets: thread i scans bins [kSchedBins-1 - PER*i, -PER) of the
  // descending order, the per-thread sums meet in a block-wide scan
  {
    constexpr int PER = kSchedBins / kSchedThreads;
    static_assert(PER * kSchedThreads == kSchedBins, "bins per thread");
    int local[PER];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      local[k] = hist[kSchedBins - 1 - (PER * tid + k)];
      sum += local[k];
    }
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kSchedThreads; off <<= 1) {
      const int add = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    int acc = part[tid] - sum;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      hist[kSchedBins - 1 - (PER * tid + k)] = acc;
      acc += local[k];
    }
    if (tid == 0) *count = min(total, max_tasks);
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
  int64_t lo = 0, hi = p.T, klo = 0, khi = p.T_k;
  if (p.cu != nullptr) {
    int d = 0;
    while (d + 1 < p.n_seq && p.cu[d + 1] <= t) ++d;
    lo = min(max<int64_t>(p.cu[d], 0), p.T);
    hi = min(max<int64_t>(p.cu[d + 1], lo), p.T);
    klo = min(max<int64_t>(p.cu_k[d], 0), p.T_k);
    khi = min(max<int64_t>(p.cu_k[d + 1], klo), p.T_k);
  }
  // causal: the document's last query lines up with its last key
  const int64_t kend = p.causal ? min(max(t + 1 + (khi - hi), klo), khi) : khi;
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
  for (int64_t j = klo; j < kend; ++j) m = fmaxf(m, score(j));
  float l = 0.f;
  for (int64_t j = klo; j < kend; ++j) l += expf(score(j) - m);
  T *op = out + (p.o_chunk ? (t / p.o_chunk) * p.o_sc + (t % p.o_chunk) * p.o_st : t * p.o_st) + h * p.o_sh;
  constexpr int CH = 16;
  for (int v0 = 0; v0 < p.V; v0 += CH) {
    float acc[CH];
    for (int i = 0; i < CH; ++i) acc[i] = 0.f;
    for (int64_t j = klo; j < kend; ++j) {
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
// packed documents: task count | task list | first task of each document
WsLayout ws_layout(int64_t T, int n_seq) {
  WsLayout w;
  const size_t max_tasks = static_cast<size_t>((T + BM - 1) / BM + n_seq);
  w.count_off = 0;
  w.tasks_off = 256;
  w.first_off = w.tasks_off + ((max_tasks * sizeof(int2) + 255) / 256) * 256;
  w.bytes = w.first_off + ((static_cast<size_t>(n_seq) * sizeof(int) + 255) / 256) * 256;
  return w;
}

// Dense causal pairing: two softmax-state records and one arrival flag per
// (head, pair); the flags follow the records.
size_t pair_records_bytes(int64_t T, int H) {
  const int64_t n = (T + BM - 1) / BM;
  return static_cast<size_t>(H) * static_cast<size_t>(n / 2) * 2 * kRecFloats * sizeof(float);
}
size_t pair_ws_bytes(int64_t T, int H) {
  const int64_t n = (T + BM - 1) / BM;
  return pair_records_bytes(T, H) + static_cast<size_t>(H) * static_cast<size_t>(n / 2) * sizeof(unsigned long long);
}

// Fixed device scratch for mla_attention_fwd_noalloc: the workspace of a call
// that may not allocate (split-tile records and flags, or the document
// schedule). Each GPU the library runs on holds its own copy for the life of
// the process. In host code `scratch` names a host-side stand-in, never the
// device memory: its device address is looked up once per device below and
// only that address reaches a kernel.
static __device__ __align__(256) unsigned char scratch[kAttnScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

int attn_scratch(void *stream, void **ptr) {
  *ptr = nullptr;
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {   // the stream's device (the null stream is the current device's)
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // with that device current: every device holds its own copy at its own address
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

bool attn_fast_path(int N, int R, int V, int bf16) { return bf16 && N == 128 && R == 64 && V == 128; }

size_t attn_workspace_bytes(int64_t T, int H, int n_seq, int has_cu, int causal, int N, int R, int V, int bf16) {
  if (!attn_fast_path(N, R, V, bf16) || T == 0) return 0;
  if (has_cu) return ws_layout(T, n_seq).bytes;
  if (causal) return pair_ws_bytes(T, H);
  return 0;
}

int launch_attention(const AttnPlan &p, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.T == 0) return hipSuccess;
  if (!attn_fast_path(p.N, p.R, p.V, p.bf16)) {
    const int64_t blocks = (p.T * p.H + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (p.bf16)
      hipLaunchKernelGGL(attn_generic_kernel<uint16_t>, grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(attn_generic_kernel<float>, grid, dim3(256), 0, s, p);
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
  a.o_sc = p.o_sc;
  a.o_chunk = static_cast<int>(p.o_chunk);   // < T <= 2^31 - 1
  a.T = static_cast<int>(p.T);
  a.T_k = static_cast<int>(p.T_k);
  a.H = p.H;
  a.scale_log2 = p.scale * kLog2e;
  a.causal = p.causal;
  a.cu = p.cu;
  a.cu_k = p.cu_k;
  int64_t tasks;
  if (p.cu == nullptr) {
    a.tasks = nullptr;
    a.task_count = nullptr;
    a.n_qtiles = static_cast<int>((p.T + BM - 1) / BM);
    a.order = p.causal ? 1 : 0;   // dense causal: tile pairing (see pair_plan)
    a.part = nullptr;
    a.flags = nullptr;
    a.epoch = 0;
    if (a.order == 1) {
      a.part = static_cast<float *>(p.ws);
      a.flags = reinterpret_cast<unsigned long long *>(static_cast<char *>(p.ws) + pair_records_bytes(p.T, p.H));
      a.epoch = next_call_tag() & ((1ull << 62) - 1);
    }
    tasks = a.n_qtiles;
  } else {
    const WsLayout w = ws_layout(p.T, p.n_seq);
    char *ws = static_cast<char *>(p.ws);
    int *count = reinterpret_cast<int *>(ws + w.count_off);
    int2 *task_arr = reinterpret_cast<int2 *>(ws + w.tasks_off);
    int *first = reinterpret_cast<int *>(ws + w.first_off);
    const int max_tasks = static_cast<int>((p.T + BM - 1) / BM + p.n_seq);
    hipLaunchKernelGGL(attn_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, s, p.cu, p.cu_k, p.n_seq,
                       static_cast<int>(p.T), static_cast<int>(p.T_k), p.causal, max_tasks, task_arr, count, first);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.tasks = task_arr;
    a.task_count = count;
    a.n_qtiles = 0;
    a.order = 0;
    a.part = nullptr;
    a.flags = nullptr;
    a.epoch = 0;
    tasks = (p.T + BM - 1) / BM + p.n_seq;
  }
  const int64_t blocks = tasks * p.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_kernel<128, 64, 128>), dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
