// Token <-> head permutation of packed [q | kv] rows (the local send/receive
// side of the Ulysses exchange; torchtitan "MLA CP optimization", section
// "Ulysses CP").
//
// Every (token, rank) pair moves one contiguous run of sizes[r]*row_bytes
// bytes between x[t][off_r .. off_r+sizes[r]) and slab r's row t, so the copy
// is a set of contiguous runs. HBM-bound: each thread moves kUnroll vector
// chunks of the widest size (16, 8, 4 or 2 bytes) that divides the row, all
// loads issued before any store. Workgroups of 1024 threads moving one
// 16-byte chunk each (16 KB) measured best on both the cache-resident rank
// shard and the 940 MB uneven shard (256 threads x 4 chunks: 10-30 % slower
// for the small unpack, 2-4 % for the large copies). Indexing is over the
// slab side, so slab reads/writes are one contiguous stream per rank and the
// x side is a contiguous run per token.
#include <hip/hip_runtime.h>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 1024;
constexpr int kUnroll = 1;

struct PackArgs {
  const unsigned char *src;
  unsigned char *dst;
  uint32_t heads_total;
  uint32_t row_chunks;   // chunks per (token, head) row
  uint64_t tokens;
  int to_slabs;
  int sp;
  int off[kMaxRanks + 1];
};

// Index is uint32_t when every chunk index of the whole buffer fits 32 bits
// (the common case: cheap 32-bit division), else uint64_t.
// Ranks are interleaved in the block order (block b serves rank b % sp), so the
// workgroups in flight at any moment cover whole x rows of a few tokens and
// one stretch of every slab, rather than one rank's column of every x row.
// Streaming (nontemporal) stores for large outputs, ordinary stores (which
// leave the output in the caches) for small ones; the bound depends on the
// direction. Chosen in the attention step, where each copy runs between the
// other kernels: the 29.4 MB rank-shard pack output is faster through the
// caches (10.3 -> 10.0 us) and the 8.4 MB output unpack faster streamed
// (5.1 -> 4.7 us); run back to back, the opposite choices measured faster.
// Copies far beyond the 256 MB Infinity Cache stream either way. Streaming
// loads only for sources beyond kCachedLoadBytes: a source that fits the
// Infinity Cache is read through it (the rank-shard pack: 12.8 -> 10.0 us in
// the step), a larger one streams past it (the 470 MB uneven shard pack is
// 5 % slower with ordinary loads).
constexpr uint64_t kCachedStoreBytesPack = 64ull << 20;
constexpr uint64_t kCachedStoreBytesUnpack = 4ull << 20;
constexpr uint64_t kCachedStoreBytesExpanded = 16ull << 20;   // the expanded pack, measured back to back
constexpr uint64_t kCachedLoadBytes = 64ull << 20;
template <typename Chunk, typename Index, bool kStream, bool kStreamLoad>
__global__ __launch_bounds__(kThreads) void pack_kernel(PackArgs a) {
  const int r = static_cast<int>(blockIdx.x % static_cast<unsigned>(a.sp));
  const Index cb = static_cast<Index>(blockIdx.x / static_cast<unsigned>(a.sp));
  const Index q = static_cast<Index>(a.off[r + 1] - a.off[r]);
  const Index run = q * a.row_chunks;     // chunks per token in slab r
  const Index total = static_cast<Index>(a.tokens) * run;
  const Index slab_base = static_cast<Index>(a.tokens) * static_cast<Index>(a.off[r]) * a.row_chunks;
  const Index x_tok = static_cast<Index>(a.heads_total) * a.row_chunks;
  const Index x_off = static_cast<Index>(a.off[r]) * a.row_chunks;
  const Chunk *src = reinterpret_cast<const Chunk *>(a.src);
  Chunk *dst = reinterpret_cast<Chunk *>(a.dst);

  const Index first = cb * (kThreads * kUnroll) + threadIdx.x;
  Chunk v[kUnroll];
  Index didx[kUnroll];
  bool ok[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const Index c = first + static_cast<Index>(u) * kThreads;
    ok[u] = c < total;
    const Index t = ok[u] ? c / run : 0;
    const Index w = c - t * run;
    const Index xi = t * x_tok + x_off + w;
    const Index si = slab_base + c;
    const Index sidx = a.to_slabs ? xi : si;
    didx[u] = a.to_slabs ? si : xi;
    if (ok[u]) {
      if constexpr (kStreamLoad)
        v[u] = __builtin_nontemporal_load(src + sidx);
      else
        v[u] = src[sidx];
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (ok[u]) {
      if constexpr (kStream)
        __builtin_nontemporal_store(v[u], dst + didx[u]);
      else
        dst[didx[u]] = v[u];
    }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <typename Chunk>
hipError_t run(const PackPlan &p, hipStream_t s) {
  PackArgs a;
  a.src = static_cast<const unsigned char *>(p.src);
  a.dst = static_cast<unsigned char *>(p.dst);
  a.heads_total = static_cast<uint32_t>(p.heads_total);
  a.row_chunks = static_cast<uint32_t>(p.row_bytes / sizeof(Chunk));
  a.tokens = static_cast<uint64_t>(p.tokens);
  a.to_slabs = p.to_slabs;
  a.sp = p.sp;
  int maxq = 0;
  for (int r = 0; r <= p.sp; ++r) a.off[r] = p.off[r];
  for (int r = 0; r < p.sp; ++r) maxq = maxq > (p.off[r + 1] - p.off[r]) ? maxq : (p.off[r + 1] - p.off[r]);
  const uint64_t per_rank = a.tokens * static_cast<uint64_t>(maxq) * a.row_chunks;
  const uint64_t blocks = (per_rank + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  if (blocks == 0) return hipSuccess;
  if (blocks * static_cast<uint64_t>(p.sp) > 0x7fffffffULL) return hipErrorInvalidConfiguration;
  const uint64_t all = a.tokens * static_cast<uint64_t>(p.heads_total) * a.row_chunks;
  const dim3 grid(static_cast<unsigned>(blocks * static_cast<uint64_t>(p.sp)));
  const bool stream = all * sizeof(Chunk) > (p.to_slabs ? kCachedStoreBytesPack : kCachedStoreBytesUnpack);
  const bool stream_load = all * sizeof(Chunk) > kCachedLoadBytes;
  const bool narrow = all + kThreads * kUnroll < 0xffffffffULL;
  if (narrow && stream_load)
    hipLaunchKernelGGL((pack_kernel<Chunk, uint32_t, true, true>), grid, dim3(kThreads), 0, s, a);
  else if (narrow && stream)
    hipLaunchKernelGGL((pack_kernel<Chunk, uint32_t, true, false>), grid, dim3(kThreads), 0, s, a);
  else if (narrow)
    hipLaunchKernelGGL((pack_kernel<Chunk, uint32_t, false, false>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((pack_kernel<Chunk, uint64_t, true, true>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// ---- expanded pack (hyper-parallel `_expanded`): payload row per (token,
// head) [q (K) | k_nope (N) | k_rope (R) | v (V)], K = N + R, the shared RoPE
// key copied into every head. Indexing is over the slab side, one chunk per
// thread; every chunk comes from exactly one source segment (the chunk width
// divides every segment's width). q and kv stream like the plain pack; the
// k_rope row of a token is read once per head and stays in the caches.
struct PackExpArgs {
  const unsigned char *q, *kv, *kr;
  unsigned char *dst;
  uint32_t heads_total;
  uint32_t nc, rc, vc;   // N, R, V in chunks
  uint64_t tokens;
  int sp;
  int off[kMaxRanks + 1];
};

template <typename Chunk, typename Index, bool kStream>
__global__ __launch_bounds__(kThreads) void pack_expanded_kernel(PackExpArgs a) {
  const int r = static_cast<int>(blockIdx.x % static_cast<unsigned>(a.sp));
  const Index cb = static_cast<Index>(blockIdx.x / static_cast<unsigned>(a.sp));
  const Index kc = a.nc + a.rc, pc = a.nc + a.vc, wc = 2 * kc + a.vc;   // chunks per q / kv / payload row
  const Index qr = static_cast<Index>(a.off[r + 1] - a.off[r]);
  const Index per_tok = qr * wc;
  const Index total = static_cast<Index>(a.tokens) * per_tok;
  const Index c = cb * kThreads + threadIdx.x;
  if (c >= total) return;
  const Index t = c / per_tok;
  const Index rem = c - t * per_tok;
  const Index hh = rem / wc;
  const Index f = rem - hh * wc;
  const Index row = t * static_cast<Index>(a.heads_total) + static_cast<Index>(a.off[r]) + hh;
  const Chunk *q = reinterpret_cast<const Chunk *>(a.q);
  const Chunk *kv = reinterpret_cast<const Chunk *>(a.kv);
  const Chunk *kr = reinterpret_cast<const Chunk *>(a.kr);
  Chunk v;
  if (f < kc) {
    v = kStream ? __builtin_nontemporal_load(q + row * kc + f) : q[row * kc + f];
  } else if (f < kc + a.nc) {
    const Index i = row * pc + (f - kc);
    v = kStream ? __builtin_nontemporal_load(kv + i) : kv[i];
  } else if (f < 2 * kc) {
    v = kr[t * a.rc + (f - kc - a.nc)];
  } else {
    const Index i = row * pc + a.nc + (f - 2 * kc);
    v = kStream ? __builtin_nontemporal_load(kv + i) : kv[i];
  }
  Chunk *dst = reinterpret_cast<Chunk *>(a.dst) + static_cast<Index>(a.tokens) * static_cast<Index>(a.off[r]) * wc + c;
  if constexpr (kStream)
    __builtin_nontemporal_store(v, dst);
  else
    *dst = v;
}

template <typename Chunk>
hipError_t run_expanded(const PackExpandedPlan &p, hipStream_t s) {
  PackExpArgs a;
  a.q = static_cast<const unsigned char *>(p.q);
  a.kv = static_cast<const unsigned char *>(p.kv);
  a.kr = static_cast<const unsigned char *>(p.kr);
  a.dst = static_cast<unsigned char *>(p.dst);
  a.heads_total = static_cast<uint32_t>(p.heads_total);
  a.nc = static_cast<uint32_t>(p.n_bytes / sizeof(Chunk));
  a.rc = static_cast<uint32_t>(p.r_bytes / sizeof(Chunk));
  a.vc = static_cast<uint32_t>(p.v_bytes / sizeof(Chunk));
  a.tokens = static_cast<uint64_t>(p.tokens);
  a.sp = p.sp;
  int maxq = 0;
  for (int r = 0; r <= p.sp; ++r) a.off[r] = p.off[r];
  for (int r = 0; r < p.sp; ++r) maxq = maxq > (p.off[r + 1] - p.off[r]) ? maxq : (p.off[r + 1] - p.off[r]);
  const uint64_t wc = 2ull * (a.nc + a.rc) + a.vc;
  const uint64_t per_rank = a.tokens * static_cast<uint64_t>(maxq) * wc;
  const uint64_t blocks = (per_rank + kThreads - 1) / kThreads;
  if (blocks == 0) return hipSuccess;
  if (blocks * static_cast<uint64_t>(p.sp) > 0x7fffffffULL) return hipErrorInvalidConfiguration;
  const uint64_t all = a.tokens * static_cast<uint64_t>(p.heads_total) * wc;   // output chunks
  const bool stream = all * sizeof(Chunk) > kCachedStoreBytesExpanded;
  const bool narrow = all + kThreads < 0xffffffffULL;
  const dim3 grid(static_cast<unsigned>(blocks * static_cast<uint64_t>(p.sp)));
  if (narrow && stream)
    hipLaunchKernelGGL((pack_expanded_kernel<Chunk, uint32_t, true>), grid, dim3(kThreads), 0, s, a);
  else if (narrow)
    hipLaunchKernelGGL((pack_expanded_kernel<Chunk, uint32_t, false>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((pack_expanded_kernel<Chunk, uint64_t, true>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int launch_pack(const PackPlan &p, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uintptr_t align = reinterpret_cast<uintptr_t>(p.src) | reinterpret_cast<uintptr_t>(p.dst);
  auto fits = [&](int64_t g) { return p.row_bytes % g == 0 && align % g == 0; };
  if (fits(16)) return run<u32x4>(p, s);
  if (fits(8)) return run<u32x2>(p, s);
  if (fits(4)) return run<unsigned int>(p, s);
  return run<unsigned short>(p, s);
}

int launch_pack_expanded(const PackExpandedPlan &p, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uintptr_t align = reinterpret_cast<uintptr_t>(p.q) | reinterpret_cast<uintptr_t>(p.kv) |
                          reinterpret_cast<uintptr_t>(p.kr) | reinterpret_cast<uintptr_t>(p.dst);
  auto fits = [&](int64_t g) { return p.n_bytes % g == 0 && p.r_bytes % g == 0 && p.v_bytes % g == 0 && align % g == 0; };
  if (fits(16)) return run_expanded<u32x4>(p, s);
  if (fits(8)) return run_expanded<u32x2>(p, s);
  if (fits(4)) return run_expanded<unsigned int>(p, s);
  return run_expanded<unsigned short>(p, s);
}

const char *hip_error_name(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

}  // namespace mla
