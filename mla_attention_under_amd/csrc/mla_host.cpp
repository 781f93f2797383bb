// Host front end of libmla.so: argument validation, error reporting and
// dispatch to the HIP launchers. Every check runs before anything is launched,
// so a bad call changes no output (the one-GPU analogue of validating on every
// rank before the first collective, DeepSpeed PR #8316 review thread).
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <algorithm>
#include <string>
#include <utility>
#include <vector>

#include "../../include/mla.h"
#include "mla_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return MLA_OK;
}

int launched(int hip_err, const char *what) {
  if (hip_err != 0) return fail(MLA_ELAUNCH, "%s: HIP launch failed: %s", what, mla::hip_error_name(hip_err));
  return ok();
}

bool valid_dtype(int dt) { return dt == MLA_BF16 || dt == MLA_F32; }
int64_t elem_bytes(int dt) { return dt == MLA_BF16 ? 2 : 4; }

// head offsets from a host shard list; checks every entry
int shard_offsets(const int *sizes, int sp, int heads_total, int *off, const char *who) {
  if (sizes == nullptr) return fail(MLA_EINVAL, "%s: sizes is NULL", who);
  if (sp < 1 || sp > mla::kMaxRanks) return fail(MLA_EINVAL, "%s: sp=%d outside [1, %d]", who, sp, mla::kMaxRanks);
  int64_t acc = 0;
  for (int r = 0; r < sp; ++r) {
    if (sizes[r] < 1) return fail(MLA_EINVAL, "%s: sizes[%d]=%d must be positive", who, r, sizes[r]);
    off[r] = static_cast<int>(acc);
    acc += sizes[r];
  }
  if (acc != heads_total)
    return fail(MLA_EINVAL, "%s: shard sizes sum to %lld, heads_total is %d", who, static_cast<long long>(acc),
                heads_total);
  off[sp] = heads_total;
  return MLA_OK;
}

int pack_common(const void *src, void *dst, int64_t tokens, int heads_total, int feat, const int *sizes, int sp,
                int dtype, void *stream, int to_slabs, const char *who) {
  if (!valid_dtype(dtype)) return fail(MLA_EINVAL, "%s: unknown dtype %d", who, dtype);
  if (tokens < 0 || heads_total < 1 || feat < 1)
    return fail(MLA_EINVAL, "%s: need tokens >= 0, heads_total >= 1, feat >= 1 (got %lld, %d, %d)", who,
                static_cast<long long>(tokens), heads_total, feat);
  mla::PackPlan p;
  const int rc = shard_offsets(sizes, sp, heads_total, p.off, who);
  if (rc != MLA_OK) return rc;
  if (tokens == 0) return ok();
  if (src == nullptr || dst == nullptr) return fail(MLA_EINVAL, "%s: NULL buffer", who);
  const int64_t eb = elem_bytes(dtype);
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  const uint64_t bytes = static_cast<uint64_t>(tokens) * heads_total * feat * eb;
  if (a % eb || b % eb) return fail(MLA_EINVAL, "%s: buffers must be aligned to the element size", who);
  if (a < b + bytes && b < a + bytes) return fail(MLA_EINVAL, "%s: source and destination overlap", who);
  p.src = src;
  p.dst = dst;
  p.tokens = tokens;
  p.heads_total = heads_total;
  p.row_bytes = feat * eb;
  p.sp = sp;
  p.to_slabs = to_slabs;
  return launched(mla::launch_pack(p, stream), who);
}

}  // namespace

namespace mla {
unsigned long long next_call_tag() {
  static std::atomic<unsigned long long> counter{[] {
    std::random_device rd;
    return (static_cast<unsigned long long>(rd()) << 32) ^ rd() ^
           static_cast<unsigned long long>(std::chrono::steady_clock::now().time_since_epoch().count());
  }()};
  return counter.fetch_add(1, std::memory_order_relaxed);
}

}  // namespace mla

extern "C" {

const char *mla_last_error(void) { return g_err.c_str(); }

const char *mla_version(void) { return "mla 0.1 gfx950"; }

int mla_head_shard_sizes(int q_heads, int kv_heads, int sp, int *sizes_out) {
  const char *who = "mla_head_shard_sizes";
  if (sizes_out == nullptr) return fail(MLA_EINVAL, "%s: sizes_out is NULL", who);
  if (sp < 1 || q_heads < 1 || kv_heads < 1)
    return fail(MLA_EINVAL, "%s: q_heads, kv_heads and sp must be positive (got %d, %d, %d)", who, q_heads,
                kv_heads, sp);
  if (q_heads % kv_heads != 0)
    return fail(MLA_EINVAL, "%s: q_heads (%d) is not a multiple of kv_heads (%d)", who, q_heads, kv_heads);
  if (kv_heads < sp)
    return fail(MLA_EINVAL, "%s: kv_heads (%d) < sp (%d): some rank would own no KV head", who, kv_heads, sp);
  const int group = q_heads / kv_heads;
  const int base = kv_heads / sp, extra = kv_heads % sp;
  for (int r = 0; r < sp; ++r) sizes_out[r] = (base + (r < extra ? 1 : 0)) * group;
  return ok();
}

int mla_pack_heads(const void *x, void *send, int64_t tokens, int heads_total, int feat, const int *sizes, int sp,
                   int dtype, void *stream) {
  return pack_common(x, send, tokens, heads_total, feat, sizes, sp, dtype, stream, 1, "mla_pack_heads");
}

int mla_unpack_heads(const void *recv, void *x, int64_t tokens, int heads_total, int feat, const int *sizes,
                     int sp, int dtype, void *stream) {
  return pack_common(recv, x, tokens, heads_total, feat, sizes, sp, dtype, stream, 0, "mla_unpack_heads");
}

int mla_pack_expanded(const void *q, const void *kv, const void *k_rope, void *send, int64_t tokens, int heads_total,
                      int N, int R, int V, const int *sizes, int sp, int dtype, void *stream) {
  const char *who = "mla_pack_expanded";
  if (!valid_dtype(dtype)) return fail(MLA_EINVAL, "%s: unknown dtype %d", who, dtype);
  if (tokens < 0 || heads_total < 1 || N < 1 || R < 1 || V < 1)
    return fail(MLA_EINVAL, "%s: need tokens >= 0, heads_total, N, R, V >= 1 (got %lld, %d, %d, %d, %d)", who,
                static_cast<long long>(tokens), heads_total, N, R, V);
  mla::PackExpandedPlan p;
  const int rc = shard_offsets(sizes, sp, heads_total, p.off, who);
  if (rc != MLA_OK) return rc;
  if (tokens == 0) return ok();
  if (q == nullptr || kv == nullptr || k_rope == nullptr || send == nullptr)
    return fail(MLA_EINVAL, "%s: NULL buffer", who);
  const int64_t eb = elem_bytes(dtype);
  const uint64_t th = static_cast<uint64_t>(tokens) * heads_total;
  const uint64_t q_bytes = th * (N + R) * eb, kv_bytes = th * (N + V) * eb;
  const uint64_t kr_bytes = static_cast<uint64_t>(tokens) * R * eb, out_bytes = th * (2 * (N + R) + V) * eb;
  const uintptr_t pq = reinterpret_cast<uintptr_t>(q), pkv = reinterpret_cast<uintptr_t>(kv),
                  pkr = reinterpret_cast<uintptr_t>(k_rope), po = reinterpret_cast<uintptr_t>(send);
  if ((pq | pkv | pkr | po) % eb) return fail(MLA_EINVAL, "%s: buffers must be aligned to the element size", who);
  auto overlaps = [&](uintptr_t a, uint64_t na) { return a < po + out_bytes && po < a + na; };
  if (overlaps(pq, q_bytes) || overlaps(pkv, kv_bytes) || overlaps(pkr, kr_bytes))
    return fail(MLA_EINVAL, "%s: send overlaps a source", who);
  p.q = q;
  p.kv = kv;
  p.kr = k_rope;
  p.dst = send;
  p.tokens = tokens;
  p.heads_total = heads_total;
  p.n_bytes = N * eb;
  p.r_bytes = R * eb;
  p.v_bytes = V * eb;
  p.sp = sp;
  return launched(mla::launch_pack_expanded(p, stream), who);
}

int mla_apply_rope(void *x, int64_t tokens, int heads, int64_t stride_t, int64_t stride_h, int R, const void *cos,
                   const void *sin, int64_t cs_stride, int interleaved, int dtype, void *stream) {
  const char *who = "mla_apply_rope";
  if (!valid_dtype(dtype)) return fail(MLA_EINVAL, "%s: unknown dtype %d", who, dtype);
  if (tokens < 0 || heads < 1 || R < 2 || R > 256 || R % 2 || (interleaved != 0 && interleaved != 1))
    return fail(MLA_EINVAL, "%s: need tokens >= 0, heads >= 1, even 2 <= R <= 256, interleaved 0/1 (got %lld, %d, %d, %d)",
                who, static_cast<long long>(tokens), heads, R, interleaved);
  if (tokens == 0) return ok();
  if (x == nullptr || cos == nullptr || sin == nullptr) return fail(MLA_EINVAL, "%s: NULL buffer", who);
  if ((heads > 1 && stride_h < R) || (tokens > 1 && stride_t < (heads - 1) * stride_h + R) ||
      (tokens > 1 && cs_stride < R) || stride_h < 0 || stride_t < 0 || cs_stride < 0)
    return fail(MLA_EINVAL, "%s: strides let band rows overlap (stride_t %lld, stride_h %lld, cs_stride %lld)", who,
                static_cast<long long>(stride_t), static_cast<long long>(stride_h), static_cast<long long>(cs_stride));
  const int64_t eb = elem_bytes(dtype);
  const uintptr_t px = reinterpret_cast<uintptr_t>(x), pc = reinterpret_cast<uintptr_t>(cos),
                  ps = reinterpret_cast<uintptr_t>(sin);
  if ((px | pc | ps) % eb) return fail(MLA_EINVAL, "%s: buffers must be aligned to the element size", who);
  const uint64_t xb = static_cast<uint64_t>((tokens - 1) * stride_t + (heads - 1) * stride_h + R) * eb;
  const uint64_t tb = static_cast<uint64_t>((tokens - 1) * cs_stride + R) * eb;
  if ((px < pc + tb && pc < px + xb) || (px < ps + tb && ps < px + xb))
    return fail(MLA_EINVAL, "%s: the band overlaps a table", who);
  mla::RopePlan p;
  p.x = x;
  p.cos = cos;
  p.sin = sin;
  p.tokens = tokens;
  p.stride_t = stride_t;
  p.stride_h = stride_h;
  p.cs_stride = cs_stride;
  p.heads = heads;
  p.R = R;
  p.interleaved = interleaved;
  p.bf16 = dtype == MLA_BF16;
  return launched(mla::launch_rope(p, stream), who);
}

int mla_project_pack(const void *latent, const void *w, void *send, int64_t tokens, int L, int w_heads, int head_begin,
                     int heads, int P, int F, int col_offset, const int *sizes, int sp, int rope_offset, int R,
                     const void *cos, const void *sin, int64_t cs_stride, int interleaved, int dtype, void *stream) {
  const char *who = "mla_project_pack";
  if (!valid_dtype(dtype)) return fail(MLA_EINVAL, "%s: unknown dtype %d", who, dtype);
  if (tokens < 0 || L < 1 || w_heads < 1 || heads < 1 || P < 1 || F < 1 || head_begin < 0 ||
      head_begin + heads > w_heads || col_offset < 0 || col_offset + P > F || R < 0 || (interleaved != 0 && interleaved != 1))
    return fail(MLA_EINVAL, "%s: inconsistent sizes (tokens %lld, L %d, heads [%d, %d) of %d, P %d, F %d, col_offset %d, R %d)",
                who, static_cast<long long>(tokens), L, head_begin, head_begin + heads, w_heads, P, F, col_offset, R);
  if (R > 0 && (rope_offset < 0 || rope_offset + R > P || R % 2))
    return fail(MLA_EINVAL, "%s: the RoPE band [%d, %d) must be an even-width part of the %d-column block", who, rope_offset,
                rope_offset + R, P);
  if (heads > mla::kMaxSlabHeads) return fail(MLA_EUNSUPPORTED, "%s: more than %d heads", who, mla::kMaxSlabHeads);
  mla::ProjectPackPlan p;
  int offs[mla::kMaxRanks + 1];
  const int rc = shard_offsets(sizes, sp, heads, offs, who);
  if (rc != MLA_OK) return rc;
  if (dtype != MLA_BF16) return fail(MLA_EUNSUPPORTED, "%s: bf16 only", who);
  if (L % 8 || P % 8 || F % 8 || col_offset % 8)
    return fail(MLA_EUNSUPPORTED, "%s: L, P, F and col_offset must be multiples of 8", who);
  // the band is rotated on the accumulators of the one wave that holds its 64 columns
  if (R > 0 && (R != 64 || rope_offset % 64 || P % 64))
    return fail(MLA_EUNSUPPORTED, "%s: the RoPE band must be 64 wide at a multiple of 64 in a block whose width "
                "is a multiple of 64 (got R %d at %d of %d)", who, R, rope_offset, P);
  if (tokens == 0) return ok();
  if (latent == nullptr || w == nullptr || send == nullptr || (R > 0 && (cos == nullptr || sin == nullptr)))
    return fail(MLA_EINVAL, "%s: NULL buffer", who);
  const uintptr_t al = reinterpret_cast<uintptr_t>(latent) | reinterpret_cast<uintptr_t>(w) |
                       reinterpret_cast<uintptr_t>(send) |
                       (R > 0 ? reinterpret_cast<uintptr_t>(cos) | reinterpret_cast<uintptr_t>(sin) : 0);
  if (al % 16 || (R > 0 && (cs_stride % 8 || (tokens > 1 && cs_stride < R))))
    return fail(MLA_EUNSUPPORTED, "%s: buffers must be 16-byte aligned, table rows multiples of 8 elements", who);
  if (tokens >= (int64_t(1) << 31)) return fail(MLA_EUNSUPPORTED, "%s: too many tokens", who);
  // the tiles address their rows by 32-bit byte offsets: 128 latent rows and 64 weight rows must fit 4 GiB
  if (int64_t(128) * L * 2 >= (int64_t(1) << 32) || int64_t(64) * w_heads * P * 2 >= (int64_t(1) << 32))
    return fail(MLA_EUNSUPPORTED, "%s: latent width %d or weight width %lld too large for the tiles", who, L,
                static_cast<long long>(int64_t(w_heads) * P));
  if ((tokens + 127) / 128 * ((int64_t(heads) * P + 127) / 128) >= (int64_t(1) << 31))
    return fail(MLA_EUNSUPPORTED, "%s: more than 2^31 output tiles", who);
  const uint64_t sb = static_cast<uint64_t>(tokens) * heads * F * 2;
  const uintptr_t ps = reinterpret_cast<uintptr_t>(send), pl = reinterpret_cast<uintptr_t>(latent),
                  pw = reinterpret_cast<uintptr_t>(w);
  const uint64_t lb = static_cast<uint64_t>(tokens) * L * 2, wb = static_cast<uint64_t>(L) * w_heads * P * 2;
  if ((ps < pl + lb && pl < ps + sb) || (ps < pw + wb && pw < ps + sb))
    return fail(MLA_EINVAL, "%s: send overlaps an input", who);
  for (int r = 0; r < sp; ++r)
    for (int h = offs[r]; h < offs[r + 1]; ++h) {
      p.off[h] = offs[r];
      p.qr[h] = sizes[r];
    }
  p.latent = latent;
  p.w = w;
  p.send = send;
  p.T = tokens;
  p.L = L;
  p.ldw = static_cast<int64_t>(w_heads) * P;
  p.col0 = static_cast<int64_t>(head_begin) * P;
  p.heads = heads;
  p.P = P;
  p.F = F;
  p.col_off = col_offset;
  p.rope_off = rope_offset;
  p.R = R;
  p.interleaved = interleaved;
  p.cos = cos;
  p.sin = sin;
  p.cs_stride = cs_stride;
  return launched(mla::launch_project_pack(p, stream), who);
}

namespace {
// A half-open token interval.
struct Span {
  int64_t lo = 0, hi = 0;
  int64_t size() const { return hi > lo ? hi - lo : 0; }
};
Span meet(Span a, Span b) { return Span{std::max(a.lo, b.lo), std::min(a.hi, b.hi)}; }

// Packed documents given by their cumulative ends (documents tile [0, total)
// back to back, empty ones allowed): checks the ends.
int check_ends(const int64_t *ends, int n, const char *who) {
  if (ends == nullptr || n < 1) return fail(MLA_EINVAL, "%s: need at least one document end", who);
  for (int i = 0; i < n; ++i)
    if (ends[i] < (i ? ends[i - 1] : 0))
      return fail(MLA_EINVAL, "%s: document ends must be non-negative and non-decreasing", who);
  return MLA_OK;
}

// Keys needed by the queries of partition r, i.e. the token range
// Q = [r*len, (r+1)*len): a query sees its own document up to itself, so the
// documents meeting Q contribute the causal prefixes that end at their
// clipped ends, and those prefixes tile one interval: from the start of the
// document holding the first query to the end of Q. Fails when the documents
// end before Q does.
int key_span(const int64_t *ends, int n, int64_t len, int64_t r, Span &keys, const char *who) {
  const Span q{r * len, (r + 1) * len};
  if (ends[n - 1] < q.hi)
    return fail(MLA_EINVAL, "%s: the documents do not cover the queries [%lld, %lld)", who,
                static_cast<long long>(q.lo), static_cast<long long>(q.hi));
  // first document whose end lies past the first query: it holds that query
  const int64_t *first = std::upper_bound(ends, ends + n, q.lo);
  keys = Span{first == ends ? 0 : first[-1], q.hi};
  return MLA_OK;
}
}  // namespace

int mla_causal_partition(const int64_t *doc_ends, int n_docs, int64_t query_length, int query_rank, int batch,
                         int64_t *key_begin, int64_t *key_end, int64_t *query_ends, int64_t *key_ends, int cap,
                         int *n_out) {
  const char *who = "mla_causal_partition";
  if (query_length < 1 || query_rank < 0 || batch < 1)
    return fail(MLA_EINVAL, "%s: need query_length >= 1, query_rank >= 0, batch >= 1", who);
  if (query_rank > INT64_MAX / query_length - 1) return fail(MLA_EINVAL, "%s: query range overflows", who);
  if (key_begin == nullptr || key_end == nullptr || query_ends == nullptr || key_ends == nullptr || n_out == nullptr)
    return fail(MLA_EINVAL, "%s: NULL output", who);
  int rc = check_ends(doc_ends, n_docs, who);
  if (rc != MLA_OK) return rc;
  Span keys;
  rc = key_span(doc_ends, n_docs, query_length, query_rank, keys, who);
  if (rc != MLA_OK) return rc;
  const Span q{query_rank * query_length, (query_rank + 1) * query_length};
  // Each document meeting Q ends its share at c = min(its end, Q's end); since
  // the documents are contiguous, the cumulative query count up to it is c -
  // Q.lo and the cumulative key count c - keys.lo.
  std::vector<int64_t> cut;
  for (int i = 0; i < n_docs; ++i) {
    const Span d{i ? doc_ends[i - 1] : 0, doc_ends[i]};
    if (meet(d, q).size() > 0) cut.push_back(std::min(d.hi, q.hi));
  }
  const int64_t m = static_cast<int64_t>(cut.size());
  if (m * batch > cap)
    return fail(MLA_EINVAL, "%s: %lld output entries needed, capacity %d", who, static_cast<long long>(m * batch),
                cap);
  const int64_t nq = q.size(), nk = keys.size();   // per-sequence totals, the batch strides
  for (int b = 0; b < batch; ++b)
    for (int64_t j = 0; j < m; ++j) {
      query_ends[b * m + j] = b * nq + (cut[j] - q.lo);
      key_ends[b * m + j] = b * nk + (cut[j] - keys.lo);
    }
  *key_begin = keys.lo;
  *key_end = keys.hi;
  *n_out = static_cast<int>(m * batch);
  return ok();
}

int mla_kv_exchange_ranges(const int64_t *doc_ends, int n_docs, int64_t source_length, int64_t query_length,
                           int head_copies, int degree, int rank, int64_t *send_offset, int64_t *send_count,
                           int64_t *recv_count, int *local_only) {
  const char *who = "mla_kv_exchange_ranges";
  if (source_length < 0 || query_length < 1 || head_copies < 1 || degree < 1 || rank < 0 || rank >= degree)
    return fail(MLA_EINVAL, "%s: need source_length >= 0, query_length >= 1, head_copies >= 1, 0 <= rank < degree",
                who);
  if (source_length > 0 && degree > INT64_MAX / source_length) return fail(MLA_EINVAL, "%s: ranges overflow", who);
  if (send_offset == nullptr || send_count == nullptr || recv_count == nullptr || local_only == nullptr)
    return fail(MLA_EINVAL, "%s: NULL output", who);
  int rc = check_ends(doc_ends, n_docs, who);
  if (rc != MLA_OK) return rc;
  // every rank's source tokens and the keys its queries need
  std::vector<Span> src(degree), need(degree);
  for (int p = 0; p < degree; ++p) {
    src[p] = Span{p * source_length, (p + 1) * source_length};
    rc = key_span(doc_ends, n_docs, query_length, p / head_copies, need[p], who);
    if (rc != MLA_OK) return rc;
  }
  // what moves from a to b is a's source inside b's need; nothing moves at all
  // when every rank's need lies inside its own source
  bool local = true;
  for (int p = 0; p < degree; ++p) {
    const Span out = meet(src[rank], need[p]);
    send_count[p] = out.size();
    send_offset[p] = out.size() ? out.lo - src[rank].lo : 0;
    recv_count[p] = meet(src[p], need[rank]).size();
    local = local && meet(src[p], need[p]).size() == need[p].size();
  }
  *local_only = local ? 1 : 0;
  return ok();
}

int mla_latent_up_proj(const void *latent, const void *w_kvb, void *kv_out, int64_t T, int L, int heads_total,
                       int head_begin, int heads, int N, int V, int dtype, void *stream) {
  const char *who = "mla_latent_up_proj";
  if (!valid_dtype(dtype)) return fail(MLA_EINVAL, "%s: unknown dtype %d", who, dtype);
  if (T < 0 || L < 1 || N < 1 || V < 1 || heads < 1 || heads_total < 1)
    return fail(MLA_EINVAL, "%s: need T >= 0 and L, N, V, heads, heads_total >= 1", who);
  if (head_begin < 0 || head_begin + heads > heads_total)
    return fail(MLA_EINVAL, "%s: head range [%d, %d) outside the %d heads of the weight", who, head_begin,
                head_begin + heads, heads_total);
  if (T == 0) return ok();
  if (latent == nullptr || w_kvb == nullptr || kv_out == nullptr) return fail(MLA_EINVAL, "%s: NULL buffer", who);
  const int64_t P = static_cast<int64_t>(N) + V;
  const int64_t eb = elem_bytes(dtype);
  const uintptr_t al = reinterpret_cast<uintptr_t>(latent) | reinterpret_cast<uintptr_t>(w_kvb) |
                       reinterpret_cast<uintptr_t>(kv_out);
  if (al % eb) return fail(MLA_EINVAL, "%s: buffers must be aligned to the element size", who);
  if (dtype == MLA_BF16 && (L % 8 || P % 8 || (heads_total * P) % 8 || al % 16))
    return fail(MLA_EUNSUPPORTED, "%s: bf16 needs L and N+V multiples of 8 and 16-byte aligned buffers", who);
  mla::UpProjPlan p;
  p.latent = latent;
  p.w = w_kvb;
  p.out = kv_out;
  p.T = T;
  p.L = L;
  p.ldw = heads_total * P;
  p.col0 = head_begin * P;
  p.ncols = heads * P;
  p.bf16 = dtype == MLA_BF16;
  return launched(mla::launch_up_proj(p, stream), who);
}

int mla_latent_up_proj_linear(const void *latent, const void *w_lin, void *kv_out, int64_t T, int L,
                              int heads_total, int head_begin, int heads, int N, int V, int dtype, void *stream) {
  const char *who = "mla_latent_up_proj_linear";
  if (!valid_dtype(dtype)) return fail(MLA_EINVAL, "%s: unknown dtype %d", who, dtype);
  if (T < 0 || L < 1 || N < 1 || V < 1 || heads < 1 || heads_total < 1)
    return fail(MLA_EINVAL, "%s: need T >= 0 and L, N, V, heads, heads_total >= 1", who);
  if (head_begin < 0 || head_begin + heads > heads_total)
    return fail(MLA_EINVAL, "%s: head range [%d, %d) outside the %d heads of the weight", who, head_begin,
                head_begin + heads, heads_total);
  if (T == 0) return ok();
  if (latent == nullptr || w_lin == nullptr || kv_out == nullptr) return fail(MLA_EINVAL, "%s: NULL buffer", who);
  const int64_t P = static_cast<int64_t>(N) + V;
  const int64_t eb = elem_bytes(dtype);
  const uintptr_t al = reinterpret_cast<uintptr_t>(latent) | reinterpret_cast<uintptr_t>(w_lin) |
                       reinterpret_cast<uintptr_t>(kv_out);
  if (al % eb) return fail(MLA_EINVAL, "%s: buffers must be aligned to the element size", who);
  if (dtype == MLA_BF16 && (L % 8 || P % 8 || al % 16))
    return fail(MLA_EUNSUPPORTED, "%s: bf16 needs L and N+V multiples of 8 and 16-byte aligned buffers", who);
  mla::UpProjPlan p;
  p.latent = latent;
  p.w = w_lin;
  p.out = kv_out;
  p.T = T;
  p.L = L;
  p.ldw = L;                 // row stride of the [heads_total*(N+V)][L] weight
  p.col0 = head_begin * P;   // first weight row of the head range
  p.ncols = heads * P;
  p.bf16 = dtype == MLA_BF16;
  p.w_kmajor = true;
  return launched(mla::launch_up_proj(p, stream), who);
}

static int attn_validate(const mla_attn_args *a, const char *who) {
  if (a == nullptr) return fail(MLA_EINVAL, "%s: args is NULL", who);
  if (!valid_dtype(a->dtype)) return fail(MLA_EINVAL, "%s: unknown dtype %d", who, a->dtype);
  if (a->T_q < 0 || a->T_k < 0 || a->H < 1 || a->N < 1 || a->R < 0 || a->V < 1)
    return fail(MLA_EINVAL, "%s: need T_q >= 0, T_k >= 0, H >= 1, N >= 1, R >= 0, V >= 1", who);
  if (a->R % 2) return fail(MLA_EINVAL, "%s: the RoPE band width R=%d must be even", who, a->R);
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return fail(MLA_EINVAL, "%s: scale must be finite and positive", who);
  if (a->T_q > 0x7fffffffLL || a->T_k > 0x7fffffffLL)
    return fail(MLA_EUNSUPPORTED, "%s: T_q or T_k above 2^31-1", who);
  if (a->cu_seqlens != nullptr && a->n_seq < 1)
    return fail(MLA_EINVAL, "%s: cu_seqlens needs n_seq >= 1", who);
  if (a->cu_seqlens_k != nullptr && a->cu_seqlens == nullptr)
    return fail(MLA_EINVAL, "%s: cu_seqlens_k needs the queries' cu_seqlens", who);
  if (a->cu_seqlens != nullptr && a->cu_seqlens_k == nullptr && a->T_k != a->T_q)
    return fail(MLA_EINVAL, "%s: T_k (%lld) != T_q (%lld) with documents needs cu_seqlens_k", who,
                static_cast<long long>(a->T_k), static_cast<long long>(a->T_q));
  const int64_t K = static_cast<int64_t>(a->N) + a->R;
  if (a->q_stride_h < K || a->q_stride_t < a->H * a->q_stride_h - (a->q_stride_h - K))
    return fail(MLA_EINVAL, "%s: q strides (%lld, %lld) overlap rows of width %lld", who,
                static_cast<long long>(a->q_stride_t), static_cast<long long>(a->q_stride_h),
                static_cast<long long>(K));
  const int64_t P = static_cast<int64_t>(a->N) + a->V;
  if (a->kv_stride_h < P || a->kv_stride_t < a->kv_stride_h * (a->H - 1) + P)
    return fail(MLA_EINVAL, "%s: kv strides overlap rows of width N+V=%lld", who, static_cast<long long>(P));
  if (a->kr_stride_t < a->R) return fail(MLA_EINVAL, "%s: k_rope stride below R", who);
  const int64_t o_head_span = a->o_stride_h * (a->H - 1) + a->V;   // one token's rows of all heads
  if (a->o_chunk_tokens < 0) return fail(MLA_EINVAL, "%s: o_chunk_tokens is negative", who);
  if (a->o_chunk_tokens == 0 || a->o_chunk_tokens >= a->T_q) {
    if (a->o_stride_h < a->V || a->o_stride_t < o_head_span)
      return fail(MLA_EINVAL, "%s: out strides overlap rows of width V", who);
  } else {
    // chunks one after another, or side by side within a token row
    const int64_t C = a->o_chunk_tokens, chunks = (a->T_q + C - 1) / C;
    const bool stacked = a->o_stride_t >= o_head_span && a->o_stride_chunk >= C * a->o_stride_t;
    const bool side = a->o_stride_chunk >= o_head_span && a->o_stride_t >= (chunks - 1) * a->o_stride_chunk + o_head_span;
    if (a->o_stride_h < a->V || !(stacked || side))
      return fail(MLA_EINVAL, "%s: out chunk strides (%lld per chunk, %lld per token) overlap rows", who,
                  static_cast<long long>(a->o_stride_chunk), static_cast<long long>(a->o_stride_t));
  }
  if (a->T_q == 0) return MLA_OK;
  if (!a->q || !a->out || (a->T_k > 0 && (!a->kv || (a->R > 0 && !a->k_rope))))
    return fail(MLA_EINVAL, "%s: NULL buffer", who);
  if (mla::attn_fast_path(a->N, a->R, a->V, a->dtype == MLA_BF16)) {
    const uintptr_t al = reinterpret_cast<uintptr_t>(a->q) | reinterpret_cast<uintptr_t>(a->kv) |
                         reinterpret_cast<uintptr_t>(a->k_rope) | reinterpret_cast<uintptr_t>(a->out);
    const int64_t st = a->q_stride_t | a->q_stride_h | a->kv_stride_t | a->kv_stride_h | a->kr_stride_t |
                       a->o_stride_t | a->o_stride_h | a->o_stride_chunk;
    if (al % 16 || st % 8)
      return fail(MLA_EUNSUPPORTED, "%s: bf16 tiles need 16-byte aligned buffers and strides multiple of 8", who);
    // a tile's rows are addressed by 32-bit byte offsets from its first row
    constexpr int64_t kMaxRowStride = int64_t(1) << 24;
    if (a->q_stride_t > kMaxRowStride || a->kv_stride_t > kMaxRowStride || a->kr_stride_t > kMaxRowStride)
      return fail(MLA_EUNSUPPORTED, "%s: token strides above 2^24 elements are not supported by the bf16 tiles",
                  who);
    const size_t need = mla::attn_workspace_bytes(a->T_q, a->H, a->n_seq, a->cu_seqlens != nullptr, a->causal != 0,
                                                  a->N, a->R, a->V, 1);
    if (need > 0 && (a->workspace == nullptr || a->workspace_bytes < need ||
                     reinterpret_cast<uintptr_t>(a->workspace) % 256))
      return fail(MLA_EINVAL, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", who, need,
                  a->workspace_bytes);
  }
  return MLA_OK;
}

size_t mla_attention_workspace_size(const mla_attn_args *a) {
  if (a == nullptr) return 0;
  if (a->T_q < 0 || a->H < 1) return 0;
  return mla::attn_workspace_bytes(a->T_q, a->H, a->n_seq, a->cu_seqlens != nullptr, a->causal != 0, a->N, a->R,
                                   a->V, a->dtype == MLA_BF16);
}

static int attention_fwd(const mla_attn_args *a, void *stream, const char *who) {
  const int rc = attn_validate(a, who);
  if (rc != MLA_OK) return rc;
  if (a->T_q == 0) return ok();
  mla::AttnPlan p;
  p.q = a->q;
  p.q_st = a->q_stride_t;
  p.q_sh = a->q_stride_h;
  p.kv = a->kv;
  p.kv_st = a->kv_stride_t;
  p.kv_sh = a->kv_stride_h;
  p.kr = a->k_rope;
  p.kr_st = a->kr_stride_t;
  p.out = a->out;
  p.o_st = a->o_stride_t;
  p.o_sh = a->o_stride_h;
  p.o_chunk = a->o_chunk_tokens < a->T_q ? a->o_chunk_tokens : 0;
  p.o_sc = p.o_chunk ? a->o_stride_chunk : 0;
  p.lse = a->lse;
  p.cu = a->cu_seqlens;
  // keys' offsets: their own, else the queries' (then T_k == T_q, checked above)
  p.cu_k = a->cu_seqlens_k != nullptr ? a->cu_seqlens_k : a->cu_seqlens;
  p.n_seq = a->cu_seqlens ? a->n_seq : 1;
  p.T = a->T_q;
  p.T_k = a->T_k;
  p.H = a->H;
  p.N = a->N;
  p.R = a->R;
  p.V = a->V;
  p.scale = a->scale;
  p.causal = a->causal ? 1 : 0;
  p.bf16 = a->dtype == MLA_BF16;
  p.ws = a->workspace;
  p.ws_bytes = a->workspace_bytes;
  return launched(mla::launch_attention(p, stream), who);
}

int mla_attention_fwd(const mla_attn_args *a, void *stream) { return attention_fwd(a, stream, "mla_attention_fwd"); }

int mla_attention_fwd_noalloc(const mla_attn_args *a, void *stream) {
  const char *who = "mla_attention_fwd_noalloc";
  static_assert(MLA_NOALLOC_SCRATCH_BYTES == mla::kAttnScratchBytes, "header and library agree on the scratch size");
  if (a == nullptr) return fail(MLA_EINVAL, "%s: args is NULL", who);
  mla_attn_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  const size_t need = mla_attention_workspace_size(a);
  if (need > mla::kAttnScratchBytes)
    return fail(MLA_EUNSUPPORTED, "%s: this call needs %zu bytes of scratch, more than the %zu bytes the library "
                "holds per GPU (use mla_attention_fwd with a workspace)", who, need, mla::kAttnScratchBytes);
  if (need > 0) {
    void *p = nullptr;
    const int e = mla::attn_scratch(stream, &p);
    if (e != 0) return fail(MLA_ELAUNCH, "%s: device scratch unavailable (%s)", who, mla::hip_error_name(e));
    b.workspace = p;
    b.workspace_bytes = mla::kAttnScratchBytes;
  }
  return attention_fwd(&b, stream, who);
}

static int attn_bwd_validate(const mla_attn_bwd_args *a, const char *who) {
  if (a == nullptr) return fail(MLA_EINVAL, "%s: args is NULL", who);
  if (!valid_dtype(a->dtype)) return fail(MLA_EINVAL, "%s: unknown dtype %d", who, a->dtype);
  if (a->T < 0 || a->H < 1 || a->N < 1 || a->R < 0 || a->V < 1)
    return fail(MLA_EINVAL, "%s: need T >= 0, H >= 1, N >= 1, R >= 0, V >= 1", who);
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return fail(MLA_EINVAL, "%s: scale must be finite and positive", who);
  if (a->cu_seqlens != nullptr && a->n_seq < 1) return fail(MLA_EINVAL, "%s: cu_seqlens needs n_seq >= 1", who);
  const int64_t K = static_cast<int64_t>(a->N) + a->R, P = static_cast<int64_t>(a->N) + a->V;
  if (a->q_stride_h < K || a->q_stride_t < a->q_stride_h * (a->H - 1) + K)
    return fail(MLA_EINVAL, "%s: q strides overlap rows of width N+R", who);
  if (a->kv_stride_h < P || a->kv_stride_t < a->kv_stride_h * (a->H - 1) + P)
    return fail(MLA_EINVAL, "%s: kv strides overlap rows of width N+V", who);
  if (a->kr_stride_t < a->R) return fail(MLA_EINVAL, "%s: k_rope stride below R", who);
  if (a->o_stride_h < a->V || a->o_stride_t < a->o_stride_h * (a->H - 1) + a->V ||
      a->do_stride_h < a->V || a->do_stride_t < a->do_stride_h * (a->H - 1) + a->V)
    return fail(MLA_EINVAL, "%s: out / dout strides overlap rows of width V", who);
  if (a->dtype != MLA_BF16 || !mla::attn_bwd_supported(a->N, a->R, a->V))
    return fail(MLA_EUNSUPPORTED, "%s: runs bf16 with N=128, R=64, V=128 (got dtype %d, N=%d R=%d V=%d)", who,
                a->dtype, a->N, a->R, a->V);
  if (a->T > (1LL << 30)) return fail(MLA_EUNSUPPORTED, "%s: T above 2^30", who);
  if (a->T == 0) return MLA_OK;
  if (!a->q || !a->kv || !a->k_rope || !a->out || !a->dout || !a->lse || !a->dq || !a->dkv || !a->dk_rope)
    return fail(MLA_EINVAL, "%s: NULL buffer", who);
  const uintptr_t al = reinterpret_cast<uintptr_t>(a->q) | reinterpret_cast<uintptr_t>(a->kv) |
                       reinterpret_cast<uintptr_t>(a->k_rope) | reinterpret_cast<uintptr_t>(a->out) |
                       reinterpret_cast<uintptr_t>(a->dout) | reinterpret_cast<uintptr_t>(a->dk_rope);
  const int64_t st = a->q_stride_t | a->q_stride_h | a->kv_stride_t | a->kv_stride_h | a->kr_stride_t |
                     a->o_stride_t | a->o_stride_h | a->do_stride_t | a->do_stride_h;
  if (al % 16 || st % 8)
    return fail(MLA_EUNSUPPORTED, "%s: needs 16-byte aligned inputs and dk_rope, strides multiple of 8", who);
  // a stage's rows are addressed by 32-bit byte offsets from its first row
  constexpr int64_t kMaxRowStride = int64_t(1) << 24;
  if (a->q_stride_t > kMaxRowStride || a->kv_stride_t > kMaxRowStride || a->kr_stride_t > kMaxRowStride ||
      a->do_stride_t > kMaxRowStride)
    return fail(MLA_EUNSUPPORTED, "%s: token strides above 2^24 elements are not supported", who);
  const size_t need = mla::attn_bwd_workspace_bytes(a->T, a->H, a->R);
  if (a->workspace == nullptr || a->workspace_bytes < need || reinterpret_cast<uintptr_t>(a->workspace) % 256)
    return fail(MLA_EINVAL, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", who, need,
                a->workspace_bytes);
  return MLA_OK;
}

size_t mla_attention_bwd_workspace_size(const mla_attn_bwd_args *a) {
  if (a == nullptr || a->T < 0 || a->H < 1 || a->R < 0) return 0;
  return mla::attn_bwd_workspace_bytes(a->T, a->H, a->R);
}

int mla_attention_bwd(const mla_attn_bwd_args *a, void *stream) {
  const char *who = "mla_attention_bwd";
  const int rc = attn_bwd_validate(a, who);
  if (rc != MLA_OK) return rc;
  if (a->T == 0) return ok();
  mla::AttnBwdPlan p;
  p.q = a->q;
  p.kv = a->kv;
  p.kr = a->k_rope;
  p.out = a->out;
  p.dout = a->dout;
  p.q_st = a->q_stride_t;
  p.q_sh = a->q_stride_h;
  p.kv_st = a->kv_stride_t;
  p.kv_sh = a->kv_stride_h;
  p.kr_st = a->kr_stride_t;
  p.o_st = a->o_stride_t;
  p.o_sh = a->o_stride_h;
  p.do_st = a->do_stride_t;
  p.do_sh = a->do_stride_h;
  p.lse = a->lse;
  p.dq = a->dq;
  p.dkv = a->dkv;
  p.dkr = a->dk_rope;
  p.cu = a->cu_seqlens;
  p.n_seq = a->cu_seqlens ? a->n_seq : 1;
  p.T = a->T;
  p.H = a->H;
  p.scale = a->scale;
  p.causal = a->causal ? 1 : 0;
  p.ws = a->workspace;
  return launched(mla::launch_attention_bwd(p, stream), who);
}

size_t mla_latent_up_proj_bwd_workspace_size(int64_t T, int L, int heads, int N, int V) {
  if (T < 0 || L < 1 || heads < 1 || N < 1 || V < 1) return 0;
  const int64_t C = (static_cast<int64_t>(N) + V) * heads;
  if (T > (1LL << 30) || C > (1LL << 30)) return 0;
  return mla::up_bwd_splits(T, L, static_cast<int>(C)).ws_bytes;
}

int mla_latent_up_proj_bwd(const void *latent, const void *w_kvb, const float *dkv, float *d_latent, float *dw,
                           int64_t T, int L, int heads_total, int head_begin, int heads, int N, int V, int dtype,
                           void *workspace, size_t workspace_bytes, void *stream) {
  const char *who = "mla_latent_up_proj_bwd";
  if (T < 0 || L < 1 || N < 1 || V < 1 || heads < 1 || head_begin < 0 || head_begin + heads > heads_total)
    return fail(MLA_EINVAL, "%s: need T >= 0, L, N, V >= 1 and a head range inside the %d heads", who, heads_total);
  if (!valid_dtype(dtype)) return fail(MLA_EINVAL, "%s: unknown dtype %d", who, dtype);
  const int64_t P = static_cast<int64_t>(N) + V, C = P * heads;
  if (dtype != MLA_BF16 || L % 32 || C % 32 || P % 8)
    return fail(MLA_EUNSUPPORTED, "%s: runs bf16 with L and heads*(N+V) multiples of 32, N+V of 8 (L=%d, C=%lld)",
                who, L, static_cast<long long>(C));
  if (T > (1LL << 30) || C > (1LL << 30)) return fail(MLA_EUNSUPPORTED, "%s: T or heads*(N+V) above 2^30", who);
  if (!dw || (T > 0 && (!latent || !w_kvb || !dkv || !d_latent))) return fail(MLA_EINVAL, "%s: NULL buffer", who);
  const uintptr_t al = reinterpret_cast<uintptr_t>(latent) | reinterpret_cast<uintptr_t>(w_kvb) |
                       reinterpret_cast<uintptr_t>(dkv);
  if (al % 16) return fail(MLA_EUNSUPPORTED, "%s: latent, w_kvb and dkv must be 16-byte aligned", who);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(MLA_EINVAL, "%s: the workspace must be 256-byte aligned", who);
  mla::UpProjBwdPlan p;
  p.latent = latent;
  p.w = w_kvb;
  p.dkv = dkv;
  p.d_latent = d_latent;
  p.dw = dw;
  p.T = T;
  p.L = L;
  p.C = static_cast<int>(C);
  p.ldw = P * heads_total;
  p.col0 = P * head_begin;
  p.ws = workspace;
  p.ws_bytes = workspace == nullptr ? 0 : workspace_bytes;
  return launched(mla::launch_up_proj_bwd(p, stream), who);
}

static int decode_validate(const mla_decode_args *a, const char *who) {
  if (a == nullptr) return fail(MLA_EINVAL, "%s: args is NULL", who);
  if (a->dtype != MLA_BF16) return fail(MLA_EUNSUPPORTED, "%s: bf16 only", who);
  if (a->B < 0 || a->S < 1 || a->L < 1 || a->H < 1 || a->N < 1 || a->R < 0 || a->V < 1 || a->num_splits < 1)
    return fail(MLA_EINVAL, "%s: need B >= 0, S >= 1 and positive L, H, N, V, num_splits", who);
  if (a->R % 2) return fail(MLA_EINVAL, "%s: the RoPE band width R=%d must be even", who, a->R);
  if (a->head_begin < 0 || a->head_begin + a->H > a->heads_total)
    return fail(MLA_EINVAL, "%s: head range [%d, %d) outside the %d heads of the weight", who, a->head_begin,
                a->head_begin + a->H, a->heads_total);
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return fail(MLA_EINVAL, "%s: scale must be finite and positive", who);
  if (a->num_splits > a->S) return fail(MLA_EINVAL, "%s: more splits (%d) than cached positions", who, a->num_splits);
  if (a->num_splits > mla::kDecodeMaxSplits)
    return fail(MLA_EUNSUPPORTED, "%s: at most %d splits", who, mla::kDecodeMaxSplits);
  if (a->B > (1 << 20)) return fail(MLA_EUNSUPPORTED, "%s: at most 2^20 sequences per call", who);
  if ((a->S + 64) * static_cast<int64_t>(a->L) * 2 >= (1LL << 32))
    return fail(MLA_EUNSUPPORTED, "%s: a sequence's latent cache must stay below 4 GiB", who);
  if (!mla::decode_supported(a->L, a->N, a->R, a->V) || a->H > 16)
    return fail(MLA_EUNSUPPORTED, "%s: no decode kernel for L=%d N=%d R=%d V=%d H=%d (needs L=512, R=64, H<=16)",
                who, a->L, a->N, a->R, a->V, a->H);
  if (a->B == 0) return MLA_OK;
  if (!a->q || !a->latent_cache || !a->w_kvb || !a->out || (a->R > 0 && !a->rope_cache))
    return fail(MLA_EINVAL, "%s: NULL buffer", who);
  const uintptr_t al = reinterpret_cast<uintptr_t>(a->q) | reinterpret_cast<uintptr_t>(a->latent_cache) |
                       reinterpret_cast<uintptr_t>(a->rope_cache) | reinterpret_cast<uintptr_t>(a->w_kvb) |
                       reinterpret_cast<uintptr_t>(a->out);
  if (al % 16) return fail(MLA_EUNSUPPORTED, "%s: buffers must be 16-byte aligned", who);
  const size_t need = mla::decode_workspace_bytes(a->B, a->H, a->L, a->N, a->R, a->V, a->num_splits);
  if (a->workspace == nullptr || a->workspace_bytes < need || reinterpret_cast<uintptr_t>(a->workspace) % 256)
    return fail(MLA_EINVAL, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", who, need,
                a->workspace_bytes);
  return MLA_OK;
}

size_t mla_latent_decode_workspace_size(const mla_decode_args *a) {
  if (a == nullptr || a->num_splits < 1) return 0;
  return mla::decode_workspace_bytes(a->B, a->H, a->L, a->N, a->R, a->V, a->num_splits);
}

int mla_latent_decode_fwd(const mla_decode_args *a, void *stream) {
  const char *who = "mla_latent_decode_fwd";
  const int rc = decode_validate(a, who);
  if (rc != MLA_OK) return rc;
  if (a->B == 0) return ok();
  mla::DecodePlan p;
  p.q = a->q;
  p.c = a->latent_cache;
  p.kr = a->rope_cache;
  p.w = a->w_kvb;
  p.out = a->out;
  p.lse = a->lse;
  p.B = a->B;
  p.S = a->S;
  p.L = a->L;
  p.H = a->H;
  p.N = a->N;
  p.R = a->R;
  p.V = a->V;
  p.ldw = static_cast<int64_t>(a->heads_total) * (a->N + a->V);
  p.col0 = static_cast<int64_t>(a->head_begin) * (a->N + a->V);
  p.splits = a->num_splits;
  p.scale = a->scale;
  p.ws = a->workspace;
  p.ws_bytes = a->workspace_bytes;
  return launched(mla::launch_decode(p, stream), who);
}

}  // extern "C"
