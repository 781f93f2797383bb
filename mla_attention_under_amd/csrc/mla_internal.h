// Internal interface between the host front end (mla_host.cpp, plain C++) and
// the HIP launchers (*.hip). Pointers are device pointers; `stream` is a
// hipStream_t passed as void*. Launchers return 0 or a hipError_t value.
#pragma once
#include <cstddef>
#include <cstdint>

namespace mla {

constexpr int kMaxRanks = 256;   // largest sequence-parallel degree the pack accepts

// ---- token <-> head pack -------------------------------------------------
struct PackPlan {
  const void *src;
  void *dst;
  int64_t tokens;
  int heads_total;
  int64_t row_bytes;       // feat * element size
  int sp;
  int to_slabs;            // 1: x -> slabs (pack), 0: slabs -> x (unpack)
  int off[kMaxRanks + 1];  // head offset of each rank, off[sp] = heads_total
};
int launch_pack(const PackPlan &p, void *stream);

// ---- expanded pack: per (token, head) row [q | k_nope | k_rope | v] -> head slabs
struct PackExpandedPlan {
  const void *q;        // [tokens][heads_total][N+R]
  const void *kv;       // [tokens][heads_total][N+V]
  const void *kr;       // [tokens][R]
  void *dst;            // concat_r [tokens][sizes[r]][2(N+R)+V]
  int64_t tokens;
  int heads_total;
  int64_t n_bytes, r_bytes, v_bytes;   // N, R, V in bytes
  int sp;
  int off[kMaxRanks + 1];
};
int launch_pack_expanded(const PackExpandedPlan &p, void *stream);

// ---- rotary embedding of a band, in place
struct RopePlan {
  void *x;
  const void *cos, *sin;
  int64_t tokens, stride_t, stride_h, cs_stride;
  int heads, R, interleaved, bf16;
};
int launch_rope(const RopePlan &p, void *stream);

// ---- latent up-projection -------------------------------------------------
struct UpProjPlan {
  const void *latent;  // [T][L]
  const void *w;       // [L][ldw], columns [col0, col0 + ncols); w_kmajor: [rows][ldw], rows [col0, col0 + ncols)
  void *out;           // [T][ncols]
  int64_t T;
  int L;
  int64_t ldw, col0, ncols;
  int bf16;
  bool w_kmajor = false;   // the weight as torch.nn.Linear stores it (k-contiguous)
};
int launch_up_proj(const UpProjPlan &p, void *stream);

// ---- projection written straight into the token->head pack (bf16)
constexpr int kMaxSlabHeads = 256;
struct ProjectPackPlan {
  const void *latent;  // [T][L]
  const void *w;       // [L][ldw], head blocks of P columns from col0
  void *send;          // concat_r [T][sizes[r]][F]; columns [col_off, col_off + P) written
  int64_t T;
  int L;
  int64_t ldw, col0;
  int heads, P, F, col_off;
  int rope_off, R, interleaved;   // R = 0: no rotation
  const void *cos, *sin;
  int64_t cs_stride;
  int off[kMaxSlabHeads], qr[kMaxSlabHeads];   // per projected head: its rank's first head, that rank's head count
};
int launch_project_pack(const ProjectPackPlan &p, void *stream);

// ---- attention ------------------------------------------------------------
struct AttnPlan {
  const void *q;
  int64_t q_st, q_sh;
  const void *kv;
  int64_t kv_st, kv_sh;
  const void *kr;
  int64_t kr_st;
  void *out;
  int64_t o_st, o_sh;
  int64_t o_chunk, o_sc;   // queries per output chunk (0: one chunk) and the chunk stride
  float *lse;
  const int32_t *cu;   // device query offsets (cu_seqlens) or nullptr
  const int32_t *cu_k; // device key offsets or nullptr (then one document of T_k keys)
  int n_seq;
  int64_t T;           // query rows
  int64_t T_k;         // key rows
  int H, N, R, V;
  float scale;
  int causal;
  int bf16;
  void *ws;
  size_t ws_bytes;
};
// true when the MFMA kernel covers these head widths (others use the generic kernel)
bool attn_fast_path(int N, int R, int V, int bf16);
size_t attn_workspace_bytes(int64_t T, int H, int n_seq, int has_cu, int causal, int N, int R, int V, int bf16);
int launch_attention(const AttnPlan &p, void *stream);
// Fixed device scratch for calls that may not allocate (one copy per GPU):
// its size, and its device address on the stream's device (looked up once per
// device). Returns 0 or a hipError_t value.
constexpr size_t kAttnScratchBytes = size_t(48) << 20;
int attn_scratch(void *stream, void **ptr);

// ---- attention backward --------------------------------------------------
struct AttnBwdPlan {
  const void *q, *kv, *kr, *out, *dout;
  int64_t q_st, q_sh, kv_st, kv_sh, kr_st, o_st, o_sh, do_st, do_sh;
  const float *lse;    // [H][T], natural log
  float *dq, *dkv, *dkr;
  const int32_t *cu;
  int n_seq;
  int64_t T;
  int H;
  float scale;
  int causal;
  void *ws;            // attn_bwd_workspace_bytes(T, H, R), 256-byte aligned
};
bool attn_bwd_supported(int N, int R, int V);
size_t attn_bwd_workspace_bytes(int64_t T, int H, int R);
int launch_attention_bwd(const AttnBwdPlan &p, void *stream);

struct UpProjBwdPlan {
  const void *latent;  // bf16 [T][L]
  const void *w;       // bf16 [L][ldw]
  const float *dkv;    // [T][C]
  float *d_latent;     // [T][L]
  float *dw;           // [L][C]
  int64_t T;
  int L, C;
  int64_t ldw, col0;
  void *ws;            // optional: partial products of the split path
  size_t ws_bytes;
};
int launch_up_proj_bwd(const UpProjBwdPlan &p, void *stream);
// split path of the up-projection backward: taken for T, L, C multiples of 128
// when the workspace holds ws_bytes; s_dl / s_dw are the contraction splits
struct UpBwdSplits {
  bool aligned = false;
  int s_dl = 1, s_dw = 1;
  size_t ws_bytes = 0;
};
UpBwdSplits up_bwd_splits(int64_t T, int L, int C);

// ---- latent-cache decode ------------------------------------------------
struct DecodePlan {
  const void *q;       // [B][H][N+R]
  const void *c;       // [B][S][L]
  const void *kr;      // [B][S][R]
  const void *w;       // [L][ldw]
  void *out;           // [B][H][V]
  float *lse;          // [B][H] or nullptr
  int B;
  int64_t S;
  int L, H, N, R, V;
  int64_t ldw, col0;   // head h uses columns col0 + h*(N+V) ...
  int splits;
  float scale;
  void *ws;
  size_t ws_bytes;
};
constexpr int kDecodeMaxSplits = 256;   // KV chunks one decode call may reduce
bool decode_supported(int L, int N, int R, int V);
size_t decode_workspace_bytes(int B, int H, int L, int N, int R, int V, int splits);
int launch_decode(const DecodePlan &p, void *stream);

const char *hip_error_name(int err);

// Per-call tag for the arrival flags that kernels keep in a caller's
// workspace: a process-wide counter that starts at a random 64-bit value, so
// a flag left by another call (or never written) does not match.
unsigned long long next_call_tag();

}  // namespace mla
