/*
 * mla.h -- C ABI of libmla.so: one Ulysses rank's share of Multi-head Latent
 * Attention (MLA) on an AMD Instinct MI355X (gfx950).
 *
 * Notation (torchtitan PR #5445, "MLA CP optimization" commit message, opening
 * paragraph): T tokens, H heads, L KV latent width, N non-positional key width,
 * R shared (RoPE) key width, V value width; K = N+R, P = N+V, F = K+P.
 *
 * Conventions for every call
 *  - All tensors are dense row-major arrays of the stated element type, passed
 *    as plain device pointers; sizes and strides are in ELEMENTS.
 *  - Element type: MLA_BF16 (bfloat16 storage, fp32 accumulation, outputs
 *    rounded to nearest-even) or MLA_F32 (fp32 throughout).
 *  - `stream` is a hipStream_t cast to void* (NULL = the null stream). Every
 *    call is asynchronous on that stream; the library never synchronises.
 *  - Ownership: the caller owns every buffer, including the workspace. The
 *    library allocates no device memory and keeps no per-model state (no head
 *    count is ever stored between calls).
 *  - Errors: all arguments are validated on the host BEFORE anything is
 *    launched. On failure the call returns a negative mla_status, launches
 *    nothing, writes no output, and mla_last_error() describes the problem.
 *    MLA_ELAUNCH reports a HIP launch error (the message names it).
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_EINVAL = -1,       /* an argument is out of range or inconsistent      */
  MLA_EUNSUPPORTED = -2, /* valid, but not a shape/alignment this build runs */
  MLA_ELAUNCH = -3       /* the HIP runtime rejected a launch               */
} mla_status;

typedef enum { MLA_BF16 = 0, MLA_F32 = 1 } mla_dtype;

/* Thread-local text of the last error on this thread ("" if none). Never NULL. */
const char *mla_last_error(void);

/* Library version string, e.g. "mla 0.1 gfx950". */
const char *mla_version(void);

/*
 * Head shard list (host only, no GPU use).
 * DeepSpeed PR #8316 "[Ulysses] Carry the KV head count per DistributedAttention",
 * sections "What breaks" and "The change": the query heads of a sequence-parallel
 * group follow the KV head count. KV heads are dealt out as evenly as possible,
 * remainder to the lowest ranks, and each KV head takes its whole group of
 * q_heads/kv_heads query heads: rank r gets
 *     sizes_out[r] = (kv_heads / sp + (r < kv_heads % sp)) * (q_heads / kv_heads)
 * heads, contiguous and ascending (rank r owns [sum_{s<r} sizes[s], +sizes[r])).
 * Examples: (12,12,4) -> [3,3,3,3]; (3,3,2) -> [2,1]; (6,3,2) -> [4,2].
 * Rejected with MLA_EINVAL (the same review thread: fail before any exchange):
 * sp < 1, q_heads < 1, kv_heads < 1, q_heads % kv_heads != 0, kv_heads < sp.
 * sizes_out: caller array of sp ints, written only on success.
 */
int mla_head_shard_sizes(int q_heads, int kv_heads, int sp, int *sizes_out);

/*
 * Token->head pack: the local send side of the Ulysses token->head exchange of
 * concat(q_THK, kv_THP) (torchtitan "MLA CP optimization", section "Ulysses CP";
 * hyper-parallel mla_context_parallel.py, `_expanded`).
 *   x    : [tokens][heads_total][feat]
 *   send : concatenation over ranks r of slabs [tokens][sizes[r]][feat]:
 *          send[T*off_r*feat + (t*sizes[r] + h)*feat + f] = x[t][off_r + h][f]
 *          with off_r = sizes[0] + ... + sizes[r-1].
 * sizes: HOST array of sp positive ints summing to heads_total (e.g. from
 * mla_head_shard_sizes). The copy is bit-exact; dtype only fixes the element
 * size (MLA_BF16: 2 bytes, MLA_F32: 4 bytes). x and send must not overlap.
 * tokens == 0 is a valid no-op. sp <= 256.
 */
int mla_pack_heads(const void *x, void *send, int64_t tokens, int heads_total, int feat,
                   const int *sizes, int sp, int dtype, void *stream);

/*
 * Expanded token->head pack: the send side of one sequence-to-head exchange of
 * unequal-width (q, k, v) per head (hyper-parallel mla_context_parallel.py,
 * `_expanded`; the key is assembled as in `_assemble_key_value`, the shared
 * RoPE key copied into every head). Per (token t, head h) the payload row is
 *     [ q[t][h][0:N+R] | kv[t][h][0:N] | k_rope[t][0:R] | kv[t][h][N:N+V] ]
 * of width W = 2(N+R)+V, split into per-rank head slabs as mla_pack_heads does:
 *   q      : [tokens][heads_total][N+R]
 *   kv     : [tokens][heads_total][N+V]   (row [k_nope | v])
 *   k_rope : [tokens][R]                  (one row per token, all heads)
 *   send   : concat_r [tokens][sizes[r]][W]
 * All contiguous. sizes: HOST array of sp positive ints summing to heads_total.
 * Bit-exact copy (dtype fixes the element size only); N, R, V >= 1; send must
 * not overlap any source. tokens == 0 is a valid no-op. sp <= 256.
 */
int mla_pack_expanded(const void *q, const void *kv, const void *k_rope, void *send, int64_t tokens,
                      int heads_total, int N, int R, int V, const int *sizes, int sp, int dtype, void *stream);

/*
 * Rotary embedding of a RoPE band, in place (hyper-parallel mla_context_parallel.py,
 * `apply_mla_rope`; used on q's band of every head and on the shared k_rope).
 *   x   : row (t, h) of the band is the R contiguous elements at
 *         x + t*stride_t + h*stride_h (elements), t < tokens, h < heads;
 *   cos, sin : [tokens][R] tables with row stride cs_stride, in x's element type
 *         (the pages cast the position tables to the tensor's dtype).
 * interleaved == 0 (half-band): with the row [a | b] (halves of R/2),
 *     out = [a*cos[:R/2] - b*sin[:R/2] | b*cos[R/2:] + a*sin[R/2:]].
 * interleaved == 1: the pairs (x[2i], x[2i+1]) are rotated by cos[i], sin[i]
 *     (i < R/2) and stored as real parts then imaginary parts (half-band order).
 * fp32 arithmetic; bf16 results rounded to nearest even. R even, 2 <= R <= 256.
 * Rows must not overlap each other (stride_h >= R when heads > 1, stride_t >=
 * (heads-1)*stride_h + R when tokens > 1) nor the tables. tokens == 0 is a no-op.
 */
int mla_apply_rope(void *x, int64_t tokens, int heads, int64_t stride_t, int64_t stride_h, int R, const void *cos,
                   const void *sin, int64_t cs_stride, int interleaved, int dtype, void *stream);

/*
 * Projection written straight into the token->head pack (torchtitan "MLA CP
 * optimization", section "Ulysses CP": the pack of concat(q_THK, kv_THP) whose
 * parts come from q_b_proj with RoPE and from wkv_b; hyper-parallel `_query`,
 * `apply_mla_rope`). One call writes one part of every payload row:
 *   out[t][h][j] = sum_l latent[t][l] * w[l][(head_begin+h)*P + j],  h < heads, j < P
 * rotated like mla_apply_rope on its columns [rope_offset, rope_offset+R) when
 * R > 0 (cos, sin: [tokens][R] tables, row stride cs_stride), then stored as
 *   send[T*off_r*F + (t*sizes[r] + h-off_r)*F + col_offset + j]
 * for the rank r holding head h (sizes: HOST list of sp positive ints summing
 * to heads). Columns of send outside [col_offset, col_offset+P) are untouched.
 * The band is rotated in fp32 on the projection's accumulators and rounded to
 * bf16 once; the other columns equal mla_latent_up_proj (then mla_pack_heads)
 * bit for bit.
 *   latent : [tokens][L] bf16;  w : [L][w_heads*P] bf16;  send: bf16.
 * Runs bf16 only (MLA_EUNSUPPORTED otherwise) with L, P, F, col_offset
 * multiples of 8, 16-byte aligned buffers and tables (cs_stride a multiple of
 * 8), and, when R > 0, R = 64 with rope_offset and P multiples of 64 (the MLA
 * query block: P = 192, rope_offset = 128, R = 64).
 * heads <= 256, sp <= 256, L < 2^24 and w_heads*P < 2^25 (the tiles' 32-bit
 * row offsets). tokens == 0 is a no-op.
 */
int mla_project_pack(const void *latent, const void *w, void *send, int64_t tokens, int L, int w_heads, int head_begin,
                     int heads, int P, int F, int col_offset, const int *sizes, int sp, int rope_offset, int R,
                     const void *cos, const void *sin, int64_t cs_stride, int interleaved, int dtype, void *stream);

/*
 * Query partition (host only, no GPU use): hyper-parallel `_causal_partition`.
 * Documents are given by their cumulative ends doc_ends[0..n_docs) (non-
 * negative, non-decreasing; empty documents allowed). The rank owns the query
 * positions [query_rank*query_length, (query_rank+1)*query_length). Each
 * document [a, b) overlapping that range in [s, e) contributes e-s queries,
 * which see the document's keys [a, e) (causal, document-local). The selected
 * key prefixes are adjacent:
 *   *key_begin = start of the first overlapping document, *key_end = end of the
 *   query range;
 *   query_ends / key_ends = cumulative per-document query / key counts (no
 *   leading 0), repeated for each of `batch` sequences with the per-sequence
 *   totals as strides; *n_out = batch * (number of overlapping documents).
 * cap: capacity of query_ends and key_ends, in entries. Fails with MLA_EINVAL,
 * writing nothing, if the documents do not cover the query range or cap is
 * too small (the message gives the count needed).
 */
int mla_causal_partition(const int64_t *doc_ends, int n_docs, int64_t query_length, int query_rank, int batch,
                         int64_t *key_begin, int64_t *key_end, int64_t *query_ends, int64_t *key_ends, int cap,
                         int *n_out);

/*
 * KV exchange ranges (host only): hyper-parallel `_kv_exchange_ranges`. Rank p
 * holds the source tokens [p*source_length, (p+1)*source_length) and owns the
 * queries of partition p / head_copies (mla_causal_partition with batch 1).
 * For every peer p of the `degree` ranks, rank `rank`
 *   sends send_count[p] tokens starting at offset send_offset[p] of its source
 *   range: the part of its source range inside p's key range (0, 0 if none);
 *   receives recv_count[p] tokens: the part of p's source range inside its own
 *   key range.
 * *local_only = 1 when every rank's key range lies inside its own source
 * range (nothing needs to move), else 0. Output arrays hold `degree` entries.
 * Fails with MLA_EINVAL (nothing written) on an invalid argument or when some
 * rank's queries are not covered by the documents.
 */
int mla_kv_exchange_ranges(const int64_t *doc_ends, int n_docs, int64_t source_length, int64_t query_length,
                           int head_copies, int degree, int rank, int64_t *send_offset, int64_t *send_count,
                           int64_t *recv_count, int *local_only);

/*
 * Head->token unpack: the exact inverse of mla_pack_heads (the receive side of
 * the head->token exchange of the attention output, torchtitan "Ulysses CP"
 * `all_to_all_head_to_token(out_THV)`; hyper-parallel `restore_output`).
 *   recv : concatenation over r of slabs [tokens][sizes[r]][feat]
 *   x    : [tokens][heads_total][feat], x[t][off_r + h][f] = slab_r[t][h][f]
 * Same argument rules as mla_pack_heads.
 */
int mla_unpack_heads(const void *recv, void *x, int64_t tokens, int heads_total, int feat,
                     const int *sizes, int sp, int dtype, void *stream);

/*
 * Latent up-projection through wkv_b for a contiguous head range
 * (torchtitan "MLA CP optimization", sections "K/V all-gather CP" and "Ulysses CP":
 * kv_THP = reshape_per_head(wkv_b(kv_c_normed_TL)); hyper-parallel
 * `_head_projection_request`: only the rows of heads [head_begin, head_begin+heads)):
 *   kv_out[t][h][j] = sum_l latent[t][l] * w_kvb[l][(head_begin + h)*(N+V) + j]
 *   latent : [T][L]
 *   w_kvb  : [L][heads_total*(N+V)]  (each head's column block is [k_nope N | v V];
 *            note torch.nn.Linear stores the transpose of this)
 *   kv_out : [T][heads][N+V]         (k_nope = [..., :N], v = [..., N:])
 * Requires 0 <= head_begin, heads >= 1, head_begin + heads <= heads_total,
 * L >= 1, N >= 1, V >= 1, T >= 0. MLA_BF16 additionally needs L, N+V and
 * heads_total*(N+V) to be multiples of 8 and 16-byte aligned pointers.
 */
int mla_latent_up_proj(const void *latent, const void *w_kvb, void *kv_out, int64_t T, int L,
                       int heads_total, int head_begin, int heads, int N, int V, int dtype,
                       void *stream);

/*
 * The same up-projection with the weight as torch.nn.Linear stores wkv_b
 * (hyper-parallel `_validate_up_projections`: weight shape
 * (heads * head_dim, in_features)):
 *   kv_out[t][h][j] = sum_l latent[t][l] * w_lin[(head_begin + h)*(N+V) + j][l]
 *   w_lin  : [heads_total*(N+V)][L], the transpose of mla_latent_up_proj's w_kvb
 * Same arguments, rules and errors as mla_latent_up_proj (MLA_BF16 needs L and
 * N+V multiples of 8 and 16-byte aligned pointers). With the same weight
 * values the result equals mla_latent_up_proj's bit for bit (same products in
 * the same order).
 */
int mla_latent_up_proj_linear(const void *latent, const void *w_lin, void *kv_out, int64_t T, int L,
                              int heads_total, int head_begin, int heads, int N, int V, int dtype,
                              void *stream);

/*
 * Attention of one rank's heads with a head-shared RoPE key band
 * (torchtitan "MLA CP optimization", section "Ulysses CP":
 * k_THK = concat(k_nope_THN, expand_per_head(k_shared_TR)),
 * out_THV = attention(q_THK, k_THK, v_THV); hyper-parallel
 * `_assemble_key_value` and `MLAContextParallel.__call__`, which passes the
 * query and key lengths separately):
 *   s[t][j] = scale * (q[t][h][:N] . kv[j][h][:N] + q[t][h][N:] . k_rope[j][:])
 *   out[t][h][:] = sum_j softmax_j(s[t][.]) * kv[j][h][N:N+V]
 * over the keys j of t's document. When causal, the i-th query of a document
 * (0-based) sees the document's keys with local index <= i + (keys - queries
 * of the document): the last query lines up with the last key, which is
 * "no look-ahead" when the lengths are equal and lets a chunk of queries
 * attend over the whole prefix before it (chunked prefill, attention over an
 * already-projected cache). A query that sees no key (more queries than keys)
 * gets output 0 and lse -inf. The shared band is read once per key tile and
 * never expanded in memory.
 *   q      : [T_q][H][N+R] rows at q + t*q_stride_t + h*q_stride_h
 *   kv     : [T_k][H][N+V] rows at kv + j*kv_stride_t + h*kv_stride_h
 *   k_rope : [T_k][R]      rows at k_rope + j*kr_stride_t
 *   out    : [T_q][H][V]   rows at out + t*o_stride_t + h*o_stride_h, or, with
 *            o_chunk_tokens = C > 0, at out + (t/C)*o_stride_chunk +
 *            (t%C)*o_stride_t + h*o_stride_h: the queries in chunks of C.
 *            With C = T_q/sp, o_stride_chunk = H*V, o_stride_t = sp*H*V and
 *            o_stride_h = V, chunk r (the queries of sequence rank r) lands in
 *            its heads' columns of a token-major [T_q/sp][sp*H][V] buffer:
 *            the output leaves already in the layout that mla_unpack_heads
 *            gives after the head->token exchange (torchtitan "Ulysses CP";
 *            hyper-parallel `restore_output`), with no separate copy. The
 *            chunks' rows must not overlap: either o_stride_chunk >=
 *            C*o_stride_t (chunks one after another) or o_stride_t >=
 *            (ceil(T_q/C)-1)*o_stride_chunk + (H-1)*o_stride_h + V and
 *            o_stride_chunk >= (H-1)*o_stride_h + V (chunks side by side in a
 *            row); MLA_EINVAL otherwise. o_chunk_tokens = 0 is one chunk.
 *   lse    : optional fp32 [H][T_q] (NULL to skip): natural-log softmax denominator
 *   cu_seqlens   : optional DEVICE int32 array of n_seq+1 non-decreasing query
 *            offsets starting at 0 and ending at T_q (packed documents;
 *            hyper-parallel `_causal_partition` uses the same ends without the
 *            leading 0). NULL means one document of T_q queries.
 *   cu_seqlens_k : optional DEVICE int32 array of n_seq+1 key offsets ending at
 *            T_k, the keys of the same documents. NULL means the query offsets
 *            (then T_k must equal T_q), or one document of T_k keys when
 *            cu_seqlens is NULL too. Needs cu_seqlens.
 * Device offsets cannot be checked on the host: the kernels clamp them to
 * [0, T_q] / [0, T_k], so malformed offsets give wrong documents, never an
 * access outside the buffers.
 * bf16 with N=128, R=64, V=128 runs the MFMA tiles, which need 16-byte
 * aligned buffers, strides that are multiples of 8 elements and token strides
 * of at most 2^24 elements (MLA_EUNSUPPORTED otherwise); other widths and
 * MLA_F32 run a plain kernel.
 * The packed q+kv rows of mla_pack_heads can be read in place with
 * q_stride_h = kv_stride_h = F and kv = q + K.
 * Split-KV reductions are not an argument here: the dense causal path splits
 * paired query tiles between workgroups by itself, and the decode step with
 * one query per sequence over a long cache is mla_latent_decode_fwd
 * (num_splits).
 * Workspace: mla_attention_workspace_size() bytes of device memory, 256-byte
 * aligned (0 when none is needed); scratch whose contents need not be
 * initialised and are left arbitrary. Dense causal calls keep there the
 * partial softmax states of the query tiles they split between two
 * workgroups and one arrival flag per split tile. A flag carries a per-call
 * tag drawn when the call is made, so no clearing is needed, and every call
 * leaves each of its flags at "merged" for its tag: a launch captured in a
 * HIP graph (one tag for every replay) can be replayed back to back, with new
 * inputs, on the same workspace. Packed-document calls keep the device-built
 * tile schedule. Calls that may run concurrently (overlapping launches or
 * replays on different streams) need separate workspaces.
 */
typedef struct mla_attn_args {
  const void *q;
  int64_t q_stride_t, q_stride_h;
  const void *kv;
  int64_t kv_stride_t, kv_stride_h;
  const void *k_rope;
  int64_t kr_stride_t;
  void *out;
  int64_t o_stride_t, o_stride_h;
  float *lse;
  const int32_t *cu_seqlens;
  const int32_t *cu_seqlens_k;
  int n_seq;
  int64_t T_q, T_k;
  int H, N, R, V;
  float scale;
  int causal;
  int dtype;
  void *workspace;
  size_t workspace_bytes;
  int64_t o_chunk_tokens, o_stride_chunk;   /* 0, 0: out rows at t*o_stride_t (see out above) */
} mla_attn_args;

size_t mla_attention_workspace_size(const mla_attn_args *a);
int mla_attention_fwd(const mla_attn_args *a, void *stream);

/*
 * mla_attention_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, result and validation as mla_attention_fwd,
 * except that a->workspace and a->workspace_bytes are ignored: the call's
 * scratch is a fixed array of MLA_NOALLOC_SCRATCH_BYTES inside the library,
 * one copy per GPU, held until the process ends (its device address is
 * looked up on the first call on each device). The call allocates nothing.
 * A call whose mla_attention_workspace_size() exceeds MLA_NOALLOC_SCRATCH_BYTES
 * fails with MLA_EUNSUPPORTED and launches nothing (48 MiB covers, e.g., dense
 * causal attention of 16 heads up to T = 8192 or 22 heads at T = 4096, and any
 * packed-document call up to millions of tokens). Every call on a GPU shares
 * that GPU's array: calls that overlap on one GPU (different streams, or
 * graphs replayed concurrently) race and give wrong results. Nothing in the
 * scratch needs clearing between calls.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
int mla_attention_fwd_noalloc(const mla_attn_args *a, void *stream);

/*
 * Backward of mla_attention_fwd (torchtitan "MLA CP optimization", section
 * "Numerical comparison": the method is trained end to end; hyper-parallel
 * `_assemble_key_value`: the shared band is one tensor repeated over the
 * heads, so it receives the SUM of the heads' band gradients). With p the
 * probabilities rebuilt from lse, D_t = dout[t][h] . out[t][h] and the key
 * k = [k_nope | k_rope]:
 *   dv = p^T dout, ds = p (dout v^T - D), dq = scale ds k, dk = scale ds^T q,
 *   dk_rope[j] = sum over h of dk[j][h][N:].
 * Inputs as in mla_attention_fwd (same strides, documents and causal flag),
 * plus:
 *   out    : [T][H][V] the forward's output, rows at out + t*o_stride_t + h*o_stride_h
 *   dout   : [T][H][V] gradient of out, rows at dout + t*do_stride_t + h*do_stride_h
 *   lse    : fp32 [H][T], the forward's natural-log softmax denominator
 * Outputs (fp32, contiguous, every element written):
 *   dq     : [T][H][N+R]
 *   dkv    : [T][H][N+V]  (= [dk_nope | dv], the layout of kv)
 *   dk_rope: [T][R]
 * Runs bf16 with N=128, R=64, V=128 (MLA_EUNSUPPORTED otherwise), 16-byte
 * aligned inputs and dk_rope, strides that are multiples of 8 elements and
 * token strides of at most 2^24 elements.
 * Workspace: mla_attention_bwd_workspace_size() bytes, 256-byte aligned,
 * contents need not be initialised (row terms and per-head band gradients).
 * The result does not depend on scheduling: every sum runs in a fixed order.
 */
typedef struct mla_attn_bwd_args {
  const void *q;
  int64_t q_stride_t, q_stride_h;
  const void *kv;
  int64_t kv_stride_t, kv_stride_h;
  const void *k_rope;
  int64_t kr_stride_t;
  const void *out;
  int64_t o_stride_t, o_stride_h;
  const void *dout;
  int64_t do_stride_t, do_stride_h;
  const float *lse;
  float *dq;
  float *dkv;
  float *dk_rope;
  const int32_t *cu_seqlens;
  int n_seq;
  int64_t T;
  int H, N, R, V;
  float scale;
  int causal;
  int dtype;
  void *workspace;
  size_t workspace_bytes;
} mla_attn_bwd_args;

size_t mla_attention_bwd_workspace_size(const mla_attn_bwd_args *a);
int mla_attention_bwd(const mla_attn_bwd_args *a, void *stream);

/*
 * Backward of mla_latent_up_proj (torchtitan "MLA CP optimization", section
 * "Ulysses CP": k_nope and v are linear in the KV latent; section "Numerical
 * comparison": the method is trained): with C = heads*(N+V) and the head
 * range's weight columns w[:, col0 + c], col0 = head_begin*(N+V),
 *   d_latent[t][l] = sum_c dkv[t][c] w[l][col0 + c]
 *   dw[l][c]       = sum_t latent[t][l] dkv[t][c]
 *   latent   : bf16 [T][L]
 *   w_kvb    : bf16 [L][heads_total*(N+V)]
 *   dkv      : fp32 [T][heads][N+V] (mla_attention_bwd's dkv of these heads)
 *   d_latent : fp32 [T][L], overwritten
 *   dw       : fp32 [L][heads*(N+V)], overwritten: the gradient of the head
 *              range's columns (the other columns get none from these heads)
 * dkv is rounded to bf16 as an MFMA operand; products accumulate in fp32.
 * Runs bf16 with L and heads*(N+V) multiples of 32, N+V a multiple of 8, and
 * 16-byte aligned latent, w_kvb and dkv (MLA_EUNSUPPORTED otherwise).
 * T = 0 zeroes dw.
 * workspace (optional, 256-byte aligned, contents need not be initialised):
 * with T, L and heads*(N+V) multiples of 128 and workspace_bytes at least
 * mla_latent_up_proj_bwd_workspace_size(), each product's contraction is
 * split over more workgroups and the fp32 partials are summed in a fixed
 * order (the results do not depend on scheduling either way); otherwise, or
 * with workspace NULL, single-pass kernels run and the workspace is unused.
 * The workspace must not be shared with work running concurrently.
 */
size_t mla_latent_up_proj_bwd_workspace_size(int64_t T, int L, int heads, int N, int V);
int mla_latent_up_proj_bwd(const void *latent, const void *w_kvb, const float *dkv, float *d_latent, float *dw,
                           int64_t T, int L, int heads_total, int head_begin, int heads, int N, int V, int dtype,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Latent-cache decode: one new query token per sequence attends over its whole
 * cached latent, reduced in num_splits KV chunks with an online softmax
 * (DeepSpeed PR #8602, "Components": decode attention with KV split-K and an
 * online softmax) and combined as m = max_c m_c, l = sum_c l_c e^(m_c - m),
 * o = sum_c l_c e^(m_c - m) o_c / l.
 * The keys and values are the latent-first up-projection of the cache
 * (k_nope, v = latent_cache[b] @ w_kvb columns of each head) with the shared
 * band rope_cache[b]; no mask (the query is the newest token).
 *   q            : [B][H][N+R]
 *   latent_cache : [B][S][L]
 *   rope_cache   : [B][S][R]
 *   w_kvb        : [L][heads_total*(N+V)], heads [head_begin, head_begin+H)
 *   out          : [B][H][V]
 *   lse          : optional fp32 [B][H]
 * MLA_BF16 only; 1 <= num_splits <= min(S, 256) (more than 256: MLA_EUNSUPPORTED).
 * B <= 2^20 sequences per call (MLA_EUNSUPPORTED beyond).
 * Workspace: mla_latent_decode_workspace_size() bytes, 256-byte aligned;
 * contents need not be initialised.
 */
typedef struct mla_decode_args {
  const void *q;
  const void *latent_cache;
  const void *rope_cache;
  const void *w_kvb;
  void *out;
  float *lse;
  int B;
  int64_t S;
  int L, H, heads_total, head_begin, N, R, V;
  int num_splits;
  float scale;
  int dtype;
  void *workspace;
  size_t workspace_bytes;
} mla_decode_args;

size_t mla_latent_decode_workspace_size(const mla_decode_args *a);
int mla_latent_decode_fwd(const mla_decode_args *a, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H_ */
