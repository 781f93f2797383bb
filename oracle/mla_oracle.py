"""fp64 CPU oracle for one Ulysses rank's share of Multi-head Latent Attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
library never imports, links or calls it, and it shares no code with the HIP
library: the only module both sides use is ``mla_inputs`` (seeded random draws).

Every function is the plain definition of what the pages compute, written in
NumPy float64, with no blocking or fusion beyond what that definition states:

* head shard lists      -- DeepSpeed PR #8316 "[Ulysses] Carry the KV head count
                           per DistributedAttention", sections "What breaks" and
                           "The change" (KV-following split, GQA groups), and the
                           review thread (reject fewer KV heads than ranks before
                           any collective).
* token<->head pack     -- torchtitan PR #5445 carrying the "MLA CP optimization"
                           commit message, section "Ulysses CP" (one exchange of
                           concat(q_THK, kv_THP)); hyper-parallel
                           mla_context_parallel.py, ``_expanded``/``restore_output``.
* latent up-projection  -- torchtitan "MLA CP optimization", sections "K/V
                           all-gather CP" and "Ulysses CP" (``wkv_b`` then
                           ``unpack``); hyper-parallel ``_head_projection_request``
                           (contiguous head rows) and ``_assemble_key_value``.
* attention             -- the same sections (``attention(q_THK, k_THK, v_THV)``
                           with ``k_THK = concat(k_nope, expand_per_head(k_shared))``);
                           hyper-parallel ``MLAContextParallel.__call__`` (scaling,
                           causal with no look-ahead) and ``_causal_partition``
                           (documents as cumulative ends).
* split-KV decode       -- DeepSpeed PR #8602, "Components" table (decode
                           attention with KV split-K and an online softmax).
* expanded pack         -- hyper-parallel ``_expanded`` (one sequence-to-head
                           exchange of concat(q, k, v) with unequal widths, the
                           key assembled by ``_assemble_key_value``).
* backward              -- torchtitan "MLA CP optimization", section
                           "Numerical comparison" (the two forms' gradients);
                           hyper-parallel ``_selective_kv_launch`` (SUM
                           gradients through repeated slices: the shared RoPE
                           key's gradient is the sum over heads).
* rotary embedding      -- hyper-parallel ``apply_mla_rope`` (position tables
                           given by the caller in the tensor's dtype; half-band
                           rotation, or adjacent pairs rotated and returned as
                           real then imaginary half-bands).
* query partition and   -- hyper-parallel ``_causal_partition`` and
  KV exchange ranges       ``_kv_exchange_ranges`` (document-local causal
                           prefixes of a rank's contiguous query range; the key
                           interval each rank sends to and receives from every
                           peer).

Readings where the pages are silent (each also listed in the design doc):
the scale is an explicit argument; key j is visible to query t iff j <= t in the
same document; documents are given as cu_seqlens with a leading 0; inputs are
post-RoPE; the weight is row-major [L][heads_total*(N+V)] with each head's
column block [k_nope N | v V]; the packed row is [q_nope | q_rope | k_nope | v].

Parity status: every function below is pinned by tests in ``tests/`` against
worked examples printed on the pages, closed forms, library routines or brute
force (see ``tests/test_oracle_*.py``). None is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "widen", "head_shard_rule", "head_shard_sizes", "head_offsets",
    "pack_heads", "unpack_heads", "latent_up_proj", "attention_probs",
    "attention", "decode_split_kv", "decode_reference", "doc_bounds",
    "ulysses_materialise_k_first", "ulysses_latent_first",
    "pack_expanded", "causal_partition", "kv_exchange_ranges", "rope", "key_bounds",
    "attention_backward", "latent_up_proj_backward",
]


def widen(x) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) or fp32 arrays to float64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# --------------------------------------------------------------------------
# Head shard lists (DeepSpeed PR #8316)
# --------------------------------------------------------------------------

def head_shard_rule(q_heads: int, kv_heads: int, sp: int) -> list[int]:
    """The split rule alone, without the guard.

    KV heads are dealt out as evenly as possible with the remainder going to the
    lowest ranks, and every KV head carries its whole group of q_heads/kv_heads
    query heads, so a query head always lands on the rank that holds its KV head
    (PR #8316, "The change": Q=6/KV=3 over sp=2 must give [4, 2]).
    """
    group = q_heads // kv_heads
    base, extra = divmod(kv_heads, sp)
    return [(base + (1 if r < extra else 0)) * group for r in range(sp)]


def head_shard_sizes(q_heads: int, kv_heads: int, sp: int) -> list[int]:
    """Validated shard list: query heads per rank, ranks in order.

    Rejected before any exchange (PR #8316 review thread): sp < 1, q_heads < 1,
    kv_heads < 1, a query count that is not a whole number of KV groups, and
    fewer KV heads than ranks (a rank would receive zero heads).
    """
    if sp < 1 or q_heads < 1 or kv_heads < 1:
        raise ValueError(f"heads and sp must be positive (q={q_heads}, kv={kv_heads}, sp={sp})")
    if q_heads % kv_heads:
        raise ValueError(f"q_heads ({q_heads}) is not a multiple of kv_heads ({kv_heads})")
    if kv_heads < sp:
        raise ValueError(f"kv_heads ({kv_heads}) < sp ({sp}): some rank would own no KV head")
    return head_shard_rule(q_heads, kv_heads, sp)


def head_offsets(sizes) -> list[int]:
    """First head of each rank: rank r owns heads [off_r, off_r + sizes[r])."""
    offs, acc = [], 0
    for s in sizes:
        offs.append(acc)
        acc += s
    return offs


# --------------------------------------------------------------------------
# Token <-> head pack (torchtitan "Ulysses CP"; hyper-parallel _expanded)
# --------------------------------------------------------------------------

def pack_heads(x: np.ndarray, sizes) -> np.ndarray:
    """Send side of the token->head exchange.

    x is [T][heads_total][F]. The result is the concatenation over ranks r of
    the slab x[:, off_r:off_r+sizes[r], :], each slab laid out [T][sizes[r]][F]:
    send[base_r + (t*q_r + h')*F + f] = x[t][off_r + h'][f], base_r = T*off_r*F.
    Returned flat (1-D), in the dtype of x (a pure permutation of elements).
    """
    T, H, F = x.shape
    assert sum(sizes) == H
    slabs = [np.ascontiguousarray(x[:, o:o + q, :]).reshape(-1)
             for o, q in zip(head_offsets(sizes), sizes)]
    return np.concatenate(slabs) if slabs else np.zeros(0, x.dtype)


def unpack_heads(send: np.ndarray, sizes, tokens: int, feat: int) -> np.ndarray:
    """Exact inverse of ``pack_heads``: back to [T][heads_total][F]."""
    H = sum(sizes)
    out = np.empty((tokens, H, feat), dtype=send.dtype)
    for o, q in zip(head_offsets(sizes), sizes):
        base = tokens * o * feat
        out[:, o:o + q, :] = send[base:base + tokens * q * feat].reshape(tokens, q, feat)
    return out


# --------------------------------------------------------------------------
# Latent up-projection (torchtitan wkv_b; hyper-parallel head-range rows)
# --------------------------------------------------------------------------

def latent_up_proj(latent, w_kvb, head_begin: int, heads: int, N: int, V: int) -> np.ndarray:
    """kv[t][h][j] = sum_l latent[t][l] * W[l][(head_begin+h)*(N+V) + j].

    latent [T][L], W [L][heads_total*(N+V)] -> kv [T][heads][N+V] (float64);
    kv[..., :N] is k_nope and kv[..., N:] is v. The head range must lie inside W.
    """
    c = widen(latent)
    W = widen(w_kvb)
    P = N + V
    if not (0 <= head_begin and heads >= 1 and (head_begin + heads) * P <= W.shape[1]):
        raise ValueError("head range outside the projection weight")
    cols = W[:, head_begin * P:(head_begin + heads) * P]
    return (c @ cols).reshape(c.shape[0], heads, P)


# --------------------------------------------------------------------------
# Attention with a head-shared RoPE key band
# --------------------------------------------------------------------------

def doc_bounds(cu_seqlens=None, T: int | None = None, ends=None) -> list[tuple[int, int]]:
    """Document [start, end) ranges.

    Accepts cu_seqlens with a leading 0 (n+1 entries) or, as hyper-parallel's
    ``_causal_partition`` passes them, cumulative document ends without the 0.
    With neither, the whole sequence of length T is one document.
    """
    if cu_seqlens is None and ends is None:
        return [(0, int(T))]
    if ends is not None:
        cu = [0] + [int(e) for e in ends]
    else:
        cu = [int(e) for e in cu_seqlens]
        if cu[0] != 0:
            raise ValueError("cu_seqlens must start at 0")
    if any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must be non-decreasing")
    return [(a, b) for a, b in zip(cu, cu[1:])]


def key_bounds(cu_seqlens_k=None, T_k: int | None = None, n_docs: int = 1) -> list[tuple[int, int]]:
    """Key document [start, end) ranges: from cu_seqlens_k (leading 0), else one range of T_k keys."""
    if cu_seqlens_k is None:
        assert n_docs == 1, "documents of queries need the keys' document offsets"
        return [(0, int(T_k))]
    return doc_bounds(cu_seqlens_k)


def _scores(q, kv, k_rope, h, rows, cols, N, scale):
    """s[t][j] = scale * (q_nope[t]·k_nope[j] + q_rope[t]·k_rope[j]) for head h."""
    qn, qr = q[rows, h, :N], q[rows, h, N:]
    kn = kv[cols, h, :N]
    kr = k_rope[cols]
    return scale * (qn @ kn.T + qr @ kr.T)


def attention_probs(q, kv, k_rope, N, scale, causal=True, cu_seqlens=None, h=0):
    """Full [T][T] probability matrix of head h (0 where a key is not visible)."""
    q, kv, k_rope = widen(q), widen(kv), widen(k_rope)
    T = q.shape[0]
    Pm = np.zeros((T, T))
    for a, b in doc_bounds(cu_seqlens, T):
        if b == a:
            continue
        s = _scores(q, kv, k_rope, h, slice(a, b), slice(a, b), N, scale)
        if causal:
            s = np.where(np.tril(np.ones((b - a, b - a), bool)), s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        Pm[a:b, a:b] = e / e.sum(axis=1, keepdims=True)
    return Pm


def attention(q, kv, k_rope, N: int, scale: float, causal: bool = True, cu_seqlens=None,
              rows=None, cu_seqlens_k=None):
    """Causal (or full) softmax attention of one rank's heads.

    q [T_q][H][N+R] (= [q_nope | q_rope]), kv [T_k][H][N+V] (= [k_nope | v]),
    k_rope [T_k][R] shared by every head. Query documents come from cu_seqlens
    (over the T_q query rows) and key documents from cu_seqlens_k (over the
    T_k key rows; None: the same offsets as the queries, which needs T_k =
    T_q). A query attends to the keys of its own document; when causal, the
    i-th query of a document (0-based) sees the document's keys j <= i +
    (keys - queries of that document): the last query lines up with the last
    key, so with equal lengths this is j <= i (no look-ahead), and a chunk of
    queries at the end of a longer key sequence sees the whole prefix before
    it. A query that sees no key (more queries than keys) has output 0 and
    lse -inf. Returns out [T_q][H][V] and lse [H][T_q] (natural log of the
    softmax denominator, including the max). ``rows`` optionally restricts the
    computation to those query rows (the rest of ``out``/``lse`` is NaN) so
    large workloads can be sampled.
    """
    q, kv, k_rope = widen(q), widen(kv), widen(k_rope)
    T, H, _ = q.shape
    T_k = kv.shape[0]
    V = kv.shape[2] - N
    out = np.full((T, H, V), np.nan)
    lse = np.full((H, T), np.nan)
    want = None if rows is None else np.zeros(T, bool)
    if want is not None:
        want[np.asarray(rows)] = True
    qdocs = doc_bounds(cu_seqlens, T)
    if cu_seqlens_k is None and cu_seqlens is not None:
        if T_k != T:
            raise ValueError("documents of queries and keys with T_k != T_q need cu_seqlens_k")
        kdocs = qdocs
    else:
        kdocs = key_bounds(cu_seqlens_k, T_k, len(qdocs))
    if len(kdocs) != len(qdocs):
        raise ValueError("cu_seqlens and cu_seqlens_k describe different document counts")
    for (a, b), (ka, kb) in zip(qdocs, kdocs):
        if b == a:
            continue
        qi = np.arange(a, b) if want is None else np.arange(a, b)[want[a:b]]
        if qi.size == 0:
            continue
        shift = (kb - ka) - (b - a)                      # the last query lines up with the last key
        for h in range(H):
            s = _scores(q, kv, k_rope, h, qi, slice(ka, kb), N, scale)
            if causal:
                s = np.where((np.arange(ka, kb) - ka)[None, :] <= (qi - a)[:, None] + shift, s, -np.inf)
            seen = np.isfinite(s).any(axis=1) if s.shape[1] else np.zeros(len(qi), bool)
            m = np.where(seen, s.max(axis=1) if s.shape[1] else 0.0, 0.0)[:, None]
            e = np.where(seen[:, None], np.exp(s - m), 0.0)
            den = e.sum(axis=1, keepdims=True)
            o = np.zeros((len(qi), V))
            o[seen] = (e[seen] / den[seen]) @ kv[ka:kb, h, N:]
            out[qi, h, :] = o
            lse[h, qi] = np.where(seen, (m + np.log(np.where(seen[:, None], den, 1.0)))[:, 0], -np.inf)
    return out, lse


# --------------------------------------------------------------------------
# Latent-cache decode with a split-KV online-softmax reduction
# --------------------------------------------------------------------------

def decode_split_kv(q, latent, k_rope, w_kvb, N: int, V: int, scale: float, splits: int,
                    seqs=None):
    """One new query per sequence over its whole cached latent, in ``splits`` chunks.

    For each sequence b: up-project the cached latent for all heads (the
    latent-first projection), score every cached position (no mask: the query
    is the newest token), and reduce chunk by chunk. Chunk c yields its own max
    m_c, denominator l_c and normalised output o_c; the chunks combine as
    m = max_c m_c, l = sum_c l_c e^(m_c-m), o = sum_c l_c e^(m_c-m) o_c / l.
    q [B][H][N+R], latent [B][S][L], k_rope [B][S][R] -> out [B][H][V] and the
    partials (m, l [B][H][splits], o_c [B][H][splits][V]). ``seqs`` samples b.
    """
    q, c_all, kr_all = widen(q), widen(latent), widen(k_rope)
    B, H, _ = q.shape
    S = c_all.shape[1]
    seqs = range(B) if seqs is None else seqs
    out = np.full((B, H, V), np.nan)
    m_p = np.full((B, H, splits), np.nan)
    l_p = np.full((B, H, splits), np.nan)
    o_p = np.full((B, H, splits, V), np.nan)
    chunk = -(-S // splits)
    for b in seqs:
        kv = latent_up_proj(c_all[b], w_kvb, 0, H, N, V)          # [S][H][N+V]
        for h in range(H):
            s = scale * (kv[:, h, :N] @ q[b, h, :N] + kr_all[b] @ q[b, h, N:])   # [S]
            for ci in range(splits):
                lo, hi = ci * chunk, min(S, (ci + 1) * chunk)
                if hi <= lo:
                    m_p[b, h, ci], l_p[b, h, ci], o_p[b, h, ci] = -np.inf, 0.0, 0.0
                    continue
                mc = s[lo:hi].max()
                e = np.exp(s[lo:hi] - mc)
                m_p[b, h, ci], l_p[b, h, ci] = mc, e.sum()
                o_p[b, h, ci] = (e @ kv[lo:hi, h, N:]) / e.sum()
            m = m_p[b, h].max()
            wgt = l_p[b, h] * np.exp(m_p[b, h] - m)
            out[b, h] = (wgt[:, None] * o_p[b, h]).sum(axis=0) / wgt.sum()
    return out, (m_p, l_p, o_p)


def decode_reference(q, latent, k_rope, w_kvb, N: int, V: int, scale: float, seqs=None):
    """Direct (unsplit) softmax for the decode step: the definition split-KV must reach."""
    q, c_all, kr_all = widen(q), widen(latent), widen(k_rope)
    B, H, _ = q.shape
    seqs = range(B) if seqs is None else seqs
    out = np.full((B, H, V), np.nan)
    for b in seqs:
        kv = latent_up_proj(c_all[b], w_kvb, 0, H, N, V)
        for h in range(H):
            s = scale * (kv[:, h, :N] @ q[b, h, :N] + kr_all[b] @ q[b, h, N:])
            e = np.exp(s - s.max())
            out[b, h] = (e / e.sum()) @ kv[:, h, N:]
    return out


# --------------------------------------------------------------------------
# The two orders of the rank computation (torchtitan "MLA CP optimization")
# --------------------------------------------------------------------------

def ulysses_materialise_k_first(latent, w_kvb, q, k_rope, sizes, N, V, scale):
    """Project every head on each rank's own tokens, pack [q | kv], exchange, attend.

    Simulates sp ranks that each hold T/sp consecutive tokens of latent, q
    (all heads) and k_rope. Each rank projects all heads, builds F-rows
    [q_nope | q_rope | k_nope | v], packs them by the shard list; rank r then
    receives slice r of every peer (in rank order, i.e. token order), splits
    the rows and attends over the full sequence with the all-gathered k_rope.
    Returns the per-rank outputs [T][sizes[r]][V].
    """
    latent, w_kvb, q, k_rope = widen(latent), widen(w_kvb), widen(q), widen(k_rope)
    sp = len(sizes)
    T, Htot, K = q.shape
    P = N + V
    F = K + P
    Tl = T // sp
    sends = []
    for s in range(sp):
        tok = slice(s * Tl, (s + 1) * Tl)
        kv_loc = latent_up_proj(latent[tok], w_kvb, 0, Htot, N, V)
        rows = np.concatenate([q[tok], kv_loc], axis=2)            # [Tl][Htot][F]
        sends.append(pack_heads(rows, sizes))
    outs = []
    for r, (o, qr) in enumerate(zip(head_offsets(sizes), sizes)):
        base, n = Tl * o * F, Tl * qr * F
        recv = np.concatenate([snd[base:base + n].reshape(Tl, qr, F) for snd in sends], axis=0)
        q_r, kv_r = recv[:, :, :K], recv[:, :, K:]
        out, _ = attention(q_r, kv_r, k_rope, N, scale, causal=True)
        outs.append(out)
    return outs


def ulysses_latent_first(latent, w_kvb, q, k_rope, sizes, N, V, scale):
    """Gather the latents first, then project only the rank's own head range, attend."""
    latent, w_kvb, q, k_rope = widen(latent), widen(w_kvb), widen(q), widen(k_rope)
    outs = []
    for o, qr in zip(head_offsets(sizes), sizes):
        kv = latent_up_proj(latent, w_kvb, o, qr, N, V)
        out, _ = attention(q[:, o:o + qr, :], kv, k_rope, N, scale, causal=True)
        outs.append(out)
    return outs


# --------------------------------------------------------------------------
# Expanded pack (hyper-parallel _expanded, key from _assemble_key_value)
# --------------------------------------------------------------------------

def pack_expanded(q: np.ndarray, kv: np.ndarray, k_rope: np.ndarray, N: int, sizes) -> np.ndarray:
    """Send side of the expanded exchange: one payload row per (token, head),
    [q (N+R) | k_nope (N) | k_rope (R) | v (V)], the shared RoPE key copied into
    every head's key, then split into per-rank head slabs exactly as
    ``pack_heads``.

    q [T][H][N+R], kv [T][H][N+V] ([k_nope | v]), k_rope [T][R] -> flat send.
    A pure permutation-with-copies of elements: dtypes are kept.
    """
    T, H, K = q.shape
    assert kv.shape[:2] == (T, H) and k_rope.shape[0] == T
    R = k_rope.shape[1]
    assert K == N + R
    key = np.concatenate([kv[:, :, :N], np.broadcast_to(k_rope[:, None, :], (T, H, R))], axis=2)
    payload = np.concatenate([q, key, kv[:, :, N:]], axis=2)
    return pack_heads(payload, sizes)


# --------------------------------------------------------------------------
# Query partition and KV exchange ranges (hyper-parallel _causal_partition,
# _kv_exchange_ranges)
# --------------------------------------------------------------------------

def causal_partition(ends, query_length: int, query_rank: int, batch: int = 1) -> dict:
    """The documents' causal prefixes needed by one rank's contiguous queries.

    Documents are given by their cumulative ends. The rank owns global query
    positions [query_rank*query_length, (query_rank+1)*query_length). For every
    document [a, b) that overlaps that range in [s, e), the rank holds e-s
    queries of the document, and those queries see the document's keys [a, e)
    (causal, no look-ahead, document-local). The selected prefixes are
    adjacent, so the keys form one range [key_begin, key_end) with key_end the
    end of the query range. query_ends / key_ends are the cumulative per-
    document query and key counts (variable-length offsets without the leading
    0), repeated for each of ``batch`` sequences with the per-sequence totals
    as strides. Raises ValueError when the documents do not cover the range.
    """
    q0, q1 = query_rank * query_length, (query_rank + 1) * query_length
    parts = []
    for a, b in doc_bounds(ends=ends):
        s, e = max(a, q0), min(b, q1)
        if s < e:
            parts.append((a, s, e))
    if sum(e - s for _, s, e in parts) != query_length:
        raise ValueError("documents do not cover the query partition")
    q_lens = [e - s for _, s, e in parts]
    k_lens = [e - a for a, _, e in parts]
    q_ends = list(np.cumsum(q_lens, dtype=np.int64))
    k_ends = list(np.cumsum(k_lens, dtype=np.int64))
    nq, nk = int(sum(q_lens)), int(sum(k_lens))
    return {
        "key_begin": int(parts[0][0]),
        "key_end": int(q1),
        "query_ends": [int(x) + i * nq for i in range(batch) for x in q_ends],
        "key_ends": [int(x) + i * nk for i in range(batch) for x in k_ends],
        "documents": tuple(int(x) for x in ends),
    }


def kv_exchange_ranges(ends, source_length: int, query_length: int, head_copies: int, degree: int, rank: int):
    """Which key tokens rank ``rank`` sends to and receives from every peer.

    Rank p holds the source tokens [p*source_length, (p+1)*source_length) and
    owns the queries of query partition p // head_copies (head_copies ranks
    share one query range). A rank sends to peer p the part of its source
    range inside p's key range (as (offset in its source range, count)), and
    receives from peer p the part of p's source range inside its own key
    range (a count). local_only: every rank's key range lies inside its own
    source range, so nothing needs to move.
    """
    dest = [causal_partition(ends, query_length, p // head_copies, 1) for p in range(degree)]

    def overlap(a0, a1, b0, b1):
        return max(a0, b0), min(a1, b1)

    s0, s1 = rank * source_length, (rank + 1) * source_length
    sends, receives = [], []
    for p in range(degree):
        b, e = overlap(s0, s1, dest[p]["key_begin"], dest[p]["key_end"])
        sends.append((b - s0, e - b) if b < e else (0, 0))
        b, e = overlap(p * source_length, (p + 1) * source_length, dest[rank]["key_begin"], dest[rank]["key_end"])
        receives.append(max(0, e - b))
    local_only = all(p * source_length <= d["key_begin"] and d["key_end"] <= (p + 1) * source_length
                     for p, d in enumerate(dest))
    return tuple(sends), tuple(receives), local_only


# --------------------------------------------------------------------------
# Rotary embedding of the RoPE band (hyper-parallel apply_mla_rope)
# --------------------------------------------------------------------------

def rope(x, cos, sin, interleaved: bool = False) -> np.ndarray:
    """Rotate the RoPE band x [T][...][R] by per-token tables cos, sin [T][R].

    The tables are the caller's position embeddings in the tensor's dtype (the
    pages cast them to it), one angle per pair: for the half-band form entry i
    and i + R/2 carry the same angle. Half-band (interleaved=False): with
    x = [a | b] (halves of R/2), out = [a cos - b sin | b cos + a sin], i.e. the
    complex number a + i b times e^{i angle}. Interleaved: the pairs are
    adjacent, (x[2i], x[2i+1]) times e^{i angle_i} with angle_i from the first
    R/2 table entries, and the result is returned as the real parts followed by
    the imaginary parts (half-band order). float64 result.
    """
    x = widen(x)
    c, sn = widen(cos), widen(sin)
    T, R = c.shape
    assert x.shape[0] == T and x.shape[-1] == R and R % 2 == 0
    h = R // 2
    shape = (T,) + (1,) * (x.ndim - 2) + (R,)
    c, sn = c.reshape(shape), sn.reshape(shape)
    if not interleaved:
        a, b = x[..., :h], x[..., h:]
        return np.concatenate([a * c[..., :h] - b * sn[..., :h], b * c[..., h:] + a * sn[..., h:]], axis=-1)
    re_in, im_in = x[..., 0::2], x[..., 1::2]
    ci, si = c[..., :h], sn[..., :h]
    return np.concatenate([re_in * ci - im_in * si, im_in * ci + re_in * si], axis=-1)


# --------------------------------------------------------------------------
# Backward of the shard: attention, then the latent up-projection
# --------------------------------------------------------------------------

def attention_backward(q, kv, k_rope, dout, N: int, scale: float, causal: bool = True, cu_seqlens=None):
    """Gradients of ``attention``'s output against dout [T][H][V].

    Per document and head, with p the probabilities, v the values and k the
    assembled key [k_nope | k_rope]: dv = p^T dout, dp = dout v^T, the row term
    D_t = sum_j p_tj dp_tj, ds = p (dp - D), dq = scale ds k, dk = scale ds^T q.
    Returns dq [T][H][N+R], dkv [T][H][N+V] (= [dk_nope | dv]) and dk_rope [T][R]:
    the shared band receives the SUM over heads of each head's band gradient.
    float64.
    """
    q, kv, k_rope, dout = widen(q), widen(kv), widen(k_rope), widen(dout)
    T, H, _ = q.shape
    dq = np.zeros_like(q)
    dkv = np.zeros_like(kv)
    dkr = np.zeros_like(k_rope)
    for a, b in doc_bounds(cu_seqlens, T):
        if b == a:
            continue
        for h in range(H):
            s = _scores(q, kv, k_rope, h, slice(a, b), slice(a, b), N, scale)
            if causal:
                s = np.where(np.tril(np.ones((b - a, b - a), bool)), s, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            v, do = kv[a:b, h, N:], dout[a:b, h]
            dp = do @ v.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            k = np.concatenate([kv[a:b, h, :N], k_rope[a:b]], axis=1)
            dq[a:b, h] = scale * (ds @ k)
            dk = scale * (ds.T @ q[a:b, h])
            dkv[a:b, h, :N] = dk[:, :N]
            dkv[a:b, h, N:] = p.T @ do
            dkr[a:b] += dk[:, N:]
    return dq, dkv, dkr


def latent_up_proj_backward(latent, w_kvb, head_begin: int, heads: int, dkv, N: int, V: int):
    """Gradients of ``latent_up_proj`` against dkv [T][heads][N+V]: d_latent [T][L] =
    dkv W_cols^T and dW = latent^T dkv on the head range's columns (zero elsewhere). float64."""
    c, W, g = widen(latent), widen(w_kvb), widen(dkv)
    P = N + V
    cols = slice(head_begin * P, (head_begin + heads) * P)
    g2 = g.reshape(c.shape[0], heads * P)
    dW = np.zeros_like(W)
    dW[:, cols] = c.T @ g2
    return g2 @ W[:, cols].T, dW
