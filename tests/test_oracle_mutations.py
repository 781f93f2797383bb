"""Planted mistakes: each plausible slip in the oracle must fail at least one pin.

Mistakes are planted in the oracle only, on the CPU, by monkeypatching.
"""
import numpy as np
import pytest

import oracle
import oracle.mla_oracle as om
import test_oracle_numerics as tn
import test_oracle_shard_pack as ts
from golden_io import shard_cases


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(om, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)


def _fails(fn, *args):
    try:
        fn(*args)
    except (Exception, pytest.fail.Exception):
        return True
    return False


def _any_attention_pin_fails():
    pins = [
        lambda: tn.test_attention_matches_sdpa_with_expanded_key(True),
        tn.test_attention_tiny_config_matches_sdpa,
        tn.test_varlen_matches_sdpa_block_diagonal_mask_and_separate_runs,
        tn.test_first_token_of_each_document_returns_its_value_row,
        tn.test_zero_query_gives_running_mean_of_values,
        tn.test_attention_brute_force_tiny,
    ]
    return any(_fails(p) for p in pins)


def test_dropped_rope_term_is_caught(monkeypatch):
    def bad(q, kv, k_rope, h, rows, cols, N, scale):
        return scale * (q[rows, h, :N] @ kv[cols, h, :N].T)
    _patch(monkeypatch, "_scores", bad)
    assert _any_attention_pin_fails()


def test_missing_scale_is_caught(monkeypatch):
    def bad(q, kv, k_rope, h, rows, cols, N, scale):
        return q[rows, h, :N] @ kv[cols, h, :N].T + q[rows, h, N:] @ k_rope[cols].T
    _patch(monkeypatch, "_scores", bad)
    assert _any_attention_pin_fails()


def test_rope_band_taken_from_wrong_operand_is_caught(monkeypatch):
    # q_rope paired with k_nope's tail instead of the shared band
    def bad(q, kv, k_rope, h, rows, cols, N, scale):
        R = k_rope.shape[1]
        return scale * (q[rows, h, :N] @ kv[cols, h, :N].T + q[rows, h, N:] @ kv[cols, h, N - R:N].T)
    _patch(monkeypatch, "_scores", bad)
    assert _any_attention_pin_fails()


def test_wrong_sign_is_caught(monkeypatch):
    orig = om._scores
    _patch(monkeypatch, "_scores", lambda *a: -orig(*a))
    assert _any_attention_pin_fails()


def test_strict_causal_mask_is_caught(monkeypatch):
    # a query that may not see itself (j < t): the first-token pin must fail
    orig = om.attention

    def bad(q, kv, k_rope, N, scale, causal=True, cu_seqlens=None, rows=None):
        out, lse = orig(q, kv, k_rope, N, scale, causal, cu_seqlens, rows)
        qq, kk, rr = om.widen(q), om.widen(kv), om.widen(k_rope)
        out = out.copy()
        # shift by one key: o_t := o_{t-1} within each document (the j < t answer up to scale)
        for a, b in om.doc_bounds(cu_seqlens, qq.shape[0]):
            out[a + 1:b] = out[a:b - 1].copy()
        return out, lse
    _patch(monkeypatch, "attention", bad)
    assert _any_attention_pin_fails()


def _probs_with(score):
    """attention_probs rebuilt around a planted score function (scale and mask as before)."""
    def bad(q, kv, k_rope, N, scale, causal=True, cu_seqlens=None, h=0):
        q, kv, k_rope = om.widen(q), om.widen(kv), om.widen(k_rope)
        T = q.shape[0]
        Pm = np.zeros((T, T))
        for a, b in om.doc_bounds(cu_seqlens, T):
            if b == a:
                continue
            s = score(q[a:b, h], kv[a:b, h, :N], k_rope[a:b], N, scale)
            if causal:
                s = np.where(np.tril(np.ones((b - a, b - a), bool)), s, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            Pm[a:b, a:b] = e / e.sum(axis=1, keepdims=True)
        return Pm
    return bad


def _probs_pins_fail():
    pins = [lambda c=c: tn.test_attention_probs_match_torch_softmax_of_expanded_scores(*c) for c in tn.PROBS_CASES]
    pins += [lambda c=c: tn.test_attention_probs_times_values_is_the_attention_output(*c) for c in tn.PROBS_CASES]
    return any(_fails(p) for p in pins)


def test_probs_without_the_scale_are_caught(monkeypatch):
    _patch(monkeypatch, "attention_probs",
           _probs_with(lambda qh, kn, kr, N, scale: qh[:, :N] @ kn.T + qh[:, N:] @ kr.T))
    assert _probs_pins_fail()


def test_probs_without_the_rope_term_are_caught(monkeypatch):
    _patch(monkeypatch, "attention_probs", _probs_with(lambda qh, kn, kr, N, scale: scale * (qh[:, :N] @ kn.T)))
    assert _probs_pins_fail()


def test_probs_as_planted_here_are_otherwise_right(monkeypatch):
    # the rebuilt function with the right score passes every pin, so the two above fail for their mistake
    _patch(monkeypatch, "attention_probs",
           _probs_with(lambda qh, kn, kr, N, scale: scale * (qh[:, :N] @ kn.T + qh[:, N:] @ kr.T)))
    assert not _probs_pins_fail()


def test_widen_as_fp16_is_caught(monkeypatch):
    real = om.widen
    _patch(monkeypatch, "widen", lambda x: np.asarray(x).view(np.float16).astype(np.float64)
           if np.asarray(x).dtype == np.uint16 else real(x))
    assert _fails(tn.test_widen_matches_torch_bfloat16_for_every_bit_pattern)


def test_widen_shifted_by_15_is_caught(monkeypatch):
    real = om.widen
    _patch(monkeypatch, "widen", lambda x: (np.asarray(x).astype(np.uint32) << 15).view(np.float32).astype(np.float64)
           if np.asarray(x).dtype == np.uint16 else real(x))
    assert _fails(tn.test_widen_matches_torch_bfloat16_for_every_bit_pattern)


def test_cross_length_alignment_from_the_first_key_is_caught(monkeypatch):
    # causal mask j <= i counted from the first key (top-left) instead of lining up the last query with the last key
    real = om.attention

    def bad(q, kv, k_rope, N, scale, causal=True, cu_seqlens=None, rows=None, cu_seqlens_k=None):
        qq = om.widen(q)
        if cu_seqlens is None and om.widen(kv).shape[0] != qq.shape[0] and causal:
            n = qq.shape[0]
            return real(q, np.asarray(kv)[:n], np.asarray(k_rope)[:n], N, scale, causal, None, rows)
        return real(q, kv, k_rope, N, scale, causal, cu_seqlens, rows, cu_seqlens_k)
    _patch(monkeypatch, "attention", bad)
    assert _fails(tn.test_a_chunk_of_queries_reproduces_the_full_causal_rows)


def test_value_and_key_swapped_in_projection_is_caught(monkeypatch):
    orig = om.latent_up_proj

    def bad(latent, w_kvb, head_begin, heads, N, V):
        kv = orig(latent, w_kvb, head_begin, heads, N, V)
        return np.concatenate([kv[..., V:], kv[..., :V]], axis=-1) if N == V else kv[..., ::-1].copy()
    _patch(monkeypatch, "latent_up_proj", bad)
    pins = [tn.test_up_proj_brute_force_tiny_config, tn.test_up_proj_one_hot_latent_returns_weight_rows,
            tn.test_up_proj_matches_torch_linear_layout]
    assert any(_fails(p) for p in pins)


def test_transposed_head_blocks_in_projection_is_caught(monkeypatch):
    # columns read as [j][head] instead of [head][j]
    def bad(latent, w_kvb, head_begin, heads, N, V):
        c, W = om.widen(latent), om.widen(w_kvb)
        P = N + V
        Ht = W.shape[1] // P
        Wt = W.reshape(W.shape[0], P, Ht).transpose(0, 2, 1).reshape(W.shape[0], -1)
        return (c @ Wt[:, head_begin * P:(head_begin + heads) * P]).reshape(c.shape[0], heads, P)
    _patch(monkeypatch, "latent_up_proj", bad)
    pins = [tn.test_up_proj_brute_force_tiny_config, tn.test_up_proj_one_hot_latent_returns_weight_rows,
            tn.test_up_proj_matches_torch_linear_layout]
    assert any(_fails(p) for p in pins)


def test_remainder_to_last_ranks_is_caught(monkeypatch):
    def bad(q_heads, kv_heads, sp):
        g = q_heads // kv_heads
        base, extra = divmod(kv_heads, sp)
        return [(base + (1 if r >= sp - extra else 0)) * g for r in range(sp)]
    _patch(monkeypatch, "head_shard_rule", bad)
    assert any(_fails(ts.test_shard_lists_printed_on_pages, *c) for c in shard_cases())


def test_query_side_split_is_caught(monkeypatch):
    # splitting the query count instead of following the KV heads gives [3, 3] for Q6/KV3
    def bad(q_heads, kv_heads, sp):
        base, extra = divmod(q_heads, sp)
        return [base + (1 if r < extra else 0) for r in range(sp)]
    _patch(monkeypatch, "head_shard_rule", bad)
    assert any(_fails(ts.test_shard_lists_printed_on_pages, *c) for c in shard_cases())


def test_missing_guard_is_caught(monkeypatch):
    _patch(monkeypatch, "head_shard_sizes", lambda q, kv, sp: om.head_shard_rule(q, kv, sp))
    assert any(_fails(ts.test_shard_lists_printed_on_pages, *c) for c in shard_cases())


def test_pack_token_major_slabs_is_caught(monkeypatch):
    # interleaving ranks per token ([T][H][F] unchanged) instead of per-rank slabs
    _patch(monkeypatch, "pack_heads", lambda x, sizes: np.ascontiguousarray(x).reshape(-1))
    assert _fails(ts.test_pack_index_coded_brute_force, 3, [2, 1], 5)


def test_split_combine_without_rescale_is_caught(monkeypatch):
    orig = om.decode_split_kv

    def bad(q, latent, k_rope, w_kvb, N, V, scale, splits, seqs=None):
        out, (m, l, o) = orig(q, latent, k_rope, w_kvb, N, V, scale, splits, seqs)
        out = (l[..., None] * o).sum(axis=2) / l.sum(axis=2)[..., None]   # forgets e^(m_c - m)
        return out, (m, l, o)
    _patch(monkeypatch, "decode_split_kv", bad)
    assert _fails(tn.test_split_kv_equals_direct_softmax, 3)


# ---- query partition, exchange ranges and the expanded pack

import test_oracle_partition as tp  # noqa: E402


def _partition_pins_fail():
    pins = [lambda: tp.test_causal_partition_matches_brute_force(s) for s in range(4)]
    pins.append(tp.test_causal_partition_packed_workload)
    return any(_fails(p) for p in pins)


def test_partition_counting_keys_from_the_query_start_is_caught(monkeypatch):
    # keys counted from the first owned query instead of the document start
    real = om.causal_partition

    def bad(ends, query_length, query_rank, batch=1):
        out = real(ends, query_length, query_rank, batch)
        out["key_ends"] = list(out["query_ends"])
        return out
    _patch(monkeypatch, "causal_partition", bad)
    assert _partition_pins_fail()


def test_exchange_receiving_against_the_peer_range_is_caught(monkeypatch):
    # receives measured against the peer's key range instead of this rank's
    real = om.kv_exchange_ranges

    def bad(ends, source_length, query_length, head_copies, degree, rank):
        sends, _, local = real(ends, source_length, query_length, head_copies, degree, rank)
        return sends, tuple(c for _, c in sends), local
    _patch(monkeypatch, "kv_exchange_ranges", bad)
    assert any(_fails(lambda: tp.test_kv_exchange_ranges_match_brute_force_and_pair_up(s)) for s in range(6))


def test_expanded_pack_with_rope_before_nope_is_caught(monkeypatch):
    def bad(q, kv, k_rope, N, sizes):
        T, H, _ = q.shape
        R = k_rope.shape[1]
        key = np.concatenate([np.broadcast_to(k_rope[:, None, :], (T, H, R)), kv[:, :, :N]], axis=2)
        return om.pack_heads(np.concatenate([q, key, kv[:, :, N:]], axis=2), sizes)
    _patch(monkeypatch, "pack_expanded", bad)
    assert _fails(tp.test_pack_expanded_index_loops) and _fails(tp.test_pack_expanded_key_band_is_the_attention_key)


def test_rope_with_a_flipped_rotation_is_caught(monkeypatch):
    def bad(x, cos, sin, interleaved=False):
        x = om.widen(x)
        c, sn = om.widen(cos), om.widen(sin)
        R = c.shape[1]
        h = R // 2
        shape = (c.shape[0],) + (1,) * (x.ndim - 2) + (R,)
        c, sn = c.reshape(shape), sn.reshape(shape)
        a, b = (x[..., 0::2], x[..., 1::2]) if interleaved else (x[..., :h], x[..., h:])
        return np.concatenate([a * c[..., :h] + b * sn[..., :h], b * c[..., :h] - a * sn[..., :h]], axis=-1)
    _patch(monkeypatch, "rope", bad)
    assert _fails(lambda: tp.test_rope_is_complex_multiplication(False))
    assert _fails(lambda: tp.test_rope_is_complex_multiplication(True))


# ---- backward

import test_oracle_backward as tb  # noqa: E402


def _backward_pins_fail():
    pins = [lambda: tb.test_attention_backward_matches_autograd(True, None),
            tb.test_attention_backward_matches_finite_differences,
            tb.test_shard_backward_chain_matches_autograd]
    return any(_fails(p) for p in pins)


def _backward_with(mutate):
    real = om.attention_backward

    def bad(q, kv, k_rope, dout, N, scale, causal=True, cu_seqlens=None):
        return mutate(real, q, kv, k_rope, dout, N, scale, causal, cu_seqlens)
    return bad


def test_backward_without_the_row_term_is_caught(monkeypatch):
    # ds = p * dp, the softmax Jacobian's row term D = sum_j p dp forgotten
    def bad(q, kv, k_rope, dout, N, scale, causal=True, cu_seqlens=None):
        q, kv, k_rope, dout = (om.widen(x) for x in (q, kv, k_rope, dout))
        T, H, _ = q.shape
        dq, dkv, dkr = np.zeros_like(q), np.zeros_like(kv), np.zeros_like(k_rope)
        for a, b in om.doc_bounds(cu_seqlens, T):
            for h in range(H):
                s = om._scores(q, kv, k_rope, h, slice(a, b), slice(a, b), N, scale)
                if causal:
                    s = np.where(np.tril(np.ones((b - a, b - a), bool)), s, -np.inf)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                p = e / e.sum(axis=1, keepdims=True)
                ds = p * (dout[a:b, h] @ kv[a:b, h, N:].T)
                k = np.concatenate([kv[a:b, h, :N], k_rope[a:b]], axis=1)
                dq[a:b, h] = scale * ds @ k
                dk = scale * ds.T @ q[a:b, h]
                dkv[a:b, h, :N], dkv[a:b, h, N:] = dk[:, :N], p.T @ dout[a:b, h]
                dkr[a:b] += dk[:, N:]
        return dq, dkv, dkr
    _patch(monkeypatch, "attention_backward", bad)
    assert _backward_pins_fail()


def test_backward_shared_band_from_one_head_is_caught(monkeypatch):
    def mutate(real, q, kv, k_rope, dout, N, scale, causal, cu):
        dq, dkv, _ = real(q, kv, k_rope, dout, N, scale, causal, cu)
        one = real(q[:, :1], kv[:, :1], k_rope, dout[:, :1], N, scale, causal, cu)[2]
        return dq, dkv, one
    _patch(monkeypatch, "attention_backward", _backward_with(mutate))
    assert _backward_pins_fail() or _fails(tb.test_shared_band_gradient_is_the_sum_over_heads)
