"""Pins for the oracle's up-projection, attention, path agreement and split-KV decode.

Each pin checks the oracle against something other than itself: a library
routine (torch's scaled_dot_product_attention in float64 on the CPU, with the
shared key band expanded per head), a closed form, an invariant the pages state,
or pure-Python brute force on tiny shapes.
"""
import math

import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _tiny(T=9, H=3, N=4, R=2, V=3, seed=0):
    q = _rand((T, H, N + R), seed)
    kv = _rand((T, H, N + V), seed + 1)
    kr = _rand((T, R), seed + 2)
    return q, kv, kr


# ----------------------------------------------------------------------------- bf16 widening

def test_widen_matches_torch_bfloat16_for_every_bit_pattern():
    """All 65 536 bf16 encodings: the oracle's bit widening against torch's own
    bfloat16 -> float64 conversion (NaN patterns must stay NaN, signed zeros keep
    their sign). Reading the bits as fp16, or shifting by 15, fails here."""
    pat = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen(pat)
    ref = torch.from_numpy(pat.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127                    # exponent all ones, non-zero mantissa, both signs
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # a few values fixed by the format itself: 1.0 = 0x3f80, -2.0 = 0xc000, the largest finite 0x7f7f
    assert oracle.widen(np.array([0x3F80, 0xC000, 0x7F7F, 0x0001], np.uint16)).tolist() == [
        1.0, -2.0, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133]
    # fp32 input widens exactly
    x = np.random.default_rng(1).standard_normal(64).astype(np.float32)
    assert np.array_equal(oracle.widen(x), x.astype(np.float64))


# ----------------------------------------------------------------------------- up-projection

def _proj_brute(c, W, hb, heads, N, V):
    T, L = c.shape
    P = N + V
    out = [[[0.0] * P for _ in range(heads)] for _ in range(T)]
    for t in range(T):
        for h in range(heads):
            for j in range(P):
                acc = 0.0
                for l in range(L):
                    acc += c[t, l] * W[l, (hb + h) * P + j]
                out[t][h][j] = acc
    return np.array(out)


def test_up_proj_brute_force_tiny_config():
    w = mi.WORKLOADS["tiny"]
    d = mi.shard_inputs(w, T=6)
    c, W = d["latent"].astype(np.float64), d["w_kvb"].astype(np.float64)
    got = oracle.latent_up_proj(d["latent"], d["w_kvb"], 1, 2, w.N, w.V)
    np.testing.assert_allclose(got, _proj_brute(c, W, 1, 2, w.N, w.V), rtol=1e-13, atol=1e-13)


def test_up_proj_one_hot_latent_returns_weight_rows():
    # latent row t = e_{l(t)} picks row l(t) of the head's column block: pins orientation
    L, N, V, Ht = 5, 2, 3, 4
    W = _rand((L, Ht * (N + V)), 3)
    ls = [4, 0, 2]
    c = np.zeros((3, L))
    c[np.arange(3), ls] = 1.0
    kv = oracle.latent_up_proj(c, W, 2, 2, N, V)
    for t, l in enumerate(ls):
        np.testing.assert_array_equal(kv[t].reshape(-1), W[l, 2 * (N + V):4 * (N + V)])
    # and k_nope / v are the first N / last V columns of each head block
    np.testing.assert_array_equal(kv[0, 1, :N], W[4, 3 * (N + V):3 * (N + V) + N])
    np.testing.assert_array_equal(kv[0, 1, N:], W[4, 3 * (N + V) + N:4 * (N + V)])


def test_up_proj_head_range_is_a_slice_of_all_heads():
    c, W = _rand((7, 6), 4), _rand((6, 5 * 7), 5)
    full = oracle.latent_up_proj(c, W, 0, 5, 3, 4)
    for hb, n in [(0, 1), (1, 3), (4, 1), (2, 3)]:
        np.testing.assert_array_equal(oracle.latent_up_proj(c, W, hb, n, 3, 4), full[:, hb:hb + n])
    for hb, n in [(-1, 2), (4, 2), (0, 0), (5, 1)]:
        with pytest.raises(ValueError):
            oracle.latent_up_proj(c, W, hb, n, 3, 4)


def test_up_proj_matches_torch_linear_layout():
    # nn.Linear stores the transpose: weight [H*(N+V)][L]; F.linear(c, W.T) is the same map
    c, W = _rand((5, 8), 6), _rand((8, 2 * 6), 7)
    ref = torch.nn.functional.linear(torch.from_numpy(c), torch.from_numpy(W.T.copy())).numpy()
    np.testing.assert_allclose(oracle.latent_up_proj(c, W, 0, 2, 2, 4).reshape(5, -1), ref,
                               rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------- attention

def _sdpa_expanded(q, kv, kr, N, scale, mask=None, causal=True):
    """torch SDPA (float64, CPU) with k = [k_nope | k_rope] expanded to every head."""
    T, H, K = q.shape
    k = np.concatenate([kv[:, :, :N], np.broadcast_to(kr[:, None, :], (T, H, kr.shape[1]))], axis=2)
    Q = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    Kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))
    Vt = torch.from_numpy(np.ascontiguousarray(kv[:, :, N:].transpose(1, 0, 2)))
    if mask is not None:
        o = torch.nn.functional.scaled_dot_product_attention(
            Q, Kt, Vt, attn_mask=torch.from_numpy(mask), scale=scale)
    else:
        o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, is_causal=causal, scale=scale)
    return o.numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("causal", [True, False])
def test_attention_matches_sdpa_with_expanded_key(causal):
    q, kv, kr = _tiny(T=17, H=3, N=8, R=4, V=5, seed=10)
    scale = 1 / math.sqrt(12)
    out, _ = oracle.attention(q, kv, kr, 8, scale, causal=causal)
    np.testing.assert_allclose(out, _sdpa_expanded(q, kv, kr, 8, scale, causal=causal),
                               rtol=1e-12, atol=1e-12)


def test_attention_tiny_config_matches_sdpa():
    w = mi.WORKLOADS["tiny"]
    d = mi.shard_inputs(w)
    kv = oracle.latent_up_proj(d["latent"], d["w_kvb"], 0, w.H, w.N, w.V)
    q, kr = oracle.widen(d["q"]), oracle.widen(d["k_rope"])
    scale = 1 / math.sqrt(w.K)
    out, _ = oracle.attention(q, kv, kr, w.N, scale)
    np.testing.assert_allclose(out, _sdpa_expanded(q, kv, kr, w.N, scale), rtol=1e-12, atol=1e-12)


def test_varlen_matches_sdpa_block_diagonal_mask_and_separate_runs():
    q, kv, kr = _tiny(T=20, H=2, N=4, R=2, V=3, seed=20)
    cu = [0, 7, 8, 8, 15, 20]                     # includes an empty and a 1-token document
    scale = 0.37
    out, lse = oracle.attention(q, kv, kr, 4, scale, cu_seqlens=cu)
    doc = np.repeat(np.arange(len(cu) - 1), np.diff(cu))
    allowed = (doc[:, None] == doc[None, :]) & (np.arange(20)[None, :] <= np.arange(20)[:, None])
    np.testing.assert_allclose(out, _sdpa_expanded(q, kv, kr, 4, scale, mask=allowed),
                               rtol=1e-12, atol=1e-12)
    # packed == each document run on its own, concatenated
    for a, b in zip(cu, cu[1:]):
        if b > a:
            o2, l2 = oracle.attention(q[a:b], kv[a:b], kr[a:b], 4, scale)
            np.testing.assert_array_equal(out[a:b], o2)
            np.testing.assert_array_equal(lse[:, a:b], l2)
    # cumulative ends without the leading zero describe the same documents
    assert oracle.doc_bounds(ends=cu[1:]) == oracle.doc_bounds(cu_seqlens=cu)


def test_probability_rows_sum_to_one_and_respect_the_mask():
    q, kv, kr = _tiny(T=12, H=2, N=4, R=2, V=3, seed=30)
    cu = [0, 5, 12]
    for h in range(2):
        Pm = oracle.attention_probs(q, kv, kr, 4, 0.5, cu_seqlens=cu, h=h)
        assert np.all(np.abs(Pm.sum(axis=1) - 1) <= 1e-12)
        doc = np.repeat([0, 1], [5, 7])
        allowed = (doc[:, None] == doc[None, :]) & (np.arange(12)[None, :] <= np.arange(12)[:, None])
        assert np.all(Pm[~allowed] == 0) and np.all(Pm[allowed] > 0)


def _probs_torch(q, kv, kr, N, scale, allowed, h):
    """torch float64: the key band expanded per head, scaled scores, masked softmax."""
    T, H, _ = q.shape
    k = np.concatenate([kv[:, h, :N], kr], axis=1)                    # [T][N+R], this head's expanded key
    s = scale * (torch.from_numpy(np.ascontiguousarray(q[:, h])) @ torch.from_numpy(k).T)
    s = s.masked_fill(~torch.from_numpy(allowed), float("-inf"))
    p = torch.softmax(s, dim=1)
    return torch.nan_to_num(p, nan=0.0).numpy()                       # rows of empty documents do not exist


PROBS_CASES = [(True, None), (False, None), (True, [0, 5, 6, 6, 12, 15]), (False, [0, 9, 15])]


@pytest.mark.parametrize("causal,cu", PROBS_CASES)
def test_attention_probs_match_torch_softmax_of_expanded_scores(causal, cu):
    """The probability matrix itself, against torch.softmax of scale * q . [k_nope | k_rope]
    with the causal / document mask. A dropped scale or rope term fails here."""
    q, kv, kr = _tiny(T=15, H=3, N=4, R=2, V=3, seed=80)
    q[:, :, 4:] *= 3.0                                 # a strong band, so the rope term is visible
    scale = 0.45
    bounds = [(0, 15)] if cu is None else list(zip(cu, cu[1:]))
    doc = np.zeros(15, int)
    for i, (a, b) in enumerate(bounds):
        doc[a:b] = i
    allowed = doc[:, None] == doc[None, :]
    if causal:
        allowed &= np.arange(15)[None, :] <= np.arange(15)[:, None]
    for h in range(3):
        Pm = oracle.attention_probs(q, kv, kr, 4, scale, causal=causal, cu_seqlens=cu, h=h)
        np.testing.assert_allclose(Pm, _probs_torch(q, kv, kr, 4, scale, allowed, h), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("causal,cu", PROBS_CASES)
def test_attention_probs_times_values_is_the_attention_output(causal, cu):
    q, kv, kr = _tiny(T=15, H=3, N=4, R=2, V=3, seed=81)
    out, _ = oracle.attention(q, kv, kr, 4, 0.6, causal=causal, cu_seqlens=cu)
    for h in range(3):
        Pm = oracle.attention_probs(q, kv, kr, 4, 0.6, causal=causal, cu_seqlens=cu, h=h)
        np.testing.assert_allclose(Pm @ kv[:, h, 4:], out[:, h], rtol=1e-12, atol=1e-13)


# ---- separate query and key lengths (chunked prefill, attention over a projected cache)

def test_a_chunk_of_queries_reproduces_the_full_causal_rows():
    """Queries [c0, c1) of a sequence attending to its keys [0, c1) give exactly the rows [c0, c1) of the full
    causal attention: the last query of the chunk lines up with the last key. Pins the causal alignment for
    T_q != T_k."""
    q, kv, kr = _tiny(T=20, H=2, N=4, R=2, V=3, seed=90)
    full, flse = oracle.attention(q, kv, kr, 4, 0.4)
    for c0, c1 in [(13, 20), (5, 12), (0, 6), (19, 20)]:
        out, lse = oracle.attention(q[c0:c1], kv[:c1], kr[:c1], 4, 0.4)
        np.testing.assert_allclose(out, full[c0:c1], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse, flse[:, c0:c1], rtol=1e-13, atol=1e-14)


def _bottom_right_allowed(qlens, klens, causal=True):
    Tq, Tk = sum(qlens), sum(klens)
    allowed = np.zeros((Tq, Tk), bool)
    qa = ka = 0
    for nq, nk in zip(qlens, klens):
        for i in range(nq):
            for j in range(nk):
                allowed[qa + i, ka + j] = (j <= i + nk - nq) if causal else True
        qa, ka = qa + nq, ka + nk
    return allowed


@pytest.mark.parametrize("causal", [True, False])
def test_cross_length_documents_match_sdpa_with_the_bottom_right_mask(causal):
    qlens, klens = [3, 1, 4, 2], [7, 1, 4, 9]          # a chunk over a prefix, one query, equal, a short chunk
    rng = np.random.default_rng(91)
    q = rng.standard_normal((sum(qlens), 2, 6))
    kv = rng.standard_normal((sum(klens), 2, 7))
    kr = rng.standard_normal((sum(klens), 2))
    cq, ck = np.concatenate([[0], np.cumsum(qlens)]), np.concatenate([[0], np.cumsum(klens)])
    out, _ = oracle.attention(q, kv, kr, 4, 0.3, causal=causal, cu_seqlens=list(cq), cu_seqlens_k=list(ck))
    allowed = _bottom_right_allowed(qlens, klens, causal)
    k = np.concatenate([kv[:, :, :4], np.broadcast_to(kr[:, None, :], (kv.shape[0], 2, 2))], axis=2)
    Q = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    K = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))
    V = torch.from_numpy(np.ascontiguousarray(kv[:, :, 4:].transpose(1, 0, 2)))
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=torch.from_numpy(allowed), scale=0.3)
    np.testing.assert_allclose(out, ref.numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-12)
    # packed == each document on its own
    for d in range(len(qlens)):
        o2, _ = oracle.attention(q[cq[d]:cq[d + 1]], kv[ck[d]:ck[d + 1]], kr[ck[d]:ck[d + 1]], 4, 0.3, causal=causal)
        np.testing.assert_array_equal(out[cq[d]:cq[d + 1]], o2)


def test_queries_that_see_no_key_give_zero_rows():
    # 5 queries over 3 keys, causal: query i sees keys j <= i - 2, so the first two see nothing
    q, kv, kr = _tiny(T=5, H=2, N=4, R=2, V=3, seed=92)
    out, lse = oracle.attention(q, kv[:3], kr[:3], 4, 0.5)
    assert np.all(out[:2] == 0) and np.all(np.isneginf(lse[:, :2]))
    for i in range(2, 5):
        o, l_ = oracle.attention(q[i:i + 1], kv[:i - 1], kr[:i - 1], 4, 0.5, causal=False)
        np.testing.assert_allclose(out[i], o[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[:, i], l_[:, 0], rtol=1e-13, atol=1e-14)


def test_one_query_over_a_cache_is_a_plain_softmax_either_way():
    # a single query per document over its whole cache (decode): the causal bound admits every key
    rng = np.random.default_rng(93)
    q = rng.standard_normal((3, 2, 6))
    kv = rng.standard_normal((30, 2, 7))
    kr = rng.standard_normal((30, 2))
    cq, ck = [0, 1, 2, 3], [0, 10, 22, 30]
    a, _ = oracle.attention(q, kv, kr, 4, 0.25, causal=True, cu_seqlens=cq, cu_seqlens_k=ck)
    b, _ = oracle.attention(q, kv, kr, 4, 0.25, causal=False, cu_seqlens=cq, cu_seqlens_k=ck)
    np.testing.assert_array_equal(a, b)
    for d in range(3):
        s = 0.25 * (kv[ck[d]:ck[d + 1], :, :4].transpose(1, 0, 2) @ q[d, :, :4, None])[..., 0] \
            + 0.25 * (q[d, :, 4:] @ kr[ck[d]:ck[d + 1]].T)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(a[d], np.einsum("hj,jhv->hv", p, kv[ck[d]:ck[d + 1], :, 4:]), rtol=1e-12)


def test_first_token_of_each_document_returns_its_value_row():
    q, kv, kr = _tiny(T=11, H=2, N=4, R=2, V=3, seed=40)
    cu = [0, 4, 11]
    out, lse = oracle.attention(q, kv, kr, 4, 0.3, cu_seqlens=cu)
    for a in cu[:-1]:
        np.testing.assert_array_equal(out[a], kv[a, :, 4:])
        # a single visible key: lse is exactly that key's scaled score
        s = 0.3 * (np.einsum("hd,hd->h", q[a, :, :4], kv[a, :, :4]) + q[a, :, 4:] @ kr[a])
        np.testing.assert_allclose(lse[:, a], s, rtol=1e-14, atol=1e-14)


def test_zero_query_gives_running_mean_of_values():
    # q = 0: every visible key has the same score, so o_t is the mean of v over j <= t
    _, kv, kr = _tiny(T=10, H=2, N=4, R=2, V=3, seed=50)
    q = np.zeros((10, 2, 6))
    out, lse = oracle.attention(q, kv, kr, 4, 1.0)
    v = kv[:, :, 4:]
    ref = np.cumsum(v, axis=0) / np.arange(1, 11)[:, None, None]
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(np.arange(1, 11))[None, :].repeat(2, 0), rtol=1e-14)


def test_zero_rope_band_reduces_to_plain_mha():
    q, kv, kr = _tiny(T=13, H=2, N=6, R=4, V=5, seed=60)
    q[:, :, 6:] = 0.0
    kr[:] = 0.0
    out, _ = oracle.attention(q, kv, kr, 6, 0.41)
    Q = torch.from_numpy(np.ascontiguousarray(q[:, :, :6].transpose(1, 0, 2)))
    K = torch.from_numpy(np.ascontiguousarray(kv[:, :, :6].transpose(1, 0, 2)))
    V = torch.from_numpy(np.ascontiguousarray(kv[:, :, 6:].transpose(1, 0, 2)))
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=0.41)
    np.testing.assert_allclose(out, ref.numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-13)


def test_shared_rope_band_changes_every_head_the_same_way():
    # one band serves every head: with q_nope = 0 and the same q_rope in every head,
    # all heads of a token see the same scores, so their probability rows agree exactly.
    q, kv, kr = _tiny(T=8, H=3, N=4, R=2, V=3, seed=70)
    q[:, :, :4] = 0.0
    q[:, 1:, 4:] = q[:, :1, 4:]
    Pm = [oracle.attention_probs(q, kv, kr, 4, 0.7, h=h) for h in range(3)]
    np.testing.assert_allclose(Pm[1], Pm[0], rtol=0, atol=0)
    np.testing.assert_allclose(Pm[2], Pm[0], rtol=0, atol=0)


def _attn_brute(q, kv, kr, N, scale):
    T, H, _ = q.shape
    V = kv.shape[2] - N
    out = np.zeros((T, H, V))
    for h in range(H):
        for t in range(T):
            s = []
            for j in range(t + 1):
                acc = 0.0
                for d in range(N):
                    acc += q[t, h, d] * kv[j, h, d]
                for d in range(kr.shape[1]):
                    acc += q[t, h, N + d] * kr[j, d]
                s.append(scale * acc)
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for v in range(V):
                out[t, h, v] = sum(e[j] * kv[j, h, N + v] for j in range(t + 1)) / z
    return out


def test_attention_brute_force_tiny():
    q, kv, kr = _tiny(T=7, H=2, N=3, R=2, V=2, seed=80)
    out, _ = oracle.attention(q, kv, kr, 3, 0.6)
    np.testing.assert_allclose(out, _attn_brute(q, kv, kr, 3, 0.6), rtol=1e-12, atol=1e-13)


def test_row_sampling_matches_full_run():
    q, kv, kr = _tiny(T=15, H=2, N=4, R=2, V=3, seed=90)
    full, lf = oracle.attention(q, kv, kr, 4, 0.5, cu_seqlens=[0, 6, 15])
    rows = [0, 5, 6, 14]
    part, lp = oracle.attention(q, kv, kr, 4, 0.5, cu_seqlens=[0, 6, 15], rows=rows)
    np.testing.assert_array_equal(part[rows], full[rows])
    np.testing.assert_array_equal(lp[:, rows], lf[:, rows])
    assert np.isnan(part[1]).all()


# ----------------------------------------------------------------------------- path agreement

@pytest.mark.parametrize("Htot,kvh,sp", [(12, 12, 4), (3, 3, 2), (6, 3, 2), (4, 4, 1)])
def test_latent_first_equals_materialise_k_first(Htot, kvh, sp):
    # torchtitan "MLA CP optimization": compact (latent-first) and materialised
    # paths give the same forward; the same float64 routines give identical values.
    T, L, N, R, V = 8 * sp, 16, 4, 2, 3
    latent, W = _rand((T, L), 1), _rand((L, Htot * (N + V)), 2, L ** -0.5)
    q, kr = _rand((T, Htot, N + R), 3), _rand((T, R), 4)
    sizes = oracle.head_shard_sizes(Htot, kvh, sp)
    a = oracle.ulysses_materialise_k_first(latent, W, q, kr, sizes, N, V, 0.5)
    b = oracle.ulysses_latent_first(latent, W, q, kr, sizes, N, V, 0.5)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-14)


def test_path_agreement_dsv3_scaled_down():
    T, Htot, sp, L, N, R, V = 256, 32, 8, 64, 16, 8, 16
    latent, W = _rand((T, L), 5), _rand((L, Htot * (N + V)), 6, L ** -0.5)
    q, kr = _rand((T, Htot, N + R), 7), _rand((T, R), 8)
    sizes = oracle.head_shard_sizes(Htot, Htot, sp)
    a = oracle.ulysses_materialise_k_first(latent, W, q, kr, sizes, N, V, 1 / math.sqrt(N + R))
    b = oracle.ulysses_latent_first(latent, W, q, kr, sizes, N, V, 1 / math.sqrt(N + R))
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- split-KV decode

@pytest.mark.parametrize("splits", [1, 3, 8])
def test_split_kv_equals_direct_softmax(splits):
    B, S, H, L, N, R, V = 3, 40, 2, 12, 4, 2, 3
    q, c, kr = _rand((B, H, N + R), 1), _rand((B, S, L), 2), _rand((B, S, R), 3)
    W = _rand((L, H * (N + V)), 4, L ** -0.5)
    out, (m, l, o) = oracle.decode_split_kv(q, c, kr, W, N, V, 0.8, splits)
    ref = oracle.decode_reference(q, c, kr, W, N, V, 0.8)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)
    assert m.shape == (B, H, splits) and o.shape == (B, H, splits, V)


def test_decode_single_split_is_the_attention_definition():
    # one query that sees every cached key == non-causal attention with a 1-row query
    B, S, H, L, N, R, V = 2, 9, 2, 6, 3, 2, 2
    q, c, kr = _rand((B, H, N + R), 11), _rand((B, S, L), 12), _rand((B, S, R), 13)
    W = _rand((L, H * (N + V)), 14)
    out, (m, l, o) = oracle.decode_split_kv(q, c, kr, W, N, V, 0.4, 1)
    for b in range(B):
        kv = oracle.latent_up_proj(c[b], W, 0, H, N, V)
        ref = _sdpa_expanded(np.repeat(q[b][None], S, 0), kv, kr[b], N, 0.4, causal=False)
        np.testing.assert_allclose(out[b], ref[0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(o[b, :, 0], out[b], rtol=1e-13, atol=1e-14)


def test_decode_zero_query_is_mean_of_projected_values():
    B, S, H, L, N, R, V = 1, 16, 2, 5, 3, 2, 2
    c, kr, W = _rand((B, S, L), 21), _rand((B, S, R), 22), _rand((L, H * (N + V)), 23)
    out, _ = oracle.decode_split_kv(np.zeros((B, H, N + R)), c, kr, W, N, V, 1.0, 4)
    kv = c[0] @ W
    ref = kv.reshape(S, H, N + V)[:, :, N:].mean(axis=0)
    np.testing.assert_allclose(out[0], ref, rtol=1e-13, atol=1e-14)
