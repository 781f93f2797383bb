"""Pins for the oracle's expanded pack, query partition and KV exchange ranges (CPU only).

The partition and exchange ranges are checked against brute force over token
sets (which keys each owned query may see, document-local and causal), and the
exchange ranges also against the consistency of every rank pair (what rank r
sends to p is what p expects from r). The expanded pack is checked against
index loops on index-coded payloads and against the attention definition.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _docs(rng, total, n):
    cuts = np.sort(rng.choice(np.arange(1, total), size=n - 1, replace=False)) if n > 1 else np.array([], int)
    return [int(x) for x in cuts] + [total]


def _doc_of(ends, t):
    for d, e in enumerate(ends):
        if t < e:
            return d
    raise AssertionError


def _brute_partition(ends, Lq, r, batch):
    starts = [0] + list(ends[:-1])
    q0, q1 = r * Lq, (r + 1) * Lq
    if ends[-1] < q1:
        return None
    keys, per_doc_q, per_doc_k = set(), {}, {}
    for t in range(q0, q1):
        d = _doc_of(ends, t)
        visible = set(range(starts[d], t + 1))          # document-local, no look-ahead
        keys |= visible
        per_doc_q[d] = per_doc_q.get(d, 0) + 1
        per_doc_k[d] = max(per_doc_k.get(d, 0), t + 1 - starts[d])
    kb, ke = min(keys), max(keys) + 1
    assert keys == set(range(kb, ke)), "selected prefixes are adjacent"
    ds = sorted(per_doc_q)
    qe = list(np.cumsum([per_doc_q[d] for d in ds]))
    kend = list(np.cumsum([per_doc_k[d] for d in ds]))
    nq, nk = sum(per_doc_q.values()), sum(per_doc_k.values())
    return {"key_begin": kb, "key_end": ke,
            "query_ends": [int(x) + i * nq for i in range(batch) for x in qe],
            "key_ends": [int(x) + i * nk for i in range(batch) for x in kend]}


@pytest.mark.parametrize("seed", range(12))
def test_causal_partition_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    degree = int(rng.integers(1, 6))
    Lq = int(rng.integers(1, 40))
    total = degree * Lq
    ends = _docs(rng, total, int(rng.integers(1, min(total, 7) + 1)))
    batch = int(rng.integers(1, 4))
    for r in range(degree):
        got = oracle.causal_partition(ends, Lq, r, batch)
        exp = _brute_partition(ends, Lq, r, batch)
        for k in exp:
            assert got[k] == exp[k], (k, ends, Lq, r)
        assert got["documents"] == tuple(ends)


def test_causal_partition_packed_workload():
    # the 8192/4096/2048/2048 packed documents over four query ranks of 4096
    ends = [8192, 12288, 14336, 16384]
    parts = [oracle.causal_partition(ends, 4096, r) for r in range(4)]
    assert [(p["key_begin"], p["key_end"]) for p in parts] == [(0, 4096), (0, 8192), (8192, 12288), (12288, 16384)]
    assert parts[1]["query_ends"] == [4096] and parts[1]["key_ends"] == [8192]
    assert parts[3]["query_ends"] == [2048, 4096] and parts[3]["key_ends"] == [2048, 4096]


def test_causal_partition_rejects_uncovered_queries():
    with pytest.raises(ValueError):
        oracle.causal_partition([10, 20], 8, 2)          # queries [16, 24) but documents end at 20


def _brute_exchange(ends, S, Lq, copies, degree, rank):
    dest = [_brute_partition(ends, Lq, p // copies, 1) for p in range(degree)]
    src = lambda p: set(range(p * S, (p + 1) * S))
    sends, receives = [], []
    for p in range(degree):
        need = set(range(dest[p]["key_begin"], dest[p]["key_end"])) & src(rank)
        if need:
            lo = min(need)
            assert need == set(range(lo, max(need) + 1))
            sends.append((lo - rank * S, len(need)))
        else:
            sends.append((0, 0))
        receives.append(len(set(range(dest[rank]["key_begin"], dest[rank]["key_end"])) & src(p)))
    local = all(set(range(d["key_begin"], d["key_end"])) <= src(p) for p, d in enumerate(dest))
    return tuple(sends), tuple(receives), local


@pytest.mark.parametrize("seed", range(12))
def test_kv_exchange_ranges_match_brute_force_and_pair_up(seed):
    rng = np.random.default_rng(200 + seed)
    copies = int(rng.integers(1, 4))
    qparts = int(rng.integers(1, 5))
    degree = copies * qparts
    Lq = int(rng.integers(1, 30))
    total = qparts * Lq
    S = total // degree if total % degree == 0 else None
    if S is None or S == 0:
        Lq = degree * int(rng.integers(1, 6))
        total = qparts * Lq
        S = total // degree
    ends = _docs(rng, total, int(rng.integers(1, min(total, 6) + 1)))
    table = [oracle.kv_exchange_ranges(tuple(ends), S, Lq, copies, degree, r) for r in range(degree)]
    for r in range(degree):
        assert table[r] == _brute_exchange(ends, S, Lq, copies, degree, r), (ends, S, Lq, copies, degree, r)
        for p in range(degree):
            assert table[r][0][p][1] == table[p][1][r], "what r sends to p is what p receives from r"


def test_kv_exchange_ranges_local_only_for_one_document_per_rank():
    # every rank's queries are a whole document: nothing moves
    S = 16
    ends = [S * (r + 1) for r in range(4)]
    sends, receives, local = oracle.kv_exchange_ranges(tuple(ends), S, S, 1, 4, 2)
    assert local and sends[2] == (0, S) and receives == (0, 0, S, 0)


def test_pack_expanded_index_loops():
    T, H, N, R, V = 3, 5, 4, 2, 3
    K = N + R
    sizes = [2, 2, 1]
    rng = np.random.default_rng(7)
    q = rng.integers(0, 1 << 30, size=(T, H, K)).astype(np.uint32)
    kv = rng.integers(0, 1 << 30, size=(T, H, N + V)).astype(np.uint32)
    kr = rng.integers(0, 1 << 30, size=(T, R)).astype(np.uint32)
    got = oracle.pack_expanded(q, kv, kr, N, sizes)
    W = 2 * K + V
    exp = np.zeros(T * H * W, np.uint32)
    i = 0
    off = 0
    for qr in sizes:
        for t in range(T):
            for hh in range(qr):
                h = off + hh
                row = list(q[t, h]) + list(kv[t, h, :N]) + list(kr[t]) + list(kv[t, h, N:])
                for f in range(W):
                    exp[i] = row[f]
                    i += 1
        off += qr
    assert np.array_equal(got, exp)


def test_pack_expanded_key_band_is_the_attention_key():
    # attention over the expanded payload's (q, k, v) equals the shared-band attention
    T, H, N, R, V = 9, 3, 4, 2, 5
    rng = np.random.default_rng(11)
    q, kv, kr = rng.standard_normal((T, H, N + R)), rng.standard_normal((T, H, N + V)), rng.standard_normal((T, R))
    send = oracle.pack_expanded(q, kv, kr, N, [H]).reshape(T, H, 2 * (N + R) + V)
    qe, ke, ve = send[..., :N + R], send[..., N + R:2 * (N + R)], send[..., 2 * (N + R):]
    scale = 1 / math.sqrt(N + R)
    sdpa = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qe).transpose(0, 1), torch.from_numpy(ke).transpose(0, 1),
        torch.from_numpy(ve).transpose(0, 1), is_causal=True, scale=scale).transpose(0, 1).numpy()
    ref, _ = oracle.attention(q, kv, kr, N, scale)
    assert np.max(np.abs(sdpa - ref)) < 1e-12


# ---- rotary embedding

def _tables(T, R, base=10000.0, offset=0):
    inv = base ** (-np.arange(0, R, 2) / R)
    ang = np.outer(np.arange(offset, offset + T), inv)          # [T][R/2]
    ang = np.concatenate([ang, ang], axis=1)                     # half-band table layout
    return np.cos(ang), np.sin(ang), ang[:, :R // 2]


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_is_complex_multiplication(interleaved):
    T, H, R = 7, 3, 16
    rng = np.random.default_rng(21)
    x = rng.standard_normal((T, H, R))
    c, s, ang = _tables(T, R)
    got = oracle.rope(x, c, s, interleaved)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) if interleaved else (x[..., :R // 2] + 1j * x[..., R // 2:])
    w = z * np.exp(1j * ang)[:, None, :]
    assert np.max(np.abs(got - np.concatenate([w.real, w.imag], axis=-1))) < 1e-12


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_scores_depend_on_relative_position_only(interleaved):
    R = 32
    rng = np.random.default_rng(22)
    q, k = rng.standard_normal((1, R)), rng.standard_normal((1, R))
    dots = []
    for shift in (0, 5, 1000):
        cq, sq, _ = _tables(1, R, offset=37 + shift)
        ck, sk, _ = _tables(1, R, offset=11 + shift)
        dots.append((oracle.rope(q, cq, sq, interleaved) @ oracle.rope(k, ck, sk, interleaved).T).item())
    assert max(dots) - min(dots) < 1e-9


def test_rope_at_position_zero():
    R = 8
    x = np.arange(3 * R, dtype=np.float64).reshape(3, R)
    c, s = np.ones((3, R)), np.zeros((3, R))
    assert np.array_equal(oracle.rope(x, c, s, False), x)
    assert np.array_equal(oracle.rope(x, c, s, True), np.concatenate([x[:, 0::2], x[:, 1::2]], axis=1))


def test_rope_interleaved_is_half_band_of_deinterleaved_input():
    T, R = 5, 12
    rng = np.random.default_rng(23)
    x = rng.standard_normal((T, 2, R))
    c, s, _ = _tables(T, R)
    de = np.concatenate([x[..., 0::2], x[..., 1::2]], axis=-1)
    assert np.max(np.abs(oracle.rope(x, c, s, True) - oracle.rope(de, c, s, False))) < 1e-15
