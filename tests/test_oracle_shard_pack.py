"""Pins for the oracle's head shard lists and token<->head pack (CPU only)."""
import itertools

import numpy as np
import pytest

import oracle
from golden_io import exchange_shape_cases, head_id_cases, shard_cases


@pytest.mark.parametrize("q,kv,sp,exp,src", shard_cases())
def test_shard_lists_printed_on_pages(q, kv, sp, exp, src):
    if exp is None:
        with pytest.raises(ValueError):
            oracle.head_shard_sizes(q, kv, sp)
    else:
        assert oracle.head_shard_sizes(q, kv, sp) == exp, src


@pytest.mark.parametrize("q,kv,sp,exp,src", shard_cases("workload_shards.txt"))
def test_shard_lists_of_workloads(q, kv, sp, exp, src):
    assert oracle.head_shard_sizes(q, kv, sp) == exp, src


@pytest.mark.parametrize("q,kv,sp,exp,src", shard_cases("shard_rule_unguarded.txt"))
def test_unguarded_rule_reproduces_the_broken_split(q, kv, sp, exp, src):
    # the guard rejects it, the bare rule reproduces the page's broken output
    assert oracle.head_shard_rule(q, kv, sp) == exp, src
    with pytest.raises(ValueError):
        oracle.head_shard_sizes(q, kv, sp)


@pytest.mark.parametrize("q,kv,sp,ids,src", head_id_cases())
def test_contiguous_head_ids(q, kv, sp, ids, src):
    sizes = oracle.head_shard_sizes(q, kv, sp)
    got = [list(range(o, o + s)) for o, s in zip(oracle.head_offsets(sizes), sizes)]
    assert got == ids, src


def test_shard_list_invariants_brute_force():
    # every valid (q, kv, sp): sums to q, each rank a whole number of KV groups,
    # sizes differ by at most one group, larger shards first, and each query
    # head's KV head (h // group) lives on the same rank as the query head.
    for kv in range(1, 17):
        for g in range(1, 5):
            q = kv * g
            for sp in range(1, kv + 1):
                s = oracle.head_shard_sizes(q, kv, sp)
                assert sum(s) == q and len(s) == sp
                assert all(x % g == 0 and x > 0 for x in s)
                assert max(s) - min(s) <= g and s == sorted(s, reverse=True)
                kv_sizes = oracle.head_shard_sizes(kv, kv, sp)
                offs, kv_offs = oracle.head_offsets(s), oracle.head_offsets(kv_sizes)
                for r in range(sp):
                    for h in range(offs[r], offs[r] + s[r]):
                        assert kv_offs[r] <= h // g < kv_offs[r] + kv_sizes[r]


def test_shard_list_rejections():
    for bad in [(0, 1, 1), (4, 4, 0), (6, 4, 2), (2, 1, 2), (8, 3, 4), (4, 0, 1)]:
        with pytest.raises(ValueError):
            oracle.head_shard_sizes(*bad)


def _pack_brute(x, sizes):
    """Pure-Python index loops of the send layout (independent of NumPy slicing)."""
    T, H, F = x.shape
    flat = x.reshape(-1).tolist()
    out = []
    off = 0
    for q in sizes:
        for t in range(T):
            for hp in range(q):
                for f in range(F):
                    out.append(flat[(t * H + off + hp) * F + f])
        off += q
    return out


@pytest.mark.parametrize("T,sizes,F", [(3, [2, 1], 5), (4, [3, 3, 3, 3], 2), (5, [4, 2], 3),
                                       (1, [1], 1), (2, [2, 2, 1, 1, 1], 4)])
def test_pack_index_coded_brute_force(T, sizes, F):
    H = sum(sizes)
    x = np.arange(T * H * F, dtype=np.uint32).reshape(T, H, F)   # value = source index
    send = oracle.pack_heads(x, sizes)
    assert send.tolist() == _pack_brute(x, sizes)
    # bijection: every source index appears exactly once
    assert sorted(send.tolist()) == list(range(T * H * F))
    back = oracle.unpack_heads(send, sizes, T, F)
    assert np.array_equal(back, x)


def test_pack_matches_transpose_for_even_split():
    # even split: the send buffer is x viewed as [T][sp][q][F] transposed to [sp][T][q][F]
    rng = np.random.default_rng(7)
    T, sp, q, F = 6, 4, 3, 5
    x = rng.integers(0, 65535, size=(T, sp * q, F), dtype=np.uint16)
    ref = x.reshape(T, sp, q, F).transpose(1, 0, 2, 3).reshape(-1)
    assert np.array_equal(oracle.pack_heads(x, [q] * sp), ref)


@pytest.mark.parametrize("heads,sp,batch,tokens,dim,shapes,src", exchange_shape_cases())
def test_exchange_shapes_printed_on_page(heads, sp, batch, tokens, dim, shapes, src):
    # every rank packs its local [tokens][heads][dim] block; rank r receives slice r
    # of every peer in rank order, i.e. [sp*tokens][q_r][dim] (batch 1 in front)
    sizes = oracle.head_shard_sizes(heads, heads, sp)
    offs = oracle.head_offsets(sizes)
    blocks = [np.arange(tokens * heads * dim, dtype=np.uint32).reshape(tokens, heads, dim) + 1000 * s
              for s in range(sp)]
    sends = [oracle.pack_heads(b, sizes) for b in blocks]
    for r in range(sp):
        base, n = tokens * offs[r] * dim, tokens * sizes[r] * dim
        recv = np.concatenate([s[base:base + n].reshape(tokens, sizes[r], dim) for s in sends])
        assert (batch,) + recv.shape == shapes[r], src
        # and the received rows are the right heads of the right tokens
        for s in range(sp):
            assert np.array_equal(recv[s * tokens:(s + 1) * tokens],
                                  blocks[s][:, offs[r]:offs[r] + sizes[r], :])


def test_unpack_is_inverse_on_random_bits():
    rng = np.random.default_rng(11)
    for sizes in ([22, 22, 21, 21, 21, 21], [3, 1], [5]):
        x = rng.integers(0, 65535, size=(7, sum(sizes), 9), dtype=np.uint16)
        assert np.array_equal(oracle.unpack_heads(oracle.pack_heads(x, sizes), sizes, 7, 9), x)
        # pack of unpack is the identity on the send buffer as well
        s = oracle.pack_heads(x, sizes)
        assert np.array_equal(oracle.pack_heads(oracle.unpack_heads(s, sizes, 7, 9), sizes), s)


def test_pack_every_small_split_brute_force():
    for H in range(1, 6):
        for sp in range(1, H + 1):
            sizes = oracle.head_shard_sizes(H, H, sp)
            for T, F in itertools.product([1, 3], [1, 2]):
                x = np.arange(T * H * F, dtype=np.uint32).reshape(T, H, F)
                assert oracle.pack_heads(x, sizes).tolist() == _pack_brute(x, sizes)
