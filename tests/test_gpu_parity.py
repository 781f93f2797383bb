"""GPU parity: every C-ABI call against the fp64 oracle on the same seeded inputs.

Permutations (pack/unpack) must match bit for bit. bf16 outputs must satisfy
max|diff| <= 2e-2 and relative L2 <= 1e-2; the fp32 tiny workload 1e-5.
Workloads: tiny fp32, the DeepSeek-V3-shaped rank shard (T=2048, H=16), the
uneven 22-head shard (T=4096), packed documents (T=16384) and latent-cache
decode (32 x 8192), plus ragged sizes that leave partial tiles.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from gpu_helpers import bits, check_close, dev, host64

pytestmark = pytest.mark.gpu

mla = pytest.importorskip("mla_attention_under_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load_library()
    yield
    torch.cuda.synchronize()


def _sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------------- pack / unpack

PACK_CASES = [
    # (name, tokens, sizes, feat, elem_bytes)
    ("tiny_fp32", 64, [3, 1], 56, 4),
    ("dsv3_rank_pack", 256, [16] * 8, 448, 2),
    ("dsv3_rank_out_restore", 256, [16] * 8, 128, 2),
    ("uneven22_pack", 4096, [22, 22, 21, 21, 21, 21], 448, 2),
    ("ragged_2byte_rows", 7, [5, 3, 2], 9, 2),
    ("ragged_4byte_rows", 3, [2, 1], 6, 2),
    ("ragged_8byte_rows", 5, [3], 4, 2),
    ("one_token_one_head", 1, [1], 8, 2),
    ("gqa_q6_kv3", 33, [4, 2], 448, 2),
]


@pytest.mark.parametrize("name,tokens,sizes,feat,eb", PACK_CASES, ids=[c[0] for c in PACK_CASES])
def test_pack_unpack_bit_exact(name, tokens, sizes, feat, eb):
    Ht = sum(sizes)
    x = mi.pack_payload(tokens, Ht, feat, cfg=7, elem_bytes=eb)
    tdt = torch.int16 if eb == 2 else torch.int32
    npdt = np.int16 if eb == 2 else np.int32
    xd = torch.from_numpy(x.view(npdt)).cuda()
    send = torch.empty(x.size, dtype=tdt, device="cuda")
    send.fill_(-1)
    mla.mla_pack_heads(xd, send, sizes)
    back = torch.empty_like(xd)
    back.fill_(-1)
    mla.mla_unpack_heads(send, back, sizes)
    _sync()
    ref = oracle.pack_heads(x, sizes)
    assert np.array_equal(bits(send), ref), name
    assert np.array_equal(bits(back), x), name


EXP_CASES = [
    # (name, tokens, sizes, N, R, V, elem_bytes)
    ("dsv3_rank_expanded", 256, [16] * 8, 128, 64, 128, 2),
    ("uneven22_expanded", 4096, [22, 22, 21, 21, 21, 21], 128, 64, 128, 2),
    ("tiny_fp32_expanded", 64, [3, 1], 16, 8, 16, 4),
    ("ragged_2byte_widths", 7, [2, 3], 5, 3, 7, 2),
    ("ragged_4byte_widths", 5, [1, 2], 2, 2, 4, 2),
    ("one_token_one_head", 1, [1], 8, 8, 8, 2),
]


@pytest.mark.parametrize("name,tokens,sizes,N,R,V,eb", EXP_CASES, ids=[c[0] for c in EXP_CASES])
def test_pack_expanded_bit_exact(name, tokens, sizes, N, R, V, eb):
    Ht = sum(sizes)
    rng = np.random.default_rng(17)
    npdt = np.uint16 if eb == 2 else np.uint32
    tdt = torch.int16 if eb == 2 else torch.int32
    sdt = np.int16 if eb == 2 else np.int32
    q = rng.integers(0, 1 << (8 * eb), size=(tokens, Ht, N + R), dtype=np.uint64).astype(npdt)
    kv = rng.integers(0, 1 << (8 * eb), size=(tokens, Ht, N + V), dtype=np.uint64).astype(npdt)
    kr = rng.integers(0, 1 << (8 * eb), size=(tokens, R), dtype=np.uint64).astype(npdt)
    to = lambda a: torch.from_numpy(a.view(sdt)).cuda()
    send = torch.empty(tokens * Ht * (2 * (N + R) + V), dtype=tdt, device="cuda")
    mla.mla_pack_expanded(to(q), to(kv), to(kr), send, sizes, N)
    _sync()
    got = send.cpu().numpy().view(npdt)
    exp = oracle.pack_expanded(q, kv, kr, N, sizes)
    assert np.array_equal(got, exp), name


def _rope_tables(T, R, dtype_bf16, offset=0, base=10000.0):
    """Position tables [T][R] (half-band layout, one angle per pair) in the band's dtype."""
    inv = base ** (-np.arange(0, R, 2) / R)
    ang = np.outer(np.arange(offset, offset + T), inv)
    ang = np.concatenate([ang, ang], axis=1)
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    return (mi.f32_to_bf16_bits(c), mi.f32_to_bf16_bits(s)) if dtype_bf16 else (c, s)


ROPE_CASES = [
    # (name, T, H, N, R, bf16)
    ("dsv3_rank_q", 2048, 16, 128, 64, True),
    ("pack_side_q_all_heads", 4096, 128, 128, 64, True),
    ("shared_key_band", 2048, 0, 0, 64, True),
    ("tiny_fp32_q", 64, 4, 16, 8, False),
    ("odd_band_bf16", 37, 3, 6, 10, True),
    ("one_token", 1, 1, 128, 64, True),
]


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("name,T,H,N,R,bf16", ROPE_CASES, ids=[c[0] for c in ROPE_CASES])
def test_rope_matches_oracle(name, T, H, N, R, bf16, interleaved):
    shape = (T, R) if H == 0 else (T, H, N + R)
    x = mi.draw(shape, 31, 1, bf16=bf16)
    c, s = _rope_tables(T, R, bf16, offset=17)
    xd, cd, sd = dev(x), dev(c), dev(s)
    band = xd if H == 0 else xd[..., N:]
    mla.mla_apply_rope(band, cd, sd, interleaved=interleaved)
    _sync()
    got = host64(xd)
    ref_band = oracle.rope(x if H == 0 else x[..., N:], c, s, interleaved)
    check_close(got if H == 0 else got[..., N:], ref_band, bf16=bf16, name=f"{name} interleaved={interleaved}")
    if H:
        assert np.array_equal(bits(xd)[..., :N], x[..., :N].view(bits(xd).dtype)), "columns outside the band changed"


PROJ_CASES = [
    # (name, T, L, w_heads, head_begin, heads, P, F, col_offset, sizes, rope_offset, R)
    ("q_part_rank_shard", 256, 1536, 128, 0, 128, 192, 448, 0, [16] * 8, 128, 64),
    ("kv_part_rank_shard", 256, 512, 128, 0, 128, 256, 448, 192, [16] * 8, -1, 0),
    ("q_part_uneven_ragged", 300, 1536, 128, 0, 128, 192, 448, 0, [22, 22, 21, 21, 21, 21], 128, 64),
    ("q_part_head_range", 37, 512, 32, 8, 12, 192, 448, 0, [5, 4, 3], 128, 64),
    ("band_second_group", 70, 256, 4, 0, 4, 128, 200, 72, [2, 2], 64, 64),
    ("band_every_group", 45, 256, 6, 1, 4, 64, 64, 0, [3, 1], 0, 64),
]


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("name,T,L,w_heads,hb,heads,P,F,col,sizes,ro,R", PROJ_CASES, ids=[c[0] for c in PROJ_CASES])
def test_project_pack_matches_oracle_and_separate_calls(name, T, L, w_heads, hb, heads, P, F, col, sizes, ro, R, interleaved):
    if R == 0 and interleaved:
        pytest.skip("no band")
    lat = dev(mi.draw((T, L), 41, 0))
    W = dev(mi.draw((L, w_heads * P), 41, 1, std=L ** -0.5))
    fill = dev(mi.draw((T, heads, F), 41, 2))
    cos = sin = None
    if R:
        c, s = _rope_tables(T, R, True, offset=512)
        cos, sin = dev(c), dev(s)
    # separate calls: projection, rotation of the band, pack of the payload with that part in place
    part = torch.empty((T, heads, P), dtype=torch.bfloat16, device="cuda")
    mla.mla_latent_up_proj(lat, W, part, w_heads, hb, heads, P // 2, P - P // 2)   # any split of the P columns
    if R:
        mla.mla_apply_rope(part[..., ro:ro + R], cos, sin, interleaved=interleaved)
    x = fill.clone()
    x[..., col:col + P] = part
    ref = torch.empty(x.numel(), dtype=torch.bfloat16, device="cuda")
    mla.mla_pack_heads(x, ref, sizes)
    # fused: the pack of the fill, then the projection written into its columns
    send = torch.empty_like(ref)
    mla.mla_pack_heads(fill, send, sizes)
    mla.mla_project_pack(lat, W, send, w_heads, hb, heads, P, F, col, sizes, rope_offset=ro, cos=cos, sin=sin,
                         interleaved=interleaved)
    _sync()
    # against the oracle: the fp64 projection, the band rotated, packed into the head slabs
    part64 = oracle.latent_up_proj(bits(lat), bits(W), hb, heads, P // 2, P - P // 2)
    if R:
        part64[..., ro:ro + R] = oracle.rope(part64[..., ro:ro + R], c, s, interleaved)
    x64 = oracle.widen(bits(fill))
    x64[..., col:col + P] = part64
    check_close(oracle.widen(bits(send)), oracle.pack_heads(x64, sizes), name=f"{name} vs oracle")
    # outside the band, bit for bit the separate calls (the projection rounds once in both); the band is
    # rotated in fp32 before its one rounding, the separate calls round the projection first
    got_rows = oracle.unpack_heads(bits(send), sizes, T, F)
    ref_rows = oracle.unpack_heads(bits(ref), sizes, T, F)
    keep = np.ones(F, bool)
    if R:
        keep[col + ro:col + ro + R] = False
    assert np.array_equal(got_rows[..., keep], ref_rows[..., keep]), name


def test_pack_zero_tokens_is_a_no_op():
    x = torch.zeros((0, 4, 8), dtype=torch.int16, device="cuda")
    send = torch.zeros(0, dtype=torch.int16, device="cuda")
    mla.mla_pack_heads(x, send, [2, 2])
    _sync()


def test_pack_shard_list_from_the_library():
    sizes = mla.mla_head_shard_sizes(6, 3, 2)          # GQA: [4, 2]
    x = mi.pack_payload(9, 6, 12, cfg=8)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    send = torch.empty(x.size, dtype=torch.int16, device="cuda")
    mla.mla_pack_heads(xd, send, sizes)
    _sync()
    assert np.array_equal(bits(send), oracle.pack_heads(x, oracle.head_shard_sizes(6, 3, 2)))


# ------------------------------------------------------------------------- up-projection

def _up_proj_case(w, T, head_begin, heads, seed_cfg=None):
    d = mi.shard_inputs(w, T=T, seed_cfg=seed_cfg)
    lat, W = dev(d["latent"]), dev(d["w_kvb"])
    out = torch.empty((T, heads, w.P), dtype=lat.dtype, device="cuda")
    mla.mla_latent_up_proj(lat, W, out, w.heads_total, head_begin, heads, w.N, w.V)
    _sync()
    ref = oracle.latent_up_proj(d["latent"], d["w_kvb"], head_begin, heads, w.N, w.V)
    return host64(out), ref


@pytest.mark.parametrize("wname,T,hb,heads", [
    ("tiny", 64, 0, 4), ("tiny", 37, 1, 2),
    ("dsv3_rank", 2048, 0, 16),
    ("uneven22", 4096, 0, 22), ("uneven22", 300, 22, 22),
    ("dsv3_rank", 1, 3, 2), ("dsv3_rank", 129, 0, 16), ("dsv3_rank", 1000, 5, 3),
])
def test_up_proj_matches_oracle(wname, T, hb, heads):
    w = mi.WORKLOADS[wname]
    got, ref = _up_proj_case(w, T, hb, heads)
    check_close(got, ref, bf16=w.bf16, name=f"{wname} T={T} heads[{hb},{hb + heads})")


def test_up_proj_as_the_query_projection():
    # q_b_proj of the DeepSeek-V3 rank shard: latent width 1536 -> 16 heads of [q_nope 128 | q_rope 64]
    w = mi.Workload("q_proj", 12, T=2048, H=16, L=1536, N=128, R=64, V=64, heads_total=16)
    got, ref = _up_proj_case(w, 2048, 0, 16)
    check_close(got, ref, name="query projection L=1536, 16 x 192")


def test_up_proj_generic_widths():
    # N+V = 64: the column count is not a multiple of the 128-wide tile
    w = mi.Workload("odd", 11, T=200, H=3, L=40, N=40, R=8, V=24, heads_total=5)
    got, ref = _up_proj_case(w, 200, 1, 3)
    check_close(got, ref, name="N=40 V=24 L=40")


@pytest.mark.parametrize("wname,T,hb,heads", [
    ("tiny", 37, 1, 2), ("dsv3_rank", 2048, 0, 16), ("uneven22", 300, 22, 22),
    ("dsv3_rank", 129, 0, 16), ("dsv3_rank", 1000, 5, 3), ("odd", 200, 1, 3),
])
def test_up_proj_linear_layout(wname, T, hb, heads):
    # the weight as torch.nn.Linear stores it ([heads_total*(N+V)][L]): the oracle's product, and the same bits as
    # the [L][heads_total*(N+V)] entry point on the same values
    w = (mi.Workload("odd", 11, T=200, H=3, L=40, N=40, R=8, V=24, heads_total=5) if wname == "odd"
         else mi.WORKLOADS[wname])
    d = mi.shard_inputs(w, T=T)
    lat, W = dev(d["latent"]), dev(d["w_kvb"])
    W_lin = dev(np.ascontiguousarray(d["w_kvb"].T))
    out = torch.empty((T, heads, w.P), dtype=lat.dtype, device="cuda")
    out_rm = torch.empty_like(out)
    mla.mla_latent_up_proj_linear(lat, W_lin, out, w.heads_total, hb, heads, w.N, w.V)
    mla.mla_latent_up_proj(lat, W, out_rm, w.heads_total, hb, heads, w.N, w.V)
    _sync()
    ref = oracle.latent_up_proj(d["latent"], d["w_kvb"], hb, heads, w.N, w.V)
    check_close(host64(out), ref, bf16=w.bf16, name=f"nn.Linear weight, {wname} T={T} heads[{hb},{hb + heads})")
    assert torch.equal(out.view(torch.int16) if w.bf16 else out, out_rm.view(torch.int16) if w.bf16 else out_rm)


# ------------------------------------------------------------------------- attention

def _attn_inputs(w, T, seed_cfg=None, kv_direct=True):
    """q, k_rope and kv as bf16 bits (kv drawn directly, isolating the attention kernel)."""
    d = mi.shard_inputs(w, T=T, seed_cfg=seed_cfg)
    if kv_direct:
        d["kv"] = mi.draw((T, w.H, w.P), w.cfg if seed_cfg is None else seed_cfg, 9, bf16=w.bf16)
    return d


def _run_attn(w, d, T, causal=True, cu=None, want_lse=False):
    q, kv, kr = dev(d["q"]), dev(d["kv"]), dev(d["k_rope"])
    out = torch.full((T, w.H, w.V), float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((w.H, T), float("nan"), dtype=torch.float32, device="cuda") if want_lse else None
    cud = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    mla.mla_attention_fwd(q, kv, kr, out, w.N, w.R, w.V, 1 / math.sqrt(w.K), causal=causal, lse=lse, cu_seqlens=cud)
    _sync()
    return host64(out), (None if lse is None else lse.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("T", [64, 1, 37])
def test_attention_tiny_fp32(T):
    w = mi.WORKLOADS["tiny"]
    d = _attn_inputs(w, T)
    got, lse = _run_attn(w, d, T, want_lse=True)
    ref, rlse = oracle.attention(d["q"], d["kv"], d["k_rope"], w.N, 1 / math.sqrt(w.K))
    check_close(got, ref, bf16=False, name=f"tiny T={T}")
    check_close(lse, rlse, bf16=False, name=f"tiny lse T={T}")


@pytest.mark.parametrize("T,H", [(2048, 16), (1, 2), (63, 2), (192, 2), (200, 3), (1000, 2), (2112, 3), (4097, 1)])
def test_attention_dense_causal(T, H):
    w = mi.WORKLOADS["dsv3_rank"]
    w = mi.Workload(w.name, w.cfg, T=T, H=H, L=w.L, N=w.N, R=w.R, V=w.V, heads_total=H)
    d = _attn_inputs(w, T)
    got, lse = _run_attn(w, d, T, want_lse=True)
    ref, rlse = oracle.attention(d["q"], d["kv"], d["k_rope"], w.N, 1 / math.sqrt(w.K))
    check_close(got, ref, name=f"dense T={T} H={H}")
    check_close(lse, rlse, name=f"lse T={T} H={H}")


def test_attention_non_causal():
    w = mi.WORKLOADS["dsv3_rank"]
    w = mi.Workload(w.name, w.cfg, T=333, H=2, L=w.L, N=w.N, R=w.R, V=w.V, heads_total=2)
    d = _attn_inputs(w, 333)
    got, _ = _run_attn(w, d, 333, causal=False)
    ref, _ = oracle.attention(d["q"], d["kv"], d["k_rope"], w.N, 1 / math.sqrt(w.K), causal=False)
    check_close(got, ref, name="non-causal T=333")


def test_attention_composed_with_up_projection_dsv3():
    """Rank shard end to end: GPU up-projection feeds the GPU attention (T=2048, H=16)."""
    w = mi.WORKLOADS["dsv3_rank"]
    d = mi.shard_inputs(w)
    lat, W, q, kr = dev(d["latent"]), dev(d["w_kvb"]), dev(d["q"]), dev(d["k_rope"])
    kv = torch.empty((w.T, w.H, w.P), dtype=torch.bfloat16, device="cuda")
    mla.mla_latent_up_proj(lat, W, kv, w.heads_total, 0, w.H, w.N, w.V)
    out = torch.empty((w.T, w.H, w.V), dtype=torch.bfloat16, device="cuda")
    mla.mla_attention_fwd(q, kv, kr, out, w.N, w.R, w.V, 1 / math.sqrt(w.K))
    _sync()
    kv_ref = oracle.latent_up_proj(d["latent"], d["w_kvb"], 0, w.H, w.N, w.V)
    ref, _ = oracle.attention(d["q"], kv_ref, d["k_rope"], w.N, 1 / math.sqrt(w.K))
    check_close(host64(out), ref, name="dsv3 composed")


def test_attention_uneven22_sampled_rows():
    """22 heads at T=4096 with the weight's head range [0, 22) of 128; sampled query rows."""
    w = mi.WORKLOADS["uneven22"]
    d = mi.shard_inputs(w)
    lat, W, q, kr = dev(d["latent"]), dev(d["w_kvb"]), dev(d["q"]), dev(d["k_rope"])
    kv = torch.empty((w.T, w.H, w.P), dtype=torch.bfloat16, device="cuda")
    mla.mla_latent_up_proj(lat, W, kv, w.heads_total, 0, w.H, w.N, w.V)
    out = torch.empty((w.T, w.H, w.V), dtype=torch.bfloat16, device="cuda")
    mla.mla_attention_fwd(q, kv, kr, out, w.N, w.R, w.V, 1 / math.sqrt(w.K))
    _sync()
    # the first and last row of every 128-row query tile (each dense causal tile pair, split tile
    # included), plus random rows
    tiles = np.arange(0, w.T, 128)
    rows = np.unique(np.concatenate([tiles, tiles + 127, [1, 2047], np.random.default_rng(3).integers(0, 4096, 40)]))
    kv_ref = oracle.latent_up_proj(d["latent"], d["w_kvb"], 0, w.H, w.N, w.V)
    ref, _ = oracle.attention(d["q"], kv_ref, d["k_rope"], w.N, 1 / math.sqrt(w.K), rows=rows)
    check_close(host64(out)[rows], ref[rows], name="uneven22 sampled")


@pytest.mark.parametrize("cu", [
    [0, 100, 101, 101, 400, 531],          # empty and one-token documents, ragged tiles
    [0, 128, 256, 640],
    [0, 1, 2, 3],
])
def test_attention_varlen_small(cu):
    T = cu[-1]
    w = mi.WORKLOADS["varlen16k"]
    w = mi.Workload(w.name, w.cfg, T=T, H=2, L=w.L, N=w.N, R=w.R, V=w.V, heads_total=2)
    d = _attn_inputs(w, T)
    got, lse = _run_attn(w, d, T, cu=cu, want_lse=True)
    ref, rlse = oracle.attention(d["q"], d["kv"], d["k_rope"], w.N, 1 / math.sqrt(w.K), cu_seqlens=cu)
    check_close(got, ref, name=f"varlen {cu}")
    check_close(lse, rlse, name=f"varlen lse {cu}")


def test_attention_varlen16k_sampled_rows():
    w = mi.WORKLOADS["varlen16k"]
    cu = [int(x) for x in w.cu_seqlens]
    d = _attn_inputs(w, w.T)
    got, _ = _run_attn(w, d, w.T, cu=cu)
    rng = np.random.default_rng(4)
    # the first and last row of every 128-row query tile of every document (each schedule
    # entry), the document ends, plus random rows
    tile_rows = [r for a, b in zip(cu, cu[1:]) for t0 in range(a, b, 128) for r in (t0, min(t0 + 127, b - 1))]
    rows = np.unique(np.concatenate([np.array(tile_rows), np.array(cu[1:]) - 1, rng.integers(0, w.T, 48)]))
    ref, _ = oracle.attention(d["q"], d["kv"], d["k_rope"], w.N, 1 / math.sqrt(w.K), cu_seqlens=cu, rows=rows)
    check_close(got[rows], ref[rows], name="varlen16k sampled")
    # a document's first token returns its own value row
    for a in cu[:-1]:
        np.testing.assert_allclose(got[a], oracle.widen(d["kv"])[a, :, w.N:], atol=1e-2, rtol=0)


def _unpacked(w, d, T, sp, causal=True, cu=None, noalloc=False):
    """The attention written straight into the token-major [T/sp][sp*H][V] layout (unpack_sp), and the same call
    into [T][H][V] followed by mla_unpack_heads, both into NaN-filled buffers."""
    q, kv, kr = dev(d["q"]), dev(d["kv"]), dev(d["k_rope"])
    cud = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    scale = 1 / math.sqrt(w.K)
    fwd = mla.mla_attention_fwd_noalloc if noalloc else mla.mla_attention_fwd
    y = torch.full((T // sp, sp * w.H, w.V), float("nan"), dtype=q.dtype, device="cuda")
    lse_y = torch.full((w.H, T), float("nan"), dtype=torch.float32, device="cuda")
    fwd(q, kv, kr, y, w.N, w.R, w.V, scale, causal=causal, lse=lse_y, cu_seqlens=cud, unpack_sp=sp)
    out = torch.full((T, w.H, w.V), float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((w.H, T), float("nan"), dtype=torch.float32, device="cuda")
    fwd(q, kv, kr, out, w.N, w.R, w.V, scale, causal=causal, lse=lse, cu_seqlens=cud)
    y2 = torch.full_like(y, float("nan"))
    mla.mla_unpack_heads(out.reshape(-1), y2, [w.H] * sp)
    _sync()
    return y, y2, out, lse_y, lse


@pytest.mark.parametrize("T,H,sp,causal", [(384, 2, 3, True), (200, 3, 5, True), (256, 2, 4, False)])
def test_attention_unpacked_output_against_oracle(T, H, sp, causal):
    """Output chunks of T/sp queries land in rank r's head columns; chunks of 40 queries cut 128-query tiles."""
    w = mi.WORKLOADS["dsv3_rank"]
    w = mi.Workload(w.name, w.cfg, T=T, H=H, L=w.L, N=w.N, R=w.R, V=w.V, heads_total=H)
    d = _attn_inputs(w, T)
    y, _, _, lse_y, _ = _unpacked(w, d, T, sp, causal=causal)
    ref, rlse = oracle.attention(d["q"], d["kv"], d["k_rope"], w.N, 1 / math.sqrt(w.K), causal=causal)
    ref_y = oracle.unpack_heads(ref.reshape(-1), [H] * sp, T // sp, w.V)
    check_close(host64(y), ref_y, name=f"unpacked T={T} H={H} sp={sp}")
    check_close(lse_y.cpu().numpy().astype(np.float64), rlse, name=f"unpacked lse T={T}")


@pytest.mark.parametrize("case", ["dsv3_causal", "dsv3_noncausal", "documents", "noalloc", "tiny_fp32", "uneven22"])
def test_attention_unpacked_output_equals_unpack_call(case):
    """The fused layout is the separate unpack of the same call, bit for bit (rank shard: T=2048, H=16, sp=8;
    the uneven shard: T=4096, H=22, chunks of 512)."""
    if case == "tiny_fp32":
        w, T, sp = mi.WORKLOADS["tiny"], 64, 4
    elif case == "uneven22":
        w, T, sp = mi.WORKLOADS["uneven22"], 4096, 8
    else:
        w, T, sp = mi.WORKLOADS["dsv3_rank"], 2048, 8
    d = _attn_inputs(w, T)
    cu = [0, 300, 301, 1100, 2048] if case == "documents" else None
    y, y2, out, lse_y, lse = _unpacked(w, d, T, sp, causal=case != "dsv3_noncausal", cu=cu,
                                       noalloc=case == "noalloc")
    assert torch.isfinite(out).all()
    assert np.array_equal(bits(y), bits(y2)), case
    assert np.array_equal(bits(lse_y), bits(lse)), case
    if case == "dsv3_causal":   # the launch the step times, against the oracle directly
        ref, _ = oracle.attention(d["q"], d["kv"], d["k_rope"], w.N, 1 / math.sqrt(w.K))
        check_close(host64(y), oracle.unpack_heads(ref.reshape(-1), [w.H] * sp, T // sp, w.V), name="dsv3 unpacked")


def test_attention_reads_packed_rows_in_place():
    """torchtitan 'Ulysses CP' order on one rank: every simulated rank projects its own
    tokens for all heads and packs [q | kv] rows by the shard list; rank r's slab of
    every peer forms its receive buffer, which the attention reads in place."""
    Htot, sp, Tl = 16, 4, 96
    base = mi.WORKLOADS["dsv3_rank"]
    w = mi.Workload("pipe", 12, T=sp * Tl, H=Htot, L=base.L, N=base.N, R=base.R, V=base.V, heads_total=Htot)
    d = mi.shard_inputs(w)
    sizes = mla.mla_head_shard_sizes(Htot, Htot, sp)
    offs = oracle.head_offsets(sizes)
    lat, W, q, kr = dev(d["latent"]), dev(d["w_kvb"]), dev(d["q"]), dev(d["k_rope"])
    sends = []
    for s in range(sp):
        kv_s = torch.empty((Tl, Htot, w.P), dtype=torch.bfloat16, device="cuda")
        mla.mla_latent_up_proj(lat[s * Tl:(s + 1) * Tl].contiguous(), W, kv_s, Htot, 0, Htot, w.N, w.V)
        rows = torch.cat([q[s * Tl:(s + 1) * Tl], kv_s], dim=2).contiguous()       # [Tl][Htot][F]
        send = torch.empty(rows.numel(), dtype=torch.bfloat16, device="cuda")
        mla.mla_pack_heads(rows, send, sizes)
        sends.append(send)
    refs = oracle.ulysses_materialise_k_first(d["latent"], d["w_kvb"], d["q"], d["k_rope"], sizes, w.N, w.V,
                                               1 / math.sqrt(w.K))
    for r in range(sp):
        n = Tl * sizes[r] * w.F
        recv = torch.cat([snd[Tl * offs[r] * w.F:Tl * offs[r] * w.F + n] for snd in sends]).view(sp * Tl, sizes[r], w.F)
        out = torch.empty((sp * Tl, sizes[r], w.V), dtype=torch.bfloat16, device="cuda")
        mla.mla_attention_fwd(recv[:, :, :w.K], recv[:, :, w.K:], kr, out, w.N, w.R, w.V, 1 / math.sqrt(w.K))
        _sync()
        check_close(host64(out), refs[r], name=f"packed rank {r}")
    # and the latent-first order gives the same answer on the GPU as well
    latent_first = oracle.ulysses_latent_first(d["latent"], d["w_kvb"], d["q"], d["k_rope"], sizes, w.N, w.V,
                                               1 / math.sqrt(w.K))
    for r in range(sp):
        kv = torch.empty((w.T, sizes[r], w.P), dtype=torch.bfloat16, device="cuda")
        mla.mla_latent_up_proj(lat, W, kv, Htot, offs[r], sizes[r], w.N, w.V)
        out = torch.empty((w.T, sizes[r], w.V), dtype=torch.bfloat16, device="cuda")
        mla.mla_attention_fwd(q[:, offs[r]:offs[r] + sizes[r]], kv, kr, out, w.N, w.R, w.V, 1 / math.sqrt(w.K))
        _sync()
        check_close(host64(out), latent_first[r], name=f"latent-first rank {r}")


def test_attention_is_deterministic():
    w = mi.WORKLOADS["dsv3_rank"]
    d = _attn_inputs(w, 1024)
    q, kv, kr = dev(d["q"][:1024]), dev(d["kv"]), dev(d["k_rope"][:1024])
    outs = []
    for _ in range(2):
        o = torch.empty((1024, w.H, w.V), dtype=torch.bfloat16, device="cuda")
        mla.mla_attention_fwd(q, kv, kr, o, w.N, w.R, w.V, 1 / math.sqrt(w.K))
        outs.append(bits(o))
    assert np.array_equal(outs[0], outs[1])


# ------------------------------------------------------------------------- decode

def _decode_case(w, B, S, splits, seqs):
    d = mi.decode_inputs(w, batch=B, kv_len=S)
    q, c, kr, W = dev(d["q"]), dev(d["latent"]), dev(d["k_rope"]), dev(d["w_kvb"])
    out = torch.full((B, w.H, w.V), float("nan"), dtype=torch.bfloat16, device="cuda")
    mla.mla_latent_decode_fwd(q, c, kr, W, out, w.heads_total, 0, w.N, w.R, w.V, splits, 1 / math.sqrt(w.K))
    _sync()
    ref, _ = oracle.decode_split_kv(d["q"], d["latent"], d["k_rope"], d["w_kvb"], w.N, w.V, 1 / math.sqrt(w.K),
                                    splits, seqs=seqs)
    return host64(out), ref


@pytest.mark.parametrize("B,S,splits", [(3, 1000, 8), (2, 64, 1), (1, 130, 3), (2, 9, 4), (2, 333, 2)])
def test_decode_small(B, S, splits):
    w = mi.WORKLOADS["decode32"]
    got, ref = _decode_case(w, B, S, splits, seqs=range(B))
    check_close(got, ref, name=f"decode B={B} S={S} splits={splits}")


def test_decode_head_subset():
    """Five heads starting at head 3 of a 16-head weight: the rank's column block."""
    w = dataclasses.replace(mi.WORKLOADS["decode32"], H=5)
    B, S, splits, hb = 3, 300, 2, 3
    d = mi.decode_inputs(w, batch=B, kv_len=S)
    q, c, kr, W = dev(d["q"]), dev(d["latent"]), dev(d["k_rope"]), dev(d["w_kvb"])
    out = torch.full((B, w.H, w.V), float("nan"), dtype=torch.bfloat16, device="cuda")
    mla.mla_latent_decode_fwd(q, c, kr, W, out, w.heads_total, hb, w.N, w.R, w.V, splits, 1 / math.sqrt(w.K))
    _sync()
    w_cols = d["w_kvb"][:, hb * w.P:(hb + w.H) * w.P]
    ref, _ = oracle.decode_split_kv(d["q"], d["latent"], d["k_rope"], w_cols, w.N, w.V, 1 / math.sqrt(w.K), splits)
    check_close(host64(out), ref, name="decode head subset")


def test_decode32_sampled_sequences():
    w = mi.WORKLOADS["decode32"]
    seqs = [0, 17, 31]
    got, ref = _decode_case(w, w.batch, w.kv_len, w.kv_splits, seqs=seqs)
    check_close(got[seqs], ref[seqs], name="decode32 sampled")
    assert np.all(np.isfinite(got))


def test_dense_causal_workspace_reuse_across_shapes():
    """The dense causal path splits paired query tiles between workgroups through a
    reusable workspace; calls of different shapes in a row must each be exact."""
    base = mi.WORKLOADS["dsv3_rank"]
    rng = np.random.default_rng(5)
    for T, H in [(2048, 16), (4097, 1), (200, 3), (1000, 2), (2048, 16), (640, 5)]:
        w = mi.Workload(base.name, base.cfg, T=T, H=H, L=base.L, N=base.N, R=base.R, V=base.V, heads_total=H)
        d = _attn_inputs(w, T, seed_cfg=T + H)
        got, lse = _run_attn(w, d, T, want_lse=True)
        rows = np.unique(np.concatenate([[0, T - 1, T // 2], rng.integers(0, T, 24)]))
        ref, rlse = oracle.attention(d["q"], d["kv"], d["k_rope"], w.N, 1 / math.sqrt(w.K), rows=rows)
        check_close(got[rows], ref[rows], name=f"reuse T={T} H={H}")
        check_close(lse[:, rows], rlse[:, rows], name=f"reuse lse T={T} H={H}")


def test_dense_causal_arbitrary_workspace():
    """The workspace needs no clearing: split-tile flags left by other calls, or
    arbitrary bytes, must not be taken for this call's arrivals."""
    base = mi.WORKLOADS["dsv3_rank"]
    T, H = 2048, 16
    w = mi.Workload(base.name, base.cfg, T=T, H=H, L=base.L, N=base.N, R=base.R, V=base.V, heads_total=H)
    d = _attn_inputs(w, T)
    q, kv, kr = dev(d["q"]), dev(d["kv"]), dev(d["k_rope"])
    out = torch.empty((T, H, w.V), dtype=torch.bfloat16, device="cuda")
    scale = 1 / math.sqrt(w.K)
    nbytes = mla.mla_attention_workspace_size(q, kv, kr, out, w.N, w.R, w.V, scale)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ref, _ = oracle.attention(d["q"], d["kv"], d["k_rope"], w.N, scale)
    for fill in ("random", "ones", "zeros"):
        if fill == "random":
            ws.copy_(torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda"))
        else:
            ws.fill_(255 if fill == "ones" else 0)
        out.fill_(float("nan"))
        mla.mla_attention_fwd(q, kv, kr, out, w.N, w.R, w.V, scale, workspace=ws)
        _sync()
        check_close(host64(out), ref, name=f"workspace {fill}")


def test_dense_causal_graph_replays():
    """A captured dense causal call gives the eager result on every replay, with
    eager attention calls (fresh tags, the same workspace on another stream)
    between the replays."""
    base = mi.WORKLOADS["dsv3_rank"]
    T, H = 2048, 16
    w = mi.Workload(base.name, base.cfg, T=T, H=H, L=base.L, N=base.N, R=base.R, V=base.V, heads_total=H)
    d = _attn_inputs(w, T)
    q, kv, kr = dev(d["q"]), dev(d["kv"]), dev(d["k_rope"])
    scale = 1 / math.sqrt(w.K)
    eager = torch.empty((T, H, w.V), dtype=torch.bfloat16, device="cuda")
    mla.mla_attention_fwd(q, kv, kr, eager, w.N, w.R, w.V, scale)   # also allocates the cached workspace
    _sync()
    out = torch.full((T, H, w.V), float("nan"), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mla.mla_attention_fwd(q, kv, kr, out, w.N, w.R, w.V, scale)
    for i in range(3):
        out.fill_(float("nan"))
        g.replay()
        _sync()
        assert torch.equal(out, eager), f"replay {i} differs from the eager call"
        mla.mla_attention_fwd(q, kv, kr, eager, w.N, w.R, w.V, scale)   # eager work between replays
        _sync()


def test_unpacked_output_graph_replays():
    """A captured call writing the restored layout gives the eager result on every replay."""
    base = mi.WORKLOADS["dsv3_rank"]
    T, H, sp = 2048, 16, 8
    w = mi.Workload(base.name, base.cfg, T=T, H=H, L=base.L, N=base.N, R=base.R, V=base.V, heads_total=H)
    d = _attn_inputs(w, T)
    q, kv, kr = dev(d["q"]), dev(d["kv"]), dev(d["k_rope"])
    scale = 1 / math.sqrt(w.K)
    eager = torch.empty((T // sp, sp * H, w.V), dtype=torch.bfloat16, device="cuda")
    mla.mla_attention_fwd(q, kv, kr, eager, w.N, w.R, w.V, scale, unpack_sp=sp)
    _sync()
    y = torch.full_like(eager, float("nan"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mla.mla_attention_fwd(q, kv, kr, y, w.N, w.R, w.V, scale, unpack_sp=sp)
    for i in range(3):
        y.fill_(float("nan"))
        g.replay()
        _sync()
        assert torch.equal(y, eager), f"replay {i} differs from the eager call"
        mla.mla_attention_fwd(q, kv, kr, eager, w.N, w.R, w.V, scale, unpack_sp=sp)
        _sync()


def test_attention_dominant_keys():
    """A few keys outscore all others by far more than the fp32 exp2 range (score
    gaps of ~200 in log2 units), in both halves of the key sub-tiles: the row max
    must cover every key of a tile or the weights overflow."""
    base = mi.WORKLOADS["dsv3_rank"]
    T, H = 300, 2
    w = mi.Workload(base.name, base.cfg, T=T, H=H, L=base.L, N=base.N, R=base.R, V=base.V, heads_total=H)
    d = _attn_inputs(w, T, seed_cfg=77)
    q = mi.bf16_bits_to_f32(d["q"]).copy()
    kv = mi.bf16_bits_to_f32(d["kv"]).copy()
    q[:, :, : w.N] += 4.0
    hot = [5, 70, 133, 250, 252]        # offsets 5, 6, 5 (upper lanes) and 2, 4 within 8-key groups
    kv[hot, :, : w.N] = 4.0
    d["q"], d["kv"] = mi.f32_to_bf16_bits(q), mi.f32_to_bf16_bits(kv)
    got, lse = _run_attn(w, d, T, want_lse=True)
    ref, rlse = oracle.attention(d["q"], d["kv"], d["k_rope"], w.N, 1 / math.sqrt(w.K))
    assert np.isfinite(got).all() and np.isfinite(lse).all()
    check_close(got, ref, name="dominant keys")
    check_close(lse, rlse, name="dominant keys lse")


def test_dense_causal_graph_replays_back_to_back_with_new_inputs():
    """One captured dense causal call (T=2048, H=16) replayed three times in a row.
    The split-tile flags keep the capture's tag on every replay; new seeded q, kv
    and k_rope are copied into the captured buffers before each replay, with no
    other attention call in between, and every replay is checked against the
    oracle element by element (a stale partial softmax record from the previous
    replay would be merged into a split tile)."""
    base = mi.WORKLOADS["dsv3_rank"]
    T, H = 2048, 16
    w = mi.Workload(base.name, base.cfg, T=T, H=H, L=base.L, N=base.N, R=base.R, V=base.V, heads_total=H)
    scale = 1 / math.sqrt(w.K)
    d0 = _attn_inputs(w, T, seed_cfg=100)
    q, kv, kr = dev(d0["q"]), dev(d0["kv"]), dev(d0["k_rope"])
    out = torch.full((T, H, w.V), float("nan"), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mla.mla_attention_fwd(q, kv, kr, out, w.N, w.R, w.V, scale)
    _sync()
    for i in range(3):
        d = _attn_inputs(w, T, seed_cfg=101 + i)
        q.copy_(dev(d["q"]))
        kv.copy_(dev(d["kv"]))
        kr.copy_(dev(d["k_rope"]))
        out.fill_(float("nan"))
        g.replay()
        _sync()
        ref, _ = oracle.attention(d["q"], d["kv"], d["k_rope"], w.N, scale)
        check_close(host64(out), ref, name=f"back-to-back replay {i}")


# ------------------------------------------------------------------------- separate query and key lengths

def _cross_inputs(T_q, T_k, H, seed):
    base = mi.WORKLOADS["dsv3_rank"]
    wq = mi.Workload(base.name, base.cfg, T=T_q, H=H, L=base.L, N=base.N, R=base.R, V=base.V, heads_total=H)
    wk = mi.Workload(base.name, base.cfg, T=max(T_k, 1), H=H, L=base.L, N=base.N, R=base.R, V=base.V, heads_total=H)
    q = mi.shard_inputs(wq, T=T_q, seed_cfg=seed)["q"]
    dk = mi.shard_inputs(wk, T=max(T_k, 1), seed_cfg=seed + 1)
    kv = mi.draw((max(T_k, 1), H, wk.P), seed + 1, 9)[:T_k]
    return wq, q, kv, dk["k_rope"][:T_k]


def _run_cross(w, q, kv, kr, causal, cu=None, cu_k=None):
    T_q = q.shape[0]
    qd, kvd, krd = dev(q), dev(kv), dev(kr)
    out = torch.full((T_q, w.H, w.V), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.H, T_q), float("nan"), dtype=torch.float32, device="cuda")
    cud = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    cukd = None if cu_k is None else torch.tensor(cu_k, dtype=torch.int32, device="cuda")
    mla.mla_attention_fwd(qd, kvd, krd, out, w.N, w.R, w.V, 1 / math.sqrt(w.K), causal=causal, lse=lse,
                          cu_seqlens=cud, cu_seqlens_k=cukd)
    _sync()
    return host64(out), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("T_q,T_k,H,causal", [
    (512, 2048, 3, True),      # a chunk at the end of the sequence, key shift a multiple of 64
    (100, 1000, 2, True),      # shift 900: partial key tiles
    (2048, 4096, 16, True),    # the rank shard's queries over twice the keys (paired query tiles, split tiles)
    (77, 333, 2, False),
    (200, 70, 2, True),        # more queries than keys: the first 130 rows see nothing
    (1, 2048, 4, True),
])
def test_attention_query_chunk_over_longer_keys(T_q, T_k, H, causal):
    w, q, kv, kr = _cross_inputs(T_q, T_k, H, 400 + T_q + T_k)
    got, lse = _run_cross(w, q, kv, kr, causal)
    tiles = np.arange(0, T_q, 128)
    rows = np.unique(np.concatenate([tiles, np.minimum(tiles + 127, T_q - 1), [T_q - 1],
                                     np.random.default_rng(T_q).integers(0, T_q, 24)]))
    ref, rlse = oracle.attention(q, kv, kr, w.N, 1 / math.sqrt(w.K), causal=causal, rows=rows)
    check_close(got[rows], ref[rows], name=f"chunk T_q={T_q} T_k={T_k}")
    seen = np.isfinite(rlse[:, rows])
    assert np.array_equal(np.isfinite(lse[:, rows]), seen), "rows with no visible key must give lse -inf"
    check_close(lse[:, rows][seen], rlse[:, rows][seen], name=f"chunk lse T_q={T_q} T_k={T_k}")
    if T_q > T_k and causal:
        assert np.all(got[:T_q - T_k] == 0), "queries that see no key give zero rows"


def test_attention_with_no_keys():
    w, q, kv, kr = _cross_inputs(40, 0, 2, 450)
    got, lse = _run_cross(w, q, kv, kr, True)
    assert np.all(got == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("causal", [True, False])
def test_attention_documents_with_their_own_key_offsets(causal):
    cu = [0, 3, 4, 132, 200, 200, 457]
    cu_k = [0, 700, 701, 829, 1000, 1064, 1100]      # a chunk over its prefix, one query, equal, short, keys only, ...
    w, q, kv, kr = _cross_inputs(cu[-1], cu_k[-1], 2, 460)
    got, lse = _run_cross(w, q, kv, kr, causal, cu=cu, cu_k=cu_k)
    ref, rlse = oracle.attention(q, kv, kr, w.N, 1 / math.sqrt(w.K), causal=causal, cu_seqlens=cu, cu_seqlens_k=cu_k)
    check_close(got, ref, name=f"documents with key offsets causal={causal}")
    seen = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(lse), seen)
    check_close(lse[seen], rlse[seen], name="documents with key offsets lse")


def test_attention_one_query_per_sequence_over_its_cache():
    """Decode shape through the general call: 4 sequences, one query each, over caches of 1000..1500 keys."""
    cu = [0, 1, 2, 3, 4]
    cu_k = [0, 1000, 1500, 3000, 3100]
    w, q, kv, kr = _cross_inputs(4, 3100, 16, 470)
    got, _ = _run_cross(w, q, kv, kr, True, cu=cu, cu_k=cu_k)
    ref, _ = oracle.attention(q, kv, kr, w.N, 1 / math.sqrt(w.K), causal=True, cu_seqlens=cu, cu_seqlens_k=cu_k)
    check_close(got, ref, name="one query per sequence")
