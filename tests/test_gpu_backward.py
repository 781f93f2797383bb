"""GPU parity of mla_attention_bwd against the oracle's attention_backward, and of
mla_latent_up_proj_bwd against latent_up_proj_backward.

Tolerance, derived from the kernel's arithmetic rather than fixed: the inputs
are exact bf16 and every product accumulates in fp32, so the rounding that
matters is p and ds taken to bf16 as MFMA operands (relative 2^-9 each), the
row term D formed from the bf16 forward output, and fp32 accumulation of dp.
With u = 2^-8 (twice the bf16 unit roundoff) and, per head,
  E_s = u |ds| + p (dD + 2^-16 |dout| |v|^T),   dD_t = rel_out * sum_v |dout||out|,
the elementwise bounds are
  |dv err| <= u p^T |dout|,  |dk err| <= scale E_s^T |q|,  |dq err| <= scale E_s |k|,
  |dk_rope err| <= sum over heads of the band part of the dk bound,
and each output must sit within twice its bound (plus 1e-7). A transposed
operand, a dropped row term or a missing head in the band sum breaks it by
orders of magnitude. A norm-wise relative error of at most 1e-2 is also
required. p, ds and the bounds come from the oracle's probabilities in fp64.
"""
import math

import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from gpu_helpers import dev, host64

pytestmark = pytest.mark.gpu

mla = pytest.importorskip("mla_attention_under_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load_library()
    yield
    torch.cuda.synchronize()


W = mi.WORKLOADS["dsv3_rank"]
N, R, V = W.N, W.R, W.V
K = N + R
SCALE = 1 / math.sqrt(K)


def _inputs(T, H, seed):
    cfg = W.cfg * 1000 + seed
    return {
        "q": mi.draw((T, H, K), cfg, 1),
        "kv": mi.draw((T, H, N + V), cfg, 9),
        "k_rope": mi.draw((T, R), cfg, 2),
        "dout": mi.draw((T, H, V), cfg, 21),
    }


def _bounds(d, out, causal, cu, rel_out):
    q, kv, kr = oracle.widen(d["q"]), oracle.widen(d["kv"]), oracle.widen(d["k_rope"])
    do, o = oracle.widen(d["dout"]), np.asarray(out, np.float64)
    T, H, _ = q.shape
    u = 2.0 ** -8
    bq, bkv, bkr = np.zeros((T, H, K)), np.zeros((T, H, N + V)), np.zeros((T, R))
    for h in range(H):
        P = oracle.attention_probs(d["q"], d["kv"], d["k_rope"], N, SCALE, causal, cu, h=h)
        v, g = kv[:, h, N:], do[:, h]
        dP = g @ v.T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dD = rel_out * (np.abs(g) * np.abs(o[:, h])).sum(axis=1)
        Es = u * np.abs(dS) + P * (dD[:, None] + 2.0 ** -16 * (np.abs(g) @ np.abs(v).T))
        k = np.concatenate([kv[:, h, :N], kr], axis=1)
        bkv[:, h, N:] = u * (P.T @ np.abs(g))
        dk = SCALE * (Es.T @ np.abs(q[:, h]))
        bkv[:, h, :N] = dk[:, :N]
        bkr += dk[:, N:]
        bq[:, h] = SCALE * (Es @ np.abs(k))
    return bq, bkv, bkr


def _check(got, ref, bound, name):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    err = np.abs(got - ref)
    lim = 2 * bound + 1e-7
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err / lim), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} elements past the bound; worst at {i}: "
                             f"got {got[i]:.6g} ref {ref[i]:.6g} bound {lim[i]:.3g}")
    nrm = np.linalg.norm(ref)
    if nrm > 0:
        assert np.linalg.norm(got - ref) / nrm <= 1e-2, f"{name}: relative L2 {np.linalg.norm(got - ref) / nrm:.3e}"


def _run_bwd(d, out_bits, lse, causal, cu):
    q, kv, kr, g = dev(d["q"]), dev(d["kv"]), dev(d["k_rope"]), dev(d["dout"])
    out = dev(out_bits)
    T, H = q.shape[0], q.shape[1]
    cud = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    dq = torch.full((T, H, K), float("nan"), **f32)
    dkv = torch.full((T, H, N + V), float("nan"), **f32)
    dkr = torch.full((T, R), float("nan"), **f32)
    mla.mla_attention_bwd(q, kv, kr, out, g, lse, N, R, V, SCALE, causal=causal, cu_seqlens=cud,
                          dq=dq, dkv=dkv, dk_rope=dkr)
    torch.cuda.synchronize()
    return host64(dq), host64(dkv), host64(dkr)


def _compare(d, got, causal, cu, out64, rel_out, name):
    ref = oracle.attention_backward(d["q"], d["kv"], d["k_rope"], d["dout"], N, SCALE, causal=causal, cu_seqlens=cu)
    bounds = _bounds(d, out64, causal, cu, rel_out)
    for nm, gv, rv, bv in zip(("dq", "dkv", "dk_rope"), got, ref, bounds):
        _check(gv, rv, bv, f"{name} {nm}")


CASES = [
    # name, T, H, causal, cu_seqlens
    ("one_block", 32, 2, True, None),
    ("ragged_tail", 37, 1, True, None),
    ("several_blocks", 200, 3, True, None),
    ("single_token", 1, 2, True, None),
    ("non_causal", 150, 2, False, None),
    ("docs_empty_and_one_token", 531, 2, True, [0, 100, 101, 101, 400, 531]),
    ("docs_non_causal", 640, 1, False, [0, 128, 256, 640]),
]


@pytest.mark.parametrize("name,T,H,causal,cu", CASES, ids=[c[0] for c in CASES])
def test_attention_bwd_matches_oracle(name, T, H, causal, cu):
    print(f"[bwd] {name} T={T} H={H} causal={causal} cu={cu}", flush=True)
    d = _inputs(T, H, seed=len(name))
    out, lse = oracle.attention(d["q"], d["kv"], d["k_rope"], N, SCALE, causal=causal, cu_seqlens=cu)
    out_bits = mi.f32_to_bf16_bits(out.astype(np.float32))
    lse_t = torch.from_numpy(lse.astype(np.float32)).cuda()
    got = _run_bwd(d, out_bits, lse_t, causal, cu)
    _compare(d, got, causal, cu, oracle.widen(out_bits), 2.0 ** -8, name)


def test_attention_bwd_dsv3_rank_full_size():
    # the rank shard itself: T=2048, H=16, dense causal
    T, H = W.T, W.H
    print(f"[bwd] dsv3_rank T={T} H={H}", flush=True)
    d = _inputs(T, H, seed=0)
    out, lse = oracle.attention(d["q"], d["kv"], d["k_rope"], N, SCALE)
    out_bits = mi.f32_to_bf16_bits(out.astype(np.float32))
    got = _run_bwd(d, out_bits, torch.from_numpy(lse.astype(np.float32)).cuda(), True, None)
    _compare(d, got, True, None, oracle.widen(out_bits), 2.0 ** -8, "dsv3_rank")


def test_attention_bwd_after_the_forward_kernel():
    # forward and backward both on the GPU: out and lse are the forward kernel's
    T, H = 300, 2
    print(f"[bwd] pipeline T={T} H={H}", flush=True)
    d = _inputs(T, H, seed=99)
    q, kv, kr = dev(d["q"]), dev(d["kv"]), dev(d["k_rope"])
    out = torch.empty(T, H, V, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(H, T, dtype=torch.float32, device="cuda")
    mla.mla_attention_fwd(q, kv, kr, out, N, R, V, SCALE, causal=True, lse=lse)
    torch.cuda.synchronize()
    out_bits = out.cpu().view(torch.int16).numpy().view(np.uint16)
    got = _run_bwd(d, out_bits, lse, True, None)
    # the forward output carries its own rounding (bf16 p in its PV product): allow 2^-6 in D
    _compare(d, got, True, None, host64(out), 2.0 ** -6, "pipeline")


def test_attention_bwd_is_deterministic():
    T, H = 200, 2
    d = _inputs(T, H, seed=5)
    out, lse = oracle.attention(d["q"], d["kv"], d["k_rope"], N, SCALE)
    out_bits = mi.f32_to_bf16_bits(out.astype(np.float32))
    lse_t = torch.from_numpy(lse.astype(np.float32)).cuda()
    a = _run_bwd(d, out_bits, lse_t, True, None)
    b = _run_bwd(d, out_bits, lse_t, True, None)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ---- backward of the latent up-projection

def _up_bounds(latent, w, dkv, head_begin, heads, P):
    """Elementwise bounds: dkv rounded to bf16 (relative 2^-9, taken as 2^-8) plus worst-case fp32 accumulation
    over the contraction length n (n * 2^-24), each times the matching product of absolute values."""
    c, W, g = oracle.widen(latent), oracle.widen(w), np.asarray(dkv, np.float64)
    T = c.shape[0]
    Wc = np.abs(W[:, head_begin * P:(head_begin + heads) * P])
    g2 = np.abs(g.reshape(T, heads * P))
    C = heads * P
    b_dl = (2.0 ** -8 + C * 2.0 ** -24) * (g2 @ Wc.T)
    b_dw = (2.0 ** -8 + T * 2.0 ** -24) * (np.abs(c).T @ g2)
    return b_dl, b_dw


UP_CASES = [
    # name, T, L, heads_total, head_begin, heads, N, V
    ("small_head_range", 64, 64, 3, 1, 2, 32, 32),
    ("ragged_tokens", 37, 96, 2, 0, 2, 16, 16),
    ("uneven_columns", 100, 32, 4, 3, 1, 16, 48),
    ("dsv3_rank", 2048, 512, 128, 16, 16, 128, 128),
    # multiples of 128: the split contraction (d_latent and dw in 2 splits of 2 parts, one slice each)
    ("aligned_split", 256, 128, 4, 1, 2, 64, 64),
    # d_latent in 2 parts of 3 slices (one split), dw in 4 splits of 2 parts of one slice
    ("aligned_multi_slice", 512, 128, 3, 0, 3, 64, 64),
]


@pytest.mark.parametrize("name,T,L,ht,hb,heads,Nn,Vv", UP_CASES, ids=[c[0] for c in UP_CASES])
def test_latent_up_proj_bwd_matches_oracle(name, T, L, ht, hb, heads, Nn, Vv):
    print(f"[up_bwd] {name} T={T} L={L} heads {hb}..{hb + heads} of {ht}", flush=True)
    P = Nn + Vv
    cfg = W.cfg * 1000 + 77
    latent = mi.draw((T, L), cfg, 3)
    w = mi.draw((L, ht * P), cfg, 4, std=0.05)
    dkv = mi.normal_f32((T, heads, P), cfg, 5)
    dl, dw = mla.mla_latent_up_proj_bwd(dev(latent), dev(w), dev(dkv), ht, hb, heads, Nn, Vv)
    torch.cuda.synchronize()
    ref_dl, ref_dw = oracle.latent_up_proj_backward(latent, w, hb, heads, dkv, Nn, Vv)
    b_dl, b_dw = _up_bounds(latent, w, dkv, hb, heads, P)
    _check(host64(dl), ref_dl, b_dl, f"{name} d_latent")
    cols = slice(hb * P, (hb + heads) * P)
    _check(host64(dw), ref_dw[:, cols], b_dw, f"{name} dw")
    assert not np.any(ref_dw[:, :hb * P]) and not np.any(ref_dw[:, (hb + heads) * P:])


@pytest.mark.parametrize("name", ["dsv3_rank", "aligned_multi_slice"])
def test_latent_up_proj_bwd_single_pass_and_split_agree(name):
    """Without a workspace the single-pass kernels run: both forms meet the oracle's bounds, and the split form
    gives the same bits on a second call (its partials are summed in a fixed order)."""
    _, T, L, ht, hb, heads, Nn, Vv = next(c for c in UP_CASES if c[0] == name)
    print(f"[up_bwd] {name} single pass and split", flush=True)
    assert mla.mla_latent_up_proj_bwd_workspace_size(T, L, heads, Nn, Vv) > 0
    P = Nn + Vv
    cfg = W.cfg * 1000 + 79
    latent = mi.draw((T, L), cfg, 3)
    w = mi.draw((L, ht * P), cfg, 4, std=0.05)
    dkv = mi.normal_f32((T, heads, P), cfg, 5)
    args = (dev(latent), dev(w), dev(dkv), ht, hb, heads, Nn, Vv)
    one = mla.mla_latent_up_proj_bwd(*args, split=False)
    spl = mla.mla_latent_up_proj_bwd(*args)
    again = mla.mla_latent_up_proj_bwd(*args)
    torch.cuda.synchronize()
    ref_dl, ref_dw = oracle.latent_up_proj_backward(latent, w, hb, heads, dkv, Nn, Vv)
    b_dl, b_dw = _up_bounds(latent, w, dkv, hb, heads, P)
    cols = slice(hb * P, (hb + heads) * P)
    for form, (dl, dw) in (("single pass", one), ("split", spl)):
        _check(host64(dl), ref_dl, b_dl, f"{name} {form} d_latent")
        _check(host64(dw), ref_dw[:, cols], b_dw, f"{name} {form} dw")
    assert torch.equal(spl[0], again[0]) and torch.equal(spl[1], again[1])


def test_latent_up_proj_bwd_no_tokens_zeroes_dw():
    L, P, heads = 64, 64, 2
    latent = torch.empty((0, L), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((L, heads * P), dtype=torch.bfloat16, device="cuda")
    dkv = torch.empty((0, heads, P), dtype=torch.float32, device="cuda")
    dw = torch.full((L, heads * P), float("nan"), dtype=torch.float32, device="cuda")
    dl, dw = mla.mla_latent_up_proj_bwd(latent, w, dkv, heads, 0, heads, 32, 32, dw=dw)
    torch.cuda.synchronize()
    assert dl.shape == (0, L) and torch.all(dw == 0)


# ---- the other attention workloads at full size, checked on sampled heads
#
# Heads are independent apart from the shared band, so the oracle runs on one
# head (and one document) at a time; dq and dkv of the sampled heads are
# checked against it with the same derived bound. The band's head sum is
# checked at full size on the rank shard above. out and lse come from the
# forward kernel, hence the wider allowance for the row term.

def _pipeline(T, H, seed, cu):
    d = _inputs(T, H, seed)
    q, kv, kr = dev(d["q"]), dev(d["kv"]), dev(d["k_rope"])
    out = torch.empty(T, H, V, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(H, T, dtype=torch.float32, device="cuda")
    cud = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    mla.mla_attention_fwd(q, kv, kr, out, N, R, V, SCALE, causal=True, lse=lse, cu_seqlens=cud)
    got = mla.mla_attention_bwd(q, kv, kr, out, dev(d["dout"]), lse, N, R, V, SCALE, causal=True, cu_seqlens=cud)
    torch.cuda.synchronize()
    return d, host64(out), [host64(x) for x in got]


def _check_sampled(d, out64, got, heads, docs, name):
    for a, b in docs:
        for h in heads:
            sub = {"q": d["q"][a:b, h:h + 1], "kv": d["kv"][a:b, h:h + 1], "k_rope": d["k_rope"][a:b],
                   "dout": d["dout"][a:b, h:h + 1]}
            ref = oracle.attention_backward(sub["q"], sub["kv"], sub["k_rope"], sub["dout"], N, SCALE, causal=True)
            bq, bkv, _ = _bounds(sub, out64[a:b, h:h + 1], True, None, 2.0 ** -6)
            _check(got[0][a:b, h:h + 1], ref[0], bq, f"{name} dq tokens [{a},{b}) head {h}")
            _check(got[1][a:b, h:h + 1], ref[1], bkv, f"{name} dkv tokens [{a},{b}) head {h}")
    assert np.all(np.isfinite(got[2])), f"{name}: non-finite dk_rope"


def test_attention_bwd_uneven22_sampled_heads():
    w = mi.WORKLOADS["uneven22"]
    print(f"[bwd] uneven22 T={w.T} H={w.H}, heads 0, 13, 21", flush=True)
    d, out64, got = _pipeline(w.T, w.H, 22, None)
    _check_sampled(d, out64, got, [0, 13, 21], [(0, w.T)], "uneven22")


def test_attention_bwd_varlen16k_sampled_heads():
    w = mi.WORKLOADS["varlen16k"]
    cu = [int(x) for x in w.cu_seqlens]
    print(f"[bwd] varlen16k T={w.T} H={w.H} documents {cu}, head 5", flush=True)
    d, out64, got = _pipeline(w.T, w.H, 16, cu)
    _check_sampled(d, out64, got, [5], list(zip(cu[:-1], cu[1:])), "varlen16k")
