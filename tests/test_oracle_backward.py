"""Pins for the oracle's backward of the shard (CPU only).

The gradients are checked against float64 autograd of the expanded-key form
(the shared RoPE key broadcast to every head, so autograd itself sums its
gradient over heads) and against central finite differences, which use
nothing but the forward oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _inputs(T, H, N, R, V, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, H, N + R)), rng.standard_normal((T, H, N + V)), rng.standard_normal((T, R)),
            rng.standard_normal((T, H, V)))


def _autograd(q, kv, kr, do, N, scale, causal, cu):
    qt, kvt, krt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, kv, kr))
    T, H, _ = q.shape
    bounds = oracle.doc_bounds(cu, T)
    out = torch.zeros((T, H, kv.shape[2] - N), dtype=torch.float64)
    outs = []
    for a, b in bounds:
        k = torch.cat([kvt[a:b, :, :N], krt[a:b, None, :].expand(b - a, H, kr.shape[1])], dim=2)   # shared band
        s = scale * torch.einsum("thk,jhk->htj", qt[a:b], k)
        if causal:
            s = s.masked_fill(~torch.tril(torch.ones(b - a, b - a, dtype=torch.bool)), float("-inf"))
        outs.append(torch.einsum("htj,jhv->thv", torch.softmax(s, dim=-1), kvt[a:b, :, N:]))
    out = torch.cat(outs, dim=0)
    (out * torch.tensor(do)).sum().backward()
    return qt.grad.numpy(), kvt.grad.numpy(), krt.grad.numpy()


@pytest.mark.parametrize("causal,cu", [(True, None), (False, None), (True, [0, 5, 6, 13])])
def test_attention_backward_matches_autograd(causal, cu):
    T, H, N, R, V = 13, 3, 6, 4, 5
    q, kv, kr, do = _inputs(T, H, N, R, V, 31)
    scale = 1 / math.sqrt(N + R)
    got = oracle.attention_backward(q, kv, kr, do, N, scale, causal, cu)
    exp = _autograd(q, kv, kr, do, N, scale, causal, cu)
    for g, e, name in zip(got, exp, ("dq", "dkv", "dk_rope")):
        assert np.max(np.abs(g - e)) < 1e-10, name


def test_attention_backward_matches_finite_differences():
    T, H, N, R, V = 7, 2, 4, 2, 3
    q, kv, kr, do = _inputs(T, H, N, R, V, 32)
    scale = 1 / math.sqrt(N + R)
    dq, dkv, dkr = oracle.attention_backward(q, kv, kr, do, N, scale)
    f = lambda q_, kv_, kr_: float(np.sum(oracle.attention(q_, kv_, kr_, N, scale)[0] * do))
    rng = np.random.default_rng(33)
    eps = 1e-6
    for _ in range(3):
        uq, ukv, ukr = rng.standard_normal(q.shape), rng.standard_normal(kv.shape), rng.standard_normal(kr.shape)
        num = (f(q + eps * uq, kv + eps * ukv, kr + eps * ukr) - f(q - eps * uq, kv - eps * ukv, kr - eps * ukr)) / (2 * eps)
        ana = np.sum(dq * uq) + np.sum(dkv * ukv) + np.sum(dkr * ukr)
        assert abs(num - ana) < 1e-6 * max(1.0, abs(ana)), (num, ana)


def test_shared_band_gradient_is_the_sum_over_heads():
    # each head alone (one-head slices) gives its band gradient; the shared band gets their sum
    T, H, N, R, V = 9, 4, 4, 2, 3
    q, kv, kr, do = _inputs(T, H, N, R, V, 34)
    scale = 1 / math.sqrt(N + R)
    _, _, dkr = oracle.attention_backward(q, kv, kr, do, N, scale)
    per_head = [oracle.attention_backward(q[:, h:h + 1], kv[:, h:h + 1], kr, do[:, h:h + 1], N, scale)[2]
                for h in range(H)]
    assert np.max(np.abs(dkr - sum(per_head))) < 1e-12


def test_latent_up_proj_backward_matches_autograd():
    T, L, Ht, hb, hs, N, V = 6, 8, 4, 1, 2, 3, 2
    rng = np.random.default_rng(35)
    c, W = rng.standard_normal((T, L)), rng.standard_normal((L, Ht * (N + V)))
    g = rng.standard_normal((T, hs, N + V))
    dl, dW = oracle.latent_up_proj_backward(c, W, hb, hs, g, N, V)
    ct, Wt = torch.tensor(c, requires_grad=True), torch.tensor(W, requires_grad=True)
    P = N + V
    out = (ct @ Wt[:, hb * P:(hb + hs) * P]).reshape(T, hs, P)
    (out * torch.tensor(g)).sum().backward()
    assert np.max(np.abs(dl - ct.grad.numpy())) < 1e-12
    assert np.max(np.abs(dW - Wt.grad.numpy())) < 1e-12
    assert not dW[:, :hb * P].any() and not dW[:, (hb + hs) * P:].any()


def test_shard_backward_chain_matches_autograd():
    # latent -> kv (head range) -> attention: the chained oracle gradients equal end-to-end autograd
    T, L, Ht, hb, H, N, R, V = 10, 6, 3, 1, 2, 4, 2, 3
    rng = np.random.default_rng(36)
    c, W = rng.standard_normal((T, L)), rng.standard_normal((L, Ht * (N + V)))
    q, kr, do = rng.standard_normal((T, H, N + R)), rng.standard_normal((T, R)), rng.standard_normal((T, H, V))
    scale = 1 / math.sqrt(N + R)
    kv = oracle.latent_up_proj(c, W, hb, H, N, V)
    dq, dkv, dkr = oracle.attention_backward(q, kv, kr, do, N, scale)
    dl, dW = oracle.latent_up_proj_backward(c, W, hb, H, dkv, N, V)
    ct, Wt, qt, krt = (torch.tensor(x, requires_grad=True) for x in (c, W, q, kr))
    P = N + V
    kvt = (ct @ Wt[:, hb * P:(hb + H) * P]).reshape(T, H, P)
    k = torch.cat([kvt[..., :N], krt[:, None, :].expand(T, H, R)], dim=2)
    s = scale * torch.einsum("thk,jhk->htj", qt, k)
    s = s.masked_fill(~torch.tril(torch.ones(T, T, dtype=torch.bool)), float("-inf"))
    out = torch.einsum("htj,jhv->thv", torch.softmax(s, dim=-1), kvt[..., N:])
    (out * torch.tensor(do)).sum().backward()
    for got, ref in ((dq, qt.grad), (dkr, krt.grad), (dl, ct.grad), (dW, Wt.grad)):
        assert np.max(np.abs(got - ref.numpy())) < 1e-10
