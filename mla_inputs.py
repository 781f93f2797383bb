"""Seeded synthetic inputs for the MLA rank-shard workloads.

This module is the only code shared by the fp64 oracle and the HIP path. It
draws random numbers and encodes them as bfloat16 bit patterns; it holds none
of the method's arithmetic (no projection, no softmax, no shard rule).

Every tensor is drawn from ``numpy.random.default_rng(1000 * cfg + tid)``:
standard normal float32, except the up-projection weight, which is scaled by
``L ** -0.5`` (variance 1/L). bf16 inputs are the float32 draws rounded to
nearest-even on their bit patterns; the same uint16 buffer is handed to the GPU
and, widened exactly, to the oracle.
"""
from __future__ import annotations

import dataclasses

import numpy as np

# tensor ids for the seed 1000*cfg + tid
TID_LATENT, TID_W, TID_Q, TID_KROPE, TID_PACK = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one rank-shard workload (notation T, H, L, N, R, V)."""

    name: str
    cfg: int
    T: int
    H: int
    L: int
    N: int
    R: int
    V: int
    heads_total: int
    head_begin: int = 0
    bf16: bool = True
    causal: bool = True
    doc_lens: tuple = ()          # packed documents (empty: one sequence)
    batch: int = 1                # decode: number of cached sequences
    kv_len: int = 0               # decode: cached positions per sequence
    kv_splits: int = 1            # decode: KV chunks per sequence
    pack_tokens: int = 0          # token->head pack: local tokens
    pack_shards: tuple = ()       # token->head pack: heads per rank

    @property
    def K(self):
        return self.N + self.R

    @property
    def P(self):
        return self.N + self.V

    @property
    def F(self):
        return self.K + self.P

    @property
    def cu_seqlens(self):
        lens = self.doc_lens or (self.T,)
        return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


WORKLOADS = {
    "tiny": Workload("tiny", 1, T=64, H=4, L=32, N=16, R=8, V=16, heads_total=4,
                     bf16=False, pack_tokens=64, pack_shards=(3, 1)),
    "dsv3_rank": Workload("dsv3_rank", 2, T=2048, H=16, L=512, N=128, R=64, V=128,
                          heads_total=16, pack_tokens=256, pack_shards=(16,) * 8),
    "uneven22": Workload("uneven22", 3, T=4096, H=22, L=512, N=128, R=64, V=128,
                         heads_total=128, pack_tokens=4096,
                         pack_shards=(22, 22, 21, 21, 21, 21)),
    "varlen16k": Workload("varlen16k", 4, T=16384, H=16, L=512, N=128, R=64, V=128,
                          heads_total=16, doc_lens=(8192, 4096, 2048, 2048)),
    "decode32": Workload("decode32", 5, T=1, H=16, L=512, N=128, R=64, V=128,
                         heads_total=16, causal=False, batch=32, kv_len=8192,
                         kv_splits=8),
}


def rng(cfg: int, tid: int) -> np.random.Generator:
    return np.random.default_rng(1000 * cfg + tid)


def normal_f32(shape, cfg: int, tid: int, std: float = 1.0) -> np.ndarray:
    x = rng(cfg, tid).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32 (for building test inputs)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw(shape, cfg, tid, std=1.0, bf16=True):
    """Return the input the GPU receives: uint16 bf16 bits, or float32 for fp32 runs."""
    x = normal_f32(shape, cfg, tid, std)
    return f32_to_bf16_bits(x) if bf16 else x


def shard_inputs(w: Workload, T: int | None = None, seed_cfg: int | None = None):
    """latent [T][L], W [L][heads_total*(N+V)], q [T][H][N+R], k_rope [T][R]."""
    T = w.T if T is None else T
    c = w.cfg if seed_cfg is None else seed_cfg
    return dict(
        latent=draw((T, w.L), c, TID_LATENT, bf16=w.bf16),
        w_kvb=draw((w.L, w.heads_total * w.P), c, TID_W, std=w.L ** -0.5, bf16=w.bf16),
        q=draw((T, w.H, w.K), c, TID_Q, bf16=w.bf16),
        k_rope=draw((T, w.R), c, TID_KROPE, bf16=w.bf16),
    )


def decode_inputs(w: Workload, batch: int | None = None, kv_len: int | None = None):
    """q [B][H][N+R], latent cache [B][S][L], rope cache [B][S][R], W [L][H*(N+V)]."""
    B = w.batch if batch is None else batch
    S = w.kv_len if kv_len is None else kv_len
    c = w.cfg
    return dict(
        q=draw((B, w.H, w.K), c, TID_Q),
        latent=draw((B, S, w.L), c, TID_LATENT),
        k_rope=draw((B, S, w.R), c, TID_KROPE),
        w_kvb=draw((w.L, w.heads_total * w.P), c, TID_W, std=w.L ** -0.5),
    )


def pack_payload(tokens: int, heads_total: int, feat: int, cfg: int, elem_bytes: int = 2):
    """Random bit patterns for the token->head permutation (copy is dtype-agnostic)."""
    dt = np.uint16 if elem_bytes == 2 else np.uint32
    info = np.iinfo(dt)
    return rng(cfg, TID_PACK).integers(0, info.max, size=(tokens, heads_total, feat),
                                       dtype=dt, endpoint=True)
