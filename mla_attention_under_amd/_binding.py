"""Thin ctypes binding of libmla.so (argument marshalling only).

Every function has the name of the C entry point it wraps (include/mla.h).
Tensors are torch tensors on the GPU; PyTorch supplies device memory and the
current stream, and every step of the computation runs in libmla.so. There is
no fallback: if the library is missing or a call fails, an exception says so.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_OK, MLA_EINVAL, MLA_EUNSUPPORTED, MLA_ELAUNCH = 0, -1, -2, -3
MLA_BF16, MLA_F32 = 0, 1

# every symbol include/mla.h declares
EXPORTS = (
    "mla_last_error", "mla_version", "mla_head_shard_sizes", "mla_pack_heads", "mla_unpack_heads",
    "mla_latent_up_proj", "mla_latent_up_proj_linear", "mla_attention_workspace_size", "mla_attention_fwd",
    "mla_latent_decode_workspace_size", "mla_latent_decode_fwd",
    "mla_pack_expanded", "mla_causal_partition", "mla_kv_exchange_ranges", "mla_apply_rope", "mla_project_pack",
    "mla_attention_bwd_workspace_size", "mla_attention_bwd", "mla_latent_up_proj_bwd_workspace_size",
    "mla_latent_up_proj_bwd",
    "mla_attention_fwd_noalloc",
)
# the measurement probe declared in include/mla_peak.h
PEAK_EXPORTS = ("mla_peak_mfma_bf16",)


class MlaError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


class mla_attn_args(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("q_stride_t", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
        ("kv", ctypes.c_void_p), ("kv_stride_t", ctypes.c_int64), ("kv_stride_h", ctypes.c_int64),
        ("k_rope", ctypes.c_void_p), ("kr_stride_t", ctypes.c_int64),
        ("out", ctypes.c_void_p), ("o_stride_t", ctypes.c_int64), ("o_stride_h", ctypes.c_int64),
        ("lse", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
        ("n_seq", ctypes.c_int), ("T_q", ctypes.c_int64), ("T_k", ctypes.c_int64),
        ("H", ctypes.c_int), ("N", ctypes.c_int), ("R", ctypes.c_int), ("V", ctypes.c_int),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int), ("dtype", ctypes.c_int),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("o_chunk_tokens", ctypes.c_int64), ("o_stride_chunk", ctypes.c_int64),
    ]


class mla_attn_bwd_args(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("q_stride_t", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
        ("kv", ctypes.c_void_p), ("kv_stride_t", ctypes.c_int64), ("kv_stride_h", ctypes.c_int64),
        ("k_rope", ctypes.c_void_p), ("kr_stride_t", ctypes.c_int64),
        ("out", ctypes.c_void_p), ("o_stride_t", ctypes.c_int64), ("o_stride_h", ctypes.c_int64),
        ("dout", ctypes.c_void_p), ("do_stride_t", ctypes.c_int64), ("do_stride_h", ctypes.c_int64),
        ("lse", ctypes.c_void_p), ("dq", ctypes.c_void_p), ("dkv", ctypes.c_void_p), ("dk_rope", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p), ("n_seq", ctypes.c_int),
        ("T", ctypes.c_int64), ("H", ctypes.c_int), ("N", ctypes.c_int), ("R", ctypes.c_int), ("V", ctypes.c_int),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int), ("dtype", ctypes.c_int),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class mla_decode_args(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("latent_cache", ctypes.c_void_p), ("rope_cache", ctypes.c_void_p),
        ("w_kvb", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("B", ctypes.c_int), ("S", ctypes.c_int64), ("L", ctypes.c_int), ("H", ctypes.c_int),
        ("heads_total", ctypes.c_int), ("head_begin", ctypes.c_int), ("N", ctypes.c_int), ("R", ctypes.c_int),
        ("V", ctypes.c_int), ("num_splits", ctypes.c_int), ("scale", ctypes.c_float), ("dtype", ctypes.c_int),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmla.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m mla_attention_under_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_version.restype = ctypes.c_char_p
    lib.mla_head_shard_sizes.argtypes = [i32, i32, i32, ctypes.POINTER(i32)]
    for fn in (lib.mla_pack_heads, lib.mla_unpack_heads):
        fn.argtypes = [vp, vp, i64, i32, i32, ctypes.POINTER(i32), i32, i32, vp]
    lib.mla_latent_up_proj.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.mla_latent_up_proj_linear.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.mla_pack_expanded.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, i32, ctypes.POINTER(i32), i32, i32, vp]
    lib.mla_apply_rope.argtypes = [vp, i64, i32, i64, i64, i32, vp, vp, i64, i32, i32, vp]
    lib.mla_project_pack.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(i32), i32,
                                     i32, i32, vp, vp, i64, i32, i32, vp]
    p64 = ctypes.POINTER(i64)
    lib.mla_causal_partition.argtypes = [p64, i32, i64, i32, i32, p64, p64, p64, p64, i32, ctypes.POINTER(i32)]
    lib.mla_kv_exchange_ranges.argtypes = [p64, i32, i64, i64, i32, i32, i32, p64, p64, p64, ctypes.POINTER(i32)]
    lib.mla_attention_workspace_size.argtypes = [ctypes.POINTER(mla_attn_args)]
    lib.mla_attention_workspace_size.restype = sz
    lib.mla_attention_fwd.argtypes = [ctypes.POINTER(mla_attn_args), vp]
    lib.mla_attention_fwd_noalloc.argtypes = [ctypes.POINTER(mla_attn_args), vp]
    lib.mla_attention_bwd_workspace_size.argtypes = [ctypes.POINTER(mla_attn_bwd_args)]
    lib.mla_attention_bwd_workspace_size.restype = sz
    lib.mla_attention_bwd.argtypes = [ctypes.POINTER(mla_attn_bwd_args), vp]
    lib.mla_latent_up_proj_bwd_workspace_size.argtypes = [i64, i32, i32, i32, i32]
    lib.mla_latent_up_proj_bwd_workspace_size.restype = sz
    lib.mla_latent_up_proj_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.mla_latent_decode_workspace_size.argtypes = [ctypes.POINTER(mla_decode_args)]
    lib.mla_latent_decode_workspace_size.restype = sz
    lib.mla_latent_decode_fwd.argtypes = [ctypes.POINTER(mla_decode_args), vp]
    lib.mla_peak_mfma_bf16.argtypes = [i32, i32, vp, vp, vp]
    for name in EXPORTS + PEAK_EXPORTS:
        getattr(lib, name).restype = getattr(lib, name).restype or ctypes.c_int
    _lib = lib
    return lib


def _check(fn, rc):
    if rc != MLA_OK:
        raise MlaError(fn, rc, load_library().mla_last_error().decode())


_ws_cache = {}
_ws_retired = []


def _workspace(nbytes: int, device, stream=None) -> "torch.Tensor | None":
    """Device scratch of at least nbytes for calls on one (device, stream).

    Each stream has its own workspace, so calls on different streams never
    share scratch, and a launch captured into a HIP graph (on its capture
    stream) keeps a workspace that later eager calls do not touch. A workspace
    that grows is replaced, but the old tensor is kept alive for the life of the
    process: a captured graph still holds its address, so its memory must never
    return to the caching allocator. Calls that overlap on ONE stream are
    ordered by the stream, so they may share it.
    """
    if nbytes == 0:
        return None
    dev = torch.device(device)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    key = (dev, int(stream.cuda_stream))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _ws_retired.append(ws)
        ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _ws_cache[key] = ws
    return ws


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype(t):
    if t.dtype == torch.float32:
        return MLA_F32
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _need(cond, fn, what):
    """Caller errors the C ABI cannot see (it gets pointers, not tensor sizes): checked before any launch."""
    if not cond:
        raise ValueError(f"{fn}: {what}")


def _same_dtype(fn, *ts):
    _need(len({t.dtype for t in ts if t is not None}) == 1, fn, "all inputs and outputs must share one dtype")


def _shape_at_least(t, dims, fn, name):
    """t has len(dims) dims, each at least dims[i] (None: any), e.g. a strided view of a wider buffer."""
    _need(t.dim() == len(dims) and all(d is None or t.shape[i] >= d for i, d in enumerate(dims)), fn,
          f"{name} has shape {tuple(t.shape)}, need {tuple(dims)}")


def _attn_shapes(fn, q, kv, k_rope, out, N, R, V, lse, cu_seqlens, cu_seqlens_k, unpack_sp=None):
    _need(q.dim() == 3 and kv.dim() == 3 and out.dim() == 3 and k_rope.dim() == 2, fn,
          "q, kv, out are [T][H][.] and k_rope [T_k][R]")
    T, H, T_k = q.shape[0], q.shape[1], kv.shape[0]
    _shape_at_least(q, (T, H, N + R), fn, "q")
    _shape_at_least(kv, (T_k, H, N + V), fn, "kv")
    _shape_at_least(k_rope, (T_k, R), fn, "k_rope")
    if unpack_sp is None:
        _need(tuple(out.shape[:2]) == (T, H) and out.shape[2] >= V, fn, f"out has shape {tuple(out.shape)}")
    else:
        _need(unpack_sp >= 1 and T % unpack_sp == 0, fn, f"T_q={T} is not a multiple of unpack_sp={unpack_sp}")
        _need(tuple(out.shape[:2]) == (T // unpack_sp, unpack_sp * H) and out.shape[2] >= V, fn,
              f"out has shape {tuple(out.shape)}, the unpacked layout is [T_q/sp][sp*H][V]")
    _need(kv.shape[1] == H and k_rope.shape[0] == T_k, fn, "kv / k_rope rows do not match")
    _same_dtype(fn, q, kv, k_rope, out)
    if lse is not None:
        _need(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == H * T, fn,
              "lse must be a contiguous fp32 [H][T_q] tensor")
    for cu in (cu_seqlens, cu_seqlens_k):
        if cu is not None:
            _need(cu.dtype == torch.int32 and cu.is_contiguous() and cu.dim() == 1 and cu.numel() >= 2, fn,
                  "document offsets are contiguous int32 [n_seq + 1] tensors")
    if cu_seqlens is not None and cu_seqlens_k is not None:
        _need(cu_seqlens_k.numel() == cu_seqlens.numel(), fn, "query and key offsets list the same documents")


def mla_head_shard_sizes(q_heads: int, kv_heads: int, sp: int) -> list[int]:
    lib = load_library()
    out = (ctypes.c_int * max(sp, 1))()
    _check("mla_head_shard_sizes", lib.mla_head_shard_sizes(q_heads, kv_heads, sp, out))
    return list(out)[:sp]


def _pack(name, src, dst, sizes, tokens, heads_total, feat, stream):
    lib = load_library()
    _dev(src, dst)
    if src.element_size() != dst.element_size():
        raise ValueError("source and destination element sizes differ")
    dt = {2: MLA_BF16, 4: MLA_F32}[src.element_size()]
    arr = (ctypes.c_int * len(sizes))(*sizes)
    _check(name, getattr(lib, name)(_ptr(src), _ptr(dst), tokens, heads_total, feat, arr, len(sizes), dt,
                                    _stream(stream)))
    return dst


def mla_pack_heads(x, send, sizes, stream=None):
    """x [T][heads_total][F] (contiguous) -> send (flat, concat_r [T][sizes[r]][F])."""
    assert x.is_contiguous() and send.is_contiguous() and x.dim() == 3 and send.numel() == x.numel()
    T, Ht, F = x.shape
    return _pack("mla_pack_heads", x, send, sizes, T, Ht, F, stream)


def mla_unpack_heads(recv, x, sizes, stream=None):
    """recv (flat, concat_r [T][sizes[r]][F]) -> x [T][heads_total][F] (contiguous)."""
    assert x.is_contiguous() and recv.is_contiguous() and x.dim() == 3 and recv.numel() == x.numel()
    T, Ht, F = x.shape
    return _pack("mla_unpack_heads", recv, x, sizes, T, Ht, F, stream)


def mla_pack_expanded(q, kv, k_rope, send, sizes, N, stream=None):
    """q [T][Ht][N+R], kv [T][Ht][N+V], k_rope [T][R] -> send (flat, concat_r [T][sizes[r]][2(N+R)+V])."""
    lib = load_library()
    _dev(q, kv, k_rope, send)
    assert all(t.is_contiguous() for t in (q, kv, k_rope, send))
    T, Ht, K = q.shape
    R = k_rope.shape[1]
    V = kv.shape[2] - N
    assert kv.shape[:2] == (T, Ht) and k_rope.shape[0] == T and K == N + R
    assert send.numel() == T * Ht * (2 * K + V)
    if len({t.element_size() for t in (q, kv, k_rope, send)}) != 1:
        raise ValueError("all buffers must have one element size")
    dt = {2: MLA_BF16, 4: MLA_F32}[q.element_size()]
    arr = (ctypes.c_int * len(sizes))(*sizes)
    _check("mla_pack_expanded", lib.mla_pack_expanded(_ptr(q), _ptr(kv), _ptr(k_rope), _ptr(send), T, Ht, N, R, V,
                                                       arr, len(sizes), dt, _stream(stream)))
    return send


def mla_apply_rope(band, cos, sin, interleaved=False, stream=None):
    """Rotate a RoPE band in place: band is a view [T][H][R] (e.g. q[..., N:]) or [T][R] with unit last
    stride; cos, sin are [T][R] tables of the band's dtype."""
    lib = load_library()
    _dev(band, cos, sin)
    if band.dim() == 2:
        T, R = band.shape
        H, st, sh = 1, band.stride(0), R
    else:
        T, H, R = band.shape
        st, sh = band.stride(0), band.stride(1)
    assert band.stride(-1) == 1 and cos.shape == (T, R) and sin.shape == (T, R)
    assert cos.stride(-1) == 1 and sin.stride() == cos.stride() and cos.dtype == sin.dtype == band.dtype
    _check("mla_apply_rope", lib.mla_apply_rope(_ptr(band), T, H, st, sh, R, _ptr(cos), _ptr(sin), cos.stride(0),
                                                 int(bool(interleaved)), _dtype(band), _stream(stream)))
    return band


def mla_project_pack(latent, w, send, w_heads, head_begin, heads, P, F, col_offset, sizes, rope_offset=-1,
                     cos=None, sin=None, interleaved=False, stream=None):
    """latent [T][L] x w [L][w_heads*P] (heads [head_begin, +heads)) -> columns [col_offset, +P) of every
    payload row of send (flat, concat_r [T][sizes[r]][F]); RoPE on the block's columns [rope_offset, +R)
    when cos/sin ([T][R]) are given."""
    lib = load_library()
    _dev(latent, w, send, *(t for t in (cos, sin) if t is not None))
    T, L = latent.shape
    assert latent.is_contiguous() and w.is_contiguous() and send.is_contiguous()
    assert w.shape == (L, w_heads * P) and send.numel() == T * heads * F
    _same_dtype("mla_project_pack", latent, w, send, cos, sin)
    _need((cos is None) == (sin is None), "mla_project_pack", "give both RoPE tables or neither")
    if cos is not None:
        _need(cos.dim() == 2 and cos.shape[0] >= T and cos.stride(-1) == 1 and sin.shape == cos.shape and
              sin.stride() == cos.stride(), "mla_project_pack", "cos and sin are [T][R] tables with one stride")
    R = 0 if cos is None else cos.shape[1]
    cs = 0 if cos is None else cos.stride(0)
    arr = (ctypes.c_int * len(sizes))(*sizes)
    _check("mla_project_pack", lib.mla_project_pack(
        _ptr(latent), _ptr(w), _ptr(send), T, L, w_heads, head_begin, heads, P, F, col_offset, arr, len(sizes),
        rope_offset, R, _ptr(cos), _ptr(sin), cs, int(bool(interleaved)), _dtype(latent), _stream(stream)))
    return send


def _i64s(xs):
    return (ctypes.c_int64 * max(len(xs), 1))(*[int(x) for x in xs])


def mla_causal_partition(doc_ends, query_length, query_rank, batch=1):
    """Host interval algebra: dict(key_begin, key_end, query_ends, key_ends)."""
    lib = load_library()
    cap = batch * len(doc_ends)
    kb, ke, n = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int()
    qe, kend = (ctypes.c_int64 * max(cap, 1))(), (ctypes.c_int64 * max(cap, 1))()
    _check("mla_causal_partition", lib.mla_causal_partition(
        _i64s(doc_ends), len(doc_ends), query_length, query_rank, batch, ctypes.byref(kb), ctypes.byref(ke), qe, kend,
        cap, ctypes.byref(n)))
    return {"key_begin": kb.value, "key_end": ke.value, "query_ends": list(qe)[:n.value],
            "key_ends": list(kend)[:n.value]}


def mla_kv_exchange_ranges(doc_ends, source_length, query_length, head_copies, degree, rank):
    """Host interval algebra: (((offset, count) sent to each peer), (count received from each peer), local_only)."""
    lib = load_library()
    so, sc, rc = (ctypes.c_int64 * degree)(), (ctypes.c_int64 * degree)(), (ctypes.c_int64 * degree)()
    local = ctypes.c_int()
    _check("mla_kv_exchange_ranges", lib.mla_kv_exchange_ranges(
        _i64s(doc_ends), len(doc_ends), source_length, query_length, head_copies, degree, rank, so, sc, rc,
        ctypes.byref(local)))
    return tuple(zip(list(so), list(sc))), tuple(rc), bool(local.value)


def mla_latent_up_proj(latent, w_kvb, kv_out, heads_total, head_begin, heads, N, V, stream=None):
    """latent [T][L], w_kvb [L][heads_total*(N+V)] -> kv_out [T][heads][N+V]."""
    lib = load_library()
    _dev(latent, w_kvb, kv_out)
    assert latent.is_contiguous() and w_kvb.is_contiguous() and kv_out.is_contiguous()
    T, L = latent.shape
    assert w_kvb.shape == (L, heads_total * (N + V)) and kv_out.numel() == T * heads * (N + V)
    _same_dtype("mla_latent_up_proj", latent, w_kvb, kv_out)
    _check("mla_latent_up_proj", lib.mla_latent_up_proj(
        _ptr(latent), _ptr(w_kvb), _ptr(kv_out), T, L, heads_total, head_begin, heads, N, V, _dtype(latent),
        _stream(stream)))
    return kv_out


def mla_latent_up_proj_linear(latent, w_lin, kv_out, heads_total, head_begin, heads, N, V, stream=None):
    """latent [T][L], w_lin [heads_total*(N+V)][L] (torch.nn.Linear's weight) -> kv_out [T][heads][N+V]."""
    lib = load_library()
    _dev(latent, w_lin, kv_out)
    assert latent.is_contiguous() and w_lin.is_contiguous() and kv_out.is_contiguous()
    T, L = latent.shape
    assert w_lin.shape == (heads_total * (N + V), L) and kv_out.numel() == T * heads * (N + V)
    _same_dtype("mla_latent_up_proj_linear", latent, w_lin, kv_out)
    _check("mla_latent_up_proj_linear", lib.mla_latent_up_proj_linear(
        _ptr(latent), _ptr(w_lin), _ptr(kv_out), T, L, heads_total, head_begin, heads, N, V, _dtype(latent),
        _stream(stream)))
    return kv_out


def _attn_args(q, kv, k_rope, out, N, R, V, scale, causal, lse, cu_seqlens, workspace, cu_seqlens_k=None,
               unpack_sp=None):
    T, H = q.shape[0], q.shape[1]
    a = mla_attn_args()
    a.q, a.q_stride_t, a.q_stride_h = q.data_ptr(), q.stride(0), q.stride(1)
    a.kv, a.kv_stride_t, a.kv_stride_h = kv.data_ptr(), kv.stride(0), kv.stride(1)
    a.k_rope, a.kr_stride_t = k_rope.data_ptr(), k_rope.stride(0)
    a.out, a.o_stride_t, a.o_stride_h = out.data_ptr(), out.stride(0), out.stride(1)
    if unpack_sp is not None:
        # query chunk r = rank r's tokens, written to heads [r*H, (r+1)*H) of the token-major rows
        a.o_chunk_tokens, a.o_stride_chunk = T // unpack_sp, H * out.stride(1)
    a.lse = None if lse is None else lse.data_ptr()
    a.cu_seqlens = None if cu_seqlens is None else cu_seqlens.data_ptr()
    a.cu_seqlens_k = None if cu_seqlens_k is None else cu_seqlens_k.data_ptr()
    a.n_seq = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    a.T_q, a.T_k = T, kv.shape[0]
    a.H, a.N, a.R, a.V = H, N, R, V
    a.scale, a.causal, a.dtype = float(scale), int(bool(causal)), _dtype(q)
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return a


def mla_attention_workspace_size(q, kv, k_rope, out, N, R, V, scale, causal=True, cu_seqlens=None,
                                 cu_seqlens_k=None) -> int:
    a = _attn_args(q, kv, k_rope, out, N, R, V, scale, causal, None, cu_seqlens, None, cu_seqlens_k)
    return int(load_library().mla_attention_workspace_size(ctypes.byref(a)))


def _check_offsets(*cus):
    for cu in cus:
        if cu is not None:
            assert cu.dtype == torch.int32 and cu.is_contiguous()


def mla_attention_fwd(q, kv, k_rope, out, N, R, V, scale, causal=True, lse=None, cu_seqlens=None,
                      workspace=None, stream=None, cu_seqlens_k=None, unpack_sp=None):
    """q [T_q][H][N+R], kv [T_k][H][N+V], k_rope [T_k][R] (last dims unit-stride) -> out [T_q][H][V].

    Strided views are passed through (e.g. q and kv read in place from a packed
    [T][H][F] buffer). cu_seqlens / cu_seqlens_k: int32 device tensors [n_seq+1]
    of query / key document offsets, or None. The workspace, when needed and not
    given, is allocated through PyTorch. With unpack_sp = sp, out is the
    token-major [T_q/sp][sp*H][V] buffer that follows the head->token exchange:
    query t of head h is written to out[t % (T_q/sp)][(t // (T_q/sp))*H + h],
    which is mla_unpack_heads(out [T_q][H][V], y, [H]*sp) without the copy.
    """
    lib = load_library()
    _dev(q, kv, k_rope, out, lse, cu_seqlens, cu_seqlens_k, workspace)
    for t in (q, kv, k_rope, out):
        assert t.stride(-1) == 1
    _check_offsets(cu_seqlens, cu_seqlens_k)
    _attn_shapes("mla_attention_fwd", q, kv, k_rope, out, N, R, V, lse, cu_seqlens, cu_seqlens_k, unpack_sp)
    if workspace is None:
        workspace = _workspace(mla_attention_workspace_size(q, kv, k_rope, out, N, R, V, scale, causal, cu_seqlens,
                                                            cu_seqlens_k), q.device, stream)
    a = _attn_args(q, kv, k_rope, out, N, R, V, scale, causal, lse, cu_seqlens, workspace, cu_seqlens_k, unpack_sp)
    _check("mla_attention_fwd", lib.mla_attention_fwd(ctypes.byref(a), _stream(stream)))
    return out


def mla_attention_fwd_noalloc(q, kv, k_rope, out, N, R, V, scale, causal=True, lse=None, cu_seqlens=None,
                              stream=None, cu_seqlens_k=None, unpack_sp=None):
    """mla_attention_fwd with the library's fixed per-GPU scratch instead of a workspace: nothing is
    allocated (for graph capture and serving loops). Calls overlapping on one GPU race on that scratch."""
    lib = load_library()
    _dev(q, kv, k_rope, out, lse, cu_seqlens, cu_seqlens_k)
    for t in (q, kv, k_rope, out):
        assert t.stride(-1) == 1
    _check_offsets(cu_seqlens, cu_seqlens_k)
    _attn_shapes("mla_attention_fwd_noalloc", q, kv, k_rope, out, N, R, V, lse, cu_seqlens, cu_seqlens_k,
                 unpack_sp)
    a = _attn_args(q, kv, k_rope, out, N, R, V, scale, causal, lse, cu_seqlens, None, cu_seqlens_k, unpack_sp)
    _check("mla_attention_fwd_noalloc", lib.mla_attention_fwd_noalloc(ctypes.byref(a), _stream(stream)))
    return out


def _attn_bwd_args(q, kv, k_rope, out, dout, lse, dq, dkv, dk_rope, N, R, V, scale, causal, cu_seqlens,
                   workspace):
    T, H = q.shape[0], q.shape[1]
    a = mla_attn_bwd_args()
    a.q, a.q_stride_t, a.q_stride_h = q.data_ptr(), q.stride(0), q.stride(1)
    a.kv, a.kv_stride_t, a.kv_stride_h = kv.data_ptr(), kv.stride(0), kv.stride(1)
    a.k_rope, a.kr_stride_t = k_rope.data_ptr(), k_rope.stride(0)
    a.out, a.o_stride_t, a.o_stride_h = out.data_ptr(), out.stride(0), out.stride(1)
    a.dout, a.do_stride_t, a.do_stride_h = dout.data_ptr(), dout.stride(0), dout.stride(1)
    a.lse = None if lse is None else lse.data_ptr()
    a.dq = None if dq is None else dq.data_ptr()
    a.dkv = None if dkv is None else dkv.data_ptr()
    a.dk_rope = None if dk_rope is None else dk_rope.data_ptr()
    a.cu_seqlens = None if cu_seqlens is None else cu_seqlens.data_ptr()
    a.n_seq = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    a.T, a.H, a.N, a.R, a.V = T, H, N, R, V
    a.scale, a.causal, a.dtype = float(scale), int(bool(causal)), _dtype(q)
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return a


def mla_attention_bwd_workspace_size(q, kv, k_rope, out, dout, N, R, V, scale, causal=True, cu_seqlens=None) -> int:
    a = _attn_bwd_args(q, kv, k_rope, out, dout, None, None, None, None, N, R, V, scale, causal, cu_seqlens, None)
    return int(load_library().mla_attention_bwd_workspace_size(ctypes.byref(a)))


def mla_attention_bwd(q, kv, k_rope, out, dout, lse, N, R, V, scale, causal=True, cu_seqlens=None,
                      dq=None, dkv=None, dk_rope=None, workspace=None, stream=None):
    """Gradients of mla_attention_fwd: (dq [T][H][N+R], dkv [T][H][N+V], dk_rope [T][R]), fp32.

    out and lse are the forward's output and log-sum-exp; dout the gradient of
    out. Missing outputs and the workspace are allocated through PyTorch.
    """
    lib = load_library()
    _dev(q, kv, k_rope, out, dout, lse, cu_seqlens, dq, dkv, dk_rope, workspace)
    for t in (q, kv, k_rope, out, dout):
        assert t.stride(-1) == 1
    fn = "mla_attention_bwd"
    _attn_shapes(fn, q, kv, k_rope, out, N, R, V, lse, cu_seqlens, None)
    _need(lse is not None, fn, "the forward's lse is required")
    T, H = q.shape[0], q.shape[1]
    _need(kv.shape[0] == T, fn, "queries and keys are the same tokens")
    _need(dout.dim() == 3 and tuple(dout.shape[:2]) == (T, H) and dout.shape[2] >= V and dout.dtype == q.dtype, fn,
          "dout has the shape and dtype of out")
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(T, H, N + R, **f32) if dq is None else dq
    dkv = torch.empty(T, H, N + V, **f32) if dkv is None else dkv
    dk_rope = torch.empty(T, R, **f32) if dk_rope is None else dk_rope
    for t in (dq, dkv, dk_rope, lse):
        assert t.dtype == torch.float32 and t.is_contiguous()
    _need(tuple(dq.shape) == (T, H, N + R) and tuple(dkv.shape) == (T, H, N + V) and tuple(dk_rope.shape) == (T, R),
          fn, "dq [T][H][N+R], dkv [T][H][N+V] and dk_rope [T][R]")
    if workspace is None:
        workspace = _workspace(mla_attention_bwd_workspace_size(q, kv, k_rope, out, dout, N, R, V, scale, causal,
                                                                cu_seqlens), q.device, stream)
    a = _attn_bwd_args(q, kv, k_rope, out, dout, lse, dq, dkv, dk_rope, N, R, V, scale, causal, cu_seqlens,
                       workspace)
    _check("mla_attention_bwd", lib.mla_attention_bwd(ctypes.byref(a), _stream(stream)))
    return dq, dkv, dk_rope


def mla_latent_up_proj_bwd_workspace_size(T, L, heads, N, V) -> int:
    return int(load_library().mla_latent_up_proj_bwd_workspace_size(T, L, heads, N, V))


def mla_latent_up_proj_bwd(latent, w_kvb, dkv, w_heads, head_begin, heads, N, V, d_latent=None, dw=None,
                           workspace=None, split=True, stream=None):
    """Gradients of mla_latent_up_proj: (d_latent [T][L], dw [L][heads*(N+V)]), fp32.

    latent [T][L] and w_kvb [L][w_heads*(N+V)] bf16; dkv [T][heads][N+V] fp32
    (mla_attention_bwd's dkv); dw covers the head range's weight columns.
    split=False passes no workspace (the single-pass kernels); otherwise a
    workspace of the size the library asks for is taken from the per-stream cache
    unless one is given.
    """
    lib = load_library()
    _dev(latent, w_kvb, dkv, d_latent, dw)
    for t in (latent, w_kvb, dkv):
        assert t.is_contiguous()
    T, L = latent.shape
    assert dkv.dtype == torch.float32 and dkv.shape == (T, heads, N + V)
    fn = "mla_latent_up_proj_bwd"
    _need(tuple(w_kvb.shape) == (L, w_heads * (N + V)), fn, "w_kvb is [L][w_heads*(N+V)]")
    _same_dtype(fn, latent, w_kvb)
    f32 = dict(dtype=torch.float32, device=latent.device)
    d_latent = torch.empty(T, L, **f32) if d_latent is None else d_latent
    dw = torch.empty(L, heads * (N + V), **f32) if dw is None else dw
    assert d_latent.is_contiguous() and dw.is_contiguous()
    _need(d_latent.dtype == dw.dtype == torch.float32 and tuple(d_latent.shape) == (T, L) and
          tuple(dw.shape) == (L, heads * (N + V)), fn, "d_latent [T][L] and dw [L][heads*(N+V)], fp32")
    if not split:
        workspace = None
    elif workspace is None:
        workspace = _workspace(mla_latent_up_proj_bwd_workspace_size(T, L, heads, N, V), latent.device, stream)
    _check("mla_latent_up_proj_bwd", lib.mla_latent_up_proj_bwd(
        latent.data_ptr(), w_kvb.data_ptr(), dkv.data_ptr(), d_latent.data_ptr(), dw.data_ptr(), T, L, w_heads,
        head_begin, heads, N, V, _dtype(latent), _ptr(workspace), 0 if workspace is None else workspace.numel(),
        _stream(stream)))
    return d_latent, dw


def _decode_args(q, latent_cache, rope_cache, w_kvb, out, heads_total, head_begin, N, R, V, num_splits, scale,
                 lse, workspace):
    B, H = q.shape[0], q.shape[1]
    a = mla_decode_args()
    a.q, a.latent_cache, a.rope_cache = q.data_ptr(), latent_cache.data_ptr(), rope_cache.data_ptr()
    a.w_kvb, a.out = w_kvb.data_ptr(), out.data_ptr()
    a.lse = None if lse is None else lse.data_ptr()
    a.B, a.S, a.L, a.H = B, latent_cache.shape[1], latent_cache.shape[2], H
    a.heads_total, a.head_begin, a.N, a.R, a.V = heads_total, head_begin, N, R, V
    a.num_splits, a.scale, a.dtype = num_splits, float(scale), _dtype(q)
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return a


def mla_latent_decode_workspace_size(q, latent_cache, rope_cache, w_kvb, out, heads_total, head_begin, N, R, V,
                                     num_splits, scale) -> int:
    a = _decode_args(q, latent_cache, rope_cache, w_kvb, out, heads_total, head_begin, N, R, V, num_splits, scale,
                     None, None)
    return int(load_library().mla_latent_decode_workspace_size(ctypes.byref(a)))


def mla_latent_decode_fwd(q, latent_cache, rope_cache, w_kvb, out, heads_total, head_begin, N, R, V, num_splits,
                          scale, lse=None, workspace=None, stream=None):
    """q [B][H][N+R], latent_cache [B][S][L], rope_cache [B][S][R], w_kvb [L][heads_total*(N+V)] -> out [B][H][V]."""
    lib = load_library()
    _dev(q, latent_cache, rope_cache, w_kvb, out, lse, workspace)
    for t in (q, latent_cache, rope_cache, w_kvb, out):
        assert t.is_contiguous()
    fn = "mla_latent_decode_fwd"
    _need(q.dim() == 3 and latent_cache.dim() == 3 and rope_cache.dim() == 3, fn,
          "q [B][H][N+R], latent_cache [B][S][L], rope_cache [B][S][R]")
    B, H = q.shape[0], q.shape[1]
    S, L = latent_cache.shape[1], latent_cache.shape[2]
    _need(tuple(q.shape) == (B, H, N + R) and tuple(latent_cache.shape[:1]) == (B,) and
          tuple(rope_cache.shape) == (B, S, R) and tuple(w_kvb.shape) == (L, heads_total * (N + V)) and
          tuple(out.shape) == (B, H, V), fn, "shapes do not match q [B][H][N+R] ... out [B][H][V]")
    _same_dtype(fn, q, latent_cache, rope_cache, w_kvb, out)
    if lse is not None:
        _need(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == B * H, fn,
              "lse must be a contiguous fp32 [B][H] tensor")
    if workspace is None:
        workspace = _workspace(mla_latent_decode_workspace_size(q, latent_cache, rope_cache, w_kvb, out, heads_total,
                                                                head_begin, N, R, V, num_splits, scale), q.device, stream)
    a = _decode_args(q, latent_cache, rope_cache, w_kvb, out, heads_total, head_begin, N, R, V, num_splits, scale,
                     lse, workspace)
    _check("mla_latent_decode_fwd", lib.mla_latent_decode_fwd(ctypes.byref(a), _stream(stream)))
    return out


def mla_peak_mfma_bf16(blocks, iters, clocks, sink, stream=None):
    """Launch the MFMA peak probe (include/mla_peak.h): clocks int64 [blocks*16], sink float32 [blocks*512]."""
    lib = load_library()
    _dev(clocks, sink)
    assert clocks.numel() >= blocks * 16 and sink.numel() >= blocks * 512
    rc = lib.mla_peak_mfma_bf16(blocks, iters, _ptr(clocks), _ptr(sink), _stream(stream))
    if rc != 0:
        raise MlaError("mla_peak_mfma_bf16", rc, "bad argument" if rc == -1 else "launch failed")
