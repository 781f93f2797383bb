"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, computes shard lists bit-exactly like the oracle, and rejects bad
arguments on the host before anything is launched."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from golden_io import shard_cases

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

mla = pytest.importorskip("mla_attention_under_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mla.LIB_PATH):
        pytest.fail("libmla.so is not built (python -m mla_attention_under_amd.build)")
    return mla.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(mla_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_path_calls():
    fns = declared_functions()
    for name in ("mla_pack_heads", "mla_latent_up_proj", "mla_attention_fwd", "mla_unpack_heads"):
        assert name in fns
    assert set(fns) == set(mla.EXPORTS)


def test_peak_probe_header_matches_the_exports(lib):
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mla_peak.h")).read(), flags=re.S)
    fns = sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(mla_\w+)\s*\(", text, flags=re.M)))
    assert fns == sorted(mla.PEAK_EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", mla.LIB_PATH], capture_output=True, text=True).stdout
    for f in fns:
        assert re.search(rf"\bT {f}$", out, flags=re.M), f
    assert lib.mla_peak_mfma_bf16(0, 10, None, None, None) == -1      # bad argument: nothing launched


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", mla.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (mla_\w+)$", out, flags=re.M))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    for f in declared_functions():
        getattr(lib, f)


def test_struct_layouts_match_the_header():
    # offsets computed by the C compiler from the header itself
    src = r'''
#include <stddef.h>
#include <stdio.h>
#include "mla.h"
#define P(s, f) printf(#s "." #f " %zu\n", offsetof(s, f));
int main(void) {
  P(mla_attn_args, q) P(mla_attn_args, kv_stride_h) P(mla_attn_args, out) P(mla_attn_args, lse)
  P(mla_attn_args, cu_seqlens) P(mla_attn_args, cu_seqlens_k) P(mla_attn_args, n_seq) P(mla_attn_args, T_q)
  P(mla_attn_args, T_k) P(mla_attn_args, V)
  P(mla_attn_args, scale) P(mla_attn_args, dtype) P(mla_attn_args, workspace) P(mla_attn_args, workspace_bytes)
  P(mla_attn_args, o_chunk_tokens) P(mla_attn_args, o_stride_chunk)
  P(mla_decode_args, lse) P(mla_decode_args, B) P(mla_decode_args, S) P(mla_decode_args, num_splits)
  P(mla_decode_args, scale) P(mla_decode_args, workspace) P(mla_decode_args, workspace_bytes)
  P(mla_attn_bwd_args, dout) P(mla_attn_bwd_args, do_stride_h) P(mla_attn_bwd_args, lse) P(mla_attn_bwd_args, dq)
  P(mla_attn_bwd_args, dk_rope) P(mla_attn_bwd_args, cu_seqlens) P(mla_attn_bwd_args, T) P(mla_attn_bwd_args, V)
  P(mla_attn_bwd_args, scale) P(mla_attn_bwd_args, dtype) P(mla_attn_bwd_args, workspace_bytes)
  printf("sizeof.attn %zu\nsizeof.decode %zu\nsizeof.bwd %zu\n", sizeof(mla_attn_args), sizeof(mla_decode_args),
         sizeof(mla_attn_bwd_args));
  return 0;
}'''
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "off.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "off")
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()
    got = dict(zip(lines[0::2], (int(x) for x in lines[1::2])))
    from mla_attention_under_amd._binding import mla_attn_args, mla_attn_bwd_args, mla_decode_args
    for key, off in got.items():
        s, f = key.split(".")
        if s == "sizeof":
            assert ctypes.sizeof({"attn": mla_attn_args, "decode": mla_decode_args, "bwd": mla_attn_bwd_args}[f]) == off
        else:
            cls = {"mla_attn_args": mla_attn_args, "mla_decode_args": mla_decode_args,
                   "mla_attn_bwd_args": mla_attn_bwd_args}[s]
            assert getattr(cls, f).offset == off, key


@pytest.mark.parametrize("q,kv,sp,exp,src", shard_cases() + shard_cases("workload_shards.txt"))
def test_shard_lists_match_pages_and_oracle(lib, q, kv, sp, exp, src):
    if exp is None:
        with pytest.raises(mla.MlaError) as e:
            mla.mla_head_shard_sizes(q, kv, sp)
        assert e.value.code == mla.MLA_EINVAL
    else:
        assert mla.mla_head_shard_sizes(q, kv, sp) == exp == oracle.head_shard_sizes(q, kv, sp)


def test_shard_lists_bit_exact_against_oracle_exhaustive(lib):
    for kv in range(1, 33):
        for g in (1, 2, 3, 8):
            for sp in range(1, 40):
                q = kv * g
                try:
                    ref = oracle.head_shard_sizes(q, kv, sp)
                except ValueError:
                    with pytest.raises(mla.MlaError):
                        mla.mla_head_shard_sizes(q, kv, sp)
                    continue
                assert mla.mla_head_shard_sizes(q, kv, sp) == ref


def test_shard_list_error_leaves_output_untouched(lib):
    out = (ctypes.c_int * 2)(-7, -7)
    assert lib.mla_head_shard_sizes(2, 1, 2, out) == mla.MLA_EINVAL
    assert list(out) == [-7, -7]
    assert b"sp" in lib.mla_last_error()
    assert lib.mla_head_shard_sizes(6, 3, 2, out) == mla.MLA_OK and list(out) == [4, 2]
    assert lib.mla_last_error() == b""


FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x20000000)


def _pack(lib, tokens, Ht, F, sizes, dtype=mla.MLA_BF16, src=FAKE, dst=FAKE2):
    arr = (ctypes.c_int * len(sizes))(*sizes)
    return lib.mla_pack_heads(src, dst, tokens, Ht, F, arr, len(sizes), dtype, None)


def test_pack_validation_before_launch(lib):
    assert _pack(lib, 4, 5, 8, [3, 1]) == mla.MLA_EINVAL           # sizes do not sum to heads_total
    assert _pack(lib, 4, 4, 8, [4, 0]) == mla.MLA_EINVAL           # a rank with no heads
    assert _pack(lib, -1, 4, 8, [2, 2]) == mla.MLA_EINVAL
    assert _pack(lib, 4, 4, 0, [2, 2]) == mla.MLA_EINVAL
    assert _pack(lib, 4, 4, 8, [2, 2], dtype=7) == mla.MLA_EINVAL
    assert _pack(lib, 4, 4, 8, [2, 2], dst=FAKE) == mla.MLA_EINVAL  # overlapping buffers
    assert _pack(lib, 4, 4, 8, [2, 2], src=ctypes.c_void_p(0x10001)) == mla.MLA_EINVAL   # misaligned
    assert _pack(lib, 0, 4, 8, [2, 2]) == mla.MLA_OK                 # empty: nothing to do
    assert lib.mla_pack_heads(FAKE, FAKE2, 4, 4, 8, None, 2, 0, None) == mla.MLA_EINVAL
    assert lib.mla_pack_heads(FAKE, FAKE2, 4, 300, 8, (ctypes.c_int * 300)(*([1] * 300)), 300, 0,
                              None) == mla.MLA_EINVAL               # sp above the supported maximum


def test_up_proj_validation_before_launch(lib):
    f = lib.mla_latent_up_proj
    assert f(FAKE, FAKE, FAKE2, 16, 32, 4, 3, 2, 16, 16, 0, None) == mla.MLA_EINVAL    # head range past W
    assert f(FAKE, FAKE, FAKE2, 16, 32, 4, -1, 2, 16, 16, 0, None) == mla.MLA_EINVAL
    assert f(FAKE, FAKE, FAKE2, 16, 0, 4, 0, 2, 16, 16, 0, None) == mla.MLA_EINVAL
    assert f(FAKE, FAKE, FAKE2, 16, 30, 4, 0, 2, 16, 16, 0, None) == mla.MLA_EUNSUPPORTED   # bf16 needs L%8
    assert f(FAKE, FAKE, FAKE2, 0, 32, 4, 0, 2, 16, 16, 0, None) == mla.MLA_OK            # T = 0


def test_up_proj_linear_validation_before_launch(lib):
    f = lib.mla_latent_up_proj_linear
    assert f(FAKE, FAKE, FAKE2, 16, 32, 4, 3, 2, 16, 16, 0, None) == mla.MLA_EINVAL    # head range past W
    assert f(FAKE, FAKE, FAKE2, 16, 32, 4, -1, 2, 16, 16, 0, None) == mla.MLA_EINVAL
    assert f(FAKE, FAKE, FAKE2, 16, 32, 4, 0, 2, 16, 0, 0, None) == mla.MLA_EINVAL     # V = 0
    assert f(FAKE, None, FAKE2, 16, 32, 4, 0, 2, 16, 16, 0, None) == mla.MLA_EINVAL    # NULL weight
    assert f(FAKE, FAKE, FAKE2, 16, 30, 4, 0, 2, 16, 16, 0, None) == mla.MLA_EUNSUPPORTED   # bf16 needs L%8
    assert f(FAKE, FAKE, FAKE2, 16, 32, 4, 0, 2, 12, 16, 0, None) == mla.MLA_EUNSUPPORTED   # bf16 needs (N+V)%8
    assert f(FAKE, FAKE, FAKE2, 0, 32, 4, 0, 2, 16, 16, 0, None) == mla.MLA_OK            # T = 0
    assert f(FAKE, FAKE, FAKE2, 16, 32, 4, 0, 2, 16, 16, 7, None) == mla.MLA_EINVAL     # unknown dtype


def _attn(**kw):
    from mla_attention_under_amd._binding import mla_attn_args
    a = mla_attn_args()
    a.q, a.kv, a.k_rope, a.out = 0x10000, 0x20000, 0x30000, 0x40000
    a.T_q, a.T_k, a.H, a.N, a.R, a.V = 256, 256, 2, 128, 64, 128
    a.q_stride_h, a.q_stride_t = 192, 384
    a.kv_stride_h, a.kv_stride_t = 256, 512
    a.kr_stride_t = 64
    a.o_stride_h, a.o_stride_t = 128, 256
    a.scale, a.causal, a.dtype = 0.07, 1, mla.MLA_BF16
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_attention_validation_before_launch(lib):
    f = lambda **kw: lib.mla_attention_fwd(ctypes.byref(_attn(**kw)), None)  # noqa: E731
    assert f(R=63) == mla.MLA_EINVAL                       # odd rope band
    assert f(scale=0.0) == mla.MLA_EINVAL
    assert f(scale=float("nan")) == mla.MLA_EINVAL
    assert f(q_stride_h=100) == mla.MLA_EINVAL             # rows overlap
    assert f(kv_stride_t=300) == mla.MLA_EINVAL
    assert f(o_stride_h=64) == mla.MLA_EINVAL
    assert f(q=0x10002) == mla.MLA_EUNSUPPORTED            # misaligned for the tiled path
    assert f(cu_seqlens=0x50000, n_seq=2) == mla.MLA_EINVAL   # missing workspace (packed documents)
    assert f() == mla.MLA_EINVAL                              # missing workspace (dense causal pairing)
    assert f(workspace=0x60000, workspace_bytes=64) == mla.MLA_EINVAL   # too small
    assert f(cu_seqlens=0x50000, n_seq=0) == mla.MLA_EINVAL
    assert f(T_q=0) == mla.MLA_OK
    assert f(T_k=-1) == mla.MLA_EINVAL
    assert f(cu_seqlens_k=0x50000, n_seq=2) == mla.MLA_EINVAL          # key offsets without query offsets
    assert f(cu_seqlens=0x50000, n_seq=2, T_k=300, workspace=0x60000, workspace_bytes=1 << 20) == mla.MLA_EINVAL
    assert lib.mla_attention_fwd(None, None) == mla.MLA_EINVAL
    # output in query chunks (the unpacked layout): chunk rows must not overlap
    assert f(o_chunk_tokens=-1) == mla.MLA_EINVAL
    assert f(o_chunk_tokens=128, o_stride_chunk=0) == mla.MLA_EINVAL and b"chunk" in lib.mla_last_error()
    assert f(o_chunk_tokens=128, o_stride_chunk=256) == mla.MLA_EINVAL and b"chunk" in lib.mla_last_error()
    assert f(o_chunk_tokens=128, o_stride_chunk=200, o_stride_t=512) == mla.MLA_EINVAL   # heads of two chunks overlap
    # side by side (sp=2: [128][2*2][128]) and one after another pass the layout check (then need the workspace)
    assert f(o_chunk_tokens=128, o_stride_chunk=256, o_stride_t=512) == mla.MLA_EINVAL
    assert b"workspace" in lib.mla_last_error()
    assert f(o_chunk_tokens=128, o_stride_chunk=128 * 256) == mla.MLA_EINVAL and b"workspace" in lib.mla_last_error()
    assert f(o_chunk_tokens=300, o_stride_chunk=0) == mla.MLA_EINVAL and b"workspace" in lib.mla_last_error()
    assert f(o_chunk_tokens=128, o_stride_chunk=260, o_stride_t=520) == mla.MLA_EUNSUPPORTED   # tiles need % 8
    a = _attn(cu_seqlens=0x50000, n_seq=4, T_q=16384, T_k=16384)
    assert lib.mla_attention_workspace_size(ctypes.byref(a)) > 0
    assert lib.mla_attention_workspace_size(ctypes.byref(_attn())) > 0          # dense causal
    assert lib.mla_attention_workspace_size(ctypes.byref(_attn(causal=0))) == 0  # non-causal needs none
    assert lib.mla_attention_workspace_size(ctypes.byref(_attn(N=16, R=8, V=16))) == 0   # generic kernel
    # the no-alloc variant: beyond its fixed scratch (128 heads at T=4096, dense causal) it launches nothing
    g = lambda **kw: lib.mla_attention_fwd_noalloc(ctypes.byref(_attn(**kw)), None)  # noqa: E731
    assert g(T_q=4096, T_k=4096, H=128, q_stride_t=128 * 192, kv_stride_t=128 * 256,
             o_stride_t=128 * 128) == mla.MLA_EUNSUPPORTED
    assert b"scratch" in lib.mla_last_error()
    assert g(R=63) == mla.MLA_EINVAL                       # validated like mla_attention_fwd
    assert lib.mla_attention_fwd_noalloc(None, None) == mla.MLA_EINVAL


def _attn_bwd(**kw):
    from mla_attention_under_amd._binding import mla_attn_bwd_args
    a = mla_attn_bwd_args()
    a.q, a.kv, a.k_rope, a.out, a.dout = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000
    a.lse, a.dq, a.dkv, a.dk_rope = 0x60000, 0x70000, 0x80000, 0x90000
    a.T, a.H, a.N, a.R, a.V = 256, 2, 128, 64, 128
    a.q_stride_h, a.q_stride_t = 192, 384
    a.kv_stride_h, a.kv_stride_t = 256, 512
    a.kr_stride_t = 64
    a.o_stride_h, a.o_stride_t = 128, 256
    a.do_stride_h, a.do_stride_t = 128, 256
    a.scale, a.causal, a.dtype = 0.07, 1, mla.MLA_BF16
    a.workspace = 0x100000
    a.workspace_bytes = lib_ws(a) if kw.pop("sized", True) else 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def lib_ws(a):
    return mla.load_library().mla_attention_bwd_workspace_size(ctypes.byref(a))


def test_attention_bwd_validation_before_launch(lib):
    f = lambda **kw: lib.mla_attention_bwd(ctypes.byref(_attn_bwd(**kw)), None)  # noqa: E731
    a = _attn_bwd()
    # row terms [H][T] and per-head band gradients [H][T][R], fp32, each padded to 256 bytes
    assert lib.mla_attention_bwd_workspace_size(ctypes.byref(a)) == 256 * 2 * 4 + 256 * 2 * 64 * 4
    assert f(scale=0.0) == mla.MLA_EINVAL
    assert f(q_stride_h=100) == mla.MLA_EINVAL              # rows overlap
    assert f(do_stride_t=200) == mla.MLA_EINVAL
    assert f(N=64) == mla.MLA_EUNSUPPORTED                  # no kernel for these widths
    assert f(dtype=mla.MLA_F32) == mla.MLA_EUNSUPPORTED
    assert f(dout=0x50002) == mla.MLA_EUNSUPPORTED          # misaligned
    assert f(dk_rope=0x90004) == mla.MLA_EUNSUPPORTED       # misaligned fp32 output
    assert f(lse=None) == mla.MLA_EINVAL                     # the forward's lse is required
    assert f(dk_rope=None) == mla.MLA_EINVAL
    assert f(sized=False) == mla.MLA_EINVAL                  # workspace too small
    assert f(workspace=0x100010) == mla.MLA_EINVAL           # workspace misaligned
    assert f(cu_seqlens=0x50000, n_seq=0) == mla.MLA_EINVAL
    assert f(kv_stride_t=(1 << 24) + 8) == mla.MLA_EUNSUPPORTED   # beyond the stages' 32-bit row offsets
    assert f(do_stride_t=(1 << 24) + 8) == mla.MLA_EUNSUPPORTED
    assert f(T=0, sized=False) == mla.MLA_OK
    assert lib.mla_attention_bwd(None, None) == mla.MLA_EINVAL


def test_up_proj_bwd_validation_before_launch(lib):
    f = lambda *a: lib.mla_latent_up_proj_bwd(0x10000, 0x20000, 0x30000, 0x40000, 0x50000, *a,  # noqa: E731
                                              None, 0, None)
    # T, L, heads_total, head_begin, heads, N, V, dtype
    assert f(64, 512, 128, 16, 16, 128, 128, mla.MLA_F32) == mla.MLA_EUNSUPPORTED   # bf16 only
    assert f(64, 500, 128, 16, 16, 128, 128, mla.MLA_BF16) == mla.MLA_EUNSUPPORTED   # L % 32
    assert f(64, 512, 4, 0, 1, 8, 8, mla.MLA_BF16) == mla.MLA_EUNSUPPORTED          # heads*(N+V) % 32
    assert f(64, 512, 128, 120, 16, 128, 128, mla.MLA_BF16) == mla.MLA_EINVAL       # head range outside
    assert f(-1, 512, 128, 16, 16, 128, 128, mla.MLA_BF16) == mla.MLA_EINVAL
    assert lib.mla_latent_up_proj_bwd(0x10008, 0x20000, 0x30000, 0x40000, 0x50000, 64, 512, 128, 16, 16, 128, 128,
                                      mla.MLA_BF16, None, 0, None) == mla.MLA_EUNSUPPORTED   # misaligned latent
    assert lib.mla_latent_up_proj_bwd(0x10000, 0x20000, 0x30000, 0x40000, None, 64, 512, 128, 16, 16, 128, 128,
                                      mla.MLA_BF16, None, 0, None) == mla.MLA_EINVAL          # no dw
    assert lib.mla_latent_up_proj_bwd(0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 64, 512, 128, 16, 16, 128, 128,
                                      mla.MLA_BF16, 0x60010, 1 << 20, None) == mla.MLA_EINVAL   # misaligned workspace


def test_up_proj_bwd_workspace_size(lib):
    ws = lib.mla_latent_up_proj_bwd_workspace_size
    # the rank shard: d_latent split 4 ways (64 tiles of 128x128), dw 2 ways (128 tiles): 4 x [2048][512] fp32
    assert ws(2048, 512, 16, 128, 128) == 4 * 2048 * 512 * 4
    assert ws(2048, 512, 16, 128, 128) >= 2 * 512 * 4096 * 4
    # not a multiple of 128 in T, L or heads*(N+V): the single-pass kernels, no workspace
    assert ws(2000, 512, 16, 128, 128) == 0
    assert ws(2048, 480, 16, 128, 128) == 0
    assert ws(2048, 512, 1, 32, 32) == 0
    # enough tiles in both products without splitting: no workspace
    assert ws(65536, 512, 128, 128, 128) == 0
    assert ws(-1, 512, 16, 128, 128) == 0


def test_decode_validation_before_launch(lib):
    from mla_attention_under_amd._binding import mla_decode_args

    def args(**kw):
        a = mla_decode_args()
        a.q, a.latent_cache, a.rope_cache, a.w_kvb, a.out = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000
        a.B, a.S, a.L, a.H, a.heads_total, a.head_begin = 32, 8192, 512, 16, 16, 0
        a.N, a.R, a.V, a.num_splits, a.scale, a.dtype = 128, 64, 128, 8, 0.07, mla.MLA_BF16
        for k, v in kw.items():
            setattr(a, k, v)
        return a
    f = lambda **kw: lib.mla_latent_decode_fwd(ctypes.byref(args(**kw)), None)  # noqa: E731
    assert f() == mla.MLA_EINVAL                            # no workspace
    assert f(head_begin=1) == mla.MLA_EINVAL                # head range past W
    assert f(num_splits=0) == mla.MLA_EINVAL
    assert f(S=4, num_splits=8) == mla.MLA_EINVAL
    assert f(dtype=mla.MLA_F32) == mla.MLA_EUNSUPPORTED
    assert f(L=256) == mla.MLA_EUNSUPPORTED
    assert f(num_splits=257) == mla.MLA_EUNSUPPORTED
    assert f(B=(1 << 20) + 1) == mla.MLA_EUNSUPPORTED       # beyond the per-call sequence count
    assert f(B=0) == mla.MLA_OK
    assert lib.mla_latent_decode_workspace_size(ctypes.byref(args())) > 0


# ---- expanded pack validation, and the host interval algebra against the oracle

def _pack_exp(lib, tokens, Ht, N, R, V, sizes, dtype=mla.MLA_BF16, q=FAKE, kv=FAKE2, kr=FAKE2, send=None):
    arr = (ctypes.c_int * len(sizes))(*sizes) if sizes is not None else None
    send = send if send is not None else ctypes.c_void_p(0x7f0000000000)
    return lib.mla_pack_expanded(q, kv, kr, send, tokens, Ht, N, R, V, arr, len(sizes or [1]), dtype, None)


def test_pack_expanded_validation_before_launch(lib):
    assert _pack_exp(lib, 4, 5, 8, 4, 8, [3, 1]) == mla.MLA_EINVAL      # sizes do not sum to heads_total
    assert _pack_exp(lib, 4, 4, 0, 4, 8, [2, 2]) == mla.MLA_EINVAL      # N < 1
    assert _pack_exp(lib, 4, 4, 8, 0, 8, [2, 2]) == mla.MLA_EINVAL      # R < 1
    assert _pack_exp(lib, 4, 4, 8, 4, 0, [2, 2]) == mla.MLA_EINVAL      # V < 1
    assert _pack_exp(lib, 4, 4, 8, 4, 8, [2, 2], dtype=9) == mla.MLA_EINVAL
    assert _pack_exp(lib, 4, 4, 8, 4, 8, [2, 2], send=FAKE) == mla.MLA_EINVAL        # send overlaps q
    assert _pack_exp(lib, 4, 4, 8, 4, 8, [2, 2], kr=ctypes.c_void_p(0x10001)) == mla.MLA_EINVAL   # misaligned
    assert _pack_exp(lib, 4, 4, 8, 4, 8, None) == mla.MLA_EINVAL
    assert _pack_exp(lib, 0, 4, 8, 4, 8, [2, 2]) == mla.MLA_OK          # empty: nothing to do


def _random_layout(rng):
    copies = int(rng.integers(1, 4))
    qparts = int(rng.integers(1, 5))
    degree = copies * qparts
    Lq = degree * int(rng.integers(1, 8))
    total = qparts * Lq
    n = int(rng.integers(1, min(total, 6) + 1))
    cuts = sorted(int(x) for x in rng.choice(np.arange(1, total), size=n - 1, replace=False)) if n > 1 else []
    return cuts + [total], Lq, copies, degree, total // degree


@pytest.mark.parametrize("seed", range(16))
def test_causal_partition_matches_oracle(seed):
    rng = np.random.default_rng(300 + seed)
    ends, Lq, _, _, _ = _random_layout(rng)
    batch = int(rng.integers(1, 4))
    for r in range(ends[-1] // Lq):
        got = mla.mla_causal_partition(ends, Lq, r, batch)
        exp = oracle.causal_partition(ends, Lq, r, batch)
        assert got == {k: exp[k] for k in ("key_begin", "key_end", "query_ends", "key_ends")}, (ends, Lq, r)


@pytest.mark.parametrize("seed", range(16))
def test_kv_exchange_ranges_match_oracle(seed):
    rng = np.random.default_rng(400 + seed)
    ends, Lq, copies, degree, S = _random_layout(rng)
    for r in range(degree):
        got = mla.mla_kv_exchange_ranges(ends, S, Lq, copies, degree, r)
        assert got == oracle.kv_exchange_ranges(tuple(ends), S, Lq, copies, degree, r), (ends, S, Lq, copies, r)


def test_interval_algebra_errors_leave_outputs_untouched(lib):
    ends = (ctypes.c_int64 * 2)(10, 20)
    kb, ke, n = ctypes.c_int64(-5), ctypes.c_int64(-5), ctypes.c_int(-5)
    qe, kend = (ctypes.c_int64 * 4)(*[-5] * 4), (ctypes.c_int64 * 4)(*[-5] * 4)
    # queries [16, 24) are not covered by documents ending at 20
    assert lib.mla_causal_partition(ends, 2, 8, 2, 1, ctypes.byref(kb), ctypes.byref(ke), qe, kend, 4,
                                    ctypes.byref(n)) == mla.MLA_EINVAL
    assert "cover" in lib.mla_last_error().decode()
    # capacity too small: queries [0, 16) touch two documents, batch 3 needs 6 entries
    assert lib.mla_causal_partition(ends, 2, 16, 0, 3, ctypes.byref(kb), ctypes.byref(ke), qe, kend, 4,
                                    ctypes.byref(n)) == mla.MLA_EINVAL
    assert (kb.value, ke.value, n.value, list(qe), list(kend)) == (-5, -5, -5, [-5] * 4, [-5] * 4)
    bad = (ctypes.c_int64 * 2)(10, 5)                       # decreasing ends
    assert lib.mla_causal_partition(bad, 2, 5, 0, 1, ctypes.byref(kb), ctypes.byref(ke), qe, kend, 4,
                                    ctypes.byref(n)) == mla.MLA_EINVAL
    so, sc, rc = (ctypes.c_int64 * 2)(-5, -5), (ctypes.c_int64 * 2)(-5, -5), (ctypes.c_int64 * 2)(-5, -5)
    loc = ctypes.c_int(-5)
    assert lib.mla_kv_exchange_ranges(ends, 2, 10, 10, 1, 2, 2, so, sc, rc, ctypes.byref(loc)) == mla.MLA_EINVAL
    assert lib.mla_kv_exchange_ranges(ends, 2, 10, 12, 1, 2, 0, so, sc, rc, ctypes.byref(loc)) == mla.MLA_EINVAL
    assert (list(so), list(sc), list(rc), loc.value) == ([-5, -5], [-5, -5], [-5, -5], -5)


def test_rope_validation_before_launch(lib):
    f = lib.mla_apply_rope
    X, C, S = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000)
    ok = dict(tokens=4, heads=2, st=384, sh=192, R=64, cs=64, inter=0, dt=mla.MLA_BF16)

    def call(**kw):
        a = dict(ok, **kw)
        return f(kw.get("x", X), a["tokens"], a["heads"], a["st"], a["sh"], a["R"], kw.get("c", C), S, a["cs"],
                 a["inter"], a["dt"], None)
    assert call(R=63) == mla.MLA_EINVAL            # odd band
    assert call(R=258) == mla.MLA_EINVAL           # wider than supported
    assert call(heads=0) == mla.MLA_EINVAL
    assert call(inter=2) == mla.MLA_EINVAL
    assert call(dt=5) == mla.MLA_EINVAL
    assert call(sh=32) == mla.MLA_EINVAL           # head rows overlap
    assert call(st=200) == mla.MLA_EINVAL          # token rows overlap
    assert call(cs=8) == mla.MLA_EINVAL            # table rows overlap
    assert call(c=X) == mla.MLA_EINVAL             # band overlaps a table
    assert call(x=ctypes.c_void_p(0x100001)) == mla.MLA_EINVAL   # misaligned
    assert call(tokens=0) == mla.MLA_OK


def test_project_pack_validation_before_launch(lib):
    f = lib.mla_project_pack
    A, Wp, S = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x4000000), ctypes.c_void_p(0x8000000)
    C, Sn = ctypes.c_void_p(0xc000000), ctypes.c_void_p(0xd000000)
    sizes = (ctypes.c_int * 2)(2, 2)
    base = dict(T=8, L=512, wh=4, hb=0, heads=4, P=192, F=448, col=0, ro=128, R=64, cs=64, inter=0, dt=mla.MLA_BF16)

    def call(sz=sizes, sp=2, **kw):
        a = dict(base, **kw)
        return f(A, Wp, kw.get("send", S), a["T"], a["L"], a["wh"], a["hb"], a["heads"], a["P"], a["F"], a["col"],
                 sz, sp, a["ro"], a["R"], C, Sn, a["cs"], a["inter"], a["dt"], None)
    assert call(hb=1) == mla.MLA_EINVAL                 # head range outside the weight
    assert call(col=300) == mla.MLA_EINVAL              # part wider than the payload row
    assert call(ro=160) == mla.MLA_EINVAL               # band outside the block
    assert call(sz=(ctypes.c_int * 2)(3, 2)) == mla.MLA_EINVAL   # sizes do not sum to heads
    assert call(dt=mla.MLA_F32) == mla.MLA_EUNSUPPORTED
    assert call(L=500) == mla.MLA_EUNSUPPORTED          # not a multiple of 8
    assert call(P=184, ro=120) == mla.MLA_EUNSUPPORTED  # block width not a multiple of 64
    assert call(ro=96, R=64, P=192) == mla.MLA_EUNSUPPORTED   # band not at a multiple of 64
    assert call(R=32, ro=128) == mla.MLA_EUNSUPPORTED   # band width other than 64
    assert call(send=A) == mla.MLA_EINVAL               # send overlaps the latent
    # tiles address rows by 32-bit byte offsets; the grid holds at most 2^31 - 1 workgroups
    assert call(L=1 << 24) == mla.MLA_EUNSUPPORTED      # 128 latent rows of 32 MiB
    assert call(wh=1 << 18) == mla.MLA_EUNSUPPORTED     # 64 weight rows of 96 MiB
    big = (ctypes.c_int * 2)(128, 128)
    assert call(sz=big, T=1 << 30, wh=256, heads=256) == mla.MLA_EUNSUPPORTED   # 2^23 x 384 tiles
    assert call(T=0) == mla.MLA_OK


def test_binding_rejects_mismatched_tensors_before_any_call(monkeypatch):
    """The C ABI sees pointers, not sizes: the binding checks shapes and dtypes first (invalid cases only, so no
    call ever reaches the library; host tensors stand in with the device check switched off)."""
    import torch
    from mla_attention_under_amd import _binding as b
    monkeypatch.setattr(b, "_dev", lambda *ts: None)
    bf = dict(dtype=torch.bfloat16)
    T, H, N, R, V = 8, 2, 128, 64, 128
    q, kv, kr = torch.zeros(T, H, N + R, **bf), torch.zeros(T, H, N + V, **bf), torch.zeros(T, R, **bf)
    out, lse = torch.zeros(T, H, V, **bf), torch.zeros(H, T)
    fwd = lambda **kw: b.mla_attention_fwd(**dict(dict(q=q, kv=kv, k_rope=kr, out=out, N=N, R=R, V=V,  # noqa: E731
                                                        scale=0.1, lse=lse), **kw))
    for bad in (dict(out=torch.zeros(T, H, V // 2, **bf)),                # output rows too narrow
                dict(out=torch.zeros(T - 1, H, V, **bf)),                 # too few output rows
                dict(kv=torch.zeros(T, H + 1, N + V, **bf)),              # heads disagree
                dict(k_rope=torch.zeros(T + 1, R, **bf)),                 # band rows disagree with kv
                dict(q=torch.zeros(T, H, N + R)),                         # fp32 q with bf16 kv
                dict(lse=torch.zeros(H, T - 1)),                          # lse too small
                dict(cu_seqlens=torch.tensor([0, T], dtype=torch.int32),
                     cu_seqlens_k=torch.tensor([0, 4, T], dtype=torch.int32)),    # different document counts
                dict(unpack_sp=3, out=torch.zeros(2, 3 * H, V, **bf)),        # T not a multiple of sp
                dict(unpack_sp=2, out=torch.zeros(T, H, V, **bf)),            # not the [T/sp][sp*H][V] layout
                dict(unpack_sp=4, out=torch.zeros(T // 4, 4 * H, V - 8, **bf))):   # rows too narrow
        with pytest.raises(ValueError):
            fwd(**bad)
    with pytest.raises(ValueError):
        b.mla_attention_fwd_noalloc(q, kv, kr, torch.zeros(T, H, 64, **bf), N, R, V, 0.1)
    f32 = dict(dtype=torch.float32)
    bwd = lambda **kw: b.mla_attention_bwd(**dict(dict(q=q, kv=kv, k_rope=kr, out=out, dout=out, lse=lse,  # noqa
                                                        N=N, R=R, V=V, scale=0.1), **kw))
    for bad in (dict(dq=torch.zeros(T, H, N, **f32)), dict(dkv=torch.zeros(T, H - 1, N + V, **f32)),
                dict(dk_rope=torch.zeros(T - 1, R, **f32)), dict(dout=torch.zeros(T, H, V - 8, **bf)),
                dict(lse=None), dict(kv=torch.zeros(T + 8, H, N + V, **bf), k_rope=torch.zeros(T + 8, R, **bf))):
        with pytest.raises(ValueError):
            bwd(**bad)
    lat, w = torch.zeros(T, 512, **bf), torch.zeros(512, 4 * (N + V), **bf)
    with pytest.raises(ValueError):
        b.mla_latent_up_proj(lat, w.float(), torch.zeros(T, H, N + V, **bf), 4, 0, H, N, V)
    with pytest.raises(ValueError):
        b.mla_latent_up_proj_bwd(lat, w, torch.zeros(T, H, N + V, **f32), 4, 0, H, N, V,
                                 dw=torch.zeros(512, N + V, **f32))
    B, S = 2, 64
    dq_ = torch.zeros(B, H, N + R, **bf)
    cache, rope = torch.zeros(B, S, 512, **bf), torch.zeros(B, S, R, **bf)
    for bad in (dict(out=torch.zeros(B, H, V - 8, **bf)), dict(rope_cache=torch.zeros(B, S - 1, R, **bf)),
                dict(lse=torch.zeros(B * H - 1)), dict(w_kvb=torch.zeros(512, 3 * (N + V), **bf))):
        args = dict(q=dq_, latent_cache=cache, rope_cache=rope, w_kvb=w, out=torch.zeros(B, H, V, **bf),
                    heads_total=4, head_begin=0, N=N, R=R, V=V, num_splits=2, scale=0.1)
        args.update(bad)
        with pytest.raises(ValueError):
            b.mla_latent_decode_fwd(**args)
