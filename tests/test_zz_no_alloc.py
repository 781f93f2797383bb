"""mla_attention_fwd_noalloc: the attention call that allocates nothing (its
scratch is the library's fixed per-GPU array) against mla_attention_fwd with a
caller workspace, on calls in a row of decreasing size, and under graph capture."""
import math

import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from gpu_helpers import check_close, dev, host64

pytestmark = pytest.mark.gpu

mla = pytest.importorskip("mla_attention_under_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load_library()
    yield
    torch.cuda.synchronize()


def _workload(T, H):
    b = mi.WORKLOADS["dsv3_rank"]
    return mi.Workload(b.name, b.cfg, T=T, H=H, L=b.L, N=b.N, R=b.R, V=b.V, heads_total=H)


# dense causal at the rank shard (split-tile records and flags in the scratch), then a smaller dense causal
# call and a smaller packed-document call (the device-built schedule in the scratch)
CALLS = [(2048, 16, None), (1000, 3, None), (531, 2, [0, 100, 101, 101, 400, 531])]


def test_noalloc_matches_the_workspace_call_on_calls_in_a_row():
    for i, (T, H, cu) in enumerate(CALLS):
        print(f"noalloc call {i}: T={T} H={H} cu={cu}", flush=True)
        w = _workload(T, H)
        d = mi.shard_inputs(w, T=T, seed_cfg=200 + i)
        d["kv"] = mi.draw((T, H, w.P), 200 + i, 9)
        q, kv, kr = dev(d["q"]), dev(d["kv"]), dev(d["k_rope"])
        cud = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
        scale = 1 / math.sqrt(w.K)
        ref = torch.full((T, H, w.V), float("nan"), dtype=torch.bfloat16, device="cuda")
        ref_lse = torch.full((H, T), float("nan"), dtype=torch.float32, device="cuda")
        got = torch.full_like(ref, float("nan"))
        got_lse = torch.full_like(ref_lse, float("nan"))
        mla.mla_attention_fwd(q, kv, kr, ref, w.N, w.R, w.V, scale, lse=ref_lse, cu_seqlens=cud)
        mla.mla_attention_fwd_noalloc(q, kv, kr, got, w.N, w.R, w.V, scale, lse=got_lse, cu_seqlens=cud)
        torch.cuda.synchronize()
        # the same kernels on the same inputs: identical bits
        assert torch.equal(got, ref), f"call {i}: output differs from mla_attention_fwd"
        assert torch.equal(got_lse, ref_lse), f"call {i}: lse differs from mla_attention_fwd"
        # and within the bf16 bar of the oracle (every 128-row tile's first and last row)
        rows = np.unique(np.concatenate([np.arange(0, T, 128), np.minimum(np.arange(0, T, 128) + 127, T - 1),
                                         [T - 1]]))
        oref, olse = oracle.attention(d["q"], d["kv"], d["k_rope"], w.N, scale, cu_seqlens=cu, rows=rows)
        check_close(host64(got)[rows], oref[rows], name=f"noalloc call {i} vs oracle")
        check_close(got_lse.cpu().numpy().astype(np.float64)[:, rows], olse[:, rows], name=f"noalloc lse {i}")


def test_noalloc_rejects_calls_beyond_the_scratch():
    # 128 heads at T = 4096, dense causal: 277 MB of split-tile records, more than the 48 MiB scratch
    w = _workload(4096, 128)
    q = torch.zeros((w.T, w.H, w.K), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((w.T, w.H, w.P), dtype=torch.bfloat16, device="cuda")
    kr = torch.zeros((w.T, w.R), dtype=torch.bfloat16, device="cuda")
    out = torch.full((w.T, w.H, w.V), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MlaError) as e:
        mla.mla_attention_fwd_noalloc(q, kv, kr, out, w.N, w.R, w.V, 0.1)
    assert e.value.code == mla.MLA_EUNSUPPORTED and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a rejected call wrote output"


def test_noalloc_under_graph_capture():
    """Captured once (no allocation inside the capture), replayed twice with new inputs."""
    T, H = 2048, 16
    w = _workload(T, H)
    scale = 1 / math.sqrt(w.K)
    d0 = mi.shard_inputs(w, T=T, seed_cfg=300)
    q, kr = dev(d0["q"]), dev(d0["k_rope"])
    kv = dev(mi.draw((T, H, w.P), 300, 9))
    out = torch.full((T, H, w.V), float("nan"), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mla.mla_attention_fwd_noalloc(q, kv, kr, out, w.N, w.R, w.V, scale)
    torch.cuda.synchronize()
    for i in range(2):
        d = mi.shard_inputs(w, T=T, seed_cfg=301 + i)
        d["kv"] = mi.draw((T, H, w.P), 301 + i, 9)
        q.copy_(dev(d["q"]))
        kv.copy_(dev(d["kv"]))
        kr.copy_(dev(d["k_rope"]))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref, _ = oracle.attention(d["q"], d["kv"], d["k_rope"], w.N, scale)
        check_close(host64(out), ref, name=f"noalloc replay {i}")
