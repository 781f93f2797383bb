#!/usr/bin/env python3
"""Throughput of one Ulysses rank's MLA shard on one MI355X.

A step is one pass of the whole hot path over one batch of seeded synthetic
input, all in libmla.so:
  1. pack      : token->head pack of the rank's local [q | kv] rows,
                 [256 tokens][128 heads][448] -> 8 slabs of 16 heads
  2. up-proj   : latent [2048][512] x wkv_b [512][16*256] -> kv [2048][16][256]
  3. attention : causal, shared 64-wide RoPE band, q [2048][16][192] -> out, written
                 straight into the head->token restored layout [256][128][128] (the
                 unpack of 8 x [256][16][128], fused into the attention's row stores)
(the DeepSeek-V3-shaped rank of 128 heads over sp=8: T=2048, H=16, L=512,
N=128, R=64, V=128, bf16 storage with fp32 accumulation).

value = algorithmic FLOPs of the step (up-projection 2*T*L*H*(N+V) plus
attention 2*H*T(T+1)/2*(N+R+V), unmasked pairs only) / measured step time.
The timed region is K steps launched back to back on one stream, with the
inputs resident in HBM, bracketed by HIP events after a synchronize.
A second pass times every kernel on its own with events for the roofline.
Extra fields, outside value: the uneven 22-head pack/unpack beyond the
Infinity Cache, packed-document attention (T=16384) and latent-cache decode
(32 x 8192 positions, cache swept before each call).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(kernel: str, workload: str, launches_per_unit=1):
    """HBM bytes per launch from committed rocprofv3 counters, if taken on the current source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{kernel}@{workload}")
    if not rec:
        return None
    src = os.path.join(ROOT, "mla_attention_under_amd", "csrc", rec["source"])
    if not os.path.exists(src) or _sha(src) != rec["source_sha"]:
        return None
    return rec["bytes_per_launch"]


_lead_buf = []


def _busy(torch, ms=30):
    """Keep the GPU loaded for roughly `ms` so the host can queue the timed launches ahead of it.

    The lead is a stream of 256 MB fills (about 0.05-0.1 ms each), not an idle spin. After 30 ms of one
    spinning wave the chip had lowered its clock, and the steps of the next 10 ms ran up to 20 % slower
    (events every 20 steps: 58.7, 61.6, 64.8, 65.0, ... 55.7 us), which put about 6 % on a 200-step
    average. Behind the fills the step runs at its steady rate from the first event on. The fills also
    evict the Infinity Cache, so the first timed launch finds its inputs in HBM.
    """
    if not _lead_buf:
        _lead_buf.append(torch.empty(1 << 26, dtype=torch.float32, device="cuda"))
    x = _lead_buf[0]
    for _ in range(max(1, 10 * ms)):
        x.fill_(1.0)


def cpu_baseline(w, d, x_pack, sizes, flops_step):
    """The fp64 oracle on the host cores over the same workload, for about 10 s."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    scale = 1 / math.sqrt(w.K)
    out_slabs = np.zeros((w.T, w.H, w.V), dtype=np.float64)

    def one_step():
        oracle.pack_heads(x_pack, sizes)
        kv = oracle.latent_up_proj(d["latent"], d["w_kvb"], 0, w.H, w.N, w.V)
        out, _ = oracle.attention(d["q"], kv, d["k_rope"], w.N, scale)
        out_slabs[:] = out
        oracle.unpack_heads(out_slabs.reshape(-1), [w.H] * 8, w.T // 8, w.V)

    t0 = time.perf_counter()
    n = 0
    while True:
        one_step()
        n += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or (n >= 1 and el / n > 15.0):
            break
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu_model)
    except OSError:  # pragma: no cover - not Linux
        pass
    return {"value": round(flops_step * n / el / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model, "host_cpus": os.cpu_count(),
            "sample": f"{n} full step(s) of the same workload (pack, up-projection, attention of all "
                      f"{w.H} heads, unpack) in float64 NumPy, {el:.1f} s"}


def _median_us(torch, fn, reps, before=None):
    """Median of reps event-timed calls on the current stream; before() runs untimed ahead of each."""
    ts = []
    for _ in range(reps):
        if before is not None:
            before()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    ts.sort()
    return ts[len(ts) // 2]


def _pct(xs):
    """p10 / median / p90 / mean of a list of durations (us)."""
    xs = sorted(xs)
    n = len(xs)
    q = lambda f: xs[min(n - 1, int(round(f * (n - 1))))]  # noqa: E731
    return {"p10": round(q(0.1), 3), "median": round(q(0.5), 3), "p90": round(q(0.9), 3),
            "mean": round(sum(xs) / n, 3)}


def _mfma_peak(torch, mla):
    """Dense bf16 MFMA rate and shader clock under an all-MFMA load (include/mla_peak.h): 256 workgroups of 8
    waves, each wave four independent 32x32x16 MFMA chains from registers. Median of 5 event-timed launches."""
    blocks, iters = 256, 4000
    clocks = torch.empty(blocks * 16, dtype=torch.int64, device="cuda")
    sink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    for _ in range(3):
        mla.mla_peak_mfma_bf16(blocks, iters, clocks, sink)
    ts = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        mla.mla_peak_mfma_bf16(blocks, iters, clocks, sink)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    sec = sorted(ts)[len(ts) // 2]
    c = clocks.view(blocks * 8, 2).double().cpu()
    ghz = float((c[:, 0] / (c[:, 1] / 100e6)).mean()) / 1e9
    flops = 2.0 * 32 * 32 * 16 * 4 * iters * 8 * blocks
    tf = flops / sec / 1e12
    return {"tflops": round(tf, 1), "clock_ghz": round(ghz, 3),
            "spec_tflops_at_clock": round(PEAK_BF16_TFLOPS * ghz / 2.4, 1),
            "note": "256 x 8 waves of four independent 32x32x16 bf16 MFMA chains, no memory traffic; clock from "
                    "s_memtime / s_memrealtime; the data-sheet 2500 TFLOP/s assumes 2.4 GHz"}


def _flushed(torch, fn, reps, sweep):
    """Event-timed calls of fn, each after a read-only sweep of `sweep` (512 MB, twice the 256 MB Infinity Cache)
    so the call starts with cold caches (a writing sweep would leave dirty lines to write back during the call)."""
    ts = []
    for _ in range(reps):
        sweep.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    return _pct(ts)


def _expanded(torch, mla):
    """Expanded pack ([q | k_nope | k_rope | v] per head -> head slabs), back-to-back event timing.
    Bytes = q + kv + one k_rope row per token read, payload written."""
    out = {}
    for name, tokens, sizes in (("uneven22", 4096, [22, 22, 21, 21, 21, 21]), ("dsv3_rank", 256, [16] * 8)):
        Ht, N, R, V = sum(sizes), 128, 64, 128
        g = torch.Generator(device="cuda").manual_seed(5)
        q = torch.randint(-32768, 32767, (tokens, Ht, N + R), dtype=torch.int16, device="cuda", generator=g)
        kv = torch.randint(-32768, 32767, (tokens, Ht, N + V), dtype=torch.int16, device="cuda", generator=g)
        kr = torch.randint(-32768, 32767, (tokens, R), dtype=torch.int16, device="cuda", generator=g)
        send = torch.empty(tokens * Ht * (2 * (N + R) + V), dtype=torch.int16, device="cuda")
        reps = 20 if tokens > 1024 else 200
        for _ in range(3):
            mla.mla_pack_expanded(q, kv, kr, send, sizes, N)
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        _busy(torch, 10)
        st.record()
        for _ in range(reps):
            mla.mla_pack_expanded(q, kv, kr, send, sizes, N)
        en.record()
        torch.cuda.synchronize()
        us = st.elapsed_time(en) * 1e3 / reps
        nbytes = 2.0 * (q.numel() + kv.numel() + kr.numel() + send.numel())
        out[f"{name}_expanded_pack_us"] = round(us, 2)
        out[f"{name}_expanded_pack_gbps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        if tokens > 1024:
            out[f"{name}_expanded_pack_hbm_frac"] = round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
        del q, kv, kr, send
    out["expanded_pack_note"] = ("payload [q | k_nope | k_rope | v] = 512 per head; uneven22 beyond the Infinity "
                                 "Cache, dsv3_rank cache-resident")
    return out


def _rope(torch, mla):
    """In-place RoPE of q's band for all 128 heads of 4096 tokens (the pack side), both conventions.
    Bytes = band read + band written + the two [T][R] tables."""
    T, H, N, R = 4096, 128, 128, 64
    g = torch.Generator(device="cuda").manual_seed(6)
    q = torch.randn((T, H, N + R), device="cuda", generator=g).bfloat16()
    ang = torch.arange(T, device="cuda", dtype=torch.float32)[:, None] * (
        10000.0 ** (-torch.arange(0, R, 2, device="cuda", dtype=torch.float32) / R))[None, :]
    ang = torch.cat([ang, ang], dim=1)
    c, s = ang.cos().bfloat16(), ang.sin().bfloat16()
    out = {}
    for inter in (False, True):
        reps = 50
        for _ in range(3):
            mla.mla_apply_rope(q[..., N:], c, s, interleaved=inter)
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        _busy(torch, 10)
        st.record()
        for _ in range(reps):
            mla.mla_apply_rope(q[..., N:], c, s, interleaved=inter)
        en.record()
        torch.cuda.synchronize()
        us = st.elapsed_time(en) * 1e3 / reps
        nbytes = 2.0 * (2 * T * H * R + 2 * T * R)
        key = "rope_interleaved" if inter else "rope_half_band"
        out[f"{key}_us"] = round(us, 2)
        out[f"{key}_gbps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
    out["rope_note"] = "q band of 128 heads x 4096 tokens in place (67 MB each way), beyond the Infinity Cache"
    del q, c, s
    return out


def _project_pack(torch, mla):
    """The rank's send buffer straight from latents: q_b_proj + RoPE and wkv_b written into the 8 head slabs of
    [256 tokens][128 heads][448] (DeepSeek-V3 widths: q latent 1536, kv latent 512). Against the separate calls
    (two projections, the rotation, the pack of an already assembled payload)."""
    T, Hq, Lq, Lkv, N, R, V, sp = 256, 128, 1536, 512, 128, 64, 128, 8
    F = 2 * N + R + V
    g = torch.Generator(device="cuda").manual_seed(7)
    rnd = lambda *shape, std=1.0: (torch.randn(shape, device="cuda", generator=g) * std).bfloat16()
    ql, kl = rnd(T, Lq), rnd(T, Lkv)
    wq, wkv = rnd(Lq, Hq * (N + R), std=Lq ** -0.5), rnd(Lkv, Hq * (N + V), std=Lkv ** -0.5)
    ang = torch.arange(T, device="cuda", dtype=torch.float32)[:, None] * (
        10000.0 ** (-torch.arange(0, R, 2, device="cuda", dtype=torch.float32) / R))[None, :]
    ang = torch.cat([ang, ang], dim=1)
    c, s = ang.cos().bfloat16(), ang.sin().bfloat16()
    sizes = [Hq // sp] * sp
    send = torch.empty(T * Hq * F, dtype=torch.bfloat16, device="cuda")
    q = torch.empty((T, Hq, N + R), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((T, Hq, N + V), dtype=torch.bfloat16, device="cuda")
    x = torch.empty((T, Hq, F), dtype=torch.bfloat16, device="cuda")

    def fused():
        mla.mla_project_pack(ql, wq, send, Hq, 0, Hq, N + R, F, 0, sizes, rope_offset=N, cos=c, sin=s)
        mla.mla_project_pack(kl, wkv, send, Hq, 0, Hq, N + V, F, N + R, sizes)

    def separate():
        mla.mla_latent_up_proj(ql, wq, q, Hq, 0, Hq, N, R)
        mla.mla_apply_rope(q[..., N:], c, s)
        mla.mla_latent_up_proj(kl, wkv, kv, Hq, 0, Hq, N, V)
        mla.mla_pack_heads(x, send, sizes)

    out = {}
    for name, fn in (("fused", fused), ("separate", separate)):
        for _ in range(5):
            fn()
        reps = 100
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        _busy(torch, 10)
        st.record()
        for _ in range(reps):
            fn()
        en.record()
        torch.cuda.synchronize()
        out[f"project_pack_{name}_us"] = round(st.elapsed_time(en) * 1e3 / reps, 2)
    flops = 2.0 * T * (Lq * Hq * (N + R) + Lkv * Hq * (N + V))
    out["project_pack_fused_tflops"] = round(flops / (out["project_pack_fused_us"] * 1e-6) / 1e12, 1)
    out["project_pack_note"] = ("send [256][128][448] -> 8 x 16 heads from the q latent (1536, RoPE on 64) and the kv "
                                "latent (512); separate = two projections + rotation + pack of an assembled payload")
    return out


def _backward(torch, mla):
    """Backward of the rank shard's attention (T=2048, H=16, dense causal): the whole mla_attention_bwd call.
    FLOPs = the five products per visible (query, key) pair of the standard backward (scores, dp, dv, dk, dq):
    2*(3*(N+R) + 2*V) per pair, H*T(T+1)/2 pairs; the kernels also recompute scores and dp for dq."""
    T, H, N, R, V = 2048, 16, 128, 64, 128
    g = torch.Generator(device="cuda").manual_seed(8)
    q = torch.randn((T, H, N + R), device="cuda", generator=g).bfloat16()
    kv = torch.randn((T, H, N + V), device="cuda", generator=g).bfloat16()
    kr = torch.randn((T, R), device="cuda", generator=g).bfloat16()
    dout = torch.randn((T, H, V), device="cuda", generator=g).bfloat16()
    out = torch.empty((T, H, V), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    scale = 1 / math.sqrt(N + R)
    mla.mla_attention_fwd(q, kv, kr, out, N, R, V, scale, causal=True, lse=lse)
    f32 = dict(dtype=torch.float32, device="cuda")
    dq, dkv, dkr = torch.empty((T, H, N + R), **f32), torch.empty((T, H, N + V), **f32), torch.empty((T, R), **f32)
    ws = torch.empty(mla.mla_attention_bwd_workspace_size(q, kv, kr, out, dout, N, R, V, scale), dtype=torch.uint8,
                     device="cuda")
    call = lambda: mla.mla_attention_bwd(q, kv, kr, out, dout, lse, N, R, V, scale, causal=True,  # noqa: E731
                                         dq=dq, dkv=dkv, dk_rope=dkr, workspace=ws)
    for _ in range(3):
        call()
    reps = 20
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    st.record()
    for _ in range(reps):
        call()
    en.record()
    torch.cuda.synchronize()
    us = st.elapsed_time(en) * 1e3 / reps
    flops = 2.0 * (3 * (N + R) + 2 * V) * H * T * (T + 1) / 2
    tf = flops / (us * 1e-6) / 1e12
    res = {"attention_bwd_us": round(us, 2), "attention_bwd_tflops": round(tf, 1),
           "attention_bwd_mfma_frac": round(tf / 2500.0, 4),
           "attention_bwd_note": "dsv3_rank shard (T=2048, H=16, causal), row terms + dk/dv + dq + band sum, "
                                 "fp32 gradients; 5 products per visible pair counted"}
    # the latent up-projection's backward for the same heads (16 of 128, latent 512): d_latent and dW
    L, HT, P = 512, 128, N + V
    latent = torch.randn((T, L), device="cuda", generator=g).bfloat16()
    w = (torch.randn((L, HT * P), device="cuda", generator=g) * 0.05).bfloat16()
    dl, dw = torch.empty((T, L), **f32), torch.empty((L, H * P), **f32)
    up = lambda: mla.mla_latent_up_proj_bwd(latent, w, dkv, HT, 16, H, N, V, d_latent=dl, dw=dw)  # noqa: E731
    for _ in range(3):
        up()
    torch.cuda.synchronize()
    st.record()
    for _ in range(reps):
        up()
    en.record()
    torch.cuda.synchronize()
    us = st.elapsed_time(en) * 1e3 / reps
    tf = 2 * 2.0 * T * L * H * P / (us * 1e-6) / 1e12
    res.update({"up_proj_bwd_us": round(us, 2), "up_proj_bwd_tflops": round(tf, 1),
                "up_proj_bwd_note": "d_latent [2048][512] and dW [512][4096] from fp32 dkv, 2 x 8.6 GFLOP"})
    return res


def _varlen(torch, mla, mi, dev):
    """Packed documents 8192/4096/2048/2048 (T=16384, H=16): block-diagonal causal attention."""
    w = mi.WORKLOADS["varlen16k"]
    d = mi.shard_inputs(w)
    latent, W, q, kr = dev(d["latent"]), dev(d["w_kvb"]), dev(d["q"]), dev(d["k_rope"])
    kv = torch.empty((w.T, w.H, w.P), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((w.T, w.H, w.V), dtype=torch.bfloat16, device="cuda")
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    mla.mla_latent_up_proj(latent, W, kv, w.heads_total, 0, w.H, w.N, w.V)
    fn = lambda: mla.mla_attention_fwd(q, kv, kr, out, w.N, w.R, w.V, 1 / math.sqrt(w.K), cu_seqlens=cu)  # noqa: E731
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    us = _median_us(torch, fn, 10)
    pairs = sum(n * (n + 1) // 2 for n in w.doc_lens)
    flops = 2.0 * w.H * pairs * (w.K + w.V)
    return {"varlen16k_attention_us": round(us, 2), "varlen16k_attention_tflops": round(flops / (us * 1e-6) / 1e12, 2),
            "varlen16k_mfma_frac": round(flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def _decode(torch, mla, mi, dev):
    """Latent-cache decode: 32 sequences, one query each over 8192 cached positions, 8 KV chunks.

    The 302 MB cache exceeds the 256 MB Infinity Cache only slightly, so every timed call
    follows a read-only sweep of 512 MB (a sweep that writes would leave dirty lines whose
    write-back competes with the measured call)."""
    w = mi.WORKLOADS["decode32"]
    d = mi.decode_inputs(w)
    q, c, kr, W = dev(d["q"]), dev(d["latent"]), dev(d["k_rope"]), dev(d["w_kvb"])
    out = torch.empty((w.batch, w.H, w.V), dtype=torch.bfloat16, device="cuda")
    fn = lambda: mla.mla_latent_decode_fwd(q, c, kr, W, out, w.heads_total, 0, w.N, w.R, w.V,  # noqa: E731
                                           w.kv_splits, 1 / math.sqrt(w.K))
    sweep = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    us = _median_us(torch, fn, 20, before=sweep.sum)
    cache_bytes = 2.0 * (c.numel() + kr.numel())
    gbps = (cache_bytes + 2.0 * W.numel()) / (us * 1e-6) / 1e9
    del sweep
    return {"decode32_us": round(us, 2), "decode32_cache_gbps": round(gbps, 1),
            "decode32_hbm_frac": round(gbps / PEAK_HBM_GBS, 4),
            "decode32_note": "whole mla_latent_decode_fwd call (absorb, split, merge, project) after a 512 MB "
                             "read-only sweep; bytes = latent + rope cache + weight"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the uneven22 pack/unpack, varlen16k and decode32 measurements")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache passes and the MFMA peak probe (for kernel traces whose averages should "
                         "cover back-to-back calls only)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain contiguous copy of 1 GiB (the pack kernel with one rank) 3 times, "
                         "to scale the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time the backward of the rank shard (attention, then the up-projection) and print "
                         "its figures as one JSON line (for profiling the backward kernels on their own)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): this build has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(1)

    import numpy as np
    import torch

    import mla_attention_under_amd as mla
    import mla_inputs as mi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    mla.load_library()

    if args.backward_only:
        print(json.dumps(_backward(torch, mla)))
        return

    if args.copy_calibration:
        n = 1 << 29                                   # 2-byte elements: 1 GiB read + 1 GiB written
        src = torch.randint(-32768, 32767, (n // 512, 1, 512), dtype=torch.int16, device="cuda")
        dst = torch.empty(n, dtype=torch.int16, device="cuda")
        for _ in range(3):
            mla.mla_pack_heads(src, dst, [1])
        torch.cuda.synchronize()
        assert torch.equal(dst.view_as(src), src)
        print(json.dumps({"copy_calibration_bytes_each_way": 2 * n, "launches": 3}), flush=True)
        return

    w = mi.WORKLOADS["dsv3_rank"]
    T, H, L, N, R, V, P, K = w.T, w.H, w.L, w.N, w.R, w.V, w.P, w.K
    scale = 1 / math.sqrt(K)
    sp, Ttok, Htot_pack = 8, w.pack_tokens, sum(w.pack_shards)
    sizes = mla.mla_head_shard_sizes(Htot_pack, Htot_pack, sp)           # [16] * 8

    d = mi.shard_inputs(w)
    x_pack = mi.pack_payload(Ttok, Htot_pack, w.F, cfg=w.cfg)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    latent, W, q, kr = dev(d["latent"]), dev(d["w_kvb"]), dev(d["q"]), dev(d["k_rope"])
    xp = dev(x_pack)
    send = torch.empty(xp.numel(), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((T, H, P), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((T, H, V), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T // sp, sp * H, V), dtype=torch.bfloat16, device="cuda")
    out_flat = out.view(-1)

    # the caller's workspace, allocated once, as a serving loop holds it
    ws_attn = torch.empty(max(1, mla.mla_attention_workspace_size(q, kv, kr, out, N, R, V, scale)), dtype=torch.uint8,
                          device="cuda")
    kernels = ["pack", "up_proj", "attention"]
    calls = {
        "pack": lambda: mla.mla_pack_heads(xp, send, sizes),
        "up_proj": lambda: mla.mla_latent_up_proj(latent, W, kv, w.heads_total, 0, H, N, V),
        # the output goes straight to y: query chunk r (rank r's 256 tokens) into heads [16r, 16r+16)
        "attention": lambda: mla.mla_attention_fwd(q, kv, kr, y, N, R, V, scale, workspace=ws_attn, unpack_sp=sp),
        # the separate restore copy, timed on its own (not part of the step)
        "unpack": lambda: mla.mla_unpack_heads(out_flat, y, [H] * sp),
    }

    def step():
        for k in kernels:
            calls[k]()

    flops_up = 2.0 * T * L * H * P
    pairs = T * (T + 1) / 2
    flops_attn = 2.0 * H * pairs * (K + V)
    flops_step = flops_up + flops_attn
    bytes_pack = 2.0 * xp.numel() * 2
    bytes_unpack = 2.0 * out.numel() * 2

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K steps back to back
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    _busy(torch)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps

    # ---- per-kernel pass: events around every launch, on the launch stream
    ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for k in kernels + ["unpack"]}
    torch.cuda.synchronize()
    _busy(torch)
    for i in range(args.steps):
        for k in kernels + ["unpack"]:
            ev[k][i][0].record()
            calls[k]()
            ev[k][i][1].record()
    torch.cuda.synchronize()
    kern_us = {k: 1e3 * sum(a.elapsed_time(b) for a, b in ev[k]) / args.steps for k in kernels + ["unpack"]}
    kern_pct = {k: _pct([1e3 * a.elapsed_time(b) for a, b in ev[k]]) for k in kernels + ["unpack"]}

    # ---- per-step pass: events around every whole step, back to back (for p10 / p90 of the step)
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    _busy(torch)
    for i in range(args.steps):
        sev[i][0].record()
        step()
        sev[i][1].record()
    torch.cuda.synchronize()
    step_pct = _pct([1e3 * a.elapsed_time(b) for a, b in sev])

    # ---- cold caches: a 512 MB read-only sweep before every timed step / pack
    step_cold = pack_cold = mfma_peak = None
    if not args.no_cold:
        sweep = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
        reps_cold = max(10, min(args.steps, 50))
        step_cold = _flushed(torch, step, reps_cold, sweep)
        pack_cold = _flushed(torch, calls["pack"], reps_cold, sweep)
        del sweep
        mfma_peak = _mfma_peak(torch, mla)

    attn_tflops = flops_attn / (kern_us["attention"] * 1e-6) / 1e12
    extra = {
        "kernel_us": {k: round(v, 3) for k, v in kern_us.items()},
        "kernel_us_pct": kern_pct,
        "step_us_pct": step_pct,
        "cold_cache": None if step_cold is None else {
            "step_us": step_cold,
            "step_tflops_median": round(flops_step / (step_cold["median"] * 1e-6) / 1e12, 2),
            "pack_us": pack_cold,
            "pack_gbps_median": round(bytes_pack / (pack_cold["median"] * 1e-6) / 1e9, 1),
            "note": "each timed step / pack after a 512 MB read-only sweep (twice the Infinity Cache); value and "
                    "the other figures are back to back with inputs resident"},
        "mfma_peak_measured": mfma_peak,
        "up_proj_tflops": round(flops_up / (kern_us["up_proj"] * 1e-6) / 1e12, 2),
        "attention_tflops": round(attn_tflops, 2),
        "compute_only_tflops": round(flops_step / ((kern_us["up_proj"] + kern_us["attention"]) * 1e-6) / 1e12, 2),
        "pack_gbps": round(bytes_pack / (kern_us["pack"] * 1e-6) / 1e9, 1),
        "unpack_gbps": round(bytes_unpack / (kern_us["unpack"] * 1e-6) / 1e9, 1),
        "pack_note": "dsv3_rank pack/unpack buffers (58.7 MB, 16.8 MB) fit the 256 MB Infinity Cache",
    }

    if not args.no_extra:
        # uneven 22-head shard: [4096][128][448] <-> 6 slabs; 940 MB of traffic per direction, beyond the cache
        sz6 = mla.mla_head_shard_sizes(128, 128, 6)
        big = torch.randint(-32768, 32767, (4096, 128, 448), dtype=torch.int16, device="cuda")
        big_send = torch.empty(big.numel(), dtype=torch.int16, device="cuda")
        big_back = torch.empty_like(big)
        for _ in range(3):
            mla.mla_pack_heads(big, big_send, sz6)
            mla.mla_unpack_heads(big_send, big_back, sz6)
        reps = 20
        e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2 * reps)]
        torch.cuda.synchronize()
        _busy(torch)
        for i in range(reps):
            e[2 * i][0].record()
            mla.mla_pack_heads(big, big_send, sz6)
            e[2 * i][1].record()
            e[2 * i + 1][0].record()
            mla.mla_unpack_heads(big_send, big_back, sz6)
            e[2 * i + 1][1].record()
        torch.cuda.synchronize()
        nbytes = 2.0 * big.numel() * 2
        pk = sum(e[2 * i][0].elapsed_time(e[2 * i][1]) for i in range(reps)) / reps
        up = sum(e[2 * i + 1][0].elapsed_time(e[2 * i + 1][1]) for i in range(reps)) / reps
        extra["uneven22_pack_gbps"] = round(nbytes / (pk * 1e-3) / 1e9, 1)
        extra["uneven22_unpack_gbps"] = round(nbytes / (up * 1e-3) / 1e9, 1)
        extra["uneven22_pack_us"] = round(pk * 1e3, 2)
        assert torch.equal(big_back, big), "uneven22 pack/unpack round trip failed"
        del big, big_send, big_back
        extra.update(_expanded(torch, mla))
        extra.update(_rope(torch, mla))
        extra.update(_project_pack(torch, mla))
        extra.update(_backward(torch, mla))
        extra.update(_varlen(torch, mla, mi, dev))
        extra.update(_decode(torch, mla, mi, dev))

    value = flops_step / (ms_step * 1e-3) / 1e12
    traffic = _traffic("attention", "dsv3_rank")
    roof = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
            "measured_peak": mfma_peak and mfma_peak["tflops"],
            "frac_of_measured_peak": mfma_peak and round(attn_tflops / mfma_peak["tflops"], 4),
            "kernel": "mla_attention_fwd (attn_fwd_kernel<128,64,128>)",
            "algorithmic": f"{flops_attn / 1e9:.3f} GFLOP per launch = 2*H*T(T+1)/2*(N+R+V)"}
    line = {
        "metric": "MLA shard attention TFLOP/s (+pack GB/s), T=2048 H=16 bf16, 1 MI355X",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "dsv3_rank", "T": T, "H": H, "L": L, "N": N, "R": R, "V": V, "heads_total": 128,
                   "sp": sp, "pack": "[256][128][448] -> 8 x 16 heads", "causal": True,
                   "step": "pack + up_proj + attention (head->token unpack fused into its output stores)",
                   "flops_per_step": flops_step},
        "roofline": roof,
    }
    line.update(extra)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, d, x_pack, sizes, flops_step)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
