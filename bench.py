#!/usr/bin/env python3
"""Benchmark of the frame-wise GDN forward path on one MI355X.

One step = one gdn_frame_forward call over the whole minute-scale 720p-shaped
workload (B1 H20 T961 S880 D112, bf16 I/O, fp32 state, ERASE mode), inputs
already resident in HBM.  Prints ONE JSON line with tokens/s (B*H*T*S per
second), the roofline of the dominant kernel, the whole-path roofline and the
oracle's CPU rate on a bounded sample.  A `streaming` field adds the
chunk-causal rollout check: the short-clip shape (B1 H16 T81 S880 D64) fed 4
frames per gdn_frame_step call, its per-chunk latency and back-to-back rate.
A `variants` field times the same 720p-shaped step with OCP E4M3 Q, K, V, O
(the low-precision I/O variant, 4*D bytes per token-head), and a `backward`
field times gdn_frame_backward on the bf16 inputs (14*D algorithmic bytes per
token-head), and a `training_step` field the pair gdn_frame_forward_train +
gdn_frame_backward_saved (the backward without the forward replay).  A `temporal_conv` field times gdn_tconv_forward, the block-causal
temporal convolution of the streaming FFN, on a 720p-shaped activation
(B1 T961 S880 C2240, blocks of 4 frames, bf16: 4*C algorithmic bytes per
token), plus one block's call latency.  An `attention` field times
gdn_attention_forward, the block-causal softmax attention of the hybrid's
softmax blocks, on an 81-frame 720p-shaped clip (B1 H20 S880 D112, blocks of
4 frames) and on one 4-frame chunk of queries against the whole clip, against
the dense bf16 MFMA peak (4*D flops per visible query-key pair).  The headline
`value` stays the bf16 forward step.

The default bf16 path is the Gram pipeline (gram pass, serial state pass,
readout); --path direct times the single-pass recurrence instead.

Timing: `value` and `ms_per_step` come from K plain steps between two device
synchronisations.  The per-kernel device times come from a second run of the
same K steps in which the library brackets every launch with HIP events on the
stream it runs on (the events cost a little, reported as
`ms_per_step_with_kernel_events`).

Roofline bookkeeping (algorithmic bytes only; the per-frame G/B staging, the
state snapshots and any re-reads are overhead, not algorithm):
  whole path   8*D bytes per token-head (Q, K, V read; O written, bf16)
  gram         4*D bytes per token-head (K, V read)
  recurrence   4*D bytes per token-head (K, V read) + 8 per frame-head (gamma, beta)
  state        8 bytes per frame-head (gamma, beta)
  readout      4*D bytes per token-head (Q read, O written)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFS = 2500.0    # dense bf16 MFMA, TFLOP/s
KERNEL_SRCS = [os.path.join(ROOT, "frame_wise_gated_gdn_amd", "csrc", f)
               for f in ("gdn_device.h", "gdn_kernels.hip", "gdn_gram.hip", "gdn_fused.hip")]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_traffic_minute720p.json")


def kernel_hash() -> str:
    """Hash of the device sources (the counters are only valid for the kernels they were taken on)."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def pmc_traffic(kernel: str):
    """HBM traffic per launch from a stored rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    if it was taken on the current kernel source; else None."""
    try:
        s = json.load(open(PMC_SUMMARY))
    except (OSError, ValueError):
        return None
    if s.get("kernel_source_sha256_16") != kernel_hash():
        return None
    k = s.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, heads: int):
    """Oracle (as it stands, compiled -O3 -march=native on this host) on `heads`
    whole heads of the same workload, OpenMP over all host threads."""
    import tempfile
    from oracle import gdn_oracle
    from frame_wise_gated_gdn_amd import workloads as wl
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    # built here, for this host's CPU (a library built elsewhere may use
    # instructions this CPU lacks); same arithmetic as the -O2 build
    lib = gdn_oracle.build(os.path.join(tempfile.gettempdir(), f"liboracle_gdn_native_{os.getpid()}.so"),
                           native=True)
    tok = 0
    t0 = time.perf_counter()
    for h in range(heads):
        q, k, v = (wl.to_numpy_io(inp[n][0, h]) for n in ("q", "k", "v"))
        g = inp["gamma"][0, h].cpu().numpy()
        b = inp["beta"][0, h].cpu().numpy()
        gdn_oracle.head(q, k, v, g, b, beta_mode=w.beta_mode, want_out=True, threads=threads, lib_path=lib)
        tok += w.T * w.S
    dt = time.perf_counter() - t0
    return {"value": tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "build": "gcc -O3 -march=native -fopenmp -fno-fast-math -ffp-contract=off",
            "sample": f"{heads} whole head(s) (b=0, h=0..{heads - 1}) of {w.name}: {tok} tokens, "
                      f"{dt:.1f} s wall, fp64, OpenMP {threads} threads"}


def one_shot_ms(gdn, torch, dev, w, reps: int, flush_bytes: int = 512 << 20):
    """Median and minimum device time of one whole-sequence gdn_frame_forward on
    workload `w` (HIP events on the call's stream), with a 512 MB buffer
    overwritten between the calls so that the 256 MB Infinity Cache holds none
    of the inputs."""
    from frame_wise_gated_gdn_amd import workloads as wl
    inp = wl.generate(w, device=dev)
    desc = gdn.make_desc(w.B, w.H, w.T, w.S, w.D, w.dtype, w.beta_mode)
    ws = torch.empty(gdn.workspace_size(desc), dtype=torch.uint8, device=dev)
    out = torch.empty_like(inp["q"])
    st = torch.empty((w.B, w.H, w.D, w.D), dtype=torch.float32, device=dev)
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device=dev)
    call = lambda: gdn.frame_forward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"],
                                     beta_mode=w.beta_mode, out=out, state_out=st, workspace=ws)
    for _ in range(3):
        call()
    ts = []
    for _ in range(reps):
        flush.fill_(1)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    alg = w.B * w.H * w.T * (w.S * 4 * w.D * {"bf16": 2, "f32": 4, "fp8": 1}[w.dtype] + 8)
    med = ts[len(ts) // 2]
    return {"workload": w.name, "io_dtype": w.dtype, "ms_median": med, "ms_min": ts[0], "reps": reps,
            "tokens_per_s": w.tokens / (med * 1e-3), "algorithmic_bytes": alg,
            "hbm_frac": alg / (med * 1e-3) / 1e9 / HBM_PEAK_GBS}


def stress_variant(gdn, wl, torch, dev, steps: int):
    """The stability/throughput stress shape (B2 H20 T961 S3600 D128, beta = 1,
    K ~ N(0, 4)): tokens/s and the path roofline (8*D bytes per token-head)."""
    w = wl.STRESS
    inp = wl.generate(w, device=dev)
    desc = gdn.make_desc(w.B, w.H, w.T, w.S, w.D, w.dtype, w.beta_mode)
    ws = torch.empty(gdn.workspace_size(desc), dtype=torch.uint8, device=dev)
    out = torch.empty_like(inp["q"])
    st = torch.empty((w.B, w.H, w.D, w.D), dtype=torch.float32, device=dev)
    nm = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=dev)
    call = lambda: gdn.frame_forward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"],
                                     beta_mode=w.beta_mode, out=out, state_out=st, norms=nm, workspace=ws)
    call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    path_bytes = w.tokens * 8 * w.D
    gbs = path_bytes / (ms * 1e-3) / 1e9
    finite = bool(torch.isfinite(nm).all()) and bool(torch.isfinite(st).all())
    res = {"workload": w.name, "value": w.tokens / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
           "steps": steps, "norms_and_state_finite": finite, "max_state_norm": float(nm.max()),
           "path_roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_step": path_bytes}}
    del inp, out, ws
    torch.cuda.empty_cache()
    return res


def streaming_latency(gdn, wl, torch, dev, reps: int):
    """Chunk-causal rollout of the short-clip shape, 4 frames per gdn_frame_step call
    with the state committed in place: per-chunk latency (enqueue to completion,
    one chunk at a time), the per-chunk time of back-to-back chunks and the
    whole rollout."""
    w = wl.CHUNKED
    inp = wl.generate(w, device=dev)
    T, c = w.T, w.chunk
    chunks = [tuple(inp[n][:, :, t0:min(T, t0 + c)].contiguous() for n in ("q", "k", "v", "gamma", "beta"))
              for t0 in range(0, T, c)]
    outs = [torch.empty_like(ch[0]) for ch in chunks]
    state = torch.zeros((w.B, w.H, w.D, w.D), dtype=torch.float32, device=dev)
    desc = gdn.make_desc(w.B, w.H, c, w.S, w.D, w.dtype, w.beta_mode)
    ws = torch.empty(gdn.workspace_size(desc), dtype=torch.uint8, device=dev)

    def rollout(sync_each):
        state.zero_()
        lat = []
        for ch, o in zip(chunks, outs):
            t0 = time.perf_counter()
            gdn.frame_step(*ch, state, beta_mode=w.beta_mode, out=o, commit="inplace", workspace=ws)
            if sync_each:
                torch.cuda.synchronize()
                if ch[0].shape[2] == c:
                    lat.append(time.perf_counter() - t0)
        return lat

    rollout(True)
    lat = sorted(x for _ in range(reps) for x in rollout(True))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        rollout(False)
    torch.cuda.synchronize()
    per_chunk = (time.perf_counter() - t0) / (reps * len(chunks))
    pct = lambda p: lat[min(len(lat) - 1, int(round(p * (len(lat) - 1))))] * 1e6
    return {"workload": w.name, "frames_per_chunk": c, "chunks_per_rollout": len(chunks), "rollouts": reps,
            "latency_us_p50": pct(0.5), "latency_us_p99": pct(0.99), "latency_samples": len(lat),
            "back_to_back_us_per_chunk": per_chunk * 1e6,
            "whole_rollout_ms": per_chunk * len(chunks) * 1e3,
            "back_to_back_tokens_per_s": w.B * w.H * w.T * w.S / (per_chunk * len(chunks))}


def fp8_variant(gdn, wl, torch, dev, steps: int, warmup: int):
    """The same 720p-shaped step with OCP E4M3 Q, K, V and O (the low-precision
    I/O variant): 4*D bytes per token-head instead of 8*D."""
    w = wl.MINUTE_720P.with_(dtype="fp8")
    inp = wl.generate(w, device=dev)
    desc = gdn.make_desc(w.B, w.H, w.T, w.S, w.D, w.dtype, w.beta_mode)
    ws = torch.empty(gdn.workspace_size(desc), dtype=torch.uint8, device=dev)
    out = torch.empty_like(inp["q"])
    st = torch.empty((w.B, w.H, w.D, w.D), dtype=torch.float32, device=dev)
    call = lambda timed: gdn.frame_forward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"],
                                           beta_mode=w.beta_mode, out=out, state_out=st, workspace=ws,
                                           time_kernels=timed)
    for _ in range(warmup):
        call(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call(False)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    gdn.kernel_times(reset=True)
    for _ in range(steps):
        call(True)
    torch.cuda.synchronize()
    kms = {name: t / steps for name, (t, n) in gdn.kernel_times(reset=True).items() if n > 0}
    path_bytes = w.B * w.H * w.T * w.S * 4 * w.D
    gbs = path_bytes / (ms * 1e-3) / 1e9
    return {"io_dtype": "fp8_e4m3 (OCP)", "workload": w.name, "value": w.tokens / (ms * 1e-3),
            "unit": "tokens/s", "ms_per_step": ms, "kernels_ms_per_step": kms,
            "path_roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_step": path_bytes,
                              "traffic": pmc_traffic("fused_fp8")}}


def backward_variant(gdn, wl, torch, dev, inp, steps: int, warmup: int):
    """gdn_frame_backward on the same 720p-shaped inputs (dL/dO Gaussian, bf16):
    algorithmic bytes 14*D per token-head (q, k, v, dO read; dq, dk, dv written)."""
    w = wl.MINUTE_720P
    g = torch.Generator(device=dev).manual_seed(11)
    d_out = torch.randn((w.B, w.H, w.T, w.S, w.D), generator=g, device=dev).to(torch.bfloat16)
    desc = gdn.make_desc(w.B, w.H, w.T, w.S, w.D, "bf16", w.beta_mode)
    ws = torch.empty(gdn.backward_workspace_size(desc), dtype=torch.uint8, device=dev)
    call = lambda timed: gdn.frame_backward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], d_out,
                                            beta_mode=w.beta_mode, workspace=ws, time_kernels=timed)
    for _ in range(warmup):
        call(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call(False)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    gdn.kernel_times(reset=True)
    for _ in range(steps):
        call(True)
    torch.cuda.synchronize()
    kms = {name: t / steps for name, (t, n) in gdn.kernel_times(reset=True).items() if n > 0}
    path_bytes = w.B * w.H * w.T * w.S * 14 * w.D
    gbs = path_bytes / (ms * 1e-3) / 1e9
    return {"workload": w.name, "value": w.tokens / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
            "kernels_ms_per_step": kms,
            "path_roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_step": path_bytes}}


def tconv_variant(gdn, wl, torch, dev, steps: int, warmup: int, block_reps: int = 50):
    """gdn_tconv_forward over the whole 720p-shaped activation in one call, and one
    block of `chunk` frames per call (the streaming use) with the cache handed on."""
    w = wl.TCONV_720P
    inp = wl.generate_tconv(w, device=dev)
    y = torch.empty_like(inp["x"])
    cache_out = torch.empty_like(inp["cache"])
    call = lambda timed: gdn.tconv_forward(inp["x"], inp["w"], inp["bias"], w.chunk, inp["cache"], out=y,
                                           cache_out=cache_out, time_kernels=timed)
    for _ in range(warmup):
        call(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call(False)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    gdn.kernel_times(reset=True)
    for _ in range(steps):
        call(True)
    torch.cuda.synchronize()
    kms = gdn.kernel_times(reset=True)["tconv"][0] / steps
    alg = w.B * w.T * w.S * w.C * 2 * 2
    gbs = alg / (kms * 1e-3) / 1e9
    # one block per call, cache updated in place
    xb = inp["x"][:, :w.chunk].contiguous()
    yb = torch.empty_like(xb)
    cache = inp["cache"].clone()
    blk = lambda: gdn.tconv_forward(xb, inp["w"], inp["bias"], w.chunk, cache, out=yb, cache_out="inplace")
    for _ in range(5):
        blk()
    torch.cuda.synchronize()
    lat = []
    for _ in range(block_reps):
        t1 = time.perf_counter()
        blk()
        torch.cuda.synchronize()
        lat.append((time.perf_counter() - t1) * 1e6)
    t1 = time.perf_counter()
    for _ in range(block_reps):
        blk()
    torch.cuda.synchronize()
    b2b = (time.perf_counter() - t1) * 1e6 / block_reps
    lat.sort()
    return {"workload": w.name, "value": w.tokens / (ms * 1e-3), "unit": "tokens/s (B*T*S)", "ms_per_step": ms,
            "kernel_ms": kms,
            "roofline": {"bound": "hbm", "kernel": "tconv", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": alg},
            "block_call": {"frames": w.chunk, "latency_us_median": lat[len(lat) // 2],
                           "back_to_back_us": b2b}}


def attn_flops(w) -> int:
    """4*D flops per visible (query, key) pair: Q K^T and P V, 2*D each."""
    S, Tq, Tk, c = w.S, w.Tq, w.Tk, w.chunk
    pairs = 0
    for f in range(Tk - Tq, Tk):
        pairs += S * min(Tk, (f // c + 1) * c) * S
    return w.B * w.H * pairs * 4 * w.D


def attention_variant(gdn, wl, torch, dev, steps: int, warmup: int):
    res = {}
    for key, w in (("clip", wl.ATTN_CLIP_720P), ("stream_chunk", wl.ATTN_STREAM_720P)):
        inp = wl.generate_attn(w, device=dev)
        o = torch.empty_like(inp["q"])
        nws = gdn.attention_workspace_size(gdn.make_attn_desc(w.B, w.H, w.Tq, w.Tk, w.S, w.D, w.chunk))
        ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
        call = lambda timed: gdn.attention_forward(inp["q"], inp["k"], inp["v"], w.chunk, out=o, workspace=ws,
                                                   time_kernels=timed)
        for _ in range(warmup):
            call(False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            call(False)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        gdn.kernel_times(reset=True)
        for _ in range(steps):
            call(True)
        torch.cuda.synchronize()
        kms = gdn.kernel_times(reset=True)["attention"][0] / steps
        fl = attn_flops(w)
        tfs = fl / (kms * 1e-3) / 1e12
        res[key] = {"workload": w.name, "value": w.tokens / (ms * 1e-3), "unit": "query tokens/s (B*H*Tq*S)",
                    "ms_per_step": ms, "kernel_ms": kms, "key_split_workspace_bytes": nws,
                    "roofline": {"bound": "mfma", "kernel": "attention", "achieved": tfs, "peak": BF16_MFMA_PEAK_TFS,
                                 "unit": "TFLOP/s", "frac": tfs / BF16_MFMA_PEAK_TFS, "flops_per_launch": fl}}
        del inp, o, ws
    return res


def training_variant(gdn, wl, torch, dev, inp, steps: int, warmup: int):
    """One training step on the 720p-shaped inputs: gdn_frame_forward_train
    (the forward that keeps G_t, B_t and the state snapshots) then
    gdn_frame_backward_saved (no replay).  Also the saved backward alone, with
    its roofline on 14*D algorithmic bytes per token-head."""
    w = wl.MINUTE_720P
    g = torch.Generator(device=dev).manual_seed(11)
    d_out = torch.randn((w.B, w.H, w.T, w.S, w.D), generator=g, device=dev).to(torch.bfloat16)
    desc = gdn.make_desc(w.B, w.H, w.T, w.S, w.D, "bf16", w.beta_mode)
    saved = torch.empty(gdn.saved_size(desc), dtype=torch.uint8, device=dev)
    ws = torch.empty(gdn.backward_saved_workspace_size(desc), dtype=torch.uint8, device=dev)
    o = torch.empty_like(inp["q"])
    args = (inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"])
    fwd = lambda timed: gdn.frame_forward_train(*args, beta_mode=w.beta_mode, out=o, saved=saved,
                                                time_kernels=timed)
    bwd = lambda timed: gdn.frame_backward_saved(*args, saved, d_out, beta_mode=w.beta_mode, workspace=ws,
                                                 time_kernels=timed)
    for _ in range(warmup):
        fwd(False)
        bwd(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fwd(False)
        bwd(False)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    t0 = time.perf_counter()
    for _ in range(steps):
        bwd(False)
    torch.cuda.synchronize()
    ms_bwd = (time.perf_counter() - t0) * 1e3 / steps
    gdn.kernel_times(reset=True)
    for _ in range(steps):
        bwd(True)
    torch.cuda.synchronize()
    kms = {name: t / steps for name, (t, n) in gdn.kernel_times(reset=True).items() if n > 0}
    path_bytes = w.B * w.H * w.T * w.S * 14 * w.D
    gbs = path_bytes / (ms_bwd * 1e-3) / 1e9
    return {"workload": w.name, "ms_per_training_step": ms_step,
            "training_tokens_per_s": w.tokens / (ms_step * 1e-3),
            "backward_saved": {"ms": ms_bwd, "kernels_ms": kms,
                               "path_roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                                 "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                                 "algorithmic_bytes_per_step": path_bytes}}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-heads", type=int, default=12, help="oracle heads timed for cpu_baseline (0 = skip)")
    ap.add_argument("--no-backward", dest="backward", action="store_false",
                    help="skip the timing of gdn_frame_backward on the same inputs")
    ap.add_argument("--no-tconv", dest="tconv", action="store_false",
                    help="skip the timing of the block-causal temporal convolution")
    ap.add_argument("--no-attention", dest="attention", action="store_false",
                    help="skip the timing of the block-causal softmax attention")
    ap.add_argument("--no-fp8", dest="fp8", action="store_false",
                    help="skip the E4M3 I/O variant of the step")
    ap.add_argument("--stream-reps", type=int, default=5,
                    help="rollouts of the chunk-causal streaming latency check (0 = skip)")
    ap.add_argument("--path", choices=("auto", "three_pass", "direct"), default="auto",
                    help="bf16 path: one-launch forward (auto), the Gram pipeline as three launches, "
                         "or the single-pass recurrence")
    ap.add_argument("--no-configs", dest="configs", action="store_false",
                    help="skip the one-shot timings of the tiny and short-clip workloads")
    ap.add_argument("--stress-steps", type=int, default=3,
                    help="steps of the stress workload (B2 H20 T961 S3600 D128; 0 = skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device copy (for rocprofv3 counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path shards "
              "by (batch, head) with no communication, so N GPUs would each run their own heads.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import frame_wise_gated_gdn_amd as gdn
    from frame_wise_gated_gdn_amd import workloads as wl

    w = wl.MINUTE_720P
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = wl.generate(w, device=dev)
    desc = gdn.make_desc(w.B, w.H, w.T, w.S, w.D, w.dtype, w.beta_mode,
                         {"auto": 0, "direct": gdn.binding.FLAG_DIRECT,
                          "three_pass": gdn.binding.FLAG_THREE_PASS}[args.path])
    ws = torch.empty(gdn.workspace_size(desc), dtype=torch.uint8, device=dev)
    out = torch.empty_like(inp["q"])
    st = torch.empty((w.B, w.H, w.D, w.D), dtype=torch.float32, device=dev)
    call = lambda timed: gdn.frame_forward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"],
                                           beta_mode=w.beta_mode, out=out, state_out=st, workspace=ws,
                                           time_kernels=timed, path=args.path)
    for _ in range(args.warmup):
        call(False)
    torch.cuda.synchronize()
    # throughput: K plain steps (no per-kernel events between the launches)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call(False)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    # per-kernel device time: the same K steps again, each launch bracketed by
    # HIP events on the stream it runs on
    gdn.kernel_times(reset=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        call(True)
    torch.cuda.synchronize()
    dt_ev = time.perf_counter() - t1
    ktimes = gdn.kernel_times(reset=True)
    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    ms_step = dt * 1e3 / args.steps
    tokens = w.tokens
    value = tokens / (ms_step * 1e-3)
    D, BH, T, S = w.D, w.B * w.H, w.T, w.S
    # kernel time per step (sum over the launches of one step) and per launch
    kms = {name: ms / args.steps for name, (ms, n) in ktimes.items() if n > 0}
    klaunch = {name: n // args.steps for name, (ms, n) in ktimes.items() if n > 0}
    alg_bytes = {"gram": BH * T * S * 4 * D, "recurrence": BH * T * S * 4 * D + BH * T * 8,
                 "state": BH * T * 8, "readout": BH * T * S * 4 * D,
                 "fused": BH * T * S * 8 * D + BH * T * 8 + BH * D * D * 4}
    dom = max(kms, key=kms.get)
    launches_per_step = max(klaunch[dom], 1)
    dom_bytes, dom_ms = alg_bytes[dom], kms[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    path_bytes = BH * T * S * 8 * D
    path_flops = BH * T * S * 6 * D * D
    path_gbs = path_bytes / (ms_step * 1e-3) / 1e9
    rec = {
        "metric": "GDN frame-wise fwd tokens/s (B·H·T·S) at 1 GPU; % of HBM/MFMA roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian Q/K/V, uniform gamma/beta; no dataset)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "S": w.S, "D": w.D,
                   "io_dtype": w.dtype, "state_dtype": "f32", "beta_mode": w.beta_mode,
                   "path": {"auto": "one-launch", "three_pass": "gram three-launch",
                            "direct": "direct"}[args.path],
                   "calls_per_step": 1, "launches_per_kernel_per_step": launches_per_step},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": pmc_traffic(dom),
                     "algorithmic_bytes_per_launch": dom_bytes // launches_per_step,
                     "avg_launch_ms": dom_ms / launches_per_step},
        "path_roofline": {"bound": "hbm", "achieved": path_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": path_gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_step": path_bytes,
                          "mfma_frac": path_flops / (ms_step * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFS},
        "kernels_ms_per_step": kms,
        "ms_per_step_with_kernel_events": dt_ev * 1e3 / args.steps,
    }
    # context for the HBM fraction: one elementwise kernel with the same
    # bytes as the step (three bf16 reads of the input size, one write),
    # torch.addcmul on the same tensors
    sink = torch.empty_like(out)
    for _ in range(2):
        torch.addcmul(inp["q"], inp["k"], inp["v"], out=sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(5):
        e0.record()
        torch.addcmul(inp["q"], inp["k"], inp["v"], out=sink)
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    del sink
    ems = min(ts)
    rec["streaming_reference"] = {
        "what": "torch.addcmul(q, k, v) on the step's tensors: one elementwise kernel, 3 reads + 1 write of "
                "the step's bf16 size (no recurrence)",
        "ms": ems, "GB_per_s": path_bytes / (ems * 1e-3) / 1e9,
        "frac_of_peak": path_bytes / (ems * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "step_over_reference": ms_step / ems}
    if args.path == "auto":
        # the same step as three launches (same bits), for context
        ws3 = torch.empty(gdn.workspace_size(gdn.make_desc(w.B, w.H, w.T, w.S, w.D, w.dtype, w.beta_mode,
                                                           gdn.binding.FLAG_THREE_PASS)),
                          dtype=torch.uint8, device=dev)
        call3 = lambda: gdn.frame_forward(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"],
                                          beta_mode=w.beta_mode, out=out, state_out=st, workspace=ws3,
                                          path="three_pass")
        call3()
        torch.cuda.synchronize()
        t3 = time.perf_counter()
        for _ in range(args.steps):
            call3()
        torch.cuda.synchronize()
        rec["three_launch_ms_per_step"] = (time.perf_counter() - t3) * 1e3 / args.steps
        del ws3
    if args.configs:
        rec["configs"] = {"tiny": one_shot_ms(gdn, torch, dev, wl.TINY, 50),
                          "short_clip": one_shot_ms(gdn, torch, dev, wl.SHORT, 50)}
        rec["configs"]["short_clip"]["bar_us_60pct_roofline"] = 122.0
    if args.stream_reps > 0:
        rec["streaming"] = streaming_latency(gdn, wl, torch, dev, args.stream_reps)
        if args.configs:
            rec["streaming"]["one_shot_ms_same_shape"] = rec["configs"]["short_clip"]["ms_median"]
    if args.backward and args.path == "auto":
        rec["backward"] = backward_variant(gdn, wl, torch, dev, inp, max(1, args.steps // 4), 1)
        rec["training_step"] = training_variant(gdn, wl, torch, dev, inp, max(1, args.steps // 4), 1)
    if args.tconv:
        rec["temporal_conv"] = tconv_variant(gdn, wl, torch, dev, args.steps, args.warmup)
    if args.attention:
        rec["attention"] = attention_variant(gdn, wl, torch, dev, max(1, args.steps // 4), 1)
    if args.fp8 and args.path == "auto":
        rec["variants"] = {"fp8_e4m3_io": fp8_variant(gdn, wl, torch, dev, args.steps, args.warmup)}
    if args.stress_steps > 0:
        rec["stress"] = stress_variant(gdn, wl, torch, dev, args.stress_steps)
    if args.cpu_heads > 0:
        rec["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_heads)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
