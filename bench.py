"""Benchmark of the fused grouped-MLP MoE expert block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config mixtral]
                    [--prec bf16|mxfp8|mxfp4] [--cached-weights]

One step = the whole hot path of a training step of one expert layer:
route + permute (X), FC1 grouped GEMM with the fused SwiGLU + prob-scale
epilogue, FC2 grouped GEMM, unpermute; permute (dOut), FC2 dgrad grouped GEMM
with the fused dSwiGLU epilogue, FC1 dgrad grouped GEMM, unpermute (dX) +
dprobs.  With --prec mxfp8 the permutes write MXFP8 rows, the four GEMMs take
MXFP8 operands and the epilogues also write MXFP8 copies (rowwise and
transposed) of a and dz.  An MX step starts by making the weight copies
from the bf16 master weights, which change every training step (one pass
per weight writes both of its copies); --cached-weights reuses copies made
before the step instead (as over the microbatches of one optimizer step)
and times the quantization on its own.  Inputs are
synthetic (seeded), already resident in HBM when the timed region starts.
The value is algorithmic GEMM TFLOP/s of the step: 12 * M * H * I flops (18 with
--wgrad, which adds the weight-gradient GEMMs)
(M = routed rows; no padding counted).  --recompute (activation recompute)
keeps no z in the forward and rebuilds it with FC1's GEMM in the backward;
that GEMM is timed but its flops are not counted, being no model work.

Timing: the whole step is captured in one HIP graph (global capture mode, so
the step holds no host sync or allocation), replayed `--warmup` times, then
`--steps` replays are timed: hipEvents around each replay give the median and
the 10th / 90th percentiles, the wall clock around all of them (synchronised
on both sides) the mean, which is `value`.  Per-kernel times come from a
separate eager pass with hipEvents between the library's launches.  The
default run (Mixtral, bf16) also measures the Mixtral layer with MXFP8
operands in the same process (`secondary`, with its own fp8 roofline
fraction), the GPT-OSS layer (MXFP8) and the DeepSeek-V3 share (bf16 and
MXFP8) as compact lines (`other_layers`), the top-k router, and a plain
device copy as the practical HBM ceiling of the gather and combine kernels.  The GPT-OSS layer runs in MXFP8
(slope 1.702, clamp at +-7) unless --prec says otherwise.

Prints one JSON line (stdout).  Progress goes to stderr.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0,    # MI355X dense MFMA, published
               "mxfp4": 10100.0}
PEAK_HBM_GBS = 8000.0

# name -> workload config (workloads.gen.CONFIGS) and default precision
BENCH_CONFIGS = {
    "mixtral": ("mixtral", "bf16"),
    "mixtral_mx": ("mixtral_mx", "mxfp8"),
    "dsv3": ("dsv3", "bf16"),
    "gptoss": ("gptoss", "mxfp8"),
}

def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (recorded by the library on its stream)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [
            ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev.append(h.value)

    def record(self, i, stream):
        assert self.hip.hipEventRecord(self.ev[i], stream) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[a], self.ev[b])
        assert rc == 0, rc
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


GEMM_SRCS = [os.path.join(ROOT, "moe_grouped_mlp_amd", "csrc", f)
             for f in ("gemm_kernel.h", "act.h", "common.h", "mx.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fc1_mixtral_traffic.json")


def gemm_source_hash():
    h = hashlib.sha256()
    for src in GEMM_SRCS:
        with open(src, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per FC1 launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs, or None if the kernel source changed since."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("gemm_src_sha256") != gemm_source_hash():
        return None
    return rec.get("bytes_per_launch")


def device_inputs(cfg, seed, device):
    """Seeded synthetic inputs: routing (expert_idx, probs) from the same
    host generator the parity tests use (workloads.gen.route_inputs); X,
    dOut ~ N(0,1) and weights ~ N(0, 0.02^2) drawn on the device, in bf16."""
    import torch
    from workloads.gen import route_inputs
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    E, k, T, H, I = (cfg[n] for n in ("E", "k", "T", "H", "I"))
    n1 = 2 * I if cfg["act"] != "srelu" else I
    bf = torch.bfloat16
    x = torch.randn(T, H, generator=g, device=device).to(bf)
    dout = torch.randn(T, H, generator=g, device=device).to(bf)
    w1 = torch.empty(E, n1, H, dtype=bf, device=device)
    w2 = torch.empty(E, H, I, dtype=bf, device=device)
    for e in range(E):
        w1[e] = (torch.randn(n1, H, generator=g, device=device) * 0.02).to(bf)
        w2[e] = (torch.randn(H, I, generator=g, device=device) * 0.02).to(bf)
    idx, probs = route_inputs(cfg, seed, T, E, k)
    return (x, dout, w1, w2, torch.from_numpy(idx).to(device),
            torch.from_numpy(probs).to(device))


def cpu_baseline(cfg, seed, mx=False, target_s=15.0):
    """Time the CPU oracle (as it stands) on a bounded sample of the same
    workload: the rows routed to expert 0, full H and I, forward + backward
    (with MXFP8 operands when mx)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import moe as om
    from workloads.gen import _normal_bf16, route_inputs

    E, k, T, H, I = (cfg[n] for n in ("E", "k", "T", "H", "I"))
    idx, probs = route_inputs(cfg, seed, T, E, k)
    e0 = int(np.bincount(idx.reshape(-1), minlength=E).argmax())
    t_sel, s_sel = np.nonzero(idx == e0)
    rows = 64
    rng = np.random.default_rng(seed + 7)
    w1 = _normal_bf16(rng, (1, 2 * I, H), 0.02)
    w2 = _normal_bf16(rng, (1, H, I), 0.02)
    prm = om.ActParams.clamped(cfg["clamp"], beta=cfg["beta"], act=cfg["act"])
    done_flops, t_used, runs = 0.0, 0.0, 0
    while True:
        n = min(rows, len(t_sel))
        x = _normal_bf16(rng, (n, H), 1.0)
        dout = _normal_bf16(rng, (n, H), 1.0)
        sub_idx = np.zeros((n, 1), np.int32)
        sub_p = probs[t_sel[:n], s_sel[:n]].reshape(n, 1)
        t0 = time.perf_counter()
        fw = om.forward(x, w1, w2, sub_idx, sub_p, 1, prm, mx=mx)
        om.backward(fw, dout, w1, w2, prm, mx=mx)
        dt = time.perf_counter() - t0
        done_flops += 12.0 * n * H * I
        t_used += dt
        runs += 1
        if t_used >= target_s or runs >= 6:
            break
        rows = min(len(t_sel), max(rows, int(rows * target_s / max(dt, 1e-3) / 2)))
    threads = 0
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 0)))
    cores = threads or len(os.sched_getaffinity(0))
    return {"value": done_flops / t_used / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": (f"oracle forward+backward on rows routed to expert {e0} of the "
                       f"{E}-expert layer (H={H}, I={I}, "
                       f"{'MXFP8 operands' if mx else 'bf16 storage'}, fp64 math), "
                       f"{runs} runs, {done_flops / 1e12:.3f} TFLOP in {t_used:.1f} s")}


def gemm_bench(args):
    """--gemm: the FC2-shaped plain grouped GEMM (A = a [M][I], B = W2
    [E][H][I], the config's routed group sizes) through moe_grouped_gemm in
    bf16, MXFP8 and MXFP4, operands quantized before the timed region (the
    weights once per update; a by moe_quantize_mxfp8 / _mxfp4, timed on its
    own).  Prints one JSON line whose value is the MXFP4 rate."""
    import numpy as np
    import torch
    import moe_grouped_mlp_amd as mg
    from workloads.gen import CONFIGS, route_inputs
    wl_name, _ = BENCH_CONFIGS[args.config]
    cfg = dict(CONFIGS[wl_name])
    E, k, T, H, I = (cfg[n] for n in ("E", "k", "T", "H", "I"))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    idx, _ = route_inputs(cfg, args.seed, T, E, k)
    flat = idx.reshape(-1)
    sizes = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E).tolist()
    pad = [0]
    for n in sizes:
        pad.append(pad[-1] + -(-n // mg.GROUP_ALIGN) * mg.GROUP_ALIGN)
    M, M_cap, N, K = sum(sizes), max(pad[-1], 128), H, I
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    a = torch.randn(M_cap, K, generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn(E, N, K, generator=g, device=dev) * 0.02).to(torch.bfloat16)
    out = torch.empty(M_cap, N, dtype=torch.bfloat16, device=dev)
    split = torch.tensor(sizes, dtype=torch.int32, device=dev)
    padded = torch.tensor(pad, dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, mg.moe_grouped_mlp_workspace_size(E, N, K, M_cap)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    u8 = dict(dtype=torch.uint8, device=dev)
    flops = 2.0 * M * N * K
    evs = HipEvents(2)
    kernels = {}
    clocks = {}

    def timed(fn, n, tag=None):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        trace = GemmClockTrace(dev, 1)
        if tag:   # every launch rewrites the one record area: the last one stays
            mg.moe_gemm_clock_trace(trace.buf, 1)
        try:
            evs.record(0, stream)
            for _ in range(n):
                fn()
            evs.record(1, stream)
            torch.cuda.synchronize()
        finally:
            trace.stop()
        if tag:
            clocks[tag] = trace.clocks()[0] if trace.buf[0].any() else None
        return evs.elapsed_ms(0, 1) / n

    for prec in ("bf16", "mxfp8", "mxfp4"):
        log(f"grouped GEMM {prec}: E={E} M={M} N={N} K={K}")
        if prec == "bf16":
            args_ = dict(a=a, b=w, prec=mg.PREC_BF16, workspace=ws)
        else:
            f4 = prec == "mxfp4"
            div = 2 if f4 else 1
            a_q, a_s = torch.empty(M_cap * K // div, **u8), torch.empty(M_cap * K // 32, **u8)
            b_q, b_s = torch.empty(E * N * K // div, **u8), torch.empty(E * N * K // 32, **u8)
            if f4:
                qa = lambda: mg.moe_quantize_mxfp4(batch=1, rows=M_cap, cols=K, x=a, q=a_q,
                                                   s=a_s)
                mg.moe_quantize_mxfp4(batch=E, rows=N, cols=K, x=w, q=b_q, s=b_s)
            else:
                qa = lambda: mg.moe_quantize_mxfp8(mode=mg.QUANT_ROW, batch=1, rows=M_cap,
                                                   cols=K, x=a, q=a_q, s=a_s)
                mg.moe_quantize_mxfp8(mode=mg.QUANT_ROW, batch=E, rows=N, cols=K, x=w,
                                      q=b_q, s=b_s)
            qms = timed(qa, args.steps)
            kernels[f"quantize_a_{prec}"] = {
                "ms": round(qms, 4), "unit": "GB/s",
                "rate": round(M_cap * K * (2 + 1 / div + 1 / 32) / (qms * 1e-3) / 1e9, 1)}
            args_ = dict(a=a_q, b=b_q, a_s=a_s, b_s=b_s,
                         prec=mg.PREC_MXFP4 if f4 else mg.PREC_MXFP8)
        ms = timed(lambda: mg.moe_grouped_gemm(E=E, N=N, K=K, M_cap=M_cap, split_sizes=split,
                                               padded_offsets=padded, c=out, **args_),
                   args.steps, tag=prec)
        tf = flops / (ms * 1e-3) / 1e12
        kernels[f"gemm_{prec}"] = {"ms": round(ms, 4), "unit": "TFLOP/s", "rate": round(tf, 2),
                                   "pct_peak": round(100 * tf / PEAK_TFLOPS[prec], 2)}
        ck = clocks.get(prec)
        if ck:
            kernels[f"gemm_{prec}"]["shader_clock_ghz"] = round(ck, 4)
            kernels[f"gemm_{prec}"]["pct_peak_at_measured_clock"] = round(
                100 * tf / (PEAK_TFLOPS[prec] * ck / 2.4), 2)
        log(f"  {ms:.3f} ms, {tf:.1f} TFLOP/s ({100 * tf / PEAK_TFLOPS[prec]:.1f}% of peak)"
            f"{f', clock {ck:.3f} GHz' if ck else ''}")
    # overlap with another kernel (the pages' reason for dynamic scheduling):
    # a kernel holds 64 of the CUs for the first 1 ms of the bf16 GEMM; with
    # the work counters the other workgroups take the busy CUs' tiles, with
    # the static walk those tiles wait for their CUs
    ws_dyn = torch.zeros(mg.moe_grouped_gemm_workspace_size(True), **u8)
    ws_sta = torch.zeros(mg.moe_grouped_gemm_workspace_size(False), **u8)
    side = torch.cuda.Stream()
    busy_ticks = int(mg.moe_clock_tick_rate_hz() * 1e-3)
    ev2 = HipEvents(2)

    def overlapped(ws, busy, reps=5):
        gemm = lambda: mg.moe_grouped_gemm(E=E, N=N, K=K, M_cap=M_cap, split_sizes=split,
                                           padded_offsets=padded, a=a, b=w, c=out,
                                           workspace=ws)
        gemm()
        torch.cuda.synchronize()
        tot = 0.0
        for _ in range(reps):
            if busy:
                with torch.cuda.stream(side):
                    mg.moe_bench_occupy(workgroups=64, ticks=busy_ticks)
            ev2.record(0, stream)
            gemm()
            ev2.record(1, stream)
            torch.cuda.synchronize()
            tot += ev2.elapsed_ms(0, 1)
        return tot / reps

    ov = {"what": "bf16 FC2 GEMM while another kernel holds 64 of the CUs for its first 1 ms",
          "alone_ms": round(overlapped(ws_dyn, False), 4),
          "static_ms": round(overlapped(ws_sta, True), 4),
          "dynamic_ms": round(overlapped(ws_dyn, True), 4)}
    kernels["overlap_busy_cus"] = ov
    log(f"overlap: alone {ov['alone_ms']:.3f} ms, beside a 64-CU 1 ms kernel: static "
        f"{ov['static_ms']:.3f} ms, dynamic {ov['dynamic_ms']:.3f} ms")
    ev2.close()
    del a, w, out
    torch.cuda.empty_cache()
    # reference point: the vendor BLAS (hipBLASLt through torch.matmul) on one
    # dense bf16 product of the same FLOPs, [M][K] x [K][N], both operands
    # contiguous (no grouping, no epilogue)
    xa = torch.randn(M, K, generator=g, device=dev).to(torch.bfloat16)
    xb = (torch.randn(K, N, generator=g, device=dev) * 0.02).to(torch.bfloat16)
    xc = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: torch.matmul(xa, xb, out=xc), args.steps)
    tf = flops / (ms * 1e-3) / 1e12
    kernels["library_dense_bf16"] = {
        "what": "torch.matmul (vendor BLAS) on one dense bf16 [M][K] x [K][N] product, same FLOPs",
        "ms": round(ms, 4), "unit": "TFLOP/s", "rate": round(tf, 2),
        "pct_peak": round(100 * tf / PEAK_TFLOPS["bf16"], 2)}
    log(f"library dense bf16: {ms:.3f} ms, {tf:.1f} TFLOP/s")
    del xa, xb, xc
    evs.close()
    f4 = kernels["gemm_mxfp4"]
    print(json.dumps({
        "metric": "FC2-shaped grouped GEMM TFLOP/s, MXFP4 operands, 1 GPU",
        "value": f4["rate"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": f4["ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4-e2m1", "data": "synthetic",
        "config": {"workload": f"{args.config} FC2 grouped GEMM: E={E} routed rows {M} "
                               f"(group sizes of the layer's routing) x N={N} x K={K}",
                   "E": E, "M": M, "N": N, "K": K},
        "kernels": kernels,
        "roofline": {"bound": "mfma", "kernel": "MXFP4 grouped GEMM (plain store)",
                     "achieved": f4["rate"], "peak": PEAK_TFLOPS["mxfp4"], "unit": "TFLOP/s",
                     "frac": round(f4["rate"] / PEAK_TFLOPS["mxfp4"], 4), "traffic": None,
                     "avg_launch_ms": f4["ms"]},
        "cpu_baseline": None}))


class GemmClockTrace:
    """The shader clock the grouped GEMMs ran at.  While the library's GEMM
    clock trace is set, each grouped-GEMM launch takes the next record area
    and its persistent workgroups write their shader cycles and
    constant-rate ticks from start to end; a launch's clock is the mean of
    cycles / ticks x tick rate over its workgroups.  One area more than the
    expected launches is set up: if it gets written, the launches were not
    the expected ones and no clock is reported."""

    def __init__(self, dev, launches):
        import torch
        import moe_grouped_mlp_amd as mg
        self.mg = mg
        self.n = launches
        self.buf = torch.zeros(launches + 1, mg.CLOCK_MAX_WORKGROUPS, 2, dtype=torch.int64,
                               device=dev)
        self.rate = mg.moe_clock_tick_rate_hz()

    def start(self):
        self.mg.moe_gemm_clock_trace(self.buf, self.n + 1)

    def stop(self):
        self.mg.moe_gemm_clock_trace(None)

    def clocks(self):
        """Clock of each launch in GHz (None where nothing was recorded), or
        None if the launches were not the expected ones."""
        b = self.buf.cpu().numpy()
        if self.rate <= 0 or b[self.n].any():
            return None
        out = []
        for j in range(self.n):
            r = b[j]
            ok = (r[:, 0] > 0) & (r[:, 1] > 0)
            out.append(float((r[ok, 0] / (r[ok, 1] / self.rate)).mean() / 1e9)
                       if ok.any() else None)
        return out


def copy_ceiling_gbs(dev, mb=1024, reps=10):
    """Device-to-device copy rate (read + write bytes / time) of a plain
    copy kernel over `mb` MB: the practical HBM ceiling the gather and
    combine kernels are compared with."""
    import torch
    n = mb << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents(2)
    ev.record(0, stream)
    for _ in range(reps):
        dst.copy_(src)
    ev.record(1, stream)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(0, 1) / reps
    ev.close()
    del src, dst
    return 2.0 * n / (ms * 1e-3) / 1e9


def _pct(sorted_vals, q):
    i = min(len(sorted_vals) - 1, max(0, int(round(q * (len(sorted_vals) - 1)))))
    return sorted_vals[i]


def measure(args, config, prec, log_prefix=""):
    """One layer configuration: builds the block, captures one whole step in
    a HIP graph (global capture mode, so no host sync or allocation can hide
    in it), replays it `warmup` times, then times `steps` replays (each
    bracketed by hipEvents on the replay stream; the wall clock around all of
    them gives the mean), and runs a separate eager pass with hipEvents
    between the kernels for the per-kernel times.  Returns a dict."""
    import torch
    import moe_grouped_mlp_amd as mg
    from workloads.gen import CONFIGS

    wl_name, _ = BENCH_CONFIGS[config]
    mx = prec == "mxfp8"
    cfg = dict(CONFIGS[wl_name])
    E, k, T, H, I = (cfg[n] for n in ("E", "k", "T", "H", "I"))
    dev = torch.device("cuda:0")
    log(f"{log_prefix}generating {config} inputs ({prec})")
    x, dout, w1, w2, idx, probs = device_inputs(cfg, args.seed, dev)
    act_kind = {"swiglu": mg.ACT_SWIGLU, "geglu": mg.ACT_GEGLU, "srelu": mg.ACT_SRELU}[cfg["act"]]
    act = mg.act_params(act_kind, beta=cfg["beta"], clamp=cfg["clamp"])
    blk = mg.ExpertBlock(E, H, I, T, k, act=act,
                         prec={"bf16": mg.PREC_BF16, "mxfp8": mg.PREC_MXFP8,
                               "mxfp4": mg.PREC_MXFP4}[prec], wgrad=args.wgrad,
                         recompute=args.recompute,
                         # the unfused MX layers need bf16 a and dz; the fused
                         # MXFP4 layer writes only its MXFP4 copies
                         bf16_copies=(True if (args.unfused and prec != "bf16")
                                      else (False if prec == "mxfp4" else None)),
                         unfused=args.unfused)
    blk.load_weights(w1, w2)
    del w1, w2
    torch.cuda.synchronize()
    M = T * k                       # every expert is local
    gated = cfg["act"] != "srelu"
    n1 = 2 * I if gated else I
    flops = {"fc1": 2.0 * M * H * n1, "fc2": 2.0 * M * H * I,
             "fc2_dgrad": 2.0 * M * H * I, "fc1_dgrad": 2.0 * M * H * n1}
    if args.wgrad:
        flops.update(wgrad_dw1=2.0 * M * H * n1, wgrad_dw2=2.0 * M * H * I)
    flops_step = sum(flops.values())

    # events per step: 0 start, 1-3 forward GEMMs (library), 4 after
    # unpermute, 5-7 backward GEMMs (library), 8 after dX unpermute; with
    # --wgrad 9-11 around the weight-gradient GEMMs (library); with
    # --recompute the last one before the z rebuild (which ends at 5)
    n_ev = 12 if args.wgrad else 9
    if args.unfused:
        n_ev = 11
    ev_rc = None
    if args.recompute:
        ev_rc = n_ev
        n_ev += 1
    # MX layers quantize the bf16 master weights in every step (they change
    # every training step), right after the routing, skipping the experts
    # that received no rows; the event before it closes the routing
    qw_in_step = prec != "bf16" and not args.cached_weights
    ev_qw = None
    if qw_in_step:
        ev_qw = n_ev
        n_ev += 1

    def cur_stream():
        return torch.cuda.current_stream().cuda_stream

    class _Rec:   # events of one step, recorded on the library's stream
        def __init__(self, evs, base):
            self.evs, self.base = evs, base

        def record(self, i):
            self.evs.record(self.base + i, cur_stream())

    def quantize_weights(evs, base):
        if qw_in_step:
            if evs is not None:
                evs.record(base + ev_qw, cur_stream())
            blk.quantize_weights(live_only=True)

    def step_unfused(evs=None, base=0):
        # 0 start; 1-4 forward GEMM / act / GEMM boundaries; 5 after the
        # unpermute; 6-9 backward boundaries; 10 after the dX unpermute
        if evs is not None:
            evs.record(base + 0, cur_stream())
        blk.route(idx, probs, x)
        quantize_weights(evs, base)
        blk.experts_forward_unfused(None if evs is None else _Rec(evs, base + 1))
        blk.combine(blk.yp, blk.out)
        if evs is not None:
            evs.record(base + 5, cur_stream())
        if mx:
            blk.gather(dout, None, blk.dyp_q, blk.dyp_s)
        else:
            blk.gather(dout, blk.dyp)
        blk.experts_backward_unfused(None if evs is None else _Rec(evs, base + 6))
        blk.combine(blk.dxp, blk.dx, dprobs=True)
        if evs is not None:
            evs.record(base + 10, cur_stream())

    def step(evs=None, base=0):
        if args.unfused:
            return step_unfused(evs, base)
        if evs is not None:
            evs.record(base + 0, cur_stream())
        blk.route(idx, probs, x)
        quantize_weights(evs, base)
        blk.experts_forward(None if evs is None else
                            [evs.ev[base + 1], evs.ev[base + 2], evs.ev[base + 3]])
        blk.combine(blk.yp, blk.out)
        if evs is not None:
            evs.record(base + 4, cur_stream())
        blk.gather(dout, blk.dyp, *blk._mx_dst("dyp"))
        if args.recompute:
            if evs is not None:
                evs.record(base + ev_rc, cur_stream())
            blk.recompute_z()
        blk.experts_backward(None if evs is None else
                             [evs.ev[base + 5], evs.ev[base + 6], evs.ev[base + 7]])
        blk.combine(blk.dxp, blk.dx, dprobs=True)
        if evs is not None:
            evs.record(base + 8, cur_stream())
        if args.wgrad:
            blk.weight_grads(None if evs is None else
                             [evs.ev[base + 9], evs.ev[base + 10], evs.ev[base + 11]])

    if args.calib_copy_mb:
        n = args.calib_copy_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {n} bytes done")
        del src, dst

    # ---- eager warm-up, then the step captured in one graph ----
    log(f"{log_prefix}eager warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the grouped GEMMs of one step, in launch order: the captured launches
    # keep their clock-trace record areas, so every replay rewrites them
    gemm_names = (["fc1", "fc2"] + (["fc1_recompute"] if args.recompute else []) +
                  ["fc2_dgrad", "fc1_dgrad"] + (["wgrad_dw1", "wgrad_dw2"] if args.wgrad else []))
    trace = GemmClockTrace(dev, len(gemm_names))
    gstream = torch.cuda.Stream()
    gstream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gstream):
        step()
        torch.cuda.synchronize()
        trace.start()
        try:
            with torch.cuda.graph(graph, stream=gstream, capture_error_mode="global"):
                step()
        finally:
            trace.stop()
    torch.cuda.synchronize()
    log(f"{log_prefix}graph warmup {args.warmup}")
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    stream = cur_stream()
    ge = HipEvents(2 * args.steps)
    log(f"{log_prefix}timing {args.steps} graph replays")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ge.record(2 * i, stream)
        graph.replay()
        ge.record(2 * i + 1, stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    per = sorted(ge.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps))
    ge.close()
    # the GEMMs' clocks in the last timed replay
    clk_list = trace.clocks()
    gemm_clock = (dict(zip(gemm_names, clk_list)) if clk_list is not None
                  else {n: None for n in gemm_names})
    del graph, trace
    timing = {"method": "HIP graph replays of the whole step (global capture mode)",
              "mean_ms": round(ms_step, 4), "median_ms": round(_pct(per, 0.5), 4),
              "p10_ms": round(_pct(per, 0.1), 4), "p90_ms": round(_pct(per, 0.9), 4)}

    # ---- eager pass with events between the kernels ----
    n_eager = min(args.steps, 10)
    evs = HipEvents(n_ev * n_eager)
    torch.cuda.synchronize()
    te = time.perf_counter()
    for i in range(n_eager):
        step(evs, n_ev * i)
    torch.cuda.synchronize()
    timing["eager_ms_per_step"] = round((time.perf_counter() - te) * 1e3 / n_eager, 4)

    def seg(a, b):
        return sum(evs.elapsed_ms(n_ev * i + a, n_ev * i + b) for i in range(n_eager)) / n_eager

    r1 = ev_qw if qw_in_step else 1    # the weight quantization follows the routing
    if args.unfused:
        seg_ms = {"route_permute_x": seg(0, r1), "fc1": seg(1, 2), "act_fwd": seg(2, 3),
                  "fc2": seg(3, 4), "unpermute_out": seg(4, 5), "permute_dout": seg(5, 6),
                  "fc2_dgrad": seg(6, 7), "act_bwd": seg(7, 8), "fc1_dgrad": seg(8, 9),
                  "unpermute_dx": seg(9, 10)}
    else:
        seg_ms = {"route_permute_x": seg(0, r1), "fc1": seg(1, 2), "fc2": seg(2, 3),
                  "unpermute_out": seg(3, 4), "permute_dout": seg(4, 5),
                  "fc2_dgrad": seg(5, 6), "fc1_dgrad": seg(6, 7), "unpermute_dx": seg(7, 8)}
    if args.wgrad:
        seg_ms.update(wgrad_quantize=seg(8, 9), wgrad_dw1=seg(9, 10), wgrad_dw2=seg(10, 11))
    if args.recompute:
        seg_ms.update(permute_dout=seg(4, ev_rc), fc1_recompute=seg(ev_rc, 5))
    if qw_in_step:
        seg_ms["quantize_weights"] = seg(ev_qw, 1)
    evs.close()
    assert int(blk.err_flag.cpu()[0]) == 0
    value = flops_step / (ms_step * 1e-3) / 1e12

    # HBM-bound steps: algorithmic bytes
    fused4 = prec == "mxfp4" and not args.unfused
    row_bytes = H * (1 + 1 / 32) if mx else (H * (0.5 + 1 / 32) if fused4 else 2 * H)
    idx_bytes = T * k * 4 * 2 + T * k * 4 + M * 8
    kernels = {}
    if args.recompute:
        flops_k = dict(flops, fc1_recompute=flops["fc1"])   # not model work
    else:
        flops_k = flops
    for name in ("fc1", "fc2", "fc2_dgrad", "fc1_dgrad") + (
            ("wgrad_dw1", "wgrad_dw2") if args.wgrad else ()) + (
            ("fc1_recompute",) if args.recompute else ()):
        kernels[name] = {"ms": round(seg_ms[name], 4), "unit": "TFLOP/s",
                         "rate": round(flops_k[name] / (seg_ms[name] * 1e-3) / 1e12, 2)}
        if gemm_clock.get(name):
            kernels[name]["shader_clock_ghz"] = round(gemm_clock[name], 4)
    mem = {"route_permute_x": T * H * 2 + M * row_bytes + idx_bytes,
           "unpermute_out": M * H * 2 + T * H * 2 + T * k * 4,
           "permute_dout": T * H * 2 + M * row_bytes + T * k * 4,
           "unpermute_dx": M * H * 2 + T * H * 2 + T * k * 12}
    if args.unfused:
        # the separate activation passes: z in, a out; dA and z in, dz out
        # (MXFP8: plus the quantize passes, bf16 read twice, codes + scales
        # written rowwise and transposed)
        q = (2 * 2 + 2 * (1 + 1 / 32)) if mx else 0.0
        mem["act_fwd"] = M * n1 * 2 + M * I * 2 + M * I * q
        mem["act_bwd"] = M * I * 2 + 2 * M * n1 * 2 + M * 4 + M * n1 * q
    if args.wgrad and (mx or prec == "mxfp4"):
        # MX transposed copies of Xp and dYp (bf16 in, codes + scales out)
        mem["wgrad_quantize"] = 2 * M * H * (2 + (1 if mx else 0.5) + 1 / 32)
    if qw_in_step:
        # the two weights of every expert that has rows, read once each,
        # both MX copies of each written
        live = int((blk.split_sizes > 0).sum().item())
        n_w = live * (n1 * H + H * I)
        mem["quantize_weights"] = n_w * (2 + 2 * ((1 if mx else 0.5) + 1 / 32))
    for name, b in mem.items():
        kernels[name] = {"ms": round(seg_ms[name], 4), "unit": "GB/s",
                         "rate": round(b / (seg_ms[name] * 1e-3) / 1e9, 1)}
    if (mx or prec == "mxfp4") and not qw_in_step:
        # MX weight copies, timed on their own (--cached-weights: the step
        # reuses copies made before it)
        qe = HipEvents(2)
        reps = 5
        qe.record(0, stream)
        for _ in range(reps):
            blk.quantize_weights()
        qe.record(1, stream)
        torch.cuda.synchronize()
        q_ms = qe.elapsed_ms(0, 1) / reps
        qe.close()
        n_w = E * n1 * H + E * H * I             # both copies of each weight in one pass
        q_bytes = n_w * (2 + 2 * ((1 if mx else 0.5) + 1 / 32))
        kernels["quantize_weights"] = {"ms": round(q_ms, 4), "unit": "GB/s",
                                       "rate": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
                                       "outside_step": True}
    # the clock of the step's GEMMs, weighted by their times
    gk = [(kernels[n]["ms"], gemm_clock[n]) for n in gemm_names if gemm_clock.get(n)]
    timing["gemm_shader_clock_ghz"] = (
        round(sum(ms * c for ms, c in gk) / sum(ms for ms, _ in gk), 4)
        if len(gk) == len(gemm_names) else None)
    timing["clock_method"] = ("each grouped-GEMM launch of the last timed replay: shader "
                              "cycles over constant-rate ticks of its persistent workgroups, "
                              "weighted by the GEMMs' times")
    sizes = blk.split_sizes.cpu().tolist()
    del blk
    torch.cuda.empty_cache()
    fc1_ms = seg_ms["fc1"]
    return {"cfg": cfg, "E": E, "k": k, "T": T, "H": H, "I": I, "M": M, "prec": prec,
            "flops": flops, "flops_step": flops_step, "ms_step": ms_step, "value": value,
            "timing": timing, "kernels": kernels, "fc1_ms": fc1_ms,
            "fc1_rate": flops["fc1"] / (fc1_ms * 1e-3) / 1e12,
            "skew": {"max_over_mean": round(max(sizes) / (sum(sizes) / len(sizes)), 3),
                     "empty_groups": sum(1 for n in sizes if n == 0)}}


def router_timing(T, E, k, dev):
    """The top-k router (softmax over the experts, top-k) on logits of the
    config's shape, launched from a captured graph so the host's launch
    rate is not what is timed; outside the step, whose routing is an
    input."""
    import torch
    import moe_grouped_mlp_amd as mg
    lg = torch.randn(T, E, device=dev, dtype=torch.float32)
    r_idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    r_p = torch.empty(T, k, dtype=torch.float32, device=dev)
    reps = 20
    gstream = torch.cuda.Stream()
    gstream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gstream):
        mg.moe_router_topk(T=T, E=E, k=k, logits=lg, expert_idx=r_idx, probs=r_p,
                           stream=gstream.cuda_stream)
        with torch.cuda.graph(graph, stream=gstream):
            for _ in range(reps):
                mg.moe_router_topk(T=T, E=E, k=k, logits=lg, expert_idx=r_idx,
                                   probs=r_p, stream=gstream.cuda_stream)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    re = HipEvents(2)
    re.record(0, stream)
    graph.replay()
    re.record(1, stream)
    torch.cuda.synchronize()
    r_ms = re.elapsed_ms(0, 1) / reps
    re.close()
    del graph
    return {"ms": round(r_ms, 4), "unit": "GB/s",
            "rate": round((T * E * 4 + T * k * 8) / (r_ms * 1e-3) / 1e9, 1),
            "outside_step": True}


# the router shapes: (T tokens, router experts, top-k, local experts)
ROUTING_SHAPES = {
    "mixtral": (8192, 8, 2, 8),
    "gptoss": (16384, 128, 4, 128),
    "dsv3_share": (16384, 256, 8, 32),   # 32 local experts of 256, top-8
}


def routing_timing(dev, reps=20):
    """Router + routing metadata from logits: one launch (moe_router_route)
    against moe_router_topk followed by moe_permute(BUILD_MAP) (four
    launches), both replayed from a captured graph (so the host's launch
    rate is not what is timed), at the Mixtral, GPT-OSS and DSv3-share
    router shapes.  Microseconds per call."""
    import torch
    import moe_grouped_mlp_amd as mg
    out = {}
    for name, (T, E_all, k, E) in ROUTING_SHAPES.items():
        g = torch.Generator(device=dev)
        g.manual_seed(1)
        lg = torch.randn(T, E_all, generator=g, device=dev, dtype=torch.float32)
        M_cap = T * k + E * 127
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        bufs = dict(expert_idx=torch.empty(T, k, **i32), probs=torch.empty(T, k, **f32),
                    split_sizes=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                    padded_offsets=torch.empty(E + 1, **i32),
                    row_id_map=torch.empty(T, k, **i32), row_src=torch.empty(M_cap, **i32),
                    probs_p=torch.empty(M_cap, **f32), err_flag=torch.zeros(1, **i32))
        ws_f = torch.zeros(mg.moe_router_route_workspace_size(T, E_all, E), dtype=torch.uint8,
                           device=dev)
        ws_p = torch.empty(mg.moe_permute_workspace_size(T, E), dtype=torch.uint8, device=dev)

        def fused(st):
            mg.moe_router_route(T=T, E_total=E_all, k=k, E=E, M_cap=M_cap, logits=lg,
                                workspace=ws_f, stream=st, **bufs)

        def separate(st):
            mg.moe_router_topk(T=T, E=E_all, k=k, logits=lg, expert_idx=bufs["expert_idx"],
                               probs=bufs["probs"], stream=st)
            mg.moe_permute(flags=mg.PERMUTE_BUILD_MAP, T=T, k=k, E=E, H=64, M_cap=M_cap,
                           expert_idx=bufs["expert_idx"], probs=bufs["probs"],
                           split_sizes=bufs["split_sizes"], offsets=bufs["offsets"],
                           padded_offsets=bufs["padded_offsets"],
                           row_id_map=bufs["row_id_map"], row_src=bufs["row_src"],
                           probs_p=bufs["probs_p"], err_flag=bufs["err_flag"],
                           workspace=ws_p, stream=st)

        def router_only(st):
            mg.moe_router_topk(T=T, E=E_all, k=k, logits=lg, expert_idx=bufs["expert_idx"],
                               probs=bufs["probs"], stream=st)

        res = {}
        for label, fn in (("fused_us", fused), ("router_plus_metadata_4_launches_us", separate),
                          ("router_only_us", router_only)):
            gs = torch.cuda.Stream()
            gs.wait_stream(torch.cuda.current_stream())
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(gs):
                fn(gs.cuda_stream)
                with torch.cuda.graph(graph, stream=gs):
                    for _ in range(reps):
                        fn(gs.cuda_stream)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            stream = torch.cuda.current_stream().cuda_stream
            ev = HipEvents(2)
            ev.record(0, stream)
            graph.replay()
            ev.record(1, stream)
            torch.cuda.synchronize()
            res[label] = round(ev.elapsed_ms(0, 1) / reps * 1e3, 2)
            ev.close()
            del graph
        assert int(bufs["err_flag"].cpu()[0]) == 0
        res["shape"] = f"T={T} E_total={E_all} k={k} local E={E}"
        out[name] = res
        log(f"routing {name}: fused {res['fused_us']} us, four launches "
            f"{res['router_plus_metadata_4_launches_us']} us, router alone "
            f"{res['router_only_us']} us")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral", choices=sorted(BENCH_CONFIGS))
    ap.add_argument("--prec", choices=("bf16", "mxfp8", "mxfp4"), default=None,
                    help="operand precision (default: the config's)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary Mixtral MXFP8 and the other-layer measurements "
                         "of the default run")
    ap.add_argument("--unfused", action="store_true",
                    help="the unfused baseline (bf16): plain grouped GEMMs with the "
                         "activation and its gradient as separate passes")
    ap.add_argument("--gemm", action="store_true",
                    help="time the FC2-shaped plain grouped GEMM in bf16, MXFP8 and MXFP4")
    ap.add_argument("--cached-weights", action="store_true",
                    help="MX layers: reuse weight copies made before the step (as over "
                         "the microbatches of one optimizer step) instead of quantizing "
                         "the bf16 master weights inside it")
    ap.add_argument("--recompute", action="store_true",
                    help="activation recompute: the forward stores no z, the backward "
                         "rebuilds it with FC1's GEMM (timed as fc1_recompute)")
    ap.add_argument("--wgrad", action="store_true",
                    help="add the weight-gradient grouped GEMMs (dW1, dW2) to the "
                         "step: a full training step of the layer")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="before timing, run one device copy of this many MB "
                         "(a known-size kernel for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.gemm:
        return gemm_bench(args)

    import torch

    _, prec_default = BENCH_CONFIGS[args.config]
    prec = args.prec or prec_default
    if args.unfused and (args.wgrad or args.recompute):
        print("--unfused is the baseline of the fused step (no --wgrad, --recompute)",
              file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    r = measure(args, args.config, prec)
    E, k, T, H, I, M = (r[n] for n in ("E", "k", "T", "H", "I", "M"))
    cfg = r["cfg"]
    kernels = r["kernels"]
    kernels["router_topk"] = router_timing(T, E, k, dev)
    routing = routing_timing(dev)
    ceiling = copy_ceiling_gbs(dev)
    for name in ("route_permute_x", "unpermute_out", "permute_dout", "unpermute_dx"):
        kernels[name]["frac_of_copy"] = round(kernels[name]["rate"] / ceiling, 3)
    peak = PEAK_TFLOPS[prec]
    value, ms_step = r["value"], r["ms_step"]
    clock = r["timing"]["gemm_shader_clock_ghz"]
    log(f"step {ms_step:.3f} ms (median {r['timing']['median_ms']:.3f}), {value:.1f} TFLOP/s; " +
        ", ".join(f"{n} {v['ms']:.3f} ms {v['rate']} {v['unit']}" for n, v in kernels.items()))

    # secondary: the same Mixtral layer with MXFP8 operands, in the same run
    secondary = None
    if (args.config == "mixtral" and prec == "bf16" and not args.no_secondary
            and not (args.unfused or args.wgrad or args.recompute)):
        s = measure(args, "mixtral_mx", "mxfp8", log_prefix="secondary: ")
        pk8 = PEAK_TFLOPS["mxfp8"]
        secondary = {
            "config": "mixtral_mx expert layer, MXFP8 operands (E4M3 with E8M0 scales per 32 "
                      "along K), bf16 master weights quantized inside the step, fused quantize "
                      "+ transposed copies in the FC1 and dSwiGLU epilogues",
            "value": round(s["value"], 3), "unit": "TFLOP/s", "ms_per_step": round(s["ms_step"], 4),
            "pct_mfma_peak": round(100.0 * s["value"] / pk8, 2), "timing": s["timing"],
            "pct_mfma_peak_at_measured_clock": (
                round(100.0 * s["value"] / (pk8 * s["timing"]["gemm_shader_clock_ghz"] / 2.4), 2)
                if s["timing"]["gemm_shader_clock_ghz"] else None),
            "kernels": s["kernels"],
            "roofline": {"bound": "mfma", "kernel": "FC1 grouped GEMM + activation epilogue "
                                                    "(MXFP8)",
                         "achieved": round(s["fc1_rate"], 3), "peak": pk8, "unit": "TFLOP/s",
                         "frac": round(s["fc1_rate"] / pk8, 4), "traffic": None,
                         "avg_launch_ms": round(s["fc1_ms"], 4)},
        }
        qw = s["kernels"].get("quantize_weights", {}).get("ms")
        if qw is not None and not s["kernels"]["quantize_weights"].get("outside_step"):
            # the same step less the weight quantization (once per optimizer
            # step, so shared by the microbatches of gradient accumulation):
            # derived from the eager pass's segment time, not timed apart
            ms_wo = s["ms_step"] - qw
            secondary["weight_quantize_ms"] = qw
            secondary["ms_per_step_without_weight_quantize"] = round(ms_wo, 4)
            secondary["value_without_weight_quantize"] = round(
                s["flops_step"] / (ms_wo * 1e-3) / 1e12, 3)
        log(f"secondary MXFP8: step {s['ms_step']:.3f} ms, {s['value']:.1f} TFLOP/s "
            f"({100 * s['value'] / pk8:.1f}% of fp8 peak)")

    # the other layers the pages measure, each at its own configuration, in
    # the same run (GPT-OSS: MXFP8 with beta 1.702 and clamp 7; DSv3 share:
    # bf16 and MXFP8); compact lines, the full ones come from --config
    others = None
    if (args.config == "mixtral" and prec == "bf16" and not args.no_secondary
            and not (args.unfused or args.wgrad or args.recompute)):
        others = {}
        for oc, op in (("gptoss", "mxfp8"), ("dsv3", "bf16"), ("dsv3", "mxfp8")):
            o = measure(args, oc, op, log_prefix=f"{oc} {op}: ")
            pko = PEAK_TFLOPS[op]
            ck = o["timing"]["gemm_shader_clock_ghz"]
            others[f"{oc}_{op}"] = {
                "workload": f"{oc} expert layer: E={o['E']} top-{o['k']} T={o['T']} "
                            f"H={o['H']} I={o['I']} {o['cfg']['act']} beta={o['cfg']['beta']} "
                            f"clamp={o['cfg']['clamp']}, {op}",
                "value": round(o["value"], 3), "unit": "TFLOP/s",
                "ms_per_step": round(o["ms_step"], 4),
                "median_ms": o["timing"]["median_ms"], "p10_ms": o["timing"]["p10_ms"],
                "p90_ms": o["timing"]["p90_ms"],
                "pct_mfma_peak": round(100.0 * o["value"] / pko, 2),
                "pct_mfma_peak_at_measured_clock": (
                    round(100.0 * o["value"] / (pko * ck / 2.4), 2) if ck else None),
                "gemm_shader_clock_ghz": ck, "group_skew": o["skew"],
                "kernel_ms": {n: v["ms"] for n, v in o["kernels"].items()},
            }
            log(f"{oc} {op}: step {o['ms_step']:.3f} ms, {o['value']:.1f} TFLOP/s "
                f"({100 * o['value'] / pko:.1f}% of {op} peak)")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(cfg, args.seed, mx=prec == "mxfp8")
        log(f"cpu oracle {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads")

    # the recorded counters are those of FC1 storing z
    traffic = (measured_traffic() if (args.config == "mixtral" and prec == "bf16"
                                      and not args.recompute and not args.unfused)
               else None)
    out = {
        "metric": "fused grouped-MLP fwd/bwd TFLOP/s and % MFMA peak, Mixtral-shaped "
                  "layer, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "pct_mfma_peak": round(100.0 * value / peak, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "mxfp8": "mxfp8-e4m3", "mxfp4": "mxfp4-e2m1"}[prec],
        "data": "synthetic",
        "config": {"workload": f"{args.config} expert layer: E={E} top-{k} T={T} H={H} "
                               f"I={I} {cfg['act']} beta={cfg['beta']} clamp={cfg['clamp']}, "
                               f"{prec}, "
                               f"{'weight quantization (bf16 masters -> MX copies)+' if prec != 'bf16' and not args.cached_weights else ''}"
                               f"route+permute+FC1+FC2+unpermute and backward "
                               f"(FC2 dgrad+dAct, FC1 dgrad, dX, dprobs"
                               f"{', dW1, dW2' if args.wgrad else ''})"
                               f"{'; unfused baseline (plain GEMMs + separate activation passes)' if args.unfused else ''}"
                               f"{'; activation recompute (z rebuilt in the backward, its FLOPs not counted)' if args.recompute else ''}",
                   "E": E, "k": k, "T": T, "H": H, "I": I, "routed_rows": M,
                   "prec": prec, "flops_per_step": r["flops_step"],
                   "group_skew": r["skew"]},
        "timing": r["timing"],
        "value_at_median": round(r["flops_step"] / (r["timing"]["median_ms"] * 1e-3) / 1e12, 3),
        "kernels": kernels,
        "copy_ceiling_gbs": round(ceiling, 1),
        "routing_from_logits": routing,
        "roofline": {"bound": "mfma",
                     "kernel": ("FC1 grouped GEMM, plain store (unfused; with the operand "
                                "quantization for MXFP4)" if args.unfused
                                else "FC1 grouped GEMM + activation epilogue"),
                     "achieved": round(r["fc1_rate"], 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(r["fc1_rate"] / peak, 4),
                     "traffic": traffic, "avg_launch_ms": round(r["fc1_ms"], 4)},
        "cpu_baseline": cpu,
    }
    if clock:
        # the dense MFMA peak scales with the shader clock: 2.4 GHz for the
        # published figure; `clock` is the average over the timed replays
        out["measured_clock_ghz"] = clock
        out["pct_mfma_peak_at_measured_clock"] = round(100.0 * value / (peak * clock / 2.4), 2)
        out["roofline"]["frac_at_measured_clock"] = round(
            r["fc1_rate"] / (peak * clock / 2.4), 4)
    if secondary is not None:
        out["secondary"] = secondary
    if others is not None:
        out["other_layers"] = others
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
