"""Benchmark of the fused grouped-MLP MoE expert block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config mixtral]

One step = the whole hot path of a training step of one expert layer:
route + permute (X), FC1 grouped GEMM with the fused SwiGLU + prob-scale
epilogue, FC2 grouped GEMM, unpermute; permute (dOut), FC2 dgrad grouped GEMM
with the fused dSwiGLU epilogue, FC1 dgrad grouped GEMM, unpermute (dX) +
dprobs.  Inputs are synthetic (seeded), already resident in HBM when the
timed region starts.  The value is algorithmic GEMM TFLOP/s of the step:
12 * M * H * I flops (M = routed rows; no padding counted).

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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0

WORKLOADS = {
    # name: (E, k, T, H, I, beta, clamp, logit routing)
    "mixtral": dict(E=8, k=2, T=8192, H=4096, I=14336, beta=1.0, clamp=None),
    "gptoss": dict(E=128, k=4, T=16384, H=2880, I=2880, beta=1.702, clamp=7.0),
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
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev.append(h.value)

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[a], self.ev[b])
        assert rc == 0, rc
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


GEMM_SRC = os.path.join(ROOT, "moe_grouped_mlp_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fc1_mixtral_traffic.json")


def gemm_source_hash():
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


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
    """Seeded synthetic inputs drawn on the device: X, dOut ~ N(0,1) bf16,
    weights ~ N(0, 0.02^2) bf16, router logits ~ N(0,1) -> fp32 softmax ->
    top-k (descending probability, no renormalisation)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    E, k, T, H, I = (cfg[n] for n in ("E", "k", "T", "H", "I"))
    bf = torch.bfloat16
    x = torch.randn(T, H, generator=g, device=device).to(bf)
    dout = torch.randn(T, H, generator=g, device=device).to(bf)
    w1 = torch.empty(E, 2 * I, H, dtype=bf, device=device)
    w2 = torch.empty(E, H, I, dtype=bf, device=device)
    for e in range(E):
        w1[e] = (torch.randn(2 * I, H, generator=g, device=device) * 0.02).to(bf)
        w2[e] = (torch.randn(H, I, generator=g, device=device) * 0.02).to(bf)
    logits = torch.randn(T, E, generator=g, device=device)
    p = torch.softmax(logits, dim=1)
    probs, idx = torch.topk(p, k, dim=1)
    return x, dout, w1, w2, idx.to(torch.int32).contiguous(), probs.contiguous()


def cpu_baseline(cfg, seed, target_s=15.0):
    """Time the CPU oracle (as it stands) on a bounded sample of the same
    workload: the rows routed to expert 0, full H and I, forward + backward."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import moe as om
    from workloads.gen import _normal_bf16, route_inputs, CONFIGS

    E, k, T, H, I = (cfg[n] for n in ("E", "k", "T", "H", "I"))
    idx, probs = route_inputs(dict(CONFIGS["mixtral"]), seed, T, E, k)
    t_sel, s_sel = np.nonzero(idx == 0)
    rows = 64
    rng = np.random.default_rng(seed + 7)
    w1 = _normal_bf16(rng, (1, 2 * I, H), 0.02)
    w2 = _normal_bf16(rng, (1, H, I), 0.02)
    prm = om.ActParams.clamped(cfg["clamp"], beta=cfg["beta"])
    done_flops, t_used, runs = 0.0, 0.0, 0
    while True:
        n = min(rows, len(t_sel))
        x = _normal_bf16(rng, (n, H), 1.0)
        dout = _normal_bf16(rng, (n, H), 1.0)
        sub_idx = np.zeros((n, 1), np.int32)
        sub_p = probs[t_sel[:n], s_sel[:n]].reshape(n, 1)
        t0 = time.perf_counter()
        fw = om.forward(x, w1, w2, sub_idx, sub_p, 1, prm)
        om.backward(fw, dout, w1, w2, prm)
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
            "sample": (f"oracle forward+backward on rows routed to expert 0 of the "
                       f"{E}-expert layer (H={H}, I={I}, bf16 storage, fp64 math), "
                       f"{runs} runs, {done_flops / 1e12:.3f} TFLOP in {t_used:.1f} s")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral", choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="before timing, run one device copy of this many MB "
                         "(a known-size kernel for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_grouped_mlp_amd as mg

    cfg = WORKLOADS[args.config]
    E, k, T, H, I = (cfg[n] for n in ("E", "k", "T", "H", "I"))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"generating {args.config} inputs on the device")
    x, dout, w1, w2, idx, probs = device_inputs(cfg, args.seed, dev)
    act = mg.act_params(mg.ACT_SWIGLU, beta=cfg["beta"], clamp=cfg["clamp"])
    blk = mg.ExpertBlock(E, H, I, T, k, act=act)
    blk.load_weights(w1, w2)
    del w1, w2
    M = T * k
    flops_step = 12.0 * M * H * I
    flops_fc1 = 4.0 * M * H * I

    def step(ev=None):
        blk.forward(x, idx, probs, timing_events=ev)
        blk.backward(dout)

    if args.calib_copy_mb:
        n = args.calib_copy_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {n} bytes done")
        del src, dst

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = HipEvents(2 * args.steps)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step((evs.ev[2 * i], evs.ev[2 * i + 1], None))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    fc1_ms = sum(evs.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)) / args.steps
    evs.close()
    assert int(blk.err_flag.cpu()[0]) == 0
    value = flops_step / (ms_step * 1e-3) / 1e12
    achieved = flops_fc1 / (fc1_ms * 1e-3) / 1e12
    log(f"step {ms_step:.3f} ms, {value:.1f} TFLOP/s; FC1 {fc1_ms:.3f} ms {achieved:.1f} TFLOP/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(cfg, args.seed)
        log(f"cpu oracle {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads")

    out = {
        "metric": "fused grouped-MLP fwd/bwd TFLOP/s and % MFMA peak, Mixtral-shaped "
                  "layer, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "pct_bf16_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.config} expert layer: E={E} top-{k} T={T} H={H} "
                               f"I={I} SwiGLU, bf16, route+permute+FC1+FC2+unpermute "
                               f"and backward (FC2 dgrad+dSwiGLU, FC1 dgrad, dX, dprobs)",
                   "E": E, "k": k, "T": T, "H": H, "I": I, "routed_rows": M,
                   "flops_per_step": flops_step},
        "roofline": {"bound": "mfma", "kernel": "FC1 grouped GEMM + SwiGLU epilogue",
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(), "avg_launch_ms": round(fc1_ms, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
