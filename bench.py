"""Benchmark of the fused dense attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--configs A,B,..]

One step is one attn_fwd call over the whole workload (all heads, all query
tiles), inputs already resident in device memory.  Prints ONE JSON line.  The
headline figures (value, ms_per_step, roofline) are those of --workload; the
other workloads of --configs (by default the three hd128 bf16 workloads at
S = 4K / 8K / 16K that the metric names) are timed the same way in the same
run and reported under "configs", each with the shader clock and socket power
sampled by amd-smi during an untimed burst of the same launches right after
its timed region.

* value / metric: attention-forward throughput, 4·B·H·S²·D / t, in TFLOP/s.
* roofline: the kernel is MFMA bound (dense bf16 contraction); achieved is the
  algorithmic FLOP per launch over the average launch duration measured with
  HIP events on the launch stream over the timed region; peak is MI355X's dense
  bf16 MFMA figure.  traffic is the HBM bytes per launch measured by rocprofv3
  counters (see profiles/), reported only while the kernel sources still match
  the ones the counters were taken on.
* cpu_baseline: the float64 CPU oracle timed on a bounded sample (whole query
  rows of one head) of the same workload on this host.
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

METRIC = "attn-fwd TFLOP/s (4BHS²D/t) + % bf16 MFMA peak, hd128 bf16 S=4K/8K/16K"
DEFAULT_WORKLOAD = "b2_h16_s8192_d128_bf16"
# The metric's three shapes: hd128 bf16 at S = 4K, 8K and 16K.
METRIC_WORKLOADS = ["b4_h16_s4096_d128_bf16", "b2_h16_s8192_d128_bf16", "b1_h16_s16384_d128_bf16"]
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0}   # MI355X dense MFMA, no sparsity
KERNEL_SOURCES = ["dense_attention_amd/csrc/attn_fwd_kernel.h", "dense_attention_amd/csrc/attn_api.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counters, if they match these sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("kernel_source_hash") != kernel_source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_baseline(w, q, k, v, seconds: float, causal: bool = False):
    """Times the float64 oracle on whole heads of the workload for about `seconds`.

    Heads (b, h) are taken in order until the time budget is spent (at least
    one head); every query row of a sampled head is computed against all of
    its keys, exactly as for the full workload.
    """
    import threadpoolctl
    import workloads as W
    from oracle import attention_forward

    flops = 0.0
    heads = 0
    t0 = time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            qn = W.to_f64(q[b:b + 1, h:h + 1])
            kn = W.to_f64(k[b:b + 1, h:h + 1])
            vn = W.to_f64(v[b:b + 1, h:h + 1])
            attention_forward(qn, kn, vn, w.scale, causal_offset=0 if causal else None)
            flops += 4.0 * w.D * (w.S * (w.S + 1) / 2 if causal else w.S * w.S)
            heads += 1
            if time.perf_counter() - t0 >= seconds:
                break
        else:
            continue
        break
    dt = time.perf_counter() - t0
    blas = [p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()
            if p.get("user_api") == "blas"]
    cores = max(blas) if blas else 1
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{heads} of {w.B * w.H} heads, all {w.S} query rows each against all keys, "
                   f"D={w.D}, float64 numpy (BLAS matmul on {cores} threads, exp single-threaded); "
                   f"{dt:.1f} s on {os.cpu_count()} visible CPUs"),
    }


class ClockSampler:
    """Polls the GPU's shader (gfx) clock and socket power through amd-smi while
    the caller keeps the GPU busy.  Every reading is optional: on any error the
    sampler reports None instead."""

    def __init__(self):
        self.handle = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            self.handle = self._match_device(amdsmi, handles)
            self.smi = amdsmi
        except Exception:
            self.handle = None

    @staticmethod
    def _match_device(amdsmi, handles):
        import torch
        if len(handles) == 1:
            return handles[0]
        prop = torch.cuda.get_device_properties(0)
        bus = getattr(prop, "pci_bus_id", None)
        for h in handles:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)     # "dddd:bb:dd.f"
            if bus is not None and int(bdf.split(":")[1], 16) == bus:
                return h
        return None

    def read(self):
        m = self.smi.amdsmi_get_gpu_metrics_info(self.handle)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int) and c > 0]
        clk = sum(clks) / len(clks) if clks else m.get("current_gfxclk")
        if not isinstance(clk, (int, float)) or clk <= 0:
            clk = self.smi.amdsmi_get_clock_info(self.handle, self.smi.AmdSmiClkType.GFX)["clk"]
        pw = m.get("current_socket_power")
        if not isinstance(pw, (int, float)) or pw <= 0:
            pw = m.get("average_socket_power")
        return float(clk), (float(pw) if isinstance(pw, (int, float)) and pw > 0 else None)

    def sample_during(self, busy, ms: float):
        """Runs ``busy()`` repeatedly for about ``ms`` milliseconds while a thread
        reads the clock every 20 ms; returns the median MHz and W of the readings
        taken after the first second.  The firmware refreshes these metrics about
        once a second, so earlier readings can still describe the load before."""
        import threading
        import torch
        if self.handle is None:
            return None, None
        clks, pws, stop = [], [], threading.Event()

        def poll():
            t_start = time.perf_counter()
            while not stop.is_set():
                try:
                    c, p = self.read()
                    if time.perf_counter() - t_start >= 1.0:
                        clks.append(c)
                        if p is not None:
                            pws.append(p)
                except Exception:
                    pass
                time.sleep(0.02)

        th = threading.Thread(target=poll, daemon=True)
        t0 = time.perf_counter()
        th.start()
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(5):
                busy()
            torch.cuda.synchronize()
        stop.set()
        th.join()
        med = lambda xs: sorted(xs)[len(xs) // 2] if xs else None
        return med(clks), med(pws)


def copy_calibration(args):
    """A plain device-to-device copy of known size (reads N bytes, writes N bytes)."""
    import torch
    n = args.copy_mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    t = ev0.elapsed_time(ev1) * 1e-3 / args.steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "steps": args.steps,
                      "seconds_per_copy": t, "GB_per_s": 2 * n / t / 1e9}), flush=True)


def time_workload(w, args, da, sampler):
    """Times --steps launches of workload ``w`` after the clock settle and the
    warmup, then samples the clock during an untimed burst.  Returns the timing
    record and the host copies of the inputs (for the CPU baseline)."""
    import torch
    import workloads as W

    q, k, v = W.workload_qkv(w)
    dev = torch.device("cuda", 0)
    if args.layout == "bshd":
        qd, kd, vd = (t.transpose(1, 2).contiguous().to(dev).transpose(1, 2) for t in (q, k, v))
        od = torch.empty((w.B, w.S, w.H, w.D), dtype=q.dtype, device=dev).transpose(1, 2)
    else:
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        od = torch.empty_like(qd)
    lsed = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ws = None
    if args.kv_splits >= 0:
        nbytes = da.attn_fwd_split_workspace_size(w.B, w.H, w.S, w.D, args.kv_splits)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)

    def step():
        if args.kv_splits >= 0:
            da.attn_fwd_split(qd, kd, vd, od, lsed, w.scale, kv_splits=args.kv_splits,
                              workspace=ws, stream=stream, variant=args.variant,
                              causal=args.causal)
        elif args.layout == "bshd":
            da.attn_fwd_strided(qd, kd, vd, od, lsed, w.scale, stream=stream, variant=args.variant,
                                causal=args.causal)
        else:
            da.attn_fwd_ex(qd, kd, vd, od, lsed, w.scale, stream=stream, variant=args.variant,
                           causal=args.causal)

    # Clock settle (untimed): the first ~100 ms of load run at transitional clocks.
    t_settle = time.perf_counter()
    while args.settle_ms > 0 and (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: exactly --steps launches, bracketed by device synchronisations.
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_s = ev0.elapsed_time(ev1) * 1e-3 / args.steps      # average launch duration
    step_s = wall / args.steps
    # Untimed: the shader clock and power the same launches sustain.
    clk, pw = sampler.sample_during(step, args.clock_ms) if args.clock_ms > 0 else (None, None)

    # 4·D FLOP per visible score: B·H·S² without a mask, B·H·S(S+1)/2 with it.
    flops = w.flops if not args.causal else 4.0 * w.D * w.B * w.H * w.S * (w.S + 1) / 2
    peak = PEAK_TFLOPS[w.dtype]
    rec = {
        "ms_per_step": round(step_s * 1e3, 4),
        "kernel_ms": round(kernel_s * 1e3, 4),
        "tflops": round(flops / step_s / 1e12, 2),
        "pct_of_peak": round(100.0 * flops / step_s / 1e12 / peak, 2),
        "roofline_frac": round(flops / kernel_s / 1e12 / peak, 4),
        "gfx_clock_mhz": None if clk is None else round(clk),
        "socket_power_w": None if pw is None else round(pw),
        "kernel": da.attn_get_config(w.B, w.H, w.S, w.D, q.dtype, variant=args.variant,
                                     causal=args.causal),
    }
    del qd, kd, vd, od, lsed, ws
    torch.cuda.empty_cache()
    return rec, flops, step_s, kernel_s, (q, k, v)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--configs", default=None,
                    help="comma-separated workloads timed in the same run and reported under "
                         "'configs' (default: the metric's three hd128 workloads when --workload "
                         "is one of them, else --workload alone; 'none' for --workload alone)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the oracle's CPU-baseline sample (0 skips it)")
    ap.add_argument("--variant", type=int, default=0)
    ap.add_argument("--kv-splits", type=int, default=-1,
                    help="-1: attn_fwd; 0: attn_fwd_split with the library's split count; "
                         "n > 0: attn_fwd_split with at most n key ranges (partials + merge)")
    ap.add_argument("--causal", action="store_true",
                    help="causal mask (query i sees keys j <= i); FLOPs count visible scores only")
    ap.add_argument("--layout", choices=["bhsd", "bshd"], default="bhsd",
                    help="bshd: inputs and output stored token-major [B, S, H, D], run through "
                         "attn_fwd_strided without conversion copies")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed back-to-back launches before the warmup steps, so GPU clocks "
                         "reach their loaded steady state (0 disables)")
    ap.add_argument("--clock-ms", type=float, default=1300.0,
                    help="untimed launches after each timed region while amd-smi samples the "
                         "shader clock and power; readings count after the first second "
                         "(0 disables)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of attention, time a plain device copy of this many MiB "
                         "(calibrates the HBM byte counters of rocprofv3)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only (the attention forward runs on one device's "
              "share; there is no multi-GPU path). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_attention_amd as da
    import workloads as W

    if args.copy_mib > 0:
        return copy_calibration(args)
    if args.kv_splits >= 0 and args.layout != "bhsd":
        sys.exit("bench.py: --kv-splits runs on the contiguous [B, H, S, D] layout only")

    if args.configs is None:
        names = METRIC_WORKLOADS if args.workload in METRIC_WORKLOADS else [args.workload]
    elif args.configs == "none":
        names = [args.workload]
    else:
        names = [n for n in args.configs.split(",") if n]
    names = [args.workload] + [n for n in names if n != args.workload]   # headline first
    for n in names:
        if n not in W.BY_NAME:
            sys.exit(f"bench.py: unknown workload {n}; known: {', '.join(W.BY_NAME)}")

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    sampler = ClockSampler()
    per = {}
    head = None
    for n in names:
        rec, flops, step_s, kernel_s, host = time_workload(W.BY_NAME[n], args, da, sampler)
        per[n] = rec
        if head is None:
            head = (W.BY_NAME[n], rec, flops, step_s, kernel_s, host)

    w, rec, flops, step_s, kernel_s, (q, k, v) = head
    value = flops / step_s / 1e12
    achieved = flops / kernel_s / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: iid N(0,1) q/k/v from numpy PCG64 seed, rounded to dtype",
        "config": dict(w.as_dict(), kernel=rec["kernel"],
                       api=("attn_fwd" if args.kv_splits < 0 and args.layout == "bhsd"
                            else "attn_fwd_strided" if args.kv_splits < 0
                            else f"attn_fwd_split(kv_splits={args.kv_splits})"),
                       layout=args.layout, causal=args.causal),
        "pct_of_peak": round(100.0 * value / peak, 2),
        "gfx_clock_mhz": rec["gfx_clock_mhz"],
        "socket_power_w": rec["socket_power_w"],
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(w.name),
        },
        "configs": per,
        "cpu_baseline": None,
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds, args.causal)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
