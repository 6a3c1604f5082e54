#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
fa_fwd (tiled QK^T, online softmax, PV, O + LSE) followed by fa_bwd (row dot,
recomputed P, dV, dP, dS, dK, dQ). The default workload is the long-context
self-attention shape B=1, H=32, N=8192, d=128, bf16, non-causal; its inputs
(Q, K, V, dO) are resident in HBM before the timed region starts.

FLOPs follow the attention convention: forward 4*N^2*d per head (halved under
causal masking), backward 2.5x that. Prints ONE JSON line.

`--suite` instead times the general-shape workloads (a sliding window, new
queries over a long key cache, fp16, a [B, N, H, d] layout, head dimensions
32, 96 and 256, an additive per-head bias) through
fa_fwd_ex / fa_bwd_ex and prints one JSON line per workload; there FLOPs are
4*d per visible (query, key) pair, counted exactly for the mask.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s (4·N²·d per head) and % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0


# HBM bytes per launch of the forward kernel, from the FETCH_SIZE / WRITE_SIZE
# counter passes summarised in this file (scaled by a copy of known size). The
# figure is only reported while the kernel's sources hash to the recorded value.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_bf16_n8192_d128_hbm_bytes.md")
FWD_SOURCES = ("fa_device.h", "fa_fwd_mfma.hip", "fa_kernels.h")


def fwd_source_sha256():
    h = hashlib.sha256()
    for name in FWD_SOURCES:
        with open(os.path.join(ROOT, "exact_attention_122_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


TRAFFIC_WORKLOAD = "fwd_n8192_d128"   # the workload the counter passes ran


def measured_traffic(kernel):
    """Counter-derived HBM bytes per launch of `kernel` on TRAFFIC_WORKLOAD, or
    None if not measured for the current sources."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"kernel=(\S+) read_bytes=(\d+) write_bytes=(\d+) traffic_bytes=(\d+) "
                  r"source_sha256=([0-9a-f]{64})", text)
    if not m or m.group(1) != kernel or m.group(5) != fwd_source_sha256():
        return None
    return int(m.group(4))


def attention_flops(B, H, N, d, causal):
    f = 4.0 * N * N * d * B * H
    return f / 2 if causal else f


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fwd_n8192_d128")
    ap.add_argument("--causal", type=int, default=None, help="override the workload's mask")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=32, help="heads the CPU oracle times (at most B*H)")
    ap.add_argument("--fwd-only", action="store_true", help="time fa_fwd alone (profiling aid)")
    ap.add_argument("--suite", action="store_true",
                    help="time the general-shape workloads instead (one JSON line each)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run a plain device copy of MIB MiB (read + write) instead, to scale "
                         "hardware byte counters")
    return ap.parse_args()


def visible_pairs(nq, nk, window):
    """(query, key) pairs a band mask keeps: query i sees keys
    [i + nk - nq - left, i + nk - nq + right] within [0, nk)."""
    import numpy as np
    left, right = window
    a = np.arange(nq, dtype=np.int64) + (nk - nq)
    lo = np.zeros(nq, np.int64) if left is None else np.maximum(0, a - left)
    hi = np.full(nq, nk - 1, np.int64) if right is None else np.minimum(nk - 1, a + right)
    return int(np.maximum(0, hi - lo + 1).sum())


SUITE = ("window_n16384_d128_w1024", "prefill_q512_k16384_d128", "fp16_n8192_d128", "bnhd_n8192_d128",
         "d32_n8192", "d96_n8192", "d256_n8192", "bias_n4096_d128")


def run_suite(args):
    """Event-timed fa_fwd_ex / fa_bwd_ex on each general-shape workload."""
    import torch
    from exact_attention_122_amd import fa, inputs
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    for name in SUITE:
        w = inputs.WORKLOADS[name]
        B, H, N, d = w["B"], w["H"], w["N"], w["d"]
        nk = w.get("nk", N)
        window = w.get("window", (None, 0) if w["causal"] else (None, None))
        scale = inputs.default_scale(d)
        g = inputs.generate_workload(name)
        q, k, v, do = (g[x].to_torch(dev) for x in ("q", "k", "v", "do"))
        layout = w.get("layout", "bhnd")
        if layout == "bnhd":  # [B, N, H, d] memory seen as [B, H, N, d]
            q, k, v, do = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v, do))
            o = torch.empty(B, N, H, d, dtype=q.dtype, device=dev).transpose(1, 2)
            grads = [torch.empty(B, n, H, d, dtype=q.dtype, device=dev).transpose(1, 2) for n in (N, nk, nk)]
        else:
            o = torch.empty_like(q)
            grads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, fa.fa_bwd_ex_workspace_bytes(B, H, N, nk, d, fa._dtype_code(q))),
                         dtype=torch.uint8, device=dev)
        wl = -1 if window[0] is None else window[0]
        wr = -1 if window[1] is None else window[1]
        bias = None
        if "bias" in w:
            bias = torch.from_numpy(inputs.generate_bias(w["bias"], w["seed"] + 1)).to(dev)

        def fwd():
            fa.fa_fwd_ex(q, k, v, window=(wl, wr), scale=scale, out=o, lse=lse, bias=bias)

        def bwd():
            fa.fa_bwd_ex(q, k, v, o, do, lse, window=(wl, wr), scale=scale, dq=grads[0], dk=grads[1],
                         dv=grads[2], workspace=ws, bias=bias)

        res = {}
        pairs = visible_pairs(N, nk, window) * B * H
        for tag, fn, flops in (("fwd", fwd, 4.0 * d * pairs), ("bwd", bwd, 10.0 * d * pairs)):
            for _ in range(args.warmup):
                fn()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
            torch.cuda.synchronize()
            ev[0].record()
            for i in range(args.steps):
                fn()
                ev[i + 1].record()
            torch.cuda.synchronize()
            ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
            med = ms[len(ms) // 2]
            res[tag] = {"ms": round(med, 4), "tflops": round(flops / med / 1e9, 2),
                        "frac_peak": round(flops / med / 1e9 / PEAK_BF16_TFLOPS, 4)}
        extra = {}
        if bias is not None:
            # the bias is read once per (batch, head) in the forward, twice in the backward
            bias_bytes = B * H * N * nk * 4
            extra = {"bias_shape": list(w["bias"]), "bias_read_GBps_fwd": round(bias_bytes / res["fwd"]["ms"] / 1e6, 1)}
        print(json.dumps({"suite": name, "dtype": w["dtype"], "layout": layout,
                          "config": {"B": B, "H": H, "Nq": N, "Nk": nk, "d": d,
                                     "window": [wl, wr], "seed": w["seed"]}, **extra,
                          "visible_pairs": pairs, "flops_fwd": 4.0 * d * pairs, **res,
                          "peak": PEAK_BF16_TFLOPS}), flush=True)


def calibrate_copy(mib):
    """A plain elementwise copy kernel of known size: reads and writes mib MiB."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "elementwise copy (torch.neg) of float32", "launches": 3,
                      "bytes_read_per_launch": n * 4, "bytes_written_per_launch": n * 4}), flush=True)


def cpu_baseline(g, w, scale, causal, heads):
    """The fp64 oracle on a bounded sample: the first `heads` (b, h) heads,
    forward + backward. Returns the timing record and the oracle's outputs
    (O, LSE, dQ, dK, dV) for those heads, flattened to [heads, ...]."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    q, k, v, do = (g[x].to_f64().reshape((-1,) + g[x].shape[2:])[:heads] for x in ("q", "k", "v", "do"))
    t0 = time.perf_counter()
    o, lse = oracle.forward(q, k, v, scale, causal, workers=cores)
    dq, dk, dv = oracle.backward(q, k, v, do, scale, causal, workers=cores)
    dt = time.perf_counter() - t0
    flops = attention_flops(1, heads, w["N"], w["d"], causal) * 3.5
    rec = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "seconds": round(dt, 3),
           "sample": f"{heads} of {w['B'] * w['H']} heads, forward + backward, fp64 numpy "
                     f"(S materialised row-chunk by row-chunk), same input bytes"}
    return rec, {"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv}


def parity(gpu, ref, heads):
    """Max-abs and relative Frobenius error of each GPU output against the
    oracle's, over the first `heads` heads, with the bound each must meet."""
    import numpy as np
    bounds = {"O": 2e-2, "LSE": 1e-3, "dQ": 2e-2, "dK": 2e-2, "dV": 2e-2}
    out = {}
    for name, r in ref.items():
        t = gpu[name]
        x = t.detach().float().cpu().numpy().astype(np.float64)
        x = x.reshape((-1,) + x.shape[2:])[:heads]
        diff = x - r
        err = float(np.abs(diff).max())
        fro = float(np.linalg.norm(diff) / np.linalg.norm(r))
        out[name] = {"max_abs": float(f"{err:.4g}"), "rel_fro": float(f"{fro:.4g}"), "bound": bounds[name],
                     "ok": bool(err <= bounds[name] and (name == "LSE" or fro <= 2e-2))}
    out["heads"] = heads
    out["all_ok"] = all(v["ok"] for k, v in out.items() if isinstance(v, dict))
    return out


def percentiles(ms):
    """mean, median, p10 and p90 of per-launch times (ms)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90))}


def provenance():
    """The git commit when the repository's history is present (it is not
    copied everywhere the bench runs), and a SHA-256 of the library's sources
    and this file, which identifies the code either way."""
    import subprocess
    head = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        if r.returncode == 0:
            head = r.stdout.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_122_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    for path in (os.path.join(ROOT, "include", "fa.h"), os.path.abspath(__file__)):
        with open(path, "rb") as f:
            h.update(f.read())
    return {"git_head": head, "source_sha256": h.hexdigest()}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path: heads are independent and would shard with no exchange.", file=sys.stderr)
        sys.exit(2)
    if args.suite:
        run_suite(args)
        return

    import torch
    from exact_attention_122_amd import fa, inputs

    w = dict(inputs.WORKLOADS[args.workload])
    if args.causal is not None:
        w["causal"] = bool(args.causal)
    B, H, N, d, causal = w["B"], w["H"], w["N"], w["d"], w["causal"]
    if w["dtype"] != "bf16":
        raise SystemExit("bench.py times the bf16 path")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    scale = inputs.default_scale(d)
    g = inputs.generate(B, H, N, d, "bf16", w["seed"], with_grad_output=True)
    q, k, v, do = (g[x].to_torch(dev) for x in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
        if ev is not None:
            ev[1].record()
        if not args.fwd_only:
            fa.fa_bwd(q, k, v, o, do, lse, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv, workspace=ws)
            if ev is not None:
                ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record()
    for i in range(args.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()

    total_ms = t_begin.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    f_fwd = attention_flops(B, H, N, d, causal)
    f_bwd = 2.5 * f_fwd
    # algorithmic HBM bytes (bf16): forward reads Q, K, V and writes O, LSE;
    # backward reads Q, K, V, O, dO, LSE and writes dQ, dK, dV
    fwd_bytes = B * H * (4 * N * d * 2 + N * 4)
    bwd_bytes = B * H * (8 * N * d * 2 + N * 4)

    def summary(ms, flops, nbytes):
        # rates at the mean launch time; the median and the 10th / 90th
        # percentiles of the per-launch times show the spread
        pc = percentiles(ms)
        return {"ms": round(pc["mean"], 4), "ms_median": round(pc["median"], 4),
                "ms_p10": round(pc["p10"], 4), "ms_p90": round(pc["p90"], 4),
                "tflops": round(flops / pc["mean"] / 1e9, 2),
                "tflops_median": round(flops / pc["median"] / 1e9, 2),
                "frac_peak": round(flops / pc["mean"] / 1e9 / PEAK_BF16_TFLOPS, 4),
                "hbm_GBps": round(nbytes / pc["mean"] / 1e6, 1)}

    res = {"fwd": summary([e[0].elapsed_time(e[1]) for e in evs], f_fwd, fwd_bytes)}
    fwd_avg = res["fwd"]["ms"]
    step_flops = f_fwd
    if not args.fwd_only:
        res["bwd"] = summary([e[1].elapsed_time(e[2]) for e in evs], f_bwd, bwd_bytes)
        step_flops += f_bwd
    value = step_flops / ms_per_step / 1e9   # TFLOP/s

    # roofline of fa_fwd's kernel: algorithmic FLOPs per launch / its mean
    # event-timed launch duration
    ach = f_fwd / fwd_avg / 1e9
    kname = f"fwd_kernel<bf16,{d},{'upper' if causal else 'none'}>"
    roof = {"kernel": f"{kname} (fa_fwd)",
            "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(kname) if args.workload == TRAFFIC_WORKLOAD else None,
            "algorithmic_bytes": fwd_bytes}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"bf16 self-attention B={B} H={H} N={N} d={d} "
                               f"{'causal' if causal else 'non-causal'}, step = fa_fwd + fa_bwd"
                               + (" (fwd only)" if args.fwd_only else ""),
                   "B": B, "H": H, "N": N, "d": d, "causal": causal, "seed": w["seed"],
                   "scale": scale,
                   "inputs_sha256": {x: g[x].sha256 for x in ("q", "k", "v", "do")}},
        **res,
        "frac_peak_step": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roof,
        "device": torch.cuda.get_device_name(dev),
        "cu_count": torch.cuda.get_device_properties(dev).multi_processor_count,
        **provenance(),
    }
    if not args.no_cpu_baseline and not args.fwd_only:
        heads = min(args.cpu_heads, B * H)
        out["cpu_baseline"], ref = cpu_baseline(g, w, scale, causal, heads)
        # the outputs of the last timed step against the oracle's
        out["parity"] = parity({"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv}, ref, heads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
