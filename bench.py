"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --op softmax_rows      (the standalone row softmax instead)

A step is one call of attn_fwd (the whole fused forward, one kernel launch) on the
seeded synthetic inputs of a workload, already resident in device memory.  W
untimed steps, then exactly K timed steps between two device synchronisations.
Prints ONE JSON line:

* value / unit: attention TFLOP/s = 4*B*H*Nq*Nk*D (halved when causal) / time
* roofline: the same algorithmic flop count divided by the kernel's mean launch
  duration (HIP events around each launch, on the launch stream), against the
  bf16 dense matrix peak of MI355X (2.5 PFLOP/s); ``traffic`` is the measured
  device-memory traffic per launch from a committed rocprofv3 counter summary,
  reported only if it was taken on the current kernel source (else null)
* cpu_baseline: the fp64 CPU oracle timed on a bounded sample of the same
  workload on this host, in the same unit.

``--op softmax_rows`` times the row softmax (fp32, 8192 x 8192) instead: value in
GB/s of one read + one write per element, roofline against 8 TB/s of HBM, the
unfused four-pass baseline's time in ``config``.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def kernel_source_hash():
    """Hash of the bf16 kernel sources: a traffic record taken from other sources is stale."""
    from exact_attention_89_amd.traffic import _kernel_hash
    return _kernel_hash()


def measured_traffic(workload):
    """HBM bytes per launch from profiles/traffic_<workload>.json, if current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    fused = rec.get("fused", {})
    if fused.get("kernel_source_hash") != kernel_source_hash():
        return None
    return fused.get("bytes_per_launch")


def cpu_baseline(w, q, k, v, lens, budget_s):
    """Time the fp64 oracle on whole heads of the workload until ``budget_s`` passes."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    heads = 0
    t0 = time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            oracle.attention_oracle(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                    v[b:b + 1, h:h + 1], w.scale, causal=w.causal,
                                    kv_lens=None if lens is None else lens[b:b + 1])
            heads += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = w.metric_flops() / (w.B * w.H) * heads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} (batch, head) pairs of {w.name}, every query "
                      f"row, fp64 numpy oracle, {dt:.1f} s wall; flops counted as in the "
                      f"metric"}


SOFTMAX_ROWS, SOFTMAX_COLS, SOFTMAX_SEED = 8192, 8192, 6
PEAK_HBM_GBS = 8000.0


def softmax_traffic():
    """Fused row-softmax HBM bytes per launch at 8192 x 8192 from the committed profile."""
    path = os.path.join(ROOT, "profiles", "traffic_softmax_rows_fused_vs_unfused.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from exact_attention_89_amd.traffic import _softmax_hash
    if rec.get("kernel_source_hash") != _softmax_hash():
        return None
    for e in rec.get("entries", []):
        if e["rows"] == SOFTMAX_ROWS and e["cols"] == SOFTMAX_COLS:
            return e["fused"]["read_bytes"] + e["fused"]["write_bytes"]
    return None


def fp8_traffic():
    """FP8 fused forward HBM bytes per launch at the throughput shape, if current."""
    path = os.path.join(ROOT, "profiles", "traffic_fp8_causal_b1h32_n8192_d128.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from exact_attention_89_amd.traffic import _fp8_hash
    e = rec.get("fp8", {})
    return e.get("bytes_per_launch") if e.get("kernel_source_hash") == _fp8_hash() else None


def decode_traffic():
    """Split-key decode HBM bytes per call (both launches) from the committed profile."""
    path = os.path.join(ROOT, "profiles", "traffic_decode_b1h8_nq1_d128_nk_sweep.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from exact_attention_89_amd.traffic import _decode_hash
    if rec.get("kernel_source_hash") != _decode_hash():
        return None
    for e in rec.get("entries", []):
        if all(e[k] == DECODE[k] for k in ("B", "H", "Nq", "Nk", "D")):
            return e["read_bytes"] + e["write_bytes"]
    return None


def softmax_cpu_baseline(x, budget_s):
    """Time the fp64 row-softmax oracle on whole rows of the input until budget_s."""
    from threadpoolctl import threadpool_info

    import oracle
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    rows, chunk = 0, 64
    t0 = time.perf_counter()
    while rows < x.shape[0] and time.perf_counter() - t0 < budget_s:
        oracle.softmax_rows(x[rows:rows + chunk])
        rows += chunk
    dt = time.perf_counter() - t0
    return {"value": 2.0 * rows * x.shape[1] * 4 / dt / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows} of {x.shape[0]} rows of the {x.shape[0]}x{x.shape[1]} fp32 input, "
                      f"fp64 numpy oracle, {dt:.1f} s wall; bytes counted as in the metric"}


def bench_softmax(args):
    """Row softmax (fp32, 8192 x 8192): fused kernel, with the unfused four-pass one beside it."""
    import numpy as np
    import torch

    from exact_attention_89_amd import api
    api.load_library()
    rng = np.random.default_rng(SOFTMAX_SEED)
    x = (rng.standard_normal((SOFTMAX_ROWS, SOFTMAX_COLS), dtype=np.float32) * 3.0)
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    ws = torch.empty(api.load_library().softmax_rows_unfused_workspace_bytes(SOFTMAX_ROWS),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    algo = 2.0 * SOFTMAX_ROWS * SOFTMAX_COLS * 4

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for s, e in ev:
            s.record(stream)
            fn()
            e.record(stream)
        torch.cuda.synchronize()
        total = ev[0][0].elapsed_time(ev[-1][1]) / args.steps
        launch = float(np.mean([s.elapsed_time(e) for s, e in ev]))
        return total, launch

    fused_ms, fused_launch = timed(lambda: api.softmax_rows(xd, out=y))
    ref_rows = [0, SOFTMAX_ROWS // 2, SOFTMAX_ROWS - 1]
    got = y[ref_rows].cpu().numpy()
    unf_ms, _ = timed(lambda: api.softmax_rows_unfused(xd, out=y, workspace=ws))
    assert not np.isnan(got).any()
    log(f"[bench] softmax_rows {SOFTMAX_ROWS}x{SOFTMAX_COLS}: fused {fused_ms:.4f} ms, "
        f"unfused {unf_ms:.4f} ms")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = softmax_cpu_baseline(x, args.cpu_seconds)
    value = algo / (fused_ms * 1e-3) / 1e9
    achieved = algo / (fused_launch * 1e-3) / 1e9
    line = {
        "metric": "row softmax GB/s (fp32, 8192 rows x 8192 cols, one read + one write)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(fused_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"softmax_rows_{SOFTMAX_ROWS}x{SOFTMAX_COLS}_f32",
                   "rows": SOFTMAX_ROWS, "cols": SOFTMAX_COLS, "seed": SOFTMAX_SEED,
                   "unfused_ms_per_step": round(unf_ms, 5),
                   "unfused_gbs": round(algo / (unf_ms * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": softmax_traffic()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


DECODE = dict(B=1, H=8, Nq=1, Nk=65536, D=128, seed=7)


def bench_decode(args):
    """Split-key decode: one query per head against a 65536-key cache (bf16)."""
    import numpy as np
    import torch

    from exact_attention_89_amd import api
    from exact_attention_89_amd.workloads import round_to_bf16
    api.load_library()
    B, H, Nq, Nk, D = (DECODE[k] for k in ("B", "H", "Nq", "Nk", "D"))
    rng = np.random.default_rng(DECODE["seed"])
    q, k, v = (round_to_bf16(rng.standard_normal(s, dtype=np.float32))
               for s in ((B, H, Nq, D), (B, H, Nk, D), (B, H, Nk, D)))
    qd, kd, vd = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (q, k, v))
    scale = 1.0 / D ** 0.5
    ws = torch.empty(api.attn_splitkv_workspace_bytes(B, H, Nq, Nk, D, 0), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for s_, e in ev:
            s_.record(stream)
            fn()
            e.record(stream)
        torch.cuda.synchronize()
        return (ev[0][0].elapsed_time(ev[-1][1]) / args.steps,
                float(np.mean([s_.elapsed_time(e) for s_, e in ev])))

    split_ms, split_launch = timed(lambda: api.attn_fwd_splitkv(
        qd, kd, vd, scale=scale, workspace=ws, out=o, lse=lse))
    assert not torch.isnan(o).any().item()
    fused_ms, _ = timed(lambda: api.attn_fwd(qd, kd, vd, scale=scale, out=o, lse=lse))
    kv_bytes = 2.0 * B * H * Nk * D * 2
    log(f"[bench] decode: splitkv {split_ms:.4f} ms, fused {fused_ms:.4f} ms")
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        import oracle
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
        t0, heads = time.perf_counter(), 0
        for h in range(H):
            oracle.attention_oracle(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], scale)
            heads += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        cpu = {"value": kv_bytes / H * heads / dt / 1e9, "unit": "GB/s", "cores": int(threads),
               "kind": "oracle",
               "sample": f"{heads} of {H} heads, every key, fp64 numpy oracle, {dt:.1f} s wall; "
                         f"bytes counted as in the metric (K and V read once)"}
    achieved = kv_bytes / (split_launch * 1e-3) / 1e9
    line = {
        "metric": "split-KV decode GB/s of K+V (bf16, B=1 H=8 Nq=1 Nk=65536 D=128)",
        "value": round(kv_bytes / (split_ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(split_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_b1h8_nq1_nk65536_d128", **DECODE,
                   "num_splits": int(api.load_library().attn_splitkv_num_splits(B, H, Nq, Nk, 0)),
                   "fused_attn_fwd_ms_per_step": round(fused_ms, 5)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": decode_traffic()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


PEAK_FP8_TFLOPS = 5000.0


def bench_fp8(args):
    """The fused forward on E4M3 inputs at the throughput workload's shape."""
    import numpy as np
    import torch

    import exact_attention_89_amd.workloads as W
    from exact_attention_89_amd import api
    api.load_library()
    name = W.HEADLINE
    w = W.WORKLOADS[name]
    log(f"[bench] generating {name} as E4M3 codes")
    q8, k8, v8, ds, lens = W.generate_fp8(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q8, k8, v8))
    o = torch.empty(qd.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for s_, e in ev:
            s_.record(stream)
            fn()
            e.record(stream)
        torch.cuda.synchronize()
        launch = [s_.elapsed_time(e) for s_, e in ev]
        return ev[0][0].elapsed_time(ev[-1][1]) / args.steps, launch

    ms, launch = timed(lambda: api.attn_fwd_fp8(qd, kd, vd, *ds, scale=w.scale, causal=w.causal,
                                                out=o, lse=lse))
    assert not torch.isnan(o).any().item(), "NaN in the output"
    flops = w.metric_flops()
    value = flops / (ms * 1e-3) / 1e12
    achieved = flops / (float(np.mean(launch)) * 1e-3) / 1e12
    log(f"[bench] fp8 {name}: {ms:.4f} ms/step, launch median {np.median(launch):.4f} ms, p10 "
        f"{np.percentile(launch, 10):.4f}, p90 {np.percentile(launch, 90):.4f}")
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        import oracle
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
        t0, heads = time.perf_counter(), 0
        for h in range(w.H):
            oracle.attention_fp8_oracle(q8[:, h:h + 1], k8[:, h:h + 1], v8[:, h:h + 1], w.scale,
                                        *ds, causal=w.causal)
            heads += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        cpu = {"value": flops / w.H * heads / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
               "kind": "oracle",
               "sample": f"{heads} of {w.H} heads of the E4M3 workload, every query row, fp64 "
                         f"numpy oracle of the dequantised inputs, {dt:.1f} s wall; flops "
                         f"counted as in the metric"}
    line = {
        "metric": "fused attn fwd TFLOP/s, E4M3 inputs (B,H,N,D=1,32,8192,128 causal)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": "fp8_causal_b1h32_n8192_d128", "B": w.B, "H": w.H, "Nq": w.Nq,
                   "Nk": w.Nk, "D": w.D, "causal": w.causal, "seed": w.seed,
                   "pct_of_fp8_peak": round(100.0 * value / PEAK_FP8_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "traffic": fp8_traffic()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def versions(torch):
    """torch / HIP versions and the device name, recorded with every headline line."""
    return {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
            "device": torch.cuda.get_device_name(0)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="calls timed with a 512 MiB buffer written before each (0: skip)")
    ap.add_argument("--op", choices=["attention", "partial", "materialized", "softmax_rows",
                                     "decode", "fp8"],
                    default="attention",
                    help="attention: the fused attention forward (default); partial: QK^T + "
                         "softmax fused, P through device memory, then P V; materialized: the "
                         "three-launch baseline; softmax_rows: the standalone row softmax; "
                         "decode: split-key attention for one query against a long cache; "
                         "fp8: the fused forward on E4M3 inputs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the fused "
              "forward shards by (batch, head) with no communication, so a multi-GPU figure "
              "would be N independent copies of this one", file=sys.stderr)
        sys.exit(2)

    if args.op in ("softmax_rows", "decode", "fp8"):
        if not os.path.exists(os.path.join(ROOT, "exact_attention_89_amd", "libattn89.so")):
            from exact_attention_89_amd import build
            build.build()
        return {"softmax_rows": bench_softmax, "decode": bench_decode,
                "fp8": bench_fp8}[args.op](args)

    import numpy as np
    import torch

    from exact_attention_89_amd import api
    from exact_attention_89_amd.workloads import HEADLINE, WORKLOADS, generate

    if not os.path.exists(api.library_path()):
        from exact_attention_89_amd import build
        build.build()
    api.load_library()
    name = args.workload or HEADLINE
    w = WORKLOADS[name]
    if w.dtype != "bf16":
        raise SystemExit("bench.py times the bf16 path")
    log(f"[bench] generating {name}")
    q, k, v, lens = generate(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v))
    ld = None if lens is None else torch.from_numpy(lens).to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)

    ldk = (w.Nk + 63) // 64 * 64
    if args.op == "attention":
        def step():
            api.attn_fwd(qd, kd, vd, scale=w.scale, causal=w.causal, kv_lens=ld, out=o, lse=lse)
        extra_bytes = 0
    elif args.op == "partial":
        ws = torch.empty(api.attn_partial_workspace_bytes(w.B, w.H, w.Nq, w.Nk),
                         dtype=torch.uint8, device=dev)

        def step():
            api.attn_partial(qd, kd, vd, scale=w.scale, causal=w.causal, kv_lens=ld,
                             workspace=ws, out=o, lse=lse)
        extra_bytes = 2 * 2 * w.B * w.H * w.Nq * ldk            # P written once, read once
    else:
        ws = torch.empty(api.attn_materialized_workspace_bytes(w.B, w.H, w.Nq, w.Nk),
                         dtype=torch.uint8, device=dev)

        def step():
            api.attn_materialized(qd, kd, vd, scale=w.scale, causal=w.causal, kv_lens=ld,
                                  workspace=ws, out=o, lse=lse)
        # S fp32 written once and read twice, P bf16 written once and read once
        extra_bytes = (4 + 8 + 2 + 2) * w.B * w.H * w.Nq * ldk

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in ev]
    total_ms = ev[0][0].elapsed_time(ev[-1][1])
    ms_per_step = total_ms / args.steps
    flops = w.metric_flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    mean_launch_ms = float(np.mean(launch_ms))
    achieved = flops / (mean_launch_ms * 1e-3) / 1e12
    log(f"[bench] {name}: {ms_per_step:.4f} ms/step (events), wall {wall / args.steps * 1e3:.4f}"
        f" ms/step, launch median {np.median(launch_ms):.4f} ms, p10 "
        f"{np.percentile(launch_ms, 10):.4f}, p90 {np.percentile(launch_ms, 90):.4f}")
    assert not torch.isnan(o).any().item(), "NaN in the output"
    launch_stats = {"median": round(float(np.median(launch_ms)), 5),
                    "p10": round(float(np.percentile(launch_ms, 10)), 5),
                    "p90": round(float(np.percentile(launch_ms, 90)), 5)}
    cold = None
    if args.op == "attention" and args.cold_steps > 0:
        # cold variant: a 512 MiB buffer is written between calls, so K and V are not
        # left in the caches by the previous call; only the attention launch is timed
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.cold_steps)]
        for s_, e in cev:
            scratch.fill_(1)
            s_.record(stream)
            step()
            e.record(stream)
        torch.cuda.synchronize()
        cold_ms = [s_.elapsed_time(e) for s_, e in cev]
        cold = {"median_ms": round(float(np.median(cold_ms)), 5),
                "p10_ms": round(float(np.percentile(cold_ms, 10)), 5),
                "p90_ms": round(float(np.percentile(cold_ms, 90)), 5),
                "calls": args.cold_steps}
        del scratch
        log(f"[bench] cold (512 MiB written between calls): median {cold['median_ms']:.4f} ms")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu_baseline: fp64 oracle for ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(w, q, k, v, lens, args.cpu_seconds)

    if args.op != "attention":
        # multi-launch paths: bound by device memory; bytes = inputs + outputs + the
        # score-sized tensors the path moves, over the whole call
        io_bytes = 2 * (2 * w.B * w.H * w.Nq * w.D + 2 * w.B * w.H * w.Nk * w.D) + \
            4 * w.B * w.H * w.Nq
        algo_bytes = io_bytes + extra_bytes
        gbs = algo_bytes / (mean_launch_ms * 1e-3) / 1e9
        line = {
            "metric": f"attn fwd TFLOP/s, {args.op} path (B,H,N,D=1,32,8192,128 causal)",
            "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": name, "op": args.op, "B": w.B, "H": w.H, "Nq": w.Nq,
                       "Nk": w.Nk, "D": w.D, "causal": w.causal, "seed": w.seed,
                       "algorithmic_bytes_per_call": algo_bytes},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
            "cpu_baseline": cpu,
        }
        print(json.dumps(line), flush=True)
        return

    traffic = measured_traffic(name)
    line = {
        "metric": "fused attn fwd TFLOP/s + % bf16 MFMA peak (B,H,N,D=1,32,8192,128 causal)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "D": w.D,
                   "causal": w.causal, "seed": w.seed,
                   "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
                   "launch_ms": launch_stats, "cold": cold, "versions": versions(torch)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
