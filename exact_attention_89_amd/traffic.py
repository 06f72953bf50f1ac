"""Device-memory traffic of the fused kernel against the materialised baseline.

Two subcommands.  ``run`` launches one path on synthetic inputs for several
sequence lengths, in a fixed order, and writes a manifest of the dispatches it
made; it is meant to run under ``rocprofv3 --pmc FETCH_SIZE`` (then, in its own
run, ``WRITE_SIZE``):

    rocprofv3 --pmc FETCH_SIZE --kernel-include-regex attn89 -d OUT -o fetch \
        --output-format csv -- python3 -m exact_attention_89_amd.traffic run \
        --impl fused --N 1024 2048 ... --manifest OUT/manifest.json

``--impl copy`` launches a plain elementwise kernel of known size (read S bytes,
write S bytes) to calibrate what the two counters report.  ``summarize`` joins
the counter CSVs with the manifests and writes a JSON record and a Markdown table.

The claim being measured (page "Attention softmax fusion", sections "What fused
has to mean" and "Things that break"; page "Kernel Fusion and the Memory Wall",
section "FlashAttention: avoid the full score matrix"): the materialised
pipeline moves Θ(N²) bytes per head through device memory, the fused kernel's
traffic stays O(N·D) per query block and shows no score-sized term; a single
short length would hide the difference, so lengths are swept.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _kernel_hash():
    h = hashlib.sha256()
    for fn in ("attn_fwd_bf16_pp.hip", "attn_fwd_bf16_4w.hip", "attn_bf16_tiles.hpp",
               "common.hpp"):
        with open(os.path.join(HERE, "csrc", fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def cmd_run(a):
    import torch

    from exact_attention_89_amd import api
    api.load_library()
    dev = torch.device("cuda:0")
    torch.manual_seed(0)
    manifest = {"impl": a.label or a.impl, "calls": a.calls, "entries": []}
    if a.impl == "copy":
        n = a.copy_mib * (1 << 20) // 4
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(a.calls):
            torch.mul(x, 2.0, out=y)
        torch.cuda.synchronize()
        manifest["entries"].append({"bytes_read": n * 4, "bytes_written": n * 4,
                                    "dispatches_per_call": 1})
    else:
        for N in a.N:
            for causal in a.causal:
                shape = (a.B, a.H, N, a.D)
                q = torch.randn(shape, device=dev, dtype=torch.bfloat16)
                k = torch.randn(shape, device=dev, dtype=torch.bfloat16)
                v = torch.randn(shape, device=dev, dtype=torch.bfloat16)
                o = torch.empty_like(q)
                lse = torch.empty((a.B, a.H, N), device=dev, dtype=torch.float32)
                ws = None
                if a.impl == "materialized":
                    ws = torch.empty(api.attn_materialized_workspace_bytes(a.B, a.H, N, N),
                                     dtype=torch.uint8, device=dev)
                torch.cuda.synchronize()
                print(f"[traffic] {a.impl} N={N} causal={causal}", flush=True)
                for _ in range(a.calls):
                    if a.impl == "fused":
                        api.attn_fwd(q, k, v, causal=bool(causal), out=o, lse=lse)
                    else:
                        api.attn_materialized(q, k, v, causal=bool(causal), workspace=ws,
                                              out=o, lse=lse)
                torch.cuda.synchronize()
                elt = 2
                manifest["entries"].append({
                    "N": N, "causal": causal, "B": a.B, "H": a.H, "D": a.D,
                    "dispatches_per_call": 1 if a.impl == "fused" else 3,
                    "algorithmic_bytes": a.B * a.H * N * a.D * elt * 4 + a.B * a.H * N * 4,
                    "one_score_matrix_16bit_all_heads": a.B * a.H * N * N * 2,
                })
                del q, k, v, o, lse, ws
                torch.cuda.empty_cache()
    manifest["kernel_source_hash"] = _kernel_hash()
    with open(a.manifest, "w") as f:
        json.dump(manifest, f, indent=1)


def _read_counters(path_glob):
    """Per-dispatch counter values, in dispatch order: list of (kernel, value_bytes)."""
    rows = []
    for path in sorted(glob.glob(path_glob, recursive=True)):
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append(r)
    out = {}
    for r in rows:
        did = int(r.get("Dispatch_Id") or r.get("Correlation_Id") or len(out))
        name = r.get("Kernel_Name", "?")
        val = float(r.get("Counter_Value", "nan"))
        key = (did, name)
        out[key] = out.get(key, 0.0) + val
    return [(name, val * 1024.0) for (did, name), val in sorted(out.items())]  # KiB -> B


def cmd_summarize(a):
    res = {}
    for impl in ("copy", "fused", "materialized", "headline"):
        mpath = os.path.join(a.dir, impl, "manifest.json")
        if not os.path.exists(mpath):
            continue
        man = json.load(open(mpath))
        fetch = _read_counters(os.path.join(a.dir, impl, "fetch", "**", "*counter_collection*.csv"))
        write = _read_counters(os.path.join(a.dir, impl, "write", "**", "*counter_collection*.csv"))
        if impl == "copy":
            fetch, write = fetch[-man["calls"]:], write[-man["calls"]:]
        entries = []
        pos = 0
        for e in man["entries"]:
            n = e["dispatches_per_call"] * man["calls"]
            fsl, wsl = fetch[pos:pos + n], write[pos:pos + n]
            pos += n
            per_call_f = sum(v for _, v in fsl) / man["calls"]
            per_call_w = sum(v for _, v in wsl) / man["calls"]
            kern = {}
            for (nm, fv), (_, wv) in zip(fsl, wsl):
                kk = kern.setdefault(nm, [0.0, 0.0])
                kk[0] += fv / man["calls"]
                kk[1] += wv / man["calls"]
            e = dict(e, fetch_bytes=per_call_f, write_bytes=per_call_w, per_kernel=kern)
            entries.append(e)
        res[impl] = {"entries": entries, "kernel_source_hash": man.get("kernel_source_hash")}
    cal = None
    if "copy" in res:
        c = res["copy"]["entries"][0]
        cal = {"fetch_factor": c["bytes_read"] / c["fetch_bytes"],
               "write_factor": c["bytes_written"] / c["write_bytes"]}
    res["calibration"] = cal
    res["commands"] = a.command or []
    if a.headline_json and "headline" in res and cal:
        e = res["headline"]["entries"][0]
        rd = e["fetch_bytes"] * cal["fetch_factor"]
        wr = e["write_bytes"] * cal["write_factor"]
        rec = {"workload": a.headline_name,
               "fused": {"bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
                         "algorithmic_bytes": e["algorithmic_bytes"],
                         "kernel_source_hash": res["headline"]["kernel_source_hash"]},
               "calibration": cal, "commands": a.command or []}
        with open(a.headline_json, "w") as f:
            json.dump(rec, f, indent=1)
        print(f"headline: read {rd / 2**20:.1f} MiB, write {wr / 2**20:.1f} MiB per launch "
              f"(algorithmic {e['algorithmic_bytes'] / 2**20:.1f} MiB)")
    with open(a.out_json, "w") as f:
        json.dump(res, f, indent=1)
    # Markdown table
    lines = ["# Device-memory traffic: fused kernel vs materialised 3-launch baseline", ""]
    for c in a.command or []:
        lines.append(f"    {c}")
    lines.append("")
    if cal:
        lines.append(f"Calibration (plain elementwise kernel, known bytes): FETCH_SIZE x "
                     f"{cal['fetch_factor']:.3f}, WRITE_SIZE x {cal['write_factor']:.3f} "
                     "= true bytes.  Figures below are calibrated.")
        lines.append("")
    lines.append("| N | causal | fused read MiB | fused write MiB | algorithmic MiB | "
                 "materialised read MiB | materialised write MiB | one score matrix (16-bit, "
                 "all heads) MiB | materialised / fused |")
    lines.append("|---|---|---|---|---|---|---|---|---|")
    ff = cal["fetch_factor"] if cal else 1.0
    wf = cal["write_factor"] if cal else 1.0
    fused = {(e["N"], e["causal"]): e for e in res.get("fused", {}).get("entries", [])}
    mat = {(e["N"], e["causal"]): e for e in res.get("materialized", {}).get("entries", [])}
    for key in sorted(set(fused) | set(mat)):
        f = fused.get(key)
        m = mat.get(key)
        mib = 1 << 20
        fr = f["fetch_bytes"] * ff / mib if f else float("nan")
        fw = f["write_bytes"] * wf / mib if f else float("nan")
        mr = m["fetch_bytes"] * ff / mib if m else float("nan")
        mw = m["write_bytes"] * wf / mib if m else float("nan")
        alg = (f or m)["algorithmic_bytes"] / mib
        sm = (f or m)["one_score_matrix_16bit_all_heads"] / mib
        ratio = (mr + mw) / (fr + fw) if f and m else float("nan")
        lines.append(f"| {key[0]} | {key[1]} | {fr:.1f} | {fw:.1f} | {alg:.1f} | {mr:.1f} | "
                     f"{mw:.1f} | {sm:.1f} | {ratio:.1f} |")
    with open(a.out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--impl", choices=["fused", "materialized", "copy"], required=True)
    r.add_argument("--label", default=None, help="manifest label (e.g. headline)")
    r.add_argument("--N", type=int, nargs="+", default=[1024, 2048, 4096, 8192, 16384, 32768])
    r.add_argument("--causal", type=int, nargs="+", default=[1, 0])
    r.add_argument("--B", type=int, default=1)
    r.add_argument("--H", type=int, default=8)
    r.add_argument("--D", type=int, default=128)
    r.add_argument("--calls", type=int, default=2)
    r.add_argument("--copy-mib", type=int, default=1024)
    r.add_argument("--manifest", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--dir", required=True)
    s.add_argument("--out-json", required=True)
    s.add_argument("--out-md", required=True)
    s.add_argument("--command", action="append")
    s.add_argument("--headline-json", default=None)
    s.add_argument("--headline-name", default="bf16_causal_b1h32_n8192_d128")
    a = ap.parse_args()
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    {"run": cmd_run, "summarize": cmd_summarize}[a.cmd](a)


if __name__ == "__main__":
    main()
