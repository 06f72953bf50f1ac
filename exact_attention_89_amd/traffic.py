"""Device-memory traffic of the fused kernels against their unfused baselines.

Two kinds of subcommands.  ``run`` launches one path on synthetic inputs over a
sweep of sizes, in a fixed order, and writes a manifest of the dispatches it made;
it is meant to run under ``rocprofv3 --pmc FETCH_SIZE`` (then, in its own run,
``WRITE_SIZE``), with ``--kernel-include-regex 'MulFunctor|attn89'``:

    rocprofv3 --pmc FETCH_SIZE --kernel-include-regex 'MulFunctor|attn89' -d OUT \\
        -o fetch --output-format csv -- python3 -m exact_attention_89_amd.traffic \\
        run --impl fused --N 1024 2048 ... --manifest OUT/manifest.json

Every run first launches a plain elementwise copy (torch.mul, the only MulFunctor
dispatches of the run) of a known size, so the counters are calibrated against
bytes that are known, in the same process on the same GPU: how many bytes one
FETCH_SIZE unit stands for has differed between runs.  ``summarize`` and
``summarize-softmax`` join the counter CSVs with the manifests and write a JSON
record and a Markdown table.

The claims being measured:
* fused attention (page "Attention softmax fusion", sections "What fused has to
  mean" and "Things that break"; page "Kernel Fusion and the Memory Wall", section
  "FlashAttention: avoid the full score matrix"): the materialised pipeline moves
  Theta(N^2) bytes per head through device memory, the fused kernel's traffic stays
  O(N D) per query block and shows no score-sized term; a single short length would
  hide the difference, so lengths are swept;
* row softmax (page "Kernel Fusion and the Memory Wall", section "Softmax needs a
  global row statistic"): four reads and two writes per row unfused, one read and
  one write fused while the row fits on chip;
* split-key decode: K and V are read once whatever the number of key ranges; the
  partial results the ranges hand to the merge are small beside them.
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
KERNEL_REGEX = "MulFunctor|attn89"


def _hash(files):
    h = hashlib.sha256()
    for fn in files:
        with open(os.path.join(HERE, "csrc", fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _kernel_hash():
    """Sources of the bf16 fused attention kernels."""
    return _hash(("attn_fwd_bf16_pp.hip", "attn_fwd_bf16_4w.hip", "attn_bf16_tiles.hpp",
                  "common.hpp", "mfma_schedule.hpp"))


def _headline_hash():
    """Sources of the kernel the throughput workload runs (the 8-wave ping-pong kernel)."""
    return _hash(("attn_fwd_bf16_pp.hip", "attn_bf16_tiles.hpp", "common.hpp"))


def _decode_hash():
    """Sources of the split-key decode path (the 4-wave kernel plus the merge)."""
    return _hash(("attn_fwd_bf16_4w.hip", "attn_bf16_tiles.hpp", "common.hpp",
                  "attn_splitkv.hip", "mfma_schedule.hpp"))


def _fp8_hash():
    """Sources of the FP8 fused forward kernels."""
    return _hash(("attn_fwd_fp8.hip", "attn_fwd_fp8_pp.hip", "attn_fp8_tiles.hpp",
                  "attn_bf16_tiles.hpp", "common.hpp", "mfma_schedule.hpp"))


def _softmax_hash():
    """Sources of the row-softmax kernels."""
    return _hash(("softmax_rows.hip", "common.hpp"))


def _calibrate(torch, dev, mib, calls):
    n = mib * (1 << 20) // 4
    x = torch.empty(n, dtype=torch.float32, device=dev).normal_()
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    print(f"[traffic] calibration copy {mib} MiB x {calls}", flush=True)
    for _ in range(calls):
        torch.mul(x, 2.0, out=y)
    torch.cuda.synchronize()
    del x, y
    torch.cuda.empty_cache()
    return {"bytes_read": n * 4, "bytes_written": n * 4, "dispatches": calls}


def cmd_run(a):
    import torch

    from exact_attention_89_amd import api
    api.load_library()
    dev = torch.device("cuda:0")
    torch.manual_seed(0)
    manifest = {"impl": a.label or a.impl, "calls": a.calls, "entries": [],
                "calibration": _calibrate(torch, dev, a.copy_mib, a.calls)}
    if a.impl in ("softmax_fused", "softmax_unfused"):
        fn = api.softmax_rows if a.impl == "softmax_fused" else api.softmax_rows_unfused
        for cols in a.cols:
            rows = max(1, a.softmax_elems // cols)
            x = torch.empty(rows, cols, device=dev).normal_(0.0, 3.0)
            y = torch.empty_like(x)
            torch.cuda.synchronize()
            print(f"[traffic] {a.impl} rows={rows} cols={cols}", flush=True)
            for _ in range(a.calls):
                fn(x, out=y)
            torch.cuda.synchronize()
            manifest["entries"].append({
                "rows": rows, "cols": cols,
                "dispatches_per_call": 1 if a.impl == "softmax_fused" else 4,
                "algorithmic_bytes": 2 * rows * cols * 4,
            })
            del x, y
            torch.cuda.empty_cache()
        manifest["kernel_source_hash"] = _softmax_hash()
    elif a.impl == "decode":
        for Nk in a.Nk:
            q = torch.randn((a.B, a.H, a.Nq, a.D), device=dev, dtype=torch.bfloat16)
            k = torch.randn((a.B, a.H, Nk, a.D), device=dev, dtype=torch.bfloat16)
            v = torch.randn_like(k)
            o = torch.empty_like(q)
            lse = torch.empty((a.B, a.H, a.Nq), device=dev, dtype=torch.float32)
            ws = torch.empty(api.attn_splitkv_workspace_bytes(a.B, a.H, a.Nq, Nk, a.D, 0),
                             dtype=torch.uint8, device=dev)
            torch.cuda.synchronize()
            print(f"[traffic] decode Nk={Nk}", flush=True)
            for _ in range(a.calls):
                api.attn_fwd_splitkv(q, k, v, workspace=ws, out=o, lse=lse)
            torch.cuda.synchronize()
            manifest["entries"].append({
                "Nk": Nk, "B": a.B, "H": a.H, "Nq": a.Nq, "D": a.D,
                "num_splits": int(api.load_library().attn_splitkv_num_splits(
                    a.B, a.H, a.Nq, Nk, 0)),
                "dispatches_per_call": 2,
                "algorithmic_bytes": (2 * a.B * a.H * Nk * a.D * 2
                                      + 2 * a.B * a.H * a.Nq * a.D * 2 + 4 * a.B * a.H * a.Nq),
            })
            del q, k, v, o, lse, ws
            torch.cuda.empty_cache()
        manifest["kernel_source_hash"] = _decode_hash()
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
                if a.impl == "fp8":
                    q, k, v = (torch.randn(shape, device=dev).clamp_(-448, 448)
                               .to(torch.float8_e4m3fn) for _ in range(3))
                    o = torch.empty(shape, device=dev, dtype=torch.bfloat16)
                if a.impl == "materialized":
                    ws = torch.empty(api.attn_materialized_workspace_bytes(a.B, a.H, N, N),
                                     dtype=torch.uint8, device=dev)
                elif a.impl == "partial":
                    ws = torch.empty(api.attn_partial_workspace_bytes(a.B, a.H, N, N),
                                     dtype=torch.uint8, device=dev)
                torch.cuda.synchronize()
                print(f"[traffic] {a.impl} N={N} causal={causal}", flush=True)
                for _ in range(a.calls):
                    if a.impl == "fused":
                        api.attn_fwd(q, k, v, causal=bool(causal), out=o, lse=lse)
                    elif a.impl == "fp8":
                        api.attn_fwd_fp8(q, k, v, 1.0, 1.0, 1.0, causal=bool(causal), out=o,
                                         lse=lse)
                    elif a.impl == "partial":
                        api.attn_partial(q, k, v, causal=bool(causal), workspace=ws,
                                         out=o, lse=lse)
                    else:
                        api.attn_materialized(q, k, v, causal=bool(causal), workspace=ws,
                                              out=o, lse=lse)
                torch.cuda.synchronize()
                esize = 1 if a.impl == "fp8" else 2     # bytes per element of Q, K, V
                manifest["entries"].append({
                    "N": N, "causal": causal, "B": a.B, "H": a.H, "D": a.D,
                    "dispatches_per_call": {"fused": 1, "fp8": 1, "partial": 2}.get(a.impl, 3),
                    "algorithmic_bytes": (a.B * a.H * N * a.D * (3 * esize + 2)
                                          + a.B * a.H * N * 4),
                    "one_score_matrix_16bit_all_heads": a.B * a.H * N * N * 2,
                })
                del q, k, v, o, lse, ws
                torch.cuda.empty_cache()
        manifest["kernel_source_hash"] = (_fp8_hash() if a.impl == "fp8" else
                                          _headline_hash() if a.label == "headline" else
                                          _kernel_hash())
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


def _load_run(dirpath, impl):
    """Manifest, calibration factors and per-call calibrated bytes of one run."""
    man = json.load(open(os.path.join(dirpath, impl, "manifest.json")))
    fetch = _read_counters(os.path.join(dirpath, impl, "fetch", "**", "*counter_collection*.csv"))
    write = _read_counters(os.path.join(dirpath, impl, "write", "**", "*counter_collection*.csv"))
    cal = man["calibration"]
    nc = cal["dispatches"]
    if not all("MulFunctor" in n for n, _ in fetch[:nc] + write[:nc]):
        raise SystemExit(f"{impl}: the first {nc} dispatches are not the calibration copy")
    ff = cal["bytes_read"] * nc / sum(v for _, v in fetch[:nc])
    wf = cal["bytes_written"] * nc / sum(v for _, v in write[:nc])
    fetch, write = fetch[nc:], write[nc:]
    entries, pos = [], 0
    for e in man["entries"]:
        n = e["dispatches_per_call"] * man["calls"]
        fsl, wsl = fetch[pos:pos + n], write[pos:pos + n]
        pos += n
        kern = {}
        for (nm, fv), (_, wv) in zip(fsl, wsl):
            kk = kern.setdefault(nm, [0.0, 0.0])
            kk[0] += fv * ff / man["calls"]
            kk[1] += wv * wf / man["calls"]
        entries.append(dict(e, read_bytes=sum(v for _, v in fsl) * ff / man["calls"],
                            write_bytes=sum(v for _, v in wsl) * wf / man["calls"],
                            per_kernel=kern))
    return man, {"fetch_factor": ff, "write_factor": wf}, entries


def cmd_summarize(a):
    """Fused attention against the materialised baseline, plus the headline record."""
    res = {"commands": a.command or []}
    for impl in ("fused", "partial", "materialized", "headline", "fp8"):
        if os.path.exists(os.path.join(a.dir, impl, "manifest.json")):
            man, cal, entries = _load_run(a.dir, impl)
            res[impl] = {"entries": entries, "calibration": cal,
                         "kernel_source_hash": man.get("kernel_source_hash")}
    if a.headline_json and "headline" in res:
        e = res["headline"]["entries"][0]
        rec = {"workload": a.headline_name,
               "fused": {"bytes_per_launch": e["read_bytes"] + e["write_bytes"],
                         "read_bytes": e["read_bytes"], "write_bytes": e["write_bytes"],
                         "algorithmic_bytes": e["algorithmic_bytes"],
                         "kernel_source_hash": res["headline"]["kernel_source_hash"]},
               "calibration": res["headline"]["calibration"], "commands": a.command or []}
        with open(a.headline_json, "w") as f:
            json.dump(rec, f, indent=1)
        print(f"headline: read {e['read_bytes'] / 2**20:.1f} MiB, write "
              f"{e['write_bytes'] / 2**20:.1f} MiB per launch (algorithmic "
              f"{e['algorithmic_bytes'] / 2**20:.1f} MiB)")
    if a.fp8_json and "fp8" in res:
        e = res["fp8"]["entries"][0]
        rec = {"workload": "fp8_causal_b1h32_n8192_d128",
               "fp8": {"bytes_per_launch": e["read_bytes"] + e["write_bytes"],
                       "read_bytes": e["read_bytes"], "write_bytes": e["write_bytes"],
                       "algorithmic_bytes": e["algorithmic_bytes"],
                       "kernel_source_hash": res["fp8"]["kernel_source_hash"]},
               "calibration": res["fp8"]["calibration"], "commands": a.command or []}
        with open(a.fp8_json, "w") as f:
            json.dump(rec, f, indent=1)
        print(f"fp8: read {e['read_bytes'] / 2**20:.1f} MiB, write "
              f"{e['write_bytes'] / 2**20:.1f} MiB per launch (algorithmic "
              f"{e['algorithmic_bytes'] / 2**20:.1f} MiB)")
    with open(a.out_json, "w") as f:
        json.dump(res, f, indent=1)
    lines = ["# Device-memory traffic: fused kernel vs materialised 3-launch baseline", ""]
    lines += [f"    {c}" for c in a.command or []]
    lines.append("")
    for impl in ("fused", "partial", "materialized", "headline"):
        if impl in res:
            c = res[impl]["calibration"]
            lines.append(f"* calibration of the {impl} run (1 GiB copy in the same process): "
                         f"FETCH_SIZE x {c['fetch_factor']:.3f}, WRITE_SIZE x "
                         f"{c['write_factor']:.3f} = true bytes")
    lines += ["", "Figures below are calibrated (MiB per call).", "",
              "| N | causal | algorithmic | one score matrix (16-bit, all heads) | fused read | "
              "fused write | partial read | partial write | materialised read | materialised "
              "write | partial / fused | materialised / fused | materialised / partial |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    runs = {impl: {(e["N"], e["causal"]): e for e in res.get(impl, {}).get("entries", [])}
            for impl in ("fused", "partial", "materialized")}
    mib = float(1 << 20)
    nan = float("nan")

    def rw(e):
        return (e["read_bytes"] / mib, e["write_bytes"] / mib) if e else (nan, nan)

    keys = sorted(set().union(*[set(r) for r in runs.values()]))
    for key in keys:
        f, pa, m = (runs[i].get(key) for i in ("fused", "partial", "materialized"))
        (fr, fw), (pr, pw), (mr, mw) = rw(f), rw(pa), rw(m)
        base = f or pa or m
        lines.append(f"| {key[0]} | {key[1]} | {base['algorithmic_bytes'] / mib:.1f} | "
                     f"{base['one_score_matrix_16bit_all_heads'] / mib:.1f} | {fr:.1f} | "
                     f"{fw:.1f} | {pr:.1f} | {pw:.1f} | {mr:.1f} | {mw:.1f} | "
                     f"{(pr + pw) / (fr + fw):.1f} | {(mr + mw) / (fr + fw):.1f} | "
                     f"{(mr + mw) / (pr + pw):.2f} |")
    with open(a.out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_summarize_softmax(a):
    """Fused row softmax against the unfused four-pass baseline."""
    fman, fcal, fused = _load_run(a.dir, "softmax_fused")
    _, ucal, unf = _load_run(a.dir, "softmax_unfused")
    rec = {"calibration": {"fused_run": fcal, "unfused_run": ucal},
           "kernel_source_hash": fman.get("kernel_source_hash"), "commands": a.command or [],
           "entries": []}
    lines = ["# Device-memory traffic: fused row softmax vs the unfused four-pass baseline", ""]
    lines += [f"    {c}" for c in a.command or []]
    lines += ["", f"Calibration (1 GiB copy in the same process): fused run FETCH_SIZE x "
              f"{fcal['fetch_factor']:.3f}, WRITE_SIZE x {fcal['write_factor']:.3f}; unfused run "
              f"FETCH_SIZE x {ucal['fetch_factor']:.3f}, WRITE_SIZE x {ucal['write_factor']:.3f}.  "
              "fp32, rows x cols = 64 Mi elements (256 MiB) per case.", "",
              "| rows | cols | algorithmic MiB (1 read + 1 write) | fused read MiB | fused write MiB "
              "| unfused read MiB | unfused write MiB | unfused / fused |",
              "|---|---|---|---|---|---|---|---|"]
    mib = float(1 << 20)
    for f, u in zip(fused, unf):
        rec["entries"].append({"rows": f["rows"], "cols": f["cols"],
                               "algorithmic_bytes": f["algorithmic_bytes"],
                               "fused": {"read_bytes": f["read_bytes"],
                                         "write_bytes": f["write_bytes"]},
                               "unfused": {"read_bytes": u["read_bytes"],
                                           "write_bytes": u["write_bytes"]}})
        ratio = (u["read_bytes"] + u["write_bytes"]) / (f["read_bytes"] + f["write_bytes"])
        lines.append(f"| {f['rows']} | {f['cols']} | {f['algorithmic_bytes'] / mib:.1f} | "
                     f"{f['read_bytes'] / mib:.1f} | {f['write_bytes'] / mib:.1f} | "
                     f"{u['read_bytes'] / mib:.1f} | {u['write_bytes'] / mib:.1f} | "
                     f"{ratio:.2f} |")
    with open(a.out_json, "w") as fh:
        json.dump(rec, fh, indent=1)
    with open(a.out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_summarize_decode(a):
    """Split-key decode: bytes per call against K + V read once."""
    man, cal, entries = _load_run(a.dir, "decode")
    rec = {"calibration": cal, "kernel_source_hash": man.get("kernel_source_hash"),
           "commands": a.command or [], "entries": entries}
    mib = float(1 << 20)
    lines = ["# Device-memory traffic: split-key decode (one query per head)", ""]
    lines += [f"    {c}" for c in a.command or []]
    lines += ["", f"* calibration (1 GiB copy in the same process): FETCH_SIZE x "
              f"{cal['fetch_factor']:.3f}, WRITE_SIZE x {cal['write_factor']:.3f} = true bytes",
              "", "Calibrated MiB per call (both launches: the split kernel and the merge).", "",
              "| B | H | Nq | Nk | D | splits | algorithmic | read | write | split kernel read "
              "| split kernel write | merge read | merge write | (read + write) / algorithmic |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for e in entries:
        pk = e["per_kernel"]
        sk = next((v for n, v in pk.items() if "4w" in n), [float("nan")] * 2)
        mk = next((v for n, v in pk.items() if "merge" in n), [float("nan")] * 2)
        lines.append(f"| {e['B']} | {e['H']} | {e['Nq']} | {e['Nk']} | {e['D']} | "
                     f"{e['num_splits']} | {e['algorithmic_bytes'] / mib:.2f} | "
                     f"{e['read_bytes'] / mib:.2f} | {e['write_bytes'] / mib:.2f} | "
                     f"{sk[0] / mib:.2f} | {sk[1] / mib:.2f} | {mk[0] / mib:.2f} | "
                     f"{mk[1] / mib:.2f} | "
                     f"{(e['read_bytes'] + e['write_bytes']) / e['algorithmic_bytes']:.3f} |")
    with open(a.out_json, "w") as fh:
        json.dump(rec, fh, indent=1)
    with open(a.out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--impl", choices=["fused", "partial", "materialized", "softmax_fused",
                                      "softmax_unfused", "decode", "fp8"], required=True)
    r.add_argument("--label", default=None, help="manifest label (e.g. headline)")
    r.add_argument("--N", type=int, nargs="+", default=[1024, 2048, 4096, 8192, 16384, 32768])
    r.add_argument("--causal", type=int, nargs="+", default=[1, 0])
    r.add_argument("--B", type=int, default=1)
    r.add_argument("--H", type=int, default=8)
    r.add_argument("--D", type=int, default=128)
    r.add_argument("--Nq", type=int, default=1, help="queries per head of the decode sweep")
    r.add_argument("--Nk", type=int, nargs="+", default=[8192, 16384, 32768, 65536, 131072],
                   help="cache lengths of the decode sweep")
    r.add_argument("--calls", type=int, default=2)
    r.add_argument("--copy-mib", type=int, default=1024)
    r.add_argument("--cols", type=int, nargs="+", default=[1024, 4096, 8192, 16384, 65536],
                   help="row lengths of the softmax sweep")
    r.add_argument("--softmax-elems", type=int, default=64 << 20,
                   help="rows * cols of every softmax case (256 MiB of fp32)")
    r.add_argument("--manifest", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--dir", required=True)
    s.add_argument("--out-json", required=True)
    s.add_argument("--out-md", required=True)
    s.add_argument("--command", action="append")
    s.add_argument("--headline-json", default=None)
    s.add_argument("--headline-name", default="bf16_causal_b1h32_n8192_d128")
    s.add_argument("--fp8-json", default=None)
    ss = sub.add_parser("summarize-softmax")
    ss.add_argument("--dir", required=True)
    ss.add_argument("--out-json", required=True)
    ss.add_argument("--out-md", required=True)
    ss.add_argument("--command", action="append")
    sd = sub.add_parser("summarize-decode")
    sd.add_argument("--dir", required=True)
    sd.add_argument("--out-json", required=True)
    sd.add_argument("--out-md", required=True)
    sd.add_argument("--command", action="append")
    a = ap.parse_args()
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    {"run": cmd_run, "summarize": cmd_summarize,
     "summarize-softmax": cmd_summarize_softmax,
     "summarize-decode": cmd_summarize_decode}[a.cmd](a)


if __name__ == "__main__":
    main()
