"""Summaries of rocprofv3 output for the benchmark's workloads (CPU only).

    python -m shared_prefix_scoring_amd.rocprof_summary trace DIR
        Per-kernel table of a --kernel-trace run of ``bench.py``: dispatches,
        average duration, the union of the dispatch intervals, and the
        average over dispatches that ran with no other dispatch beside them;
        then, per phase of the benchmark, the average duration of each
        kernel.  Phases are delimited by the benchmark's marker launches (a
        16-byte ``k_copy`` before each phase).

    python -m shared_prefix_scoring_amd.rocprof_summary counters DIR
        Per-kernel averages of every counter of a --pmc run.

    python -m shared_prefix_scoring_amd.rocprof_summary traffic DIR --kernel NAME --which W
        HBM traffic per dispatch of one kernel from four --pmc passes under
        DIR (fetch/ and write/: FETCH_SIZE and WRITE_SIZE of the workload;
        cal_fetch/ and cal_write/: the same counters of a 1 GiB copy), each
        counter scaled by what it reads for the copy's known bytes, against
        the algorithmic bytes per dispatch (see alg-bytes); JSON on stdout.

    python -m shared_prefix_scoring_amd.rocprof_summary alg-bytes --which W
        Algorithmic HBM bytes per dispatch when every call scores the
        headline pool's first 64 requests (bench.py --same-batch), for
        W = attn_branch (a branch-only attention launch: every request's
        prefix K and V once per KV head, each candidate's query, own K/V and
        output), gemm_resid (the residual-epilogue GEMM, the average of an O
        and a down projection over all rows: weights, activations in, the
        fp32 residual read and written), gemm_gateup or gemm_qkv (weights,
        activations in, bf16 output).  The JSON also records a hash of the
        kernel's code (comments aside), so that a benchmark on changed kernels reports no
        traffic.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sys


def short_name(n: str) -> str:
    n = n.replace("duolm::", "").replace("(anonymous namespace)::", "").replace("void ", "")
    return n[:n.index("(")] if "(" in n else n


def _csv_rows(d: str, suffix: str):
    rows = []
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith(suffix):
                with open(os.path.join(root, fn)) as f:
                    rows += list(csv.DictReader(f))
    return rows


def _union_us(iv):
    u, lo, hi = 0, None, None
    for a, b in sorted(iv):
        if lo is None or a > hi:
            if lo is not None:
                u += hi - lo
            lo, hi = a, b
        else:
            hi = max(hi, b)
    if lo is not None:
        u += hi - lo
    return u / 1e3


def trace(d: str) -> None:
    rows = _csv_rows(d, "kernel_trace.csv")
    if not rows:
        sys.exit(f"no kernel_trace.csv under {d}")
    ev = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), short_name(r["Kernel_Name"])) for r in rows)
    alone, hi = [], -1
    for i, (a, b, _) in enumerate(ev):
        nxt = ev[i + 1][0] if i + 1 < len(ev) else b + 1
        alone.append(a >= hi and b <= nxt)
        hi = max(hi, b)
    stats = {}
    for (a, b, n), solo in zip(ev, alone):
        st = stats.setdefault(n, {"n": 0, "sum": 0, "iv": [], "solo": []})
        st["n"] += 1
        st["sum"] += b - a
        st["iv"].append((a, b))
        if solo:
            st["solo"].append(b - a)
    total = sum(st["sum"] for st in stats.values())
    print("| kernel | dispatches | avg us | union ms | alone: dispatches, avg us | % of summed time |")
    print("|---|---|---|---|---|---|")
    for name, st in sorted(stats.items(), key=lambda kv: -kv[1]["sum"]):
        solo = st["solo"]
        solo_txt = f"{len(solo)}, {sum(solo) / len(solo) / 1e3:.1f}" if solo else "0, -"
        print(f"| `{name}` | {st['n']} | {st['sum'] / st['n'] / 1e3:.1f} | {_union_us(st['iv']) / 1e3:.2f} | "
              f"{solo_txt} | {st['sum'] / total * 100:.1f} |")
    # phases: the benchmark launches one marker copy before each phase
    marks = [a for a, _, n in ev if n == "k_copy"]
    if not marks:
        return
    bounds = marks + [float("inf")]
    print()
    print("Per phase (between marker launches): dispatches and average duration per kernel")
    print()
    print("| phase | kernel | dispatches | avg us |")
    print("|---|---|---|---|")
    for p in range(len(marks)):
        per = {}
        for a, b, n in ev:
            if bounds[p] < a < bounds[p + 1] and n != "k_copy":
                per.setdefault(n, []).append(b - a)
        for n, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            print(f"| {p + 1} | `{n}` | {len(v)} | {sum(v) / len(v) / 1e3:.1f} |")


def counters(d: str) -> None:
    acc = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        acc.setdefault(short_name(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
            float(r["Counter_Value"]))
    names = sorted({c for v in acc.values() for c in v})
    print("| kernel | dispatches | " + " | ".join(names) + " |")
    print("|---|---|" + "---|" * len(names))
    for n, v in sorted(acc.items()):
        cells = [f"{sum(v[c]) / len(v[c]):.4g}" if c in v else "-" for c in names]
        print(f"| `{n}` | {len(next(iter(v.values())))} | " + " | ".join(cells) + " |")


def _per_dispatch(d: str, counter: str, kernel: str):
    vals = [float(r["Counter_Value"]) for r in _csv_rows(d, "counter_collection.csv")
            if r["Counter_Name"] == counter and short_name(r["Kernel_Name"]) == kernel]
    if not vals:
        sys.exit(f"no {counter} rows for {kernel} under {d}")
    return sum(vals) / len(vals), len(vals)


def alg_bytes(which: str) -> float:
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import synth
    cfg = synth.QWEN3_0P6B
    reqs = synth.make_requests(3, cfg, n_requests=64)
    H, Hk, hd, d, F = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.d_model, cfg.d_ffn
    if which == "attn_branch":
        return float(sum(r.L * Hk * hd * 4 + r.K * (H * hd * 2 + Hk * hd * 4 + H * hd * 2) for r in reqs))
    T = sum(r.L + r.K for r in reqs)
    if which == "gemm_resid":
        o = (d * H * hd + T * H * hd) * 2 + T * d * 8
        down = (d * F + T * F) * 2 + T * d * 8
        return (o + down) / 2.0
    if which == "gemm_gateup":
        return float((2 * F * d + T * d + T * F) * 2)
    if which == "gemm_qkv":
        nq = (H + 2 * Hk) * hd
        return float((nq * d + T * d + T * nq) * 2)
    raise SystemExit(f"unknown kernel class {which}")


SOURCES = {"attn_branch": ("k_attn.hip", "common.h", "launch.h"),
           "gemm_resid": ("k_gemm.hip", "common.h", "launch.h"),
           "gemm_gateup": ("k_gemm.hip", "common.h", "launch.h"),
           "gemm_qkv": ("k_gemm.hip", "common.h", "launch.h")}


def code_hash(names) -> str:
    """Hash of the kernel sources with comments, blank lines and indentation
    removed, so that a change of code (not of comments) makes recorded
    counters stale."""
    import hashlib
    import re
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", n)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for line in text.split("\n"):
            line = re.sub(r"//.*$", "", line).strip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


def src_hash(which: str) -> str:
    return code_hash(SOURCES[which])


def traffic(d: str, kernel: str, which: str) -> None:
    f_kib, n = _per_dispatch(os.path.join(d, "fetch"), "FETCH_SIZE", kernel)
    w_kib, _ = _per_dispatch(os.path.join(d, "write"), "WRITE_SIZE", kernel)
    cf_kib, _ = _per_dispatch(os.path.join(d, "cal_fetch"), "FETCH_SIZE", "k_copy")
    cw_kib, _ = _per_dispatch(os.path.join(d, "cal_write"), "WRITE_SIZE", "k_copy")
    copy_kib = (1 << 30) / 1024.0
    fs, ws = copy_kib / cf_kib, copy_kib / cw_kib
    alg = alg_bytes(which)
    meas = (f_kib * fs + w_kib * ws) * 1024.0
    print(json.dumps({
        "kernel": kernel,
        "dispatches": n,
        "calibration": {"copy_kernel": "k_copy, 1 GiB read + 1 GiB written", "FETCH_SIZE_KiB": round(cf_kib, 1),
                        "WRITE_SIZE_KiB": round(cw_kib, 1), "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)},
        "FETCH_SIZE_KiB_per_dispatch": round(f_kib, 1),
        "WRITE_SIZE_KiB_per_dispatch": round(w_kib, 1),
        "bytes_per_launch": round(meas),
        "algorithmic_bytes_per_launch": round(alg),
        "ratio_measured_to_algorithmic": round(meas / alg, 3),
        "kernel_src_hash": src_hash(which),
    }, indent=1))


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("trace").add_argument("dir")
    sub.add_parser("counters").add_argument("dir")
    t = sub.add_parser("traffic")
    t.add_argument("dir")
    t.add_argument("--kernel", required=True, help="kernel name as in the trace table, e.g. 'k_gemm<192, 256, 2, 4, 1>'")
    t.add_argument("--which", required=True, choices=list(SOURCES))
    sub.add_parser("alg-bytes").add_argument("--which", required=True, choices=list(SOURCES))
    a = ap.parse_args()
    if a.cmd == "trace":
        trace(a.dir)
    elif a.cmd == "counters":
        counters(a.dir)
    elif a.cmd == "alg-bytes":
        print(alg_bytes(a.which))
    else:
        traffic(a.dir, a.kernel, a.which)


if __name__ == "__main__":
    main()
