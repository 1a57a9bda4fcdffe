"""Summaries of rocprofv3 output for the decode launches, written as short text under profiles/.

    python -m moe_routed_expert_route_amd.profsum kernels --stats DIR/run_kernel_stats.csv \\
        --workload nl4_2560x768_t1 --command "..."
    python -m moe_routed_expert_route_amd.profsum traffic --fetch DIR1/run_counter_collection.csv \\
        --write DIR2/run_counter_collection.csv --workload nl4_2560x768_t1 --command "..."

`kernels` turns a `--kernel-trace --stats` table into profiles/kernels_<workload>.md and .json
(average launch duration per kernel); `traffic` turns two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE`
runs of `bench.py --calib` into profiles/traffic_<workload>.md and .json: HBM bytes per launch,
each counter scaled by what it reads for a device-to-device copy of known size in the same run.
Both .json files carry the SHA-256 of the kernel sources, so bench.py uses them only while the
kernels are the ones they were taken from.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ("moe_routed_expert_route_amd/csrc/moe_route.hip",
                  "moe_routed_expert_route_amd/csrc/moe_device.hpp",
                  "moe_routed_expert_route_amd/build.py")
# the decode launches by their mangled-name prefix (template arguments: formats, mode); the prompt
# path's GEMM (gate/up and down launches share the kernel)
KINDS = {"gate_up": "void moe::k_gate_up<", "down": "void moe::k_down<"}
PF_KIND = {"prefill_gemm": "void moe::k_pf_gemm<"}
CALIB = "__amd_rocclr_copyBuffer"


def source_digest() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(f"none of {names} in {sorted(row)}")


def kernel_stats(path):
    """name -> {calls, avg_ns, min_ns, max_ns, total_ns} from a rocprofv3 kernel stats table."""
    out = {}
    for r in _rows(path):
        name = _col(r, "Name", "KernelName", "Kernel_Name")
        out[name] = {"calls": int(_col(r, "Calls")), "avg_ns": float(_col(r, "AverageNs")),
                     "min_ns": float(_col(r, "MinNs")), "max_ns": float(_col(r, "MaxNs")),
                     "total_ns": float(_col(r, "TotalDurationNs"))}
    return out


def pick(names, kind):
    """The kernels of `kind` among `names` (callers take the most-called)."""
    return [n for n in names if n.startswith(KINDS[kind])]


def write_kernels(stats_csv, workload, command):
    st = kernel_stats(stats_csv)
    total = sum(v["total_ns"] for v in st.values())
    doc = {"workload": workload, "source_sha256": source_digest(), "command": command, "kernels": {}}
    for kind in KINDS:
        names = pick(st, kind)
        if names:
            n = max(names, key=lambda k: st[k]["calls"])
            doc["kernels"][kind] = {"kernel": n, **st[n]}
    lines = [f"# Kernel trace: {workload}", "", "Command (repo root, one MI355X):", "", f"    {command}", "",
             "rocprofv3 kernel stats, durations in ns:", "",
             "| kernel | calls | average ns | min ns | max ns | share |", "|---|---|---|---|---|---|"]
    for n, v in sorted(st.items(), key=lambda kv: -kv[1]["total_ns"])[:10]:
        lines.append(f"| `{n[:90]}` | {v['calls']} | {v['avg_ns']:.0f} | {v['min_ns']:.0f} | "
                     f"{v['max_ns']:.0f} | {100 * v['total_ns'] / total:.1f}% |")
    lines += ["", f"Kernel sources SHA-256: `{doc['source_sha256']}`", ""]
    base = os.path.join(PROFILES, f"kernels_{workload}")
    with open(base + ".md", "w") as f:
        f.write("\n".join(lines))
    with open(base + ".json", "w") as f:
        json.dump(doc, f, indent=1)
    return doc


def counter_per_dispatch(path, counter):
    """name -> (mean value per dispatch, dispatches) of `counter` in a rocprofv3 counter table
    (values of one dispatch summed over the table's dimension rows)."""
    per = defaultdict(float)
    names = {}
    for r in _rows(path):
        if _col(r, "Counter_Name", "Counter-Name") != counter:
            continue
        d = _col(r, "Dispatch_Id", "Dispatch-Id")
        per[d] += float(_col(r, "Counter_Value", "Counter-Value"))
        names[d] = _col(r, "Kernel_Name", "Kernel-Name")
    agg = defaultdict(list)
    for d, v in per.items():
        agg[names[d]].append(v)
    return {n: (sum(v) / len(v), len(v)) for n, v in agg.items()}


def dispatch_values(path, counter, prefix):
    """Per-dispatch values of `counter` (summed over dimension rows) for kernels named `prefix`..."""
    per = defaultdict(float)
    for r in _rows(path):
        if _col(r, "Counter_Name", "Counter-Name") == counter and \
                _col(r, "Kernel_Name", "Kernel-Name").startswith(prefix):
            per[_col(r, "Dispatch_Id", "Dispatch-Id")] += float(_col(r, "Counter_Value", "Counter-Value"))
    return list(per.values())


def write_traffic(fetch_csv, write_csv, workload, command, calib_kib=262144.0, algorithmic=None):
    fe = counter_per_dispatch(fetch_csv, "FETCH_SIZE")
    wr = counter_per_dispatch(write_csv, "WRITE_SIZE")
    # the calibration copy is the largest copy dispatch of the run (256 MiB read, 256 MiB written)
    f_cal = max(dispatch_values(fetch_csv, "FETCH_SIZE", CALIB))
    w_cal = max(dispatch_values(write_csv, "WRITE_SIZE", CALIB))
    fs, ws = calib_kib / f_cal, calib_kib / w_cal
    doc = {"workload": workload, "source_sha256": source_digest(), "command": command,
           "calibration": {"kernel": f"{CALIB}, 256 MiB device-to-device copy (bench.py --calib)",
                           "expected_kib": calib_kib, "fetch_kib": f_cal, "write_kib": w_cal,
                           "fetch_scale": fs, "write_scale": ws},
           "kernels": {}}
    for kind in KINDS:
        names = [n for n in fe if n.startswith(KINDS[kind])]
        if not names:
            continue
        n = max(names, key=lambda k: fe[k][1])
        fk, nd = fe[n]
        wk = wr.get(n, (0.0, 0))[0]
        hbm = int(round((fk * fs + wk * ws) * 1024))
        doc["kernels"][kind] = {"kernel": n, "fetch_kib": fk, "write_kib": wk, "hbm_bytes_per_launch": hbm,
                                "dispatches": nd}
        if algorithmic and kind in algorithmic:
            doc["kernels"][kind]["algorithmic_bytes_per_launch"] = algorithmic[kind]
            doc["kernels"][kind]["traffic_over_algorithmic"] = round(hbm / algorithmic[kind], 4)
    lines = [f"# HBM traffic per launch: {workload}", "", "Commands (repo root, one MI355X), one counter per run:",
             "", f"    {command}", "",
             f"Calibration: a 256 MiB device-to-device copy reads FETCH_SIZE {f_cal:.1f} KiB and WRITE_SIZE "
             f"{w_cal:.1f} KiB per dispatch; scales {fs:.4f} (fetch) and {ws:.4f} (write).", "",
             "| launch | kernel | FETCH KiB | WRITE KiB | HBM bytes (scaled) | algorithmic bytes | ratio |",
             "|---|---|---|---|---|---|---|"]
    for kind, v in doc["kernels"].items():
        alg = v.get("algorithmic_bytes_per_launch")
        lines.append(f"| {kind} | `{v['kernel'][:60]}` | {v['fetch_kib']:.1f} | {v['write_kib']:.1f} | "
                     f"{v['hbm_bytes_per_launch']} | {alg if alg else '-'} | "
                     f"{v.get('traffic_over_algorithmic', '-')} |")
    lines += ["", f"Kernel sources SHA-256: `{doc['source_sha256']}`", ""]
    base = os.path.join(PROFILES, f"traffic_{workload}")
    with open(base + ".md", "w") as f:
        f.write("\n".join(lines))
    with open(base + ".json", "w") as f:
        json.dump(doc, f, indent=1)
    return doc


SQ = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM", "SQ_ACTIVE_INST_VALU",
      "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT")


def write_sq(csv_path, name, title, command, weights=None, kinds=None):
    """profiles/sq_<name>.md: per-launch SQ counters of each kind (mean over the run's dispatches)
    and what follows from them: instructions per wave, VALU lane-instructions per weight (weights:
    kind -> weights per launch), SALU per VALU, the share of LDS cycles lost to bank conflicts."""
    kinds = kinds or KINDS
    per = {c: counter_per_dispatch(csv_path, c) for c in SQ}
    rows = {}
    for kind, prefix in kinds.items():
        for c in SQ:
            hits = {n: v for n, v in per[c].items() if n.startswith(prefix)}
            if hits:
                n = max(hits, key=lambda k: hits[k][1])
                rows.setdefault(kind, {"kernel": n, "dispatches": hits[n][1]})[c] = hits[n][0]
    lines = [f"# SQ counters: {title}", "", "Command (repo root, one MI355X):", "", f"    {command}", "",
             "Mean per launch over the run's dispatches (whole-device sums):", "",
             "| counter | " + " | ".join(rows) + " |", "|---" * (len(rows) + 1) + "|"]
    for c in SQ:
        lines.append(f"| {c} | " + " | ".join(f"{rows[k].get(c, 0):.0f}" for k in rows) + " |")
    lines += ["", "| figure | " + " | ".join(rows) + " |", "|---" * (len(rows) + 1) + "|"]
    def fig(label, f):
        vals = []
        for k in rows:
            try:
                vals.append(f(k, rows[k]))
            except (KeyError, ZeroDivisionError, TypeError):
                vals.append("-")
        lines.append(f"| {label} | " + " | ".join(v if isinstance(v, str) else f"{v:.3f}" for v in vals) + " |")
    fig("VALU instructions per wave", lambda k, r: r["SQ_INSTS_VALU"] / r["SQ_WAVES"])
    fig("SALU instructions per wave", lambda k, r: r["SQ_INSTS_SALU"] / r["SQ_WAVES"])
    fig("LDS instructions per wave", lambda k, r: r["SQ_INSTS_LDS"] / r["SQ_WAVES"])
    fig("VMEM instructions per wave", lambda k, r: r["SQ_INSTS_VMEM"] / r["SQ_WAVES"])
    if weights:
        fig("VALU lane-instructions per weight (x 64)", lambda k, r: r["SQ_INSTS_VALU"] * 64 / weights[k])
    fig("SALU per VALU instruction", lambda k, r: r["SQ_INSTS_SALU"] / r["SQ_INSTS_VALU"])
    fig("LDS bank-conflict cycles / LDS active cycles",
        lambda k, r: r["SQ_LDS_BANK_CONFLICT"] / r["SQ_LDS_IDX_ACTIVE"])
    lines += [""] + [f"- {k}: `{r['kernel'][:100]}` ({r['dispatches']} dispatches)" for k, r in rows.items()]
    if weights:
        lines += [f"- weights per launch: " + ", ".join(f"{k} {w:,}" for k, w in weights.items())]
    lines += ["", f"Kernel sources SHA-256: `{source_digest()}`", ""]
    with open(os.path.join(PROFILES, f"sq_{name}.md"), "w") as f:
        f.write("\n".join(lines))
    return rows


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("--stats", required=True)
    k.add_argument("--workload", required=True)
    k.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--gate-up-bytes", type=int, default=0, help="algorithmic bytes per gate/up launch")
    t.add_argument("--down-bytes", type=int, default=0, help="algorithmic bytes per down launch")
    q = sub.add_parser("sq")
    q.add_argument("--csv", required=True)
    q.add_argument("--name", required=True)
    q.add_argument("--title", required=True)
    q.add_argument("--command", required=True)
    q.add_argument("--gate-up-weights", type=int, default=0)
    q.add_argument("--down-weights", type=int, default=0)
    q.add_argument("--prefill", action="store_true", help="the prompt path's GEMM launches")
    a = ap.parse_args()
    if a.what == "sq":
        w = {k: v for k, v in (("gate_up", a.gate_up_weights), ("down", a.down_weights)) if v}
        rows = write_sq(a.csv, a.name, a.title, a.command, weights=w or None,
                        kinds=PF_KIND if a.prefill else None)
        print(json.dumps(rows, indent=1))
        return
    if a.what == "kernels":
        doc = write_kernels(a.stats, a.workload, a.command)
    else:
        alg = {k: v for k, v in (("gate_up", a.gate_up_bytes), ("down", a.down_bytes)) if v}
        doc = write_traffic(a.fetch, a.write, a.workload, a.command, algorithmic=alg or None)
    print(json.dumps(doc["kernels"], indent=1))


if __name__ == "__main__":
    main()
