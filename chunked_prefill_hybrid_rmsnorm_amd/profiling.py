"""Turn rocprofv3 output for the layer into per-kernel-slot summaries.

The library launches at most one kernel per slot (``hl_stage_name``), in a
fixed order per layer call.  rocprofv3 names kernels, not slots, and one
kernel template can fill two slots (the residual GEMM runs both the O and the
down projection), so each dispatch is labelled from its name and the slot
that came before it in the same call.

Inputs are rocprofv3 CSV files:

* ``--kernel-trace --stats`` -> ``*_kernel_trace.csv`` (durations), and
* ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` -> ``*_counter_collection.csv``
  (KiB per dispatch).  Both byte counters are scaled by what they read for a
  plain device-to-device copy of 256 MiB that the profiled program runs first
  (``bench.py --calibrate-copy``): the counters' units and coverage differ
  from one chip to another, a copy of known size does not.

Usage::

    python -m chunked_prefill_hybrid_rmsnorm_amd.profiling \\
        --trace kt_kernel_trace.csv --fetch f_counter_collection.csv \\
        --write w_counter_collection.csv --workload "..." --command "..." \\
        --md profiles/layer_kernels_mistral7b.md --traffic profiles/traffic.json
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
from collections import defaultdict
from typing import Dict, Iterable, List, Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

SLOTS = ("rmsnorm1", "gemm_qkv", "rope_kv_append", "attention", "attention_merge", "gemm_o",
         "gemm_o_reduce_rmsnorm2", "gemm_gate_up", "gemm_gate_up_reduce", "gemm_down",
         "gemm_down_reduce")
CALIBRATION_BYTES = 256 << 20


def source_hash() -> str:
    """Digest of every source the kernels and their launch shapes come from."""
    h = hashlib.sha256()
    files = []
    for d in (os.path.join(PKG, "csrc"), os.path.join(ROOT, "include")):
        files += [os.path.join(d, f) for f in sorted(os.listdir(d))
                  if f.endswith((".hip", ".h"))]
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def _base_name(name: str) -> str:
    return name.split("(")[0].replace("void ", "").strip()


def _gemm_epilogue(name: str) -> Optional[int]:
    """Epilogue template argument of a GEMM kernel name (0 store, 1 residual,
    2 SwiGLU): the fifth of gemm_dma_kernel<...>, the third of
    gemm_agpr_kernel<...>."""
    m = re.search(r"gemm_dma_kernel<([^>]*)>", name)
    if m:
        return int(m.group(1).split(",")[4])
    m = re.search(r"gemm_agpr_kernel<([^>]*)>", name)
    if m:
        return int(m.group(1).split(",")[2])
    return None


class SlotLabeler:
    """Labels the library's dispatches, one call after another."""

    def __init__(self, chained: bool = False):
        self.last = -1  # slot index of the previous dispatch of this call
        # calls with the cross-layer RMSNorm fusion: an RMSNorm right after an
        # unsplit down projection is that call's next-layer norm, not the
        # first RMSNorm of the next call
        self.chained = chained

    def label(self, kernel_name: str) -> Optional[str]:
        n = _base_name(kernel_name)
        if not n.startswith("hl::"):
            return None
        idx = SLOTS.index
        if "rmsnorm_kernel" in n:
            # the first RMSNorm; the second one when the O projection was not
            # split; the next layer's one after an unsplit down projection
            # (cross-layer fusion)
            if self.last == idx("gemm_o"):
                s = "gemm_o_reduce_rmsnorm2"
            elif self.last == idx("gemm_down") and self.chained:
                s = "gemm_down_reduce"
            else:
                s = "rmsnorm1"
        elif "gemm_splitk_reduce_swiglu" in n:
            s = "gemm_gate_up_reduce"
        elif "gemm_splitk_reduce_norm" in n:
            # after the down projection it also forms the next layer's RMSNorm
            s = "gemm_down_reduce" if self.last == idx("gemm_down") else "gemm_o_reduce_rmsnorm2"
        elif re.search(r"gemm_splitk_reduce<1[,>]", n):  # <EPI_RESIDUAL[, splits]>
            s = "gemm_down_reduce"
        elif "gemm_swiglu_agpr" in n:
            s = "gemm_gate_up"
        elif "rope_append_wide" in n or "rope_kv_append" in n:
            s = "rope_kv_append"
        elif "attention_merge" in n:
            s = "attention_merge"
        elif "attention_kernel" in n:
            s = "attention"
        elif "gemm_dma_kernel" in n or "gemm_agpr_kernel" in n:
            epi = _gemm_epilogue(kernel_name)
            if epi == 0:
                s = "gemm_qkv"
            elif epi == 2:
                s = "gemm_gate_up"
            else:
                s = "gemm_down" if self.last >= idx("gemm_gate_up") else "gemm_o"
        elif "slot_map" in n:
            return None
        else:
            return None
        self.last = idx(s)
        return s


def _rows(path: str) -> List[dict]:
    with open(path, newline="") as f:
        rows = list(csv.DictReader(f))
    key = "Dispatch_Id" if rows and "Dispatch_Id" in rows[0] else None
    if key:
        rows.sort(key=lambda r: int(r[key]))
    return rows


def kernel_durations(trace_csv: str, skip: int = 0) -> Dict[str, List[float]]:
    """Per slot, the duration (ns) of every dispatch in a kernel trace, without
    the first `skip` dispatches of each slot (the GPU's clock ramp)."""
    lab = SlotLabeler()
    out: Dict[str, List[float]] = defaultdict(list)
    for r in _rows(trace_csv):
        s = lab.label(r["Kernel_Name"])
        if s:
            out[s].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    return _drop_setup({k: v[skip:] if len(v) > skip else v for k, v in out.items()})


def _drop_setup(per_slot: Dict[str, List[float]]) -> Dict[str, List[float]]:
    """Leave out slots dispatched in fewer than a tenth of the calls: set-up
    work of the profiled program, such as the one RMSNorm that forms the
    first normalised input of the chained (layer-stack) call, whose own first
    RMSNorm slot is empty."""
    most = max((len(v) for v in per_slot.values()), default=0)
    return {k: v for k, v in per_slot.items() if 10 * len(v) >= most}


def counter_values(counter_csv: str, counter: str) -> Tuple[Dict[str, List[float]], float]:
    """Per slot, the counter's value (KiB) of every dispatch, and the value of
    the first plain copy: the 256 MiB calibration copy, which the profiled
    program runs before any other copy (later copies, e.g. the rotated
    weight clones, can be larger)."""
    lab = SlotLabeler()
    out: Dict[str, List[float]] = defaultdict(list)
    calib = 0.0
    for r in _rows(counter_csv):
        if r["Counter_Name"] != counter:
            continue
        v = float(r["Counter_Value"])
        if "copyBuffer" in r["Kernel_Name"]:
            if calib == 0.0:
                calib = v
            continue
        s = lab.label(r["Kernel_Name"])
        if s:
            out[s].append(v)
    return _drop_setup(out), calib


def _mean(v: Iterable[float]) -> float:
    v = list(v)
    return sum(v) / len(v) if v else 0.0


def summarize(trace_csv: Optional[str], fetch_csv: Optional[str], write_csv: Optional[str],
              skip: int = 0):
    res = {"slots": {}}
    durs = kernel_durations(trace_csv, skip) if trace_csv else {}
    fetch, fcal = counter_values(fetch_csv, "FETCH_SIZE") if fetch_csv else ({}, 0.0)
    write, wcal = counter_values(write_csv, "WRITE_SIZE") if write_csv else ({}, 0.0)
    fscale = CALIBRATION_BYTES / (fcal * 1024) if fcal else None
    wscale = CALIBRATION_BYTES / (wcal * 1024) if wcal else None
    res["fetch_scale"] = fscale
    res["write_scale"] = wscale
    for s in SLOTS:
        e = {}
        if s in durs:
            d = durs[s]
            e.update(calls=len(d), avg_us=_mean(d) / 1e3, min_us=min(d) / 1e3, max_us=max(d) / 1e3)
        if s in fetch and fscale:
            e["fetch_bytes"] = _mean(fetch[s]) * 1024 * fscale
        if s in write and wscale:
            e["write_bytes"] = _mean(write[s]) * 1024 * wscale
        if "fetch_bytes" in e and "write_bytes" in e:
            e["traffic_bytes"] = e["fetch_bytes"] + e["write_bytes"]
        if e:
            res["slots"][s] = e
    return res


def n_chunk_fetch(counter_csv: str, reps: int, kv_bytes_per_token: int, prompt: int = 2048) -> dict:
    """HBM bytes the attention kernel reads over the N calls of a prompt
    prefilled in N chunks (sweep --n-chunk-counters), against the closed
    form of the re-read of earlier chunks, C N (N-1)/2 kvB.

    The groups are delimited by one-element fill kernels whose order gives N
    (1, 2, 4, 8, 16); FETCH_SIZE is scaled by the first copy of the run (256
    MiB).  Every group reads the prompt's own KV once, its q rows and the
    same amount of other data, so the measured re-read is the group's bytes
    minus those of N = 1."""
    rows = _rows(counter_csv)
    calib = 0.0
    groups: List[float] = []
    lab = SlotLabeler()
    for r in rows:
        if r["Counter_Name"] != "FETCH_SIZE":
            continue
        name = r["Kernel_Name"]
        v = float(r["Counter_Value"])
        if "copyBuffer" in name:
            if calib == 0.0:
                calib = v
            continue
        if "FillFunctor" in name and int(r.get("Grid_Size", 0) or 0) <= 1024:
            groups.append(0.0)
            continue
        if groups and lab.label(name) == "attention":
            groups[-1] += v
    scale = CALIBRATION_BYTES / (calib * 1024) if calib else 1.0
    groups = groups[-5:]  # the last five markers are the N = 1 .. 16 groups
    ns = (1, 2, 4, 8, 16)[:len(groups)]
    per_n = {n: g * 1024 * scale / reps for n, g in zip(ns, groups)}
    base = per_n.get(1, 0.0)
    out = {"fetch_scale": scale, "rows": []}
    for n in ns:
        c = prompt // n
        closed = c * n * (n - 1) // 2 * kv_bytes_per_token
        meas = per_n[n] - base
        out["rows"].append({"n": n, "chunk": c, "attention_fetch_bytes": per_n[n],
                            "reread_measured_bytes": meas, "reread_closed_form_bytes": closed,
                            "ratio": meas / closed if closed else None})
    return out


def write_n_chunk_markdown(path: str, res: dict, commands: List[str]) -> None:
    lines = ["# KV re-read of chunked prefill, measured by counters", "",
             "Mistral-7B-shaped layer (8 kv heads, head_dim 128: kvB = 4096 bytes of K and V per "
             "token), a 2048-token prompt prefilled in N equal chunks over N layer calls, Bd = 0. "
             "Chunk k reads the KV of the k chunks before it (Sarathi-Serve digest, section 4), so "
             "the whole prompt re-reads C N(N-1)/2 tokens of KV.", "",
             "Commands (run from the repository root):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", f"Kernel sources digest: `{source_hash()}`", "",
              f"FETCH_SIZE scale from the 256 MiB copy: x{res['fetch_scale']:.4f}. "
              "Measured re-read = HBM bytes the attention kernel fetched over the N calls minus "
              "those of the N = 1 call, which reads the same prompt KV, q rows and tables once.", "",
              "| N | chunk C | attention HBM read over the N calls, MB | re-read measured, MB | "
              "closed form C N(N-1)/2 kvB, MB | measured / closed form |",
              "|---:|---:|---:|---:|---:|---:|"]
    for r in res["rows"]:
        ratio = f"{r['ratio']:.3f}" if r["ratio"] is not None else "-"
        lines.append(f"| {r['n']} | {r['chunk']} | {r['attention_fetch_bytes'] / 1e6:.2f} | "
                     f"{r['reread_measured_bytes'] / 1e6:.2f} | "
                     f"{r['reread_closed_form_bytes'] / 1e6:.2f} | {ratio} |")
    lines.append("")
    with open(path, "w") as fh:
        fh.write("\n".join(lines))


def stats_table(stats_csv: str) -> List[str]:
    """rocprofv3's --stats summary (kernel_stats.csv) as markdown rows: every
    kernel of the profiled run, its calls and average / min / max duration."""
    lines = ["| kernel | calls | avg us | min us | max us | share of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in _rows(stats_csv):
        name = _base_name(r["Name"])
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} % |")
    return lines


def write_markdown(path: str, res: dict, workload: str, commands: List[str],
                   stats_csv: Optional[str] = None) -> None:
    lines = [f"# Layer kernels, {workload}", "", "Commands (run from the repository root):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", f"Kernel sources digest: `{source_hash()}`", ""]
    if res.get("fetch_scale"):
        lines += [f"Byte-counter scale from the 256 MiB copy: FETCH_SIZE x{res['fetch_scale']:.4f}, "
                  f"WRITE_SIZE x{res['write_scale']:.4f}", ""]
    lines += ["| slot | calls | avg us | min us | max us | HBM read MB | HBM write MB |",
              "|---|---:|---:|---:|---:|---:|---:|"]
    tot = 0.0
    for s in SLOTS:
        e = res["slots"].get(s)
        if not e:
            continue
        tot += e.get("avg_us", 0.0)
        f = f"{e['fetch_bytes'] / 1e6:.1f}" if "fetch_bytes" in e else "-"
        w = f"{e['write_bytes'] / 1e6:.1f}" if "write_bytes" in e else "-"
        if "avg_us" in e:
            lines.append(f"| {s} | {e['calls']} | {e['avg_us']:.2f} | {e['min_us']:.2f} | "
                         f"{e['max_us']:.2f} | {f} | {w} |")
        else:
            lines.append(f"| {s} | - | - | - | - | {f} | {w} |")
    lines += ["", f"Sum of slot averages: {tot:.1f} us per layer call.", ""]
    if stats_csv:
        lines += ["rocprofv3 `--kernel-trace --stats` summary of the traced run (every dispatch, "
                  "the clock ramp included):", ""] + stats_table(stats_csv) + [""]
    with open(path, "w") as fh:
        fh.write("\n".join(lines))


def write_traffic(path: str, res: dict, workload: str, key: str) -> None:
    """Store the per-slot HBM bytes of one workload under `key`, beside the
    other workloads' entries; every entry carries the digest of the kernel
    sources it was measured on."""
    kern = {s: {"traffic_bytes": round(e["traffic_bytes"]),
                "fetch_bytes": round(e["fetch_bytes"]), "write_bytes": round(e["write_bytes"])}
            for s, e in res["slots"].items() if "traffic_bytes" in e}
    try:
        t = json.load(open(path))
    except (OSError, ValueError):
        t = {}
    if "workloads" not in t:
        t = {"workloads": {}}
    t["workloads"][key] = {"source_sha": source_hash(), "workload": workload,
                           "fetch_scale": res["fetch_scale"], "write_scale": res["write_scale"],
                           "kernels": kern}
    with open(path, "w") as fh:
        json.dump(t, fh, indent=1)
        fh.write("\n")


def stored_traffic(path: str, slot: str, key: str) -> Optional[float]:
    """HBM bytes per launch of `slot` in workload `key` from a committed
    measurement, or None when there is none or any kernel source changed
    since it was taken."""
    try:
        t = json.load(open(path))
    except (OSError, ValueError):
        return None
    w = t.get("workloads", {}).get(key)
    if not w or w.get("source_sha") != source_hash():
        return None
    e = w.get("kernels", {}).get(slot)
    return e.get("traffic_bytes") if e else None


# MFMA utilisation from one rocprofv3 --pmc pass with these four counters.
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES",
                 "GRBM_GUI_ACTIVE")
SIMDS = 256 * 4  # MI355X: 256 CUs of 4 SIMDs
XCDS = 8         # GRBM_GUI_ACTIVE counts each XCD's active cycles


def mfma_summary(counter_csv: str, trace_csv: Optional[str] = None, skip: int = 0) -> dict:
    """Per slot: bf16 MFMA flops counted by the hardware (MOPS are units of
    512 flops), MFMA busy cycles summed over all SIMDs, the kernel's active
    cycles per XCD, and from them the MFMA pipe utilisation
    busy / (SIMDS * active cycles per XCD).  With a kernel trace, also the
    counted flops over the traced average duration, against 2.5 PFLOP/s."""
    vals = {c: counter_values(counter_csv, c)[0] for c in MFMA_COUNTERS}
    durs = kernel_durations(trace_csv, skip) if trace_csv else {}
    out = {}
    for s in SLOTS:
        if s not in vals[MFMA_COUNTERS[0]]:
            continue
        mops, busy, _, active = (_mean(vals[c].get(s, [])) for c in MFMA_COUNTERS)
        if mops <= 0:
            continue
        e = {"flops": mops * 512, "busy_cycles": busy, "active_cycles_per_xcd": active / XCDS}
        e["mfma_util"] = busy / (SIMDS * e["active_cycles_per_xcd"]) if active else None
        if s in durs and durs[s]:
            t = _mean(durs[s]) / 1e9
            e["trace_us"] = t * 1e6
            e["tflops"] = e["flops"] / t / 1e12
            e["frac_of_peak"] = e["flops"] / t / 2.5e15
        out[s] = e
    return out


def write_mfma_markdown(path: str, res: dict, workload: str, commands: List[str]) -> None:
    lines = [f"# MFMA utilisation per kernel, {workload}", "", "Commands (run from the repository root):",
             ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", f"Kernel sources digest: `{source_hash()}`", "",
              "Counted flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512. MFMA util = SQ_VALU_MFMA_BUSY_CYCLES "
              f"(summed over the {SIMDS} SIMDs) / ({SIMDS} x GRBM_GUI_ACTIVE / {XCDS}), i.e. the share "
              "of the kernel's cycles each SIMD's matrix pipe was busy. In a counter pass the active "
              "cycles span the whole serialised dispatch, start-up included, so for short kernels "
              "this is a lower bound. Trace columns use the kernel trace's average duration; frac of "
              "peak is the counted flops over that duration against 2.5 PFLOP/s dense bf16.", "",
              "| slot | counted GFLOP | MFMA busy Mcycles | active kcycles / XCD | MFMA util | trace us "
              "| TFLOP/s | frac of peak |",
              "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for s, e in res.items():
        def f(k, fmt):
            return format(e[k], fmt) if e.get(k) is not None else "-"
        lines.append(f"| {s} | {e['flops'] / 1e9:.2f} | {e['busy_cycles'] / 1e6:.2f} | "
                     f"{e['active_cycles_per_xcd'] / 1e3:.1f} | {f('mfma_util', '.3f')} | "
                     f"{f('trace_us', '.2f')} | {f('tflops', '.0f')} | {f('frac_of_peak', '.3f')} |")
    lines.append("")
    with open(path, "w") as fh:
        fh.write("\n".join(lines))


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--trace")
    p.add_argument("--fetch")
    p.add_argument("--write")
    p.add_argument("--workload", default="")
    p.add_argument("--command", action="append", default=[])
    p.add_argument("--md")
    p.add_argument("--traffic")
    p.add_argument("--key", default="mistral", help="workload key of the --traffic entry")
    p.add_argument("--skip", type=int, default=0,
                   help="drop the first N dispatches of each slot (clock ramp)")
    p.add_argument("--stats", help="rocprofv3 kernel_stats.csv of the traced run")
    p.add_argument("--mfma", help="counter CSV of a pass over MFMA_COUNTERS")
    p.add_argument("--mfma-md")
    p.add_argument("--n-chunk", help="FETCH_SIZE CSV of sweep --n-chunk-counters")
    p.add_argument("--n-chunk-reps", type=int, default=5)
    p.add_argument("--n-chunk-md")
    a = p.parse_args()
    if a.n_chunk:
        res = n_chunk_fetch(a.n_chunk, a.n_chunk_reps, 4096)
        if a.n_chunk_md:
            write_n_chunk_markdown(a.n_chunk_md, res, a.command)
        print(json.dumps(res, indent=1))
        return
    if a.mfma:
        res = mfma_summary(a.mfma, a.trace, a.skip)
        if a.mfma_md:
            write_mfma_markdown(a.mfma_md, res, a.workload, a.command)
        print(json.dumps(res, indent=1))
        return
    res = summarize(a.trace, a.fetch, a.write, a.skip)
    if a.md:
        write_markdown(a.md, res, a.workload, a.command, a.stats)
    if a.traffic:
        write_traffic(a.traffic, res, a.workload, a.key)
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
