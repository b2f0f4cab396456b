"""Per-config HBM traffic from two rocprofv3 counter passes.

A ``bench.py --counter-pass MANIFEST`` run launches a plain copy kernel of
known size, then every config a few times over rotated weight copies, and
writes MANIFEST: for each config, in launch order, the kernels one step of
it launches and how many steps it ran.  Run it twice under rocprofv3, once
with ``--pmc FETCH_SIZE`` and once with ``--pmc WRITE_SIZE`` (they cannot
share a pass), then::

    python -m weight_streaming_gemv_decode_amd.profsum --fetch F.csv --write W.csv \\
        --manifest MANIFEST --out profiles/traffic_hbm_counters_per_config.md

Each counter is scaled by what it reads for the copy kernel (which reads
and writes a known number of bytes), dispatches are assigned to configs in
launch order (the dispatches of other kernels, such as input set-up, are
skipped), and every config's bytes per step are compared with its
algorithmic bytes.  The summary ends with one ``traffic-json:`` line per
config that bench.py attaches to its results while the kernel sources still
hash to the ones measured.  Pure Python: no torch, no GPU.

The same run under one pass of shader counters (``--pmc`` with the SQ_ and
GRBM_ counters of SQ_COUNTERS) is summarised per config and kernel with
``--sq CSV`` instead of ``--fetch/--write``: resident waves per SIMD, the
vector ALU's and the matrix cores' busy fractions, and instructions per
wave.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
from typing import Dict, List, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)
# device code and launch planning of every measured kernel
SOURCES = ["weight_streaming_gemv_decode_amd/csrc/dense.hip", "weight_streaming_gemv_decode_amd/csrc/w4.hip",
           "weight_streaming_gemv_decode_amd/csrc/wsg_common.hpp", "weight_streaming_gemv_decode_amd/csrc/argmax.hpp",
           "weight_streaming_gemv_decode_amd/csrc/conv1d.hpp", "weight_streaming_gemv_decode_amd/csrc/api.cpp"]
COPY_KERNEL = "AUnaryFunctor"   # torch's elementwise multiply, the calibration copy
JSON_TAG = "traffic-json: "


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed, so that
    a change of comments alone keeps the hash."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_sha256(repo: str = REPO) -> str:
    """Hash of the code (not the comments) of every measured kernel source."""
    h = hashlib.sha256()
    for s in SOURCES:
        with open(os.path.join(repo, s), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def measured_traffic(path: str, label: str = "c3_grouped") -> Optional[dict]:
    """The counter record of one config from a summary, or None when the
    summary or the config is missing or the kernel sources changed since
    the counters were taken."""
    recs = measured_traffic_all(path)
    return None if recs is None else recs.get(label)


def measured_traffic_all(path: str) -> Optional[Dict[str, dict]]:
    if not path or not os.path.exists(path):
        return None
    recs = {}
    with open(path) as f:
        for line in f:
            if line.startswith(JSON_TAG):
                r = json.loads(line[len(JSON_TAG):])
                recs[r.get("label", "c3_grouped")] = r
    if not recs:
        return None
    sha = source_sha256()
    return {k: v for k, v in recs.items() if v.get("source_sha256") == sha} or None


def _dispatches(path: str, counter: str) -> List[tuple]:
    """(dispatch id, kernel name, value) of one counter, in dispatch order."""
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, v = rows.get(d, (r["Kernel_Name"], 0.0))
            rows[d] = (name, v + float(r["Counter_Value"]))
    return [(d, n, v) for d, (n, v) in sorted(rows.items())]


def per_config(path: str, counter: str, manifest: List[dict]) -> Dict[str, dict]:
    """Average counter value per step of every manifest entry, plus the
    copy kernel's average (entry label 'calibration')."""
    disp = _dispatches(path, counter)
    out = {}
    i = 0
    for e in manifest:
        kernels = e["kernels"]
        need = e["steps"] * len(kernels)
        vals, names = [], collections.Counter()
        while len(vals) < need and i < len(disp):
            _, name, v = disp[i]
            i += 1
            hit = [k for k in kernels if k in name]
            if hit:
                vals.append(v)
                names[hit[0]] += 1
        if len(vals) < need:
            raise ValueError(f"{e['label']}: found {len(vals)} of {need} dispatches of {kernels} in {path}")
        out[e["label"]] = {"per_step": sum(vals) / e["steps"], "dispatches": len(vals), "kernels": dict(names)}
    return out


# One counter pass on MI355X: at most 8 SQ_ and 2 GRBM_ counters.
SQ_COUNTERS = ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_MFMA",
               "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"]
# A second pass for the memory units: the vector-memory address unit's busy
# cycles (average over its instances), the L1 cache's cycles stalled on it
# (worst instance), and the L2's busy cycles (average over its channels).
MEM_COUNTERS = ["TA_BUSY_avr", "TCP_TCP_TA_DATA_STALL_CYCLES_max", "TCC_BUSY_avr", "GRBM_GUI_ACTIVE"]
XCDS, SIMDS = 8, 1024   # MI355X: 8 compute dies, 256 CUs of 4 SIMDs


def _sq_dispatches(path: str) -> List[dict]:
    """Per dispatch, in order: kernel name, duration (ns), registers, LDS
    bytes and the sum of each counter over its rows."""
    rows: Dict[int, dict] = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            e = rows.setdefault(d, {"name": r["Kernel_Name"], "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                                    "vgpr": int(r["VGPR_Count"]), "agpr": int(r["Accum_VGPR_Count"]),
                                    "sgpr": int(r["SGPR_Count"]), "lds": int(r["LDS_Block_Size"]), "c": {}})
            e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [rows[d] for d in sorted(rows)]


def sq_per_config(path: str, manifest: List[dict], counters: List[str] = SQ_COUNTERS) -> List[dict]:
    """Average counters per dispatch of every (config, kernel), dispatches
    assigned to configs in launch order as in per_config."""
    disp = _sq_dispatches(path)
    out, i = [], 0
    for e in manifest:
        kernels = e["kernels"]
        need = e["steps"] * len(kernels)
        got: Dict[str, List[dict]] = collections.defaultdict(list)
        n = 0
        while n < need and i < len(disp):
            d = disp[i]
            i += 1
            hit = [k for k in kernels if k in d["name"]]
            if hit:
                got[hit[0]].append(d)
                n += 1
        if n < need:
            raise ValueError(f"{e['label']}: found {n} of {need} dispatches of {kernels} in {path}")
        for k, ds in got.items():
            avg = {c: sum(d["c"].get(c, 0.0) for d in ds) / len(ds) for c in counters}
            out.append({"label": e["label"], "workload": e["workload"], "kernel": k, "dispatches": len(ds),
                        "per_step": len(ds) / e["steps"], "algorithmic_bytes": e["algorithmic_bytes"],
                        "ns": sum(d["ns"] for d in ds) / len(ds), "vgpr": ds[0]["vgpr"], "agpr": ds[0]["agpr"],
                        "sgpr": ds[0]["sgpr"], **avg})
    return out


def sq_derived(r: dict) -> dict:
    """GRBM_GUI_ACTIVE adds the busy cycles of the 8 compute dies (about 20
    per ns of kernel time on MI355X, 8 dies at ~2.5 GHz: grbm_per_ns shows
    it), so one die was busy g = GRBM_GUI_ACTIVE / 8 cycles.  SQ_WAVE_CYCLES
    and SQ_ACTIVE_INST_VALU count quad-cycles summed over all SIMDs;
    SQ_VALU_MFMA_BUSY_CYCLES counts cycles."""
    g = r["GRBM_GUI_ACTIVE"] / XCDS
    kib = r["algorithmic_bytes"] / 1024.0 / r["per_step"] if r["per_step"] else 0.0  # per dispatch
    return {"grbm_per_ns": r["GRBM_GUI_ACTIVE"] / r["ns"] if r["ns"] else 0.0,
            "valu_per_kib": r["SQ_INSTS_VALU"] / kib if kib else 0.0,
            "mfma_per_kib": r["SQ_INSTS_MFMA"] / kib if kib else 0.0,
            "waves_per_simd": 4 * r["SQ_WAVE_CYCLES"] / (g * SIMDS) if g else 0.0,
            "valu_busy": 4 * r["SQ_ACTIVE_INST_VALU"] / (g * SIMDS) if g else 0.0,
            "mfma_busy": r["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * SIMDS) if g else 0.0,
            "valu_per_wave": r["SQ_INSTS_VALU"] / r["SQ_WAVES"] if r["SQ_WAVES"] else 0.0,
            "mfma_per_wave": r["SQ_INSTS_MFMA"] / r["SQ_WAVES"] if r["SQ_WAVES"] else 0.0,
            "lds_per_wave": r["SQ_INSTS_LDS"] / r["SQ_WAVES"] if r["SQ_WAVES"] else 0.0}


def mem_derived(r: dict) -> dict:
    """Busy fractions of the memory units over the same die-busy cycles g."""
    g = r["GRBM_GUI_ACTIVE"] / XCDS
    return {"ta_busy": r["TA_BUSY_avr"] / g if g else 0.0,
            "tcp_stall": r["TCP_TCP_TA_DATA_STALL_CYCLES_max"] / g if g else 0.0,
            "tcc_busy": r["TCC_BUSY_avr"] / g if g else 0.0}


def render_sq(recs: List[dict], commands: List[str], notes: List[str] = (), mem: Optional[List[dict]] = None) -> str:
    lines = ["# Shader counters per config and kernel", "",
             "One counter pass on one MI355X over a `bench.py --counter-pass` run (every config a few steps, "
             f"in launch order), counters {', '.join(SQ_COUNTERS)}. Commands (repository root as `$REPO`, run "
             "from `/tmp`):", "", "```"] + commands + ["```", "",
             "Derived: one compute die was busy g = GRBM_GUI_ACTIVE / 8 cycles (GRBM_GUI_ACTIVE adds the 8 dies; "
             "the `GRBM/ns` column, about 20 = 8 dies at ~2.5 GHz, checks it against the dispatch timestamps); "
             "waves/SIMD = 4 SQ_WAVE_CYCLES / (g x 1024 SIMDs) (quad-cycles), VALU busy = 4 SQ_ACTIVE_INST_VALU "
             "/ (g x 1024), MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (g x 1024); VALU/KiB and MFMA/KiB are wave "
             "instructions per KiB of the config's algorithmic bytes. VGPR, AGPR and SGPR are the counts the "
             "profiler reports (in its allocation units, not the compiler's register numbers)." +
             (f" The memory-unit columns come from a second pass over the same run ({', '.join(MEM_COUNTERS)}), "
              "each over the same g: the vector-memory address unit (TA) busy, averaged over its instances; the "
              "L1 cache (TCP) stalled on TA data, worst instance; the L2 (TCC) busy, averaged over its channels."
              if mem else ""), "",
             "| Config | Kernel | Dispatches | us | GRBM/ns | VGPR/AGPR/SGPR | waves/SIMD | VALU busy "
             "| MFMA busy | VALU/KiB | MFMA/KiB | VALU/wave | LDS/wave |" + (" TA busy | TCP stalled on TA | TCC busy |" if mem else ""),
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|" + ("---|---|---|" if mem else "")]
    mem_by = {(m["label"], m["kernel"]): m for m in (mem or [])}
    for r in recs:
        d = sq_derived(r)
        m = mem_by.get((r["label"], r["kernel"]))
        extra = ""
        if mem:
            if m:
                md = mem_derived(m)
                extra = f" {100 * md['ta_busy']:.0f}% | {100 * md['tcp_stall']:.0f}% | {100 * md['tcc_busy']:.0f}% |"
            else:
                extra = " — | — | — |"
        lines.append(f"| {r['workload']} | `{r['kernel']}` | {r['dispatches']} | {r['ns'] / 1e3:.1f} "
                     f"| {d['grbm_per_ns']:.1f} | {r['vgpr']}/{r['agpr']}/{r['sgpr']} "
                     f"| {d['waves_per_simd']:.2f} | {100 * d['valu_busy']:.0f}% | {100 * d['mfma_busy']:.0f}% "
                     f"| {d['valu_per_kib']:.2f} | {d['mfma_per_kib']:.3f} | {d['valu_per_wave']:.0f} "
                     f"| {d['lds_per_wave']:.0f} |" + extra)
    lines.append("")
    lines += [n + "\n" for n in notes]
    return "\n".join(lines) + "\n"


def summarize(fetch_csv: str, write_csv: str, manifest_path: str) -> List[dict]:
    with open(manifest_path) as f:
        man = json.load(f)
    entries = man["configs"]
    fetch = per_config(fetch_csv, "FETCH_SIZE", entries)
    write = per_config(write_csv, "WRITE_SIZE", entries)
    cal = man["calibration"]
    fs = cal["read_bytes"] / 1024.0 / fetch[cal["label"]]["per_step"]
    ws = cal["write_bytes"] / 1024.0 / write[cal["label"]]["per_step"]
    sha = source_sha256()
    recs = []
    for e in entries:
        if e["label"] == cal["label"]:
            continue
        fk, wk = fetch[e["label"]]["per_step"], write[e["label"]]["per_step"]
        rb, wb = round(fk * 1024 * fs), round(wk * 1024 * ws)
        recs.append({"label": e["label"], "workload": e["workload"], "kernels": e["kernels"],
                     "steps_sampled": e["steps"], "fetch_kib_per_step": round(fk, 1), "write_kib_per_step": round(wk, 1),
                     "fetch_scale": round(fs, 4), "write_scale": round(ws, 4), "read_bytes": rb, "write_bytes": wb,
                     "bytes": rb + wb, "algorithmic_bytes": e["algorithmic_bytes"],
                     "ratio_to_algorithmic": round((rb + wb) / e["algorithmic_bytes"], 4), "source_sha256": sha})
    return recs, {"fetch_scale": fs, "write_scale": ws, "label": cal["label"],
                  "fetch_kib": fetch[cal["label"]]["per_step"], "write_kib": write[cal["label"]]["per_step"],
                  "read_bytes": cal["read_bytes"], "write_bytes": cal["write_bytes"]}


def render(recs: List[dict], cal: dict, commands: List[str], notes: List[str] = ()) -> str:
    lines = ["# HBM traffic per config: FETCH_SIZE and WRITE_SIZE counter passes", "",
             "Two counter passes on one MI355X (one counter each), over the same `bench.py --counter-pass` run: "
             "a plain fp32 copy of known size first, then every config over rotated weight copies (more bytes "
             "than the 256 MB Infinity Cache), a few steps each. Commands (repository root as `$REPO`, run "
             "from `/tmp`):", "", "```"] + commands + ["```", "",
             f"Calibration: the copy kernel reads {cal['read_bytes']:,} B and writes {cal['write_bytes']:,} B; "
             f"FETCH_SIZE reads {cal['fetch_kib']:.1f} KiB for it (scale {cal['fetch_scale']:.4f}) and WRITE_SIZE "
             f"{cal['write_kib']:.1f} KiB (scale {cal['write_scale']:.4f}). Every config's counters are scaled by "
             "these factors.", "",
             "| Config | Kernels of one step | Steps | Read (B/step) | Written (B/step) | Algorithmic (B/step) "
             "| Traffic / algorithmic |", "|---|---|---|---|---|---|---|"]
    for r in recs:
        ks = ", ".join(f"`{k}`" for k in r["kernels"])
        lines.append(f"| {r['workload']} | {ks} | {r['steps_sampled']} | {r['read_bytes']:,} | {r['write_bytes']:,} "
                     f"| {r['algorithmic_bytes']:,} | {r['ratio_to_algorithmic']:.4f} |")
    lines += ["", "Algorithmic bytes are weights + scales + activations + outputs that a step needs; split-K "
              "partials and re-read activations are excess and show up above 1.0. `source_sha256` hashes the "
              "code of the measured kernel sources (comments and whitespace left out); bench.py attaches a record "
              "to its results only while that code is unchanged.",
              ""]
    lines += [n + "\n" for n in notes]
    lines += [JSON_TAG + json.dumps(r) for r in recs]
    return "\n".join(lines) + "\n"


# ---------------------------------------------------------- chain trace --
#
# A persistent step traced with wsg_decode_step_trace leaves four 64-bit words
# per work unit: start, input staged, finished (the 100 MHz real-time clock,
# one time base for the whole chip) and linear | workgroup << 32.  Per linear
# j of the dependent chain: when its first and last units had their input,
# when its last unit finished, and from these the parts of a stage.

CHAIN_TICK_US = 0.01  # the real-time clock counts at 100 MHz


def chain_trace_stats(words: List[int], tick_us: float = CHAIN_TICK_US) -> dict:
    """words: the trace buffer, 4 words per unit in unit order."""
    import statistics as st
    n = len(words) // 4
    if n == 0:
        raise ValueError("empty trace")
    rec = [words[4 * u:4 * u + 4] for u in range(n)]
    base = min(r[0] for r in rec)
    per: Dict[int, dict] = collections.OrderedDict()
    for r in rec:
        t0, t1, t2 = ((r[k] - base) * tick_us for k in range(3))
        lin = r[3] & 0xFFFFFFFF
        d = per.setdefault(lin, {"units": 0, "start": t0, "inputs": [], "end": t2, "compute": []})
        d["units"] += 1
        d["start"] = min(d["start"], t0)
        d["end"] = max(d["end"], t2)
        d["inputs"].append(t1)
        d["compute"].append(t2 - t1)
    lins = []
    prev_end = 0.0
    for j, d in per.items():
        ins = sorted(d["inputs"])
        row = {"linear": j, "units": d["units"], "start_us": d["start"], "input_first_us": ins[0],
               "input_median_us": st.median(ins), "input_last_us": ins[-1], "end_us": d["end"],
               "compute_median_us": st.median(d["compute"])}
        row["detect_us"] = ins[0] - prev_end      # last producer done -> first consumer has its input
        row["spread_us"] = ins[-1] - ins[0]       # first -> last consumer
        row["tail_us"] = d["end"] - ins[-1]       # last input -> linear done
        row["stage_us"] = d["end"] - prev_end
        prev_end = d["end"]
        lins.append(row)
    # the layer stages: every linear but the first (its input is ready at
    # launch) and the last (the head, bandwidth-bound over many units)
    mid = lins[1:-1] if len(lins) > 2 else lins
    med = {k: st.median(r[k] for r in mid) for k in ("stage_us", "detect_us", "spread_us", "compute_median_us",
                                                     "tail_us")}
    waits = sorted((r[1] - r[0]) * tick_us for r in rec)
    return {"units": n, "linears": len(lins), "span_us": max(r["end_us"] for r in lins), "per_linear": lins,
            "median_stage": med, "unit_wait_median_us": st.median(waits),
            "unit_wait_p90_us": waits[int(0.9 * (len(waits) - 1))]}


def render_chain_trace(stats: dict, names: List[str], command: str, step_us: float, traced_us: float,
                       notes: List[str] = ()) -> str:
    """Markdown summary of chain_trace_stats (names: one per linear, in order)."""
    m = stats["median_stage"]
    out = ["# Persistent dependent step: where a stage's time goes", "",
           "Command (repository root as `$REPO`, one MI355X):", "", "```", command, "```", "",
           f"One traced step of the dependent chain: {stats['units']:,} work units over {stats['linears']} "
           f"linears. The step took {traced_us:.1f} us traced (HIP events) against {step_us:.1f} us untraced; "
           f"the trace spans {stats['span_us']:.1f} us of the chip's 100 MHz real-time clock (a check on that "
           "rate). Tracing adds one workgroup barrier per unit.", "",
           "Per linear: `in first/median/last` is when its units had their input staged; `detect` is from the "
           "previous linear's last finished unit to this linear's first staged input, `spread` from its first "
           "to its last staged input, `tail` from its last input to its last finished unit, `compute` the "
           "median time of a unit after its input (us).", "",
           "| # | Linear | Units | Start | In first | In median | In last | End | Detect | Spread | Compute | Tail |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    rows = stats["per_linear"]
    show = list(range(min(8, len(rows)))) + list(range(max(8, len(rows) - 5), len(rows)))
    for i in show:
        r = rows[i]
        nm = names[r["linear"]] if r["linear"] < len(names) else str(r["linear"])
        out.append(f"| {r['linear']} | {nm} | {r['units']} | {r['start_us']:.1f} | {r['input_first_us']:.1f} | "
                   f"{r['input_median_us']:.1f} | {r['input_last_us']:.1f} | {r['end_us']:.1f} | "
                   f"{r['detect_us']:.2f} | {r['spread_us']:.2f} | {r['compute_median_us']:.2f} | "
                   f"{r['tail_us']:.2f} |")
    out += ["", f"Medians over the layer stages (every linear but the first and the head): a stage "
                f"{m['stage_us']:.2f} us end to end; detect {m['detect_us']:.2f}, spread {m['spread_us']:.2f}, "
                f"compute {m['compute_median_us']:.2f}, tail {m['tail_us']:.2f}. A unit waited "
                f"{stats['unit_wait_median_us']:.2f} us (median; p90 {stats['unit_wait_p90_us']:.2f}) from its "
                "start, weight loads issued, to its staged input."]
    for n_ in notes:
        out += ["", n_]
    return "\n".join(out) + "\n"


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--sq", help="a shader-counter pass (SQ_COUNTERS) instead of --fetch/--write")
    ap.add_argument("--mem", help="with --sq: a memory-unit pass (MEM_COUNTERS) of the same run")
    ap.add_argument("--manifest", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", action="append", default=[], help="a command line that produced the passes")
    ap.add_argument("--note", action="append", default=[], help="a paragraph to add under the table")
    a = ap.parse_args(argv)
    if a.sq:
        with open(a.manifest) as f:
            entries = json.load(f)["configs"]
        recs = sq_per_config(a.sq, entries)
        mem = sq_per_config(a.mem, entries, MEM_COUNTERS) if a.mem else None
        with open(a.out, "w") as f:
            f.write(render_sq(recs, a.command, a.note, mem))
        for r in recs:
            d = sq_derived(r)
            print(f"{r['label']:24s} {r['kernel']:34s} waves/SIMD {d['waves_per_simd']:.2f} "
                  f"VALU {d['valu_busy']:.2f} MFMA {d['mfma_busy']:.2f}")
        return
    if not (a.fetch and a.write):
        ap.error("--fetch and --write (or --sq) are required")
    recs, cal = summarize(a.fetch, a.write, a.manifest)
    with open(a.out, "w") as f:
        f.write(render(recs, cal, a.command, a.note))
    for r in recs:
        print(f"{r['label']:28s} {r['ratio_to_algorithmic']:.4f}")


if __name__ == "__main__":
    main()
