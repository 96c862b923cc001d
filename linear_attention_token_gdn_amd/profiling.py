"""Summaries of rocprofv3 output for the profiles/ directory.

    python -m linear_attention_token_gdn_amd.profiling trace  <kernel_trace.csv> "<command>"
    python -m linear_attention_token_gdn_amd.profiling traffic <fetch_dir> <write_dir> \
           <copy_fetch_dir> <copy_write_dir> "<command>" <prefill_workload_label> [segments]
    python -m linear_attention_token_gdn_amd.profiling mfma <label> <mfma_dir> <lds_dir> \
           <algorithmic_flops_per_call> "<command>" [segments]

`trace` prints a markdown table of per-kernel launch counts and durations (from a
`rocprofv3 --kernel-trace` CSV).  `traffic` turns two counter passes over the benchmark
(`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`) and the same two passes over a plain 1 GiB copy
into HBM bytes per launch: each counter is scaled by (known copy bytes / what the counter read
for the copy).  It prints markdown and writes profiles/traffic.json (the prefill kernels'
record labelled with the prefill workload, e.g. workload3; the decode kernel's with
workload4), which bench.py reports while the kernel sources and the workload are unchanged.
A split-plan prefill that runs in `segments` segments launches prep and scan that many times
per call; its record holds bytes per call (all their launches over the number of calls).  The
segmented plan's three kernels (transition pass, combine, single pass) launch once per call and
are recorded together under "segmented".  `mfma` reads one counter pass with
`--pmc MfmaUtil MfmaFlopsF16 MfmaFlopsBF16 SQ_INSTS_VALU_MFMA_MOPS_F32 GRBM_GUI_ACTIVE` and one with
`--pmc LdsBankConflict SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE` over a run of one prefill
workload, prints per-kernel matrix-core busy time, matrix-core flops as issued (which include
the redundant and selection products the kernels issue, so they exceed the algorithmic count)
and LDS bank conflicts, and records them under <label> in profiles/mfma.json.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = {
    # the split plan (prep + scan), the fused kernel and decode, each with the shared header
    "prefill": [os.path.join(ROOT, "linear_attention_token_gdn_amd", "csrc", n)
                for n in ("chunk_split.hip", "gdn_internal.h")],
    "fused": [os.path.join(ROOT, "linear_attention_token_gdn_amd", "csrc", n)
              for n in ("chunk_mfma.hip", "gdn_internal.h")],
    # the segmented plan: the fused kernel's file (transition pass, combine, single pass)
    "segmented": [os.path.join(ROOT, "linear_attention_token_gdn_amd", "csrc", n)
                  for n in ("chunk_mfma.hip", "gdn_internal.h")],
    "decode": [os.path.join(ROOT, "linear_attention_token_gdn_amd", "csrc", n)
               for n in ("decode.hip", "gdn_internal.h")],
}


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


_TARG = {"t": "bf16", "f": "float", "Lb0E": "false", "Lb1E": "true"}


def _unmangle(name: str) -> str:
    """`_ZN3gdn12_GLOBAL__N_1<len><name>I<args>E...` -> `name<args>` for the template
    arguments used here (integers, bools, bf16, float); other names unchanged."""
    import re
    m = re.match(r"_ZN3gdn12_GLOBAL__N_1(\d+)", name)
    if not m:
        return name
    i = m.end()
    n = int(m.group(1))
    base, rest = name[i:i + n], name[i + n:]
    if not rest.startswith("I"):
        return base
    args = re.findall(r"Li(\d+)E|(Lb[01]E)|([tf])(?=[^a-z]|$)", rest[1:rest.find("EE") + 1])
    out = [a or _TARG[b or c] for a, b, c in args]
    return "%s<%s>" % (base, ", ".join(out))


def short_name(name: str) -> str:
    """Kernel name without namespaces, return type and parameter list."""
    name = _unmangle(name)
    name = name.replace("(anonymous namespace)::", "").replace("void ", "", 1)
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):  # first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    return name[:cut].replace("gdn::", "").replace("unsigned short", "bf16").strip()


def read_trace(path):
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            rows.append((short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]),
                         (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    return rows


def _label(name, width=70):
    return name if len(name) <= width else name[:width] + "..."


def read_stats(path):
    """rocprofv3 --stats kernel summary: (name, calls, average us, min us, max us, share %)."""
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            rows.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return rows


def trace_table(path, command):
    groups = {}
    for name, grid, us in read_trace(path):
        groups.setdefault((name, grid), []).append(us)
    out = ["Command: `%s`" % command, "",
           "Per-launch durations from the kernel trace:", "",
           "| kernel | grid (threads) | launches | mean us | median us | min us |",
           "|---|---|---|---|---|---|"]
    for (name, grid), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        out.append("| `%s` | %d | %d | %.1f | %.1f | %.1f |" % (
            _label(name), grid, len(v), statistics.mean(v), statistics.median(v), min(v)))
    stats = glob.glob(os.path.join(os.path.dirname(path), "*kernel_stats.csv"))
    if stats:
        out += ["", "`--stats` summary (%s):" % os.path.basename(stats[0]), "",
                "| kernel | calls | average us | min us | max us | % of GPU time |",
                "|---|---|---|---|---|---|"]
        for name, calls, avg, mn, mx, pct in read_stats(stats[0]):
            out.append("| `%s` | %d | %.1f | %.1f | %.1f | %.2f |" % (_label(name), calls, avg, mn,
                                                                     mx, pct))
    return "\n".join(out)


def read_counter(dirpath, counter):
    """Per-dispatch counter values (KiB as rocprofv3 reports them) keyed by kernel name."""
    files = glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError("no counter_collection.csv under %s" % dirpath)
    per = {}
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            if r.get("Counter_Name") != counter:
                continue
            key = (short_name(r["Kernel_Name"]), r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    by_kernel = {}
    for (name, _), val in per.items():
        by_kernel.setdefault(name, []).append(val)
    return by_kernel


def traffic(fetch_dir, write_dir, cfetch_dir, cwrite_dir, command, workload, segments="1"):
    segments = int(segments)
    fetch, write = read_counter(fetch_dir, "FETCH_SIZE"), read_counter(write_dir, "WRITE_SIZE")
    cf, cw = read_counter(cfetch_dir, "FETCH_SIZE"), read_counter(cwrite_dir, "WRITE_SIZE")
    copy_f = max(statistics.median(v) for v in cf.values())
    copy_w = max(statistics.median(v) for v in cw.values())
    ref = (1 << 30)
    sf, sw = ref / (copy_f * 1024.0), ref / (copy_w * 1024.0)
    out = ["Command: `%s`" % command, "",
           "Copy calibration (1 GiB read + 1 GiB written): FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB "
           "per launch -> scale %.4f / %.4f" % (copy_f, copy_w, sf, sw), "",
           "| kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB |",
           "|---|---|---|---|---|---|"]
    res = {}
    for name in sorted(set(fetch) | set(write)):
        if "gdn" not in name and "kernel" not in name:
            continue
        f = statistics.median(fetch.get(name, [0.0]))
        w = statistics.median(write.get(name, [0.0]))
        rd, wr = f * 1024 * sf, w * 1024 * sw
        res[name] = (rd, wr)
        out.append("| `%s` | %d | %.0f | %.0f | %.1f | %.1f |" % (
            _label(name), len(fetch.get(name, [])), f, w, rd / 1e6, wr / 1e6))
    rec = {"copy_scale_fetch": sf, "copy_scale_write": sw, "command": command}
    segmented = any(n.startswith("seg_combine_kernel") for n in res)
    for key, names, seg in (("prefill", ("prep_kernel", "scan_kernel"), segments),
                            ("segmented" if segmented else "fused",
                             ("chunk_kernel", "seg_combine_kernel"), 1)):
        pre = [n for n in res if n.startswith(names)]
        if pre:
            # per call: every launch of these kernels over the number of calls (the launches of
            # the last kernel of the call over the launches it makes per call)
            calls = len(fetch.get(pre[-1], [])) / seg
            rd = sum(sum(fetch.get(n, [])) for n in pre) * 1024 * sf / calls
            wr = sum(sum(write.get(n, [])) for n in pre) * 1024 * sw / calls
            rec[key] = {"kernels": pre, "bytes_per_call": rd + wr,
                        "read_bytes_per_call": rd, "write_bytes_per_call": wr,
                        "launches_per_call": {n: seg for n in pre},
                        "workload": workload, "source_sha256_16": source_hash(SOURCES[key])}
            out += ["", "%s per call (%d launch(es) of each kernel per call): %.1f MB read, "
                    "%.1f MB written" % (key, seg, rd / 1e6, wr / 1e6)]
    # the single-token decode kernel (MULTI = false) of the benchmark step
    dec = [n for n in res if n.startswith("decode_kernel") and n.endswith("false>")]
    if dec:
        rec["decode"] = {"kernels": dec, "bytes_per_launch": sum(sum(res[n]) for n in dec),
                         "workload": "workload4",
                         "source_sha256_16": source_hash(SOURCES["decode"])}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    return "\n".join(out)


PREFILL_KERNELS = ("prep_kernel", "scan_kernel", "chunk_kernel", "seg_combine_kernel")


def mfma(label, mfma_dir, lds_dir, algo_flops, command, segments="1"):
    """Matrix-core and LDS counters per kernel (medians over its launches); the prefill call's
    totals sum every launch of its kernels over the number of calls (`segments` launches of
    each kernel per call for a split-plan prefill in segments)."""
    algo_flops = float(algo_flops)
    segments = int(segments)
    med = lambda d, n: statistics.median(d[n]) if n in d else 0.0
    util = read_counter(mfma_dir, "MfmaUtil")
    f16, bf16 = read_counter(mfma_dir, "MfmaFlopsF16"), read_counter(mfma_dir, "MfmaFlopsBF16")
    f32 = read_counter(mfma_dir, "SQ_INSTS_VALU_MFMA_MOPS_F32")
    gui = read_counter(mfma_dir, "GRBM_GUI_ACTIVE")
    conf = read_counter(lds_dir, "LdsBankConflict")
    cyc = read_counter(lds_dir, "SQ_LDS_BANK_CONFLICT")
    act = read_counter(lds_dir, "SQ_LDS_IDX_ACTIVE")
    out = ["Command: `%s`" % command, "",
           "Counters per launch (medians over the launches of each kernel). Matrix-core busy is "
           "rocprofv3's MfmaUtil (busy cycles of the matrix cores over GPU-active cycles of all "
           "SIMDs); flops issued = 512 x the MFMA op counts; LDS conflicts per access is "
           "LdsBankConflict.", "",
           "| kernel | launches | MFMA busy % | MFMA flops issued (G) | of which f16 / bf16 / f32 (G) "
           "| LDS conflicts / access | LDS conflict cycles % of LDS active |",
           "|---|---|---|---|---|---|---|"]
    rec = {"command": command, "kernels": {}}
    pre = []
    for name in sorted(util, key=lambda n: -med(gui, n)):
        if name.startswith(("at::", "__amd", "Cijk")):  # torch, runtime and library kernels
            continue
        a, b, c = med(f16, name), med(bf16, name), 512.0 * med(f32, name)
        lds_pct = 100.0 * med(cyc, name) / med(act, name) if med(act, name) > 0 else 0.0
        out.append("| `%s` | %d | %.1f | %.3f | %.3f / %.3f / %.3f | %.4f | %.1f |" % (
            _label(name), len(util[name]), med(util, name), (a + b + c) / 1e9, a / 1e9, b / 1e9,
            c / 1e9, med(conf, name), lds_pct))
        rec["kernels"][name] = {"mfma_busy_pct": med(util, name), "mfma_flops_issued": a + b + c,
                                "gui_active": med(gui, name), "lds_conflicts_per_access":
                                med(conf, name), "lds_conflict_cycles_pct": lds_pct}
        if name.startswith(PREFILL_KERNELS):
            pre.append(name)
    if pre:
        calls = len(util[pre[-1]]) / (segments if not pre[-1].startswith("chunk_kernel") else 1)
        issued = sum(sum(f16.get(n, [])) + sum(bf16.get(n, [])) + 512.0 * sum(f32.get(n, []))
                     for n in pre) / calls
        w = sum(sum(gui.get(n, [])) for n in pre)
        busy = sum(u * g for n in pre for u, g in zip(util.get(n, []), gui.get(n, []))) / w \
            if w > 0 else 0.0
        rec["prefill"] = {"kernels": pre, "mfma_flops_issued_per_call": issued,
                          "algorithmic_flops_per_call": algo_flops,
                          "issued_over_algorithmic": issued / algo_flops,
                          "mfma_busy_pct_weighted": busy,
                          "source_sha256_16": source_hash(
                              SOURCES["fused" if any(n.startswith("chunk_kernel") for n in pre)
                                      else "prefill"])}
        out += ["", "Prefill call (%s): %.3f G MFMA flops issued against %.3f G algorithmic "
                "(x%.2f); matrix cores busy %.1f%% of the call's GPU-active time (kernels "
                "weighted by their active cycles)." % (", ".join("`%s`" % n for n in pre),
                                                        issued / 1e9, algo_flops / 1e9,
                                                        issued / algo_flops, busy)]
    path = os.path.join(ROOT, "profiles", "mfma.json")
    allrec = {}
    if os.path.exists(path):
        with open(path) as fh:
            allrec = json.load(fh)
    allrec[label] = rec
    with open(path, "w") as fh:
        json.dump(allrec, fh, indent=1)
    return "\n".join(out)


def main(argv):
    if argv and argv[0] == "trace":
        print(trace_table(argv[1], argv[2]))
    elif argv and argv[0] == "traffic":
        print(traffic(*argv[1:8]))
    elif argv and argv[0] == "mfma":
        print(mfma(*argv[1:8]))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
