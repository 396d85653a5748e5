"""Short text summaries of rocprofv3 CSV output (kernel traces and counter runs).

    python -m sparse_moe_layer_logits_amd.rocprof_summary kt DIR [--top N]
        per (kernel, grid size) group: calls, average / min / max duration

    python -m sparse_moe_layer_logits_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR \\
            --group SUBSTR@GRID [--group ...] --probe-mib M --source-sha SHA [--stage S] --out FILE.json
        HBM bytes per launch of a stage (the sum over its kernel groups, one
        launch each) from a FETCH_SIZE run and a WRITE_SIZE run.  Each counter is scaled by what it reads for the plain
        copy launches of the same run (bench.py --copy-probe-mib M: M MiB read
        and M MiB written per launch).

    python -m sparse_moe_layer_logits_amd.rocprof_summary mfma PMC_DIR --group SUBSTR@GRID [...] \\
            --alg-flops F --source-sha SHA --out FILE.json
        MFMA work of a stage (its kernel groups, one launch each) from a run with
        SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE:
        executed flops (512 per MOPS unit) against the stage's algorithmic flops,
        and MFMA-busy cycles against the SIMD cycles of the launches' duration
        (GRBM_GUI_ACTIVE counts every XCC; SIMD and XCC counts come from the run's
        agent information).

DIR is the rocprofv3 output directory (-d) of a run with --output-format csv.
"""
import argparse
import collections
import csv
import glob
import json
import os
import sys


def _one(dir_, pattern):
    files = sorted(glob.glob(os.path.join(dir_, "**", pattern), recursive=True))
    if not files:
        raise SystemExit("no %s under %s" % (pattern, dir_))
    return files[0]


def kernel_groups(dir_):
    """(kernel name, grid size) -> list of durations in ns, from *kernel_trace.csv."""
    groups = collections.defaultdict(list)
    for r in csv.DictReader(open(_one(dir_, "*kernel_trace.csv"))):
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        groups[(r["Kernel_Name"], grid)].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return groups


def cmd_kt(a):
    groups = kernel_groups(a.dir)
    total = sum(sum(v) for v in groups.values())
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))[: a.top]
    print("| kernel | grid (threads) | calls | avg us | min us | max us | % time |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for (name, grid), v in rows:
        print("| `%s` | %d | %d | %.1f | %.1f | %.1f | %.1f |" % (
            name[:90], grid, len(v), sum(v) / len(v) / 1e3, min(v) / 1e3, max(v) / 1e3,
            100.0 * sum(v) / total))


def counter_per_dispatch(dir_, counter):
    """(kernel name, grid size) -> list of per-dispatch values of one counter."""
    out = collections.defaultdict(list)
    for r in csv.DictReader(open(_one(dir_, "*counter_collection.csv"))):
        if r["Counter_Name"] == counter:
            out[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return out


def _pick(groups, kernel, grid):
    hits = [(k, v) for k, v in groups.items() if kernel in k[0] and (grid is None or k[1] == grid)]
    if len(hits) != 1:
        raise SystemExit("kernel %r grid %s matches %d groups: %s" % (
            kernel, grid, len(hits), [k for k, _ in hits][:8]))
    return hits[0]


def cmd_traffic(a):
    probe_bytes = a.probe_mib * (1 << 20)
    groups_spec = [(g.rsplit("@", 1)[0], int(g.rsplit("@", 1)[1])) for g in a.group]
    res = {"groups": []}
    for counter, dir_ in (("FETCH_SIZE", a.fetch_dir), ("WRITE_SIZE", a.write_dir)):
        groups = counter_per_dispatch(dir_, counter)
        # the copy probe: elementwise launches that move about probe_bytes each
        probe = [v for (k, g), vs in groups.items() if "elementwise" in k
                 for v in vs if probe_bytes / 4 < v * 1024 < probe_bytes * 4]
        if not probe:
            raise SystemExit("no copy-probe launches in %s" % dir_)
        probe_kib = sorted(probe)[len(probe) // 2]
        factor = probe_bytes / (probe_kib * 1024)
        kib, launches, names = 0.0, [], []
        for kernel, grid in groups_spec:
            (name, g), vals = _pick(groups, kernel, grid)
            kib += sum(vals) / len(vals)
            launches.append(len(vals))
            names.append("%s @%d" % (name, g))
        res[counter] = {"kib_per_launch": kib, "launches": launches, "probe_kib": probe_kib,
                        "factor": factor, "bytes_per_launch": kib * 1024 * factor}
        res["groups"] = names
    res["hbm_bytes_per_launch"] = int(res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"])
    res["source_sha"] = a.source_sha
    if a.stage:
        res["stage"] = a.stage
    res["command"] = a.command
    json.dump(res, open(a.out, "w"), indent=1)
    print(json.dumps(res, indent=1))


def gpu_agent(dir_):
    for r in csv.DictReader(open(_one(dir_, "*agent_info.csv"))):
        if int(r.get("Simd_Count") or 0) > 0:
            return r
    raise SystemExit("no GPU agent in %s" % dir_)


def cmd_mfma(a):
    agent = gpu_agent(a.dir)
    simds, xcc = int(agent["Simd_Count"]), int(agent["Num_Xcc"])
    max_ghz = int(agent["Max_Engine_Clk_Fcompute"]) / 1e3
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    n = collections.Counter()
    dur = collections.defaultdict(float)
    seen = set()
    for r in csv.DictReader(open(_one(a.dir, "*counter_collection.csv"))):
        key = (r["Kernel_Name"], int(r["Grid_Size"]))
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
        if (r["Dispatch_Id"], key) not in seen:
            seen.add((r["Dispatch_Id"], key))
            n[key] += 1
            dur[key] += (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    mops = busy = cycles = seconds = 0.0
    names = []
    for kernel, grid in [(g.rsplit("@", 1)[0], int(g.rsplit("@", 1)[1])) for g in a.group]:
        (name, g), v = _pick(per, kernel, grid)
        c = n[(name, g)]
        mops += v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] / c
        busy += v["SQ_VALU_MFMA_BUSY_CYCLES"] / c
        cycles += v["GRBM_GUI_ACTIVE"] / c / xcc
        seconds += dur[(name, g)] / c
        names.append("%s @%d (%d launches)" % (name, g, c))
    executed = mops * 512
    res = {
        "groups": names,
        "executed_tflop_per_launch": executed / 1e12,
        "algorithmic_tflop_per_launch": a.alg_flops / 1e12,
        "executed_over_algorithmic": executed / a.alg_flops,
        "mfma_busy_frac": busy / (simds * cycles),
        "launch_ms": seconds * 1e3,
        "clock_ghz": cycles / seconds / 1e9,
        "executed_tflops": executed / seconds / 1e12,
        "algorithmic_tflops": a.alg_flops / seconds / 1e12,
        "peak_at_max_clock_tflops": simds * 1024 * max_ghz / 1e3,
        "source_sha": a.source_sha,
        "command": a.command,
    }
    json.dump(res, open(a.out, "w"), indent=1)
    print(json.dumps(res, indent=1))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kt")
    k.add_argument("dir")
    k.add_argument("--top", type=int, default=20)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--group", action="append", required=True,
                   help="kernel name substring @ grid size (threads); repeat for a stage of several launches")
    t.add_argument("--probe-mib", type=int, required=True)
    t.add_argument("--source-sha", required=True)
    t.add_argument("--stage", default="", help="the layer stage the groups make up (e.g. expert_up)")
    t.add_argument("--command", default="")
    t.add_argument("--out", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("--group", action="append", required=True,
                   help="kernel name substring @ grid size (threads); repeat for a stage of several launches")
    m.add_argument("--alg-flops", type=float, required=True, help="algorithmic flops of one launch of the stage")
    m.add_argument("--source-sha", required=True)
    m.add_argument("--command", default="")
    m.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    {"kt": cmd_kt, "traffic": cmd_traffic, "mfma": cmd_mfma}[a.cmd](a)


if __name__ == "__main__":
    main()
