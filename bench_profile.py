"""Summaries of rocprofv3 runs of bench.py, for profiles/.

    python bench_profile.py --workload NAME --trace DIR --fetch DIR --write DIR [--copy-mib 1024]
                            [--bench-json FILE] [--commands FILE]

DIR: the -d directory of one rocprofv3 run with --output-format csv:
  --trace  a --kernel-trace run of bench.py for one workload,
  --fetch  a --pmc FETCH_SIZE run, --write a --pmc WRITE_SIZE run of the same
           bench.py command with --copy-calib-mib (the known-size copy that
           scales the counters to bytes).
Writes profiles/moe_layer_fwd__NAME.md (kernel times, one cold expert-FFN
call, HBM bytes per dispatch) and profiles/traffic__expert_ffn__NAME.json
(the HBM bytes of one expert-FFN call, which bench.py reports as the
roofline's `traffic` while the FFN kernels' sources are unchanged).

    python bench_profile.py counters --workload NAME --runs DIR [DIR ...] [--commands FILE]

writes profiles/mfma_counters__expert_ffn__NAME.md from --pmc runs (CSV) of
bench.py restricted to the FFN kernels: per kernel (name and grid), the
averages per dispatch of the clock, MFMA busy, MFMA FLOP rate, wave wait,
LDS bank conflicts, L2 hit rate and HBM bytes, from whichever of these
counters the runs hold: SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16,
SQ_WAIT_INST_ANY, SQ_WAVE_CYCLES, SQ_LDS_BANK_CONFLICT, GRBM_GUI_ACTIVE,
TCC_HIT_sum, TCC_MISS_sum, FETCH_SIZE, WRITE_SIZE.

    python bench_profile.py backward --workload NAME --trace DIR [--bench-json FILE] [--commands FILE]

writes profiles/moe_layer_bwd__NAME.md from a --kernel-trace run of bench.py
with its backward timing: the launches of one moe_layer_bwd call (each call
starts at its gate-gradient zeroing kernel, zero_f32_kernel; one-head
layers), averaged over the traced calls, in launch order.

An expert-FFN call is the run of dispatches that starts at its tile-prefix
kernel (gemm_prep_kernel or mlp_prefix_kernel) and holds only FFN kernels
(grouped_gemm_kernel, mlp_kernel); it is cold when the dispatch before it is
the reduction that ends bench.py's 1 GiB cache eviction.
"""
import argparse
import csv
import glob
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))

FFN = ("grouped_gemm_kernel", "mlp_kernel")
PREP = ("gemm_prep_kernel", "mlp_prefix_kernel")


def short(name):
    n = re.sub(r"^void ", "", name.strip())
    n = re.sub(r"^moe::", "", n)
    n = re.sub(r"<(.*)>\(.*\)$", lambda m: "<" + m.group(1).replace("moe::", "") + ">", n)
    n = re.sub(r"\(.*\)$", "", n)
    return n


def is_ffn(n):
    return any(n.startswith(k) for k in FFN)


def is_prep(n):
    return any(n.startswith(k) for k in PREP)


def _col(row, *names):
    low = {k.lower(): k for k in row}
    for n in names:
        if n.lower() in low:
            return row[low[n.lower()]]
    raise KeyError(names)


def _grid(row):
    try:
        return int(_col(row, "Grid_Size"))
    except KeyError:
        g = 1
        for a in ("X", "Y", "Z"):
            g *= int(_col(row, "Grid_Size_" + a))
        return g


def _one(d, pattern):
    fs = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not fs:
        sys.exit(f"no {pattern} under {d}")
    return fs[0]


def load_trace(d):
    """Dispatches of a kernel-trace run, in start order: (name, grid, start_ns, end_ns)."""
    with open(_one(d, "*kernel_trace.csv")) as f:
        rows = [(short(_col(r, "Kernel_Name")), _grid(r), int(_col(r, "Start_Timestamp")),
                 int(_col(r, "End_Timestamp"))) for r in csv.DictReader(f)]
    return sorted(rows, key=lambda r: r[2])


def load_counter(d, counter):
    """Dispatches of a counter run, in dispatch order: (name, grid, value)."""
    acc = {}
    with open(_one(d, "*counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if _col(r, "Counter_Name") != counter:
                continue
            i = int(_col(r, "Dispatch_Id"))
            name, grid = short(_col(r, "Kernel_Name")), _grid(r)
            v = float(_col(r, "Counter_Value"))
            if i in acc:
                acc[i][2] += v
            else:
                acc[i] = [name, grid, v]
    return [tuple(acc[i]) for i in sorted(acc)]


def cold_calls(names):
    """Index ranges [b, e) of the cold expert-FFN calls in a dispatch sequence."""
    out = []
    i = 0
    while i < len(names):
        if is_prep(names[i]):
            j = i + 1
            while j < len(names) and is_ffn(names[j]):
                j += 1
            if j > i + 1 and i > 0 and names[i - 1].startswith("at::native::reduce_kernel"):
                out.append((i, j))
            i = j
        else:
            i += 1
    return out


def per_kernel(rows, calls, val):
    """Mean over the calls of each position's value, keyed (position, name, grid)."""
    n = len(calls)
    shape = [(rows[k][0], rows[k][1]) for k in range(*calls[0])]
    for b, e in calls:
        if [(rows[k][0], rows[k][1]) for k in range(b, e)] != shape:
            sys.exit("the cold expert-FFN calls launch different kernels")
    return [(nm, g, sum(val(rows[b + p]) for b, _ in calls) / n) for p, (nm, g) in enumerate(shape)]


def calib(rows, mib):
    cp = [r for r in rows if "copyBuffer" in r[0] or "copy" in r[0].lower()]
    if not cp:
        sys.exit("no copy kernel in the counter run (bench.py --copy-calib-mib)")
    kib = max(cp, key=lambda r: r[2])[2]
    return mib * 1024.0 / kib, kib


def load_all_counters(d):
    """Every counter of a counter run, per dispatch: {dispatch: (name, grid, dur_ns, {counter: value})}."""
    out = {}
    with open(_one(d, "*counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            i = int(_col(r, "Dispatch_Id"))
            if i not in out:
                dur = int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))
                out[i] = (short(_col(r, "Kernel_Name")), _grid(r), dur, {})
            c = _col(r, "Counter_Name")
            out[i][3][c] = out[i][3].get(c, 0.0) + float(_col(r, "Counter_Value"))
    return out


def counters_main(argv):
    ap = argparse.ArgumentParser(prog="bench_profile.py counters")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--runs", nargs="+", required=True)
    ap.add_argument("--commands", default="")
    a = ap.parse_args(argv)
    agg = {}  # (name, grid) -> counter -> [values]; "_dur" -> durations
    order = []
    for d in a.runs:
        for _, (name, grid, dur, cs) in sorted(load_all_counters(d).items()):
            if not is_ffn(name):
                continue
            k = (name, grid)
            if k not in agg:
                agg[k] = {}
                order.append(k)
            for c, v in cs.items():
                agg[k].setdefault(c, []).append(v)
            if "GRBM_GUI_ACTIVE" in cs:
                agg[k].setdefault("_dur", []).append(dur)
    mean = lambda k, c: (sum(agg[k][c]) / len(agg[k][c])) if agg[k].get(c) else None
    lines = [f"# rocprofv3 counters: expert-FFN kernels, {a.workload}", "",
             "Commands (from the repository root on one MI355X, after `cd /tmp && export TMPDIR=/tmp`; one counter "
             "set per run):", ""]
    if a.commands:
        lines += ["    " + c.strip() for c in open(a.commands) if c.strip()]
    lines += ["    python bench_profile.py counters --workload " + a.workload + " --runs " + " ".join(a.runs), "",
              "Averages per dispatch over every traced call of each kernel (warm-up, timed steps and the stage "
              "timing; kernels serialised by the counter collection).  `GRBM_GUI_ACTIVE` is summed over the 8 XCDs, "
              "so the clock is GUI / 8 / duration; MFMA busy = `SQ_VALU_MFMA_BUSY_CYCLES` / (GUI / 8 x 1024 SIMDs); "
              "`SQ_INSTS_VALU_MFMA_MOPS_BF16` x 512 = the MFMA FLOPs; L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS); HBM "
              "bytes: FETCH_SIZE x 2 (see the forward summary's copy calibration) and WRITE_SIZE x 1, in GB.", "",
              "| kernel | grid | calls | avg us (counter run) | clock GHz | MFMA busy | MFMA TFLOP/s | wait "
              "(SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES) | LDS bank conflict cycles | L2 hit | read GB | write GB |",
              "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    f1 = lambda v, fmt: (fmt % v) if v is not None else "-"
    for k in order:
        n, g = k
        dur = mean(k, "_dur")
        gui = mean(k, "GRBM_GUI_ACTIVE")
        clk = gui / 8 / dur if gui and dur else None
        busy = mean(k, "SQ_VALU_MFMA_BUSY_CYCLES")
        mb = busy / (gui / 8 * 1024) if busy is not None and gui else None
        mops = mean(k, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        tf = mops * 512 / dur / 1e3 if mops is not None and dur else None
        wt, wc = mean(k, "SQ_WAIT_INST_ANY"), mean(k, "SQ_WAVE_CYCLES")
        hit, miss = mean(k, "TCC_HIT_sum"), mean(k, "TCC_MISS_sum")
        fe, wr = mean(k, "FETCH_SIZE"), mean(k, "WRITE_SIZE")
        calls = max(len(v) for c, v in agg[k].items())
        lines.append(f"| `{n}` | {g} | {calls} | {f1(dur / 1e3 if dur else None, '%.1f')} | {f1(clk, '%.2f')} | "
                     f"{f1(100 * mb if mb is not None else None, '%.1f %%')} | {f1(tf, '%.0f')} | "
                     f"{f1(100 * wt / wc if wt is not None and wc else None, '%.0f %%')} | "
                     f"{f1(mean(k, 'SQ_LDS_BANK_CONFLICT'), '%.0f')} | "
                     f"{f1(100 * hit / (hit + miss) if hit is not None and miss is not None and hit + miss > 0 else None, '%.0f %%')} | "
                     f"{f1(fe * 2 * 1024 / 1e9 if fe is not None else None, '%.3f')} | "
                     f"{f1(wr * 1024 / 1e9 if wr is not None else None, '%.3f')} |")
    lines.append("")
    with open(os.path.join(ROOT, "profiles", f"mfma_counters__expert_ffn__{a.workload}.md"), "w") as f:
        f.write("\n".join(lines))
    print(f"{a.workload}: {len(order)} FFN kernels")


def backward_main(argv):
    ap = argparse.ArgumentParser(prog="bench_profile.py backward")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--bench-json", default="")
    ap.add_argument("--commands", default="")
    a = ap.parse_args(argv)
    tr = load_trace(a.trace)
    starts = [i for i, r in enumerate(tr) if r[0].startswith("zero_f32_kernel")]
    if not starts:
        sys.exit("no backward call in the trace")
    calls = []
    for j, b in enumerate(starts):
        e = starts[j + 1] if j + 1 < len(starts) else len(tr)
        while e > b and (tr[e - 1][0].startswith("at::native") or tr[e - 1][0].startswith("__amd")):
            e -= 1
        calls.append((b, e))
    # the backward calls are the ones with the most common launch sequence (the warm-up and timed calls)
    shapes = {}
    for b, e in calls:
        shapes.setdefault(tuple((tr[k][0], tr[k][1]) for k in range(b, e)), []).append((b, e))
    shape, cs = max(shapes.items(), key=lambda kv: len(kv[1]))
    n = len(cs)
    avg = [sum((tr[b + p][3] - tr[b + p][2]) / 1e3 for b, _ in cs) / n for p in range(len(shape))]
    span = sum((tr[e - 1][3] - tr[b][2]) / 1e3 for b, e in cs) / n
    lines = [f"# rocprofv3 summary: MoE layer backward (moe_layer_bwd), {a.workload}", "",
             "Commands (from the repository root on one MI355X, after `cd /tmp && export TMPDIR=/tmp`):", ""]
    if a.commands:
        lines += ["    " + c.strip() for c in open(a.commands) if c.strip()]
    lines += ["    python bench_profile.py backward --workload " + a.workload + " --trace " + a.trace +
              (f" --bench-json {a.bench_json}" if a.bench_json else ""), "",
              f"{n} backward calls traced (warm-up + timed). Kernel durations below are averages over the calls,",
              "in launch order; the span is first launch start to last launch end.", "",
              "| # | kernel | grid (threads) | avg us |", "|---:|---|---:|---:|"]
    lines += [f"| {p} | `{nm}` | {g} | {v:.1f} |" for p, ((nm, g), v) in enumerate(zip(shape, avg))]
    bw = ""
    if a.bench_json:
        with open(a.bench_json) as f:
            d = json.loads([l for l in f.read().splitlines() if l.strip().startswith("{")][-1])
        b = d.get("backward") or {}
        if b:
            bw = (f"; bench.py's HIP-event figure for the same calls: {b['ms_per_step'] * 1e3:.1f} us per call"
                  + (" (pre-activations kept by the forward)" if b.get("kept_preactivations") else ""))
    lines += ["", f"Span of one call: {span:.1f} us{bw}.", ""]
    with open(os.path.join(ROOT, "profiles", f"moe_layer_bwd__{a.workload}.md"), "w") as f:
        f.write("\n".join(lines))
    print(f"{a.workload}: backward span {span:.1f} us over {n} calls")


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        return counters_main(sys.argv[2:])
    if len(sys.argv) > 1 and sys.argv[1] == "backward":
        return backward_main(sys.argv[2:])
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--bench-json", default="", help="bench.py's JSON line of the trace run")
    ap.add_argument("--commands", default="", help="file with the rocprofv3 command lines, one per line")
    a = ap.parse_args()
    sys.path.insert(0, ROOT)
    from bench import ffn_source_sha256

    tr = load_trace(a.trace)
    fe = load_counter(a.fetch, "FETCH_SIZE")
    wr = load_counter(a.write, "WRITE_SIZE")
    fr, fk = calib(fe, a.copy_mib)
    wf, wk = calib(wr, a.copy_mib)

    # kernel time over the whole trace run
    tot = {}
    for n, g, s, e in tr:
        tot.setdefault((n, g), []).append((e - s) / 1e3)
    alltime = sum(sum(v) for v in tot.values())
    lines = [f"# rocprofv3 summary: MoE layer forward, {a.workload}", ""]
    lines += ["Commands (from the repository root on one MI355X, after `cd /tmp && export TMPDIR=/tmp`; "
              "paths as seen from the root):", ""]
    if a.commands:
        lines += ["    " + c.strip() for c in open(a.commands) if c.strip()]
    lines += ["    " + "python bench_profile.py --workload " + a.workload + f" --trace {a.trace} --fetch {a.fetch} "
              f"--write {a.write} --copy-mib {a.copy_mib}" + (f" --bench-json {a.bench_json}" if a.bench_json else ""),
              ""]
    lines += ["## Kernel time (kernel trace: warm-up and timed layer steps, plus the per-stage timing calls)", "",
              "| kernel | grid (threads) | calls | avg us | share |", "|---|---:|---:|---:|---:|"]
    for (n, g), v in sorted(tot.items(), key=lambda kv: -sum(kv[1]))[:16]:
        if n.startswith("at::native") or n.startswith("__amd"):
            continue
        lines.append(f"| `{n}` | {g} | {len(v)} | {sum(v) / len(v):.1f} | {100 * sum(v) / alltime:.1f} % |")

    names = [r[0] for r in tr]
    cc = cold_calls(names)
    if not cc:
        sys.exit("no cold expert-FFN call found in the trace")
    tk = per_kernel(tr, cc, lambda r: (r[3] - r[2]) / 1e3)
    span = sum((tr[e - 1][3] - tr[b + 1][2]) / 1e3 for b, e in cc) / len(cc)
    lines += ["", f"## One expert-FFN call ({len(cc)} cold calls of the stage timing, each after the 1 GiB eviction)",
              "", "| kernel | grid | avg us |", "|---|---:|---:|"]
    lines += [f"| `{n}` | {g} | {v:.1f} |" for n, g, v in tk]
    bench_us = None
    if a.bench_json:
        with open(a.bench_json) as f:
            d = json.loads([l for l in f.read().splitlines() if l.strip().startswith("{")][-1])
        bench_us = d["stages"]["expert_ffn"]["us"]
    lines += ["", f"Span of one call in the trace (first FFN kernel start to last FFN kernel end), averaged: "
              f"{span:.1f} us" + (f"; bench.py's HIP-event figure for the cold calls in this run: {bench_us:.1f} us"
                                  f" (its mean covers all its cold calls)." if bench_us else ".")]

    fc = cold_calls([r[0] for r in fe])
    wc = cold_calls([r[0] for r in wr])
    if not fc or not wc:
        sys.exit("no cold expert-FFN call found in a counter run")
    fk_ = per_kernel(fe, fc, lambda r: r[2])
    wk_ = per_kernel(wr, wc, lambda r: r[2])
    lines += ["", "## HBM bytes per dispatch (FETCH_SIZE, WRITE_SIZE)", "",
              f"Calibration: a {a.copy_mib} MiB device-to-device copy reads FETCH_SIZE = {fk:.0f} KiB and "
              f"WRITE_SIZE = {wk:.0f} KiB, so reads are scaled by {fr:.3f} and writes by {wf:.3f}.", "",
              f"Expert-FFN call ({len(fc)} / {len(wc)} cold calls in the two counter runs):", "",
              "| kernel | grid | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB | write GB |",
              "|---|---:|---:|---:|---:|---:|"]
    rd = wt = 0.0
    for (n, g, fv), (_, _, wv) in zip(fk_, wk_):
        rb, wb = fv * 1024 * fr, wv * 1024 * wf
        rd += rb
        wt += wb
        lines.append(f"| `{n}` | {g} | {fv:.0f} | {wv:.0f} | {rb / 1e9:.3f} | {wb / 1e9:.3f} |")
    lines += ["", f"Per expert-FFN call: {rd / 1e9:.3f} GB read + {wt / 1e9:.3f} GB written = {(rd + wt) / 1e9:.3f} GB.",
              ""]
    with open(os.path.join(ROOT, "profiles", f"moe_layer_fwd__{a.workload}.md"), "w") as f:
        f.write("\n".join(lines))
    rec = {"what": f"HBM bytes per expert-FFN call (its grouped_gemm_kernel / mlp_kernel launches), from rocprofv3 "
                   f"FETCH_SIZE (x{fr:.3f}) and WRITE_SIZE (x{wf:.3f}) per dispatch, scaled by a "
                   f"{a.copy_mib} MiB device copy",
           "workload": a.workload, "ffn_source_sha256": ffn_source_sha256(),
           "read_bytes": rd, "write_bytes": wt, "traffic_bytes": rd + wt, "calls": [len(fc), len(wc)]}
    with open(os.path.join(ROOT, "profiles", f"traffic__expert_ffn__{a.workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(f"{a.workload}: FFN span {span:.1f} us, {(rd + wt) / 1e9:.3f} GB per call")


if __name__ == "__main__":
    main()
