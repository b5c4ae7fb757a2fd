"""Summaries of rocprofv3 output for the pmoe kernels (short text files).

    python -m precision_moe_amd.profiling stats <rocprofv3 csv dir> <workload> <out.txt> "<command>"
        [<kernel> <n>]
        per-kernel call count and average / total duration from a
        `rocprofv3 --kernel-trace --stats --output-format csv` run; with a
        kernel name and n, also the average of that kernel's first n dispatches
    python -m precision_moe_amd.profiling traffic <fetch dir> <write dir> <copy fetch dir>
        <copy write dir> <copy bytes> <kernel substring> <workload> <out.txt> "<commands>"
        [<launches per step>]
        HBM bytes per dispatch of one kernel from `--pmc FETCH_SIZE` and
        `--pmc WRITE_SIZE` runs, each scaled by what the same counter reads for
        a plain device copy of known size, and per step (launches per step x
        the mean per dispatch)
    python -m precision_moe_amd.profiling table <trace dir> <fetch dir> <write dir> <copy fetch dir>
        <copy write dir> <copy bytes> <mfma counter dir> <workload> <out.txt> "<commands>"
        every pmoe kernel: HBM bytes and GB/s, MFMA instructions and busy fraction

    python -m precision_moe_amd.profiling spans <rocprofv3 csv dir> <workload> <out.txt>
        "<command>" <kernel> <first pair> <pairs>
        in-step span of a grouped GEMM run as two half launches on two streams:
        its dispatches by start time, taken two at a time (the two parts of one
        step), each pair from the first start to the last end; the mean over all
        pairs and over pairs [first, first + pairs)

The traffic summary records a hash of the GEMM sources it was measured with
(comments and whitespace excluded); bench.py reports the figure only while the
sources still match.
"""
import csv
import glob
import hashlib
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCES = [os.path.join(PKG, "csrc", n) for n in ("gemm.hip", "device.h", "kernels.h")]


# FLOPs of one v_mfma_f32_16x16x32_f16 / _bf16 wave instruction (the grouped GEMMs' only MFMA)
MFMA_FLOPS = 2 * 16 * 16 * 32


def _code_only(text):
    """C++ source without comments and with whitespace collapsed: edits to
    comments or layout do not change the kernel, so they do not change the hash."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def gemm_source_hash():
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(p) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _rows(directory, pattern):
    out = []
    for f in sorted(glob.glob(os.path.join(directory, "**", pattern), recursive=True)):
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    return out


def _col(row, *names):
    low = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    raise KeyError(names)


def _short(name):
    """Kernel name without its trailing parameter list (template arguments kept)."""
    name = name.strip()
    if name.endswith(")"):
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                name = name[:i]
                break
    return name.replace("void ", "").strip()


def kernel_stats(directory):
    """{kernel: (calls, avg_us, total_us)} from *kernel_stats.csv."""
    res = {}
    for r in _rows(directory, "*kernel_stats.csv"):
        name = _col(r, "Name", "KernelName", "Kernel_Name")
        calls = int(float(_col(r, "Calls")))
        total = float(_col(r, "TotalDurationNs", "Total_Duration_Ns")) / 1e3
        res[_short(name)] = (calls, total / max(calls, 1), total)
    return res


def counter_means(directory, counter):
    """{kernel: mean counter value per dispatch} from *counter_collection.csv."""
    acc = {}
    for r in _rows(directory, "*counter_collection.csv"):
        if _col(r, "Counter_Name") != counter:
            continue
        k = _short(_col(r, "Kernel_Name"))
        acc.setdefault(k, []).append(float(_col(r, "Counter_Value")))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def write_stats(directory, workload, out, command, first=None):
    st = kernel_stats(directory)
    lines = [f"# rocprofv3 kernel trace, workload {workload}", f"# command: {command}",
             "# kernel | calls | avg us | total us"]
    pm = {k: v for k, v in st.items() if "pmoe" in k}
    for k, (c, a, t) in sorted(pm.items(), key=lambda kv: -kv[1][2]):
        lines.append(f"{k} | {c} | {a:.2f} | {t:.1f}")
    other = [v for k, v in st.items() if "pmoe" not in k]
    lines.append(f"(other kernels: input generation and setup) | {sum(c for c, _, _ in other)} | - | "
                 f"{sum(t for _, _, t in other):.1f}")
    if first:
        kernel, n = first
        durs = first_dispatches(directory, kernel, n)
        lines.append(f"# {kernel}, its first {len(durs)} dispatches in launch order (bench.py's "
                     f"FC1 loop, timed there with HIP events): avg us "
                     f"{sum(durs) / max(len(durs), 1):.2f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def first_dispatches(directory, kernel, n):
    """Durations (us) of the first n dispatches of `kernel` (exact short name) by start time."""
    rows = [r for r in _rows(directory, "*kernel_trace.csv")
            if _short(_col(r, "Kernel_Name")) == kernel]
    rows.sort(key=lambda r: int(_col(r, "Start_Timestamp")))
    return [(int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) / 1e3 for r in rows[:n]]


def dispatch_times(directory, kernel):
    """(start, end) in ns of every dispatch of `kernel` (exact short name), by start time."""
    rows = [r for r in _rows(directory, "*kernel_trace.csv")
            if _short(_col(r, "Kernel_Name")) == kernel]
    t = [(int(_col(r, "Start_Timestamp")), int(_col(r, "End_Timestamp"))) for r in rows]
    return sorted(t)


def pair_spans(times):
    """Spans (us) of consecutive dispatch pairs: first start to last end of each pair."""
    return [(max(times[i][1], times[i + 1][1]) - min(times[i][0], times[i + 1][0])) / 1e3
            for i in range(0, len(times) - 1, 2)]


def write_spans(directory, workload, out, command, kernel, first, count):
    times = dispatch_times(directory, kernel)
    spans = pair_spans(times)
    own = [(e - b) / 1e3 for b, e in times]
    sel = spans[first:first + count]
    mean = lambda v: sum(v) / max(len(v), 1)
    lines = [f"# rocprofv3 kernel trace, workload {workload}: in-step span of {kernel}",
             f"# command: {command}",
             "# dispatches by start time, two per step (the two parts of the experts on two "
             "streams); span = first start to last end of a pair",
             f"kernel={kernel}",
             f"workload={workload}",
             f"dispatches={len(times)}",
             f"avg_dispatch_us={mean(own):.2f}",
             f"pairs={len(spans)}",
             f"avg_span_us_all_pairs={mean(spans):.2f}",
             f"pairs_selected={first}..{first + len(sel) - 1}",
             f"avg_span_us_selected={mean(sel):.2f}"]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_traffic(fetch_dir, write_dir, cf_dir, cw_dir, copy_bytes, kernel, workload, out, command,
                  launches=1):
    """HBM bytes of `kernel` per dispatch from the FETCH_SIZE / WRITE_SIZE runs, each
    scaled by what the counter reads for a plain device copy of copy_bytes; with
    launches > 1 (a kernel the step launches that many times, e.g. once per part of
    the experts) also the bytes per step: launches x the mean per dispatch."""
    def one(d, counter):
        vals = {k: v for k, v in counter_means(d, counter).items() if kernel in k}
        if len(vals) != 1:
            raise SystemExit(f"{counter}: expected one kernel matching {kernel!r}, got {list(vals)}")
        return next(iter(vals.items()))
    name, fetch = one(fetch_dir, "FETCH_SIZE")
    _, write = one(write_dir, "WRITE_SIZE")
    def copy_kernel(d, counter):
        vals = counter_means(d, counter)
        copies = [v for k, v in vals.items() if "copy" in k.lower()]
        return max(copies or vals.values())
    cf = copy_kernel(cf_dir, "FETCH_SIZE")
    cw = copy_kernel(cw_dir, "WRITE_SIZE")
    ff = copy_bytes / (cf * 1024.0)
    wf = copy_bytes / (cw * 1024.0)
    hbm = fetch * 1024 * ff + write * 1024 * wf
    lines = [
        f"# rocprofv3 HBM byte counters for {name}, workload {workload}",
        f"# commands: {command}",
        f"# calibration: a plain device copy of {copy_bytes} bytes reads FETCH_SIZE={cf:.1f} KiB "
        f"(factor {ff:.4f}) and WRITE_SIZE={cw:.1f} KiB (factor {wf:.4f})",
        f"kernel={name}",
        f"workload={workload}",
        f"source_sha256={gemm_source_hash()}",
        f"fetch_kib_per_dispatch={fetch:.1f}",
        f"write_kib_per_dispatch={write:.1f}",
        f"fetch_factor={ff:.6f}",
        f"write_factor={wf:.6f}",
        f"hbm_bytes_per_dispatch={hbm:.0f}",
        f"launches_per_step={launches}",
        f"hbm_bytes_per_step={hbm * launches:.0f}",
    ]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_table(kt_dir, fetch_dir, write_dir, cf_dir, cw_dir, copy_bytes, mfma_dir, workload, out,
                command):
    """Per pmoe kernel: HBM bytes and GB/s from the byte counters over the trace's
    average duration, and MFMA busy fraction from SQ_VALU_MFMA_BUSY_CYCLES."""
    st = kernel_stats(kt_dir)
    fetch = counter_means(fetch_dir, "FETCH_SIZE")
    write = counter_means(write_dir, "WRITE_SIZE")

    def copy_kernel(d, counter):
        vals = counter_means(d, counter)
        copies = [v for k, v in vals.items() if "copy" in k.lower()]
        return max(copies or vals.values())
    ff = copy_bytes / (copy_kernel(cf_dir, "FETCH_SIZE") * 1024.0)
    wf = copy_bytes / (copy_kernel(cw_dir, "WRITE_SIZE") * 1024.0)
    busy = counter_means(mfma_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    insts = counter_means(mfma_dir, "SQ_INSTS_MFMA")
    lines = [
        f"# rocprofv3 per-kernel HBM bytes and MFMA utilisation, workload {workload}",
        f"# commands: {command}",
        f"# HBM bytes = FETCH_SIZE x {ff:.4f} + WRITE_SIZE x {wf:.4f} (factors from a {copy_bytes}-byte "
        "device copy); GB/s over the kernel trace's average duration",
        "# MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (duration x 2.4 GHz x 1024 SIMDs): the share of the "
        "nominal MFMA issue capacity; MFMA TFLOP/s = SQ_INSTS_MFMA x 16384 (16x16x32) / duration, "
        "padded rows included",
        "# kernel | avg us | read MB | write MB | HBM GB/s | MFMA insts | MFMA busy | MFMA TFLOP/s",
    ]
    for k, (calls, avg, _) in sorted(st.items(), key=lambda kv: -kv[1][2]):
        if "pmoe" not in k or k not in fetch:
            continue
        rd = fetch[k] * 1024 * ff
        wr = write.get(k, 0.0) * 1024 * wf
        util = busy.get(k, 0.0) / (avg * 1e-6 * 2.4e9 * 1024)
        tf = insts.get(k, 0.0) * MFMA_FLOPS / (avg * 1e-6) / 1e12
        lines.append(f"{k} | {avg:.2f} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | {(rd + wr) / (avg * 1e3):.0f} | "
                     f"{insts.get(k, 0.0):.4g} | {util:.3f} | {tf:.0f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_traffic(path, workload):
    """HBM bytes per step (all of the kernel's launches in a step; per dispatch in
    summaries that give no step figure) from a traffic summary, or None if absent,
    for another workload, or measured with different GEMM sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k] = v
    if kv.get("workload") != workload or kv.get("source_sha256") != gemm_source_hash():
        return None
    return float(kv.get("hbm_bytes_per_step", kv["hbm_bytes_per_dispatch"]))


if __name__ == "__main__":
    cmd = sys.argv[1]
    if cmd == "stats":
        first = (sys.argv[6], int(sys.argv[7])) if len(sys.argv) > 7 else None
        write_stats(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], first)
    elif cmd == "traffic":
        write_traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], int(sys.argv[6]), sys.argv[7],
                      sys.argv[8], sys.argv[9], sys.argv[10], int(sys.argv[11]) if len(sys.argv) > 11 else 1)
    elif cmd == "spans":
        write_spans(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6], int(sys.argv[7]),
                    int(sys.argv[8]))
    elif cmd == "table":
        write_table(*sys.argv[2:7], int(sys.argv[7]), *sys.argv[8:12])
    else:
        raise SystemExit(__doc__)
