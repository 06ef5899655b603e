"""rocprofv3 harness: the commands that profile the benchmark on one MI355X and the summarisers
that turn their raw CSV output into the short text files under profiles/.

Nothing here runs a kernel.  The raw output (``*_kernel_trace.csv``, ``*_kernel_stats.csv``,
``*_counter_collection.csv``, ``*_agent_info.csv``) comes from ``rocprofv3`` runs of ``bench.py``
whose exact command lines are listed in ``RUNS``; ``python -m long_context_la_amd.profiling
commands ROOT`` prints them, and ``python -m long_context_la_amd.profiling summarize ROOT`` writes
every profile from what those runs left under ROOT.

Definitions used in the summaries:
  * HBM traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the factor that makes
    the same counter read the known byte count of a plain device copy (bench.py --copy-probe).
  * MFMA utilisation: SQ_VALU_MFMA_BUSY_CYCLES / (kernel cycles x SIMDs), kernel cycles =
    GRBM_GUI_ACTIVE / XCDs.
  * Peaks: compute units x maximum engine clock x 4096 bf16 flop per clock per CU (gfx950 dense
    MFMA), from the agent information (rocprofv3's agent table, else ``rocminfo``), else the
    datasheet constants; HBM 8 TB/s (datasheet).
"""
from __future__ import annotations

import csv
import hashlib
import os
import re
import statistics
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PREFILL_SOURCE = os.path.join(HERE, "csrc", "la_prefill_bf16.hip")
PROFILES = os.path.join(ROOT, "profiles")

PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, datasheet
BF16_FLOP_PER_CLK_PER_CU = 4096  # gfx950 dense bf16 MFMA
DATASHEET = {"cus": 256, "max_clock_mhz": 2400, "xcds": 8, "simds": 1024}


# ------------------------------------------------------------------ device and host description
def peaks_from(cus, max_clock_mhz, source):
    return {"cus": int(cus), "max_clock_mhz": float(max_clock_mhz),
            "bf16_tflops": cus * max_clock_mhz * 1e6 * BF16_FLOP_PER_CLK_PER_CU / 1e12,
            "hbm_gbs": PEAK_HBM_GBS, "source": source}


def agent_peaks(agent_csv):
    """Peaks from rocprofv3's agent table (first GPU agent)."""
    for r in read_csv(agent_csv):
        if r.get("Agent_Type") == "GPU":
            return peaks_from(int(r["Cu_Count"]), float(r["Max_Engine_Clk_Fcompute"]), "rocprofv3 agent info")
    raise ValueError(f"no GPU agent in {agent_csv}")


def parse_rocminfo(text):
    """(compute units, max clock MHz) of the first gfx GPU agent in ``rocminfo`` output."""
    for block in re.split(r"\n\*{5,}\s*\n", text):
        if not re.search(r"Name:\s+gfx\d", block):
            continue
        cu = re.search(r"Compute Unit:\s+(\d+)", block)
        clk = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", block)
        if cu and clk:
            return int(cu.group(1)), int(clk.group(1))
    return None


def device_peaks():
    """Peaks of the GPU on this machine from ``rocminfo``, else the datasheet constants."""
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
        got = parse_rocminfo(out)
        if got:
            return peaks_from(got[0], got[1], "rocminfo")
    except (OSError, subprocess.SubprocessError):
        pass
    return peaks_from(DATASHEET["cus"], DATASHEET["max_clock_mhz"], "datasheet constants")


def cpu_description():
    """Host CPU model and logical CPU count (for the CPU-baseline record)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count()}


def source_digest(path=PREFILL_SOURCE):
    """sha256[:16] of the kernel source's code: line comments, trailing blanks and empty lines are
    dropped first, so that editing a comment does not disown the profiles of unchanged code (the
    file holds no string literal with a double slash)."""
    lines = []
    with open(path, encoding="utf-8") as f:
        for line in f:
            cut = line.find("//")
            line = (line if cut < 0 else line[:cut]).rstrip()
            if line:
                lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


# ------------------------------------------------------------------ raw CSV access
def read_csv(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def short_name(name):
    """Kernel name without namespaces, argument lists and mangling noise."""
    n = name
    m = re.match(r"_ZN2la12_GLOBAL__N_1\d+(\w+?)I", n)
    if m:
        return m.group(1)
    n = re.sub(r"^void ", "", n)
    n = n.replace("la::(anonymous namespace)::", "")
    n = re.sub(r"\(la::FwdArgs\)$", "", n)
    n = re.sub(r"\((float|long|int|char|bool|unsigned|const|\*|,|\s)*\)$", "", n)
    if n.startswith("at::native::") or n.startswith("void at::native::"):
        return "torch elementwise (bench set-up)"
    return n


def dispatches(trace_csv):
    """Kernel dispatches of a kernel trace, in order: dicts with name, short, workgroups, us."""
    out = []
    for r in read_csv(trace_csv):
        if r.get("Kind", "KERNEL_DISPATCH") != "KERNEL_DISPATCH":
            continue
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        out.append({"id": int(r["Dispatch_Id"]), "name": r["Kernel_Name"], "short": short_name(r["Kernel_Name"]),
                    "workgroups": grid // max(wg, 1), "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
    out.sort(key=lambda d: d["id"])
    return out


def counters(counter_csv, counter):
    """Per-dispatch values of one counter: dicts with id, name, short, workgroups, value, us."""
    per = {}
    for r in read_csv(counter_csv):
        if r["Counter_Name"] != counter:
            continue
        i = int(r["Dispatch_Id"])
        d = per.setdefault(i, {"id": i, "name": r["Kernel_Name"], "short": short_name(r["Kernel_Name"]),
                               "workgroups": int(r["Grid_Size"]) // max(int(r["Workgroup_Size"]), 1),
                               "value": 0.0,
                               "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
        d["value"] += float(r["Counter_Value"])
    return [per[i] for i in sorted(per)]


def select(rows, pattern, workgroups=None):
    rx = re.compile(pattern)
    return [r for r in rows if rx.search(r["name"]) and (workgroups is None or r["workgroups"] == workgroups)]


# ------------------------------------------------------------------ summaries
def kernel_table(rows, top=30):
    """Dispatches grouped by (kernel, workgroups): calls, average, median, min, max (us), % time."""
    groups = {}
    for d in rows:
        groups.setdefault((d["short"], d["workgroups"]), []).append(d["us"])
    total = sum(d["us"] for d in rows) or 1.0
    table = []
    for (name, wg), us in groups.items():
        table.append({"kernel": name, "workgroups": wg, "calls": len(us), "avg_us": statistics.fmean(us),
                      "median_us": statistics.median(us), "min_us": min(us), "max_us": max(us),
                      "pct": 100.0 * sum(us) / total})
    table.sort(key=lambda t: -t["pct"])
    return table[:top]


def format_table(table):
    lines = ["  %-58s %10s %6s %10s %10s %10s %10s %6s" % ("kernel", "workgroups", "calls", "avg_us", "median_us",
                                                            "min_us", "max_us", "pct")]
    for t in table:
        lines.append("  %-58s %10d %6d %10.1f %10.1f %10.1f %10.1f %6.2f" % (
            t["kernel"][:58], t["workgroups"], t["calls"], t["avg_us"], t["median_us"], t["min_us"], t["max_us"],
            t["pct"]))
    return "\n".join(lines)


def copy_factor(copy_counter_csv, counter, copy_bytes):
    """Bytes per counter KiB for a plain device copy of copy_bytes bytes (median over dispatches)."""
    vals = [r["value"] for r in counters(copy_counter_csv, counter) if "copyBuffer" in r["name"] and r["value"] > 0]
    big = [v for v in vals if v * 1024 > copy_bytes / 8]
    if not big:
        raise ValueError(f"no copy dispatch of about {copy_bytes} bytes in {copy_counter_csv}")
    return copy_bytes / (statistics.median(big) * 1024)


def traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, pattern, copy_bytes, workgroups=None, last=None):
    """HBM bytes per dispatch of the selected kernel from FETCH_SIZE and WRITE_SIZE."""
    f = [r["value"] for r in select(counters(fetch_csv, "FETCH_SIZE"), pattern, workgroups)]
    w = [r["value"] for r in select(counters(write_csv, "WRITE_SIZE"), pattern, workgroups)]
    if not f or not w:
        raise ValueError(f"no dispatch of {pattern!r} in the counter files")
    if last:
        f, w = f[-last:], w[-last:]
    ff = copy_factor(copy_fetch_csv, "FETCH_SIZE", copy_bytes)
    wf = copy_factor(copy_write_csv, "WRITE_SIZE", copy_bytes)
    fk, wk = statistics.median(f), statistics.median(w)
    return {"dispatches": len(f), "fetch_kib": fk, "write_kib": wk, "fetch_factor": ff, "write_factor": wf,
            "fetch_min": min(f), "fetch_max": max(f), "write_min": min(w), "write_max": max(w),
            "bytes": fk * 1024 * ff + wk * 1024 * wf}


def mfma_utilisation(pmc_csv, pattern, simds, xcds, tiles_per_simd=None, workgroups=None, last=5):
    """MFMA instructions, busy cycles and utilisation of the selected kernel (medians over the last
    dispatches)."""
    def sel(counter):
        rows = select(counters(pmc_csv, counter), pattern, workgroups)[-last:]
        if not rows:
            raise ValueError(f"no {counter} for {pattern!r}")
        return rows

    def med(counter):
        return statistics.median(r["value"] for r in sel(counter))
    mfma, busy, valu, gui = (med(c) for c in ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU",
                                              "GRBM_GUI_ACTIVE"))
    cycles = gui / xcds
    ghz = statistics.median(r["value"] / xcds / (r["us"] * 1e3) for r in sel("GRBM_GUI_ACTIVE") if r["us"] > 0)
    res = {"SQ_INSTS_MFMA": mfma, "SQ_VALU_MFMA_BUSY_CYCLES": busy, "SQ_INSTS_VALU": valu, "GRBM_GUI_ACTIVE": gui,
           "kernel_cycles": cycles, "busy_per_mfma": busy / mfma if mfma else 0.0,
           "utilisation": busy / (cycles * simds) if cycles else 0.0, "clock_ghz": ghz}
    if tiles_per_simd:
        res["mfma_per_tile_simd"] = mfma / (tiles_per_simd * simds)
        res["valu_per_tile_simd"] = (valu - mfma) / (tiles_per_simd * simds)
        res["cycles_per_tile"] = cycles / tiles_per_simd
    return res


# ------------------------------------------------------------------ the profiling runs
BENCH = "python3 {root}/bench.py"
ONLY_FULL = "--no-cpu-baseline --no-decode --no-backward --no-varlen --no-other-workloads"
# The prefill kernel with outputs, no gate, forward walk, no SiLU prologue, d = 128, float16
# operands (k_fwd_bf16<MODE, GATE, REV, ACT, D, WIDE, value columns per workgroup>): every profiled
# prefill (full layer, share, long context) runs 64-column slices in chunks, after the chunk
# summaries and their prefix combine.
MAIN_KERNEL = r"k_fwd_bf16<0, false, false, false, 128, false, 64>"
WIDE_MAIN_KERNEL = MAIN_KERNEL
CHUNK_KERNELS = (("chunk summaries (k_summary_bf16)", r"k_summary_bf16", None),
                 ("prefix combine (k_scan_sub)", r"k_scan_sub", None))

RUNS = {
    # name: (rocprofv3 arguments, bench arguments)
    "stats_full": ("--kernel-trace --stats", "--steps 5 --warmup 1 " + ONLY_FULL),
    "stats_all": ("--kernel-trace --stats", "--steps 5 --warmup 1 --no-cpu-baseline --no-other-workloads "
                                             "--decode-steps 100"),
    "stats_share": ("--kernel-trace --stats", "--workload share --steps 5 --warmup 1 " + ONLY_FULL),
    "stats_long": ("--kernel-trace --stats", "--workload long --steps 5 --warmup 1 " + ONLY_FULL),
    "fetch_full": ("--pmc FETCH_SIZE", "--steps 2 --warmup 1 " + ONLY_FULL),
    "write_full": ("--pmc WRITE_SIZE", "--steps 2 --warmup 1 " + ONLY_FULL),
    "fetch_share": ("--pmc FETCH_SIZE", "--workload share --steps 3 --warmup 1 " + ONLY_FULL),
    "write_share": ("--pmc WRITE_SIZE", "--workload share --steps 3 --warmup 1 " + ONLY_FULL),
    "fetch_long": ("--pmc FETCH_SIZE", "--workload long --steps 2 --warmup 1 " + ONLY_FULL),
    "write_long": ("--pmc WRITE_SIZE", "--workload long --steps 2 --warmup 1 " + ONLY_FULL),
    "fetch_decode": ("--pmc FETCH_SIZE", "--decode-only --decode-steps 20"),
    "write_decode": ("--pmc WRITE_SIZE", "--decode-only --decode-steps 20"),
    "copy_fetch": ("--pmc FETCH_SIZE", "--copy-probe"),
    "copy_write": ("--pmc WRITE_SIZE", "--copy-probe"),
    "mfma_full": ("--pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU GRBM_GUI_ACTIVE",
                  "--steps 2 --warmup 1 --settle-s 0.05 " + ONLY_FULL),
}
COPY_BYTES = 4 << 30


def command(name, out_root, root="$GRAFT_REPO_ROOT"):
    prof, bench = RUNS[name]
    return (f"rocprofv3 {prof} --output-format csv -d {out_root}/{name} -o run -- "
            f"{BENCH.format(root=root)} {bench}")


def _csv(out_root, name, kind):
    path = os.path.join(out_root, name, f"run_{kind}.csv")
    if not os.path.exists(path):
        raise FileNotFoundError(path)
    return path


def _shown(out_root):
    """out_root as the profiling commands name it: under the repository root on the GPU machine."""
    return out_root if os.path.isabs(out_root) else "$GRAFT_REPO_ROOT/" + out_root


def _header(title, names, out_root):
    lines = [f"# {title}", "# Commands (repository root as $GRAFT_REPO_ROOT, one MI355X, `cd /tmp` first):"]
    lines += [f"#   {command(n, _shown(out_root))}" for n in names]
    lines.append(f"# Summarised with: python -m long_context_la_amd.profiling summarize {out_root}")
    return lines


def summarize_stats(out_root, name, title, last_of=None, also=()):
    """Kernel table of a trace.  last_of = (pattern, workgroups, n): the average of the last n
    dispatches of that kernel (the timed steps); also = ((label, pattern), ...): the prefill's other
    launches, whose last-n averages are added into a per-step total."""
    rows = dispatches(_csv(out_root, name, "kernel_trace"))
    lines = _header(title, [name], out_root)
    lines.append(f"# kernel code digest (sha256[:16] of la_prefill_bf16.hip without comments): {source_digest()}")
    lines.append("# Durations from the kernel trace, all dispatches of the run (settling, warm-up and timed steps).")
    if last_of:
        pattern, wg, n = last_of
        sel = select(rows, pattern, wg)[-n:]
        if sel:
            main = statistics.fmean(d['us'] for d in sel)
            lines.append(f"# Last {len(sel)} dispatches of {sel[0]['short']} with {wg} workgroups (the timed steps): "
                         f"average {main:.1f} us")
            parts, total = [], main
            for label, pat in also:
                other = select(rows, pat, None)[-n:]
                if other:
                    avg = statistics.fmean(d['us'] for d in other)
                    parts.append(f"{label} {avg:.1f} us")
                    total += avg
            if parts:
                lines.append(f"# The prefill's launches per timed step (last {n} of each): main {main:.1f} us + "
                             + " + ".join(parts) + f" = {total:.1f} us")
    lines.append(format_table(kernel_table(rows)))
    return "\n".join(lines) + "\n"


def summarize_traffic(out_root, workload, pattern, alg_bytes, workgroups=None, last=None, extra_kernels=()):
    fetch, write = f"fetch_{workload}", f"write_{workload}"
    names = [fetch, write, "copy_fetch", "copy_write"]
    t = traffic(_csv(out_root, fetch, "counter_collection"), _csv(out_root, write, "counter_collection"),
                _csv(out_root, "copy_fetch", "counter_collection"), _csv(out_root, "copy_write", "counter_collection"),
                pattern, COPY_BYTES, workgroups, last)
    lines = _header(f"HBM traffic of the {workload} workload's main kernel ({pattern}, {workgroups or 'any'} "
                    "workgroups)", names, out_root)
    lines += [f"# FETCH_SIZE KiB per dispatch: {t['dispatches']} dispatches, min {t['fetch_min']:.0f}, median "
              f"{t['fetch_kib']:.0f}, max {t['fetch_max']:.0f}",
              f"# WRITE_SIZE KiB per dispatch: min {t['write_min']:.0f}, median {t['write_kib']:.0f}, max "
              f"{t['write_max']:.0f}",
              f"# copy calibration ({COPY_BYTES} bytes read and written): fetch factor {t['fetch_factor']:.4f}, "
              f"write factor {t['write_factor']:.4f} bytes per KiB-count",
              f"# scaled HBM bytes per dispatch: {t['bytes'] / 1e9:.4f} GB; algorithmic {alg_bytes / 1e9:.4f} GB "
              f"(ratio {t['bytes'] / alg_bytes:.3f})"]
    for label, pat, wg in extra_kernels:
        try:
            e = traffic(_csv(out_root, fetch, "counter_collection"), _csv(out_root, write, "counter_collection"),
                        _csv(out_root, "copy_fetch", "counter_collection"),
                        _csv(out_root, "copy_write", "counter_collection"), pat, COPY_BYTES, wg, last)
            lines.append(f"# {label}: {e['bytes'] / 1e9:.4f} GB per dispatch (fetch {e['fetch_kib']:.0f} KiB, write "
                         f"{e['write_kib']:.0f} KiB, {e['dispatches']} dispatches)")
        except ValueError:
            lines.append(f"# {label}: no dispatch")
    lines += ["# bench.py reads the lines below while the kernel source hash matches.",
              f"kernel_source_sha256_16 = {source_digest()}",
              f"fetch_kib_per_dispatch = {t['fetch_kib']:.0f}", f"write_kib_per_dispatch = {t['write_kib']:.0f}",
              f"copy_fetch_factor = {t['fetch_factor']:.6f}", f"copy_write_factor = {t['write_factor']:.6f}",
              f"algorithmic_bytes = {alg_bytes}", f"traffic_bytes = {t['bytes']:.0f}"]
    return "\n".join(lines) + "\n"


def summarize_mfma(out_root, tiles_per_simd, pattern, workgroups):
    agent = agent_peaks(_csv(out_root, "mfma_full", "agent_info"))
    m = mfma_utilisation(_csv(out_root, "mfma_full", "counter_collection"), pattern, DATASHEET["simds"],
                         DATASHEET["xcds"], tiles_per_simd, workgroups)
    lines = _header("MFMA utilisation of the full-layer prefill kernel (1 x 64 heads x 131072 tokens, d=128)",
                    ["mfma_full"], out_root)
    lines += [f"# device: {agent['cus']} CUs at up to {agent['max_clock_mhz']:.0f} MHz -> bf16 peak "
              f"{agent['bf16_tflops']:.0f} TFLOP/s ({agent['source']})",
              f"# medians over the last 5 dispatches of {pattern} with {workgroups} workgroups:"]
    lines += [f"{k} = {m[k]:.0f}" for k in ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU",
                                            "GRBM_GUI_ACTIVE")]
    lines += [f"# kernel cycles (GRBM_GUI_ACTIVE / {DATASHEET['xcds']} XCDs) = {m['kernel_cycles']:.4g}",
              f"# busy cycles per MFMA = {m['busy_per_mfma']:.2f}",
              f"# effective clock (kernel cycles / dispatch duration) = {m['clock_ghz']:.3f} GHz",
              f"# MFMA utilisation = busy cycles / (kernel cycles x {DATASHEET['simds']} SIMDs) = "
              f"{m['utilisation']:.4f}",
              f"# per 64-token tile and SIMD: {m['mfma_per_tile_simd']:.1f} MFMA, {m['valu_per_tile_simd']:.1f} other "
              f"VALU, {m['cycles_per_tile']:.0f} cycles",
              "# bench.py reads the lines below while the kernel source hash matches.",
              f"kernel_source_sha256_16 = {source_digest()}",
              f"mfma_utilisation = {m['utilisation']:.4f}",
              f"cycles_per_tile = {m['cycles_per_tile']:.1f}"]
    return "\n".join(lines) + "\n"


def read_profile_values(path):
    """key = value lines of a profile summary (comments skipped)."""
    vals = {}
    if not os.path.exists(path):
        return vals
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, _, v = line.partition("=")
                vals[k.strip()] = v.strip()
    return vals


def current_value(path, key):
    """A profile value when the profile was taken on the current prefill source, else None."""
    vals = read_profile_values(path)
    if vals.get("kernel_source_sha256_16") != source_digest() or key not in vals:
        return None
    return float(vals[key])


def summarize_all(out_root, profiles_dir=PROFILES):
    """Writes every profile whose raw output is present under out_root; returns the files written."""
    full_bytes = 1024 * 64 * 131072
    eight_heads = lambda n: 1024 * 8 * n
    jobs = {
        "kernel_stats_prefill_full_64x131072.txt": lambda: summarize_stats(
            out_root, "stats_full", "kernel statistics of the full-layer prefill (1 x 64 heads x 131072 tokens, d=128, "
            "bf16): settling, 1 warm-up, 5 timed steps and 5 per-kernel timings",
            (MAIN_KERNEL, 256, 5), also=tuple((label.split(" (")[0], pat) for label, pat, _ in CHUNK_KERNELS)),
        "kernel_stats_bench_all_legs.txt": lambda: summarize_stats(
            out_root, "stats_all", "kernel statistics of bench.py: full-layer prefill (1 x 64 heads x 131072 tokens, "
            "d=128, bf16), backward, packed and mixed legs, decode (128 x 64 units, 100 steps)"),
        "kernel_stats_prefill_share_8x32768.txt": lambda: summarize_stats(
            out_root, "stats_share", "kernel statistics of the chunked share prefill (1 x 8 heads x 32768, d=128)"),
        "kernel_stats_prefill_long_8x1048576.txt": lambda: summarize_stats(
            out_root, "stats_long", "kernel statistics of the chunked long-context prefill (1 x 8 heads x 1048576, "
            "d=128, checkpoints every 65536)"),
        "prefill_full_hbm_traffic.txt": lambda: summarize_traffic(
            out_root, "full", MAIN_KERNEL, full_bytes, 256, extra_kernels=CHUNK_KERNELS),
        "prefill_share_hbm_traffic.txt": lambda: summarize_traffic(
            out_root, "share", WIDE_MAIN_KERNEL, eight_heads(32768), 256,
            extra_kernels=CHUNK_KERNELS),
        "prefill_long_hbm_traffic.txt": lambda: summarize_traffic(
            out_root, "long", WIDE_MAIN_KERNEL, eight_heads(1 << 20), 256,
            extra_kernels=CHUNK_KERNELS),
        "decode_128x64_hbm_traffic.txt": lambda: summarize_traffic(
            out_root, "decode", r"k_decode", 8192 * (2 * 128 * 128 * 4 + 4 * 128 * 2), 8192),
        "prefill_full_mfma_util.txt": lambda: summarize_mfma(out_root, 1024, MAIN_KERNEL,
                                                             256),
    }
    written = []
    for fname, job in jobs.items():
        try:
            text = job()
        except (FileNotFoundError, ValueError) as e:
            print(f"skip {fname}: {e}", file=sys.stderr)
            continue
        with open(os.path.join(profiles_dir, fname), "w") as f:
            f.write(text)
        written.append(fname)
    return written


def main(argv=None):
    import argparse

    ap = argparse.ArgumentParser(prog="python -m long_context_la_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("commands", help="print the rocprofv3 commands, one per line")
    c.add_argument("out_root")
    c.add_argument("--only", nargs="*")
    s = sub.add_parser("summarize", help="write profiles/*.txt from the raw output under out_root")
    s.add_argument("out_root")
    s.add_argument("--profiles", default=PROFILES)
    a = ap.parse_args(argv)
    if a.cmd == "commands":
        for name in a.only or RUNS:
            print(command(name, a.out_root))
    else:
        for f in summarize_all(a.out_root, a.profiles):
            print(f)


if __name__ == "__main__":
    main()
