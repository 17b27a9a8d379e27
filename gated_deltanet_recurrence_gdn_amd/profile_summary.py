"""Summarise rocprofv3 CSV output of bench.py runs into short text files under profiles/.

Three rocprofv3 runs of bench.py feed it (each its own process; see the command lines
written into the summaries):

  kernel trace:  rocprofv3 --kernel-trace --stats --output-format csv -d DIR/kt -o kt -- \\
                     python bench.py --no-cpu --no-forms
  fetch bytes:   rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/fetch -o fetch -- \\
                     python bench.py --steps 2 --warmup 1 --no-cpu --no-forms --calib-copy
  write bytes:   rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/write -o write -- \\
                     python bench.py --steps 2 --warmup 1 --no-cpu --no-forms --calib-copy

and, for --forms-only, a kernel trace of the bench with its secondary forms:

  forms:         rocprofv3 --kernel-trace --stats --output-format csv -d DIR/forms -o forms -- \\
                     python bench.py --no-cpu --steps 5 --warmup 5

    python -m gated_deltanet_recurrence_gdn_amd.profile_summary DIR [--workload NAME]

One chunked gdn_forward is two launches, tm_kernel (the per-chunk triangular
inverses) and chunk_kernel (the sequential pass); both are summarised and summed.
FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what the same counters
read for the plain 512 MiB device copy that --calib-copy adds to the run: the copy
reads and writes exactly 512 MiB, so scale = 512 MiB / counter.  The scaled bytes
per gdn_forward (both kernels) are written to
profiles/chunk_kernel_<workload>_traffic.json together with a hash of the kernel
source, which bench.py checks before reporting them.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
from gated_deltanet_recurrence_gdn_amd.srchash import code_hash  # noqa: E402
PROFILES = os.path.join(ROOT, "profiles")
CHUNK = "chunk_kernel"
TM = "tm_kernel"
KERNELS = (TM, CHUNK)
COPY = "copyBuffer"
COPY_BYTES = 512 * 1024 * 1024

KT_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d {d}/kt -o kt -- "
          "python bench.py --no-cpu --no-forms")
TIMED_STEPS = 40  # bench.py's default --steps: the last dispatches of the trace are its timed region
PMC_CMD = ("rocprofv3 --pmc {c} --output-format csv -d {d}/{n} -o {n} -- "
           "python bench.py --steps 2 --warmup 1 --no-cpu --no-forms --calib-copy")


def _csv(path_glob):
    paths = glob.glob(path_glob, recursive=True)
    if not paths:
        raise FileNotFoundError(path_glob)
    with open(paths[0]) as f:
        return list(csv.DictReader(f))


def src_hash():
    return code_hash("gdn_chunk.hip")


def kernel_stats(d):
    rows = _csv(os.path.join(d, "kt", "**", "*kernel_stats.csv"))
    out = []
    for r in rows:
        out.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]), float(r["AverageNs"]),
                    float(r["Percentage"])))
    return out


def trace_durations(d, kernel):
    rows = _csv(os.path.join(d, "kt", "**", "*kernel_trace.csv"))
    rows = [r for r in rows if kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]


def counter_per_dispatch(d, sub, counter):
    rows = _csv(os.path.join(d, sub, "**", "*counter_collection.csv"))
    vals = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    copy = [v for k, vs in vals.items() if COPY in k for v in vs]
    if not copy:
        raise RuntimeError(f"{counter}: copy dispatch missing in {d}/{sub}")
    per = {}
    for kn in KERNELS:
        ks = [v for k, vs in vals.items() if kn in k for v in vs]
        if not ks:
            raise RuntimeError(f"{counter}: {kn} dispatch missing in {d}/{sub}")
        per[kn] = (statistics.mean(ks), len(ks))
    return per, statistics.mean(copy)


FORMS_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d {d}/forms -o forms -- "
             "python bench.py --no-cpu --steps 5 --warmup 5")


def rel_dir(d):
    """The output directory the profiled commands were given, relative to the repo root
    when it lies inside it (the commands run from there)."""
    a = os.path.abspath(d)
    return os.path.relpath(a, ROOT) if a.startswith(ROOT + os.sep) else a


def forms_summary(d):
    """Per-kernel-instantiation stats of a bench run with its secondary forms."""
    rows = _csv(os.path.join(d, "forms", "**", "*kernel_stats.csv"))
    lines = ["rocprofv3 kernel trace: bench.py with its secondary forms (scan, 5-call streaming warm and",
             "cold, 3-frame d=64 warm and cold, each also segmented, bidirectional, fused prologue from",
             "packed qkv, FP8 inputs)",
             "", "command (MI355X, repo root, TMPDIR=/tmp):", "  " + FORMS_CMD.format(d=rel_dir(d)),
             f"kernel code sha256[:16] (gdn_chunk.hip, comments and whitespace removed): {src_hash()}", "",
             "template arguments: chunk_kernel<d_k, input type (1 bf16, 2 FP8), prologue, sweep (0 the whole",
             "call; 1 and 2 the first and second launch of the bidirectional split; 3 the segment rows of the",
             "segmented form)>, tm_kernel<d_k, input type, prologue>, scan_kernel<d_k, state values per lane,",
             "input type (0 fp32, 1 bf16, 2 FP8), prologue>; combine_rows_kernel: the bidirectional split's",
             "middle rows; seg_combine_kernel<d_k, d_v>: the segmented form's start states and corrections", "",
             f"  {'kernel':78s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}"]
    for r in rows:
        name = r["Name"].replace("void gdn::(anonymous namespace)::", "")
        name = name.split("(gdn::")[0].split("(void*")[0]
        lines.append(f"  {name[:78]:78s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                     f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f}")
    return lines


# Hardware-counter passes (one rocprofv3 --pmc run each) over the bench's chunked call.
COUNTER_SETS = [
    "TA_BUSY_avr TA_ADDR_STALLED_BY_TC_CYCLES_sum",
    "TA_DATA_STALLED_BY_TC_CYCLES_sum TA_TA_BUSY_sum",
    "TCC_HIT_sum TCC_MISS_sum",
    "TCP_PENDING_STALL_CYCLES_sum TCP_TOTAL_CACHE_ACCESSES_sum",
    "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_INSTS_VMEM_RD SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT "
    "SQ_INSTS_VALU SQ_INSTS_MFMA",
]
CTR_CMD = ("rocprofv3 --pmc {c} --output-format csv -d {d}/ctr_{i} -o ctr -- "
           "python bench.py --steps 2 --warmup 1 --no-cpu --no-forms")


def counters_summary(d):
    """Mean per-dispatch counter values of tm_kernel and chunk_kernel from the DIR/ctr_<i> passes."""
    vals = {kn: {} for kn in KERNELS}
    for i in range(len(COUNTER_SETS)):
        rows = _csv(os.path.join(d, f"ctr_{i}", "**", "*counter_collection.csv"))
        acc = {}
        for r in rows:
            for kn in KERNELS:
                if kn in r["Kernel_Name"]:
                    acc.setdefault((kn, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
        for (kn, cn), v in acc.items():
            vals[kn][cn] = statistics.mean(v)
    lines = ["rocprofv3 hardware counters: chunked GDN forward (tm_kernel + chunk_kernel), workload "
             "batched_bf16_d128", "(mean per dispatch; *_sum counters are summed over the 256 CUs' "
             "instances, *_avr averaged over them)", "",
             "commands (MI355X, repo root, TMPDIR=/tmp), one counter set per run:"]
    lines += ["  " + CTR_CMD.format(c=c, d=rel_dir(d), i=i) for i, c in enumerate(COUNTER_SETS)]
    lines += [f"kernel code sha256[:16] (comments and whitespace removed): {src_hash()}", ""]
    for kn in KERNELS:
        lines.append(f"{kn}:")
        for cn in sorted(vals[kn]):
            lines.append(f"  {cn:42s} {vals[kn][cn]:16.6g}")
    return lines


MFMA_SETS = ["MfmaUtil", "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_MFMA"]
MFMA_CMD = ("rocprofv3 --pmc {c} --output-format csv -d {d}/mfma_{i} -o mfma -- "
            "python bench.py --steps 2 --warmup 1 --no-cpu --no-forms")
SIMDS = 256 * 4  # MI355X: 256 CUs x 4 SIMDs


def _pass_means(d, sub, kernels):
    rows = _csv(os.path.join(d, sub, "**", "*counter_collection.csv"))
    acc = {}
    for r in rows:
        for kn in kernels:
            if kn in r["Kernel_Name"]:
                acc.setdefault((kn, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    return {k: statistics.mean(v) for k, v in acc.items()}


def mfma_summary(d):
    """MFMA utilisation of tm_kernel and chunk_kernel from the DIR/mfma_<i> passes: rocprofv3's
    derived MfmaUtil, and SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1024 SIMDs) from the raw
    counters as a cross-check; bf16 MFMA flops from SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512."""
    vals = {}
    for i in range(len(MFMA_SETS)):
        vals.update(_pass_means(d, f"mfma_{i}", KERNELS))
    rec = {"workload": "batched_bf16_d128", "kernel_code_sha256_16": src_hash(), "simds": SIMDS, "kernels": {}}
    lines = ["rocprofv3 MFMA counters: chunked GDN forward (tm_kernel + chunk_kernel), workload batched_bf16_d128",
             "(mean per dispatch)", "", "commands (MI355X, repo root, TMPDIR=/tmp), one counter set per run:"]
    lines += ["  " + MFMA_CMD.format(c=c, d=rel_dir(d), i=i) for i, c in enumerate(MFMA_SETS)]
    lines += [f"kernel code sha256[:16] (comments and whitespace removed): {src_hash()}", "",
              "MfmaUtil = 100 x SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1024 SIMDs) (rocprofv3's derived "
              "counter); flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512", ""]
    for kn in KERNELS:
        g = lambda c: vals.get((kn, c))
        util = g("MfmaUtil")
        busy, gui, mops, ninst = (g("SQ_VALU_MFMA_BUSY_CYCLES"), g("GRBM_GUI_ACTIVE"),
                                  g("SQ_INSTS_VALU_MFMA_MOPS_BF16"), g("SQ_INSTS_MFMA"))
        raw = busy / (gui * SIMDS) if busy is not None and gui else None
        rec["kernels"][kn] = {"MfmaUtil_pct": util, "SQ_VALU_MFMA_BUSY_CYCLES": busy, "GRBM_GUI_ACTIVE": gui,
                              "busy_over_gui_x_simds": raw, "bf16_mfma_flops": (mops * 512 if mops else None),
                              "SQ_INSTS_MFMA": ninst}
        lines.append(f"{kn}: MfmaUtil {util}%  busy/(gui x 1024) {raw}  GRBM_GUI_ACTIVE {gui}  "
                     f"MFMA instructions {ninst}  bf16 MFMA flops {mops * 512 if mops else None}")
    ck = rec["kernels"][CHUNK]
    rec["mfma_busy"] = (ck["MfmaUtil_pct"] / 100.0 if ck["MfmaUtil_pct"] is not None else ck["busy_over_gui_x_simds"])
    lines += ["", f"chunk_kernel MFMA busy fraction reported by bench.py: {rec['mfma_busy']}"]
    return rec, lines


SCAN = "scan_kernel"
SCAN_CMD = ("rocprofv3 --pmc {c} --output-format csv -d {d}/{n} -o {n} -- "
            "python bench.py --form scan --steps 2 --warmup 1 --no-cpu --no-forms --calib-copy")


def scan_traffic_summary(d):
    """HBM bytes of one scan_kernel dispatch on the batched d=128 workload (DIR/scan_fetch, DIR/scan_write),
    scaled like the chunked kernel's by the run's plain 512 MiB copy."""
    import bench
    from gated_deltanet_recurrence_gdn_amd import inputs
    w = inputs.WORKLOADS["batched_bf16_d128"]
    out = {}
    for sub, cn in (("scan_fetch", "FETCH_SIZE"), ("scan_write", "WRITE_SIZE")):
        rows = _csv(os.path.join(d, sub, "**", "*counter_collection.csv"))
        ks = [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == cn and SCAN in r["Kernel_Name"]]
        cp = [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == cn and COPY in r["Kernel_Name"]]
        if not ks or not cp:
            raise RuntimeError(f"{cn}: scan or copy dispatch missing in {d}/{sub}")
        out[cn] = (statistics.mean(ks), len(ks), statistics.mean(cp))
    f_kib, nf, f_copy = out["FETCH_SIZE"]
    w_kib, nw, w_copy = out["WRITE_SIZE"]
    fb = f_kib * 1024 * COPY_BYTES / (f_copy * 1024)
    wb = w_kib * 1024 * COPY_BYTES / (w_copy * 1024)
    abytes = bench.algorithmic_bytes(w.B, w.T, w.H, w.dk, w.dv)
    rec = {"workload": w.name, "kernel": SCAN, "kernel_code_sha256_16": code_hash("gdn_scan.hip"),
           "bytes_per_launch": fb + wb, "fetch_bytes": fb, "write_bytes": wb, "fetch_kib_raw": f_kib,
           "write_kib_raw": w_kib, "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
           "algorithmic_bytes_per_launch": abytes, "dispatches": [nf, nw]}
    lines = [f"rocprofv3 HBM traffic counters: sequential scan (scan_kernel), workload {w.name}", "",
             "commands (MI355X, repo root, TMPDIR=/tmp), one counter per run:",
             "  " + SCAN_CMD.format(c="FETCH_SIZE", d=rel_dir(d), n="scan_fetch"),
             "  " + SCAN_CMD.format(c="WRITE_SIZE", d=rel_dir(d), n="scan_write"),
             f"kernel code sha256[:16] (gdn_scan.hip, comments and whitespace removed): {rec['kernel_code_sha256_16']}",
             "", f"scale: the run's plain 512 MiB copy reads FETCH_SIZE {f_copy:.0f} KiB, WRITE_SIZE {w_copy:.0f} KiB",
             f"scan_kernel per dispatch (mean of {nf} / {nw}): FETCH_SIZE {f_kib:.0f} KiB raw -> {fb / 1e9:.4f} GB, "
             f"WRITE_SIZE {w_kib:.0f} KiB raw -> {wb / 1e9:.4f} GB",
             f"total {(fb + wb) / 1e9:.4f} GB vs algorithmic {abytes / 1e9:.4f} GB ({(fb + wb) / abytes:.3f}x)"]
    return rec, lines


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--counters-only", action="store_true",
                    help="only summarise the DIR/ctr_<i> hardware-counter passes")
    ap.add_argument("dir", help="directory holding the kt/, fetch/ and write/ rocprofv3 outputs")
    ap.add_argument("--forms-only", action="store_true",
                    help="only summarise DIR/forms (the kernel trace of a bench run with its secondary forms)")
    ap.add_argument("--workload", default="batched_bf16_d128")
    ap.add_argument("--mfma-only", action="store_true", help="only summarise the DIR/mfma_<i> passes")
    ap.add_argument("--scan-only", action="store_true", help="only summarise DIR/scan_fetch and DIR/scan_write")
    ap.add_argument("--algorithmic-bytes", type=float, default=None,
                    help="algorithmic bytes per launch (default: bench.py's formula for the workload)")
    a = ap.parse_args()
    os.makedirs(PROFILES, exist_ok=True)
    if a.mfma_only or a.scan_only:
        rec, lines = mfma_summary(a.dir) if a.mfma_only else scan_traffic_summary(a.dir)
        name = "chunk_kernel_batched_bf16_d128_mfma" if a.mfma_only else "scan_kernel_batched_bf16_d128_traffic"
        with open(os.path.join(PROFILES, name + ".json"), "w") as f:
            json.dump(rec, f, indent=1)
        with open(os.path.join(PROFILES, name + ".txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return
    if a.counters_only:
        lines = counters_summary(a.dir)
        with open(os.path.join(PROFILES, "chunk_kernel_batched_bf16_d128_counters.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return
    if a.forms_only:
        lines = forms_summary(a.dir)
        with open(os.path.join(PROFILES, "forms_batched_bf16_d128.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return
    import bench
    from gated_deltanet_recurrence_gdn_amd import inputs
    w = inputs.WORKLOADS[a.workload]
    abytes = a.algorithmic_bytes or bench.algorithmic_bytes(w.B, w.T, w.H, w.dk, w.dv)

    stats = kernel_stats(a.dir)
    lines = [f"rocprofv3 kernel trace: chunked GDN forward (tm_kernel + chunk_kernel), workload {w.name}",
             f"(B={w.B}, H={w.H}, T={w.T}, d_k={w.dk}, d_v={w.dv}, bf16 I/O, chunk_len=64, fp32 state in/out)",
             "", "command (MI355X, repo root, TMPDIR=/tmp):", "  " + KT_CMD.format(d=rel_dir(a.dir)),
             f"kernel code sha256[:16] (comments and whitespace removed): {src_hash()}", "",
             "kernel stats (durations in ns):",
             f"  {'name':60s} {'calls':>6s} {'total_ns':>14s} {'avg_ns':>12s} {'pct':>7s}"]
    for n, c, t, av, pc in stats:
        lines.append(f"  {n[:60]:60s} {c:6d} {t:14.0f} {av:12.0f} {pc:7.2f}")
    path = 0.0
    lines.append("")
    for kn in KERNELS:
        dur = trace_durations(a.dir, kn)
        timed = dur[-TIMED_STEPS:]
        tav = statistics.mean(timed)
        path += tav
        lines += [f"{kn}: average over the last {len(timed)} of {len(dur)} dispatches (bench.py's timed steps): "
                  f"{tav / 1e6:.4f} ms",
                  f"  per-dispatch durations (ms): " + " ".join(f"{x / 1e6:.3f}" for x in dur)]
    lines += ["", f"one gdn_forward (both kernels): {path / 1e6:.4f} ms -> algorithmic "
              f"{abytes / (path * 1e-9) / 1e9:.1f} GB/s ({abytes:.0f} B per call)"]
    with open(os.path.join(PROFILES, f"chunk_kernel_{w.name}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    fetch, fetch_c = counter_per_dispatch(a.dir, "fetch", "FETCH_SIZE")
    write, write_c = counter_per_dispatch(a.dir, "write", "WRITE_SIZE")
    f_scale = COPY_BYTES / (fetch_c * 1024.0)
    w_scale = COPY_BYTES / (write_c * 1024.0)
    fetch_b = sum(fetch[kn][0] for kn in KERNELS) * 1024.0 * f_scale
    write_b = sum(write[kn][0] for kn in KERNELS) * 1024.0 * w_scale
    rec = {"workload": w.name, "kernel_code_sha256_16": src_hash(),
           "bytes_per_launch": fetch_b + write_b, "fetch_bytes": fetch_b, "write_bytes": write_b,
           "per_kernel_kib_raw": {kn: {"fetch": fetch[kn][0], "write": write[kn][0]} for kn in KERNELS},
           "copy_fetch_kib": fetch_c, "copy_write_kib": write_c,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "algorithmic_bytes_per_launch": abytes,
           "dispatches": {kn: [fetch[kn][1], write[kn][1]] for kn in KERNELS}}
    with open(os.path.join(PROFILES, f"chunk_kernel_{w.name}_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    tl = [f"rocprofv3 HBM traffic counters: chunked GDN forward (tm_kernel + chunk_kernel), workload {w.name}", "",
          "commands (MI355X, repo root, TMPDIR=/tmp), one counter per run:",
          "  " + PMC_CMD.format(c="FETCH_SIZE", d=rel_dir(a.dir), n="fetch"),
          "  " + PMC_CMD.format(c="WRITE_SIZE", d=rel_dir(a.dir), n="write"),
          f"kernel code sha256[:16] (comments and whitespace removed): {src_hash()}", "",
          "scale: the run's plain 512 MiB device copy (--calib-copy) reads and writes 512 MiB;",
          f"  FETCH_SIZE reads {fetch_c:.0f} KiB for it -> scale {f_scale:.3f}",
          f"  WRITE_SIZE reads {write_c:.0f} KiB for it -> scale {w_scale:.3f}", ""]
    for kn in KERNELS:
        tl.append(f"{kn} per dispatch (mean of {fetch[kn][1]} / {write[kn][1]} dispatches): "
                  f"FETCH_SIZE {fetch[kn][0]:.0f} KiB raw -> {fetch[kn][0] * 1024 * f_scale / 1e9:.4f} GB, "
                  f"WRITE_SIZE {write[kn][0]:.0f} KiB raw -> {write[kn][0] * 1024 * w_scale / 1e9:.4f} GB")
    tl += [f"one gdn_forward: fetch {fetch_b / 1e9:.4f} GB + write {write_b / 1e9:.4f} GB = "
           f"{(fetch_b + write_b) / 1e9:.4f} GB vs algorithmic {abytes / 1e9:.4f} GB "
           f"({(fetch_b + write_b) / abytes:.3f}x)"]
    with open(os.path.join(PROFILES, f"chunk_kernel_{w.name}_traffic.txt"), "w") as f:
        f.write("\n".join(tl) + "\n")
    print("\n".join(lines + [""] + tl))


if __name__ == "__main__":
    main()
