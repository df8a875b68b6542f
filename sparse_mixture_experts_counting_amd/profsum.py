"""Summaries of rocprofv3 output for the committed profiles.

    python -m sparse_mixture_experts_counting_amd.profsum stats KERNEL_STATS_CSV TITLE COMMAND
        Markdown table of per-kernel calls and durations (microseconds) from a
        `rocprofv3 --kernel-trace --stats` run.

    python -m sparse_mixture_experts_counting_amd.profsum kernels FETCH_CSV WRITE_CSV STATS_CSV TITLE \
            PMC_COMMAND ;; STATS_COMMAND
        Markdown table of every library kernel's HBM bytes read and written per dispatch and the
        rate over its average duration (PMC_COMMAND names the counter COUNTER; STATS_COMMAND is
        the kernel-trace run the durations come from).

    python -m sparse_mixture_experts_counting_amd.profsum mfma PMC_CSV[,PMC_CSV] STATS_CSV KERNEL \
            TITLE COMMANDS
        Matrix-core busy fraction, clock and wait fractions of one kernel from `--pmc` runs.

    python -m sparse_mixture_experts_counting_amd.profsum traffic FETCH_CSV WRITE_CSV WORKLOAD KERNEL \
            OUT_JSON COMMAND
        HBM bytes per launch of the kernels whose name contains KERNEL, from two
        `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs (KiB per dispatch), each scaled by
        what the same counter reads for the benchmark's untimed 256 MiB device copy (the
        calibration).  Writes OUT_JSON (read by bench.py) and prints a Markdown summary.
"""

import collections
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SRC = os.path.join(ROOT, "sparse_mixture_experts_counting_amd", "csrc", "gemm_bf16.hip")
CALIB_BYTES = 256 << 20          # the benchmark's calibration copy (bytes read and written)


def source_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def short_name(name):
    """Kernel name without its argument list (the last parenthesised group that ends the name)."""
    name = name.strip()
    if not name.endswith(")"):
        return name
    depth = 0
    for i in range(len(name) - 1, -1, -1):
        depth += {")": 1, "(": -1}.get(name[i], 0)
        if depth == 0:
            return name[:i].rstrip() or name
    return name


def stats(path, title, command):
    rows = list(csv.DictReader(open(path)))
    out = ["# Kernel time: %s" % title, "", "Command (run from /tmp with TMPDIR=/tmp on one MI355X; "
           "repository at $R):", "", "    " + command, "",
           "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = short_name(r["Name"])
        if len(name) > 100:
            name = name[:97] + "..."
        out.append("| `%s` | %s | %.1f | %.1f | %.1f | %.2f |" % (
            name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return "\n".join(out) + "\n"


def _per_kernel(path):
    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def traffic(fetch_csv, write_csv, workload, kernel, out_json, command):
    fetch, write = _per_kernel(fetch_csv), _per_kernel(write_csv)

    def calib(vals):   # the largest copy: the benchmark's 256 MiB calibration copy
        best = max((max(v) for k, v in vals.items() if "copyBuffer" in k or "copy_kernel" in k),
                   default=0.0)
        if best <= 0:
            raise SystemExit("no copy kernel found for the calibration")
        return CALIB_BYTES / (best * 1024.0), best

    f_scale, f_cal = calib(fetch)
    w_scale, w_cal = calib(write)
    # KERNEL may name several kernels joined by '+' (one operation's kernels); their averages add.
    picked = []
    for part in kernel.split("+"):
        names = [k for k in fetch if part in k]
        if not names:
            raise SystemExit("kernel %r not in %s" % (part, fetch_csv))
        picked.append(names[0])
    fk = sum(sum(fetch[n]) / len(fetch[n]) for n in picked)
    wk = sum(sum(write.get(n, [0.0])) / max(1, len(write.get(n, []))) for n in picked)
    hbm = fk * 1024.0 * f_scale + wk * 1024.0 * w_scale
    rec = {"workload": workload, "kernel": " + ".join(short_name(n) for n in picked),
           "kernel_source_sha256_16": source_hash(),
           "fetch_kib_per_launch": fk, "write_kib_per_launch": wk,
           "calibration": {"bytes": CALIB_BYTES, "fetch_kib": f_cal, "write_kib": w_cal,
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "hbm_bytes_per_launch": hbm, "command": command}
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    md = ["# HBM traffic: %s, `%s`" % (workload, rec["kernel"]), "",
          "Commands (run from /tmp with TMPDIR=/tmp on one MI355X; repository at $R):", "",
          "    " + command.replace("COUNTER", "FETCH_SIZE"),
          "    " + command.replace("COUNTER", "WRITE_SIZE"), "",
          "| quantity | value |", "|---|---|",
          "| FETCH_SIZE per launch | %.0f KiB |" % fk,
          "| WRITE_SIZE per launch | %.0f KiB |" % wk,
          "| 256 MiB calibration copy: FETCH_SIZE / WRITE_SIZE | %.0f / %.0f KiB |" % (f_cal, w_cal),
          "| scale applied (fetch, write) | %.4f, %.4f |" % (f_scale, w_scale),
          "| HBM bytes per launch | %.3f GB |" % (hbm / 1e9),
          "| kernel source sha256[:16] | %s |" % rec["kernel_source_sha256_16"]]
    return "\n".join(md) + "\n"


def _stats_us(stats_csv):
    out = {}
    for r in csv.DictReader(open(stats_csv)):
        out[r["Name"]] = (int(r["Calls"]), float(r["AverageNs"]) / 1e3)
    return out


def kernels(fetch_csv, write_csv, stats_csv, title, command):
    """Per-kernel HBM bytes (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by the calibration
    copy) and the rate they imply over each kernel's average duration, for the library's kernels.
    `command` is the counter runs' command (COUNTER for the counter name), then " ;; " and the
    kernel-trace run's command."""
    pmc_cmd, _, stats_cmd = command.partition(" ;; ")
    fetch, write = _per_kernel(fetch_csv), _per_kernel(write_csv)
    f_cal = max((max(v) for k, v in fetch.items() if "copyBuffer" in k or "copy_kernel" in k))
    w_cal = max((max(v) for k, v in write.items() if "copyBuffer" in k or "copy_kernel" in k))
    f_scale, w_scale = CALIB_BYTES / (f_cal * 1024.0), CALIB_BYTES / (w_cal * 1024.0)
    st = _stats_us(stats_csv)
    out = ["# HBM traffic per kernel: %s" % title, "",
           "Commands (run from /tmp with TMPDIR=/tmp on one MI355X; repository at $R):", "",
           "    " + pmc_cmd.replace("COUNTER", "FETCH_SIZE"),
           "    " + pmc_cmd.replace("COUNTER", "WRITE_SIZE"),
           "    " + (stats_cmd or pmc_cmd.replace("--pmc COUNTER", "--kernel-trace --stats")), "",
           "FETCH_SIZE and WRITE_SIZE are KiB per dispatch between L2 and the memory fabric; each is "
           "scaled by what it reads for the benchmark's untimed 256 MiB device copy (fetch x%.3f, "
           "write x%.3f). Durations are the kernel-trace averages of the last command." %
           (f_scale, w_scale), "",
           "| kernel | dispatches | avg us | read MB | written MB | GB/s |", "|---|---|---|---|---|---|"]
    rows = []
    for name, fv in fetch.items():
        if "moe::" not in name:
            continue
        wv = write.get(name, [0.0])
        fb = sum(fv) / len(fv) * 1024.0 * f_scale
        wb = sum(wv) / len(wv) * 1024.0 * w_scale
        calls, us = st.get(name, (len(fv), float("nan")))
        rows.append((us * calls, name, len(fv), us, fb, wb))
    for _, name, n, us, fb, wb in sorted(rows, reverse=True):
        sn = short_name(name)
        if len(sn) > 90:
            sn = sn[:87] + "..."
        out.append("| `%s` | %d | %.1f | %.1f | %.1f | %.0f |" % (
            sn, n, us, fb / 1e6, wb / 1e6, (fb + wb) / (us * 1e-6) / 1e9 if us > 0 else 0.0))
    return "\n".join(out) + "\n"


def mfma(pmc_csvs, stats_csv, kernel, title, command):
    """Matrix-core busy fraction and clock of one kernel: SQ_VALU_MFMA_BUSY_CYCLES is summed over
    the 1024 SIMDs, GRBM_GUI_ACTIVE over the 8 XCDs, so busy = MFMA_BUSY / GUI_ACTIVE / 128; the
    clock is GUI_ACTIVE / 8 over the kernel's average duration."""
    vals = collections.defaultdict(list)
    for path in pmc_csvs.split(","):
        for r in csv.DictReader(open(path)):
            if kernel in r["Kernel_Name"]:
                vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    st = _stats_us(stats_csv)
    us = [t for n, (c, t) in st.items() if kernel in n]
    us = us[0] if us else float("nan")
    out = ["# Matrix-core counters: %s, `%s`" % (title, kernel), "",
           "Commands (run from /tmp with TMPDIR=/tmp on one MI355X; repository at $R):", ""]
    out += ["    " + c for c in command.split(" ;; ")]
    out += ["", "| counter (per dispatch) | value |", "|---|---|"]
    for k in sorted(avg):
        out.append("| %s | %.4g |" % (k, avg[k]))
    if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg:
        busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / avg["GRBM_GUI_ACTIVE"] / 128.0
        out.append("| matrix cores busy (MFMA_BUSY / GUI_ACTIVE / 128) | %.1f%% |" % (100 * busy))
        clk = avg["GRBM_GUI_ACTIVE"] / 8.0 / (us * 1e-6) / 1e6
        out.append("| clock (GUI_ACTIVE / 8 / %.1f us) | %.0f MHz |" % (us, clk))
    if "SQ_WAVE_CYCLES" in avg:
        for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS"):
            if c in avg:
                out.append("| %s / SQ_WAVE_CYCLES | %.1f%% |" % (c, 100 * avg[c] / avg["SQ_WAVE_CYCLES"]))
    return "\n".join(out) + "\n"


def main(argv):
    if len(argv) >= 4 and argv[0] == "stats":
        sys.stdout.write(stats(argv[1], argv[2], " ".join(argv[3:])))
    elif len(argv) >= 7 and argv[0] == "traffic":
        sys.stdout.write(traffic(argv[1], argv[2], argv[3], argv[4], argv[5], " ".join(argv[6:])))
    elif len(argv) >= 6 and argv[0] == "kernels":
        sys.stdout.write(kernels(argv[1], argv[2], argv[3], argv[4], " ".join(argv[5:])))
    elif len(argv) >= 6 and argv[0] == "mfma":
        sys.stdout.write(mfma(argv[1], argv[2], argv[3], argv[4], " ".join(argv[5:])))
    else:
        sys.stderr.write(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
