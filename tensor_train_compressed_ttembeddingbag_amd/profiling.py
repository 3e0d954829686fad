"""Summaries of rocprofv3 output for the committed measurement files under profiles/.

    python -m tensor_train_compressed_ttembeddingbag_amd.profiling stats DIR --out FILE.md \
        --title T --command C
        per-kernel table of a `rocprofv3 --kernel-trace --stats --output-format csv` run

    python -m tensor_train_compressed_ttembeddingbag_amd.profiling mfma DIR --trace TDIR \
        --kernels k_fwd,k_bwd --out FILE.txt --command C --trace-command C
        executed fp32 MFMA work per launch from SQ_INSTS_VALU_MFMA_F32 (16x16x4 f32:
        2048 flop per instruction) and SQ_INSTS_VALU_MFMA_MOPS_F32 (512 flop per unit),
        over the kernel's average duration in a separate --kernel-trace --stats run

    python -m tensor_train_compressed_ttembeddingbag_amd.profiling sq DIR [DIR ...] \
        --kernels k_fwd,k_bwd --out FILE.txt --command C [--command C ...]
        per-dispatch means of the SQ counters of several --pmc runs, with the ratios used to
        read them (time waiting, instructions per MFMA, LDS bank conflicts per LDS access)

    python -m tensor_train_compressed_ttembeddingbag_amd.profiling traffic \
        --kernel k_bwd --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
        --copy-bytes N --out FILE.txt --command-fetch C --command-write C
        HBM bytes per launch of one kernel from the FETCH_SIZE and WRITE_SIZE counters
        (KiB per dispatch), each scaled by the factor that turns the same counter's
        reading for a plain device copy of N bytes into N

The traffic file also records a digest of the library's HIP sources; bench.py reports
the traffic only while the sources still have that digest.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))


def source_digest() -> str:
    """sha256 over the library's HIP sources and headers (the kernels measured)."""
    h = hashlib.sha256()
    root = os.path.dirname(PKG)
    files = sorted(glob.glob(os.path.join(PKG, "csrc", "*"))) + [os.path.join(root, "include",
                                                                             "tt_bag.h")]
    for f in files:
        if f.endswith((".hip", ".h")):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    """`void ttb::k_fwd<32>(ttb::DevArgs)` -> `k_fwd<32>`."""
    n = name.replace("(anonymous namespace)::", "").split("(")[0]
    n = re.sub(r"^void\s+", "", n)
    return n.replace("ttb::", "")


def _find(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, d))
    return sorted(hits)[0]


def kernel_stats(d: str):
    """Rows (kernel, calls, total_us, avg_us, percent) of a --stats run."""
    rows = []
    with open(_find(d, "kernel_stats.csv")) as fh:
        for r in csv.DictReader(fh):
            rows.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3,
                         float(r["AverageNs"]) / 1e3, float(r["Percentage"])))
    rows.sort(key=lambda x: -x[2])
    return rows


def counter_means(d: str):
    """{kernel (short name): {counter: mean value per dispatch}} of a --pmc run."""
    acc = {}
    with open(_find(d, "counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            k = _short(r["Kernel_Name"])
            acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    return {k: {c: statistics.fmean(v) for c, v in cs.items()} for k, cs in acc.items()}


def _copy_reading(d: str, counter: str) -> float:
    """The counter's mean reading for the largest device copy in a calibration run."""
    m = counter_means(d)
    best = None
    for k, cs in m.items():
        if counter in cs and (best is None or cs[counter] > best):
            best = cs[counter]
    if best is None:
        raise RuntimeError("no %s readings in %s" % (counter, d))
    return best


def _match(m: dict, kernel: str):
    ks = [k for k in m if k == kernel or k.startswith(kernel + "<")]
    if not ks:
        raise RuntimeError("kernel %s not in %s" % (kernel, sorted(m)))
    return m[ks[0]]


def cmd_stats(a):
    import json
    rows = kernel_stats(a.dir)
    ev = {}
    if a.bench:
        with open(a.bench) as fh:
            ev = json.loads(fh.readline()).get("kernels", {})
    out = ["# %s" % a.title, "", "Command (run from /tmp with TMPDIR=/tmp):", "",
           "    " + a.command, "",
           "rocprofv3 kernel statistics (durations in microseconds); the last column is the",
           "average bench.py measured for the same kernel with HIP events in its own run",
           "(`kernels` of its JSON line: %s):" % (a.bench_command or "-"), "",
           "| kernel | calls | total us | avg us | % | bench.py events avg us |",
           "|---|---|---|---|---|---|"]
    # bench.py's events cover the kernels of its timed loop: per base name, the variant
    # with the most calls (other template variants run outside the loop)
    top = {}
    for n, c, _, _, _ in rows:
        k = _short(n).split("<")[0]
        if k not in top or c > top[k][1]:
            top[k] = (n, c)
    for n, c, t, av, p in rows:
        k = _short(n).split("<")[0]
        e = ev.get(k, {}).get("avg_us") if top[k][0] == n else None
        out.append("| `%s` | %d | %.1f | %.2f | %.1f | %s |"
                   % (n, c, t, av, p, "%.2f" % e if e is not None else "-"))
    with open(a.out, "w") as fh:
        fh.write("\n".join(out) + "\n")
    print("\n".join(out))


def cmd_traffic(a):
    f = _match(counter_means(a.fetch), a.kernel)["FETCH_SIZE"]
    w = _match(counter_means(a.write), a.kernel)["WRITE_SIZE"]
    kib = a.copy_bytes / 1024.0
    ff = kib / _copy_reading(a.copy_fetch, "FETCH_SIZE")
    fw = kib / _copy_reading(a.copy_write, "WRITE_SIZE")
    traffic = (f * ff + w * fw) * 1024.0
    lines = [
        "kernel=%s" % a.kernel,
        "source_digest=%s" % source_digest(),
        "fetch_kib_per_dispatch=%.3f" % f,
        "write_kib_per_dispatch=%.3f" % w,
        "copy_bytes=%d" % a.copy_bytes,
        "fetch_factor=%.6f" % ff,
        "write_factor=%.6f" % fw,
        "traffic_bytes_per_launch=%.0f" % traffic,
        "command_fetch=%s" % a.command_fetch,
        "command_write=%s" % a.command_write,
        "command_copy_fetch=%s" % a.command_copy_fetch,
        "command_copy_write=%s" % a.command_copy_write,
    ]
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


PEAK_FP32_MFMA_TFLOPS = 157.3


def cmd_mfma(a):
    m = counter_means(a.dir)
    durs = {}
    for n, c, t, av, p in kernel_stats(a.trace):
        k = _short(n)
        if k not in durs or c > durs[k][1]:
            durs[k] = (av, c)
    lines = ["command=%s" % a.command, "trace_command=%s" % a.trace_command]
    for kern in a.kernels.split(","):
        cs = _match(m, kern)
        dk = [k for k in durs if k == kern or k.startswith(kern + "<")]
        dk = max(dk, key=lambda k: durs[k][1])
        us = durs[dk][0]
        inst = cs.get("SQ_INSTS_VALU_MFMA_F32", float("nan"))
        mops = cs.get("SQ_INSTS_VALU_MFMA_MOPS_F32", float("nan"))
        lines += ["kernel=%s" % dk,
                  "avg_us=%.3f" % us,
                  "mfma_f32_insts_per_launch=%.0f" % inst,
                  "mfma_mops_f32_per_launch=%.0f" % mops,
                  "executed_flop_from_insts=%.4g" % (inst * 2048.0),
                  "executed_flop_from_mops=%.4g" % (mops * 512.0),
                  "executed_tflops=%.3f" % (inst * 2048.0 / (us * 1e-6) / 1e12),
                  "executed_frac_of_fp32_mfma_peak=%.4f"
                  % (inst * 2048.0 / (us * 1e-6) / 1e12 / PEAK_FP32_MFMA_TFLOPS)]
        for c in sorted(cs):
            lines.append("%s=%.6g" % (c, cs[c]))
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_sq(a):
    m = {}
    for d in a.dirs:
        for k, cs in counter_means(d).items():
            m.setdefault(k, {}).update(cs)
    lines = ["command=%s" % c for c in a.command]
    for kern in a.kernels.split(","):
        cs = _match(m, kern)
        name = [k for k in m if k == kern or k.startswith(kern + "<")][0]
        lines.append("kernel=%s" % name)
        for c in sorted(cs):
            lines.append("%s=%.6g" % (c, cs[c]))
        g = cs.get
        if g("SQ_WAVE_CYCLES"):
            if g("SQ_WAIT_ANY") is not None:
                lines.append("ratio_wait_any_per_wave_cycle=%.3f"
                             % (g("SQ_WAIT_ANY") / g("SQ_WAVE_CYCLES")))
            if g("SQ_ACTIVE_INST_ANY") is not None:
                lines.append("ratio_active_inst_per_wave_cycle=%.3f"
                             % (g("SQ_ACTIVE_INST_ANY") / g("SQ_WAVE_CYCLES")))
        if g("SQ_INSTS_MFMA"):
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
                if g(c) is not None:
                    lines.append("ratio_%s_per_mfma=%.2f"
                                 % (c[9:].lower(), g(c) / g("SQ_INSTS_MFMA")))
        if g("SQ_INSTS_LDS") and g("SQ_LDS_BANK_CONFLICT") is not None:
            lines.append("ratio_lds_bank_conflict_cycles_per_lds_inst=%.2f"
                         % (g("SQ_LDS_BANK_CONFLICT") / g("SQ_INSTS_LDS")))
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_traffic(path: str, kernel: str):
    """Bytes per launch of `kernel` from a traffic file, or None when the file is
    missing, names another kernel, or was measured on other sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line:
                k, v = line.rstrip("\n").split("=", 1)
                kv[k] = v
    if kv.get("kernel") != kernel or kv.get("source_digest") != source_digest():
        return None
    return float(kv["traffic_bytes_per_launch"])


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--out", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--bench", default=None, help="bench.py JSON line with per-kernel events")
    s.add_argument("--bench-command", default=None)
    t = sub.add_parser("traffic")
    for k in ("kernel", "fetch", "write", "copy-fetch", "copy-write", "out", "command-fetch",
              "command-write", "command-copy-fetch", "command-copy-write"):
        t.add_argument("--" + k, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    sq = sub.add_parser("sq")
    sq.add_argument("dirs", nargs="+")
    sq.add_argument("--kernels", required=True)
    sq.add_argument("--out", required=True)
    sq.add_argument("--command", action="append", required=True)
    mm = sub.add_parser("mfma")
    mm.add_argument("dir")
    for k in ("trace", "kernels", "out", "command", "trace-command"):
        mm.add_argument("--" + k, required=True)
    sub.add_parser("digest")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        cmd_stats(a)
    elif a.cmd == "traffic":
        cmd_traffic(a)
    elif a.cmd == "mfma":
        cmd_mfma(a)
    elif a.cmd == "sq":
        cmd_sq(a)
    else:
        print(source_digest())


if __name__ == "__main__":
    sys.exit(main())
