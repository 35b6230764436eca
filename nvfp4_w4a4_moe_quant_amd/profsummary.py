"""Condense rocprofv3 output into short text summaries.

Kernel timing table from a kernel_stats.csv:

    python -m nvfp4_w4a4_moe_quant_amd.profsummary <kernel_stats.csv> [command]

HBM traffic per dispatch from two counter passes (FETCH_SIZE, then
WRITE_SIZE, both in KiB per dispatch), each scaled by the factor that the same
counter shows on a plain copy of known size (copycal: 3 copies of MiB MiB):

    python -m nvfp4_w4a4_moe_quant_amd.profsummary traffic \\
        <fetch.csv> <write.csv> <cal_fetch.csv> <cal_write.csv> <MiB> \\
        <kernel substring> <source file> <out.json> [command]

The JSON records the kernel, the raw and scaled byte counts, the factors and
the SHA-256 of the kernel's source file, so that a reader can tell whether the
counters still describe the current kernel.
"""
import collections
import csv
import hashlib
import json
import re
import sys


def short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    name = re.sub(r"^void ", "", name)
    return re.sub(r"\((?:[^()]|\([^()]*\))*\)$", "", name).strip()


def main(path, command=""):
    rows = list(csv.DictReader(open(path)))
    out = []
    if command:
        out.append(f"command: {command}")
    out.append(f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'%':>6s}")
    for r in rows:
        out.append(f"{short(r['Name'])[:60]:60s} {int(r['Calls']):6d} "
                   f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                   f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}")
    print("\n".join(out))


def counter_means(path, counter):
    """Mean counter value per kernel (short name) -> (dispatches, mean)."""
    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        vals[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: (len(v), sum(v) / len(v)) for k, v in vals.items()}


def calibration(path, counter, mib):
    """Factor = bytes one copy moves / counter bytes, taken on the copy's
    elementwise kernel (the dispatch that both reads and writes MiB)."""
    m = {k: v for k, v in counter_means(path, counter).items() if "elementwise" in k}
    name, (n, kib) = max(m.items(), key=lambda kv: kv[1][1])
    return name, kib, (mib * 1024.0) / kib


def traffic(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, mib, match, source, out_json,
            command=""):
    mib = float(mib)
    cf_name, cf_kib, f_fac = calibration(cal_fetch_csv, "FETCH_SIZE", mib)
    cw_name, cw_kib, w_fac = calibration(cal_write_csv, "WRITE_SIZE", mib)
    fetch = counter_means(fetch_csv, "FETCH_SIZE")
    write = counter_means(write_csv, "WRITE_SIZE")
    lines = []
    if command:
        lines.append(f"command: {command}")
    lines.append(f"calibration: copy of {mib:.0f} MiB ({cf_name}): FETCH_SIZE {cf_kib:.0f} KiB "
                 f"-> factor {f_fac:.4f}; WRITE_SIZE {cw_kib:.0f} KiB ({cw_name}) -> factor "
                 f"{w_fac:.4f}")
    lines.append(f"{'kernel':60s} {'n':>4s} {'fetch_MB':>10s} {'write_MB':>10s} (scaled, per dispatch)")
    rec = None
    for k in sorted(set(fetch) | set(write)):
        fb = fetch.get(k, (0, 0.0))[1] * 1024.0 * f_fac
        wb = write.get(k, (0, 0.0))[1] * 1024.0 * w_fac
        n = max(fetch.get(k, (0, 0))[0], write.get(k, (0, 0))[0])
        lines.append(f"{k[:60]:60s} {n:4d} {fb / 1e6:10.2f} {wb / 1e6:10.2f}")
        if match in k and (rec is None or fb + wb > rec["hbm_bytes"]):
            rec = dict(kernel=k, fetch_kib=fetch.get(k, (0, 0.0))[1],
                       write_kib=write.get(k, (0, 0.0))[1], fetch_factor=f_fac,
                       write_factor=w_fac, fetch_bytes=fb, write_bytes=wb, hbm_bytes=fb + wb)
    if rec is None:
        raise SystemExit(f"no kernel matches {match!r}")
    rec["source"] = source
    rec["source_sha256"] = hashlib.sha256(open(source, "rb").read()).hexdigest()
    rec["command"] = command
    json.dump(rec, open(out_json, "w"), indent=1)
    print("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "traffic":
        traffic(*sys.argv[2:10], command=" ".join(sys.argv[10:]))
    else:
        main(sys.argv[1], " ".join(sys.argv[2:]))
