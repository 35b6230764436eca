"""Condense a rocprofv3 kernel_stats.csv into a short text table.

    python -m nvfp4_w4a4_moe_quant_amd.profsummary <kernel_stats.csv> [command]
"""
import csv
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


if __name__ == "__main__":
    main(sys.argv[1], " ".join(sys.argv[2:]))
