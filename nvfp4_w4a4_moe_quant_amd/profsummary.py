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

Ceiling of the quantizer kernels (k_amax, k_quant, k_rank, k_residual,
k_zero_stats; one row per kernel and grid size, so the passes over X and H
stay apart): the larger of the VALU issue time of the counted instructions
and the time a plain copy kernel needs for the counted HBM bytes, against
the measured duration.  Inputs: the kernel trace, a counter pass with
GRBM_GUI_ACTIVE SQ_INSTS_VALU, the FETCH_SIZE and WRITE_SIZE passes and their
copy calibration (copycal), and a kernel trace of the calibration copy:

    python -m nvfp4_w4a4_moe_quant_amd.profsummary valu \
        <kernel_trace.csv> <valu_pass.csv> <fetch.csv> <write.csv> \
        <cal_fetch.csv> <cal_write.csv> <cal_trace.csv> <MiB> <XCDs> <SIMDs> [command]

Clock and matrix-core utilisation of the GEMM kernels from a kernel trace and
two counter passes (GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES
SQ_VALU_MFMA_COEXEC_CYCLES SQ_WAVE_CYCLES SQ_ACTIVE_INST_VALU SQ_WAIT_ANY, then
GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_F8
SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT):

    python -m nvfp4_w4a4_moe_quant_amd.profsummary mfma \\
        <kernel_trace.csv> <pass1.csv> <pass2.csv> <XCDs> <SIMDs> [command]
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


def _per_dispatch(path):
    """{kernel: {counter: [value per dispatch]}} from a counter_collection.csv
    (values summed over the rows of one dispatch)."""
    d = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(path)):
        key = r["Dispatch_Id"]
        names[key] = short(r["Kernel_Name"])
        d[key][r["Counter_Name"]] += float(r["Counter_Value"])
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for key, cs in d.items():
        for c, v in cs.items():
            out[names[key]][c].append(v)
    return out


def mfma(trace_csv, pass1_csv, pass2_csv, n_xcd, n_simd, command=""):
    """Clock, matrix-core utilisation and wait/LDS fractions per GEMM kernel:
    clock = GRBM_GUI_ACTIVE per XCD / kernel duration (kernel trace); MFMA
    busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x SIMDs);
    co-exec = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES (matrix-core
    cycles during which the SIMD also ran VALU work); executed MFMA FLOPs =
    (SQ_INSTS_VALU_MFMA_MOPS_F16 + _F8) x 512."""
    n_xcd, n_simd = int(n_xcd), int(n_simd)
    dur = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        dur[short(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    c1, c2 = _per_dispatch(pass1_csv), _per_dispatch(pass2_csv)
    med = lambda xs: sorted(xs)[len(xs) // 2]
    lines = [f"command: {command}"] if command else []
    lines.append(f"{'kernel':58s} {'n':>3s} {'us':>7s} {'GHz':>5s} {'MFMA%':>6s} {'coex%':>6s} "
                 f"{'GFLOP':>7s} {'TF/s':>6s} {'VALU%':>6s} {'wait%':>6s} {'LDS%':>5s} "
                 f"{'bank%':>6s}")
    for k in sorted(c1):
        if "gemm" not in k or k not in c2 or k not in dur:
            continue
        a = {c: med(v) for c, v in c1[k].items()}
        b = {c: med(v) for c, v in c2[k].items()}
        t = med(dur[k])
        gui = a["GRBM_GUI_ACTIVE"] / n_xcd
        flops = (b.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) +
                 b.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)) * 512
        lines.append(
            f"{k[:58]:58s} {len(c1[k]['GRBM_GUI_ACTIVE']):3d} {t:7.1f} {gui / t / 1e3:5.2f} "
            f"{100 * a['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui * n_simd):6.1f} "
            f"{100 * a['SQ_VALU_MFMA_COEXEC_CYCLES'] / max(a['SQ_VALU_MFMA_BUSY_CYCLES'], 1.0):6.1f} "
            f"{flops / 1e9:7.1f} "
            f"{flops / t / 1e6:6.0f} {100 * a['SQ_ACTIVE_INST_VALU'] / a['SQ_WAVE_CYCLES']:6.1f} "
            f"{100 * a['SQ_WAIT_ANY'] / a['SQ_WAVE_CYCLES']:6.1f} "
            f"{100 * b['SQ_LDS_IDX_ACTIVE'] / (gui * n_simd / 4):5.1f} "
            f"{100 * b['SQ_LDS_BANK_CONFLICT'] / max(b['SQ_LDS_IDX_ACTIVE'], 1.0):6.1f}")
    lines.append("columns: median over dispatches; MFMA% = matrix cores busy; coex% = share of "
                 "those cycles with VALU work running beside; VALU% and wait% "
                 "= SQ_ACTIVE_INST_VALU and SQ_WAIT_ANY over SQ_WAVE_CYCLES; LDS% = LDS "
                 "active cycles per CU; bank% = bank-conflict cycles over LDS active cycles")
    print("\n".join(lines))


def _by_grid(path, kind):
    """{(kernel, grid size): [per-dispatch values]} for a counter pass
    (kind = counter name) or a kernel trace (kind = None: durations in us)."""
    out = collections.defaultdict(list)
    if kind is None:
        for r in csv.DictReader(open(path)):
            g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            out[(short(r["Kernel_Name"]), g)].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        return out
    per = collections.defaultdict(float)
    meta = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != kind:
            continue
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
        meta[r["Dispatch_Id"]] = (short(r["Kernel_Name"]), int(r["Grid_Size"]))
    for d, v in per.items():
        out[meta[d]].append(v)
    return out


QUANT_KERNELS = ("k_amax", "k_quant", "k_rank", "k_residual", "k_zero_stats")
PEAK_CLOCK_HZ = 2.4e9  # MI355X peak engine clock


def valu(trace_csv, valu_csv, fetch_csv, write_csv, cal_fetch_csv, cal_write_csv,
         cal_trace_csv, mib, n_xcd, n_simd, command=""):
    """Per quantizer kernel and grid size (medians over dispatches):
    clock f = GRBM_GUI_ACTIVE per XCD / duration, at most the chip's 2.4
    GHz (for kernels of a few tens of microseconds the GUI-active count
    also covers the counter collection around the dispatch, which would put
    f above the peak); VALU issue time
    T_v = SQ_INSTS_VALU x 4 cycles / (SIMDs x f) (a wave64 VALU instruction
    occupies a 16-lane SIMD for 4 cycles; FP64 and transcendental
    instructions take longer, so T_v is a lower bound); HBM bytes from the
    scaled FETCH_SIZE + WRITE_SIZE; T_m = bytes / B_copy with B_copy the
    bytes per second of the calibration copy (2 x MiB per dispatch over its
    traced duration); ceiling = max(T_v, T_m); frac = ceiling / duration."""
    mib, n_xcd, n_simd = float(mib), int(n_xcd), int(n_simd)
    med = lambda xs: sorted(xs)[len(xs) // 2]
    _, _, f_fac = calibration(cal_fetch_csv, "FETCH_SIZE", mib)
    _, _, w_fac = calibration(cal_write_csv, "WRITE_SIZE", mib)
    copy_us = max((med(v) for k, v in _by_grid(cal_trace_csv, None).items()
                   if "elementwise" in k[0] and "add" in k[0].lower()), default=None)
    if copy_us is None:
        copy_us = max(med(v) for v in _by_grid(cal_trace_csv, None).values())
    b_copy = 2.0 * mib * (1 << 20) / (copy_us * 1e-6)  # bytes per second
    dur = _by_grid(trace_csv, None)
    gui, insts = _by_grid(valu_csv, "GRBM_GUI_ACTIVE"), _by_grid(valu_csv, "SQ_INSTS_VALU")
    fetch, write = _by_grid(fetch_csv, "FETCH_SIZE"), _by_grid(write_csv, "WRITE_SIZE")
    lines = [f"command: {command}"] if command else []
    lines.append(f"copy calibration: {2 * mib:.0f} MiB moved in {copy_us:.1f} us = "
                 f"{b_copy / 1e12:.2f} TB/s; FETCH_SIZE x{f_fac:.4f}, WRITE_SIZE x{w_fac:.4f}")
    lines.append(f"{'kernel':24s} {'grid':>8s} {'n':>3s} {'us':>7s} {'GHz':>5s} {'VALU_Minst':>10s} "
                 f"{'T_valu':>7s} {'MB':>8s} {'TB/s':>5s} {'T_mem':>7s} {'frac':>5s}")
    for key in sorted(dur):
        name, grid = key
        if not name.startswith(QUANT_KERNELS) or key not in gui or key not in insts:
            continue
        t = med(dur[key])
        f = min(med(gui[key]) / n_xcd / (t * 1e-6), PEAK_CLOCK_HZ)
        tv = med(insts[key]) * 4.0 / (n_simd * f) * 1e6
        nbytes = (med(fetch[key]) * 1024.0 * f_fac if key in fetch else 0.0) + \
                 (med(write[key]) * 1024.0 * w_fac if key in write else 0.0)
        tm = nbytes / b_copy * 1e6
        lines.append(f"{name[:24]:24s} {grid:8d} {len(dur[key]):3d} {t:7.1f} {f / 1e9:5.2f} "
                     f"{med(insts[key]) / 1e6:10.2f} {tv:7.1f} {nbytes / 1e6:8.1f} "
                     f"{nbytes / (t * 1e-6) / 1e12:5.2f} {tm:7.1f} {max(tv, tm) / t:5.2f}")
    lines.append("columns: medians over dispatches; GHz = measured clock, capped at 2.4; "
                 "T_valu = VALU issue time of the counted instructions at that clock; MB = "
                 "scaled HBM bytes; T_mem = those bytes at the calibration copy's rate; "
                 "frac = max(T_valu, T_mem) / us")
    print("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "traffic":
        traffic(*sys.argv[2:10], command=" ".join(sys.argv[10:]))
    elif len(sys.argv) > 1 and sys.argv[1] == "mfma":
        mfma(*sys.argv[2:7], command=" ".join(sys.argv[7:]))
    elif len(sys.argv) > 1 and sys.argv[1] == "valu":
        valu(*sys.argv[2:12], command=" ".join(sys.argv[12:]))
    else:
        main(sys.argv[1], " ".join(sys.argv[2:]))
