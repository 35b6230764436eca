"""Host checks of the rocprofv3 summary tool (no GPU): the counter arithmetic
behind the committed profiles, on small hand-made CSV files whose expected
figures follow from the definitions by hand."""
import csv
import json

from nvfp4_w4a4_moe_quant_amd import profsummary as S

TRACE_HDR = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
PMC_HDR = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_mfma_summary(tmp_path, capsys):
    k = "void (anonymous namespace)::k_gemm<64, 256, true>(GemmParams)"
    other = "void (anonymous namespace)::k_quant<true>(float const*)"
    # two dispatches of 100 us each (timestamps in ns)
    _write(tmp_path / "t.csv", TRACE_HDR,
           [[k, 0, 100_000], [k, 200_000, 300_000], [other, 0, 5_000]])
    # per dispatch: GRBM_GUI_ACTIVE summed over 2 XCDs = 2 x 200000 cycles
    # -> 200000 cycles per XCD in 100 us = 2.0 GHz; 4 SIMDs busy 50% of them
    p1, p2 = [], []
    for d in ("1", "2"):
        p1 += [[d, k, "GRBM_GUI_ACTIVE", 200_000], [d, k, "GRBM_GUI_ACTIVE", 200_000],
               [d, k, "SQ_VALU_MFMA_BUSY_CYCLES", 400_000],
               [d, k, "SQ_VALU_MFMA_COEXEC_CYCLES", 100_000],
               [d, k, "SQ_WAVE_CYCLES", 1_000_000], [d, k, "SQ_ACTIVE_INST_VALU", 250_000],
               [d, k, "SQ_WAIT_ANY", 300_000]]
        p2 += [[d, k, "GRBM_GUI_ACTIVE", 400_000],
               [d, k, "SQ_INSTS_VALU_MFMA_MOPS_F16", 1_000_000],
               [d, k, "SQ_LDS_IDX_ACTIVE", 20_000], [d, k, "SQ_LDS_BANK_CONFLICT", 5_000]]
    p1.append(["3", other, "GRBM_GUI_ACTIVE", 1])
    _write(tmp_path / "p1.csv", PMC_HDR, p1)
    _write(tmp_path / "p2.csv", PMC_HDR, p2)
    S.mfma(str(tmp_path / "t.csv"), str(tmp_path / "p1.csv"), str(tmp_path / "p2.csv"), 2, 4,
           command="cmd")
    out = capsys.readouterr().out.splitlines()
    row = [l for l in out if l.startswith("k_gemm")]
    assert len(row) == 1 and "k_quant" not in "\n".join(out[2:-1])
    f = row[0].split()[-10:]
    # us, GHz, MFMA% (400000 / (200000 * 4)), co-exec% (100000 / 400000),
    # GFLOP (1e6 * 512), TF/s (5.12e8 / 100 us), VALU%, wait%,
    # LDS% (20000 / (200000 * 4 / 4)), bank% (5000 / 20000)
    assert f == ["100.0", "2.00", "50.0", "25.0", "0.5", "5", "25.0", "30.0", "10.0", "25.0"]


def test_traffic_scaling(tmp_path, capsys):
    k = "void (anonymous namespace)::k_gemm<64, 256, true, true, true>(GemmParams)"
    cp = "void at::native::vectorized_elementwise_kernel<4, add>(int)"  # the copy
    # calibration: a 1 MiB copy reads 512 KiB by FETCH_SIZE (factor 2) and
    # writes 1024 KiB by WRITE_SIZE (factor 1)
    _write(tmp_path / "cf.csv", PMC_HDR, [["1", cp, "FETCH_SIZE", 512.0]])
    _write(tmp_path / "cw.csv", PMC_HDR, [["1", cp, "WRITE_SIZE", 1024.0]])
    _write(tmp_path / "f.csv", PMC_HDR, [["1", k, "FETCH_SIZE", 100.0],
                                         ["2", k, "FETCH_SIZE", 300.0]])
    _write(tmp_path / "w.csv", PMC_HDR, [["1", k, "WRITE_SIZE", 50.0],
                                         ["2", k, "WRITE_SIZE", 50.0]])
    src = tmp_path / "src.hip"
    src.write_text("kernel source\n")
    out_json = tmp_path / "t.json"
    S.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
              str(tmp_path / "cw.csv"), "1", "true, true, true", str(src), str(out_json))
    rec = json.load(open(out_json))
    # mean fetch 200 KiB x 2, write 50 KiB x 1
    assert abs(rec["fetch_bytes"] - 200 * 1024 * 2) < 1e-6
    assert abs(rec["write_bytes"] - 50 * 1024) < 1e-6
    assert abs(rec["hbm_bytes"] - (400 + 50) * 1024) < 1e-6
    assert len(rec["source_sha256"]) == 64


def test_kernel_stats_summary(tmp_path, capsys):
    hdr = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
           "StdDev"]
    _write(tmp_path / "s.csv", hdr, [
        ["void (anonymous namespace)::k_gemm<64, 256, true>((anonymous namespace)::GemmParams)",
         13, 6020773, 463136.4, 13.6, 436500, 486853, 1.0],
        ["(anonymous namespace)::k_amax(void const*, int, long, long, long, float*)",
         2, 9000, 4500.0, 0.1, 4000, 5000, 1.0]])
    S.main(str(tmp_path / "s.csv"), command="cmd x")
    out = capsys.readouterr().out.splitlines()
    assert out[0] == "command: cmd x"
    # names lose the namespace, the leading "void" and the argument list
    assert out[2].split()[:3] == ["k_gemm<64,", "256,", "true>"]
    assert out[2].split()[-5:] == ["13", "463.14", "436.50", "486.85", "13.60"]
    assert out[3].split() == ["k_amax", "2", "4.50", "4.00", "5.00", "0.10"]


def test_valu_ceiling(tmp_path, capsys):
    """Quantizer ceiling rows: clock, VALU issue time, scaled bytes, copy-rate
    memory time and the fraction, by hand from the definitions."""
    q = "void (anonymous namespace)::k_quant<true, true, 0>(void const*)"
    cp = "void at::native::vectorized_elementwise_kernel<4, add>(int)"
    TR = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y",
          "Grid_Size_Z"]
    PM = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    # two quantize dispatches on different grids (X and H): 50 us and 100 us
    _write(tmp_path / "t.csv", TR, [[q, 0, 50_000, 1024, 4, 1], [q, 0, 100_000, 1024, 8, 1]])
    # grid 4096: GRBM_GUI_ACTIVE 2 XCDs x 100000 -> 100000 cycles in 50 us = 2 GHz;
    # 1e6 VALU instructions x 4 cycles / (4 SIMDs x 2e9) = 500 us ... scaled below
    _write(tmp_path / "v.csv", PM, [
        ["1", q, 4096, "GRBM_GUI_ACTIVE", 100_000], ["1", q, 4096, "GRBM_GUI_ACTIVE", 100_000],
        ["1", q, 4096, "SQ_INSTS_VALU", 40_000],
        ["2", q, 8192, "GRBM_GUI_ACTIVE", 200_000], ["2", q, 8192, "GRBM_GUI_ACTIVE", 200_000],
        ["2", q, 8192, "SQ_INSTS_VALU", 20_000]])
    # bytes: grid 4096 fetch 1000 KiB x2 + write 500 KiB x1 = 2500 KiB
    _write(tmp_path / "f.csv", PM, [["1", q, 4096, "FETCH_SIZE", 1000.0],
                                    ["2", q, 8192, "FETCH_SIZE", 0.0]])
    _write(tmp_path / "w.csv", PM, [["1", q, 4096, "WRITE_SIZE", 500.0],
                                    ["2", q, 8192, "WRITE_SIZE", 0.0]])
    _write(tmp_path / "cf.csv", PMC_HDR, [["1", cp, "FETCH_SIZE", 512.0]])
    _write(tmp_path / "cw.csv", PMC_HDR, [["1", cp, "WRITE_SIZE", 1024.0]])
    # the 1 MiB copy (2 MiB moved) takes 1 us -> 2 MiB per us
    _write(tmp_path / "ct.csv", TR, [[cp, 0, 1_000, 256, 1, 1]])
    S.valu(*(str(tmp_path / n) for n in ("t.csv", "v.csv", "f.csv", "w.csv", "cf.csv",
                                         "cw.csv", "ct.csv")), "1", "2", "4")
    out = capsys.readouterr().out.splitlines()
    rows = [l.split() for l in out if l.startswith("k_quant")]
    assert len(rows) == 2
    r = {int(x[-10]): x[-9:] for x in rows}
    # grid 4096: 50 us, 2.00 GHz, 0.04 Minst, T_v = 40000*4/(4*2e9) = 20 us,
    # 2.56 MB = 2500 KiB, 51.2 GB/s... = 0.05 TB/s, T_m = 2500 KiB / 2 MiB/us
    # = 1.2 us, frac = 20 / 50 = 0.40
    assert r[4096] == ["1", "50.0", "2.00", "0.04", "20.0", "2.6", "0.05", "1.2", "0.40"]
    # grid 8192: 100 us, 2.00 GHz, T_v = 20000*4/(4*2e9) = 10 us, frac 0.10
    assert r[8192][:5] == ["1", "100.0", "2.00", "0.02", "10.0"]
    assert r[8192][-1] == "0.10"
