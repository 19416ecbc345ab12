"""The rocprof harness's host logic on synthetic rocprofv3 CSV files (no GPU):
command shape, parsing, the copy calibration of the byte counters, the MFMA
busy share and the traffic line that bench.py reads back."""
import csv
import os

import pytest

import bench
import rocprof_harness as rh

FWD = "void sdpa::(anonymous namespace)::fwd_bf16_kernel<64, 64, 64, 4, 1, false, false, false>(sdpa::bf16k::KParams)"
COPY = "__amd_rocclr_copyBuffer"


def write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_ALL)
        w.writerow(header)
        w.writerows(rows)


def counter_rows(entries):
    """entries: (dispatch, kernel, counter, value)"""
    hdr = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    return hdr, [[i, d, 1, k, c, v] for i, (d, k, c, v) in enumerate(entries)]


def test_commands_put_the_program_after_the_separator_and_keep_counters_apart(tmp_path):
    for kind in ("trace", "mfma", "fetch", "write"):
        argv, out = rh.pass_command(kind, "encoder_d64", "forward", str(tmp_path), 50, 60)
        assert argv[0] == "rocprofv3"
        sep = argv.index("--")
        assert argv[sep + 1:sep + 3] == ["python3", "bench.py"]
        prof = argv[1:sep]
        if "--pmc" in prof:
            assert not ({"--kernel-trace", "--stats", "-s", "--sys-trace", "-r", "--runtime-trace"} & set(prof))
            assert len([a for a in prof[prof.index("--pmc") + 1:] if a.isupper()]) <= 4
        if kind in ("fetch", "write"):
            assert "--copy-calibration-mib" in argv
        assert "--no-cpu-baseline" in argv and "--no-configs" in argv


def test_trace_parsing_and_timed_dispatches(tmp_path):
    hdr = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    rows = [["KERNEL_DISPATCH", i + 1, FWD, 1000 * i, 1000 * i + (900 if i < 3 else 500)] for i in range(8)]
    rows.append(["KERNEL_DISPATCH", 99, COPY, 0, 5])
    write_csv(tmp_path / "run_kernel_trace.csv", hdr, rows)
    d = rh.dispatch_durations(rh.read_csv(rh.find(str(tmp_path), "_kernel_trace.csv")), rh.LEG_KERNELS["forward"])
    assert list(d) == [FWD] and d[FWD][:3] == [900] * 3 and d[FWD][3:] == [500] * 5


def test_copy_calibration_and_traffic_bytes(tmp_path):
    # a 1 GiB copy reads FETCH_SIZE = 512 Mi KiB-units / 2 (the counter counts half)
    gib_kib = 1 << 20
    f_dir, w_dir = tmp_path / "fetch", tmp_path / "write"
    f_dir.mkdir(), w_dir.mkdir()
    hdr, rows = counter_rows([(1, COPY, "FETCH_SIZE", gib_kib / 2), (2, COPY, "FETCH_SIZE", gib_kib / 2),
                              (3, COPY, "FETCH_SIZE", 10.0), (4, FWD, "FETCH_SIZE", 1000.0),
                              (5, FWD, "FETCH_SIZE", 1000.0)])
    write_csv(f_dir / "run_counter_collection.csv", hdr, rows)
    hdr, rows = counter_rows([(1, COPY, "WRITE_SIZE", gib_kib), (4, FWD, "WRITE_SIZE", 300.0)])
    write_csv(w_dir / "run_counter_collection.csv", hdr, rows)
    disp = rh.counters_by_dispatch(rh.read_csv(str(f_dir / "run_counter_collection.csv")))
    factor, kib = rh.calibration(disp, "FETCH_SIZE", rh.COPY_MIB << 20)
    # mean of the three largest copy readings: (2 * 2^19 + 10) / 3
    assert kib == pytest.approx((gib_kib + 10.0) / 3)
    out = tmp_path / "profiles"
    out.mkdir()
    cmds = {"fetch": ["rocprofv3", "--pmc", "FETCH_SIZE"], "write": ["rocprofv3", "--pmc", "WRITE_SIZE"]}
    total = rh.write_traffic(str(out), "encoder_d64", "forward", cmds, {"fetch": str(f_dir), "write": str(w_dir)},
                             algorithmic_bytes=1.0e6)
    wf, _ = rh.calibration(rh.counters_by_dispatch(rh.read_csv(str(w_dir / "run_counter_collection.csv"))),
                           "WRITE_SIZE", rh.COPY_MIB << 20)
    assert wf == pytest.approx(1.0)
    expect = 1000.0 * 1024 * factor + 300.0 * 1024 * wf
    assert total == pytest.approx(expect)
    text = (out / "encoder_d64_hbm_traffic.md").read_text()
    assert f"kernel_source_sha256: {bench.kernel_source_hash()}" in text
    # bench.py reads the figure back while the kernel source is unchanged
    old = bench.PROFILES
    try:
        bench.PROFILES = str(out)
        assert bench.read_traffic("encoder_d64") == pytest.approx(expect, rel=1e-5)
    finally:
        bench.PROFILES = old


def test_mfma_busy_share_and_clock(tmp_path):
    hdr, rows = counter_rows([(7, FWD, "GRBM_GUI_ACTIVE", 8 * 1e6), (7, FWD, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 6e5),
                              (7, FWD, "SQ_BUSY_CYCLES", 1.0), (7, FWD, "SQ_INSTS_MFMA", 10.0)])
    write_csv(tmp_path / "run_counter_collection.csv", hdr, rows)
    write_csv(tmp_path / "run_agent_info.csv", ["Agent_Type", "Simd_Count", "Num_Xcc", "Name"],
              [["CPU", 0, 1, "cpu"], ["GPU", 1024, 8, "gfx950"]])
    out = tmp_path / "p"
    out.mkdir()
    res = rh.write_mfma(str(out), "encoder_d64", "forward", ["rocprofv3"], str(tmp_path), {FWD: 500e3})
    assert res[FWD]["busy"] == pytest.approx(0.6)
    assert res[FWD]["cycles"] == pytest.approx(1e6)
    assert res[FWD]["flops"] == pytest.approx(10 * 32 * 32 * 16 * 2)
    assert "2.00 GHz" in (out / "encoder_d64_mfma_util.md").read_text()   # 1e6 cycles in 500 us
    # a short kernel: the counter pass's own cycles dominate, no clock given
    rh.write_mfma(str(out), "encoder_d64", "forward", ["rocprofv3"], str(tmp_path), {FWD: 5e3})
    assert "n/a" in (out / "encoder_d64_mfma_util.md").read_text()


def test_bench_json_is_found_among_other_output():
    assert rh.bench_json("noise\n{\"metric\": \"m\", \"value\": 1}\n[bench] x\n")["value"] == 1
    assert rh.bench_json("no json here") is None


def test_each_leg_hashes_its_own_kernel_sources():
    # bench.py trusts the forward hash; the backward and decode summaries
    # carry the hash of the sources their kernels come from
    fwd = rh.kernel_source_hash("forward")
    assert fwd == bench.kernel_source_hash() == rh.kernel_source_hash("forward_ex")
    hashes = {fwd, rh.kernel_source_hash("backward"), rh.kernel_source_hash("decode")}
    assert len(hashes) == 3
    for rel in rh.LEG_SOURCES["backward"] + rh.LEG_SOURCES["decode"]:
        assert os.path.exists(os.path.join(rh.ROOT, rel)), rel
