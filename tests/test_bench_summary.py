"""Host checks of bench.py's rocprofv3 summarizer on small synthetic csv files
(no GPU): the variants matcher pairs each variant with its own dispatches and
refuses a run whose dispatches do not fit the bench's record."""
import csv
import json
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

TRACE_COLS = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp",
              "VGPR_Count", "Workgroup_Size_X", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
PMC_COLS = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "VGPR_Count", "Counter_Name",
            "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _kname(k):
    return f"void rga::(anonymous namespace)::{k}(int const*, long)"


def _run(variants, cold_reps):
    """(kernel, grid) per dispatch of a run: a flush before each cold call,
    torch's own kernels between the variants, as the bench issues them."""
    seq = [("gate_add_full_kernel<0>", 4096)] * 7   # earlier parts of the run
    for _, k, g in variants:
        seq.append(("void at::native::fill_kernel", 64))
        for _ in range(cold_reps):
            seq.append(("read_kernel", 262144))
            seq.append((k, g))
        seq.extend([(k, g)] * 100)
    return seq


def _write_trace(path, seq, us_of):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(TRACE_COLS)
        t = 1000
        for i, (k, g) in enumerate(seq, 1):
            name = _kname(k) if not k.startswith("void at::") else k
            d = int(us_of(k) * 1000)
            w.writerow(["KERNEL_DISPATCH", i, name, t, t + d, 32, 64, g, 1, 1])
            t += d + 10


def _write_pmc(path, seq, counter, value_of):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(PMC_COLS)
        for i, (k, g) in enumerate(seq, 1):
            name = _kname(k) if not k.startswith("void at::") else k
            w.writerow([i, g, name, 32, counter, value_of(k), 0, 1000])


def _bench_line(path, variants, cold_reps):
    v = {name: {"kernel": kern.split("<")[0], "bytes": 2 ** 20, "cold_reps": cold_reps,
                "warm_reps": 100, "cold_us_median": 10.0, "back_to_back_us": 9.0,
                "frac_of_hbm_peak": 0.5} for name, kern, _ in variants}
    with open(path, "w") as f:
        f.write("[bench] log line\n")
        f.write(json.dumps({"variants": v}) + "\n")


VARIANTS = [("a_rms_[2,16,64]", "rms_modulate_kernel<8, 0, 0, true>", 2048),
            ("b_rms_[2,16,64]", "rms_modulate_kernel<8, 0, 0, true>", 2048),
            ("c_gate_[1,8,128]", "gate_add_bcast_kernel<1>", 1024)]


def test_variants_trace_pairs_each_variant_with_its_calls(tmp_path, capsys):
    seq = _run(VARIANTS, 3)
    _write_trace(tmp_path / "t.csv", seq, lambda k: 5.0 if "rms" in k else 2.0)
    _bench_line(tmp_path / "b.json", VARIANTS, 3)
    bench.summarize(["variants", str(tmp_path / "b.json"), str(tmp_path / "t.csv")])
    out = capsys.readouterr().out
    lines = [l for l in out.splitlines() if l.startswith(("a_", "b_", "c_"))]
    assert [l.split()[0] for l in lines] == [v[0] for v in VARIANTS]
    assert "rms_modulate_kernel<8, 0, 0, true>" in lines[0]
    assert "gate_add_bcast_kernel<1>" in lines[2] and " 1024 " in lines[2]
    # the bench's cold and b2b, then the trace's own cold median and b2b mean
    assert lines[0].split()[-5:] == ["10.00", "9.00", "5.00", "5.00", "0.5000"]
    assert lines[2].split()[-5:] == ["10.00", "9.00", "2.00", "2.00", "0.5000"]


def test_variants_counters_scale_by_the_copy(tmp_path, capsys):
    seq = [("copy_kernel", bench.FLUSH_BYTES // 16)] + _run(VARIANTS, 2)
    # FETCH_SIZE in KiB; the copy's reads half the true bytes (scale 2)
    fetch = lambda k: (bench.FLUSH_BYTES / 2048 if k == "copy_kernel" else 512)
    _write_pmc(tmp_path / "f.csv", seq, "FETCH_SIZE", fetch)
    _write_pmc(tmp_path / "w.csv", seq, "WRITE_SIZE",
               lambda k: bench.FLUSH_BYTES / 1024 if k == "copy_kernel" else 1024)
    _bench_line(tmp_path / "b.json", VARIANTS, 2)
    bench.summarize(["variants", str(tmp_path / "b.json"), str(tmp_path / "f.csv"),
                     str(tmp_path / "w.csv")])
    out = capsys.readouterr().out
    assert "FETCH_SIZE scale 2.00000" in out
    line = next(l for l in out.splitlines() if l.startswith("a_rms"))
    read_b, write_b, ratio = line.split()[-3:]
    assert int(read_b) == 512 * 1024 * 2 and int(write_b) == 1024 * 1024
    assert float(ratio) == pytest.approx(2.0)


def test_variants_refuse_a_mismatched_run(tmp_path):
    seq = _run(VARIANTS, 3)
    seq[-50] = ("gate_add_full_kernel<0>", 1024)   # a foreign launch inside the last variant
    _write_trace(tmp_path / "t.csv", seq, lambda k: 1.0)
    _bench_line(tmp_path / "b.json", VARIANTS, 3)
    with pytest.raises(SystemExit, match="do not match"):
        bench.summarize(["variants", str(tmp_path / "b.json"), str(tmp_path / "t.csv")])
    # the bench named another kernel than the one the dispatches ran
    bad = [VARIANTS[0], VARIANTS[1], ("c_gate_[1,8,128]", "gate_add_full_kernel<1>", 1024)]
    _write_trace(tmp_path / "t.csv", _run(VARIANTS, 3), lambda k: 1.0)
    _bench_line(tmp_path / "b.json", bad, 3)
    with pytest.raises(SystemExit, match="the bench names"):
        bench.summarize(["variants", str(tmp_path / "b.json"), str(tmp_path / "t.csv")])
