"""Host logic of bench.py: the one-GPU refusal and the counter record built from rocprofv3
`--pmc` csv output (per-dispatch sums over counter dimensions, means over dispatches,
FETCH_SIZE and WRITE_SIZE scaled by the elementwise probe that moves 1 GiB each way, and
the record used only while the kernel sources hash the same)."""
import csv
import json
import os

import bench

PREFILL = "void (anonymous namespace)::prefill_fp8_kernel<1, 0>((anonymous namespace)::PrefillParams)"
PROBE = "void at::native::vectorized_elementwise_kernel<16, at::native::AUnaryFunctor<...>>"
OTHER = "(anonymous namespace)::quant_static_kernel((anonymous namespace)::QuantParams)"


def _pass(tmp_path, name, rows):
    """One rocprofv3 output directory: rows of (dispatch id, kernel, counter, value)."""
    d = tmp_path / name / "host" / "1234"
    d.mkdir(parents=True)
    with open(d / "p_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)
    return str(tmp_path / name)


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err


def test_counter_record(tmp_path):
    # pass 1: FETCH_SIZE of two prefill dispatches (each reported over two dimension
    # rows), the probe and an unrelated kernel; pass 2: WRITE_SIZE; pass 3: cycles
    p1 = _pass(tmp_path, "p1", [
        (1, PREFILL, "FETCH_SIZE", 100.0), (1, PREFILL, "FETCH_SIZE", 300.0),
        (2, PREFILL, "FETCH_SIZE", 250.0), (2, PREFILL, "FETCH_SIZE", 350.0),
        (3, PROBE, "FETCH_SIZE", 524288.0), (4, OTHER, "FETCH_SIZE", 7.0)])
    p2 = _pass(tmp_path, "p2", [
        (1, PREFILL, "WRITE_SIZE", 40.0), (2, PREFILL, "WRITE_SIZE", 60.0),
        (3, PROBE, "WRITE_SIZE", 1048576.0)])
    p3 = _pass(tmp_path, "p3", [
        (1, PREFILL, "GRBM_GUI_ACTIVE", 8000.0), (2, PREFILL, "GRBM_GUI_ACTIVE", 8016.0),
        (1, PREFILL, "SQ_VALU_MFMA_BUSY_CYCLES", 1024.0 * 500),
        (2, PREFILL, "SQ_VALU_MFMA_BUSY_CYCLES", 1024.0 * 700),
        (3, PROBE, "GRBM_GUI_ACTIVE", 1.0)])
    out = tmp_path / "rec.json"
    rec = bench.record_counters([p1, p2, p3], "C3", path=str(out))
    assert json.loads(out.read_text()) == rec
    # per-dispatch sums 400 and 600 KiB, mean 500; probe fetch reads half of 1 GiB: scale 2
    assert rec["fetch_size_kib"] == 500.0 and rec["fetch_scale"] == 2.0
    assert rec["write_size_kib"] == 50.0 and rec["write_scale"] == 1.0
    assert rec["hbm_bytes_per_launch"] == (500 * 2 + 50 * 1) * 1024
    assert rec["gfx_cycles_per_launch"] == 1001  # mean 8008 over the 8 XCDs
    assert rec["mfma_busy_cycles_per_simd"] == 600
    assert rec["kernel_hash"] == bench.kernel_source_hash()
    # the record serves only the kernel sources it was taken on
    assert bench.load_counters(rec["kernel_hash"], "C3", path=str(out)) == rec
    assert bench.load_counters("0" * 16, "C3", path=str(out)) == {}
    assert bench.load_counters(rec["kernel_hash"], "C3", path=str(tmp_path / "none.json")) == {}


def test_kernel_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    src = os.path.join(bench.ROOT, "fp8_mla_context_amd", "csrc")
    base = bench.kernel_source_hash()
    # a copy of the three hashed files, with a comment line and blank lines added
    root = tmp_path / "r"
    (root / "fp8_mla_context_amd" / "csrc").mkdir(parents=True)
    for fn in ("device_common.h", "mla_internal.h", "prefill_fp8.hip"):
        with open(os.path.join(src, fn)) as f:
            text = f.read()
        if fn == "prefill_fp8.hip":
            text = "// an added comment\n\n" + text.replace("\n", "\n\n", 3)
        (root / "fp8_mla_context_amd" / "csrc" / fn).write_text(text)
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.kernel_source_hash() == base
    # a code change does change it
    p = root / "fp8_mla_context_amd" / "csrc" / "prefill_fp8.hip"
    p.write_text(p.read_text() + "\nint an_added_symbol;\n")
    assert bench.kernel_source_hash() != base
