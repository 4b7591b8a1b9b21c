"""Host arithmetic of bench.py's counter summaries, on synthetic rocprofv3 CSVs.

The summaries turn per-dispatch counter rows into the figures the profiles quote: the
copy calibration factor, HBM bytes per decode call, and for prefill the clock from
GRBM_GUI_ACTIVE per XCD, the MFMA-busy fraction, the bank-conflict share and the L2 hit
rate.  Each expected value below is worked out by hand from the rows written here.
"""

import csv
import json
import os
import re

import pytest

import bench

COLS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value",
        "Start_Timestamp", "End_Timestamp"]


def write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(COLS, r)))


def write_agent(path, simds=1024, xcc=8):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Simd_Count", "Num_Xcc"])
        w.writeheader()
        w.writerow({"Name": "gfx950", "Simd_Count": simds, "Num_Xcc": xcc})


def test_decode_summary_calibrates_and_sums_per_call(tmp_path, monkeypatch):
    out = tmp_path / "decode.json"
    monkeypatch.setattr(bench, "COUNTERS", str(out))
    copy_kib = bench.COPY_BYTES / 2 / 1024          # FETCH_SIZE reads the copy as half its bytes
    fetch = [(1, "void at::native::neg_kernel", 1, "FETCH_SIZE", copy_kib, 0, 1)]
    write = [(1, "void at::native::neg_kernel", 1, "WRITE_SIZE", bench.COPY_BYTES / 1024, 0, 1)]
    # two decode calls: stream-K + fixup each; counters split over two rows per dispatch
    did = 2
    for _ in range(2):
        for name, kib in (("nkv::decode_streamk_kernel<128, 4>", 1000.0), ("nkv::decode_fixup_kernel<128, 4>", 10.0)):
            fetch += [(did, name, 1, "FETCH_SIZE", kib / 2, 0, 1), (did, name, 1, "FETCH_SIZE", kib / 2, 0, 1)]
            write += [(did, name, 1, "WRITE_SIZE", kib / 10, 0, 1)]
            did += 1
    write_csv(tmp_path / "f.csv", fetch)
    write_csv(tmp_path / "w.csv", write)
    bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    c = json.loads(out.read_text())
    assert c["fetch"]["factor"] == pytest.approx(2.0)
    assert c["write"]["factor"] == pytest.approx(1.0)
    assert c["fetch"]["decode_calls"] == 2
    assert c["fetch"]["bytes_per_call"] == int(1010.0 * 1024 * 2.0)
    assert c["write"]["bytes_per_call"] == int(101.0 * 1024 * 1.0)
    assert c["hbm_bytes_per_decode_call"] == int(1010.0 * 1024 * 2.0 + 101.0 * 1024)


def test_prefill_summary_derived_figures(tmp_path, monkeypatch):
    out = tmp_path / "prefill.md"
    monkeypatch.setattr(bench, "PREFILL_COUNTERS", str(out))
    monkeypatch.setattr(bench, "PREFILL_COUNTERS_JSON", str(tmp_path / "prefill.json"))
    c3, c4 = bench.PREFILL_GRIDS["C3"], bench.PREFILL_GRIDS["C4"]
    k = "void nkv::prefill_bf16_kernel<128, 4, 8>(...)"
    dur_ns = {c3: 400_000, c4: 200_000}               # 400 us and 200 us per dispatch
    gui = {c3: 8 * 800_000, c4: 8 * 420_000}          # summed over 8 XCDs: 2000 and 2100 MHz
    busy = {c3: 1024 * 800_000 * 0.35, c4: 1024 * 420_000 * 0.40}
    passes = [[], [], []]
    did = 1
    passes[2].append((did, "void at::native::neg_kernel", 1, "FETCH_SIZE", bench.COPY_BYTES / 2 / 1024, 0, 1))
    did += 1
    for grid in (c3, c4):
        for call in range(6):                          # the first 2 of each leg are dropped
            warm = 5.0 if call < 2 else 1.0            # warm-up values that must not count
            t0 = 1_000_000 * did
            t1 = t0 + dur_ns[grid]
            passes[0] += [(did, k, grid, "SQ_VALU_MFMA_BUSY_CYCLES", busy[grid] * warm, t0, t1),
                          (did, k, grid, "GRBM_GUI_ACTIVE", gui[grid], t0, t1),
                          (did, k, grid, "SQ_VALU_MFMA_COEXEC_CYCLES", busy[grid] * 0.25, t0, t1)]
            passes[1] += [(did, k, grid, "SQ_LDS_BANK_CONFLICT", 30.0, t0, t1),
                          (did, k, grid, "SQ_LDS_IDX_ACTIVE", 120.0, t0, t1),
                          (did, k, grid, "TCC_HIT_sum", 600.0, t0, t1),
                          (did, k, grid, "TCC_MISS_sum", 400.0, t0, t1)]
            passes[2] += [(did, k, grid, "FETCH_SIZE", 100_000.0, t0, t1)]
            did += 1
    paths = []
    for i, rows in enumerate(passes):
        d = tmp_path / f"p{i}"
        d.mkdir()
        write_csv(d / "pass_counter_collection.csv", rows)
        write_agent(d / "pass_agent_info.csv")
        paths.append(str(d / "pass_counter_collection.csv"))
    bench.summarize_prefill_counters(paths)
    text = out.read_text()

    def row(label):
        m = re.search(r"^\| " + re.escape(label) + r"[^|]*\| ([^|]+) \| ([^|]+) \|$", text, re.M)
        assert m, label
        return m.group(1).strip(), m.group(2).strip()

    assert row("shader clock, MHz") == ("2,000", "2,100")
    assert row("MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES") == ("0.350", "0.400")
    assert row("VALU-MFMA co-execution / MFMA busy") == ("0.250", "0.250")
    assert row("LDS bank conflicts / LDS active") == ("0.250", "0.250")
    assert row("L2 hit rate") == ("0.600", "0.600")
    assert row("bytes read from beyond L2") == ("204.8 MB", "204.8 MB")
    tf3 = bench.PREFILL_FLOP["C3"] / 400.0 / 1e6
    assert row("TFLOP/s in the counted dispatches")[0] == f"{tf3:,.1f}"
    assert row("duration_us") == ("400.00", "200.00")


def test_prefill_summary_writes_the_roofline_record(tmp_path, monkeypatch):
    # the JSON record beside the markdown: per-leg MFMA busy, co-execution share, clock and
    # calibrated FETCH bytes, tagged with the prefill sources' sha
    monkeypatch.setattr(bench, "PREFILL_COUNTERS", str(tmp_path / "prefill.md"))
    monkeypatch.setattr(bench, "PREFILL_COUNTERS_JSON", str(tmp_path / "prefill.json"))
    c3 = bench.PREFILL_GRIDS["C3"]
    k = "void nkv::prefill_bf16_kernel<128, 4, 8>(...)"
    passes = [[], [], [(1, "void at::native::neg_kernel", 1, "FETCH_SIZE", bench.COPY_BYTES / 4 / 1024, 0, 1)]]
    for did in range(2, 6):
        t0, t1 = 1_000_000 * did, 1_000_000 * did + 500_000          # 500 us
        passes[0] += [(did, k, c3, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1_000_000 * 0.5, t0, t1),
                      (did, k, c3, "GRBM_GUI_ACTIVE", 8 * 1_000_000, t0, t1),
                      (did, k, c3, "SQ_VALU_MFMA_COEXEC_CYCLES", 1024 * 1_000_000 * 0.1, t0, t1)]
        passes[1] += [(did, k, c3, "SQ_LDS_BANK_CONFLICT", 10.0, t0, t1),
                      (did, k, c3, "SQ_LDS_IDX_ACTIVE", 40.0, t0, t1)]
        passes[2] += [(did, k, c3, "FETCH_SIZE", 1000.0, t0, t1)]
    paths = []
    for i, rows in enumerate(passes):
        d = tmp_path / f"p{i}"
        d.mkdir()
        write_csv(d / "pass_counter_collection.csv", rows)
        write_agent(d / "pass_agent_info.csv")
        paths.append(str(d / "pass_counter_collection.csv"))
    bench.summarize_prefill_counters(paths)
    rec = json.loads((tmp_path / "prefill.json").read_text())
    assert rec["source_sha"] == bench.kernel_source_sha(bench.PREFILL_SOURCES)
    c = rec["legs"]["C3"]
    assert c["duration_us"] == 500.0 and c["clock_mhz"] == 2000
    assert c["mfma_busy"] == 0.5 and c["coexec_of_mfma_busy"] == 0.2
    assert c["lds_bank_conflict_share"] == 0.25
    assert c["fetch_bytes_per_call"] == 1000 * 1024 * 4          # the copy reads as a quarter
    assert rec["legs"]["C4"]["mfma_busy"] is None
    # the bench reads it back only for the same sources
    monkeypatch.setattr(bench, "PREFILL_COUNTERS_JSON", str(tmp_path / "prefill.json"))
    assert bench.prefill_counter_record(rec["source_sha"]) == rec
    assert bench.prefill_counter_record("0" * 16) is None
    r = bench.prefill_roofline("C3", 1000.0, 2.75e11, 275.0, rec)
    assert r["frac"] == 0.4 and r["mfma_busy"] == 0.5 and r["traffic"] == 1000 * 1024 * 4
    assert bench.prefill_roofline("C3", 1000.0, 2.75e11, 275.0, None)["traffic"] is None


def test_clock_sampler_reads_the_current_level():
    text = "0: 500Mhz\n1: 2400Mhz\nS: 2013Mhz *\n"
    assert bench.ClockSampler.parse(text) == 2013
    assert bench.ClockSampler.parse("0: 500Mhz *\n1: 2400Mhz\n") == 500
    assert bench.ClockSampler.parse("0: 500Mhz\n") is None
