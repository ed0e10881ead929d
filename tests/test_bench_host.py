"""Host-side logic of bench.py that turns rocprofv3 databases into the committed
summaries: kernel-name cleanup and the matrix-core busy table (calibrated by
the fp32 probe). CPU only; the databases here are small synthetic stand-ins
with the columns rocprofv3 writes."""
import os
import shutil
import sqlite3
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_short_name_plain():
    nm = "void quip::(anonymous namespace)::ldl_block_kernel<64, 1>(float const*, long)"
    assert bench._short_name(nm) == "quip::ldl_block_kernel<64, 1>"


@pytest.mark.skipif(shutil.which("c++filt") is None, reason="c++filt not installed")
def test_short_name_demangles_float16_parameters():
    # a _Float16 parameter is mangled DF16_, which older demanglers reject
    nm = "_ZN4quip12_GLOBAL__N_115qmv_mfma_kernelILi2ELi2ELi3EEEvPKhllPKDF16_fPfjj"
    assert bench._short_name(nm) == "quip::qmv_mfma_kernel<2, 2, 3>"


def _counter_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (dispatch_id integer, kernel_name text, "
                "counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_mfma_busy_table_is_calibrated_by_the_fp32_probe(tmp_path):
    probe = "void quip::(anonymous namespace)::peak_mfma_f32_kernel(long, float, float*)"
    gemm = "void quip::(anonymous namespace)::gemm_kernel<128, 128, true, false, 0>(x)"
    fill = "void quip::(anonymous namespace)::fill_f32_kernel(float*, long, float)"
    rows = []
    # probe: 100 busy cycles per 1 active cycle; the GEMM: 50 per 1 (two
    # dispatches, counters split over two rows as per-block readings can be)
    rows += [(1, probe, "SQ_VALU_MFMA_BUSY_CYCLES", 1000.0), (1, probe, "GRBM_GUI_ACTIVE", 10.0),
             (1, probe, "SQ_BUSY_CYCLES", 10.0)]
    rows += [(2, gemm, "SQ_VALU_MFMA_BUSY_CYCLES", 300.0), (2, gemm, "SQ_VALU_MFMA_BUSY_CYCLES", 200.0),
             (2, gemm, "GRBM_GUI_ACTIVE", 10.0), (3, gemm, "SQ_VALU_MFMA_BUSY_CYCLES", 1000.0),
             (3, gemm, "GRBM_GUI_ACTIVE", 20.0)]
    rows += [(4, fill, "SQ_VALU_MFMA_BUSY_CYCLES", 0.0), (4, fill, "GRBM_GUI_ACTIVE", 5.0)]
    db = str(tmp_path / "c.db")
    _counter_db(db, rows)
    out = str(tmp_path / "t.md")
    bench.summarize_mfma(db, "cmd", out)
    text = open(out).read()
    assert "| `quip::gemm_kernel<128, 128, true, false, 0>` | 2 | 0.500 | 15 |" in text
    assert "| `quip::peak_mfma_f32_kernel` | 1 | 1.000 | 10 |" in text
    assert "fill_f32_kernel" not in text  # no matrix-core work


def test_mfma_busy_table_needs_the_probe(tmp_path):
    db = str(tmp_path / "c.db")
    _counter_db(db, [(1, "void quip::gemm_kernel<64, 64, false, true, 0>(x)",
                      "SQ_VALU_MFMA_BUSY_CYCLES", 5.0)])
    with pytest.raises(SystemExit):
        bench.summarize_mfma(db, "cmd", None)


def test_counter_summary_scales_by_the_copy(tmp_path):
    # FETCH_SIZE reads half of a 256 MiB copy's bytes and WRITE_SIZE all of
    # them: a kernel reading 100 KiB-as-counted is credited 200 KiB of reads
    import json

    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>>(x)"
    kern = "void quip::(anonymous namespace)::ldl_block_kernel<64, 1>(float const*)"
    mib = bench.COPY_MIB * 1024.0  # KiB each way
    fdb, wdb = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    _counter_db(fdb, [(1, copy, "FETCH_SIZE", mib / 2), (2, copy, "FETCH_SIZE", 1.0),
                      (3, kern, "FETCH_SIZE", 100.0), (4, kern, "FETCH_SIZE", 300.0)])
    _counter_db(wdb, [(1, copy, "WRITE_SIZE", mib), (3, kern, "WRITE_SIZE", 50.0),
                      (4, kern, "WRITE_SIZE", 50.0)])
    out = str(tmp_path / "c.json")
    bench.summarize_counters(fdb, wdb, "ldl_block_kernel", "ldl_block_kernel", "cmd", out)
    d = json.load(open(out))
    assert d["dispatches"] == [2, 2]
    assert d["scale_read"] == pytest.approx(2.0) and d["scale_write"] == pytest.approx(1.0)
    assert d["read_bytes_per_launch"] == pytest.approx(200.0 * 2 * 1024)
    assert d["write_bytes_per_launch"] == pytest.approx(50.0 * 1024)
    assert d["source"] == "ldl.hip" and len(d["source_sha"]) == 16


def test_rht_targets_use_the_hbm_resident_rates():
    """The RHT targets divide the HBM-resident rates by the HBM peak; the
    back-to-back (cache-resident) rates are reported beside them without a
    target, and without HBM-resident figures the cache-resident ones stand in."""
    class Cfg:
        m = n = 4096

    peak = bench.HBM_PEAK_GBS
    hot = {"right_pass_GBps": 0.62 * peak, "left_pass_GBps": 0.56 * peak,
           "two_sided_effective_GBps": 0.60 * peak}
    cold = {"right_pass_GBps": 0.63 * peak, "left_pass_GBps": 0.50 * peak,
            "two_sided_effective_GBps": 0.64 * peak}
    t = bench.pass_targets({}, {}, dict(hot, hbm_resident=cold), Cfg)
    assert t["rht_two_sided_frac_of_hbm"] == {"measured": 0.64, "target": 0.60, "meets": True}
    assert t["rht_left_pass_frac_of_hbm"] == {"measured": 0.5, "target": 0.60, "meets": False}
    assert t["rht_left_pass_frac_of_hbm_cache_resident"] == {"measured": 0.56, "target": None}
    t = bench.pass_targets({}, {}, hot, Cfg)
    assert t["rht_right_pass_frac_of_hbm"]["measured"] == 0.62
    assert "rht_right_pass_frac_of_hbm_cache_resident" not in t
