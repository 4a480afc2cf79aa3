"""Host logic of bench.py that the committed profiles come from, on synthetic
rocprofv3 CSVs with known answers (CPU only): the kernel-trace summary (mean,
median, p10, p90), the FETCH_SIZE / WRITE_SIZE calibration against the 1 GiB
copy probe, the join of the shader and L2 counter passes, the code-hash gate on
roofline.traffic, the byte counts of the workloads, and the refusal of more
than one GPU."""
import argparse
import csv
import json
import os

import numpy as np
import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _args(**kw):
    base = dict(summarize_trace=None, kernel_filter="mfr_", stats_csv="", title="t", command="c",
                out=None, fetch_csv=None, write_csv=None, counter_csv=[], json_out="")
    base.update(kw)
    return argparse.Namespace(**base)


def test_trace_summary_statistics(tmp_path):
    trace = tmp_path / "kernel_trace.csv"
    durations_us = [float(v) for v in range(1, 101)]  # 1..100 µs
    with open(trace, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp",
                    "End_Timestamp"])
        t = 0
        for d in durations_us:
            w.writerow(["void mfr::mfr_fused_kernel<3, 8, 16, 0, false>(mfr::Params)", 2048, 256,
                        t, t + int(d * 1000)])
            t += 10 ** 6
        w.writerow(["__amd_rocclr_copyBuffer", 1, 1, 0, 5000])  # filtered out
    stats = tmp_path / "kernel_stats.csv"
    stats.write_text('"Name","Calls"\n"x",1\n')
    out = tmp_path / "summary.md"
    bench.summarize_trace(_args(summarize_trace=str(trace), stats_csv=str(stats), out=str(out)))
    text = out.read_text()
    row = [ln for ln in text.splitlines() if ln.startswith("| `void mfr::")]
    assert len(row) == 1 and "copyBuffer" not in row[0]
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    # kernel, grid, workgroup, tokens, calls, avg, median, p10, p90, min, max
    assert cells[1:5] == ["2048", "256", "8", "100"]
    assert cells[5:] == ["50.50", "50.50", "10.00", "90.00", "1.00", "100.00"]
    assert '"Name","Calls"' in text  # the stats table is appended verbatim


def _pmc_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for name, value in rows:
            w.writerow([name, counter, value])


def test_pmc_calibration(tmp_path, monkeypatch):
    """The copy probe moves exactly 1 GiB each way; the counters it reads
    give the scale factors for the fused kernel's counters."""
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    fused = "void mfr::mfr_fused_kernel<3, 8, 16, 0, false>(mfr::Params)"
    copy = "mfr_copy_probe_kernel(u32x4 const*, u32x4*, long)"
    _pmc_csv(fetch, "FETCH_SIZE", [(fused, 500000.0), (fused, 500002.0), (copy, 524288.0)])
    _pmc_csv(write, "WRITE_SIZE", [(fused, 196608.0), (copy, 1048576.0)])
    monkeypatch.setattr(bench, "kernel_code_hash", lambda: "abc")
    out = tmp_path / "traffic.json"
    bench.summarize_pmc(_args(fetch_csv=str(fetch), write_csv=str(write), out=str(out)))
    t = json.loads(out.read_text())
    assert t["copy_probe"]["fetch_scale"] == 2.0 and t["copy_probe"]["write_scale"] == 1.0
    assert t["fetch_kib_per_dispatch"] == 500001.0
    assert t["traffic_bytes_per_launch"] == round(500001.0 * 1024 * 2 + 196608.0 * 1024)
    assert t["algorithmic_bytes"] == 1208496128 and t["code_hash"] == "abc"


def test_traffic_gate_follows_the_code_hash(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"code_hash": "h1", "traffic_bytes_per_launch": 123}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    monkeypatch.setattr(bench, "kernel_code_hash", lambda: "h1")
    assert bench.traffic_for_headline() == 123
    monkeypatch.setattr(bench, "kernel_code_hash", lambda: "h2")
    assert bench.traffic_for_headline() is None
    monkeypatch.setattr(bench, "kernel_code_hash", lambda: None)
    assert bench.traffic_for_headline() is None


def test_code_hash_reads_the_embedded_code_objects(tmp_path):
    pytest.importorskip("top_finalize_residual_amd", reason="HIP library not built")
    from top_finalize_residual_amd import build as b
    with open(b.LIB, "rb") as f:
        host = bench._elf_sections(f.read())
    bundle = bench._offload_bundle(host[".hip_fatbin"])
    assert any("gfx950" in triple for triple, _ in bundle)
    assert bench.kernel_code_hash() == bench.kernel_code_hash() is not None
    not_elf = tmp_path / "x.so"
    not_elf.write_bytes(b"not an ELF file")
    assert bench.kernel_code_hash(str(not_elf)) is None
    assert bench._offload_bundle(b"something else") is None


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_code_hash_is_the_same_for_builds_at_different_paths(tmp_path):
    """The same kernel source compiled in two directories (different source
    and output paths, so different per-build identifiers in the symbol
    tables) hashes the same, so a traffic record taken on one build is
    recognised on another."""
    import shutil
    import subprocess
    from top_finalize_residual_amd import build as b
    procs, libs = [], []
    for sub in ("a", os.path.join("b", "deeper")):
        d = tmp_path / sub
        shutil.copytree(b.CSRC, d / "csrc")
        shutil.copytree(b.INCLUDE, d / "include")
        lib = str(d / "libmoe_finalize_rmsnorm.so")
        cmd = [b.HIPCC, *b.HIPFLAGS, *b.PRELOAD, "-I", str(d / "include"), "-I", str(d / "csrc"),
               "-o", lib, str(d / "csrc" / "mfr_kernels.hip")]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE))
        libs.append(lib)
    for p in procs:
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, err.decode()[-2000:]
    h = [bench.kernel_code_hash(lib) for lib in libs]
    assert h[0] is not None and h[0] == h[1]


def test_closed_form_bytes_match_drawn_inputs():
    d = synth.config_inputs("batch512", 512)
    assert synth.config_algorithmic_bytes("batch512", 512) == synth.algorithmic_bytes(
        d["perm_idx"], d["H"], d["K"])
    with pytest.raises(ValueError):
        synth.config_algorithmic_bytes("decode_masked", 4)
    for normed in (False, True):
        assert synth.config_fp8_algorithmic_bytes("batch512", 512, normed) == \
            synth.fp8_algorithmic_bytes(d["perm_idx"], d["H"], d["K"], bf16_normed=normed)
    with pytest.raises(ValueError):
        synth.config_fp8_algorithmic_bytes("decode_masked", 4)


def test_variant_bytes_follow_the_template_arguments():
    T, H, K = 8192, 6144, 8
    assert bench.variant_algorithmic_bytes("void mfr::mfr_fused_kernel<3, -1, 16, 0, false>(x)") == \
        8 * H * T + 2 * H
    # FP8 codes only: reads as the fused op, residual_out, codes and one scale per token
    assert bench.variant_algorithmic_bytes("void mfr::mfr_fused_kernel<3, 8, 16, 1, false>(x)") == \
        2 * H * T * K + 4 * H * T + 8 * K * T + 2 * H + (2 * H + H + 4) * T
    assert bench.variant_algorithmic_bytes("void mfr::mfr_fused_kernel<3, 8, 16, 2, false>(x)") == \
        2 * H * T * K + 4 * H * T + 8 * K * T + 2 * H + (4 * H + H + 4) * T
    assert bench.variant_algorithmic_bytes("void mfr::mfr_fused_kernel<3, 8, 16, 0, false>(x)") == \
        1208496128
    # dense FP8: x, residual, residual_out, codes and one scale per token
    assert bench.variant_algorithmic_bytes("void mfr::mfr_fused_kernel<3, -1, 16, 1, false>(x)") == \
        (6 * H + H + 4) * T + 2 * H
    assert bench.variant_algorithmic_bytes("void mfr::mfr_fused_kernel<3, -1, 16, 2, false>(x)") == \
        (8 * H + H + 4) * T + 2 * H


def test_pmc_variants_calibration(tmp_path, monkeypatch):
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    dense = "void mfr::mfr_fused_kernel<3, -1, 16, 0, false>(mfr::Params)"
    fp8 = "void mfr::mfr_fused_kernel<3, 8, 16, 1, false>(mfr::Params)"
    copy = "mfr_copy_probe_kernel(u32x4 const*, u32x4*, long)"
    _pmc_csv(fetch, "FETCH_SIZE", [(dense, 100000.0), (dense, 100002.0), (fp8, 490000.0),
                                   (copy, 524288.0)])
    _pmc_csv(write, "WRITE_SIZE", [(dense, 196608.0), (fp8, 147456.0), (copy, 1048576.0)])
    monkeypatch.setattr(bench, "kernel_code_hash", lambda: "abc")
    out, js = tmp_path / "v.md", tmp_path / "v.json"
    bench.summarize_pmc_variants(_args(fetch_csv=str(fetch), write_csv=str(write), out=str(out),
                                       json_out=str(js)))
    t = json.loads(js.read_text())
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0 and t["code_hash"] == "abc"
    k = t["kernels"]["mfr::mfr_fused_kernel<3, -1, 16, 0, false>"]
    assert k["traffic_bytes"] == round(100001.0 * 1024 * 2 + 196608.0 * 1024)
    assert k["ratio"] == pytest.approx(k["traffic_bytes"] / (8 * 6144 * 8192 + 2 * 6144))
    assert set(t["kernels"]) == {"mfr::mfr_fused_kernel<3, -1, 16, 0, false>",
                                 "mfr::mfr_fused_kernel<3, 8, 16, 1, false>"}
    assert out.read_text().count("| `mfr::mfr_fused_kernel<") == 2


def test_counter_summary_joins_passes(tmp_path):
    """Three passes over two dispatches of one launch shape and one of
    another: means per shape, instructions per wave, and the L2 hit rate."""
    cols = ["Kernel_Name", "Grid_Size", "Workgroup_Size", "VGPR_Count", "SGPR_Count",
            "LDS_Block_Size", "Counter_Name", "Counter_Value"]
    fused = "void mfr::mfr_fused_kernel<3, 8, 16, 0, false>(mfr::Params)"
    small = "void mfr::mfr_fused_kernel<1, 8, 0, 0, false>(mfr::Params)"
    passes = [
        [(fused, 2048, 256, "SQ_WAVES", 32), (fused, 2048, 256, "SQ_INSTS_VALU", 3200),
         (fused, 2048, 256, "SQ_LDS_BANK_CONFLICT", 0),
         (fused, 2048, 256, "SQ_WAVES", 32), (fused, 2048, 256, "SQ_INSTS_VALU", 3840),
         (fused, 2048, 256, "SQ_LDS_BANK_CONFLICT", 10),
         (small, 768, 768, "SQ_WAVES", 12), (small, 768, 768, "SQ_INSTS_VALU", 1200),
         ("__amd_rocclr_copyBuffer", 64, 64, "SQ_WAVES", 1)],
        [(fused, 2048, 256, "TCC_HIT_sum", 30), (fused, 2048, 256, "TCC_MISS_sum", 70),
         (fused, 2048, 256, "TCC_HIT_sum", 10), (fused, 2048, 256, "TCC_MISS_sum", 90)],
        [(fused, 2048, 256, "OccupancyPercent", 40.0), (fused, 2048, 256, "OccupancyPercent", 60.0),
         (fused, 2048, 256, "VALUBusy", 5.0), (fused, 2048, 256, "VALUBusy", 7.0)],
    ]
    paths = []
    for i, rows in enumerate(passes):
        p = tmp_path / f"pass{i}.csv"
        with open(p, "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(cols)
            for name, grid, wg, c, v in rows:
                w.writerow([name, grid, wg, 72, 64, 512, c, v])
        paths.append(str(p))
    out, js = tmp_path / "c.md", tmp_path / "c.json"
    bench.summarize_counters(_args(counter_csv=paths, out=str(out), json_out=str(js)))
    rec = json.loads(js.read_text())
    assert len(rec) == 2  # the copy kernel is filtered out
    big = rec["mfr::mfr_fused_kernel<3, 8, 16, 0, false> grid=2048 wg=256"]
    assert big["dispatches"] == 2 and big["waves"] == 32
    assert big["valu_per_wave"] == pytest.approx(3520 / 32)
    assert big["lds_bank_conflict"] == 5
    assert big["l2_hit_pct"] == pytest.approx(20.0)
    assert big["occupancy_pct"] == 50.0 and big["valu_busy_pct"] == 6.0
    assert (big["vgpr"], big["sgpr"], big["lds_bytes"]) == (72, 64, 512)
    tiny = rec["mfr::mfr_fused_kernel<1, 8, 0, 0, false> grid=768 wg=768"]
    assert tiny["valu_per_wave"] == 100 and tiny["l2_hit_pct"] is None
    text = out.read_text()
    assert "| `mfr::mfr_fused_kernel<3, 8, 16, 0, false>` | 8 × 256 | 2 |" in text
    assert "| `mfr::mfr_fused_kernel<1, 8, 0, 0, false>` | 1 × 768 | 1 |" in text


def test_rate_units():
    # 1,208,496,128 bytes in 195 µs is 6197.4 GB/s, 77.47% of 8 TB/s
    r = bench._rate(195.0, 1208496128)
    assert r == {"us": 195.0, "gbs": 6197.4, "frac": 0.7747}


def test_more_than_one_gpu_is_refused():
    """The bench measures one GPU: --gpus above 1 (or a multi-rank launch)
    exits with status 2 and says why, before touching a GPU."""
    import subprocess
    import sys
    for args, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT,
                           env=dict(os.environ, **env), capture_output=True, text=True, timeout=120)
        assert r.returncode == 2, r.stderr
        assert "measures one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_all_cores_covers_every_token(monkeypatch):
    """The all-cores oracle leg splits the tokens into disjoint ranges that
    together cover the workload once per pass, one thread per allowed core."""
    import oracle
    d = synth.config_inputs("tiny", 4)
    seen = []
    real = oracle.finalize_rmsnorm

    def spy(expert_out, perm_idx, *a, **kw):
        seen.append(perm_idx.copy())
        return real(expert_out, perm_idx, *a, **kw)
    monkeypatch.setattr(oracle, "finalize_rmsnorm", spy)
    nb = synth.algorithmic_bytes(d["perm_idx"], d["H"], d["K"])
    r = bench.cpu_baseline_all_cores(d, nb, min_seconds=0.0, max_passes=1)
    n = len(os.sched_getaffinity(0))
    assert r["cores"] == n and r["value"] > 0 and r["unit"] == "GB/s"
    # a warm-up pass, then one timed pass, each of the n ranges (in any order)
    assert len(seen) == 2 * n
    for p in range(2):
        got = np.concatenate([s for s in seen[p * n:(p + 1) * n] if s.size], axis=0)
        assert np.array_equal(np.sort(got, axis=None), np.sort(d["perm_idx"], axis=None))
        assert got.shape == d["perm_idx"].shape


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_summarize_phases_maps_dispatches_by_order(tmp_path):
    """Phase runs label the fused-kernel dispatches by their position: the
    trace summary attributes durations, and the counter summary values and
    calibrated traffic, to the right phase; other kernels (cache scrubs, the
    copy probe) are left out of the count."""
    phases = {"phases": [{"label": "T512/auto", "dispatches": 2, "bytes": 1000},
                         {"label": "T512/persist", "dispatches": 1, "bytes": 1000}]}
    pj = tmp_path / "phases.json"
    pj.write_text("noise line\n" + json.dumps(phases) + "\n")
    fused = "void mfr::mfr_fused_kernel<3, 8, 0, 0, false>(int const*)"
    persist = "void mfr::mfr_persist_kernel<8, 0, 0, false>(int const*)"
    trace = tmp_path / "trace.csv"
    hdr = ["Dispatch_Id", "Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp",
           "End_Timestamp"]
    _write_csv(trace, hdr, [[3, persist, 196608, 768, 5000, 8000],
                            [1, fused, 131072, 256, 1000, 2000],
                            [0, "mfr_touch_probe_kernel", 1024, 256, 0, 10],
                            [2, fused, 131072, 256, 3000, 5000]])
    out = tmp_path / "t.md"
    bench.summarize_phases(argparse.Namespace(phases_json=str(pj), trace_csv=str(trace),
                                              counter_csv=[], title="t", command="c",
                                              out=str(out), append_sweep="", append_states=""))
    text = out.read_text()
    row_auto = next(ln for ln in text.splitlines() if ln.startswith("| T512/auto"))
    row_persist = next(ln for ln in text.splitlines() if ln.startswith("| T512/persist"))
    assert "| 2 | 1.50 |" in row_auto and "mfr_fused_kernel" in row_auto
    assert "| 1 | 3.00 |" in row_persist and "mfr_persist_kernel" in row_persist
    # counters: 2 counters per dispatch, plus the copy probe for calibration
    cnt = tmp_path / "c.csv"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    for i, (k, fv, wv) in enumerate([(fused, 400, 200), (fused, 600, 200), (persist, 500, 300)]):
        rows += [[i, k, "FETCH_SIZE", fv / 1024.0], [i, k, "WRITE_SIZE", wv / 1024.0]]
    rows += [[9, "mfr_copy_probe_kernel", "FETCH_SIZE", (1 << 30) / 1024.0 / 2],
             [9, "mfr_copy_probe_kernel", "WRITE_SIZE", (1 << 30) / 1024.0]]
    _write_csv(cnt, hdr, rows)
    bench.summarize_phases(argparse.Namespace(phases_json=str(pj), trace_csv=None,
                                              counter_csv=[str(cnt)], title="t", command="c",
                                              out=str(out), append_sweep="", append_states=""))
    lines = out.read_text().splitlines()
    # fetch scaled by 2 (the copy's fetch counts half), write by 1
    assert any(ln.startswith("| T512/auto | 1,200 | 1,000 | 1.2000 |") for ln in lines), lines
    assert any(ln.startswith("| T512/persist | 1,300 | 1,000 | 1.3000 |") for ln in lines), lines
    # a mismatch between the phase table and the dispatches is refused
    _write_csv(trace, ["Dispatch_Id", "Kernel_Name", "Grid_Size_X", "Workgroup_Size_X",
                       "Start_Timestamp", "End_Timestamp"], [[0, fused, 1, 1, 0, 1]])
    with pytest.raises(SystemExit):
        bench.summarize_phases(argparse.Namespace(phases_json=str(pj), trace_csv=str(trace),
                                                  counter_csv=[], title="t", command="c",
                                                  out=str(out), append_sweep="", append_states=""))


def test_sweep_and_cold_tables(tmp_path):
    """The sweep table marks the fastest entry of each column and names the
    alternatives and the hidden size; the cold table prints µs and TB/s."""
    sw = {"shape_sweep": {"kind": "alternatives", "H": 5120, "K": 8, "unit": "us", "reps": 5,
                          "T": {"2048": {"auto": 45.0, "cap-2-per-CU": 44.0, "auto_path": "stream",
                                         "bytes": 1},
                                "8192, 2 output sets": {"auto": 170.0, "cap-2-per-CU": 171.0,
                                                        "auto_path": "stream", "bytes": 1}}}}
    p = tmp_path / "sw.json"
    p.write_text(json.dumps(sw) + "\n")
    lines = bench.sweep_table_lines(str(p))
    assert "for the fused op at H = 5120, K = 8" in lines[0] and "--alternatives" in lines[0]
    assert lines[2] == "| alternative | T = 2048 | T = 8192, 2 output sets |"
    assert "| auto | 45.00 | **170.00** |" in lines and "| cap-2-per-CU | **44.00** | 171.00 |" in lines
    ct = {"cold_table": {"28": {m: {"us": 4.5, "gbs": 900.0, "sets": 100}
                                for m in ("bf16", "fp8", "dense")}}}
    c = tmp_path / "c.json"
    c.write_text("log line\n" + json.dumps(ct) + "\n")
    lines = bench.cold_table_lines(str(c))
    assert "| fused, µs | 4.50 |" in lines and "| fused, TB/s | 0.90 |" in lines


def test_mix_probe_byte_counts_and_refusals():
    """The mixed-stream probe's buffers are the headline chunk's own read and
    write bytes, in whole units of one token in both output forms; the probe
    refuses an uninstantiated proportion, the FP8-code form on any pair but
    (30, 3) and that pair without it, bad flags, misaligned or missing
    buffers, buffers below one unit and a pipelined launch with no grid
    before any launch (so this runs without a GPU)."""
    import ctypes
    H, T, K = 6144, 8192, 8
    assert bench.MIX_READ_BYTES == (T * K + 2 * T) * H * 2
    assert bench.MIX_WRITE_BYTES["bf16"] == 2 * T * H * 2
    assert bench.MIX_WRITE_BYTES["fp8"] == T * H * 2 + T * H
    for mode, (a, b) in bench.MIX_PAIRS.items():
        unit_r = a * 256 * 16
        unit_w = b * 256 * (24 if bench.MIX_FORM[mode] & bench.MIX_CODES else 16)
        assert bench.MIX_READ_BYTES % unit_r == 0 and bench.MIX_WRITE_BYTES[mode] % unit_w == 0
        assert bench.MIX_READ_BYTES // unit_r == bench.MIX_WRITE_BYTES[mode] // unit_w == T
    # one token at 256 threads: 8 rows + shared + residual = 30 vectors per thread in; out,
    # 6 vectors (residual_out, normed_out), or 3 and 3 half vectors (residual_out, codes)
    assert bench.MIX_PAIRS["bf16"] == (30, 6) and bench.MIX_FORM["bf16"] == 0
    assert bench.MIX_PAIRS["fp8"] == (30, 3) and bench.MIX_FORM["fp8"] == bench.MIX_CODES
    lib = bench._probe_lib()
    rb, wb = ctypes.c_int64(0), ctypes.c_int64(0)
    ok = 1 << 20  # stands in for a 16-byte aligned device address; never dereferenced here

    def call(src, sb, dst, db, reads=30, writes=6, flags=0, grid=0, per_cu=0):
        return lib.mfr_mix_probe(src, sb, dst, db, reads, writes, flags, grid, per_cu,
                                 ctypes.byref(rb), ctypes.byref(wb), None)
    big = (ok, 1 << 30, ok + (1 << 30), 1 << 28)
    assert call(*big, reads=30, writes=5) == 1        # not an instantiated proportion
    assert call(*big, reads=35, writes=7) == 1
    assert call(*big, flags=4) == 1 and call(*big, flags=8) == 1 and call(*big, flags=-1) == 1
    assert call(*big, reads=30, writes=3) == 1        # (30, 3) only in the FP8-code form
    assert call(*big, reads=20, writes=3, flags=4) == 1
    assert call(ok, 1 << 30, ok + (1 << 30), 3 * 4096 * 3 // 2 - 16, reads=30, writes=3,
                flags=4) == 1                         # below one unit of both regions
    assert call(*big, flags=2) == 1                   # pipelined needs a grid
    assert call(None, 1 << 30, ok, 1 << 28) == 1      # missing buffer
    assert call(ok + 8, 1 << 30, ok, 1 << 28) == 1    # misaligned
    assert call(ok, 30 * 4096 - 16, ok + (1 << 30), 1 << 28) == 1  # below one unit read
    assert call(ok, 1 << 30, ok + (1 << 30), 6 * 4096 - 16) == 1   # below one unit written
    assert call(*big, grid=-1) == 1
    assert call(*big, per_cu=-1) == 1 and call(*big, per_cu=33) == 1


def test_mix_sweep_summary(tmp_path):
    """The depth sweep's summary puts each record in its table cell, with a
    dash where a residency was not reachable."""
    rec = {f"unit/A{a}/cap{n}": 1000.0 * n + a for a in bench.MIX_DEPTHS for n in bench.MIX_CAPS}
    del rec["unit/A40/cap4"]
    rec.update({f"unit/A{a}/nocap": 7.0 for a in bench.MIX_DEPTHS})
    rec.update({f"pipe/A{a}/{n}-per-cu": 9.0 for a in bench.MIX_DEPTHS for n in bench.MIX_CAPS})
    rec.update({"fp8/A20/cap1": 6001.0, "fp8/A40/cap2": 6002.0, "fp8codes/A30/cap3": 6003.0})
    path = tmp_path / "mix.json"
    path.write_text(json.dumps(rec))
    lines = bench.mix_sweep_lines(str(path))
    assert "| 30 (120) | 1,030 | 2,030 | 3,030 | 4,030 | 7 |" in lines
    assert "| 40 (160) | 1,040 | 2,040 | 3,040 | — | 7 |" in lines
    assert "| 20 (80) | 6,001 | — | — |" in lines and "| 40 (160) | — | 6,002 | — |" in lines
    assert "| 30 (120), codes form | — | — | 6,003 |" in lines
