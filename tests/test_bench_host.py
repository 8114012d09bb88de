"""Host-side logic of bench.py, on the CPU: the algorithmic byte counts it divides by,
the traffic record it reads from profiles/ (and drops once the prefill kernel's
source changes), the single-GPU guard, the kernel-trace summary that recomputes
the bench's figures from rocprofv3 kernel durations (run here on a synthetic trace
database laid out like the per-kernel runs of the bench), and the reading of
amd-smi's power and clock report."""
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
LIB = os.path.join(ROOT, "w6a6_w6a8_integer_amd", "libflexq.so")

import bench  # noqa: E402


def test_algorithmic_bytes():
    # 0.75 N K (packed W) + 2 N G (fp16 s_w) + M K (q_a) + 4 M G (fp32 s_a) + 2 M N (Y)
    assert bench.gemm_bytes(1, 16, 128) == 0.75 * 16 * 128 + 2 * 16 + 128 + 4 + 2 * 16
    M, N, K = 16, 8192, 28672
    G = K // 128
    assert bench.gemm_bytes(M, N, K) == 0.75 * N * K + 2 * N * G + M * K + 4 * M * G + 2 * M * N
    # fp16 X in, int8 codes and fp32 scales out
    assert bench.quant_bytes(4, 256) == 2 * 4 * 256 + 4 * 256 + 4 * 4 * 2


def test_traffic_record_follows_the_kernel_source(tmp_path, monkeypatch):
    rec = bench.recorded_traffic()
    text = open(bench.TRAFFIC_FILE).read()
    assert rec is not None and f"traffic_bytes_per_launch: {rec}" in text
    # another source (one byte changed) no longer matches the recorded hash
    src = open(bench.PREFILL_SRC, "rb").read()
    other = tmp_path / "gemm_prefill.hip"
    other.write_bytes(src + b"\n")
    monkeypatch.setattr(bench, "PREFILL_SRC", str(other))
    assert bench.recorded_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.recorded_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.skipif(not os.path.exists(LIB), reason="libflexq.so not built")
def test_trace_summary_recomputes_the_figures(tmp_path, capsys):
    """Per-kernel runs as the bench launches them (a busy kernel, `reps` quantizer
    launches, the GEMM launches of one shape), for two shapes of the 70B o layer and
    two runs each: the summary must find every run, give each shape its median time
    per call and the prefill and decode rates those times imply."""
    import w6a6_w6a8_integer_amd as fq
    fq.lib()
    layers = {"o": (8192, 8192)}
    m_list = (1, 4096)
    reps = 3
    # bench order of the shapes: largest M first, A6 then A8
    keys = sorted({(M, ab, n) for M in m_list for ab in bench.ABITS for n in layers},
                  key=lambda k: (-k[0], k[1]))
    per_call_ns = {(4096, 6, "o"): [300e3, 310e3], (4096, 8, "o"): [320e3, 330e3],
                   (1, 6, "o"): [11e3, 12e3], (1, 8, "o"): [12e3, 13e3]}
    rows, t = [], 0
    for r in range(2):
        for k in keys:
            rows.append(("void flexq::peak_mfma_kernel<0>(int)", 50e3, 65536, 256, t))
            t += 1
            for _ in range(reps):
                rows.append(("void flexq::quant_act_kernel<false>(...)", 2e3, 4096, 256, t))
                t += 1
            name = ("void flexq::gemm_prefill_kernel<256, 128, false>(...)" if k[0] > 64 else
                    "void flexq::gemm_decode_kernel<1, 2, 8, 2, 1, false, false>(...)")
            for _ in range(reps):
                rows.append((name, per_call_ns[k][r], 1024 * 512, 512, t))
                t += 1
    db = tmp_path / "trace.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, duration real, grid_x int, workgroup_x int, "
                "start int)")
    con.executemany("insert into kernels values (?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()
    bench.summarize_trace(str(db), layers, m_list, reps)
    out = capsys.readouterr().out
    assert "| o | 4096 | 6 | 256x128 | 305.00 |" in out
    assert "| o | 1 | 8 | decode | 12.50 |" in out
    # prefill: 2 M N K ops per call over the median call times of both precisions
    ops = 2.0 * 4096 * 8192 * 8192
    tops = 2 * ops / ((305e3 + 325e3) * 1e-9) / 1e12
    assert f"prefill {tops:.1f} TOP/s" in out
    dec = 2 * bench.gemm_bytes(1, 8192, 8192) / ((11.5e3 + 12.5e3) * 1e-9) / 1e9
    assert f"decode at M <= 16: {dec:.1f} GB/s" in out
    assert "4 runs of 3 calls" not in out and "8 runs of 3 calls" in out


def test_power_readings():
    """amd-smi metric JSON -> (socket W, mean gfx clock); per-phase medians with the
    lagging first readings of a phase dropped."""
    import json
    gfx = {f"gfx_{i}": {"clk": {"value": 1900 + 10 * i, "unit": "MHz"}} for i in range(8)}
    doc = {"gpu_data": [{"gpu": 0, "power": {"socket_power": {"value": 1372, "unit": "W"}},
                         "clock": {**gfx, "mem_0": {"clk": {"value": 2000, "unit": "MHz"}},
                                   "fclk_0": {"clk": "N/A"}}}]}
    assert bench.parse_smi_power(json.dumps(doc)) == (1372.0, 1935.0)
    assert bench.parse_smi_power("not json") is None
    assert bench.parse_smi_power(json.dumps({"gpu_data": []})) is None
    samples = [("a", (300.0, 100.0)), ("a", (900.0, 2300.0))] + \
        [("a", (1370.0 + i, 1940.0)) for i in range(5)] + [("b", None), ("b", (1000.0, 2400.0))]
    out = bench.summarize_power(samples)
    assert out["a"] == {"watts_median": 1372.0, "gfx_mhz_median": 1940.0, "samples": 5}
    assert out["b"]["samples"] == 1 and out["b"]["watts_median"] == 1000.0
