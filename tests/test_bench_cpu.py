"""bench.py's host-side contract pieces on a machine without a GPU: the
multi-GPU refusal, the FLOP / byte formulas its roofline uses, the kernel
trace summary and the counter file's guard against stale sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_flop_formulas():
    # 2 * H * (576 + 512) FLOPs per cached token: 278,528 at 128 heads (score + latent P.V)
    assert bench.core_flops(1, 128, 1) == 278528
    assert bench.core_flops(32, 128, 32 * 4096) == 36507222016
    # absorb + expand: 2 * 2 * B * H * 128 * 512
    assert bench.proj_flops(32, 128) == 2 * 2 * 32 * 128 * 128 * 512


def test_summarize_trace(tmp_path, capsys):
    cols = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id", "Kernel_Name",
            "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
            "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z",
            "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    rows = [
        ["KERNEL_DISPATCH", "1", "1", "0", "1", "1", "7", '"void mla::(anonymous namespace)::cache_append_kernel<false, false>(mla::AppendArgs)"',
         "1", "1000", "3000", "0", "0", "40", "0", "20", "256", "1", "1", "1024", "1", "1"],
        ["KERNEL_DISPATCH", "1", "1", "0", "1", "2", "7", '"void mla::(anonymous namespace)::cache_append_kernel<false, false>(mla::AppendArgs)"',
         "2", "5000", "9000", "0", "0", "40", "0", "20", "256", "1", "1", "1024", "1", "1"],
        ["KERNEL_DISPATCH", "1", "1", "0", "1", "3", "8", '"at::native::some_torch_kernel(int)"',
         "3", "5000", "9000", "0", "0", "40", "0", "20", "256", "1", "1", "1024", "1", "1"],
    ]
    path = tmp_path / "trace.csv"
    path.write_text(",".join(f'"{c}"' for c in cols) + "\n" + "\n".join(",".join(r) for r in rows) + "\n")
    bench.summarize_trace(str(path))
    out = capsys.readouterr().out
    assert "`cache_append_kernel<false, false>` | 4x1x1 | 2 | 3.00 | 2.00 | 4.00 |" in out
    assert "some_torch_kernel" not in out


def test_counter_file_guard(tmp_path, monkeypatch):
    good = {"workload": "v3_b32_s4096", "kernel_source_hash": bench.kernel_source_hash(),
            "hbm_bytes_per_launch": 123}
    f = tmp_path / "c.json"
    f.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(f))
    assert bench.traffic_from_counters("v3_b32_s4096") == 123
    assert bench.traffic_from_counters("v2lite_b64_s4096") is None       # another workload
    f.write_text(json.dumps(dict(good, kernel_source_hash="0" * 16)))
    assert bench.traffic_from_counters("v3_b32_s4096") is None           # the kernel changed since
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_from_counters("v3_b32_s4096") is None

