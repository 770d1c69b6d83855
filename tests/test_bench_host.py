"""Host-side logic of bench.py (no GPU): the rocprofv3 CSV summary and its
counter calibration, the source-hash guard on the stored traffic figure, the
one-GPU refusal and the CPU-baseline extrapolation."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from diffusion_transformer_fwd_amd import synth  # noqa: E402

GEMM = "void dit::(anonymous namespace)::gemm_bf16_kernel<256>(dit::GemmBatch)"
NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"


def _write_counters(d, rows):
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_summary_scales_fetch_by_the_calibration_kernel(tmp_path, capsys):
    # the calibration kernel reads COPY_CAL_BYTES and FETCH_SIZE counts it as
    # half as many KiB, so one counted unit is 2 KiB; values of one dispatch
    # are summed over their dimension rows
    cal = bench.COPY_CAL_BYTES / 2048
    _write_counters(tmp_path, [
        (1, GEMM, "FETCH_SIZE", 600.0), (1, GEMM, "FETCH_SIZE", 400.0),
        (2, GEMM, "FETCH_SIZE", 3000.0),
        (3, NEG, "FETCH_SIZE", cal),
    ])
    bench.summarize(str(tmp_path))
    out = capsys.readouterr().out
    # mean of 1000 and 3000 units at 2 KiB each
    assert "gemm_fetch_size_bytes_per_launch: 4096000" in out
    assert "| void gemm_bf16_kernel<256> | 2 | FETCH_SIZE | 2000 |" in out


def test_summary_of_mfma_counters(tmp_path, capsys):
    # 1024 SIMDs busy half of the GUI-active cycles (GRBM summed over 8 XCDs)
    _write_counters(tmp_path, [
        (1, GEMM, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e6),
        (1, GEMM, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1000 * 1024),
        (1, GEMM, "GRBM_GUI_ACTIVE", 8 * 1000.0),
    ])
    bench.summarize(str(tmp_path))
    out = capsys.readouterr().out
    assert "| void gemm_bf16_kernel<256> | 1 | 0.51 | 50.0 | 1000 |" in out


def test_stored_traffic_needs_the_same_gemm_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text(f"bytes_per_launch: 12345\ngemm_source_sha256: {bench.gemm_source_hash()}\n")
    assert bench.stored_gemm_traffic() == 12345.0
    f.write_text("bytes_per_launch: 12345\ngemm_source_sha256: 0000000000000000\n")
    assert bench.stored_gemm_traffic() is None
    f.unlink()
    assert bench.stored_gemm_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_times_one_whole_fp32_step():
    cfg = synth.DitConfig(hidden=256, heads=2, head_dim=128, mlp_hidden=768, n_dual=2,
                          n_single=6, in_channels=128, txt_channels=256)
    wl = synth.Workload("s", 1, 16, (4, 4), (), 0.75)
    mw = synth.ModelWeights(cfg, 0, cache=True)
    sec, threads, flops = bench.cpu_baseline(cfg, mw, wl)
    assert threads >= 1 and sec > 0
    # algorithmic FLOPs of the whole step: 8 blocks + embeddings + final layer
    S, D, F = wl.seq, cfg.hidden, cfg.mlp_hidden
    blk = 2 * S * D * (3 * D + 2 * F) + 2 * S * (D + F) * D + 4 * S * S * D
    rest = 2 * D * (16 * 256 + 16 * 128 + 16 * 128)
    assert flops == 8 * blk + rest


def test_decode_cpu_baseline_times_one_fp32_decode():
    # a small grid keeps the test quick; the bench uses 32 x 32 tokens
    sec, threads, fl, fl_1024 = bench.decode_cpu_baseline(hp=2, wp=3)
    assert sec > 0 and threads >= 1
    from oracle import vae_oracle as V
    assert fl == V.decode_flops(synth.VAE_KLEIN, 1, 2, 3)
    assert fl_1024 == V.decode_flops(synth.VAE_KLEIN, 1, 64, 64)
    assert 10.4e12 < fl_1024 < 10.6e12
