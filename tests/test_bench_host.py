"""Host-side checks of bench.py: its byte model against the minimal algorithmic bytes of every
workload (each input read once, each output written once, parameters and statistics once),
computed independently per workload below, and its refusal of a multi-GPU run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402

MiB = 1 << 20


def test_forward_bytes():
    # RMSNorm f32 256 x 1024: x, y f32; gamma f32; rsigma
    assert bench.fwd_bytes(W.WORKLOADS["rms_f32_256x1024"]) == 256 * 1024 * 4 * 2 + 1024 * 4 + 256 * 4 == 2102272
    # LayerNorm bf16 16384 x 4096: x, y bf16; gamma, beta f32; mu, rsigma
    assert bench.fwd_bytes(W.WORKLOADS["ln_bf16_16384x4096"]) == 16384 * 4096 * 2 * 2 + 4096 * 8 + 16384 * 8
    # delayed E4M3 32768 x 8192: x bf16, rowwise + columnwise codes, gamma, rsigma, and five
    # float32 scalars: scale and amax in; updated amax, scale_inv and colwise scale_inv out
    assert (bench.fwd_bytes(W.WORKLOADS["rms_bf16_32768x8192_delayed_e4m3"])
            == 32768 * 8192 * (2 + 1 + 1) + 8192 * 4 + 32768 * 4 + 5 * 4 == 1073905684)
    # MXFP8 16384 x 12288: x bf16, both codes, both E8M0 grids, gamma, rsigma
    assert (bench.fwd_bytes(W.WORKLOADS["rms_bf16_16384x12288_mxfp8_e4m3"])
            == 16384 * 12288 * 4 + 16384 * (12288 // 32) + 12288 * (16384 // 32) + 12288 * 4 + 16384 * 4
            == 818003968)
    # LayerNorm bf16 1024 x 65536
    assert bench.fwd_bytes(W.WORKLOADS["ln_bf16_1024x65536"]) == 1024 * 65536 * 4 + 65536 * 8 + 1024 * 8 == 268967936


def test_backward_bytes():
    # dy, x in; dx out; rsigma (+ mu); gamma in; dgamma (+ dbeta) out
    assert bench.bwd_bytes(W.WORKLOADS["rms_f32_256x1024"], False) == 256 * 1024 * 4 * 3 + 256 * 4 + 1024 * 4 * 2 == 3154944
    assert (bench.bwd_bytes(W.WORKLOADS["ln_bf16_16384x4096"], False)
            == 16384 * 4096 * 2 * 3 + 16384 * 8 + 4096 * 4 * 3 == 402833408)
    # the fused add reads residual_dy as well
    assert (bench.bwd_bytes(W.WORKLOADS["rms_bf16_32768x8192_bwd_add"], True)
            == 32768 * 8192 * 2 * 4 + 32768 * 4 + 8192 * 4 * 2 == 2147680256)


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
