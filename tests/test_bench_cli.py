"""bench.py's contract on the CPU: more than one GPU is refused with a message before
anything touches a device, a host without a GPU exits with status 1 (after the library
loads, so a missing library still fails loudly), and the FLOP model gives the headline
workload's figures (forward 2 GEMM units, backward 5, a unit being 2·B·H·N²·d halved
under causal masking; packed batches sum their sequences)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    err = capsys.readouterr().err
    assert "one GPU only" in err and "--gpus 2" in err


def test_no_gpu_exits_with_status_1(capsys):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert bench.main(["--steps", "1", "--warmup", "0", "--cpu-budget", "0"]) == 1
    assert "no GPU visible" in capsys.readouterr().err


def test_flop_model_of_the_headline_workload():
    # B=4, H=32, N=4096, d=128, causal: one unit = 2*4*32*4096^2*128 / 2 = 274.9 GFLOP
    unit = bench.gemm_unit(4, 32, 4096, 128, True)
    assert unit == 2.0 * 4 * 32 * 4096 * 4096 * 128 / 2
    assert round(2 * unit / 1e9, 1) == 549.8     # forward
    assert round(5 * unit / 1e9, 1) == 1374.4    # backward = 2.5 x forward
    # the time the targets mean at the published peak (50 % forward, 35 % backward)
    peak = 2516.6e12
    assert round(2 * unit / (0.50 * peak) * 1e6) == 437
    assert round(5 * unit / (0.35 * peak) * 1e6) == 1560


def test_flop_model_of_packed_batches():
    lengths = [3, 5, 8]
    unit = bench.gemm_unit(0, 2, 0, 4, True, lengths)
    assert unit == sum(2.0 * 2 * L * L * 4 / 2 for L in lengths)
    assert bench.gemm_unit(0, 2, 0, 4, False, lengths) == 2 * unit
