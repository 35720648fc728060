"""The benchmark's roofline arithmetic on the CPU: algorithmic bytes and
flops per launch against tensor-by-tensor counts written out independently
for tiny shapes, the peak constants, and the one-GPU guard.  No GPU."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_attention_speculative_spec_amd import synth  # noqa: E402

SH = synth.LayerShape(B=2, T=3, H=2, HV=4, K=8, V=6, L=16, max_spec=3, num_slots=5, act="bf16")


def _tensor_bytes(items):
    return sum(int(np.prod(shape)) * eb for shape, eb in items)


def test_verify_bytes_by_tensor():
    hist = np.array([5, 0])
    B, T, H, HV, K, V = SH.B, SH.T, SH.H, SH.HV, SH.K, SH.V
    record = [((H, K), 2), ((HV, V), 2), ((HV,), 4), ((HV,), 4)]        # raw k, raw v, g, beta
    expect = _tensor_bytes([((B, HV, V, K), 4)])                         # checkpoint rows read
    expect += int(hist.sum()) * _tensor_bytes(record)                    # committed history read
    expect += _tensor_bytes([((B * T, H, K), 2), ((B * T, H, K), 2),     # q, k
                             ((B * T, HV, V), 2),                        # v
                             ((B * T, HV), 2), ((B * T, HV), 2)])        # a, b
    expect += _tensor_bytes([((B * T, HV, V), 2)])                       # outputs
    expect += B * T * _tensor_bytes(record)                              # ring write
    expect += B * 4 * 4                                                  # slot index and three cursors
    assert bench.verify_alg_bytes(SH, hist) == expect == 3856


def test_dcache_and_fold_and_snapshot_bytes_by_tensor():
    hist = np.array([5, 0])
    B, T, H, HV, K, V = SH.B, SH.T, SH.H, SH.HV, SH.K, SH.V
    raw_record = _tensor_bytes([((H, K), 2), ((HV, V), 2), ((HV,), 4), ((HV,), 4)])
    delta = _tensor_bytes([((HV, V), 4)])
    hist_record = _tensor_bytes([((H, K), 2), ((HV,), 4), ((HV,), 4)]) + delta   # key, gate, beta, delta
    expect = (_tensor_bytes([((B, HV, V, K), 4)]) + int(hist.sum()) * hist_record +
              _tensor_bytes([((B * T, H, K), 2)] * 2 + [((B * T, HV, V), 2), ((B * T, HV), 2), ((B * T, HV), 2)]) +
              _tensor_bytes([((B * T, HV, V), 2)]) + B * T * (raw_record + delta) + B * 16)
    assert bench.dcache_alg_bytes(SH, hist) == expect
    folded = np.array([7, 2, 9])
    state = _tensor_bytes([((HV, V, K), 4)])
    assert bench.fold_alg_bytes(SH, folded) == len(folded) * 2 * state + int(folded.sum()) * raw_record
    snap = (_tensor_bytes([((B, HV, V, K), 4), ((B, T, HV, V, K), 4)]) +
            _tensor_bytes([((B * T, H, K), 2)] * 2 + [((B * T, HV, V), 2), ((B * T, HV), 2), ((B * T, HV), 2)]) +
            _tensor_bytes([((B * T, HV, V), 2)]))
    assert bench.snapshot_alg_bytes(SH) == snap


def test_kda_flops_and_bytes_by_counting_steps():
    # one state element costs a decay multiply (1), a dot FMA (2) and an
    # update FMA (2) per step; a readout costs one FMA (2) per element
    B, T, H, HV, K, V = SH.B, SH.T, SH.H, SH.HV, SH.K, SH.V
    replayed, flagged = 11, 1
    steps = replayed + B * T
    flops = sum(1 + 2 + 2 for _ in range(steps) for _ in range(HV * V * K))
    flops += sum(2 for _ in range(B * T) for _ in range(HV * V * K))
    record = _tensor_bytes([((H, K), 2), ((HV, V), 2), ((HV, K), 4), ((HV,), 4)])
    byts = (_tensor_bytes([((B, HV, V, K), 4)]) + flagged * _tensor_bytes([((HV, V, K), 4)]) +
            replayed * record +
            _tensor_bytes([((B * T, H, K), 2)] * 2 + [((B * T, HV, V), 2), ((B * T, HV, K), 2), ((B * T, HV), 2)]) +
            _tensor_bytes([((B * T, HV, V), 2)]) + B * T * record + B * 16)
    f, b = bench.kda_alg(SH, replayed, flagged)
    assert (f, b) == (flops, byts)
    assert bench.kda_record_bytes(SH) == record


def test_peaks():
    assert bench.HBM_PEAK_GBS == 8000.0
    # 256 CUs x 4 SIMDs x 16 lanes x one FMA (2 flops) per clock at 2.4 GHz
    assert abs(bench.ALU_F32_PEAK_TFLOPS - 78.6432) < 1e-9


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
