"""The seeded input generators (host and device draws) hold the workload's
distributions and round to the storage dtype exactly as stated."""
from __future__ import annotations

import numpy as np
import torch

from linear_attention_speculative_spec_amd import synth


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is halfway between two bf16 neighbours: rounds to the even one (1.0)
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1e-40], dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    assert got[0] == 1.0
    assert got[1] == np.float32(1.0 + 4 * 2.0 ** -8)
    assert got[2] == -2.5
    # torch's own conversion agrees bit for bit on random values
    y = np.random.default_rng(0).normal(size=4096).astype(np.float32) * 7
    tb = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(tb, synth.f32_to_bf16_bits(y))


def test_device_windows_shapes_rows_and_distribution():
    sh = synth.CONFIGS["long_window_t8"].replace(B=6)
    dw = synth.DeviceWindows(5, sh, "beta_high", device="cpu")
    w = dw.draw()
    n = sh.B * sh.T
    assert tuple(w["q"].shape) == (n, sh.H, sh.K) and w["q"].dtype == torch.bfloat16
    assert tuple(w["v"].shape) == (n, sh.HV, sh.V)
    assert tuple(w["b"].shape) == (n, sh.HV)
    qf = w["q"].float().numpy()
    assert abs(qf.mean()) < 0.05 and abs(qf.std() - 1.0) < 0.05
    assert abs(w["b"].float().mean().item() - 4.0) < 0.2
    rows = [1, 4]
    hw = dw.host_rows(w, rows, sh.T)
    for name, x in zip("qkvab", (hw.q, hw.k, hw.v, hw.a, hw.b)):
        full = w[name].view(torch.int16).numpy().view(np.uint16)
        want = np.concatenate([full[r * sh.T:(r + 1) * sh.T] for r in rows])
        assert x.dtype == np.uint16 and np.array_equal(x, want), name
    # the same seed draws the same values
    w2 = synth.DeviceWindows(5, sh, "beta_high", device="cpu").draw()
    assert all(torch.equal(w[k], w2[k]) for k in w)
