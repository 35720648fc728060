"""Shared test plumbing: widening synthetic inputs and building ring states.

Holds no arithmetic of the method: it only moves the seeded inputs around.
"""
from __future__ import annotations

import numpy as np

from linear_attention_speculative_spec_amd import synth


def win_f64(win: synth.Window, act: str):
    """(q, k, v, a, b) widened exactly to float64."""
    return tuple(synth.act_to_f64(x, act) for x in (win.q, win.k, win.v, win.a, win.b))


def window_rows(win: synth.Window, rows, T: int) -> synth.Window:
    """Sub-window holding the given rows (token-major packing kept)."""
    idx = (np.asarray(rows)[:, None] * T + np.arange(T)[None, :]).reshape(-1)
    return synth.Window(*(x[idx] for x in (win.q, win.k, win.v, win.a, win.b)))


def prefill_plan(slot_idx, write_pos, n_records):
    """For record r: the slot list of rows still filling (others padded to -1)."""
    plan = []
    wp_rows = write_pos[slot_idx]
    for r in range(n_records):
        plan.append(np.where(wp_rows > r, slot_idx, -1).astype(np.int32))
    return plan


def max_rel(x, ref):
    """max |x - ref| / max |ref| over a whole tensor."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / (den if den > 0 else 1.0))


def elem_rel(x, ref, floor: float = 1e-3):
    """max over elements of |x - ref| / (|ref| + floor * max |ref|): the
    elementwise relative error, with a floor so that values near zero are
    judged against the tensor's scale rather than their own."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.max(np.abs(ref))
    den = np.abs(ref) + floor * (scale if scale > 0 else 1.0)
    return float(np.max(np.abs(x - ref) / den))


# Lines collected by the tests and printed once at the end of the session
# (see conftest.py), so that figures such as drift curves and full-size error
# metrics appear in the run's output even when pytest captures test output.
REPORT: list = []


def report(line: str) -> None:
    print(line, flush=True)
    REPORT.append(line)
