"""Pins of the per-channel-gate (KDA) oracle to things other than itself.

The KDA layer keeps one gate value per key channel (PR #36821 summary: the
KDA spec ring stores g as [slots, HV, L, K] fp32, a per-K gate).  Its oracle
is pinned by: the reduction to the pinned GDN oracle when every channel's
gate is equal; hand-computed steps with distinct channel decays; an
independent closed-form solve of the window with per-channel decays; the
beta = 0 and beta = 1 special cases; a lifecycle against plain replay of the
committed records; and the ring write's positions.  CPU only.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import closed_form
from oracle.cursors import CursorState, advance, clamp_write_pos, phys
from linear_attention_speculative_spec_amd import synth

import helpers

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def setup_module(_m):
    oracle.build(force=True)


def _shape(**kw):
    base = dict(B=3, T=3, H=2, HV=4, K=8, V=6, L=16, max_spec=4, num_slots=5, act="f32")
    base.update(kw)
    return synth.LayerShape(**base)


def test_kda_gate_is_the_gdn_gate_of_each_channel():
    rng = synth.make_rng(201)
    for _ in range(10):
        a = rng.normal(size=7)
        dt = rng.normal(size=7) * 0.1
        b, A_log = rng.normal(), rng.normal()
        g, beta = oracle.kda_gate(a, b, A_log, dt)
        for c in range(7):
            gc, bc = oracle.gate(a[c], b, A_log, dt[c])
            assert g[c] == gc and beta == bc


def test_kda_step_with_equal_channel_gates_is_the_gdn_step():
    rng = synth.make_rng(202)
    for _ in range(5):
        S = rng.normal(size=(6, 9))
        k, v = rng.normal(size=9), rng.normal(size=6)
        g, beta = -abs(rng.normal()), rng.uniform(0, 1)
        np.testing.assert_array_equal(oracle.kda_step(S, k, v, np.full(9, g), beta),
                                      oracle.step(S, k, v, g, beta))


def test_kda_step_hand_computed():
    with open(os.path.join(GOLDEN, "kda_step_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        out = oracle.kda_step(np.array(c["S"], float), c["k"], c["v"], c["g"], c["beta"], c["eps"])
        np.testing.assert_allclose(out, np.array(c["expect"], float), rtol=0, atol=1e-13)


def test_kda_beta_special_cases():
    rng = synth.make_rng(203)
    S = rng.normal(size=(5, 7))
    k, v = rng.normal(size=7), rng.normal(size=5)
    g = -np.abs(rng.normal(size=7))
    # beta = 0: each key channel only decays
    np.testing.assert_allclose(oracle.kda_step(S, k, v, g, 0.0), S * np.exp(g)[None, :],
                               rtol=1e-15, atol=0)
    # beta = 1: the value is written along the normalised key
    out = oracle.kda_step(S, k, v, g, 1.0, eps=0.0)
    np.testing.assert_allclose(out @ (k / np.linalg.norm(k)), v, rtol=0, atol=1e-12)


def _prefilled(shape, seed, wp_by_slot, base_by_slot, variant="base"):
    rng = synth.make_rng(seed)
    p = synth.kda_layer_params(rng, shape, variant)
    layer = oracle.OracleKDA(shape, p.A_log, p.dt_bias, p.S0)
    slots = synth.slot_choice(rng, shape)
    nrec = int(max(wp_by_slot))
    hist = synth.kda_history_windows(rng, shape, nrec, variant)
    cur = CursorState.zeros(shape.num_slots)
    cur.cache_base[:] = base_by_slot
    for r, (sl, w) in enumerate(zip(helpers.prefill_plan(slots, wp_by_slot, nrec), hist)):
        cur.write_pos[:] = r
        layer.write_ring(cur, sl, helpers.win_f64(w, shape.act), T=1)
    cur.write_pos[:] = wp_by_slot
    cur.is_flush[:] = 0
    win = synth.kda_window(rng, shape, variant)
    return layer, cur, slots, hist, win, p


@pytest.mark.parametrize("variant", ["base", "low_decay", "beta_high"])
def test_kda_recurrence_matches_closed_form(variant):
    shape = _shape(scale=0.7)
    wp = np.array([0, 5, 13, 9, 1], dtype=np.int32)
    base = np.array([3, 14, 9, 0, 15], dtype=np.int32)
    layer, cur, slots, _, win, p = _prefilled(shape, 211, wp, base, variant)
    q, k, v, a, b = helpers.win_f64(win, shape.act)
    o = layer.verify(cur, slots, (q, k, v, a, b), write_ring=False, fold_flagged=False)
    G = shape.HV // shape.H
    worst = 0.0
    for row, s in enumerate(slots):
        s = int(s)
        hist = clamp_write_pos(cur.write_pos[s], shape.L, shape.T)
        for hv in range(shape.HV):
            h = hv // G
            ph = [phys(cur.cache_base[s], j, shape.L) for j in range(hist)]
            keys = [layer.rawk[s, h, x] for x in ph]
            vals = [layer.rawv[s, hv, x] for x in ph]
            gs = [layer.g[s, hv, x] for x in ph]
            bs = [layer.beta[s, hv, x] for x in ph]
            for t in range(shape.T):
                tok = row * shape.T + t
                g, beta = oracle.kda_gate(a[tok, hv], b[tok, hv], p.A_log[hv], p.dt_bias[hv])
                keys.append(k[tok, h])
                vals.append(v[tok, hv])
                gs.append(g)
                bs.append(beta)
            qs = np.stack([q[row * shape.T + t, h] for t in range(shape.T)])
            ref = closed_form.kda_window_outputs(layer.S[s, hv], np.stack(keys), np.stack(vals),
                                                 np.stack(gs), np.array(bs), qs, hist,
                                                 shape.scale, shape.l2norm_eps)
            worst = max(worst, helpers.max_rel(o[row * shape.T:(row + 1) * shape.T, hv], ref))
    assert worst < 1e-12, worst


def test_kda_closed_form_with_equal_channel_gates_is_the_gdn_closed_form():
    rng = synth.make_rng(212)
    n, K, V, T = 7, 5, 4, 3
    S0 = rng.normal(size=(V, K))
    keys, vals = rng.normal(size=(n, K)), rng.normal(size=(n, V))
    g = -np.abs(rng.normal(size=n))
    beta = rng.uniform(0.1, 0.9, size=n)
    qs = rng.normal(size=(T, K))
    a = closed_form.window_outputs(S0, keys, vals, g, beta, qs, n - T, 0.9)
    b = closed_form.kda_window_outputs(S0, keys, vals, np.repeat(g[:, None], K, axis=1), beta, qs,
                                       n - T, 0.9)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_kda_ring_write_is_a_side_channel_and_lands_at_write_pos():
    shape = _shape()
    wp = np.array([3, 0, 8, 12, 5], np.int32)
    base = np.array([1, 15, 12, 6, 0], np.int32)
    layer, cur, slots, _, win, p = _prefilled(shape, 221, wp, base)
    win64 = helpers.win_f64(win, shape.act)
    before = {n: getattr(layer, n).copy() for n in ("rawk", "rawv", "g", "beta")}
    o_off = layer.verify(cur, slots, win64, write_ring=False)
    o_on = layer.verify(cur, slots, win64, write_ring=True)
    assert np.array_equal(o_off, o_on)
    q, k, v, a, b = win64
    expect = {n: x.copy() for n, x in before.items()}
    for row, s in enumerate(slots):
        for t in range(shape.T):
            ps = phys(base[s], wp[s] + t, shape.L)
            tok = row * shape.T + t
            expect["rawk"][s, :, ps] = k[tok]
            expect["rawv"][s, :, ps] = v[tok]
            for hv in range(shape.HV):
                g, beta = oracle.kda_gate(a[tok, hv], b[tok, hv], p.A_log[hv], p.dt_bias[hv])
                expect["g"][s, hv, ps] = g
                expect["beta"][s, hv, ps] = beta
    for n in expect:
        np.testing.assert_array_equal(getattr(layer, n), expect[n], err_msg=n)


def test_kda_lifecycle_matches_plain_replay_of_committed_records():
    """40 verify -> commit steps of a tiny KDA layer, with flushes, against a
    plain per-slot list of committed records replayed from the original
    checkpoint by the pinned step."""
    shape = _shape(B=2, T=4, H=2, HV=4, K=8, V=6, L=16, max_spec=4, num_slots=4, scale=1.1)
    rng = synth.make_rng(231)
    p = synth.kda_layer_params(rng, shape, "low_decay")
    layer = oracle.OracleKDA(shape, p.A_log, p.dt_bias, p.S0)
    slots = synth.slot_choice(rng, shape)
    cur = CursorState.zeros(shape.num_slots)
    cur.cache_base[:] = rng.integers(0, shape.L, size=shape.num_slots)
    committed = {int(s): [] for s in slots}
    accepts = synth.accept_counts(rng, shape.B, shape.T, 40)
    S_orig = p.S0.astype(np.float64)
    G = shape.HV // shape.H
    flushes = 0
    for step_i in range(40):
        win64 = helpers.win_f64(synth.kda_window(rng, shape, "low_decay"), shape.act)
        flushes += int(cur.is_flush[slots].sum())
        o = layer.verify(cur, slots, win64, write_ring=True, fold_flagged=True)
        q, k, v, a, b = win64
        for row, s in enumerate(slots):
            s = int(s)
            for hv in range(shape.HV):
                h = hv // G
                Sref = S_orig[s, hv].copy()
                for (kk, vv, aa, bb) in committed[s]:
                    g, beta = oracle.kda_gate(aa[hv], bb[hv], p.A_log[hv], p.dt_bias[hv])
                    Sref = oracle.kda_step(Sref, kk[h], vv[hv], g, beta, shape.l2norm_eps)
                for t in range(shape.T):
                    tok = row * shape.T + t
                    g, beta = oracle.kda_gate(a[tok, hv], b[tok, hv], p.A_log[hv], p.dt_bias[hv])
                    Sref = oracle.kda_step(Sref, k[tok, h], v[tok, hv], g, beta, shape.l2norm_eps)
                    ref = oracle.kda_readout(Sref, q[tok, h], shape.scale, shape.l2norm_eps)
                    np.testing.assert_allclose(o[tok, hv], ref, rtol=1e-11, atol=1e-13)
            for t in range(int(accepts[step_i, row])):
                tok = row * shape.T + t
                committed[s].append((k[tok], v[tok], a[tok], b[tok]))
        advance(cur, slots, accepts[step_i], shape.L, shape.T, shape.max_spec)
    assert flushes >= 2


def test_kda_fold_consumes_exactly_the_committed_records():
    shape = _shape()
    wp = np.array([12, 0, 7, 3, 9], np.int32)
    base = np.array([9, 2, 14, 0, 5], np.int32)
    layer, cur, slots, hist, _, p = _prefilled(shape, 241, wp, base)
    cur.is_flush[:] = 1
    S_before = layer.S.copy()
    layer.fold(cur, slots, only_flagged=True)
    G = shape.HV // shape.H
    for row, s in enumerate(slots):
        for hv in range(shape.HV):
            h = hv // G
            Sref = S_before[s, hv]
            for r in range(wp[s]):
                q, k, v, a, b = helpers.win_f64(hist[r], shape.act)
                g, beta = oracle.kda_gate(a[row, hv], b[row, hv], p.A_log[hv], p.dt_bias[hv])
                Sref = oracle.kda_step(Sref, k[row, h], v[row, hv], g, beta, shape.l2norm_eps)
            np.testing.assert_allclose(layer.S[s, hv], Sref, rtol=1e-13, atol=1e-15)
    for s in set(range(shape.num_slots)) - set(slots.tolist()):
        assert np.array_equal(layer.S[s], S_before[s])
