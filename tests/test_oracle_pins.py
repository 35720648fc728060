"""Pins of the fp64 oracle to things other than itself.

Each test fixes the oracle against the pages' printed examples, a closed form
derived independently, a textbook special case or an invariant, chosen so a
plausible mistake (a dropped term, a wrong sign or index, a transposed
operand, a wrong ring address) fails one of them.  CPU only.
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


# ------------------------------------------------------------------ gating

def test_gate_special_values():
    # a + dt_bias = 0: softplus(0) = ln 2, so g = -e^{A_log} ln 2; b = 0: beta = 1/2
    g, beta = oracle.gate(0.3, 0.0, math.log(5.0), -0.3)
    assert g == pytest.approx(-5.0 * math.log(2.0), rel=1e-14)
    assert beta == 0.5
    # exact values: sigmoid(ln 3) = 3/4 and softplus(ln 3) = ln 4
    g, beta = oracle.gate(math.log(3.0), math.log(3.0), 0.0, 0.0)
    assert beta == pytest.approx(0.75, rel=1e-15)
    assert g == pytest.approx(-math.log(4.0), rel=1e-15)
    g, beta = oracle.gate(-math.log(3.0), -math.log(3.0), math.log(2.0), 0.0)
    assert beta == pytest.approx(0.25, rel=1e-15)
    assert g == pytest.approx(-2.0 * math.log(4.0 / 3.0), rel=1e-14)
    # above the threshold softplus is the identity
    g, _ = oracle.gate(25.0, 0.0, 0.0, 0.0, threshold=20.0)
    assert g == -25.0
    # softplus(x) - softplus(-x) = x and sigmoid(x) + sigmoid(-x) = 1
    for x in (-3.7, -0.2, 0.9, 6.1):
        gp, bp = oracle.gate(x, x, 0.7, 0.0)
        gm, bm = oracle.gate(-x, -x, 0.7, 0.0)
        assert gp - gm == pytest.approx(-math.exp(0.7) * x, rel=1e-12)
        assert bp + bm == pytest.approx(1.0, abs=1e-15)
    # gates never exceed 0 and beta stays in (0, 1)
    rng = synth.make_rng(7)
    for a, b, al, db in rng.normal(size=(50, 4)):
        g, beta = oracle.gate(a, b, al, db)
        assert g <= 0.0 and 0.0 < beta < 1.0


def test_rnorm():
    assert oracle.rnorm([3.0, 4.0], eps=0.0) == 0.2
    assert oracle.rnorm([3.0, 4.0], eps=1e-6) == pytest.approx(1.0 / math.sqrt(25.000001), rel=1e-15)


# -------------------------------------------------------------------- step

def test_step_hand_computed():
    with open(os.path.join(GOLDEN, "step_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        out = oracle.step(np.array(c["S"], float), c["k"], c["v"], c["g"], c["beta"], c["eps"])
        np.testing.assert_allclose(out, np.array(c["expect"], float), rtol=0, atol=1e-13)


def test_step_beta_one_writes_value_along_key():
    rng = synth.make_rng(11)
    S = rng.normal(size=(6, 5))
    k = rng.normal(size=5)
    v = rng.normal(size=6)
    out = oracle.step(S, k, v, -0.4, 1.0, eps=0.0)
    khat = k / np.linalg.norm(k)
    np.testing.assert_allclose(out @ khat, v, rtol=0, atol=1e-12)


def test_step_beta_zero_is_pure_decay():
    rng = synth.make_rng(12)
    S = rng.normal(size=(4, 7))
    out = oracle.step(S, rng.normal(size=7), rng.normal(size=4), -1.3, 0.0)
    np.testing.assert_allclose(out, math.exp(-1.3) * S, rtol=1e-15, atol=0)


def test_step_contracts_without_injection():
    # with v = 0 the step is S e^g (I - beta k k^T): never grows in Frobenius norm
    rng = synth.make_rng(13)
    S = rng.normal(size=(8, 8))
    for _ in range(30):
        n0 = np.linalg.norm(S)
        S = oracle.step(S, rng.normal(size=8), np.zeros(8), -abs(rng.normal()) * 0.1,
                        rng.uniform(0, 1))
        assert np.linalg.norm(S) <= n0 * (1 + 1e-12)


def test_readout_is_state_times_normalised_query():
    S = np.array([[1.0, 2.0], [3.0, 4.0]])
    o = oracle.readout(S, [0.0, 5.0], scale=0.5, eps=0.0)
    np.testing.assert_allclose(o, [1.0, 2.0], rtol=0, atol=1e-15)


# --------------------------------------------------------- closed-form pins

def _tiny_shape(**kw):
    base = dict(B=3, T=3, H=2, HV=4, K=8, V=6, L=16, max_spec=4, num_slots=5, act="f32")
    base.update(kw)
    return synth.LayerShape(**base)


def _prefilled_layer(shape, seed, wp_by_slot, base_by_slot, variant="base"):
    rng = synth.make_rng(seed)
    p = synth.layer_params(rng, shape, variant)
    layer = oracle.OracleLayer(shape, p.A_log, p.dt_bias, p.S0)
    slots = synth.slot_choice(rng, shape)
    nrec = int(max(wp_by_slot)) if len(wp_by_slot) else 0
    hist = synth.history_windows(rng, shape, nrec, variant)
    cur = CursorState.zeros(shape.num_slots)
    cur.cache_base[:] = base_by_slot
    for r, (sl, w) in enumerate(zip(helpers.prefill_plan(slots, wp_by_slot, nrec), hist)):
        cur.write_pos[:] = r
        layer.write_ring(cur, sl, helpers.win_f64(w, shape.act), T=1)
    cur.write_pos[:] = wp_by_slot
    cur.is_flush[:] = 0
    win = synth.window(rng, shape, variant)
    return layer, cur, slots, hist, win, p


def _closed_form_row(layer, shape, cur, slot, row, hv, hist_windows, win64):
    """Gather the row's history+window sequence and evaluate the closed form."""
    G = shape.HV // shape.H
    h = hv // G
    hist = clamp_write_pos(cur.write_pos[slot], shape.L, shape.T)
    keys, vals, gs, bs = [], [], [], []
    for j in range(hist):
        p = phys(cur.cache_base[slot], j, shape.L)
        keys.append(layer.rawk[slot, h, p])
        vals.append(layer.rawv[slot, hv, p])
        gs.append(layer.g[slot, hv, p])
        bs.append(layer.beta[slot, hv, p])
    q, k, v, a, b = win64
    for t in range(shape.T):
        tok = row * shape.T + t
        g, beta = oracle.gate(a[tok, hv], b[tok, hv], layer.A_log[hv], layer.dt_bias[hv],
                              shape.softplus_threshold)
        keys.append(k[tok, h])
        vals.append(v[tok, hv])
        gs.append(g)
        bs.append(beta)
    queries = np.stack([q[row * shape.T + t, h] for t in range(shape.T)])
    return closed_form.window_outputs(layer.S[slot, hv], np.stack(keys), np.stack(vals),
                                      np.array(gs), np.array(bs), queries, hist,
                                      shape.scale, shape.l2norm_eps)


@pytest.mark.parametrize("variant", ["base", "low_decay", "beta_high"])
def test_recurrence_matches_closed_form(variant):
    shape = _tiny_shape(scale=0.75)
    wp = np.array([0, 5, 13, 9, 1], dtype=np.int32)        # includes empty and max (L-T)
    base = np.array([3, 14, 9, 0, 15], dtype=np.int32)      # wraps around the ring
    layer, cur, slots, hist, win, _ = _prefilled_layer(shape, 21, wp, base, variant)
    win64 = helpers.win_f64(win, shape.act)
    o = layer.verify(cur, slots, win64, write_ring=False, fold_flagged=False)
    worst = 0.0
    for row, s in enumerate(slots):
        for hv in range(shape.HV):
            ref = _closed_form_row(layer, shape, cur, int(s), row, hv, hist, win64)
            got = o[row * shape.T:(row + 1) * shape.T, hv]
            worst = max(worst, helpers.max_rel(got, ref))
    assert worst < 1e-12, worst


def test_unit_lower_inverse_is_the_neumann_series():
    rng = synth.make_rng(5)
    A = np.tril(rng.normal(size=(9, 9)) * 0.3, k=-1)
    np.testing.assert_allclose(closed_form.unit_lower_inverse(A), np.linalg.inv(np.eye(9) + A),
                               rtol=0, atol=1e-12)


def test_single_token_window_closed_form():
    # T = 1 with no history: o = scale (e^g S0 qh + beta (v - e^g S0 kh)(kh . qh))
    shape = _tiny_shape(B=1, T=1, num_slots=1, scale=1.3)
    rng = synth.make_rng(31)
    p = synth.layer_params(rng, shape)
    layer = oracle.OracleLayer(shape, p.A_log, p.dt_bias, p.S0)
    win = synth.window(rng, shape)
    q, k, v, a, b = helpers.win_f64(win, shape.act)
    o = layer.verify(CursorState.zeros(1), np.array([0], np.int32), (q, k, v, a, b),
                     write_ring=False)
    for hv in range(shape.HV):
        h = hv // (shape.HV // shape.H)
        g, beta = oracle.gate(a[0, hv], b[0, hv], p.A_log[hv], p.dt_bias[hv])
        kh = k[0, h] / math.sqrt(k[0, h] @ k[0, h] + shape.l2norm_eps)
        qh = q[0, h] / math.sqrt(q[0, h] @ q[0, h] + shape.l2norm_eps)
        S0 = p.S0[0, hv].astype(np.float64)
        ref = shape.scale * (math.exp(g) * S0 @ qh + beta * (v[0, hv] - math.exp(g) * S0 @ kh) * (kh @ qh))
        np.testing.assert_allclose(o[0, hv], ref, rtol=1e-12, atol=1e-14)


def test_orthogonal_keys_decouple_the_window():
    # mutually orthogonal keys make A = 0, so each token's delta is its own residual
    shape = _tiny_shape(B=1, T=4, H=1, HV=1, K=8, V=3, num_slots=1)
    rng = synth.make_rng(41)
    p = synth.layer_params(rng, shape)
    layer = oracle.OracleLayer(shape, p.A_log, p.dt_bias, p.S0)
    win = synth.window(rng, shape)
    q, k, v, a, b = helpers.win_f64(win, shape.act)
    k = np.zeros_like(k)
    for t in range(4):
        k[t, 0, 2 * t] = 1.0 + t                               # disjoint supports
    o = layer.verify(CursorState.zeros(1), np.array([0], np.int32), (q, k, v, a, b),
                     write_ring=False)
    S0 = p.S0[0, 0].astype(np.float64)
    gs = [oracle.gate(a[t, 0], b[t, 0], p.A_log[0], p.dt_bias[0]) for t in range(4)]
    Gam = np.cumsum([g for g, _ in gs])
    kh = k[:, 0] / np.sqrt(np.sum(k[:, 0] ** 2, axis=1, keepdims=True) + shape.l2norm_eps)
    d = [gs[t][1] * (v[t, 0] - math.exp(Gam[t]) * S0 @ kh[t]) for t in range(4)]
    for t in range(4):
        qh = q[t, 0] / math.sqrt(q[t, 0] @ q[t, 0] + shape.l2norm_eps)
        ref = math.exp(Gam[t]) * S0 @ qh + sum(math.exp(Gam[t] - Gam[j]) * (kh[j] @ qh) * d[j]
                                               for j in range(t + 1))
        np.testing.assert_allclose(o[t, 0], ref, rtol=1e-12, atol=1e-14)


# ------------------------------------------------- corrected deltas (d ring)

def test_step_delta_is_the_rank_one_factor():
    # S_new - e^g S_old = d kh^T: the delta the oracle reports is exactly what
    # the step adds along the normalised key
    rng = synth.make_rng(17)
    for _ in range(5):
        S = rng.normal(size=(6, 9))
        k, v = rng.normal(size=9), rng.normal(size=6)
        g, beta = -abs(rng.normal()), rng.uniform(0.05, 0.95)
        S1, d = oracle.step_d(S, k, v, g, beta)
        kh = k / math.sqrt(k @ k + 1e-6)
        np.testing.assert_allclose(S1 - math.exp(g) * S, np.outer(d, kh), rtol=0, atol=1e-13)
        np.testing.assert_array_equal(S1, oracle.step(S, k, v, g, beta))


def _prefilled_layer_dcache(shape, seed, wp_by_slot, base_by_slot, variant="base"):
    """Like _prefilled_layer, but the history is committed through one-token
    d-cache verifies, so the d ring holds what those verifies recorded."""
    rng = synth.make_rng(seed)
    p = synth.layer_params(rng, shape, variant)
    layer = oracle.OracleLayer(shape, p.A_log, p.dt_bias, p.S0)
    slots = synth.slot_choice(rng, shape)
    nrec = int(max(wp_by_slot))
    hist = synth.history_windows(rng, shape, nrec, variant)
    cur = CursorState.zeros(shape.num_slots)
    cur.cache_base[:] = base_by_slot
    for r, (sl, w) in enumerate(zip(helpers.prefill_plan(slots, wp_by_slot, nrec), hist)):
        cur.write_pos[:] = r
        layer.verify(cur, sl, helpers.win_f64(w, shape.act), write_ring=True,
                     fold_flagged=False, T=1, dcache=True)
    cur.write_pos[:] = wp_by_slot
    cur.is_flush[:] = 0
    win = synth.window(rng, shape, variant)
    return layer, cur, slots, win


def _sequence(layer, shape, cur, slot, row, hv, win64):
    """(keys, values, g, beta, queries, hist, d_ring_hist) of one (row, value head)."""
    h = hv // (shape.HV // shape.H)
    hist = clamp_write_pos(cur.write_pos[slot], shape.L, shape.T)
    ph = [phys(cur.cache_base[slot], j, shape.L) for j in range(hist)]
    keys = [layer.rawk[slot, h, p] for p in ph]
    vals = [layer.rawv[slot, hv, p] for p in ph]
    gs = [layer.g[slot, hv, p] for p in ph]
    bs = [layer.beta[slot, hv, p] for p in ph]
    dh = np.array([layer.d[slot, hv, p] for p in ph]).reshape(hist, shape.V)
    q, k, v, a, b = win64
    for t in range(shape.T):
        tok = row * shape.T + t
        g, beta = oracle.gate(a[tok, hv], b[tok, hv], layer.A_log[hv], layer.dt_bias[hv],
                              shape.softplus_threshold)
        keys.append(k[tok, h])
        vals.append(v[tok, hv])
        gs.append(g)
        bs.append(beta)
    queries = np.stack([q[row * shape.T + t, h] for t in range(shape.T)])
    return np.stack(keys), np.stack(vals), np.array(gs), np.array(bs), queries, hist, dh


@pytest.mark.parametrize("variant", ["base", "low_decay"])
def test_dcache_route_matches_the_recurrence(variant):
    # The d ring written by one-token d-cache verifies holds the deltas of the
    # full system (each depends only on its prefix), the window's deltas match
    # an independent numpy solve, and the d-cache closed form (history only
    # through stored deltas, a T x T window solve) reproduces the outputs.
    shape = _tiny_shape(scale=0.8)
    wp = np.array([0, 5, 13, 9, 1], dtype=np.int32)
    base = np.array([3, 14, 9, 0, 15], dtype=np.int32)
    layer, cur, slots, win = _prefilled_layer_dcache(shape, 23, wp, base, variant)
    win64 = helpers.win_f64(win, shape.act)
    o = layer.verify(cur, slots, win64, write_ring=False, fold_flagged=False, dcache=True)
    dwin = layer.last_dwin
    worst = {"ring": 0.0, "dwin": 0.0, "out": 0.0, "dw": 0.0}
    for row, s in enumerate(slots):
        s = int(s)
        for hv in range(shape.HV):
            keys, vals, gs, bs, queries, hist, dh = _sequence(layer, shape, cur, s, row, hv, win64)
            D = closed_form.deltas(layer.S[s, hv], keys, vals, gs, bs, shape.l2norm_eps)
            got_w = dwin[row * shape.T:(row + 1) * shape.T, hv]
            if hist:
                worst["ring"] = max(worst["ring"], helpers.max_rel(dh, D[:hist]))
            worst["dwin"] = max(worst["dwin"], helpers.max_rel(got_w, D[hist:]))
            out, Dw = closed_form.dcache_window(layer.S[s, hv], D[:hist], keys, vals, gs, bs,
                                               queries, hist, shape.scale, shape.l2norm_eps)
            worst["out"] = max(worst["out"], helpers.max_rel(o[row * shape.T:(row + 1) * shape.T, hv], out))
            worst["dw"] = max(worst["dw"], helpers.max_rel(got_w, Dw))
    assert max(worst.values()) < 1e-12, worst


def test_dcache_ring_write_lands_at_write_pos():
    shape = _tiny_shape()
    wp = np.array([3, 0, 8, 12, 5], np.int32)
    layer, cur, slots, win = _prefilled_layer_dcache(shape, 27, wp, np.array([1, 4, 15, 7, 0], np.int32))
    slots = slots.copy()
    slots[1] = -1                                   # a padding row writes nothing
    before = layer.d.copy()
    win64 = helpers.win_f64(win, shape.act)
    o_plain = layer.verify(cur, slots, win64, write_ring=False, fold_flagged=False)
    o = layer.verify(cur, slots, win64, write_ring=True, fold_flagged=False, dcache=True)
    assert np.array_equal(o, o_plain, equal_nan=True)   # the d ring changes no output
    written = np.zeros(layer.d.shape[:3], bool)
    for row, s in enumerate(slots):
        if s < 0:
            continue
        for t in range(shape.T):
            p = phys(cur.cache_base[s], int(cur.write_pos[s]) + t, shape.L)
            written[s, :, p] = True
            np.testing.assert_array_equal(layer.d[s, :, p], layer.last_dwin[row * shape.T + t])
    same = ~written
    assert np.array_equal(np.isnan(layer.d[same]), np.isnan(before[same]))
    np.testing.assert_array_equal(np.nan_to_num(layer.d[same]), np.nan_to_num(before[same]))


def test_one_pass_dring_fill_equals_one_token_verifies():
    # the one-pass fill (used to pre-fill large d rings in the GPU tests)
    # stores exactly the deltas that one-token d-cache verifies recorded
    shape = _tiny_shape()
    wp = np.array([0, 5, 13, 9, 1], dtype=np.int32)
    base = np.array([3, 14, 9, 0, 15], dtype=np.int32)
    layer, cur, slots, _ = _prefilled_layer_dcache(shape, 27, wp, base, "low_decay")
    other = oracle.OracleLayer(shape, layer.A_log, layer.dt_bias, layer.S)
    for n in ("rawk", "rawv", "g", "beta"):
        setattr(other, n, getattr(layer, n).copy())
    other.fill_dring(cur, slots)
    for s in slots:
        for j in range(int(wp[s])):
            p = phys(base[s], j, shape.L)
            np.testing.assert_allclose(other.d[s, :, p], layer.d[s, :, p], rtol=1e-14, atol=1e-16)
            assert not np.isnan(other.d[s, :, p]).any()
    # nothing past the committed records is written
    for s in slots:
        for j in range(int(wp[s]), shape.L):
            assert np.isnan(other.d[s, :, phys(base[s], j, shape.L)]).all()


# ------------------------------------------------------- structural invariants

def test_causality_later_tokens_do_not_change_earlier_outputs():
    shape = _tiny_shape()
    wp = np.array([4, 2, 7, 0, 11], np.int32)
    layer, cur, slots, _, win, _ = _prefilled_layer(shape, 51, wp, np.arange(5, dtype=np.int32) * 3)
    win64 = [x.copy() for x in helpers.win_f64(win, shape.act)]
    o1 = layer.verify(cur, slots, tuple(win64), write_ring=False, fold_flagged=False)
    for x in win64:                       # perturb the last token of every row
        x[shape.T - 1::shape.T] += 0.5
    o2 = layer.verify(cur, slots, tuple(win64), write_ring=False, fold_flagged=False)
    for t in range(shape.T - 1):
        assert np.array_equal(o1[t::shape.T], o2[t::shape.T])
    assert not np.array_equal(o1[shape.T - 1::shape.T], o2[shape.T - 1::shape.T])


def test_cache_base_shift_leaves_outputs_unchanged():
    shape = _tiny_shape()
    wp = np.array([6, 9, 3, 12, 0], np.int32)
    outs = []
    for base in (np.zeros(5, np.int32), np.array([15, 7, 10, 2, 9], np.int32)):
        layer, cur, slots, _, win, _ = _prefilled_layer(shape, 61, wp, base)
        outs.append(layer.verify(cur, slots, helpers.win_f64(win, shape.act), write_ring=False))
    assert np.array_equal(outs[0], outs[1])


def test_ring_write_is_a_pure_side_channel_and_lands_at_write_pos():
    shape = _tiny_shape()
    wp = np.array([3, 0, 8, 12, 5], np.int32)
    base = np.array([1, 15, 12, 6, 0], np.int32)
    layer, cur, slots, _, win, _ = _prefilled_layer(shape, 71, wp, base)
    win64 = helpers.win_f64(win, shape.act)
    before = {n: getattr(layer, n).copy() for n in ("rawk", "rawv", "g", "beta")}
    o_off = layer.verify(cur, slots, win64, write_ring=False)
    o_on = layer.verify(cur, slots, win64, write_ring=True)
    assert np.array_equal(o_off, o_on)
    q, k, v, a, b = win64
    expect = {n: x.copy() for n, x in before.items()}
    for row, s in enumerate(slots):
        for t in range(shape.T):
            p = phys(base[s], wp[s] + t, shape.L)
            tok = row * shape.T + t
            expect["rawk"][s, :, p] = k[tok]
            expect["rawv"][s, :, p] = v[tok]
            for hv in range(shape.HV):
                g, beta = oracle.gate(a[tok, hv], b[tok, hv], layer.A_log[hv], layer.dt_bias[hv])
                expect["g"][s, hv, p] = g
                expect["beta"][s, hv, p] = beta
    for n in expect:
        np.testing.assert_array_equal(getattr(layer, n), expect[n], err_msg=n)


def test_lifecycle_matches_plain_replay_of_committed_records():
    """Ring + cursors + fold over the tiny fp32 workload's 40-step loop.

    The reference keeps the committed records as a plain list per slot and
    rebuilds the committed state by stepping through them from the original
    checkpoint: no ring, no cursors, no fold.  A wrong physical index, base
    move, flush rule or fold order changes the oracle's outputs or state.
    """
    shape = synth.CONFIGS["tiny_f32"]
    rng = synth.make_rng(1000)
    p = synth.layer_params(rng, shape)
    layer = oracle.OracleLayer(shape, p.A_log, p.dt_bias, p.S0)
    slots = synth.slot_choice(rng, shape)
    cur = CursorState.zeros(shape.num_slots)
    cur.cache_base[:] = rng.integers(0, shape.L, size=shape.num_slots)
    wp0 = np.zeros(shape.num_slots, np.int32)
    wp0[slots] = 5
    hist = synth.history_windows(rng, shape, 5)
    committed = {int(s): [] for s in slots}
    for r, (sl, w) in enumerate(zip(helpers.prefill_plan(slots, wp0, 5), hist)):
        cur.write_pos[:] = r
        layer.write_ring(cur, sl, helpers.win_f64(w, shape.act), T=1)
        q, k, v, a, b = helpers.win_f64(w, shape.act)
        for row, s in enumerate(sl):
            if s >= 0:
                committed[int(s)].append((k[row], v[row], a[row], b[row]))
    cur.write_pos[:] = wp0
    cur.is_flush[:] = (wp0 + 2 * shape.max_spec > shape.L).astype(np.int32)
    accepts = synth.accept_counts(rng, shape.B, shape.T, 40)
    S_orig = p.S0.astype(np.float64)
    flushes = 0
    for step_i in range(40):
        win = synth.window(rng, shape)
        win64 = helpers.win_f64(win, shape.act)
        flushes += int(cur.is_flush[slots].sum())
        o = layer.verify(cur, slots, win64, write_ring=True, fold_flagged=True)
        q, k, v, a, b = win64
        for row, s in enumerate(slots):
            s = int(s)
            G = shape.HV // shape.H
            for hv in range(shape.HV):
                h = hv // G
                Sref = S_orig[s, hv].copy()
                for (kk, vv, aa, bb) in committed[s]:
                    g, beta = oracle.gate(aa[hv], bb[hv], p.A_log[hv], p.dt_bias[hv])
                    Sref = oracle.step(Sref, kk[h], vv[hv], g, beta, shape.l2norm_eps)
                for t in range(shape.T):
                    tok = row * shape.T + t
                    g, beta = oracle.gate(a[tok, hv], b[tok, hv], p.A_log[hv], p.dt_bias[hv])
                    Sref = oracle.step(Sref, k[tok, h], v[tok, hv], g, beta, shape.l2norm_eps)
                    ref = oracle.readout(Sref, q[tok, h], shape.scale, shape.l2norm_eps)
                    np.testing.assert_allclose(o[tok, hv], ref, rtol=1e-11, atol=1e-13)
            for t in range(int(accepts[step_i, row])):
                tok = row * shape.T + t
                committed[s].append((k[tok], v[tok], a[tok], b[tok]))
        advance(cur, slots, accepts[step_i], shape.L, shape.T, shape.max_spec)
        # checkpoint + history replay equals the plain replay at every step
        for s in (int(x) for x in slots):
            wp = clamp_write_pos(cur.write_pos[s], shape.L, shape.T)
            folded = len(committed[s]) - wp
            for hv in range(2):
                h = hv // (shape.HV // shape.H)
                Sref = S_orig[s, hv].copy()
                for (kk, vv, aa, bb) in committed[s][:folded]:
                    g, beta = oracle.gate(aa[hv], bb[hv], p.A_log[hv], p.dt_bias[hv])
                    Sref = oracle.step(Sref, kk[h], vv[hv], g, beta, shape.l2norm_eps)
                np.testing.assert_allclose(layer.S[s, hv], Sref, rtol=1e-11, atol=1e-13)
    assert flushes >= 2      # the loop must exercise the fold


# ------------------------------------------------------------------ cursors

def test_cursor_walks_printed_on_the_pages():
    with open(os.path.join(GOLDEN, "cursor_walks.json")) as f:
        gold = json.load(f)
    for w in gold["walks"]:
        L, T, M = w["L"], w["T"], w["max_spec"]
        cur = CursorState.zeros(1)
        cur.write_pos[0] = w["start"]["write_pos"]
        cur.cache_base[0] = w["start"]["cache_base"]
        cur.is_flush[0] = w["start"]["is_flush"]
        for st in w["steps"]:
            wpc = clamp_write_pos(cur.write_pos[0], L, T)
            assert [phys(cur.cache_base[0], wpc + t, L) for t in range(T)] == st["window_phys"], w["cite"]
            advance(cur, np.array([0]), np.array([st["accept"]]), L, T, M)
            got = {"write_pos": int(cur.write_pos[0]), "cache_base": int(cur.cache_base[0]),
                   "is_flush": int(cur.is_flush[0])}
            assert got == st["after"], w["cite"]
    for c in gold["phys"]:
        assert [phys(c["cache_base"], j, c["L"]) for j in c["logical"]] == c["phys"], c["cite"]


@pytest.mark.parametrize("L,T,M", [(16, 4, 4), (64, 4, 4), (128, 8, 8), (64, 3, 4), (8, 2, 2)])
def test_cursor_invariants_over_long_random_walks(L, T, M):
    rng = synth.make_rng(L * 100 + T)
    S = 7
    cur = CursorState.zeros(S)
    cur.cache_base[:] = rng.integers(0, L, size=S)
    slots = np.arange(S, dtype=np.int32)
    committed = np.zeros(S, dtype=np.int64)
    folded = np.zeros(S, dtype=np.int64)
    for _ in range(3000):
        acc = rng.integers(0, T + 1, size=S)
        # the window [wp, wp+T) sits physically after the history, never on it
        for s in range(S):
            hist = 0 if cur.is_flush[s] else int(cur.write_pos[s])
            h_phys = {phys(cur.cache_base[s], j, L) for j in range(hist)}
            w_phys = {phys(cur.cache_base[s], int(cur.write_pos[s]) + t, L) for t in range(T)}
            assert not (h_phys & w_phys) and len(w_phys) == T
            if cur.is_flush[s]:
                folded[s] += int(cur.write_pos[s])
        advance(cur, slots, acc, L, T, M)
        committed += acc
        assert np.all(cur.write_pos >= 0) and np.all(cur.write_pos <= L - T)
        assert np.array_equal(cur.is_flush, (cur.write_pos + 2 * M > L).astype(np.int32))
        assert np.all(cur.cache_base >= 0) and np.all(cur.cache_base < L)
        # nothing is lost: folded + pending history = everything accepted
        assert np.array_equal(folded + cur.write_pos, committed)


def test_padding_rows_and_accept_clamp():
    cur = CursorState.zeros(3)
    cur.write_pos[:] = [2, 5, 1]
    advance(cur, np.array([-1, 1, 7]), np.array([3, 9, 2]), 16, 4, 4)
    assert cur.write_pos.tolist() == [2, 9, 1]          # accept clamped to T=4
    assert cur.is_flush.tolist() == [0, 1, 0]


def test_fold_consumes_exactly_the_committed_records():
    # fold(S0, ring) equals stepping through the same records in logical order
    shape = _tiny_shape()
    wp = np.array([12, 0, 7, 3, 9], np.int32)
    base = np.array([9, 2, 14, 0, 5], np.int32)
    layer, cur, slots, hist, _, p = _prefilled_layer(shape, 81, wp, base)
    cur.is_flush[:] = 1
    S_before = layer.S.copy()
    layer.fold(cur, slots, only_flagged=True)
    for row, s in enumerate(slots):
        for hv in range(shape.HV):
            h = hv // (shape.HV // shape.H)
            Sref = S_before[s, hv]
            for r in range(wp[s]):
                q, k, v, a, b = helpers.win_f64(hist[r], shape.act)
                g, beta = oracle.gate(a[row, hv], b[row, hv], p.A_log[hv], p.dt_bias[hv])
                Sref = oracle.step(Sref, k[row, h], v[row, hv], g, beta, shape.l2norm_eps)
            np.testing.assert_allclose(layer.S[s, hv], Sref, rtol=1e-13, atol=1e-15)
    untouched = [s for s in range(shape.num_slots) if s not in set(slots.tolist())]
    for s in untouched:
        assert np.array_equal(layer.S[s], S_before[s])


# --------------------------------------------------------- snapshot baseline

def test_snapshot_hand_computed_two_token_window():
    # the per-token baseline on a window small enough to follow by hand
    with open(os.path.join(GOLDEN, "snapshot_t2.json")) as f:
        gold = json.load(f)
    g = gold["shape"]
    shape = synth.LayerShape(B=g["B"], T=g["T"], H=g["H"], HV=g["HV"], K=g["K"], V=g["V"],
                             L=g["L"], max_spec=g["max_spec"], num_slots=g["num_slots"],
                             act="f32", scale=g["scale"], l2norm_eps=g["l2norm_eps"])
    S0 = np.array(gold["S0"], float)[None, None]
    layer = oracle.OracleLayer(shape, gold["A_log"], gold["dt_bias"], S0)
    toks = gold["tokens"]
    q = np.array([t["q"] for t in toks], float)[:, None, :]
    k = np.array([t["k"] for t in toks], float)[:, None, :]
    v = np.array([t["v"] for t in toks], float)[:, None, :]
    a = np.array([[t["a"]] for t in toks], float)
    b = np.array([[t["b"]] for t in toks], float)
    o, snap = layer.snapshot(np.array([0], np.int32), (q, k, v, a, b))
    for t, tok in enumerate(toks):
        np.testing.assert_allclose(snap[0, t, 0], np.array(tok["snap"], float), rtol=0, atol=1e-14)
        np.testing.assert_allclose(o[t, 0], np.array(tok["o"], float), rtol=0, atol=1e-14)
    # the checkpoint itself is read, never written
    np.testing.assert_array_equal(layer.S[0, 0], np.array(gold["S0"], float))


def test_snapshot_states_are_folds_of_the_window_prefixes():
    # snap[b, t] is the committed state after accepting t + 1 drafts: the
    # pinned exact fold of the window's records 0..t, recorded at a wrapping
    # base, reproduces it; the outputs are the pinned verify's with an empty
    # history.  Rows, tokens and heads all differ, so a transposed or shifted
    # snapshot index fails.
    shape = _tiny_shape(scale=0.9)
    rng = synth.make_rng(91)
    p = synth.layer_params(rng, shape, "low_decay")
    layer = oracle.OracleLayer(shape, p.A_log, p.dt_bias, p.S0)
    slots = synth.slot_choice(rng, shape)
    slots[1] = -1                                         # one padding row
    win64 = helpers.win_f64(synth.window(rng, shape, "low_decay"), shape.act)
    S_before = layer.S.copy()
    o_snap, snap = layer.snapshot(slots, win64)
    np.testing.assert_array_equal(layer.S, S_before)
    o_ver = layer.verify(CursorState.zeros(shape.num_slots), slots, win64, write_ring=False,
                         fold_flagged=False)
    live = [r for r, s in enumerate(slots) if s >= 0]
    for r in live:
        rows = slice(r * shape.T, (r + 1) * shape.T)
        assert helpers.max_rel(o_snap[rows], o_ver[rows]) < 1e-12
    # the padding row's outputs and snapshots are left as they were (NaN)
    assert np.isnan(o_snap[shape.T:2 * shape.T]).all() and np.isnan(snap[1]).all()
    for t in range(shape.T):
        fold_layer = oracle.OracleLayer(shape, p.A_log, p.dt_bias, p.S0)
        cur = CursorState.zeros(shape.num_slots)
        cur.cache_base[:] = shape.L - 2                   # records 0..t wrap past the ring end
        fold_layer.write_ring(cur, slots, win64)
        cur.write_pos[:] = t + 1
        cur.is_flush[:] = 1
        fold_layer.fold(cur, slots, only_flagged=True)
        for r in live:
            s = int(slots[r])
            np.testing.assert_allclose(snap[r, t], fold_layer.S[s], rtol=0, atol=1e-13)
            assert helpers.max_rel(snap[r, t], fold_layer.S[s]) < 1e-12


# ------------------------------------------------------------- cursor reset

def test_reset_hands_slots_to_decode_with_an_empty_history():
    # replayssm(B)SpecDecode App. A.2: at the prefill -> decode handoff a slot
    # starts over from its checkpoint.  Pinned by behaviour: after the reset
    # a verify of the slot equals the pinned snapshot path (no history), its
    # window lands at physical positions 0..T-1, the next advance starts from
    # zero, other slots keep their cursors, and list entries outside
    # [0, num_slots) are skipped.
    shape = _tiny_shape()
    wp = np.array([7, 3, 12, 0, 9], np.int32)
    base = np.array([5, 14, 9, 2, 11], np.int32)
    layer, cur, slots, _, win, _ = _prefilled_layer(shape, 101, wp, base)
    cur.is_flush[:] = [0, 1, 0, 0, 1]
    win64 = helpers.win_f64(win, shape.act)
    targets = [int(slots[0]), int(slots[2])]
    for init_flush in (0, 1):
        c = cur.copy()
        oracle.reset(c, targets + [-1, shape.num_slots, 10 ** 6], init_flush=init_flush)
        for s in range(shape.num_slots):
            if s in targets:
                assert (c.write_pos[s], c.cache_base[s], c.is_flush[s]) == (0, 0, init_flush)
            else:
                assert (c.write_pos[s], c.cache_base[s], c.is_flush[s]) == \
                    (cur.write_pos[s], cur.cache_base[s], cur.is_flush[s])
        lay = oracle.OracleLayer(shape, layer.A_log, layer.dt_bias, layer.S)
        for n in ("rawk", "rawv", "g", "beta"):
            setattr(lay, n, getattr(layer, n).copy())
        S_before = lay.S.copy()
        o = lay.verify(c, slots, win64, write_ring=True, fold_flagged=True)
        o_snap, _ = lay.snapshot(slots, win64)
        q, k, v, a, b = win64
        for row in (0, 2):
            s = int(slots[row])
            rows = slice(row * shape.T, (row + 1) * shape.T)
            assert helpers.max_rel(o[rows], o_snap[rows]) < 1e-12
            np.testing.assert_array_equal(lay.S[s], S_before[s])   # nothing was folded
            for t in range(shape.T):
                np.testing.assert_array_equal(lay.rawk[s, :, t], k[row * shape.T + t])
                np.testing.assert_array_equal(lay.rawv[s, :, t], v[row * shape.T + t])
        acc = np.arange(len(slots), dtype=np.int32) % (shape.T + 1)
        advance(c, slots, acc, shape.L, shape.T, shape.max_spec)
        for row in (0, 2):
            s = int(slots[row])
            assert (c.write_pos[s], c.cache_base[s]) == (acc[row], 0)
