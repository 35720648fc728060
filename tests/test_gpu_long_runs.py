"""GPU parity at the full workload sizes and over long runs.

* the bandwidth-bound batch (B=256 rows over 512 slots) in the launch
  configuration the benchmark times, every row and value head checked;
* the long-window stress (T=8, L=128, B=64): thousands of
  verify -> commit -> flush iterations, the drift of the checkpoint against the
  fp64 oracle logged at every flush of the rows the oracle follows;
* the 48-layer chain (B=128, T=4, L=64): each layer's inputs are a seeded
  random linear map of the previous layer's RMS-normalised outputs.  The
  oracle runs its own glue from its own outputs (its inputs never come from
  the GPU); the rows it follows are teacher-forced on the GPU side with the
  oracle's next-layer inputs, so every layer is checked on identical inputs
  and rounding differences do not compound through the stack.  The gap
  between the GPU's own next-layer inputs and the oracle's is reported.

Bars as in the other parity tests: cursors bit-exact; outputs and checkpoints
within max|x-ref|/max|ref| of 3e-2 (bf16 activations).
"""
from __future__ import annotations

import os
import time

import numpy as np
import pytest
import torch

import oracle
from oracle.cursors import CursorState, advance
from linear_attention_speculative_spec_amd import gdnverify as gv
from linear_attention_speculative_spec_amd import synth

import helpers
from gpu_harness import (DEV, Pair, dev_cursors, dev_i32, host_bits, host_cursors, host_f64,
                         require_gpu)

pytestmark = pytest.mark.gpu

TOL = {synth.ACT_F32: 2e-3, synth.ACT_BF16: 3e-2}


def say(*a):
    print(*a, flush=True)


def _cursors_equal(dcur, cur: CursorState, where):
    got = host_cursors(dcur)
    for name in ("write_pos", "cache_base", "is_flush"):
        assert np.array_equal(getattr(got, name), getattr(cur, name)), (name, where)


class _DevWin:
    def __init__(self, d):
        self.q, self.k, self.v, self.a, self.b = d["q"], d["k"], d["v"], d["a"], d["b"]


# ------------------------------------------------- bandwidth-bound batch, B=256

FOLD_TIGHT = 1e-5   # the fold is fp32 arithmetic on exactly widened records


def test_bandwidth_batch_b256_all_rows():
    """Four steps at B=256 / 512 slots, fold then verify as the benchmark
    launches them, every row and value head compared with the oracle.

    Besides the spec bar, folded checkpoints meet a tight internal bar: the
    fold runs in fp32 on exactly widened records, so it lands within about
    1e-7 of the fp64 fold; FOLD_TIGHT catches a fold error far below 3e-2."""
    require_gpu()
    shape = synth.CONFIGS["qwen3next_b256"]
    rng = synth.make_rng(1102)
    slots = synth.slot_choice(rng, shape)
    cd = synth.random_cursors(rng, shape)
    P = Pair(shape, 1002, slots=slots, wp_by_slot=cd.write_pos, base_by_slot=cd.cache_base)
    say(f"b256: all {shape.B} rows followed, "
        f"{int(P.cur.is_flush[P.slots].sum())} flagged at the start")
    tol = TOL[shape.act]
    g = P.gpu
    sel = torch.from_numpy(P.slots.astype(np.int64)).to(DEV)
    folded_total = 0
    for step_i in range(4):
        win = P.window()
        o = g.new_out()
        S_before = g.S.clone()
        fl = P.cur.is_flush[P.slots].astype(bool)
        gv.gdn_exact_fold(g.gs, 1, 0, 0, g.S, *g.ring(), P.dslots, *P.dcur, 1)
        g.verify(P.dcur, P.dslots, helpers_devwin(win, shape.act), o, write_ring=1,
                 fold_flagged=0)
        ref = P.oracle_verify(win)
        got = P.gpu_out_rows(o)
        err = helpers.max_rel(got, ref)
        eerr = helpers.elem_rel(got, ref)
        # every output written and finite; unflagged checkpoints bitwise untouched
        assert bool(torch.isfinite(o.float()).all())
        keep = torch.from_numpy(P.slots[~fl].astype(np.int64)).to(DEV)
        assert torch.equal(g.S.index_select(0, keep), S_before.index_select(0, keep))
        del S_before
        Sg = host_f64(g.S.index_select(0, sel))
        serr = helpers.max_rel(Sg, P.orc.S)
        ferr = helpers.max_rel(Sg[fl], P.orc.S[fl]) if fl.any() else 0.0
        folded_total += int(fl.sum())
        helpers.report(f"b256 step {step_i}: {shape.B} rows x {shape.HV} heads, max_rel(o) = {err:.2e}, "
                       f"elementwise rel(o) = {eerr:.2e}, max_rel(S) = {serr:.2e}, "
                       f"folded rows ({int(fl.sum())}) max_rel(S) = {ferr:.2e}")
        assert err <= tol, err
        assert serr <= tol, serr
        assert ferr <= FOLD_TIGHT, ferr
        del Sg
        acc = P.rng.integers(0, shape.T + 1, size=shape.B).astype(np.int32)
        gv.gdn_advance_cursors(g.gs, P.dslots, dev_i32(acc), *P.dcur)
        advance(P.cur, P.slots, acc, shape.L, shape.T, shape.max_spec)
        advance(P.ocur, P.oslots, acc[P.orows], shape.L, shape.T, shape.max_spec)
        _cursors_equal(P.dcur, P.cur, step_i)
    assert folded_total >= 8


def test_padding_rows_interleaved_at_full_size():
    """B=256 with half the rows padding, alternating along every workgroup's
    sequence of items (rows 16 apart): the valid rows' outputs are bitwise
    those of the same call without padding, padding rows are left untouched,
    and sampled valid rows match the oracle."""
    require_gpu()
    shape = synth.CONFIGS["qwen3next_b256"]
    rng = synth.make_rng(1202)
    pad = (np.arange(shape.B) // 16) % 2 == 1
    pad |= rng.random(shape.B) < 0.1
    valid_rows = np.flatnonzero(~pad)
    pick = np.sort(rng.choice(valid_rows, 6, replace=False))
    P = Pair(shape, 1202, oracle_rows=pick)
    g = P.gpu
    win = P.window()
    dwin = helpers_devwin(win, shape.act)
    o_full = g.new_out()
    g.verify(P.dcur, P.dslots, dwin, o_full, write_ring=0, fold_flagged=0)
    slots = P.slots.copy()
    slots[pad] = -1
    slots[np.flatnonzero(pad)[::7]] = shape.num_slots       # out of range counts as padding too
    o_pad = g.new_out()
    sentinel = host_bits(o_pad)
    g.verify(P.dcur, dev_i32(slots), dwin, o_pad, write_ring=0, fold_flagged=0)
    a, b_ = host_bits(o_full), host_bits(o_pad)
    tok_valid = np.repeat(~pad, shape.T)
    assert np.array_equal(b_[tok_valid], a[tok_valid]), "valid rows changed by padding elsewhere"
    assert np.array_equal(b_[~tok_valid], sentinel[~tok_valid]), "padding rows written"
    ref = P.oracle_verify(win, write_ring=False, fold_flagged=False)
    err = helpers.max_rel(P.gpu_out_rows(o_pad), ref)
    say(f"padding interleaved: {int(pad.sum())} padding rows, max_rel(o) = {err:.2e}")
    assert err <= TOL[shape.act]


def helpers_devwin(win: synth.Window, act: str):
    from gpu_harness import DevWindow
    return DevWindow(win, act)


# ------------------------------------------------- fold-every-commit design

def test_fold_every_commit_matches_ring_with_history():
    """The fold-every-commit design (a ring of 2T records holding only the
    window; every commit folded into the checkpoint at once, then the cursors
    reset) against the oracle, and against the ring-with-history design on the
    same inputs and accept counts: both compute the same outputs, and the
    committed states agree."""
    require_gpu()
    shape_r = synth.CONFIGS["qwen3next_b32"]
    shape_f = shape_r.replace(L=2 * shape_r.max_spec)
    steps = 12
    zeros = np.zeros(shape_r.num_slots, np.int32)
    Pr = Pair(shape_r, 2600, "low_decay", wp_by_slot=zeros, base_by_slot=zeros)
    Pf = Pair(shape_f, 2600, "low_decay", wp_by_slot=zeros, base_by_slot=zeros, slots=Pr.slots)
    assert np.array_equal(Pr.params.S0, Pf.params.S0)
    wrng = synth.make_rng(2601)
    accepts = synth.accept_counts(wrng, shape_r.B, shape_r.T, steps)
    tol = TOL[shape_r.act]
    for i in range(steps):
        win = synth.window(wrng, shape_r, "low_decay")
        dwin = helpers_devwin(win, shape_r.act)
        acc = accepts[i]
        # ring with history
        o_r = Pr.gpu.new_out()
        Pr.gpu.verify(Pr.dcur, Pr.dslots, dwin, o_r)
        gv.gdn_advance_cursors(Pr.gpu.gs, Pr.dslots, dev_i32(acc), *Pr.dcur)
        advance(Pr.cur, Pr.slots, acc, shape_r.L, shape_r.T, shape_r.max_spec)
        _cursors_equal(Pr.dcur, Pr.cur, i)
        # fold every commit: the verify sees no history
        o_f = Pf.gpu.new_out()
        Pf.gpu.verify(Pf.dcur, Pf.dslots, dwin, o_f, fold_flagged=0)
        ref = Pf.oracle_verify(win, fold_flagged=False)
        gv.gdn_advance_cursors(Pf.gpu.gs, Pf.dslots, dev_i32(acc), *Pf.dcur)
        gv.gdn_exact_fold(Pf.gpu.gs, 1, 0, 0, Pf.gpu.S, *Pf.gpu.ring(), Pf.dslots, *Pf.dcur, 0)
        gv.gdn_reset_cursors(Pf.gpu.gs, Pf.dslots, shape_f.B, 0, *Pf.dcur)
        advance(Pf.ocur, Pf.oslots, acc, shape_f.L, shape_f.T, shape_f.max_spec)
        Pf.orc.fold(Pf.ocur, Pf.oslots, only_flagged=False)
        oracle.reset(Pf.ocur, Pf.oslots)
        advance(Pf.cur, Pf.slots, acc, shape_f.L, shape_f.T, shape_f.max_spec)
        oracle.reset(Pf.cur, Pf.slots)
        _cursors_equal(Pf.dcur, Pf.cur, i)
        err_o = helpers.max_rel(Pf.gpu_out_rows(o_f), ref)
        err_rf = helpers.max_rel(host_f64(o_f), host_f64(o_r))
        assert err_o <= tol, (i, err_o)
        assert err_rf <= tol, (i, err_rf)
    # the committed states: the history design folds what its ring still holds
    S_r = Pr.gpu.S.clone()
    fl = dev_i32(np.ones(shape_r.num_slots))
    gv.gdn_exact_fold(Pr.gpu.gs, 1, 0, 0, S_r, *Pr.gpu.ring(), Pr.dslots, Pr.dcur[0], Pr.dcur[1], fl, 0)
    sel = torch.from_numpy(Pr.slots.astype(np.int64)).to(DEV)
    err_s = helpers.max_rel(host_f64(S_r.index_select(0, sel)), host_f64(Pf.gpu.S.index_select(0, sel)))
    err_so = helpers.max_rel(host_f64(Pf.gpu.S.index_select(0, sel)), Pf.orc.S)
    say(f"fold every commit: {steps} steps, checkpoints vs history design {err_s:.2e}, "
        f"vs oracle {err_so:.2e}")
    assert err_s <= tol and err_so <= tol


# ------------------------------------------------- long-window drift, T=8 L=128

def drift_run(variant: str, iters: int, seed: int, n_orows: int = 4, check_every: int = 32,
              dcache: bool = False):
    """With ``dcache`` the GPU verifies through its ring of stored deltas while
    the oracle keeps replaying the raw records: any drift of the stored fp32
    deltas shows in the outputs."""
    shape = synth.CONFIGS["long_window_t8"]
    pick = np.sort(synth.make_rng(seed + 1).choice(shape.B, n_orows, replace=False))
    P = Pair(shape, seed, variant, oracle_rows=pick, dcache=dcache)
    gpu_verify = P.gpu.verify_dcache if dcache else P.gpu.verify
    dw = synth.DeviceWindows(seed + 2, shape, variant)
    accepts = synth.accept_counts(P.rng, shape.B, shape.T, iters)
    tol = TOL[shape.act]
    gslots_t = torch.from_numpy(P.slots[P.orows].astype(np.int64)).to(DEV)
    nflush = np.zeros(n_orows, np.int64)
    s_curve = []       # (iteration, oracle row, flush number of that row, max_rel S)
    o_curve = []       # (iteration, max_rel o)
    t0 = time.time()
    for i in range(iters):
        win = dw.draw()
        o = P.gpu.new_out()
        flagged = P.ocur.is_flush[P.oslots].astype(bool)
        gpu_verify(P.dcur, P.dslots, _DevWin(win), o)            # folds flagged rows
        w64 = helpers.win_f64(dw.host_rows(win, P.orows, shape.T), shape.act)
        if i % check_every == 0 or i == iters - 1:
            ref = P.orc.verify(P.ocur, P.oslots, w64)
            err = helpers.max_rel(P.gpu_out_rows(o), ref)
            o_curve.append((i, err))
            assert err <= tol, (i, err)
        else:
            if flagged.any():
                P.orc.fold(P.ocur, P.oslots, only_flagged=True)
            P.orc.write_ring(P.ocur, P.oslots, w64)
        if flagged.any():
            Sg = host_f64(P.gpu.S.index_select(0, gslots_t))
            for r in np.flatnonzero(flagged):
                nflush[r] += 1
                err = helpers.max_rel(Sg[r], P.orc.S[r])
                s_curve.append((i, int(r), int(nflush[r]), err))
                assert err <= tol, (i, r, err)
        acc = accepts[i]
        gv.gdn_advance_cursors(P.gpu.gs, P.dslots, dev_i32(acc), *P.dcur)
        advance(P.cur, P.slots, acc, shape.L, shape.T, shape.max_spec)
        advance(P.ocur, P.oslots, acc[P.orows], shape.L, shape.T, shape.max_spec)
        if i % 64 == 0 or i == iters - 1:
            _cursors_equal(P.dcur, P.cur, i)
        if i % 512 == 511:
            say(f"drift {variant}{' d-cache' if dcache else ''}: {i + 1}/{iters} iterations, {int(nflush.sum())} oracle-row "
                f"flushes, {time.time() - t0:.0f}s")
    return s_curve, o_curve


def _drift_iters() -> int:
    return int(os.environ.get("GDN_DRIFT_ITERS", "4096"))


@pytest.mark.parametrize("variant", ["base", "low_decay", "low_decay_dcache"])
def test_long_window_drift_curve(variant):
    iters = _drift_iters()
    dcache = variant.endswith("_dcache")
    law = variant[:-len("_dcache")] if dcache else variant
    s_curve, o_curve = drift_run(law, iters, 1003 if law == "base" else 1013, dcache=dcache)
    # the curve: worst checkpoint error per flush number over the followed rows
    by_flush = {}
    for _, _, n, e in s_curve:
        by_flush[n] = max(by_flush.get(n, 0.0), e)
    ns = sorted(by_flush)
    say(f"drift {variant}: {iters} iterations, flush numbers 1..{ns[-1] if ns else 0}")
    for n in ns:
        say(f"drift {variant} flush {n:4d}: max_rel(S) = {by_flush[n]:.3e}")
    for i, e in o_curve:
        say(f"drift {variant} iteration {i:5d}: max_rel(o) = {e:.3e}")
    # the curve in compact form for the session report: the worst checkpoint
    # error per 20 flush numbers, and the worst output error per 512 iterations
    buckets = []
    for lo in range(1, (ns[-1] if ns else 0) + 1, 20):
        vals = [by_flush[n] for n in ns if lo <= n < lo + 20]
        if vals:
            buckets.append(f"{lo}-{min(lo + 19, ns[-1])}: {max(vals):.1e}")
    helpers.report(f"drift {variant} (T=8, L=128, {iters} iterations) max_rel(S) by flush "
                   f"number: " + ", ".join(buckets))
    ob = []
    for lo in range(0, iters, 512):
        vals = [e for i, e in o_curve if lo <= i < lo + 512]
        if vals:
            ob.append(f"{lo}-{min(lo + 511, iters - 1)}: {max(vals):.1e}")
    helpers.report(f"drift {variant} max_rel(o) by iteration: " + ", ".join(ob))
    assert len(ns) >= (4 if iters >= 256 else 1)


# ------------------------------------------------------------ 48-layer chain

GLUE_EPS = 1e-6


def _glue_width(sh) -> int:
    return 2 * sh.H * sh.K + sh.HV * sh.V + 2 * sh.HV


def _split_dev(y: torch.Tensor, sh):
    """Cut a [tokens, glue width] tensor into contiguous q, k, v, a, b."""
    n = y.shape[0]
    hk, vv = sh.H * sh.K, sh.HV * sh.V
    q = y[:, :hk].reshape(n, sh.H, sh.K).contiguous()
    k = y[:, hk:2 * hk].reshape(n, sh.H, sh.K).contiguous()
    v = y[:, 2 * hk:2 * hk + vv].reshape(n, sh.HV, sh.V).contiguous()
    a = y[:, 2 * hk + vv:2 * hk + vv + sh.HV].contiguous()
    b = y[:, 2 * hk + vv + sh.HV:].contiguous()
    return q, k, v, a, b


def _split_host(y: np.ndarray, sh):
    n = y.shape[0]
    hk, vv = sh.H * sh.K, sh.HV * sh.V
    return (y[:, :hk].reshape(n, sh.H, sh.K), y[:, hk:2 * hk].reshape(n, sh.H, sh.K),
            y[:, 2 * hk:2 * hk + vv].reshape(n, sh.HV, sh.V), y[:, 2 * hk + vv:2 * hk + vv + sh.HV],
            y[:, 2 * hk + vv + sh.HV:])


def _bf16_round_f64(x: np.ndarray) -> np.ndarray:
    """Store float64 values as bf16 (via fp32, nearest even) and widen back."""
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x.astype(np.float32))).astype(np.float64)


def _rmsnorm_f64(o: np.ndarray) -> np.ndarray:
    return o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + GLUE_EPS)


def _chain_layers() -> int:
    return int(os.environ.get("GDN_CHAIN_LAYERS", "48"))


def test_layer_chain_48_layers():
    require_gpu()
    sh = synth.CONFIGS["layer_chain_b128"]
    NL = _chain_layers()
    steps = 4
    seed = 1004
    gs = gv.GdnShape.from_layer(sh)
    dw = synth.DeviceWindows(seed, sh)
    rng = synth.make_rng(seed)
    n_o = 4
    orows = np.sort(rng.choice(sh.B, n_o, replace=False))
    slots = synth.slot_choice(rng, sh)
    cd = synth.random_cursors(rng, sh)
    wp0, base0 = cd.write_pos.copy(), cd.cache_base.copy()
    gslots = slots[orows]
    W = _glue_width(sh)
    HVV = sh.HV * sh.V
    say(f"chain: {NL} layers, B={sh.B}, oracle rows {orows.tolist()}")

    # per-layer parameters and state, drawn on the device from the seeded generator
    gen = dw.gen
    A_log = torch.log(torch.rand((NL, sh.HV), generator=gen, device=DEV) * 15.0 + 1.0)
    dt_bias = torch.randn((NL, sh.HV), generator=gen, device=DEV) * 0.1
    S = torch.empty((NL, sh.num_slots, sh.HV, sh.V, sh.K), dtype=torch.float32, device=DEV)
    for l in range(NL):
        S[l].normal_(0.0, 0.02, generator=gen)
    rawk = torch.zeros((NL, sh.num_slots, sh.H, sh.L, sh.K), dtype=torch.bfloat16, device=DEV)
    rawv = torch.zeros((NL, sh.num_slots, sh.HV, sh.L, sh.V), dtype=torch.bfloat16, device=DEV)
    rg = torch.zeros((NL, sh.num_slots, sh.HV, sh.L), dtype=torch.float32, device=DEV)
    rb = torch.zeros_like(rg)
    Wt = torch.empty((NL, HVV, W), dtype=torch.bfloat16, device=DEV)
    for l in range(NL):
        Wt[l] = (torch.randn((HVV, W), generator=gen, device=DEV) / np.sqrt(HVV)).to(torch.bfloat16)
    torch.cuda.synchronize()

    # oracle layers for the followed rows (slots renumbered 0..n_o-1)
    osh = sh.replace(B=n_o, num_slots=n_o)
    oslots = np.arange(n_o, dtype=np.int32)
    A_h, dt_h = A_log.cpu().numpy(), dt_bias.cpu().numpy()
    gsl_t = torch.from_numpy(gslots.astype(np.int64)).to(DEV)
    orcs = [oracle.OracleLayer(osh, A_h[l], dt_h[l], host_f64(S[l].index_select(0, gsl_t)))
            for l in range(NL)]
    W_h = [synth.bf16_bits_to_f32(Wt[l].cpu().view(torch.int16).numpy().view(np.uint16))
           .astype(np.float64) for l in range(NL)]

    # pre-fill every layer's ring with committed records (one token per call)
    nrec = int(wp0[slots].max())
    plan = helpers.prefill_plan(slots, wp0, nrec)
    gs1 = gs.replace(T=1)
    scratch = torch.empty((sh.B, sh.HV, sh.V), dtype=torch.bfloat16, device=DEV)
    zeros = dev_i32(np.zeros(sh.num_slots))
    base_d = dev_i32(base0)
    dw1 = synth.DeviceWindows(seed + 1, sh.replace(T=1))
    cur_o = CursorState(np.zeros(n_o, np.int32), base0[gslots].copy(), np.zeros(n_o, np.int32))
    for r in range(nrec):
        sl = dev_i32(plan[r])
        osl = np.where(plan[r][orows] >= 0, oslots, -1).astype(np.int32)
        cur_o.write_pos[:] = r
        wp_r = dev_i32(np.full(sh.num_slots, r))
        for l in range(NL):
            w = dw1.draw()
            gv.gdn_spec_verify_ring(gs1, w["q"], w["k"], w["v"], w["a"], w["b"], A_log[l],
                                    dt_bias[l], S[l], sl, wp_r, base_d, zeros, rawk[l], rawv[l],
                                    rg[l], rb[l], 1, 0, scratch)
            wo = helpers.win_f64(dw1.host_rows(w, orows, 1), sh.act)
            orcs[l].write_ring(cur_o, osl, wo, T=1)
    torch.cuda.synchronize()
    say(f"chain: rings pre-filled with up to {nrec} records")

    cur = CursorState(wp0.copy(), base0.copy(), (wp0 + 2 * sh.max_spec > sh.L).astype(np.int32))
    ocur = CursorState(wp0[gslots].copy(), base0[gslots].copy(), cur.is_flush[gslots].copy())
    dcur = dev_cursors(cur)
    dslots = dev_i32(slots)
    accepts = synth.accept_counts(rng, sh.B, sh.T, steps)
    tol = TOL[sh.act]
    o = torch.empty((sh.B * sh.T, sh.HV, sh.V), dtype=torch.bfloat16, device=DEV)
    tok_idx = (orows[:, None] * sh.T + np.arange(sh.T)[None, :]).reshape(-1)
    tok_t = torch.from_numpy(tok_idx.astype(np.int64)).to(DEV)
    worst = np.zeros(NL)
    glue_gap = np.zeros(NL)

    def glue(o_l, l):
        xf = o_l.float().reshape(sh.B * sh.T, HVV)
        xf = xf * torch.rsqrt(xf.pow(2).mean(dim=-1, keepdim=True) + GLUE_EPS)
        return (xf @ Wt[l].float()).to(torch.bfloat16)
    for step_i in range(steps):
        x0 = dw.normal((sh.B * sh.T, W))                       # layer-0 inputs, bf16
        y_h = synth.bf16_bits_to_f32(x0.index_select(0, tok_t).cpu().view(torch.int16).numpy()
                                     .view(np.uint16)).astype(np.float64)
        y = x0
        gv.gdn_exact_fold(gs, NL, 0, 0, S, rawk, rawv, rg, rb, dslots, *dcur, 1)
        for l in range(NL):
            q, k, v, a, b = _split_dev(y, sh)
            gv.gdn_spec_verify_ring(gs, q, k, v, a, b, A_log[l], dt_bias[l], S[l], dslots,
                                    *dcur, rawk[l], rawv[l], rg[l], rb[l], 1, 0, o)
            # oracle layer l on its own inputs
            ref = orcs[l].verify(ocur, oslots, _split_host(y_h, sh))
            err = helpers.max_rel(host_f64(o.index_select(0, tok_t)), ref)
            worst[l] = max(worst[l], err)
            # glue to the next layer: the GPU from its outputs, the oracle from its own
            y = glue(o, l)
            o_h = _bf16_round_f64(ref).reshape(n_o * sh.T, HVV)
            y_h = _bf16_round_f64(_rmsnorm_f64(o_h) @ W_h[l])
            # the rows the oracle follows continue from the oracle's inputs on
            # both sides (free-running chains drift apart through rounding)
            y_own = host_f64(y.index_select(0, tok_t))
            glue_gap[l] = max(glue_gap[l], helpers.max_rel(y_own, y_h))
            forced = synth.f32_to_bf16_bits(y_h.astype(np.float32)).view(np.int16)
            y.index_copy_(0, tok_t, torch.from_numpy(forced).view(torch.bfloat16).to(DEV))
        acc = accepts[step_i]
        gv.gdn_advance_cursors(gs, dslots, dev_i32(acc), *dcur)
        advance(cur, slots, acc, sh.L, sh.T, sh.max_spec)
        advance(ocur, oslots, acc[orows], sh.L, sh.T, sh.max_spec)
        _cursors_equal(dcur, cur, step_i)
        say(f"chain step {step_i}: worst layer max_rel(o) so far {worst.max():.2e} "
            f"(layer {int(worst.argmax())}), worst input gap {glue_gap.max():.2e}")
    for l in range(NL):
        say(f"chain layer {l:2d}: max_rel(o) over {steps} steps = {worst[l]:.3e}; "
            f"own next-layer inputs vs the oracle's {glue_gap[l]:.3e}")
    assert worst.max() <= tol, (int(worst.argmax()), worst.max())
    # fold every layer's committed records in one launch and compare checkpoints
    fl_all = dev_i32(np.ones(sh.num_slots))
    gv.gdn_exact_fold(gs, NL, 0, 0, S, rawk, rawv, rg, rb, dslots, dcur[0], dcur[1], fl_all, 1)
    ocur_f = CursorState(ocur.write_pos.copy(), ocur.cache_base.copy(), np.ones(n_o, np.int32))
    for l in range(NL):
        orcs[l].fold(ocur_f, oslots, only_flagged=True)
        serr = helpers.max_rel(host_f64(S[l].index_select(0, gsl_t)), orcs[l].S)
        assert serr <= tol, (l, serr)
    # latency of one whole-stack verify step, GPU only: the fold over all layers
    # plus the per-layer verifies, and the glue separately (not part of the path)
    x0 = dw.normal((sh.B * sh.T, W))
    for rep in range(2):
        ev_g = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(NL + 1)]
        ev_x = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(NL)]
        y = x0
        ev_g[NL][0].record()
        gv.gdn_exact_fold(gs, NL, 0, 0, S, rawk, rawv, rg, rb, dslots, *dcur, 1)
        ev_g[NL][1].record()
        for l in range(NL):
            ev_x[l][0].record()
            q, k, v, a, b = _split_dev(y, sh)
            ev_x[l][1].record()
            ev_g[l][0].record()
            gv.gdn_spec_verify_ring(gs, q, k, v, a, b, A_log[l], dt_bias[l], S[l], dslots,
                                    *dcur, rawk[l], rawv[l], rg[l], rb[l], 1, 0, o)
            ev_g[l][1].record()
            y = glue(o, l)
        torch.cuda.synchronize()
    gdn_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev_g)
    glue_ms = sum(ev_g[l][1].elapsed_time(ev_x[l + 1][0]) if l + 1 < NL else 0.0
                  for l in range(NL))
    helpers.report(f"chain latency: {NL}-layer GDN {gdn_ms:.3f} ms per verify step (all-layer "
                   f"fold {ev_g[NL][0].elapsed_time(ev_g[NL][1]) * 1e3:.1f} us), glue "
                   f"{glue_ms:.3f} ms; worst layer max_rel(o) {worst.max():.2e}")
    ring_stack = NL * gv.gdn_ring_bytes(gs)
    snap_stack = NL * gv.gdn_snapshot_bytes(gs)
    helpers.report(f"chain memory: ring {ring_stack / 1e9:.2f} GB vs snapshot "
                   f"{snap_stack / 1e9:.2f} GB for {NL} layers (checkpoints "
                   f"{S.numel() * 4 / 1e9:.2f} GB in both)")
