"""GPU parity of the per-channel-gate (KDA) layer: the HIP path through the C
ABI against the fp64 KDA oracle.

The KDA ring keeps K fp32 gate values per record (PR #36821 summary: g
[slots, HV, L, K], the per-K KDA gate).  The kernel replays the committed
records from the frozen checkpoint in fp32 and steps through the window, so
the only roundings are fp32 arithmetic and, for bf16 activations, the final
rounding of each output.  Bars (written in each test):
  - raw ring records and cursors bit-exact; ring g/beta within 5e-5 absolute;
  - states: max|x-ref|/max|ref| <= 1e-4 (fp32 on both sides, whatever the
    activation dtype);
  - outputs: <= 1e-4 (fp32) and <= 5e-3 (bf16: one rounding to bf16 is at
    most 2^-8 of the value, plus the fp32 error);
  - the fold a verify stores and the exact fold are bitwise equal (same
    records, same arithmetic).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle.cursors import CursorState, advance, clamp_write_pos, phys
from linear_attention_speculative_spec_amd import gdnverify as gv
from linear_attention_speculative_spec_amd import synth

import helpers
from gpu_harness import DEV, DevWindow, KdaPair, dev_i32, host_bits, host_cursors, host_f64

pytestmark = pytest.mark.gpu

TOL_O = {synth.ACT_F32: 1e-4, synth.ACT_BF16: 5e-3}
TOL_S = 1e-4
GB_TOL = 5e-5


def say(*a):
    print(*a, flush=True)


class KdaRingTracker:
    """Expected ring bits: the garbage template plus every record written."""

    def __init__(self, template, shape):
        self.shape = shape
        self.bits = (lambda x: x.view(np.uint16)) if shape.act == synth.ACT_BF16 else \
            (lambda x: x.view(np.uint32))
        self.rawk = self.bits(template["rawk"]).copy()
        self.rawv = self.bits(template["rawv"]).copy()
        self.g_tmpl = template["g"].view(np.uint32).copy()
        self.b_tmpl = template["beta"].view(np.uint32).copy()
        self.written = np.zeros(template["beta"].shape, dtype=bool)     # [slots, HV, L]

    def record(self, slots, cur: CursorState, win: synth.Window, T: int):
        sh = self.shape
        for row, s in enumerate(np.asarray(slots).tolist()):
            if not (0 <= s < sh.num_slots):
                continue
            wpc = clamp_write_pos(cur.write_pos[s], sh.L, T)
            for t in range(T):
                p = phys(cur.cache_base[s], wpc + t, sh.L)
                tok = row * T + t
                self.rawk[s, :, p, :] = self.bits(win.k[tok])
                self.rawv[s, :, p, :] = self.bits(win.v[tok])
                self.written[s, :, p] = True

    def check(self, gpu, orc=None, gslots=None):
        assert np.array_equal(host_bits(gpu.rawk), self.rawk), "rawk ring bits"
        assert np.array_equal(host_bits(gpu.rawv), self.rawv), "rawv ring bits"
        g_bits, b_bits = host_bits(gpu.g), host_bits(gpu.beta)
        un = ~self.written
        assert np.array_equal(g_bits[un], self.g_tmpl[un]), "g written outside the windows"
        assert np.array_equal(b_bits[un], self.b_tmpl[un]), "beta written outside the windows"
        if orc is not None:
            w = self.written[gslots]
            g = g_bits.view(np.float32)[gslots].astype(np.float64)
            b = b_bits.view(np.float32)[gslots].astype(np.float64)
            assert np.max(np.abs(g[w] - orc.g[w]), initial=0) < GB_TOL
            assert np.max(np.abs(b[w] - orc.beta[w]), initial=0) < GB_TOL


def prefill_tracker(P: KdaPair) -> KdaRingTracker:
    tr = KdaRingTracker(P.template, P.shape)
    cur = CursorState(np.zeros_like(P.wp0), P.base0.copy(), np.zeros_like(P.wp0))
    for r, (sl, w) in enumerate(zip(helpers.prefill_plan(P.slots, P.wp0, len(P.hist)), P.hist)):
        cur.write_pos[:] = r
        tr.record(sl, cur, w, 1)
    return tr


def run_kda_lifecycle(shape, seed, steps, variant="base", wp_by_slot=None, oracle_rows=None,
                      check_ring=True):
    P = KdaPair(shape, seed, variant, wp_by_slot=wp_by_slot, oracle_rows=oracle_rows)
    tol = TOL_O[shape.act]
    tr = prefill_tracker(P) if check_ring else None
    accepts = synth.accept_counts(P.rng, shape.B, shape.T, steps)
    worst_o = worst_e = worst_s = 0.0
    flushes = 0
    for i in range(steps):
        win = P.window()
        o = P.gpu.new_out()
        flushes += int(P.cur.is_flush[P.slots].sum())
        P.gpu.verify(P.dcur, P.dslots, DevWindow(win, shape.act), o)
        ref = P.oracle_verify(win)
        if tr is not None:
            tr.record(P.slots, P.cur, win, shape.T)
        got = P.gpu_out_rows(o)
        err = helpers.max_rel(got, ref)
        worst_o = max(worst_o, err)
        worst_e = max(worst_e, helpers.elem_rel(got, ref))
        assert err <= tol, (i, err)
        acc = accepts[i]
        gv.gdn_advance_cursors(P.gpu.gs, P.dslots, dev_i32(acc), *P.dcur)
        advance(P.cur, P.slots, acc, shape.L, shape.T, shape.max_spec)
        advance(P.ocur, P.oslots, acc[P.orows], shape.L, shape.T, shape.max_spec)
        hc = host_cursors(P.dcur)
        for name in ("write_pos", "cache_base", "is_flush"):
            assert np.array_equal(getattr(hc, name), getattr(P.cur, name)), (name, i)
        serr = helpers.max_rel(host_f64(P.gpu.S)[P.gslots], P.orc.S)
        worst_s = max(worst_s, serr)
        assert serr <= TOL_S, (i, serr)
    if tr is not None:
        tr.check(P.gpu, P.orc, P.gslots)
    helpers.report(f"kda lifecycle {shape.act} B={shape.B} T={shape.T} K={shape.K} V={shape.V} "
                   f"L={shape.L} {variant}: steps={steps} flushes={flushes} "
                   f"max_rel(o)={worst_o:.2e} elem_rel(o)={worst_e:.2e} max_rel(S)={worst_s:.2e}")
    return P, flushes


@pytest.mark.parametrize("variant", ["base", "low_decay", "beta_high"])
def test_kda_tiny_f32_lifecycle_40_steps(variant):
    shape = synth.CONFIGS["tiny_f32"].replace(B=2, num_slots=4)
    wp = np.full(shape.num_slots, 5, np.int32)
    _, flushes = run_kda_lifecycle(shape, 3000, 40, variant, wp_by_slot=wp)
    assert flushes >= 2


@pytest.mark.parametrize("variant", ["base", "low_decay"])
def test_kda_qwen_shaped_b32_lifecycle(variant):
    shape = synth.CONFIGS["qwen3next_b32"]
    run_kda_lifecycle(shape, 3001, 20, variant, oracle_rows=np.arange(0, 32, 3))


def test_kda_single_token_decode_lifecycle():
    # T = 1 windows (plain decode through the ring), several flushes
    shape = synth.CONFIGS["tiny_f32"].replace(B=3, num_slots=5, T=1, max_spec=1, L=8,
                                              act=synth.ACT_BF16)
    _, flushes = run_kda_lifecycle(shape, 3002, 30, "low_decay")
    assert flushes >= 3


KDA_SWEEP = [
    dict(K=64, V=64, H=2, HV=4, T=2, L=16, max_spec=2, act=synth.ACT_F32),
    dict(K=128, V=192, H=4, HV=8, T=3, L=32, max_spec=4, act=synth.ACT_BF16),
    dict(K=256, V=256, H=2, HV=2, T=16, L=64, max_spec=16, act=synth.ACT_BF16),
    dict(K=256, V=64, H=1, HV=4, T=1, L=8, max_spec=1, act=synth.ACT_F32),
    dict(K=64, V=128, H=4, HV=4, T=8, L=128, max_spec=8, act=synth.ACT_BF16),
    dict(K=128, V=64, H=1, HV=1, T=4, L=64, max_spec=4, act=synth.ACT_F32),
]


@pytest.mark.parametrize("kw", KDA_SWEEP, ids=lambda kw: "K{K}V{V}T{T}L{L}{act}".format(**kw))
def test_kda_shape_sweep_three_step_lifecycle(kw):
    shape = synth.LayerShape(B=3, num_slots=5, **kw)
    say("kda sweep", kw)
    run_kda_lifecycle(shape, 3100 + kw["K"] + kw["V"] + kw["T"], 3)


def test_kda_ring_write_is_a_bitwise_side_channel():
    shape = synth.CONFIGS["qwen3next_b32"]
    P = KdaPair(shape, 3200, oracle_rows=[0])
    win = DevWindow(P.window(), shape.act)
    S0 = P.gpu.S.clone()
    outs = []
    for wr in (0, 1, 0):
        P.gpu.S.copy_(S0)
        o = P.gpu.new_out()
        P.gpu.verify(P.dcur, P.dslots, win, o, write_ring=wr, fold_flagged=1)
        outs.append(host_bits(o))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


def test_kda_padding_rows_read_and_write_nothing():
    shape = synth.CONFIGS["qwen3next_b32"]
    P = KdaPair(shape, 3300, oracle_rows=[0])
    slots = P.slots.copy()
    slots[[1, 9, 30]] = [-1, shape.num_slots, -7]
    tr = prefill_tracker(P)
    S_before = host_bits(P.gpu.S)
    win = P.window()
    o = P.gpu.new_out()
    sentinel = host_bits(o)
    P.gpu.verify(P.dcur, dev_i32(slots), DevWindow(win, shape.act), o)
    tr.record(slots, P.cur, win, shape.T)
    tr.check(P.gpu)
    got = host_bits(o)
    for r in (1, 9, 30):
        rows = slice(r * shape.T, (r + 1) * shape.T)
        assert np.array_equal(got[rows], sentinel[rows])
        assert np.array_equal(host_bits(P.gpu.S)[P.slots[r]], S_before[P.slots[r]])
    assert not np.isnan(host_f64(o)[0: shape.T]).any()


def test_kda_verify_fold_equals_exact_fold_bitwise_and_oracle():
    """A flagged row's checkpoint: the state a fold_flagged verify stores, the
    exact fold's, and the oracle fold's."""
    shape = synth.CONFIGS["qwen3next_b32"]
    wp = np.random.default_rng(0).integers(0, shape.L - shape.T + 1, shape.num_slots).astype(np.int32)
    wp[:8] = shape.L - shape.T                   # some rows at the end of the ring
    P = KdaPair(shape, 3400, wp_by_slot=wp, oracle_rows=np.arange(0, 32, 4))
    flag = (np.arange(shape.num_slots) % 2).astype(np.int32)     # half the slots flagged
    dcur = (P.dcur[0], P.dcur[1], dev_i32(flag))
    S0 = P.gpu.S.clone()
    win = DevWindow(P.window(), shape.act)
    o = P.gpu.new_out()
    P.gpu.verify(dcur, P.dslots, win, o, write_ring=0, fold_flagged=1)
    S_verify = host_bits(P.gpu.S)
    P.gpu.S.copy_(S0)
    P.gpu.fold(dcur, P.dslots, only_flagged=1)
    S_fold = host_bits(P.gpu.S)
    assert np.array_equal(S_verify, S_fold)
    S0h = host_bits(S0)
    for s in range(shape.num_slots):
        if not (flag[s] and s in set(P.slots.tolist())):
            assert np.array_equal(S_fold[s], S0h[s]), s
    ocur = CursorState(P.ocur.write_pos.copy(), P.ocur.cache_base.copy(), flag[P.gslots].copy())
    P.orc.fold(ocur, P.oslots, only_flagged=True)
    err = helpers.max_rel(host_f64(P.gpu.S)[P.gslots], P.orc.S)
    helpers.report(f"kda fold B=32 flagged half: max_rel(S)={err:.2e}")
    assert err <= TOL_S


def test_kda_exact_fold_layers_at_strides():
    # two layers of one pool laid out [layer][slot][...] with gaps between the
    # layers' checkpoints and rings; the cursors and slots are shared by the
    # layers, each layer folds against its own oracle
    sh = synth.CONFIGS["qwen3next_b32"].replace(B=8, num_slots=12)
    rng = synth.make_rng(3499)
    slots = synth.slot_choice(rng, sh)
    cd = synth.random_cursors(rng, sh)
    layers = [KdaPair(sh, 3500 + l, wp_by_slot=cd.write_pos, base_by_slot=cd.cache_base,
                      slots=slots) for l in range(2)]
    gap_S, gap_R = 4 * 1024, 3
    per_S = sh.num_slots * sh.HV * sh.V * sh.K
    lsS, lsR = per_S + gap_S, sh.num_slots + gap_R
    S = torch.full((2 * lsS,), -1234.5, dtype=torch.float32, device=DEV)

    def ring_pool(name, per_slot):
        src0 = getattr(layers[0].gpu, name)
        t = torch.full((2 * lsR * per_slot,), float("nan"), dtype=src0.dtype, device=DEV)
        for l, P in enumerate(layers):
            src = getattr(P.gpu, name).reshape(-1)
            t[l * lsR * per_slot: l * lsR * per_slot + src.numel()].copy_(src)
        return t

    rk = ring_pool("rawk", sh.H * sh.L * sh.K)
    rv = ring_pool("rawv", sh.HV * sh.L * sh.V)
    rg = ring_pool("g", sh.HV * sh.L * sh.K)
    rb = ring_pool("beta", sh.HV * sh.L)
    for l, P in enumerate(layers):
        S[l * lsS: l * lsS + per_S].copy_(P.gpu.S.reshape(-1))
    P0 = layers[0]
    gv.gdn_kda_exact_fold(P0.gpu.gs, 2, lsS, lsR, S, rk, rv, rg, rb, P0.dslots, P0.dcur[0],
                          P0.dcur[1], None, 0)
    Sh = host_f64(S)
    for l, P in enumerate(layers):
        P.orc.fold(P.ocur, P.oslots, only_flagged=False)
        Sl = Sh[l * lsS: l * lsS + per_S].reshape(sh.num_slots, sh.HV, sh.V, sh.K)
        err = helpers.max_rel(Sl[P.gslots], P.orc.S)
        assert err <= TOL_S, (l, err)
        untouched = np.setdiff1d(np.arange(sh.num_slots), P.slots)
        assert np.array_equal(Sl[untouched], P.params.S0[untouched].astype(np.float64))
        gap = Sh[l * lsS + per_S: (l + 1) * lsS]
        assert np.all(gap == -1234.5), l


def test_kda_full_batch_b256_all_rows():
    """The B=256 Qwen3-Next-shaped layer: one verify of every row against the
    oracle (outputs, the checkpoints of flagged rows, the whole ring)."""
    shape = synth.CONFIGS["qwen3next_b256"]
    say("kda b256: building the pair")
    P = KdaPair(shape, 3600)
    tr = prefill_tracker(P)
    win = P.window()
    o = P.gpu.new_out()
    S_before = host_bits(P.gpu.S)
    say("kda b256: verify")
    P.gpu.verify(P.dcur, P.dslots, DevWindow(win, shape.act), o)
    torch.cuda.synchronize()
    ref = P.oracle_verify(win)
    got = P.gpu_out_rows(o)
    err, eerr = helpers.max_rel(got, ref), helpers.elem_rel(got, ref)
    serr = helpers.max_rel(host_f64(P.gpu.S)[P.gslots], P.orc.S)
    nflag = int(P.cur.is_flush[P.slots].sum())
    helpers.report(f"kda b256 all rows: max_rel(o)={err:.2e} elem_rel(o)={eerr:.2e} "
                   f"max_rel(S)={serr:.2e} flagged={nflag}")
    assert err <= TOL_O[shape.act]
    assert serr <= TOL_S
    assert nflag > 0
    tr.record(P.slots, P.cur, win, shape.T)
    tr.check(P.gpu, P.orc, P.gslots)
    S_after = host_bits(P.gpu.S)
    flagged = set(P.slots[P.cur.is_flush[P.slots] != 0].tolist())
    for s in range(shape.num_slots):
        if s not in flagged:
            assert np.array_equal(S_after[s], S_before[s]), s
