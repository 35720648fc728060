"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bars (written in each test): cursors and raw ring records bit-exact; ring
g/beta within 5e-5 of the oracle and bitwise equal between the two GPU
producers; outputs and folded states within max|x-ref|/max|ref| of 2e-3
(fp32 activations) or 3e-2 (bf16 activations).
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

from oracle.cursors import CursorState, advance, clamp_write_pos, phys, reset
from linear_attention_speculative_spec_amd import gdnverify as gv
from linear_attention_speculative_spec_amd import synth

import helpers
from gpu_harness import (DevWindow, Pair, dev_cursors, dev_i32, host_bits, host_cursors,
                         host_f64, require_gpu)

pytestmark = pytest.mark.gpu

TOL = {synth.ACT_F32: 2e-3, synth.ACT_BF16: 3e-2}
GB_TOL = 5e-5
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------ ring tracking

class RingTracker:
    """Expected raw ring bits: the garbage template with every record written so far."""

    def __init__(self, template, shape):
        self.shape = shape
        bits = (lambda x: x.view(np.uint16)) if shape.act == synth.ACT_BF16 else \
            (lambda x: x.view(np.uint32))
        self.bits = bits
        self.rawk = bits(template["rawk"]).copy()
        self.rawv = bits(template["rawv"]).copy()
        self.g_tmpl = template["g"].view(np.uint32).copy()
        self.b_tmpl = template["beta"].view(np.uint32).copy()
        self.written = np.zeros(template["g"].shape, dtype=bool)

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

    def check(self, gpu, oracle_layer=None, gslots=None):
        assert np.array_equal(host_bits(gpu.rawk), self.rawk), "rawk ring bits"
        assert np.array_equal(host_bits(gpu.rawv), self.rawv), "rawv ring bits"
        g_bits, b_bits = host_bits(gpu.g), host_bits(gpu.beta)
        un = ~self.written
        assert np.array_equal(g_bits[un], self.g_tmpl[un]), "g written outside the windows"
        assert np.array_equal(b_bits[un], self.b_tmpl[un]), "beta written outside the windows"
        if oracle_layer is not None:
            g = g_bits.view(np.float32)[gslots].astype(np.float64)
            b = b_bits.view(np.float32)[gslots].astype(np.float64)
            w = self.written[gslots]
            assert np.max(np.abs(g[w] - oracle_layer.g[w]), initial=0) < GB_TOL
            assert np.max(np.abs(b[w] - oracle_layer.beta[w]), initial=0) < GB_TOL


def prefill_tracker(P: Pair) -> RingTracker:
    tr = RingTracker(P.template, P.shape)
    cur = CursorState(np.zeros_like(P.wp0), P.base0.copy(), np.zeros_like(P.wp0))
    for r, (sl, w) in enumerate(zip(helpers.prefill_plan(P.slots, P.wp0, len(P.hist)), P.hist)):
        cur.write_pos[:] = r
        tr.record(sl, cur, w, 1)
    return tr


# ------------------------------------------------------------------ cursors

def _cursor_shape(B, T, L, M, num_slots):
    return gv.GdnShape(B=B, T=T, H=1, HV=1, K=64, V=16, L=L, max_spec_len=M,
                       num_slots=num_slots, act=gv.GDN_BF16, scale=1.0,
                       softplus_threshold=20.0, l2norm_eps=1e-6)


@pytest.mark.parametrize("L,T,M", [(16, 4, 4), (64, 4, 4), (128, 8, 8), (8, 2, 2), (64, 3, 4)])
def test_cursor_kernels_bit_exact(L, T, M):
    require_gpu()
    say("cursors", L, T, M)
    rng = synth.make_rng(500 + L + T)
    num_slots, B = 40, 32
    gs = _cursor_shape(B, T, L, M, num_slots)
    cur = CursorState.zeros(num_slots)
    cur.cache_base[:] = rng.integers(0, L, size=num_slots)
    cur.write_pos[:] = rng.integers(0, L - T + 1, size=num_slots)
    cur.is_flush[:] = (cur.write_pos + 2 * M > L).astype(np.int32)
    slots = rng.permutation(num_slots)[:B].astype(np.int32)
    slots[3], slots[17] = -1, num_slots + 5          # padding rows
    dcur = dev_cursors(cur)
    dslots = dev_i32(slots)
    for step in range(300):
        acc = rng.integers(-2, T + 3, size=B).astype(np.int32)   # clamped to [0, T]
        gv.gdn_advance_cursors(gs, dslots, dev_i32(acc), *dcur)
        advance(cur, slots, acc, L, T, M)
        if step % 37 == 36:
            rs = rng.choice(num_slots, size=5, replace=False).astype(np.int32)
            rs = np.concatenate([rs, np.array([-3, num_slots], np.int32)])
            init = int(step % 2)
            gv.gdn_reset_cursors(gs, dev_i32(rs), len(rs), init, *dcur)
            reset(cur, rs, init)
        got = host_cursors(dcur)
        for name in ("write_pos", "cache_base", "is_flush"):
            assert np.array_equal(getattr(got, name), getattr(cur, name)), (name, step)


def test_cursor_walks_printed_on_the_pages_on_gpu():
    require_gpu()
    with open(os.path.join(GOLDEN, "cursor_walks.json")) as f:
        gold = json.load(f)
    for w in gold["walks"]:
        gs = _cursor_shape(1, w["T"], w["L"], w["max_spec"], 1)
        dcur = (dev_i32([w["start"]["write_pos"]]), dev_i32([w["start"]["cache_base"]]),
                dev_i32([w["start"]["is_flush"]]))
        for st in w["steps"]:
            gv.gdn_advance_cursors(gs, dev_i32([0]), dev_i32([st["accept"]]), *dcur)
            got = host_cursors(dcur)
            assert {"write_pos": int(got.write_pos[0]), "cache_base": int(got.cache_base[0]),
                    "is_flush": int(got.is_flush[0])} == st["after"], w["cite"]


# ------------------------------------------------------------ lifecycles

def run_lifecycle(shape, seed, steps, variant="base", wp_by_slot=None, oracle_rows=None,
                  check_ring=True):
    P = Pair(shape, seed, variant, wp_by_slot=wp_by_slot, oracle_rows=oracle_rows)
    tol = TOL[shape.act]
    tr = prefill_tracker(P) if check_ring else None
    accepts = synth.accept_counts(P.rng, shape.B, shape.T, steps)
    gslots = P.slots[P.orows]
    worst_o = worst_s = 0.0
    flushes = 0
    for i in range(steps):
        win = P.window()
        o = P.gpu.new_out()
        flushes += int(P.cur.is_flush[P.slots].sum())
        P.gpu.verify(P.dcur, P.dslots, DevWindow(win, shape.act), o)
        ref = P.oracle_verify(win)
        if tr is not None:
            tr.record(P.slots, P.cur, win, shape.T)
        err = helpers.max_rel(P.gpu_out_rows(o), ref)
        worst_o = max(worst_o, err)
        assert err <= tol, (i, err)
        acc = accepts[i]
        gv.gdn_advance_cursors(P.gpu.gs, P.dslots, dev_i32(acc), *P.dcur)
        advance(P.cur, P.slots, acc, shape.L, shape.T, shape.max_spec)
        advance(P.ocur, P.oslots, acc[P.orows], shape.L, shape.T, shape.max_spec)
        got = host_cursors(P.dcur)
        for name in ("write_pos", "cache_base", "is_flush"):
            assert np.array_equal(getattr(got, name), getattr(P.cur, name)), (name, i)
        Sg = host_f64(P.gpu.S)[gslots]
        serr = helpers.max_rel(Sg, P.orc.S)
        worst_s = max(worst_s, serr)
        assert serr <= tol, (i, serr)
    if tr is not None:
        tr.check(P.gpu, P.orc, gslots)
    helpers.report(f"lifecycle {shape.act} B={shape.B} T={shape.T} K={shape.K} V={shape.V} L={shape.L} "
                   f"{variant}: steps={steps} flushes={flushes} max_rel(o)={worst_o:.2e} "
                   f"max_rel(S)={worst_s:.2e}")
    return P, flushes


@pytest.mark.parametrize("variant", ["base", "low_decay", "beta_high"])
def test_tiny_f32_lifecycle_40_steps(variant):
    shape = synth.CONFIGS["tiny_f32"]
    wp = np.full(shape.num_slots, 5, np.int32)          # 5 committed records
    _, flushes = run_lifecycle(shape, 1000, 40, variant, wp_by_slot=wp)
    assert flushes >= 2


@pytest.mark.parametrize("variant", ["base", "low_decay"])
def test_qwen3next_b32_lifecycle(variant):
    shape = synth.CONFIGS["qwen3next_b32"]
    run_lifecycle(shape, 1001, 24, variant, oracle_rows=np.arange(0, 32, 3))


def test_long_window_t8_lifecycle_reduced_batch():
    # the T=8, L=128 layer shape with 8 rows, long enough for several flushes
    shape = synth.CONFIGS["long_window_t8"].replace(B=8, num_slots=16)
    _, flushes = run_lifecycle(shape, 1003, 60, "low_decay")
    assert flushes >= 4


# --------------------------------------------------------- single verifies

@pytest.mark.parametrize("name,variant", [("qwen3next_b32", "base"), ("qwen3next_b32", "beta_high"),
                                          ("tiny_f32", "base")])
def test_verify_random_cursors_and_ring_contents(name, variant):
    shape = synth.CONFIGS[name]
    if name == "tiny_f32":
        shape = shape.replace(B=3, num_slots=4)
    P = Pair(shape, 2000, variant)
    tr = prefill_tracker(P)
    S_before = host_bits(P.gpu.S)
    win = P.window()
    o = P.gpu.new_out()
    P.gpu.verify(P.dcur, P.dslots, DevWindow(win, shape.act), o)
    ref = P.oracle_verify(win)
    tr.record(P.slots, P.cur, win, shape.T)
    err = helpers.max_rel(P.gpu_out_rows(o), ref)
    say(f"verify {name} {variant}: max_rel(o)={err:.2e} flagged={int(P.cur.is_flush[P.slots].sum())}")
    assert err <= TOL[shape.act]
    tr.check(P.gpu, P.orc, P.slots[P.orows])
    # the checkpoint changes only for flagged rows, and matches the exact fold
    S_after = host_bits(P.gpu.S)
    flagged = set(P.slots[P.cur.is_flush[P.slots] != 0].tolist())
    for s in range(shape.num_slots):
        if s not in flagged:
            assert np.array_equal(S_after[s], S_before[s]), s
    assert helpers.max_rel(host_f64(P.gpu.S)[P.slots], P.orc.S) <= TOL[shape.act]


def test_ring_write_is_a_bitwise_side_channel():
    shape = synth.CONFIGS["qwen3next_b32"]
    P = Pair(shape, 2100)
    win = DevWindow(P.window(), shape.act)
    S0 = P.gpu.S.clone()
    outs = []
    for wr in (0, 1, 0):
        P.gpu.S.copy_(S0)
        o = P.gpu.new_out()
        P.gpu.verify(P.dcur, P.dslots, win, o, write_ring=wr, fold_flagged=1)
        outs.append(host_bits(o))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


def test_padding_rows_read_and_write_nothing():
    shape = synth.CONFIGS["qwen3next_b32"]
    P = Pair(shape, 2200)
    slots = P.slots.copy()
    slots[[1, 9, 30]] = [-1, shape.num_slots, -7]
    tr = prefill_tracker(P)
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
    assert not np.isnan(host_f64(o)[0: shape.T]).any()


def test_cache_base_shift_gives_identical_outputs():
    shape = synth.CONFIGS["qwen3next_b32"]
    wp = np.full(shape.num_slots, 37, np.int32)
    outs = []
    for base in (np.zeros(shape.num_slots, np.int32),
                 np.full(shape.num_slots, shape.L - 5, np.int32)):
        P = Pair(shape, 2300, wp_by_slot=wp, base_by_slot=base, oracle_rows=[0])
        o = P.gpu.new_out()
        P.gpu.verify(P.dcur, P.dslots, DevWindow(P.window(), shape.act), o)
        outs.append(host_bits(o))
    assert np.array_equal(outs[0], outs[1])


# ------------------------------------------------ snapshot baseline and fold

SNAPSHOT_SHAPES = {
    "qwen3next_b32": synth.CONFIGS["qwen3next_b32"],
    "qwen3next_b256": synth.CONFIGS["qwen3next_b256"],
    # fp32 activations at the widest key: the snapshot kernel's largest LDS
    "f32_k256": synth.LayerShape(B=3, T=4, H=2, HV=4, K=256, V=32, L=64, max_spec=4,
                                 num_slots=5, act="f32"),
    "f32_k64_t8": synth.LayerShape(B=4, T=8, H=1, HV=2, K=64, V=48, L=32, max_spec=8,
                                   num_slots=6, act="f32"),
}


@pytest.mark.parametrize("name", list(SNAPSHOT_SHAPES))
def test_snapshot_matches_oracle_and_fold_reproduces_it_bitwise(name):
    # at B=256 every row is folded (rows spread over all waves of the fold's
    # row compaction); the oracle follows a sample of rows
    shape = SNAPSHOT_SHAPES[name]
    wp0 = np.zeros(shape.num_slots, np.int32)            # empty history everywhere
    orows = None if shape.B <= 32 else np.sort(synth.make_rng(2401).choice(shape.B, 8, replace=False))
    P = Pair(shape, 2400, wp_by_slot=wp0, oracle_rows=orows)
    g = P.gpu
    win = P.window()
    dwin = DevWindow(win, shape.act)
    gs = g.gs
    # producer 1: snapshot verify with the ring write
    snap = torch.empty((shape.B, shape.T, shape.HV, shape.V, shape.K), dtype=torch.float32,
                       device="cuda:0")
    o_snap = g.new_out()
    ring_snap = [t.clone() for t in g.ring()]
    gv.gdn_recurrent_verify_snapshot(gs, dwin.q, dwin.k, dwin.v, dwin.a, dwin.b, g.A_log,
                                     g.dt_bias, g.S, P.dslots, snap, o_snap, *ring_snap,
                                     P.dcur[0], P.dcur[1], write_ring=1)
    # producer 2: ring verify
    o = g.new_out()
    g.verify(P.dcur, P.dslots, dwin, o)
    for a_, b_ in zip(ring_snap, g.ring()):
        assert np.array_equal(host_bits(a_), host_bits(b_)), "two producers wrote different rings"
    # snapshot outputs and states against the oracle
    o_ref, snap_ref = P.orc.snapshot(P.oslots, helpers.win_f64(helpers.window_rows(win, P.orows, shape.T), shape.act))
    assert helpers.max_rel(P.gpu_out_rows(o_snap), o_ref) <= TOL[shape.act]
    sel = torch.from_numpy(np.asarray(P.orows, np.int64)).to("cuda:0")
    assert helpers.max_rel(host_f64(snap.index_select(0, sel)), snap_ref) <= TOL[shape.act]
    assert helpers.max_rel(P.gpu_out_rows(o), o_ref) <= TOL[shape.act]
    # fold the recorded window by accept count: bit-identical to snap[b, a-1]
    acc = P.rng.integers(0, shape.T + 1, size=shape.B).astype(np.int32)
    wp = np.zeros(shape.num_slots, np.int32)
    wp[P.slots] = acc
    fl = np.ones(shape.num_slots, np.int32)
    S_fold = g.S.clone()
    gv.gdn_exact_fold(gs, 1, 0, 0, S_fold, *g.ring(), P.dslots, dev_i32(wp), P.dcur[1], dev_i32(fl), 1)
    # and the snapshot path's own commit
    S_commit = g.S.clone()
    gv.gdn_snapshot_commit(gs, snap, P.dslots, dev_i32(acc), S_commit)
    Sf, Sc, S0, sn = host_bits(S_fold), host_bits(S_commit), host_bits(g.S), host_bits(snap)
    for row, s in enumerate(P.slots):
        a = int(acc[row])
        want = S0[s] if a == 0 else sn[row, a - 1]
        assert np.array_equal(Sf[s], want), (row, a)
        assert np.array_equal(Sc[s], want), (row, a)


def test_exact_fold_multi_layer_matches_oracle():
    # three layers with their own checkpoints and rings, one set of cursors
    shape = synth.CONFIGS["qwen3next_b32"].replace(B=8, num_slots=12)
    rng = synth.make_rng(2500)
    slots = rng.permutation(shape.num_slots)[: shape.B].astype(np.int32)
    wp = rng.integers(0, shape.L - shape.T + 1, size=shape.num_slots).astype(np.int32)
    base = rng.integers(0, shape.L, size=shape.num_slots).astype(np.int32)
    layers = [Pair(shape, 2501 + l, wp_by_slot=wp, base_by_slot=base, slots=slots)
              for l in range(3)]
    cat = lambda ts: torch.cat([t.reshape(-1) for t in ts])  # noqa: E731
    S = cat([P.gpu.S for P in layers])
    ring = [cat([P.gpu.ring()[i] for P in layers]) for i in range(4)]
    fl = np.ones(shape.num_slots, np.int32)
    P0 = layers[0]
    gv.gdn_exact_fold(P0.gpu.gs, 3, 0, 0, S, *ring, P0.dslots, dev_i32(wp), dev_i32(base),
                      dev_i32(fl), 1)
    Sh = host_f64(S).reshape(3, shape.num_slots, shape.HV, shape.V, shape.K)
    for l, P in enumerate(layers):
        ocur = CursorState(P.ocur.write_pos.copy(), P.ocur.cache_base.copy(),
                           np.ones(len(P.oslots), np.int32))
        P.orc.fold(ocur, P.oslots, only_flagged=True)
        err = helpers.max_rel(Sh[l][slots], P.orc.S)
        say(f"multi-layer fold layer {l}: max_rel(S)={err:.2e}")
        assert err <= TOL[shape.act]
        untouched = np.setdiff1d(np.arange(shape.num_slots), slots)
        assert np.array_equal(Sh[l][untouched], P.params.S0[untouched].astype(np.float64))


def test_exact_fold_layers_at_strides():
    # three layers of a pool laid out [layer][slot][...] with more slots per
    # layer than the shape uses: S placed layer_stride_S elements apart, the
    # ring arrays layer_stride_ring slots apart.  One launch folds all three;
    # each layer matches the oracle and nothing between the layers is written.
    shape = synth.CONFIGS["qwen3next_b32"].replace(B=8, num_slots=12)
    rng = synth.make_rng(2550)
    slots = rng.permutation(shape.num_slots)[: shape.B].astype(np.int32)
    wp = rng.integers(0, shape.L - shape.T + 1, size=shape.num_slots).astype(np.int32)
    base = rng.integers(0, shape.L, size=shape.num_slots).astype(np.int32)
    layers = [Pair(shape, 2551 + l, wp_by_slot=wp, base_by_slot=base, slots=slots)
              for l in range(3)]
    per_S = shape.num_slots * shape.HV * shape.V * shape.K
    ls_S = per_S + 4 * 777                      # 16-byte aligned gap after each layer
    ls_R = shape.num_slots + 5                  # five unused slots after each layer's ring
    S = torch.full((3 * ls_S,), -1234.5, dtype=torch.float32, device="cuda:0")
    g0 = layers[0].gpu
    per_slot = [t[0].numel() for t in g0.ring()]
    ring = [torch.zeros(3 * ls_R * n, dtype=t.dtype, device="cuda:0")
            for t, n in zip(g0.ring(), per_slot)]
    for l, P in enumerate(layers):
        S[l * ls_S: l * ls_S + per_S].copy_(P.gpu.S.reshape(-1))
        for buf, t, n in zip(ring, P.gpu.ring(), per_slot):
            buf[l * ls_R * n: l * ls_R * n + t.numel()].copy_(t.reshape(-1))
    fl = np.ones(shape.num_slots, np.int32)
    gv.gdn_exact_fold(g0.gs, 3, ls_S, ls_R, S, *ring, layers[0].dslots, dev_i32(wp),
                      dev_i32(base), dev_i32(fl), 1)
    Sh = host_f64(S)
    for l, P in enumerate(layers):
        ocur = CursorState(P.ocur.write_pos.copy(), P.ocur.cache_base.copy(),
                           np.ones(len(P.oslots), np.int32))
        P.orc.fold(ocur, P.oslots, only_flagged=True)
        Sl = Sh[l * ls_S: l * ls_S + per_S].reshape(shape.num_slots, shape.HV, shape.V, shape.K)
        err = helpers.max_rel(Sl[slots], P.orc.S)
        say(f"strided fold layer {l}: max_rel(S)={err:.2e}")
        assert err <= 1e-5
        untouched = np.setdiff1d(np.arange(shape.num_slots), slots)
        assert np.array_equal(Sl[untouched], P.params.S0[untouched].astype(np.float64))
        gap = Sh[l * ls_S + per_S: (l + 1) * ls_S]
        assert np.all(gap == -1234.5), l


# ------------------------------------------------------------ shape sweep

SWEEP = [
    dict(B=5, T=1, H=2, HV=4, K=64, V=16, L=8, max_spec=2, num_slots=9, act="bf16"),
    dict(B=4, T=2, H=2, HV=2, K=128, V=48, L=16, max_spec=2, num_slots=6, act="bf16"),
    dict(B=3, T=4, H=1, HV=4, K=256, V=32, L=32, max_spec=4, num_slots=4, act="bf16"),
    dict(B=3, T=3, H=2, HV=8, K=128, V=256, L=64, max_spec=4, num_slots=5, act="bf16"),
    dict(B=2, T=4, H=4, HV=8, K=128, V=128, L=64, max_spec=4, num_slots=3, act="f32"),
    dict(B=2, T=16, H=2, HV=4, K=64, V=64, L=128, max_spec=16, num_slots=3, act="bf16"),
    dict(B=6, T=5, H=3, HV=6, K=64, V=80, L=16, max_spec=8, num_slots=7, act="f32"),
    # fp32 activations with a 128-record ring (32-row value tiles, the
    # largest verify LDS) and at the widest key
    dict(B=3, T=8, H=2, HV=4, K=128, V=64, L=128, max_spec=8, num_slots=4, act="f32"),
    dict(B=2, T=4, H=2, HV=4, K=256, V=32, L=64, max_spec=4, num_slots=3, act="f32"),
]


@pytest.mark.parametrize("kw", SWEEP, ids=[f"K{d['K']}V{d['V']}T{d['T']}L{d['L']}{d['act']}" for d in SWEEP])
def test_shape_sweep_two_step_lifecycle(kw):
    shape = synth.LayerShape(**kw, scale=0.5)
    # include the empty and the full history, and flagged rows
    rng = synth.make_rng(3000 + kw["K"] + kw["V"])
    wp = rng.integers(0, shape.L - shape.T + 1, size=shape.num_slots).astype(np.int32)
    wp[:2] = [0, shape.L - shape.T]
    run_lifecycle(shape, 3000 + kw["L"], 6, "low_decay", wp_by_slot=wp)


def test_empty_batch_is_a_no_op():
    require_gpu()
    shape = synth.CONFIGS["qwen3next_b32"]
    gs = gv.GdnShape.from_layer(shape, B=0)
    z = torch.zeros(shape.num_slots, dtype=torch.int32, device="cuda:0")
    gv.gdn_advance_cursors(gs, z, z, z, z.clone(), z.clone())
    torch.cuda.synchronize()
    assert int(z.abs().sum()) == 0
