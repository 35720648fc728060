"""Device-side state for the GPU parity tests, mirrored by an oracle layer.

Both sides consume the same seeded inputs from ``synth``; the GPU side goes
through the C ABI binding only.  Ring pre-fill runs through the library's own
verify with a one-token window (write_ring on, no fold), i.e. the rings hold
exactly what verifies would have recorded; the oracle pre-fills its ring from
the same raw records with its own gating.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle.cursors import CursorState
from linear_attention_speculative_spec_amd import gdnverify as gv
from linear_attention_speculative_spec_amd import synth

import helpers

DEV = "cuda:0"


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X; none is visible")


def dev_act(x: np.ndarray, act: str) -> torch.Tensor:
    if act == synth.ACT_BF16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def dev_f32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def dev_i32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Exact bit pattern of a device tensor as an unsigned integer array."""
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.bfloat16, torch.float16, torch.int16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class DevWindow:
    def __init__(self, win: synth.Window, act: str):
        self.q, self.k, self.v, self.a, self.b = (dev_act(x, act) for x in
                                                  (win.q, win.k, win.v, win.a, win.b))


class GpuLayer:
    """One layer's device tensors: checkpoint, ring (from a garbage template)."""

    def __init__(self, shape: synth.LayerShape, params: synth.LayerParams, template: dict):
        self.shape = shape
        self.gs = gv.GdnShape.from_layer(shape)
        self.A_log = dev_f32(params.A_log)
        self.dt_bias = dev_f32(params.dt_bias)
        self.S = dev_f32(params.S0)
        self.rawk = dev_act(template["rawk"], shape.act)
        self.rawv = dev_act(template["rawv"], shape.act)
        self.g = dev_f32(template["g"])
        self.beta = dev_f32(template["beta"])

    def ring(self):
        return self.rawk, self.rawv, self.g, self.beta

    def verify_dcache(self, cur, slot_idx, win: DevWindow, o, write_ring=1, fold_flagged=1,
                      gs=None):
        gv.gdn_spec_verify_dcache(gs or self.gs, win.q, win.k, win.v, win.a, win.b, self.A_log,
                                  self.dt_bias, self.S, slot_idx, cur[0], cur[1], cur[2],
                                  self.rawk, self.rawv, self.g, self.beta, self.rd, write_ring,
                                  fold_flagged, o)

    def verify(self, cur, slot_idx, win: DevWindow, o, write_ring=1, fold_flagged=1, gs=None):
        gv.gdn_spec_verify_ring(gs or self.gs, win.q, win.k, win.v, win.a, win.b, self.A_log,
                                self.dt_bias, self.S, slot_idx, cur[0], cur[1], cur[2],
                                self.rawk, self.rawv, self.g, self.beta, write_ring,
                                fold_flagged, o)

    def new_out(self, B=None, T=None):
        sh = self.shape
        B = sh.B if B is None else B
        T = sh.T if T is None else T
        dt = torch.bfloat16 if sh.act == synth.ACT_BF16 else torch.float32
        return torch.full((B * T, sh.HV, sh.V), float("nan"), dtype=dt, device=DEV)


def dev_cursors(cur: CursorState):
    return (dev_i32(cur.write_pos), dev_i32(cur.cache_base), dev_i32(cur.is_flush))


def host_cursors(dc) -> CursorState:
    return CursorState(*(t.cpu().numpy().astype(np.int32) for t in dc))


class Pair:
    """A GPU layer and an oracle layer built from one seed, rings pre-filled."""

    def __init__(self, shape: synth.LayerShape, seed: int, variant: str = "base",
                 wp_by_slot=None, base_by_slot=None, slots=None, oracle_rows=None,
                 dcache=False):
        require_gpu()
        self.shape = shape
        self.act = shape.act
        rng = synth.make_rng(seed)
        self.rng = rng
        self.variant = variant
        self.params = synth.layer_params(rng, shape, variant)
        self.slots = synth.slot_choice(rng, shape) if slots is None else np.asarray(slots, np.int32)
        cd = synth.random_cursors(rng, shape)
        wp = cd.write_pos if wp_by_slot is None else np.asarray(wp_by_slot, np.int32)
        base = cd.cache_base if base_by_slot is None else np.asarray(base_by_slot, np.int32)
        self.template = synth.ring_garbage_template(rng, shape)
        self.gpu = GpuLayer(shape, self.params, self.template)
        self.dcache = dcache
        if dcache:
            # d ring of NaN payloads from a generator of its own (the main
            # stream stays as without it)
            drng = synth.make_rng(seed + 7919)
            n = shape.num_slots * shape.HV * shape.L * shape.V
            bits = (np.uint32(0x7FC00000) | drng.integers(1, 0x3FFFFF, size=n, dtype=np.uint32))
            self.d_template = bits.astype(np.uint32).reshape(shape.num_slots, shape.HV, shape.L, shape.V)
            self.gpu.rd = torch.from_numpy(self.d_template.view(np.float32).copy()).to(DEV)
        # oracle: only the rows asked for (all by default), slots renumbered
        self.orows = np.arange(shape.B) if oracle_rows is None else np.asarray(oracle_rows)
        osh = shape.replace(B=len(self.orows), num_slots=len(self.orows))
        self.oshape = osh
        self.oslots = np.arange(len(self.orows), dtype=np.int32)
        gslots = self.slots[self.orows]
        self.orc = oracle.OracleLayer(osh, self.params.A_log, self.params.dt_bias,
                                      self.params.S0[gslots])
        # pre-fill both rings with committed records
        nrec = int(wp[self.slots].max()) if len(self.slots) else 0
        hist = synth.history_windows(rng, shape, nrec, variant)
        gs1 = self.gpu.gs.replace(T=1)
        cur_g = CursorState(np.zeros(shape.num_slots, np.int32), base.copy(),
                            np.zeros(shape.num_slots, np.int32))
        cur_o = CursorState(np.zeros(osh.num_slots, np.int32), base[gslots].copy(),
                            np.zeros(osh.num_slots, np.int32))
        scratch = self.gpu.new_out(T=1)
        plan = helpers.prefill_plan(self.slots, wp, nrec)
        for r, (sl, w) in enumerate(zip(plan, hist)):
            cur_g.write_pos[:] = r
            verify = self.gpu.verify_dcache if dcache else self.gpu.verify
            verify(dev_cursors(cur_g), dev_i32(sl), DevWindow(w, self.act), scratch,
                   write_ring=1, fold_flagged=0, gs=gs1)
            cur_o.write_pos[:] = r
            osl = np.where(sl[self.orows] >= 0, self.oslots, -1).astype(np.int32)
            wo = helpers.window_rows(w, self.orows, 1)
            self.orc.write_ring(cur_o, osl, helpers.win_f64(wo, self.act), T=1)
        if dcache:
            # the deltas those one-token d-cache verifies record, in one pass
            # per (row, value head) (a pinned identity of the oracle)
            cur_o.write_pos[:] = wp[gslots]
            self.orc.fill_dring(cur_o, self.oslots)
        torch.cuda.synchronize()
        self.cur = CursorState(wp.copy(), base.copy(),
                               (wp + 2 * shape.max_spec > shape.L).astype(np.int32))
        self.ocur = CursorState(wp[gslots].copy(), base[gslots].copy(),
                                self.cur.is_flush[gslots].copy())
        self.dcur = dev_cursors(self.cur)
        self.dslots = dev_i32(self.slots)
        self.hist = hist
        self.wp0 = wp.copy()
        self.base0 = base.copy()

    def window(self) -> synth.Window:
        return synth.window(self.rng, self.shape, self.variant)

    def oracle_verify(self, win: synth.Window, write_ring=True, fold_flagged=True, pairs=None,
                      dcache=False):
        wo = helpers.window_rows(win, self.orows, self.shape.T)
        return self.orc.verify(self.ocur, self.oslots, helpers.win_f64(wo, self.act),
                               write_ring=write_ring, fold_flagged=fold_flagged, pairs=pairs,
                               dcache=dcache)

    def gpu_out_rows(self, o: torch.Tensor) -> np.ndarray:
        """GPU outputs of the oracle's rows, widened to float64."""
        T = self.shape.T
        idx = (self.orows[:, None] * T + np.arange(T)[None, :]).reshape(-1)
        return host_f64(o)[idx]


# ------------------------------------------------- per-channel-gate (KDA) layer

class KdaGpuLayer(GpuLayer):
    """One KDA layer's device tensors: dt_bias [HV, K], ring g [slots, HV, L, K]."""

    def verify(self, cur, slot_idx, win: DevWindow, o, write_ring=1, fold_flagged=1, gs=None):
        gv.gdn_kda_spec_verify_ring(gs or self.gs, win.q, win.k, win.v, win.a, win.b, self.A_log,
                                    self.dt_bias, self.S, slot_idx, cur[0], cur[1], cur[2],
                                    self.rawk, self.rawv, self.g, self.beta, write_ring,
                                    fold_flagged, o)

    def fold(self, cur, slot_idx, only_flagged=1, gs=None):
        gv.gdn_kda_exact_fold(gs or self.gs, 1, 0, 0, self.S, self.rawk, self.rawv, self.g,
                              self.beta, slot_idx, cur[0], cur[1], cur[2], only_flagged)


class KdaPair:
    """A GPU KDA layer and an oracle KDA layer from one seed, rings pre-filled
    (GPU: the library's verify with one-token windows, write_ring on, no fold;
    oracle: its own ring write of the same raw records)."""

    def __init__(self, shape: synth.LayerShape, seed: int, variant: str = "base",
                 wp_by_slot=None, base_by_slot=None, slots=None, oracle_rows=None):
        require_gpu()
        self.shape = shape
        self.act = shape.act
        rng = synth.make_rng(seed)
        self.rng = rng
        self.variant = variant
        self.params = synth.kda_layer_params(rng, shape, variant)
        self.slots = synth.slot_choice(rng, shape) if slots is None else np.asarray(slots, np.int32)
        cd = synth.random_cursors(rng, shape)
        wp = cd.write_pos if wp_by_slot is None else np.asarray(wp_by_slot, np.int32)
        base = cd.cache_base if base_by_slot is None else np.asarray(base_by_slot, np.int32)
        self.template = synth.kda_ring_garbage_template(rng, shape)
        self.gpu = KdaGpuLayer(shape, self.params, self.template)
        self.orows = np.arange(shape.B) if oracle_rows is None else np.asarray(oracle_rows)
        osh = shape.replace(B=len(self.orows), num_slots=len(self.orows))
        self.oshape = osh
        self.oslots = np.arange(len(self.orows), dtype=np.int32)
        gslots = self.slots[self.orows]
        self.gslots = gslots
        self.orc = oracle.OracleKDA(osh, self.params.A_log, self.params.dt_bias,
                                    self.params.S0[gslots])
        nrec = int(wp[self.slots].max()) if len(self.slots) else 0
        hist = synth.kda_history_windows(rng, shape, nrec, variant)
        gs1 = self.gpu.gs.replace(T=1)
        cur_g = CursorState(np.zeros(shape.num_slots, np.int32), base.copy(),
                            np.zeros(shape.num_slots, np.int32))
        cur_o = CursorState(np.zeros(osh.num_slots, np.int32), base[gslots].copy(),
                            np.zeros(osh.num_slots, np.int32))
        scratch = self.gpu.new_out(T=1)
        for r, (sl, w) in enumerate(zip(helpers.prefill_plan(self.slots, wp, nrec), hist)):
            cur_g.write_pos[:] = r
            self.gpu.verify(dev_cursors(cur_g), dev_i32(sl), DevWindow(w, self.act), scratch,
                            write_ring=1, fold_flagged=0, gs=gs1)
            cur_o.write_pos[:] = r
            osl = np.where(sl[self.orows] >= 0, self.oslots, -1).astype(np.int32)
            wo = helpers.window_rows(w, self.orows, 1)
            self.orc.write_ring(cur_o, osl, helpers.win_f64(wo, self.act), T=1)
        torch.cuda.synchronize()
        self.cur = CursorState(wp.copy(), base.copy(),
                               (wp + 2 * shape.max_spec > shape.L).astype(np.int32))
        self.ocur = CursorState(wp[gslots].copy(), base[gslots].copy(),
                                self.cur.is_flush[gslots].copy())
        self.dcur = dev_cursors(self.cur)
        self.dslots = dev_i32(self.slots)
        self.hist = hist
        self.wp0 = wp.copy()
        self.base0 = base.copy()

    def window(self) -> synth.Window:
        return synth.kda_window(self.rng, self.shape, self.variant)

    def oracle_verify(self, win: synth.Window, write_ring=True, fold_flagged=True):
        wo = helpers.window_rows(win, self.orows, self.shape.T)
        return self.orc.verify(self.ocur, self.oslots, helpers.win_f64(wo, self.act),
                               write_ring=write_ring, fold_flagged=fold_flagged)

    def gpu_out_rows(self, o: torch.Tensor) -> np.ndarray:
        T = self.shape.T
        idx = (self.orows[:, None] * T + np.arange(T)[None, :]).reshape(-1)
        return host_f64(o)[idx]
