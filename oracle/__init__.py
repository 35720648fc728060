"""fp64 CPU oracle for the GDN ReplaySSM ring spec-verify.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the library.  It shares no code with
the HIP path; the only thing both sides share is the seeded input generator.

* ``gdn_oracle.c``  - plain fp64 recurrence: gating, l2 norm, the gated delta
  step, verify (history replay then window), exact fold, snapshot baseline.
* ``kda_oracle.c``  - the same for the per-channel-gate (KDA) layer.
* ``cursors.py``    - the integer ring/cursor algorithm.
* ``closed_form.py``- the chunked closed form, used only to pin the recurrence.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
to something other than itself: the verify by an independent closed-form
solve, special cases and causality; the fold by step-by-step replay; the
snapshot baseline by a hand-computed two-token window and by the pinned fold
of each window prefix; the cursor advance by the walks printed on the pages
and by invariants; the cursor reset by its behaviour at the prefill -> decode
handoff.  A planted mistake in each of them fails one of those tests.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import cursors  # noqa: F401  (re-export)
from .cursors import CursorState, advance, reset  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_SRC_KDA = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libgdnoracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, _SRC_KDA, "-o", tmp,
                               "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("B", "T", "H", "HV", "K", "V", "L", "max_spec", "num_slots")] + \
               [(n, ctypes.c_double) for n in ("scale", "softplus_threshold", "eps")]


_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)


class _Args(ctypes.Structure):
    _fields_ = [("sh", _Shape),
                ("S", _dp), ("rawk", _dp), ("rawv", _dp), ("rg", _dp), ("rb", _dp),
                ("wp", _ip), ("base", _ip), ("flush", _ip), ("slot", _ip),
                ("q", _dp), ("k", _dp), ("v", _dp), ("a", _dp), ("b", _dp),
                ("A_log", _dp), ("dt_bias", _dp),
                ("o", _dp), ("snap", _dp),
                ("fold_flagged", ctypes.c_int), ("only_flagged", ctypes.c_int),
                ("pair_row", _ip), ("pair_hv", _ip), ("n_pairs", ctypes.c_int),
                ("dwin", _dp), ("rd", _dp)]


class _KArgs(ctypes.Structure):
    _fields_ = [("sh", _Shape),
                ("S", _dp), ("rawk", _dp), ("rawv", _dp), ("rg", _dp), ("rb", _dp),
                ("wp", _ip), ("base", _ip), ("flush", _ip), ("slot", _ip),
                ("q", _dp), ("k", _dp), ("v", _dp), ("a", _dp), ("b", _dp),
                ("A_log", _dp), ("dt_bias", _dp), ("o", _dp),
                ("fold_flagged", ctypes.c_int), ("only_flagged", ctypes.c_int)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        for fn in ("orc_verify", "orc_snapshot"):
            getattr(lib, fn).argtypes = [ctypes.POINTER(_Args), ctypes.c_int, ctypes.c_int]
            getattr(lib, fn).restype = None
        lib.orc_write_ring.argtypes = [ctypes.POINTER(_Args)]
        lib.orc_write_ring.restype = None
        lib.orc_fold.argtypes = [ctypes.POINTER(_Args), ctypes.c_int]
        lib.orc_fold.restype = None
        lib.orc_fill_dring.argtypes = [ctypes.POINTER(_Args), ctypes.c_int]
        lib.orc_fill_dring.restype = None
        lib.orc_step.argtypes = [_dp, ctypes.c_int, ctypes.c_int, _dp, _dp,
                                 ctypes.c_double, ctypes.c_double, ctypes.c_double]
        lib.orc_step.restype = None
        lib.orc_step_d.argtypes = [_dp, ctypes.c_int, ctypes.c_int, _dp, _dp,
                                   ctypes.c_double, ctypes.c_double, ctypes.c_double, _dp]
        lib.orc_step_d.restype = None
        lib.orc_gate.argtypes = [ctypes.c_double] * 5 + [_dp, _dp]
        lib.orc_gate.restype = None
        lib.orc_rnorm.argtypes = [_dp, ctypes.c_int, ctypes.c_double]
        lib.orc_rnorm.restype = ctypes.c_double
        lib.orc_readout.argtypes = [_dp, ctypes.c_int, ctypes.c_int, _dp, ctypes.c_double,
                                    ctypes.c_double, _dp]
        lib.orc_readout.restype = None
        assert lib.orc_args_size() == ctypes.sizeof(_Args)
        for fn in ("kda_verify",):
            getattr(lib, fn).argtypes = [ctypes.POINTER(_KArgs), ctypes.c_int, ctypes.c_int]
            getattr(lib, fn).restype = None
        lib.kda_write_ring.argtypes = [ctypes.POINTER(_KArgs)]
        lib.kda_write_ring.restype = None
        lib.kda_fold.argtypes = [ctypes.POINTER(_KArgs), ctypes.c_int]
        lib.kda_fold.restype = None
        lib.kda_gate.argtypes = [_dp, ctypes.c_double, ctypes.c_double, _dp, ctypes.c_int,
                                 ctypes.c_double, _dp, _dp]
        lib.kda_gate.restype = None
        lib.kda_step.argtypes = [_dp, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp,
                                 ctypes.c_double, ctypes.c_double]
        lib.kda_step.restype = None
        lib.kda_readout.argtypes = [_dp, ctypes.c_int, ctypes.c_int, _dp, ctypes.c_double,
                                    ctypes.c_double, _dp]
        lib.kda_readout.restype = None
        assert lib.kda_args_size() == ctypes.sizeof(_KArgs)
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x, kind=_dp):
    return x.ctypes.data_as(kind) if x is not None else None


def default_threads() -> int:
    """Host threads for the pair loop: the affinity mask, capped by OMP_NUM_THREADS."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = int(os.environ.get("OMP_NUM_THREADS", n) or n)
    return max(1, min(n, cap))


# ------------------------------------------------------------- scalar pieces

def gate(a: float, b: float, A_log: float, dt_bias: float, threshold: float = 20.0):
    """(g, beta) for one token and value head."""
    g, beta = ctypes.c_double(), ctypes.c_double()
    _load().orc_gate(a, b, A_log, dt_bias, threshold, ctypes.byref(g), ctypes.byref(beta))
    return g.value, beta.value


def rnorm(x, eps: float = 1e-6) -> float:
    x = _f64(x)
    return _load().orc_rnorm(_ptr(x), x.size, eps)


def step(S, k_raw, v, g: float, beta: float, eps: float = 1e-6) -> np.ndarray:
    """One gated delta-rule step on a copy of S (V x K)."""
    S = _f64(S).copy()
    k_raw, v = _f64(k_raw), _f64(v)
    V, K = S.shape
    _load().orc_step(_ptr(S), V, K, _ptr(k_raw), _ptr(v), g, beta, eps)
    return S


def step_d(S, k_raw, v, g: float, beta: float, eps: float = 1e-6):
    """One step on a copy of S; returns (new S, corrected delta d [V])."""
    S = _f64(S).copy()
    k_raw, v = _f64(k_raw), _f64(v)
    V, K = S.shape
    d = np.empty(V)
    _load().orc_step_d(_ptr(S), V, K, _ptr(k_raw), _ptr(v), g, beta, eps, _ptr(d))
    return S, d


def readout(S, q_raw, scale: float = 1.0, eps: float = 1e-6) -> np.ndarray:
    S, q_raw = _f64(S), _f64(q_raw)
    V, K = S.shape
    o = np.empty(V)
    _load().orc_readout(_ptr(S), V, K, _ptr(q_raw), scale, eps, _ptr(o))
    return o


# ------------------------------------------------------------- layer state

class OracleLayer:
    """fp64 state of one GDN layer: checkpoint and raw-record ring.

    ``shape`` is a ``LayerShape``; S0 is any float array [num_slots, HV, V, K].
    Ring entries start as NaN so a read of an unwritten record poisons outputs.
    """

    def __init__(self, shape, A_log, dt_bias, S0):
        self.shape = shape
        self.A_log = _f64(A_log)
        self.dt_bias = _f64(dt_bias)
        self.S = _f64(S0).copy()
        sh = shape
        self.rawk = np.full((sh.num_slots, sh.H, sh.L, sh.K), np.nan)
        self.rawv = np.full((sh.num_slots, sh.HV, sh.L, sh.V), np.nan)
        self.g = np.full((sh.num_slots, sh.HV, sh.L), np.nan)
        self.beta = np.full((sh.num_slots, sh.HV, sh.L), np.nan)
        # ring of corrected deltas [num_slots, HV, L, V], made on first use
        # by a d-cache verify
        self.d = None
        self.last_dwin = None

    def _args(self, cur, slot_idx, win=None, o=None, snap=None, pairs=None, shape=None):
        sh = shape or self.shape
        keep = []

        def hold(x):
            keep.append(x)
            return x

        A = _Args()
        A.sh = _Shape(sh.B, sh.T, sh.H, sh.HV, sh.K, sh.V, sh.L, sh.max_spec, sh.num_slots,
                      sh.scale, sh.softplus_threshold, sh.l2norm_eps)
        A.S, A.rawk, A.rawv = _ptr(self.S), _ptr(self.rawk), _ptr(self.rawv)
        A.rg, A.rb = _ptr(self.g), _ptr(self.beta)
        A.wp, A.base, A.flush = _ptr(cur.write_pos, _ip), _ptr(cur.cache_base, _ip), \
            _ptr(cur.is_flush, _ip)
        A.slot = _ptr(hold(np.ascontiguousarray(slot_idx, dtype=np.int32)), _ip)
        if win is not None:
            A.q, A.k, A.v, A.a, A.b = (_ptr(hold(_f64(x))) for x in win)
        A.A_log, A.dt_bias = _ptr(self.A_log), _ptr(self.dt_bias)
        if o is not None:
            A.o = _ptr(o)
        if snap is not None:
            A.snap = _ptr(snap)
        if pairs is not None:
            pr = hold(np.ascontiguousarray([p[0] for p in pairs], dtype=np.int32))
            ph = hold(np.ascontiguousarray([p[1] for p in pairs], dtype=np.int32))
            A.pair_row, A.pair_hv, A.n_pairs = _ptr(pr, _ip), _ptr(ph, _ip), len(pairs)
        return A, keep

    def verify(self, cur, slot_idx, win, write_ring=True, fold_flagged=True,
               nthreads=None, pairs=None, T=None, dcache=False):
        """Outputs [B*T, HV, V] for every window position.

        ``win`` = (q, k, v, a, b) widened to float64, packed token-major.
        With ``dcache`` the window's corrected deltas are kept in
        ``last_dwin`` [B*T, HV, V] and, with ``write_ring``, recorded in the
        d ring ``self.d`` beside the raw records.
        """
        sh = self.shape if T is None else self.shape.replace(T=T)
        B = len(slot_idx)
        sh = sh.replace(B=B)
        o = np.full((B * sh.T, sh.HV, sh.V), np.nan)
        A, keep = self._args(cur, slot_idx, win, o=o, pairs=pairs, shape=sh)
        A.fold_flagged = int(fold_flagged)
        if dcache:
            if self.d is None:
                self.d = np.full((sh.num_slots, sh.HV, sh.L, sh.V), np.nan)
            self.last_dwin = np.full((B * sh.T, sh.HV, sh.V), np.nan)
            A.dwin, A.rd = _ptr(self.last_dwin), _ptr(self.d)
        _load().orc_verify(ctypes.byref(A), int(write_ring), nthreads or default_threads())
        del keep
        return o

    def write_ring(self, cur, slot_idx, win, T=None):
        """Record a window's raw records at logical positions write_pos + t."""
        sh = self.shape if T is None else self.shape.replace(T=T)
        sh = sh.replace(B=len(slot_idx))
        A, keep = self._args(cur, slot_idx, win, shape=sh)
        _load().orc_write_ring(ctypes.byref(A))
        del keep

    def fold(self, cur, slot_idx, only_flagged=True, nthreads=None):
        sh = self.shape.replace(B=len(slot_idx))
        A, keep = self._args(cur, slot_idx, shape=sh)
        A.only_flagged = int(only_flagged)
        _load().orc_fold(ctypes.byref(A), nthreads or default_threads())
        del keep

    def fill_dring(self, cur, slot_idx, nthreads=None):
        """Record the committed history's corrected deltas in the d ring in one
        pass per (row, value head): what one-token d-cache verifies of the same
        records would have stored."""
        sh = self.shape.replace(B=len(slot_idx))
        if self.d is None:
            self.d = np.full((sh.num_slots, sh.HV, sh.L, sh.V), np.nan)
        A, keep = self._args(cur, slot_idx, shape=sh)
        A.rd = _ptr(self.d)
        _load().orc_fill_dring(ctypes.byref(A), nthreads or default_threads())
        del keep

    def snapshot(self, slot_idx, win, cur=None, write_ring=False, nthreads=None):
        """Baseline: (o [B*T,HV,V], snap [B,T,HV,V,K]) from the checkpoint alone."""
        sh = self.shape.replace(B=len(slot_idx))
        if cur is None:
            cur = CursorState.zeros(sh.num_slots)
        o = np.full((sh.B * sh.T, sh.HV, sh.V), np.nan)
        snap = np.full((sh.B, sh.T, sh.HV, sh.V, sh.K), np.nan)
        A, keep = self._args(cur, slot_idx, win, o=o, snap=snap, shape=sh)
        _load().orc_snapshot(ctypes.byref(A), int(write_ring), nthreads or default_threads())
        del keep
        return o, snap


# ------------------------------------------------------ KDA (per-channel gate)

def kda_gate(a, b: float, A_log: float, dt_bias, threshold: float = 20.0):
    """(g [K], beta) of one token and value head with a per-channel gate."""
    a, dt_bias = _f64(a), _f64(dt_bias)
    g = np.empty(a.size)
    beta = ctypes.c_double()
    _load().kda_gate(_ptr(a), b, A_log, _ptr(dt_bias), a.size, threshold, _ptr(g), ctypes.byref(beta))
    return g, beta.value


def kda_step(S, k_raw, v, g, beta: float, eps: float = 1e-6) -> np.ndarray:
    """One per-channel-gate step on a copy of S (V x K); g has K entries."""
    S = _f64(S).copy()
    k_raw, v, g = _f64(k_raw), _f64(v), _f64(g)
    V, K = S.shape
    _load().kda_step(_ptr(S), V, K, _ptr(k_raw), _ptr(v), _ptr(g), beta, eps)
    return S


def kda_readout(S, q_raw, scale: float = 1.0, eps: float = 1e-6) -> np.ndarray:
    S, q_raw = _f64(S), _f64(q_raw)
    V, K = S.shape
    o = np.empty(V)
    _load().kda_readout(_ptr(S), V, K, _ptr(q_raw), scale, eps, _ptr(o))
    return o


class OracleKDA:
    """fp64 state of one KDA layer: checkpoint and a ring whose gate records
    hold K channels.  A_log [HV], dt_bias [HV, K]; windows carry a [B*T, HV, K].
    Ring entries start as NaN."""

    def __init__(self, shape, A_log, dt_bias, S0):
        self.shape = shape
        self.A_log = _f64(A_log)
        self.dt_bias = _f64(dt_bias)
        self.S = _f64(S0).copy()
        sh = shape
        self.rawk = np.full((sh.num_slots, sh.H, sh.L, sh.K), np.nan)
        self.rawv = np.full((sh.num_slots, sh.HV, sh.L, sh.V), np.nan)
        self.g = np.full((sh.num_slots, sh.HV, sh.L, sh.K), np.nan)
        self.beta = np.full((sh.num_slots, sh.HV, sh.L), np.nan)

    def _args(self, cur, slot_idx, win=None, o=None, shape=None):
        sh = shape or self.shape
        keep = []

        def hold(x):
            keep.append(x)
            return x

        A = _KArgs()
        A.sh = _Shape(sh.B, sh.T, sh.H, sh.HV, sh.K, sh.V, sh.L, sh.max_spec, sh.num_slots,
                      sh.scale, sh.softplus_threshold, sh.l2norm_eps)
        A.S, A.rawk, A.rawv = _ptr(self.S), _ptr(self.rawk), _ptr(self.rawv)
        A.rg, A.rb = _ptr(self.g), _ptr(self.beta)
        A.wp, A.base, A.flush = _ptr(cur.write_pos, _ip), _ptr(cur.cache_base, _ip), \
            _ptr(cur.is_flush, _ip)
        A.slot = _ptr(hold(np.ascontiguousarray(slot_idx, dtype=np.int32)), _ip)
        if win is not None:
            A.q, A.k, A.v, A.a, A.b = (_ptr(hold(_f64(x))) for x in win)
        A.A_log, A.dt_bias = _ptr(self.A_log), _ptr(self.dt_bias)
        if o is not None:
            A.o = _ptr(o)
        return A, keep

    def verify(self, cur, slot_idx, win, write_ring=True, fold_flagged=True, nthreads=None, T=None):
        """Outputs [B*T, HV, V]; win = (q, k, v, a [B*T,HV,K], b) widened to float64."""
        sh = self.shape if T is None else self.shape.replace(T=T)
        sh = sh.replace(B=len(slot_idx))
        o = np.full((sh.B * sh.T, sh.HV, sh.V), np.nan)
        A, keep = self._args(cur, slot_idx, win, o=o, shape=sh)
        A.fold_flagged = int(fold_flagged)
        _load().kda_verify(ctypes.byref(A), int(write_ring), nthreads or default_threads())
        del keep
        return o

    def write_ring(self, cur, slot_idx, win, T=None):
        sh = self.shape if T is None else self.shape.replace(T=T)
        sh = sh.replace(B=len(slot_idx))
        A, keep = self._args(cur, slot_idx, win, shape=sh)
        _load().kda_write_ring(ctypes.byref(A))
        del keep

    def fold(self, cur, slot_idx, only_flagged=True, nthreads=None):
        sh = self.shape.replace(B=len(slot_idx))
        A, keep = self._args(cur, slot_idx, shape=sh)
        A.only_flagged = int(only_flagged)
        _load().kda_fold(ctypes.byref(A), nthreads or default_threads())
        del keep
