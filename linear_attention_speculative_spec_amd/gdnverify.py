"""ctypes binding of libgdnverify with the C ABI's names.

Argument marshalling only: tensors become device pointers, the stream
defaults to torch's current stream, a negative status raises GdnError.  Every
computation runs in the HIP library; there is no fallback.  Because the C ABI
sees raw pointers, this layer also checks each tensor's device, dtype,
contiguity and size against the shape before anything is enqueued.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdnverify.so")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_ELAUNCH = 0, -1, -2, -3
GDN_F32, GDN_BF16 = 0, 1

EXPORTED = (
    "gdn_spec_verify_ring", "gdn_exact_fold", "gdn_advance_cursors", "gdn_reset_cursors",
    "gdn_recurrent_verify_snapshot", "gdn_snapshot_commit", "gdn_ring_bytes",
    "gdn_snapshot_bytes", "gdn_validate_shape", "gdn_status_str",
    "gdn_spec_verify_dcache", "gdn_dring_bytes",
    "gdn_kda_spec_verify_ring", "gdn_kda_exact_fold", "gdn_kda_ring_bytes",
)


class GdnShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "H", "HV", "K", "V", "L", "max_spec_len", "num_slots", "act")] + \
               [(n, ctypes.c_float) for n in ("scale", "softplus_threshold", "l2norm_eps")]

    @classmethod
    def from_layer(cls, ls, **override) -> "GdnShape":
        """From a synth.LayerShape (or any object with the same fields)."""
        d = dict(B=ls.B, T=ls.T, H=ls.H, HV=ls.HV, K=ls.K, V=ls.V, L=ls.L,
                 max_spec_len=ls.max_spec, num_slots=ls.num_slots,
                 act=GDN_BF16 if ls.act == "bf16" else GDN_F32, scale=ls.scale,
                 softplus_threshold=ls.softplus_threshold, l2norm_eps=ls.l2norm_eps)
        d.update(override)
        return cls(**d)

    def replace(self, **kw) -> "GdnShape":
        d = {n: getattr(self, n) for n, _ in self._fields_}
        d.update(kw)
        return GdnShape(**d)


class GdnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_str(status)} (status {status})")
        self.status = status


_lib = None
_vp = ctypes.c_void_p
_sp = ctypes.POINTER(GdnShape)
_i = ctypes.c_int


def lib():
    """The loaded library; raises if it was not built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it first "
                               "(python -m linear_attention_speculative_spec_amd._build)")
        L = ctypes.CDLL(_LIB_PATH)
        L.gdn_spec_verify_ring.argtypes = [_sp] + [_vp] * 16 + [_i, _i, _vp, _vp]
        L.gdn_spec_verify_dcache.argtypes = [_sp] + [_vp] * 17 + [_i, _i, _vp, _vp]
        L.gdn_exact_fold.argtypes = [_sp, _i, ctypes.c_int64, ctypes.c_int64] + [_vp] * 9 + [_i, _vp]
        L.gdn_kda_spec_verify_ring.argtypes = [_sp] + [_vp] * 16 + [_i, _i, _vp, _vp]
        L.gdn_kda_exact_fold.argtypes = [_sp, _i, ctypes.c_int64, ctypes.c_int64] + [_vp] * 9 + [_i, _vp]
        L.gdn_advance_cursors.argtypes = [_sp] + [_vp] * 6
        L.gdn_reset_cursors.argtypes = [_sp, _vp, ctypes.c_int32, ctypes.c_int32] + [_vp] * 4
        L.gdn_recurrent_verify_snapshot.argtypes = [_sp] + [_vp] * 17 + [_i, _vp]
        L.gdn_snapshot_commit.argtypes = [_sp] + [_vp] * 5
        for fn in ("gdn_spec_verify_ring", "gdn_spec_verify_dcache", "gdn_exact_fold", "gdn_advance_cursors",
                   "gdn_reset_cursors", "gdn_recurrent_verify_snapshot", "gdn_snapshot_commit",
                   "gdn_validate_shape", "gdn_kda_spec_verify_ring", "gdn_kda_exact_fold"):
            getattr(L, fn).restype = ctypes.c_int
        L.gdn_validate_shape.argtypes = [_sp]
        L.gdn_ring_bytes.argtypes = [_sp]
        L.gdn_ring_bytes.restype = ctypes.c_size_t
        L.gdn_snapshot_bytes.argtypes = [_sp]
        L.gdn_snapshot_bytes.restype = ctypes.c_size_t
        L.gdn_dring_bytes.argtypes = [_sp]
        L.gdn_dring_bytes.restype = ctypes.c_size_t
        L.gdn_kda_ring_bytes.argtypes = [_sp]
        L.gdn_kda_ring_bytes.restype = ctypes.c_size_t
        L.gdn_status_str.argtypes = [_i]
        L.gdn_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().gdn_status_str(int(status)).decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return _vp(x.data_ptr())
    return _vp(int(x))


def _stream(stream):
    if stream is None:
        return _vp(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return _vp(stream.cuda_stream)
    return _vp(int(stream))


def _act_dtype(shape: GdnShape):
    return torch.bfloat16 if shape.act == GDN_BF16 else torch.float32


def _need(name, t, numel, dtype):
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        return                                  # raw device pointer: caller's contract
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")


def _check(fn, status):
    if status != GDN_OK:
        raise GdnError(fn, status)


def _window_checks(sh, q, k, v, a, b, A_log, dt_bias):
    act = _act_dtype(sh)
    n = sh.B * sh.T
    _need("q", q, n * sh.H * sh.K, act)
    _need("k", k, n * sh.H * sh.K, act)
    _need("v", v, n * sh.HV * sh.V, act)
    _need("a", a, n * sh.HV, act)
    _need("b", b, n * sh.HV, act)
    _need("A_log", A_log, sh.HV, torch.float32)
    _need("dt_bias", dt_bias, sh.HV, torch.float32)


def _ring_checks(sh, rawk, rawv, g, beta, layers=1, slot_stride=0):
    """Ring arrays of `layers` layers placed `slot_stride` slots apart."""
    act = _act_dtype(sh)
    slots = (layers - 1) * (slot_stride or sh.num_slots) + sh.num_slots
    _need("ring_rawk", rawk, slots * sh.H * sh.L * sh.K, act)
    _need("ring_rawv", rawv, slots * sh.HV * sh.L * sh.V, act)
    _need("ring_g", g, slots * sh.HV * sh.L, torch.float32)
    _need("ring_beta", beta, slots * sh.HV * sh.L, torch.float32)


def _kda_window_checks(sh, q, k, v, a, b, A_log, dt_bias):
    act = _act_dtype(sh)
    n = sh.B * sh.T
    _need("q", q, n * sh.H * sh.K, act)
    _need("k", k, n * sh.H * sh.K, act)
    _need("v", v, n * sh.HV * sh.V, act)
    _need("a", a, n * sh.HV * sh.K, act)
    _need("b", b, n * sh.HV, act)
    _need("A_log", A_log, sh.HV, torch.float32)
    _need("dt_bias", dt_bias, sh.HV * sh.K, torch.float32)


def _kda_ring_checks(sh, rawk, rawv, g, beta, layers=1, slot_stride=0):
    act = _act_dtype(sh)
    slots = (layers - 1) * (slot_stride or sh.num_slots) + sh.num_slots
    _need("ring_rawk", rawk, slots * sh.H * sh.L * sh.K, act)
    _need("ring_rawv", rawv, slots * sh.HV * sh.L * sh.V, act)
    _need("ring_g", g, slots * sh.HV * sh.L * sh.K, torch.float32)
    _need("ring_beta", beta, slots * sh.HV * sh.L, torch.float32)


def _cursor_checks(sh, *cur):
    for name, c in zip(("write_pos", "cache_base", "is_flush"), cur):
        _need(name, c, sh.num_slots, torch.int32)


def gdn_spec_verify_ring(shape, q, k, v, a, b, A_log, dt_bias, S, slot_idx, write_pos,
                         cache_base, is_flush, ring_rawk, ring_rawv, ring_g, ring_beta,
                         write_ring, fold_flagged, o, stream=None):
    _window_checks(shape, q, k, v, a, b, A_log, dt_bias)
    _need("S", S, shape.num_slots * shape.HV * shape.V * shape.K, torch.float32)
    _need("slot_idx", slot_idx, shape.B, torch.int32)
    _cursor_checks(shape, write_pos, cache_base, is_flush)
    _ring_checks(shape, ring_rawk, ring_rawv, ring_g, ring_beta)
    _need("o", o, shape.B * shape.T * shape.HV * shape.V, _act_dtype(shape))
    st = lib().gdn_spec_verify_ring(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log),
        _ptr(dt_bias), _ptr(S), _ptr(slot_idx), _ptr(write_pos), _ptr(cache_base),
        _ptr(is_flush), _ptr(ring_rawk), _ptr(ring_rawv), _ptr(ring_g), _ptr(ring_beta),
        int(write_ring), int(fold_flagged), _ptr(o), _stream(stream))
    _check("gdn_spec_verify_ring", st)


def gdn_spec_verify_dcache(shape, q, k, v, a, b, A_log, dt_bias, S, slot_idx, write_pos,
                           cache_base, is_flush, ring_rawk, ring_rawv, ring_g, ring_beta,
                           ring_d, write_ring, fold_flagged, o, stream=None):
    _window_checks(shape, q, k, v, a, b, A_log, dt_bias)
    _need("S", S, shape.num_slots * shape.HV * shape.V * shape.K, torch.float32)
    _need("slot_idx", slot_idx, shape.B, torch.int32)
    _cursor_checks(shape, write_pos, cache_base, is_flush)
    _ring_checks(shape, ring_rawk, ring_rawv, ring_g, ring_beta)
    _need("ring_d", ring_d, shape.num_slots * shape.HV * shape.L * shape.V, torch.float32)
    _need("o", o, shape.B * shape.T * shape.HV * shape.V, _act_dtype(shape))
    st = lib().gdn_spec_verify_dcache(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log),
        _ptr(dt_bias), _ptr(S), _ptr(slot_idx), _ptr(write_pos), _ptr(cache_base),
        _ptr(is_flush), _ptr(ring_rawk), _ptr(ring_rawv), _ptr(ring_g), _ptr(ring_beta),
        _ptr(ring_d), int(write_ring), int(fold_flagged), _ptr(o), _stream(stream))
    _check("gdn_spec_verify_dcache", st)


def gdn_exact_fold(shape, num_layers, layer_stride_S, layer_stride_ring, S, ring_rawk, ring_rawv,
                   ring_g, ring_beta, slot_idx, write_pos, cache_base, is_flush, only_flagged,
                   stream=None):
    per_layer = shape.num_slots * shape.HV * shape.V * shape.K
    _need("S", S, (num_layers - 1) * (layer_stride_S or per_layer) + per_layer, torch.float32)
    _ring_checks(shape, ring_rawk, ring_rawv, ring_g, ring_beta, layers=num_layers,
                 slot_stride=layer_stride_ring)
    _need("slot_idx", slot_idx, shape.B, torch.int32)
    _cursor_checks(shape, write_pos, cache_base, *((is_flush,) if only_flagged else ()))
    st = lib().gdn_exact_fold(ctypes.byref(shape), int(num_layers), int(layer_stride_S),
                              int(layer_stride_ring), _ptr(S), _ptr(ring_rawk),
                              _ptr(ring_rawv), _ptr(ring_g), _ptr(ring_beta), _ptr(slot_idx),
                              _ptr(write_pos), _ptr(cache_base), _ptr(is_flush),
                              int(only_flagged), _stream(stream))
    _check("gdn_exact_fold", st)


def gdn_kda_spec_verify_ring(shape, q, k, v, a, b, A_log, dt_bias, S, slot_idx, write_pos,
                             cache_base, is_flush, ring_rawk, ring_rawv, ring_g, ring_beta,
                             write_ring, fold_flagged, o, stream=None):
    _kda_window_checks(shape, q, k, v, a, b, A_log, dt_bias)
    _need("S", S, shape.num_slots * shape.HV * shape.V * shape.K, torch.float32)
    _need("slot_idx", slot_idx, shape.B, torch.int32)
    _cursor_checks(shape, write_pos, cache_base, is_flush)
    _kda_ring_checks(shape, ring_rawk, ring_rawv, ring_g, ring_beta)
    _need("o", o, shape.B * shape.T * shape.HV * shape.V, _act_dtype(shape))
    st = lib().gdn_kda_spec_verify_ring(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log),
        _ptr(dt_bias), _ptr(S), _ptr(slot_idx), _ptr(write_pos), _ptr(cache_base),
        _ptr(is_flush), _ptr(ring_rawk), _ptr(ring_rawv), _ptr(ring_g), _ptr(ring_beta),
        int(write_ring), int(fold_flagged), _ptr(o), _stream(stream))
    _check("gdn_kda_spec_verify_ring", st)


def gdn_kda_exact_fold(shape, num_layers, layer_stride_S, layer_stride_ring, S, ring_rawk,
                       ring_rawv, ring_g, ring_beta, slot_idx, write_pos, cache_base, is_flush,
                       only_flagged, stream=None):
    per_layer = shape.num_slots * shape.HV * shape.V * shape.K
    _need("S", S, (num_layers - 1) * (layer_stride_S or per_layer) + per_layer, torch.float32)
    _kda_ring_checks(shape, ring_rawk, ring_rawv, ring_g, ring_beta, layers=num_layers,
                     slot_stride=layer_stride_ring)
    _need("slot_idx", slot_idx, shape.B, torch.int32)
    _cursor_checks(shape, write_pos, cache_base, *((is_flush,) if only_flagged else ()))
    st = lib().gdn_kda_exact_fold(ctypes.byref(shape), int(num_layers), int(layer_stride_S),
                                  int(layer_stride_ring), _ptr(S), _ptr(ring_rawk),
                                  _ptr(ring_rawv), _ptr(ring_g), _ptr(ring_beta), _ptr(slot_idx),
                                  _ptr(write_pos), _ptr(cache_base), _ptr(is_flush),
                                  int(only_flagged), _stream(stream))
    _check("gdn_kda_exact_fold", st)


def gdn_kda_ring_bytes(shape) -> int:
    return int(lib().gdn_kda_ring_bytes(ctypes.byref(shape)))


def gdn_advance_cursors(shape, slot_idx, accept, write_pos, cache_base, is_flush, stream=None):
    _need("slot_idx", slot_idx, shape.B, torch.int32)
    _need("accept", accept, shape.B, torch.int32)
    _cursor_checks(shape, write_pos, cache_base, is_flush)
    st = lib().gdn_advance_cursors(ctypes.byref(shape), _ptr(slot_idx), _ptr(accept),
                                   _ptr(write_pos), _ptr(cache_base), _ptr(is_flush),
                                   _stream(stream))
    _check("gdn_advance_cursors", st)


def gdn_reset_cursors(shape, slots, n, init_flush, write_pos, cache_base, is_flush, stream=None):
    if n:
        _need("slots", slots, n, torch.int32)
    _cursor_checks(shape, write_pos, cache_base, is_flush)
    st = lib().gdn_reset_cursors(ctypes.byref(shape), _ptr(slots), int(n), int(init_flush),
                                 _ptr(write_pos), _ptr(cache_base), _ptr(is_flush),
                                 _stream(stream))
    _check("gdn_reset_cursors", st)


def gdn_recurrent_verify_snapshot(shape, q, k, v, a, b, A_log, dt_bias, S, slot_idx, snap, o,
                                  ring_rawk=None, ring_rawv=None, ring_g=None, ring_beta=None,
                                  write_pos=None, cache_base=None, write_ring=0, stream=None):
    _window_checks(shape, q, k, v, a, b, A_log, dt_bias)
    _need("S", S, shape.num_slots * shape.HV * shape.V * shape.K, torch.float32)
    _need("slot_idx", slot_idx, shape.B, torch.int32)
    _need("snap", snap, shape.B * shape.T * shape.HV * shape.V * shape.K, torch.float32)
    _need("o", o, shape.B * shape.T * shape.HV * shape.V, _act_dtype(shape))
    if write_ring:
        _ring_checks(shape, ring_rawk, ring_rawv, ring_g, ring_beta)
        _need("write_pos", write_pos, shape.num_slots, torch.int32)
        _need("cache_base", cache_base, shape.num_slots, torch.int32)
    st = lib().gdn_recurrent_verify_snapshot(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log),
        _ptr(dt_bias), _ptr(S), _ptr(slot_idx), _ptr(snap), _ptr(o), _ptr(ring_rawk),
        _ptr(ring_rawv), _ptr(ring_g), _ptr(ring_beta), _ptr(write_pos), _ptr(cache_base),
        int(write_ring), _stream(stream))
    _check("gdn_recurrent_verify_snapshot", st)


def gdn_snapshot_commit(shape, snap, slot_idx, accept, S, stream=None):
    _need("snap", snap, shape.B * shape.T * shape.HV * shape.V * shape.K, torch.float32)
    _need("slot_idx", slot_idx, shape.B, torch.int32)
    _need("accept", accept, shape.B, torch.int32)
    _need("S", S, shape.num_slots * shape.HV * shape.V * shape.K, torch.float32)
    st = lib().gdn_snapshot_commit(ctypes.byref(shape), _ptr(snap), _ptr(slot_idx),
                                   _ptr(accept), _ptr(S), _stream(stream))
    _check("gdn_snapshot_commit", st)


def gdn_ring_bytes(shape) -> int:
    return int(lib().gdn_ring_bytes(ctypes.byref(shape)))


def gdn_snapshot_bytes(shape) -> int:
    return int(lib().gdn_snapshot_bytes(ctypes.byref(shape)))


def gdn_dring_bytes(shape) -> int:
    return int(lib().gdn_dring_bytes(ctypes.byref(shape)))


def gdn_validate_shape(shape) -> int:
    return int(lib().gdn_validate_shape(ctypes.byref(shape)))
