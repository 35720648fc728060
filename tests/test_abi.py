"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and rejects malformed arguments on the host before any launch.
No call here reaches the GPU."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from linear_attention_speculative_spec_amd import gdnverify as gv
from linear_attention_speculative_spec_amd import synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "gdnverify.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    assert header_functions() == sorted(gv.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(gv._LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for st in (gv.GDN_OK, gv.GDN_EINVAL, gv.GDN_EUNSUPPORTED, gv.GDN_ELAUNCH):
        assert gv.status_str(st) and gv.status_str(st) != "unknown status"
    assert gv.status_str(-99) == "unknown status"


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_workload_shapes_are_valid(name):
    assert gv.gdn_validate_shape(gv.GdnShape.from_layer(synth.CONFIGS[name])) == gv.GDN_OK


BAD = [
    (dict(L=48), gv.GDN_EINVAL),                      # ring length not a power of two
    (dict(L=4, max_spec_len=4, T=4), gv.GDN_EINVAL),  # L < 2 * max_spec_len
    (dict(T=5), gv.GDN_EINVAL),                       # T > max_spec_len
    (dict(T=0), gv.GDN_EINVAL),
    (dict(HV=24), gv.GDN_EINVAL),                     # HV % H != 0
    (dict(act=7), gv.GDN_EINVAL),
    (dict(B=-1), gv.GDN_EINVAL),
    (dict(num_slots=0), gv.GDN_EINVAL),
    (dict(l2norm_eps=-1.0), gv.GDN_EINVAL),
    (dict(scale=float("inf")), gv.GDN_EINVAL),
    (dict(K=96), gv.GDN_EUNSUPPORTED),
    (dict(V=120), gv.GDN_EUNSUPPORTED),
    (dict(V=272), gv.GDN_EUNSUPPORTED),
    (dict(L=256), gv.GDN_EUNSUPPORTED),
    (dict(max_spec_len=32, T=4, L=128), gv.GDN_EUNSUPPORTED),
    (dict(K=256, L=128, max_spec_len=8, T=8), gv.GDN_EUNSUPPORTED),   # LDS over 160 KiB
]


@pytest.mark.parametrize("override,status", BAD)
def test_invalid_shapes_are_rejected(override, status):
    sh = gv.GdnShape.from_layer(synth.CONFIGS["qwen3next_b32"], **override)
    assert gv.gdn_validate_shape(sh) == status
    assert gv.gdn_ring_bytes(sh) == 0 and gv.gdn_snapshot_bytes(sh) == 0
    # every entry point refuses it before touching the device
    L = gv.lib()
    n = None
    assert L.gdn_spec_verify_ring(ctypes.byref(sh), *([n] * 16), 1, 1, n, n) == status
    assert L.gdn_exact_fold(ctypes.byref(sh), 1, 0, 0, *([n] * 9), 1, n) == status
    assert L.gdn_advance_cursors(ctypes.byref(sh), *([n] * 6)) == status
    assert L.gdn_reset_cursors(ctypes.byref(sh), n, 0, 0, n, n, n, n) == status
    assert L.gdn_recurrent_verify_snapshot(ctypes.byref(sh), *([n] * 17), 0, n) == status
    assert L.gdn_snapshot_commit(ctypes.byref(sh), *([n] * 5)) == status
    assert L.gdn_kda_spec_verify_ring(ctypes.byref(sh), *([n] * 16), 1, 1, n, n) == status
    assert L.gdn_kda_exact_fold(ctypes.byref(sh), 1, 0, 0, *([n] * 9), 1, n) == status
    assert gv.gdn_kda_ring_bytes(sh) == 0


def test_null_and_misaligned_pointers_are_rejected():
    # every call below must be refused on the host: none may reach a launch
    sh = gv.GdnShape.from_layer(synth.CONFIGS["qwen3next_b32"])
    L = gv.lib()
    n = None
    good = ctypes.c_void_p(1 << 20)           # never dereferenced: rejected first
    bad = ctypes.c_void_p((1 << 20) + 2)
    args = [good] * 16
    assert L.gdn_spec_verify_ring(ctypes.byref(sh), *([n] * 16), 1, 1, good, n) == gv.GDN_EINVAL
    args[0] = bad                              # q misaligned
    assert L.gdn_spec_verify_ring(ctypes.byref(sh), *args, 1, 1, good, n) == gv.GDN_EINVAL
    # output aliasing an input
    args = [good] * 16
    assert L.gdn_spec_verify_ring(ctypes.byref(sh), *args, 1, 1, good, n) == gv.GDN_EINVAL
    assert L.gdn_exact_fold(ctypes.byref(sh), 0, 0, 0, *([good] * 9), 1, n) == gv.GDN_EINVAL
    assert L.gdn_reset_cursors(ctypes.byref(sh), good, -1, 0, good, good, good, n) == gv.GDN_EINVAL
    assert L.gdn_advance_cursors(ctypes.byref(sh), good, n, good, good, good, n) == gv.GDN_EINVAL
    assert L.gdn_snapshot_commit(ctypes.byref(sh), good, good, n, good, n) == gv.GDN_EINVAL
    # the d-cache verify: null ring_d, misaligned ring_d, o aliasing ring_d
    args = [good] * 17
    args[16] = n
    assert L.gdn_spec_verify_dcache(ctypes.byref(sh), *args, 1, 1, ctypes.c_void_p(2 << 20), n) == gv.GDN_EINVAL
    args[16] = bad
    assert L.gdn_spec_verify_dcache(ctypes.byref(sh), *args, 1, 1, ctypes.c_void_p(2 << 20), n) == gv.GDN_EINVAL
    args = [ctypes.c_void_p((3 + i) << 20) for i in range(17)]
    assert L.gdn_spec_verify_dcache(ctypes.byref(sh), *args, 1, 1, args[16], n) == gv.GDN_EINVAL


def test_footprints():
    sh = gv.GdnShape.from_layer(synth.CONFIGS["qwen3next_b256"])
    rec = 16 * 128 * 2 + 32 * (128 * 2 + 8)          # 12544 bytes per slot-record
    assert rec == 12544
    assert gv.gdn_ring_bytes(sh) == 512 * 64 * rec
    assert gv.gdn_snapshot_bytes(sh) == 256 * 4 * 32 * 128 * 128 * 4
    assert gv.gdn_snapshot_bytes(sh) > 5 * gv.gdn_ring_bytes(sh)
    # the d ring: one fp32 delta row per (slot, value head, record)
    assert gv.gdn_dring_bytes(sh) == 512 * 32 * 64 * 128 * 4


def test_binding_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(gv, "_lib", None)
    monkeypatch.setattr(gv, "_LIB_PATH", "/nonexistent/libgdnverify.so")
    with pytest.raises(RuntimeError, match="missing"):
        gv.lib()


def test_fold_layer_strides_are_validated():
    # per-layer placement: fp32 elements of S, slots of the ring arrays; 0
    # means back to back.  Negative, overlapping or misaligned strides are
    # refused on the host.
    sh = gv.GdnShape.from_layer(synth.CONFIGS["qwen3next_b32"])
    L = gv.lib()
    per_S = sh.num_slots * sh.HV * sh.V * sh.K
    ptrs = [ctypes.c_void_p((3 + i) << 20) for i in range(9)]
    n = None
    for nl, ls, lr in ((2, -4, 0), (2, 0, -1), (3, per_S - 4, 0), (3, 0, sh.num_slots - 1),
                       (2, per_S + 2, 0), (1, -4, 0)):
        assert L.gdn_exact_fold(ctypes.byref(sh), nl, ls, lr, *ptrs, 1, n) == gv.GDN_EINVAL, (nl, ls, lr)


def test_bf16_gate_words_stay_inside_the_buffers():
    # the ring verify reads bf16 gate inputs as aligned words of two
    # activations: misaligned a/b are refused, and so is an odd B*T*HV
    # (its last word would reach past the end of a and b)
    L = gv.lib()
    n = None
    base = gv.GdnShape.from_layer(synth.CONFIGS["qwen3next_b32"])
    args = [ctypes.c_void_p((3 + i) << 20) for i in range(16)]
    out = ctypes.c_void_p(40 << 20)
    odd = base.replace(B=3, T=1, H=1, HV=1, max_spec_len=1, L=64)
    assert gv.gdn_validate_shape(odd) == gv.GDN_OK
    assert L.gdn_spec_verify_ring(ctypes.byref(odd), *args, 1, 1, out, n) == gv.GDN_EUNSUPPORTED
    mis = list(args)
    mis[3] = ctypes.c_void_p((6 << 20) + 2)      # a: 2-byte aligned only
    assert L.gdn_spec_verify_ring(ctypes.byref(base), *mis, 1, 1, out, n) == gv.GDN_EINVAL
    # fp32 activations read a and b element by element: an odd count is fine
    odd32 = odd.replace(act=gv.GDN_F32)
    assert gv.gdn_validate_shape(odd32) == gv.GDN_OK


def test_kda_envelope_pointers_and_footprint():
    # the per-channel-gate layer: 64-row state tiles (V a multiple of 64),
    # 16-byte aligned ring_g, is_flush required by the fold only with
    # only_flagged; refused on the host before any launch
    L = gv.lib()
    n = None
    base = gv.GdnShape.from_layer(synth.CONFIGS["qwen3next_b32"])
    args = [ctypes.c_void_p((3 + i) << 20) for i in range(16)]
    out = ctypes.c_void_p(40 << 20)
    v48 = base.replace(V=48)
    assert gv.gdn_validate_shape(v48) == gv.GDN_OK
    assert L.gdn_kda_spec_verify_ring(ctypes.byref(v48), *args, 1, 1, out, n) == gv.GDN_EUNSUPPORTED
    assert L.gdn_kda_exact_fold(ctypes.byref(v48), 1, 0, 0, *args[:9], 1, n) == gv.GDN_EUNSUPPORTED
    assert gv.gdn_kda_ring_bytes(v48) == 0
    mis = list(args)
    mis[14] = ctypes.c_void_p((17 << 20) + 4)    # ring_g: 4-byte aligned only
    assert L.gdn_kda_spec_verify_ring(ctypes.byref(base), *mis, 1, 1, out, n) == gv.GDN_EINVAL
    fold = [ctypes.c_void_p((3 + i) << 20) for i in range(9)]
    fold[3] = ctypes.c_void_p((6 << 20) + 4)     # ring_g of the fold
    assert L.gdn_kda_exact_fold(ctypes.byref(base), 1, 0, 0, *fold, 1, n) == gv.GDN_EINVAL
    fold = [ctypes.c_void_p((3 + i) << 20) for i in range(8)] + [n]   # no is_flush
    assert L.gdn_kda_exact_fold(ctypes.byref(base), 1, 0, 0, *fold, 1, n) == gv.GDN_EINVAL
    # output aliasing an input; negative and overlapping layer strides
    assert L.gdn_kda_spec_verify_ring(ctypes.byref(base), *args, 1, 1, args[0], n) == gv.GDN_EINVAL
    per_S = base.num_slots * base.HV * base.V * base.K
    fold = [ctypes.c_void_p((3 + i) << 20) for i in range(9)]
    for nl, ls, lr in ((2, -4, 0), (3, per_S - 4, 0), (3, 0, base.num_slots - 1), (0, 0, 0)):
        assert L.gdn_kda_exact_fold(ctypes.byref(base), nl, ls, lr, *fold, 1, n) == gv.GDN_EINVAL
    # per slot-record: raw k per qk head, raw v, K fp32 gates and a beta per value head
    sh = gv.GdnShape.from_layer(synth.CONFIGS["qwen3next_b256"])
    rec = 16 * 128 * 2 + 32 * (128 * 2 + 128 * 4 + 4)
    assert gv.gdn_kda_ring_bytes(sh) == 512 * 64 * rec


def test_fold_work_item_count_fits_32_bits():
    # rows x layers x value heads x 16-row tiles is counted in 32-bit ints
    L = gv.lib()
    n = None
    sh = gv.GdnShape.from_layer(synth.CONFIGS["qwen3next_b32"], B=65535, num_slots=65535)
    fold = [ctypes.c_void_p((3 + i) << 20) for i in range(9)]
    for fn in (L.gdn_exact_fold, L.gdn_kda_exact_fold):
        assert fn(ctypes.byref(sh), 2047, 0, 0, *fold, 1, n) == gv.GDN_EUNSUPPORTED
