"""Seeded synthetic workloads for the GDN ring spec-verify path.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic (no gating, no normalisation, no
recurrence): the CPU oracle and the HIP path each compute those themselves
from the identical input bits produced here.

Distributions follow the synthetic Qwen3-Next-shaped GDN layers the method is
quoted on: q, k, v, a, b ~ N(0, 1); A_log = log U[1, 16] and
dt_bias ~ N(0, 0.1) per value head; the fp32 checkpoint S ~ N(0, 0.02)
(standard deviations).  Two stress variants widen what parity can see:
``low_decay`` draws A_log = log U[1e-3, 1e-2] so gates stay near zero and the
ring history dominates the outputs; ``beta_high`` draws b ~ N(4, 1) so that
beta is close to one.

bf16 tensors are carried as ``uint16`` bit patterns (round-to-nearest-even
from fp32), fp32 tensors as ``float32``.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

ACT_F32 = "f32"
ACT_BF16 = "bf16"


@dataclass(frozen=True)
class LayerShape:
    """One GDN layer's verify geometry.

    B rows (sequences) each verify a window of T draft tokens; H qk-heads and
    HV value heads (HV % H == 0, contiguous GQA groups); head dims K and V;
    ring length L (a power of two, L >= 2 * max_spec); num_slots state slots.
    """

    B: int
    T: int
    H: int
    HV: int
    K: int
    V: int
    L: int
    max_spec: int
    num_slots: int
    act: str
    scale: float = 1.0
    softplus_threshold: float = 20.0
    l2norm_eps: float = 1e-6

    def replace(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)

    @property
    def act_bytes(self) -> int:
        return 4 if self.act == ACT_F32 else 2


# The workloads, named by what they are.
CONFIGS = {
    # tiny single layer, fp32 throughout; 5 committed records, 40 steps
    "tiny_f32": LayerShape(B=1, T=4, H=4, HV=8, K=64, V=64, L=16, max_spec=4,
                           num_slots=4, act=ACT_F32),
    # Qwen3-Next-shaped GDN layer, B=32
    "qwen3next_b32": LayerShape(B=32, T=4, H=16, HV=32, K=128, V=128, L=64,
                                max_spec=4, num_slots=64, act=ACT_BF16),
    # bandwidth-bound batch: B=256 over 512 state slots (S is 1.07 GB fp32)
    "qwen3next_b256": LayerShape(B=256, T=4, H=16, HV=32, K=128, V=128, L=64,
                                 max_spec=4, num_slots=512, act=ACT_BF16),
    # long window: T=8 drafts, L=128 ring
    "long_window_t8": LayerShape(B=64, T=8, H=16, HV=32, K=128, V=128, L=128,
                                 max_spec=8, num_slots=128, act=ACT_BF16),
    # one layer of the 48-layer chain
    "layer_chain_b128": LayerShape(B=128, T=4, H=16, HV=32, K=128, V=128, L=64,
                                   max_spec=4, num_slots=256, act=ACT_BF16),
}

VARIANTS = ("base", "low_decay", "beta_high")


def make_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even) and return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def as_act(x: np.ndarray, act: str) -> np.ndarray:
    """Store fp32 draws in the activation dtype (bits for bf16)."""
    if act == ACT_BF16:
        return f32_to_bf16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def act_to_f64(x: np.ndarray, act: str) -> np.ndarray:
    """Exact widening of activation-dtype storage to float64."""
    if act == ACT_BF16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _normal(rng, shape, mean=0.0, std=1.0) -> np.ndarray:
    return rng.normal(mean, std, size=shape).astype(np.float32)


@dataclass
class LayerParams:
    A_log: np.ndarray      # [HV] fp32
    dt_bias: np.ndarray    # [HV] fp32
    S0: np.ndarray         # [num_slots, HV, V, K] fp32


def layer_params(rng, shape: LayerShape, variant: str = "base") -> LayerParams:
    lo, hi = (1e-3, 1e-2) if variant == "low_decay" else (1.0, 16.0)
    A_log = np.log(rng.uniform(lo, hi, size=shape.HV)).astype(np.float32)
    dt_bias = _normal(rng, shape.HV, 0.0, 0.1)
    S0 = _normal(rng, (shape.num_slots, shape.HV, shape.V, shape.K), 0.0, 0.02)
    return LayerParams(A_log=A_log, dt_bias=dt_bias, S0=S0)


@dataclass
class Window:
    """Packed draft-window activations, token index = row * T + t."""

    q: np.ndarray  # [B*T, H, K]
    k: np.ndarray  # [B*T, H, K]
    v: np.ndarray  # [B*T, HV, V]
    a: np.ndarray  # [B*T, HV]
    b: np.ndarray  # [B*T, HV]


def window(rng, shape: LayerShape, variant: str = "base", n_tok: int | None = None) -> Window:
    n = shape.B * shape.T if n_tok is None else n_tok
    bmean = 4.0 if variant == "beta_high" else 0.0
    act = shape.act
    return Window(
        q=as_act(_normal(rng, (n, shape.H, shape.K)), act),
        k=as_act(_normal(rng, (n, shape.H, shape.K)), act),
        v=as_act(_normal(rng, (n, shape.HV, shape.V)), act),
        a=as_act(_normal(rng, (n, shape.HV)), act),
        b=as_act(_normal(rng, (n, shape.HV), bmean), act),
    )


def slot_choice(rng, shape: LayerShape) -> np.ndarray:
    """Distinct slots for the B rows: a random permutation prefix."""
    return rng.permutation(shape.num_slots)[: shape.B].astype(np.int32)


@dataclass
class CursorDraw:
    cache_base: np.ndarray   # [num_slots] int32
    write_pos: np.ndarray    # [num_slots] int32 (committed records to pre-fill)


def random_cursors(rng, shape: LayerShape) -> CursorDraw:
    """Ring start U{0..L-1} and committed length U{0..L-T} per slot."""
    base = rng.integers(0, shape.L, size=shape.num_slots).astype(np.int32)
    wp = rng.integers(0, shape.L - shape.T + 1, size=shape.num_slots).astype(np.int32)
    return CursorDraw(cache_base=base, write_pos=wp)


def history_windows(rng, shape: LayerShape, n_records: int, variant: str = "base") -> list:
    """Raw records for pre-filling rings, one single-token window per record.

    Element r of the list is a Window with B tokens (T=1 per row): the raw
    q/k/v/a/b of committed record r for every row.
    """
    return [window(rng, shape, variant, n_tok=shape.B) for _ in range(n_records)]


def accept_counts(rng, B: int, T: int, steps: int) -> np.ndarray:
    """Accepted-draft counts U{0..T}, [steps, B] int32; never output-dependent."""
    return rng.integers(0, T + 1, size=(steps, B)).astype(np.int32)


def ring_garbage_template(rng, shape: LayerShape, num_layers: int = 1) -> dict:
    """NaN-patterned ring contents: any stray read poisons outputs and any
    stray write shows up in a full-tensor bit compare.

    bf16 NaN payloads are 0x7Fxx with random low bits; fp32 ones 0x7FC0xxxx.
    """
    lead = (num_layers,) if num_layers > 1 else ()
    S, H, HV, L, K, V = shape.num_slots, shape.H, shape.HV, shape.L, shape.K, shape.V

    def nan_bits16(n):
        return (np.uint16(0x7FC0) | rng.integers(1, 0x3F, size=n, dtype=np.uint16)).astype(np.uint16)

    def nan_bits32(n):
        return (np.uint32(0x7FC00000) | rng.integers(1, 0x3FFFFF, size=n, dtype=np.uint32)).astype(np.uint32)

    def act_nan(shp):
        n = int(np.prod(shp))
        if shape.act == ACT_BF16:
            return nan_bits16(n).reshape(shp)
        return nan_bits32(n).view(np.float32).reshape(shp)

    return {
        "rawk": act_nan(lead + (S, H, L, K)),
        "rawv": act_nan(lead + (S, HV, L, V)),
        "g": nan_bits32(int(np.prod(lead + (S, HV, L)))).view(np.float32).reshape(lead + (S, HV, L)),
        "beta": nan_bits32(int(np.prod(lead + (S, HV, L)))).view(np.float32).reshape(lead + (S, HV, L)),
    }


# ------------------------------------------------ KDA (per-channel gate)
#
# The KDA layer's gate input a and bias dt_bias carry one value per key
# channel: a [B*T, HV, K] ~ N(0, 1) and dt_bias [HV, K] ~ N(0, 0.1); A_log stays
# one value per value head.  The ring's gate records hold K fp32 values.


def kda_layer_params(rng, shape: LayerShape, variant: str = "base") -> LayerParams:
    lo, hi = (1e-3, 1e-2) if variant == "low_decay" else (1.0, 16.0)
    A_log = np.log(rng.uniform(lo, hi, size=shape.HV)).astype(np.float32)
    dt_bias = _normal(rng, (shape.HV, shape.K), 0.0, 0.1)
    S0 = _normal(rng, (shape.num_slots, shape.HV, shape.V, shape.K), 0.0, 0.02)
    return LayerParams(A_log=A_log, dt_bias=dt_bias, S0=S0)


def kda_window(rng, shape: LayerShape, variant: str = "base", n_tok: int | None = None) -> Window:
    n = shape.B * shape.T if n_tok is None else n_tok
    bmean = 4.0 if variant == "beta_high" else 0.0
    act = shape.act
    return Window(
        q=as_act(_normal(rng, (n, shape.H, shape.K)), act),
        k=as_act(_normal(rng, (n, shape.H, shape.K)), act),
        v=as_act(_normal(rng, (n, shape.HV, shape.V)), act),
        a=as_act(_normal(rng, (n, shape.HV, shape.K)), act),
        b=as_act(_normal(rng, (n, shape.HV), bmean), act),
    )


def kda_history_windows(rng, shape: LayerShape, n_records: int, variant: str = "base") -> list:
    """Raw KDA records for pre-filling rings, one single-token window each."""
    return [kda_window(rng, shape, variant, n_tok=shape.B) for _ in range(n_records)]


def kda_ring_garbage_template(rng, shape: LayerShape) -> dict:
    """As ring_garbage_template, with K gate values per record."""
    t = ring_garbage_template(rng, shape)
    n = shape.num_slots * shape.HV * shape.L * shape.K
    g = (np.uint32(0x7FC00000) | rng.integers(1, 0x3FFFFF, size=n, dtype=np.uint32)).astype(np.uint32)
    t["g"] = g.view(np.float32).reshape(shape.num_slots, shape.HV, shape.L, shape.K)
    return t


class DeviceWindows:
    """Seeded draft windows drawn on the device, for long runs.

    Same distributions as ``window`` (``beta_high`` moves b's mean to 4), drawn
    by torch's seeded device generator in fp32 and rounded to the activation
    dtype by torch's conversion (round to nearest even).  Host drawing would
    dominate runs of thousands of verifies; the CPU side of a parity check
    reads back the exact bits of the rows it follows (``host_rows``).
    """

    def __init__(self, seed: int, shape: LayerShape, variant: str = "base",
                 device: str = "cuda:0", kda: bool = False):
        import torch

        self.torch = torch
        self.shape = shape
        self.kda = kda          # per-channel gate inputs: a is [n, HV, K]
        self.variant = variant
        self.device = device
        self.gen = torch.Generator(device=device)
        self.gen.manual_seed(seed)
        self.dtype = torch.bfloat16 if shape.act == ACT_BF16 else torch.float32

    def normal(self, size, mean: float = 0.0):
        t = self.torch.randn(size, generator=self.gen, device=self.device,
                             dtype=self.torch.float32)
        if mean:
            t += mean
        return t.to(self.dtype)

    def draw(self, n_tok: int | None = None) -> dict:
        sh = self.shape
        n = sh.B * sh.T if n_tok is None else n_tok
        bmean = 4.0 if self.variant == "beta_high" else 0.0
        return {"q": self.normal((n, sh.H, sh.K)), "k": self.normal((n, sh.H, sh.K)),
                "v": self.normal((n, sh.HV, sh.V)),
                "a": self.normal((n, sh.HV, sh.K) if self.kda else (n, sh.HV)),
                "b": self.normal((n, sh.HV), bmean)}

    def host_rows(self, win: dict, rows, T: int) -> Window:
        """The given rows' tokens as a host ``Window`` (bf16 as uint16 bits)."""
        torch = self.torch
        idx = (np.asarray(rows)[:, None] * T + np.arange(T)[None, :]).reshape(-1)
        sel = torch.from_numpy(idx.astype(np.int64)).to(self.device)
        out = []
        for name in ("q", "k", "v", "a", "b"):
            x = win[name].index_select(0, sel).cpu()
            out.append(x.view(torch.int16).numpy().view(np.uint16) if self.shape.act == ACT_BF16
                       else x.numpy().astype(np.float32))
        return Window(*out)
