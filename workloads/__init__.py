"""Seeded synthetic inputs for the diagonal affine scan workloads.

This module holds no arithmetic of the scan itself: it only draws random
tensors and stores them in the I/O format (float32, or bfloat16 bit patterns
rounded to nearest-even).  Both the oracle side (tests, CPU baseline) and the
GPU side (tests, bench, smoke) take their inputs from here, so both see the
same bits.

Recipes (one per workload; the five named workloads below are the shapes the
scan is specified on, with the value distributions stated for each):

* ``small``   B=2  T=256    D=64   fp32  a~U(0.9,0.999)   b=N(0,1)*sqrt(1-a^2)
* ``wide``    B=8  T=2048   D=2560 bf16  a=clip(sigmoid(N(4,1)),0.8,0.9999)
                                         b=N(0,1)*sqrt(1-a^2)
* ``long32``  B=4  T=8192   D=4096 fp32  a~U(0.95,0.9999)  b~N(0,1)
* ``longseq`` B=1  T=131072 D=1024 bf16  a~U(0.99,0.99999) b~N(0, sd 0.1)
* ``masked``  B=16 T=4096   D=2560 bf16  a~U(0.5,0.9999); per token (b,t)
              10% padding steps (a=1, b=0, g=0) and 5% reset steps (a=0);
              b=N(0,1)*sqrt(1-a^2) using the final a.

In every recipe grad_out ~ N(0,1) (zero at padding tokens), the draws are
i.i.d. per element, numpy ``default_rng(seed)`` (PCG64) is used in float64 in
the order a, masks, b, grad_out, and the values are then cast to float32 and,
for bf16 workloads, rounded to bfloat16 (nearest-even).  The draws are made
one batch row at a time (a, masks, b, grad_out for row 0, then row 1, ...),
which bounds host memory; that row order is part of the recipe.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    D: int
    dtype: str  # "f32" or "bf16"
    recipe: str  # key into _RECIPES
    chunk: int = 0  # chunk length the workload is specified with (0: unspecified)

    @property
    def N(self) -> int:
        return self.B * self.T * self.D

    @property
    def itemsize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_shape(self, B=None, T=None, D=None, name=None) -> "Workload":
        return dataclasses.replace(self, B=B or self.B, T=T or self.T, D=D or self.D,
                                   name=name or self.name)


WORKLOADS = {
    "small": Workload("small", 2, 256, 64, "f32", "small", 64),
    "wide": Workload("wide", 8, 2048, 2560, "bf16", "wide"),
    "long32": Workload("long32", 4, 8192, 4096, "f32", "long32", 64),
    "longseq": Workload("longseq", 1, 131072, 1024, "bf16", "longseq", 64),
    "masked": Workload("masked", 16, 4096, 2560, "bf16", "masked"),
}


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    NaN inputs map to a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    r = np.where(nan, ((u >> np.uint64(16)).astype(np.uint32) | np.uint32(0x40)), r)
    return (r & np.uint32(0xFFFF)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 draw -> stored I/O representation (float32, or uint16 bf16 bits)."""
    x32 = x64.astype(np.float32)
    return x32 if dtype == "f32" else f32_to_bf16_bits(x32)


def storage_to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored representation -> the exact values it holds, in float64."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    return bf16_bits_to_f32(x).astype(np.float64)


# ----------------------------------------------------------------------------
# recipes: each returns float64 (a, b, g) for one batch row of shape [T, D]
# ----------------------------------------------------------------------------
def _row_small(rng, T, D):
    a = rng.uniform(0.9, 0.999, size=(T, D))
    b = rng.standard_normal((T, D)) * np.sqrt(1.0 - a * a)
    g = rng.standard_normal((T, D))
    return a, b, g


def _row_wide(rng, T, D):
    z = rng.normal(4.0, 1.0, size=(T, D))
    a = np.clip(1.0 / (1.0 + np.exp(-z)), 0.8, 0.9999)
    b = rng.standard_normal((T, D)) * np.sqrt(1.0 - a * a)
    g = rng.standard_normal((T, D))
    return a, b, g


def _row_long32(rng, T, D):
    a = rng.uniform(0.95, 0.9999, size=(T, D))
    b = rng.standard_normal((T, D))
    g = rng.standard_normal((T, D))
    return a, b, g


def _row_longseq(rng, T, D):
    a = rng.uniform(0.99, 0.99999, size=(T, D))
    b = rng.normal(0.0, 0.1, size=(T, D))
    g = rng.standard_normal((T, D))
    return a, b, g


PAD_FRACTION = 0.10
RESET_FRACTION = 0.05


def _row_masked(rng, T, D):
    a = rng.uniform(0.5, 0.9999, size=(T, D))
    # token masks, per (b, t) across all D: padding with p=0.10, then resets
    # among the non-padding tokens so that 5% of all tokens are resets.
    pad = rng.random(T) < PAD_FRACTION
    reset = (rng.random(T) < RESET_FRACTION / (1.0 - PAD_FRACTION)) & ~pad
    a[pad, :] = 1.0
    a[reset, :] = 0.0
    b = rng.standard_normal((T, D)) * np.sqrt(1.0 - a * a)
    b[pad, :] = 0.0
    g = rng.standard_normal((T, D))
    g[pad, :] = 0.0
    return a, b, g, pad, reset


_RECIPES = {
    "small": _row_small,
    "wide": _row_wide,
    "long32": _row_long32,
    "longseq": _row_longseq,
    "masked": _row_masked,
}


@dataclasses.dataclass
class Inputs:
    """Stored inputs of one workload: float32 arrays, or uint16 bf16 bit arrays."""
    workload: Workload
    a: np.ndarray
    b: np.ndarray
    g: np.ndarray
    pad: Optional[np.ndarray] = None  # [B, T] bool (masked workload only)
    reset: Optional[np.ndarray] = None

    def f64(self, name: str, lanes=None) -> np.ndarray:
        """Exact stored values as float64, optionally restricted to lanes.

        ``lanes`` is a list of (b, d) pairs; the result is then [1, T, len]."""
        x = getattr(self, name)
        if lanes is not None:
            bs = np.array([l[0] for l in lanes])
            ds = np.array([l[1] for l in lanes])
            x = x[bs, :, ds].T[None]  # [1, T, L]
        return storage_to_f64(x, self.workload.dtype)


def generate(wl: Workload, seed: int = 0, need_grad: bool = True) -> Inputs:
    """Draw the stored inputs of ``wl`` (row by row over the batch)."""
    recipe = _RECIPES[wl.recipe]
    st = np.float32 if wl.dtype == "f32" else np.uint16
    a = np.empty((wl.B, wl.T, wl.D), st)
    b = np.empty_like(a)
    g = np.empty_like(a) if need_grad else None
    pad = reset = None
    if wl.recipe == "masked":
        pad = np.zeros((wl.B, wl.T), bool)
        reset = np.zeros((wl.B, wl.T), bool)
    rng = np.random.default_rng(seed)
    for bi in range(wl.B):
        res = recipe(rng, wl.T, wl.D)
        a[bi] = to_storage(res[0], wl.dtype)
        b[bi] = to_storage(res[1], wl.dtype)
        if need_grad:
            g[bi] = to_storage(res[2], wl.dtype)
        if pad is not None:
            pad[bi], reset[bi] = res[3], res[4]
    return Inputs(wl, a, b, g, pad, reset)


def sample_lanes(wl: Workload, count: int, seed: int = 1):
    """A reproducible set of distinct (b, d) lanes, always including the corners."""
    rng = np.random.default_rng(seed)
    lanes = {(0, 0), (wl.B - 1, wl.D - 1), (0, wl.D - 1), (wl.B - 1, 0)}
    total = wl.B * wl.D
    while len(lanes) < min(count, total):
        k = int(rng.integers(total))
        lanes.add((k // wl.D, k % wl.D))
    return sorted(lanes)


def random_inputs(B: int, T: int, D: int, dtype: str, seed: int = 0, a_lo: float = 0.5,
                  a_hi: float = 1.0, with_state: bool = False):
    """Ad-hoc inputs for edge shapes: a ~ U(a_lo, a_hi), b, g ~ N(0,1), and
    (optionally) h0, grad_last ~ N(0,1) as float32 [B, D].  Drawn in float64 in
    the order a, b, g, h0, grad_last, then stored like the named workloads."""
    rng = np.random.default_rng(seed)
    a = rng.uniform(a_lo, a_hi, size=(B, T, D))
    b = rng.standard_normal((B, T, D))
    g = rng.standard_normal((B, T, D))
    wl = Workload(f"random_B{B}_T{T}_D{D}_{dtype}", B, T, D, dtype, "random")
    inp = Inputs(wl, to_storage(a, dtype), to_storage(b, dtype), to_storage(g, dtype))
    if with_state:
        h0 = rng.standard_normal((B, D)).astype(np.float32)
        gl = rng.standard_normal((B, D)).astype(np.float32)
        return inp, h0, gl
    return inp


# ----------------------------------------------------------------------------
# complex workloads (planar storage: separate real / imaginary arrays)
# ----------------------------------------------------------------------------
# ``cwide``  B=8 T=2048 M=2560 bf16: the wide workload with complex values.
#            a = r e^{i theta}, r = clip(sigmoid(N(4,1)), 0.8, 0.9999),
#            theta ~ U(-pi/8, pi/8); b = (N(0,1) + i N(0,1)) sqrt((1-r^2)/2);
#            grad_out = N(0,1) + i N(0,1).  Drawn one batch row at a time in
#            the order r, theta, b (re, im), grad_out (re, im).
COMPLEX_WORKLOADS = {
    "cwide": Workload("cwide", 8, 2048, 2560, "bf16", "cwide"),
    "csmall": Workload("csmall", 2, 256, 64, "f32", "cwide"),
}


@dataclasses.dataclass
class ComplexInputs:
    """Stored planar inputs: float32 arrays, or uint16 bf16 bit arrays."""
    workload: Workload
    ar: np.ndarray
    ai: np.ndarray
    br: np.ndarray
    bi: np.ndarray
    gr: np.ndarray
    gi: np.ndarray

    def c128(self, name: str, lanes=None) -> np.ndarray:
        """Exact stored values of "a", "b" or "g" as complex128 (optionally
        restricted to a list of (b, m) lanes: [1, T, len])."""
        re, im = getattr(self, name + "r"), getattr(self, name + "i")
        if lanes is not None:
            bs = np.array([l[0] for l in lanes])
            ms = np.array([l[1] for l in lanes])
            re, im = re[bs, :, ms].T[None], im[bs, :, ms].T[None]
        dt = self.workload.dtype
        return storage_to_f64(re, dt) + 1j * storage_to_f64(im, dt)


def complex_inputs(B: int, T: int, M: int, dtype: str, seed: int = 0, r_lo: float = 0.8,
                   r_hi: float = 0.9999, theta: float = np.pi / 8,
                   name: str = "complex") -> ComplexInputs:
    """Complex planar inputs with the cwide recipe (|a| = r clipped to
    [r_lo, r_hi] from sigmoid(N(4,1)), phase ~ U(-theta, theta))."""
    st = np.float32 if dtype == "f32" else np.uint16
    arrs = [np.empty((B, T, M), st) for _ in range(6)]
    rng = np.random.default_rng(seed)
    for bi in range(B):
        z = rng.normal(4.0, 1.0, size=(T, M))
        r = np.clip(1.0 / (1.0 + np.exp(-z)), r_lo, r_hi)
        th = rng.uniform(-theta, theta, size=(T, M))
        scale = np.sqrt((1.0 - r * r) / 2.0)
        b_re = rng.standard_normal((T, M)) * scale
        b_im = rng.standard_normal((T, M)) * scale
        g_re = rng.standard_normal((T, M))
        g_im = rng.standard_normal((T, M))
        vals = (r * np.cos(th), r * np.sin(th), b_re, b_im, g_re, g_im)
        for dst, v in zip(arrs, vals):
            dst[bi] = to_storage(v, dtype)
    wl = Workload(name, B, T, M, dtype, "cwide")
    return ComplexInputs(wl, *arrs)


def generate_complex(wl: Workload, seed: int = 0) -> ComplexInputs:
    return complex_inputs(wl.B, wl.T, wl.D, wl.dtype, seed, name=wl.name)


# ----------------------------------------------------------------------------
# fused-transition (SAMU-form) workloads: the transition is not stored; it is
# rebuilt from per-token controls eta, delta [B, T] (I/O type) and per-mode
# parameters nu_log, theta_log [M] (float32).
# ----------------------------------------------------------------------------
# ``swide``  B=8 T=2048 M=2560 bf16: the wide shape with rebuilt transitions.
#            Per mode (drawn first, in this order): nu = U(0.005, 0.5),
#            theta = U(0.001, pi), stored as nu_log = ln nu, theta_log =
#            ln theta.  Then per batch row: eta ~ N(0, 0.5^2),
#            delta ~ N(0, 0.1^2) per token, b = 0.3 (N(0,1) + i N(0,1)),
#            grad_out = N(0,1) + i N(0,1).  The decay exp(-nu e^eta) then
#            spans about 0.25 .. 0.998.
SAMU_WORKLOADS = {
    "swide": Workload("swide", 8, 2048, 2560, "bf16", "swide"),
    "ssmall": Workload("ssmall", 2, 256, 64, "f32", "swide"),
}


@dataclasses.dataclass
class SamuInputs:
    """Stored inputs: eta, delta [B, T] and planar b, grad_out [B, T, M] in the
    I/O format (float32 or bf16 bits); nu_log, theta_log float32 [M]."""
    workload: Workload
    eta: np.ndarray
    delta: np.ndarray
    nu_log: np.ndarray
    theta_log: np.ndarray
    br: np.ndarray
    bi: np.ndarray
    gr: np.ndarray
    gi: np.ndarray

    def controls(self, rows=None):
        """Exact stored (eta, delta, nu_log, theta_log) as float64 (eta and
        delta optionally restricted to a list of batch rows)."""
        dt = self.workload.dtype
        e, d = self.eta, self.delta
        if rows is not None:
            e, d = e[rows], d[rows]
        return (storage_to_f64(e, dt), storage_to_f64(d, dt),
                self.nu_log.astype(np.float64), self.theta_log.astype(np.float64))

    def c128(self, name: str, rows=None) -> np.ndarray:
        """Exact stored "b" or "g" as complex128 (optionally only some batch rows)."""
        re, im = getattr(self, name + "r"), getattr(self, name + "i")
        if rows is not None:
            re, im = re[rows], im[rows]
        dt = self.workload.dtype
        return storage_to_f64(re, dt) + 1j * storage_to_f64(im, dt)


def samu_inputs(B: int, T: int, M: int, dtype: str, seed: int = 0, nu_hi: float = 0.5,
                eta_sd: float = 0.5, name: str = "samu") -> SamuInputs:
    """Inputs with the swide recipe (``nu_hi`` and ``eta_sd`` adjustable)."""
    st = np.float32 if dtype == "f32" else np.uint16
    rng = np.random.default_rng(seed)
    nu = rng.uniform(0.005, nu_hi, size=M)
    theta = rng.uniform(0.001, np.pi, size=M)
    eta = np.empty((B, T), st)
    delta = np.empty((B, T), st)
    arrs = [np.empty((B, T, M), st) for _ in range(4)]
    for bi in range(B):
        eta[bi] = to_storage(rng.normal(0.0, eta_sd, size=T), dtype)
        delta[bi] = to_storage(rng.normal(0.0, 0.1, size=T), dtype)
        vals = (0.3 * rng.standard_normal((T, M)), 0.3 * rng.standard_normal((T, M)),
                rng.standard_normal((T, M)), rng.standard_normal((T, M)))
        for dst, v in zip(arrs, vals):
            dst[bi] = to_storage(v, dtype)
    wl = Workload(name, B, T, M, dtype, "swide")
    return SamuInputs(wl, eta, delta, np.log(nu).astype(np.float32),
                      np.log(theta).astype(np.float32), *arrs)


def generate_samu(wl: Workload, seed: int = 0) -> SamuInputs:
    return samu_inputs(wl.B, wl.T, wl.D, wl.dtype, seed, name=wl.name)
