"""fp64 CPU oracle for the diagonal affine recurrence scan (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and this package never
imports the product path.

The arithmetic lives in ``oracle.c`` and ``oracle_complex.c`` (plain C,
double precision, one lane at a time; see the headers of those files for the
definitions and where they come from).  This module only compiles it with gcc when the shared object is
missing or older than the source, and marshals numpy float64 arrays.

Definitions (page "triton_training_scan.py", kernels ``_real_forward``,
``_real_backward`` and the ``_real_chunk_*`` / ``_real_reverse_chunk_*``
family):

* forward   ``h_t = a_t h_{t-1} + b_t`` from ``h_{-1} = h0`` (zero by default),
  ``out = h``, ``last = h_{T-1}``;
* backward  ``lambda_t = g_t + a_{t+1} lambda_{t+1}`` seeded with
  ``grad_last``, ``grad_b = lambda``, ``grad_a_t = lambda_t h_{t-1}``,
  ``grad_h0 = a_0 lambda_0``;
* chunk summary ``(P_k, Q_k)``, exclusive prefix ``chunk_in``, replay, and the
  reverse-time trio.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SRC_COMPLEX = os.path.join(_HERE, "oracle_complex.c")
SOURCES = (_SRC, _SRC_COMPLEX)
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-pthread"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp contraction off)."""
    stale = not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(f)
                                             for f in SOURCES)
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, *SOURCES, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_D = ctypes.POINTER(ctypes.c_double)
_U8 = ctypes.POINTER(ctypes.c_uint8)
_I = ctypes.c_int64


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # The mutation tests point this at a deliberately broken copy of
            # oracle.c, compiled elsewhere, to show that the pins catch it.
            override = os.environ.get("ORACLE_LIBRARY_OVERRIDE")
            if override:
                path = override
            else:
                path = build()
            lib = ctypes.CDLL(path)
            sigs = {
                "oracle_scan_fwd": [_I, _I, _I, _D, _D, _D, _U8, _D, _D],
                "oracle_scan_bwd": [_I, _I, _I, _D, _D, _D, _D, _D, _U8, _D, _D, _D],
                "oracle_chunk_summary": [_I, _I, _I, _I, _D, _D, _D, _D],
                "oracle_chunk_prefix": [_I, _I, _I, _D, _D, _D, _D, _D],
                "oracle_chunk_replay": [_I, _I, _I, _I, _D, _D, _D, _D, _D],
                "oracle_reverse_chunk_summary": [_I, _I, _I, _I, _D, _D, _D, _D],
                "oracle_reverse_chunk_prefix": [_I, _I, _I, _D, _D, _D, _D, _D],
                "oracle_reverse_chunk_replay": [_I, _I, _I, _I, _D, _D, _D, _D, _D, _D, _D],
                "oracle_parallel_fwd": [_I, _I, _I, _D, _D, _D, _U8, _D, _D, ctypes.c_int],
                "oracle_parallel_bwd": [_I, _I, _I, _D, _D, _D, _D, _D, _U8, _D, _D, _D,
                                        ctypes.c_int],
                "oracle_complex_fwd": [_I, _I, _I, _D, _D, _D, _D, _D, _D, _U8, _D, _D, _D, _D],
                "oracle_complex_bwd": [_I, _I, _I, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, _U8,
                                       _D, _D, _D, _D, _D, _D],
                "oracle_samu_fwd": [_I, _I, _I] + [_D] * 8 + [_U8] + [_D] * 4,
                "oracle_samu_bwd": [_I, _I, _I] + [_D] * 12 + [_U8] + [_D] * 8,
            }
            for name, args in sigs.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = ctypes.c_int if name.startswith("oracle_parallel") else None
            _lib = lib
    return _lib


def _f64(x, shape=None):
    if x is None:
        return None
    arr = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if shape is not None and arr.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {arr.shape}")
    return arr


def _p(arr):
    if arr is None:
        return None
    return arr.ctypes.data_as(_U8 if arr.dtype == np.uint8 else _D)


def _bdt(a):
    if a.ndim != 3:
        raise ValueError("expected a [B, T, D] array")
    return a.shape


def _mask(reset, B, T):
    """[B, T] segment-start mask as contiguous uint8 (None stays None)."""
    if reset is None:
        return None
    m = np.ascontiguousarray(np.asarray(reset), dtype=np.uint8)
    if m.shape != (B, T):
        raise ValueError(f"reset mask has shape {m.shape}, expected {(B, T)}")
    return m


def scan_fwd(a, b, h0=None, threads: int = 1, reset=None):
    """Forward scan in fp64.  Returns (out [B,T,D], last [B,D]).  ``reset``
    ([B, T], nonzero = a segment starts there) drops the entering state."""
    a = _f64(a)
    B, T, D = _bdt(a)
    b = _f64(b, a.shape)
    h0 = _f64(h0, (B, D))
    rm = _mask(reset, B, T)
    out = np.empty((B, T, D))
    last = np.empty((B, D))
    lib = _load()
    if threads > 1:
        rc = lib.oracle_parallel_fwd(B, T, D, _p(a), _p(b), _p(h0), _p(rm), _p(out), _p(last),
                                     threads)
        if rc != 0:
            raise RuntimeError("oracle thread start failed")
    else:
        lib.oracle_scan_fwd(B, T, D, _p(a), _p(b), _p(h0), _p(rm), _p(out), _p(last))
    return out, last


def scan_bwd(a, h, g, h0=None, grad_last=None, threads: int = 1, reset=None):
    """Backward scan in fp64.  ``h`` are the forward states (of the same
    ``reset`` mask).

    Returns (grad_a, grad_b, grad_h0)."""
    a = _f64(a)
    B, T, D = _bdt(a)
    h = _f64(h, a.shape)
    g = _f64(g, a.shape)
    h0 = _f64(h0, (B, D))
    grad_last = _f64(grad_last, (B, D))
    rm = _mask(reset, B, T)
    grad_a = np.empty((B, T, D))
    grad_b = np.empty((B, T, D))
    grad_h0 = np.empty((B, D))
    lib = _load()
    if threads > 1:
        rc = lib.oracle_parallel_bwd(B, T, D, _p(a), _p(h), _p(g), _p(h0), _p(grad_last),
                                     _p(rm), _p(grad_a), _p(grad_b), _p(grad_h0), threads)
        if rc != 0:
            raise RuntimeError("oracle thread start failed")
    else:
        lib.oracle_scan_bwd(B, T, D, _p(a), _p(h), _p(g), _p(h0), _p(grad_last), _p(rm),
                            _p(grad_a), _p(grad_b), _p(grad_h0))
    return grad_a, grad_b, grad_h0


def n_chunks(T: int, C: int) -> int:
    return (T + C - 1) // C


def chunk_summary(a, b, C: int):
    """Per-chunk affine maps (P, Q), each [B, NC, D]."""
    a = _f64(a)
    B, T, D = _bdt(a)
    b = _f64(b, a.shape)
    NC = n_chunks(T, C)
    P = np.empty((B, NC, D))
    Q = np.empty((B, NC, D))
    _load().oracle_chunk_summary(B, T, D, C, _p(a), _p(b), _p(P), _p(Q))
    return P, Q


def chunk_prefix(P, Q, h0=None):
    """Exclusive forward prefix over chunk maps.  Returns (chunk_in, last)."""
    P = _f64(P)
    B, NC, D = _bdt(P)
    Q = _f64(Q, P.shape)
    h0 = _f64(h0, (B, D))
    chunk_in = np.empty((B, NC, D))
    last = np.empty((B, D))
    _load().oracle_chunk_prefix(B, NC, D, _p(P), _p(Q), _p(h0), _p(chunk_in), _p(last))
    return chunk_in, last


def chunk_replay(a, b, chunk_in, C: int):
    """Replay every chunk from its entering state.  Returns (out, last)."""
    a = _f64(a)
    B, T, D = _bdt(a)
    b = _f64(b, a.shape)
    chunk_in = _f64(chunk_in, (B, n_chunks(T, C), D))
    out = np.empty((B, T, D))
    last = np.empty((B, D))
    _load().oracle_chunk_replay(B, T, D, C, _p(a), _p(b), _p(chunk_in), _p(out), _p(last))
    return out, last


def reverse_chunk_summary(a, g, C: int):
    """Per-chunk reverse adjoint maps (P, Q), each [B, NC, D]."""
    a = _f64(a)
    B, T, D = _bdt(a)
    g = _f64(g, a.shape)
    NC = n_chunks(T, C)
    P = np.empty((B, NC, D))
    Q = np.empty((B, NC, D))
    _load().oracle_reverse_chunk_summary(B, T, D, C, _p(a), _p(g), _p(P), _p(Q))
    return P, Q


def reverse_chunk_prefix(P, Q, grad_last=None):
    """Exclusive right-to-left prefix.  Returns (future, grad_h0)."""
    P = _f64(P)
    B, NC, D = _bdt(P)
    Q = _f64(Q, P.shape)
    grad_last = _f64(grad_last, (B, D))
    future = np.empty((B, NC, D))
    grad_h0 = np.empty((B, D))
    _load().oracle_reverse_chunk_prefix(B, NC, D, _p(P), _p(Q), _p(grad_last), _p(future),
                                        _p(grad_h0))
    return future, grad_h0


def reverse_chunk_replay(a, h, g, future, C: int, h0=None):
    """Replay every chunk backwards from its future carry.  Returns (grad_a, grad_b)."""
    a = _f64(a)
    B, T, D = _bdt(a)
    h = _f64(h, a.shape)
    g = _f64(g, a.shape)
    future = _f64(future, (B, n_chunks(T, C), D))
    h0 = _f64(h0, (B, D))
    grad_a = np.empty((B, T, D))
    grad_b = np.empty((B, T, D))
    _load().oracle_reverse_chunk_replay(B, T, D, C, _p(a), _p(h), _p(g), _p(future), _p(h0),
                                        _p(grad_a), _p(grad_b))
    return grad_a, grad_b


# ----------------------------------------------------------------------------
# complex diagonal scan (planar storage in the C oracle; complex128 here)
# ----------------------------------------------------------------------------
def _planar(z, shape):
    """(real, imag) contiguous float64 arrays of a complex array (None -> None)."""
    if z is None:
        return None, None
    z = np.asarray(z)
    if tuple(z.shape) != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {z.shape}")
    return (np.ascontiguousarray(z.real, dtype=np.float64),
            np.ascontiguousarray(z.imag, dtype=np.float64))


def complex_fwd(a, b, h0=None, reset=None):
    """Complex scan h_t = a_t h_{t-1} + b_t in fp64.  a, b: complex [B, T, M];
    h0: complex [B, M] or None; reset: [B, T] mask or None.
    Returns (out [B, T, M], last [B, M]) as complex128."""
    a = np.asarray(a)
    if a.ndim != 3:
        raise ValueError("expected a [B, T, M] array")
    B, T, M = a.shape
    ar, ai = _planar(a, (B, T, M))
    br, bi = _planar(b, (B, T, M))
    h0r, h0i = _planar(h0, (B, M))
    rm = _mask(reset, B, T)
    out_r, out_i = np.empty((B, T, M)), np.empty((B, T, M))
    last_r, last_i = np.empty((B, M)), np.empty((B, M))
    _load().oracle_complex_fwd(B, T, M, _p(ar), _p(ai), _p(br), _p(bi), _p(h0r), _p(h0i), _p(rm),
                               _p(out_r), _p(out_i), _p(last_r), _p(last_i))
    return out_r + 1j * out_i, last_r + 1j * last_i


def complex_bwd(a, h, g, h0=None, grad_last=None, reset=None):
    """Adjoint of the complex scan for L = sum Re(conj(g) h) + Re(conj(grad_last) h_{T-1}):
    gradients as dL/dRe + i dL/dIm.  Returns (grad_a, grad_b, grad_h0) complex128."""
    a = np.asarray(a)
    B, T, M = a.shape
    ar, ai = _planar(a, (B, T, M))
    hr, hi = _planar(h, (B, T, M))
    gr, gi = _planar(g, (B, T, M))
    h0r, h0i = _planar(h0, (B, M))
    glr, gli = _planar(grad_last, (B, M))
    rm = _mask(reset, B, T)
    gar, gai, gbr, gbi = (np.empty((B, T, M)) for _ in range(4))
    gh0r, gh0i = np.empty((B, M)), np.empty((B, M))
    _load().oracle_complex_bwd(B, T, M, _p(ar), _p(ai), _p(hr), _p(hi), _p(gr), _p(gi), _p(h0r),
                               _p(h0i), _p(glr), _p(gli), _p(rm), _p(gar), _p(gai), _p(gbr),
                               _p(gbi), _p(gh0r), _p(gh0i))
    return gar + 1j * gai, gbr + 1j * gbi, gh0r + 1j * gh0i


# ----------------------------------------------------------------------------
# fused-transition (SAMU-form) complex scan
# ----------------------------------------------------------------------------
def _f64v(x, shape):
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {x.shape}")
    return x


def samu_fwd(eta, delta, nu_log, theta_log, b, h0=None, reset=None):
    """Scan with transitions rebuilt from controls: eta, delta [B, T];
    nu_log, theta_log [M]; b complex [B, T, M].  Returns (out, last) complex."""
    b = np.asarray(b)
    B, T, M = b.shape
    e, dl = _f64v(eta, (B, T)), _f64v(delta, (B, T))
    nl, tl = _f64v(nu_log, (M,)), _f64v(theta_log, (M,))
    br, bi = _planar(b, (B, T, M))
    h0r, h0i = _planar(h0, (B, M))
    rm = _mask(reset, B, T)
    out_r, out_i = np.empty((B, T, M)), np.empty((B, T, M))
    last_r, last_i = np.empty((B, M)), np.empty((B, M))
    _load().oracle_samu_fwd(B, T, M, _p(e), _p(dl), _p(nl), _p(tl), _p(br), _p(bi), _p(h0r),
                            _p(h0i), _p(rm), _p(out_r), _p(out_i), _p(last_r), _p(last_i))
    return out_r + 1j * out_i, last_r + 1j * last_i


def samu_bwd(eta, delta, nu_log, theta_log, h, g, h0=None, grad_last=None, reset=None):
    """Gradients of L = sum Re(conj(g) h) + Re(conj(grad_last) h_{T-1}).
    Returns (grad_eta [B,T], grad_delta [B,T], grad_nu_log [M],
    grad_theta_log [M], grad_b complex [B,T,M], grad_h0 complex [B,M])."""
    h = np.asarray(h)
    B, T, M = h.shape
    e, dl = _f64v(eta, (B, T)), _f64v(delta, (B, T))
    nl, tl = _f64v(nu_log, (M,)), _f64v(theta_log, (M,))
    hr, hi = _planar(h, (B, T, M))
    gr, gi = _planar(g, (B, T, M))
    h0r, h0i = _planar(h0, (B, M))
    glr, gli = _planar(grad_last, (B, M))
    rm = _mask(reset, B, T)
    ge, gd = np.empty((B, T)), np.empty((B, T))
    gn, gt = np.empty(M), np.empty(M)
    gbr, gbi = np.empty((B, T, M)), np.empty((B, T, M))
    gh0r, gh0i = np.empty((B, M)), np.empty((B, M))
    _load().oracle_samu_bwd(B, T, M, _p(e), _p(dl), _p(nl), _p(tl), _p(hr), _p(hi), _p(gr),
                            _p(gi), _p(h0r), _p(h0i), _p(glr), _p(gli), _p(rm), _p(ge), _p(gd),
                            _p(gn), _p(gt), _p(gbr), _p(gbi), _p(gh0r), _p(gh0i))
    return ge, gd, gn, gt, gbr + 1j * gbi, gh0r + 1j * gh0i
