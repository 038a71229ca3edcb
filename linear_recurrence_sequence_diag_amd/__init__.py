"""Diagonal affine recurrence scan on MI355X (gfx950): Python binding of liblrscan.

The scan ``h_t = a_t * h_{t-1} + b_t`` over [B, T, D] tensors and its
reverse-time adjoint run entirely in the HIP kernels of ``liblrscan.so``
(built from ``csrc/`` by ``build.py``).  This module only marshals arguments:
the raw entry points keep the C names of ``include/lrscan.h`` and take device
pointers; the tensor helpers below allocate outputs with torch (device memory
and the current stream are all torch is used for) and call them.

There is no fallback: if the library is not built, or no GPU is present, the
calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblrscan.so")

F32, BF16 = 0, 1
ALGO_AUTO, ALGO_SEQ, ALGO_CHUNKED, ALGO_FUSED = 0, 1, 2, 3
ALGOS = {"auto": ALGO_AUTO, "seq": ALGO_SEQ, "chunked": ALGO_CHUNKED, "fused": ALGO_FUSED}

STATUS = {
    0: "LRSCAN_OK", -1: "LRSCAN_ERR_NULL", -2: "LRSCAN_ERR_DIM", -3: "LRSCAN_ERR_DTYPE",
    -4: "LRSCAN_ERR_CHUNK", -5: "LRSCAN_ERR_WORKSPACE", -6: "LRSCAN_ERR_HIP", -7: "LRSCAN_ERR_ALGO",
    -8: "LRSCAN_ERR_CAPTURE", -9: "LRSCAN_ERR_TOO_BIG",
}


class LRScanError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


class Opts(ctypes.Structure):
    """Mirror of ``lrscan_opts``."""
    _fields_ = [
        ("algo", ctypes.c_int),
        ("chunk", ctypes.c_int),
        ("width", ctypes.c_int),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("h0", ctypes.c_void_p),
        ("grad_h0", ctypes.c_void_p),
        ("polls", ctypes.c_int),
        ("reset", ctypes.c_void_p),
    ]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SIGS = {
    "scan_fwd": ([_P, _P, _P, _P, _I64, _I64, _I64, _INT, _P], _INT),
    "scan_bwd": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _P], _INT),
    "scan_fwd_ex": ([_P, _P, _P, _P, _I64, _I64, _I64, _INT, _P, ctypes.POINTER(Opts)], _INT),
    "scan_bwd_ex": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _P, ctypes.POINTER(Opts)], _INT),
    "scan_fwd_noalloc": ([_P, _P, _P, _P, _I64, _I64, _I64, _INT, _P, ctypes.POINTER(Opts)], _INT),
    "scan_workspace_bytes": ([_I64, _I64, _I64, _INT, ctypes.POINTER(Opts)], ctypes.c_size_t),
    "scan_status_string": ([_INT], ctypes.c_char_p),
    "scan_step": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _INT, _P], _INT),
    "scan_complex_fwd": ([_P] * 10 + [_I64, _I64, _I64, _INT, _P, ctypes.POINTER(Opts)], _INT),
    "scan_complex_bwd": ([_P] * 16 + [_I64, _I64, _I64, _INT, _P, ctypes.POINTER(Opts)], _INT),
    "scan_samu_fwd": ([_P] * 12 + [_I64, _I64, _I64, _INT, _P, ctypes.POINTER(Opts)], _INT),
    "scan_samu_bwd": ([_P] * 20 + [_I64, _I64, _I64, _INT, _P, ctypes.POINTER(Opts)], _INT),
    "scan_samu_workspace_bytes": ([_I64, _I64, _I64, _INT, ctypes.POINTER(Opts)],
                                  ctypes.c_size_t),
    "scan_complex_workspace_bytes": ([_I64, _I64, _I64, _INT, ctypes.POINTER(Opts)],
                                     ctypes.c_size_t),
    "scan_auto_algo": ([_I64, _I64, _I64, _INT, _INT, ctypes.POINTER(_INT), ctypes.POINTER(_INT)],
                       _INT),
    "scan_chunk_summary": ([_P, _P, _P, _P, _I64, _I64, _I64, _INT, _INT, _P], _INT),
    "scan_chunk_prefix": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P], _INT),
    "scan_chunk_replay": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _INT, _P], _INT),
    "scan_reverse_chunk_summary": ([_P, _P, _P, _P, _I64, _I64, _I64, _INT, _INT, _P], _INT),
    "scan_reverse_chunk_prefix": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P], _INT),
    "scan_reverse_chunk_replay": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _INT, _P], _INT),
}

_lock = threading.Lock()
_lib = None


def library():
    """The loaded liblrscan (ctypes.CDLL).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is not built; run `python -m linear_recurrence_sequence_diag_amd.build`")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in _SIGS.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = res
            _lib = lib
    return _lib


def _check(status: int, what: str) -> int:
    if status < 0 and what != "scan_auto_algo":
        raise LRScanError(status, what)
    return status


def scan_status_string(status: int) -> str:
    return library().scan_status_string(status).decode()


status_string = scan_status_string


# ---------------------------------------------------------------------------
# raw entry points: same names and arguments as the C ABI (device pointers as
# ints, a stream handle as an int); negative status codes raise LRScanError
# ---------------------------------------------------------------------------
def scan_fwd(a, b, out, last, B, T, D, dtype, stream):
    return _check(library().scan_fwd(a, b, out, last, B, T, D, dtype, stream), "scan_fwd")


def scan_bwd(a, out, grad_out, grad_last, grad_a, grad_b, B, T, D, dtype, stream):
    return _check(library().scan_bwd(a, out, grad_out, grad_last, grad_a, grad_b, B, T, D, dtype,
                                     stream), "scan_bwd")


def scan_fwd_ex(a, b, out, last, B, T, D, dtype, stream, opts):
    return _check(library().scan_fwd_ex(a, b, out, last, B, T, D, dtype, stream,
                                        ctypes.byref(opts) if opts is not None else None),
                  "scan_fwd_ex")


def scan_bwd_ex(a, out, grad_out, grad_last, grad_a, grad_b, B, T, D, dtype, stream, opts):
    return _check(library().scan_bwd_ex(a, out, grad_out, grad_last, grad_a, grad_b, B, T, D, dtype,
                                        stream, ctypes.byref(opts) if opts is not None else None),
                  "scan_bwd_ex")


def scan_fwd_noalloc(a, b, out, last, B, T, D, dtype, stream, opts):
    return _check(library().scan_fwd_noalloc(a, b, out, last, B, T, D, dtype, stream,
                                             ctypes.byref(opts) if opts is not None else None),
                  "scan_fwd_noalloc")


def scan_step(a, b, state_in, reset, out, state_out, B, D, dtype, stream):
    return _check(library().scan_step(a, b, state_in, reset, out, state_out, B, D, dtype, stream),
                  "scan_step")


def scan_complex_fwd(ar, ai, br, bi, out_r, out_i, last_r, last_i, h0_r, h0_i, B, T, M, dtype,
                     stream, opts):
    return _check(library().scan_complex_fwd(ar, ai, br, bi, out_r, out_i, last_r, last_i, h0_r,
                                             h0_i, B, T, M, dtype, stream,
                                             ctypes.byref(opts) if opts is not None else None),
                  "scan_complex_fwd")


def scan_complex_bwd(ar, ai, out_r, out_i, grad_out_r, grad_out_i, grad_last_r, grad_last_i, h0_r,
                     h0_i, grad_ar, grad_ai, grad_br, grad_bi, grad_h0_r, grad_h0_i, B, T, M,
                     dtype, stream, opts):
    return _check(library().scan_complex_bwd(ar, ai, out_r, out_i, grad_out_r, grad_out_i,
                                             grad_last_r, grad_last_i, h0_r, h0_i, grad_ar,
                                             grad_ai, grad_br, grad_bi, grad_h0_r, grad_h0_i, B,
                                             T, M, dtype, stream,
                                             ctypes.byref(opts) if opts is not None else None),
                  "scan_complex_bwd")


def scan_complex_workspace_bytes(B, T, M, dtype, opts=None):
    return library().scan_complex_workspace_bytes(B, T, M, dtype,
                                                  ctypes.byref(opts) if opts is not None else None)


def scan_samu_fwd(eta, delta, nu_log, theta_log, br, bi, out_r, out_i, last_r, last_i, h0_r, h0_i,
                  B, T, M, dtype, stream, opts):
    return _check(library().scan_samu_fwd(eta, delta, nu_log, theta_log, br, bi, out_r, out_i,
                                          last_r, last_i, h0_r, h0_i, B, T, M, dtype, stream,
                                          ctypes.byref(opts) if opts is not None else None),
                  "scan_samu_fwd")


def scan_samu_bwd(eta, delta, nu_log, theta_log, out_r, out_i, grad_out_r, grad_out_i,
                  grad_last_r, grad_last_i, h0_r, h0_i, grad_eta, grad_delta, grad_nu_log,
                  grad_theta_log, grad_br, grad_bi, grad_h0_r, grad_h0_i, B, T, M, dtype, stream,
                  opts):
    return _check(library().scan_samu_bwd(eta, delta, nu_log, theta_log, out_r, out_i,
                                          grad_out_r, grad_out_i, grad_last_r, grad_last_i, h0_r,
                                          h0_i, grad_eta, grad_delta, grad_nu_log,
                                          grad_theta_log, grad_br, grad_bi, grad_h0_r, grad_h0_i,
                                          B, T, M, dtype, stream,
                                          ctypes.byref(opts) if opts is not None else None),
                  "scan_samu_bwd")


def scan_samu_workspace_bytes(B, T, M, dtype, opts=None):
    return library().scan_samu_workspace_bytes(B, T, M, dtype,
                                               ctypes.byref(opts) if opts is not None else None)


def scan_workspace_bytes(B, T, D, dtype, opts=None):
    return library().scan_workspace_bytes(B, T, D, dtype,
                                          ctypes.byref(opts) if opts is not None else None)


def scan_auto_algo(B, T, D, dtype, direction):
    """(algo, chunk, width) the library picks for this shape."""
    chunk = ctypes.c_int(0)
    width = ctypes.c_int(0)
    algo = library().scan_auto_algo(B, T, D, dtype, direction, ctypes.byref(chunk),
                                    ctypes.byref(width))
    if algo < 0:
        raise LRScanError(algo, "scan_auto_algo")
    return algo, chunk.value, width.value


def scan_chunk_summary(a, b, P, Q, B, T, D, chunk, dtype, stream):
    return _check(library().scan_chunk_summary(a, b, P, Q, B, T, D, chunk, dtype, stream),
                  "scan_chunk_summary")


def scan_chunk_prefix(P, Q, h0, chunk_in, last, B, NC, D, stream):
    return _check(library().scan_chunk_prefix(P, Q, h0, chunk_in, last, B, NC, D, stream),
                  "scan_chunk_prefix")


def scan_chunk_replay(a, b, chunk_in, out, last, B, T, D, chunk, dtype, stream):
    return _check(library().scan_chunk_replay(a, b, chunk_in, out, last, B, T, D, chunk, dtype,
                                              stream), "scan_chunk_replay")


def scan_reverse_chunk_summary(a, grad_out, P, Q, B, T, D, chunk, dtype, stream):
    return _check(library().scan_reverse_chunk_summary(a, grad_out, P, Q, B, T, D, chunk, dtype,
                                                       stream), "scan_reverse_chunk_summary")


def scan_reverse_chunk_prefix(P, Q, grad_last, future, grad_h0, B, NC, D, stream):
    return _check(library().scan_reverse_chunk_prefix(P, Q, grad_last, future, grad_h0, B, NC, D,
                                                      stream), "scan_reverse_chunk_prefix")


def scan_reverse_chunk_replay(a, out, grad_out, future, h0, grad_a, grad_b, B, T, D, chunk, dtype,
                              stream):
    return _check(library().scan_reverse_chunk_replay(a, out, grad_out, future, h0, grad_a, grad_b,
                                                      B, T, D, chunk, dtype, stream),
                  "scan_reverse_chunk_replay")


# ---------------------------------------------------------------------------
# torch tensor helpers (allocation + marshalling only)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {dt}; use float32 or bfloat16")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t):
    return _torch().cuda.current_stream(t.device).cuda_stream


def _check_seq(name, t, ref=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dim() != 3:
        raise ValueError(f"{name} must be [B, T, D]")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ref is not None and (t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device):
        raise ValueError(f"{name} must match a in shape, dtype and device")


def _check_state(name, t, ref):
    if t is None:
        return
    torch = _torch()
    B, _, D = ref.shape
    if t.shape != (B, D) or t.dtype != torch.float32 or t.device != ref.device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 [B, D] tensor on a's device")


def _check_mask(t, ref):
    """Segment-start mask: a contiguous bool or uint8 [B, T] tensor on a's device."""
    if t is None:
        return
    torch = _torch()
    B, T, _ = ref.shape
    if (t.shape != (B, T) or t.dtype not in (torch.bool, torch.uint8) or t.device != ref.device
            or not t.is_contiguous()):
        raise ValueError("reset must be a contiguous bool or uint8 [B, T] tensor on a's device")


def make_opts(algo="auto", chunk=0, h0=None, grad_h0=None, workspace=None, width=0, polls=0,
              reset=None):
    o = Opts()
    o.algo = ALGOS[algo] if isinstance(algo, str) else int(algo)
    o.chunk = int(chunk)
    o.width = int(width)
    o.workspace = None if workspace is None else workspace.data_ptr()
    o.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    o.h0 = _ptr(h0)
    o.grad_h0 = _ptr(grad_h0)
    o.polls = int(polls)
    o.reset = _ptr(reset)
    return o


def scan(a, b, h0=None, algo="auto", chunk=0, with_last=True, width=0, polls=0, reset=None,
         with_out=True):
    """Forward scan.  Returns (out, last); out has a's dtype, last is float32 [B, D].
    ``reset`` ([B, T] bool/uint8) starts a new segment wherever it is set.
    ``with_out=False`` runs the state-only forward (out is None)."""
    torch = _torch()
    _check_seq("a", a)
    _check_mask(reset, a)
    _check_seq("b", b, a)
    _check_state("h0", h0, a)
    B, T, D = a.shape
    if not (with_out or with_last):
        raise ValueError("a forward needs out or last")
    out = torch.empty_like(a) if with_out else None
    last = torch.empty((B, D), device=a.device, dtype=torch.float32) if with_last else None
    with torch.cuda.device(a.device):
        scan_fwd_ex(a.data_ptr(), b.data_ptr(), _ptr(out), _ptr(last), B, T, D,
                    dtype_code(a.dtype), _stream(a),
                    make_opts(algo, chunk, h0=h0, width=width, polls=polls, reset=reset))
    return out, last


def scan_backward(a, out, grad_out, grad_last=None, h0=None, algo="auto", chunk=0,
                  need_grad_h0=False, width=0, polls=0, reset=None):
    """Reverse-time adjoint.  Returns (grad_a, grad_b, grad_h0 or None).  ``reset``
    must be the mask the forward used."""
    torch = _torch()
    _check_seq("a", a)
    _check_mask(reset, a)
    _check_seq("out", out, a)
    _check_seq("grad_out", grad_out, a)
    _check_state("grad_last", grad_last, a)
    _check_state("h0", h0, a)
    B, T, D = a.shape
    grad_a = torch.empty_like(a)
    grad_b = torch.empty_like(a)
    grad_h0 = torch.empty((B, D), device=a.device, dtype=torch.float32) if need_grad_h0 else None
    with torch.cuda.device(a.device):
        scan_bwd_ex(a.data_ptr(), out.data_ptr(), grad_out.data_ptr(), _ptr(grad_last),
                    grad_a.data_ptr(), grad_b.data_ptr(), B, T, D, dtype_code(a.dtype), _stream(a),
                    make_opts(algo, chunk, h0=h0, grad_h0=grad_h0, width=width, polls=polls,
                              reset=reset))
    return grad_a, grad_b, grad_h0


def step(a, b, state=None, reset=None, with_out=True, out_state=None):
    """One decoding step on [B, D]: h = a*state + b (state None: zero; rows
    with reset set start from zero).  Returns (out in a's dtype or None,
    the new float32 state).  ``out_state`` may be ``state`` (in place)."""
    torch = _torch()
    if not isinstance(a, torch.Tensor) or not a.is_cuda or a.dim() != 2 or not a.is_contiguous():
        raise ValueError("a must be a contiguous CUDA (HIP) [B, D] tensor")
    if not isinstance(b, torch.Tensor) or b.shape != a.shape or b.dtype != a.dtype or \
            b.device != a.device or not b.is_contiguous():
        raise ValueError("b must match a in shape, dtype and device")
    B, D = a.shape
    for name, t in (("state", state), ("out_state", out_state)):
        if t is not None and (t.shape != (B, D) or t.dtype != torch.float32 or t.device != a.device
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 [B, D] tensor on a's device")
    if reset is not None and (reset.shape != (B,) or reset.dtype not in (torch.bool, torch.uint8)
                              or reset.device != a.device or not reset.is_contiguous()):
        raise ValueError("reset must be a contiguous bool or uint8 [B] tensor on a's device")
    out = torch.empty_like(a) if with_out else None
    new = out_state if out_state is not None else torch.empty((B, D), device=a.device,
                                                              dtype=torch.float32)
    with torch.cuda.device(a.device):
        scan_step(a.data_ptr(), b.data_ptr(), _ptr(state), _ptr(reset), _ptr(out), new.data_ptr(),
                  B, D, dtype_code(a.dtype), _stream(a))
    return out, new


def _pair(x):
    return (None, None) if x is None else (x[0], x[1])


def complex_scan(ar, ai, br, bi, h0=None, algo="auto", with_last=True, with_out=True, polls=0,
                 reset=None):
    """Complex scan h_t = a_t h_{t-1} + b_t on planar [B, T, M] tensors (real
    and imaginary parts separate).  h0: (re, im) float32 [B, M] pair or None.
    Returns (out_r, out_i, last_r, last_i); parts not asked for are None."""
    torch = _torch()
    _check_seq("ar", ar)
    for name, t in (("ai", ai), ("br", br), ("bi", bi)):
        _check_seq(name, t, ar)
    _check_mask(reset, ar)
    h0r, h0i = _pair(h0)
    _check_state("h0 (real part)", h0r, ar)
    _check_state("h0 (imaginary part)", h0i, ar)
    if not (with_out or with_last):
        raise ValueError("a forward needs out or last")
    B, T, M = ar.shape
    out_r = torch.empty_like(ar) if with_out else None
    out_i = torch.empty_like(ar) if with_out else None
    mk = (lambda: torch.empty((B, M), device=ar.device, dtype=torch.float32))
    last_r, last_i = (mk(), mk()) if with_last else (None, None)
    with torch.cuda.device(ar.device):
        scan_complex_fwd(ar.data_ptr(), ai.data_ptr(), br.data_ptr(), bi.data_ptr(), _ptr(out_r),
                         _ptr(out_i), _ptr(last_r), _ptr(last_i), _ptr(h0r), _ptr(h0i), B, T, M,
                         dtype_code(ar.dtype), _stream(ar),
                         make_opts(algo, polls=polls, reset=reset))
    return out_r, out_i, last_r, last_i


def complex_scan_backward(ar, ai, out_r, out_i, grad_out_r, grad_out_i, grad_last=None, h0=None,
                          algo="auto", need_grad_h0=False, polls=0, reset=None):
    """Adjoint of complex_scan for L = sum Re(conj(g) out) + Re(conj(grad_last) last).
    Returns (grad_ar, grad_ai, grad_br, grad_bi, (grad_h0_r, grad_h0_i) or None)."""
    torch = _torch()
    _check_seq("ar", ar)
    for name, t in (("ai", ai), ("out_r", out_r), ("out_i", out_i), ("grad_out_r", grad_out_r),
                    ("grad_out_i", grad_out_i)):
        _check_seq(name, t, ar)
    _check_mask(reset, ar)
    glr, gli = _pair(grad_last)
    h0r, h0i = _pair(h0)
    for name, t in (("grad_last", glr), ("grad_last", gli), ("h0", h0r), ("h0", h0i)):
        _check_state(name, t, ar)
    B, T, M = ar.shape
    g = [torch.empty_like(ar) for _ in range(4)]
    gh0 = ((torch.empty((B, M), device=ar.device, dtype=torch.float32),
            torch.empty((B, M), device=ar.device, dtype=torch.float32)) if need_grad_h0 else None)
    gh0r, gh0i = _pair(gh0)
    with torch.cuda.device(ar.device):
        scan_complex_bwd(ar.data_ptr(), ai.data_ptr(), out_r.data_ptr(), out_i.data_ptr(),
                         grad_out_r.data_ptr(), grad_out_i.data_ptr(), _ptr(glr), _ptr(gli),
                         _ptr(h0r), _ptr(h0i), g[0].data_ptr(), g[1].data_ptr(), g[2].data_ptr(),
                         g[3].data_ptr(), _ptr(gh0r), _ptr(gh0i), B, T, M, dtype_code(ar.dtype),
                         _stream(ar), make_opts(algo, polls=polls, reset=reset))
    return g[0], g[1], g[2], g[3], gh0


def _check_controls(eta, delta, nu_log, theta_log, ref):
    """eta, delta: contiguous [B, T] tensors of b's dtype; nu_log, theta_log:
    contiguous float32 [M] tensors, all on b's device."""
    torch = _torch()
    B, T, M = ref.shape
    for name, t in (("eta", eta), ("delta", delta)):
        if (not isinstance(t, torch.Tensor) or t.shape != (B, T) or t.dtype != ref.dtype
                or t.device != ref.device or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous [B, T] tensor of b's dtype and device")
    for name, t in (("nu_log", nu_log), ("theta_log", theta_log)):
        if (not isinstance(t, torch.Tensor) or t.shape != (M,) or t.dtype != torch.float32
                or t.device != ref.device or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 [M] tensor on b's device")


def samu_scan(eta, delta, nu_log, theta_log, br, bi, h0=None, with_last=True, with_out=True,
              polls=0, reset=None, workspace=None, algo="auto"):
    """Fused-transition complex scan: a_t = exp(-e^nu_log e^eta) exp(i (e^theta_log + delta))
    is rebuilt in the kernel; h_t = a_t h_{t-1} + b_t on planar [B, T, M] b.
    Returns (out_r, out_i, last_r, last_i); parts not asked for are None."""
    torch = _torch()
    _check_seq("br", br)
    _check_seq("bi", bi, br)
    _check_controls(eta, delta, nu_log, theta_log, br)
    _check_mask(reset, br)
    h0r, h0i = _pair(h0)
    _check_state("h0 (real part)", h0r, br)
    _check_state("h0 (imaginary part)", h0i, br)
    if not (with_out or with_last):
        raise ValueError("a forward needs out or last")
    B, T, M = br.shape
    out_r = torch.empty_like(br) if with_out else None
    out_i = torch.empty_like(br) if with_out else None
    mk = (lambda: torch.empty((B, M), device=br.device, dtype=torch.float32))
    last_r, last_i = (mk(), mk()) if with_last else (None, None)
    with torch.cuda.device(br.device):
        scan_samu_fwd(eta.data_ptr(), delta.data_ptr(), nu_log.data_ptr(), theta_log.data_ptr(),
                      br.data_ptr(), bi.data_ptr(), _ptr(out_r), _ptr(out_i), _ptr(last_r),
                      _ptr(last_i), _ptr(h0r), _ptr(h0i), B, T, M, dtype_code(br.dtype),
                      _stream(br), make_opts(algo=algo, polls=polls, reset=reset,
                                             workspace=workspace))
    return out_r, out_i, last_r, last_i


def samu_scan_backward(eta, delta, nu_log, theta_log, out_r, out_i, grad_out_r, grad_out_i,
                       grad_last=None, h0=None, need_grad_h0=False, polls=0, reset=None,
                       workspace=None, algo="auto"):
    """Adjoint of samu_scan for L = sum Re(conj(g) out) + Re(conj(grad_last) last).
    Returns (grad_eta [B,T], grad_delta [B,T], grad_nu_log [M], grad_theta_log [M]
    (all float32), grad_br, grad_bi, (grad_h0_r, grad_h0_i) or None)."""
    torch = _torch()
    _check_seq("out_r", out_r)
    for name, t in (("out_i", out_i), ("grad_out_r", grad_out_r), ("grad_out_i", grad_out_i)):
        _check_seq(name, t, out_r)
    _check_controls(eta, delta, nu_log, theta_log, out_r)
    _check_mask(reset, out_r)
    glr, gli = _pair(grad_last)
    h0r, h0i = _pair(h0)
    for name, t in (("grad_last", glr), ("grad_last", gli), ("h0", h0r), ("h0", h0i)):
        _check_state(name, t, out_r)
    B, T, M = out_r.shape
    dev = out_r.device
    ge = torch.empty((B, T), device=dev, dtype=torch.float32)
    gd = torch.empty((B, T), device=dev, dtype=torch.float32)
    gn = torch.empty((M,), device=dev, dtype=torch.float32)
    gt = torch.empty((M,), device=dev, dtype=torch.float32)
    gbr, gbi = torch.empty_like(out_r), torch.empty_like(out_r)
    gh0 = ((torch.empty((B, M), device=dev, dtype=torch.float32),
            torch.empty((B, M), device=dev, dtype=torch.float32)) if need_grad_h0 else None)
    gh0r, gh0i = _pair(gh0)
    with torch.cuda.device(dev):
        scan_samu_bwd(eta.data_ptr(), delta.data_ptr(), nu_log.data_ptr(), theta_log.data_ptr(),
                      out_r.data_ptr(), out_i.data_ptr(), grad_out_r.data_ptr(),
                      grad_out_i.data_ptr(), _ptr(glr), _ptr(gli), _ptr(h0r), _ptr(h0i),
                      ge.data_ptr(), gd.data_ptr(), gn.data_ptr(), gt.data_ptr(), gbr.data_ptr(),
                      gbi.data_ptr(), _ptr(gh0r), _ptr(gh0i), B, T, M, dtype_code(out_r.dtype),
                      _stream(out_r), make_opts(algo=algo, polls=polls, reset=reset, workspace=workspace))
    return ge, gd, gn, gt, gbr, gbi, gh0


def n_chunks(T, chunk):
    return (T + chunk - 1) // chunk


def chunk_summary(a, b, chunk, reverse=False):
    """(P, Q) per chunk, float32 [B, NC, D] (reverse: b is grad_out)."""
    torch = _torch()
    _check_seq("a", a)
    _check_seq("b", b, a)
    B, T, D = a.shape
    NC = n_chunks(T, chunk)
    P = torch.empty((B, NC, D), device=a.device, dtype=torch.float32)
    Q = torch.empty_like(P)
    fn = scan_reverse_chunk_summary if reverse else scan_chunk_summary
    with torch.cuda.device(a.device):
        fn(a.data_ptr(), b.data_ptr(), P.data_ptr(), Q.data_ptr(), B, T, D, chunk,
           dtype_code(a.dtype), _stream(a))
    return P, Q


def chunk_prefix(P, Q, init=None, reverse=False):
    """Exclusive scan over chunk maps.  Returns (entering [B,NC,D], final [B,D])."""
    torch = _torch()
    B, NC, D = P.shape
    ent = torch.empty_like(P)
    fin = torch.empty((B, D), device=P.device, dtype=torch.float32)
    fn = scan_reverse_chunk_prefix if reverse else scan_chunk_prefix
    with torch.cuda.device(P.device):
        fn(P.data_ptr(), Q.data_ptr(), _ptr(init), ent.data_ptr(), fin.data_ptr(), B, NC, D,
           _stream(P))
    return ent, fin


def chunk_replay(a, b, chunk_in, chunk):
    torch = _torch()
    B, T, D = a.shape
    out = torch.empty_like(a)
    last = torch.empty((B, D), device=a.device, dtype=torch.float32)
    with torch.cuda.device(a.device):
        scan_chunk_replay(a.data_ptr(), b.data_ptr(), chunk_in.data_ptr(), out.data_ptr(),
                          last.data_ptr(), B, T, D, chunk, dtype_code(a.dtype), _stream(a))
    return out, last


def reverse_chunk_replay(a, out, grad_out, future, chunk, h0=None):
    torch = _torch()
    B, T, D = a.shape
    ga = torch.empty_like(a)
    gb = torch.empty_like(a)
    with torch.cuda.device(a.device):
        scan_reverse_chunk_replay(a.data_ptr(), out.data_ptr(), grad_out.data_ptr(),
                                  future.data_ptr(), _ptr(h0), ga.data_ptr(), gb.data_ptr(), B, T,
                                  D, chunk, dtype_code(a.dtype), _stream(a))
    return ga, gb


def _scan_function(run_forward, run_backward):
    """A torch.autograd.Function over one pair of C entry points.

    ``run_forward(reset, inputs)`` returns (outputs, kept): the outputs the
    caller gets and the tensors the backward entry point reads (for every
    scan here: the transition operands and the forward's ``out``, never
    ``b``).  ``run_backward(reset, kept, grads)`` returns one gradient per
    input.  Inputs and incoming gradients are made contiguous before they
    reach the C ABI, which takes only contiguous [B, T, D] storage; the
    segment mask is passed through and gets no gradient."""
    torch = _torch()

    class ScanFunction(torch.autograd.Function):
        @staticmethod
        def forward(ctx, reset, *inputs):
            outs, kept = run_forward(reset, [t.contiguous() for t in inputs])
            ctx.save_for_backward(*kept)
            ctx.reset = reset
            return outs[0] if len(outs) == 1 else tuple(outs)

        @staticmethod
        def backward(ctx, *grads):
            grads = [g.contiguous() for g in grads]
            return (None, *run_backward(ctx.reset, ctx.saved_tensors, grads))

    return ScanFunction


def _real_forward(reset, inputs):
    a, b = inputs
    out, _ = scan(a, b, with_last=False, reset=reset)
    return [out], (a, out)


def _real_backward(reset, kept, grads):
    a, out = kept
    ga, gb, _ = scan_backward(a, out, grads[0], reset=reset)
    return ga, gb


def _complex_forward(reset, inputs):
    ar, ai, br, bi = inputs
    out_r, out_i, _, _ = complex_scan(ar, ai, br, bi, with_last=False, reset=reset)
    return [out_r, out_i], (ar, ai, out_r, out_i)


def _complex_backward(reset, kept, grads):
    ar, ai, out_r, out_i = kept
    gar, gai, gbr, gbi, _ = complex_scan_backward(ar, ai, out_r, out_i, grads[0], grads[1],
                                                  reset=reset)
    return gar, gai, gbr, gbi


def _samu_forward(reset, inputs):
    eta, delta, nu_log, theta_log, br, bi = inputs
    out_r, out_i, _, _ = samu_scan(eta, delta, nu_log, theta_log, br, bi, with_last=False,
                                   reset=reset)
    return [out_r, out_i], (eta, delta, nu_log, theta_log, out_r, out_i)


def _samu_backward(reset, kept, grads):
    eta, delta, nu_log, theta_log, out_r, out_i = kept
    ge, gd, gn, gt, gbr, gbi, _ = samu_scan_backward(eta, delta, nu_log, theta_log, out_r, out_i,
                                                     grads[0], grads[1], reset=reset)
    # the per-token gradients come back in fp32; the controls may be bf16
    return ge.to(eta.dtype), gd.to(delta.dtype), gn, gt, gbr, gbi


_functions = {}


def _function(name):
    if name not in _functions:
        pair = {"real": (_real_forward, _real_backward),
                "complex": (_complex_forward, _complex_backward),
                "samu": (_samu_forward, _samu_backward)}[name]
        _functions[name] = _scan_function(*pair)
    return _functions[name]


def diagonal_scan(a, b, reset=None):
    """Differentiable scan (torch autograd) returning every state; ``reset``
    ([B, T] bool/uint8, not differentiated) starts new segments."""
    return _function("real").apply(reset, a, b)


def complex_diagonal_scan(ar, ai, br, bi, reset=None):
    """Differentiable complex scan (torch autograd) on planar tensors; returns (out_r, out_i)."""
    return _function("complex").apply(reset, ar, ai, br, bi)


def samu_diagonal_scan(eta, delta, nu_log, theta_log, br, bi, reset=None):
    """Differentiable fused-transition scan (torch autograd); returns (out_r, out_i)."""
    return _function("samu").apply(reset, eta, delta, nu_log, theta_log, br, bi)
