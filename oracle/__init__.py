"""fp64 CPU oracle of the selective state-space scan.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are its only users. It shares no code with the GPU library
and imports nothing from it.

The arithmetic lives in ``ssm_oracle.c`` (a plain loop over the recurrence of
the page "Mamba and State Space Models", sections "A State of Fixed Size" and
"Chosen by the Token"); this module only marshals arrays into fp64 and calls
it. Inputs may be numpy arrays or torch tensors of any float dtype: they are
widened exactly to fp64 (bf16 and fp32 values are representable in fp64), so
the oracle sees the very values the GPU consumed. Results stay fp64.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def library_path():
    return os.environ.get("SSM_ORACLE_LIB", _build.LIBRARY)


def _load(path=None):
    path = path or library_path()
    if not os.path.exists(path):
        _build.compile_oracle(output=path)
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_scan_fwd.argtypes = [i64, i64, i64, i64] + [dp] * 10 + [ctypes.c_int, dp,
                                                                       ctypes.c_int]
    lib.oracle_scan_fwd.restype = ctypes.c_int
    lib.oracle_state_update.argtypes = [i64, i64, i64] + [dp] * 9 + [dp, ctypes.c_int]
    lib.oracle_state_update.restype = ctypes.c_int
    lib.oracle_max_dstate.restype = ctypes.c_int
    lib.oracle_scan_bwd.argtypes = ([i64] * 4 + [dp] * 9 + [ctypes.c_int] + [dp] * 11)
    lib.oracle_scan_bwd.restype = ctypes.c_int
    lib.oracle_ssd_fwd.argtypes = [i64] * 5 + [dp] * 10 + [dp, ctypes.c_int]
    lib.oracle_ssd_fwd.restype = ctypes.c_int
    lib.oracle_conv1d_fwd.argtypes = [i64] * 4 + [dp] * 6 + [ctypes.c_int]
    lib.oracle_conv1d_fwd.restype = ctypes.c_int
    lib.oracle_conv1d_update.argtypes = [i64] * 3 + [dp] * 5 + [ctypes.c_int]
    lib.oracle_conv1d_update.restype = ctypes.c_int
    return lib


def _f64(a):
    """Exact widening of a numpy array or torch tensor to a C-contiguous fp64 array."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: widen on the host with torch (knows bf16)
        import torch
        a = a.detach().to("cpu").to(torch.float64).contiguous().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class Oracle:
    """Handle on one compiled oracle library (the default one, or a test build)."""

    def __init__(self, path=None):
        self.lib = _load(path)
        self.max_dstate = self.lib.oracle_max_dstate()

    def scan_fwd(self, x, delta, A, B, C, D=None, z=None, h0=None, zoh=False,
                 return_state=True, delta_bias=None, delta_softplus=False):
        """Scan a whole sequence.

        Shapes: x, delta, z (batch, L, dim); A (dim, N); B, C (batch, L, N);
        D, delta_bias (dim,); h0 (batch, dim, N). With delta_softplus the
        delta used is softplus(delta + delta_bias). Returns (y, hL) as fp64
        numpy arrays, y of shape (batch, L, dim) and hL of shape (batch, dim, N).
        """
        x, delta, A, B, C = (_f64(v) for v in (x, delta, A, B, C))
        D, z, h0, bias = _f64(D), _f64(z), _f64(h0), _f64(delta_bias)
        batch, seqlen, dim = x.shape
        dstate = A.shape[1]
        assert delta.shape == x.shape and A.shape == (dim, dstate)
        assert B.shape == (batch, seqlen, dstate) and C.shape == B.shape
        assert D is None or D.shape == (dim,)
        assert z is None or z.shape == x.shape
        assert h0 is None or h0.shape == (batch, dim, dstate)
        assert bias is None or bias.shape == (dim,)
        y = np.zeros((batch, seqlen, dim), dtype=np.float64)
        hL = np.zeros((batch, dim, dstate), dtype=np.float64) if return_state else None
        rc = self.lib.oracle_scan_fwd(batch, seqlen, dim, dstate, _ptr(x), _ptr(delta),
                                      _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                      _ptr(h0), _ptr(y), _ptr(hL), int(bool(zoh)), _ptr(bias),
                                      int(bool(delta_softplus)))
        if rc != 0:
            raise ValueError(f"oracle_scan_fwd rejected its arguments (status {rc})")
        return y, hL

    def state_update(self, h, x, delta, A, B, C, D=None, z=None, delta_bias=None,
                     delta_softplus=False):
        """One decode step. Shapes: h (batch, dim, N); x, delta, z (batch, dim);
        B, C (batch, N). Returns (y, h_new); the input h is not modified."""
        h = _f64(h).copy()
        x, delta, A, B, C = (_f64(v) for v in (x, delta, A, B, C))
        D, z, bias = _f64(D), _f64(z), _f64(delta_bias)
        batch, dim, dstate = h.shape
        assert x.shape == (batch, dim) and delta.shape == x.shape
        assert A.shape == (dim, dstate) and B.shape == (batch, dstate) and C.shape == B.shape
        y = np.zeros((batch, dim), dtype=np.float64)
        rc = self.lib.oracle_state_update(batch, dim, dstate, _ptr(h), _ptr(x), _ptr(delta),
                                          _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y),
                                          _ptr(bias), int(bool(delta_softplus)))
        if rc != 0:
            raise ValueError(f"oracle_state_update rejected its arguments (status {rc})")
        return y, h


    def scan_bwd(self, x, delta, A, B, C, D=None, z=None, h0=None, dy=None, dhL=None,
                 delta_bias=None, delta_softplus=False):
        """Gradients of L = sum(dy * y) + sum(dhL * hL) with respect to every
        input of scan_fwd (same shapes and options). Returns a dict of fp64
        arrays: dx, ddelta, dz (batch, L, dim); dB, dC (batch, L, N); dA
        (dim, N); dD, ddelta_bias (dim,); dh0 (batch, dim, N). Entries for
        absent optional inputs (D, z, delta_bias) are None; dh0 is always
        returned (the gradient at a zero initial state when h0 is None)."""
        x, delta, A, B, C = (_f64(v) for v in (x, delta, A, B, C))
        D, z, h0, bias = _f64(D), _f64(z), _f64(h0), _f64(delta_bias)
        dy, dhL = _f64(dy), _f64(dhL)
        batch, seqlen, dim = x.shape
        dstate = A.shape[1]
        assert delta.shape == x.shape and dy.shape == x.shape
        assert B.shape == (batch, seqlen, dstate) and C.shape == B.shape
        out = dict(dx=np.zeros_like(x), ddelta=np.zeros_like(x),
                   dA=np.zeros((dim, dstate)), dB=np.zeros_like(B), dC=np.zeros_like(C),
                   dD=None if D is None else np.zeros(dim),
                   dz=None if z is None else np.zeros_like(x),
                   dh0=np.zeros((batch, dim, dstate)),
                   ddelta_bias=None if bias is None else np.zeros(dim))
        rc = self.lib.oracle_scan_bwd(
            batch, seqlen, dim, dstate, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
            _ptr(D), _ptr(z), _ptr(h0), _ptr(bias), int(bool(delta_softplus)), _ptr(dy),
            _ptr(dhL), _ptr(out["dx"]), _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]),
            _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]), _ptr(out["dh0"]),
            _ptr(out["ddelta_bias"]))
        if rc != 0:
            raise ValueError(f"oracle_scan_bwd rejected its arguments (status {rc})")
        return out

    def ssd_fwd(self, x, dt, A, B, C, D=None, z=None, h0=None, headdim=64, dt_bias=None,
                dt_softplus=False, return_state=True):
        """Mamba-2 dual form with a scalar decay per head. Shapes: x, z
        (batch, L, nheads*headdim); dt (batch, L, nheads); A, dt_bias
        (nheads,); B, C (batch, L, N); D (nheads*headdim,); h0 (batch, nheads,
        headdim, N). Returns (y, hL) as fp64 arrays."""
        x, dt, A, B, C = (_f64(v) for v in (x, dt, A, B, C))
        D, z, h0, bias = _f64(D), _f64(z), _f64(h0), _f64(dt_bias)
        batch, seqlen, dim = x.shape
        nheads = dt.shape[2]
        assert dim == nheads * headdim and A.shape == (nheads,)
        dstate = B.shape[2]
        y = np.zeros((batch, seqlen, dim), dtype=np.float64)
        hL = np.zeros((batch, nheads, headdim, dstate)) if return_state else None
        rc = self.lib.oracle_ssd_fwd(batch, seqlen, nheads, headdim, dstate, _ptr(x), _ptr(dt),
                                     _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                     _ptr(y), _ptr(hL), _ptr(bias), int(bool(dt_softplus)))
        if rc != 0:
            raise ValueError(f"oracle_ssd_fwd rejected its arguments (status {rc})")
        return y, hL

    def conv1d_fwd(self, x, weight, bias=None, state_in=None, silu=True, return_state=True):
        """Short causal depthwise convolution over whole sequences.

        Shapes: x (batch, L, dim); weight (dim, W); bias (dim,); state_in
        (batch, dim, W), the last W inputs before the sequence (None: zeros).
        Returns (y, state_out) as fp64 numpy arrays: y (batch, L, dim) and
        state_out (batch, dim, W), the last W inputs after the sequence.
        """
        x, weight, bias, state_in = _f64(x), _f64(weight), _f64(bias), _f64(state_in)
        batch, seqlen, dim = x.shape
        width = weight.shape[1]
        assert weight.shape == (dim, width)
        assert bias is None or bias.shape == (dim,)
        assert state_in is None or state_in.shape == (batch, dim, width)
        y = np.zeros((batch, seqlen, dim), dtype=np.float64)
        st = np.zeros((batch, dim, width), dtype=np.float64) if return_state else None
        rc = self.lib.oracle_conv1d_fwd(batch, seqlen, dim, width, _ptr(x), _ptr(weight),
                                        _ptr(bias), _ptr(state_in), _ptr(y), _ptr(st),
                                        int(bool(silu)))
        if rc != 0:
            raise ValueError(f"oracle_conv1d_fwd rejected its arguments (status {rc})")
        return y, st

    def conv1d_update(self, state, x, weight, bias=None, silu=True):
        """One decode step of the convolution. Shapes: state (batch, dim, W);
        x (batch, dim). Returns (y, state_new); the input state is not modified."""
        state = _f64(state).copy()
        x, weight, bias = _f64(x), _f64(weight), _f64(bias)
        batch, dim, width = state.shape
        assert x.shape == (batch, dim) and weight.shape == (dim, width)
        y = np.zeros((batch, dim), dtype=np.float64)
        rc = self.lib.oracle_conv1d_update(batch, dim, width, _ptr(state), _ptr(x), _ptr(weight),
                                           _ptr(bias), _ptr(y), int(bool(silu)))
        if rc != 0:
            raise ValueError(f"oracle_conv1d_update rejected its arguments (status {rc})")
        return y, state


def get():
    """The shared oracle instance built from ``ssm_oracle.c``."""
    global _LIB
    if _LIB is None:
        _LIB = Oracle()
    return _LIB
