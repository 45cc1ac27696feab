"""Selective state-space scan for AMD Instinct MI355X (gfx950).

Python binding of the C ABI in include/mamba_scan.h. It only marshals
arguments: it checks shapes and dtypes, allocates outputs and scratch with
torch on the tensors' device, and passes raw device pointers and the current
HIP stream to libmamba_scan.so, whose kernels do every step of the scan.
There is no other code path: without the built library every call raises.

    y, hL = scan_fwd(x, delta, A, B, C, D=None, z=None, h0=None,
                     delta_bias=None, delta_softplus=False)
    scan_fwd_noalloc(x, delta, A, B, C, D, z, h0, y=y, hL=hL)  # outputs given, nothing allocated
    y = state_update(h, x, delta, A, B, C, D=None, z=None,
                     delta_bias=None, delta_softplus=False)   # h updated in place
    grads = scan_bwd(x, delta, A, B, C, D=None, z=None, h0=None, dy=dy, dhL=None,
                     delta_bias=None, delta_softplus=False)      # dict of gradients
    y, hL = ssd_fwd(x, dt, A_heads, B, C, D=None, z=None, h0=None)   # Mamba-2 dual form
    y, state = conv1d_fwd(x, weight, bias=None, state_in=None, silu=True)
    y = conv1d_update(state, x, weight, bias=None, silu=True)  # state updated in place

Shapes (row-major, contiguous): x, delta, z, y (batch, L, dim); B, C
(batch, L, N); A (dim, N) fp32; D and delta_bias (dim,) fp32; h0, hL
(batch, dim, N) fp32. With delta_softplus the kernels use
softplus(delta + delta_bias) in place of delta. The short convolution takes
x, y (batch, L, dim), weight (dim, W) fp32, bias (dim,) fp32 and a state of
the last W inputs (batch, dim, W) in the dtype of x.
x, delta, z, B and C share one dtype, float32 or bfloat16, and y has it too.
"""
import collections
import ctypes
import os

import torch

__all__ = ["scan_fwd", "scan_fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "scan_bwd", "ssd_fwd", "state_update", "conv1d_fwd", "conv1d_update", "workspace_size", "resolve_plan", "library_path",
           "load_library", "MambaScanError", "MAX_DSTATE", "ScanPlan", "ScanOptions", "Plan",
           "CARRY_AUTO", "CARRY_RERUN", "CARRY_REPAIR", "HALVES_AUTO", "HALVES_NONE"]

MAX_DSTATE = 16
NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024  # MAMBA_NOALLOC_SCRATCH_BYTES
_DTYPES = {torch.float32: 0, torch.bfloat16: 1}
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_WS = {}


CARRY_AUTO, CARRY_RERUN, CARRY_REPAIR = 0, 1, 2


HALVES_AUTO, HALVES_NONE = 0, -1


class ScanPlan(ctypes.Structure):
    """mamba_scan_plan: chunk_len (tokens per parallel chunk), state_split
    (waves sharing one channel's states), carry (CARRY_RERUN: summary pass
    and a rerun of every chunk; CARRY_REPAIR: one pass from zero states and a
    rerun of each chunk's head while the entering state still counts) and
    halves (the last channel groups run as two 32-channel halves; -1 none,
    k > 0 the last k groups); 0 means automatic."""
    _fields_ = [("chunk_len", ctypes.c_int64), ("state_split", ctypes.c_int32),
                ("carry", ctypes.c_int32), ("halves", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


Plan = collections.namedtuple("Plan", "chunk_len state_split carry halves workspace_bytes")


class ScanOptions(ctypes.Structure):
    """mamba_scan_options: optional delta bias (device pointer) and softplus."""
    _fields_ = [("delta_bias", ctypes.c_void_p), ("delta_softplus", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class MambaScanError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


def library_path():
    return os.environ.get("MAMBA_SCAN_LIB", os.path.join(_HERE, "libmamba_scan.so"))


def load_library():
    """Load libmamba_scan.so (built in-tree by __graft_entry__.build())."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise MambaScanError(-5, f"HIP library not built: {path} is missing "
                                 "(run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    pp = ctypes.POINTER(ScanPlan)
    po = ctypes.POINTER(ScanOptions)
    lib.ssm_scan_fwd_workspace_size.argtypes = [i64, i64, i64, i32, i32, pp, pp,
                                                ctypes.POINTER(ctypes.c_size_t)]
    lib.ssm_scan_fwd_workspace_size.restype = i32
    lib.ssm_scan_fwd.argtypes = ([i64, i64, i64, i32, i32] + [vp] * 10 +
                                 [po, pp, vp, ctypes.c_size_t, vp])
    lib.ssm_scan_fwd.restype = i32
    lib.ssm_scan_fwd_noalloc.argtypes = [i64, i64, i64, i32, i32] + [vp] * 10 + [po, pp, vp]
    lib.ssm_scan_fwd_noalloc.restype = i32
    lib.ssm_state_update.argtypes = [i64, i64, i32, i32] + [vp] * 9 + [po, vp]
    lib.ssm_state_update.restype = i32
    lib.ssm_scan_bwd_workspace_size.argtypes = [i64, i64, i64, i32, i32, pp, pp,
                                                ctypes.POINTER(ctypes.c_size_t)]
    lib.ssm_scan_bwd_workspace_size.restype = i32
    lib.ssm_scan_bwd.argtypes = ([i64, i64, i64, i32, i32] + [vp] * 8 + [po, pp] + [vp] * 11 +
                                 [vp, ctypes.c_size_t, vp])
    lib.ssm_scan_bwd.restype = i32
    lib.ssd_fwd.argtypes = [i64, i64, i64, i64, i32, i32] + [vp] * 10 + [po, vp]
    lib.ssd_fwd.restype = i32
    lib.causal_conv1d_fwd.argtypes = [i64, i64, i64, i32, i32] + [vp] * 6 + [i32, vp]
    lib.causal_conv1d_fwd.restype = i32
    lib.causal_conv1d_update.argtypes = [i64, i64, i32, i32] + [vp] * 5 + [i32, vp]
    lib.causal_conv1d_update.restype = i32
    lib.mamba_status_string.argtypes = [i32]
    lib.mamba_status_string.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _check(status, what):
    if status != 0:
        msg = load_library().mamba_status_string(status).decode()
        raise MambaScanError(status, f"{what}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, shape, dtype, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _options(delta_bias, delta_softplus):
    if delta_bias is None and not delta_softplus:
        return None
    return ctypes.byref(ScanOptions(None if delta_bias is None else delta_bias.data_ptr(),
                                    1 if delta_softplus else 0, 0))


def resolve_plan(batch, seqlen, dim, dstate, dtype=torch.bfloat16, chunk_len=0, state_split=0,
                 carry=CARRY_AUTO, halves=HALVES_AUTO):
    """The plan ssm_scan_fwd uses for this shape, and its scratch bytes, as a
    Plan (chunk_len, state_split, carry, halves, workspace_bytes); halves is
    the number of channel groups split. Automatic fields query the current
    device."""
    req = ScanPlan(chunk_len, state_split, carry, halves, 0)
    out = ScanPlan(0, 0, 0, 0, 0)
    nbytes = ctypes.c_size_t(0)
    _check(load_library().ssm_scan_fwd_workspace_size(batch, seqlen, dim, dstate, _DTYPES[dtype],
                                                      ctypes.byref(req), ctypes.byref(out),
                                                      ctypes.byref(nbytes)),
           "ssm_scan_fwd_workspace_size")
    return Plan(out.chunk_len, out.state_split, out.carry, out.halves, nbytes.value)


def resolve_bwd_plan(batch, seqlen, dim, dstate, dtype=torch.bfloat16, chunk_len=0,
                     halves=HALVES_AUTO):
    """The plan ssm_scan_bwd uses for this shape, and its scratch bytes, as a
    Plan (chunk_len: the chunk length, the whole sequence when uncut; halves:
    the channel groups split; state_split and carry 0)."""
    req = ScanPlan(chunk_len, 0, 0, halves, 0)
    out = ScanPlan(0, 0, 0, 0, 0)
    nbytes = ctypes.c_size_t(0)
    _check(load_library().ssm_scan_bwd_workspace_size(batch, seqlen, dim, dstate, _DTYPES[dtype],
                                                      ctypes.byref(req), ctypes.byref(out),
                                                      ctypes.byref(nbytes)),
           "ssm_scan_bwd_workspace_size")
    return Plan(out.chunk_len, 0, 0, out.halves, nbytes.value)


def workspace_size(batch, seqlen, dim, dstate, dtype=torch.bfloat16, chunk_len=0, state_split=0,
                   carry=CARRY_AUTO, halves=HALVES_AUTO):
    """Scratch bytes ssm_scan_fwd needs for this shape and plan."""
    return resolve_plan(batch, seqlen, dim, dstate, dtype, chunk_len, state_split, carry,
                        halves).workspace_bytes


def _workspace(device, nbytes, kind="fwd"):
    if nbytes == 0:
        return None
    key = (device, torch.cuda.current_stream(device).cuda_stream, kind)
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _WS[key] = buf
    return buf


def scan_fwd(x, delta, A, B, C, D=None, z=None, h0=None, *, delta_bias=None,
             delta_softplus=False, chunk_len=0, state_split=0, carry=CARRY_AUTO,
             halves=HALVES_AUTO, return_state=True, out=None, state_out=None):
    """Selective scan over whole sequences; returns (y, hL) (hL is None when
    return_state is False). `delta_bias` (dim,) fp32 is added to delta and
    `delta_softplus` applies softplus after it, inside the kernels.
    `chunk_len` > 0 forces the parallel chunk length, `state_split` > 0 the
    number of waves sharing a channel's states, `carry` how chunks join
    (CARRY_RERUN or CARRY_REPAIR) and `halves` how many of the last channel
    groups run as two 32-channel halves (HALVES_NONE: none)."""
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (batch, L, dim)")
    batch, seqlen, dim = x.shape
    if A.dim() != 2 or A.shape[0] != dim:
        raise ValueError("A must be (dim, N)")
    dstate = A.shape[1]
    dev, dt = x.device, x.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported I/O dtype {dt}")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    _need(x, "x", (batch, seqlen, dim), dt, dev)
    _need(delta, "delta", (batch, seqlen, dim), dt, dev)
    _need(A, "A", (dim, dstate), torch.float32, dev)
    _need(B, "B", (batch, seqlen, dstate), dt, dev)
    _need(C, "C", (batch, seqlen, dstate), dt, dev)
    _need(D, "D", (dim,), torch.float32, dev)
    _need(z, "z", (batch, seqlen, dim), dt, dev)
    _need(h0, "h0", (batch, dim, dstate), torch.float32, dev)
    _need(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    y = out if out is not None else torch.empty_like(x)
    _need(y, "out", (batch, seqlen, dim), dt, dev)
    hL = None
    if return_state:
        hL = state_out if state_out is not None else torch.empty(batch, dim, dstate,
                                                                 dtype=torch.float32, device=dev)
        _need(hL, "state_out", (batch, dim, dstate), torch.float32, dev)
    plan = ScanPlan(chunk_len, state_split, carry, halves, 0)
    with torch.cuda.device(dev):
        nbytes = workspace_size(batch, seqlen, dim, dstate, dt, chunk_len, state_split, carry,
                                halves)
        ws = _workspace(dev, nbytes)
        st = lib.ssm_scan_fwd(batch, seqlen, dim, dstate, _DTYPES[dt], _ptr(x), _ptr(delta),
                              _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y),
                              _ptr(hL), _options(delta_bias, delta_softplus), ctypes.byref(plan),
                              _ptr(ws), nbytes, _stream(dev))
    _check(st, "ssm_scan_fwd")
    return y, hL


def scan_fwd_noalloc(x, delta, A, B, C, D=None, z=None, h0=None, *, y, hL=None,
                     delta_bias=None, delta_softplus=False, chunk_len=0, state_split=0,
                     carry=CARRY_AUTO, halves=HALVES_AUTO):
    """scan_fwd through ssm_scan_fwd_noalloc: the caller passes the outputs
    y (like x) and hL ((batch, dim, N) fp32 or None) and nothing is
    allocated, on the device or by torch; a chunked plan uses the library's
    fixed per-GPU scratch (NOALLOC_SCRATCH_BYTES), which calls that overlap
    on one GPU share. Returns (y, hL)."""
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (batch, L, dim)")
    batch, seqlen, dim = x.shape
    if A.dim() != 2 or A.shape[0] != dim:
        raise ValueError("A must be (dim, N)")
    dstate = A.shape[1]
    dev, dt = x.device, x.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported I/O dtype {dt}")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    _need(x, "x", (batch, seqlen, dim), dt, dev)
    _need(delta, "delta", (batch, seqlen, dim), dt, dev)
    _need(A, "A", (dim, dstate), torch.float32, dev)
    _need(B, "B", (batch, seqlen, dstate), dt, dev)
    _need(C, "C", (batch, seqlen, dstate), dt, dev)
    _need(D, "D", (dim,), torch.float32, dev)
    _need(z, "z", (batch, seqlen, dim), dt, dev)
    _need(h0, "h0", (batch, dim, dstate), torch.float32, dev)
    _need(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    if y is None:
        raise ValueError("y (the output) is required")
    _need(y, "y", (batch, seqlen, dim), dt, dev)
    _need(hL, "hL", (batch, dim, dstate), torch.float32, dev)
    plan = ScanPlan(chunk_len, state_split, carry, halves, 0)
    with torch.cuda.device(dev):
        st = lib.ssm_scan_fwd_noalloc(batch, seqlen, dim, dstate, _DTYPES[dt], _ptr(x),
                                      _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                      _ptr(h0), _ptr(y), _ptr(hL),
                                      _options(delta_bias, delta_softplus), ctypes.byref(plan),
                                      _stream(dev))
    _check(st, "ssm_scan_fwd_noalloc")
    return y, hL


def scan_bwd(x, delta, A, B, C, D=None, z=None, h0=None, *, dy, dhL=None, delta_bias=None,
             delta_softplus=False, want_dh0=True, halves=HALVES_AUTO, chunk_len=0):
    """Gradients of sum(dy * y) + sum(dhL * hL) for the scan_fwd call with the
    same inputs. Returns a dict: dx, ddelta, dz (like x, I/O dtype); dB, dC
    (batch, L, N) fp32; dA (dim, N) fp32; dD, ddelta_bias (dim,) fp32; dh0
    (batch, dim, N) fp32. Entries of absent optional inputs are None.
    `halves` is the number of the last channel groups run as two 32-channel
    halves (HALVES_AUTO: the library's choice, HALVES_NONE: none; N 13..16);
    `chunk_len` > 0 (a multiple of 8) cuts the sequence into chunks that run
    in parallel (0: the library's choice)."""
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (batch, L, dim)")
    batch, seqlen, dim = x.shape
    if A.dim() != 2 or A.shape[0] != dim:
        raise ValueError("A must be (dim, N)")
    dstate = A.shape[1]
    dev, dt = x.device, x.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported I/O dtype {dt}")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    _need(x, "x", (batch, seqlen, dim), dt, dev)
    _need(delta, "delta", (batch, seqlen, dim), dt, dev)
    _need(A, "A", (dim, dstate), torch.float32, dev)
    _need(B, "B", (batch, seqlen, dstate), dt, dev)
    _need(C, "C", (batch, seqlen, dstate), dt, dev)
    _need(D, "D", (dim,), torch.float32, dev)
    _need(z, "z", (batch, seqlen, dim), dt, dev)
    _need(h0, "h0", (batch, dim, dstate), torch.float32, dev)
    _need(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    _need(dy, "dy", (batch, seqlen, dim), dt, dev)
    _need(dhL, "dhL", (batch, dim, dstate), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dx=torch.empty_like(x), ddelta=torch.empty_like(x),
             dA=torch.empty(dim, dstate, **f32), dB=torch.empty(batch, seqlen, dstate, **f32),
             dC=torch.empty(batch, seqlen, dstate, **f32),
             dD=None if D is None else torch.empty(dim, **f32),
             dz=None if z is None else torch.empty_like(x),
             dh0=torch.empty(batch, dim, dstate, **f32) if want_dh0 else None,
             ddelta_bias=None if delta_bias is None else torch.empty(dim, **f32))
    with torch.cuda.device(dev):
        plan = ScanPlan(chunk_len, 0, 0, halves, 0)
        nbytes = ctypes.c_size_t(0)
        _check(lib.ssm_scan_bwd_workspace_size(batch, seqlen, dim, dstate, _DTYPES[dt],
                                               ctypes.byref(plan), None, ctypes.byref(nbytes)),
               "ssm_scan_bwd_workspace_size")
        ws = _workspace(dev, nbytes.value, "bwd")
        st = lib.ssm_scan_bwd(batch, seqlen, dim, dstate, _DTYPES[dt], _ptr(x), _ptr(delta),
                              _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                              _options(delta_bias, delta_softplus),
                              ctypes.byref(plan), _ptr(dy), _ptr(dhL),
                              _ptr(g["dx"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]),
                              _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]),
                              _ptr(g["ddelta_bias"]), _ptr(ws), nbytes.value, _stream(dev))
    _check(st, "ssm_scan_bwd")
    return g


def state_update(h, x, delta, A, B, C, D=None, z=None, *, delta_bias=None,
                 delta_softplus=False, out=None):
    """One decode step: h (batch, dim, N) fp32 is updated in place; returns y
    (batch, dim). delta_bias and delta_softplus act as in scan_fwd."""
    lib = load_library()
    if h.dim() != 3:
        raise ValueError("h must be (batch, dim, N)")
    batch, dim, dstate = h.shape
    dev, dt = x.device, x.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported I/O dtype {dt}")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    _need(h, "h", (batch, dim, dstate), torch.float32, dev)
    _need(x, "x", (batch, dim), dt, dev)
    _need(delta, "delta", (batch, dim), dt, dev)
    _need(A, "A", (dim, dstate), torch.float32, dev)
    _need(B, "B", (batch, dstate), dt, dev)
    _need(C, "C", (batch, dstate), dt, dev)
    _need(D, "D", (dim,), torch.float32, dev)
    _need(z, "z", (batch, dim), dt, dev)
    _need(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    y = out if out is not None else torch.empty_like(x)
    _need(y, "out", (batch, dim), dt, dev)
    with torch.cuda.device(dev):
        st = lib.ssm_state_update(batch, dim, dstate, _DTYPES[dt], _ptr(h), _ptr(x), _ptr(delta),
                                  _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y),
                                  _options(delta_bias, delta_softplus), _stream(dev))
    _check(st, "ssm_state_update")
    return y


def conv1d_fwd(x, weight, bias=None, state_in=None, *, silu=True, return_state=True, out=None,
               state_out=None):
    """Short causal depthwise convolution over whole sequences; returns
    (y, state_out) where state_out (batch, dim, W) holds the last W inputs
    (None when return_state is False). state_in (batch, dim, W), in the dtype
    of x, holds the W inputs before the sequence (None: zeros); state_out may
    be the same tensor."""
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (batch, L, dim)")
    batch, seqlen, dim = x.shape
    if weight.dim() != 2 or weight.shape[0] != dim:
        raise ValueError("weight must be (dim, W)")
    width = weight.shape[1]
    dev, dt = x.device, x.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported I/O dtype {dt}")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    _need(x, "x", (batch, seqlen, dim), dt, dev)
    _need(weight, "weight", (dim, width), torch.float32, dev)
    _need(bias, "bias", (dim,), torch.float32, dev)
    _need(state_in, "state_in", (batch, dim, width), dt, dev)
    y = out if out is not None else torch.empty_like(x)
    _need(y, "out", (batch, seqlen, dim), dt, dev)
    st = None
    if return_state:
        st = state_out if state_out is not None else torch.empty(batch, dim, width, dtype=dt,
                                                                 device=dev)
        _need(st, "state_out", (batch, dim, width), dt, dev)
    with torch.cuda.device(dev):
        rc = lib.causal_conv1d_fwd(batch, seqlen, dim, width, _DTYPES[dt], _ptr(x), _ptr(weight),
                                   _ptr(bias), _ptr(state_in), _ptr(y), _ptr(st),
                                   1 if silu else 0, _stream(dev))
    _check(rc, "causal_conv1d_fwd")
    return y, st


def conv1d_update(state, x, weight, bias=None, *, silu=True, out=None):
    """One decode step of the convolution: state (batch, dim, W), in the
    dtype of x, is updated in place; returns y (batch, dim)."""
    lib = load_library()
    if state.dim() != 3:
        raise ValueError("state must be (batch, dim, W)")
    batch, dim, width = state.shape
    dev, dt = x.device, x.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported I/O dtype {dt}")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    _need(state, "state", (batch, dim, width), dt, dev)
    _need(x, "x", (batch, dim), dt, dev)
    _need(weight, "weight", (dim, width), torch.float32, dev)
    _need(bias, "bias", (dim,), torch.float32, dev)
    y = out if out is not None else torch.empty_like(x)
    _need(y, "out", (batch, dim), dt, dev)
    with torch.cuda.device(dev):
        rc = lib.causal_conv1d_update(batch, dim, width, _DTYPES[dt], _ptr(state), _ptr(x),
                                      _ptr(weight), _ptr(bias), _ptr(y), 1 if silu else 0,
                                      _stream(dev))
    _check(rc, "causal_conv1d_update")
    return y


SSD_HEADDIM = 64


def ssd_fwd(x, dt, A, B, C, D=None, z=None, h0=None, *, dt_bias=None, dt_softplus=False,
            return_state=True, out=None, state_out=None):
    """Mamba-2 dual form: heads of 64 channels share the step dt (batch, L,
    nheads) and the decay a_h (A: (nheads,) fp32). x, z (batch, L, nheads*64)
    and B, C (batch, L, N) are bf16; N is 64 or 128. Returns (y, hL) with
    hL (batch, nheads, 64, N) fp32 (None when return_state is False)."""
    lib = load_library()
    if x.dim() != 3 or dt.dim() != 3:
        raise ValueError("x must be (batch, L, nheads*64) and dt (batch, L, nheads)")
    batch, seqlen, dim = x.shape
    nheads = dt.shape[2]
    if dim != nheads * SSD_HEADDIM:
        raise ValueError(f"x has {dim} channels, expected nheads*{SSD_HEADDIM}")
    dstate = B.shape[2]
    dev, dtp = x.device, x.dtype
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    _need(x, "x", (batch, seqlen, dim), dtp, dev)
    _need(dt, "dt", (batch, seqlen, nheads), dtp, dev)
    _need(A, "A", (nheads,), torch.float32, dev)
    _need(B, "B", (batch, seqlen, dstate), dtp, dev)
    _need(C, "C", (batch, seqlen, dstate), dtp, dev)
    _need(D, "D", (dim,), torch.float32, dev)
    _need(z, "z", (batch, seqlen, dim), dtp, dev)
    _need(h0, "h0", (batch, nheads, SSD_HEADDIM, dstate), torch.float32, dev)
    _need(dt_bias, "dt_bias", (nheads,), torch.float32, dev)
    y = out if out is not None else torch.empty_like(x)
    _need(y, "out", (batch, seqlen, dim), dtp, dev)
    hL = None
    if return_state:
        hL = state_out if state_out is not None else torch.empty(
            batch, nheads, SSD_HEADDIM, dstate, dtype=torch.float32, device=dev)
        _need(hL, "state_out", (batch, nheads, SSD_HEADDIM, dstate), torch.float32, dev)
    with torch.cuda.device(dev):
        st = lib.ssd_fwd(batch, seqlen, nheads, SSD_HEADDIM, dstate, _DTYPES.get(dtp, -1),
                         _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                         _ptr(h0), _ptr(y), _ptr(hL), _options(dt_bias, dt_softplus),
                         _stream(dev))
    _check(st, "ssd_fwd")
    return y, hL
