"""Seeded synthetic inputs for the selective-scan workloads.

This module draws random tensors and nothing else: it holds none of the
scan's arithmetic, and both the GPU library's tests and the CPU oracle take
their inputs from it. Every tensor comes from a seeded torch generator, on the
device the caller names, with the shape, dtype and distribution of one
workload. The shapes are the layer shapes of the page "Mamba and State Space
Models" (world.lapla.si): 5,120 channels of 16 states for Mamba-2.8B, 64
layers (section "A State of Fixed Size"), A running from -1 to -16 (section
"Every Step the Same"), 2,048-token training context (section "What It Does
Not Say") and million-token sequences (section "Remembering Selectively").

Recipe shared by every workload:
  - A (dim, N) fp32: "logunif" draws A = -exp(U(-1, 1)); "s4d_real" sets
    A[d, n] = -(n + 1) for every channel.
  - D (dim,) fp32 ~ N(0, 1).
  - delta = softplus(N(0, 1) * delta_std + delta_shift), computed in fp32 and
    then rounded to the I/O dtype (round to nearest even).
  - x, z, B, C ~ N(0, 1), drawn in fp32 and rounded to the I/O dtype.
  - h0: None (zero state) or N(0, 1) fp32.
Draw order: A, D, x, delta, z, B, C, h0.

With raw_delta=True the inputs are those of a call that leaves the delta
activation to the kernels: delta is the pre-activation N(0, 1) * delta_std
(rounded to the I/O dtype) and delta_bias (dim,) fp32 is
delta_shift + N(0, 1) * 0.5, drawn last; softplus(delta + delta_bias) then
has the distribution of the default recipe's delta, give or take the
per-channel spread.
"""
from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "WORKLOADS", "generate_scan", "generate_decode_layer",
           "io_torch_dtype", "ConvWorkload", "CONV_WORKLOADS", "generate_conv",
           "generate_conv_decode_layer", "SsdWorkload", "SSD_WORKLOADS", "generate_ssd"]


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "scan" or "decode"
    batch: int
    seqlen: int          # tokens per sequence (1 for decode)
    dim: int             # channels D
    dstate: int          # states per channel N
    io: str              # "f32" or "bf16": dtype of x, delta, z, B, C, y
    a_init: str          # "logunif" or "s4d_real"
    delta_shift: float
    delta_std: float
    h0: str              # "zero" or "normal"
    seed: int
    layers: int = 1      # decode only: independent layers per step
    note: str = field(default="", compare=False)

    @property
    def elements(self):
        """Scan elements B*L*D (decode: per step over all layers)."""
        return self.batch * self.seqlen * self.dim * self.layers


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", "scan", 1, 64, 16, 4, "f32", "logunif", -2.0, 1.0, "zero", 0,
        note="tiny fp32 scan the oracle checks in milliseconds"),
    "mamba130m_layer": Workload(
        "mamba130m_layer", "scan", 8, 2048, 1536, 16, "bf16", "logunif", -4.0, 1.0, "zero", 1,
        note="Mamba-130M-shaped layer scan"),
    "mamba28b_layer": Workload(
        "mamba28b_layer", "scan", 8, 2048, 5120, 16, "bf16", "s4d_real", -4.0, 0.5, "zero", 2,
        note="Mamba-2.8B-shaped layer scan"),
    "million_length": Workload(
        "million_length", "scan", 1, 1 << 20, 2048, 16, "bf16", "s4d_real", -4.0, 0.5, "zero", 3,
        note="million-token scan at batch 1"),
    "decode_64layer": Workload(
        "decode_64layer", "decode", 256, 1, 5120, 16, "bf16", "s4d_real", -4.0, 0.5, "normal", 4,
        layers=64, note="single-token state update, batch 256, 64 layers of D=5120"),
}


def io_torch_dtype(io):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[io]


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, g, device, dtype, mean=0.0, std=1.0, chunk=1 << 27):
    """N(mean, std) drawn in fp32 and rounded to `dtype`, in slabs along dim 0
    so very large tensors never need a full fp32 temporary."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            v.mul_(std)
        if mean != 0.0:
            v.add_(mean)
        flat[s:e] = v.to(dtype)
    return out


def _softplus_normal(shape, g, device, dtype, mean, std, chunk=1 << 27):
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        v = torch.nn.functional.softplus(v * std + mean)
        flat[s:e] = v.to(dtype)
    return out


def _a_matrix(w, g, device, dim=None):
    dim = w.dim if dim is None else dim
    if w.a_init == "s4d_real":
        row = -torch.arange(1, w.dstate + 1, dtype=torch.float32, device=device)
        return row.expand(dim, w.dstate).contiguous()
    if w.a_init == "logunif":
        u = torch.rand(dim, w.dstate, generator=g, device=device, dtype=torch.float32)
        return -torch.exp(u * 2.0 - 1.0)
    raise ValueError(w.a_init)


def generate_scan(w, device="cpu", batch=None, seqlen=None, dim=None, seed=None,
                  raw_delta=False):
    """Inputs for one scan call of workload `w` (sizes may be overridden for
    small parity cases). Returns a dict with keys x, delta, A, B, C, D, z, h0
    (and delta_bias with raw_delta=True)."""
    batch = w.batch if batch is None else batch
    seqlen = w.seqlen if seqlen is None else seqlen
    dim = w.dim if dim is None else dim
    seed = w.seed if seed is None else seed
    dt = io_torch_dtype(w.io)
    g = _gen(seed, device)
    A = _a_matrix(w, g, device, dim)
    D = torch.randn(dim, generator=g, device=device, dtype=torch.float32)
    x = _normal((batch, seqlen, dim), g, device, dt)
    if raw_delta:
        delta = _normal((batch, seqlen, dim), g, device, dt, std=w.delta_std)
    else:
        delta = _softplus_normal((batch, seqlen, dim), g, device, dt, w.delta_shift, w.delta_std)
    z = _normal((batch, seqlen, dim), g, device, dt)
    B = _normal((batch, seqlen, w.dstate), g, device, dt)
    C = _normal((batch, seqlen, w.dstate), g, device, dt)
    h0 = None
    if w.h0 == "normal":
        h0 = torch.randn(batch, dim, w.dstate, generator=g, device=device, dtype=torch.float32)
    out = dict(x=x, delta=delta, A=A, B=B, C=C, D=D, z=z, h0=h0)
    if raw_delta:
        out["delta_bias"] = _bias(dim, g, device, w.delta_shift)
    return out


def _bias(dim, g, device, shift):
    return torch.randn(dim, generator=g, device=device, dtype=torch.float32) * 0.5 + shift


def generate_decode_layer(w, layer, device="cpu", batch=None, dim=None, raw_delta=False):
    """Inputs of one layer of a decode step: h (batch, dim, N) fp32 state and
    one token of x, delta, z (batch, dim) and B, C (batch, N) (and
    delta_bias with raw_delta=True, as in generate_scan)."""
    batch = w.batch if batch is None else batch
    dim = w.dim if dim is None else dim
    dt = io_torch_dtype(w.io)
    g = _gen(w.seed * 1000003 + layer, device)
    A = _a_matrix(w, g, device, dim)
    D = torch.randn(dim, generator=g, device=device, dtype=torch.float32)
    x = _normal((batch, dim), g, device, dt)
    if raw_delta:
        delta = _normal((batch, dim), g, device, dt, std=w.delta_std)
    else:
        delta = _softplus_normal((batch, dim), g, device, dt, w.delta_shift, w.delta_std)
    z = _normal((batch, dim), g, device, dt)
    B = _normal((batch, w.dstate), g, device, dt)
    C = _normal((batch, w.dstate), g, device, dt)
    h = torch.randn(batch, dim, w.dstate, generator=g, device=device, dtype=torch.float32)
    out = dict(h=h, x=x, delta=delta, A=A, B=B, C=C, D=D, z=z)
    if raw_delta:
        out["delta_bias"] = _bias(dim, g, device, w.delta_shift)
    return out


# ---------------------------------------------------------------------------
# Short causal convolution workloads. The pages give the convolution's width
# (the last 4 inputs of each channel, section "A State of Fixed Size") and
# the Mamba-2.8B channel count, not its weights; the recipe:
#   - weight (dim, W) and bias (dim,) fp32 ~ U(-1/sqrt(W), 1/sqrt(W)), the
#     usual fan-in bound of a depthwise filter of W taps;
#   - x ~ N(0, 1), drawn in fp32 and rounded to the I/O dtype;
#   - carried state (batch, dim, W) in the I/O dtype: zeros for a sequence
#     that starts fresh, N(0, 1) for decode.
# Draw order: weight, bias, x, state.


@dataclass(frozen=True)
class ConvWorkload:
    name: str
    kind: str            # "conv" or "conv_decode"
    batch: int
    seqlen: int
    dim: int
    width: int
    io: str
    state: str           # "zero" or "normal": the carried inputs before the sequence
    seed: int
    layers: int = 1
    note: str = field(default="", compare=False)

    @property
    def elements(self):
        return self.batch * self.seqlen * self.dim * self.layers


CONV_WORKLOADS = {
    "conv_mamba28b_layer": ConvWorkload(
        "conv_mamba28b_layer", "conv", 8, 2048, 5120, 4, "bf16", "zero", 5,
        note="short convolution + silu over a Mamba-2.8B-shaped layer input"),
    "conv_decode_64layer": ConvWorkload(
        "conv_decode_64layer", "conv_decode", 256, 1, 5120, 4, "bf16", "normal", 6, layers=64,
        note="convolution decode step, batch 256, 64 layers of D=5120"),
}


def _taps(w, g, device, dim):
    bound = 1.0 / float(w.width) ** 0.5
    weight = (torch.rand(dim, w.width, generator=g, device=device) * 2.0 - 1.0) * bound
    bias = (torch.rand(dim, generator=g, device=device) * 2.0 - 1.0) * bound
    return weight, bias


def generate_conv(w, device="cpu", batch=None, seqlen=None, dim=None, seed=None, state=None):
    """Inputs of one convolution call: x, weight, bias, state_in (None for a
    fresh sequence)."""
    batch = w.batch if batch is None else batch
    seqlen = w.seqlen if seqlen is None else seqlen
    dim = w.dim if dim is None else dim
    seed = w.seed if seed is None else seed
    state = w.state if state is None else state
    dt = io_torch_dtype(w.io)
    g = _gen(seed, device)
    weight, bias = _taps(w, g, device, dim)
    x = _normal((batch, seqlen, dim), g, device, dt)
    st = _normal((batch, dim, w.width), g, device, dt) if state == "normal" else None
    return dict(x=x, weight=weight, bias=bias, state_in=st)


def generate_conv_decode_layer(w, layer, device="cpu", batch=None, dim=None):
    """One layer of a convolution decode step: state (batch, dim, W), x
    (batch, dim), weight, bias."""
    batch = w.batch if batch is None else batch
    dim = w.dim if dim is None else dim
    dt = io_torch_dtype(w.io)
    g = _gen(w.seed * 1000003 + layer, device)
    weight, bias = _taps(w, g, device, dim)
    x = _normal((batch, dim), g, device, dt)
    st = _normal((batch, dim, w.width), g, device, dt)
    return dict(state=st, x=x, weight=weight, bias=bias)


# ---------------------------------------------------------------------------
# Mamba-2 dual-form workloads (section "Mamba-2: Two Algorithms": one decay
# per head, 128 numbers of state per channel). The pages give the state size,
# not the head size; heads of 64 channels are the reading used (the channel
# count is the Mamba-2.8B layer's 5,120, so 80 heads). Recipe:
#   - A (nheads,) fp32 = -U(1, 16), the -1 .. -16 range of section "Every
#     Step the Same" spread over the heads;
#   - dt (batch, L, nheads) = softplus(N(0, 1) * delta_std + delta_shift) in
#     fp32, rounded to bf16; raw_dt=True gives N(0, 1) * delta_std and a
#     per-head bias delta_shift + N(0, 1) * 0.5 (drawn last) instead;
#   - x, z, B, C ~ N(0, 1) rounded to bf16; D (nheads*64,) fp32 ~ N(0, 1);
#   - h0: zeros, or N(0, 1) fp32 (batch, nheads, 64, N).
# Draw order: A, D, x, dt, z, B, C, h0.


@dataclass(frozen=True)
class SsdWorkload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    dstate: int
    delta_shift: float
    delta_std: float
    h0: str
    seed: int
    headdim: int = 64
    io: str = "bf16"
    note: str = field(default="", compare=False)

    @property
    def dim(self):
        return self.nheads * self.headdim

    @property
    def elements(self):
        return self.batch * self.seqlen * self.dim


SSD_WORKLOADS = {
    "ssd_mamba2_layer": SsdWorkload(
        "ssd_mamba2_layer", 8, 2048, 80, 128, -4.0, 0.5, "zero", 7,
        note="Mamba-2 dual form over a 5,120-channel layer, 80 heads of 64, state 128"),
}


def generate_ssd(w, device="cpu", batch=None, seqlen=None, nheads=None, dstate=None, seed=None,
                 h0=None, raw_dt=False):
    """Inputs of one ssd_fwd call: x, dt, A, B, C, D, z, h0 (and dt_bias with
    raw_dt=True)."""
    batch = w.batch if batch is None else batch
    seqlen = w.seqlen if seqlen is None else seqlen
    nheads = w.nheads if nheads is None else nheads
    dstate = w.dstate if dstate is None else dstate
    seed = w.seed if seed is None else seed
    h0 = w.h0 if h0 is None else h0
    dt_ = io_torch_dtype(w.io)
    dim = nheads * w.headdim
    g = _gen(seed, device)
    A = -(1.0 + 15.0 * torch.rand(nheads, generator=g, device=device, dtype=torch.float32))
    D = torch.randn(dim, generator=g, device=device, dtype=torch.float32)
    x = _normal((batch, seqlen, dim), g, device, dt_)
    if raw_dt:
        dt = _normal((batch, seqlen, nheads), g, device, dt_, std=w.delta_std)
    else:
        dt = _softplus_normal((batch, seqlen, nheads), g, device, dt_, w.delta_shift, w.delta_std)
    z = _normal((batch, seqlen, dim), g, device, dt_)
    B = _normal((batch, seqlen, dstate), g, device, dt_)
    C = _normal((batch, seqlen, dstate), g, device, dt_)
    hs = None
    if h0 == "normal":
        hs = torch.randn(batch, nheads, w.headdim, dstate, generator=g, device=device,
                         dtype=torch.float32)
    out = dict(x=x, dt=dt, A=A, B=B, C=C, D=D, z=z, h0=hs)
    if raw_dt:
        out["dt_bias"] = _bias(nheads, g, device, w.delta_shift)
    return out
