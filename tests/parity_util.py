"""Helpers shared by the GPU parity tests: tolerances, comparisons and
channel-sampled oracle runs. Holds no scan arithmetic."""
import numpy as np
import torch

# Max abs error allowed, relative to the largest |value| the oracle produces
# for the same output tensor: fp32 I/O 1e-5, bf16 I/O (fp32 state) 2e-2.
TOL = {"f32": 1e-5, "bf16": 2e-2, torch.float32: 1e-5, torch.bfloat16: 2e-2}


def to_f64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def assert_close(got, want, tol, what):
    g, w = to_f64(got), to_f64(want)
    assert g.shape == w.shape, f"{what}: shape {g.shape} vs {w.shape}"
    if w.size == 0:
        return
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    scale = float(np.max(np.abs(w)))
    err = float(np.max(np.abs(g - w)))
    assert err <= tol * scale, f"{what}: max abs error {err:.3e} > {tol:g} * {scale:.3e}"
    return err / scale if scale else 0.0


def sample_channels(dim, count=24, seed=0):
    """Channel indices that cover the first, last and wave-boundary channels
    plus a seeded random spread."""
    fixed = [0, 1, 63, 64, 65, 127, dim // 2, dim - 65, dim - 64, dim - 2, dim - 1]
    rng = np.random.default_rng(seed)
    extra = rng.choice(dim, size=min(dim, count), replace=False).tolist()
    return sorted({c for c in fixed + extra if 0 <= c < dim})


def oracle_on_channels(orc, inp, idx):
    """The oracle over a subset of channels (channels are independent).
    Inputs that carry a delta_bias are raw-delta inputs (ssm_workloads'
    raw_delta=True) and run with the softplus activation."""
    ix = torch.as_tensor(idx, dtype=torch.long, device=inp["x"].device)
    sub = dict(
        x=inp["x"].index_select(2, ix), delta=inp["delta"].index_select(2, ix),
        A=inp["A"].index_select(0, ix), B=inp["B"], C=inp["C"],
        D=None if inp.get("D") is None else inp["D"].index_select(0, ix),
        z=None if inp.get("z") is None else inp["z"].index_select(2, ix),
        h0=None if inp.get("h0") is None else inp["h0"].index_select(1, ix),
        delta_bias=(None if inp.get("delta_bias") is None
                    else inp["delta_bias"].index_select(0, ix)))
    return orc.scan_fwd(**sub, delta_softplus=inp.get("delta_bias") is not None)
