"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each pin takes an oracle handle (``oracle.Oracle``) and raises AssertionError
when it disagrees with an independent statement of the result:

- pin_lti_convolution: with Delta, B and C constant over time the scan is a
  convolution of x with one fixed kernel K_k = sum_n C_n Abar_n^k Delta B_n
  (page "Mamba and State Space Models", section "Every Step the Same"),
  evaluated with numpy's convolve, plus the closed-form decay of h0.
- pin_brute_force: for sequences of at most 8 tokens, the unrolled solution
  h_t = exp(A*S_(0..t)) h0 + sum_s exp(A*(S_t - S_s)) Delta_s B_s x_s,
  with S the running sum of Delta (section "A State of Fixed Size" unrolled).
- pin_chunk_split: scanning [0, L) equals scanning [0, m) and then [m, L)
  from the carried state, bit for bit (the state is the whole memory,
  section "A State of Fixed Size").
- pin_theorem1: with one state, A = -1, B = C = 1 and Delta = softplus(u),
  zero-order hold gives exactly the gated recurrence h <- (1-g)h + g*x with
  g = sigmoid(u) (section "Chosen by the Token", the paper's Theorem 1); the
  first-order form gives h <- (1-g)h + softplus(u)*x.
- pin_ssd_matrix: for A a scalar per channel, the whole sequence map is one
  lower-triangular matrix with entry (i, j) = (C_i . B_j) times the decay
  from j to i (section "Mamba-2: Two Algorithms"), applied with a numpy
  matmul to Delta*x.
- pin_limits: Delta -> 0 keeps the state; a large Delta resets it to
  Delta*B*x; x = 0 leaves pure decay (section "Chosen by the Token").
- pin_structure: linearity in x, superposition of x and h0, the exact skip
  contribution D*x*silu(z), channel permutation and batch independence.
- pin_decode: the single-token update equals the scan over one token, and
  T updates equal the scan over T tokens (section "Taken Apart").
- pin_delta_activation: delta given before its activation. With one state,
  A ~ 0 and x = B = C = 1 the first output is delta itself, which must equal
  softplus(delta_raw + bias) as numpy's logaddexp(0, .) computes it; and the
  Theorem 1 gate identity holds with the softplus applied inside the scan.
- pin_conv_numpy: the short causal convolution (section "A State of Fixed
  Size": the last 4 inputs of each channel) equals numpy's convolve of the
  carried inputs followed by the sequence with the reversed taps, plus the
  bias, through scipy's logistic silu; the state it hands on is the last W
  inputs of that same concatenation.
- pin_conv_impulse: a unit impulse at token t0 (zero carried state) reads
  out the taps newest-first: pre[t0 + j] = bias + weight[W-1-j], bias
  elsewhere.
- pin_bwd_finite_differences: every gradient the backward pass returns
  (x, delta, A, B, C, D, z, h0, and the raw delta and its bias under the
  fused softplus) equals central differences of the forward scan's loss
  sum(dy * y) + sum(dhL * hL) in fp64, entry by entry (section "A Scan on
  the Chip": training runs a backward pass through the same recurrence).
- pin_bwd_linearity: the gradients are linear in (dy, dhL), and with dy = 0
  and dhL = 0 they all vanish.
- pin_ssd_dual_matrix: Mamba-2's form with one decay per head (section
  "Mamba-2: Two Algorithms") equals the whole-sequence lower-triangular
  matrix M[i, j] = (C_i . B_j) exp(a (S_i - S_j)), S the running sum of dt,
  applied to dt * x as one numpy matmul per head ("masked attention" with C
  as queries and B as keys), plus the decayed initial state.
- pin_ssd_chunked: the same result from the chunked algorithm the section
  describes: matrix products inside each chunk and only the state passed
  from chunk to chunk, for several chunk lengths.
- pin_ssd_heads_of_one: with one channel per head the dual form is the
  selective scan with A[d, n] = a_d for every n.
- pin_conv_split_and_decode: convolving [0, L) equals [0, m) then [m, L)
  from the handed-on state, bit for bit, and T decode steps equal the
  convolution over T tokens.

silu(z) = z * sigmoid(z) is evaluated with scipy's logistic function.
"""
import numpy as np
from scipy.special import expit

RTOL = 1e-12


def _silu(z):
    return z * expit(z)


def _close(got, want, rtol=RTOL, what=""):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    if want.size == 0:
        return
    scale = max(1.0, float(np.max(np.abs(want))))
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    assert err <= rtol * scale, f"{what}: max abs error {err:.3e} > {rtol:.1e} * {scale:.3e}"


def _rand_inputs(rng, batch, seqlen, dim, dstate, h0=True):
    x = rng.standard_normal((batch, seqlen, dim))
    delta = np.log1p(np.exp(rng.standard_normal((batch, seqlen, dim)) - 1.0))
    A = -np.exp(rng.uniform(-1.0, 1.0, (dim, dstate)))
    B = rng.standard_normal((batch, seqlen, dstate))
    C = rng.standard_normal((batch, seqlen, dstate))
    D = rng.standard_normal(dim)
    z = rng.standard_normal((batch, seqlen, dim))
    h = rng.standard_normal((batch, dim, dstate)) if h0 else None
    return dict(x=x, delta=delta, A=A, B=B, C=C, D=D, z=z, h0=h)


def pin_lti_convolution(orc, seed=11):
    rng = np.random.default_rng(seed)
    batch, L, dim, N = 2, 48, 5, 3
    dconst = 0.05 + rng.uniform(0.0, 0.6, dim)           # one Delta per channel
    A = -np.exp(rng.uniform(-1.0, 1.0, (dim, N)))
    Bc = rng.standard_normal((batch, N))                  # one B, one C per batch
    Cc = rng.standard_normal((batch, N))
    x = rng.standard_normal((batch, L, dim))
    z = rng.standard_normal((batch, L, dim))
    D = rng.standard_normal(dim)
    h0 = rng.standard_normal((batch, dim, N))
    delta = np.broadcast_to(dconst, (batch, L, dim)).copy()
    B = np.broadcast_to(Bc[:, None, :], (batch, L, N)).copy()
    C = np.broadcast_to(Cc[:, None, :], (batch, L, N)).copy()
    y, hL = orc.scan_fwd(x, delta, A, B, C, D=D, z=z, h0=h0)

    k = np.arange(L)
    want_y = np.empty((batch, L, dim))
    want_h = np.empty((batch, dim, N))
    for b in range(batch):
        for d in range(dim):
            powers = np.exp(np.outer(k, dconst[d] * A[d]))          # Abar^k, (L, N)
            kernel = powers @ (Cc[b] * dconst[d] * Bc[b])           # K_k
            conv = np.convolve(x[b, :, d], kernel)[:L]
            init = np.exp(np.outer(k + 1, dconst[d] * A[d])) @ (Cc[b] * h0[b, d])
            pre = conv + init + D[d] * x[b, :, d]
            want_y[b, :, d] = pre * _silu(z[b, :, d])
            rev = x[b, ::-1, d]                                       # x_{L-1-k}
            want_h[b, d] = (powers * (dconst[d] * Bc[b])).T @ rev + np.exp(L * dconst[d] * A[d]) * h0[b, d]
    _close(y, want_y, what="LTI y")
    _close(hL, want_h, what="LTI hL")


def pin_brute_force(orc, seed=12):
    rng = np.random.default_rng(seed)
    for L in range(1, 9):
        inp = _rand_inputs(rng, 2, L, 3, 4)
        x, dl, A, B, C, D, z, h0 = (inp[k] for k in ("x", "delta", "A", "B", "C", "D", "z", "h0"))
        y, hL = orc.scan_fwd(**inp)
        want = np.empty_like(y)
        want_h = np.empty_like(hL)
        for b in range(2):
            for d in range(3):
                S = np.cumsum(dl[b, :, d])
                for t in range(L):
                    h = np.exp(A[d] * S[t]) * h0[b, d]
                    for s in range(t + 1):
                        h = h + np.exp(A[d] * (S[t] - S[s])) * dl[b, s, d] * B[b, s] * x[b, s, d]
                    pre = float(np.dot(C[b, t], h)) + D[d] * x[b, t, d]
                    want[b, t, d] = pre * _silu(z[b, t, d])
                    if t == L - 1:
                        want_h[b, d] = h
        _close(y, want, rtol=1e-11, what=f"brute force y, L={L}")
        _close(hL, want_h, rtol=1e-11, what=f"brute force hL, L={L}")


def pin_chunk_split(orc, seed=13):
    rng = np.random.default_rng(seed)
    inp = _rand_inputs(rng, 3, 37, 4, 5)
    y, hL = orc.scan_fwd(**inp)
    for m in (0, 1, 7, 20, 36, 37):
        first = {k: (v[:, :m] if k in ("x", "delta", "B", "C", "z") else v) for k, v in inp.items()}
        second = {k: (v[:, m:] if k in ("x", "delta", "B", "C", "z") else v) for k, v in inp.items()}
        y1, h1 = orc.scan_fwd(**first)
        second["h0"] = h1
        y2, h2 = orc.scan_fwd(**second)
        assert np.array_equal(np.concatenate([y1, y2], axis=1), y), f"split at {m}: y differs"
        assert np.array_equal(h2, hL), f"split at {m}: hL differs"


def pin_theorem1(orc, seed=14):
    rng = np.random.default_rng(seed)
    batch, L, dim = 2, 30, 3
    u = 2.0 * rng.standard_normal((batch, L, dim))
    x = rng.standard_normal((batch, L, dim))
    delta = np.logaddexp(0.0, u)                  # softplus(u)
    A = -np.ones((dim, 1))
    ones = np.ones((batch, L, 1))
    h0 = rng.standard_normal((batch, dim, 1))
    for zoh in (True, False):
        y, hL = orc.scan_fwd(x, delta, A, ones, ones, h0=h0, zoh=zoh)
        want = np.empty_like(y)
        for b in range(batch):
            for d in range(dim):
                h = h0[b, d, 0]
                for t in range(L):
                    g = expit(u[b, t, d])
                    write = g if zoh else delta[b, t, d]
                    h = (1.0 - g) * h + write * x[b, t, d]
                    want[b, t, d] = h
        _close(y, want, what=f"Theorem 1 gate (zoh={zoh})")
        _close(hL[:, :, 0], want[:, -1, :], what=f"Theorem 1 state (zoh={zoh})")


def pin_ssd_matrix(orc, seed=15):
    rng = np.random.default_rng(seed)
    batch, L, dim, N = 2, 33, 4, 6
    inp = _rand_inputs(rng, batch, L, dim, N, h0=False)
    a = -np.exp(rng.uniform(-1.0, 1.0, dim))
    inp["A"] = np.repeat(a[:, None], N, axis=1)
    y, hL = orc.scan_fwd(**inp)
    x, dl, B, C, D, z = (inp[k] for k in ("x", "delta", "B", "C", "D", "z"))
    mask = np.tril(np.ones((L, L), dtype=bool))
    for b in range(batch):
        for d in range(dim):
            S = np.cumsum(dl[b, :, d])
            gap = np.where(mask, S[:, None] - S[None, :], 0.0)
            M = (C[b] @ B[b].T) * np.exp(a[d] * gap) * mask
            v = dl[b, :, d] * x[b, :, d]
            pre = M @ v + D[d] * x[b, :, d]
            _close(y[b, :, d], pre * _silu(z[b, :, d]), what="SSD matrix form y")
            decay = np.exp(a[d] * (S[-1] - S))
            _close(hL[b, d], B[b].T @ (decay * v), what="SSD matrix form hL")


def pin_limits(orc, seed=16):
    rng = np.random.default_rng(seed)
    inp = _rand_inputs(rng, 2, 12, 3, 4)
    x, B, C, D, z, h0 = (inp[k] for k in ("x", "B", "C", "D", "z", "h0"))
    # Delta -> 0: the state is kept, y = C.h0 + D x
    tiny = dict(inp, delta=np.full_like(x, 1e-14))
    y, hL = orc.scan_fwd(**tiny)
    want = (np.einsum("btn,bdn->btd", C, h0) + D * x) * _silu(z)
    _close(y, want, rtol=1e-10, what="Delta -> 0 keeps the state")
    _close(hL, h0, rtol=1e-10, what="Delta -> 0 final state")
    # large Delta with A <= -1: h_t = Delta * B_t * x_t (reset to the current token)
    big = dict(inp, delta=np.full_like(x, 60.0), A=-1.0 - rng.uniform(0, 1, inp["A"].shape))
    y, hL = orc.scan_fwd(**big)
    want = (60.0 * np.einsum("btn,btn->bt", C, B)[:, :, None] * x + D * x) * _silu(z)
    _close(y, want, rtol=1e-10, what="large Delta resets the state")
    # x = 0: pure decay of h0
    zero = dict(inp, x=np.zeros_like(x))
    y, hL = orc.scan_fwd(**zero)
    S = np.cumsum(inp["delta"], axis=1)                                   # (b, t, d)
    h = np.exp(S[:, :, :, None] * inp["A"][None, None]) * h0[:, None]     # (b, t, d, n)
    _close(y, np.einsum("btn,btdn->btd", C, h) * _silu(z), what="x = 0 decays h0")
    _close(hL, h[:, -1], what="x = 0 final state")


def pin_structure(orc, seed=17):
    rng = np.random.default_rng(seed)
    inp = _rand_inputs(rng, 3, 25, 6, 5)
    x2 = rng.standard_normal(inp["x"].shape)
    nozero = dict(inp, h0=None)
    y1, h1 = orc.scan_fwd(**nozero)
    y2, h2 = orc.scan_fwd(**dict(nozero, x=x2))
    y12, h12 = orc.scan_fwd(**dict(nozero, x=2.0 * inp["x"] - 3.0 * x2))
    _close(y12, 2.0 * y1 - 3.0 * y2, what="linearity in x")
    _close(h12, 2.0 * h1 - 3.0 * h2, what="linearity in x (state)")
    # superposition of input and initial state
    y, hL = orc.scan_fwd(**inp)
    y0, s0 = orc.scan_fwd(**dict(inp, x=np.zeros_like(inp["x"])))
    _close(y, y1 + y0, what="superposition of x and h0")
    _close(hL, h1 + s0, what="superposition of x and h0 (state)")
    # the skip term contributes exactly D * x * silu(z)
    ynd, _ = orc.scan_fwd(**dict(inp, D=None))
    _close(y - ynd, inp["D"] * inp["x"] * _silu(inp["z"]), what="skip term")
    # no gate: y is the ungated readout, and gating multiplies by silu(z)
    yng, _ = orc.scan_fwd(**dict(inp, z=None))
    _close(y, yng * _silu(inp["z"]), what="gate")
    # channels are independent: permuting them permutes the outputs
    p = rng.permutation(inp["x"].shape[2])
    perm = dict(inp, x=inp["x"][:, :, p], delta=inp["delta"][:, :, p], z=inp["z"][:, :, p],
                A=inp["A"][p], D=inp["D"][p], h0=inp["h0"][:, p])
    yp, hp = orc.scan_fwd(**perm)
    assert np.array_equal(yp, y[:, :, p]) and np.array_equal(hp, hL[:, p]), "channel permutation"
    # batches are independent
    yb, hb = orc.scan_fwd(**{k: (v[1:2] if k in ("x", "delta", "B", "C", "z", "h0") else v)
                             for k, v in inp.items()})
    assert np.array_equal(yb, y[1:2]) and np.array_equal(hb, hL[1:2]), "batch independence"


def pin_decode(orc, seed=18):
    rng = np.random.default_rng(seed)
    inp = _rand_inputs(rng, 3, 6, 5, 4)
    y, hL = orc.scan_fwd(**inp)
    h = inp["h0"].copy()
    for t in range(6):
        yt, h = orc.state_update(h, inp["x"][:, t], inp["delta"][:, t], inp["A"],
                                 inp["B"][:, t], inp["C"][:, t], D=inp["D"], z=inp["z"][:, t])
        assert np.array_equal(yt, y[:, t]), f"decode step {t} differs from the scan"
    assert np.array_equal(h, hL), "decode state after T steps differs from the scan"


def pin_delta_activation(orc, seed=19):
    rng = np.random.default_rng(seed)
    batch, dim = 40, 7
    u = np.concatenate([rng.uniform(-60.0, 60.0, (batch - 8, 1, dim)),
                        np.array([-800.0, -40.0, -1.0, 0.0, 1e-9, 1.0, 40.0, 800.0])
                        .reshape(8, 1, 1).repeat(dim, axis=2)])
    bias = rng.uniform(-3.0, 3.0, dim)
    ones = np.ones((batch, 1, 1))
    A = -np.full((dim, 1), 1e-300)
    for softplus in (True, False):
        y, hL = orc.scan_fwd(np.ones((batch, 1, dim)), u, A, ones, ones, delta_bias=bias,
                             delta_softplus=softplus)
        v = u + bias
        want = np.logaddexp(0.0, v) if softplus else v
        _close(y, want, rtol=1e-14, what=f"delta activation (softplus={softplus})")
    # Theorem 1 with the activation inside the scan: delta = softplus(u)
    batch, L, dim = 2, 30, 3
    u = 2.0 * rng.standard_normal((batch, L, dim))
    x = rng.standard_normal((batch, L, dim))
    shift = rng.uniform(-1.0, 1.0, dim)
    ones = np.ones((batch, L, 1))
    y, _ = orc.scan_fwd(x, u - shift, -np.ones((dim, 1)), ones, ones, zoh=True,
                        delta_bias=shift, delta_softplus=True)
    want = np.empty_like(y)
    for b in range(batch):
        for d in range(dim):
            h = 0.0
            for t in range(L):
                g = expit(u[b, t, d])
                h = (1.0 - g) * h + g * x[b, t, d]
                want[b, t, d] = h
    _close(y, want, what="Theorem 1 gate with the fused activation")
    # decode applies the same activation
    inp = _rand_inputs(rng, 3, 1, 5, 4)
    yo, ho = orc.scan_fwd(**dict(inp, delta=inp["delta"] - 1.0), delta_bias=np.arange(5) * 0.1,
                          delta_softplus=True)
    yd, hd = orc.state_update(inp["h0"], inp["x"][:, 0], inp["delta"][:, 0] - 1.0, inp["A"],
                              inp["B"][:, 0], inp["C"][:, 0], D=inp["D"], z=inp["z"][:, 0],
                              delta_bias=np.arange(5) * 0.1, delta_softplus=True)
    assert np.array_equal(yd, yo[:, 0]) and np.array_equal(hd, ho), "decode activation"


def _conv_inputs(rng, batch, L, dim, width):
    return dict(x=rng.standard_normal((batch, L, dim)),
                weight=rng.standard_normal((dim, width)),
                bias=rng.standard_normal(dim),
                state_in=rng.standard_normal((batch, dim, width)))


def pin_conv_numpy(orc, seed=21):
    rng = np.random.default_rng(seed)
    for width in (1, 2, 3, 4):
        for L in (0, 1, 2, 3, 5, 17):
            inp = _conv_inputs(rng, 2, L, 5, width)
            for silu in (True, False):
                for with_state in (True, False):
                    args = dict(inp) if with_state else dict(inp, state_in=None)
                    y, st = orc.conv1d_fwd(**args, silu=silu)
                    want_y = np.empty((2, L, 5))
                    want_s = np.empty((2, 5, width))
                    for b in range(2):
                        for d in range(5):
                            carried = (inp["state_in"][b, d] if with_state else np.zeros(width))
                            ext = np.concatenate([carried, inp["x"][b, :, d]])
                            taps = inp["weight"][d]
                            # valid[i] = sum_m ext[i + m] * taps[m]; token t is i = t + 1
                            valid = np.convolve(ext, taps[::-1], mode="valid")
                            pre = valid[1:] + inp["bias"][d]
                            want_y[b, :, d] = _silu(pre) if silu else pre
                            want_s[b, d] = ext[-width:]
                    _close(y, want_y, what=f"conv numpy W={width} L={L} silu={silu}")
                    assert np.array_equal(st, want_s), f"conv state W={width} L={L}"


def pin_conv_impulse(orc, seed=22):
    rng = np.random.default_rng(seed)
    width, L, t0 = 4, 12, 5
    w = rng.standard_normal((3, width))
    bias = rng.standard_normal(3)
    x = np.zeros((1, L, 3))
    x[0, t0, :] = 1.0
    y, st = orc.conv1d_fwd(x, w, bias, silu=False)
    for d in range(3):
        want = np.full(L, bias[d])
        for j in range(width):
            want[t0 + j] += w[d, width - 1 - j]
        _close(y[0, :, d], want, rtol=1e-15, what="conv impulse response")


def pin_conv_split_and_decode(orc, seed=23):
    rng = np.random.default_rng(seed)
    width = 4
    inp = _conv_inputs(rng, 3, 23, 6, width)
    y, st = orc.conv1d_fwd(**inp)
    for m in (0, 1, 2, 3, 4, 10, 22, 23):
        y1, s1 = orc.conv1d_fwd(**dict(inp, x=inp["x"][:, :m]))
        y2, s2 = orc.conv1d_fwd(**dict(inp, x=inp["x"][:, m:], state_in=s1))
        assert np.array_equal(np.concatenate([y1, y2], axis=1), y), f"conv split at {m}: y"
        assert np.array_equal(s2, st), f"conv split at {m}: state"
    s = inp["state_in"].copy()
    for t in range(23):
        yt, s = orc.conv1d_update(s, inp["x"][:, t], inp["weight"], inp["bias"])
        assert np.array_equal(yt, y[:, t]), f"conv decode step {t}"
    assert np.array_equal(s, st), "conv decode state"


def _fd_grad(loss, arr, eps):
    fd = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        a1 = arr.copy()
        a1[i] += eps
        a2 = arr.copy()
        a2[i] -= eps
        fd[i] = (loss(a1) - loss(a2)) / (2.0 * eps)
    return fd


def pin_bwd_finite_differences(orc, seed=24):
    rng = np.random.default_rng(seed)
    cases = [dict(softplus=False, opt=True), dict(softplus=True, opt=True),
             dict(softplus=False, opt=False)]
    for case in cases:
        batch, L, dim, N = 2, 6, 3, 4
        inp = _rand_inputs(rng, batch, L, dim, N, h0=case["opt"])
        if not case["opt"]:
            inp["D"] = None
            inp["z"] = None
        if case["softplus"]:
            inp["delta"] = rng.standard_normal((batch, L, dim)) - 0.5
            inp["delta_bias"] = rng.uniform(-1.0, 1.0, dim)
        dy = rng.standard_normal((batch, L, dim))
        dhL = rng.standard_normal((batch, dim, N)) if case["opt"] else None
        sp = case["softplus"]
        g = orc.scan_bwd(**inp, dy=dy, dhL=dhL, delta_softplus=sp)

        def loss_of(name):
            def f(v):
                y, hL = orc.scan_fwd(**dict(inp, **{name: v}), delta_softplus=sp)
                total = float(np.sum(dy * y))
                if dhL is not None:
                    total += float(np.sum(dhL * hL))
                return total
            return f
        names = [("x", "dx"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC")]
        if case["opt"]:
            names += [("D", "dD"), ("z", "dz"), ("h0", "dh0")]
        if sp:
            names += [("delta_bias", "ddelta_bias")]
        for name, key in names:
            fd = _fd_grad(loss_of(name), inp[name], 1e-6)
            _close(g[key], fd, rtol=1e-7, what=f"backward {key} vs finite differences ({case})")
        if not case["opt"]:
            # zero initial state: dh0 is still the gradient at h0 = 0
            zero = np.zeros((batch, dim, N))
            fd = _fd_grad(loss_of("h0"), zero, 1e-6)
            _close(g["dh0"], fd, rtol=1e-7, what="backward dh0 at a zero start")
            assert g["dD"] is None and g["dz"] is None


def pin_bwd_linearity(orc, seed=25):
    rng = np.random.default_rng(seed)
    inp = _rand_inputs(rng, 2, 9, 4, 3)
    dy1, dy2 = rng.standard_normal((2, 2, 9, 4))
    dh1, dh2 = rng.standard_normal((2, 2, 4, 3))
    g1 = orc.scan_bwd(**inp, dy=dy1, dhL=dh1)
    g2 = orc.scan_bwd(**inp, dy=dy2, dhL=dh2)
    g12 = orc.scan_bwd(**inp, dy=2.0 * dy1 - dy2, dhL=2.0 * dh1 - dh2)
    for k in g1:
        if g1[k] is not None:
            _close(g12[k], 2.0 * g1[k] - g2[k], what=f"backward linear in (dy, dhL): {k}")
    g0 = orc.scan_bwd(**inp, dy=np.zeros_like(dy1), dhL=None)
    for k in g0:
        if g0[k] is not None:
            assert not np.any(g0[k]), f"backward {k} not zero for zero upstream gradients"


def _ssd_inputs(rng, batch, L, nheads, headdim, N, h0=True):
    dim = nheads * headdim
    return dict(x=rng.standard_normal((batch, L, dim)),
                dt=np.log1p(np.exp(rng.standard_normal((batch, L, nheads)) - 1.0)),
                A=-np.exp(rng.uniform(-1.0, 1.0, nheads)),
                B=rng.standard_normal((batch, L, N)), C=rng.standard_normal((batch, L, N)),
                D=rng.standard_normal(dim), z=rng.standard_normal((batch, L, dim)),
                h0=rng.standard_normal((batch, nheads, headdim, N)) if h0 else None)


def _ssd_gate_skip(pre, inp, b, sl, cols):
    out = pre + inp["D"][cols] * inp["x"][b, sl][:, cols]
    return out * _silu(inp["z"][b, sl][:, cols])


def pin_ssd_dual_matrix(orc, seed=26):
    rng = np.random.default_rng(seed)
    batch, L, H, P, N = 2, 29, 3, 4, 5
    inp = _ssd_inputs(rng, batch, L, H, P, N)
    y, hL = orc.ssd_fwd(**inp, headdim=P)
    mask = np.tril(np.ones((L, L), dtype=bool))
    for b in range(batch):
        G = inp["C"][b] @ inp["B"][b].T                               # (L, L): C_i . B_j
        for h in range(H):
            a = inp["A"][h]
            S = np.cumsum(inp["dt"][b, :, h])
            M = np.where(mask, G * np.exp(a * (S[:, None] - S[None, :])), 0.0)
            cols = slice(h * P, (h + 1) * P)
            V = inp["dt"][b, :, h][:, None] * inp["x"][b, :, cols]   # (L, P)
            h0 = inp["h0"][b, h]                                     # (P, N)
            pre = M @ V + np.exp(a * S)[:, None] * (inp["C"][b] @ h0.T)
            _close(y[b, :, cols], _ssd_gate_skip(pre, inp, b, slice(None), cols),
                   what="SSD whole-sequence matrix y")
            w = np.exp(a * (S[-1] - S)) * inp["dt"][b, :, h]
            want_h = (inp["x"][b, :, cols] * w[:, None]).T @ inp["B"][b] + np.exp(a * S[-1]) * h0
            _close(hL[b, h], want_h, what="SSD whole-sequence matrix hL")


def _ssd_chunked(inp, P, Q):
    """The chunked dual form: matmuls inside each chunk, state between chunks."""
    x, dt, A, B, C = inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"]
    batch, L, _ = x.shape
    H = dt.shape[2]
    N = B.shape[2]
    pre = np.zeros_like(x)
    state = np.zeros((batch, H, P, N)) if inp["h0"] is None else inp["h0"].copy()
    for c0 in range(0, L, Q):
        sl = slice(c0, min(L, c0 + Q))
        q = sl.stop - sl.start
        mask = np.tril(np.ones((q, q), dtype=bool))
        for b in range(batch):
            G = C[b, sl] @ B[b, sl].T
            for h in range(H):
                S = np.cumsum(dt[b, sl, h]) * A[h]                    # log decay inside the chunk
                cols = slice(h * P, (h + 1) * P)
                V = dt[b, sl, h][:, None] * x[b, sl, cols]
                M = np.where(mask, G * np.exp(S[:, None] - S[None, :]), 0.0)
                pre[b, sl, cols] = M @ V + np.exp(S)[:, None] * (C[b, sl] @ state[b, h].T)
                w = np.exp(S[-1] - S)
                state[b, h] = np.exp(S[-1]) * state[b, h] + (V * w[:, None]).T @ B[b, sl]
    return pre, state


def pin_ssd_chunked(orc, seed=27):
    rng = np.random.default_rng(seed)
    batch, L, H, P, N = 2, 23, 2, 3, 6
    inp = _ssd_inputs(rng, batch, L, H, P, N)
    y, hL = orc.ssd_fwd(**inp, headdim=P)
    for Q in (1, 3, 7, 23, 40):
        pre, state = _ssd_chunked(inp, P, Q)
        want = np.empty_like(pre)
        for b in range(batch):
            want[b] = _ssd_gate_skip(pre[b], inp, b, slice(None), slice(None))
        _close(y, want, what=f"SSD chunked y (Q={Q})")
        _close(hL, state, what=f"SSD chunked hL (Q={Q})")
    # raw dt through bias and softplus is the activated dt
    raw = rng.standard_normal(inp["dt"].shape)
    bias = rng.uniform(-2.0, 0.0, H)
    y1, h1 = orc.ssd_fwd(**dict(inp, dt=raw), headdim=P, dt_bias=bias, dt_softplus=True)
    y2, h2 = orc.ssd_fwd(**dict(inp, dt=np.logaddexp(0.0, raw + bias)), headdim=P)
    _close(y1, y2, what="SSD fused dt activation y")
    _close(h1, h2, what="SSD fused dt activation hL")


def pin_ssd_heads_of_one(orc, seed=28):
    rng = np.random.default_rng(seed)
    batch, L, H, N = 2, 17, 5, 4
    inp = _ssd_inputs(rng, batch, L, H, 1, N)
    y, hL = orc.ssd_fwd(**inp, headdim=1)
    ys, hs = orc.scan_fwd(inp["x"], inp["dt"], np.repeat(inp["A"][:, None], N, axis=1),
                          inp["B"], inp["C"], D=inp["D"], z=inp["z"], h0=inp["h0"][:, :, 0, :])
    _close(y, ys, what="SSD with one channel per head is the scan (y)")
    _close(hL[:, :, 0, :], hs, what="SSD with one channel per head is the scan (hL)")


ALL_PINS = [pin_lti_convolution, pin_brute_force, pin_chunk_split, pin_theorem1,
            pin_ssd_matrix, pin_limits, pin_structure, pin_decode, pin_delta_activation,
            pin_conv_numpy, pin_conv_impulse, pin_conv_split_and_decode,
            pin_bwd_finite_differences, pin_bwd_linearity, pin_ssd_dual_matrix,
            pin_ssd_chunked, pin_ssd_heads_of_one]
