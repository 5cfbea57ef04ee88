"""Pins that tie the p4 group-convolution oracle to its definition and to
mathematics.

Each ``check_*`` takes an implementation namespace exposing ``conv_forward``,
``conv_backward_input``, ``conv_backward_weight`` and ``conv_mac_counts`` -- the
oracle, or a deliberately broken copy of it in the mutant tests -- and raises
``AssertionError`` when it disagrees.

Reading (Flash EQ-Linear, gist.science summary: "Limitazioni e Lavoro Futuro"
names equivariant convolutions as the next operator; "Intuizione Centrale" for
the group-axis convolution): on fields f[N, H, W, C, 4] over the plane and p4,
    y[n,i,j,d,t] = b[d] + sum_{c,s,v} psi[d, c, h + R^-t v, (t-s) mod 4] f[n, i+a, j+b, c, s]
with zero padding and R(a, b) = (-b, a).

None of the checks uses the oracle's tap matrices.  They use hand-derived
values (tests/golden), direct loops over numpy's rot90 of the filter, scipy's
2-D correlation, the EQ-Linear oracle (pinned on its own), invariance under
turning the image together with the group shift, an adjoint identity, exact
differences of a linear map, and a separately written spectral evaluation
over rotation-aware patches with numpy's FFT.
"""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "p4conv_worked_examples.txt")


def _rng(seed):
    return np.random.default_rng(seed)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / den)


# ------------------------------------------------------------------ golden

def load_golden(path=GOLDEN):
    cases, cur, sec = [], None, None
    for raw in open(path):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "case":
            cur = {"name": tok[1], "f": [], "psi": [], "y": [], "b": None}
            sec = None
        elif tok[0] == "H":
            cur["H"], cur["W"], cur["k"] = int(tok[1]), int(tok[2]), int(tok[3])
        elif tok[0] in ("f", "psi", "y"):
            sec = tok[0]
        elif tok[0] == "b":
            cur["b"] = None if tok[1] == "none" else float(tok[1])
        elif tok[0] == "end":
            cases.append(cur)
            cur = None
        else:
            cur[sec].append([int(v) for v in tok[:3]] + [float(tok[3])])
    return cases


def check_golden(impl):
    for case in load_golden():
        H, W, k = case["H"], case["W"], case["k"]
        f = np.zeros((1, H, W, 1, 4))
        for i, j, s, v in case["f"]:
            f[0, i, j, 0, s] = v
        psi = np.zeros((1, 1, k, k, 4))
        for a, b, r, v in case["psi"]:
            psi[0, 0, a, b, r] = v
        bias = None if case["b"] is None else np.array([case["b"]])
        want = np.full((1, H, W, 1, 4), 0.0 if bias is None else case["b"])
        for i, j, t, v in case["y"]:
            want[0, i, j, 0, t] = v
        got = impl.conv_forward(f, psi, bias)
        assert np.array_equal(got, want), case["name"]


# --------------------------------------------------------------- brute force

def brute_forward(f, psi, bias):
    """Direct loops; the filter for output group element t is numpy's rot90
    of psi by t quarter turns on its spatial axes."""
    N, H, W, C, _ = f.shape
    D, _, k, _, _ = psi.shape
    h = k // 2
    rot = [np.rot90(psi, t, axes=(2, 3)) for t in range(4)]
    y = np.zeros((N, H, W, D, 4))
    for n in range(N):
        for i in range(H):
            for j in range(W):
                for t in range(4):
                    acc = np.zeros(D) if bias is None else np.array(bias, np.float64)
                    for a in range(-h, h + 1):
                        for b in range(-h, h + 1):
                            if not (0 <= i + a < H and 0 <= j + b < W):
                                continue
                            for s in range(4):
                                acc = acc + rot[t][:, :, h + a, h + b, (t - s) % 4] @ f[n, i + a, j + b, :, s]
                    y[n, i, j, :, t] = acc
    return y


def check_brute_force(impl):
    rng = _rng(11)
    for (N, H, W, C, D, k) in [(2, 4, 5, 2, 3, 3), (1, 5, 3, 1, 2, 5), (1, 3, 4, 2, 1, 1)]:
        f = rng.standard_normal((N, H, W, C, 4))
        psi = rng.standard_normal((D, C, k, k, 4))
        bias = rng.standard_normal(D)
        assert _rel(impl.conv_forward(f, psi, bias), brute_forward(f, psi, bias)) < 1e-13


def check_scipy_correlate(impl):
    """One channel each way and a filter that does not shift the group axis:
    output plane t is scipy's 2-D correlation of input plane t with the
    spatial kernel turned t quarter turns."""
    from scipy.signal import correlate2d
    rng = _rng(12)
    H, W, k = 7, 6, 5
    g = rng.standard_normal((k, k))
    psi = np.zeros((1, 1, k, k, 4))
    psi[0, 0, :, :, 0] = g
    f = rng.standard_normal((1, H, W, 1, 4))
    y = impl.conv_forward(f, psi, None)
    for t in range(4):
        want = correlate2d(f[0, :, :, 0, t], np.rot90(g, t), mode="same", boundary="fill")
        assert _rel(y[0, :, :, 0, t], want) < 1e-13, t


# ----------------------------------------------------------------- invariants

def _turn(z, r):
    return np.roll(np.rot90(z, r, axes=(1, 2)), r, axis=4)


def check_equivariance(impl):
    rng = _rng(13)
    f = rng.standard_normal((2, 6, 6, 3, 4))
    psi = rng.standard_normal((2, 3, 3, 3, 4))
    bias = rng.standard_normal(2)
    y = impl.conv_forward(f, psi, bias)
    for r in (1, 2, 3):
        assert _rel(impl.conv_forward(_turn(f, r), psi, bias), _turn(y, r)) < 1e-13, r


def check_linear_reduction(impl):
    """A 1 x 1 kernel, or a 3 x 3 kernel with only the centre tap, is the
    EQ-Linear layer applied to every pixel (the EQ-Linear oracle, pinned on
    its own in tests/oracle_pins.py)."""
    import oracle
    rng = _rng(14)
    N, H, W, C, D = 2, 3, 4, 3, 5
    f = rng.standard_normal((N, H, W, C, 4))
    Wl = rng.standard_normal((D, C, 4))
    bias = rng.standard_normal(D)
    want = oracle.forward(f.reshape(-1, C, 4), Wl, bias).reshape(N, H, W, D, 4)
    assert _rel(impl.conv_forward(f, Wl[:, :, None, None, :], bias), want) < 1e-13
    psi = np.zeros((D, C, 3, 3, 4))
    psi[:, :, 1, 1, :] = Wl
    assert _rel(impl.conv_forward(f, psi, bias), want) < 1e-13


# ------------------------------------------------------- spectral evaluation

def patch_spectral_forward(f, psi, bias):
    """The same layer through rotation-aware patches and the length-4 DFT,
    written independently of the oracle.

    Offsets other than 0 fall into orbits {R^j u : j = 0..3} under the
    quarter turn, one representative u per orbit (rows >= 1, columns >= 0).
    For an orbit the input values f[p + R^j u, c, (j + e) mod 4] are, for
    each (c, e), a function of j that the layer convolves cyclically with
    phi_(c,e)[m] = psi[., c, h + R^-m u, (m - e) mod 4]; the centre tap is the
    plain group convolution.  So y = IDFT( sum over patch channels of
    DFT(phi) * DFT(x) ) and every patch channel costs one product per kept
    frequency pair: 6 real multiplies per (patch channel, output channel).
    Returns (y, real multiplies counted)."""
    N, H, W, C, _ = f.shape
    D, _, k, _, _ = psi.shape
    h = k // 2
    fp = np.pad(f, ((0, 0), (h, h), (h, h), (0, 0), (0, 0)))

    def rot(a, b, m):
        for _ in range(m % 4):
            a, b = -b, a
        return a, b

    reps = [(a, b) for a in range(1, h + 1) for b in range(0, h + 1)]
    xs, ws = [], []
    xs.append(f)                                        # centre: [N,H,W,C,4]
    ws.append(psi[:, :, h, h, :])                       # [D,C,4], index (t - s)
    for (ua, ub) in reps:
        for e in range(4):
            xj = np.stack([fp[:, h + rot(ua, ub, j)[0]:h + rot(ua, ub, j)[0] + H,
                              h + rot(ua, ub, j)[1]:h + rot(ua, ub, j)[1] + W, :, (j + e) % 4]
                           for j in range(4)], axis=-1)
            xs.append(xj)
            ws.append(np.stack([psi[:, :, h + rot(ua, ub, -m)[0], h + rot(ua, ub, -m)[1], (m - e) % 4]
                                for m in range(4)], axis=-1))
    X = np.fft.fft(np.concatenate(xs, axis=3), axis=-1)   # [N,H,W,k^2 C,4]
    Wf = np.fft.fft(np.concatenate(ws, axis=1), axis=-1)  # [D,k^2 C,4]
    Ck = X.shape[3]
    Y = np.zeros((N, H, W, D, 4), dtype=np.complex128)
    mults = 0
    for q in range(3):                                    # kept frequencies 0, 1, 2
        Y[..., q] = np.einsum("nhwc,dc->nhwd", X[..., q], Wf[:, :, q])
        mults += (1 if q in (0, 2) else 4) * Ck * D * N * H * W
    Y[..., 3] = np.conj(Y[..., 1])
    y = np.fft.ifft(Y, axis=-1).real
    if bias is not None:
        y = y + np.asarray(bias)[None, None, None, :, None]
    return y, mults


def check_patch_spectral(impl):
    rng = _rng(15)
    for (N, H, W, C, D, k) in [(1, 5, 4, 2, 3, 3), (1, 6, 6, 1, 2, 5)]:
        f = rng.standard_normal((N, H, W, C, 4))
        psi = rng.standard_normal((D, C, k, k, 4))
        bias = rng.standard_normal(D)
        y, mults = patch_spectral_forward(f, psi, bias)
        assert _rel(impl.conv_forward(f, psi, bias), y) < 1e-12
        spec, dense = impl.conv_mac_counts(N * H * W, C, D, k)
        assert spec == mults
        assert dense == 16 * k * k * C * D * N * H * W
        assert spec * 8 == dense * 3


# ----------------------------------------------------------------- backward

def check_backward_input_adjoint(impl):
    """<dy, conv(f)> = <conv^T(dy), f> for the bias-free layer."""
    rng = _rng(16)
    N, H, W, C, D, k = 2, 5, 4, 3, 2, 3
    f = rng.standard_normal((N, H, W, C, 4))
    dy = rng.standard_normal((N, H, W, D, 4))
    psi = rng.standard_normal((D, C, k, k, 4))
    lhs = float(np.sum(dy * impl.conv_forward(f, psi, None)))
    rhs = float(np.sum(impl.conv_backward_input(dy, psi) * f))
    assert abs(lhs - rhs) <= 1e-12 * max(abs(lhs), 1.0)


def check_backward_weight_exact_differences(impl):
    """The loss L = <dy, conv(f, psi) + b> is linear in psi and b, so its
    derivative along a unit filter entry is L(psi + e) - L(psi) exactly
    (up to rounding), with no step-size error."""
    rng = _rng(17)
    N, H, W, C, D, k = 1, 4, 3, 2, 2, 3
    f = rng.standard_normal((N, H, W, C, 4))
    dy = rng.standard_normal((N, H, W, D, 4))
    psi = rng.standard_normal((D, C, k, k, 4))
    dpsi, dbias = impl.conv_backward_weight(f, dy, k)
    base = float(np.sum(dy * impl.conv_forward(f, psi, None)))
    want = np.zeros_like(psi)
    for idx in np.ndindex(*psi.shape):
        e = psi.copy()
        e[idx] += 1.0
        want[idx] = float(np.sum(dy * impl.conv_forward(f, e, None))) - base
    assert _rel(dpsi, want) < 1e-11
    wantb = np.array([np.sum(dy[..., d, :]) for d in range(D)])
    assert _rel(dbias, wantb) < 1e-13


def check_backward_weight_brute(impl):
    """dpsi from the rot90 loops: the derivative of brute_forward's sum with
    respect to each filter entry, accumulated term by term."""
    rng = _rng(18)
    N, H, W, C, D, k = 1, 3, 4, 2, 1, 3
    h = k // 2
    f = rng.standard_normal((N, H, W, C, 4))
    dy = rng.standard_normal((N, H, W, D, 4))
    # d/dpsi of sum_t dy[.,t] * rot90(psi, t)[h+a, h+b, (t-s)] f[i+a, j+b, s]:
    # accumulate into a rotated-filter gradient, then turn it back.
    g = [np.zeros((D, C, k, k, 4)) for _ in range(4)]
    for n in range(N):
        for i in range(H):
            for j in range(W):
                for t in range(4):
                    for a in range(-h, h + 1):
                        for b in range(-h, h + 1):
                            if not (0 <= i + a < H and 0 <= j + b < W):
                                continue
                            for s in range(4):
                                g[t][:, :, h + a, h + b, (t - s) % 4] += np.outer(
                                    dy[n, i, j, :, t], f[n, i + a, j + b, :, s])
    want = sum(np.rot90(g[t], -t, axes=(2, 3)) for t in range(4))
    dpsi, _ = impl.conv_backward_weight(f, dy, k)
    assert _rel(dpsi, want) < 1e-13


def check_counts(impl):
    assert impl.conv_mac_counts(10, 3, 5, 3) == (6 * 9 * 3 * 5 * 10, 16 * 9 * 3 * 5 * 10)
    assert impl.conv_mac_counts(1, 2, 2, 1) == (24, 64)


def check_param_counts(impl):
    """Parameters counted on the unrolled filter ("Livello di Rete", Flash
    EQ-Linear summary: the equivariant layer shares its weights over the
    group, 1/T of the parameters of the unconstrained layer it equals).  The
    unconstrained convolution on the same fields has one weight per (output
    channel d, output element t, input channel c, input element s, offset);
    brute_forward's rot90 loops say which filter entry fills each of those
    slots.  With every filter entry a distinct label, the compact count is
    the number of labels seen, the dense count the number of slots, and each
    label fills exactly T = 4 slots."""
    for C, D, k in ((1, 1, 1), (3, 5, 3), (2, 4, 5)):
        h = k // 2
        psi = np.arange(1, D * C * k * k * 4 + 1, dtype=np.float64).reshape(D, C, k, k, 4)
        rot = [np.rot90(psi, t, axes=(2, 3)) for t in range(4)]
        slots = [rot[t][d, c, h + a, h + b, (t - s) % 4]
                 for d in range(D) for t in range(4) for c in range(C) for s in range(4)
                 for a in range(-h, h + 1) for b in range(-h, h + 1)]
        labels, uses = np.unique(np.array(slots), return_counts=True)
        assert np.all(uses == 4)
        assert impl.conv_param_counts(C, D, k) == (len(labels), len(slots))
        assert len(slots) == 4 * len(labels)


ALL_CHECKS = [
    check_golden,
    check_brute_force,
    check_scipy_correlate,
    check_equivariance,
    check_linear_reduction,
    check_patch_spectral,
    check_backward_input_adjoint,
    check_backward_weight_exact_differences,
    check_backward_weight_brute,
    check_counts,
    check_param_counts,
]


def failing_checks(impl):
    failed = []
    for check in ALL_CHECKS:
        try:
            check(impl)
        except AssertionError:
            failed.append(check.__name__)
    return failed
