"""Pins that tie the oracle to the pages' definition and to mathematics.

Each ``check_*`` takes an implementation namespace exposing ``forward``,
``backward_input``, ``backward_weight``, ``mac_counts`` and ``param_counts``
(the oracle, or a deliberately broken copy of it in the mutant tests) and raises
``AssertionError`` when the implementation disagrees with the pin.

None of the checks recomputes the oracle's own dense block-circulant product:
they use hand-derived values (tests/golden), direct loops over the convolution
sum, special cases that reduce to ordinary matrix products, numpy's FFT,
invariants (group equivariance, the adjoint identity) and finite differences.

Definition followed (Flash EQ-Linear, gist.science summary, "Intuizione
Centrale"; authors' English abstract): y[n,d,t] = sum_c sum_s
W[d,c,(t-s) mod T] x[n,c,s], plus a per-channel bias shared over t.
"""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "p4_worked_examples.txt")


def _rng(seed):
    return np.random.default_rng(seed)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / den)


def load_golden(path=GOLDEN):
    """Parse the hand-derived worked examples."""
    cases, cur, key = [], None, None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "case":
                cur = {"name": tok[1], "x": [], "W": [], "b": [], "y": []}
                key = None
            elif tok[0] in ("C", "D"):
                cur[tok[0]] = int(tok[1])
            elif tok[0] in ("x", "W", "b", "y") and len(tok) == 1:
                key = tok[0]
            elif tok[0] == "end":
                C, D = cur["C"], cur["D"]
                case = {
                    "name": cur["name"],
                    "x": np.array(cur["x"], np.float64).reshape(1, C, 4),
                    "W": np.array(cur["W"], np.float64).reshape(D, C, 4),
                    "b": None if cur["b"] == ["none"] else np.array(cur["b"], np.float64),
                    "y": np.array(cur["y"], np.float64).reshape(1, D, 4),
                }
                cases.append(case)
                cur = None
            else:
                if tok == ["none"]:
                    cur[key] = ["none"]
                else:
                    cur[key].extend(float(v) for v in tok)
    return cases


# ---------------------------------------------------------------- forward pins

def check_golden(impl):
    """Hand-derived worked examples reproduce exactly."""
    cases = load_golden()
    assert len(cases) >= 3
    for c in cases:
        y = impl.forward(c["x"], c["W"], c["b"])
        assert np.array_equal(np.asarray(y), c["y"]), (c["name"], y, c["y"])


def _brute_forward(x, W, b):
    N, C, T = x.shape
    D = W.shape[0]
    y = np.zeros((N, D, T))
    for n in range(N):
        for d in range(D):
            for t in range(T):
                acc = 0.0
                for c in range(C):
                    for s in range(T):
                        acc += W[d, c, (t - s) % T] * x[n, c, s]
                y[n, d, t] = acc + (b[d] if b is not None else 0.0)
    return y


def check_brute_force(impl):
    """Direct loops over the circular-convolution sum, tiny sizes, several T."""
    rng = _rng(11)
    for T in (1, 2, 3, 4, 5, 6, 8, 12, 16):
        for (N, C, D) in ((1, 1, 1), (3, 2, 3), (5, 3, 2)):
            x = rng.standard_normal((N, C, T))
            W = rng.standard_normal((D, C, T))
            b = rng.standard_normal(D)
            for bb in (None, b):
                got = impl.forward(x, W, bb)
                ref = _brute_forward(x, W, bb)
                assert _rel(got, ref) < 1e-13, (T, N, C, D, _rel(got, ref))


def check_one_hot(impl):
    """C = D = 1 and x = e_s (one-hot on group element s): y = W rolled by s."""
    rng = _rng(12)
    for T in (4, 5, 8, 16):
        W = rng.standard_normal((1, 1, T))
        for s in range(T):
            x = np.zeros((1, 1, T))
            x[0, 0, s] = 1.0
            y = np.asarray(impl.forward(x, W, None))
            assert np.array_equal(y[0, 0], np.roll(W[0, 0], s)), (T, s, y, W)


def check_per_group_gemm(impl):
    """W = delta_r (x) A: the layer is one ordinary matrix product per group
    element, y[:,:,t] = x[:,:,(t-r) mod T] A^T (np.matmul)."""
    rng = _rng(13)
    N, C, D, T = 7, 5, 6, 4
    x = rng.standard_normal((N, C, T))
    A = rng.standard_normal((D, C))
    b = rng.standard_normal(D)
    for r in range(T):
        W = np.zeros((D, C, T))
        W[:, :, r] = A
        y = np.asarray(impl.forward(x, W, b))
        for t in range(T):
            ref = np.matmul(x[:, :, (t - r) % T], A.T) + b
            assert _rel(y[:, :, t], ref) < 1e-13, (r, t)


def check_group_constant(impl):
    """x constant over the group axis gives y constant over it, equal to
    (sum_r W[:,:,r]) u."""
    rng = _rng(14)
    N, C, D, T = 4, 3, 5, 4
    u = rng.standard_normal((N, C))
    x = np.repeat(u[:, :, None], T, axis=2)
    W = rng.standard_normal((D, C, T))
    y = np.asarray(impl.forward(x, W, None))
    ref = u @ W.sum(axis=2).T
    for t in range(T):
        assert _rel(y[:, :, t], ref) < 1e-13


def check_trivial_group(impl):
    """T = 1 is an ordinary linear layer y = x W^T + b."""
    rng = _rng(15)
    x = rng.standard_normal((6, 4, 1))
    W = rng.standard_normal((3, 4, 1))
    b = rng.standard_normal(3)
    y = np.asarray(impl.forward(x, W, b))
    assert _rel(y[:, :, 0], x[:, :, 0] @ W[:, :, 0].T + b) < 1e-13


def check_equivariance(impl):
    """Rolling x along the group axis rolls y the same way (rotation
    equivariance, "Contributi Chiave")."""
    rng = _rng(16)
    for T in (3, 4, 8, 16):
        N, C, D = 5, 3, 4
        x = rng.standard_normal((N, C, T))
        W = rng.standard_normal((D, C, T))
        b = rng.standard_normal(D)
        y = np.asarray(impl.forward(x, W, b))
        for r in range(1, T):
            yr = np.asarray(impl.forward(np.roll(x, r, axis=2), W, b))
            assert _rel(yr, np.roll(y, r, axis=2)) < 1e-13, (T, r)


def _fft_forward(x, W, b):
    # convolution theorem along the group axis, with numpy's FFT
    X = np.fft.fft(x, axis=2)          # [N, C, T]
    Wh = np.fft.fft(W, axis=2)         # [D, C, T]
    Y = np.einsum("dck,nck->ndk", Wh, X)
    y = np.fft.ifft(Y, axis=2).real
    return y + (b[None, :, None] if b is not None else 0.0)


def check_fft_identity(impl):
    """The DFT path (numpy FFT, per-frequency products) equals the layer."""
    rng = _rng(17)
    for T in (2, 3, 4, 5, 6, 7, 8, 12, 16):
        x = rng.standard_normal((6, 5, T))
        W = rng.standard_normal((7, 5, T))
        b = rng.standard_normal(7)
        assert _rel(impl.forward(x, W, b), _fft_forward(x, W, b)) < 1e-13, T


# --------------------------------------------------------------- backward pins

def _loss(impl, x, W, b, dy):
    return float(np.sum(np.asarray(impl.forward(x, W, b)) * dy))


def check_backward_input_adjoint(impl):
    """<dy, f(x)> = <f*(dy), x> for the bias-free layer f."""
    rng = _rng(21)
    for T in (3, 4, 8, 16):
        x = rng.standard_normal((5, 3, T))
        W = rng.standard_normal((4, 3, T))
        dy = rng.standard_normal((5, 4, T))
        lhs = np.sum(dy * np.asarray(impl.forward(x, W, None)))
        rhs = np.sum(np.asarray(impl.backward_input(dy, W)) * x)
        assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs)), (lhs, rhs)


def check_backward_input_fd(impl):
    """Central differences of L = <dy, y(x)> (exact up to rounding: L is linear in x)."""
    rng = _rng(22)
    N, C, D, T = 3, 2, 3, 4
    x = rng.standard_normal((N, C, T))
    W = rng.standard_normal((D, C, T))
    b = rng.standard_normal(D)
    dy = rng.standard_normal((N, D, T))
    dx = np.asarray(impl.backward_input(dy, W))
    for idx in np.ndindex(N, C, T):
        e = np.zeros_like(x)
        e[idx] = 1.0
        fd = (_loss(impl, x + e, W, b, dy) - _loss(impl, x - e, W, b, dy)) / 2.0
        assert abs(fd - dx[idx]) < 1e-10, (idx, fd, dx[idx])


def check_backward_input_as_forward(impl):
    """dx equals a forward with the adjoint weight W*[c,d,u] = W[d,c,(-u) mod T]."""
    rng = _rng(23)
    for T in (4, 8, 13):
        N, C, D = 6, 3, 5
        W = rng.standard_normal((D, C, T))
        dy = rng.standard_normal((N, D, T))
        Wadj = np.empty((C, D, T))
        for u in range(T):
            Wadj[:, :, u] = W[:, :, (-u) % T].T
        assert _rel(impl.backward_input(dy, W), _brute_forward(dy, Wadj, None)) < 1e-13, T


def check_backward_weight_fd(impl):
    """Central differences of L = <dy, y(W, b)> w.r.t. every W and b entry."""
    rng = _rng(24)
    N, C, D, T = 4, 2, 3, 4
    x = rng.standard_normal((N, C, T))
    W = rng.standard_normal((D, C, T))
    b = rng.standard_normal(D)
    dy = rng.standard_normal((N, D, T))
    dW, db = impl.backward_weight(x, dy)
    dW, db = np.asarray(dW), np.asarray(db)
    assert dW.shape == W.shape and db.shape == b.shape
    for idx in np.ndindex(D, C, T):
        e = np.zeros_like(W)
        e[idx] = 1.0
        fd = (_loss(impl, x, W + e, b, dy) - _loss(impl, x, W - e, b, dy)) / 2.0
        assert abs(fd - dW[idx]) < 1e-10, (idx, fd, dW[idx])
    for d in range(D):
        e = np.zeros_like(b)
        e[d] = 1.0
        fd = (_loss(impl, x, W, b + e, dy) - _loss(impl, x, W, b - e, dy)) / 2.0
        assert abs(fd - db[d]) < 1e-10, (d, fd, db[d])


def check_backward_weight_brute(impl):
    """dW[d,c,r] = sum_{n,t} dy[n,d,t] x[n,c,(t-r) mod T], by direct loops."""
    rng = _rng(25)
    for T in (3, 4, 8, 16):
        N, C, D = 4, 3, 2
        x = rng.standard_normal((N, C, T))
        dy = rng.standard_normal((N, D, T))
        ref = np.zeros((D, C, T))
        for d in range(D):
            for c in range(C):
                for r in range(T):
                    ref[d, c, r] = sum(dy[n, d, t] * x[n, c, (t - r) % T]
                                       for n in range(N) for t in range(T))
        dW, db = impl.backward_weight(x, dy)
        assert _rel(dW, ref) < 1e-13, T
        assert _rel(db, dy.sum(axis=(0, 2))) < 1e-13


# ---------------------------------------------------------- activation pins

# Standard normal distribution function at a few points (values of the
# normal table, to 16 digits): Phi(0.5), Phi(1), Phi(2).
_PHI = {0.5: 0.6914624612740131, 1.0: 0.8413447460685429, 2.0: 0.9772498680518208}


def check_gelu_normal_cdf(impl):
    """GELU(v) = v Phi(v): the normal table, Phi(-v) = 1 - Phi(v), GELU(0) = 0."""
    assert float(np.asarray(impl.gelu(np.array([0.0])))[0]) == 0.0
    for v, phi in _PHI.items():
        for sv, ph in ((v, phi), (-v, 1.0 - phi)):
            got = float(np.asarray(impl.gelu(np.array([sv])))[0])
            assert abs(got - sv * ph) < 1e-15, (sv, got, sv * ph)


def check_gelu_odd_part(impl):
    """GELU(v) - GELU(-v) = v for both forms (Phi(v) + Phi(-v) = 1, and
    tanh is odd); large |v| gives v or 0."""
    rng = _rng(31)
    v = rng.standard_normal(1000) * 3
    for f in (impl.gelu, impl.gelu_tanh):
        g = np.asarray(f(v)) - np.asarray(f(-v))
        assert np.max(np.abs(g - v)) < 1e-14
        big = np.asarray(f(np.array([12.0, -12.0])))
        assert abs(big[0] - 12.0) < 1e-12 and abs(big[1]) < 1e-12


def check_gelu_tanh_close(impl):
    """The tanh form stays within 1e-3 of GELU everywhere (it is an
    approximation of the same function, not another one)."""
    v = np.linspace(-8, 8, 16001)
    d = np.abs(np.asarray(impl.gelu(v)) - np.asarray(impl.gelu_tanh(v)))
    assert d.max() < 1e-3, d.max()


def check_forward_act(impl):
    """forward_act = brute-force layer, then the activation per value with
    math.erf (independent of the oracle's erf); equivariant under rolls."""
    import math
    rng = _rng(32)
    for T in (3, 4, 8):
        x = rng.standard_normal((5, 3, T))
        W = rng.standard_normal((4, 3, T))
        b = rng.standard_normal(4)
        lin = _brute_forward(x, W, b)
        ref = np.vectorize(lambda v: 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))))(lin)
        got = np.asarray(impl.forward_act(x, W, b, "gelu"))
        assert _rel(got, ref) < 1e-14, T
        assert _rel(impl.forward_act(x, W, b, None), lin) < 1e-13, T
        for r in range(1, T):
            yr = np.asarray(impl.forward_act(np.roll(x, r, axis=2), W, b, "gelu_tanh"))
            assert _rel(yr, np.roll(np.asarray(impl.forward_act(x, W, b, "gelu_tanh")), r,
                                    axis=2)) < 1e-13, (T, r)


# ------------------------------------------------------------------ cost pins

def check_mac_counts(impl):
    """p4: 6 real products against 16 ("Specializzazione ... p4", 16/6 = 2.67x);
    general even T: the ratio 2(T-1)/T^2 (authors' abstract)."""
    s, d = impl.mac_counts(10, 3, 7, 4)
    assert (s, d) == (6 * 10 * 3 * 7, 16 * 10 * 3 * 7)
    assert s * 8 == d * 3  # 3/8
    for T in (2, 4, 6, 8, 16):
        s, d = impl.mac_counts(5, 4, 3, T)
        assert s * T * T == d * 2 * (T - 1), T
    # odd T: one real frequency and (T-1)/2 complex ones -> 2T - 1 products
    for T in (3, 5, 7):
        s, d = impl.mac_counts(1, 1, 1, T)
        assert s == 2 * T - 1 and d == T * T, T


def check_param_counts(impl):
    """The compact weight has T times fewer entries than the dense matrix
    ("Livello di Rete": about 4x fewer at T = 4)."""
    for T in (2, 4, 8):
        comp, dense = impl.param_counts(12, 20, T)
        assert dense == T * comp


ALL_CHECKS = [
    check_golden, check_brute_force, check_one_hot, check_per_group_gemm,
    check_group_constant, check_trivial_group, check_equivariance, check_fft_identity,
    check_backward_input_adjoint, check_backward_input_fd, check_backward_input_as_forward,
    check_backward_weight_fd, check_backward_weight_brute, check_mac_counts, check_param_counts,
    check_gelu_normal_cdf, check_gelu_odd_part, check_gelu_tanh_close, check_forward_act,
]


def failing_checks(impl):
    """Names of the checks that fail (an exception of any kind counts)."""
    bad = []
    for chk in ALL_CHECKS:
        try:
            chk(impl)
        except Exception:  # noqa: BLE001 -- a crash is a detected mistake too
            bad.append(chk.__name__)
    return bad
