"""Pins that tie the dihedral-group oracle to its definition and to mathematics.

Each ``check_*`` takes an implementation namespace exposing ``forward``,
``backward_input``, ``backward_weight``, ``mac_counts`` and ``tap_table`` (each
taking a ``group`` argument) -- the oracle, or a deliberately broken copy of it
in the mutant tests -- and raises ``AssertionError`` when it disagrees.

Reading (Flash EQ-Linear, gist.science summary: "Intuizione Centrale" for the
layer as a convolution along the group axis composed with a linear map along
channels; "Limitazioni e Lavoro Futuro" for reflection groups as the next
groups): over the dihedral group D_n of the regular n-gon the layer is the
group convolution y[n,d,g] = sum_c sum_h W[d,c,h^-1 g] x[n,c,h] (+ b[d]), with
group index m*n + r for rho^r sigma^m.

None of the checks uses the oracle's own composition rule.  The group law
here comes from the faithful 2 x 2 orthogonal representation (rho the
rotation by 2 pi / n, sigma the reflection diag(1, -1)), products of those
matrices are looked up among the 2n element matrices, and the checks use
hand-derived values (tests/golden), direct loops, ordinary matrix products,
the group Fourier transform over the real irreducible representations,
invariants and finite differences.
"""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "p4m_worked_examples.txt")
DIH = "dihedral"


def _rng(seed):
    return np.random.default_rng(seed)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / den)


# ------------------------------------------------- group law from 2x2 matrices

def _rot(theta):
    c, s = np.cos(theta), np.sin(theta)
    return np.array([[c, -s], [s, c]])


_FLIP = np.array([[1.0, 0.0], [0.0, -1.0]])


def element_matrix(idx, n, k=1):
    """pi_k(rho^r sigma^m) = R(2 pi k r / n) F^m for index m*n + r."""
    m, r = divmod(idx, n)
    M = _rot(2.0 * np.pi * k * r / n)
    return M @ _FLIP if m else M


def _lookup(M, n):
    dist = [np.abs(element_matrix(u, n) - M).max() for u in range(2 * n)]
    u = int(np.argmin(dist))
    assert dist[u] < 1e-9
    return u


def mat_mul(a, b, n):
    """Index of a*b through the matrix representation."""
    return _lookup(element_matrix(a, n) @ element_matrix(b, n), n)


def mat_inv(a, n):
    return _lookup(element_matrix(a, n).T, n)


def check_group_law(impl):
    """The oracle's tap table is h^-1 g of the matrix group, for n = 2..8, and
    the group is non-abelian for n >= 3 (sigma rho sigma = rho^-1)."""
    for n in range(2, 9):
        table = np.asarray(impl.tap_table(2 * n, DIH))
        for g in range(2 * n):
            for h in range(2 * n):
                assert table[g, h] == mat_mul(mat_inv(h, n), g, n), (n, g, h)
        if n >= 3:
            assert mat_mul(1, n, n) != mat_mul(n, 1, n)


# ---------------------------------------------------------------- forward pins

def load_golden(path=GOLDEN):
    cases, cur, key = [], None, None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "case":
                cur = {"name": tok[1], "x": [], "W": [], "b": [], "y": []}
            elif tok[0] in ("C", "D"):
                cur[tok[0]] = int(tok[1])
            elif tok[0] in ("x", "W", "b", "y") and len(tok) == 1:
                key = tok[0]
            elif tok[0] == "end":
                C, D = cur["C"], cur["D"]
                cases.append({
                    "name": cur["name"],
                    "x": np.array(cur["x"], np.float64).reshape(1, C, 8),
                    "W": np.array(cur["W"], np.float64).reshape(D, C, 8),
                    "b": None if cur["b"] == ["none"] else np.array(cur["b"], np.float64),
                    "y": np.array(cur["y"], np.float64).reshape(1, D, 8),
                })
            elif tok == ["none"]:
                cur[key] = ["none"]
            else:
                cur[key].extend(float(v) for v in tok)
    return cases


def check_golden(impl):
    """Hand-derived p4m examples reproduce exactly."""
    cases = load_golden()
    assert len(cases) >= 4
    for c in cases:
        y = np.asarray(impl.forward(c["x"], c["W"], c["b"], group=DIH))
        assert np.array_equal(y, c["y"]), (c["name"], y, c["y"])


def _brute_forward(x, W, b, n):
    N, C, T = x.shape
    D = W.shape[0]
    tap = [[mat_mul(mat_inv(h, n), g, n) for h in range(T)] for g in range(T)]
    y = np.zeros((N, D, T))
    for i in range(N):
        for d in range(D):
            for g in range(T):
                acc = 0.0
                for c in range(C):
                    for h in range(T):
                        acc += W[d, c, tap[g][h]] * x[i, c, h]
                y[i, d, g] = acc + (b[d] if b is not None else 0.0)
    return y


def check_brute_force(impl):
    """Direct loops over the group-convolution sum, n = 2..8, tiny sizes."""
    rng = _rng(31)
    for n in range(2, 9):
        for (N, C, D) in ((1, 1, 1), (3, 2, 3)):
            x = rng.standard_normal((N, C, 2 * n))
            W = rng.standard_normal((D, C, 2 * n))
            b = rng.standard_normal(D)
            for bb in (None, b):
                got = impl.forward(x, W, bb, group=DIH)
                assert _rel(got, _brute_forward(x, W, bb, n)) < 1e-13, (n, N, C, D)


def check_per_element_gemm(impl):
    """W = delta_u (x) A: one ordinary matrix product per group element,
    y[:,:,g] = x[:,:,g u^-1] A^T + b (np.matmul)."""
    rng = _rng(32)
    n, N, C, D = 4, 5, 4, 3
    x = rng.standard_normal((N, C, 2 * n))
    A = rng.standard_normal((D, C))
    b = rng.standard_normal(D)
    for u in range(2 * n):
        W = np.zeros((D, C, 2 * n))
        W[:, :, u] = A
        y = np.asarray(impl.forward(x, W, b, group=DIH))
        for g in range(2 * n):
            src = mat_mul(g, mat_inv(u, n), n)
            assert _rel(y[:, :, g], np.matmul(x[:, :, src], A.T) + b) < 1e-13, (u, g)


def _left(x, a, n):
    """(L_a x)[h] = x[a^-1 h] along the last axis."""
    perm = [mat_mul(mat_inv(a, n), h, n) for h in range(2 * n)]
    return np.asarray(x)[..., perm]


def check_equivariance(impl):
    """Transforming x by any rotation or reflection transforms y the same way:
    y(L_a x) = L_a y(x) for every a in D_n."""
    rng = _rng(33)
    for n in (2, 3, 4, 6):
        x = rng.standard_normal((4, 3, 2 * n))
        W = rng.standard_normal((5, 3, 2 * n))
        b = rng.standard_normal(5)
        y = np.asarray(impl.forward(x, W, b, group=DIH))
        for a in range(2 * n):
            ya = np.asarray(impl.forward(_left(x, a, n), W, b, group=DIH))
            assert _rel(ya, _left(y, a, n)) < 1e-13, (n, a)


def check_cyclic_reduction(impl):
    """x supported on the rotations: the rotation outputs are the cyclic layer
    with the rotation taps of W, the reflection outputs the cyclic layer with
    the reflection taps (h^-1 g stays in the coset of g)."""
    rng = _rng(34)
    for n in (3, 4, 5):
        x = np.zeros((3, 2, 2 * n))
        x[:, :, :n] = rng.standard_normal((3, 2, n))
        W = rng.standard_normal((4, 2, 2 * n))
        y = np.asarray(impl.forward(x, W, None, group=DIH))
        rot = np.asarray(impl.forward(x[:, :, :n], W[:, :, :n], None, group="cyclic"))
        ref = np.asarray(impl.forward(x[:, :, :n], W[:, :, n:], None, group="cyclic"))
        assert _rel(y[:, :, :n], rot) < 1e-13 and _rel(y[:, :, n:], ref) < 1e-13, n


def irreps(n):
    """Real irreducible representations of D_n as functions of the element
    index: (dimension, matrix function).  One-dimensional: rho -> +-1 (-1 only
    for even n) times sigma -> +-1; two-dimensional: pi_k for
    1 <= k <= (n - 1) // 2."""
    reps = []
    for a in ((1, -1) if n % 2 == 0 else (1,)):
        for bsgn in (1, -1):
            reps.append((1, lambda u, a=a, bsgn=bsgn: np.array(
                [[float(a ** (u % n) * bsgn ** (u // n))]])))
    for k in range(1, (n - 1) // 2 + 1):
        reps.append((2, lambda u, k=k: element_matrix(u, n, k)))
    return reps


def fourier_forward(x, W, b, n):
    """The layer through the group Fourier transform, fp64: per irreducible
    representation pi, x^(pi) = sum_h x[h] pi(h), the same for W, the block
    product y^(pi) = x^(pi) W^(pi), and the inversion
    y[g] = (1/|G|) sum_pi dim(pi) tr(y^(pi) pi(g)^T)."""
    T = 2 * n
    N, C, _ = x.shape
    D = W.shape[0]
    y = np.zeros((N, D, T))
    for dim, pi in irreps(n):
        P = np.stack([pi(u) for u in range(T)])            # [T, dim, dim]
        xh = np.einsum("nch,hij->ncij", x, P)
        wh = np.einsum("dch,hij->dcij", W, P)
        yh = np.einsum("ncik,dckj->ndij", xh, wh)
        y += dim * np.einsum("ndij,gij->ndg", yh, P) / T
    return y + (b[None, :, None] if b is not None else 0.0)


def check_fourier_identity(impl):
    """The group Fourier transform path equals the layer (convolution theorem
    on a non-abelian group: the block products need the order x^ W^)."""
    rng = _rng(35)
    for n in range(2, 9):
        x = rng.standard_normal((5, 4, 2 * n))
        W = rng.standard_normal((6, 4, 2 * n))
        b = rng.standard_normal(6)
        got = impl.forward(x, W, b, group=DIH)
        assert _rel(got, fourier_forward(x, W, b, n)) < 1e-12, n


# --------------------------------------------------------------- backward pins

def check_backward_input_adjoint(impl):
    """<dy, f(x)> = <f*(dy), x> for the bias-free layer."""
    rng = _rng(36)
    for n in (2, 3, 4, 6):
        x = rng.standard_normal((4, 3, 2 * n))
        W = rng.standard_normal((5, 3, 2 * n))
        dy = rng.standard_normal((4, 5, 2 * n))
        lhs = np.sum(dy * np.asarray(impl.forward(x, W, None, group=DIH)))
        rhs = np.sum(np.asarray(impl.backward_input(dy, W, group=DIH)) * x)
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), n


def check_backward_input_as_forward(impl):
    """dx is the forward layer with the adjoint weight W*[c, d, v] =
    W[d, c, v^-1] (a group convolution's transpose convolves with the
    inverted kernel)."""
    rng = _rng(37)
    for n in (3, 4):
        W = rng.standard_normal((3, 4, 2 * n))
        dy = rng.standard_normal((5, 3, 2 * n))
        inv = [mat_inv(v, n) for v in range(2 * n)]
        Wadj = np.transpose(W, (1, 0, 2))[:, :, inv]
        got = impl.backward_input(dy, W, group=DIH)
        assert _rel(got, impl.forward(dy, Wadj, None, group=DIH)) < 1e-13, n


def check_backward_weight_fd(impl):
    """Central finite differences of L = <dy, y> with respect to entries of W
    and of the bias (L is linear in W, so the difference quotient is exact up
    to rounding)."""
    rng = _rng(38)
    n = 4
    x = rng.standard_normal((3, 2, 2 * n))
    W = rng.standard_normal((3, 2, 2 * n))
    b = rng.standard_normal(3)
    dy = rng.standard_normal((3, 3, 2 * n))
    dW, db = impl.backward_weight(x, dy, group=DIH)
    loss = lambda W_, b_: float(np.sum(dy * np.asarray(impl.forward(x, W_, b_, group=DIH))))
    h = 1e-3
    for (d, c, u) in ((0, 0, 0), (1, 1, 3), (2, 0, 5), (2, 1, 7), (0, 1, 4)):
        Wp, Wm = W.copy(), W.copy()
        Wp[d, c, u] += h
        Wm[d, c, u] -= h
        fd = (loss(Wp, b) - loss(Wm, b)) / (2 * h)
        assert abs(fd - dW[d, c, u]) < 1e-8 * max(1.0, abs(fd)), (d, c, u, fd, dW[d, c, u])
    for d in range(3):
        bp, bm = b.copy(), b.copy()
        bp[d] += h
        bm[d] -= h
        fd = (loss(W, bp) - loss(W, bm)) / (2 * h)
        assert abs(fd - db[d]) < 1e-8 * max(1.0, abs(fd)), d


def check_backward_weight_brute(impl):
    """dW[d,c,u] = sum_rows sum_h dy[., d, h u] x[., c, h], by direct loops."""
    rng = _rng(39)
    for n in (2, 3, 4):
        T = 2 * n
        x = rng.standard_normal((3, 2, T))
        dy = rng.standard_normal((3, 3, T))
        dW, db = impl.backward_weight(x, dy, group=DIH)
        ref = np.zeros((3, 2, T))
        for u in range(T):
            for h in range(T):
                g = mat_mul(h, u, n)
                ref[:, :, u] += np.einsum("nd,nc->dc", dy[:, :, g], x[:, :, h])
        assert _rel(dW, ref) < 1e-13, n
        assert _rel(db, dy.sum(axis=(0, 2))) < 1e-13, n


# ------------------------------------------------------------------ cost pins

def check_mac_counts(impl):
    """p4m (D_4): 4 one-dimensional products and one 2 x 2 block product of 8,
    12 real products against 64; even n: 4n - 4 of 4n^2, odd n: 4n - 2."""
    s, d = impl.mac_counts(10, 3, 7, 8, group=DIH)
    assert (s, d) == (12 * 210, 64 * 210)
    for n in range(2, 9):
        s, d = impl.mac_counts(1, 1, 1, 2 * n, group=DIH)
        assert d == 4 * n * n and s == (4 * n - 4 if n % 2 == 0 else 4 * n - 2), n
        # the count equals the sum over the real irreducible representations
        # of dim^3 (a dim x dim block product per channel pair)
        assert s == sum(dim ** 3 for dim, _ in irreps(n)), n


ALL_CHECKS = [
    check_group_law, check_golden, check_brute_force, check_per_element_gemm,
    check_equivariance, check_cyclic_reduction, check_fourier_identity,
    check_backward_input_adjoint, check_backward_input_as_forward,
    check_backward_weight_fd, check_backward_weight_brute, check_mac_counts,
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
