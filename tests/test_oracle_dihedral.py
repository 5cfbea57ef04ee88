"""The dihedral-group oracle against its pins, and planted mistakes in copies of
it that the pins must catch (CPU only).  The mistakes live here, in test code;
the oracle itself is untouched."""
import types

import numpy as np
import pytest

import oracle
from oracle import eqlinear_oracle as O
from tests import oracle_pins_dihedral as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_dihedral_pin(check):
    check(oracle)


def test_golden_file_has_citation_and_cases():
    text = open(P.GOLDEN).read()
    assert "Limitazioni e Lavoro Futuro" in text and "Intuizione Centrale" in text
    assert len(P.load_golden()) == 4


def test_dihedral_rejects_odd_order():
    with pytest.raises(ValueError):
        oracle.tap_table(7, "dihedral")
    with pytest.raises(ValueError):
        oracle.tap_table(4, "octahedral")


# ------------------------------------------------------------------- mutants

def _impl_with_table(table_fn, **over):
    """A copy of the oracle whose dihedral tap table comes from table_fn(T)."""
    def unroll(W, group):
        W = np.asarray(W, np.float64)
        D, C, T = W.shape
        tab = table_fn(T) if group == "dihedral" else O.tap_table(T, group)
        Wd = np.empty((D * T, C * T))
        for g in range(T):
            for h in range(T):
                Wd[g::T, h::T] = W[:, :, tab[g, h]]
        return Wd

    def forward(x, W, bias=None, group="cyclic"):
        x = np.asarray(x, np.float64)
        N, C, T = x.shape
        y = (x.reshape(N, C * T) @ unroll(W, group).T).reshape(N, np.shape(W)[0], T)
        return y if bias is None else y + np.asarray(bias, np.float64)[None, :, None]

    def backward_input(dy, W, group="cyclic"):
        dy = np.asarray(dy, np.float64)
        N, D, T = dy.shape
        return (dy.reshape(N, D * T) @ unroll(W, group)).reshape(N, np.shape(W)[1], T)

    def backward_weight(x, dy, group="cyclic"):
        x, dy = np.asarray(x, np.float64), np.asarray(dy, np.float64)
        N, C, T = x.shape
        D = dy.shape[1]
        tab = table_fn(T) if group == "dihedral" else O.tap_table(T, group)
        dWd = dy.reshape(N, D * T).T @ x.reshape(N, C * T)
        dW = np.zeros((D, C, T))
        for g in range(T):
            for h in range(T):
                dW[:, :, tab[g, h]] += dWd[g::T, h::T]
        return dW, dy.sum(axis=(0, 2))

    ns = dict(forward=forward, backward_input=backward_input, backward_weight=backward_weight,
              mac_counts=oracle.mac_counts,
              tap_table=lambda T, group="cyclic": table_fn(T) if group == "dihedral"
              else O.tap_table(T, group))
    ns.update(over)
    return types.SimpleNamespace(**ns)


def _table(rule):
    def fn(T):
        n = T // 2
        return np.array([[rule(g, h, n) for h in range(T)] for g in range(T)])
    return fn


def _mul_abelian(a, b, n):       # forgets sigma rho sigma = rho^-1: Z_n x Z_2
    (m1, r1), (m2, r2) = divmod(a, n), divmod(b, n)
    return ((m1 + m2) % 2) * n + (r1 + r2) % n


def _inv_bad(a, n):              # reflections inverted like rotations
    m, r = divmod(a, n)
    return m * n + (-r) % n


MUTANTS = {
    "abelian_product": _table(lambda g, h, n: _mul_abelian(O.dihedral_inverse(h, n), g, n)),
    "correlation_g_inv_h": _table(lambda g, h, n: O.dihedral_multiply(O.dihedral_inverse(g, n), h, n)),
    "right_convolution_g_h_inv": _table(lambda g, h, n: O.dihedral_multiply(g, O.dihedral_inverse(h, n), n)),
    "bad_reflection_inverse": _table(lambda g, h, n: O.dihedral_multiply(_inv_bad(h, n), g, n)),
    "h_g_inverse_order": _table(lambda g, h, n: O.dihedral_multiply(g, O.dihedral_inverse(h, n), n)
                                if (g // n) else O.dihedral_multiply(O.dihedral_inverse(h, n), g, n)),
    "interleaved_index": _table(lambda g, h, n: (lambda u: (u % n) * 2 + u // n)(
        O.dihedral_multiply(O.dihedral_inverse((g % 2) * n + g // 2, n), (h % 2) * n + h // 2, n))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    impl = _impl_with_table(MUTANTS[name])
    assert P.failing_checks(impl), f"mutant {name} passed every dihedral pin"


def test_mutant_transposed_weight_fold_is_caught():
    def backward_weight(x, dy, group="cyclic"):
        dW, db = oracle.backward_weight(x, dy, group)
        if group != "dihedral":
            return dW, db
        n = x.shape[2] // 2
        return dW[:, :, [O.dihedral_inverse(u, n) for u in range(2 * n)]], db
    impl = _impl_with_table(lambda T: O.tap_table(T, "dihedral"), backward_weight=backward_weight)
    assert P.failing_checks(impl)


def test_mutant_bias_over_rotations_only_is_caught():
    def backward_weight(x, dy, group="cyclic"):
        dW, _ = oracle.backward_weight(x, dy, group)
        n = x.shape[2] // 2
        return dW, np.asarray(dy, np.float64)[:, :, :n].sum(axis=(0, 2))
    impl = _impl_with_table(lambda T: O.tap_table(T, "dihedral"), backward_weight=backward_weight)
    assert P.failing_checks(impl)


def test_mutant_complex_count_for_2d_blocks_is_caught():
    def mac_counts(N, C, D, T, group="cyclic"):
        s, d = oracle.mac_counts(N, C, D, T, group)
        if group == "dihedral":
            n = T // 2
            s = ((4 if n % 2 == 0 else 2) + 4 * ((n - 1) // 2)) * N * C * D
        return s, d
    impl = _impl_with_table(lambda T: O.tap_table(T, "dihedral"), mac_counts=mac_counts)
    assert P.failing_checks(impl) == ["check_mac_counts"]


def test_unmutated_copy_passes():
    impl = _impl_with_table(lambda T: O.tap_table(T, "dihedral"))
    assert P.failing_checks(impl) == []
