"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one (CPU only).  The mistakes live here, in test code; the oracle
itself is untouched."""
import types

import numpy as np
import pytest

import oracle
from oracle import eqlinear_oracle as O
from tests import oracle_pins as P


def _unroll_with(tap):
    def unroll(W):
        W = np.asarray(W, np.float64)
        D, C, T = W.shape
        Wd = np.empty((D * T, C * T))
        for t in range(T):
            for s in range(T):
                Wd[t::T, s::T] = W[:, :, tap(t, s, T)]
        return Wd
    return unroll


def _impl(**over):
    ns = {k: getattr(oracle, k) for k in
          ("forward", "backward_input", "backward_weight", "mac_counts", "param_counts",
           "unroll_block_circulant", "gelu", "gelu_tanh", "forward_act")}
    ns.update(over)
    return types.SimpleNamespace(**ns)


def _forward_with_unroll(unroll):
    def forward(x, W, bias=None):
        x = np.asarray(x, np.float64)
        N, C, T = x.shape
        D = np.shape(W)[0]
        y = (x.reshape(N, C * T) @ unroll(W).T).reshape(N, D, T)
        if bias is not None:
            y = y + np.asarray(bias, np.float64)[None, :, None]
        return y
    return forward


def _bwd_input_with_unroll(unroll):
    def backward_input(dy, W):
        dy = np.asarray(dy, np.float64)
        N, D, T = dy.shape
        C = np.shape(W)[1]
        return (dy.reshape(N, D * T) @ unroll(W)).reshape(N, C, T)
    return backward_input


def _bwd_weight_with_fold(src_index, bias_sum=lambda dy: dy.sum(axis=(0, 2))):
    def backward_weight(x, dy):
        x = np.asarray(x, np.float64)
        dy = np.asarray(dy, np.float64)
        N, C, T = x.shape
        D = dy.shape[1]
        dWd = dy.reshape(N, D * T).T @ x.reshape(N, C * T)
        dW = np.zeros((D, C, T))
        for r in range(T):
            for t in range(T):
                dW[:, :, r] += dWd[t::T, src_index(t, r, T)::T]
        return dW, bias_sum(dy)
    return backward_weight


def _fwd_bias_t0(x, W, bias=None):
    y = O.forward(x, W, None)
    if bias is not None:
        y = y.copy()
        y[:, :, 0] += np.asarray(bias)
    return y


def _mac_counts_no_symmetry(N, C, D, T):
    # forgets conjugate symmetry: T complex products
    return 4 * T * N * C * D, T * T * N * C * D


def _mac_counts_gauss(N, C, D, T):
    # 3-multiply complex products (not what the pages count)
    real = 2 if T % 2 == 0 else 1
    cplx = T // 2 + 1 - real
    return (real + 3 * cplx) * N * C * D, T * T * N * C * D


def _gelu_no_sqrt2(v):
    from scipy.special import erf
    v = np.asarray(v, np.float64)
    return 0.5 * v * (1.0 + erf(v))


def _gelu_tanh_const(k):
    def f(v):
        v = np.asarray(v, np.float64)
        return 0.5 * v * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (v + k * v ** 3)))
    return f


def _act_before_bias(x, W, bias=None, act=None):
    y = O.ACTIVATIONS[act](O.forward(x, W, None))
    return y + (np.asarray(bias, np.float64)[None, :, None] if bias is not None else 0.0)


corr = _unroll_with(lambda t, s, T: (s - t) % T)
off_by_one = _unroll_with(lambda t, s, T: (t - s + 1) % T)
no_shift = _unroll_with(lambda t, s, T: 0 if t == s else (t - s) % T if (t + s) % 2 else 1)

MUTANTS = {
    "forward_correlation_not_convolution": _impl(forward=_forward_with_unroll(corr)),
    "forward_tap_off_by_one": _impl(forward=_forward_with_unroll(off_by_one)),
    "forward_wrong_tap_table": _impl(forward=_forward_with_unroll(no_shift)),
    "forward_drops_bias": _impl(forward=lambda x, W, bias=None: O.forward(x, W, None)),
    "forward_bias_only_t0": _impl(forward=_fwd_bias_t0),
    "forward_transposed_input_group": _impl(
        forward=lambda x, W, bias=None: O.forward(np.asarray(x)[:, :, ::-1], W, bias)),
    "backward_input_correlation": _impl(backward_input=_bwd_input_with_unroll(corr)),
    "backward_input_sign": _impl(backward_input=lambda dy, W: -O.backward_input(dy, W)),
    "backward_input_forward_weight_order": _impl(
        backward_input=lambda dy, W: O.forward(dy, np.swapaxes(np.asarray(W), 0, 1), None)),
    "backward_weight_fold_plus": _impl(backward_weight=_bwd_weight_with_fold(lambda t, r, T: (t + r) % T)),
    "backward_weight_fold_reversed": _impl(backward_weight=_bwd_weight_with_fold(lambda t, r, T: (r - t) % T)),
    "backward_weight_dbias_t0_only": _impl(
        backward_weight=_bwd_weight_with_fold(lambda t, r, T: (t - r) % T,
                                              bias_sum=lambda dy: dy[:, :, 0].sum(axis=0))),
    "backward_weight_scaled": _impl(
        backward_weight=lambda x, dy: tuple(np.asarray(a) * 2 for a in O.backward_weight(x, dy))),
    "mac_counts_without_symmetry": _impl(mac_counts=_mac_counts_no_symmetry),
    "mac_counts_gauss_trick": _impl(mac_counts=_mac_counts_gauss),
    "param_counts_dense_equal": _impl(param_counts=lambda C, D, T: (D * C * T, D * C * T)),
    "gelu_erf_without_sqrt2": _impl(gelu=_gelu_no_sqrt2),
    "gelu_missing_half": _impl(gelu=lambda v: np.asarray(O.gelu(v)) * 2),
    "gelu_tanh_cubic_constant": _impl(gelu_tanh=_gelu_tanh_const(0.44715)),
    "gelu_tanh_without_cubic": _impl(gelu_tanh=_gelu_tanh_const(0.0)),
    "forward_act_before_bias": _impl(forward_act=_act_before_bias),
    "forward_act_ignores_act": _impl(forward_act=lambda x, W, bias=None, act=None: O.forward(x, W, bias)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    bad = P.failing_checks(MUTANTS[name])
    assert bad, f"no pin catches mutant {name}"


def test_unmutated_oracle_passes_all_pins():
    assert P.failing_checks(oracle) == []
