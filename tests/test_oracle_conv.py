"""The p4 group-convolution oracle against its pins, and planted mistakes in
copies of it that the pins must catch (CPU only).  The mistakes live here, in
test code; the oracle itself is untouched."""
import types

import numpy as np
import pytest

import oracle
from tests import oracle_pins_conv as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_conv_pin(check):
    check(oracle)


def test_golden_file_has_citation_and_cases():
    text = open(P.GOLDEN).read()
    assert "Limitazioni e Lavoro Futuro" in text and "Intuizione Centrale" in text
    assert len(P.load_golden()) == 7


def test_even_kernel_rejected():
    with pytest.raises(ValueError):
        oracle.conv_forward(np.zeros((1, 2, 2, 1, 4)), np.zeros((1, 1, 2, 2, 4)))


# ------------------------------------------------------------------- mutants

def _impl(rot_sign=-1, group_sign=1, swap=False, pad="constant", with_bias=True,
          bwd_sign=-1, fold_sign=1, count=6, dense_params=16):
    """A copy of the oracle with one knob turned away from the definition:
    rot_sign     -- filter tap R^(rot_sign * t) v (definition: -1)
    group_sign   -- weight index (group_sign * (t - s)) mod 4 (definition: +1)
    swap         -- spatial filter axes transposed
    pad          -- numpy pad mode at the border (definition: zeros)
    with_bias    -- bias added
    bwd_sign     -- backward_input reads dy at q + bwd_sign * v (definition: -1)
    fold_sign    -- weight gradient replica at v = R^(fold_sign * t) w
    count        -- real products per (patch channel, output channel)
    dense_params -- unrolled weights per (filter tap, c, d) (definition: 16)"""
    def tap(psi, a, b):
        D, C, k, _, _ = psi.shape
        h = k // 2
        K = np.empty((D * 4, C * 4))
        for t in range(4):
            ra, rb = oracle.rotate_offset(a, b, rot_sign * t)
            if swap:
                ra, rb = rb, ra
            for s in range(4):
                K[t::4, s::4] = psi[:, :, h + ra, h + rb, (group_sign * (t - s)) % 4]
        return K

    def offs(k):
        h = k // 2
        return [(a, b) for a in range(-h, h + 1) for b in range(-h, h + 1)]

    def padf(z, h):
        return np.pad(z, ((0, 0), (h, h), (h, h), (0, 0), (0, 0)), mode=pad)

    def conv_forward(f, psi, bias=None):
        f, psi = np.asarray(f, np.float64), np.asarray(psi, np.float64)
        N, H, W, C, _ = f.shape
        D, k = psi.shape[0], psi.shape[2]
        h = k // 2
        fp = padf(f, h).reshape(N, H + 2 * h, W + 2 * h, C * 4)
        y = np.zeros((N, H, W, D * 4))
        for a, b in offs(k):
            y += fp[:, h + a:h + a + H, h + b:h + b + W] @ tap(psi, a, b).T
        y = y.reshape(N, H, W, D, 4)
        if bias is not None and with_bias:
            y = y + np.asarray(bias)[None, None, None, :, None]
        return y

    def conv_backward_input(dy, psi):
        dy, psi = np.asarray(dy, np.float64), np.asarray(psi, np.float64)
        N, H, W, D, _ = dy.shape
        C, k = psi.shape[1], psi.shape[2]
        h = k // 2
        dyp = padf(dy, h).reshape(N, H + 2 * h, W + 2 * h, D * 4)
        df = np.zeros((N, H, W, C * 4))
        for a, b in offs(k):
            sa, sb = bwd_sign * a, bwd_sign * b
            df += dyp[:, h + sa:h + sa + H, h + sb:h + sb + W] @ tap(psi, a, b)
        return df.reshape(N, H, W, C, 4)

    def conv_backward_weight(f, dy, k):
        f, dy = np.asarray(f, np.float64), np.asarray(dy, np.float64)
        N, H, W, C, _ = f.shape
        D = dy.shape[3]
        h = k // 2
        fp = padf(f, h).reshape(N, H + 2 * h, W + 2 * h, C * 4)
        dyf = dy.reshape(-1, D * 4)
        dK = {(a, b): dyf.T @ fp[:, h + a:h + a + H, h + b:h + b + W].reshape(-1, C * 4)
              for a, b in offs(k)}
        dpsi = np.zeros((D, C, k, k, 4))
        for wa, wb in offs(k):
            for r in range(4):
                for t in range(4):
                    va, vb = oracle.rotate_offset(wa, wb, fold_sign * t)
                    dpsi[:, :, h + wa, h + wb, r] += dK[(va, vb)][t::4, (t - r) % 4::4]
        return dpsi, dy.sum(axis=(0, 1, 2, 4))

    def conv_mac_counts(pixels, C, D, k):
        return count * k * k * C * D * pixels, 16 * k * k * C * D * pixels

    def conv_param_counts(C, D, k):
        return D * C * k * k * 4, dense_params * D * C * k * k

    return types.SimpleNamespace(conv_forward=conv_forward,
                                 conv_backward_input=conv_backward_input,
                                 conv_backward_weight=conv_backward_weight,
                                 conv_mac_counts=conv_mac_counts,
                                 conv_param_counts=conv_param_counts)


MUTANTS = {
    "taps_turned_the_other_way": dict(rot_sign=1),
    "group_correlation_not_convolution": dict(group_sign=-1),
    "filter_axes_transposed": dict(swap=True),
    "wrap_around_border": dict(pad="wrap"),
    "reflected_border": dict(pad="reflect"),
    "bias_dropped": dict(with_bias=False),
    "backward_input_shifted_forward": dict(bwd_sign=1),
    "weight_fold_turned_the_other_way": dict(fold_sign=-1),
    "dense_product_count": dict(count=16),
    "dense_params_not_unrolled": dict(dense_params=4),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    failed = P.failing_checks(_impl(**MUTANTS[name]))
    assert failed, f"mutant {name} passed every convolution pin"


def test_unmutated_copy_passes():
    assert P.failing_checks(_impl()) == []
