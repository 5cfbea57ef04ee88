"""fp64 dense oracle for the p4 group convolution on the plane.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Source: "Flash EQ-Linear" technical summary (gist.science), section
"Limitazioni e Lavoro Futuro": the authors name the extension of their
principle to other equivariant operators, equivariant convolutions among
them, as future work, and give no definition.  The layer here is the plainest
reading that the rest of the pages supports:

* features are fields over the plane with one value per element of the
  rotation group p4 (the regular representation the EQ-Linear layer acts on,
  "Intuizione Centrale"), stored f[N, H, W, C, 4] with the group index fastest,
  so every pixel is one EQ-Linear row [C, 4];
* the layer is a k x k convolution (k odd, stride 1, zero padding, output the
  size of the input) whose taps are rotated together with the group shift:
      y[n, i, j, d, t] = bias[d] + sum over c, s and offsets v = (a, b) in
          [-h, h]^2 (h = k // 2) of
          psi[d, c, h + R^-t v, (t - s) mod 4] * f[n, i + a, j + b, c, s],
  with f = 0 outside the image, psi[D, C, k, k, 4] the compact filter (its
  spatial index is the offset plus h), and R the quarter turn of offsets
  R(a, b) = (-b, a) in (row, column) coordinates, R^-1(a, b) = (b, -a);
* a 1 x 1 kernel is exactly the EQ-Linear layer with weight psi[:, :, 0, 0, :]
  (the circular convolution along the group axis, weight index (t - s) mod 4);
* the layer commutes with turning the image a quarter turn, as numpy's rot90
  does on the (H, W) axes, together with the cyclic shift of the group axis by
  one: y(L f) = L y(f), L f = roll(rot90(f), 1) on the group axis.  That is
  what fixes the direction of R above.

The oracle is the definition: per offset v it builds the dense
(4D) x (4C) matrix K(v)[d*4 + t, c*4 + s] = psi[d, c, h + R^-t v, (t - s) mod 4]
and sums K(v) f[p + v] over the offsets.  No DFT and no group transform.  The
one library primitive is a dense fp64 matrix product.
"""
import numpy as np

T4 = 4


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def rotate_offset(a, b, turns):
    """R^turns (a, b) for the quarter turn R(a, b) = (-b, a); negative turns
    rotate the other way."""
    for _ in range(turns % 4):
        a, b = -b, a
    return a, b


def _half(k):
    if k % 2 != 1 or k < 1:
        raise ValueError("the kernel size must be odd")
    return k // 2


def tap_matrix(psi, a, b):
    """K(v) for the offset v = (a, b): the dense (4D) x (4C) matrix carrying
    the input pixel p + v to the output pixel p,
        K[d*4 + t, c*4 + s] = psi[d, c, h + R^-t v, (t - s) mod 4]."""
    psi = _f64(psi)
    D, C, k, _, _ = psi.shape
    h = _half(k)
    K = np.empty((D * T4, C * T4), dtype=np.float64)
    for t in range(T4):
        ra, rb = rotate_offset(a, b, -t)
        for s in range(T4):
            K[t::T4, s::T4] = psi[:, :, h + ra, h + rb, (t - s) % T4]
    return K


def _offsets(k):
    h = _half(k)
    return [(a, b) for a in range(-h, h + 1) for b in range(-h, h + 1)]


def _pad(f, h):
    return np.pad(f, ((0, 0), (h, h), (h, h), (0, 0), (0, 0)))


def conv_forward(f, psi, bias=None):
    """y[N, H, W, D, 4] in fp64, by the definition in the module docstring."""
    f = _f64(f)
    N, H, W, C, _ = f.shape
    D, _, k, _, _ = np.shape(psi)
    h = _half(k)
    fp = _pad(f, h).reshape(N, H + 2 * h, W + 2 * h, C * T4)
    y = np.zeros((N, H, W, D * T4), dtype=np.float64)
    for a, b in _offsets(k):
        K = tap_matrix(psi, a, b)
        y += fp[:, h + a:h + a + H, h + b:h + b + W, :] @ K.T
    y = y.reshape(N, H, W, D, T4)
    if bias is not None:
        y = y + _f64(bias)[None, None, None, :, None]
    return y


def conv_forward_act(f, psi, bias=None, act=None):
    """act(conv_forward(f, psi, bias)), the activation pointwise after the bias
    (the same activations as the EQ-Linear oracle)."""
    from .eqlinear_oracle import ACTIVATIONS
    return ACTIVATIONS[act](conv_forward(f, psi, bias))


def conv_backward_input(dy, psi):
    """df = the transpose of the forward map applied to dy, in fp64:
    df[n, q] = sum over offsets v of K(v)^T dy[n, q - v] (dy = 0 outside)."""
    dy = _f64(dy)
    N, H, W, D, _ = dy.shape
    _, C, k, _, _ = np.shape(psi)
    h = _half(k)
    dyp = _pad(dy, h).reshape(N, H + 2 * h, W + 2 * h, D * T4)
    df = np.zeros((N, H, W, C * T4), dtype=np.float64)
    for a, b in _offsets(k):
        K = tap_matrix(psi, a, b)
        df += dyp[:, h - a:h - a + H, h - b:h - b + W, :] @ K
    return df.reshape(N, H, W, C, T4)


def conv_backward_weight(f, dy, k):
    """(dpsi[D, C, k, k, 4], dbias[D]) in fp64.

    The dense gradient of the tap matrix is dK(v) = sum over (n, p) of
    dy[n, p] (outer) f[n, p + v].  Each filter entry psi[d, c, h + w, r]
    appears in K(v) at row d*4 + t and column c*4 + s exactly when R^-t v = w
    and (t - s) mod 4 = r, i.e. v = R^t w and s = (t - r) mod 4, one place per
    t; its gradient is the sum of those four replicas (one replica per t even
    for the centre tap w = 0, where v = 0 for every t).
    dbias[d] = sum of dy[..., d, :]."""
    f, dy = _f64(f), _f64(dy)
    N, H, W, C, _ = f.shape
    D = dy.shape[3]
    h = _half(k)
    fp = _pad(f, h).reshape(N, H + 2 * h, W + 2 * h, C * T4)
    dyf = dy.reshape(N * H * W, D * T4)
    dK = {}
    for a, b in _offsets(k):
        xs = fp[:, h + a:h + a + H, h + b:h + b + W, :].reshape(N * H * W, C * T4)
        dK[(a, b)] = dyf.T @ xs
    dpsi = np.zeros((D, C, k, k, T4), dtype=np.float64)
    for wa, wb in _offsets(k):
        for r in range(T4):
            for t in range(T4):
                va, vb = rotate_offset(wa, wb, t)
                s = (t - r) % T4
                dpsi[:, :, h + wa, h + wb, r] += dK[(va, vb)][t::T4, s::T4]
    return dpsi, dy.sum(axis=(0, 1, 2, 4))


def conv_mac_counts(pixels, C, D, k):
    """(spectral MACs, dense MACs) per forward over ``pixels`` output pixels.

    Dense: every output pixel applies the k*k unrolled (4D) x (4C) tap
    matrices, 16 k^2 C D.  The layer equals an EQ-Linear layer with k^2 C
    input channels over rotation-aware patches (the tap orbits under the
    quarter turn are folded into the group axis), so the p4 transform applies
    with its 6 real products per (input channel, output channel): 6 k^2 C D,
    the same 3/8 as the linear layer."""
    return 6 * k * k * C * D * pixels, 16 * k * k * C * D * pixels


def conv_param_counts(C, D, k):
    """(compact, dense) filter parameter counts: D C k^2 4 against the
    (4D) x (4C) k^2 of an unconstrained convolution on the same fields."""
    return D * C * k * k * T4, (D * T4) * (C * T4) * k * k
