"""fp64 dense group-matrix oracle for the equivariant linear layer (EQ-Linear).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Sources (the pages' own words are not reproduced; each fact is restated):

* "Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise
  Discrete Fourier Transform", gist.science technical summary, sections
  "Problematica" (existing layers expand the shared weights into a dense matrix
  and hand it to a generic dense kernel such as PyTorch's F.linear) and
  "Intuizione Centrale" (the layer is a circular convolution along the group
  axis composed with a linear map along channels; the weight matrix is
  group-circulant, built by cyclically shifting and replicating one set of
  learnable parameters).
* Same paper, authors' English abstract (arxivdaily page): the same
  decomposition; the exact method costs 2(T-1)/T^2 of the dense form.
* Same summary, "Limitazioni e Lavoro Futuro": the authors' kernels cover the
  rotation group p4 only and name reflection groups as the next groups.  For
  those the layer is read as the same construction over the dihedral group
  D_n (rotations by multiples of 2 pi / n and the reflections; p4m is D_4):
  the convolution along the group axis becomes the group convolution
  y[g] = sum_h W[h^-1 g] x[h], which for the cyclic group is the circular
  convolution above.

The oracle is the *definition*, not the fast method: it builds the dense
group matrix and multiplies by it.  It uses no DFT/FFT and no group Fourier
transform.  The one library primitive it uses is a dense fp64 matrix product
(numpy / BLAS).

Layout reading (the pages give none): x is [N, C, T], W is [D, C, T], y is
[N, D, T], all row-major with the group index fastest, so the flat feature
index of (c, s) is c*T + s.  Convolution reading: the weight applied from
input group element h to output group element g is W[d, c, h^-1 g]; for the
cyclic group that is W[d, c, (t - s) mod T].

Groups (``group`` argument, default "cyclic"):
* "cyclic": C_T, element index t = rotation by t steps, product = addition
  mod T.
* "dihedral": D_n with T = 2n elements rho^r sigma^m (rho the rotation by one
  step, sigma a reflection), index m*n + r, so the n rotations come first.
  The product follows from sigma rho sigma = rho^-1:
  (rho^r1 sigma^m1)(rho^r2 sigma^m2) = rho^(r1 + (-1)^m1 r2) sigma^(m1 + m2).
"""
import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


GROUPS = ("cyclic", "dihedral")


def _check_group(group, T):
    if group not in GROUPS:
        raise ValueError(f"unknown group {group!r}")
    if group == "dihedral" and (T % 2 != 0 or T < 4):
        raise ValueError("a dihedral group D_n has T = 2n elements, n >= 2")


def dihedral_multiply(a, b, n):
    """Index of the product a*b in D_n, with index m*n + r for rho^r sigma^m.

    Moving sigma^m1 past rho^r2 turns it into rho^(-r2) when m1 = 1 (the
    defining relation sigma rho sigma = rho^-1), so the rotation parts add
    with the sign (-1)^m1 and the reflection parts add mod 2."""
    m1, r1 = divmod(a, n)
    m2, r2 = divmod(b, n)
    r = (r1 + (r2 if m1 == 0 else -r2)) % n
    m = (m1 + m2) % 2
    return m * n + r


def dihedral_inverse(a, n):
    """Index of a^-1 in D_n: rotations invert to the opposite rotation, and
    every reflection rho^r sigma is its own inverse."""
    m, r = divmod(a, n)
    return (-r) % n if m == 0 else a


def tap_table(T, group="cyclic"):
    """table[g, h] = index of h^-1 g, the weight tap that carries input group
    element h to output group element g."""
    _check_group(group, T)
    table = np.empty((T, T), dtype=np.int64)
    for g in range(T):
        for h in range(T):
            if group == "cyclic":
                table[g, h] = (g - h) % T
            else:
                n = T // 2
                table[g, h] = dihedral_multiply(dihedral_inverse(h, n), g, n)
    return table


def unroll_group(W, group="cyclic"):
    """Dense (D*T) x (C*T) group matrix from the compact weight:
    Wd[d*T + g, c*T + h] = W[d, c, h^-1 g].

    For the cyclic group each output block row g is the compact weight
    cyclically shifted by g ("Intuizione Centrale": cyclic shift and
    replication of the learnable set).  W values are widened exactly to fp64.
    """
    W = _f64(W)
    D, C, T = W.shape
    table = tap_table(T, group)
    Wd = np.empty((D * T, C * T), dtype=np.float64)
    for g in range(T):
        for h in range(T):
            Wd[g::T, h::T] = W[:, :, table[g, h]]
    return Wd


def unroll_block_circulant(W):
    """The cyclic case of ``unroll_group``:
    Wd[d*T + t, c*T + s] = W[d, c, (t - s) mod T]."""
    return unroll_group(W, "cyclic")


def forward(x, W, bias=None, group="cyclic"):
    """y = x_flat . Wd^T (+ bias[d] on every group element), in fp64.

    This is the naive "unroll, then dense multiply" form of the layer
    ("Problematica"); the fast method must reach the same result exactly up to
    rounding ("Contributi Chiave": exactness from DFT invertibility and the
    convolution theorem).  Bias reading: one value per output channel d,
    shared by the T outputs of that channel (the pages name no bias).
    """
    x = _f64(x)
    N, C, T = x.shape
    D = np.shape(W)[0]
    Wd = unroll_group(W, group)
    y = (x.reshape(N, C * T) @ Wd.T).reshape(N, D, T)
    if bias is not None:
        y = y + _f64(bias)[None, :, None]
    return y


def gelu(v):
    """GELU in fp64: v * Phi(v), Phi the standard normal distribution
    function, written (v/2)(1 + erf(v / sqrt 2)) with scipy's erf.

    The pages do not define the activation; this is the GELU of the
    transformer MLP blocks (EQ-Linear -> GELU -> EQ-Linear) in the networks
    the layer is built into ("Livello di Rete": Flash EQ-ViT)."""
    from scipy.special import erf
    v = _f64(v)
    return 0.5 * v * (1.0 + erf(v / np.sqrt(2.0)))


def gelu_tanh(v):
    """GELU with its usual tanh approximation, fp64:
    (v/2)(1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))."""
    v = _f64(v)
    return 0.5 * v * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (v + 0.044715 * v ** 3)))


ACTIVATIONS = {None: lambda v: _f64(v), "gelu": gelu, "gelu_tanh": gelu_tanh}


def forward_act(x, W, bias=None, act=None, group="cyclic"):
    """act(forward(x, W, bias)): the activation applied to every output value
    after the bias (a pointwise map, so the result stays equivariant)."""
    return ACTIVATIONS[act](forward(x, W, bias, group))


def backward_input(dy, W, group="cyclic"):
    """dx = dy_flat . Wd (the transpose of the forward map), in fp64.

    Gradient of the forward with respect to x; the pages state that the method
    covers the backward pass ("Implementazione") without writing it out.
    """
    dy = _f64(dy)
    N, D, T = dy.shape
    C = np.shape(W)[1]
    Wd = unroll_group(W, group)
    return (dy.reshape(N, D * T) @ Wd).reshape(N, C, T)


def backward_weight(x, dy, group="cyclic"):
    """(dW, dbias) for the compact weight and the per-channel bias, in fp64.

    The dense gradient is dWd = dy_flat^T . x_flat.  Each compact entry
    W[d, c, u] appears in the dense matrix at every (g, h) with h^-1 g == u,
    so its gradient is the sum of those replicas:
        dW[d, c, u] = sum over (g, h) with h^-1 g = u of dWd[d*T + g, c*T + h]
    (cyclic: (g, h) = (t, (t - u) mod T)).
    dbias[d] = sum over rows and group elements of dy[:, d, :].
    """
    x = _f64(x)
    dy = _f64(dy)
    N, C, T = x.shape
    D = dy.shape[1]
    table = tap_table(T, group)
    dWd = dy.reshape(N, D * T).T @ x.reshape(N, C * T)  # (D*T, C*T)
    dW = np.zeros((D, C, T), dtype=np.float64)
    for g in range(T):
        for h in range(T):
            dW[:, :, table[g, h]] += dWd[g::T, h::T]
    dbias = dy.sum(axis=(0, 2))
    return dW, dbias


def mac_counts(N, C, D, T, group="cyclic"):
    """(spectral MACs, dense MACs) per forward, with C and D per group element.

    Dense: the unrolled (D*T) x (C*T) matrix times N rows, T^2 * N*C*D.
    Cyclic (authors' abstract; "Specializzazione per il Gruppo di Rotazione
    p4"): by conjugate symmetry of the real DFT only frequencies 0..floor(T/2)
    are formed; k = 0 (and k = T/2 for even T) are real and cost one real
    N x C x D product each, every other kept frequency is complex and costs
    four.  For even T this totals 2(T - 1) products; p4 gives 6 against 16.
    Dihedral D_n (T = 2n): the group Fourier transform splits the layer into
    one real product per one-dimensional representation (four for even n,
    two for odd n) and a 2 x 2 block product, eight real products, per
    two-dimensional representation ((n - 1) // 2 of them): 12 against 64 for
    p4m (D_4).
    """
    _check_group(group, T)
    dense = T * T * N * C * D
    if group == "dihedral":
        n = T // 2
        one_dim = 4 if n % 2 == 0 else 2
        two_dim = (n - 1) // 2
        return (one_dim + 8 * two_dim) * N * C * D, dense
    real_freqs = 2 if T % 2 == 0 else 1
    complex_freqs = T // 2 + 1 - real_freqs
    spectral = (real_freqs + 4 * complex_freqs) * N * C * D
    return spectral, dense


def param_counts(C, D, T):
    """(compact, dense) parameter counts of the weight ("Livello di Rete":
    about T times fewer parameters than the dense layer of equal width)."""
    return D * C * T, (D * T) * (C * T)
