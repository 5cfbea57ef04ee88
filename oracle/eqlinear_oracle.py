"""fp64 dense block-circulant oracle for the equivariant linear layer (EQ-Linear).

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

The oracle is the *definition*, not the fast method: it builds the dense
block-circulant matrix and multiplies by it.  It uses no DFT/FFT.  The one
library primitive it uses is a dense fp64 matrix product (numpy / BLAS).

Layout reading (the pages give none): x is [N, C, T], W is [D, C, T], y is
[N, D, T], all row-major with the group index fastest, so the flat feature
index of (c, s) is c*T + s.  Convolution reading: the weight applied from
input group element s to output group element t is W[d, c, (t - s) mod T].
"""
import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def unroll_block_circulant(W):
    """Dense (D*T) x (C*T) group-circulant matrix from the compact weight.

    Wd[d*T + t, c*T + s] = W[d, c, (t - s) mod T]: each output block row t is
    the compact weight cyclically shifted by t ("Intuizione Centrale": cyclic
    shift and replication of the learnable set).  W values are widened exactly
    to fp64.
    """
    W = _f64(W)
    D, C, T = W.shape
    Wd = np.empty((D * T, C * T), dtype=np.float64)
    for t in range(T):
        for s in range(T):
            # block (t, s) of every (d, c) pair holds tap (t - s) mod T
            Wd[t::T, s::T] = W[:, :, (t - s) % T]
    return Wd


def forward(x, W, bias=None):
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
    Wd = unroll_block_circulant(W)
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


def forward_act(x, W, bias=None, act=None):
    """act(forward(x, W, bias)): the activation applied to every output value
    after the bias (a pointwise map, so the result stays equivariant)."""
    return ACTIVATIONS[act](forward(x, W, bias))


def backward_input(dy, W):
    """dx = dy_flat . Wd (the transpose of the forward map), in fp64.

    Gradient of the forward with respect to x; the pages state that the method
    covers the backward pass ("Implementazione") without writing it out.
    """
    dy = _f64(dy)
    N, D, T = dy.shape
    C = np.shape(W)[1]
    Wd = unroll_block_circulant(W)
    return (dy.reshape(N, D * T) @ Wd).reshape(N, C, T)


def backward_weight(x, dy):
    """(dW, dbias) for the compact weight and the per-channel bias, in fp64.

    The dense gradient is dWd = dy_flat^T . x_flat.  Each compact entry
    W[d, c, r] appears in the dense matrix at every (t, s) with (t - s) mod T
    == r, so its gradient is the sum of those replicas:
        dW[d, c, r] = sum_t dWd[d*T + t, c*T + (t - r) mod T].
    dbias[d] = sum over rows and group elements of dy[:, d, :].
    """
    x = _f64(x)
    dy = _f64(dy)
    N, C, T = x.shape
    D = dy.shape[1]
    dWd = dy.reshape(N, D * T).T @ x.reshape(N, C * T)  # (D*T, C*T)
    dW = np.zeros((D, C, T), dtype=np.float64)
    for r in range(T):
        for t in range(T):
            s = (t - r) % T
            dW[:, :, r] += dWd[t::T, s::T]
    dbias = dy.sum(axis=(0, 2))
    return dW, dbias


def mac_counts(N, C, D, T):
    """(spectral MACs, dense MACs) per forward, with C and D per group element.

    Dense: the unrolled (D*T) x (C*T) matrix times N rows, T^2 * N*C*D.
    Spectral (authors' abstract; "Specializzazione per il Gruppo di Rotazione
    p4"): by conjugate symmetry of the real DFT only frequencies 0..floor(T/2)
    are formed; k = 0 (and k = T/2 for even T) are real and cost one real
    N x C x D product each, every other kept frequency is complex and costs
    four.  For even T this totals 2(T - 1) products; p4 gives 6 against 16.
    """
    real_freqs = 2 if T % 2 == 0 else 1
    complex_freqs = T // 2 + 1 - real_freqs
    spectral = (real_freqs + 4 * complex_freqs) * N * C * D
    dense = T * T * N * C * D
    return spectral, dense


def param_counts(C, D, T):
    """(compact, dense) parameter counts of the weight ("Livello di Rete":
    about T times fewer parameters than the dense layer of equal width)."""
    return D * C * T, (D * T) * (C * T)
