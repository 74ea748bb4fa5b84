"""Reference for the BF16 matmul on QDQ'd operands (oracle; test infrastructure only).

Source: QATFactory project page, "Overview" and the arXiv abstract on the
index page: simulated quantization rounds weights, and optionally activations,
onto the format grid while every matrix multiplication runs in BF16; "Key
findings" 02: MXFP4 benefits from quantizing activations too (W4A4 training).

Y = QDQ(X) . QDQ(W)^T with X [M, K] (tokens x hidden) and W [N, K]
(out x in), blocks along K.  The reference is float64 (numpy matmul / BLAS) on
the bit-exact QDQ'd operands.  An fp32-accumulating kernel that rounds its
output to bf16 satisfies, for every output element,

    |y - y_ref| <= 2^-8 |y_ref| + (1 + 2^-8) * gamma_K * sum_k |xq_k wq_k|,
    gamma_K = K u / (1 - K u),  u = 2^-24,

Higham's bound for recursive summation in any order (Accuracy and Stability of
Numerical Algorithms, sec. 3.1) plus one bf16 rounding of the result.

Pins: float64 matmul against exact math.fsum dot products on sampled entries;
tests/test_oracle_misc.py.
"""

import numpy as np

from .primitives import bf16_to_f32


def reference(Xq_bits, Wq_bits):
    X = bf16_to_f32(Xq_bits).astype(np.float64)
    W = bf16_to_f32(Wq_bits).astype(np.float64)
    return X @ W.T


def abs_dot(Xq_bits, Wq_bits):
    X = np.abs(bf16_to_f32(Xq_bits).astype(np.float64))
    W = np.abs(bf16_to_f32(Wq_bits).astype(np.float64))
    return X @ W.T


def gamma(K, u=2.0 ** -24):
    return K * u / (1.0 - K * u)


def elementwise_bound(y_ref, absdot, K, out_unit=2.0 ** -8):
    """Largest |y - y_ref| allowed per element for an fp32-accumulated, bf16-rounded result."""
    return out_unit * np.abs(y_ref) + (1.0 + out_unit) * gamma(K) * absdot
