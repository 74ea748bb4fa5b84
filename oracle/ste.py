"""Straight-through estimator backward (oracle; test infrastructure only).

Source: QATFactory project page, "Method" section, "Framework overview": the
forward pass applies the lossy quantize-dequantize transform and the backward
pass uses a straight-through estimator to update the continuous latent
weights (the STE of Bengio et al., "Estimating or Propagating Gradients
Through Stochastic Neurons", in the page's bibliography).

Reading (stated choice): the plain identity STE with no clipping mask, so the
gradient of the latent weight is the gradient of the QDQ'd weight:
g_latent = f32(g_q), or g_latent += f32(g_q) when accumulating (one float32
rounding per element).

Pins: exact widening (bf16 -> f32 is exact) and float32 accumulation checked
against float64 sums of two terms; tests/test_oracle_misc.py.
"""

import numpy as np

from .primitives import bf16_to_f32


def ste_backward(g_q_bits, g_latent=None, accumulate=False):
    g = bf16_to_f32(g_q_bits)
    if accumulate:
        return (np.asarray(g_latent, np.float32) + g).astype(np.float32)
    return g.copy()
