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

A second reading is kept as an option, the clipped STE: the gradient reaches the latent
weight only where the quantizer did not saturate the element (its scaled magnitude lay
within the grid, see nvfp4.saturated and mxfp4.saturated); a saturated element gets
+0.0, or adds +0.0 when accumulating.

Pins: exact widening (bf16 -> f32 is exact) and float32 accumulation checked
against float64 sums of two terms; tests/test_oracle_misc.py.  The saturation
masks: tests/test_oracle_ste_clip.py.
"""

import numpy as np

from .primitives import F32, bf16_to_f32


def ste_backward(g_q_bits, g_latent=None, accumulate=False):
    g = bf16_to_f32(g_q_bits)
    if accumulate:
        return (np.asarray(g_latent, np.float32) + g).astype(np.float32)
    return g.copy()


def ste_backward_clipped(g_q_bits, saturated, g_latent=None, accumulate=False):
    """Clipped STE: f32(g_q) where the element was not saturated, +0.0 where it was."""
    g = np.where(np.asarray(saturated, bool), F32(0.0), bf16_to_f32(g_q_bits)).astype(np.float32)
    if accumulate:
        return (np.asarray(g_latent, np.float32) + g).astype(np.float32)
    return g
