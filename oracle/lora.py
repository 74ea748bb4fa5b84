"""LoRA merge-then-quantize and adapter gradients (oracle; test infrastructure only).

Source: QATFactory project page, "Method" section, "Quantization-aware
distillation": LoRA-QAD keeps one frozen base, trains only the adapters and
quantizes the merged weight; for MoE models it merges and quantizes one expert
at a time to bound peak memory.  With the identity STE (see ste.py) the
gradient that reaches the merged weight M = W + B.A passes to the adapters as
dB = G . A^T and dA = B^T . G.

Readings (stated choices):
* No alpha/r factor: the merge is exactly W + B.A (B is [rows, r], A is
  [r, cols]).
* Merge arithmetic: acc = 0; for k = 0 .. r-1 in order, acc = fl(acc +
  fl(B[i,k] * A[k,j])) in float32 (each bf16 x bf16 product is exact in
  float32, so this equals a chain of fused multiply-adds);
  M[i,j] = bf16(fl(W[i,j] + acc)).  M is then quantized like any weight
  (NVFP4 with one tensor scale per expert per fused matrix).
* Adapter gradients: float64 reference (exact products, BLAS sums).

Pins: B = 0 gives M = W bit for bit; power-of-two adapters give the exact sum;
float64 adapter gradients against math.fsum on sampled entries;
tests/test_oracle_misc.py.
"""

import numpy as np

from .primitives import bf16_to_f32, f32_to_bf16


def merge(W_bits, A_bits, B_bits):
    """BF16 bits of M = bf16(W + sum_k B[:,k] A[k,:]) with the fixed float32 order."""
    W = bf16_to_f32(W_bits)
    A = bf16_to_f32(A_bits)
    B = bf16_to_f32(B_bits)
    r = A.shape[0]
    acc = np.zeros(W.shape, np.float32)
    for k in range(r):
        acc = (acc + (B[:, k:k + 1] * A[k:k + 1, :]).astype(np.float32)).astype(np.float32)
    return f32_to_bf16((W + acc).astype(np.float32))


def adapter_grads(G_bits, A_bits, B_bits):
    """float64 (dA [r, cols], dB [rows, r]) for M = W + B.A under the identity STE."""
    G = bf16_to_f32(G_bits).astype(np.float64)
    A = bf16_to_f32(A_bits).astype(np.float64)
    B = bf16_to_f32(B_bits).astype(np.float64)
    dB = G @ A.T
    dA = B.T @ G
    return dA, dB
