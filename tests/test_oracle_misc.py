"""Pins of the oracle's STE, LoRA merge, adapter gradients and GEMM reference."""

import math

import numpy as np

import torch

from oracle import gemm, lora, nvfp4, ste
from oracle import primitives as P
from oracle import mxfp4
from tests import pins

RNG = np.random.default_rng(5)


def _bf(x):
    return pins.bf16_torch(np.asarray(x, np.float32))


# ------------------------------------------------------------------ STE ----
def test_ste_identity_and_accumulate():
    g = _bf(RNG.standard_normal((64, 96)))
    out = ste.ste_backward(g)
    assert np.array_equal(out, pins.widen(g).astype(np.float32))       # exact widening
    acc = RNG.standard_normal((64, 96)).astype(np.float32)
    out2 = ste.ste_backward(g, acc, accumulate=True)
    want = pins.f32(acc.astype(np.float64) + pins.widen(g))             # one rounding per element
    assert np.array_equal(out2.view(np.uint32), want.view(np.uint32))


# ----------------------------------------------------------------- LoRA ----
def test_lora_zero_B_is_identity():
    W = _bf(RNG.standard_normal((32, 64)) * 0.02)
    A = _bf(RNG.standard_normal((16, 64)) * 0.01)
    B = np.zeros((32, 16), np.uint16)
    assert np.array_equal(lora.merge(W, A, B), W)


def test_lora_power_of_two_adapters_give_exact_sum():
    W = _bf(RNG.standard_normal((32, 64)) * 0.02)
    A = _bf(np.exp2(RNG.integers(-10, -5, size=(16, 64))) * RNG.choice([-1, 1], size=(16, 64)))
    B = _bf(np.exp2(RNG.integers(-10, -5, size=(32, 16))) * RNG.choice([-1, 1], size=(32, 16)))
    exact = pins.widen(W) + pins.widen(B) @ pins.widen(A)               # exact: few bits, close exponents
    assert np.all(np.abs(pins.f32(exact).astype(np.float64) - exact) == 0)
    assert np.array_equal(lora.merge(W, A, B), _bf(exact))


def test_lora_merge_order_is_ascending_k():
    """Products [1, 2^-24, 2^-24] in k order: ascending gives fl(fl(1 + 2^-24) + 2^-24) = 1
    (both sums are ties to even), descending would give 1 + 2^-23.  With W = -1 the merged
    value is therefore exactly 0 (hand-derived from the stated order)."""
    A = _bf([[1.0], [2.0 ** -12], [2.0 ** -12]])          # r = 3, cols = 1
    B = _bf([[1.0, 2.0 ** -12, 2.0 ** -12]])              # rows = 1
    W = _bf([[-1.0]])
    assert lora.merge(W, A, B)[0, 0] == 0
    W = _bf([[0.0]])
    assert lora.merge(W, A, B)[0, 0] == 0x3F80             # bf16(1.0)


def test_lora_merge_within_rounding_of_exact():
    W = _bf(RNG.standard_normal((48, 80)) * 0.02)
    A = _bf(RNG.standard_normal((16, 80)) * 0.01)
    B = _bf(RNG.standard_normal((48, 16)) * 0.001)
    M = pins.widen(lora.merge(W, A, B))
    exact = pins.widen(W) + pins.widen(B) @ pins.widen(A)
    absum = np.abs(pins.widen(B)) @ np.abs(pins.widen(A))
    # bf16 half-ulp of the result plus 16 fp32 roundings of the partial sums
    tol = np.abs(exact) * 2.0 ** -8 + 17 * 2.0 ** -24 * (absum + np.abs(exact))
    assert np.all(np.abs(M - exact) <= tol)


def test_adapter_grads_against_fsum():
    G = _bf(RNG.standard_normal((24, 40)))
    A = _bf(RNG.standard_normal((16, 40)) * 0.01)
    B = _bf(RNG.standard_normal((24, 16)) * 0.001)
    dA, dB = lora.adapter_grads(G, A, B)
    g, a, b = pins.widen(G), pins.widen(A), pins.widen(B)
    for (i, k) in [(0, 0), (23, 15), (7, 3), (11, 9)]:
        assert math.isclose(dB[i, k], math.fsum(g[i, j] * a[k, j] for j in range(40)), rel_tol=1e-13, abs_tol=1e-300)
    for (k, j) in [(0, 0), (15, 39), (4, 17)]:
        assert math.isclose(dA[k, j], math.fsum(b[i, k] * g[i, j] for i in range(24)), rel_tol=1e-13, abs_tol=1e-300)
    assert dA.shape == (16, 40) and dB.shape == (24, 16)


# ----------------------------------------------------------------- GEMM ----
def test_gemm_reference_against_fsum_and_bound():
    X = _bf(RNG.standard_t(3, size=(20, 96)) * 0.5)
    W = _bf(RNG.standard_normal((12, 96)) * 0.02)
    Xq, Wq = mxfp4.qdq(X), mxfp4.qdq(W)
    Y = gemm.reference(Xq, Wq)
    xv, wv = pins.widen(Xq), pins.widen(Wq)
    for (i, j) in [(0, 0), (19, 11), (5, 7)]:
        assert Y[i, j] == math.fsum(xv[i, k] * wv[j, k] for k in range(96))
    # an fp32 sequential accumulation, rounded to bf16, satisfies the per-element bound
    acc = np.zeros((20, 12), np.float32)
    for k in range(96):
        acc = (acc + (xv[:, k:k + 1] * wv[None, :, k]).astype(np.float32)).astype(np.float32)
    y = pins.widen(_bf(acc))
    bound = gemm.elementwise_bound(Y, gemm.abs_dot(Xq, Wq), 96)
    assert np.all(np.abs(y - Y) <= bound)
    assert gemm.gamma(4096) < 2.45e-4


def test_tracked_scale_is_the_scale_of_all_batches_seen():
    """The tracked NVFP4 activation scale after any number of batches is the tensor scale of
    all those batches taken together (a max over their union, from torch's amax of the
    float values), in any order of the batches; a zero state with a zero batch gives 1."""
    rng = np.random.default_rng(17)
    batches = []
    for i in range(6):
        x = (rng.standard_t(3, size=(64, 128)) * (0.5 if i != 3 else 4.0)).astype(np.float32)
        batches.append(P.f32_to_bf16(x))
    for order in (range(6), [5, 2, 0, 4, 1, 3]):
        amax = np.float32(0.0)
        seen = []
        for i in order:
            amax, s_t = nvfp4.tracked_scale(amax, [batches[i]])
            seen.append(batches[i])
            union = torch.from_numpy(P.bf16_to_f32(np.concatenate(seen)))
            want_amax = np.float32(union.abs().max().item())
            assert amax == want_amax
            assert s_t == np.float32(np.float64(want_amax) / 2688.0)      # one rounding of A / 2688
        assert amax == np.float32(max(np.abs(P.bf16_to_f32(b)).max() for b in batches))
    z = np.zeros((4, 16), np.uint16)
    assert nvfp4.tracked_scale(np.float32(0.0), [z]) == (np.float32(0.0), np.float32(1.0))
    # a batch below the state leaves it unchanged
    big = np.float32(np.abs(P.bf16_to_f32(batches[3])).max() * 2)
    amax, s_t = nvfp4.tracked_scale(big, [batches[0]])
    assert amax == big and s_t == np.float32(np.float64(big) / 2688.0)
