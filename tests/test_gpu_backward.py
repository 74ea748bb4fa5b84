"""GPU parity of the backward products of the quantized linear layer and of the transpose.

qf_transpose_bf16 is compared bit for bit with the oracle (x^T, or QDQ(x)^T under the
MXFP4 rule).  qf_linear_backward_mxfp4's dX = dY . Wq and dW = dY^T . Xq are compared
element by element with the float64 products of the oracle's QDQ'd operands, within
|y - y_ref| <= 2^-8 |y_ref| + (1 + 2^-8) gamma_n sum |products| (fp32 accumulation in
any order plus one bf16 rounding; n = N for dX, M for dW), and in relative Frobenius
norm.  At the 32768 x 14336 x 4096 shape the oracle checks sampled rows and sampled
32-column blocks of K (whole MXFP4 blocks, so the QDQ'd columns are exact).
"""

import numpy as np
import pytest
import torch

import fp4_fake_quant_amd as fq
import workloads
from oracle import gemm, mxfp4
from oracle import primitives as P
from tests.gpu_util import dev, host, first_mismatch, sample_rows

pytestmark = pytest.mark.gpu
RNG = np.random.default_rng(4242)


def _bits(a):
    return P.f32_to_bf16(np.asarray(a, np.float32))


def _check(got_bits, A_bits, B_bits, n, what):
    """got ~ A . B^T (float64 reference on bf16 bit inputs)."""
    y_ref = gemm.reference(A_bits, B_bits)
    bound = gemm.elementwise_bound(y_ref, gemm.abs_dot(A_bits, B_bits), n)
    y = P.bf16_to_f32(got_bits).astype(np.float64)
    err = np.abs(y - y_ref)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{what}: {bad.shape[0]} over the bound, first {tuple(bad[0])}"
    rel = np.linalg.norm(y - y_ref) / max(np.linalg.norm(y_ref), 1e-300)
    assert rel <= 1e-2, f"{what}: relative Frobenius error {rel}"
    return rel


_TR_CASES = [(shape, mode) for shape in [(64, 64), (200, 96), (8, 32), (520, 1056), (64, 8)]
             for mode in ("copy", "floor", "noclip") if mode == "copy" or shape[1] % 32 == 0]


@pytest.mark.parametrize("shape,mode", _TR_CASES)
def test_transpose_bit_exact(shape, mode):
    rows, cols = shape
    x = _bits(RNG.standard_t(3, size=(rows, cols)) * 0.3)
    rule = fq.QF_MX_RULE_NOCLIP if mode == "noclip" else fq.QF_MX_RULE_FLOOR
    y = host(fq.qf_transpose_bf16(dev(x), qdq_mxfp4=mode != "copy", rule=rule))
    want = (x if mode == "copy" else mxfp4.qdq(x, rule=mode)).T
    assert np.array_equal(y, want), first_mismatch(y, want)


@pytest.mark.parametrize("rule", ["floor", "noclip"])
def test_transpose_planted_maxima(rule):
    """Block maxima at every decision of both exponent rules, up to the largest finite bf16
    (which must not become Inf under noclip)."""
    from tests import pins
    b = pins.planted_mx_blocks()
    b = np.ascontiguousarray(b[: b.shape[0] // 8 * 8])
    r = fq.QF_MX_RULE_NOCLIP if rule == "noclip" else fq.QF_MX_RULE_FLOOR
    y = host(fq.qf_transpose_bf16(dev(b), qdq_mxfp4=True, rule=r))
    want = mxfp4.qdq(b, rule=rule).T
    assert np.array_equal(y, want), first_mismatch(y, want)
    assert not np.any((y & 0x7F80) == 0x7F80)


def test_transpose_tallest_source():
    """The largest row count the call takes (rows < 2^22, a multiple of 8) spans more
    row tiles than one launch grid holds; the launcher splits it into bands."""
    rows, cols = (1 << 22) - 8, 8
    x = RNG.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint64).astype(np.uint16)
    y = host(fq.qf_transpose_bf16(dev(x)))
    assert np.array_equal(y, x.T), first_mismatch(y, x.T)


def test_transpose_strided():
    rows, cols = 72, 96
    x = _bits(RNG.standard_normal((rows, cols)))
    xb = torch.zeros((rows, cols + 32), dtype=torch.bfloat16, device="cuda")
    xb[:, 16:16 + cols] = dev(x)
    yb = torch.full((cols, rows + 24), 3.0, dtype=torch.bfloat16, device="cuda")
    fq.qf_transpose_bf16(xb[:, 16:16 + cols], yb[:, 8:8 + rows], qdq_mxfp4=True)
    assert np.array_equal(host(yb[:, 8:8 + rows]), mxfp4.qdq(x).T)
    assert torch.all(yb[:, :8] == 3.0) and torch.all(yb[:, 8 + rows:] == 3.0)


@pytest.mark.parametrize("shape", [(64, 64, 32), (128, 192, 96), (320, 256, 160)])
@pytest.mark.parametrize("flags", [3, 0, 1, 2, 11, 9, 10])
def test_linear_backward_small(shape, flags):
    """flags 8 | ...: QF_MX_NOCLIP, the backward of a forward run under the noclip rule."""
    M, N, K = shape
    X = _bits(RNG.standard_t(3, size=(M, K)) * 0.5)
    W = _bits(RNG.standard_normal((N, K)) * 0.02)
    dY = _bits(RNG.standard_normal((M, N)))
    dX, dW = fq.qf_linear_backward_mxfp4(dev(X), dev(W), dev(dY), flags=flags)
    rule = "noclip" if flags & 8 else "floor"
    Xq = mxfp4.qdq(X, rule=rule) if flags & 1 else X
    Wq = mxfp4.qdq(W, rule=rule) if flags & 2 else W
    _check(host(dX), dY, np.ascontiguousarray(Wq.T), N, f"dX {shape} flags={flags}")
    _check(host(dW), np.ascontiguousarray(dY.T), np.ascontiguousarray(Xq.T), M, f"dW {shape} flags={flags}")


def test_linear_backward_one_output():
    M, N, K = 128, 64, 64
    X, W = _bits(RNG.standard_normal((M, K))), _bits(RNG.standard_normal((N, K)) * 0.02)
    dY = _bits(RNG.standard_normal((M, N)))
    dX, dW = fq.qf_linear_backward_mxfp4(dev(X), dev(W), dev(dY), want=(True, False))
    assert dW is None
    _check(host(dX), dY, np.ascontiguousarray(mxfp4.qdq(W).T), N, "dX only")
    dX, dW = fq.qf_linear_backward_mxfp4(dev(X), dev(W), dev(dY), want=(False, True))
    assert dX is None
    _check(host(dW), np.ascontiguousarray(dY.T), np.ascontiguousarray(mxfp4.qdq(X).T), M, "dW only")


def test_linear_backward_full_size_sampled():
    """The W4A4 GEMM shape (X 32768 x 4096, W 14336 x 4096) with an N(0,1) upstream
    gradient dY [32768, 14336] drawn on the device; sampled rows of dX and dW on 4
    sampled 32-blocks of K."""
    g = workloads.w4a4_gemm()
    X, W = g["X"], g["W"]
    M, K = X.shape
    N = W.shape[0]
    gen = torch.Generator(device="cuda").manual_seed(7)
    dYd = torch.randn((M, N), generator=gen, device="cuda").to(torch.bfloat16)
    dX, dW = fq.qf_linear_backward_mxfp4(dev(X), dev(W), dYd)
    torch.cuda.synchronize()
    kb = np.sort(np.random.default_rng(8).choice(K // 32, 4, replace=False))
    kcols = np.concatenate([np.arange(32 * b, 32 * b + 32) for b in kb])
    mrows = sample_rows(M, 48, seed=9)
    nrows = sample_rows(N, 48, seed=10)
    # dX[m, k] = sum_n dY[m, n] Wq[n, k]
    dY_m = host(dYd[torch.from_numpy(mrows).cuda()])
    Wq_k = mxfp4.qdq(np.ascontiguousarray(W[:, kcols]))
    got = host(dX[torch.from_numpy(mrows).cuda()][:, torch.from_numpy(kcols).cuda()])
    rel = _check(got, dY_m, np.ascontiguousarray(Wq_k.T), N, "dX full size")
    assert rel < 2e-3
    # dW[n, k] = sum_m dY[m, n] Xq[m, k]
    dY_n = host(dYd[:, torch.from_numpy(nrows).cuda()])
    Xq_k = mxfp4.qdq(np.ascontiguousarray(X[:, kcols]))
    got = host(dW[torch.from_numpy(nrows).cuda()][:, torch.from_numpy(kcols).cuda()])
    rel = _check(got, np.ascontiguousarray(dY_n.T), np.ascontiguousarray(Xq_k.T), M, "dW full size")
    assert rel < 2e-3
