"""GPU parity of the two-pass forward of the quantized linear (qf_linear_forward_mxfp4,
qf_linear_forward_nvfp4): QDQ of each flagged operand into a bf16 buffer, then the BF16
GEMM with no QDQ.

- Xq and Wq equal the oracle's QDQ bit for bit;
- Y equals the fused kernel's output (qf_gemm_mxfp4 / qf_gemm_nvfp4 with the same flags)
  bit for bit: the matrix cores see the same values in the same order;
- Y obeys the per-element bound against the float64 product of the oracle's operands.
Shapes: small and ragged (several tiles, partial tiles), strided operands and outputs,
in-place QDQ (Xq = X), and the 32768 x 14336 x 4096 workload (bit equality everywhere,
oracle on sampled rows and columns).
"""

import numpy as np
import pytest
import torch

import fp4_fake_quant_amd as fq
import workloads
from oracle import gemm, mxfp4, nvfp4
from oracle import primitives as P
from tests.gpu_util import dev, host, sample_rows, first_mismatch

pytestmark = pytest.mark.gpu
RNG = np.random.default_rng(2024)


def _check(Y, Xq, Wq, K, what):
    y_ref = gemm.reference(Xq, Wq)
    bound = gemm.elementwise_bound(y_ref, gemm.abs_dot(Xq, Wq), K)
    y = P.bf16_to_f32(Y).astype(np.float64)
    bad = np.argwhere(np.abs(y - y_ref) > bound)
    assert bad.size == 0, f"{what}: {bad.shape[0]} elements over the bound, first {tuple(bad[0])}"
    rel = np.linalg.norm(y - y_ref) / max(np.linalg.norm(y_ref), 1e-300)
    assert rel <= 1e-2, f"{what}: relative Frobenius error {rel}"
    return rel


def _ops(M, N, K):
    X = P.f32_to_bf16((RNG.standard_t(3, size=(M, K)) * 0.5).astype(np.float32))
    W = P.f32_to_bf16((RNG.standard_normal((N, K)) * 0.02).astype(np.float32))
    return X, W


def _same(a, b, what):
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{what}: {first_mismatch(host(a), host(b))}"


SHAPES = [(256, 256, 64), (300, 200, 128), (33, 517, 192), (1, 1, 64), (513, 257, 256)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("flags", [3, 1, 2, 3 | 8])
def test_forward_mxfp4_small(shape, flags):
    M, N, K = shape
    X, W = _ops(M, N, K)
    rule = "noclip" if flags & 8 else "floor"
    Xd, Wd = dev(X), dev(W)
    Y, Xq, Wq = fq.qf_linear_forward_mxfp4(Xd, Wd, flags=flags)
    Xq_ref = mxfp4.qdq(X, rule=rule) if flags & 1 else X
    Wq_ref = mxfp4.qdq(W, rule=rule) if flags & 2 else W
    if flags & 1:
        assert np.array_equal(host(Xq), Xq_ref), first_mismatch(host(Xq), Xq_ref)
    else:
        assert Xq is None
    if flags & 2:
        assert np.array_equal(host(Wq), Wq_ref), first_mismatch(host(Wq), Wq_ref)
    _same(Y, fq.qf_gemm_mxfp4(Xd, Wd, flags=flags), f"two-pass vs fused {shape} flags={flags}")
    _check(host(Y), Xq_ref, Wq_ref, K, f"{shape} flags={flags}")


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("flags", [3, 1, 2])
def test_forward_nvfp4_small(shape, flags):
    M, N, K = shape
    X, W = _ops(M, N, K)
    Xd, Wd = dev(X), dev(W)
    sx, sw = fq.qf_nvfp4_tensor_scale(Xd), fq.qf_nvfp4_tensor_scale(Wd)
    sx_ref, sw_ref = nvfp4.tensor_scale([X]), nvfp4.tensor_scale([W])
    a, b = (sx if flags & 1 else None), (sw if flags & 2 else None)
    Y, Xq, Wq = fq.qf_linear_forward_nvfp4(Xd, Wd, a, b, flags=flags)
    Xq_ref = nvfp4.qdq(X, sx_ref) if flags & 1 else X
    Wq_ref = nvfp4.qdq(W, sw_ref) if flags & 2 else W
    if flags & 1:
        assert np.array_equal(host(Xq), Xq_ref), first_mismatch(host(Xq), Xq_ref)
    if flags & 2:
        assert np.array_equal(host(Wq), Wq_ref), first_mismatch(host(Wq), Wq_ref)
    _same(Y, fq.qf_gemm_nvfp4(Xd, Wd, a, b, flags=flags), f"nvfp4 two-pass vs fused {shape} flags={flags}")
    _check(host(Y), Xq_ref, Wq_ref, K, f"nvfp4 {shape} flags={flags}")


def test_forward_strided_and_in_place():
    M, N, K = 320, 288, 192
    X, W = _ops(M, N, K)
    X[:, 5] = P.f32_to_bf16(np.full(M, 300.0, np.float32))       # an outlier channel
    X[7] = 0
    Xb = torch.zeros((M, K + 64), dtype=torch.bfloat16, device="cuda")
    Xb[:, 32:32 + K] = dev(X)
    Wd = dev(W)
    Xqb = torch.full((M, K + 32), 9.0, dtype=torch.bfloat16, device="cuda")
    Yb = torch.full((M, N + 40), 7.0, dtype=torch.bfloat16, device="cuda")
    fq.qf_linear_forward_mxfp4(Xb[:, 32:32 + K], Wd, Yb[:, 8:8 + N], flags=3, Xq=Xqb[:, 16:16 + K])
    assert np.array_equal(host(Xqb[:, 16:16 + K]), mxfp4.qdq(X))
    assert torch.all(Xqb[:, :16] == 9.0) and torch.all(Xqb[:, 16 + K:] == 9.0)
    assert torch.all(Yb[:, :8] == 7.0) and torch.all(Yb[:, 8 + N:] == 7.0)
    _same(Yb[:, 8:8 + N].contiguous(), fq.qf_gemm_mxfp4(Xb[:, 32:32 + K], Wd), "strided two-pass vs fused")
    _check(host(Yb[:, 8:8 + N]), mxfp4.qdq(X), mxfp4.qdq(W), K, "strided")
    # in place: X and W overwritten by their QDQ
    Xi, Wi = dev(X), dev(W)
    Y, Xq, Wq = fq.qf_linear_forward_mxfp4(Xi, Wi, Xq=Xi, Wq=Wi)
    assert Xq.data_ptr() == Xi.data_ptr()
    assert np.array_equal(host(Xi), mxfp4.qdq(X)) and np.array_equal(host(Wi), mxfp4.qdq(W))
    _check(host(Y), mxfp4.qdq(X), mxfp4.qdq(W), K, "in place")


def test_forward_full_size():
    """The 32768 x 14336 x 4096 workload: Y equal to the fused kernels' everywhere (MXFP4
    and NVFP4); the oracle checks 48 sampled rows x 48 sampled columns and sampled rows
    of Xq and Wq."""
    g = workloads.w4a4_gemm()
    X, W = g["X"], g["W"]
    K = X.shape[1]
    rows = sample_rows(X.shape[0], 48, seed=5)
    cols = sample_rows(W.shape[0], 48, seed=6)
    Xd, Wd = dev(X), dev(W)
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    Y, Xq, Wq = fq.qf_linear_forward_mxfp4(Xd, Wd)
    _same(Y, fq.qf_gemm_mxfp4(Xd, Wd), "full size mxfp4 two-pass vs fused")
    Xq_ref, Wq_ref = mxfp4.qdq(X[rows]), mxfp4.qdq(W[cols])
    assert np.array_equal(host(Xq[ri]), Xq_ref) and np.array_equal(host(Wq[ci]), Wq_ref)
    assert _check(host(Y[ri][:, ci]), Xq_ref, Wq_ref, K, "full size mxfp4") < 2e-3
    sx, sw = fq.qf_nvfp4_tensor_scale(Xd), fq.qf_nvfp4_tensor_scale(Wd)
    Y, Xq, Wq = fq.qf_linear_forward_nvfp4(Xd, Wd, sx, sw, Y=Y, Xq=Xq, Wq=Wq)
    _same(Y, fq.qf_gemm_nvfp4(Xd, Wd, sx, sw), "full size nvfp4 two-pass vs fused")
    sx_ref, sw_ref = nvfp4.tensor_scale([X]), nvfp4.tensor_scale([W])
    Xq_ref, Wq_ref = nvfp4.qdq(X[rows], sx_ref), nvfp4.qdq(W[cols], sw_ref)
    assert np.array_equal(host(Xq[ri]), Xq_ref) and np.array_equal(host(Wq[ci]), Wq_ref)
    assert _check(host(Y[ri][:, ci]), Xq_ref, Wq_ref, K, "full size nvfp4") < 2e-3


def test_forward_nvfp4_tracked_activation_scale():
    """NVFP4 W4A4 training steps with a tracked activation scale: each step's activations
    update the running amax on the device (qf_nvfp4_tensor_scale_tracked), and the forward
    quantizes X with the tracked scale.  State, scale, Xq and Y checked against the oracle
    after every step; one step with an outlier raises the state, later smaller batches keep
    it; the state is per group (two tied groups, Q/K/V-like activations tied)."""
    M, N, K = 200, 160, 128
    W = P.f32_to_bf16((RNG.standard_normal((N, K)) * 0.02).astype(np.float32))
    Wd = dev(W)
    sw = fq.qf_nvfp4_tensor_scale(Wd)
    sw_ref = nvfp4.tensor_scale([W])
    amax_d = torch.zeros(2, dtype=torch.float32, device="cuda")
    amax_ref = [np.float32(0.0), np.float32(0.0)]
    for step in range(5):
        X = (RNG.standard_t(3, size=(M, K)) * 0.5).astype(np.float32)
        if step == 1:
            X[3, 7] = 900.0                                          # an outlier the state keeps
        X = P.f32_to_bf16(X)
        X2 = P.f32_to_bf16((RNG.standard_normal((64, K)) * (step + 1)).astype(np.float32))
        Xd, X2d = dev(X), dev(X2)
        sc = fq.qf_nvfp4_tensor_scale_tracked([dict(x=Xd, group=0), dict(x=X2d, group=1)], 2, amax_d)
        s_ref = []
        for g, t in ((0, X), (1, X2)):
            amax_ref[g], s = nvfp4.tracked_scale(amax_ref[g], [t])
            s_ref.append(s)
        got_amax, got_s = amax_d.cpu().numpy(), sc.cpu().numpy()
        assert np.array_equal(got_amax.view(np.uint32), np.array(amax_ref, np.float32).view(np.uint32)), step
        assert np.array_equal(got_s.view(np.uint32), np.array(s_ref, np.float32).view(np.uint32)), step
        Y, Xq, Wq = fq.qf_linear_forward_nvfp4(Xd, Wd, sc[0:1], sw, flags=3)
        Xq_ref, Wq_ref = nvfp4.qdq(X, s_ref[0]), nvfp4.qdq(W, sw_ref)
        assert np.array_equal(host(Xq), Xq_ref), f"step {step}: {first_mismatch(host(Xq), Xq_ref)}"
        _check(host(Y), Xq_ref, Wq_ref, K, f"tracked step {step}")
    assert amax_ref[0] == np.float32(900.0)
