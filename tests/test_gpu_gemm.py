"""GPU parity of the fused W4A4 MXFP4 GEMM against the float64 oracle.

Y = QDQ(X) . QDQ(W)^T is checked element by element against the per-element bound
|y - y_ref| <= 2^-8 |y_ref| + (1 + 2^-8) gamma_K sum_k |xq_k wq_k| (fp32 accumulation
in any order plus one bf16 rounding) and in relative Frobenius norm (<= 1e-2), where
y_ref is the exact float64 product of the oracle's bit-exact MXFP4 QDQ of X and W.
"""

import numpy as np
import pytest
import torch

import fp4_fake_quant_amd as fq
import workloads
from oracle import gemm, mxfp4, nvfp4
from oracle import primitives as P
from tests.gpu_util import dev, host, sample_rows

pytestmark = pytest.mark.gpu
RNG = np.random.default_rng(99)


def _check(Y, Xq, Wq, K, what):
    y_ref = gemm.reference(Xq, Wq)
    bound = gemm.elementwise_bound(y_ref, gemm.abs_dot(Xq, Wq), K)
    y = P.bf16_to_f32(Y).astype(np.float64)
    err = np.abs(y - y_ref)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{what}: {bad.shape[0]} elements over the bound, first {tuple(bad[0])}: " \
                          f"got {y[tuple(bad[0])]} want {y_ref[tuple(bad[0])]} bound {bound[tuple(bad[0])]}"
    rel = np.linalg.norm(y - y_ref) / max(np.linalg.norm(y_ref), 1e-300)
    assert rel <= 1e-2, f"{what}: relative Frobenius error {rel}"
    return rel


def _ops(M, N, K, scale_x=0.5, scale_w=0.02):
    X = P.f32_to_bf16((RNG.standard_t(3, size=(M, K)) * scale_x).astype(np.float32))
    W = P.f32_to_bf16((RNG.standard_normal((N, K)) * scale_w).astype(np.float32))
    return X, W


@pytest.mark.parametrize("shape", [(256, 256, 64), (300, 200, 128), (33, 517, 192), (1, 1, 64), (513, 257, 256)])
@pytest.mark.parametrize("flags", [3, 1, 2, 0, 7])
def test_gemm_small_shapes(shape, flags):
    M, N, K = shape
    X, W = _ops(M, N, K)
    Y = fq.qf_gemm_mxfp4(dev(X), dev(W), flags=flags)
    Xq = mxfp4.qdq(X) if flags & 1 else X
    Wq = mxfp4.qdq(W) if flags & 2 else W
    _check(host(Y), Xq, Wq, K, f"{shape} flags={flags}")


@pytest.mark.parametrize("shape", [(256, 256, 64), (300, 200, 128), (33, 517, 192), (513, 257, 256), (64, 96, 320)])
def test_gemm_packed_w_matches_in_kernel_fp4_path(shape):
    """W packed by qf_pack_mxfp4 feeds the FP4 cores directly: same bound, and the same
    bits as quantizing W inside the GEMM (identical operands, identical MFMA order)."""
    M, N, K = shape
    X, W = _ops(M, N, K)
    Wc, Ws = fq.qf_pack_mxfp4(dev(W))
    Y = fq.qf_gemm_mxfp4_packed_w(dev(X), Wc, Ws)
    _check(host(Y), mxfp4.qdq(X), mxfp4.qdq(W), K, f"packed W {shape}")
    Y2 = fq.qf_gemm_mxfp4(dev(X), dev(W), flags=7)
    assert np.array_equal(host(Y), host(Y2))


@pytest.mark.parametrize("shape", [(256, 256, 128), (300, 200, 256), (33, 517, 384), (513, 257, 512), (1, 1, 128),
                                   (64, 96, 896)])
def test_gemm_both_packed_matches_packed_w(shape):
    """X and W both packed by qf_pack_mxfp4: buffer-to-LDS path, same bound and the same
    bits as the packed-W path (the same MFMAs in the same K order)."""
    M, N, K = shape
    X, W = _ops(M, N, K)
    Xc, Xs = fq.qf_pack_mxfp4(dev(X))
    Wc, Ws = fq.qf_pack_mxfp4(dev(W))
    Y = fq.qf_gemm_mxfp4_packed(Xc, Xs, Wc, Ws)
    _check(host(Y), mxfp4.qdq(X), mxfp4.qdq(W), K, f"both packed {shape}")
    assert np.array_equal(host(Y), host(fq.qf_gemm_mxfp4_packed_w(dev(X), Wc, Ws)))


def test_gemm_strided_operands_and_output():
    M, N, K = 320, 288, 192
    X, W = _ops(M, N, K)
    Xb = torch.zeros((M, K + 64), dtype=torch.bfloat16, device="cuda")
    Xb[:, 32:32 + K] = dev(X)
    Wb = torch.zeros((N, K + 128), dtype=torch.bfloat16, device="cuda")
    Wb[:, :K] = dev(W)
    Yb = torch.full((M, N + 40), 7.0, dtype=torch.bfloat16, device="cuda")
    for flags in (3, 7):
        Yb.fill_(7.0)
        fq.qf_gemm_mxfp4(Xb[:, 32:32 + K], Wb[:, :K], Yb[:, 8:8 + N], flags=flags)
        _check(host(Yb[:, 8:8 + N]), mxfp4.qdq(X), mxfp4.qdq(W), K, f"strided flags={flags}")
        assert torch.all(Yb[:, :8] == 7.0) and torch.all(Yb[:, 8 + N:] == 7.0)


def test_gemm_outlier_columns_and_zero_rows():
    M, N, K = 256, 256, 256
    X, W = _ops(M, N, K)
    X[:, 5] = P.f32_to_bf16(np.full(M, 300.0, np.float32))     # an outlier channel
    X[7] = 0
    X[9] = 0x8000
    W[3] = 0
    for flags in (3, 7):
        Y = fq.qf_gemm_mxfp4(dev(X), dev(W), flags=flags)
        _check(host(Y), mxfp4.qdq(X), mxfp4.qdq(W), K, f"outliers flags={flags}")
        assert np.all(P.bf16_to_f32(host(Y))[7] == 0) and np.all(P.bf16_to_f32(host(Y))[:, 3] == 0)


def test_gemm_w4a4_full_size_sampled():
    """The 32768 x 14336 x 4096 workload in the launch the benchmark times; the oracle
    checks 64 sampled rows x 64 sampled columns (plus the first and last of each)."""
    g = workloads.w4a4_gemm()
    X, W = g["X"], g["W"]
    rows = sample_rows(X.shape[0], 64, seed=1)
    cols = sample_rows(W.shape[0], 64, seed=2)
    Xq, Wq = mxfp4.qdq(X[rows]), mxfp4.qdq(W[cols])
    Xd, Wd = dev(X), dev(W)
    Wc, Ws = fq.qf_pack_mxfp4(Wd)
    Xc, Xs = fq.qf_pack_mxfp4(Xd)
    for name, Y in (("bf16 cores", fq.qf_gemm_mxfp4(Xd, Wd)), ("fp4 cores", fq.qf_gemm_mxfp4(Xd, Wd, flags=7)),
                    ("packed W", fq.qf_gemm_mxfp4_packed_w(Xd, Wc, Ws)),
                    ("both packed", fq.qf_gemm_mxfp4_packed(Xc, Xs, Wc, Ws))):
        Ys = host(Y[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
        rel = _check(Ys, Xq, Wq, X.shape[1], f"full size, {name}")
        assert rel < 2e-3
        del Y


# ----------------------------------------------------------- NVFP4 W4A4 ----
def _nv_scale(bits):
    """The operand's tensor scale on the device (qf_nvfp4_tensor_scale) after checking it
    against the oracle's, so both sides quantize with the same fp32."""
    s_dev = fq.qf_nvfp4_tensor_scale(dev(bits))
    s_ref = nvfp4.tensor_scale([bits])
    torch.cuda.synchronize()
    assert np.float32(s_dev.cpu().numpy()[0]).view(np.uint32) == np.float32(s_ref).view(np.uint32)
    return s_dev, s_ref


@pytest.mark.parametrize("shape", [(256, 256, 64), (300, 200, 128), (33, 517, 192), (1, 1, 64), (513, 257, 256)])
@pytest.mark.parametrize("flags", [3, 1, 2])
def test_gemm_nvfp4_small_shapes(shape, flags):
    M, N, K = shape
    X, W = _ops(M, N, K)
    sx, sx_ref = _nv_scale(X)
    sw, sw_ref = _nv_scale(W)
    Y = fq.qf_gemm_nvfp4(dev(X), dev(W), sx if flags & 1 else None, sw if flags & 2 else None, flags=flags)
    Xq = nvfp4.qdq(X, sx_ref) if flags & 1 else X
    Wq = nvfp4.qdq(W, sw_ref) if flags & 2 else W
    _check(host(Y), Xq, Wq, K, f"nvfp4 {shape} flags={flags}")


def test_gemm_nvfp4_caller_scales():
    """The kernel quantizes with whatever fp32 the scale pointers hold (a tracked activation
    scale): one far below the data's (block scales saturate at 448, codes at 6) and one far
    above it (many blocks round to zero)."""
    M, N, K = 192, 320, 256
    X, W = _ops(M, N, K)
    for sx_val, sw_val in ((1e-5, 3e-6), (0.5, 0.01)):
        sx = torch.tensor([sx_val], dtype=torch.float32, device="cuda")
        sw = torch.tensor([sw_val], dtype=torch.float32, device="cuda")
        Y = fq.qf_gemm_nvfp4(dev(X), dev(W), sx, sw)
        _check(host(Y), nvfp4.qdq(X, np.float32(sx_val)), nvfp4.qdq(W, np.float32(sw_val)), K,
               f"nvfp4 scales {sx_val}, {sw_val}")


def test_gemm_nvfp4_strided_outliers_and_zero_rows():
    M, N, K = 320, 288, 192
    X, W = _ops(M, N, K)
    X[:, 5] = P.f32_to_bf16(np.full(M, 300.0, np.float32))     # an outlier channel
    X[7] = 0
    X[9] = 0x8000
    W[3] = 0
    sx, sx_ref = _nv_scale(X)
    sw, sw_ref = _nv_scale(W)
    Xb = torch.zeros((M, K + 64), dtype=torch.bfloat16, device="cuda")
    Xb[:, 32:32 + K] = dev(X)
    Wb = torch.zeros((N, K + 128), dtype=torch.bfloat16, device="cuda")
    Wb[:, :K] = dev(W)
    Yb = torch.full((M, N + 40), 7.0, dtype=torch.bfloat16, device="cuda")
    fq.qf_gemm_nvfp4(Xb[:, 32:32 + K], Wb[:, :K], sx, sw, Yb[:, 8:8 + N])
    Y = host(Yb[:, 8:8 + N])
    _check(Y, nvfp4.qdq(X, sx_ref), nvfp4.qdq(W, sw_ref), K, "nvfp4 strided")
    assert torch.all(Yb[:, :8] == 7.0) and torch.all(Yb[:, 8 + N:] == 7.0)
    assert np.all(P.bf16_to_f32(Y)[7] == 0) and np.all(P.bf16_to_f32(Y)[:, 3] == 0)


def test_gemm_nvfp4_full_size_sampled():
    """NVFP4 W4A4 at the 32768 x 14336 x 4096 shape, tensor scales from the tensor-scale
    pass; 64 sampled rows x 64 sampled columns against the oracle."""
    g = workloads.w4a4_gemm()
    X, W = g["X"], g["W"]
    rows = sample_rows(X.shape[0], 64, seed=3)
    cols = sample_rows(W.shape[0], 64, seed=4)
    sx_ref, sw_ref = nvfp4.tensor_scale([X]), nvfp4.tensor_scale([W])
    Xd, Wd = dev(X), dev(W)
    sx, sw = fq.qf_nvfp4_tensor_scale(Xd), fq.qf_nvfp4_tensor_scale(Wd)
    Y = fq.qf_gemm_nvfp4(Xd, Wd, sx, sw)
    assert np.float32(sx.cpu().numpy()[0]) == sx_ref and np.float32(sw.cpu().numpy()[0]) == sw_ref
    Ys = host(Y[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    rel = _check(Ys, nvfp4.qdq(X[rows], sx_ref), nvfp4.qdq(W[cols], sw_ref), X.shape[1], "nvfp4 full size")
    assert rel < 2e-3


@pytest.mark.parametrize("shape", [(256, 256, 64), (300, 200, 128), (33, 517, 192)])
@pytest.mark.parametrize("flags", [3, 1, 2])
def test_gemm_mxfp4_noclip(shape, flags):
    """QF_MX_NOCLIP: both operands quantized under the noclip exponent rule."""
    M, N, K = shape
    X, W = _ops(M, N, K)
    Y = fq.qf_gemm_mxfp4(dev(X), dev(W), flags=flags | fq.QF_MX_NOCLIP)
    Xq = mxfp4.qdq(X, rule="noclip") if flags & 1 else X
    Wq = mxfp4.qdq(W, rule="noclip") if flags & 2 else W
    _check(host(Y), Xq, Wq, K, f"noclip {shape} flags={flags}")


def test_gemm_mxfp4_noclip_top_binade():
    """W rows whose 32-blocks have maxima up to the largest finite bf16 (the planted maxima
    of the noclip pins, two blocks per row), X scaled by 2^-120 so the products stay finite:
    the fused noclip QDQ must cap the exponent at 252 as the oracle does (a block maximum in
    [1.75, 2) * 2^127 would otherwise dequantize to 2^128 and turn the row into Inf)."""
    from tests import pins
    b = pins.planted_mx_blocks()
    b = b[(b[:, 31] & 0x7F80) >= (191 << 7)]                 # maxima of 2^64 and above: no fp32 underflow
    assert b.shape[0] >= 8 and np.any((b[:, 31] & 0x7FFF) == 0x7F7F)
    b = np.ascontiguousarray(b[: b.shape[0] // 2 * 2].reshape(-1, 64))
    N, K = b.shape
    M = 96
    X = P.f32_to_bf16((RNG.standard_t(3, size=(M, K)) * np.ldexp(1.0, -120)).astype(np.float32))
    for flags in (2, 3):
        Y = fq.qf_gemm_mxfp4(dev(X), dev(b), flags=flags | fq.QF_MX_NOCLIP)
        Xq = mxfp4.qdq(X, rule="noclip") if flags & 1 else X
        Wq = mxfp4.qdq(b, rule="noclip")
        assert np.all(np.isfinite(P.bf16_to_f32(Wq)))
        _check(host(Y), Xq, Wq, K, f"noclip top binade flags={flags}")
        Y2, _, Wq_d = fq.qf_linear_forward_mxfp4(dev(X), dev(b), flags=flags | fq.QF_MX_NOCLIP)
        assert np.array_equal(host(Wq_d), Wq)
        assert np.array_equal(host(Y2), host(Y))


# ------------------------------------------- more tiles than workgroups ----
@pytest.mark.parametrize("K", [64, 192])
def test_gemm_many_tiles_per_workgroup(K):
    """22 x 15 tiles with ragged last tile row and column, more tiles than the launch has
    workgroups (at most one per CU), so workgroups run several tiles in turn and load the
    next tile's first K slice during the last one (K = 64: a single K step per tile).
    Each product is checked against the oracle, and Y must be the same bits whichever way
    it is stored: 16-byte rows through LDS, 8-byte stores (ldy = N + 4) and element stores
    (ldy = N + 1); the fused kernel must equal the two-pass forward."""
    M, N = 21 * 256 + 37, 14 * 256 + 96
    X, W = _ops(M, N, K)
    Xd, Wd = dev(X), dev(W)
    Xq, Wq = mxfp4.qdq(X), mxfp4.qdq(W)
    for flags in (0, 3):
        ys = []
        for pad in (0, 4, 1):
            Yb = torch.full((M, N + pad), 7.0, dtype=torch.bfloat16, device="cuda")
            fq.qf_gemm_mxfp4(Xd, Wd, Yb[:, :N], flags=flags)
            if pad:
                assert torch.all(Yb[:, N:] == 7.0)
            ys.append(host(Yb[:, :N]))
        _check(ys[0], Xq if flags else X, Wq if flags else W, K, f"many tiles K={K} flags={flags}")
        assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2]), f"store modes, flags={flags}"
        if flags:
            Y2, _, _ = fq.qf_linear_forward_mxfp4(Xd, Wd)
            assert np.array_equal(host(Y2), ys[0])
    sx, sx_ref = _nv_scale(X)
    sw, sw_ref = _nv_scale(W)
    Y = fq.qf_gemm_nvfp4(Xd, Wd, sx, sw)
    _check(host(Y), nvfp4.qdq(X, sx_ref), nvfp4.qdq(W, sw_ref), K, f"nvfp4 many tiles K={K}")


@pytest.mark.parametrize("ldy", [(1 << 22) - 8, (1 << 22) + 8])
def test_gemm_output_stride_at_the_store_limit(ldy):
    """Y rows 2^22 - 8 elements apart (the widest stride that still leaves through LDS in
    16-byte buffer stores: a tile's rows then span just under 2^31 bytes) and 2^22 + 8
    (8-byte stores from the accumulators instead), two tile rows with a ragged second;
    the columns past N stay untouched."""
    M, N, K = 260, 136, 128
    X, W = _ops(M, N, K)
    Yb = torch.full((M, ldy), 7.0, dtype=torch.bfloat16, device="cuda")
    fq.qf_gemm_mxfp4(dev(X), dev(W), Yb[:, :N], flags=3)
    _check(host(Yb[:, :N]), mxfp4.qdq(X), mxfp4.qdq(W), K, f"ldy={ldy}")
    assert torch.all(Yb[:, N:N + 256] == 7.0) and torch.all(Yb[:, -8:] == 7.0)
    del Yb
