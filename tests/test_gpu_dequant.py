"""GPU parity of the dequant (packed -> BF16) entry points against the oracle.

Two kinds of input, each compared bit for bit:
- packed bytes the GPU pack calls wrote: dequant must give back exactly the QDQ'd bf16
  the fused QDQ+pack call wrote next to them, and the oracle's QDQ;
- arbitrary bytes inside the contract (every code, every scale byte a pack call can
  write, random Q4_K headers with finite non-negative d and dmin, every 6-bit sc/m):
  the oracle's dequantize of its own unpack is the reference.
Shapes: the 256 x 512 workload, ragged row counts, one block per row, strided outputs,
empty tensors, and the dense 8B layer at full size (sampled rows).
"""

import numpy as np
import pytest
import torch

import fp4_fake_quant_amd as fq
import workloads
from oracle import mxfp4, nvfp4, q4k
from tests.gpu_util import dev, host, first_mismatch, sample_rows

pytestmark = pytest.mark.gpu
RNG = np.random.default_rng(1234)


def assert_same(got, want, what):
    assert np.array_equal(got, want), f"{what}: {first_mismatch(got, want)}"


def t8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def f32dev(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("shape", [(256, 512), (37, 768), (3, 96), (1, 256), (5, 4096)])
def test_dequant_inverts_gpu_pack(shape):
    rows, cols = shape
    x = workloads.to_bf16_bits(RNG.standard_normal((rows, cols)).astype(np.float32) * 0.02)
    xd = dev(x)
    # NVFP4
    s = fq.qf_nvfp4_tensor_scale(xd)
    y, c, sc = fq.qf_qdq_pack_nvfp4(xd, s)
    assert_same(host(fq.qf_dequant_nvfp4(c, sc, s)), host(y), "nvfp4 dequant vs QDQ")
    assert_same(host(y), nvfp4.qdq(x, nvfp4.tensor_scale([x])), "nvfp4 QDQ vs oracle")
    # MXFP4
    y, c, sc = fq.qf_qdq_pack_mxfp4(xd)
    assert_same(host(fq.qf_dequant_mxfp4(c, sc)), host(y), "mxfp4 dequant vs QDQ")
    assert_same(host(y), mxfp4.qdq(x), "mxfp4 QDQ vs oracle")
    if cols % 256:
        return                                                       # no whole Q4_K super-block
    # Q4_K
    y, b = fq.qf_qdq_pack_q4k(xd)
    assert_same(host(fq.qf_dequant_q4k(b, rows, cols)), host(y), "q4k dequant vs QDQ")
    assert_same(host(y), q4k.qdq(x), "q4k QDQ vs oracle")


@pytest.mark.parametrize("rows,cols", [(64, 512), (3, 16 * 33)])
def test_dequant_nvfp4_arbitrary_bytes(rows, cols):
    codes = RNG.integers(0, 16, size=(rows, cols), dtype=np.uint8)
    S = RNG.integers(0, 0x7F, size=(rows, cols // 16), dtype=np.uint8)   # every E4M3 byte a pack writes
    if S.size >= 0x7F:
        S.flat[:0x7F] = np.arange(0x7F, dtype=np.uint8)
    pc, ps = nvfp4.pack(codes, S)
    for s_t in (np.float32(1.0), np.float32(3.1e-5), np.float32(0.75)):
        got = host(fq.qf_dequant_nvfp4(t8(pc), t8(ps), f32dev(float(s_t))))
        assert_same(got, nvfp4.dequantize(codes, S, s_t), f"nvfp4 bytes, s_t={s_t}")


@pytest.mark.parametrize("rows,cols", [(64, 512), (3, 32 * 9)])
def test_dequant_mxfp4_arbitrary_bytes(rows, cols):
    codes = RNG.integers(0, 16, size=(rows, cols), dtype=np.uint8)
    E = RNG.integers(0, 255, size=(rows, cols // 32), dtype=np.uint8)    # E8M0 0..254
    if E.size >= 255:
        E.flat[:255] = np.arange(255, dtype=np.uint8)
    pc, ps = mxfp4.pack(codes, E)
    assert_same(host(fq.qf_dequant_mxfp4(t8(pc), t8(ps))), mxfp4.dequantize(codes, E), "mxfp4 bytes")


@pytest.mark.parametrize("rows,cols", [(40, 1024), (1, 256)])
def test_dequant_q4k_arbitrary_bytes(rows, cols):
    nsb = cols // 256
    p = dict(d=RNG.integers(0, 0x7C00, size=(rows, nsb), dtype=np.uint16),        # finite, >= 0
             dmin=RNG.integers(0, 0x7C00, size=(rows, nsb), dtype=np.uint16),
             sc=RNG.integers(0, 64, size=(rows, nsb, 8), dtype=np.uint8),
             m=RNG.integers(0, 64, size=(rows, nsb, 8), dtype=np.uint8),
             q=RNG.integers(0, 16, size=(rows, cols), dtype=np.uint8))
    p["d"].flat[0], p["dmin"].flat[0] = 0, 0x7BFF                               # zero d, largest dmin
    blocks = q4k.pack(p)
    assert_same(host(fq.qf_dequant_q4k(t8(blocks), rows, cols)), q4k.dequantize(p), "q4k bytes")


def test_dequant_strided_output_and_empty():
    rows, cols = 48, 512
    x = workloads.to_bf16_bits(RNG.standard_normal((rows, cols)).astype(np.float32))
    xd = dev(x)
    yb = torch.full((rows, cols + 24), 5.0, dtype=torch.bfloat16, device="cuda")
    c, sc = fq.qf_pack_mxfp4(xd)
    fq.qf_dequant_mxfp4(c, sc, yb[:, 8:8 + cols])
    assert_same(host(yb[:, 8:8 + cols]), mxfp4.qdq(x), "strided y")
    assert torch.all(yb[:, :8] == 5.0) and torch.all(yb[:, 8 + cols:] == 5.0)
    b = fq.qf_pack_q4k(xd)
    yb.fill_(5.0)
    fq.qf_dequant_q4k(b, rows, cols, yb[:, 16:16 + cols])
    assert_same(host(yb[:, 16:16 + cols]), q4k.qdq(x), "strided y q4k")
    assert torch.all(yb[:, :16] == 5.0) and torch.all(yb[:, 16 + cols:] == 5.0)
    e = torch.empty((0, 256), dtype=torch.uint8, device="cuda")
    assert fq.qf_dequant_mxfp4(e[:, :128], torch.empty((0, 8), dtype=torch.uint8, device="cuda")).shape == (0, 256)


def test_dequant_dense_layer_full_size_sampled():
    """The dense 8B layer packed in NVFP4 (tied tensor scales per fused matrix) and Q4_K:
    dequant equals the fused QDQ output everywhere and the oracle on sampled rows."""
    layer = workloads.dense_layer_8b(with_grad=False)
    for name, (x, _) in layer.items():
        rows = sample_rows(x.shape[0], 24, seed=len(name))
        xd = dev(x)
        s = fq.qf_nvfp4_tensor_scale(xd)
        y, c, sc = fq.qf_qdq_pack_nvfp4(xd, s)
        yd = fq.qf_dequant_nvfp4(c, sc, s)
        assert torch.equal(yd.view(torch.int16), y.view(torch.int16)), f"{name}: nvfp4 dequant vs QDQ"
        assert_same(host(yd)[rows], nvfp4.qdq(x[rows], nvfp4.tensor_scale([x])), f"{name}: nvfp4 vs oracle")
        y, b = fq.qf_qdq_pack_q4k(xd)
        yd = fq.qf_dequant_q4k(b, *x.shape)
        assert torch.equal(yd.view(torch.int16), y.view(torch.int16)), f"{name}: q4k dequant vs QDQ"
        assert_same(host(yd)[rows], q4k.qdq(x[rows]), f"{name}: q4k vs oracle")
        del xd, y, yd, c, sc, b
        torch.cuda.empty_cache()
