"""GPU parity of the clipped STE (qf_ste_backward_clipped_nvfp4 / _mxfp4) against the
oracle, bit for bit on the fp32 output (+0.0 where the quantizer saturated, f32(g_q)
elsewhere, or those added to g_latent).

Cases: the 256 x 512 workload under the tensor-scale pass's s_t and under caller scales
far below and above it; MXFP4 under the floor and the noclip rule; ragged rows, one block
per row, strided x; accumulation onto existing values (including -0.0); empty tensors; the
dense 8B layer at full size (every element against the oracle's mask on sampled rows, and
the count of saturated elements against the oracle's over whole matrices).
"""

import numpy as np
import pytest
import torch

import fp4_fake_quant_amd as fq
import workloads
from oracle import mxfp4, nvfp4, ste
from oracle import primitives as P
from tests.gpu_util import dev, first_mismatch, sample_rows

pytestmark = pytest.mark.gpu
RNG = np.random.default_rng(321)


def f32(t):
    return t.detach().cpu().numpy()


def same_bits(got, want, what):
    got, want = np.asarray(got, np.float32), np.asarray(want, np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{what}: {first_mismatch(got.view(np.uint32), want.view(np.uint32))}"


def _g(shape):
    return P.f32_to_bf16(RNG.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("scale", ["tensor", 1e-5, 0.5])
def test_nvfp4_workload(scale):
    w = workloads.single_256x512()
    x, g = w["W"], w["G"]
    xd = dev(x)
    if scale == "tensor":
        sd = fq.qf_nvfp4_tensor_scale(xd)
        s_t = nvfp4.tensor_scale([x])
    else:
        s_t = np.float32(scale)
        sd = torch.tensor([float(s_t)], dtype=torch.float32, device="cuda")
    mask = nvfp4.saturated(x, s_t)
    got = f32(fq.qf_ste_backward_clipped_nvfp4(dev(g), xd, sd))
    same_bits(got, ste.ste_backward_clipped(g, mask), f"nvfp4 scale={scale}")
    assert 0 < mask.sum() < mask.size or scale == 0.5
    acc0 = RNG.standard_normal(x.shape).astype(np.float32)
    acc0[:3] = -0.0
    acc = torch.from_numpy(acc0.copy()).cuda()
    fq.qf_ste_backward_clipped_nvfp4(dev(g), xd, sd, acc, accumulate=True)
    same_bits(f32(acc), ste.ste_backward_clipped(g, mask, acc0, accumulate=True), f"nvfp4 acc scale={scale}")


@pytest.mark.parametrize("rule", [fq.QF_MX_RULE_FLOOR, fq.QF_MX_RULE_NOCLIP])
def test_mxfp4_workload(rule):
    w = workloads.single_256x512()
    x, g = w["W"], w["G"]
    r = "noclip" if rule == fq.QF_MX_RULE_NOCLIP else "floor"
    mask = mxfp4.saturated(x, r)
    got = f32(fq.qf_ste_backward_clipped_mxfp4(dev(g), dev(x), rule=rule))
    same_bits(got, ste.ste_backward_clipped(g, mask), f"mxfp4 {r}")
    acc0 = np.full(x.shape, -0.0, np.float32)
    acc = torch.from_numpy(acc0.copy()).cuda()
    fq.qf_ste_backward_clipped_mxfp4(dev(g), dev(x), acc, accumulate=True, rule=rule)
    same_bits(f32(acc), ste.ste_backward_clipped(g, mask, acc0, accumulate=True), f"mxfp4 acc {r}")


# (1, 384) and (3, 160) leave 48 and 60 chunks in the last wave: its second half of lanes
# (4 elements each, two halves of 64 chunks per wave segment) is only partly filled
@pytest.mark.parametrize("shape", [(37, 768), (5, 32), (1, 64), (300, 96), (1, 384), (3, 160)])
@pytest.mark.parametrize("accumulate", [False, True])
def test_ragged_and_strided(shape, accumulate):
    rows, cols = shape
    x = P.f32_to_bf16((RNG.standard_t(3, size=(rows, cols)) * 0.3).astype(np.float32))
    g = _g((rows, cols))
    xb = torch.zeros((rows, cols + 40), dtype=torch.bfloat16, device="cuda")
    xb[:, 24:24 + cols] = dev(x)
    xs = xb[:, 24:24 + cols]
    acc0 = RNG.standard_normal((rows, cols)).astype(np.float32)

    def run(call, mask, what):
        if accumulate:
            out = torch.from_numpy(acc0.copy()).cuda()
            call(out)
            same_bits(f32(out), ste.ste_backward_clipped(g, mask, acc0, accumulate=True), what)
        else:
            same_bits(f32(call(None)), ste.ste_backward_clipped(g, mask), what)

    for rule, r in ((fq.QF_MX_RULE_FLOOR, "floor"), (fq.QF_MX_RULE_NOCLIP, "noclip")):
        run(lambda o: fq.qf_ste_backward_clipped_mxfp4(dev(g), xs, o, accumulate=accumulate, rule=rule),
            mxfp4.saturated(x, r), f"mxfp4 {r} {shape} acc={accumulate}")
    s_t = nvfp4.tensor_scale([x])
    sd = torch.tensor([float(s_t)], dtype=torch.float32, device="cuda")
    run(lambda o: fq.qf_ste_backward_clipped_nvfp4(dev(g), xs, sd, o, accumulate=accumulate),
        nvfp4.saturated(x, s_t), f"nvfp4 {shape} acc={accumulate}")


@pytest.mark.parametrize("rule", [fq.QF_MX_RULE_FLOOR, fq.QF_MX_RULE_NOCLIP])
def test_mxfp4_top_binade(rule):
    """Block maxima up to the largest finite bf16: under both rules the blocks in the top
    binade take E = 252 and elements above 6 * 2^125 saturate (the mask is the oracle's)."""
    from tests import pins
    x = pins.planted_mx_blocks()
    r = "noclip" if rule == fq.QF_MX_RULE_NOCLIP else "floor"
    mask = mxfp4.saturated(x, r)
    assert mask[x[:, 31] & 0x7FFF == 0x7F7F].any()
    g = _g(x.shape)
    same_bits(f32(fq.qf_ste_backward_clipped_mxfp4(dev(g), dev(x), rule=rule)), ste.ste_backward_clipped(g, mask),
              f"mxfp4 {r} planted maxima")


def test_empty():
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    assert fq.qf_ste_backward_clipped_mxfp4(e, e).shape == (0, 64)


def test_dense_layer_full_size():
    """The dense 8B layer's four matrices at full size, each under its own tensor scale:
    sampled rows against the oracle bit for bit, and the saturated count of every whole
    matrix (elements where the output is +0.0 but the gradient is not) against the oracle's."""
    layer = workloads.dense_layer_8b(with_grad=True)
    for name, (x, g) in layer.items():
        xd, gd = dev(x), dev(g)
        sd = fq.qf_nvfp4_tensor_scale(xd)
        s_t = nvfp4.tensor_scale([x])
        rows = sample_rows(x.shape[0], 16, seed=len(name))
        ri = torch.from_numpy(rows).cuda()
        for fmt in ("nvfp4", "mxfp4"):
            if fmt == "nvfp4":
                out = fq.qf_ste_backward_clipped_nvfp4(gd, xd, sd)
                mask = nvfp4.saturated(x, s_t)
            else:
                out = fq.qf_ste_backward_clipped_mxfp4(gd, xd)
                mask = mxfp4.saturated(x)
            same_bits(f32(out[ri]), ste.ste_backward_clipped(g[rows], mask[rows]), f"{name} {fmt} sampled rows")
            gz = torch.from_numpy(P.bf16_to_f32(g) == 0).cuda()
            zeroed = int(((out == 0) & ~gz).sum().item())
            assert zeroed == int((mask & (P.bf16_to_f32(g) != 0)).sum()), f"{name} {fmt} saturated count"
            del out
        del xd, gd
        torch.cuda.empty_cache()
