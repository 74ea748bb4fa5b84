"""GPU parity: the stacked-experts LoRA calls (qf_lora_experts_*).

One descriptor covers E experts of one shape stored one after another; expert e uses
tied group group + e * group_stride.  Each expert's tensor scale, QDQ'd weight, packed
codes and block scales must be the oracle's bits, its adapter gradients within the
fp32 bound, and everything must equal, bit for bit, what the grouped calls give for the
same expert as a descriptor of its own (the kernels are the same; only the launch
covers more matrices).  Cases: ragged shapes and an odd rank, group strides 1 and 2,
the accumulate flag, and the MoE share's real shapes with 8 and 32 experts per call.
"""

import numpy as np
import pytest
import torch

import fp4_fake_quant_amd as fq
from oracle import lora, nvfp4
from tests.gpu_util import dev, host, u8, f32bits, first_mismatch
from tests.test_gpu_lora import make_case, check_grads

pytestmark = pytest.mark.gpu


def assert_same(got, want, what):
    assert np.array_equal(got, want), f"{what}: {first_mismatch(got, want)}"


def stacked(cases):
    """Device tensors [E, ...] of per-expert cases (make_case dicts) plus outputs."""
    E = len(cases)
    rows, cols = cases[0]["W"].shape
    r = cases[0]["A"].shape[0]
    st = lambda k: torch.stack([dev(c[k]) for c in cases])
    return dict(
        W=st("W"), A=st("A"), B=st("B"), G=st("G"),
        y=torch.empty((E, rows, cols), dtype=torch.bfloat16, device="cuda"),
        codes=torch.empty((E, rows, cols // 2), dtype=torch.uint8, device="cuda"),
        scales=torch.empty((E, rows, cols // 16), dtype=torch.uint8, device="cuda"),
        dA=torch.empty((E, r, cols), dtype=torch.float32, device="cuda"),
        dB=torch.empty((E, rows, r), dtype=torch.float32, device="cuda"),
    )


def run_experts(descs, n_groups, accumulate=False):
    ex = fq.LoraExperts(descs)
    s = fq.qf_lora_experts_merge_tensor_scale_nvfp4(ex, n_groups)
    fq.qf_lora_experts_merge_qdq_pack_nvfp4(ex, s)
    fq.qf_lora_experts_adapter_grads(ex, accumulate=accumulate)
    torch.cuda.synchronize()
    return s.cpu().numpy()


@pytest.mark.parametrize("stride", [1, 2])
def test_experts_against_the_oracle(stride):
    """Two descriptors (3 experts of 100 x 1056 rank 16, 3 of 37 x 544 rank 7), groups
    0, s, 2s and 1, 1 + s, 1 + 2s (stride 1: the two descriptors share groups 1 and 2)."""
    shapes = [(100, 1056, 16), (37, 544, 7)]
    per = [[make_case(r_, c_, k_, seed=40 + 10 * j + e, a_scale=0.1, b_scale=0.1) for e in range(3)]
           for j, (r_, c_, k_) in enumerate(shapes)]
    descs = []
    for j, cases in enumerate(per):
        d = stacked(cases)
        d.update(group=j, group_stride=stride)
        descs.append(d)
    n_groups = 1 + 2 * stride + 1
    s = run_experts(descs, n_groups)
    members = {}
    for j, cases in enumerate(per):
        for e, c in enumerate(cases):
            members.setdefault(j + e * stride, []).append(lora.merge(c["W"], c["A"], c["B"]))
    s_want = [nvfp4.tensor_scale(members[g]) if g in members else np.float32(1.0) for g in range(n_groups)]
    assert_same(f32bits(s[:n_groups]), f32bits(s_want), "tensor scales")
    for j, cases in enumerate(per):
        d = descs[j]
        for e, c in enumerate(cases):
            g = j + e * stride
            M = lora.merge(c["W"], c["A"], c["B"])
            codes, S = nvfp4.quantize(M, s_want[g])
            pc, ps = nvfp4.pack(codes, S)
            assert_same(host(d["y"][e]), nvfp4.dequantize(codes, S, s_want[g]), f"y[{j}][{e}]")
            assert_same(u8(d["codes"][e]), pc, f"codes[{j}][{e}]")
            assert_same(u8(d["scales"][e]), ps, f"block scales[{j}][{e}]")
            check_grads(c, d["dA"][e].cpu().numpy(), d["dB"][e].cpu().numpy(), f"expert {j}/{e}")


def _grouped_twin(descs):
    """The same experts as single-expert descriptors of the grouped calls, with outputs
    of their own; returns (items, groups)."""
    items = []
    for d in descs:
        E = d["W"].shape[0]
        for e in range(E):
            items.append(dict(W=d["W"][e], A=d["A"][e], B=d["B"][e], G=d["G"][e],
                              group=d["group"] + e * d["group_stride"], M=None,
                              y=torch.empty_like(d["y"][e]), codes=torch.empty_like(d["codes"][e]),
                              scales=torch.empty_like(d["scales"][e]), dA=torch.empty_like(d["dA"][e]),
                              dB=torch.empty_like(d["dB"][e])))
    return items


def _compare_with_grouped(descs, n_groups, chunk):
    s = run_experts(descs, n_groups)
    items = _grouped_twin(descs)
    s2 = torch.empty(n_groups, dtype=torch.float32, device="cuda")
    for c0 in range(0, len(items), chunk):
        part = items[c0:c0 + chunk]
        # the grouped call takes group indices below its own n_groups: remap per chunk
        gs = sorted({it["group"] for it in part})
        local = [dict(it, group=gs.index(it["group"])) for it in part]
        b = fq.LoraBatch(local)
        sl = fq.qf_lora_merge_tensor_scale_nvfp4_grouped(b, len(gs))
        fq.qf_lora_merge_qdq_pack_nvfp4_grouped(b, sl)
        fq.qf_lora_adapter_grads_grouped(b)
        s2[torch.tensor(gs, device="cuda")] = sl
    torch.cuda.synchronize()
    assert_same(f32bits(s), f32bits(s2.cpu().numpy()), "tensor scales")
    k = 0
    for d in descs:
        for e in range(d["W"].shape[0]):
            it = items[k]
            for name in ("y", "codes", "scales"):
                assert torch.equal(d[name][e], it[name]), f"{name} of expert {k}"
            for name in ("dA", "dB"):
                assert torch.equal(d[name][e].view(torch.int32), it[name].view(torch.int32)), f"{name} of expert {k}"
            k += 1


def test_experts_equal_the_grouped_calls_ragged():
    shapes = [(70, 608, 5), (129, 1056, 16)]
    descs = []
    for j, (r_, c_, k_) in enumerate(shapes):
        cases = [make_case(r_, c_, k_, seed=300 + 7 * j + e) for e in range(4)]
        d = stacked(cases)
        d.update(group=j, group_stride=2)
        descs.append(d)
    _compare_with_grouped(descs, 8, chunk=16)


@pytest.mark.parametrize("experts", [8, 32])
def test_experts_real_shapes_equal_the_grouped_calls(experts):
    """The MoE share's matrices (gate/up 3072 x 3072, down 3072 x 1536, rank 16): one call
    for all experts against the grouped calls 8 experts at a time, every bit."""
    g = torch.Generator(device="cuda").manual_seed(experts)
    descs = []
    for j, (rows, cols) in enumerate(((3072, 3072), (3072, 1536))):
        kw = dict(generator=g, device="cuda")
        d = dict(W=(torch.randn((experts, rows, cols), **kw) * 0.02).bfloat16(),
                 A=(torch.randn((experts, 16, cols), **kw) * 0.01).bfloat16(),
                 B=(torch.randn((experts, rows, 16), **kw) * 0.001).bfloat16(),
                 G=torch.randn((experts, rows, cols), **kw).bfloat16(),
                 y=torch.empty((experts, rows, cols), dtype=torch.bfloat16, device="cuda"),
                 codes=torch.empty((experts, rows, cols // 2), dtype=torch.uint8, device="cuda"),
                 scales=torch.empty((experts, rows, cols // 16), dtype=torch.uint8, device="cuda"),
                 dA=torch.empty((experts, 16, cols), dtype=torch.float32, device="cuda"),
                 dB=torch.empty((experts, rows, 16), dtype=torch.float32, device="cuda"),
                 group=j, group_stride=2)
        descs.append(d)
    # interleave the grouped twin's order as the bench does: expert-major
    _compare_with_grouped(descs, 2 * experts, chunk=16)


def test_experts_accumulate():
    cases = [make_case(64, 512, 16, seed=900 + e) for e in range(3)]
    d = stacked(cases)
    d.update(group=0, group_stride=1)
    run_experts([d], 3)
    first = (d["dA"].clone(), d["dB"].clone())
    run_experts([d], 3, accumulate=True)
    for e, c in enumerate(cases):
        want_dA, want_dB = lora.adapter_grads(c["G"], c["A"], c["B"])
        got_dA = d["dA"][e].cpu().numpy().astype(np.float64)
        got_dB = d["dB"][e].cpu().numpy().astype(np.float64)
        # accumulate adds the same fp32 values again: exactly twice the first result's sum
        assert np.array_equal(d["dA"][e].cpu().numpy(), (first[0][e] + first[0][e]).cpu().numpy())
        assert np.array_equal(d["dB"][e].cpu().numpy(), (first[1][e] + first[1][e]).cpu().numpy())
        assert np.allclose(got_dA, 2 * want_dA, rtol=1e-4, atol=1e-6)
        assert np.allclose(got_dB, 2 * want_dB, rtol=1e-4, atol=1e-6)
