"""GPU parity: LoRA merge-then-quantize per MoE expert and the adapter gradients.

The merged weight M, the tied NVFP4 tensor scales, the QDQ'd values, the packed
codes and the block scales are compared with the oracle bit for bit.  The fp32
adapter gradients are compared with the float64 reference within Higham's bound
for fp32 sums in any order (Accuracy and Stability of Numerical Algorithms,
sec. 3.1): |g - g_ref| <= gamma_n * sum |products| with n the number of terms.
Cases: ragged shapes (rows not a multiple of the 32-row unit, a partial last
512-column slab), strided W, odd rank (B rows starting on odd elements), rank 1,
several descriptors in one launch with shared and separate tied groups, the
accumulate flag, and one full-size MoE expert (gate/up 3072x3072 and down
3072x1536, rank 16).
"""

import numpy as np
import pytest
import torch

import fp4_fake_quant_amd as fq
import workloads
from oracle import lora, nvfp4
from oracle import primitives as P
from oracle.gemm import gamma
from tests.gpu_util import dev, host, u8, f32bits, first_mismatch, sample_rows

pytestmark = pytest.mark.gpu


def _bits(x):
    return P.f32_to_bf16(np.asarray(x, np.float32))


def assert_same(got, want, what):
    assert np.array_equal(got, want), f"{what}: {first_mismatch(got, want)}"


def make_case(rows, cols, r, seed, w_scale=0.02, a_scale=0.01, b_scale=0.001):
    rng = np.random.default_rng(seed)
    return dict(
        W=_bits(rng.standard_normal((rows, cols)) * w_scale),
        A=_bits(rng.standard_normal((r, cols)) * a_scale),
        B=_bits(rng.standard_normal((rows, r)) * b_scale),
        G=_bits(rng.standard_normal((rows, cols))),
    )


def device_item(c, group, ldw_pad=0, with_M=True):
    rows, cols = c["W"].shape
    r = c["A"].shape[0]
    if ldw_pad:
        Wfull = torch.zeros((rows, cols + ldw_pad), dtype=torch.bfloat16, device="cuda")
        Wfull[:, :cols] = dev(c["W"])
        W = Wfull[:, :cols]
    else:
        W = dev(c["W"])
    return dict(
        W=W, A=dev(c["A"]), B=dev(c["B"]), G=dev(c["G"]), group=group,
        M=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda") if with_M else None,
        y=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda"),
        codes=torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda"),
        scales=torch.empty((rows, cols // 16), dtype=torch.uint8, device="cuda"),
        dA=torch.empty((r, cols), dtype=torch.float32, device="cuda"),
        dB=torch.empty((rows, r), dtype=torch.float32, device="cuda"),
    )


def check_grads(c, dA, dB, what, extra_terms=0):
    dA_ref, dB_ref = lora.adapter_grads(c["G"], c["A"], c["B"])
    G = np.abs(P.bf16_to_f32(c["G"]).astype(np.float64))
    A = np.abs(P.bf16_to_f32(c["A"]).astype(np.float64))
    B = np.abs(P.bf16_to_f32(c["B"]).astype(np.float64))
    rows, cols = G.shape
    # dB sums cols products per entry, dA rows products (plus the partial sums)
    bound_dB = gamma(cols) * (G @ A.T)
    bound_dA = gamma(rows + extra_terms + 16) * (B.T @ G)
    errB = np.abs(dB.astype(np.float64) - dB_ref)
    errA = np.abs(dA.astype(np.float64) - dA_ref)
    assert np.all(errB <= bound_dB), f"{what} dB: worst excess {np.max(errB - bound_dB):.3e}"
    assert np.all(errA <= bound_dA), f"{what} dA: worst excess {np.max(errA - bound_dA):.3e}"


def run_merge_quant(items, n_groups):
    scales = fq.qf_lora_merge_tensor_scale_nvfp4_grouped(items, n_groups)
    fq.qf_lora_merge_qdq_pack_nvfp4_grouped(items, scales)
    torch.cuda.synchronize()
    return scales.cpu().numpy()


def check_merge_quant(cases, groups, items, s_got, n_groups):
    Ms = [lora.merge(c["W"], c["A"], c["B"]) for c in cases]
    for i, (M, it) in enumerate(zip(Ms, items)):
        if it["M"] is not None:
            assert_same(host(it["M"]), M, f"M[{i}]")
    s_want = []
    for g in range(n_groups):
        members = [M for M, gg in zip(Ms, groups) if gg == g]
        s_want.append(nvfp4.tensor_scale(members) if members else np.float32(1.0))
    assert_same(f32bits(s_got), f32bits(s_want), "tensor scales")
    for i, (M, it, g) in enumerate(zip(Ms, items, groups)):
        c, S = nvfp4.quantize(M, s_want[g])
        pc, ps = nvfp4.pack(c, S)
        if it["y"] is not None:
            assert_same(host(it["y"]), nvfp4.dequantize(c, S, s_want[g]), f"y[{i}]")
        if it["codes"] is not None:
            assert_same(u8(it["codes"]), pc, f"codes[{i}]")
            assert_same(u8(it["scales"]), ps, f"block scales[{i}]")


@pytest.mark.parametrize("rows,cols,r", [(100, 1056, 16), (37, 544, 7), (64, 32, 1), (33, 512, 16)])
def test_lora_single_descriptor(rows, cols, r):
    c = make_case(rows, cols, r, seed=rows * 7 + r)
    it = device_item(c, 0)
    s = run_merge_quant([it], 1)
    check_merge_quant([c], [0], [it], s, 1)
    fq.qf_lora_adapter_grads_grouped([it])
    torch.cuda.synchronize()
    check_grads(c, it["dA"].cpu().numpy(), it["dB"].cpu().numpy(), f"{rows}x{cols} r{r}")


def test_lora_grouped_strided_and_large_adapters():
    """Four descriptors in one launch, groups [0, 1, 0, 2], strided W, adapters big enough
    that the B.A term moves most bf16 values."""
    shapes = [(96, 1024, 16), (70, 608, 5), (129, 1056, 16), (16, 64, 3)]
    cases = [make_case(r_, c_, k_, seed=11 + i, a_scale=0.1, b_scale=0.1) for i, (r_, c_, k_) in enumerate(shapes)]
    groups = [0, 1, 0, 2]
    items = [device_item(c, g, ldw_pad=(64 if i == 2 else 0)) for i, (c, g) in enumerate(zip(cases, groups))]
    s = run_merge_quant(items, 4)                                 # group 3 has no member: scale 1
    check_merge_quant(cases, groups, items, s, 4)
    fq.qf_lora_adapter_grads_grouped(items)
    torch.cuda.synchronize()
    for i, (c, it) in enumerate(zip(cases, items)):
        check_grads(c, it["dA"].cpu().numpy(), it["dB"].cpu().numpy(), f"desc {i}")


@pytest.mark.parametrize("rank16", [False, True])
@pytest.mark.parametrize("with_M", [True, False])
def test_lora_sixteen_descriptors_runs_cross_matrices(rank16, with_M):
    """The most descriptors a launch takes, all small and ragged (1 to 130 rows, 32 to 640
    columns), in 6 tied groups in no order: a wave's run of tiles crosses several matrices,
    columns and groups, and a partial last 32-column group.  Odd and even ranks (the
    general path) or all rank 16."""
    rng = np.random.default_rng(123 + rank16 + 2 * with_M)
    shapes = [(int(rng.integers(1, 131)), 32 * int(rng.integers(1, 21)), 16 if rank16 else int(rng.integers(1, 17)))
              for _ in range(16)]
    groups = [int(g) for g in rng.integers(0, 6, 16)]
    cases = [make_case(r_, c_, k_, seed=500 + i, a_scale=0.1, b_scale=0.1) for i, (r_, c_, k_) in enumerate(shapes)]
    items = [device_item(c, g, ldw_pad=(32 if i % 3 == 0 else 0), with_M=with_M)
             for i, (c, g) in enumerate(zip(cases, groups))]
    s = run_merge_quant(items, 6)
    check_merge_quant(cases, groups, items, s, 6)


def test_lora_zero_adapter_is_identity():
    """B = 0 gives M = W bit for bit, so the result is the plain NVFP4 QDQ of W."""
    c = make_case(64, 512, 16, seed=5)
    c["B"] = np.zeros_like(c["B"])
    it = device_item(c, 0)
    s = run_merge_quant([it], 1)
    assert_same(host(it["M"]), c["W"], "M == W")
    y_plain = fq.qf_qdq_nvfp4(dev(c["W"]), torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    assert_same(host(it["y"]), host(y_plain), "y == plain NVFP4 QDQ")


def test_lora_accumulate_adds():
    c = make_case(80, 544, 16, seed=9)
    it = device_item(c, 0)
    fq.qf_lora_adapter_grads_grouped([it])
    dA1, dB1 = it["dA"].clone(), it["dB"].clone()
    fq.qf_lora_adapter_grads_grouped([it], accumulate=True)
    torch.cuda.synchronize()
    assert_same(f32bits(it["dA"].cpu().numpy()), f32bits((dA1 + dA1).cpu().numpy()), "dA accumulate")
    assert_same(f32bits(it["dB"].cpu().numpy()), f32bits((dB1 + dB1).cpu().numpy()), "dB accumulate")


def test_lora_full_size_expert():
    """One MoE expert at its real shape: both fused matrices in one launch, each its own group."""
    e = workloads.moe_expert(3)
    cases, items = [], []
    for g, name in enumerate(("gate_up", "down")):
        W, A, B, G = e[name]
        c = dict(W=W, A=A, B=B, G=G)
        cases.append(c)
        items.append(device_item(c, g))
    s = run_merge_quant(items, 2)
    Ms = [lora.merge(c["W"], c["A"], c["B"]) for c in cases]
    for i, (M, it) in enumerate(zip(Ms, items)):
        assert_same(host(it["M"]), M, f"M[{i}]")
    s_want = [nvfp4.tensor_scale([M]) for M in Ms]
    assert_same(f32bits(s), f32bits(s_want), "tensor scales")
    for i, (M, it) in enumerate(zip(Ms, items)):
        rows_ = sample_rows(M.shape[0], 48, seed=i)
        c, S = nvfp4.quantize(M[rows_], s_want[i])
        pc, ps = nvfp4.pack(c, S)
        assert_same(host(it["y"])[rows_], nvfp4.dequantize(c, S, s_want[i]), f"y[{i}] sampled rows")
        assert_same(u8(it["codes"])[rows_], pc, f"codes[{i}] sampled rows")
        assert_same(u8(it["scales"])[rows_], ps, f"block scales[{i}] sampled rows")
    fq.qf_lora_adapter_grads_grouped(items)
    torch.cuda.synchronize()
    for i, (c, it) in enumerate(zip(cases, items)):
        check_grads(c, it["dA"].cpu().numpy(), it["dB"].cpu().numpy(), f"expert 3 matrix {i}")


@pytest.mark.parametrize("rows,cols,r", [(100, 1056, 16), (37, 544, 7), (64, 32, 1), (33, 512, 16), (1, 96, 2)])
def test_lora_without_scratch(rows, cols, r):
    """M = None: pass 1 only takes the maximum, pass 2 merges again in registers and
    quantizes; the tensor scale, y, codes and block scales are the same bits."""
    c = make_case(rows, cols, r, seed=rows * 5 + r + 1, a_scale=0.1, b_scale=0.1)
    it = device_item(c, 0, with_M=False)
    s = run_merge_quant([it], 1)
    check_merge_quant([c], [0], [it], s, 1)


def test_lora_without_scratch_mixed_batch_and_partial_outputs():
    """One launch mixing descriptors with and without M, strided W, odd ranks, shared
    groups, and descriptors that write only y or only the packed arrays."""
    shapes = [(96, 1024, 16), (70, 608, 5), (129, 1056, 16), (16, 64, 3), (45, 576, 9)]
    cases = [make_case(r_, c_, k_, seed=31 + i, a_scale=0.1, b_scale=0.1) for i, (r_, c_, k_) in enumerate(shapes)]
    groups = [0, 1, 0, 2, 1]
    with_M = [False, True, False, False, True]
    items = [device_item(c, g, ldw_pad=(64 if i in (0, 2) else 0), with_M=m)
             for i, (c, g, m) in enumerate(zip(cases, groups, with_M))]
    items[2]["codes"] = items[2]["scales"] = None                 # y only
    items[3]["y"] = None                                           # packed only
    s = run_merge_quant(items, 3)
    check_merge_quant(cases, groups, items, s, 3)


def test_lora_without_scratch_full_size_expert():
    """One MoE expert at its real shape with no merge scratch: sampled rows bit-exact."""
    e = workloads.moe_expert(5)
    cases, items = [], []
    for g, name in enumerate(("gate_up", "down")):
        W, A, B, G = e[name]
        c = dict(W=W, A=A, B=B, G=G)
        cases.append(c)
        items.append(device_item(c, g, with_M=False))
    s = run_merge_quant(items, 2)
    Ms = [lora.merge(c["W"], c["A"], c["B"]) for c in cases]
    s_want = [nvfp4.tensor_scale([M]) for M in Ms]
    assert_same(f32bits(s), f32bits(s_want), "tensor scales")
    for i, (M, it) in enumerate(zip(Ms, items)):
        rows_ = sample_rows(M.shape[0], 48, seed=10 + i)
        c, S = nvfp4.quantize(M[rows_], s_want[i])
        pc, ps = nvfp4.pack(c, S)
        assert_same(host(it["y"])[rows_], nvfp4.dequantize(c, S, s_want[i]), f"y[{i}] sampled rows")
        assert_same(u8(it["codes"])[rows_], pc, f"codes[{i}] sampled rows")
        assert_same(u8(it["scales"])[rows_], ps, f"block scales[{i}] sampled rows")


def test_lora_grads_512_row_units():
    """16 descriptors of 600 x 4096 fill the chip with 512-row gradient units (ragged
    second unit of 88 rows): dA and dB of every descriptor within the bound, mixed ranks."""
    ranks = [16, 16, 7, 16, 1, 16, 16, 9, 16, 16, 16, 3, 16, 16, 16, 16]
    cases = [make_case(600, 4096, r, seed=200 + i) for i, r in enumerate(ranks)]
    items = [device_item(c, i) for i, c in enumerate(cases)]
    b = fq.LoraBatch(items)
    assert b.workspace_bytes == 4 * (16 * 2 * 16 * 4096 + 16 * 8 * 600 * 16)   # 2 dA blocks per matrix
    fq.qf_lora_adapter_grads_grouped(b)
    torch.cuda.synchronize()
    for i, (c, it) in enumerate(zip(cases, items)):
        check_grads(c, it["dA"].cpu().numpy(), it["dB"].cpu().numpy(), f"desc {i}")


# ------------------------------------------------ the MoE share's launch layouts ----
_EXPERT_CACHE = {}


def _expert_oracle(e):
    """Host bits of expert e (both matrices), its merged weights and their tensor scales."""
    if e not in _EXPERT_CACHE:
        ex = workloads.moe_expert(e)
        mats = []
        for name in ("gate_up", "down"):
            W, A, B, G = ex[name]
            M = lora.merge(W, A, B)
            mats.append(dict(W=W, A=A, B=B, G=G, M=M, s=nvfp4.tensor_scale([M])))
        _EXPERT_CACHE[e] = mats
    return _EXPERT_CACHE[e]


@pytest.mark.parametrize("experts,tiles_per_wave", [(8, 18), (2, 5)])
@pytest.mark.parametrize("with_M", [True, False])
def test_moe_launch_layout(experts, tiles_per_wave, with_M):
    """The layout the MoE step runs: `experts` full-size experts (gate/up 3072x3072 and
    down 3072x1536, rank 16) per launch, one tied group per matrix (2 x experts groups),
    with and without the merge scratch.  8 experts per launch is the benchmark's layout
    (768 pass-1 workgroups whose waves stream runs of up to 18 tiles across column and
    matrix boundaries, 512-row gradient blocks); 2 experts give runs of up to 5 tiles
    (one expert is test_lora_full_size_expert).
    Every tensor scale and every merged weight bit for bit; y, codes and block scales on
    sampled rows of every matrix; dA and dB of every matrix within Higham's bound."""
    ids = list(range(11, 11 + experts))
    mats = [m for e in ids for m in _expert_oracle(e)]
    items = []
    for k, m in enumerate(mats):
        c = dict(W=m["W"], A=m["A"], B=m["B"], G=m["G"])
        items.append(device_item(c, k, with_M=with_M))
    batch = fq.LoraBatch(items)
    layout = fq.qf_lora_layout(batch)
    assert layout[0] == tiles_per_wave, layout
    if experts == 8:
        assert layout[2] == 512, layout
    s = fq.qf_lora_merge_tensor_scale_nvfp4_grouped(batch, len(items))
    fq.qf_lora_merge_qdq_pack_nvfp4_grouped(batch, s)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    assert_same(f32bits(s), f32bits([m["s"] for m in mats]), "tensor scales of all groups")
    for k, (m, it) in enumerate(zip(mats, items)):
        if with_M:
            assert_same(host(it["M"]), m["M"], f"M[{k}]")
        rows_ = sample_rows(m["M"].shape[0], 24, seed=100 + k)
        c, S = nvfp4.quantize(m["M"][rows_], m["s"])
        pc, ps = nvfp4.pack(c, S)
        assert_same(host(it["y"])[rows_], nvfp4.dequantize(c, S, m["s"]), f"y[{k}] sampled rows")
        assert_same(u8(it["codes"])[rows_], pc, f"codes[{k}] sampled rows")
        assert_same(u8(it["scales"])[rows_], ps, f"block scales[{k}] sampled rows")
    if with_M:
        fq.qf_lora_adapter_grads_grouped(batch)
        torch.cuda.synchronize()
        for k, (m, it) in enumerate(zip(mats, items)):
            check_grads(m, it["dA"].cpu().numpy(), it["dB"].cpu().numpy(), f"matrix {k}")


def test_single_matrix_calls_equal_the_grouped_form():
    """The single-matrix calls (merge in registers, no scratch) give the bits of a grouped
    launch of one descriptor, for a full-size gate/up matrix and a ragged one."""
    e = _expert_oracle(11)[0]
    for c in (dict(W=e["W"], A=e["A"], B=e["B"], G=e["G"]), make_case(37, 544, 7, seed=3)):
        Wd, Ad, Bd, Gd = dev(c["W"]), dev(c["A"]), dev(c["B"]), dev(c["G"])
        s = fq.qf_lora_merge_tensor_scale_nvfp4(Wd, Ad, Bd)
        y, codes, scales = fq.qf_lora_merge_qdq_pack_nvfp4(Wd, Ad, Bd, s)
        dA, dB = fq.qf_lora_adapter_grads(Gd, Ad, Bd)
        it = device_item(c, 0, with_M=False)
        s2 = fq.qf_lora_merge_tensor_scale_nvfp4_grouped([it], 1)
        fq.qf_lora_merge_qdq_pack_nvfp4_grouped([it], s2)
        fq.qf_lora_adapter_grads_grouped([it])
        torch.cuda.synchronize()
        M = lora.merge(c["W"], c["A"], c["B"])
        assert_same(f32bits(s.cpu().numpy()), f32bits([nvfp4.tensor_scale([M])]), "single tensor scale")
        assert_same(f32bits(s.cpu().numpy()), f32bits(s2.cpu().numpy()), "single vs grouped scale")
        assert torch.equal(y.view(torch.int16), it["y"].view(torch.int16))
        assert torch.equal(codes, it["codes"]) and torch.equal(scales, it["scales"])
        assert_same(f32bits(dA.cpu().numpy()), f32bits(it["dA"].cpu().numpy()), "dA")
        assert_same(f32bits(dB.cpu().numpy()), f32bits(it["dB"].cpu().numpy()), "dB")
        check_grads(c, dA.cpu().numpy(), dB.cpu().numpy(), "single-matrix grads")
