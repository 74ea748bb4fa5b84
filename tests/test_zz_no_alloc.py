"""The no-allocation tensor-scale entry point (qf_nvfp4_tensor_scale_grouped_noalloc)
against the workspace form (qf_nvfp4_tensor_scale_grouped), through the C ABI.

Two calls in a row, the second with a smaller input (fewer partials, so stale partials of
the first call sit beyond what the second reads), each bit for bit equal to the workspace
form and to the oracle; and a call whose partials would not fit the fixed array is refused
with QF_ERR_WORKSPACE before anything runs.
"""

import ctypes

import numpy as np
import pytest
import torch

import fp4_fake_quant_amd as fq
from fp4_fake_quant_amd import _lib
from oracle import nvfp4
from oracle import primitives as P
from tests.gpu_util import dev

RNG = np.random.default_rng(4321)


def _descs(tensors, groups):
    arr = (_lib.TensorDesc * len(tensors))()
    for i, (t, g) in enumerate(zip(tensors, groups)):
        arr[i].x, arr[i].rows, arr[i].cols, arr[i].ldx = t.data_ptr(), t.shape[0], t.shape[1], t.stride(0)
        arr[i].group = g
    return arr


def _noalloc(tensors, groups, n_groups):
    L = _lib.lib()
    arr = _descs(tensors, groups)
    out = torch.full((n_groups,), -1.0, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = L.qf_nvfp4_tensor_scale_grouped_noalloc(ctypes.byref(arr), len(tensors), n_groups, out.data_ptr(),
                                                 flag.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, L.qf_status_str(st)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(flag.item())


@pytest.mark.gpu
def test_noalloc_matches_workspace_form_twice():
    L = _lib.lib()
    assert L.qf_noalloc_scratch_bytes() == 4 * 2048 * 16
    big = [P.f32_to_bf16((RNG.standard_normal((rows, 4096)) * s).astype(np.float32))
           for rows, s in ((6144, 0.02), (2048, 0.05), (4096, 0.3))]
    small = [P.f32_to_bf16((RNG.standard_normal((40, 512)) * s).astype(np.float32)) for s in (0.7, 0.01)]
    for tensors, groups, n_groups in ((big, [0, 2, 1], 3), (small, [1, 1], 2)):
        td = [dev(t) for t in tensors]
        got, flag = _noalloc(td, groups, n_groups)
        ref = fq.qf_nvfp4_tensor_scale_grouped([dict(x=t, group=g) for t, g in zip(td, groups)], n_groups)
        assert np.array_equal(got.view(np.uint32), ref.cpu().numpy().view(np.uint32))
        want = [nvfp4.tensor_scale([t for t, g in zip(tensors, groups) if g == k]) if k in groups else np.float32(1)
                for k in range(n_groups)]
        assert np.array_equal(got.view(np.uint32), np.array(want, np.float32).view(np.uint32))
        assert flag == 0


@pytest.mark.gpu
def test_noalloc_refuses_what_does_not_fit():
    """64 groups of a launch that fills the persistent grid need 512 KiB of partials."""
    L = _lib.lib()
    x = torch.zeros((4096, 4096), dtype=torch.bfloat16, device="cuda")
    arr = _descs([x], [63])
    out = torch.empty(64, dtype=torch.float32, device="cuda")
    st = L.qf_nvfp4_tensor_scale_grouped_noalloc(ctypes.byref(arr), 1, 64, out.data_ptr(), None,
                                                 torch.cuda.current_stream().cuda_stream)
    assert st == 4
