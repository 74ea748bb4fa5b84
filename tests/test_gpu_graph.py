"""The hot path captured once in a HIP graph and replayed (GPU).

Every library call only enqueues kernels on the caller's stream (no memset, copy, allocation
or synchronization), so a caller can capture a whole step: here the NVFP4 tensor scale, the
NVFP4 and MXFP4 QDQ+pack and the STE, captured with torch.cuda.CUDAGraph on its capture
stream.  Between replays the inputs are rewritten by eager copies and the device is
synchronized; every replay's outputs must equal, bit for bit, both an eager run of the same
calls on the same inputs and the oracle.  300 rows: not a multiple of any kernel's rows per
workgroup.
"""

import numpy as np
import pytest
import torch

import fp4_fake_quant_amd as fq
from oracle import mxfp4, nvfp4, ste
from oracle import primitives as P
from tests.gpu_util import dev, first_mismatch, host, u8

pytestmark = pytest.mark.gpu
ROWS, COLS = 300, 512
NAMES = ("s_t", "nvfp4 y", "nvfp4 codes", "nvfp4 scales", "mxfp4 y", "mxfp4 codes", "mxfp4 scales", "g_latent")


def _inputs(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((ROWS, COLS)) * 0.02).astype(np.float32)
    x[rng.integers(0, ROWS, 40), rng.integers(0, COLS, 40)] *= 25.0               # outliers
    g = rng.standard_normal((ROWS, COLS)).astype(np.float32)
    return P.f32_to_bf16(x), P.f32_to_bf16(g)


class Step:
    def __init__(self):
        def u8buf(c):
            return torch.empty((ROWS, c), dtype=torch.uint8, device="cuda")
        self.x = torch.empty((ROWS, COLS), dtype=torch.bfloat16, device="cuda")
        self.g = torch.empty_like(self.x)
        need = fq.qf_nvfp4_tensor_scale_workspace([dict(x=self.x, group=0)])
        self.ws = torch.empty(max(need, 4), dtype=torch.uint8, device="cuda")
        self.sc = torch.empty(1, dtype=torch.float32, device="cuda")
        self.y, self.c, self.s = torch.empty_like(self.x), u8buf(COLS // 2), u8buf(COLS // 16)
        self.ym, self.cm, self.sm = torch.empty_like(self.x), u8buf(COLS // 2), u8buf(COLS // 32)
        self.gl = torch.empty((ROWS, COLS), dtype=torch.float32, device="cuda")

    def run(self):
        fq.qf_nvfp4_tensor_scale(self.x, self.sc, None, self.ws)
        fq.qf_qdq_pack_nvfp4(self.x, self.sc, self.y, self.c, self.s)
        fq.qf_qdq_pack_mxfp4(self.x, self.ym, self.cm, self.sm)
        fq.qf_ste_backward(self.g, self.gl)

    def outputs(self):
        return [self.sc.cpu().numpy().view(np.uint32).copy(), host(self.y), u8(self.c), u8(self.s),
                host(self.ym), u8(self.cm), u8(self.sm), self.gl.cpu().numpy().view(np.uint32).copy()]


def _oracle(x, g):
    s_t = nvfp4.tensor_scale([x])
    codes, S = nvfp4.quantize(x, s_t)
    pc, ps = nvfp4.pack(codes, S)
    mcodes, E = mxfp4.quantize(x)
    mc, ms = mxfp4.pack(mcodes, E)
    return [np.float32(s_t).reshape(1).view(np.uint32), nvfp4.dequantize(codes, S, s_t), pc, ps,
            mxfp4.dequantize(mcodes, E), mc, ms, np.asarray(ste.ste_backward(g), np.float32).view(np.uint32)]


def _same(got, want, what):
    for name, a, b in zip(NAMES, got, want):
        a, b = np.asarray(a), np.asarray(b).reshape(np.asarray(a).shape)
        assert np.array_equal(a, b), f"{what}, {name}: {first_mismatch(a, b)}"


def test_graph_replays_match_eager_and_oracle():
    st = Step()
    x0, g0 = _inputs(0)
    st.x.copy_(dev(x0))
    st.g.copy_(dev(g0))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run()                                                 # first calls outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.run()
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        x, g = _inputs(seed)
        st.x.copy_(dev(x))                                       # eager work between replays
        st.g.copy_(dev(g))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = st.outputs()
        _same(got, _oracle(x, g), f"replay {seed} against the oracle")
        for t in (st.sc, st.y, st.c, st.s, st.ym, st.cm, st.sm, st.gl):
            t.zero_()                                            # the eager run must write everything again
        st.run()
        torch.cuda.synchronize()
        _same(got, st.outputs(), f"replay {seed} against the eager calls")
