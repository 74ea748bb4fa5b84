"""GPU-packed checkpoints written to their containers and read back (the path the Method
section's export takes: train, pack in the engine layout, save).

NVFP4: the dense layer's tied Q/K/V (as three tensors sharing one tensor scale) and O,
packed on the GPU, written with the tracked activation scale of a few activation batches;
MXFP4: the same matrices; both read back with the safetensors library and compared with
the oracle's packed bytes and scales bit for bit.  Q4_K: GPU-packed blocks written to the
GGUF-style file and compared with the oracle's blocks (the container's engine
compatibility is unpinned).
"""

import numpy as np
import pytest
import torch
from safetensors import safe_open

import fp4_fake_quant_amd as fq
from oracle import mxfp4, nvfp4, q4k
from oracle import primitives as P
from tests.gpu_util import dev
from tests.test_export import _read_gguf

pytestmark = pytest.mark.gpu
RNG = np.random.default_rng(606)


def _bits(a):
    return P.f32_to_bf16(np.asarray(a, np.float32))


def test_fp4_checkpoint_round_trip(tmp_path):
    q, k, v = (_bits(RNG.standard_normal((r, 512)) * s) for r, s in ((256, 0.02), (64, 0.05), (64, 0.01)))
    o = _bits(RNG.standard_normal((512, 256)) * 0.03)
    qd, kd, vd, od = (dev(t) for t in (q, k, v, o))
    s_qkv = fq.qf_nvfp4_tensor_scale([qd, kd, vd])
    s_o = fq.qf_nvfp4_tensor_scale(od)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    amax_ref = np.float32(0.0)
    for i in range(3):
        x = _bits(RNG.standard_t(3, size=(128, 512)) * 0.5)
        s_in = fq.qf_nvfp4_tensor_scale_tracked([dict(x=dev(x), group=0)], 1, amax)
        amax_ref, s_in_ref = nvfp4.tracked_scale(amax_ref, [x])
    tensors, meta = [], {"quantization": "nvfp4 (qkv tied) + mxfp4"}
    qkv = torch.cat([qd, kd, vd])
    c, s = fq.qf_pack_nvfp4(qkv, s_qkv)
    tensors += fq.export_fp4_tensors("layers.0.self_attn.qkv_proj", fq.QF_FMT_NVFP4, c, s, s_qkv, s_in)
    c, s = fq.qf_pack_nvfp4(od, s_o)
    tensors += fq.export_fp4_tensors("layers.0.self_attn.o_proj", fq.QF_FMT_NVFP4, c, s, s_o)
    c, s = fq.qf_pack_mxfp4(od)
    tensors += fq.export_fp4_tensors("mx.o_proj", fq.QF_FMT_MXFP4, c, s)
    path = tmp_path / "ckpt.safetensors"
    fq.qf_write_safetensors(path, tensors, meta)
    with safe_open(str(path), framework="pt") as f:
        got = {kk: f.get_tensor(kk) for kk in f.keys()}
        assert f.metadata() == meta
    fused = np.concatenate([q, k, v])
    st_ref = nvfp4.tensor_scale([fused])
    pc, ps = nvfp4.pack(*nvfp4.quantize(fused, st_ref))
    pre = "layers.0.self_attn.qkv_proj"
    assert np.array_equal(got[pre + ".weight_packed"].numpy(), pc)
    assert np.array_equal(got[pre + ".weight_scale"].view(torch.uint8).numpy(), ps)
    assert got[pre + ".weight_global_scale"].numpy().view(np.uint32)[0] == np.float32(st_ref).view(np.uint32)
    assert got[pre + ".input_global_scale"].numpy().view(np.uint32)[0] == np.float32(s_in_ref).view(np.uint32)
    so_ref = nvfp4.tensor_scale([o])
    pc, ps = nvfp4.pack(*nvfp4.quantize(o, so_ref))
    assert np.array_equal(got["layers.0.self_attn.o_proj.weight_packed"].numpy(), pc)
    assert np.array_equal(got["layers.0.self_attn.o_proj.weight_scale"].view(torch.uint8).numpy(), ps)
    assert "layers.0.self_attn.o_proj.input_global_scale" not in got
    mc, ms = mxfp4.pack(*mxfp4.quantize(o))
    assert np.array_equal(got["mx.o_proj.weight_packed"].numpy(), mc)
    assert np.array_equal(got["mx.o_proj.weight_scale"].view(torch.uint8).numpy(), ms)
    # the file's bytes dequantize on the GPU to the oracle's QDQ of the weights
    y = fq.qf_dequant_nvfp4(got[pre + ".weight_packed"].cuda(), got[pre + ".weight_scale"].view(torch.uint8).cuda(),
                            got[pre + ".weight_global_scale"].cuda())
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), nvfp4.qdq(fused, st_ref))


def test_q4k_checkpoint_round_trip(tmp_path):
    W = _bits(RNG.standard_normal((96, 1024)) * 0.02 + 0.001)
    _, blocks = fq.qf_qdq_pack_q4k(dev(W))
    path = tmp_path / "ckpt.gguf"
    fq.qf_write_gguf(path, [fq.export_q4k_tensor("blk.0.attn_v.weight", blocks, 96, 1024)],
                     {"qf.q4k.block_layout": fq.Q4K_BLOCK_LAYOUT})
    _, kv, infos, b, start = _read_gguf(path)
    ref = q4k.pack(q4k.quantize(W))
    assert infos == [("blk.0.attn_v.weight", [1024, 96], 12, 0)]
    assert np.array_equal(np.frombuffer(b, np.uint8, ref.nbytes, start), ref.reshape(-1))
