"""Checkpoint containers (host code, no GPU): qf_write_safetensors and qf_write_gguf.

The safetensors file is read back with the safetensors library (an independent reader):
names, dtypes, shapes, the bytes of the oracle's packed NVFP4 / MXFP4 arrays and the
metadata must come back exactly.  The GGUF-style file is parsed here from the layout the
header states (magic, version, counts, string key-values, tensor infos, 32-byte aligned
data); no GGUF reader is installed, and whether an engine reads this library's Q4_K block
bytes the same way is parity unpinned.
"""

import struct

import numpy as np
import pytest
import torch
from safetensors import safe_open

import fp4_fake_quant_amd as fq
import workloads
from fp4_fake_quant_amd import _lib
from oracle import mxfp4, nvfp4, q4k


def _w():
    return workloads.single_256x512()["W"]


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a))


def test_safetensors_round_trip_of_packed_layers(tmp_path):
    W = _w()
    s_t = nvfp4.tensor_scale([W])
    pc, ps = nvfp4.pack(*nvfp4.quantize(W, s_t))
    mc, ms = mxfp4.pack(*mxfp4.quantize(W))
    s_in = np.float32(0.0123)
    tensors = (fq.export_fp4_tensors("layers.0.qkv", fq.QF_FMT_NVFP4, _t(pc), _t(ps),
                                     _t(np.array([s_t], np.float32)), _t(np.array([s_in], np.float32))) +
               fq.export_fp4_tensors("layers.0.o", fq.QF_FMT_MXFP4, _t(mc), _t(ms)) +
               [("bias \"quoted\"\\n", _t(np.arange(6, dtype=np.float32).reshape(2, 3)), None),
                ("empty", _t(np.zeros((0, 4), np.uint8)), None)])
    path = tmp_path / "model.safetensors"
    fq.qf_write_safetensors(path, tensors, {"format": "nvfp4+mxfp4", "tensor_scale": "dequant multiplier"})
    with safe_open(str(path), framework="pt") as f:
        assert sorted(f.keys()) == sorted(n for n, _, _ in tensors)
        assert f.metadata() == {"format": "nvfp4+mxfp4", "tensor_scale": "dequant multiplier"}
        got = {k: f.get_tensor(k) for k in f.keys()}
    assert got["layers.0.qkv.weight_packed"].dtype == torch.uint8
    assert np.array_equal(got["layers.0.qkv.weight_packed"].numpy(), pc)
    assert got["layers.0.qkv.weight_scale"].dtype == torch.float8_e4m3fn
    assert np.array_equal(got["layers.0.qkv.weight_scale"].view(torch.uint8).numpy(), ps)
    assert got["layers.0.qkv.weight_global_scale"].numpy().view(np.uint32)[0] == np.float32(s_t).view(np.uint32)
    assert got["layers.0.qkv.input_global_scale"].numpy()[0] == s_in
    assert got["layers.0.o.weight_scale"].dtype == torch.float8_e8m0fnu
    assert np.array_equal(got["layers.0.o.weight_scale"].view(torch.uint8).numpy(), ms)
    assert np.array_equal(got["layers.0.o.weight_packed"].numpy(), mc)
    assert np.array_equal(got["bias \"quoted\"\\n"].numpy(), np.arange(6, dtype=np.float32).reshape(2, 3))
    assert tuple(got["empty"].shape) == (0, 4)
    # the scale bytes decode to the oracle's scales through torch's own fp8 casts
    assert np.array_equal(got["layers.0.qkv.weight_scale"].float().numpy(), nvfp4.e4m3_value(ps))
    hdr_len = struct.unpack("<Q", path.read_bytes()[:8])[0]
    assert hdr_len % 8 == 0
    # bits per weight of the NVFP4 payload: codes + block scales + one fp32 per tied group
    nbytes = pc.nbytes + ps.nbytes + 4
    assert nbytes * 8 / W.size == pytest.approx(4.5, abs=4 * 8 / W.size)


def test_safetensors_errors(tmp_path):
    L = _lib.lib()
    a = _t(np.zeros(4, np.uint8))
    with pytest.raises(RuntimeError):
        fq.qf_write_safetensors(tmp_path / "x.st", [("a", a, None), ("a", a, None)])     # repeated name
    with pytest.raises(RuntimeError):
        fq.qf_write_safetensors(tmp_path / "no_such_dir" / "x.st", [("a", a, None)])    # cannot write
    arr = (_lib.StTensor * 1)()
    arr[0].name, arr[0].dtype, arr[0].ndim = b"a", b"F4", 0                           # unknown dtype
    assert L.qf_write_safetensors(str(tmp_path / "y.st").encode(), arr, 1, None, None, 0) == 7
    arr[0].dtype, arr[0].ndim = b"U8", 9                                                # too many dims
    assert L.qf_write_safetensors(str(tmp_path / "y.st").encode(), arr, 1, None, None, 0) == 2
    arr[0].ndim = 0                                                                     # a scalar with no data
    assert L.qf_write_safetensors(str(tmp_path / "y.st").encode(), arr, 1, None, None, 0) == 1
    assert not (tmp_path / "y.st").exists()
    assert L.qf_write_safetensors(None, arr, 1, None, None, 0) == 1


def _read_gguf(path):
    b = path.read_bytes()
    pos = 0

    def u32():
        nonlocal pos
        v = struct.unpack_from("<I", b, pos)[0]
        pos += 4
        return v

    def u64():
        nonlocal pos
        v = struct.unpack_from("<Q", b, pos)[0]
        pos += 8
        return v

    def string():
        nonlocal pos
        n = u64()
        s = b[pos:pos + n].decode()
        pos += n
        return s

    assert b[:4] == b"GGUF"
    pos = 4
    version, nt, nkv = u32(), u64(), u64()
    kv = {}
    for _ in range(nkv):
        k = string()
        assert u32() == 8
        kv[k] = string()
    infos = []
    for _ in range(nt):
        name = string()
        nd = u32()
        dims = [u64() for _ in range(nd)]
        infos.append((name, dims, u32(), u64()))
    start = (pos + 31) // 32 * 32
    assert all(c == 0 for c in b[pos:start])
    return version, kv, infos, b, start


def test_gguf_style_file_of_q4k_blocks(tmp_path):
    W = _w()
    blocks = q4k.pack(q4k.quantize(W))
    W2 = W[:64, :256].copy()
    blocks2 = q4k.pack(q4k.quantize(W2))
    path = tmp_path / "model.gguf"
    fq.qf_write_gguf(path, [fq.export_q4k_tensor("blk.0.ffn_down.weight", _t(blocks), *W.shape),
                            fq.export_q4k_tensor("blk.0.attn_q.weight", _t(blocks2), *W2.shape)],
                     {"general.name": "qf test", "qf.q4k.block_layout": fq.Q4K_BLOCK_LAYOUT})
    version, kv, infos, b, start = _read_gguf(path)
    assert version == 3
    assert kv == {"general.name": "qf test", "qf.q4k.block_layout": fq.Q4K_BLOCK_LAYOUT}
    assert [i[0] for i in infos] == ["blk.0.ffn_down.weight", "blk.0.attn_q.weight"]
    assert infos[0][1] == [512, 256] and infos[0][2] == 12 and infos[0][3] == 0
    assert infos[1][1] == [256, 64] and infos[1][3] == (blocks.nbytes + 31) // 32 * 32
    # 144 bytes per 256 weights: 4.50 bits per weight ("Supported formats" table)
    assert blocks.nbytes * 8 / W.size == 4.5
    got0 = np.frombuffer(b, np.uint8, blocks.nbytes, start + infos[0][3])
    got1 = np.frombuffer(b, np.uint8, blocks2.nbytes, start + infos[1][3])
    assert np.array_equal(got0, blocks.reshape(-1)) and np.array_equal(got1, blocks2.reshape(-1))
    assert len(b) == start + infos[1][3] + (blocks2.nbytes + 31) // 32 * 32


def test_gguf_errors(tmp_path):
    L = _lib.lib()
    arr = (_lib.GgufTensor * 1)()
    arr[0].name, arr[0].ndim = b"t", 0
    assert L.qf_write_gguf(str(tmp_path / "z.gguf").encode(), arr, 1, None, None, 0) == 2     # ndim 0
    assert not (tmp_path / "z.gguf").exists()
    with pytest.raises(RuntimeError):
        fq.qf_write_gguf(tmp_path / "z.gguf", [("a", _t(np.zeros(4, np.uint8)), (4,), 0)] * 2)   # repeated name
