"""Seeded synthetic inputs for the five workloads (shared by tests and bench).

This module only draws random numbers and rounds them to BF16 storage; it
holds none of the quantization arithmetic, and neither the oracle nor the HIP
path is imported here.  Every tensor is returned as a numpy uint16 array of
BF16 bit patterns, row-major [out, in] (weights) or [tokens, hidden]
(activations).

Recipe (all draws float32/float64 from numpy's PCG64, then BF16 RNE through
torch's float32 -> bfloat16 cast):

* Streams: ``SeedSequence(seed).spawn(n)`` with one child per tensor, in the
  order listed for each workload (seed 0 unless stated).
* single_256x512: W ~ N(0, 0.02^2) with round(0.1% of 131072) = 131 distinct
  positions (``rng.choice`` without replacement) replaced by N(0, 0.5^2); upstream
  gradient G ~ N(0, 1).
* dense_layer_8b: hidden 4096, 32 query + 8 KV heads of dim 128, MLP 14336.
  Fused QKV 6144x4096, fused gate/up 28672x4096, down 4096x14336, O 4096x4096.
  Row r of each matrix is N(0, 0.02^2) * exp(0.3 z_r), z_r ~ N(0, 1) (LogNormal
  row jitter).  G ~ N(0, 1) per matrix.
* w4a4_gemm: X 32768x4096 = 0.5 * Student-t(nu = 3) with 8 distinct columns
  scaled by 20; W 14336x4096 ~ N(0, 0.02^2).
* q4k_set: shapes of single_256x512 plus the four dense_layer_8b matrices plus a
  151936x4096 vocabulary projection; entries 0.001 + 0.02 z + o_r with a per-row
  offset o_r ~ U(-0.01, 0.01).
* moe_lora: 128 experts; per expert gate/up 3072x3072 and down 3072x1536 base
  weights ~ N(0, 0.02^2), LoRA rank 16 with A ~ N(0, 0.01^2) [16, in] and
  B ~ N(0, 0.001^2) [out, 16], upstream gradient G ~ N(0, 1) of the weight's
  shape.  Each expert has its own child stream (``spawn(128)``), split again per
  tensor, so any single expert can be drawn on its own.

The ``*_device`` variants draw the same distributions on the GPU with torch's
seeded Philox generator (different values, same recipe) for the throughput
runs whose inputs are too large to draw quickly on the host.
"""

import numpy as np
import torch

DENSE_8B_SHAPES = {
    "qkv": (6144, 4096),
    "gate_up": (28672, 4096),
    "down": (4096, 14336),
    "o": (4096, 4096),
}
SINGLE_SHAPE = (256, 512)
GEMM_SHAPE = dict(M=32768, N=14336, K=4096)
VOCAB_SHAPE = (151936, 4096)
MOE = dict(experts=128, hidden=3072, inter=1536, rank=16)


def to_bf16_bits(a):
    """float32/float64 numpy array -> uint16 BF16 bit patterns (RNE, via torch)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rngs(seed, n):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def single_256x512(seed=0):
    rw, ro_pos, ro_val, rg = _rngs(seed, 4)
    rows, cols = SINGLE_SHAPE
    w = rw.standard_normal((rows, cols), dtype=np.float32) * np.float32(0.02)
    n_out = int(round(0.001 * rows * cols))
    pos = ro_pos.choice(rows * cols, size=n_out, replace=False)
    w.reshape(-1)[pos] = ro_val.standard_normal(n_out, dtype=np.float32) * np.float32(0.5)
    g = rg.standard_normal((rows, cols), dtype=np.float32)
    return dict(W=to_bf16_bits(w), G=to_bf16_bits(g), outlier_pos=np.sort(pos))


def _jittered(rng, rows, cols):
    w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(0.02)
    w *= np.exp(np.float32(0.3) * rng.standard_normal((rows, 1), dtype=np.float32))
    return w


def dense_layer_8b(seed=0, names=None, with_grad=True):
    """dict name -> (W bits, G bits or None) for the four matrices of the 8B layer."""
    names = list(DENSE_8B_SHAPES) if names is None else names
    rngs = _rngs(seed, 2 * len(DENSE_8B_SHAPES))
    out = {}
    for i, name in enumerate(DENSE_8B_SHAPES):
        if name not in names:
            continue
        rows, cols = DENSE_8B_SHAPES[name]
        w = to_bf16_bits(_jittered(rngs[2 * i], rows, cols))
        g = to_bf16_bits(rngs[2 * i + 1].standard_normal((rows, cols), dtype=np.float32)) if with_grad else None
        out[name] = (w, g)
    return out


def w4a4_gemm(seed=0, M=None, N=None, K=None):
    M = GEMM_SHAPE["M"] if M is None else M
    N = GEMM_SHAPE["N"] if N is None else N
    K = GEMM_SHAPE["K"] if K is None else K
    rx, rc, rw = _rngs(seed, 3)
    x = (rx.standard_t(3, size=(M, K)) * 0.5).astype(np.float32)
    cols = rc.choice(K, size=min(8, K), replace=False)
    x[:, cols] *= np.float32(20.0)
    w = rw.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return dict(X=to_bf16_bits(x), W=to_bf16_bits(w), outlier_cols=np.sort(cols))


def q4k_shapes():
    return [("single", SINGLE_SHAPE)] + list(DENSE_8B_SHAPES.items()) + [("vocab", VOCAB_SHAPE)]


def q4k_set(seed=0, names=None):
    """dict name -> W bits for the Q4_K union (optionally only some names)."""
    shapes = q4k_shapes()
    rngs = _rngs(seed, 2 * len(shapes))
    out = {}
    for i, (name, (rows, cols)) in enumerate(shapes):
        if names is not None and name not in names:
            continue
        z = rngs[2 * i].standard_normal((rows, cols), dtype=np.float32)
        off = rngs[2 * i + 1].uniform(-0.01, 0.01, size=(rows, 1)).astype(np.float32)
        out[name] = to_bf16_bits(np.float32(0.001) + np.float32(0.02) * z + off)
    return out


def moe_expert(e, seed=0, rank=None):
    """Expert e of the MoE share: dict with 'gate_up' and 'down', each (W, A, B, G) bits."""
    rank = MOE["rank"] if rank is None else rank
    H, I = MOE["hidden"], MOE["inter"]
    child = np.random.SeedSequence(seed).spawn(MOE["experts"])[e]
    rngs = [np.random.Generator(np.random.PCG64(s)) for s in child.spawn(8)]
    out = {}
    for j, (name, (rows, cols)) in enumerate([("gate_up", (2 * I, H)), ("down", (H, I))]):
        r = rngs[4 * j: 4 * j + 4]
        W = r[0].standard_normal((rows, cols), dtype=np.float32) * np.float32(0.02)
        A = r[1].standard_normal((rank, cols), dtype=np.float32) * np.float32(0.01)
        B = r[2].standard_normal((rows, rank), dtype=np.float32) * np.float32(0.001)
        G = r[3].standard_normal((rows, cols), dtype=np.float32)
        out[name] = tuple(to_bf16_bits(t) for t in (W, A, B, G))
    return out


# ------------------------------------------------------- device variants ---
def _dev_gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _bf16(t):
    return t.to(torch.bfloat16)


def q4k_set_device(seed=0, device="cuda"):
    """Same recipe as q4k_set, drawn on the device; dict name -> bf16 tensor."""
    g = _dev_gen(seed, device)
    out = {}
    for name, (rows, cols) in q4k_shapes():
        z = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
        off = torch.rand((rows, 1), generator=g, device=device, dtype=torch.float32) * 0.02 - 0.01
        out[name] = _bf16(0.001 + 0.02 * z + off)
        del z
    return out


def moe_experts_device(seed=0, device="cuda", experts=None, rank=None):
    """All experts, same recipe as moe_expert, drawn on the device.

    Returns dict name -> dict(W, A, B, G) of stacked bf16 tensors [experts, ...].
    """
    experts = MOE["experts"] if experts is None else experts
    rank = MOE["rank"] if rank is None else rank
    H, I = MOE["hidden"], MOE["inter"]
    g = _dev_gen(seed, device)
    out = {}
    for name, (rows, cols) in [("gate_up", (2 * I, H)), ("down", (H, I))]:
        kw = dict(generator=g, device=device, dtype=torch.float32)
        out[name] = dict(
            W=_bf16(torch.randn((experts, rows, cols), **kw) * 0.02),
            A=_bf16(torch.randn((experts, rank, cols), **kw) * 0.01),
            B=_bf16(torch.randn((experts, rows, rank), **kw) * 0.001),
            G=_bf16(torch.randn((experts, rows, cols), **kw)),
        )
    return out


def w4a4_gemm_device(seed=0, device="cuda", M=None, N=None, K=None):
    """Same recipe as w4a4_gemm drawn on the device (t(3) = z / sqrt(chi2_3 / 3))."""
    M = GEMM_SHAPE["M"] if M is None else M
    N = GEMM_SHAPE["N"] if N is None else N
    K = GEMM_SHAPE["K"] if K is None else K
    g = _dev_gen(seed, device)
    kw = dict(generator=g, device=device, dtype=torch.float32)
    z = torch.randn((M, K), **kw)
    chi2 = torch.zeros((M, K), device=device, dtype=torch.float32)
    for _ in range(3):
        chi2 += torch.randn((M, K), **kw) ** 2
    x = 0.5 * z / torch.sqrt(chi2 / 3.0)
    del z, chi2
    cols = torch.randperm(K, generator=g, device=device)[:8]
    x[:, cols] *= 20.0
    w = torch.randn((N, K), **kw) * 0.02
    return dict(X=_bf16(x), W=_bf16(w))


def dense_layer_8b_device(seed=0, device="cuda"):
    g = _dev_gen(seed, device)
    kw = dict(generator=g, device=device, dtype=torch.float32)
    out = {}
    for name, (rows, cols) in DENSE_8B_SHAPES.items():
        w = torch.randn((rows, cols), **kw) * 0.02 * torch.exp(0.3 * torch.randn((rows, 1), **kw))
        out[name] = (_bf16(w), _bf16(torch.randn((rows, cols), **kw)))
    return out
