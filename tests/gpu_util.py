"""Host <-> device helpers for the GPU parity tests (bf16 bit patterns as uint16)."""

import numpy as np
import torch


def dev(bits, device="cuda"):
    """numpy uint16 bf16 bits -> torch.bfloat16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def host(t):
    """torch.bfloat16 tensor -> numpy uint16 bf16 bits."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u8(t):
    return t.detach().contiguous().cpu().numpy()


def f32bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def first_mismatch(a, b):
    """Index and values of the first differing element (for assertion messages)."""
    a, b = np.asarray(a), np.asarray(b)
    if a.shape != b.shape:
        return f"shape {a.shape} != {b.shape}"
    idx = np.argwhere(a != b)
    if idx.size == 0:
        return "equal"
    i = tuple(idx[0])
    return f"{idx.shape[0]} mismatches; first at {i}: got {a[i]!r} want {b[i]!r}"


def sample_rows(rows, k, seed=0):
    """k distinct rows including the first and the last."""
    rng = np.random.default_rng(seed)
    pick = set([0, rows - 1])
    pick.update(rng.choice(rows, size=min(k, rows), replace=False).tolist())
    return np.array(sorted(pick))
