"""Writes q4k_mse_near_ties.json: Q4_K sub-blocks (32 bf16 inputs each) on which the
"mse" sub-block scale rule's choice depends on the float32 summation order of the
candidates' squared errors.

The rule (a search of our own; the QATFactory project page names an MSE-optimal
quantizer only as the llama.cpp PTQ baseline and gives no rule) scores each of the 8
candidate scales by a float32 sum in a stated order: each quarter of 8 elements in index
order, then (quarter 0 + quarter 1) + (quarter 2 + quarter 3).  Where two candidates'
exact scores lie within float32 rounding of each other, another order (plain index
order over all 32) can pick a different candidate.  These sub-blocks are such near ties;
the pin in tests/test_oracle_q4k_mse.py checks that the oracle decides them the stated
way.  Only inputs are stored: no expected value.

The search is its own float32 code (numpy), independent of oracle/: 31 elements are
drawn N(0.001, 0.02^2) and rounded to bf16, then the 32nd element runs over every bf16
value strictly between the others' minimum and maximum (so the extremes stay), and the
two summation orders are compared.  Such flips are rare: the search takes about ten
minutes on one core.  Run: python tests/golden/q4k_mse_near_ties.py
"""

import json
import os

import numpy as np
import torch

F = np.float32
HERE = os.path.dirname(os.path.abspath(__file__))


def bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def widen(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def scores(x):
    """x: float32 [n, 32].  Candidate scores [n, 8] in the stated order and in plain index order."""
    mn = np.minimum(x.min(-1), F(0))
    mx = x.max(-1)
    base = ((mx - mn).astype(F) / F(15)).astype(F)
    t = (x - mn[:, None]).astype(F)
    tree, seq = [], []
    for k in range(8):
        s = (base * F(1 - k / 16)).astype(F)
        r = (F(1) / s).astype(F)
        q = np.clip(np.rint((t * r[:, None]).astype(F)), 0, 15).astype(F)
        e = (((q * s[:, None]).astype(F) + mn[:, None]).astype(F) - x).astype(F)
        sq = (e * e).astype(F)
        part = []
        for quarter in range(4):
            acc = sq[:, 8 * quarter]
            for i in range(1, 8):
                acc = (acc + sq[:, 8 * quarter + i]).astype(F)
            part.append(acc)
        tree.append(((part[0] + part[1]).astype(F) + (part[2] + part[3]).astype(F)).astype(F))
        acc = sq[:, 0]
        for i in range(1, 32):
            acc = (acc + sq[:, i]).astype(F)
        seq.append(acc)
    return np.stack(tree, -1), np.stack(seq, -1)


def first_min(err):
    return np.argmin(err, axis=-1)          # numpy's argmin returns the first minimum


def search(want=2, seed=11):
    rng = np.random.default_rng(seed)
    found = []
    tries = 0
    while len(found) < want and tries < 4000:
        tries += 1
        base = bf16((rng.standard_normal(31) * 0.02 + 0.001).astype(F))
        xb = widen(base)
        lo, hi = xb.min(), xb.max()
        # every bf16 strictly inside (lo, hi): walk the bit patterns of both signs
        cand = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
        cand = cand[(cand & 0x7F80) != 0x7F80]
        v = widen(cand)
        cand = cand[(v > lo) & (v < hi)]
        pos = int(rng.integers(0, 32))
        blocks = np.empty((cand.size, 32), np.uint16)
        blocks[:, :pos] = base[:pos]
        blocks[:, pos] = cand
        blocks[:, pos + 1:] = base[pos:]
        tree, seq = scores(widen(blocks))
        flip = np.nonzero(first_min(tree) != first_min(seq))[0]
        if flip.size:
            found.append(blocks[flip[0]])
    return found, tries


def main():
    found, tries = search()
    out = {"_source": __doc__.strip().splitlines()[0],
           "_how": f"tests/golden/q4k_mse_near_ties.py, seed 11, {tries} base sub-blocks searched",
           "subblocks_bf16_bits": [[int(b) for b in blk] for blk in found]}
    with open(os.path.join(HERE, "q4k_mse_near_ties.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(f"{len(found)} sub-blocks after {tries} tries")


if __name__ == "__main__":
    main()
