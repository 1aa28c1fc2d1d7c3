"""Write train11m_hot_slices.npz: the fp64 oracle's core gradients on the
hottest slices of the train11m workload (G1 slice i1 = 0, G2 slice i2 = 0,
G3 slice i3 = 0), with a fingerprint of the inputs they were computed from.

Under Zipf(1.1) row popularity without a permutation, row 0 and its
neighbours take the bulk of the lookups, so these slices sum the most terms
of the whole backward: they are where accumulation precision shows first.
Only the lookups with i1 = 0, i2 = 0 or i3 = 0 contribute to them, so the
oracle runs on that subset (Tensor-Train decomposition of the embedding
table, the gradients of the three cores). Calls only the oracle and the
seeded input generators; takes a few minutes on a multi-core CPU.

    python tests/golden/make_train11m_hot_slices.py
"""
from __future__ import annotations

import hashlib
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "train11m_hot_slices.npz")


def fingerprint(p) -> str:
    """sha256 prefix over every input array of the problem."""
    h = hashlib.sha256()
    for a in (p.indices, p.offsets, p.grad_out, p.g1, p.g2, p.g3):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:32]


def main():
    sys.path.insert(0, ROOT)
    import oracle
    import workloads as wl

    p = wl.make("train11m")
    t = p.tables[0]
    m1 = t.m[0]
    n1, n2, n3 = t.n
    R = t.rank
    pl = oracle.plan_problem(p, 256)
    key = pl["key"].astype(np.int64)
    i1, i2, i3 = key % m1, key // m1, pl["i3"].astype(np.int64)
    mask = ((i1 == 0) | (i2 == 0) | (i3 == 0)).astype(np.uint8)
    d1, d2, d3 = oracle.backward_problem(p, mask=mask)
    np.savez_compressed(OUT, fingerprint=np.array(fingerprint(p)),
                        lookups=np.array(int(mask.sum())),
                        dg1_i1_0=d1[:n1 * R], dg2_i2_0=d2[:R * n2 * R], dg3_i3_0=d3[:R * n3])
    print("wrote", OUT, "from", int(mask.sum()), "lookups")


if __name__ == "__main__":
    main()
