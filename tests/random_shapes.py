"""Seeded random workload shapes for the sweep tests.

Each case draws a shape the five named workloads do not reach: dtype and
head dim, the GQA group and KV-head count, the tree budget and its stage
split, the draft count, ragged prefixes (empty, one token, page and tile
edges, long), the vocabulary (sometimes not a multiple of the vector width),
the page table layout and the confidence model.  Sizes stay where the oracle
finishes each whole step in about a second.
"""
import numpy as np

import workloads as W

N_CASES = 24
MAX_ROWS = 24000  # B * n_max * Hq, the attention rows the oracle computes
MAX_DRAFT = 256   # draft nodes per sequence the build call accepts


def random_spec(i: int) -> dict:
    rng = np.random.default_rng(7000 + i)
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    while Hkv * G > 64:
        G //= 2
    kmax = int(rng.choice([1, 2, 7, 15, 16, 31, 33, 60, 64, 100, 127]))
    k1 = int(rng.integers(0, kmax + 1))
    k2 = int(rng.integers(0, k1 + 1))
    k3 = int(rng.integers(0, k2 + 1))
    n_draft = int(rng.integers(0, min(2 * kmax + 2, MAX_DRAFT + 1)))
    B = int(rng.integers(1, 7))
    while B > 1 and B * (kmax + 1) * Hkv * G > MAX_ROWS:
        B -= 1
    prefix = []
    for _ in range(B):
        kind = int(rng.integers(0, 6))
        if kind == 0:
            p = 0
        elif kind == 1:
            p = 1
        elif kind == 2:
            p = int(rng.integers(2, 100))
        elif kind == 3:
            p = 16 * int(rng.integers(1, 64))              # a page edge
        elif kind == 4:
            p = 64 * int(rng.integers(1, 40)) + int(rng.integers(-1, 2))  # a tile edge
        else:
            p = int(rng.integers(100, 3000))
        prefix.append(max(p, 0))
    V = int(rng.integers(300, 5000))
    if rng.random() < 0.5:
        V -= V % 8
    conf = str(rng.choice(["product", "uniform"]))
    if n_draft >= 8 and rng.random() < 0.3:
        conf = "forced"  # needs trees deep enough for every stage outcome
    return dict(dtype=dtype, B=B, Hq=Hkv * G, Hkv=Hkv, D=D, prefix_list=prefix, kmax=kmax,
                stage_k_ret=[k1, k2, k3], n_draft=n_draft, V=V, S=int(rng.choice([2, 4, 8])),
                conf=conf, table=str(rng.choice(["identity", "permuted"])), seed=9000 + i,
                prefix=(0, 0))


def make_case(i: int):
    return W.make("qwen3_8b_b16", **random_spec(i))
