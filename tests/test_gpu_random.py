"""Randomised parity: seeded draws over the shape and parameter space the C ABI accepts
(branching factor, levels, head dim, dtype, GQA ratio, batch, queries per sequence, p,
anchor, a ragged cache, query positions), each compared with the oracle head by head.
Top nodes of up to 65,536 tokens: every geometry of the geometry sweep with b^L in that
range is reachable.

The draws are fixed by their seeds, so a failure names a reproducible case.
"""

import numpy as np
import pytest
import torch

import gpu_harness as H
import workloads as W
from oracle import compare as C

pytestmark = pytest.mark.gpu

O_TOL = H.O_TOL


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_indexed_sparse_amd as Z
    Z.load()


def _draw(seed, max_top=4096, max_n=16384):
    """One seeded configuration: top nodes of at most max_top tokens, caches of at most
    max_n tokens."""
    rng = np.random.default_rng(1000 + seed)
    b = int(rng.choice([2, 3, 4, 5, 8, 16, 64]))
    lmax = 1
    while b ** (lmax + 1) <= max_top and lmax < 12:
        lmax += 1
    # half the draws take one of the three deepest trees the cache size allows
    L = int(rng.integers(max(1, lmax - 2), lmax + 1) if rng.random() < 0.5
            else rng.integers(1, lmax + 1))
    top = b ** L
    N_cap = top * int(rng.integers(1, max(2, max_n // top) + 1))
    N_cap = min(N_cap, top * max(1, max_n // top))
    ragged = bool(rng.random() < 0.3)
    N = int(rng.integers(1, N_cap + 1)) if ragged else N_cap
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2]))
    T = int(rng.integers(1, 4))
    spec = W.spec("tiny", B=int(rng.integers(1, 3)), T=T, Hq=G * Hkv, Hkv=Hkv,
                  d=int(rng.choice([64, 128])), dtype=str(rng.choice(["f32", "bf16"])),
                  N=N_cap, b=b, L=L, needles="none")
    p = float(rng.choice([0.3, 0.5, 0.8, 0.95, 0.99, 1.0]))
    anchor = int(min(rng.choice([0, 1, 3]), N))
    positions = None
    if rng.random() < 0.4:
        positions = rng.integers(0, N, size=(spec["B"], T)).astype(np.int32)
    return spec, N, ragged, p, anchor, positions


@pytest.mark.parametrize("seed", range(96))
def test_random_configuration(seed):
    """Seeds 0-63 draw top nodes of up to 4,096 tokens in caches of up to 16K; seeds 64-95
    top nodes of up to 65,536 tokens (b^L up to 4^8, 16^4, 3^10, 2^12) in caches of up to
    128K."""
    spec, N, ragged, p, anchor, positions = (_draw(seed) if seed < 64 else
                                             _draw(seed, max_top=65536, max_n=131072))
    desc = (f"seed {seed}: b={spec['b']} L={spec['L']} N={N}/{spec['N']} d={spec['d']} "
            f"{spec['dtype']} B={spec['B']} T={spec['T']} Hq={spec['Hq']} Hkv={spec['Hkv']} "
            f"p={p} anchor={anchor} positions={'yes' if positions is not None else 'no'}")
    print(f"[{desc}]", flush=True)
    res = H.run_gpu(spec, p, anchor=anchor, N=N if ragged else None, positions=positions)
    reps, pyr = H.check_units(spec, res, p, anchor=anchor, n_tokens=N if ragged else None,
                              positions=positions)
    summ = C.summarize(reps)
    print(f"[{desc}] pyramid {pyr:.2e} {summ}", flush=True)
    H.assert_parity(spec, summ, pyr)
