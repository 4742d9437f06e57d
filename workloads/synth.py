"""Seeded synthetic workloads: clustered keys, Gaussian values, planted needles.

The recipe follows the decode workloads described for Zyphra Hierarchical
Attention's tree-indexed sparse attention (MarkTechPost summary as printed by
Le Fil IA, paragraph 1: deep tree of blocks of 4 with 6 levels, wide tree of
blocks of 256 with 1 level, p = 0.95) and stands in for the long-context
retrieval suites that page reports on (RULER-13 at 256K, LongBench v2), which
are not available here: long contexts of clustered keys with a few planted
"facts" (needle keys aimed at particular query heads) among distractors.

Recipe (all draws are float32 from numpy's PCG64, keyed by
``SeedSequence([seed, sequence, kv_head, stream])`` so any (sequence, KV head)
slice can be regenerated alone):

* keys      K[b,g,i] = mu[b,g,i // 64] + 0.3 * eps[b,g,i],  mu, eps ~ N(0, I_d)
* values    V[b,g,i] ~ N(0, I_d)
* reference queries R[g] ~ N(0, I_d / d) (16 per KV head; variance 1/d)
* queries   Q[b,t,h] ~ N(0, I_d); in the "agree" variant the G heads of a KV head share
            most of one direction and every score is scaled up (gen_Q)
* needle    K[b, h // G, pos] = 4 * q / |q| for the aimed query q; never at token 0

then every tensor is rounded once to the storage dtype (bf16 round-to-nearest-
even through torch, or kept as float32). The rounded values are the canonical
inputs for every consumer.

Streams: 0 centroids, 1 key noise, 2 values, 3 queries, 4 reference queries,
5 needle placement, 6 shared query directions.
"""

from __future__ import annotations

import math

import numpy as np

CLUSTER = 64
N_REF = 16

# name -> shapes. "dtype" is the storage dtype of K, V, Q and R.
WORKLOADS = {
    # tiny fp32 case the oracle finishes in well under a second
    "tiny": dict(dtype="f32", B=1, T=8, Hq=1, Hkv=1, d=64, N=4096, b=4, L=3,
                 p=(0.95,), seed=1, needles="tiny"),
    # single layer, 32K context, GQA 32/4, deep tree (8 top nodes)
    "32k_deep": dict(dtype="bf16", B=8, T=1, Hq=32, Hkv=4, d=128, N=32768, b=4, L=6,
                     p=(0.95,), seed=2, needles="per_head4"),
    # single layer, 256K context, deep tree b=4 L=6 (64 top nodes of 4096 tokens)
    "256k_deep": dict(dtype="bf16", B=4, T=1, Hq=32, Hkv=4, d=128, N=262144, b=4, L=6,
                      p=(0.95,), seed=3, needles="stratified16"),
    # the same keys and values as 256k_deep, with queries whose 8 heads per KV head share
    # most of one direction (correlation 0.81) and scores three times as sharp: each head
    # reads about 2% of the keys (near the ~1.1% read on real attention with the deep tree
    # at p = 0.95 in the Le Fil IA page's paragraph 2) and the union of a KV head's heads
    # about 7%, where the independent queries above read 41% per head and 98.5% in union
    "256k_deep_agree": dict(dtype="bf16", B=4, T=1, Hq=32, Hkv=4, d=128, N=262144, b=4, L=6,
                            p=(0.95,), seed=3, needles="stratified16", q_shared=0.9,
                            q_scale=3.0),
    # the same tensors as 256k_deep (same seed), wide tree b=256 L=1
    "256k_wide": dict(dtype="bf16", B=4, T=1, Hq=32, Hkv=4, d=128, N=262144, b=256, L=1,
                      p=(0.8, 0.95, 0.99), seed=3, needles="stratified16"),
    # single layer, 1M context, deep tree b=4 L=7 (64 top nodes of 16384 tokens)
    "1m_deep": dict(dtype="bf16", B=8, T=1, Hq=32, Hkv=4, d=128, N=1048576, b=4, L=7,
                    p=(0.95,), seed=5, needles="stratified16"),
}


def spec(name: str, **overrides) -> dict:
    """Return a copy of a named workload with optional shape overrides.

    ``r_std`` (default 1/sqrt(d)) and ``needles`` may also be overridden, e.g.
    ``r_std=1.0`` for sharp pooling softmaxes in tests.
    """
    s = dict(WORKLOADS[name])
    s["name"] = name
    s.update(overrides)
    s.setdefault("r_std", 1.0 / math.sqrt(s["d"]))
    s.setdefault("anchor", 1)
    return s


def _rng(seed: int, b: int, g: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, b, g, stream])))


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype; return them as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        import torch

        return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(f"unknown dtype {dtype}")


def gen_R(s: dict) -> np.ndarray:
    """Reference queries, [Hkv, 16, d], rounded to the storage dtype."""
    out = np.empty((s["Hkv"], N_REF, s["d"]), np.float32)
    for g in range(s["Hkv"]):
        out[g] = _rng(s["seed"], 0, g, 4).standard_normal((N_REF, s["d"]), dtype=np.float32)
        out[g] *= np.float32(s["r_std"])
    return to_storage(out, s["dtype"])


def gen_Q(s: dict) -> np.ndarray:
    """Decode queries, [B, T, Hq, d], rounded to the storage dtype.

    By default every query is an independent N(0, I_d) draw. With ``q_shared`` = rho > 0
    the G query heads of a KV head lean on one shared direction per (sequence, query,
    KV head), u ~ N(0, I_d) from stream 6: q = q_scale * (sqrt(1 - rho^2) eps + rho u),
    which keeps each query N(0, q_scale^2 I_d) while the heads of a group agree; a
    ``q_scale`` above 1 sharpens every softmax over the keys."""
    out = np.empty((s["B"], s["T"], s["Hq"], s["d"]), np.float32)
    for b in range(s["B"]):
        out[b] = _rng(s["seed"], b, 0, 3).standard_normal((s["T"], s["Hq"], s["d"]), dtype=np.float32)
    rho, scale = float(s.get("q_shared", 0.0)), float(s.get("q_scale", 1.0))
    if rho != 0.0 or scale != 1.0:
        G = s["Hq"] // s["Hkv"]
        for b in range(s["B"]):
            u = _rng(s["seed"], b, 0, 6).standard_normal((s["T"], s["Hkv"], s["d"]),
                                                        dtype=np.float32)
            shared = np.repeat(u, G, axis=1)                       # [T, Hq, d]
            out[b] = np.float32(scale) * (np.float32(math.sqrt(1.0 - rho * rho)) * out[b]
                                          + np.float32(rho) * shared)
    return to_storage(out, s["dtype"])


def _segment(N: int, j: int, parts: int):
    lo = 1 + (j * (N - 1)) // parts
    hi = 1 + ((j + 1) * (N - 1)) // parts
    return lo, max(hi, lo + 1)


def needle_plan(s: dict, b: int) -> list:
    """Needles of sequence b as a list of (position, t, h): K[b, h // G, position]
    is set from the query Q[b, t, h]. Positions are distinct and never 0."""
    kind = s.get("needles", "none")
    N, T, Hq, Hkv = s["N"], s["T"], s["Hq"], s["Hkv"]
    G = Hq // Hkv
    rng = _rng(s["seed"], b, 0, 5)
    plan = []
    if kind == "none" or N < 4:
        return plan
    if kind == "tiny":
        # 3 needles in distinct top nodes, aimed by queries t = 0, 1, 2 of head 0
        top = s["b"] ** s["L"]
        n_top = N // top
        k = min(3, T, n_top)
        nodes = rng.choice(n_top, size=k, replace=False)
        for t, node in enumerate(nodes):
            lo = max(1, int(node) * top)
            pos = int(rng.integers(lo, (int(node) + 1) * top))
            plan.append((pos, t, 0))
    elif kind == "per_head4":
        # 4 distinct query heads, one needle each at a uniform position
        k = min(4, Hq)
        heads = rng.choice(Hq, size=k, replace=False)
        pos = rng.choice(np.arange(1, N), size=k, replace=False)
        for h, p in zip(heads, pos):
            plan.append((int(p), 0, int(h)))
    elif kind == "stratified16":
        # needle j uniform in segment j of 16 equal segments of [1, N);
        # 8 aimed heads (two per KV group when Hkv = 4), head i aimed at needles i and i + 8
        pos = [int(rng.integers(*_segment(N, j, 16))) for j in range(16)]
        n_aim = min(8, Hq)
        heads = []
        for i in range(n_aim):
            g = i % Hkv
            choices = [g * G + j for j in range(G) if g * G + j not in heads]
            heads.append(int(rng.choice(choices)) if choices else int(rng.integers(Hq)))
        for i, h in enumerate(heads):
            plan.append((pos[i], 0, h))
            plan.append((pos[i + 8], 0, h))
    else:
        raise ValueError(f"unknown needle scheme {kind}")
    return plan


def gen_KV_unit(s: dict, b: int, g: int, Q: np.ndarray | None = None):
    """Keys and values of sequence b, KV head g: two float32 [N, d] arrays whose
    values are exactly representable in the storage dtype, needles planted."""
    N, d = s["N"], s["d"]
    n_cl = -(-N // CLUSTER)
    mu = _rng(s["seed"], b, g, 0).standard_normal((n_cl, d), dtype=np.float32)
    K = _rng(s["seed"], b, g, 1).standard_normal((N, d), dtype=np.float32)
    K *= np.float32(0.3)
    K += np.repeat(mu, CLUSTER, axis=0)[:N]
    V = _rng(s["seed"], b, g, 2).standard_normal((N, d), dtype=np.float32)
    plan = needle_plan(s, b)
    if plan:
        if Q is None:
            Q = gen_Q(s)
        G = s["Hq"] // s["Hkv"]
        for pos, t, h in plan:
            if h // G != g:
                continue
            q = Q[b, t, h].astype(np.float64)
            K[pos] = (4.0 * q / np.linalg.norm(q)).astype(np.float32)
    return to_storage(K, s["dtype"]), to_storage(V, s["dtype"])


def gen_all(s: dict, device=None):
    """Every input of a workload as torch tensors in the storage dtype.

    Returns dict(K, V: [B, Hkv, N, d]; Q: [B, T, Hq, d]; R: [Hkv, 16, d]).
    Slices are generated one (sequence, KV head) at a time and copied into the
    destination (on ``device`` if given) so the host never holds a float32 copy
    of the whole cache.
    """
    import torch

    tdt = torch.bfloat16 if s["dtype"] == "bf16" else torch.float32
    B, Hkv, N, d = s["B"], s["Hkv"], s["N"], s["d"]
    Q = gen_Q(s)
    R = gen_R(s)
    K = torch.empty((B, Hkv, N, d), dtype=tdt, device=device)
    V = torch.empty((B, Hkv, N, d), dtype=tdt, device=device)
    for b in range(B):
        for g in range(Hkv):
            k, v = gen_KV_unit(s, b, g, Q)
            K[b, g].copy_(torch.from_numpy(k).to(tdt))
            V[b, g].copy_(torch.from_numpy(v).to(tdt))
    return dict(
        K=K,
        V=V,
        Q=torch.from_numpy(Q).to(tdt).to(device) if device is not None else torch.from_numpy(Q).to(tdt),
        R=torch.from_numpy(R).to(tdt).to(device) if device is not None else torch.from_numpy(R).to(tdt),
    )
