"""CPU oracle for tree-indexed sparse decode attention (Zyphra Hierarchical Attention).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product path (the HIP library and
its Python binding) never calls it, and it shares no code with that path.

Source: "Zyphra présente Zyphra Hierarchical Attention (ZHA), une voie vers une
attention vraiment sous-quadratique" (Le Fil IA, from MarkTechPost), paragraph 1,
which states the whole mechanism:

* the full KV cache is kept; the tree only decides which keys each query reads;
* keys are cut into contiguous blocks, each summarised by one summary key
  obtained from 16 learned reference queries, then grouped level by level
  (blocks of 4 with 6 levels give top nodes of 4,096 tokens);
* at inference a query scores the top nodes, keeps the smallest set covering a
  fraction p of the estimated attention mass, then expands only those branches
  down to raw KV entries;
* the first token is always kept as an anchor.

Paragraph 2 of the same page fixes p = 0.95 and the two geometries (blocks of
4 with 6 levels; blocks of 256 with 1 level).

Readings where the page is silent:

* pooling (not stated beyond "from 16 reference queries"): each reference query
  attends over a node's b children with a softmax at scale tau = 1/sqrt(d); the
  16 attention outputs are averaged. The summary is a convex combination of the
  children. Upper levels pool the stored level below with the same rule and
  the same reference queries.
* estimated mass: softmax over the current frontier of sigma * q . X, sigma =
  1/sqrt(d) (renormalised at every level); the same top-p rule is applied at
  every level to the children of the nodes kept one level up.
* order: score descending, ties by ascending node index; "covering" means the
  cumulative mass reaches p (>=); p >= 1 keeps every node.
* anchor: tokens 0 .. anchor-1 are added after the selection (anchor = 1 is the
  page's rule); they take no part in the mass.
* final attention: exact softmax attention at scale sigma over the gathered keys.
* a cache that does not fill whole top nodes (the page is silent; needed to use the
  tree while tokens are appended one at a time): a node exists once every token under
  it is cached, and is pooled from its complete children; the search runs over the
  complete top nodes, and the tail (tokens after the last complete top node) is always
  attended, like the anchor, taking no part in the mass. With no complete top node the
  whole cache is the tail.

Precision: inputs are upcast exactly to float64 and every sum is float64. The
method stores two float32 quantities that decide integers downstream, and the
oracle rounds at exactly those points: the summary pyramid (stored float32) and
the node scores (float32, so the selection decision is taken on float32 scores
as the GPU path takes it). Masses are exp(s - max s) of those float32 scores,
evaluated in float64; cumulative masses are float64.

Pins (tests marked "not gpu"): dense attention through torch's SDPA at p = 1
and for a one-level tree with one node; closed forms of the pooling rule
(R = 0 gives the mean, identical children, one-hot softmax, two-way split,
permutation invariance, convexity); subtree coverage of b^L tokens; token 0
always kept; a brute-force minimal-set search over every subset of small
frontiers; score-scale and cut-condition closed forms. The pooling rule and the
per-level renormalisation are readings the pages do not fix: the oracle is
pinned to those readings, not to the pages ("parity unpinned by the pages" for
those two choices; everything else about them is pinned by the tests above).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

N_REF = 16           # reference queries per KV head (page 3, paragraph 1)
NEAR_TIE_REL = 1e-5  # relative score gap / mass gap under which a decision is fragile


def sigma(d: int) -> float:
    """Scale of scaled dot-product attention, 1/sqrt(d), used both for node
    scores and for the final attention (reading of page 3, paragraph 1)."""
    return 1.0 / np.sqrt(float(d))


# ---------------------------------------------------------------------------
# Build: the summary-key pyramid (page 3, paragraph 1: contiguous blocks, one
# summary key per block from 16 reference queries, grouped level by level).
# ---------------------------------------------------------------------------

def pool(children: np.ndarray, R: np.ndarray, tau: float) -> np.ndarray:
    """One summary key per node from its children.

    children: [n, b, d] float64, R: [16, d] float64 -> [n, d] float64.
    For each reference query r and child c: z[r, c] = tau * R[r] . x[c];
    a[r, :] = softmax over the b children; w[c] = mean over r of a[r, c];
    summary = sum_c w[c] * x[c].
    """
    n, b, d = children.shape
    z = tau * (children.reshape(n * b, d) @ R.T).reshape(n, b, R.shape[0])   # [n, b, 16]
    z = z - z.max(axis=1, keepdims=True)
    a = np.exp(z)
    a = a / a.sum(axis=1, keepdims=True)        # softmax over children, per reference query
    w = a.mean(axis=2)                          # [n, b]: average over reference queries
    return np.einsum("nb,nbd->nd", w, children)


def build_tree_unit(K_u: np.ndarray, R_g: np.ndarray, b: int, L: int) -> list:
    """Pyramid of one (sequence, KV head): levels[l] is the float32 [N // b^l, d]
    array of level-l summary keys for l = 1..L (levels[0] is the raw keys). Only
    complete nodes exist: node j of level l is pooled from children j b .. j b + b - 1
    of level l - 1, all of which exist."""
    N, d = K_u.shape
    if b < 2 or L < 1:
        raise ValueError("need b >= 2 and L >= 1")
    tau = sigma(d)
    R64 = np.asarray(R_g, np.float64)
    levels = [np.asarray(K_u, np.float32)]
    X = np.asarray(K_u, np.float64)
    for _ in range(L):
        n = X.shape[0] // b
        Xn = pool(X[:n * b].reshape(n, b, d), R64, tau).astype(np.float32)   # stored float32
        levels.append(Xn)
        X = Xn.astype(np.float64)
    return levels


def tail_tokens(N: int, n_top: int, b: int, L: int) -> np.ndarray:
    """Tokens after the last complete top node: always attended."""
    return np.arange(n_top * b ** L, N, dtype=np.int64)


# ---------------------------------------------------------------------------
# Search: score, top-p, expand (page 3, paragraph 1).
# ---------------------------------------------------------------------------

def node_scores(X_rows: np.ndarray, q: np.ndarray) -> np.ndarray:
    """sigma * q . X for each row, evaluated in float64, stored float32."""
    d = X_rows.shape[1]
    return (sigma(d) * (np.asarray(X_rows, np.float64) @ np.asarray(q, np.float64))).astype(np.float32)


@dataclass
class LevelDecision:
    level: int
    frontier: np.ndarray          # node ids, ascending
    scores: np.ndarray            # float32, aligned with frontier
    kept: np.ndarray              # node ids, ascending
    fragile: list = field(default_factory=list)   # [(kind, gap)]


def select_top_p(F: np.ndarray, s: np.ndarray, p: float):
    """Smallest set of frontier nodes whose estimated mass reaches p.

    Mass of node c = exp(s_c - max s) / sum over the frontier (softmax over the
    frontier). Nodes are taken in order of descending score, ties by ascending
    node id, until the cumulative mass is >= p. p >= 1 keeps every node.
    Returns (kept ids ascending, fragility list). A decision is fragile when the
    last kept and first dropped scores are within NEAR_TIE_REL (relative, floor
    1), or when a cumulative mass at the cut is within NEAR_TIE_REL of p.
    """
    F = np.asarray(F, np.int64)
    s = np.asarray(s, np.float32)
    if p >= 1.0:
        return F.copy(), []
    s64 = s.astype(np.float64)
    order = np.lexsort((F, -s64))                 # score descending, then id ascending
    e = np.exp(s64 - s64.max())
    C = np.cumsum(e[order]) / e.sum()
    hit = np.nonzero(C >= p)[0]
    k = int(hit[0]) + 1 if hit.size else F.size
    fragile = []
    if k < F.size:
        a, c = s64[order[k - 1]], s64[order[k]]
        gap = a - c
        if gap <= NEAR_TIE_REL * max(1.0, abs(a), abs(c)):
            fragile.append(("score", float(gap)))
        if C[k - 1] - p <= NEAR_TIE_REL:
            fragile.append(("mass_hi", float(C[k - 1] - p)))
    if k >= 2 and p - C[k - 2] <= NEAR_TIE_REL:
        fragile.append(("mass_lo", float(p - C[k - 2])))
    return np.sort(F[order[:k]]), fragile


def expand(kept: np.ndarray, b: int) -> np.ndarray:
    """Children of the kept nodes, ascending: {c * b + i : c in kept, i < b}."""
    kept = np.asarray(kept, np.int64)
    return (kept[:, None] * b + np.arange(b, dtype=np.int64)[None, :]).reshape(-1)


@dataclass
class HeadResult:
    O: np.ndarray                 # [d] float64
    S: np.ndarray                 # selected token ids, ascending, unique
    levels: list                  # LevelDecision for l = L .. 1

    @property
    def fragile(self) -> list:
        return [(lv.level, kind, gap) for lv in self.levels for kind, gap in lv.fragile]


def search(q: np.ndarray, levels: list, b: int, L: int, p: float, anchor: int):
    """Tree descent for one query head over one (sequence, KV head) pyramid.
    Returns (S, [LevelDecision for l = L .. 1])."""
    N = levels[0].shape[0]
    p = float(np.float32(p))          # p is a float32 argument on the C boundary
    n_top = levels[L].shape[0]
    F = np.arange(n_top, dtype=np.int64)
    decisions = []
    kept = F
    if n_top:
        for l in range(L, 0, -1):
            s = node_scores(levels[l][F], q)
            kept, fragile = select_top_p(F, s, p)
            decisions.append(LevelDecision(l, F, s, kept, fragile))
            if l > 1:
                F = expand(kept, b)
    S = np.union1d(np.arange(min(anchor, N), dtype=np.int64), expand(kept, b))
    S = np.union1d(S, tail_tokens(N, n_top, b, L))
    return S, decisions


# ---------------------------------------------------------------------------
# Router in FP4 (page 3, paragraph 4: a variant of the router in FP4 was also
# tested; nothing more is said). Reading: the router is what decides which keys a
# query reads, i.e. the summary keys and the node scores. Both operands of every
# node score are held in MXFP4 (OCP Microscaling Formats v1.0: blocks of 32
# elements along d, E2M1 elements, one E8M0 power-of-two scale per block) and the
# dot products are exact sums of their products, stored float32 like the float32
# router's scores. The pyramid itself is built in float32 as above and quantised
# level by level; the final attention still uses the unquantised query and keys.
# ---------------------------------------------------------------------------

MX_BLOCK = 32          # elements per shared scale (OCP MX v1.0)
E2M1_EMAX = 2          # exponent of the largest normal E2M1 value (6 = 1.5 * 2^2)


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code from the format's definition: sign bit 3,
    exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is subnormal
    (0.5 * mantissa)."""
    sign = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return sign * mag


def _e2m1_round(v: np.ndarray) -> np.ndarray:
    """E2M1 code of each value v (float64, already divided by its block scale):
    the nearest of the 8 magnitudes after clamping to the largest (6), ties to the
    magnitude whose mantissa bit is 0; the sign bit is the sign of v."""
    mags = [e2m1_value(c) for c in range(8)]
    a = np.minimum(np.abs(v), mags[-1])
    idx = np.zeros(a.shape, np.int64)
    best = np.abs(a - mags[0])
    for c in range(1, 8):
        dist = np.abs(a - mags[c])
        # strictly nearer, or equally near with mantissa bit 0 (the even one)
        take = (dist < best) | ((dist == best) & (c % 2 == 0))
        idx = np.where(take, c, idx)
        best = np.where(take, dist, best)
    return (idx | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def mxfp4_quantize(x: np.ndarray):
    """MXFP4 encoding of float32 rows x [..., d] (d a multiple of 32).

    Returns (codes uint8 [..., d], one 4-bit code per element, and scale exponents
    int16 [..., d / 32]). Per block: X = floor(log2(max |x|)) - 2 clamped to
    [-127, 127] (X = -127 for an all-zero block), and each element is the E2M1
    rounding of x / 2^X (OCP MX v1.0, conversion of a vector to MX format)."""
    x = np.asarray(x, np.float32).astype(np.float64)
    d = x.shape[-1]
    blocks = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))), -1000.0)
    X = np.clip(e - E2M1_EMAX, -127, 127).astype(np.int16)
    scaled = blocks / np.ldexp(1.0, X.astype(np.int64))[..., None]
    codes = _e2m1_round(scaled).reshape(x.shape)
    return codes, X


def mxfp4_dequantize(codes: np.ndarray, X: np.ndarray) -> np.ndarray:
    """float64 values of MXFP4 codes [..., d] with scale exponents [..., d / 32]."""
    table = np.array([e2m1_value(c) for c in range(16)])
    v = table[np.asarray(codes, np.int64)]
    d = v.shape[-1]
    v = v.reshape(v.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    return (v * np.ldexp(1.0, np.asarray(X, np.int64))[..., None]).reshape(codes.shape)


def mxfp4_round_trip(x: np.ndarray) -> np.ndarray:
    """x quantised to MXFP4 and read back (float64)."""
    return mxfp4_dequantize(*mxfp4_quantize(x))


def router_levels(levels: list) -> list:
    """The FP4 router's view of one unit's pyramid: levels[0] (raw keys) unchanged,
    every summary level replaced by its MXFP4 round trip."""
    return [levels[0]] + [mxfp4_round_trip(lv) for lv in levels[1:]]


def search_fp4(q: np.ndarray, levels: list, b: int, L: int, p: float, anchor: int):
    """Tree descent with the FP4 router: the same search, with the query and every
    summary level quantised to MXFP4 for the node scores."""
    return search(mxfp4_round_trip(q), router_levels(levels), b, L, p, anchor)


def attend_head_fp4(q, levels, K_u, V_u, b, L, p, anchor=1) -> HeadResult:
    """FP4-router search, then exact attention of the unquantised query over the
    selected keys."""
    S, decisions = search_fp4(q, levels, b, L, p, anchor)
    return HeadResult(attention_over(q, K_u, V_u, S), S, decisions)


def attention_over(q: np.ndarray, K_u: np.ndarray, V_u: np.ndarray, S: np.ndarray) -> np.ndarray:
    """Exact softmax attention of q over the keys/values with ids in S
    (scale sigma), float64."""
    d = K_u.shape[1]
    lam = sigma(d) * (np.asarray(K_u[S], np.float64) @ np.asarray(q, np.float64))
    w = np.exp(lam - lam.max())
    w = w / w.sum()
    return w @ np.asarray(V_u[S], np.float64)


def attend_head(q, levels, K_u, V_u, b, L, p, anchor=1) -> HeadResult:
    S, decisions = search(q, levels, b, L, p, anchor)
    return HeadResult(attention_over(q, K_u, V_u, S), S, decisions)


# ---------------------------------------------------------------------------
# Several queries of one sequence at different positions, causally masked (page 3,
# paragraph 3: making the search itself sparse opens the way to attention that is truly
# sub-quadratic, i.e. to running it for every position of a sequence). Reading: the
# query at position t (0-based) sees exactly the cache of its first t + 1 tokens; its
# search, anchor and tail are those of that cache (the reading for a cache that does not
# fill whole top nodes): nodes that reach past t are not complete for it and are not
# searched, and the tokens after its last complete top node are attended like the anchor.
# The pyramid is built once over the whole cache; a node's summary depends only on the
# tokens under it, so the prefix of the full pyramid is the pyramid of the prefix.
# ---------------------------------------------------------------------------

def causal_view(levels: list, K_u: np.ndarray, V_u: np.ndarray, b: int, L: int, pos: int):
    """The pyramid levels and K, V that a query at position `pos` sees (tokens
    0 .. pos)."""
    n = int(pos) + 1
    if not 1 <= n <= K_u.shape[0]:
        raise ValueError("position outside the cache")
    lv = [levels[0][:n]] + [levels[l][: n // b ** l] for l in range(1, L + 1)]
    return lv, K_u[:n], V_u[:n]


def attend_head_causal(q, levels, K_u, V_u, b, L, p, anchor, pos) -> HeadResult:
    """Search and exact attention of the query at position `pos` over what it sees."""
    lv, Kc, Vc = causal_view(levels, K_u, V_u, b, L, pos)
    return attend_head(q, lv, Kc, Vc, b, L, p, anchor)
