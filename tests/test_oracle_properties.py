"""Property tests of the oracle over randomly drawn inputs (hypothesis), each property
fixed by the mathematics of the method rather than by the oracle's own code:

* the top-p selection: the kept set is the first k nodes in (score descending, id
  ascending) order, its softmax mass (scipy's, not the oracle's) reaches p while one node
  fewer does not, it does not depend on the order the frontier is listed in nor on a common
  shift of the scores, and on small frontiers no smaller set reaches p (brute force over
  every subset, ties included);
* the pooling rule: a summary is a convex combination of its children, and shifting every
  child by one vector shifts the summary by that vector (the softmax over children sees
  the same shift of R . x on every child and is unchanged);
* the descent: the selected tokens are ascending, unique and inside the cache, hold the
  anchor and the tail, and apart from those are whole blocks of b tokens under the kept
  level-1 nodes; each level's frontier is the children of the nodes kept one level up;
* the attention output is a convex combination of the selected values.

Each property is also run against planted mistakes (a wrong tie-break, a strict cut, a
mass without the exponential), which must fail it. All CPU.

Source: "Zyphra présente Zyphra Hierarchical Attention (ZHA), une voie vers une attention
vraiment sous-quadratique" (Le Fil IA), paragraph 1: contiguous blocks, one summary key
per block from 16 reference queries, the smallest set covering a fraction p of the
estimated mass at each level, expansion of the kept branches, the first token always kept.
"""

import itertools

import numpy as np
import pytest
import scipy.special
from hypothesis import HealthCheck, assume, given, settings
from hypothesis import strategies as st

import oracle as O

SETTINGS = settings(max_examples=150, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])


# ------------------------------------------------------------------------ selection

@st.composite
def frontiers(draw, max_n=40, integer_scores=False):
    """(F ascending distinct node ids, float32 scores, p). Integer-valued scores draw many
    exact ties."""
    n = draw(st.integers(1, max_n))
    ids = draw(st.lists(st.integers(0, 10_000), min_size=n, max_size=n, unique=True))
    F = np.sort(np.array(ids, np.int64))
    if integer_scores:
        s = np.array(draw(st.lists(st.integers(-6, 6), min_size=n, max_size=n)), np.float32)
    else:
        s = np.array(draw(st.lists(st.floats(-8, 8, allow_nan=False, width=32),
                                   min_size=n, max_size=n)), np.float32)
    p = float(np.float32(draw(st.floats(0.01, 1.0))))
    return F, s, p


def _rank_order(F, s):
    """Positions of the frontier in (score descending, id ascending) order."""
    return sorted(range(F.size), key=lambda i: (-float(s[i]), int(F[i])))


def _clear_of_boundaries(F, s, p):
    """True when no prefix mass of the ranked frontier lies within 1e-9 of p, so that
    float64 rounding of the masses cannot move the cut."""
    m = scipy.special.softmax(s.astype(np.float64))
    C = np.cumsum(m[_rank_order(F, s)])
    return bool(np.all(np.abs(C - p) > 1e-9))


def check_cut(select, F, s, p):
    kept, _ = select(F, s, p)
    assert np.all(np.diff(kept) > 0)
    if p >= 1.0:
        assert np.array_equal(kept, F)
        return
    m = scipy.special.softmax(s.astype(np.float64))
    order = _rank_order(F, s)
    k = kept.size
    # the kept set is a prefix of the ranked frontier ...
    assert np.array_equal(kept, np.sort(F[order[:k]]))
    # ... the shortest one whose mass reaches p
    assert m[order[:k]].sum() >= p
    assert k == 1 or m[order[:k - 1]].sum() < p


def check_listing_order_and_shift(select, F, s, p, seed):
    kept, _ = select(F, s, p)
    perm = np.random.default_rng(seed).permutation(F.size)
    kept_p, _ = select(F[perm], s[perm], p)
    assert np.array_equal(kept_p, kept)
    # a common shift of every score (exact in float32 for integer-valued scores)
    s_int = np.round(s).astype(np.float32)
    a, _ = select(F, s_int, p)
    b, _ = select(F, (s_int + np.float32(5.0)).astype(np.float32), p)
    assert np.array_equal(a, b)


def check_minimal_by_brute_force(select, F, s, p):
    kept, _ = select(F, s, p)
    m = scipy.special.softmax(s.astype(np.float64))
    if p >= 1.0:
        assert kept.size == F.size
        return
    best = None
    for k in range(1, F.size + 1):
        if any(m[list(c)].sum() >= p for c in itertools.combinations(range(F.size), k)):
            best = k
            break
    assert kept.size == best


@SETTINGS
@given(frontiers())
def test_cut_is_the_shortest_ranked_prefix_reaching_p(fsp):
    F, s, p = fsp
    assume(_clear_of_boundaries(F, s, p))
    check_cut(O.select_top_p, F, s, p)


@SETTINGS
@given(frontiers(integer_scores=True), st.integers(0, 2 ** 31 - 1))
def test_cut_with_ties_ignores_listing_order_and_score_shift(fsp, seed):
    F, s, p = fsp
    assume(_clear_of_boundaries(F, s, p))
    check_cut(O.select_top_p, F, s, p)
    check_listing_order_and_shift(O.select_top_p, F, s, p, seed)


@SETTINGS
@given(frontiers(max_n=9, integer_scores=True))
def test_no_smaller_set_reaches_p(fsp):
    F, s, p = fsp
    assume(_clear_of_boundaries(F, s, p))
    check_minimal_by_brute_force(O.select_top_p, F, s, p)


# planted mistakes: each must break at least one of the properties above on these inputs

def _sel_wrong_tiebreak(F, s, p):
    F = np.asarray(F, np.int64)
    s64 = np.asarray(s, np.float64)
    if p >= 1.0:
        return F.copy(), []
    order = np.lexsort((-F, -s64))               # ties by descending id
    e = np.exp(s64 - s64.max())
    C = np.cumsum(e[order]) / e.sum()
    k = int(np.nonzero(C >= p)[0][0]) + 1
    return np.sort(F[order[:k]]), []


def _sel_strict_cut(F, s, p):
    F = np.asarray(F, np.int64)
    s64 = np.asarray(s, np.float64)
    if p >= 1.0:
        return F.copy(), []
    order = np.lexsort((F, -s64))
    e = np.exp(s64 - s64.max())
    C = np.cumsum(e[order]) / e.sum()
    hit = np.nonzero(C > p)[0]                   # strictly above p
    k = int(hit[0]) + 1 if hit.size else F.size
    return np.sort(F[order[:k]]), []


def _sel_no_exp(F, s, p):
    F = np.asarray(F, np.int64)
    s64 = np.asarray(s, np.float64)
    if p >= 1.0:
        return F.copy(), []
    order = np.lexsort((F, -s64))
    e = s64 - s64.min() + 1.0                    # mass linear in the score
    C = np.cumsum(e[order]) / e.sum()
    k = int(np.nonzero(C >= p)[0][0]) + 1
    return np.sort(F[order[:k]]), []


def _fixed_cases():
    """Seeded frontiers with ties and a few exact mass boundaries."""
    rng = np.random.default_rng(7)
    cases = []
    for _ in range(60):
        n = int(rng.integers(2, 9))
        F = np.sort(rng.choice(1000, size=n, replace=False)).astype(np.int64)
        s = rng.integers(-3, 4, size=n).astype(np.float32)
        p = float(np.float32(rng.uniform(0.05, 0.99)))
        cases.append((F, s, p))
    # equal scores with p a whole number of nodes' mass: the cut sits exactly on p
    F = np.arange(4, dtype=np.int64)
    cases.append((F, np.zeros(4, np.float32), 0.5))
    return cases


def _fails(select):
    for i, (F, s, p) in enumerate(_fixed_cases()):
        try:
            check_cut(select, F, s, p)
            check_listing_order_and_shift(select, F, s, p, i)
            check_minimal_by_brute_force(select, F, s, p)
        except AssertionError:
            return True
    return False


def test_the_oracle_passes_the_fixed_cases():
    assert not _fails(O.select_top_p)


@pytest.mark.parametrize("mistake", [_sel_wrong_tiebreak, _sel_strict_cut, _sel_no_exp])
def test_planted_selection_mistakes_fail_the_properties(mistake):
    assert _fails(mistake)


# -------------------------------------------------------------------------- pooling

@st.composite
def nodes(draw):
    n = draw(st.integers(1, 4))
    b = draw(st.integers(2, 6))
    d = draw(st.sampled_from([4, 8, 16]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    scale = draw(st.sampled_from([0.1, 1.0, 4.0]))
    rng = np.random.default_rng(seed)
    children = rng.standard_normal((n, b, d)) * scale
    R = rng.standard_normal((O.N_REF, d)) * draw(st.sampled_from([0.0, 0.3, 1.0, 3.0]))
    return children, R, rng.standard_normal(d) * scale


def check_pool(pool, children, R, v):
    d = children.shape[2]
    tau = O.sigma(d)
    X = pool(children, R, tau)
    lo, hi = children.min(axis=1), children.max(axis=1)
    tol = 1e-12 * (1.0 + np.abs(children).max())
    assert np.all(X >= lo - tol) and np.all(X <= hi + tol)     # convex combination
    Xs = pool(children + v[None, None, :], R, tau)
    assert np.allclose(Xs, X + v[None, :], rtol=0, atol=1e-9 * (1.0 + np.abs(children).max()))


@SETTINGS
@given(nodes())
def test_pool_is_convex_and_translation_equivariant(case):
    check_pool(O.pool, *case)


def _pool_unnormalised(children, R, tau):
    n, b, d = children.shape
    z = tau * (children.reshape(n * b, d) @ R.T).reshape(n, b, R.shape[0])
    a = np.exp(z - z.max(axis=1, keepdims=True))              # softmax without its division
    return np.einsum("nb,nbd->nd", a.mean(axis=2), children)


def _pool_softmax_over_queries(children, R, tau):
    n, b, d = children.shape
    z = tau * (children.reshape(n * b, d) @ R.T).reshape(n, b, R.shape[0])
    a = scipy.special.softmax(z, axis=2)                        # over the 16 queries
    w = a.mean(axis=2)
    return np.einsum("nb,nbd->nd", w, children)


@pytest.mark.parametrize("mistake", [_pool_unnormalised, _pool_softmax_over_queries])
def test_planted_pooling_mistakes_fail_the_properties(mistake):
    rng = np.random.default_rng(3)
    failed = False
    for _ in range(20):
        children = rng.standard_normal((3, 4, 8)) * 2.0
        R = rng.standard_normal((O.N_REF, 8))
        try:
            check_pool(mistake, children, R, rng.standard_normal(8) * 2.0)
        except AssertionError:
            failed = True
            break
    assert failed


# -------------------------------------------------------------------------- descent

@st.composite
def trees(draw):
    b = draw(st.integers(2, 4))
    L = draw(st.integers(1, 3))
    n_top = draw(st.integers(0, 5))
    tail = draw(st.integers(0, b ** L - 1))
    N = n_top * b ** L + tail
    assume(N >= 1)
    d = draw(st.sampled_from([4, 8]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    p = float(np.float32(draw(st.floats(0.05, 1.0))))
    anchor = draw(st.integers(0, N))
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((N, d)).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    R = (rng.standard_normal((O.N_REF, d)) / np.sqrt(d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    return dict(b=b, L=L, N=N, n_top=n_top, d=d, p=p, anchor=anchor, K=K, V=V, R=R, q=q)


@SETTINGS
@given(trees())
def test_descent_structure(t):
    b, L, N = t["b"], t["L"], t["N"]
    levels = O.build_tree_unit(t["K"], t["R"], b, L)
    res = O.attend_head(t["q"], levels, t["K"], t["V"], b, L, t["p"], t["anchor"])
    S = res.S
    assert np.all(np.diff(S) > 0) and (S.size == 0 or (S[0] >= 0 and S[-1] < N))
    fixed = set(range(min(t["anchor"], N))) | set(range(t["n_top"] * b ** L, N))
    assert fixed <= set(S.tolist())
    if t["n_top"]:
        decisions = res.levels                                  # levels L .. 1
        assert np.array_equal(decisions[0].frontier, np.arange(t["n_top"]))
        for up, down in zip(decisions, decisions[1:]):
            want = (up.kept[:, None] * b + np.arange(b)[None, :]).reshape(-1)
            assert np.array_equal(down.frontier, want)
        for dec in decisions:
            assert set(dec.kept.tolist()) <= set(dec.frontier.tolist()) and dec.kept.size >= 1
        blocks = {int(c) * b + i for c in decisions[-1].kept for i in range(b)}
        assert set(S.tolist()) == blocks | fixed
    else:
        assert S.size == N                                      # the whole cache is the tail
    # the output is a convex combination of the selected values
    Vs = t["V"][S].astype(np.float64)
    tol = 1e-9 * (1.0 + np.abs(Vs).max())
    assert np.all(res.O >= Vs.min(axis=0) - tol) and np.all(res.O <= Vs.max(axis=0) + tol)
