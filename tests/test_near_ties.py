"""Pins of the near-tie rule (oracle.select_top_p's fragility flags) and of the comparator
rule that decides which GPU resolutions of a fragile decision a parity test accepts
(oracle.compare.fragile_ok), on hand-built frontiers whose cumulative masses come from
scipy's softmax, not from the oracle.

Each rule is also checked against planted mistakes: a copy of the function with one
mistake written into its source (a wrong cumulative entry, a wrong window, an allowance not
tied to its kind, ...) must fail at least one of the pins. All CPU.

Source of the rule: "Zyphra présente Zyphra Hierarchical Attention (ZHA), une voie vers
une attention vraiment sous-quadratique" (Le Fil IA), paragraph 1 (the kept set is the
smallest one covering a fraction p of the estimated mass). The window of 1e-5 is the
near-tie bound of this implementation's parity bar, applied to score gaps (relative, floor
1) and to cumulative masses at the cut.
"""

import inspect
import textwrap

import numpy as np
import pytest
import scipy.special

import oracle as O
from oracle import compare as C

W = O.NEAR_TIE_REL


def _frontier(n=400, step=1e-3, seed=0):
    """n nodes in shuffled id order with scores -i*step (distinct well beyond the score
    window), and the cumulative masses in descending-score order from scipy's softmax."""
    rng = np.random.default_rng(seed)
    F = np.sort(rng.choice(10 * n, size=n, replace=False)).astype(np.int64)
    rank = rng.permutation(n)                       # rank[i]: position of F[i] in the order
    s = (-rank * step).astype(np.float32)
    m = scipy.special.softmax(s.astype(np.float64))
    order = np.argsort(rank)
    Cum = np.cumsum(m[order])
    return F, s, order, Cum


def _kinds(frag):
    return sorted(k for k, _ in frag)


# --------------------------------------------------------------------------- select_top_p

def check_mass_windows(select):
    """The two mass flags fire exactly inside their 1e-5 windows, on the right entries."""
    F, s, order, Cum = _frontier()
    for j in (37, 150, 300):
        # p just below C[j]: the cut is k = j + 1 and C[k-1] - p is the window
        for delta, flagged in ((0.99 * W, True), (1.01 * W, False)):
            p = Cum[j] - delta
            kept, frag = select(F, s, p)
            assert kept.size == j + 1
            assert ("mass_hi" in _kinds(frag)) == flagged, (j, delta, frag)
            assert "mass_lo" not in _kinds(frag)
            assert "score" not in _kinds(frag)
            assert np.array_equal(kept, np.sort(F[order[:j + 1]]))
        # p just above C[j - 1]: the cut is still k = j + 1 and p - C[k-2] is the window
        for delta, flagged in ((0.99 * W, True), (1.01 * W, False)):
            p = Cum[j - 1] + delta
            kept, frag = select(F, s, p)
            assert kept.size == j + 1
            assert ("mass_lo" in _kinds(frag)) == flagged, (j, delta, frag)
            assert "mass_hi" not in _kinds(frag)
    # mid-way between two cumulative masses: nothing is fragile
    p = 0.5 * (Cum[99] + Cum[100])
    kept, frag = select(F, s, p)
    assert kept.size == 101 and frag == []


def check_score_window(select):
    """The score flag fires exactly when the last kept and the first dropped scores are
    within 1e-5, relative to the larger magnitude with a floor of 1."""
    for base in (0.25, -3.0, 40.0):
        scale = max(1.0, abs(base))
        for gap, flagged in ((0.5 * W * scale, True), (2.0 * W * scale, False)):
            s = np.array([base + 1.0, base, base - gap, base - 2.0], np.float32)
            g = float(s[1]) - float(s[2])            # the gap after float32 rounding
            F = np.arange(4)
            m = scipy.special.softmax(s.astype(np.float64))
            p = m[0] + 0.5 * m[1]                    # the cut falls on node 1
            kept, frag = select(F, s, p)
            assert kept.tolist() == [0, 1]
            assert ("score" in _kinds(frag)) == (g <= W * max(1.0, abs(float(s[1])),
                                                             abs(float(s[2])))) == flagged


def check_flags_never_fire_at_the_ends(select):
    """No mass_hi when every node is kept by the mass (nothing dropped); no mass_lo when a
    single node covers p."""
    F, s, order, Cum = _frontier(n=8, step=0.5)
    kept, frag = select(F, s, Cum[-1] - 0.5 * W)
    assert kept.size == F.size and "mass_hi" not in _kinds(frag)
    kept, frag = select(F, s, Cum[0] - 0.5 * W)
    assert kept.size == 1 and "mass_lo" not in _kinds(frag) and "mass_hi" in _kinds(frag)


SELECT_PINS = [check_mass_windows, check_score_window, check_flags_never_fire_at_the_ends]


@pytest.mark.parametrize("pin", SELECT_PINS, ids=lambda f: f.__name__)
def test_select_top_p_near_tie_flags(pin):
    pin(O.select_top_p)


def _mutant(fn, old, new, extra_globals=None):
    """A copy of fn with `old` replaced by `new` (exactly once) in its source."""
    src = textwrap.dedent(inspect.getsource(fn))
    assert src.count(old) == 1, (fn.__name__, old)
    ns = dict(fn.__globals__)
    ns.update(extra_globals or {})
    exec(compile(src.replace(old, new), f"<mutant of {fn.__name__}>", "exec"), ns)
    return ns[fn.__name__]


SELECT_MUTANTS = [
    ("mass_lo reads the cut's entry", "p - C[k - 2] <= NEAR_TIE_REL", "p - C[k - 1] <= NEAR_TIE_REL"),
    ("mass_lo reads two entries before", "p - C[k - 2] <= NEAR_TIE_REL", "p - C[k - 3] <= NEAR_TIE_REL"),
    ("mass_hi reads the entry before", "C[k - 1] - p <= NEAR_TIE_REL", "C[k - 2] - p <= NEAR_TIE_REL"),
    ("mass_hi window ten times wider", "C[k - 1] - p <= NEAR_TIE_REL", "C[k - 1] - p <= 10 * NEAR_TIE_REL"),
    ("mass_lo window halved", "p - C[k - 2] <= NEAR_TIE_REL", "p - C[k - 2] <= 0.5 * NEAR_TIE_REL"),
    ("score window without the floor of 1", "max(1.0, abs(a), abs(c))", "max(abs(a), abs(c))"),
    ("score gap as an absolute value", "gap <= NEAR_TIE_REL", "abs(gap) <= 10 * NEAR_TIE_REL"),
    ("flags swapped", '("mass_hi", float(C[k - 1] - p))', '("mass_lo", float(C[k - 1] - p))'),
]


@pytest.mark.parametrize("name,old,new", SELECT_MUTANTS, ids=[m[0] for m in SELECT_MUTANTS])
def test_select_pins_catch_planted_mistakes(name, old, new):
    bad = _mutant(O.select_top_p, old, new)
    failed = 0
    for pin in SELECT_PINS:
        try:
            pin(bad)
        except (AssertionError, IndexError):
            failed += 1
    assert failed > 0, f"no pin fails with the planted mistake: {name}"


# --------------------------------------------------------------------------- fragile_ok

def _ten():
    """Ten nodes (ids shuffled against the order) with scores 10, 9, ..., 1 (clearly
    apart), and the ids in descending-score order."""
    F = np.array([3, 8, 11, 14, 20, 21, 30, 41, 42, 57], np.int64)
    s = np.array([4, 9, 1, 7, 10, 2, 6, 3, 8, 5], np.float32)
    order = F[np.argsort(-s, kind="stable")]
    return F, s, order


def _top(order, k):
    return np.sort(order[:k])


def check_sizes_follow_the_kind(ok):
    F, s, order = _ten()
    k = 5
    kept = _top(order, k)
    hi, lo, sc = [("mass_hi", 1e-6)], [("mass_lo", 1e-6)], [("score", 0.0)]
    assert ok(F, s, kept, _top(order, k + 1), hi)          # one more: first dropped node
    assert ok(F, s, kept, _top(order, k - 1), lo)          # one fewer: last kept node dropped
    assert not ok(F, s, kept, _top(order, k + 1), lo)      # +1 needs mass_hi
    assert not ok(F, s, kept, _top(order, k - 1), hi)      # -1 needs mass_lo
    assert not ok(F, s, kept, _top(order, k + 1), sc)      # a score tie does not resize
    assert not ok(F, s, kept, _top(order, k - 1), sc)
    assert not ok(F, s, kept, _top(order, k + 2), hi + lo)  # never a size change of two
    assert not ok(F, s, kept, _top(order, k - 2), hi + lo)
    assert ok(F, s, kept, _top(order, k + 1), hi + lo + sc)
    assert ok(F, s, kept, _top(order, k - 1), hi + lo + sc)


def check_membership(ok):
    F, s, order = _ten()
    k = 5
    kept = _top(order, k)
    hi = [("mass_hi", 1e-6)]
    # a clearly-above node dropped for the first dropped one: same size, not allowed
    swapped = np.sort(np.r_[order[1:k], order[k]])
    assert not ok(F, s, kept, swapped, hi + [("score", 0.0)])
    # one more, but not the first dropped node
    assert not ok(F, s, kept, np.sort(np.r_[order[:k], order[k + 1]]), hi)
    # one more with a clearly-above node missing
    assert not ok(F, s, kept, np.sort(np.r_[order[1:k], order[k:k + 2]]), hi)
    # a node outside the frontier, a duplicate
    assert not ok(F, s, kept, np.sort(np.r_[order[:k], 99]), hi)
    assert not ok(F, s, kept, np.sort(np.r_[order[:k], order[0]]), hi)


def check_near_tied_swap(ok):
    F, s, order = _ten()
    k = 5
    s = s.astype(np.float64)
    # make the first dropped node (score 5) tie the last kept one (score 6) within the window
    i_last, i_first = np.where(F == order[k - 1])[0][0], np.where(F == order[k])[0][0]
    s[i_first] = s[i_last] - 0.5 * W * s[i_last]
    s = s.astype(np.float32)
    kept = _top(order, k)
    sc = [("score", float(s[i_last]) - float(s[i_first]))]
    swapped = np.sort(np.r_[order[:k - 1], order[k]])
    assert ok(F, s, kept, swapped, sc)
    assert not ok(F, s, kept, swapped, [("mass_hi", 1e-6)])   # a swap needs the score flag
    # swapping in the second dropped node (clearly below) is not a near-tie
    assert not ok(F, s, kept, np.sort(np.r_[order[:k - 1], order[k + 1]]), sc)
    # far from the cut a swap is never allowed
    far = np.sort(np.r_[order[1:k], order[k]])
    assert not ok(F, s, kept, far, sc)


FRAGILE_PINS = [check_sizes_follow_the_kind, check_membership, check_near_tied_swap]


@pytest.mark.parametrize("pin", FRAGILE_PINS, ids=lambda f: f.__name__)
def test_fragile_ok_rule(pin):
    pin(C.fragile_ok)


FRAGILE_MUTANTS = [
    ("+1 allowed for any kind", 'if "mass_hi" in kinds:', "if True:"),
    ("-1 allowed for any kind", 'if "mass_lo" in kinds:', "if True:"),
    ("+1 and -1 tied to the wrong kinds", 'if "mass_hi" in kinds:', 'if "mass_lo" in kinds:'),
    ("size change of two allowed", "sizes.add(k + 1)", "sizes.update((k + 1, k + 2))"),
    ("membership unchecked", "return bool(s64[inG].min() >= s64[~inG].max() - tol)", "return True"),
    ("membership window 1e5 times wider", "s64[~inG].max() - tol)", "s64[~inG].max() - 1e5 * tol)"),
    ("same-size swap without a score tie",
     'if G.size == k and "score" not in kinds and', 'if G.size == k and False and'),
    ("duplicates and foreign nodes accepted",
     "if np.unique(G).size != G.size or not np.all(np.isin(G, F)):", "if False:"),
]


@pytest.mark.parametrize("name,old,new", FRAGILE_MUTANTS, ids=[m[0] for m in FRAGILE_MUTANTS])
def test_fragile_pins_catch_planted_mistakes(name, old, new):
    bad = _mutant(C.fragile_ok, old, new)
    failed = 0
    for pin in FRAGILE_PINS:
        try:
            pin(bad)
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin fails with the planted mistake: {name}"
