"""Pins of the CPU oracle against facts it does not derive from itself:
library routines (torch SDPA, scipy), closed forms, brute force on tiny trees,
and the geometries printed on the pages (tests/golden/geometries.txt).

All CPU; no GPU, no HIP library.
"""

import itertools
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "geometries.txt")


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa(q, K, V, mask=None):
    """Independent dense reference: torch's scaled_dot_product_attention in fp64."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None, None, :]
    Kt = torch.from_numpy(np.asarray(K, np.float64))[None, None]
    Vt = torch.from_numpy(np.asarray(V, np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=m)[0, 0, 0].numpy()


def _golden_geometries():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, b, L, top, *_ = line.split()
        rows.append((name, int(b), int(L), int(top)))
    return rows


# --------------------------------------------------------------------------- build

def test_pool_zero_reference_queries_gives_subtree_mean():
    rng = _rng(0)
    N, d, b, L = 256, 16, 4, 3
    K = rng.standard_normal((N, d)).astype(np.float32)
    lv = O.build_tree_unit(K, np.zeros((16, d), np.float32), b, L)
    for l in range(1, L + 1):
        want = K.astype(np.float64).reshape(N // b ** l, b ** l, d).mean(axis=1)
        np.testing.assert_allclose(lv[l], want, rtol=2e-6, atol=2e-6)


def test_pool_identical_children_is_that_child():
    rng = _rng(1)
    x = rng.standard_normal(32).astype(np.float32)
    R = rng.standard_normal((16, 32)).astype(np.float32)
    K = np.tile(x, (16, 1))
    lv = O.build_tree_unit(K, R, 4, 2)
    assert np.array_equal(lv[1], np.tile(x, (4, 1)))
    assert np.array_equal(lv[2], x[None, :])


def test_pool_sharp_softmax_picks_argmax_child_per_reference_query():
    # All 16 reference queries along +u with a huge norm: each one's softmax over
    # the children is one-hot on the child with the largest u-projection.
    rng = _rng(2)
    d, b = 8, 4
    u = np.zeros(d); u[0] = 1.0
    X = rng.standard_normal((b, d))
    X[:, 0] = [0.1, 0.7, -0.3, 0.2]
    R = np.tile(1e4 * u, (16, 1))
    out = O.pool(X[None], R, O.sigma(d))[0]
    np.testing.assert_allclose(out, X[1], atol=1e-12)


def test_pool_averages_the_sixteen_reference_queries():
    # Half the reference queries pick the child with the largest u-projection,
    # the other half the smallest: the summary is the midpoint of the two.
    rng = _rng(3)
    d, b = 8, 4
    u = np.zeros(d); u[0] = 1.0
    X = rng.standard_normal((b, d))
    X[:, 0] = [0.1, 0.7, -0.3, 0.2]
    R = np.concatenate([np.tile(1e4 * u, (8, 1)), np.tile(-1e4 * u, (8, 1))])
    out = O.pool(X[None], R, O.sigma(d))[0]
    np.testing.assert_allclose(out, 0.5 * (X[1] + X[2]), atol=1e-12)


def test_pool_two_children_closed_form_with_scale():
    # b = 2: w0 = mean_r sigmoid(tau * R_r . (x0 - x1)), tau = 1/sqrt(d).
    rng = _rng(4)
    d = 32
    X = rng.standard_normal((2, d))
    R = rng.standard_normal((16, d))
    w0 = scipy.special.expit((R @ (X[0] - X[1])) / np.sqrt(d)).mean()
    want = w0 * X[0] + (1 - w0) * X[1]
    np.testing.assert_allclose(O.pool(X[None], R, O.sigma(d))[0], want, rtol=1e-12, atol=1e-12)


def test_pool_permutation_invariant_and_convex():
    rng = _rng(5)
    d, b = 16, 8
    X = rng.standard_normal((b, d))
    R = 3 * rng.standard_normal((16, d))
    a = O.pool(X[None], R, O.sigma(d))[0]
    perm = rng.permutation(b)
    np.testing.assert_allclose(O.pool(X[perm][None], R, O.sigma(d))[0], a, atol=1e-12)
    assert np.linalg.norm(a) <= np.linalg.norm(X, axis=1).max() + 1e-12
    # the summary lies in the convex hull: recover weights by least squares
    w, *_ = np.linalg.lstsq(np.vstack([X.T, np.ones(b)]), np.append(a, 1.0), rcond=None)
    assert w.min() > -1e-9 and abs(w.sum() - 1) < 1e-9


@pytest.mark.parametrize("name,b,L,top", _golden_geometries())
def test_top_node_depends_on_exactly_its_b_to_the_L_tokens(name, b, L, top):
    assert b ** L == top
    rng = _rng(6)
    d = 4
    N = 3 * top
    K = rng.standard_normal((N, d)).astype(np.float32)
    R = rng.standard_normal((16, d)).astype(np.float32)
    base = O.build_tree_unit(K, R, b, L)[L]
    assert base.shape == (3, d)
    for tok in (top - 1, top, 2 * top - 1, 2 * top):
        K2 = K.copy()
        K2[tok] += 1.0
        new = O.build_tree_unit(K2, R, b, L)[L]
        changed = np.nonzero(np.any(new != base, axis=1))[0].tolist()
        assert changed == [tok // top]


# --------------------------------------------------------------------------- search

def test_node_scores_are_scaled_dot_products():
    rng = _rng(7)
    X = rng.standard_normal((50, 64)).astype(np.float32)
    q = rng.standard_normal(64).astype(np.float32)
    want = np.array([np.dot(x.astype(np.float64), q.astype(np.float64)) for x in X]) / 8.0
    np.testing.assert_allclose(O.node_scores(X, q), want, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("target,expect", [(0.94, [0, 1]), (0.96, [0])])
def test_score_scale_decides_the_cut(target, expect):
    # Two top nodes (b = 2, L = 1). Node 0's children are both a*e0, node 1's
    # children are 0. Mass of node 0 = sigmoid(sigma * a * q0); choose a so it
    # equals `target` (scipy's logit), with p = 0.95.
    d = 16
    q = np.zeros(d, np.float32); q[0] = 2.0
    a = scipy.special.logit(target) * np.sqrt(d) / 2.0
    K = np.zeros((4, d), np.float32)
    K[0, 0] = K[1, 0] = a
    levels = O.build_tree_unit(K, np.zeros((16, d), np.float32), 2, 1)
    S, dec = O.search(q, levels, 2, 1, 0.95, anchor=0)
    assert dec[0].kept.tolist() == expect


@pytest.mark.parametrize("p,k", [(0.5, 2), (0.75, 3), (0.25, 1), (0.76, 4), (1.0, 4)])
def test_cut_is_cumulative_mass_at_least_p_with_low_index_first(p, k):
    # four equal scores: masses 1/4 each; ">= p" and ascending-id tie-break
    F = np.arange(4)
    kept, _ = O.select_top_p(F, np.zeros(4, np.float32), np.float32(p))
    assert kept.tolist() == list(range(k))


def test_near_ties_are_logged():
    F = np.arange(3)
    _, frag = O.select_top_p(F, np.array([1.0, 0.5, 0.5], np.float32), 0.7)
    kinds = [k for k, _ in frag]
    assert "score" in kinds


def _bruteforce_min_set(m, p):
    """Every subset of the frontier: minimum cardinality with mass >= p, and the
    largest mass among subsets of that cardinality."""
    n = m.size
    bits = ((np.arange(2 ** n)[:, None] >> np.arange(n)[None, :]) & 1).astype(np.float64)
    mass = bits @ m
    card = bits.sum(1)
    ok = mass >= p
    k = int(card[ok].min())
    best = mass[ok & (card == k)].max()
    return k, best


@pytest.mark.parametrize("N,b,L,d,seed", [(64, 4, 2, 8, 0), (128, 2, 4, 8, 1), (64, 4, 2, 8, 2),
                                          (128, 2, 4, 6, 3), (256, 4, 3, 8, 4)])
@pytest.mark.parametrize("p", [0.5, 0.8, 0.95])
def test_selection_is_a_minimum_set_by_brute_force(N, b, L, d, seed, p):
    rng = _rng(100 + seed)
    K = (rng.standard_normal((N // 8, d))[np.arange(N) // 8] + 0.5 * rng.standard_normal((N, d))).astype(np.float32)
    R = rng.standard_normal((16, d)).astype(np.float32)
    levels = O.build_tree_unit(K, R, b, L)
    checked = 0
    for trial in range(6):
        q = (3 * rng.standard_normal(d)).astype(np.float32)
        _, decs = O.search(q, levels, b, L, p, anchor=1)
        for dec in decs:
            if dec.frontier.size > 16 or dec.fragile:
                continue
            # masses from the float32 scores, independently via scipy's softmax
            m = scipy.special.softmax(dec.scores.astype(np.float64))
            k, best = _bruteforce_min_set(m, float(np.float32(p)))
            pos = np.searchsorted(dec.frontier, dec.kept)
            assert dec.kept.size == k
            assert abs(m[pos].sum() - best) < 1e-12
            assert m[pos].sum() >= np.float32(p) - 1e-15
            checked += 1
    assert checked > 0


def test_frontier_is_the_children_of_kept_nodes_renormalised():
    # the level-l frontier is exactly the children of the level-(l+1) kept set
    rng = _rng(9)
    N, b, L, d = 1024, 4, 4, 8
    K = rng.standard_normal((N, d)).astype(np.float32)
    levels = O.build_tree_unit(K, rng.standard_normal((16, d)).astype(np.float32), b, L)
    q = (2 * rng.standard_normal(d)).astype(np.float32)
    _, decs = O.search(q, levels, b, L, 0.8, anchor=1)
    for up, down in zip(decs[:-1], decs[1:]):
        want = sorted(c * b + i for c in up.kept.tolist() for i in range(b))
        assert down.frontier.tolist() == want
        # masses over each frontier sum to one: the kept mass alone reaches p
        m = scipy.special.softmax(down.scores.astype(np.float64))
        assert m[np.searchsorted(down.frontier, down.kept)].sum() >= np.float32(0.8)


def _hot_path_keys(N, d, b, L, leaf, scale):
    """Zero keys except the b tokens of level-1 node `leaf`, set to scale * e0."""
    K = np.zeros((N, d), np.float32)
    K[leaf * b:(leaf + 1) * b, 0] = scale
    return K


@pytest.mark.parametrize("name,b,L,top", _golden_geometries() + [("tiny", 4, 3, 64), ("deep7", 4, 7, 16384)])
def test_descent_follows_the_one_hot_branch(name, b, L, top):
    # Mean pooling (R = 0): a node's summary is scale * e0 * (b / b^l) if it
    # contains the hot leaf and 0 otherwise. A large scale makes the hot node the
    # only one kept at every level, so S is the hot leaf's b tokens plus token 0.
    d = 8
    N = 2 * top
    q = np.zeros(d, np.float32); q[0] = 1.0
    scale = np.float32(64.0 * np.sqrt(d) * b ** (L - 1))
    for leaf in sorted({N // b - 1, (N // b) // 2 + 1 if N // b > 2 else 1, 0}):
        K = _hot_path_keys(N, d, b, L, leaf, scale)
        levels = O.build_tree_unit(K, np.zeros((16, d), np.float32), b, L)
        S, decs = O.search(q, levels, b, L, 0.95, anchor=1)
        for dec in decs:
            assert dec.kept.tolist() == [leaf // b ** (dec.level - 1)]
        want = sorted(set(range(leaf * b, (leaf + 1) * b)) | {0})
        assert S.tolist() == want
        # the hot top node covers exactly b^L tokens
        assert (leaf * b) // top == decs[0].kept[0]


# --------------------------------------------------------------------------- attention

def test_p_equal_one_is_dense_attention():
    rng = _rng(10)
    N, d, b, L = 256, 16, 4, 2
    K = rng.standard_normal((N, d)).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    R = rng.standard_normal((16, d)).astype(np.float32)
    levels = O.build_tree_unit(K, R, b, L)
    for _ in range(4):
        q = rng.standard_normal(d).astype(np.float32)
        r = O.attend_head(q, levels, K, V, b, L, 1.0, anchor=1)
        assert r.S.tolist() == list(range(N))
        np.testing.assert_allclose(r.O, _sdpa(q, K, V), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("N", [64, 256, 4096])
@pytest.mark.parametrize("p", [0.1, 0.5, 0.95])
def test_one_level_tree_with_block_n_is_dense(N, p):
    rng = _rng(11)
    d = 64
    K = rng.standard_normal((N, d)).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    R = rng.standard_normal((16, d)).astype(np.float32) / 8
    levels = O.build_tree_unit(K, R, N, 1)
    q = rng.standard_normal(d).astype(np.float32)
    r = O.attend_head(q, levels, K, V, N, 1, p, anchor=1)
    assert r.S.tolist() == list(range(N))
    np.testing.assert_allclose(r.O, _sdpa(q, K, V), rtol=1e-12, atol=1e-12)


def test_anchor_token_zero_always_kept_and_attended():
    import workloads as W

    s = W.spec("tiny")
    Q = W.gen_Q(s)
    R = W.gen_R(s)
    K, V = W.gen_KV_unit(s, 0, 0, Q)
    levels = O.build_tree_unit(K, R[0], s["b"], s["L"])
    for t in range(s["T"]):
        r = O.attend_head(Q[0, t, 0], levels, K, V, s["b"], s["L"], 0.95, anchor=1)
        assert r.S[0] == 0 and np.all(np.diff(r.S) > 0)
        mask = np.zeros(s["N"], bool)
        mask[r.S] = True
        np.testing.assert_allclose(r.O, _sdpa(Q[0, t, 0], K, V, mask), rtol=1e-10, atol=1e-12)


def test_anchor_is_added_after_selection_without_duplicates():
    d, b, L = 8, 4, 2
    N = 64
    q = np.zeros(d, np.float32); q[0] = 1.0
    scale = np.float32(64.0 * np.sqrt(d) * b)
    K = _hot_path_keys(N, d, b, L, 5, scale)
    levels = O.build_tree_unit(K, np.zeros((16, d), np.float32), b, L)
    assert O.search(q, levels, b, L, 0.95, anchor=1)[0].tolist() == [0, 20, 21, 22, 23]
    assert O.search(q, levels, b, L, 0.95, anchor=0)[0].tolist() == [20, 21, 22, 23]
    assert O.search(q, levels, b, L, 0.95, anchor=3)[0].tolist() == [0, 1, 2, 20, 21, 22, 23]
    K = _hot_path_keys(N, d, b, L, 0, scale)
    levels = O.build_tree_unit(K, np.zeros((16, d), np.float32), b, L)
    assert O.search(q, levels, b, L, 0.95, anchor=1)[0].tolist() == [0, 1, 2, 3]


def test_attention_over_a_subset_matches_masked_sdpa():
    rng = _rng(12)
    N, d = 300, 32
    K = rng.standard_normal((N, d)).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    S = np.sort(rng.choice(N, 77, replace=False))
    mask = np.zeros(N, bool)
    mask[S] = True
    np.testing.assert_allclose(O.attention_over(q, K, V, S), _sdpa(q, K, V, mask), rtol=1e-12, atol=1e-12)


def test_workload_recipe_shapes_and_needles():
    import workloads as W

    s = W.spec("tiny")
    Q = W.gen_Q(s)
    K, V = W.gen_KV_unit(s, 0, 0, Q)
    assert K.shape == (s["N"], s["d"]) and V.shape == K.shape
    plan = W.needle_plan(s, 0)
    assert len(plan) == 3 and all(pos > 0 for pos, _, _ in plan)
    for pos, t, h in plan:
        q = Q[0, t, h].astype(np.float64)
        np.testing.assert_allclose(K[pos], 4 * q / np.linalg.norm(q), rtol=1e-6)
    s2 = W.spec("256k_deep", N=4096, B=2)
    plan = W.needle_plan(s2, 1)
    assert len(plan) == 16 and len({h for _, _, h in plan}) == 8
    K2, _ = W.gen_KV_unit(W.spec("32k_deep", N=1024, B=1), 0, 1)
    assert K2.dtype == np.float32
    import torch
    assert torch.equal(torch.from_numpy(K2).to(torch.bfloat16).float(), torch.from_numpy(K2))


def test_agreeing_query_recipe():
    """The agreeing-heads variant of the query recipe: the default draws are untouched;
    q = scale (sqrt(1 - rho^2) eps + rho u) with u shared by the G heads of a KV head, so
    heads of one group correlate at about rho^2, heads of different groups not at all, and
    every coordinate has variance scale^2."""
    import workloads as W

    base = W.spec("256k_deep", N=4096, B=3, T=2)
    Q0 = W.gen_Q(base)
    assert np.array_equal(Q0, W.gen_Q(dict(base, q_shared=0.0, q_scale=1.0)))
    s = dict(base, q_shared=0.9, q_scale=3.0, dtype="f32")
    Q = W.gen_Q(s).astype(np.float64)
    G = s["Hq"] // s["Hkv"]
    same, other = [], []
    for b in range(s["B"]):
        for t in range(s["T"]):
            for h in range(s["Hq"]):
                for h2 in range(h + 1, s["Hq"]):
                    c = np.corrcoef(Q[b, t, h], Q[b, t, h2])[0, 1]
                    (same if h // G == h2 // G else other).append(c)
    assert abs(np.mean(same) - 0.81) < 0.03 and abs(np.mean(other)) < 0.03
    assert abs(Q.std() - 3.0) < 0.05
    # the named workload carries the recipe and the 256K deep keys and values
    a = W.spec("256k_deep_agree")
    assert (a["q_shared"], a["q_scale"], a["seed"], a["N"]) == (0.9, 3.0, 3, 262144)


def test_agreeing_heads_select_few_keys_and_a_small_union():
    """What the agreeing-heads workload is for, on one (sequence, KV head) unit of 64K
    tokens through the oracle: its heads each read a few percent of the keys and their
    union stays small, where the independent heads of the same cache read ~40% each and
    almost all of it together (the 256K workloads measure 2.0% / 7.0% and 41% / 98.5%)."""
    import workloads as W

    def shares(name):
        s = W.spec(name, N=65536, B=1)
        Q, R = W.gen_Q(s), W.gen_R(s)
        K, V = W.gen_KV_unit(s, 0, 1, Q)
        lv = O.build_tree_unit(K, R[1], s["b"], s["L"])
        sets = [O.search(Q[0, 0, h], lv, s["b"], s["L"], 0.95, 1)[0] for h in range(8, 16)]
        per_head = np.array([x.size for x in sets]) / s["N"]
        return per_head, np.unique(np.concatenate(sets)).size / s["N"]

    agree, agree_union = shares("256k_deep_agree")
    indep, indep_union = shares("256k_deep")
    assert agree.max() < 0.06 and agree_union < 0.15
    assert indep.min() > 0.30 and indep_union > 0.90


# ------------------------------------------------------------- ragged caches (tail)

@pytest.mark.parametrize("b,L", [(4, 3), (2, 5), (8, 2)])
def test_complete_nodes_do_not_change_when_tokens_are_appended(b, L):
    """A node depends only on the tokens under it: the pyramid of a shorter cache is a
    bit-identical prefix of the pyramid of a longer one, at every level."""
    rng = _rng(20)
    d = 16
    top = b ** L
    K = rng.standard_normal((3 * top + top // 2 + 3, d)).astype(np.float32)
    R = rng.standard_normal((16, d)).astype(np.float32)
    full = O.build_tree_unit(K, R, b, L)
    for n in (1, b - 1, b, top - 1, top, top + 1, 2 * top + b + 1, K.shape[0]):
        part = O.build_tree_unit(K[:n], R, b, L)
        for l in range(1, L + 1):
            assert part[l].shape[0] == n // b ** l
            assert np.array_equal(part[l], full[l][:n // b ** l])


@pytest.mark.parametrize("r", [1, 3, 17, 63])
def test_ragged_cache_searches_complete_top_nodes_and_attends_the_tail(r):
    """N = (whole top nodes) + r: the decisions are those of the complete part, and the
    tail [N_full, N) is added to every head's set; O is masked SDPA over that set."""
    import workloads as W

    s = W.spec("tiny")
    Q = W.gen_Q(s)
    R = W.gen_R(s)
    K, V = W.gen_KV_unit(s, 0, 0, Q)
    b, L, top = s["b"], s["L"], s["b"] ** s["L"]
    N_full = 40 * top
    N = N_full + r
    lv_full = O.build_tree_unit(K[:N_full], R[0], b, L)
    lv = O.build_tree_unit(K[:N], R[0], b, L)
    for t in range(s["T"]):
        S_f, dec_f = O.search(Q[0, t, 0], lv_full, b, L, 0.9, 1)
        S, dec = O.search(Q[0, t, 0], lv, b, L, 0.9, 1)
        assert [d.kept.tolist() for d in dec] == [d.kept.tolist() for d in dec_f]
        assert S.tolist() == S_f.tolist() + list(range(N_full, N))
        res = O.attend_head(Q[0, t, 0], lv, K[:N], V[:N], b, L, 0.9, 1)
        mask = np.zeros(N, bool)
        mask[S] = True
        np.testing.assert_allclose(res.O, _sdpa(Q[0, t, 0], K[:N], V[:N], mask),
                                   rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("N,L", [(1, 3), (5, 3), (63, 3), (4095, 6)])
def test_no_complete_top_node_is_dense_attention(N, L):
    """Below one top node (b^L tokens) there is nothing to search: every token is the tail."""
    rng = _rng(21)
    d, b = 16, 4
    K = rng.standard_normal((N, d)).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    R = rng.standard_normal((16, d)).astype(np.float32)
    levels = O.build_tree_unit(K, R, b, L)
    q = rng.standard_normal(d).astype(np.float32)
    r = O.attend_head(q, levels, K, V, b, L, 0.5, anchor=1)
    assert r.S.tolist() == list(range(N)) and r.levels == []
    np.testing.assert_allclose(r.O, _sdpa(q, K, V), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# FP4 router: MXFP4 encoding (OCP Microscaling Formats v1.0), pinned to the
# specification's stated properties and to numpy's IEEE round-half-even.
# ---------------------------------------------------------------------------

MX_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_mx.txt")


def _mx_facts():
    out = {}
    for line in open(MX_GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        k, v = line.split()
        out[k] = float(v)
    return out


def test_e2m1_values_match_the_specification():
    f = _mx_facts()
    vals = [O.e2m1_value(c) for c in range(16)]
    mags = sorted(set(abs(v) for v in vals))
    assert len(mags) == 8 and mags[0] == 0.0
    assert max(mags) == f["e2m1_max_normal"]
    normals = [O.e2m1_value(c) for c in range(8) if (c >> 1) & 3]
    subnormals = [O.e2m1_value(c) for c in range(8) if not (c >> 1) & 3 and c & 1]
    assert min(normals) == f["e2m1_min_normal"]
    assert subnormals == [f["e2m1_max_subnormal"]] == [f["e2m1_min_subnormal"]]
    assert np.log2(f["e2m1_max_normal"] / 1.5) == f["e2m1_emax"]
    for c in range(8):   # sign bit mirrors every magnitude
        assert O.e2m1_value(c | 8) == -O.e2m1_value(c)
    assert O.MX_BLOCK == f["mx_block_size"]


def _rne_binade(a):
    """E2M1 rounding of magnitudes a (already scaled) by numpy's round-half-even on each
    binade's uniform grid: spacing 0.5 below 2, 1 in [2, 4), 2 in [4, 8); clamp to 6."""
    r = np.where(a < 2, np.rint(a * 2) / 2, np.where(a < 4, np.rint(a), 2 * np.rint(a / 2)))
    return np.minimum(r, 6.0)


def test_e2m1_rounding_is_round_half_even():
    rng = _rng(71)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0])
    a = np.concatenate([ties, rng.uniform(0, 7.99, 4000), np.arange(0, 8, 0.125)])
    a = a[: (a.size // 32) * 32]
    # one element of 6 per block fixes the scale at 2^0 whatever the others are
    blocks = a.reshape(-1, 32).copy()
    blocks[:, 0] = 6.0
    codes, X = O.mxfp4_quantize(blocks.astype(np.float32))
    assert np.all(X == 0)
    got = np.abs(O.mxfp4_dequantize(codes, X))
    np.testing.assert_array_equal(got, _rne_binade(blocks.astype(np.float32).astype(np.float64)))


def test_mxfp4_shared_scale():
    f = _mx_facts()
    lo, hi = int(f["e8m0_min_exponent"]), int(f["e8m0_max_exponent"])
    emax = int(f["e2m1_emax"])
    for k in (-20, -3, 0, 1, 7, 30):
        for m in (1.0, 1.5, 1.999):
            x = np.zeros((1, 32), np.float32)
            x[0, 5] = -m * 2.0 ** k
            x[0, 9] = 0.3 * 2.0 ** k
            _, X = O.mxfp4_quantize(x)
            assert int(X[0, 0]) == k - emax
    _, X = O.mxfp4_quantize(np.zeros((1, 32), np.float32))
    assert int(X[0, 0]) == lo
    # float32 stays below 2^128, so the upper clamp is never reached: X <= 125
    big = np.full((1, 32), 2.0 ** 127, np.float32)
    codes, X = O.mxfp4_quantize(big)
    assert int(X[0, 0]) == 127 - emax < hi
    assert np.all(O.mxfp4_dequantize(codes, X) == 2.0 ** 127)
    tiny = np.full((1, 32), 2.0 ** -140, np.float32)
    _, X = O.mxfp4_quantize(tiny)
    assert int(X[0, 0]) == lo


def test_mxfp4_round_trip_of_representable_blocks():
    rng = _rng(72)
    codes = rng.integers(0, 16, size=(200, 128)).astype(np.uint8)
    codes[:, ::32] = rng.choice([6, 7, 14, 15], size=(200, 4))   # a magnitude of 4 or 6
    X = rng.integers(-40, 40, size=(200, 4)).astype(np.int16)
    x = O.mxfp4_dequantize(codes, X)
    assert np.all(x.astype(np.float32).astype(np.float64) == x)
    c2, X2 = O.mxfp4_quantize(x.astype(np.float32))
    np.testing.assert_array_equal(X2, X)
    np.testing.assert_array_equal(c2, codes)


def test_mxfp4_error_bound_and_sign_symmetry():
    rng = _rng(73)
    x = (rng.standard_normal((300, 64)) * np.exp(rng.uniform(-8, 8, (300, 1)))).astype(np.float32)
    codes, X = O.mxfp4_quantize(x)
    deq = O.mxfp4_dequantize(codes, X)
    unit = np.repeat(np.ldexp(1.0, X.astype(np.int64)), 32, axis=1)
    err = np.abs(deq - x.astype(np.float64))
    scaled = np.abs(x.astype(np.float64)) / unit
    # half the grid spacing of the element's binade; the clamp above 6 costs at most 2
    half = np.where(scaled < 2, 0.25, np.where(scaled < 4, 0.5, 1.0))
    assert np.all(err[scaled <= 6] <= half[scaled <= 6] * unit[scaled <= 6])
    assert np.all(err <= 2 * unit)
    amax = np.repeat(np.abs(x).reshape(300, 2, 32).max(axis=2), 32, axis=1)
    assert np.all(err <= amax / 4 + 1e-300)
    cn, Xn = O.mxfp4_quantize(-x)
    np.testing.assert_array_equal(Xn, X)
    np.testing.assert_array_equal(cn, codes ^ 8)


def test_fp4_router_search_reduces_to_the_float_search_on_representable_inputs():
    """When the query and every summary row are already MXFP4 values, quantising changes
    nothing, so the FP4-router descent must be the float32-router descent."""
    rng = _rng(74)
    b, L, d = 4, 3, 64
    N = 2 * b ** L
    K = rng.standard_normal((N, d)).astype(np.float32)
    levels = [K]
    for l in range(1, L + 1):
        n = N // b ** l
        c = rng.integers(0, 16, size=(n, d)).astype(np.uint8)
        Xs = rng.integers(-6, 2, size=(n, d // 32)).astype(np.int16)
        levels.append(O.mxfp4_dequantize(c, Xs).astype(np.float32))
    for t in range(20):
        cq = rng.integers(0, 16, size=(1, d)).astype(np.uint8)
        q = O.mxfp4_dequantize(cq, np.zeros((1, d // 32), np.int16))[0].astype(np.float32)
        S_f, dec_f = O.search(q, levels, b, L, 0.9, 1)
        S_4, dec_4 = O.search_fp4(q, levels, b, L, 0.9, 1)
        np.testing.assert_array_equal(S_f, S_4)
        for a, c in zip(dec_f, dec_4):
            np.testing.assert_array_equal(a.scores, c.scores)


def test_fp4_router_quantises_the_router_only():
    """The FP4 descent scores quantised rows with a quantised query, and the final
    attention is exact over the keys it selects with the unquantised query."""
    rng = _rng(75)
    b, L, d, N = 4, 2, 64, 256
    K = rng.standard_normal((N, d)).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    R = (rng.standard_normal((16, d)) / np.sqrt(d)).astype(np.float32)
    levels = O.build_tree_unit(K, R, b, L)
    q = rng.standard_normal(d).astype(np.float32)
    res = O.attend_head_fp4(q, levels, K, V, b, L, 0.9, 1)
    mask = np.zeros(N, bool)
    mask[res.S] = True
    np.testing.assert_allclose(res.O, _sdpa(q, K, V, mask), rtol=1e-12, atol=1e-12)
    top = res.levels[0]
    want = O.node_scores(O.mxfp4_round_trip(levels[L]), O.mxfp4_round_trip(q))
    np.testing.assert_array_equal(top.scores, want)


# ---------------------------------------------------------------------------
# Causal multi-query: a query at position t sees tokens 0 .. t only.
# ---------------------------------------------------------------------------

def _causal_unit(seed, N=512, d=32, b=4, L=3):
    rng = _rng(seed)
    K = rng.standard_normal((N, d)).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    R = (rng.standard_normal((16, d)) / np.sqrt(d)).astype(np.float32)
    return rng, K, V, R, O.build_tree_unit(K, R, b, L)


def test_causal_p_one_is_causally_masked_sdpa():
    rng, K, V, R, levels = _causal_unit(90)
    for pos in (0, 1, 5, 63, 64, 200, 511):
        q = rng.standard_normal(K.shape[1]).astype(np.float32)
        res = O.attend_head_causal(q, levels, K, V, 4, 3, 1.0, 1, pos)
        mask = np.arange(K.shape[0]) <= pos
        np.testing.assert_allclose(res.O, _sdpa(q, K, V, mask), rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(res.S, np.arange(pos + 1))


def test_causal_result_does_not_depend_on_later_tokens():
    """Rewriting every key and value after the query's position (and so the pyramid
    nodes over them) changes nothing the query selects or outputs."""
    rng, K, V, R, levels = _causal_unit(91)
    for pos in (70, 130, 300, 448):
        K2, V2 = K.copy(), V.copy()
        K2[pos + 1:] = rng.standard_normal(K2[pos + 1:].shape).astype(np.float32) * 3
        V2[pos + 1:] = rng.standard_normal(V2[pos + 1:].shape).astype(np.float32)
        levels2 = O.build_tree_unit(K2, R, 4, 3)
        q = rng.standard_normal(K.shape[1]).astype(np.float32)
        a = O.attend_head_causal(q, levels, K, V, 4, 3, 0.9, 1, pos)
        c = O.attend_head_causal(q, levels2, K2, V2, 4, 3, 0.9, 1, pos)
        np.testing.assert_array_equal(a.S, c.S)
        np.testing.assert_array_equal(a.O, c.O)


def test_causal_last_position_is_the_decode_query():
    rng, K, V, R, levels = _causal_unit(92)
    q = rng.standard_normal(K.shape[1]).astype(np.float32)
    a = O.attend_head_causal(q, levels, K, V, 4, 3, 0.9, 1, K.shape[0] - 1)
    c = O.attend_head(q, levels, K, V, 4, 3, 0.9, 1)
    np.testing.assert_array_equal(a.S, c.S)
    np.testing.assert_array_equal(a.O, c.O)


def test_causal_selection_structure():
    """Tokens selected: never past the position; the anchor and the query's own tail
    (after its last complete top node, 64 tokens here) always; a position before the first
    complete top node attends densely."""
    rng, K, V, R, levels = _causal_unit(93)
    for pos in range(0, 512, 7):
        q = rng.standard_normal(K.shape[1]).astype(np.float32)
        res = O.attend_head_causal(q, levels, K, V, 4, 3, 0.8, 2, pos)
        assert res.S.max() <= pos and np.all(np.diff(res.S) > 0)
        assert set(range(min(2, pos + 1))) <= set(res.S.tolist())
        full = (pos + 1) // 64 * 64
        assert set(range(max(full, 2), pos + 1)) <= set(res.S.tolist())
        if pos < 63:
            np.testing.assert_array_equal(res.S, np.arange(pos + 1))
