"""GPU parity of several queries per sequence at their own positions, causally masked
(zha_attend_causal), against the oracle's reading: the query at position t is the decode
query of a cache holding tokens 0 .. t (its complete top nodes searched, its own tail and
anchor attended, no later token read).

Positions cover a query before the first complete top node (dense), on and next to
top-node boundaries, before the anchor's end, and spread at random; the paths cover the
fused top levels, the narrow and the chunked selections (chunked at the top level too),
the wide tree, the FP4 router and the dense causal comparator.
"""

import zlib

import numpy as np
import pytest
import torch

import gpu_harness as H
import oracle as O
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


def _Z():
    import tree_indexed_sparse_amd as Z
    return Z


def _positions(spec, seed, fixed=()):
    """[B, T] positions: the `fixed` ones first, the rest uniform in [0, N)."""
    rng = np.random.default_rng(seed)
    pos = rng.integers(0, spec["N"], size=(spec["B"], spec["T"]))
    fx = list(fixed)[: spec["T"]]
    for bb in range(spec["B"]):
        pos[bb, : len(fx)] = fx
    return pos.astype(np.int32)


def _check(spec, name, p, anchor, positions, n_tokens=None, **kw):
    res = H.run_gpu(spec, p, anchor=anchor, positions=positions, N=n_tokens, **kw)
    reps, pyr = H.check_units(spec, res, p, anchor=anchor, positions=positions,
                              check_pyramid=False, n_tokens=n_tokens)
    summ = C.summarize(reps)
    print(f"[{name}] {summ}", flush=True)
    H.assert_parity(spec, summ)
    # no head reads a token after its position
    for bb in range(spec["B"]):
        for t in range(spec["T"]):
            for h in range(spec["Hq"]):
                n = int(res["cnt"][bb, t, h])
                assert n <= positions[bb, t] + 1
                if n:
                    assert int(res["sel"][bb, t, h, n - 1]) <= positions[bb, t]
    return res


@pytest.mark.parametrize("case", [
    dict(name="tiny, boundaries", wl="tiny", p=0.95,
         fixed=(0, 62, 63, 64, 127, 128, 2047, 4095)),
    dict(name="tiny p=0.5 random", wl="tiny", p=0.5, fixed=(5,)),
    dict(name="tiny anchor 7", wl="tiny", p=0.9, anchor=7, fixed=(0, 3, 6, 7, 70)),
    dict(name="32k deep 8k, 4 queries", wl="32k_deep", p=0.95, N=8192, B=2, T=4,
         fixed=(8191, 4095, 4096)),
    dict(name="bf16 d=64, 8 queries", wl="32k_deep", p=0.9, N=8192, B=1, Hq=8, Hkv=2, L=4, T=8,
         d=64, fixed=(255, 256, 257)),
    dict(name="64k deep, chunked level 1", wl="32k_deep", p=0.95, N=65536, B=1, T=2,
         fixed=(65535, 40000)),
    # a head with no complete top node shares units with heads that have some: it has no
    # entry at any chunked level (level 1 and 2 here), or none at a chunked top level
    dict(name="64k deep, chunked levels, empty member", wl="32k_deep", p=0.95, N=65536, B=1,
         T=2, fixed=(65535, 3000)),
    dict(name="64k one level, chunked top", wl="32k_deep", p=0.95, N=65536, B=1, L=1, T=2,
         fixed=(65535, 33000)),
    dict(name="64k one level, chunked top, empty member", wl="32k_deep", p=0.9, N=65536, B=1,
         L=1, T=2, fixed=(40000, 2)),
    dict(name="b=3", wl="tiny", p=0.9, N=3 ** 7, b=3, L=4, fixed=(80, 81, 2186)),
    dict(name="wide tree b=256", wl="256k_wide", p=0.95, N=16384, B=1, T=2, fixed=(300, 16383)),
    dict(name="wide tree, head before the first node", wl="256k_wide", p=0.9, N=16384, B=1,
         T=2, fixed=(9000, 100)),
    # 4 x 16 x 8 = 512 query heads: the fused top levels in two workgroups per CU
    dict(name="tiny, 16 queries x 8 heads x 4 sequences", wl="tiny", p=0.9, B=4, T=16, Hq=8,
         Hkv=2, fixed=(4095, 2047, 2048, 63, 64, 0)),
    dict(name="ragged cache of 3000 tokens", wl="tiny", p=0.9, n_tokens=3000,
         fixed=(2999, 1500, 2047, 2048, 63, 64, 0, 2990)),
])
def test_causal_matches_oracle(case):
    case = dict(case)
    name, wl, p = case.pop("name"), case.pop("wl"), case.pop("p")
    anchor = case.pop("anchor", 1)
    fixed = case.pop("fixed", ())
    n_tokens = case.pop("n_tokens", None)
    spec = W.spec(wl, **case)
    pos = _positions(spec, seed=zlib.crc32(name.encode()) % 1000, fixed=fixed)
    if n_tokens is not None:
        pos = np.minimum(pos, n_tokens - 1)
    _check(spec, name, p, anchor, pos, n_tokens=n_tokens)


def test_unit_whose_queries_see_no_complete_top_node():
    """The chunked level-1 path with a unit that searches nothing: sequence 1's two queries
    sit before the first complete top node (4,096 tokens) while sequence 0's reach the
    chunked frontiers, so sequence 1's units keep no node at any level and each of their
    queries attends its whole prefix. The workspace starts filled with a small nonzero
    pattern (every word 5), so a union count or list that the call failed to write would
    show up as extra keys attended."""
    Z = _Z()
    spec = W.spec("32k_deep", N=65536, B=2, T=2)
    pos = np.array([[65535, 40000], [3000, 100]], np.int32)
    inp = W.gen_all(spec, device="cuda")
    tree = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"])
    need = Z.workspace_bytes(tree, spec["T"], spec["Hq"])
    ws = torch.full(((need + 3) // 4,), 5, dtype=torch.int32, device="cuda").view(torch.uint8)
    O_, sel, cnt = Z.attend(inp["Q"], inp["K"], inp["V"], tree, 0.95, 1, workspace=ws,
                            positions=torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    res = dict(tree=tree, O=O_.cpu().numpy(), sel=sel.cpu().numpy(), cnt=cnt.cpu().numpy(),
               lists={l: Z.level_view(tree, spec["T"], spec["Hq"], l, ws)
                      for l in range(1, spec["L"] + 1)}, inputs=inp)
    for t in range(spec["T"]):  # dense over the prefix: every token up to the position
        assert (res["cnt"][1, t] == pos[1, t] + 1).all()
    reps, pyr = H.check_units(spec, res, 0.95, anchor=1, positions=pos)
    summ = C.summarize(reps)
    print(f"[empty unit] pyramid {pyr:.2e}; {summ}", flush=True)
    H.assert_parity(spec, summ, pyr)


def test_causal_fp4_router():
    Z = _Z()
    spec = W.spec("32k_deep", N=8192, B=1, Hq=8, Hkv=2, T=4)
    inp = W.gen_all(spec, device="cuda")
    tree = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"])
    Z.quantize_router(tree)
    Q, R = W.gen_Q(spec), W.gen_R(spec)
    lv = {}
    for g in range(spec["Hkv"]):
        _, _, levels = H.oracle_unit(spec, 0, g, Q, R)
        for l in range(1, spec["L"] + 1):
            Z.pyramid_level(tree, l)[0, g, :levels[l].shape[0]].copy_(torch.from_numpy(levels[l]))
            codes, X = O.mxfp4_quantize(levels[l])
            gc, gs = Z.router_level(tree, l)
            gc[0, g, :codes.shape[0]].copy_(torch.from_numpy(
                (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)))
            gs[0, g, :codes.shape[0]].copy_(torch.from_numpy((X + 127).astype(np.uint8)))
        lv[(0, g)] = levels
    pos = _positions(spec, seed=11, fixed=(8191, 100, 4096))
    res = H.run_gpu(spec, 0.95, inputs=inp, tree=tree, positions=pos)
    reps, _ = H.check_units(spec, res, 0.95, oracle_levels=lv, check_pyramid=False, fp4=True,
                            positions=pos)
    summ = C.summarize(reps)
    print(f"[causal fp4] {summ}", flush=True)
    H.assert_parity(spec, summ)


def test_last_positions_equal_the_decode_entry_point():
    """Every query at N - 1: zha_attend_causal gives zha_attend's selections and counts bit
    for bit, and its outputs up to the order of the split combine (the causal path cuts
    the decode into finer pieces, since its units' work differs)."""
    Z = _Z()
    spec = W.spec("32k_deep", N=16384, B=2, T=2)
    inp = W.gen_all(spec, device="cuda")
    tree = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"])
    pos = torch.full((spec["B"], spec["T"]), spec["N"] - 1, dtype=torch.int32, device="cuda")
    a = Z.attend(inp["Q"], inp["K"], inp["V"], tree, 0.95, 1)
    c = Z.attend(inp["Q"], inp["K"], inp["V"], tree, 0.95, 1, positions=pos)
    torch.cuda.synchronize()
    assert torch.equal(a[2], c[2])
    n = a[2].cpu().numpy()
    sa, sc = a[1].cpu().numpy(), c[1].cpu().numpy()
    for idx in np.ndindex(n.shape):
        assert np.array_equal(sa[idx][: n[idx]], sc[idx][: n[idx]])
    oa, oc = a[0].cpu().numpy(), c[0].cpu().numpy()
    err = float(np.max(np.abs(oa - oc)))
    print(f"[last positions] max |O_decode - O_causal| {err:.2e}", flush=True)
    assert np.allclose(oa, oc, rtol=1e-5, atol=1e-6), err


@pytest.mark.parametrize("wl,kw", [("tiny", {}), ("32k_deep", dict(N=8192, B=2, T=3))])
def test_dense_causal_comparator(wl, kw):
    """zha_dense_attend_causal: exact attention over tokens [0, position] per query."""
    Z = _Z()
    spec = W.spec(wl, **kw)
    inp = W.gen_all(spec, device="cuda")
    pos = _positions(spec, seed=21, fixed=(0, 1, spec["N"] - 1))
    O_ = Z.dense_attend(inp["Q"], inp["K"], inp["V"],
                        positions=torch.from_numpy(pos).cuda()).cpu().numpy()
    Q = W.gen_Q(spec)
    G = spec["Hq"] // spec["Hkv"]
    err = rel = 0.0
    for bb in range(spec["B"]):
        for g in range(spec["Hkv"]):
            K_u, V_u = W.gen_KV_unit(spec, bb, g, Q)
            for t in range(spec["T"]):
                S = np.arange(pos[bb, t] + 1)
                for h in range(g * G, (g + 1) * G):
                    want = O.attention_over(Q[bb, t, h], K_u, V_u, S)
                    e, r = H.output_errors(O_[bb, t, h], want)
                    err, rel = max(err, e), max(rel, r)
    print(f"[dense causal {wl}] max err {err:.2e}, relative {rel:.2e}", flush=True)
    assert err <= O_TOL[spec["dtype"]]
    assert rel <= C.O_REL_TOL


def test_256k_deep_causal_sampled_units():
    """The benchmark cache at full size with four positioned queries per sequence (the
    last token, the middle, inside a top node, before the first complete top node); every
    head of two (sequence, KV head) units is checked."""
    spec = W.spec("256k_deep", T=4)
    pos = np.tile(np.array([262143, 131071, 100001, 4000], np.int32), (spec["B"], 1))
    res = H.run_gpu(spec, 0.95, positions=pos)
    reps, _ = H.check_units(spec, res, 0.95, units=[(0, 0), (3, 3)], positions=pos,
                            check_pyramid=False)
    summ = C.summarize(reps)
    print(f"[256k deep causal sampled] {summ}", flush=True)
    H.assert_parity(spec, summ)
    H.assert_exact_selection(summ)
