"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: selected sets exact at every non-fragile decision (near-ties follow the rule in
oracle/compare.py), token lists exact, O within max-abs 1e-4 (fp32 inputs) or 2e-2 (bf16
inputs, unit-scale V) and within 1e-3 of each head's largest output magnitude, pyramid
within 1e-5 relative to each level's largest magnitude.
"""

import numpy as np
import pytest
import torch

import gpu_harness as H
import workloads as W
from oracle import compare as C

pytestmark = pytest.mark.gpu

O_TOL = H.O_TOL


def _report(name, summ, pyr):
    print(f"[{name}] pyramid {pyr:.2e} {summ}", flush=True)


def _assert_ok(spec, summ, pyr):
    H.assert_parity(spec, summ, pyr)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_indexed_sparse_amd as Z
    Z.load()


@pytest.mark.parametrize("p", [0.95, 0.5, 0.8])
def test_tiny_fp32(p):
    spec = W.spec("tiny")
    res = H.run_gpu(spec, p)
    reps, pyr = H.check_units(spec, res, p)
    summ = C.summarize(reps)
    _report(f"tiny p={p}", summ, pyr)
    _assert_ok(spec, summ, pyr)


def test_tiny_search_on_oracle_pyramid():
    """Feed the oracle's own pyramid, so scores differ only by dot-product rounding."""
    import tree_indexed_sparse_amd as Z

    spec = W.spec("tiny")
    inp = W.gen_all(spec, device="cuda")
    tree = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"])
    _, _, levels = H.oracle_unit(spec, 0, 0)
    for l in range(1, spec["L"] + 1):
        Z.pyramid_level(tree, l)[0, 0].copy_(torch.from_numpy(levels[l]))
    res = H.run_gpu(spec, 0.95, inputs=inp, tree=tree)
    reps, pyr = H.check_units(spec, res, 0.95, oracle_levels={(0, 0): levels})
    summ = C.summarize(reps)
    _report("tiny on oracle pyramid", summ, pyr)
    _assert_ok(spec, summ, pyr)


def test_32k_deep_all_heads():
    spec = W.spec("32k_deep")
    res = H.run_gpu(spec, 0.95)
    reps, pyr = H.check_units(spec, res, 0.95)
    summ = C.summarize(reps)
    _report("32k deep", summ, pyr)
    _assert_ok(spec, summ, pyr)
    H.assert_exact_selection(summ)
    kr = np.array([r.keys for r in reps]) / spec["N"]
    print(f"[32k deep] keys read mean {100 * kr.mean():.1f}%", flush=True)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_p_one_keeps_every_token(dtype, d):
    spec = W.spec("32k_deep", dtype=dtype, d=d, N=4096, B=2, Hq=8, Hkv=2, L=3,
                  r_std=1.0 / np.sqrt(d))
    res = H.run_gpu(spec, 1.0)
    assert np.all(res["cnt"] == spec["N"])
    assert np.array_equal(res["sel"][0, 0, 0], np.arange(spec["N"]))
    reps, pyr = H.check_units(spec, res, 1.0)
    summ = C.summarize(reps)
    _report(f"p=1 {dtype}", summ, pyr)
    _assert_ok(spec, summ, pyr)


@pytest.mark.parametrize("dtype,d,N", [("f32", 64, 4096), ("bf16", 128, 1024)])
def test_one_level_block_n_is_dense(dtype, d, N):
    spec = W.spec("tiny", dtype=dtype, d=d, N=N, b=N, L=1, T=4, needles="none")
    res = H.run_gpu(spec, 0.5)
    assert np.all(res["cnt"] == N)
    reps, pyr = H.check_units(spec, res, 0.5)
    summ = C.summarize(reps)
    _report(f"block=N {dtype}", summ, pyr)
    _assert_ok(spec, summ, pyr)


@pytest.mark.parametrize("p", [0.8, 0.95, 0.99])
def test_wide_tree(p):
    spec = W.spec("256k_wide", N=16384, B=2)
    res = H.run_gpu(spec, p)
    reps, pyr = H.check_units(spec, res, p)
    summ = C.summarize(reps)
    _report(f"wide N=16384 p={p}", summ, pyr)
    _assert_ok(spec, summ, pyr)


@pytest.mark.parametrize("case", [
    dict(name="anchor0", anchor=0),
    dict(name="anchor3", anchor=3),
    dict(name="anchor=b+1", anchor=5),
    dict(name="one top node", N=64, L=3),
    dict(name="T3 G4", T=3, Hq=8, Hkv=2),
    dict(name="T5 G2 two blocks", T=5, Hq=4, Hkv=2),
    dict(name="G16", Hq=16, Hkv=1),
    dict(name="b2 L5", b=2, L=5, N=2048),
    dict(name="b8 L2", b=8, L=2, N=4096),
    dict(name="b3 L4", b=3, L=4, N=81 * 25),
    dict(name="b5 L3", b=5, L=3, N=125 * 20, anchor=7),
    dict(name="sharp pooling", r_std=1.0),
])
def test_edge_cases(case):
    case = dict(case)
    name = case.pop("name")
    anchor = case.pop("anchor", 1)
    spec = W.spec("tiny", **case)
    res = H.run_gpu(spec, 0.9, anchor=anchor)
    reps, pyr = H.check_units(spec, res, 0.9, anchor=anchor)
    summ = C.summarize(reps)
    _report(name, summ, pyr)
    _assert_ok(spec, summ, pyr)


@pytest.mark.parametrize("B,Hkv", [(16, 48), (5, 60)])
def test_many_units_few_decode_splits(B, Hkv):
    """768 (sequence, KV head) units, which get one decode split each, and 300 units, which
    get two: three sampled units against the oracle."""
    spec = W.spec("tiny", B=B, Hkv=Hkv, Hq=Hkv, T=1, N=1024, needles="none")
    res = H.run_gpu(spec, 0.9)
    units = [(0, 0), (B - 1, Hkv - 1), (B // 2, Hkv // 3)]
    reps, pyr = H.check_units(spec, res, 0.9, units=units)
    summ = C.summarize(reps)
    _report(f"{B * Hkv} units", summ, pyr)
    _assert_ok(spec, summ, pyr)


@pytest.mark.parametrize("case", [
    dict(name="f32 d=64 L=6", wl="tiny", N=16384, L=6, T=2),
    dict(name="f32 d=64 L=6, ragged", wl="tiny", N=16384, L=6, T=2, n_tokens=16384 - 1000),
    dict(name="bf16 d=64 L=6", wl="32k_deep", d=64, N=16384, B=1, Hq=8, Hkv=2),
    dict(name="bf16 d=128 L=7", wl="32k_deep", N=32768, B=1, L=7),
])
def test_upper_pyramid_levels(case):
    """Deep trees whose levels above the third are pooled by the float32 wave kernel (three
    fused levels at b = 4): float32 and bf16 reference queries, d = 64 and 128, a cache
    that ends inside a tile, and a seventh level above them."""
    case = dict(case)
    name, wl = case.pop("name"), case.pop("wl")
    n_tokens = case.pop("n_tokens", None)
    spec = W.spec(wl, needles="none", **case)
    res = H.run_gpu(spec, 0.9, N=n_tokens)
    reps, pyr = H.check_units(spec, res, 0.9, n_tokens=n_tokens)
    summ = C.summarize(reps)
    _report(name, summ, pyr)
    _assert_ok(spec, summ, pyr)


@pytest.mark.parametrize("case", [
    dict(name="bf16 b=1024", wl="32k_deep", N=16384, B=1, b=1024, L=1),
    dict(name="bf16 b=300, ragged top", wl="32k_deep", N=300 * 20, B=1, b=300, L=1),
    dict(name="f32 d=64 b=512", wl="tiny", N=8192, b=512, L=1, T=2),
    dict(name="bf16 b=128 L=2", wl="32k_deep", N=32768, B=1, b=128, L=2),
    dict(name="f32 d=64 b=100 L=2", wl="tiny", N=20000, b=100, L=2, T=2),
])
def test_very_wide_nodes(case):
    """Nodes of more than 64 children: one-level trees of 300, 512 and 1024 keys per node
    (the large-node pooling kernel), and two-level trees of 128 and 100 whose second level
    pools float32 rows."""
    case = dict(case)
    name, wl = case.pop("name"), case.pop("wl")
    spec = W.spec(wl, needles="none", **case)
    res = H.run_gpu(spec, 0.9)
    reps, pyr = H.check_units(spec, res, 0.9)
    summ = C.summarize(reps)
    _report(name, summ, pyr)
    _assert_ok(spec, summ, pyr)


def test_bf16_d64_and_multi_sequence():
    spec = W.spec("32k_deep", d=64, N=8192, B=3, Hq=8, Hkv=2, L=4, r_std=0.125)
    res = H.run_gpu(spec, 0.95)
    reps, pyr = H.check_units(spec, res, 0.95)
    summ = C.summarize(reps)
    _report("bf16 d64", summ, pyr)
    _assert_ok(spec, summ, pyr)


@pytest.mark.parametrize("case", [
    dict(name="512 heads, G=16", d=128, N=8192, B=4, Hq=128, Hkv=8, p=0.95),
    dict(name="272 heads (68 units), f32 d=64", wl="tiny", B=17, Hq=16, Hkv=4, T=1, p=0.9),
])
def test_more_heads_than_compute_units(case):
    """More query heads than the GPU has compute units: the fused top levels run two
    half-size workgroups per CU, which must keep exactly the same sets; every head checked."""
    case = dict(case)
    name, p = case.pop("name"), case.pop("p")
    spec = W.spec(case.pop("wl", "32k_deep"), **case)
    res = H.run_gpu(spec, p)
    reps, pyr = H.check_units(spec, res, p)
    summ = C.summarize(reps)
    _report(name, summ, pyr)
    _assert_ok(spec, summ, pyr)


@pytest.mark.parametrize("case", [
    dict(name="64k deep p=0.95", N=65536, p=0.95),
    dict(name="64k deep p=0.5", N=65536, p=0.5),
    dict(name="64k deep p=1", N=65536, p=1.0),
    dict(name="64k b=2, two chunked levels", N=65536, b=2, L=10, p=0.9),
    dict(name="64k one level, chunked top", N=65536, L=1, p=0.95),
    dict(name="96k ragged last chunk, anchor 7", N=98304, p=0.8, anchor=7),
])
def test_chunked_selection(case):
    """Frontiers of 16384 entries or more take the chunked selection (histogram, cut and
    emit launches over frontier chunks); every head of one sequence is checked."""
    case = dict(case)
    name = case.pop("name")
    p = case.pop("p")
    anchor = case.pop("anchor", 1)
    spec = W.spec("32k_deep", B=1, **case)
    res = H.run_gpu(spec, p, anchor=anchor)
    reps, pyr = H.check_units(spec, res, p, anchor=anchor)
    summ = C.summarize(reps)
    _report(name, summ, pyr)
    _assert_ok(spec, summ, pyr)


@pytest.mark.parametrize("case", [
    dict(name="64k deep, 384 heads", N=65536, B=3, Hq=128, Hkv=8, p=0.95),
    dict(name="64k one level, chunked top, 384 heads", N=65536, B=3, Hq=128, Hkv=8, L=1, p=0.9),
])
def test_chunked_selection_more_heads_than_compute_units(case):
    """The chunked selection's cut in half-size workgroups (two buckets per thread), which
    run when the query heads outnumber the CUs; three sampled units (48 heads) checked."""
    case = dict(case)
    name, p = case.pop("name"), case.pop("p")
    spec = W.spec("32k_deep", **case)
    res = H.run_gpu(spec, p)
    reps, pyr = H.check_units(spec, res, p, units=[(0, 0), (2, 7), (1, 3)])
    summ = C.summarize(reps)
    _report(name, summ, pyr)
    _assert_ok(spec, summ, pyr)


@pytest.mark.parametrize("N,T", [(16384, 2), (65536, 2), (65536, 300)])
def test_exact_ties_broken_by_lowest_index(N, T):
    """Identical keys everywhere: every score at every level ties. The cut must keep the
    lowest node ids; the boundary bucket holds N / 4 entries, past the sort capacity
    (at N = 65536 in the chunked selection)."""
    import tree_indexed_sparse_amd as Z

    spec = W.spec("tiny", N=N, b=4, L=1, T=T, needles="none")
    inp = W.gen_all(spec, device="cuda")
    inp["K"][:] = inp["K"][0, 0, 0]
    res = H.run_gpu(spec, 0.95, inputs=inp)
    import oracle as O
    K_u = inp["K"][0, 0].cpu().numpy()
    V_u = inp["V"][0, 0].cpu().numpy()
    levels = O.build_tree_unit(K_u, inp["R"][0].cpu().numpy(), 4, 1)
    for t in sorted({0, 1, T - 1}):
        r = O.attend_head(inp["Q"][0, t, 0].cpu().numpy(), levels, K_u, V_u, 4, 1, 0.95, 1)
        n = int(res["cnt"][0, t, 0])
        assert np.array_equal(res["sel"][0, t, 0, :n], r.S)
        e, rel = H.output_errors(res["O"][0, t, 0], r.O)
        assert e < 1e-4 and rel <= C.O_REL_TOL, (e, rel)
    Z.attend.last_workspace = None


@pytest.mark.parametrize("case", [
    dict(N=16384, L=5, groups=1, p=0.95),     # every score ties at every level
    dict(N=16384, L=5, groups=8, p=0.9),      # 8 distinct keys in runs of 2048 tokens
    dict(N=4096, L=4, groups=64, p=0.8),      # runs of 64 tokens: ties inside each top node
])
def test_exact_ties_in_fused_top_levels(case):
    """Tied scores in the fused top levels (frontiers of at most 1024 entries walked per
    head in one workgroup): boundary buckets both small enough to be sorted in one wave
    and too large for it (the radix fallback); the kept sets take the lowest node ids
    among tied entries, as in the oracle."""
    import tree_indexed_sparse_amd as Z
    import oracle as O

    N, L, groups, p = case["N"], case["L"], case["groups"], case["p"]
    spec = W.spec("tiny", N=N, b=4, L=L, T=2, needles="none")
    inp = W.gen_all(spec, device="cuda")
    K = inp["K"]
    run = N // groups
    K[0, 0] = K[0, 0, ::run].clone().repeat_interleave(run, dim=0)
    res = H.run_gpu(spec, p, inputs=inp)
    K_u = K[0, 0].cpu().numpy()
    V_u = inp["V"][0, 0].cpu().numpy()
    levels = O.build_tree_unit(K_u, inp["R"][0].cpu().numpy(), 4, L)
    for t in range(2):
        r = O.attend_head(inp["Q"][0, t, 0].cpu().numpy(), levels, K_u, V_u, 4, L, p, 1)
        n = int(res["cnt"][0, t, 0])
        print(f"[ties in top levels {case}] t={t} kept {n} tokens, oracle {len(r.S)}", flush=True)
        assert n == len(r.S), (t, n, len(r.S))
        assert np.array_equal(res["sel"][0, t, 0, :n], r.S)
        e, rel = H.output_errors(res["O"][0, t, 0], r.O)
        assert e < 1e-4 and rel <= C.O_REL_TOL, (e, rel)
    Z.attend.last_workspace = None


@pytest.mark.parametrize("run,T", [(2048, 2), (2048, 300), (4096, 300), (16384, 300)])
def test_tied_groups_in_chunked_selection(run, T):
    """Keys repeat in runs of `run` tokens (run / 4 nodes), so the 16384-node top frontier
    (chunked selection) has 65536 / run distinct scores, each shared by run / 4 nodes: the
    cut falls inside a tied group and must keep its lowest node ids, a count taken from the
    mass. Groups of 512, 1024 and 4096 nodes put the boundary bucket in each of the exact
    cut's paths; 300 queries (more than the CUs) run the half-size cut workgroups, and a
    sample of them is checked."""
    import tree_indexed_sparse_amd as Z
    import oracle as O

    spec = W.spec("tiny", N=65536, b=4, L=1, T=T, needles="none")
    inp = W.gen_all(spec, device="cuda")
    K = inp["K"]
    groups = K[0, 0, ::run].clone()
    K[0, 0] = groups.repeat_interleave(run, dim=0)
    for p in (0.5, 0.9):
        res = H.run_gpu(spec, p, inputs=inp)
        K_u = K[0, 0].cpu().numpy()
        V_u = inp["V"][0, 0].cpu().numpy()
        levels = O.build_tree_unit(K_u, inp["R"][0].cpu().numpy(), 4, 1)
        for t in sorted({0, 1, T // 2, T - 1}):
            r = O.attend_head(inp["Q"][0, t, 0].cpu().numpy(), levels, K_u, V_u, 4, 1, p, 1)
            n = int(res["cnt"][0, t, 0])
            assert n == len(r.S), (p, t, n, len(r.S))
            assert np.array_equal(res["sel"][0, t, 0, :n], r.S)
            e, rel = H.output_errors(res["O"][0, t, 0], r.O)
            assert e < 1e-4 and rel <= C.O_REL_TOL, (e, rel)
    Z.attend.last_workspace = None


def test_deterministic_repeat():
    spec = W.spec("32k_deep", N=8192, B=2)
    inp = W.gen_all(spec, device="cuda")
    a = H.run_gpu(spec, 0.95, inputs=inp)
    b = H.run_gpu(spec, 0.95, inputs=inp, tree=a["tree"])
    assert np.array_equal(a["cnt"], b["cnt"])
    assert np.array_equal(a["sel"], b["sel"])
    assert np.array_equal(a["O"], b["O"])


def test_append_equals_one_shot_build():
    import tree_indexed_sparse_amd as Z

    spec = W.spec("32k_deep", N=16384, B=2)
    inp = W.gen_all(spec, device="cuda")
    full = Z.build_tree(inp["K"], inp["R"], 4, 6)
    part = Z.build_tree(inp["K"], inp["R"], 4, 6, N=4096)
    for _ in range(3):
        Z.tree_append(part, inp["K"], inp["R"], 4096)
    torch.cuda.synchronize()
    assert part.N == full.N == 16384
    for l in range(1, 7):
        assert torch.equal(Z.pyramid_level(part, l), Z.pyramid_level(full, l))


def test_256k_deep_every_unit():
    """The benchmark workload at full size, in the benchmark's launch configuration: every
    (sequence, KV head) unit, i.e. all 128 query heads, against the oracle."""
    spec = W.spec("256k_deep")
    res = H.run_gpu(spec, 0.95)
    reps, pyr = H.check_units(spec, res, 0.95)
    summ = C.summarize(reps)
    _report("256k deep, every unit", summ, pyr)
    assert summ["heads"] == spec["B"] * spec["Hq"]
    _assert_ok(spec, summ, pyr)
    # every head has a decision inside the near-tie windows here; none resolves differently
    H.assert_exact_selection(summ)


def test_256k_deep_agreeing_heads_sampled_units():
    """The 256K deep workload's keys with queries whose heads agree and whose scores are
    sharp (about 2% of the keys read per head, 7% per KV head): small frontiers at every
    level, a short union list for the decode; every head of three units."""
    spec = W.spec("256k_deep_agree")
    res = H.run_gpu(spec, 0.95)
    reps, pyr = H.check_units(spec, res, 0.95, units=[(0, 0), (1, 2), (3, 3)])
    summ = C.summarize(reps)
    _report("256k deep agreeing heads, sampled", summ, pyr)
    _assert_ok(spec, summ, pyr)
    H.assert_exact_selection(summ)
    kr = np.array([r.keys for r in reps]) / spec["N"]
    print(f"[256k deep agreeing heads] keys read mean {100 * kr.mean():.2f}%", flush=True)


@pytest.mark.parametrize("b,L,N", [(2, 12, 65536), (4, 8, 131072), (16, 4, 131072)])
def test_sweep_geometries(b, L, N):
    """Tree geometries of the geometry sweep beyond the two the benchmark runs: binary
    trees of the maximum depth (b = 2, L = 12, 4,096 tokens per top node), and top nodes
    of 65,536 tokens as 8 levels of 4 or 4 levels of 16; the benchmark's key distribution,
    two sequences, two sampled units."""
    spec = W.spec("256k_deep", N=N, B=2, b=b, L=L)
    res = H.run_gpu(spec, 0.95)
    reps, pyr = H.check_units(spec, res, 0.95, units=[(0, 0), (1, 3)])
    summ = C.summarize(reps)
    _report(f"b={b} L={L} N={N}", summ, pyr)
    _assert_ok(spec, summ, pyr)


def test_graph_replay_matches_eager():
    """The whole step (pyramid build + attend) captured as a HIP graph: three replays, with
    eager library work and synchronisation between them, each equal bit for bit to the
    eager result."""
    import ctypes
    import tree_indexed_sparse_amd as Z
    from tree_indexed_sparse_amd import _lib as LB

    spec = W.spec("32k_deep", N=65536, B=2)
    inp = W.gen_all(spec, device="cuda")
    K, V, Q, R = inp["K"], inp["V"], inp["Q"], inp["R"]
    B, T, Hq, Hkv, d, N, b, L = (spec[k] for k in ("B", "T", "Hq", "Hkv", "d", "N", "b", "L"))
    lib = Z.load()
    tree = Z.build_tree(K, R, b, L)
    O = torch.empty((B, T, Hq, d), dtype=torch.float32, device="cuda")
    sel = torch.full((B, T, Hq, N), -1, dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, T, Hq), dtype=torch.int32, device="cuda")
    ws = torch.empty(Z.workspace_bytes(tree, T, Hq), dtype=torch.uint8, device="cuda")
    c_tree = tree.c

    def step():
        LB.check(lib.zha_build_tree(K.data_ptr(), R.data_ptr(), c_tree.dtype, B, Hkv, N, N, d, b,
                                    L, tree.storage.data_ptr(), tree.storage.numel(),
                                    ctypes.byref(c_tree), torch.cuda.current_stream().cuda_stream))
        Z.attend(Q, K, V, tree, 0.95, 1, out=O, sel_idx=sel, sel_count=cnt, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = (O.clone(), sel.clone(), cnt.clone(), tree.storage.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        # eager work in between: a different p into the same buffers, then garbage
        Z.attend(Q, K, V, tree, 0.5, 1, out=O, sel_idx=sel, sel_count=cnt, workspace=ws)
        O.fill_(float("nan"))
        cnt.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(tree.storage, ref[3]), i
        assert torch.equal(cnt, ref[2]), i
        assert torch.equal(O, ref[0]), i
        n = cnt.cpu().numpy()
        s_now, s_ref = sel.cpu().numpy(), ref[1].cpu().numpy()
        for idx in np.ndindex(*n.shape):
            assert np.array_equal(s_now[idx][:n[idx]], s_ref[idx][:n[idx]]), (i, idx)
    Z.attend.last_workspace = None


@pytest.mark.parametrize("case", [
    dict(name="tiny fp32, N not a multiple of any tile", wl="tiny", N=4000, N_cap=4096),
    dict(name="32k bf16 G8", wl="32k_deep", B=2),
    dict(name="bf16 d64, T3 G4", wl="32k_deep", B=1, d=64, T=3, Hq=8, Hkv=2, N=8192),
])
def test_dense_comparator(case):
    """zha_dense_attend: every query head attends over all N keys of its KV head."""
    import tree_indexed_sparse_amd as Z
    import oracle as O

    case = dict(case)
    name = case.pop("name")
    wl = case.pop("wl")
    N_cap = case.pop("N_cap", None)
    spec = W.spec(wl, **case)
    if N_cap is not None:
        spec["N"] = N_cap
    inp = W.gen_all(spec, device="cuda")
    N = case.get("N", spec["N"])
    out = Z.dense_attend(inp["Q"], inp["K"], inp["V"], N)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    Q = inp["Q"].float().cpu().numpy()
    K = inp["K"].float().cpu().numpy()
    V = inp["V"].float().cpu().numpy()
    G = spec["Hq"] // spec["Hkv"]
    err = rel = 0.0
    S = np.arange(N)
    for b in range(spec["B"]):
        for t in range(spec["T"]):
            for h in range(spec["Hq"]):
                ref = O.attention_over(Q[b, t, h], K[b, h // G], V[b, h // G], S)
                e, r = H.output_errors(got[b, t, h], ref)
                err, rel = max(err, e), max(rel, r)
    print(f"[dense {name}] max |O - oracle| {err:.2e}, relative {rel:.2e}", flush=True)
    assert err <= O_TOL[spec["dtype"]], err
    assert rel <= C.O_REL_TOL, rel


@pytest.mark.parametrize("p", [0.8, 0.95, 0.99])
def test_256k_wide_sampled_units(p):
    """The wide tree (b = 256, L = 1) at full size, as the benchmark runs it; one unit of
    every sequence."""
    spec = W.spec("256k_wide")
    res = H.run_gpu(spec, p)
    reps, pyr = H.check_units(spec, res, p, units=[(0, 2), (1, 0), (2, 3), (3, 1)])
    summ = C.summarize(reps)
    _report(f"256k wide sampled p={p}", summ, pyr)
    _assert_ok(spec, summ, pyr)
    H.assert_exact_selection(summ)


def test_1m_deep_sampled_units():
    """1M keys, b = 4, L = 7, B = 8 (the benchmark's launch configuration); one unit of
    every sequence, every KV head among them."""
    spec = W.spec("1m_deep")
    res = H.run_gpu(spec, 0.95)
    reps, pyr = H.check_units(spec, res, 0.95, units=[(bb, (3 * bb) % 4) for bb in range(8)])
    summ = C.summarize(reps)
    _report("1m deep sampled", summ, pyr)
    _assert_ok(spec, summ, pyr)


@pytest.mark.parametrize("case", [
    dict(name="32k + 1 token", extra=1),
    dict(name="32k + 77 tokens, anchor 5", extra=77, anchor=5),
    dict(name="32k + 4095 tokens", extra=4095),
    dict(name="below one top node (N = 3000)", total=3000),
    dict(name="tiny fp32 + 13 tokens", wl="tiny", extra=13),
])
def test_ragged_cache(case):
    """Caches that do not fill whole top nodes: the search runs over the complete top nodes
    and the tail after them is attended by every head."""
    wl = case.get("wl", "32k_deep")
    kw = {"B": 1} if wl == "32k_deep" else {}
    base = W.spec(wl, **kw)
    top = base["b"] ** base["L"]
    N = case.get("total", base["N"] + case.get("extra", 0))
    anchor = case.get("anchor", 1)
    spec = W.spec(wl, N=-(-N // top) * top, **kw)
    res = H.run_gpu(spec, 0.9, anchor=anchor, N=N)
    assert int(res["tree"].N) == N
    reps, pyr = H.check_units(spec, res, 0.9, anchor=anchor, n_tokens=N)
    summ = C.summarize(reps)
    _report(f"ragged {case['name']}", summ, pyr)
    _assert_ok(spec, summ, pyr)


def test_token_by_token_appends_match_one_shot_build():
    """Appends of one token at a time (then chunks of assorted sizes, across top-node
    boundaries) write the pyramid a one-shot build over the same tokens writes, bit for
    bit; the attend over the appended tree matches the oracle."""
    import tree_indexed_sparse_amd as Z

    spec = W.spec("32k_deep", B=2, N=16384)
    inp = W.gen_all(spec, device="cuda")
    K, R = inp["K"], inp["R"]
    n = 8192 - 37
    tree = Z.build_tree(K, R, 4, 6, N=n)
    for k in [1] * 300 + [5, 64, 1000, 3, 4097]:
        Z.tree_append(tree, K, R, k)
        n += k
    torch.cuda.synchronize()
    assert tree.N == n
    one = Z.build_tree(K, R, 4, 6, N=n)
    torch.cuda.synchronize()
    for l in range(1, 7):
        valid = n // 4 ** l
        assert torch.equal(Z.pyramid_level(tree, l)[:, :, :valid],
                           Z.pyramid_level(one, l)[:, :, :valid]), l
    res = H.run_gpu(spec, 0.95, inputs=inp, tree=tree)
    reps, pyr = H.check_units(spec, res, 0.95, units=[(1, 2)], n_tokens=n)
    summ = C.summarize(reps)
    _report(f"appended to N={n}", summ, pyr)
    _assert_ok(spec, summ, pyr)


def test_sweep_retained_mass_matches_the_oracle():
    """The geometry sweep's measurement on every geometry it runs (the benchmark's key
    distribution, 65,536 tokens): the share of dense attention weight on each head's
    selected keys, as the sweep computes it on the GPU, against the oracle's float64 value
    for the same keys; and the selections of one unit against the oracle."""
    import bench
    import oracle as O
    import tree_indexed_sparse_amd as Z

    spec0 = W.spec("256k_deep", N=65536, B=1)
    inp = W.gen_all(spec0, device="cuda")
    wts = bench.dense_weights(inp["Q"], inp["K"])
    Q = W.gen_Q(spec0)
    K_u, V_u = W.gen_KV_unit(spec0, 0, 0, Q)
    G = spec0["Hq"] // spec0["Hkv"]
    lam = O.sigma(spec0["d"]) * (K_u.astype(np.float64) @ Q[0, 0, :G].astype(np.float64).T)
    w64 = np.exp(lam - lam.max(0))
    w64 /= w64.sum(0)                                   # [N, G] dense weights, float64
    for (b, L) in bench.SWEEP_GEOMETRIES:
        spec = W.spec("256k_deep", N=65536, B=1, b=b, L=L)
        if spec["N"] % (b ** L):
            continue
        tree = Z.build_tree(inp["K"], inp["R"], b, L)
        res = H.run_gpu(spec, 0.95, inputs=inp, tree=tree)
        mass = bench.selected_mass(wts, torch.from_numpy(res["sel"]).cuda(),
                                   torch.from_numpy(res["cnt"]).cuda()).cpu().numpy()
        err = 0.0
        for h in range(G):
            S = res["sel"][0, 0, h, :res["cnt"][0, 0, h]]
            err = max(err, abs(float(mass[h]) - float(w64[S, h].sum())))
        reps, pyr = H.check_units(spec, res, 0.95, units=[(0, 0)])
        summ = C.summarize(reps)
        _report(f"sweep b={b} L={L}: retained-mass error {err:.1e}", summ, pyr)
        assert err <= 1e-4, (b, L, err)
        _assert_ok(spec, summ, pyr)
        Z.attend.last_workspace = None
