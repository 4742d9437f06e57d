"""GPU parity of the FP4 router (MXFP4 summaries and query, OCP Microscaling Formats v1.0)
against the oracle's reading: quantise the float32 summaries and the query, score, select.

* The encoder is bit-exact: the library's MXFP4 copy of a float32 pyramid equals the
  oracle's encoding of the same float32 values, code for code and scale for scale
  (the oracle's pyramid loaded into the GPU tree, and crafted rows with ties, zeros,
  signed zeros, subnormals and scales at both ends of the range).
* The FP4 search is exact at every non-fragile decision (oracle/compare.py's rule) when it
  scores the oracle's own MXFP4 codes, loaded into the tree's router copy.
* On its own pyramid the GPU's codes differ from the oracle's only where the two float32
  pyramids (equal within 1e-5 of each level's largest magnitude) straddle a rounding
  threshold or a power of two.
* Appends encode exactly the nodes they complete: token by token equals one-shot.
"""

import numpy as np
import pytest
import torch

import gpu_harness as H
import oracle as O
import workloads as W
from oracle import compare as C

pytestmark = pytest.mark.gpu

O_TOL = H.O_TOL
PYR_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_indexed_sparse_amd as Z
    Z.load()


def _Z():
    import tree_indexed_sparse_amd as Z
    return Z


def _unpack(codes: np.ndarray) -> np.ndarray:
    """[..., d/2] bytes -> [..., d] E2M1 codes (element 2i in the low nibble)."""
    codes = np.asarray(codes, np.uint8)
    out = np.empty(codes.shape[:-1] + (2 * codes.shape[-1],), np.uint8)
    out[..., 0::2] = codes & 15
    out[..., 1::2] = codes >> 4
    return out


def _pack(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def _gpu_router(tree, b, g, l, n):
    codes, scales = _Z().router_level(tree, l)
    return _unpack(codes[b, g, :n].cpu().numpy()), scales[b, g, :n].cpu().numpy()


def _load_oracle_pyramid(spec, tree, units):
    """Overwrite the tree's float32 pyramid for `units` with the oracle's pyramid."""
    Q, R = W.gen_Q(spec), W.gen_R(spec)
    out = {}
    for (b, g) in units:
        _, _, levels = H.oracle_unit(spec, b, g, Q, R)
        for l in range(1, spec["L"] + 1):
            n = levels[l].shape[0]
            _Z().pyramid_level(tree, l)[b, g, :n].copy_(torch.from_numpy(levels[l]))
        out[(b, g)] = levels
    return out


def _load_oracle_router(tree, units_levels):
    """Write the oracle's MXFP4 encoding of its pyramid into the tree's router copy."""
    for (b, g), levels in units_levels.items():
        for l in range(1, len(levels)):
            codes, X = O.mxfp4_quantize(levels[l])
            n = codes.shape[0]
            gc, gs = _Z().router_level(tree, l)
            gc[b, g, :n].copy_(torch.from_numpy(_pack(codes)))
            gs[b, g, :n].copy_(torch.from_numpy((X.astype(np.int64) + 127).astype(np.uint8)))


def _summ_ok(spec, name, reps):
    summ = C.summarize(reps)
    print(f"[{name}] {summ}", flush=True)
    H.assert_parity(spec, summ)
    return summ


@pytest.mark.parametrize("wl,kw", [
    ("tiny", {}),
    ("32k_deep", dict(N=8192, B=2, Hq=8, Hkv=2, L=4)),
    ("32k_deep", dict(N=8192, B=1, Hq=8, Hkv=2, L=4, d=64)),
])
def test_encoder_is_bit_exact_on_the_oracle_pyramid(wl, kw):
    Z = _Z()
    spec = W.spec(wl, **kw)
    inp = W.gen_all(spec, device="cuda")
    tree = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"])
    units = [(b, g) for b in range(spec["B"]) for g in range(spec["Hkv"])]
    lv = _load_oracle_pyramid(spec, tree, units)
    Z.quantize_router(tree)
    torch.cuda.synchronize()
    total = 0
    for (b, g), levels in lv.items():
        for l in range(1, spec["L"] + 1):
            want_c, want_X = O.mxfp4_quantize(levels[l])
            got_c, got_s = _gpu_router(tree, b, g, l, levels[l].shape[0])
            np.testing.assert_array_equal(got_s.astype(np.int64) - 127, want_X)
            np.testing.assert_array_equal(got_c, want_c)
            total += want_c.size
    print(f"[encoder {wl} {kw}] {total} codes equal", flush=True)


def _crafted_rows(n, d, seed):
    """float32 rows that reach every branch of the encoding: exact ties between E2M1
    neighbours, values past the clamp, zeros, negative zeros, subnormals, block maxima at
    and just below powers of two, and magnitudes from 2^-140 to 2^120."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((n, d)) * np.exp2(rng.integers(-140, 120, (n, 1)))).astype(np.float32)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 5.5, 0.1])
    for i in range(0, n, 7):                     # tie rows: one block max of 6 * 2^k
        k = int(rng.integers(-120, 110))
        row = rng.choice(ties, d) * rng.choice([-1.0, 1.0], d)
        row[::32] = 6.0
        x[i] = (row * 2.0 ** k).astype(np.float32)
    x[3] = 0.0
    x[5] = -0.0
    x[9, : d // 2] = -0.0
    x[11] = (rng.integers(-2 ** 20, 2 ** 20, d) * 2.0 ** -149).astype(np.float32)   # subnormal
    x[13] = (rng.uniform(-1.5, 1.5, d) * 2.0 ** -126).astype(np.float32)  # around the smallest normal
    x[15, ::32] = 2.0 ** 10                      # block max exactly a power of two
    x[17, ::32] = np.nextafter(np.float32(2.0 ** 10), np.float32(0))   # just below it
    x[19, ::32] = np.float32(3.0e38)             # the largest exponents a float holds
    return x


@pytest.mark.parametrize("d", [64, 128])
def test_encoder_special_values(d):
    Z = _Z()
    spec = W.spec("tiny", d=d, dtype="f32", needles="none")
    inp = W.gen_all(spec, device="cuda")
    tree = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"])
    lvl = Z.pyramid_level(tree, 1)
    n = lvl.shape[2]
    x = _crafted_rows(n, d, seed=80 + d)
    lvl[0, 0].copy_(torch.from_numpy(x))
    Z.quantize_router(tree)
    torch.cuda.synchronize()
    want_c, want_X = O.mxfp4_quantize(x)
    got_c, got_s = _gpu_router(tree, 0, 0, 1, n)
    np.testing.assert_array_equal(got_s.astype(np.int64) - 127, want_X)
    np.testing.assert_array_equal(got_c, want_c)


@pytest.mark.parametrize("case", [
    dict(name="tiny p=0.95", wl="tiny", p=0.95),
    dict(name="tiny p=0.5", wl="tiny", p=0.5),
    dict(name="32k deep, 8k", wl="32k_deep", N=8192, B=2, p=0.95),
    dict(name="bf16 d=64", wl="32k_deep", N=8192, B=1, Hq=8, Hkv=2, L=4, d=64, p=0.9),
    dict(name="64k deep, chunked level 1", wl="32k_deep", N=65536, B=1, p=0.95),
    dict(name="b=3", wl="tiny", N=3 ** 7, b=3, L=4, p=0.9),
    dict(name="wide tree b=256", wl="256k_wide", N=16384, B=1, p=0.95),
    # more query heads than CUs: the fused top levels in two half-size workgroups per CU
    dict(name="512 heads, G=16", wl="32k_deep", N=8192, B=4, Hq=128, Hkv=8, p=0.95),
])
def test_fp4_search_on_the_oracle_router(case):
    """The tree's router copy holds the oracle's MXFP4 codes of the oracle's pyramid, so
    the FP4 scores differ from the oracle's only by the float32 accumulation order."""
    Z = _Z()
    case = dict(case)
    name, wl, p = case.pop("name"), case.pop("wl"), case.pop("p")
    spec = W.spec(wl, **case)
    inp = W.gen_all(spec, device="cuda")
    tree = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"])
    Z.quantize_router(tree)                     # allocates the copy and selects it
    units = [(b, g) for b in range(spec["B"]) for g in range(spec["Hkv"])]
    lv = _load_oracle_pyramid(spec, tree, units)
    _load_oracle_router(tree, lv)
    res = H.run_gpu(spec, p, inputs=inp, tree=tree)
    reps, _ = H.check_units(spec, res, p, oracle_levels=lv, check_pyramid=False, fp4=True)
    _summ_ok(spec, f"fp4 {name}", reps)


def test_fp4_and_f32_routers_switch_on_one_tree():
    """set_router flips which copy the search scores; each matches its own oracle."""
    Z = _Z()
    spec = W.spec("tiny")
    inp = W.gen_all(spec, device="cuda")
    tree = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"])
    Z.quantize_router(tree)
    lv = _load_oracle_pyramid(spec, tree, [(0, 0)])
    _load_oracle_router(tree, lv)
    for router, fp4 in (("mxfp4", True), ("f32", False), ("mxfp4", True)):
        Z.set_router(tree, router)
        res = H.run_gpu(spec, 0.9, inputs=inp, tree=tree)
        reps, _ = H.check_units(spec, res, 0.9, oracle_levels=lv, check_pyramid=False, fp4=fp4)
        _summ_ok(spec, f"switch {router}", reps)


def _thresholds():
    mags = [O.e2m1_value(c) for c in range(8)]
    return np.array([(a + b) / 2 for a, b in zip(mags[:-1], mags[1:])])


def test_gpu_pyramid_codes_differ_only_at_rounding_boundaries():
    """GPU pyramid -> GPU encoder against oracle pyramid -> oracle encoder. A code may
    differ only where the oracle's value lies within the pyramid tolerance of a rounding
    threshold, and a block's scale only where its largest magnitude lies that close to a
    power of two (then the whole block may differ)."""
    Z = _Z()
    spec = W.spec("32k_deep", N=16384, B=1, Hq=8, Hkv=2)
    inp = W.gen_all(spec, device="cuda")
    tree = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"])
    Z.quantize_router(tree)
    torch.cuda.synchronize()
    Q, R = W.gen_Q(spec), W.gen_R(spec)
    th = _thresholds()
    n_codes = n_diff = 0
    for g in range(spec["Hkv"]):
        _, _, levels = H.oracle_unit(spec, 0, g, Q, R)
        for l in range(1, spec["L"] + 1):
            x = levels[l].astype(np.float64)
            n, d = x.shape
            eps = PYR_TOL * np.abs(x).max()
            want_c, want_X = O.mxfp4_quantize(levels[l])
            got_c, got_s = _gpu_router(tree, 0, g, l, n)
            got_X = got_s.astype(np.int64) - 127
            blocks = np.abs(x).reshape(n, d // 32, 32)
            amax = blocks.max(axis=2)
            p2 = np.exp2(np.round(np.log2(np.maximum(amax, 1e-300))))
            block_fragile = np.abs(amax - p2) <= eps
            assert np.all((got_X == want_X) | block_fragile), f"level {l}: scale differs"
            unit = np.repeat(np.exp2(want_X.astype(np.float64)), 32, axis=1)
            dist = np.min(np.abs(np.abs(x)[..., None] - th * unit[..., None]), axis=-1)
            elem_fragile = (dist <= eps) | np.repeat(block_fragile, 32, axis=1)
            diff = got_c != want_c
            assert not np.any(diff & ~elem_fragile), f"level {l}: code differs off a boundary"
            n_codes += diff.size
            n_diff += int(diff.sum())
    print(f"[gpu pyramid codes] {n_diff} of {n_codes} codes differ, all at boundaries",
          flush=True)
    assert n_diff <= 1e-3 * n_codes


def test_appends_encode_the_nodes_they_complete():
    """A router copy made on an empty tree and kept up to date by appends of 1, 3 and 64
    tokens equals the one-shot encoding of the one-shot pyramid, bit for bit."""
    Z = _Z()
    spec = W.spec("32k_deep", N=4096, B=2, Hq=8, Hkv=2, L=3)
    inp = W.gen_all(spec, device="cuda")
    full = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"])
    Z.quantize_router(full)
    part = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"], N=0)
    Z.quantize_router(part)
    n, steps = 0, [1, 3, 64, 1, 1, 200]
    i = 0
    while n < spec["N"]:
        k = min(steps[i % len(steps)], spec["N"] - n)
        Z.tree_append(part, inp["K"], inp["R"], k)
        n += k
        i += 1
    torch.cuda.synchronize()
    for l in range(1, spec["L"] + 1):
        a_c, a_s = Z.router_level(full, l)
        b_c, b_s = Z.router_level(part, l)
        assert torch.equal(a_c, b_c) and torch.equal(a_s, b_s), f"level {l}"
    # the copy follows a ragged cache too: encode a prefix, then append the rest
    mid = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"], N=1001)
    Z.quantize_router(mid)
    Z.tree_append(mid, inp["K"], inp["R"], spec["N"] - 1001)
    torch.cuda.synchronize()
    for l in range(1, spec["L"] + 1):
        a_c, a_s = Z.router_level(full, l)
        m_c, m_s = Z.router_level(mid, l)
        assert torch.equal(a_c, m_c) and torch.equal(a_s, m_s), f"level {l}"


@pytest.mark.parametrize("wl,kw", [
    ("32k_deep", dict(N=16384, B=2, Hq=8, Hkv=2)),           # bf16 b = 4: pooling encodes
    ("32k_deep", dict(N=8192, B=1, Hq=8, Hkv=2, L=4, d=64)),
    ("tiny", {}),                                            # fp32: the encoder pass
    ("32k_deep", dict(N=4096, B=1, Hq=8, Hkv=2, L=3, b=8)),  # b = 8: the encoder pass
])
def test_build_with_router_equals_encoding_the_built_pyramid(wl, kw):
    """build_tree(router=True) (pooling launches that write the MXFP4 rows themselves,
    the encoder for the levels they do not cover) equals the standalone encoder run over
    the one-shot pyramid, bit for bit, and both pyramids are equal."""
    Z = _Z()
    spec = W.spec(wl, **kw)
    inp = W.gen_all(spec, device="cuda")
    a = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"], router=True)
    ref = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"])
    Z.quantize_router(ref)
    torch.cuda.synchronize()
    assert a.c.router == ref.c.router == 1
    for l in range(1, spec["L"] + 1):
        assert torch.equal(Z.pyramid_level(a, l), Z.pyramid_level(ref, l)), f"pyramid level {l}"
        x_c, x_s = Z.router_level(a, l)
        y_c, y_s = Z.router_level(ref, l)
        assert torch.equal(x_c, y_c) and torch.equal(x_s, y_s), f"router level {l}"


def test_256k_deep_fp4_sampled_units():
    """The benchmark workload at full size with the FP4 router: two (sequence, KV head)
    units carry the oracle's pyramid and MXFP4 codes; every head of them is checked."""
    Z = _Z()
    spec = W.spec("256k_deep")
    inp = W.gen_all(spec, device="cuda")
    tree = Z.build_tree(inp["K"], inp["R"], spec["b"], spec["L"])
    Z.quantize_router(tree)
    lv = _load_oracle_pyramid(spec, tree, [(0, 0), (3, 3)])
    _load_oracle_router(tree, lv)
    res = H.run_gpu(spec, 0.95, inputs=inp, tree=tree)
    reps, _ = H.check_units(spec, res, 0.95, units=[(0, 0), (3, 3)], oracle_levels=lv,
                            check_pyramid=False, fp4=True)
    H.assert_exact_selection(_summ_ok(spec, "256k deep fp4 sampled", reps))
