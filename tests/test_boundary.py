"""The C-ABI library without a GPU: it loads, exports every declared entry point, and
rejects bad arguments on the host before enqueueing anything."""

import ctypes
import math
import os
import re

import pytest

from abi_views import lay_out
from tree_indexed_sparse_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zha.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation
ODD8 = ctypes.c_void_p(0x1008)  # 8- but not 16-byte aligned
ODD16 = ctypes.c_void_p(0x1010)  # 16- but not 256-byte aligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libzha.so not built")
    return L.load()


def test_every_declared_function_is_exported(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(zha_[a-z_]+)\s*\(", text))
    assert declared == set(L.EXPORTS)
    for name in declared:
        assert hasattr(lib, name)


def test_tree_bytes_closed_form(lib):
    # levels of B*Hkv*(N/b^l)*d float32, each rounded up to 256 bytes
    def want(B, H, N, d, b, Ll):
        tot = 0
        for l in range(1, Ll + 1):
            tot += 4 * B * H * (N // b ** l) * d
            tot = (tot + 255) // 256 * 256
        return tot
    assert lib.zha_tree_bytes(4, 4, 262144, 128, 4, 6) == want(4, 4, 262144, 128, 4, 6)
    assert lib.zha_tree_bytes(1, 1, 4096, 64, 4, 3) == want(1, 1, 4096, 64, 4, 3)
    assert lib.zha_tree_bytes(4, 4, 262144, 128, 256, 1) == 4 * 16 * 1024 * 128
    assert lib.zha_tree_bytes(1, 1, 4096, 96, 4, 3) == 0      # d unsupported
    assert lib.zha_tree_bytes(1, 1, 4000, 64, 4, 3) == 0      # not a multiple of b^L
    assert lib.zha_tree_bytes(1, 1, 4096, 64, 1, 3) == 0      # b < 2


@pytest.mark.parametrize("b,Ll,n_cap", [(65536, 4, 65536), (1024, 12, 1 << 20),
                                        (2 ** 31 - 1, 2, 4096), (46341, 2, 4096),
                                        (7, 12, 7 ** 11)])
def test_geometry_with_b_pow_L_past_2_pow_31_is_an_error(lib, b, Ll, n_cap):
    # b^L wraps 64 bits for the first two (65536^4 = 2^64): the check must stop the power
    # at 2^31 instead of dividing by a wrapped zero
    assert lib.zha_tree_bytes(1, 1, n_cap, 64, b, Ll) == 0
    assert lib.zha_router_bytes(1, 1, n_cap, 64, b, Ll) == 0
    assert _build(lib, N=0, N_cap=n_cap, b=b, L=Ll) == -2
    assert "exceeds 2^31" in lib.zha_last_error().decode()
    assert _attend(lib, t=_tree(N=0, N_cap=n_cap, b=b, L=Ll)) == -2


def test_geometry_with_b_pow_L_just_inside_passes_the_power_check(lib):
    # b^L = 2^30 tokens per top node is accepted; 2^32 is not
    assert lib.zha_tree_bytes(1, 1, 2 ** 30, 64, 2 ** 15, 2) > 0
    assert lib.zha_tree_bytes(1, 1, 2 ** 30, 64, 2 ** 16, 2) == 0


def _build(lib, **kw):
    a = dict(K=FAKE, R=FAKE, dtype=1, B=1, Hkv=1, N=4096, N_cap=4096, d=64, b=4, L=3,
             pyr=FAKE, nbytes=1 << 30)
    a.update(kw)
    t = L.ZhaTree()
    return lib.zha_build_tree(a["K"], a["R"], a["dtype"], a["B"], a["Hkv"], a["N"], a["N_cap"],
                              a["d"], a["b"], a["L"], a["pyr"], a["nbytes"], ctypes.byref(t), None)


@pytest.mark.parametrize("kw,code", [
    (dict(K=None), -1), (dict(R=None), -1), (dict(pyr=None), -1),
    (dict(dtype=7), -3), (dict(d=96), -5), (dict(b=1), -1), (dict(L=0), -1), (dict(L=13), -5),
    (dict(N_cap=4000, N=0), -2), (dict(N=8192), -2), (dict(nbytes=1024), -2),
    (dict(B=0), -2), (dict(N_cap=4 * 2 ** 22, N=64, b=4, L=3), -5),
    (dict(K=ODD8), -1), (dict(R=ODD8), -1), (dict(pyr=ODD8), -1),
])
def test_build_rejects_bad_arguments(lib, kw, code):
    assert _build(lib, **kw) == code
    assert len(lib.zha_last_error()) > 0


def _tree(**kw):
    t = L.ZhaTree()
    a = dict(B=1, Hkv=2, N=4096, N_cap=4096, d=64, b=4, L=3, dtype=1)
    a.update(kw)
    for k, v in a.items():
        setattr(t, k, v)
    t.pyramid = 0x2000
    return lay_out(L.load(), t)


def _attend(lib, t=None, **kw):
    t = _tree() if t is None else t
    a = dict(Q=FAKE, T=1, Hq=8, K=FAKE, V=FAKE, p=0.95, anchor=1, O=FAKE, sel=FAKE, cap=4096,
             cnt=FAKE, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return lib.zha_attend(ctypes.byref(t), a["Q"], a["T"], a["Hq"], a["K"], a["V"], a["p"],
                          a["anchor"], a["O"], a["sel"], a["cap"], a["cnt"], a["ws"], a["wsb"],
                          None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), -1), (dict(K=None), -1), (dict(V=None), -1), (dict(O=None), -1),
    (dict(cnt=None), -1), (dict(ws=None), -1),
    (dict(p=0.0), -1), (dict(p=-0.5), -1), (dict(p=1.5), -1), (dict(p=math.nan), -1),
    (dict(anchor=-1), -1), (dict(anchor=4097), -1),
    (dict(cap=4095), -4), (dict(Hq=7), -2), (dict(Hq=64), -5), (dict(T=0), -2),
    (dict(wsb=1024), -2),
    (dict(Q=ODD8), -1), (dict(K=ODD8), -1), (dict(V=ODD8), -1), (dict(O=ODD8), -1),
    (dict(ws=ODD16), -1),
])
def test_attend_rejects_bad_arguments(lib, kw, code):
    assert _attend(lib, **kw) == code
    assert len(lib.zha_last_error()) > 0


def test_tree_view_offsets_must_be_the_librarys(lib):
    """A view whose level offsets (or attached router copy's offsets) differ from where the
    library lays them out is rejected before anything is enqueued: a kernel would otherwise
    read a level at an arbitrary place."""
    t = _tree()
    assert lib.zha_attend_workspace_bytes(ctypes.byref(t), 1, 8) > 0
    for level, delta in ((1, 64), (2, -4), (3, 1 << 20)):
        bad = _tree()
        bad.level_off[level] += delta
        assert _attend(lib, t=bad) == -1
        assert b"level_off" in lib.zha_last_error()
        assert lib.zha_attend_workspace_bytes(ctypes.byref(bad), 1, 8) == 0
        assert lib.zha_tree_append(ctypes.byref(bad), FAKE, FAKE, 0, None) == -1
    # an attached router copy must sit where zha_router_quantize puts it
    r = _tree()
    r.router_data = 0x4000
    assert _attend(lib, t=r) == -1
    assert b"router offsets" in lib.zha_last_error()
    # zha_router_quantize lays the copy out itself: over zero tokens it enqueues nothing
    q = _tree(N=0)
    assert lib.zha_router_quantize(ctypes.byref(q), 0, FAKE, 1 << 40, None) == 0
    assert q.router == L.ZHA_ROUTER_MXFP4 and q.router_data == FAKE.value
    assert q.router_code_off[2] > 0 and q.router_scale_off[1] > q.router_code_off[1]
    assert lib.zha_tree_append(ctypes.byref(q), FAKE, FAKE, 0, None) == 0
    q.router_scale_off[3] += 16
    assert lib.zha_tree_append(ctypes.byref(q), FAKE, FAKE, 0, None) == -1


def test_attend_rejects_query_head_counts_past_int32(lib):
    # B * T * Hq = 2 * 2^26 * 16 = 2^31 query heads: numbered in int32, so rejected on the
    # host (before, the product wrapped negative and the workspace check passed)
    t = _tree(B=2, Hkv=2)
    assert _attend(lib, t=t, T=2 ** 26, Hq=16) == -5
    assert "exceeds 2^31 - 1" in lib.zha_last_error().decode()
    assert lib.zha_attend_workspace_bytes(ctypes.byref(t), 2 ** 26, 16) == 0
    assert lib.zha_attend_workspace_bytes(ctypes.byref(t), 2 ** 20, 16) > 0


def test_attend_rejects_bad_trees(lib):
    assert _attend(lib, t=_tree(d=80)) == -5
    assert _attend(lib, t=_tree(N=4100)) == -2       # N > N_cap
    assert _attend(lib, t=_tree(dtype=3)) == -3
    assert _attend(lib, t=_tree(N=0)) == -2
    t = _tree()
    t.pyramid = None
    assert _attend(lib, t=t) == -1
    assert lib.zha_attend(None, FAKE, 1, 8, FAKE, FAKE, 0.9, 1, FAKE, FAKE, 4096, FAKE, FAKE,
                          1 << 40, None) == -1


def test_workspace_size_grows_with_queries_and_is_zero_when_invalid(lib):
    t = _tree()
    a = lib.zha_attend_workspace_bytes(ctypes.byref(t), 1, 8)
    b = lib.zha_attend_workspace_bytes(ctypes.byref(t), 4, 8)
    assert 0 < a < b
    assert lib.zha_attend_workspace_bytes(ctypes.byref(t), 1, 7) == 0
    assert lib.zha_attend_workspace_bytes(ctypes.byref(_tree(N=0)), 1, 8) == 0


def test_level_view_offsets_are_inside_the_workspace(lib):
    t = _tree()
    need = lib.zha_attend_workspace_bytes(ctypes.byref(t), 3, 8)
    vals = [ctypes.c_int64() for _ in range(5)]
    assert lib.zha_attend_level_view(ctypes.byref(t), 3, 8, 1,
                                     *[ctypes.byref(v) for v in vals]) == 0
    o_n, o_m, o_c, stride, units = (v.value for v in vals)
    assert stride == 4096 // 4
    assert units == 1 * 2 * 1           # Tb = min(3, 16 / 4) = 3 queries per unit
    assert max(o_n, o_m) + 4 * units * stride <= need and o_c + 4 * units <= need
    for level in (2, 3, 4):               # only level 1 keeps a union list
        assert lib.zha_attend_level_view(ctypes.byref(t), 3, 8, level,
                                         *[ctypes.byref(v) for v in vals]) == -1


def test_level_bits_offsets_are_inside_the_workspace(lib):
    """Levels 2..L: every head's row of kept bits lies inside the workspace (the tree is
    b = 4, L = 3 over 4096 tokens: 64 top nodes, so 256 level-2 nodes)."""
    t = _tree()
    QH = 1 * 3 * 8
    need = lib.zha_attend_workspace_bytes(ctypes.byref(t), 3, 8)
    vals = [ctypes.c_int64() for _ in range(3)]
    for level in (2, 3):
        assert lib.zha_attend_level_bits(ctypes.byref(t), 3, 8, level,
                                         *[ctypes.byref(v) for v in vals]) == 0
        off, words, nodes = (v.value for v in vals)
        assert nodes == 4096 // 4 ** level
        assert 32 * words >= nodes
        last = off + 4 * ((QH - 1) * words + (nodes + 31) // 32)  # end of the last row's bits
        assert off % 4 == 0 and last <= need
    for level in (0, 1, 4):
        assert lib.zha_attend_level_bits(ctypes.byref(t), 3, 8, level,
                                         *[ctypes.byref(v) for v in vals]) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), -1), (dict(O=None), -1), (dict(ws=None), -1), (dict(K=ODD8), -1),
    (dict(dtype=5), -3), (dict(d=80), -5), (dict(N=0), -2), (dict(N=5000), -2),
    (dict(Hq=7), -2), (dict(Hq=64), -5), (dict(wsb=1024), -2), (dict(B=0), -2),
])
def test_dense_rejects_bad_arguments(lib, kw, code):
    a = dict(Q=FAKE, T=1, Hq=8, K=FAKE, V=FAKE, dtype=1, B=1, Hkv=2, N=4096, N_cap=4096, d=64,
             O=FAKE, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    assert lib.zha_dense_attend(a["Q"], a["T"], a["Hq"], a["K"], a["V"], a["dtype"], a["B"],
                                a["Hkv"], a["N"], a["N_cap"], a["d"], a["O"], a["ws"], a["wsb"],
                                None) == code
    assert len(lib.zha_last_error()) > 0


def test_dense_workspace_bytes(lib):
    n = lib.zha_dense_workspace_bytes(4, 4, 262144, 262144, 128, 1, 32)
    assert n >= 16 * 16 * 130 * 4          # one (d + 2)-float partial per member and split
    assert lib.zha_dense_workspace_bytes(1, 1, 0, 4096, 64, 1, 1) == 0
    assert lib.zha_dense_workspace_bytes(1, 1, 4096, 4096, 96, 1, 1) == 0
    # the documented bound N <= 2^21
    assert lib.zha_dense_workspace_bytes(1, 1, 2 ** 21, 2 ** 21, 64, 1, 1) > 0
    assert lib.zha_dense_workspace_bytes(1, 1, 2 ** 21 + 1, 2 ** 22, 64, 1, 1) == 0


def test_router_bytes_closed_form(lib):
    # per level: d/2 code bytes and d/32 scale bytes per node, each array rounded to 256 B
    def want(B, H, N, d, b, Ll):
        tot = 0
        for l in range(1, Ll + 1):
            rows = B * H * (N // b ** l)
            tot = (tot + rows * d // 2 + 255) // 256 * 256
            tot = (tot + rows * d // 32 + 255) // 256 * 256
        return tot
    assert lib.zha_router_bytes(4, 4, 262144, 128, 4, 6) == want(4, 4, 262144, 128, 4, 6)
    assert lib.zha_router_bytes(1, 1, 4096, 64, 4, 3) == want(1, 1, 4096, 64, 4, 3)
    assert lib.zha_router_bytes(1, 1, 4096, 96, 4, 3) == 0
    assert lib.zha_router_bytes(1, 1, 4000, 64, 4, 3) == 0
    # the MXFP4 copy is 17/128 of the float32 pyramid at d = 128 (68 of 512 bytes per node)
    r = lib.zha_router_bytes(4, 4, 262144, 128, 4, 6) / lib.zha_tree_bytes(4, 4, 262144, 128, 4, 6)
    assert abs(r - 68 / 512) < 1e-3


@pytest.mark.parametrize("kw,code", [
    (dict(data=None), -1), (dict(data=ODD8), -1), (dict(nbytes=1024), -2),
    (dict(n_from=-1), -2), (dict(n_from=4097), -2),
])
def test_router_quantize_rejects_bad_arguments(lib, kw, code):
    a = dict(data=FAKE, nbytes=1 << 30, n_from=0)
    a.update(kw)
    t = _tree()
    before = bytes(t)
    assert lib.zha_router_quantize(ctypes.byref(t), a["n_from"], a["data"], a["nbytes"],
                                   None) == code
    assert len(lib.zha_last_error()) > 0
    assert bytes(t) == before          # a rejected call leaves the tree as it was
    assert lib.zha_router_quantize(None, 0, FAKE, 1 << 30, None) == -1


def test_attend_rejects_bad_router_fields(lib):
    t = _tree()
    t.router = 1                       # MXFP4 without a copy
    assert _attend(lib, t=t) == -1
    t.router = 2                       # unknown
    t.router_data = 0x3000
    assert _attend(lib, t=t) == -1
    assert b"router" in lib.zha_last_error()


def test_causal_entry_points_reject_bad_positions(lib):
    t = _tree()
    args = (1, 8)
    for pos, code in ((None, -1), (ctypes.c_void_p(0x1002), -1)):
        assert lib.zha_attend_causal(ctypes.byref(t), FAKE, *args, pos, FAKE, FAKE, 0.9, 1, FAKE,
                                     FAKE, 4096, FAKE, FAKE, 1 << 40, None) == code
        assert lib.zha_dense_attend_causal(FAKE, 1, 8, pos, FAKE, FAKE, 1, 1, 2, 4096, 4096, 64,
                                           FAKE, FAKE, 1 << 40, None) == code
    # the other checks are zha_attend's
    assert lib.zha_attend_causal(ctypes.byref(t), FAKE, 1, 7, FAKE, FAKE, FAKE, 0.9, 1, FAKE,
                                 FAKE, 4096, FAKE, FAKE, 1 << 40, None) == -2


def test_missing_library_fails_loudly():
    """Without the built HIP library every entry point raises: there is no CPU fallback."""
    import subprocess
    import sys

    code = (
        "import torch\n"
        "import tree_indexed_sparse_amd._lib as L\n"
        "L.LIB_PATH = '/nonexistent/libzha.so'\n"
        "import tree_indexed_sparse_amd as Z\n"
        "K = torch.zeros(1, 1, 64, 64)\n"
        "R = torch.zeros(1, 16, 64)\n"
        "for call in (Z.load, lambda: Z.build_tree(K, R, 4, 1), lambda: Z.tree_bytes(1, 1, 64, 64, 4, 1)):\n"
        "    try:\n"
        "        call()\n"
        "    except ImportError as e:\n"
        "        assert 'not built' in str(e)\n"
        "    else:\n"
        "        raise SystemExit('no error')\n"
        "print('raised')\n"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "raised" in r.stdout


def test_noalloc_rejects_a_workspace_beyond_its_scratch(lib):
    """zha_attend_noalloc: a shape whose workspace exceeds the fixed device scratch (a 1M-token
    batch of 8) is rejected on the host with ZHA_ERR_CAPACITY before anything is enqueued."""
    t = L.ZhaTree()
    t.B, t.Hkv, t.N, t.N_cap, t.d, t.b, t.L, t.dtype = 8, 4, 1 << 20, 1 << 20, 128, 4, 7, 1
    t.pyramid = FAKE.value
    lay_out(lib, t)
    assert lib.zha_attend_workspace_bytes(ctypes.byref(t), 1, 32) > L.ZHA_NOALLOC_SCRATCH_BYTES
    code = lib.zha_attend_noalloc(ctypes.byref(t), FAKE, 1, 32, FAKE, FAKE, 0.95, 1, FAKE, None,
                                  1 << 20, FAKE, None)
    assert code == -4
    assert b"scratch" in lib.zha_last_error()
    t.B = 0
    assert lib.zha_attend_noalloc(ctypes.byref(t), FAKE, 1, 32, FAKE, FAKE, 0.95, 1, FAKE, None,
                                  1 << 20, FAKE, None) == -2


def test_level_view_assembles_unit_masks_from_head_bits(lib):
    """The diagnostic reader of levels >= 2 (tree_indexed_sparse_amd.level_view) on a host
    workspace whose rows of kept bits are filled by hand: the fused levels' rows end at the
    workspace's last byte, and the unit masks must be the members' bits, member m at bit m."""
    import numpy as np
    import torch
    import tree_indexed_sparse_amd as Z

    t = _tree(Hkv=1)
    T, Hq = 8, 1                          # one unit of 8 queries
    need = lib.zha_attend_workspace_bytes(ctypes.byref(t), T, Hq)
    ws = torch.zeros(need, dtype=torch.uint8)
    words = ws.view(torch.int32)
    vals = [ctypes.c_int64() for _ in range(3)]
    rng = np.random.default_rng(5)

    class _T:
        c = t

    for level in (2, 3):
        assert lib.zha_attend_level_bits(ctypes.byref(t), T, Hq, level,
                                         *[ctypes.byref(v) for v in vals]) == 0
        off, W, n = (v.value for v in vals)
        truth = rng.random((T, n)) < 0.05
        for qh in range(T):
            for j in np.nonzero(truth[qh])[0]:
                bit = 1 << (int(j) % 32)
                words[off // 4 + qh * W + int(j) // 32] |= bit if bit < 2 ** 31 else -2 ** 31
        nodes, masks, count = Z.level_view(_T(), T, Hq, level, ws)
        union = np.nonzero(truth.any(0))[0]
        assert count[0] == union.size
        assert (nodes[0, :union.size] == union).all()
        want = [sum(int(truth[m, j]) << m for m in range(T)) for j in union]
        assert list(masks[0, :union.size]) == want
