"""Tree views for host-only tests of the C ABI: the library lays out a view itself
(zha_build_tree over zero tokens enqueues nothing), so tests that hand-fill a view's
geometry take its level offsets from there."""

import ctypes

from tree_indexed_sparse_amd import _lib as L

PLACEHOLDER = ctypes.c_void_p(0x1000)  # never dereferenced: nothing is enqueued


def lay_out(lib, t):
    """Give the hand-filled view t the level offsets zha_build_tree writes for its geometry.
    An invalid geometry leaves t as it is: its own check fails before the offsets'."""
    v = L.ZhaTree()
    dtype = t.dtype if t.dtype in (L.ZHA_F32, L.ZHA_BF16) else L.ZHA_BF16
    st = lib.zha_build_tree(PLACEHOLDER, PLACEHOLDER, dtype, t.B, t.Hkv, 0, t.N_cap, t.d, t.b,
                            t.L, PLACEHOLDER, 1 << 40, ctypes.byref(v), None)
    if st == 0:
        for l in range(len(t.level_off)):
            t.level_off[l] = v.level_off[l]
    return t
