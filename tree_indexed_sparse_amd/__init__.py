"""Tree-indexed sparse decode attention (Zyphra Hierarchical Attention) on MI355X.

Python face of the C ABI in include/zha.h. torch supplies device memory and the current
HIP stream; the pyramid build, the tree search and the sparse decode all run in the
library's hand-written gfx950 kernels (libzha.so). Names follow the C entry points:

    tree = build_tree(K, R, b, L)             # zha_build_tree
    tree_append(tree, K, R, n_new)            # zha_tree_append
    quantize_router(tree)                     # zha_router_quantize (the FP4 router)
    O, sel_idx, sel_count = attend(Q, K, V, tree, p, anchor=1)   # zha_attend
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from ._lib import (  # noqa: F401
    ZHA_BF16,
    ZHA_F32,
    ZHA_N_REF,
    ZHA_NOALLOC_SCRATCH_BYTES,
    ZHA_ROUTER_F32,
    ZHA_ROUTER_MXFP4,
    ZhaError,
    ZhaTree,
    check,
    load,
)

__all__ = ["Tree", "build_tree", "tree_append", "attend", "attend_noalloc", "workspace_bytes",
           "level_view",
           "tree_bytes", "pyramid_level", "router_bytes", "quantize_router", "set_router",
           "router_level", "ZhaError", "load"]

_DTYPES = {torch.float32: ZHA_F32, torch.bfloat16: ZHA_BF16}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise ZhaError(-3, f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ZhaError(-1, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ZhaError(-2, f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _shape(t: torch.Tensor, name: str, want: tuple, dtype=None) -> None:
    """Raise unless t has shape `want` (None entries match any size) and, if given, dtype.
    The library takes bare pointers, so a tensor smaller than the call implies would be
    read or written out of bounds on the GPU: the checks run on the host, before the call."""
    got = tuple(t.shape)
    if len(got) != len(want) or any(w is not None and g != w for g, w in zip(got, want)):
        shown = ", ".join("*" if w is None else str(w) for w in want)
        raise ZhaError(-2, f"{name} has shape {list(got)}, expected [{shown}]")
    if dtype is not None and t.dtype != dtype:
        raise ZhaError(-3, f"{name} has dtype {t.dtype}, expected {dtype}")


def _same_device(device, **tensors) -> None:
    for name, t in tensors.items():
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise ZhaError(-1, f"{name} must be a torch tensor (got {type(t).__name__})")
        if t.device != device:
            raise ZhaError(-1, f"{name} is on {t.device}, expected {device}")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _check_kv(tree: "Tree", K: torch.Tensor, V: torch.Tensor | None = None) -> None:
    """K (and V) must be the cache the tree indexes: [B, Hkv, N_cap, d] in its dtype."""
    c = tree.c
    want = (int(c.B), int(c.Hkv), int(c.N_cap), int(c.d))
    _shape(K, "K", want)
    if _DTYPES.get(K.dtype) != int(c.dtype):
        raise ZhaError(-3, f"K has dtype {K.dtype}; the tree was built from another dtype")
    if V is not None:
        _shape(V, "V", want, K.dtype)


def tree_bytes(B: int, Hkv: int, N_cap: int, d: int, b: int, L: int) -> int:
    return int(load().zha_tree_bytes(B, Hkv, N_cap, d, b, L))


@dataclass
class Tree:
    """A built pyramid: the C view plus the tensors that own its storage (the float32
    pyramid, and the MXFP4 router copy once quantize_router made one)."""
    c: ZhaTree
    storage: torch.Tensor
    router_storage: torch.Tensor | None = None

    @property
    def N(self) -> int:
        return int(self.c.N)

    @property
    def b(self) -> int:
        return int(self.c.b)

    @property
    def L(self) -> int:
        return int(self.c.L)


def pyramid_level(tree: Tree, level: int) -> torch.Tensor:
    """Float32 view [B, Hkv, N_cap / b^level, d] of one pyramid level."""
    c = tree.c
    n = c.N_cap // c.b ** level
    numel = c.B * c.Hkv * n * c.d
    flat = tree.storage.view(torch.float32)
    off = int(c.level_off[level])
    return flat[off:off + numel].view(c.B, c.Hkv, n, c.d)


def build_tree(K: torch.Tensor, R: torch.Tensor, b: int, L: int, N: int | None = None,
               router: bool = False) -> Tree:
    """zha_build_tree over tokens [0, N) of the cache K [B, Hkv, N_cap, d].
    router=True also writes the MXFP4 router copy and selects it: the tree is started
    empty, given its copy (zha_router_quantize), and extended by N tokens
    (zha_tree_append), so the pooling launches encode the rows they write."""
    lib = load()
    _shape(K, "K", (None, None, None, None))
    B, Hkv, N_cap, d = K.shape
    N = N_cap if N is None else N
    if R.dtype != K.dtype:
        raise ZhaError(-3, "K and R must share a dtype")
    _shape(R, "R", (Hkv, ZHA_N_REF, d))
    _same_device(K.device, R=R)
    nbytes = tree_bytes(B, Hkv, N_cap, d, b, L)
    storage = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=K.device)
    c = ZhaTree()
    check(lib.zha_build_tree(_dev(K, "K"), _dev(R, "R"), _dt(K), B, Hkv, 0 if router else N,
                             N_cap, d, b, L, storage.data_ptr(), nbytes, ctypes.byref(c),
                             _stream(K.device)))
    tree = Tree(c, storage)
    if router:
        quantize_router(tree)
        tree_append(tree, K, R, N)
    return tree


def tree_append(tree: Tree, K: torch.Tensor, R: torch.Tensor, n_new: int) -> None:
    """zha_tree_append: pool tokens [N, N + n_new) and extend the tree."""
    _check_kv(tree, K)
    _shape(R, "R", (int(tree.c.Hkv), ZHA_N_REF, int(tree.c.d)), K.dtype)
    _same_device(tree.storage.device, K=K, R=R)
    check(load().zha_tree_append(ctypes.byref(tree.c), _dev(K, "K"), _dev(R, "R"), n_new,
                                 _stream(K.device)))


def router_bytes(B: int, Hkv: int, N_cap: int, d: int, b: int, L: int) -> int:
    return int(load().zha_router_bytes(B, Hkv, N_cap, d, b, L))


def quantize_router(tree: Tree, n_from: int = 0) -> None:
    """zha_router_quantize: encode the pyramid's nodes complete at tree.N (those not yet
    complete at n_from tokens) as MXFP4 and make zha_attend score that copy. The copy's
    storage is allocated on the first call and kept with the tree; later appends encode
    the nodes they complete."""
    c = tree.c
    nbytes = router_bytes(c.B, c.Hkv, c.N_cap, c.d, c.b, c.L)
    if tree.router_storage is None:
        tree.router_storage = torch.empty(max(nbytes, 4), dtype=torch.uint8,
                                          device=tree.storage.device)
    check(load().zha_router_quantize(ctypes.byref(c), int(n_from),
                                     tree.router_storage.data_ptr(), tree.router_storage.numel(),
                                     _stream(tree.storage.device)))


def set_router(tree: Tree, router: str) -> None:
    """Choose which copy zha_attend scores: "f32" (the float32 pyramid) or "mxfp4" (the
    copy quantize_router wrote)."""
    if router == "f32":
        tree.c.router = ZHA_ROUTER_F32
    elif router == "mxfp4":
        if tree.router_storage is None:
            raise ZhaError(-1, "the tree has no MXFP4 router copy; call quantize_router")
        tree.c.router = ZHA_ROUTER_MXFP4
    else:
        raise ZhaError(-1, f"unknown router {router!r}")


def router_level(tree: Tree, level: int):
    """Views of one level of the MXFP4 router copy: (codes [B, Hkv, N_cap / b^level, d / 2]
    uint8, two E2M1 codes per byte, low nibble first; scales [B, Hkv, N_cap / b^level,
    d / 32] uint8, E8M0)."""
    c = tree.c
    if tree.router_storage is None:
        raise ZhaError(-1, "the tree has no MXFP4 router copy")
    n = c.N_cap // c.b ** level
    rows = c.B * c.Hkv * n
    co, so = int(c.router_code_off[level]), int(c.router_scale_off[level])
    w = tree.router_storage
    codes = w[co:co + rows * (c.d // 2)].view(c.B, c.Hkv, n, c.d // 2)
    scales = w[so:so + rows * (c.d // 32)].view(c.B, c.Hkv, n, c.d // 32)
    return codes, scales


def workspace_bytes(tree: Tree, T: int, Hq: int) -> int:
    return int(load().zha_attend_workspace_bytes(ctypes.byref(tree.c), T, Hq))


def _check_outputs(B, T, Hq, d, out, sel_idx, sel_count, required=False) -> None:
    """Caller-supplied outputs: O [B, T, Hq, d] float32, sel_idx [B, T, Hq, cap] int32 (the
    library checks cap against N), sel_count [B, T, Hq] int32."""
    if required and (out is None or sel_count is None):
        raise ZhaError(-1, "out and sel_count must be given")
    if out is not None:
        _shape(out, "out", (B, T, Hq, d), torch.float32)
    if sel_idx is not None:
        _shape(sel_idx, "sel_idx", (B, T, Hq, None), torch.int32)
    if sel_count is not None:
        _shape(sel_count, "sel_count", (B, T, Hq), torch.int32)


def attend(Q, K, V, tree: Tree, p: float, anchor: int = 1, *, want_lists: bool = True,
           out=None, sel_idx=None, sel_count=None, workspace=None, positions=None):
    """zha_attend (or zha_attend_causal when `positions`, an int32 device tensor [B, T] of
    query positions, is given). Returns (O [B,T,Hq,d] float32, sel_idx [B,T,Hq,N] int32 or
    None, sel_count [B,T,Hq] int32). Buffers may be passed in to avoid allocation."""
    lib = load()
    _check_kv(tree, K, V)
    _shape(Q, "Q", (int(tree.c.B), None, None, int(tree.c.d)))
    B, T, Hq, d = Q.shape
    dev = Q.device
    if Q.dtype != K.dtype or V.dtype != K.dtype:
        raise ZhaError(-3, "Q, K and V must share a dtype")
    _check_outputs(B, T, Hq, d, out, sel_idx, sel_count)
    _same_device(dev, K=K, V=V, out=out, sel_idx=sel_idx, sel_count=sel_count,
                 workspace=workspace, positions=positions, pyramid=tree.storage)
    if out is None:
        out = torch.empty((B, T, Hq, d), dtype=torch.float32, device=dev)
    cap = tree.N
    if want_lists and sel_idx is None:
        sel_idx = torch.empty((B, T, Hq, cap), dtype=torch.int32, device=dev)
    if sel_idx is not None:
        cap = sel_idx.shape[-1]
    if sel_count is None:
        sel_count = torch.empty((B, T, Hq), dtype=torch.int32, device=dev)
    need = workspace_bytes(tree, T, Hq)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    sel_ptr = _dev(sel_idx, "sel_idx") if sel_idx is not None else None
    if positions is None:
        check(lib.zha_attend(ctypes.byref(tree.c), _dev(Q, "Q"), T, Hq, _dev(K, "K"),
                             _dev(V, "V"), float(p), int(anchor), _dev(out, "O"), sel_ptr, cap,
                             _dev(sel_count, "sel_count"), _dev(workspace, "workspace"),
                             _nbytes(workspace), _stream(dev)))
    else:
        check(lib.zha_attend_causal(ctypes.byref(tree.c), _dev(Q, "Q"), T, Hq,
                                    _positions(positions, B, T), _dev(K, "K"), _dev(V, "V"),
                                    float(p), int(anchor), _dev(out, "O"), sel_ptr, cap,
                                    _dev(sel_count, "sel_count"), _dev(workspace, "workspace"),
                                    _nbytes(workspace), _stream(dev)))
    attend.last_workspace = workspace
    return out, sel_idx, sel_count


def attend_noalloc(Q, K, V, tree: Tree, p: float, anchor: int = 1, *, out, sel_idx,
                   sel_count):
    """zha_attend_noalloc: zha_attend with the library's fixed device scratch as its
    workspace; the caller passes the outputs (O [B,T,Hq,d] float32, sel_idx [B,T,Hq,cap]
    int32 or None, sel_count [B,T,Hq] int32), so nothing is allocated."""
    lib = load()
    _check_kv(tree, K, V)
    _shape(Q, "Q", (int(tree.c.B), None, None, int(tree.c.d)))
    B, T, Hq, d = Q.shape
    if Q.dtype != K.dtype or V.dtype != K.dtype:
        raise ZhaError(-3, "Q, K and V must share a dtype")
    _check_outputs(B, T, Hq, d, out, sel_idx, sel_count, required=True)
    _same_device(Q.device, K=K, V=V, out=out, sel_idx=sel_idx, sel_count=sel_count,
                 pyramid=tree.storage)
    cap = sel_idx.shape[-1] if sel_idx is not None else tree.N
    sel_ptr = _dev(sel_idx, "sel_idx") if sel_idx is not None else None
    check(lib.zha_attend_noalloc(ctypes.byref(tree.c), _dev(Q, "Q"), T, Hq, _dev(K, "K"),
                                 _dev(V, "V"), float(p), int(anchor), _dev(out, "O"), sel_ptr,
                                 cap, _dev(sel_count, "sel_count"), _stream(Q.device)))
    return out, sel_idx, sel_count


def dense_workspace_bytes(B: int, Hkv: int, N: int, N_cap: int, d: int, T: int, Hq: int) -> int:
    return int(load().zha_dense_workspace_bytes(B, Hkv, N, N_cap, d, T, Hq))


def _positions(positions, B: int, T: int) -> int:
    if positions.dtype != torch.int32 or tuple(positions.shape) != (B, T):
        raise ZhaError(-2, f"positions must be int32 [{B}, {T}]")
    return _dev(positions, "positions")


def dense_attend(Q, K, V, N: int | None = None, *, out=None, workspace=None, positions=None):
    """zha_dense_attend: exact attention over all N cached keys (the dense comparator), or
    zha_dense_attend_causal over keys [0, position] when `positions` [B, T] is given.
    K, V [B,Hkv,N_cap,d]; returns O [B,T,Hq,d] float32."""
    lib = load()
    _shape(Q, "Q", (None, None, None, None))
    _shape(K, "K", (Q.shape[0], None, None, Q.shape[3]))
    _shape(V, "V", tuple(K.shape))
    B, T, Hq, d = Q.shape
    _, Hkv, N_cap, _ = K.shape
    N = N_cap if N is None else N
    dev = Q.device
    if Q.dtype != K.dtype or V.dtype != K.dtype:
        raise ZhaError(-3, "Q, K and V must share a dtype")
    if out is not None:
        _shape(out, "out", (B, T, Hq, d), torch.float32)
    _same_device(dev, K=K, V=V, out=out, workspace=workspace, positions=positions)
    if out is None:
        out = torch.empty((B, T, Hq, d), dtype=torch.float32, device=dev)
    need = dense_workspace_bytes(B, Hkv, N, N_cap, d, T, Hq)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    if positions is None:
        check(lib.zha_dense_attend(_dev(Q, "Q"), T, Hq, _dev(K, "K"), _dev(V, "V"), _dt(K), B,
                                   Hkv, N, N_cap, d, _dev(out, "O"), _dev(workspace, "workspace"),
                                   _nbytes(workspace), _stream(dev)))
    else:
        check(lib.zha_dense_attend_causal(_dev(Q, "Q"), T, Hq, _positions(positions, B, T),
                                          _dev(K, "K"), _dev(V, "V"), _dt(K), B, Hkv, N, N_cap, d,
                                          _dev(out, "O"), _dev(workspace, "workspace"),
                                          _nbytes(workspace), _stream(dev)))
    return out


def level_view(tree: Tree, T: int, Hq: int, level: int, workspace: torch.Tensor):
    """Per-level union lists a finished zha_attend left in `workspace`, on the host:
    (nodes [U, stride] int64, masks [U, stride] int64, count [U] int64) with bit m of a
    mask set when member m of the unit kept the node. Level 1 is read as the library keeps
    it (zha_attend_level_view); the levels above are assembled here from the heads' kept
    bits (zha_attend_level_bits), a diagnostic view of what the search kept."""
    import numpy as np

    lib = load()
    w = workspace.view(torch.uint8)

    def u32(off, n):
        return w[off:off + 4 * n].view(torch.int32).cpu().numpy().astype("int64") & 0xFFFFFFFF

    if level == 1:
        o_n, o_m, o_c, st, units = (ctypes.c_int64() for _ in range(5))
        check(lib.zha_attend_level_view(ctypes.byref(tree.c), T, Hq, level, ctypes.byref(o_n),
                                        ctypes.byref(o_m), ctypes.byref(o_c), ctypes.byref(st),
                                        ctypes.byref(units)))
        U, S = units.value, st.value
        return (u32(o_n.value, U * S).reshape(U, S), u32(o_m.value, U * S).reshape(U, S),
                u32(o_c.value, U))
    o_b, words, nodes = (ctypes.c_int64() for _ in range(3))
    check(lib.zha_attend_level_bits(ctypes.byref(tree.c), T, Hq, level, ctypes.byref(o_b),
                                    ctypes.byref(words), ctypes.byref(nodes)))
    B, Hkv = int(tree.c.B), int(tree.c.Hkv)
    QH, n, W = B * T * Hq, nodes.value, words.value
    nw = (n + 31) // 32  # the words that hold nodes 0 .. n - 1 in each head's row
    span = 4 * ((QH - 1) * W + nw)  # rows are W words apart; the last ends inside the workspace
    raw = w[o_b.value:o_b.value + span].cpu().numpy()
    rows = np.stack([raw[4 * W * qh:4 * W * qh + 4 * nw] for qh in range(QH)])
    kept = np.unpackbits(rows, axis=1, bitorder="little")[:, :n]  # [QH, n]
    # units: the G heads of a KV head and Tb queries of a sequence
    G = Hq // Hkv
    Tb = min(T, 16 // G)
    nTB = -(-T // Tb)
    U = B * Hkv * nTB
    masks = np.zeros((U, n), np.int64)
    for u in range(U):
        tb, kv, bb = u % nTB, (u // nTB) % Hkv, u // (nTB * Hkv)
        for m in range(min(Tb, T - tb * Tb) * G):
            t, h = tb * Tb + m // G, kv * G + m % G
            masks[u] |= kept[(bb * T + t) * Hq + h].astype(np.int64) << m
    out_nodes = np.zeros((U, n), np.int64)
    out_masks = np.zeros((U, n), np.int64)
    count = np.zeros(U, np.int64)
    for u in range(U):
        nz = np.nonzero(masks[u])[0]
        count[u] = nz.size
        out_nodes[u, :nz.size] = nz
        out_masks[u, :nz.size] = masks[u, nz]
    return out_nodes, out_masks, count
