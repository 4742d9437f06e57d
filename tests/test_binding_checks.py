"""The Python binding's host-side checks of tensor shapes, dtypes and devices. The C ABI
takes bare pointers and sizes, so a tensor smaller than the call implies would be read or
written out of bounds on the GPU; the binding rejects such calls before anything reaches
the library. All CPU: the tensors here are host tensors, so a call whose shapes are right
gets as far as the device check and is refused there ("must be a device tensor")."""

import os

import pytest
import torch

import tree_indexed_sparse_amd as Z
from abi_views import lay_out
from tree_indexed_sparse_amd import _lib as LB

pytestmark = pytest.mark.skipif(not os.path.exists(LB.LIB_PATH), reason="libzha.so not built")

B, HKV, NCAP, D, BR, LV = 2, 2, 4096, 64, 4, 3
HQ, T = 8, 3


def _tree(dtype=LB.ZHA_BF16):
    c = LB.ZhaTree()
    for k, v in dict(B=B, Hkv=HKV, N=NCAP, N_cap=NCAP, d=D, b=BR, L=LV, dtype=dtype).items():
        setattr(c, k, v)
    c.pyramid = 0x2000  # never dereferenced: every call below stops on the host
    return Z.Tree(lay_out(LB.load(), c), torch.empty(4, dtype=torch.uint8))


def _inputs(dt=torch.bfloat16):
    return dict(Q=torch.zeros(B, T, HQ, D, dtype=dt), K=torch.zeros(B, HKV, NCAP, D, dtype=dt),
                V=torch.zeros(B, HKV, NCAP, D, dtype=dt))


def _code(fn):
    with pytest.raises(Z.ZhaError) as e:
        fn()
    return e.value.code, str(e.value)


def test_well_formed_attend_reaches_the_device_check():
    a = _inputs()
    code, msg = _code(lambda: Z.attend(a["Q"], a["K"], a["V"], _tree(), 0.95))
    assert code == -1 and "device tensor" in msg


@pytest.mark.parametrize("which,shape", [
    ("K", (B, HKV, NCAP // 2, D)),      # shorter cache than the tree indexes
    ("K", (B, HKV + 1, NCAP, D)),
    ("V", (B, HKV, NCAP // 2, D)),
    ("V", (B, HKV, NCAP)),
    ("Q", (B, T, HQ, D // 2)),          # head dim other than the tree's
    ("Q", (B + 1, T, HQ, D)),           # more sequences than the cache holds
    ("Q", (T, HQ, D)),
])
def test_attend_rejects_mis_shaped_inputs(which, shape):
    a = _inputs()
    a[which] = torch.zeros(shape, dtype=torch.bfloat16)
    for fn in (lambda: Z.attend(a["Q"], a["K"], a["V"], _tree(), 0.95),
               lambda: Z.attend_noalloc(a["Q"], a["K"], a["V"], _tree(), 0.95,
                                        out=torch.zeros(B, T, HQ, D),
                                        sel_idx=None,
                                        sel_count=torch.zeros(B, T, HQ, dtype=torch.int32))):
        code, msg = _code(fn)
        assert code == -2 and which in msg, msg


def test_attend_rejects_a_cache_in_another_dtype_than_the_tree():
    a = _inputs(torch.float32)  # the tree was built from bf16 keys
    code, msg = _code(lambda: Z.attend(a["Q"], a["K"], a["V"], _tree(LB.ZHA_BF16), 0.95))
    assert code == -3 and "dtype" in msg
    a = _inputs()
    a["V"] = a["V"].float()
    code, _ = _code(lambda: Z.attend(a["Q"], a["K"], a["V"], _tree(), 0.95))
    assert code == -3


@pytest.mark.parametrize("kw", [
    dict(out=torch.zeros(B, T, HQ, D // 2)),
    dict(out=torch.zeros(B, T, HQ, D, dtype=torch.bfloat16)),
    dict(sel_idx=torch.zeros(B, T, HQ - 1, NCAP, dtype=torch.int32)),
    dict(sel_idx=torch.zeros(B, T, HQ, NCAP, dtype=torch.int64)),
    dict(sel_count=torch.zeros(B, T + 1, HQ, dtype=torch.int32)),
    dict(sel_count=torch.zeros(B, T, HQ, dtype=torch.float32)),
])
def test_attend_rejects_mis_shaped_outputs(kw):
    a = _inputs()
    code, _ = _code(lambda: Z.attend(a["Q"], a["K"], a["V"], _tree(), 0.95, **kw))
    assert code in (-2, -3)


def test_attend_noalloc_needs_its_outputs():
    a = _inputs()
    code, msg = _code(lambda: Z.attend_noalloc(a["Q"], a["K"], a["V"], _tree(), 0.95, out=None,
                                               sel_idx=None, sel_count=None))
    assert code == -1 and "must be given" in msg


def test_attend_rejects_tensors_on_another_device():
    a = _inputs()
    meta = torch.zeros(B, T, HQ, D, device="meta")
    code, msg = _code(lambda: Z.attend(a["Q"], a["K"], a["V"], _tree(), 0.95, out=meta))
    assert code == -1 and "meta" in msg
    import numpy as np
    pos = np.zeros((B, T), np.int32)  # positions must be a tensor, not an array
    code, msg = _code(lambda: Z.attend(a["Q"], a["K"], a["V"], _tree(), 0.95, positions=pos))
    assert code == -1 and "torch tensor" in msg


def test_build_and_append_reject_mis_shaped_reference_queries():
    K = torch.zeros(B, HKV, NCAP, D, dtype=torch.bfloat16)
    for R in (torch.zeros(HKV, 8, D, dtype=torch.bfloat16),
              torch.zeros(HKV + 1, 16, D, dtype=torch.bfloat16),
              torch.zeros(HKV, 16, D // 2, dtype=torch.bfloat16)):
        code, msg = _code(lambda: Z.build_tree(K, R, BR, LV))
        assert code == -2 and "R" in msg
        code, msg = _code(lambda: Z.tree_append(_tree(), K, R, 1))
        assert code == -2 and "R" in msg
    R = torch.zeros(HKV, 16, D, dtype=torch.bfloat16)
    code, msg = _code(lambda: Z.tree_append(_tree(), K[:, :, :NCAP // 2], R, 1))
    assert code == -2 and "K" in msg
    code, msg = _code(lambda: Z.tree_append(_tree(LB.ZHA_F32), K, R, 1))
    assert code == -3
    code, msg = _code(lambda: Z.build_tree(K, R, BR, LV))  # well formed: refused as host memory
    assert code == -1 and "device tensor" in msg


def test_dense_attend_rejects_mis_shaped_inputs():
    a = _inputs()
    code, msg = _code(lambda: Z.dense_attend(a["Q"], a["K"], a["V"][:, :, :100]))
    assert code == -2 and "V" in msg
    code, msg = _code(lambda: Z.dense_attend(a["Q"][..., :32], a["K"], a["V"]))
    assert code == -2 and "K" in msg
    code, msg = _code(lambda: Z.dense_attend(a["Q"], a["K"], a["V"],
                                             out=torch.zeros(B, T, HQ, D // 2)))
    assert code == -2 and "out" in msg
    code, msg = _code(lambda: Z.dense_attend(a["Q"], a["K"], a["V"]))
    assert code == -1 and "device tensor" in msg
