"""zha_attend_noalloc (the workspace-free zha_attend, for callers that cannot allocate)
against zha_attend on the same inputs, through the C ABI: two calls in a row, the second
on a smaller input, each bit-identical in outputs, selected lists and counts to
zha_attend with its own workspace."""

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_indexed_sparse_amd as Z
    Z.load()


def _both(spec, p):
    import tree_indexed_sparse_amd as Z

    inp = W.gen_all(spec, device="cuda")
    Q, K, V, R = inp["Q"], inp["K"], inp["V"], inp["R"]
    B, T, Hq, d, N = (spec[k] for k in ("B", "T", "Hq", "d", "N"))
    tree = Z.build_tree(K, R, spec["b"], spec["L"])
    assert Z.workspace_bytes(tree, T, Hq) <= Z.ZHA_NOALLOC_SCRATCH_BYTES
    ref = Z.attend(Q, K, V, tree, p, 1)
    O = torch.full((B, T, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    sel = torch.full((B, T, Hq, N), -1, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, T, Hq), -1, dtype=torch.int32, device="cuda")
    Z.attend_noalloc(Q, K, V, tree, p, 1, out=O, sel_idx=sel, sel_count=cnt)
    torch.cuda.synchronize()
    assert torch.equal(cnt, ref[2])
    assert torch.equal(O, ref[0])
    n = cnt.cpu().numpy()
    s_now, s_ref = sel.cpu().numpy(), ref[1].cpu().numpy()
    for idx in np.ndindex(*n.shape):
        assert np.array_equal(s_now[idx][:n[idx]], s_ref[idx][:n[idx]]), idx
    Z.attend.last_workspace = None
    return int(n.sum())


def test_noalloc_matches_attend_on_two_calls():
    """A 32K-token batch (two sequences, 32/4 heads, the deep tree), then a smaller one
    (tiny float32 workload): the second call runs on the scratch the first one left."""
    big = W.spec("32k_deep", B=2)
    small = W.spec("tiny")
    kept_big = _both(big, 0.95)
    kept_small = _both(small, 0.9)
    print(f"[noalloc] {kept_big} and {kept_small} selected tokens, bit-identical to zha_attend",
          flush=True)
