"""Compare the GPU path's outputs with the oracle (test infrastructure only).

The comparison walks each query head's descent level by level, following the GPU's kept
sets (read back from the union lists zha_attend leaves in its workspace):

* at every level the oracle recomputes its own decision on the GPU's frontier; the GPU's
  kept set must equal it exactly unless the oracle marks that decision fragile (near-tie
  in score or in cumulative mass, NEAR_TIE_REL); a fragile decision may instead resolve
  to any set that keeps every node clearly above the cut score, drops every node clearly
  below it, and differs in size by at most one;
* the GPU's selected-token list must equal the anchor tokens plus the b tokens of every
  GPU-kept level-1 node, exactly;
* the GPU's output must match the oracle's exact attention over the GPU's own list.

Heads whose oracle descent has no fragile decision are also compared unguided: the GPU's
list must equal the oracle's own list.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import zha_oracle as O


def unit_member(b: int, t: int, h: int, T: int, Hq: int, Hkv: int):
    """(unit, member) of query head (b, t, h), matching the layout in include/zha.h."""
    G = Hq // Hkv
    Tb = min(T, 16 // G)
    nTB = -(-T // Tb)
    g = h // G
    return (b * Hkv + g) * nTB + t // Tb, (t % Tb) * G + h % G


def gpu_kept(level_lists, u: int, m: int) -> np.ndarray:
    nodes, masks, count = level_lists
    n = int(count[u])
    sel = ((masks[u, :n] >> m) & 1).astype(bool)
    return nodes[u, :n][sel].astype(np.int64)


def _fragile_ok(F, s, kept_o, G):
    """Is the GPU set G an allowed resolution of a fragile decision? It must keep every
    node scored clearly above the oracle's cut score, keep no node clearly below it
    except the oracle's first dropped node (when a near-p cumulative mass grows the set by
    one), and differ in size by at most one."""
    k = kept_o.size
    if abs(G.size - k) > 1 or not np.all(np.isin(G, F)):
        return False
    s64 = s.astype(np.float64)
    order = np.lexsort((F, -s64))
    cut = s64[order[k - 1]]
    tol = O.NEAR_TIE_REL * max(1.0, abs(cut))
    inG = np.isin(F, G)
    if np.any(~inG & (s64 > cut + tol)):
        return False
    extra = F[inG & (s64 < cut - tol)]
    if extra.size == 0:
        return True
    return G.size == k + 1 and extra.size == 1 and k < F.size and extra[0] == F[order[k]]


@dataclass
class HeadReport:
    qh: tuple
    exact_unguided: bool | None      # None when the oracle's own path has a fragile decision
    fragile_levels: list = field(default_factory=list)
    mismatch: str | None = None
    o_err: float = 0.0
    keys: int = 0


def check_head(q, levels, K_u, V_u, b, L, p, anchor, lists_by_level, u, m, sel_row, count,
               O_gpu, qh=None, fp4=False) -> HeadReport:
    """Guided comparison of one query head. lists_by_level[l] = level_view(...) at level l.
    fp4: the descent scored MXFP4 summaries with an MXFP4 query (the FP4 router); the
    final attention uses the unquantised query either way."""
    p = float(np.float32(p))
    rep = HeadReport(qh=qh, exact_unguided=None)
    n_top = levels[L].shape[0]
    q_r, levels_r = (O.mxfp4_round_trip(q), O.router_levels(levels)) if fp4 else (q, levels)
    F = np.arange(n_top, dtype=np.int64)
    kept = F
    for l in (range(L, 0, -1) if n_top else ()):
        Gk = gpu_kept(lists_by_level[l], u, m)
        s = O.node_scores(levels_r[l][F], q_r)
        kept_o, fragile = O.select_top_p(F, s, p)
        if not np.array_equal(Gk, kept_o):
            if not fragile or not _fragile_ok(F, s, kept_o, Gk):
                rep.mismatch = (f"level {l}: gpu kept {Gk.size} nodes, oracle {kept_o.size}; "
                                f"fragile={fragile}; first diffs "
                                f"{np.setxor1d(Gk, kept_o)[:8].tolist()}")
                return rep
        if fragile:
            rep.fragile_levels.append((l, fragile))
        kept = Gk
        if l > 1:
            F = O.expand(kept, b)
    N = K_u.shape[0]
    S_want = np.union1d(np.arange(min(anchor, N), dtype=np.int64), O.expand(kept, b))
    S_want = np.union1d(S_want, O.tail_tokens(N, n_top, b, L))
    S_gpu = np.asarray(sel_row[:count], np.int64) if sel_row is not None else None
    if int(count) != S_want.size:
        rep.mismatch = f"count {int(count)} != {S_want.size}"
        return rep
    if S_gpu is not None and not np.array_equal(S_gpu, S_want):
        rep.mismatch = "token list differs from the expansion of the kept level-1 nodes"
        return rep
    rep.keys = S_want.size
    O_want = O.attention_over(q, K_u, V_u, S_want)
    rep.o_err = float(np.max(np.abs(np.asarray(O_gpu, np.float64) - O_want)))
    S_own, decs = O.search(q_r, levels_r, b, L, p, anchor)
    if not any(d.fragile for d in decs):
        rep.exact_unguided = bool(np.array_equal(S_own, S_want))
        if not rep.exact_unguided:
            rep.mismatch = "unguided token list differs although no decision is fragile"
    return rep


def summarize(reports: list) -> dict:
    fr = [r for r in reports if r.exact_unguided is None]
    return dict(
        heads=len(reports),
        mismatches=sum(r.mismatch is not None for r in reports),
        exact_unguided=sum(bool(r.exact_unguided) for r in reports),
        heads_with_fragile_decisions=len(fr),
        max_o_err=max((r.o_err for r in reports), default=0.0),
        first_mismatch=next((f"{r.qh}: {r.mismatch}" for r in reports if r.mismatch), None),
    )


def pyramid_rel_err(gpu_level: np.ndarray, oracle_level: np.ndarray) -> float:
    """max |gpu - oracle| / max |oracle| over one level of one unit."""
    scale = max(float(np.max(np.abs(oracle_level))), 1e-30)
    return float(np.max(np.abs(gpu_level.astype(np.float64) - oracle_level.astype(np.float64)))) / scale
