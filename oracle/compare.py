"""Compare the GPU path's outputs with the oracle (test infrastructure only).

The comparison walks each query head's descent level by level, following the GPU's kept
sets (read back from the union lists zha_attend leaves in its workspace):

* at every level the oracle recomputes its own decision on the GPU's frontier; the GPU's
  kept set must equal it exactly unless the oracle marks that decision fragile (near-tie
  in score or in cumulative mass, NEAR_TIE_REL); a fragile decision may instead resolve
  to another set only in the way its kind allows (fragile_ok);
* the GPU's selected-token list must equal the anchor tokens plus the b tokens of every
  GPU-kept level-1 node, exactly;
* the GPU's output must match the oracle's exact attention over the GPU's own list, both
  in absolute terms and relative to the output's own magnitude, and be finite.

Every head is also compared unguided (the GPU's list against the oracle's own list);
the match is required when the oracle's own descent has no fragile decision and counted
otherwise.

Source: "Zyphra présente Zyphra Hierarchical Attention (ZHA), une voie vers une attention
vraiment sous-quadratique" (Le Fil IA), paragraph 1: the selected set is the smallest
one covering a fraction p of the estimated mass; the attention over it is exact.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import zha_oracle as O

# Output bound relative to the magnitude of the oracle's output, on top of the absolute
# bounds the tests state: at 256K the outputs are ~1e-2 in magnitude, so an absolute 2e-2
# alone would accept an all-zero output.
O_REL_TOL = 1e-3


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


def fragile_ok(F, s, kept_o, G, fragile) -> bool:
    """Is the set G an allowed resolution of the oracle's fragile decision kept_o?

    F: frontier ids, s: their float32 scores, kept_o: the oracle's kept ids, fragile: the
    oracle's [(kind, gap)] for this decision. The size of G may be
      * the oracle's k (always),
      * k + 1 only under "mass_hi" (the cumulative mass at the cut is within NEAR_TIE_REL
        above p: other rounding can fall short of p there and take the next node),
      * k - 1 only under "mass_lo" (the cumulative mass one node before the cut is within
        NEAR_TIE_REL below p: other rounding can reach p there).
    A set of size k other than kept_o needs "score" (the last kept and first dropped
    scores are near-tied). G must be the top |G| nodes of F in score order up to near-ties:
    no node outside G may score more than NEAR_TIE_REL (relative to the cut score, floor 1)
    above a node inside it."""
    kinds = {kind for kind, _ in fragile}
    G = np.asarray(G, np.int64)
    k = int(np.asarray(kept_o).size)
    sizes = {k}
    if "mass_hi" in kinds:
        sizes.add(k + 1)
    if "mass_lo" in kinds:
        sizes.add(k - 1)
    if G.size not in sizes or G.size < 1 or G.size > F.size:
        return False
    if np.unique(G).size != G.size or not np.all(np.isin(G, F)):
        return False
    if G.size == k and "score" not in kinds and not np.array_equal(np.sort(G), np.sort(kept_o)):
        return False
    if G.size == F.size:
        return True
    s64 = np.asarray(s, np.float32).astype(np.float64)
    order = np.lexsort((F, -s64))
    cut = s64[order[k - 1]]
    tol = O.NEAR_TIE_REL * max(1.0, abs(cut))
    inG = np.isin(F, G)
    return bool(s64[inG].min() >= s64[~inG].max() - tol)


@dataclass
class HeadReport:
    qh: tuple
    exact_unguided: bool | None = None   # GPU list == the oracle's own list
    own_fragile: bool = False            # the oracle's own descent has a fragile decision
    fragile_levels: list = field(default_factory=list)
    diverged_levels: list = field(default_factory=list)   # fragile decisions the GPU resolved otherwise
    mismatch: str | None = None
    o_err: float = 0.0
    o_rel: float = 0.0
    o_scale: float = 0.0
    keys: int = 0


def check_head(q, levels, K_u, V_u, b, L, p, anchor, lists_by_level, u, m, sel_row, count,
               O_gpu, qh=None, fp4=False) -> HeadReport:
    """Guided comparison of one query head. lists_by_level[l] = level_view(...) at level l.
    fp4: the descent scored MXFP4 summaries with an MXFP4 query (the FP4 router); the
    final attention uses the unquantised query either way."""
    p = float(np.float32(p))
    rep = HeadReport(qh=qh)
    n_top = levels[L].shape[0]
    q_r, levels_r = (O.mxfp4_round_trip(q), O.router_levels(levels)) if fp4 else (q, levels)
    F = np.arange(n_top, dtype=np.int64)
    kept = F
    for l in (range(L, 0, -1) if n_top else ()):
        Gk = gpu_kept(lists_by_level[l], u, m)
        s = O.node_scores(levels_r[l][F], q_r)
        kept_o, fragile = O.select_top_p(F, s, p)
        if not np.array_equal(Gk, kept_o):
            if not fragile or not fragile_ok(F, s, kept_o, Gk, fragile):
                rep.mismatch = (f"level {l}: gpu kept {Gk.size} nodes, oracle {kept_o.size}; "
                                f"fragile={fragile}; first diffs "
                                f"{np.setxor1d(Gk, kept_o)[:8].tolist()}")
                return rep
            rep.diverged_levels.append((l, Gk.size - kept_o.size))
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
    O_got = np.asarray(O_gpu, np.float64)
    if not np.all(np.isfinite(O_got)):
        rep.mismatch = "output is not finite"
        return rep
    rep.o_err = float(np.max(np.abs(O_got - O_want)))
    rep.o_scale = float(np.max(np.abs(O_want)))
    rep.o_rel = rep.o_err / max(rep.o_scale, 1e-30)
    S_own, decs = O.search(q_r, levels_r, b, L, p, anchor)
    rep.own_fragile = any(d.fragile for d in decs)
    rep.exact_unguided = bool(np.array_equal(S_own, S_want))
    if not rep.own_fragile and not rep.exact_unguided:
        rep.mismatch = "unguided token list differs although no decision is fragile"
    return rep


def summarize(reports: list) -> dict:
    return dict(
        heads=len(reports),
        mismatches=sum(r.mismatch is not None for r in reports),
        exact_unguided=sum(bool(r.exact_unguided) for r in reports),
        heads_with_fragile_decisions=sum(r.own_fragile for r in reports),
        fragile_decisions=sum(len(r.fragile_levels) for r in reports),
        diverged_decisions=sum(len(r.diverged_levels) for r in reports),
        max_o_err=max((r.o_err for r in reports), default=0.0),
        max_o_rel=max((r.o_rel for r in reports), default=0.0),
        min_o_scale=min((r.o_scale for r in reports), default=0.0),
        first_mismatch=next((f"{r.qh}: {r.mismatch}" for r in reports if r.mismatch), None),
    )


def pyramid_rel_err(gpu_level: np.ndarray, oracle_level: np.ndarray) -> float:
    """max |gpu - oracle| / max |oracle| over one level of one unit."""
    scale = max(float(np.max(np.abs(oracle_level))), 1e-30)
    return float(np.max(np.abs(gpu_level.astype(np.float64) - oracle_level.astype(np.float64)))) / scale
