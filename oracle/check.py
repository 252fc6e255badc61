"""Tie-aware parity checker: HIP-path outputs against the CPU oracle.

TEST INFRASTRUCTURE ONLY (see oracle/dartree_oracle.py).

The HIP path computes scores in fp32, the oracle in fp64. Where two children
(or two supertree nodes) sit within the tolerance of each other at a top-W
or top-B boundary, either may legitimately be kept, and the whole subtree
below differs. The checker therefore replays the oracle level by level from
the node set the HIP path kept:

  * candidates: ids and widened logits must be bit-identical;
  * level d: the oracle scores every child of the HIP path's level d-1 in
    fp64 and ranks them. If the oracle's W-th and (W+1)-th scores are more
    than ``tol`` apart the kept sets must be identical; otherwise (a tie
    event) no child left out may outscore a kept one by more than ``tol``
    (min over kept >= max over excluded - tol, both in fp64). Each kept
    node's cum and s_beta must be within ``tol`` of the oracle's value, and
    the level must be sorted under the comparator by its own fp32 scores;
  * top-B: the same rule at the B/(B+1) boundary over the HIP path's
    supertree;
  * emission, parents and mask: bit-identical to the oracle's emission of
    the selected set (breadth-first order depends only on the set), and the
    mask to the ancestor closure of the emitted parents.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from . import dartree_oracle as O


@dataclass
class Report:
    tie_events_level: int = 0
    tie_events_topB: int = 0
    max_cum_err: float = 0.0
    max_score_err: float = 0.0
    max_h_err: float = 0.0
    nodes_checked: int = 0
    notes: List[str] = field(default_factory=list)
    tie_log: List[str] = field(default_factory=list)

    def merge(self, o: "Report") -> "Report":
        self.tie_events_level += o.tie_events_level
        self.tie_events_topB += o.tie_events_topB
        self.max_cum_err = max(self.max_cum_err, o.max_cum_err)
        self.max_score_err = max(self.max_score_err, o.max_score_err)
        self.max_h_err = max(self.max_h_err, o.max_h_err)
        self.nodes_checked += o.nodes_checked
        self.notes += o.notes
        self.tie_log += o.tie_log
        return self


class ParityError(AssertionError):
    pass


def _fail(msg):
    raise ParityError(msg)


def check_candidates(gpu_ids: np.ndarray, gpu_vals: np.ndarray, logits_f64_rows: np.ndarray, K: int, where=""):
    """Bit-exact top-K rows: gpu_ids [R][K] int, gpu_vals [R][K] fp32."""
    for i in range(logits_f64_rows.shape[0]):
        ids, vals = O.topk_candidates(logits_f64_rows[i], K)
        if not np.array_equal(np.asarray(gpu_ids[i], np.int64), ids):
            bad = np.nonzero(np.asarray(gpu_ids[i], np.int64) != ids)[0]
            _fail(f"{where} row {i}: candidate ids differ at {bad[:8]}: gpu {np.asarray(gpu_ids[i])[bad[:8]]} oracle {ids[bad[:8]]}")
        if not np.array_equal(np.asarray(gpu_vals[i], np.float64), vals):
            _fail(f"{where} row {i}: candidate logits differ")


@dataclass
class GpuSupertree:
    tok: np.ndarray          # [L][W]
    parent_slot: np.ndarray  # [L][W]
    cum: np.ndarray          # [L][W] fp32
    sbeta: np.ndarray        # [L][W] fp32
    count: np.ndarray        # [L]


@dataclass
class GpuSelection:
    n_sel: int
    tok: np.ndarray      # [B]
    depth: np.ndarray    # [B]
    parent: np.ndarray   # [B]
    score: np.ndarray    # [B] fp32
    slot: np.ndarray     # [B]  slot of the node in its supertree level
    mask: Optional[np.ndarray] = None  # [B][words] uint64


def _check_cut(chosen, score_of, tol: float, where: str, what: str):
    """A chosen subset of a pool is a valid top-n under tolerance ``tol`` iff
    no excluded member outscores a chosen one by more than ``tol``:
    min over chosen of the oracle score >= max over excluded - tol. This is
    the near-tie rule of the parity bar, applied to both sides of the cut (a
    set that keeps near-tied nodes but drops a clearly better one is
    invalid)."""
    lo_key = min(chosen, key=lambda k: score_of[k])
    excluded = [k for k in score_of if k not in chosen]
    if not excluded:
        return
    hi_key = max(excluded, key=lambda k: score_of[k])
    if score_of[lo_key] < score_of[hi_key] - tol:
        _fail(f"{where}: {what} {lo_key} scores {score_of[lo_key]:.9f} but excluded {hi_key} scores "
              f"{score_of[hi_key]:.9f} (more than tol {tol:g} better)")


def _sorted_by_comparator(sb: np.ndarray, tok: np.ndarray, ps: np.ndarray) -> bool:
    for s in range(1, sb.shape[0]):
        a = (-float(sb[s - 1]), int(tok[s - 1]), int(ps[s - 1]))
        b = (-float(sb[s]), int(tok[s]), int(ps[s]))
        if not a < b:
            return False
    return True


def replay_supertree(gst: GpuSupertree, cand_ids, cand_vals, h, A, E, U, W, beta, tol, d_lo=1, d_hi=None,
                     where="") -> (List[List[O.Node]], Report):
    """Replay levels d_lo..d_hi of the oracle from the HIP path's kept sets.
    Returns oracle nodes (fp64 scores, states) arranged in the HIP path's
    slot order, and a report."""
    rep = Report()
    L = cand_ids.shape[0]
    d_hi = L if d_hi is None else d_hi
    root = O.Node(depth=0, tok=-1, slot=0, parent_slot=-1, cum=0.0, sbeta=0.0, state=np.asarray(h[0], np.float64))
    levels = [[root]]
    for d in range(1, d_hi + 1):
        parents = levels[-1]
        C = cand_ids[d - 1]
        base = cand_vals[d - 1]
        U_rows = U[C]
        tok_pos = {int(c): k for k, c in enumerate(C)}
        scores = {}
        allsb = []
        for p in parents:
            logq = O.corrected_logprobs(base, U_rows, p.state)
            cum = p.cum + logq
            sb = cum + beta * d
            for k in range(C.shape[0]):
                key = O.node_key(sb[k], d, int(C[k]), p.slot)
                scores[(p.slot, int(C[k]))] = (float(cum[k]), float(sb[k]), key)
                allsb.append(key)
        allsb.sort()
        n_keep = min(W, len(allsb))
        oracle_set = set((k[3], k[2]) for k in allsb[:n_keep])
        cnt = int(gst.count[d - 1])
        if cnt != n_keep:
            _fail(f"{where} depth {d}: kept {cnt} nodes, expected {n_keep}")
        g_tok = np.asarray(gst.tok[d - 1][:cnt], np.int64)
        g_ps = np.asarray(gst.parent_slot[d - 1][:cnt], np.int64)
        g_cum = np.asarray(gst.cum[d - 1][:cnt], np.float64)
        g_sb = np.asarray(gst.sbeta[d - 1][:cnt], np.float64)
        gpu_set = set()
        for s in range(cnt):
            key = (int(g_ps[s]), int(g_tok[s]))
            if key not in scores:
                _fail(f"{where} depth {d} slot {s}: (parent {key[0]}, token {key[1]}) is not a child of level {d-1}")
            if key in gpu_set:
                _fail(f"{where} depth {d}: duplicate node {key}")
            gpu_set.add(key)
        if not _sorted_by_comparator(g_sb, g_tok, g_ps):
            _fail(f"{where} depth {d}: level not sorted by (s_beta desc, token asc, parent slot asc)")
        if gpu_set != oracle_set:
            w_score = -allsb[n_keep - 1][0]
            nxt = -allsb[n_keep][0] if n_keep < len(allsb) else -np.inf
            if w_score - nxt > tol:
                _fail(f"{where} depth {d}: kept set differs with a clear boundary "
                      f"(W-th {w_score:.7f}, next {nxt:.7f}); gpu-only {sorted(gpu_set - oracle_set)[:4]} "
                      f"oracle-only {sorted(oracle_set - gpu_set)[:4]}")
            _check_cut(gpu_set, {k: v[1] for k, v in scores.items()}, tol, f"{where} depth {d}", "kept")
            rep.tie_events_level += 1
            rep.tie_log.append(f"{where} depth {d}: W-th {w_score:.9f} next {nxt:.9f}")
        level = []
        for s in range(cnt):
            key = (int(g_ps[s]), int(g_tok[s]))
            ocum, osb, _ = scores[key]
            ec, es = abs(g_cum[s] - ocum), abs(g_sb[s] - osb)
            rep.max_cum_err = max(rep.max_cum_err, ec)
            rep.max_score_err = max(rep.max_score_err, es)
            if ec > tol or es > tol:
                _fail(f"{where} depth {d} slot {s}: cum {g_cum[s]:.7f} vs {ocum:.7f}, s_beta {g_sb[s]:.7f} vs {osb:.7f}")
            p = parents[key[0]]
            st = O.child_state(A, p.state, E[key[1]], h[d]) if d < L else None
            level.append(O.Node(depth=d, tok=key[1], slot=s, parent_slot=key[0], cum=ocum, sbeta=osb, state=st))
            rep.nodes_checked += 1
        levels.append(level)
    return levels, rep


def check_selection(levels: List[List[O.Node]], gst: GpuSupertree, sel: GpuSelection, B: int, tol: float,
                    where="", budget: Optional[int] = None) -> Report:
    """Global top-B over the replayed supertree, emission, and mask. ``B`` is
    the output stride; ``budget`` (default B) the number of nodes to select."""
    rep = Report()
    pool = [nd for lvl in levels[1:] for nd in lvl]
    pool_sorted = sorted(pool, key=lambda nd: O.node_key(nd.sbeta, nd.depth, nd.tok, nd.parent_slot))
    n_exp = min(B if budget is None else budget, len(pool))
    if int(sel.n_sel) != n_exp:
        _fail(f"{where}: n_sel {sel.n_sel}, expected {n_exp}")
    n = n_exp
    oracle_set = set((nd.depth, nd.slot) for nd in pool_sorted[:n])
    g_depth = np.asarray(sel.depth[:n], np.int64)
    g_slot = np.asarray(sel.slot[:n], np.int64)
    gpu_set = set(zip(g_depth.tolist(), g_slot.tolist()))
    if len(gpu_set) != n:
        _fail(f"{where}: duplicate selected nodes")
    by_key = {(nd.depth, nd.slot): nd for nd in pool}
    for k in gpu_set:
        if k not in by_key:
            _fail(f"{where}: selected node {k} is not in the supertree")
    if gpu_set != oracle_set:
        b_score = pool_sorted[n - 1].sbeta
        nxt = pool_sorted[n].sbeta if n < len(pool_sorted) else -np.inf
        if b_score - nxt > tol:
            _fail(f"{where}: top-B set differs with a clear boundary (B-th {b_score:.7f}, next {nxt:.7f})")
        _check_cut(gpu_set, {k: nd.sbeta for k, nd in by_key.items()}, tol, where, "selected")
        rep.tie_events_topB += 1
        rep.tie_log.append(f"{where} top-B: B-th {b_score:.9f} next {nxt:.9f}")
    # prefix closure of the HIP path's own selection
    for (d, s) in gpu_set:
        if d > 1 and (d - 1, by_key[(d, s)].parent_slot) not in gpu_set:
            _fail(f"{where}: selection not prefix-closed at node {(d, s)}")
    # emission: canonical breadth-first order of the selected set
    chosen = [by_key[k] for k in gpu_set]
    em = O.emit(chosen, B)
    for name, g, o in (("tok", sel.tok, em.tok), ("depth", sel.depth, em.depth),
                       ("parent", sel.parent, em.parent), ("slot", sel.slot, em.slot)):
        if not np.array_equal(np.asarray(g, np.int64), o):
            bad = np.nonzero(np.asarray(g, np.int64) != o)[0]
            _fail(f"{where}: emitted {name} differs at {bad[:8]}: gpu {np.asarray(g)[bad[:8]]} oracle {o[bad[:8]]}")
    g_score = np.asarray(sel.score, np.float64)
    for i in range(n):
        d, s = int(sel.depth[i]), int(sel.slot[i])
        e = abs(g_score[i] - by_key[(d, s)].sbeta)
        rep.max_score_err = max(rep.max_score_err, e)
        if e > tol:
            _fail(f"{where}: emitted score {i} off by {e}")
        if np.float32(g_score[i]) != np.float32(gst.sbeta[d - 1][s]):
            _fail(f"{where}: emitted score {i} is not the supertree's s_beta")
    if n < B and not np.all(np.isneginf(g_score[n:])):
        _fail(f"{where}: score padding is not -inf")
    if sel.mask is not None:
        m = O.tree_mask(np.asarray(sel.parent, np.int64), n, B)
        if not np.array_equal(np.asarray(sel.mask, np.uint64), m):
            bad = np.nonzero(np.any(np.asarray(sel.mask, np.uint64) != m, axis=1))[0]
            _fail(f"{where}: mask rows differ at {bad[:8]}")
    return rep


def widen_head(head):
    """The head's weights widened exactly to float64: (A, E, U, Pt or None)."""
    wd = head.dtype
    return (O.widen(head.A, wd), O.widen(head.E, wd), O.widen(head.U, wd),
            None if head.Pt is None else O.widen(head.Pt, wd))


def check_round(cfg, head, rnd, gpu: Dict[str, np.ndarray], tol: float = 1e-4,
                oracle_h: Optional[np.ndarray] = None, requests=None, widths=None, budgets=None,
                widened=None) -> Report:
    """Full-round parity for every request. ``gpu`` holds numpy copies of the
    HIP path's outputs: cand_ids, cand_logit [n][L][K]; h [n][L][r] (when
    D > 0); st_tok, st_parent, st_cum, st_sbeta [n][L][W]; st_count [n][L];
    n_sel [n]; tok, depth, parent, score, slot [n][B]; mask [n][B][words].
    ``requests`` restricts the check to a sample of requests; ``widths`` and
    ``budgets`` give per-request W_q and B_q (default cfg.W and cfg.B; the
    output strides stay cfg.W and cfg.B). ``widened`` may carry
    ``widen_head(head)`` computed once for many calls."""
    wd = head.dtype
    A, E, U, Pt = widen_head(head) if widened is None else widened
    qs = list(range(cfg.n_req)) if requests is None else list(requests)
    logits = {q: O.widen(rnd.logits[q], cfg.logits_dtype) for q in qs}
    if cfg.D > 0:
        h_all = {q: (oracle_h[q] if oracle_h is not None else O.head_states(O.widen(rnd.H[q], wd), Pt)) for q in qs}
    else:
        h_all = {q: np.asarray(rnd.h[q], np.float64) for q in qs}
    rep = Report()
    for q in qs:
        where = f"[{cfg.name} req {q}]"
        check_candidates(gpu["cand_ids"][q], gpu["cand_logit"][q], logits[q], cfg.K, where)
        if cfg.D > 0 and "h" in gpu:
            eh = float(np.max(np.abs(np.asarray(gpu["h"][q], np.float64) - h_all[q])))
            rep.max_h_err = max(rep.max_h_err, eh)
            if eh > tol:
                _fail(f"{where}: head states off by {eh}")
        ids = np.asarray(gpu["cand_ids"][q], np.int64)
        vals = np.asarray(gpu["cand_logit"][q], np.float64)
        gst = GpuSupertree(tok=gpu["st_tok"][q], parent_slot=gpu["st_parent"][q], cum=gpu["st_cum"][q],
                           sbeta=gpu["st_sbeta"][q], count=gpu["st_count"][q])
        wq = cfg.W if widths is None else int(widths[q])
        bq = cfg.B if budgets is None else int(budgets[q])
        levels, r1 = replay_supertree(gst, ids, vals, h_all[q], A, E, U, wq, cfg.beta, tol, where=where)
        rep.merge(r1)
        if "n_sel" in gpu:
            sel = GpuSelection(n_sel=int(gpu["n_sel"][q]), tok=gpu["tok"][q], depth=gpu["depth"][q],
                               parent=gpu["parent"][q], score=gpu["score"][q], slot=gpu["slot"][q],
                               mask=gpu["mask"][q] if "mask" in gpu else None)
            for i in range(sel.n_sel, cfg.B):
                if not (sel.tok[i] == -1 and sel.depth[i] == 0 and sel.parent[i] == -2 and sel.slot[i] == -1):
                    _fail(f"{where}: padding wrong at {i}")
            rep.merge(check_selection(levels, gst, sel, cfg.B, tol, where, budget=bq))
    return rep


def check_lmhead_topk(gpu_ids: np.ndarray, gpu_vals: np.ndarray, X: np.ndarray, Wlm: np.ndarray, K: int,
                      tol: float = 1e-4, rows=None, where="") -> Report:
    """Fused LM head + top-K against the oracle's fp64 logits. The HIP path
    accumulates the logits in fp32, so near-ties (within ``tol``) at the K-th
    logit may legitimately resolve either way. Per row: ids distinct and in
    range; each value within ``tol`` of the oracle's logit of its id; the
    row's order follows the HIP path's own values (descending, ids ascending
    among equal values) and never inverts two oracle logits by more than
    ``tol``; and the set is a valid top-K (no excluded token's logit beats a
    chosen one's by more than ``tol``). A set that differs from the oracle's
    counts as a tie event. ``X`` [R][D] and ``Wlm`` [V][D] are float64."""
    rep = Report()
    rows = range(X.shape[0]) if rows is None else rows
    for i in rows:
        logits = np.asarray(X[i], np.float64) @ np.asarray(Wlm, np.float64).T
        ids = np.asarray(gpu_ids[i], np.int64)
        vals = np.asarray(gpu_vals[i], np.float64)
        V = logits.shape[0]
        n = min(K, V)
        w = f"{where} row {i}"
        if np.any(ids[:n] < 0) or np.any(ids[:n] >= V) or len(set(ids[:n].tolist())) != n:
            _fail(f"{w}: ids out of range or repeated: {ids[:8]}")
        err = np.abs(vals[:n] - logits[ids[:n]])
        rep.max_score_err = max(rep.max_score_err, float(err.max()))
        if err.max() > tol:
            j = int(err.argmax())
            _fail(f"{w}: value of id {ids[j]} is {vals[j]:.7f}, oracle {logits[ids[j]]:.7f}")
        for j in range(1, n):
            if not (vals[j - 1] > vals[j] or (vals[j - 1] == vals[j] and ids[j - 1] < ids[j])):
                _fail(f"{w}: order broken at {j}: ({vals[j-1]}, {ids[j-1]}) then ({vals[j]}, {ids[j]})")
            if logits[ids[j]] > logits[ids[j - 1]] + tol:
                _fail(f"{w}: positions {j-1}, {j} invert oracle logits by more than tol")
        o_ids, _ = O.topk_candidates(logits, n)
        chosen = set(ids[:n].tolist())
        if chosen != set(o_ids.tolist()):
            score = {v: float(logits[v]) for v in range(V)}
            _check_cut(chosen, score, tol, w, "chosen")
            rep.tie_events_level += 1
            rep.tie_log.append(f"{w}: K-th oracle logit {logits[o_ids[-1]]:.9f}")
        rep.nodes_checked += n
    return rep

