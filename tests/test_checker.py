"""Self-tests of the tie-aware parity checker (CPU only)."""
import copy

import numpy as np
import pytest

from diffusion_drafter_tree_amd import inputs as I
from oracle import check as C
from oracle import dartree_oracle as O
from tests._helpers import oracle_as_outputs


def _case(seed=0, **kw):
    cfg = I.small_variant("tiny", **kw)
    head = I.make_head(cfg, seed)
    rnd = I.make_round(cfg, seed, 0)
    res = O.round_all(cfg, head, rnd)
    return cfg, head, rnd, oracle_as_outputs(cfg, res)


@pytest.mark.parametrize("seed", range(6))
def test_oracle_outputs_pass(seed):
    cfg, head, rnd, out = _case(seed, n_req=2, W=4, B=12)
    rep = C.check_round(cfg, head, rnd, out)
    assert rep.tie_events_level == 0 and rep.tie_events_topB == 0
    assert rep.max_score_err < 1e-6


def test_score_error_above_tolerance_fails():
    cfg, head, rnd, out = _case(1)
    out["st_cum"][0, 2, 1] += 2e-4
    with pytest.raises(C.ParityError):
        C.check_round(cfg, head, rnd, out)


def test_swapped_node_at_clear_boundary_fails():
    cfg, head, rnd, out = _case(2)
    # replace the last kept node of depth 2 with a child the oracle pruned
    r = O.round_all(cfg, head, rnd)[0]
    kept = set((n.parent_slot, n.tok) for n in r.levels[2])
    C2 = r.cand_ids[1]
    for p in range(len(r.levels[1])):
        for c in C2:
            if (p, int(c)) not in kept:
                out["st_tok"][0, 1, cfg.W - 1] = int(c)
                out["st_parent"][0, 1, cfg.W - 1] = p
                with pytest.raises(C.ParityError):
                    C.check_round(cfg, head, rnd, out)
                return


def test_wrong_parent_pointer_and_mask_fail():
    cfg, head, rnd, out = _case(3)
    bad = copy.deepcopy(out)
    i = int(np.nonzero(bad["parent"][0] >= 0)[0][0])
    bad["parent"][0, i] = bad["parent"][0, i] + 1 if bad["parent"][0, i] + 1 < i else -1
    with pytest.raises(C.ParityError):
        C.check_round(cfg, head, rnd, bad)
    bad = copy.deepcopy(out)
    bad["mask"][0, 3, 0] ^= np.uint64(1 << 5)
    with pytest.raises(C.ParityError):
        C.check_round(cfg, head, rnd, bad)


def test_candidate_error_fails():
    cfg, head, rnd, out = _case(4)
    out["cand_ids"][0, 0, [0, 1]] = out["cand_ids"][0, 0, [1, 0]]
    with pytest.raises(C.ParityError):
        C.check_round(cfg, head, rnd, out)


def test_exact_tie_choice_is_accepted_as_tie_event():
    # two candidates of depth 1 with equal base logits and equal U rows score
    # exactly alike; W = 1 keeps the lower token in exact arithmetic, and a
    # path that kept the other one is accepted as a tie event
    cfg = I.small_variant("tiny", W=1, B=3, L=3)
    head = I.make_head(cfg, 0)
    rnd = I.make_round(cfg, 0, 0)
    lg = rnd.logits.copy()
    row = lg[0, 0]
    top = np.argsort(-row)[:2]
    a, b = sorted(top.tolist())
    row[b] = row[a]
    head.U[b] = head.U[a]
    rnd.logits = lg
    res = O.round_all(cfg, head, rnd)
    out = oracle_as_outputs(cfg, res)
    assert out["st_tok"][0, 0, 0] == a
    # emulate a path whose fp32 arithmetic preferred token b (and its subtree)
    cfg_b = cfg
    A, E, U = O.widen(head.A, "f32"), O.widen(head.E, "f32"), O.widen(head.U, "f32")
    h = np.asarray(rnd.h[0], np.float64)
    r0 = res[0]
    ids, vals = r0.cand_ids.copy(), r0.cand_vals.copy()
    root = O.Node(0, -1, 0, -1, 0.0, 0.0, h[0])
    lv1 = O.expand_level([root], 1, ids[0], vals[0], h, A, E, U, 2, cfg.beta, cfg.L)
    alt = [n for n in lv1 if n.tok == b][0]
    alt.slot = 0
    levels = [[root], [alt]]
    for d in range(2, cfg.L + 1):
        levels.append(O.expand_level(levels[-1], d, ids[d - 1], vals[d - 1], h, A, E, U, 1, cfg.beta, cfg.L))
    sel = O.select_topB(levels, cfg.B)
    em = O.emit(sel, cfg.B)
    fake = O.RequestResult(ids, vals, h, levels, sel, em, O.tree_mask(em.parent, em.n_sel, cfg.B))
    out_b = oracle_as_outputs(cfg_b, [fake])
    rep = C.check_round(cfg, head, rnd, out_b)
    assert rep.tie_events_level >= 1


def _flat_level(scores, depth=1):
    """One supertree level of oracle nodes with the given fp64 s_beta values
    (slot order = given order), children of the root."""
    return [O.Node(depth=depth, tok=10 + i, slot=i, parent_slot=0, cum=s, sbeta=s, state=None)
            for i, s in enumerate(scores)]


def _gst_of(level, W):
    L = 1
    tok = np.full((L, W), -1, np.int32)
    ps = np.full((L, W), -1, np.int32)
    cum = np.full((L, W), -np.inf, np.float32)
    sb = np.full((L, W), -np.inf, np.float32)
    for nd in level:
        tok[0, nd.slot], ps[0, nd.slot] = nd.tok, nd.parent_slot
        cum[0, nd.slot], sb[0, nd.slot] = nd.cum, nd.sbeta
    return C.GpuSupertree(tok=tok, parent_slot=ps, cum=cum, sbeta=sb, count=np.array([len(level)], np.int32))


def _selection(level, slots, B):
    chosen = [level[s] for s in slots]
    em = O.emit(chosen, B)
    score = np.array([level[em.slot[i]].sbeta if i < em.n_sel else -np.inf for i in range(B)], np.float32)
    return C.GpuSelection(n_sel=em.n_sel, tok=em.tok, depth=em.depth, parent=em.parent, score=score,
                          slot=em.slot, mask=O.tree_mask(em.parent, em.n_sel, B))


def test_topB_near_tie_that_drops_the_best_node_fails():
    # scores {0, -4, -4.00001}, B = 2: the B-th and (B+1)-th are within the
    # tolerance, but a selection of the two near-tied nodes drops the node
    # scoring 0, which beats both by 4 -- not a valid top-2 at any tolerance
    level = _flat_level([0.0, -4.0, -4.00001])
    gst = _gst_of(level, 3)
    with pytest.raises(C.ParityError):
        C.check_selection([[None], level], gst, _selection(level, [1, 2], 2), 2, 1e-4)
    # the tie choice itself (either near-tied node next to the best) is valid
    rep = C.check_selection([[None], level], gst, _selection(level, [0, 2], 2), 2, 1e-4)
    assert rep.tie_events_topB == 1
    rep = C.check_selection([[None], level], gst, _selection(level, [0, 1], 2), 2, 1e-4)
    assert rep.tie_events_topB == 0


def test_level_near_tie_that_drops_the_best_child_fails():
    # depth 1 with W = 2: make the 2nd and 3rd best children tie exactly, then
    # present a level that keeps those two and drops the clearly best child
    cfg = I.small_variant("tiny", W=2, B=4, L=3)
    head = I.make_head(cfg, 5)
    rnd = I.make_round(cfg, 5, 0)
    res = O.round_all(cfg, head, rnd)[0]
    A, E, U = O.widen(head.A, "f32"), O.widen(head.E, "f32"), O.widen(head.U, "f32")
    h = np.asarray(rnd.h[0], np.float64)
    root = O.Node(0, -1, 0, -1, 0.0, 0.0, h[0])
    ranked = O.expand_level([root], 1, res.cand_ids[0], res.cand_vals[0], h, A, E, U, cfg.K, cfg.beta, cfg.L)
    best, b, c = ranked[0].tok, ranked[1].tok, ranked[2].tok
    assert ranked[0].sbeta - ranked[1].sbeta > 1e-3   # a clearly best child
    lg = rnd.logits.copy()
    lg[0, 0, c] = lg[0, 0, b]
    rnd.logits = lg
    head.U[c] = head.U[b]
    res = O.round_all(cfg, head, rnd)[0]
    U = O.widen(head.U, "f32")
    ids, vals = res.cand_ids.copy(), res.cand_vals.copy()
    lv1 = O.expand_level([root], 1, ids[0], vals[0], h, A, E, U, cfg.K, cfg.beta, cfg.L)
    tied = sorted([n for n in lv1 if n.tok in (b, c)], key=lambda n: n.tok)
    assert tied[0].sbeta == tied[1].sbeta and lv1[0].tok == best

    def fake_with_level1(first):
        for s, nd in enumerate(first):
            nd.slot = s
        levels = [[root], first]
        for d in range(2, cfg.L + 1):
            levels.append(O.expand_level(levels[-1], d, ids[d - 1], vals[d - 1], h, A, E, U, cfg.W, cfg.beta,
                                         cfg.L))
        sel = O.select_topB(levels, cfg.B)
        em = O.emit(sel, cfg.B)
        fake = O.RequestResult(ids, vals, h, levels, sel, em, O.tree_mask(em.parent, em.n_sel, cfg.B))
        return oracle_as_outputs(cfg, [fake])

    # valid: the best child and either of the exactly tied pair
    rep = C.check_round(cfg, head, rnd, fake_with_level1([lv1[0], tied[1]]))
    assert rep.tie_events_level >= 1 and rep.tie_log
    # invalid: the tied pair without the best child (its gap to them is > tol)
    with pytest.raises(C.ParityError, match="excluded"):
        C.check_round(cfg, head, rnd, fake_with_level1([tied[0], tied[1]]))
