"""Pins of the oracle's LM-head step (the drafter's base logits, then the
candidates) and self-tests of its parity checker. CPU only."""
import numpy as np
import pytest

from diffusion_drafter_tree_amd import inputs as I
from oracle import check as C
from oracle import dartree_oracle as O


def test_one_hot_head_gives_the_closed_form():
    # Wlm[v] = s_v * e_{p(v)} with a permutation p that is not symmetric:
    # logit[i][v] = X[i][p(v)] * s_v exactly (one product); D == V so a
    # transposed operand would still multiply, and fail here
    rng = np.random.default_rng(0)
    D = V = 12
    perm = (np.arange(V) * 5 + 3) % D
    s = rng.uniform(0.5, 2.0, V)
    Wlm = np.zeros((V, D))
    Wlm[np.arange(V), perm] = s
    X = rng.standard_normal((3, D))
    got = O.lmhead_logits(X, Wlm)
    assert np.array_equal(got, X[:, perm] * s[None, :])


def test_hand_worked_candidates_with_ties():
    # D = 2, X = [1, 2]; rows chosen so the logits are 3, 5, 5, -1, 4, 5, 0
    Wlm = np.array([[1, 1], [1, 2], [3, 1], [1, -1], [0, 2], [5, 0], [0, 0]], np.float64)
    X = np.array([[1.0, 2.0]])
    ids, vals, logits = O.lmhead_topk(X, Wlm, 4)
    assert logits[0].tolist() == [3, 5, 5, -1, 4, 5, 0]
    assert ids[0].tolist() == [1, 2, 5, 4]          # the three 5s by id, then 4
    assert vals[0].tolist() == [5, 5, 5, 4]


def test_linearity_in_the_hidden_state():
    rng = np.random.default_rng(1)
    Wlm = rng.standard_normal((50, 16))
    X1, X2 = rng.standard_normal((2, 16)), rng.standard_normal((2, 16))
    assert np.allclose(O.lmhead_logits(X1 + X2, Wlm), O.lmhead_logits(X1, Wlm) + O.lmhead_logits(X2, Wlm),
                       rtol=0, atol=1e-12)


def test_generated_states_boost_their_tokens():
    cfg = I.small_variant("qwen3_4b", n_req=2, L=4, V=3000, D=256)
    W = I.make_lmhead(cfg, 0)
    X = I.make_lmhead_states(cfg, W, 0, 0)
    assert W.shape == (cfg.V, cfg.D) and W.dtype == np.uint16 and X.shape == (2, 4, cfg.D)
    assert np.array_equal(W, I.make_lmhead(cfg, 0, chunk_rows=700))   # chunking does not change the draw
    ids, vals, logits = O.lmhead_topk(O.widen(X.reshape(8, cfg.D), "bf16"), O.widen(W, "bf16"), 64)
    assert 1.5 < logits.std() < 4.0   # noise sigma = 2 plus the boosts' cross terms (~sqrt(n_boost / D))
    # most of the top 16 of each row are boosted tokens (their logit gains ~4..12)
    assert np.mean(vals[:, 15]) > np.mean(np.sort(logits, axis=1)[:, -100])


def _case(seed=2, K=16):
    cfg = I.small_variant("qwen3_4b", n_req=1, L=3, V=2000, D=128)
    W = O.widen(I.make_lmhead(cfg, seed), "bf16")
    X = O.widen(I.make_lmhead_states(cfg, I.make_lmhead(cfg, seed), seed, 0).reshape(3, cfg.D), "bf16")
    ids, vals, logits = O.lmhead_topk(X, W, K)
    return X, W, ids, vals.astype(np.float32), logits


def test_checker_accepts_the_oracle_and_fp32_rounding():
    X, W, ids, vals, _ = _case()
    rep = C.check_lmhead_topk(ids, vals, X, W, 16)
    assert rep.tie_events_level == 0 and rep.max_score_err < 1e-6


def test_checker_rejects_a_wrong_value_an_order_swap_and_a_dropped_best():
    X, W, ids, vals, logits = _case()
    bad = vals.copy()
    bad[0, 3] += 2e-4
    with pytest.raises(C.ParityError):
        C.check_lmhead_topk(ids, bad, X, W, 16)
    sw = ids.copy()
    sw[1, [0, 1]] = sw[1, [1, 0]]
    with pytest.raises(C.ParityError):
        C.check_lmhead_topk(sw, vals, X, W, 16)
    # replace the best id by the (K+1)-th: excluded beats chosen by far
    o, _ = O.topk_candidates(logits[2], 17)
    dr = ids.copy()
    dv = vals.copy()
    dr[2] = np.concatenate([o[1:16], o[16:17]])
    dv[2] = logits[2][dr[2]].astype(np.float32)
    with pytest.raises(C.ParityError):
        C.check_lmhead_topk(dr, dv, X, W, 16)


def test_checker_accepts_a_near_tie_at_the_cut_either_way():
    # make the K-th and (K+1)-th logits of row 0 equal to within 1e-6 by
    # nudging one hidden-state entry is awkward; instead nudge the head row
    X, W, ids, vals, logits = _case()
    o, ov = O.topk_candidates(logits[0], 17)
    a, b = int(o[15]), int(o[16])
    W2 = W.copy()
    j = int(np.argmax(np.abs(X[0])))
    W2[b, j] += (logits[0][a] - logits[0][b] + 3e-7) / X[0][j]   # b now 3e-7 above a
    l2 = X[0] @ W2.T
    o2, _ = O.topk_candidates(l2, 16)
    assert b in o2.tolist() and a not in o2.tolist()
    alt = np.array([v if v != b else a for v in o2.tolist()])
    alt_vals = l2[alt].astype(np.float32)
    order = np.lexsort((alt, -alt_vals.astype(np.float64)))
    ids2, vals2 = ids.copy(), vals.copy()
    ids2[0], vals2[0] = alt[order], alt_vals[order]
    rep = C.check_lmhead_topk(ids2, vals2, X, W2, 16, rows=[0])
    assert rep.tie_events_level == 1


# planted mistakes in the oracle's LM-head step, each caught by the pins above
LMHEAD_MUTANTS = {
    "untransposed_head": ("@ np.asarray(Wlm, dtype=np.float64).T", "@ np.asarray(Wlm, dtype=np.float64)"),
    "reversed_rows": ("@ np.asarray(Wlm, dtype=np.float64).T", "@ np.asarray(Wlm, dtype=np.float64)[::-1].T"),
    "one_fewer_candidate": ("ids[i], vals[i] = topk_candidates(logits[i], K)\n    return ids, vals, logits",
                            "ids[i], vals[i] = topk_candidates(logits[i], K + 1)[0][1:], topk_candidates(logits[i], K + 1)[1][1:]\n    return ids, vals, logits"),
    "dropped_state_column": ("return np.asarray(X, dtype=np.float64) @", "return np.asarray(X, dtype=np.float64)[:, ::-1] @"),
}


@pytest.mark.parametrize("name", sorted(LMHEAD_MUTANTS))
def test_lmhead_planted_mistakes_are_caught(name):
    import importlib
    src = open(O.__file__).read()
    old, new = LMHEAD_MUTANTS[name]
    assert old in src, f"mutation site for {name} not found"
    try:
        exec(compile(src.replace(old, new), O.__file__, "exec"), O.__dict__)
        caught = False
        try:
            test_one_hot_head_gives_the_closed_form()
            test_hand_worked_candidates_with_ties()
        except (AssertionError, ValueError, IndexError):
            caught = True
        assert caught, f"mutant {name} survived the pins"
    finally:
        importlib.reload(O)
