"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a worked
example derived by hand from the score equation, closed forms, brute-force
enumeration, the literal heaps, or special cases that reduce to a simpler
object. A plausible mistake (a dropped term, a wrong sign, a wrong row or
index, a transposed operand) fails at least one of them; the mutation tests at
the end plant such mistakes in the oracle and check that they are caught.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import dartree_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(seed, V=40, L=4, K=5, r=6, scale_u=1.0, A_zero=False, E_zero=False, U_zero=False, ties=False):
    rng = np.random.default_rng(seed)
    logits = rng.normal(0, 2, (L, V))
    if ties:
        logits = np.round(logits * 2) / 2
    A = np.zeros((r, r)) if A_zero else rng.normal(0, 1 / math.sqrt(r), (r, r))
    E = np.zeros((V, r)) if E_zero else rng.normal(0, 1, (V, r))
    U = np.zeros((V, r)) if U_zero else rng.normal(0, scale_u / math.sqrt(r), (V, r))
    h = rng.normal(0, 1, (L, r))
    return logits, h, A, E, U


def cands(logits, K):
    L = logits.shape[0]
    ids = np.empty((L, K), np.int64)
    vals = np.empty((L, K))
    for i in range(L):
        ids[i], vals[i] = O.topk_candidates(logits[i], K)
    return ids, vals


# --------------------------------------------------------------------------
# hand-worked example (score equation of the blog's section 3.1)
# --------------------------------------------------------------------------
def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_tiny.json")))
    logits = np.array(g["logits"])
    r, V = g["r"], g["V"]
    A = np.ones((r, r)) * 0.3
    E = np.arange(V * r, dtype=float).reshape(V, r) * 0.1
    U = np.zeros((V, r))
    h = np.ones((g["L"], r))
    res = O.round_one_request(logits, h, A, E, U, g["K"], g["W"], g["B"], g["beta"])
    ex = g["expected"]
    assert res.cand_ids.tolist() == ex["cand_ids"]
    ln = math.log
    l1 = [ln(3 / 4) - 0.5, ln(1 / 4) - 0.5]
    l2 = [ln(3 / 4) + ln(4 / 5) - 1, ln(1 / 4) + ln(4 / 5) - 1]
    assert [n.tok for n in res.levels[1]] == ex["level1"]["tok"]
    assert np.allclose([n.sbeta for n in res.levels[1]], l1, atol=1e-12)
    paths = [[res.levels[1][n.parent_slot].tok, n.tok] for n in res.levels[2]]
    assert paths == ex["level2"]["path"]
    assert np.allclose([n.sbeta for n in res.levels[2]], l2, atol=1e-12)
    em = res.emitted
    assert em.n_sel == ex["n_sel"]
    assert em.tok[:3].tolist() == ex["tok"]
    assert em.depth[:3].tolist() == ex["depth"]
    assert em.parent[:3].tolist() == ex["parent"]
    assert np.allclose(em.score[:3], [l1[0], l1[1], ln(3 / 4) + ln(4 / 5) - 1], atol=1e-12)
    assert [int(x) for x in res.mask[:3, 0]] == ex["mask_rows"]


# --------------------------------------------------------------------------
# top-K: rank-count definition on tie-heavy rows
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(30))
def test_topk_matches_rank_count(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(1, 60))
    K = int(rng.integers(1, V + 1))
    row = rng.integers(-3, 4, V).astype(float) * 0.5   # many exact ties
    if seed % 5 == 0:
        row[rng.integers(0, V, max(1, V // 4))] = -0.0
    ids, vals = O.topk_candidates(row, K)
    # element i is selected iff fewer than K elements beat it, where j beats
    # i when row[j] > row[i] or (row[j] == row[i] and j < i)
    rank = [sum(1 for j in range(V) if row[j] > row[i] or (row[j] == row[i] and j < i)) for i in range(V)]
    expect = sorted(range(V), key=lambda i: rank[i])[:K]
    assert ids.tolist() == expect
    assert vals.tolist() == [row[i] for i in expect]
    assert sorted(rank) == list(range(V))


# --------------------------------------------------------------------------
# log-softmax closed form
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(10))
def test_log_softmax_closed_form(seed):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 5, int(rng.integers(1, 100)))
    lq = O.log_softmax(z)
    assert np.all(lq <= 0)
    assert abs(np.sum(np.exp(lq)) - 1) < 1e-12
    # differences of log q equal differences of z (q proportional to e^z)
    assert np.allclose(lq - lq[0], z - z[0], atol=1e-12)
    # two candidates: q = sigmoid(z0 - z1)
    a, b = rng.normal(0, 3, 2)
    lq2 = O.log_softmax(np.array([a, b]))
    assert abs(lq2[0] - (-math.log1p(math.exp(b - a)))) < 1e-12


# --------------------------------------------------------------------------
# head input projection and the state recursion
# --------------------------------------------------------------------------
def test_head_states_onehot_and_linearity():
    rng = np.random.default_rng(3)
    D, r = 9, 5
    Pt = rng.normal(0, 1, (r, D))           # Pt[j][i] = P[i][j]
    H = np.eye(D)
    h = O.head_states(H, Pt)
    # H = e_i gives row i of P, i.e. column i of Pt
    assert np.array_equal(h, Pt.T)
    H1, H2 = rng.normal(0, 1, (4, D)), rng.normal(0, 1, (4, D))
    assert np.allclose(O.head_states(2 * H1 - 3 * H2, Pt), 2 * O.head_states(H1, Pt) - 3 * O.head_states(H2, Pt))


def test_state_is_tanh_h_when_A_and_E_vanish():
    logits, h, A, E, U = rand_problem(5, A_zero=True, E_zero=True)
    ids, vals = cands(logits, 5)
    levels = O.build_supertree(ids, vals, h, A, E, U, W=3, beta=-0.1)
    L = logits.shape[0]
    assert np.array_equal(levels[0][0].state, h[0])
    for d in range(1, L):
        for nd in levels[d]:
            assert np.allclose(nd.state, np.tanh(h[d]), atol=0, rtol=0)
    assert all(nd.state is None for nd in levels[L])


def test_state_recursion_chain_explicit():
    # W = 1 makes a single chain; its states follow s_d = tanh(A s_{d-1} + E[u_d] + h_d)
    logits, h, A, E, U = rand_problem(8)
    ids, vals = cands(logits, 5)
    levels = O.build_supertree(ids, vals, h, A, E, U, W=1, beta=-0.2)
    s = h[0]
    for d in range(1, logits.shape[0]):
        nd = levels[d][0]
        s = np.tanh(A.dot(s) + E[nd.tok] + h[d])
        assert np.allclose(nd.state, s, atol=1e-14)


def test_U_zero_logq_is_base_softmax():
    logits, h, A, E, U = rand_problem(11, U_zero=True)
    K = 5
    ids, vals = cands(logits, K)
    levels = O.build_supertree(ids, vals, h, A, E, U, W=50, beta=0.0)
    for nd in levels[1]:
        k = list(ids[0]).index(nd.tok)
        p = np.exp(vals[0]) / np.exp(vals[0]).sum()
        assert abs(nd.cum - math.log(p[k])) < 1e-12


# --------------------------------------------------------------------------
# U = 0: the beam is exact, so level d is the top-W of all K^d sequences
# --------------------------------------------------------------------------
def brute_force_levels(logits, K, W, beta):
    """Enumerate every sequence of candidates (U = 0: q_d does not depend on
    the prefix) and take the W best per length under the comparator, with
    ties broken by token and then recursively by the prefix."""
    L = logits.shape[0]
    cand = []
    for i in range(L):
        order = sorted(range(logits.shape[1]), key=lambda j: (-logits[i, j], j))[:K]
        v = np.array([logits[i, j] for j in order])
        q = np.exp(v - v.max()) / np.exp(v - v.max()).sum()
        cand.append((order, np.log(q)))
    out = {}
    for d in range(1, L + 1):
        seqs = []
        for combo in itertools.product(range(K), repeat=d):
            cum = 0.0
            key_tail = ()
            toks = []
            for i, k in enumerate(combo):
                cum = cum + cand[i][1][k]
                toks.append(cand[i][0][k])
            sb = cum + beta * d
            # comparator key built from the last position outwards
            key = ()
            c2 = 0.0
            partial = []
            for i, k in enumerate(combo):
                c2 = c2 + cand[i][1][k]
                partial.append((-(c2 + beta * (i + 1)), cand[i][0][k]))
            for item in partial:
                key = (item[0], item[1], key)
            seqs.append(((-sb, toks[-1], key), tuple(toks), cum, sb))
        seqs.sort(key=lambda s: s[0])
        out[d] = seqs[:W]
    return out


@pytest.mark.parametrize("seed,W,beta", [(s, w, b) for s in range(4) for w in (1, 2, 3, 7) for b in (0.0, -0.1, -5.0)])
def test_U_zero_beam_equals_brute_force(seed, W, beta):
    K, L = 4, 4
    logits, h, A, E, U = rand_problem(100 + seed, V=12, L=L, K=K, U_zero=True)
    ids, vals = cands(logits, K)
    levels = O.build_supertree(ids, vals, h, A, E, U, W=W, beta=beta)
    bf = brute_force_levels(logits, K, W, beta)

    def path(d, nd):
        toks = [nd.tok]
        while d > 1:
            nd = levels[d - 1][nd.parent_slot]
            d -= 1
            toks.append(nd.tok)
        return tuple(reversed(toks))

    for d in range(1, L + 1):
        got = [(path(d, nd), nd.cum, nd.sbeta) for nd in levels[d]]
        exp = [(s[1], s[2], s[3]) for s in bf[d]]
        assert [g[0] for g in got] == [e[0] for e in exp], f"depth {d}"
        assert np.allclose([g[1] for g in got], [e[1] for e in exp], atol=1e-12)
        assert np.allclose([g[2] for g in got], [e[2] for e in exp], atol=1e-12)


# --------------------------------------------------------------------------
# W = 1: one greedy corrected chain (Domino's single chain)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(8))
def test_W1_is_greedy_chain(seed):
    logits, h, A, E, U = rand_problem(200 + seed, V=30, L=6, K=6)
    K, B = 6, 4
    res = O.round_one_request(logits, h, A, E, U, K, 1, B, -0.3)
    s = h[0]
    chain = []
    cum = 0.0
    for d in range(1, 7):
        order = sorted(range(30), key=lambda j: (-logits[d - 1, j], j))[:K]
        z = [logits[d - 1, j] + float(U[j].dot(s)) for j in order]
        best = max(range(K), key=lambda k: (z[k], -order[k]))
        m = max(z)
        cum += z[best] - (m + math.log(sum(math.exp(x - m) for x in z)))
        chain.append((order[best], cum))
        if d < 6:
            s = np.tanh(A.dot(s) + E[order[best]] + h[d])
    assert [lv[0].tok for lv in res.levels[1:]] == [c[0] for c in chain]
    assert np.allclose([lv[0].cum for lv in res.levels[1:]], [c[1] for c in chain], atol=1e-10)
    assert res.emitted.n_sel == min(B, 6)
    assert res.emitted.tok[:B].tolist() == [c[0] for c in chain[:B]]
    assert res.emitted.parent[:B].tolist() == [-1] + list(range(B - 1))


# --------------------------------------------------------------------------
# Lemma 1: deferred top-B equals best-first heap pops on the supertree
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed,beta", [(s, b) for s in range(12) for b in (0.0, -0.1, -0.5, -5.0)])
def test_lemma1_heap_equals_deferred(seed, beta):
    rng = np.random.default_rng(seed)
    W = int(rng.integers(1, 6))
    B = int(rng.integers(1, 20))
    logits, h, A, E, U = rand_problem(300 + seed, V=25, L=5, K=5, ties=(seed % 3 == 0))
    ids, vals = cands(logits, 5)
    levels = O.build_supertree(ids, vals, h, A, E, U, W=W, beta=beta)
    deferred = O.select_topB(levels, B)
    heap = O.heap_materialized(levels, B)
    assert [(n.depth, n.slot) for n in heap] == [(n.depth, n.slot) for n in deferred]
    sel = set((n.depth, n.slot) for n in deferred)
    for n in deferred:
        assert n.depth == 1 or (n.depth - 1, n.parent_slot) in sel     # prefix closed
    assert len(deferred) == min(B, sum(len(l) for l in levels[1:])) <= B


# --------------------------------------------------------------------------
# W >= B: deferred construction equals the serial "pop then correct" heap
# over the full tree (derived: a node of the full-tree top-B can only be
# pruned at its depth if W >= B better nodes of that depth exist, all of them
# in the top-B, which would make it more than B)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed,beta", [(s, b) for s in range(10) for b in (0.0, -0.15, -1.0)])
def test_deferred_equals_serial_heap_when_W_ge_B(seed, beta):
    K, L, B = 6, 6, 12
    W = B + (seed % 3)
    logits, h, A, E, U = rand_problem(400 + seed, V=20, L=L, K=K, scale_u=3.0)
    ids, vals = cands(logits, K)
    levels = O.build_supertree(ids, vals, h, A, E, U, W=W, beta=beta)
    deferred = O.select_topB(levels, B)
    serial = O.heap_serial_full(ids, vals, h, A, E, U, beta, B)

    def path_st(n):
        toks = []
        d = n.depth
        while d >= 1:
            toks.append(n.tok)
            n = levels[d - 1][n.parent_slot] if d > 1 else None
            d -= 1
        return tuple(reversed(toks))

    def path_full(n):
        toks = []
        while n.depth >= 1:
            toks.append(n.tok)
            n = n.parent
        return tuple(reversed(toks))

    assert [path_st(n) for n in deferred] == [path_full(n) for n in serial]
    assert np.allclose([n.sbeta for n in deferred], [n.sbeta for n in serial], atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_budgets_nest_and_stay_prefix_closed(seed):
    """A per-request budget b <= B selects the first b nodes of the budget-B
    ranking (the comparator is a total order), and every such prefix is an
    ancestor-closed tree for beta <= 0 (Lemma 1 at each budget); the b-node
    tree is what b best-first heap pops give."""
    logits, h, A, E, U = rand_problem(500 + seed, V=30, L=5, K=5, ties=(seed % 2 == 0))
    ids, vals = cands(logits, 5)
    levels = O.build_supertree(ids, vals, h, A, E, U, W=4, beta=-0.2)
    full = O.select_topB(levels, 18)
    for b in range(1, 19):
        sel = O.select_topB(levels, b)
        assert [(n.depth, n.slot) for n in sel] == [(n.depth, n.slot) for n in full[:b]]
        assert [(n.depth, n.slot) for n in O.heap_materialized(levels, b)] == [(n.depth, n.slot) for n in sel]
        keys = set((n.depth, n.slot) for n in sel)
        for n in sel:
            assert n.depth == 1 or (n.depth - 1, n.parent_slot) in keys


def _same_token_parent_pairs(levels):
    """(equal, differing) counts over pairs of kept nodes of one depth whose
    parents differ but carry the same token, comparing the child's log q."""
    eq = diff = 0
    for d in range(2, len(levels)):
        seen = {}
        for nd in levels[d]:
            p = levels[d - 1][nd.parent_slot]
            key, lq = (p.tok, nd.tok), nd.cum - p.cum
            if key in seen and seen[key][0] != nd.parent_slot:
                if abs(seen[key][1] - lq) <= 1e-12:
                    eq += 1
                else:
                    diff += 1
            seen.setdefault(key, (nd.parent_slot, lq))
    return eq, diff


def test_markov_head_children_depend_on_parent_token_only():
    """The Markov-head variant (the child distribution conditioned on the
    parent token only) is the head with A = 0: then two parents of one depth
    with the same token give every child the same log q. With the recurrence
    (A != 0) the parent's path matters and such pairs differ."""
    logits, h, A, E, U = rand_problem(91, V=12, L=5, K=6, r=6)
    ids, vals = cands(logits, 6)
    lv0 = O.build_supertree(ids, vals, h, np.zeros_like(A), E, U, W=20, beta=-0.1)
    eq, diff = _same_token_parent_pairs(lv0)
    assert eq > 0 and diff == 0
    lv1 = O.build_supertree(ids, vals, h, A, E, U, W=20, beta=-0.1)
    eq, diff = _same_token_parent_pairs(lv1)
    assert diff > 0


def test_whole_supertree_selected_when_WL_le_B():
    logits, h, A, E, U = rand_problem(77, V=30, L=5, K=6)
    W, L = 3, 5
    res = O.round_one_request(logits, h, A, E, U, 6, W, W * L + 2, -0.1)
    assert res.emitted.n_sel == W * L
    assert len(res.selected) == sum(len(l) for l in res.levels[1:])


def test_very_negative_beta_is_depth_major():
    logits, h, A, E, U = rand_problem(78, V=30, L=5, K=6)
    res = O.round_one_request(logits, h, A, E, U, 6, 3, 8, -1e3)
    assert [n.depth for n in res.selected] == [1, 1, 1, 2, 2, 2, 3, 3]


# --------------------------------------------------------------------------
# emission and mask
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(10))
def test_emission_and_mask_invariants(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 130))
    logits, h, A, E, U = rand_problem(500 + seed, V=40, L=8, K=6)
    res = O.round_one_request(logits, h, A, E, U, 6, 20, B, -0.1)
    em, m = res.emitted, res.mask
    n = em.n_sel
    words = (B + 63) // 64
    assert m.shape == (B, words)
    for i in range(n):
        p = em.parent[i]
        assert -1 <= p < i
        assert em.depth[i] == (1 if p == -1 else em.depth[p] + 1)
        bits = sum(bin(int(w)).count("1") for w in m[i])
        assert bits == em.depth[i]
        assert (int(m[i, i // 64]) >> (i % 64)) & 1
        if p >= 0:
            assert np.all((m[i] & m[p]) == m[p])
        # lower triangular: no bit above the diagonal
        for j in range(i + 1, B):
            assert not (int(m[i, j // 64]) >> (j % 64)) & 1
    assert np.all(m[n:] == 0)
    assert np.all(em.tok[n:] == -1) and np.all(em.parent[n:] == -2) and np.all(np.isneginf(em.score[n:]))
    # breadth-first: depth non-decreasing, then parent index, then token
    keys = [(em.depth[i], em.parent[i], em.tok[i]) for i in range(n)]
    assert keys == sorted(keys)
    # the mask built row by row from parent rows equals the ancestor walk
    m2 = np.zeros_like(m)
    for i in range(n):
        if em.parent[i] >= 0:
            m2[i] = m2[em.parent[i]]
        m2[i, i // 64] |= np.uint64(1) << np.uint64(i % 64)
    assert np.array_equal(m, m2)


# --------------------------------------------------------------------------
# equal scores of a parent and its child: depth breaks the tie (prefix closure)
# --------------------------------------------------------------------------
def test_equal_parent_child_score_depth_tiebreak():
    # base logits [0, -800] over K = 2 give log q = [0, -800] exactly in
    # float64, so with beta = 0 the best child scores exactly as its parent
    V, L, r = 4, 3, 2
    logits = np.full((L, V), -900.0)
    logits[:, 0] = 0.0
    logits[:, 1] = -800.0
    h = np.zeros((L, r)); A = np.zeros((r, r)); E = np.zeros((V, r)); U = np.zeros((V, r))
    for B in (1, 2, 3):
        res = O.round_one_request(logits, h, A, E, U, 2, 2, B, 0.0)
        assert [n.depth for n in res.selected] == list(range(1, B + 1))
        assert all(n.sbeta == 0.0 for n in res.selected)
        assert res.emitted.parent[:B].tolist() == [-1] + list(range(B - 1))


# --------------------------------------------------------------------------
# planted mistakes must be caught by the pins above
# --------------------------------------------------------------------------
import importlib

MUTANTS = {
    "drop_lse": ("return z - (m + np.log(np.sum(np.exp(z - m))))", "return z - m"),
    "beta_sign": ("sb = cum + beta * d", "sb = cum - beta * d"),
    "drop_parent_cum": ("cum = p.cum + logq", "cum = logq"),
    "wrong_h_row": ("child_state(A, p.state, E[tok], h[d])", "child_state(A, p.state, E[tok], h[d - 1])"),
    "transposed_A": ("np.tanh(A @ s_parent + e_row + h_d)", "np.tanh(A.T @ s_parent + e_row + h_d)"),
    "E_for_U": ("U_rows = U[C]", "U_rows = E[C]"),
    "token_desc_tiebreak": ("order = np.lexsort((ids, -v))", "order = np.lexsort((-ids, -v))"),
    "wrong_logits_row": ("cand_ids[d - 1], cand_vals[d - 1], h, A, E, U, W, beta, L)",
                         "cand_ids[d % L], cand_vals[d % L], h, A, E, U, W, beta, L)"),
    "keep_W_minus_1": ("children[:W]", "children[:max(W - 1, 1)]"),
    "depth_desc_tiebreak": ("return (-sbeta, depth, tok, parent_slot)", "return (-sbeta, -depth, tok, parent_slot)"),
    "emit_token_first": ("nodes.sort(key=lambda nd: (pidx(nd), nd.tok))", "nodes.sort(key=lambda nd: (nd.tok, pidx(nd)))"),
    "mask_without_self": ("        j = i\n        while j >= 0:", "        j = int(parent[i])\n        while j >= 0:"),
    "projection_untransposed": ("@ np.asarray(Pt, dtype=np.float64).T", "@ np.asarray(Pt, dtype=np.float64).T[::-1]"),
}


def _run_pins():
    test_hand_worked_example()
    test_equal_parent_child_score_depth_tiebreak()
    test_head_states_onehot_and_linearity()
    for s in range(5):
        test_topk_matches_rank_count(s)
    for s in range(2):
        test_W1_is_greedy_chain(s)
        for b in (0.0, -0.1):
            test_deferred_equals_serial_heap_when_W_ge_B(s, b)
        test_emission_and_mask_invariants(s)
    test_U_zero_beam_equals_brute_force(0, 2, -0.1)
    test_state_is_tanh_h_when_A_and_E_vanish()
    test_state_recursion_chain_explicit()
    test_U_zero_logq_is_base_softmax()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name):
    src = open(O.__file__).read()
    old, new = MUTANTS[name]
    assert old in src, f"mutation site for {name} not found"
    try:
        exec(compile(src.replace(old, new), O.__file__, "exec"), O.__dict__)
        caught = False
        try:
            _run_pins()
        except (AssertionError, KeyError, IndexError, ValueError):
            caught = True
        assert caught, f"mutant {name} survived the pins"
    finally:
        importlib.reload(O)


def test_unmutated_oracle_passes_pin_set():
    _run_pins()


# ---- verification consumer (blog section 3.2; readings R10-R12) -------------
def _hand_tree():
    # emitted breadth-first: 0:(5,d1) 1:(7,d1) 2:(3,d2,p0) 3:(9,d2,p0) 4:(3,d2,p1) 5:(4,d3,p4)
    tok = np.array([5, 7, 3, 9, 3, 4, -1, -1])
    dep = np.array([1, 1, 2, 2, 2, 3, 0, 0])
    par = np.array([-1, -1, 0, 0, 1, 4, -2, -2])
    return tok, dep, par, 6


@pytest.mark.parametrize("target,tau,nodes", [
    ([7, 3, 4, 8], 4, [1, 4, 5]),   # the whole deepest path, then the bonus token
    ([5, 3, 1, 1], 3, [0, 2]),
    ([2, 3, 4, 8], 1, []),          # nothing accepted: the target's own token only
    ([7, 9, 4, 8], 2, [1]),         # 9 sits under node 0, not under the accepted node 1
])
def test_accept_longest_hand_tree(target, tau, nodes):
    tok, dep, par, n = _hand_tree()
    t, path = O.accept_longest(tok, dep, par, n, np.array(target))
    assert t == tau and path == nodes


def _random_tree(rng, n, B):
    par = np.full(B, -2)
    for i in range(n):
        par[i] = -1 if i < 3 else int(rng.integers(-1, i))
    return par


def test_tree_attention_uniform_scores_give_the_masked_mean():
    """K = 0: every allowed score is 0, so each row is the plain mean of the V
    rows its mask allows (computed here as a 0/1 matrix product)."""
    rng = np.random.default_rng(5)
    B, n, dh = 24, 20, 16
    par = _random_tree(rng, n, B)
    mask = O.tree_mask(par, n, B)
    M = np.array([[(int(mask[i, j // 64]) >> (j % 64)) & 1 for j in range(B)] for i in range(B)], float)
    Q, V = rng.standard_normal((B, dh)), rng.standard_normal((B, dh))
    out = O.tree_attention(Q, np.zeros((B, dh)), V, mask, n)
    exp = (M @ V)[:n] / M.sum(axis=1)[:n, None]
    assert np.allclose(out[:n], exp, atol=1e-12)
    assert np.all(out[n:] == 0)


def test_tree_attention_depth_one_nodes_see_only_themselves():
    rng = np.random.default_rng(6)
    B, n, dh = 16, 12, 8
    par = _random_tree(rng, n, B)
    mask = O.tree_mask(par, n, B)
    Q, K, V = (rng.standard_normal((B, dh)) for _ in range(3))
    out = O.tree_attention(Q, K, V, mask, n)
    for i in range(n):
        if par[i] == -1:
            assert np.array_equal(out[i], V[i])


def test_tree_attention_scale_is_one_over_sqrt_dh():
    """Duplicating every column of Q and K doubles the dot products while dh
    doubles, so the logits grow by sqrt(2): the same as scaling Q and K by
    2^(1/4) at the original width."""
    rng = np.random.default_rng(7)
    B, n, dh = 16, 14, 8
    par = _random_tree(rng, n, B)
    mask = O.tree_mask(par, n, B)
    Q, K, V = (rng.standard_normal((B, dh)) for _ in range(3))
    wide = O.tree_attention(np.hstack([Q, Q]), np.hstack([K, K]), np.hstack([V, V]), mask, n)[:, :dh]
    scaled = O.tree_attention(Q * 2 ** 0.25, K * 2 ** 0.25, V, mask, n)
    assert np.allclose(wide, scaled, atol=1e-12)


# ----------------------------------------------------------------------------
# the oracle's exact widening of bf16 bit patterns, pinned to the bfloat16
# definition (1 sign bit, 8 exponent bits with bias 127, 7 fraction bits; the
# value is (-1)^s * 2^(e-127) * (1 + f/128) for 0 < e < 255 and
# (-1)^s * 2^-126 * (f/128) for e = 0), not to the float32 bit view the
# oracle uses
# ----------------------------------------------------------------------------
def _bf16_value_by_definition(bits: int) -> float:
    s, e, f = bits >> 15, (bits >> 7) & 0xFF, bits & 0x7F
    assert e != 0xFF
    mag = math.ldexp(1.0 + f / 128.0, e - 127) if e else math.ldexp(f / 128.0, -126)
    return -mag if s else mag


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xC020, -2.5), (0x4049, 3.140625), (0x3F81, 1.0078125), (0x0000, 0.0),
    (0x7F7F, 3.3895313892515355e38),     # largest finite bf16, (2 - 2^-7) * 2^127
    (0x0001, 2.0 ** -133),               # smallest subnormal
    (0x0080, 2.0 ** -126),               # smallest normal
    (0xFF7F, -3.3895313892515355e38),
    (0x4780, 65536.0),                   # beyond the fp16 range
])
def test_widen_bf16_hand_patterns(bits, value):
    got = O.widen(np.array([bits], np.uint16), "bf16")
    assert got.dtype == np.float64 and got[0] == value
    assert _bf16_value_by_definition(bits) == value


def test_widen_bf16_negative_zero_keeps_its_sign():
    got = O.widen(np.array([0x8000], np.uint16), "bf16")[0]
    assert got == 0.0 and math.copysign(1.0, got) == -1.0


def test_widen_bf16_every_finite_pattern_matches_the_definition():
    bits = np.array([b for b in range(1 << 16) if ((b >> 7) & 0xFF) != 0xFF], np.uint16)
    got = O.widen(bits, "bf16")
    ref = np.array([_bf16_value_by_definition(int(b)) for b in bits], np.float64)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), (bits >> 15).astype(bool))
    # a 2-D array keeps its shape
    assert O.widen(bits[:12].reshape(3, 4), "bf16").shape == (3, 4)


def test_widen_f32_is_exact():
    x = np.array([1.0, -0.1, 3.4028234663852886e38, 1.401298464324817e-45], np.float32)
    got = O.widen(x, "f32")
    assert got.dtype == np.float64
    assert [float(v) for v in got] == [1.0, float(np.float32(-0.1)), 3.4028234663852886e38, 2.0 ** -149]
