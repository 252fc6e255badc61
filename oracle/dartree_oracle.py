"""CPU oracle for one DARTree draft-tree construction round.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product path never calls it, and
it shares no code with the HIP library (its inputs come from the seeded
generator module, which holds no arithmetic of the method).

Everything is plain numpy in float64. bf16 and fp32 inputs are widened
exactly before use. The functions follow the method as the DARTree pages
state it:

  * marsggbo blog "DARTree: give a diffusion drafter an AR tree", section 3.1
    (basic flow): top-K candidates per position from the base logits; depth
    by depth, all surviving parents are scored by the correction head in one
    batched call; the score s_beta(u_1..u_d) = sum_i log q_i(u_i) + beta*d
    (the section's only equation) with beta <= 0; each depth keeps its top W;
    after the supertree is built, one global top-B pass, which Lemma 1 says
    equals best-first heap pops on the materialised tree; section 3.2: the
    drafted tree is verified in one pass under a tree-attention mask.
  * AINews summary "DARTree builds trees in batches before pruning":
    the same steps (K=64, fixed width per depth, supertree larger than the
    verification tree, one-pass selection of the 64 best nodes, prefix
    closure for a non-positive depth reward).
  * 866data commentary: fixed-width tree expanded one layer per batch, then
    best-first pruning.

Readings taken where the pages are silent (listed with reasons in the design
notes of the repository):
  R1  q is the softmax over the K candidates of that position.
  R2  a node at depth d builds its state with h_d; the root state is h_0.
  R3  logits row i holds the base logits of depth i+1.
  R4  per-depth pruning and global selection use one comparator:
      s_beta descending, then depth ascending, then token id ascending, then
      the parent's rank under this same comparator (its slot in its level).
  R5  only the W nodes kept per depth form the supertree.
  R6  the anchor (root) is not counted in B.
  R7  emission order is breadth-first: depth, then the parent's emitted
      index, then token id.
  R8  mask row i has bit j set iff j == i or node j is an ancestor of i.
  R9  values compare numerically (so -0.0 == +0.0); ties go to the lower id.
  R10 verification (section 3.2) with a synthetic target: the target's greedy
      continuation is one token per depth, independent of the draft; a node is
      accepted when its whole root path matches it.
  R11 the acceptance length tau counts the accepted draft tokens plus the
      target's own next token (at least 1).
  R12 the tree-attention step is one head over the draft nodes only: node i
      attends to the nodes whose bit is set in mask row i, softmax of the
      scaled dot products (the prefix's keys, which every node also sees, are
      left out of this synthetic step).
  R15 the drafter's LM head (the step before the candidates) is a synthetic
      bf16 matrix Wlm [V][D] over the block's final hidden states X [R][D]:
      base logits = X Wlm^T; the pages give no architecture or precision.
  R13 the Markov head of section 4.3 (Table 3), whose architecture the pages
      do not state, is the synthetic head with A = 0: a node's state is
      tanh(E[u] + h_d), so its children's distribution depends on its token
      (and its depth) alone. The oracle takes it as A = 0; nothing else
      changes.
"""
from __future__ import annotations

import heapq
from dataclasses import dataclass
from typing import List, Optional

import numpy as np


# ----------------------------------------------------------------------------
# exact widening of stored inputs
# ----------------------------------------------------------------------------
def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a stored tensor: bf16 as uint16 bits, or fp32."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# step a1: top-K candidates (blog section 3.1, "candidate generation")
# ----------------------------------------------------------------------------
def topk_candidates(row: np.ndarray, K: int):
    """The K largest values of one base-logit row, ordered by value
    descending and, among equal values, by token id ascending (R9).

    Returns (ids int64[K], values float64[K]). A stable sort of the row is the
    plain definition; numpy's lexsort is that sort."""
    v = np.asarray(row, dtype=np.float64)
    ids = np.arange(v.shape[0])
    order = np.lexsort((ids, -v))
    sel = order[:K]
    return sel.astype(np.int64), v[sel]


# ----------------------------------------------------------------------------
# the step before a1: the drafter's LM head (blog section 3.1, basic flow: one
# block-parallel forward of the drafter gives the block's base logits, from
# which the candidates are taken)
# ----------------------------------------------------------------------------
def lmhead_logits(X: np.ndarray, Wlm: np.ndarray) -> np.ndarray:
    """Base logits of a synthetic drafter LM head: logits[i][v] = sum_j
    X[i][j] * Wlm[v][j] for hidden states X [R][D] and head rows Wlm [V][D]
    (both widened to float64; one library matrix product)."""
    return np.asarray(X, dtype=np.float64) @ np.asarray(Wlm, dtype=np.float64).T


def lmhead_topk(X: np.ndarray, Wlm: np.ndarray, K: int):
    """Candidates straight from the hidden states: the base logits of the LM
    head, then the K best of each row as in topk_candidates (value descending,
    token id ascending). Returns (ids int64[R][K], values float64[R][K],
    logits float64[R][V])."""
    logits = lmhead_logits(X, Wlm)
    R = logits.shape[0]
    ids = np.empty((R, K), np.int64)
    vals = np.empty((R, K), np.float64)
    for i in range(R):
        ids[i], vals[i] = topk_candidates(logits[i], K)
    return ids, vals, logits


# ----------------------------------------------------------------------------
# step a0: head input h_d = P^T H_d (synthetic stand-in head)
# ----------------------------------------------------------------------------
def head_states(H: np.ndarray, Pt: np.ndarray) -> np.ndarray:
    """h[..., j] = sum_i H[..., i] * P[i, j], with the projection stored as
    Pt[j][i] = P[i][j]. Inputs already widened to float64."""
    return np.asarray(H, dtype=np.float64) @ np.asarray(Pt, dtype=np.float64).T


# ----------------------------------------------------------------------------
# the synthetic correction head
# ----------------------------------------------------------------------------
def log_softmax(z: np.ndarray) -> np.ndarray:
    """log q over one candidate set: z - logsumexp(z) (R1)."""
    m = np.max(z)
    return z - (m + np.log(np.sum(np.exp(z - m))))


def child_state(A: np.ndarray, s_parent: np.ndarray, e_row: np.ndarray, h_d: np.ndarray) -> np.ndarray:
    """s = tanh(A s_parent + E[u] + h_d) (R2)."""
    return np.tanh(A @ s_parent + e_row + h_d)


def corrected_logprobs(base: np.ndarray, U_rows: np.ndarray, s_parent: np.ndarray) -> np.ndarray:
    """log q_d(c | parent) for the K candidates c of depth d:
    log-softmax over c of Lbase_d[c] + <s_parent, U[c]>."""
    return log_softmax(base + U_rows @ s_parent)


# ----------------------------------------------------------------------------
# the supertree (blog section 3.1: depth-by-depth expansion, fixed width W)
# ----------------------------------------------------------------------------
@dataclass
class Node:
    depth: int
    tok: int
    slot: int                 # rank within its level (0 = best)
    parent_slot: int          # slot of the parent in level depth-1 (root: 0)
    cum: float                # sum of log q along the path
    sbeta: float              # cum + beta * depth
    state: Optional[np.ndarray]  # head state (None for depth-L nodes)


def node_key(sbeta: float, depth: int, tok: int, parent_slot: int):
    """Sort key of the comparator R4 (smaller sorts first)."""
    return (-sbeta, depth, tok, parent_slot)


def expand_level(parents: List[Node], d: int, C: np.ndarray, base: np.ndarray, h: np.ndarray,
                 A: np.ndarray, E: np.ndarray, U: np.ndarray, W: int, beta: float, L: int) -> List[Node]:
    """One depth of the batched expansion: score every (parent, candidate)
    pair, rank the children by R4, keep the first W, and give the survivors
    their states when d < L."""
    U_rows = U[C]
    children = []
    for p in parents:
        logq = corrected_logprobs(base, U_rows, p.state)
        cum = p.cum + logq
        sb = cum + beta * d
        for k in range(C.shape[0]):
            children.append((node_key(sb[k], d, int(C[k]), p.slot), float(cum[k]), float(sb[k]), int(C[k]), p))
    children.sort(key=lambda c: c[0])
    level = []
    for slot, (_, cum, sb, tok, p) in enumerate(children[:W]):
        st = child_state(A, p.state, E[tok], h[d]) if d < L else None
        level.append(Node(depth=d, tok=tok, slot=slot, parent_slot=p.slot, cum=cum, sbeta=sb, state=st))
    return level


def build_supertree(cand_ids: np.ndarray, cand_vals: np.ndarray, h: np.ndarray, A: np.ndarray,
                    E: np.ndarray, U: np.ndarray, W: int, beta: float) -> List[List[Node]]:
    """Levels 0..L of the supertree for one request. Level 0 is the root
    (state h_0, cum 0). cand_ids/cand_vals: [L][K]; h: [L][r]."""
    L = cand_ids.shape[0]
    root = Node(depth=0, tok=-1, slot=0, parent_slot=-1, cum=0.0, sbeta=0.0, state=np.asarray(h[0], np.float64))
    levels = [[root]]
    for d in range(1, L + 1):
        levels.append(expand_level(levels[-1], d, cand_ids[d - 1], cand_vals[d - 1], h, A, E, U, W, beta, L))
    return levels


# ----------------------------------------------------------------------------
# step a4: deferred global top-B (blog section 3.1, "deferred pruning")
# ----------------------------------------------------------------------------
def select_topB(levels: List[List[Node]], B: int) -> List[Node]:
    """The best min(B, |supertree|) nodes of levels 1..L under R4, in rank
    order."""
    pool = [nd for lvl in levels[1:] for nd in lvl]
    pool.sort(key=lambda nd: node_key(nd.sbeta, nd.depth, nd.tok, nd.parent_slot))
    return pool[:B]


# ----------------------------------------------------------------------------
# step a5: emission in canonical breadth-first order, and the ancestor mask
# ----------------------------------------------------------------------------
@dataclass
class Emitted:
    n_sel: int
    tok: np.ndarray        # int64[B], pad -1
    depth: np.ndarray      # int64[B], pad 0
    parent: np.ndarray     # int64[B], -1 = anchor, pad -2
    score: np.ndarray      # float64[B], pad -inf
    slot: np.ndarray       # int64[B], the node's slot in its level, pad -1


def emit(selected: List[Node], B: int) -> Emitted:
    """Order the selected set breadth-first (R7): depth ascending, then the
    emitted index of the parent, then token id. Parent pointers index into
    this order; depth-1 nodes point at the anchor (-1)."""
    by_depth = {}
    for nd in selected:
        by_depth.setdefault(nd.depth, []).append(nd)
    tok = np.full(B, -1, np.int64)
    dep = np.zeros(B, np.int64)
    par = np.full(B, -2, np.int64)
    sc = np.full(B, -np.inf)
    slot = np.full(B, -1, np.int64)
    emitted_index = {}          # (depth, slot) -> index
    i = 0
    for d in sorted(by_depth):
        nodes = by_depth[d]
        def pidx(nd):
            return -1 if d == 1 else emitted_index[(d - 1, nd.parent_slot)]
        nodes.sort(key=lambda nd: (pidx(nd), nd.tok))
        for nd in nodes:
            emitted_index[(d, nd.slot)] = i
            tok[i], dep[i], par[i], sc[i], slot[i] = nd.tok, d, pidx(nd), nd.sbeta, nd.slot
            i += 1
    return Emitted(n_sel=i, tok=tok, depth=dep, parent=par, score=sc, slot=slot)


def tree_mask(parent: np.ndarray, n_sel: int, B: int) -> np.ndarray:
    """Ancestor bitmask (R8): uint64[B][ceil(B/64)], bit j%64 of word j//64 of
    row i is set iff j == i or j is an ancestor of i. Rows >= n_sel are 0.
    Built by walking each node's parent chain."""
    words = (B + 63) // 64
    m = np.zeros((B, words), dtype=np.uint64)
    for i in range(n_sel):
        j = i
        while j >= 0:
            m[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
            j = int(parent[j])
    return m


# ----------------------------------------------------------------------------
# verification consumer (blog section 3.2: the drafted tree is verified in
# one target pass under the tree-attention mask), with a synthetic target
# ----------------------------------------------------------------------------
def accept_longest(tok: np.ndarray, depth: np.ndarray, parent: np.ndarray, n_sel: int,
                   target: np.ndarray):
    """Greedy verification against a target continuation target[0..L-1]
    (target[d-1] is the target's token at depth d): a node is accepted iff its
    token equals the target's at its depth and its parent is the anchor or
    accepted (R10). Every root path is enumerated and compared token by token.
    Returns (tau, nodes): tau = 1 + the depth of the deepest accepted node
    (the accepted draft tokens plus the target's own next token, R11); nodes =
    the emitted indices along the accepted path, depth 1 first."""
    best = []
    for i in range(n_sel):
        path = []
        j = i
        while j >= 0:
            path.append(j)
            j = int(parent[j])
        path.reverse()
        if all(int(tok[v]) == int(target[k]) for k, v in enumerate(path)) and len(path) > len(best):
            best = path
    return 1 + len(best), best


def tree_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, mask: np.ndarray, n_sel: int) -> np.ndarray:
    """One attention step over the draft nodes under the tree mask (R12):
    out[i] = sum_j softmax_j(<Q[i], K[j]> / sqrt(dh)) V[j] over the j whose
    bit is set in mask row i (the node and its ancestors); rows >= n_sel are 0.
    Q, K, V: [B][dh]; mask: uint64[B][ceil(B/64)]."""
    B, dh = Q.shape
    out = np.zeros((B, dh))
    for i in range(n_sel):
        js = [j for j in range(B) if (int(mask[i, j // 64]) >> (j % 64)) & 1]
        s = np.array([np.dot(Q[i], K[j]) for j in js]) / np.sqrt(dh)
        w = np.exp(s - s.max())
        w /= w.sum()
        out[i] = sum(wk * V[j] for wk, j in zip(w, js))
    return out


# ----------------------------------------------------------------------------
# literal heaps
# ----------------------------------------------------------------------------
def heap_materialized(levels: List[List[Node]], B: int) -> List[Node]:
    """Best-first pops on the materialised supertree (Lemma 1, blog section
    3.1; AINews: heap selection item by item on the materialised tree).
    The heap starts with level 1; each pop pushes the popped node's
    supertree children."""
    L = len(levels) - 1
    children = [dict() for _ in range(L + 1)]
    for d in range(1, L + 1):
        for nd in levels[d]:
            children[d - 1].setdefault(nd.parent_slot, []).append(nd)
    heap = []
    for nd in levels[1]:
        heapq.heappush(heap, (node_key(nd.sbeta, nd.depth, nd.tok, nd.parent_slot), id(nd), nd))
    out = []
    while heap and len(out) < B:
        _, _, nd = heapq.heappop(heap)
        out.append(nd)
        if nd.depth < L:
            for ch in children[nd.depth].get(nd.slot, []):
                heapq.heappush(heap, (node_key(ch.sbeta, ch.depth, ch.tok, ch.parent_slot), id(ch), ch))
    return out


@dataclass
class FullNode:
    depth: int
    tok: int
    cum: float
    sbeta: float
    key: tuple
    parent: Optional["FullNode"]
    state: Optional[np.ndarray] = None


def heap_serial_full(cand_ids: np.ndarray, cand_vals: np.ndarray, h: np.ndarray, A: np.ndarray,
                     E: np.ndarray, U: np.ndarray, beta: float, B: int) -> List[FullNode]:
    """The serial "pop then correct" construction (blog section 2 and Table 2):
    best-first over the full K-ary tree with no per-depth width; every pop
    runs the head on the popped node and pushes all K of its children.
    Ties use R4 with the parent rank taken recursively (the parent's own key).
    Returns the B popped nodes in pop order."""
    L = cand_ids.shape[0]
    root = FullNode(depth=0, tok=-1, cum=0.0, sbeta=0.0, key=(), parent=None, state=np.asarray(h[0], np.float64))
    heap = []

    def push_children(p: FullNode):
        d = p.depth + 1
        C = cand_ids[d - 1]
        logq = corrected_logprobs(cand_vals[d - 1], U[C], p.state)
        for k in range(C.shape[0]):
            cum = p.cum + logq[k]
            sb = cum + beta * d
            key = (-sb, d, int(C[k]), p.key)
            heapq.heappush(heap, (key, FullNode(depth=d, tok=int(C[k]), cum=cum, sbeta=sb, key=key, parent=p)))

    push_children(root)
    out = []
    while heap and len(out) < B:
        _, nd = heapq.heappop(heap)
        out.append(nd)
        if nd.depth < L:
            nd.state = child_state(A, nd.parent.state, E[nd.tok], h[nd.depth])
            push_children(nd)
    return out


# ----------------------------------------------------------------------------
# one whole round
# ----------------------------------------------------------------------------
@dataclass
class RequestResult:
    cand_ids: np.ndarray     # [L][K] int64
    cand_vals: np.ndarray    # [L][K] float64
    h: np.ndarray            # [L][r] float64
    levels: List[List[Node]]
    selected: List[Node]
    emitted: Emitted
    mask: np.ndarray


def round_one_request(logits_rows: np.ndarray, h: np.ndarray, A: np.ndarray, E: np.ndarray,
                      U: np.ndarray, K: int, W: int, B: int, beta: float) -> RequestResult:
    """All steps for one request, inputs already in float64:
    logits_rows [L][V], h [L][r], A [r][r], E [V][r], U [V][r]."""
    if beta > 0:
        raise ValueError("Lemma 1 needs beta <= 0")
    L = logits_rows.shape[0]
    ids = np.empty((L, K), np.int64)
    vals = np.empty((L, K), np.float64)
    for i in range(L):
        ids[i], vals[i] = topk_candidates(logits_rows[i], K)
    levels = build_supertree(ids, vals, h, A, E, U, W, beta)
    sel = select_topB(levels, B)
    em = emit(sel, B)
    mask = tree_mask(em.parent, em.n_sel, B)
    return RequestResult(cand_ids=ids, cand_vals=vals, h=h, levels=levels, selected=sel, emitted=em, mask=mask)


def round_all(cfg, head, rnd) -> List[RequestResult]:
    """The oracle round for every request of a generated round. ``cfg``,
    ``head`` and ``rnd`` are the generator's Config, Head and Round."""
    wd = head.dtype
    A, E, U = widen(head.A, wd), widen(head.E, wd), widen(head.U, wd)
    logits = widen(rnd.logits, cfg.logits_dtype)
    if cfg.D > 0:
        h_all = head_states(widen(rnd.H, wd), widen(head.Pt, wd))
    else:
        h_all = np.asarray(rnd.h, np.float64)
    return [round_one_request(logits[q], h_all[q], A, E, U, cfg.K, cfg.W, cfg.B, cfg.beta)
            for q in range(cfg.n_req)]
