"""GPU parity of the fused drafter LM head + top-K (dartree_lmhead_topk)
against the oracle's fp64 logits and stable top-K, through the C ABI."""
import numpy as np
import pytest
import torch

from diffusion_drafter_tree_amd import inputs as I
from diffusion_drafter_tree_amd import ops
from oracle import check as CK
from oracle import dartree_oracle as O
from tests import _parity_pool as PP

pytestmark = pytest.mark.gpu
TOL = 1e-4


def run_lmhead(cfg, X_bits, W_bits):
    dims = ops.make_dims(cfg)
    rows = cfg.n_req * cfg.L
    ids = torch.full((rows, cfg.K), -7, dtype=torch.int32, device="cuda")
    vals = torch.zeros((rows, cfg.K), dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.lmhead_workspace_size(dims), dtype=torch.uint8, device="cuda")
    ops.lmhead_topk(dims, ops.to_device(X_bits), ops.to_device(W_bits), ids, vals, ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), vals.cpu().numpy()


CASES = {
    "rows16_V5003_D256": dict(n_req=1, L=16, V=5003, D=256, K=64),
    "rows40_ragged_V20000_D512": dict(n_req=5, L=8, V=20000, D=512, K=64),
    "ring8_D768_K17": dict(n_req=1, L=16, V=30011, D=768, K=17),
    "K1": dict(n_req=1, L=7, V=9000, D=256, K=1),
    "tiny_V100": dict(n_req=1, L=3, V=100, D=256, K=64),
    "V_eq_K": dict(n_req=1, L=2, V=64, D=256, K=64),
    "qwen3_4b_full": dict(n_req=1, L=16, V=151936, D=2560, K=64),
    "qwen3_8b_full_two_chunks": dict(n_req=1, L=16, V=151936, D=4096, K=64),
}


@pytest.mark.parametrize("name", list(CASES))
def test_lmhead_topk_against_oracle(name):
    cfg = I.small_variant("qwen3_4b", name=name, **CASES[name])
    print(f"[lmhead] case {name}", flush=True)
    W = I.make_lmhead(cfg, 0)
    X = I.make_lmhead_states(cfg, W, 0, 0)
    ids, vals = run_lmhead(cfg, X, W)
    rows = cfg.n_req * cfg.L
    rep = CK.check_lmhead_topk(ids, vals, O.widen(X.reshape(rows, cfg.D), "bf16"), O.widen(W, "bf16"), cfg.K,
                               tol=TOL, where=name)
    PP.log_case(f"lmhead {name}", rep, rows=rows)


def test_lmhead_exact_ties_at_the_cut_take_the_lower_id():
    """Duplicate head rows give bit-equal logits; where such a pair straddles
    the K-th place the lower token id must be kept (no tie event allowed)."""
    cfg = I.small_variant("qwen3_4b", name="lmhead_ties", n_req=1, L=4, V=40000, D=512, K=64)
    W = I.make_lmhead(cfg, 3)
    X = I.make_lmhead_states(cfg, W, 3, 0)
    rows = cfg.n_req * cfg.L
    Xf, Wf = O.widen(X.reshape(rows, cfg.D), "bf16"), O.widen(W, "bf16")
    logits = Xf @ Wf.T
    # copy the head row of row 0's K-th best token a onto its neighbours
    # a - 1 and a + 1: three bit-equal logits in every row, straddling the cut
    # in row 0, where only the lowest id of them may be kept
    o, _ = O.topk_candidates(logits[0], cfg.K)
    a = int(o[-1])
    assert 0 < a < cfg.V - 1
    W2 = W.copy()
    W2[a - 1] = W2[a]
    W2[a + 1] = W2[a]
    Wf2 = O.widen(W2, "bf16")
    l2 = Xf[0] @ Wf2.T
    o2, v2 = O.topk_candidates(l2, cfg.K + 1)
    assert v2[cfg.K - 1] == v2[cfg.K] and int(o2[cfg.K - 1]) == a - 1
    ids, vals = run_lmhead(cfg, X, W2)
    rep = CK.check_lmhead_topk(ids, vals, Xf, Wf2, cfg.K, tol=TOL, where="ties")
    PP.log_case("lmhead exact ties", rep, rows=rows)
    assert rep.tie_events_level == 0, rep.tie_log


def test_lmhead_all_logits_equal_takes_the_lowest_ids():
    """Zero hidden states: every logit is exactly 0, so the K best are the K
    lowest token ids. Far more than K keys of the slab lists reach the
    K-th largest slab maximum here, which sends the merge down its full
    (unpruned) path."""
    cfg = I.small_variant("qwen3_4b", name="lmhead_flat", n_req=1, L=3, V=151936, D=256, K=64)
    W = I.make_lmhead(cfg, 5)
    rows = cfg.n_req * cfg.L
    X = np.zeros((rows, cfg.D), dtype=np.uint16)
    ids, vals = run_lmhead(cfg, X, W)
    assert (ids == np.arange(cfg.K, dtype=np.int32)[None, :]).all()
    assert (vals == 0.0).all()
    rep = CK.check_lmhead_topk(ids, vals, O.widen(X, "bf16"), O.widen(W, "bf16"), cfg.K, tol=TOL, where="flat")
    PP.log_case("lmhead all logits equal", rep, rows=rows)


@pytest.mark.parametrize("period", [97, 1009])
def test_lmhead_periodic_head_rows(period):
    """Head rows repeating with a period: each logit value recurs V / period
    times, spread over every slab, so the keys that reach the pruning bound
    are many bit-equal logits across slabs, ranked by token id."""
    cfg = I.small_variant("qwen3_4b", name=f"lmhead_period{period}", n_req=1, L=4, V=151936, D=512, K=64)
    W = I.make_lmhead(cfg, 6)
    W = W[np.arange(cfg.V) % period].copy()
    X = I.make_lmhead_states(cfg, W, 6, 0)
    rows = cfg.n_req * cfg.L
    ids, vals = run_lmhead(cfg, X, W)
    rep = CK.check_lmhead_topk(ids, vals, O.widen(X.reshape(rows, cfg.D), "bf16"), O.widen(W, "bf16"), cfg.K,
                               tol=TOL, where=f"period{period}")
    PP.log_case(f"lmhead periodic head rows {period}", rep, rows=rows)
