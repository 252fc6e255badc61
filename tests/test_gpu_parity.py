"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: candidate ids, parents, emission and masks bit-exact; fp32 scores within
1e-4 absolute of the fp64 oracle; kept sets may differ only at near-ties
(gap <= 1e-4), which the tie-aware checker replays.
"""
import copy
import sys

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


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


_heads = {}


def device_head(cfg, seed=0):
    key = (cfg, seed)
    if key not in _heads:
        hd = I.make_head(cfg, seed)
        _heads[key] = (hd, ops.DeviceHead(hd))
    return _heads[key]


def run_gpu(cfg, hd, dhd, rnd, mode="build", chunks=None):
    rb = ops.RoundBuffers(cfg)
    logits = ops.to_device(rnd.logits)
    hin = ops.to_device(rnd.H if cfg.D > 0 else rnd.h)
    if mode == "build":
        ops.build_round(rb.dims, dhd, logits, hin, rb)
    else:
        ops.run_steps(rb.dims, dhd, logits, hin, rb, depth_chunks=chunks)
    torch.cuda.synchronize()
    return rb.numpy()


def check(cfg, seed=0, t=0, mode="build", chunks=None, requests=None):
    hd, dhd = device_head(cfg, seed)
    rnd = I.make_round(cfg, seed, t)
    say(f"case {cfg.name} n={cfg.n_req} V={cfg.V} L={cfg.L} K={cfg.K} W={cfg.W} B={cfg.B} r={cfg.r} D={cfg.D} "
        f"seed={seed} t={t} mode={mode}")
    out = run_gpu(cfg, hd, dhd, rnd, mode, chunks)
    rep = CK.check_round(cfg, hd, rnd, out, tol=TOL, requests=requests)
    say(f"  ok: nodes={rep.nodes_checked} ties(level/topB)={rep.tie_events_level}/{rep.tie_events_topB} "
        f"max|dscore|={rep.max_score_err:.2e} max|dh|={rep.max_h_err:.2e}")
    PP.log_case(f"{cfg.name} seed={seed} t={t} mode={mode}", rep)
    return out, rep


def check_many_rounds(cfg, ts, seed=0, label=None):
    """Full-round parity on many seeded rounds: the rounds are drawn and
    checked against the oracle in spawned worker processes while this process
    runs them on the GPU, one round at a time."""
    hd, dhd = device_head(cfg, seed)
    rep, ties, n = CK.Report(), 0, 0
    label = label or f"{cfg.name} rounds {ts[0]}..{ts[-1]}"
    with PP.pool() as ex:
        futs = []
        for t, rnd in zip(ts, ex.map(PP.gen_round, [cfg] * len(ts), [seed] * len(ts), ts)):
            out = run_gpu(cfg, hd, dhd, rnd)
            futs.append(ex.submit(PP.check_job, cfg, seed, t, out, None, TOL))
        for f in futs:
            r, tb = f.result()
            rep.merge(r)
            ties += tb
            n += 1
            if n % 100 == 0:
                PP.log_case(f"{label} progress", rounds=n)
    PP.log_case(label, rep, rounds=n, rows=n * cfg.n_req * cfg.L, rows_tied_at_K=ties,
                tie_events_per_1000_rounds=1000.0 * (rep.tie_events_level + rep.tie_events_topB) / max(n, 1))
    return rep


SMALL = {
    "tiny_f32": I.CONFIGS["tiny"],
    "bf16_ragged_odd_V": I.small_variant("qwen3_4b", n_req=3, V=5003, L=5, K=40, W=7, B=20, r=64, D=96),
    "bf16_multichunk": I.small_variant("qwen3_4b", n_req=2, V=40000, L=4, K=64, W=12, B=30, r=128, D=256),
    "f32_multichunk_valu": I.small_variant("tiny", n_req=2, V=20000, L=7, K=16, W=5, B=25, r=24, D=40),
    "bf16_r48_valu": I.small_variant("qwen3_4b", n_req=1, V=3000, L=6, K=24, W=6, B=30, r=48, D=64),
    "wide_W32_K256": I.small_variant("qwen3_4b", n_req=2, V=9000, L=6, K=256, W=32, B=100, r=128, D=128),
    "big_B200": I.small_variant("qwen3_4b", n_req=1, V=3000, L=8, K=30, W=40, B=200, r=32, D=64),
    "chain_W1": I.small_variant("qwen3_4b", n_req=2, V=4000, L=9, K=32, W=1, B=6, r=64, D=64),
    "beta0": I.small_variant("qwen3_4b", n_req=1, V=4000, L=6, K=32, W=5, B=20, r=64, D=64, beta=0.0),
    "beta_neg5": I.small_variant("qwen3_4b", n_req=1, V=4000, L=6, K=32, W=5, B=12, r=64, D=64, beta=-5.0),
    "whole_supertree_WL_le_B": I.small_variant("qwen3_4b", n_req=1, V=4000, L=5, K=16, W=4, B=64, r=64, D=64),
    "K_eq_V": I.small_variant("tiny", V=48, K=48, L=4, W=6, B=10, r=16),
    "L1": I.small_variant("qwen3_4b", n_req=2, V=5000, L=1, K=20, W=5, B=3, r=32, D=32),
    # block-decoding kernel shapes (bf16 weights, r = 256, K in {16, 32, 64}, W <= 16)
    "fast_K16_W16_L31_B100": I.small_variant("qwen3_4b", n_req=2, V=5000, L=31, K=16, W=16, B=100, r=256, D=64),
    "fast_K32_W1_beta0": I.small_variant("qwen3_4b", n_req=1, V=4000, L=9, K=32, W=1, B=6, r=256, D=64, beta=0.0),
    "fast_K64_W12_L6": I.small_variant("qwen3_4b", n_req=2, V=6000, L=6, K=64, W=12, B=40, r=256, D=96),
    "fast_W16_whole_supertree_B256": I.small_variant("qwen3_4b", n_req=1, V=5000, L=16, K=64, W=16, B=256, r=256,
                                                     D=64),
    "fast_L1": I.small_variant("qwen3_4b", n_req=3, V=3000, L=1, K=64, W=8, B=5, r=256, D=32),
    "fast_multislice_K64": I.small_variant("qwen3_4b", n_req=1, V=100000, L=4, K=64, W=10, B=30, r=256, D=64,
                                           beta=-5.0),
    "fast_f32_logits_multislice": I.small_variant("qwen3_4b", n_req=2, V=60000, L=5, K=64, W=8, B=24, r=256, D=64,
                                                  logits_dtype="f32"),
}
FAST = sorted(k for k in SMALL if k.startswith("fast_"))


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_configs_build_round(name):
    check(SMALL[name].with_(name=name))


@pytest.mark.parametrize("name", ["tiny_f32", "bf16_multichunk", "f32_multichunk_valu", "wide_W32_K256",
                                  "fast_K64_W12_L6", "fast_K16_W16_L31_B100"])
def test_step_entry_points_match_fused_round(name):
    cfg = SMALL[name].with_(name=name)
    a, _ = check(cfg, mode="build")
    b, _ = check(cfg, mode="steps")
    c, _ = check(cfg, mode="steps", chunks=[(1, 2), (3, cfg.L)])
    for k in a:
        assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a[k], c[k]), k


@pytest.mark.parametrize("name", ["fast_K64_W12_L6", "fast_K16_W16_L31_B100", "bf16_ragged_odd_V"])
def test_select_on_stored_levels_out_of_order(name):
    """select_topB on a supertree whose stored levels are not in the order the
    expansion writes them (each level's filled slots permuted, the next
    level's parent slots remapped to match). The top-B ranking compares every
    node's key with every other, so it must not depend on slot order: the
    tree must be the same, with each emitted slot mapped through the
    permutation."""
    cfg = SMALL[name].with_(name=name)
    hd, dhd = device_head(cfg)
    rnd = I.make_round(cfg, 0, 0)
    say(f"case {name}: select on permuted levels")
    rb = ops.RoundBuffers(cfg)
    ops.build_round(rb.dims, dhd, ops.to_device(rnd.logits), ops.to_device(rnd.H if cfg.D > 0 else rnd.h), rb)
    torch.cuda.synchronize()
    ref = rb.numpy()
    n, L, W = cfg.n_req, cfg.L, cfg.W
    cnt = ref["st_count"]
    arrs = {k: ref[k].copy() for k in ("st_tok", "st_parent", "st_cum", "st_sbeta")}
    rng = np.random.default_rng(11)
    new_of_old = np.tile(np.arange(W), (n, L, 1))
    moved = 0
    for q in range(n):
        for d in range(L):
            c = int(cnt[q, d])
            perm = np.arange(W)
            perm[:c] = rng.permutation(c)   # new slot j holds old slot perm[j]
            moved += int((perm[:c] != np.arange(c)).sum())
            for a in arrs.values():
                a[q, d] = a[q, d][perm]
            new_of_old[q, d][perm] = np.arange(W)
    for q in range(n):
        for d in range(1, L):
            c = int(cnt[q, d])
            arrs["st_parent"][q, d, :c] = new_of_old[q, d - 1][arrs["st_parent"][q, d, :c]]
    assert moved > 0
    for k, a in arrs.items():
        getattr(rb, k).copy_(torch.from_numpy(a))
    ops.select_topB(rb.dims, rb)
    torch.cuda.synchronize()
    out = rb.numpy()
    for k in ("n_sel", "tok", "depth", "parent", "score"):
        assert np.array_equal(out[k], ref[k]), k
    for q in range(n):
        for e in range(int(ref["n_sel"][q])):
            d, sl = int(ref["depth"][q, e]), int(ref["slot"][q, e])
            assert out["slot"][q, e] == new_of_old[q, d - 1][sl]


SPLIT_EXTRA = {
    # W (K + r) near the 16384 limit with parts' block ranges that round up:
    # more exchanged vectors than three a thread
    "split_ragged_blocks": I.small_variant("qwen3_4b", n_req=2, V=5000, L=4, K=170, W=48, B=60, r=160, D=64),
}


@pytest.mark.parametrize("name", ["bf16_multichunk", "wide_W32_K256", "big_B200", "beta0", "split_ragged_blocks"])
def test_split_parts_computing_alone_match_the_exchange(name):
    """The general kernel spreads a request over several workgroups that
    exchange contraction slices; with the wait bound at 0 every part computes
    the whole contraction itself (the path of a part whose partners are not
    resident). Both runs must give identical bits, and match the oracle."""
    cfg = (SMALL[name] if name in SMALL else SPLIT_EXTRA[name]).with_(name=name)
    assert ops.round_plan(ops.make_dims(cfg))["tree_parts"] > 1
    a, _ = check(cfg)
    try:
        ops.set_split_wait(0)
        b, _ = check(cfg)
    finally:
        ops.set_split_wait(200)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_split_rounds_sharing_the_gpu_match_rounds_alone():
    """Two 64-request rounds of the general kernel (four workgroups a request,
    one a CU for their LDS) launched together on two streams: 512 workgroups
    for 256 CUs, so parts of a round are not all resident at once and wait for
    each other only up to the bound, then compute the missing slices
    themselves. Every output must equal the same rounds run one after the
    other, bit for bit, and the oracle on sampled requests."""
    cfg = I.small_variant("stress_64req", name="split_shared", V=8000, L=6, K=512, W=12, B=40, r=512, D=256)
    plan = ops.round_plan(ops.make_dims(cfg))
    assert plan["tree_parts"] == 4 and plan["tree_lds_bytes"] > 80 * 1024, plan
    hd, dhd = device_head(cfg)
    rnds = [I.make_round(cfg, 0, t) for t in range(2)]
    ins = [(ops.to_device(r.logits), ops.to_device(r.H)) for r in rnds]
    alone = []
    for lg, H in ins:
        rb = ops.RoundBuffers(cfg)
        ops.build_round(rb.dims, dhd, lg, H, rb)
        torch.cuda.synchronize()
        alone.append(rb.numpy())
    say("case split_shared: two rounds on two streams")
    rbs = [ops.RoundBuffers(cfg) for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    torch.cuda.synchronize()
    for _ in range(3):
        for (lg, H), rb, st in zip(ins, rbs, streams):
            ops.build_round(rb.dims, dhd, lg, H, rb, stream=st)
        torch.cuda.synchronize()
        for rb, ref in zip(rbs, alone):
            out = rb.numpy()
            for k in ref:
                assert np.array_equal(out[k], ref[k]), k
    for t in range(2):
        rep = CK.check_round(cfg, hd, rnds[t], alone[t], tol=TOL, requests=[0, 31, 63])
        PP.log_case(f"split_shared t={t} requests 0, 31, 63", rep)


def test_rejected_calls_leave_every_output_untouched():
    """Every call validates completely on the host before it enqueues
    anything: a rejected dartree_build_round (and dartree_topk_candidates)
    must return its status and leave every output and the workspace byte for
    byte as they were (canary-filled)."""
    import ctypes
    from diffusion_drafter_tree_amd import _lib as C
    cfg = SMALL["bf16_multichunk"].with_(name="canary")
    hd, dhd = device_head(cfg)
    rnd = I.make_round(cfg, 0, 0)
    logits, H = ops.to_device(rnd.logits), ops.to_device(rnd.H)
    rb = ops.RoundBuffers(cfg)
    outs = [rb.cand_ids, rb.cand_logit, rb.h, rb.st_tok, rb.st_parent, rb.st_cum, rb.st_sbeta, rb.st_count,
            rb.st_state, rb.n_sel, rb.tok, rb.depth, rb.parent, rb.score, rb.slot, rb.mask, rb.ws]
    for t in outs:
        t.view(torch.uint8).fill_(0xA5)
    torch.cuda.synchronize()
    before = [t.view(torch.uint8).cpu().clone() for t in outs]
    lib = C.load()

    def build(dims, head=dhd, logits=logits, ws_bytes=rb.ws_bytes):
        rb.st.next_depth = 1
        return lib.dartree_build_round(ctypes.byref(dims), ctypes.byref(head.c), ops._p(logits), ops._p(H),
                                       ops._p(rb.cand_ids), ops._p(rb.cand_logit), ops._p(rb.h), ctypes.byref(rb.st),
                                       ops._p(rb.n_sel), ops._p(rb.tok), ops._p(rb.depth), ops._p(rb.parent),
                                       ops._p(rb.score), ops._p(rb.slot), ops._p(rb.mask), ops._p(rb.ws), ws_bytes,
                                       ops._stream())
    good = ops.make_dims(cfg)
    bad_beta = ops.make_dims(cfg.with_(beta=0.5))
    bad_k = ops.make_dims(cfg.with_(K=cfg.V + 1))
    bad_flags = copy.copy(dhd)
    bad_flags.c = C.Head(A=dhd.c.A, E=dhd.c.E, U=dhd.c.U, Pt=dhd.c.Pt, flags=0x100)
    cases = [
        ("beta > 0", build(bad_beta), C.ERR_INVALID_ARGUMENT),
        ("K > V", build(bad_k), C.ERR_INVALID_ARGUMENT),
        ("workspace too small", build(good, ws_bytes=rb.ws_bytes - 256), C.ERR_WORKSPACE_TOO_SMALL),
        ("misaligned logits", build(good, logits=logits.view(torch.uint8)[2:]), C.ERR_INVALID_ARGUMENT),
        ("unknown head flag", build(good, head=bad_flags), C.ERR_INVALID_ARGUMENT),
        ("topk: workspace too small",
         lib.dartree_topk_candidates(ctypes.byref(good), ops._p(logits), ops._p(rb.cand_ids), ops._p(rb.cand_logit),
                                     ops._p(rb.ws), 16, ops._stream()), C.ERR_WORKSPACE_TOO_SMALL),
    ]
    torch.cuda.synchronize()
    for what, got, want in cases:
        say(f"  rejected call: {what}: {C.status_string(got)}")
        assert got == want, (what, C.status_string(got), C.last_error())
    for t, b0 in zip(outs, before):
        assert torch.equal(t.view(torch.uint8).cpu(), b0)


@pytest.mark.parametrize("chunk", range(4))
def test_metric_config_qwen3_4b_1000_rounds(chunk):
    """All 1000 seeded rounds of the metric config, 250 per case: the whole
    round (16,000 candidate rows bit-exact, every level replayed, top-B,
    emission and mask) against the oracle."""
    ts = list(range(chunk * 250, (chunk + 1) * 250))
    check_many_rounds(I.CONFIGS["qwen3_4b"], ts)


def test_tiny_config_500_seeds():
    """The tiny fp32 config on 500 head-and-round seeds."""
    cfg = I.CONFIGS["tiny"]
    rep = CK.Report()
    for seed in range(500):
        hd = I.make_head(cfg, seed)
        dhd = ops.DeviceHead(hd)
        rnd = I.make_round(cfg, seed, 0)
        out = run_gpu(cfg, hd, dhd, rnd)
        rep.merge(CK.check_round(cfg, hd, rnd, out, tol=TOL))
    PP.log_case("tiny 500 seeds", rep, rounds=500)


def test_fixed_width_qwen3_8b():
    check(I.CONFIGS["fixed_w4_qwen3_8b"])


def test_concurrent_c4():
    check(I.CONFIGS["concurrent_c4"])


@pytest.mark.parametrize("t", [0, 1])
def test_stress_64req_all_requests(t):
    """Every one of the 64 requests of a stress round (K = 512, r = 512, the
    general tree kernel), checked in eight-request slices by worker
    processes."""
    cfg = I.CONFIGS["stress_64req"]
    hd, dhd = device_head(cfg)
    say(f"case stress_64req all requests t={t}")
    rnd = I.make_round(cfg, 0, t)
    out = run_gpu(cfg, hd, dhd, rnd)
    del rnd
    rep, ties = CK.Report(), 0
    with PP.pool() as ex:
        futs = [ex.submit(PP.check_job, cfg, 0, t, out, list(range(q0, q0 + 8)), TOL) for q0 in range(0, 64, 8)]
        for f in futs:
            r, tb = f.result()
            rep.merge(r)
            ties += tb
    assert rep.nodes_checked == cfg.n_req * cfg.L * cfg.W
    PP.log_case(f"stress_64req t={t} all 64 requests", rep, rows_tied_at_K=ties)


def test_repeat_runs_are_bit_identical():
    """100 runs of one round: every output bit-identical (a race in any
    kernel would show as a difference between runs)."""
    cfg = I.CONFIGS["qwen3_4b"]
    hd, dhd = device_head(cfg)
    rnd = I.make_round(cfg, 0, 5)
    say("case repeat-determinism qwen3_4b x100")
    rb = ops.RoundBuffers(cfg)
    logits, hin = ops.to_device(rnd.logits), ops.to_device(rnd.H)
    ref = None
    for i in range(100):
        ops.build_round(rb.dims, dhd, logits, hin, rb)
        torch.cuda.synchronize()
        o = rb.numpy()
        if ref is None:
            ref = o
            continue
        for k in o:
            assert np.array_equal(o[k], ref[k]), (i, k)
    PP.log_case("repeat-determinism qwen3_4b", runs=100)


def _tie_head_round(cfg, seed, huge_gap):
    """U = 0 (the corrected distribution is the base one, so children of one
    parent with equal base logits tie exactly in fp32 and fp64 alike) and
    base logits on a grid of 0.5 (many exact ties among the candidates). With
    ``huge_gap``, the first candidate of each position sits 240 above the
    rest: its log q is exactly 0 in both precisions, so with beta = 0 a chain
    of nodes ties its parent across depths."""
    import dataclasses
    hd = I.make_head(cfg, seed)
    hd = dataclasses.replace(hd, U=np.zeros_like(hd.U))
    rnd = I.make_round(cfg, seed, 0)
    x = np.round(I.as_f64(rnd.logits, cfg.logits_dtype) * 2) / 2
    if huge_gap:
        for q in range(cfg.n_req):
            for i in range(cfg.L):
                x[q, i, int(np.argmax(x[q, i]))] = 240.0
    else:
        # force exact ties at both cuts of the first position: the W-th and
        # (W+1)-th best base logits, and the B-th and (B+1)-th, made equal
        # (the higher token id takes the lower one's value)
        for q in range(cfg.n_req):
            order = np.lexsort((np.arange(cfg.V), -x[q, 0]))
            for cut in (cfg.W, cfg.B):
                a, b = order[cut - 1], order[cut]
                x[q, 0, max(a, b)] = x[q, 0, min(a, b)]
                order = np.lexsort((np.arange(cfg.V), -x[q, 0]))
    rnd.logits = I.f32_to_bf16_bits(x.astype(np.float32)) if cfg.logits_dtype == "bf16" else x.astype(np.float32)
    return hd, rnd


@pytest.mark.parametrize("name,huge_gap", [("fast_ties", False), ("fast_ties_depth", True),
                                           ("general_ties", False), ("general_ties_depth", True)])
def test_exact_ties_at_the_cut_follow_the_comparator(name, huge_gap):
    """Exact ties (equal in fp32 and in fp64) at the top-W and top-B cuts
    must be settled by the comparator -- token ascending among children of
    one parent, depth ascending across depths -- so the kept sets equal the
    oracle's with no tie event at all."""
    # one depth without the gap: every child has the root as its parent, so
    # equal base logits give bit-equal scores at the W and B cuts. With the
    # gap, each level's survivors are the chain node and its best children
    # (other parents' children sit ~240 lower), so exact ties again fall
    # between children of one parent, and across depths on the chain.
    base = dict(n_req=2, V=6000, L=8 if huge_gap else 1, K=64, W=6, B=5 if huge_gap else 4, D=64,
                beta=0.0 if huge_gap else -0.1)
    if name.startswith("fast"):
        cfg = I.small_variant("qwen3_4b", name=name, r=256, **base)
    else:
        cfg = I.small_variant("qwen3_4b", name=name, r=64, **base)
    hd, rnd = _tie_head_round(cfg, 11, huge_gap)
    dhd = ops.DeviceHead(hd)
    say(f"case exact ties {name}")
    out = run_gpu(cfg, hd, dhd, rnd)
    rep = CK.check_round(cfg, hd, rnd, out, tol=TOL)
    ties = PP.boundary_ties(rnd.logits, cfg.logits_dtype, cfg.K)
    PP.log_case(f"exact ties {name}", rep, rows_tied_at_K=ties)
    assert ties > 0
    if not huge_gap:
        # the oracle itself sees exact ties at both cuts
        for r in O.round_all(cfg, hd, rnd):
            sb = sorted((nd.sbeta for nd in r.levels[1]), reverse=True)
            allc = sorted(O.corrected_logprobs(r.cand_vals[0], np.zeros((cfg.K, cfg.r)), r.h[0]), reverse=True)
            assert allc[cfg.W - 1] == allc[cfg.W] and sb[cfg.B - 1] == sb[cfg.B]
    assert rep.tie_events_level == 0 and rep.tie_events_topB == 0, rep.tie_log
    if huge_gap:
        # the chain of first candidates scores exactly 0 at every depth, and
        # the selection takes it depth by depth
        for q in range(cfg.n_req):
            zero = [i for i in range(int(out["n_sel"][q])) if out["score"][q, i] == 0.0]
            assert [int(out["depth"][q, i]) for i in zero] == list(range(1, cfg.B + 1)), (q, zero)


def _request_sizes(cfg):
    """Per-request widths and budgets covering the full size, the minimum, a
    middle value and out-of-range values (clamped by the library)."""
    n = cfg.n_req
    w_raw = [cfg.W, 1, max(1, cfg.W // 2), cfg.W + 5, 0, -3][:n]
    b_raw = [cfg.B, 1, max(1, cfg.B // 3), cfg.B + 7, 0, 2][:n]
    w_eff = [min(max(x, 1), cfg.W) for x in w_raw]
    b_eff = [min(max(x, 1), cfg.B) for x in b_raw]
    return w_raw, b_raw, w_eff, b_eff


@pytest.mark.parametrize("name,mode", [("fast_K64_W12_L6", "build"), ("fast_K64_W12_L6", "steps"),
                                       ("bf16_multichunk", "build"), ("wide_W32_K256", "steps"),
                                       ("tiny_f32", "build"), ("qwen3_4b_x4", "build")])
def test_per_request_width_and_budget(name, mode):
    """Per-request W_q and B_q inside one batch against the oracle run with
    each request's own sizes; supertree slots past W_q and outputs past n_sel
    are padding."""
    if name == "qwen3_4b_x4":
        cfg = I.CONFIGS["qwen3_4b"].with_(n_req=4, name=name)
    else:
        cfg = SMALL[name].with_(name=name, n_req=4)
    w_raw, b_raw, w_eff, b_eff = _request_sizes(cfg)
    hd, dhd = device_head(cfg)
    rnd = I.make_round(cfg, 0, 3)
    say(f"case per-request sizes {name} mode={mode} widths={w_raw} budgets={b_raw}")
    rb = ops.RoundBuffers(cfg)
    rb.set_request_sizes(torch.tensor(w_raw, dtype=torch.int32, device="cuda"),
                         torch.tensor(b_raw, dtype=torch.int32, device="cuda"))
    logits = ops.to_device(rnd.logits)
    hin = ops.to_device(rnd.H if cfg.D > 0 else rnd.h)
    if mode == "build":
        ops.build_round(rb.dims, dhd, logits, hin, rb)
    else:
        ops.run_steps(rb.dims, dhd, logits, hin, rb, depth_chunks=[(1, 2), (3, cfg.L)])
    torch.cuda.synchronize()
    out = rb.numpy()
    rep = CK.check_round(cfg, hd, rnd, out, tol=TOL, widths=w_eff, budgets=b_eff)
    for q in range(cfg.n_req):
        cnt = out["st_count"][q]
        assert cnt[0] == min(w_eff[q], cfg.K), q
        for d in range(1, cfg.L):
            assert cnt[d] == min(w_eff[q], int(cnt[d - 1]) * cfg.K), (q, d)
        for d in range(cfg.L):
            assert np.all(out["st_tok"][q, d, cnt[d]:] == -1), (q, d)
            assert np.all(np.isneginf(out["st_sbeta"][q, d, cnt[d]:])), (q, d)
        assert out["n_sel"][q] == min(b_eff[q], int(cnt.sum())), q
    say(f"  ok: nodes={rep.nodes_checked} ties(level/topB)={rep.tie_events_level}/{rep.tie_events_topB}")
    # the request with the full sizes equals its result in a uniform batch
    ref = run_gpu(cfg, hd, dhd, rnd)
    for k in ("st_tok", "st_parent", "st_count", "n_sel", "tok", "depth", "parent", "slot", "mask"):
        assert np.array_equal(out[k][0], ref[k][0]), k


@pytest.mark.parametrize("name", ["fast_K64_W12_L6", "bf16_multichunk", "tiny_f32", "qwen3_4b"])
def test_markov_head_variant(name):
    """The Markov-head variant (the child distribution conditioned on the
    parent's token only) is the head with A = 0: a node's state is
    tanh(E[u] + h_d), a function of its own token and depth. Parity with the
    oracle at A = 0, and on the HIP path's own supertree: two kept nodes of
    one depth with the same token give their children the same log q."""
    import dataclasses
    cfg = I.CONFIGS[name] if name in I.CONFIGS else SMALL[name].with_(name=name)
    hd0 = I.make_head(cfg, 0)
    hd = dataclasses.replace(hd0, A=np.zeros_like(hd0.A))
    dhd = ops.DeviceHead(hd)
    rnd = I.make_round(cfg, 0, 1)
    say(f"case markov head (A = 0) {name}")
    out = run_gpu(cfg, hd, dhd, rnd)
    rep = CK.check_round(cfg, hd, rnd, out, tol=TOL)
    pairs = 0
    for q in range(cfg.n_req):
        tok, par, cum, cnt = out["st_tok"][q], out["st_parent"][q], out["st_cum"][q], out["st_count"][q]
        for d in range(1, cfg.L):
            logq = {}
            for sl in range(cnt[d]):
                pt = int(tok[d - 1][par[d][sl]])
                lq = float(cum[d][sl]) - float(cum[d - 1][par[d][sl]])
                key = (pt, int(tok[d][sl]))
                if key in logq and logq[key][0] != par[d][sl]:
                    assert abs(logq[key][1] - lq) <= TOL, (q, d, key)
                    pairs += 1
                logq.setdefault(key, (par[d][sl], lq))
    say(f"  ok: nodes={rep.nodes_checked} same-token parent pairs compared={pairs}")
    # the boundary's Markov head (no A): the kernels skip the A*S contraction;
    # the result equals the A = 0 run bit for bit, fused and step by step
    dhm = ops.DeviceHead(hd0, markov=True)
    outm = run_gpu(cfg, hd, dhm, rnd)
    outs = run_gpu(cfg, hd, dhm, rnd, mode="steps", chunks=[(1, 1), (2, cfg.L)])
    for k in out:
        assert np.array_equal(outm[k], out[k]), k
        assert np.array_equal(outs[k], out[k]), k
    if cfg.B <= 511:
        so0, som = _serial_gpu_head(cfg, dhd, rnd), _serial_gpu_head(cfg, dhm, rnd)
        for k in so0:
            assert np.array_equal(so0[k], som[k]), k


def _serial_gpu_head(cfg, dhd, rnd):
    rb = ops.RoundBuffers(cfg)
    logits = ops.to_device(rnd.logits)
    hin = ops.to_device(rnd.H if cfg.D > 0 else rnd.h)
    ops.build_round(rb.dims, dhd, logits, hin, rb)
    so = ops.SerialOutputs(cfg)
    ops.build_serial(rb.dims, dhd, rb.cand_ids, rb.cand_logit, rb.h if cfg.D > 0 else hin, so)
    torch.cuda.synchronize()
    return so.numpy()


def _topk_rows(logits_bits, K, dtype="bf16"):
    """Run only the candidate step over [rows][V] logits."""
    rows, V = logits_bits.shape
    cfg = I.CONFIGS["qwen3_4b"].with_(n_req=1, L=rows, V=V, K=K, W=1, B=1, r=32, D=0, logits_dtype=dtype,
                                      weight_dtype="f32")
    dims = ops.make_dims(cfg)
    lg = ops.to_device(logits_bits.reshape(1, rows, V))
    ids = torch.zeros((1, rows, K), dtype=torch.int32, device="cuda")
    vals = torch.zeros((1, rows, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.workspace_size(dims), dtype=torch.uint8, device="cuda")
    ops.workspace_init(dims, ws)
    ops.topk_candidates(dims, lg, ids, vals, ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy()[0], vals.cpu().numpy()[0]


@pytest.mark.parametrize("K", [64, 512, 1024])
def test_topk_tie_heavy_rows_bit_exact(K):
    rng = np.random.default_rng(K)
    V = 151936
    rows = []
    rows.append(np.round(rng.normal(0, 2, V) * 4) / 4)            # heavy exact ties
    rows.append(np.full(V, 1.5))                                   # all equal
    r = np.zeros(V)
    r[rng.choice(V, V // 3, replace=False)] = -0.0                 # +0 / -0 mix
    r[rng.choice(V, 5, replace=False)] = 3.0
    rows.append(r)
    rows.append(rng.normal(0, 2, V))
    rows.append(np.round(rng.normal(0, 2, V)))                     # integer ties
    x = np.stack(rows).astype(np.float32)
    bits = I.f32_to_bf16_bits(x)
    say(f"case topk tie-heavy bf16 rows={x.shape[0]} V={V} K={K}")
    ids, vals = _topk_rows(bits, K)
    ref = I.bf16_bits_to_f32(bits).astype(np.float64)
    CK.check_candidates(ids, vals, ref, K, where=f"topk K={K}")
    say(f"case topk tie-heavy f32 rows={x.shape[0]} V={V} K={K}")
    ids, vals = _topk_rows(x, K, dtype="f32")
    CK.check_candidates(ids, vals, x.astype(np.float64), K, where=f"topk f32 K={K}")


def test_topk_stress_shape_all_rows():
    """Every row of a 64-request round at K = 512 (1024 rows of V = 151936
    bf16: four slices a row through the wide selection, then the slice-list
    merge) against the oracle's top-K, bit for bit."""
    cfg = I.CONFIGS["stress_64req"]
    rnd = I.make_round(cfg, 0, 0)
    rows = cfg.n_req * cfg.L
    say(f"case topk stress shape rows={rows} V={cfg.V} K={cfg.K}")
    dims = ops.make_dims(cfg)
    lg = ops.to_device(rnd.logits)
    ids = torch.zeros((cfg.n_req, cfg.L, cfg.K), dtype=torch.int32, device="cuda")
    vals = torch.zeros((cfg.n_req, cfg.L, cfg.K), dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.workspace_size(dims), dtype=torch.uint8, device="cuda")
    ops.workspace_init(dims, ws)
    ops.topk_candidates(dims, lg, ids, vals, ws)
    torch.cuda.synchronize()
    ref = I.bf16_bits_to_f32(rnd.logits.reshape(rows, cfg.V)).astype(np.float64)
    CK.check_candidates(ids.cpu().numpy().reshape(rows, cfg.K), vals.cpu().numpy().reshape(rows, cfg.K), ref, cfg.K,
                        where="stress topk")


@pytest.mark.parametrize("K", [65, 128, 256])
def test_topk_wide_selection_boosted_rows(K):
    """K above 64 takes the wide selection; rows drawn like the workloads'
    (noise plus boosted ids), bf16 and fp32."""
    cfg = I.CONFIGS["stress_64req"].with_(n_req=1, L=16)
    rnd = I.make_round(cfg, 3, K)
    bits = rnd.logits.reshape(cfg.L, cfg.V)
    say(f"case topk wide bf16 rows={cfg.L} V={cfg.V} K={K}")
    ids, vals = _topk_rows(bits, K)
    ref = I.bf16_bits_to_f32(bits).astype(np.float64)
    CK.check_candidates(ids, vals, ref, K, where=f"wide bf16 K={K}")
    x = ref.astype(np.float32) + np.float32(1e-3) * np.random.default_rng(K).standard_normal(ref.shape).astype(np.float32)
    say(f"case topk wide f32 rows={cfg.L} V={cfg.V} K={K}")
    ids, vals = _topk_rows(x, K, dtype="f32")
    CK.check_candidates(ids, vals, x.astype(np.float64), K, where=f"wide f32 K={K}")


@pytest.mark.parametrize("n_req,L,D,r", [(64, 16, 4096, 512), (5, 20, 2560, 256), (4, 16, 2560, 256)])
def test_head_states_many_rows(n_req, L, D, r):
    """h = P^T H through dartree_head_states at many rows (64 x 64 tiles
    staged through LDS; M = 100 leaves a partial tile) against the oracle's
    projection, within the score tolerance."""
    cfg = I.CONFIGS["stress_64req"].with_(n_req=n_req, L=L, D=D, r=r)
    rng = np.random.default_rng(n_req * 1000 + D)
    M = n_req * L
    Hb = I.f32_to_bf16_bits(rng.standard_normal((M, D)).astype(np.float32))
    Pb = I.f32_to_bf16_bits((rng.standard_normal((r, D)) / np.sqrt(D)).astype(np.float32))
    say(f"case head_states M={M} D={D} r={r}")
    dims = ops.make_dims(cfg)
    h = torch.zeros((M, r), dtype=torch.float32, device="cuda")
    ops.head_states(dims, ops.to_device(Hb), ops.to_device(Pb), h)
    torch.cuda.synchronize()
    ref = O.head_states(O.widen(Hb, "bf16"), O.widen(Pb, "bf16"))
    err = float(np.max(np.abs(h.cpu().numpy().astype(np.float64) - ref)))
    say(f"  max|dh| = {err:.2e}")
    assert err <= TOL, err


def _serial_gpu(cfg, seed=0, t=0):
    """The round (for its candidates and h), then the heap-serial builder."""
    hd, dhd = device_head(cfg, seed)
    rnd = I.make_round(cfg, seed, t)
    rb = ops.RoundBuffers(cfg)
    hin = ops.to_device(rnd.H if cfg.D > 0 else rnd.h)
    ops.build_round(rb.dims, dhd, ops.to_device(rnd.logits), hin, rb)
    so = ops.SerialOutputs(cfg)
    ops.build_serial(rb.dims, dhd, rb.cand_ids, rb.cand_logit, rb.h if cfg.D > 0 else hin, so)
    torch.cuda.synchronize()
    return hd, rnd, rb.numpy(), so.numpy()


def _paths(tok, parent, n):
    out = []
    for i in range(n):
        p, path = i, []
        while p >= 0:
            path.append(int(tok[p]))
            p = int(parent[p])
        out.append(tuple(reversed(path)))
    return out


@pytest.mark.parametrize("name", ["tiny", "serial_bf16", "qwen3_4b"])
def test_serial_heap_matches_oracle_pop_order(name):
    """dartree_build_serial against the oracle's literal serial heap (O7), pop
    by pop: token, depth, parent pop index exact, s_beta within 1e-4; a
    divergence is accepted only where the oracle's scores there are within
    the tolerance (a near-tie), and the comparison stops at it."""
    cfg = I.CONFIGS["tiny"] if name == "tiny" else (
        I.small_variant("qwen3_4b", name="serial_bf16", n_req=2, V=60000, L=6, K=64, W=12, B=32, r=256, D=256)
        if name == "serial_bf16" else I.CONFIGS["qwen3_4b"])
    say(f"case serial heap {cfg.name} n={cfg.n_req} L={cfg.L} K={cfg.K} B={cfg.B} r={cfg.r}")
    hd, rnd, _, g = _serial_gpu(cfg)
    wd = hd.dtype
    A, E, U = O.widen(hd.A, wd), O.widen(hd.E, wd), O.widen(hd.U, wd)
    logits = O.widen(rnd.logits, cfg.logits_dtype)
    h_all = O.head_states(O.widen(rnd.H, wd), O.widen(hd.Pt, wd)) if cfg.D > 0 else np.asarray(rnd.h, np.float64)
    checked = 0
    for q in range(cfg.n_req):
        ids = np.empty((cfg.L, cfg.K), np.int64)
        vals = np.empty((cfg.L, cfg.K), np.float64)
        for i in range(cfg.L):
            ids[i], vals[i] = O.topk_candidates(logits[q, i], cfg.K)
        pops = O.heap_serial_full(ids, vals, h_all[q], A, E, U, cfg.beta, cfg.B)
        index = {id(nd): i for i, nd in enumerate(pops)}
        n = int(g["n_sel"][q])
        assert n == len(pops), (n, len(pops))
        # the GPU's own sequence: parents first, depths chain, scores never rise
        seq = f"gpu tok {g['tok'][q, :n].tolist()} depth {g['depth'][q, :n].tolist()} parent {g['parent'][q, :n].tolist()}"
        for i in range(n):
            pi = int(g["parent"][q, i])
            assert -1 <= pi < i, seq
            assert int(g["depth"][q, i]) == (1 if pi < 0 else int(g["depth"][q, pi]) + 1), seq
            if i:
                assert g["score"][q, i] <= g["score"][q, i - 1] + TOL
        assert np.all(g["tok"][q, n:] == -1) and np.all(g["parent"][q, n:] == -2)
        for i, nd in enumerate(pops):
            po = index[id(nd.parent)] if nd.parent is not None and nd.parent.depth > 0 else -1
            same = (int(g["tok"][q, i]) == nd.tok and int(g["depth"][q, i]) == nd.depth
                    and int(g["parent"][q, i]) == po)
            if not same:
                assert abs(float(g["score"][q, i]) - nd.sbeta) <= TOL, (q, i, float(g["score"][q, i]), nd.sbeta)
                say(f"  request {q}: near-tie at pop {i}, compared {i} pops")
                break
            assert abs(float(g["score"][q, i]) - nd.sbeta) <= TOL, (q, i)
            checked += 1
    say(f"  ok: {checked} pops matched")


def test_serial_equals_deferred_when_width_covers_budget():
    """With W >= B the deferred round and the serial heap select the same
    nodes (both on the GPU; compared as sets of token paths)."""
    cfg = I.small_variant("qwen3_4b", name="serial_wide", n_req=2, V=60000, L=6, K=32, W=16, B=16, r=256, D=256)
    say(f"case serial vs deferred {cfg.name} W={cfg.W} B={cfg.B}")
    _, _, d, g = _serial_gpu(cfg)
    for q in range(cfg.n_req):
        nd, ns = int(d["n_sel"][q]), int(g["n_sel"][q])
        assert nd == ns
        pd = set(_paths(d["tok"][q], d["parent"][q], nd))
        ps = set(_paths(g["tok"][q], g["parent"][q], ns))
        assert pd == ps, (q, sorted(pd ^ ps)[:4])


@pytest.mark.parametrize("name,dh", [("tiny", 64), ("verify_bf16", 100), ("qwen3_4b", 128)])
def test_verify_tree_against_oracle(name, dh):
    """dartree_verify_tree on emitted rounds: acceptance length and path exact
    against the oracle's path enumeration, for targets taken from a random
    emitted path (then random tokens) and for random targets; the attention
    step within 1e-4 of the oracle's masked softmax."""
    cfg = I.CONFIGS["tiny"] if name == "tiny" else (
        I.small_variant("qwen3_4b", name="verify_bf16", n_req=3, V=60000, L=6, K=64, W=12, B=32, r=256, D=256)
        if name == "verify_bf16" else I.CONFIGS["qwen3_4b"])
    say(f"case verify {cfg.name} n={cfg.n_req} B={cfg.B} dh={dh}")
    hd, dhd = device_head(cfg)
    rnd = I.make_round(cfg, 0, 0)
    rb = ops.RoundBuffers(cfg)
    ops.build_round(rb.dims, dhd, ops.to_device(rnd.logits), ops.to_device(rnd.H if cfg.D > 0 else rnd.h), rb)
    torch.cuda.synchronize()
    e = rb.numpy()
    rng = np.random.default_rng(dh)
    n, L, B = cfg.n_req, cfg.L, cfg.B
    Q, K, V = (rng.standard_normal((n, B, dh)).astype(np.float32) for _ in range(3))
    for mode in ("path", "random"):
        target = rng.integers(0, cfg.V, (n, L)).astype(np.int32)
        if mode == "path":
            for q in range(n):
                ns = int(e["n_sel"][q])
                v = int(rng.integers(0, ns))
                while v >= 0:
                    target[q, int(e["depth"][q, v]) - 1] = int(e["tok"][q, v])
                    v = int(e["parent"][q, v])
        acc_len = torch.zeros((n,), dtype=torch.int32, device="cuda")
        acc_nodes = torch.zeros((n, L), dtype=torch.int32, device="cuda")
        out = torch.zeros((n, B, dh), dtype=torch.float32, device="cuda")
        ops.verify_tree(rb.dims, rb.n_sel, rb.tok, rb.depth, rb.parent, rb.mask, ops.to_device(target),
                        ops.to_device(Q), ops.to_device(K), ops.to_device(V), acc_len, acc_nodes, out)
        torch.cuda.synchronize()
        gl, gn, go = acc_len.cpu().numpy(), acc_nodes.cpu().numpy(), out.cpu().numpy()
        for q in range(n):
            ns = int(e["n_sel"][q])
            tau, path = O.accept_longest(e["tok"][q], e["depth"][q], e["parent"][q], ns, target[q])
            assert int(gl[q]) == tau, (mode, q, int(gl[q]), tau)
            assert gn[q].tolist() == path + [-1] * (L - len(path)), (mode, q)
            ref = O.tree_attention(Q[q].astype(np.float64), K[q].astype(np.float64), V[q].astype(np.float64),
                                   e["mask"][q], ns)
            err = float(np.max(np.abs(go[q].astype(np.float64) - ref)))
            assert err <= TOL, (mode, q, err)
        say(f"  {mode}: tau {gl.tolist()}")


def test_topk_small_and_ragged_rows():
    rng = np.random.default_rng(7)
    for V, K in [(1, 1), (7, 7), (9, 3), (4099, 64), (8192, 64), (8193, 100), (16385, 1024), (24577, 17)]:
        x = (np.round(rng.normal(0, 1, (3, V)) * 2) / 2).astype(np.float32)
        bits = I.f32_to_bf16_bits(x)
        say(f"case topk small V={V} K={K}")
        ids, vals = _topk_rows(bits, K)
        CK.check_candidates(ids, vals, I.bf16_bits_to_f32(bits).astype(np.float64), K, where=f"V={V}")


def test_topk_merge_of_several_slices():
    """Rows long enough to span 3, 4, 5 and 7 vocabulary slices with K > 64, so
    the slice lists go through the separate merge (lists padded to a power of
    two: 3 -> 4, 5 and 7 -> 8), up to the largest vocabulary the ABI takes
    (2^18), with tie-heavy values (steps of 0.5) and K not a power of two."""
    rng = np.random.default_rng(11)
    for V, K in [(100000, 128), (140000, 65), (200000, 333), (262144, 200)]:
        x = (np.round(rng.normal(0, 1, (3, V)) * 2) / 2).astype(np.float32)
        bits = I.f32_to_bf16_bits(x)
        say(f"case topk merge V={V} K={K}")
        ids, vals = _topk_rows(bits, K)
        CK.check_candidates(ids, vals, I.bf16_bits_to_f32(bits).astype(np.float64), K, where=f"V={V}")


def test_tree_mask_on_handmade_parents():
    B = 130
    rng = np.random.default_rng(3)
    par = np.full((2, B), -2, np.int32)
    n_sel = np.array([B, 70], np.int32)
    for q in range(2):
        for i in range(n_sel[q]):
            par[q, i] = rng.integers(-1, i) if i > 0 else -1
    par[0, 50] = 60      # forward pointer: ends the chain
    par[0, 51] = -7      # invalid: ends the chain
    cfg = I.small_variant("tiny", n_req=2, B=B)
    dims = ops.make_dims(cfg)
    words = (B + 63) // 64
    mask = torch.full((2, B, words), -1, dtype=torch.int64, device="cuda")
    say("case tree_mask handmade parents")
    ops.tree_mask(dims, torch.from_numpy(n_sel).cuda(), torch.from_numpy(par).cuda(), mask)
    torch.cuda.synchronize()
    got = mask.cpu().numpy().view(np.uint64)
    for q in range(2):
        exp = np.zeros((B, words), np.uint64)
        for i in range(n_sel[q]):
            j = i
            for _ in range(B + 1):
                exp[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
                p = par[q, j]
                if p >= j or p < -1 or p == -1:
                    break
                j = p
        assert np.array_equal(got[q], exp), q


# ---- the block-decoding kernel's numeric precondition (fp16 weights) ---------
def _range_case(seed=4):
    """A block-decoding shape (bf16 weights, r = 256, K = 64) with the head
    state supplied directly (D = 0)."""
    import dataclasses
    cfg = I.small_variant("qwen3_4b", name="range", n_req=2, V=6000, L=6, K=64, W=12, B=40, r=256, D=0)
    hd = I.make_head(cfg, seed)
    rnd = I.make_round(cfg, seed, 0)
    return cfg, dataclasses.replace(hd, A=hd.A.copy(), E=hd.E.copy(), U=hd.U.copy()), rnd


def test_head_check_flags_weights_beyond_fp16():
    cfg, hd, _ = _range_case()
    dims = ops.make_dims(cfg)
    assert ops.head_check(dims, ops.DeviceHead(hd)) == 0
    assert ops.head_check(dims, ops.DeviceHead(hd, markov=True)) == 0
    hd.U[5, 7] = I.f32_to_bf16_bits(np.array([70000.0], np.float32))[0]
    assert ops.head_check(dims, ops.DeviceHead(hd)) == 2
    hd.A[3, 4] = I.f32_to_bf16_bits(np.array([-1e5], np.float32))[0]
    assert ops.head_check(dims, ops.DeviceHead(hd)) == 3
    assert ops.head_check(dims, ops.DeviceHead(hd, markov=True)) == 2
    # 65280 (the largest bf16 below 2^16) is within fp16's range
    _, hd2, _ = _range_case()
    hd2.U[:, 3] = I.f32_to_bf16_bits(np.full(cfg.V, 65280.0, np.float32))
    assert ops.head_check(dims, ops.DeviceHead(hd2)) == 0


def test_head_beyond_fp16_runs_exactly_on_the_general_kernel():
    """One state column j of U holds 69632 (beyond fp16) for half of the
    tokens and 59904 (within it) for the other half, and only the root state
    reaches it (h_0[j] = 1e-3; A[j, :], E[:, j] and h_d[j] zero below the
    root, so every later state has s[j] = 0): the two halves' depth-1 logits
    differ by ~0.97, which the fp16 kernel would clamp to ~0.56. head_check
    flags U, and with DARTREE_HEAD_EXACT the round matches the oracle; the
    fp16 kernel, whose precondition the head breaks, does not."""
    cfg, hd, rnd = _range_case()
    j = 37
    big = np.random.default_rng(0).random(cfg.V) < 0.5
    hd.U[:, j] = I.f32_to_bf16_bits(np.where(big, 70000.0, 60000.0).astype(np.float32))
    hd.A[j, :] = 0
    hd.E[:, j] = 0
    h = rnd.h.copy()
    h[:, 0, j] = 1e-3
    h[:, 1:, j] = 0.0
    rnd.h = h
    dims = ops.make_dims(cfg)
    dx = ops.DeviceHead(hd, exact=True)
    assert ops.head_check(dims, dx) == 2
    say("case head beyond fp16, exact general kernel")
    out = run_gpu(cfg, hd, dx, rnd)
    rep = CK.check_round(cfg, hd, rnd, out, tol=TOL)
    PP.log_case("head beyond fp16 (exact)", rep)
    say("case head beyond fp16 on the fp16 kernel (precondition broken: must differ)")
    bad = run_gpu(cfg, hd, ops.DeviceHead(hd), rnd)
    with pytest.raises(CK.ParityError):
        CK.check_round(cfg, hd, rnd, bad, tol=TOL)


def test_large_root_state_is_rescaled_on_the_fp16_kernel():
    """h_0[j] = 70000 (beyond fp16) with U[c, j] = 2^-10 u_c, u_c uniform
    in [0, 1): the root's depth-1 logits get 68 u_c, which a state clamped to
    fp16's 65504 would turn into 64 u_c (the oracle run with that clamp
    differs from the true one, so the case can tell). The block-decoding
    kernel scales the root state by a power of two and must match the
    oracle."""
    cfg, hd, rnd = _range_case(5)
    j = 101
    u = np.random.default_rng(1).random(cfg.V).astype(np.float32)
    hd.U[:, j] = I.f32_to_bf16_bits(2.0 ** -10 * u)
    h = rnd.h.copy()
    h[:, 0, j] = 70000.0
    rnd.h = h
    clamped = copy.deepcopy(rnd)
    clamped.h[:, 0, j] = 65504.0
    a = O.round_all(cfg, hd, rnd)[0].levels[1]
    b = O.round_all(cfg, hd, clamped)[0].levels[1]
    assert max(abs(x.sbeta - y.sbeta) for x, y in zip(a, b)) > 1e-2
    dhd = ops.DeviceHead(hd)
    assert ops.head_check(ops.make_dims(cfg), dhd) == 0
    say("case large root state on the fp16 kernel")
    out = run_gpu(cfg, hd, dhd, rnd)
    rep = CK.check_round(cfg, hd, rnd, out, tol=TOL)
    PP.log_case("large root state (fp16 kernel)", rep)
