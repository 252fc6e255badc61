"""Oracle work for the GPU parity tests, spread over worker processes.

The workers are *spawned* (never forked from a process that holds a GPU
context). They import numpy, the seeded input generators and the oracle only;
never torch or the HIP library. A worker draws a head once per (config, seed)
and keeps it with its exactly widened weights.

``log_case`` appends one JSON line per checked case to the file named by the
environment variable DARTREE_PARITY_LOG (when set), so a GPU run keeps its
tie-event counts and error maxima even when pytest swallows stdout.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import multiprocessing as mp
import os
import time

import numpy as np

from diffusion_drafter_tree_amd import inputs as I
from oracle import check as CK
from oracle import dartree_oracle as O

_HEAD = {}


def _head(cfg, seed):
    key = (cfg, seed)
    if key not in _HEAD:
        _HEAD.clear()
        hd = I.make_head(cfg, seed)
        _HEAD[key] = (hd, CK.widen_head(hd))
    return _HEAD[key]


def gen_round(cfg, seed, t):
    """The seeded round t (worker side)."""
    return I.make_round(cfg, seed, t)


def boundary_ties(logits_rows, dtype, K):
    """Rows whose K-th and (K+1)-th largest values are equal: an exact tie
    across the candidate boundary, settled by the token-id order."""
    x = O.widen(logits_rows, dtype).reshape(-1, logits_rows.shape[-1])
    if x.shape[1] <= K:
        return 0
    part = -np.partition(-x, K, axis=1)[:, :K + 1]
    part.sort(axis=1)
    return int(np.sum(part[:, 0] == part[:, 1]))


def check_job(cfg, seed, t, out, requests, tol):
    """check_round for round t (restricted to ``requests``); returns the
    report and the number of rows with an exact tie at the K boundary."""
    hd, wid = _head(cfg, seed)
    rnd = I.make_round(cfg, seed, t)
    rep = CK.check_round(cfg, hd, rnd, out, tol=tol, requests=requests, widened=wid)
    qs = list(range(cfg.n_req)) if requests is None else list(requests)
    ties = boundary_ties(rnd.logits[qs], cfg.logits_dtype, cfg.K)
    return rep, ties


def workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def pool(n=None):
    return cf.ProcessPoolExecutor(max_workers=n or workers(), mp_context=mp.get_context("spawn"))


def log_case(case, rep=None, **fields):
    path = os.environ.get("DARTREE_PARITY_LOG")
    rec = {"case": case, "time": time.strftime("%H:%M:%S")}
    if rep is not None:
        rec.update(nodes=rep.nodes_checked, tie_events_level=rep.tie_events_level,
                   tie_events_topB=rep.tie_events_topB, max_score_err=rep.max_score_err,
                   max_cum_err=rep.max_cum_err, max_h_err=rep.max_h_err, tie_log=rep.tie_log[:20])
    rec.update(fields)
    line = json.dumps(rec)
    print(f"[parity] {line}", flush=True)
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "a") as f:
            f.write(line + "\n")
