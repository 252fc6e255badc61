"""Shared test helpers: oracle results laid out like the library's outputs."""
import numpy as np


def oracle_as_outputs(cfg, results):
    """Pack oracle RequestResults into the arrays the HIP path returns
    (fp32 scores), for checker self-tests."""
    n, L, K, W, B = cfg.n_req, cfg.L, cfg.K, cfg.W, cfg.B
    words = (B + 63) // 64
    out = {
        "cand_ids": np.zeros((n, L, K), np.int32), "cand_logit": np.zeros((n, L, K), np.float32),
        "st_tok": np.full((n, L, W), -1, np.int32), "st_parent": np.full((n, L, W), -1, np.int32),
        "st_cum": np.full((n, L, W), -np.inf, np.float32), "st_sbeta": np.full((n, L, W), -np.inf, np.float32),
        "st_count": np.zeros((n, L), np.int32), "n_sel": np.zeros(n, np.int32),
        "tok": np.zeros((n, B), np.int32), "depth": np.zeros((n, B), np.int32), "parent": np.zeros((n, B), np.int32),
        "score": np.zeros((n, B), np.float32), "slot": np.zeros((n, B), np.int32),
        "mask": np.zeros((n, B, words), np.uint64),
    }
    for q, r in enumerate(results):
        out["cand_ids"][q] = r.cand_ids
        out["cand_logit"][q] = r.cand_vals
        for d in range(1, L + 1):
            lvl = r.levels[d]
            out["st_count"][q, d - 1] = len(lvl)
            for s, nd in enumerate(lvl):
                out["st_tok"][q, d - 1, s] = nd.tok
                out["st_parent"][q, d - 1, s] = nd.parent_slot
                out["st_cum"][q, d - 1, s] = nd.cum
                out["st_sbeta"][q, d - 1, s] = nd.sbeta
        em = r.emitted
        out["n_sel"][q] = em.n_sel
        out["tok"][q], out["depth"][q], out["parent"][q] = em.tok, em.depth, em.parent
        out["slot"][q] = em.slot
        for i in range(B):
            out["score"][q, i] = out["st_sbeta"][q, em.depth[i] - 1, em.slot[i]] if i < em.n_sel else -np.inf
        out["mask"][q] = r.mask
    return out
