"""Torch-facing binding of libdartree (argument marshalling only).

PyTorch supplies device memory and the current stream; every step of the
round runs in the library's HIP kernels. Each function mirrors one C entry
point of include/dartree.h and raises DartreeError on a non-OK status.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

from . import _lib as C
from . import inputs as I


class DartreeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {C.status_string(status)}: {C.last_error()}")


def _check(status: int, where: str):
    if status != C.OK:
        raise DartreeError(status, where)


def _p(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(None)


def _stream(stream: Optional[torch.cuda.Stream] = None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_dims(cfg: I.Config) -> C.Dims:
    return C.Dims(n_req=cfg.n_req, L=cfg.L, V=cfg.V, K=cfg.K, W=cfg.W, B=cfg.B, r=cfg.r, D=cfg.D,
                  beta=cfg.beta, logits_dtype=C.BF16 if cfg.logits_dtype == I.BF16 else C.F32,
                  weight_dtype=C.BF16 if cfg.weight_dtype == I.BF16 else C.F32)


def to_device(arr: Optional[np.ndarray], device="cuda") -> Optional[torch.Tensor]:
    """Upload a generator array (uint16 bf16 bits travel as int16)."""
    if arr is None:
        return None
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceHead:
    """Head weights resident on the GPU."""

    def __init__(self, head: I.Head, device="cuda", markov: bool = False, exact: bool = False):
        """``markov``: pass no A (the Markov-head variant, A = 0); the kernels
        then skip the A s_parent contraction. ``exact``: set
        DARTREE_HEAD_EXACT (the general kernel for every shape; needed for a
        head that head_check flags)."""
        self.A = None if markov else to_device(head.A, device)
        self.E = to_device(head.E, device)
        self.U = to_device(head.U, device)
        self.Pt = to_device(head.Pt, device)
        self.c = C.Head(A=self.A.data_ptr() if self.A is not None else None, E=self.E.data_ptr(),
                        U=self.U.data_ptr(), Pt=self.Pt.data_ptr() if self.Pt is not None else None,
                        flags=C.HEAD_EXACT if exact else 0)


def head_check(dims: C.Dims, head: DeviceHead, stream=None) -> int:
    """dartree_head_check: bit 0 when A, bit 1 when U holds entries beyond
    fp16's range (the block-decoding kernel's precondition). Waits for the
    result (meant for once per head)."""
    flags = torch.full((1,), -1, dtype=torch.int32, device=head.E.device)
    _check(C.load().dartree_head_check(ctypes.byref(dims), ctypes.byref(head.c), _p(flags), _stream(stream)),
           "head_check")
    return int(flags.item())


def workspace_size(dims: C.Dims) -> int:
    n = ctypes.c_size_t(0)
    _check(C.load().dartree_workspace_size(ctypes.byref(dims), ctypes.byref(n)), "workspace_size")
    return int(n.value)


def round_plan(dims: C.Dims) -> dict:
    """How build_round runs for these sizes (launch count, scan slices and
    workgroups, where the slice lists are merged, which tree kernel, its LDS)."""
    info = C.RoundInfo()
    _check(C.load().dartree_round_plan(ctypes.byref(dims), ctypes.byref(info)), "round_plan")
    return {f: int(getattr(info, f)) for f, _ in C.RoundInfo._fields_}


class RoundBuffers:
    """Every device output of a round for one config, plus the workspace."""

    def __init__(self, cfg: I.Config, device="cuda"):
        self.cfg = cfg
        self.dims = make_dims(cfg)
        n, L, K, W, B, r = cfg.n_req, cfg.L, cfg.K, cfg.W, cfg.B, cfg.r
        i32, f32 = torch.int32, torch.float32
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)
        self.cand_ids = z((n, L, K), i32)
        self.cand_logit = z((n, L, K), f32)
        self.h = z((n, L, r), f32)
        self.st_tok = z((n, L, W), i32)
        self.st_parent = z((n, L, W), i32)
        self.st_cum = z((n, L, W), f32)
        self.st_sbeta = z((n, L, W), f32)
        self.st_count = z((n, L), i32)
        self.st_state = z((n, W, r), f32)
        self.n_sel = z((n,), i32)
        self.tok = z((n, B), i32)
        self.depth = z((n, B), i32)
        self.parent = z((n, B), i32)
        self.score = z((n, B), f32)
        self.slot = z((n, B), i32)
        self.mask = z((n, B, (B + 63) // 64), torch.int64)
        self.ws_bytes = workspace_size(self.dims)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.st = C.Supertree(tok=self.st_tok.data_ptr(), parent_slot=self.st_parent.data_ptr(),
                              cum=self.st_cum.data_ptr(), sbeta=self.st_sbeta.data_ptr(),
                              count=self.st_count.data_ptr(), state=self.st_state.data_ptr(), next_depth=1)
        workspace_init(self.dims, self.ws)
        self.width: Optional[torch.Tensor] = None
        self.budget: Optional[torch.Tensor] = None

    def set_request_sizes(self, width: Optional[torch.Tensor] = None, budget: Optional[torch.Tensor] = None):
        """Per-request width W_q and node budget B_q (device int32 [n_req], or
        None for the config's W and B); the library clamps them to [1, W] and
        [1, B]. The tensors are kept here so they outlive the calls that read
        them."""
        n = self.cfg.n_req
        for name, t in (("width", width), ("budget", budget)):
            if t is not None and (t.dtype != torch.int32 or t.numel() != n or not t.is_cuda or not t.is_contiguous()):
                raise ValueError(f"{name}: a contiguous device int32 tensor of {n} entries is required")
        self.width, self.budget = width, budget
        self.st.width = _p(width)
        self.st.budget = _p(budget)

    def numpy(self) -> Dict[str, np.ndarray]:
        """Host copies laid out as the parity checker expects."""
        g = lambda t: t.detach().cpu().numpy()
        return {"cand_ids": g(self.cand_ids), "cand_logit": g(self.cand_logit), "h": g(self.h),
                "st_tok": g(self.st_tok), "st_parent": g(self.st_parent), "st_cum": g(self.st_cum),
                "st_sbeta": g(self.st_sbeta), "st_count": g(self.st_count), "n_sel": g(self.n_sel),
                "tok": g(self.tok), "depth": g(self.depth), "parent": g(self.parent), "score": g(self.score),
                "slot": g(self.slot), "mask": g(self.mask).view(np.uint64)}


def workspace_init(dims: C.Dims, ws: torch.Tensor, stream=None):
    _check(C.load().dartree_workspace_init(ctypes.byref(dims), _p(ws), ws.numel(), _stream(stream)),
           "workspace_init")


def head_states(dims: C.Dims, H: torch.Tensor, Pt: torch.Tensor, h: torch.Tensor, stream=None):
    _check(C.load().dartree_head_states(ctypes.byref(dims), _p(H), _p(Pt), _p(h), _stream(stream)), "head_states")


def topk_candidates(dims: C.Dims, logits: torch.Tensor, cand_ids: torch.Tensor, cand_logit: torch.Tensor,
                    ws: torch.Tensor, stream=None):
    _check(C.load().dartree_topk_candidates(ctypes.byref(dims), _p(logits), _p(cand_ids), _p(cand_logit), _p(ws),
                                            ws.numel(), _stream(stream)), "topk_candidates")


def lmhead_workspace_size(dims: C.Dims) -> int:
    n = ctypes.c_size_t(0)
    _check(C.load().dartree_lmhead_workspace_size(ctypes.byref(dims), ctypes.byref(n)), "lmhead_workspace_size")
    return int(n.value)


def lmhead_topk(dims: C.Dims, X: torch.Tensor, Wlm: torch.Tensor, cand_ids: torch.Tensor, cand_logit: torch.Tensor,
                ws: torch.Tensor, stream=None):
    """Candidates straight from the drafter's hidden states through
    dartree_lmhead_topk (the LM head fused with the top-K)."""
    _check(C.load().dartree_lmhead_topk(ctypes.byref(dims), _p(X), _p(Wlm), _p(cand_ids), _p(cand_logit), _p(ws),
                                        ws.numel(), _stream(stream)), "lmhead_topk")


def expand_depth(dims: C.Dims, head: DeviceHead, cand_ids: torch.Tensor, cand_logit: torch.Tensor,
                 h: torch.Tensor, rb: RoundBuffers, depth_begin: int, depth_end: int, stream=None):
    _check(C.load().dartree_expand_depth(ctypes.byref(dims), ctypes.byref(head.c), _p(cand_ids), _p(cand_logit),
                                         _p(h), ctypes.byref(rb.st), depth_begin, depth_end, _stream(stream)),
           "expand_depth")


def select_topB(dims: C.Dims, rb: RoundBuffers, stream=None):
    _check(C.load().dartree_select_topB(ctypes.byref(dims), ctypes.byref(rb.st), _p(rb.n_sel), _p(rb.tok),
                                        _p(rb.depth), _p(rb.parent), _p(rb.score), _p(rb.slot), _stream(stream)),
           "select_topB")


def tree_mask(dims: C.Dims, n_sel: torch.Tensor, parent: torch.Tensor, mask: torch.Tensor, stream=None):
    _check(C.load().dartree_tree_mask(ctypes.byref(dims), _p(n_sel), _p(parent), _p(mask), _stream(stream)),
           "tree_mask")


def build_round(dims: C.Dims, head: DeviceHead, logits: torch.Tensor, H_or_h: torch.Tensor, rb: RoundBuffers,
                stream=None):
    """The whole round (a0..a5) through dartree_build_round."""
    rb.st.next_depth = 1
    _check(C.load().dartree_build_round(ctypes.byref(dims), ctypes.byref(head.c), _p(logits), _p(H_or_h),
                                        _p(rb.cand_ids), _p(rb.cand_logit), _p(rb.h), ctypes.byref(rb.st),
                                        _p(rb.n_sel), _p(rb.tok), _p(rb.depth), _p(rb.parent), _p(rb.score),
                                        _p(rb.slot), _p(rb.mask), _p(rb.ws), rb.ws_bytes, _stream(stream)),
           "build_round")


def build_round_noalloc(dims: C.Dims, head: DeviceHead, logits: torch.Tensor, H_or_h: torch.Tensor,
                        rb: RoundBuffers, stream=None):
    """The whole round through dartree_build_round_noalloc: the library's own
    device scratch instead of rb.ws (which is not touched)."""
    rb.st.next_depth = 1
    _check(C.load().dartree_build_round_noalloc(ctypes.byref(dims), ctypes.byref(head.c), _p(logits), _p(H_or_h),
                                                _p(rb.cand_ids), _p(rb.cand_logit), _p(rb.h), ctypes.byref(rb.st),
                                                _p(rb.n_sel), _p(rb.tok), _p(rb.depth), _p(rb.parent),
                                                _p(rb.score), _p(rb.slot), _p(rb.mask), _stream(stream)),
           "build_round_noalloc")


def run_steps(dims: C.Dims, head: DeviceHead, logits: torch.Tensor, H_or_h: torch.Tensor, rb: RoundBuffers,
              depth_chunks=None, stream=None):
    """The round through the individual entry points: head_states (D > 0),
    topk_candidates, expand_depth over ``depth_chunks`` ranges (default: one
    call per depth), select_topB and tree_mask."""
    cfg = rb.cfg
    h = H_or_h
    if cfg.D > 0:
        head_states(dims, H_or_h, head.Pt, rb.h, stream)
        h = rb.h
    topk_candidates(dims, logits, rb.cand_ids, rb.cand_logit, rb.ws, stream)
    rb.st.next_depth = 1
    ranges = depth_chunks or [(d, d) for d in range(1, cfg.L + 1)]
    for d0, d1 in ranges:
        expand_depth(dims, head, rb.cand_ids, rb.cand_logit, h, rb, d0, d1, stream)
    select_topB(dims, rb, stream)
    tree_mask(dims, rb.n_sel, rb.parent, rb.mask, stream)


def serial_workspace_size(dims: C.Dims) -> int:
    n = ctypes.c_size_t(0)
    _check(C.load().dartree_serial_workspace_size(ctypes.byref(dims), ctypes.byref(n)), "serial_workspace_size")
    return n.value


class SerialOutputs:
    """Outputs of the heap-serial construction for one config, in pop order."""

    def __init__(self, cfg: I.Config, device="cuda"):
        n, B = cfg.n_req, cfg.B
        self.dims = make_dims(cfg)
        self.n_sel = torch.zeros((n,), dtype=torch.int32, device=device)
        self.tok = torch.zeros((n, B), dtype=torch.int32, device=device)
        self.depth = torch.zeros((n, B), dtype=torch.int32, device=device)
        self.parent = torch.zeros((n, B), dtype=torch.int32, device=device)
        self.score = torch.zeros((n, B), dtype=torch.float32, device=device)
        self.ws_bytes = serial_workspace_size(self.dims)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)

    def numpy(self) -> Dict[str, np.ndarray]:
        g = lambda t: t.detach().cpu().numpy()
        return {"n_sel": g(self.n_sel), "tok": g(self.tok), "depth": g(self.depth), "parent": g(self.parent),
                "score": g(self.score)}


def build_serial(dims: C.Dims, head: DeviceHead, cand_ids: torch.Tensor, cand_logit: torch.Tensor,
                 h: torch.Tensor, out: SerialOutputs, stream=None):
    """The heap-serial construction through dartree_build_serial."""
    _check(C.load().dartree_build_serial(ctypes.byref(dims), ctypes.byref(head.c), _p(cand_ids), _p(cand_logit),
                                         _p(h), _p(out.n_sel), _p(out.tok), _p(out.depth), _p(out.parent),
                                         _p(out.score), _p(out.ws), out.ws_bytes, _stream(stream)),
           "build_serial")


def verify_tree(dims: C.Dims, n_sel: torch.Tensor, tok: torch.Tensor, depth: torch.Tensor, parent: torch.Tensor,
                mask: torch.Tensor, target: torch.Tensor, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                accepted_len: torch.Tensor, accepted_nodes: torch.Tensor, attn_out: torch.Tensor, stream=None):
    """The verification consumer through dartree_verify_tree."""
    _check(C.load().dartree_verify_tree(ctypes.byref(dims), _p(n_sel), _p(tok), _p(depth), _p(parent), _p(mask),
                                        _p(target), _p(Q), _p(K), _p(V), int(Q.shape[-1]), _p(accepted_len),
                                        _p(accepted_nodes), _p(attn_out), _stream(stream)),
           "verify_tree")


def set_split_wait(microseconds: int):
    """Bound of the split general tree kernel's wait for another part of a
    request (dartree_set_split_wait); 0 makes every part compute the whole
    contraction itself."""
    _check(C.load().dartree_set_split_wait(int(microseconds)), "set_split_wait")


def set_stage_events(events: Optional[list]):
    """Profiling hook: record the given four torch.cuda.Event objects around the
    stages of every following build_round on this thread (scan, merge, tree
    kernel); None clears it. Argument marshalling only."""
    lib = C.load()
    if not events:
        _check(lib.dartree_set_stage_events(None, 0), "set_stage_events")
        return
    if len(events) != 4:
        raise ValueError("need four events")
    for e in events:
        if int(e.cuda_event) == 0:   # torch creates the HIP event on its first record
            e.record()
    arr = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(int(e.cuda_event)) for e in events])
    _check(lib.dartree_set_stage_events(arr, 4), "set_stage_events")


def stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Measurement utility: one read-only pass over buf (dartree_stream_read)."""
    nbytes = (buf.numel() * buf.element_size()) // 16 * 16
    _check(C.load().dartree_stream_read(_p(buf), nbytes, _p(sink), _stream(stream)), "stream_read")



def cu_read(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Measurement utility: the same read by one workgroup (dartree_cu_read)."""
    nbytes = (buf.numel() * buf.element_size()) // 16 * 16
    _check(C.load().dartree_cu_read(_p(buf), nbytes, _p(sink), _stream(stream)), "cu_read")
