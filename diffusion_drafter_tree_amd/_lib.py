"""ctypes declarations of libdartree's C ABI (include/dartree.h).

Argument marshalling only: every step of the round runs in the library's HIP
kernels. Loading fails loudly when the library has not been built; there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdartree.so")

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_UNSUPPORTED = 2
ERR_WORKSPACE_TOO_SMALL = 3
ERR_HIP = 4

F32 = 0
BF16 = 1

NOALLOC_SCRATCH_BYTES = 32 << 20   # DARTREE_NOALLOC_SCRATCH_BYTES


class Dims(ctypes.Structure):
    _fields_ = [("n_req", c_int32), ("L", c_int32), ("V", c_int32), ("K", c_int32), ("W", c_int32),
                ("B", c_int32), ("r", c_int32), ("D", c_int32), ("beta", c_float),
                ("logits_dtype", c_int32), ("weight_dtype", c_int32)]


HEAD_EXACT = 1   # DARTREE_HEAD_EXACT


class Head(ctypes.Structure):
    _fields_ = [("A", c_void_p), ("E", c_void_p), ("U", c_void_p), ("Pt", c_void_p), ("flags", c_int32)]


class RoundInfo(ctypes.Structure):
    _fields_ = [("n_launches", c_int32), ("scan_slices", c_int32), ("scan_workgroups", c_int32),
                ("merge_separate", c_int32), ("tree_kernel", c_int32), ("tree_lds_bytes", c_int32),
                ("tree_parts", c_int32)]


class Supertree(ctypes.Structure):
    _fields_ = [("tok", c_void_p), ("parent_slot", c_void_p), ("cum", c_void_p), ("sbeta", c_void_p),
                ("count", c_void_p), ("state", c_void_p), ("next_depth", c_int32),
                ("width", c_void_p), ("budget", c_void_p)]


PD = POINTER(Dims)
PH = POINTER(Head)
PS = POINTER(Supertree)

# name -> (restype, argtypes)
SIGNATURES = {
    "dartree_status_string": (c_char_p, [c_int32]),
    "dartree_last_error": (c_char_p, []),
    "dartree_version": (c_int32, []),
    "dartree_workspace_size": (c_int32, [PD, POINTER(c_size_t)]),
    "dartree_round_plan": (c_int32, [PD, POINTER(RoundInfo)]),
    "dartree_workspace_init": (c_int32, [PD, c_void_p, c_size_t, c_void_p]),
    "dartree_head_states": (c_int32, [PD, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dartree_head_check": (c_int32, [PD, PH, c_void_p, c_void_p]),
    "dartree_topk_candidates": (c_int32, [PD, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "dartree_expand_depth": (c_int32, [PD, PH, c_void_p, c_void_p, c_void_p, PS, c_int32, c_int32, c_void_p]),
    "dartree_select_topB": (c_int32, [PD, PS, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p]),
    "dartree_tree_mask": (c_int32, [PD, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dartree_build_round": (c_int32, [PD, PH, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, PS,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_size_t, c_void_p]),
    "dartree_build_round_noalloc": (c_int32, [PD, PH, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, PS,
                                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_void_p]),
    "dartree_lmhead_workspace_size": (c_int32, [PD, POINTER(c_size_t)]),
    "dartree_lmhead_topk": (c_int32, [PD, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "dartree_stream_read": (c_int32, [c_void_p, c_size_t, c_void_p, c_void_p]),
    "dartree_cu_read": (c_int32, [c_void_p, c_size_t, c_void_p, c_void_p]),
    "dartree_set_stage_events": (c_int32, [POINTER(c_void_p), c_int32]),
    "dartree_set_split_wait": (c_int32, [c_int32]),
    "dartree_serial_workspace_size": (c_int32, [PD, POINTER(c_size_t)]),
    "dartree_verify_tree": (c_int32, [PD, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dartree_build_serial": (c_int32, [PD, PH, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
}

_lib = None


class LibraryMissing(ImportError):
    pass


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdartree.so (once) and declare its prototypes."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise LibraryMissing(f"{path} is not built; run __graft_entry__.build() "
                             f"(python -m diffusion_drafter_tree_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(s: int) -> str:
    return load().dartree_status_string(s).decode()


def last_error() -> str:
    return load().dartree_last_error().decode()
