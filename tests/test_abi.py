"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects invalid arguments on the host before touching the device."""
import ctypes
import os
import re

import pytest

from diffusion_drafter_tree_amd import _lib as C
from diffusion_drafter_tree_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dartree.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dartree_[a-z_A-Z0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(C.LIB_PATH):
        pytest.fail("libdartree.so is not built (run __graft_entry__.build())")
    return C.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(C.SIGNATURES), "binding and header disagree"


def test_version_and_status_strings(lib):
    assert lib.dartree_version() == 4
    assert C.status_string(0) == "DARTREE_OK"
    assert C.status_string(3) == "DARTREE_ERR_WORKSPACE_TOO_SMALL"
    assert C.status_string(99) == "DARTREE_UNKNOWN_STATUS"


def dims(**kw):
    base = dict(n_req=1, L=16, V=151936, K=64, W=12, B=64, r=256, D=2560, beta=-0.15,
                logits_dtype=C.BF16, weight_dtype=C.BF16)
    base.update(kw)
    return C.Dims(**base)


def ws_size(lib, d):
    n = ctypes.c_size_t(0)
    st = lib.dartree_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def test_workspace_size_values(lib):
    st, n = ws_size(lib, dims())
    assert st == C.OK
    # a 151936-entry bf16 row spans 4 slices of <= 1024 threads x 5 vectors x 8
    # values: 16 rows x 4 sorted lists x 64 keys of 8 bytes, then an fp16 copy
    # of A (256 x 256) for bf16 weights of rank 256
    afrag = 256 * 256 * 2
    assert n == 16 * 4 * 64 * 8 + afrag
    # fp32 rows of that length take 8 slices (4 values per vector)
    st, n = ws_size(lib, dims(logits_dtype=C.F32))
    assert st == C.OK and n == 16 * 8 * 64 * 8 + afrag
    # fp32 weights: no A copy
    st, n = ws_size(lib, dims(weight_dtype=C.F32))
    assert st == C.OK and n == 16 * 4 * 64 * 8
    st, n = ws_size(lib, dims(V=1024, L=6, K=8, W=3, B=16, r=16, D=0, logits_dtype=C.F32, weight_dtype=C.F32))
    assert st == C.OK and n >= 6 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(beta=0.1), C.ERR_INVALID_ARGUMENT),
    (dict(beta=float("nan")), C.ERR_INVALID_ARGUMENT),
    (dict(beta=float("inf")), C.ERR_INVALID_ARGUMENT),
    (dict(K=0), C.ERR_INVALID_ARGUMENT),
    (dict(n_req=0), C.ERR_INVALID_ARGUMENT),
    (dict(K=200000), C.ERR_INVALID_ARGUMENT),
    (dict(D=-1), C.ERR_INVALID_ARGUMENT),
    (dict(L=32), C.ERR_UNSUPPORTED),
    (dict(K=2048), C.ERR_UNSUPPORTED),
    (dict(W=65), C.ERR_UNSUPPORTED),
    (dict(B=1025), C.ERR_UNSUPPORTED),
    (dict(r=1056), C.ERR_UNSUPPORTED),
    (dict(V=300000), C.ERR_UNSUPPORTED),
    (dict(W=64, r=256), C.ERR_UNSUPPORTED),
    (dict(W=16, K=1024), C.ERR_UNSUPPORTED),
    (dict(logits_dtype=7), C.ERR_UNSUPPORTED),
])
def test_invalid_dims_are_rejected(lib, kw, status):
    st, _ = ws_size(lib, dims(**kw))
    assert st == status, C.last_error()
    assert C.last_error() != ""


def test_beta_zero_is_allowed(lib):
    assert ws_size(lib, dims(beta=0.0))[0] == C.OK
    assert ws_size(lib, dims(beta=-0.0))[0] == C.OK


def test_null_and_misaligned_pointers_rejected_before_any_launch(lib):
    d = dims()
    st, n = ws_size(lib, d)
    fake = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
    mis = ctypes.c_void_p(0x10004)
    s = ctypes.c_void_p(None)
    assert lib.dartree_topk_candidates(ctypes.byref(d), None, fake, fake, fake, n, s) == C.ERR_INVALID_ARGUMENT
    assert "logits" in C.last_error()
    assert lib.dartree_topk_candidates(ctypes.byref(d), mis, fake, fake, fake, n, s) == C.ERR_INVALID_ARGUMENT
    assert "aligned" in C.last_error()
    assert lib.dartree_topk_candidates(ctypes.byref(d), fake, fake, fake, fake, n - 1, s) == \
        C.ERR_WORKSPACE_TOO_SMALL
    assert lib.dartree_head_states(ctypes.byref(dims(D=0)), fake, fake, fake, s) == C.ERR_INVALID_ARGUMENT
    assert lib.dartree_tree_mask(ctypes.byref(d), fake, fake, ctypes.c_void_p(0x10004), s) == C.ERR_INVALID_ARGUMENT


def test_read_probes_validate_on_host(lib):
    """The two measurement utilities reject NULL or misaligned buffers and byte
    counts that are zero or not a multiple of 16 before any launch."""
    fake = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
    s = ctypes.c_void_p(None)
    for fn in (lib.dartree_stream_read, lib.dartree_cu_read):
        assert fn(None, 1024, fake, s) == C.ERR_INVALID_ARGUMENT
        assert fn(ctypes.c_void_p(0x10008), 1024, fake, s) == C.ERR_INVALID_ARGUMENT
        assert "aligned" in C.last_error()
        assert fn(fake, 1024, None, s) == C.ERR_INVALID_ARGUMENT
        for nbytes in (0, 15, 1000):
            assert fn(fake, nbytes, fake, s) == C.ERR_INVALID_ARGUMENT
            assert "multiple of 16" in C.last_error()


def test_expand_depth_order_is_enforced(lib):
    d = dims()
    fake = 0x10000
    head = C.Head(A=fake, E=fake, U=fake, Pt=fake)
    st = C.Supertree(tok=fake, parent_slot=fake, cum=fake, sbeta=fake, count=fake, state=fake, next_depth=1)
    s = ctypes.c_void_p(None)
    f = ctypes.c_void_p(fake)
    # depth_begin must equal next_depth
    assert lib.dartree_expand_depth(ctypes.byref(d), ctypes.byref(head), f, f, f, ctypes.byref(st), 2, 2, s) == \
        C.ERR_INVALID_ARGUMENT
    # range outside [1, L]
    assert lib.dartree_expand_depth(ctypes.byref(d), ctypes.byref(head), f, f, f, ctypes.byref(st), 1, 17, s) == \
        C.ERR_INVALID_ARGUMENT
    assert lib.dartree_expand_depth(ctypes.byref(d), ctypes.byref(head), f, f, f, ctypes.byref(st), 1, 0, s) == \
        C.ERR_INVALID_ARGUMENT
    assert st.next_depth == 1
    # select needs a complete supertree
    assert lib.dartree_select_topB(ctypes.byref(d), ctypes.byref(st), f, f, f, f, f, f, s) == C.ERR_INVALID_ARGUMENT
    assert "incomplete" in C.last_error()
    # a round must start at depth 1
    st.next_depth = 5
    assert lib.dartree_build_round(ctypes.byref(d), ctypes.byref(head), f, f, f, f, f, ctypes.byref(st), f, f, f, f,
                                   f, f, f, f, 1 << 20, s) == C.ERR_INVALID_ARGUMENT


def test_binding_config_dims_match_header_limits():
    from diffusion_drafter_tree_amd import ops
    for name in I.CONFIG_ORDER:
        d = ops.make_dims(I.CONFIGS[name])
        st, _ = ws_size(C.load(), d)
        assert st == C.OK, (name, C.last_error())


def test_stage_event_hook_validates_on_host(lib):
    assert lib.dartree_set_stage_events(None, 0) == C.OK
    assert lib.dartree_set_stage_events(None, 4) == C.ERR_INVALID_ARGUMENT
    arr = (ctypes.c_void_p * 4)(0x10, None, 0x30, 0x40)
    assert lib.dartree_set_stage_events(arr, 4) == C.ERR_INVALID_ARGUMENT
    assert "NULL" in C.last_error()
    assert lib.dartree_set_stage_events(arr, 3) == C.ERR_INVALID_ARGUMENT


def test_round_plan_query(lib):
    from diffusion_drafter_tree_amd import ops
    info = ops.round_plan(ops.make_dims(I.CONFIGS["qwen3_4b"]))
    # bf16 weights, K=64, W=12, r=256: the block-decoding kernel merges the slice lists itself
    assert info["tree_kernel"] == 1 and info["merge_separate"] == 0 and info["n_launches"] == 2
    assert info["scan_slices"] > 1
    # 16 rows x slices, 16 head projection tiles, 16 workgroups staging A fragments
    assert info["scan_workgroups"] == 16 * info["scan_slices"] + (256 // 16) * 1 + 16
    assert 0 < info["tree_lds_bytes"] <= 160 * 1024
    # r=512 and K=512: the general tree kernel, with the merge as its own launch
    big = ops.round_plan(ops.make_dims(I.CONFIGS["stress_64req"]))
    assert big["tree_kernel"] == 0 and big["merge_separate"] == (1 if big["scan_slices"] > 1 else 0)
    assert big["n_launches"] == 2 + big["merge_separate"]
    tiny = ops.round_plan(ops.make_dims(I.CONFIGS["tiny"]))
    assert tiny["scan_slices"] == 1 and tiny["merge_separate"] == 0 and tiny["n_launches"] == 2
    assert lib.dartree_round_plan(ctypes.byref(ops.make_dims(I.CONFIGS["tiny"])), None) == C.ERR_INVALID_ARGUMENT
    d = ops.make_dims(I.CONFIGS["tiny"])
    d.beta = 0.5
    assert lib.dartree_round_plan(ctypes.byref(d), ctypes.byref(C.RoundInfo())) == C.ERR_INVALID_ARGUMENT


def test_gpu_parity_cases_cover_the_block_decoding_kernel(lib):
    """The fast_* GPU parity cases run on the block-decoding tree kernel (the
    others on the general one), so its shapes are covered: K = 16, 32, 64,
    W = 1 .. 16, L = 1 .. 31, B up to 256 (several mask words), one and many
    vocabulary slices."""
    import importlib.util
    from diffusion_drafter_tree_amd import ops
    path = os.path.join(ROOT, "tests", "test_gpu_parity.py")
    spec = importlib.util.spec_from_file_location("gpu_parity_cases", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert len(mod.FAST) >= 6
    for name, cfg in mod.SMALL.items():
        info = ops.round_plan(ops.make_dims(cfg))
        assert info["tree_kernel"] == (1 if name in mod.FAST else 0), (name, info)
    slices = {ops.round_plan(ops.make_dims(mod.SMALL[n]))["scan_slices"] for n in mod.FAST}
    assert 1 in slices and max(slices) > 1
    # both key widths of the slice-list merge: bf16 and fp32 logits over several slices
    multi = [mod.SMALL[n] for n in mod.FAST if ops.round_plan(ops.make_dims(mod.SMALL[n]))["scan_slices"] > 1]
    assert {c.logits_dtype for c in multi} == {"bf16", "f32"}


def test_serial_builder_validates_on_host(lib):
    """dartree_build_serial: workspace size n (B + 1) r fp32; B above 511,
    NULL or misaligned pointers and a short workspace are rejected before any
    launch."""
    d = dims()
    n = ctypes.c_size_t(0)
    assert lib.dartree_serial_workspace_size(ctypes.byref(d), ctypes.byref(n)) == C.OK
    assert n.value == d.n_req * (d.B + 1) * d.r * 4
    fake = ctypes.c_void_p(0x10000)
    s = ctypes.c_void_p(None)
    head = C.Head(A=0x10000, E=0x10000, U=0x10000, Pt=0x10000)
    args = lambda dd, ws_bytes, **kw: [ctypes.byref(dd), ctypes.byref(head)] + [kw.get(k, fake) for k in (
        "cand_ids", "cand_logit", "h", "n_sel", "tok", "depth", "parent", "score", "ws")] + [ws_bytes, s]
    big = dims(B=600, W=16)
    nb = ctypes.c_size_t(0)
    assert lib.dartree_serial_workspace_size(ctypes.byref(big), ctypes.byref(nb)) == C.OK
    assert lib.dartree_build_serial(*args(big, nb.value)) == C.ERR_UNSUPPORTED
    assert "511" in C.last_error()
    assert lib.dartree_build_serial(*args(d, n.value, h=None)) == C.ERR_INVALID_ARGUMENT
    assert "h" in C.last_error()
    assert lib.dartree_build_serial(*args(d, n.value, score=ctypes.c_void_p(0x10002))) == C.ERR_INVALID_ARGUMENT
    assert lib.dartree_build_serial(*args(d, n.value - 1)) == C.ERR_WORKSPACE_TOO_SMALL
    assert lib.dartree_build_serial(ctypes.byref(d), None, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                    n.value, s) == C.ERR_INVALID_ARGUMENT


def test_verify_tree_validates_on_host(lib):
    """dartree_verify_tree: dh outside 1..256, NULL or misaligned pointers
    are rejected before any launch."""
    d = dims()
    f = ctypes.c_void_p(0x10000)
    s = ctypes.c_void_p(None)
    call = lambda dh, mask=f, q=f: lib.dartree_verify_tree(ctypes.byref(d), f, f, f, f, mask, f, q, f, f, dh, f, f,
                                                           f, s)
    assert call(0) == C.ERR_UNSUPPORTED
    assert call(257) == C.ERR_UNSUPPORTED
    assert call(128, q=None) == C.ERR_INVALID_ARGUMENT
    assert "Q" in C.last_error()
    assert call(128, mask=ctypes.c_void_p(0x10004)) == C.ERR_INVALID_ARGUMENT
    assert "aligned" in C.last_error()



def test_struct_layouts_match_the_header(tmp_path):
    """Every struct of the header has, compiled by the host C compiler, the
    size and field offsets of its ctypes mirror in the binding."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    structs = {"dartree_dims": C.Dims, "dartree_head": C.Head, "dartree_supertree": C.Supertree,
               "dartree_round_info": C.RoundInfo}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "dartree.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)


def test_noalloc_round_rejects_sizes_beyond_its_scratch(lib):
    # 256 requests at K = 512: 64 MiB of slice lists, beyond the 32 MiB the
    # allocation-free round holds; rejected on the host before any device call
    d = dims(n_req=256, K=512, r=512, D=4096)
    st, need = ws_size(lib, d)
    assert st == C.OK and need > C.NOALLOC_SCRATCH_BYTES
    head = C.Head(A=None, E=16, U=16, Pt=16)
    sup = C.Supertree(tok=16, parent_slot=16, cum=16, sbeta=16, count=16, state=16, next_depth=1)
    p = ctypes.c_void_p(16)
    s = lib.dartree_build_round_noalloc(ctypes.byref(d), ctypes.byref(head), p, p, p, p, p, ctypes.byref(sup),
                                        p, p, p, p, p, p, p, None)
    assert s == C.ERR_UNSUPPORTED
    assert "allocation-free" in C.last_error()
    # the metric config's scratch fits
    st, need = ws_size(lib, dims())
    assert st == C.OK and need <= C.NOALLOC_SCRATCH_BYTES
    # invalid dims are reported like dartree_build_round reports them
    s = lib.dartree_build_round_noalloc(ctypes.byref(dims(beta=0.5)), ctypes.byref(head), p, p, p, p, p,
                                        ctypes.byref(sup), p, p, p, p, p, p, p, None)
    assert s == C.ERR_INVALID_ARGUMENT


def test_unknown_head_flags_are_rejected_before_any_device_call(lib):
    d = dims()
    head = C.Head(A=16, E=16, U=16, Pt=16, flags=4)
    flags = ctypes.c_void_p(16)
    assert lib.dartree_head_check(ctypes.byref(d), ctypes.byref(head), flags, None) == C.ERR_INVALID_ARGUMENT
    assert "flags" in C.last_error()


def test_split_wait_bounds(lib):
    assert lib.dartree_set_split_wait(-1) == C.ERR_INVALID_ARGUMENT
    assert lib.dartree_set_split_wait(1000001) == C.ERR_INVALID_ARGUMENT
    assert lib.dartree_set_split_wait(0) == C.OK
    assert lib.dartree_set_split_wait(200) == C.OK


def test_general_kernel_parts_and_exchange_space(lib):
    """bf16 weights outside the block-decoding shapes: up to 4 workgroups a
    request while n_req * parts <= 256, with room in the workspace for the
    exchanged slices [n][L][W][K + r] fp32 and the flags [n][parts][L]."""
    def plan(**kw):
        info = C.RoundInfo()
        assert lib.dartree_round_plan(ctypes.byref(dims(**kw)), ctypes.byref(info)) == C.OK
        return info
    stress = dict(n_req=64, K=512, W=12, B=64, r=512, D=4096)
    assert plan(**stress).tree_parts == 4
    assert plan(**dict(stress, n_req=100)).tree_parts == 2
    assert plan(**dict(stress, n_req=200)).tree_parts == 1
    assert plan(**dict(stress, weight_dtype=C.F32)).tree_parts == 1
    assert plan().tree_parts == 1            # block-decoding shape
    st, n = ws_size(lib, dims(**stress))
    assert st == C.OK
    lists = 64 * 16 * 4 * 512 * 8    # 1024 rows x 4 slices x K keys of 8 bytes
    xch = 64 * 16 * 12 * (512 + 512) * 4
    flags = 64 * 4 * 16 * 4
    assert lists + xch + flags <= n <= lists + xch + flags + 3 * 256
