"""The allocation-free round (dartree_build_round_noalloc) against the round
with a caller workspace (dartree_build_round): bit-identical outputs, on
calls in a row whose inputs shrink, through the C ABI. At the 64-request
shape the workspace round spreads each request over four workgroups while the
allocation-free one keeps one (its scratch has no room for the exchange), so
that case also checks the two plans of the general kernel against each
other."""
import numpy as np
import pytest
import torch

from diffusion_drafter_tree_amd import inputs as I
from diffusion_drafter_tree_amd import ops

pytestmark = pytest.mark.gpu

SEQUENCE = [
    I.CONFIGS["stress_64req"],                                     # 64 requests, K = 512: 16 MiB of lists; its
                                                                   # split exchange (50 MiB) does not fit, so the
                                                                   # general kernel runs one workgroup a request
    I.CONFIGS["concurrent_c4"],                                    # 4 requests, K = 64: 256 KiB of scratch
    I.CONFIGS["qwen3_4b"],                                         # 1 request: smaller
    I.small_variant("qwen3_4b", name="general_lists", n_req=2, V=40000, L=4, K=64, W=12, B=30, r=128, D=256),
    I.CONFIGS["tiny"],                                             # fp32, one slice: smallest
]


def _outputs(cfg, fn, hd, rnd):
    rb = ops.RoundBuffers(cfg)
    fn(rb.dims, hd, ops.to_device(rnd.logits), ops.to_device(rnd.H if cfg.D > 0 else rnd.h), rb)
    torch.cuda.synchronize()
    return rb.numpy()


def test_noalloc_round_equals_workspace_round_on_shrinking_inputs():
    for i, cfg in enumerate(SEQUENCE):
        print(f"[no-alloc] call {i}: {cfg.name} n={cfg.n_req} V={cfg.V} K={cfg.K} "
              f"workspace={ops.workspace_size(ops.make_dims(cfg))} bytes", flush=True)
        hd = I.make_head(cfg, 0)
        dhd = ops.DeviceHead(hd)
        rnd = I.make_round(cfg, 0, 7)
        ref = _outputs(cfg, ops.build_round, dhd, rnd)
        got = _outputs(cfg, ops.build_round_noalloc, dhd, rnd)
        for k in ref:
            assert np.array_equal(got[k], ref[k]), (cfg.name, k)


def test_noalloc_round_twice_in_a_row_same_shape_new_round():
    cfg = I.CONFIGS["qwen3_4b"]
    hd = I.make_head(cfg, 0)
    dhd = ops.DeviceHead(hd)
    for t in (3, 4):
        rnd = I.make_round(cfg, 0, t)
        ref = _outputs(cfg, ops.build_round, dhd, rnd)
        got = _outputs(cfg, ops.build_round_noalloc, dhd, rnd)
        for k in ref:
            assert np.array_equal(got[k], ref[k]), (t, k)
