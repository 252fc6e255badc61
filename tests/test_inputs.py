"""The seeded input generator: determinism, layouts and distributions."""
import numpy as np
import pytest

from diffusion_drafter_tree_amd import inputs as I


def test_bf16_round_trip_and_rne():
    x = np.array([1.0, -2.5, 3.140625, 1.0 + 2**-8, 1.0 + 3 * 2**-9, 0.0, -0.0], np.float32)
    b = I.f32_to_bf16_bits(x)
    back = I.bf16_bits_to_f32(b)
    assert back[0] == 1.0 and back[1] == -2.5 and back[2] == 3.140625
    assert back[3] == 1.0            # halfway rounds to even
    assert back[4] == 1.0 + 2**-7    # above halfway rounds up
    assert b[6] == 0x8000


def test_round_determinism_and_distinct_streams():
    cfg = I.CONFIGS["tiny"]
    a, b = I.make_round(cfg, 0, 3), I.make_round(cfg, 0, 3)
    c = I.make_round(cfg, 0, 4)
    assert np.array_equal(a.logits, b.logits) and np.array_equal(a.h, b.h)
    assert not np.array_equal(a.logits, c.logits)
    ha, hb = I.make_head(cfg, 0), I.make_head(cfg, 0)
    assert np.array_equal(ha.E, hb.E)


@pytest.mark.parametrize("name", ["tiny", "concurrent_c4"])
def test_shapes_and_boost(name):
    cfg = I.CONFIGS[name]
    if name != "tiny":
        cfg = cfg.with_(V=4096, r=32, D=64)
    rnd = I.make_round(cfg, 1, 0)
    assert rnd.logits.shape == (cfg.n_req, cfg.L, cfg.V)
    assert rnd.logits.dtype == (np.uint16 if cfg.logits_dtype == "bf16" else np.float32)
    ids = rnd.boost_ids
    for q in range(cfg.n_req):
        for i in range(cfg.L):
            assert len(set(ids[q, i].tolist())) == cfg.n_boost
    x = I.as_f64(rnd.logits, cfg.logits_dtype)
    mask = np.ones_like(x, bool)
    for q in range(cfg.n_req):
        for i in range(cfg.L):
            mask[q, i, ids[q, i]] = False
    noise = x[mask]
    assert abs(noise.std() - cfg.sigma) < 0.05 * cfg.sigma
    assert abs(noise.mean()) < 0.05
    # boosted ids sit above the noise on average, less so deeper in the block
    gain = [float(np.mean(x[0, i, ids[0, i]])) for i in range(cfg.L)]
    assert gain[0] > gain[-1]


def test_head_scales():
    cfg = I.CONFIGS["tiny"].with_(r=64, V=2048)
    hd = I.make_head(cfg, 0)
    assert abs(hd.A.std() - 1 / 8) < 0.01
    assert abs(hd.E.std() - 1.0) < 0.02
    assert abs(hd.U.std() - 1 / 8) < 0.005
    cfg2 = I.CONFIGS["qwen3_4b"].with_(V=512, D=256, r=32)
    hd2 = I.make_head(cfg2, 0)
    assert hd2.Pt.shape == (32, 256) and hd2.Pt.dtype == np.uint16
    assert abs(I.as_f64(hd2.Pt, "bf16").std() - 1 / 16) < 0.005
