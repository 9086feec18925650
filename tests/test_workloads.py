"""Host checks of the synthetic input generators (no method arithmetic here)."""

import numpy as np
import torch

import workloads as W
from workloads import gen as G


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate(
        [rng.normal(scale=3.0, size=100_000), [0.0, -0.0, 1.0, 1.00390625, 1.0078125, 1.01171875, 65504.0, 1e-40]]
    ).astype(np.float32)
    ours = G.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_generators_are_deterministic_and_shaped():
    for cid in (1, 2, 3):
        cfg = W.get(cid)
        B = min(cfg.B, 16)
        a = W.sampler_inputs(cfg, B=B)
        b = W.sampler_inputs(cfg, B=B)
        for k in ("target_logits", "draft_logits", "draft_tokens", "uniforms"):
            assert np.array_equal(a[k], b[k])
        assert a["target_logits"].shape == (B, cfg.gamma + 1, cfg.V)
        assert a["draft_logits"].shape == (B, cfg.gamma, cfg.V)
        assert a["draft_tokens"].dtype == np.int32 and a["draft_tokens"].max() < cfg.V
        assert a["uniforms"].min() >= 0 and a["uniforms"].max() < 1
    cfg = W.get(3)
    att = W.attention_inputs(cfg, B=4)
    assert att["k_cache"].shape == (4, cfg.Hkv, cfg.max_T, cfg.D)
    assert np.all(att["lens"] == 384)


def test_bf16_config_shapes_small():
    cfg = W.get(4)
    s = W.sampler_inputs(cfg, B=2)
    assert s["target_logits"].dtype == np.uint16 and s["target_logits"].shape == (2, 5, cfg.V)
    att = W.attention_inputs(cfg, B=2)
    assert att["q"].dtype == np.uint16
    assert 1024 <= att["lens"].min() and att["lens"].max() <= 4096
    assert att["lens"].max() + cfg.n_q <= cfg.max_T


def test_gumbel_drafts_follow_softmax_of_draft_logits():
    # The draft sampler must draw from softmax(z_d / T); chi-square at 4 sigma.
    rng = np.random.default_rng(9)
    V, N, T = 6, 200_000, 0.7
    z = rng.normal(size=V)
    x = G._gumbel_argmax(np.broadcast_to(z / T, (N, V)), rng.random((N, V)))
    e = np.exp(z / T - (z / T).max())
    p = e / e.sum()
    cnt = np.bincount(x, minlength=V)
    chi2 = np.sum((cnt - N * p) ** 2 / (N * p))
    assert chi2 < V - 1 + 4 * np.sqrt(2 * (V - 1))


def test_repeated_row_inputs_repeat_one_pair():
    a = W.repeated_row_inputs(5, 65, 3, 1000, 0.7, chunk=300)
    b = W.repeated_row_inputs(5, 65, 3, 1000, 0.7)
    for k in ("target_logits", "draft_logits", "draft_tokens", "uniforms"):
        assert np.array_equal(a[k], b[k])  # chunking does not change the draws
    assert a["target_logits"].shape == (1000, 4, 65) and a["draft_logits"].shape == (1000, 3, 65)
    assert np.all(a["target_logits"] == a["target_row"]) and np.all(a["draft_logits"] == a["draft_row"])
    assert a["draft_tokens"].dtype == np.int32 and 0 <= a["draft_tokens"].min() and a["draft_tokens"].max() < 65
    assert a["uniforms"].min() >= 0 and a["uniforms"].max() < 1
