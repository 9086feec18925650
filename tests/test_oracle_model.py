"""Pins of the model oracle (oracle/model.py): the verify forward of the
pages' GPT-2-type decoder.

[P2] section numpyで小さなTransformerを自作する fixes what is pinned here: the
parameter counts of the two models, and that the cached forward equals the
uncached one.  LayerNorm and GELU (undefined on the page) are pinned to
PyTorch's routines with GPT-2's readings; the attention inside the model to
the attention oracle (itself pinned to PyTorch's scaled-dot-product
attention); the residual stream and the q/k/v layout to closed forms of
degenerate weights.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import model as M
from workloads import gen

HERE = os.path.dirname(os.path.abspath(__file__))


def _params(cfg, seed=0):
    return gen.model_params(M.param_shapes(cfg), seed).astype(np.float64)


def test_param_counts_match_the_pages():
    g = json.load(open(os.path.join(HERE, "golden", "p2_model_params.json")))
    for m in g["models"]:
        cfg = M.ModelConfig(m["V"], m["C"], m["L"], m["H"], m["T"])
        assert M.param_count(cfg) == m["params"], m["name"]


def test_layer_norm_matches_torch():
    r = np.random.default_rng(1)
    x = r.standard_normal((7, 96)) * 3 + 1
    g = 1 + 0.1 * r.standard_normal(96)
    b = 0.1 * r.standard_normal(96)
    want = torch.nn.functional.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), torch.from_numpy(b),
                                          eps=1e-5).numpy()
    np.testing.assert_allclose(M.layer_norm(x, g, b), want, rtol=0, atol=1e-12)


def test_gelu_matches_torch_tanh_form():
    x = np.linspace(-8, 8, 1001)
    want = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(M.gelu(x), want, rtol=0, atol=1e-14)


def test_model_attention_matches_attention_oracle():
    r = np.random.default_rng(2)
    H, n, D, p0 = 4, 5, 24, 9
    q = r.standard_normal((H, n, D))
    K = r.standard_normal((H, p0 + n, D))
    V = r.standard_normal((H, p0 + n, D))
    got = M._causal_attention(q, K, V, p0)
    kc = np.zeros((1, H, p0 + n, D))
    vc = np.zeros((1, H, p0 + n, D))
    kc[0, :, :p0] = K[:, :p0]
    vc[0, :, :p0] = V[:, :p0]
    want = A.verify_attention(q[None], K[None, :, p0:], V[None, :, p0:], kc, vc, [p0])[0]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("cfg", [M.TARGET, M.DRAFT], ids=["target", "draft"])
def test_cached_equals_uncached(cfg):
    """[P2]: the cached forward gives the uncached forward's logits."""
    flat = _params(cfg, 3)
    r = np.random.default_rng(4)
    seq = r.integers(0, cfg.V, size=23)
    kv, lens = M.prefill(flat, cfg, [seq[:18]], max_T=32)
    got, _ = M.forward_cached(flat, cfg, seq[None, 18:], kv, lens)
    want = M.forward_uncached(flat, cfg, seq)[18:]
    np.testing.assert_allclose(got[0], want, rtol=0, atol=1e-10)


def test_greedy_generation_same_tokens_cached_and_uncached():
    """[P2] checks that greedy generation gives the same characters either way."""
    cfg = M.TARGET
    flat = _params(cfg, 5)
    prompt = list(np.random.default_rng(6).integers(0, cfg.V, size=6))
    # cached: prefill all but the last prompt token, then one token per call
    kv, _ = M.prefill(flat, cfg, [prompt[:-1]], max_T=40)
    L, tok, cached = len(prompt) - 1, prompt[-1], []
    seq = list(prompt)
    for _ in range(12):
        lg, kv = M.forward_cached(flat, cfg, np.array([[tok]]), kv, [L])
        L += 1
        tok = int(np.argmax(lg[0, -1]))
        cached.append(tok)
    for _ in range(12):
        seq.append(int(np.argmax(M.forward_uncached(flat, cfg, np.array(seq))[-1])))
    assert cached == seq[len(prompt):]


def test_chunked_prefill_equals_one_shot():
    cfg = M.TARGET
    flat = _params(cfg, 7)
    seq = np.random.default_rng(8).integers(0, cfg.V, size=17)
    one, _ = M.prefill(flat, cfg, [seq], max_T=24)
    two, lens = M.prefill(flat, cfg, [seq[:10]], max_T=24)
    _, two = M.forward_cached(flat, cfg, seq[None, 10:], two, lens)
    np.testing.assert_allclose(two[:, :, :, :, :17], one[:, :, :, :, :17], rtol=0, atol=1e-12)


def test_uncached_is_causal():
    cfg = M.TARGET
    flat = _params(cfg, 9)
    seq = np.random.default_rng(10).integers(0, cfg.V, size=12)
    a = M.forward_uncached(flat, cfg, seq)
    seq2 = seq.copy()
    seq2[8] = (seq2[8] + 1) % cfg.V
    b = M.forward_uncached(flat, cfg, seq2)
    np.testing.assert_array_equal(a[:8], b[:8])
    assert np.abs(a[8:] - b[8:]).max() > 1e-6


def _zeroed(cfg, flat):
    """Parameters with every block's matrices zero (the stream passes through)."""
    P = {k: v.copy() for k, v in M.unpack(flat, cfg).items()}
    for l in range(cfg.L):
        for k in ("attn.in", "attn.out", "mlp.up", "mlp.down"):
            P[f"block{l}.{k}"][:] = 0.0
    return np.concatenate([P[name].ravel() for name, _ in M.param_shapes(cfg)]), P


def _ln(x, g, b, eps=1e-5):
    return (x - x.mean()) / np.sqrt(x.var() + eps) * g + b


def test_residual_stream_closed_form():
    """With zero block matrices each block adds only its MLP down bias: the
    logits of token t at position p are LNf(E_tok[t] + E_pos[p] + sum_l
    down_bias_l) W_unembed."""
    cfg = M.TARGET
    flat, P = _zeroed(cfg, _params(cfg, 11))
    tok, p = 17, 5
    kv = np.zeros((cfg.L, 2, 1, cfg.H, 8, cfg.D))
    got, _ = M.forward_cached(flat, cfg, np.array([[tok]]), kv, [p])
    x = P["token_embedding"][tok] + P["position_embedding"][p] + sum(P[f"block{l}.mlp.down_bias"] for l in range(cfg.L))
    want = _ln(x, P["final_norm.gain"], P["final_norm.bias"]) @ P["unembedding"]
    np.testing.assert_allclose(got[0, 0], want, rtol=0, atol=1e-12)


def test_value_path_and_head_layout_closed_form():
    """One layer, first token (p0 = 0, one key): attention returns v exactly,
    so x = e + v W_out with v = LN1(e) W_in[:, 2C:3C] -- and the cache rows
    hold k and v split by head as [h, d] = column h D + d of their thirds."""
    cfg = M.ModelConfig(V=11, C=8, L=1, H=2, T=4)
    flat = gen.model_params(M.param_shapes(cfg), 12).astype(np.float64)
    P = M.unpack(flat, cfg)
    kv = np.zeros((1, 2, 1, 2, 4, 4))
    got_logits, got_kv = M.forward_cached(flat, cfg, np.array([[3]]), kv, [0])
    e = P["token_embedding"][3] + P["position_embedding"][0]
    h = _ln(e, P["block0.norm1.gain"], P["block0.norm1.bias"])
    k, v = h @ P["block0.attn.in"][:, 8:16], h @ P["block0.attn.in"][:, 16:24]
    np.testing.assert_allclose(got_kv[0, 0, 0, :, 0], k.reshape(2, 4), rtol=0, atol=1e-12)
    np.testing.assert_allclose(got_kv[0, 1, 0, :, 0], v.reshape(2, 4), rtol=0, atol=1e-12)
    x = e + v @ P["block0.attn.out"]
    u = M.gelu(_ln(x, P["block0.norm2.gain"], P["block0.norm2.bias"]) @ P["block0.mlp.up"] + P["block0.mlp.up_bias"])
    x = x + u @ P["block0.mlp.down"] + P["block0.mlp.down_bias"]
    want = _ln(x, P["final_norm.gain"], P["final_norm.bias"]) @ P["unembedding"]
    np.testing.assert_allclose(got_logits[0, 0], want, rtol=0, atol=1e-12)
