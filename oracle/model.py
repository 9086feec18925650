"""Oracle: the verify forward of the pages' decoder-only model (fp64, CPU).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Follows [P2] section numpyで小さなTransformerを自作する: a GPT-2-type decoder
(pre-LayerNorm blocks, learned token and position embeddings, a GELU MLP);
the ``forward_cached`` listing there takes n new tokens, adds their token and
position embeddings (positions p0 .. p0+n-1, p0 = the cache length), and in
every layer normalises, projects to q, k, v with one fused matrix, writes the
n new K/V rows into the layer's cache at [p0, p0+n), attends causally (new
row i sees cache rows [0, p0+i]) with scores scaled by 1/sqrt(D), projects
the heads back, adds, normalises again and adds the MLP; a final
normalisation and the output matrix give the n rows of logits.  The same
section states that the uncached forward (the whole sequence every time)
gives the same logits, up to fp32 rounding.

The parameter set is fixed by the same section's counts: the 4-layer,
width-96, 4-head model over 96 characters with 512 positions has 513,600
parameters and the 1-layer, width-48, 2-head draft 61,968.  Both counts hold
exactly for: MLP width 4C; biases on the MLP only (none on the q/k/v, output
and vocabulary projections); LayerNorm gain and bias per norm.  The listing
calls ``ln_fwd`` and ``gelu`` without defining them; the readings here are
GPT-2's: LayerNorm over the last axis with the population variance and
eps = 1e-5, and GELU in its tanh form.

Parameters are one flat array in the order of ``param_shapes``:
  wte [V, C], wpe [T, C],
  per layer: ln1_g [C], ln1_b [C], wqkv [C, 3C], wo [C, C], ln2_g [C],
             ln2_b [C], w1 [C, F], b1 [F], w2 [F, C], b2 [C],
  lnf_g [C], lnf_b [C], wout [C, V].
wqkv's columns are q, then k, then v, each head-major (head h owns columns
[h D, (h+1) D) of its third).  Caches are [L][2][B][H][max_T][D] (layer,
k/v, sequence, head, position, dimension).
"""

from dataclasses import dataclass

import numpy as np

LN_EPS = 1e-5


@dataclass(frozen=True)
class ModelConfig:
    V: int  # vocabulary
    C: int  # width
    L: int  # layers
    H: int  # heads
    T: int  # positions (rows of wpe)

    @property
    def F(self):
        return 4 * self.C

    @property
    def D(self):
        return self.C // self.H


# The two models of [P2] section 実験の作り方 (the confirmation environment).
TARGET = ModelConfig(V=96, C=96, L=4, H=4, T=512)
DRAFT = ModelConfig(V=96, C=48, L=1, H=2, T=512)


def param_shapes(cfg):
    """Ordered (name, shape) list of the flat parameter array."""
    C, F, V, T = cfg.C, cfg.F, cfg.V, cfg.T
    out = [("wte", (V, C)), ("wpe", (T, C))]
    for l in range(cfg.L):
        out += [
            (f"{l}.ln1_g", (C,)), (f"{l}.ln1_b", (C,)),
            (f"{l}.wqkv", (C, 3 * C)), (f"{l}.wo", (C, C)),
            (f"{l}.ln2_g", (C,)), (f"{l}.ln2_b", (C,)),
            (f"{l}.w1", (C, F)), (f"{l}.b1", (F,)),
            (f"{l}.w2", (F, C)), (f"{l}.b2", (C,)),
        ]
    out += [("lnf_g", (C,)), ("lnf_b", (C,)), ("wout", (C, V))]
    return out


def param_count(cfg):
    return int(sum(int(np.prod(s)) for _, s in param_shapes(cfg)))


def unpack(flat, cfg):
    """Dict name -> fp64 array from the flat parameter array."""
    flat = np.asarray(flat, dtype=np.float64)
    assert flat.shape == (param_count(cfg),)
    P, off = {}, 0
    for name, shape in param_shapes(cfg):
        n = int(np.prod(shape))
        P[name] = flat[off : off + n].reshape(shape)
        off += n
    return P


def layer_norm(x, g, b):
    """(x - mean) / sqrt(var + eps) * g + b over the last axis (population var)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + LN_EPS) * g + b


def gelu(x):
    """GELU, tanh form: x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x**3)))


def softmax(s):
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _attend(q, K, V, p0):
    """q [H, n, D] against K, V [H, p0+n, D]; new row i sees keys [0, p0+i]."""
    H, n, D = q.shape
    out = np.zeros_like(q)
    for i in range(n):
        m = p0 + i + 1
        s = np.einsum("hd,hkd->hk", q[:, i], K[:, :m]) / np.sqrt(D)
        out[:, i] = np.einsum("hk,hkd->hd", softmax(s), V[:, :m])
    return out


def forward_cached(flat, cfg, tokens, kv, lens):
    """Logits [B, n, V] of the n new tokens of every sequence, and the caches.

    tokens [B, n] int, kv [L, 2, B, H, max_T, D] (any float; rows >= lens[b]
    are never read), lens [B] the cache length p0 of each sequence.  Returns
    (logits fp64, kv fp64 copy with rows [p0, p0+n) of every layer written).
    """
    P = unpack(flat, cfg)
    C, H, D = cfg.C, cfg.H, cfg.D
    tokens = np.asarray(tokens)
    B, n = tokens.shape
    kv = np.array(kv, dtype=np.float64, copy=True)
    logits = np.zeros((B, n, cfg.V))
    for b in range(B):
        p0 = int(lens[b])
        x = P["wte"][tokens[b]] + P["wpe"][p0 : p0 + n]
        for l in range(cfg.L):
            h = layer_norm(x, P[f"{l}.ln1_g"], P[f"{l}.ln1_b"])
            qkv = h @ P[f"{l}.wqkv"]
            q, k, v = (qkv[:, j * C : (j + 1) * C].reshape(n, H, D).transpose(1, 0, 2) for j in range(3))
            kv[l, 0, b, :, p0 : p0 + n] = k
            kv[l, 1, b, :, p0 : p0 + n] = v
            y = _attend(q, kv[l, 0, b, :, : p0 + n], kv[l, 1, b, :, : p0 + n], p0)
            x = x + y.transpose(1, 0, 2).reshape(n, C) @ P[f"{l}.wo"]
            h2 = layer_norm(x, P[f"{l}.ln2_g"], P[f"{l}.ln2_b"])
            x = x + gelu(h2 @ P[f"{l}.w1"] + P[f"{l}.b1"]) @ P[f"{l}.w2"] + P[f"{l}.b2"]
        logits[b] = layer_norm(x, P["lnf_g"], P["lnf_b"]) @ P["wout"]
    return logits, kv


def forward_uncached(flat, cfg, tokens):
    """Logits [T_b, V] of every position of one whole sequence, no cache.

    The full causal forward over tokens[0:T_b] ([P2] section
    numpyで小さなTransformerを自作する, the uncached version it compares
    against): every position attends to itself and all earlier positions.
    """
    P = unpack(flat, cfg)
    C, H, D = cfg.C, cfg.H, cfg.D
    tokens = np.asarray(tokens)
    n = tokens.shape[0]
    x = P["wte"][tokens] + P["wpe"][:n]
    for l in range(cfg.L):
        h = layer_norm(x, P[f"{l}.ln1_g"], P[f"{l}.ln1_b"])
        qkv = h @ P[f"{l}.wqkv"]
        q, k, v = (qkv[:, j * C : (j + 1) * C].reshape(n, H, D).transpose(1, 0, 2) for j in range(3))
        y = _attend(q, k, v, 0)
        x = x + y.transpose(1, 0, 2).reshape(n, C) @ P[f"{l}.wo"]
        h2 = layer_norm(x, P[f"{l}.ln2_g"], P[f"{l}.ln2_b"])
        x = x + gelu(h2 @ P[f"{l}.w1"] + P[f"{l}.b1"]) @ P[f"{l}.w2"] + P[f"{l}.b2"]
    return layer_norm(x, P["lnf_g"], P["lnf_b"]) @ P["wout"]


def empty_cache(cfg, B, max_T):
    return np.zeros((cfg.L, 2, B, cfg.H, max_T, cfg.D))


def prefill(flat, cfg, prefixes, max_T):
    """Caches holding the K/V of each sequence's prefix (one cached forward of
    the whole prefix from an empty cache), and the prefix lengths."""
    B = len(prefixes)
    kv = empty_cache(cfg, B, max_T)
    lens = np.array([len(p) for p in prefixes])
    for b, pre in enumerate(prefixes):
        if len(pre) == 0:
            continue
        one = np.zeros((cfg.L, 2, 1, cfg.H, max_T, cfg.D))
        _, one = forward_cached(flat, cfg, np.asarray(pre)[None, :], one, [0])
        kv[:, :, b] = one[:, :, 0]
    return kv, lens
