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

Parameters are one flat array in the order of ``param_shapes`` (the packing
is a convention of this oracle, which the library defines again on its own):
  token embedding [V, C], position embedding [T, C],
  per block: norm1 gain [C], bias [C]; attention in [C, 3C]; attention
             out [C, C]; norm2 gain [C], bias [C]; MLP up [C, F], up bias
             [F]; MLP down [F, C], down bias [C],
  final norm gain [C], bias [C], unembedding [C, V].
The attention-in matrix's columns are q, then k, then v, each head-major
(head h owns columns [h D, (h+1) D) of its third).  Caches are
[L][2][B][H][max_T][D] (layer, k/v, sequence, head, position, dimension).

Structure: the parameters are unpacked into a ``Model`` of ``Block``s; one
function, ``_block``, is a whole residual block given how attention sees the
keys, and the cached and uncached forwards differ only in that: the cached one
writes the block's new key/value rows into the cache and attends over the
cache's first p0 + n rows, the uncached one over the sequence's own rows.
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
    T: int  # positions (rows of the position embedding)

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
    out = [("token_embedding", (V, C)), ("position_embedding", (T, C))]
    for l in range(cfg.L):
        out += [
            (f"block{l}.norm1.gain", (C,)), (f"block{l}.norm1.bias", (C,)),
            (f"block{l}.attn.in", (C, 3 * C)), (f"block{l}.attn.out", (C, C)),
            (f"block{l}.norm2.gain", (C,)), (f"block{l}.norm2.bias", (C,)),
            (f"block{l}.mlp.up", (C, F)), (f"block{l}.mlp.up_bias", (F,)),
            (f"block{l}.mlp.down", (F, C)), (f"block{l}.mlp.down_bias", (C,)),
        ]
    out += [("final_norm.gain", (C,)), ("final_norm.bias", (C,)), ("unembedding", (C, V))]
    return out


def param_count(cfg):
    return int(sum(int(np.prod(s)) for _, s in param_shapes(cfg)))


def unpack(flat, cfg):
    """Dict name -> fp64 array from the flat parameter array."""
    flat = np.asarray(flat, dtype=np.float64)
    assert flat.shape == (param_count(cfg),)
    named, off = {}, 0
    for name, shape in param_shapes(cfg):
        n = int(np.prod(shape))
        named[name] = flat[off : off + n].reshape(shape)
        off += n
    return named


@dataclass
class Norm:
    gain: np.ndarray
    bias: np.ndarray

    def __call__(self, x):
        return layer_norm(x, self.gain, self.bias)


@dataclass
class Block:
    norm1: Norm
    attn_in: np.ndarray    # [C, 3C]: q | k | v, each head-major
    attn_out: np.ndarray   # [C, C]
    norm2: Norm
    up: np.ndarray         # [C, F]
    up_bias: np.ndarray    # [F]
    down: np.ndarray       # [F, C]
    down_bias: np.ndarray  # [C]


@dataclass
class Model:
    cfg: ModelConfig
    token_embedding: np.ndarray     # [V, C]
    position_embedding: np.ndarray  # [T, C]
    blocks: list
    final_norm: Norm
    unembedding: np.ndarray         # [C, V]

    def embed(self, tokens, first_position):
        """Token plus position embedding of tokens at first_position, +1, ..."""
        pos = np.arange(first_position, first_position + len(tokens))
        return self.token_embedding[np.asarray(tokens)] + self.position_embedding[pos]

    def logits(self, x):
        return self.final_norm(x) @ self.unembedding


def model_from_flat(flat, cfg):
    """The flat parameter array as a ``Model``."""
    named = unpack(flat, cfg)
    blocks = []
    for l in range(cfg.L):
        g = lambda k: named[f"block{l}.{k}"]  # noqa: E731
        blocks.append(Block(Norm(g("norm1.gain"), g("norm1.bias")), g("attn.in"), g("attn.out"),
                            Norm(g("norm2.gain"), g("norm2.bias")), g("mlp.up"), g("mlp.up_bias"),
                            g("mlp.down"), g("mlp.down_bias")))
    return Model(cfg, named["token_embedding"], named["position_embedding"], blocks,
                 Norm(named["final_norm.gain"], named["final_norm.bias"]), named["unembedding"])


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


def _heads(m, H):
    """[n, C] -> [H, n, D]: head h takes columns [h D, (h+1) D)."""
    n, C = m.shape
    return m.reshape(n, H, C // H).transpose(1, 0, 2)


def _unheads(a):
    """[H, n, D] -> [n, H D]."""
    H, n, D = a.shape
    return a.transpose(1, 0, 2).reshape(n, H * D)


def _causal_attention(q, keys, values, first):
    """q [H, n, D] against keys/values [H, first + n, D]: the query of new
    position first + i sees keys [0, first + i], scores scaled by 1/sqrt(D)."""
    H, n, D = q.shape
    out = np.empty_like(q)
    for i in range(n):
        visible = first + i + 1
        s = np.einsum("hd,hkd->hk", q[:, i], keys[:, :visible]) / np.sqrt(D)
        out[:, i] = np.einsum("hk,hkd->hd", softmax(s), values[:, :visible])
    return out


def _block(blk, x, H, keys_values):
    """One pre-norm residual block on the rows x [n, C].

    ``keys_values(k, v)`` receives the rows' own key and value heads [H, n, D]
    and returns the keys, values and first position the rows attend over.
    """
    C = x.shape[1]
    proj = blk.norm1(x) @ blk.attn_in
    q, k, v = (_heads(proj[:, j * C : (j + 1) * C], H) for j in range(3))
    keys, values, first = keys_values(k, v)
    x = x + _unheads(_causal_attention(q, keys, values, first)) @ blk.attn_out
    hidden = gelu(blk.norm2(x) @ blk.up + blk.up_bias)
    return x + hidden @ blk.down + blk.down_bias


def forward_cached(flat, cfg, tokens, kv, lens):
    """Logits [B, n, V] of the n new tokens of every sequence, and the caches.

    tokens [B, n] int, kv [L, 2, B, H, max_T, D] (any float; rows >= lens[b]
    are never read), lens [B] the cache length p0 of each sequence.  Returns
    (logits fp64, kv fp64 copy with rows [p0, p0+n) of every layer written).
    """
    model = model_from_flat(flat, cfg)
    tokens = np.asarray(tokens)
    B, n = tokens.shape
    kv = np.array(kv, dtype=np.float64, copy=True)
    logits = np.zeros((B, n, cfg.V))
    for b in range(B):
        p0 = int(lens[b])

        def through_cache(k, v, layer):
            kv[layer, 0, b, :, p0 : p0 + n] = k
            kv[layer, 1, b, :, p0 : p0 + n] = v
            return kv[layer, 0, b, :, : p0 + n], kv[layer, 1, b, :, : p0 + n], p0

        x = model.embed(tokens[b], p0)
        for layer, blk in enumerate(model.blocks):
            x = _block(blk, x, cfg.H, lambda k, v: through_cache(k, v, layer))
        logits[b] = model.logits(x)
    return logits, kv


def forward_uncached(flat, cfg, tokens):
    """Logits [T_b, V] of every position of one whole sequence, no cache.

    The full causal forward over tokens[0:T_b] ([P2] section
    numpyで小さなTransformerを自作する, the uncached version it compares
    against): every position attends to itself and all earlier positions.
    """
    model = model_from_flat(flat, cfg)
    x = model.embed(np.asarray(tokens), 0)
    for blk in model.blocks:
        x = _block(blk, x, cfg.H, lambda k, v: (k, v, 0))
    return model.logits(x)


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
