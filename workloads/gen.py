"""Seeded generators for the synthetic workloads.

Host generators (numpy, ``default_rng([config, stream, rep])``) serve configs
1-4 and any reduced-size case; they are deterministic and device independent.
Stream 0 draws logits and Q/K/V, stream 1 the draft-sampling noise, stream 2
the verify uniforms, stream 3 the cache lengths.

Device generators (torch, a seeded generator on the GPU) serve config 5, whose
KV cache (about 34 GB) cannot be drawn on the host in reasonable time.  Its
lengths still come from the host stream 3, so they match the host recipe.

bfloat16 tensors are carried as uint16 bit patterns on the host and as
``torch.bfloat16`` on the device.  fp32 -> bf16 is round-to-nearest-even on
both (torch's conversion is RNE).
"""

import numpy as np

from .configs import Config


def rng(cfg: Config, stream: int, rep: int = 0):
    return np.random.default_rng([cfg.cid, stream, rep])


def bf16_bits(x):
    """Round an fp32 array to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x32, dtype):
    if dtype == "bf16":
        return bf16_bits(x32)
    if dtype == "f16":  # IEEE half, rounded to nearest even
        return np.ascontiguousarray(x32, dtype=np.float16)
    return np.ascontiguousarray(x32, dtype=np.float32)


def _as_f32(stored, dtype):
    if dtype == "bf16":
        return bf16_bits_to_f32(stored)
    return np.asarray(stored, dtype=np.float32)


def _gumbel_argmax(z_over_t, noise_uniform):
    """Index of max(z/T + Gumbel), i.e. one draw from softmax(z/T) per row."""
    with np.errstate(divide="ignore"):
        g = -np.log(-np.log(noise_uniform))
    return np.argmax(z_over_t + g, axis=-1).astype(np.int32)


def sampler_inputs(cfg: Config, temperature=None, rep: int = 0, B=None):
    """Host arrays for the rejection sampler.

    Returns target_logits [B, gamma+1, V], draft_logits [B, gamma, V] (fp32, or
    uint16 bf16 bits), draft_tokens int32 [B, gamma] drawn from
    softmax(draft/T), uniforms fp64 [B, gamma+1] in [0, 1), and temperature.
    """
    T = cfg.temperatures[0] if temperature is None else float(temperature)
    B = cfg.B if B is None else int(B)
    g, V = cfg.gamma, cfg.V
    r0 = rng(cfg, 0, rep)
    if cfg.p is not None:
        # Toy: every target row is ln p, the draft row is ln q.
        zt = np.broadcast_to(np.log(np.array(cfg.p, np.float64)).astype(np.float32), (B, g + 1, V))
        zd = np.broadcast_to(np.log(np.array(cfg.q, np.float64)).astype(np.float32), (B, g, V))
        zt = np.ascontiguousarray(zt)
        zd = np.ascontiguousarray(zd)
    else:
        zt = (cfg.t_std * r0.standard_normal((B, g + 1, V), dtype=np.float32)).astype(np.float32)
        zd = (cfg.mix * zt[:, :g] + cfg.noise_std * r0.standard_normal((B, g, V), dtype=np.float32)).astype(
            np.float32
        )
    zt_s = _store(zt, cfg.dtype)
    zd_s = _store(zd, cfg.dtype)
    # Drafts come from the distribution the verifier will see: the stored values.
    zd_seen = _as_f32(zd_s, cfg.dtype).astype(np.float64) / T
    noise = rng(cfg, 1, rep).random((B, g, V))
    x = _gumbel_argmax(zd_seen, noise)
    u = rng(cfg, 2, rep).random((B, g + 1))
    return {
        "target_logits": zt_s,
        "draft_logits": zd_s,
        "draft_tokens": np.ascontiguousarray(x, dtype=np.int32),
        "uniforms": np.ascontiguousarray(u, dtype=np.float64),
        "temperature": T,
    }


def repeated_row_inputs(seed: int, V: int, gamma: int, N: int, temperature: float = 1.0, t_std: float = 2.5,
                        noise_std: float = 0.45, chunk: int = 8192):
    """N sequences that all verify one fixed (target row, draft row) pair.

    Every target position holds the same fp32 logit row z_t ~ t_std * N(0, 1)
    over V tokens, every draft position the row z_d = z_t + noise_std * N(0, 1)
    (for V = 65 and the defaults the two distributions overlap by 0.78 to
    0.97 depending on the seed, around the 0.86 to 0.90 acceptance of the
    character models the pages measure).
    Each sequence draws its own draft tokens from softmax(z_d / T) and its own
    uniforms, so the N results are independent draws of one verification.
    Streams: ``default_rng([seed, 0])`` the rows, ``[seed, 1]`` the
    draft-sampling noise (drawn chunk by chunk), ``[seed, 2]`` the uniforms.
    """
    T = float(temperature)
    r0 = np.random.default_rng([seed, 0])
    zt_row = (t_std * r0.standard_normal(V)).astype(np.float32)
    zd_row = (zt_row + noise_std * r0.standard_normal(V)).astype(np.float32)
    zt = np.ascontiguousarray(np.broadcast_to(zt_row, (N, gamma + 1, V)))
    zd = np.ascontiguousarray(np.broadcast_to(zd_row, (N, gamma, V)))
    r1 = np.random.default_rng([seed, 1])
    x = np.empty((N, gamma), np.int32)
    zs = zd_row.astype(np.float64) / T
    for s in range(0, N, chunk):
        e = min(N, s + chunk)
        x[s:e] = _gumbel_argmax(zs, r1.random((e - s, gamma, V)))
    u = np.random.default_rng([seed, 2]).random((N, gamma + 1))
    return {
        "target_logits": zt,
        "draft_logits": zd,
        "draft_tokens": x,
        "uniforms": np.ascontiguousarray(u, dtype=np.float64),
        "temperature": T,
        "target_row": zt_row,
        "draft_row": zd_row,
    }


def lengths(cfg: Config, rep: int = 0, B=None):
    B = cfg.B if B is None else int(B)
    lo, hi = cfg.L
    return rng(cfg, 3, rep).integers(lo, hi + 1, size=B).astype(np.int32)


def attention_inputs(cfg: Config, rep: int = 0, B=None, max_T=None, lens=None):
    """Host arrays for verify attention (configs 3-5 shapes, or reduced B).

    q [B, Hq, n_q, D], k_new / v_new [B, Hkv, n_q, D], k_cache / v_cache
    [B, Hkv, max_T, D] -- every row filled with N(0,1), including rows past the
    committed length, which the verifier must never read -- and lens int32 [B].
    """
    B = cfg.B if B is None else int(B)
    max_T = cfg.max_T if max_T is None else int(max_T)
    r0 = rng(cfg, 0, rep)
    n, D = cfg.n_q, cfg.D

    def draw(*shape):
        return _store(r0.standard_normal(shape, dtype=np.float32), cfg.dtype)

    out = {
        "q": draw(B, cfg.Hq, n, D),
        "k_new": draw(B, cfg.Hkv, n, D),
        "v_new": draw(B, cfg.Hkv, n, D),
        "k_cache": draw(B, cfg.Hkv, max_T, D),
        "v_cache": draw(B, cfg.Hkv, max_T, D),
        "lens": lengths(cfg, rep, B) if lens is None else np.asarray(lens, np.int32),
    }
    assert int(out["lens"].max()) + n <= max_T and int(out["lens"].min()) >= 0
    return out


# ----------------------------------------------------------------------------
# device generators (torch); used for config 5 and for the benchmark
# ----------------------------------------------------------------------------


def _torch_gen(cfg: Config, stream: int, rep: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * cfg.cid + 10_007 * stream + rep)
    return g


def attention_inputs_device(cfg: Config, device, rep: int = 0, B=None):
    """Device tensors for verify attention; lens from the host stream 3."""
    import torch

    B = cfg.B if B is None else int(B)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(cfg.dtype, torch.float32)
    g = _torch_gen(cfg, 0, rep, device)
    n, D = cfg.n_q, cfg.D

    def draw(*shape):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dt)

    k_cache = torch.empty((B, cfg.Hkv, cfg.max_T, D), device=device, dtype=dt)
    v_cache = torch.empty_like(k_cache)
    for b in range(B):  # slab by sequence to bound the fp32 temporary
        k_cache[b] = draw(cfg.Hkv, cfg.max_T, D)
        v_cache[b] = draw(cfg.Hkv, cfg.max_T, D)
    lens = torch.from_numpy(lengths(cfg, rep, B)).to(device)
    return {
        "q": draw(B, cfg.Hq, n, D),
        "k_new": draw(B, cfg.Hkv, n, D),
        "v_new": draw(B, cfg.Hkv, n, D),
        "k_cache": k_cache,
        "v_cache": v_cache,
        "lens": lens,
    }


def sampler_inputs_device(cfg: Config, device, temperature=None, rep: int = 0, B=None):
    """Device tensors for the rejection sampler (same recipe as the host one)."""
    import torch

    T = cfg.temperatures[0] if temperature is None else float(temperature)
    B = cfg.B if B is None else int(B)
    gm, V = cfg.gamma, cfg.V
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(cfg.dtype, torch.float32)
    g0 = _torch_gen(cfg, 0, rep, device)
    g1 = _torch_gen(cfg, 1, rep, device)
    g2 = _torch_gen(cfg, 2, rep, device)
    zt = torch.empty((B, gm + 1, V), device=device, dtype=dt)
    zd = torch.empty((B, gm, V), device=device, dtype=dt)
    x = torch.empty((B, gm), device=device, dtype=torch.int32)
    for b in range(B):
        t32 = cfg.t_std * torch.randn((gm + 1, V), generator=g0, device=device)
        d32 = cfg.mix * t32[:gm] + cfg.noise_std * torch.randn((gm, V), generator=g0, device=device)
        zt[b] = t32.to(dt)
        zd[b] = d32.to(dt)
        u = torch.rand((gm, V), generator=g1, device=device, dtype=torch.float64)
        gum = -torch.log(-torch.log(u))
        x[b] = torch.argmax(zd[b].double() / T + gum, dim=-1).to(torch.int32)
    uni = torch.rand((B, gm + 1), generator=g2, device=device, dtype=torch.float64)
    return {
        "target_logits": zt,
        "draft_logits": zd,
        "draft_tokens": x,
        "uniforms": uni,
        "temperature": T,
    }


def attention_inputs_int8(cfg: Config, rep: int = 0, B=None, max_T=None, lens=None):
    """Host arrays for verify attention over an int8 cache.

    q, k_new, v_new as ``attention_inputs`` (bf16 bits); k_cache / v_cache int8
    [B, Hkv, max_T, D] and k_scale / v_scale float16 [B, Hkv, max_T], drawn so
    that code * scale looks like the N(0, 1) rows of the other workloads: codes
    are N(0, 1) * 127 / 2.7 rounded and clipped to [-127, 127], with one code
    of magnitude 127 per row (the row's largest value), and scales 2.7 / 127
    times a log-normal factor of spread 0.1.
    """
    base = attention_inputs(cfg, rep=rep, B=B, max_T=max_T, lens=lens)
    B, Hkv, T, D = base["k_cache"].shape
    r = rng(cfg, 4, rep)
    out = {k: base[k] for k in ("q", "k_new", "v_new", "lens")}
    for name in ("k", "v"):
        codes = np.clip(np.rint(r.standard_normal((B, Hkv, T, D)) * (127 / 2.7)), -127, 127).astype(np.int8)
        pos = r.integers(0, D, (B, Hkv, T))
        sign = np.where(r.random((B, Hkv, T)) < 0.5, -127, 127).astype(np.int8)
        np.put_along_axis(codes, pos[..., None], sign[..., None], axis=-1)
        out[f"{name}_cache"] = codes
        out[f"{name}_scale"] = (np.exp(0.1 * r.standard_normal((B, Hkv, T))) * (2.7 / 127)).astype(np.float16)
    return out


def attention_inputs_int8_device(cfg: Config, device, rep: int = 0, B=None):
    """Device tensors for verify attention over an int8 cache, with the recipe
    of ``attention_inputs_int8``: q, k_new, v_new N(0, 1) in the workload's
    16-bit type, lens from the host stream 3, int8 codes of N(0, 1) rows with
    one code of magnitude 127 per row, fp16 scales 2.7 / 127 times a
    log-normal factor of spread 0.1.  Drawn sequence by sequence from a seeded
    device stream (4) so no full-size 16-bit cache is ever formed."""
    import torch

    B = cfg.B if B is None else int(B)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(cfg.dtype, torch.float32)
    g = _torch_gen(cfg, 4, rep, device)
    n, D, T, Hkv = cfg.n_q, cfg.D, cfg.max_T, cfg.Hkv

    def draw(*shape):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dt)

    out = {"q": draw(B, cfg.Hq, n, D), "k_new": draw(B, Hkv, n, D), "v_new": draw(B, Hkv, n, D),
           "lens": torch.from_numpy(lengths(cfg, rep, B)).to(device)}
    for name in ("k", "v"):
        codes = torch.empty((B, Hkv, T, D), dtype=torch.int8, device=device)
        for b in range(B):
            c = torch.clamp(torch.round(torch.randn((Hkv, T, D), generator=g, device=device) * (127 / 2.7)), -127, 127)
            pos = torch.randint(0, D, (Hkv, T, 1), generator=g, device=device)
            sign = torch.where(torch.rand((Hkv, T, 1), generator=g, device=device) < 0.5, -127.0, 127.0)
            codes[b] = c.scatter(2, pos, sign).to(torch.int8)
        out[f"{name}_cache"] = codes
        out[f"{name}_scale"] = (torch.exp(0.1 * torch.randn((B, Hkv, T), generator=g, device=device))
                                * (2.7 / 127)).to(torch.float16)
    return out


# ---------------------------------------------------------------------------
# the verify forward of a decoder model (random weights)
# ---------------------------------------------------------------------------


def model_params(shapes, seed: int):
    """Random fp32 weights for a packed parameter layout.

    ``shapes`` is the ordered (name, shape) list of the layout.  Matrices are
    N(0, 1/rows); LayerNorm gains (names ending in ``gain``) 1 + N(0, 0.1^2);
    every other vector N(0, 0.1^2).  Stream 5 of ``default_rng([seed, 5])``.
    """
    r = np.random.default_rng([int(seed), 5])
    parts = []
    for name, shape in shapes:
        if len(shape) == 2:
            a = r.standard_normal(shape) / np.sqrt(shape[0])
        elif name.endswith("gain"):
            a = 1.0 + 0.1 * r.standard_normal(shape)
        else:
            a = 0.1 * r.standard_normal(shape)
        parts.append(a.astype(np.float32).ravel())
    return np.concatenate(parts)


def forward_inputs(V: int, L: int, H: int, D: int, B: int, n: int, lens_range, max_T: int, seed: int):
    """Tokens [B, n] uniform over the vocabulary, cache lengths [B] uniform in
    ``lens_range`` (inclusive), and an fp32 cache [L, 2, B, H, max_T, D] of
    N(0, 1) entries (stream 6 of ``default_rng([seed, 6])``)."""
    r = np.random.default_rng([int(seed), 6])
    tokens = r.integers(0, V, size=(B, n)).astype(np.int32)
    lens = r.integers(lens_range[0], lens_range[1] + 1, size=B).astype(np.int32)
    kv = r.standard_normal((L, 2, B, H, max_T, D)).astype(np.float32)
    return {"tokens": tokens, "lens": lens, "kv": kv}
