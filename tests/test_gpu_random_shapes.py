"""GPU parity at seeded random shapes, beside the hand-picked ones.

Valid shapes drawn once from fixed seeds, each case checked against the
oracle exactly as the fixed-shape tests check theirs:
  * verify attention over bf16, fp16 and fp32 caches: GQA/MQA/MHA groupings,
    1-16 verify rows, caches from empty to 6,000 keys, hints at and above
    the longest length, rows past each length poisoned with NaN;
  * long caches of up to 32K keys drawn on the device, whose shares are long
    enough that the launch merges each slab's pieces itself (sampled
    sequences checked);
  * the same attention over 16- and 32-position pages at random slots, and
    over the int8 cache;
  * the verify forward of random decoders (widths 32-144, head dimensions
    24-128, 1-4 layers, vocabularies 5-5,000);
  * whole speculative rounds of random target and draft decoders (gamma
    1-15, T 0-1.5);
  * the rejection sampler over fp32 and bf16 logits (V from 1 to 200,003,
    gamma 1-31, T 0.3-1.6, sharp to flat distributions), and large batches
    drawn on the device (sampled sequences checked);
  * greedy verification.
Every case prints its shape first.
"""

import numpy as np
import pytest
import torch

import speculative_decoding_verification_spec_amd as sv
import workloads as W
from oracle import model as M
from tests import _gpu
from tests import test_gpu_attention as TA
from tests import test_gpu_forward as TF
from tests import test_gpu_greedy as TG
from tests import test_gpu_int8 as TI
from tests import test_gpu_paged as TP
from tests import test_gpu_round as TR
from tests import test_gpu_sampler as TS
from workloads import gen

pytestmark = pytest.mark.gpu


def _attention_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype = ["bf16", "f16", "f32"][rng.integers(3)]
        D = int(rng.choice([64, 128])) if dtype != "f32" else int(rng.choice([24, 32, 64, 128]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8]))
        n_q = int(rng.integers(1, 17))
        while G * n_q > 256:
            n_q //= 2
        Lmax = int(rng.choice([5, 40, 300, 2000, 6000]))
        B = int(rng.integers(1, 25))
        while B * G * Hkv * n_q * max(Lmax, 1) > 3e7 and B > 1:
            B //= 2
        lens = rng.integers(0, Lmax + 1, size=B).astype(np.int32)
        hint = int(lens.max()) + int(rng.choice([0, 0, 7, 100]))
        max_T = hint + n_q + int(rng.integers(0, 9))
        out.append(dict(dtype=dtype, B=B, Hq=G * Hkv, Hkv=Hkv, n_q=n_q, D=D, lens=lens, hint=hint, max_T=max_T))
    return out


def _sampler_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype = ["f32", "bf16"][rng.integers(2)]
        V = int(rng.choice([1, 2, 17, 96, 1000, 4097, 32000, 65536, 128256, 151936, 200003]))
        gamma = int(rng.integers(1, 32))
        B = int(rng.integers(1, 200))
        while B * (2 * gamma + 1) * V > 6e7 and B > 1:
            B //= 2
        out.append(dict(dtype=dtype, V=V, gamma=gamma, B=B, T=float(rng.choice([0.3, 0.7, 1.0, 1.6])),
                        t_std=float(rng.choice([1.0, 2.5, 4.0])), mix=float(rng.choice([0.5, 0.9, 1.0])),
                        noise_std=float(rng.choice([0.3, 1.0]))))
    return out


def _greedy_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype = ["f32", "bf16"][rng.integers(2)]
        V = int(rng.choice([1, 3, 96, 2048, 4096, 4097, 50000, 131072, 151936]))
        gamma = int(rng.integers(1, 32))
        B = int(rng.integers(1, 200))
        while B * (gamma + 1) * V > 6e7 and B > 1:
            B //= 2
        out.append(dict(dtype=dtype, V=V, gamma=gamma, B=B))
    return out


def _cache_cases(n, seed, int8):
    """bf16 attention shapes for the paged and int8 caches (D 64 or 128)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8]))
        n_q = int(rng.integers(1, 17))
        while G * n_q > 256:
            n_q //= 2
        Lmax = int(rng.choice([5, 40, 300, 3000]))
        B = int(rng.integers(1, 21))
        while B * G * Hkv * n_q * max(Lmax, 1) > 2e7 and B > 1:
            B //= 2
        lens = rng.integers(0, Lmax + 1, size=B).astype(np.int32)
        hint = int(lens.max()) + int(rng.choice([0, 0, 7, 100]))
        c = dict(B=B, Hq=G * Hkv, Hkv=Hkv, n_q=n_q, D=D, lens=lens, hint=hint)
        if int8:
            c["max_T"] = (hint + n_q + int(rng.integers(0, 9)) + 7) // 8 * 8
        else:
            c["page"] = int(rng.choice([16, 32]))
            c["max_T"] = hint + n_q + int(rng.integers(0, 9))
        out.append(c)
    return out


def _forward_cases(n, seed):
    """Decoder shapes the forward supports: C a multiple of 16 up to 144, C/H
    a head dimension of the fp32 attention."""
    rng = np.random.default_rng(seed)
    shapes = [(48, 2), (96, 4), (144, 6), (32, 1), (64, 2), (96, 3), (128, 4), (64, 1), (128, 2), (128, 1)]
    out = []
    for _ in range(n):
        C, H = shapes[rng.integers(len(shapes))]
        V = int(rng.choice([5, 96, 1000, 1500, 5000]))
        L = int(rng.integers(1, 5))
        nq = int(rng.integers(1, 17))
        B = int(rng.integers(1, 21))
        hi = int(rng.choice([0, 30, 200, 480]))
        lo = int(rng.integers(0, hi + 1))
        max_T = hi + nq + int(rng.integers(0, 9))
        T = max(max_T, int(rng.choice([64, 512])))
        out.append(dict(V=V, C=C, L=L, H=H, T=T, B=B, n=nq, lo=lo, hi=hi, max_T=max_T))
    return out


def _round_cases(n, seed):
    """Target and draft decoders of one vocabulary, round counts and lengths
    that fit the caches (prompts of 4-12 tokens)."""
    rng = np.random.default_rng(seed)
    shapes = [(48, 2), (96, 4), (144, 6), (32, 1), (64, 2), (96, 3), (128, 4), (64, 1), (128, 2)]
    out = []
    for _ in range(n):
        V = int(rng.choice([96, 500, 1500]))
        (tc, th), (dc, dh) = shapes[rng.integers(len(shapes))], shapes[rng.integers(len(shapes))]
        gamma = int(rng.integers(1, 16))
        rounds = int(rng.integers(2, 5))
        max_len = 12 + rounds * (gamma + 1) + 2
        out.append(dict(V=V, target=(tc, int(rng.integers(1, 4)), th), draft=(dc, int(rng.integers(1, 3)), dh),
                        gamma=gamma, T=float(rng.choice([0.0, 0.5, 1.0, 1.5])), rounds=rounds,
                        B=int(rng.integers(2, 13)), max_len=max_len))
    return out


def _long_cases(n, seed):
    """Batches of long caches (device-drawn), sequences sampled for the check.
    65-80 rows per KV head run the five-wave kernel on 512 workgroups, and the
    batch is large enough that an equal share of the key blocks exceeds 300
    blocks, so the launch merges the pieces itself."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        # 65-80 rows per KV head: the five-wave kernel (512 workgroups)
        Hq, Hkv, n_q = [(64, 8, 9), (32, 4, 9), (64, 4, 5), (128, 8, 5)][rng.integers(4)]
        hi = int(rng.integers(24576, 32769))
        lo = int(rng.integers(8192, hi + 1))
        need = -(-300 * 512 * 32 * 2 // (Hkv * (lo + hi)))  # sequences for a 300-block share
        B = max(need, int(rng.integers(8, 65)))
        out.append(dict(dtype=["bf16", "f16"][rng.integers(2)], D=int(rng.choice([64, 128])), Hq=Hq, Hkv=Hkv,
                        n_q=n_q, B=B, L=(lo, hi)))
    return out


def _large_sampler_cases(n, seed):
    """bf16 logits drawn on the device, batches of over 65,536 row segments of
    2,048 logits (the statistics pass's large-batch launch shape)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        V = int(rng.choice([65536, 100003, 128256, 151936]))
        gamma = int(rng.integers(2, 16))
        nseg = -(-V // 2048)
        need = -(-65537 // ((2 * gamma + 1) * nseg))
        out.append(dict(V=V, gamma=gamma, B=max(need, int(rng.integers(16, 129))), T=float(rng.choice([0.7, 1.0, 1.3])),
                        t_std=float(rng.choice([2.5, 4.0])), mix=float(rng.choice([0.8, 0.95])),
                        noise_std=float(rng.choice([0.5, 1.0]))))
    return out


ATT = _attention_cases(40, 2026)
SMP_LARGE = _large_sampler_cases(4, 2034)
LONG = _long_cases(4, 2033)
RND = _round_cases(8, 2032)
FWD = _forward_cases(12, 2031)
PAGED = _cache_cases(15, 2029, int8=False)
INT8 = _cache_cases(15, 2030, int8=True)
SMP = _sampler_cases(30, 2027)
GR = _greedy_cases(20, 2028)


@pytest.mark.parametrize("i", range(len(ATT)))
def test_attention_random_shape(i):
    c = ATT[i]
    print(f"\n[case] attention {i} " + " ".join(f"{k}={v}" for k, v in c.items() if k != "lens")
          + f" lens[:8]={c['lens'][:8].tolist()}", flush=True)
    cfg = W.Config(90, "random", B=c["B"], gamma=c["n_q"] - 1, V=1, dtype=c["dtype"], Hq=c["Hq"], Hkv=c["Hkv"],
                   D=c["D"], L=(0, max(int(c["lens"].max()), 1)), max_T=c["max_T"])
    inp = W.attention_inputs(cfg, B=c["B"], max_T=c["max_T"], lens=c["lens"])
    out, kc, vc = TA._run_host(inp, hint=c["hint"], poison_tail=True)
    TA._check(inp, out, kc, vc, c["dtype"])


@pytest.mark.parametrize("i", range(len(LONG)))
def test_attention_random_long(i):
    c = LONG[i]
    print(f"\n[case] long attention {i} {c}", flush=True)
    cfg = W.Config(89, "random-long", B=c["B"], gamma=c["n_q"] - 1, V=1, dtype=c["dtype"], Hq=c["Hq"], Hkv=c["Hkv"],
                   D=c["D"], L=c["L"], max_T=c["L"][1] + c["n_q"] + 8)
    d = W.attention_inputs_device(cfg, "cuda")
    seqs = TA._sample_long(_gpu.to_host(d["lens"]), 4, 89 + i)
    before = TA._rows_before(d, seqs)
    out = sv.spec_verify_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["lens"], c["L"][1])
    torch.cuda.synchronize()
    TA._check_one_by_one(d, out, seqs, c["dtype"], before)
    del d
    torch.cuda.empty_cache()


def _describe(c):
    return " ".join(f"{k}={v}" for k, v in c.items() if k != "lens") + f" lens[:8]={c['lens'][:8].tolist()}"


@pytest.mark.parametrize("i", range(len(PAGED)))
def test_paged_random_shape(i):
    c = PAGED[i]
    print(f"\n[case] paged {i} " + _describe(c), flush=True)
    cfg = W.Config(93, "random", B=c["B"], gamma=c["n_q"] - 1, V=1, dtype="bf16", Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"],
                   L=(0, max(int(c["lens"].max()), 1)), max_T=c["max_T"])
    inp = W.attention_inputs(cfg, B=c["B"], max_T=c["max_T"], lens=c["lens"])
    TP._check(inp, c["page"], TP._run(inp, c["page"], rng=1000 + i, hint=c["hint"]))


@pytest.mark.parametrize("i", range(len(INT8)))
def test_int8_random_shape(i):
    c = INT8[i]
    print(f"\n[case] int8 {i} " + _describe(c), flush=True)
    cfg = W.Config(94, "random", B=c["B"], gamma=c["n_q"] - 1, V=1, dtype="bf16", Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"],
                   L=(0, max(int(c["lens"].max()), 1)), max_T=c["max_T"])
    inp = W.attention_inputs_int8(cfg, B=c["B"], max_T=c["max_T"], lens=c["lens"])
    TI._check(inp, TI._run(inp, hint=c["hint"]))


@pytest.mark.parametrize("i", range(len(FWD)))
def test_forward_random_shape(i):
    c = FWD[i]
    print(f"\n[case] forward {i} {c}", flush=True)
    cfg = M.ModelConfig(c["V"], c["C"], c["L"], c["H"], c["T"])
    params = gen.model_params(M.param_shapes(cfg), 300 + i)
    inp = gen.forward_inputs(cfg.V, cfg.L, cfg.H, cfg.D, c["B"], c["n"], (c["lo"], c["hi"]), c["max_T"], 400 + i)
    lg_g, kv_g = TF._run(cfg, params, inp["tokens"], inp["lens"], inp["kv"], c["hi"])
    lg_o, kv_o = M.forward_cached(params, cfg, inp["tokens"], inp["kv"], inp["lens"])
    err = np.abs(lg_g - lg_o).max()
    print(f"max |logit error| {err:.3g}", flush=True)
    assert err < TF.TOL
    for b in range(c["B"]):
        p0 = int(inp["lens"][b])
        np.testing.assert_allclose(kv_g[:, :, b, :, p0 : p0 + c["n"]], kv_o[:, :, b, :, p0 : p0 + c["n"]], rtol=0,
                                   atol=TF.TOL)
        np.testing.assert_array_equal(kv_g[:, :, b, :, :p0], inp["kv"][:, :, b, :, :p0])
        np.testing.assert_array_equal(kv_g[:, :, b, :, p0 + c["n"] :], inp["kv"][:, :, b, :, p0 + c["n"] :])


@pytest.mark.parametrize("i", range(len(RND)))
def test_round_random_shape(i):
    c = RND[i]
    print(f"\n[case] round {i} {c}", flush=True)
    ct = M.ModelConfig(c["V"], c["target"][0], c["target"][1], c["target"][2], 128)
    cd = M.ModelConfig(c["V"], c["draft"][0], c["draft"][1], c["draft"][2], 128)
    TR.run_rounds(ct, cd, c["T"], c["gamma"], c["rounds"], B=c["B"], max_len=c["max_len"], max_T=c["max_len"],
                  seed=500 + i)


@pytest.mark.parametrize("i", range(len(SMP)))
def test_sampler_random_shape(i):
    c = SMP[i]
    print(f"\n[case] sampler {i} {c}", flush=True)
    cfg = W.Config(91, "random", B=c["B"], gamma=c["gamma"], V=c["V"], dtype=c["dtype"], t_std=c["t_std"],
                   mix=c["mix"], noise_std=c["noise_std"])
    inp = W.sampler_inputs(cfg, temperature=c["T"])
    n, tok, p, q = TS._run(inp)
    print("stats", _gpu.compare_sampler(TS._oracle(inp), n, tok, p, q), flush=True)


@pytest.mark.parametrize("i", range(len(SMP_LARGE)))
def test_sampler_random_large_batch(i):
    c = SMP_LARGE[i]
    print(f"\n[case] large-batch sampler {i} {c}", flush=True)
    cfg = W.Config(88, "random-large", B=c["B"], gamma=c["gamma"], V=c["V"], dtype="bf16", t_std=c["t_std"],
                   mix=c["mix"], noise_std=c["noise_std"])
    d = W.sampler_inputs_device(cfg, "cuda", temperature=c["T"])
    n, tok, p, q = sv.spec_reject_sample(d["target_logits"], d["draft_logits"], d["draft_tokens"], d["uniforms"],
                                         c["T"], want_probs=True)
    torch.cuda.synchronize()
    seqs = np.sort(np.random.default_rng(88 + i).choice(c["B"], size=16, replace=False))
    host = {k: _gpu.to_host(d[k][seqs]) for k in ("target_logits", "draft_logits", "draft_tokens", "uniforms")}
    host["temperature"] = c["T"]
    st = _gpu.compare_sampler(TS._oracle(host), _gpu.to_host(n)[seqs], _gpu.to_host(tok)[seqs],
                              _gpu.to_host(p)[seqs], _gpu.to_host(q)[seqs])
    print("stats", st, flush=True)


@pytest.mark.parametrize("i", range(len(GR)))
def test_greedy_random_shape(i):
    c = GR[i]
    print(f"\n[case] greedy {i} {c}", flush=True)
    cfg = W.Config(92, "random", B=c["B"], gamma=c["gamma"], V=c["V"], dtype=c["dtype"], t_std=2.0, mix=0.9,
                   noise_std=0.5)
    inp = W.sampler_inputs(cfg)
    zt = inp["target_logits"]
    x = TG._greedy_drafts(inp["draft_logits"])
    TG._check(zt, x, TG._run(zt, x))
