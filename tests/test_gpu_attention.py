"""GPU parity of spec_verify_attention (KV append + causal multi-query attention).

Compared with the oracle element by element on seeded inputs (fp32: 1e-4,
bf16: 2e-2 absolute) and, for 16-bit outputs, row by row relative to each
row's size (tests/_gpu.ROW_REL_TOL: tight enough that a lost 32-key block of
a 32K-key cache fails); the appended cache rows must equal k_new / v_new bit
for bit and no other cache row may change.  Every case prints its name first.
"""

import dataclasses

import numpy as np
import pytest
import torch

import speculative_decoding_verification_spec_amd as sv
import workloads as W
from oracle import attention as A
from tests import _gpu

pytestmark = pytest.mark.gpu


def _case(name, **kw):
    print(f"\n[case] {name} {kw}", flush=True)


def _run_host(inp, hint=None, poison_tail=False):
    """Upload host inputs, run the ABI call, return (out, k_cache, v_cache) on the host."""
    dev = {k: _gpu.to_dev(v) for k, v in inp.items()}
    lens = inp["lens"]
    if poison_tail:  # rows at and past L_b hold NaN: they must never be read
        for b, L in enumerate(lens):
            dev["k_cache"][b, :, L:] = float("nan")
            dev["v_cache"][b, :, L:] = float("nan")
    hint = int(lens.max()) if hint is None else hint
    out = sv.spec_verify_attention(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                                   dev["lens"], hint)
    torch.cuda.synchronize()
    return _gpu.to_host(out), _gpu.to_host(dev["k_cache"]), _gpu.to_host(dev["v_cache"])


def _check(inp, out, kc, vc, dtype, seqs=None, cache_before=None):
    seqs = range(inp["q"].shape[0]) if seqs is None else list(seqs)
    want = A.verify_attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                              inp["lens"], seqs=seqs)
    got = _gpu.as_f64(out[list(seqs)])
    _gpu.check_attention(got, want, dtype)
    n = inp["k_new"].shape[2]
    before_k = inp["k_cache"] if cache_before is None else cache_before[0]
    before_v = inp["v_cache"] if cache_before is None else cache_before[1]
    for b in seqs:
        L = int(inp["lens"][b])
        assert np.array_equal(kc[b, :, L:L + n], inp["k_new"][b])
        assert np.array_equal(vc[b, :, L:L + n], inp["v_new"][b])
        assert np.array_equal(kc[b, :, :L], before_k[b, :, :L])
        assert np.array_equal(vc[b, :, :L], before_v[b, :, :L])


def test_config3_full_and_uncached():
    cfg = W.get(3)
    _case("config3", B=cfg.B, H=cfg.Hq, D=cfg.D, L=cfg.L)
    inp = W.attention_inputs(cfg)
    out, kc, vc = _run_host(inp)
    _check(inp, out, kc, vc, "f32")
    # against the uncached recompute over the whole sequence (random queries
    # stand in for the prefix rows, whose outputs are discarded)
    rng = np.random.default_rng(3)
    for b in (0, 17, 63):
        L = int(inp["lens"][b])
        q_all = np.concatenate([rng.normal(size=(cfg.Hq, L, cfg.D)), inp["q"][b].astype(np.float64)], axis=1)
        k_all = np.concatenate([inp["k_cache"][b, :, :L], inp["k_new"][b]], axis=1)
        v_all = np.concatenate([inp["v_cache"][b, :, :L], inp["v_new"][b]], axis=1)
        un = A.attention_uncached(q_all, k_all, v_all, cfg.n_q)
        assert np.max(np.abs(out[b] - un)) < 1e-4


def test_config4_full():
    cfg = W.get(4)
    _case("config4", B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, D=cfg.D)
    inp = W.attention_inputs(cfg)
    out, kc, vc = _run_host(inp, hint=cfg.L[1])
    _check(inp, out, kc, vc, "bf16")


def _sample_long(lens, k, seed):
    """The shortest and the longest sequence and k - 2 others at random: with
    thousands of slabs cut into equal shares, most sequences hold a slab whose
    pieces are merged from two workgroups."""
    lens = np.asarray(lens)
    first = [int(np.argmin(lens)), int(np.argmax(lens))]
    rest = [b for b in np.random.default_rng(seed).permutation(len(lens)) if b not in first]
    return first + [int(b) for b in rest[: k - 2]]


def _check_one_by_one(d, out, seqs, dtype, rows_before=None):
    """The check of ``_check`` on sequences copied to the host one at a time
    (each only up to its own length), so the host holds one sequence's cache."""
    n = d["k_new"].shape[2]
    for b in seqs:
        L = int(_gpu.to_host(d["lens"][b : b + 1])[0])
        one = {k: _gpu.to_host(d[k][b : b + 1]) for k in ("q", "k_new", "v_new")}
        one["lens"] = np.array([L], np.int32)
        if rows_before is None:
            one["k_cache"] = _gpu.to_host(d["k_cache"][b : b + 1, :, :L])
            one["v_cache"] = _gpu.to_host(d["v_cache"][b : b + 1, :, :L])
        else:
            one["k_cache"], one["v_cache"] = rows_before[b]
        kc = _gpu.to_host(d["k_cache"][b : b + 1, :, : L + n])
        vc = _gpu.to_host(d["v_cache"][b : b + 1, :, : L + n])
        print(f"sequence {b} L={L}", end=": ", flush=True)
        _check(one, _gpu.to_host(out[b : b + 1]), kc, vc, dtype)


def _rows_before(d, seqs):
    """Host copies of the cached rows [0, L_b) of the listed sequences."""
    out = {}
    for b in seqs:
        L = int(_gpu.to_host(d["lens"][b : b + 1])[0])
        out[b] = (_gpu.to_host(d["k_cache"][b : b + 1, :, :L]), _gpu.to_host(d["v_cache"][b : b + 1, :, :L]))
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_config5_full_size_sampled(dtype):
    """Config 5's shape as bench.py times it, with its bf16 cache and with an
    fp16 cache (as with --kv f16): 18 (bf16) or 10 (fp16) sequences, the
    shortest and the longest among them, compared one by one."""
    cfg = dataclasses.replace(W.get(5), dtype=dtype)
    _case("config5", dtype=dtype, B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, D=cfg.D, max_T=cfg.max_T)
    d = W.attention_inputs_device(cfg, "cuda")
    seqs = _sample_long(_gpu.to_host(d["lens"]), 18 if dtype == "bf16" else 10, 5)
    before = _rows_before(d, seqs)
    out = sv.spec_verify_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["lens"], cfg.L[1])
    torch.cuda.synchronize()
    _check_one_by_one(d, out, seqs, dtype, before)
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_long_caches_merged_in_launch(dtype):
    """Shares long enough that the stream launch merges each slab's pieces
    itself (its last workgroup), with empty, ragged, full-hint and rejected
    lengths in one batch."""
    cfg = W.Config(95, "merge", B=20, gamma=8, V=1, dtype=dtype, Hq=64, Hkv=8, D=128, L=(8192, 32768),
                   max_T=32800)
    hint = 32768
    _case("merge-in-launch", dtype=dtype, B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, D=cfg.D, hint=hint)
    d = W.attention_inputs_device(cfg, "cuda")
    for b, L in ((1, 0), (2, 31), (3, hint + 1), (4, hint)):
        d["lens"][b] = L
    seqs = [b for b in range(cfg.B) if b != 3]  # every sequence with a valid length
    before = _rows_before(d, seqs)
    k3 = _gpu.to_host(d["k_cache"][3])
    out = sv.spec_verify_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["lens"], hint)
    torch.cuda.synchronize()
    assert np.all(np.isnan(_gpu.as_f64(_gpu.to_host(out[3]))))  # length above the hint: flagged
    assert np.array_equal(_gpu.to_host(d["k_cache"][3]), k3)
    _check_one_by_one(d, out, seqs, dtype, before)
    del d
    torch.cuda.empty_cache()


def test_f16_outside_its_support_is_refused():
    _case("f16 status")
    dev = "cuda"
    q = torch.zeros((1100, 2, 2, 64), dtype=torch.float16, device=dev)
    kn = torch.zeros((1100, 1, 2, 64), dtype=torch.float16, device=dev)
    kc = torch.zeros((1100, 1, 8, 64), dtype=torch.float16, device=dev)
    lens = torch.zeros(1100, dtype=torch.int32, device=dev)
    with pytest.raises(sv.SpecError) as e:  # B > 1024: the fp16 cache has no fixed-split kernel
        sv.spec_verify_attention(q, kn, kn, kc, kc.clone(), lens, 4)
    assert e.value.status == 3


@pytest.mark.parametrize(
    "dtype,B,Hq,Hkv,n_q,D,lens",
    [
        ("bf16", 3, 8, 2, 5, 128, [0, 31, 33]),       # empty cache, block edges
        ("bf16", 2, 4, 4, 1, 64, [1, 1000]),           # n_q = 1, MHA, D = 64
        ("bf16", 2, 16, 2, 9, 128, [257, 4095]),       # 72 rows per KV head (5 tiles)
        ("bf16", 2, 32, 1, 7, 64, [70, 5]),            # MQA, 224 rows -> row groups
        ("f32", 3, 4, 4, 5, 24, [0, 384, 500]),
        ("f32", 2, 6, 3, 3, 32, [45, 9]),
        ("f32", 2, 8, 2, 2, 128, [130, 64]),
        ("f32", 2, 16, 2, 5, 24, [200, 77]),     # 3 row tiles, two splits merged in one workgroup
        ("f32", 2, 4, 4, 5, 24, [700, 1000]),    # 8 splits in one workgroup, idle waves for the shorter cache
        ("f32", 1, 32, 8, 4, 64, [300]),         # GQA, 3 splits in a 4-wave workgroup
        ("f32", 2, 4, 2, 5, 24, [3000, 1200]),   # 24 splits: partial slots and attn_combine
        ("f16", 3, 8, 2, 5, 128, [0, 31, 33]),   # the fp16 cache: empty, block edges
        ("f16", 2, 4, 4, 1, 64, [1, 1000]),      # fp16, n_q = 1, MHA, D = 64
        ("f16", 4, 32, 8, 5, 128, [1024, 4096, 2000, 3001]),  # fp16 at config 4's head layout and lengths
        ("bf16", 2, 16, 1, 16, 128, [100, 300]),  # n_q = 16, 256 rows per KV head: the largest group
        ("f32", 1, 16, 1, 16, 64, [50]),          # the same for fp32
    ],
)
def test_shapes_and_edges(dtype, B, Hq, Hkv, n_q, D, lens):
    _case("shape", dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, n_q=n_q, D=D, lens=lens)
    max_T = max(lens) + n_q + 7
    cfg = W.Config(98, "shape", B=B, gamma=n_q - 1, V=1, dtype=dtype, Hq=Hq, Hkv=Hkv, D=D,
                   L=(0, max(lens)), max_T=max_T)
    inp = W.attention_inputs(cfg, B=B, max_T=max_T, lens=lens)
    out, kc, vc = _run_host(inp, poison_tail=True)
    _check(inp, out, kc, vc, dtype)


@pytest.mark.parametrize(
    "B,Hq,Hkv,n_q,D,lo,hi",
    [
        (1, 8, 1, 5, 128, 5000, 5000),    # one slab cut into hundreds of pieces
        (300, 4, 4, 3, 128, 0, 3),        # many slabs of one or two blocks
        (1024, 2, 1, 2, 64, 0, 40),       # B = 1024: the largest batch of the stream scheme
        (1100, 2, 1, 2, 64, 0, 70),       # B > 1024: the fixed-split scheme
    ],
)
def test_work_distribution_edges(B, Hq, Hkv, n_q, D, lo, hi):
    """Batch shapes at the edges of how the bf16 kernel spreads key blocks over workgroups."""
    _case("distribution", B=B, Hq=Hq, Hkv=Hkv, n_q=n_q, D=D, lens=(lo, hi))
    lens = np.random.default_rng([B, lo, hi]).integers(lo, hi + 1, size=B).astype(np.int32)
    max_T = hi + n_q + 3
    cfg = W.Config(97, "distribution", B=B, gamma=n_q - 1, V=1, dtype="bf16", Hq=Hq, Hkv=Hkv, D=D,
                   L=(lo, hi), max_T=max_T)
    inp = W.attention_inputs(cfg, B=B, max_T=max_T, lens=lens)
    out, kc, vc = _run_host(inp, poison_tail=True)
    _check(inp, out, kc, vc, "bf16")


def test_cache_full_to_capacity():
    cfg = W.get(4)
    B, max_T = 2, 1024
    _case("capacity", B=B, max_T=max_T)
    inp = W.attention_inputs(cfg, B=B, max_T=max_T, lens=[max_T - cfg.n_q, 3])
    out, kc, vc = _run_host(inp, hint=max_T - cfg.n_q)
    _check(inp, out, kc, vc, "bf16")


@pytest.mark.parametrize("cid", [4, 3])
def test_length_beyond_hint_is_flagged_not_written(cid):
    cfg = W.get(cid)
    B, max_T = 2, 512
    _case("bad-length", B=B, config=cid)
    inp = W.attention_inputs(cfg, B=B, max_T=max_T, lens=[100, 400])
    out, kc, vc = _run_host(inp, hint=200)  # sequence 1 exceeds the hint
    assert np.all(np.isnan(_gpu.as_f64(out[1])))
    assert np.array_equal(kc[1], inp["k_cache"][1]) and np.array_equal(vc[1], inp["v_cache"][1])
    _check({k: v[:1] for k, v in inp.items()}, out[:1], kc[:1], vc[:1], cfg.dtype)


def test_status_codes():
    _case("status")
    dev = "cuda"
    q = torch.zeros((1, 4, 5, 128), dtype=torch.bfloat16, device=dev)
    kn = torch.zeros((1, 2, 5, 128), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device=dev)
    lens = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(sv.SpecError) as e:
        sv.spec_verify_attention(q, kn, kn, kc, kc.clone(), lens, 60)  # 60 + 5 > 64
    assert e.value.status == 2
    q3 = torch.zeros((1, 3, 5, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(sv.SpecError) as e:
        sv.spec_verify_attention(q3, kn, kn, kc, kc.clone(), lens, 10)  # 3 % 2 != 0
    assert e.value.status in (1, 3)
    q24 = torch.zeros((1, 2, 5, 24), dtype=torch.bfloat16, device=dev)
    k24 = torch.zeros((1, 2, 5, 24), dtype=torch.bfloat16, device=dev)
    c24 = torch.zeros((1, 2, 64, 24), dtype=torch.bfloat16, device=dev)
    with pytest.raises(sv.SpecError) as e:
        sv.spec_verify_attention(q24, k24, k24, c24, c24.clone(), lens, 10)  # bf16 D=24 unsupported
    assert e.value.status == 3
