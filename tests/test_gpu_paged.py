"""GPU parity of spec_verify_attention_paged (paged KV cache, block tables).

The caches of the contiguous workloads are cut into pages placed at seeded
random physical slots; unused slots hold NaN.  The output must match the
oracle (bf16 tolerance) and be bit-identical to the contiguous kernel on the
same data; the new rows must land in the slots the table names and no other
slot may change.  Every case prints its name first.
"""

import numpy as np
import pytest
import torch

import speculative_decoding_verification_spec_amd as sv
import workloads as W
from oracle import paged as P
from tests import _gpu

pytestmark = pytest.mark.gpu

NAN_BF16 = np.uint16(0x7FC0)


def _case(name, **kw):
    print(f"\n[case] {name} {kw}", flush=True)


def _paginate(cache, lens, n_q, page, rng, hint, spare=3, share_prefix=False):
    """Pages [Hkv, num_pages, page, D] and table [B, max_blocks] holding cache[b, :, :L_b].

    The table has room for hint + n_q positions, as the call requires.
    """
    B, Hkv, _, D = cache.shape
    need = [P.blocks_needed(int(L) + n_q, page) for L in lens]
    max_blocks = max(max(need), P.blocks_needed(hint + n_q, page))
    num_pages = sum(need) + spare
    perm = rng.permutation(num_pages)
    pages = np.full((Hkv, num_pages, page, D), NAN_BF16, dtype=cache.dtype)
    table = np.full((B, max_blocks), -7, np.int32)  # entries past a sequence's blocks are never used
    k = 0
    for b in range(B):
        for i in range(need[b]):
            table[b, i] = perm[k]
            k += 1
    if share_prefix:  # sequence 1 reads sequence 0's first full blocks
        full0 = min(int(lens[0]), int(lens[1])) // page
        table[1, :full0] = table[0, :full0]
    for b in range(B):
        L = int(lens[b])
        for pos0 in range(0, L, page):
            m = min(page, L - pos0)
            pages[:, table[b, pos0 // page], :m] = cache[b, :, pos0 : pos0 + m]
    return pages, table


def _run(inp, page, rng, hint=None, share_prefix=False, corrupt=None):
    lens = inp["lens"]
    n_q = inp["q"].shape[2]
    if share_prefix:
        full0 = min(int(lens[0]), int(lens[1])) // page * page
        inp["k_cache"][1, :, :full0] = inp["k_cache"][0, :, :full0]
        inp["v_cache"][1, :, :full0] = inp["v_cache"][0, :, :full0]
    hint = int(lens.max()) if hint is None else hint
    kp, table = _paginate(inp["k_cache"], lens, n_q, page, np.random.default_rng(rng), hint, share_prefix=share_prefix)
    vp, _ = _paginate(inp["v_cache"], lens, n_q, page, np.random.default_rng(rng), hint, share_prefix=share_prefix)
    if corrupt is not None:
        b, i, val = corrupt
        table[b, i] = val
    d = {k: _gpu.to_dev(v) for k, v in inp.items()}
    dkp, dvp, dtab = _gpu.to_dev(kp), _gpu.to_dev(vp), _gpu.to_dev(table)
    out = sv.spec_verify_attention_paged(d["q"], d["k_new"], d["v_new"], dkp, dvp, dtab, d["lens"], hint)
    ref = sv.spec_verify_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["lens"], hint)
    torch.cuda.synchronize()
    return (_gpu.to_host(out), _gpu.to_host(ref), kp, vp, table, _gpu.to_host(dkp), _gpu.to_host(dvp))


def _check(inp, page, res, skip=()):
    out, ref, kp, vp, table, kp2, vp2 = res
    lens = inp["lens"]
    n_q = inp["q"].shape[2]
    seqs = [b for b in range(len(lens)) if b not in skip]
    want = P.verify_attention_paged(inp["q"], inp["k_new"], inp["v_new"], kp, vp, table, lens, seqs=seqs)
    got = _gpu.as_f64(out[seqs])
    _gpu.check_attention(got, want, "bf16")
    assert np.array_equal(out[seqs], ref[seqs])  # same bits as the contiguous kernel
    # the new rows, and nothing else, were written
    kw, vw = P.kv_append_paged(kp, vp, inp["k_new"][seqs], inp["v_new"][seqs], table[seqs], lens[seqs])
    assert np.array_equal(kp2, kw) and np.array_equal(vp2, vw)


@pytest.mark.parametrize("page", [16, 32])
def test_config4_paged(page):
    cfg = W.get(4)
    _case("paged config4", B=cfg.B, page=page)
    inp = W.attention_inputs(cfg)
    _check(inp, page, _run(inp, page, rng=page, hint=cfg.L[1]))


@pytest.mark.parametrize(
    "B,Hq,Hkv,n_q,D,lens,page",
    [
        (3, 8, 2, 5, 128, [0, 31, 33], 16),       # empty cache, block edges
        (2, 16, 2, 9, 128, [257, 2000], 32),      # 72 rows per KV head (5 tiles)
        (2, 4, 4, 1, 64, [1, 1000], 16),          # n_q = 1, D = 64
        (1, 8, 1, 5, 128, [3000], 32),            # one sequence over many workgroups
        (2, 16, 1, 16, 128, [100, 300], 16),      # 256 rows per KV head: row groups
        (2, 32, 1, 7, 64, [70, 5], 32),           # MQA at D = 64, 224 rows
        (300, 4, 4, 3, 128, None, 16),            # many one- or two-block slabs
    ],
)
def test_shapes(B, Hq, Hkv, n_q, D, lens, page):
    _case("paged shape", B=B, Hq=Hq, Hkv=Hkv, n_q=n_q, D=D, lens=lens, page=page)
    if lens is None:
        lens = np.random.default_rng(B).integers(0, 40, B).astype(np.int32)
    max_T = max(lens) + n_q + 7
    cfg = W.Config(96, "paged", B=B, gamma=n_q - 1, V=1, dtype="bf16", Hq=Hq, Hkv=Hkv, D=D, L=(0, max(lens)),
                   max_T=max_T)
    inp = W.attention_inputs(cfg, B=B, max_T=max_T, lens=lens)
    _check(inp, page, _run(inp, page, rng=B))


def test_shared_prefix_pages():
    cfg = W.get(4)
    _case("paged shared prefix")
    inp = W.attention_inputs(cfg, B=4, lens=[1500, 1700, 1024, 2100])
    _check(inp, 16, _run(inp, 16, rng=5, share_prefix=True))


def test_bad_table_entry_flags_only_its_sequence():
    cfg = W.get(4)
    _case("paged bad entry")
    inp = W.attention_inputs(cfg, B=3, lens=[700, 900, 1200])
    res = _run(inp, 32, rng=7, corrupt=(1, 5, 10 ** 6))  # sequence 1, block 5: no such page
    out = res[0]
    assert np.all(np.isnan(_gpu.as_f64(out[1])))
    out2, ref, kp, vp, table, kp2, vp2 = res
    # the others are exact; sequence 1's new rows may or may not be written
    want = P.verify_attention_paged(inp["q"], inp["k_new"], inp["v_new"], kp, vp, table, inp["lens"], seqs=[0, 2])
    assert np.max(np.abs(_gpu.as_f64(out[[0, 2]]) - want)) < _gpu.ATT_TOL["bf16"]


def test_status_codes():
    _case("paged status")
    dev = "cuda"
    q = torch.zeros((1, 4, 5, 128), dtype=torch.bfloat16, device=dev)
    kn = torch.zeros((1, 2, 5, 128), dtype=torch.bfloat16, device=dev)
    pages = torch.zeros((2, 4, 16, 128), dtype=torch.bfloat16, device=dev)
    table = torch.zeros((1, 4), dtype=torch.int32, device=dev)
    lens = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(sv.SpecError) as e:
        sv.spec_verify_attention_paged(q, kn, kn, pages, pages.clone(), table, lens, 60)  # 60 + 5 > 4 * 16
    assert e.value.status == 2
    p8 = torch.zeros((2, 4, 8, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(sv.SpecError) as e:
        sv.spec_verify_attention_paged(q, kn, kn, p8, p8.clone(), table, lens, 10)  # page size 8
    assert e.value.status == 3
    B = 1025  # above the stream scheme's 1024 sequences
    with pytest.raises(sv.SpecError) as e:
        sv.spec_verify_attention_paged(torch.zeros((B, 4, 5, 128), dtype=torch.bfloat16, device=dev),
                                       torch.zeros((B, 2, 5, 128), dtype=torch.bfloat16, device=dev),
                                       torch.zeros((B, 2, 5, 128), dtype=torch.bfloat16, device=dev), pages,
                                       pages.clone(), torch.zeros((B, 4), dtype=torch.int32, device=dev),
                                       torch.zeros(B, dtype=torch.int32, device=dev), 10)
    assert e.value.status == 3


def _device_paged(dtype, kind):
    """Device inputs of a long (merged in the launch) or short (combine launch)
    batch with empty, ragged, full-hint and rejected lengths, and their pages
    at random slots (32 positions a page; unused slots NaN)."""
    if kind == "long":
        cfg = W.Config(95, "merge", B=20, gamma=8, V=1, dtype=dtype, Hq=64, Hkv=8, D=128, L=(8192, 32768),
                       max_T=32800)
        hint = 32768
    else:
        cfg = W.Config(94, "short", B=6, gamma=4, V=1, dtype=dtype, Hq=32, Hkv=8, D=128, L=(100, 3000),
                       max_T=3040)
        hint = 3000
    page, n_q = 32, cfg.n_q
    d = W.attention_inputs_device(cfg, "cuda")
    for b, L in ((1, 0), (2, 31), (3, hint + 1), (4, hint)):
        d["lens"][b] = L
    lens = _gpu.to_host(d["lens"]).astype(np.int64)
    rng = np.random.default_rng(96)
    need = [(min(int(L), hint) + n_q + page - 1) // page for L in lens]
    max_blocks = (hint + n_q + page - 1) // page
    num_pages = sum(need) + 3
    perm = torch.from_numpy(rng.permutation(num_pages)).to("cuda")
    table = torch.full((cfg.B, max_blocks), -7, dtype=torch.int32, device="cuda")
    pages = [torch.full((cfg.Hkv, num_pages, page, cfg.D), float("nan"), dtype=d["k_cache"].dtype, device="cuda")
             for _ in range(2)]
    k = 0
    for b in range(cfg.B):
        idx = perm[k : k + need[b]]
        k += need[b]
        table[b, : need[b]] = idx.to(torch.int32)
        L = min(int(lens[b]), hint)
        nf = L // page
        for src, dst in ((d["k_cache"], pages[0]), (d["v_cache"], pages[1])):
            if nf:
                dst[:, idx[:nf]] = src[b, :, : nf * page].reshape(cfg.Hkv, nf, page, cfg.D)
            if L % page:
                dst[:, idx[nf], : L % page] = src[b, :, nf * page : L]
    return cfg, hint, page, d, lens, need, table, pages


@pytest.mark.parametrize("dtype,kind", [("bf16", "long"), ("f16", "long"), ("f16", "short")])
def test_paged_equals_contiguous_device_built(dtype, kind):
    """The paged kernel must give the contiguous kernel's bits (which
    tests/test_gpu_attention.py checks against the oracle), with empty,
    ragged, full-hint and rejected lengths and pages at random slots: long
    shares (the launch merges each slab's pieces itself) and short ones (a
    combine launch), bf16 and fp16 caches."""
    _case("paged vs contiguous", dtype=dtype, kind=kind)
    cfg, hint, page, d, lens, need, table, pages = _device_paged(dtype, kind)
    n_q = cfg.n_q
    out_p = sv.spec_verify_attention_paged(d["q"], d["k_new"], d["v_new"], pages[0], pages[1], table, d["lens"], hint)
    out_c = sv.spec_verify_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["lens"], hint)
    torch.cuda.synchronize()
    assert torch.equal(out_p.view(torch.int16), out_c.view(torch.int16))
    assert torch.isnan(out_p[3].float()).all()
    for b in (0, 4, cfg.B - 1):  # the appended rows landed in the tabled slots
        L = int(lens[b])
        for t in range(n_q):
            slot = int(table[b, (L + t) // page])
            assert torch.equal(pages[0][:, slot, (L + t) % page], d["k_cache"][b, :, L + t])
            assert torch.equal(pages[1][:, slot, (L + t) % page], d["v_cache"][b, :, L + t])


@pytest.mark.parametrize("kind", ["long", "short"])
def test_bad_entries_over_the_first_pieces_flag_the_sequence(kind):
    """Bad page entries over the first 60% of a long sequence's table: every
    piece that meets one leaves NaN, and the merge of the slab's pieces (in
    the launch or in the combine launch) must keep the NaN even when a whole
    group of the first pieces it merges together is flagged.  The other
    sequences keep the contiguous kernel's bits."""
    _case("paged bad first pieces", kind=kind)
    cfg, hint, page, d, lens, need, table, pages = _device_paged("bf16", kind)
    bad = 4  # length = hint: the longest table
    table[bad, : need[bad] * 6 // 10] = 10 ** 6
    out_p = sv.spec_verify_attention_paged(d["q"], d["k_new"], d["v_new"], pages[0], pages[1], table, d["lens"], hint)
    out_c = sv.spec_verify_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["lens"], hint)
    torch.cuda.synchronize()
    assert torch.isnan(out_p[bad].float()).all()
    good = [b for b in range(cfg.B) if b not in (3, bad)]
    assert torch.equal(out_p[good].view(torch.int16), out_c[good].view(torch.int16))


def test_config5_shape_paged_equals_contiguous():
    """The shape bench.py times with --paged: config 5 (256 sequences, GQA
    64/8, 8K-32K keys per KV head), its cache copied into 32- and then
    16-position pages at seeded random slots.  The paged call must give the
    contiguous call's bits on every sequence (the contiguous kernel is checked
    against the oracle at this shape in tests/test_gpu_attention.py), and the
    appended rows must land in the tabled slots."""
    cfg = W.get(5)
    hint, n_q = cfg.L[1], cfg.n_q
    d = W.attention_inputs_device(cfg, "cuda")
    lens = _gpu.to_host(d["lens"]).astype(np.int64)
    out_c = sv.spec_verify_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["lens"], hint)
    torch.cuda.synchronize()
    for page in (32, 16):
        _case("paged vs contiguous, config 5", B=cfg.B, page=page)
        need = [(int(L) + n_q + page - 1) // page for L in lens]
        max_blocks = (hint + n_q + page - 1) // page
        num_pages = sum(need) + 5
        perm = torch.from_numpy(np.random.default_rng(page).permutation(num_pages)).to("cuda")
        table = torch.full((cfg.B, max_blocks), -1, dtype=torch.int32, device="cuda")
        pages = [torch.full((cfg.Hkv, num_pages, page, cfg.D), float("nan"), dtype=torch.bfloat16, device="cuda")
                 for _ in range(2)]
        k = 0
        for b in range(cfg.B):
            idx = perm[k : k + need[b]]
            k += need[b]
            table[b, : need[b]] = idx.to(torch.int32)
            L = int(lens[b])
            nf = L // page
            for src, dst in ((d["k_cache"], pages[0]), (d["v_cache"], pages[1])):  # rows < L: before any append
                dst[:, idx[:nf]] = src[b, :, : nf * page].reshape(cfg.Hkv, nf, page, cfg.D)
                if L % page:
                    dst[:, idx[nf], : L % page] = src[b, :, nf * page : L]
        out_p = sv.spec_verify_attention_paged(d["q"], d["k_new"], d["v_new"], pages[0], pages[1], table, d["lens"],
                                               hint)
        torch.cuda.synchronize()
        same = (out_p.view(torch.int16) == out_c.view(torch.int16)).flatten(1).all(dim=1)
        print("sequences identical", int(same.sum()), "of", cfg.B, flush=True)
        assert bool(same.all()), torch.nonzero(~same).flatten()[:10].tolist()
        for b in (0, 1, int(np.argmax(lens)), cfg.B - 1):
            L = int(lens[b])
            for t in range(n_q):
                slot = int(table[b, (L + t) // page])
                assert torch.equal(pages[0][:, slot, (L + t) % page], d["k_cache"][b, :, L + t])
                assert torch.equal(pages[1][:, slot, (L + t) % page], d["v_cache"][b, :, L + t])
        del pages, table, out_p
        torch.cuda.empty_cache()
