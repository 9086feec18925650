"""spec_reject_sample_noalloc through the C ABI.

The no-allocation variant must give exactly the outputs of spec_reject_sample
called with a caller workspace (same kernels, its scratch in place of the
workspace), and those must be the oracle's (the parity rule of the sampler
tests).  Two calls in a row, the second with a smaller input, so the second
runs over scratch the first left behind; then a greedy call; then the size
limit, refused before any launch.
"""

import ctypes

import numpy as np
import pytest
import torch

import speculative_decoding_verification_spec_amd as sv
import workloads as W
from oracle import greedy as Gr
from oracle import sampler as S
from speculative_decoding_verification_spec_amd import _lib
from tests import _gpu

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dev_inputs(inp):
    return {k: _gpu.to_dev(inp[k]) for k in ("target_logits", "draft_logits", "draft_tokens", "uniforms")}


def _outputs(B, G):
    return (torch.full((B,), -7, dtype=torch.int32, device="cuda"),
            torch.full((B, G + 1), -7, dtype=torch.int32, device="cuda"),
            torch.full((B, G), -7.0, dtype=torch.float32, device="cuda"),
            torch.full((B, G), -7.0, dtype=torch.float32, device="cuda"))


def _run(d, T, noalloc):
    """One call through the C ABI; returns host (n, tokens, p, q)."""
    L = sv.load()
    tl = d["target_logits"]
    B, G1, V = tl.shape
    G = G1 - 1
    dt = _lib.SPEC_BF16 if tl.dtype == torch.bfloat16 else _lib.SPEC_F32
    n, tok, p, q = _outputs(B, G)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [_p(tl), _p(d["draft_logits"]), _p(d["draft_tokens"]), _p(d["uniforms"]), B, G, V, float(T), dt,
            _p(n), _p(tok), _p(p), _p(q)]
    if noalloc:
        st = L.spec_reject_sample_noalloc(*args, stream)
    else:
        nbytes = L.spec_reject_sample_workspace_size(B, G, V, dt)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        st = L.spec_reject_sample(*args, _p(ws), nbytes, stream)
    assert st == _lib.SPEC_OK, L.spec_status_string(st)
    torch.cuda.synchronize()
    return tuple(_gpu.to_host(t) for t in (n, tok, p, q))


def _same_bits(a, b):
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                              y.view(np.uint32) if y.dtype == np.float32 else y)


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_noalloc_equals_the_workspace_call_twice_in_a_row(T):
    big = W.get(4)  # 32 sequences over 151,936 bf16 logits
    small = W.Config(99, "ragged", B=9, gamma=3, V=1003, dtype="bf16", t_std=2.5, mix=0.9, noise_std=1.0)
    for cfg in (big, small):  # the second call is the smaller one
        print(f"\n[case] noalloc T={T} B={cfg.B} gamma={cfg.gamma} V={cfg.V}", flush=True)
        inp = W.sampler_inputs(cfg, temperature=1.0 if T == 0 else T)
        if T == 0:  # greedy: the drafts are the draft model's argmax
            inp["draft_tokens"] = np.argmax(_gpu.as_f64(inp["draft_logits"]), axis=-1).astype(np.int32)
        d = _dev_inputs(inp)
        want = _run(d, T, noalloc=False)
        got = _run(d, T, noalloc=True)
        _same_bits(got, want)
        if T == 0:
            n_o, tok_o, _ = Gr.verify_batch(inp["target_logits"], inp["draft_tokens"])
            assert np.array_equal(got[0], n_o) and np.array_equal(got[1], tok_o)
        else:
            orc = S.verify_batch(inp["target_logits"], inp["draft_logits"], inp["draft_tokens"], inp["uniforms"], T)
            print("stats", _gpu.compare_sampler(orc, got[0], got[1], got[2], got[3]), flush=True)


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_noalloc_at_config5_then_config4(T):
    """Config 5 (256 sequences over 128,256 tokens: the statistics pass's
    large-batch launch shape, 4.6 MiB of scratch), then config 4 over the
    scratch it left: bit for bit the workspace call's outputs (which the
    sampler tests check against the oracle at both shapes)."""
    for cid in (5, 4):
        cfg = W.get(cid)
        print(f"\n[case] noalloc T={T} config{cid} B={cfg.B} gamma={cfg.gamma} V={cfg.V}", flush=True)
        d = W.sampler_inputs_device(cfg, "cuda", temperature=1.0 if T == 0 else T)
        d = {k: d[k] for k in ("target_logits", "draft_logits", "draft_tokens", "uniforms")}
        if T == 0:
            d["draft_tokens"] = torch.argmax(d["draft_logits"].float(), dim=-1).to(torch.int32)
        want = _run(d, T, noalloc=False)
        got = _run(d, T, noalloc=True)
        _same_bits(got, want)
        del d
        torch.cuda.empty_cache()


def test_noalloc_refuses_more_than_its_scratch():
    print("\n[case] noalloc size limit", flush=True)
    L = sv.load()
    dummy = torch.zeros(16, dtype=torch.int32, device="cuda")
    B, G, V = 4096, 31, 1 << 20  # needs far more than 16 MiB of workspace
    assert L.spec_reject_sample_workspace_size(B, G, V, _lib.SPEC_BF16) > (16 << 20)
    st = L.spec_reject_sample_noalloc(_p(dummy), _p(dummy), _p(dummy), _p(dummy), B, G, V, 1.0, _lib.SPEC_BF16,
                                      _p(dummy), _p(dummy), None, None, None)
    assert st == _lib.SPEC_ERR_SCRATCH
    assert L.spec_status_string(st) == b"SPEC_ERR_SCRATCH"
