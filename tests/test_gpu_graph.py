"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph on ROCm).

Every entry point only enqueues kernels on the caller's stream (no memset
nodes, no host synchronisation, no allocation once the workspace exists), so
a whole verification step -- and a whole speculative round -- can be captured
once and replayed.  Each test replays the graph several times, with eager
calls and synchronisations between the replays, and checks every replay
against the eager result of the same inputs (bit for bit: the same kernels
with the same work split).  Every case prints its name first.
"""

import numpy as np
import pytest
import torch

import speculative_decoding_verification_spec_amd as sv
import workloads as W
from oracle import model as M
from workloads.device import to_dev
from oracle import round as R
from workloads import gen

pytestmark = pytest.mark.gpu


def _case(name, **kw):
    print(f"\n[case] {name} {kw}", flush=True)


def test_verify_step_graph_replays_match_eager():
    _case("step-graph", config=4, B=8)
    dev = torch.device("cuda:0")
    cfg = W.get(4)
    a = W.attention_inputs(cfg, B=8)
    s = W.sampler_inputs(cfg, B=8)
    t = {k: to_dev(v, dev) for k, v in a.items()}
    u = {k: to_dev(v, dev) for k, v in s.items() if k != "temperature"}
    T = s["temperature"]
    hint = int(a["lens"].max())
    lens0 = t["lens"].clone()
    out = torch.empty_like(t["q"])
    n = torch.empty(8, dtype=torch.int32, device=dev)
    tok = torch.empty((8, cfg.gamma + 1), dtype=torch.int32, device=dev)
    wa, wr = sv.Workspace(), sv.Workspace()

    def step():
        sv.spec_verify_attention(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["lens"], hint,
                                 out=out, workspace=wa)
        sv.spec_reject_sample(u["target_logits"], u["draft_logits"], u["draft_tokens"], u["uniforms"], T,
                              n_accepted=n, out_tokens=tok, workspace=wr)
        sv.spec_kv_truncate(t["lens"], n, cfg.n_q)

    step()  # eager: sizes the workspaces, loads the library
    torch.cuda.synchronize()
    want = (out.clone(), n.clone(), tok.clone(), t["lens"].clone())
    t["lens"].copy_(lens0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        t["lens"].copy_(lens0)
        out.zero_()
        tok.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (out, n, tok, t["lens"])
        for w_, g_ in zip(want, got):
            assert torch.equal(w_, g_), f"replay {rep} differs from the eager step"
        t["lens"].copy_(lens0)
        step()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_sampler_large_batch_graph_replays_match_eager(T):
    """The sampler at a batch above 65,536 row segments (its large-batch launch
    shape) and greedy verification, captured and replayed."""
    B = 100
    _case("sampler-graph", config=4, B=B, T=T)
    dev = torch.device("cuda:0")
    cfg = W.get(4)
    s = W.sampler_inputs(cfg, B=B, temperature=1.0)
    u = {k: to_dev(v, dev) for k, v in s.items() if k != "temperature"}
    if T == 0.0:
        u["draft_tokens"] = torch.argmax(u["draft_logits"].float(), dim=-1).to(torch.int32)
    n = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty((B, cfg.gamma + 1), dtype=torch.int32, device=dev)
    p = torch.empty((B, cfg.gamma), dtype=torch.float32, device=dev)
    q = torch.empty((B, cfg.gamma), dtype=torch.float32, device=dev)
    ws = sv.Workspace()

    def call():
        sv.spec_reject_sample(u["target_logits"], None if T == 0.0 else u["draft_logits"], u["draft_tokens"],
                              None if T == 0.0 else u["uniforms"], T, n_accepted=n, out_tokens=tok, p_draft=p,
                              q_draft=q, workspace=ws)

    call()
    torch.cuda.synchronize()
    want = (n.clone(), tok.clone(), p.clone(), q.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        n.fill_(-9)
        tok.fill_(-7)
        p.zero_()
        q.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for w_, g_ in zip(want, (n, tok, p, q)):
            assert torch.equal(w_.view(torch.int32), g_.view(torch.int32)), f"replay {rep} differs from the eager call"
        call()  # eager work between replays
        torch.cuda.synchronize()


def test_speculative_round_graph_replays_match_eager():
    _case("round-graph", B=4, gamma=4)
    dev = torch.device("cuda:0")
    ct, cd = M.TARGET, M.DRAFT
    pt = torch.from_numpy(gen.model_params(M.param_shapes(ct), 60)).to(dev)
    pd = torch.from_numpy(gen.model_params(M.param_shapes(cd), 61)).to(dev)
    B, gamma, L0, max_len, max_T = 4, 4, 40, 64, 64
    r = np.random.default_rng(62)
    ti = gen.forward_inputs(ct.V, ct.L, ct.H, ct.D, B, 1, (0, 0), max_T, 63)
    di = gen.forward_inputs(cd.V, cd.L, cd.H, cd.D, B, 1, (0, 0), max_T, 64)
    base = {
        "seq": torch.from_numpy(r.integers(0, ct.V, size=(B, max_len)).astype(np.int32)).to(dev),
        "seq_len": torch.full((B,), L0, dtype=torch.int32, device=dev),
        "tkv": torch.from_numpy(ti["kv"]).to(dev),
        "tlen": torch.full((B,), L0 - 1, dtype=torch.int32, device=dev),
        "dkv": torch.from_numpy(di["kv"]).to(dev),
        "dlen": torch.full((B,), L0 - 2, dtype=torch.int32, device=dev),
    }
    st = {k: v.clone() for k, v in base.items()}
    ud = torch.from_numpy(r.random((B, gamma))).to(dev)
    uv = torch.from_numpy(r.random((B, gamma + 1))).to(dev)
    n = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    ws = sv.Workspace()

    def reset():
        for k in base:
            st[k].copy_(base[k])

    def one():
        sv.spec_speculative_round(ct, pt, cd, pd, st["seq"], st["seq_len"], st["tkv"], st["tlen"], st["dkv"],
                                  st["dlen"], ud, uv, 1.0, L0, n_accepted=n, out_tokens=tok, workspace=ws)

    one()
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in st.items()}
    want_n, want_tok = n.clone(), tok.clone()
    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one()
    for rep in range(3):
        reset()
        n.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(n, want_n) and torch.equal(tok, want_tok), f"replay {rep}: tokens differ"
        for k in want:
            assert torch.equal(st[k], want[k]), f"replay {rep}: {k} differs"
        reset()
        one()  # eager work between replays
        torch.cuda.synchronize()
    print(f"n_accepted {n.cpu().tolist()}", flush=True)


def test_merging_attention_graph_replays_match_eager():
    """Long shares: the launch that zeroes the per-slab counters and the
    stream launch that merges each slab's pieces, replayed from one graph."""
    cfg = W.Config(95, "merge", B=20, gamma=8, V=1, dtype="bf16", Hq=64, Hkv=8, D=128, L=(8192, 32768),
                   max_T=32800)
    hint = 32768
    _case("merge-graph", B=cfg.B, hint=hint)
    d = W.attention_inputs_device(cfg, "cuda")
    d["lens"][3] = hint + 1  # a rejected length: NaN rows from the counter launch
    out = torch.empty_like(d["q"])
    wa = sv.Workspace()

    def call():
        sv.spec_verify_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["lens"], hint,
                                 out=out, workspace=wa)

    call()
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {rep} differs from the eager call"
        call()  # eager work between replays
        torch.cuda.synchronize()
