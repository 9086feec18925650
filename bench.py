"""Benchmark of the verification step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5|c4|c3|model]
                    [--temperature T] [--kv bf16|f16|int8] [--paged 16|32]
                    [--page-order random|sequential] [--no-cpu-baseline] [--no-extras]
                    [--copy-calibration]

A step is one pass of the whole hot path on one batch: verify attention with
KV append, rejection sampling, length reset (three C-ABI calls on one
stream).  Inputs are synthetic, seeded and already resident in HBM.  The
default workload is the long-context large-batch configuration (B=256,
gamma=8, GQA 64/8, head dim 128, bf16 cache with lengths uniform in
[8192, 32768], vocabulary 128,256).  Lengths are restored before each step
(a 1 KB device copy) so every step verifies the same batch.

Prints one JSON line: verified draft positions per second for the whole step
(K steps between two events), per-call durations measured with HIP events on
the launch stream in a second loop and back to back, the achieved fraction of
the HBM roofline for each part, and the CPU oracle timed on a bounded sample
of the same workload (one thread, and on all host cores).  At the default
workload the line also carries config 5's sampler at T = 0.7 and config 4's
step (``--no-extras`` leaves them out).
"""

import argparse
import contextlib
import gc
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense
MFMA_F32_PEAK_TFLOPS = 157.3
METRIC = "verified draft positions/sec + % of MI355X HBM peak (sampler, verify attn)"

WORKLOADS = {"c3": 3, "c4": 4, "c5": 5}

# Sources of the verify-attention kernels; the HBM byte counts stored under
# profiles/ are used only while their code is unchanged.
ATTN_SOURCES = (
    "speculative_decoding_verification_spec_amd/csrc/attention.hip",
    "speculative_decoding_verification_spec_amd/csrc/spec_common.h",
)


def attn_source_hash():
    """Hash of the sources' code: every line with its // comment and trailing
    blanks removed, blank lines dropped (an edit to comments alone keeps it)."""
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(cid):
    """HBM bytes per spec_verify_attention call from the rocprofv3 byte counters.

    profiles/verify_attention_config<cid>.hbm_traffic.md carries one JSON line
    (FETCH_SIZE and WRITE_SIZE per call, each scaled by what the counter reads
    for a plain device copy of known size).  None when the file is missing or
    was taken from other kernel sources.
    """
    path = os.path.join(ROOT, "profiles", f"verify_attention_config{cid}.hbm_traffic.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith('{"hbm_traffic"'):
                d = json.loads(line)["hbm_traffic"]
                if d.get("source_sha256") == attn_source_hash():
                    return d
    return None


@contextlib.contextmanager
def no_gc():
    """Python's cyclic garbage collector off inside a timed region.  A full
    collection inside one stalls the launching thread for tens of
    milliseconds while the GPU runs dry behind it: measured, a step loop's
    launches took 43.7 ms of host time instead of 2.2 ms and the loop 44 ms
    longer on the GPU.  No collection is forced before the region: one
    forced there was followed by slower kernels in the region (attention
    3.35 against 3.29 ms per call, same box and inputs)."""
    was = gc.isenabled()
    gc.disable()
    try:
        yield
    finally:
        if was:
            gc.enable()


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence.

    Recording a default event (torch.cuda.Event) also performs a system-scope
    release: a cache write-back and invalidate that costs the stream a few
    microseconds per record and is charged to the calls between events.  This
    event only writes its timestamp once the work before it on the stream is
    done.  The HIP runtime is the one torch has loaded (found by its path in
    the process's mappings), so torch's streams are valid handles.  Read it
    only after torch.cuda.synchronize().
    """

    _hip = None
    _DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes

            with open("/proc/self/maps") as f:
                paths = sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln and ln.split()[-1].startswith("/")})
            if len(paths) != 1:
                raise RuntimeError(f"expected one HIP runtime mapped in this process, found {paths}")
            hip = ctypes.CDLL(paths[0])
            vp = ctypes.c_void_p
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [vp, vp]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            hip.hipEventDestroy.argtypes = [vp]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes

        self._ev = ctypes.c_void_p()
        if self._lib().hipEventCreateWithFlags(ctypes.byref(self._ev), self._DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if self._lib().hipEventRecord(self._ev, stream.cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        import ctypes

        ms = ctypes.c_float()
        if self._lib().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._hip is not None and self._ev:
            self._hip.hipEventDestroy(self._ev)


def algorithmic(cfg, lens, B, greedy=False, kv="bf16"):
    """Bytes and flops the step must move / compute (every input read once).

    Greedy verification (T = 0) reads only the gamma+1 target rows and no uniforms.
    """
    e = cfg.elem_bytes
    n, D = cfg.n_q, cfg.D
    L = lens.astype(np.int64)
    if kv == "int8":  # cached rows: D int8 values + one fp16 scale; new rows read in bf16
        kv_read = int(np.sum(2 * cfg.Hkv * (D + 2) * L) + B * 2 * cfg.Hkv * n * D * e)
        append = int(B * 2 * cfg.Hkv * n * (D + 2))
    else:
        kv_read = int(np.sum(2 * cfg.Hkv * D * e * (L + n)))
        append = int(B * 2 * cfg.Hkv * n * D * e)
    q_o = int(B * 2 * cfg.Hq * n * D * e)
    att_bytes = kv_read + append + q_o
    att_flops = int(4 * cfg.Hq * D * np.sum(n * L + n * (n + 1) // 2))
    g = cfg.gamma
    if greedy:
        smp_bytes = int(B * (g + 1) * cfg.V * e + B * (g * 4 + 4 + (g + 1) * 4 + 8 * g))
    else:
        smp_bytes = int(B * (2 * g + 1) * cfg.V * e + B * (g * 4 + (g + 1) * 8 + 4 + (g + 1) * 4 + 8 * g))
    return att_bytes, att_flops, smp_bytes


def paginate(att, cfg, hint, page, rep, order="random"):
    """Paged copies of the caches: [Hkv, num_pages, page, D] plus the block table.

    order "random": pages at seeded random slots; "sequential": each sequence's
    pages in order, sequences one after another.
    """
    import torch

    lens = att["lens"].cpu().numpy().astype(np.int64)
    need = -(-(lens + cfg.n_q) // page)
    max_blocks = -(-(hint + cfg.n_q) // page)
    num_pages = int(need.sum())
    g = torch.Generator(device="cpu").manual_seed(7919 * cfg.cid + rep)
    perm = (torch.randperm(num_pages, generator=g) if order == "random" else torch.arange(num_pages)).to(torch.int32)
    table = torch.full((cfg.B, max_blocks), -1, dtype=torch.int32)
    off = 0
    for b in range(cfg.B):
        table[b, : need[b]] = perm[off : off + need[b]]
        off += int(need[b])
    table = table.to(att["k_cache"].device)
    out = {}
    for name in ("k_cache", "v_cache"):
        c = att[name]
        pages = torch.empty((cfg.Hkv, num_pages, page, cfg.D), dtype=c.dtype, device=c.device)
        for b in range(cfg.B):
            nb = int(need[b])
            rows = min(nb * page, c.shape[2])
            blk = torch.zeros((cfg.Hkv, nb * page, cfg.D), dtype=c.dtype, device=c.device)
            blk[:, :rows] = c[b, :, :rows]
            pages[:, table[b, :nb].long()] = blk.view(cfg.Hkv, nb, page, cfg.D)
        out[name.replace("cache", "pages")] = pages
    out["table"] = table
    return out


def quantized_cache(att, cfg, rep):
    """int8 caches and fp16 scales drawn on the device with the recipe of
    ``workloads.attention_inputs_int8`` (input generation only)."""
    import workloads as W

    d = W.attention_inputs_int8_device(cfg, att["q"].device, rep=rep)
    return {"k_q": d["k_cache"], "k_scale": d["k_scale"], "v_q": d["v_cache"], "v_scale": d["v_scale"]}


def make_inputs(cfg, device, temperature, rep):
    import torch

    import workloads as W

    t_gen = temperature if temperature > 0 else 1.0  # greedy: drafts are the draft model's argmax
    if cfg.cid == 5:
        att = W.attention_inputs_device(cfg, device, rep=rep)
        smp = W.sampler_inputs_device(cfg, device, temperature=t_gen, rep=rep)
    else:
        from workloads.device import to_dev

        a = W.attention_inputs(cfg, rep=rep)
        s = W.sampler_inputs(cfg, temperature=t_gen, rep=rep)
        att = {k: to_dev(v, device=device) for k, v in a.items()}
        smp = {k: (to_dev(v, device=device) if k != "temperature" else v) for k, v in s.items()}
    if temperature == 0:
        smp["draft_tokens"] = torch.argmax(smp["draft_logits"].float(), dim=-1).to(torch.int32)
        smp["temperature"] = 0.0
    att["lens_base"] = att["lens"].clone()
    att["out"] = torch.empty_like(att["q"])
    smp["n"] = torch.empty(cfg.B, dtype=torch.int32, device=device)
    smp["tok"] = torch.empty((cfg.B, cfg.gamma + 1), dtype=torch.int32, device=device)
    torch.cuda.synchronize()
    return att, smp


def cpu_baseline(cfg, att, smp, temperature, budget_s=12.0):
    """The oracle as it stands, on whole sequences of the workload, one BLAS thread."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as A
    from oracle import greedy as Gr
    from oracle import paged as Pg
    from oracle import quant as Qn
    from oracle import sampler as S
    from workloads.device import to_host

    B = att["q"].shape[0]
    order = np.random.default_rng(0).permutation(B)
    done, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1):
        for b in order:
            sl = slice(int(b), int(b) + 1)
            L = int(att["lens_base"][sl].item())
            host = {k: to_host(att[k][sl]) for k in ("q", "k_new", "v_new")}
            if "k_q" in att:
                kq, ks = to_host(att["k_q"][sl, :, :L]), to_host(att["k_scale"][sl, :, :L])
                vq, vs = to_host(att["v_q"][sl, :, :L]), to_host(att["v_scale"][sl, :, :L])
                s0 = time.perf_counter()
                Qn.verify_attention_int8(host["q"], host["k_new"], host["v_new"], kq, ks, vq, vs, np.array([L]))
            elif "k_pages" in att:  # this sequence's pages, renumbered 0..nb-1
                page = att["k_pages"].shape[2]
                nb = -(-L // page)
                rows = att["table"][b, :nb].long()
                kp, vp = to_host(att["k_pages"][:, rows]), to_host(att["v_pages"][:, rows])
                tab = np.arange(nb, dtype=np.int32)[None]
                s0 = time.perf_counter()
                Pg.verify_attention_paged(host["q"], host["k_new"], host["v_new"], kp, vp, tab, np.array([L]))
            else:
                host["k_cache"] = to_host(att["k_cache"][sl, :, :L])
                host["v_cache"] = to_host(att["v_cache"][sl, :, :L])
                s0 = time.perf_counter()
                A.verify_attention(host["q"], host["k_new"], host["v_new"], host["k_cache"], host["v_cache"],
                                   np.array([L]))
            t_att = time.perf_counter() - s0
            sh = {k: to_host(smp[k][sl]) for k in ("target_logits", "draft_logits", "draft_tokens", "uniforms")}
            s1 = time.perf_counter()
            if temperature == 0:
                Gr.verify_batch(sh["target_logits"], sh["draft_tokens"])
            else:
                S.verify_batch(sh["target_logits"], sh["draft_logits"], sh["draft_tokens"], sh["uniforms"],
                               temperature)
            t_smp = time.perf_counter() - s1
            done += 1
            if done == 1:
                elapsed = t_att + t_smp
            else:
                elapsed += t_att + t_smp
            if time.perf_counter() - t0 > budget_s:
                break
    pos = done * cfg.gamma
    return {
        "value": pos / elapsed,
        "unit": "positions/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} whole sequences of the workload (attention over their full cache + "
        + (f"greedy verification over the {cfg.gamma + 1} target rows" if temperature == 0 else
           f"sampler over all {2 * cfg.gamma + 1} vocab rows")
        + "), numpy fp64, one BLAS thread; host copies excluded from the time",
        "seconds": elapsed,
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_worker(job):
    """One worker of the all-core oracle leg: draws whole sequences of the
    workload with the host generators (seeded by worker and count) and times
    the oracle on each (attention over the full cache, then the sampler over
    all vocabulary rows, or greedy verification at T = 0), one BLAS thread,
    until ``budget_s`` of oracle time.  Returns (positions, oracle seconds)."""
    cid, temperature, worker, budget_s = job
    from threadpoolctl import threadpool_limits

    import workloads as W
    from oracle import attention as A
    from oracle import greedy as Gr
    from oracle import sampler as S

    cfg = W.get(cid)
    pos, spent, i = 0, 0.0, 0
    with threadpool_limits(limits=1):
        while spent < budget_s:
            rep = 1000 + 100 * worker + i
            i += 1
            att = W.attention_inputs(cfg, rep=rep, B=1)
            L = int(att["lens"][0])
            smp = W.sampler_inputs(cfg, temperature=temperature if temperature > 0 else 1.0, rep=rep, B=1)
            kc, vc = att["k_cache"][:, :, :L], att["v_cache"][:, :, :L]
            t0 = time.perf_counter()
            A.verify_attention(att["q"], att["k_new"], att["v_new"], kc, vc, att["lens"])
            if temperature == 0:
                Gr.verify_batch(smp["target_logits"], smp["draft_tokens"])
            else:
                S.verify_batch(smp["target_logits"], smp["draft_logits"], smp["draft_tokens"], smp["uniforms"],
                               temperature)
            spent += time.perf_counter() - t0
            pos += cfg.gamma
    return pos, spent


def all_core_baseline(pool, workers, cid, temperature, budget_s=4.0):
    """The oracle on every worker of ``pool`` at once (each on its own
    sequences): the summed rate of the workers."""
    t0 = time.perf_counter()
    res = pool.map(_oracle_worker, [(cid, temperature, w, budget_s) for w in range(workers)])
    wall = time.perf_counter() - t0
    return {
        "value": sum(p / t for p, t in res if t > 0),
        "unit": "positions/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{workers} processes at once, each timing the oracle for about {budget_s:g} s on whole sequences "
                  "of the workload drawn with the host generators (attention over the full cache + "
                  + ("greedy verification" if temperature == 0 else "sampler over every vocabulary row")
                  + "), numpy fp64, one BLAS thread each; the value sums the processes' rates; drawing the "
                  "inputs is not timed",
        "sequences": int(sum(p for p, _ in res) // W_GAMMA.get(cid, 1)),
        "wall_s": wall,
    }


W_GAMMA = {3: 4, 4: 4, 5: 8}


def copy_ceiling(torch, nbytes=2 << 30, reps=5):
    """Achieved HBM bytes/s of a plain 2 GiB device-to-device copy (read + write).

    A practical ceiling beside the 8 TB/s specification peak: the fraction
    of it that the path's kernels reach is reported too.
    """
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with no_gc():
        e0.record()
        for _ in range(reps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"GB/s": gbs, "what": "torch device-to-device copy of 2 GiB, bytes read + written per second"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c5", choices=sorted(WORKLOADS) + ["model"],
                    help="a config of the verification step, or 'model': the pages' char models "
                         "(verify forward and whole speculative rounds, random weights)")
    ap.add_argument("--temperature", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--paged", type=int, default=0, choices=(0, 16, 32),
                    help="run attention over a paged copy of the cache with this page size")
    ap.add_argument("--page-order", default="random", choices=("random", "sequential"),
                    help="where the pages sit: seeded random slots, or in sequence order")
    ap.add_argument("--kv", default="bf16", choices=("bf16", "f16", "int8"),
                    help="cache storage: the workload's bf16, the same values in fp16, or int8 codes with an fp16 scale per row")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB device buffer 5 times (reference for HBM byte counters)")
    ap.add_argument("--no-extras", action="store_true",
                    help="at the default workload, skip the other measured points (config 5's sampler at T=0.7 "
                         "and config 4's step)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the verification step has no multi-GPU "
              "path; sharded, each GPU would own B/N sequences and run the same calls with no exchange.",
              file=sys.stderr)
        sys.exit(2)
    # The all-core oracle leg's worker processes are forked now, before this
    # process touches the GPU, and never use it.
    pool, workers = None, 0
    if not args.no_cpu_baseline and args.workload != "model" and not args.copy_calibration:
        import multiprocessing as mp

        workers = max(1, min(16, os.cpu_count() or 1))
        pool = mp.get_context("fork").Pool(workers)

    import torch

    import speculative_decoding_verification_spec_amd as sv
    import workloads as W

    if args.copy_calibration:
        # A plain device-to-device copy of known size: its FETCH_SIZE / WRITE_SIZE
        # per launch is the scale for the byte counters of the path's kernels.
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}))
        return

    if not os.path.exists(sv.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    sv.load()
    dev = torch.device("cuda:0")
    if args.workload == "model":
        model_bench(args, torch, sv, dev)
        return
    cfg = W.get(WORKLOADS[args.workload])
    T = cfg.temperatures[-1] if args.temperature is None else args.temperature
    extras = (not args.no_extras and cfg.cid == 5 and T == 1.0 and args.kv == "bf16" and not args.paged)
    print(f"[bench] workload config{cfg.cid} ({cfg.name}) T={T}: generating inputs", file=sys.stderr, flush=True)
    sets = input_sets(cfg, dev, T)
    nsets = len(sets)
    hint = cfg.L[1]
    if args.kv == "int8":
        if args.paged or cfg.dtype != "bf16":
            print("--kv int8 needs a contiguous cache and bf16 activations", file=sys.stderr)
            sys.exit(2)
        for rep, (att, _) in enumerate(sets):
            att.update(quantized_cache(att, cfg, rep))
            del att["k_cache"], att["v_cache"]
        torch.cuda.empty_cache()
    if args.kv == "f16":  # the same values (bf16 ones are exact in fp16), in IEEE half
        if args.paged or cfg.dtype != "bf16":
            print("--kv f16 needs a contiguous cache and a bf16 workload", file=sys.stderr)
            sys.exit(2)
        for att, _ in sets:
            for k in ("q", "k_new", "v_new", "k_cache", "v_cache", "out"):
                att[k] = att[k].to(torch.float16)
        torch.cuda.empty_cache()
    if args.paged:
        for rep, (att, _) in enumerate(sets):
            att.update(paginate(att, cfg, hint, args.paged, rep, args.page_order))
            del att["k_cache"], att["v_cache"]  # the paged copies are the cache now
        torch.cuda.empty_cache()
    B = cfg.B
    t = time_steps(torch, sv, cfg, T, sets, hint, args.steps, args.warmup, kv=args.kv, paged=args.paged)
    ms_step, att_ms, smp_ms, trn_ms = t["ms_step"], t["att_ms"], t["smp_ms"], t["trn_ms"]
    b2b_ms = attention_back_to_back(torch, sv, sets, hint, min(args.steps, 20), kv=args.kv, paged=args.paged)
    s2s_ms = sampler_back_to_back(torch, sv, sets[0][1], T, args.steps)

    # Algorithmic bytes per call, averaged over the rotated input sets (their
    # lengths differ); set k is used by steps k, k + nsets, ...
    per_set = [algorithmic(cfg, st[0]["lens_base"].cpu().numpy(), B, greedy=(T == 0), kv=args.kv) for st in sets]
    counts = [len(range(k, args.steps, nsets)) for k in range(nsets)]
    att_b = sum(c * a[0] for c, a in zip(counts, per_set)) / args.steps
    att_f = sum(c * a[1] for c, a in zip(counts, per_set)) / args.steps
    smp_b = per_set[0][2]
    att_gbs = att_b / (att_ms * 1e-3) / 1e9
    smp_gbs = smp_b / (smp_ms * 1e-3) / 1e9
    positions = B * cfg.gamma
    n_last = sets[(args.steps - 1) % nsets][1]["n"].cpu().numpy()
    traffic = measured_traffic(cfg.cid) if (not args.paged and args.kv == "bf16") else None
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS

    res = {
        "metric": METRIC,
        "value": positions / (ms_step * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"config{cfg.cid} {cfg.name}: B={B} gamma={cfg.gamma} GQA {cfg.Hq}/{cfg.Hkv} D={cfg.D} "
            f"{cfg.dtype} KV, lengths U[{cfg.L[0]},{cfg.L[1]}], vocab {cfg.V}, T={T}",
            "batch": B,
            "gamma": cfg.gamma,
            "temperature": T,
            "input_sets": nsets,
            "kv_cache": (f"paged, {args.paged}-position pages at {args.page_order} slots" if args.paged
                         else "int8 codes + fp16 row scales, contiguous" if args.kv == "int8" else "contiguous"),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": att_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": att_gbs / HBM_PEAK_GBS,
            "traffic": None if traffic is None else traffic["bytes_per_call"],
            "kernel": ("spec_verify_attention_int8: quant_new_rows + attn_stream_i8w with attn_combine_i8 or, for long shares, attn_stream_prep and attn_exact_i8, one call"
                       if args.kv == "int8" else
                       "spec_verify_attention: attn_stream_bf16 with attn_combine_stream or, for long shares, "
                       "attn_stream_prep, one call"
                       if cfg.dtype == "bf16" and cfg.B <= 1024
                       else f"spec_verify_attention: attn_split_{cfg.dtype} (+ attn_combine past 8 splits), one call"),
            "algorithmic_bytes": att_b,
            "avg_ms": att_ms,
        },
        "parts": {
            "attention": {"ms": att_ms, "bytes": att_b, "GB/s": att_gbs, "hbm_frac": att_gbs / HBM_PEAK_GBS,
                          "positions/s": positions / (att_ms * 1e-3), "flops": att_f,
                          "mfma_frac": att_f / (att_ms * 1e-3) / (mfma_peak * 1e12),
                          "back_to_back": {"ms": b2b_ms,
                                           "hbm_frac": sum(a[0] for a in per_set) / len(per_set) / (b2b_ms * 1e-3) / 8e12,
                                           "calls": min(args.steps, 20)}},
            "sampler": {"ms": smp_ms, "bytes": smp_b, "GB/s": smp_gbs, "hbm_frac": smp_gbs / HBM_PEAK_GBS,
                        "positions/s": positions / (smp_ms * 1e-3),
                        "back_to_back": {"ms": s2s_ms, "hbm_frac": smp_b / (s2s_ms * 1e-3) / 8e12,
                                         "calls": args.steps}},
            "truncate": {"ms": trn_ms},
            "step_with_part_events_ms": t["ms_step_with_part_events"],
            "mean_accepted": float(n_last.mean()),
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        att0, smp0 = sets[0]
        cb = cpu_baseline(cfg, att0, smp0, T)
        cb["cpu_model"] = cpu_model()
        cb["os_cpu_count"] = os.cpu_count()
        del att0, smp0
    del sets
    torch.cuda.empty_cache()
    if extras:
        # The other points the targets are set on, measured in the same run:
        # config 5's sampler at its other temperature, and config 4's step.
        res["sampler_c5_T0.7"] = sampler_only(torch, sv, cfg, 0.7, dev, args.steps, args.warmup)
        res["parts_c4"] = step_parts(torch, sv, W.get(4), dev, max(args.steps, 50), max(args.warmup, 10))
    res["copy_ceiling"] = copy_ceiling(torch)
    if not args.no_cpu_baseline:
        if pool is not None:
            print(f"[bench] timing the CPU oracle on {workers} processes", file=sys.stderr, flush=True)
            cb["all_cores"] = all_core_baseline(pool, workers, cfg.cid, T)
        res["cpu_baseline"] = cb
    if pool is not None:
        pool.close()
        pool.join()
    print(json.dumps(res), flush=True)


def time_steps(torch, sv, cfg, T, sets, hint, steps, warmup, kv="bf16", paged=0):
    """Warm up, then time ``steps`` verification steps between two events on
    the launch stream (the step time), then ``steps`` more with per-call
    timing events (TimingEvent: no system-scope fence) around attention, the
    sampler and the length reset (the parts; even so each event costs the
    stream a little, so they stay out of the step time).  Step k uses input
    set k mod len(sets); lengths are restored before each step (a 1 KB device
    copy, inside the step time and outside the per-call events)."""
    nsets = len(sets)
    stream = torch.cuda.current_stream()
    ev = [[TimingEvent() for _ in range(4)] for _ in range(steps)]

    def step(k, events=None):
        att, smp = sets[k % nsets]
        att["lens"].copy_(att["lens_base"])
        if events:
            events[0].record(stream)
        if kv == "int8":
            sv.spec_verify_attention_int8(att["q"], att["k_new"], att["v_new"], att["k_q"], att["k_scale"],
                                          att["v_q"], att["v_scale"], att["lens"], hint, out=att["out"])
        elif paged:
            sv.spec_verify_attention_paged(att["q"], att["k_new"], att["v_new"], att["k_pages"], att["v_pages"],
                                           att["table"], att["lens"], hint, out=att["out"])
        else:
            sv.spec_verify_attention(att["q"], att["k_new"], att["v_new"], att["k_cache"], att["v_cache"],
                                     att["lens"], hint, out=att["out"])
        if events:
            events[1].record(stream)
        greedy = T == 0
        n, tok, _, _ = sv.spec_reject_sample(smp["target_logits"], None if greedy else smp["draft_logits"],
                                             smp["draft_tokens"], None if greedy else smp["uniforms"], T,
                                             n_accepted=smp["n"], out_tokens=smp["tok"])
        if events:
            events[2].record(stream)
        sv.spec_kv_truncate(att["lens"], n, cfg.n_q)
        if events:
            events[3].record(stream)
        return n

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    print(f"[bench] config{cfg.cid}: warmup {warmup} done; timing {steps} steps", file=sys.stderr, flush=True)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with no_gc():
        t_start.record(stream)
        for k in range(steps):
            step(k)
        t_end.record(stream)
        torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / steps
    with no_gc():
        t_start.record(stream)
        for k in range(steps):
            step(k, ev[k])
        t_end.record(stream)
        torch.cuda.synchronize()
    return {"ms_step": ms_step, "ms_step_with_part_events": t_start.elapsed_time(t_end) / steps,
            "att_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in ev])),
            "smp_ms": float(np.mean([e[1].elapsed_time(e[2]) for e in ev])),
            "trn_ms": float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))}


def input_sets(cfg, dev, T):
    """Enough input sets that a step's bytes exceed the 256 MB last-level cache."""
    att_bytes_est = cfg.B * 2 * cfg.Hkv * cfg.D * cfg.elem_bytes * (sum(cfg.L) / 2 + cfg.n_q)
    smp_bytes_est = cfg.B * (2 * cfg.gamma + 1) * cfg.V * cfg.elem_bytes
    nsets = max(1, min(4, math.ceil(768e6 / (att_bytes_est + smp_bytes_est))))
    return [make_inputs(cfg, dev, T, rep) for rep in range(nsets)]


def sampler_only(torch, sv, cfg, T, dev, steps, warmup):
    """spec_reject_sample alone at temperature T over one batch of the
    workload's logits (drafts drawn at T), timed with events per call."""
    import workloads as W

    print(f"[bench] config{cfg.cid} sampler at T={T}", file=sys.stderr, flush=True)
    smp = W.sampler_inputs_device(cfg, dev, temperature=T)
    n = torch.empty(cfg.B, dtype=torch.int32, device=dev)
    tok = torch.empty((cfg.B, cfg.gamma + 1), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        sv.spec_reject_sample(smp["target_logits"], smp["draft_logits"], smp["draft_tokens"], smp["uniforms"], T,
                              n_accepted=n, out_tokens=tok)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
    with no_gc():
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    nbytes = algorithmic(cfg, np.zeros(cfg.B), cfg.B)[2]
    smp["n"], smp["tok"] = n, tok
    b2b = sampler_back_to_back(torch, sv, smp, T, steps)
    del smp
    torch.cuda.empty_cache()
    return {"ms": ms, "bytes": nbytes, "GB/s": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "positions/s": cfg.B * cfg.gamma / (ms * 1e-3), "mean_accepted": float(n.float().mean().item()),
            "back_to_back": {"ms": b2b, "hbm_frac": nbytes / (b2b * 1e-3) / 1e9 / HBM_PEAK_GBS, "calls": steps}}


def attention_back_to_back(torch, sv, sets, hint, calls, kv="bf16", paged=0):
    """Milliseconds per attention call when ``calls`` calls run back to back
    (input sets alternating) between two events on the launch stream: the
    call's own throughput, without the per-call events of the step loop
    (each of which costs the stream a little).  Lengths are left as they
    are, so every call appends the same rows again."""
    stream = torch.cuda.current_stream()
    for att, _ in sets:
        att["lens"].copy_(att["lens_base"])

    def call(att):
        if kv == "int8":
            sv.spec_verify_attention_int8(att["q"], att["k_new"], att["v_new"], att["k_q"], att["k_scale"],
                                          att["v_q"], att["v_scale"], att["lens"], hint, out=att["out"])
        elif paged:
            sv.spec_verify_attention_paged(att["q"], att["k_new"], att["v_new"], att["k_pages"], att["v_pages"],
                                           att["table"], att["lens"], hint, out=att["out"])
        else:
            sv.spec_verify_attention(att["q"], att["k_new"], att["v_new"], att["k_cache"], att["v_cache"],
                                     att["lens"], hint, out=att["out"])

    for k in range(len(sets)):
        call(sets[k][0])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with no_gc():
        e0.record(stream)
        for k in range(calls):
            call(sets[k % len(sets)][0])
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / calls


def sampler_back_to_back(torch, sv, smp, T, calls):
    """Milliseconds per spec_reject_sample call, ``calls`` calls back to back
    between two events on the launch stream (outputs overwritten).  When one
    call's logits are smaller than three times the 256 MB memory-side cache,
    the calls cycle through copies of them in separate buffers (at most 8),
    so that a call does not find the previous call's rows still cached."""
    stream = torch.cuda.current_stream()
    greedy = T == 0
    keys = ("target_logits",) if greedy else ("target_logits", "draft_logits")
    nbytes = sum(smp[k].numel() * smp[k].element_size() for k in keys)
    copies = [smp] + [{**smp, **{k: smp[k].clone() for k in keys}}
                      for _ in range(max(1, min(8, math.ceil(768e6 / nbytes))) - 1)]

    def call(c):
        sv.spec_reject_sample(c["target_logits"], None if greedy else c["draft_logits"], c["draft_tokens"],
                              None if greedy else c["uniforms"], T, n_accepted=c["n"], out_tokens=c["tok"])

    for c in copies:
        call(c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with no_gc():
        e0.record(stream)
        for k in range(calls):
            call(copies[k % len(copies)])
        e1.record(stream)
        torch.cuda.synchronize()
    del copies
    return e0.elapsed_time(e1) / calls


def step_parts(torch, sv, cfg, dev, steps, warmup):
    """The whole step at another configuration (its first temperature):
    per-call event times and HBM fractions of attention and the sampler."""
    T = cfg.temperatures[-1]
    print(f"[bench] config{cfg.cid}: generating inputs", file=sys.stderr, flush=True)
    sets = input_sets(cfg, dev, T)
    t = time_steps(torch, sv, cfg, T, sets, cfg.L[1], steps, warmup)
    per_set = [algorithmic(cfg, st[0]["lens_base"].cpu().numpy(), cfg.B) for st in sets]
    counts = [len(range(k, steps, len(sets))) for k in range(len(sets))]
    att_b = sum(c * a[0] for c, a in zip(counts, per_set)) / steps
    b2b = attention_back_to_back(torch, sv, sets, cfg.L[1], steps)
    b2b_b = sum(a[0] for a in per_set) / len(per_set)
    s2s = sampler_back_to_back(torch, sv, sets[0][1], T, steps)
    smp_b = per_set[0][2]
    pos = cfg.B * cfg.gamma
    out = {"workload": f"config{cfg.cid} {cfg.name}: B={cfg.B} gamma={cfg.gamma} GQA {cfg.Hq}/{cfg.Hkv} "
                       f"D={cfg.D} {cfg.dtype} KV, lengths U[{cfg.L[0]},{cfg.L[1]}], vocab {cfg.V}, T={T}",
           "steps": steps, "input_sets": len(sets), "ms_per_step": t["ms_step"],
           "positions/s": pos / (t["ms_step"] * 1e-3),
           "attention": {"ms": t["att_ms"], "bytes": att_b, "hbm_frac": att_b / (t["att_ms"] * 1e-3) / 8e12,
                         "positions/s": pos / (t["att_ms"] * 1e-3),
                         "back_to_back": {"ms": b2b, "hbm_frac": b2b_b / (b2b * 1e-3) / 8e12,
                                          "calls": steps}},
           "sampler": {"ms": t["smp_ms"], "bytes": smp_b, "hbm_frac": smp_b / (t["smp_ms"] * 1e-3) / 8e12,
                       "positions/s": pos / (t["smp_ms"] * 1e-3),
                       "back_to_back": {"ms": s2s, "hbm_frac": smp_b / (s2s * 1e-3) / 8e12, "calls": steps}},
           "truncate": {"ms": t["trn_ms"]}}
    del sets
    torch.cuda.empty_cache()
    return out


def model_bench(args, torch, sv, dev):
    """The pages' char models with random weights ([P2] section
    numpyで小さなTransformerを自作する: target V=96 C=96 L=4 H=4, draft C=48 L=1
    H=2, 512 positions), B=64 sequences with 384 cached tokens, gamma=4, T=1:
      * the target's verify forward over gamma+1 tokens (spec_verify_forward);
      * whole speculative rounds (spec_speculative_round), generated tokens/s,
        against target-only decoding (one forward of one token per sequence
        per generated token; its draw is left out, which favours the
        baseline);
    all inputs resident on the device.  Random weights make the draft a poor
    guesser, so the acceptance rate (and the round's gain) is low; the numbers
    measure the machinery, not a trained draft."""
    from workloads import gen

    tcfg = dict(V=96, C=96, L=4, H=4, T=512)
    dcfg = dict(V=96, C=48, L=1, H=2, T=512)
    B, gamma, prefix, T, max_T = 64, 4, 384, 1.0, 512
    pt = torch.from_numpy(gen.model_params(sv.model_param_layout(tcfg), 40)).to(dev)
    pd = torch.from_numpy(gen.model_params(sv.model_param_layout(dcfg), 41)).to(dev)
    ti = gen.forward_inputs(96, 4, 4, 24, B, gamma + 1, (prefix, prefix), max_T, 42)
    di = gen.forward_inputs(96, 1, 2, 24, B, 1, (prefix, prefix), max_T, 43)
    tkv0 = torch.from_numpy(ti["kv"]).to(dev)
    dkv0 = torch.from_numpy(di["kv"]).to(dev)
    tok = torch.from_numpy(ti["tokens"]).to(dev)
    lens = torch.from_numpy(ti["lens"]).to(dev)
    stream = torch.cuda.current_stream()

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with no_gc():
            a.record(stream)
            for _ in range(steps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
        return a.elapsed_time(b) / steps  # ms

    print("[bench] model: verify forward", file=sys.stderr, flush=True)
    tkv = tkv0.clone()
    fwd_ms = timed(lambda: sv.spec_verify_forward(tcfg, pt, tok, lens, tkv, prefix), args.steps, args.warmup)
    one = tok[:, :1].contiguous()
    base_ms = timed(lambda: sv.spec_verify_forward(tcfg, pt, one, lens, tkv, prefix), args.steps, args.warmup)

    print("[bench] model: speculative rounds", file=sys.stderr, flush=True)
    rounds = min(args.steps, (max_T - prefix - gamma - 2) // (gamma + 1))
    max_len = max_T
    seq = torch.from_numpy(np.random.default_rng(44).integers(0, 96, size=(B, max_len)).astype(np.int32)).to(dev)
    r = np.random.default_rng(45)
    ud = [torch.from_numpy(r.random((B, gamma))).to(dev) for _ in range(rounds + 2)]
    uv = [torch.from_numpy(r.random((B, gamma + 1))).to(dev) for _ in range(rounds + 2)]

    def fresh():
        st = {"seq_len": torch.full((B,), prefix, dtype=torch.int32, device=dev),
              "tlen": torch.full((B,), prefix - 1, dtype=torch.int32, device=dev),
              "dlen": torch.full((B,), prefix - 2, dtype=torch.int32, device=dev),
              "tkv": tkv0.clone(), "dkv": dkv0.clone(), "k": 0}
        return st

    def one_round(st, k):
        return sv.spec_speculative_round(tcfg, pt, dcfg, pd, seq, st["seq_len"], st["tkv"], st["tlen"], st["dkv"],
                                         st["dlen"], ud[k], uv[k], T, prefix + k * (gamma + 1))

    st = fresh()
    one_round(st, 0)  # warm-up round (and library load)
    torch.cuda.synchronize()
    st = fresh()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ns = []
    with no_gc():
        a.record(stream)
        for k in range(rounds):
            n, _ = one_round(st, k)
            ns.append(n)
        b.record(stream)
        torch.cuda.synchronize()
    round_ms = a.elapsed_time(b) / rounds
    nacc = torch.stack(ns).cpu().numpy()

    # The same rounds replayed from one captured graph (the hint fixed at the
    # largest length any of them can reach); the state advances as before.
    print("[bench] model: rounds from a captured graph", file=sys.stderr, flush=True)
    st = fresh()
    hint_max = prefix + rounds * (gamma + 1)
    gud, guv = ud[0].clone(), uv[0].clone()
    sv.spec_speculative_round(tcfg, pt, dcfg, pd, seq, st["seq_len"], st["tkv"], st["tlen"], st["dkv"], st["dlen"],
                              gud, guv, T, hint_max)  # sizes the workspace for the largest hint
    torch.cuda.synchronize()
    st = fresh()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sv.spec_speculative_round(tcfg, pt, dcfg, pd, seq, st["seq_len"], st["tkv"], st["tlen"], st["dkv"],
                                  st["dlen"], gud, guv, T, hint_max)
    torch.cuda.synchronize()
    with no_gc():
        a.record(stream)
        for k in range(rounds):
            graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
    graph_ms = a.elapsed_time(b) / rounds
    gen_tokens = int((nacc + 1).sum())
    tested = np.where(nacc < gamma, nacc + 1, gamma)
    alpha = float(nacc.sum() / tested.sum())
    tok_s = gen_tokens / (rounds * round_ms * 1e-3)
    base_tok_s = B / (base_ms * 1e-3)
    # verify forward bytes: weights once, every layer's K/V read over prefix + n
    # rows and the n new rows written, activations ignored
    n = gamma + 1
    w_bytes = 4 * sv.model_param_count(tcfg)
    kv_bytes = 4 * 4 * B * 4 * 24 * 2 * ((prefix + n) + n)
    fwd_bytes = w_bytes + kv_bytes
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] model: timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = model_cpu_baseline(tcfg, dcfg, pt, pd, ti, di, gamma, T, prefix)
    line = {
        "metric": "generated tokens/sec (speculative rounds) and verified positions/sec (verify forward)",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": rounds,
        "warmup": 1,
        "ms_per_step": round_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: random weights, random tokens, N(0,1) cached K/V",
        "config": {"workload": f"pages' char models (target V=96 C=96 L=4 H=4, draft C=48 L=1 H=2), B={B}, "
                               f"cached prefix {prefix}, gamma={gamma}, T={T}"},
        "roofline": {"bound": "hbm", "achieved": fwd_bytes / (fwd_ms * 1e-3) / 1e9, "peak": 8000.0, "unit": "GB/s",
                     "frac": fwd_bytes / (fwd_ms * 1e-3) / 8e12, "traffic": None,
                     "kernel": "spec_verify_forward (target, gamma+1 tokens): 9 launches, launch-latency bound",
                     "algorithmic_bytes": fwd_bytes, "avg_ms": fwd_ms},
        "parts": {
            "verify_forward": {"ms": fwd_ms, "positions/s": B * gamma / (fwd_ms * 1e-3)},
            "target_only_decode": {"ms_per_token_step": base_ms, "tokens/s": base_tok_s},
            "round_graph": {"ms": graph_ms, "what": "the same rounds replayed from one captured HIP graph"},
            "round": {"ms": round_ms, "tokens/s": tok_s, "speedup_vs_target_only": tok_s / base_tok_s,
                      "alpha": alpha, "tokens_per_target_call": float((nacc + 1).mean()),
                      "accepted_per_proposed": float(nacc.sum() / (gamma * nacc.size))},
        },
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line))


def model_cpu_baseline(tcfg, dcfg, pt, pd, ti, di, gamma, T, prefix, budget_s=10.0):
    """The model and round oracles as they stand (fp64 numpy, one BLAS thread)
    on whole sequences of the model workload: the target's verify forward of
    gamma+1 tokens over each sequence's 384 cached rows, then whole rounds."""
    from threadpoolctl import threadpool_limits

    from oracle import model as M
    from oracle import round as R

    ct, cd = M.ModelConfig(**tcfg), M.ModelConfig(**dcfg)
    flat_t, flat_d = pt.cpu().numpy(), pd.cpu().numpy()
    B = ti["tokens"].shape[0]
    with threadpool_limits(limits=1):
        done, t0 = 0, time.perf_counter()
        while done < B and time.perf_counter() - t0 < budget_s / 2:
            b = done
            M.forward_cached(flat_t, ct, ti["tokens"][b : b + 1], ti["kv"][:, :, b : b + 1], ti["lens"][b : b + 1])
            done += 1
        fwd_s = time.perf_counter() - t0
        r = np.random.default_rng(46)
        toks, rounds, t1 = 0, 0, time.perf_counter()
        while time.perf_counter() - t1 < budget_s / 2:
            st = {"seq": [list(r.integers(0, ct.V, size=prefix))],
                  "tkv": ti["kv"][:, :, :1].astype(np.float64), "tlen": np.array([prefix - 1]),
                  "dkv": di["kv"][:, :, :1].astype(np.float64), "dlen": np.array([prefix - 2])}
            res = R.speculative_round(flat_t, ct, flat_d, cd, st, gamma, T, r.random((1, gamma)),
                                      r.random((1, gamma + 1)))
            toks += int(res["n_accepted"][0]) + 1
            rounds += 1
        round_s = time.perf_counter() - t1
    return {
        "value": toks / round_s,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{rounds} whole rounds of one sequence (4 draft forwards, the target's verify forward, the "
                  f"sampler) and {done} target verify forwards over 384 cached rows, numpy fp64, one BLAS thread",
        "verify_forward_positions/s": done * gamma / fwd_s,
        "seconds": fwd_s + round_s,
    }

if __name__ == "__main__":
    main()
