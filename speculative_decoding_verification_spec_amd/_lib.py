"""ctypes binding of libspecverify.so (the C ABI declared in include/spec_verify.h).

Argument marshalling only: shapes and dtypes of PyTorch tensors are checked and
turned into the plain pointers and sizes the C functions take; every step of
the verification path runs in the library's HIP kernels.  PyTorch provides the
device memory and the current stream.  There is no fallback: if the library is
missing, or a call returns an error status, a Python exception is raised.
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SPEC_OK, SPEC_ERR_ARG, SPEC_ERR_OVERFLOW, SPEC_ERR_UNSUPPORTED, SPEC_ERR_LAUNCH, SPEC_ERR_SCRATCH = range(6)
SPEC_F32, SPEC_BF16, SPEC_F16 = 0, 1, 2

EXPORTED = (
    "spec_version",
    "spec_status_string",
    "spec_verify_attention_workspace_size",
    "spec_verify_attention",
    "spec_verify_attention_paged",
    "spec_verify_attention_int8_workspace_size",
    "spec_verify_attention_int8",
    "spec_reject_sample_workspace_size",
    "spec_reject_sample",
    "spec_reject_sample_noalloc",
    "spec_kv_truncate",
    "spec_model_param_count",
    "spec_verify_forward_workspace_size",
    "spec_verify_forward",
    "spec_speculative_round_workspace_size",
    "spec_speculative_round",
)


class SpecModel(ctypes.Structure):
    """spec_model_t: the shape of a GPT-2-type decoder (MLP width 4C)."""

    _fields_ = [("V", ctypes.c_int), ("C", ctypes.c_int), ("L", ctypes.c_int), ("H", ctypes.c_int),
                ("T", ctypes.c_int)]


class SpecError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} returned {msg} ({status})")
        self.status = status


_lib = None


def load(path=LIB_PATH):
    """Load the library (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m speculative_decoding_verification_spec_amd.build` "
            "(or __graft_entry__.build())"
        )
    L = ctypes.CDLL(path)
    c_int, c_size, vp, c_float = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    L.spec_version.restype = ctypes.c_char_p
    L.spec_version.argtypes = []
    L.spec_status_string.restype = ctypes.c_char_p
    L.spec_status_string.argtypes = [c_int]
    L.spec_verify_attention_workspace_size.restype = c_size
    L.spec_verify_attention_workspace_size.argtypes = [c_int] * 6 + [c_int]
    L.spec_verify_attention.restype = c_int
    L.spec_verify_attention.argtypes = [vp] * 7 + [c_int] * 7 + [c_float, c_int, vp, c_size, vp]
    L.spec_verify_attention_int8_workspace_size.restype = c_size
    L.spec_verify_attention_int8_workspace_size.argtypes = [c_int] * 6
    L.spec_verify_attention_int8.restype = c_int
    L.spec_verify_attention_int8.argtypes = [vp] * 9 + [c_int] * 7 + [c_float, vp, c_size, vp]
    L.spec_verify_attention_paged.restype = c_int
    L.spec_verify_attention_paged.argtypes = [vp] * 8 + [c_int] * 9 + [c_float, c_int, vp, c_size, vp]
    L.spec_reject_sample_workspace_size.restype = c_size
    L.spec_reject_sample_workspace_size.argtypes = [c_int] * 4
    L.spec_reject_sample.restype = c_int
    L.spec_reject_sample.argtypes = [vp] * 4 + [c_int] * 3 + [c_float, c_int] + [vp] * 5 + [c_size, vp]
    L.spec_reject_sample_noalloc.restype = c_int
    L.spec_reject_sample_noalloc.argtypes = [vp] * 4 + [c_int] * 3 + [c_float, c_int] + [vp] * 5
    L.spec_kv_truncate.restype = c_int
    L.spec_kv_truncate.argtypes = [vp, vp, c_int, c_int, vp]
    pm = ctypes.POINTER(SpecModel)
    L.spec_model_param_count.restype = c_size
    L.spec_model_param_count.argtypes = [pm]
    L.spec_verify_forward_workspace_size.restype = c_size
    L.spec_verify_forward_workspace_size.argtypes = [pm, c_int, c_int, c_int]
    L.spec_verify_forward.restype = c_int
    L.spec_verify_forward.argtypes = [pm, vp, vp, vp, vp, c_int, vp, c_int, c_int, c_int, vp, c_size, vp]
    L.spec_speculative_round_workspace_size.restype = c_size
    L.spec_speculative_round_workspace_size.argtypes = [pm, pm, c_int, c_int, c_int]
    L.spec_speculative_round.restype = c_int
    L.spec_speculative_round.argtypes = ([pm, vp, pm, vp, vp, vp, c_int, vp, vp, c_int, vp, vp, c_int, vp, vp,
                                          c_int, c_int, c_float, c_int, vp, vp, vp, c_size, vp])
    _lib = L
    return L


def version():
    return load().spec_version().decode()


def _check(fn, status):
    if status != SPEC_OK:
        raise SpecError(fn, status, load().spec_status_string(status).decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    if t.dtype == torch.float16:
        return SPEC_F16
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16, float16 or float32)")


def _need(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


class Workspace:
    """A device buffer grown on demand and reused across calls of any sizes.

    The library writes every workspace word before reading it, so the buffer
    needs no initialisation between calls.  Calls sharing a workspace must be
    ordered (one stream).
    """

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes, device):
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return self.buf


_default_ws = {}


def _workspace(ws, key, nbytes, device):
    if ws is None:
        ws = _default_ws.setdefault((key, str(device)), Workspace())
    return ws.get(nbytes, device)


def verify_attention_workspace_size(B, Hq, Hkv, n_q, D, max_len_hint, dtype_code):
    return load().spec_verify_attention_workspace_size(B, Hq, Hkv, n_q, D, max_len_hint, dtype_code)


def spec_verify_attention(q, k_new, v_new, k_cache, v_cache, cache_len, max_len_hint, out=None, scale=None,
                          workspace=None, stream=None):
    """Verify attention with KV append; returns ``out`` [B, Hq, n_q, D]."""
    L = load()
    _need(q, "q")
    B, Hq, n_q, D = q.shape
    Hkv = k_new.shape[1]
    max_T = k_cache.shape[2]
    _need(k_new, "k_new", q.dtype, (B, Hkv, n_q, D))
    _need(v_new, "v_new", q.dtype, (B, Hkv, n_q, D))
    _need(k_cache, "k_cache", q.dtype, (B, Hkv, max_T, D))
    _need(v_cache, "v_cache", q.dtype, (B, Hkv, max_T, D))
    _need(cache_len, "cache_len", torch.int32, (B,))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, q.shape)
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nbytes = L.spec_verify_attention_workspace_size(B, Hq, Hkv, n_q, D, int(max_len_hint), dt)
    if nbytes == 0:
        raise SpecError("spec_verify_attention_workspace_size", SPEC_ERR_UNSUPPORTED, "no valid size")
    ws = _workspace(workspace, "attn", nbytes, q.device)
    st = L.spec_verify_attention(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), _ptr(out),
        B, Hq, Hkv, n_q, D, max_T, int(max_len_hint), scale, dt, _ptr(ws), ws.numel(), _stream(stream),
    )
    _check("spec_verify_attention", st)
    return out


def spec_verify_attention_paged(q, k_new, v_new, k_pages, v_pages, block_table, cache_len, max_len_hint, out=None,
                                scale=None, workspace=None, stream=None):
    """Verify attention with KV append over a paged cache; returns ``out`` [B, Hq, n_q, D].

    k_pages, v_pages: [Hkv, num_pages, page_size, D]; block_table: int32 [B, max_blocks].
    """
    L = load()
    _need(q, "q")
    B, Hq, n_q, D = q.shape
    Hkv = k_new.shape[1]
    _, num_pages, page, _ = k_pages.shape
    _need(k_new, "k_new", q.dtype, (B, Hkv, n_q, D))
    _need(v_new, "v_new", q.dtype, (B, Hkv, n_q, D))
    _need(k_pages, "k_pages", q.dtype, (Hkv, num_pages, page, D))
    _need(v_pages, "v_pages", q.dtype, (Hkv, num_pages, page, D))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise SpecError("spec_verify_attention_paged", SPEC_ERR_ARG, "block_table must be [B, max_blocks]")
    _need(cache_len, "cache_len", torch.int32, (B,))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, q.shape)
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nbytes = L.spec_verify_attention_workspace_size(B, Hq, Hkv, n_q, D, int(max_len_hint), dt)
    if nbytes == 0:
        raise SpecError("spec_verify_attention_workspace_size", SPEC_ERR_UNSUPPORTED, "no valid size")
    ws = _workspace(workspace, "attn", nbytes, q.device)
    st = L.spec_verify_attention_paged(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(cache_len),
        _ptr(out), B, Hq, Hkv, n_q, D, page, num_pages, block_table.shape[1], int(max_len_hint), scale, dt,
        _ptr(ws), ws.numel(), _stream(stream),
    )
    _check("spec_verify_attention_paged", st)
    return out


def spec_verify_attention_int8(q, k_new, v_new, k_cache, k_scale, v_cache, v_scale, cache_len, max_len_hint,
                               out=None, scale=None, workspace=None, stream=None):
    """Verify attention with KV append over an int8 cache; returns ``out`` [B, Hq, n_q, D] (bf16).

    k_cache, v_cache: int8 [B, Hkv, max_T, D]; k_scale, v_scale: float16 [B, Hkv, max_T]
    (one scale per head and position); q, k_new, v_new: bfloat16.
    """
    L = load()
    _need(q, "q", torch.bfloat16)
    B, Hq, n_q, D = q.shape
    Hkv = k_new.shape[1]
    max_T = k_cache.shape[2]
    _need(k_new, "k_new", torch.bfloat16, (B, Hkv, n_q, D))
    _need(v_new, "v_new", torch.bfloat16, (B, Hkv, n_q, D))
    _need(k_cache, "k_cache", torch.int8, (B, Hkv, max_T, D))
    _need(v_cache, "v_cache", torch.int8, (B, Hkv, max_T, D))
    _need(k_scale, "k_scale", torch.float16, (B, Hkv, max_T))
    _need(v_scale, "v_scale", torch.float16, (B, Hkv, max_T))
    _need(cache_len, "cache_len", torch.int32, (B,))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, q.shape)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nbytes = L.spec_verify_attention_int8_workspace_size(B, Hq, Hkv, n_q, D, int(max_len_hint))
    if nbytes == 0:
        raise SpecError("spec_verify_attention_int8_workspace_size", SPEC_ERR_UNSUPPORTED, "no valid size")
    ws = _workspace(workspace, "attn8", nbytes, q.device)
    st = L.spec_verify_attention_int8(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache), _ptr(v_scale),
        _ptr(cache_len), _ptr(out), B, Hq, Hkv, n_q, D, max_T, int(max_len_hint), scale, _ptr(ws), ws.numel(),
        _stream(stream),
    )
    _check("spec_verify_attention_int8", st)
    return out


def reject_sample_workspace_size(B, gamma, V, dtype_code):
    return load().spec_reject_sample_workspace_size(B, gamma, V, dtype_code)


def spec_reject_sample(target_logits, draft_logits, draft_tokens, uniforms, temperature, n_accepted=None,
                       out_tokens=None, p_draft=None, q_draft=None, want_probs=False, workspace=None, stream=None):
    """Modified rejection sampling; returns (n_accepted [B], out_tokens [B, gamma+1], p_draft, q_draft).

    temperature 0 is greedy verification: draft_logits and uniforms are not
    read and may be None.
    """
    L = load()
    _need(target_logits, "target_logits")
    B, G1, V = target_logits.shape
    G = G1 - 1
    greedy = float(temperature) == 0.0
    if not (greedy and draft_logits is None):
        _need(draft_logits, "draft_logits", target_logits.dtype, (B, G, V))
    _need(draft_tokens, "draft_tokens", torch.int32, (B, G))
    if not (greedy and uniforms is None):
        _need(uniforms, "uniforms", torch.float64, (B, G + 1))
    dev = target_logits.device
    if n_accepted is None:
        n_accepted = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    if want_probs and p_draft is None:
        p_draft = torch.empty((B, G), dtype=torch.float32, device=dev)
    if want_probs and q_draft is None:
        q_draft = torch.empty((B, G), dtype=torch.float32, device=dev)
    _need(n_accepted, "n_accepted", torch.int32, (B,))
    _need(out_tokens, "out_tokens", torch.int32, (B, G + 1))
    for t, name in ((p_draft, "p_draft"), (q_draft, "q_draft")):
        if t is not None:
            _need(t, name, torch.float32, (B, G))
    dt = _dtype_code(target_logits)
    nbytes = L.spec_reject_sample_workspace_size(B, G, V, dt)
    if nbytes == 0:
        raise SpecError("spec_reject_sample_workspace_size", SPEC_ERR_ARG, "no valid size")
    ws = _workspace(workspace, "rs", nbytes, dev)
    st = L.spec_reject_sample(
        _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(uniforms), B, G, V, float(temperature),
        dt, _ptr(n_accepted), _ptr(out_tokens), _ptr(p_draft), _ptr(q_draft), _ptr(ws), ws.numel(),
        _stream(stream),
    )
    _check("spec_reject_sample", st)
    return n_accepted, out_tokens, p_draft, q_draft


def spec_kv_truncate(cache_len, n_accepted, n_q, stream=None):
    """cache_len += 1 + n_accepted (in place)."""
    L = load()
    _need(cache_len, "cache_len", torch.int32)
    B = cache_len.shape[0]
    _need(n_accepted, "n_accepted", torch.int32, (B,))
    _check("spec_kv_truncate", L.spec_kv_truncate(_ptr(cache_len), _ptr(n_accepted), B, int(n_q), _stream(stream)))
    return cache_len


def _model(model):
    if isinstance(model, SpecModel):
        return model
    if isinstance(model, dict):
        return SpecModel(model["V"], model["C"], model["L"], model["H"], model["T"])
    V, C, L, H, T = (getattr(model, k) for k in ("V", "C", "L", "H", "T"))
    return SpecModel(V, C, L, H, T)


def model_param_layout(model):
    """(name, shape) of every parameter in the packed array, in order (the
    layout documented with spec_model_param_count)."""
    m = _model(model)
    C, F, V, T = m.C, 4 * m.C, m.V, m.T
    out = [("token_embedding", (V, C)), ("position_embedding", (T, C))]
    for l in range(m.L):
        out += [(f"block{l}.norm1.gain", (C,)), (f"block{l}.norm1.bias", (C,)), (f"block{l}.attn.in", (C, 3 * C)),
                (f"block{l}.attn.out", (C, C)), (f"block{l}.norm2.gain", (C,)), (f"block{l}.norm2.bias", (C,)),
                (f"block{l}.mlp.up", (C, F)), (f"block{l}.mlp.up_bias", (F,)), (f"block{l}.mlp.down", (F, C)),
                (f"block{l}.mlp.down_bias", (C,))]
    out += [("final_norm.gain", (C,)), ("final_norm.bias", (C,)), ("unembedding", (C, V))]
    return out


def model_param_count(model):
    """Floats in the packed parameter array (the library's count)."""
    m = _model(model)
    return int(load().spec_model_param_count(ctypes.byref(m)))


def spec_verify_forward(model, params, tokens, cache_len, kv_cache, max_len_hint, logits=None, workspace=None,
                        stream=None):
    """Cached verify forward; returns ``logits`` [B, n, V] (fp32).

    params: [param_count] float32; tokens: [B, n] int32; cache_len: [B] int32
    (not modified); kv_cache: [L, 2, B, H, max_T, D] float32 (rows
    [cache_len[b], cache_len[b] + n) of every layer are written).
    """
    Lb = load()
    m = _model(model)
    _need(params, "params", torch.float32, (model_param_count(m),))
    _need(tokens, "tokens", torch.int32)
    B, n = tokens.shape
    _need(cache_len, "cache_len", torch.int32, (B,))
    _need(kv_cache, "kv_cache", torch.float32)
    if kv_cache.dim() != 6 or tuple(kv_cache.shape[:4]) != (m.L, 2, B, m.H) or kv_cache.shape[5] != m.C // m.H:
        raise ValueError(f"kv_cache has shape {tuple(kv_cache.shape)}, expected ({m.L}, 2, {B}, {m.H}, max_T, "
                         f"{m.C // max(m.H, 1)})")
    max_T = kv_cache.shape[4]
    if logits is None:
        logits = torch.empty((B, n, m.V), dtype=torch.float32, device=tokens.device)
    _need(logits, "logits", torch.float32, (B, n, m.V))
    nbytes = Lb.spec_verify_forward_workspace_size(ctypes.byref(m), B, n, int(max_len_hint))
    if nbytes == 0:
        raise SpecError("spec_verify_forward_workspace_size", SPEC_ERR_UNSUPPORTED, "no valid size")
    ws = _workspace(workspace, "fwd", nbytes, tokens.device)
    st = Lb.spec_verify_forward(ctypes.byref(m), _ptr(params), _ptr(tokens), _ptr(cache_len), _ptr(kv_cache), max_T,
                                _ptr(logits), B, n, int(max_len_hint), _ptr(ws), ws.numel(), _stream(stream))
    _check("spec_verify_forward", st)
    return logits


def spec_speculative_round(target, target_params, draft, draft_params, seq, seq_len, target_kv, target_len, draft_kv,
                           draft_len, u_draft, u_verify, temperature, max_len_hint, n_accepted=None, out_tokens=None,
                           workspace=None, stream=None):
    """One speculative round on the device; returns (n_accepted [B], out_tokens [B, gamma+1]).

    seq [B, max_len] / seq_len [B] (committed tokens), target_len [B] = L - 1,
    draft_len [B] = L - 2 and both caches are updated in place.  u_draft
    [B, gamma] and u_verify [B, gamma+1] float64 (None at temperature 0; then
    gamma comes from n_accepted/out_tokens or u shapes must be given).
    """
    Lb = load()
    mt, md = _model(target), _model(draft)
    _need(seq, "seq", torch.int32)
    B, max_len = seq.shape
    greedy = float(temperature) == 0.0
    if u_verify is not None:
        gamma = u_verify.shape[1] - 1
    elif out_tokens is not None:
        gamma = out_tokens.shape[1] - 1
    else:
        raise ValueError("give u_verify or out_tokens so that gamma is known")
    _need(target_params, "target_params", torch.float32, (model_param_count(mt),))
    _need(draft_params, "draft_params", torch.float32, (model_param_count(md),))
    for t, name in ((seq_len, "seq_len"), (target_len, "target_len"), (draft_len, "draft_len")):
        _need(t, name, torch.int32, (B,))
    _need(target_kv, "target_kv", torch.float32)
    _need(draft_kv, "draft_kv", torch.float32)
    if not greedy:
        _need(u_draft, "u_draft", torch.float64, (B, gamma))
        _need(u_verify, "u_verify", torch.float64, (B, gamma + 1))
    if n_accepted is None:
        n_accepted = torch.empty(B, dtype=torch.int32, device=seq.device)
    if out_tokens is None:
        out_tokens = torch.empty((B, gamma + 1), dtype=torch.int32, device=seq.device)
    nbytes = Lb.spec_speculative_round_workspace_size(ctypes.byref(mt), ctypes.byref(md), B, gamma,
                                                      int(max_len_hint))
    if nbytes == 0:
        raise SpecError("spec_speculative_round_workspace_size", SPEC_ERR_UNSUPPORTED, "no valid size")
    ws = _workspace(workspace, "round", nbytes, seq.device)
    st = Lb.spec_speculative_round(
        ctypes.byref(mt), _ptr(target_params), ctypes.byref(md), _ptr(draft_params), _ptr(seq), _ptr(seq_len),
        max_len, _ptr(target_kv), _ptr(target_len), target_kv.shape[4], _ptr(draft_kv), _ptr(draft_len),
        draft_kv.shape[4], _ptr(None if greedy else u_draft), _ptr(None if greedy else u_verify), B, gamma,
        float(temperature), int(max_len_hint), _ptr(n_accepted), _ptr(out_tokens), _ptr(ws), ws.numel(),
        _stream(stream))
    _check("spec_speculative_round", st)
    return n_accepted, out_tokens
