"""Thin Python binding of libgdn.so (include/gdn.h), argument marshalling only.

Each function has the name of the C entry point it calls. It checks that the
torch tensors it is given live on the GPU, are contiguous and have the dtype
and element count the ABI expects, passes their device pointers and the
current HIP stream, and raises ``GdnError`` on any status other than
GDN_OK. All compute happens in the library's HIP kernels. PyTorch only
provides device memory and streams.

There is no fallback: if libgdn.so is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_E_INVALID_ARG, GDN_E_UNSUPPORTED, GDN_E_HIP, GDN_E_WORKSPACE, GDN_E_TOO_LARGE = 0, 1, 2, 3, 4, 5
GDN_STATIC_SCRATCH_BYTES = 256 << 20   # the static scratch of gdn_prefill_fused_static (gdn.h)
GDN_F32, GDN_BF16 = 0, 1
GDN_L2_CLAMP, GDN_L2_RSQRT = 0, 1
HEAD_DIM = 128
CONV_K = 4

# Every entry point include/gdn.h declares.
EXPORTS = ("gdn_default_config", "gdn_conv_gate_prep", "gdn_prefill_chunked",
           "gdn_prefill_workspace_bytes", "gdn_decode_step", "gdn_decode_fused", "gdn_decode_verify",
           "gdn_gated_rmsnorm", "gdn_prefill_chunked_ckpt", "gdn_conv_state_ckpt", "gdn_state_check",
           "gdn_in_proj", "gdn_out_proj", "gdn_prefill_fused", "gdn_prefill_fused_workspace_bytes",
           "gdn_status_string", "gdn_version", "gdn_prefill_fused_static", "gdn_prefill_fused_ckpt")


class GdnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class gdn_config(ctypes.Structure):
    _fields_ = [("n_qk_heads", ctypes.c_int32), ("n_v_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("conv_kernel", ctypes.c_int32),
                ("l2_eps", ctypes.c_float), ("norm_eps", ctypes.c_float),
                ("act_dtype", ctypes.c_int), ("l2_mode", ctypes.c_int)]


_P = ctypes.c_void_p
_lib = None


def load(path: Optional[str] = None):
    """Load libgdn.so (no GPU work happens here). Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(p)
    lib.gdn_default_config.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int]
    lib.gdn_default_config.restype = gdn_config
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_version.argtypes = []
    lib.gdn_version.restype = ctypes.c_char_p
    cfgp = ctypes.POINTER(gdn_config)
    lib.gdn_conv_gate_prep.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int32] + [_P] * 14 + [_P]
    lib.gdn_conv_gate_prep.restype = ctypes.c_int
    lib.gdn_prefill_chunked.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int32] + [_P] * 10 + [ctypes.c_size_t, _P]
    lib.gdn_prefill_chunked.restype = ctypes.c_int
    lib.gdn_prefill_chunked_ckpt.argtypes = ([cfgp, ctypes.c_int32, ctypes.c_int32] + [_P] * 9
                                             + [ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P])
    lib.gdn_prefill_chunked_ckpt.restype = ctypes.c_int
    lib.gdn_conv_state_ckpt.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, ctypes.c_int32,
                                        ctypes.c_int32, _P, _P]
    lib.gdn_conv_state_ckpt.restype = ctypes.c_int
    lib.gdn_state_check.argtypes = [_P, ctypes.c_int64, _P, _P]
    lib.gdn_state_check.restype = ctypes.c_int
    lib.gdn_prefill_workspace_bytes.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int32]
    lib.gdn_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_decode_step.argtypes = [cfgp, ctypes.c_int32] + [_P] * 8 + [_P]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_decode_fused.argtypes = [cfgp, ctypes.c_int32] + [_P] * 13 + [_P]
    lib.gdn_decode_fused.restype = ctypes.c_int
    lib.gdn_decode_verify.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int32] + [_P] * 13 + [_P]
    lib.gdn_decode_verify.restype = ctypes.c_int
    lib.gdn_prefill_fused.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int32] + [_P] * 15 + [ctypes.c_size_t, _P]
    lib.gdn_prefill_fused.restype = ctypes.c_int
    lib.gdn_prefill_fused_ckpt.argtypes = ([cfgp, ctypes.c_int32, ctypes.c_int32] + [_P] * 14
                                           + [ctypes.c_int32, ctypes.c_int32, _P, _P, _P, ctypes.c_size_t, _P])
    lib.gdn_prefill_fused_ckpt.restype = ctypes.c_int
    lib.gdn_prefill_fused_static.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int32] + [_P] * 15
    lib.gdn_prefill_fused_static.restype = ctypes.c_int
    lib.gdn_prefill_fused_workspace_bytes.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int32]
    lib.gdn_prefill_fused_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_in_proj.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int32] + [_P] * 9 + [_P]
    lib.gdn_in_proj.restype = ctypes.c_int
    lib.gdn_out_proj.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P]
    lib.gdn_out_proj.restype = ctypes.c_int
    lib.gdn_gated_rmsnorm.argtypes = [cfgp, ctypes.c_int64, _P, _P, _P, _P, _P]
    lib.gdn_gated_rmsnorm.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def make_config(n_qk_heads: int, n_v_heads: int, act: str = "bf16", l2_eps: float = 1e-6,
                norm_eps: float = 1e-6, head_dim: int = HEAD_DIM, conv_kernel: int = CONV_K,
                l2_mode: str = "clamp") -> gdn_config:
    """``l2_mode``: "clamp" (x / max(|x|, eps)) or "rsqrt" (x / sqrt(sum x^2 + eps))."""
    if l2_mode not in ("clamp", "rsqrt"):
        raise ValueError(f"l2_mode: {l2_mode!r}, expected 'clamp' or 'rsqrt'")
    c = gdn_config()
    c.n_qk_heads, c.n_v_heads, c.head_dim, c.conv_kernel = n_qk_heads, n_v_heads, head_dim, conv_kernel
    c.l2_eps, c.norm_eps = l2_eps, norm_eps
    c.act_dtype = GDN_BF16 if act == "bf16" else GDN_F32
    c.l2_mode = GDN_L2_RSQRT if l2_mode == "rsqrt" else GDN_L2_CLAMP
    return c


def status_string(status: int) -> str:
    return load().gdn_status_string(status).decode()


def _check(fn: str, status: int):
    if status != GDN_OK:
        raise GdnError(fn, status, status_string(status))


def _act_dtype(cfg: gdn_config):
    return torch.bfloat16 if cfg.act_dtype == GDN_BF16 else torch.float32


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, numel: Optional[int] = None):
    """Device pointer of a contiguous GPU tensor (0 for None)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    return t.data_ptr() if t.numel() else None


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def gdn_conv_gate_prep(cfg: gdn_config, n_seqs: int, n_tokens: int, cu_seqlens, qkv, beta_logit,
                       alpha_logit, conv_w, dt_bias, A_log, conv_state_in, conv_state_out,
                       q, k, v, beta, g, stream=None):
    Hqk, Hv, d = cfg.n_qk_heads, cfg.n_v_heads, cfg.head_dim
    C, T, N, ad = d * (2 * Hqk + Hv), n_tokens, n_seqs, _act_dtype(cfg)
    st = _ptr(conv_state_out, "conv_state_out", ad, N * (CONV_K - 1) * C)
    s = load().gdn_conv_gate_prep(
        ctypes.byref(cfg), N, T, _ptr(cu_seqlens, "cu_seqlens", torch.int32, N + 1),
        _ptr(qkv, "qkv", ad, T * C), _ptr(beta_logit, "beta_logit", ad, T * Hv),
        _ptr(alpha_logit, "alpha_logit", ad, T * Hv), _ptr(conv_w, "conv_w", torch.float32, C * CONV_K),
        _ptr(dt_bias, "dt_bias", torch.float32, Hv), _ptr(A_log, "A_log", torch.float32, Hv),
        _ptr(conv_state_in, "conv_state_in", ad, N * (CONV_K - 1) * C), st,
        _ptr(q, "q", torch.float32, T * Hqk * d), _ptr(k, "k", torch.float32, T * Hqk * d),
        _ptr(v, "v", torch.float32, T * Hv * d), _ptr(beta, "beta", torch.float32, T * Hv),
        _ptr(g, "g", torch.float32, T * Hv), _stream(stream))
    _check("gdn_conv_gate_prep", s)


def gdn_prefill_workspace_bytes(cfg: gdn_config, n_seqs: int, n_tokens: int) -> int:
    return int(load().gdn_prefill_workspace_bytes(ctypes.byref(cfg), n_seqs, n_tokens))


def gdn_prefill_chunked(cfg: gdn_config, n_seqs: int, n_tokens: int, cu_seqlens, q, k, v, beta, g,
                        S_in, S_out, o, workspace, stream=None):
    Hqk, Hv, d = cfg.n_qk_heads, cfg.n_v_heads, cfg.head_dim
    T, N = n_tokens, n_seqs
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = load().gdn_prefill_chunked(
        ctypes.byref(cfg), N, T, _ptr(cu_seqlens, "cu_seqlens", torch.int32, N + 1),
        _ptr(q, "q", torch.float32, T * Hqk * d), _ptr(k, "k", torch.float32, T * Hqk * d),
        _ptr(v, "v", torch.float32, T * Hv * d), _ptr(beta, "beta", torch.float32, T * Hv),
        _ptr(g, "g", torch.float32, T * Hv), _ptr(S_in, "S_in", torch.float32, N * Hv * d * d),
        _ptr(S_out, "S_out", torch.float32, N * Hv * d * d), _ptr(o, "o", _act_dtype(cfg), T * Hv * d),
        _ptr(workspace, "workspace"), ws_bytes, _stream(stream))
    _check("gdn_prefill_chunked", s)


def gdn_prefill_chunked_ckpt(cfg: gdn_config, n_seqs: int, n_tokens: int, cu_seqlens, q, k, v, beta, g,
                             S_in, S_out, o, ckpt_every: int, ckpt_cap: int, S_ckpt, workspace, stream=None):
    Hqk, Hv, d = cfg.n_qk_heads, cfg.n_v_heads, cfg.head_dim
    T, N = n_tokens, n_seqs
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = load().gdn_prefill_chunked_ckpt(
        ctypes.byref(cfg), N, T, _ptr(cu_seqlens, "cu_seqlens", torch.int32, N + 1),
        _ptr(q, "q", torch.float32, T * Hqk * d), _ptr(k, "k", torch.float32, T * Hqk * d),
        _ptr(v, "v", torch.float32, T * Hv * d), _ptr(beta, "beta", torch.float32, T * Hv),
        _ptr(g, "g", torch.float32, T * Hv), _ptr(S_in, "S_in", torch.float32, N * Hv * d * d),
        _ptr(S_out, "S_out", torch.float32, N * Hv * d * d), _ptr(o, "o", _act_dtype(cfg), T * Hv * d),
        ckpt_every, ckpt_cap, _ptr(S_ckpt, "S_ckpt", torch.float32, N * ckpt_cap * Hv * d * d),
        _ptr(workspace, "workspace"), ws_bytes, _stream(stream))
    _check("gdn_prefill_chunked_ckpt", s)


def gdn_conv_state_ckpt(cfg: gdn_config, n_seqs: int, n_tokens: int, cu_seqlens, qkv, conv_state_in,
                        ckpt_every: int, ckpt_cap: int, conv_ckpt, stream=None):
    Hqk, Hv, d = cfg.n_qk_heads, cfg.n_v_heads, cfg.head_dim
    C, ad, N, T = d * (2 * Hqk + Hv), _act_dtype(cfg), n_seqs, n_tokens
    s = load().gdn_conv_state_ckpt(
        ctypes.byref(cfg), N, T, _ptr(cu_seqlens, "cu_seqlens", torch.int32, N + 1), _ptr(qkv, "qkv", ad, T * C),
        _ptr(conv_state_in, "conv_state_in", ad, N * (CONV_K - 1) * C), ckpt_every, ckpt_cap,
        _ptr(conv_ckpt, "conv_ckpt", ad, N * ckpt_cap * (CONV_K - 1) * C), _stream(stream))
    _check("gdn_conv_state_ckpt", s)


def gdn_state_check(S, stats, stream=None):
    """Non-finite guard: stats (int32[2] on the GPU) <- [count of NaN/Inf in S,
    bits of max |x| over the finite values]."""
    s = load().gdn_state_check(_ptr(S, "S", torch.float32), S.numel(), _ptr(stats, "stats", torch.int32, 2),
                               _stream(stream))
    _check("gdn_state_check", s)


def gdn_decode_step(cfg: gdn_config, n_seqs: int, q, k, v, beta, g, S_in, S_out, o, stream=None):
    Hqk, Hv, d, N = cfg.n_qk_heads, cfg.n_v_heads, cfg.head_dim, n_seqs
    s = load().gdn_decode_step(
        ctypes.byref(cfg), N, _ptr(q, "q", torch.float32, N * Hqk * d),
        _ptr(k, "k", torch.float32, N * Hqk * d), _ptr(v, "v", torch.float32, N * Hv * d),
        _ptr(beta, "beta", torch.float32, N * Hv), _ptr(g, "g", torch.float32, N * Hv),
        _ptr(S_in, "S_in", torch.float32, N * Hv * d * d), _ptr(S_out, "S_out", torch.float32, N * Hv * d * d),
        _ptr(o, "o", _act_dtype(cfg), N * Hv * d), _stream(stream))
    _check("gdn_decode_step", s)


def gdn_decode_fused(cfg: gdn_config, n_seqs: int, qkv, beta_logit, alpha_logit, z, conv_w, dt_bias,
                     A_log, norm_w, conv_state_in, conv_state_out, S_in, S_out, y, stream=None):
    Hqk, Hv, d, N = cfg.n_qk_heads, cfg.n_v_heads, cfg.head_dim, n_seqs
    C, ad = d * (2 * Hqk + Hv), _act_dtype(cfg)
    s = load().gdn_decode_fused(
        ctypes.byref(cfg), N, _ptr(qkv, "qkv", ad, N * C), _ptr(beta_logit, "beta_logit", ad, N * Hv),
        _ptr(alpha_logit, "alpha_logit", ad, N * Hv), _ptr(z, "z", ad, N * Hv * d),
        _ptr(conv_w, "conv_w", torch.float32, C * CONV_K), _ptr(dt_bias, "dt_bias", torch.float32, Hv),
        _ptr(A_log, "A_log", torch.float32, Hv), _ptr(norm_w, "norm_w", torch.float32, d),
        _ptr(conv_state_in, "conv_state_in", ad, N * (CONV_K - 1) * C),
        _ptr(conv_state_out, "conv_state_out", ad, N * (CONV_K - 1) * C),
        _ptr(S_in, "S_in", torch.float32, N * Hv * d * d), _ptr(S_out, "S_out", torch.float32, N * Hv * d * d),
        _ptr(y, "y", ad, N * Hv * d), _stream(stream))
    _check("gdn_decode_fused", s)


def gdn_decode_verify(cfg: gdn_config, n_seqs: int, n_tokens: int, qkv, beta_logit, alpha_logit, z, conv_w,
                      dt_bias, A_log, norm_w, conv_state_in, conv_snap, S_in, S_snap, y, stream=None):
    Hqk, Hv, d, N, K = cfg.n_qk_heads, cfg.n_v_heads, cfg.head_dim, n_seqs, n_tokens
    C, ad = d * (2 * Hqk + Hv), _act_dtype(cfg)
    s = load().gdn_decode_verify(
        ctypes.byref(cfg), N, K, _ptr(qkv, "qkv", ad, N * K * C), _ptr(beta_logit, "beta_logit", ad, N * K * Hv),
        _ptr(alpha_logit, "alpha_logit", ad, N * K * Hv), _ptr(z, "z", ad, N * K * Hv * d),
        _ptr(conv_w, "conv_w", torch.float32, C * CONV_K), _ptr(dt_bias, "dt_bias", torch.float32, Hv),
        _ptr(A_log, "A_log", torch.float32, Hv), _ptr(norm_w, "norm_w", torch.float32, d),
        _ptr(conv_state_in, "conv_state_in", ad, N * (CONV_K - 1) * C),
        _ptr(conv_snap, "conv_snap", ad, N * K * (CONV_K - 1) * C),
        _ptr(S_in, "S_in", torch.float32, N * Hv * d * d), _ptr(S_snap, "S_snap", torch.float32, N * K * Hv * d * d),
        _ptr(y, "y", ad, N * K * Hv * d), _stream(stream))
    _check("gdn_decode_verify", s)


def gdn_gated_rmsnorm(cfg: gdn_config, n_rows: int, o, z, norm_w, y, stream=None):
    d, ad = cfg.head_dim, _act_dtype(cfg)
    s = load().gdn_gated_rmsnorm(
        ctypes.byref(cfg), n_rows, _ptr(o, "o", ad, n_rows * d), _ptr(z, "z", ad, n_rows * d),
        _ptr(norm_w, "norm_w", torch.float32, d), _ptr(y, "y", ad, n_rows * d), _stream(stream))
    _check("gdn_gated_rmsnorm", s)


def gdn_prefill_fused_workspace_bytes(cfg: gdn_config, n_seqs: int, n_tokens: int) -> int:
    return int(load().gdn_prefill_fused_workspace_bytes(ctypes.byref(cfg), n_seqs, n_tokens))


def gdn_prefill_fused(cfg: gdn_config, n_seqs: int, n_tokens: int, cu_seqlens, qkv, beta_logit, alpha_logit, z,
                      conv_w, dt_bias, A_log, norm_w, conv_state_in, conv_state_out, S_in, S_out, y, workspace,
                      stream=None):
    Hqk, Hv, d, N, T = cfg.n_qk_heads, cfg.n_v_heads, cfg.head_dim, n_seqs, n_tokens
    C, ad = d * (2 * Hqk + Hv), _act_dtype(cfg)
    ws = _ptr(workspace, "workspace", torch.uint8)
    s = load().gdn_prefill_fused(
        ctypes.byref(cfg), N, T, _ptr(cu_seqlens, "cu_seqlens", torch.int32, N + 1), _ptr(qkv, "qkv", ad, T * C),
        _ptr(beta_logit, "beta_logit", ad, T * Hv), _ptr(alpha_logit, "alpha_logit", ad, T * Hv),
        _ptr(z, "z", ad, T * Hv * d), _ptr(conv_w, "conv_w", torch.float32, C * CONV_K),
        _ptr(dt_bias, "dt_bias", torch.float32, Hv), _ptr(A_log, "A_log", torch.float32, Hv),
        _ptr(norm_w, "norm_w", torch.float32, d), _ptr(conv_state_in, "conv_state_in", ad, N * (CONV_K - 1) * C),
        _ptr(conv_state_out, "conv_state_out", ad, N * (CONV_K - 1) * C),
        _ptr(S_in, "S_in", torch.float32, N * Hv * d * d), _ptr(S_out, "S_out", torch.float32, N * Hv * d * d),
        _ptr(y, "y", ad, T * Hv * d), ws, workspace.numel() if workspace is not None else 0, _stream(stream))
    _check("gdn_prefill_fused", s)


def gdn_prefill_fused_ckpt(cfg: gdn_config, n_seqs: int, n_tokens: int, cu_seqlens, qkv, beta_logit, alpha_logit, z,
                           conv_w, dt_bias, A_log, norm_w, conv_state_in, conv_state_out, S_in, S_out, y,
                           ckpt_every: int, ckpt_cap: int, S_ckpt, conv_ckpt, workspace, stream=None):
    Hqk, Hv, d, N, T = cfg.n_qk_heads, cfg.n_v_heads, cfg.head_dim, n_seqs, n_tokens
    C, ad = d * (2 * Hqk + Hv), _act_dtype(cfg)
    ws = _ptr(workspace, "workspace", torch.uint8)
    s = load().gdn_prefill_fused_ckpt(
        ctypes.byref(cfg), N, T, _ptr(cu_seqlens, "cu_seqlens", torch.int32, N + 1), _ptr(qkv, "qkv", ad, T * C),
        _ptr(beta_logit, "beta_logit", ad, T * Hv), _ptr(alpha_logit, "alpha_logit", ad, T * Hv),
        _ptr(z, "z", ad, T * Hv * d), _ptr(conv_w, "conv_w", torch.float32, C * CONV_K),
        _ptr(dt_bias, "dt_bias", torch.float32, Hv), _ptr(A_log, "A_log", torch.float32, Hv),
        _ptr(norm_w, "norm_w", torch.float32, d), _ptr(conv_state_in, "conv_state_in", ad, N * (CONV_K - 1) * C),
        _ptr(conv_state_out, "conv_state_out", ad, N * (CONV_K - 1) * C),
        _ptr(S_in, "S_in", torch.float32, N * Hv * d * d), _ptr(S_out, "S_out", torch.float32, N * Hv * d * d),
        _ptr(y, "y", ad, T * Hv * d), ckpt_every, ckpt_cap,
        _ptr(S_ckpt, "S_ckpt", torch.float32, N * ckpt_cap * Hv * d * d),
        _ptr(conv_ckpt, "conv_ckpt", ad, N * ckpt_cap * (CONV_K - 1) * C),
        ws, workspace.numel() if workspace is not None else 0, _stream(stream))
    _check("gdn_prefill_fused_ckpt", s)


def gdn_prefill_fused_static(cfg: gdn_config, n_seqs: int, n_tokens: int, cu_seqlens, qkv, beta_logit, alpha_logit,
                             z, conv_w, dt_bias, A_log, norm_w, conv_state_in, conv_state_out, S_in, S_out, y,
                             stream=None):
    """gdn_prefill_fused with the library's static device scratch as its
    workspace: allocates nothing (GdnError with GDN_E_TOO_LARGE when the call
    needs more than GDN_STATIC_SCRATCH_BYTES)."""
    Hqk, Hv, d, N, T = cfg.n_qk_heads, cfg.n_v_heads, cfg.head_dim, n_seqs, n_tokens
    C, ad = d * (2 * Hqk + Hv), _act_dtype(cfg)
    s = load().gdn_prefill_fused_static(
        ctypes.byref(cfg), N, T, _ptr(cu_seqlens, "cu_seqlens", torch.int32, N + 1), _ptr(qkv, "qkv", ad, T * C),
        _ptr(beta_logit, "beta_logit", ad, T * Hv), _ptr(alpha_logit, "alpha_logit", ad, T * Hv),
        _ptr(z, "z", ad, T * Hv * d), _ptr(conv_w, "conv_w", torch.float32, C * CONV_K),
        _ptr(dt_bias, "dt_bias", torch.float32, Hv), _ptr(A_log, "A_log", torch.float32, Hv),
        _ptr(norm_w, "norm_w", torch.float32, d), _ptr(conv_state_in, "conv_state_in", ad, N * (CONV_K - 1) * C),
        _ptr(conv_state_out, "conv_state_out", ad, N * (CONV_K - 1) * C),
        _ptr(S_in, "S_in", torch.float32, N * Hv * d * d), _ptr(S_out, "S_out", torch.float32, N * Hv * d * d),
        _ptr(y, "y", ad, T * Hv * d), _stream(stream))
    _check("gdn_prefill_fused_static", s)


def gdn_in_proj(cfg: gdn_config, n_tokens: int, hidden: int, x, w_qkv, w_gate, w_beta, w_alpha, qkv, z,
                beta_logit, alpha_logit, stream=None):
    Hqk, Hv, d, T, bf = cfg.n_qk_heads, cfg.n_v_heads, cfg.head_dim, n_tokens, torch.bfloat16
    C = d * (2 * Hqk + Hv)
    s = load().gdn_in_proj(
        ctypes.byref(cfg), T, hidden, _ptr(x, "x", bf, T * hidden), _ptr(w_qkv, "w_qkv", bf, C * hidden),
        _ptr(w_gate, "w_gate", bf, Hv * d * hidden), _ptr(w_beta, "w_beta", bf, Hv * hidden),
        _ptr(w_alpha, "w_alpha", bf, Hv * hidden), _ptr(qkv, "qkv", bf, T * C), _ptr(z, "z", bf, T * Hv * d),
        _ptr(beta_logit, "beta_logit", bf, T * Hv), _ptr(alpha_logit, "alpha_logit", bf, T * Hv), _stream(stream))
    _check("gdn_in_proj", s)


def gdn_out_proj(cfg: gdn_config, n_tokens: int, hidden: int, y, w_out, out, stream=None):
    Hv, d, T, bf = cfg.n_v_heads, cfg.head_dim, n_tokens, torch.bfloat16
    s = load().gdn_out_proj(
        ctypes.byref(cfg), T, hidden, _ptr(y, "y", bf, T * Hv * d), _ptr(w_out, "w_out", bf, hidden * Hv * d),
        _ptr(out, "out", bf, T * hidden), _stream(stream))
    _check("gdn_out_proj", s)


__all__ = ["load", "make_config", "gdn_config", "GdnError", "status_string", "EXPORTS",
           "gdn_conv_gate_prep", "gdn_prefill_chunked", "gdn_prefill_workspace_bytes",
           "gdn_decode_step", "gdn_decode_fused", "gdn_decode_verify", "gdn_gated_rmsnorm",
           "gdn_prefill_chunked_ckpt", "gdn_conv_state_ckpt", "gdn_state_check", "gdn_in_proj",
           "gdn_out_proj", "gdn_prefill_fused", "gdn_prefill_fused_workspace_bytes", "gdn_prefill_fused_static",
           "gdn_prefill_fused_ckpt", "GDN_F32", "GDN_BF16", "GDN_STATIC_SCRATCH_BYTES"]
