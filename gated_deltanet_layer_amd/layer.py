"""Chained calls of the C ABI over preallocated device buffers.

``Prefill`` runs gdn_conv_gate_prep -> gdn_prefill_chunked -> gdn_gated_rmsnorm
over packed sequences; ``Decode`` runs gdn_conv_gate_prep -> gdn_decode_step ->
gdn_gated_rmsnorm for one token per sequence; ``DecodeFused`` runs the same
step as the single launch gdn_decode_fused. ``PrefillFused`` is the whole prefill
mixer as one gdn_prefill_fused call. ``Block`` and ``DecodeBlock`` put
gdn_in_proj before and gdn_out_proj after ``PrefillFused`` and
``DecodeFused`` (the whole token-mixer block from the layer input). Each allocates its intermediates
(q, k, v, beta, g, o, y, workspace, the second conv-state buffer) once with
torch and then only calls the library, so a timed loop allocates nothing.
"""
from __future__ import annotations

import torch

from . import binding as B


def _act(cfg):
    return torch.bfloat16 if cfg.act_dtype == B.GDN_BF16 else torch.float32


class Prefill:
    def __init__(self, cfg: B.gdn_config, n_seqs: int, n_tokens: int, device="cuda"):
        self.cfg, self.N, self.T = cfg, n_seqs, n_tokens
        Hqk, Hv, d = cfg.n_qk_heads, cfg.n_v_heads, cfg.head_dim
        f32 = dict(dtype=torch.float32, device=device)
        self.q = torch.empty(n_tokens, Hqk, d, **f32)
        self.k = torch.empty(n_tokens, Hqk, d, **f32)
        self.v = torch.empty(n_tokens, Hv, d, **f32)
        self.beta = torch.empty(n_tokens, Hv, **f32)
        self.g = torch.empty(n_tokens, Hv, **f32)
        self.o = torch.empty(n_tokens, Hv, d, dtype=_act(cfg), device=device)
        self.y = torch.empty(n_tokens, Hv, d, dtype=_act(cfg), device=device)
        wsb = B.gdn_prefill_workspace_bytes(cfg, n_seqs, n_tokens)
        self.ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=device) if wsb else None

    def prep(self, cu, qkv, b, a, conv_w, dt_bias, A_log, conv_in, conv_out, stream=None):
        B.gdn_conv_gate_prep(self.cfg, self.N, self.T, cu, qkv, b, a, conv_w, dt_bias, A_log,
                             conv_in, conv_out, self.q, self.k, self.v, self.beta, self.g, stream)

    def core(self, cu, S_in, S_out, stream=None):
        B.gdn_prefill_chunked(self.cfg, self.N, self.T, cu, self.q, self.k, self.v, self.beta, self.g,
                              S_in, S_out, self.o, self.ws, stream)

    def norm(self, z, norm_w, stream=None):
        B.gdn_gated_rmsnorm(self.cfg, self.T * self.cfg.n_v_heads, self.o, z, norm_w, self.y, stream)

    def __call__(self, cu, qkv, z, b, a, conv_w, dt_bias, A_log, norm_w, conv_in, conv_out, S_in, S_out,
                 stream=None):
        self.prep(cu, qkv, b, a, conv_w, dt_bias, A_log, conv_in, conv_out, stream)
        self.core(cu, S_in, S_out, stream)
        self.norm(z, norm_w, stream)
        return self.y


class PrefillFused:
    """The whole mixer over packed sequences in one gdn_prefill_fused call
    (q, k, v, beta and g are never stored); the workspace also holds o."""

    def __init__(self, cfg: B.gdn_config, n_seqs: int, n_tokens: int, device="cuda"):
        self.cfg, self.N, self.T = cfg, n_seqs, n_tokens
        Hv, d = cfg.n_v_heads, cfg.head_dim
        self.y = torch.empty(n_tokens, Hv, d, dtype=_act(cfg), device=device)
        wsb = B.gdn_prefill_fused_workspace_bytes(cfg, n_seqs, n_tokens)
        self.ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=device) if wsb else None

    def __call__(self, cu, qkv, z, b, a, conv_w, dt_bias, A_log, norm_w, conv_in, conv_out, S_in, S_out,
                 stream=None):
        B.gdn_prefill_fused(self.cfg, self.N, self.T, cu, qkv, b, a, z, conv_w, dt_bias, A_log, norm_w, conv_in,
                            conv_out, S_in, S_out, self.y, self.ws, stream)
        return self.y


class Decode:
    """One token for each of n_seqs sequences per call; states updated in place."""

    def __init__(self, cfg: B.gdn_config, n_seqs: int, device="cuda"):
        self.cfg, self.N = cfg, n_seqs
        Hqk, Hv, d = cfg.n_qk_heads, cfg.n_v_heads, cfg.head_dim
        f32 = dict(dtype=torch.float32, device=device)
        self.cu = torch.arange(n_seqs + 1, dtype=torch.int32, device=device)
        self.q = torch.empty(n_seqs, Hqk, d, **f32)
        self.k = torch.empty(n_seqs, Hqk, d, **f32)
        self.v = torch.empty(n_seqs, Hv, d, **f32)
        self.beta = torch.empty(n_seqs, Hv, **f32)
        self.g = torch.empty(n_seqs, Hv, **f32)
        self.o = torch.empty(n_seqs, Hv, d, dtype=_act(cfg), device=device)

    def __call__(self, qkv, z, b, a, conv_w, dt_bias, A_log, norm_w, conv_state, S, y, stream=None):
        cfg, N = self.cfg, self.N
        B.gdn_conv_gate_prep(cfg, N, N, self.cu, qkv, b, a, conv_w, dt_bias, A_log, conv_state, conv_state,
                             self.q, self.k, self.v, self.beta, self.g, stream)
        B.gdn_decode_step(cfg, N, self.q, self.k, self.v, self.beta, self.g, S, S, self.o, stream)
        B.gdn_gated_rmsnorm(cfg, N * cfg.n_v_heads, self.o, z, norm_w, y, stream)
        return y


class DecodeFused:
    """One token for each of n_seqs sequences per call, in one launch.

    gdn_decode_fused needs distinct old and new conv-state buffers, so the
    runner alternates between ``conv_state`` (given, used as the first
    buffer and overwritten) and a second buffer of its own;
    ``self.conv_state`` is the current one. S is updated in place."""

    def __init__(self, cfg: B.gdn_config, n_seqs: int, conv_state: torch.Tensor):
        self.cfg, self.N = cfg, n_seqs
        self.bufs = [conv_state, torch.empty_like(conv_state)]
        self.cur = 0

    @property
    def conv_state(self) -> torch.Tensor:
        return self.bufs[self.cur]

    def __call__(self, qkv, z, b, a, conv_w, dt_bias, A_log, norm_w, S, y, stream=None):
        src, dst = self.bufs[self.cur], self.bufs[1 - self.cur]
        B.gdn_decode_fused(self.cfg, self.N, qkv, b, a, z, conv_w, dt_bias, A_log, norm_w, src, dst, S, S, y,
                           stream)
        self.cur = 1 - self.cur
        return y


class _Proj:
    """Buffers of the projected streams and of the block output (bf16)."""

    def __init__(self, cfg: B.gdn_config, n_tokens: int, hidden: int, device):
        Hqk, Hv, d = cfg.n_qk_heads, cfg.n_v_heads, cfg.head_dim
        bf = dict(dtype=torch.bfloat16, device=device)
        self.hidden = hidden
        self.qkv = torch.empty(n_tokens, d * (2 * Hqk + Hv), **bf)
        self.z = torch.empty(n_tokens, Hv, d, **bf)
        self.b = torch.empty(n_tokens, Hv, **bf)
        self.a = torch.empty(n_tokens, Hv, **bf)
        self.out = torch.empty(n_tokens, hidden, **bf)

    def project_in(self, cfg, T, x, w_qkv, w_gate, w_beta, w_alpha, stream):
        B.gdn_in_proj(cfg, T, self.hidden, x, w_qkv, w_gate, w_beta, w_alpha, self.qkv, self.z, self.b, self.a,
                      stream)

    def project_out(self, cfg, T, y, w_out, stream):
        B.gdn_out_proj(cfg, T, self.hidden, y, w_out, self.out, stream)
        return self.out


class Block:
    """The block over packed sequences: gdn_in_proj -> gdn_prefill_fused -> gdn_out_proj."""

    def __init__(self, cfg: B.gdn_config, n_seqs: int, n_tokens: int, hidden: int, device="cuda"):
        self.cfg, self.T = cfg, n_tokens
        self.mixer = PrefillFused(cfg, n_seqs, n_tokens, device)
        self.proj = _Proj(cfg, n_tokens, hidden, device)

    def __call__(self, cu, x, w_qkv, w_gate, w_beta, w_alpha, w_out, conv_w, dt_bias, A_log, norm_w, conv_in,
                 conv_out, S_in, S_out, stream=None):
        P = self.proj
        P.project_in(self.cfg, self.T, x, w_qkv, w_gate, w_beta, w_alpha, stream)
        y = self.mixer(cu, P.qkv, P.z, P.b, P.a, conv_w, dt_bias, A_log, norm_w, conv_in, conv_out, S_in, S_out,
                       stream)
        return P.project_out(self.cfg, self.T, y, w_out, stream)


class DecodeBlock:
    """One token per sequence through the block: gdn_in_proj -> gdn_decode_fused
    -> gdn_out_proj (conv state handled as in ``DecodeFused``)."""

    def __init__(self, cfg: B.gdn_config, n_seqs: int, hidden: int, conv_state: torch.Tensor):
        self.cfg, self.N = cfg, n_seqs
        self.mixer = DecodeFused(cfg, n_seqs, conv_state)
        self.proj = _Proj(cfg, n_seqs, hidden, conv_state.device)
        self.y = torch.empty_like(self.proj.z)

    def __call__(self, x, w_qkv, w_gate, w_beta, w_alpha, w_out, conv_w, dt_bias, A_log, norm_w, S, stream=None):
        P = self.proj
        P.project_in(self.cfg, self.N, x, w_qkv, w_gate, w_beta, w_alpha, stream)
        self.mixer(P.qkv, P.z, P.b, P.a, conv_w, dt_bias, A_log, norm_w, S, self.y, stream)
        return P.project_out(self.cfg, self.N, self.y, w_out, stream)
