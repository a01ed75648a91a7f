"""Seeded synthetic workloads for the gated DeltaNet token mixer.

This module only draws random numbers and lays them out in the shapes the
mixer consumes. It holds none of the mixer's arithmetic: the oracle under
``oracle/`` and the HIP library both take what it returns, so that the two are
fed byte-identical inputs and never share any step of the computation.

Shapes follow the Qwen 3.6 hybrid layers as the xwen ``CLAUDE.md`` page
describes them (section "Architecture cheat sheet": 16 K-heads, 48 V-heads on
the 27B, 32 V-heads on the 35B-A3B, head dim 128, fused width
128 * (2 * H_qk + H_v), fp32 delta state, conv kernel 4).

Every buffer is drawn from its own counter-keyed PCG64 stream
(``SeedSequence([seed, stream_id])``), so truncating a workload to fewer
tokens or steps yields exactly the leading part of the full-size one.

Activation buffers are returned either as ``float32`` arrays (``act="f32"``)
or as ``uint16`` arrays holding bfloat16 bit patterns (``act="bf16"``),
rounded from float32 to nearest-even. Parameters and the delta state are
always ``float32``.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Sequence

import numpy as np

HEAD_DIM = 128
CONV_K = 4

# Stream ids: one independent PCG64 stream per buffer.
_STREAM = {
    "lengths": 1, "conv_w": 2, "norm_w": 3, "dt_bias": 4, "A_log": 5,
    "S0": 6, "conv0": 7, "qkv": 8, "z": 9, "b": 10, "a": 11,
    "x": 12, "w_qkv": 13, "w_gate": 14, "w_beta": 15, "w_alpha": 16, "w_out": 17, "y": 18,
}

# Hidden sizes of the two models' layer input (the page's section
# "Architecture cheat sheet": 5120 on the 27B, 2048 on the 35B-A3B).
HIDDEN = {48: 5120, 32: 2048}


@dataclass(frozen=True)
class Workload:
    """One synthetic problem.

    kind "prefill": ``lengths`` gives each packed sequence's token count.
    kind "decode": ``steps`` single-token steps for each of ``n_seqs``
    sequences; streams are laid out [steps, n_seqs, ...].
    """
    name: str
    kind: str                      # "prefill" | "decode"
    n_seqs: int
    n_qk_heads: int
    n_v_heads: int
    act: str                       # "f32" | "bf16"
    seed: int
    lengths: Optional[Sequence[int]] = None   # prefill only
    steps: int = 0                            # decode only
    s0_std: float = 0.0            # initial delta state ~ N(0, s0_std); 0 = zero
    conv0_std: float = 0.0         # initial conv state ~ N(0, conv0_std); 0 = zero
    head_dim: int = HEAD_DIM
    varlen_range: Optional[tuple] = None      # draw lengths ~ U{lo..hi} when set
    extra: dict = field(default_factory=dict)

    @property
    def conv_width(self) -> int:
        return self.head_dim * (2 * self.n_qk_heads + self.n_v_heads)

    @property
    def n_tokens(self) -> int:
        if self.kind == "decode":
            return self.steps * self.n_seqs
        return int(sum(self.seq_lengths()))

    def seq_lengths(self):
        if self.kind == "decode":
            return [self.steps] * self.n_seqs
        if self.lengths is not None:
            return list(self.lengths)
        lo, hi = self.varlen_range
        rng = _rng(self.seed, "lengths")
        return [int(x) for x in rng.integers(lo, hi, size=self.n_seqs, endpoint=True)]


def _rng(seed: int, stream: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _STREAM[stream]])))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (inputs finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f32(arr: np.ndarray, act: str) -> np.ndarray:
    """An activation buffer as exact float32 values."""
    return bf16_to_f32(arr) if act == "bf16" else np.ascontiguousarray(arr, dtype=np.float32)


def _normal(seed, stream, shape, mean=0.0, std=1.0) -> np.ndarray:
    x = _rng(seed, stream).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def _act(x: np.ndarray, act: str) -> np.ndarray:
    return bf16_bits(x) if act == "bf16" else x


def generate(w: Workload, max_tokens: Optional[int] = None,
             max_steps: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw every buffer of workload ``w``.

    ``max_tokens`` (prefill, single sequence only) or ``max_steps`` (decode)
    truncate the streams; the values drawn are the leading part of the
    full-size streams.

    Returns a dict with:
      conv_w [C,4] f32, norm_w [d] f32, dt_bias [Hv] f32, A_log [Hv] f32,
      S0 [N,Hv,d,d] f32, conv0 [N,3,C] act,
      prefill: qkv [T,C] act, z [T,Hv,d] act, b [T,Hv] act, a [T,Hv] act,
               cu_seqlens [N+1] int32
      decode:  qkv [S,N,C] act, z [S,N,Hv,d] act, b [S,N,Hv] act, a [S,N,Hv] act
    """
    N, Hv, d, C, act, seed = w.n_seqs, w.n_v_heads, w.head_dim, w.conv_width, w.act, w.seed
    out: Dict[str, np.ndarray] = {}
    out["conv_w"] = _normal(seed, "conv_w", (C, CONV_K), 0.0, 0.5)
    out["norm_w"] = _normal(seed, "norm_w", (d,), 1.0, 0.1)
    out["dt_bias"] = _rng(seed, "dt_bias").uniform(-1.0, 1.0, size=Hv).astype(np.float32)
    out["A_log"] = _rng(seed, "A_log").uniform(0.0, np.log(16.0), size=Hv).astype(np.float32)
    if w.s0_std > 0:
        out["S0"] = _normal(seed, "S0", (N, Hv, d, d), 0.0, w.s0_std)
    else:
        out["S0"] = np.zeros((N, Hv, d, d), np.float32)
    if w.conv0_std > 0:
        out["conv0"] = _act(_normal(seed, "conv0", (N, CONV_K - 1, C), 0.0, w.conv0_std), act)
    else:
        out["conv0"] = _act(np.zeros((N, CONV_K - 1, C), np.float32), act)

    if w.kind == "decode":
        S = w.steps if max_steps is None else min(w.steps, max_steps)
        lead = (S, N)
    else:
        lens = w.seq_lengths()
        if max_tokens is not None:
            if N != 1:
                raise ValueError("max_tokens truncation applies to single-sequence prefill")
            lens = [min(lens[0], max_tokens)]
        T = int(sum(lens))
        lead = (T,)
        out["cu_seqlens"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    # Streams are drawn in token (or step) major order from their own generators,
    # so a truncated draw is the leading slice of the full one.
    out["qkv"] = _act(_normal(seed, "qkv", lead + (C,)), act)
    out["z"] = _act(_normal(seed, "z", lead + (Hv, d)), act)
    out["b"] = _act(_normal(seed, "b", lead + (Hv,)), act)
    out["a"] = _act(_normal(seed, "a", lead + (Hv,)), act)
    return out


def generate_block(w: Workload, hidden: int, max_tokens: Optional[int] = None,
                   max_steps: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of the whole token-mixer block: ``generate(w)``'s parameters,
    states and cu_seqlens, plus the layer input and the projection weights
    (Linear layout, one row per output), all bf16 bit patterns:
      x [T, hidden] (decode: [S, N, hidden]) ~ N(0, 1)
      w_qkv [C, hidden], w_gate [Hv*d, hidden], w_beta, w_alpha [Hv, hidden]
        ~ N(0, 1/hidden), so that the projected streams are ~ N(0, 1) like
        the mixer's own synthetic inputs
      w_out [hidden, Hv*d] ~ N(0, 1/(Hv*d))
      y [T, Hv*d] ~ N(0, 1)   (ssm_out's input, for testing it on its own)
    The mixer streams qkv, z, b, a of ``generate`` are dropped: the block
    computes them from x."""
    if w.act != "bf16":
        raise ValueError("the projections take bf16 operands")
    out = generate(w, max_tokens=max_tokens, max_steps=max_steps)
    lead = out.pop("qkv").shape[:-1]
    for k in ("z", "b", "a"):
        out.pop(k)
    Hv, d, C, seed = w.n_v_heads, w.head_dim, w.conv_width, w.seed
    out["x"] = bf16_bits(_normal(seed, "x", lead + (hidden,)))
    s_in = 1.0 / np.sqrt(hidden)
    out["w_qkv"] = bf16_bits(_normal(seed, "w_qkv", (C, hidden), 0.0, s_in))
    out["w_gate"] = bf16_bits(_normal(seed, "w_gate", (Hv * d, hidden), 0.0, s_in))
    out["w_beta"] = bf16_bits(_normal(seed, "w_beta", (Hv, hidden), 0.0, s_in))
    out["w_alpha"] = bf16_bits(_normal(seed, "w_alpha", (Hv, hidden), 0.0, s_in))
    out["w_out"] = bf16_bits(_normal(seed, "w_out", (hidden, Hv * d), 0.0, 1.0 / np.sqrt(Hv * d)))
    # A stand-in for the mixer's output, to drive ssm_out on its own.
    out["y"] = bf16_bits(_normal(seed, "y", lead + (Hv * d,)))
    return out


# The five synthetic workloads (shapes of the Qwen 3.6 27B / 35B-A3B GDN layers).
WORKLOADS = {
    1: Workload("tiny single-chunk prefill T=64 Hqk=2 Hv=4 f32", "prefill", 1, 2, 4, "f32",
                seed=1, lengths=[64]),
    2: Workload("decode batch 1 Hqk=16 Hv=32 bf16 x1024 steps", "decode", 1, 16, 32, "bf16",
                seed=2, steps=1024, s0_std=0.02, conv0_std=1.0),
    3: Workload("prefill T=4096 Hqk=16 Hv=48 bf16", "prefill", 1, 16, 48, "bf16",
                seed=3, lengths=[4096]),
    4: Workload("batched decode 64 seqs Hqk=16 Hv=32 bf16 x256 steps", "decode", 64, 16, 32,
                "bf16", seed=4, steps=256, s0_std=0.02, conv0_std=1.0),
    5: Workload("varlen prefill 8 seqs L~U[512,8192] Hqk=16 Hv=48 bf16", "prefill", 8, 16, 48,
                "bf16", seed=5, varlen_range=(512, 8192), s0_std=0.02),
}


def custom(kind: str, n_seqs: int, n_qk_heads: int, n_v_heads: int, act: str, seed: int,
           lengths=None, steps: int = 0, s0_std: float = 0.0, conv0_std: float = 0.0,
           head_dim: int = HEAD_DIM, name: str = "custom") -> Workload:
    """A workload of the same distributions at any shape (for parity and edge cases)."""
    return Workload(name, kind, n_seqs, n_qk_heads, n_v_heads, act, seed, lengths=lengths,
                    steps=steps, s0_std=s0_std, conv0_std=conv0_std, head_dim=head_dim)


__all__ = ["Workload", "WORKLOADS", "generate", "generate_block", "HIDDEN", "custom", "bf16_bits", "bf16_to_f32", "as_f32",
           "HEAD_DIM", "CONV_K", "replace"]
