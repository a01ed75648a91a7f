"""Precision budget of the chunked delta rule: which products need fp32-grade
operands to meet the output tolerance.

A numpy emulation of the chunked form (the exact rewrite of the xwen
CLAUDE.md page's recurrent step over chunks of 64, section "Architecture
cheat sheet", gated DeltaNet paragraph) in which each product's operands can
be taken in one of three precisions, the choices a kernel on bf16 matrix
cores has:
  "f32"    operands as fp32 values (what fp32 MFMA, or an exact product, gets)
  "split"  each operand x as hi = bf16(x) plus lo = bf16(x - hi), the product
           formed as hi*hi + hi*lo + lo*hi (three bf16 passes; lo*lo dropped)
  "bf16"   each operand rounded once to bf16 (one pass)
Sums are exact (fp64) and each product's result is rounded to fp32, as an
fp32 accumulator holds it. o is rounded to bf16 as the prefill stores it, then
normalised by the gated RMSNorm in fp64, and y rounded to bf16 as stored.
The result is compared with the fp64 oracle at the bar of the bf16
workloads, |got - ref| <= 2e-3 + 1e-2 |ref|, as a worst ratio (<= 1 passes).

This file holds only the emulation; tests/test_precision_budget.py runs it.
It shares nothing with the HIP library.
"""
from __future__ import annotations

import math
from typing import Dict, Sequence

import numpy as np

from gated_deltanet_layer_amd import workloads as wl

CHUNK = 64
PRODUCTS = ("gram", "KS", "QS", "TmR", "PD", "KtD")


def _f32(x):
    return np.asarray(x, np.float32).astype(np.float64)


def _bf16(x):
    return wl.bf16_to_f32(wl.bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


def _operands(x, mode: str):
    """(hi, lo) parts of an operand in the given precision (lo None: one part)."""
    x32 = _f32(x)
    if mode == "f32":
        return x32, None
    hi = _bf16(x32)
    if mode == "bf16":
        return hi, None
    return hi, _bf16(x32 - hi)


def matmul(a, b, mode: str):
    """a @ b with both operands in `mode`, fp32 result."""
    ah, al = _operands(a, mode)
    bh, bl = _operands(b, mode)
    r = ah @ bh
    if al is not None:
        r = r + ah @ bl + al @ bh
    return _f32(r)


def chunked(q, k, v, beta, g, S0, n_qk: int, heads: Sequence[int], prec: Dict[str, str]):
    """o [T, len(heads), d] and S_end [len(heads), d, d] of one sequence.

    q, k [T, Hqk, d], v [T, Hv, d], beta, g [T, Hv], S0 [Hv, d, d] (fp64 values
    of what the kernel holds). prec maps each of PRODUCTS to a precision:
      gram  K K^T and Q K^T (the decay-masked A and P)
      KS    X = K S        QS  Y = Q S
      TmR   D = Tm (V - Gam X)
      PD    P D (the in-chunk part of the readout)
      KtD   K^T (k~ D) (the state update)
    The triangular solve and the decays are exact."""
    T, _, d = q.shape
    s = 1.0 / math.sqrt(d)
    o = np.zeros((T, len(heads), d))
    S_end = []
    for jj, j in enumerate(heads):
        hk = j % n_qk
        S = S0[j].astype(np.float64).copy()
        for c0 in range(0, T, CHUNK):
            c1 = min(T, c0 + CHUNK)
            n = c1 - c0
            K, Q, V = k[c0:c1, hk], q[c0:c1, hk], v[c0:c1, j]
            b = beta[c0:c1, j]
            gam = np.cumsum(g[c0:c1, j])
            lower = np.tril(np.ones((n, n), bool))
            strict = np.tril(np.ones((n, n), bool), -1)
            dec = np.where(lower, np.exp(np.where(lower, gam[:, None] - gam[None, :], 0.0)), 0.0)
            A = _f32(np.where(strict, b[:, None] * dec * matmul(K, K.T, prec["gram"]), 0.0))
            P = _f32(np.where(lower, dec * matmul(Q, K.T, prec["gram"]), 0.0))
            Tm = _f32(np.linalg.solve(np.eye(n) + A, np.diag(b)))
            G = np.exp(gam)
            X = matmul(K, S, prec["KS"])
            Y = matmul(Q, S, prec["QS"])
            R = _f32(V - G[:, None] * X)
            D = matmul(Tm, R, prec["TmR"])
            o[c0:c1, jj] = s * (G[:, None] * Y + matmul(P, D, prec["PD"]))
            kt = np.exp(gam[-1] - gam)
            S = _f32(G[-1] * S + matmul(K.T, kt[:, None] * D, prec["KtD"]))
        S_end.append(S)
    return o, np.array(S_end)


def bar_ratio(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref) / (2e-3 + 1e-2 * np.abs(ref))))


def budget_table(T: int = 1024, heads: Sequence[int] = (0, 7, 13, 22, 31, 40, 47), g_scale: float = 1.0,
                 only: Sequence[str] = None):
    """Worst y, o and S_out ratios for each precision variant, on the first T
    tokens of the 4,096-token prefill workload (16 K-heads, 48 V-heads, bf16
    inputs) and the given V-heads. g_scale != 1 multiplies every log-decay g
    (weaker decays carry the state further across chunks); the reference is
    then the oracle's recurrence on those gates. `only` restricts the
    variants computed."""
    import oracle
    w = wl.WORKLOADS[3]
    x = wl.generate(w, max_tokens=T)
    X = {key: (wl.as_f32(v, w.act).astype(np.float64) if key in ("qkv", "z", "b", "a", "conv0") else v)
         for key, v in x.items()}
    Hqk, Hv, d = w.n_qk_heads, w.n_v_heads, w.head_dim
    heads = list(heads)
    orc = oracle.default()
    ref = orc.layer(X["cu_seqlens"], Hqk, Hv, d, X["qkv"], X["z"], X["b"], X["a"], X["conv_w"], X["dt_bias"],
                    X["A_log"], X["norm_w"], X["conv0"], X["S0"], heads=heads)
    z = X["z"].reshape(T, Hv, d)[:, heads]
    beta, g = _f32(ref["beta"]), _f32(_f32(ref["g"]) * g_scale)
    if g_scale != 1.0:
        o_ref, S_ref = orc.delta_rule(X["cu_seqlens"], Hqk, Hv, d, ref["q"], ref["k"], ref["v"], ref["beta"], g,
                                      X["S0"], heads=heads)
        ref["o"], ref["S_out"] = o_ref, S_ref
        ref["y"] = np.full_like(o_ref, np.nan)
        ref["y"][:, heads] = orc.gated_rmsnorm(o_ref[:, heads], z, X["norm_w"])
    ref_o, ref_y, ref_S = ref["o"][:, heads], ref["y"][:, heads], ref["S_out"][0][heads]
    S0 = X["S0"][0]
    f32_qkv = (_f32(ref["q"]), _f32(ref["k"]), _f32(ref["v"]))
    bf_qkv = (_bf16(ref["q"]), _bf16(ref["k"]), _bf16(ref["v"]))
    split_all = {p: "split" for p in PRODUCTS}
    variants = {
        "fp32 operands everywhere": (f32_qkv, {p: "f32" for p in PRODUCTS}),
        "split bf16 everywhere": (f32_qkv, split_all),
        "one bf16 pass everywhere": (f32_qkv, {p: "bf16" for p in PRODUCTS}),
        "q, k, v stored in bf16 (products split)": (bf_qkv, split_all),
    }
    for p in PRODUCTS:
        variants[f"one bf16 pass on {p} only"] = (f32_qkv, dict(split_all, **{p: "bf16"}))
    out = {}
    for name, ((q, k, v), prec) in variants.items():
        if only is not None and name not in only:
            continue
        o, S = chunked(q, k, v, beta, g, S0, Hqk, heads, prec)
        ob = _bf16(o)
        y = _bf16(orc.gated_rmsnorm(ob, z, X["norm_w"]))
        out[name] = {"y": bar_ratio(y, ref_y), "o": bar_ratio(ob, ref_o), "S_out": bar_ratio(S, ref_S)}
    return out


if __name__ == "__main__":
    # from the repository root: python3 -m tests.precision_budget
    for name, r in budget_table().items():
        print(f"{name:45s} y {r['y']:8.3f}  o {r['o']:8.3f}  S_out {r['S_out']:8.3f}")
