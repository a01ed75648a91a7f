"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each ``pin_*(orc)`` raises AssertionError when the oracle ``orc`` disagrees with
what the xwen CLAUDE.md page (section "Architecture cheat sheet", gated
DeltaNet paragraph) and the mathematics fix: a hand-worked example, closed
forms, algebraically different formulations (the chunked form, the dense
transition matrix), library routines for the special cases that reduce to
one, and invariants (packing, continuation, head map).

The pins are plain functions so that ``test_oracle_mutants.py`` can run them
against deliberately broken builds of the oracle and show that every
plausible mistake trips at least one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from gated_deltanet_layer_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers
def _unit_rows(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _core_inputs(seed, T, Hqk, Hv, d, N=1, s0=0.3, g_scale=0.3):
    """Random delta-rule inputs (unit q/k, beta in (0,1), g <= 0)."""
    rng = np.random.default_rng(seed)
    q = _unit_rows(rng, (T, Hqk, d))
    k = _unit_rows(rng, (T, Hqk, d))
    v = rng.standard_normal((T, Hv, d))
    beta = rng.uniform(0.05, 0.95, (T, Hv))
    g = -g_scale * rng.uniform(0.0, 2.0, (T, Hv))
    S0 = s0 * rng.standard_normal((N, Hv, d, d))
    return q, k, v, beta, g, S0


def _layer_inputs(seed, lengths, Hqk, Hv, d, s0_std=0.02, conv0_std=1.0):
    w = wl.custom("prefill", len(lengths), Hqk, Hv, "f32", seed, lengths=lengths,
                  s0_std=s0_std, conv0_std=conv0_std, head_dim=d)
    x = wl.generate(w)
    return {k: (v.astype(np.float64) if v.dtype != np.int32 else v) for k, v in x.items()}


def _run_layer(orc, x, Hqk, Hv, d, heads=None):
    return orc.layer(x["cu_seqlens"], Hqk, Hv, d, x["qkv"], x["z"], x["b"], x["a"], x["conv_w"],
                     x["dt_bias"], x["A_log"], x["norm_w"], x["conv0"], x["S0"], heads=heads)


def _close(a, b, rtol, what, atol=0.0):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(np.max(np.abs(b)) if b.size else 0.0, 1e-300)
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= rtol * scale + atol, f"{what}: max err {err:.3e} vs scale {scale:.3e}"


def _chunked_fp64(q, k, v, beta, g, S0, Hqk, CH=64):
    """The chunked (WY/UT) form of the delta rule, one sequence, in fp64 numpy.

    Derived from the recurrent step alone: within a chunk of n tokens with
    cumulative log-decay gam, the deltas D solve (I + A) D = diag(beta) (V -
    diag(exp(gam)) K S0) with A[r][m] = beta_r exp(gam_r - gam_m) k_r.k_m for
    m < r; the outputs are s (diag(exp(gam)) Q S0 + (M o Q K^T) D) with M the
    lower-inclusive decay mask, and the chunk-end state is exp(gam_n) S0 +
    (diag(exp(gam_n - gam)) K)^T D.
    """
    T, Hv, d = v.shape
    s = 1.0 / math.sqrt(d)
    o = np.zeros((T, Hv, d))
    S_out = np.zeros((Hv, d, d))
    for j in range(Hv):
        S = S0[j].copy()
        hk = j % Hqk
        for c0 in range(0, T, CH):
            c1 = min(T, c0 + CH)
            K, Q, V = k[c0:c1, hk], q[c0:c1, hk], v[c0:c1, j]
            b, gam = beta[c0:c1, j], np.cumsum(g[c0:c1, j])
            n = c1 - c0
            diff = gam[:, None] - gam[None, :]
            low_strict = np.tril(np.ones((n, n), bool), -1)
            low_incl = np.tril(np.ones((n, n), bool), 0)
            Mdec = np.where(low_incl, np.exp(np.where(low_incl, diff, 0.0)), 0.0)
            A = np.where(low_strict, b[:, None] * Mdec * (K @ K.T), 0.0)
            P = np.where(low_incl, Mdec * (Q @ K.T), 0.0)
            G = np.exp(gam)
            rhs = b[:, None] * (V - G[:, None] * (K @ S))
            D = np.linalg.solve(np.eye(n) + A, rhs)
            o[c0:c1, j] = s * (G[:, None] * (Q @ S) + P @ D)
            S = G[-1] * S + (np.exp(gam[-1] - gam)[:, None] * K).T @ D
        S_out[j] = S
    return o, S_out


# -------------------------------------------------------------------- pins
def pin_hand_worked_d2(orc):
    """Two steps at d=2 worked by hand (tests/golden/hand_d2.json)."""
    with open(os.path.join(GOLDEN, "hand_d2.json")) as f:
        ex = json.load(f)
    toks = ex["tokens"]
    T = len(toks)
    q = np.array([t["q"] for t in toks]).reshape(T, 1, 2)
    k = np.array([t["k"] for t in toks]).reshape(T, 1, 2)
    v = np.array([t["v"] for t in toks]).reshape(T, 1, 2)
    beta = np.array([[t["beta"]] for t in toks])
    g = np.full((T, 1), -math.log(2.0))
    S0 = np.array(ex["S0"]).reshape(1, 1, 2, 2)
    o, S = orc.delta_rule([0, T], 1, 1, 2, q, k, v, beta, g, S0)
    _close(o[:, 0] * math.sqrt(2.0), ex["expected"]["o_times_sqrt2"], 1e-14, "hand o")
    _close(S[0, 0], ex["expected"]["S_final"], 1e-14, "hand S")


def pin_chunked_equals_recurrent(orc):
    """The chunked form (several chunks and a ragged tail) reaches the same result."""
    for (T, d, seed) in ((150, 16, 11), (70, 128, 12)):
        Hqk, Hv = 2, 4
        q, k, v, beta, g, S0 = _core_inputs(seed, T, Hqk, Hv, d)
        o, S = orc.delta_rule([0, T], Hqk, Hv, d, q, k, v, beta, g, S0)
        oc, Sc = _chunked_fp64(q, k, v, beta, g, S0[0], Hqk)
        _close(o, oc, 1e-11, f"chunked o T={T} d={d}")
        _close(S[0], Sc, 1e-11, f"chunked S T={T} d={d}")


def pin_dense_transition(orc):
    """S_t = e^g (I - beta k k^T) S_{t-1} + beta k v^T with explicit matrices; o = s S_t^T q."""
    T, Hqk, Hv, d = 9, 2, 4, 8
    q, k, v, beta, g, S0 = _core_inputs(21, T, Hqk, Hv, d)
    o, S = orc.delta_rule([0, T], Hqk, Hv, d, q, k, v, beta, g, S0)
    for j in range(Hv):
        M = S0[0, j].copy()
        hk = j % Hqk
        for t in range(T):
            kk = k[t, hk][:, None]
            M = math.exp(g[t, j]) * (np.eye(d) - beta[t, j] * kk @ kk.T) @ M \
                + beta[t, j] * kk @ v[t, j][None, :]
            _close(o[t, j], M.T @ q[t, hk] / math.sqrt(d), 1e-12, f"dense o t={t} j={j}")
        _close(S[0, j], M, 1e-12, f"dense S j={j}")


def pin_beta_zero_pure_decay(orc):
    """beta = 0: S_T = exp(sum g) S0 and o_t = (1/sqrt d) e^{gamma_t} S0^T q_t."""
    T, Hqk, Hv, d = 20, 2, 4, 16
    q, k, v, _, _, S0 = _core_inputs(31, T, Hqk, Hv, d)
    beta = np.zeros((T, Hv))
    g = np.full((T, Hv), -math.log(2.0))
    o, S = orc.delta_rule([0, T], Hqk, Hv, d, q, k, v, beta, g, S0)
    _close(S[0], S0[0] * 0.5 ** T, 1e-13, "pure decay S")
    for t in range(T):
        for j in range(Hv):
            exp_o = 0.5 ** (t + 1) * S0[0, j].T @ q[t, j % Hqk] / math.sqrt(d)
            _close(o[t, j], exp_o, 1e-12, f"readout scale t={t}")


def pin_unit_key_reads_back_v(orc):
    """g = 0, beta = 1, |k| = 1: after the update S^T k = v; with q = k, o = v / sqrt(d)."""
    T, Hqk, Hv, d = 5, 1, 2, 32
    _, k, v, _, _, S0 = _core_inputs(41, T, Hqk, Hv, d, s0=1.0)
    o, S = orc.delta_rule([0, T], Hqk, Hv, d, k, k, v, np.ones((T, Hv)), np.zeros((T, Hv)), S0)
    _close(o * math.sqrt(d), v, 1e-13, "read back v")
    for j in range(Hv):
        _close(S[0, j].T @ k[-1, 0], v[-1, j], 1e-13, "S^T k = v")


def pin_single_token_zero_state(orc):
    """One token from S0 = 0: S1 = beta k v^T and o = s beta (k.q) v."""
    Hqk, Hv, d = 2, 4, 64
    q, k, v, beta, g, _ = _core_inputs(51, 1, Hqk, Hv, d)
    o, S = orc.delta_rule([0, 1], Hqk, Hv, d, q, k, v, beta, g, np.zeros((1, Hv, d, d)))
    for j in range(Hv):
        hk = j % Hqk
        _close(S[0, j], beta[0, j] * np.outer(k[0, hk], v[0, j]), 1e-14, "S1")
        _close(o[0, j], beta[0, j] * (k[0, hk] @ q[0, hk]) * v[0, j] / math.sqrt(d), 1e-13, "o1")


def pin_scalar_functions(orc):
    """sigmoid and softplus at exact points and through identities; SiLU's identity."""
    assert orc.sigmoid(0.0) == 0.5
    assert abs(orc.softplus(0.0) - math.log(2.0)) <= 1e-16
    for x in (-30.0, -3.7, -0.25, 0.5, 2.0, 17.0, 40.0):
        assert abs(orc.sigmoid(x) + orc.sigmoid(-x) - 1.0) <= 2e-16, x
        assert abs(orc.softplus(x) - orc.softplus(-x) - x) <= 4e-15 * max(1.0, abs(x)), x
        assert abs(orc.silu(x) - orc.silu(-x) - x) <= 4e-15 * max(1.0, abs(x)), x
    # Far tails: softplus(x) -> x, softplus(-x) -> e^-x; both finite, no overflow.
    assert orc.softplus(800.0) == 800.0
    assert 0.0 <= orc.softplus(-800.0) < 1e-300
    assert abs(orc.softplus(-30.0) / math.exp(-30.0) - 1.0) < 1e-12
    assert orc.sigmoid(-800.0) == 0.0 and orc.sigmoid(800.0) == 1.0


def _prep(orc, x, Hqk, Hv, d, l2_mode=0):
    return orc.conv_gate_prep(x["cu_seqlens"], Hqk, Hv, d, x["qkv"], x["b"], x["a"], x["conv_w"],
                              x["dt_bias"], x["A_log"], x["conv0"], l2_mode=l2_mode)


def pin_conv_against_library_correlation(orc):
    """Conv + SiLU per channel equals numpy's correlation over [state; x] then x*sigmoid(x)."""
    Hqk, Hv, d = 1, 2, 8
    x = _layer_inputs(61, [13], Hqk, Hv, d)
    r = _prep(orc, x, Hqk, Hv, d)
    C = d * (2 * Hqk + Hv)
    Xt = np.concatenate([x["conv0"][0], x["qkv"]], axis=0)   # [3+L, C]
    conv = np.stack([np.correlate(Xt[:, c], x["conv_w"][c], mode="valid") for c in range(C)], 1)
    act = conv / (1.0 + np.exp(-conv))
    _close(r["v"].reshape(13, -1), act[:, 2 * d * Hqk:], 1e-14, "v = silu(conv)")
    qraw = act[:, :d * Hqk].reshape(13, Hqk, d)
    _close(r["q"], qraw / np.linalg.norm(qraw, axis=-1, keepdims=True), 1e-14, "q")
    kraw = act[:, d * Hqk:2 * d * Hqk].reshape(13, Hqk, d)
    _close(r["k"], kraw / np.linalg.norm(kraw, axis=-1, keepdims=True), 1e-14, "k")


def pin_conv_taps_and_state(orc):
    """One-hot taps: tap 3 is the current token, tap 0 three back (into the state);
    the new conv state is the last 3 raw rows of [state; x] for every length."""
    Hqk, Hv, d = 1, 1, 4
    C = d * 3
    for L in (0, 1, 2, 3, 5):
        x = _layer_inputs(70 + L, [L], Hqk, Hv, d)
        Xt = np.concatenate([x["conv0"][0], x["qkv"]], axis=0)
        for tap in range(4):
            x["conv_w"] = np.zeros((C, 4))
            x["conv_w"][:, tap] = 1.0
            r = _prep(orc, x, Hqk, Hv, d)
            _close(r["conv_out"][0], Xt[L:L + 3], 0.0, f"conv state L={L}")
            src = Xt[tap:tap + L, 2 * d:]     # the raw rows the v channels must see
            _close(r["v"].reshape(L, d), src / (1.0 + np.exp(-src)), 1e-15, f"tap {tap} L={L}")


def pin_zero_conv_weights(orc):
    """conv_w = 0: q = k = v = 0 (the clamp keeps them finite), S decays, o = 0, y = 0."""
    Hqk, Hv, d = 2, 4, 16
    x = _layer_inputs(81, [7], Hqk, Hv, d, s0_std=0.5)
    x["conv_w"][:] = 0.0
    r = _run_layer(orc, x, Hqk, Hv, d)
    for name in ("q", "k", "v", "o", "y"):
        assert np.all(r[name] == 0.0), name
    decay = np.exp(r["g"].sum(axis=0))          # [Hv]
    _close(r["S_out"][0], x["S0"][0] * decay[:, None, None], 1e-13, "decay only")


def pin_l2_clamp(orc):
    """x / max(|x|, 1e-6): a zero head maps to 0, a tiny head to silu(x)/1e-6 (not unit),
    a head of norm between 1e-6 and 1e-3 and an ordinary head to unit vectors."""
    Hqk, Hv, d = 4, 3, 8
    x = _layer_inputs(91, [1], Hqk, Hv, d)
    C = d * (2 * Hqk + Hv)
    x["conv_w"] = np.zeros((C, 4))
    x["conv_w"][:, 3] = 1.0                       # identity conv, then silu
    x["qkv"][0, 0:d] = 0.0                        # q head 0: zero
    x["qkv"][0, d:2 * d] = 1e-9 * np.arange(1, d + 1)   # q head 1: |silu(x)| ~ 1e-8 < eps
    x["qkv"][0, 3 * d:4 * d] = 2e-5 * np.arange(1, d + 1)  # q head 3: |silu(x)| ~ 1.4e-4
    r = _prep(orc, x, Hqk, Hv, d)
    assert np.all(r["q"][0, 0] == 0.0)
    assert abs(np.linalg.norm(r["q"][0, 3]) - 1.0) < 1e-14
    tiny = 1e-9 * np.arange(1, d + 1)
    # silu(x) = x/2 + x^2/4 + O(x^4): for |x| <= 1e-8 this is x/2 to 1e-9 relative.
    _close(r["q"][0, 1], (tiny / 2.0) / 1e-6, 1e-8, "tiny head divided by eps")
    assert abs(np.linalg.norm(r["q"][0, 2]) - 1.0) < 1e-14
    assert np.allclose(np.linalg.norm(r["k"][0], axis=-1), 1.0, atol=1e-14)


def pin_l2_rsqrt_form(orc):
    """The HF form x / sqrt(sum x^2 + 1e-6): zero head -> 0; a head of 8 equal
    entries s with 8 s^2 = 1e-6 -> every entry s / sqrt(2e-6) = 1/4 exactly
    (the clamp form would give 1/sqrt(8)); an O(1) head -> x / |x| shrunk by
    the factor 1 / sqrt(1 + 1e-6 / |x|^2)."""
    Hqk, Hv, d = 3, 3, 8
    x = _layer_inputs(93, [1], Hqk, Hv, d)
    C = d * (2 * Hqk + Hv)
    x["conv_w"] = np.zeros((C, 4))
    x["conv_w"][:, 3] = 1.0                       # identity conv, then silu
    s_target = 1e-3 / math.sqrt(8.0)
    c = 2.0 * s_target                            # solve silu(c) = s_target by Newton steps
    for _ in range(60):
        sg = 1.0 / (1.0 + math.exp(-c))
        c -= (c * sg - s_target) / (sg + c * sg * (1.0 - sg))
    x["qkv"][0, 0:d] = 0.0                        # q head 0: zero
    x["qkv"][0, d:2 * d] = c                      # q head 1: 8 x s_target
    x["qkv"][0, 2 * d:3 * d] = 3.0                # q head 2: silu(3) each
    r = _prep(orc, x, Hqk, Hv, d, l2_mode=1)
    assert np.all(r["q"][0, 0] == 0.0)
    _close(r["q"][0, 1], np.full(d, 0.25), 1e-12, "8 s with 8 s^2 = eps")
    s3 = 3.0 / (1.0 + math.exp(-3.0))
    _close(r["q"][0, 2], np.full(d, s3 / math.sqrt(d * s3 * s3 + 1e-6)), 1e-14, "O(1) head")
    assert abs(r["q"][0, 2, 0] - 1.0 / math.sqrt(d)) > 1e-9      # eps is felt even here
    rc = _prep(orc, x, Hqk, Hv, d)
    _close(rc["q"][0, 1], np.full(d, 1.0 / math.sqrt(d)), 1e-12, "clamp form on the same head")
    for name in ("v", "beta", "g"):
        assert np.array_equal(r[name], rc[name]), name


def pin_gates(orc):
    """beta = sigmoid(b); g = -exp(A_log) softplus(a + dt_bias), per V-head index."""
    Hqk, Hv, d = 1, 4, 4
    x = _layer_inputs(101, [3], Hqk, Hv, d)
    x["b"][:] = 0.0
    x["A_log"] = np.log(np.array([1.0, 2.0, 4.0, 8.0]))
    x["dt_bias"] = np.array([0.0, 1.0, -2.0, 3.0])
    x["a"] = -x["dt_bias"][None, :].repeat(3, 0)  # a + dt_bias = 0 -> softplus = ln 2
    x["a"][2, 1] = 800.0 - 1.0                    # a + dt_bias = 800 -> softplus = 800
    r = _prep(orc, x, Hqk, Hv, d)
    assert np.all(r["beta"] == 0.5)
    exp_g = -np.array([1.0, 2.0, 4.0, 8.0])[None, :] * math.log(2.0) * np.ones((3, 1))
    exp_g[2, 1] = -2.0 * 800.0
    _close(r["g"], exp_g, 1e-15, "g")
    x["b"] = np.array([[-2.0, -1.0, 1.0, 2.0]] * 3)
    r2 = _prep(orc, x, Hqk, Hv, d)
    _close(r2["beta"] + r2["beta"][:, ::-1], np.ones((3, 4)), 1e-15, "sigmoid symmetry")
    assert np.all(np.diff(r2["beta"], axis=1) > 0)


def pin_gated_rmsnorm_closed_forms(orc):
    """o = c*1: y = c/sqrt(c^2 + eps) w silu(z); z = 0: y = 0; mean, not sum, of squares."""
    d = 128
    rng = np.random.default_rng(111)
    w = rng.normal(1.0, 0.1, d)
    z = rng.standard_normal((3, d))
    c = np.array([0.5, -2.0, 1e-4])
    o = c[:, None] * np.ones((3, d))
    y = orc.gated_rmsnorm(o, z, w)
    sz = z / (1.0 + np.exp(-z))
    _close(y, (c / np.sqrt(c * c + 1e-6))[:, None] * w[None] * sz, 1e-14, "constant row")
    assert np.all(orc.gated_rmsnorm(o, np.zeros((3, d)), w) == 0.0)
    # A one-hot row: mean(o^2) = a^2/d, so y at the hot index is a/sqrt(a^2/d + eps) w silu(z).
    oh = np.zeros((1, d))
    oh[0, 5] = 3.0
    y1 = orc.gated_rmsnorm(oh, z[:1], w)
    exp = 3.0 / math.sqrt(9.0 / d + 1e-6) * w[5] * sz[0, 5]
    assert abs(y1[0, 5] - exp) <= 1e-13 * abs(exp)
    assert np.all(np.delete(y1[0], 5) == 0.0)


def pin_head_map_tiled(orc):
    """Perturbing K-head h changes exactly the V-heads j with j mod Hqk == h."""
    Hqk, Hv, d = 3, 6, 8
    x = _layer_inputs(121, [9], Hqk, Hv, d)
    base = _run_layer(orc, x, Hqk, Hv, d)
    for h in range(Hqk):
        for part in (0, 1):                        # q block, then k block
            x2 = {k: v.copy() for k, v in x.items()}
            c0 = part * d * Hqk + h * d
            x2["qkv"][:, c0:c0 + d] += 0.5
            r = _run_layer(orc, x2, Hqk, Hv, d)
            changed = [j for j in range(Hv) if not np.array_equal(r["o"][:, j], base["o"][:, j])]
            assert changed == [j for j in range(Hv) if j % Hqk == h], (h, part, changed)
            other = (r["k"] if part == 0 else r["q"])
            assert np.array_equal(other, base["k"] if part == 0 else base["q"])
            assert np.array_equal(r["beta"], base["beta"]) and np.array_equal(r["g"], base["g"])


def pin_split_order(orc):
    """Fused width is q | k | v: perturbing v channels of head j changes only v_j."""
    Hqk, Hv, d = 2, 4, 8
    x = _layer_inputs(131, [4], Hqk, Hv, d)
    base = _prep(orc, x, Hqk, Hv, d)
    x["qkv"][:, 2 * d * Hqk + 2 * d: 2 * d * Hqk + 3 * d] += 1.0
    r = _prep(orc, x, Hqk, Hv, d)
    assert np.array_equal(r["q"], base["q"]) and np.array_equal(r["k"], base["k"])
    changed = [j for j in range(Hv) if not np.array_equal(r["v"][:, j], base["v"][:, j])]
    assert changed == [2], changed


def pin_varlen_packing(orc):
    """Packed sequences give bit-identical results to separate runs."""
    Hqk, Hv, d = 2, 4, 16
    lens = [5, 0, 17, 2]
    x = _layer_inputs(141, lens, Hqk, Hv, d)
    packed = _run_layer(orc, x, Hqk, Hv, d)
    cu = x["cu_seqlens"]
    for n, L in enumerate(lens):
        sl = slice(cu[n], cu[n + 1])
        xs = dict(x)
        xs.update(cu_seqlens=np.array([0, L], np.int32), qkv=x["qkv"][sl], z=x["z"][sl],
                  b=x["b"][sl], a=x["a"][sl], conv0=x["conv0"][n:n + 1], S0=x["S0"][n:n + 1])
        one = _run_layer(orc, xs, Hqk, Hv, d)
        for name in ("q", "k", "v", "beta", "g", "o", "y"):
            assert np.array_equal(one[name], packed[name][sl]), (name, n)
        assert np.array_equal(one["S_out"][0], packed["S_out"][n])
        assert np.array_equal(one["conv_out"][0], packed["conv_out"][n])


def pin_split_continuation(orc):
    """Running [0,T1) then [T1,T) with both states carried equals one run over [0,T)."""
    Hqk, Hv, d = 2, 4, 16
    T = 130
    x = _layer_inputs(151, [T], Hqk, Hv, d)
    whole = _run_layer(orc, x, Hqk, Hv, d)
    for T1 in (1, 2, 63, 64, 65):
        a_, b_ = slice(0, T1), slice(T1, T)
        xa = dict(x, cu_seqlens=np.array([0, T1], np.int32), qkv=x["qkv"][a_], z=x["z"][a_],
                  b=x["b"][a_], a=x["a"][a_])
        ra = _run_layer(orc, xa, Hqk, Hv, d)
        xb = dict(x, cu_seqlens=np.array([0, T - T1], np.int32), qkv=x["qkv"][b_], z=x["z"][b_],
                  b=x["b"][b_], a=x["a"][b_], conv0=ra["conv_out"], S0=ra["S_out"])
        rb = _run_layer(orc, xb, Hqk, Hv, d)
        assert np.array_equal(np.concatenate([ra["y"], rb["y"]]), whole["y"]), T1
        assert np.array_equal(rb["S_out"], whole["S_out"]), T1
        assert np.array_equal(rb["conv_out"], whole["conv_out"]), T1


def pin_head_subset(orc):
    """Computing a subset of V-heads gives the same values as computing all of them."""
    Hqk, Hv, d = 2, 6, 16
    x = _layer_inputs(161, [11, 6], Hqk, Hv, d)
    full = _run_layer(orc, x, Hqk, Hv, d)
    sub = _run_layer(orc, x, Hqk, Hv, d, heads=[1, 4])
    for name in ("o", "y"):
        assert np.array_equal(sub[name][:, [1, 4]], full[name][:, [1, 4]])
        assert np.all(np.isnan(sub[name][:, [0, 2, 3, 5]]))
    assert np.array_equal(sub["S_out"][:, [1, 4]], full["S_out"][:, [1, 4]])


# ------------------------------------------------------------ projections
def pin_linear_hand_worked(orc):
    """y = x W^T on integers, worked by hand: row (1, 2) against weight rows
    (3, 4), (5, 6), (7, 8) gives 11, 17, 23; row (3, -1) gives 5, 9, 13."""
    x = np.array([[1.0, 2.0], [3.0, -1.0]])
    W = np.array([[3.0, 4.0], [5.0, 6.0], [7.0, 8.0]])
    y = orc.linear(x, W)
    assert np.array_equal(y, np.array([[11.0, 17.0, 23.0], [5.0, 9.0, 13.0]])), y


def pin_linear_library(orc):
    """A non-square product against numpy's matmul of x and W^T."""
    rng = np.random.default_rng(171)
    x = rng.standard_normal((7, 13))
    W = rng.standard_normal((5, 13))
    _close(orc.linear(x, W), x @ W.T, 1e-13, "linear")


def pin_in_proj_routing(orc):
    """Each of the four projections takes its own weight: with identity
    blocks as weights, qkv, z, b and a are the matching slices of x; with
    random weights each equals numpy's product with its weight."""
    Hqk, Hv, d = 1, 2, 4
    C = d * (2 * Hqk + Hv)
    widths = [C, Hv * d, Hv, Hv]
    hidden = sum(widths)
    rng = np.random.default_rng(172)
    x = rng.standard_normal((5, hidden))
    eye = np.eye(hidden)
    cuts = np.cumsum([0] + widths)
    ws = [eye[cuts[i]:cuts[i + 1]] for i in range(4)]
    r = orc.in_proj(Hqk, Hv, d, x, *ws)
    for i, name in enumerate(("qkv", "z", "b", "a")):
        assert np.array_equal(r[name].reshape(5, -1), x[:, cuts[i]:cuts[i + 1]]), name
    ws = [rng.standard_normal((w, hidden)) for w in widths]
    r = orc.in_proj(Hqk, Hv, d, x, *ws)
    for i, name in enumerate(("qkv", "z", "b", "a")):
        _close(r[name].reshape(5, -1), x @ ws[i].T, 1e-13, name)


def pin_round_bf16(orc):
    """bf16 rounding: hand-worked ties to even at 8 significant bits, and
    agreement with the integer bit-pattern rounding of fp32 values."""
    import oracle
    u = 2.0 ** -8
    cases = {1.0 + u: 1.0, 1.0 + 3 * u: 1.0 + 4 * u, 1.0 + u + 2.0 ** -20: 1.0 + 2 * u,
             -(1.0 + u): -1.0, 0.0: 0.0, 3.0: 3.0, 255.5: 256.0, 2.0 ** -100 * 1.5: 2.0 ** -100 * 1.5}
    for x, want in cases.items():
        got = float(oracle.round_bf16(np.array([x]))[0])
        assert got == want, (x, got, want)
    rng = np.random.default_rng(173)
    v = (rng.standard_normal(4096) * np.exp(rng.uniform(-20, 20, 4096))).astype(np.float32)
    ref = wl.bf16_to_f32(wl.bf16_bits(v)).astype(np.float64)
    assert np.array_equal(oracle.round_bf16(v.astype(np.float64)), ref)


def pin_block_composition(orc):
    """The block with identity-block weights is the mixer on slices of x: the
    in-projections feed the mixer unchanged and ssm_out passes y through."""
    Hqk, Hv, d = 1, 2, 8
    C = d * (2 * Hqk + Hv)
    widths = [C, Hv * d, Hv, Hv]
    hidden = sum(widths)
    cuts = np.cumsum([0] + widths)
    lx = _layer_inputs(174, [9, 70], Hqk, Hv, d)
    T = int(lx["cu_seqlens"][-1])
    x = np.concatenate([lx["qkv"].reshape(T, -1), lx["z"].reshape(T, -1), lx["b"], lx["a"]], axis=1)
    eye = np.eye(hidden)
    ws = [eye[cuts[i]:cuts[i + 1]] for i in range(4)]
    w_out = np.eye(hidden)[:, :Hv * d]                   # out[:, :Hv*d] = y, the rest 0
    import oracle
    for rnd, rnd_o in ((False, False), (True, False), (True, True)):
        r = orc.block(lx["cu_seqlens"], Hqk, Hv, d, x, *ws, w_out, lx["conv_w"], lx["dt_bias"],
                      lx["A_log"], lx["norm_w"], lx["conv0"], lx["S0"], round_act=rnd, round_o=rnd_o)
        f = oracle.round_bf16 if rnd else (lambda a: a)
        ref = orc.layer(lx["cu_seqlens"], Hqk, Hv, d, f(lx["qkv"]), f(lx["z"]), f(lx["b"]), f(lx["a"]),
                        lx["conv_w"], lx["dt_bias"], lx["A_log"], lx["norm_w"], lx["conv0"], lx["S0"])
        y = ref["y"]
        if rnd_o:   # the norm reads the readout after its bf16 rounding
            y = orc.gated_rmsnorm(oracle.round_bf16(ref["o"]), f(lx["z"]), lx["norm_w"])
        assert np.array_equal(r["out"][:, :Hv * d], f(y).reshape(T, -1)), (rnd, rnd_o)
        assert np.array_equal(r["out"][:, Hv * d:], np.zeros((T, hidden - Hv * d))), (rnd, rnd_o)
        assert np.array_equal(r["S_out"], ref["S_out"]), (rnd, rnd_o)
        assert not rnd_o or not np.array_equal(y, ref["y"]), "rounding o must change y"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
