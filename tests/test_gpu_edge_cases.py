"""The method's degenerate cases through the kernels, via the C ABI.

Each case builds inputs that drive one special branch of the arithmetic the
xwen CLAUDE.md page specifies (section "Architecture cheat sheet", gated
DeltaNet paragraph) and checks the GPU against the fp64 oracle on the same
bytes, and where the mathematics fixes the answer in closed form, against
that closed form too:

  * q/k heads that are exactly zero or far below the clamp epsilon, where
    the clamp form x / max(||x||, eps) differs from a plain division: a zero
    head must stay zero (no NaN), a sub-eps head becomes x / eps. Run through
    every kernel that normalises q and k (prep, the fused prefill's parallel
    kernel, the fused decode step and the verify call).
  * beta = 0 (every update vanishes): the state only decays,
    S_T = exp(sum g) S_0, and the readout is o_t = s exp(gamma_t) S_0^T q_t.
  * g = 0, beta = 1 and q = k of unit norm: after each update S^T k = v, so
    the readout is exactly o_t = v_t / sqrt(128).
  * extreme gates: an alpha logit of 800 makes g about -800 .. -12800, so the
    cumulative log-decay inside a chunk drops far below where exp underflows
    (-745 in fp64, -104 in fp32); beta logits of +-1e4 saturate beta at 0, 1.
  * the verify call at the size the benchmark times it (64 sequences,
    16 K-heads, 32 V-heads, 16 draft tokens), against the oracle's prefixes
    on sampled sequences.
"""
import math
import sys

import numpy as np
import pytest
import torch

from gated_deltanet_layer_amd import binding as B
from gated_deltanet_layer_amd import layer as Lyr
from gated_deltanet_layer_amd import workloads as wl
from tests import parity as P
from tests.test_gpu_parity import compare_decode, compare_prefill

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128.0)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------ clamp
def clamp_inputs(act: str, kind: str, seed: int, **kw):
    """A workload with 4 K-heads (8 V-heads) whose conv taps make
    K-head 0's q exactly zero, K-head 1's k exactly zero (SiLU(0) = 0), and
    K-head 2's q and k about 1e-9 (norms ~1e-8, far below eps = 1e-6);
    K-head 3 is left as drawn."""
    w = wl.custom(kind, 2, 4, 8, act, seed=seed, s0_std=0.02, conv0_std=1.0, **kw)
    x = wl.generate(w)
    d, Hqk = w.head_dim, w.n_qk_heads
    cw = x["conv_w"].copy()
    cw[0 * d:1 * d] = 0.0                                 # q of K-head 0
    cw[Hqk * d + 1 * d:Hqk * d + 2 * d] = 0.0             # k of K-head 1
    cw[2 * d:3 * d] *= np.float32(1e-9)                   # q of K-head 2
    cw[Hqk * d + 2 * d:Hqk * d + 3 * d] *= np.float32(1e-9)   # k of K-head 2
    x["conv_w"] = cw
    return w, x


def check_clamped_qk(q, k, w, x):
    """The clamp's own effect on the q, k the prep stored, beside the oracle
    comparison: zero heads exactly zero, sub-eps heads equal to x / eps
    (norm well below 1), the others of unit norm."""
    assert np.all(q[:, 0] == 0.0) and np.all(k[:, 1] == 0.0)
    nq2 = np.linalg.norm(q[:, 2].astype(np.float64), axis=-1)
    nk2 = np.linalg.norm(k[:, 2].astype(np.float64), axis=-1)
    assert np.all(nq2 < 0.1) and np.all(nk2 < 0.1) and np.all(nq2 > 0.0)
    n3 = np.linalg.norm(q[:, 3].astype(np.float64), axis=-1)
    assert np.allclose(n3, 1.0, atol=1e-5)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_clamp_prefill_three_call_and_fused(act):
    w, x = clamp_inputs(act, "prefill", 400, lengths=[130, 5])
    say(f"case clamp prefill three-call {act}")
    got = P.gpu_prefill(w, x)
    check_clamped_qk(got["q"], got["k"], w, x)
    compare_prefill(w, x, got)
    say(f"case clamp prefill fused {act}")
    compare_prefill(w, x, P.gpu_prefill_fused(w, x))


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_clamp_decode_three_call_and_fused(act):
    w, x = clamp_inputs(act, "decode", 401, steps=6)
    say(f"case clamp decode three-call {act}")
    compare_decode(w, x, P.gpu_decode(w, x))
    say(f"case clamp decode fused {act}")
    compare_decode(w, x, P.gpu_decode_fused(w, x))


def test_clamp_verify():
    w, x = clamp_inputs("bf16", "decode", 402, steps=5)
    K, N = x["qkv"].shape[:2]
    say(f"case clamp verify K={K} N={N}")
    y, S_snap, conv_snap = run_verify(w, x)
    for m in (K, 2):
        check_verify_prefix(w, x, y, S_snap, conv_snap, m, list(range(N)))


# ------------------------------------------------------- core-level inputs
def unit_rows(rng, shape):
    a = rng.standard_normal(size=shape)
    return (a / np.linalg.norm(a, axis=-1, keepdims=True)).astype(np.float32)


def run_core_prefill(cfg, cu, q, k, v, beta, g, S0):
    """gdn_prefill_chunked on given q, k, v, beta, g (host fp32 arrays)."""
    N, T = len(cu) - 1, int(cu[-1])
    run = Lyr.Prefill(cfg, N, T)
    run.q.copy_(torch.from_numpy(q))
    run.k.copy_(torch.from_numpy(k))
    run.v.copy_(torch.from_numpy(v))
    run.beta.copy_(torch.from_numpy(beta))
    run.g.copy_(torch.from_numpy(g))
    S_in = P.dev(S0)
    S_out = torch.empty_like(S_in)
    run.core(P.dev(cu), S_in, S_out)
    torch.cuda.synchronize()
    return P.host(run.o), P.host(S_out)


def run_core_decode(cfg, q, k, v, beta, g, S0):
    """gdn_decode_step over steps [S][N] ... with S updated in place."""
    steps, N = q.shape[:2]
    Hv, d = cfg.n_v_heads, cfg.head_dim
    S = P.dev(S0)
    o = torch.empty((steps, N, Hv, d), dtype=torch.bfloat16 if cfg.act_dtype == B.GDN_BF16 else torch.float32,
                    device="cuda")
    tq, tk, tv, tb, tg = (P.dev(a) for a in (q, k, v, beta, g))
    for s in range(steps):
        B.gdn_decode_step(cfg, N, tq[s], tk[s], tv[s], tb[s], tg[s], S, S, o[s])
    torch.cuda.synchronize()
    return P.host(o), P.host(S)


def readout_pure_decay(q, S0, cu, g, hqk):
    """o_t = s exp(gamma_t) S_0^T q_t for beta = 0 (gamma_t = g (t + 1) for the
    t-th token of its sequence, g constant)."""
    T, Hv = q.shape[0], S0.shape[1]
    o = np.empty((T, Hv, 128))
    for n in range(len(cu) - 1):
        for t in range(cu[n], cu[n + 1]):
            gam = math.exp(g * (t - cu[n] + 1))
            for j in range(Hv):
                o[t, j] = SCALE * gam * (S0[n, j].astype(np.float64).T @ q[t, j % hqk].astype(np.float64))
    return o


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("gval", [-math.log(2.0), -math.log(2.0) / 16])
def test_beta_zero_pure_decay_prefill(act, gval):
    hqk, hv, lens = 2, 4, [1, 63, 64, 65, 130]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, N = int(cu[-1]), len(lens)
    rng = np.random.default_rng(410)
    q, k = unit_rows(rng, (T, hqk, 128)), unit_rows(rng, (T, hqk, 128))
    v = rng.standard_normal((T, hv, 128)).astype(np.float32)
    beta = np.zeros((T, hv), np.float32)
    g = np.full((T, hv), gval, np.float32)
    S0 = rng.standard_normal((N, hv, 128, 128)).astype(np.float32)
    say(f"case beta=0 prefill g={gval:.4f} {act}")
    cfg = B.make_config(hqk, hv, act)
    o, S = run_core_prefill(cfg, cu, q, k, v, beta, g, S0)
    ref_o = readout_pure_decay(q, S0, cu, float(np.float32(gval)), hqk)
    ref_S = np.stack([math.exp(float(np.float32(gval)) * L) * S0[n].astype(np.float64) for n, L in enumerate(lens)])
    rep = {}
    P.check("o", o, ref_o, act, rep)
    P.check("S_out", S, ref_S, act, rep)
    say("  closed form: " + ", ".join(f"{a}={b:.3f}" for a, b in rep.items()))


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_beta_zero_pure_decay_decode(act):
    hqk, hv, N, steps = 2, 4, 3, 9
    rng = np.random.default_rng(411)
    q, k = unit_rows(rng, (steps, N, hqk, 128)), unit_rows(rng, (steps, N, hqk, 128))
    v = rng.standard_normal((steps, N, hv, 128)).astype(np.float32)
    gval = -math.log(2.0)
    beta = np.zeros((steps, N, hv), np.float32)
    g = np.full((steps, N, hv), gval, np.float32)
    S0 = rng.standard_normal((N, hv, 128, 128)).astype(np.float32)
    say(f"case beta=0 decode {act}")
    cfg = B.make_config(hqk, hv, act)
    o, S = run_core_decode(cfg, q, k, v, beta, g, S0)
    g32 = float(np.float32(gval))
    ref_S = math.exp(g32 * steps) * S0.astype(np.float64)
    ref_o = np.empty((steps, N, hv, 128))
    for s in range(steps):
        for n in range(N):
            for j in range(hv):
                ref_o[s, n, j] = SCALE * math.exp(g32 * (s + 1)) * (S0[n, j].astype(np.float64).T @ q[s, n, j % hqk])
    rep = {}
    P.check("o", o, ref_o, act, rep)
    P.check("S_out", S, ref_S, act, rep)
    say("  closed form: " + ", ".join(f"{a}={b:.3f}" for a, b in rep.items()))


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_unit_key_reads_back_v_prefill(act):
    """g = 0, beta = 1, q = k unit: o = v / sqrt(128) for every token; the
    final state against the oracle's recurrence."""
    hqk, hv, lens = 2, 4, [70, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, N = int(cu[-1]), len(lens)
    rng = np.random.default_rng(412)
    k = unit_rows(rng, (T, hqk, 128))
    v = rng.standard_normal((T, hv, 128)).astype(np.float32)
    beta = np.ones((T, hv), np.float32)
    g = np.zeros((T, hv), np.float32)
    S0 = (0.02 * rng.standard_normal((N, hv, 128, 128))).astype(np.float32)
    say(f"case g=0 beta=1 unit key prefill {act}")
    cfg = B.make_config(hqk, hv, act)
    o, S = run_core_prefill(cfg, cu, k, k, v, beta, g, S0)
    rep = {}
    P.check("o", o, SCALE * v.astype(np.float64), act, rep)
    import oracle
    _, ref_S = oracle.default().delta_rule(cu, hqk, hv, 128, k, k, v, beta, g, S0)
    P.check("S_out", S, ref_S, act, rep)
    say("  closed form / oracle: " + ", ".join(f"{a}={b:.3f}" for a, b in rep.items()))


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_unit_key_reads_back_v_decode(act):
    hqk, hv, N, steps = 2, 4, 3, 7
    rng = np.random.default_rng(413)
    k = unit_rows(rng, (steps, N, hqk, 128))
    v = rng.standard_normal((steps, N, hv, 128)).astype(np.float32)
    beta = np.ones((steps, N, hv), np.float32)
    g = np.zeros((steps, N, hv), np.float32)
    S0 = (0.02 * rng.standard_normal((N, hv, 128, 128))).astype(np.float32)
    say(f"case g=0 beta=1 unit key decode {act}")
    cfg = B.make_config(hqk, hv, act)
    o, _ = run_core_decode(cfg, k, k, v, beta, g, S0)
    rep = {}
    P.check("o", o, SCALE * v.astype(np.float64), act, rep)
    say("  closed form: " + ", ".join(f"{a}={b:.3f}" for a, b in rep.items()))


# ------------------------------------------------------------ extreme gates
def extreme_gate_inputs(act: str, kind: str, seed: int, **kw):
    """alpha logit 800 on a few tokens of every V-head (inside a chunk, at a
    chunk's first and last rows), beta logits of +-1e4 on a few others."""
    w = wl.custom(kind, 2, 2, 4, act, seed=seed, s0_std=0.02, conv0_std=1.0, **kw)
    x = wl.generate(w)
    a = wl.as_f32(x["a"], act).copy()
    b = wl.as_f32(x["b"], act).copy()
    flat_a, flat_b = a.reshape(-1, a.shape[-1]), b.reshape(-1, b.shape[-1])
    rows = flat_a.shape[0]
    for r in (3, 63, 64, 100, rows - 1):
        if r < rows:
            flat_a[r, :] = 800.0
    for r, val in ((5, 1e4), (6, -1e4), (70, 1e4)):
        if r < rows:
            flat_b[r, :] = val
    x["a"] = wl.bf16_bits(a) if act == "bf16" else a
    x["b"] = wl.bf16_bits(b) if act == "bf16" else b
    return w, x


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_extreme_gates_prefill(act):
    w, x = extreme_gate_inputs(act, "prefill", 420, lengths=[140, 70])
    say(f"case extreme gates prefill three-call {act}")
    got = P.gpu_prefill(w, x)
    assert np.min(got["g"]) < -700.0
    compare_prefill(w, x, got)
    say(f"case extreme gates prefill fused {act}")
    compare_prefill(w, x, P.gpu_prefill_fused(w, x))


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_extreme_gates_decode(act):
    w, x = extreme_gate_inputs(act, "decode", 421, steps=8)
    say(f"case extreme gates decode three-call {act}")
    compare_decode(w, x, P.gpu_decode(w, x))
    say(f"case extreme gates decode fused {act}")
    compare_decode(w, x, P.gpu_decode_fused(w, x))


# ------------------------------------------------------------------ verify
def run_verify(w, x, keep=None):
    """One gdn_decode_verify call over the decode workload's steps as K draft
    tokens; returns host copies (of the sequences in `keep` only)."""
    cfg = B.make_config(w.n_qk_heads, w.n_v_heads, w.act)
    K, N = x["qkv"].shape[:2]
    t = {k: P.dev(v) for k, v in x.items()}
    seq_major = lambda a: a.transpose(0, 1).contiguous()
    qkv, z, b, a = (seq_major(t[k]) for k in ("qkv", "z", "b", "a"))
    Hv, d = w.n_v_heads, w.head_dim
    conv_snap = torch.empty((N, K) + tuple(t["conv0"].shape[1:]), dtype=t["conv0"].dtype, device="cuda")
    S_snap = torch.empty((N, K, Hv, d, d), dtype=torch.float32, device="cuda")
    y = torch.empty_like(z)
    B.gdn_decode_verify(cfg, N, K, qkv, b, a, z, t["conv_w"], t["dt_bias"], t["A_log"], t["norm_w"],
                        t["conv0"], conv_snap, t["S0"], S_snap, y)
    torch.cuda.synchronize()
    sel = list(range(N)) if keep is None else list(keep)
    return (P.host(y[sel]), P.host(S_snap[sel]), P.bits(conv_snap[sel]))


def check_verify_prefix(w, x, y, S_snap, conv_bits, m, seqs):
    """Plane K - m of the sequences `seqs` (in the order y, S_snap,
    conv_bits hold them) against the oracle over their first m tokens."""
    K = x["qkv"].shape[0]
    Hv, d = w.n_v_heads, w.head_dim
    xm = dict(x)
    for key in ("qkv", "z", "b", "a"):
        xm[key] = x[key][:m]
    xp = P.decode_as_packed(xm, seqs)
    ref = P.oracle_layer(w, P.inputs_f64(xp, w.act), xp["cu_seqlens"])
    rep = {}
    P.check("S_plane", S_snap[:, K - m], ref["S_out"], w.act, rep)
    P.check("y", y[:, :m].reshape(len(seqs) * m, Hv, d), ref["y"], w.act, rep)
    ref_conv = ref["conv_out"].astype(np.float32)
    exp_bits = wl.bf16_bits(ref_conv) if w.act == "bf16" else ref_conv.view(np.uint32)
    assert np.array_equal(conv_bits[:, K - m], exp_bits), f"conv plane {K - m}"
    say(f"  prefix {m}: " + ", ".join(f"{a}={b:.3f}" for a, b in rep.items()))


def test_verify_at_benched_size():
    """64 sequences, 16 K-heads, 32 V-heads, 16 draft tokens (the launch the
    benchmark times); 4 sampled sequences against the oracle's prefixes."""
    w = wl.custom("decode", 64, 16, 32, "bf16", seed=430, steps=16, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    seqs = [0, 17, 42, 63]
    say("case verify N=64 Hqk=16 Hv=32 K=16, sequences " + str(seqs))
    y, S_snap, conv_bits = run_verify(w, x, keep=seqs)
    for m in (16, 9, 1):
        check_verify_prefix(w, x, y, S_snap, conv_bits, m, seqs)
