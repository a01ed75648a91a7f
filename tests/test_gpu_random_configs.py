"""Seeded random configurations through the three-call prefill, the fused
prefill, the fused decode step, the verify call and the fused prefill with
checkpoints, each against the fp64 oracle on every head and sequence.

Each case draws (from its own seed) the K-head count, the V-heads per K-head
(tiled head map), the activation dtype, the L2 form, the number of packed
sequences and their lengths from a pool that mixes the edge lengths (0, 1,
2, 3, exact chunk multiples and one past them) with arbitrary ones, and the
initial-state scales. The shapes the named workloads use are covered
elsewhere; these cases exercise the index arithmetic between them (head
maps, chunk and tile boundaries, packed offsets) at sizes the oracle
finishes in well under a second.
"""
import sys

import numpy as np
import pytest

from gated_deltanet_layer_amd import workloads as wl
from tests import parity as P
from tests.test_gpu_parity import compare_decode, compare_prefill

pytestmark = pytest.mark.gpu

LENGTHS = [0, 1, 2, 3, 5, 17, 31, 63, 64, 65, 100, 127, 128, 129, 191, 200]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def draw(seed):
    rng = np.random.default_rng(seed)
    hqk = int(rng.choice([1, 2, 3, 4]))
    ratio = int(rng.choice([1, 2, 3, 4]))
    act = str(rng.choice(["f32", "bf16"]))
    l2 = str(rng.choice(["clamp", "rsqrt"]))
    n = int(rng.integers(1, 5))
    lens = [int(v) for v in rng.choice(LENGTHS, size=n)]
    if sum(lens) == 0:
        lens[0] = 70
    s0 = float(rng.choice([0.0, 0.02, 0.3]))
    c0 = float(rng.choice([0.0, 1.0]))
    return hqk, hqk * ratio, act, l2, lens, s0, c0


@pytest.mark.parametrize("seed", range(700, 712))
def test_random_prefill_three_call_and_fused(seed):
    hqk, hv, act, l2, lens, s0, c0 = draw(seed)
    w = wl.custom("prefill", len(lens), hqk, hv, act, seed=seed, lengths=lens, s0_std=s0, conv0_std=c0)
    x = wl.generate(w)
    say(f"case seed={seed} prefill lengths={lens} Hqk={hqk} Hv={hv} {act} l2={l2} s0={s0} conv0={c0}")
    compare_prefill(w, x, P.gpu_prefill(w, x, l2_mode=l2), l2_mode=l2)
    compare_prefill(w, x, P.gpu_prefill_fused(w, x, l2_mode=l2), l2_mode=l2)


@pytest.mark.parametrize("seed", range(720, 726))
def test_random_decode_fused(seed):
    hqk, hv, act, l2, lens, s0, c0 = draw(seed)
    n = len(lens)
    steps = int(np.random.default_rng(seed + 1).integers(1, 9))
    w = wl.custom("decode", n, hqk, hv, act, seed=seed, steps=steps, s0_std=max(s0, 0.02), conv0_std=c0)
    x = wl.generate(w)
    say(f"case seed={seed} decode N={n} steps={steps} Hqk={hqk} Hv={hv} {act} l2={l2}")
    compare_decode(w, x, P.gpu_decode_fused(w, x, l2_mode=l2), l2_mode=l2)


@pytest.mark.parametrize("seed", range(730, 736))
def test_random_verify_planes(seed):
    """gdn_decode_verify on a random configuration: every snapshot plane
    against the oracle run over the matching accepted prefix."""
    from tests.test_gpu_decode_verify import run_verify
    hqk, hv, act, l2, lens, s0, c0 = draw(seed)
    n = len(lens)
    K = int(np.random.default_rng(seed + 1).integers(1, 9))
    w = wl.custom("decode", n, hqk, hv, act, seed=seed, steps=K, s0_std=max(s0, 0.02), conv0_std=c0)
    x = wl.generate(w)
    say(f"case seed={seed} verify N={n} K={K} Hqk={hqk} Hv={hv} {act}")
    y, S_snap, conv_snap = run_verify(w, x)
    Hv, d = w.n_v_heads, w.head_dim
    for m in range(K, 0, -1):                   # accepted prefix length m <-> plane K - m
        xm = dict(x)
        for k in ("qkv", "z", "b", "a"):
            xm[k] = x[k][:m]
        xp = P.decode_as_packed(xm)
        ref = P.oracle_layer(w, P.inputs_f64(xp, act), xp["cu_seqlens"])
        rep = {}
        P.check("S_plane", P.host(S_snap[:, K - m]), ref["S_out"], act, rep)
        P.check("y", P.host(y[:, :m]).reshape(n * m, Hv, d), ref["y"], act, rep)
        ref_conv = ref["conv_out"].astype(np.float32)
        exp = wl.bf16_bits(ref_conv) if act == "bf16" else ref_conv.view(np.uint32)
        assert np.array_equal(P.bits(conv_snap[:, K - m]), exp), f"conv plane {K - m}"


@pytest.mark.parametrize("seed", range(740, 746))
def test_random_fused_checkpoints(seed):
    """gdn_prefill_fused_ckpt on a random configuration and spacing: every
    plane against the oracle's prefix, planes past a sequence's end or past
    the capacity left untouched, and y, S_out, the new conv state identical
    to the call without checkpoints."""
    import torch
    from gated_deltanet_layer_amd import binding as B
    from gated_deltanet_layer_amd import layer as Lyr
    from tests.test_gpu_checkpoints import _prefix
    rng = np.random.default_rng(seed)
    hqk, hv, act, l2, _, s0, c0 = draw(seed)
    lengths = [int(v) for v in rng.choice([0, 63, 64, 65, 128, 129, 200, 256, 300], size=int(rng.integers(1, 4)))]
    if sum(lengths) == 0:
        lengths[0] = 129
    every = 64 * int(rng.integers(1, 3))
    cap = int(rng.integers(1, 5))
    w = wl.custom("prefill", len(lengths), hqk, hv, act, seed=seed, lengths=lengths, s0_std=max(s0, 0.02),
                  conv0_std=c0)
    x = wl.generate(w)
    say(f"case seed={seed} fused ckpt lengths={lengths} every={every} cap={cap} Hqk={hqk} Hv={hv} {act}")
    cfg = B.make_config(hqk, hv, act)
    N, T, d = len(lengths), sum(lengths), w.head_dim
    t = {k: P.dev(v) for k, v in x.items()}
    plain = Lyr.PrefillFused(cfg, N, T)
    conv_plain, S_plain = torch.empty_like(t["conv0"]), torch.empty_like(t["S0"])
    plain(t["cu_seqlens"], t["qkv"], t["z"], t["b"], t["a"], t["conv_w"], t["dt_bias"], t["A_log"], t["norm_w"],
          t["conv0"], conv_plain, t["S0"], S_plain)
    conv_new, S_out, y = torch.empty_like(t["conv0"]), torch.empty_like(t["S0"]), torch.empty_like(plain.y)
    S_ckpt = torch.full((N, cap, hv, d, d), float("nan"), device="cuda")
    conv_ckpt = torch.zeros((N, cap) + tuple(t["conv0"].shape[1:]), dtype=t["conv0"].dtype, device="cuda")
    B.gdn_prefill_fused_ckpt(cfg, N, T, t["cu_seqlens"], t["qkv"], t["b"], t["a"], t["z"], t["conv_w"],
                             t["dt_bias"], t["A_log"], t["norm_w"], t["conv0"], conv_new, t["S0"], S_out, y, every,
                             cap, S_ckpt, conv_ckpt, plain.ws)
    torch.cuda.synchronize()
    assert np.array_equal(P.bits(S_out), P.bits(S_plain)), "checkpointing changed S_out"
    assert np.array_equal(P.bits(y), P.bits(plain.y)), "checkpointing changed y"
    assert np.array_equal(P.bits(conv_new), P.bits(conv_plain)), "checkpointing changed the new conv state"
    for c in range(cap):
        m = [min(L, (c + 1) * every) for L in lengths]
        xm = _prefix(x, m)
        ref = P.oracle_layer(w, P.inputs_f64(xm, act), xm["cu_seqlens"])
        ref_conv = ref["conv_out"].astype(np.float32)
        exp_bits = wl.bf16_bits(ref_conv) if act == "bf16" else ref_conv.view(np.uint32)
        for n, L in enumerate(lengths):
            if (c + 1) * every > L:
                assert torch.isnan(S_ckpt[n, c]).all(), f"plane {c} of sequence {n} written past its end"
                continue
            P.check(f"S_ckpt[{n},{c}]", P.host(S_ckpt[n, c]), ref["S_out"][n], act)
            assert np.array_equal(P.bits(conv_ckpt[n, c]), exp_bits[n]), f"conv plane {c} of sequence {n}"
