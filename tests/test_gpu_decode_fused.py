"""Parity of gdn_decode_fused (one launch per decode step) with the fp64
oracle, and of HIP-graph replays of the decode loop with the eager loop.

The fused step must meet the same bar as the three-call step: y and the
final delta state within the act dtype's tolerance, the conv state bit for
bit. A captured graph must reproduce the eager results exactly (same
kernels on the same bytes) on every replay."""
import sys

import numpy as np
import pytest
import torch

from gated_deltanet_layer_amd import binding as B
from gated_deltanet_layer_amd import layer as Lyr
from gated_deltanet_layer_amd import workloads as wl
from tests import parity as P
from tests.test_gpu_parity import compare_decode

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("heads", [(2, 4), (2, 6), (4, 4)])
def test_fused_decode_small(act, heads):
    hqk, hv = heads
    w = wl.custom("decode", 3, hqk, hv, act, seed=300 + hv, steps=40, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case fused decode N=3 steps=40 Hqk={hqk} Hv={hv} {act}")
    compare_decode(w, x, P.gpu_decode_fused(w, x))


def test_fused_decode_many_sequences():
    w = wl.custom("decode", 100, 1, 2, "bf16", seed=310, steps=5, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say("case fused decode N=100 steps=5 Hqk=1 Hv=2 bf16")
    compare_decode(w, x, P.gpu_decode_fused(w, x))


def test_fused_decode_workload2_full():
    w = wl.WORKLOADS[2]
    x = wl.generate(w)
    say(f"case fused {w.name}")
    compare_decode(w, x, P.gpu_decode_fused(w, x))


def test_fused_decode_workload4_full_size():
    w = wl.WORKLOADS[4]
    x = wl.generate(w)
    say(f"case fused {w.name}")
    compare_decode(w, x, P.gpu_decode_fused(w, x), seqs=[0, 21, 42, 63])


def test_fused_matches_three_call_step():
    """Same state to the fp32 bar; y within bf16 rounding of o (the fused
    step normalises the fp32 readout, the three calls its bf16 copy)."""
    w = wl.custom("decode", 4, 2, 4, "bf16", seed=311, steps=24, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say("case fused vs three-call decode")
    a = P.gpu_decode(w, x)
    b = P.gpu_decode_fused(w, x)
    P.check("S_out", b["S_out"], a["S_out"], "f32")
    P.check("y", b["y"], a["y"], "bf16")
    assert np.array_equal(a["conv_out_bits"], b["conv_out_bits"])


def _decode_inputs(w):
    x = wl.generate(w)
    return {k: P.dev(v) for k, v in x.items()}


@pytest.mark.parametrize("fused", [True, False])
def test_graph_replay_matches_eager(fused):
    """Capture 8 decode steps in a HIP graph; every replay, with eager work
    and synchronisations between replays, must equal the eager loop bit for
    bit."""
    w = wl.custom("decode", 2, 2, 4, "bf16", seed=312, steps=8, s0_std=0.02, conv0_std=1.0)
    t = _decode_inputs(w)
    cfg = B.make_config(w.n_qk_heads, w.n_v_heads, w.act)
    steps, N = t["qkv"].shape[:2]
    S = t["S0"].clone()
    conv = t["conv0"].clone()
    ys = torch.empty_like(t["z"])
    run = Lyr.DecodeFused(cfg, N, conv) if fused else Lyr.Decode(cfg, N)

    def loop():
        for s in range(steps):
            if fused:
                run(t["qkv"][s], t["z"][s], t["b"][s], t["a"][s], t["conv_w"], t["dt_bias"], t["A_log"],
                    t["norm_w"], S, ys[s])
            else:
                run(t["qkv"][s], t["z"][s], t["b"][s], t["a"][s], t["conv_w"], t["dt_bias"], t["A_log"],
                    t["norm_w"], conv, S, ys[s])

    def reset():
        S.copy_(t["S0"])
        conv.copy_(t["conv0"])
        ys.zero_()
        if fused:
            run.cur = 0

    def state():
        c = run.conv_state if fused else conv
        return P.bits(ys).copy(), P.bits(S).copy(), P.bits(c).copy()

    say(f"case graph replay fused={fused}: eager")
    reset()
    loop()
    torch.cuda.synchronize()
    ref = state()

    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop()
    for rep in range(3):
        say(f"  replay {rep}")
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = state()
        for name, a, b in zip(("y", "S", "conv"), got, ref):
            assert np.array_equal(a, b), f"replay {rep}: {name} differs from the eager loop"
        # Eager work between replays.
        (t["z"].float() * 2.0).sum().item()


def test_prefill_graph_replay_matches_eager():
    """The prefill step (prep, chunked delta rule, norm) captured in a HIP
    graph: every replay equals the eager step bit for bit."""
    w = wl.custom("prefill", 2, 2, 4, "bf16", seed=313, lengths=[150, 77], s0_std=0.02)
    x = wl.generate(w)
    t = {k: P.dev(v) for k, v in x.items()}
    cfg = B.make_config(w.n_qk_heads, w.n_v_heads, w.act)
    cu = x["cu_seqlens"]
    N, T = len(cu) - 1, int(cu[-1])
    run = Lyr.Prefill(cfg, N, T)
    conv_out = torch.empty_like(t["conv0"])
    S_out = torch.empty_like(t["S0"])

    def step():
        run(t["cu_seqlens"], t["qkv"], t["z"], t["b"], t["a"], t["conv_w"], t["dt_bias"], t["A_log"],
            t["norm_w"], t["conv0"], conv_out, t["S0"], S_out)

    def state():
        return P.bits(run.y).copy(), P.bits(S_out).copy(), P.bits(conv_out).copy()

    say("case prefill graph replay: eager")
    step()
    torch.cuda.synchronize()
    ref = state()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        say(f"  replay {rep}")
        run.y.zero_()
        S_out.zero_()
        conv_out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "S", "conv"), state(), ref):
            assert np.array_equal(a, b), f"replay {rep}: {name} differs from the eager step"
        (t["z"].float() * 2.0).sum().item()
