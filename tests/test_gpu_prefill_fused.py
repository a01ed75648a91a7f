"""Parity of gdn_prefill_fused (the whole mixer in one call, q, k, v, beta
and g computed inside the chunked kernels) with the fp64 oracle, at the same
bars as the three-call prefill: y and the final state within the act dtype's
tolerance, the conv state bit for bit. Also: in-place states, packed equals
separate, the HF L2 form, agreement with the three calls on the GPU, and the
full-size prefill workloads on sampled heads and sequences."""
import sys

import numpy as np
import pytest

from gated_deltanet_layer_amd import workloads as wl
from tests import parity as P
from tests.test_gpu_parity import compare_prefill

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_fused_several_chunks_ragged_tail(act):
    w = wl.custom("prefill", 1, 2, 4, act, seed=501, lengths=[200], s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case fused prefill T=200 Hqk=2 Hv=4 {act}")
    compare_prefill(w, x, P.gpu_prefill_fused(w, x))


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_fused_varlen_edge_lengths(act):
    lens = [0, 1, 2, 3, 5, 63, 64, 65, 129, 0]
    w = wl.custom("prefill", len(lens), 2, 6, act, seed=502, lengths=lens, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case fused varlen {lens} Hqk=2 Hv=6 {act}")
    compare_prefill(w, x, P.gpu_prefill_fused(w, x))


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("heads", [(1, 7), (2, 8)])
def test_fused_many_v_heads_per_k_head(heads, act):
    # Several rounds of V-heads per K-head in chunk_local (three at a time).
    hqk, hv = heads
    w = wl.custom("prefill", 2, hqk, hv, act, seed=503, lengths=[150, 67], s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case fused prefill lengths [150, 67] Hqk={hqk} Hv={hv} {act}")
    compare_prefill(w, x, P.gpu_prefill_fused(w, x))


def test_fused_many_short_sequences():
    # 150 packed sequences (0..40 tokens), beyond one 64-sequence scan step.
    lens = [int(v) for v in np.random.default_rng(504).integers(0, 41, size=150)]
    w = wl.custom("prefill", len(lens), 1, 2, "bf16", seed=504, lengths=lens, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case fused prefill 150 sequences, T={sum(lens)} Hqk=1 Hv=2 bf16")
    compare_prefill(w, x, P.gpu_prefill_fused(w, x))


def test_fused_empty_call_passes_states_through():
    w = wl.custom("prefill", 3, 2, 4, "bf16", seed=503, lengths=[0, 0, 0], s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say("case fused all-empty")
    got = P.gpu_prefill_fused(w, x)
    assert np.array_equal(got["S_out"], x["S0"])
    assert np.array_equal(got["conv_out_bits"], x["conv0"])


def test_fused_inplace_states_match_out_of_place():
    w = wl.custom("prefill", 3, 2, 4, "bf16", seed=504, lengths=[70, 2, 150], s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say("case fused in-place states")
    a = P.gpu_prefill_fused(w, x, inplace=False)
    b = P.gpu_prefill_fused(w, x, inplace=True)
    for k in ("y", "S_out", "conv_out_bits"):
        assert np.array_equal(a[k], b[k]), k


def test_fused_packed_equals_separate_runs():
    lens = [130, 7, 64]
    w = wl.custom("prefill", 3, 2, 4, "bf16", seed=505, lengths=lens, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say("case fused packed vs separate")
    packed = P.gpu_prefill_fused(w, x)
    cu = x["cu_seqlens"]
    for n in range(3):
        one = P.gpu_prefill_fused(wl.custom("prefill", 1, 2, 4, "bf16", seed=505, lengths=[lens[n]]),
                                  P.slice_seqs(x, [n]))
        assert np.array_equal(one["y"], packed["y"][cu[n]:cu[n + 1]]), n
        assert np.array_equal(one["S_out"][0], packed["S_out"][n])
        assert np.array_equal(one["conv_out_bits"][0], packed["conv_out_bits"][n])


def _norm_folded(n_seqs, hv):
    """Whether gdn_prefill_fused forms y and the new conv states inside the
    sequential kernel's launch: its 4 blocks per (sequence, V-head), rounded
    up to whole rounds of the 8 XCDs, leave at least 32 of the 256 CUs idle."""
    return 256 - (n_seqs * hv + 7) // 8 * 8 * 4 >= 32


# (lengths, Hqk, Hv): the folded norm (20 pairs, 96 sequential blocks) and the
# norm launch (60 pairs, 256 sequential blocks), both with empty sequences.
FOLD_CASES = [([0, 65, 130, 0, 3], 2, 4),
              ([40, 0, 1, 64, 2, 100, 7, 0, 12, 33, 5, 70, 9, 0, 90], 2, 4)]


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("case", [0, 1], ids=["folded", "norm_launch"])
def test_fused_norm_folded_and_apart(case, act):
    """Both forms of the call against the oracle, and in-place states equal
    to out-of-place ones (the folded form overwrites each part of the old conv
    state inside the launch that reads it)."""
    lens, hqk, hv = FOLD_CASES[case]
    assert _norm_folded(len(lens), hv) == (case == 0)
    w = wl.custom("prefill", len(lens), hqk, hv, act, seed=508 + case, lengths=lens, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case fused {'folded' if case == 0 else 'norm launch'} {lens} Hqk={hqk} Hv={hv} {act}")
    a = P.gpu_prefill_fused(w, x)
    compare_prefill(w, x, a)
    b = P.gpu_prefill_fused(w, x, inplace=True)
    for k in ("y", "S_out", "conv_out_bits"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("case", [0, 1], ids=["folded", "norm_launch"])
def test_fused_graph_replay_matches_eager(case):
    """The fused prefill captured in a HIP graph: every replay, with eager
    work and synchronisations between replays, equals the eager call bit for
    bit (the folded form's counters are cleared by a kernel of the call, not a
    memset)."""
    import torch
    from gated_deltanet_layer_amd import binding as B
    from gated_deltanet_layer_amd import layer as Lyr
    lens, hqk, hv = FOLD_CASES[case]
    w = wl.custom("prefill", len(lens), hqk, hv, "bf16", seed=510 + case, lengths=lens, s0_std=0.02,
                  conv0_std=1.0)
    x = wl.generate(w)
    t = {k: P.dev(v) for k, v in x.items()}
    run = Lyr.PrefillFused(B.make_config(hqk, hv, "bf16"), len(lens), sum(lens))
    conv_out, S_out = torch.empty_like(t["conv0"]), torch.empty_like(t["S0"])

    def step():
        run(t["cu_seqlens"], t["qkv"], t["z"], t["b"], t["a"], t["conv_w"], t["dt_bias"], t["A_log"],
            t["norm_w"], t["conv0"], conv_out, t["S0"], S_out)

    def state():
        return P.bits(run.y).copy(), P.bits(S_out).copy(), P.bits(conv_out).copy()

    say(f"case fused graph replay ({'folded' if case == 0 else 'norm launch'}): eager")
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
            assert np.array_equal(a, b), f"replay {rep}: {name} differs from the eager call"
        (t["z"].float() * 2.0).sum().item()


def test_fused_concurrent_calls_on_two_streams():
    """Two folded calls (the 4,096-token shape's head counts, shorter) on two
    streams at once, each with its own workspace: the norm blocks of one
    launch wait only for that launch's slab blocks, so interleaved launches
    give the same bits as the calls run one after the other."""
    import torch
    from gated_deltanet_layer_amd import binding as B
    from gated_deltanet_layer_amd import layer as Lyr
    cfg = B.make_config(16, 48, "bf16")
    assert _norm_folded(1, 48)
    runs = []
    for seed, T in ((520, 1000), (521, 777)):
        w = wl.custom("prefill", 1, 16, 48, "bf16", seed=seed, lengths=[T], s0_std=0.02, conv0_std=1.0)
        x = wl.generate(w)
        t = {k: P.dev(v) for k, v in x.items()}
        runs.append((t, Lyr.PrefillFused(cfg, 1, T), torch.empty_like(t["conv0"]), torch.empty_like(t["S0"])))

    def call(r):
        t, f, conv_o, S_o = r
        f(t["cu_seqlens"], t["qkv"], t["z"], t["b"], t["a"], t["conv_w"], t["dt_bias"], t["A_log"], t["norm_w"],
          t["conv0"], conv_o, t["S0"], S_o)

    say("case fused concurrent calls: serial")
    ref = []
    for r in runs:
        call(r)
        torch.cuda.synchronize()
        ref.append((P.bits(r[1].y).copy(), P.bits(r[3]).copy(), P.bits(r[2]).copy()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        say(f"  concurrent {rep}")
        for r in runs:
            r[1].y.zero_()
            r[3].zero_()
            r[2].zero_()
        torch.cuda.synchronize()
        for st, r in zip(streams, runs):
            with torch.cuda.stream(st):
                call(r)
        torch.cuda.synchronize()
        for k, r in enumerate(runs):
            got = (P.bits(r[1].y), P.bits(r[3]), P.bits(r[2]))
            for name, a, b in zip(("y", "S", "conv"), got, ref[k]):
                assert np.array_equal(a, b), f"rep {rep}, call {k}: {name} differs from the serial call"


def test_fused_l2_rsqrt_form():
    w = wl.custom("prefill", 2, 2, 4, "bf16", seed=506, lengths=[100, 37], s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say("case fused prefill, HF L2 form")
    compare_prefill(w, x, P.gpu_prefill_fused(w, x, l2_mode="rsqrt"), l2_mode="rsqrt")


def test_fused_matches_three_calls():
    """The same state to the fp32 bar and y within bf16 rounding of the
    three-call path on the GPU (the q/k norms sum in another order)."""
    w = wl.custom("prefill", 2, 2, 4, "bf16", seed=507, lengths=[190, 66], s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say("case fused vs three calls")
    a = P.gpu_prefill(w, x)
    b = P.gpu_prefill_fused(w, x)
    P.check("S_out", b["S_out"], a["S_out"], "f32")
    P.check("y", b["y"], a["y"], "bf16")
    assert np.array_equal(a["conv_out_bits"], b["conv_out_bits"])


def test_fused_workload3_prefill_4096_full_size():
    w = wl.WORKLOADS[3]
    x = wl.generate(w)
    say(f"case fused {w.name}")
    compare_prefill(w, x, P.gpu_prefill_fused(w, x), heads=[0, 7, 16, 31, 47])


def test_fused_workload5_varlen_full_size():
    w = wl.WORKLOADS[5]
    x = wl.generate(w)
    lens = np.diff(x["cu_seqlens"])
    say(f"case fused {w.name}: lengths {lens.tolist()}")
    seqs = [int(np.argmin(lens)), int(np.argmax(lens))]
    compare_prefill(w, x, P.gpu_prefill_fused(w, x), heads=[1, 18, 40], seqs=seqs)
