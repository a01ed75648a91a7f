"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on seeded
inputs: small cases that span several chunks and ragged tails, the edge
lengths, and every workload at its full size (the GPU runs the whole
workload in the launch configuration the benchmark times; the oracle
recomputes a sample of sequences and V-heads)."""
import sys

import numpy as np
import pytest

from gated_deltanet_layer_amd import workloads as wl
from tests import parity as P

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def compare_prefill(w, x, got, heads=None, seqs=None, report=None, l2_mode="clamp"):
    """Check every output of a prefill run against the oracle (optionally on
    a sample of V-heads and sequences)."""
    xs = P.slice_seqs(x, seqs) if seqs is not None else x
    xf = P.inputs_f64(xs, w.act)
    ref = P.oracle_layer(w, xf, xs["cu_seqlens"], heads=heads, l2_mode=l2_mode)
    cu = x["cu_seqlens"]
    rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in (seqs if seqs is not None else range(len(cu) - 1))])
    sn = list(seqs) if seqs is not None else list(range(len(cu) - 1))
    hs = list(heads) if heads is not None else list(range(w.n_v_heads))
    rep = {} if report is None else report
    # A run returns the outputs its path stores (the fused prefill keeps q, k,
    # v, beta, g and o internal).
    for name in ("q", "k"):
        if name in got:
            P.check(name, got[name][rows], ref[name], "f32", rep)
    for name in ("v", "beta", "g"):
        if name in got:
            P.check(name, got[name][rows][:, hs], ref[name][:, hs], "f32", rep)
    for name in ("o", "y"):
        if name in got:
            P.check(name, got[name][rows][:, hs], ref[name][:, hs], w.act, rep)
    P.check("S_out", got["S_out"][sn][:, hs], ref["S_out"][:, hs], w.act, rep)
    ref_conv = ref["conv_out"].astype(np.float32)
    exp_bits = wl.bf16_bits(ref_conv) if w.act == "bf16" else ref_conv.view(np.uint32)
    assert np.array_equal(got["conv_out_bits"][sn], exp_bits), "conv state not bit-exact"
    say(f"  ratios: " + ", ".join(f"{k}={v:.3f}" for k, v in rep.items()))
    return rep


def compare_decode(w, x, got, seqs=None, l2_mode="clamp"):
    steps, N = x["qkv"].shape[:2]
    seqs = list(range(N)) if seqs is None else list(seqs)
    xp = P.decode_as_packed(x, seqs)
    ref = P.oracle_layer(w, P.inputs_f64(xp, w.act), xp["cu_seqlens"], l2_mode=l2_mode)
    Hv, d = w.n_v_heads, w.head_dim
    rep = {}
    for name in ("o", "y"):
        if name not in got:
            continue
        g = np.swapaxes(got[name][:, seqs], 0, 1).reshape(len(seqs) * steps, Hv, d)
        P.check(name, g, ref[name], w.act, rep)
    P.check("S_out", got["S_out"][seqs], ref["S_out"], w.act, rep)
    ref_conv = ref["conv_out"].astype(np.float32)
    exp_bits = wl.bf16_bits(ref_conv) if w.act == "bf16" else ref_conv.view(np.uint32)
    assert np.array_equal(got["conv_out_bits"][seqs], exp_bits), "conv state not bit-exact"
    say(f"  ratios: " + ", ".join(f"{k}={v:.3f}" for k, v in rep.items()))


# ----------------------------------------------------------- small cases
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_prefill_several_chunks_ragged_tail(act):
    w = wl.custom("prefill", 1, 2, 4, act, seed=201, lengths=[200], s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case prefill T=200 Hqk=2 Hv=4 {act}")
    compare_prefill(w, x, P.gpu_prefill(w, x))


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_prefill_varlen_edge_lengths(act):
    lens = [0, 1, 2, 3, 5, 63, 64, 65, 129, 0]
    w = wl.custom("prefill", len(lens), 2, 6, act, seed=202, lengths=lens, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case varlen {lens} Hqk=2 Hv=6 {act}")
    compare_prefill(w, x, P.gpu_prefill(w, x))


@pytest.mark.parametrize("lens", [[1, 40, 64, 23], [1, 40, 64, 22]])
def test_prep_tile_regimes(lens):
    # The prep kernel takes 32-token tiles when sequences average at least 32
    # tokens (first case: T = 128 = 32 N) and 8-token tiles otherwise (T = 127):
    # both, with tiles that end inside and at the end of sequences.
    w = wl.custom("prefill", len(lens), 2, 4, "bf16", seed=209, lengths=lens, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case prep tiles {lens} Hqk=2 Hv=4 bf16")
    compare_prefill(w, x, P.gpu_prefill(w, x))


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("heads", [(1, 7), (2, 8)])
def test_prefill_many_v_heads_per_k_head(heads, act):
    # chunk_local handles the V-heads of a K-head three at a time: seven and
    # four of them take three and two rounds (the last one partial).
    hqk, hv = heads
    w = wl.custom("prefill", 2, hqk, hv, act, seed=210, lengths=[150, 67], s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case prefill lengths [150, 67] Hqk={hqk} Hv={hv} {act}")
    compare_prefill(w, x, P.gpu_prefill(w, x))


def test_prefill_many_short_sequences():
    # 150 packed sequences (0..40 tokens): the kernels find their sequence
    # and chunk by scanning the lengths 64 sequences at a time.
    lens = [int(v) for v in np.random.default_rng(211).integers(0, 41, size=150)]
    w = wl.custom("prefill", len(lens), 1, 2, "bf16", seed=211, lengths=lens, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case prefill 150 sequences, T={sum(lens)} Hqk=1 Hv=2 bf16")
    compare_prefill(w, x, P.gpu_prefill(w, x))


def test_prefill_empty_call_passes_states_through():
    w = wl.custom("prefill", 3, 2, 4, "bf16", seed=203, lengths=[0, 0, 0], s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say("case all-empty prefill")
    got = P.gpu_prefill(w, x)
    assert np.array_equal(got["S_out"], x["S0"])
    assert np.array_equal(got["conv_out_bits"], x["conv0"])


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_decode_small(act):
    w = wl.custom("decode", 3, 2, 4, act, seed=204, steps=40, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case decode N=3 steps=40 Hqk=2 Hv=4 {act}")
    compare_decode(w, x, P.gpu_decode(w, x))


def test_decode_many_sequences():
    # 100 sequences: the prep kernel of each step scans them 64 at a time.
    w = wl.custom("decode", 100, 1, 2, "bf16", seed=212, steps=5, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say("case decode N=100 steps=5 Hqk=1 Hv=2 bf16")
    compare_decode(w, x, P.gpu_decode(w, x))


def test_workload1_tiny_fp32_full():
    w = wl.WORKLOADS[1]
    x = wl.generate(w)
    say(f"case {w.name}")
    compare_prefill(w, x, P.gpu_prefill(w, x))


# --------------------------------------------------- invariants on the GPU
def test_inplace_states_match_out_of_place():
    w = wl.custom("prefill", 2, 2, 4, "bf16", seed=205, lengths=[70, 3], s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say("case in-place states")
    a = P.gpu_prefill(w, x, inplace=False)
    b = P.gpu_prefill(w, x, inplace=True)
    for k in ("o", "y", "S_out", "conv_out_bits"):
        assert np.array_equal(a[k], b[k]), k


def test_varlen_packed_equals_separate_runs():
    lens = [130, 7, 64]
    w = wl.custom("prefill", 3, 2, 4, "bf16", seed=206, lengths=lens, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say("case packed vs separate")
    packed = P.gpu_prefill(w, x)
    cu = x["cu_seqlens"]
    for n in range(3):
        xs = P.slice_seqs(x, [n])
        ws = wl.custom("prefill", 1, 2, 4, "bf16", seed=206, lengths=[lens[n]])
        one = P.gpu_prefill(ws, xs)
        sl = slice(cu[n], cu[n + 1])
        for k in ("q", "k", "v", "beta", "g", "o", "y"):
            assert np.array_equal(one[k], packed[k][sl]), (k, n)
        assert np.array_equal(one["S_out"][0], packed["S_out"][n])
        assert np.array_equal(one["conv_out_bits"][0], packed["conv_out_bits"][n])


@pytest.mark.parametrize("split", [1, 2, 63, 64, 65])
def test_split_prefill_continuation(split):
    T = 150
    w = wl.custom("prefill", 1, 2, 4, "f32", seed=207, lengths=[T], s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case split continuation at {split}")
    whole = P.gpu_prefill(w, x)
    xa = dict(x, cu_seqlens=np.array([0, split], np.int32), qkv=x["qkv"][:split], z=x["z"][:split],
              b=x["b"][:split], a=x["a"][:split])
    ra = P.gpu_prefill(wl.custom("prefill", 1, 2, 4, "f32", 207, lengths=[split]), xa)
    xb = dict(x, cu_seqlens=np.array([0, T - split], np.int32), qkv=x["qkv"][split:], z=x["z"][split:],
              b=x["b"][split:], a=x["a"][split:], conv0=ra["conv_out"].cpu().numpy(), S0=ra["S_out"])
    rb = P.gpu_prefill(wl.custom("prefill", 1, 2, 4, "f32", 207, lengths=[T - split]), xb)
    P.check("y", np.concatenate([ra["y"], rb["y"]]), whole["y"], "f32")
    P.check("S_out", rb["S_out"], whole["S_out"], "f32")
    assert np.array_equal(rb["conv_out_bits"], whole["conv_out_bits"])


def test_prefill_equals_decode_loop():
    """The chunked form and the recurrent form, both on the GPU, agree."""
    steps = 130
    wd = wl.custom("decode", 2, 2, 4, "f32", seed=208, steps=steps, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(wd)
    say("case prefill vs decode loop")
    dec = P.gpu_decode(wd, x)
    xp = P.decode_as_packed(x)
    wp = wl.custom("prefill", 2, 2, 4, "f32", seed=208, lengths=[steps, steps])
    pre = P.gpu_prefill(wp, xp)
    d = np.swapaxes(dec["y"], 0, 1).reshape(2 * steps, 4, 128)
    P.check("y", pre["y"], d, "f32")
    P.check("S_out", pre["S_out"], dec["S_out"], "f32")


# ------------------------------------------------------- full workloads
def test_workload2_decode_batch1_full():
    w = wl.WORKLOADS[2]
    x = wl.generate(w)
    say(f"case {w.name}")
    compare_decode(w, x, P.gpu_decode(w, x))


def test_workload3_prefill_4096_full_size():
    w = wl.WORKLOADS[3]
    x = wl.generate(w)
    say(f"case {w.name}")
    got = P.gpu_prefill(w, x)
    compare_prefill(w, x, got, heads=[0, 7, 16, 31, 47])


def test_workload4_batched_decode_full_size():
    w = wl.WORKLOADS[4]
    x = wl.generate(w)
    say(f"case {w.name}")
    compare_decode(w, x, P.gpu_decode(w, x), seqs=[0, 21, 42, 63])


def test_workload5_varlen_full_size():
    w = wl.WORKLOADS[5]
    x = wl.generate(w)
    lens = np.diff(x["cu_seqlens"])
    say(f"case {w.name}: lengths {lens.tolist()} total {int(lens.sum())}")
    got = P.gpu_prefill(w, x)
    seqs = [int(np.argmin(lens)), int(np.argmax(lens))]
    compare_prefill(w, x, got, heads=[1, 18, 40], seqs=seqs)
