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
