"""Seeded random configurations through the three-call prefill, the fused
prefill and the fused decode step, each against the fp64 oracle on every
head and sequence.

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
