"""Parity of the HF form of the q/k L2 norm (gdn_config.l2_mode =
GDN_L2_RSQRT, x / sqrt(sum x^2 + eps)) with the oracle in the same form, on
every entry point that normalises q and k: the prep of prefill, the prep of
the three-call decode step and the fused decode step. Each case includes
near-zero q/k heads, where the two forms differ most."""
import sys

import numpy as np
import pytest

from gated_deltanet_layer_amd import workloads as wl
from tests import parity as P
from tests.test_gpu_parity import compare_decode, compare_prefill

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_prefill_rsqrt_form(act):
    w = wl.custom("prefill", 2, 2, 4, act, seed=320, lengths=[97, 40], s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case prefill l2 rsqrt {act}")
    got = P.gpu_prefill(w, x, l2_mode="rsqrt")
    compare_prefill(w, x, got, l2_mode="rsqrt")


@pytest.mark.parametrize("fused", [False, True])
def test_decode_rsqrt_form(fused):
    w = wl.custom("decode", 3, 2, 4, "bf16", seed=321, steps=24, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    say(f"case decode l2 rsqrt fused={fused}")
    got = P.gpu_decode_fused(w, x, l2_mode="rsqrt") if fused else P.gpu_decode(w, x, l2_mode="rsqrt")
    compare_decode(w, x, got, l2_mode="rsqrt")


def test_rsqrt_and_clamp_differ_on_small_heads():
    """With the conv weights of K-head 1 scaled to ~1e-4 its q, k norms fall
    near sqrt(eps): the two forms must give visibly different q, and each
    must match the oracle in its own form."""
    w = wl.custom("prefill", 1, 2, 2, "f32", seed=322, lengths=[33])
    x = wl.generate(w)
    d = w.head_dim
    x["conv_w"] = x["conv_w"].copy()
    x["conv_w"][d:2 * d] *= 1e-4          # q channels of K-head 1
    x["conv_w"][3 * d:4 * d] *= 1e-4      # k channels of K-head 1
    say("case clamp vs rsqrt on small heads")
    a = P.gpu_prefill(w, x, l2_mode="clamp")
    b = P.gpu_prefill(w, x, l2_mode="rsqrt")
    compare_prefill(w, x, a, l2_mode="clamp")
    compare_prefill(w, x, b, l2_mode="rsqrt")
    assert np.max(np.abs(a["q"][:, 1] - b["q"][:, 1])) > 1e-3
