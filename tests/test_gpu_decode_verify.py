"""gdn_decode_verify: K tokens per sequence in one launch with the state and
conv state after every token as snapshot planes, most recent first.

Checked two ways: bit for bit against K consecutive gdn_decode_fused steps
(the same per-token arithmetic), and against the fp64 oracle, whose layer
over the first m tokens of each sequence gives the state that plane K - m
must hold."""
import sys

import numpy as np
import pytest
import torch

from gated_deltanet_layer_amd import binding as B
from gated_deltanet_layer_amd import layer as Lyr
from gated_deltanet_layer_amd import workloads as wl
from tests import parity as P

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_verify(w, x):
    """One gdn_decode_verify call over the decode workload's steps as K tokens."""
    cfg = B.make_config(w.n_qk_heads, w.n_v_heads, w.act)
    K, N = x["qkv"].shape[:2]
    t = {k: P.dev(v) for k, v in x.items()}
    seq_major = lambda a: a.transpose(0, 1).contiguous()          # [K][N] -> [N][K]
    qkv, z, b, a = (seq_major(t[k]) for k in ("qkv", "z", "b", "a"))
    Hv, d = w.n_v_heads, w.head_dim
    conv_snap = torch.empty((N, K) + tuple(t["conv0"].shape[1:]), dtype=t["conv0"].dtype, device="cuda")
    S_snap = torch.empty((N, K, Hv, d, d), dtype=torch.float32, device="cuda")
    y = torch.empty_like(z)
    B.gdn_decode_verify(cfg, N, K, qkv, b, a, z, t["conv_w"], t["dt_bias"], t["A_log"], t["norm_w"],
                        t["conv0"], conv_snap, t["S0"], S_snap, y)
    torch.cuda.synchronize()
    return y, S_snap, conv_snap


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("heads", [(2, 4), (2, 6)])
def test_verify_equals_fused_steps(act, heads):
    hqk, hv = heads
    w = wl.custom("decode", 3, hqk, hv, act, seed=330 + hv, steps=5, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    K, N = x["qkv"].shape[:2]
    say(f"case verify K={K} N={N} Hqk={hqk} Hv={hv} {act} vs fused steps")
    y, S_snap, conv_snap = run_verify(w, x)
    cfg = B.make_config(hqk, hv, act)
    t = {k: P.dev(v) for k, v in x.items()}
    run = Lyr.DecodeFused(cfg, N, t["conv0"].clone())
    S = t["S0"].clone()
    ys = torch.empty_like(t["z"])
    for s in range(K):
        run(t["qkv"][s], t["z"][s], t["b"][s], t["a"][s], t["conv_w"], t["dt_bias"], t["A_log"], t["norm_w"],
            S, ys[s])
        torch.cuda.synchronize()
        plane = K - 1 - s
        assert np.array_equal(P.bits(S_snap[:, plane]), P.bits(S)), f"S plane {plane}"
        assert np.array_equal(P.bits(conv_snap[:, plane]), P.bits(run.conv_state)), f"conv plane {plane}"
    assert np.array_equal(P.bits(y), P.bits(ys.transpose(0, 1).contiguous())), "y"


def test_verify_against_oracle_prefixes():
    w = wl.custom("decode", 2, 2, 4, "bf16", seed=335, steps=6, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    K, N = x["qkv"].shape[:2]
    say(f"case verify K={K} N={N} vs oracle")
    y, S_snap, conv_snap = run_verify(w, x)
    Hv, d = w.n_v_heads, w.head_dim
    for m in (K, K - 2, 1):                      # accepted prefix length m <-> plane K - m
        xm = dict(x)
        for k in ("qkv", "z", "b", "a"):
            xm[k] = x[k][:m]
        xp = P.decode_as_packed(xm)
        ref = P.oracle_layer(w, P.inputs_f64(xp, w.act), xp["cu_seqlens"])
        rep = {}
        P.check("S_plane", P.host(S_snap[:, K - m]), ref["S_out"], w.act, rep)
        got_y = P.host(y[:, :m]).reshape(N * m, Hv, d)
        P.check("y", got_y, ref["y"], w.act, rep)
        ref_conv = ref["conv_out"].astype(np.float32)
        assert np.array_equal(P.bits(conv_snap[:, K - m]), wl.bf16_bits(ref_conv)), f"conv plane {K - m}"
        say(f"  prefix {m}: " + ", ".join(f"{k}={v:.3f}" for k, v in rep.items()))
