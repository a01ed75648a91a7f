"""Element offsets past 2^31 through every entry point's kernels.

Token and sequence counts are 32-bit at the boundary, but the element offsets
the kernels form from them (token x channels, (sequence x V-heads + head) x
128 x 128, row x columns) pass 2^31 at sizes that fit one GPU. Each case puts
a small seeded problem at the far end of large buffers whose other tokens or
sequences are zeros, and checks it against the fp64 oracle on the small
problem alone:

  * two packed sequences: a filler sequence of zeros, then the sequence under
    test with its own initial states (the filler never touches them);
  * one sequence whose leading tokens are zeros, with zero initial states:
    zero q, k and v rows leave a zero state exactly zero (the decay multiplies
    zero, the update adds beta (v - S^T k) k^T = 0) and read out exactly
    zero, so the tokens after them compute what the same tokens compute as a
    sequence of their own from zero states. The filler's length is not a
    multiple of the 64-token chunk, so one chunk holds both kinds of token.
    With one sequence the fused call folds the gated RMSNorm into the
    sequential kernel's launch, with two it launches it on its own;
  * decode with thousands of sequences of zeros before the two under test;
  * the projections with hundreds of thousands of zero rows before the rows
    under test.

The arithmetic follows the xwen CLAUDE.md page, section "Architecture cheat
sheet", gated DeltaNet paragraph (the oracle's source). About 50 GB of device
memory at most, freed after each case.
"""
import sys

import numpy as np
import pytest
import torch

from gated_deltanet_layer_amd import binding as B
from gated_deltanet_layer_amd import layer as Lyr
from gated_deltanet_layer_amd import workloads as wl
from tests import parity as P
from tests.test_gpu_edge_cases import check_verify_prefix
from tests.test_gpu_parity import compare_decode, compare_prefill
from tests.test_gpu_proj import _check_in_proj, _f64, check_rounded

import oracle

pytestmark = pytest.mark.gpu

HQK, HV, D = 16, 48, 128
C = D * (2 * HQK + HV)
LIM = 2 ** 31
# Tokens before the sequence under test: token x C and token x Hv x 128
# (q, k, v rows; z, o and y rows) both pass 2^31.
T_FILL = 360_037
assert T_FILL * C > LIM and T_FILL * HV * D > LIM and T_FILL % 64 != 0


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _prefill_big(x, one_sequence: bool):
    """Device inputs: T_FILL zero tokens, then the small problem's tokens;
    the filler is a sequence of its own unless one_sequence."""
    L = int(x["cu_seqlens"][-1])
    T = T_FILL + L
    bf = dict(dtype=torch.bfloat16, device="cuda")
    t = dict(qkv=torch.zeros(T, C, **bf), z=torch.zeros(T, HV, D, **bf), b=torch.zeros(T, HV, **bf),
             a=torch.zeros(T, HV, **bf))
    for k in ("qkv", "z", "b", "a"):
        t[k][T_FILL:] = P.dev(x[k])
    for k in ("conv_w", "dt_bias", "A_log", "norm_w"):
        t[k] = P.dev(x[k])
    if one_sequence:
        t["cu_seqlens"] = P.dev(np.array([0, T], np.int32))
        t["conv0"], t["S0"] = P.dev(x["conv0"]), P.dev(x["S0"])
    else:
        t["cu_seqlens"] = P.dev(np.array([0, T_FILL, T], np.int32))
        t["conv0"] = torch.cat([torch.zeros_like(P.dev(x["conv0"])), P.dev(x["conv0"])])
        t["S0"] = torch.cat([torch.zeros_like(P.dev(x["S0"])), P.dev(x["S0"])])
    return t, T


@pytest.mark.parametrize("one_sequence", [True, False], ids=["one_sequence", "two_sequences"])
@pytest.mark.parametrize("path", ["fused", "three_call"])
def test_prefill_past_2g_elements(path, one_sequence):
    L = 197
    # One sequence: its initial states are zero, as the filler before the
    # tokens under test requires.
    std = 0.0 if one_sequence else 0.02
    w = wl.custom("prefill", 1, HQK, HV, "bf16", seed=940 + one_sequence, lengths=[L], s0_std=std,
                  conv0_std=0.0 if one_sequence else 1.0)
    x = wl.generate(w)
    say(f"case prefill {path} past 2^31 elements: {T_FILL} filler tokens "
        f"({'same' if one_sequence else 'own'} sequence) + {L}, Hqk={HQK} Hv={HV} bf16")
    t, T = _prefill_big(x, one_sequence)
    N = 1 if one_sequence else 2
    cfg = B.make_config(HQK, HV, "bf16")
    run = (Lyr.PrefillFused if path == "fused" else Lyr.Prefill)(cfg, N, T)
    conv_out, S_out = torch.empty_like(t["conv0"]), torch.empty_like(t["S0"])
    run(t["cu_seqlens"], t["qkv"], t["z"], t["b"], t["a"], t["conv_w"], t["dt_bias"], t["A_log"], t["norm_w"],
        t["conv0"], conv_out, t["S0"], S_out)
    torch.cuda.synchronize()
    got = dict(y=P.host(run.y[T_FILL:]), S_out=P.host(S_out[N - 1:]), conv_out_bits=P.bits(conv_out[N - 1:]))
    if path == "three_call":
        for k in ("q", "k", "v", "beta", "g", "o"):
            got[k] = P.host(getattr(run, k)[T_FILL:])
    del run, t, conv_out, S_out
    _free()
    compare_prefill(w, x, got)


N_FILL = 2_740   # sequences before the two under test: (n Hv + j) x 128 x 128 passes 2^31
assert N_FILL * HV * D * D > LIM


def _decode_big(x):
    steps = x["qkv"].shape[0]
    N = N_FILL + 2
    bf = dict(dtype=torch.bfloat16, device="cuda")
    t = dict(qkv=torch.zeros(steps, N, C, **bf), z=torch.zeros(steps, N, HV, D, **bf),
             b=torch.zeros(steps, N, HV, **bf), a=torch.zeros(steps, N, HV, **bf),
             conv0=torch.zeros(N, 3, C, **bf), S0=torch.zeros(N, HV, D, D, dtype=torch.float32, device="cuda"))
    for k in ("qkv", "z", "b", "a"):
        t[k][:, N_FILL:] = P.dev(x[k])
    t["conv0"][N_FILL:] = P.dev(x["conv0"])
    t["S0"][N_FILL:] = P.dev(x["S0"])
    for k in ("conv_w", "dt_bias", "A_log", "norm_w"):
        t[k] = P.dev(x[k])
    return t, N


@pytest.mark.parametrize("path", ["fused", "three_call"])
def test_decode_past_2g_state_elements(path):
    w = wl.custom("decode", 2, HQK, HV, "bf16", seed=950, steps=3, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    steps = x["qkv"].shape[0]
    say(f"case decode {path} past 2^31 state elements: {N_FILL} zero sequences + 2, {steps} steps, "
        f"Hqk={HQK} Hv={HV} bf16")
    t, N = _decode_big(x)
    cfg = B.make_config(HQK, HV, "bf16")
    ys = torch.empty_like(t["z"])
    S = t["S0"]
    if path == "fused":
        run = Lyr.DecodeFused(cfg, N, t["conv0"])
    else:
        run = Lyr.Decode(cfg, N)
    for s in range(steps):
        if path == "fused":
            run(t["qkv"][s], t["z"][s], t["b"][s], t["a"][s], t["conv_w"], t["dt_bias"], t["A_log"],
                t["norm_w"], S, ys[s])
        else:
            run(t["qkv"][s], t["z"][s], t["b"][s], t["a"][s], t["conv_w"], t["dt_bias"], t["A_log"],
                t["norm_w"], t["conv0"], S, ys[s])
    torch.cuda.synchronize()
    conv = run.conv_state if path == "fused" else t["conv0"]
    got = dict(y=P.host(ys[:, N_FILL:]), S_out=P.host(S[N_FILL:]), conv_out_bits=P.bits(conv[N_FILL:]))
    del run, t, ys, S, conv
    _free()
    compare_decode(w, x, got)


def test_verify_past_2g_snapshot_elements():
    w = wl.custom("decode", 2, HQK, HV, "bf16", seed=951, steps=2, s0_std=0.02, conv0_std=1.0)
    x = wl.generate(w)
    K = x["qkv"].shape[0]
    say(f"case verify past 2^31 snapshot elements: {N_FILL} zero sequences + 2, K={K}, Hqk={HQK} Hv={HV} bf16")
    t, N = _decode_big(x)
    cfg = B.make_config(HQK, HV, "bf16")
    seq_major = lambda a: a.transpose(0, 1).contiguous()          # [K][N] -> [N][K]
    qkv, z, b, a = (seq_major(t[k]) for k in ("qkv", "z", "b", "a"))
    conv_snap = torch.empty((N, K, 3, C), dtype=torch.bfloat16, device="cuda")
    S_snap = torch.empty((N, K, HV, D, D), dtype=torch.float32, device="cuda")
    y = torch.empty_like(z)
    B.gdn_decode_verify(cfg, N, K, qkv, b, a, z, t["conv_w"], t["dt_bias"], t["A_log"], t["norm_w"],
                        t["conv0"], conv_snap, t["S0"], S_snap, y)
    torch.cuda.synchronize()
    got_y, got_S, got_conv = P.host(y[N_FILL:]), P.host(S_snap[N_FILL:]), P.bits(conv_snap[N_FILL:])
    del t, qkv, z, b, a, conv_snap, S_snap, y
    _free()
    for m in (K, 1):
        check_verify_prefix(w, x, got_y, got_S, got_conv, m, [0, 1])


M_FILL = 420_000   # rows before the 64 under test: row x 5120 and row x 10240 pass 2^31
assert M_FILL * 5120 > LIM


def test_projections_past_2g_elements():
    hidden, rows = wl.HIDDEN[HV], 64
    w = wl.custom("prefill", 1, HQK, HV, "bf16", seed=960, lengths=[rows])
    x = wl.generate_block(w, hidden)
    M = M_FILL + rows
    say(f"case projections past 2^31 elements: {M_FILL} zero rows + {rows}, hidden={hidden} Hv={HV}")
    cfg = B.make_config(HQK, HV, "bf16")
    xb = torch.zeros(M, hidden, dtype=torch.bfloat16, device="cuda")
    xb[M_FILL:] = P.dev(x["x"])
    pr = Lyr._Proj(cfg, M, hidden, "cuda")
    pr.project_in(cfg, M, xb, P.dev(x["w_qkv"]), P.dev(x["w_gate"]), P.dev(x["w_beta"]), P.dev(x["w_alpha"]), None)
    torch.cuda.synchronize()
    got = {k: P.host(getattr(pr, k)[M_FILL:]) for k in ("qkv", "z", "b", "a")}
    del xb
    yb = torch.zeros(M, HV * D, dtype=torch.bfloat16, device="cuda")
    yb[M_FILL:] = P.dev(x["y"])
    pr.project_out(cfg, M, yb, P.dev(x["w_out"]), None)
    torch.cuda.synchronize()
    got_out = P.host(pr.out[M_FILL:])
    del pr, yb
    _free()
    _check_in_proj(w, x, got)
    ref = oracle.default().linear(_f64(x["y"]), _f64(x["w_out"]))
    absref = oracle.default().linear(np.abs(_f64(x["y"])), np.abs(_f64(x["w_out"])))
    check_rounded("out_proj", got_out, ref, absref, HV * D)
