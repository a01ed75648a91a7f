"""Parity of the projections around the mixer (gdn_in_proj, gdn_out_proj) and
of the whole block (in-projections -> mixer -> ssm_out) with the fp64 oracle.

The projections round each fp32-accumulated output once to bf16: each
element must be a bf16 rounding of a value within the fp32 accumulation
error bound of the oracle's, and equal to the oracle's own rounding for all
but a rare few (sums near a rounding midpoint), on top of the bf16 bar. At the full sizes of the 27B and 35B-A3B layers
the oracle computes sampled rows (every column of them): the rows that open
and close 256-row and 128-row tiles, the first and last rows, and random ones.

In the block the oracle rounds qkv, z, the logits and y to bf16 as the HIP
path stores them (and the readout o where the path stores it in bf16: the
three-call prefill does, the fused decode step does not). The two sides
round values that differ in their last fp32 bits, so an element that lies
near a rounding midpoint can land on either neighbour: a stored bf16 value
is then one step (at most 2^-7 of its magnitude) from the oracle's. The
state and the conv state are held to the bf16 bar (the fp32 bar of the
mixer alone assumes identical inputs). ssm_out sums hundreds of stored y
values, so its bar adds what one step of every y can move an output:
    |out - ref| <= 2e-3 + 1e-2 |ref| + 2^-7 sum_k |y_k| |W_out[n][k]|
and, so that the slack cannot hide a systematic error, the median element
must sit well inside the plain bf16 bar."""
import sys

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_layer_amd import binding as B
from gated_deltanet_layer_amd import layer as Lyr
from gated_deltanet_layer_amd import workloads as wl
from tests import parity as P

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _f64(bits):
    return wl.bf16_to_f32(bits).astype(np.float64)


def _ordinal(bits):
    """bf16 bit patterns -> integers in value order (adjacent values differ by 1)."""
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def check_rounded(name, got, ref, absref, K):
    """A product rounded once from fp32 to bf16. The fp32 sum of K bf16
    products (exact in fp32) takes one rounding per 32-wide MFMA step and a
    few inside each, so it lies within E = (K/32 + 8) 2^-24 sum_k |x_k w_k|
    (``absref``) of the exact value; the stored element must be the bf16
    rounding of some value in [ref - E, ref + E]. It differs from the
    oracle's own rounding only for sums near a rounding midpoint (rare)."""
    P.check(name, got, ref, "bf16")
    E = (K / 32 + 8) * 2.0 ** -24 * absref
    og = _ordinal(wl.bf16_bits(np.asarray(got, np.float32)))
    lo = _ordinal(wl.bf16_bits(oracle.round_bf16(ref - E).astype(np.float32)))
    hi = _ordinal(wl.bf16_bits(oracle.round_bf16(ref + E).astype(np.float32)))
    bad = (og < lo) | (og > hi)
    assert not bad.any(), f"{name}: {int(bad.sum())} elements outside the rounding of [ref - E, ref + E]"
    frac = float(np.mean(og != _ordinal(wl.bf16_bits(oracle.round_bf16(ref).astype(np.float32)))))
    assert frac <= 2e-3, f"{name}: {frac:.2e} of the elements round differently from the oracle"


def _in_proj_gpu(cfg, x, hidden):
    t = {k: P.dev(x[k]) for k in ("x", "w_qkv", "w_gate", "w_beta", "w_alpha")}
    T = x["x"].shape[0]
    pr = Lyr._Proj(cfg, T, hidden, "cuda")
    pr.project_in(cfg, T, t["x"], t["w_qkv"], t["w_gate"], t["w_beta"], t["w_alpha"], None)
    torch.cuda.synchronize()
    return {k: P.host(getattr(pr, k)) for k in ("qkv", "z", "b", "a")}


def _in_proj_oracle(w, x, rows=None):
    xs = x["x"] if rows is None else x["x"][rows]
    return oracle.default().in_proj(w.n_qk_heads, w.n_v_heads, w.head_dim, _f64(xs), _f64(x["w_qkv"]),
                                    _f64(x["w_gate"]), _f64(x["w_beta"]), _f64(x["w_alpha"]))


def _in_proj_abs(w, x, rows=None):
    xs = x["x"] if rows is None else x["x"][rows]
    a = lambda k: np.abs(_f64(x[k]))
    return oracle.default().in_proj(w.n_qk_heads, w.n_v_heads, w.head_dim, np.abs(_f64(xs)), a("w_qkv"),
                                    a("w_gate"), a("w_beta"), a("w_alpha"))


def _check_in_proj(w, x, got, rows=None):
    ref = _in_proj_oracle(w, x, rows)
    absref = _in_proj_abs(w, x, rows)
    K = x["x"].shape[-1]
    for k in ("qkv", "z", "b", "a"):
        g = got[k] if rows is None else got[k][rows]
        check_rounded(f"in_proj {k}", g.reshape(ref[k].shape), ref[k], absref[k], K)


def _rows(T, seed):
    base = {0, 1, T - 1, T - 2}
    # Tiles are 256 rows, and 128 in the half-height tiles that take the
    # last column tiles when a launch's last round would be mostly idle.
    for t in range(127, T, 128):
        base.update({t, min(t + 1, T - 1)})
    rng = np.random.default_rng(seed)
    base.update(int(r) for r in rng.integers(0, T, 4))
    return sorted(r for r in base if 0 <= r < T)


# Row counts up to 16 take the column-split kernel (1 to 5 column fragments
# of 16 per block by width), 17 to 64 the tiled kernel with 32- or 64-row
# tiles (32 to 96 columns; rows past the count are clamped on load and
# masked on store), more its 256-row tiles; 4096 rows x 2576 columns run 256
# tiles of 256 rows and the last 5 column tiles as 128-row tiles.
@pytest.mark.parametrize("T,hidden,heads", [(1, 64, (1, 1)), (20, 128, (2, 6)), (40, 192, (2, 4)),
                                            (5, 64, (16, 64)), (64, 128, (16, 48)), (77, 128, (2, 6)),
                                            (300, 192, (2, 4)), (513, 256, (4, 4)), (256, 320, (1, 2)),
                                            (4096, 256, (2, 8)), (64, 128, (16, 16)), (17, 64, (1, 2)),
                                            (33, 192, (2, 4)), (48, 256, (16, 32))])
def test_in_proj_small(T, hidden, heads):
    hqk, hv = heads
    w = wl.custom("prefill", 1, hqk, hv, "bf16", seed=400 + T, lengths=[T])
    x = wl.generate_block(w, hidden)
    say(f"case in_proj T={T} hidden={hidden} Hqk={hqk} Hv={hv}")
    cfg = B.make_config(hqk, hv, "bf16")
    _check_in_proj(w, x, _in_proj_gpu(cfg, x, hidden))


@pytest.mark.parametrize("T,hv", [(4096, 48), (64, 48), (64, 32), (1, 32)])
def test_in_proj_full_size_sampled(T, hv):
    hidden = wl.HIDDEN[hv]
    w = wl.custom("prefill", 1, 16, hv, "bf16", seed=410 + hv, lengths=[T])
    x = wl.generate_block(w, hidden)
    say(f"case in_proj full size T={T} hidden={hidden} Hv={hv}")
    got = _in_proj_gpu(B.make_config(16, hv, "bf16"), x, hidden)
    rows = _rows(T, 7) if T > 64 else list(range(T))
    _check_in_proj(w, x, got, rows)


def _out_proj_gpu(cfg, x, hidden):
    T = x["y"].shape[0]
    pr = Lyr._Proj(cfg, T, hidden, "cuda")
    y = P.dev(x["y"])
    pr.project_out(cfg, T, y, P.dev(x["w_out"]), None)
    torch.cuda.synchronize()
    return P.host(pr.out)


@pytest.mark.parametrize("T,hidden,hv,full", [(1, 64, 1, False), (77, 200, 6, False), (513, 256, 4, False),
                                              (4096, 5120, 48, True), (64, 2048, 32, True),
                                              (4096, 2720, 16, True), (64, 5120, 48, True), (17, 128, 2, False),
                                              (33, 192, 4, False), (48, 2048, 32, True)])
def test_out_proj(T, hidden, hv, full):
    hqk = 16 if full else 1
    w = wl.custom("prefill", 1, hqk, hv, "bf16", seed=420 + T + hv, lengths=[T])
    x = wl.generate_block(w, hidden)
    say(f"case out_proj T={T} hidden={hidden} Hv={hv}")
    got = _out_proj_gpu(B.make_config(hqk, hv, "bf16"), x, hidden)
    rows = _rows(T, 8) if full and T > 64 else list(range(T))
    ref = oracle.default().linear(_f64(x["y"][rows]), _f64(x["w_out"]))
    absref = oracle.default().linear(np.abs(_f64(x["y"][rows])), np.abs(_f64(x["w_out"])))
    check_rounded("out_proj", got[rows], ref, absref, hv * 128)


def _check_block_out(name, got, ref, w_out_bits):
    """The derived bar for the block output (see the module docstring)."""
    y = np.abs(oracle.round_bf16(ref["y"])).reshape(got.shape[0], -1)
    slack = 2.0 ** -7 * (y @ np.abs(_f64(w_out_bits)).T)
    bar = P.BF16_ATOL + P.BF16_RTOL * np.abs(ref["out"])
    err = np.abs(got - ref["out"])
    worst = float(np.max(err / (bar + slack)))
    med = float(np.median(err / bar))
    assert worst <= 1.0, f"{name}: worst error is {worst:.3f}x the derived bar"
    assert med <= 0.25, f"{name}: median error is {med:.3f}x the bf16 bar"


def _oracle_block(w, x, hidden, round_o):
    xf = {k: (_f64(v) if v.dtype == np.uint16 else v) for k, v in x.items()}
    xf = {k: (v.astype(np.float64) if v.dtype == np.float32 else v) for k, v in xf.items()}
    return oracle.default().block(xf["cu_seqlens"], w.n_qk_heads, w.n_v_heads, w.head_dim, xf["x"],
                                  xf["w_qkv"], xf["w_gate"], xf["w_beta"], xf["w_alpha"], xf["w_out"],
                                  xf["conv_w"], xf["dt_bias"], xf["A_log"], xf["norm_w"], xf["conv0"], xf["S0"],
                                  round_o=round_o)


@pytest.mark.parametrize("lengths,heads,hidden", [([150, 77], (2, 4), 256), ([64, 1, 0, 200], (1, 2), 128)])
def test_block_prefill(lengths, heads, hidden):
    hqk, hv = heads
    w = wl.custom("prefill", len(lengths), hqk, hv, "bf16", seed=430 + hidden, lengths=lengths,
                  s0_std=0.02, conv0_std=1.0)
    x = wl.generate_block(w, hidden)
    say(f"case block prefill lengths={lengths} Hqk={hqk} Hv={hv} hidden={hidden}")
    cfg = B.make_config(hqk, hv, "bf16")
    cu = x["cu_seqlens"]
    N, T = len(cu) - 1, int(cu[-1])
    t = {k: P.dev(v) for k, v in x.items() if k != "y"}
    run = Lyr.Block(cfg, N, T, hidden)
    conv_out = torch.empty_like(t["conv0"])
    S_out = torch.empty_like(t["S0"])
    out = run(t["cu_seqlens"], t["x"], t["w_qkv"], t["w_gate"], t["w_beta"], t["w_alpha"], t["w_out"],
              t["conv_w"], t["dt_bias"], t["A_log"], t["norm_w"], t["conv0"], conv_out, t["S0"], S_out)
    torch.cuda.synchronize()
    ref = _oracle_block(w, x, hidden, round_o=True)     # the prefill stores o in bf16 before the norm
    _check_block_out("block out", P.host(out), ref, x["w_out"])
    P.check("block S_out", P.host(S_out), ref["S_out"], "bf16")
    P.check("block conv_out", P.host(conv_out), ref["conv_out"], "bf16")


def test_block_decode():
    """Decode steps through the block (one token per sequence per step) equal
    the oracle's block over the same tokens packed by sequence."""
    steps, N, hqk, hv, hidden = 12, 3, 2, 4, 192
    w = wl.custom("decode", N, hqk, hv, "bf16", seed=440, steps=steps, s0_std=0.02, conv0_std=1.0)
    x = wl.generate_block(w, hidden)
    say(f"case block decode N={N} steps={steps} Hqk={hqk} Hv={hv} hidden={hidden}")
    cfg = B.make_config(hqk, hv, "bf16")
    t = {k: P.dev(v) for k, v in x.items() if k != "y"}
    run = Lyr.DecodeBlock(cfg, N, hidden, t["conv0"].clone())
    S = t["S0"].clone()
    outs = []
    for s in range(steps):
        o = run(t["x"][s], t["w_qkv"], t["w_gate"], t["w_beta"], t["w_alpha"], t["w_out"], t["conv_w"],
                t["dt_bias"], t["A_log"], t["norm_w"], S)
        outs.append(P.host(o).copy())
    torch.cuda.synchronize()
    got = np.stack(outs)                                   # [steps, N, hidden]
    packed = dict(x)
    packed["x"] = np.ascontiguousarray(np.swapaxes(x["x"], 0, 1).reshape(N * steps, hidden))
    packed["cu_seqlens"] = (np.arange(N + 1) * steps).astype(np.int32)
    ref = _oracle_block(w, packed, hidden, round_o=False)   # the fused step keeps o in fp32
    _check_block_out("decode block out", np.swapaxes(got, 0, 1).reshape(N * steps, hidden), ref, x["w_out"])
    P.check("decode block S", P.host(S), ref["S_out"], "bf16")
