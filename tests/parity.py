"""Shared helpers of the GPU parity tests: seeded inputs on the device, the
HIP path run through the C ABI, the oracle on the same bytes, and the
tolerance checks.

Tolerances (the stated bar, read elementwise):
  * bf16 activations: |gpu - ref| <= 2e-3 + 1e-2 |ref| for every element of
    o, y and the final delta state.
  * fp32 activations: max |gpu - ref| <= 1e-5 max |ref| per tensor.
  * The fp32 intermediates q, k, v, beta, g meet the fp32 bar in every
    configuration; the conv state is a copy of raw inputs and must match bit
    for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from gated_deltanet_layer_amd import binding as B
from gated_deltanet_layer_amd import layer as Lyr
from gated_deltanet_layer_amd import workloads as wl

F32_RTOL = 1e-5
BF16_ATOL, BF16_RTOL = 2e-3, 1e-2


def dev(x: np.ndarray) -> torch.Tensor:
    """numpy -> GPU tensor; uint16 arrays are bf16 bit patterns."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a tensor (for exact comparisons)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def f32_ratio(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)) / (F32_RTOL * max(np.max(np.abs(ref)), 1e-30)))


def bf16_ratio(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (BF16_ATOL + BF16_RTOL * np.abs(ref))))


def check(name: str, got, ref, act: str, report: dict = None):
    """Assert the bar for `act`; returns the worst ratio (<= 1 passes)."""
    got = np.asarray(got)
    assert np.all(np.isfinite(got)), f"{name}: non-finite GPU values"
    r = f32_ratio(got, ref) if act == "f32" else bf16_ratio(got, ref)
    if report is not None:
        report[name] = r
    assert r <= 1.0, f"{name}: worst error is {r:.3f}x the {act} tolerance"
    return r


def inputs_f64(x: dict, act: str) -> dict:
    """Exact fp64 values of the generated inputs (bf16 bits widened exactly)."""
    out = {}
    for k, v in x.items():
        if k in ("qkv", "z", "b", "a", "conv0"):
            out[k] = wl.as_f32(v, act).astype(np.float64)
        elif v.dtype == np.int32:
            out[k] = v
        else:
            out[k] = v.astype(np.float64)
    return out


def oracle_layer(w: wl.Workload, xf: dict, cu, heads=None, l2_mode: str = "clamp"):
    return oracle.default().layer(cu, w.n_qk_heads, w.n_v_heads, w.head_dim, xf["qkv"], xf["z"], xf["b"],
                                  xf["a"], xf["conv_w"], xf["dt_bias"], xf["A_log"], xf["norm_w"],
                                  xf["conv0"], xf["S0"], heads=heads,
                                  l2_mode=oracle.L2_RSQRT if l2_mode == "rsqrt" else oracle.L2_CLAMP)


def gpu_prefill(w: wl.Workload, x: dict, inplace: bool = False, l2_mode: str = "clamp"):
    """Run prep -> chunked prefill -> gated RMSNorm on the GPU; host copies of every output."""
    cfg = B.make_config(w.n_qk_heads, w.n_v_heads, w.act, l2_mode=l2_mode)
    cu = x["cu_seqlens"]
    N, T = len(cu) - 1, int(cu[-1])
    run = Lyr.Prefill(cfg, N, T)
    t = {k: dev(v) for k, v in x.items()}
    conv_out = t["conv0"] if inplace else torch.empty_like(t["conv0"])
    S_out = t["S0"] if inplace else torch.empty_like(t["S0"])
    run(t["cu_seqlens"], t["qkv"], t["z"], t["b"], t["a"], t["conv_w"], t["dt_bias"], t["A_log"],
        t["norm_w"], t["conv0"], conv_out, t["S0"], S_out)
    torch.cuda.synchronize()
    return dict(q=host(run.q), k=host(run.k), v=host(run.v), beta=host(run.beta), g=host(run.g),
                o=host(run.o), y=host(run.y), S_out=host(S_out), conv_out=conv_out,
                conv_out_bits=bits(conv_out))


def gpu_prefill_fused(w: wl.Workload, x: dict, inplace: bool = False, l2_mode: str = "clamp"):
    """Run the whole mixer as one gdn_prefill_fused call on the GPU; host
    copies of y and the states."""
    cfg = B.make_config(w.n_qk_heads, w.n_v_heads, w.act, l2_mode=l2_mode)
    cu = x["cu_seqlens"]
    N, T = len(cu) - 1, int(cu[-1])
    run = Lyr.PrefillFused(cfg, N, T)
    t = {k: dev(v) for k, v in x.items()}
    conv_out = t["conv0"] if inplace else torch.empty_like(t["conv0"])
    S_out = t["S0"] if inplace else torch.empty_like(t["S0"])
    run(t["cu_seqlens"], t["qkv"], t["z"], t["b"], t["a"], t["conv_w"], t["dt_bias"], t["A_log"],
        t["norm_w"], t["conv0"], conv_out, t["S0"], S_out)
    torch.cuda.synchronize()
    return dict(y=host(run.y), S_out=host(S_out), conv_out=conv_out, conv_out_bits=bits(conv_out))


def gpu_decode(w: wl.Workload, x: dict, l2_mode: str = "clamp"):
    """Run the decode loop (prep -> step -> norm per step) on the GPU.
    Returns y, o [steps, N, Hv, d], final S and conv state."""
    cfg = B.make_config(w.n_qk_heads, w.n_v_heads, w.act, l2_mode=l2_mode)
    steps, N = x["qkv"].shape[:2]
    run = Lyr.Decode(cfg, N)
    t = {k: dev(v) for k, v in x.items()}
    conv, S = t["conv0"].clone(), t["S0"].clone()
    ys = torch.empty_like(t["z"])
    os_ = torch.empty(ys.shape, dtype=ys.dtype, device=ys.device)
    for s in range(steps):
        run(t["qkv"][s], t["z"][s], t["b"][s], t["a"][s], t["conv_w"], t["dt_bias"], t["A_log"], t["norm_w"],
            conv, S, ys[s])
        os_[s].copy_(run.o)
    torch.cuda.synchronize()
    return dict(y=host(ys), o=host(os_), S_out=host(S), conv_out_bits=bits(conv), conv_out=conv)


def gpu_decode_fused(w: wl.Workload, x: dict, l2_mode: str = "clamp"):
    """Run the decode loop as one gdn_decode_fused launch per step on the GPU.
    Returns y [steps, N, Hv, d], final S and conv state."""
    cfg = B.make_config(w.n_qk_heads, w.n_v_heads, w.act, l2_mode=l2_mode)
    steps, N = x["qkv"].shape[:2]
    t = {k: dev(v) for k, v in x.items()}
    run = Lyr.DecodeFused(cfg, N, t["conv0"].clone())
    S = t["S0"].clone()
    ys = torch.empty_like(t["z"])
    for s in range(steps):
        run(t["qkv"][s], t["z"][s], t["b"][s], t["a"][s], t["conv_w"], t["dt_bias"], t["A_log"], t["norm_w"],
            S, ys[s])
    torch.cuda.synchronize()
    conv = run.conv_state
    return dict(y=host(ys), S_out=host(S), conv_out_bits=bits(conv), conv_out=conv)


def decode_as_packed(x: dict, seqs=None) -> dict:
    """Decode streams [steps, N, ...] -> packed prefill layout (sequence-major)."""
    steps, N = x["qkv"].shape[:2]
    seqs = list(range(N)) if seqs is None else list(seqs)
    out = dict(x)
    for k in ("qkv", "z", "b", "a"):
        a = np.swapaxes(x[k][:, seqs], 0, 1)
        out[k] = np.ascontiguousarray(a.reshape((len(seqs) * steps,) + a.shape[2:]))
    out["conv0"] = x["conv0"][seqs]
    out["S0"] = x["S0"][seqs]
    out["cu_seqlens"] = (np.arange(len(seqs) + 1) * steps).astype(np.int32)
    return out


def slice_seqs(x: dict, seqs) -> dict:
    """The packed inputs of a subset of sequences."""
    cu = x["cu_seqlens"]
    out = dict(x)
    idx = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs]) if len(seqs) else np.zeros(0, int)
    for k in ("qkv", "z", "b", "a"):
        out[k] = np.ascontiguousarray(x[k][idx])
    out["conv0"] = x["conv0"][list(seqs)]
    out["S0"] = x["S0"][list(seqs)]
    lens = [int(cu[n + 1] - cu[n]) for n in seqs]
    out["cu_seqlens"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return out
