"""fp64 CPU oracle of the gated DeltaNet token mixer (ctypes over gdn_oracle.c).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code
with the HIP library and imports nothing from it; it takes plain numpy arrays.

The arithmetic lives in ``gdn_oracle.c`` (fp64, libm only). This wrapper only
converts arrays to contiguous fp64, allocates outputs and calls the C entry
points; ``layer`` chains the three steps in the order the xwen CLAUDE.md page
lists them (section "Architecture cheat sheet", gated DeltaNet paragraph), and
``block`` adds the projections before and after it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")

CONV_K = 4
L2_EPS = 1e-6
NORM_EPS = 1e-6
L2_CLAMP, L2_RSQRT = 0, 1   # L2-norm forms of q and k (see conv_gate_prep)

_lib = None


def build(force: bool = False, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (plain -O2, IEEE semantics, no fast-math)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off",
                        "-shared", "-fPIC", "-o", tmp, src, "-lm"], check=True)
        os.replace(tmp, out)
    return out


_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int)


def load(path: Optional[str] = None):
    """Load (building if needed) the oracle library. ``path`` loads another build."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    lib = ctypes.CDLL(path or build())
    lib.gdno_conv_gate_prep.argtypes = [ctypes.c_int, _I, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        _D, _D, _D, _D, _D, _D, _D, ctypes.c_double, ctypes.c_int,
                                        _D, _D, _D, _D, _D, _D]
    lib.gdno_conv_gate_prep.restype = None
    lib.gdno_delta_rule.argtypes = [ctypes.c_int, _I, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    _D, _D, _D, _D, _D, _D, _D, _D, _I, _D]
    lib.gdno_delta_rule.restype = None
    lib.gdno_gated_rmsnorm.argtypes = [ctypes.c_long, ctypes.c_int, _D, _D, _D, ctypes.c_double, _D]
    lib.gdno_gated_rmsnorm.restype = None
    lib.gdno_linear.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, _D, _D, _D]
    lib.gdno_linear.restype = None
    lib.gdno_in_proj.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 _D, _D, _D, _D, _D, _D, _D, _D, _D]
    lib.gdno_in_proj.restype = None
    for f in ("gdno_sigmoid", "gdno_softplus", "gdno_silu"):
        getattr(lib, f).argtypes = [ctypes.c_double]
        getattr(lib, f).restype = ctypes.c_double
    if path is None:
        _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(x: np.ndarray):
    return x.ctypes.data_as(_D)


def _cu(cu) -> np.ndarray:
    return np.ascontiguousarray(cu, dtype=np.int32)


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to bfloat16 precision (8 significant bits), to nearest
    with ties to even, returned as fp64. Finite inputs in bf16's normal range;
    this is how a value is stored in a bf16 tensor."""
    x = _f64(x)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


class Oracle:
    """Bound to one build of the oracle library (the default, or a test variant)."""

    def __init__(self, path: Optional[str] = None):
        self.lib = load(path)

    def sigmoid(self, x: float) -> float:
        return self.lib.gdno_sigmoid(float(x))

    def softplus(self, x: float) -> float:
        return self.lib.gdno_softplus(float(x))

    def silu(self, x: float) -> float:
        return self.lib.gdno_silu(float(x))

    def conv_gate_prep(self, cu, n_qk_heads: int, n_v_heads: int, head_dim: int,
                       qkv, b, a, conv_w, dt_bias, A_log, conv_in, l2_eps: float = L2_EPS,
                       l2_mode: int = L2_CLAMP):
        """Conv + SiLU + split + L2 norm + gates. Returns a dict of fp64 arrays.

        ``l2_mode``: L2_CLAMP (x / max(|x|, eps), the page's form) or L2_RSQRT
        (x / sqrt(sum x^2 + eps), the HF form the page notes)."""
        cu = _cu(cu)
        N, T = len(cu) - 1, int(cu[-1])
        Hqk, Hv, d = n_qk_heads, n_v_heads, head_dim
        C = d * (2 * Hqk + Hv)
        qkv, b, a = _f64(qkv).reshape(T, C), _f64(b).reshape(T, Hv), _f64(a).reshape(T, Hv)
        conv_w, dt_bias, A_log = _f64(conv_w).reshape(C, CONV_K), _f64(dt_bias), _f64(A_log)
        conv_in = _f64(conv_in).reshape(N, CONV_K - 1, C)
        out = dict(conv_out=np.empty((N, CONV_K - 1, C)), q=np.empty((T, Hqk, d)),
                   k=np.empty((T, Hqk, d)), v=np.empty((T, Hv, d)),
                   beta=np.empty((T, Hv)), g=np.empty((T, Hv)))
        self.lib.gdno_conv_gate_prep(N, cu.ctypes.data_as(_I), Hqk, Hv, d, _p(qkv), _p(b), _p(a),
                                     _p(conv_w), _p(dt_bias), _p(A_log), _p(conv_in), float(l2_eps), int(l2_mode),
                                     _p(out["conv_out"]), _p(out["q"]), _p(out["k"]), _p(out["v"]),
                                     _p(out["beta"]), _p(out["g"]))
        return out

    def delta_rule(self, cu, n_qk_heads: int, n_v_heads: int, head_dim: int,
                   q, k, v, beta, g, S_in, heads: Optional[Sequence[int]] = None):
        """Recurrent delta rule. Returns (o [T,Hv,d], S_out [N,Hv,d,d]).

        ``heads``: compute only these V-heads (others of o / S_out are NaN).
        """
        cu = _cu(cu)
        N, T = len(cu) - 1, int(cu[-1])
        Hqk, Hv, d = n_qk_heads, n_v_heads, head_dim
        q, k = _f64(q).reshape(T, Hqk, d), _f64(k).reshape(T, Hqk, d)
        v, beta, g = _f64(v).reshape(T, Hv, d), _f64(beta).reshape(T, Hv), _f64(g).reshape(T, Hv)
        S_in = _f64(S_in).reshape(N, Hv, d, d)
        o = np.full((T, Hv, d), np.nan)
        S_out = np.full((N, Hv, d, d), np.nan)
        sel = None
        if heads is not None:
            sel = np.zeros(Hv, np.int32)
            sel[list(heads)] = 1
        work = np.empty(d * d + 2 * d)
        self.lib.gdno_delta_rule(N, cu.ctypes.data_as(_I), Hqk, Hv, d, _p(q), _p(k), _p(v),
                                 _p(beta), _p(g), _p(S_in), _p(S_out), _p(o),
                                 sel.ctypes.data_as(_I) if sel is not None else None, _p(work))
        return o, S_out

    def gated_rmsnorm(self, o, z, w, eps: float = NORM_EPS):
        """Gated RMSNorm over the last axis (length d). Returns y, same shape as o."""
        o = _f64(o)
        d = o.shape[-1]
        z = _f64(z).reshape(o.shape)
        w = _f64(w)
        y = np.empty_like(o)
        self.lib.gdno_gated_rmsnorm(o.size // d, d, _p(o), _p(z), _p(w), float(eps), _p(y))
        return y

    def layer(self, cu, n_qk_heads: int, n_v_heads: int, head_dim: int, qkv, z, b, a,
              conv_w, dt_bias, A_log, norm_w, conv_in, S_in, heads=None,
              l2_eps: float = L2_EPS, norm_eps: float = NORM_EPS, l2_mode: int = L2_CLAMP):
        """The whole mixer: prep, recurrent delta rule, gated RMSNorm. fp64 dict out."""
        r = self.conv_gate_prep(cu, n_qk_heads, n_v_heads, head_dim, qkv, b, a, conv_w,
                                dt_bias, A_log, conv_in, l2_eps, l2_mode)
        o, S_out = self.delta_rule(cu, n_qk_heads, n_v_heads, head_dim, r["q"], r["k"], r["v"],
                                   r["beta"], r["g"], S_in, heads=heads)
        T = int(_cu(cu)[-1])
        zz = _f64(z).reshape(T, n_v_heads, head_dim)
        if heads is None:
            y = self.gated_rmsnorm(o, zz, norm_w, norm_eps)
        else:
            y = np.full_like(o, np.nan)
            hs = list(heads)
            y[:, hs] = self.gated_rmsnorm(o[:, hs], zz[:, hs], norm_w, norm_eps)
        r.update(o=o, S_out=S_out, y=y)
        return r


    def linear(self, x, W):
        """y = x W^T for x [..., n_in], W [n_out, n_in] (a Linear without bias)."""
        W = _f64(W)
        n_out, n_in = W.shape
        x = _f64(x)
        lead = x.shape[:-1]
        xx = x.reshape(-1, n_in)
        y = np.empty((xx.shape[0], n_out))
        self.lib.gdno_linear(xx.shape[0], n_in, n_out, _p(xx), _p(W), _p(y))
        return y.reshape(lead + (n_out,))

    def in_proj(self, n_qk_heads: int, n_v_heads: int, head_dim: int, x, w_qkv, w_gate, w_beta, w_alpha):
        """The four input projections of x [T, hidden]: dict of fp64 qkv [T, C],
        z [T, Hv, d], b [T, Hv], a [T, Hv]."""
        x = _f64(x)
        T, hidden = x.shape
        Hqk, Hv, d = n_qk_heads, n_v_heads, head_dim
        C = d * (2 * Hqk + Hv)
        ws = [_f64(w_qkv).reshape(C, hidden), _f64(w_gate).reshape(Hv * d, hidden),
              _f64(w_beta).reshape(Hv, hidden), _f64(w_alpha).reshape(Hv, hidden)]
        out = dict(qkv=np.empty((T, C)), z=np.empty((T, Hv, d)), b=np.empty((T, Hv)), a=np.empty((T, Hv)))
        self.lib.gdno_in_proj(T, hidden, Hqk, Hv, d, _p(x), *[_p(w) for w in ws],
                              _p(out["qkv"]), _p(out["z"]), _p(out["b"]), _p(out["a"]))
        return out

    def block(self, cu, n_qk_heads: int, n_v_heads: int, head_dim: int, x, w_qkv, w_gate, w_beta,
              w_alpha, w_out, conv_w, dt_bias, A_log, norm_w, conv_in, S_in, round_act: bool = True,
              round_o: bool = False, l2_eps: float = L2_EPS, norm_eps: float = NORM_EPS,
              l2_mode: int = L2_CLAMP):
        """The token-mixer block from the layer input x [T, hidden]: the input
        projections, the mixer's steps (conv/gates, delta rule, gated RMSNorm),
        then ssm_out (the page's gated DeltaNet paragraph, in its order).

        With ``round_act`` the tensors that cross the mixer's boundary (qkv,
        z, the logits in; y out) are rounded to bf16, the dtype they are
        stored in; with ``round_o`` also the readout o between the delta rule
        and the norm (a path that stores o in bf16 there). Returns the step
        outputs (as ``layer``) plus ``proj`` (the in-projections as the mixer
        saw them) and ``out`` [T, hidden]."""
        rnd = round_bf16 if round_act else _f64
        Hqk, Hv, d = n_qk_heads, n_v_heads, head_dim
        pr = {k: rnd(v) for k, v in self.in_proj(Hqk, Hv, d, x, w_qkv, w_gate, w_beta, w_alpha).items()}
        r = self.conv_gate_prep(cu, Hqk, Hv, d, pr["qkv"], pr["b"], pr["a"], conv_w, dt_bias, A_log, conv_in,
                                l2_eps, l2_mode)
        o, S_out = self.delta_rule(cu, Hqk, Hv, d, r["q"], r["k"], r["v"], r["beta"], r["g"], S_in)
        o_n = round_bf16(o) if (round_act and round_o) else o
        y = self.gated_rmsnorm(o_n, pr["z"], norm_w, norm_eps)
        T = pr["qkv"].shape[0]
        r.update(proj=pr, o=o, S_out=S_out, y=y, out=self.linear(rnd(y).reshape(T, Hv * d), w_out))
        return r


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


__all__ = ["Oracle", "default", "build", "load", "round_bf16", "CONV_K", "L2_EPS", "NORM_EPS"]
