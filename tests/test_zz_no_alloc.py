"""gdn_prefill_fused_static (the allocation-free prefill, for callers that
cannot allocate device memory) against gdn_prefill_fused with a caller
workspace, through the C ABI.

Both run the same kernels, so their outputs must be identical bit for bit
(stronger than the parity bar). Two calls in a row share the device's static
scratch: the first at the 4,096-token prefill shape (16 K-heads, 48 V-heads),
the second a smaller packed call, so a second call that read anything the
first left behind would show. A call needing more scratch than the library
holds is rejected before anything is launched."""
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


def run_both(w, x):
    cfg = B.make_config(w.n_qk_heads, w.n_v_heads, w.act)
    cu = x["cu_seqlens"]
    N, T = len(cu) - 1, int(cu[-1])
    t = {k: P.dev(v) for k, v in x.items()}
    ref = Lyr.PrefillFused(cfg, N, T)
    conv_a, S_a = torch.empty_like(t["conv0"]), torch.empty_like(t["S0"])
    ref(t["cu_seqlens"], t["qkv"], t["z"], t["b"], t["a"], t["conv_w"], t["dt_bias"], t["A_log"], t["norm_w"],
        t["conv0"], conv_a, t["S0"], S_a)
    conv_b, S_b = torch.empty_like(t["conv0"]), torch.empty_like(t["S0"])
    y_b = torch.empty_like(ref.y)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    B.gdn_prefill_fused_static(cfg, N, T, t["cu_seqlens"], t["qkv"], t["b"], t["a"], t["z"], t["conv_w"],
                               t["dt_bias"], t["A_log"], t["norm_w"], t["conv0"], conv_b, t["S0"], S_b, y_b)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert np.array_equal(P.bits(y_b), P.bits(ref.y)), "y differs"
    assert np.array_equal(P.bits(S_b), P.bits(S_a)), "S_out differs"
    assert np.array_equal(P.bits(conv_b), P.bits(conv_a)), "conv state differs"
    return P.host(y_b)


def test_static_scratch_two_calls_match_workspace_call():
    w1 = wl.WORKLOADS[3]
    x1 = wl.generate(w1)
    say("case static scratch call 1: T=4096 Hqk=16 Hv=48 bf16")
    y1 = run_both(w1, x1)
    assert np.all(np.isfinite(y1))
    w2 = wl.custom("prefill", 3, 2, 6, "bf16", seed=440, lengths=[70, 0, 129], s0_std=0.02, conv0_std=1.0)
    x2 = wl.generate(w2)
    say("case static scratch call 2: 3 sequences (70, 0, 129 tokens) Hqk=2 Hv=6 bf16")
    y2 = run_both(w2, x2)
    # The second call's output also meets the parity bar against the oracle.
    ref = P.oracle_layer(w2, P.inputs_f64(x2, "bf16"), x2["cu_seqlens"])
    P.check("y", y2, ref["y"], "bf16")


def test_static_scratch_rejects_oversize_call():
    import ctypes
    cfg = B.make_config(16, 48, "bf16")
    T = 8192
    assert B.gdn_prefill_fused_workspace_bytes(cfg, 1, T) > B.GDN_STATIC_SCRATCH_BYTES
    dummy = torch.zeros(16, dtype=torch.uint8, device="cuda").data_ptr()
    s = B.load().gdn_prefill_fused_static(ctypes.byref(cfg), 1, T, *([dummy] * 15), None)
    assert s == B.GDN_E_TOO_LARGE
