"""C ABI checks that need no GPU: the library loads, exports every entry point
include/gdn.h declares, and its host-side validation rejects bad arguments
before anything is launched (every call here fails validation or returns
early, so no HIP work is issued)."""
import ctypes
import os
import re

import pytest

from gated_deltanet_layer_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from gated_deltanet_layer_amd import build
        build.build()
    return B.load()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"GDN_API\s+[\w\s\*]+?\b(gdn_\w+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert declared_symbols() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_only_abi_symbols_are_exported(lib):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    mine = sorted({ln.split()[-1] for ln in out.splitlines() if " T " in ln and ln.split()[-1].startswith("gdn_")})
    assert mine == declared_symbols()


def test_status_strings_and_version(lib):
    assert B.status_string(0) == "ok"
    assert "workspace" in B.status_string(B.GDN_E_WORKSPACE)
    assert lib.gdn_version().decode().startswith("gdn-mi355x")


def test_default_config(lib):
    c = lib.gdn_default_config(16, 48, B.GDN_BF16)
    assert (c.n_qk_heads, c.n_v_heads, c.head_dim, c.conv_kernel, c.act_dtype) == (16, 48, 128, 4, B.GDN_BF16)
    assert c.l2_eps == pytest.approx(1e-6) and c.norm_eps == pytest.approx(1e-6)


def test_workspace_size(lib):
    cfg = B.make_config(16, 48)
    # (ceil(T/64) + N) chunks x (Hqk x K, Q operands + Hv x (Tm, P operands + 64 fp64))
    chunks = 64 + 1
    assert B.gdn_prefill_workspace_bytes(cfg, 1, 4096) == chunks * (16 * 2 * 64 * 128 * 4 + 48 * (2 * 64 * 64 * 4 + 64 * 8))
    assert B.gdn_prefill_workspace_bytes(cfg, 1, 0) == 0
    # Fused: the chunked workspace, o (act dtype) and one 128-byte ready
    # counter per (chunk, V-head), each part starting 256-byte aligned.
    up = lambda v: (v + 255) // 256 * 256
    for act, asz in (("bf16", 2), ("f32", 4)):
        c = B.make_config(16, 48, act)
        for n, t in ((1, 4096), (3, 1000), (2, 1)):
            ch = (t + 63) // 64 + n
            base = ch * (16 * 2 * 64 * 128 * 4 + 48 * (2 * 64 * 64 * 4 + 64 * 8))
            assert B.gdn_prefill_fused_workspace_bytes(c, n, t) == up(up(base) + t * 48 * 128 * asz) + ch * 48 * 128
    assert B.gdn_prefill_fused_workspace_bytes(cfg, 1, 0) == 0
    bad = B.make_config(16, 40)
    assert B.gdn_prefill_workspace_bytes(bad, 1, 64) == 0


FAKE = [0x100000 * (i + 1) for i in range(20)]   # distinct, never dereferenced


def _decode(lib, cfg, n, ptrs):
    return lib.gdn_decode_step(ctypes.byref(cfg), n, *ptrs, None)


def test_decode_validation(lib):
    cfg = B.make_config(2, 4)
    p = FAKE[:8]
    assert _decode(lib, cfg, 0, p) == B.GDN_OK                       # nothing to do
    assert _decode(lib, cfg, -1, p) == B.GDN_E_INVALID_ARG
    assert _decode(lib, cfg, 1, [None] + p[1:]) == B.GDN_E_INVALID_ARG
    assert _decode(lib, B.make_config(2, 3), 1, p) == B.GDN_E_INVALID_ARG   # Hv % Hqk
    assert _decode(lib, B.make_config(2, 4, head_dim=64), 1, p) == B.GDN_E_UNSUPPORTED
    assert _decode(lib, B.make_config(2, 4, conv_kernel=3), 1, p) == B.GDN_E_UNSUPPORTED
    neg = B.make_config(2, 4)
    neg.norm_eps = -1.0
    assert _decode(lib, neg, 1, p) == B.GDN_E_INVALID_ARG
    bad_dtype = B.make_config(2, 4)
    bad_dtype.act_dtype = 7
    assert _decode(lib, bad_dtype, 1, p) == B.GDN_E_INVALID_ARG
    # o overlapping v: rejected.
    q = p[:]
    q[7] = q[2] + 64
    assert _decode(lib, cfg, 1, q) == B.GDN_E_INVALID_ARG
    # S_out overlapping S_in partially: rejected.
    q = p[:]
    q[6] = q[5] + 4096
    assert _decode(lib, cfg, 1, q) == B.GDN_E_INVALID_ARG
    assert lib.gdn_decode_step(None, 1, *p, None) == B.GDN_E_INVALID_ARG


def test_prefill_validation(lib):
    cfg = B.make_config(2, 4)
    need = B.gdn_prefill_workspace_bytes(cfg, 1, 100)
    args = lambda ws, wsb, n=1, t=100: (ctypes.byref(cfg), n, t, *FAKE[:9], ws, wsb, None)
    base = list(args(FAKE[10], need))
    assert lib.gdn_prefill_chunked(*args(None, 0)) == B.GDN_E_WORKSPACE
    assert lib.gdn_prefill_chunked(*args(FAKE[10], need - 1)) == B.GDN_E_WORKSPACE
    assert lib.gdn_prefill_chunked(*args(FAKE[10], need, n=0, t=5)) == B.GDN_E_INVALID_ARG
    assert lib.gdn_prefill_chunked(*args(FAKE[10], need, n=0, t=0)) == B.GDN_OK
    bad = base[:]
    bad[3] = None    # cu_seqlens
    assert lib.gdn_prefill_chunked(*bad) == B.GDN_E_INVALID_ARG


def test_prep_and_norm_validation(lib):
    cfg = B.make_config(2, 4)
    p = FAKE[:14]
    assert lib.gdn_conv_gate_prep(ctypes.byref(cfg), 0, 0, *p, None) == B.GDN_OK
    assert lib.gdn_conv_gate_prep(ctypes.byref(cfg), 1, -3, *p, None) == B.GDN_E_INVALID_ARG
    nulls = p[:]
    nulls[0] = None  # cu_seqlens
    assert lib.gdn_conv_gate_prep(ctypes.byref(cfg), 1, 4, *nulls, None) == B.GDN_E_INVALID_ARG
    # q overlapping the qkv input: rejected.
    ov = p[:]
    ov[10] = ov[1] + 16
    assert lib.gdn_conv_gate_prep(ctypes.byref(cfg), 1, 4, *ov, None) == B.GDN_E_INVALID_ARG
    assert lib.gdn_gated_rmsnorm(ctypes.byref(cfg), 0, *FAKE[:4], None) == B.GDN_OK
    assert lib.gdn_gated_rmsnorm(ctypes.byref(cfg), -1, *FAKE[:4], None) == B.GDN_E_INVALID_ARG
    assert lib.gdn_gated_rmsnorm(ctypes.byref(cfg), 4, None, *FAKE[1:4], None) == B.GDN_E_INVALID_ARG
    yz = FAKE[:4]
    yz = [yz[0], yz[1], yz[2], yz[1] + 16]   # y overlapping z
    assert lib.gdn_gated_rmsnorm(ctypes.byref(cfg), 4, *yz, None) == B.GDN_E_INVALID_ARG


def test_decode_fused_validation(lib):
    cfg = B.make_config(2, 4)
    p = FAKE[:13]   # qkv, b, a, z, conv_w, dt_bias, A_log, norm_w, conv_in, conv_out, S_in, S_out, y
    call = lambda n, ptrs, c=cfg: lib.gdn_decode_fused(ctypes.byref(c), n, *ptrs, None)
    assert call(0, p) == B.GDN_OK
    assert call(-1, p) == B.GDN_E_INVALID_ARG
    for i in range(13):
        q = p[:]
        q[i] = None
        assert call(1, q) == B.GDN_E_INVALID_ARG, i
    # The new conv state may not be the old one (other blocks still read it).
    q = p[:]
    q[9] = q[8]
    assert call(1, q) == B.GDN_E_INVALID_ARG
    # y overlapping z, S_out partly overlapping S_in: rejected.
    q = p[:]
    q[12] = q[3] + 8
    assert call(1, q) == B.GDN_E_INVALID_ARG
    q = p[:]
    q[11] = q[10] + 4096
    assert call(1, q) == B.GDN_E_INVALID_ARG
    assert call(1, p, B.make_config(2, 4, head_dim=64)) == B.GDN_E_UNSUPPORTED
    assert lib.gdn_decode_fused(None, 1, *p, None) == B.GDN_E_INVALID_ARG


def test_l2_mode_validation(lib):
    c = lib.gdn_default_config(2, 4, B.GDN_BF16)
    assert c.l2_mode == B.GDN_L2_CLAMP
    assert B.make_config(2, 4, l2_mode="rsqrt").l2_mode == B.GDN_L2_RSQRT
    bad = B.make_config(2, 4)
    bad.l2_mode = 5
    p = FAKE[:8]
    assert lib.gdn_decode_step(ctypes.byref(bad), 1, *p, None) == B.GDN_E_INVALID_ARG
    with pytest.raises(ValueError):
        B.make_config(2, 4, l2_mode="hf")


def test_decode_verify_validation(lib):
    cfg = B.make_config(2, 4)
    p = FAKE[:13]   # qkv, b, a, z, conv_w, dt_bias, A_log, norm_w, conv_in, conv_snap, S_in, S_snap, y
    call = lambda n, k, ptrs: lib.gdn_decode_verify(ctypes.byref(cfg), n, k, *ptrs, None)
    assert call(0, 4, p) == B.GDN_OK
    assert call(2, 0, p) == B.GDN_OK
    assert call(2, -1, p) == B.GDN_E_INVALID_ARG
    q = p[:]
    q[11] = q[10]               # snapshot planes on top of S_in with K > 1
    assert call(1, 2, q) == B.GDN_E_INVALID_ARG
    q = p[:]
    q[9] = q[8]                 # conv snapshots on top of the old conv state
    assert call(1, 3, q) == B.GDN_E_INVALID_ARG
    q = p[:]
    q[3] = None
    assert call(1, 3, q) == B.GDN_E_INVALID_ARG


def test_checkpoint_and_guard_validation(lib):
    cfg = B.make_config(2, 4)
    need = B.gdn_prefill_workspace_bytes(cfg, 1, 200)
    args = lambda every, cap, sck: (ctypes.byref(cfg), 1, 200, *FAKE[:9], every, cap, sck, FAKE[12], need, None)
    assert lib.gdn_prefill_chunked_ckpt(*args(100, 2, FAKE[11])) == B.GDN_E_INVALID_ARG   # not a multiple of 64
    assert lib.gdn_prefill_chunked_ckpt(*args(-64, 2, FAKE[11])) == B.GDN_E_INVALID_ARG
    assert lib.gdn_prefill_chunked_ckpt(*args(64, 2, None)) == B.GDN_E_INVALID_ARG
    c = (ctypes.byref(cfg), 1, 200, FAKE[0], FAKE[1], FAKE[2])
    assert lib.gdn_conv_state_ckpt(*c, 0, 2, FAKE[3], None) == B.GDN_E_INVALID_ARG     # every >= 1
    assert lib.gdn_conv_state_ckpt(*c, 5, 0, FAKE[3], None) == B.GDN_OK               # nothing to write
    assert lib.gdn_conv_state_ckpt(*c, 5, 2, FAKE[1] + 8, None) == B.GDN_E_INVALID_ARG  # overlaps qkv
    assert lib.gdn_state_check(FAKE[0], 16, None, None) == B.GDN_E_INVALID_ARG
    assert lib.gdn_state_check(FAKE[0] + 4, 16, FAKE[1], None) == B.GDN_E_INVALID_ARG  # S not 16-byte aligned
    assert lib.gdn_state_check(FAKE[0], -1, FAKE[1], None) == B.GDN_E_INVALID_ARG


def test_projection_validation(lib):
    cfg = B.make_config(2, 4, "bf16")
    p = FAKE[:9]   # x, w_qkv, w_gate, w_beta, w_alpha, qkv, z, beta_logit, alpha_logit
    call = lambda t, h, ptrs, c=cfg: lib.gdn_in_proj(ctypes.byref(c), t, h, *ptrs, None)
    assert call(0, 64, p) == B.GDN_OK
    assert call(-1, 64, p) == B.GDN_E_INVALID_ARG
    assert call(4, 0, p) == B.GDN_E_INVALID_ARG
    assert call(4, 96, p) == B.GDN_E_UNSUPPORTED          # hidden not a multiple of 64
    assert call(4, 64, p, B.make_config(2, 4, "f32")) == B.GDN_E_UNSUPPORTED
    for i, bad in ((0, FAKE[0] + 8), (1, FAKE[1] + 8), (6, FAKE[6] + 1)):   # misaligned operands
        q = p[:]
        q[i] = bad
        assert call(4, 64, q) == B.GDN_E_INVALID_ARG, i
    q = p[:]
    q[6] = q[5] + 2                                       # z overlaps qkv
    assert call(4, 64, q) == B.GDN_E_INVALID_ARG
    q = p[:]
    q[5] = q[0]                                           # qkv on top of x
    assert call(4, 64, q) == B.GDN_E_INVALID_ARG
    q = p[:]
    q[3] = None
    assert call(4, 64, q) == B.GDN_E_INVALID_ARG

    out = lambda t, h, y, w, o, c=cfg: lib.gdn_out_proj(ctypes.byref(c), t, h, y, w, o, None)
    assert out(0, 80, *FAKE[:3]) == B.GDN_OK
    assert out(2, 0, *FAKE[:3]) == B.GDN_E_INVALID_ARG
    assert out(2, 80, *FAKE[:3], c=B.make_config(2, 4, "f32")) == B.GDN_E_UNSUPPORTED
    assert out(2, 80, FAKE[0], FAKE[1], FAKE[0] + 64) == B.GDN_E_INVALID_ARG   # out overlaps y
    assert out(2, 80, FAKE[0] + 2, FAKE[1], FAKE[2]) == B.GDN_E_INVALID_ARG    # y misaligned
    assert out(2, 80, FAKE[0], None, FAKE[2]) == B.GDN_E_INVALID_ARG


def test_prefill_fused_validation(lib):
    cfg = B.make_config(2, 4, "bf16")
    need = B.gdn_prefill_fused_workspace_bytes(cfg, 2, 100)
    base = B.gdn_prefill_workspace_bytes(cfg, 2, 100)
    assert need >= base + 100 * 4 * 128 * 2 and need % 2 == 0
    # qkv, b, a, z, conv_w, dt_bias, A_log, norm_w, conv_in, conv_out, S_in, S_out, y, ws
    p = FAKE[:14]
    call = lambda t, ptrs, ws_bytes=need, n=2: lib.gdn_prefill_fused(ctypes.byref(cfg), n, t, FAKE[15], *ptrs,
                                                                  ws_bytes, None)
    assert call(100, p, need - 1) == B.GDN_E_WORKSPACE
    q = p[:]
    q[13] = FAKE[13] + 64                  # workspace not 256-byte aligned
    assert call(100, q) == B.GDN_E_WORKSPACE
    q = p[:]
    q[0] = FAKE[0] + 8                     # qkv not 16-byte aligned
    assert call(100, q) == B.GDN_E_INVALID_ARG
    q = p[:]
    q[12] = q[3]                           # y on top of z
    assert call(100, q) == B.GDN_E_INVALID_ARG
    q = p[:]
    q[9] = q[8] + 256                      # conv states partly overlapping
    assert call(100, q) == B.GDN_E_INVALID_ARG
    q = p[:]
    q[3] = None
    assert call(100, q) == B.GDN_E_INVALID_ARG
    assert call(5, p, need, n=0) == B.GDN_E_INVALID_ARG     # tokens without sequences
    assert call(0, p, 0, n=0) == B.GDN_OK


def test_misaligned_vector_pointers_are_rejected(lib):
    """Every pointer a kernel reads or writes with vector accesses must meet
    the alignment gdn.h states for it; an offset pointer is GDN_E_INVALID_ARG
    (and nothing is launched)."""
    cfg = B.make_config(2, 4, "bf16")
    f32 = B.make_config(2, 4, "f32")
    # gdn_gated_rmsnorm: o, z, y, norm_w 16 bytes.
    for i in range(4):
        p = FAKE[:4]
        p[i] += 8
        assert lib.gdn_gated_rmsnorm(ctypes.byref(cfg), 4, *p, None) == B.GDN_E_INVALID_ARG, i
    # gdn_decode_step: q, k, v, S_in, S_out 16 bytes; o 4 values (8 bytes bf16, 16 fp32).
    for i, off in ((0, 8), (1, 8), (2, 8), (5, 8), (6, 8), (7, 4)):
        p = FAKE[:8]
        p[i] += off
        assert _decode(lib, cfg, 1, p) == B.GDN_E_INVALID_ARG, i
    p = FAKE[:8]
    p[7] += 8
    assert _decode(lib, f32, 1, p) == B.GDN_E_INVALID_ARG
    # gdn_decode_fused: S_in, S_out, norm_w, conv_w 16 bytes; z, y 4 values; qkv, conv states 2 values.
    for i, off in ((10, 8), (11, 8), (7, 8), (4, 8), (3, 4), (12, 4), (0, 2), (8, 2), (9, 2)):
        p = FAKE[:13]
        p[i] += off
        assert lib.gdn_decode_fused(ctypes.byref(cfg), 1, *p, None) == B.GDN_E_INVALID_ARG, i
    # gdn_decode_verify: the same pointers.
    p = FAKE[:13]
    p[11] += 8
    assert lib.gdn_decode_verify(ctypes.byref(cfg), 1, 2, *p, None) == B.GDN_E_INVALID_ARG
    # gdn_conv_gate_prep: conv_w 16; qkv and conv states 2 values; q, k, v 8 bytes.
    for i, off in ((4, 8), (1, 2), (7, 2), (8, 2), (9, 4), (10, 4), (11, 4)):
        p = FAKE[:14]
        p[i] += off
        assert lib.gdn_conv_gate_prep(ctypes.byref(cfg), 1, 4, *p, None) == B.GDN_E_INVALID_ARG, i
    # gdn_prefill_chunked: q, k, v 16 bytes; o 4 values.
    need = B.gdn_prefill_workspace_bytes(cfg, 1, 100)
    for i, off in ((1, 8), (2, 8), (3, 8), (8, 4)):
        p = FAKE[:9]
        p[i] += off
        assert lib.gdn_prefill_chunked(ctypes.byref(cfg), 1, 100, *p, FAKE[10], need, None) == B.GDN_E_INVALID_ARG, i
    # gdn_prefill_fused: z, y, norm_w 16 bytes too.
    need = B.gdn_prefill_fused_workspace_bytes(cfg, 2, 100)
    for i in (3, 7, 12):
        p = FAKE[:14]
        p[i] += 8
        assert lib.gdn_prefill_fused(ctypes.byref(cfg), 2, 100, FAKE[15], *p, need, None) == B.GDN_E_INVALID_ARG, i
    # gdn_conv_state_ckpt: qkv, conv_state_in, conv_ckpt 2 values.
    c = (ctypes.byref(cfg), 1, 200)
    assert lib.gdn_conv_state_ckpt(*c, FAKE[0], FAKE[1] + 2, FAKE[2], 5, 2, FAKE[3], None) == B.GDN_E_INVALID_ARG
    assert lib.gdn_conv_state_ckpt(*c, FAKE[0], FAKE[1], FAKE[2], 5, 2, FAKE[3] + 2, None) == B.GDN_E_INVALID_ARG


def test_static_scratch_entry_point_limits(lib):
    """gdn_prefill_fused_static checks its size against the static scratch
    before touching the device: an oversize call is GDN_E_TOO_LARGE, a bad
    config or count is rejected as in gdn_prefill_fused, an empty call is a
    no-op."""
    cfg = B.make_config(16, 48, "bf16")
    p = FAKE[:15]
    call = lambda n, t, c=cfg: lib.gdn_prefill_fused_static(ctypes.byref(c), n, t, *p, None)
    assert B.gdn_prefill_fused_workspace_bytes(cfg, 1, 4096) <= B.GDN_STATIC_SCRATCH_BYTES
    assert B.gdn_prefill_fused_workspace_bytes(cfg, 1, 8192) > B.GDN_STATIC_SCRATCH_BYTES
    assert call(1, 8192) == B.GDN_E_TOO_LARGE
    assert call(-1, 10) == B.GDN_E_INVALID_ARG
    assert call(1, 64, B.make_config(16, 48, head_dim=64)) == B.GDN_E_UNSUPPORTED
    assert call(0, 0) == B.GDN_OK
    assert "static scratch" in B.status_string(B.GDN_E_TOO_LARGE)


def test_prefill_fused_ckpt_validation(lib):
    cfg = B.make_config(2, 4, "bf16")
    need = B.gdn_prefill_fused_workspace_bytes(cfg, 2, 100)
    p = FAKE[:13]   # qkv, b, a, z, conv_w, dt_bias, A_log, norm_w, conv_in, conv_out, S_in, S_out, y
    call = lambda every, cap, sck, cck: lib.gdn_prefill_fused_ckpt(ctypes.byref(cfg), 2, 100, FAKE[15], *p, every, cap,
                                                                   sck, cck, FAKE[13], need, None)
    assert call(100, 2, FAKE[16], None) == B.GDN_E_INVALID_ARG            # not a multiple of 64
    assert call(-64, 2, FAKE[16], None) == B.GDN_E_INVALID_ARG
    assert call(64, 2, None, None) == B.GDN_E_INVALID_ARG                # planes missing
    assert call(64, 2, FAKE[16], FAKE[16]) == B.GDN_E_INVALID_ARG        # S and conv planes overlap
    assert call(64, 2, FAKE[0] + 64, None) == B.GDN_E_INVALID_ARG        # S planes on top of qkv
    assert call(64, 2, FAKE[16], FAKE[17] + 2) == B.GDN_E_INVALID_ARG    # conv planes misaligned
