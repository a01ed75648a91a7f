"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
each one makes at least one pin fail: a dropped term, a wrong sign, a wrong
index or a transposed operand anywhere in the oracle must not go unnoticed.

The mutants are built from temporary copies of gdn_oracle.c; the oracle
itself is not touched.
"""
import os

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

# (name, text to replace, replacement, replace every occurrence?)
MUTANTS = [
    ("delta_sign", "dl[c] = bt * (vv[c] - u[c])", "dl[c] = bt * (vv[c] + u[c])", False),
    ("delta_no_beta", "dl[c] = bt * (vv[c] - u[c])", "dl[c] = (vv[c] - u[c])", False),
    ("update_transposed", "S[(size_t)i * d + c] += kv[i] * dl[c]",
     "S[(size_t)c * d + i] += kv[i] * dl[c]", False),
    ("read_transposed", "acc += S[(size_t)i * d + c] * kv[i]",
     "acc += S[(size_t)c * d + i] * kv[i]", False),
    ("readout_transposed", "acc += S[(size_t)i * d + c] * qv[i]",
     "acc += S[(size_t)c * d + i] * qv[i]", False),
    ("readout_uses_k", "acc += S[(size_t)i * d + c] * qv[i]",
     "acc += S[(size_t)i * d + c] * kv[i]", False),
    ("head_map_interleave", "const int hk = j % Hqk;", "const int hk = j / (Hv / Hqk);", False),
    ("no_readout_scale", "ov[c] = scale * acc;", "ov[c] = acc;", False),
    ("no_decay", "const double decay = exp(g[tok * Hv + j]);", "const double decay = 1.0;", False),
    ("decay_sign", "const double decay = exp(g[tok * Hv + j]);",
     "const double decay = exp(-g[tok * Hv + j]);", False),
    ("conv_taps_reversed", "conv_w[(size_t)c * GDNO_CONV_K + j]",
     "conv_w[(size_t)c * GDNO_CONV_K + (GDNO_CONV_K - 1 - j)]", True),
    ("l2_hf_form", "const double den = nrm > l2_eps ? nrm : l2_eps;",
     "const double den = sqrt(ss + l2_eps);", False),
    ("l2_eps_on_square", "const double den = nrm > l2_eps ? nrm : l2_eps;",
     "const double den = ss > l2_eps ? nrm : l2_eps;", False),
    ("l2_rsqrt_eps_outside", "const double den_hf = sqrt(ss + l2_eps);",
     "const double den_hf = sqrt(ss) + l2_eps;", False),
    ("l2_rsqrt_no_eps", "const double den_hf = sqrt(ss + l2_eps);", "const double den_hf = sqrt(ss);", False),
    ("l2_mode_ignored", "dst[i] /= (l2_mode == 1 ? den_hf : den);", "dst[i] /= den;", False),
    ("g_no_dt_bias", "softplus(a[e] + dt_bias[jh])", "softplus(a[e])", False),
    ("g_no_exp", "-exp(A_log[jh]) * softplus", "-A_log[jh] * softplus", False),
    ("softplus_unstable_tail", "log1p(exp(-fabs(x)))", "log1p(exp(-x))", False),
    ("beta_sign", "beta[e] = sigmoid(b[e]);", "beta[e] = sigmoid(-b[e]);", False),
    ("rms_sum_not_mean", "sqrt(ss / d + eps)", "sqrt(ss + eps)", False),
    ("rms_eps_outside", "sqrt(ss / d + eps)", "(sqrt(ss / d) + eps)", False),
    ("gate_not_silu", "w[c] * silu(zrow[c])", "w[c] * zrow[c]", False),
    ("norm_weight_plus_one", "w[c] * silu(zrow[c])", "(1.0 + w[c]) * silu(zrow[c])", False),
    ("conv_state_rows", "const int src = L + r;", "const int src = r;", False),
    ("qk_no_silu", "dst[i] = silu(acc);\n                        ss +=",
     "dst[i] = acc;\n                        ss +=", False),
    ("qk_interleaved_split", "const int c0 = part * d * Hqk + h * d;",
     "const int c0 = part * d + h * 2 * d;", False),
    ("v_offset", "const int c0 = 2 * d * Hqk + jh * d;", "const int c0 = d * Hqk + jh * d;", False),
    ("sigmoid_wrong", "return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));", False),
    ("linear_transposed", "acc += wr[i] * xr[i];", "acc += W[(size_t)i * n_out + o] * xr[i];", False),
    ("linear_dropped_term", "for (int i = 0; i < n_in; ++i) acc", "for (int i = 1; i < n_in; ++i) acc", False),
    ("in_proj_beta_alpha_swapped", "gdno_linear(T, hidden, Hv, x, w_beta, b);",
     "gdno_linear(T, hidden, Hv, x, w_alpha, b);", False),
    ("in_proj_gate_weight", "gdno_linear(T, hidden, Hv * d, x, w_gate, z);",
     "gdno_linear(T, hidden, Hv * d, x, w_qkv, z);", False),
]


def _build_mutant(tmp_path, name, old, new, every):
    with open(SRC) as f:
        text = f.read()
    assert old in text, f"mutant {name}: pattern not found"
    text = text.replace(old, new) if every else text.replace(old, new, 1)
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    return oracle.build(force=True, src=str(src), out=str(tmp_path / f"lib{name}.so"))


@pytest.mark.parametrize("name,old,new,every", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, every):
    orc = oracle.Oracle(_build_mutant(tmp_path, name, old, new, every))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, FloatingPointError, ValueError, IndexError,
                ZeroDivisionError, RuntimeWarning):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
