"""Why every product of the chunked delta rule takes fp32-grade operands.

Runs the emulation in tests/precision_budget.py (per-product operand
precision: fp32, three-pass split bf16, one bf16 pass) on the 4,096-token
prefill workload (10 of its 48 V-heads) and checks the facts the kernels'
precision rests on, against the fp64 oracle at the bf16 bar:
  * split bf16 on every product meets the bar (as fp32 does);
  * one bf16 pass on every product, or q, k, v stored in bf16, does not;
  * one bf16 pass on any single product fails, except X = K S, which passes
    here only because the workload's decays are strong: the chunk-start
    state enters as exp(gam_r) K S, and exp(gam_r) is negligible past a
    chunk's first rows. With every log-decay scaled by 0.01 (first 2,048
    tokens) it fails too.
"""
import pytest

from tests.precision_budget import budget_table

HEADS = (0, 11, 22, 33, 44)
HEADS_FULL = (0, 5, 11, 17, 22, 28, 33, 39, 44, 47)


@pytest.fixture(scope="module")
def table():
    t = budget_table(T=4096, heads=HEADS_FULL)
    for name, r in t.items():
        print(f"{name:45s} y {r['y']:8.3f}  o {r['o']:8.3f}  S_out {r['S_out']:8.3f}")
    return t


def test_split_meets_the_bar(table):
    for name in ("split bf16 everywhere", "fp32 operands everywhere"):
        r = table[name]
        assert r["y"] <= 1.0 and r["o"] <= 1.0 and r["S_out"] <= 1.0, (name, r)


def test_single_pass_everywhere_fails(table):
    assert table["one bf16 pass everywhere"]["y"] > 1.0
    assert table["q, k, v stored in bf16 (products split)"]["y"] > 1.0


@pytest.mark.parametrize("product", ["gram", "QS", "TmR", "PD", "KtD"])
def test_single_pass_on_one_product_fails(table, product):
    assert table[f"one bf16 pass on {product} only"]["y"] > 1.0


def test_single_pass_on_state_read_passes_only_with_strong_decays(table):
    assert table["one bf16 pass on KS only"]["y"] <= 1.0
    weak = budget_table(T=2048, heads=HEADS, g_scale=0.01,
                        only=("split bf16 everywhere", "one bf16 pass on KS only"))
    assert weak["split bf16 everywhere"]["y"] <= 1.0
    assert weak["one bf16 pass on KS only"]["y"] > 1.0
