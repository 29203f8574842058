"""Pins of the FP8 (e4m3) variant's CPU reference: the rounding against
torch's float8_e4m3fn conversion and against the value table decoded from
the format definition, the block exponent rule, and the variant's error
against exact attention on the benchmark's input distribution."""

import math

import numpy as np
import torch

from oracle import isa_oracle as orc
from oracle import isa_oracle_fp8 as f8


def _e4m3_table():
    vals = []
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue  # NaN
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals.append(-v if s else v)
    return np.array(sorted(set(vals)))


def test_e4m3_round_matches_the_format_table_and_torch():
    table = _e4m3_table()
    assert table.max() == 448.0 and len(table) == 253  # +-0 merge, 254 finite codes
    np.testing.assert_array_equal(f8.e4m3_round(table), table)
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-3, 2.5, 20000),
                        (table[:-1] + table[1:]) / 2.0])          # every midpoint (ties)
    x = x[np.abs(x) <= 448.0]
    got = f8.e4m3_round(x)
    ref = torch.tensor(x, dtype=torch.float64).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, ref)
    # nearest by brute force on the table, ties to the even code
    i = np.searchsorted(table, x)
    lo, hi = table[np.clip(i - 1, 0, len(table) - 1)], table[np.clip(i, 0, len(table) - 1)]
    assert np.all(np.minimum(np.abs(x - lo), np.abs(x - hi)) == np.abs(x - got))


def test_block_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(1)
    amax = np.concatenate([10.0 ** rng.uniform(-30, 30, 5000), [448.0, 449.0, 224.0, 1.0, 896.0]])
    e = f8.block_exponent(amax)
    assert np.all(amax / np.exp2(e) <= 448.0)
    assert np.all(amax / np.exp2(e - 1) > 448.0)
    assert f8.block_exponent(np.array([0.0]))[0] == 0


def test_quantize_rows_is_exact_on_representable_blocks():
    rng = np.random.default_rng(2)
    table = _e4m3_table()
    X = rng.choice(table[np.abs(table) <= 8], size=(5, 64)) * 2.0 ** rng.integers(-5, 5, size=(5, 1))
    np.testing.assert_array_equal(f8.quantize_rows(X), X)


def test_fp8_error_budget_on_the_benchmark_distribution():
    """The evaluation behind the FP8 variant, on the benchmark's inputs
    (N(0,1) rows, 20 % of the queries sharpened towards a key): e4m3 logits
    cost well under a percent of the output norm, e4m3 probabilities and
    values a few percent each.  Queries that are large but aligned with no key
    make e4m3 logits far worse (about 10 %), which the second case shows."""
    from sparse_attention_context_amd.synth import make_inputs
    Q, K, V = make_inputs(1, 1, 128, 1536, 1536, seed=7, dtype="bf16")
    e = f8.error_budget(Q[0, 0, ::6], K[0, 0], V[0, 0])
    assert e["q,k"] < 1e-2, e
    assert 0.01 < e["v"] < 0.05 and 0.01 < e["p"] < 0.05 and e["q,k,p,v"] < 0.06, e
    rng = np.random.default_rng(3)
    q = rng.standard_normal((64, 128))
    q[::5] += 4 * rng.standard_normal((13, 128))
    e2 = f8.error_budget(q, rng.standard_normal((1536, 128)), rng.standard_normal((1536, 128)))
    assert e2["q,k"] > 0.05, e2


def test_fp8_rows_without_rounding_are_exact_attention():
    """With no operand rounded the FP8 route is softmax attention itself: the
    exp2-domain logits, the whole-number reference maximum and the unrounded
    row sum cancel exactly (up to fp64 rounding)."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((37, 64)) * 2.0
    Kt = rng.standard_normal((101, 64))
    Vt = rng.standard_normal((101, 64))
    got = f8.fp8_full_attention_rows(q, Kt, Vt, parts=())
    np.testing.assert_allclose(got, orc.full_attention_rows(q, Kt, Vt), rtol=1e-12, atol=1e-12)


def test_fp8_rows_are_exact_on_representable_operands():
    """Q, K and V built from e4m3 values whose every scale block holds an
    entry of magnitude 256..448 (times the block's power of two) have exact
    block scales, so rounding them changes nothing and the route equals exact
    attention.  V's blocks run along the keys (32 consecutive keys of one
    column, the short last block padded): its columns 0 and 32 are large and
    the others 2^-20 smaller, so blocks taken along a key row instead would
    carry the large scale and flush the small columns to zero."""
    rng = np.random.default_rng(5)
    table = _e4m3_table()
    mid = table[(np.abs(table) >= 1.0) & (np.abs(table) <= 448.0)]
    big = table[(np.abs(table) >= 256.0) & (np.abs(table) <= 448.0)]

    def qk_rows(n, d):                       # one big entry per (row, 32 columns)
        X = rng.choice(mid, size=(n, d))
        for j in range(0, d, 32):
            X[:, j] = rng.choice(big, size=n)
        return X / 64.0                      # a power of two keeps every block exact

    q = qk_rows(20, 64)
    Kt = qk_rows(70, 64)
    Vt = rng.choice(mid, size=(70, 64)) * 2.0 ** -20
    for i in range(0, 70, 32):               # one big entry per (column, 32 keys)
        Vt[i, :] = rng.choice(big, size=64) * 2.0 ** -20
    Vt[:, 0] = rng.choice(big, size=70)
    Vt[:, 32] = rng.choice(big, size=70)
    assert np.array_equal(f8.quantize_rows(q), q) and np.array_equal(f8.quantize_rows(Kt), Kt)
    got = f8.fp8_full_attention_rows(q, Kt, Vt, parts=("q", "k", "v"))
    ref = orc.full_attention_rows(q, Kt, Vt)
    # (per column: the columns differ in scale by 2^20, and a cancelling sum
    # carries the fp64 rounding of its column's magnitude)
    assert np.all(np.abs(got - ref) <= 1e-12 * np.abs(Vt).max(axis=0)[None, :])
    # the same values with scale blocks along the key rows lose the small columns
    wrong = f8.quantize_rows(Vt)
    assert np.abs(wrong[:, 1:32]).max() == 0.0
