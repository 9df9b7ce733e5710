"""Pins of the fp8-QK flavour's oracle (oracle/fp8.py).

The E4M3 value set is built here from the format's fields (sign, exponent with bias 7, 3-bit
mantissa, zero exponent = subnormals, the all-ones pattern excluded), independently of the
rounding code; the whole-pass checks use closed forms (a constant V, equal logits, inputs that
E4M3 holds exactly) and the distance to the exact result under the format's error bound.
"""
import math

import numpy as np
import pytest

from oracle import dense, fp8, solattn


def e4m3_values():
    vals = []
    for ex in range(16):
        for m in range(8):
            if ex == 15 and m == 7:
                continue                                    # the NaN pattern
            vals.append(m / 8 * 2.0 ** -6 if ex == 0 else (1 + m / 8) * 2.0 ** (ex - 7))
    return np.array(vals)


def test_every_format_value_is_fixed_and_the_range_is_right():
    v = e4m3_values()
    assert v.size == 127 and v.max() == 448.0 and np.sort(v)[1] == 2.0 ** -9
    np.testing.assert_array_equal(fp8.e4m3_round(v), v)
    np.testing.assert_array_equal(fp8.e4m3_round(-v), -v)


def test_ties_go_to_the_even_mantissa():
    v = np.sort(e4m3_values())
    mids = (v[1:] + v[:-1]) / 2
    got = fp8.e4m3_round(mids)
    # the even neighbour is the one whose index in the ordered value list is even (codes and
    # order coincide for non-negative values)
    lo_even = (np.arange(v.size - 1) % 2) == 0
    np.testing.assert_array_equal(got, np.where(lo_even, v[:-1], v[1:]))
    np.testing.assert_array_equal(fp8.e4m3_round(-mids), -got)


def test_rounding_is_nearest_within_the_format_bounds():
    rng = np.random.default_rng(3)
    x = np.copysign(2.0 ** rng.uniform(-12, 8.8, 20000), rng.standard_normal(20000))
    x = x[np.abs(x) <= 448]
    r = fp8.e4m3_round(x)
    v = np.sort(np.concatenate([-e4m3_values(), e4m3_values()]))
    nearest = v[np.abs(x[:, None] - v[None, :]).argmin(axis=1)]
    assert (np.abs(r - x) <= np.abs(nearest - x) + 0.0).all()
    normal = np.abs(x) >= 2.0 ** -6
    assert (np.abs(r - x)[normal] <= 2.0 ** -4 * np.abs(x[normal])).all()
    assert (np.abs(r - x)[~normal] <= 2.0 ** -10).all()
    np.testing.assert_array_equal(fp8.e4m3_round(r), r)
    with pytest.raises(ValueError):
        fp8.e4m3_round(np.array([449.0]))


def test_scale_exponent_puts_the_group_max_in_the_top_binade():
    rng = np.random.default_rng(4)
    amax = 2.0 ** rng.uniform(-40, 40, 5000)
    assert fp8.scale_exp(np.array([2.0 ** -200]))[0] == -127
    e = fp8.scale_exp(amax)
    s = amax / 2.0 ** e
    assert ((s > 224) & (s <= 448)).all()
    assert fp8.scale_exp(np.array([448.0 * 8]))[0] == 3 and fp8.scale_exp(np.array([0.0]))[0] == 0


def test_quantize_rows_and_cols():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 32)) * 2.0 ** rng.uniform(-8, 8, (64, 1))
    xr, er = fp8.quantize_rows(x)
    assert (np.abs(xr - x) <= 2.0 ** -4 * np.abs(x).max(axis=1, keepdims=True)).all()
    assert np.abs(xr).max(axis=1).max() <= (448 * 2.0 ** er).max()
    xc, ec = fp8.quantize_cols(x)
    assert ec.shape == (32,)
    assert (np.abs(xc - x) <= 2.0 ** -4 * np.abs(x).max(axis=0, keepdims=True)).all()
    # idempotent: quantising a quantised tensor with the same scales changes nothing
    np.testing.assert_array_equal(fp8.quantize(xr, er[:, None]), xr)


def sel_for(mode, q, k, v, **kw):
    r = solattn.head_forward(mode, q, k, v, want_out=False, **kw)
    return r, (r["kept"], r["extra"])


@pytest.mark.parametrize("mode", ["sol", "sla"])
def test_constant_values_come_out_exactly(mode):
    # V = 1.5 everywhere: the weights are normalised, so out = 1.5 whatever the logits
    rng = np.random.default_rng(6)
    N, d = 512, 16
    q, k = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    v = np.full((N, d), 1.5)
    kw = dict(block_q=32, block_k=32, tau=1.0, keep_percent=20.0, extra_tokens=9)
    _, sel = sel_for(mode, q, k, v, **kw)
    out = fp8.head_forward_fp8qk(mode, q, k, v, selection=sel, **kw)
    np.testing.assert_allclose(out, 1.5, rtol=0, atol=1e-14)


@pytest.mark.parametrize("mode", ["sol", "sla"])
def test_inputs_e4m3_holds_exactly_match_the_exact_pass(mode):
    # Q rows and block-constant K rows with entries j/8, |j| <= 8: every row (and every pooled
    # key, which equals its block's rows) scales by its power of two onto values j * 2^k that
    # E4M3 holds exactly, so the flavour must equal the exact (bf16-oracle) pass
    rng = np.random.default_rng(9)
    N, d, bk = 256, 8, 32
    q = rng.integers(-8, 9, (N, d)) / 8.0
    k = np.repeat(rng.integers(-8, 9, (N // bk, d)) / 8.0, bk, axis=0)
    v = rng.standard_normal((N, d))
    kw = dict(block_q=32, block_k=bk, tau=0.5, keep_percent=25.0, extra_tokens=5)
    for x in (q, k):
        xr, _ = fp8.quantize_rows(x)
        np.testing.assert_array_equal(xr, x)
    _, sel = sel_for(mode, q, k, v, **kw)
    out = fp8.head_forward_fp8qk(mode, q, k, v, selection=sel, **kw)
    exact = solattn.head_forward(mode, q, k, v, selection=sel, **kw)["out"]
    np.testing.assert_allclose(out, exact, rtol=0, atol=1e-12)


def test_equal_logits_give_the_mean_of_the_values():
    # identical keys: every logit of a row is the same, so out = mean of v over every key
    rng = np.random.default_rng(7)
    N, d = 256, 8
    q = rng.standard_normal((N, d))
    k = np.tile(rng.standard_normal(d), (N, 1))
    v = rng.standard_normal((N, d))
    kw = dict(block_q=32, block_k=32, tau=-math.inf)
    _, sel = sel_for("sol", q, k, v, **kw)
    out = fp8.head_forward_fp8qk("sol", q, k, v, selection=sel, **kw)
    np.testing.assert_allclose(out, np.tile(v.mean(axis=0), (N, 1)), rtol=0, atol=1e-12)


def test_close_to_the_exact_result_within_the_format_error():
    # dense selection: the flavour against textbook attention.  Each logit moves by at most
    # about 2^-4 * |q| * |k| / sqrt(d) under the rounding, so outputs stay within a few percent
    # of the value range; a dropped dequantisation scale would be far outside.
    rng = np.random.default_rng(8)
    N, d = 512, 32
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    kw = dict(block_q=64, block_k=64, tau=-math.inf)
    _, sel = sel_for("sol", q, k, v, **kw)
    out = fp8.head_forward_fp8qk("sol", q, k, v, selection=sel, **kw)
    ref = dense.dense_attention(q, k, v)
    err = np.abs(out - ref)
    assert err.max() < 0.05 and err.mean() < 0.01, (err.max(), err.mean())
    assert err.max() > 0            # the flavour is not value-identical to the exact pass
