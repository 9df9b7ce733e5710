"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test states the closed form, limit, invariant or page figure it checks.
None of them re-types the oracle's own formula: the dense limit uses a separate
textbook routine, the brute-force twin takes a different route (per-token table,
statistics module, sorted()), and the hand-worked cases are derived in the test.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import brute, dense, solattn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def rnd(N, d, seed, H=None):
    rng = np.random.default_rng(seed)
    shape = (N, d) if H is None else (H, N, d)
    return [rng.standard_normal(shape) for _ in range(3)]


def head(mode, q, k, v, **kw):
    return solattn.head_forward(mode, q, k, v, **kw)


# ------------------------------------------------------------------ P1: dense limits

@pytest.mark.parametrize("bq,bk", [(32, 32), (64, 32), (32, 64)])
def test_tau_minus_inf_is_dense(bq, bk):
    q, k, v = rnd(256, 16, 1)
    r = head("sol", q, k, v, block_q=bq, block_k=bk, tau=-math.inf, sink_range=40, extra_tokens=16)
    assert r["kept"].all()
    assert all(e.size == 0 for e in r["extra"])
    np.testing.assert_allclose(r["out"], dense.dense_attention(q, k, v), rtol=0, atol=1e-12)


def test_sla_keep_all_is_dense():
    q, k, v = rnd(256, 16, 2)
    r = head("sla", q, k, v, block_q=64, block_k=32, keep_percent=100.0, extra_tokens=8)
    assert r["kept"].all()
    np.testing.assert_allclose(r["out"], dense.dense_attention(q, k, v), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", ["sol", "sla"])
def test_sink_everything_is_dense(mode):
    q, k, v = rnd(192, 8, 3)
    r = head(mode, q, k, v, block_q=64, block_k=32, tau=2.0, keep_percent=5.0, sink_range=192)
    np.testing.assert_allclose(r["out"], dense.dense_attention(q, k, v), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ P2, P3: exact centroids

@pytest.mark.parametrize("tau,extra", [(0.5, 0), (1.3, 0), (2.5, 5), (1.0, 17)])
def test_one_token_blocks_are_exact(tau, extra):
    # block_k = 1: each centroid is its token, so the sol pass equals dense attention
    q, k, v = rnd(128, 8, 4)
    r = head("sol", q, k, v, block_q=8, block_k=1, tau=tau, extra_tokens=extra)
    assert not r["kept"].all()
    np.testing.assert_allclose(r["out"], dense.dense_attention(q, k, v), rtol=0, atol=1e-12)


def test_block_constant_keys_are_exact():
    # K constant inside each key block: n_j exp(q.k̄_j) v̄_j = sum_t exp(q.k_t) v_t
    q, k, v = rnd(256, 16, 5)
    kb = np.repeat(k[::32], 32, axis=0)
    r = head("sol", q, kb, v, block_q=32, block_k=32, tau=1.0)
    assert not r["kept"].all()
    np.testing.assert_allclose(r["out"], dense.dense_attention(q, kb, v), rtol=0, atol=1e-12)


def test_block_constant_keys_and_values_with_extras_are_exact():
    # K and V block-constant: extra tokens taken out of a skipped block leave an exact remainder
    q, k, v = rnd(256, 16, 6)
    kb = np.repeat(k[::32], 32, axis=0)
    vb = np.repeat(v[::32], 32, axis=0)
    r = head("sol", q, kb, vb, block_q=32, block_k=32, tau=1.0, extra_tokens=40)
    assert sum(e.size for e in r["extra"]) > 0
    np.testing.assert_allclose(r["out"], dense.dense_attention(q, kb, vb), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ P4, P5: invariants

@pytest.mark.parametrize("mode", ["sol", "sla"])
def test_constant_values_give_constant_output(mode):
    q, k, _ = rnd(256, 16, 7)
    cvec = np.linspace(-2, 3, 16)
    v = np.tile(cvec, (256, 1))
    r = head(mode, q, k, v, block_q=64, block_k=32, tau=1.3, keep_percent=20.0,
             sink_range=50, extra_tokens=24, dense_rows=(192, 256))
    np.testing.assert_allclose(r["out"], v, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", ["sol", "sla"])
def test_key_shift_invariance(mode):
    # adding one vector w to every key shifts each row of every score by a constant
    q, k, v = rnd(256, 16, 8)
    w = np.random.default_rng(80).standard_normal(16) * 3
    kw = dict(block_q=32, block_k=32, tau=1.1, keep_percent=25.0, sink_range=20, extra_tokens=24)
    a = head(mode, q, k, v, **kw)
    b = head(mode, q, k + w, v, **kw)
    assert np.array_equal(a["kept"], b["kept"])
    assert all(np.array_equal(x, y) for x, y in zip(a["extra"], b["extra"]))
    np.testing.assert_allclose(a["out"], b["out"], rtol=0, atol=1e-12)


def test_key_scale_keeps_masks():
    q, k, v = rnd(256, 16, 9)
    kw = dict(block_q=32, block_k=32, tau=1.3, extra_tokens=16)
    a = head("sol", q, k, v, **kw)
    b = head("sol", q, 2.5 * k, v, **kw)
    assert np.array_equal(a["kept"], b["kept"])
    assert all(np.array_equal(x, y) for x, y in zip(a["extra"], b["extra"]))


# ------------------------------------------------------------------ P6: the pages' tau figures

@pytest.mark.parametrize("tau", [1.0, 1.5, 2.0])
def test_kept_fraction_matches_page_figures(tau):
    figs = json.load(open(GOLDEN))["tau_kept_fraction"]["values"]
    M, rows = 256, 4000
    rng = np.random.default_rng(60 + int(tau * 10))
    # scores with a non-unit spread and an offset: mean + tau*std must be used, not tau*var
    s = 0.7 + 0.3 * rng.standard_normal((rows, M))
    kept = 0
    for i in range(rows):
        f = np.zeros(M, dtype=bool)
        f[i % M] = True                      # one diagonal block per row
        kept += solattn.select_sol(s[i], tau, f).sum()
    frac = kept / (rows * M)
    tail = 0.5 * math.erfc(tau / math.sqrt(2))
    closed = tail * (M - 1) / M + 1.0 / M
    assert abs(frac - closed) < 0.0025
    assert abs(frac - figs[f"{tau:.1f}"]) < 0.005


# ------------------------------------------------------------------ P7: sla count

@pytest.mark.parametrize("p", [0.5, 10.0, 15.0, 37.5, 95.0])
def test_sla_row_count(p):
    q, k, v = rnd(1024, 8, 11)
    r = head("sla", q, k, v, block_q=128, block_k=64, keep_percent=p, sink_range=64,
              want_out=False)
    M = 16
    for i in range(8):
        f = solattn.forced_blocks(i, 1024, 128, 64, 64)
        kk = min(M - f.sum(), math.ceil(p * M / 100.0))
        assert r["kept"][i].sum() == kk + f.sum()


# ------------------------------------------------------------------ P8: brute-force twin

CASES = [
    ("sol", dict(block_q=16, block_k=16, tau=1.0)),
    ("sol", dict(block_q=32, block_k=16, tau=0.7, sink_range=20, extra_tokens=6)),
    ("sol", dict(block_q=16, block_k=8, tau=1.3, extra_tokens=9, dense_rows=(96, 128))),
    ("sol", dict(block_q=24, block_k=16, tau=0.5, extra_tokens=5, dense_rows=(100, 140))),
    ("sla", dict(block_q=32, block_k=16, keep_percent=20.0, sink_range=16)),
    ("sla", dict(block_q=16, block_k=16, keep_percent=30.0, extra_tokens=7)),
]


@pytest.mark.parametrize("N", [144, 150])
@pytest.mark.parametrize("mode,kw", CASES)
def test_brute_force_twin(mode, kw, N):
    q, k, v = rnd(N, 6, 12 + N)
    a = head(mode, q, k, v, **kw)
    out, kept, extra = brute.brute_head(mode, q, k, v, **kw)
    M = a["kept"].shape[1]
    for i in range(a["kept"].shape[0]):
        assert set(np.flatnonzero(a["kept"][i])) == kept[i]
        assert set(a["extra"][i].tolist()) == extra[i]
    assert a["kept"].sum() < a["kept"].size or kw.get("keep_percent", 0) >= 100
    np.testing.assert_allclose(a["out"], np.array(out), rtol=0, atol=1e-12)
    assert M == -(-N // kw["block_k"])


# ------------------------------------------------------------------ P9: extra-token limits

def test_extra_zero_is_empty():
    q, k, v = rnd(256, 8, 13)
    r = head("sol", q, k, v, block_q=32, block_k=32, tau=1.3, extra_tokens=0)
    assert all(e.size == 0 for e in r["extra"])


@pytest.mark.parametrize("mode", ["sol", "sla"])
def test_extra_covering_all_candidates_is_dense(mode):
    # more extra tokens than candidates: every token is attended exactly ("approach dense")
    q, k, v = rnd(64, 8, 14)
    r = head(mode, q, k, v, block_q=8, block_k=4, tau=1.0, keep_percent=10.0, extra_tokens=256)
    np.testing.assert_allclose(r["out"], dense.dense_attention(q, k, v), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ P10: independence

def test_head_permutation():
    q, k, v = rnd(128, 8, 15, H=3)
    perm = [2, 0, 1]
    kw = dict(block_q=32, block_k=16, tau=1.2, extra_tokens=5)
    a = solattn.forward("sol", q[None], k[None], v[None], **kw)["out"][0]
    b = solattn.forward("sol", q[perm][None], k[perm][None], v[perm][None], **kw)["out"][0]
    np.testing.assert_array_equal(a[perm], b)


# ------------------------------------------------------------------ hand-worked cases

def test_threshold_uses_population_std_and_strict_compare():
    none = np.zeros(4, dtype=bool)
    # mean 1, population std sqrt(3): 1 + 1.5*sqrt(3) = 3.598 < 4 -> block 3 kept
    # (the sample std, 2, would give threshold 4 and drop it)
    assert list(np.flatnonzero(solattn.select_sol(np.array([0., 0, 0, 4]), 1.5, none))) == [3]
    # a constant row has std 0: threshold = mean, and nothing exceeds it strictly
    f = np.array([False, True, False, False])
    assert list(np.flatnonzero(solattn.select_sol(np.full(4, 2.5), 1.3, f))) == [1]
    # tau = 0: threshold is the mean
    assert list(np.flatnonzero(solattn.select_sol(np.array([0., 1, 2, 3]), 0.0, none))) == [2, 3]


def test_forced_geometry():
    # Q128/K64: the diagonal is both key blocks under the query block; sinks cover [0, 100)
    f = solattn.forced_blocks(3, 1024, 128, 64, 100)
    assert list(np.flatnonzero(f)) == [0, 1, 6, 7]
    f = solattn.forced_blocks(0, 1024, 64, 64, 0)
    assert list(np.flatnonzero(f)) == [0]
    # a 24-token query block straddling two 16-token key blocks
    f = solattn.forced_blocks(1, 96, 24, 16, 0)
    assert list(np.flatnonzero(f)) == [1, 2]


def test_sla_ties_go_to_lower_index():
    s = np.array([1.0, 3.0, 3.0, 2.0, 3.0])
    keep = solattn.select_sla(s, 40.0, np.zeros(5, dtype=bool))     # ceil(2.0) = 2 blocks
    assert list(np.flatnonzero(keep)) == [1, 2]
    keep = solattn.select_sla(s, 40.0, np.array([0, 1, 0, 0, 0], dtype=bool))
    assert list(np.flatnonzero(keep)) == [1, 2, 4]


def test_extra_ties_go_to_lower_token():
    e = np.array([5.0, 1.0, 7.0, 7.0, 2.0, 7.0, 0.0, 9.0])
    kept = np.array([False, False, False, True])                      # tokens 6, 7 excluded
    assert list(solattn.extra_select(e, kept, 2, 3)) == [2, 3, 5]
    assert list(solattn.extra_select(e, kept, 2, 2)) == [2, 3]
    assert list(solattn.extra_select(e, kept, 2, 10)) == [0, 1, 2, 3, 4, 5]


def test_hand_worked_centroid_and_extra_token():
    # d = 1 (scale 1), blocks of 2.  k = [0, 2, 1, 1], v = [1, 3, 10, 20]:
    # k̄ = [1, 1], v̄ = [2, 15].  Query rows q = [1, 1, 0.5, 0.5]: q̄_0 = 1, q̄_1 = 0.5.
    # Row 0 scores [1, 1]: std 0, threshold = mean, so only the diagonal block 0 is kept.
    q = np.array([[1.0], [1.0], [0.5], [0.5]])
    k = np.array([[0.0], [2.0], [1.0], [1.0]])
    v = np.array([[1.0], [3.0], [10.0], [20.0]])
    e, e2 = math.e, math.e ** 2
    r = head("sol", q, k, v, block_q=2, block_k=2, tau=1.0)
    assert r["kept"].tolist() == [[True, False], [False, True]]
    # row 0: exact tokens 0,1 (logits 0, 2) + centroid of block 1, weight 2, logit 1, value 15
    want0 = (1 * 1 + e2 * 3 + 2 * e * 15) / (1 + e2 + 2 * e)
    assert abs(r["out"][0, 0] - want0) < 1e-12
    # one extra token: candidates 2, 3 tie at q̄_0.k = 1 -> token 2; block 1 keeps weight 1
    r = head("sol", q, k, v, block_q=2, block_k=2, tau=1.0, extra_tokens=1)
    assert r["extra"][0].tolist() == [2]
    want0 = (1 + e2 * 3 + e * 10 + e * 15) / (1 + e2 + e + e)
    assert abs(r["out"][0, 0] - want0) < 1e-12
    # sla drops the skipped block entirely
    r = head("sla", q, k, v, block_q=2, block_k=2, keep_percent=1.0, sink_range=0)
    # M = 2, forced {0}: k = min(1, ceil(0.02)) = 1 -> block 1 routed too; use p small with M-|F|=1
    assert r["kept"][0].tolist() == [True, True]


def test_hand_worked_sla_drop():
    q = np.array([[1.0], [1.0], [0.5], [0.5], [0.0], [0.0]])
    k = np.array([[0.0], [2.0], [1.0], [1.0], [-1.0], [-1.0]])
    v = np.array([[1.0], [3.0], [10.0], [20.0], [7.0], [9.0]])
    # M = 3; row 0 forced {0}; scores of blocks 1, 2: 1*1 = 1 and 1*(-1) = -1; p = 10 -> k = 1
    r = head("sla", q, k, v, block_q=2, block_k=2, keep_percent=10.0)
    assert r["kept"][0].tolist() == [True, True, False]
    e, e2 = math.e, math.e ** 2
    want0 = (1 + e2 * 3 + e * 10 + e * 20) / (1 + e2 + 2 * e)
    assert abs(r["out"][0, 0] - want0) < 1e-12


def test_sink_boundary_and_score_values():
    # a sink range ending one token into block 1 forces block 1; ending at its start does not
    assert list(np.flatnonzero(solattn.forced_blocks(5, 1024, 64, 64, 65))) == [0, 1, 5]
    assert list(np.flatnonzero(solattn.forced_blocks(5, 1024, 64, 64, 64))) == [0, 5]
    assert list(np.flatnonzero(solattn.forced_blocks(5, 1024, 64, 64, 1))) == [0, 5]
    # block scores carry the 1/sqrt(d) scale: d = 4, q̄_0 = (1,1,1,1), k̄_1 = (1,2,3,4)/... by hand
    q = np.array([[1.0, 1, 1, 1], [1, 1, 1, 1], [2, 0, 0, 0], [0, 0, 0, 0]])
    k = np.array([[1.0, 0, 0, 0], [1, 0, 0, 0], [1, 2, 3, 4], [3, 2, 1, 0]])
    r = head("sol", q, k, q, block_q=2, block_k=2, tau=1.0, want_out=False)
    # q̄ = [(1,1,1,1), (1,0,0,0)], k̄ = [(1,0,0,0), (2,2,2,2)], scale 1/2
    assert np.allclose(r["scores"], [[0.5, 4.0], [0.5, 1.0]], rtol=0, atol=1e-15)
