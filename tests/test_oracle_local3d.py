"""Pins of the oracle's static local 3-D routing (the article on block sparse attention for H3
in ComfyUI, section 1: the centre block, its neighbours one frame back and forward, and its
spatial neighbours one block up, down, left and right; every other block is zero).

The oracle states the pattern on tokens and lifts it to blocks.  These tests check it by other
routes: the cross stencil on the grid of blocks written from block coordinates (where the grid
of blocks exists), a pairwise Manhattan-distance search over token coordinates from
numpy.unravel_index (any grid), the edge count of a 3-D grid graph, symmetry, and the masked
textbook softmax for the output.
"""
import math

import numpy as np
import pytest

from oracle import solattn


def rnd(N, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((N, d)) for _ in range(3)]


def masks(N, bq, bk, grid, sink_range=0):
    Mq = -(-N // bq)
    return np.stack([solattn.select_local3d(
        solattn.local3d_neighbours(i, N, bq, bk, grid),
        solattn.forced_blocks(i, N, bq, bk, sink_range)) for i in range(Mq)])


def block_grid(F, Hh, Ww, bk):
    """Shape (frames, block rows, block columns) of the grid of blocks, when it exists."""
    if Ww % bk == 0:
        return F, Hh, Ww // bk
    assert bk % Ww == 0 and (Hh * Ww) % bk == 0
    return F, Hh * Ww // bk, 1


def cross_stencil(F, R, C):
    """kept[i, j] = block coordinates of i and j differ by at most one step along one axis."""
    n = F * R * C
    t, r, c = np.unravel_index(np.arange(n), (F, R, C))
    dist = (np.abs(t[:, None] - t[None, :]) + np.abs(r[:, None] - r[None, :]) +
            np.abs(c[:, None] - c[None, :]))
    return dist <= 1


ALIGNED = [(3, 4, 128), (2, 6, 32), (4, 2, 64), (2, 3, 192), (5, 1, 64), (1, 8, 16)]


@pytest.mark.parametrize("F,Hh,Ww", ALIGNED)
def test_aligned_grid_is_the_block_cross_stencil(F, Hh, Ww):
    N = F * Hh * Ww
    got = masks(N, 64, 64, (F, Hh, Ww))
    np.testing.assert_array_equal(got, cross_stencil(*block_grid(F, Hh, Ww, 64)))


@pytest.mark.parametrize("F,Hh,Ww", ALIGNED)
def test_aligned_edge_count(F, Hh, Ww):
    # every block plus both directions of each edge of the F x R x C grid graph
    Fb, R, C = block_grid(F, Hh, Ww, 64)
    edges = (Fb - 1) * R * C + Fb * (R - 1) * C + Fb * R * (C - 1)
    got = masks(F * Hh * Ww, 64, 64, (F, Hh, Ww))
    assert got.sum() == Fb * R * C + 2 * edges


@pytest.mark.parametrize("F,Hh,Ww", [(3, 4, 128), (2, 6, 32), (4, 2, 64)])
def test_query_block_of_two_key_blocks_is_the_union(F, Hh, Ww):
    N = F * Hh * Ww
    got = masks(N, 128, 64, (F, Hh, Ww))
    ref = cross_stencil(*block_grid(F, Hh, Ww, 64))
    np.testing.assert_array_equal(got, ref[0::2] | ref[1::2])


@pytest.mark.parametrize("F,Hh,Ww,bq,bk", [(3, 5, 7, 8, 8), (2, 4, 9, 16, 8), (4, 3, 5, 8, 16),
                                           (1, 7, 11, 12, 12), (6, 1, 13, 8, 8)])
def test_any_grid_matches_token_distance_search(F, Hh, Ww, bq, bk):
    N = F * Hh * Ww
    t, y, x = np.unravel_index(np.arange(N), (F, Hh, Ww))
    near = (np.abs(t[:, None] - t[None, :]) + np.abs(y[:, None] - y[None, :]) +
            np.abs(x[:, None] - x[None, :])) <= 1                     # [query token, key token]
    Mq, M = -(-N // bq), -(-N // bk)
    ref = np.zeros((Mq, M), dtype=bool)
    for i in range(Mq):
        for j in range(M):
            ref[i, j] = near[i * bq:(i + 1) * bq, j * bk:(j + 1) * bk].any()
    got = masks(N, bq, bk, (F, Hh, Ww))
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("F,Hh,Ww", [(3, 5, 7), (2, 9, 4), (7, 3, 3)])
def test_equal_blocks_give_a_symmetric_pattern(F, Hh, Ww):
    # token adjacency is symmetric, so with one block size for queries and keys so is the pattern
    N = F * Hh * Ww
    got = masks(N, 8, 8, (F, Hh, Ww))
    np.testing.assert_array_equal(got, got.T)


@pytest.mark.parametrize("grid", [(1, 1, 512), (8, 1, 64), (8, 8, 8), (6, 4, 16), (1, 16, 32)])
def test_one_block_lines_give_a_band(grid):
    # a single row, frames of one block, or a single column of blocks: the blocks form a line
    # and the pattern is the tridiagonal band |i - j| <= 1
    F, Hh, Ww = grid
    N = F * Hh * Ww
    got = masks(N, 64, 64, grid)
    M = N // 64
    band = np.abs(np.arange(M)[:, None] - np.arange(M)[None, :]) <= 1
    np.testing.assert_array_equal(got, band)


def test_sinks_are_added_on_top():
    F, Hh, Ww = 4, 4, 64
    N = F * Hh * Ww
    got = masks(N, 64, 64, (F, Hh, Ww), sink_range=100)
    ref = cross_stencil(*block_grid(F, Hh, Ww, 64))
    ref[:, :2] = True                   # tokens [0, 100) touch blocks 0 and 1
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("extra", [0, 9])
def test_output_is_the_masked_softmax(extra):
    # skipped blocks contribute nothing: out = softmax over the kept blocks' and extra tokens only
    F, Hh, Ww, bq, bk = 3, 4, 8, 16, 8
    N, d = F * Hh * Ww, 5
    q, k, v = rnd(N, d, 31)
    r = solattn.head_forward("local3d", q, k, v, block_q=bq, block_k=bk, extra_tokens=extra,
                             grid=(F, Hh, Ww))
    assert not r["kept"].all()
    allowed = np.repeat(np.repeat(r["kept"], bq, axis=0), bk, axis=1)[:N, :N]
    for i, e in enumerate(r["extra"]):
        assert e.size == min(extra, int((~r["kept"][i]).sum()) * bk)
        assert not r["kept"][i][e // bk].any()
        allowed[i * bq:(i + 1) * bq, e] = True
    logits = q @ k.T / math.sqrt(d)
    logits = np.where(allowed, logits, -np.inf)
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    ref = (w @ v) / w.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(r["out"], ref, rtol=0, atol=1e-12)


def test_dense_rows_attend_everything():
    F, Hh, Ww = 4, 2, 64
    N, d = F * Hh * Ww, 4
    q, k, v = rnd(N, d, 32)
    r = solattn.head_forward("local3d", q, k, v, block_q=64, block_k=64, dense_rows=(128, 256),
                             grid=(F, Hh, Ww))
    assert r["kept"][2:4].all() and not r["kept"][0].all()
    logits = q[128:256] @ k.T / math.sqrt(d)
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    np.testing.assert_allclose(r["out"][128:256], (w @ v) / w.sum(axis=1, keepdims=True),
                               rtol=0, atol=1e-12)


def test_scores_do_not_change_the_pattern():
    F, Hh, Ww = 3, 2, 128
    N = F * Hh * Ww
    a = rnd(N, 8, 33)
    b = rnd(N, 8, 34)
    ra = solattn.head_forward("local3d", *a, block_q=64, block_k=64, grid=(F, Hh, Ww), want_out=False)
    rb = solattn.head_forward("local3d", *b, block_q=64, block_k=64, grid=(F, Hh, Ww), want_out=False)
    np.testing.assert_array_equal(ra["kept"], rb["kept"])
