"""Host checks of the attention kernel's work schedule (solattn_pair_schedule, the same function
the kernel runs to map a workgroup to its query blocks): every query block is computed by
exactly one workgroup, dense blocks first, pairs as the stride defines them."""
import numpy as np
import pytest

import block_sparse_attention_scores_amd as sa


def check(Mq, dense, s):
    sched = sa.pair_schedule(Mq, dense, s)
    d0, d1 = dense if dense[1] > dense[0] else (0, 0)
    nd = d1 - d0
    assert len(sched) == (nd + 1) // 2 + (Mq - nd + 1) // 2
    seen = np.zeros(Mq, dtype=int)
    for a, b in sched:
        assert 0 <= a < Mq and -1 <= b < Mq and a != b
        seen[a] += 1
        if b >= 0:
            seen[b] += 1
    np.testing.assert_array_equal(seen, 1)
    nu_d = (nd + 1) // 2
    for j, (a, b) in enumerate(sched):
        in_dense = d0 <= a < d1
        assert in_dense == (j < nu_d)
        if b >= 0:
            assert (d0 <= b < d1) == in_dense
    # the non-dense blocks, numbered with the dense run cut out, pair t with t + s in each
    # whole run of 2s, then neighbours
    rest = [i for i in range(Mq) if not d0 <= i < d1]
    pos = {blk: i for i, blk in enumerate(rest)}
    Ms, C = len(rest), len(rest) // (2 * s)
    for a, b in sched[nu_d:]:
        ia = pos[a]
        if ia < 2 * s * C:
            assert ia % (2 * s) < s and b == rest[ia + s]
        else:
            assert (ia - 2 * s * C) % 2 == 0
            assert b == (rest[ia + 1] if ia + 1 < Ms else -1)
    return sched


@pytest.mark.parametrize("Mq", [1, 2, 3, 7, 16, 31, 288, 1001])
@pytest.mark.parametrize("s", [1, 2, 3, 8])
def test_every_query_block_once(Mq, s):
    check(Mq, (0, 0), s)
    rng = np.random.default_rng(Mq * 10 + s)
    for _ in range(6):
        d0 = int(rng.integers(0, Mq + 1))
        d1 = int(rng.integers(d0, Mq + 1))
        check(Mq, (d0, d1), s)
    check(Mq, (0, Mq), s)


def test_stride_one_is_neighbour_pairing():
    assert sa.pair_schedule(7) == [(0, 1), (2, 3), (4, 5), (6, -1)]
    # dense blocks 3..5 first, then the rest with the dense run cut out
    assert sa.pair_schedule(9, (3, 6), 1) == [(3, 4), (5, -1), (0, 1), (2, 6), (7, 8)]


def test_stride_three_pairs_each_block_with_the_one_three_on():
    assert sa.pair_schedule(14, (0, 0), 3) == [(0, 3), (1, 4), (2, 5), (6, 9), (7, 10), (8, 11),
                                               (12, 13)]


@pytest.mark.parametrize("args", [(0, 0, 0, 1), (4, 3, 2, 1), (4, 0, 5, 1), (4, 0, 0, 0),
                                  (4, 0, 0, sa.PAIR_STRIDES + 1), (4, -1, 0, 1)])
def test_invalid_arguments(args):
    Mq, d0, d1, s = args
    assert sa.lib().solattn_pair_schedule(Mq, d0, d1, s, None, None, 0) == sa.EINVAL
