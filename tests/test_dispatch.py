"""The dispatch policy around the sparse forward (BlockSparseAttention node documentation,
common-inputs table and constraints section): host logic, no GPU except the last test."""
import logging
import math

import numpy as np
import pytest

from block_sparse_attention_scores_amd.dispatch import (Decision, SinkLayout, SparseAttentionPolicy,
                                                        parse_dense_blocks)


def test_dense_blocks_parser_page_example():
    # the page's own example
    assert parse_dense_blocks("0, 1, 47-49") == {0, 1, 47, 48, 49}
    assert parse_dense_blocks("") == frozenset()
    assert parse_dense_blocks("  ") == frozenset()
    assert parse_dense_blocks("5") == {5}
    assert parse_dense_blocks("3-3,3") == {3}
    assert parse_dense_blocks("2 - 4 ,") == {2, 3, 4}


@pytest.mark.parametrize("bad", ["a", "1-", "-2", "4-2", "1.5", "1;2", "1-2-3"])
def test_dense_blocks_parser_rejects(bad):
    with pytest.raises(ValueError):
        parse_dense_blocks(bad)


def test_defaults_are_the_pages():
    p = SparseAttentionPolicy()
    assert (p.method, p.tau, p.keep_percent, p.extra_tokens) == ("sol-attn", 1.3, 10.0, 256)
    assert (p.start_percent, p.end_percent, p.dense_blocks, p.min_tokens) == (0.2, 1.0, "", 12288)
    assert (p.sink_conditioning, p.verbose) == ("exact_kv_and_rows", False)


@pytest.mark.parametrize("kw", [dict(tau=4.5), dict(tau=-0.1), dict(keep_percent=0.4),
                                dict(keep_percent=96), dict(extra_tokens=300), dict(min_tokens=-1),
                                dict(start_percent=1.5), dict(method="dense"),
                                dict(sink_conditioning="rows"), dict(dense_blocks="x")])
def test_ranges_validated(kw):
    with pytest.raises(ValueError):
        SparseAttentionPolicy(**kw)


def test_min_tokens_and_window():
    p = SparseAttentionPolicy()
    assert not p.decide(12287).sparse                     # shorter than min_tokens
    assert p.decide(12288).sparse                         # not shorter
    assert not p.decide(65536, progress=0.19).sparse      # before start_percent
    assert p.decide(65536, progress=0.2).sparse           # window ends included
    assert p.decide(65536, progress=1.0).sparse
    q = SparseAttentionPolicy(end_percent=0.8)
    assert not q.decide(65536, progress=0.81).sparse      # after end_percent
    assert q.decide(65536).sparse                         # progress unknown: inside


def test_dense_blocks_rule(caplog):
    p = SparseAttentionPolicy(dense_blocks="0, 1, 47-49", verbose=True)
    assert not p.decide(65536, block_index=48).sparse
    assert p.decide(65536, block_index=46).sparse
    with caplog.at_level(logging.INFO, logger="block_sparse_attention_scores_amd"):
        d = p.decide(65536, block_index=None)             # no block index: the list is ignored
    assert d.sparse and "ignored" in caplog.text


def test_sink_conditioning_layouts():
    lay = SinkLayout(seq_len=65536, packed_rows=1024, audio_rows=(63488, 65536))
    d = SparseAttentionPolicy().decide(65536, layout=lay)
    assert d == Decision(True, "sparse sol-attn", 1024, (63488, 65536))
    d = SparseAttentionPolicy(sink_conditioning="exact_kv").decide(65536, layout=lay)
    assert (d.sink_range, d.dense_rows) == (1024, (0, 0))
    d = SparseAttentionPolicy(sink_conditioning="off").decide(65536, layout=lay)
    assert (d.sink_range, d.dense_rows) == (0, (0, 0))
    d = SparseAttentionPolicy().decide(32768, layout=lay)  # layout for another length
    assert d.sparse and (d.sink_range, d.dense_rows) == (0, (0, 0))


def test_vsa_stays_dense_with_reason():
    d = SparseAttentionPolicy(method="vsa").decide(65536)
    assert not d.sparse and "vsa" in d.reason


@pytest.mark.gpu
def test_policy_runs_the_library():
    import torch
    import block_sparse_attention_scores_amd as sa
    from gen import random_qkv
    from oracle import dense
    x = random_qkv(1, 2, 4096, 64, seed=21, dtype="bf16")
    f = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = f(x.q_bits), f(x.k_bits), f(x.v_bits)
    # dense: below min_tokens
    out = SparseAttentionPolicy().attention(q, k, v).float().cpu().numpy()
    ref = np.stack([dense.dense_attention(x.q[0, h], x.k[0, h], x.v[0, h]) for h in range(2)])
    err = np.abs(out[0] - ref)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    # sparse: the same call as sol_attn with the policy's parameters
    p = SparseAttentionPolicy(min_tokens=0, extra_tokens=64)
    a = p.attention(q, k, v, progress=0.5).float()
    b = sa.sol_attn(q, k, v, tau=1.3, extra_tokens=64).float()
    assert torch.equal(a, b)
