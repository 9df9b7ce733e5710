"""The allocation-free entry point (sol_attn_fwd_noalloc) through the C ABI: its output equals
the workspace entry point's (sol_attn_fwd) bit for bit on two calls in a row, the second on a
smaller input, so the scratch kept from the first call does not leak into the second; a call
that does not fit in the scratch, or that passes a workspace, is refused before anything runs."""
import numpy as np
import pytest
import torch

import block_sparse_attention_scores_amd as sa
from gen import make_inputs, workload
from parity import device_inputs

pytestmark = pytest.mark.gpu


def _both(w, x):
    q, k, v = device_inputs(x)
    kw = dict(tau=w.tau, block_q=64, block_k=64, sink_range=w.sink_range,
              extra_tokens=w.extra_tokens, dense_rows=w.dense_rows)
    need = sa.workspace_bytes(sa.MODE_SOL, sa.BF16, *q.shape, 64, 64, None, w.extra_tokens)
    assert need <= sa.NOALLOC_SCRATCH_BYTES, need
    print(f"\n[noalloc] N={w.N} H={q.shape[1]} extra={w.extra_tokens} workspace {need} bytes", flush=True)
    ref = sa.sol_attn(q, k, v, **kw)
    out = torch.full_like(q, float("nan"))
    got = sa.sol_attn_noalloc(q, k, v, out=out, **kw)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    return got


def test_noalloc_equals_the_workspace_call_twice():
    big = workload(2, H=2, T=2, extra_tokens=128, dense_rows=(8192 - 512, 8192))
    small = workload(2, H=1, T=1, Hh=64, Ww=64, extra_tokens=64, sink_range=256)
    assert big.N == 8192 and small.N == 4096
    _both(big, make_inputs(big))
    _both(small, make_inputs(small))


def test_noalloc_refuses_what_does_not_fit_and_a_workspace():
    w = workload(2, H=4, T=4, extra_tokens=256)
    x = make_inputs(w, heads=[0, 1, 2, 3])
    q, k, v = device_inputs(x)
    need = sa.workspace_bytes(sa.MODE_SOL, sa.BF16, *q.shape, 64, 64, None, 256)
    assert need > sa.NOALLOC_SCRATCH_BYTES
    out = torch.zeros_like(q)
    with pytest.raises(sa.SolattnError) as e:
        sa.sol_attn_noalloc(q, k, v, out=out, extra_tokens=256)
    assert e.value.status == sa.EWORKSPACE and str(need) in e.value.detail
    # a query-row window small enough for the scratch runs, and matches the workspace call
    rows = (4096, 8192)
    assert sa.workspace_bytes(sa.MODE_SOL, sa.BF16, *q.shape, 64, 64, rows[1] - rows[0], 256) \
        <= sa.NOALLOC_SCRATCH_BYTES
    got = sa.sol_attn_noalloc(q, k, v, out=out, extra_tokens=256, q_rows=rows)
    ref = sa.sol_attn(q, k, v, extra_tokens=256, q_rows=rows, out=torch.zeros_like(q))
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert torch.count_nonzero(got[:, :, :rows[0]].float()) == 0
    # a workspace passed to the allocation-free call is an error
    o = sa.make_opts(workspace=1 << 40, workspace_bytes=1 << 30)
    rc = sa.lib().sol_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       *q.shape, 1.3, 64, 64, 0, 0, o)
    assert rc == sa.EINVAL and "workspace" in sa.last_error()
