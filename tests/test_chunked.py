"""The row-chunked driver: the halving rule on the CPU (a fake attempt that runs out of memory
above a size), and on the GPU that chunked calls reproduce one whole call bit for bit, also when
the workspace allocation runs out of memory and the chunk is halved."""
import math

import numpy as np
import pytest

from block_sparse_attention_scores_amd.chunked import ChunkTooLarge, run_chunks


def fake(limit, log):
    def attempt(b, e):
        log.append((b, e))
        if e - b > limit:
            raise ChunkTooLarge(f"{e - b} rows")
    return attempt


def covered(rep, n):
    rows = np.zeros(n, dtype=int)
    for b, e in rep.chunks:
        rows[b:e] += 1
    return (rows == 1).all()


def test_no_halving_when_everything_fits():
    log = []
    rep = run_chunks(4096, 64, 1024, fake(10 ** 9, log))
    assert rep.chunks == [(0, 1024), (1024, 2048), (2048, 3072), (3072, 4096)]
    assert rep.halvings == 0 and rep.final_chunk == 1024 and log == rep.chunks


def test_halving_until_it_fits_then_keeps_the_size():
    log = []
    rep = run_chunks(4096, 64, 4096, fake(700, log))
    # 4096 -> 2048 -> 1024 -> 512 fits; then the rest in 512-row chunks
    assert rep.halvings == 3 and rep.final_chunk == 512
    assert log[:4] == [(0, 4096), (0, 2048), (0, 1024), (0, 512)]
    assert rep.chunks == [(b, b + 512) for b in range(0, 4096, 512)]
    assert covered(rep, 4096)


def test_halving_rounds_to_whole_blocks_and_ragged_tail():
    log = []
    rep = run_chunks(64 * 13, 64, 64 * 5, fake(64 * 2, log))
    # 320 -> 128 (160 rounded down to whole 64-row blocks); the last chunk is the ragged rest
    assert rep.final_chunk == 128
    assert rep.chunks[-1] == (768, 832)
    assert covered(rep, 832)


def test_one_block_that_does_not_fit_is_an_error():
    with pytest.raises(ChunkTooLarge):
        run_chunks(1024, 64, 1024, fake(32, []))


def test_rows_must_be_whole_blocks():
    with pytest.raises(ValueError):
        run_chunks(1000, 64, 256, fake(10 ** 9, []))


# ---------------------------------------------------------------------------------------- GPU

def _chunk_collector(method, B, H, N, d, bq, store):
    """on_chunk hook: copies each chunk's selection (whole-sequence block numbering) to the host."""
    import block_sparse_attention_scores_amd as sa
    import torch
    mode = {"sol": sa.MODE_SOL, "sla": sa.MODE_SLA, "local3d": sa.MODE_LOCAL3D}[method]

    def hook(begin, end, ws):
        torch.cuda.synchronize()
        views = sa.selection_views(ws, mode, sa.BF16, B, H, N, d, bq, 64, q_rows=(begin, end))
        store.append((begin, end, {k_: v_.cpu().numpy().copy() for k_, v_ in views.items()}))
    return hook


def _assemble(store, Mq):
    """The chunks' selections put together in whole-sequence query-block order."""
    import numpy as np
    store = sorted(store, key=lambda t: t[0])
    names = ("qbar", "scores", "kept_cnt", "kept_idx", "kept_bm", "mult", "extra_cnt", "extra_idx",
             "extra_flag")
    sel = {n: np.concatenate([c[2][n] for c in store], axis=1) for n in names}
    sel["kbar"], sel["vbar"] = store[0][2]["kbar"], store[0][2]["vbar"]
    assert sel["kept_cnt"].shape[1] == Mq
    return sel


def _check_against_oracle(method, x, w, out, sel, bq, params, seed):
    """Selection of both heads against the oracle's own, and outputs of sampled query blocks
    against the oracle run on that selection."""
    import numpy as np
    from oracle import solattn
    from parity import Report, check_head
    p = dict(block_q=bq, block_k=64, tau=params.get("tau", w.tau),
             keep_percent=params.get("keep_percent", w.keep_percent), sink_range=w.sink_range,
             extra_tokens=w.extra_tokens, dense_rows=w.dense_rows)
    if method == "local3d":
        p["grid"] = params["grid"]
    o = out.float().cpu().numpy().astype(np.float64)
    rep = Report()
    for h in range(w.H):
        xin = tuple(t[0, h].astype(np.float64) for t in (x.q, x.k, x.v))
        ref = solattn.head_forward(method, *xin, **p, want_out=False)
        rng = np.random.default_rng(seed + h)
        sp, dn = np.flatnonzero(~ref["dense"]), np.flatnonzero(ref["dense"])
        qb = sorted(set(rng.choice(sp, 12, replace=False).tolist() + rng.choice(dn, 2, replace=False).tolist()))
        check_head(method, ref, sel, h, x_in=xin, d=w.d, N=w.N, report=rep, qblocks=qb,
                   out_gpu=o[0, h], dtype="bf16", **p)
    return rep


@pytest.mark.gpu
@pytest.mark.parametrize("method", ["sol", "sla", "local3d"])
def test_chunked_equals_whole_call(method):
    import torch

    import block_sparse_attention_scores_amd as sa
    from block_sparse_attention_scores_amd.chunked import chunked_attention
    from gen import make_inputs, workload
    from parity import device_inputs

    bq = 128 if method == "sla" else 64
    w = workload(2, mode=method, H=2, extra_tokens=128, dense_rows=(16384 - 1024, 16384),
                 block_q=bq, keep_percent=15.0)
    x = make_inputs(w)
    q, k, v = device_inputs(x)
    params = dict(sink_range=w.sink_range, extra_tokens=w.extra_tokens, dense_rows=w.dense_rows)
    if method == "sol":
        params["tau"] = w.tau
    elif method == "sla":
        params["keep_percent"] = w.keep_percent
    else:
        params["grid"] = (w.T, w.Hh, w.Ww)
    call = {"sol": sa.sol_attn, "sla": sa.sla_attn, "local3d": sa.local3d_attn}[method]
    Mq = w.N // bq
    print(f"\n[chunked] {method}: whole call", flush=True)
    ref = call(q, k, v, block_q=bq, **params)
    print(f"[chunked] {method}: 5 chunks of 3328 rows", flush=True)
    store = []
    got, rep = chunked_attention(method, q, k, v, chunk_rows=3328, block_q=bq,
                                 on_chunk=_chunk_collector(method, 1, w.H, w.N, w.d, bq, store),
                                 flags=sa.FLAG_KEEP_SELECTION, **params)
    torch.cuda.synchronize()
    assert len(rep.chunks) == math.ceil(16384 / (3328 // bq * bq)) and rep.halvings == 0
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    # the chunked path against the oracle: every chunk's selection, and sampled outputs
    r1 = _check_against_oracle(method, x, w, got, _assemble(store, Mq), bq, params, seed=300)
    print(f"[chunked] {method}: vs oracle mask flips {r1.mask_flips} extra flips {r1.extra_flips} "
          f"max {r1.max_abs:.3e} mean {r1.mean_abs:.3e}", flush=True)

    # an allocator that refuses more than the workspace of 2048 rows: the chunk is halved
    limit = sa.workspace_bytes({"sol": sa.MODE_SOL, "sla": sa.MODE_SLA,
                                "local3d": sa.MODE_LOCAL3D}[method], sa.BF16, 1, w.H, w.N, w.d,
                               bq, 64, 2048, w.extra_tokens)

    def alloc(nbytes):
        if nbytes > limit:
            raise torch.cuda.OutOfMemoryError(f"test allocator: {nbytes} > {limit} bytes")
        return torch.empty(nbytes, dtype=torch.uint8, device=q.device)

    print(f"[chunked] {method}: 16384-row chunk under a 2048-row memory limit", flush=True)
    store2 = []
    got2, rep2 = chunked_attention(method, q, k, v, chunk_rows=16384, block_q=bq, alloc=alloc,
                                   on_chunk=_chunk_collector(method, 1, w.H, w.N, w.d, bq, store2),
                                   flags=sa.FLAG_KEEP_SELECTION, **params)
    torch.cuda.synchronize()
    assert rep2.halvings == 3 and rep2.final_chunk == 2048 and len(rep2.chunks) == 8
    assert torch.equal(got2.view(torch.int16), ref.view(torch.int16))
    r2 = _check_against_oracle(method, x, w, got2, _assemble(store2, Mq), bq, params, seed=400)
    print(f"[chunked] {method}: halved, vs oracle max {r2.max_abs:.3e} mean {r2.mean_abs:.3e}",
          flush=True)
