"""Row-chunked driver over the library call, halving the chunk when memory runs out (the
minimax-h3-chunk-star7 node-pack page: the paragraph on chunking along the token dimension so
that only the current chunk's intermediates are held, and the main-features table, row on the
automatic VRAM step-down: when a chunkable stage runs out of memory, that stage's chunk is
halved and retried while every other setting stays as it was).

The library computes one window of query rows per call (``q_rows``: the ``q_row_begin`` /
``q_row_end`` options) with a workspace that covers the window only, so a call's extra memory
scales with its chunk.  This driver walks the sequence in chunks of query rows (whole query
blocks), allocates each chunk's workspace, and when that allocation or the call fails for lack
of memory, halves the chunk (never below one query block) and retries the same rows; the halved
size is kept for the rest of the sequence.  A query block's result does not depend on how the
rows are chunked, so the output equals that of one whole call.
"""
from __future__ import annotations

from dataclasses import dataclass, field


class ChunkTooLarge(Exception):
    """Raised by an attempt when its chunk does not fit in memory."""


@dataclass
class ChunkReport:
    chunks: list = field(default_factory=list)      # (begin, end) of every chunk computed
    halvings: int = 0                                # times the chunk size was halved
    final_chunk: int = 0                             # chunk size at the end


def run_chunks(n_rows: int, block: int, chunk: int, attempt) -> ChunkReport:
    """Cover rows [0, n_rows) with chunks of ``chunk`` rows (rounded down to whole blocks, at
    least one block), calling ``attempt(begin, end)`` for each.  An attempt that raises
    ChunkTooLarge is retried on the same rows with the chunk halved; at one block the error is
    re-raised."""
    if n_rows % block:
        raise ValueError(f"{n_rows} rows are not a whole number of {block}-row blocks")
    size = max(block, min(chunk, n_rows) // block * block)
    rep = ChunkReport()
    begin = 0
    while begin < n_rows:
        end = min(begin + size, n_rows)
        try:
            attempt(begin, end)
        except ChunkTooLarge:
            if size == block:
                raise
            size = max(block, size // 2 // block * block)
            rep.halvings += 1
            continue
        rep.chunks.append((begin, end))
        begin = end
    rep.final_chunk = size
    return rep


def _is_oom(exc) -> bool:
    import torch
    from ._lib import EHIP, SolattnError
    if isinstance(exc, torch.cuda.OutOfMemoryError):
        return True
    if isinstance(exc, SolattnError) and exc.status == EHIP:
        d = exc.detail.lower()
        return "hipmalloc" in d or "out of memory" in d
    return False


def chunked_attention(method: str, q, k, v, *, chunk_rows: int, block_q: int = 64,
                      block_k: int = 64, out=None, alloc=None, on_chunk=None, **params):
    """Run ``method`` ("sol", "sla" or "local3d") over [B, H, N, d] GPU tensors in chunks of
    ``chunk_rows`` query rows.  ``params`` go to the library call (tau, keep_percent, grid,
    sink_range, extra_tokens, dense_rows, flags, stream, qk_fp8).  ``alloc(nbytes)`` returns a uint8
    workspace tensor (default: torch.empty on q's device); an out-of-memory error from it or
    from the call halves the chunk.  ``on_chunk(begin, end, workspace)``, if given, is called
    after each chunk's call was enqueued (e.g. to read the chunk's selection from its
    workspace).  Returns (out, ChunkReport)."""
    import torch

    from . import _lib as L
    calls = {"sol": L.sol_attn, "sla": L.sla_attn, "local3d": L.local3d_attn}
    modes = {"sol": L.MODE_SOL, "sla": L.MODE_SLA, "local3d": L.MODE_LOCAL3D}
    if method not in calls:
        raise ValueError(f"method {method!r} not in {tuple(calls)}")
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if alloc is None:
        def alloc(nbytes):
            return torch.empty(nbytes, dtype=torch.uint8, device=q.device)

    def attempt(begin, end):
        try:
            nbytes = L.workspace_bytes(modes[method], L._dtype_code(q, params.get("qk_fp8", False)),
                                       B, H, N, d, block_q, block_k, end - begin,
                                       params.get("extra_tokens", 0))
            ws = alloc(nbytes)
            calls[method](q, k, v, block_q=block_q, block_k=block_k, out=out, workspace=ws,
                          q_rows=(begin, end), **params)
        except Exception as exc:  # noqa: BLE001 - only memory failures are retried
            if _is_oom(exc):
                raise ChunkTooLarge(str(exc)) from exc
            raise
        if on_chunk is not None:
            on_chunk(begin, end, ws)

    rep = run_chunks(N, block_q, chunk_rows, attempt)
    return out, rep
