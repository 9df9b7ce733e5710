"""Per-call dispatch policy around the sparse forward: when a call runs sparse attention, and when
it stays dense and why (BlockSparseAttention node documentation, common-inputs table:
start_percent, end_percent, dense_blocks, min_tokens, sink_conditioning, verbose; and the
constraints section).

Rules, as the node documentation states them:
  * sequences shorter than ``min_tokens`` stay dense;
  * transformer blocks listed in ``dense_blocks`` (a string such as ``"0, 1, 47-49"``) stay dense;
    the list is ignored for a model that reports no block index (noted when verbose);
  * before ``start_percent`` and after ``end_percent`` of the sampling schedule attention stays
    dense (sparse inside the window, both ends included);
  * ``sink_conditioning`` (exact_kv / exact_kv_and_rows / off) applies only when the conditioning
    layout matches the current sequence length: ``exact_kv`` makes every query attend the packed
    conditioning rows exactly (a key sink at the front), ``exact_kv_and_rows`` also runs the
    target audio query rows densely;
  * ``vsa`` needs the FastH3 model's learned coarse branch and is not provided here.

Dense calls run the same library with every key block kept (tau = -inf), which is exact dense
attention, unless the caller passes its own dense backend.
"""
from __future__ import annotations

import logging
import math
from dataclasses import dataclass, field

log = logging.getLogger("block_sparse_attention_scores_amd")

METHODS = ("sol-attn", "sla", "vsa")
SINK_MODES = ("exact_kv", "exact_kv_and_rows", "off")
MAX_DENSE_BLOCK = 1 << 20


def parse_dense_blocks(text: str) -> frozenset:
    """Transformer block indices from a string of comma-separated indices and inclusive ranges,
    e.g. ``"0, 1, 47-49"`` -> {0, 1, 47, 48, 49}.  Empty or blank text gives the empty set.
    Raises ValueError on anything else (negative numbers, reversed ranges, stray characters)."""
    out = set()
    if text is None:
        return frozenset()
    for part in text.split(","):
        part = part.strip()
        if not part:
            continue
        if "-" in part:
            lo, _, hi = part.partition("-")
            lo, hi = lo.strip(), hi.strip()
            if not (lo.isdigit() and hi.isdigit()):
                raise ValueError(f"dense_blocks: bad range {part!r}")
            a, b = int(lo), int(hi)
            if b < a:
                raise ValueError(f"dense_blocks: reversed range {part!r}")
            if b > MAX_DENSE_BLOCK:
                raise ValueError(f"dense_blocks: index too large in {part!r}")
            out.update(range(a, b + 1))
        else:
            if not part.isdigit():
                raise ValueError(f"dense_blocks: bad index {part!r}")
            out.add(int(part))
    return frozenset(out)


@dataclass(frozen=True)
class SinkLayout:
    """The conditioning layout a model reports for one sequence: ``seq_len`` tokens in total, of
    which the first ``packed_rows`` are packed text/audio/reference rows, and the target audio
    query rows are ``[audio_rows[0], audio_rows[1])``."""
    seq_len: int
    packed_rows: int
    audio_rows: tuple = (0, 0)


@dataclass(frozen=True)
class Decision:
    sparse: bool
    reason: str
    sink_range: int = 0
    dense_rows: tuple = (0, 0)


@dataclass
class SparseAttentionPolicy:
    """The node's inputs (defaults and ranges from its documentation)."""
    method: str = "sol-attn"
    tau: float = 1.3                   # 0 .. 4, step 0.05
    keep_percent: float = 10.0         # 0.5 .. 95, step 0.5 (sla)
    extra_tokens: int = 256            # 0 .. 256, step 64
    start_percent: float = 0.2         # 0 .. 1
    end_percent: float = 1.0           # 0 .. 1
    dense_blocks: str = ""
    min_tokens: int = 12288            # 0 .. 1048576, step 512
    sink_conditioning: str = "exact_kv_and_rows"
    verbose: bool = False
    _blocks: frozenset = field(default=frozenset(), init=False, repr=False)

    def __post_init__(self):
        if self.method not in METHODS:
            raise ValueError(f"method {self.method!r} not in {METHODS}")
        if self.sink_conditioning not in SINK_MODES:
            raise ValueError(f"sink_conditioning {self.sink_conditioning!r} not in {SINK_MODES}")
        if not (0.0 <= self.tau <= 4.0):
            raise ValueError(f"tau {self.tau} outside [0, 4]")
        if not (0.5 <= self.keep_percent <= 95.0):
            raise ValueError(f"keep_percent {self.keep_percent} outside [0.5, 95]")
        if not (0 <= self.extra_tokens <= 256):
            raise ValueError(f"extra_tokens {self.extra_tokens} outside [0, 256]")
        if not (0.0 <= self.start_percent <= 1.0 and 0.0 <= self.end_percent <= 1.0):
            raise ValueError("start_percent and end_percent must lie in [0, 1]")
        if not (0 <= self.min_tokens <= 1048576):
            raise ValueError(f"min_tokens {self.min_tokens} outside [0, 1048576]")
        self._blocks = parse_dense_blocks(self.dense_blocks)

    def decide(self, seq_len: int, *, block_index=None, progress=None,
               layout: SinkLayout | None = None) -> Decision:
        """Sparse or dense for one attention call: ``seq_len`` tokens, transformer block
        ``block_index`` (None if the model does not report it), sampling ``progress`` in [0, 1]
        (None if unknown: treated as inside the window), conditioning ``layout`` (None if the
        model reports none)."""
        if self.method == "vsa":
            return Decision(False, "vsa needs the FastH3 model's coarse branch, not provided here")
        if seq_len < self.min_tokens:
            return Decision(False, f"sequence of {seq_len} tokens is shorter than min_tokens={self.min_tokens}")
        if self._blocks:
            if block_index is None:
                if self.verbose:
                    log.info("dense_blocks ignored: the model reports no block index")
            elif block_index in self._blocks:
                return Decision(False, f"block {block_index} is listed in dense_blocks")
        if progress is not None:
            if progress < self.start_percent:
                return Decision(False, f"progress {progress:.3f} is before start_percent={self.start_percent}")
            if progress > self.end_percent:
                return Decision(False, f"progress {progress:.3f} is after end_percent={self.end_percent}")
        sink, rows = 0, (0, 0)
        if self.sink_conditioning != "off" and layout is not None:
            if layout.seq_len != seq_len:
                if self.verbose:
                    log.info("sink_conditioning skipped: layout for %d tokens, sequence has %d",
                             layout.seq_len, seq_len)
            else:
                sink = int(layout.packed_rows)
                if self.sink_conditioning == "exact_kv_and_rows":
                    rows = (int(layout.audio_rows[0]), int(layout.audio_rows[1]))
        return Decision(True, f"sparse {self.method}", sink, rows)

    def attention(self, q, k, v, *, block_index=None, progress=None, layout=None,
                  dense_backend=None, block_q=None, block_k=64):
        """Run one attention call on [B, H, N, d] GPU tensors under this policy; returns the
        output.  The sparse path is libsolattn; the dense path is ``dense_backend(q, k, v)`` if
        given, else libsolattn with every block kept (exact dense attention)."""
        from . import _lib as L
        N = q.shape[2]
        dec = self.decide(N, block_index=block_index, progress=progress, layout=layout)
        if self.verbose:
            log.info("attention %s: %s (%s)", tuple(q.shape), "sparse" if dec.sparse else "dense",
                     dec.reason)
        if not dec.sparse:
            if dense_backend is not None:
                return dense_backend(q, k, v)
            return L.sol_attn(q, k, v, tau=-math.inf, block_q=block_q or 64, block_k=block_k,
                              sink_range=0, extra_tokens=0)
        if self.method == "sol-attn":
            return L.sol_attn(q, k, v, tau=self.tau, block_q=block_q or 64, block_k=block_k,
                              sink_range=dec.sink_range, extra_tokens=self.extra_tokens,
                              dense_rows=dec.dense_rows)
        return L.sla_attn(q, k, v, keep_percent=self.keep_percent, block_q=block_q or 128,
                          block_k=block_k, sink_range=dec.sink_range,
                          extra_tokens=self.extra_tokens, dense_rows=dec.dense_rows)
