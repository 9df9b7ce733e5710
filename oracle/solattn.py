"""Plain fp64 CPU oracle of the block-sparse attention forward (sol-attn, sla and the static
local 3-D neighbourhood pattern).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module; only the tests, the smoke check and the bench's CPU-baseline leg do.  It
shares no code with the HIP library.

Sources (pages on the ComfyUI "BlockSparseAttention" node and its relatives):
  [node-zh]  "BlockSparseAttention - ComfyUI Built-in Node Documentation" (Chinese),
             tables "通用输入" (common inputs), "sol-attn 输入", "sla 输入".
  [node-ja]  the same document in Japanese (tables "共通入力", "sol-attn 入力", "sla 入力").
  [star7]    README of the minimax-h3-chunk-star7 node pack, sections "SLA" and "Sol".
  [h3-bsa]   the article on why block sparse attention matters for H3 in ComfyUI, section 1:
             a fixed pattern keeping the centre block, its neighbours one frame back and
             forward, and its spatial neighbours one block up, down, left and right; every
             other block is zero.

The method, step by step (one (batch, head) problem at a time; every problem is
independent):
  1. pool     q̄_i, k̄_j, v̄_j = means over the query block I_i and key block J_j
              ([star7] "Sol": skipped blocks enter through K/V centroids; a
              centroid is the block mean).
  2. score    s_ij = c * q̄_i . k̄_j, c = 1/sqrt(d)  ([node-zh] sol-attn table, tau
              row: the threshold is measured in standard deviations of this
              score distribution).
  3. select   sol: keep j when s_ij > mean_i + tau * std_i  (population std over
              all M blocks of the row); sla: keep the top ceil(p*M/100) blocks
              among the non-forced ones.  Sink blocks and the diagonal block(s)
              are always kept on top ([node-zh]/[node-ja] sla table, keep_percent
              row; common-inputs table, sink_conditioning row).
  4. extra    each query block also attends up to `extra_tokens` individual keys,
              the highest scoring q̄_i . k_t among tokens outside its kept blocks
              ([node-zh] common-inputs table, extra_tokens row).
  5. attend   every key token enters each query row exactly once, all in one
              softmax: exactly (logit c q_r.k_t, value v_t) when its block is kept
              or it is an extra token; otherwise, for sol, through its block's
              centroid (logit c q_r.k̄_j, value v̄_j), which for block j amounts to
              a term of multiplicity m_ij = n_j - |E_i ∩ J_j|; for sla, not at all
              ([star7] "SLA": only routed K/V blocks are computed; "Sol": exact
              kept blocks plus centroid terms merged in one FP32 online softmax).
  Query rows inside the dense row range attend every key exactly
  ([node-zh] common-inputs table, sink_conditioning row: exact_kv_and_rows).
  local3d replaces step 3 by the fixed pattern of [h3-bsa] section 1 (no scores are
  used) and drops skipped blocks in step 5 like sla.  The sequence is a video grid of
  frames x height x width tokens in raster order (frame-major, then row, then column)
  and blocks are runs of consecutive tokens, so the pattern is stated on tokens and
  lifted to blocks: key block j is kept for query block i when some token of j is a
  token of i or one of its six grid neighbours (same row and column one frame away,
  same frame and column one row away, same frame and row one column away).  When a
  frame holds a whole number of blocks and a block holds a whole number of rows, or
  a row a whole number of blocks, this is exactly the centre / +-1 frame / +-1 block
  up, down, left, right stencil on the grid of blocks.

Readings where the pages are silent (each listed in the design notes):
  c = 1/sqrt(d); non-causal; mean pooling over the block's actual tokens; strict
  '>' in the threshold; sigma = 0 gives threshold = mean; tau = -inf keeps all;
  sla count k = ceil(p*M/100) capped at M - |F_i|, ties to the lower block index;
  extra-token score unscaled q̄_i . k_t, ties to the lower token index, one set
  per query block; the diagonal is every key block overlapping the query
  block's token range; sink blocks are the key blocks overlapping [0, sink_range).
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------- geometry

def block_ranges(N: int, bs: int):
    """Token ranges [lo, hi) of the ceil(N/bs) blocks of size bs (the last may be short)."""
    return [(lo, min(lo + bs, N)) for lo in range(0, N, bs)]


def forced_blocks(i: int, N: int, block_q: int, block_k: int, sink_range: int) -> np.ndarray:
    """F_i: key blocks that overlap the sink region [0, sink_range) or query block i's tokens.

    Sink blocks and the diagonal are kept on top of the routed ones ([node-ja] sla
    table, keep_percent row; [node-zh] sink_conditioning row: every query attends
    the packed conditioning rows exactly).
    """
    M = -(-N // block_k)
    f = np.zeros(M, dtype=bool)
    qlo, qhi = i * block_q, min((i + 1) * block_q, N)
    for j, (lo, hi) in enumerate(block_ranges(N, block_k)):
        if lo < sink_range:
            f[j] = True
        if lo < qhi and qlo < hi:
            f[j] = True
    return f


# ---------------------------------------------------------------- step 1, 2

def pool(x: np.ndarray, bs: int) -> np.ndarray:
    """Block means of x [N, d] over consecutive blocks of bs tokens ([star7] "Sol": K/V centroids)."""
    return np.stack([x[lo:hi].mean(axis=0) for lo, hi in block_ranges(x.shape[0], bs)])


def scores(qbar: np.ndarray, kbar: np.ndarray, d: int) -> np.ndarray:
    """s_ij = q̄_i . k̄_j / sqrt(d): the block score whose per-row spread tau is measured in."""
    return (qbar @ kbar.T) / math.sqrt(d)


# ---------------------------------------------------------------- step 3

def row_stats(s_row: np.ndarray):
    """Mean and population standard deviation of one row of block scores, in two passes."""
    M = s_row.shape[0]
    mu = s_row.sum() / M
    var = ((s_row - mu) ** 2).sum() / M
    return mu, math.sqrt(var)


def select_sol(s_row: np.ndarray, tau: float, forced: np.ndarray) -> np.ndarray:
    """sol-attn adaptive threshold ([node-zh] sol-attn table, tau row).

    Keep block j when s_ij > mean + tau*std; forced blocks are always kept.
    tau = -inf keeps everything; std = 0 makes the threshold the mean.
    """
    if tau == -math.inf:
        return np.ones_like(forced)
    mu, sd = row_stats(s_row)
    theta = mu + tau * sd if sd > 0 else mu
    return forced | (s_row > theta)


def sla_count(keep_percent: float, M: int) -> int:
    """Number of routed blocks per row before the forced ones: ceil(p*M/100)."""
    return int(math.ceil(float(keep_percent) * M / 100.0))


def select_sla(s_row: np.ndarray, keep_percent: float, forced: np.ndarray) -> np.ndarray:
    """sla fixed-percentage routing ([node-zh]/[node-ja] sla table, keep_percent row).

    Keep the k = min(M-|F|, ceil(p*M/100)) highest-scoring non-forced blocks
    (ties to the lower index), plus every forced block on top.
    """
    M = s_row.shape[0]
    free = np.flatnonzero(~forced)
    k = min(len(free), sla_count(keep_percent, M))
    # lexsort: last key is primary -> order by score descending, then index ascending
    order = free[np.lexsort((free, -s_row[free]))]
    keep = forced.copy()
    keep[order[:k]] = True
    return keep


def local3d_neighbours(i: int, N: int, block_q: int, block_k: int, grid) -> np.ndarray:
    """Key blocks holding a token of query block i or a grid neighbour of one ([h3-bsa] §1).

    grid = (frames, height, width) with frames*height*width == N; token p sits at frame
    p // (height*width), row (p % (height*width)) // width, column p % width.  Neighbours
    differ by one in exactly one coordinate and stay inside the grid (no wrap-around).
    """
    F, Hh, Ww = (int(g) for g in grid)
    assert F * Hh * Ww == N, "the grid must cover the sequence"
    M = -(-N // block_k)
    keep = np.zeros(M, dtype=bool)
    p = np.arange(i * block_q, min((i + 1) * block_q, N))
    t, rem = np.divmod(p, Hh * Ww)
    y, x = np.divmod(rem, Ww)
    for dt, dy, dx in ((0, 0, 0), (-1, 0, 0), (1, 0, 0), (0, -1, 0), (0, 1, 0), (0, 0, -1),
                       (0, 0, 1)):
        tt, yy, xx = t + dt, y + dy, x + dx
        ok = (tt >= 0) & (tt < F) & (yy >= 0) & (yy < Hh) & (xx >= 0) & (xx < Ww)
        keep[(tt[ok] * Hh * Ww + yy[ok] * Ww + xx[ok]) // block_k] = True
    return keep


def select_local3d(neighbours: np.ndarray, forced: np.ndarray) -> np.ndarray:
    """Static local routing ([h3-bsa] §1): the neighbourhood plus the forced blocks."""
    return forced | neighbours


# ---------------------------------------------------------------- step 4

def extra_select(e_row: np.ndarray, kept: np.ndarray, block_k: int, n_extra: int) -> np.ndarray:
    """Extra tokens of one query block ([node-zh] common-inputs table, extra_tokens row).

    e_row[t] = q̄_i . k_t for every token t.  Among the tokens whose key block is
    not kept, take the top min(n_extra, count) by e (descending, ties to the lower
    token index).  Returns the chosen token indices in ascending order.
    """
    if n_extra <= 0:
        return np.zeros(0, dtype=np.int64)
    N = e_row.shape[0]
    cand = np.flatnonzero(~kept[np.arange(N) // block_k])
    if cand.size <= n_extra:
        return cand.astype(np.int64)
    e = e_row[cand]
    # every candidate scoring at least the n-th largest value (ties included),
    # then the exact order: score descending, token index ascending
    nth = -np.partition(-e, n_extra - 1)[n_extra - 1]
    short = np.flatnonzero(e >= nth)
    order = short[np.lexsort((cand[short], -e[short]))]
    return np.sort(cand[order[:n_extra]]).astype(np.int64)


def extra_scores(qbar_rows: np.ndarray, k: np.ndarray) -> np.ndarray:
    """e[i, t] = q̄_i . k_t (unscaled: only the order matters)."""
    return qbar_rows @ k.T


# ---------------------------------------------------------------- step 5

def attend_rows(qr: np.ndarray, k: np.ndarray, v: np.ndarray, kbar: np.ndarray,
                vbar: np.ndarray, exact: np.ndarray, mult: np.ndarray, scale: float) -> np.ndarray:
    """One softmax over exact tokens and centroid terms, for query rows qr [R, d].

    exact: token indices attended exactly; mult[j]: multiplicity of key block j's
    centroid term (0 = absent).  Term weight m * exp(logit - L), L the row max
    ([star7] "Sol": exact blocks and centroid terms in one online softmax).
    """
    logit_x = (qr @ k[exact].T) * scale                      # [R, |X|]
    cj = np.flatnonzero(mult > 0)
    logit_c = (qr @ kbar[cj].T) * scale                      # [R, |C|]
    L = np.full(qr.shape[0], -np.inf)
    if logit_x.size:
        L = np.maximum(L, logit_x.max(axis=1))
    if logit_c.size:
        L = np.maximum(L, logit_c.max(axis=1))
    wx = np.exp(logit_x - L[:, None])
    wc = mult[cj][None, :] * np.exp(logit_c - L[:, None])
    num = wx @ v[exact] + wc @ vbar[cj]
    den = wx.sum(axis=1) + wc.sum(axis=1)
    return num / den[:, None]


# ---------------------------------------------------------------- whole pass

def head_forward(mode: str, q: np.ndarray, k: np.ndarray, v: np.ndarray, *, block_q: int,
                 block_k: int, tau: float = 1.3, keep_percent: float = 10.0, sink_range: int = 0,
                 extra_tokens: int = 0, dense_rows=(0, 0), selection=None, qblocks=None,
                 want_out: bool = True, grid=None):
    """The pass for one (batch, head): q, k, v [N, d] (any float dtype, widened to fp64).

    mode: "sol", "sla" or "local3d" (which needs grid = (frames, height, width)).

    Returns a dict with
      out     [N, d] fp64 (rows of query blocks not in `qblocks` are NaN),
      kept    [Mq, M] bool kept-block masks (all True for query blocks wholly
              inside the dense row range, whose selection is not computed),
      dense   [Mq] bool, query block wholly inside the dense row range,
      extra   list of Mq sorted int arrays (extra token indices),
      scores  [Mq, M] block scores, theta [Mq] thresholds (sol; NaN for sla),
      qbar, kbar, vbar.
    `selection=(kept, extra)` replaces steps 3-4 with the given lists.
    """
    assert mode in ("sol", "sla", "local3d")
    assert mode != "local3d" or grid is not None, "local3d needs the video grid"
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    scale = 1.0 / math.sqrt(d)
    qr_ = block_ranges(N, block_q)
    kr_ = block_ranges(N, block_k)
    Mq, M = len(qr_), len(kr_)
    n_j = np.array([hi - lo for lo, hi in kr_], dtype=np.float64)
    d0, d1 = dense_rows

    qbar, kbar, vbar = pool(q, block_q), pool(k, block_k), pool(v, block_k)
    s = scores(qbar, kbar, d)
    dense = np.array([d0 <= lo and hi <= d1 for lo, hi in qr_], dtype=bool)

    kept = np.ones((Mq, M), dtype=bool)
    extra = [np.zeros(0, dtype=np.int64) for _ in range(Mq)]
    theta = np.full(Mq, np.nan)
    if selection is not None:
        kept = np.asarray(selection[0], dtype=bool).copy()
        extra = [np.asarray(e, dtype=np.int64) for e in selection[1]]
    else:
        for i in range(Mq):
            if dense[i]:
                continue
            f = forced_blocks(i, N, block_q, block_k, sink_range)
            if mode == "sol":
                kept[i] = select_sol(s[i], tau, f)
                if tau != -math.inf:
                    mu, sd = row_stats(s[i])
                    theta[i] = mu + tau * sd if sd > 0 else mu
            elif mode == "sla":
                kept[i] = select_sla(s[i], keep_percent, f)
            else:
                kept[i] = select_local3d(local3d_neighbours(i, N, block_q, block_k, grid), f)
        if extra_tokens > 0:
            for i0 in range(0, Mq, 64):
                rows = [i for i in range(i0, min(i0 + 64, Mq)) if not dense[i]]
                if not rows:
                    continue
                e = extra_scores(qbar[rows], k)
                for r, i in enumerate(rows):
                    extra[i] = extra_select(e[r], kept[i], block_k, extra_tokens)

    out = np.full((N, d), np.nan) if want_out else None
    if want_out:
        todo = range(Mq) if qblocks is None else qblocks
        for i in todo:
            lo, hi = qr_[i]
            rows = np.arange(lo, hi)
            in_dense = (rows >= d0) & (rows < d1)
            if in_dense.any():
                r = rows[in_dense]
                out[r] = attend_rows(q[r], k, v, kbar, vbar, np.arange(N), np.zeros(M), scale)
            r = rows[~in_dense]
            if r.size == 0:
                continue
            kb = np.flatnonzero(kept[i])
            blk_tok = np.concatenate([np.arange(*kr_[j]) for j in kb]) if kb.size else \
                np.zeros(0, dtype=np.int64)
            ex = extra[i]
            exact = np.union1d(blk_tok, ex).astype(np.int64)
            mult = np.zeros(M)
            if mode == "sol":
                mult = np.where(kept[i], 0.0, n_j)
                if ex.size:
                    np.subtract.at(mult, ex // block_k, 1.0)
            out[r] = attend_rows(q[r], k, v, kbar, vbar, exact, mult, scale)
    return dict(out=out, kept=kept, dense=dense, extra=extra, scores=s, theta=theta,
                qbar=qbar, kbar=kbar, vbar=vbar)


def forward(mode: str, q, k, v, **kw):
    """The pass over [B, H, N, d] inputs: loops over (b, h), see head_forward."""
    B, H = q.shape[:2]
    res = [[head_forward(mode, q[b, h], k[b, h], v[b, h], **kw) for h in range(H)]
           for b in range(B)]
    out = None
    if kw.get("want_out", True):
        out = np.stack([np.stack([r["out"] for r in rb]) for rb in res])
    return dict(out=out, heads=res)


def kept_fraction(kept: np.ndarray, dense: np.ndarray) -> float:
    """Σ|A_i| / (#selected rows · M): the kept-block fraction over rows that run selection."""
    sel = ~dense
    if not sel.any():
        return float("nan")
    return float(kept[sel].sum()) / float(sel.sum() * kept.shape[1])
