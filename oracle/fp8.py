"""fp8 (OCP E4M3) flavour of the attention step, in fp64: TEST INFRASTRUCTURE ONLY (see
oracle/solattn.py; nothing on the product path may import this module).

The pages name reduced-precision speed variants of the same method without fixing a scheme
(the star7 node-pack page: INT8 QK with FP16 PV, all-INT8 SLA and Sol; the Triton SolAttnPatch
page: int8_qk / int8_pv) and say they are not value-identical to BF16.  This flavour takes the
"low-precision QK, 16-bit PV" form on the FP8 format, a reading listed in the design notes:
  * E4M3 values: sign, 4-bit exponent with bias 7, 3-bit mantissa; the zero exponent field
    holds the subnormals (step 2^-9); the largest finite value is 448; rounding is to nearest,
    ties to even.
  * scales are powers of two 2^e with e = ceil(log2(amax / 448)) (e = 0 when amax = 0; e kept
    in [-127, 127], the range of the E8M0 scale code), so that the largest scaled magnitude
    lies in (224, 448]: Q per query row, K per token, the pooled K per pooled row.
  * every logit (exact tokens and centroids) is the product of the dequantised Q and K rows;
    the softmax, the centroid multiplicities and the value products are those of the bf16
    pass, with V and the pooled V unquantised.
  * selection (kept blocks, extra tokens) is the bf16 pass's, unchanged.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def e4m3_round(x):
    """Round to the nearest E4M3 value, ties to even (values of magnitude above 448 are an
    error: the scaling keeps every input at or below it)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if (a > E4M3_MAX).any():
        raise ValueError("value beyond the E4M3 range")
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)                 # below 2^-6 the spacing stays 2^-9 (subnormals)
    q = 2.0 ** (e - 3)                      # spacing of the binade
    r = np.round(a / q) * q                 # numpy rounds halves to even
    return np.where(a > 0, np.copysign(r, x), 0.0)


def scale_exp(amax):
    """e = ceil(log2(amax / 448)) in [-127, 127], 0 for amax = 0: the power-of-two scale of a
    group."""
    amax = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / E4M3_MAX))
    return np.clip(np.where(amax > 0, e, 0.0), -127, 127)


def quantize(x, e):
    """Dequantised E4M3 image of x under scales 2^e (e broadcast against x)."""
    s = 2.0 ** np.asarray(e, dtype=np.float64)
    return e4m3_round(np.asarray(x, dtype=np.float64) / s) * s


def quantize_rows(x):
    e = scale_exp(np.abs(x).max(axis=-1))
    return quantize(x, e[..., None]), e


def quantize_cols(x):
    e = scale_exp(np.abs(x).max(axis=0))
    return quantize(x, e[None, :]), e


def head_forward_fp8qk(mode, q, k, v, *, block_q, block_k, selection, qblocks=None,
                       dense_rows=(0, 0), kbar=None, **_):
    """The fp8-QK flavour for one (batch, head) on the given selection (kept masks, extra
    lists), e.g. the GPU's own.  kbar: the pooled keys to quantise (default: the fp64 block
    means).  Returns out [N, d] fp64 (NaN outside `qblocks`)."""
    from . import solattn
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    scale = 1.0 / math.sqrt(d)
    kept, extra = np.asarray(selection[0], dtype=bool), [np.asarray(e, np.int64) for e in selection[1]]
    qr_ = solattn.block_ranges(N, block_q)
    kr_ = solattn.block_ranges(N, block_k)
    M = len(kr_)
    n_j = np.array([hi - lo for lo, hi in kr_], dtype=np.float64)
    if kbar is None:
        kbar = solattn.pool(k, block_k)
    vbar = solattn.pool(v, block_k)
    qh, _ = quantize_rows(q)
    kh, _ = quantize_rows(k)
    kbh, _ = quantize_rows(np.asarray(kbar, dtype=np.float64))
    d0, d1 = dense_rows
    out = np.full((N, d), np.nan)
    todo = range(len(qr_)) if qblocks is None else qblocks
    for i in todo:
        lo, hi = qr_[i]
        rows = np.arange(lo, hi)
        in_dense = (rows >= d0) & (rows < d1)
        if in_dense.any():
            r = rows[in_dense]
            out[r] = solattn.attend_rows(qh[r], kh, v, kbh, vbar, np.arange(N), np.zeros(M), scale)
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
        out[r] = solattn.attend_rows(qh[r], kh, v, kbh, vbar, exact, mult, scale)
    return out
