"""Textbook dense softmax attention in fp64: out = softmax(Q K^T / sqrt(d)) V.

TEST INFRASTRUCTURE ONLY (see oracle/solattn.py).  This is the limit the sparse
pass must reach when every key block is kept; it is written independently of the
block oracle so that the two can pin each other.
"""
import math

import numpy as np


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """q, k, v [N, d] (or [..., N, d]); non-causal, scale 1/sqrt(d)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    logits = q @ np.swapaxes(k, -1, -2) / math.sqrt(q.shape[-1])
    logits = logits - logits.max(axis=-1, keepdims=True)
    w = np.exp(logits)
    return (w @ v) / w.sum(axis=-1, keepdims=True)
