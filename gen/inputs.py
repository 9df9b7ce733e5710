"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module holds none of the attention method's arithmetic: it only draws the
Q, K, V tensors (and names the workload parameters) that both the CPU oracle
and the HIP path consume, bit for bit.

Workload stand-in. The pages measure end to end on a video diffusion model
(MiniMax-H3 in ComfyUI); no weights or prompts are used here. Instead Q and K
carry the structure of video latents: a Gaussian-blurred noise field z over a
T x Hh x Ww token grid (token order n = (t*Hh + y)*Ww + x), projected per head
by random matrices, plus independent noise.  V is plain N(0, 1).

Recipe, per configuration (seed = 1000 + config id):
  1. z0 ~ N(0, 1), shape [T, Hh, Ww, d], float32 (one draw per batch entry).
  2. Separable discrete Gaussian blur of every channel: weights proportional to
     exp(-k^2 / (2 sigma^2)) for |k| <= ceil(3 sigma), normalised; mirror
     boundary (abcd|dcba).  Temporal sigma 1 frame, spatial sigma per config.
  3. Standardise every channel to mean 0 and variance 1 over all tokens.
  4. Per head h: Wq, Wk ~ N(0, 1/d) [d x d]; eps_q, eps_k ~ N(0, 1) [N x d];
     V ~ N(0, 1) [N x d]; Q = z Wq + 0.5 eps_q, K = z Wk + 0.5 eps_k.
  5. bf16 configurations round Q, K, V to bfloat16 with round-to-nearest-even;
     the oracle widens exactly those bits.
Every (batch, head) has its own counter-free numpy PCG64 stream seeded by
(seed, 1, b, h), so any subset of heads can be drawn on its own.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: the token grid, the head shape and the call's parameters."""
    cid: int
    name: str
    B: int
    H: int
    T: int
    Hh: int
    Ww: int
    d: int
    dtype: str                 # "bf16" or "fp32"
    mode: str                  # "sol", "sla" or "local3d"
    block_q: int
    block_k: int
    tau: float = 1.3
    keep_percent: float = 10.0
    sink_range: int = 0
    extra_tokens: int = 0
    dense_rows: tuple = (0, 0)
    blur_space: float = 2.0
    blur_time: float = 1.0
    taus: tuple = field(default_factory=tuple)

    @property
    def N(self) -> int:
        return self.T * self.Hh * self.Ww

    @property
    def seed(self) -> int:
        return 1000 + self.cid


# Shapes follow the pages: 64-token blocks for sol-attn, Q128/K64 for sla, 200k+
# tokens for long videos, 17n+5 frame counts (T=22), packed conditioning rows
# first, dense target-audio query rows.
WORKLOADS = {
    1: Workload(1, "tiny-sol-fp32", B=1, H=2, T=4, Hh=32, Ww=32, d=64, dtype="fp32", mode="sol",
                block_q=64, block_k=64, tau=1.3, blur_space=2.0),
    2: Workload(2, "sol-bf16-n16k", B=1, H=24, T=4, Hh=64, Ww=64, d=128, dtype="bf16", mode="sol",
                block_q=64, block_k=64, tau=1.3, sink_range=512, blur_space=2.0,
                taus=(1.0, 1.3, 2.0)),
    3: Workload(3, "sla-bf16-n32k", B=1, H=24, T=8, Hh=64, Ww=64, d=128, dtype="bf16", mode="sla",
                block_q=128, block_k=64, keep_percent=15.0, sink_range=64, blur_space=3.0),
    4: Workload(4, "sol-full-bf16-n64k", B=1, H=24, T=16, Hh=64, Ww=64, d=128, dtype="bf16",
                mode="sol", block_q=64, block_k=64, tau=1.3, extra_tokens=256, sink_range=1024,
                dense_rows=(65536 - 2048, 65536), blur_space=2.0),
    5: Workload(5, "sol-long-bf16-n203k", B=1, H=24, T=22, Hh=96, Ww=96, d=128, dtype="bf16",
                mode="sol", block_q=64, block_k=64, tau=1.3, extra_tokens=256, sink_range=1024,
                blur_space=2.0),
}


def workload(cid: int, **overrides) -> Workload:
    w = WORKLOADS[cid]
    return replace(w, **overrides) if overrides else w


def _gauss_weights(sigma: float) -> np.ndarray:
    r = int(math.ceil(3.0 * sigma))
    k = np.arange(-r, r + 1, dtype=np.float64)
    w = np.exp(-(k * k) / (2.0 * sigma * sigma))
    return (w / w.sum()).astype(np.float32)


def _blur_axis(z: np.ndarray, axis: int, sigma: float) -> np.ndarray:
    if sigma <= 0:
        return z
    w = _gauss_weights(sigma)
    r = (len(w) - 1) // 2
    n = z.shape[axis]
    pad = [(0, 0)] * z.ndim
    pad[axis] = (r, r)
    # 'symmetric' repeats the edge sample: abcd|dcba.  Radius may exceed n for
    # tiny grids; numpy then reflects repeatedly, which is still well defined.
    zp = np.pad(z, pad, mode="symmetric")
    out = np.zeros_like(z)
    for i, wi in enumerate(w):
        sl = [slice(None)] * z.ndim
        sl[axis] = slice(i, i + n)
        out += wi * zp[tuple(sl)]
    return out


def latent_field(w: Workload, b: int = 0) -> np.ndarray:
    """Blurred, per-channel standardised noise field z, shape [N, d] float32."""
    rng = np.random.default_rng([w.seed, 0, b])
    z = rng.standard_normal((w.T, w.Hh, w.Ww, w.d), dtype=np.float32)
    z = _blur_axis(z, 0, w.blur_time)
    z = _blur_axis(z, 1, w.blur_space)
    z = _blur_axis(z, 2, w.blur_space)
    z = z.reshape(w.N, w.d)
    mu = z.mean(axis=0, dtype=np.float64).astype(np.float32)
    sd = z.std(axis=0, dtype=np.float64).astype(np.float32)
    return (z - mu) / sd


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def head_tensors(w: Workload, z: np.ndarray, b: int, h: int):
    """Q, K, V of one (batch, head) as float32 [N, d] (before any rounding)."""
    rng = np.random.default_rng([w.seed, 1, b, h])
    d = w.d
    s = np.float32(1.0 / math.sqrt(d))
    wq = rng.standard_normal((d, d), dtype=np.float32) * s
    wk = rng.standard_normal((d, d), dtype=np.float32) * s
    eq = rng.standard_normal((w.N, d), dtype=np.float32)
    ek = rng.standard_normal((w.N, d), dtype=np.float32)
    v = rng.standard_normal((w.N, d), dtype=np.float32)
    q = z @ wq + np.float32(0.5) * eq
    k = z @ wk + np.float32(0.5) * ek
    return q, k, v


@dataclass
class Inputs:
    """Q, K, V as stored for the GPU (bits) and as exact float32 values for the oracle."""
    w: Workload
    heads: tuple
    q: np.ndarray          # [B, len(heads), N, d] float32, exactly representable in w.dtype
    k: np.ndarray
    v: np.ndarray
    q_bits: np.ndarray | None = None   # uint16 bf16 patterns (bf16 workloads only)
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None


def make_inputs(w: Workload | int, heads=None, threads: int | None = None) -> Inputs:
    """Draw Q, K, V for workload ``w`` (all heads, or the listed subset).

    Heads are drawn in parallel threads; each has its own random stream, so the result does
    not depend on the thread count.
    """
    from concurrent.futures import ThreadPoolExecutor

    if isinstance(w, int):
        w = WORKLOADS[w]
    heads = tuple(range(w.H)) if heads is None else tuple(heads)
    shape = (w.B, len(heads), w.N, w.d)
    bf = w.dtype == "bf16"
    out = {n: np.empty(shape, np.float32) for n in "qkv"}
    bits = {n: np.empty(shape, np.uint16) for n in "qkv"} if bf else None
    nthr = threads or min(8, os.cpu_count() or 1)
    for b in range(w.B):
        z = latent_field(w, b)

        def one(item):
            hi, h = item
            for name, x in zip("qkv", head_tensors(w, z, b, h)):
                if bf:
                    bb = bf16_round(x)
                    bits[name][b, hi] = bb
                    out[name][b, hi] = bf16_to_f32(bb)
                else:
                    out[name][b, hi] = x

        with ThreadPoolExecutor(max_workers=nthr) as ex:
            list(ex.map(one, enumerate(heads)))
    if bf:
        return Inputs(w, heads, out["q"], out["k"], out["v"], bits["q"], bits["k"], bits["v"])
    return Inputs(w, heads, out["q"], out["k"], out["v"])


def random_qkv(B, H, N, d, seed, dtype="fp32"):
    """Plain iid N(0,1) Q, K, V (edge-case tests); same Inputs container."""
    rng = np.random.default_rng([seed, 7])
    xs = [rng.standard_normal((B, H, N, d), dtype=np.float32) for _ in range(3)]
    w = Workload(0, "iid", B=B, H=H, T=1, Hh=1, Ww=N, d=d, dtype=dtype, mode="sol",
                 block_q=64, block_k=64)
    if dtype == "bf16":
        bits = [bf16_round(x) for x in xs]
        vals = [bf16_to_f32(b) for b in bits]
        return Inputs(w, tuple(range(H)), *vals, *bits)
    return Inputs(w, tuple(range(H)), *xs)
