"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI and compare
its intermediate and final results with the CPU oracle under the stated tolerances.

Tolerances:
  * pooled means: fp32 sums of 64 values, |Δ| <= 4e-6 * max|input| of the head;
  * block scores: one fp32 dot product of d terms, |Δ| <= 1e-5 * scale * (|q̄| . |k̄|);
  * kept masks: bit-exact except blocks whose fp64 score lies within 1e-4 * σ_i of the row's
    threshold (sol) or of the k-th non-forced score (sla); such flips are counted.  The static
    local 3-D pattern uses no scores: its masks are bit-exact, and its scores are not written;
  * extra sets (rows whose masks agree): exact except tokens within 1e-4 * σ_e of the boundary
    score, σ_e the std of the row's candidate scores;
  * outputs, against the oracle run on the GPU's own selection: bf16 max-abs 2e-2 and
    mean-abs 2e-3; fp32 max-abs 1e-4.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import block_sparse_attention_scores_amd as sa
from oracle import solattn

BAND = 1e-4


def device_inputs(x):
    if x.w.dtype == "bf16" or x.q_bits is not None:
        f = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
        return f(x.q_bits), f(x.k_bits), f(x.v_bits)
    return tuple(torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (x.q, x.k, x.v))


MODES = {"sol": sa.MODE_SOL, "sla": sa.MODE_SLA, "local3d": sa.MODE_LOCAL3D}


def run_gpu(mode, q, k, v, *, block_q, block_k, tau=1.3, keep_percent=10.0, sink_range=0,
            extra_tokens=0, dense_rows=(0, 0), flags=0, grid=None):
    # the kept lists and multiplicities are written on request only; the parity checks read them
    flags |= sa.FLAG_KEEP_SELECTION
    if mode == "local3d":
        out, ws = sa.local3d_attn(q, k, v, grid=grid, block_q=block_q, block_k=block_k,
                                  sink_range=sink_range, extra_tokens=extra_tokens,
                                  dense_rows=dense_rows, return_workspace=True, flags=flags)
    elif mode == "sol":
        out, ws = sa.sol_attn(q, k, v, tau=tau, block_q=block_q, block_k=block_k,
                              sink_range=sink_range, extra_tokens=extra_tokens,
                              dense_rows=dense_rows, return_workspace=True, flags=flags)
    else:
        out, ws = sa.sla_attn(q, k, v, keep_percent=keep_percent, block_q=block_q,
                              block_k=block_k, sink_range=sink_range, extra_tokens=extra_tokens,
                              dense_rows=dense_rows, return_workspace=True, flags=flags)
    torch.cuda.synchronize()
    B, H, N, d = q.shape
    dt = sa.BF16 if q.dtype == torch.bfloat16 else sa.FP32
    views = sa.selection_views(ws, MODES[mode], dt, B, H, N, d, block_q, block_k)
    sel = {k_: v_.cpu().numpy() for k_, v_ in views.items()}
    return out.float().cpu().numpy().astype(np.float64), sel


def gpu_kept_mask(sel, bh, M):
    cnt = sel["kept_cnt"][bh]
    idx = sel["kept_idx"][bh]
    mask = np.zeros((cnt.shape[0], M), dtype=bool)
    for i in range(cnt.shape[0]):
        mask[i, idx[i, :cnt[i]]] = True
    return mask


def gpu_extra_sets(sel, bh):
    cnt = sel["extra_cnt"][bh]
    idx = sel["extra_idx"][bh]
    return [idx[i, :cnt[i]].astype(np.int64) for i in range(cnt.shape[0])]


class Report:
    def __init__(self):
        self.mask_flips = 0
        self.extra_flips = 0
        self.rows = 0
        self.max_abs = 0.0
        self.mean_abs = 0.0


def check_head(mode, ref, sel, bh, *, x_in, d, block_k, tau, keep_percent, sink_range, block_q,
               N, extra_tokens, report, qblocks=None, out_gpu=None, q=None, k=None, v=None,
               dense_rows=(0, 0), dtype="bf16", grid=None):
    """Compare one head's intermediates and (sampled) outputs. ref = oracle head_forward dict."""
    Mq, M = ref["kept"].shape
    scale = 1.0 / math.sqrt(d)
    # pooled means
    mx = max(np.abs(x_in[t]).max() for t in range(3))
    for name in ("qbar", "kbar", "vbar"):
        g = sel[name][bh].astype(np.float64)
        np.testing.assert_allclose(g, ref[name], rtol=0, atol=4e-6 * mx, err_msg=name)
    # scores (the static local pattern computes none)
    if mode != "local3d":
        bound = 1e-5 * scale * (np.abs(ref["qbar"]) @ np.abs(ref["kbar"]).T) + 1e-30
        ds = np.abs(sel["scores"][bh].astype(np.float64) - ref["scores"])
        assert (ds <= bound).all(), f"score error {ds.max()} > bound"
    # masks: the ascending lists and the bitmap the attention kernel walks hold the same sets
    gmask = gpu_kept_mask(sel, bh, M)
    assert np.array_equal(gmask, sa.kept_masks(sel, bh, M)), "kept lists and bitmap differ"
    s = ref["scores"]
    for i in range(Mq):
        if ref["dense"][i]:
            assert gmask[i].all()
            continue
        diff = np.flatnonzero(gmask[i] != ref["kept"][i])
        if diff.size == 0:
            continue
        assert mode != "local3d", f"row {i}: static pattern differs at blocks {diff}"
        mu, sd = solattn.row_stats(s[i])
        if mode == "sol":
            edge = mu + tau * sd if sd > 0 else mu
        else:
            f = solattn.forced_blocks(i, N, block_q, block_k, sink_range)
            free = np.flatnonzero(~f)
            kk = min(free.size, solattn.sla_count(keep_percent, M))
            order = free[np.lexsort((free, -s[i][free]))]
            edge = s[i][order[kk - 1]] if kk > 0 else np.inf
        assert (np.abs(s[i][diff] - edge) <= BAND * sd).all(), \
            f"row {i}: mask flips outside the band: {diff} {s[i][diff]} edge {edge} sd {sd}"
        report.mask_flips += diff.size
    report.rows += Mq
    # extra sets
    gextra = gpu_extra_sets(sel, bh)
    if extra_tokens > 0:
        kk_ = ref["kbar"]  # noqa: F841
        for i in range(Mq):
            if ref["dense"][i] or not np.array_equal(gmask[i], ref["kept"][i]):
                continue
            a, b = set(gextra[i].tolist()), set(ref["extra"][i].tolist())
            assert len(gextra[i]) == len(ref["extra"][i]), f"row {i}: extra count"
            assert np.all(np.diff(gextra[i]) > 0), f"row {i}: extra list not ascending/unique"
            if a == b:
                continue
            kt = x_in[1]
            e_all = kt @ ref["qbar"][i]
            cand = np.flatnonzero(~ref["kept"][i][np.arange(N) // block_k])
            sd_e = e_all[cand].std()
            edge = min(e_all[list(b)])
            for t in a ^ b:
                assert abs(e_all[t] - edge) <= BAND * sd_e, f"row {i}: extra flip {t} outside band"
            report.extra_flips += len(a ^ b)
        # every gpu extra token lies outside the gpu kept blocks
        for i in range(Mq):
            if gextra[i].size:
                assert not gmask[i][gextra[i] // block_k].any()
    # multiplicities (sol): block size minus the extra tokens taken from it, 0 if kept
    if mode == "sol":
        for i in range(Mq):
            if ref["dense"][i]:
                continue
            m = np.where(gmask[i], 0, block_k).astype(np.int64)
            if gextra[i].size:
                np.subtract.at(m, gextra[i] // block_k, 1)
            assert np.array_equal(sel["mult"][bh][i][:M].astype(np.int64), m), f"row {i}: multiplicity"
    # outputs against the oracle on the GPU's own selection
    if out_gpu is not None:
        inj = solattn.head_forward(mode, x_in[0], x_in[1], x_in[2], block_q=block_q, block_k=block_k,
                                   tau=tau, keep_percent=keep_percent, sink_range=sink_range,
                                   extra_tokens=extra_tokens, dense_rows=dense_rows,
                                   selection=(gmask, gextra), qblocks=qblocks, grid=grid)
        rows = np.flatnonzero(~np.isnan(inj["out"][:, 0]))
        err = np.abs(out_gpu[rows] - inj["out"][rows])
        report.max_abs = max(report.max_abs, float(err.max()))
        report.mean_abs = max(report.mean_abs, float(err.mean()))
        if dtype == "bf16":
            assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
        else:
            assert err.max() <= 1e-4, err.max()
