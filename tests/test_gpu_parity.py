"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on seeded inputs.

Small cases are compared element by element on every output row; the full-size workloads
(N = 65536 and N = 202752, all 24 heads, the launch the bench times) are checked on every
intermediate of sampled heads and on the outputs of sampled query blocks.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_scores_amd as sa
from gen import Inputs, Workload, bf16_round, bf16_to_f32, make_inputs, random_qkv, workload
from oracle import dense, solattn
from parity import Report, check_head, device_inputs, gpu_kept_mask, run_gpu

pytestmark = pytest.mark.gpu


def params(w, mode=None, **ov):
    p = dict(block_q=w.block_q, block_k=w.block_k, tau=w.tau, keep_percent=w.keep_percent,
             sink_range=w.sink_range, extra_tokens=w.extra_tokens, dense_rows=w.dense_rows)
    if (mode or w.mode) == "local3d":
        p["grid"] = (w.T, w.Hh, w.Ww)
    p.update(ov)
    return p


def run_and_check(w, x, heads_to_check, qblocks=None, mode=None, flags=0, **ov):
    mode = mode or w.mode
    p = params(w, mode, **ov)
    print(f"\n[parity] {w.name} mode={mode} H={x.q.shape[1]} N={w.N} flags={flags} {p}", flush=True)
    q, k, v = device_inputs(x)
    out, sel = run_gpu(mode, q, k, v, flags=flags, **p)
    rep = Report()
    for h in heads_to_check:
        xin = (x.q[0, h].astype(np.float64), x.k[0, h].astype(np.float64), x.v[0, h].astype(np.float64))
        ref = solattn.head_forward(mode, *xin, **p, want_out=False)
        qb = qblocks(h, ref, sel) if callable(qblocks) else qblocks
        check_head(mode, ref, sel, h, x_in=xin, d=w.d, N=w.N, report=rep, qblocks=qb,
                   out_gpu=out[0, h], dtype=x.w.dtype, **p)
    print(f"[parity] rows={rep.rows} mask_flips={rep.mask_flips} extra_flips={rep.extra_flips} "
          f"max_abs={rep.max_abs:.3e} mean_abs={rep.mean_abs:.3e}", flush=True)
    return out, sel, rep


def test_tiny_sol_fp32():
    w = workload(1)
    x = make_inputs(w)
    run_and_check(w, x, range(w.H))


@pytest.mark.parametrize("tau", [1.0, 1.3, 2.0])
def test_sol_bf16_n16k_tau_sweep(tau):
    w = workload(2, tau=tau)
    x = make_inputs(w, heads=[0, 7, 19])
    run_and_check(w, x, range(3))


def test_sla_bf16_n32k():
    w = workload(3)
    x = make_inputs(w, heads=[0, 11])
    run_and_check(w, x, range(2))


@pytest.mark.parametrize("extra", [64, 192])
def test_sol_bf16_extra_partial_tiles(extra):
    w = workload(2, extra_tokens=extra, dense_rows=(16384 - 1024, 16384))
    x = make_inputs(w, heads=[3])
    run_and_check(w, x, range(1))


def test_sol_bf16_d64_extra_tokens():
    # head dim 64: the attention kernel's 64-wide instance, with a partial extra-token tile
    # (V of the gathered tokens read row-major at d = 64) and a dense run
    w = workload(2, d=64, H=2, extra_tokens=96, dense_rows=(16384 - 512, 16384))
    x = make_inputs(w, heads=[0, 1])
    _, sel, _ = run_and_check(w, x, range(2))
    assert (sel["extra_cnt"] == 96).any()


def _sample(rng_seed, n_sparse=6, n_dense=2, n_flagged=2):
    # random sparse and dense query blocks, plus query blocks whose extra tokens were selected
    # by the exact pass after the sampled pass fell short (if any)
    def pick(h, ref, sel):
        rng = np.random.default_rng(rng_seed + h)
        sparse = np.flatnonzero(~ref["dense"])
        dn = np.flatnonzero(ref["dense"])
        out = list(rng.choice(sparse, size=min(n_sparse, sparse.size), replace=False))
        if dn.size:
            out += list(rng.choice(dn, size=min(n_dense, dn.size), replace=False))
        fl = np.flatnonzero(sel["extra_flag"][min(h, sel["extra_flag"].shape[0] - 1)] == 1)
        fl = fl[~ref["dense"][fl]]
        if fl.size:
            out += list(rng.choice(fl, size=min(n_flagged, fl.size), replace=False))
        return sorted(set(int(i) for i in out))
    return pick


def test_sol_full_options_n64k_all_heads():
    w = workload(4)
    x = make_inputs(w)
    run_and_check(w, x, [0, 13, 23], qblocks=_sample(40))


def test_sol_long_n203k_all_heads():
    # the headline length: the selection (masks, extra sets, multiplicities) of three heads in
    # full, outputs of sampled query blocks of each
    w = workload(5)
    x = make_inputs(w)
    run_and_check(w, x, [2, 11, 21], qblocks=_sample(50, n_sparse=8))


def test_sol_bf16_batch2_extra_dense_rows():
    # two batch entries in bf16: every (b, h) problem of the attention and extra-token kernels
    # is addressed through the batch stride
    w = workload(2, B=2, H=2, extra_tokens=128, dense_rows=(16384 - 1024, 16384))
    x = make_inputs(w)
    q, k, v = device_inputs(x)
    p = params(w)
    print(f"\n[parity] {w.name} B=2 H=2 bf16", flush=True)
    out, sel = run_gpu("sol", q, k, v, **p)
    for b in range(2):
        for h in range(2):
            xin = (x.q[b, h].astype(np.float64), x.k[b, h].astype(np.float64), x.v[b, h].astype(np.float64))
            ref = solattn.head_forward("sol", *xin, **p, want_out=False)
            sub = {k_: v_[b * 2 + h:b * 2 + h + 1] for k_, v_ in sel.items()}
            check_head("sol", ref, sub, 0, x_in=xin, d=w.d, N=w.N, report=Report(),
                       qblocks=_sample(70 + 2 * b, n_sparse=16, n_dense=4)(h, ref, sub),
                       out_gpu=out[b, h], dtype="bf16", **p)


def test_pairing_stride_on_a_96_wide_grid():
    # 64-token blocks straddle the rows of a 96-token-wide grid, so a block's kept set overlaps
    # most with the block three on (one grid row down), not with its neighbour: the attention
    # kernel must pick stride 3 and still compute every query block, across a dense run of
    # odd start and length
    w = workload(2, T=2, Hh=96, Ww=96, extra_tokens=64, dense_rows=(64 * 101, 64 * 110))
    x = make_inputs(w, heads=[0, 5])
    out, sel, rep = run_and_check(w, x, range(2))      # every output row against the oracle
    Mq, M = w.N // 64, w.N // 64
    for bh in range(2):
        kept = gpu_kept_mask(sel, bh, M)
        tot = []
        for s in range(1, sa.PAIR_STRIDES + 1):
            units = sa.pair_schedule(Mq, (101, 110), s)[5:]     # the 5 dense units first
            tot.append(sum(int((kept[a] | kept[b]).sum()) if b >= 0 else int(kept[a].sum())
                           for a, b in units))
        np.testing.assert_array_equal(sel["pair_plan"][bh], tot)
        assert int(np.argmin(tot)) + 1 == 3, tot


@pytest.mark.parametrize("mode,bq", [("sol", 64), ("sla", 128)])
def test_fp32_d128_both_block_sizes(mode, bq):
    # the fp32 attention kernel at d = 128 with 64- and 128-row query blocks (two tile slots
    # merged at the end, or four waves on one slot), extra tokens and dense rows, every output
    # row against the oracle
    x = random_qkv(1, 2, 4096, 128, seed=13, dtype="fp32")
    w = workload(1, d=128, mode=mode, block_q=bq, keep_percent=20.0, extra_tokens=96, sink_range=64,
                 dense_rows=(3584, 4096))
    x.w = w
    run_and_check(w, x, range(2))


@pytest.mark.parametrize("extra", [0, 64])
def test_local3d_fp32_tiny(extra):
    # 32-token rows: a block holds two rows, so the pattern is a line of blocks plus frame hops
    w = workload(1, mode="local3d", extra_tokens=extra, sink_range=128)
    x = make_inputs(w)
    _, sel, _ = run_and_check(w, x, range(w.H))
    assert (sel["kept_cnt"] < w.N // 64).all()


def test_local3d_bf16_n16k():
    # 64 x 64 frames: one block per row, so the centre / +-1 frame / +-1 row stencil, plus sinks
    w = workload(2, mode="local3d")
    x = make_inputs(w, heads=[0, 7])
    run_and_check(w, x, range(2))


def test_local3d_bf16_q128_extra_dense_rows():
    w = workload(3, mode="local3d", H=2, extra_tokens=256, dense_rows=(32768 - 1024, 32768))
    x = make_inputs(w)
    run_and_check(w, x, range(2), qblocks=_sample(60, n_sparse=48, n_dense=4))


def test_local3d_bf16_frames_straddle_blocks():
    # 45 x 80 frames (3600 tokens, not a whole number of 64-token blocks): the token-level rule
    w = workload(2, mode="local3d", H=2, T=4, Hh=45, Ww=80, extra_tokens=128, sink_range=0)
    x = make_inputs(w)
    assert w.N % 64 == 0 and (w.Hh * w.Ww) % 64 != 0
    run_and_check(w, x, range(2))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("case", ["tau_neg_inf", "sla_all", "sink_all"])
def test_dense_limits(dtype, case):
    x = random_qkv(1, 2, 2048, 64, seed=5, dtype=dtype)
    q, k, v = device_inputs(x)
    if case == "tau_neg_inf":
        out, sel = run_gpu("sol", q, k, v, block_q=64, block_k=64, tau=-math.inf, extra_tokens=128)
    elif case == "sla_all":
        out, sel = run_gpu("sla", q, k, v, block_q=128, block_k=64, keep_percent=100.0)
    else:
        out, sel = run_gpu("sol", q, k, v, block_q=64, block_k=64, tau=1.3, sink_range=2048,
                           extra_tokens=64)
    ref = np.stack([dense.dense_attention(x.q[0, h], x.k[0, h], x.v[0, h]) for h in range(2)])
    err = np.abs(out[0] - ref)
    tol = (2e-2, 2e-3) if dtype == "bf16" else (1e-4, 1e-4)
    assert err.max() <= tol[0] and err.mean() <= tol[1], (err.max(), err.mean())


def test_few_candidates_for_extra_tokens():
    # tau = -2 keeps almost every block: fewer candidate tokens than extra_tokens.  Some query
    # blocks then have no extra token while their neighbour has some, the case where the
    # attention kernel's extra-token loop starts with the second block of a pair.
    w = workload(1, dtype="bf16", d=128, H=2, tau=-2.0, extra_tokens=256)
    x = make_inputs(w)
    _, sel, _ = run_and_check(w, x, range(2))
    cnt = sel["extra_cnt"].reshape(2, -1)
    assert (cnt < 256).any()
    Mq = w.N // 64
    starts_with_second = 0
    for bh in range(2):
        stride = int(np.argmin(sel["pair_plan"][bh])) + 1
        for a, b in sa.pair_schedule(Mq, (0, 0), stride):
            starts_with_second += int(b >= 0 and cnt[bh, a] == 0 and cnt[bh, b] > 0)
    assert starts_with_second > 0


@pytest.mark.parametrize("flags", [0, sa.FLAG_EXACT_EXTRA])
def test_extra_selection_exact_pass(flags):
    # The first 32 keys of every key block score far above the rest, a distribution far from the
    # sampled pass's assumptions; with SOLATTN_FLAG_EXACT_EXTRA every query block takes the exact
    # pass (flagged in extra_flag).  Either way the selection must be the oracle's.
    B, H, N, d = 1, 2, 4096, 128
    rng = np.random.default_rng([11, 3])
    u = rng.standard_normal(d).astype(np.float32)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((B, H, N, d), dtype=np.float32) + 2.0 * u
    k = rng.standard_normal((B, H, N, d), dtype=np.float32)
    k[:, :, (np.arange(N) % 64) < 32, :] += 5.0 * u
    v = rng.standard_normal((B, H, N, d), dtype=np.float32)
    bits = [bf16_round(a) for a in (q, k, v)]
    w = Workload(0, "repair", B=B, H=H, T=1, Hh=1, Ww=N, d=d, dtype="bf16", mode="sol",
                 block_q=64, block_k=64, tau=1.3, extra_tokens=256, sink_range=128)
    x = Inputs(w, tuple(range(H)), *[bf16_to_f32(b) for b in bits], *bits)
    _, sel, rep = run_and_check(w, x, range(H), flags=flags)
    assert rep.extra_flips == 0
    if flags:
        assert (sel["extra_flag"] == 1).all(), sel["extra_flag"]
    assert (sel["extra_cnt"] == 256).all()


def test_extra_selection_overflow_goes_to_exact_pass():
    # The opposite failure of the seed: every key block the seed's sample reads scores far below
    # the rest, so the seed admits nearly every token and the sampled pass's lists would
    # overflow.  Such query blocks must be flagged and selected again by the exact pass; the
    # selection must still be the oracle's.  The sample here is the first 32 tokens of key block
    # 8s + (37 s mod 8) for run s of 64 (N = 32768: 512 key blocks, 64 runs); whole blocks are
    # lowered so the construction does not depend on the run's half.
    B, H, N, d = 1, 2, 32768, 128
    M = N // 64
    runs = 64
    sampled = {(s * M) // runs + (s * 37) % (M // runs) for s in range(runs)}
    rng = np.random.default_rng([11, 5])
    u = rng.standard_normal(d).astype(np.float32)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((B, H, N, d), dtype=np.float32) + 2.0 * u
    k = rng.standard_normal((B, H, N, d), dtype=np.float32)
    low = np.zeros(N, dtype=bool)
    for j in sampled:
        low[64 * j:64 * j + 64] = True
    k[:, :, ~low, :] += 3.0 * u
    v = rng.standard_normal((B, H, N, d), dtype=np.float32)
    bits = [bf16_round(a) for a in (q, k, v)]
    w = Workload(0, "overflow", B=B, H=H, T=1, Hh=1, Ww=N, d=d, dtype="bf16", mode="sol",
                 block_q=64, block_k=64, tau=1.3, extra_tokens=256, sink_range=64)
    x = Inputs(w, tuple(range(H)), *[bf16_to_f32(b) for b in bits], *bits)
    _, sel, rep = run_and_check(w, x, range(H), qblocks=[0, 1, 63, 200, 257, 400, 511])
    assert rep.extra_flips == 0
    flagged = int((sel["extra_flag"] == 1).sum())
    print(f"[overflow] query blocks sent to the exact pass: {flagged} of {sel['extra_flag'].size}", flush=True)
    assert flagged > 0
    assert (sel["extra_cnt"] == 256).all()


def test_seeds_do_not_depend_on_the_sample_split():
    # The seeds' pass deals a group's sampled tiles to 1, 2 or 4 workgroups (about 768
    # workgroups in all) and merges their best-of lists; the merged lists equal one workgroup's
    # over all tiles, so each head's seeds must be bit for bit the same whether the head runs
    # with 1, 191 or 383 other heads (N = 16384: 4, 2 and 1 splits), and so must its extra-token
    # sets and output (the selection is exact whatever the seeds).
    N, d = 16384, 128
    x = random_qkv(1, 2, N, d, seed=21, dtype="bf16")
    q2, k2, v2 = device_inputs(x)
    kw = dict(tau=1.3, block_q=64, block_k=64, sink_range=256, extra_tokens=256,
              dense_rows=(N - 1024, N), return_workspace=True)
    seeds, outs, extras = [], [], []
    for H in (2, 192, 384):
        q, k, v = (t.repeat(1, H // 2, 1, 1).contiguous() for t in (q2, k2, v2))
        print(f"\n[seed split] H={H}", flush=True)
        out, ws = sa.sol_attn(q, k, v, **kw)
        torch.cuda.synchronize()
        L = sa.workspace_layout(sa.MODE_SOL, sa.BF16, 1, H, N, d, 64, 64)
        seed = ws[L.extra_seed:L.extra_seed + 4 * H * L.Mq].view(torch.int32).view(H, L.Mq)
        views = sa.selection_views(ws, sa.MODE_SOL, sa.BF16, 1, H, N, d, 64, 64)
        seeds.append(seed[:2].cpu())
        outs.append(out[:, :2].cpu())
        extras.append((views["extra_cnt"][:2].cpu(), views["extra_idx"][:2].cpu(),
                       views["extra_flag"][:2].cpu()))
        del q, k, v, out, ws
        torch.cuda.empty_cache()
    sparse = seeds[0][:, :(N - 1024) // 64]
    assert (sparse != 0).float().mean() > 0.99        # a seed for (nearly) every sparse block
    for j in (1, 2):
        assert torch.equal(seeds[j], seeds[0])
        assert torch.equal(outs[j].view(torch.int16), outs[0].view(torch.int16))
        # (which query blocks the exact pass takes may differ: the token slices of the sampled
        # pass, and so its lists' capacity per token, depend on the head count)
        cnt, idx, _ = extras[j]
        assert torch.equal(cnt, extras[0][0])
        # the lists' entries past each query block's count are not written
        live = torch.arange(idx.shape[-1])[None, None, :] < cnt[..., None]
        assert torch.equal(torch.where(live, idx, 0), torch.where(live, extras[0][1], 0))


def test_block_constant_keys_and_values_tie_breaks_and_dense_limit():
    # Every key block holds one key vector and one value vector 64 times.  The extra-token
    # scores of a block's tokens are then equal bit for bit, so a cut inside a block (96 extra
    # tokens: one and a half blocks' worth) must take its lowest-numbered tokens, as the
    # oracle's (score desc, token asc) order says; and a skipped block's centroid term is
    # exactly the sum over its tokens not taken as extra tokens, so the sparse output must
    # equal dense attention on every row.
    B, H, N, d = 1, 2, 8192, 128
    rng = np.random.default_rng([31, 2])
    q = rng.standard_normal((B, H, N, d), dtype=np.float32)
    kb = rng.standard_normal((B, H, N // 64, 1, d), dtype=np.float32)
    k = np.broadcast_to(kb, (B, H, N // 64, 64, d)).reshape(B, H, N, d).copy()
    vb = rng.standard_normal((B, H, N // 64, 1, d), dtype=np.float32)
    v = np.broadcast_to(vb, (B, H, N // 64, 64, d)).reshape(B, H, N, d).copy()
    bits = [bf16_round(a) for a in (q, k, v)]
    w = Workload(0, "block-constant-keys", B=B, H=H, T=1, Hh=1, Ww=N, d=d, dtype="bf16", mode="sol",
                 block_q=64, block_k=64, tau=1.3, extra_tokens=96, sink_range=64)
    x = Inputs(w, tuple(range(H)), *[bf16_to_f32(b) for b in bits], *bits)
    out, sel, rep = run_and_check(w, x, range(H), qblocks=[0, 1, 37, 127])
    assert rep.mask_flips == 0 and rep.extra_flips == 0
    # the cut falls inside a block for (nearly) every query block: its lowest tokens were taken
    partial = 0
    for bh in range(H):
        for i in range(N // 64):
            idx = np.sort(sel["extra_idx"][bh, i, :sel["extra_cnt"][bh, i]])
            blocks, counts = np.unique(idx // 64, return_counts=True)
            for j, c in zip(blocks, counts):
                if c < 64:
                    partial += 1
                    assert (idx[idx // 64 == j] == 64 * j + np.arange(c)).all()
    assert partial > 0
    ref = np.stack([dense.dense_attention(x.q[0, h], x.k[0, h], x.v[0, h]) for h in range(H)])
    err = np.abs(out[0] - ref)
    print(f"[block-constant keys] dense limit: max {err.max():.3e} mean {err.mean():.3e}; "
          f"partial blocks {partial}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_batch_and_dense_rows_fp32():
    x = random_qkv(2, 2, 4096, 64, seed=9, dtype="fp32")
    w = workload(1, B=2, dense_rows=(3072, 4096), extra_tokens=64, sink_range=100)
    x.w = w
    q, k, v = device_inputs(x)
    p = params(w)
    out, sel = run_gpu("sol", q, k, v, **p)
    for b in range(2):
        for h in range(2):
            xin = (x.q[b, h].astype(np.float64), x.k[b, h].astype(np.float64), x.v[b, h].astype(np.float64))
            ref = solattn.head_forward("sol", *xin, **p, want_out=False)
            sub = {k_: v_[b * 2 + h:b * 2 + h + 1] for k_, v_ in sel.items()}
            check_head("sol", ref, sub, 0, x_in=xin, d=64, N=4096, report=Report(),
                       out_gpu=out[b, h], dtype="fp32", **p)


def test_deterministic_and_strided_views():
    w = workload(2, H=2, extra_tokens=128, dense_rows=(15360, 16384))
    x = make_inputs(w)
    q, k, v = device_inputs(x)
    p = params(w)
    o1, _ = run_gpu("sol", q, k, v, **p)
    o2, _ = run_gpu("sol", q, k, v, **p)
    assert np.array_equal(o1, o2)
    # the call without the kept lists (the bench's call) gives the same output, bit for bit
    o4 = sa.sol_attn(q, k, v, tau=p["tau"], block_q=64, block_k=64, sink_range=p["sink_range"],
                     extra_tokens=p["extra_tokens"], dense_rows=p["dense_rows"])
    torch.cuda.synchronize()
    assert np.array_equal(o1, o4.float().cpu().numpy().astype(np.float64))
    # the same tensors as views of a [B, N, H, d] buffer
    qs, ks, vs = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
    assert not qs.is_contiguous()
    o3, _ = run_gpu("sol", qs, ks, vs, **p)
    assert np.array_equal(o1, o3)


def test_library_errors_raise():
    x = random_qkv(1, 1, 4096, 64, seed=1, dtype="bf16")
    q, k, v = device_inputs(x)
    with pytest.raises(sa.SolattnError) as e:
        sa.sol_attn(q, k, v, tau=float("nan"))
    assert e.value.status == sa.EINVAL
    with pytest.raises(sa.SolattnError) as e:
        sa.sol_attn(q, k, v, block_k=32)
    assert e.value.status == sa.ENOTSUP
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(sa.SolattnError) as e:
        sa.sol_attn(q, k, v, workspace=ws)
    assert e.value.status == sa.EWORKSPACE


def _host_counters(sel, mode, B, H, Mq, M, bq, bk, N, dense_rows, extra_tokens, tau):
    kept = sel["kept_cnt"].astype(np.int64)
    extra = sel["extra_cnt"].astype(np.int64)
    dense = np.zeros(Mq, dtype=bool)
    dense[dense_rows[0] // bq:dense_rows[1] // bq] = True
    sp = ~dense
    c = np.zeros(8, dtype=np.int64)
    c[0] = kept[:, sp].sum()
    c[1] = B * H * sp.sum()
    c[2] = (bq * (kept[:, sp] * bk + extra[:, sp])).sum() + B * H * dense.sum() * bq * N
    if mode == "sol":
        c[3] = bq * (sel["mult"][:, sp, :M] > 0).sum()
    c[4] = extra[:, sp].sum()
    if extra_tokens > 0 and tau != -math.inf:
        c[6] = (sel["extra_flag"][:, sp] == 1).sum()
    return c


@pytest.mark.parametrize("mode", ["sol", "sla", "local3d"])
def test_call_counters(mode):
    # the per-call counters against recounts from the call's own selection lists
    w = workload(2, mode=mode, H=2, extra_tokens=128, dense_rows=(16384 - 1024, 16384),
                 block_q=128 if mode == "sla" else 64, keep_percent=15.0)
    x = make_inputs(w)
    q, k, v = device_inputs(x)
    stats = torch.zeros(sa.NSTATS, dtype=torch.int64, device="cuda")
    print(f"\n[counters] mode={mode} N={w.N}", flush=True)
    kw = dict(block_q=w.block_q, block_k=64, sink_range=w.sink_range, extra_tokens=w.extra_tokens,
              dense_rows=w.dense_rows, return_workspace=True, stats=stats, flags=sa.FLAG_KEEP_SELECTION)
    if mode == "sol":
        out, ws = sa.sol_attn(q, k, v, tau=w.tau, **kw)
    elif mode == "sla":
        out, ws = sa.sla_attn(q, k, v, keep_percent=w.keep_percent, **kw)
    else:
        out, ws = sa.local3d_attn(q, k, v, grid=(w.T, w.Hh, w.Ww), **kw)
    torch.cuda.synchronize()
    m = {"sol": sa.MODE_SOL, "sla": sa.MODE_SLA, "local3d": sa.MODE_LOCAL3D}[mode]
    views = sa.selection_views(ws, m, sa.BF16, 1, w.H, w.N, w.d, w.block_q, 64)
    sel = {k_: v_.cpu().numpy() for k_, v_ in views.items()}
    got = stats.cpu().numpy()
    Mq, M = w.N // w.block_q, w.N // 64
    ref = _host_counters(sel, mode, 1, w.H, Mq, M, w.block_q, 64, w.N, w.dense_rows,
                         w.extra_tokens, w.tau)
    print(f"[counters] {dict(zip(sa.STAT_NAMES, got.tolist()))}", flush=True)
    for idx in (0, 1, 2, 3, 4, 6):
        assert got[idx] == ref[idx], (sa.STAT_NAMES[idx], got[idx], ref[idx])
    assert got[7] == -1
    if mode == "sol":
        # near-threshold blocks, recounted in fp64 from the call's scores (a diagnostic: the two
        # may differ on a block that sits exactly at the band's edge)
        s_ = sel["scores"].astype(np.float64)
        dense = np.zeros(Mq, dtype=bool)
        dense[w.dense_rows[0] // 64:w.dense_rows[1] // 64] = True
        s_ = s_[:, ~dense]
        mu = s_.mean(axis=2, keepdims=True)
        sd = s_.std(axis=2, keepdims=True)
        near = int((np.abs(s_ - (mu + w.tau * sd)) <= 1e-4 * sd).sum())
        assert abs(int(got[5]) - near) <= max(2, near // 10), (got[5], near)
    else:
        assert got[5] == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_finite_check_counts_nonfinite_values(dtype):
    x = random_qkv(1, 2, 2048, 64, seed=9, dtype=dtype)
    q, k, v = device_inputs(x)
    stats = torch.zeros(sa.NSTATS, dtype=torch.int64, device="cuda")
    print(f"\n[finite] dtype={dtype} clean", flush=True)
    sa.sol_attn(q, k, v, tau=1.3, stats=stats, flags=sa.FLAG_CHECK_FINITE)
    torch.cuda.synchronize()
    assert stats[7].item() == 0
    q[0, 0, 5, 3] = float("inf")
    k[0, 1, 100, 7] = float("nan")
    v[0, 1, 2000, 0] = float("-inf")
    print(f"[finite] dtype={dtype} with three non-finite inputs", flush=True)
    out = sa.sol_attn(q, k, v, tau=1.3, stats=stats, flags=sa.FLAG_CHECK_FINITE)
    torch.cuda.synchronize()
    n_out = int((~torch.isfinite(out.float())).sum().item())
    assert n_out > 0
    assert stats[7].item() == 3 + n_out


def test_finite_check_counts_only_the_window_rows():
    # a query-row window leaves the other rows of out untouched; filled with NaN there, they
    # must not be counted: the count is the non-finite inputs plus the window's outputs
    x = random_qkv(1, 2, 2048, 64, seed=9, dtype="bf16")
    q, k, v = device_inputs(x)
    out = torch.full_like(q, float("nan"))
    stats = torch.zeros(sa.NSTATS, dtype=torch.int64, device="cuda")
    print("\n[finite] window rows 512..1024, clean inputs", flush=True)
    sa.sol_attn(q, k, v, tau=1.3, out=out, q_rows=(512, 1024), stats=stats, flags=sa.FLAG_CHECK_FINITE)
    torch.cuda.synchronize()
    assert torch.isfinite(out[:, :, 512:1024].float()).all()
    assert torch.isnan(out[:, :, :512].float()).all() and torch.isnan(out[:, :, 1024:].float()).all()
    assert stats[7].item() == 0
    k[0, 0, 3, 1] = float("nan")            # a sink-range key: every row of head 0 attends it
    stats.zero_()
    print("[finite] window rows 512..1024, one NaN key", flush=True)
    sa.sol_attn(q, k, v, tau=1.3, sink_range=64, out=out, q_rows=(512, 1024), stats=stats,
                flags=sa.FLAG_CHECK_FINITE)
    torch.cuda.synchronize()
    n_win = int((~torch.isfinite(out[:, :, 512:1024].float())).sum().item())
    assert n_win > 0
    assert stats[7].item() == 1 + n_win


@pytest.mark.parametrize("mode", ["sol", "sla", "local3d"])
def test_fp8qk_flavour(mode):
    # the fp8-QK flavour: the selection must be the bf16 path's, bit for bit, and the output
    # within the bf16 tolerance of the fp8-QK oracle run on the GPU's selection; the oracle pools
    # the keys itself in fp64 and quantises them (no GPU intermediate enters the expected output)
    from oracle import fp8
    bq = 128 if mode == "sla" else 64
    w = workload(2, mode=mode, H=2, extra_tokens=128, dense_rows=(16384 - 1024, 16384),
                 block_q=bq, keep_percent=15.0)
    x = make_inputs(w)
    q, k, v = device_inputs(x)
    call = {"sol": sa.sol_attn, "sla": sa.sla_attn, "local3d": sa.local3d_attn}[mode]
    kw = dict(block_q=bq, block_k=64, sink_range=w.sink_range, extra_tokens=w.extra_tokens,
              dense_rows=w.dense_rows, return_workspace=True, flags=sa.FLAG_KEEP_SELECTION)
    if mode == "sol":
        kw["tau"] = w.tau
    elif mode == "sla":
        kw["keep_percent"] = w.keep_percent
    else:
        kw["grid"] = (w.T, w.Hh, w.Ww)
    print(f"\n[fp8qk] {mode}: bf16 and fp8-QK calls", flush=True)
    out_b, ws_b = call(q, k, v, **kw)
    out_8, ws_8 = call(q, k, v, qk_fp8=True, **kw)
    torch.cuda.synchronize()
    m = {"sol": sa.MODE_SOL, "sla": sa.MODE_SLA, "local3d": sa.MODE_LOCAL3D}[mode]
    vb = sa.selection_views(ws_b, m, sa.BF16, 1, w.H, w.N, w.d, bq, 64)
    v8 = sa.selection_views(ws_8, m, sa.BF16_FP8QK, 1, w.H, w.N, w.d, bq, 64)
    from parity import gpu_extra_sets, gpu_kept_mask
    for name in ("kept_cnt", "extra_cnt", "mult"):
        assert torch.equal(vb[name], v8[name]), name
    sel = {k_: v_.cpu().numpy() for k_, v_ in v8.items()}
    selb = {k_: v_.cpu().numpy() for k_, v_ in vb.items()}
    for h in range(w.H):       # the lists' valid prefixes (the rest of each row is scratch)
        np.testing.assert_array_equal(gpu_kept_mask(sel, h, w.N // 64), gpu_kept_mask(selb, h, w.N // 64))
        for a_, b_ in zip(gpu_extra_sets(sel, h), gpu_extra_sets(selb, h)):
            np.testing.assert_array_equal(a_, b_)
    out8 = out_8.float().cpu().numpy().astype(np.float64)
    worst = (0.0, 0.0)
    code_flips = 0
    for h in range(w.H):
        xin = (x.q[0, h].astype(np.float64), x.k[0, h].astype(np.float64), x.v[0, h].astype(np.float64))
        M = w.N // 64
        gsel = (gpu_kept_mask(sel, h, M), gpu_extra_sets(sel, h))
        ref = fp8.head_forward_fp8qk(mode, *xin, block_q=bq,
                                     block_k=64, selection=gsel, dense_rows=w.dense_rows)
        # pooled-key E4M3 codes: the GPU quantises its fp32 block means, the oracle its fp64
        # ones; a code may differ only where the scaled fp64 mean lies within the fp32 mean's
        # error of a rounding boundary (counted, like the selection's near-threshold blocks)
        kb64 = solattn.pool(xin[1], 64)
        kq64, e64 = fp8.quantize_rows(kb64)
        kq32, e32 = fp8.quantize_rows(sel["kbar"][h].astype(np.float64))
        diff = kq64 != kq32
        if diff.any():
            r, c = np.nonzero(diff)
            y = kb64[r, c] / 2.0 ** e64[r]                  # scaled fp64 means at the flips
            lo = np.abs(y)
            ex = np.floor(np.log2(np.maximum(lo, 2.0 ** -6)))
            step = 2.0 ** (ex - 3)
            to_mid = np.abs(lo / step - np.floor(lo / step) - 0.5) * step
            err32 = 64 * 2.0 ** -24 * np.abs(xin[1]).max() / 2.0 ** e64[r]
            assert (np.equal(e64[r], e32[r]) & (to_mid <= err32)).all(), "pooled-key code flip outside the band"
            code_flips += int(diff.sum())
        err = np.abs(out8[0, h] - ref)
        worst = (max(worst[0], float(err.max())), max(worst[1], float(err.mean())))
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, (h, err.max(), err.mean())
    # not value-identical to the bf16 path, but close to it
    d = (out_8.float() - out_b.float()).abs()
    print(f"[fp8qk] {mode}: pooled-key code flips {code_flips}; vs oracle max {worst[0]:.3e} "
          f"mean {worst[1]:.3e}; vs bf16 path "
          f"max {d.max().item():.3e} mean {d.mean().item():.3e}", flush=True)
    assert d.max().item() > 0 and d.mean().item() < 0.05


def test_fp8qk_chunked_equals_whole_call():
    from block_sparse_attention_scores_amd.chunked import chunked_attention
    w = workload(2, H=2, extra_tokens=128, dense_rows=(16384 - 1024, 16384))
    x = make_inputs(w)
    q, k, v = device_inputs(x)
    pr = dict(tau=w.tau, sink_range=w.sink_range, extra_tokens=w.extra_tokens,
              dense_rows=w.dense_rows, qk_fp8=True)
    print("\n[fp8qk] chunked vs whole", flush=True)
    ref = sa.sol_attn(q, k, v, **pr)
    got, rep = chunked_attention("sol", q, k, v, chunk_rows=4096, **pr)
    torch.cuda.synchronize()
    assert len(rep.chunks) == 4
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
