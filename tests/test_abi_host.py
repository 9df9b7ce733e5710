"""The C ABI on the host: the library loads, exports every symbol include/solattn.h declares,
and validates arguments before any launch (no GPU needed: every call here fails validation or
only plans the workspace)."""
import ctypes
import json
import math
import os

import pytest

import block_sparse_attention_scores_amd as sa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")

# fake, non-overlapping, 256-aligned "device" addresses: never dereferenced
QP, KP, VP, OP = 1 << 32, 2 << 32, 3 << 32, 4 << 32


def check(mode=0, q=QP, k=KP, v=VP, o=OP, B=1, H=2, N=4096, d=64, tau=1.3, keep=10.0, bq=64, bk=64,
          sink=0, extra=0, opts=None):
    return sa.lib().solattn_check_args(mode, q, k, v, o, B, H, N, d, tau, keep, bq, bk, sink, extra,
                                       ctypes.byref(opts) if opts is not None else None)


def test_exports_every_declared_symbol():
    L = sa.lib()
    names = sa.header_functions()
    # the calls of the boundary's specification, by name
    assert {"sol_attn_fwd", "sla_attn_fwd", "solattn_workspace_bytes", "solattn_status_string",
            "solattn_last_error_detail", "solattn_selection_view"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_last_error_detail_names_the_argument():
    assert check(extra=300) == sa.EINVAL
    detail = sa.lib().solattn_last_error_detail().decode()
    assert "extra_tokens" in detail and detail == sa.lib().solattn_last_error().decode()
    assert check() == sa.OK
    assert sa.lib().solattn_last_error_detail().decode() == ""


def test_keep_selection_flag_is_accepted():
    assert check(opts=sa.make_opts(flags=sa.FLAG_KEEP_SELECTION)) == sa.OK
    assert check(opts=sa.make_opts(flags=sa.FLAG_KEEP_SELECTION | sa.FLAG_EXACT_EXTRA)) == sa.OK
    assert check(opts=sa.make_opts(flags=8)) == sa.EINVAL


def test_workspace_bytes_any_dtype_and_extra_tokens():
    # the specification's call: (mode, B, H, N, d, block_q, block_k, extra_tokens), enough for
    # any dtype; the candidate lists of the extra-token selection only when extra_tokens > 0
    for ex in (0, 64, 256):
        any_ = sa.workspace_bytes_any(0, 1, 4, 16384, 128, 64, 64, ex)
        per = [sa.workspace_bytes(0, dt, 1, 4, 16384, 128, 64, 64, None, ex)
               for dt in (sa.BF16, sa.FP32, sa.BF16_FP8QK)]
        assert any_ == max(per) > 0
    assert sa.workspace_bytes(0, sa.BF16, 1, 4, 16384, 128, 64, 64, None, 0) < \
        sa.workspace_bytes(0, sa.BF16, 1, 4, 16384, 128, 64, 64, None, 64)
    assert sa.workspace_bytes_any(0, 1, 4, 16384, 128, 64, 64, 257) == 0
    assert sa.workspace_bytes_any(0, 1, 4, 16384, 128, 64, 64, -1) == 0


def test_selection_view_points_into_the_workspace():
    base = 1 << 40
    o = sa.make_opts(workspace=base, workspace_bytes=1 << 30)
    v = sa.Selection()
    assert sa.lib().solattn_selection_view(ctypes.byref(o), 0, 1, 2, 4096, 64, 64, ctypes.byref(v)) == sa.OK
    L = sa.workspace_layout(0, sa.BF16, 1, 2, 4096, 128, 64, 64)
    assert (v.Mq, v.M, v.Mpad) == (64, 64, 64)
    for name in ("kept_cnt", "kept_bm", "kept_idx", "mult", "extra_cnt", "extra_idx", "extra_flag",
                 "scores"):
        assert getattr(v, name) == base + getattr(L, name), name
    # the same offsets for every dtype, d and extra_tokens
    for dt, d, ex in ((sa.FP32, 64, 0), (sa.BF16_FP8QK, 128, 256), (sa.BF16, 64, 64)):
        L2 = sa.workspace_layout(0, dt, 1, 2, 4096, d, 64, 64, extra_tokens=ex)
        assert (L2.kept_cnt, L2.kept_bm, L2.extra_idx, L2.scores) == (L.kept_cnt, L.kept_bm, L.extra_idx, L.scores)
    # a window: its query blocks only
    o = sa.make_opts(workspace=base, workspace_bytes=1 << 30, q_rows=(1024, 2048))
    assert sa.lib().solattn_selection_view(ctypes.byref(o), 0, 1, 2, 4096, 64, 64, ctypes.byref(v)) == sa.OK
    assert v.Mq == 16
    # no workspace, or a bad window: an error naming it
    o = sa.make_opts()
    assert sa.lib().solattn_selection_view(ctypes.byref(o), 0, 1, 2, 4096, 64, 64, ctypes.byref(v)) == sa.EINVAL
    assert "workspace" in sa.last_error()
    o = sa.make_opts(workspace=base, workspace_bytes=1 << 30, q_rows=(2048, 1024))
    assert sa.lib().solattn_selection_view(ctypes.byref(o), 0, 1, 2, 4096, 64, 64, ctypes.byref(v)) == sa.EINVAL


def test_valid_arguments_pass():
    assert check() == sa.OK
    assert check(mode=1, bq=128, keep=15.0) == sa.OK
    assert check(d=128, extra=256, sink=1024, tau=-math.inf) == sa.OK


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(o=0), dict(B=0), dict(H=0), dict(N=0), dict(d=0),
    dict(tau=float("nan")), dict(mode=1, keep=0.0), dict(mode=1, keep=100.5),
    dict(mode=1, keep=float("nan")), dict(extra=-1), dict(extra=257), dict(sink=-1),
    dict(sink=4097), dict(mode=7), dict(bq=0), dict(o=QP + 64),
])
def test_invalid_arguments(kw):
    assert check(**kw) == sa.EINVAL
    assert sa.last_error() != ""


@pytest.mark.parametrize("kw", [
    dict(d=96), dict(bk=32), dict(bq=32), dict(N=4000), dict(q=QP + 8), dict(N=64 * 4097),
])
def test_unsupported_shapes(kw):
    assert check(**kw) == sa.ENOTSUP


def test_dense_row_and_stride_validation():
    o = sa.make_opts(dense_rows=(4096 - 1024, 4096))
    assert check(opts=o) == sa.OK
    assert check(opts=sa.make_opts(dense_rows=(100, 50))) == sa.EINVAL
    assert check(opts=sa.make_opts(dense_rows=(0, 5000))) == sa.EINVAL
    assert check(opts=sa.make_opts(dense_rows=(32, 4096))) == sa.ENOTSUP
    bad = sa.make_opts()
    bad.struct_size = 8
    assert check(opts=bad) == sa.EINVAL
    assert check(opts=sa.make_opts(dtype=5)) == sa.EINVAL
    # out rows overlapping each other
    st = [(0, 0, 0)] * 3 + [(2 * 4096 * 64, 4096 * 64, 32)]
    assert check(opts=sa.make_opts(strides=st)) == sa.EINVAL
    # a strided q view ([B, N, H, d] memory) is fine
    st = [(4096 * 2 * 64, 64, 2 * 64)] + [(0, 0, 0)] * 3
    assert check(opts=sa.make_opts(strides=st)) == sa.OK


def test_forward_calls_fail_before_launching():
    L = sa.lib()
    rc = L.sol_attn_fwd(QP, KP, VP, QP, 1, 2, 4096, 64, 1.3, 64, 64, 0, 0, None)
    assert rc == sa.EINVAL and "overlaps" in sa.last_error()
    rc = L.sla_attn_fwd(QP, KP, VP, OP, 1, 2, 4096, 64, 128, 64, 0, 0, -3.0, None)
    assert rc == sa.EINVAL and "keep_percent" in sa.last_error()


def check3(grid=(4, 16, 64), N=4096, fp32=False, **kw):
    a = dict(q=QP, k=KP, v=VP, o=OP, B=1, H=2, d=64, bq=64, bk=64, sink=0, extra=0)
    a.update(kw)
    o = sa.make_opts(dtype=sa.FP32) if fp32 else None
    return sa.lib().local3d_check_args(a["q"], a["k"], a["v"], a["o"], a["B"], a["H"], N, a["d"],
                                       *grid, a["bq"], a["bk"], a["sink"], a["extra"],
                                       ctypes.byref(o) if o is not None else None)


def test_local3d_validation():
    assert check3() == sa.OK
    assert check3(grid=(1, 1, 4096)) == sa.OK
    assert check3(grid=(3, 5, 448), N=105 * 64) == sa.OK          # any grid that holds N tokens
    assert check3(grid=(4, 45, 80), N=14400) == sa.OK             # frames that straddle blocks
    assert check3(bq=128, extra=256, sink=512) == sa.OK
    for g in [(0, 64, 64), (4, -1, 64), (4, 16, 0), (4, 16, 65), (2, 16, 64)]:
        assert check3(grid=g) == sa.EINVAL, g
        assert "grid" in sa.last_error()
    assert check3(grid=(1 << 16, 1 << 16, 1 << 16)) == sa.EINVAL   # product overflows int32
    assert check3(extra=257) == sa.EINVAL
    assert check3(bk=32) == sa.ENOTSUP
    # the neighbourhood bitmap bounds the key blocks (bf16 is bounded earlier)
    N = 64 * 65537
    assert check3(grid=(65537, 1, 64), N=N, fp32=True) == sa.ENOTSUP
    assert "local 3-D" in sa.last_error()
    assert check3(grid=(65536, 1, 64), N=N - 64, fp32=True) == sa.OK
    # the sol/sla check refuses the mode that needs a grid
    assert check(mode=sa.MODE_LOCAL3D) == sa.EINVAL
    L = sa.lib()
    rc = L.local3d_attn_fwd(QP, KP, VP, OP, 1, 2, 4096, 64, 4, 16, 63, 64, 64, 0, 0, None)
    assert rc == sa.EINVAL and "grid" in sa.last_error()


def test_stats_and_flag_validation():
    assert check(opts=sa.make_opts(stats=1 << 33)) == sa.OK
    assert check(opts=sa.make_opts(stats=1 << 33, flags=sa.FLAG_CHECK_FINITE)) == sa.OK
    assert check(opts=sa.make_opts(flags=sa.FLAG_CHECK_FINITE)) == sa.EINVAL
    assert "stats" in sa.last_error()
    assert check(opts=sa.make_opts(stats=(1 << 33) + 4)) == sa.EINVAL
    assert check(opts=sa.make_opts(flags=8)) == sa.EINVAL
    assert "flags" in sa.last_error()
    assert check(opts=sa.make_opts(flags=sa.FLAG_EXACT_EXTRA | sa.FLAG_CHECK_FINITE, stats=1 << 33)) == sa.OK


def test_query_row_window_validation_and_layout():
    assert check(opts=sa.make_opts(q_rows=(1024, 2048))) == sa.OK
    assert check(opts=sa.make_opts(q_rows=(0, 4096))) == sa.OK
    for rows in [(2048, 1024), (-64, 64), (0, 4160), (1024, 1024)]:
        assert check(opts=sa.make_opts(q_rows=rows)) == sa.EINVAL, rows
        assert "window" in sa.last_error()
    assert check(opts=sa.make_opts(q_rows=(32, 1024))) == sa.ENOTSUP
    assert check(mode=1, bq=128, opts=sa.make_opts(q_rows=(64, 1024))) == sa.ENOTSUP
    # the window's workspace: query-block arrays shrink with the window, key arrays do not
    full = sa.workspace_layout(0, sa.BF16, 1, 2, 4096, 64, 64, 64)
    part = sa.workspace_layout(0, sa.BF16, 1, 2, 4096, 64, 64, 64, q_rows=1024)
    assert (full.Mq, part.Mq, full.M, part.M) == (64, 16, 64, 64)
    assert part.total < full.total
    assert part.kbar - part.qbar == 2 * 16 * 64 * 4
    assert sa.workspace_bytes(0, sa.BF16, 1, 2, 4096, 64, 64, 64, 4096) == full.total
    assert sa.workspace_bytes(0, sa.BF16, 1, 2, 4096, 64, 64, 64, 0) == 0
    assert sa.workspace_bytes(0, sa.BF16, 1, 2, 4096, 64, 64, 64, 4097) == 0


def test_fp8qk_layout():
    assert check(opts=sa.make_opts(dtype=sa.BF16_FP8QK)) == sa.OK
    assert check(opts=sa.make_opts(dtype=3)) == sa.EINVAL
    bf = sa.workspace_layout(0, sa.BF16, 1, 2, 4096, 128, 64, 64)
    f8 = sa.workspace_layout(0, sa.BF16_FP8QK, 1, 2, 4096, 128, 64, 64)
    assert bf.k8 == 0 and bf.kb8 == 0
    # the bf16 buffers are where they were; the E4M3 tiles follow them
    assert (f8.qbar, f8.extra_flag, f8.v_t) == (bf.qbar, bf.extra_flag, bf.v_t)
    tb = 64 * 128 + 64
    v_t_bytes = 2 * 64 * 128 * 64 * 2
    assert f8.k8 >= bf.v_t + v_t_bytes and f8.kb8 - f8.k8 >= 2 * 64 * tb
    assert f8.total - f8.kb8 >= 2 * 1 * tb


def test_pair_plan_layout():
    # the pairing sums exist for the 16-bit kernel with 64-row query blocks only
    # (ahead of the extra-token scratch, so that its offset does not depend on extra_tokens)
    bf = sa.workspace_layout(0, sa.BF16, 1, 2, 4096, 128, 64, 64)
    assert bf.pair_plan > bf.vbar and bf.extra_buf - bf.pair_plan >= 2 * sa.PAIR_STRIDES * 8
    assert bf.pair_plan % 256 == 0
    assert sa.workspace_layout(0, sa.BF16, 1, 2, 4096, 128, 64, 64, extra_tokens=0).pair_plan == bf.pair_plan
    assert sa.workspace_layout(0, sa.FP32, 1, 2, 4096, 128, 64, 64).pair_plan == 0
    assert sa.workspace_layout(1, sa.BF16, 1, 2, 4096, 128, 128, 64).pair_plan == 0
    assert sa.workspace_layout(0, sa.BF16_FP8QK, 1, 2, 4096, 128, 64, 64).pair_plan > 0


def test_page_parameter_ranges_are_accepted():
    g = json.load(open(GOLDEN))
    assert check(extra=g["extra_tokens_range"]["max"]) == sa.OK
    assert check(extra=g["extra_tokens_range"]["max"] + 1) == sa.EINVAL
    assert check(mode=1, bq=128, keep=g["keep_percent_range"]["min"]) == sa.OK
    assert check(mode=1, bq=128, keep=g["keep_percent_range"]["max"]) == sa.OK
    for t in (g["tau_range"]["min"], g["tau_range"]["max"], g["tau_range"]["default"]):
        assert check(tau=t) == sa.OK
    bq, bk = g["block_sizes"]["sla"]
    assert check(mode=1, bq=bq, bk=bk) == sa.OK


def test_workspace_layout():
    L = sa.workspace_layout(sa.MODE_SOL, sa.BF16, 1, 24, 65536, 128, 64, 64)
    assert (L.Mq, L.M, L.Mpad) == (1024, 1024, 1024)
    offs = [L.kept_cnt, L.kept_bm, L.kept_idx, L.mult, L.extra_cnt, L.extra_idx, L.extra_flag, L.scores,
            L.qbar, L.kbar, L.vbar, L.extra_buf, L.extra_part, L.extra_seed, L.kbar_bf, L.vbar_t, L.v_t]
    assert all(o % 256 == 0 for o in offs)
    assert offs == sorted(offs) and L.total > L.v_t
    assert L.qbar - L.scores >= 24 * 1024 * 1024 * 4        # scores rows of Mpad floats
    assert L.kbar - L.qbar >= 24 * 1024 * 128 * 4
    a = sa.workspace_bytes(0, 0, 1, 24, 16384, 128, 64, 64)
    b = sa.workspace_bytes(0, 0, 1, 24, 32768, 128, 64, 64)
    assert 0 < a < b
    assert sa.workspace_bytes(0, 0, 0, 24, 16384, 128, 64, 64) == 0
    # rows of ragged length: M = 100 key blocks, scores padded to Mpad = 128 per row
    Lr = sa.workspace_layout(sa.MODE_SOL, sa.BF16, 1, 1, 6400, 128, 64, 64)
    assert (Lr.M, Lr.Mpad) == (100, 128) and Lr.qbar - Lr.scores >= 100 * 128 * 4
    Lf = sa.workspace_layout(sa.MODE_SLA, sa.FP32, 1, 2, 4096, 64, 128, 64)
    assert Lf.Mpad == 64 and Lf.v_t == 0


def test_status_strings_and_kernel_names():
    assert sa.status_string(0) == "ok"
    assert "workspace" in sa.status_string(sa.EWORKSPACE)
    assert sa.kernel_names() == ["block_pool", "block_score", "block_select", "extra_select",
                                 "sparse_flash_fwd"]


def test_noalloc_scratch_size_matches_the_header():
    import re
    text = open(os.path.join(os.path.dirname(__file__), "..", "include", "solattn.h")).read()
    m = re.search(r"#define SOLATTN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == sa.NOALLOC_SCRATCH_BYTES


def test_noalloc_validates_before_any_device_call():
    # invalid arguments and a caller workspace are refused on the host (no GPU here)
    L = sa.lib()
    assert L.sol_attn_fwd_noalloc(QP, KP, VP, OP, 1, 2, 4096, 64, float("nan"), 64, 64, 0, 0, None) == sa.EINVAL
    assert "tau" in sa.last_error()
    o = sa.make_opts(workspace=1 << 40, workspace_bytes=1 << 30)
    assert L.sol_attn_fwd_noalloc(QP, KP, VP, OP, 1, 2, 4096, 64, 1.3, 64, 64, 0, 0, ctypes.byref(o)) == sa.EINVAL
    assert "workspace" in sa.last_error()


def test_peak_probe_validates_before_any_device_call():
    # unknown kinds, small or misaligned buffers and zero trips are refused on the host
    L = sa.lib()
    work = ctypes.c_double()
    big = 64 << 20
    assert L.solattn_peak_probe(0, None, big, 1, None, ctypes.byref(work)) == sa.EINVAL
    assert L.solattn_peak_probe(0, QP, big, 0, None, ctypes.byref(work)) == sa.EINVAL
    assert L.solattn_peak_probe(0, QP + 8, big, 1, None, ctypes.byref(work)) == sa.EINVAL
    assert L.solattn_peak_probe(4, QP, big, 1, None, ctypes.byref(work)) == sa.EINVAL
    assert L.solattn_peak_probe(0, QP, 1 << 20, 1, None, ctypes.byref(work)) == sa.EINVAL
    assert L.solattn_peak_probe(3, QP, 1 << 20, 1, None, ctypes.byref(work)) == sa.EINVAL
    assert L.solattn_peak_probe(2, QP, 16, 1, None, ctypes.byref(work)) == sa.EINVAL
    assert L.solattn_peak_probe(0, QP, big, 1, None, None) == sa.EINVAL
