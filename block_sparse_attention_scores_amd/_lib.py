"""ctypes binding of libsolattn (include/solattn.h): argument marshalling only.

Every step of the pass runs in the library's HIP kernels.  PyTorch supplies device
memory (inputs, outputs, the workspace) and the current HIP stream.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsolattn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "solattn.h")

OK, EINVAL, ENOTSUP, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
BF16, FP32, BF16_FP8QK = 0, 1, 2
MODE_SOL, MODE_SLA, MODE_LOCAL3D = 0, 1, 2
MAX_EXTRA = 256
NKERNELS = 5


PAIR_STRIDES = 8           # candidate pairing strides of the bf16 attention kernel
NOALLOC_SCRATCH_BYTES = 64 << 20   # SOLATTN_NOALLOC_SCRATCH_BYTES


class SolattnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"libsolattn status {status} ({status_string(status)}): {detail}")


FLAG_EXACT_EXTRA = 1   # SOLATTN_FLAG_EXACT_EXTRA
FLAG_CHECK_FINITE = 2  # SOLATTN_FLAG_CHECK_FINITE
FLAG_KEEP_SELECTION = 4  # SOLATTN_FLAG_KEEP_SELECTION
NSTATS = 8             # SOLATTN_NSTATS
STAT_NAMES = ("kept_blocks", "selected_qblocks", "exact_pairs", "centroid_terms", "extra_tokens",
              "near_threshold", "exact_extra_qblocks", "nonfinite")


class Opts(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("q_stride", ctypes.c_int64 * 3),
        ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3),
        ("dense_row_begin", ctypes.c_int),
        ("dense_row_end", ctypes.c_int),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("flags", ctypes.c_uint),
        ("stats", ctypes.c_void_p),
        ("q_row_begin", ctypes.c_int),
        ("q_row_end", ctypes.c_int),
    ]


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "total", "kept_cnt", "kept_bm", "kept_idx", "mult", "extra_cnt", "extra_idx", "extra_flag",
        "scores", "qbar", "kbar", "vbar", "extra_buf", "extra_part", "extra_seed", "kbar_bf", "vbar_t",
        "v_t", "k8", "kb8", "pair_plan")] + [
        ("Mq", ctypes.c_int), ("M", ctypes.c_int), ("Mpad", ctypes.c_int)]


class Selection(ctypes.Structure):
    _fields_ = [("Mq", ctypes.c_int), ("M", ctypes.c_int), ("Mpad", ctypes.c_int)] + [
        (n, ctypes.c_void_p) for n in ("kept_cnt", "kept_bm", "kept_idx", "mult", "extra_cnt",
                                       "extra_idx", "extra_flag", "scores")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m block_sparse_attention_scores_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.sol_attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, f, i, i, i, i, ctypes.POINTER(Opts)]
    L.sol_attn_fwd.restype = i
    L.sol_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, f, i, i, i, i, ctypes.POINTER(Opts)]
    L.sol_attn_fwd_noalloc.restype = i
    L.sla_attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, ctypes.POINTER(Opts)]
    L.sla_attn_fwd.restype = i
    L.local3d_attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, i, ctypes.POINTER(Opts)]
    L.local3d_attn_fwd.restype = i
    L.solattn_check_args.argtypes = [i, vp, vp, vp, vp, i, i, i, i, f, f, i, i, i, i, ctypes.POINTER(Opts)]
    L.solattn_check_args.restype = i
    L.local3d_check_args.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, i, ctypes.POINTER(Opts)]
    L.local3d_check_args.restype = i
    L.solattn_workspace_layout.argtypes = [i, i, i, i, i, i, i, i, i, i, ctypes.POINTER(WsLayout)]
    L.solattn_workspace_layout.restype = i
    L.solattn_workspace_bytes_ex.argtypes = [i, i, i, i, i, i, i, i, i, i]
    L.solattn_workspace_bytes_ex.restype = ctypes.c_size_t
    L.solattn_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
    L.solattn_workspace_bytes.restype = ctypes.c_size_t
    L.solattn_selection_view.argtypes = [ctypes.POINTER(Opts), i, i, i, i, i, i, ctypes.POINTER(Selection)]
    L.solattn_selection_view.restype = i
    L.solattn_free_default_workspaces.argtypes = []
    L.solattn_free_default_workspaces.restype = i
    L.solattn_status_string.argtypes = [i]
    L.solattn_status_string.restype = ctypes.c_char_p
    L.solattn_last_error_detail.argtypes = []
    L.solattn_last_error_detail.restype = ctypes.c_char_p
    L.solattn_last_error.argtypes = []
    L.solattn_last_error.restype = ctypes.c_char_p
    L.solattn_timing_enable.argtypes = [i]
    L.solattn_timing_enable.restype = i
    L.solattn_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_longlong), i]
    L.solattn_timing_read.restype = i
    L.solattn_kernel_name.argtypes = [i]
    L.solattn_kernel_name.restype = ctypes.c_char_p
    L.solattn_peak_probe.argtypes = [i, vp, ctypes.c_size_t, i, vp, ctypes.POINTER(ctypes.c_double)]
    L.solattn_peak_probe.restype = i
    ip = ctypes.POINTER(ctypes.c_int)
    L.solattn_pair_schedule.argtypes = [i, i, i, i, ip, ip, i]
    L.solattn_pair_schedule.restype = i
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().solattn_status_string(status).decode()


def last_error() -> str:
    """Detail of the last failing call on this thread (solattn_last_error_detail)."""
    return lib().solattn_last_error_detail().decode()


def kernel_names():
    return [lib().solattn_kernel_name(k).decode() for k in range(NKERNELS)]


def pair_schedule(Mq: int, dense=(0, 0), stride: int = 1):
    """[(qa, qb), ...]: the query blocks of each unit of one head of the bf16 attention kernel
    with 64-row query blocks (qb = -1: a single block), dense query blocks [dense[0], dense[1]),
    under pairing `stride`."""
    n = lib().solattn_pair_schedule(Mq, dense[0], dense[1], stride, None, None, 0)
    if n < 0:
        raise SolattnError(n, last_error())
    qa, qb = (ctypes.c_int * max(n, 1))(), (ctypes.c_int * max(n, 1))()
    lib().solattn_pair_schedule(Mq, dense[0], dense[1], stride, qa, qb, n)
    return [(qa[j], qb[j]) for j in range(n)]


def workspace_layout(mode: int, dtype: int, B: int, H: int, N: int, d: int, block_q: int,
                     block_k: int, q_rows: int | None = None, extra_tokens: int = MAX_EXTRA) -> WsLayout:
    """Offsets of the intermediate buffers; q_rows: rows of a query-row window (default N)."""
    L = WsLayout()
    rows = N if q_rows is None else int(q_rows)
    rc = lib().solattn_workspace_layout(mode, dtype, B, H, N, d, block_q, block_k, int(extra_tokens),
                                        rows, ctypes.byref(L))
    if rc != OK:
        raise SolattnError(rc, "invalid workspace shape")
    return L


def workspace_bytes(mode, dtype, B, H, N, d, block_q, block_k, q_rows=None,
                    extra_tokens=MAX_EXTRA) -> int:
    """Bytes of a caller workspace for this call shape (solattn_workspace_bytes_ex)."""
    rows = N if q_rows is None else int(q_rows)
    return int(lib().solattn_workspace_bytes_ex(mode, dtype, B, H, N, d, block_q, block_k,
                                                int(extra_tokens), rows))


def workspace_bytes_any(mode, B, H, N, d, block_q, block_k, extra_tokens) -> int:
    """Bytes enough for a whole-sequence call of this shape in any dtype (solattn_workspace_bytes)."""
    return int(lib().solattn_workspace_bytes(mode, B, H, N, d, block_q, block_k, int(extra_tokens)))


def free_default_workspaces() -> None:
    rc = lib().solattn_free_default_workspaces()
    if rc != OK:
        raise SolattnError(rc, last_error())


def make_opts(dtype=BF16, strides=None, dense_rows=(0, 0), workspace=0, workspace_bytes=0,
              stream=0, flags=0, stats=0, q_rows=None) -> Opts:
    o = Opts()
    o.struct_size = ctypes.sizeof(Opts)
    o.dtype = dtype
    if strides is not None:
        for name, st in zip(("q_stride", "k_stride", "v_stride", "o_stride"), strides):
            arr = getattr(o, name)
            for j in range(3):
                arr[j] = int(st[j])
    o.dense_row_begin, o.dense_row_end = int(dense_rows[0]), int(dense_rows[1])
    o.workspace = workspace or None
    o.workspace_bytes = int(workspace_bytes)
    o.stream = stream or None
    o.flags = int(flags)
    o.stats = stats or None
    if q_rows is not None:
        o.q_row_begin, o.q_row_end = int(q_rows[0]), int(q_rows[1])
    return o


def peak_probe(kind: int, buf, iters: int = 1, stream=None) -> float:
    """Launch one achievable-peak probe (solattn_peak_probe) on buf (a uint8 GPU tensor) and
    return its work per launch (flop for kinds 0 and 1, bytes moved for kind 2)."""
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(buf.device).cuda_stream
    work = ctypes.c_double()
    rc = lib().solattn_peak_probe(int(kind), buf.data_ptr(), buf.numel() * buf.element_size(), int(iters),
                                  stream, ctypes.byref(work))
    if rc != OK:
        raise SolattnError(rc, "peak probe")
    return work.value


def timing_enable(on: bool = True) -> None:
    lib().solattn_timing_enable(1 if on else 0)


def timing_read():
    """{kernel name: (total ms, launches)} since the last read; waits for the recorded events."""
    ms = (ctypes.c_double * NKERNELS)()
    n = (ctypes.c_longlong * NKERNELS)()
    rc = lib().solattn_timing_read(ms, n, NKERNELS)
    if rc != OK:
        raise SolattnError(rc, "timing read")
    return {name: (ms[k], n[k]) for k, name in enumerate(kernel_names())}


# ----------------------------------------------------------------------------- torch front end

def _torch():
    import torch
    return torch


def _dtype_code(t, qk_fp8=False) -> int:
    torch = _torch()
    if qk_fp8:
        if t.dtype != torch.bfloat16:
            raise TypeError("the fp8-QK flavour takes bfloat16 tensors")
        return BF16_FP8QK
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check_tensor(name, t, shape, dtype):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != 4 or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} dtype {t.dtype} != {dtype}")
    if t.stride(3) != 1:
        raise ValueError(f"{name}: the d axis must be contiguous")


def alloc_workspace(mode, q, block_q, block_k, q_rows=None, qk_fp8=False, extra_tokens=MAX_EXTRA):
    """A workspace for a call on q's shape (or on the query-row window q_rows = (begin, end))
    with up to extra_tokens extra tokens."""
    torch = _torch()
    B, H, N, d = q.shape
    rows = None if q_rows is None else q_rows[1] - q_rows[0]
    nbytes = workspace_bytes(mode, _dtype_code(q, qk_fp8), B, H, N, d, block_q, block_k, rows,
                             extra_tokens)
    return torch.empty(nbytes, dtype=torch.uint8, device=q.device)


def _call(mode, q, k, v, *, tau, keep_percent, block_q, block_k, sink_range, extra_tokens,
          dense_rows, out, workspace, stream, flags=0, grid=None, stats=None, q_rows=None,
          qk_fp8=False):
    torch = _torch()
    B, H, N, d = q.shape
    for n, t in (("k", k), ("v", v)):
        _check_tensor(n, t, q.shape, q.dtype)
    _check_tensor("q", q, q.shape, q.dtype)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    _check_tensor("out", out, q.shape, q.dtype)
    if workspace is None:
        workspace = alloc_workspace(mode, q, block_q, block_k, q_rows, qk_fp8, extra_tokens)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    strides = [tuple(t.stride()[:3]) for t in (q, k, v, out)]
    if stats is not None:
        if not stats.is_cuda or stats.dtype != torch.int64 or stats.numel() < NSTATS \
                or not stats.is_contiguous():
            raise ValueError(f"stats must be a contiguous int64 GPU tensor of >= {NSTATS} elements")
    opts = make_opts(_dtype_code(q, qk_fp8), strides, dense_rows, workspace.data_ptr(),
                     workspace.numel() * workspace.element_size(), stream, flags,
                     stats.data_ptr() if stats is not None else 0, q_rows)
    L = lib()
    if mode == MODE_SOL:
        rc = L.sol_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, d,
                            float(tau), block_q, block_k, sink_range, extra_tokens, ctypes.byref(opts))
    elif mode == MODE_LOCAL3D:
        F, Hh, Ww = (int(g) for g in grid)
        rc = L.local3d_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, d,
                                F, Hh, Ww, block_q, block_k, sink_range, extra_tokens,
                                ctypes.byref(opts))
    else:
        rc = L.sla_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, d,
                            block_q, block_k, sink_range, extra_tokens, float(keep_percent),
                            ctypes.byref(opts))
    if rc != OK:
        raise SolattnError(rc, last_error())
    return out, workspace


def sol_attn(q, k, v, *, tau=1.3, block_q=64, block_k=64, sink_range=0, extra_tokens=0,
             dense_rows=(0, 0), out=None, workspace=None, stream=None, return_workspace=False,
             flags=0, stats=None, q_rows=None, qk_fp8=False):
    """sol-attn forward on [B, H, N, d] GPU tensors (bfloat16 or float32); see include/solattn.h.
    stats: optional int64 GPU tensor of NSTATS elements for the per-call counters; q_rows:
    optional (begin, end) query-row window (only those rows of out are written); qk_fp8: the
    fp8-QK flavour (SOLATTN_BF16_FP8QK, bfloat16 tensors)."""
    o, ws = _call(MODE_SOL, q, k, v, tau=tau, keep_percent=0.0, block_q=block_q, block_k=block_k,
                  sink_range=sink_range, extra_tokens=extra_tokens, dense_rows=dense_rows, out=out,
                  workspace=workspace, stream=stream, flags=flags, stats=stats, q_rows=q_rows,
                  qk_fp8=qk_fp8)
    return (o, ws) if return_workspace else o


def sol_attn_noalloc(q, k, v, *, tau=1.3, block_q=64, block_k=64, sink_range=0, extra_tokens=0,
                     dense_rows=(0, 0), out=None, stream=None, flags=0, stats=None, q_rows=None,
                     qk_fp8=False):
    """sol-attn forward through sol_attn_fwd_noalloc: the library's own scratch buffer is the
    workspace, nothing is allocated by the call (out must then be given by callers that cannot
    allocate; None allocates it here, in torch).  Raises SolattnError with EWORKSPACE when the
    call does not fit in NOALLOC_SCRATCH_BYTES."""
    torch = _torch()
    B, H, N, d = q.shape
    for n, t in (("k", k), ("v", v)):
        _check_tensor(n, t, q.shape, q.dtype)
    _check_tensor("q", q, q.shape, q.dtype)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    _check_tensor("out", out, q.shape, q.dtype)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    strides = [tuple(t.stride()[:3]) for t in (q, k, v, out)]
    opts = make_opts(_dtype_code(q, qk_fp8), strides, dense_rows, 0, 0, stream, flags,
                     stats.data_ptr() if stats is not None else 0, q_rows)
    rc = lib().sol_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, d,
                                    float(tau), block_q, block_k, sink_range, extra_tokens,
                                    ctypes.byref(opts))
    if rc != OK:
        raise SolattnError(rc, last_error())
    return out


def sla_attn(q, k, v, *, keep_percent=10.0, block_q=128, block_k=64, sink_range=0, extra_tokens=0,
             dense_rows=(0, 0), out=None, workspace=None, stream=None, return_workspace=False,
             flags=0, stats=None, q_rows=None, qk_fp8=False):
    """sla forward on [B, H, N, d] GPU tensors (bfloat16 or float32); see include/solattn.h."""
    o, ws = _call(MODE_SLA, q, k, v, tau=0.0, keep_percent=keep_percent, block_q=block_q,
                  block_k=block_k, sink_range=sink_range, extra_tokens=extra_tokens,
                  dense_rows=dense_rows, out=out, workspace=workspace, stream=stream, flags=flags,
                  stats=stats, q_rows=q_rows, qk_fp8=qk_fp8)
    return (o, ws) if return_workspace else o


def local3d_attn(q, k, v, *, grid, block_q=64, block_k=64, sink_range=0, extra_tokens=0,
                 dense_rows=(0, 0), out=None, workspace=None, stream=None, return_workspace=False,
                 flags=0, stats=None, q_rows=None, qk_fp8=False):
    """Static local 3-D neighbourhood forward on [B, H, N, d] GPU tensors; grid = (frames,
    height, width) with frames*height*width == N; see include/solattn.h."""
    if len(grid) != 3:
        raise ValueError("grid must be (frames, height, width)")
    o, ws = _call(MODE_LOCAL3D, q, k, v, tau=0.0, keep_percent=100.0, block_q=block_q,
                  block_k=block_k, sink_range=sink_range, extra_tokens=extra_tokens,
                  dense_rows=dense_rows, out=out, workspace=workspace, stream=stream, flags=flags,
                  grid=grid, stats=stats, q_rows=q_rows, qk_fp8=qk_fp8)
    return (o, ws) if return_workspace else o


def selection_views(workspace, mode, dtype, B, H, N, d, block_q, block_k, q_rows=None):
    """Views of a call's intermediate results inside its workspace tensor (torch, on device);
    q_rows = (begin, end) for a call on a query-row window (its query blocks count from 0).
    The selection comes from solattn_selection_view; kept_idx and mult hold the call's values
    only when it ran with FLAG_KEEP_SELECTION (or on fp32 tensors).  scores: [BH, Mq, M] (the
    padding columns of the library's rows are cut off)."""
    torch = _torch()
    L = workspace_layout(mode, dtype, B, H, N, d, block_q, block_k,
                         None if q_rows is None else q_rows[1] - q_rows[0])
    BH, Mq, M, Mpad = B * H, L.Mq, L.M, L.Mpad
    base = workspace.data_ptr()
    o = make_opts(dtype, workspace=base, workspace_bytes=workspace.numel(), q_rows=q_rows)
    sv = Selection()
    rc = lib().solattn_selection_view(ctypes.byref(o), mode, B, H, N, block_q, block_k, ctypes.byref(sv))
    if rc != OK:
        raise SolattnError(rc, last_error())
    assert (sv.Mq, sv.M, sv.Mpad) == (Mq, M, Mpad)

    def view(off, count, dt, shape):
        nbytes = count * torch.tensor([], dtype=dt).element_size()
        return workspace[off:off + nbytes].view(dt).reshape(shape)

    def sel(ptr, count, dt, shape):
        return view(int(ptr) - base, count, dt, shape)

    extra = {}
    if L.pair_plan:
        extra["pair_plan"] = view(L.pair_plan, BH * PAIR_STRIDES, torch.int64, (BH, PAIR_STRIDES))
    return dict(
        **extra,
        qbar=view(L.qbar, BH * Mq * d, torch.float32, (BH, Mq, d)),
        kbar=view(L.kbar, BH * M * d, torch.float32, (BH, M, d)),
        vbar=view(L.vbar, BH * M * d, torch.float32, (BH, M, d)),
        scores=sel(sv.scores, BH * Mq * Mpad, torch.float32, (BH, Mq, Mpad))[:, :, :M],
        kept_cnt=sel(sv.kept_cnt, BH * Mq, torch.int32, (BH, Mq)),
        kept_idx=sel(sv.kept_idx, BH * Mq * M, torch.int32, (BH, Mq, M)),
        kept_bm=sel(sv.kept_bm, BH * Mq * (Mpad // 64), torch.int64, (BH, Mq, Mpad // 64)),
        mult=sel(sv.mult, BH * Mq * Mpad, torch.uint8, (BH, Mq, Mpad)),
        extra_cnt=sel(sv.extra_cnt, BH * Mq, torch.int32, (BH, Mq)),
        extra_idx=sel(sv.extra_idx, BH * Mq * MAX_EXTRA, torch.int32, (BH, Mq, MAX_EXTRA)),
        extra_flag=sel(sv.extra_flag, BH * Mq, torch.int32, (BH, Mq)),
    )


def kept_masks(sel_np, bh: int, M: int):
    """[Mq, M] bool kept masks of (b, h) index bh from a numpy copy of selection_views' kept_bm
    (the bitmap every call writes)."""
    import numpy as np
    words = sel_np["kept_bm"][bh].astype(np.int64).view(np.uint64)
    bits = ((words[:, :, None] >> np.arange(64, dtype=np.uint64)[None, None, :]) & np.uint64(1))
    return bits.reshape(words.shape[0], -1)[:, :M].astype(bool)


def header_functions():
    """Names of the functions include/solattn.h declares."""
    import re
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)) - {"if"})
