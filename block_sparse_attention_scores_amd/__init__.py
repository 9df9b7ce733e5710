"""MI355X-native block-sparse attention forward (sol-attn, sla and static local 3-D routing).

The compute path is libsolattn, hand-written HIP for gfx950 behind a C ABI
(include/solattn.h); this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    BF16, FP32, BF16_FP8QK, MODE_SOL, MODE_SLA, MODE_LOCAL3D, MAX_EXTRA, OK, EINVAL, ENOTSUP, EWORKSPACE, EHIP,
    FLAG_EXACT_EXTRA, FLAG_CHECK_FINITE, FLAG_KEEP_SELECTION, NSTATS, STAT_NAMES,
    SolattnError, Opts, WsLayout, Selection, lib, sol_attn, sol_attn_noalloc, sla_attn, local3d_attn, workspace_layout,
    workspace_bytes, workspace_bytes_any, free_default_workspaces, kept_masks,
    alloc_workspace, selection_views, status_string, last_error, kernel_names, timing_enable,
    timing_read, peak_probe, make_opts, header_functions, pair_schedule, PAIR_STRIDES, NOALLOC_SCRATCH_BYTES,
)
