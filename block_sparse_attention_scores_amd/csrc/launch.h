// Host-side launchers of the libsolattn kernels (one per kernel family).
#pragma once
#include "common.h"

namespace solattn {

hipError_t launch_block_pool(const Problem& P, hipStream_t stream);
hipError_t launch_quantize_k(const Problem& P, hipStream_t stream);   // fp8-QK key tiles
hipError_t launch_block_score(const Problem& P, hipStream_t stream);
hipError_t launch_block_select(const Problem& P, hipStream_t stream);
// Kept-block union of every pairing stride (bf16 kernel, 64-row query blocks only).
hipError_t launch_pair_plan(const Problem& P, hipStream_t stream);
hipError_t launch_extra_select(const Problem& P, hipStream_t stream);
hipError_t launch_sparse_flash(const Problem& P, hipStream_t stream);
// Per-call counters into stats[0..7] (see include/solattn.h); reuses extra_buf as scratch.
hipError_t launch_stats(const Problem& P, long long* stats, int check_finite, hipStream_t stream);
size_t stats_scratch_bytes();

}  // namespace solattn
