// Host-side launchers of the libsolattn kernels (one per kernel family).
#pragma once
#include "../../include/solattn.h"
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
hipError_t launch_sparse_flash_f32(const Problem& P, hipStream_t stream);   // fp32 tensors
// Per-call counters into stats[0..7] (see include/solattn.h); reuses extra_buf as scratch.
hipError_t launch_stats(const Problem& P, long long* stats, int check_finite, hipStream_t stream);
size_t stats_scratch_bytes();

// Host side of the C ABI (api.cpp), for the allocation-free entry point (noalloc.hip).
// Sets the thread's error detail and returns code.
int set_error(int code, const char* detail);
// sol_attn_fwd on a given device buffer as workspace (opts->workspace is ignored): never
// allocates and records no timing events.  A layout larger than ws_bytes is an error.
int run_sol_on_buffer(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                      float tau, int block_q, int block_k, int sink_range, int extra_tokens,
                      const ::solattn_opts* opts, void* ws, size_t ws_bytes);

}  // namespace solattn
