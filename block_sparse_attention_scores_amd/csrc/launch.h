// Host-side launchers of the libsolattn kernels (one per kernel family).
#pragma once
#include "common.h"

namespace solattn {

hipError_t launch_block_pool(const Problem& P, hipStream_t stream);
hipError_t launch_block_score(const Problem& P, hipStream_t stream);
hipError_t launch_block_select(const Problem& P, hipStream_t stream);
hipError_t launch_extra_select(const Problem& P, hipStream_t stream);
hipError_t launch_sparse_flash(const Problem& P, hipStream_t stream);

}  // namespace solattn
