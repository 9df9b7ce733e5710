// sol_attn_fwd_noalloc: the sol-attn forward on a scratch buffer the library holds in device
// memory, for callers that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  The buffer is a file-scope device array, one copy per GPU
// (each GPU the library runs on holds it until the process ends); its device address is
// looked up once per device, with that device current, and kept.  The call then runs the same
// kernels as sol_attn_fwd with that buffer as its workspace and allocates nothing.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/solattn.h"
#include "launch.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SOLATTN_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

// The current device's copy of `scratch` (its device address, looked up on first use).
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return solattn::set_error(SOLATTN_EHIP, "sol_attn_fwd_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= MAX_DEVICES)
    return solattn::set_error(SOLATTN_ENOTSUP, "sol_attn_fwd_noalloc: device index beyond 64");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return solattn::set_error(SOLATTN_EHIP, "sol_attn_fwd_noalloc: hipGetSymbolAddress of the scratch failed");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return SOLATTN_OK;
}

}  // namespace

extern "C" int sol_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, int B, int H, int N,
                                    int d, float tau, int block_q, int block_k, int sink_range,
                                    int extra_tokens, const solattn_opts* opts) {
  if (opts && opts->workspace)
    return solattn::set_error(SOLATTN_EINVAL,
                              "sol_attn_fwd_noalloc runs on the library's scratch: opts->workspace must be NULL");
  // validate first (no device call), so that a bad argument is reported as such
  int rc = solattn_check_args(SOLATTN_MODE_SOL, q, k, v, out, B, H, N, d, tau, 100.f, block_q, block_k,
                              sink_range, extra_tokens, opts);
  if (rc != SOLATTN_OK) return rc;
  void* p = nullptr;
  if ((rc = scratch_ptr(&p)) != SOLATTN_OK) return rc;
  return solattn::run_sol_on_buffer(q, k, v, out, B, H, N, d, tau, block_q, block_k, sink_range, extra_tokens,
                                    opts, p, SOLATTN_NOALLOC_SCRATCH_BYTES);
}
