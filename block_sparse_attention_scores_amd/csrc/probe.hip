// Achievable-peak probes for the measurement of the library's kernels against their rooflines:
// the chip's published peaks are the rooflines, and these loops measure what the matrix cores
// and the memory system actually deliver on the machine the bench runs on.
//   kind 0: bf16 32x32x16 matrix instructions, four independent accumulators per wave, no memory
//   kind 1: fp32 32x32x2 matrix instructions, likewise
//   kind 2: device copy of bytes/2 bytes from the first half of buf to the second (16-byte
//           vector loads and stores, grid-stride), the HBM streaming rate
//   kind 3: the kind-0 loop with the first wave of workgroup 0 reading the shader clock counter
//           and the constant-rate wall clock counter before and after it: their ratio times
//           the wall clock's rate is the shader clock while every matrix core is busy
// The caller times the launch on its stream (events) and divides the work (flop_per_launch or
// the bytes moved) by the time.
#include "../../include/solattn.h"
#include "common.h"

namespace {

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float f32x16_p __attribute__((ext_vector_type(16)));

constexpr int PROBE_WG = 256 * 8;       // workgroups: eight per compute unit
constexpr int PROBE_THREADS = 256;

__global__ __launch_bounds__(PROBE_THREADS) void mfma_bf16_probe(float* out, int iters) {
  const int l = threadIdx.x & 63;
  bf16x8_p a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(static_cast<float>((l + e) & 7) * 0.125f);
    b[e] = static_cast<__bf16>(static_cast<float>((l * 3 + e) & 7) * 0.0625f);
  }
  f32x16_p c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (s == 1.2345f) out[blockIdx.x * PROBE_THREADS + threadIdx.x] = s;   // keeps the loop live
}

// kind 3: out[0] = shader clock ticks, out[1] = wall clock ticks over the loop of wave 0 of
// workgroup 0 (a vector store by its first lane)
__global__ __launch_bounds__(PROBE_THREADS) void clock_probe(unsigned long long* out, int iters) {
  const int l = threadIdx.x & 63;
  bf16x8_p a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(static_cast<float>((l + e) & 7) * 0.125f);
    b[e] = static_cast<__bf16>(static_cast<float>((l * 3 + e) & 7) * 0.0625f);
  }
  f32x16_p c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const unsigned long long t0 = clock64(), w0 = wall_clock64();
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  const unsigned long long t1 = clock64(), w1 = wall_clock64();
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    out[0] = t1 - t0;
    out[1] = w1 - w0;
  }
  if (s == 1.2345f) reinterpret_cast<float*>(out)[4 + blockIdx.x * PROBE_THREADS + threadIdx.x] = s;
}

__global__ __launch_bounds__(PROBE_THREADS) void mfma_f32_probe(float* out, int iters) {
  const int l = threadIdx.x & 63;
  const float a = static_cast<float>(l & 7) * 0.125f, b = static_cast<float>((l * 3) & 7) * 0.0625f;
  f32x16_p c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (s == 1.2345f) out[blockIdx.x * PROBE_THREADS + threadIdx.x] = s;
}

__global__ __launch_bounds__(PROBE_THREADS) void copy_probe(const uint4* src, uint4* dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * PROBE_THREADS;
  for (size_t i = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" int solattn_peak_probe(int kind, void* buf, size_t bytes, int iters, void* stream,
                                  double* work_per_launch) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!buf || !work_per_launch || iters < 1) return SOLATTN_EINVAL;
  if (reinterpret_cast<uintptr_t>(buf) % 16) return SOLATTN_EINVAL;
  const double waves = (double)PROBE_WG * (PROBE_THREADS / 64);
  if (kind == 0 || kind == 1) {
    if (bytes < (size_t)PROBE_WG * PROBE_THREADS * sizeof(float)) return SOLATTN_EINVAL;
    if (kind == 0) {
      hipLaunchKernelGGL(mfma_bf16_probe, dim3(PROBE_WG), dim3(PROBE_THREADS), 0, s, static_cast<float*>(buf), iters);
      *work_per_launch = waves * iters * 4.0 * (2.0 * 32 * 32 * 16);
    } else {
      hipLaunchKernelGGL(mfma_f32_probe, dim3(PROBE_WG), dim3(PROBE_THREADS), 0, s, static_cast<float*>(buf), iters);
      *work_per_launch = waves * iters * 4.0 * (2.0 * 32 * 32 * 2);
    }
  } else if (kind == 3) {
    if (bytes < (size_t)(PROBE_WG * PROBE_THREADS + 4) * sizeof(float)) return SOLATTN_EINVAL;
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
      return SOLATTN_EHIP;
    hipLaunchKernelGGL(clock_probe, dim3(PROBE_WG), dim3(PROBE_THREADS), 0, s,
                       static_cast<unsigned long long*>(buf), iters);
    *work_per_launch = 1e3 * khz;              // the wall clock's rate in Hz
  } else if (kind == 2) {
    const size_t half = bytes / 2 / 16 * 16;
    if (half == 0) return SOLATTN_EINVAL;
    const char* src = static_cast<const char*>(buf);
    hipLaunchKernelGGL(copy_probe, dim3(PROBE_WG), dim3(PROBE_THREADS), 0, s, reinterpret_cast<const uint4*>(src),
                       reinterpret_cast<uint4*>(static_cast<char*>(buf) + half), half / 16);
    *work_per_launch = 2.0 * (double)half;     // bytes read + written
  } else {
    return SOLATTN_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? SOLATTN_OK : SOLATTN_EHIP;
}
