// block_score: s_ij = q̄_i . k̄_j / sqrt(d) for every (query block, key block) pair of a head
// (node docs, sol-attn table, tau row: the threshold is measured in standard deviations of
// this block-score distribution).
//
// fp32 throughout: the selection compares scores against mean + tau*std of the row, and a
// bf16 rounding of the pooled vectors would move scores far more than the 1e-4*std band the
// masks are checked to.  The products run on the fp32 matrix instruction (32x32x2: exact fp32
// products, fp32 accumulation): a 128x128 output tile per workgroup, each wave 64x64 as four
// 32x32 accumulators; q̄ and k̄ rows are staged through LDS in slices of 32 dimensions.
#include "common.h"
#include "launch.h"

namespace solattn {

typedef float f32x16_s __attribute__((ext_vector_type(16)));

template <int D>
__global__ __launch_bounds__(256) void block_score_kernel(Problem P) {
  constexpr int DC = 32;                       // dimensions per LDS slice
  constexpr int LD = DC + 1;                   // padded row: 32 rows read at one column hit distinct banks
  __shared__ float As[128 * LD];
  __shared__ float Bs[128 * LD];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * 128, j0 = blockIdx.x * 128;
  const int tid = threadIdx.x, l = tid % 64, w = tid / 64;
  const int c32 = l % 32, h = l / 32;
  const int wi = 64 * (w / 2), wj = 64 * (w % 2);   // this wave's 64x64 sub-tile
  // buffer resources over this head's pooled rows: rows past Mq (M) read zero, so the loads
  // need no branch; a slice's loads are issued while the previous slice is multiplied
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(P.qbar + (size_t)bh * P.Mq * D, static_cast<uint32_t>(P.Mq) * D * 4u);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(P.kbar + (size_t)bh * P.M * D, static_cast<uint32_t>(P.M) * D * 4u);

  f32x16_s acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16_s{};

  // 128 rows x 32 floats of each operand per slice: 1024 float4 per operand, four per thread
  typedef float f32x4_s __attribute__((ext_vector_type(4)));
  f32x4_s xq[4], yk[4];
  auto fetch = [&](int d0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = tid + 256 * u, r = idx / 8, c4 = idx % 8;
      xq[u] = __builtin_bit_cast(f32x4_s, __builtin_amdgcn_raw_buffer_load_b128(
                  qrs, static_cast<uint32_t>(((i0 + r) * D + d0 + 4 * c4) * 4), 0, 0));
      yk[u] = __builtin_bit_cast(f32x4_s, __builtin_amdgcn_raw_buffer_load_b128(
                  krs, static_cast<uint32_t>(((j0 + r) * D + d0 + 4 * c4) * 4), 0, 0));
    }
  };
  fetch(0);
  for (int d0 = 0; d0 < D; d0 += DC) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = tid + 256 * u, r = idx / 8, c4 = idx % 8;
      float* a = As + r * LD + 4 * c4;
      float* b = Bs + r * LD + 4 * c4;
      a[0] = xq[u].x; a[1] = xq[u].y; a[2] = xq[u].z; a[3] = xq[u].w;
      b[0] = yk[u].x; b[1] = yk[u].y; b[2] = yk[u].z; b[3] = yk[u].w;
    }
    __syncthreads();
    if (d0 + DC < D) fetch(d0 + DC);
    // step kk: lanes 0-31 supply dimension 2kk, lanes 32-63 dimension 2kk+1 (A row / B column c32)
#pragma unroll 4
    for (int kk = 0; kk < DC / 2; ++kk) {
      const int k = 2 * kk + h;
      float av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        av[t] = As[(wi + 32 * t + c32) * LD + k];
        bv[t] = Bs[(wj + 32 * t + c32) * LD + k];
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
  }
  // accumulator register r of tile (a, b): row wi + 32a + (r/4)*8 + 4h + r%4, column wj + 32b + c32
  float* S = P.scores + (size_t)bh * P.Mq * P.Mpad;     // rows of Mpad floats
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int j = j0 + wj + 32 * b + c32;
      if (j >= P.M) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + wi + 32 * a + (r / 4) * 8 + 4 * h + (r % 4);
        if (i < P.Mq) S[(size_t)i * P.Mpad + j] = acc[a][b][r] * P.scale;
      }
    }
}

hipError_t launch_block_score(const Problem& P, hipStream_t stream) {
  dim3 grid((P.M + 127) / 128, (P.Mq + 127) / 128, P.B * P.H);
  if (P.d == 128) hipLaunchKernelGGL(block_score_kernel<128>, grid, dim3(256), 0, stream, P);
  else hipLaunchKernelGGL(block_score_kernel<64>, grid, dim3(256), 0, stream, P);
  return hipGetLastError();
}

}  // namespace solattn
