// block_score: s_ij = q̄_i . k̄_j / sqrt(d) for every (query block, key block) pair of a head
// (node docs, sol-attn table, tau row: the threshold is measured in standard deviations of
// this block-score distribution).
//
// fp32 throughout: the selection compares scores against mean + tau*std of the row, and a
// bf16 rounding of the pooled vectors would move scores far more than the 1e-4*std band the
// masks are checked to.  A 64x64 output tile per workgroup, d staged through LDS in slices
// of 32; every output is one sequential fp32 FMA chain over d.
#include "common.h"
#include "launch.h"

namespace solattn {

template <int D>
__global__ __launch_bounds__(256) void block_score_kernel(Problem P) {
  constexpr int DS = 32;
  __shared__ float As[DS][64 + 4];
  __shared__ float Bs[DS][64 + 4];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const float* qb = P.qbar + (size_t)bh * P.Mq * D;
  const float* kb = P.kbar + (size_t)bh * P.M * D;

  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;

  for (int d0 = 0; d0 < D; d0 += DS) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + 256 * u, r = idx / 8, c4 = idx % 8;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
      if (i0 + r < P.Mq) x = *reinterpret_cast<const float4*>(qb + (size_t)(i0 + r) * D + d0 + 4 * c4);
      if (j0 + r < P.M) y = *reinterpret_cast<const float4*>(kb + (size_t)(j0 + r) * D + d0 + 4 * c4);
      As[4 * c4 + 0][r] = x.x; As[4 * c4 + 1][r] = x.y; As[4 * c4 + 2][r] = x.z; As[4 * c4 + 3][r] = x.w;
      Bs[4 * c4 + 0][r] = y.x; Bs[4 * c4 + 1][r] = y.y; Bs[4 * c4 + 2][r] = y.z; Bs[4 * c4 + 3][r] = y.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int e = 0; e < DS; ++e) {
      float av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = As[e][ty + 16 * a];
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = Bs[e][tx + 16 * b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(av[a], bv[b], acc[a][b]);
    }
  }
  float* S = P.scores + (size_t)bh * P.Mq * P.M;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int i = i0 + ty + 16 * a;
    if (i >= P.Mq) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int j = j0 + tx + 16 * b;
      if (j < P.M) S[(size_t)i * P.M + j] = acc[a][b] * P.scale;
    }
  }
}

hipError_t launch_block_score(const Problem& P, hipStream_t stream) {
  dim3 grid((P.M + 63) / 64, (P.Mq + 63) / 64, P.B * P.H);
  if (P.d == 128) hipLaunchKernelGGL(block_score_kernel<128>, grid, dim3(256), 0, stream, P);
  else hipLaunchKernelGGL(block_score_kernel<64>, grid, dim3(256), 0, stream, P);
  return hipGetLastError();
}

}  // namespace solattn
