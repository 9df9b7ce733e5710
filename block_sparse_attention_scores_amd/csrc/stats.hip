// Optional per-call statistics (written only when the caller passes a stats array): how much of
// the attention was exact, how much went through centroids, how many extra tokens were used,
// how many blocks sat within 1e-4 standard deviations of the sol-attn threshold, how many query
// blocks needed the exact extra-token pass, and, on request, how many input or output values
// are not finite.  The counters are sums over every (batch, head).
//
// Two steps, both deterministic: each workgroup writes its partial sums to a scratch area
// (the extra-token candidate buffer, free once the attention has run), and one workgroup adds
// the partials in a fixed order and writes the counters.
#include "common.h"
#include "launch.h"

namespace solattn {

namespace {

constexpr int NSTAT = 8;
constexpr int ROW_WG = 512;      // workgroups of the per-query-block pass (at most)
constexpr int FIN_WG = 256;      // workgroups per tensor of the finite-value pass (at most)

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ long long wave_sum_i(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// One wave per query block (4 per workgroup, grid-stride); partial sums of counters 0..6.
__global__ __launch_bounds__(256) void stats_rows_kernel(Problem P, long long* part) {
  __shared__ long long sh[4][NSTAT];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long rows = (long)P.B * P.H * P.Mq;
  const int M = P.M;
  long long acc[NSTAT] = {0, 0, 0, 0, 0, 0, 0, 0};
  const bool extra_ran = P.extra > 0 && !P.keep_all;
  for (long row = (long)blockIdx.x * 4 + wv; row < rows; row += (long)gridDim.x * 4) {
    const int i = static_cast<int>(row % P.Mq);
    const bool dense = i >= P.dense_q0 && i < P.dense_q1;
    const long long nrows = P.bq;
    if (dense) {
      acc[2] += nrows * P.N;
      continue;
    }
    const int kc = P.kept_cnt[row];
    const int ec = P.extra_cnt[row];
    acc[0] += kc;
    acc[1] += 1;
    acc[2] += nrows * ((long long)kc * P.bk + ec);
    acc[4] += ec;
    if (extra_ran) acc[6] += P.extra_flag[row] == 1 ? 1 : 0;
    if (P.mode == 0) {
      // centroid terms: every key block not kept, except blocks whose 64 tokens are all extra
      // tokens (multiplicity 0).  The extra list is ascending and unique, so a block is whole
      // exactly when its first token sits at position p and its last at p + 63.
      const int* el = P.extra_idx + row * MAX_EXTRA;
      int whole = 0;
      for (int p = lane; p + 63 < ec; p += 64) {
        const int t = el[p];
        whole += ((t & 63) == 0 && el[p + 63] == t + 63) ? 1 : 0;
      }
      acc[3] += nrows * ((long long)(M - kc) - wave_sum_i(whole));
      if (!P.keep_all) {
        // the row's threshold, recomputed in fp32 (two passes, population deviation)
        const float* s = P.scores + row * P.Mpad;
        float a = 0.f;
        for (int j = lane; j < M; j += 64) a += s[j];
        const float mu = wave_sum_f(a) / static_cast<float>(M);
        float b = 0.f;
        for (int j = lane; j < M; j += 64) {
          const float dv = s[j] - mu;
          b = fmaf(dv, dv, b);
        }
        const float sd = sqrtf(wave_sum_f(b) / static_cast<float>(M));
        const float theta = sd > 0.f ? fmaf(P.tau, sd, mu) : mu;
        const float band = 1e-4f * sd;
        int n = 0;
        for (int j = lane; j < M; j += 64) n += fabsf(s[j] - theta) <= band ? 1 : 0;
        acc[5] += wave_sum_i(n);
      }
    }
  }
  if (lane == 0)
    for (int k = 0; k < NSTAT; ++k) sh[wv][k] = acc[k];
  __syncthreads();
  if (threadIdx.x < NSTAT) {
    const int k = threadIdx.x;
    part[(size_t)blockIdx.x * NSTAT + k] = k == 7 ? 0 : ((sh[0][k] + sh[1][k]) + sh[2][k]) + sh[3][k];
  }
}

// Non-finite values of one strided [B, H, N, d] tensor (blockIdx.y: q, k, v, out); counter 7.
// Each thread reads 16-byte chunks (rows start 16-byte aligned and hold a whole number of
// chunks), walking the (row, chunk) index space with a grid stride.
template <typename T>
__global__ __launch_bounds__(256) void stats_finite_kernel(Problem P, long long* part, int first) {
  __shared__ long long sh[4];
  const Tensor t = blockIdx.y == 0 ? P.q : blockIdx.y == 1 ? P.k : blockIdx.y == 2 ? P.v : P.o;
  const T* base = static_cast<const T*>(t.p);
  constexpr int PER = 16 / sizeof(T);                 // elements per chunk
  const int cpr = P.d / PER;                          // chunks per row
  // out: only the rows of the computed window (the others are not written by the call)
  const bool is_out = blockIdx.y == 3;
  const long tok0 = is_out ? (long)P.q0 * P.bq : 0;
  const long ntok = is_out ? (long)P.Mq * P.bq : P.N;
  const long chunks = (long)P.B * P.H * ntok * cpr;
  long long n = 0;
  for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < chunks; e += (long)gridDim.x * 256) {
    const long r = e / cpr;
    const int c = static_cast<int>(e - r * cpr);
    const int b = static_cast<int>(r / ((long)P.H * ntok));
    const int h = static_cast<int>((r / ntok) % P.H);
    const long tok = tok0 + r % ntok;
    const uint4 v = *reinterpret_cast<const uint4*>(base + (int64_t)b * t.sb + (int64_t)h * t.sh +
                                                    tok * t.sn + (int64_t)c * PER);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (sizeof(T) == 2) {
        n += (w[q] & 0x7F80u) == 0x7F80u ? 1 : 0;
        n += (w[q] & 0x7F800000u) == 0x7F800000u ? 1 : 0;
      } else {
        n += (w[q] & 0x7F800000u) == 0x7F800000u ? 1 : 0;
      }
    }
  }
  n = wave_sum_i(n);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x < NSTAT) {
    const int k = threadIdx.x;
    const size_t at = (size_t)first + (size_t)blockIdx.y * gridDim.x + blockIdx.x;
    part[at * NSTAT + k] = k == 7 ? ((sh[0] + sh[1]) + sh[2]) + sh[3] : 0;
  }
}

// Fixed-order sum of the partials into the caller's counters.
__global__ __launch_bounds__(256) void stats_final_kernel(const long long* part, int nparts, int finite,
                                                          long long* stats) {
  __shared__ long long sh[256];
  for (int k = 0; k < NSTAT; ++k) {
    long long a = 0;
    for (int p = threadIdx.x; p < nparts; p += 256) a += part[(size_t)p * NSTAT + k];
    sh[threadIdx.x] = a;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) stats[k] = (k == 7 && !finite) ? -1 : sh[0];
    __syncthreads();
  }
}

}  // namespace

size_t stats_scratch_bytes() { return (size_t)(ROW_WG + 4 * FIN_WG) * NSTAT * sizeof(long long); }

hipError_t launch_stats(const Problem& P, long long* stats, int check_finite, hipStream_t stream) {
  long long* part = reinterpret_cast<long long*>(P.extra_buf);
  const long rows = (long)P.B * P.H * P.Mq;
  const int nrow = static_cast<int>(rows / 4 + 1 < ROW_WG ? rows / 4 + 1 : ROW_WG);
  hipLaunchKernelGGL(stats_rows_kernel, dim3(nrow), dim3(256), 0, stream, P, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int nparts = nrow;
  if (check_finite) {
    const long chunks = (long)P.B * P.H * P.N * P.d * (P.dtype == 0 ? 2 : 4) / 16;
    const long want = (chunks + 255) / 256;
    const int nf = static_cast<int>(want < FIN_WG ? want : FIN_WG);
    if (P.dtype == 0)
      hipLaunchKernelGGL(stats_finite_kernel<uint16_t>, dim3(nf, 4), dim3(256), 0, stream, P, part, nrow);
    else
      hipLaunchKernelGGL(stats_finite_kernel<float>, dim3(nf, 4), dim3(256), 0, stream, P, part, nrow);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    nparts += 4 * nf;
  }
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(256), 0, stream, part, nparts, check_finite, stats);
  return hipGetLastError();
}

}  // namespace solattn
