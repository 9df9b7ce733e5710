// fp8 (E4M3) key tiles for the fp8-QK flavour of the attention kernel.
//
// Every key row (and every pooled key row) is scaled by a power of two 2^e, e the smallest
// integer with amax <= 448 * 2^e (amax = the row's largest magnitude; e = 0 for a zero row;
// e >= -127), and rounded to E4M3 (nearest, ties to even).  A tile is the 64 rows of one key
// block (or of 64 pooled keys) as 64 x D bytes, row-major, followed by the 64 rows' scale
// codes e + 127 (the E8M0 form the matrix instruction takes): 64 * D + 64 bytes.
#include "common.h"
#include "launch.h"

namespace solattn {

// grid: x = key block j (< M: K rows) or M + c (pooled-key tile c), y = b*H + h.
// 256 threads: D/8 threads per row, each taking 8 consecutive values.
template <int D>
__global__ __launch_bounds__(256) void quantize_k_kernel(Problem P) {
  constexpr int TPR = D / 8;                 // threads per row
  constexpr int RPP = 256 / TPR;             // rows per pass
  constexpr size_t TB = 64 * D + 64;         // tile bytes
  const int bh = blockIdx.y, j = blockIdx.x;
  const int tid = threadIdx.x, t = tid % TPR, r0 = tid / TPR;
  const bool pooled = j >= P.M;
  const int c = j - P.M;                     // pooled-key tile index
  uint8_t* tile = pooled ? P.kb8 + ((size_t)bh * (P.Mpad / 64) + c) * TB
                         : P.k8 + ((size_t)bh * P.M + j) * TB;
  const int b = bh / P.H, h = bh % P.H;
  const uint16_t* Kb = static_cast<const uint16_t*>(P.k.p) + (int64_t)b * P.k.sb + (int64_t)h * P.k.sh;
  for (int r = r0; r < 64; r += RPP) {
    float x[8];
    if (!pooled) {
      const uint4 raw = *reinterpret_cast<const uint4*>(Kb + (int64_t)(j * 64 + r) * P.k.sn + 8 * t);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    } else {
      const int row = 64 * c + r;            // pooled key index (rows past M are zero)
      if (row < P.M) {
        const float4* src = reinterpret_cast<const float4*>(P.kbar + ((size_t)bh * P.M + row) * D + 8 * t);
        const float4 a = src[0], bb = src[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = bb.x; x[5] = bb.y; x[6] = bb.z; x[7] = bb.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));   // within the row's group
    const int ex = e4m3_scale_exp(amax);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = ldexpf(x[e], -ex);
    *reinterpret_cast<uint2*>(tile + (size_t)r * D + 8 * t) = pack8_e4m3(x);
    if (t == 0) tile[64 * D + r] = static_cast<uint8_t>(ex + 127);
  }
}

hipError_t launch_quantize_k(const Problem& P, hipStream_t stream) {
  dim3 grid(P.M + P.Mpad / 64, P.B * P.H);
  if (P.d == 128) hipLaunchKernelGGL(quantize_k_kernel<128>, grid, dim3(256), 0, stream, P);
  else hipLaunchKernelGGL(quantize_k_kernel<64>, grid, dim3(256), 0, stream, P);
  return hipGetLastError();
}

}  // namespace solattn
