// block_pool: block means of Q, K and V (star7 README, "Sol": skipped K/V blocks are
// represented by their centroids, i.e. block means; the same pooling gives the query
// block representatives that the node docs' sol-attn threshold scores).
//
// One workgroup of 256 threads reduces one block of each of the three tensors of one (b, h),
// in turn: rows are read as coalesced 16-byte chunks, summed in fp32 per thread, then across
// the row groups through LDS in a fixed order.  The K and V passes also write the bf16 operand copies the
// attention kernel reads: k̄ rows (bf16), and V and v̄ as transposed 64-key tiles.
#include "common.h"
#include "launch.h"

namespace solattn {

template <typename T>
struct Chunk8;

template <>
struct Chunk8<uint16_t> {
  uint16_t x[8];
  __device__ void load(const uint16_t* p) {
    uint4 r = *reinterpret_cast<const uint4*>(p);
    const uint16_t* s = reinterpret_cast<const uint16_t*>(&r);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = s[e];
  }
  __device__ float f(int e) const { return bf16_to_f32(x[e]); }
  __device__ uint16_t bits(int e) const { return x[e]; }
};

template <>
struct Chunk8<float> {
  float x[8];
  __device__ void load(const float* p) {
    float4 a = reinterpret_cast<const float4*>(p)[0];
    float4 b = reinterpret_cast<const float4*>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  __device__ float f(int e) const { return x[e]; }
  __device__ uint16_t bits(int e) const { return f32_to_bf16(x[e]); }
};

// grid: x = block index (covers max(Mq, Mpad)), y = b*H + h; tensor 0 q, 1 k, 2 v in turn.
template <typename T, int D>
__global__ __launch_bounds__(256) void block_pool_kernel(Problem P) {
  constexpr int CPR = D / 8;        // 8-element chunks per row
  constexpr int RPP = 256 / CPR;    // rows per pass
  __shared__ float red[RPP][D + 4];
  __shared__ uint16_t vt[D][64 + 8];

  const int bh = blockIdx.y;
  for (int which = 0; which < 3; ++which) {
    if (which) __syncthreads();             // the LDS staging of the previous tensor is free
    const int blk = blockIdx.x;
    const int tid = threadIdx.x;
    const bool is_q = which == 0;
    const int bs = is_q ? P.bq : P.bk;
    const int nblk = is_q ? P.Mq : P.M;
    const bool bf_copies = (P.dtype == 0) && !is_q;   // operand copies for the MFMA kernel

    if (blk >= nblk) {
      // zero padding of the bf16 centroid operands (key blocks M .. Mpad-1)
      if (bf_copies && blk < P.Mpad) {
        for (int e = tid; e < D; e += 256) {
          if (which == 1) P.kbar_bf[((size_t)bh * P.Mpad + blk) * D + e] = 0;
          else P.vbar_t[(((size_t)bh * (P.Mpad / 64) + blk / 64) * D + e) * 64 + vt_pos(blk % 64)] = 0;
        }
      }
      continue;
    }

    const Tensor X = is_q ? P.q : (which == 1 ? P.k : P.v);
    const int b = bh / P.H, h = bh % P.H;
    const int gblk = is_q ? blk + P.q0 : blk;        // query blocks are counted from the window start
    const T* base = static_cast<const T*>(X.p) + (int64_t)b * X.sb + (int64_t)h * X.sh +
                    (int64_t)gblk * bs * X.sn;
    const int c = tid % CPR, r0 = tid / CPR;
    const bool write_vt = bf_copies && which == 2;     // bs == 64 for key blocks

    float acc[8];
  #pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int r = r0; r < bs; r += RPP) {
      Chunk8<T> ch;
      ch.load(base + (int64_t)r * X.sn + c * 8);
  #pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += ch.f(e);
      if (write_vt) {
  #pragma unroll
        for (int e = 0; e < 8; ++e) vt[c * 8 + e][vt_pos(r)] = ch.bits(e);
      }
    }
  #pragma unroll
    for (int e = 0; e < 8; ++e) red[r0][c * 8 + e] = acc[e];
    __syncthreads();

    if (tid < D) {
      float s = 0.f;
      for (int r = 0; r < RPP; ++r) s += red[r][tid];
      const float mean = s / static_cast<float>(bs);
      float* dst = is_q ? P.qbar : (which == 1 ? P.kbar : P.vbar);
      const int rows = is_q ? P.Mq : P.M;
      dst[((size_t)bh * rows + blk) * D + tid] = mean;
      if (bf_copies) {
        if (which == 1) {
          P.kbar_bf[((size_t)bh * P.Mpad + blk) * D + tid] = f32_to_bf16(mean);
        } else {
          P.vbar_t[(((size_t)bh * (P.Mpad / 64) + blk / 64) * D + tid) * 64 + vt_pos(blk % 64)] =
              f32_to_bf16(mean);
        }
      }
    }
    if (write_vt) {
      // the whole transposed tile, 16-byte stores: D rows of 64 keys
      uint16_t* dst = P.v_t + ((size_t)bh * P.M + blk) * D * 64;
      for (int u = tid; u < D * 8; u += 256) {
        const int row = u / 8, col = (u % 8) * 8;
        *reinterpret_cast<uint4*>(dst + row * 64 + col) = *reinterpret_cast<const uint4*>(&vt[row][col]);
      }
    }
  }
}

hipError_t launch_block_pool(const Problem& P, hipStream_t stream) {
  // q, k and v (v̄ is unused by sla, but its pass also writes the transposed V tiles)
  const int gx = P.Mq > P.Mpad ? P.Mq : P.Mpad;
  dim3 grid(gx, P.B * P.H);
  if (P.dtype == 0) {
    if (P.d == 128) hipLaunchKernelGGL((block_pool_kernel<uint16_t, 128>), grid, dim3(256), 0, stream, P);
    else hipLaunchKernelGGL((block_pool_kernel<uint16_t, 64>), grid, dim3(256), 0, stream, P);
  } else {
    if (P.d == 128) hipLaunchKernelGGL((block_pool_kernel<float, 128>), grid, dim3(256), 0, stream, P);
    else hipLaunchKernelGGL((block_pool_kernel<float, 64>), grid, dim3(256), 0, stream, P);
  }
  return hipGetLastError();
}

}  // namespace solattn
