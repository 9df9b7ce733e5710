// sparse_flash_fwd: the attention of one query block over its work list, in one FP32 online
// softmax (star7 README, "Sol": kept K/V blocks exactly, skipped blocks through their
// centroids, merged in one FP32 online softmax; "SLA": only the routed blocks):
//   1. the kept key blocks (for dense query blocks: every block),
//   2. the extra tokens, gathered 64 at a time,
//   3. sol only: the centroid terms of every key block, 64 per tile, each with logit
//      q.k̄_j / sqrt(d) + ln(m_ij) (m_ij = tokens of block j not attended exactly; a kept
//      block has m = 0 and drops out).
// Every tile is the same computation on a 64-key K tile and a transposed V tile in LDS with a
// per-key additive bias, so one inner loop serves all three phases.
//
// bf16 kernel: each wave owns 32 query rows.  S^T = K Q^T and O^T += V^T P^T run on the
// 32x32x16 bf16 matrix instruction: the score accumulator's lane layout (lane = query row,
// 16 registers = keys) feeds P^T straight to the second product, so P never leaves registers;
// the V tile is stored transposed with a key permutation that matches that layout.  Running
// max and sum are fp32 and kept per lane (the two half-waves hold the same query rows and
// combine their partial sums at the end).  Logits are taken in base 2.
//
// fp32 kernel: one thread per query row, exact fp32 dot products, the same three phases.
#include "common.h"
#include "launch.h"

namespace solattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float LOG2E = 1.4426950408889634f;

template <int D>
struct FlashSmem {
  uint16_t k[64][D + 8];      // K tile, key-major, padded rows
  uint16_t vt[D][64 + 8];     // V tile transposed (d-major), keys permuted by vt_pos
  float bias[64];             // additive base-2 logit bias per key of the tile
};

// Map the flat workgroup index to (head, query block): dense query blocks (the heaviest work)
// first, and consecutive workgroups on the same head.
__device__ __forceinline__ void flash_work(const Problem& P, int g, int* bh, int* qi) {
  const int nd = P.dense_q1 - P.dense_q0;
  const int BH = P.B * P.H;
  if (g < BH * nd) {
    *bh = g / nd;
    *qi = P.dense_q0 + g % nd;
    return;
  }
  g -= BH * nd;
  const int ns = P.Mq - nd;
  *bh = g / ns;
  int r = g % ns;
  *qi = r < P.dense_q0 ? r : r + nd;
}

template <int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void sparse_flash_bf16_kernel(Problem P) {
  __shared__ FlashSmem<D> sm;
  constexpr int NT = 64 * WAVES;
  int bh, qi;
  flash_work(P, blockIdx.x, &bh, &qi);
  const int tid = threadIdx.x, w = tid / 64, l = tid % 64, h32 = l / 32, c32 = l % 32;
  const int b = bh / P.H, hh = bh % P.H;
  const size_t row = (size_t)bh * P.Mq + qi;
  const uint16_t* Kb = static_cast<const uint16_t*>(P.k.p) + (int64_t)b * P.k.sb + (int64_t)hh * P.k.sh;
  const uint16_t* Vb = static_cast<const uint16_t*>(P.v.p) + (int64_t)b * P.v.sb + (int64_t)hh * P.v.sh;
  const uint16_t* Qb = static_cast<const uint16_t*>(P.q.p) + (int64_t)b * P.q.sb + (int64_t)hh * P.q.sh;

  // this wave's 32 query rows: Q^T operand fragments
  const int q0 = qi * P.bq + 32 * w;
  bf16x8_t qf[D / 16];
  {
    const uint16_t* qr = Qb + (int64_t)(q0 + c32) * P.q.sn + 8 * h32;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qr + 16 * ks);
  }

  const bool dense = qi >= P.dense_q0 && qi < P.dense_q1;
  const int nk = P.kept_cnt[row];
  const int ne = dense ? 0 : P.extra_cnt[row];
  const int nx = (ne + 63) / 64;
  const int nc = (P.mode == 0 && !dense && nk < P.M) ? P.Mpad / 64 : 0;
  const int ntiles = nk + nx + nc;
  const int* klist = P.kept_idx + row * P.M;
  const int* elist = P.extra_idx + row * MAX_EXTRA;
  const uint8_t* mrow = P.mult + row * P.Mpad;
  const float sl2 = P.scale * LOG2E;

  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16_t{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    // ---- stage the tile in LDS
    if (t < nk) {
      const int j = klist[t];
      const uint16_t* ks = Kb + (int64_t)j * 64 * P.k.sn;
      for (int u = tid; u < 64 * (D / 8); u += NT) {
        const int r = u / (D / 8), c = (u % (D / 8)) * 8;
        *reinterpret_cast<uint4*>(&sm.k[r][c]) = *reinterpret_cast<const uint4*>(ks + (int64_t)r * P.k.sn + c);
      }
      const uint16_t* vs = P.v_t + ((size_t)bh * P.M + j) * D * 64;
      for (int u = tid; u < D * 8; u += NT) {
        const int r = u / 8, c = (u % 8) * 8;
        *reinterpret_cast<uint4*>(&sm.vt[r][c]) = *reinterpret_cast<const uint4*>(vs + r * 64 + c);
      }
      if (tid < 64) sm.bias[tid] = 0.f;
    } else if (t < nk + nx) {
      const int e0 = (t - nk) * 64;
      for (int u = tid; u < 64 * (D / 8); u += NT) {
        const int r = u / (D / 8), c = (u % (D / 8)) * 8;
        uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = kv;
        if (e0 + r < ne) {
          const int tok = elist[e0 + r];
          kv = *reinterpret_cast<const uint4*>(Kb + (int64_t)tok * P.k.sn + c);
          vv = *reinterpret_cast<const uint4*>(Vb + (int64_t)tok * P.v.sn + c);
        }
        *reinterpret_cast<uint4*>(&sm.k[r][c]) = kv;
        const uint16_t* vx = reinterpret_cast<const uint16_t*>(&vv);
        const int pr = vt_pos(r);
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.vt[c + e][pr] = vx[e];
      }
      if (tid < 64) sm.bias[tid] = (e0 + tid < ne) ? 0.f : -__builtin_inff();
    } else {
      const int c0 = (t - nk - nx) * 64;
      const uint16_t* ks = P.kbar_bf + ((size_t)bh * P.Mpad + c0) * D;
      for (int u = tid; u < 64 * (D / 8); u += NT) {
        const int r = u / (D / 8), c = (u % (D / 8)) * 8;
        *reinterpret_cast<uint4*>(&sm.k[r][c]) = *reinterpret_cast<const uint4*>(ks + (size_t)r * D + c);
      }
      const uint16_t* vs = P.vbar_t + ((size_t)bh * (P.Mpad / 64) + c0 / 64) * D * 64;
      for (int u = tid; u < D * 8; u += NT) {
        const int r = u / 8, c = (u % 8) * 8;
        *reinterpret_cast<uint4*>(&sm.vt[r][c]) = *reinterpret_cast<const uint4*>(vs + r * 64 + c);
      }
      if (tid < 64) {
        const int m = mrow[c0 + tid];    // 0 for kept blocks and for padding beyond M
        sm.bias[tid] = m > 0 ? __log2f(static_cast<float>(m)) : -__builtin_inff();
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for the 64 keys (two 32-key halves)
    f32x16_t s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&sm.k[32 * kt + c32][16 * ks + 8 * h32]);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kt], 0, 0, 0);
      }
    }
    // ---- online softmax (base 2); register r of half kt holds key 32kt + (r/4)*8 + 4*h32 + r%4
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + (r / 4) * 8 + 4 * h32 + (r % 4);
        const float x = s[kt][r] * sl2 + sm.bias[key];
        s[kt][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
    bf16x8_t pf[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(s[kt][r] - m_use);
        psum += p;
        pf[2 * kt + r / 8][r % 8] = __builtin_bit_cast(__bf16, f32_to_bf16(p));
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&sm.vt[32 * dt + c32][16 * ks + 8 * h32]);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], o[dt], 0, 0, 0);
      }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  uint16_t* Ob = static_cast<uint16_t*>(const_cast<void*>(P.o.p)) + (int64_t)b * P.o.sb +
                 (int64_t)hh * P.o.sh + (int64_t)(q0 + c32) * P.o.sn;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * dt + 8 * g + 4 * h32;
      uint2 pk;
      pk.x = static_cast<uint32_t>(f32_to_bf16(o[dt][4 * g + 0] * inv)) |
             (static_cast<uint32_t>(f32_to_bf16(o[dt][4 * g + 1] * inv)) << 16);
      pk.y = static_cast<uint32_t>(f32_to_bf16(o[dt][4 * g + 2] * inv)) |
             (static_cast<uint32_t>(f32_to_bf16(o[dt][4 * g + 3] * inv)) << 16);
      *reinterpret_cast<uint2*>(Ob + d0) = pk;
    }
}

// ------------------------------------------------------------------ fp32 path

template <int D, int BQ>
__global__ __launch_bounds__(BQ) void sparse_flash_f32_kernel(Problem P) {
  // every thread reads the same key row at a time, so rows come straight from the cache
  __shared__ const float* krow[64];
  __shared__ const float* vrow[64];
  __shared__ float bias[64];
  int bh, qi;
  flash_work(P, blockIdx.x, &bh, &qi);
  const int tid = threadIdx.x;
  const int b = bh / P.H, hh = bh % P.H;
  const size_t row = (size_t)bh * P.Mq + qi;
  const float* Kb = static_cast<const float*>(P.k.p) + (int64_t)b * P.k.sb + (int64_t)hh * P.k.sh;
  const float* Vb = static_cast<const float*>(P.v.p) + (int64_t)b * P.v.sb + (int64_t)hh * P.v.sh;
  const float* Qb = static_cast<const float*>(P.q.p) + (int64_t)b * P.q.sb + (int64_t)hh * P.q.sh;
  const int qrow = qi * BQ + tid;

  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = Qb[(int64_t)qrow * P.q.sn + e];
    o[e] = 0.f;
  }
  const bool dense = qi >= P.dense_q0 && qi < P.dense_q1;
  const int nk = P.kept_cnt[row];
  const int ne = dense ? 0 : P.extra_cnt[row];
  const int nx = (ne + 63) / 64;
  const int nc = (P.mode == 0 && !dense && nk < P.M) ? P.Mpad / 64 : 0;
  const int ntiles = nk + nx + nc;
  const int* klist = P.kept_idx + row * P.M;
  const int* elist = P.extra_idx + row * MAX_EXTRA;
  const uint8_t* mrow = P.mult + row * P.Mpad;
  const float sl2 = P.scale * LOG2E;
  float m_run = -__builtin_inff(), l_run = 0.f;

  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    if (tid < 64) {
      const int r = tid;
      const float* kp = Kb;
      const float* vp = Vb;
      float bv = -__builtin_inff();
      if (t < nk) {
        const int tok = klist[t] * 64 + r;
        kp = Kb + (int64_t)tok * P.k.sn;
        vp = Vb + (int64_t)tok * P.v.sn;
        bv = 0.f;
      } else if (t < nk + nx) {
        const int ei = (t - nk) * 64 + r;
        if (ei < ne) {
          const int tok = elist[ei];
          kp = Kb + (int64_t)tok * P.k.sn;
          vp = Vb + (int64_t)tok * P.v.sn;
          bv = 0.f;
        }
      } else {
        const int j = (t - nk - nx) * 64 + r;
        const int m = mrow[j];            // 0 for kept blocks and for padding beyond M
        if (m > 0) {
          kp = P.kbar + ((size_t)bh * P.M + j) * D;
          vp = P.vbar + ((size_t)bh * P.M + j) * D;
          bv = __log2f(static_cast<float>(m));
        }
      }
      krow[r] = kp;
      vrow[r] = vp;
      bias[r] = bv;
    }
    __syncthreads();
    float sc[64];
    float mx = -__builtin_inff();
    for (int r = 0; r < 64; ++r) {
      float x = -__builtin_inff();
      if (bias[r] != -__builtin_inff()) {
        const float* kp = krow[r];
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) s = fmaf(q[e], kp[e], s);
        x = s * sl2 + bias[r];
      }
      sc[r] = x;
      mx = fmaxf(mx, x);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] *= alpha;
    for (int r = 0; r < 64; ++r) {
      if (sc[r] == -__builtin_inff()) continue;
      const float p = exp2f(sc[r] - m_use);
      l_run += p;
      const float* vp = vrow[r];
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] = fmaf(p, vp[e], o[e]);
    }
    m_run = m_new;
  }
  float* Ob = static_cast<float*>(const_cast<void*>(P.o.p)) + (int64_t)b * P.o.sb +
              (int64_t)hh * P.o.sh + (int64_t)qrow * P.o.sn;
  const float inv = 1.f / l_run;
#pragma unroll
  for (int e = 0; e < D; ++e) Ob[e] = o[e] * inv;
}

hipError_t launch_sparse_flash(const Problem& P, hipStream_t stream) {
  dim3 grid(P.B * P.H * P.Mq);
  if (P.dtype == 0) {
    if (P.bq == 64) {
      if (P.d == 128) hipLaunchKernelGGL((sparse_flash_bf16_kernel<128, 2>), grid, dim3(128), 0, stream, P);
      else hipLaunchKernelGGL((sparse_flash_bf16_kernel<64, 2>), grid, dim3(128), 0, stream, P);
    } else {
      if (P.d == 128) hipLaunchKernelGGL((sparse_flash_bf16_kernel<128, 4>), grid, dim3(256), 0, stream, P);
      else hipLaunchKernelGGL((sparse_flash_bf16_kernel<64, 4>), grid, dim3(256), 0, stream, P);
    }
  } else {
    if (P.bq == 64) {
      if (P.d == 128) hipLaunchKernelGGL((sparse_flash_f32_kernel<128, 64>), grid, dim3(64), 0, stream, P);
      else hipLaunchKernelGGL((sparse_flash_f32_kernel<64, 64>), grid, dim3(64), 0, stream, P);
    } else {
      if (P.d == 128) hipLaunchKernelGGL((sparse_flash_f32_kernel<128, 128>), grid, dim3(128), 0, stream, P);
      else hipLaunchKernelGGL((sparse_flash_f32_kernel<64, 128>), grid, dim3(128), 0, stream, P);
    }
  }
  return hipGetLastError();
}

}  // namespace solattn
