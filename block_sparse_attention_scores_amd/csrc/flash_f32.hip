// sparse_flash_fwd for fp32 tensors: the same attention as the bf16 kernel (star7 README, "Sol":
// kept K/V blocks exactly, skipped blocks through their centroids, one FP32 online softmax;
// "SLA": only the routed blocks), with every product on the fp32 matrix instruction
// (32x32x2: exact fp32 products, fp32 accumulation), so the result is the fp32 definition up to
// summation order.
//
// A workgroup of four waves owns one query block.  Its work list is cut into 32-key tiles:
//   1. the kept key blocks (two tiles each; for dense query blocks every block),
//   2. the extra tokens, 32 to a tile,
//   3. sol only: the centroid terms, 32 pooled keys to a tile, each with logit
//      q.k̄_j / sqrt(d) + ln(m_ij) (m_ij = tokens of block j not attended exactly; a kept block
//      has m = 0 and drops out).
// A wave owns 32 query rows of one tile slot: with 64-row query blocks two slots (waves 0, 1
// and 2, 3) take alternate tiles and their softmax states are merged at the end; with 128-row
// blocks the four waves share every tile.  Per tile and wave, S^T = K Q^T (keys x rows) and
// O^T += V^T P^T; the pair of reduction indices of one instruction is (dim t, dim t + d/2) for
// the score product and a key pair for the value product, chosen so that each lane's operands
// are its own registers: q, and the probabilities exactly where the score product left them.
// Tiles go through LDS with padded rows; the next step's rows are loaded into registers while
// the current one is computed.
#include "common.h"
#include "launch.h"

namespace solattn {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr float LOG2E_F32 = 1.4426950408889634f;

// fp32 work order: workgroup -> (head, query block), dense query blocks (the heaviest) first.
__device__ __forceinline__ void f32_work(const Problem& P, int g, int* bh, int* qi) {
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
  const int r = g % ns;
  *qi = r < P.dense_q0 ? r : r + nd;
}

}  // namespace

template <int D, int BQ>
__global__ __launch_bounds__(256, 1) void sparse_flash_f32_kernel(Problem P) {
  constexpr int KT = 32;                  // keys per tile
  constexpr int RW = BQ / 32;             // waves per tile slot (32 query rows each)
  constexpr int NS = 4 / RW;              // tile slots per step
  constexpr int LD = D + 4;               // padded LDS row (floats): rows start on distinct banks
  constexpr int ROWS = NS * KT;           // K and V rows per step
  constexpr int TPR = 256 / ROWS;         // threads per row in the copy
  constexpr int CPT = D / 4 / TPR;        // float4 chunks per thread and tensor
  static_assert(CPT * TPR * 4 == D, "row split");
  __shared__ float ks[NS][KT][LD];
  __shared__ float vs[NS][KT][LD];
  __shared__ float bs[NS][KT];            // per-key logit bias (base 2): 0, log2(m) or -inf

  int bh, qi;
  f32_work(P, blockIdx.x, &bh, &qi);
  const int tid = threadIdx.x, l = tid % 64, w = tid / 64;
  const int c32 = l % 32, h = l / 32;
  const int slot = w / RW, rg = w % RW;
  const int b = bh / P.H, hh = bh % P.H;
  const size_t row = (size_t)bh * P.Mq + qi;
  const float* Kb = static_cast<const float*>(P.k.p) + (int64_t)b * P.k.sb + (int64_t)hh * P.k.sh;
  const float* Vb = static_cast<const float*>(P.v.p) + (int64_t)b * P.v.sb + (int64_t)hh * P.v.sh;
  const float* Qb = static_cast<const float*>(P.q.p) + (int64_t)b * P.q.sb + (int64_t)hh * P.q.sh;
  const int qrow = (qi + P.q0) * BQ + 32 * rg + c32;      // this lane's query row

  const bool dense = qi >= P.dense_q0 && qi < P.dense_q1;
  const int nk = P.kept_cnt[row];
  const int ne = dense ? 0 : P.extra_cnt[row];
  const int nx = (ne + KT - 1) / KT;
  const int nc = (P.mode == 0 && !dense && nk < P.M) ? P.Mpad / KT : 0;
  const int ntile = 2 * nk + nx + nc;
  const int nstep = (ntile + NS - 1) / NS;
  const int* klist = P.kept_idx + row * P.M;
  const int* elist = P.extra_idx + row * MAX_EXTRA;
  const uint8_t* mrow = P.mult + row * P.Mpad;
  const float sl2 = P.scale * LOG2E_F32;

  // B operand of the score product, step t: dims t (lanes 0-31) and t + D/2 (lanes 32-63)
  float qv[D / 2];
  {
    const float* qp = Qb + (int64_t)qrow * P.q.sn + h * (D / 2);
#pragma unroll
    for (int t = 0; t < D / 2; t += 4) {
      const float4 x = *reinterpret_cast<const float4*>(qp + t);
      qv[t] = x.x;
      qv[t + 1] = x.y;
      qv[t + 2] = x.z;
      qv[t + 3] = x.w;
    }
  }

  // copy of one step: thread -> (row of the step, part of the row)
  const int crow = tid / TPR, cpart = tid % TPR;
  const int cslot = crow / KT, cr = crow % KT;
  float4 pk[CPT], pv[CPT];
  float pb = -__builtin_inff();
  auto fetch = [&](int s) {
    const int t = s * NS + cslot;
    const float* kp = nullptr;
    const float* vp = nullptr;
    pb = -__builtin_inff();
    if (t < 2 * nk) {
      const int tok = klist[t / 2] * 64 + KT * (t % 2) + cr;
      kp = Kb + (int64_t)tok * P.k.sn;
      vp = Vb + (int64_t)tok * P.v.sn;
      pb = 0.f;
    } else if (t < 2 * nk + nx) {
      const int e = (t - 2 * nk) * KT + cr;
      if (e < ne) {
        const int tok = elist[e];
        kp = Kb + (int64_t)tok * P.k.sn;
        vp = Vb + (int64_t)tok * P.v.sn;
        pb = 0.f;
      }
    } else if (t < ntile) {
      const int j = (t - 2 * nk - nx) * KT + cr;
      const int m = mrow[j];                // 0 for kept blocks and for padding beyond M
      if (m > 0) {
        kp = P.kbar + ((size_t)bh * P.M + j) * D;
        vp = P.vbar + ((size_t)bh * P.M + j) * D;
        pb = __log2f(static_cast<float>(m));
      }
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int col = 4 * (cpart * CPT + c);
      pk[c] = kp ? *reinterpret_cast<const float4*>(kp + col) : make_float4(0.f, 0.f, 0.f, 0.f);
      pv[c] = vp ? *reinterpret_cast<const float4*>(vp + col) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int col = 4 * (cpart * CPT + c);
      *reinterpret_cast<float4*>(&ks[cslot][cr][col]) = pk[c];
      *reinterpret_cast<float4*>(&vs[cslot][cr][col]) = pv[c];
    }
    if (cpart == 0) bs[cslot][cr] = pb;
  };

  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16_t{};
  float m_run = -__builtin_inff(), l_run = 0.f;

  if (nstep > 0) fetch(0);
#pragma unroll 1
  for (int s = 0; s < nstep; ++s) {
    __syncthreads();                      // every wave is done with the previous step's rows
    store();
    __syncthreads();
    if (s + 1 < nstep) fetch(s + 1);      // in flight while this step is computed
    if (s * NS + slot >= ntile) continue;
    // S^T: register r holds key 8(r/4) + 4h + r%4 of the tile for query row c32
    f32x16_t acc = {};
    const float* kr = &ks[slot][c32][h * (D / 2)];
#pragma unroll
    for (int t = 0; t < D / 2; t += 4) {
      const float4 a = *reinterpret_cast<const float4*>(kr + t);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, qv[t], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, qv[t + 1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, qv[t + 2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, qv[t + 3], acc, 0, 0, 0);
    }
    float x[16];
    float mx = -__builtin_inff();
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 bb = *reinterpret_cast<const float4*>(&bs[slot][8 * g + 4 * h]);
      x[4 * g + 0] = fmaf(acc[4 * g + 0], sl2, bb.x);
      x[4 * g + 1] = fmaf(acc[4 * g + 1], sl2, bb.y);
      x[4 * g + 2] = fmaf(acc[4 * g + 2], sl2, bb.z);
      x[4 * g + 3] = fmaf(acc[4 * g + 3], sl2, bb.w);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));   // lanes l and l+32 hold the same row
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    m_run = m_new;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(x[r] - m_use);
      l_run += p[r];
    }
    // O^T += V^T P^T: step r takes the key pair (8(r/4) + r%4, that + 4), lane half h the
    // key its own register r holds
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float* vr = &vs[slot][8 * (r / 4) + 4 * h + (r % 4)][c32];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[32 * dt], p[r], o[dt], 0, 0, 0);
    }
  }

  // merge the two slots' states (64-row query blocks): slot 1 hands its state to slot 0
  if constexpr (NS == 2) {
    __syncthreads();                      // the tile rows are no longer read
    float* st = &ks[0][0][0] + (size_t)rg * 64 * (2 + D / 2);   // per lane: m, l, D/2 outputs
    if (slot == 1) {
      st[l] = m_run;
      st[64 + l] = l_run;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[128 + (dt * 16 + r) * 64 + l] = o[dt][r];
    }
    __syncthreads();
    if (slot == 1) return;
    const float m2 = st[l], l2 = st[64 + l];
    const float m_new = fmaxf(m_run, m2);
    const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
    const float a1 = __builtin_amdgcn_exp2f(m_run - m_use), a2 = __builtin_amdgcn_exp2f(m2 - m_use);
    l_run = l_run * a1 + l2 * a2;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] = o[dt][r] * a1 + st[128 + (dt * 16 + r) * 64 + l] * a2;
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  float* Ob = static_cast<float*>(const_cast<void*>(P.o.p)) + (int64_t)b * P.o.sb +
              (int64_t)hh * P.o.sh + (int64_t)qrow * P.o.sn;
  // register r of block dt holds dim 32dt + 8(r/4) + 4h + r%4
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(Ob + 32 * dt + 8 * g + 4 * h) =
          make_float4(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv, o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
}

hipError_t launch_sparse_flash_f32(const Problem& P, hipStream_t stream) {
  dim3 grid(P.B * P.H * P.Mq);
  if (P.bq == 64) {
    if (P.d == 128) hipLaunchKernelGGL((sparse_flash_f32_kernel<128, 64>), grid, dim3(256), 0, stream, P);
    else hipLaunchKernelGGL((sparse_flash_f32_kernel<64, 64>), grid, dim3(256), 0, stream, P);
  } else {
    if (P.d == 128) hipLaunchKernelGGL((sparse_flash_f32_kernel<128, 128>), grid, dim3(256), 0, stream, P);
    else hipLaunchKernelGGL((sparse_flash_f32_kernel<64, 128>), grid, dim3(256), 0, stream, P);
  }
  return hipGetLastError();
}

}  // namespace solattn
