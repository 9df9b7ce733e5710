// extra_select: for each sparse query block i, the up to E = extra_tokens individual keys with
// the highest q̄_i . k_t among tokens outside its kept blocks, ties to the lower token (node
// docs, common inputs table, extra_tokens row: extra high-score tokens each query block
// attends beyond its selected blocks).
//
// A workgroup (4 waves) owns 32 query blocks of one head and streams the head's keys once,
// 128 tokens per step (32 per wave).  Scores come from the 32x32x16 bf16 matrix instruction
// with q̄ split into two bf16 parts (hi + lo), so each score is accurate to ~2^-17 relative,
// i.e. fp32-like, while the keys are exact bf16.  Each lane owns one query block (column of
// the 32x32 accumulator); a score above the row's running threshold is appended to the row's
// candidate buffer in the workspace.  When a buffer holds more than E entries after a step,
// one wave finds the E-th best entry by radix selection on (score, token) and compacts the
// buffer to exactly E entries; that entry's score becomes the new threshold.  Keys stream in
// increasing token order, so a later token that ties the threshold always loses the tie and a
// strict comparison suffices.  At the end the E tokens are ranked ascending, written out, and
// the centroid multiplicity of every block they came from drops by their count.
#include "common.h"
#include "launch.h"

namespace solattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int XR = 32;      // query blocks per workgroup
constexpr int XCHUNK = 128; // tokens per step

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint16_t bf16_bits(float f) { return f32_to_bf16(f); }

// One radix digit step inside one wave: given the 256-bin histogram `h` (in LDS) of the
// candidates still matching the prefix, find the digit holding the `need`-th largest.
// Returns digit, and writes the count above it and the count at it.
__device__ int wave_pick_digit(const int* h, int need, int* above, int* at, int* scratch) {
  const int l = threadIdx.x & 63;
  int c[4], s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c[q] = h[255 - 4 * l - q];
    s += c[q];
  }
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(incl, o);
    if (l >= o) incl += t;
  }
  int ex = incl - s;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (ex < need && need <= ex + c[q]) {
      scratch[0] = 255 - 4 * l - q;
      scratch[1] = ex;
      scratch[2] = c[q];
    }
    ex += c[q];
  }
  wave_sync();
  const int dg = scratch[0];
  *above = scratch[1];
  *at = scratch[2];
  wave_sync();
  return dg;
}

constexpr int XPL = EXTRA_CAP / 64;   // buffer entries per lane during a selection

// Radix selection over 32-bit keys held XPL per lane (valid[] marks live entries).  Finds the
// `need`-th largest key K*, returns it; *need_eq = how many entries equal to K* are taken and
// *cnt_eq = how many entries equal K*.
__device__ uint32_t wave_radix_select(const uint32_t* key, const bool* valid, int need, int* hist,
                                      int* scratch, int* need_eq, int* cnt_eq) {
  const int l = threadIdx.x & 63;
  uint32_t prefix = 0, pmask = 0;
  int at = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
#pragma unroll
    for (int q = 0; q < 4; ++q) hist[4 * l + q] = 0;
    wave_sync();
#pragma unroll
    for (int u = 0; u < XPL; ++u)
      if (valid[u] && (key[u] & pmask) == prefix) atomicAdd(&hist[(key[u] >> shift) & 255u], 1);
    wave_sync();
    int above;
    const int dg = wave_pick_digit(hist, need, &above, &at, scratch);
    prefix |= static_cast<uint32_t>(dg) << shift;
    pmask |= 0xFFu << shift;
    need -= above;
  }
  *need_eq = need;
  *cnt_eq = at;
  return prefix;
}

// Reduce one row's buffer (cnt > E entries) to its E best entries under (score desc, token asc).
__device__ float wave_compact_row(uint2* buf, int cnt, int E, int* hist, int* scratch) {
  const int l = threadIdx.x & 63;
  uint32_t key[XPL], tok[XPL];
  bool valid[XPL];
#pragma unroll
  for (int u = 0; u < XPL; ++u) {
    const int p = l + 64 * u;
    valid[u] = p < cnt;
    uint2 e = valid[u] ? buf[p] : make_uint2(0u, 0u);
    key[u] = float_key(__uint_as_float(e.x));
    tok[u] = e.y;
  }
  int need_eq, cnt_eq;
  const uint32_t kstar = wave_radix_select(key, valid, E, hist, scratch, &need_eq, &cnt_eq);
  uint32_t tmax = 0xFFFFFFFFu;   // largest token taken among those tying K*
  if (need_eq < cnt_eq) {
    uint32_t k2[XPL];
    bool v2[XPL];
#pragma unroll
    for (int u = 0; u < XPL; ++u) {
      v2[u] = valid[u] && key[u] == kstar;
      k2[u] = ~tok[u];            // larger k2 = smaller token
    }
    int ne2, ce2;
    const uint32_t t2 = wave_radix_select(k2, v2, need_eq, hist, scratch, &ne2, &ce2);
    tmax = ~t2;
  }
  bool keep[XPL];
#pragma unroll
  for (int u = 0; u < XPL; ++u)
    keep[u] = valid[u] && (key[u] > kstar || (key[u] == kstar && tok[u] <= tmax));
  // every lane holds its entries in registers now; write the survivors to the front
  int base = 0;
#pragma unroll
  for (int u = 0; u < XPL; ++u) {
    const uint64_t m = __ballot(keep[u]);
    const int pos = base + __popcll(m & ((1ull << l) - 1ull));
    if (keep[u]) buf[pos] = make_uint2(__float_as_uint(key_float(key[u])), tok[u]);
    base += __popcll(m);
  }
  return key_float(kstar);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void extra_select_kernel(Problem P) {
  __shared__ float theta[XR];
  __shared__ int cnt[XR];
  __shared__ int whist[4][256];
  __shared__ int wscr[4][4];
  __shared__ float qs[(sizeof(T) == 4) ? XR : 1][D];

  const int bh = blockIdx.y, i0 = blockIdx.x * XR;
  const int tid = threadIdx.x, w = tid / 64, l = tid % 64;
  const int rl = l % 32, i = i0 + rl;
  const int E = P.extra, N = P.N;
  const int b = bh / P.H, h = bh % P.H;
  const bool row_ok = i < P.Mq && !(i >= P.dense_q0 && i < P.dense_q1);
  const size_t grow = (size_t)bh * P.Mq + (i < P.Mq ? i : 0);
  const uint8_t* mrow = P.mult + grow * P.Mpad;
  const T* kbase = static_cast<const T*>(P.k.p) + (int64_t)b * P.k.sb + (int64_t)h * P.k.sh;

  if (tid < XR) {
    theta[tid] = -__builtin_inff();
    cnt[tid] = 0;
  }

  // q̄ operands: split bf16 hi/lo fragments (bf16 inputs) or an fp32 copy in LDS
  bf16x8_t qhi[D / 16], qlo[D / 16];
  if constexpr (sizeof(T) == 2) {
    const float* qb = P.qbar + grow * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (i < P.Mq) ? qb[16 * ks + 8 * (l / 32) + e] : 0.f;
        const uint16_t hb = bf16_bits(x);
        const uint16_t lb = bf16_bits(x - bf16_to_f32(hb));
        qhi[ks][e] = __builtin_bit_cast(__bf16, hb);
        qlo[ks][e] = __builtin_bit_cast(__bf16, lb);
      }
    }
  } else {
    for (int u = tid; u < XR * D; u += 256) {
      const int r = u / D, e = u % D;
      qs[r][e] = (i0 + r < P.Mq) ? P.qbar[((size_t)bh * P.Mq + i0 + r) * D + e] : 0.f;
    }
  }
  __syncthreads();

  uint2* buf = P.extra_buf + grow * EXTRA_CAP;
  for (int t0 = 0; t0 < N; t0 += XCHUNK) {
    const int tw = t0 + 32 * w;
    if (tw < N) {
      float acc[16];
      if constexpr (sizeof(T) == 2) {
        f32x16_t c = {};
        const T* kr = kbase + (int64_t)(tw + rl) * P.k.sn + 8 * (l / 32);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(kr + 16 * ks);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qhi[ks], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qlo[ks], c, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = c[r];
      } else {
#pragma unroll 1
        for (int r = 0; r < 16; ++r) {
          const int tk = tw + (r / 4) * 8 + (l / 32) * 4 + (r % 4);
          const float* kr = reinterpret_cast<const float*>(kbase) + (int64_t)tk * P.k.sn;
          float s = 0.f;
#pragma unroll 8
          for (int e = 0; e < D; ++e) s = fmaf(qs[rl][e], kr[e], s);
          acc[r] = s;
        }
      }
      const bool cand = row_ok && mrow[tw / P.bk] > 0;
      const float th = theta[rl];
      if (cand) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (acc[r] > th) {
            const int tk = tw + (r / 4) * 8 + (l / 32) * 4 + (r % 4);
            const int pos = atomicAdd(&cnt[rl], 1);
            buf[pos] = make_uint2(__float_as_uint(acc[r]), static_cast<uint32_t>(tk));
          }
        }
      }
    }
    __syncthreads();
    // cut a buffer back to its E best entries when the next step could overflow it, and
    // after the last step
    const bool last = t0 + XCHUNK >= N;
    for (int rr = w; rr < XR; rr += 4) {
      const int c = cnt[rr];
      if (c > EXTRA_CAP - XCHUNK || (last && c > E)) {
        uint2* rb = P.extra_buf + ((size_t)bh * P.Mq + i0 + rr) * EXTRA_CAP;
        const float th = wave_compact_row(rb, c, E, whist[w], wscr[w]);
        if (l == 0) {
          theta[rr] = th;
          cnt[rr] = E;
        }
      }
    }
    __syncthreads();
  }

  // rank the survivors by token, write them out, and take them out of their blocks' centroids
  for (int rr = w; rr < XR; rr += 4) {
    const int ii = i0 + rr;
    if (ii >= P.Mq || (ii >= P.dense_q0 && ii < P.dense_q1)) continue;
    const size_t row = (size_t)bh * P.Mq + ii;
    const uint2* rb = P.extra_buf + row * EXTRA_CAP;
    const int c = cnt[rr];
    int* toks = whist[w];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = l + 64 * u;
      if (p < c) toks[p] = static_cast<int>(rb[p].y);
    }
    wave_sync();
    int* out = P.extra_idx + row * MAX_EXTRA;
    uint8_t* mr = P.mult + row * P.Mpad;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = l + 64 * u;
      if (p >= c) continue;
      const int t = toks[p], bt = t / P.bk;
      int rank = 0, same = 0, same_before = 0;
      for (int q = 0; q < c; ++q) {
        const int o = toks[q];
        rank += o < t;
        const bool sb = (o / P.bk) == bt;
        same += sb;
        same_before += sb && o < t;
      }
      out[rank] = t;
      if (same_before == 0) mr[bt] = static_cast<uint8_t>(P.bk - same);
    }
    if (l == 0) P.extra_cnt[row] = c;
    wave_sync();
  }
}

hipError_t launch_extra_select(const Problem& P, hipStream_t stream) {
  dim3 grid((P.Mq + XR - 1) / XR, P.B * P.H);
  if (P.dtype == 0) {
    if (P.d == 128) hipLaunchKernelGGL((extra_select_kernel<uint16_t, 128>), grid, dim3(256), 0, stream, P);
    else hipLaunchKernelGGL((extra_select_kernel<uint16_t, 64>), grid, dim3(256), 0, stream, P);
  } else {
    if (P.d == 128) hipLaunchKernelGGL((extra_select_kernel<float, 128>), grid, dim3(256), 0, stream, P);
    else hipLaunchKernelGGL((extra_select_kernel<float, 64>), grid, dim3(256), 0, stream, P);
  }
  return hipGetLastError();
}

}  // namespace solattn
