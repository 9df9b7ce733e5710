// block_select: per (head, query block) row of block scores, choose the key blocks attended
// exactly and compact them into an ascending index list.
//   sol-attn (node docs, sol-attn table, tau row): keep s_ij > mean + tau*std of the row,
//     std the population deviation over all M blocks (two passes).
//   sla (node docs, sla table, keep_percent row): keep the k highest non-forced blocks,
//     ties to the lower index (radix select on order-preserving keys).
//   local 3-D (the article on block sparse attention for H3 in ComfyUI, section 1): a fixed
//     pattern with no scores.  The sequence is a frames x height x width token grid in raster
//     order; key block j is kept when it holds a token of the query block or a grid neighbour
//     of one (one step along one axis, no wrap-around).  Where the grid of blocks exists this
//     is the centre, +-1 frame and +-1 block up/down/left/right stencil.
//   Sink blocks and the diagonal block(s) are kept on top in every mode (node docs, sla
//   table, and sink_conditioning row).  Query blocks in the dense row range keep every block.
// The kept set is written as a bitmap (bit j of word j/64), which the attention kernel walks
// without touching memory, with its count; the ascending index lists and the centroid
// multiplicities are written only when asked for (fp32 tensors, or a caller keeping the
// selection).
// One wave per row (four rows per workgroup); the row's scores are read from memory once, into
// registers (RU per lane, M <= 64 RU), and every pass (mean, deviation, threshold or radix
// select, compaction) works on them; rows longer than that are read once per pass.  All
// reductions have a fixed order, so results are deterministic.
#include "common.h"
#include "launch.h"

namespace solattn {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Orders this wave's LDS accesses before and after it (the waves of a workgroup work on
// different rows and never share LDS here).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
}

// One wave per row, SEL_ROWS rows per workgroup; no workgroup barrier, every reduction is a
// fixed-order wave reduction (deterministic).
constexpr int SEL_ROWS = 4;

// RU > 0: the row (M <= 64 * RU blocks) is held in registers, block 64u + lane in register u.
// RU == 0: the row is read from memory on every pass (any M).
template <int RU>
__global__ __launch_bounds__(256) void block_select_kernel(Problem P) {
  extern __shared__ uint32_t nbm_all[];   // local 3-D mode: one neighbourhood bitmap (Mpad/32 words) per wave
  __shared__ int hist_all[SEL_ROWS][256];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = blockIdx.x * SEL_ROWS + wv, bh = blockIdx.y;
  if (i >= P.Mq) return;                   // the whole wave: nothing below waits for other waves
  const int M = P.M, nu = (M + 63) >> 6, nw = P.Mpad >> 6;
  const size_t row = (size_t)bh * P.Mq + i;
  const float* s = P.scores + row * P.Mpad;
  int* kidx = P.kept_idx + row * M;
  uint8_t* mult = P.mult + row * P.Mpad;
  uint64_t* bm = P.kept_bm + row * nw;
  const bool lists = P.keep_lists != 0;

  const bool dense = i >= P.dense_q0 && i < P.dense_q1;
  if (dense || (P.mode == 0 && P.keep_all)) {
    for (int wd = lane; wd < nw; wd += 64) {
      const int nb = M - 64 * wd;       // blocks of this word that exist
      bm[wd] = nb >= 64 ? ~0ull : (nb > 0 ? ((1ull << nb) - 1ull) : 0ull);
    }
    if (lists)
      for (int j = lane; j < P.Mpad; j += 64) {
        if (j < M) kidx[j] = j;
        mult[j] = 0;
      }
    if (lane == 0) {
      P.kept_cnt[row] = M;
      P.extra_cnt[row] = 0;
    }
    return;
  }

  // the row's scores: block 64u + lane (padding columns up to Mpad exist but are never used)
  float sv[RU > 0 ? RU : 1];
  if constexpr (RU > 0) {
    if (P.mode != 2) {
#pragma unroll
      for (int u = 0; u < RU; ++u) sv[u] = u < nu ? s[64 * u + lane] : 0.f;
    }
  }
  auto score = [&](int u) -> float {
    if constexpr (RU > 0) return sv[u];
    else return s[64 * u + lane];
  };
  // loop bound over the row's 64-block groups: a constant (unrolled, registers indexed
  // statically) when the row is held in registers
  const int ulim = RU > 0 ? RU : nu;

  // forced blocks: the sinks and every key block overlapping this query block's tokens
  const int gi = i + P.q0;                       // global query block (rows are window-local)
  const int diag_lo = (gi * P.bq) / P.bk;
  const int diag_hi = min(M - 1, ((gi + 1) * P.bq - 1) / P.bk);
  auto forced = [&](int j) { return j < P.sink_blocks || (j >= diag_lo && j <= diag_hi); };

  float theta = 0.f;          // sol threshold
  uint32_t kstar = 0;         // sla: key of the k-th largest non-forced score
  int need_eq = 0;            // sla: how many scores equal to kstar to take (lowest index first)
  bool sla_any = false;
  uint32_t* nbm = nbm_all + (size_t)wv * (P.Mpad / 32);

  if (P.mode == 0) {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < ulim; ++u)
      if (u < nu && 64 * u + lane < M) acc += score(u);
    const float mu = wave_sum(acc) / static_cast<float>(M);
    float acc2 = 0.f;
#pragma unroll
    for (int u = 0; u < ulim; ++u)
      if (u < nu && 64 * u + lane < M) {
        const float dv = score(u) - mu;
        acc2 = fmaf(dv, dv, acc2);
      }
    const float var = wave_sum(acc2) / static_cast<float>(M);
    const float sd = sqrtf(var);
    theta = sd > 0.f ? fmaf(P.tau, sd, mu) : mu;
  } else if (P.mode == 2) {
    // one lane per query token: mark the blocks of the token and of its grid neighbours
    for (int wd = lane; wd < P.Mpad / 32; wd += 64) nbm[wd] = 0u;
    wave_lds_sync();
    const int hw = P.height * P.width;
    for (int q = lane; q < P.bq; q += 64) {
      const int p = gi * P.bq + q;
      const int t = p / hw, r = p - t * hw;
      const int y = r / P.width, x = r - y * P.width;
      auto mark = [&](int tok) {
        const int j = tok / P.bk;
        atomicOr(&nbm[j >> 5], 1u << (j & 31));
      };
      mark(p);
      if (t > 0) mark(p - hw);
      if (t + 1 < P.frames) mark(p + hw);
      if (y > 0) mark(p - P.width);
      if (y + 1 < P.height) mark(p + P.width);
      if (x > 0) mark(p - 1);
      if (x + 1 < P.width) mark(p + 1);
    }
    wave_lds_sync();
  } else {
    const int nforced = min(P.sink_blocks, M) + (diag_hi - diag_lo + 1) -
                        max(0, min(diag_hi, P.sink_blocks - 1) - diag_lo + 1);
    int need = min(M - nforced, P.k_sla);
    sla_any = need > 0;
    if (sla_any) {
      int* hist = hist_all[wv];
      uint32_t prefix = 0, pmask = 0;
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
#pragma unroll
        for (int q = 0; q < 4; ++q) hist[4 * lane + q] = 0;
        wave_lds_sync();
#pragma unroll
        for (int u = 0; u < ulim; ++u) {
          const int j = 64 * u + lane;
          if (u < nu && j < M && !forced(j)) {
            const uint32_t key = float_key(score(u));
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
          }
        }
        wave_lds_sync();
        // lane l holds digits 255-4l .. 252-4l; counts accumulate from the top digit down
        int c[4], sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c[q] = hist[255 - 4 * lane - q];
          sum += c[q];
        }
        int incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_up(incl, o);
          if (lane >= o) incl += t;
        }
        int ex = incl - sum, dig = -1, above = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (dig < 0 && ex < need && need <= ex + c[q]) {
            dig = 255 - 4 * lane - q;
            above = ex;
          }
          ex += c[q];
        }
        const uint64_t hit = __ballot(dig >= 0);     // exactly one lane
        const int src = static_cast<int>(__builtin_ctzll(hit));
        dig = __builtin_amdgcn_readlane(dig, src);
        above = __builtin_amdgcn_readlane(above, src);
        prefix |= static_cast<uint32_t>(dig) << shift;
        pmask |= 0xFFu << shift;
        need -= above;
        wave_lds_sync();                               // the histogram is cleared next pass
      }
      kstar = prefix;
      need_eq = need;
    }
  }

  // ordered compaction of the kept blocks, 64 at a time: the keep ballot is the bitmap word u,
  // which lane u keeps and writes at the end (one coalesced store per row)
  int base = 0, eq_base = 0;
  uint64_t myword = 0;
#pragma unroll
  for (int u = 0; u < ulim; ++u) {
    if (u < nu) {
      const int j = 64 * u + lane;
      bool keep = false, eq = false;
      if (j < M) {
        if (forced(j)) {
          keep = true;
        } else if (P.mode == 0) {
          keep = score(u) > theta;
        } else if (P.mode == 2) {
          keep = (nbm[j >> 5] >> (j & 31)) & 1u;
        } else if (sla_any) {
          const uint32_t key = float_key(score(u));
          keep = key > kstar;
          eq = key == kstar;
        }
      }
      const uint64_t eqm = __ballot(eq);
      if (eq && eq_base + lanes_below(eqm) < need_eq) keep = true;
      eq_base += __popcll(eqm);
      const uint64_t word = __ballot(keep);
      if (RU > 0) {
        myword = lane == u ? word : myword;
      } else if (lane == 0) {
        bm[u] = word;
      }
      if (lists) {
        if (keep) kidx[base + lanes_below(word)] = j;
        if (j < M) mult[j] = keep ? 0 : static_cast<uint8_t>(P.bk);
      }
      base += __popcll(word);
    }
  }
  if (RU > 0) {
    if (lane < nw) bm[lane] = lane < nu ? myword : 0ull;
  } else {
    for (int wd = nu + lane; wd < nw; wd += 64) bm[wd] = 0ull;
  }
  if (lists)
    for (int j = M + lane; j < P.Mpad; j += 64) mult[j] = 0;
  if (lane == 0) {
    P.kept_cnt[row] = base;
    P.extra_cnt[row] = 0;
  }
}

// The tile steps a head's pairs of query blocks would take under pairing stride
// s = blockIdx.y + 1: the kept-block union of each pair, summed (one workgroup per head and
// stride; the threads stride over the (pair, bitmap word) index space, so that every lane
// issues its own independent loads).
__global__ __launch_bounds__(256) void pair_plan_kernel(Problem P) {
  const int bh = blockIdx.x, s = blockIdx.y + 1;
  const int nd = P.dense_q1 - P.dense_q0, Ms = P.Mq - nd, npair = (Ms + 1) / 2;
  const int nw = P.Mpad / 64;
  const uint64_t* bm = P.kept_bm + (size_t)bh * P.Mq * nw;
  const int total = npair * nw;
  int acc = 0;
#pragma unroll 4
  for (int e = threadIdx.x; e < total; e += 256) {
    const int p = e / nw, w = e - p * nw;
    int a, b;
    sparse_pair(p, s, Ms, P.dense_q0, nd, &a, &b);
    uint64_t x = bm[(size_t)a * nw + w];
    if (b >= 0) x |= bm[(size_t)b * nw + w];
    acc += __popcll(x);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  __shared__ int part[4];
  if (threadIdx.x % 64 == 0) part[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0)
    P.pair_plan[(size_t)bh * PAIR_STRIDES + blockIdx.y] =
        (long long)part[0] + part[1] + part[2] + part[3];
}

hipError_t launch_pair_plan(const Problem& P, hipStream_t stream) {
  if (!P.pair_plan) return hipSuccess;
  hipLaunchKernelGGL(pair_plan_kernel, dim3(P.B * P.H, PAIR_STRIDES), dim3(256), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_block_select(const Problem& P, hipStream_t stream) {
  dim3 grid((P.Mq + SEL_ROWS - 1) / SEL_ROWS, P.B * P.H);
  const size_t lds = P.mode == 2 ? (size_t)SEL_ROWS * (P.Mpad / 32) * 4 : 0;
  // registers for the row: the smallest instance that holds it
  if (P.mode == 2 || P.M > 64 * 64)
    hipLaunchKernelGGL(block_select_kernel<0>, grid, dim3(256), lds, stream, P);
  else if (P.M <= 64 * 16)
    hipLaunchKernelGGL(block_select_kernel<16>, grid, dim3(256), lds, stream, P);
  else
    hipLaunchKernelGGL(block_select_kernel<64>, grid, dim3(256), lds, stream, P);
  return hipGetLastError();
}

}  // namespace solattn
