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
#include <algorithm>
#include <type_traits>

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

// One row (query block i of problem bh) by one wave.  RU > 0: the row's scores arrive in
// registers (rsv: block 64u + lane in register u, M <= 64 RU); RU == 0: the row is read from
// memory on every pass (any M).  hist: this wave's 256-bin histogram; nbm: its local 3-D bitmap.
// MODE: 0 sol, 1 sla, 2 local 3-D, -1 any (taken from P.mode at run time).
template <int RU, int MODE>
__device__ __forceinline__ void select_row(const Problem& P, int bh, int i, const float* rsv, int* hist,
                                           uint32_t* nbm) {
  const int mode = MODE >= 0 ? MODE : P.mode;
  const int lane = threadIdx.x & 63;
  const int M = P.M, nu = (M + 63) >> 6, nw = P.Mpad >> 6;
  const size_t row = (size_t)bh * P.Mq + i;
  const float* s = P.scores + row * P.Mpad;
  int* kidx = P.kept_idx + row * M;
  uint8_t* mult = P.mult + row * P.Mpad;
  uint64_t* bm = P.kept_bm + row * nw;
  const bool lists = P.keep_lists != 0;

  const bool dense = i >= P.dense_q0 && i < P.dense_q1;
  if (dense || (mode == 0 && P.keep_all)) {
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
  auto score = [&](int u) -> float {
    if constexpr (RU > 0) return rsv[u];
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

  if (mode == 0) {
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
  } else if (mode == 2) {
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
        } else if (mode == 0) {
          keep = score(u) > theta;
        } else if (mode == 2) {
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

// The sol row in registers, lean: per group of 64 blocks, a few per-lane compares and one ballot
// give the bitmap word, which lane 0 parks in LDS (wbuf, 64 words per wave); the row's words go
// out in one coalesced store at the end.  Only the last, partial group's deviation terms are
// masked: rsv holds the row's scores with every padding position zero (see the loads below).
template <int RU, bool LISTS>
__device__ __forceinline__ void select_row_sol(const Problem& P, int bh, int i, const float* rsv,
                                               uint64_t* wbuf) {
  const int lane = threadIdx.x & 63;
  const int M = P.M, nu = (M + 63) >> 6, nw = P.Mpad >> 6;
  const size_t row = (size_t)bh * P.Mq + i;
  uint64_t* bm = P.kept_bm + row * nw;
  constexpr bool lists = LISTS;
  const bool dense = i >= P.dense_q0 && i < P.dense_q1;
  if (dense || P.keep_all) {
    for (int wd = lane; wd < nw; wd += 64) {
      const int nb = M - 64 * wd;
      bm[wd] = nb >= 64 ? ~0ull : (nb > 0 ? ((1ull << nb) - 1ull) : 0ull);
    }
    if (lists)
      for (int j = lane; j < P.Mpad; j += 64) {
        if (j < M) P.kept_idx[row * M + j] = j;
        P.mult[row * P.Mpad + j] = 0;
      }
    if (lane == 0) {
      P.kept_cnt[row] = M;
      P.extra_cnt[row] = 0;
    }
    return;
  }
  const int gi = i + P.q0;
  const int diag_lo = (gi * P.bq) / P.bk;
  const int diag_hi = min(M - 1, ((gi + 1) * P.bq - 1) / P.bk);
  // mean (padding adds zeros), then the deviation over the M real blocks (two passes)
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < RU; ++u) acc += rsv[u];
  const float mu = wave_sum(acc) / static_cast<float>(M);
  float acc2 = 0.f;
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const float dv = 64 * u + lane < M ? rsv[u] - mu : 0.f;
    acc2 = fmaf(dv, dv, acc2);
  }
  const float sd = sqrtf(wave_sum(acc2) / static_cast<float>(M));
  const float theta = sd > 0.f ? fmaf(P.tau, sd, mu) : mu;
  int base = 0;
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    if (u < nu) {
      const int j = 64 * u + lane;
      const bool forced = j < P.sink_blocks || static_cast<unsigned>(j - diag_lo) <= static_cast<unsigned>(diag_hi - diag_lo);
      const bool keep = j < M && (rsv[u] > theta || forced);
      const uint64_t word = __ballot(keep);
      if (lane == 0) wbuf[u] = word;
      if (lists) {
        if (keep) P.kept_idx[row * M + base + lanes_below(word)] = j;
        if (j < M) P.mult[row * P.Mpad + j] = keep ? 0 : static_cast<uint8_t>(P.bk);
      }
      base += __popcll(word);
    }
  }
  wave_lds_sync();
  if (lane < nw) bm[lane] = lane < nu ? wbuf[lane] : 0ull;
  wave_lds_sync();                          // the words are read before the next row's writes
  if (lists)
    for (int j = M + lane; j < P.Mpad; j += 64) P.mult[row * P.Mpad + j] = 0;
  if (lane == 0) {
    P.kept_cnt[row] = base;
    P.extra_cnt[row] = 0;
  }
}

// The pairing sums start from zero: the selection kernels clear them (any thread may, the plan
// kernel runs after them on the stream).
__device__ __forceinline__ void clear_pair_plan(const Problem& P) {
  if (!P.pair_plan) return;
  const int n = P.B * P.H * PAIR_STRIDES;
  const int t = (blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
  const int nt = gridDim.x * gridDim.y * blockDim.x;
  for (int e = t; e < n; e += nt) P.pair_plan[e] = 0;
}

// Generic rows (sla, and sol rows longer than 2048 blocks; M <= 64 RU): one wave per row, its
// scores read once into registers.
template <int RU, int MODE>
__global__ __launch_bounds__(256) void block_select_reg_kernel(Problem P) {
  __shared__ int hist_all[SEL_ROWS][256];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long r = (long)blockIdx.x * SEL_ROWS + wv;
  clear_pair_plan(P);
  if (r >= (long)P.B * P.H * P.Mq) return;
  const int nu = (P.M + 63) >> 6;
  const float* s = P.scores + r * P.Mpad;
  // buffer loads bounded by the row's M scores: columns past M read zero, so the loads need
  // no branch and are all in flight together
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, static_cast<uint32_t>(P.M) * 4u);
  float v[RU];
#pragma unroll
  for (int u = 0; u < RU; ++u)
    v[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<uint32_t>(64 * u + lane) * 4u, 0, 0));
  select_row<RU, MODE>(P, static_cast<int>(r / P.Mq), static_cast<int>(r % P.Mq), v, hist_all[wv], nullptr);
}

// sol rows (M <= 64 RU): one wave per row, its scores read once into registers (padding zero),
// the lean row routine above.  A wave that walked several rows would let the compiler keep every
// group's lane conditions live across the walk (they do not change between rows), which costs
// more than the walk saves.
template <int RU, bool LISTS>
__global__ __launch_bounds__(256) void block_select_sol_kernel(Problem P) {
  __shared__ uint64_t wbuf_all[SEL_ROWS][64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long r = (long)blockIdx.x * SEL_ROWS + wv;
  clear_pair_plan(P);
  if (r >= (long)P.B * P.H * P.Mq) return;
  const int nu = (P.M + 63) >> 6;
  const float* s = P.scores + r * P.Mpad;
  // buffer loads bounded by the row's M scores: the padding columns past M read zero, and the
  // loads need no branch, so all of them are in flight together
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, static_cast<uint32_t>(P.M) * 4u);
  float v[RU];
#pragma unroll
  for (int u = 0; u < RU; ++u)
    v[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<uint32_t>(64 * u + lane) * 4u, 0, 0));
  select_row_sol<RU, LISTS>(P, static_cast<int>(r / P.Mq), static_cast<int>(r % P.Mq), v, wbuf_all[wv]);
}

// Memory path (the local 3-D pattern, and rows longer than 4096 blocks): one wave per row.
__global__ __launch_bounds__(256) void block_select_kernel(Problem P) {
  extern __shared__ uint32_t nbm_all[];   // local 3-D mode: one neighbourhood bitmap (Mpad/32 words) per wave
  __shared__ int hist_all[SEL_ROWS][256];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = blockIdx.x * SEL_ROWS + wv, bh = blockIdx.y;
  clear_pair_plan(P);
  if (i >= P.Mq) return;                   // the whole wave: nothing below waits for other waves
  select_row<0, -1>(P, bh, i, nullptr, hist_all[wv], nbm_all + (size_t)wv * (P.Mpad / 32));
}

// The tile steps a head's pairs of query blocks would take under pairing stride
// s = blockIdx.y + 1: the kept-block union of each pair, summed.  Workgroups (head, stride,
// chunk of pairs); the threads stride over the chunk's (pair, bitmap word) index space, so that
// every lane issues its own independent loads, and each workgroup adds its integer sum into the
// head's total (zeroed by the selection kernel before it; integer sums do not depend on order).
constexpr int PLAN_CHUNKS = 8;

__global__ __launch_bounds__(256) void pair_plan_kernel(Problem P) {
  const int bh = blockIdx.x, s = blockIdx.y + 1, chunk = blockIdx.z;
  const int nd = P.dense_q1 - P.dense_q0, Ms = P.Mq - nd, npair = (Ms + 1) / 2;
  const int nw = P.Mpad / 64;
  const uint64_t* bm = P.kept_bm + (size_t)bh * P.Mq * nw;
  const int per = (npair + PLAN_CHUNKS - 1) / PLAN_CHUNKS;
  const int p0 = chunk * per, p1 = min(npair, p0 + per);
  const int total = max(0, p1 - p0) * nw;
  int acc = 0;
#pragma unroll 4
  for (int e = threadIdx.x; e < total; e += 256) {
    const int p = p0 + e / nw, w = e % nw;
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
  if (threadIdx.x == 0 && total > 0)
    atomicAdd(reinterpret_cast<unsigned long long*>(P.pair_plan + (size_t)bh * PAIR_STRIDES + blockIdx.y),
              static_cast<unsigned long long>(part[0] + part[1] + part[2] + part[3]));
}

hipError_t launch_pair_plan(const Problem& P, hipStream_t stream) {
  if (!P.pair_plan) return hipSuccess;
  hipLaunchKernelGGL(pair_plan_kernel, dim3(P.B * P.H, PAIR_STRIDES, PLAN_CHUNKS), dim3(256), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_block_select(const Problem& P, hipStream_t stream) {
  dim3 grid((P.Mq + SEL_ROWS - 1) / SEL_ROWS, P.B * P.H);
  const size_t lds = P.mode == 2 ? (size_t)SEL_ROWS * (P.Mpad / 32) * 4 : 0;
  if (P.mode == 2 || P.M > 64 * 64) {
    hipLaunchKernelGGL(block_select_kernel, grid, dim3(256), lds, stream, P);
    return hipGetLastError();
  }
  // registers for the row: the smallest instance that holds it, one wave per row
  const long rows = (long)P.B * P.H * P.Mq;
  const int wgs = static_cast<int>((rows + SEL_ROWS - 1) / SEL_ROWS);
  auto go = [&](auto ru) {
    constexpr int RU = decltype(ru)::value;
    if (P.mode == 0 && RU <= 32) {
      constexpr int R = RU <= 32 ? RU : 32;
      if (!P.keep_lists) hipLaunchKernelGGL((block_select_sol_kernel<R, false>), dim3(wgs), dim3(256), 0, stream, P);
      else hipLaunchKernelGGL((block_select_sol_kernel<R, true>), dim3(wgs), dim3(256), 0, stream, P);
    } else if (P.mode == 0) {
      hipLaunchKernelGGL((block_select_reg_kernel<RU, 0>), dim3(wgs), dim3(256), 0, stream, P);
    } else {
      hipLaunchKernelGGL((block_select_reg_kernel<RU, 1>), dim3(wgs), dim3(256), 0, stream, P);
    }
  };
  if (P.M <= 64 * 16) go(std::integral_constant<int, 16>{});
  else if (P.M <= 64 * 32) go(std::integral_constant<int, 32>{});
  else go(std::integral_constant<int, 64>{});
  return hipGetLastError();
}

}  // namespace solattn
