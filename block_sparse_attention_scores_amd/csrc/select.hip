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
// The kept set is written twice: as an ascending index list and as a bitmap (bit j of word
// j/64), which the attention kernel walks without touching memory.
// One 256-thread workgroup per row; all reductions have a fixed order, so results are
// deterministic.  Also writes each block's centroid multiplicity (0 = attended exactly).
#include "common.h"
#include "launch.h"

namespace solattn {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum over the 256 threads, identical result on every thread.
__device__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return ((sh[0] + sh[1]) + sh[2]) + sh[3];
}

// Inclusive prefix sum over the 256 threads (thread order).  *total gets the sum.
__device__ int block_scan_incl(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x / 64;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  __syncthreads();
  if (lane == 63) sh[w] = v;
  __syncthreads();
  int before = 0;
  for (int u = 0; u < w; ++u) before += sh[u];
  *total = sh[0] + sh[1] + sh[2] + sh[3];
  return v + before;
}

__global__ __launch_bounds__(256) void block_select_kernel(Problem P) {
  extern __shared__ uint32_t nbm[];   // local 3-D mode: neighbourhood bitmap, Mpad/32 words
  __shared__ float fsh[4];
  __shared__ int ish[4];
  __shared__ int hist[256];
  __shared__ int pick[2];

  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int M = P.M;
  const size_t row = (size_t)bh * P.Mq + i;
  const float* s = P.scores + row * M;
  int* kidx = P.kept_idx + row * M;
  uint8_t* mult = P.mult + row * P.Mpad;
  float* cb = P.cbias + row * P.Mpad;
  uint64_t* bm = P.kept_bm + row * (P.Mpad / 64);
  const int lane = tid & 63, wv = tid >> 6;
  // centroid logit offset in raw-score units: ln(block size) / scale
  const float log2_bk = __logf(static_cast<float>(P.bk)) / P.scale;

  const bool dense = i >= P.dense_q0 && i < P.dense_q1;
  if (dense || (P.mode == 0 && P.keep_all)) {
    for (int j = tid; j < P.Mpad; j += 256) {
      if (j < M) kidx[j] = j;
      mult[j] = 0;
      cb[j] = -__builtin_inff();
    }
    for (int wd = tid; wd < P.Mpad / 64; wd += 256) {
      const int nb = M - 64 * wd;       // blocks of this word that exist
      bm[wd] = nb >= 64 ? ~0ull : ((1ull << nb) - 1ull);
    }
    if (tid == 0) {
      P.kept_cnt[row] = M;
      P.extra_cnt[row] = 0;
    }
    return;
  }

  // forced blocks: the sinks and every key block overlapping this query block's tokens
  const int gi = i + P.q0;                       // global query block (rows are window-local)
  const int diag_lo = (gi * P.bq) / P.bk;
  const int diag_hi = min(M - 1, ((gi + 1) * P.bq - 1) / P.bk);
  auto forced = [&](int j) { return j < P.sink_blocks || (j >= diag_lo && j <= diag_hi); };

  float theta = 0.f;          // sol threshold
  uint32_t kstar = 0;         // sla: key of the k-th largest non-forced score
  int need_eq = 0;            // sla: how many scores equal to kstar to take (lowest index first)
  bool sla_any = false;

  if (P.mode == 0) {
    float acc = 0.f;
    for (int j = tid; j < M; j += 256) acc += s[j];
    const float mu = block_sum(acc, fsh) / static_cast<float>(M);
    float acc2 = 0.f;
    for (int j = tid; j < M; j += 256) {
      const float dv = s[j] - mu;
      acc2 = fmaf(dv, dv, acc2);
    }
    const float var = block_sum(acc2, fsh) / static_cast<float>(M);
    const float sd = sqrtf(var);
    theta = sd > 0.f ? fmaf(P.tau, sd, mu) : mu;
  } else if (P.mode == 2) {
    // one thread per query token: mark the blocks of the token and of its grid neighbours
    for (int wd = tid; wd < P.Mpad / 32; wd += 256) nbm[wd] = 0u;
    __syncthreads();
    if (tid < P.bq) {
      const int hw = P.height * P.width;
      const int p = gi * P.bq + tid;
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
    __syncthreads();
  } else {
    const int nforced = min(P.sink_blocks, M) + (diag_hi - diag_lo + 1) -
                        max(0, min(diag_hi, P.sink_blocks - 1) - diag_lo + 1);
    int need = min(M - nforced, P.k_sla);
    sla_any = need > 0;
    if (sla_any) {
      uint32_t prefix = 0, pmask = 0;
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        hist[tid] = 0;
        __syncthreads();
        for (int j = tid; j < M; j += 256) {
          if (forced(j)) continue;
          const uint32_t key = float_key(s[j]);
          if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        // thread t looks at digit 255-t; counts accumulate from the top digit down
        const int c = hist[255 - tid];
        int total;
        const int incl = block_scan_incl(c, ish, &total);
        const int excl = incl - c;
        if (excl < need && need <= incl) {
          pick[0] = 255 - tid;
          pick[1] = excl;
        }
        __syncthreads();
        prefix |= static_cast<uint32_t>(pick[0]) << shift;
        pmask |= 0xFFu << shift;
        need -= pick[1];
        __syncthreads();
      }
      kstar = prefix;
      need_eq = need;
    }
  }

  // ordered compaction of the kept blocks
  int base = 0, eq_base = 0;
  for (int j0 = 0; j0 < M; j0 += 256) {
    const int j = j0 + tid;
    bool keep = false, eq = false;
    if (j < M) {
      if (forced(j)) {
        keep = true;
      } else if (P.mode == 0) {
        keep = s[j] > theta;
      } else if (P.mode == 2) {
        keep = (nbm[j >> 5] >> (j & 31)) & 1u;
      } else if (sla_any) {
        const uint32_t key = float_key(s[j]);
        keep = key > kstar;
        eq = key == kstar;
      }
    }
    int tot_eq;
    const int eq_rank = block_scan_incl(eq ? 1 : 0, ish, &tot_eq) - (eq ? 1 : 0) + eq_base;
    if (eq && eq_rank < need_eq) keep = true;
    eq_base += tot_eq;
    int tot;
    const int pos = block_scan_incl(keep ? 1 : 0, ish, &tot) - (keep ? 1 : 0) + base;
    if (keep) kidx[pos] = j;
    const uint64_t word = __ballot(keep);
    const int wd = (j0 >> 6) + wv;
    if (lane == 0 && wd < P.Mpad / 64) bm[wd] = word;
    if (j < M) {
      mult[j] = keep ? 0 : static_cast<uint8_t>(P.bk);
      cb[j] = keep ? -__builtin_inff() : log2_bk;
    }
    base += tot;
  }
  for (int j = M + tid; j < P.Mpad; j += 256) {
    mult[j] = 0;
    cb[j] = -__builtin_inff();
  }
  if (tid == 0) {
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
  dim3 grid(P.Mq, P.B * P.H);
  const size_t lds = P.mode == 2 ? (size_t)(P.Mpad / 32) * 4 : 0;
  hipLaunchKernelGGL(block_select_kernel, grid, dim3(256), lds, stream, P);
  return hipGetLastError();
}

}  // namespace solattn
