// extra_select: for each sparse query block i, the up to E = extra_tokens individual keys with
// the highest q̄_i . k_t among tokens outside its kept blocks, ties to the lower token (node
// docs, common inputs table, extra_tokens row: extra high-score tokens each query block
// attends beyond its selected blocks).
//
// Pass 1 keeps, per query block, every key whose score reaches a threshold, in candidate lists
// in the workspace.  The sampled pass (16-bit tensors) holds the threshold at a seed taken from
// a sample of the keys and sends a query block whose lists could overflow to the exact pass;
// the exact pass and the fp32 pass raise the threshold whenever a list is cut back to its E best
// entries (by radix selection on (score, token)): any list's E-th best is a lower bound of the
// final E-th best, so no key of the final selection is ever dropped.
//   16-bit tensors (extra_seed_kernel, extra_tile_kernel): scores come from the 32x32x16 bf16
//   matrix instruction with q̄ split into two bf16 parts (hi + lo), accurate to ~2^-17
//   relative (fp32-like), while the keys are exact bf16; a workgroup owns 128 query blocks and
//   shares key tiles staged in LDS among them (described below).
//   fp32 (extra_select_kernel): a workgroup of 4 waves owns 32 query blocks of one head and one
//   slice of the token range; the waves take turns over 32-token steps with exact fp32 dot
//   products, each wave with its own candidate list per query block and one shared threshold
//   per query block in LDS.
//
// Pass 2 (extra_merge_kernel).  One wave per query block takes the best E of the partial lists
// (one per wave and slice), ranks them by token, writes them out, and takes the chosen tokens
// out of their blocks' centroid terms.
#include <type_traits>
#include <utility>

#include "common.h"
#include "launch.h"

namespace solattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int XR = EXTRA_GROUP_F32;   // query blocks per workgroup (fp32 first pass)

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int XSTEP = 32;   // tokens per wave step

// Fill of a candidate list of the 16-bit sampled pass one of whose halves could have
// overflowed (its query block goes to the exact pass).
constexpr int EXTRA_PART_OVERFLOW = -1;
// A half list that could overflow holds at least EXTRA_CAP / 2 - 32 candidates at or above the
// seed, which must be at least E for the exact pass to start from the seed.
static_assert(EXTRA_CAP / 2 - 32 >= MAX_EXTRA, "an overflowing half list holds E candidates");

// Median of three unsigned values (one v_med3_u32).
__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

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

// Radix selection over 32-bit keys held NPL per lane (valid[] marks live entries).  Finds the
// `need`-th largest key K* and returns it; *need_eq = how many entries equal to K* are taken.
// *cnt_eq = how many entries equal K*.  The passes start below the bits all live keys share,
// so keys of similar magnitude take few passes and spread over many histogram bins.
template <int NPL>
__device__ uint32_t wave_radix_select(const uint32_t* key, const bool* valid, int need, int* hist,
                                      int* scratch, int* need_eq, int* cnt_eq) {
  const int l = threadIdx.x & 63;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  int n = 0;
#pragma unroll
  for (int u = 0; u < NPL; ++u)
    if (valid[u]) {
      kmin = min(kmin, key[u]);
      kmax = max(kmax, key[u]);
      ++n;
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), o)));
    kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), o)));
    n += __shfl_xor(n, o);
  }
  const uint32_t diff = kmin ^ kmax;
  if (diff == 0u) {                         // all live keys equal
    *need_eq = need;
    *cnt_eq = n;
    return kmax;
  }
  const int hb = 31 - __builtin_clz(diff);
  uint32_t pmask = hb == 31 ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = kmax & pmask;
  int at = 0;
  for (int top = hb; top >= 0; top -= 8) {
    const int shift = top >= 7 ? top - 7 : 0;
    const uint32_t dmask = (2u << (top - shift)) - 1u;
#pragma unroll
    for (int q = 0; q < 4; ++q) hist[4 * l + q] = 0;
    wave_sync();
#pragma unroll
    for (int u = 0; u < NPL; ++u)
      if (valid[u] && (key[u] & pmask) == prefix) atomicAdd(&hist[(key[u] >> shift) & dmask], 1);
    wave_sync();
    int above;
    const int dg = wave_pick_digit(hist, need, &above, &at, scratch);
    prefix |= static_cast<uint32_t>(dg) << shift;
    pmask |= dmask << shift;
    need -= above;
  }
  *need_eq = need;
  *cnt_eq = at;
  return prefix;
}

// Marks in keep[] the E best entries under (score desc, token asc) of NPL-per-lane entries
// (all valid entries if there are at most E).  Returns the key of the E-th best (0 if fewer).
template <int NPL>
__device__ uint32_t wave_best(const uint32_t* key, const uint32_t* tok, const bool* valid, int cnt,
                              int E, int* hist, int* scratch, bool* keep) {
  if (cnt <= E) {
#pragma unroll
    for (int u = 0; u < NPL; ++u) keep[u] = valid[u];
    return 0u;
  }
  int need_eq, cnt_eq;
  const uint32_t kstar = wave_radix_select<NPL>(key, valid, E, hist, scratch, &need_eq, &cnt_eq);
  uint32_t tmax = 0xFFFFFFFFu;   // largest token taken among those tying K*
  if (need_eq < cnt_eq) {
    uint32_t k2[NPL];
    bool v2[NPL];
#pragma unroll
    for (int u = 0; u < NPL; ++u) {
      v2[u] = valid[u] && key[u] == kstar;
      k2[u] = ~tok[u];            // larger k2 = smaller token
    }
    int ne2, ce2;
    tmax = ~wave_radix_select<NPL>(k2, v2, need_eq, hist, scratch, &ne2, &ce2);
  }
#pragma unroll
  for (int u = 0; u < NPL; ++u)
    keep[u] = valid[u] && (key[u] > kstar || (key[u] == kstar && tok[u] <= tmax));
  return kstar;
}

// Cut one wave buffer (cnt > E entries) to its E best, in place; returns the E-th best key.
__device__ uint32_t wave_cut(uint2* buf, int cnt, int E, int* hist, int* scratch) {
  constexpr int NPL = EXTRA_CAP / 64;
  const int l = threadIdx.x & 63;
  uint32_t key[NPL], tok[NPL];
  bool valid[NPL], keep[NPL];
#pragma unroll
  for (int u = 0; u < NPL; ++u) {
    const int p = l + 64 * u;
    valid[u] = p < cnt;
    const uint2 e = valid[u] ? buf[p] : make_uint2(0u, 0u);
    key[u] = float_key(__uint_as_float(e.x));
    tok[u] = e.y;
  }
  const uint32_t kstar = wave_best<NPL>(key, tok, valid, cnt, E, hist, scratch, keep);
  // every lane holds its entries in registers now; write the survivors to the front
  int base = 0;
#pragma unroll
  for (int u = 0; u < NPL; ++u) {
    const uint64_t m = __ballot(keep[u]);
    const int pos = base + __popcll(m & ((1ull << l) - 1ull));
    if (keep[u]) buf[pos] = make_uint2(__float_as_uint(key_float(key[u])), tok[u]);
    base += __popcll(m);
  }
  return kstar;
}

// Sample used to seed the thresholds: runs of 32 consecutive tokens spread over the sequence
// (run s of n: half a key block near s*M/n, offset by a fixed jitter), SAMPLE_STEPS of them or
// one per 1024 tokens, whichever is more (at most 4 * SAMPLE_STEPS).
// Each lane keeps its SAMPLE_KEEP best candidate scores; the seed of a query block is the r-th
// best of the kept scores, with r chosen so that about SAMPLE_MARGIN * E candidates are
// expected at or above it (r at most the 64 kept scores).
constexpr int SAMPLE_STEPS = 64;
constexpr int SAMPLE_KEEP = 8;
constexpr int SAMPLE_MARGIN = 4;

__device__ __forceinline__ int sample_run(int s, int nsteps, int M) {
  const int span = max(1, M / nsteps);
  const int j = static_cast<int>((static_cast<long>(s) * M) / nsteps) + (s * 37) % span;
  return j * 64 + ((nsteps > M) ? 32 * (s & 1) : 0);
}

// Pass 1, fp32.  repair = 0: every sparse query block, with thresholds seeded from the sample.
// repair = 1: only the query blocks the merge flagged (fewer candidates than it needs), with
// the threshold at its minimum, so that every candidate competes (the exact selection).
template <int D>
__global__ __launch_bounds__(256, 2) void extra_select_kernel(Problem P, int repair) {
  __shared__ uint32_t thr[XR];            // shared threshold keys: append when key >= thr
  __shared__ int whist[4][256];
  __shared__ int wscr[4][4];
  __shared__ float qs[XR][D];
  __shared__ uint32_t samp[XR][8 * SAMPLE_KEEP];   // per query block: the best sample keys of 8 lanes
  __shared__ int scnt[XR];                          // sample candidates per query block
  __shared__ int any_row;

  const int bh = blockIdx.y, i0 = blockIdx.x * XR, slice = blockIdx.z;
  const int S = P.extra_slices;
  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int rl = l % 32, i = i0 + rl;
  const int E = P.extra, N = P.N;
  const int b = bh / P.H, h = bh % P.H;
  const size_t grow = (size_t)bh * P.Mq + (i < P.Mq ? i : 0);
  bool row_ok = i < P.Mq && !(i >= P.dense_q0 && i < P.dense_q1);
  if (repair) row_ok = row_ok && P.extra_flag[grow] != 0;
  if (repair) {
    // nothing to do unless one of this group's query blocks was flagged
    if (tid == 0) any_row = 0;
    __syncthreads();
    if (row_ok) any_row = 1;
    __syncthreads();
    if (!any_row) return;
  }
  const uint64_t* bmrow = P.kept_bm + grow * (P.Mpad / 64);
  const float* kbase = static_cast<const float*>(P.k.p) + (int64_t)b * P.k.sb + (int64_t)h * P.k.sh;
  const int ts = (((N + S - 1) / S) + 127) / 128 * 128;       // tokens per slice
  const int t_lo = slice * ts, t_hi = min(N, t_lo + ts);

  if (tid < XR) thr[tid] = 0u;

  // q̄ of the group's query blocks, in LDS
  for (int u = tid; u < XR * D; u += 256) {
    const int r = u / D, e = u % D;
    qs[r][e] = (i0 + r < P.Mq) ? P.qbar[((size_t)bh * P.Mq + i0 + r) * D + e] : 0.f;
  }
  __syncthreads();

  // scores of 32 consecutive tokens from tw for this lane's query block: register r holds token
  // tw + (r/4)*8 + (l/32)*4 + r%4 (the layout of the 16-bit pass's accumulator)
  uint8_t mflag = 0;      // 1: the block of token tw is not kept (its tokens are candidates)
  auto load_keys = [&](int tw) {
    const int j = tw >> 6;
    mflag = row_ok ? static_cast<uint8_t>(((bmrow[j >> 6] >> (j & 63)) & 1ull) ^ 1ull) : 0;
  };
  auto scores = [&](int tw, float* acc, auto&& prefetch) {
#pragma unroll 1
    for (int r = 0; r < 16; ++r) {
      const int tk = tw + (r / 4) * 8 + (l / 32) * 4 + (r % 4);
      const float* kr = kbase + (int64_t)tk * P.k.sn;
      float sc = 0.f;
#pragma unroll 8
      for (int e = 0; e < D; ++e) sc = fmaf(qs[rl][e], kr[e], sc);
      acc[r] = sc;
    }
    prefetch();
  };

  if (!repair) {
    // ---- seed the thresholds.  The sample's candidates are candidates of the query block, so
    // when at least E candidates score at or above the seed, the E best all do; the merge checks
    // that count and sends the query block to the exact repair pass otherwise.
    if (tid < XR) scnt[tid] = 0;
    __syncthreads();
    // the sample grows with the sequence (one run per 1024 tokens, 64 to 256 runs), so that its
    // share of a long sequence's candidates, and with it the rank used below, stays large
    const int nsteps = min(2 * P.M, min(4 * SAMPLE_STEPS, max(SAMPLE_STEPS, N / 1024)));
    uint32_t best[SAMPLE_KEEP];             // this lane's best sample keys, descending
#pragma unroll
    for (int q = 0; q < SAMPLE_KEEP; ++q) best[q] = 0u;
    int nsamp = 0;
#pragma unroll 1
    for (int st = w; st < nsteps; st += 4) {
      const int tw = sample_run(st, nsteps, P.M);
      float acc[16];
      load_keys(tw);
      const bool cand_s = mflag > 0;
      scores(tw, acc, [] {});
      if (cand_s) {
        nsamp += 16;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          uint32_t k = float_key(acc[r]);
#pragma unroll
          for (int q = 0; q < SAMPLE_KEEP; ++q) {
            const uint32_t hi = max(best[q], k), lo = min(best[q], k);
            best[q] = hi;
            k = lo;
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < SAMPLE_KEEP; ++q) samp[rl][(w * 2 + l / 32) * SAMPLE_KEEP + q] = best[q];
    if (nsamp) atomicAdd(&scnt[rl], nsamp);
    __syncthreads();
    // the r-th best kept key is the largest key with at least r kept keys >= it
    constexpr int NK = 8 * SAMPLE_KEEP;
    for (int task = tid; task < XR * NK; task += 256) {
      const int rr = task / NK, a = task % NK;
      const int ii = i0 + rr;
      if (ii >= P.Mq || (ii >= P.dense_q0 && ii < P.dense_q1)) continue;
      const int ncand = N - P.bk * P.kept_cnt[(size_t)bh * P.Mq + ii];
      if (ncand <= 0) continue;
      const long want = (static_cast<long>(SAMPLE_MARGIN) * E * scnt[rr] + ncand - 1) / ncand;
      const int r = static_cast<int>(min(static_cast<long>(NK), max(1l, want)));
      const uint32_t v = samp[rr][a];
      int cge = 0;
#pragma unroll 8
      for (int bq = 0; bq < NK; ++bq) cge += samp[rr][bq] >= v ? 1 : 0;
      if (cge >= r) atomicMax(&thr[rr], v);
    }
    __syncthreads();
  }

  // candidate stores go through a buffer resource over this wave's buffers of the group's
  // query blocks; a lane with nothing to store uses an offset past the end, which the buffer
  // bounds check discards.  Every step that stores issues the same number of stores.
  const uint32_t row_stride = (uint32_t)S * 4u * EXTRA_CAP * 8u;        // bytes between query blocks
  const int nvalid = min(XR, P.Mq - i0);
  const __amdgpu_buffer_rsrc_t brsrc =
      make_rsrc(P.extra_buf + (((size_t)bh * P.Mq + i0) * S + slice) * 4 * EXTRA_CAP + (size_t)w * EXTRA_CAP,
            (uint32_t)(nvalid - 1) * row_stride + EXTRA_CAP * 8u);
  const uint32_t my_off = (uint32_t)rl * row_stride;
  // fill of this wave's buffer for the lane's query block; lanes l and l+32 share the block
  // and keep the same count
  int cnt = 0;
  // the next step's key fragments are loaded while this step is scored
  if (t_lo + XSTEP * w < t_hi) load_keys(t_lo + XSTEP * w);
#pragma unroll 1
  for (int tw = t_lo + XSTEP * w; tw < t_hi; tw += 4 * XSTEP) {
    float acc[16];
    const bool cand = mflag > 0;
    scores(tw, acc, [&] {
      if (tw + 4 * XSTEP < t_hi) load_keys(tw + 4 * XSTEP);
    });
    const uint32_t th = thr[rl];
    uint32_t bits = 0;
    if (cand) {
#pragma unroll
      for (int r = 0; r < 16; ++r) bits |= (float_key(acc[r]) >= th ? 1u : 0u) << r;
    }
    if (__ballot(bits != 0) == 0) continue;
    // append: lane l first, then its partner l+32, each in register order
    const int mine = __popc(bits);
    const int other = __shfl_xor(mine, 32);
    const int pos0 = cnt + (l < 32 ? 0 : other);
    cnt += mine + other;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tk = tw + (r / 4) * 8 + (l / 32) * 4 + (r % 4);
      const uint32_t off = ((bits >> r) & 1u)
                               ? my_off + (uint32_t)(pos0 + __popc(bits & ((1u << r) - 1u))) * 8u
                               : 0xFFFFFFF0u;
      u32x2 v2;
      v2.x = __float_as_uint(acc[r]);
      v2.y = static_cast<uint32_t>(tk);
      __builtin_amdgcn_raw_buffer_store_b64(v2, brsrc, off, 0, 0);
    }
    // cut the buffers that the next step could overflow
    uint64_t m = __ballot(l < 32 && cnt > EXTRA_CAP - XSTEP);
    if (m) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // this wave's stores, visible
      while (m) {
        const int rr = __builtin_ctzll(m);
        m &= m - 1;
        uint2* rb = P.extra_buf + ((((size_t)bh * P.Mq + i0 + rr) * S + slice) * 4 + w) * EXTRA_CAP;
        const int crr = __shfl(cnt, rr);
        const uint32_t kth = wave_cut(rb, crr, E, whist[w], wscr[w]);
        if (l == 0) atomicMax(&thr[rr], kth);
        if (rl == rr) cnt = E;
        wave_sync();
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  // publish the buffer fills; the merge pass takes the best E over all lists of a query block
  // (in the repair pass only for the flagged query blocks, whose lists were rebuilt)
  for (int rr = 0; rr < XR; ++rr) {
    const int ii = i0 + rr;
    if (ii >= P.Mq) break;
    const size_t row = (size_t)bh * P.Mq + ii;
    const int c = __shfl(cnt, rr);
    const bool ok = __shfl(row_ok ? 1 : 0, rr) != 0;
    if (l == 0 && (!repair || ok)) P.extra_part[(row * S + slice) * 4 + w] = c;
  }
}

// ---------------------------------------------------------------------- 16-bit first pass
//
// A workgroup owns EXTRA_GROUP_BF16 = 128 query blocks of one head (wave w: blocks
// i0 + 32w .. i0 + 32w + 31, one per accumulator column) and one token slice.  Key tiles of
// XTOK = 64 tokens are copied into LDS with buffer-to-LDS loads (chunk-swizzled rows) and read by
// all four waves as the A operand, so every key byte fetched serves 128 query blocks.  XNB
// buffers keep XNB - 1 tiles in flight: the wait before a tile leaves the later tiles' copies
// outstanding (loads complete in issue order) and the barrier after it orders LDS only, so
// nothing drains the queue.  A query block belongs to one wave, so its threshold lives in
// registers; its candidates go to the list of its (query block, slice), stored one tile late
// so that the stores complete while the next tile is scored.  The seeded thresholds come from
// extra_seed_kernel, once per query block for all slices.

constexpr int XTOK = 64;                   // tokens per key tile (2 steps of 32)
constexpr int XNB = 4;                     // LDS tile buffers

template <int D>
struct ExtraSmem {
  uint16_t k[XNB][XTOK * D];
  uint32_t fl[XNB][2][256];  // per tile and run: each thread's kept-bitmap dword of the run's block
  int hist[4][256];
  int scr[4][4];
  int any;
};

// The sampled pass: three tile buffers (two tiles in flight), one flag run per tile and no cut
// scratch, so that three workgroups fit in a compute unit's LDS.
constexpr int XNB_S = 3;
template <int D>
struct ExtraSampledSmem {
  uint16_t k[XNB_S][XTOK * D];
  uint32_t fl[XNB_S][1][256];
  int any;
};

// The seeds' pass: three tile buffers as well; a tile's two sampled runs share one flag array
// (lane l < 32 of wave w holds its query block's bitmap dword of run 0's key block at 64w + l,
// lane l + 32 that of run 1's block at 64w + 32 + l), so three workgroups fit a compute unit.
template <int D>
struct ExtraSeedSmem {
  uint16_t k[XNB_S][XTOK * D];
  uint32_t fl[XNB_S][256];
};

// Barrier for the tile loop: every wave has waited for its own copies of the tile (vmcnt), so
// after it the whole tile is in LDS; the memory clobber keeps LDS accesses on their side.  No
// memory fence: a fence would wait for every outstanding copy, including the later tiles'.
__device__ __forceinline__ void tile_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Wait until at most `later` tiles' copies (OPS per tile and thread) are outstanding.
template <int OPS>
__device__ __forceinline__ void wait_tiles(int later) {
  if (later >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * OPS) : "memory");
  else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(OPS) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Asynchronous 4-byte global -> LDS copy with a scalar offset: lane l's dword lands at
// `wave_dst` + 4*l.
__device__ __forceinline__ void buf_to_lds4s(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                             void* wave_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(wave_dst), 4, voff, soff, 0, 0);
}

// Asynchronous 4-byte global -> LDS copy: lane l's dword lands at `wave_dst` + 4*l.
__device__ __forceinline__ void buf_to_lds4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, void* wave_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(wave_dst), 4, voff, 0, 0, 0);
}

// Candidate flags travel with the key tiles: each thread copies the dword of its query block's
// kept bitmap that holds key block j (a block is a candidate source when its bit is clear).
struct FlagCopy {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t row_off;                        // byte offset of the lane's bitmap row (past the end if none)
  __device__ void init(const Problem& P, int bh, int i) {
    const uint32_t nwb = static_cast<uint32_t>(P.Mpad / 64) * 8u;
    rs = make_rsrc(P.kept_bm + (size_t)bh * P.Mq * (P.Mpad / 64), static_cast<uint32_t>(P.Mq) * nwb);
    row_off = static_cast<uint32_t>(i < P.Mq ? i : P.Mq) * nwb;
  }
  __device__ void issue(int j, uint32_t* dst) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    buf_to_lds4(rs, row_off + static_cast<uint32_t>(j >> 5) * 4u, dst + 64 * w);
  }
  __device__ static bool kept(const uint32_t* src, int j) {
    return (src[threadIdx.x] >> (j & 31)) & 1u;
  }
  // both runs of a tile in one copy: lanes 0-31 take key block j0's dword, lanes 32-63 j1's
  __device__ void issue_pair(int j0, int j1, uint32_t* dst) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int j = (threadIdx.x & 63) < 32 ? j0 : j1;
    buf_to_lds4(rs, row_off + static_cast<uint32_t>(j >> 5) * 4u, dst + 64 * w);
  }
  // run q's flag of this lane's query block from an issue_pair copy
  __device__ static bool kept_pair(const uint32_t* src, int q, int j) {
    const int t = threadIdx.x;
    return (src[(t & ~63) + 32 * q + (t & 31)] >> (j & 31)) & 1u;
  }
};

// float -> bfloat16 bits, round to nearest even, NaN kept a NaN; both results are computed and
// one selected, so a loop of these has no branch.
__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return static_cast<uint16_t>((u & 0x7fffffffu) > 0x7f800000u ? ((u >> 16) | 0x40u) : r);
}

// The per-lane part shared by the two kernels: q̄ split into bf16 hi + lo fragments for this
// lane's query block (zero past the last one), the tile loader and the score products.
template <int D>
struct ExtraTiles {
  static constexpr int KCH = D / 8;                    // 16-byte chunks per key row
  static constexpr int PT = XTOK * KCH / 256;          // chunk copies per thread per tile
  bf16x8_t qhi[D / 16], qlo[D / 16];
  uint32_t ak;                                         // lane's A-fragment byte offset in a 32-row step
  uint32_t ksn_b;

  // row: a valid row of qbar (callers clamp it); has_row = false zeroes the fragments.  The
  // loads are unconditional 16-byte loads, all in flight together, and the conversion has no
  // branch, so the set-up costs one memory round trip.
  __device__ void init(const Problem& P, size_t row, bool has_row) {
    const float* qb = P.qbar + row * D;
    const int l = threadIdx.x & 63;
    float4 x4[D / 8];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const float4* src = reinterpret_cast<const float4*>(qb + 16 * ks + 8 * (l / 32));
      x4[2 * ks] = src[0];
      x4[2 * ks + 1] = src[1];
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4 v = x4[2 * ks + e / 4];
        const float c = (e % 4 == 0) ? v.x : (e % 4 == 1) ? v.y : (e % 4 == 2) ? v.z : v.w;
        const float x = has_row ? c : 0.f;
        const uint16_t hb = bf16_bits_rne(x);
        const uint16_t lb = bf16_bits_rne(x - bf16_to_f32(hb));
        qhi[ks][e] = __builtin_bit_cast(__bf16, hb);
        qlo[ks][e] = __builtin_bit_cast(__bf16, lb);
      }
    }
    const int c32 = l % 32, h32 = l / 32;
    ak = c32 * (D * 2) + 16 * kswz<D>(c32, h32);
    ksn_b = static_cast<uint32_t>(P.k.sn) * 2u;
  }

  // Copy key rows into `dst`: the tile is 2 runs of 32 rows; run(q) gives the first key row of
  // run q and the bytes its buffer resource covers (rows past them read zero).
  template <typename Run>
  __device__ void issue(uint16_t* dst, Run&& run) {
    const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int s = (u * 4 + w) * 64 + l;               // 16-byte slot; the wave's 64 slots are
      const int r = s / KCH, c = s % KCH;               // rows of one run (4 or 8 rows)
      const auto rb = run((u * 4 + w) * 64 / KCH / 32);
      // the byte count is uniform but may be computed in a vector register: read it into a
      // scalar one, or every copy would be wrapped in a loop over distinct resources
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(rb.first, static_cast<uint32_t>(uniform(static_cast<int>(rb.second))));
      buf_to_lds16(rs, static_cast<uint32_t>(r % 32) * ksn_b + kswz<D>(r, c) * 16,
                   reinterpret_cast<char*>(dst) + (u * 4 + w) * 1024);
    }
  }

  // Scores of the 32 tokens of step q (rows 32q..32q+31 of the tile) for this lane's query
  // block: register r holds token 32q + (r/4)*8 + (l/32)*4 + r%4.
  __device__ f32x16_t scores(const uint16_t* tile, int q) const {
    const char* base = reinterpret_cast<const char*>(tile) + q * 32 * D * 2;
    f32x16_t c = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(base + (ak ^ (32u * ks)));
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qhi[ks], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qlo[ks], c, 0, 0, 0);
    }
    return c;
  }
};

// Workgroup -> (unit, query-block group) with every group of one unit on one XCD (workgroups
// are dealt to the 8 XCDs round-robin): the groups of a unit read the same keys, so they share
// them in that XCD's L2.  Returns false for the padding workgroups of the last round.
__device__ __forceinline__ bool xcd_unit(int units, int ngrp, int* unit, int* grp) {
  const int id = blockIdx.x, x = id % 8, k = id / 8;
  *unit = (k / ngrp) * 8 + x;
  *grp = k % ngrp;
  return *unit < units;
}
__host__ __device__ inline int xcd_grid(int units, int ngrp) { return (units + 7) / 8 * 8 * ngrp; }

// Workgroups of the seeds' pass per (head, group of 128 query blocks): with few groups the
// sampled tiles are dealt round-robin to up to four workgroups, about three per compute unit
// in all, so that more waves share each SIMD.
__host__ __device__ inline int seed_splits(int B, int H, int Mq) {
  const long groups = (long)((Mq + EXTRA_GROUP_BF16 - 1) / EXTRA_GROUP_BF16) * B * H;
  const long s = 768 / groups;
  return s < 1 ? 1 : (s > 4 ? 4 : static_cast<int>(s));
}
// Per query block and split, the words a split leaves for the combine: the two lanes' 32 keys
// each (lane half h at 32h + 8q + e: entry e of list q), then the two lanes' sample counts.
constexpr int SEED_SPLIT_WORDS = 68;
static_assert(4 * SEED_SPLIT_WORDS <= EXTRA_CAP * 2, "four splits' words fit one candidate list");

// The seed of one query block from its lanes' best-of lists (this lane's and its partner's,
// lane l ^ 32): the r-th best of the 64 kept keys.  Both lanes of the pair call it.
__device__ __forceinline__ uint32_t seed_of_lists(const Problem& P, size_t row, bool row_ok,
                                                  const uint32_t (&best)[4][SAMPLE_KEEP], int nsamp) {
  const int ntot = nsamp + __shfl_xor(nsamp, 32);
  const int ncand = P.N - P.bk * P.kept_cnt[row];
  uint32_t seed = 0u;
  if (row_ok && ncand > 0) {
    const long want = (static_cast<long>(SAMPLE_MARGIN) * P.extra * ntot + ncand - 1) / ncand;
    const int r = static_cast<int>(min(static_cast<long>(8 * SAMPLE_KEEP), max(1l, want)));
    uint32_t other[4][SAMPLE_KEEP];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < SAMPLE_KEEP; ++e)
        other[q][e] = static_cast<uint32_t>(__shfl_xor(static_cast<int>(best[q][e]), 32));
#pragma unroll 1
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < SAMPLE_KEEP; ++e) {
        const uint32_t v = q == 0 ? best[0][e] : q == 1 ? best[1][e] : q == 2 ? best[2][e] : best[3][e];
        int cge = 0;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2)
#pragma unroll
          for (int e2 = 0; e2 < SAMPLE_KEEP; ++e2)
            cge += (best[q2][e2] >= v ? 1 : 0) + (other[q2][e2] >= v ? 1 : 0);
        if (cge >= r) seed = max(seed, v);
      }
  }
  return max(seed, static_cast<uint32_t>(__shfl_xor(static_cast<int>(seed), 32)));
}

// Insertion into a best-of list kept in descending order: entry e of the new list is the median
// of old entries e-1 and e and the new key (one median-of-three per entry).
__device__ __forceinline__ void best_insert(uint32_t (&bl)[SAMPLE_KEEP], uint32_t k) {
#pragma unroll
  for (int e = SAMPLE_KEEP - 1; e > 0; --e) bl[e] = med3_u32(bl[e - 1], bl[e], k);
  bl[0] = max(bl[0], k);
}

// Seeds: the sample runs (sample_run) scored for the group's 128 query blocks, two runs per
// tile.  Each lane keeps the SAMPLE_KEEP best keys of every fourth run (four lists: list
// 2 (t % 2) + q takes run q of tile t), so a query block's two lanes hold 64 of its best sample
// keys; the seed is the r-th best of them, with r chosen so that about SAMPLE_MARGIN * E
// candidates are expected at or above it.  A best-of-a-subset is at most the best of the whole
// sample, so the seed only errs low (more candidates).  With S > 1 splits, split s takes tiles
// s, s + S, ... and leaves its lists in the candidate-list buffer (not in use before the
// sampled pass); extra_seed_combine_kernel merges the splits' lists, which gives every lane the
// same lists as one workgroup over all tiles, so the seeds do not depend on S.
template <int D>
__global__ __launch_bounds__(256, 3) void extra_seed_kernel(Problem P) {
  __shared__ ExtraSeedSmem<D> sm;
  constexpr int NB = XNB_S;
  using TT = ExtraTiles<D>;
  const int S = seed_splits(P.B, P.H, P.Mq);
  int unit, grp;
  if (!xcd_unit(P.B * P.H * S, (P.Mq + EXTRA_GROUP_BF16 - 1) / EXTRA_GROUP_BF16, &unit, &grp)) return;
  const int bh = unit / S, split = unit % S;
  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int rl = l % 32, i = grp * EXTRA_GROUP_BF16 + 32 * w + rl;
  const int b = bh / P.H, h = bh % P.H;
  const size_t row = (size_t)bh * P.Mq + (i < P.Mq ? i : 0);
  const bool row_ok = i < P.Mq && !(i >= P.dense_q0 && i < P.dense_q1);
  const uint16_t* kbase = static_cast<const uint16_t*>(P.k.p) + (int64_t)b * P.k.sb + (int64_t)h * P.k.sh;
  TT T;
  T.init(P, row, i < P.Mq);
  FlagCopy F;
  F.init(P, bh, i);
  const bool wave_on = __ballot(row_ok) != 0;

  const int nsteps = min(2 * P.M, min(4 * SAMPLE_STEPS, max(SAMPLE_STEPS, P.N / 1024)));
  const int ntile = (nsteps + 1) / 2;
  const int nmine = ntile > split ? (ntile - split + S - 1) / S : 0;   // this split's tiles
  auto run_tok = [&](int s) { return sample_run(s < nsteps ? s : 0, nsteps, P.M); };
  constexpr int OPS = TT::PT + 1;          // copies per thread per tile: keys, one flag dword
  // local tile j is tile split + j S of the sample, in buffer j % NB
  auto issue = [&](int j) {
    const int it = split + j * S;
    T.issue(sm.k[j % NB], [&](int q) {
      return std::make_pair(kbase + (int64_t)run_tok(2 * it + q) * P.k.sn, 32u * T.ksn_b);
    });
    F.issue_pair(run_tok(2 * it) >> 6, run_tok(2 * it + 1) >> 6, sm.fl[j % NB]);
  };
  uint32_t best[4][SAMPLE_KEEP];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < SAMPLE_KEEP; ++e) best[q][e] = 0u;
  int nsamp = 0;
  for (int j = 0; j < NB - 1 && j < nmine; ++j) issue(j);
#pragma unroll 1
  for (int j = 0; j < nmine; ++j) {
    const int it = split + j * S;
    wait_tiles<OPS>(min(NB - 2, nmine - 1 - j));
    tile_barrier();
    bool fl[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int s = 2 * it + q;
      fl[q] = row_ok && s < nsteps && !FlagCopy::kept_pair(sm.fl[j % NB], q, run_tok(s) >> 6);
    }
    // the refill goes to the buffer every wave finished with before this tile's barrier
    if (j + NB - 1 < nmine) issue(j + NB - 1);
    if (wave_on) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x16_t c = T.scores(sm.k[j % NB], q);
        if (fl[q]) {
          nsamp += 16;
          // run 2 it + q goes to list (2 it + q) % 4
          auto put = [&](uint32_t (&bl)[SAMPLE_KEEP]) {
#pragma unroll
            for (int r = 0; r < 16; ++r) best_insert(bl, float_key(c[r]));
          };
          if (it & 1) put(best[2 + q]);
          else put(best[q]);
        }
      }
    }
  }
  if (!wave_on) return;
  if (S > 1) {
    if (i < P.Mq) {
      uint32_t* out = reinterpret_cast<uint32_t*>(P.extra_buf + row * P.extra_lists * EXTRA_CAP) +
                      split * SEED_SPLIT_WORDS;
      const int h32 = l / 32;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < SAMPLE_KEEP; ++e) out[32 * h32 + 8 * q + e] = best[q][e];
      out[64 + h32] = static_cast<uint32_t>(nsamp);
    }
    return;
  }
  const uint32_t seed = seed_of_lists(P, row, row_ok, best, nsamp);
  if (l < 32 && i < P.Mq) P.extra_seed[row] = seed;
}

// The seeds from the splits' lists (seed_splits > 1): every lane inserts the other splits'
// entries of each list into split 0's, then the seed is taken as in the one-split pass.
__global__ __launch_bounds__(256) void extra_seed_combine_kernel(Problem P) {
  const int S = seed_splits(P.B, P.H, P.Mq);
  const int grp = blockIdx.x, bh = blockIdx.y, l = threadIdx.x % 64, w = threadIdx.x / 64;
  const int i = grp * EXTRA_GROUP_BF16 + 32 * w + l % 32, h32 = l / 32;
  if (i >= P.Mq) return;                                  // both lanes of a pair leave together
  const size_t row = (size_t)bh * P.Mq + i;
  const bool row_ok = !(i >= P.dense_q0 && i < P.dense_q1);
  const uint32_t* in = reinterpret_cast<const uint32_t*>(P.extra_buf + row * P.extra_lists * EXTRA_CAP);
  uint32_t best[4][SAMPLE_KEEP];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < SAMPLE_KEEP; ++e) best[q][e] = in[32 * h32 + 8 * q + e];
  int nsamp = static_cast<int>(in[64 + h32]);
  for (int sp = 1; sp < S; ++sp) {
    const uint32_t* o = in + sp * SEED_SPLIT_WORDS;
    uint32_t v[4][SAMPLE_KEEP];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < SAMPLE_KEEP; ++e) v[q][e] = o[32 * h32 + 8 * q + e];
    nsamp += static_cast<int>(o[64 + h32]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < SAMPLE_KEEP; ++e) best_insert(best[q], v[q][e]);
  }
  const uint32_t seed = seed_of_lists(P, row, row_ok, best, nsamp);
  if (l < 32) P.extra_seed[row] = seed;
}

// The threshold key thr as a float: a score c passes (float_key(c) >= thr) exactly when
// c >= key_threshold(thr), for every score that is not NaN (thr = 0 lets every such score pass;
// NaN scores, which only non-finite inputs produce, never become candidates).
__device__ __forceinline__ float key_threshold(uint32_t thr) {
  return thr == 0u ? -__builtin_inff() : key_float(thr);
}

// REPAIR = false: the sampled pass, every sparse query block from its seed.  The threshold never
// changes, so there is no cut: lanes l and l+32 (the two halves of a query block's 32-token
// step) append to interleaved slots of the (query block, slice) list, lane l to slots 2k and
// lane l+32 to slots 2k+1, and at the end the longer lane closes the gaps after the shorter
// one's last entry.  A lane that could overflow its half of the list stops appending and the
// list's fill is marked EXTRA_PART_OVERFLOW, which sends the query block to the exact pass.
// REPAIR = true: only the query blocks the merge flagged, from the threshold the merge left
// (the lowest after a short list, so every candidate competes: the exact selection; the seed
// after an overflow), one list per (query block, slice) cut back to its best E whenever the
// next step could overflow it.
template <int D, bool REPAIR>
__global__ __launch_bounds__(256, REPAIR ? 2 : 3) void extra_tile_kernel(Problem P) {
  constexpr bool repair = REPAIR;
  constexpr int NB = REPAIR ? XNB : XNB_S;             // tile buffers
  __shared__ std::conditional_t<REPAIR, ExtraSmem<D>, ExtraSampledSmem<D>> sm;
  using TT = ExtraTiles<D>;
  const int E = P.extra, N = P.N, S = P.extra_slices, nl = P.extra_lists;
  int unit, grp;                                 // unit = (head, slice)
  if (!xcd_unit(P.B * P.H * S, (P.Mq + EXTRA_GROUP_BF16 - 1) / EXTRA_GROUP_BF16, &unit, &grp)) return;
  const int bh = unit / S, slice = unit % S, tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int rl = l % 32, i0w = grp * EXTRA_GROUP_BF16 + 32 * w, i = i0w + rl;
  const int b = bh / P.H, h = bh % P.H;
  const size_t row = (size_t)bh * P.Mq + (i < P.Mq ? i : 0);
  bool row_ok = i < P.Mq && !(i >= P.dense_q0 && i < P.dense_q1);
  if (repair) {
    row_ok = row_ok && P.extra_flag[row] != 0;
    if (tid == 0) sm.any = 0;
    __syncthreads();
    if (row_ok) sm.any = 1;
    __syncthreads();
    if (!sm.any) return;
  }
  const uint16_t* kbase = static_cast<const uint16_t*>(P.k.p) + (int64_t)b * P.k.sb + (int64_t)h * P.k.sh;
  const int ts = (((N + S - 1) / S) + 127) / 128 * 128;       // tokens per slice
  const int t_lo = min(N, slice * ts), t_hi = min(N, t_lo + ts);
  const int ntile = (t_hi - t_lo + XTOK - 1) / XTOK;           // N is a whole number of tiles
  TT T;
  T.init(P, row, i < P.Mq);
  // the sampled pass starts from the seed; the exact pass from the threshold the merge left in
  // extra_seed (zero, or the seed after an overflow)
  uint32_t thr = row_ok ? P.extra_seed[row] : 0u;
  float tf = key_threshold(thr);
  const bool wave_on = __ballot(row_ok) != 0;

  // key copies: per tile one resource over its 64 rows (scalar arithmetic only); each lane's
  // offsets inside it are fixed
  const uint32_t ksn_b = T.ksn_b;
  uint32_t kvoff[TT::PT];
#pragma unroll
  for (int u = 0; u < TT::PT; ++u) {
    const int s = (u * 4 + w) * 64 + l, r = s / TT::KCH, c = s % TT::KCH;
    kvoff[u] = static_cast<uint32_t>(r) * ksn_b + kswz<D>(r, c) * 16;
  }
  // flag copies: the dword of the lane's kept-bitmap row that holds the tile's key block
  const uint32_t nwb = static_cast<uint32_t>(P.Mpad / 64) * 8u;
  const __amdgpu_buffer_rsrc_t frs =
      make_rsrc(P.kept_bm + (size_t)bh * P.Mq * (P.Mpad / 64), static_cast<uint32_t>(P.Mq) * nwb);
  const uint32_t fvoff = static_cast<uint32_t>(i < P.Mq ? i : P.Mq) * nwb;
  constexpr int OPS = TT::PT + 1;          // copies per thread per tile: keys, one flag dword
  auto issue = [&](int it) {
    const int t0 = t_lo + it * XTOK;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase + (int64_t)t0 * P.k.sn, 64u * ksn_b);
    char* kd = reinterpret_cast<char*>(sm.k[it % NB]);
#pragma unroll
    for (int u = 0; u < TT::PT; ++u) buf_to_lds16(krs, kvoff[u], kd + (u * 4 + w) * 1024);
    buf_to_lds4s(frs, fvoff, static_cast<uint32_t>(t0 >> 11) * 4u, sm.fl[it % NB][0] + 64 * w);
  };

  // candidate stores go through a buffer resource over this wave's lists of the slice
  const uint32_t row_stride = (uint32_t)nl * EXTRA_CAP * 8u;          // bytes between query blocks
  const int nvalid = uniform(max(1, min(32, P.Mq - i0w)));
  const __amdgpu_buffer_rsrc_t brsrc =
      make_rsrc(P.extra_buf + ((size_t)bh * P.Mq + uniform(min(i0w, P.Mq - 1))) * nl * EXTRA_CAP +
                    (size_t)slice * EXTRA_CAP,
                (uint32_t)(nvalid - 1) * row_stride + EXTRA_CAP * 8u);
  const uint32_t my_off = (uint32_t)rl * row_stride;
  int cnt = 0;

  if constexpr (!REPAIR) {
    // Sampled pass.  Lane l's k-th candidate goes to slot 2k + l/32 of its list.
    constexpr int HALF = EXTRA_CAP / 2;
    uint32_t addr = my_off + static_cast<uint32_t>(l / 32) * 8u;
    bool full = false;                            // this lane's half could overflow: stop
    auto append = [&](const f32x16_t& c, bool on, int tw) {
      if (__ballot(on) == 0) return;
      const uint32_t tk0 = static_cast<uint32_t>(tw + (l / 32) * 4);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (on && c[r] >= tf) {
          u32x2 v2;
          v2.x = __float_as_uint(c[r]);
          v2.y = tk0 + static_cast<uint32_t>((r / 4) * 8 + (r % 4));
          __builtin_amdgcn_raw_buffer_store_b64(v2, brsrc, addr, 0, 0);
          addr += 16u;
        }
      }
    };
    for (int it = 0; it < NB - 1 && it < ntile; ++it) issue(it);
    // the previous tile's scores, stored one tile late
    f32x16_t pc0 = {}, pc1 = {};
    bool pon = false;
    int ptw = 0;
#pragma unroll 1
    for (int it = 0; it < ntile; ++it) {
      const int t0 = t_lo + it * XTOK, j = t0 >> 6;
      wait_tiles<OPS>(min(NB - 2, ntile - 1 - it));
      tile_barrier();
      const bool cand = row_ok && j < P.M && !FlagCopy::kept(sm.fl[it % NB][0], j);
      // every wave has read this tile's flags before its buffer is refilled (a tile later)
      if (it + NB - 1 < ntile) issue(it + NB - 1);
      append(pc0, pon, ptw);
      append(pc1, pon, ptw + 32);
      // the next tile appends at most 32 entries per lane
      full = full || (addr - my_off) > static_cast<uint32_t>(2 * (HALF - 2 * 16)) * 8u;
      pon = false;
      if (wave_on && __ballot(cand) != 0) {
        pc0 = T.scores(sm.k[it % NB], 0);
        pc1 = T.scores(sm.k[it % NB], 1);
        pon = cand && !full;
        ptw = t0;
      }
    }
    append(pc0, pon, ptw);
    append(pc1, pon, ptw + 32);
    // Close the gaps: slots [0, 2m) hold both lanes' first m = min(count, partner's count)
    // entries; the longer lane moves its remaining entries (slots 2k + l/32, k >= m) down to
    // slots 2m, 2m + 1, ... in order, so the list is contiguous.  A slot is only written after
    // it was read (destination 2m + t <= source 2(m + t) + l/32), and the reads bypass the
    // vector cache (glc) after this lane's own stores completed.
    cnt = static_cast<int>((addr - my_off) >> 4);
    const int ocnt = __shfl_xor(cnt, 32);
    const bool ofull = __shfl_xor(full ? 1 : 0, 32) != 0;
    if (!full && !ofull && cnt > ocnt) {
      __builtin_amdgcn_s_waitcnt(0);
      const uint32_t h = static_cast<uint32_t>(l / 32);
#pragma unroll 1
      for (int k0 = ocnt; k0 < cnt; k0 += 8) {
        u32x2 e[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (k0 + t < cnt)
            e[t] = __builtin_amdgcn_raw_buffer_load_b64(
                brsrc, my_off + (2u * static_cast<uint32_t>(k0 + t) + h) * 8u, 0, 1);
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (k0 + t < cnt)
            __builtin_amdgcn_raw_buffer_store_b64(
                e[t], brsrc, my_off + static_cast<uint32_t>(ocnt + k0 + t) * 8u, 0, 0);
      }
    }
    if (l < 32 && i < P.Mq)
      P.extra_part[row * nl + slice] = (full || ofull) ? EXTRA_PART_OVERFLOW : cnt + ocnt;
  } else {
    // Exact pass.  Append the candidates (bits) of one 32-token step starting at token tw
    // (scores c): lane l first, then its partner l+32, each in register order; then cut the
    // lists that the next step could overflow.
    auto append = [&](const f32x16_t& c, uint32_t bits, int tw) {
      if (__ballot(bits != 0) == 0) return;
      const int mine = __popc(bits);
      const int other = __shfl_xor(mine, 32);
      uint32_t addr = my_off + static_cast<uint32_t>(cnt + (l < 32 ? 0 : other)) * 8u;
      cnt += mine + other;
      const uint32_t tk0 = static_cast<uint32_t>(tw + (l / 32) * 4);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t bit = (bits >> r) & 1u;
        if (bit) {
          u32x2 v2;
          v2.x = __float_as_uint(c[r]);
          v2.y = tk0 + static_cast<uint32_t>((r / 4) * 8 + (r % 4));
          __builtin_amdgcn_raw_buffer_store_b64(v2, brsrc, addr, 0, 0);
        }
        addr += bit << 3;
      }
      uint64_t m = __ballot(l < 32 && cnt > EXTRA_CAP - XSTEP);
      if (m) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // this wave's stores, visible
        while (m) {
          const int rr = __builtin_ctzll(m);
          m &= m - 1;
          uint2* rb = P.extra_buf + (((size_t)bh * P.Mq + i0w + rr) * nl + slice) * EXTRA_CAP;
          const int crr = __shfl(cnt, rr);
          const uint32_t kth = wave_cut(rb, crr, E, sm.hist[w], sm.scr[w]);
          if (rl == rr) {
            thr = max(thr, kth);
            tf = key_threshold(thr);
            cnt = E;
          }
          wave_sync();
        }
      }
    };
    auto cand_bits = [&](const f32x16_t& c) {
      uint32_t bits = 0;
#pragma unroll
      for (int r = 15; r >= 0; --r) bits = bits * 2u + (c[r] >= tf ? 1u : 0u);
      return bits;
    };

    for (int it = 0; it < NB - 1 && it < ntile; ++it) issue(it);
    // the previous tile's scores and candidate bits, stored one tile late
    f32x16_t pc0 = {}, pc1 = {};
    uint32_t pb0 = 0, pb1 = 0;
    int ptw = 0;
#pragma unroll 1
    for (int it = 0; it < ntile; ++it) {
      const int t0 = t_lo + it * XTOK, j = t0 >> 6;
      wait_tiles<OPS>(min(NB - 2, ntile - 1 - it));
      tile_barrier();
      const bool cand = row_ok && j < P.M && !FlagCopy::kept(sm.fl[it % NB][0], j);
      // every wave has read this tile's flags before its buffer is refilled (a tile later)
      if (it + NB - 1 < ntile) issue(it + NB - 1);
      append(pc0, pb0, ptw);
      append(pc1, pb1, ptw + 32);
      pb0 = pb1 = 0;
      if (wave_on && __ballot(cand) != 0) {
        pc0 = T.scores(sm.k[it % NB], 0);
        pc1 = T.scores(sm.k[it % NB], 1);
        if (cand) {
          pb0 = cand_bits(pc0);
          pb1 = cand_bits(pc1);
        }
        ptw = t0;
      }
    }
    append(pc0, pb0, ptw);
    append(pc1, pb1, ptw + 32);
    // publish the list lengths of the flagged query blocks
    if (l < 32 && i < P.Mq && row_ok) P.extra_part[row * nl + slice] = cnt;
  }
}

// Pass 2: best E of the 4*S partial lists of one query block, ranked by token.  The lists stay
// in memory (L2-resident) and every pass reads them as one flat range with 8 loads in flight
// per lane.  Radix selection starts below the bits that all keys share (scores of one query
// block have similar magnitudes), so it takes few passes and its histogram counts spread over
// many bins.

// `need`-th largest of the keys visited by `visit(f)` (f(key) for every live key), radix 8 over
// the bits below the common prefix of [kmin, kmax].  Returns it; *need_eq = how many of the keys
// equal to it are taken, *cnt_eq = how many keys equal it.
template <typename Visit>
__device__ uint32_t merge_select(Visit&& visit, uint32_t kmin, uint32_t kmax, int need, int* hist,
                                 int* scr, int* need_eq, int* cnt_eq) {
  const int l = threadIdx.x & 63;
  const uint32_t diff = kmin ^ kmax;
  if (diff == 0u) {                       // every key equal
    int n = 0;
    visit([&](uint32_t) { ++n; });
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o);
    *need_eq = need;
    *cnt_eq = n;
    return kmax;
  }
  const int hb = 31 - __builtin_clz(diff);
  uint32_t pmask = hb == 31 ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = kmax & pmask;
  int at = 0;
  for (int top = hb; top >= 0; top -= 8) {
    const int shift = top >= 7 ? top - 7 : 0;
    const uint32_t dmask = (2u << (top - shift)) - 1u;
#pragma unroll
    for (int q = 0; q < 4; ++q) hist[4 * l + q] = 0;
    wave_sync();
    visit([&](uint32_t k) {
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1);
    });
    wave_sync();
    int above;
    const int dg = wave_pick_digit(hist, need, &above, &at, scr);
    prefix |= static_cast<uint32_t>(dg) << shift;
    pmask |= dmask << shift;
    need -= above;
  }
  *need_eq = need;
  *cnt_eq = at;
  return prefix;
}

// repair: 0 = first merge (checks the seeded pass), 1 = merge of the repaired query blocks,
// 2 = flag every sparse query block for the exact pass (no merge)
__global__ __launch_bounds__(64) void extra_merge_kernel(Problem P, int repair) {
  __shared__ int hist[256];
  __shared__ int scr[4];
  __shared__ int toks[MAX_EXTRA];
  const int i = blockIdx.x, bh = blockIdx.y, l = threadIdx.x;
  const size_t row = (size_t)bh * P.Mq + i;
  const int E = P.extra;
  if (i >= P.dense_q0 && i < P.dense_q1) return;          // dense rows keep extra_cnt = 0
  const int nl = P.extra_lists;
  const int* part = P.extra_part + row * nl;
  const uint2* lists = P.extra_buf + row * nl * EXTRA_CAP;
  if (repair == 2) {                                       // exact selection for every row
    if (l == 0) {
      P.extra_flag[row] = 1;
      P.extra_seed[row] = 0u;                              // from the lowest threshold
    }
    return;
  }
  if (repair && P.extra_flag[row] == 0) return;
  int cnts[16];
  int total = 0;
  bool overflow = false;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int f = q < nl ? part[q] : 0;
    overflow = overflow || f == EXTRA_PART_OVERFLOW;
    cnts[q] = f == EXTRA_PART_OVERFLOW ? 0 : f;
    total += cnts[q];
  }
  if (!repair) {
    // every candidate scoring at or above the seeded threshold is in the lists; fewer than
    // min(E, |candidates|) of them means the seed was too high, and a list that could have
    // overflowed may have lost some: either way the query block goes to the exact repair pass.
    // That pass starts from the threshold left in extra_seed: zero after a short list (every
    // candidate competes); the seed itself after an overflow, since a half list holding more
    // than EXTRA_CAP / 2 - 32 >= E candidates at or above the seed means no candidate below it
    // can be among the E best.
    const int ncand = P.N - P.bk * P.kept_cnt[row];
    const bool short_ = total < min(E, ncand);
    const bool flag = overflow || short_;
    if (l == 0) {
      P.extra_flag[row] = flag ? 1 : 0;
      if (flag && !overflow) P.extra_seed[row] = 0u;
    }
    if (flag) return;
  }
  // the lists as one flat range: entry p lives in list q with start[q] <= p < start[q+1]
  int start[17];
  start[0] = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) start[q + 1] = start[q] + cnts[q];
  auto entry = [&](int p) {
    int q = 0;
#pragma unroll
    for (int r = 1; r < 16; ++r) q += p >= start[r] ? 1 : 0;
    return lists[q * EXTRA_CAP + (p - start[q])];
  };
  if (l == 0) scr[3] = 0;
  wave_sync();
  // The usual case: every entry in registers (NPL per lane), selected there, survivors
  // appended to toks[].  Larger lists take the streaming path below.
  auto in_registers = [&](auto nplc) {
    constexpr int NPL = decltype(nplc)::value;
    uint32_t key[NPL], tok[NPL];
    bool valid[NPL], keep[NPL];
#pragma unroll
    for (int u = 0; u < NPL; ++u) {
      const int p = u * 64 + l;
      valid[u] = p < total;
      const uint2 e = valid[u] ? entry(p) : make_uint2(0u, 0u);
      key[u] = float_key(__uint_as_float(e.x));
      tok[u] = e.y;
    }
    wave_best<NPL>(key, tok, valid, total, E, hist, scr, keep);
#pragma unroll
    for (int u = 0; u < NPL; ++u) {
      const uint64_t m = __ballot(keep[u]);
      if (keep[u]) toks[scr[3] + __popcll(m & ((1ull << l) - 1ull))] = static_cast<int>(tok[u]);
      wave_sync();
      if (l == 0) scr[3] += __popcll(m);
      wave_sync();
    }
  };
  if (total <= 16 * 64) {
    in_registers(std::integral_constant<int, 16>{});
  } else if (total <= 32 * 64) {
    in_registers(std::integral_constant<int, 32>{});
  } else {
    // streaming: every pass reads the lists again, 8 loads in flight per lane
    auto for_each = [&](auto&& f) {
#pragma unroll 1
      for (int p0 = 0; p0 < total; p0 += 8 * 64) {
        uint2 e[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int p = p0 + u * 64 + l;
          e[u] = p < total ? entry(p) : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (p0 + u * 64 + l < total) f(float_key(__uint_as_float(e[u].x)), e[u].y);
      }
    };
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for_each([&](uint32_t k, uint32_t) {
      kmin = min(kmin, k);
      kmax = max(kmax, k);
    });
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), o)));
      kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), o)));
    }
    int need_eq, cnt_eq;
    const uint32_t kstar = merge_select([&](auto&& f) { for_each([&](uint32_t k, uint32_t) { f(k); }); },
                                        kmin, kmax, E, hist, scr, &need_eq, &cnt_eq);
    uint32_t tmax = 0xFFFFFFFFu;
    if (need_eq < cnt_eq) {
      // ties at K*: keep the need_eq lowest tokens (larger ~token = smaller token)
      uint32_t tmin2 = 0xFFFFFFFFu, tmax2 = 0u;
      for_each([&](uint32_t k, uint32_t t) {
        if (k == kstar) {
          tmin2 = min(tmin2, ~t);
          tmax2 = max(tmax2, ~t);
        }
      });
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        tmin2 = min(tmin2, static_cast<uint32_t>(__shfl_xor(static_cast<int>(tmin2), o)));
        tmax2 = max(tmax2, static_cast<uint32_t>(__shfl_xor(static_cast<int>(tmax2), o)));
      }
      int ne2, ce2;
      tmax = ~merge_select([&](auto&& f) {
        for_each([&](uint32_t k, uint32_t t) {
          if (k == kstar) f(~t);
        });
      }, tmin2, tmax2, need_eq, hist, scr, &ne2, &ce2);
    }
    for_each([&](uint32_t k, uint32_t t) {
      if (k > kstar || (k == kstar && t <= tmax)) toks[atomicAdd(&scr[3], 1)] = static_cast<int>(t);
    });
  }
  wave_sync();
  // survivors are in toks[0..c): sort them ascending, write them out, and take them out of
  // their key blocks' centroid terms (key blocks are 64 tokens: block_k is 64 in this library).
  // In the register paths the survivors keep the order of the lists: slices in order, and
  // inside a list either a lane's tokens then its partner's per 32-token step (exact pass) or
  // the two lanes' ascending runs interleaved entry by entry, the longer run's rest after them
  // (sampled pass), so every token sits near its sorted place.  An odd-even transposition sort,
  // run until a whole round swaps nothing, takes few rounds there (and stays exact for any
  // order); it runs in registers, four entries per lane, a round being a few instructions and
  // two lane shifts.
  const int c = scr[3];
  wave_sync();
  {
    // the sort runs in registers: entry 4l + e in v[e] of lane l (past c: INT_MAX, which stays
    // at the end); a round compares the even pairs (4l, 4l+1), (4l+2, 4l+3), then the odd pairs
    // (4l+1, 4l+2) and (4l+3, 4l+4), the last across the lane boundary
    static_assert(MAX_EXTRA == 4 * 64, "four entries per lane");
    int v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = 4 * l + e < c ? toks[4 * l + e] : 0x7FFFFFFF;
    auto cswap = [](int& a, int& b, bool& sw) {
      const int lo = min(a, b), hi = max(a, b);
      sw = sw || lo != a;
      a = lo;
      b = hi;
    };
#pragma unroll 1
    for (;;) {
      bool sw = false;
      cswap(v[0], v[1], sw);
      cswap(v[2], v[3], sw);
      cswap(v[1], v[2], sw);
      const int next0 = __shfl_down(v[0], 1);          // lane l+1's first entry
      const int prev3 = __shfl_up(v[3], 1);            // lane l-1's last entry
      if (l < 63 && next0 < v[3]) {
        v[3] = next0;
        sw = true;
      }
      if (l > 0) v[0] = max(v[0], prev3);
      if (__ballot(sw) == 0) break;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * l + e < c) toks[4 * l + e] = v[e];
    wave_sync();
  }
  int* out = P.extra_idx + row * MAX_EXTRA;
  uint8_t* mr = P.mult + row * P.Mpad;
  for (int p = l; p < c; p += 64) {
    const int t = toks[p], bt = t >> 6;
    out[p] = t;
    if (P.keep_lists && (p == 0 || (toks[p - 1] >> 6) != bt)) {
      int e = p + 1;
      while (e < c && (toks[e] >> 6) == bt) ++e;
      mr[bt] = static_cast<uint8_t>(64 - (e - p));
    }
  }
  if (l == 0) P.extra_cnt[row] = c;
}

hipError_t launch_extra_select(const Problem& P, hipStream_t stream) {
  dim3 grid((P.Mq + XR - 1) / XR, P.B * P.H, P.extra_slices);
  const int ngrp = (P.Mq + EXTRA_GROUP_BF16 - 1) / EXTRA_GROUP_BF16;
  dim3 g16(xcd_grid(P.B * P.H * P.extra_slices, ngrp));
  const int nsplit = seed_splits(P.B, P.H, P.Mq);
  dim3 gseed(xcd_grid(P.B * P.H * nsplit, ngrp));
  dim3 g2(P.Mq, P.B * P.H);
  auto pass1 = [&](int repair) {
    if (P.dtype == 0) {
      if (!repair) {
        if (P.d == 128) hipLaunchKernelGGL(extra_seed_kernel<128>, gseed, dim3(256), 0, stream, P);
        else hipLaunchKernelGGL(extra_seed_kernel<64>, gseed, dim3(256), 0, stream, P);
        if (nsplit > 1)
          hipLaunchKernelGGL(extra_seed_combine_kernel, dim3(ngrp, P.B * P.H), dim3(256), 0, stream, P);
      }
      if (repair) {
        if (P.d == 128) hipLaunchKernelGGL((extra_tile_kernel<128, true>), g16, dim3(256), 0, stream, P);
        else hipLaunchKernelGGL((extra_tile_kernel<64, true>), g16, dim3(256), 0, stream, P);
      } else {
        if (P.d == 128) hipLaunchKernelGGL((extra_tile_kernel<128, false>), g16, dim3(256), 0, stream, P);
        else hipLaunchKernelGGL((extra_tile_kernel<64, false>), g16, dim3(256), 0, stream, P);
      }
    } else {
      if (P.d == 128) hipLaunchKernelGGL(extra_select_kernel<128>, grid, dim3(256), 0, stream, P, repair);
      else hipLaunchKernelGGL(extra_select_kernel<64>, grid, dim3(256), 0, stream, P, repair);
    }
    return hipGetLastError();
  };
  hipError_t e;
  if (P.exact_extra) {
    // every query block straight to the exact pass
    hipLaunchKernelGGL(extra_merge_kernel, g2, dim3(64), 0, stream, P, 2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    if ((e = pass1(0)) != hipSuccess) return e;
    hipLaunchKernelGGL(extra_merge_kernel, g2, dim3(64), 0, stream, P, 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = pass1(1)) != hipSuccess) return e;
  hipLaunchKernelGGL(extra_merge_kernel, g2, dim3(64), 0, stream, P, 1);
  return hipGetLastError();
}

}  // namespace solattn
