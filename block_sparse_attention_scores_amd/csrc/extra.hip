// extra_select: for each sparse query block i, the up to E = extra_tokens individual keys with
// the highest q̄_i . k_t among tokens outside its kept blocks, ties to the lower token (node
// docs, common inputs table, extra_tokens row: extra high-score tokens each query block
// attends beyond its selected blocks).
//
// Pass 1 (extra_select_kernel).  A workgroup of 4 waves owns 32 query blocks of one head and one
// slice of the token range; the waves take turns over 32-token steps.  Scores come from the
// 32x32x16 bf16 matrix instruction with q̄ split into two bf16 parts (hi + lo), accurate to
// ~2^-17 relative (fp32-like), while the keys are exact bf16.  Each lane owns one query block
// (a column of the accumulator).  Every wave keeps its own candidate buffer per query block in
// the workspace, so the streaming loop needs no barrier; the four waves share one running
// threshold per query block in LDS (any wave's E-th best is a lower bound of the final E-th
// best).  A score above the threshold is appended; when a buffer could overflow on the next
// step, the wave finds its E-th best entry by radix selection on (score, token), cuts the
// buffer to exactly E entries and raises the shared threshold.  Keys stream in increasing token
// order within a wave, so a later token that ties the threshold loses the tie and a strict
// comparison suffices.
//
// Pass 2 (extra_merge_kernel).  One wave per query block takes the best E of the partial lists
// (one per wave and slice), ranks them by token, writes them out, and takes the chosen tokens
// out of their blocks' centroid terms.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace solattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int XR = 32;      // query blocks per workgroup

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t xrsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int XSTEP = 32;   // tokens per wave step

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
constexpr int SAMPLE_MARGIN = 6;

__device__ __forceinline__ int sample_run(int s, int nsteps, int M) {
  const int span = max(1, M / nsteps);
  const int j = static_cast<int>((static_cast<long>(s) * M) / nsteps) + (s * 37) % span;
  return j * 64 + ((nsteps > M) ? 32 * (s & 1) : 0);
}

// Pass 1.  repair = 0: every sparse query block, with thresholds seeded from the sample.
// repair = 1: only the query blocks the merge flagged (fewer candidates than it needs), with
// the threshold at its minimum, so that every candidate competes (the exact selection).
template <typename T, int D>
__global__ __launch_bounds__(256, 2) void extra_select_kernel(Problem P, int repair) {
  __shared__ uint32_t thr[XR];            // shared threshold keys: append when key >= thr
  __shared__ int whist[4][256];
  __shared__ int wscr[4][4];
  __shared__ float qs[(sizeof(T) == 4) ? XR : 1][D];
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
  const uint8_t* mrow = P.mult + grow * P.Mpad;
  const T* kbase = static_cast<const T*>(P.k.p) + (int64_t)b * P.k.sb + (int64_t)h * P.k.sh;
  const int ts = (((N + S - 1) / S) + 127) / 128 * 128;       // tokens per slice
  const int t_lo = slice * ts, t_hi = min(N, t_lo + ts);

  if (tid < XR) thr[tid] = 0u;

  // q̄ operands: split bf16 hi/lo fragments (bf16 inputs) or an fp32 copy in LDS
  bf16x8_t qhi[D / 16], qlo[D / 16];
  if constexpr (sizeof(T) == 2) {
    const float* qb = P.qbar + grow * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (i < P.Mq) ? qb[16 * ks + 8 * (l / 32) + e] : 0.f;
        const uint16_t hb = f32_to_bf16(x);
        const uint16_t lb = f32_to_bf16(x - bf16_to_f32(hb));
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

  // scores of 32 consecutive tokens from tw for this lane's query block: register r holds token
  // tw + (r/4)*8 + (l/32)*4 + r%4
  // (bf16: the key fragments come from kf, loaded by load_keys, which first loads the step's
  // candidate flag into mflag, so that waiting for the flag never waits for the keys)
  bf16x8_t kf[D / 16];
  uint8_t mflag = 0;
  auto load_keys = [&](int tw) {
    mflag = row_ok ? mrow[tw >> 6] : 0;
    if constexpr (sizeof(T) == 2) {
      const T* kr = kbase + (int64_t)(tw + rl) * P.k.sn + 8 * (l / 32);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) kf[ks] = *reinterpret_cast<const bf16x8_t*>(kr + 16 * ks);
    }
  };
  // `prefetch(kc)` runs after this step's key fragments are copied out of kf (bf16), so the
  // next step's loads can go out before this step's products
  auto scores = [&](int tw, float* acc, auto&& prefetch) {
    if constexpr (sizeof(T) == 2) {
      bf16x8_t kc[D / 16];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) kc[ks] = kf[ks];
      prefetch();
      f32x16_t c = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc[ks], qhi[ks], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc[ks], qlo[ks], c, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = c[r];
    } else {
#pragma unroll 1
      for (int r = 0; r < 16; ++r) {
        const int tk = tw + (r / 4) * 8 + (l / 32) * 4 + (r % 4);
        const float* kr = reinterpret_cast<const float*>(kbase) + (int64_t)tk * P.k.sn;
        float sc = 0.f;
#pragma unroll 8
        for (int e = 0; e < D; ++e) sc = fmaf(qs[rl][e], kr[e], sc);
        acc[r] = sc;
      }
      prefetch();
    }
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
      xrsrc(P.extra_buf + (((size_t)bh * P.Mq + i0) * S + slice) * 4 * EXTRA_CAP + (size_t)w * EXTRA_CAP,
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
  const int E = P.extra, S = P.extra_slices;
  if (i >= P.dense_q0 && i < P.dense_q1) return;          // dense rows keep extra_cnt = 0
  const int nl = 4 * S;
  const int* part = P.extra_part + row * nl;
  const uint2* lists = P.extra_buf + row * nl * EXTRA_CAP;
  if (repair == 2) {                                       // exact selection for every row
    if (l == 0) P.extra_flag[row] = 1;
    return;
  }
  if (repair && P.extra_flag[row] == 0) return;
  int cnts[16];
  int total = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    cnts[q] = q < nl ? part[q] : 0;
    total += cnts[q];
  }
  if (!repair) {
    // every candidate scoring at or above the seeded threshold is in the lists (or was cut in
    // favour of better ones); fewer than min(E, |candidates|) of them means the seed was too
    // high, and the query block goes to the exact repair pass
    const int ncand = P.N - P.bk * P.kept_cnt[row];
    const bool short_ = total < min(E, ncand);
    if (l == 0) P.extra_flag[row] = short_ ? 1 : 0;
    if (short_) return;
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
  // survivors are in toks[0..c) in any order: sort them ascending (bitonic network over
  // MAX_EXTRA slots, padding at the end), write them out, and take them out of their key
  // blocks' centroid terms (key blocks are 64 tokens: block_k is 64 in this library)
  const int c = scr[3];
  for (int p = c + l; p < MAX_EXTRA; p += 64) toks[p] = 0x7fffffff;
  wave_sync();
#pragma unroll 1
  for (int kk = 2; kk <= MAX_EXTRA; kk <<= 1) {
#pragma unroll 1
    for (int j = kk >> 1; j > 0; j >>= 1) {
#pragma unroll
      for (int p = l; p < MAX_EXTRA; p += 64) {
        const int pj = p ^ j;
        if (pj > p) {
          const int x = toks[p], y = toks[pj];
          if ((x > y) == ((p & kk) == 0)) {
            toks[p] = y;
            toks[pj] = x;
          }
        }
      }
      wave_sync();
    }
  }
  int* out = P.extra_idx + row * MAX_EXTRA;
  uint8_t* mr = P.mult + row * P.Mpad;
  for (int p = l; p < c; p += 64) {
    const int t = toks[p], bt = t >> 6;
    out[p] = t;
    if (p == 0 || (toks[p - 1] >> 6) != bt) {
      int e = p + 1;
      while (e < c && (toks[e] >> 6) == bt) ++e;
      const int m = 64 - (e - p);
      mr[bt] = static_cast<uint8_t>(m);
      P.cbias[row * P.Mpad + bt] = m > 0 ? __logf(static_cast<float>(m)) / P.scale : -__builtin_inff();
    }
  }
  if (l == 0) P.extra_cnt[row] = c;
}

hipError_t launch_extra_select(const Problem& P, hipStream_t stream) {
  dim3 grid((P.Mq + XR - 1) / XR, P.B * P.H, P.extra_slices);
  dim3 g2(P.Mq, P.B * P.H);
  auto pass1 = [&](int repair) {
    if (P.dtype == 0) {
      if (P.d == 128) hipLaunchKernelGGL((extra_select_kernel<uint16_t, 128>), grid, dim3(256), 0, stream, P, repair);
      else hipLaunchKernelGGL((extra_select_kernel<uint16_t, 64>), grid, dim3(256), 0, stream, P, repair);
    } else {
      if (P.d == 128) hipLaunchKernelGGL((extra_select_kernel<float, 128>), grid, dim3(256), 0, stream, P, repair);
      else hipLaunchKernelGGL((extra_select_kernel<float, 64>), grid, dim3(256), 0, stream, P, repair);
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
