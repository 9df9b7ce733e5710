// sparse_flash_fwd: the attention of one query block over its work list, in one FP32 online
// softmax (star7 README, "Sol": kept K/V blocks exactly, skipped blocks through their
// centroids, merged in one FP32 online softmax; "SLA": only the routed blocks):
//   1. the kept key blocks (for dense query blocks: every block),
//   2. sol only: the centroid terms of every key block, 64 per tile, each with logit
//      q.k̄_j / sqrt(d) + ln(m_ij) (m_ij = tokens of block j not attended exactly; a kept
//      block has m = 0 and drops out),
//   3. the extra tokens, gathered 64 at a time.
// Every tile is the same computation on a 64-key K tile and a V tile in LDS with a per-key
// additive bias; tiles stream through double-buffered LDS (phases 1 and 2 in one loop, the
// extra tokens in a second one).
//
// bf16 kernel: each wave owns 32 query rows.  S^T = K Q^T and O^T += V^T P^T run on the
// 32x32x16 bf16 matrix instruction: the score accumulator's lane layout (lane = query row,
// 16 registers = keys) feeds P^T straight to the second product, so P never leaves registers;
// the V tile is stored transposed with a key permutation that matches that layout (extra-token
// tiles, gathered row by row, keep V row-major and read it two bytes at a time).  Running
// max and sum are fp32 and kept per lane (the two half-waves hold the same query rows and
// combine their partial sums at the end).  Logits are taken in base 2.
//
// fp32 tensors: flash_f32.hip (the same phases on the fp32 matrix instruction).
#include "common.h"
#include "launch.h"

namespace solattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr float LOG2E = 1.4426950408889634f;

// ------------------------------------------------------------------ bf16 path

// LDS swizzle of the transposed V rows (128 bytes: 64 keys), as kswz for the key rows.
__device__ __forceinline__ int vswz(int r, int c) { return c ^ ((r >> 1) & 7); }
// E4M3 key rows (fp8-QK): D bytes, D/16 chunks
template <int D>
__device__ __forceinline__ int kswz8(int r, int c) { return c ^ ((r >> 1) & (D / 16 - 1)); }

// Double-buffered LDS tiles.  K: 64 keys x D (chunk-swizzled rows; bf16, or E4M3 bytes plus the
// rows' scale codes for the fp8-QK flavour).  V: transposed, D rows of 64 keys (chunk-swizzled).
// Bias: per query block of the pair, per key (centroid and extra tiles).
template <int D, bool QK8>
struct FlashSmem {
  __attribute__((aligned(16))) uint8_t k[2][QK8 ? 64 * D : 128 * D];
  __attribute__((aligned(16))) uint16_t v[2][64 * D];
  __attribute__((aligned(16))) float bias[2][2][64];
  __attribute__((aligned(16))) float zero[64];   // the bias of plain key tiles
  __attribute__((aligned(16))) uint8_t ke[2][QK8 ? 64 : 16];   // E4M3 scale codes of the K rows
  __attribute__((aligned(16))) int eidx[2][MAX_EXTRA];         // extra-token lists of the pair
};

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

struct TileDesc {
  int kind;   // 0 kept key block, 1 extra tokens of one query block, 2 centroids, 3 end
  int idx;    // key block j | first extra position | first centroid index
  int sel;    // bit g: query block g of the pair attends this tile
};

__device__ __forceinline__ uint64_t readlane64(uint64_t x, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(x), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(x >> 32), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Orders one wave's LDS accesses before and after it.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Walks the main loop's work of a pair of query blocks: every key block kept by either of them,
// in ascending order, then the centroid tiles.  The two kept-block bitmaps are held one 64-bit
// word per lane (lane l: blocks 64l..64l+63), so finding the next tile is a ballot and a few
// lane reads, with no memory access.  Every decision is uniform across the wave.
struct TileIter {
  uint64_t w0, w1;   // this lane's words of the two bitmaps
  uint64_t rem;      // bits of w0 | w1 not visited yet
  int pos, ncent, cent_sel;
  __device__ TileDesc next() {
    const uint64_t act = __ballot(rem != 0);
    if (act) {
      const int L = static_cast<int>(__builtin_ctzll(act));
      const uint64_t word = readlane64(rem, L);
      const int bit = static_cast<int>(__builtin_ctzll(word));
      const uint64_t a = readlane64(w0, L), b = readlane64(w1, L);
      if (static_cast<int>(threadIdx.x & 63) == L) rem &= rem - 1;   // the lowest bit is `bit`
      const int sel = static_cast<int>((a >> bit) & 1u) | (static_cast<int>((b >> bit) & 1u) << 1);
      return TileDesc{0, 64 * L + bit, sel};
    }
    if (pos < ncent) {
      const int c = pos;
      pos += 64;
      return TileDesc{2, c, cent_sel};
    }
    return TileDesc{3, 0, 0};
  }
};

// Workgroup -> (head, query blocks qa and qb of the workgroup; qb = -1 if none).  Units of the
// dense query blocks (the heaviest) come first, then the rest head-major.  Consecutive units go
// to the same XCD in runs of XCD_RUN (workgroups are dealt to the 8 XCDs round-robin), so one
// XCD works on neighbouring query blocks of one head and shares their key tiles in its L2.
// G = 2: pairs as sparse_pair() defines them, under the head's stride with the least total
// kept-block union (the smallest such stride on ties); G = 1: one query block per workgroup.
constexpr int XCD_RUN = 16;

__device__ __forceinline__ bool flash_unit(const Problem& P, int G, int gid, int* bh, int* qa, int* qb) {
  const int x = gid % 8, k = gid / 8;
  const int u = (k / XCD_RUN) * 8 * XCD_RUN + x * XCD_RUN + (k % XCD_RUN);
  const int BH = P.B * P.H;
  const int nd = P.dense_q1 - P.dense_q0;
  const int nu_d = flash_dense_units(G, nd);
  const int nu_s = flash_units_per_head(G, P.Mq, nd) - nu_d;
  if (u >= BH * (nu_d + nu_s)) return false;
  int j;
  if (u < BH * nu_d) {
    *bh = u / nu_d;
    j = u % nu_d;
  } else {
    *bh = (u - BH * nu_d) / nu_s;
    j = nu_d + (u - BH * nu_d) % nu_s;
  }
  int stride = 1;
  if (G == 2 && j >= nu_d && P.pair_plan) {
    const long long* tot = P.pair_plan + (size_t)*bh * PAIR_STRIDES;
    long long best = tot[0];
    for (int c = 1; c < PAIR_STRIDES; ++c)
      if (tot[c] < best) {
        best = tot[c];
        stride = c + 1;
      }
  }
  flash_unit_blocks(G, P.Mq, P.dense_q0, P.dense_q1, stride, j, qa, qb);
  return true;
}

// WPQ waves per query block (block_q / 32), G query blocks per workgroup; WPQ * G = 4.
// QK8: the fp8-QK flavour (E4M3 key tiles and query fragments, scaled products for S).
template <int D, int WPQ, int G, bool QK8>
__device__ __forceinline__ void sparse_flash_body(const Problem& P) {
  __shared__ FlashSmem<D, QK8> sm;
  constexpr int KCH = D / 8;                 // 16-byte chunks per bf16 K row (and per V^T row pair)
  constexpr int SLOTS = 64 * D / 8;          // 16-byte slots per bf16 tile matrix
  constexpr int PER_THREAD = SLOTS / 256;
  constexpr int TILE_BYTES = 64 * D * 2;
  constexpr int KCH8 = D / 16;               // 16-byte chunks per E4M3 K row
  constexpr int PER_THREAD8 = 64 * D / 16 / 256;
  constexpr uint32_t TB8 = 64 * D + 64;      // E4M3 tile: rows, then the rows' scale codes
  int bh, qa, qb_;
  if (!flash_unit(P, G, blockIdx.x, &bh, &qa, &qb_)) return;
  // the wave index is uniform: read it into a scalar so that every per-wave decision (which
  // query block, whether the wave works on a tile) is a scalar branch, not an exec mask
  const int tid = threadIdx.x, l = tid % 64, h32 = l / 32, c32 = l % 32;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int g = w / WPQ;                     // this wave's query block within the pair
  const int b = bh / P.H, hh = bh % P.H;
  const uint16_t* Kb = static_cast<const uint16_t*>(P.k.p) + (int64_t)b * P.k.sb + (int64_t)hh * P.k.sh;
  const uint16_t* Vb = static_cast<const uint16_t*>(P.v.p) + (int64_t)b * P.v.sb + (int64_t)hh * P.v.sh;
  const uint16_t* Qb = static_cast<const uint16_t*>(P.q.p) + (int64_t)b * P.q.sb + (int64_t)hh * P.q.sh;

  // per query block of the pair
  int qb[2], nk[2], ne[2];
  bool dense[2], valid[2];
  uint64_t kw[2];
  const int* elist[2];
#pragma unroll
  for (int gg = 0; gg < 2; ++gg) {
    qb[gg] = gg == 0 ? qa : qb_;
    valid[gg] = qb[gg] >= 0;
    const int qq = valid[gg] ? qb[gg] : qa;
    const size_t row = (size_t)bh * P.Mq + qq;
    dense[gg] = qq >= P.dense_q0 && qq < P.dense_q1;
    nk[gg] = valid[gg] ? uniform(P.kept_cnt[row]) : 0;
    ne[gg] = (valid[gg] && !dense[gg]) ? uniform(P.extra_cnt[row]) : 0;
    const int nwords = P.Mpad / 64;
    kw[gg] = (valid[gg] && l < nwords) ? P.kept_bm[row * nwords + l] : 0ull;
    elist[gg] = P.extra_idx + row * MAX_EXTRA;
  }
  int cent_sel = 0;
  if (P.mode == 0) {
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
      if (valid[gg] && !dense[gg] && nk[gg] < P.M) cent_sel |= 1 << gg;
  }
  TileIter it{kw[0], kw[1], kw[0] | kw[1], 0, cent_sel ? P.Mpad : 0, cent_sel};

  // this wave's 32 query rows: Q^T operand fragments
  const bool wave_on = valid[g];
  const int q0 = ((valid[g] ? qb[g] : qb[0]) + P.q0) * P.bq + 32 * (w % WPQ);
  bf16x8_t qf[QK8 ? 1 : D / 16];
  i32x8_t qf8[QK8 ? D / 64 : 1];
  int qcode = 127;
  if constexpr (!QK8) {
    const uint16_t* qr = Qb + (int64_t)(q0 + c32) * P.q.sn + 8 * h32;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qr + 16 * ks);
  } else {
    // E4M3 query row, scaled by its power of two: lane (h32, row) holds d = 64ks + 32h32 .. +31
    const uint16_t* qr = Qb + (int64_t)(q0 + c32) * P.q.sn + 32 * h32;
    float x[D / 64][32];
    float amax = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 raw = *reinterpret_cast<const uint4*>(qr + 64 * ks + 8 * c);
        const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[ks][8 * c + 2 * e] = __uint_as_float(wd[e] << 16);
          x[ks][8 * c + 2 * e + 1] = __uint_as_float(wd[e] & 0xFFFF0000u);
          amax = fmaxf(amax, fmaxf(fabsf(x[ks][8 * c + 2 * e]), fabsf(x[ks][8 * c + 2 * e + 1])));
        }
      }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax), false, false);
    amax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));   // the whole row
    const int ex = e4m3_scale_exp(amax);
    qcode = ex + 127;
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
#pragma unroll
      for (int e = 0; e < 32; ++e) x[ks][e] = ldexpf(x[ks][e], -ex);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint2 p = pack8_e4m3(&x[ks][8 * c]);
        qf8[ks][2 * c] = static_cast<int>(p.x);
        qf8[ks][2 * c + 1] = static_cast<int>(p.y);
      }
    }
  }

  // per-lane byte offsets of the tile loads.  Instruction u of wave w moves 16-byte slot
  // s = (4u + w) * 64 + l of the tile: K row r = s / KCH, chunk c = s % KCH, stored at swizzled
  // chunk kswz(r, c); transposed V row vr = s / 8, chunk vc = s % 8, stored at vswz(vr, vc).
  // Instruction u moves rows KSTEP*u further on, which leaves both swizzles unchanged (they
  // depend on the row's low 4 bits, and KSTEP is a multiple of 16), so each offset is the lane's
  // u = 0 offset plus a wave-uniform step.
  const uint32_t ksn_b = static_cast<uint32_t>(P.k.sn) * 2u;
  const uint32_t vsn_b = static_cast<uint32_t>(P.v.sn) * 2u;
  constexpr int KSTEP = QK8 ? 256 / KCH8 : 256 / KCH;   // K rows per instruction
  static_assert(KSTEP % 16 == 0, "row step must keep the swizzle");
  uint32_t krow0, kcol0;
  if constexpr (QK8) {
    const int s0 = w * 64 + l, r = s0 / KCH8, c = s0 % KCH8;
    krow0 = r;
    kcol0 = kswz8<D>(r, c) * 16;
  } else {
    const int s0 = w * 64 + l, r = s0 / KCH, c = s0 % KCH;
    krow0 = r;
    kcol0 = kswz<D>(r, c) * 16;
  }
  uint32_t voff0;
  {
    const int s0 = w * 64 + l, vr = s0 / 8, vc = s0 % 8;
    voff0 = vr * 128 + vswz(vr, vc) * 16;
  }

  // ---- issue the asynchronous loads of one tile into buffer bf
  auto issue = [&](const TileDesc& t, int bf) {
    char* kd = reinterpret_cast<char*>(sm.k[bf]) + w * 1024;
    char* vd = reinterpret_cast<char*>(sm.v[bf]) + w * 1024;
    const void* kbase;
    uint32_t krow_b;
    const void* vbase;
    if (t.kind == 0) {
      kbase = Kb + (int64_t)t.idx * 64 * P.k.sn;
      krow_b = ksn_b;
      vbase = P.v_t + ((size_t)bh * P.M + t.idx) * D * 64;
    } else {
      kbase = P.kbar_bf + ((size_t)bh * P.Mpad + t.idx) * D;
      krow_b = D * 2;
      vbase = P.vbar_t + ((size_t)bh * (P.Mpad / 64) + t.idx / 64) * D * 64;
    }
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase, TILE_BYTES);
    if constexpr (QK8) {
      const uint8_t* k8base = t.kind == 0 ? P.k8 + ((size_t)bh * P.M + t.idx) * TB8
                                          : P.kb8 + ((size_t)bh * (P.Mpad / 64) + t.idx / 64) * TB8;
      const __amdgpu_buffer_rsrc_t kr = make_rsrc(k8base, TB8);
#pragma unroll
      for (int u = 0; u < PER_THREAD8; ++u) buf_to_lds16s(kr, krow0 * D + kcol0, u * KSTEP * D, kd + u * 4096);
      if (w == 0 && l < 4) buf_to_lds16(kr, 64 * D + 16 * l, sm.ke[bf]);   // the rows' scale codes
#pragma unroll
      for (int u = 0; u < PER_THREAD; ++u) buf_to_lds16s(vr, voff0, u * 4096, vd + u * 4096);
    } else {
      const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase, 64u * krow_b);
#pragma unroll
      for (int u = 0; u < PER_THREAD; ++u) {
        buf_to_lds16s(kr, krow0 * krow_b + kcol0, u * KSTEP * krow_b, kd + u * 4096);
        buf_to_lds16s(vr, voff0, u * 4096, vd + u * 4096);
      }
    }
    if (t.kind == 2 && w == 0) {
      // the 64 biases of each query block: ln(m) / scale for key block j = t.idx + l, where
      // m = 64 minus the block's extra tokens for a block not kept, -inf where m = 0 (kept
      // blocks, blocks taken whole as extra tokens, padding).  The extra tokens of the tile's
      // 64 blocks are counted into the bias row itself (integer counters, LDS atomics from
      // this wave only), then replaced by the biases.  The extra lists arrived in LDS with
      // the first tile; the buffer is free (every wave has passed this iteration's barrier).
      const int c = t.idx >> 6;
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        if (!valid[gg]) continue;
        int* cnt = reinterpret_cast<int*>(sm.bias[bf][gg]);
        cnt[l] = 0;
        wave_lds_sync();
        const int n = gg ? ne[1] : ne[0];
#pragma unroll
        for (int e = 0; e < MAX_EXTRA / 64; ++e) {
          const int p = l + 64 * e;
          if (p < n) {
            const int blk = sm.eidx[gg][p] >> 6;
            if ((blk >> 6) == c) atomicAdd(&cnt[blk & 63], 1);
          }
        }
        wave_lds_sync();
        const uint64_t kword = readlane64(gg ? it.w1 : it.w0, c);
        const int m = (t.idx + l < P.M && !((kword >> l) & 1ull)) ? 64 - cnt[l] : 0;
        wave_lds_sync();
        sm.bias[bf][gg][l] = m > 0 ? __logf(static_cast<float>(m)) / P.scale : -__builtin_inff();
      }
    }
  };

  // ---- extra tokens e0 .. e0+63 of block gg into buffer bf, gathered row by row (rows past
  // the count repeat the first token and get bias -inf): K rows into the swizzled key layout, V
  // rows row-major with the 16-byte chunk c of row r at position c ^ (r & 4)
  auto issue_extra = [&](int gg, int e0, int bf) {
    char* kd = reinterpret_cast<char*>(sm.k[bf]) + w * 1024;
    char* vd = reinterpret_cast<char*>(sm.v[bf]) + w * 1024;
    const int cnt = gg ? ne[1] : ne[0];
    const uint32_t vcol0 = ((static_cast<uint32_t>(l) % KCH) ^ (krow0 & 4)) << 4;
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int r = krow0 + KSTEP * u;
      const int e = e0 + r < cnt ? e0 + r : e0;
      const size_t tok = static_cast<uint32_t>(sm.eidx[gg][e]);
      glb_to_lds16(reinterpret_cast<const char*>(Kb) + tok * ksn_b + kcol0, kd + u * 4096);
      glb_to_lds16(reinterpret_cast<const char*>(Vb) + tok * vsn_b + vcol0, vd + u * 4096);
    }
    if (w == 0) sm.bias[bf][gg][l] = e0 + l < cnt ? 0.f : -__builtin_inff();
  };
  // ---- step j of the pair's extra tokens into buffer bf: rows 0-31 are block 0's tokens
  // 32j .. 32j+31, rows 32-63 block 1's (rows past a block's count repeat one of its tokens, or
  // the other block's when it has none, and get bias -inf), so each half of the workgroup works
  // on its own block's half of the tile
  const int ne0 = ne[0], ne1 = ne[1];
  auto issue_extra_pair = [&](int j, int bf) {
    char* kd = reinterpret_cast<char*>(sm.k[bf]) + w * 1024;
    char* vd = reinterpret_cast<char*>(sm.v[bf]) + w * 1024;
    const uint32_t vcol0 = ((static_cast<uint32_t>(l) % KCH) ^ (krow0 & 4)) << 4;
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int r = krow0 + KSTEP * u;
      const bool second = r >= 32;
      const int cnt = second ? ne1 : ne0;
      const int e = 32 * j + (r & 31);
      const int* el = (second == (cnt > 0)) ? sm.eidx[1] : sm.eidx[0];
      const size_t tok = static_cast<uint32_t>(el[e < cnt ? e : 0]);
      glb_to_lds16(reinterpret_cast<const char*>(Kb) + tok * ksn_b + kcol0, kd + u * 4096);
      glb_to_lds16(reinterpret_cast<const char*>(Vb) + tok * vsn_b + vcol0, vd + u * 4096);
    }
    if (w == 0) {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
        sm.bias[bf][gg][l] = ((l >> 5) == gg && 32 * j + (l & 31) < (gg ? ne1 : ne0)) ? 0.f : -__builtin_inff();
    }
  };

  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16_t{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float sl2 = P.scale * LOG2E;
  // LDS read offsets: chunk (2ks + h32) of row r sits at byte ((32ks) ^ Y) within the row, with Y
  // a lane constant, so each read is one XOR with a compile-time constant.
  const uint32_t ak = c32 * (D * 2) + 16 * (kswz<D>(c32, 0) ^ h32);
  const uint32_t av = c32 * 128 + 16 * (vswz(c32, 0) ^ h32);
  // row-major V (extra-token tiles): element (key, d) at key * 2D + 16 * ((d / 8) ^ (key & 4)) +
  // 2 * (d % 8); this lane's keys all have key & 4 = 4 h32
  const uint32_t rmo = 8 * h32 * D + 16 * (c32 >> 3) + 2 * (c32 & 7);
  const uint32_t rmx = 64 * h32;
  const bf16x2_t ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

  // The score accumulators of a tile start from its per-key bias (centroid and extra tiles:
  // ln(m) * sqrt(d) in raw-score units, or -inf; kept tiles: 0).  Register r of half kt holds
  // key 32kt + (r/4)*8 + 4*h32 + r%4.  The bias is read from LDS before the next tile's
  // asynchronous copies are issued, so the read never has to wait for them.
  auto load_bias = [&](const float* bias, f32x16_t* s) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 bv = *reinterpret_cast<const float4*>(bias + 32 * kt + r4 * 8 + 4 * h32);
        s[kt][4 * r4 + 0] = bv.x;
        s[kt][4 * r4 + 1] = bv.y;
        s[kt][4 * r4 + 2] = bv.z;
        s[kt][4 * r4 + 3] = bv.w;
      }
  };

  // Lazy rescaling: the reference max moves (and the accumulator is rescaled) only when some
  // row's max grows by more than 8 (base 2), so probabilities stay below 2^8 and most steps skip
  // the rescale.  The result is the same softmax, referenced to a different constant.
  auto rescale = [&](float mx) {
    const float m_cand = fmaxf(m_run, mx);
    if (__any(m_cand > m_run + 8.f)) {
      const float m_new = m_cand == -__builtin_inff() ? m_run : m_cand;
      const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      m_run = m_new;
    }
  };
  // Base-2 row max of one 32-key half of the scores (the scale is positive, so the max is
  // taken on the raw scores).  Lanes l and l+32 hold the same rows, different keys.
  auto half_max = [&](const f32x16_t& sh) {
    float mx = sh[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sh[r]);
    mx *= sl2;
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };

  // ---- one tile for this wave's 32 query rows; s holds the tile's per-key biases (zeros for a
  // plain key tile) and receives the scores.  The tile is two online-softmax steps of 32
  // keys each, ordered so that the vector work of one half overlaps matrix work: the max of half
  // 0 runs under the score products of half 1, the max of half 1 under the value products of
  // half 0.  Within a half, the exponentials of one 16-key step overlap the products of the
  // previous one.
  auto compute = [&](int bf, f32x16_t* s, auto rm) {
    constexpr bool RM = decltype(rm)::value;   // V row-major (extra-token tiles)
    const uint32_t ak_ = ak, av_ = RM ? rmo : av;
    const char* kt_ = reinterpret_cast<const char*>(sm.k[bf]);
    const char* vt_ = reinterpret_cast<const char*>(sm.v[bf]);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      if constexpr (!QK8) {
        // S^T (keys 32kt..32kt+31) += K Q^T; K fragments of step ks+1 read during step ks
        bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kt_ + ak_ + kt * 32 * D * 2);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          bf16x8_t n = a;
          if (ks + 1 < D / 16)
            n = *reinterpret_cast<const bf16x8_t*>(kt_ + ((ak_ ^ (32u * (ks + 1))) + kt * 32 * D * 2));
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kt], 0, 0, 0);
          a = n;
        }
      } else {
        // S^T += (K 2^ek) (Q 2^eq)^T on E4M3 operands: lane (h32, key row) holds
        // d = 64ks + 32h32 .. +31 of its row, the same d order as the query fragments
        const int row = 32 * kt + c32;
        const int kcode = sm.ke[bf][row];
#pragma unroll
        for (int ks = 0; ks < D / 64; ++ks) {
          const int c0 = 4 * ks + 2 * h32;
          const uint4 lo = *reinterpret_cast<const uint4*>(kt_ + row * D + kswz8<D>(row, c0) * 16);
          const uint4 hi = *reinterpret_cast<const uint4*>(kt_ + row * D + kswz8<D>(row, c0 + 1) * 16);
          const i32x8_t a = {static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z),
                             static_cast<int>(lo.w), static_cast<int>(hi.x), static_cast<int>(hi.y),
                             static_cast<int>(hi.z), static_cast<int>(hi.w)};
          s[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf8[ks], s[kt], 0, 0, 0, kcode, 0,
                                                                  qcode);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // O^T += V^T P^T for one 16-key step ks; the probabilities (registers 8(ks%2)..+8 of half
    // ks/2) are rounded to bf16 and summed as rounded, like the product sees them.
    auto probs = [&](int ks, float nm, float& psum) {
      bf16x8_t pf;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pf[e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s[ks / 2][8 * (ks % 2) + e], sl2, nm)));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2_t pp = {pf[2 * e], pf[2 * e + 1]};
        psum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, psum, false);
      }
      return pf;
    };
    auto vread = [&](int ks, bf16x8_t* va) {
      const uint32_t off = av_ ^ (32u * ks);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        va[dt] = *reinterpret_cast<const bf16x8_t*>(vt_ + off + dt * 32 * 128);
    };
    // one fragment of a row-major V tile: element e = V[16ks + 8(e/4) + 4h32 + e%4][32dt + c32]
    auto vread_rm = [&](int ks, int dt) {
      const char* base = vt_ + (av_ + ((64u * dt) ^ rmx)) + ks * 32 * D;
      uint32_t x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x[e] = *reinterpret_cast<const uint16_t*>(base + (8 * (e >> 2) + (e & 3)) * 2 * D);
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
      const u32x4_t pk = {x[0] | (x[1] << 16), x[2] | (x[3] << 16), x[4] | (x[5] << 16), x[6] | (x[7] << 16)};
      return __builtin_bit_cast(bf16x8_t, pk);
    };
    float mx = half_max(s[0]);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      rescale(mx);
      const float nm = m_run == -__builtin_inff() ? 0.f : -m_run;
      float psum = 0.f;
      if constexpr (RM) {
        const bf16x8_t p0 = probs(2 * kt, nm, psum);
        const bf16x8_t p1 = probs(2 * kt + 1, nm, psum);
        // one fragment in registers at a time (scheduling fences keep the reads from piling up)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread_rm(2 * kt, dt), p0, o[dt], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (kt == 0) mx = half_max(s[1]);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread_rm(2 * kt + 1, dt), p1, o[dt], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        bf16x8_t va[D / 32], vb[D / 32];
        vread(2 * kt, va);
        const bf16x8_t p0 = probs(2 * kt, nm, psum);
        vread(2 * kt + 1, vb);
        const bf16x8_t p1 = probs(2 * kt + 1, nm, psum);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt], p0, o[dt], 0, 0, 0);
        if (kt == 0) mx = half_max(s[1]);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[dt], p1, o[dt], 0, 0, 0);
      }
      l_run += psum;
    }
  };

  // ---- one 32-key half h of a gathered tile (row-major V): the score products of K rows
  // 32h..32h+31, the online-softmax step and the value products of the half's two 16-key steps
  auto compute_half_rm = [&](int bf, int h, f32x16_t& sh) {
    const char* kt_ = reinterpret_cast<const char*>(sm.k[bf]) + h * 32 * D * 2;
    const char* vt_ = reinterpret_cast<const char*>(sm.v[bf]);
    __builtin_amdgcn_s_setprio(1);
    {
      bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kt_ + ak);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        bf16x8_t n = a;
        if (ks + 1 < D / 16) n = *reinterpret_cast<const bf16x8_t*>(kt_ + (ak ^ (32u * (ks + 1))));
        sh = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sh, 0, 0, 0);
        a = n;
      }
    }
    __builtin_amdgcn_s_setprio(0);
    rescale(half_max(sh));
    const float nm = m_run == -__builtin_inff() ? 0.f : -m_run;
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      bf16x8_t pf;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pf[e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sh[8 * st + e], sl2, nm)));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2_t pp = {pf[2 * e], pf[2 * e + 1]};
        psum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, psum, false);
      }
      // one fragment of the row-major V tile at a time: element e = V[16ks + 8(e/4) + 4h32 +
      // e%4][32dt + c32], ks = 2h + st
      const int ks = 2 * h + st;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const char* base = vt_ + (rmo + ((64u * dt) ^ rmx)) + ks * 32 * D;
        uint32_t x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          x[e] = *reinterpret_cast<const uint16_t*>(base + (8 * (e >> 2) + (e & 3)) * 2 * D);
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        const u32x4_t pk = {x[0] | (x[1] << 16), x[2] | (x[3] << 16), x[4] | (x[5] << 16), x[6] | (x[7] << 16)};
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, pk), pf, o[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    l_run += psum;
  };

  if (tid < 64) sm.zero[tid] = 0.f;       // visible after the first barrier of the loop
  // the pair's extra-token lists go to LDS now (wave g copies block g's, 16 bytes a lane) and
  // arrive with the first tile, so the gather after the main loop reads its indices from LDS
  if (w < G && ne[w] > 0)
    buf_to_lds16(make_rsrc(elist[w], MAX_EXTRA * 4), static_cast<uint32_t>(l) * 16u, sm.eidx[w]);
  TileDesc cur = it.next();
  int bf = 0;
  issue(cur, 0);
  for (;;) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const bool mine = wave_on && ((cur.sel >> g) & 1);
    f32x16_t s[2];
    if (mine) load_bias(cur.kind != 0 ? sm.bias[bf][g] : sm.zero, s);
    const TileDesc nxt = it.next();
    if (nxt.kind != 3) issue(nxt, bf ^ 1);
    if (mine) compute(bf, s, BoolC<false>{});
    if (nxt.kind == 3) break;
    cur = nxt;
    bf ^= 1;
  }

  // ---- bf16: the extra tokens, gathered straight to LDS and double-buffered like the main
  // loop's tiles; pairs of 64-row blocks take 32 tokens of each block per step (every wave
  // busy), single 128-row blocks up to 4 tiles of 64
  if constexpr (!QK8 && G == 2) {
    // step i: 32 tokens of each block of the pair, each half of the workgroup on its own block
    const int nstep = (max(ne0, ne1) + 31) / 32;
    const int neg = g ? ne1 : ne0;
    if (nstep > 0) {
      __syncthreads();                    // every wave is done with the main loop's buffers
      issue_extra_pair(0, 0);
#pragma unroll 1
      for (int i = 0; i < nstep; ++i) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (i + 1 < nstep) issue_extra_pair(i + 1, (i + 1) & 1);
        if (wave_on && 32 * i < neg) {
          f32x16_t sh;
          const float* bias = sm.bias[i & 1][g] + 32 * g;
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const float4 bv = *reinterpret_cast<const float4*>(bias + r4 * 8 + 4 * h32);
            sh[4 * r4 + 0] = bv.x;
            sh[4 * r4 + 1] = bv.y;
            sh[4 * r4 + 2] = bv.z;
            sh[4 * r4 + 3] = bv.w;
          }
          compute_half_rm(i & 1, g, sh);
        }
      }
    }
  } else if constexpr (!QK8) {
    // tile j: block 0's tiles 0 .. nx0-1, then block 1's
    const int nx0 = (ne[0] + 63) / 64, nx = nx0 + (ne[1] + 63) / 64;
    auto issue_tile = [&](int j) { issue_extra(j < nx0 ? 0 : 1, 64 * (j < nx0 ? j : j - nx0), j & 1); };
    if (nx > 0) {
      __syncthreads();                    // every wave is done with the main loop's buffers
      issue_tile(0);
#pragma unroll 1
      for (int i = 0; i < nx; ++i) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const int gg = i < nx0 ? 0 : 1;
        if (i + 1 < nx) issue_tile(i + 1);
        if (wave_on && g == gg) {
          f32x16_t s[2];
          load_bias(sm.bias[i & 1][gg], s);
          compute(i & 1, s, BoolC<true>{});
        }
      }
    }
  }

  // ---- fp8-QK: the extra tokens, up to 4 gathered 64-token tiles per query block, loaded
  // synchronously after the loop: E4M3 key rows (and their scale codes) from the quantised
  // tiles; V rows through registers, stored transposed (with the same key permutation and
  // swizzle as the pre-transposed tiles).
  if constexpr (QK8) {
#pragma unroll 1
    for (int gg = 0; gg < G; ++gg) {
      const int cnt = ne[gg];
      const int* el = sm.eidx[gg];
#pragma unroll 1
      for (int e0 = 0; e0 < cnt; e0 += 64) {
        __syncthreads();
        uint16_t* vd = sm.v[0];
#pragma unroll
        for (int u = 0; u < PER_THREAD8; ++u) {
          const int sl = (u * 4 + w) * 64 + l;
          const int r = sl / KCH8, c = sl % KCH8;
          const int e = e0 + r < cnt ? e0 + r : e0;             // padding rows reuse a real token
          const uint32_t tok = static_cast<uint32_t>(el[e]);
          const uint8_t* trow = P.k8 + ((size_t)bh * P.M + tok / 64) * TB8;
          *reinterpret_cast<uint4*>(sm.k[0] + r * D + kswz8<D>(r, c) * 16) =
              *reinterpret_cast<const uint4*>(trow + (tok % 64) * D + c * 16);
          if (c == 0) sm.ke[0][r] = trow[64 * D + tok % 64];
        }
#pragma unroll
        for (int u = 0; u < PER_THREAD; ++u) {
          const int sl = (u * 4 + w) * 64 + l;
          const int r = sl / KCH, c = sl % KCH;
          const int e = e0 + r < cnt ? e0 + r : e0;
          const uint32_t tok = static_cast<uint32_t>(el[e]);
          const uint4 vv = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(Vb) +
                                                           (size_t)tok * vsn_b + c * 16);
          const uint16_t* vx = reinterpret_cast<const uint16_t*>(&vv);
          const int pos = vt_pos(r);
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int dr = c * 8 + x;                         // d row of the transposed tile
            vd[dr * 64 + (vswz(dr, pos >> 3) << 3) + (pos & 7)] = vx[x];
          }
        }
        if (tid < 64) sm.bias[0][gg][tid] = e0 + tid < cnt ? 0.f : -__builtin_inff();
        __syncthreads();
        if (wave_on && g == gg) {
          f32x16_t s[2];
          load_bias(sm.bias[0][gg], s);
          compute(0, s, BoolC<false>{});
        }
      }
    }
  }

  if (!wave_on) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  uint16_t* Ob = static_cast<uint16_t*>(const_cast<void*>(P.o.p)) + (int64_t)b * P.o.sb +
                 (int64_t)hh * P.o.sh + (int64_t)(q0 + c32) * P.o.sn;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d0 = 32 * dt + 8 * gq + 4 * h32;
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      bf16x4_t pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = static_cast<__bf16>(o[dt][4 * gq + e] * inv);
      *reinterpret_cast<bf16x4_t*>(Ob + d0) = pk;
    }
}

template <int D, int WPQ, int G>
__global__ __launch_bounds__(256, 2) void sparse_flash_bf16_kernel(Problem P) {
  sparse_flash_body<D, WPQ, G, false>(P);
}

// the fp8-QK flavour: E4M3 score products, bf16 softmax and P V
template <int D, int WPQ, int G>
__global__ __launch_bounds__(256, 2) void sparse_flash_fp8qk_kernel(Problem P) {
  sparse_flash_body<D, WPQ, G, true>(P);
}

hipError_t launch_sparse_flash(const Problem& P, hipStream_t stream) {
  if (P.dtype == 0) {
    const int G = P.bq == 64 ? 2 : 1;
    const int units = P.B * P.H * flash_units_per_head(G, P.Mq, P.dense_q1 - P.dense_q0);
    const int per_round = 8 * XCD_RUN;
    dim3 grid((units + per_round - 1) / per_round * per_round);
    if (P.fp8qk) {
      if (P.bq == 64) {
        if (P.d == 128) hipLaunchKernelGGL((sparse_flash_fp8qk_kernel<128, 2, 2>), grid, dim3(256), 0, stream, P);
        else hipLaunchKernelGGL((sparse_flash_fp8qk_kernel<64, 2, 2>), grid, dim3(256), 0, stream, P);
      } else {
        if (P.d == 128) hipLaunchKernelGGL((sparse_flash_fp8qk_kernel<128, 4, 1>), grid, dim3(256), 0, stream, P);
        else hipLaunchKernelGGL((sparse_flash_fp8qk_kernel<64, 4, 1>), grid, dim3(256), 0, stream, P);
      }
    } else if (P.bq == 64) {
      if (P.d == 128) hipLaunchKernelGGL((sparse_flash_bf16_kernel<128, 2, 2>), grid, dim3(256), 0, stream, P);
      else hipLaunchKernelGGL((sparse_flash_bf16_kernel<64, 2, 2>), grid, dim3(256), 0, stream, P);
    } else {
      if (P.d == 128) hipLaunchKernelGGL((sparse_flash_bf16_kernel<128, 4, 1>), grid, dim3(256), 0, stream, P);
      else hipLaunchKernelGGL((sparse_flash_bf16_kernel<64, 4, 1>), grid, dim3(256), 0, stream, P);
    }
  } else {
    return launch_sparse_flash_f32(P, stream);
  }
  return hipGetLastError();
}

}  // namespace solattn
