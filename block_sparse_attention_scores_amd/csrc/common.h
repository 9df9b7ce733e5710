// Shared definitions of the libsolattn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace solattn {

// A strided [B, H, N, d] tensor: element strides of the b, h and n axes; d is contiguous.
struct Tensor {
  const void* p;
  int64_t sb, sh, sn;
};

// Everything one call's kernels need, passed by value to each launch.
struct Problem {
  int B, H, N, d;
  int bq, bk;            // query / key block sizes
  int Mq, M, Mpad;       // query blocks (of the computed window), key blocks, key blocks rounded up to 64
  int q0;                // first query block of the window (global index); workspace rows are local
  int mode;              // 0 sol, 1 sla, 2 static local 3-D neighbourhood
  int dtype;             // element type of q, k, v, out: 0 bf16, 1 fp32
  int fp8qk;             // bf16 tensors, QK^T products on E4M3 operands (the fp8-QK flavour)
  float tau;
  int keep_all;          // tau == -inf: every block kept
  int k_sla;             // sla: ceil(keep_percent * M / 100)
  int sink_blocks;       // key blocks overlapping [0, sink_range)
  int extra;             // extra tokens per query block (0..256)
  int exact_extra;       // select extra tokens exactly from the start (no seeded pass)
  int dense_q0, dense_q1;  // window-local query blocks [dense_q0, dense_q1) attend every key
  int frames, height, width;  // local 3-D mode: the token grid (frames*height*width == N)
  float scale;           // 1/sqrt(d)
  Tensor q, k, v, o;
  // workspace
  float* qbar;
  float* kbar;
  float* vbar;
  float* scores;         // [B*H, Mq, Mpad]: row stride Mpad
  int* kept_cnt;
  int* kept_idx;         // ascending kept lists (written when keep_lists is set)
  uint64_t* kept_bm;     // kept blocks as a bitmap: word j/64, bit j%64
  uint8_t* mult;         // centroid multiplicities (written when keep_lists is set)
  int keep_lists;        // write kept_idx and mult (fp32 tensors, or the caller asked to keep them)
  int* extra_cnt;
  int* extra_idx;
  uint2* extra_buf;      // per query block and candidate list: (score bits, token) candidates
  int* extra_part;       // per query block and candidate list: entries left after the final cut
  uint32_t* extra_seed;  // per query block: seeded threshold key of the extra-token selection
  int extra_lists;       // candidate lists per query block (extra_buf rows hold this many)
  int* extra_flag;       // per query block: 1 when the seeded threshold left too few candidates
  int extra_slices;      // token slices of the extra-token selection
  uint8_t* k8;           // fp8-QK: E4M3 key tiles [B*H, M] of 64*d bytes + 64 scale codes
  uint8_t* kb8;          // fp8-QK: E4M3 pooled-key tiles [B*H, Mpad/64], same layout
  long long* pair_plan;  // [B*H, PAIR_STRIDES]: kept-block union summed over the pairs of each
                         // pairing stride (bf16 kernel with 64-row query blocks; else null)
  uint16_t* kbar_bf;
  uint16_t* vbar_t;
  uint16_t* v_t;
};

constexpr int MAX_EXTRA = 256;
// The local 3-D mode marks a query block's neighbourhood in a bitmap of M bits in LDS.
constexpr int MAX_BLOCKS_LOCAL3D = 65536;
// The bf16 attention kernel holds a query block's kept-block bitmap in one 64-bit word per lane.
constexpr int MAX_BLOCKS_BF16 = 64 * 64;
// Candidate buffer per (query block, token slice, wave) of the extra-token selection.  It is cut
// back to the best extra_tokens entries only when one more 32-token step could overflow it,
// which for the workloads here almost never happens.
constexpr int EXTRA_CAP = 1024;

// Pairs of 64-row query blocks of the bf16 attention kernel (one pair per workgroup; the pair
// walks the union of its two kept-block sets, so pairs whose sets overlap most waste least).
// The dense query blocks [dq0, dq0 + nd) pair with their neighbours.  The other Ms = Mq - nd
// blocks, numbered 0..Ms-1 in order with the dense run cut out, pair under a stride s chosen
// per head: in each run of 2s blocks, block t pairs with block t + s; the blocks after the last
// whole run pair with their neighbours.  Stride 1 is neighbour pairing.  A block's result does
// not depend on its partner.
constexpr int PAIR_STRIDES = 8;          // candidate strides 1..PAIR_STRIDES

__host__ __device__ inline int flash_pairs_per_head(int Mq, int nd) {
  return (nd + 1) / 2 + (Mq - nd + 1) / 2;
}

// The p-th pair (0 <= p < (Ms+1)/2) of the non-dense blocks under stride s, as query block
// numbers; *b = -1 when the last block has no partner.
__host__ __device__ inline void sparse_pair(int p, int s, int Ms, int dq0, int nd, int* a, int* b) {
  const int C = Ms / (2 * s);                // whole runs of 2s blocks
  int ia, ib;
  if (p < C * s) {
    const int c = p / s, t = p - c * s;
    ia = 2 * s * c + t;
    ib = ia + s;
  } else {
    ia = 2 * C * s + 2 * (p - C * s);
    ib = ia + 1 < Ms ? ia + 1 : -1;
  }
  *a = ia < dq0 ? ia : ia + nd;
  *b = ib < 0 ? -1 : (ib < dq0 ? ib : ib + nd);
}

// Work units of one head for the attention kernel with G query blocks per workgroup (G = 2:
// pairs; G = 1: single blocks): the dense blocks' units first, then the others.
__host__ __device__ inline int flash_units_per_head(int G, int Mq, int nd) {
  return G == 2 ? flash_pairs_per_head(Mq, nd) : Mq;
}
__host__ __device__ inline int flash_dense_units(int G, int nd) {
  return G == 2 ? (nd + 1) / 2 : nd;
}

// Query blocks of unit j (0 <= j < flash_units_per_head) of a head, dense query blocks
// [dq0, dq1); stride: the head's pairing stride (G = 2).  *qb = -1 when the unit has one block.
__host__ __device__ inline void flash_unit_blocks(int G, int Mq, int dq0, int dq1, int stride, int j,
                                                  int* qa, int* qb) {
  const int nd = dq1 - dq0, nu_d = flash_dense_units(G, nd);
  if (j < nu_d) {
    *qa = dq0 + j * G;
    *qb = (G == 2 && *qa + 1 < dq1) ? *qa + 1 : -1;
  } else if (G == 1) {
    const int r = j - nu_d;
    *qa = r < dq0 ? r : r + nd;
    *qb = -1;
  } else {
    sparse_pair(j - nu_d, stride, Mq - nd, dq0, nd, qa, qb);
  }
}

// Query blocks per workgroup of the extra-token selection's first pass: 128 for 16-bit tensors
// (four waves of 32 that share each key tile staged in LDS), 32 for fp32 (four waves that take
// turns over the token steps of the same 32 blocks).
constexpr int EXTRA_GROUP_BF16 = 128;
constexpr int EXTRA_GROUP_F32 = 32;

// Token slices of the extra-token selection and candidate lists per query block.  fp32: enough
// slices for about 1536 workgroups (at most 4), one list per slice and wave.  16-bit: the slice
// count (at most 16) whose workgroups fill the last of their rounds best (EXTRA_SLOTS resident
// at a time: three per compute unit of the 256), preferring fewer slices on near ties; one list
// per slice.
constexpr int EXTRA_SLOTS = 768;
__host__ __device__ inline void extra_split(bool f32, int B, int H, int Mq, int* slices, int* lists) {
  if (f32) {
    const long groups = (long)((Mq + EXTRA_GROUP_F32 - 1) / EXTRA_GROUP_F32) * B * H;
    long s = (1536 + groups - 1) / groups;
    s = s < 1 ? 1 : (s > 4 ? 4 : s);
    *slices = (int)s;
    *lists = 4 * (int)s;
    return;
  }
  const long groups = (long)((Mq + EXTRA_GROUP_BF16 - 1) / EXTRA_GROUP_BF16) * B * H;
  int best = 1;
  double best_eff = -1.0;
  for (int s = 1; s <= 16; ++s) {
    const long wg = groups * s;
    const long rounds = (wg + EXTRA_SLOTS - 1) / EXTRA_SLOTS;
    // a fill of one round or less leaves the chip idle; count it by its share of the slots
    const double eff = (double)wg / (double)(rounds * EXTRA_SLOTS);
    if (eff > best_eff + 0.02) {
      best_eff = eff;
      best = s;
    }
  }
  *slices = best;
  *lists = best;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Order-preserving map of a float to uint32 (larger float -> larger key); -0 maps like +0.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Position of key `kk` (0..63) inside a 64-key transposed V tile.  Inside each group of 16 keys
// bits 2 and 3 of the index are swapped, so that the 8 keys one lane feeds to the PV matrix
// instruction (given the 32x32 accumulator layout of the score tile) sit next to each other.
__host__ __device__ __forceinline__ int vt_pos(int kk) {
  return (kk & ~0xC) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

// ---- staging of key tiles in LDS (the attention kernel and the extra-token selection)

typedef __attribute__((address_space(3))) void lds_void_t;

// Asynchronous 16-byte global -> LDS copy through a buffer resource: lane l's 16 bytes land at
// `wave_dst` + 16*l (the same `wave_dst` for the whole wave); `voff` is the lane's byte offset
// from the resource base.  Out-of-range offsets read zero.
__device__ __forceinline__ void buf_to_lds16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, void* wave_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(wave_dst), 16, voff, 0, 0, 0);
}

// The same with a wave-uniform byte offset `soff` added to every lane's.
__device__ __forceinline__ void buf_to_lds16s(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                              void* wave_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(wave_dst), 16, voff, soff, 0, 0);
}

// Asynchronous 16-byte global -> LDS gather: each lane names its own source address; lane l's
// 16 bytes land at `wave_dst` + 16*l.
typedef __attribute__((address_space(1))) void global_void_t;
__device__ __forceinline__ void glb_to_lds16(const void* src, void* wave_dst) {
  __builtin_amdgcn_global_load_lds((global_void_t*)(const_cast<void*>(src)), (lds_void_t*)(wave_dst), 16, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// LDS swizzle of bf16 key rows: the 16-byte chunk c of row r is stored at chunk position
// kswz(r, c), so that any 16 consecutive rows read at one logical chunk hit 16 distinct 16-byte
// bank groups.  An involution in c: loading global chunk kswz(r, p) into position p stores it
// where it belongs.
template <int D>
__host__ __device__ __forceinline__ int kswz(int r, int c) {
  if constexpr (D == 128) return c ^ (r & 15);        // 256-byte rows
  else return c ^ ((r >> 1) & 7);                     // 128-byte rows
}

// E4M3 scaling (the fp8-QK flavour): e = the smallest integer with amax <= 448 * 2^e
// (amax > 0; 0 for amax = 0), clamped to the E8M0 code range [-127, 127].
__device__ __forceinline__ int e4m3_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int k;
  (void)frexpf(amax, &k);                     // amax in [2^(k-1), 2^k)
  const int e = (ldexpf(amax, 9 - k) <= 448.f) ? k - 9 : k - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Eight values, already scaled into [-448, 448], as eight E4M3 bytes (nearest, ties to even),
// little-endian in a uint2.
__device__ __forceinline__ uint2 pack8_e4m3(const float* x) {
  uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0u, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);
  uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0u, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], hi, true);
  return make_uint2(lo, hi);
}

}  // namespace solattn
