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
  float* scores;
  int* kept_cnt;
  int* kept_idx;
  uint64_t* kept_bm;     // kept blocks as a bitmap: word j/64, bit j%64
  uint8_t* mult;
  float* cbias;          // ln(centroid multiplicity) / scale (a raw-score offset), -inf where it is 0
  int* extra_cnt;
  int* extra_idx;
  uint2* extra_buf;      // per query block, token slice and wave: (score bits, token) candidates
  int* extra_part;       // per query block, token slice and wave: entries left after the final cut
  int* extra_flag;       // per query block: 1 when the seeded threshold left too few candidates
  int extra_slices;      // token slices of the extra-token selection
  uint8_t* k8;           // fp8-QK: E4M3 key tiles [B*H, M] of 64*d bytes + 64 scale codes
  uint8_t* kb8;          // fp8-QK: E4M3 pooled-key tiles [B*H, Mpad/64], same layout
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

// Token slices of the extra-token selection: enough workgroups to fill the chip, at most 4.
__host__ __device__ inline int extra_slice_count(int B, int H, int Mq) {
  const long groups = (long)((Mq + 31) / 32) * B * H;
  long s = (1536 + groups - 1) / groups;
  return s < 1 ? 1 : (s > 4 ? 4 : (int)s);
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
