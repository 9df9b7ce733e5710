// libsolattn C ABI: argument validation, workspace planning and the launch sequence
//   block_pool -> block_score -> block_select -> extra_select -> sparse_flash_fwd
// on the caller's stream (see include/solattn.h for the contract).  The local 3-D mode
// needs no block scores and skips block_score.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/solattn.h"
#include "common.h"
#include "launch.h"

using solattn::Problem;
using solattn::Tensor;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Strides {
  int64_t sb, sh, sn;
};

Strides resolve(const int64_t* s, int H, int N, int d) {
  if (s[0] == 0 && s[1] == 0 && s[2] == 0) return {(int64_t)H * N * d, (int64_t)N * d, (int64_t)d};
  return {s[0], s[1], s[2]};
}

// Byte range [lo, hi) touched by a strided tensor.
void extent(const void* p, Strides s, int B, int H, int N, int d, size_t es, uintptr_t* lo, uintptr_t* hi) {
  const uintptr_t base = reinterpret_cast<uintptr_t>(p);
  const int64_t last = (int64_t)(B - 1) * s.sb + (int64_t)(H - 1) * s.sh + (int64_t)(N - 1) * s.sn + (d - 1);
  *lo = base;
  *hi = base + static_cast<uintptr_t>(last + 1) * es;
}

// grid: {frames, height, width} for SOLATTN_MODE_LOCAL3D, ignored otherwise.
int check(int mode, const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
          float tau, float keep_percent, int block_q, int block_k, int sink_range, int extra_tokens,
          const solattn_opts* opts, Strides st[4], const int* grid) {
  if (mode != SOLATTN_MODE_SOL && mode != SOLATTN_MODE_SLA && mode != SOLATTN_MODE_LOCAL3D)
    return fail(SOLATTN_EINVAL, "mode %d", mode);
  if (opts && opts->struct_size != (int)sizeof(solattn_opts))
    return fail(SOLATTN_EINVAL, "opts->struct_size %d != %d", opts->struct_size, (int)sizeof(solattn_opts));
  const int dtype = opts ? opts->dtype : SOLATTN_BF16;
  if (dtype != SOLATTN_BF16 && dtype != SOLATTN_FP32 && dtype != SOLATTN_BF16_FP8QK)
    return fail(SOLATTN_EINVAL, "dtype %d", dtype);
  if (!q || !k || !v || !out) return fail(SOLATTN_EINVAL, "null tensor pointer");
  if (B < 1 || H < 1 || N < 1 || d < 1) return fail(SOLATTN_EINVAL, "sizes B=%d H=%d N=%d d=%d", B, H, N, d);
  if (block_q < 1 || block_k < 1) return fail(SOLATTN_EINVAL, "block sizes %d %d", block_q, block_k);
  if (mode == SOLATTN_MODE_SOL && std::isnan(tau)) return fail(SOLATTN_EINVAL, "tau is NaN");
  if (mode == SOLATTN_MODE_SLA && !(keep_percent > 0.f && keep_percent <= 100.f))
    return fail(SOLATTN_EINVAL, "keep_percent %g outside (0, 100]", (double)keep_percent);
  if (mode == SOLATTN_MODE_LOCAL3D) {
    if (grid[0] < 1 || grid[1] < 1 || grid[2] < 1)
      return fail(SOLATTN_EINVAL, "grid %d x %d x %d", grid[0], grid[1], grid[2]);
    if ((int64_t)grid[0] * grid[1] * grid[2] != N)
      return fail(SOLATTN_EINVAL, "grid %d x %d x %d does not hold N=%d tokens", grid[0], grid[1], grid[2], N);
  }
  if (extra_tokens < 0 || extra_tokens > SOLATTN_MAX_EXTRA)
    return fail(SOLATTN_EINVAL, "extra_tokens %d outside [0, %d]", extra_tokens, SOLATTN_MAX_EXTRA);
  if (sink_range < 0 || sink_range > N) return fail(SOLATTN_EINVAL, "sink_range %d outside [0, N]", sink_range);
  const int d0 = opts ? opts->dense_row_begin : 0, d1 = opts ? opts->dense_row_end : 0;
  if (d0 < 0 || d1 < d0 || d1 > N) return fail(SOLATTN_EINVAL, "dense rows [%d, %d) outside [0, N]", d0, d1);
  const int r0 = opts ? opts->q_row_begin : 0, r1 = opts ? opts->q_row_end : 0;
  if (!(r0 == 0 && r1 == 0) && !(r0 >= 0 && r0 < r1 && r1 <= N))
    return fail(SOLATTN_EINVAL, "query-row window [%d, %d) not inside [0, N]", r0, r1);
  const unsigned flags = opts ? opts->flags : 0u;
  if (flags & ~(SOLATTN_FLAG_EXACT_EXTRA | SOLATTN_FLAG_CHECK_FINITE | SOLATTN_FLAG_KEEP_SELECTION))
    return fail(SOLATTN_EINVAL, "unknown flags 0x%x", flags);
  if ((flags & SOLATTN_FLAG_CHECK_FINITE) && !(opts && opts->stats))
    return fail(SOLATTN_EINVAL, "SOLATTN_FLAG_CHECK_FINITE needs opts->stats");
  if (opts && opts->stats && reinterpret_cast<uintptr_t>(opts->stats) % 8)
    return fail(SOLATTN_EINVAL, "stats not 8-byte aligned");

  const int64_t zero[3] = {0, 0, 0};
  st[0] = resolve(opts ? opts->q_stride : zero, H, N, d);
  st[1] = resolve(opts ? opts->k_stride : zero, H, N, d);
  st[2] = resolve(opts ? opts->v_stride : zero, H, N, d);
  st[3] = resolve(opts ? opts->o_stride : zero, H, N, d);
  for (int t = 0; t < 4; ++t)
    if (st[t].sb < 0 || st[t].sh < 0 || st[t].sn < 0) return fail(SOLATTN_EINVAL, "negative stride");
  const Strides& so = st[3];
  if (so.sn < d || (H > 1 && so.sh < (int64_t)N * so.sn) || (B > 1 && so.sb < (int64_t)H * so.sh))
    return fail(SOLATTN_EINVAL, "out strides make rows overlap");
  const size_t es = dtype == SOLATTN_FP32 ? 4 : 2;
  uintptr_t olo, ohi;
  extent(out, so, B, H, N, d, es, &olo, &ohi);
  const void* ins[3] = {q, k, v};
  for (int t = 0; t < 3; ++t) {
    uintptr_t lo, hi;
    extent(ins[t], st[t], B, H, N, d, es, &lo, &hi);
    if (lo < ohi && olo < hi) return fail(SOLATTN_EINVAL, "out overlaps %c", "qkv"[t]);
  }

  if (d != 64 && d != 128) return fail(SOLATTN_ENOTSUP, "d=%d (supported: 64 or 128)", d);
  if (block_k != 64) return fail(SOLATTN_ENOTSUP, "block_k=%d (supported: 64)", block_k);
  if (block_q != 64 && block_q != 128) return fail(SOLATTN_ENOTSUP, "block_q=%d (supported: 64, 128)", block_q);
  if (N % block_q || N % block_k) return fail(SOLATTN_ENOTSUP, "N=%d not a multiple of the block sizes", N);
  if (d0 % block_q || d1 % block_q) return fail(SOLATTN_ENOTSUP, "dense rows not block_q aligned");
  if (r0 % block_q || r1 % block_q) return fail(SOLATTN_ENOTSUP, "query-row window not block_q aligned");
  if ((int64_t)B * H > 65535) return fail(SOLATTN_ENOTSUP, "B*H=%lld too large", (long long)B * H);
  if (dtype != SOLATTN_FP32 && N / block_k > solattn::MAX_BLOCKS_BF16)
    return fail(SOLATTN_ENOTSUP, "bf16: more than %d key blocks", solattn::MAX_BLOCKS_BF16);
  if (mode == SOLATTN_MODE_LOCAL3D && N / block_k > solattn::MAX_BLOCKS_LOCAL3D)
    return fail(SOLATTN_ENOTSUP, "local 3-D: more than %d key blocks", solattn::MAX_BLOCKS_LOCAL3D);
  for (int t = 0; t < 4; ++t)   // the kernels address up to 64 rows with 32-bit byte offsets
    if (st[t].sn >= (int64_t(1) << 24)) return fail(SOLATTN_ENOTSUP, "row stride of %c too large", "qkvo"[t]);
  for (int t = 0; t < 4; ++t) {
    const void* p = t < 3 ? ins[t] : out;
    if ((reinterpret_cast<uintptr_t>(p) % 16) || ((st[t].sb * es) % 16) || ((st[t].sh * es) % 16) ||
        ((st[t].sn * es) % 16))
      return fail(SOLATTN_ENOTSUP, "tensor %c: rows not 16-byte aligned", "qkvo"[t]);
  }
  return SOLATTN_OK;
}

// q_rows: query rows of the computed window (N for the whole sequence).  The selection regions
// come first; their offsets depend on (B, H, Mq, M) only.
int layout(int mode, int dtype, int B, int H, int N, int d, int block_q, int block_k, int extra_tokens,
           int q_rows, solattn_ws_layout* L) {
  (void)mode;
  if (B < 1 || H < 1 || N < 1 || d < 1 || block_q < 1 || block_k < 1 || q_rows < 1 || q_rows > N ||
      extra_tokens < 0 || extra_tokens > SOLATTN_MAX_EXTRA ||
      (dtype != SOLATTN_BF16 && dtype != SOLATTN_FP32 && dtype != SOLATTN_BF16_FP8QK))
    return SOLATTN_EINVAL;
  std::memset(L, 0, sizeof *L);
  const size_t BH = (size_t)B * H;
  const int Mq = (q_rows + block_q - 1) / block_q, M = (N + block_k - 1) / block_k;
  const int Mpad = (M + 63) / 64 * 64;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L->kept_cnt = take(BH * Mq * 4);
  L->kept_bm = take(BH * Mq * (Mpad / 64) * 8);
  L->kept_idx = take(BH * Mq * M * 4);
  L->mult = take(BH * Mq * Mpad);
  L->extra_cnt = take(BH * Mq * 4);
  L->extra_idx = take(BH * Mq * SOLATTN_MAX_EXTRA * 4);
  L->extra_flag = take(BH * Mq * 4);
  L->scores = take(BH * Mq * Mpad * 4);
  L->qbar = take(BH * Mq * d * 4);
  L->kbar = take(BH * M * d * 4);
  L->vbar = take(BH * M * d * 4);
  if (dtype != SOLATTN_FP32 && block_q == 64) L->pair_plan = take(BH * solattn::PAIR_STRIDES * 8);
  int S, nl;
  solattn::extra_split(dtype == SOLATTN_FP32, B, H, Mq, &S, &nl);
  // without extra tokens the candidate buffer only holds the per-call counters' partial sums
  const size_t cand = extra_tokens > 0 ? BH * Mq * nl * solattn::EXTRA_CAP * 8 : solattn::stats_scratch_bytes();
  L->extra_buf = take(std::max(cand, solattn::stats_scratch_bytes()));
  L->extra_part = take(extra_tokens > 0 ? BH * Mq * nl * 4 : 4);
  L->extra_seed = take(BH * Mq * 4);
  if (dtype != SOLATTN_FP32) {
    L->kbar_bf = take(BH * Mpad * d * 2);
    L->vbar_t = take(BH * Mpad * d * 2);
    L->v_t = take(BH * (size_t)M * d * 64 * 2);
  }
  if (dtype == SOLATTN_BF16_FP8QK) {
    const size_t tb = (size_t)64 * d + 64;
    L->k8 = take(BH * (size_t)M * tb);
    L->kb8 = take(BH * (size_t)(Mpad / 64) * tb);
  }
  L->total = off;
  L->Mq = Mq;
  L->M = M;
  L->Mpad = Mpad;
  return SOLATTN_OK;
}

// Library-owned workspaces (grow-only), one per (device, stream), used when the caller passes
// none.  The lock is held from the buffer lookup until the call's last launch is enqueued, so a
// buffer is never freed while another thread is about to launch on it.
struct DefaultWs {
  int dev;
  hipStream_t stream;
  void* p;
  size_t size;
};
std::mutex g_ws_mu;
std::vector<DefaultWs> g_ws;

// Per-kernel timing.
constexpr int NK = SOLATTN_NKERNELS;
const char* kKernelNames[NK] = {"block_pool", "block_score", "block_select", "extra_select",
                                "sparse_flash_fwd"};
struct TimedCall {
  hipEvent_t ev[NK + 1];
  bool ran[NK];
};
std::mutex g_t_mu;
bool g_timing = false;
std::vector<TimedCall> g_calls;
std::vector<hipEvent_t> g_free_events;

hipEvent_t take_event() {
  if (!g_free_events.empty()) {
    hipEvent_t e = g_free_events.back();
    g_free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// no_events: record no timing events even while timing is enabled (the allocation-free entry
// point, which must not create HIP events).
int run(int mode, const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
        float tau, float keep_percent, int block_q, int block_k, int sink_range, int extra_tokens,
        const solattn_opts* opts, const int* grid = nullptr, bool no_events = false) {
  g_err.clear();
  Strides st[4];
  const int no_grid[3] = {0, 0, 0};
  if (!grid) grid = no_grid;
  int rc = check(mode, q, k, v, out, B, H, N, d, tau, keep_percent, block_q, block_k, sink_range,
                 extra_tokens, opts, st, grid);
  if (rc != SOLATTN_OK) return rc;
  const int dtype = opts ? opts->dtype : SOLATTN_BF16;
  int r0 = opts ? opts->q_row_begin : 0, r1 = opts ? opts->q_row_end : 0;
  if (r0 == 0 && r1 == 0) r1 = N;
  solattn_ws_layout L;
  layout(mode, dtype, B, H, N, d, block_q, block_k, extra_tokens, r1 - r0, &L);
  hipStream_t stream = opts ? static_cast<hipStream_t>(opts->stream) : nullptr;

  char* ws = nullptr;
  std::unique_lock<std::mutex> ws_lock(g_ws_mu, std::defer_lock);
  if (opts && opts->workspace) {
    if (opts->workspace_bytes < L.total)
      return fail(SOLATTN_EWORKSPACE, "workspace %zu bytes < %zu required", opts->workspace_bytes, L.total);
    if (reinterpret_cast<uintptr_t>(opts->workspace) % 256)
      return fail(SOLATTN_EINVAL, "workspace not 256-byte aligned");
    ws = static_cast<char*>(opts->workspace);
  } else {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SOLATTN_EHIP, "hipGetDevice");
    ws_lock.lock();
    DefaultWs* e = nullptr;
    for (DefaultWs& x : g_ws)
      if (x.dev == dev && x.stream == stream) e = &x;
    if (!e) {
      g_ws.push_back(DefaultWs{dev, stream, nullptr, 0});
      e = &g_ws.back();
    }
    if (e->size < L.total) {
      if (e->p) {
        // only calls on this stream use this buffer: let them finish before it is freed
        hipError_t er = hipStreamSynchronize(stream);
        if (er != hipSuccess) return fail(SOLATTN_EHIP, "hipStreamSynchronize: %s", hipGetErrorString(er));
        er = hipFree(e->p);
        e->p = nullptr;
        e->size = 0;
        if (er != hipSuccess) return fail(SOLATTN_EHIP, "hipFree: %s", hipGetErrorString(er));
      }
      void* p = nullptr;
      if (hipMalloc(&p, L.total) != hipSuccess) return fail(SOLATTN_EHIP, "hipMalloc(%zu) failed", L.total);
      e->p = p;
      e->size = L.total;
    }
    ws = static_cast<char*>(e->p);
  }

  Problem P;
  std::memset(&P, 0, sizeof P);
  P.B = B; P.H = H; P.N = N; P.d = d;
  P.bq = block_q; P.bk = block_k;
  P.Mq = L.Mq; P.M = L.M; P.Mpad = L.Mpad;
  P.mode = mode;
  P.dtype = dtype == SOLATTN_FP32 ? 1 : 0;      // the element type of the tensors
  P.fp8qk = dtype == SOLATTN_BF16_FP8QK ? 1 : 0;
  P.tau = tau;
  P.keep_all = (mode == SOLATTN_MODE_SOL && std::isinf(tau) && tau < 0) ? 1 : 0;
  if (mode == SOLATTN_MODE_SLA) {
    const double kk = std::ceil((double)keep_percent * (double)L.M / 100.0);
    P.k_sla = kk > L.M ? L.M : (int)kk;
  }
  P.sink_blocks = (sink_range + block_k - 1) / block_k;
  P.extra = extra_tokens;
  P.exact_extra = (opts && (opts->flags & SOLATTN_FLAG_EXACT_EXTRA)) ? 1 : 0;
  P.q0 = r0 / block_q;
  // the dense range, intersected with the window, in window-local query blocks
  const int d0 = opts ? opts->dense_row_begin : 0, d1 = opts ? opts->dense_row_end : 0;
  P.dense_q0 = std::max(d0, r0) / block_q - P.q0;
  P.dense_q1 = std::min(d1, r1) / block_q - P.q0;
  if (P.dense_q1 <= P.dense_q0) P.dense_q0 = P.dense_q1 = 0;
  P.frames = grid[0]; P.height = grid[1]; P.width = grid[2];
  P.scale = 1.0f / std::sqrt(static_cast<float>(d));
  P.q = Tensor{q, st[0].sb, st[0].sh, st[0].sn};
  P.k = Tensor{k, st[1].sb, st[1].sh, st[1].sn};
  P.v = Tensor{v, st[2].sb, st[2].sh, st[2].sn};
  P.o = Tensor{out, st[3].sb, st[3].sh, st[3].sn};
  P.qbar = reinterpret_cast<float*>(ws + L.qbar);
  P.kbar = reinterpret_cast<float*>(ws + L.kbar);
  P.vbar = reinterpret_cast<float*>(ws + L.vbar);
  P.scores = reinterpret_cast<float*>(ws + L.scores);
  P.kept_cnt = reinterpret_cast<int*>(ws + L.kept_cnt);
  P.kept_idx = reinterpret_cast<int*>(ws + L.kept_idx);
  P.kept_bm = reinterpret_cast<uint64_t*>(ws + L.kept_bm);
  P.mult = reinterpret_cast<uint8_t*>(ws + L.mult);
  P.keep_lists = (dtype == SOLATTN_FP32 || (opts && (opts->flags & SOLATTN_FLAG_KEEP_SELECTION))) ? 1 : 0;
  P.extra_cnt = reinterpret_cast<int*>(ws + L.extra_cnt);
  P.extra_idx = reinterpret_cast<int*>(ws + L.extra_idx);
  P.extra_buf = reinterpret_cast<uint2*>(ws + L.extra_buf);
  P.extra_part = reinterpret_cast<int*>(ws + L.extra_part);
  P.extra_flag = reinterpret_cast<int*>(ws + L.extra_flag);
  solattn::extra_split(dtype == SOLATTN_FP32, B, H, L.Mq, &P.extra_slices, &P.extra_lists);
  P.extra_seed = reinterpret_cast<uint32_t*>(ws + L.extra_seed);
  if (dtype != SOLATTN_FP32) {
    P.kbar_bf = reinterpret_cast<uint16_t*>(ws + L.kbar_bf);
    P.vbar_t = reinterpret_cast<uint16_t*>(ws + L.vbar_t);
    P.v_t = reinterpret_cast<uint16_t*>(ws + L.v_t);
  }
  if (P.fp8qk) {
    P.k8 = reinterpret_cast<uint8_t*>(ws + L.k8);
    P.kb8 = reinterpret_cast<uint8_t*>(ws + L.kb8);
  }
  P.pair_plan = L.pair_plan ? reinterpret_cast<long long*>(ws + L.pair_plan) : nullptr;

  if (opts && opts->stats && L.extra_part - L.extra_buf < solattn::stats_scratch_bytes())
    return fail(SOLATTN_ENOTSUP, "stats: candidate buffer smaller than the counters' scratch");

  std::unique_lock<std::mutex> tl(g_t_mu);
  const bool timing = g_timing && !no_events;
  TimedCall tc;
  std::memset(&tc, 0, sizeof tc);
  auto release = [&]() {
    for (int e = 0; e <= NK; ++e)
      if (tc.ev[e]) g_free_events.push_back(tc.ev[e]);
  };
  if (timing) {
    for (int e = 0; e <= NK; ++e) {
      tc.ev[e] = take_event();
      if (!tc.ev[e]) {
        release();
        return fail(SOLATTN_EHIP, "hipEventCreate");
      }
    }
  } else {
    tl.unlock();
  }
  bool mark_ok = true;
  auto mark = [&](int e) {
    if (timing && hipEventRecord(tc.ev[e], stream) != hipSuccess) mark_ok = false;
  };

  // The launch sequence; returns the failing kernel's name, or nullptr.
  const bool do_extra = extra_tokens > 0 && !P.keep_all;
  hipError_t err = hipSuccess;
  auto launch_all = [&]() -> const char* {
    mark(0);
    if ((err = solattn::launch_block_pool(P, stream)) != hipSuccess) return "block_pool";
    // the fp8 key tiles need the pooled keys; their time is counted with the pooling
    if (P.fp8qk && (err = solattn::launch_quantize_k(P, stream)) != hipSuccess) return "quantize_k";
    tc.ran[0] = true;
    mark(1);
    if (mode != SOLATTN_MODE_LOCAL3D) {
      if ((err = solattn::launch_block_score(P, stream)) != hipSuccess) return "block_score";
      tc.ran[1] = true;
    }
    mark(2);
    if ((err = solattn::launch_block_select(P, stream)) != hipSuccess) return "block_select";
    // the pairing of query blocks for the attention kernel; its time counts with the selection
    if ((err = solattn::launch_pair_plan(P, stream)) != hipSuccess) return "pair_plan";
    tc.ran[2] = true;
    mark(3);
    if (do_extra) {
      if ((err = solattn::launch_extra_select(P, stream)) != hipSuccess) return "extra_select";
      tc.ran[3] = true;
    }
    mark(4);
    if ((err = solattn::launch_sparse_flash(P, stream)) != hipSuccess) return "sparse_flash_fwd";
    tc.ran[4] = true;
    mark(5);
    if (opts && opts->stats) {
      const int fin = (opts->flags & SOLATTN_FLAG_CHECK_FINITE) ? 1 : 0;
      if ((err = solattn::launch_stats(P, reinterpret_cast<long long*>(opts->stats), fin, stream)) != hipSuccess)
        return "stats";
    }
    return nullptr;
  };
  if (const char* failed = launch_all()) {
    if (timing) release();
    return fail(SOLATTN_EHIP, "%s: %s", failed, hipGetErrorString(err));
  }
  if (timing) {
    if (!mark_ok) {
      release();
      return fail(SOLATTN_EHIP, "hipEventRecord failed (the kernels were enqueued)");
    }
    g_calls.push_back(tc);
  }
  return SOLATTN_OK;
}

}  // namespace

namespace solattn {

int set_error(int code, const char* detail) { return fail(code, "%s", detail); }

int run_sol_on_buffer(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                      float tau, int block_q, int block_k, int sink_range, int extra_tokens,
                      const solattn_opts* opts, void* ws, size_t ws_bytes) {
  solattn_opts o;
  if (opts) {
    o = *opts;
  } else {
    std::memset(&o, 0, sizeof o);
    o.struct_size = sizeof o;
  }
  const int dtype = o.dtype;
  int r0 = o.q_row_begin, r1 = o.q_row_end;
  if (r0 == 0 && r1 == 0) r1 = N;
  solattn_ws_layout L;
  if (layout(SOLATTN_MODE_SOL, dtype, B, H, N, d, block_q, block_k, extra_tokens, r1 - r0, &L) != SOLATTN_OK)
    return fail(SOLATTN_EINVAL, "invalid shape");
  if (L.total > ws_bytes)
    return fail(SOLATTN_EWORKSPACE,
                "sol_attn_fwd_noalloc: this call needs %zu bytes of workspace; the library's scratch holds %zu "
                "(use sol_attn_fwd with a workspace, or a query-row window)", L.total, ws_bytes);
  o.workspace = ws;
  o.workspace_bytes = ws_bytes;
  return run(SOLATTN_MODE_SOL, q, k, v, out, B, H, N, d, tau, 100.f, block_q, block_k, sink_range, extra_tokens,
             &o, nullptr, true);
}

}  // namespace solattn

extern "C" {

int sol_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d, float tau,
                 int block_q, int block_k, int sink_range, int extra_tokens, const solattn_opts* opts) {
  return run(SOLATTN_MODE_SOL, q, k, v, out, B, H, N, d, tau, 100.f, block_q, block_k, sink_range,
             extra_tokens, opts);
}

int sla_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d, int block_q,
                 int block_k, int sink_range, int extra_tokens, float keep_percent, const solattn_opts* opts) {
  return run(SOLATTN_MODE_SLA, q, k, v, out, B, H, N, d, 0.f, keep_percent, block_q, block_k, sink_range,
             extra_tokens, opts);
}

int local3d_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                     int frames, int height, int width, int block_q, int block_k, int sink_range,
                     int extra_tokens, const solattn_opts* opts) {
  const int grid[3] = {frames, height, width};
  return run(SOLATTN_MODE_LOCAL3D, q, k, v, out, B, H, N, d, 0.f, 100.f, block_q, block_k, sink_range,
             extra_tokens, opts, grid);
}

int solattn_check_args(int mode, const void* q, const void* k, const void* v, void* out, int B, int H, int N,
                       int d, float tau, float keep_percent, int block_q, int block_k, int sink_range,
                       int extra_tokens, const solattn_opts* opts) {
  g_err.clear();
  Strides st[4];
  if (mode == SOLATTN_MODE_LOCAL3D)
    return fail(SOLATTN_EINVAL, "mode %d: use local3d_check_args", mode);
  const int no_grid[3] = {0, 0, 0};
  return check(mode, q, k, v, out, B, H, N, d, tau, keep_percent, block_q, block_k, sink_range, extra_tokens,
               opts, st, no_grid);
}

int local3d_check_args(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                       int frames, int height, int width, int block_q, int block_k, int sink_range,
                       int extra_tokens, const solattn_opts* opts) {
  g_err.clear();
  Strides st[4];
  const int grid[3] = {frames, height, width};
  return check(SOLATTN_MODE_LOCAL3D, q, k, v, out, B, H, N, d, 0.f, 100.f, block_q, block_k, sink_range,
               extra_tokens, opts, st, grid);
}

int solattn_workspace_layout(int mode, int dtype, int B, int H, int N, int d, int block_q, int block_k,
                             int extra_tokens, int q_rows, solattn_ws_layout* out) {
  if (!out) return SOLATTN_EINVAL;
  return layout(mode, dtype, B, H, N, d, block_q, block_k, extra_tokens, q_rows, out);
}

size_t solattn_workspace_bytes_ex(int mode, int dtype, int B, int H, int N, int d, int block_q, int block_k,
                                  int extra_tokens, int q_rows) {
  solattn_ws_layout L;
  if (layout(mode, dtype, B, H, N, d, block_q, block_k, extra_tokens, q_rows, &L) != SOLATTN_OK) return 0;
  return L.total;
}

size_t solattn_workspace_bytes(int mode, int B, int H, int N, int d, int block_q, int block_k, int extra_tokens) {
  size_t most = 0;
  for (int dt : {SOLATTN_BF16, SOLATTN_FP32, SOLATTN_BF16_FP8QK}) {
    solattn_ws_layout L;
    if (layout(mode, dt, B, H, N, d, block_q, block_k, extra_tokens, N, &L) != SOLATTN_OK) return 0;
    most = std::max(most, L.total);
  }
  return most;
}

int solattn_selection_view(const solattn_opts* opts, int mode, int B, int H, int N, int block_q, int block_k,
                           solattn_selection* view) {
  g_err.clear();
  if (!opts || !view) return fail(SOLATTN_EINVAL, "selection_view: null opts or view");
  if (opts->struct_size != (int)sizeof(solattn_opts))
    return fail(SOLATTN_EINVAL, "opts->struct_size %d != %d", opts->struct_size, (int)sizeof(solattn_opts));
  if (!opts->workspace) return fail(SOLATTN_EINVAL, "selection_view: opts->workspace is NULL");
  if (mode != SOLATTN_MODE_SOL && mode != SOLATTN_MODE_SLA && mode != SOLATTN_MODE_LOCAL3D)
    return fail(SOLATTN_EINVAL, "mode %d", mode);
  int r0 = opts->q_row_begin, r1 = opts->q_row_end;
  if (r0 == 0 && r1 == 0) r1 = N;
  if (N < 1 || r0 < 0 || r1 <= r0 || r1 > N) return fail(SOLATTN_EINVAL, "selection_view: window [%d, %d)", r0, r1);
  // the selection regions do not depend on the dtype, d or extra_tokens
  solattn_ws_layout L;
  if (layout(mode, SOLATTN_BF16, B, H, N, 64, block_q, block_k, 0, r1 - r0, &L) != SOLATTN_OK)
    return fail(SOLATTN_EINVAL, "selection_view: invalid shape");
  char* ws = static_cast<char*>(opts->workspace);
  view->Mq = L.Mq;
  view->M = L.M;
  view->Mpad = L.Mpad;
  view->kept_cnt = reinterpret_cast<int32_t*>(ws + L.kept_cnt);
  view->kept_bm = reinterpret_cast<uint64_t*>(ws + L.kept_bm);
  view->kept_idx = reinterpret_cast<int32_t*>(ws + L.kept_idx);
  view->mult = reinterpret_cast<uint8_t*>(ws + L.mult);
  view->extra_cnt = reinterpret_cast<int32_t*>(ws + L.extra_cnt);
  view->extra_idx = reinterpret_cast<int32_t*>(ws + L.extra_idx);
  view->extra_flag = reinterpret_cast<int32_t*>(ws + L.extra_flag);
  view->scores = reinterpret_cast<float*>(ws + L.scores);
  return SOLATTN_OK;
}

int solattn_free_default_workspaces(void) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  int rc = SOLATTN_OK;
  for (DefaultWs& e : g_ws) {
    if (!e.p) continue;
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess || hipSetDevice(e.dev) != hipSuccess) {
      rc = SOLATTN_EHIP;
      continue;
    }
    if (hipDeviceSynchronize() != hipSuccess || hipFree(e.p) != hipSuccess) rc = SOLATTN_EHIP;
    hipSetDevice(cur);
  }
  g_ws.clear();
  if (rc != SOLATTN_OK) fail(rc, "free_default_workspaces: a HIP call failed");
  return rc;
}

const char* solattn_status_string(int status) {
  switch (status) {
    case SOLATTN_OK: return "ok";
    case SOLATTN_EINVAL: return "invalid argument";
    case SOLATTN_ENOTSUP: return "not supported by the library";
    case SOLATTN_EWORKSPACE: return "workspace too small";
    case SOLATTN_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* solattn_last_error_detail(void) { return g_err.c_str(); }

const char* solattn_last_error(void) { return g_err.c_str(); }

int solattn_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_t_mu);
  g_timing = enable != 0;
  return SOLATTN_OK;
}

int solattn_timing_read(double* ms, long long* launches, int n) {
  std::lock_guard<std::mutex> lk(g_t_mu);
  if (n < 0 || (n > 0 && (!ms || !launches))) return SOLATTN_EINVAL;
  for (int i = 0; i < n; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  int rc = SOLATTN_OK;
  for (TimedCall& c : g_calls) {
    if (hipEventSynchronize(c.ev[NK]) != hipSuccess) rc = SOLATTN_EHIP;
    for (int kx = 0; kx < NK && kx < n; ++kx) {
      if (!c.ran[kx]) continue;
      float t = 0.f;
      if (hipEventElapsedTime(&t, c.ev[kx], c.ev[kx + 1]) != hipSuccess) rc = SOLATTN_EHIP;
      ms[kx] += t;
      launches[kx] += 1;
    }
    for (int e = 0; e <= NK; ++e) g_free_events.push_back(c.ev[e]);
  }
  g_calls.clear();
  return rc;
}

const char* solattn_kernel_name(int index) {
  if (index < 0 || index >= NK) return "";
  return kKernelNames[index];
}

int solattn_pair_schedule(int Mq, int dense_q0, int dense_q1, int stride, int* qa, int* qb, int cap) {
  g_err.clear();
  if (Mq < 1 || dense_q0 < 0 || dense_q1 < dense_q0 || dense_q1 > Mq || stride < 1 ||
      stride > solattn::PAIR_STRIDES || cap < 0 || (cap > 0 && (!qa || !qb)))
    return fail(SOLATTN_EINVAL, "pair_schedule: invalid arguments");
  if (dense_q1 == dense_q0) dense_q0 = dense_q1 = 0;
  const int n = solattn::flash_units_per_head(2, Mq, dense_q1 - dense_q0);
  for (int j = 0; j < n && j < cap; ++j)
    solattn::flash_unit_blocks(2, Mq, dense_q0, dense_q1, stride, j, qa + j, qb + j);
  return n;
}

}  // extern "C"
