// C ABI of libmoe: validation, workspace layout and kernel launches.
// The operations and their readings are documented in include/moe.h.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "moe.h"
#include "gemm.h"
#include "moe_common.h"
#include "moe_internal.h"

using namespace moe;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(MOE_EHIP, "%s: %s", where, hipGetErrorString(e));
}

#define HIP_TRY(expr, where)                    \
  do {                                          \
    hipError_t e_ = (expr);                     \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

// ---------------------------------------------------------------- kernel timing
// While enabled, every launch carries two HIP events that its own dispatch
// records as the kernel starts and ends (moe_timing_enable / moe_timing_read;
// see launch() in moe_internal.h).

struct TimingRec {
  const char* name;
  hipEvent_t start, stop;
};

struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<TimingRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

Timing& timing() {
  static Timing t;
  return t;
}

}  // namespace

namespace moe {
LaunchEvents& launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}
}  // namespace moe

namespace {

class KernelTimer {  // scope guard around one launch (whose dispatch records the events on its own stream)
 public:
  explicit KernelTimer(const char* name) {
    Timing& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    if (!t.on) return;
    rec_.name = name;
    rec_.start = t.get();
    rec_.stop = t.get();
    if (!rec_.start || !rec_.stop) {
      if (rec_.start) t.pool.push_back(rec_.start);
      if (rec_.stop) t.pool.push_back(rec_.stop);
      return;
    }
    launch_events() = LaunchEvents{rec_.start, rec_.stop};  // the next launch records them
    armed_ = true;
  }
  ~KernelTimer() {
    if (!armed_) return;
    LaunchEvents& ev = launch_events();
    const bool launched = ev.start == nullptr;  // a launch took the pair
    ev = LaunchEvents{};
    Timing& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    if (launched) {
      t.recs.push_back(rec_);
    } else {  // nothing was launched (an empty batch)
      t.pool.push_back(rec_.start);
      t.pool.push_back(rec_.stop);
    }
  }

 private:
  TimingRec rec_{};
  bool armed_ = false;
};

// Launch `expr` (a hipError_t expression) timed under `name`.
#define LAUNCH(name, expr, where)              \
  do {                                         \
    hipError_t e_;                             \
    {                                          \
      KernelTimer kt_(name);                   \
      e_ = (expr);                             \
    }                                          \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

struct Q {  // validated, derived dimensions
  int64_t T, D, L, E, k, R, X, W, WX, LW, WR, H, S, HS, esize, scap, rcap, prow, row_bytes, my_rank;
  bool bf16;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int derive(const moe_dims* d, Q* q) {
  if (!d) return fail(MOE_EINVAL, "dims is NULL");
  if (d->act_dtype != MOE_ACT_BF16 && d->act_dtype != MOE_ACT_F32)
    return fail(MOE_EDTYPE, "act_dtype %d is not MOE_ACT_BF16 (0) or MOE_ACT_F32 (1)", d->act_dtype);
  if (d->tokens < 0 || d->d_model <= 0 || d->latent <= 0 || d->n_experts <= 0 || d->top_k <= 0 ||
      d->n_ranks <= 0 || d->waves <= 0 || d->expert_hidden <= 0 || d->shared_experts < 0 ||
      d->shared_hidden <= 0)
    return fail(MOE_EINVAL, "dims must be positive (tokens and shared_experts may be 0)");
  if (d->n_experts % d->n_ranks) return fail(MOE_EINVAL, "n_experts %% n_ranks != 0");
  const int X = d->n_experts / d->n_ranks;
  if (X > MOE_MAX_LOCAL) return fail(MOE_EINVAL, "more than %d local experts", MOE_MAX_LOCAL);
  if (X % d->waves) return fail(MOE_EINVAL, "local experts (%d) not divisible by waves (%d)", X, d->waves);
  if (d->n_ranks > MOE_MAX_RANKS) return fail(MOE_EINVAL, "more than %d ranks", MOE_MAX_RANKS);
  if (d->top_k > 32 || d->top_k > d->n_experts) return fail(MOE_EINVAL, "top_k must be <= min(32, n_experts)");
  if (d->n_experts > 2048) return fail(MOE_EINVAL, "n_experts > 2048");
  if (d->my_rank < 0 || d->my_rank >= d->n_ranks) return fail(MOE_EINVAL, "my_rank out of range");
  if (d->send_num <= 0 || d->send_den <= 0 || d->recv_num <= 0 || d->recv_den <= 0)
    return fail(MOE_EINVAL, "capacity factors must be positive rationals");
  if (d->live_waves < 0 || d->live_waves > d->waves)
    return fail(MOE_EINVAL, "live_waves %d out of range [0, waves = %d]", d->live_waves, d->waves);
  if (d->wave_rows < 0) return fail(MOE_EINVAL, "wave_rows %d < 0", d->wave_rows);
  const bool bf16 = d->act_dtype == MOE_ACT_BF16;
  // the up-projection GEMM's K (latent plus the shared hidden units) picks its segment in float
  if ((int64_t)d->latent + (int64_t)d->shared_experts * d->shared_hidden >= (1ll << 24))
    return fail(MOE_EINVAL, "latent + shared_experts * shared_hidden must be below 2^24");
  if (bf16) {
    if (d->d_model % 64 || d->latent % 64 || d->expert_hidden % 64 || d->shared_hidden % 64)
      return fail(MOE_EINVAL, "bf16 layers need d_model, latent, expert_hidden, shared_hidden multiples of 64");
    if (d->n_experts % 4) return fail(MOE_EINVAL, "bf16 layers need n_experts to be a multiple of 4");
  } else if (d->latent % 8 || d->shared_hidden % 4) {
    // the combined [latent | shared hidden] rows are written with 16-byte stores
    return fail(MOE_EINVAL, "fp32 layers need latent a multiple of 8 and shared_hidden a multiple of 4");
  }
  q->T = d->tokens; q->D = d->d_model; q->L = d->latent; q->E = d->n_experts; q->k = d->top_k;
  q->R = d->n_ranks; q->X = X; q->W = d->waves; q->WX = X / d->waves; q->H = d->expert_hidden;
  q->LW = d->live_waves ? d->live_waves : d->waves;
  q->WR = d->wave_rows;
  q->S = d->shared_experts; q->HS = d->shared_hidden; q->my_rank = d->my_rank; q->bf16 = bf16;
  q->esize = bf16 ? 2 : 4;
  const int64_t assign = q->T * q->k;
  // capacities in exact 128-bit arithmetic: the factors are any positive
  // int32 rationals, so factor x load can exceed 64 bits before the range
  // check below rejects it
  const __int128 sd = (__int128)d->send_den * q->R, rd = (__int128)d->recv_den * q->E;
  const __int128 scap = ((__int128)d->send_num * assign + sd - 1) / sd;
  const __int128 rcap = ((__int128)d->recv_num * q->R * assign + rd - 1) / rd;
  if (assign > (1ll << 30) || scap * q->R > (1ll << 30) || rcap * q->WX > (1ll << 30) ||
      q->T * q->E > (1ll << 31) || q->T * q->D > (1ll << 40))
    return fail(MOE_EINVAL, "sizes exceed the 32-bit index range of the kernels");
  q->scap = (int64_t)scap;
  q->rcap = (int64_t)rcap;
  // widths and GEMM tile counts the kernels' 32-bit tile and column
  // arithmetic can hold (far beyond any layer's shape)
  if (q->D > (1 << 24) || q->L > (1 << 24) || q->H > (1 << 24) || q->HS > (1 << 24))
    return fail(MOE_EINVAL, "d_model, latent, expert_hidden and shared_hidden must be at most 2^24");
  auto tiles = [](int64_t groups, int64_t rows, int64_t cols) {
    return groups * ceil_div(rows, 256) * ceil_div(cols, 256);
  };
  if (tiles(1, q->T, q->E + q->L) > (1ll << 30) || tiles(1, q->T, 2 * q->S * q->HS) > (1ll << 30) ||
      tiles(q->WX, q->rcap, 2 * q->H) > (1ll << 30) || tiles(q->WX, q->rcap, q->L) > (1ll << 30) ||
      tiles(1, q->T, q->D) > (1ll << 30))
    return fail(MOE_EINVAL, "a GEMM of these dims has more output tiles than the kernels can count");
  q->row_bytes = q->L * q->esize;
  q->prow = ceil_div(q->row_bytes + 4, 128) * 128;
  return MOE_OK;
}

struct WsLayout {
  size_t ctr, s_cc, s_cb, s_lr, r_cc, r_cb, r_j, r_lr, r_rank, logits, h, cat, part, total;
  size_t h_wave, part_wave;
  int nch_s, nch_r;
};

WsLayout layout(const Q& q) {
  WsLayout w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  w.nch_s = (int)ceil_div(q.T * q.k, SCAN_CHUNK);
  w.nch_r = (int)ceil_div(q.R * q.scap, SCAN_CHUNK);
  w.ctr = take((Ctr::HEADER + 2 * q.R + 2 * q.X) * 4);
  w.s_cc = take((size_t)(q.R + 1) * w.nch_s * 4);
  w.s_cb = take((size_t)(q.R + 1) * w.nch_s * 4);
  w.s_lr = take((size_t)q.T * q.k * 4);
  w.r_cc = take((size_t)(q.X + 1) * w.nch_r * 4);
  w.r_cb = take((size_t)(q.X + 1) * w.nch_r * 4);
  w.r_j = take((size_t)q.R * q.scap * 4);
  w.r_lr = take((size_t)q.R * q.scap * 4);
  w.r_rank = take((size_t)q.R * q.scap * 4);
  w.logits = take((size_t)q.T * q.E * 4);
  // hidden rows of a wave: a recv_cap block per expert, or one ragged bank
  w.h_wave = (size_t)(q.WR > 0 ? q.WR : q.WX * q.rcap) * q.H * q.esize;
  w.h = take(w.h_wave * q.LW);  // one SwiGLU hidden block per live wave: those waves may overlap
  w.cat = take((size_t)q.T * (q.L + q.S * q.HS) * q.esize);
  w.part_wave = q.bf16 ? (size_t)PART_SLOTS * PART_FLOATS * sizeof(float) : 0;  // tail-split partial tiles
  w.part = take(w.part_wave * (q.LW + 1));  // one block per live wave, one for route / combine
  w.total = off;
  return w;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

#define NEED(p, name)                                                     \
  do {                                                                    \
    if (!(p)) return fail(MOE_EINVAL, "%s is NULL", name);                \
    if (!aligned16(p)) return fail(MOE_EALIGN, "%s is not 16-byte aligned", name); \
  } while (0)

// Index, weight and count arrays are read as 4-byte scalars.
#define NEED4(p, name)                                                    \
  do {                                                                    \
    if (!(p)) return fail(MOE_EINVAL, "%s is NULL", name);                \
    if ((uintptr_t)(p) & 3) return fail(MOE_EALIGN, "%s is not 4-byte aligned", name); \
  } while (0)

// A buffer of zero elements may be NULL.
#define NEED_IF(cond, p, name) \
  do {                         \
    if (cond) NEED(p, name);   \
  } while (0)
#define NEED4_IF(cond, p, name) \
  do {                          \
    if (cond) NEED4(p, name);   \
  } while (0)

template <class P>
P* at(void* ws, size_t off) { return (P*)((char*)ws + off); }

// ---------------------------------------------------------------- GEMM runners

// Compute units of the current device (cached per device).
int cu_count() {
  static std::atomic<int> cached[64];  // 0: not looked up yet (threads may race to fill it, with one value)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return PART_SLOTS;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (!n) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = PART_SLOTS;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// bf16 GEMM launch.  part: PART_SLOTS partial tiles for the tail split, or
// NULL (no split: launches that may run beside others on the same workspace).
// rows_fixed: every group has max_rows rows, so the split is decided here and
// the fixup kernel launched only when there is a tail to finish.
template <bool GATEUP, class A, class B, class E>
hipError_t gemm_bf16(const char* name, const char* fixup_name, A a, B b, E e, int N, int K, int64_t max_rows,
                     bool rows_fixed, int groups, float* part, hipStream_t st) {
  using Cfg = TileCfg<256, 256>;
  if (N <= 0 || max_rows <= 0 || groups <= 0) return hipSuccess;
  const int P = cu_count() < PART_SLOTS ? cu_count() : PART_SLOTS;
  const int64_t tiles_m = ceil_div(max_rows, Cfg::BM), tiles_n = ceil_div(N, Cfg::BN);
  const int64_t max_tiles = groups * tiles_m * tiles_n;
  const int nk = K / Cfg::BK;
  // no tile count gives a tail split worth taking at this K: no partials
  const int smax = nk / KSPLIT_MIN;
  bool split = part != nullptr && smax >= 2 && nk - nk / smax >= KSPLIT_GAIN;
  if (split && rows_fixed) {  // the device-side plan, for a tile count known here
    const int64_t r = max_tiles % P;
    const int64_t parts = r > 0 ? (P / r < nk / KSPLIT_MIN ? P / r : nk / KSPLIT_MIN) : 0;
    split = r > 0 && 2 * r <= P && parts >= 2 && nk - nk / parts >= KSPLIT_GAIN;
  }
  {
    KernelTimer kt(name);
    launch((gemm_bf16_mfma<Cfg, GATEUP, A, B, E>), dim3((unsigned)gemm_grid(max_tiles, P)), dim3(Cfg::NT), 0,
                       st, a, b, e, N, K, groups, (int)tiles_n, P, split ? part : nullptr);
    hipError_t r = hipGetLastError();
    if (r != hipSuccess) return r;
  }
  if (!split) return hipSuccess;
  KernelTimer kt(fixup_name);
  launch((gemm_bf16_fixup<Cfg, GATEUP, A, E>), dim3(2048u), dim3(64), 0, st, a, e,
                     N, K, groups, (int)tiles_n, P, (const float*)part);
  return hipGetLastError();
}

template <bool GATEUP, class A, class B, class E>
hipError_t gemm_f32(const char* name, A a, B b, E e, int N, int K, int64_t max_rows, int groups, hipStream_t st) {
  const int cols = GATEUP ? N / 2 : N;
  if (cols <= 0 || max_rows <= 0 || groups <= 0) return hipSuccess;
  KernelTimer kt(name);
  const dim3 grid((unsigned)ceil_div(cols, 16), (unsigned)ceil_div(max_rows, 16), (unsigned)groups);
  launch((gemm_f32_simple<GATEUP, A, B, E>), grid, dim3(16, 16), 0, st, a, b, e, N, K);
  return hipGetLastError();
}

// route GEMM: logits | z = x . [W_r ; W_d]^T
template <class T>
hipError_t route_gemm(const Q& q, const void* x, const void* wr, const void* wd, const float* bias, int brt,
                      float* logits, void* z, float* part, hipStream_t st) {
  ARows<T> a{(const T*)x, q.D, 0, nullptr, (int)q.T};
  BTwo<T> b{(const T*)wr, (const T*)wd, (int)q.E, q.D};
  ERouteDown<T> e{logits, (T*)z, bias, (int)q.E, (int)q.L, brt};
  if constexpr (sizeof(T) == 2)
    return gemm_bf16<false>("route_gemm", "route_fixup", a, b, e, (int)(q.E + q.L), (int)q.D, q.T, true, 1, part, st);
  else return gemm_f32<false>("route_gemm", a, b, e, (int)(q.E + q.L), (int)q.D, q.T, 1, st);
}

template <class T, class A>
hipError_t expert_gemms(const Q& q, A a1, int wave, const int32_t* row_src, const int32_t* wave_count,
                        const void* w13, const void* w2, void* ret, int64_t ret_src_stride, T* h, float* part,
                        hipStream_t st) {
  const int64_t x0 = (int64_t)wave * q.WX;
  BGateUp<T> b1{(const T*)w13 + x0 * 2 * q.H * q.L, q.L, 2 * q.H * q.L, (int)q.H, 0};
  ESwiGLU<T> e1{h, q.H, q.rcap * q.H, 0, wave_count, q.WR};
  ARows<T> a2{h, q.H, q.rcap * q.H, wave_count, 0, q.WR};
  BRows<T> b2{(const T*)w2 + x0 * q.L * q.H, q.H, q.L * q.H};
  EScatter<T> e2{(char*)ret, ret_src_stride, q.row_bytes, (int)q.scap, row_src, q.rcap};
  hipError_t r;
  if constexpr (sizeof(T) == 2) {
    r = gemm_bf16<true>("expert_gate_up", "gate_up_fixup", a1, b1, e1, (int)(2 * q.H), (int)q.L, q.rcap, false,
                        (int)q.WX, part, st);
    if (r != hipSuccess) return r;
    return gemm_bf16<false>("expert_down", "down_fixup", a2, b2, e2, (int)q.L, (int)q.H, q.rcap, false, (int)q.WX,
                            part, st);
  } else {
    r = gemm_f32<true>("expert_gate_up", a1, b1, e1, (int)(2 * q.H), (int)q.L, q.rcap, (int)q.WX, st);
    if (r != hipSuccess) return r;
    return gemm_f32<false>("expert_down", a2, b2, e2, (int)q.L, (int)q.H, q.rcap, (int)q.WX, st);
  }
}

template <class T>
hipError_t shared_gate(const Q& q, const void* x, const void* ws13, T* cat, hipStream_t st) {
  const int64_t ldc = q.L + q.S * q.HS;
  ARows<T> a1{(const T*)x, q.D, 0, nullptr, (int)q.T};
  BGateUp<T> b1{(const T*)ws13, q.D, 0, (int)q.HS, 2 * q.HS * q.D};
  ESwiGLU<T> e1{cat, ldc, 0, (int)q.L};
  if constexpr (sizeof(T) == 2)
    return gemm_bf16<true>("shared_gate_up", "", a1, b1, e1, (int)(2 * q.S * q.HS), (int)q.D, q.T, true, 1, nullptr,
                           st);  // may run beside the routed path: no shared partial area
  else
    return gemm_f32<true>("shared_gate_up", a1, b1, e1, (int)(2 * q.S * q.HS), (int)q.D, q.T, 1, st);
}

template <class T>
hipError_t up_and_shared_down(const Q& q, const void* ws2, const void* w_up, T* cat, void* out, float* part,
                              hipStream_t st) {
  const int64_t ldc = q.L + q.S * q.HS;
  ARows<T> a2{cat, ldc, 0, nullptr, (int)q.T};
  BKSeg<T> b2{(const T*)w_up, q.L, (int)q.L, (const T*)ws2, q.HS, (int)q.HS, q.D * q.HS, 1.0f / (float)q.HS};
  EStore<T> e2{(T*)out, q.D};
  if constexpr (sizeof(T) == 2)
    return gemm_bf16<false>("up_shared_down", "up_fixup", a2, b2, e2, (int)q.D, (int)ldc, q.T, true, 1, part, st);
  else
    return gemm_f32<false>("up_shared_down", a2, b2, e2, (int)q.D, (int)ldc, q.T, 1, st);
}

// ---------------------------------------------------------------- packing

int check_pack_args(const Q& q, const void* z, const int32_t* topk_idx, const void* send_pools,
                    int64_t dst_stride_bytes, const int32_t* slot_of, const int32_t* send_count) {
  NEED_IF(q.scap > 0, send_pools, "send_pools"); NEED4(send_count, "send_count");
  if (q.T > 0) { NEED(z, "z"); NEED4(topk_idx, "topk_idx"); NEED4(slot_of, "slot_of"); }
  if (dst_stride_bytes % 16 || dst_stride_bytes < q.scap * q.prow)
    return fail(MOE_EALIGN, "dst_stride_bytes must be a multiple of 16 and >= send_cap * pool_stride_bytes");
  return MOE_OK;
}

// Rank, scan and pack with the given scratch: ctr (counters), s_cc / s_cb
// ([R+1][nch] chunk counts and their scans) and s_lr ([T*k] ranks inside a
// chunk).  Every scratch word a kernel reads was written earlier in the same
// call, so the scratch needs no clearing.
int pack_pools_run(const Q& q, const void* z, const int32_t* topk_idx, void* send_pools, int64_t dst_stride_bytes,
                   int32_t* slot_of, int32_t* send_count, int32_t* ctr, int32_t* s_cc, int32_t* s_cb,
                   int32_t* s_lr, int nch_s, hipStream_t st) {
  LAUNCH("send_rank", launch_send_rank(topk_idx, (int)(q.T * q.k), (int)q.X, (int)q.E, (int)q.R, s_lr, s_cc, st),
         "moe_pack_pools rank");
  LAUNCH("send_scan", launch_send_scan(s_cc, nch_s, (int)q.R, (int)q.scap, s_cb, ctr, send_count, st),
         "moe_pack_pools scan");
  LAUNCH("pack", launch_pack(z, q.row_bytes, topk_idx, s_lr, s_cb, (int)q.T, (int)q.k, (int)q.X, (int)q.E,
                                 (int)q.R, (int)q.scap, send_pools, dst_stride_bytes, q.prow, slot_of, send_count,
                                 nullptr, ctr, st),
         "moe_pack_pools pack");
  return MOE_OK;
}

struct PackScratch {
  size_t ctr, s_cc, s_cb, s_lr, total;
  int nch_s;
};

// The pack path's part of the workspace layout, packed on its own.
PackScratch pack_scratch_layout(const Q& q) {
  PackScratch p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  p.nch_s = (int)ceil_div(q.T * q.k, SCAN_CHUNK);
  p.ctr = take((Ctr::HEADER + 2 * q.R + 2 * q.X) * 4);
  p.s_cc = take((size_t)(q.R + 1) * p.nch_s * 4);
  p.s_cb = take((size_t)(q.R + 1) * p.nch_s * 4);
  p.s_lr = take((size_t)q.T * q.k * 4);
  p.total = off;
  return p;
}

}  // namespace

// ------------------------------------------------------ allocation-free scratch
// Scratch of moe_pack_pools_noalloc, for callers that cannot allocate device
// memory.  Each GPU the library runs on holds its own copy of this array (at
// its own address) until the process ends.  Host code never passes the
// array's name to a kernel or a copy: in host code it is a stand-in, not a
// device address.  It uses the per-device address from hipGetSymbolAddress.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
char* g_scratch_addr[64] = {nullptr};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_base(char** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev), "moe_pack_pools_noalloc hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(MOE_EINVAL, "moe_pack_pools_noalloc: device %d out of range", dev);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "moe_pack_pools_noalloc hipGetSymbolAddress");
    if (!p) return fail(MOE_EHIP, "moe_pack_pools_noalloc: no device address for the scratch array");
    g_scratch_addr[dev] = (char*)p;
  }
  *out = g_scratch_addr[dev];
  return MOE_OK;
}

}  // namespace

// =================================================================== C ABI

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

int moe_timing_enable(int32_t on) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.on = on != 0;
  return MOE_OK;
}

int moe_timing_read(moe_kernel_time* out, int32_t max_entries, int32_t* n_entries) {
  if (!n_entries || (max_entries > 0 && !out) || max_entries < 0)
    return fail(MOE_EINVAL, "moe_timing_read: bad output arguments");
  Timing& t = timing();
  std::vector<TimingRec> recs;
  {
    std::lock_guard<std::mutex> g(t.mu);
    recs.swap(t.recs);
  }
  std::vector<moe_kernel_time> acc;
  hipError_t err = hipSuccess;
  for (const TimingRec& r : recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess && err == hipSuccess) err = e;
    size_t i = 0;
    while (i < acc.size() && strncmp(acc[i].name, r.name, sizeof(acc[i].name)) != 0) ++i;
    if (i == acc.size()) {
      moe_kernel_time k{};
      snprintf(k.name, sizeof(k.name), "%s", r.name);
      acc.push_back(k);
    }
    acc[i].launches += 1;
    acc[i].total_ms += ms;
  }
  {
    std::lock_guard<std::mutex> g(t.mu);
    for (const TimingRec& r : recs) {
      t.pool.push_back(r.start);
      t.pool.push_back(r.stop);
    }
  }
  if (err != hipSuccess) return hip_fail(err, "moe_timing_read");
  const int n = (int)acc.size() < max_entries ? (int)acc.size() : max_entries;
  for (int i = 0; i < n; ++i) out[i] = acc[i];
  *n_entries = (int32_t)acc.size();
  return MOE_OK;
}

int moe_capacity(const moe_dims* dims, int64_t* send_cap, int64_t* recv_cap, int64_t* pool_stride_bytes) {
  Q q;
  const int rc = derive(dims, &q);
  if (rc) return rc;
  if (send_cap) *send_cap = q.scap;
  if (recv_cap) *recv_cap = q.rcap;
  if (pool_stride_bytes) *pool_stride_bytes = q.prow;
  return MOE_OK;
}

int moe_workspace_size(const moe_dims* dims, size_t* bytes) {
  Q q;
  const int rc = derive(dims, &q);
  if (rc) return rc;
  if (!bytes) return fail(MOE_EINVAL, "bytes is NULL");
  *bytes = layout(q).total;
  return MOE_OK;
}

int moe_route(const moe_dims* dims, const void* x, const void* w_router, const void* w_down, const float* bias,
              int32_t bias_row_tokens, float* logits, void* z, int32_t* topk_idx, float* topk_w, void* ws,
              void* stream) {
  Q q;
  int rc = derive(dims, &q);
  if (rc) return rc;
  if (q.T == 0) return MOE_OK;
  NEED(x, "x"); NEED(w_router, "w_router"); NEED(w_down, "w_down"); NEED(z, "z");
  NEED4(topk_idx, "topk_idx"); NEED4(topk_w, "topk_w"); NEED(ws, "ws");
  if (logits && !aligned16(logits)) return fail(MOE_EALIGN, "logits is not 16-byte aligned");
  if (bias && !aligned16(bias)) return fail(MOE_EALIGN, "bias is not 16-byte aligned");
  if (bias_row_tokens < 0) return fail(MOE_EINVAL, "bias_row_tokens < 0");
  const WsLayout w = layout(q);
  hipStream_t st = (hipStream_t)stream;
  float* lg = logits ? logits : at<float>(ws, w.logits);
  HIP_TRY(q.bf16 ? route_gemm<bf16_t>(q, x, w_router, w_down, bias, bias_row_tokens, lg, z, at<float>(ws, w.part), st)
                 : route_gemm<float>(q, x, w_router, w_down, bias, bias_row_tokens, lg, z, nullptr, st),
          "moe_route gemm");
  LAUNCH("select_topk", launch_select_topk(lg, (int)q.T, (int)q.E, (int)q.k, topk_idx, topk_w, st), "moe_route select");
  return MOE_OK;
}

int moe_pack_pools(const moe_dims* dims, const void* z, const int32_t* topk_idx, void* send_pools,
                   int64_t dst_stride_bytes, int32_t* slot_of, int32_t* send_count, void* ws, void* stream) {
  Q q;
  int rc = derive(dims, &q);
  if (rc) return rc;
  NEED(ws, "ws");
  if ((rc = check_pack_args(q, z, topk_idx, send_pools, dst_stride_bytes, slot_of, send_count))) return rc;
  const WsLayout w = layout(q);
  return pack_pools_run(q, z, topk_idx, send_pools, dst_stride_bytes, slot_of, send_count, at<int32_t>(ws, w.ctr),
                        at<int32_t>(ws, w.s_cc), at<int32_t>(ws, w.s_cb), at<int32_t>(ws, w.s_lr), w.nch_s,
                        (hipStream_t)stream);
}

int moe_pack_pools_noalloc(const moe_dims* dims, const void* z, const int32_t* topk_idx, void* send_pools,
                           int64_t dst_stride_bytes, int32_t* slot_of, int32_t* send_count, void* stream) {
  Q q;
  int rc = derive(dims, &q);
  if (rc) return rc;
  const PackScratch p = pack_scratch_layout(q);
  if (p.total > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_EINVAL, "moe_pack_pools_noalloc: %lld tokens x %lld experts per token over %lld ranks need "
                "%zu bytes of scratch, more than the %zu the library holds",
                (long long)q.T, (long long)q.k, (long long)q.R, p.total, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  if ((rc = check_pack_args(q, z, topk_idx, send_pools, dst_stride_bytes, slot_of, send_count))) return rc;
  char* base = nullptr;
  if ((rc = scratch_base(&base))) return rc;
  return pack_pools_run(q, z, topk_idx, send_pools, dst_stride_bytes, slot_of, send_count, (int32_t*)(base + p.ctr),
                        (int32_t*)(base + p.s_cc), (int32_t*)(base + p.s_cb), (int32_t*)(base + p.s_lr), p.nch_s,
                        (hipStream_t)stream);
}

int moe_pack_ragged(const moe_dims* dims, const void* z, const int32_t* topk_idx, void* send_rows,
                    int32_t* send_off, int32_t* slot_of, int32_t* send_count, void* ws, void* stream) {
  Q q;
  int rc = derive(dims, &q);
  if (rc) return rc;
  NEED_IF(q.T > 0, send_rows, "send_rows"); NEED4(send_off, "send_off"); NEED4(send_count, "send_count");
  NEED(ws, "ws");
  if (q.T > 0) { NEED(z, "z"); NEED4(topk_idx, "topk_idx"); NEED4(slot_of, "slot_of"); }
  const WsLayout w = layout(q);
  hipStream_t st = (hipStream_t)stream;
  int32_t* ctr = at<int32_t>(ws, w.ctr);
  const int no_cap = INT32_MAX;
  LAUNCH("send_rank", launch_send_rank(topk_idx, (int)(q.T * q.k), (int)q.X, (int)q.E, (int)q.R, at<int32_t>(ws, w.s_lr),
                           at<int32_t>(ws, w.s_cc), st), "moe_pack_ragged rank");
  LAUNCH("send_scan", launch_send_scan(at<int32_t>(ws, w.s_cc), w.nch_s, (int)q.R, no_cap, at<int32_t>(ws, w.s_cb), ctr,
                           send_count, st), "moe_pack_ragged scan");
  LAUNCH("ragged_offsets", launch_ragged_offsets(send_count, (int)q.R, send_off, st), "moe_pack_ragged offsets");
  LAUNCH("pack", launch_pack(z, q.row_bytes, topk_idx, at<int32_t>(ws, w.s_lr), at<int32_t>(ws, w.s_cb), (int)q.T,
                      (int)q.k, (int)q.X, (int)q.E, (int)q.R, no_cap, send_rows, 0, q.prow, slot_of, send_count,
                      send_off, ctr, st), "moe_pack_ragged pack");
  return MOE_OK;
}

int moe_recv_rank(const moe_dims* dims, const void* recv_pools, int64_t src_stride_bytes, void* ws, void* stream) {
  Q q;
  int rc = derive(dims, &q);
  if (rc) return rc;
  NEED_IF(q.scap > 0, recv_pools, "recv_pools"); NEED(ws, "ws");
  if (src_stride_bytes % 16 || src_stride_bytes < q.scap * q.prow)
    return fail(MOE_EALIGN, "src_stride_bytes must be a multiple of 16 and >= send_cap * pool_stride_bytes");
  const WsLayout w = layout(q);
  hipStream_t st = (hipStream_t)stream;
  int32_t* ctr = at<int32_t>(ws, w.ctr);
  const int n_rows = (int)(q.R * q.scap);
  int32_t* arrivals = ctr + Ctr::HEADER + 2 * q.R;
  int32_t* kept = arrivals + q.X;
  LAUNCH("recv_rank", launch_recv_rank(recv_pools, src_stride_bytes, q.prow, q.row_bytes, (int)q.R, (int)q.scap, (int)q.X,
                           (int)q.my_rank, at<int32_t>(ws, w.r_j), at<int32_t>(ws, w.r_lr), at<int32_t>(ws, w.r_cc),
                           st), "moe_recv_rank rank");
  LAUNCH("recv_scan", launch_recv_scan(at<int32_t>(ws, w.r_cc), w.nch_r, (int)q.X, (int)q.rcap, at<int32_t>(ws, w.r_cb),
                           arrivals, kept, ctr, st), "moe_recv_rank scan");
  LAUNCH("recv_final", launch_recv_final(at<int32_t>(ws, w.r_j), at<int32_t>(ws, w.r_lr), at<int32_t>(ws, w.r_cb), n_rows,
                            (int)q.X, at<int32_t>(ws, w.r_rank), st), "moe_recv_rank final");
  return MOE_OK;
}

int moe_recv_waves(const moe_dims* dims, const void* recv_pools, int64_t src_stride_bytes, int32_t wave,
                   void* wave_buf, int32_t* row_src, int32_t* wave_count, void* ws, void* stream) {
  Q q;
  int rc = derive(dims, &q);
  if (rc) return rc;
  NEED4_IF(q.rcap > 0, row_src, "row_src"); NEED4(wave_count, "wave_count"); NEED(ws, "ws");
  if (wave_buf) {
    if (!aligned16(wave_buf)) return fail(MOE_EALIGN, "wave_buf is not 16-byte aligned");
    NEED_IF(q.scap > 0, recv_pools, "recv_pools (wave_buf is set)");
    if (src_stride_bytes % 16 || src_stride_bytes < q.scap * q.prow)
      return fail(MOE_EALIGN, "src_stride_bytes must be a multiple of 16 and >= send_cap * pool_stride_bytes");
  }
  if (wave < 0 || wave >= q.W) return fail(MOE_EINVAL, "wave %d out of range [0, %d)", wave, (int)q.W);
  const WsLayout w = layout(q);
  hipStream_t st = (hipStream_t)stream;
  int32_t* ctr = at<int32_t>(ws, w.ctr);
  const int j0 = wave * (int)q.WX, nj = (int)q.WX, n_rows = (int)(q.R * q.scap);
  const int32_t* kept = ctr + Ctr::HEADER + 2 * q.R + q.X;
  LAUNCH("recv_place", launch_recv_place(at<int32_t>(ws, w.r_j), at<int32_t>(ws, w.r_rank), kept, n_rows, (int)q.rcap, j0,
                            nj, q.WR, wave_count, row_src, ctr, st), "moe_recv_waves place");
  if (wave_buf)
    LAUNCH("wave_gather", launch_wave_gather(recv_pools, src_stride_bytes, q.prow, (int)q.scap, q.row_bytes, row_src, wave_count,
                               nj, (int)q.rcap, wave_buf, st), "moe_recv_waves gather");
  return MOE_OK;
}

int moe_expert_gemm(const moe_dims* dims, int32_t wave, const void* wave_buf, const void* recv_pools,
                    int64_t src_stride_bytes, const int32_t* row_src, const int32_t* wave_count, const void* w13,
                    const void* w2, void* ret_pools, int64_t ret_src_stride_bytes, void* ws, void* stream) {
  Q q;
  int rc = derive(dims, &q);
  if (rc) return rc;
  NEED4_IF(q.rcap > 0, row_src, "row_src"); NEED4(wave_count, "wave_count"); NEED(w13, "w13"); NEED(w2, "w2");
  NEED_IF(q.scap > 0, ret_pools, "ret_pools"); NEED(ws, "ws");
  if (wave < 0 || wave >= q.W) return fail(MOE_EINVAL, "wave %d out of range [0, %d)", wave, (int)q.W);
  if (ret_src_stride_bytes % 16 || ret_src_stride_bytes < q.scap * q.row_bytes)
    return fail(MOE_EALIGN, "ret_src_stride_bytes must be a multiple of 16 and >= send_cap * L * sizeof(act)");
  if (wave_buf) {
    if (!aligned16(wave_buf)) return fail(MOE_EALIGN, "wave_buf is not 16-byte aligned");
  } else {
    NEED_IF(q.scap > 0, recv_pools, "recv_pools (wave_buf is NULL)");
    if (src_stride_bytes % 16 || src_stride_bytes < q.scap * q.prow)
      return fail(MOE_EALIGN, "src_stride_bytes must be a multiple of 16 and >= send_cap * pool_stride_bytes");
  }
  const WsLayout w = layout(q);
  hipStream_t st = (hipStream_t)stream;
  hipError_t r;
  // the scratch block of the wave (SwiGLU hidden rows, tail-split partials):
  // waves in different blocks may overlap
  const int64_t blk = wave % q.LW;
  float* part = at<float>(ws, w.part + (size_t)(blk + 1) * w.part_wave);
  if (q.bf16) {
    bf16_t* h = at<bf16_t>(ws, w.h + (size_t)blk * w.h_wave);
    if (wave_buf) {
      ARows<bf16_t> a{(const bf16_t*)wave_buf, q.L, q.rcap * q.L, wave_count, 0};
      r = expert_gemms<bf16_t>(q, a, wave, row_src, wave_count, w13, w2, ret_pools, ret_src_stride_bytes, h, part, st);
    } else {
      AGather<bf16_t> a{(const char*)recv_pools, src_stride_bytes, q.prow, (int)q.scap, row_src, q.rcap, wave_count};
      r = expert_gemms<bf16_t>(q, a, wave, row_src, wave_count, w13, w2, ret_pools, ret_src_stride_bytes, h, part, st);
    }
  } else {
    float* h = at<float>(ws, w.h + (size_t)blk * w.h_wave);
    if (wave_buf) {
      ARows<float> a{(const float*)wave_buf, q.L, q.rcap * q.L, wave_count, 0};
      r = expert_gemms<float>(q, a, wave, row_src, wave_count, w13, w2, ret_pools, ret_src_stride_bytes, h, part, st);
    } else {
      AGather<float> a{(const char*)recv_pools, src_stride_bytes, q.prow, (int)q.scap, row_src, q.rcap, wave_count};
      r = expert_gemms<float>(q, a, wave, row_src, wave_count, w13, w2, ret_pools, ret_src_stride_bytes, h, part, st);
    }
  }
  HIP_TRY(r, "moe_expert_gemm gemm");
  LAUNCH("zero_dropped", launch_zero_dropped(at<int32_t>(ws, w.r_j), at<int32_t>(ws, w.r_rank), (int)(q.R * q.scap), (int)q.scap,
                              (int)q.rcap, wave * (int)q.WX, (int)q.WX, ret_pools, ret_src_stride_bytes, q.row_bytes,
                              st), "moe_expert_gemm zero rows");
  return MOE_OK;
}

int moe_shared_experts(const moe_dims* dims, const void* x, const void* ws13, void* ws, void* stream) {
  Q q;
  int rc = derive(dims, &q);
  if (rc) return rc;
  if (q.T == 0 || q.S == 0) return MOE_OK;
  NEED(x, "x"); NEED(ws13, "ws13"); NEED(ws, "ws");
  const WsLayout w = layout(q);
  hipStream_t st = (hipStream_t)stream;
  void* cat = at<char>(ws, w.cat);
  HIP_TRY(q.bf16 ? shared_gate<bf16_t>(q, x, ws13, (bf16_t*)cat, st) : shared_gate<float>(q, x, ws13, (float*)cat, st),
          "moe_shared_experts gemm");
  return MOE_OK;
}

int moe_combine(const moe_dims* dims, const void* ret_pools, int64_t ret_dst_stride_bytes, const int32_t* slot_of,
                const float* topk_w, const void* w_up, const void* ws2, void* out, void* ws, void* stream) {
  Q q;
  int rc = derive(dims, &q);
  if (rc) return rc;
  if (q.T == 0) return MOE_OK;
  NEED(ret_pools, "ret_pools"); NEED(w_up, "w_up"); NEED(out, "out"); NEED(ws, "ws");
  NEED4(slot_of, "slot_of"); NEED4(topk_w, "topk_w");
  if (q.S > 0) NEED(ws2, "ws2");
  if (ret_dst_stride_bytes % 16 || ret_dst_stride_bytes < q.scap * q.row_bytes)
    return fail(MOE_EALIGN, "ret_dst_stride_bytes must be a multiple of 16 and >= send_cap * L * sizeof(act)");
  const WsLayout w = layout(q);
  hipStream_t st = (hipStream_t)stream;
  void* cat = at<char>(ws, w.cat);
  const int64_t ldc = q.L + q.S * q.HS;
  LAUNCH("combine", launch_combine(q.bf16 ? 0 : 1, ret_pools, ret_dst_stride_bytes, q.row_bytes, (int)q.scap,
                                       (int)q.R, slot_of, topk_w, (int)q.T, (int)q.k, (int)q.L, cat, ldc,
                                       at<int32_t>(ws, w.ctr), st),
         "moe_combine combine");
  HIP_TRY(q.bf16 ? up_and_shared_down<bf16_t>(q, ws2, w_up, (bf16_t*)cat, out, at<float>(ws, w.part), st)
                 : up_and_shared_down<float>(q, ws2, w_up, (float*)cat, out, nullptr, st),
          "moe_combine gemm");
  return MOE_OK;
}

int moe_drop_stats(const moe_dims* dims, const void* ws, moe_drop_report* rep, void* stream) {
  Q q;
  int rc = derive(dims, &q);
  if (rc) return rc;
  NEED(ws, "ws");
  if (!rep) return fail(MOE_EINVAL, "report is NULL");
  const WsLayout w = layout(q);
  const size_t n = Ctr::HEADER + 2 * q.R + 2 * q.X;
  std::string buf(n * 4, '\0');
  int32_t* c = (int32_t*)&buf[0];
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipMemcpyAsync(c, (const char*)ws + w.ctr, n * 4, hipMemcpyDeviceToHost, st), "moe_drop_stats copy");
  HIP_TRY(hipStreamSynchronize(st), "moe_drop_stats sync");
  *rep = moe_drop_report{};
  rep->n_ranks = (int32_t)q.R;
  rep->local_experts = (int32_t)q.X;
  rep->send_assignments = q.T * q.k;
  int64_t kept = 0, dropped = c[Ctr::SEND_INVALID];
  for (int d = 0; d < q.R; ++d) {
    rep->send_demand[d] = c[Ctr::HEADER + d];
    rep->send_count[d] = c[Ctr::HEADER + q.R + d];
    kept += rep->send_count[d];
    dropped += rep->send_demand[d] - rep->send_count[d];
  }
  rep->send_kept = kept;
  rep->send_dropped = dropped;
  int64_t arr = 0, kp = 0;
  for (int j = 0; j < q.X; ++j) {
    rep->expert_arrivals[j] = c[Ctr::HEADER + 2 * q.R + j];
    rep->expert_kept[j] = c[Ctr::HEADER + 2 * q.R + q.X + j];
    arr += rep->expert_arrivals[j];
    kp += rep->expert_kept[j];
  }
  rep->recv_arrivals = arr;
  rep->recv_kept = kp;
  rep->recv_dropped = arr - kp;
  rep->recv_bad_ids = c[Ctr::RECV_BAD];
  if (rep->recv_bad_ids) return fail(MOE_ECAP, "%lld received rows carry an expert id of another rank",
                                     (long long)rep->recv_bad_ids);
  if (q.WR > 0 && c[Ctr::WAVE_OVER])
    return fail(MOE_ECAP, "the kept rows of a wave exceed its hidden-row bank (wave_rows = %lld)", (long long)q.WR);
#ifdef MOE_DEBUG
  if (c[Ctr::DBG_SEND]) return fail(MOE_ECAP, "debug check: a send rank below zero in the pack");
  if (c[Ctr::DBG_COMBINE])
    return fail(MOE_ECAP, "debug check: a slot_of entry outside [-1, n_ranks * send_cap) reached the combine "
                "(the assignment was left out)");
  if (c[Ctr::DBG_RECV]) return fail(MOE_ECAP, "debug check: a kept receive row ranked at or past its expert's count");
#endif
  return MOE_OK;
}

}  // extern "C"
