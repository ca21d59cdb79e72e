// GEMM core of libmoe: C[m][n] = sum_k A[m][k] * B[n][k] ("NT": both operands
// K-contiguous), fp32 accumulation, with pluggable operand sources and
// epilogues so that one kernel serves the router + down projection, the
// grouped expert FFNs (row gather from the receive pools, SwiGLU pairing,
// scatter into the return pools) and the shared experts + up-projection.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 tiles (gfx950), LDS double buffering
// with a padded row pitch (conflict-free 16-byte fragment reads).
// fp32 path: a plain per-element kernel (small layers only).
#pragma once

#include "moe_common.h"

namespace moe {

// ------------------------------------------------------------ A operands
// rows(g): rows of group g; row(g, m): pointer to element 0 of row m.

template <class T>
struct ARows {  // row m of group g at base + g*group_stride + m*lda
  const T* base;
  int64_t lda, group_stride;
  const int32_t* counts;  // device rows per group, or NULL: rows_const
  int rows_const;
  __device__ int rows(int g) const { return counts ? counts[g] : rows_const; }
  __device__ const T* row(int g, int m) const { return base + g * group_stride + (int64_t)m * lda; }
};

template <class T>
struct AGather {  // row m of group g = payload of receive-pool row row_src[g][m]
  const char* pools;
  int64_t src_stride, row_stride;
  int cap;
  const int32_t* row_src;
  int64_t rs_stride;
  const int32_t* counts;
  __device__ int rows(int g) const { return counts[g]; }
  __device__ const T* row(int g, int m) const {
    const int rs = row_src[g * rs_stride + m];
    const int s = rs / cap, sl = rs - s * cap;
    return (const T*)(pools + s * src_stride + (int64_t)sl * row_stride);
  }
};

// ------------------------------------------------------------ B operands
// ptr(g, n, k): address of B[n][k] for group g.  KSEG: the row pointer
// depends on k (re-evaluated every K tile); otherwise it is hoisted.

template <class T>
struct BRows {  // row n of group g at base + g*group_stride + n*ldb
  static constexpr bool KSEG = false;
  const T* base;
  int64_t ldb, group_stride;
  __device__ const T* ptr(int g, int n, int k) const {
    return base + g * group_stride + (int64_t)n * ldb + k;
  }
};

template <class T>
struct BTwo {  // rows [0, n_split) from b0, the rest from b1 (router | down projection)
  static constexpr bool KSEG = false;
  const T* b0;
  const T* b1;
  int n_split;
  int64_t ldb;
  __device__ const T* ptr(int, int n, int k) const {
    return n < n_split ? b0 + (int64_t)n * ldb + k : b1 + (int64_t)(n - n_split) * ldb + k;
  }
};

// SwiGLU pairing: output columns come in blocks of 64, the first 32 are gate
// rows of hidden units 32*b .. 32*b+31 and the next 32 the matching up rows.
// Hidden unit u belongs to expert u / hidden (stride expert_stride) whose
// weight holds `hidden` gate rows then `hidden` up rows.
template <class T>
struct BGateUp {
  static constexpr bool KSEG = false;
  const T* base;
  int64_t ldb, group_stride;
  int hidden;
  int64_t expert_stride;
  __device__ const T* ptr(int g, int n, int k) const {
    const int w = n & 63;
    const int u = (n >> 6) * 32 + (w & 31);
    const int j = u / hidden, h = u - j * hidden;
    return base + g * group_stride + j * expert_stride + (int64_t)((w >> 5) * hidden + h) * ldb + k;
  }
};

// K-concatenated operand: k in [0, k0) from b0 (row n at b0 + n*ld0), then
// consecutive segments of k1 from expert j of b1 (row n at b1 + j*stride1 + n*ld1).
template <class T>
struct BKSeg {
  static constexpr bool KSEG = true;
  const T* b0;
  int64_t ld0;
  int k0;
  const T* b1;
  int64_t ld1;
  int k1;
  int64_t stride1;
  __device__ const T* ptr(int, int n, int k) const {
    if (k < k0) return b0 + (int64_t)n * ld0 + k;
    const int kk = k - k0, j = kk / k1;
    return b1 + j * stride1 + (int64_t)n * ld1 + (kk - j * k1);
  }
};

// ------------------------------------------------------------ epilogues

template <class T>
struct ERouteDown {  // columns < E: fp32 logits (+bias); the rest: latent z
  float* logits;
  T* z;
  const float* bias;
  int E, L, bias_row_tokens;
  __device__ void store(int, int m, int n, float v) const {
    if (n < E) {
      float b = 0.f;
      if (bias) b = bias[(int64_t)(bias_row_tokens ? m / bias_row_tokens : 0) * E + n];
      logits[(int64_t)m * E + n] = v + b;
    } else {
      z[(int64_t)m * L + (n - E)] = Act<T>::store(v);
    }
  }
};

template <class T>
struct ESwiGLU {  // hidden unit u of row m: act(silu(gate) * up)
  T* out;
  int64_t ldo, group_stride;
  int col0;
  __device__ void store2(int g, int m, int u, float gate, float up) const {
    out[g * group_stride + (int64_t)m * ldo + col0 + u] = Act<T>::store(silu(gate) * up);
  }
};

template <class T>
struct EScatter {  // row m of group g -> return row of receive row row_src[g][m]
  char* ret;
  int64_t src_stride, row_bytes;
  int cap;
  const int32_t* row_src;
  int64_t rs_stride;
  __device__ void store(int g, int m, int n, float v) const {
    const int rs = row_src[g * rs_stride + m];
    const int s = rs / cap, sl = rs - s * cap;
    ((T*)(ret + s * src_stride + (int64_t)sl * row_bytes))[n] = Act<T>::store(v);
  }
};

template <class T>
struct EStore {
  T* out;
  int64_t ldo;
  __device__ void store(int, int m, int n, float v) const { out[(int64_t)m * ldo + n] = Act<T>::store(v); }
};

// ------------------------------------------------------------ bf16 MFMA kernel

template <int BM, int BN, int WM, int WN>
struct MfmaTile {
  static constexpr int NT = 64 * WM * WN;
  static constexpr int BK = 64;
  static constexpr int PITCH = BK + 8;  // elements; 144-byte rows
  static constexpr int LDS_BYTES = 2 * (BM + BN) * PITCH * 2;
};

// grid: (ceil(N/BN), ceil(max_rows/BM), groups); block: 64*WM*WN threads.
// K must be a multiple of 64.  GATEUP: N counts gate+up columns (blocks of
// 64) and the epilogue gets (gate, up) pairs; WN*64 must divide BN.
template <int BM, int BN, int WM, int WN, bool GATEUP, class A, class B, class E>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_bf16_mfma(A a, B b, E e, int N, int K) {
  using TL = MfmaTile<BM, BN, WM, WN>;
  constexpr int NT = TL::NT, BK = TL::BK, PITCH = TL::PITCH;
  constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 32, FN = WTN / 32;
  constexpr int CA = BM * BK / 8 / NT, CB = BN * BK / 8 / NT;
  static_assert(CA * NT * 8 == BM * BK && CB * NT * 8 == BN * BK, "tile/threads mismatch");
  static_assert(!GATEUP || (WTN % 64) == 0, "gate/up pairs need 64-column wave tiles");
  extern __shared__ __attribute__((aligned(16))) bf16_t sm[];

  const int g = blockIdx.z;
  const int M = a.rows(g);
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  if (m0 >= M) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const bf16_t* arow[CA];
  int a_sm[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = tid + i * NT, r = c >> 3, kc = (c & 7) * 8;
    arow[i] = a.row(g, min(m0 + r, M - 1)) + kc;
    a_sm[i] = r * PITCH + kc;
  }
  const bf16_t* brow[CB];
  int bn[CB], bkc[CB], b_sm[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = tid + i * NT, r = c >> 3, kc = (c & 7) * 8;
    bn[i] = min(n0 + r, N - 1);
    bkc[i] = kc;
    brow[i] = b.ptr(g, bn[i], kc);
    b_sm[i] = (BM + r) * PITCH + kc;
  }

  uint4 ra[CA], rb[CB];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CA; ++i) ra[i] = *(const uint4*)(arow[i] + k0);
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const bf16_t* p = B::KSEG ? b.ptr(g, bn[i], k0 + bkc[i]) : brow[i] + k0;
      rb[i] = *(const uint4*)p;
    }
  };
  auto sstore = [&](int buf) {
    bf16_t* s = sm + buf * (BM + BN) * PITCH;
#pragma unroll
    for (int i = 0; i < CA; ++i) *(uint4*)(s + a_sm[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < CB; ++i) *(uint4*)(s + b_sm[i]) = rb[i];
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int frag_row = lane & 31, frag_k = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const bf16_t* s = sm + buf * (BM + BN) * PITCH;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[FM], bfv[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *(const bf16x8*)(s + (wm * WTM + i * 32 + frag_row) * PITCH + ks * 16 + frag_k);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfv[j] = *(const bf16x8*)(s + (BM + wn * WTN + j * 32 + frag_row) * PITCH + ks * 16 + frag_k);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfv[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // 32x32 accumulator layout: lane l holds column l%32, rows 8*(v/4) + 4*(l/32) + v%4.
  const int col_l = lane & 31, row_l = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * WTM + i * 32 + (v >> 2) * 8 + row_l + (v & 3);
      if (m >= M) continue;
      if constexpr (GATEUP) {
#pragma unroll
        for (int j = 0; j < FN; j += 2) {
          const int n = n0 + wn * WTN + j * 32 + col_l;  // gate column
          if (n < N) e.store2(g, m, (n >> 6) * 32 + (n & 31), acc[i][j][v], acc[i][j + 1][v]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int n = n0 + wn * WTN + j * 32 + col_l;
          if (n < N) e.store(g, m, n, acc[i][j][v]);
        }
      }
    }
  }
}

// ------------------------------------------------------------ fp32 kernel
// One thread per output (or per hidden unit for GATEUP), k ascending.
// grid: (ceil(cols/16), ceil(max_rows/16), groups); block 16x16.

template <bool GATEUP, class A, class B, class E>
__global__ void __launch_bounds__(256) gemm_f32_simple(A a, B b, E e, int N, int K) {
  const int g = blockIdx.z;
  const int M = a.rows(g);
  const int m = blockIdx.y * 16 + threadIdx.y;
  const int c = blockIdx.x * 16 + threadIdx.x;
  if (m >= M) return;
  const float* ar = a.row(g, m);
  if constexpr (GATEUP) {
    if (c >= N / 2) return;
    const int ng = (c / 32) * 64 + (c % 32), nu = ng + 32;
    float sg = 0.f, su = 0.f;
    for (int k = 0; k < K; ++k) {
      sg = fmaf(ar[k], *b.ptr(g, ng, k), sg);
      su = fmaf(ar[k], *b.ptr(g, nu, k), su);
    }
    e.store2(g, m, c, sg, su);
  } else {
    if (c >= N) return;
    float s = 0.f;
    for (int k = 0; k < K; ++k) s = fmaf(ar[k], *b.ptr(g, c, k), s);
    e.store(g, m, c, s);
  }
}

}  // namespace moe
