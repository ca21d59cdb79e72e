// GEMM core of libmoe: C[m][n] = sum_k A[m][k] * B[n][k] ("NT": both operands
// K-contiguous), fp32 accumulation, with pluggable operand sources and
// epilogues so that one kernel serves the router + down projection, the
// grouped expert FFNs (row gather from the receive pools, SwiGLU pairing,
// scatter into the return pools) and the shared experts + up-projection.
//
// bf16 path (gfx950): one 256-thread workgroup (4 waves, 2 x 2) per BM x BN
// output tile; each wave owns a (BM/2) x (BN/2) sub-tile built from
// v_mfma_f32_32x32x16_bf16.  K advances in steps of 64: the next step's
// operands go straight from HBM into the second LDS buffer (direct 16-byte
// global->LDS loads, each group of 8 lanes reading one full 128-byte row
// segment) while the current step's MFMAs run.  LDS rows are 128 bytes
// with the 16-byte chunk index XOR-swizzled per row, so the fragment reads
// of any 8 (or 16) consecutive lanes touch every LDS bank once.
// The MFMA is issued with the B fragment as its first operand, so every lane
// ends up holding one output row m and runs of 4 consecutive columns n: the
// epilogue stores 8-byte pieces and resolves a row's destination once.
// Workgroup ids are remapped so that each XCD (blocks are dealt round-robin
// to the 8 XCDs) works on a contiguous, M-grouped range of tiles and reuses
// operand rows from its own L2.
//
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
// depends on k (re-evaluated every K step, which never straddles a segment);
// otherwise it is computed once.

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
// Scalar interface (fp32 kernel): store(g, m, n, v) / store2(g, m, u, gate, up).
// Vector interface (MFMA kernel): row(g, m) -> per-row context, then
// store4(ctx, n, v[4]) for columns n..n+3 (n % 4 == 0, clipped at N), or
// store4_pair(ctx, u, gate[4], up[4]) for hidden units u..u+3.

__device__ __forceinline__ uint2 pack_bf16x4(const float* v) {
  return make_uint2((uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                    (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16));
}

// 4 consecutive activations at p (8-byte aligned for bf16 when full).
template <class T>
__device__ __forceinline__ void put4(T* p, const float* v, int valid) {
  if constexpr (sizeof(T) == 2) {
    if (valid >= 4) {
      *(uint2*)p = pack_bf16x4(v);
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)  // fixed trip count: v stays in registers
    if (i < valid) p[i] = Act<T>::store(v[i]);
}

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
  // Vector interface: needs E % 4 == 0, so a group of 4 columns is either
  // all logits or all latent.
  struct Row {
    float* lg;
    T* zr;
    const float* b;
  };
  __device__ Row row(int, int m) const {
    return {logits + (int64_t)m * E, z + (int64_t)m * L,
            bias ? bias + (int64_t)(bias_row_tokens ? m / bias_row_tokens : 0) * E : nullptr};
  }
  __device__ void store4(const Row& r, int n, int N, const float* v) const {
    if (n < E) {
      float b[4] = {0.f, 0.f, 0.f, 0.f};
      if (r.b) *(float4*)b = *(const float4*)(r.b + n);
      *(float4*)(r.lg + n) = make_float4(v[0] + b[0], v[1] + b[1], v[2] + b[2], v[3] + b[3]);
    } else {
      put4(r.zr + (n - E), v, N - n);
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
  struct Row { T* p; };
  __device__ Row row(int g, int m) const { return {out + g * group_stride + (int64_t)m * ldo + col0}; }
  __device__ void store4_pair(const Row& r, int u, const float* gate, const float* up) const {
    float h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = silu(gate[i]) * up[i];
    put4(r.p + u, h, 4);
  }
};

template <class T>
struct EScatter {  // row m of group g -> return row of receive row row_src[g][m]
  char* ret;
  int64_t src_stride, row_bytes;
  int cap;
  const int32_t* row_src;
  int64_t rs_stride;
  __device__ T* dest(int g, int m) const {
    const int rs = row_src[g * rs_stride + m];
    const int s = rs / cap, sl = rs - s * cap;
    return (T*)(ret + s * src_stride + (int64_t)sl * row_bytes);
  }
  __device__ void store(int g, int m, int n, float v) const { dest(g, m)[n] = Act<T>::store(v); }
  struct Row { T* p; };
  __device__ Row row(int g, int m) const { return {dest(g, m)}; }
  __device__ void store4(const Row& r, int n, int N, const float* v) const { put4(r.p + n, v, N - n); }
};

template <class T>
struct EStore {
  T* out;
  int64_t ldo;
  __device__ void store(int, int m, int n, float v) const { out[(int64_t)m * ldo + n] = Act<T>::store(v); }
  struct Row { T* p; };
  __device__ Row row(int, int m) const { return {out + (int64_t)m * ldo}; }
  __device__ void store4(const Row& r, int n, int N, const float* v) const { put4(r.p + n, v, N - n); }
};

// ------------------------------------------------------------ bf16 MFMA kernel

template <int BM_, int BN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int NT = 256;                          // 4 waves, 2 x 2
  static constexpr int WTM = BM / 2, WTN = BN / 2;        // wave sub-tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;      // 32x32 fragments per wave
  static constexpr int LA = BM / 32, LB = BN / 32;        // 16-byte loads per lane per K step
  static constexpr int STAGE = (BM + BN) * 128;           // bytes of one LDS buffer
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile sides are multiples of 64");
};

// Logical tile of workgroup `bid`: XCD-contiguous ranges, M-grouped order
// inside a group.  Returns false past the end.
__device__ __forceinline__ void tile_of(int bid, int nb, int tiles_m, int tiles_n, int& g, int& tm, int& tn) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  const int logical = xcd * per + min(xcd, rem) + idx;
  const int tpg = tiles_m * tiles_n;
  g = logical / tpg;
  const int r = logical - g * tpg;
  constexpr int GROUP_M = 8;
  const int width = GROUP_M * tiles_n;
  const int gid = r / width, first_m = gid * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int rr = r - gid * width;
  tm = first_m + rr % gsz;
  tn = rr / gsz;
}

// 16-byte LDS read at byte address `addr`, issued as inline assembly: the
// result must be awaited with lgkm_wait before use.
__device__ __forceinline__ void lds_read16(bf16x8& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
}

// Wait until at most N LDS reads are outstanding; the fragments pass through
// the statement so that their consumers stay behind it.
template <int N, int FM, int FN>
__device__ __forceinline__ void lgkm_wait(bf16x8 (&fa)[FM], bf16x8 (&fb)[FN]) {
  static_assert(FM == 4 && FN == 4, "fragment counts of the 256 x 256 tile");
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(fa[0]), "+v"(fa[1]), "+v"(fa[2]), "+v"(fa[3]), "+v"(fb[0]), "+v"(fb[1]), "+v"(fb[2]),
                 "+v"(fb[3])
               : "i"(N)
               : "memory");
}

// 16-byte chunk swizzle of a 128-byte LDS row.  Rows r and r' with the same
// swizzle never share a 16-lane (64-bank) or an 8-lane (32-bank) read group:
// f(r) = (r >> 1) ^ 4 (r & 1) is a permutation of 0..7 over any 8 consecutive
// rows and over any 8 rows of one parity among 16 consecutive rows.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ ((row & 1) << 2)) & 7; }

// grid: (groups * tiles_m * tiles_n); block: 256.  K must be a multiple of 64.
// GATEUP: N counts gate+up columns (blocks of 64) and the epilogue gets
// (gate, up) pairs.
//
// One K step (64) of the main loop: wait for this step's tiles to land in LDS
// and pass the barrier; issue every fragment read of the step; then issue the
// direct HBM->LDS loads of the next step into the other buffer (nobody reads
// that buffer any more: all its fragment reads were consumed before the
// barrier); then run the step's MFMAs while those loads are in flight.
// Issuing the loads after the reads keeps them off the reads' dependence
// path, and no staging registers are needed.
template <class Cfg, bool GATEUP, class A, class B, class E>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_bf16_mfma(A a, B b, E e, int N, int K, int tiles_m, int tiles_n) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, WTM = Cfg::WTM, WTN = Cfg::WTN;
  constexpr int FM = Cfg::FM, FN = Cfg::FN, LA = Cfg::LA, LB = Cfg::LB, STAGE = Cfg::STAGE;
  constexpr int KS = BK / 16;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  int g, tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, g, tm, tn);
  const int M = a.rows(g);
  const int m0 = tm * BM, n0 = tn * BN;
  if (m0 >= M) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Loader: load slot i of a wave fills the 1 KB LDS block i*4 + wave, i.e.
  // rows r = (i*4 + wave)*8 + lane/8, lane landing at block + 16*lane.  That
  // LDS position holds swizzled chunk lane%8 of row r, so the lane fetches
  // global chunk (lane%8) ^ swz(r); all rows of a lane are 32 apart and share
  // the swizzle.
  const int lrow = lane >> 3, lcol = lane & 7;
  const int r0 = wave * 8 + lrow;
  const int gcol = (lcol ^ swz(r0)) * 8;
  const bf16_t* pa[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) pa[i] = a.row(g, min(m0 + r0 + 32 * i, M - 1)) + gcol;
  const bf16_t* pb[LB];
  int nb_row[LB];
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    nb_row[i] = min(n0 + r0 + 32 * i, N - 1);
    pb[i] = b.ptr(g, nb_row[i], gcol);
  }
  auto dma = [&](int st, int k0) {
    char* s = smem + st * STAGE + wave * 1024;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(pa[i] + k0), (__attribute__((address_space(3))) void*)(s + i * 4096),
                                       16, 0, 0);
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const bf16_t* p = B::KSEG ? b.ptr(g, nb_row[i], k0 + gcol) : pb[i] + k0;
      __builtin_amdgcn_global_load_lds((const void*)p,
                                       (__attribute__((address_space(3))) void*)(s + BM * 128 + i * 4096), 16, 0, 0);
    }
  };

  // Fragment reads: lane reads row (base + lane%32), 16-byte chunk ks*2 + lane/32.
  // Fragment rows are 32 apart, so one swizzle serves them all.
  const int frow = lane & 31, fhalf = lane >> 5;
  const int fswz = swz(frow);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  const uint32_t fa_base = lds0 + (wm * WTM + frow) * 128, fb_base = lds0 + BM * 128 + (wn * WTN + frow) * 128;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // The fragment reads are issued as inline ds_read_b128 so that the
  // compiler, which cannot tell the two LDS buffers apart, does not make
  // them wait for the in-flight HBM->LDS loads of the other buffer; their
  // completion is awaited explicitly (lgkm_wait ties the fragments, so no
  // MFMA can be scheduled before the wait that covers its operands).
  bf16x8 fa[KS][FM], fb[KS][FN];
  auto read_step = [&](uint32_t st_off, int ks) {
    const uint32_t ch = (uint32_t)(((ks * 2 + fhalf) ^ fswz) << 4) + st_off;
#pragma unroll
    for (int i = 0; i < FM; ++i) lds_read16(fa[ks][i], fa_base + ch + i * 4096);
#pragma unroll
    for (int j = 0; j < FN; ++j) lds_read16(fb[ks][j], fb_base + ch + j * 4096);
  };
  auto mma_step = [&](int ks) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][j], fa[ks][i], acc[i][j], 0, 0, 0);
  };

  const int nk = K / BK;
  dma(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // next step's tiles go to the other buffer, whose last reads completed
    // before the barrier; the last step re-fetches its own slice there
    dma((kt + 1) & 1, min(kt + 1, nk - 1) * BK);
    const uint32_t st_off = (kt & 1) * STAGE;
    read_step(st_off, 0);
    read_step(st_off, 1);
    lgkm_wait<FM + FN>(fa[0], fb[0]);
    mma_step(0);
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) {
      if (ks + 1 < KS) {
        read_step(st_off, ks + 1);
        lgkm_wait<FM + FN>(fa[ks], fb[ks]);
      } else {
        lgkm_wait<0>(fa[ks], fb[ks]);
      }
      mma_step(ks);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS write outlives the loop

  // Accumulator layout (B fragment first): lane holds row m = base + lane%32 and
  // columns n = base + 8*(v/4) + 4*(lane/32) + v%4.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * WTM + i * 32 + frow;
    if (m >= M) continue;
    const auto rc = e.row(g, m);
    if constexpr (GATEUP) {
#pragma unroll
      for (int j = 0; j < FN; j += 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * WTN + j * 32 + q * 8 + fhalf * 4;  // gate column (n % 64 < 32)
          if (n < N) {
            float gv[4], uv[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              gv[t] = acc[i][j][q * 4 + t];
              uv[t] = acc[i][j + 1][q * 4 + t];
            }
            e.store4_pair(rc, (n >> 6) * 32 + (n & 31), gv, uv);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * WTN + j * 32 + q * 8 + fhalf * 4;
          if (n < N) {
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = acc[i][j][q * 4 + t];
            e.store4(rc, n, N, v);
          }
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
