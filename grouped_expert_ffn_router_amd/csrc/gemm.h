// GEMM core of libmoe: C[m][n] = sum_k A[m][k] * B[n][k] ("NT": both operands
// K-contiguous), fp32 accumulation, with pluggable operand sources and
// epilogues so that one kernel serves the router + down projection, the
// grouped expert FFNs (row gather from the receive pools, SwiGLU pairing,
// scatter into the return pools) and the shared experts + up-projection.
//
// bf16 path (gfx950): one 512-thread workgroup (8 waves, 2 x 4) per BM x BN
// output tile; each wave owns a (BM/2) x (BN/4) sub-tile built from
// v_mfma_f32_32x32x16_bf16.  K advances in steps of 64 through two LDS
// buffers filled straight from HBM (16-byte global->LDS loads, each group of
// 8 lanes reading one 128-byte row segment) ahead of the MFMAs.
// LDS rows are 128 bytes with the 16-byte chunk index XOR-swizzled per row,
// so the fragment reads run at the bank-conflict-free rate.
// The MFMA is issued with the B fragment as its first operand, so every lane
// ends up holding one output row m and runs of 4 consecutive columns n.  The
// bf16 store, scatter and SwiGLU epilogues (and the router's latent tiles)
// round the tile into LDS and store whole row segments, 16 bytes per lane,
// with each row's destination read when the tile starts; the router's logit
// tiles and the tail-split fixup store a lane's 4-column pieces directly.
// Workgroup ids are remapped so that each XCD (blocks are dealt round-robin
// to the 8 XCDs) works on a contiguous, M-grouped range of tiles and reuses
// operand rows from its own L2.
//
// fp32 path: a plain per-element kernel (small layers only).
#pragma once

#include <type_traits>

#include "moe_common.h"

namespace moe {

// ------------------------------------------------------------ A operands
// rows(g): rows of group g; row(g, m): pointer to element 0 of row m.

// First row of group g in a bank whose groups are laid end to end: the rows
// of the groups before it.
__device__ __forceinline__ int64_t ragged_row0(const int32_t* counts, int g) {
  int64_t r = 0;
  for (int i = 0; i < g; ++i) r += counts[i];
  return r;
}

template <class T>
struct ARows {  // row m of group g at base + g*group_stride + m*lda
  const T* base;
  int64_t lda, group_stride;
  const int32_t* counts;  // device rows per group, or NULL: rows_const
  int rows_const;
  // > 0: the groups' rows are laid end to end in a bank of ragged_rows rows
  // (group g starts after the counts of the groups before it; group_stride
  // unused); a row past the bank reads its last row
  int64_t ragged_rows = 0;
  __device__ int rows(int g) const { return counts ? counts[g] : rows_const; }
  __device__ const T* row(int g, int m) const {
    if (ragged_rows > 0) {
      const int64_t r = ragged_row0(counts, g) + m;
      return base + (r < ragged_rows ? r : ragged_rows - 1) * lda;
    }
    return base + g * group_stride + (int64_t)m * lda;
  }
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

// Index of the k1-long segment holding K offset kk, for kk and k1 multiples
// of 64 (inv_k1 = 1 / k1 in float): floor((kk + 32) / k1) has its true value
// at least 32 / k1 away from an integer, more than the error of the float
// product for kk < 2^24, so truncating the product is exact there.
__host__ __device__ __forceinline__ int kseg_index(int kk, float inv_k1) {
  return (int)((float)(kk + 32) * inv_k1);
}

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
  float inv_k1;  // 1 / k1 (0 when there are no k1 segments)
  // The part of the address of B[n][k .. k+63] shared by every row, for k a
  // multiple of 64 (k0 and k1 are too, so a K step stays inside one
  // segment); k is uniform across the workgroup.  Branch-free, so that it
  // sits inside the MFMA-interleaved K loop without splitting it (the
  // segment index comes from kseg_index; K < 2^24 is checked on the host).
  // Row n then adds n * ld0 in the first segment and n * ld1 in the others.
  __device__ const T* kbase(int k, bool& first) const {
    first = k < k0;
    const int kk = k - k0;
    const int j = __builtin_amdgcn_readfirstlane(first ? 0 : kseg_index(kk, inv_k1));
    const uint64_t seg = (uint64_t)(b1 + (int64_t)j * stride1 + (kk - j * k1));
    const uint64_t lead = (uint64_t)(b0 + k), pick = first ? ~0ull : 0ull;  // a blend, not a branch
    return (const T*)((lead & pick) | (seg & ~pick));
  }
};

// ------------------------------------------------------------ epilogues
// Scalar interface (fp32 kernel): store(g, m, n, v) / store2(g, m, u, gate, up).
// Vector interface (MFMA kernel): row(g, m) -> per-row context, then
// store4(ctx, n, v[4]) for columns n..n+3 (n % 4 == 0, clipped at N), or
// store4_pair(ctx, u, gate[4], up[4]) for hidden units u..u+3.

__device__ __forceinline__ uint2 pack_bf16x4(const float* v) {
  return make_uint2(f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3]));
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

// Staged epilogue (STAGED = true): the MFMA kernel rounds the tile to
// activations in LDS and stores whole row segments.  row_key(g, m), which may
// read memory, is taken for every row of the tile when the tile starts (its
// latency hides behind the K loop); key_dst(key), which reads nothing, gives
// element 0 of the output row (NULL: not stored), and the kernel writes
// columns n0 .. n0 + BN - 1 (hidden units n0/2 .. for SwiGLU pairs).
template <class T>
struct ERouteDown {  // columns < E: fp32 logits (+bias); the rest: latent z
  // tiles of latent columns only go through the staged epilogue (E a
  // multiple of 8 keeps their 16-byte pieces aligned); tiles holding logits
  // store from registers
  static constexpr bool STAGED = true;
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
  __device__ bool staged_tile(int n0) const { return n0 >= E && (E & 7) == 0; }
  __device__ int64_t row_key(int, int m) const { return m; }
  // element 0 of the row in output-column numbering: column n >= E lands at z[m][n - E]
  __device__ T* key_dst(int64_t key) const { return z + key * L - E; }
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
  static constexpr bool STAGED = true;
  T* out;
  int64_t ldo, group_stride;
  int col0;
  // > 0: groups laid end to end in a bank of ragged_rows rows, as ARows
  // (rows per group from counts); a row past the bank is not stored
  const int32_t* counts = nullptr;
  int64_t ragged_rows = 0;
  __device__ T* dest(int g, int m) const {
    if (ragged_rows > 0) {
      const int64_t r = ragged_row0(counts, g) + m;
      return r < ragged_rows ? out + r * ldo + col0 : nullptr;
    }
    return out + g * group_stride + (int64_t)m * ldo + col0;
  }
  __device__ void store2(int g, int m, int u, float gate, float up) const {
    T* p = dest(g, m);
    if (p) p[u] = Act<T>::store(silu(gate) * up);
  }
  struct Row { T* p; };
  __device__ Row row(int g, int m) const { return {dest(g, m)}; }
  __device__ bool staged_tile(int) const { return true; }
  // staged epilogue: element offset of row m's first hidden unit, -1: not stored
  __device__ int64_t row_key(int g, int m) const {
    const T* p = dest(g, m);
    return p ? (int64_t)(p - out) : -1;
  }
  __device__ T* key_dst(int64_t key) const { return key < 0 ? nullptr : out + key; }
  __device__ void store4_pair(const Row& r, int u, const float* gate, const float* up) const {
    if (!r.p) return;
    float h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = silu(gate[i]) * up[i];
    put4(r.p + u, h, 4);
  }
};

template <class T>
struct EScatter {  // row m of group g -> return row of receive row row_src[g][m]
  static constexpr bool STAGED = true;
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
  __device__ bool staged_tile(int) const { return true; }
  // staged epilogue: the receive row (s * cap + slot) whose return row row m fills
  __device__ int64_t row_key(int g, int m) const { return row_src[g * rs_stride + m]; }
  __device__ T* key_dst(int64_t key) const {
    const int rs = (int)key, s = rs / cap, sl = rs - s * cap;
    return (T*)(ret + s * src_stride + (int64_t)sl * row_bytes);
  }
  __device__ void store4(const Row& r, int n, int N, const float* v) const { put4(r.p + n, v, N - n); }
};

template <class T>
struct EStore {
  static constexpr bool STAGED = true;
  T* out;
  int64_t ldo;
  __device__ bool staged_tile(int) const { return true; }
  __device__ int64_t row_key(int, int m) const { return m; }
  __device__ T* key_dst(int64_t key) const { return out + key * ldo; }
  __device__ void store(int, int m, int n, float v) const { out[(int64_t)m * ldo + n] = Act<T>::store(v); }
  struct Row { T* p; };
  __device__ Row row(int, int m) const { return {out + (int64_t)m * ldo}; }
  __device__ void store4(const Row& r, int n, int N, const float* v) const { put4(r.p + n, v, N - n); }
};

// ------------------------------------------------------------ bf16 MFMA kernel

template <int BM_, int BN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64;       // 2 LDS buffers of BK-deep tiles
  static constexpr int NT = 512;                          // 8 waves (2 per SIMD), 2 x 4
  static constexpr int WTM = BM / 2, WTN = BN / 4;        // wave sub-tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;      // 32x32 fragments per wave
  static constexpr int RPW = BM / 8;                      // rows of each operand one wave loads
  static constexpr int LA = RPW / 8, LB = RPW / 8;        // 16-byte loads per lane per K step
  static constexpr int ROW = BK * 2;                      // bytes of one LDS row (128)
  static constexpr int STAGE = (BM + BN) * ROW;           // bytes of one LDS buffer
  static_assert(BM == 256 && BN == 256, "the loader and fragment layout assume 256 x 256 tiles");
  static_assert(2 * STAGE <= 160 * 1024, "LDS budget of one workgroup");
};

// ---- work assignment
// The output tiles that exist (rows(g) of each group, so a count read on the
// device) are numbered group by group, M-grouped (GROUP_M tile rows at a
// time) inside a group.  With P workgroups running at once, T tiles take
// ceil(T / P) rounds; when the last round would hold only r <= P/2 tiles,
// those r tiles are split along K into s parts each (s * r <= P, at least
// KSPLIT_MIN steps per part) that run side by side as that round, each
// writing an fp32 partial tile; a second kernel adds the parts in part order
// and applies the epilogue.  The split is taken only where it shortens the
// tail by KSPLIT_GAIN steps or more: that kernel and the partial traffic cost
// about as much as a dozen K steps of a tile.  The other T - r tiles are dealt to the XCDs
// (workgroups go round-robin to the 8 XCDs) in contiguous ranges, so each
// XCD's L2 sees neighbouring tiles; the tail parts come after them.

constexpr int KSPLIT_MIN = 4;    // K steps of one tail part, at least
constexpr int KSPLIT_GAIN = 24;  // K steps a split must take off the tail, at least
constexpr int PART_SLOTS = 256;  // partial tiles one launch may write

struct TailPlan {
  int total, tail, parts;  // tiles, tail tiles (r), parts per tail tile (s)
};

template <class A>
__host__ __device__ __forceinline__ TailPlan tail_plan(const A& a, int groups, int tiles_n, int nk, int P, bool can_split) {
  TailPlan t{0, 0, 0};
  for (int g = 0; g < groups; ++g) t.total += (a.rows(g) + 255) / 256 * tiles_n;
  const int r = t.total % P;
  if (can_split && r > 0 && 2 * r <= P) {
    const int s = P / r < nk / KSPLIT_MIN ? P / r : nk / KSPLIT_MIN;
    if (s >= 2 && nk - nk / s >= KSPLIT_GAIN) {
      t.tail = r;
      t.parts = s;
    }
  }
  return t;
}

// Tile number t -> (group, tile row, tile column).
template <class A>
__host__ __device__ __forceinline__ void tile_coords(const A& a, int groups, int tiles_n, int t, int& g, int& tm, int& tn) {
  int mt = 0;
  for (g = 0; g < groups; ++g) {
    mt = (a.rows(g) + 255) / 256;
    if (t < mt * tiles_n) break;
    t -= mt * tiles_n;
  }
  constexpr int GROUP_M = 4;  // 32 tiles of an XCD at once: 4 tile rows x 8 tile columns
  const int width = GROUP_M * tiles_n;
  const int gid = t / width, first_m = gid * GROUP_M;
  const int gsz = mt - first_m < GROUP_M ? mt - first_m : GROUP_M;
  const int rr = t - gid * width;
  tm = first_m + rr % gsz;
  tn = rr / gsz;
}

// Work of workgroup `bid`: tile t and K steps [kb, ke); slot >= 0 names the
// partial this tail part writes.  False: nothing to do.
__host__ __device__ __forceinline__ bool block_work(const TailPlan& p, int nk, int bid, int& t, int& kb, int& ke, int& slot) {
  const int D = p.total - p.tail;
  const int xcd = bid & 7, idx = bid >> 3;
  const int per = D >> 3, rem = D & 7;
  const int len = per + (xcd < rem ? 1 : 0), maxlen = per + (rem ? 1 : 0);
  kb = 0;
  ke = nk;
  slot = -1;
  if (idx < len) {
    t = xcd * per + (xcd < rem ? xcd : rem) + idx;
    return true;
  }
  if (idx < maxlen) return false;
  const int q = (idx - maxlen) * 8 + xcd;
  if (q >= p.tail * p.parts) return false;
  t = D + q / p.parts;
  const int part = q % p.parts;
  kb = part * nk / p.parts;
  ke = (part + 1) * nk / p.parts;
  slot = q;
  return true;
}

// Workgroups a launch needs for at most max_tiles tiles (host side).
inline int64_t gemm_grid(int64_t max_tiles, int P) { return 8 * ((max_tiles + 7) / 8 + (P + 7) / 8); }

// 16-byte LDS read at byte address `addr`, issued as inline assembly: the
// result must be awaited with lgkm_wait before use.
__device__ __forceinline__ void lds_read16(bf16x8& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
}

// Wait until at most N LDS reads are outstanding; the fragments pass through
// the statement so that their consumers stay behind it.
template <int N, int FM, int FN>
__device__ __forceinline__ void lgkm_wait(bf16x8 (&fa)[FM], bf16x8 (&fb)[FN]) {
  static_assert(FM == 4 && FN == 2, "fragment counts of a 128 x 64 wave tile");
  asm volatile("s_waitcnt lgkmcnt(%6)"
               : "+v"(fa[0]), "+v"(fa[1]), "+v"(fa[2]), "+v"(fa[3]), "+v"(fb[0]), "+v"(fb[1])
               : "i"(N)
               : "memory");
}

// Workgroup barrier without a memory fence.  __syncthreads() would also wait
// for every outstanding load, including the HBM->LDS loads of later steps
// that must stay in flight; the LDS data a barrier publishes here was
// awaited explicitly (vm_wait) by the lane that loaded it, and LDS is
// coherent within the workgroup.
__device__ __forceinline__ void lds_barrier() { __builtin_amdgcn_s_barrier(); }

// Wait until at most N vector-memory loads (here: HBM->LDS loads) of this
// lane are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// 16-byte chunk swizzle of a 128-byte LDS row (8 chunks): chunk c of row r
// is stored at c ^ ((r >> 1) & 7).  Measured on gfx950 with the fragment read
// pattern below (32 rows x 2 chunks per instruction), this keeps 16-byte LDS
// reads at the bank-conflict-free rate (about 250 B/clk per CU); unswizzled
// rows run 8-way conflicted and r & 7 2-way.  Rows 16 apart share it.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// GATEUP: N counts gate+up columns (blocks of 64) and the epilogue gets
// (gate, up) pairs.
//
// Pipeline: two LDS buffers of 64-deep K steps; 8 waves, two per SIMD, so
// that one wave's MFMAs run while the other waits.  A step is 4 substeps of
// k16, each 8 MFMAs per wave on one set of fragments; every LDS read and
// every HBM->LDS load sits between two MFMAs (pinned by scheduling fences).
// Substep s reads the fragments of substep s+1.  The last substep waits for
// the next step's loads, passes the barrier (after which every wave is done
// with the current step's buffer), reads the first fragments of the next
// step and issues half of the loads of the step after next into the buffer
// just freed; the other half goes out in the next step's first substep.  A
// load so has most of a step (about 2000 MFMA cycles) to land.
// The fragment reads are inline ds_read_b128 (so the compiler, which cannot
// tell the two LDS buffers apart, does not make them wait for the loads in
// flight to the other buffer); a fragment stays live until the lgkm_wait that
// retires it, and every read is retired where the code passes from one step
// variant to another (their fragment registers differ) and at the end.
// Loads move 128-byte row segments (whole L2 lines); each wave's blocks are
// contiguous in LDS so one M0 value serves four loads through the
// instruction's immediate offset (which also shifts the HBM address; it is
// subtracted from the row pointers up front).
// Epilogue of 4 columns per fragment of one output row (context rc), columns
// nbase + j*32 + q*8 + fhalf*4 .. +3 for fragment j.  Accumulator layout (B
// fragment first): lane holds row m = base + lane%32 and columns
// n = base + 8*(v/4) + 4*(lane/32) + v%4 of a fragment.
template <bool GATEUP, int FN, class E, class Row>
__device__ __forceinline__ void epilogue_q(const E& e, const Row& rc, int nbase, int N, int fhalf, int q,
                                           const float (&v)[FN][4]) {
  if constexpr (GATEUP) {
    static_assert(FN % 2 == 0, "gate and up fragments come in pairs");
#pragma unroll
    for (int j = 0; j < FN; j += 2) {
      const int n = nbase + j * 32 + q * 8 + fhalf * 4;  // gate column (n % 64 < 32)
      if (n < N) e.store4_pair(rc, (n >> 6) * 32 + (n & 31), v[j], v[j + 1]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = nbase + j * 32 + q * 8 + fhalf * 4;
      if (n < N) e.store4(rc, n, N, v[j]);
    }
  }
}

// Epilogue of fragment row i of a wave (one output row m per lane pair).
template <bool GATEUP, int FN, class E>
__device__ __forceinline__ void epilogue_row(const E& e, int g, int m, int M, int nbase, int N, int fhalf,
                                             const f32x16 (&accr)[FN]) {
  if (m >= M) return;
  const auto rc = e.row(g, m);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v[FN][4];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) v[j][t] = accr[j][q * 4 + t];
    epilogue_q<GATEUP, FN>(e, rc, nbase, N, fhalf, q, v);
  }
}

// Staged epilogue of a whole tile (all 512 threads; LDS free of the K loop's
// operands).  Each lane rounds its accumulators (SwiGLU pairs first) to bf16
// and writes them as 8-byte pieces into a row-major copy of the output tile
// in LDS: OC output columns per row, the 16-byte chunks of a row XOR-swizzled
// with the row index so that the 32 rows a write instruction touches fall in
// different banks.  Then each wave stores 32 rows, 16 bytes per lane, whole
// row segments (OC * 2 bytes) per group of lanes: every store instruction
// writes full 128-byte lines, where the per-fragment pieces of the
// accumulator layout would write 16 bytes of 32 different rows.  The values
// and their rounding are those of the direct epilogue.
template <class Cfg, bool GATEUP, class E>
__device__ __forceinline__ void staged_epilogue(const E& e, int m0, int n0, int M, int N, char* smem,
                                                int64_t* keys, int64_t my_key,
                                                const f32x16 (&acc)[Cfg::FM][Cfg::FN]) {
  constexpr int FM = Cfg::FM, FN = Cfg::FN, WTM = Cfg::WTM, WTN = Cfg::WTN, BM = Cfg::BM;
  constexpr int OC = GATEUP ? Cfg::BN / 2 : Cfg::BN;  // output columns of the tile
  constexpr int RB = OC * 2;                         // bytes of one staged row
  constexpr int CH = RB / 16;                        // 16-byte chunks per row (a power of two)
  static_assert(BM * RB <= 2 * Cfg::STAGE, "the staged tile fits the operand buffers");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3, frow = lane & 31, fhalf = lane >> 5;
  if (tid < BM) keys[tid] = my_key;  // taken when the tile started
  __syncthreads();  // every wave is done reading operands (no loads are in flight here)
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = wm * WTM + i * 32 + frow;
    char* lrow = smem + row * RB;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int j = 0; j < FN; j += (GATEUP ? 2 : 1)) {
        const int n = wn * WTN + j * 32 + q * 8 + fhalf * 4;  // tile column (gate column for pairs)
        const int oc = GATEUP ? (n >> 6) * 32 + (n & 31) : n;
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          v[t] = GATEUP ? silu(acc[i][j][q * 4 + t]) * acc[i][j + (GATEUP ? 1 : 0)][q * 4 + t] : acc[i][j][q * 4 + t];
        const int byte = oc * 2;
        *(uint2*)(lrow + (((byte >> 4) ^ (row & (CH - 1))) << 4) + (byte & 15)) = pack_bf16x4(v);
      }
    }
  }
  __syncthreads();
  constexpr int RPI = 64 / CH;  // rows per store instruction
  const int col0 = (GATEUP ? n0 / 2 : n0), ncols = GATEUP ? N / 2 : N;
  const int c = lane % CH;
#pragma unroll 4
  for (int it = 0; it < 32 / RPI; ++it) {
    const int row = wave * 32 + it * RPI + lane / CH;
    const uint4 d = *(const uint4*)(smem + row * RB + ((c ^ (row & (CH - 1))) << 4));
    if (m0 + row < M && col0 + c * 8 < ncols) {
      bf16_t* p = e.key_dst(keys[row]);
      if (p) *(uint4*)(p + col0 + c * 8) = d;
    }
  }
}

// Partial tile layout: float4 chunk c (0..31, = (i*FN + j)*4 + v/4) of thread
// tid at float offset (c * 512 + tid) * 4 of the slot (coalesced).
constexpr int PART_FLOATS = 256 * 256;

// grid: gemm_grid(groups * ceil(max_rows / 256) * tiles_n, P); block: 512.
// K must be a multiple of 64.  part: PART_SLOTS partial tiles, or NULL (no
// tail split).
template <class Cfg, bool GATEUP, class A, class B, class E>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_bf16_mfma(A a, B b, E e, int N, int K, int groups, int tiles_n, int P, float* part) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, WTM = Cfg::WTM, WTN = Cfg::WTN;
  constexpr int FM = Cfg::FM, FN = Cfg::FN, LA = Cfg::LA, LB = Cfg::LB, STAGE = Cfg::STAGE;
  constexpr int ROW = Cfg::ROW, RPW = Cfg::RPW, NLOAD = LA + LB, WBYTES = RPW * ROW;
  static_assert(LA == 4 && LB == 4, "one M0 value per operand and wave");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int nk = K / BK;
  const TailPlan plan = tail_plan(a, groups, tiles_n, nk, P, part != nullptr);
  int t, kb, ke, slot;
  if (!block_work(plan, nk, blockIdx.x, t, kb, ke, slot)) return;
  int g, tm, tn;
  tile_coords(a, groups, tiles_n, t, g, tm, tn);
  const int M = a.rows(g);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  // the staged epilogue's row keys (e.g. a scatter's row lookups), read now
  // so that their latency hides behind the K loop
  __shared__ int64_t keys[E::STAGED ? BM : 1];
  int64_t my_key = -1;
  bool staged = false;
  if constexpr (E::STAGED) {
    staged = slot < 0 && e.staged_tile(n0);
    if (staged && tid < BM && m0 + tid < M) my_key = e.row_key(g, m0 + tid);
  }

  // wave w owns the 4 LDS blocks (1 KB = 8 rows) w*4 .. w*4+3 of A and of B:
  // slot d holds rows w*32 + d*8 + lane/8, lane lands at block + 16*lane.
  const int lrow = lane >> 3, lcol = lane & 7;
  int gcola[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) gcola[p] = (lcol ^ swz(wave * RPW + p * 8 + lrow)) * 8;
  const bf16_t* pa[LA];
#pragma unroll
  for (int d = 0; d < LA; ++d)
    pa[d] = a.row(g, min(m0 + wave * RPW + d * 8 + lrow, M - 1)) + gcola[d & 1] - 512 * d;
  const bf16_t* pb[LB];
  int nb_row[LB];
#pragma unroll
  for (int d = 0; d < LB; ++d) {
    nb_row[d] = min(n0 + wave * RPW + d * 8 + lrow, N - 1);
    pb[d] = b.ptr(g, nb_row[d], gcola[d & 1]) - 512 * d;
  }
  // K-concatenated B: each lane's row offsets in the first segment and in
  // the others; a load adds the one its (uniform) K step needs.
  // (Two arrays picked by a select: an array indexed by the segment would be
  // a dynamically indexed private array.)
  int64_t kso0[LB], kso1[LB];
  if constexpr (B::KSEG) {
#pragma unroll
    for (int d = 0; d < LB; ++d) {
      kso0[d] = (int64_t)nb_row[d] * b.ld0 + gcola[d & 1] - 512 * d;
      kso1[d] = (int64_t)nb_row[d] * b.ld1 + gcola[d & 1] - 512 * d;
    }
  }

  const int frow = lane & 31, fhalf = lane >> 5;
  const int fswz = swz(frow);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  const uint32_t fa_base = lds0 + (wm * WTM + frow) * ROW, fb_base = lds0 + BM * ROW + (wn * WTN + frow) * ROW;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  struct Frags {
    bf16x8 a[FM], b[FN];
  };
  constexpr int NF = FM + FN, NMMA = FM * FN, KS = BK / 16, LH = NLOAD / 2;
  static_assert(NF <= NMMA && LH <= NMMA && KS % 2 == 0, "one read and one load per MFMA slot at most");
  auto read1 = [&](Frags& f, int kt, int ks, int q) {
    const uint32_t st = (uint32_t)((kt & 1) * STAGE) + (uint32_t)(((ks * 2 + fhalf) ^ fswz) << 4);
    if (q < FM) lds_read16(f.a[q], fa_base + st + q * 32 * ROW);
    else lds_read16(f.b[q - FM], fb_base + st + (q - FM) * 32 * ROW);
  };
  auto load1 = [&](int kt, int d) {  // d in [0, NLOAD), kt < nk
    const int k0 = kt * BK;
    char* s = smem + (kt & 1) * STAGE;
    const void* gp;
    char* lp;
    const int dd = d < LA ? d : d - LA;
    if (d < LA) {
      gp = (const void*)(pa[dd] + k0);
      lp = s + wave * WBYTES;
    } else {
      if constexpr (B::KSEG) {
        bool first;
        const bf16_t* kb = b.kbase(k0, first);
        gp = (const void*)(kb + (first ? kso0[dd] : kso1[dd]));
      } else {
        gp = (const void*)(pb[dd] + k0);
      }
      lp = s + BM * ROW + wave * WBYTES;
    }
    auto l3 = (__attribute__((address_space(3))) void*)lp;
    switch (dd) {
      case 0: __builtin_amdgcn_global_load_lds(gp, l3, 16, 0, 0); break;
      case 1: __builtin_amdgcn_global_load_lds(gp, l3, 16, 1024, 0); break;
      case 2: __builtin_amdgcn_global_load_lds(gp, l3, 16, 2048, 0); break;
      default: __builtin_amdgcn_global_load_lds(gp, l3, 16, 3072, 0); break;
    }
  };
  auto mma1 = [&](const Frags& f, int q) {  // B fragment j held for FM consecutive MFMAs
    const int j = q / FM, i = q % FM;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  };
  Frags F[2];  // substep ks computes on F[ks & 1] while F[(ks + 1) & 1] is read
  // One K step.  MODE 0: issues loads [0, LH) of step kt+2 after its barrier;
  // 1: no new loads; 2: the last step (no barrier, no next reads).  HALF:
  // the previous step left loads [LH, NLOAD) of step kt+1 to substep 0.
  auto step = [&](int kt, auto mode_tag, auto half_tag) {
    constexpr int MODE = decltype(mode_tag)::value;
    constexpr bool HALF = decltype(half_tag)::value;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Frags& cur = F[ks & 1];
      Frags& nxt = F[(ks + 1) & 1];
      lgkm_wait<0>(cur.a, cur.b);
      if (ks + 1 < KS) {
#pragma unroll
        for (int q = 0; q < NMMA; ++q) {
          mma1(cur, q);
          if (q < NF) read1(nxt, kt, ks + 1, q);
          if (HALF && ks == 0 && q < NLOAD - LH) load1(kt + 1, LH + q);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        if (MODE != 2) {
          vm_wait<0>();   // step kt+1's tiles (this lane's part)
          lds_barrier();  // ... every lane's; every wave is done with step kt's buffer
        }
#pragma unroll
        for (int q = 0; q < NMMA; ++q) {
          mma1(cur, q);
          if (MODE != 2 && q < NF) read1(nxt, kt + 1, 0, q);
          if (MODE == 0 && q < LH) load1(kt + 2, q);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  using Loads = std::integral_constant<int, 0>;
  using NoLoads = std::integral_constant<int, 1>;
  using Last = std::integral_constant<int, 2>;
  using Half = std::true_type;
  using Whole = std::false_type;
  // K steps [kb, ke): a whole tile, or one part of a tail tile
  const int ns = ke - kb;
#pragma unroll
  for (int d = 0; d < NLOAD; ++d) load1(kb, d);
  vm_wait<0>();
  lds_barrier();
  if (ns > 1) {
#pragma unroll
    for (int d = 0; d < NLOAD; ++d) load1(kb + 1, d);
  }
#pragma unroll
  for (int q = 0; q < NF; ++q) read1(F[0], kb, 0, q);
  lgkm_wait<0>(F[0].a, F[0].b);
  if (ns >= 3) {
    step(kb, Loads(), Whole());
    lgkm_wait<0>(F[0].a, F[0].b);
    for (int kt = kb + 1; kt + 2 < ke; ++kt) step(kt, Loads(), Half());
    lgkm_wait<0>(F[0].a, F[0].b);
    step(ke - 2, NoLoads(), Half());
    lgkm_wait<0>(F[0].a, F[0].b);
    step(ke - 1, Last(), Whole());
  } else if (ns == 2) {
    step(kb, NoLoads(), Whole());
    lgkm_wait<0>(F[0].a, F[0].b);
    step(kb + 1, Last(), Whole());
  } else {
    step(kb, Last(), Whole());
  }

  if (slot >= 0) {  // one part of a tail tile: fp32 partial, finished by gemm_bf16_fixup
    float4* dst = (float4*)(part + (int64_t)slot * PART_FLOATS);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          dst[((i * FN + j) * 4 + v) * 512 + tid] =
              make_float4(acc[i][j][v * 4], acc[i][j][v * 4 + 1], acc[i][j][v * 4 + 2], acc[i][j][v * 4 + 3]);
    return;
  }
  if (staged) {  // uniform per workgroup
    if constexpr (E::STAGED) staged_epilogue<Cfg, GATEUP>(e, m0, n0, M, N, smem, keys, my_key, acc);
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      epilogue_row<GATEUP, FN>(e, g, m0 + wm * WTM + i * 32 + frow, M, n0 + wn * WTN, N, fhalf, acc[i]);
  }
}

// Tail tiles of a gemm_bf16_mfma launch with the same arguments: adds each
// tile's parts in part order and applies the epilogue.  One 64-lane
// workgroup per (tail tile, wave, fragment row, column quad), grid-stride;
// the parts are read 8 at a time so that many loads are in flight.
template <class Cfg, bool GATEUP, class A, class E>
__global__ void __launch_bounds__(64) gemm_bf16_fixup(A a, E e, int N, int K, int groups, int tiles_n, int P,
                                                      const float* part) {
  constexpr int FM = Cfg::FM, FN = Cfg::FN, PB = 8;
  const TailPlan plan = tail_plan(a, groups, tiles_n, K / Cfg::BK, P, true);
  const int items = plan.tail * 8 * FM * 4;
  const int lane = threadIdx.x, frow = lane & 31, fhalf = lane >> 5;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int ti = it / (8 * FM * 4), w = (it / (FM * 4)) % 8, i = (it / 4) % FM, q = it % 4;
    const int wm = w >> 2, wn = w & 3, tid = w * 64 + lane;
    int g, tm, tn;
    tile_coords(a, groups, tiles_n, plan.total - plan.tail + ti, g, tm, tn);
    const int m = tm * Cfg::BM + wm * Cfg::WTM + i * 32 + frow;
    if (m >= a.rows(g)) continue;
    const float4* src = (const float4*)(part + (int64_t)ti * plan.parts * PART_FLOATS);
    float4 sum[FN];
    for (int p0 = 0; p0 < plan.parts; p0 += PB) {
      float4 x[PB][FN];
#pragma unroll
      for (int u = 0; u < PB; ++u)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if (p0 + u < plan.parts) x[u][j] = src[(int64_t)(p0 + u) * (PART_FLOATS / 4) + ((i * FN + j) * 4 + q) * 512 + tid];
#pragma unroll
      for (int u = 0; u < PB; ++u)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if (p0 + u < plan.parts) {
            if (p0 + u == 0) {
              sum[j] = x[u][j];
            } else {
              sum[j].x += x[u][j].x; sum[j].y += x[u][j].y; sum[j].z += x[u][j].z; sum[j].w += x[u][j].w;
            }
          }
    }
    float v[FN][4];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      v[j][0] = sum[j].x; v[j][1] = sum[j].y; v[j][2] = sum[j].z; v[j][3] = sum[j].w;
    }
    epilogue_q<GATEUP, FN>(e, e.row(g, m), tn * Cfg::BN + wn * Cfg::WTN, N, fhalf, q, v);
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
