// Routing, slot assignment and row-movement kernels of libmoe (gfx950).
//
// Top-k selection: one wave per token, k rounds of a wave-wide maximum over
// order-preserving (logit, expert) keys, reduced with DPP and lane reads.
// Slot assignment is a deterministic two-pass scan: one 256-thread block
// ranks SCAN_CHUNK keys with wave64 ballots (the lanes holding the same key
// are found with one ballot per key bit, then a popcount of the lower
// lanes), then one block per key value scans the per-chunk counts.  No
// atomics.

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

// ------------------------------------------------------------------ top-k

// Order-preserving 64-bit key of (logit, expert): a larger logit first, then
// the lower expert index; -0.0 is folded into +0.0 so that equal logits give
// equal high halves.  Padding entries get key 0, below every real key.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)~(uint32_t)e;
}

__device__ __forceinline__ float topk_key_value(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// DPP move of a 64-bit value (two 32-bit halves) with control CTRL.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), CTRL, 0xf, 0xf, false);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Largest key of the wave, in every lane: rotations by 8, 4, 2 and 1 lanes
// inside each 16-lane row (DPP row_ror) give every lane its row's maximum,
// then the four rows' maxima are read as scalars.  No LDS round trip.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  uint64_t t;
  t = dpp_u64<0x128>(k); k = t > k ? t : k;
  t = dpp_u64<0x124>(k); k = t > k ? t : k;
  t = dpp_u64<0x122>(k); k = t > k ? t : k;
  t = dpp_u64<0x121>(k); k = t > k ? t : k;
  const uint64_t r0 = readlane_u64(k, 0), r1 = readlane_u64(k, 16), r2 = readlane_u64(k, 32),
                 r3 = readlane_u64(k, 48);
  const uint64_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

// One wave per token: k rounds of a wave-wide argmax over (logit desc,
// expert asc) keys; lane i < k keeps the i-th pick.  Weights: softmax over
// the k picked logits, relative to the largest.
template <int EPL>
__global__ void __launch_bounds__(256)
select_topk_kernel(const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ idx,
                   float* __restrict__ w) {
  const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int lane = lane_id();
  if (t >= T) return;
  const float* row = logits + (int64_t)t * E;
  uint64_t key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? topk_key(row[e], e) : 0ull;
  }
  float my_v = 0.f, v0 = 0.f;
  int my_i = 0;
  for (int r = 0; r < k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_key(best);
    const int e = (int)~(uint32_t)best;
    const float v = topk_key_value(best);
    if (r == 0) v0 = v;
    if (lane == r) {
      my_v = v;
      my_i = e;
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (lane + 64 * j == e) key[j] = 0ull;
  }
  float ex = lane < k ? expf(my_v - v0) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    idx[(int64_t)t * k + lane] = my_i;
    w[(int64_t)t * k + lane] = ex / sum;
  }
}

hipError_t launch_select_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w, hipStream_t st) {
  const int epl = (E + 63) / 64;
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (T == 0) return hipSuccess;
#define SEL(N) launch(select_topk_kernel<N>, grid, block, 0, st, logits, T, E, k, idx, w)
  if (epl <= 1) SEL(1);
  else if (epl <= 2) SEL(2);
  else if (epl <= 4) SEL(4);
  else if (epl <= 6) SEL(6);
  else if (epl <= 8) SEL(8);
  else if (epl <= 16) SEL(16);
  else SEL(32);
#undef SEL
  return hipGetLastError();
}

// ------------------------------------------------------------ chunk ranking

// Rank of each lane's key among the lanes of this wave with the same key,
// offset by the running count run[key] (wave-private LDS), which is advanced.
// key < 0: no key; keys are below 2^kbits.  All lanes of the wave must call
// this together.  The lanes holding the same key are found with one ballot
// per key bit (a lane keeps the lanes that agree with it on every bit), so
// the cost does not grow with the number of distinct keys in the wave; each
// group's lowest lane advances run[key].
__device__ __forceinline__ int peel_rank(int key, int32_t* run, int kbits) {
  const bool valid = key >= 0;
  uint64_t same = __ballot(valid);
  for (int b = 0; b < kbits; ++b) {
    const bool bit = valid && ((key >> b) & 1);
    const uint64_t ones = __ballot(bit);
    same &= bit ? ones : ~ones;
  }
  const uint64_t below = same & lanemask_lt();
  const int before = valid ? run[key] : 0;
  if (valid && below == 0) run[key] = before + __popcll(same);
  return before + __popcll(below);
}

// Block-wide: rank 1024 keys (4 waves x 4 x 64) inside the chunk; write each
// key's chunk-local rank and the per-key chunk count (column-major: [key][chunk]).
// key values in [0, KW).  get_key(i) returns -1 for "no key".
template <class GetKey>
__device__ __forceinline__ void chunk_rank(GetKey get_key, int n, int KW, int nch, int32_t* run_all,
                                           int32_t* __restrict__ local_rank, int32_t* __restrict__ chunk_count,
                                           int32_t* __restrict__ key_out) {
  for (int i = threadIdx.x; i < 4 * KW; i += 256) run_all[i] = 0;
  __syncthreads();
  int kbits = 0;
  while ((1 << kbits) < KW) ++kbits;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  int32_t* run = run_all + wave * KW;
  const int base = blockIdx.x * SCAN_CHUNK + wave * 256;
  int key[4], rk[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int i = base + it * 64 + lane;
    key[it] = i < n ? get_key(i) : -1;
    rk[it] = peel_rank(key[it], run, kbits);
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int i = base + it * 64 + lane;
    if (i < n) {
      if (key_out) key_out[i] = key[it];
      if (key[it] >= 0) {
        int off = 0;
        for (int w = 0; w < wave; ++w) off += run_all[w * KW + key[it]];
        local_rank[i] = off + rk[it];
      }
    }
  }
  for (int kk = threadIdx.x; kk < KW; kk += 256)
    chunk_count[(int64_t)kk * nch + blockIdx.x] =
        run_all[kk] + run_all[KW + kk] + run_all[2 * KW + kk] + run_all[3 * KW + kk];
}

// Exclusive scan of one key's chunk counts (one block per key column).
// Returns the column total to every thread.
__device__ __forceinline__ int column_scan(const int32_t* __restrict__ col_in, int32_t* __restrict__ col_out,
                                           int nch) {
  __shared__ int32_t part[256];
  const int per = (nch + 255) / 256;
  const int c0 = threadIdx.x * per;
  int s = 0;
  for (int c = c0; c < c0 + per && c < nch; ++c) s += col_in[c];
  part[threadIdx.x] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over 256 partial sums
  for (int off = 1; off < 256; off <<= 1) {
    const int v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = part[threadIdx.x] - s;
  for (int c = c0; c < c0 + per && c < nch; ++c) {
    const int v = col_in[c];
    col_out[c] = run;
    run += v;
  }
  const int total = part[255];
  __syncthreads();
  return total;
}

// ------------------------------------------------------------------ send

__global__ void __launch_bounds__(256)
send_rank_kernel(const int32_t* __restrict__ idx, int n_assign, int X, int E, int R,
                 int32_t* __restrict__ local_rank, int32_t* __restrict__ chunk_count, int nch) {
  extern __shared__ int32_t run_all[];
  auto key = [&](int a) {
    const int e = idx[a];
    return (e >= 0 && e < E) ? e / X : R;  // R: invalid expert id
  };
  chunk_rank(key, n_assign, R + 1, nch, run_all, local_rank, chunk_count, nullptr);
}

hipError_t launch_send_rank(const int32_t* idx, int n_assign, int X, int E, int R, int32_t* local_rank,
                            int32_t* chunk_count, hipStream_t st) {
  const int nch = (n_assign + SCAN_CHUNK - 1) / SCAN_CHUNK;
  if (nch == 0) return hipSuccess;
  launch(send_rank_kernel, dim3(nch), dim3(256), 4 * (R + 1) * sizeof(int32_t), st, idx, n_assign,
                     X, E, R, local_rank, chunk_count, nch);
  return hipGetLastError();
}

// Block d scans destination d's chunk counts; writes demand, kept count.
__global__ void __launch_bounds__(256)
send_scan_kernel(const int32_t* __restrict__ chunk_count, int nch, int R, int cap, int32_t* __restrict__ chunk_base,
                 int32_t* __restrict__ ctr, int32_t* __restrict__ send_count_out) {
  const int d = blockIdx.x;
  const int total = column_scan(chunk_count + (int64_t)d * nch, chunk_base + (int64_t)d * nch, nch);
#ifdef MOE_DEBUG
  if (d == 0 && threadIdx.x == 0) ctr[Ctr::DBG_SEND] = ctr[Ctr::DBG_COMBINE] = 0;
#endif
  if (threadIdx.x == 0) {
    if (d < R) {
      const int kept = min(total, cap);
      ctr[Ctr::HEADER + d] = total;
      ctr[Ctr::HEADER + R + d] = kept;
      send_count_out[d] = kept;
    } else {
      ctr[Ctr::SEND_INVALID] = total;
    }
  }
}

hipError_t launch_send_scan(const int32_t* chunk_count, int nch, int R, int cap, int32_t* chunk_base, int32_t* ctr,
                            int32_t* send_count_out, hipStream_t st) {
  // nch == 0 (no tokens) still runs: every column total is 0
  launch(send_scan_kernel, dim3(R + 1), dim3(256), 0, st, chunk_count, nch, R, cap, chunk_base, ctr,
                     send_count_out);
  return hipGetLastError();
}

// Ragged layout: destination d's rows start at send_off[d], the exclusive
// scan of the kept counts; send_off[R] is the total.
__global__ void __launch_bounds__(256)
ragged_offsets_kernel(const int32_t* __restrict__ send_count, int R, int32_t* __restrict__ send_off) {
  const int total = column_scan(send_count, send_off, R);
  if (threadIdx.x == 0) send_off[R] = total;
}

hipError_t launch_ragged_offsets(const int32_t* send_count, int R, int32_t* send_off, hipStream_t st) {
  launch(ragged_offsets_kernel, dim3(1), dim3(256), 0, st, send_count, R, send_off);
  return hipGetLastError();
}

// One block per token: work out the k slots, then copy the latent row once
// from HBM into every kept destination row (16 bytes per lane, coalesced).
// Blocks past T mark the empty slots of every pool with id -1.  With
// ragged_off set, the pools are laid end to end with no empty slots: the
// r-th row kept for destination d is row ragged_off[d] + r.
// The id is written together with the rest of the row's last 128-byte line
// (zeros up to prow): a lone 4-byte store would leave that line partly
// written, which costs the memory system a read-modify-write (the pack of a
// 65,536-token batch ran 13 % slower that way).
constexpr int PACK_TPB = 384;  // one 16-byte chunk per lane of a 6 KB bf16 latent row

__global__ void __launch_bounds__(PACK_TPB)
pack_kernel(const char* __restrict__ z, int64_t row_bytes, const int32_t* __restrict__ idx,
            const int32_t* __restrict__ local_rank, const int32_t* __restrict__ chunk_base, int nch, int T, int k,
            int X, int E, int R, int cap, char* __restrict__ pools, int64_t dst_stride, int64_t prow,
            int32_t* __restrict__ slot_of, const int32_t* __restrict__ send_count,
            const int32_t* __restrict__ ragged_off, int32_t* __restrict__ ctr) {
  const int t = blockIdx.x;
  const int tail = (int)((prow - row_bytes) >> 4);  // 16-byte chunks from the id to the end of the row
  if (t >= T) {
    // empty-slot ids: slots [send_count[d], cap) of every pool d, one tail chunk per lane
    const int64_t i = (int64_t)(t - T) * PACK_TPB + threadIdx.x;
    const int64_t row = i / tail;
    if (row < (int64_t)R * cap) {
      const int c = (int)(i - row * tail);
      const int d = (int)(row / cap), s = (int)(row - (int64_t)d * cap);
      if (s >= send_count[d])
        ((uint4*)(pools + d * dst_stride + s * prow + row_bytes))[c] = make_uint4(c == 0 ? ~0u : 0u, 0u, 0u, 0u);
    }
    return;
  }
  __shared__ int64_t off[32];
  __shared__ int32_t ids[32];
  if (threadIdx.x < k) {
    const int64_t a = (int64_t)t * k + threadIdx.x;
    const int e = idx[a];
    int64_t o = -1;
    int slot = -1;
    if (e >= 0 && e < E) {
      const int d = e / X;
      const int r = chunk_base[(int64_t)d * nch + (int)(a / SCAN_CHUNK)] + local_rank[a];
      MOE_DEBUG_FLAG(ctr, Ctr::DBG_SEND, r < 0);
      if (r < 0) {
        // unreachable: a rank is a count of earlier assignments
      } else if (ragged_off) {
        slot = ragged_off[d] + r;
        o = (int64_t)slot * prow;
      } else if (r < cap) {
        slot = d * cap + r;
        o = d * dst_stride + (int64_t)r * prow;
      }
    }
    slot_of[a] = slot;
    off[threadIdx.x] = o;
    ids[threadIdx.x] = e;
  }
  __syncthreads();
  const uint4* src = (const uint4*)(z + (int64_t)t * row_bytes);
  const int nchunk = (int)(row_bytes >> 4);
  for (int c = threadIdx.x; c < nchunk; c += PACK_TPB) {
    const uint4 v = src[c];
    for (int i = 0; i < k; ++i)
      if (off[i] >= 0) ((uint4*)(pools + off[i]))[c] = v;
  }
  for (int q = threadIdx.x; q < k * tail; q += PACK_TPB) {
    const int i = q / tail, c = q - i * tail;
    if (off[i] >= 0)
      ((uint4*)(pools + off[i] + row_bytes))[c] = make_uint4(c == 0 ? (uint32_t)ids[i] : 0u, 0u, 0u, 0u);
  }
}

hipError_t launch_pack(const void* z, int64_t row_bytes, const int32_t* idx, const int32_t* local_rank,
                       const int32_t* chunk_base, int T, int k, int X, int E, int R, int cap, void* pools,
                       int64_t dst_stride, int64_t prow, int32_t* slot_of, const int32_t* send_count,
                       const int32_t* ragged_off, int32_t* ctr, hipStream_t st) {
  const int nch = (T * k + SCAN_CHUNK - 1) / SCAN_CHUNK;
  const int64_t tail = (prow - row_bytes) >> 4;
  const int64_t fill_blocks = ragged_off ? 0 : ((int64_t)R * cap * tail + PACK_TPB - 1) / PACK_TPB;
  const int64_t blocks = (int64_t)T + fill_blocks;
  if (blocks == 0) return hipSuccess;
  launch(pack_kernel, dim3((unsigned)blocks), dim3(PACK_TPB), 0, st, (const char*)z, row_bytes, idx,
                     local_rank, chunk_base, nch, T, k, X, E, R, cap, (char*)pools, dst_stride, prow, slot_of,
                     send_count, ragged_off, ctr);
  return hipGetLastError();
}

// ---------------------------------------------------------------- receive

__global__ void __launch_bounds__(256)
recv_rank_kernel(const char* __restrict__ pools, int64_t src_stride, int64_t prow, int64_t id_off, int n_rows,
                 int cap, int X, int my_rank, int32_t* __restrict__ row_j, int32_t* __restrict__ row_lrank,
                 int32_t* __restrict__ chunk_count, int nch) {
  extern __shared__ int32_t run_all[];
  auto key = [&](int row) {
    const int s = row / cap, sl = row - s * cap;
    const int e = *(const int32_t*)(pools + s * src_stride + (int64_t)sl * prow + id_off);
    if (e < 0) return -1;
    const int j = e - X * my_rank;
    return (j >= 0 && j < X) ? j : X;  // X: id of another rank's expert
  };
  chunk_rank(key, n_rows, X + 1, nch, run_all, row_lrank, chunk_count, row_j);
}

hipError_t launch_recv_rank(const void* pools, int64_t src_stride, int64_t prow, int64_t id_off, int R, int cap,
                            int X, int my_rank, int32_t* row_j, int32_t* row_lrank, int32_t* chunk_count,
                            hipStream_t st) {
  const int n_rows = R * cap;
  const int nch = (n_rows + SCAN_CHUNK - 1) / SCAN_CHUNK;
  if (nch == 0) return hipSuccess;
  launch(recv_rank_kernel, dim3(nch), dim3(256), 4 * (X + 1) * sizeof(int32_t), st,
                     (const char*)pools, src_stride, prow, id_off, n_rows, cap, X, my_rank, row_j, row_lrank,
                     chunk_count, nch);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256)
recv_scan_kernel(const int32_t* __restrict__ chunk_count, int nch, int X, int rcap, int32_t* __restrict__ chunk_base,
                 int32_t* __restrict__ arrivals, int32_t* __restrict__ kept, int32_t* __restrict__ ctr) {
  const int j = blockIdx.x;
  const int total = column_scan(chunk_count + (int64_t)j * nch, chunk_base + (int64_t)j * nch, nch);
  if (threadIdx.x == 0) {
    if (j < X) {
      arrivals[j] = total;
      kept[j] = min(total, rcap);
    } else {
      ctr[Ctr::RECV_BAD] = total;
      ctr[Ctr::WAVE_OVER] = 0;
#ifdef MOE_DEBUG
      ctr[Ctr::DBG_RECV] = 0;
#endif
    }
  }
}

hipError_t launch_recv_scan(const int32_t* chunk_count, int nch, int X, int rcap, int32_t* chunk_base,
                            int32_t* arrivals, int32_t* kept, int32_t* ctr, hipStream_t st) {
  launch(recv_scan_kernel, dim3(X + 1), dim3(256), 0, st, chunk_count, nch, X, rcap, chunk_base, arrivals,
                     kept, ctr);
  return hipGetLastError();
}

// Final rank of every receive row within its local expert (-1: not one of
// this rank's experts, or an empty slot).
__global__ void __launch_bounds__(256)
recv_final_kernel(const int32_t* __restrict__ row_j, const int32_t* __restrict__ row_lrank,
                  const int32_t* __restrict__ chunk_base, int nch, int n_rows, int X,
                  int32_t* __restrict__ row_rank) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_rows) return;
  const int j = row_j[i];
  row_rank[i] = (j >= 0 && j < X) ? chunk_base[(int64_t)j * nch + i / SCAN_CHUNK] + row_lrank[i] : -1;
}

hipError_t launch_recv_final(const int32_t* row_j, const int32_t* row_lrank, const int32_t* chunk_base, int n_rows,
                             int X, int32_t* row_rank, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const int nch = (n_rows + SCAN_CHUNK - 1) / SCAN_CHUNK;
  launch(recv_final_kernel, dim3((n_rows + 255) / 256), dim3(256), 0, st, row_j, row_lrank, chunk_base,
                     nch, n_rows, X, row_rank);
  return hipGetLastError();
}

// One wave: thread i (a) writes the row_src entry of receive row i if an
// expert of the wave keeps it, (b) sets row_src slot i of the wave to -1 if it
// lies past that expert's count; threads 0..nj-1 also write wave_count.
// Reads only what moe_recv_rank left, so waves may run side by side.
__global__ void __launch_bounds__(256)
recv_place_kernel(const int32_t* __restrict__ row_j, const int32_t* __restrict__ row_rank,
                  const int32_t* __restrict__ kept, int n_rows, int rcap, int j0, int nj, int64_t wave_rows,
                  int32_t* __restrict__ wave_count, int32_t* __restrict__ row_src, int32_t* __restrict__ ctr) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0 && wave_rows > 0) {  // the wave's kept rows must fit its hidden-row bank
    int64_t n = 0;
    for (int j = 0; j < nj; ++j) n += kept[j0 + j];
    if (n > wave_rows) ctr[Ctr::WAVE_OVER] = 1;
  }
  if (i < n_rows) {
    const int j = row_j[i], rank = row_rank[i];
    if (j >= j0 && j < j0 + nj && rank >= 0 && rank < rcap) {
      // a kept row's rank lies below its expert's kept count
      MOE_DEBUG_FLAG(ctr, Ctr::DBG_RECV, rank >= kept[j]);
      row_src[(int64_t)(j - j0) * rcap + rank] = i;
    }
  }
  if (i < nj * rcap) {
    const int jw = i / rcap, r = i - jw * rcap;
    if (r >= kept[j0 + jw]) row_src[i] = -1;
  }
  if (i < nj) wave_count[i] = kept[j0 + i];
}

hipError_t launch_recv_place(const int32_t* row_j, const int32_t* row_rank, const int32_t* kept, int n_rows,
                             int rcap, int j0, int nj, int64_t wave_rows, int32_t* wave_count, int32_t* row_src,
                             int32_t* ctr, hipStream_t st) {
  const int n = max(max(n_rows, nj * rcap), nj);
  if (n == 0) return hipSuccess;
  launch(recv_place_kernel, dim3((n + 255) / 256), dim3(256), 0, st, row_j, row_rank, kept, n_rows, rcap,
                     j0, nj, wave_rows, wave_count, row_src, ctr);
  return hipGetLastError();
}

// One wave per wave-buffer row: copy the kept pool row (payload only).
__global__ void __launch_bounds__(256)
wave_gather_kernel(const char* __restrict__ pools, int64_t src_stride, int64_t prow, int cap, int64_t row_bytes,
                   const int32_t* __restrict__ row_src, const int32_t* __restrict__ wave_count, int nj, int rcap,
                   char* __restrict__ wave_buf) {
  const int64_t r_all = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r_all >= (int64_t)nj * rcap) return;
  const int jw = (int)(r_all / rcap), r = (int)(r_all - (int64_t)jw * rcap);
  if (r >= wave_count[jw]) return;
  const int rs = row_src[r_all];
  const int s = rs / cap, sl = rs - s * cap;
  const uint4* src = (const uint4*)(pools + s * src_stride + (int64_t)sl * prow);
  uint4* dst = (uint4*)(wave_buf + r_all * row_bytes);
  const int nchunk = (int)(row_bytes >> 4);
  for (int c = lane_id(); c < nchunk; c += 64) dst[c] = src[c];
}

hipError_t launch_wave_gather(const void* pools, int64_t src_stride, int64_t prow, int cap, int64_t row_bytes,
                              const int32_t* row_src, const int32_t* wave_count, int nj, int rcap, void* wave_buf,
                              hipStream_t st) {
  const int64_t rows = (int64_t)nj * rcap;
  if (rows == 0) return hipSuccess;
  launch(wave_gather_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, (const char*)pools,
                     src_stride, prow, cap, row_bytes, row_src, wave_count, nj, rcap, (char*)wave_buf);
  return hipGetLastError();
}

// A receive row of this wave's experts that did not fit gets an all-zero
// return row.  One lane checks one row; the wave then zeroes its dropped rows
// together (none, usually: the launch costs a quarter of a wave per 64 rows).
__global__ void __launch_bounds__(256)
zero_dropped_kernel(const int32_t* __restrict__ row_j, const int32_t* __restrict__ row_rank, int n_rows, int cap,
                    int rcap, int j0, int nj, char* __restrict__ ret, int64_t ret_src_stride, int64_t row_bytes) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  bool drop = false;
  if (row < n_rows) {
    const int j = row_j[row];
    drop = j >= j0 && j < j0 + nj && row_rank[row] >= rcap;
  }
  uint64_t m = __ballot(drop);
  const int base = row - lane_id();
  const int nchunk = (int)(row_bytes >> 4);
  while (m) {
    const int r = base + __builtin_ctzll(m);
    m &= m - 1;
    const int s = r / cap, sl = r - s * cap;
    uint4* dst = (uint4*)(ret + s * ret_src_stride + (int64_t)sl * row_bytes);
    for (int c = lane_id(); c < nchunk; c += 64) dst[c] = make_uint4(0, 0, 0, 0);
  }
}

hipError_t launch_zero_dropped(const int32_t* row_j, const int32_t* row_rank, int n_rows, int cap, int rcap, int j0,
                               int nj, void* ret, int64_t ret_src_stride, int64_t row_bytes, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  launch(zero_dropped_kernel, dim3((n_rows + 255) / 256), dim3(256), 0, st, row_j, row_rank, n_rows, cap,
                     rcap, j0, nj, (char*)ret, ret_src_stride, row_bytes);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine

// The returned rows are read once and the combined rows are next read by an
// MFMA-bound GEMM: nontemporal loads and stores (measured 13 % and another
// 4 % faster than plain ones here, the same bytes) keep them out of the way
// of lines that are reused.
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));

template <class T> struct Vec8;
template <> struct Vec8<bf16_t> {
  __device__ static void load(const bf16_t* p, float* f) {
    const u32x4_nt u = __builtin_nontemporal_load((const u32x4_nt*)p);
    const uint32_t w[4] = {u[0], u[1], u[2], u[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static void store(bf16_t* p, const float* f) {
    u32x4_nt w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f32x2_to_bf16x2(f[2 * i], f[2 * i + 1]);
    __builtin_nontemporal_store(w, (u32x4_nt*)p);
  }
};
template <> struct Vec8<float> {
  __device__ static void load(const float* p, float* f) {
    const u32x4_nt a = __builtin_nontemporal_load((const u32x4_nt*)p);
    const u32x4_nt b = __builtin_nontemporal_load((const u32x4_nt*)(p + 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = __uint_as_float(a[i]);
      f[4 + i] = __uint_as_float(b[i]);
    }
  }
  __device__ static void store(float* p, const float* f) {
    u32x4_nt a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = __float_as_uint(f[i]);
      b[i] = __float_as_uint(f[4 + i]);
    }
    __builtin_nontemporal_store(a, (u32x4_nt*)p);
    __builtin_nontemporal_store(b, (u32x4_nt*)(p + 4));
  }
};

constexpr int COMBINE_TPB = 384;  // one 8-element chunk per lane of a 3072-wide latent row

// One block per token: c = act(sum_i w_i * returned row i), i ascending, fp32.
template <class T>
__global__ void __launch_bounds__(COMBINE_TPB)
combine_kernel(const char* __restrict__ ret, int64_t dst_stride, int64_t row_bytes, int cap, int R,
               const int32_t* __restrict__ slot_of, const float* __restrict__ w, int k, int L,
               T* __restrict__ c_out, int64_t ldc, int32_t* __restrict__ ctr) {
  const int t = blockIdx.x;
  __shared__ int64_t off[32];
  __shared__ float ww[32];
  if (threadIdx.x < k) {
    int s = slot_of[(int64_t)t * k + threadIdx.x];
#ifdef MOE_DEBUG
    // a slot outside the return pools: reported, and the assignment left out
    const bool bad = s < -1 || s >= R * cap;
    MOE_DEBUG_FLAG(ctr, Ctr::DBG_COMBINE, bad);
    if (bad) s = -1;
#endif
    int64_t o = -1;
    if (s >= 0) {
      const int d = s / cap, sl = s - d * cap;
      o = d * dst_stride + (int64_t)sl * row_bytes;
    }
    off[threadIdx.x] = o;
    ww[threadIdx.x] = w[(int64_t)t * k + threadIdx.x];
  }
  __syncthreads();
  // The rows are read 8 at a time with every load issued before the sums
  // (a missing row reads the first pool row and is then left out), so each
  // lane keeps 8 loads in flight; the sum order stays i ascending.
  for (int c = threadIdx.x; c < L / 8; c += COMBINE_TPB) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < k; i0 += 8) {
      float f[8][8];
      bool use[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        use[u] = i0 + u < k && off[i0 + u] >= 0;
        Vec8<T>::load((const T*)(ret + (use[u] ? off[i0 + u] : 0)) + c * 8, f[u]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = use[u] ? fmaf(ww[i0 + u], f[u][q], acc[q]) : acc[q];
    }
    Vec8<T>::store(c_out + (int64_t)t * ldc + c * 8, acc);
  }
}

hipError_t launch_combine(int act, const void* ret, int64_t dst_stride, int64_t row_bytes, int cap, int R,
                          const int32_t* slot_of, const float* w, int T, int k, int L, void* c_out, int64_t ldc,
                          int32_t* ctr, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (act == 0)
    launch(combine_kernel<bf16_t>, dim3(T), dim3(COMBINE_TPB), 0, st, (const char*)ret, dst_stride,
                       row_bytes, cap, R, slot_of, w, k, L, (bf16_t*)c_out, ldc, ctr);
  else
    launch(combine_kernel<float>, dim3(T), dim3(COMBINE_TPB), 0, st, (const char*)ret, dst_stride,
                       row_bytes, cap, R, slot_of, w, k, L, (float*)c_out, ldc, ctr);
  return hipGetLastError();
}

}  // namespace moe
