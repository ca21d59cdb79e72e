// Internal launchers of libmoe (host side).  Kernels live in kernels.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace moe {

// Assignments (send side) and pool rows (receive side) are ranked in chunks
// of SCAN_CHUNK by one 256-thread block each, then the chunk counts are
// scanned by one block.  No atomics anywhere: results are deterministic.
constexpr int SCAN_CHUNK = 1024;

// Workspace counter block (int32 words).
struct Ctr {
  static constexpr int SEND_DROPPED = 0;
  static constexpr int SEND_INVALID = 1;
  static constexpr int RECV_BAD = 2;
  static constexpr int WAVE_OVER = 3;  // a wave's kept rows exceed its hidden-row bank (dims.wave_rows)
  // Debug builds (-DMOE_DEBUG) only: invariant flags.  A kernel that finds a
  // violation stores 1 in its word (every writer stores the same value, so no
  // atomics) and carries on without the offending access; nothing traps.
  // The send scan clears DBG_SEND and DBG_COMBINE, the receive scan DBG_RECV.
  static constexpr int DBG_SEND = 4;     // pack: a row rank below zero (scan and ranks disagree)
  static constexpr int DBG_COMBINE = 5;  // combine: a slot_of entry outside [-1, R * send_cap)
  static constexpr int DBG_RECV = 6;     // receive: a kept row's rank at or past its expert's kept count
  static constexpr int HEADER = 16;
  // then: demand[R], send_count[R], arrivals[X], kept[X]
};

#ifdef MOE_DEBUG
#define MOE_DEBUG_FLAG(ctr, word, cond) \
  do {                                 \
    if (cond) (ctr)[word] = 1;         \
  } while (0)
#else
#define MOE_DEBUG_FLAG(ctr, word, cond) \
  do {                                 \
  } while (0)
#endif

// Kernel timing (moe_timing_enable): the host side of a timed launch sets a
// pair of events here, and the launch below hands them to the dispatch itself
// (hipExtLaunchKernel), which records them as the kernel starts and ends, so
// the pair brackets the kernel alone.  Thread-local; a launch consumes the pair.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();

template <class F, class... Args>
void launch(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t st, Args... args) {
  LaunchEvents& ev = launch_events();
  if (ev.start) {
    const LaunchEvents e = ev;
    ev = LaunchEvents{};
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, e.start, e.stop, 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
  }
}

hipError_t launch_select_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                              hipStream_t st);

hipError_t launch_send_rank(const int32_t* idx, int n_assign, int X, int E, int R, int32_t* local_rank,
                            int32_t* chunk_count, hipStream_t st);
hipError_t launch_send_scan(const int32_t* chunk_count, int nch, int R, int cap, int32_t* chunk_base,
                            int32_t* ctr, int32_t* send_count_out, hipStream_t st);
hipError_t launch_pack(const void* z, int64_t row_bytes, const int32_t* idx, const int32_t* local_rank,
                       const int32_t* chunk_base, int T, int k, int X, int E, int R, int cap, void* pools,
                       int64_t dst_stride, int64_t pool_row_stride, int32_t* slot_of, const int32_t* send_count,
                       const int32_t* ragged_off, int32_t* ctr, hipStream_t st);
hipError_t launch_ragged_offsets(const int32_t* send_count, int R, int32_t* send_off, hipStream_t st);

hipError_t launch_recv_rank(const void* pools, int64_t src_stride, int64_t pool_row_stride, int64_t id_off,
                            int R, int cap, int X, int my_rank, int32_t* row_j, int32_t* row_lrank,
                            int32_t* chunk_count, hipStream_t st);
hipError_t launch_recv_scan(const int32_t* chunk_count, int nch, int X, int rcap, int32_t* chunk_base,
                            int32_t* ctr_arrivals, int32_t* ctr_kept, int32_t* ctr, hipStream_t st);
hipError_t launch_recv_final(const int32_t* row_j, const int32_t* row_lrank, const int32_t* chunk_base, int n_rows,
                             int X, int32_t* row_rank, hipStream_t st);
hipError_t launch_recv_place(const int32_t* row_j, const int32_t* row_rank, const int32_t* ctr_kept, int n_rows,
                             int rcap, int j0, int nj, int64_t wave_rows, int32_t* wave_count, int32_t* row_src,
                             int32_t* ctr, hipStream_t st);
hipError_t launch_wave_gather(const void* pools, int64_t src_stride, int64_t pool_row_stride, int cap,
                              int64_t row_bytes, const int32_t* row_src, const int32_t* wave_count, int nj,
                              int rcap, void* wave_buf, hipStream_t st);
hipError_t launch_zero_dropped(const int32_t* row_j, const int32_t* row_rank, int n_rows, int cap, int rcap,
                               int j0, int nj, void* ret, int64_t ret_src_stride, int64_t row_bytes,
                               hipStream_t st);
hipError_t launch_combine(int act, const void* ret, int64_t dst_stride, int64_t row_bytes, int cap, int R,
                          const int32_t* slot_of, const float* w, int T, int k, int L, void* c_out,
                          int64_t ldc, int32_t* ctr, hipStream_t st);

}  // namespace moe
