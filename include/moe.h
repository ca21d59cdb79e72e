/*
 * moe.h -- C ABI of the fixed-pool, three-wave MoE expert layer (one EP rank).
 *
 * The layer follows the Marin 535B-A23B expert-parallel design described in
 * "Marin 开始公开训练 535B 参数 MoE 模型" (lamjinlab blog), section 二
 * "稀疏模型如何组织": a router picks 8 of 384 routed experts per token, a
 * latent projection shrinks the routed activations from 6,144 to 3,072 values
 * before they cross GPUs, every sender keeps ONE fixed pool per destination
 * GPU (not one buffer per expert) with the expert id packed into each payload
 * row, the transfer runs in three consecutive waves of identical array shape,
 * a send capacity factor (1.10) caps source-to-destination traffic and a
 * receive capacity factor (1.15) caps the rows of one local expert, and
 * anything over either cap is dropped and counted separately.  The routed
 * output is projected back to model width and merged with 2 always-on shared
 * experts.
 *
 * Conventions (all entry points):
 *   - Every data pointer is a DEVICE pointer owned by the caller.  Activation,
 *     weight, pool, workspace, logit and bias buffers are 16-byte aligned;
 *     int32 / fp32 index, routing-weight and count arrays 4-byte aligned.  A buffer of zero
 *     elements may be NULL.  The library never allocates or frees caller
 *     memory.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and is asynchronous, except moe_capacity / moe_workspace_size (host
 *     only) and moe_drop_stats (synchronises `stream`).
 *   - `ws` is a caller-allocated device workspace of moe_workspace_size()
 *     bytes.  It carries counters, scan partials and GEMM partial tiles
 *     between the calls of one layer.  Calls that share a workspace run in
 *     order on one stream, except: moe_shared_experts touches only its own
 *     region and may run beside the routed calls, and after moe_recv_rank the
 *     calls of waves in different scratch blocks (dims.live_waves) may run
 *     side by side.  Layers with their own workspaces and buffers may be
 *     driven from different host threads and streams at the same time.
 *   - Activations and weights are bf16 (act_dtype 0) or fp32 (act_dtype 1);
 *     accumulation is fp32; logits and routing weights are fp32.
 *   - Return 0 (MOE_OK) or a negative MOE_E* code; moe_last_error() returns a
 *     thread-local message for the last failure.  No exception crosses the
 *     ABI.  Identical inputs give bit-identical outputs (no atomics).
 *   - bf16 layers need d_model, latent, expert_hidden and shared_hidden to be
 *     multiples of 64 and n_experts a multiple of 4; fp32 layers need latent
 *     a multiple of 8 and shared_hidden a multiple of 4.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1, /* null pointer, bad dims or bad wave index */
  MOE_EALIGN = -2, /* pointer misaligned, or stride not a multiple of 16 / too small */
  MOE_EDTYPE = -3, /* act_dtype not MOE_ACT_BF16 / MOE_ACT_F32 */
  MOE_ECAP = -4,   /* a counter exceeds its fixed capacity (report overflow) */
  MOE_EHIP = -5    /* a HIP call failed; the message holds hipGetErrorString */
};

enum { MOE_ACT_BF16 = 0, MOE_ACT_F32 = 1 };

#define MOE_MAX_RANKS 1024
#define MOE_MAX_LOCAL 64

/* Shape of one EP layer.  Symbols: T tokens per rank, D model width, L latent
 * width, E routed experts, k experts per token, R ranks in the EP domain,
 * X = E / R local experts per rank, W waves (X / W experts per wave), H routed
 * expert hidden width, S shared experts, HS shared hidden width.  Capacity
 * factors are rationals: send = send_num / send_den (1.10 = 110/100), receive
 * = recv_num / recv_den (1.15 = 115/100).
 *
 * Accepted dims (every entry point returns MOE_EINVAL otherwise, MOE_EDTYPE
 * for an unknown act_dtype): T >= 0, S >= 0, every other size positive;
 * E a multiple of R with X <= MOE_MAX_LOCAL and X a multiple of W;
 * R <= MOE_MAX_RANKS; k <= min(32, E); E <= 2048; 0 <= my_rank < R; positive
 * capacity factors; D, L, H, HS <= 2^24 and L + S * HS < 2^24; bf16: D, L, H,
 * HS multiples of 64 and E a multiple of 4; fp32: L a multiple of 8 and HS of
 * 4; T * k, R * send_cap and X/W * recv_cap at most 2^30, T * E at most 2^31,
 * and each GEMM at most 2^30 output tiles of 256 x 256. */
typedef struct moe_dims {
  int32_t tokens, d_model, latent, n_experts, top_k, n_ranks, waves;
  int32_t expert_hidden, shared_experts, shared_hidden;
  int32_t my_rank;   /* the rank whose experts moe_recv_waves / moe_expert_gemm serve */
  int32_t act_dtype; /* MOE_ACT_BF16 or MOE_ACT_F32 */
  int32_t send_num, send_den, recv_num, recv_den;
  /* Waves whose scratch (SwiGLU hidden rows, GEMM partial tiles) the
   * workspace holds at once, 1..W; 0 means W.  Wave w uses block w mod
   * live_waves, so calls of two waves in one block must not overlap (run
   * them in order on one stream).  1 keeps one wave's hidden rows live at a
   * time (section 二: the waves exist so that only part of the receive bank
   * is live); W lets every wave run beside the others. */
  int32_t live_waves;
  /* Hidden-row bank of a wave.  0: every local expert of the wave has its own
   * block of recv_cap hidden rows (X/W * recv_cap rows per wave).  > 0: the
   * hidden rows of the wave's experts are laid end to end (an expert's rows
   * start after the kept rows of the wave's experts before it) in a bank of
   * wave_rows rows; the caller guarantees that the kept rows of every wave
   * fit, as a dropless exchange can from the counts it has exchanged
   * ([P1] section 四: capacity costs memory).  A wave whose kept rows do not
   * fit is reported by moe_drop_stats (MOE_ECAP); its rows past the bank are
   * then not computed correctly (nothing is written outside the bank). */
  int32_t wave_rows;
} moe_dims;

/* Drop ledger of one layer call on one rank; send side (this rank's tokens)
 * and receive side (rows that reached this rank's experts) apart.  Receive
 * fields reflect the latest moe_recv_waves call of each wave. */
typedef struct moe_drop_report {
  int64_t send_assignments; /* T * k */
  int64_t send_kept, send_dropped;
  int64_t recv_arrivals, recv_kept, recv_dropped;
  int64_t recv_bad_ids; /* rows whose id names an expert of another rank (ignored) */
  int32_t n_ranks, local_experts;
  int32_t send_demand[MOE_MAX_RANKS]; /* assignments per destination */
  int32_t send_count[MOE_MAX_RANKS];  /* kept rows per destination pool */
  int32_t expert_arrivals[MOE_MAX_LOCAL];
  int32_t expert_kept[MOE_MAX_LOCAL];
} moe_drop_report;

/* Capacities (host only).  send_cap = ceil(send_num*T*k / (send_den*R)) rows
 * per destination pool (section 二: factor 1.10 on source-to-destination
 * traffic); recv_cap = ceil(recv_num*R*T*k / (recv_den*E)) rows per local
 * expert (factor 1.15 on rows per local expert); exact integer arithmetic.
 * pool_stride_bytes = bytes per pool row: L activations, then the int32
 * global expert id, padded to a multiple of 128.  Any output may be NULL. */
int moe_capacity(const moe_dims* dims, int64_t* send_cap, int64_t* recv_cap,
                 int64_t* pool_stride_bytes);

/* Device workspace bytes needed by every call for these dims (host only). */
int moe_workspace_size(const moe_dims* dims, size_t* bytes);

/* Router and latent down-projection (section 二: 8 of 384 experts per token;
 * 6,144 -> 3,072 latent before the exchange).
 *   x        [T][D] act
 *   w_router [E][D] act;  w_down [L][D] act
 *   bias     NULL, or fp32 [nb][E]: row t / bias_row_tokens (bias_row_tokens
 *            > 0) or row 0 (bias_row_tokens == 0) is added to the logits
 *   logits   [T][E] fp32 output, or NULL (kept in ws)
 *   z        [T][L] act output: the latent rows that are exchanged
 *   topk_idx [T][k] int32 output: experts by descending logit, equal logits
 *            by lower expert index
 *   topk_w   [T][k] fp32 output: softmax over the k chosen logits */
int moe_route(const moe_dims* dims, const void* x, const void* w_router, const void* w_down,
              const float* bias, int32_t bias_row_tokens, float* logits, void* z,
              int32_t* topk_idx, float* topk_w, void* ws, void* stream);

/* Capacity-limited packing into the fixed per-destination send pools
 * (section 二: one fixed pool per destination GPU, expert id in the payload,
 * send capacity factor).  Assignment (t, i) goes to rank topk_idx[t][i] / X;
 * within a destination, assignments are ranked in (t, i) order and the first
 * send_cap keep their rank as slot.
 *   send_pools       R pools of send_cap rows of pool_stride_bytes each; pool d
 *                    starts at send_pools + d * dst_stride_bytes; row layout:
 *                    L act values, then the int32 global expert id (-1 for an
 *                    empty slot; an empty row's payload is left unwritten),
 *                    then zeros up to pool_stride_bytes
 *   slot_of          [T][k] int32 output: d * send_cap + slot, or -1 if dropped
 *   send_count       [R] int32 output: rows kept per destination */
int moe_pack_pools(const moe_dims* dims, const void* z, const int32_t* topk_idx,
                   void* send_pools, int64_t dst_stride_bytes, int32_t* slot_of,
                   int32_t* send_count, void* ws, void* stream);

/* Allocation-free variant of moe_pack_pools, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * moe_pack_pools, without `ws`: the counters, chunk ranks and chunk scans
 * live in a device array inside the library, MOE_NOALLOC_SCRATCH_BYTES
 * large, which every GPU the library runs on holds until the process ends.
 * Needs (16 + 2R + 2X) * 4 + 2 * (R + 1) * ceil(T*k / 1024) * 4 + T*k * 4
 * bytes of it (each part rounded up to 256): at least 1,048,576
 * assignments T*k for any R <= MOE_MAX_RANKS.  Larger inputs return
 * MOE_EINVAL before anything is launched.  Nothing is allocated or freed
 * and no allocating routine is called.  Every call on one GPU shares that
 * GPU's scratch, whose contents the next call overwrites (nothing in it needs
 * to start at zero): calls that overlap on one GPU (different streams or
 * host threads without ordering between them) race.  The drop counters stay
 * in the scratch; the kept rows per destination are send_count. */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
int moe_pack_pools_noalloc(const moe_dims* dims, const void* z, const int32_t* topk_idx,
                           void* send_pools, int64_t dst_stride_bytes, int32_t* slot_of,
                           int32_t* send_count, void* stream);

/* Ragged packing for the dropless comparison (section 四 of the same page:
 * the first fallback is a dropless all-to-all whose row counts travel ahead
 * of the rows, so pools can be ragged).  No send cap applies: every valid
 * assignment is kept.  Assignment (t, i) goes to rank topk_idx[t][i] / X and
 * is ranked in (t, i) order within its destination, as in moe_pack_pools;
 * the pools are laid end to end, destination by destination, with no empty
 * rows.  The send capacity factor in dims is not used.
 *   send_rows   [T*k][pool_stride_bytes]: the r-th row for destination d is
 *               row send_off[d] + r (L act values, then the int32 global
 *               expert id, then zeros up to pool_stride_bytes); rows past
 *               send_off[R] are left unwritten
 *   send_off    [R+1] int32 output: exclusive scan of send_count; send_off[R]
 *               is the number of rows written
 *   slot_of     [T][k] int32 output: send_off[d] + r (a row index), or -1 for
 *               an invalid expert id
 *   send_count  [R] int32 output: rows per destination (= its demand)
 * The rest of the layer takes this layout as R pools of send_cap rows laid
 * end to end: moe_combine with ret_dst_stride_bytes = send_cap * L *
 * sizeof(act) reads return row s at s * L * sizeof(act) for any s, so the
 * return rows can sit in this same ragged order (at least send_off[R] rows).
 * On the receive side, a buffer of the received segments laid end to end is
 * R pools of send_cap rows with src_stride_bytes = send_cap *
 * pool_stride_bytes, once send_cap * R covers the received rows and the
 * rows past them carry id -1. */
int moe_pack_ragged(const moe_dims* dims, const void* z, const int32_t* topk_idx,
                    void* send_rows, int32_t* send_off, int32_t* slot_of,
                    int32_t* send_count, void* ws, void* stream);

/* Receive side, ranking (section 二: receive capacity factor per local
 * expert).  Every row of every received pool is visited source by source,
 * slot by slot; a row with id e goes to local expert e - X*my_rank, and the
 * first recv_cap rows of each expert are kept.  The ranks, the per-expert
 * arrival and kept counts and the count of rows with an id of no expert of
 * this rank's domain stay in `ws` for moe_recv_waves, moe_expert_gemm and
 * moe_drop_stats.  Once per layer, after the pools have arrived.
 *   recv_pools      pool from source s at recv_pools + s * src_stride_bytes
 *                   (send_cap rows of pool_stride_bytes, as moe_pack_pools) */
int moe_recv_rank(const moe_dims* dims, const void* recv_pools, int64_t src_stride_bytes,
                  void* ws, void* stream);

/* Receive side, one wave (section 二: three waves of identical shape, so that
 * only part of the receive bank is live at a time).  Wave w serves local
 * experts w*X/W .. (w+1)*X/W-1 and reads only what moe_recv_rank left in
 * `ws`: after it has completed, the calls of different waves (this one and
 * moe_expert_gemm) may run side by side on different streams.
 *   recv_pools      as for moe_recv_rank; read only when wave_buf is set
 *   wave_buf        NULL, or [X/W][recv_cap][L] act output: kept rows of the
 *                   wave's experts in rank order (rows past the count unwritten)
 *   row_src         [X/W][recv_cap] int32 output: s * send_cap + slot per kept
 *                   row; -1 past the count
 *   wave_count      [X/W] int32 output: kept rows per expert of the wave */
int moe_recv_waves(const moe_dims* dims, const void* recv_pools, int64_t src_stride_bytes,
                   int32_t wave, void* wave_buf, int32_t* row_src, int32_t* wave_count,
                   void* ws, void* stream);

/* Expert FFNs of one wave and the rows they return (section 二; the experts
 * of the '535B并不意味着…' section of the huxiu page are reduced-width FFNs;
 * SwiGLU here).  For each expert j of the wave and each kept row r:
 * h = act(silu(a)*b) with a = row . W_gate^T, b = row . W_up^T, and
 * y = act(h . W2^T) is written to the return row of (src, slot).  A row
 * dropped at receive gets an all-zero return row.
 *   wave_buf        as written by moe_recv_waves, or NULL: then rows are read
 *                   straight from recv_pools (same pools and stride as the
 *                   moe_recv_waves call of this wave)
 *   w13             [X][2H][L] act: per local expert, H gate rows then H up rows
 *   w2              [X][L][H] act
 *   ret_pools       return row of (s, slot) at ret_pools + s * ret_src_stride_bytes
 *                   + slot * L * sizeof(act)
 * Wave w uses scratch block w mod live_waves of `ws` (dims.live_waves), so
 * waves in different blocks may overlap (see moe_recv_waves); waves of one
 * block, or sharing one wave_buf, must not. */
int moe_expert_gemm(const moe_dims* dims, int32_t wave, const void* wave_buf,
                    const void* recv_pools, int64_t src_stride_bytes, const int32_t* row_src,
                    const int32_t* wave_count, const void* w13, const void* w2,
                    void* ret_pools, int64_t ret_src_stride_bytes, void* ws, void* stream);

/* Shared experts (section 二: 2 always-on experts beside the routed ones;
 * section 四: they see every token).  For every token t and shared expert j,
 * h_s[t][j] = act(silu(x_t . Wg_j^T) * (x_t . Wu_j^T)), kept in `ws` for the
 * moe_combine call of the same batch.  It reads nothing the routed path
 * writes, so it may run on another stream, concurrently with moe_route ..
 * moe_expert_gemm of the same batch, provided it completes before that
 * batch's moe_combine starts and starts after the previous batch's
 * moe_combine on the same `ws` has completed.  With S == 0 it does nothing.
 *   x [T][D] act;  ws13 [S][2HS][D] act (HS gate rows then HS up rows) */
int moe_shared_experts(const moe_dims* dims, const void* x, const void* ws13, void* ws, void* stream);

/* Weighted combine and up-projection, merged with the shared experts
 * (section 二: the routed output is projected back to model width before
 * merging with the shared path; section 四: a dropped assignment
 * contributes nothing but the token is not lost).
 *   c_t  = act(sum_i topk_w[t][i] * ret(slot_of[t][i]))   (slot -1 adds 0)
 *   out  = act(c . U^T + sum_j h_s[t][j] . W2_j^T)
 * with h_s as left in `ws` by moe_shared_experts (required first when S > 0).
 *   ret_pools       row returned for slot d*send_cap+s at ret_pools +
 *                   d * ret_dst_stride_bytes + s * L * sizeof(act)
 *   w_up  [D][L] act;  ws2 [S][D][HS] act;  out [T][D] act output */
int moe_combine(const moe_dims* dims, const void* ret_pools, int64_t ret_dst_stride_bytes,
                const int32_t* slot_of, const float* topk_w, const void* w_up, const void* ws2,
                void* out, void* ws, void* stream);

/* Copy the drop ledger held in `ws` to host memory (section 二: drops are
 * reported separately for the send and the receive side).  Synchronises
 * `stream`.  Returns MOE_ECAP if recv_bad_ids is non-zero. */
int moe_drop_stats(const moe_dims* dims, const void* ws, moe_drop_report* report, void* stream);

/* Thread-local message of the last failed call ("" if none). */
const char* moe_last_error(void);

/* Per-kernel timing, a measurement aid for the layer above (not part of the
 * layer's arithmetic).  While enabled, every kernel launched by the calls
 * above carries two HIP events that its own dispatch records as the kernel
 * starts and ends (hipExtLaunchKernel), so the elapsed time between them is
 * that kernel's duration on its stream, with no marker packets between
 * kernels.  Results are unchanged.
 * Labels: route_gemm, select_topk, send_rank, send_scan, ragged_offsets, pack, recv_rank,
 * recv_scan, recv_final, recv_place, wave_gather, expert_gate_up, expert_down,
 * zero_dropped, combine, shared_gate_up, up_shared_down, and the tail-split
 * fixups route_fixup, gate_up_fixup, down_fixup, up_fixup. */
typedef struct moe_kernel_time {
  char name[32];    /* kernel label */
  int32_t launches; /* launches recorded since the last moe_timing_read */
  double total_ms;  /* their summed durations */
} moe_kernel_time;

/* Turn recording on (on != 0) or off for the whole process.  Never fails. */
int moe_timing_enable(int32_t on);

/* Wait for every recorded launch, write up to max_entries per-label totals to
 * out (labels in first-launch order), set *n_entries to the number of labels
 * recorded, and clear the record.  MOE_EINVAL for NULL or negative
 * arguments; MOE_EHIP if an event cannot be read. */
int moe_timing_read(moe_kernel_time* out, int32_t max_entries, int32_t* n_entries);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
