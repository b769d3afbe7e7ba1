/*
 * eagle3_attn.h -- C ABI of the MI355X (gfx950) EAGLE-3 mixed-attention library
 * (libeagle3_attn.so).
 *
 * EAGLE-3 mixed attention (NeMo AutoModel API pages: speculative.eagle.ring_attention,
 * class `_CachedRingAttention`; speculative.eagle.ulysses_attention, class
 * `_CachedUlyssesAttention`; speculative.eagle.zigzag_ring_attention, module text):
 * every query row t holds ONE softmax over
 *   - block 0: the step-0 sequence keys k0_s in the same document with position
 *     s <= pos(t) (causal, self included), score scale*<q_t, k0_s>, value v0_s;
 *   - blocks i = 1..N (N = num_blocks-1, the test-time-training steps): one key per
 *     row at the same position, score scale*<q_t, kd_{i,t}>, value vd_{i,t}.
 * The blocks are joined by the online-softmax log-sum-exp merge (ring_attention page,
 * `_update_out_and_lse`, `_merge_diag`). The backward runs against the MERGED out/lse
 * (ring_attention page, `_CachedRingAttention`; zigzag_ring_attention page,
 * `zigzag_ring_flash_attn_varlen_backward`) and adds the diagonal gradients in closed
 * form.
 *
 * Conventions
 *   - Tensors use the FlashAttention layout of the pages, row-major:
 *       q, dout, out, dq         [B, T, H, D]
 *       k0, v0, dk0, dv0         [B, T_kv, H, D]  block 0, the full sequence in global order
 *       kd, vd, dkd, dvd         [B, N, T, H, D]  blocks 1..N for the local rows
 *       lse                      [B, H, T] float32, contiguous, natural log
 *     Batch and block strides of the k/v tensors may be given (0 = dense), so a cache laid
 *     out [B, num_blocks, T, H, D] is passed as k0 = cache, kd = cache + T*H*D with
 *     k0_batch_stride = kd_batch_stride = num_blocks*T*H*D and kd_block_stride = T*H*D.
 *     Gradients of k/v use the same strides as the tensors they differentiate.
 *   - Element type (E3_BF16 or E3_F32) is one for all of q, k*, v*, dout, out and the
 *     gradients. out is returned in q's dtype (ulysses_attention page,
 *     `cached_ulysses_attention`); all merging is done in float32.
 *   - Every pointer passed to a compute entry point is a DEVICE pointer unless named
 *     *_host. The caller owns (allocates and frees) every buffer, including the
 *     backward's workspace. The library allocates no device memory and keeps no
 *     per-call state.
 *   - Calls are asynchronous on the given HIP stream and never synchronise. The backward
 *     forks part of its work (the diagonal-block gradients) onto a side stream that
 *     waits for the given stream and is joined back into it before the call's last
 *     kernel, so the result is ordered on the given stream as if all ran there. The side
 *     stream and its two events are created on first use, one set per host thread and
 *     device, and kept until the process ends.
 *   - Every output is overwritten; rows of dk0/dv0 that no local query sees are written
 *     as zeros.
 *   - Errors: arguments are validated before anything is launched. On failure a negative
 *     e3_status is returned, nothing is launched and eagle3_last_error() (thread-local)
 *     describes the problem. A failed launch returns E3_EHIP.
 *
 * Layouts of a share (one GPU's part of a context-parallel run):
 *   E3_LAYOUT_FULL       the whole sequence: T_kv == T, positions 0..T-1.
 *   E3_LAYOUT_CONTIGUOUS contiguous ring shard (ring_attention page, module text and
 *                        `ring_flash_attn_forward`): rank r holds positions
 *                        [r*T, (r+1)*T) of S = cp*T; T_kv == S.
 *   E3_LAYOUT_ZIGZAG     zig-zag ring shard (zigzag_ring_attention page, module text):
 *                        S = cp*T is cut into 2*cp chunks of c = T/2; rank r holds chunk r
 *                        then chunk 2*cp-1-r; T_kv == S; B must be 1.
 *   E3_LAYOUT_HEADSHARD  Ulysses head shard (ulysses_attention page, module text): the full
 *                        sequence for H local heads; T_kv == T; cp is the Ulysses degree and
 *                        T must divide by it (`_scatter_seq_gather_heads`).
 *   k0/v0 always hold the FULL sequence in global order. Block-0 K/V segments are visited
 *   in ring order: at ring step j the share attends the K/V of rank (rank-j) mod cp
 *   (zigzag_ring_attention page, `RingComm`); the order changes rounding only.
 *
 * Documents: cu_seqlens are GLOBAL document boundaries [num_docs+1] int32 starting at 0
 * and ending at the full sequence length (ulysses_attention page, `cached_ulysses_attention`).
 * num_docs == 0 or 1 means one document. Several documents require B == 1 (varlen tensors
 * are unbatched: zigzag_ring_attention page, `squeeze_batch`) and are not supported with
 * the zig-zag layout (per-document zig-zag halving is not implemented: E3_EUNSUPPORTED).
 */
#ifndef EAGLE3_ATTN_H
#define EAGLE3_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EAGLE3_ABI_VERSION 3

typedef enum { E3_OK = 0, E3_EINVAL = -1, E3_EUNSUPPORTED = -2, E3_EHIP = -3 } e3_status;
typedef enum { E3_BF16 = 0, E3_F32 = 1 } e3_dtype;
typedef enum {
  E3_LAYOUT_FULL = 0,
  E3_LAYOUT_CONTIGUOUS = 1,
  E3_LAYOUT_ZIGZAG = 2,
  E3_LAYOUT_HEADSHARD = 3
} e3_layout;

typedef struct e3_problem {
  int32_t dtype;            /* e3_dtype */
  int32_t B;                /* batch, >= 1 */
  int32_t T;                /* local query rows, >= 0 (0 = nothing to do) */
  int32_t T_kv;             /* block-0 key rows (the full sequence length S) */
  int32_t H;                /* heads held by this share, >= 1 */
  int32_t D;                /* head dim: 64 or 128 */
  int32_t num_blocks;       /* 1 + N; 1..16 */
  float scale;              /* softmax scale, e.g. D^-0.5; finite and > 0 */
  int32_t layout;           /* e3_layout */
  int32_t cp;               /* ring size / Ulysses degree (1 for FULL) */
  int32_t rank;             /* 0 <= rank < cp (0 for FULL and HEADSHARD) */
  int32_t num_docs;         /* 0 = one document */
  const int32_t* cu_seqlens_host; /* HOST pointer, [num_docs+1], validated */
  const int32_t* cu_seqlens_dev;  /* DEVICE copy of the same values (read by the kernels) */
  int64_t k0_batch_stride;  /* elements between batch rows of k0/v0/dk0/dv0; 0 = T_kv*H*D */
  int64_t kd_batch_stride;  /* elements between batch rows of kd/vd/dkd/dvd; 0 = N*T*H*D */
  int64_t kd_block_stride;  /* elements between blocks of kd/vd/dkd/dvd; 0 = T*H*D */
} e3_problem;

/* Version of this header's ABI (EAGLE3_ABI_VERSION). Bindings refuse a mismatch rather
 * than bind arguments to the wrong slots (the same rule the ring_attention page's
 * `require_flash_attn_version` applies to the kernels it calls). */
int eagle3_abi_version(void);

/* Message for the last nonzero status returned on this thread ("" if none). */
const char* eagle3_last_error(void);

/* Bytes of device workspace eagle3_attn_bwd / eagle3_shard_bwd need: delta = rowsum(dO*O)
 * and lse*log2(e) (float32 [B, H, P], P = T with each local run, i.e. each of the two
 * zig-zag chunks, padded to a multiple of 64 positions), then, when num_blocks > 1, the
 * block-0 part of dq (float32 [B, T, H, D]). 0 when T == 0. Returns 0 and sets the last
 * error for an invalid problem. */
size_t eagle3_bwd_workspace_bytes(const e3_problem* p);

/* Forward of the full sequence (layout FULL or HEADSHARD):
 *   out [B,T,H,D] (dtype) = the joint-softmax output, lse [B,H,T] float32 = the merged
 *   log-sum-exp. kd/vd may be NULL when num_blocks == 1. No workspace. */
int eagle3_attn_fwd(const e3_problem* p, const void* q, const void* k0, const void* v0,
                    const void* kd, const void* vd, void* out, float* lse, hipStream_t stream);

/* Backward of the full sequence (layout FULL or HEADSHARD) against the MERGED out/lse
 * produced by the forward: writes dq [B,T,H,D], dk0/dv0 [B,T_kv,H,D], dkd/dvd
 * [B,N,T,H,D] (dtype; dkd/dvd may be NULL when num_blocks == 1). workspace must hold
 * eagle3_bwd_workspace_bytes(p) bytes, 256-byte aligned. */
int eagle3_attn_bwd(const e3_problem* p, const void* dout, const void* q, const void* k0,
                    const void* v0, const void* kd, const void* vd, const void* out,
                    const float* lse, void* workspace, void* dq, void* dk0, void* dv0,
                    void* dkd, void* dvd, hipStream_t stream);

/* Shard driver: the same computation for any layout (CONTIGUOUS, ZIGZAG, HEADSHARD,
 * FULL). The share's block-0 attention visits the K/V segments in ring order and merges
 * them with the diagonals in one pass, with no inter-GPU communication. Arguments as
 * eagle3_attn_fwd / eagle3_attn_bwd. */
int eagle3_shard_fwd(const e3_problem* p, const void* q, const void* k0, const void* v0,
                     const void* kd, const void* vd, void* out, float* lse, hipStream_t stream);
int eagle3_shard_bwd(const e3_problem* p, const void* dout, const void* q, const void* k0,
                     const void* v0, const void* kd, const void* vd, const void* out,
                     const float* lse, void* workspace, void* dq, void* dk0, void* dv0,
                     void* dkd, void* dvd, hipStream_t stream);

/* In-place online-softmax merge of one attention block into a running state
 * (ring_attention page, `_update_out_and_lse`; zigzag_ring_attention page,
 * `update_out_and_lse`), all float32:
 *   out   [B,T,H,D]  running output, updated in place
 *   lse   [B,H,T]    running log-sum-exp, updated in place
 *   block_out [B,T,H,D]
 *   block_lse [B,H,T] if block_lse_layout == 0, or [B,T,H] if 1 (the page's running lse
 *             is [B,S,H,1] while a kernel returns [B,H,S]; either may be given)
 *   out' = out - sigmoid(block_lse - lse) * (out - block_out)
 *   lse' = lse - log(sigmoid(lse - block_lse))
 * A block row with block_lse = -inf leaves the row unchanged; a state row with
 * lse = -inf takes the block row. The sigmoid weight that the zig-zag page also returns
 * is not produced (the merged-lse backward does not use it). */
int lse_merge(float* out, float* lse, const float* block_out, const float* block_lse,
              int B, int T, int H, int D, int block_lse_layout, hipStream_t stream);

/* ---- Measurement hook ---------------------------------------------------------------- */

/* While `events` is non-NULL, every compute entry point called on this thread records
 * events[0] on its stream before its first kernel and events[k+1] after its k-th stage
 * (at most `capacity` events; the forward has 1 stage, the attention kernel; the
 * backward 3: dQ (which also writes delta and lse*log2(e)), dK/dV, and the wait for the
 * side stream's diagonal-block gradients). The caller creates and owns the events; NULL stops
 * recording. Returns E3_OK. */
int eagle3_set_timing_events(hipEvent_t* events, int capacity);

/* Number of events recorded by the last compute entry point called on this thread. */
int eagle3_timing_events_recorded(void);

/* ---- Host-only inspection of the shard driver (no GPU needed) ---------------------- */

/* Global sequence position of every local query row: pos_host[T] (HOST memory). */
int eagle3_query_positions(const e3_problem* p, int64_t* pos_host);

/* Attended block-0 (query, key) pairs of the share, per batch row and head. */
int64_t eagle3_pair_count(const e3_problem* p);

/* Number of forward query tiles per (batch row, head) and the tile height. */
int eagle3_fwd_tiles(const e3_problem* p, int32_t* tile_rows);

/* Query tile `tile` (0-based, launch order) of the forward: writes its local row range
 * to rows_host[2] = {first, end} and the block-0 keys each key tile it visits may count,
 * in visiting order, to seg_host[3*k] = {key_begin, key_end, needs_mask} for
 * k < max_segments (the tile's keys clipped to its ring segment). Returns the number of
 * key tiles (may exceed max_segments) or a negative e3_status. */
int eagle3_fwd_tile_segments(const e3_problem* p, int tile, int32_t* rows_host,
                             int32_t* seg_host, int max_segments);

#ifdef __cplusplus
}
#endif

#endif /* EAGLE3_ATTN_H */
