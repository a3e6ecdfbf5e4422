/*
 * mla_decode.h -- C ABI of the paged MLA decode library (libmla_decode.so),
 * MI355X (gfx950).
 *
 * The operation (pages on FlashMLA):
 *   - "DeepSeek 开源记-第1天-FlashMLA", section 6 (使用方法): two calls,
 *       tile_scheduler_metadata, num_splits = get_mla_metadata(cache_seqlens,
 *           s_q * h_q // h_kv, h_kv)
 *       output, lse = flash_mla_with_kvcache(q, blocked_k, block_table,
 *           cache_seqlens, dv, tile_scheduler_metadata, num_splits, causal)
 *     section 2 (核心功能): head dim fixed at 576, value dim fixed at 512,
 *     Shared-KV (V is the first 512 dims of the cached 576-wide row);
 *     section 4 (核心实现): blockwise scores, softmax, merge of partial outputs.
 *   - "DeepSeek代碼開源第一彈Flash MLA" (ygpos news): BF16 and a paged KV cache
 *     with block size 64; variable-length sequences.
 *   - FlashMLA explainer (jsxs2.com), section 3.1: the work is cut into small
 *     blocks that run in parallel (the split-KV scheduler).
 *
 * For every sequence b, query token t < s_q and query head h < h_q, with
 * KV head g = h / (h_q / h_kv), N = cache_seqlens[b] and visible keys
 * j < L = N (or, when causal, L = min(N, N - s_q + t + 1)):
 *     K_j  = blocked_k[block_table[b][j / 64]][j % 64][g][0:576]
 *     s_j  = softmax_scale * dot(q[b][t][h][0:576], K_j)
 *     lse  = ln sum_j exp(s_j)
 *     out  = sum_j exp(s_j - lse) * K_j[0:512]
 * A row with no visible key gets out = 0 and lse = -inf.
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are device memory of the current HIP device;
 *     the caller allocates and owns every buffer, including metadata and
 *     workspace.  The library never allocates device memory and keeps no
 *     state between calls except a per-device property cache.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Compute calls
 *     only enqueue work: they never synchronize with the host and never read
 *     device memory from the host.
 *   - Every call returns MLA_OK (0) or a negative status; on failure
 *     nothing has been enqueued unless the status is MLA_ERR_HIP (a launch
 *     error reported by the runtime).  mla_last_error() gives a thread-local
 *     message for the last failure.
 *   - Preconditions only the device could check (they are not checked):
 *     block_table entries for blocks below ceil(N/64) are valid page indices
 *     in [0, num_pages); ceil(N/64) <= max_blocks_per_seq; the metadata was
 *     produced by mla_get_metadata for the same cache_seqlens, rows and h_kv.
 *     Cache rows at positions >= N and table entries >= ceil(N/64) are never
 *     used and may hold anything (NaN included).
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_OK 0
#define MLA_ERR_INVALID_ARG (-1) /* null pointer, bad size, misaligned buffer */
#define MLA_ERR_UNSUPPORTED (-2) /* d != 576, dv != 512, page size != 64, ... */
#define MLA_ERR_WORKSPACE (-3)   /* workspace smaller than mla_decode_workspace_size() */
#define MLA_ERR_HIP (-4)         /* a HIP runtime call or kernel launch failed */

#define MLA_HEAD_DIM 576
#define MLA_VALUE_DIM 512
#define MLA_PAGE_SIZE 64
/* Element type of q, blocked_k and out (one of the pages lists FP16 beside
 * BF16; the others BF16 only).  The arithmetic is the same: products of the
 * 16-bit inputs accumulated in fp32. */
#define MLA_DTYPE_BF16 0
#define MLA_DTYPE_FP16 1
#define MLA_METADATA_WORDS 8   /* int32 words per part in tile_metadata */
#define MLA_MAX_BATCH 16384
#define MLA_MAX_ROWS 4096      /* max s_q * h_q / h_kv */
#define MLA_MAX_PARTS 65536

/* Static text for a status code. */
const char *mla_status_string(int status);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char *mla_last_error(void);

/*
 * Host-only sizing for get_mla_metadata (section 6 of the cnblogs page: the
 * second argument is s_q * h_q // h_kv).  Reads the current device's compute
 * unit count (cached) and touches no device memory.
 *   q_rows_per_kv_head  M = s_q * h_q / h_kv, 1 <= M <= MLA_MAX_ROWS
 *   num_parts     out: number of parts the keys are partitioned into (the
 *                      decode grid is num_parts x ceil(M / tile_rows) x h_kv)
 *   fixed_cost    out: per-sequence overhead of the partition rule, in
 *                      32-key units (see mla_get_metadata)
 *   tile_rows     out: query rows per workgroup tile chosen for this M
 * Any out pointer may be NULL.
 */
int mla_get_metadata_shape(int batch, int q_rows_per_kv_head, int h_kv, int *num_parts,
                           int *fixed_cost, int *tile_rows);

/*
 * Call 1: split-KV scheduling metadata (the pages' get_mla_metadata).
 * One device kernel (one workgroup) reads cache_seqlens and writes the
 * partition; nothing is copied to the host.
 *
 * Partition rule (sequences are cut only at multiples of 32 keys):
 *   U_b = ceil(N_b / 32); cost_b = U_b + fixed_cost; C_b = sum_{b'<b} cost_b';
 *   T = ceil(C_B / num_parts).  Unit i of sequence b belongs to part
 *   floor((C_b + fixed_cost + i) / T); a sequence with N_b = 0 gets one empty
 *   piece in part floor((C_b + fixed_cost - 1) / T).  A piece is the run of
 *   one sequence's units inside one part.
 *
 *   cache_seqlens  device int32 [batch], every N_b >= 0 (not checked on host)
 *   num_parts      1 <= num_parts <= MLA_MAX_PARTS (normally from
 *                  mla_get_metadata_shape; other values are allowed)
 *   fixed_cost     >= 1
 *   tile_metadata  device int32 [num_parts, MLA_METADATA_WORDS]: per part
 *                  {bb = first sequence, first key of its piece,
 *                   be = last sequence, end key (exclusive) of its piece,
 *                   num_splits[bb] + split index of bb's piece (the partial
 *                   slot of that piece), N_bb, N_be, num_splits[be] (the
 *                   partial slot of be's piece, whose split index is 0)};
 *                  an empty part stores {0, 0, -1, 0, 0, 0, 0, 0}
 *   num_splits     device int32 [batch + 1]: num_splits[0] = 0 and
 *                  num_splits[b+1] - num_splits[b] = pieces of sequence b
 * batch must be in [1, MLA_MAX_BATCH].
 */
int mla_get_metadata(const int32_t *cache_seqlens, int batch, int q_rows_per_kv_head, int h_kv,
                     int num_parts, int fixed_cost, int32_t *tile_metadata, int32_t *num_splits,
                     void *stream);

/* Bytes of device workspace mla_decode needs (fp32 partial outputs and
 * their lse for up to batch + num_parts pieces); 0 on invalid arguments. */
size_t mla_decode_workspace_size(int batch, int q_rows_per_kv_head, int h_kv, int num_parts);

/*
 * Call 2: paged MLA decode (the pages' flash_mla_with_kvcache).
 *   q              device [batch, s_q, h_q, 576] of dtype, 16-byte aligned
 *   blocked_k      device [num_pages, 64, h_kv, 576] of dtype, 16-byte aligned
 *   block_table    device int32 [batch, max_blocks_per_seq]
 *   cache_seqlens  device int32 [batch]
 *   d, dv          must be 576 and 512; page_size must be 64
 *   dtype          MLA_DTYPE_BF16 or MLA_DTYPE_FP16 (else MLA_ERR_UNSUPPORTED):
 *                  the element type of q, blocked_k and out
 *   h_q % h_kv == 0; M = s_q * h_q / h_kv <= MLA_MAX_ROWS
 *   tile_metadata, num_parts, num_splits  from mla_get_metadata with
 *                  q_rows_per_kv_head = M and the same h_kv
 *   causal         0/1: query t sees keys j <= N - s_q + t
 *   softmax_scale  multiplies the scores; positive and finite (the usual value
 *                  is 576^-0.5)
 *   out            device [batch, s_q, h_q, 512] of dtype, 16-byte aligned,
 *                  rounded to nearest even
 *   lse            device fp32 [batch, s_q, h_q], natural log
 *   workspace      device, >= mla_decode_workspace_size(batch, M, h_kv,
 *                  num_parts) bytes, 16-byte aligned; contents are scratch
 * Enqueues the main kernel and, when a sequence has several pieces, the
 * combine kernel.  Concurrent calls must use distinct workspaces.
 */
int mla_decode(const void *q, const void *blocked_k, const int32_t *block_table,
               const int32_t *cache_seqlens, int batch, int s_q, int h_q, int h_kv, int d, int dv,
               int dtype, int num_pages, int page_size, int max_blocks_per_seq,
               const int32_t *tile_metadata, int num_parts, const int32_t *num_splits, int causal,
               float softmax_scale, void *out, float *lse, void *workspace,
               size_t workspace_bytes, void *stream);

/*
 * The two halves of mla_decode, for callers that schedule or time them
 * separately (same section 4 of the cnblogs page: blockwise attention, then
 * the merge of partial outputs).  mla_decode == mla_decode_splitkv followed
 * by mla_decode_combine on the same stream with the same workspace.
 *
 * mla_decode_splitkv: same arguments and checks as mla_decode; enqueues only
 * the main kernel.  Sequences with one piece get their final out/lse; the
 * others leave fp32 partials in the workspace.
 *
 * mla_decode_combine: merges the partials of sequences with several pieces
 * into out/lse (a sequence with one piece is left untouched).  batch, s_q,
 * h_q, h_kv, num_parts, dtype, num_splits, workspace and workspace_bytes must be the
 * values given to the preceding mla_decode_splitkv.
 */
int mla_decode_splitkv(const void *q, const void *blocked_k, const int32_t *block_table,
                       const int32_t *cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                       int d, int dv, int dtype, int num_pages, int page_size, int max_blocks_per_seq,
                       const int32_t *tile_metadata, int num_parts, const int32_t *num_splits,
                       int causal, float softmax_scale, void *out, float *lse, void *workspace,
                       size_t workspace_bytes, void *stream);

int mla_decode_combine(const int32_t *num_splits, int batch, int s_q, int h_q, int h_kv,
                       int num_parts, int dtype, void *out, float *lse, const void *workspace,
                       size_t workspace_bytes, void *stream);

/* ---- Measurement helpers (not part of the decode path) --------------------
 * Ceilings measured on the running machine, against which the main kernel's
 * throughput is quoted besides the datasheet peaks.  They compute nothing of
 * the method; the benchmark is their only caller.
 *
 * mla_ceiling_stream: each of num_workgroups workgroups streams the
 * pages_per_workgroup cache pages listed in
 * pages[w * pages_per_workgroup + i] through a 4-slot LDS ring of
 * 36,864-byte stages with 16-byte LDS-DMA loads, two stages ahead, as the main
 * kernel's 16-row tile does; no arithmetic.
 *   pool        device, num_pages pages of page_bytes bytes (one KV head)
 *   page_bytes  must be 73,728 (64 rows x 1152 B); num_pages * page_bytes
 *               must be below 2^31; a page index outside the pool loads
 *               zeros (no fault)
 *   pages       device int32 [num_workgroups, pages_per_workgroup]
 *   sink        device int32 [1]; written only in a case that does not occur
 *               for real data (it keeps the loads from being optimised away)
 * Bytes read = num_workgroups * pages_per_workgroup * page_bytes.
 *
 * mla_ceiling_mfma: num_workgroups workgroups of 4 waves; each wave runs
 * iters x 4 independent 32x32x16 bf16 MFMAs (32768 flops each).
 *   sink   device float [1], same role as above
 * Flops = num_workgroups * 4 * iters * 4 * 32768.
 * Both return MLA_ERR_INVALID_ARG for null pointers or sizes outside the
 * stated ranges and enqueue on `stream`.
 */
int mla_ceiling_stream(const void *pool, int num_pages, int page_bytes, const int32_t *pages,
                       int num_workgroups, int pages_per_workgroup, int32_t *sink, void *stream);
int mla_ceiling_mfma(float *sink, int num_workgroups, int iters, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
