/*
 * mla_decode.h -- C ABI of the paged MLA decode library (libmla_decode.so),
 * MI355X (gfx950).
 *
 * The operation (pages on FlashMLA):
 *   - "DeepSeek 开源记-第1天-FlashMLA" (cnblogs), section 6 (使用方法): the
 *     library is driven by two calls.  The first turns the per-sequence cache
 *     lengths, the query rows per KV head (s_q * h_q / h_kv) and the KV head
 *     count into scheduling metadata plus a per-sequence split count; the
 *     second runs the decode over the paged cache with the query, the block
 *     table, the cache lengths, the value dim, that metadata and a causal
 *     flag, and gives back the output and its log-sum-exp.  Here they are
 *     mla_get_metadata and mla_decode.
 *     Section 2 (核心功能): head dim fixed at 576, value dim fixed at 512,
 *     Shared-KV (V is the first 512 dims of the cached 576-wide row).
 *     Section 4 (核心实现): blockwise scores, softmax, merge of partial
 *     outputs.
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
 *     workspace.  No call allocates device memory.  The library keeps no
 *     state between calls except a per-device property cache and, for
 *     mla_decode_noalloc only, a scratch array in device memory that exists
 *     once per GPU for the life of the process.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Compute calls
 *     only enqueue work: they never synchronize with the host, never read
 *     device memory from the host, and enqueue no memset or copy, so a
 *     sequence of them can be captured in a HIP graph and replayed with new
 *     contents in the same buffers (the lengths are read on the device
 *     only).
 *   - Every call returns MLA_OK (0) or a negative status; on failure
 *     nothing has been enqueued unless the status is MLA_ERR_HIP (a launch
 *     error reported by the runtime).  mla_last_error() gives a thread-local
 *     message for the last failure.
 *   - Preconditions only the device could check (they are not checked):
 *     block_table entries for blocks below ceil(N/64) are valid page indices
 *     in [0, num_pages); ceil(N/64) <= max_blocks_per_seq; the metadata was
 *     produced by mla_get_metadata(_ex) for the same cache_seqlens, rows and
 *     h_kv.  Cache rows at positions >= N and table entries >= ceil(N/64) are
 *     never used and may hold anything (NaN included).  A needed table entry
 *     outside [0, num_pages) is read as a page of zeros (no memory outside
 *     the pool is touched); the result is then that of a zero page.
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
#define MLA_ERR_WORKSPACE (-3)   /* workspace smaller than mla_workspace_bytes() */
#define MLA_ERR_HIP (-4)         /* a HIP runtime call or kernel launch failed */

#define MLA_HEAD_DIM 576
#define MLA_VALUE_DIM 512
#define MLA_PAGE_SIZE 64
/* Element type of q, blocked_k and out (the cnblogs page, section 2, lists
 * FP16 beside BF16; the others BF16 only).  The arithmetic is the same:
 * products of the 16-bit inputs accumulated in fp32. */
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
 * Host-only sizing of call 1 (the cnblogs page, section 6: the metadata call
 * takes the query rows per KV head, s_q * h_q / h_kv, and h_kv).  Reads the
 * current device's compute unit count (cached) and touches no device memory.
 *   q_rows_per_kv_head  M = s_q * h_q / h_kv, 1 <= M <= MLA_MAX_ROWS
 *   num_parts       out: parts mla_get_metadata partitions the keys into
 *                        (the decode grid is num_parts x ceil(M / tile_rows)
 *                        x h_kv workgroups)
 *   words_per_part  out: MLA_METADATA_WORDS; tile_metadata is
 *                        int32 [num_parts, words_per_part]
 * Either out pointer may be NULL.
 */
int mla_metadata_shape(int batch, int q_rows_per_kv_head, int h_kv, int *num_parts,
                       int *words_per_part);

/*
 * Host-only: the row tile the decode kernel uses for M rows per KV head
 * (16, 32, 64 or 128 query rows per workgroup), the number of row tiles
 * ceil(M / tile_rows), and the partition rule's default per-sequence cost
 * in 32-key units (see mla_get_metadata).  Any out pointer may be NULL.
 */
int mla_tile_shape(int q_rows_per_kv_head, int h_kv, int *tile_rows, int *m_tiles,
                   int *fixed_cost);

/*
 * Call 1: split-KV scheduling metadata (the pages' metadata call).
 * One device kernel (one workgroup) reads cache_seqlens and writes the
 * partition; nothing is copied to the host.
 *
 * Partition rule (sequences are cut only at multiples of 32 keys), on a
 * cost line counted in half units with f = fixed_cost:
 *   U_b = ceil(N_b / 32); sequence b occupies 2 U_b + 2 f positions (f for
 *   its start, two per unit, f for its end); C_b = sum_{b'<b} (2 U_b' + 2 f).
 *   The parts share the line evenly: position x is in part
 *   part(x) = floor(x num_parts / C_B), or floor(x / 2) when
 *   C_B < 2 num_parts.  Unit i of sequence b belongs to part
 *   part(C_b + f + 2 i + 1) (the part of its midpoint); a sequence with
 *   N_b = 0 gets one empty piece in part part(C_b + f).  A piece
 *   is the run of one sequence's units inside one part; the pieces of a
 *   sequence sit in consecutive parts.  num_parts and fixed_cost are the
 *   values mla_metadata_shape and mla_tile_shape report.
 *
 *   cache_seqlens  device int32 [batch], every N_b >= 0 (not checked on host)
 *   batch          in [1, MLA_MAX_BATCH]
 *   tile_metadata  device int32 [num_parts, MLA_METADATA_WORDS], 16-byte
 *                  aligned: per part
 *                  {bb = first sequence, first key of its piece,
 *                   be = last sequence, end key (exclusive) of its piece,
 *                   num_splits[bb] + split index of bb's piece (the partial
 *                   slot of that piece), N_bb, N_be, num_splits[be] (the
 *                   partial slot of be's piece, whose split index is 0)};
 *                  an empty part stores {0, 0, -1, 0, 0, 0, 0, 0}
 *   num_splits     device int32 [batch + 1]: num_splits[0] = 0 and
 *                  num_splits[b+1] - num_splits[b] = pieces of sequence b
 */
int mla_get_metadata(const int32_t *cache_seqlens, int batch, int q_rows_per_kv_head, int h_kv,
                     int32_t *tile_metadata, int32_t *num_splits, void *stream);

/*
 * mla_get_metadata with the partition's two parameters overridable (a hook
 * for tests and tuning): num_parts_override in [1, MLA_MAX_PARTS] replaces
 * the default part count (tile_metadata must then hold num_parts_override
 * rows, and mla_decode gets num_parts = num_parts_override);
 * fixed_cost_override >= 1 replaces the default per-sequence cost.  0 means
 * the default for either.
 */
int mla_get_metadata_ex(const int32_t *cache_seqlens, int batch, int q_rows_per_kv_head, int h_kv,
                        int32_t *tile_metadata, int32_t *num_splits, void *stream,
                        int num_parts_override, int fixed_cost_override);

/* Bytes of device workspace mla_decode needs (the partial outputs of up to
 * batch + num_parts pieces, 512 values per row in the 16-bit element type of
 * q, then their fp32 lse); 0 on invalid arguments (including dv != 512). */
size_t mla_workspace_bytes(int batch, int q_rows_per_kv_head, int h_kv, int num_parts, int dv);

/*
 * Call 2: paged MLA decode (the pages' decode call).
 *   q              device [batch, s_q, h_q, 576] of dtype, 16-byte aligned
 *   blocked_k      device [num_pages, 64, h_kv, 576] of dtype, 16-byte aligned
 *   block_table    device int32 [batch, max_blocks_per_seq]
 *   cache_seqlens  device int32 [batch]
 *   d, dv          must be 576 and 512; page_size must be 64
 *   dtype          MLA_DTYPE_BF16 or MLA_DTYPE_FP16 (else MLA_ERR_UNSUPPORTED):
 *                  the element type of q, blocked_k and out
 *   h_q % h_kv == 0; M = s_q * h_q / h_kv <= MLA_MAX_ROWS
 *   tile_metadata, num_parts, num_splits  from mla_get_metadata(_ex) with
 *                  q_rows_per_kv_head = M and the same h_kv
 *   causal         0/1: query t sees keys j <= N - s_q + t
 *   softmax_scale  multiplies the scores; positive and finite (the usual value
 *                  is 576^-0.5)
 *   out            device [batch, s_q, h_q, 512] of dtype, 16-byte aligned,
 *                  rounded to nearest even
 *   lse            device fp32 [batch, s_q, h_q], natural log
 *   workspace      device, >= mla_workspace_bytes(batch, M, h_kv, num_parts,
 *                  512) bytes, 16-byte aligned; contents are scratch
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
 * others leave partials in the workspace (each piece's normalised output
 * row in the element type of q, a convex combination of value rows, and its
 * fp32 lse; the combine merges them in fp32).
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

/*
 * mla_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, checks and results as mla_decode
 * minus workspace / workspace_bytes.  The split partials go to a scratch
 * array of MLA_NOALLOC_SCRATCH_BYTES that the library holds in device memory,
 * one copy per GPU, for the life of the process (allocated when the library's
 * code object is loaded on that GPU); the call itself allocates nothing.
 *   A call whose partials would not fit (mla_workspace_bytes(batch, M, h_kv,
 *   num_parts, 512) > MLA_NOALLOC_SCRATCH_BYTES) returns MLA_ERR_WORKSPACE
 *   and enqueues nothing.
 *   Nothing in the scratch needs clearing between calls (every value read
 *   was written earlier in the same call).  All calls on one GPU share its
 *   scratch: calls that overlap in time on one GPU (different streams, or
 *   host threads without ordering) race and give wrong results.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (128u << 20)
int mla_decode_noalloc(const void *q, const void *blocked_k, const int32_t *block_table,
                       const int32_t *cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                       int d, int dv, int dtype, int num_pages, int page_size, int max_blocks_per_seq,
                       const int32_t *tile_metadata, int num_parts, const int32_t *num_splits,
                       int causal, float softmax_scale, void *out, float *lse, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
