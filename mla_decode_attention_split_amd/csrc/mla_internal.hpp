// Host <-> kernel interface inside libmla_decode.so (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kMaxBatch = 16384;  // sequences per call (scheduler keeps prefix costs in LDS)

struct DecodeArgs {
  const uint16_t* q;          // bf16 or fp16 [batch, s_q, h_q, 576]
  const uint16_t* kv;         // same type, [num_pages, 64, h_kv, 576]
  const int32_t* block_table; // [batch, max_blocks]
  const int32_t* seqlens;     // [batch]
  const int32_t* meta;        // [num_parts, 8]
  const int32_t* num_splits;  // [batch + 1]
  uint16_t* out;              // q's type, [batch, s_q, h_q, 512]
  float* lse;                 // [batch, s_q, h_q]
  uint16_t* o_part;           // [max_pieces, h_kv, M, 512] in the element type of q
  float* lse_part;            // [max_pieces, h_kv, M]
  int batch, s_q, h_q, h_kv, M, max_blocks, num_parts, m_tiles;
  int num_pages;              // pages in blocked_k: a table entry outside [0, num_pages) reads zeros
  int causal;
  int xcd_map;                // 1: the m-tiles / KV heads of one part share an XCD
  float scale_log2;           // softmax_scale * log2(e)
  int f16;                    // 1: q, cache and out are fp16; 0: bf16
};

struct CombineArgs {
  const int32_t* num_splits;
  const uint16_t* o_part;     // 16-bit partial rows (element type of out)
  const float* lse_part;
  uint16_t* out;
  float* lse;
  int batch, s_q, h_q, h_kv, M;
  int share_grid;  // 1: one workgroup per query row (set when sequences have many pieces)
  int f16;         // 1: out is fp16; 0: bf16
};

// Query rows per workgroup for M rows per KV head.  The 128-row tile serves
// one KV head only (with several heads its query-row offsets would not fit
// in its registers); more rows per head use 64-row tiles.
inline int tile_rows_for(int M, int h_kv) {
  return M <= 16 ? 16 : M <= 32 ? 32 : (M <= 64 || h_kv > 1) ? 64 : 128;
}

hipError_t launch_sched(const int32_t* seqlens, int batch, int num_parts, int fixed_cost,
                        int32_t* meta, int32_t* num_splits, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int tile_rows, hipStream_t stream);
hipError_t launch_decode_wide(const DecodeArgs& a, hipStream_t stream);  // 128-row tiles
hipError_t launch_combine(CombineArgs a, int num_parts, hipStream_t stream);

}  // namespace mla
