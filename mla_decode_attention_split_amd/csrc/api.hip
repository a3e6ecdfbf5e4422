// C ABI of libmla_decode.so: argument checks, sizing and kernel dispatch.
// Declarations and the contract of every entry point: include/mla_decode.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "../../include/mla_decode.h"
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return MLA_OK;
}

// Compute-unit count per device, read once.
constexpr int kMaxDevices = 64;
int g_cus[kMaxDevices];
std::once_flag g_cu_once[kMaxDevices];

int device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device index %d", dev);
  hipError_t err = hipSuccess;
  std::call_once(g_cu_once[dev], [&]() {
    int n = 0;
    err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    g_cus[dev] = n > 0 ? n : 256;
  });
  if (err != hipSuccess)
    return fail(MLA_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(err));
  *cus = g_cus[dev];
  return MLA_OK;
}

// MLA_DECODE_LOG=1 in the environment: every metadata and decode call prints
// its launch configuration to stderr (read once per process; no effect on
// the results).
bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("MLA_DECODE_LOG");
    return v && v[0] && !(v[0] == '0' && v[1] == '\0');
  }();
  return on;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_rows(int q_rows_per_kv_head, int h_kv) {
  if (q_rows_per_kv_head < 1 || q_rows_per_kv_head > MLA_MAX_ROWS)
    return fail(MLA_ERR_UNSUPPORTED, "rows per KV head %d outside [1, %d]", q_rows_per_kv_head,
                MLA_MAX_ROWS);
  if (h_kv < 1 || h_kv > 1024) return fail(MLA_ERR_INVALID_ARG, "h_kv %d outside [1, 1024]", h_kv);
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLA_ERR_WORKSPACE: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* mla_last_error(void) { return g_err; }

namespace {

// Default partition parameters for M rows per KV head on the current device.
int default_partition(int q_rows_per_kv_head, int h_kv, int* num_parts, int* fixed_cost,
                      int* tile_rows, int* m_tiles) {
  int rc = check_rows(q_rows_per_kv_head, h_kv);
  if (rc != MLA_OK) return rc;
  const int tr = mla::tile_rows_for(q_rows_per_kv_head, h_kv);
  const int mt = (q_rows_per_kv_head + tr - 1) / tr;
  if (num_parts) {
    int cus = 0;
    rc = device_cus(&cus);
    if (rc != MLA_OK) return rc;
    // One workgroup per compute unit: parts x row tiles x KV heads ~ CUs,
    // rounded down to a multiple of 8 so each part's tiles share an XCD.
    int parts = cus / (mt * h_kv);
    parts = parts >= 8 ? (parts / 8) * 8 : 8;
    *num_parts = parts;
  }
  // Per-sequence overhead in 32-key stage units: the query rows of a piece
  // (ceil(tile rows / 32) stages' worth) plus about one stage for the
  // epilogue and the merge of one more piece, and at least 3: the 16- and
  // 32-row tiles load their query rows straight into registers, but a piece
  // still costs its prologue's memory trips and its epilogue (3 measured
  // faster than 2 on every length mix tried with those tiles).
  if (fixed_cost) {
    const int f = (tr + 31) / 32 + 1;
    *fixed_cost = f > 3 ? f : 3;
  }
  if (tile_rows) *tile_rows = tr;
  if (m_tiles) *m_tiles = mt;
  return MLA_OK;
}

}  // namespace

int mla_metadata_shape(int batch, int q_rows_per_kv_head, int h_kv, int* num_parts,
                       int* words_per_part) {
  if (batch < 1 || batch > MLA_MAX_BATCH)
    return fail(MLA_ERR_INVALID_ARG, "batch %d outside [1, %d]", batch, MLA_MAX_BATCH);
  int parts = 0;
  int rc = default_partition(q_rows_per_kv_head, h_kv, &parts, nullptr, nullptr, nullptr);
  if (rc != MLA_OK) return rc;
  if (num_parts) *num_parts = parts;
  if (words_per_part) *words_per_part = MLA_METADATA_WORDS;
  return ok();
}

int mla_tile_shape(int q_rows_per_kv_head, int h_kv, int* tile_rows, int* m_tiles, int* fixed_cost) {
  int rc = default_partition(q_rows_per_kv_head, h_kv, nullptr, fixed_cost, tile_rows, m_tiles);
  if (rc != MLA_OK) return rc;
  return ok();
}

int mla_get_metadata_ex(const int32_t* cache_seqlens, int batch, int q_rows_per_kv_head, int h_kv,
                        int32_t* tile_metadata, int32_t* num_splits, void* stream,
                        int num_parts_override, int fixed_cost_override) {
  if (batch < 1 || batch > MLA_MAX_BATCH)
    return fail(MLA_ERR_INVALID_ARG, "batch %d outside [1, %d]", batch, MLA_MAX_BATCH);
  if (num_parts_override < 0 || num_parts_override > MLA_MAX_PARTS)
    return fail(MLA_ERR_INVALID_ARG, "num_parts_override %d outside [0, %d]", num_parts_override,
                MLA_MAX_PARTS);
  if (fixed_cost_override < 0)
    return fail(MLA_ERR_INVALID_ARG, "fixed_cost_override %d < 0", fixed_cost_override);
  if (!cache_seqlens || !tile_metadata || !num_splits)
    return fail(MLA_ERR_INVALID_ARG, "null pointer (cache_seqlens, tile_metadata, num_splits)");
  if (!aligned16(tile_metadata)) return fail(MLA_ERR_INVALID_ARG, "tile_metadata not 16-byte aligned");
  int num_parts = 0, fixed_cost = 0;
  int rc = default_partition(q_rows_per_kv_head, h_kv, num_parts_override ? nullptr : &num_parts,
                             &fixed_cost, nullptr, nullptr);
  if (rc != MLA_OK) return rc;
  if (num_parts_override) num_parts = num_parts_override;
  if (fixed_cost_override) fixed_cost = fixed_cost_override;
  if (log_enabled())
    std::fprintf(stderr, "[mla] get_metadata: batch %d rows/kv-head %d h_kv %d -> num_parts %d%s, "
                 "fixed_cost %d%s\n", batch, q_rows_per_kv_head, h_kv, num_parts,
                 num_parts_override ? " (override)" : "", fixed_cost,
                 fixed_cost_override ? " (override)" : "");
  hipError_t e = mla::launch_sched(cache_seqlens, batch, num_parts, fixed_cost, tile_metadata,
                                   num_splits, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "scheduler launch: %s", hipGetErrorString(e));
  return ok();
}

int mla_get_metadata(const int32_t* cache_seqlens, int batch, int q_rows_per_kv_head, int h_kv,
                     int32_t* tile_metadata, int32_t* num_splits, void* stream) {
  return mla_get_metadata_ex(cache_seqlens, batch, q_rows_per_kv_head, h_kv, tile_metadata,
                             num_splits, stream, 0, 0);
}

size_t mla_workspace_bytes(int batch, int q_rows_per_kv_head, int h_kv, int num_parts, int dv) {
  if (batch < 1 || batch > MLA_MAX_BATCH || q_rows_per_kv_head < 1 ||
      q_rows_per_kv_head > MLA_MAX_ROWS || h_kv < 1 || num_parts < 1 || num_parts > MLA_MAX_PARTS ||
      dv != MLA_VALUE_DIM)
    return 0;
  const size_t pieces = (size_t)batch + (size_t)num_parts;
  const size_t rows = pieces * (size_t)h_kv * (size_t)q_rows_per_kv_head;
  size_t o_bytes = rows * MLA_VALUE_DIM * sizeof(uint16_t);
  size_t l_bytes = rows * sizeof(float);
  l_bytes = (l_bytes + 255) & ~(size_t)255;
  return o_bytes + l_bytes;
}

namespace {

// Shared checks and argument packing of mla_decode / mla_decode_splitkv.
int prepare_decode(const void* q, const void* blocked_k, const int32_t* block_table,
                   const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv, int d,
                   int dv, int dtype, int num_pages, int page_size, int max_blocks_per_seq,
                   const int32_t* tile_metadata, int num_parts, const int32_t* num_splits,
                   int causal, float softmax_scale, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, mla::DecodeArgs* a, int* tile_rows) {
  if (d != MLA_HEAD_DIM) return fail(MLA_ERR_UNSUPPORTED, "head dim %d (only %d)", d, MLA_HEAD_DIM);
  if (dv != MLA_VALUE_DIM)
    return fail(MLA_ERR_UNSUPPORTED, "value dim %d (only %d)", dv, MLA_VALUE_DIM);
  if (page_size != MLA_PAGE_SIZE)
    return fail(MLA_ERR_UNSUPPORTED, "page size %d (only %d)", page_size, MLA_PAGE_SIZE);
  if (dtype != MLA_DTYPE_BF16 && dtype != MLA_DTYPE_FP16)
    return fail(MLA_ERR_UNSUPPORTED, "dtype %d (only MLA_DTYPE_BF16 or MLA_DTYPE_FP16)", dtype);
  if (batch < 1 || batch > MLA_MAX_BATCH)
    return fail(MLA_ERR_INVALID_ARG, "batch %d outside [1, %d]", batch, MLA_MAX_BATCH);
  if (s_q < 1 || h_q < 1 || h_kv < 1 || h_q % h_kv != 0)
    return fail(MLA_ERR_INVALID_ARG, "s_q %d, h_q %d, h_kv %d (need h_q %% h_kv == 0)", s_q, h_q,
                h_kv);
  const long long M_ll = (long long)s_q * (h_q / h_kv);
  if (M_ll > MLA_MAX_ROWS)
    return fail(MLA_ERR_UNSUPPORTED, "s_q * h_q / h_kv = %lld > %d", M_ll, MLA_MAX_ROWS);
  const int M = (int)M_ll;
  // the kernel addresses one sequence's queries and one 32-key stage through
  // 32-bit buffer ranges
  if ((long long)s_q * h_q * MLA_HEAD_DIM * 2 >= 0x7fffffffLL ||
      32LL * h_kv * MLA_HEAD_DIM * 2 >= 0x7fffffffLL)
    return fail(MLA_ERR_UNSUPPORTED, "s_q * h_q = %lld or h_kv = %d too large", (long long)s_q * h_q, h_kv);
  int rc = check_rows(M, h_kv);
  if (rc != MLA_OK) return rc;
  if (num_pages < 1 || max_blocks_per_seq < 1)
    return fail(MLA_ERR_INVALID_ARG, "num_pages %d, max_blocks_per_seq %d", num_pages,
                max_blocks_per_seq);
  if (num_parts < 1 || num_parts > MLA_MAX_PARTS)
    return fail(MLA_ERR_INVALID_ARG, "num_parts %d outside [1, %d]", num_parts, MLA_MAX_PARTS);
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be positive and finite");
  if (!q || !blocked_k || !block_table || !cache_seqlens || !tile_metadata || !num_splits || !out ||
      !lse || !workspace)
    return fail(MLA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(q) || !aligned16(blocked_k) || !aligned16(out) || !aligned16(workspace))
    return fail(MLA_ERR_INVALID_ARG, "q, blocked_k, out and workspace must be 16-byte aligned");
  const size_t need = mla_workspace_bytes(batch, M, h_kv, num_parts, MLA_VALUE_DIM);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);

  const int tr = mla::tile_rows_for(M, h_kv);
  const size_t pieces = (size_t)batch + (size_t)num_parts;
  const size_t rows = pieces * (size_t)h_kv * (size_t)M;
  a->q = static_cast<const uint16_t*>(q);
  a->kv = static_cast<const uint16_t*>(blocked_k);
  a->block_table = block_table;
  a->seqlens = cache_seqlens;
  a->meta = tile_metadata;
  a->num_splits = num_splits;
  a->out = static_cast<uint16_t*>(out);
  a->lse = lse;
  a->o_part = static_cast<uint16_t*>(workspace);
  a->lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         rows * MLA_VALUE_DIM * sizeof(uint16_t));
  a->batch = batch;
  a->s_q = s_q;
  a->h_q = h_q;
  a->h_kv = h_kv;
  a->M = M;
  a->max_blocks = max_blocks_per_seq;
  a->num_pages = num_pages;
  a->num_parts = num_parts;
  a->m_tiles = (M + tr - 1) / tr;
  a->causal = causal ? 1 : 0;
  a->xcd_map = (num_parts % 8 == 0) ? 1 : 0;
  a->scale_log2 = softmax_scale * 1.44269504088896340736f;
  a->f16 = dtype == MLA_DTYPE_FP16 ? 1 : 0;
  const long long grid = (long long)num_parts * a->m_tiles * h_kv;
  if (grid > 0x7fffffffLL) return fail(MLA_ERR_UNSUPPORTED, "grid too large");
  *tile_rows = tr;
  if (log_enabled())
    std::fprintf(stderr, "[mla] decode: batch %d s_q %d h_q %d h_kv %d rows/kv-head %d %s causal %d "
                 "-> tile_rows %d m_tiles %d num_parts %d grid %lld (xcd map %d)\n", batch, s_q, h_q,
                 h_kv, M, a->f16 ? "fp16" : "bf16", a->causal, tr, a->m_tiles, num_parts, grid,
                 a->xcd_map);
  return MLA_OK;
}

int enqueue_combine(const mla::DecodeArgs& a, hipStream_t st) {
  mla::CombineArgs c;
  c.num_splits = a.num_splits;
  c.o_part = a.o_part;
  c.lse_part = a.lse_part;
  c.out = a.out;
  c.lse = a.lse;
  c.batch = a.batch;
  c.s_q = a.s_q;
  c.h_q = a.h_q;
  c.h_kv = a.h_kv;
  c.M = a.M;
  c.f16 = a.f16;
  c.share_grid = 0;
  hipError_t e = mla::launch_combine(c, a.num_parts, st);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace

int mla_decode_splitkv(const void* q, const void* blocked_k, const int32_t* block_table,
                       const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                       int d, int dv, int dtype, int num_pages, int page_size, int max_blocks_per_seq,
                       const int32_t* tile_metadata, int num_parts, const int32_t* num_splits,
                       int causal, float softmax_scale, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream) {
  mla::DecodeArgs a;
  int tr = 0;
  int rc = prepare_decode(q, blocked_k, block_table, cache_seqlens, batch, s_q, h_q, h_kv, d, dv,
                          dtype, num_pages, page_size, max_blocks_per_seq, tile_metadata, num_parts,
                          num_splits, causal, softmax_scale, out, lse, workspace,
                          workspace_bytes, &a, &tr);
  if (rc != MLA_OK) return rc;
  hipError_t e = mla::launch_decode(a, tr, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

int mla_decode_combine(const int32_t* num_splits, int batch, int s_q, int h_q, int h_kv,
                       int num_parts, int dtype, void* out, float* lse, const void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (batch < 1 || batch > MLA_MAX_BATCH)
    return fail(MLA_ERR_INVALID_ARG, "batch %d outside [1, %d]", batch, MLA_MAX_BATCH);
  if (s_q < 1 || h_q < 1 || h_kv < 1 || h_q % h_kv != 0)
    return fail(MLA_ERR_INVALID_ARG, "s_q %d, h_q %d, h_kv %d (need h_q %% h_kv == 0)", s_q, h_q,
                h_kv);
  const long long M_ll = (long long)s_q * (h_q / h_kv);
  if (M_ll > MLA_MAX_ROWS)
    return fail(MLA_ERR_UNSUPPORTED, "s_q * h_q / h_kv = %lld > %d", M_ll, MLA_MAX_ROWS);
  if (num_parts < 1 || num_parts > MLA_MAX_PARTS)
    return fail(MLA_ERR_INVALID_ARG, "num_parts %d outside [1, %d]", num_parts, MLA_MAX_PARTS);
  if (dtype != MLA_DTYPE_BF16 && dtype != MLA_DTYPE_FP16)
    return fail(MLA_ERR_UNSUPPORTED, "dtype %d (only MLA_DTYPE_BF16 or MLA_DTYPE_FP16)", dtype);
  if (!num_splits || !out || !lse || !workspace)
    return fail(MLA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(out) || !aligned16(workspace))
    return fail(MLA_ERR_INVALID_ARG, "out and workspace must be 16-byte aligned");
  const int M = (int)M_ll;
  const size_t need = mla_workspace_bytes(batch, M, h_kv, num_parts, MLA_VALUE_DIM);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  const size_t rows = ((size_t)batch + (size_t)num_parts) * (size_t)h_kv * (size_t)M;
  mla::DecodeArgs a{};
  a.num_splits = num_splits;
  a.o_part = const_cast<uint16_t*>(static_cast<const uint16_t*>(workspace));
  a.lse_part = reinterpret_cast<float*>(const_cast<char*>(static_cast<const char*>(workspace)) +
                                        rows * MLA_VALUE_DIM * sizeof(uint16_t));
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.batch = batch;
  a.s_q = s_q;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.M = M;
  a.num_parts = num_parts;
  a.f16 = dtype == MLA_DTYPE_FP16 ? 1 : 0;
  int rc = enqueue_combine(a, static_cast<hipStream_t>(stream));
  if (rc != MLA_OK) return rc;
  return ok();
}

}  // extern "C"

// Scratch of mla_decode_noalloc: the 16-bit partial outputs and fp32 LSEs of split
// sequences, in device memory that the library owns (one copy per GPU, held
// until the process ends).  Host code never uses the array's name as an
// address: it resolves the address once per device (scratch_of_device) and
// passes that to the kernels.
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Address of this device's copy of `scratch` (resolved on the first call on
// the device, with that device current).
int scratch_of_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device index %d", dev);
  std::call_once(g_scratch_once[dev], [&]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev])
    return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(g_scratch_err[dev]));
  *ptr = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_noalloc(const void* q, const void* blocked_k, const int32_t* block_table,
                       const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv, int d,
                       int dv, int dtype, int num_pages, int page_size, int max_blocks_per_seq,
                       const int32_t* tile_metadata, int num_parts, const int32_t* num_splits,
                       int causal, float softmax_scale, void* out, float* lse, void* stream) {
  void* ws = nullptr;
  int rc = scratch_of_device(&ws);
  if (rc != MLA_OK) return rc;
  mla::DecodeArgs a;
  int tr = 0;
  rc = prepare_decode(q, blocked_k, block_table, cache_seqlens, batch, s_q, h_q, h_kv, d, dv, dtype,
                      num_pages, page_size, max_blocks_per_seq, tile_metadata, num_parts, num_splits,
                      causal, softmax_scale, out, lse, ws, (size_t)MLA_NOALLOC_SCRATCH_BYTES, &a, &tr);
  if (rc == MLA_ERR_WORKSPACE) {
    const size_t need = mla_workspace_bytes(batch, s_q * (h_q / h_kv), h_kv, num_parts, dv);
    return fail(MLA_ERR_WORKSPACE,
                "mla_decode_noalloc: this call needs %zu bytes of scratch, more than the library's "
                "%zu (MLA_NOALLOC_SCRATCH_BYTES); use mla_decode with a caller-owned workspace",
                need, (size_t)MLA_NOALLOC_SCRATCH_BYTES);
  }
  if (rc != MLA_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = mla::launch_decode(a, tr, st);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  rc = enqueue_combine(a, st);
  if (rc != MLA_OK) return rc;
  return ok();
}

int mla_decode(const void* q, const void* blocked_k, const int32_t* block_table,
               const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv, int d, int dv,
               int dtype, int num_pages, int page_size, int max_blocks_per_seq,
               const int32_t* tile_metadata, int num_parts, const int32_t* num_splits, int causal,
               float softmax_scale, void* out, float* lse, void* workspace,
               size_t workspace_bytes, void* stream) {
  mla::DecodeArgs a;
  int tr = 0;
  int rc = prepare_decode(q, blocked_k, block_table, cache_seqlens, batch, s_q, h_q, h_kv, d, dv,
                          dtype, num_pages, page_size, max_blocks_per_seq, tile_metadata, num_parts,
                          num_splits, causal, softmax_scale, out, lse, workspace,
                          workspace_bytes, &a, &tr);
  if (rc != MLA_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = mla::launch_decode(a, tr, st);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  rc = enqueue_combine(a, st);
  if (rc != MLA_OK) return rc;
  return ok();
}

}  // extern "C"
