// Shared device-side definitions of the paged MLA decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Fixed sizes (cnblogs FlashMLA notes, section 2: head dim 576, value dim 512;
// ygpos news: paged cache with block size 64).
constexpr int kHeadDim = 576;
constexpr int kValueDim = 512;
constexpr int kPage = 64;
constexpr int kRowBytes = kHeadDim * 2;            // one cached bf16 row
constexpr int kChunksPerRow = kRowBytes / 16;      // 72 chunks of 16 B

// A stage is 32 consecutive keys of one sequence (half a page); sequences are
// split only at stage boundaries.
constexpr int kStage = 32;
constexpr int kStageBytes = kStage * kRowBytes;    // 36864 B
constexpr int kSlots = 4;                          // LDS ring of stages
constexpr int kLdsBytes = kSlots * kStageBytes;    // 147456 B of 160 KB
constexpr int kLoadsPerStage = kStageBytes / 1024; // 1 KB per wave-wide 16 B load
constexpr int kMetaWords = 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))

// XOR swizzle of the 16-byte chunk index inside each 128-byte group of a
// cached row held in LDS (rows are 1152 B; LDS has 64 banks of 4 B).  The
// swizzle depends on the MFMA tile shape of the kernel that reads the stage;
// each choice makes that kernel's two access patterns conflict-free (checked
// with the bank-conflict counter):
//   R = 16 (16x16x32 tiles): f(r) = r & 7
//     16-byte K reads of 16 rows x one chunk, and transposed 8-byte V reads of
//     8 rows x one aligned chunk pair;
//   R = 32 (32x32x16 tiles): f(r) = bitrev3((r >> 1) & 7)
//     16-byte K reads of 16 rows x one chunk, and transposed 8-byte V reads of
//     4 rows x one aligned chunk quad.
__device__ __forceinline__ int bitrev3(int x) { return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1); }

template <int R>
__device__ __forceinline__ int swz(int row) {
  if constexpr (R == 16) return row & 7;
  else return bitrev3((row >> 1) & 7);
}

template <int R>
__device__ __forceinline__ int phys_chunk(int row, int chunk) {
  return (chunk & ~7) | ((chunk & 7) ^ swz<R>(row));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (low half = lo), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
// Two floats -> packed fp16 pair (low half = lo), round to nearest even.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}
// Element types of q, the cache, P and out.  Each gives the round-to-nearest
// pack of two floats, the MFMAs on 8-element operands with fp32 accumulation,
// and a two-element dot product with fp32 accumulation.
struct Bf16 {
  static constexpr uint32_t kOnePair = 0x3f803f80u;  // (1.0, 1.0)
  __device__ static uint32_t pack(float lo, float hi) { return pack_bf16(lo, hi); }
  __device__ static f32x16 mfma32(i16x8 a, i16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
  __device__ static f32x4 mfma16(i16x8 a, i16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
  __device__ static float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
  }
};
struct F16 {
  static constexpr uint32_t kOnePair = 0x3c003c00u;  // (1.0, 1.0)
  __device__ static uint32_t pack(float lo, float hi) { return pack_f16(lo, hi); }
  __device__ static f32x16 mfma32(i16x8 a, i16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  }
  __device__ static f32x4 mfma16(i16x8 a, i16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  }
  __device__ static float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
  }
};
// The two floats a packed bf16 pair stands for.
__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// Uniform read of read-only metadata through the scalar cache, waited on in
// the same asm block.  Used inside the stage loop, where the compiler would
// otherwise emit a vector load whose wait drains the staged key loads.
// The address must be uniform; it is passed through readfirstlane so that it
// is held in scalar registers whatever the surrounding code does with it.
__device__ __forceinline__ int sload_i32(const int32_t* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const int32_t* ps = reinterpret_cast<const int32_t*>((hi << 32) | lo);
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ps) : "memory");
  return v;
}

// Cross-lane sums and maxima without the LDS crossbar: DPP row shifts
// combine the lanes of each row of 16 (Hillis-Steele steps of 1, 2, 4, 8
// lanes; a lane with fewer than n lanes below it in its row keeps its value),
// then the row totals held by lanes 15, 31, 47 (and 63) are read into scalar
// registers and added to the later rows.  All 64 lanes must be active.
__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}
template <int N>
__device__ __forceinline__ int row_shr_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x110 + N, 0xf, 0xf, false);
}
template <int N>
__device__ __forceinline__ long long row_shr_i64(long long v) {
  const unsigned lo = (unsigned)row_shr_i32<N>((int)(unsigned)v);
  const unsigned hi = (unsigned)row_shr_i32<N>((int)(unsigned)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}
__device__ __forceinline__ long long readlane_i64(long long v, int l) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)v, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)((unsigned long long)v >> 32), l);
  return (long long)(((unsigned long long)hi << 32) | lo);
}
// Inclusive prefix sum over the 64 lanes of the wave.
__device__ __forceinline__ long long wave_inclusive_sum_i64(long long x) {
  const int r = lane_id() & 15, lane = lane_id();
#define MLA_ROW_STEP(N) { const long long t = row_shr_i64<N>(x); if (r >= N) x += t; }
  MLA_ROW_STEP(1) MLA_ROW_STEP(2) MLA_ROW_STEP(4) MLA_ROW_STEP(8)
#undef MLA_ROW_STEP
  const long long t0 = readlane_i64(x, 15), t1 = readlane_i64(x, 31), t2 = readlane_i64(x, 47);
  if (lane >= 16) x += t0;
  if (lane >= 32) x += t1;
  if (lane >= 48) x += t2;
  return x;
}
__device__ __forceinline__ int wave_inclusive_sum_i32(int x) {
  const int r = lane_id() & 15, lane = lane_id();
#define MLA_ROW_STEP(N) { const int t = row_shr_i32<N>(x); if (r >= N) x += t; }
  MLA_ROW_STEP(1) MLA_ROW_STEP(2) MLA_ROW_STEP(4) MLA_ROW_STEP(8)
#undef MLA_ROW_STEP
  const int t0 = __builtin_amdgcn_readlane(x, 15), t1 = __builtin_amdgcn_readlane(x, 31),
            t2 = __builtin_amdgcn_readlane(x, 47);
  if (lane >= 16) x += t0;
  if (lane >= 32) x += t1;
  if (lane >= 48) x += t2;
  return x;
}
// The value of x in lane l (l uniform).
__device__ __forceinline__ float row_total_f32(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
// Max / sum of x over the 64 lanes of the wave (the same value in every lane).
__device__ __forceinline__ float wave_allmax_f32(float x) {
  const int r = lane_id() & 15;
#define MLA_ROW_STEP(N) { const float t = __int_as_float(row_shr_i32<N>(__float_as_int(x))); if (r >= N) x = fmaxf(x, t); }
  MLA_ROW_STEP(1) MLA_ROW_STEP(2) MLA_ROW_STEP(4) MLA_ROW_STEP(8)
#undef MLA_ROW_STEP
  return fmaxf(fmaxf(row_total_f32(x, 15), row_total_f32(x, 31)),
               fmaxf(row_total_f32(x, 47), row_total_f32(x, 63)));
}
__device__ __forceinline__ float wave_allsum_f32(float x) {
  const int r = lane_id() & 15;
#define MLA_ROW_STEP(N) { const float t = __int_as_float(row_shr_i32<N>(__float_as_int(x))); if (r >= N) x += t; }
  MLA_ROW_STEP(1) MLA_ROW_STEP(2) MLA_ROW_STEP(4) MLA_ROW_STEP(8)
#undef MLA_ROW_STEP
  return (row_total_f32(x, 15) + row_total_f32(x, 31)) + (row_total_f32(x, 47) + row_total_f32(x, 63));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Waits and barriers written as asm so that the compiler neither moves memory
// operations across them nor adds a full drain of the vector memory counter
// (the prefetched stages must stay in flight across the barrier).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace mla
