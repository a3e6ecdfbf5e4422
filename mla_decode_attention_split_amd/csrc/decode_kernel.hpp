// Main paged MLA decode kernel for gfx950 (CDNA4): the kernel template.
// Instantiated in decode.hip (tiles of up to 64 query rows) and
// decode_wide.hip (the 128-row tile of one KV head).
//
// What it computes (cnblogs FlashMLA notes, sections 2 and 4): for every query
// row, blockwise scores against the 576-wide cached latent rows of its
// sequence, softmax, and the weighted sum of the first 512 dims of the same
// rows (Shared-KV); pages of 64 tokens are found through block_table
// (ygpos news: paged cache with block size 64, BF16).  Each workgroup handles
// one part of the split-KV partition (pieces of one or more sequences) for one
// tile of query rows; a sequence cut into several pieces leaves 16-bit partial
// outputs plus their log-sum-exp for the combine kernel (section 4, merge of
// partial outputs).
//
// Design (gfx950):
//   * One workgroup per CU, 4 waves (one per SIMD).  The part's key stages
//     (32-key blocks of its pieces; in the 64-row tile also two query stages
//     per piece) stream through a ring of 4 LDS slots of 36 KB with 16-byte
//     buffer loads straight into LDS.  Every ring position is loaded with the
//     same number of instructions per wave; lanes with nothing to load
//     address past their buffer's range, which costs no memory traffic, so
//     the per-stage waits are exact constants.
//   * The prologue needs one memory trip after the part's metadata record:
//     the record carries the lengths and partial slots of the part's first
//     and last sequence, and the page indices of the part are loaded into
//     registers (lane i holds entry i) together with the first piece's query
//     rows.
//   * Scores are computed transposed, S^T = K Q^T, with K from LDS (A
//     operand) and Q^T in registers for the whole piece (B operand; the 16-
//     and 128-row tiles load it from q straight into them); the MFMA result is
//     already laid out as the B operand P^T of O^T = V^T P^T.  V^T comes from
//     LDS through transposed 8-byte reads (ds_read_b64_tr_b16).
//   * Tiles of up to 64 rows (split-K): each wave owns R query rows (R = 16
//     or 32) and 512 / DG value dims; the DG waves of a row group each
//     contract an interleaved share of the 576 dims (and, with DG = 4, one of
//     the two 16-key blocks), then exchange fp32 partial scores through LDS
//     and add them in a fixed order, so every wave of the group holds
//     bit-identical scores.
//   * The 128-row tile (WIDE): each wave owns 32 rows and all 512 value dims
//     (output accumulators in the AGPRs) and contracts all 576 score dims
//     itself, so nothing is exchanged.
//   * Software pipeline: in the iteration of key block s a wave computes the
//     scores of block s while it finishes block s - 1 (softmax, P V); the
//     MFMAs of one overlap the vector work of the other, and one barrier per
//     stage serves both the ring and the exchange.
//   * Softmax in fp32 in the log2 domain; the running max is raised only when
//     a row's new max exceeds it by more than kTau (then O and l are
//     rescaled).  P is rounded to bf16 for the MFMA and a second row sum adds
//     the rounded values, so the output is normalised by exactly the weights
//     that multiplied V.
#pragma once

#include <type_traits>
#include <utility>

#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

constexpr float kTau = 8.0f;        // lazy-rescale threshold (log2 units)
constexpr float kMinit = -1.0e30f;  // finite "minus infinity" for the running max
constexpr float kLn2 = 0.69314718055994530942f;
#ifndef MLA_VP32
#define MLA_VP32 2
#endif
#ifndef MLA_VP16
#define MLA_VP16 4
#endif
#ifndef MLA_KP32
#define MLA_KP32 4
#endif
#ifndef MLA_KP16
#define MLA_KP16 4
#endif
#ifndef MLA_QD32
#define MLA_QD32 6
#endif
constexpr int kListPages = 128;     // page indices held in registers (2 per lane)
constexpr int kListPieces = 64;     // sequence lengths held in registers (1 per lane)
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr unsigned kOutOfRange = 0x80000000u;  // buffer offset that loads nothing

__device__ __forceinline__ i16x8 lds_read_b128(const char MLA_LDS* p) {
  return *reinterpret_cast<const i16x8 MLA_LDS*>(p);
}
__device__ __forceinline__ f32x4 lds_read_f4(const char MLA_LDS* p) {
  return *reinterpret_cast<const f32x4 MLA_LDS*>(p);
}
__device__ __forceinline__ void lds_write_f4(char MLA_LDS* p, f32x4 v) {
  *reinterpret_cast<f32x4 MLA_LDS*>(p) = v;
}
__device__ __forceinline__ i16x4 lds_read_tr(const char MLA_LDS* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 MLA_LDS*)(p));
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}
constexpr int kCpolNT = 2;  // cache policy: non-temporal (gfx950 "nt")
// 16 bytes from rsrc + voff into LDS; lane l writes dst + 16 l.  An offset
// past the buffer's range loads nothing (the LDS bytes become zero).  With
// `nt` the load is non-temporal: for data no other workgroup reads again it
// raised the membound stream from 4.48 to 4.97 TB/s, while it slows loads
// whose pages the other row tiles of a part read from L2.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, unsigned voff,
                                           char MLA_LDS* dst, bool nt) {
  if (nt) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void MLA_LDS*)dst, 16, voff, 0, 0, kCpolNT);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void MLA_LDS*)dst, 16, voff, 0, 0, 0);
}
// The same load written as asm, for the WIDE tile: the compiler then does not
// know that it writes LDS and adds no vmcnt wait of its own before later LDS
// reads (it cannot tell the ring slot being read from the one being filled,
// and its wait drained the prefetched stages).  The kernel orders the DMA
// writes against its LDS reads itself: an explicit vmcnt wait and a barrier
// before any slot is read.  M0 holds the LDS address; one wait state
// separates its write from the load.
// (clang notes that M0 is a reserved register; the clobber still tells it
// that the value it may keep there is gone, which is the intent.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool NT>
__device__ __forceinline__ void load_lds16_asm(__amdgpu_buffer_rsrc_t r, unsigned voff, char MLA_LDS* dst) {
  const unsigned m0 = (unsigned)(uintptr_t)dst;
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :: "s"(m0), "v"(voff), "s"(r) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(voff), "s"(r) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
// max of x over lanes l and l ^ 32 (v_permlane32_swap), and l ^ 16
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// x + (x of lane l ^ 32), and of lane l ^ 16 (the same sum in both lanes)
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// o *= s (the rescale when a row's running max is raised).
template <int N, typename V>
__device__ __forceinline__ void acc_scale(V& o, float s) {
#pragma unroll
  for (int i = 0; i < N; ++i) o[i] *= s;
}

// WIDE tiles hold their 16 output tiles (256 fp32 per lane) in AGPRs.  The
// compiler would place MFMA accumulators of that size partly in VGPRs, so
// every access to them is written as asm on "+a" operands, which keeps each
// tile in one fixed AGPR block: the P V MFMAs themselves, and fences that
// order the compiler's own reads and writes of the tiles (zeroing, the
// rescale, the epilogue) against them.  Wait states the compiler cannot see
// across asm are issued here: 2 between a VALU write of a VGPR or AGPR and an
// MFMA reading it (each MFMA is preceded by s_nop 1, which also covers its P
// and V operands), and 18 between the last MFMA writing a tile and a VALU
// read of it (more than the 8-pass 32x32x16 MFMA needs).
template <typename E>
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, i16x8 a, i16x8 b) {
  if constexpr (std::is_same<E, Bf16>::value)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Order every access to the 16 AGPR tiles before / after this point, with
// the wait states for reading them after an MFMA.
__device__ __forceinline__ void agpr_fence_read(f32x16 (&o)[16]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 1"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]),
                 "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]),
                 "+a"(o[14]), "+a"(o[15]));
}
// Fences on one tile: the compiler's reads or writes of that tile stay
// between them (NOPS wait states first).
template <int NOPS>
__device__ __forceinline__ void agpr_fence_one(f32x16& o) {
  if constexpr (NOPS == 18) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 1" : "+a"(o)::"memory");
  else if constexpr (NOPS == 2) asm volatile("s_nop 1" : "+a"(o)::"memory");
  else asm volatile("" : "+a"(o)::"memory");
}
// The same, for MFMAs reading the tiles after VALU writes to them.
__device__ __forceinline__ void agpr_fence_write(f32x16 (&o)[16]) {
  asm volatile("s_nop 1"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]),
                 "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]),
                 "+a"(o[14]), "+a"(o[15]));
}

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, unrolled at compile
// time (a loop the compiler might not unroll would index register arrays
// dynamically).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
// Issue order of a WIDE iteration: WA score MFMAs, then NQR more score MFMAs
// spread evenly over NV P V MFMAs.  Step g is a score MFMA (k-step
// wide_qk_of) or P V MFMA number wide_pv_of.
__host__ __device__ constexpr bool wide_is_qk(int g, int WA, int NQR, int NV) {
  return g < WA || ((g - WA + 1) * NQR) / (NQR + NV) > ((g - WA) * NQR) / (NQR + NV);
}
__host__ __device__ constexpr int wide_qk_of(int g, int WA, int NQR, int NV) {
  return g < WA ? g : WA + ((g - WA) * NQR) / (NQR + NV);
}
__host__ __device__ constexpr int wide_pv_of(int g, int WA, int NQR, int NV) {
  return (g - WA) - ((g - WA) * NQR) / (NQR + NV);
}

__device__ __forceinline__ i16x8 cat(i16x4 a, i16x4 b) {
  return i16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Tile shape.  R rows per wave (32x32x16 MFMA for R = 32, 16x16x32 for
// R = 16), RG row groups x DG value-dim groups = 4 waves (one per SIMD).
template <int R, int RG, int DG>
struct Tile {
  static constexpr int NW = RG * DG;
  static constexpr int BM = R * RG;                      // query rows per workgroup
  // WIDE tiles (DG = 1): every wave owns R query rows and all 512 value dims
  // (its output accumulators fill the AGPRs) and contracts all 576 dims of
  // its scores itself, so no partial scores are exchanged.
  static constexpr bool WIDE = DG == 1;
  // 16-byte loads per lane per stage (36 per stage = 4 waves x 9)
  static constexpr int LPW = kLoadsPerStage / NW;
  static constexpr int KSTEPS = R == 32 ? 36 : 18;       // score k-steps over 576 dims
  static constexpr int KSPLIT = WIDE ? 1 : 2;            // k-step interleave among DG waves
  static constexpr int KBSPLIT = DG / KSPLIT;            // 16-key blocks split among waves (R = 16)
  static constexpr int KS_W = KSTEPS / KSPLIT;           // k-steps per wave
  static constexpr int KB_W = R == 32 ? 1 : 2 / KBSPLIT; // score blocks per wave
  static constexpr int NT = (R == 32 ? 16 : 32) / DG;    // value-dim tiles per wave
  static constexpr int OREGS = R == 32 ? 16 : 4;         // accumulator registers per tile
  static constexpr int PARTIAL_BYTES = R == 32 ? 4096 : 1024;  // one score block, fp32
  static constexpr int XCH_ONE = NW * KB_W * PARTIAL_BYTES;    // one exchange buffer
  // 16-row tiles double-buffer the exchange; 32-row tiles have room for one
  // buffer and separate its reads from the next writes with a barrier; WIDE
  // tiles exchange nothing.
  static constexpr int XCH_BUFS = WIDE ? 0 : R == 32 ? 1 : 2;
  static constexpr int RING_BYTES = kSlots * kStageBytes;
  // WIDE tiles keep the Q^T fragments of the rope dims (the last QR_STEPS
  // k-steps of each wave) in LDS instead of registers
  static constexpr int QR_STEPS = WIDE ? 4 : 0;
  static constexpr int QREG_STEPS = KS_W - QR_STEPS;     // Q^T k-steps held in registers
  static constexpr int QR_BYTES = NW * QR_STEPS * 1024;
  // Query rows (Q^T): the 16-row and 128-row tiles load them from q straight
  // into registers (DQ).  The 64-row tile streams them through the ring as
  // NQS query stages per piece instead: a 32-row wave's direct loads touch
  // 32 rows of 32 bytes per instruction, and with 18 of them per wave in
  // each of its four waves this measured slower than two ring stages.
  static constexpr bool DQ = WIDE || R == 16;
  static constexpr int NQ = (BM + kStage - 1) / kStage;  // query stages per piece
  static constexpr int NQS = DQ ? 0 : NQ;
  static constexpr int QK_MFMA = KS_W * KB_W;
  static constexpr int PV_MFMA = R == 32 ? 2 * NT : NT;
  static constexpr int NSLOT = QK_MFMA + PV_MFMA;        // points where loads are issued
  static_assert(NW == 4 && LPW * NW == kLoadsPerStage, "four waves per workgroup, 9 loads each");
  static_assert(WIDE ? (R == 32 && NW == 4) : (DG >= 2 && DG % 2 == 0),
                "split-K tiles, or the 4-wave WIDE tile of 32-row waves");
  static_assert(KS_W * KSPLIT == KSTEPS && KBSPLIT * KSPLIT == DG, "score split");
  static_assert(R == 16 || KBSPLIT == 1, "key-block split only for 16-row tiles");
  static_assert(NSLOT >= LPW, "one load per issue point at most");
  static_assert(2 * LPW < 63, "vector memory counter capacity");
  static_assert(RING_BYTES + XCH_BUFS * XCH_ONE + QR_BYTES <= 163840, "LDS capacity");
};

// NTK: the key stages load non-temporally (the launch sets it when no other
// row tile of a part reads the same pages).  It is a template parameter so
// that every ring position is one straight run of loads, which the
// compiler's count of outstanding loads follows exactly.
template <int R, int RG, int DG, bool QG, bool NTK, typename E>
__global__ __launch_bounds__(64 * RG * DG, 1) void decode_kernel(
    const uint16_t* __restrict__ q_ptr, const uint16_t* __restrict__ kv_ptr,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seqlens,
    const int32_t* __restrict__ meta, uint16_t* __restrict__ out, float* __restrict__ lse,
    uint16_t* __restrict__ o_part, float* __restrict__ lse_part, DecodeArgs a) {
  using T = Tile<R, RG, DG>;
  constexpr int NW = T::NW, BM = T::BM, LPW = T::LPW, KS_W = T::KS_W, KB_W = T::KB_W;
  constexpr int NT = T::NT, OREGS = T::OREGS;
  using OAcc = typename std::conditional<R == 32, f32x16, f32x4>::type;
  constexpr int SREGS = R == 32 ? 16 : 8;  // scores per lane per stage

  __shared__ __attribute__((aligned(1024))) char lds_raw[T::RING_BYTES + T::XCH_BUFS * T::XCH_ONE + T::QR_BYTES];
  char MLA_LDS* lds = (char MLA_LDS*)lds_raw;
  char MLA_LDS* xch0 = lds + T::RING_BYTES;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  // this wave's Q^T rope fragments (WIDE tiles): step j at qr0 + 1024 j
  char MLA_LDS* qr0 = T::QR_STEPS > 0 ? xch0 + T::XCH_BUFS * T::XCH_ONE + w * T::QR_STEPS * 1024 + lane * 16
                                      : lds;
  const int rg = w / DG;
  const int dg = w % DG;
  const int kh = dg % T::KSPLIT;   // k-step share: steps ks = 2 j + kh
  const int kbs = dg / T::KSPLIT;  // key block of this wave when KBSPLIT = 2

  // ---- which part / row tile / KV head -------------------------------------
  const int inner = a.m_tiles * a.h_kv;
  int part, inner_idx;
  if (a.xcd_map) {  // the m-tiles and KV heads of a part run on one XCD
    const int id = blockIdx.x;
    const int jj = id >> 3;
    inner_idx = jj % inner;
    part = (jj / inner) * 8 + (id & 7);
  } else {
    part = blockIdx.x / inner;
    inner_idx = blockIdx.x % inner;
  }
  const int mtile = inner_idx / a.h_kv;
  const int g = inner_idx % a.h_kv;
  const int32_t* mp = meta + (long long)part * kMetaWords;
  const int bb = mp[0], tb = mp[1], be = mp[2], te = mp[3];
  const int slot_first = mp[4], n_first = mp[5], n_last = mp[6], slot_last = mp[7];
  if (bb > be) return;  // empty part (uniform over the workgroup)

  const int M = a.M;
  const int hpg = a.h_q / a.h_kv;
  const int row_stride = a.h_kv * kRowBytes;  // bytes between consecutive tokens
  const char* kv_bytes = reinterpret_cast<const char*>(kv_ptr) + (long long)g * kRowBytes;
  const int npieces = be - bb + 1;
  const int m_lo = mtile * BM;
  const int m_hi = (m_lo + BM < M ? m_lo + BM : M);  // end of the tile's valid rows

  // ---- lane constants --------------------------------------------------------
  const int lr = lane % R;  // this lane's query row inside the wave tile
  const int my_row = m_lo + rg * R + lr;
  const int q_row = my_row < M ? my_row : M - 1;
  const int q_t = q_row / hpg;
  const int q_h = g * hpg + q_row % hpg;

  // Q^T fragments of the current piece (B operands of the score MFMAs).  DQ
  // tiles load them straight from q into the registers: the wave's local k-step j is
  // k-step ks = KSPLIT j + kh, and lane l's fragment of it is the 16 bytes of
  // the lane's query row at dims 16 ks + 8 (l / 32) (R = 32) or
  // 32 ks + 8 (l / 16) (R = 16), one 16-byte load per k-step.  WIDE tiles
  // send their rope k-steps into the wave's LDS area by DMA instead, in the
  // layout they are read in (lane l at 16 l).  Rows past the tile's last
  // valid row load zeros (outside the buffer's range).  The next piece's Q^T
  // is loaded right after the current piece's last score MFMAs, so its
  // latency hides behind the last P V MFMAs and the epilogue, and the ring
  // carries key stages only.  The 16-row tiles (DQ, not WIDE) load piece 0's
  // Q^T in the prologue, with the part's page list (Q_EARLY).
  constexpr int QSTEP = (R == 32 ? 32 : 64) * T::KSPLIT;  // bytes between the wave's k-steps
  i16x8 qf[T::QREG_STEPS];
  int q_piece = -1;  // piece whose Q^T is in qf (or in flight)
  const unsigned q_sub = (unsigned)(R == 32 ? 16 * (lane >> 5) + 32 * kh : 16 * (lane >> 4) + 64 * kh);
  // The lane's query row in the buffer of the piece's query rows: with one KV
  // head the tile's rows are consecutive q rows (the buffer starts at the
  // tile's first row); with several, row m is token m / hpg, head
  // g hpg + m % hpg of the sequence.
  const unsigned q_lane =
      QG ? (my_row < M ? (unsigned)((q_t * a.h_q + q_h) * kRowBytes) + q_sub : kOutOfRange)
         : (unsigned)((rg * R + lr) * kRowBytes) + q_sub;
  char MLA_LDS* qr_wave = xch0 + T::XCH_BUFS * T::XCH_ONE + w * T::QR_STEPS * 1024;  // wave-uniform
  auto load_q = [&](int jn) {
    if constexpr (!T::DQ) return;
    const char* qb = reinterpret_cast<const char*>(q_ptr) +
                     ((long long)(bb + jn) * a.s_q * a.h_q + (QG ? 0 : m_lo)) * kRowBytes;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qb, (QG ? a.s_q * a.h_q : m_hi - m_lo) * kRowBytes);
    // (opaque, so that the step offsets go into the loads' offset field
    // instead of registers computed once before the loop over pieces)
    unsigned ql = q_lane;
    asm volatile("" : "+v"(ql));
#pragma unroll
    for (int ks = 0; ks < T::QREG_STEPS; ++ks)
      qf[ks] = __builtin_bit_cast(i16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, ql + QSTEP * ks, 0, 0));
#pragma unroll
    for (int j = 0; j < T::QR_STEPS; ++j)
      load_lds16_asm<false>(qrs, ql + QSTEP * (T::QREG_STEPS + j), qr_wave + 1024 * j);
    q_piece = jn;
  };
  constexpr bool Q_EARLY = T::DQ && !T::WIDE;

  // ---- the part's pages, one per lane --------------------------------------
  // Piece j (sequence bb + j) covers keys [lo_j, hi_j); its pages are entries
  // lo_j / 64 .. ceil(hi_j / 64) - 1 of the sequence's block_table row and
  // occupy positions cum_j .. cum_j + pages_j - 1 of the part's page list.
  // With one or two pieces the metadata record holds every length needed, so
  // the page loads are the prologue's only memory trip; longer parts first
  // load the lengths of their middle sequences.
  int v_n = 0;  // lane j: length of sequence bb + j (middle pieces only)
  const bool short_part = npieces <= 2;
  if (!short_part && !T::WIDE) {
    if (lane < npieces && lane < kListPieces) v_n = seqlens[bb + lane];
    asm volatile("" ::"v"(v_n));
  }
  auto piece_n = [&](int j) -> int {
    if (j == 0) return n_first;
    if (j == npieces - 1) return n_last;
    if constexpr (T::WIDE) return sload_i32(seqlens + bb + j);  // (no register to spare)
    return j < kListPieces ? readlane(v_n, j) : sload_i32(seqlens + bb + j);
  };
  // Pages of piece j (lane j) and the position of its first page in the list.
  int v_pages = 0, v_cum = 0, total_listed, p0 = 0, p1 = 0;
  if (short_part) {  // scalar: no cross-lane scan before the page loads
    const int hi0 = bb == be ? te : n_first;
    p0 = hi0 > tb ? (hi0 + kPage - 1) / kPage - tb / kPage : 0;
    p1 = (npieces == 2 && te > 0) ? (te + kPage - 1) / kPage : 0;
    total_listed = p0 + p1;
  } else {
    const int j = lane;
    if (j < npieces && j < kListPieces) {
      const int lo = j == 0 ? tb : 0;
      const int hi = bb + j == be ? te : (j == 0 ? n_first : v_n);
      v_pages = hi > lo ? (hi + kPage - 1) / kPage - lo / kPage : 0;
    }
    v_cum = wave_inclusive_sum_i32(v_pages) - v_pages;
    const int last = (npieces < kListPieces ? npieces : kListPieces) - 1;
    total_listed = readlane(v_cum, last) + readlane(v_pages, last);
  }
  const int listed_pieces = npieces < kListPieces ? npieces : kListPieces;
  // The page list is used only if it holds every page of the part.
  // WIDE tiles have no register to spare for the list: they read each
  // stage's page index with a scalar load (right after the stage barrier,
  // when the wave has no LDS operation outstanding).
  constexpr int LIST_HALVES = T::WIDE ? 1 : 2;
  const bool use_list = !T::WIDE && npieces <= kListPieces && total_listed <= 64 * LIST_HALVES;
  int v_page[LIST_HALVES] = {};
  if (Q_EARLY) load_q(0);  // (a part's piece 0 has keys unless it ends where it starts)
  if (use_list) {
#pragma unroll
    for (int half = 0; half < LIST_HALVES; ++half) {
      const int i = lane + 64 * half;
      long long idx = -1;
      if (short_part) {
        if (i < p0) idx = (long long)bb * a.max_blocks + tb / kPage + i;
        else if (i < p0 + p1) idx = (long long)be * a.max_blocks + (i - p0);
      } else {
        for (int j = 0; j < listed_pieces; ++j) {
          const int c = readlane(v_cum, j), p = readlane(v_pages, j);
          if (i >= c && i < c + p) idx = (long long)(bb + j) * a.max_blocks + (j == 0 ? tb : 0) / kPage + (i - c);
        }
      }
      if (idx >= 0) v_page[half] = block_table[idx];
    }
  }
  // The first position needs the list, and piece 0 its Q^T: wait for both
  // here, where the compiler sees it (else it finds them possibly in flight
  // wherever the stream reads them, and drains the prefetched stages there).
  if (Q_EARLY || use_list) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)


  // Byte offset (inside a stage) of this lane's k-th 16-byte load, and of the
  // LDS cell it fills (wave w's k-th load fills cells (k NW + w) 64 + lane).
  unsigned loff[LPW];
#pragma unroll
  for (int k = 0; k < LPW; ++k) {
    const int s = (k * NW + w) * 64 + lane;
    const int row = s / kChunksPerRow;
    const int pc = s - row * kChunksPerRow;
    loff[k] = row * row_stride + phys_chunk<R>(row, pc) * 16;  // the swizzle is an involution
  }

  // K / Q fragment offsets (A / B operands) for this wave's k-steps, and V^T
  // (transposed read) offsets, inside a stage.  Local step j is k-step
  // ks = 2 j + kh (WIDE: ks = j).
  //   R = 32: chunk 2 ks + h (h = lane / 32) -> koff[j % 2] + 128 (j / 2)
  //           (WIDE: koff[j % 4] + 128 (j / 4))
  //   R = 16: chunk 4 ks + lane / 16         -> koff[0] + 128 j
  int koff[T::WIDE ? 4 : 2];
  int voff[4];
  if constexpr (R == 32) {
    const int h = lane >> 5;
    int kbase[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) kbase[rr] = lr * kRowBytes + 16 * ((2 * rr + h) ^ swz<32>(lr));
    if constexpr (T::WIDE) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) koff[rr] = kbase[rr];
    } else {
      koff[0] = kh ? kbase[1] : kbase[0];
      koff[1] = kh ? kbase[3] : kbase[2];
    }
    // key row 16 kb + 8 jh + 4 h + r: swz = 4 (r >> 1) + 2 h + jh;
    // dims 32 nb + 16 dh + 4 c: chunk 8 (nb >> 1) + 4 (nb & 1) + 2 dh + (c >> 1)
    const int G = lane >> 4, i = lane & 15, dh = G & 1, r = i >> 2, c = i & 3;
#pragma unroll
    for (int nbp = 0; nbp < 2; ++nbp)
#pragma unroll
      for (int jh = 0; jh < 2; ++jh)
        voff[2 * nbp + jh] = (4 * h + r) * kRowBytes + 8 * (c & 1) +
                             16 * ((4 * nbp + 2 * dh + (c >> 1)) ^ (4 * (r >> 1) + 2 * h + jh));
  } else {
    const int gq = lane >> 4;
    koff[0] = koff[1] = lr * kRowBytes + 16 * ((4 * kh + gq) ^ swz<16>(lr));
    // key row 16 jh + 4 gq + r: swz = 4 (gq & 1) + r;
    // dims 16 nb + 4 c: chunk 8 (nb >> 2) + 2 (nb & 3) + (c >> 1)
    const int i = lane & 15, r = i >> 2, c = i & 3;
#pragma unroll
    for (int nbq = 0; nbq < 4; ++nbq)
      voff[nbq] = (4 * gq + r) * kRowBytes + 8 * (c & 1) +
                  16 * ((2 * nbq + (c >> 1)) ^ (4 * (gq & 1) + r));
  }
  auto kstep_off = [&](int j) -> int {
    if constexpr (T::WIDE) return koff[j & 3] + 128 * (j >> 2);
    else if constexpr (R == 32) return koff[j & 1] + 128 * (j >> 1);
    else return koff[0] + 128 * j;
  };
  // Key index (within a stage) of score register i of this lane is
  // key_lane + key_reg(i): a per-lane part and a compile-time part, so masks
  // compare against immediates.
  const int key_lane = R == 32 ? 4 * (lane >> 5) : 4 * (lane >> 4);
  auto key_reg = [](int i) -> int { return R == 32 ? 8 * (i >> 2) + (i & 3) : 16 * (i >> 2) + (i & 3); };

  // ---- stage stream -----------------------------------------------------------
  // For every non-empty piece: NQS query stages (32 rows of the tile each,
  // same swizzled row layout as the keys; none in DQ tiles), then the
  // piece's key stages.  Stream position c uses ring slot c % 4; position
  // c + 2 is loaded while position c is computed.  Past the end of the
  // stream the loads are out of range.
  // Cursor of the stream: piece lj, query stage lq, key token ltok (end lhi),
  // and the next key stage's page-list position lpos and page half lhalf.
  int lj = 0, lq = 0, ltok = tb, lhi = (bb == be) ? te : n_first;
  int lpos = 0, lhalf = (tb >> 5) & 1;
  bool lvalid = true;
  auto next_piece = [&]() {
    while (true) {
      if (bb + lj >= be) {
        lvalid = false;
        return;
      }
      lpos += lhalf;  // a piece that ended mid-page: the next page is the next piece's
      lhalf = 0;
      ++lj;
      lq = 0;
      ltok = 0;
      lhi = (bb + lj == be) ? te : piece_n(lj);
      if (ltok < lhi) return;
    }
  };
  if (ltok >= lhi) {  // the first piece is empty: no page of it is listed
    lhalf = 0;
    next_piece();
  }

  // The stream position being loaded: a buffer over its bytes (range 0 =
  // nothing, past the end of the stream) and per-lane offsets (the key-row
  // offsets loff, or query-row offsets for a query stage).
  __amdgpu_buffer_rsrc_t pend = make_rsrc(kv_bytes, 0);
  char MLA_LDS* pend_dst = lds;
  // Query stages: with one KV head the 32 rows of a query stage are
  // consecutive q rows, so they load with the key-row offsets loff from a
  // buffer that starts at the stage's first row and ends at the tile's last
  // valid row.  Otherwise (QG) every lane's offset is computed.
  bool pend_q = false;
  static_assert(!(QG && T::WIDE), "the WIDE tile serves one KV head");
  // (query stages use the default cache policy: the pieces of a sequence
  // split over many parts all read its query rows)
  static_assert(T::NQS == 0 || !NTK, "tiles with query stages keep the default policy");
  constexpr bool QOFF = QG && T::NQS > 0;
  unsigned qoff[QOFF ? LPW : 1];
  // Query row m of the KV head is token m / hpg, head g hpg + m % hpg; the
  // quotient comes from a float reciprocal (m is below 2^13, so the product
  // is off by far less than one and truncation errs by at most one) and one
  // correction.
  const int q_hq = a.h_q;
  const float hpg_inv = 1.0f / (float)hpg;
  auto q_offset = [m_hi, hpg, hpg_inv, q_hq, g, w, lane](int k, int m0) -> unsigned {
    const int cell = (k * NW + w) * 64 + lane;
    const int row = cell / kChunksPerRow;
    const int pc = cell - row * kChunksPerRow;
    const int m = m0 + row;
    int t = (int)((float)m * hpg_inv);
    int h = m - t * hpg;
    if (h < 0) {
      t -= 1;
      h += hpg;
    } else if (h >= hpg) {
      t += 1;
      h -= hpg;
    }
    return m < m_hi ? (unsigned)((t * q_hq + g * hpg + h) * kRowBytes + phys_chunk<R>(row, pc) * 16)
                    : kOutOfRange;
  };
  // (positions past the end of the stream load nothing, so the cache policy
  // of their loads does not matter)
  auto voff_of = [&](int k) -> unsigned {
    if constexpr (QOFF) return pend_q ? qoff[k] : loff[k];
    else return loff[k];
  };
  auto fire = [&](int k) { load_lds16(pend, voff_of(k), pend_dst + k * NW * 1024, NTK); };
  // All LPW loads of the pending position.
  auto fire_all = [&]() {
#pragma unroll
    for (int k = 0; k < LPW; ++k) {
      if constexpr (T::WIDE) load_lds16_asm<NTK>(pend, loff[k], pend_dst + k * NW * 1024);
      else load_lds16(pend, voff_of(k), pend_dst + k * NW * 1024, NTK);
    }
  };
  // issue point s of the stage's NSLOT points fires loads k with
  // k * NSLOT / LPW == s (resolved at compile time)
  auto fire_slot = [&](int s) {
#pragma unroll
    for (int k = 0; k < LPW; ++k)
      if (k * T::NSLOT / LPW == s) fire(k);
  };
  // the loads of issue points from..NSLOT-1
  auto fire_from = [&](int from) {
#pragma unroll
    for (int k = 0; k < LPW; ++k)
      if (k * T::NSLOT / LPW >= from) fire(k);
  };
  // Plan the next stream position into ring slot `wr`; the caller fires its
  // LPW loads.
  const long long page_bytes = (long long)kPage * row_stride;
  const int half_bytes = kStage * row_stride;
  auto plan = [&](char MLA_LDS* __restrict__ wr) {
    pend_dst = wr + w * 1024;
    pend_q = false;
    if (lvalid && lq >= T::NQS) {
      int page;
      if (use_list) page = readlane(LIST_HALVES == 1 || lpos < 64 ? v_page[0] : v_page[LIST_HALVES - 1], lpos & 63);
      else page = sload_i32(block_table + (long long)(bb + lj) * a.max_blocks + (ltok >> 6));
      // Rows past the end of the sequence are out of the buffer's range, so
      // they arrive as zeros: their V rows then contribute exactly nothing
      // (cache memory past the end may hold anything, NaN included).  A
      // table entry outside the pool loads nothing either: the stage reads
      // as a page of zeros, and no memory outside the pool is touched.
      const bool page_ok = (unsigned)page < (unsigned)a.num_pages;
      const int rows = !page_ok ? 0 : lhi - ltok < kStage ? lhi - ltok : kStage;
      pend = make_rsrc(kv_bytes + (page_ok ? page : 0) * page_bytes + lhalf * half_bytes, rows * row_stride);
      lpos += lhalf;
      lhalf ^= 1;
      ltok += kStage;
      if (ltok >= lhi) next_piece();
    } else if (lvalid) {
      const int b = bb + lj;
      const char* qseq = reinterpret_cast<const char*>(q_ptr) + (long long)b * a.s_q * a.h_q * kRowBytes;
      const int m0 = m_lo + kStage * lq;
      if constexpr (QOFF) {
        pend = make_rsrc(qseq, a.s_q * a.h_q * kRowBytes);
        pend_q = true;
#pragma unroll
        for (int k = 0; k < LPW; ++k) qoff[k] = q_offset(k, m0);
      } else {
        int rows = m_hi - m0 < kStage ? m_hi - m0 : kStage;
        rows = rows > 0 ? rows : 0;  // the tile's last query stage may be empty
        pend = make_rsrc(qseq + (long long)m0 * kRowBytes, rows * kRowBytes);
      }
      ++lq;
    } else {
      pend = make_rsrc(kv_bytes, 0);
    }
  };
  // WIDE tiles load the first piece with keys' Q^T before the first two
  // stream positions (the 16-row tiles loaded piece 0's with the page list).
  if (T::WIDE && lvalid) load_q(lj);
  plan(lds);
  fire_all();
  plan(lds + kStageBytes);
  fire_all();

  int cstage = 0;
  auto slot_of = [&](int c) { return lds + (c & (kSlots - 1)) * kStageBytes; };
  // Wait for stream position cstage (position cstage + 1 may stay in flight),
  // then a barrier: the stage and the previous iteration's partial scores are
  // visible to all waves, and the slot refilled next has been read by all.
  auto stage_ready = [&]() {
    wait_vmcnt<LPW>();
    block_barrier();
  };
  // query rows of this wave inside its query stage (tiles with query stages)
  const int q_stage = (rg * R) / kStage;
  const int q_row0 = (rg * R) % kStage;
  // Write the normalised output of one piece (scaled by `scale`): out and lse
  // for a whole sequence, else 16-bit partials (and an fp32 lse) for the
  // combine.  Rows leave through LDS: in the MFMA layout a lane holds a few
  // 8-byte pieces of one row, and a store of that layout touches 16-32 rows,
  // which the store path serves at a fraction of its contiguous rate.  So
  // every wave first writes its values into the two ring slots the piece's
  // last stages used (free once every wave is past them; the two positions
  // in flight use the other two slots), rows at a padded pitch, and the
  // workgroup then stores whole rows, 16 contiguous bytes per lane.  The
  // 128-row tile does this in two rounds, one per half of the value dims
  // (a 512-byte half row per 32 lanes).
  // WIDE tiles read their AGPR tiles one at a time (a fence per tile keeps
  // the compiler from moving all 256 values to VGPRs at once).
  constexpr int ROUNDS = BM > 64 ? 2 : 1;
  constexpr int DR = kValueDim / ROUNDS;                   // value dims per round
  constexpr int kStagePitch = DR * 2 + 16;                 // bytes per staged row
  constexpr int LPR = DR * 2 / 16;                         // lanes per staged row
  constexpr int RPI = 64 / LPR;                            // rows per store instruction
  constexpr int kRowsPerSlot = kStageBytes / kStagePitch / RPI * RPI;  // whole store groups
  static_assert(BM <= 2 * kRowsPerSlot, "the staged rows fit in two ring slots");
  static_assert(ROUNDS == 1 || (T::WIDE && NT % ROUNDS == 0), "two rounds: 128-row tile");
  static_assert(BM % (RPI * NW) == 0, "staged rows split evenly over the waves");
  auto write_piece = [&](OAcc* oo, float scale, bool whole_, long long row, float lse_v, int b_,
                         int slot_) {
    auto tile_fence = [&](int nt) {
      if constexpr (T::WIDE) {
        if (nt % (NT / ROUNDS) == 0) agpr_fence_one<18>(oo[nt]);
        else agpr_fence_one<0>(oo[nt]);
      }
    };
    const bool lse_writer = dg == 0 && lane < R && my_row < M;
    if (lse_writer) {
      if (whole_) lse[row] = lse_v;
      else lse_part[row] = lse_v;
    }
    // dims held by this lane: 4 consecutive dims per group of 4 accumulators
    auto dim_of = [&](int nt, int qd) {
      const int nb = dg * NT + nt;
      return R == 32 ? 32 * nb + 8 * qd + 4 * (lane >> 5) : 16 * nb + 4 * (lane >> 4);
    };
    constexpr int QUADS = OREGS / 4;
    char MLA_LDS* sA = slot_of(cstage - 2);
    char MLA_LDS* sB = slot_of(cstage - 1);
    auto srow = [&](int r) {
      return r < kRowsPerSlot ? sA + r * kStagePitch : sB + (r - kRowsPerSlot) * kStagePitch;
    };
    // The tile's destination rows: those of a partial, and with one KV head
    // those of out, are consecutive (tile row l at byte 1024 l of a buffer
    // that ends at the tile's last valid row, so rows past M store nothing).
    // With several KV heads a whole sequence's rows are found one by one.
    const int valid_rows = M - m_lo < BM ? M - m_lo : BM;
    const uint16_t* dbase = whole_ ? out + ((long long)b_ * a.s_q * a.h_q + m_lo) * kValueDim
                                   : o_part + (((long long)slot_ * a.h_kv + g) * M + m_lo) * kValueDim;
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(dbase, valid_rows * kValueDim * 2);
    // this lane's part of a store: row lane / LPR of the group, 16 bytes c
    // (opaque to the compiler, which would otherwise compute every store's
    // offset once, before the loop over pieces, and keep them all in
    // registers)
    const int c = lane % LPR;
    unsigned lds_lane = (lane / LPR) * kStagePitch + 16 * c;
    unsigned glb_lane = (lane / LPR) * kValueDim * 2 + 16 * c;
    asm volatile("" : "+v"(lds_lane), "+v"(glb_lane));
    static_for<ROUNDS>([&](auto rc) {
      constexpr int rd = decltype(rc)::value;
      // every wave is past the slots (the last stages' reads, or the
      // previous round's row stores)
      block_barrier();
      char MLA_LDS* p = srow(rg * R + lr) - 2 * rd * DR;
#pragma unroll
      for (int nt = rd * NT / ROUNDS; nt < (rd + 1) * NT / ROUNDS; ++nt) {
        tile_fence(nt);
#pragma unroll
        for (int qd = 0; qd < QUADS; ++qd) {
          const i32x2 pk = {(int)E::pack(oo[nt][4 * qd + 0] * scale, oo[nt][4 * qd + 1] * scale),
                            (int)E::pack(oo[nt][4 * qd + 2] * scale, oo[nt][4 * qd + 3] * scale)};
          *reinterpret_cast<i32x2 MLA_LDS*>(p + 2 * dim_of(nt, qd)) = pk;
        }
      }
      block_barrier();  // the round's rows are staged
      // store instruction k of wave w: tile rows l0 = (w + k NW) RPI and on
#pragma unroll
      for (int k = 0; k < BM / (RPI * NW); ++k) {
        const int l0 = (w + k * NW) * RPI;
        const i32x4 v = *reinterpret_cast<const i32x4 MLA_LDS*>(srow(l0) + lds_lane);
        if constexpr (QG) {
          if (whole_) {  // rows of several KV heads: out row of query row m
            const int m = m_lo + l0 + lane / LPR;
            const int t = m / hpg;
            const int h = g * hpg + (m - t * hpg);
            if (m < M)
              *reinterpret_cast<i32x4*>(out + (((long long)b_ * a.s_q + t) * a.h_q + h) * kValueDim +
                                        rd * DR + 8 * c) = v;
            continue;
          }
        }
        // (the whole offset goes in the checked per-lane offset)
        __builtin_amdgcn_raw_buffer_store_b128(v, drs, glb_lane + (unsigned)(l0 * kValueDim * 2 + rd * DR * 2), 0, 0);
      }
    });
  };
  // 16-row tiles hold the normalised output of the first piece that is not
  // the part's last in registers and write it after the last piece: stores
  // issued between pieces would be waited for by the next stage's vmcnt wait
  // (the counter covers stores as well as loads).  32-row tiles have too few
  // spare registers (the 4-wave tile measured slower with it).
  constexpr bool DEFER = R == 16;
  OAcc o_def[DEFER ? NT : 1];
  bool def_pending = false;  // uniform over the workgroup
  bool def_whole = false;
  long long def_row = 0;
  float def_lse = 0.f;
  int def_b = 0, def_slot = 0;

  for (int j = 0; j < npieces; ++j) {
    const int b = bb + j;
    const int N = piece_n(j);
    const int lo = (j == 0) ? tb : 0;
    const int hi = (b == be) ? te : N;
    const int nst = hi > lo ? (hi - lo + kStage - 1) / kStage : 0;
    const bool whole = lo == 0 && hi == N;  // the piece is the whole sequence
    const int slot = j == 0 ? slot_first : slot_last;  // partial slot (pieces of split sequences)
    int row_lim = a.causal ? N - a.s_q + q_t + 1 : N;
    if (row_lim > N) row_lim = N;
    // keys every row of the workgroup sees (row t = 0 has the fewest)
    const int lim_all = a.causal ? N - a.s_q + 1 : N;

    OAcc o[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[nt] = OAcc{};
    if constexpr (T::WIDE) agpr_fence_write(o);
    float m_run = kMinit, l_run = 0.f, lr_run = 0.f;

    // Mask the raw scores of key stage sp (keys past the end, or past the
    // row's causal limit).  The scale (positive) is applied later: to the
    // row max, and inside the exponent's fma.
    auto prep = [&](float* x, int sp) {
      const int tok0 = lo + sp * kStage;
      const int nvalid = N - tok0 < kStage ? N - tok0 : kStage;
      const bool full = tok0 + kStage <= lim_all;  // no key of the stage is masked
      if (!full) {
        const int lim = ((row_lim - tok0 < nvalid) ? row_lim - tok0 : nvalid) - key_lane;
#pragma unroll
        for (int i = 0; i < SREGS; ++i) x[i] = key_reg(i) < lim ? x[i] : -INFINITY;
      }
    };
    // Online softmax of one stage's scores x, cut into slices so that it can
    // be interleaved with the next stage's score MFMAs (the slices have no
    // branches).  The running max is raised only when some row's max exceeds
    // it by more than kTau; alpha is then the factor O must be scaled by
    // (1 otherwise).
    constexpr int kExpSlices = SREGS / 4;
    constexpr int kSoftSlices = 3 + kExpSlices;
    struct SoftState {
      float mx, alpha, sum, rsum;
      bool rescale;
      uint32_t pw[SREGS / 2];
    };
    auto soft_slice = [&](const float* x, SoftState& st, int slice) {
      if (slice == 0) {
        float mx = x[0];
#pragma unroll
        for (int i = 1; i < SREGS; ++i) mx = fmaxf(mx, x[i]);
        st.mx = mx;
      } else if (slice == 1) {
        if constexpr (R == 16) st.mx = max_xor16(st.mx);
        st.mx = max_xor32(st.mx) * a.scale_log2;  // = the max of the scaled scores (scale > 0)
      } else if (slice == 2) {
        const bool rs = __any(st.mx > m_run + kTau);
        const float m_new = fmaxf(m_run, st.mx);
        const float al = rs ? fast_exp2(m_run - m_new) : 1.f;
        m_run = rs ? m_new : m_run;
        l_run *= al;
        lr_run *= al;
        st.rescale = rs;
        st.alpha = al;
        st.sum = 0.f;
        st.rsum = 0.f;
      } else if (slice < kSoftSlices) {
        const int e0 = 4 * (slice - 3);
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float p0 = fast_exp2(__builtin_fmaf(x[e0 + i], a.scale_log2, -m_run));
          const float p1 = fast_exp2(__builtin_fmaf(x[e0 + i + 1], a.scale_log2, -m_run));
          const uint32_t pk = E::pack(p0, p1);
          st.pw[(e0 + i) >> 1] = pk;
          st.sum += p0 + p1;
          st.rsum = E::dot2(pk, E::kOnePair, st.rsum);
        }
        if (slice == kSoftSlices - 1) {
          l_run += st.sum;
          lr_run += st.rsum;
        }
      }
    };
    // O^T += V^T P^T for key stage sp held in ring slot `st`; loads of the
    // stage in flight are fired at issue points first_slot.. (none if < 0).
    auto pv = [&](const uint32_t* pw, bool rescale, float alpha, int sp, const char MLA_LDS* st,
                  int first_slot) {
      (void)sp;
      // (WIDE: O is still zero before the first stage of a piece; its 256
      // accumulators live in AGPRs, where a rescale costs two moves each.)
      if (rescale && (!T::WIDE || sp > 0)) {
        if constexpr (T::WIDE) {
          // one tile at a time through VGPRs (16 registers, not 256)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            if (nt == 0) agpr_fence_one<18>(o[nt]);
            else agpr_fence_one<0>(o[nt]);
            acc_scale<OREGS>(o[nt], alpha);
            if (nt == NT - 1) agpr_fence_one<2>(o[nt]);
            else agpr_fence_one<0>(o[nt]);
          }
        } else {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc_scale<OREGS>(o[nt], alpha);
        }
      }
      if constexpr (R == 32) {
        const i16x8 pb[2] = {__builtin_bit_cast(i16x8, i32x4{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]}),
                             __builtin_bit_cast(i16x8, i32x4{(int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]})};
        constexpr int NV = 2 * NT;
        constexpr int VP = MLA_VP32;
        // keys 16 kb + 4 h + r (low half) and 16 kb + 8 + 4 h + r (high half)
        auto vread = [&](int idx) {
          const int kb = idx / NT, nb = dg * NT + idx % NT;
          const char MLA_LDS* p = st + 128 * (nb >> 1) + 16 * kb * kRowBytes;
          const i16x4 v0 = lds_read_tr(p + voff[2 * (nb & 1)]);
          const i16x4 v1 = lds_read_tr(p + voff[2 * (nb & 1) + 1] + 8 * kRowBytes);
          return cat(v0, v1);
        };
        i16x8 va[VP];
#pragma unroll
        for (int j2 = 0; j2 < VP; ++j2) va[j2] = vread(j2);
#pragma unroll
        for (int idx = 0; idx < NV; ++idx) {
          const int kb = idx / NT, nt = idx % NT;
          if constexpr (T::WIDE) mfma32_agpr<E>(o[nt], va[idx % VP], pb[kb]);
          else o[nt] = E::mfma32(va[idx % VP], pb[kb], o[nt]);
          if (idx + VP < NV) va[idx % VP] = vread(idx + VP);
          if (first_slot >= 0) fire_slot(first_slot + idx);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        const i16x8 pb = __builtin_bit_cast(i16x8, i32x4{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]});
        constexpr int VP = NT < MLA_VP16 ? NT : MLA_VP16;
        auto vread = [&](int nt) {
          const int nb = dg * NT + nt;
          const char MLA_LDS* p = st + voff[nb & 3] + 128 * (nb >> 2);
          return cat(lds_read_tr(p), lds_read_tr(p + 16 * kRowBytes));
        };
        i16x8 va[VP];
#pragma unroll
        for (int j2 = 0; j2 < VP; ++j2) va[j2] = vread(j2);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          o[nt] = E::mfma16(va[nt % VP], pb, o[nt]);
          if (nt + VP < NT) va[nt % VP] = vread(nt + VP);
          if (first_slot >= 0) fire_slot(first_slot + nt);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

    // Full scores of a stage from the exchange buffer `xb`, which holds every
    // wave's partial scores; the terms are added in a fixed order (k-share 0
    // then 1), so the waves of a row group get identical scores.
    auto gather = [&](const char MLA_LDS* xb, float* sc) {
      if constexpr (R == 32) {
        const char MLA_LDS* p0 = xb + (rg * DG + 0) * 4096 + lane * 16;
        const char MLA_LDS* p1 = xb + (rg * DG + 1) * 4096 + lane * 16;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x4 u = lds_read_f4(p0 + qd * 1024), v = lds_read_f4(p1 + qd * 1024);
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[4 * qd + e] = u[e] + v[e];
        }
      } else if constexpr (KB_W == 2) {
        const char MLA_LDS* p0 = xb + (rg * DG + 0) * 2048 + lane * 16;
        const char MLA_LDS* p1 = xb + (rg * DG + 1) * 2048 + lane * 16;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const f32x4 u = lds_read_f4(p0 + t * 1024), v = lds_read_f4(p1 + t * 1024);
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[4 * t + e] = u[e] + v[e];
        }
      } else {
        // DG = 4: wave dg holds key block dg / 2, k-share dg % 2
        const char MLA_LDS* base = xb + rg * DG * 1024 + lane * 16;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const f32x4 u = lds_read_f4(base + (2 * t) * 1024), v = lds_read_f4(base + (2 * t + 1) * 1024);
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[4 * t + e] = u[e] + v[e];
        }
      }
    };

    // One iteration of the key-stage pipeline.  HP: finish the previous stage
    // sp = s - 1 (its partial scores are in xrd, its keys in ring slot prev);
    // HC: compute this wave's partial scores of stage s (ring slot rd) into
    // xwr.  The score MFMAs of stage s and the softmax of stage s - 1 are
    // independent and are scheduled into one region.
    auto kv_step = [&](auto hp, auto hc, const char MLA_LDS* __restrict__ rd,
                       const char MLA_LDS* __restrict__ prev, char MLA_LDS* __restrict__ xwr,
                       const char MLA_LDS* __restrict__ xrd, int s) {
      constexpr bool HP = decltype(hp)::value, HC = decltype(hc)::value;
      float x[SREGS];
      if constexpr (HP) {
        gather(xrd, x);
        if constexpr (T::XCH_BUFS == 1 && HC) block_barrier();  // every wave has read them
        prep(x, s - 1);
      }
      constexpr int NK = KS_W * KB_W;
      constexpr int KP = NK < (R == 32 ? MLA_KP32 : MLA_KP16) ? NK : (R == 32 ? MLA_KP32 : MLA_KP16);
      auto kaddr = [&](int i) {
        if constexpr (R == 32) return rd + kstep_off(i);
        else {
          const int kb = KB_W == 2 ? (i & 1) : kbs;
          return rd + kb * 16 * kRowBytes + kstep_off(i / KB_W);
        }
      };
      using SAcc = typename std::conditional<R == 32, f32x16, f32x4>::type;
      SAcc sacc[R == 32 ? 1 : KB_W];
      SoftState ss;
      if constexpr (HC) {
        static_assert(NK >= kSoftSlices, "softmax slices fit between the score MFMAs");
        i16x8 kf[KP];
#pragma unroll
        for (int i = 0; i < KP; ++i) kf[i] = lds_read_b128(kaddr(i));
#pragma unroll
        for (int t = 0; t < (R == 32 ? 1 : KB_W); ++t) sacc[t] = SAcc{};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NK; ++i) {
          if constexpr (R == 32) sacc[0] = E::mfma32(kf[i % KP], qf[i], sacc[0]);
          else sacc[i % KB_W] = E::mfma16(kf[i % KP], qf[i / KB_W], sacc[i % KB_W]);
          if (i + KP < NK) kf[i % KP] = lds_read_b128(kaddr(i + KP));
          fire_slot(i);
          if constexpr (HP) soft_slice(x, ss, i);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < kSoftSlices; ++i) soft_slice(x, ss, i);
      }
      if constexpr (HC) {
        if constexpr (R == 32) {
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            lds_write_f4(xwr + w * 4096 + qd * 1024 + lane * 16,
                         f32x4{sacc[0][4 * qd], sacc[0][4 * qd + 1], sacc[0][4 * qd + 2], sacc[0][4 * qd + 3]});
        } else {
#pragma unroll
          for (int t = 0; t < KB_W; ++t) lds_write_f4(xwr + (w * KB_W + t) * 1024 + lane * 16, sacc[t]);
        }
      }
      if constexpr (HP) pv(ss.pw, ss.rescale, ss.alpha, s - 1, prev, HC ? T::QK_MFMA : -1);
      else fire_from(T::QK_MFMA);
    };

    // WIDE tiles: one iteration finishes stage s - 1 (softmax of its scores,
    // held in sprev, then P V with its keys in ring slot `prev`) while the
    // score MFMAs of stage s (ring slot rd) run.  The first WA score MFMAs
    // carry the softmax slices, spread evenly (a slice holds more VALU
    // work than one MFMA hides); the remaining score MFMAs (one dependent
    // chain) are spread between the 32 independent P V MFMAs.  The K and V
    // fragments of all 68 MFMAs are read through one queue of QD fragments
    // in the order the MFMAs use them, so every LDS read is issued QD MFMAs
    // before its use.  The stage's loads are all issued before its first LDS
    // read (an LDS-DMA load issued while the wave has LDS reads outstanding
    // waits for them).
    f32x16 sprev = f32x16{};
    auto wide_vread = [&](const char MLA_LDS* st, int idx) {
      // keys 16 kb + 4 h + r (low half) and 16 kb + 8 + 4 h + r (high half)
      const int kb = idx / NT, nb = idx % NT;
      const char MLA_LDS* p = st + 128 * (nb >> 1) + 16 * kb * kRowBytes;
      const i16x4 v0 = lds_read_tr(p + voff[2 * (nb & 1)]);
      const i16x4 v1 = lds_read_tr(p + voff[2 * (nb & 1) + 1] + 8 * kRowBytes);
      return cat(v0, v1);
    };
    constexpr int W_NK = T::WIDE ? KS_W : 1;   // score MFMAs
    constexpr int W_NV = 2 * NT;               // P V MFMAs
    constexpr int W_WA = 30;                   // score MFMAs before the first P V MFMA
    constexpr int W_NQR = W_NK - W_WA;
    constexpr int W_NSTEP = W_NK + W_NV;
    // WIDE softmax of the previous stage's scores, spread over the first
    // W_WA score MFMAs with at most four VALU instructions after each (a
    // wave hides about that many under one MFMA; a whole slice of dependent
    // instructions after a single MFMA stalls the issue of the next one).
    // Every instruction's inputs come from an earlier step, except within
    // the max tree:
    //   steps 0-3  row max (a max3 tree), the cross-lane max, the scale;
    //   steps 4-6  the rescale decision, alpha, the running max and sums;
    //   steps 8-27 element i: exponent fma at step 8 + i, exp2 at 9 + i,
    //              fp32 sum (two alternating partial sums) at 10 + i; pair
    //              k = (2k, 2k + 1) rounded to the MFMA type at 11 + 2k and
    //              added to the rounded-weight sum (two partial sums) at
    //              12 + 2k;
    //   step 27    the running sums.
    // The rescale of O, when the running max rises, follows at step 7.
    struct WSoft {
      float m[5], ma, mb, mx, mn, al, th;
      bool rs;
      float f[SREGS], e[SREGS];
      float s[2], r[2];
      uint32_t pw[SREGS / 2];
    };
    constexpr int WS_LAST = 27;
    auto wide_soft = [&](auto gc, const float* x, WSoft& q) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g == 0) {
        q.m[0] = fmaxf(fmaxf(x[0], x[1]), x[2]);
        q.m[1] = fmaxf(fmaxf(x[3], x[4]), x[5]);
        q.m[2] = fmaxf(fmaxf(x[6], x[7]), x[8]);
        q.th = m_run + kTau;
      } else if constexpr (g == 1) {
        q.m[3] = fmaxf(fmaxf(x[9], x[10]), x[11]);
        q.m[4] = fmaxf(fmaxf(x[12], x[13]), x[14]);
        q.ma = fmaxf(fmaxf(q.m[0], q.m[1]), q.m[2]);
      } else if constexpr (g == 2) {
        q.mb = fmaxf(fmaxf(q.m[3], q.m[4]), x[15]);
      } else if constexpr (g == 3) {
        q.mx = max_xor32(fmaxf(q.ma, q.mb)) * a.scale_log2;  // the max of the scaled scores (scale > 0)
      } else if constexpr (g == 4) {
        q.rs = __any(q.mx > q.th);
        q.mn = fmaxf(m_run, q.mx);
      } else if constexpr (g == 5) {
        q.al = q.rs ? fast_exp2(m_run - q.mn) : 1.f;
      } else if constexpr (g == 6) {
        m_run = q.rs ? q.mn : m_run;
        l_run *= q.al;
        lr_run *= q.al;
      } else if constexpr (g >= 8 && g <= WS_LAST) {
        constexpr int i = g - 8;
        if constexpr (i <= SREGS - 1) q.f[i] = __builtin_fmaf(x[i], a.scale_log2, -m_run);
        if constexpr (i >= 1 && i <= SREGS) q.e[i - 1] = fast_exp2(q.f[i - 1]);
        if constexpr (i >= 2 && i <= SREGS + 1) {
          if constexpr (i - 2 < 2) q.s[(i - 2) & 1] = q.e[i - 2];
          else q.s[(i - 2) & 1] += q.e[i - 2];
        }
        if constexpr (i >= 3 && (i - 3) % 2 == 0 && (i - 3) / 2 < SREGS / 2) {
          constexpr int k = (i - 3) / 2;
          q.pw[k] = E::pack(q.e[2 * k], q.e[2 * k + 1]);
        }
        if constexpr (i >= 4 && (i - 4) % 2 == 0 && (i - 4) / 2 < SREGS / 2) {
          constexpr int k = (i - 4) / 2;
          q.r[k & 1] = E::dot2(q.pw[k], E::kOnePair, k < 2 ? 0.f : q.r[k & 1]);
        }
        if constexpr (g == WS_LAST) {
          l_run += q.s[0] + q.s[1];
          lr_run += q.r[0] + q.r[1];
        }
      }
    };
    auto wide_step = [&](auto hp, auto hc, const char MLA_LDS* __restrict__ rd,
                         const char MLA_LDS* __restrict__ prev, int s) {
      if constexpr (T::WIDE) {
        constexpr bool HP = decltype(hp)::value, HC = decltype(hc)::value;
        constexpr int QD = MLA_QD32;  // fragment queue depth
        static_assert(W_WA > WS_LAST && W_WA < W_NK, "the softmax fits before the P V MFMAs");
        static_assert(SREGS == 16 && 8 + SREGS + 3 <= WS_LAST, "the softmax steps cover every score");
        float x[SREGS];
        if constexpr (HP) {
#pragma unroll
          for (int i = 0; i < SREGS; ++i) x[i] = sprev[i];
          prep(x, s - 1);
        }
        SoftState ss;
        WSoft ws;
        if constexpr (HC) {
          constexpr int NS = HP ? W_NSTEP : W_NK;  // without a previous stage: scores only
          // step g: a score MFMA (k-step qk(g)) or P V MFMA pv(g)
          constexpr auto is_qk = [](int g) { return !HP || wide_is_qk(g, W_WA, W_NQR, W_NV); };
          constexpr auto qk = [](int g) { return HP ? wide_qk_of(g, W_WA, W_NQR, W_NV) : g; };
          constexpr auto pv = [](int g) { return wide_pv_of(g, W_WA, W_NQR, W_NV); };
          auto read_frag = [&](auto gc) -> i16x8 {
            constexpr int g = decltype(gc)::value;
            if constexpr (is_qk(g)) return lds_read_b128(rd + kstep_off(qk(g)));
            else return wide_vread(prev, pv(g));
          };
          i16x8 fq[QD];
          static_for<QD>([&](auto gc) { fq[decltype(gc)::value] = read_frag(gc); });
          f32x16 acc = f32x16{};
          i16x8 qrf[T::QR_STEPS];
          i16x8 pb[2];
          __builtin_amdgcn_sched_barrier(0);
          static_for<NS>([&](auto gc) {
            constexpr int g = decltype(gc)::value;
            if constexpr (is_qk(g)) {
              constexpr int i = qk(g);
              if constexpr (i >= T::QREG_STEPS - 2 && i + 2 < W_NK)  // rope fragment i + 2, two score MFMAs ahead
                qrf[i + 2 - T::QREG_STEPS] = lds_read_b128(qr0 + 1024 * (i + 2 - T::QREG_STEPS));
              if constexpr (i < T::QREG_STEPS) acc = E::mfma32(fq[g % QD], qf[i], acc);
              else acc = E::mfma32(fq[g % QD], qrf[i - T::QREG_STEPS], acc);
            } else {
              constexpr int pi = pv(g);
              mfma32_agpr<E>(o[pi % NT], fq[g % QD], pb[pi / NT]);
            }
            if constexpr (g + QD < NS) fq[g % QD] = read_frag(std::integral_constant<int, g + QD>{});
            if constexpr (HP) {
              if constexpr (g <= WS_LAST) wide_soft(gc, x, ws);
              // Right after the running max is decided: rescale O if it rose
              // (O is still zero before the first stage of a piece).
              if constexpr (g == 7) {
                if (ws.rs && s - 1 > 0) {
#pragma unroll
                  for (int nt = 0; nt < NT; ++nt) {
                    if (nt == 0) agpr_fence_one<18>(o[nt]);
                    else agpr_fence_one<0>(o[nt]);
                    acc_scale<OREGS>(o[nt], ws.al);
                    if (nt == NT - 1) agpr_fence_one<2>(o[nt]);
                    else agpr_fence_one<0>(o[nt]);
                  }
                }
              }
              if constexpr (g == W_WA - 1) {  // the softmax is complete: P as MFMA operands
                pb[0] = __builtin_bit_cast(i16x8, i32x4{(int)ws.pw[0], (int)ws.pw[1], (int)ws.pw[2], (int)ws.pw[3]});
                pb[1] = __builtin_bit_cast(i16x8, i32x4{(int)ws.pw[4], (int)ws.pw[5], (int)ws.pw[6], (int)ws.pw[7]});
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          });
          sprev = acc;
        } else if constexpr (HP) {
#pragma unroll
          for (int i = 0; i < kSoftSlices; ++i) soft_slice(x, ss, i);
          pv(ss.pw, ss.rescale, ss.alpha, s - 1, prev, -1);
        }
      }
    };

    if (nst > 0) {
      // DQ tiles: a vector-memory wait the compiler can see (a builtin, not
      // asm) at the start of each piece: the Q^T registers are then known to
      // be loaded, and the compiler puts no wait of its own into the stage
      // loop (there it drained the prefetched stages in every iteration).
      // Piece 0 of a 16-row tile needs none (its Q^T was waited for with the
      // page list).  Every later piece loaded its Q^T after its first two
      // positions and starts after the drain at the end of the previous
      // piece (which also keeps the compiler's view of the loop's back edge
      // free of loads in flight).  Tiles with query stages stream them here
      // (position cstage on).
      if constexpr (T::DQ) {
        if (!(Q_EARLY && j == 0)) {
          if (q_piece != j) load_q(j);
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        }
      }
      for (int jq = 0; jq < T::NQS; ++jq, ++cstage) {
        stage_ready();
        [&](const char MLA_LDS* __restrict__ rd, char MLA_LDS* __restrict__ wr) {
          plan(wr);
          fire_all();
          if (jq == q_stage) {
            const char MLA_LDS* qs = rd + q_row0 * kRowBytes;
#pragma unroll
            for (int ks = 0; ks < T::QREG_STEPS; ++ks) qf[ks] = lds_read_b128(qs + kstep_off(ks));
          }
        }(slot_of(cstage), slot_of(cstage + 2));
      }
      using F = std::false_type;
      using Tr = std::true_type;
      if constexpr (T::WIDE) {
        stage_ready();
        plan(slot_of(cstage + 2));
        fire_all();
        wide_step(F{}, Tr{}, slot_of(cstage), slot_of(cstage - 1), 0);
        ++cstage;
        for (int s = 1; s < nst; ++s, ++cstage) {
          stage_ready();
          plan(slot_of(cstage + 2));
          fire_all();
          wide_step(Tr{}, Tr{}, slot_of(cstage), slot_of(cstage - 1), s);
        }
        // The score MFMAs of the piece are done: the next piece's Q^T.
        if (j + 1 < npieces) load_q(j + 1);
        // drain: finish the last stage (its scores are in registers)
        wide_step(Tr{}, F{}, slot_of(cstage), slot_of(cstage - 1), nst);
      } else {
      // stage 0: scores only
      stage_ready();
      plan(slot_of(cstage + 2));
      kv_step(F{}, Tr{}, slot_of(cstage), slot_of(cstage - 1), xch0, xch0, 0);
      ++cstage;
      for (int s = 1; s < nst; ++s, ++cstage) {
        stage_ready();
        plan(slot_of(cstage + 2));
        char MLA_LDS* xw = xch0 + (T::XCH_BUFS == 2 ? (s & 1) * T::XCH_ONE : 0);
        const char MLA_LDS* xr = xch0 + (T::XCH_BUFS == 2 ? ((s + 1) & 1) * T::XCH_ONE : 0);
        kv_step(Tr{}, Tr{}, slot_of(cstage), slot_of(cstage - 1), xw, xr, s);
      }
      // The score MFMAs of the piece are done: the next piece's Q^T.
      if (T::DQ && j + 1 < npieces) load_q(j + 1);
      // drain: the last stage's partials are exchanged; finish it
      block_barrier();
      const char MLA_LDS* xr = xch0 + (T::XCH_BUFS == 2 ? ((nst - 1) & 1) * T::XCH_ONE : 0);
      kv_step(Tr{}, F{}, slot_of(cstage), slot_of(cstage - 1), nullptr, xr, nst);
      }
    }

    // ---- epilogue: normalise and write this piece --------------------------
    float lt = l_run, ltr = lr_run;
    if constexpr (R == 32) {
      lt = sum_xor32(lt);
      ltr = sum_xor32(ltr);
    } else {
      lt = sum_xor32(sum_xor16(lt));
      ltr = sum_xor32(sum_xor16(ltr));
    }
    const bool empty = !(lt > 0.f);
    const float inv = empty ? 0.f : 1.f / ltr;
    const float lse_row = empty ? -INFINITY : (m_run + fast_log2(lt)) * kLn2;
    const long long row = whole ? ((long long)b * a.s_q + q_t) * a.h_q + q_h
                                : ((long long)slot * a.h_kv + g) * M + my_row;
    if constexpr (DEFER) {
      if (j < npieces - 1 && !def_pending) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < OREGS; ++i) o_def[nt][i] = o[nt][i] * inv;
        def_pending = true;
        def_whole = whole;
        def_row = row;
        def_lse = lse_row;
        def_b = b;
        def_slot = slot;
        if constexpr (T::DQ) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): see the start of a piece
        continue;
      }
    }
    write_piece(o, inv, whole, row, lse_row, b, slot);
    if constexpr (T::DQ) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): see the start of a piece
  }
  if constexpr (DEFER) {
    if (def_pending) write_piece(o_def, 1.f, def_whole, def_row, def_lse, def_b, def_slot);
  }
  // Out-of-range loads past the end of the stream may still be in flight:
  // they must land before the workgroup's LDS is released.
  wait_vmcnt<0>();
}

}  // namespace mla
