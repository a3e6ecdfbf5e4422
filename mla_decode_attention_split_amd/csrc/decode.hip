// Main paged MLA decode kernel for gfx950 (CDNA4).
//
// What it computes (cnblogs FlashMLA notes, sections 2 and 4): for every query
// row, blockwise scores against the 576-wide cached latent rows of its
// sequence, softmax, and the weighted sum of the first 512 dims of the same
// rows (Shared-KV); pages of 64 tokens are found through block_table
// (ygpos news: paged cache with block size 64, BF16).  Each workgroup handles
// one part of the split-KV partition (pieces of one or more sequences) for one
// tile of query rows; a sequence cut into several pieces leaves fp32 partial
// outputs plus their log-sum-exp for the combine kernel (section 4, merge of
// partial outputs).
//
// Design (gfx950):
//   * One workgroup per CU: 4 waves for tiles of up to 64 query rows, 8 waves
//     (two per SIMD) for 128-row tiles.  The part's stages (query rows, then
//     32-key blocks, per piece) stream through a ring of 4 (8 waves: 3) LDS
//     slots of 36 KB with 16-byte buffer loads straight into LDS.  Every ring
//     position is loaded with the same number of instructions per wave; lanes
//     with nothing to load address past their buffer's range, which costs no
//     memory traffic, so the per-stage waits are exact constants.
//   * The prologue needs one memory trip after the part's metadata record:
//     the record carries the lengths and partial slots of the part's first
//     and last sequence, and the page indices of the part are loaded into
//     registers (lane i holds entry i) while the query stage is already in
//     flight.
//   * Each wave owns R query rows (R = 16 or 32) and 512 / DG value dims.
//     Scores are computed transposed, S^T = K Q^T, with K from LDS (A
//     operand) and Q^T resident in registers (B operand); the MFMA result is
//     already laid out as the B operand P^T of O^T = V^T P^T.  V^T comes from
//     LDS through transposed 8-byte reads (ds_read_b64_tr_b16).
//   * Split-K scores: the DG waves of a row group each contract an interleaved
//     share of the 576 dims (and, with DG = 4, one of the two 16-key blocks),
//     then exchange fp32 partial scores through LDS and add them in a fixed
//     order, so every wave of the group holds bit-identical scores.
//   * Software pipeline (4-wave tiles): in the iteration of key block s a
//     wave computes the partial scores of block s while it finishes block
//     s - 1 (partial-score sum, softmax, P V); the MFMAs of one overlap the
//     vector work of the other, and one barrier per stage serves both the ring
//     and the exchange.  8-wave tiles have no registers for that; they run
//     each stage in order and rely on the second wave of the SIMD instead,
//     and keep the Q^T fragments of the rope dims in LDS.
//   * Softmax in fp32 in the log2 domain; the running max is raised only when
//     a row's new max exceeds it by more than kTau (then O and l are
//     rescaled).  P is rounded to bf16 for the MFMA and a second row sum adds
//     the rounded values, so the output is normalised by exactly the weights
//     that multiplied V.
#include <type_traits>

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

__device__ __forceinline__ i16x8 cat(i16x4 a, i16x4 b) {
  return i16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Tile shape.  R rows per wave (32x32x16 MFMA for R = 32, 16x16x32 for
// R = 16), RG row groups x DG value-dim groups = 4 or 8 waves.
template <int R, int RG, int DG>
struct Tile {
  static constexpr int NW = RG * DG;
  static constexpr int BM = R * RG;                      // query rows per workgroup
  // 16-byte loads per lane per stage; with 8 waves the last load is issued
  // by the first LAST_WAVES waves only (36 = 4 x 8 + 4)
  static constexpr int LPW = (kLoadsPerStage + NW - 1) / NW;
  static constexpr int LAST_WAVES = kLoadsPerStage - (LPW - 1) * NW;
  static constexpr int KSTEPS = R == 32 ? 36 : 18;       // score k-steps over 576 dims
  static constexpr int KSPLIT = 2;                       // k-step interleave among DG waves
  static constexpr int KBSPLIT = DG / KSPLIT;            // 16-key blocks split among waves (R = 16)
  static constexpr int KS_W = KSTEPS / KSPLIT;           // k-steps per wave
  static constexpr int KB_W = R == 32 ? 1 : 2 / KBSPLIT; // score blocks per wave
  static constexpr int NT = (R == 32 ? 16 : 32) / DG;    // value-dim tiles per wave
  static constexpr int OREGS = R == 32 ? 16 : 4;         // accumulator registers per tile
  static constexpr int PARTIAL_BYTES = R == 32 ? 4096 : 1024;  // one score block, fp32
  static constexpr int XCH_ONE = NW * KB_W * PARTIAL_BYTES;    // one exchange buffer
  // 16-row tiles double-buffer the exchange; 32-row tiles have room for one
  // buffer and separate its reads from the next writes with a barrier.
  static constexpr int XCH_BUFS = (R == 32 || NW == 8) ? 1 : 2;
  // 8-wave 32-row tiles (128 rows, two waves per SIMD) are not software
  // pipelined: each stage's scores, softmax and P V run in order, and the
  // other wave of the SIMD fills the gaps.  Their ring has 3 slots (stage s
  // is computed while s + 1 and s + 2 load), which leaves room for the
  // 8-wave exchange buffer.
  static constexpr bool FLAT = NW == 8 && R == 32;
  static constexpr int SLOTS = FLAT ? 3 : kSlots;
  static constexpr int RING_BYTES = SLOTS * kStageBytes;
  // FLAT tiles keep the Q^T fragments of the rope dims (the last QR_STEPS
  // k-steps of each wave) in LDS instead of registers
  static constexpr int QR_STEPS = FLAT ? 2 : 0;
  static constexpr int QREG_STEPS = KS_W - QR_STEPS;     // Q^T k-steps held in registers
  static constexpr int QR_BYTES = NW * QR_STEPS * 1024;
  static constexpr int NQ = (BM + kStage - 1) / kStage;  // query stages per piece
  static constexpr int QK_MFMA = KS_W * KB_W;
  static constexpr int PV_MFMA = R == 32 ? 2 * NT : NT;
  static constexpr int NSLOT = QK_MFMA + PV_MFMA;        // points where loads are issued
  static_assert(NW == 4 || NW == 8, "four or eight waves per workgroup");
  static_assert(DG >= 2 && DG % 2 == 0, "split-K tiles only");
  static_assert(LAST_WAVES > 0 && LAST_WAVES <= NW, "stage loads split over the waves");
  static_assert(KS_W * KSPLIT == KSTEPS && KBSPLIT * KSPLIT == DG, "score split");
  static_assert(R == 16 || KBSPLIT == 1, "key-block split only for 16-row tiles");
  static_assert(NSLOT >= LPW, "one load per issue point at most");
  static_assert(2 * LPW < 63, "vector memory counter capacity");
  static_assert(RING_BYTES + XCH_BUFS * XCH_ONE + QR_BYTES <= 163840, "LDS capacity");
};

template <int R, int RG, int DG, bool QG, typename E>
__global__ __launch_bounds__(64 * RG * DG, 1) void decode_kernel(
    const uint16_t* __restrict__ q_ptr, const uint16_t* __restrict__ kv_ptr,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seqlens,
    const int32_t* __restrict__ meta, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ o_part, float* __restrict__ lse_part, DecodeArgs a) {
  using T = Tile<R, RG, DG>;
  constexpr int NW = T::NW, BM = T::BM, LPW = T::LPW, KS_W = T::KS_W, KB_W = T::KB_W;
  constexpr int NT = T::NT, OREGS = T::OREGS, NQ = T::NQ;
  using OAcc = typename std::conditional<R == 32, f32x16, f32x4>::type;
  constexpr int SREGS = R == 32 ? 16 : 8;  // scores per lane per stage

  __shared__ __attribute__((aligned(1024))) char lds_raw[T::RING_BYTES + T::XCH_BUFS * T::XCH_ONE + T::QR_BYTES];
  char MLA_LDS* lds = (char MLA_LDS*)lds_raw;
  char MLA_LDS* xch0 = lds + T::RING_BYTES;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  // this wave's Q^T rope fragments (FLAT tiles): step j at qr0 + 1024 j
  char MLA_LDS* qr0 = T::FLAT ? xch0 + T::XCH_BUFS * T::XCH_ONE + w * T::QR_STEPS * 1024 + lane * 16 : lds;
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

  // ---- the part's pages, one per lane --------------------------------------
  // Piece j (sequence bb + j) covers keys [lo_j, hi_j); its pages are entries
  // lo_j / 64 .. ceil(hi_j / 64) - 1 of the sequence's block_table row and
  // occupy positions cum_j .. cum_j + pages_j - 1 of the part's page list.
  // With one or two pieces the metadata record holds every length needed, so
  // the page loads are the prologue's only memory trip; longer parts first
  // load the lengths of their middle sequences.
  int v_n = 0;  // lane j: length of sequence bb + j (middle pieces only)
  const bool short_part = npieces <= 2;
  if (!short_part) {
    if (lane < npieces && lane < kListPieces) v_n = seqlens[bb + lane];
    asm volatile("" ::"v"(v_n));
  }
  auto piece_n = [&](int j) -> int {
    if (j == 0) return n_first;
    if (j == npieces - 1) return n_last;
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
  const bool use_list = npieces <= kListPieces && total_listed <= kListPages;
  int v_page[2] = {0, 0};
  if (use_list) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
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

  // ---- lane constants --------------------------------------------------------
  const int lr = lane % R;  // this lane's query row inside the wave tile
  const int my_row = m_lo + rg * R + lr;
  const int q_row = my_row < M ? my_row : M - 1;
  const int q_t = q_row / hpg;
  const int q_h = g * hpg + q_row % hpg;

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
  // ks = 2 j + kh.
  //   R = 32: chunk 2 ks + h (h = lane / 32) -> koff[j % 2] + 128 (j / 2)
  //   R = 16: chunk 4 ks + lane / 16         -> koff[0] + 128 j
  int koff[2];
  int voff[4];
  if constexpr (R == 32) {
    const int h = lane >> 5;
    int kbase[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) kbase[rr] = lr * kRowBytes + 16 * ((2 * rr + h) ^ swz<32>(lr));
    koff[0] = kh ? kbase[1] : kbase[0];
    koff[1] = kh ? kbase[3] : kbase[2];
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
    if constexpr (R == 32) return koff[j & 1] + 128 * (j >> 1);
    else return koff[0] + 128 * j;
  };
  // Key index (within a stage) of score register i of this lane is
  // key_lane + key_reg(i): a per-lane part and a compile-time part, so masks
  // compare against immediates.
  const int key_lane = R == 32 ? 4 * (lane >> 5) : 4 * (lane >> 4);
  auto key_reg = [](int i) -> int { return R == 32 ? 8 * (i >> 2) + (i & 3) : 16 * (i >> 2) + (i & 3); };

  // ---- stage stream -----------------------------------------------------------
  // For every non-empty piece: NQ query stages (32 rows of the tile each, same
  // swizzled row layout as the keys), then the piece's key stages.  Stream
  // position c uses ring slot c % SLOTS; position c + 2 is loaded while
  // position c is computed.  Past the end of the stream the loads are out of
  // range.
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
  bool pend_nt = false;  // the pending position's loads are non-temporal
  unsigned qoff[QG ? LPW : 1];
  // waves past LAST_WAVES skip the stage's last load
  const bool all_loads = T::LAST_WAVES == NW || w < T::LAST_WAVES;
  // Key stages load non-temporally unless other row tiles of the part read
  // the same pages; query stages never do (the pieces of a sequence split
  // over many parts all read its query rows).  The 4-wave 32-row tile
  // measured ~0.7 us slower with it on the ragged batch and keeps the
  // default policy.
  const bool nt_kv = a.m_tiles == 1 && !(R == 32 && NW == 4);
  auto fire = [&](int k) {
    if (k == LPW - 1 && !all_loads) return;
    if constexpr (QG) load_lds16(pend, pend_q ? qoff[k] : loff[k], pend_dst + k * NW * 1024, pend_nt);
    else load_lds16(pend, loff[k], pend_dst + k * NW * 1024, pend_nt);
  };
  auto fire_all = [&]() {
#pragma unroll
    for (int k = 0; k < LPW; ++k) fire(k);
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
    pend_nt = false;
    if (lvalid && lq >= NQ) {
      pend_nt = nt_kv;
      int page;
      if (use_list) page = readlane(lpos < 64 ? v_page[0] : v_page[1], lpos & 63);
      else page = sload_i32(block_table + (long long)(bb + lj) * a.max_blocks + (ltok >> 6));
      // Rows past the end of the sequence are out of the buffer's range, so
      // they arrive as zeros: their V rows then contribute exactly nothing
      // (cache memory past the end may hold anything, NaN included).
      const int rows = lhi - ltok < kStage ? lhi - ltok : kStage;
      pend = make_rsrc(kv_bytes + page * page_bytes + lhalf * half_bytes, rows * row_stride);
      lpos += lhalf;
      lhalf ^= 1;
      ltok += kStage;
      if (ltok >= lhi) next_piece();
    } else if (lvalid) {
      const int b = bb + lj;
      const char* qseq = reinterpret_cast<const char*>(q_ptr) + (long long)b * a.s_q * a.h_q * kRowBytes;
      const int m0 = m_lo + kStage * lq;
      if constexpr (QG) {
        pend = make_rsrc(qseq, a.s_q * a.h_q * kRowBytes);
        pend_q = true;
#pragma unroll
        for (int k = 0; k < LPW; ++k) {
          const int cell = (k * NW + w) * 64 + lane;
          const int row = cell / kChunksPerRow;
          const int pc = cell - row * kChunksPerRow;
          const int m = m0 + row;
          const int t = m / hpg;
          qoff[k] = m < m_hi ? (unsigned)((t * a.h_q + g * hpg + (m - t * hpg)) * kRowBytes +
                                          phys_chunk<R>(row, pc) * 16)
                             : kOutOfRange;
        }
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
  plan(lds);
  fire_all();
  plan(lds + kStageBytes);
  fire_all();

  int cstage = 0;
  auto slot_of = [&](int c) {
    if constexpr (T::SLOTS == 3) return lds + (c % 3) * kStageBytes;  // c >= 0 here
    else return lds + (c & (kSlots - 1)) * kStageBytes;
  };
  // Wait for stream position cstage (position cstage + 1 may stay in flight),
  // then a barrier: the stage and the previous iteration's partial scores are
  // visible to all waves, and the slot refilled next has been read by all.
  auto stage_ready = [&]() {
    if (all_loads) wait_vmcnt<LPW>();
    else wait_vmcnt<LPW - 1>();
    block_barrier();
  };
  // query rows of this wave inside its query stage
  const int q_stage = (rg * R) / kStage;
  const int q_row0 = (rg * R) % kStage;

  // Write the normalised output of one piece (scaled by `scale`): bf16 out and
  // lse for a whole sequence, else fp32 partials for the combine.
  auto write_piece = [&](const OAcc* oo, float scale, bool whole_, long long row, float lse_v) {
    if (my_row >= M) return;
    const bool lse_writer = dg == 0 && lane < R;
    // dims held by this lane: 4 consecutive dims per group of 4 accumulators
    auto dim_of = [&](int nt, int qd) {
      const int nb = dg * NT + nt;
      return R == 32 ? 32 * nb + 8 * qd + 4 * (lane >> 5) : 16 * nb + 4 * (lane >> 4);
    };
    constexpr int QUADS = OREGS / 4;
    if (whole_) {
      if (lse_writer) lse[row] = lse_v;
      uint16_t* orow = out + row * kValueDim;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int qd = 0; qd < QUADS; ++qd) {
          uint2 pk;
          pk.x = E::pack(oo[nt][4 * qd + 0] * scale, oo[nt][4 * qd + 1] * scale);
          pk.y = E::pack(oo[nt][4 * qd + 2] * scale, oo[nt][4 * qd + 3] * scale);
          *reinterpret_cast<uint2*>(orow + dim_of(nt, qd)) = pk;
        }
      }
    } else {
      if (lse_writer) lse_part[row] = lse_v;
      float* prow = o_part + row * kValueDim;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int qd = 0; qd < QUADS; ++qd) {
          *reinterpret_cast<float4*>(prow + dim_of(nt, qd)) =
              make_float4(oo[nt][4 * qd + 0] * scale, oo[nt][4 * qd + 1] * scale,
                          oo[nt][4 * qd + 2] * scale, oo[nt][4 * qd + 3] * scale);
        }
      }
    }
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
    float m_run = kMinit, l_run = 0.f, lr_run = 0.f;
    i16x8 qf[T::QREG_STEPS];

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
      if (rescale) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc_scale<OREGS>(o[nt], alpha);
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
          o[nt] = E::mfma32(va[idx % VP], pb[kb], o[nt]);
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

    // FLAT tiles: a stage's partial scores, their exchange with the other
    // wave of the row group (each wave keeps its own partial and adds the
    // partner's; the two sums are bit-identical since fp32 addition commutes),
    // softmax and P V.
    auto flat_scores = [&](const char MLA_LDS* __restrict__ rd) -> f32x16 {
      f32x16 sacc = f32x16{};
      if constexpr (T::FLAT) {
        constexpr int NK = KS_W;
        constexpr int KP = 2;  // K fragments read ahead (registers are tight at 2 waves per SIMD)
        i16x8 kf[KP];
#pragma unroll
        for (int i = 0; i < KP; ++i) kf[i] = lds_read_b128(rd + kstep_off(i));
        __builtin_amdgcn_sched_barrier(0);
        i16x8 qrf[T::QR_STEPS];
#pragma unroll
        for (int i = 0; i < NK; ++i) {
          if (i == T::QREG_STEPS - 4) {  // the rope fragments, a few MFMAs ahead
#pragma unroll
            for (int j = 0; j < T::QR_STEPS; ++j) qrf[j] = lds_read_b128(qr0 + 1024 * j);
          }
          if (i < T::QREG_STEPS) sacc = E::mfma32(kf[i % KP], qf[i < T::QREG_STEPS ? i : 0], sacc);
          else sacc = E::mfma32(kf[i % KP], qrf[i >= T::QREG_STEPS ? i - T::QREG_STEPS : 0], sacc);
          if (i + KP < NK) kf[i % KP] = lds_read_b128(rd + kstep_off(i + KP));
          fire_slot(i);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          lds_write_f4(xch0 + w * 4096 + qd * 1024 + lane * 16,
                       f32x4{sacc[4 * qd], sacc[4 * qd + 1], sacc[4 * qd + 2], sacc[4 * qd + 3]});
      }
      return sacc;
    };
    // Full scores of stage sp (own partial + the partner's), softmax and P V
    // with the keys of ring slot st.
    auto flat_finish = [&](const f32x16& own, int sp, const char MLA_LDS* __restrict__ st, int first_slot) {
      if constexpr (T::FLAT) {
        float x[SREGS];
        const char MLA_LDS* pp = xch0 + (w ^ 1) * 4096 + lane * 16;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x4 u = lds_read_f4(pp + qd * 1024);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * qd + e] = own[4 * qd + e] + u[e];
        }
        prep(x, sp);
        SoftState ss;
#pragma unroll
        for (int j = 0; j < kSoftSlices; ++j) soft_slice(x, ss, j);
        pv(ss.pw, ss.rescale, ss.alpha, sp, st, first_slot);
      }
    };

    if (nst > 0) {
      for (int jq = 0; jq < NQ; ++jq, ++cstage) {
        stage_ready();
        [&](const char MLA_LDS* __restrict__ rd, char MLA_LDS* __restrict__ wr) {
          plan(wr);
          fire_all();
          if (jq == q_stage) {
            const char MLA_LDS* qs = rd + q_row0 * kRowBytes;
#pragma unroll
            for (int ks = 0; ks < T::QREG_STEPS; ++ks) qf[ks] = lds_read_b128(qs + kstep_off(ks));
#pragma unroll
            for (int j = 0; j < T::QR_STEPS; ++j)
              lds_write_f4(qr0 + 1024 * j,
                           __builtin_bit_cast(f32x4, lds_read_b128(qs + kstep_off(T::QREG_STEPS + j))));
          }
        }(slot_of(cstage), slot_of(cstage + 2));
      }
      using F = std::false_type;
      using Tr = std::true_type;
      if constexpr (T::FLAT) {
        for (int s = 0; s < nst; ++s, ++cstage) {
          stage_ready();
          plan(slot_of(cstage + 2));
          const f32x16 sc = flat_scores(slot_of(cstage));
          block_barrier();  // the partial scores are exchanged
          flat_finish(sc, s, slot_of(cstage), T::QK_MFMA);
        }
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
        continue;
      }
    }
    write_piece(o, inv, whole, row, lse_row);
  }
  if constexpr (DEFER) {
    if (def_pending) write_piece(o_def, 1.f, def_whole, def_row, def_lse);
  }
  // Out-of-range loads past the end of the stream may still be in flight:
  // they must land before the workgroup's LDS is released.
  wait_vmcnt<0>();
}

#define MLA_DECODE_PARAMS                                                                   \
  const uint16_t* __restrict__, const uint16_t* __restrict__, const int32_t* __restrict__,  \
      const int32_t* __restrict__, const int32_t* __restrict__, uint16_t* __restrict__,      \
      float* __restrict__, float* __restrict__, float* __restrict__, DecodeArgs
#define MLA_DECODE_INSTANCES(E)                                                      \
  template __global__ void decode_kernel<16, 1, 4, false, E>(MLA_DECODE_PARAMS);   \
  template __global__ void decode_kernel<16, 2, 2, false, E>(MLA_DECODE_PARAMS);   \
  template __global__ void decode_kernel<32, 2, 2, false, E>(MLA_DECODE_PARAMS);   \
  template __global__ void decode_kernel<32, 4, 2, false, E>(MLA_DECODE_PARAMS);   \
  template __global__ void decode_kernel<16, 1, 4, true, E>(MLA_DECODE_PARAMS);    \
  template __global__ void decode_kernel<16, 2, 2, true, E>(MLA_DECODE_PARAMS);    \
  template __global__ void decode_kernel<32, 2, 2, true, E>(MLA_DECODE_PARAMS);    \
  template __global__ void decode_kernel<32, 4, 2, true, E>(MLA_DECODE_PARAMS);
MLA_DECODE_INSTANCES(Bf16)
MLA_DECODE_INSTANCES(F16)

template <int R, int RG, int DG, bool QG, typename E>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const int grid = a.num_parts * a.m_tiles * a.h_kv;
  hipLaunchKernelGGL((decode_kernel<R, RG, DG, QG, E>), dim3(grid), dim3(64 * RG * DG), 0, stream, a.q, a.kv,
                     a.block_table, a.seqlens, a.meta, a.out, a.lse, a.o_part, a.lse_part, a);
  return hipGetLastError();
}

template <bool QG, typename E>
static hipError_t launch_q(const DecodeArgs& a, int tile_rows, hipStream_t stream) {
  switch (tile_rows) {
    case 16: return launch_t<16, 1, 4, QG, E>(a, stream);
    case 32: return launch_t<16, 2, 2, QG, E>(a, stream);
    case 64: return launch_t<32, 2, 2, QG, E>(a, stream);
    case 128: return launch_t<32, 4, 2, QG, E>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename E>
static hipError_t launch_e(const DecodeArgs& a, int tile_rows, hipStream_t stream) {
  return a.h_kv == 1 ? launch_q<false, E>(a, tile_rows, stream) : launch_q<true, E>(a, tile_rows, stream);
}

hipError_t launch_decode(const DecodeArgs& a, int tile_rows, hipStream_t stream) {
  return a.f16 ? launch_e<F16>(a, tile_rows, stream) : launch_e<Bf16>(a, tile_rows, stream);
}

}  // namespace mla
