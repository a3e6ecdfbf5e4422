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
//   * 4 waves per workgroup, one workgroup per CU (147 KB LDS ring).
//   * Keys stream through a ring of 4 LDS slots of 32 keys (36 KB each) with
//     16-byte direct global->LDS loads; 3 stages are in flight while one is
//     computed.  Rows are XOR-swizzled in 16-byte chunks (conflict-free).
//   * Each wave owns R query rows (R = 16 or 32).  Scores are computed
//     transposed, S^T = K Q^T, with K from LDS (A operand) and Q^T resident in
//     registers (B operand); the MFMA result is then already laid out as the
//     B operand P^T of O^T = V^T P^T.  V^T comes from LDS through transposed
//     8-byte reads (ds_read_b64_tr_b16), so V needs no copy of its own.
//   * Softmax in fp32 in the log2 domain; the running max is raised only when
//     a row's new max exceeds it by more than kTau (then O and l are
//     rescaled), so most stages skip the rescale.  P is rounded to bf16 for
//     the MFMA and the row sum adds the rounded values, so normalisation uses
//     exactly the weights that multiplied V.
//   * Waves of one row group (DG > 1) split the 512 value dims; each repeats
//     the cheap score MFMAs of its rows, so no cross-wave merge is needed.
#include <type_traits>

#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

constexpr float kTau = 8.0f;        // lazy-rescale threshold (log2 units)
constexpr float kMinit = -1.0e30f;  // finite "minus infinity" for the running max
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ i16x8 lds_read_b128(const char MLA_LDS* p) {
  return *reinterpret_cast<const i16x8 MLA_LDS*>(p);
}
__device__ __forceinline__ i16x4 lds_read_tr(const char MLA_LDS* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 MLA_LDS*)(p));
}
// 16-byte global -> LDS copy per lane; the LDS address of lane l is dst + 16 l.
__device__ __forceinline__ void load_lds16(const char* src, char MLA_LDS* dst) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void MLA_LDS*)dst, 16, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(i16x8 a, i16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(i16x8 a, i16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Large accumulators (32-row tiles, 256 registers) stay in AGPRs: element
// reads/writes go through accvgpr moves so the compiler never moves a whole
// accumulator into VGPRs.  Small ones are ordinary registers.
template <bool PIN>
__device__ __forceinline__ float acc_read(float x) {
  if constexpr (!PIN) return x;
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(x));
  return v;
}
template <bool PIN>
__device__ __forceinline__ float acc_write(float v) {
  if constexpr (!PIN) return v;
  float x;
  asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(x) : "v"(v));
  return x;
}
template <bool PIN, int N, typename V>
__device__ __forceinline__ void acc_scale(V& o, float s) {
#pragma unroll
  for (int i = 0; i < N; ++i) o[i] = acc_write<PIN>(acc_read<PIN>(o[i]) * s);
}

__device__ __forceinline__ i16x8 cat(i16x4 a, i16x4 b) {
  return i16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// Zero the elements e >= first_bad of a 4-key fragment (keys past the end).
__device__ __forceinline__ i16x4 zero_from(i16x4 v, int first_bad) {
  i16x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = e < first_bad ? v[e] : (short)0;
  return r;
}

// exp2 of K masked scores -> packed bf16 B operand.  Adds the fp32 weights to
// *l (the softmax denominator behind lse) and the bf16-rounded weights to *lr
// (the normaliser of out, so out is an exact weighted mean of V with the
// weights the MFMA used).
template <int K>
__device__ __forceinline__ void weights_bf16(const float* x, float m, uint32_t* packed, float* l,
                                             float* lr) {
  float sum = 0.f, rsum = 0.f;
#pragma unroll
  for (int i = 0; i < K; i += 2) {
    const float p0 = fast_exp2(x[i] - m), p1 = fast_exp2(x[i + 1] - m);
    const uint32_t p = pack_bf16(p0, p1);
    packed[i >> 1] = p;
    sum += p0 + p1;
    rsum += bf16_lo(p) + bf16_hi(p);
  }
  *l += sum;
  *lr += rsum;
}

template <int R, int RG, int DG>
__global__ __launch_bounds__(256, 1) void decode_kernel(
    const uint16_t* __restrict__ q_ptr, const uint16_t* __restrict__ kv_ptr,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seqlens,
    const int32_t* __restrict__ meta, const int32_t* __restrict__ num_splits,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ o_part,
    float* __restrict__ lse_part, DecodeArgs a) {
  // The pointers are restrict-qualified kernel parameters so that uniform reads
  // of the read-only metadata become scalar loads (their waits never touch the
  // vector-memory counter that tracks the staged keys).
  constexpr int NW = RG * DG;
  static_assert(NW == kWaves, "four waves per workgroup");
  constexpr int BM = R * RG;
  constexpr int LPW = kLoadsPerStage / NW;  // 16-byte loads per lane per stage
  static_assert(LPW * NW == kLoadsPerStage, "stage loads split evenly");
  // R = 32: 32x32x16 MFMA tiles; R = 16: 16x16x32 tiles.
  constexpr int KSTEPS = R == 32 ? 36 : 18;     // score k-steps over 576 dims
  constexpr int NT = (R == 32 ? 16 : 32) / DG;  // value-dim tiles per wave
  constexpr int OREGS = R == 32 ? 16 : 4;       // accumulator registers per tile
  static_assert(3 * LPW + KSTEPS <= 63, "vector memory counter capacity");
  using OAcc = typename std::conditional<R == 32, f32x16, f32x4>::type;
  constexpr bool kPin = R == 32;             // pin the 256-register accumulators to AGPRs
  constexpr int NQ = (BM + kStage - 1) / kStage;  // query stages (32 rows each) per piece

  __shared__ __attribute__((aligned(1024))) char lds_raw[kLdsBytes];
  char MLA_LDS* lds = (char MLA_LDS*)lds_raw;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int rg = w / DG;
  const int dg = w % DG;

  // ---- which part / row tile / KV head -------------------------------------
  const int inner = a.m_tiles * a.h_kv;
  int part, inner_idx;
  if (a.xcd_map) {
    const int id = blockIdx.x;
    const int j = id >> 3;
    inner_idx = j % inner;
    part = (j / inner) * 8 + (id & 7);
  } else {
    part = blockIdx.x / inner;
    inner_idx = blockIdx.x % inner;
  }
  const int mtile = inner_idx / a.h_kv;
  const int g = inner_idx % a.h_kv;
  const int32_t* mp = meta + (long long)part * kMetaWords;
  const int bb = mp[0], tb = mp[1], be = mp[2], te = mp[3], k0 = mp[4];
  if (bb > be) return;  // empty part (uniform over the workgroup)

  const int M = a.M;
  const int hpg = a.h_q / a.h_kv;
  const int row_stride = a.h_kv * kRowBytes;  // bytes between consecutive tokens
  const char* kv_bytes = reinterpret_cast<const char*>(kv_ptr) + (long long)g * kRowBytes;

  // ---- lane constants --------------------------------------------------------
  const int lr = lane % R;  // this lane's query row inside the wave tile
  const int my_row = mtile * BM + rg * R + lr;
  const int q_row = my_row < M ? my_row : M - 1;
  const int q_t = q_row / hpg;
  const int q_h = g * hpg + q_row % hpg;

  // Byte offset (inside a stage) of this lane's k-th 16-byte global load.
  auto load_off = [&](int k) {
    const int s = (k * NW + w) * 64 + lane;  // 16-byte LDS cell filled by this lane
    const int row = s / kChunksPerRow;
    const int pc = s - row * kChunksPerRow;
    return row * row_stride + phys_chunk<R>(row, pc) * 16;  // swizzle is an involution
  };

  // K (A operand) LDS offsets and V^T (transposed read) offsets inside a stage.
  // K: lane reads 16 B of key row `row`, chunk c; stored at chunk c ^ swz(row).
  // V^T: a 16-lane group reads 4 key rows x 16 value dims; lane 4r + c supplies
  // the address of row r, dims 4c..4c+3 (8 B) and receives one dim of all 4.
  int koff[R == 32 ? 4 : 2];
  int voff[4];
  if constexpr (R == 32) {
    const int h = lane >> 5;
    // chunk of k-step ks = 8 (ks >> 2) + 2 (ks & 3) + h
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) koff[rr] = lr * kRowBytes + 16 * ((2 * rr + h) ^ swz<32>(lr));
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
    // chunk of k-step ks = 8 (ks >> 1) + 4 (ks & 1) + gq
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) koff[rr] = lr * kRowBytes + 16 * ((4 * rr + gq) ^ swz<16>(lr));
    // key row 16 jh + 4 gq + r: swz = 4 (gq & 1) + r;
    // dims 16 nb + 4 c: chunk 8 (nb >> 2) + 2 (nb & 3) + (c >> 1)
    const int i = lane & 15, r = i >> 2, c = i & 3;
#pragma unroll
    for (int nbq = 0; nbq < 4; ++nbq)
      voff[nbq] = (4 * gq + r) * kRowBytes + 8 * (c & 1) +
                  16 * ((2 * nbq + (c >> 1)) ^ (4 * (gq & 1) + r));
  }

  // ---- stage stream -----------------------------------------------------------
  // For every non-empty piece of the part: NQ query stages (32 query rows of
  // the tile each, same swizzled row layout as the keys), then the piece's key
  // stages.  Everything goes global -> LDS through the same ring, so the only
  // vector-memory waits are the explicit per-stage ones below.
  const int m_hi = (mtile * BM + BM < M ? mtile * BM + BM : M);  // end of the tile's valid rows
  int lb = bb, lq = 0, ltok = tb, lhi = (bb == be) ? te : seqlens[bb];
  bool lvalid = true;
  auto next_piece = [&]() {
    while (true) {
      if (lb >= be) {
        lvalid = false;
        return;
      }
      ++lb;
      lq = 0;
      ltok = 0;
      lhi = (lb == be) ? te : sload_i32(seqlens + lb);
      if (ltok < lhi) return;
    }
  };
  if (ltok >= lhi) next_piece();
  int issued = 0;
  // Issue the next stage of the stream into ring slot `wr` (= slot issued % 4).
  auto issue = [&](char MLA_LDS* __restrict__ wr) {
    if (!lvalid) return;
    char MLA_LDS* dst = wr + w * 1024;
    if (lq < NQ) {
      const char* qbase = reinterpret_cast<const char*>(q_ptr);
#pragma unroll
      for (int k = 0; k < LPW; ++k) {
        const int cell = (k * NW + w) * 64 + lane;
        const int row = cell / kChunksPerRow;
        const int pc = cell - row * kChunksPerRow;
        int m = mtile * BM + kStage * lq + row;
        m = m < m_hi ? m : m_hi - 1;
        const int t = m / hpg;
        const long long qrow = ((long long)lb * a.s_q + t) * a.h_q + g * hpg + (m - t * hpg);
        load_lds16(qbase + qrow * kRowBytes + phys_chunk<R>(row, pc) * 16, dst + k * NW * 1024);
      }
      ++lq;
    } else {
      const int page = sload_i32(block_table + (long long)lb * a.max_blocks + (ltok >> 6));
      const char* src = kv_bytes + ((long long)page * kPage + (ltok & 63)) * row_stride;
#pragma unroll
      for (int k = 0; k < LPW; ++k) load_lds16(src + load_off(k), dst + k * NW * 1024);
      ltok += kStage;
      if (ltok >= lhi) next_piece();
    }
    ++issued;
  };
  issue(lds);
  issue(lds + kStageBytes);
  issue(lds + 2 * kStageBytes);

  int cstage = 0;
  // wait for stage `cstage` (the ones issued after it may stay in flight), then
  // a barrier: the stage is visible to all waves and the slot refilled next
  // has been read by everyone
  auto stage_ready = [&]() {
    const int ahead = issued - 1 - cstage;
    if (ahead >= 2) wait_vmcnt<2 * LPW>();
    else if (ahead == 1) wait_vmcnt<LPW>();
    else wait_vmcnt<0>();
    block_barrier();
  };
  // query rows of this wave inside its query stage
  const int q_stage = (rg * R) / kStage;
  const int q_row0 = (rg * R) % kStage;

  for (int b = bb; b <= be; ++b) {
    const int N = sload_i32(seqlens + b);
    const int lo = (b == bb) ? tb : 0;
    const int hi = (b == be) ? te : N;
    const int nst = hi > lo ? (hi - lo + kStage - 1) / kStage : 0;
    const int s0 = sload_i32(num_splits + b);
    const int nsplit = sload_i32(num_splits + b + 1) - s0;
    const int split_k = (b == bb) ? k0 : 0;
    int row_lim = a.causal ? N - a.s_q + q_t + 1 : N;
    if (row_lim > N) row_lim = N;
    // keys every row of the workgroup sees (row t = 0 has the fewest)
    const int lim_all = a.causal ? N - a.s_q + 1 : N;

    OAcc o[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[nt] = OAcc{};
    float m_run = kMinit, l_run = 0.f, lr_run = 0.f;
    i16x8 qf[KSTEPS];

    if (nst > 0) {
      for (int j = 0; j < NQ; ++j, ++cstage) {
        stage_ready();
        // rd (this stage) and wr (the slot refilled now) are different slots
        [&](const char MLA_LDS* __restrict__ rd, char MLA_LDS* __restrict__ wr) {
        issue(wr);
        if (j == q_stage) {
          const char MLA_LDS* st = rd + q_row0 * kRowBytes;
          if constexpr (R == 32) {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
              qf[ks] = lds_read_b128(st + koff[ks & 3] + 128 * (ks >> 2));
          } else {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
              qf[ks] = lds_read_b128(st + koff[ks & 1] + 128 * (ks >> 1));
          }
        }
        }(lds + (cstage & (kSlots - 1)) * kStageBytes, lds + ((cstage + 3) & (kSlots - 1)) * kStageBytes);
      }
    }

    for (int s = 0; s < nst; ++s, ++cstage) {
      stage_ready();
      // rd (this stage) and wr (the slot refilled now) are different slots
      [&](const char MLA_LDS* __restrict__ rd, char MLA_LDS* __restrict__ wr) {
      issue(wr);

      const char MLA_LDS* st = rd;
      const int tok0 = lo + s * kStage;
      const int nvalid = N - tok0 < kStage ? N - tok0 : kStage;
      const bool tail = nvalid < kStage;
      const bool full = tok0 + kStage <= lim_all;  // no key of the stage is masked

      if constexpr (R == 32) {
        const int h = lane >> 5;
        // ---- scores S^T [32 keys x 32 rows]: rolling prefetch of K fragments ----
        constexpr int KP = 4;
        i16x8 kf[KP];
#pragma unroll
        for (int j = 0; j < KP; ++j) kf[j] = lds_read_b128(st + koff[j & 3] + 128 * (j >> 2));
        f32x16 sa = {};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          sa = mfma32(kf[ks % KP], qf[ks], sa);
          if (ks + KP < KSTEPS)
            kf[ks % KP] = lds_read_b128(st + koff[(ks + KP) & 3] + 128 * ((ks + KP) >> 2));
          __builtin_amdgcn_sched_barrier(0);
        }
        // ---- online softmax (lane: row lr, 16 keys) ----
        float x[16];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = sa[i] * a.scale_log2;
        if (!full) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int tk = 8 * (i >> 2) + 4 * h + (i & 3);
            x[i] = (tk < nvalid && tok0 + tk < row_lim) ? x[i] : -INFINITY;
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (__any(mx > m_run + kTau)) {
          const float m_new = fmaxf(m_run, mx);
          const float alpha = fast_exp2(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
          lr_run *= alpha;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc_scale<kPin, OREGS>(o[nt], alpha);
        }
        uint32_t pw[8];
        weights_bf16<16>(x, m_run, pw, &l_run, &lr_run);
        const i16x8 pb[2] = {__builtin_bit_cast(i16x8, i32x4{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]}),
                             __builtin_bit_cast(i16x8, i32x4{(int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]})};
        // ---- O^T += V^T P^T: rolling prefetch of V^T fragments ----
        constexpr int NV = 2 * NT;
        constexpr int VP = NV < 2 ? NV : 2;
        // jh = 0 / 1: keys 16 kb + 4 h + r and 16 kb + 8 + 4 h + r
        auto vaddr = [&](int idx, int jh) {
          const int kb = idx / NT, nb = dg * NT + idx % NT;
          return st + voff[2 * (nb & 1) + jh] + 128 * (nb >> 1) + (16 * kb + 8 * jh) * kRowBytes;
        };
        i16x4 va[VP], vb[VP];
#pragma unroll
        for (int j = 0; j < VP; ++j) {
          va[j] = lds_read_tr(vaddr(j, 0));
          vb[j] = lds_read_tr(vaddr(j, 1));
        }
#pragma unroll
        for (int idx = 0; idx < NV; ++idx) {
          const int kb = idx / NT, nt = idx % NT;
          i16x4 v0 = va[idx % VP], v1 = vb[idx % VP];
          if (tail) {
            v0 = zero_from(v0, nvalid - (16 * kb + 4 * h));
            v1 = zero_from(v1, nvalid - (16 * kb + 8 + 4 * h));
          }
          o[nt] = mfma32(cat(v0, v1), pb[kb], o[nt]);
          if (idx + VP < NV) {
            va[idx % VP] = lds_read_tr(vaddr(idx + VP, 0));
            vb[idx % VP] = lds_read_tr(vaddr(idx + VP, 1));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        const int gq = lane >> 4;
        // ---- scores S^T for two 16-key blocks x 16 rows ----
        constexpr int KP = 8;
        i16x8 kf[KP];
        auto kaddr = [&](int j) {  // j = 2 * ks + key block
          const int ks = j >> 1, tb2 = j & 1;
          return st + tb2 * 16 * kRowBytes + koff[ks & 1] + 128 * (ks >> 1);
        };
#pragma unroll
        for (int j = 0; j < KP; ++j) kf[j] = lds_read_b128(kaddr(j));
        f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int j = 0; j < 2 * KSTEPS; ++j) {
          sacc[j & 1] = mfma16(kf[j % KP], qf[j >> 1], sacc[j & 1]);
          if (j + KP < 2 * KSTEPS) kf[j % KP] = lds_read_b128(kaddr(j + KP));
          __builtin_amdgcn_sched_barrier(0);
        }
        // ---- online softmax (lane: row lr, 8 keys) ----
        float x[8];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = sacc[j >> 2][j & 3] * a.scale_log2;
        if (!full) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int tk = 16 * (j >> 2) + 4 * gq + (j & 3);
            x[j] = (tk < nvalid && tok0 + tk < row_lim) ? x[j] : -INFINITY;
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) mx = fmaxf(mx, x[j]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (__any(mx > m_run + kTau)) {
          const float m_new = fmaxf(m_run, mx);
          const float alpha = fast_exp2(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
          lr_run *= alpha;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc_scale<kPin, OREGS>(o[nt], alpha);
        }
        uint32_t pw[4];
        weights_bf16<8>(x, m_run, pw, &l_run, &lr_run);
        const i16x8 pb = __builtin_bit_cast(i16x8, i32x4{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]});
        // ---- O^T += V^T P^T ----
        constexpr int VP = NT < 4 ? NT : 4;
        auto vaddr = [&](int nt) {
          const int nb = dg * NT + nt;
          return st + voff[nb & 3] + 128 * (nb >> 2);
        };
        i16x4 va[VP], vb[VP];
#pragma unroll
        for (int j = 0; j < VP; ++j) {
          va[j] = lds_read_tr(vaddr(j));
          vb[j] = lds_read_tr(vaddr(j) + 16 * kRowBytes);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          i16x4 v0 = va[nt % VP], v1 = vb[nt % VP];
          if (tail) {
            v0 = zero_from(v0, nvalid - 4 * gq);
            v1 = zero_from(v1, nvalid - (16 + 4 * gq));
          }
          o[nt] = mfma16(cat(v0, v1), pb, o[nt]);
          if (nt + VP < NT) {
            va[nt % VP] = lds_read_tr(vaddr(nt + VP));
            vb[nt % VP] = lds_read_tr(vaddr(nt + VP) + 16 * kRowBytes);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      }(lds + (cstage & (kSlots - 1)) * kStageBytes, lds + ((cstage + 3) & (kSlots - 1)) * kStageBytes);
    }

    // ---- epilogue: normalise and write this piece --------------------------
    float lt = l_run, ltr = lr_run;
    if constexpr (R == 32) {
      lt += __shfl_xor(lt, 32);
      ltr += __shfl_xor(ltr, 32);
    } else {
      lt += __shfl_xor(lt, 16);
      lt += __shfl_xor(lt, 32);
      ltr += __shfl_xor(ltr, 16);
      ltr += __shfl_xor(ltr, 32);
    }
    const bool empty = !(lt > 0.f);
    const float inv = empty ? 0.f : 1.f / ltr;
    const float lse_row = empty ? -INFINITY : (m_run + fast_log2(lt)) * kLn2;
    if (my_row < M) {
      const long long out_row = ((long long)b * a.s_q + q_t) * a.h_q + q_h;
      const long long part_row = ((long long)(s0 + split_k) * a.h_kv + g) * M + my_row;
      const bool lse_writer = dg == 0 && lane < R;
      // dims held by this lane: 4 consecutive dims per group of 4 accumulators
      auto dim_of = [&](int nt, int qd) {
        const int nb = dg * NT + nt;
        return R == 32 ? 32 * nb + 8 * qd + 4 * (lane >> 5) : 16 * nb + 4 * (lane >> 4);
      };
      constexpr int QUADS = OREGS / 4;
      if (nsplit == 1) {
        if (lse_writer) lse[out_row] = lse_row;
        uint16_t* orow = out + out_row * kValueDim;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int qd = 0; qd < QUADS; ++qd) {
            uint2 pk;
            pk.x = pack_bf16(acc_read<kPin>(o[nt][4 * qd + 0]) * inv, acc_read<kPin>(o[nt][4 * qd + 1]) * inv);
            pk.y = pack_bf16(acc_read<kPin>(o[nt][4 * qd + 2]) * inv, acc_read<kPin>(o[nt][4 * qd + 3]) * inv);
            *reinterpret_cast<uint2*>(orow + dim_of(nt, qd)) = pk;
          }
        }
      } else {
        if (lse_writer) lse_part[part_row] = lse_row;
        float* prow = o_part + part_row * kValueDim;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int qd = 0; qd < QUADS; ++qd) {
            *reinterpret_cast<float4*>(prow + dim_of(nt, qd)) =
                make_float4(acc_read<kPin>(o[nt][4 * qd + 0]) * inv, acc_read<kPin>(o[nt][4 * qd + 1]) * inv,
                            acc_read<kPin>(o[nt][4 * qd + 2]) * inv, acc_read<kPin>(o[nt][4 * qd + 3]) * inv);
          }
        }
      }
    }
  }
}

#define MLA_DECODE_PARAMS                                                                   \
  const uint16_t* __restrict__, const uint16_t* __restrict__, const int32_t* __restrict__,  \
      const int32_t* __restrict__, const int32_t* __restrict__, const int32_t* __restrict__, \
      uint16_t* __restrict__, float* __restrict__, float* __restrict__, float* __restrict__, \
      DecodeArgs
template __global__ void decode_kernel<16, 1, 4>(MLA_DECODE_PARAMS);
template __global__ void decode_kernel<16, 2, 2>(MLA_DECODE_PARAMS);
template __global__ void decode_kernel<32, 2, 2>(MLA_DECODE_PARAMS);
template __global__ void decode_kernel<32, 4, 1>(MLA_DECODE_PARAMS);

template <int R, int RG, int DG>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const int grid = a.num_parts * a.m_tiles * a.h_kv;
  hipLaunchKernelGGL((decode_kernel<R, RG, DG>), dim3(grid), dim3(256), 0, stream, a.q, a.kv,
                     a.block_table, a.seqlens, a.meta, a.num_splits, a.out, a.lse, a.o_part,
                     a.lse_part, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int tile_rows, hipStream_t stream) {
  switch (tile_rows) {
    case 16: return launch_t<16, 1, 4>(a, stream);
    case 32: return launch_t<16, 2, 2>(a, stream);
    case 64: return launch_t<32, 2, 2>(a, stream);
    case 128: return launch_t<32, 4, 1>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mla
