// Split combine: merge the partial outputs of a sequence's pieces by their
// log-sum-exp (the merge of partial outputs, cnblogs FlashMLA notes,
// section 4; num_splits from get_mla_metadata, section 6):
//     L = ln sum_k exp(lse_k),   out = sum_k exp(lse_k - L) * o_k.
// Pieces with lse_k = -inf (no visible key) weigh nothing; if every piece is
// empty the row gets out = 0 and lse = -inf.  Sequences with a single piece
// were written directly by the main kernel and are skipped here.
//
// Partial rows are 16-bit (the element type of out: each is a convex
// combination of value rows, rounded once); LSEs and all sums are fp32.
// The kernel is latency-bound, so each wave makes two dependent trips to
// memory: the split range (scalar loads), then the piece LSEs (lane k holds
// piece k) together with the partial rows of up to kUnroll pieces (64 lanes x
// 8 value dims, one 16-byte load per lane and piece).  Two layouts, chosen
// per sequence from its piece count (so every row of a sequence is summed in
// the same order):
//   * one wave per query row, 4 rows per workgroup;
//   * in the shared-row grid, for sequences of more than kShareMin pieces:
//     the 4 waves of a workgroup share one row, each taking a 16-aligned
//     quarter of the pieces, and their sums meet in LDS in wave order.  A row
//     of 80 pieces then costs two trips per wave instead of five, on 4x as
//     many CUs.
// The shared-row grid has one workgroup per query row (in the one-row-per-
// wave layout only the first ceil(M / 4) of them work); the host picks it
// when the batch averages many pieces per sequence, since idle workgroups
// cost dispatch time.
#include <type_traits>

#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2c = 0.69314718055994530942f;
constexpr int kCombineWaves = 4;  // waves per workgroup
constexpr int kUnroll = 16;       // pieces loaded per trip
constexpr int kUnrollFew = 4;     // ... when sequences average at most 4 pieces
constexpr int kShareMin = 4;      // shared-row grid: more pieces than this, 4 waves per row
constexpr int kSharePieces = 16;  // pick the shared-row grid at this many pieces per sequence

// 16 bytes of a partial row.  Every partial is read exactly once; the
// layout of 4 pieces per trip (sequences of few pieces: mtp, large) loads
// them non-temporally (large combine 10.8 -> 9.5 us), the others with the
// default policy (non-temporal made the shared-row layout slower: ragged
// 6.4 -> 7.9 us).
template <bool NT>
__device__ __forceinline__ uint4 load_part16(const uint16_t* p) {
  if constexpr (NT) {
    const i32x4 v = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
    return make_uint4((unsigned)v[0], (unsigned)v[1], (unsigned)v[2], (unsigned)v[3]);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

// 8 partial values of one 16-byte load, widened to fp32 (exact).
template <typename E>
__device__ __forceinline__ void widen8(const uint4& u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (std::is_same<E, F16>::value) {
      f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
      f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    } else {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// UNROLL pieces per trip: 16, or 4 when the batch averages at most 4 pieces
// per sequence (then 16 instead of 64 registers hold a trip's rows, and more
// waves fit on a SIMD to keep more rows in flight).  Pieces are added in
// index order either way, so both give the same bits.
template <int UNROLL, typename E>
__global__ __launch_bounds__(64 * kCombineWaves) void combine_kernel(CombineArgs a) {
  constexpr int kUnroll = UNROLL;
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int s0 = sload_i32(a.num_splits + b);
  const int nsplit = sload_i32(a.num_splits + b + 1) - s0;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (nsplit <= 1) return;
  const bool shared = a.share_grid && nsplit > kShareMin;  // uniform over the workgroup
  int m, p_lo, p_hi;                       // this wave's row and pieces [p_lo, p_hi)
  if (shared) {
    m = blockIdx.x;
    if (m >= a.M) return;  // whole workgroup
    const int q = ((nsplit + kCombineWaves - 1) / kCombineWaves + kUnroll - 1) / kUnroll * kUnroll;
    p_lo = wave * q < nsplit ? wave * q : nsplit;
    p_hi = p_lo + q < nsplit ? p_lo + q : nsplit;
  } else {
    m = blockIdx.x * kCombineWaves + wave;
    if (m >= a.M) return;  // this wave only (no barrier in this layout)
    p_lo = 0;
    p_hi = nsplit;
  }

  const long long stride = (long long)a.h_kv * a.M;  // rows between consecutive pieces
  const long long r0 = ((long long)s0 * a.h_kv + g) * a.M + m;
  const float* lse_row = a.lse_part + r0;

  // Issue the first trip's partial rows with the LSE loads (lane k holds
  // the LSE of piece c + k), then reduce.
  const uint16_t* o_row = a.o_part + r0 * kValueDim + lane * 8;
  const int n0 = p_hi - p_lo < kUnroll ? p_hi - p_lo : kUnroll;
  uint4 x[kUnroll];
#pragma unroll
  for (int j = 0; j < kUnroll; ++j)
    if (j < n0) x[j] = load_part16<UNROLL == kUnrollFew>(o_row + (p_lo + j) * stride * kValueDim);
  auto lse_at = [&](int c) -> float {
    return c + lane < nsplit ? lse_row[(c + lane) * stride] : -INFINITY;
  };
  const float v0 = lse_at(0);
  float mx = v0;
  for (int c = 64; c < nsplit; c += 64) mx = fmaxf(mx, lse_at(c));
  mx = wave_allmax_f32(mx);
  float L = -INFINITY;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (mx > -INFINITY) {
    float sum = 0.f;
    for (int c = 0; c < nsplit; c += 64) sum += fast_exp2(((c == 0 ? v0 : lse_at(c)) - mx) * kLog2e);
    L = mx + fast_log2(wave_allsum_f32(sum)) * kLn2c;
    auto add = [&](const uint4& xj, float wk) {
      float v[8];
      widen8<E>(xj, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += wk * v[i];
    };
    // Trips start at multiples of kUnroll, so the pieces of one trip share a
    // 64-piece chunk and one weight register (lane k: piece c + k), read with a
    // uniform lane index.
    auto weights = [&](int k0) {
      const int c = k0 & ~63;
      return fast_exp2(((c == 0 ? v0 : lse_at(c)) - L) * kLog2e);
    };
    {
      const float wl = weights(p_lo);
#pragma unroll
      for (int j = 0; j < kUnroll; ++j)
        if (j < n0) add(x[j], row_total_f32(wl, (p_lo + j) & 63));
    }
    for (int k0 = p_lo + kUnroll; k0 < p_hi; k0 += kUnroll) {
      const float wl = weights(k0);
#pragma unroll
      for (int j = 0; j < kUnroll; ++j)
        if (k0 + j < p_hi) x[j] = load_part16<UNROLL == kUnrollFew>(o_row + (k0 + j) * stride * kValueDim);
#pragma unroll
      for (int j = 0; j < kUnroll; ++j)
        if (k0 + j < p_hi) add(x[j], row_total_f32(wl, (k0 + j) & 63));
    }
  }

  if (shared) {
    // The four quarter sums meet in LDS and wave 0 adds them in wave order.
    __shared__ float4 part[kCombineWaves - 1][64][2];
    if (wave > 0) {
      part[wave - 1][lane][0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      part[wave - 1][lane][1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < kCombineWaves - 1; ++w) {
      const float4 u = part[w][lane][0], v = part[w][lane][1];
      acc[0] += u.x; acc[1] += u.y; acc[2] += u.z; acc[3] += u.w;
      acc[4] += v.x; acc[5] += v.y; acc[6] += v.z; acc[7] += v.w;
    }
  }
  const int hpg = a.h_q / a.h_kv;
  const int t = m / hpg;
  const int h = g * hpg + m % hpg;
  const long long out_row = ((long long)b * a.s_q + t) * a.h_q + h;
  uint4 pk;
  pk.x = E::pack(acc[0], acc[1]);
  pk.y = E::pack(acc[2], acc[3]);
  pk.z = E::pack(acc[4], acc[5]);
  pk.w = E::pack(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(a.out + out_row * kValueDim + lane * 8) = pk;
  if (lane == 0) a.lse[out_row] = L;
}

hipError_t launch_combine(CombineArgs a, int num_parts, hipStream_t stream) {
  a.share_grid = (long long)num_parts >= (long long)kSharePieces * a.batch ? 1 : 0;
  dim3 grid(a.share_grid ? a.M : (a.M + kCombineWaves - 1) / kCombineWaves, a.h_kv, a.batch);
  // pieces per sequence <= 1 + num_parts / batch on average
  const bool few = !a.share_grid && (long long)num_parts <= (long long)(kUnrollFew - 1) * a.batch;
  auto go = [&](auto e) {
    using E = decltype(e);
    if (few)
      hipLaunchKernelGGL((combine_kernel<kUnrollFew, E>), grid, dim3(64 * kCombineWaves), 0, stream, a);
    else
      hipLaunchKernelGGL((combine_kernel<kUnroll, E>), grid, dim3(64 * kCombineWaves), 0, stream, a);
  };
  if (a.f16) go(F16{});
  else go(Bf16{});
  return hipGetLastError();
}

}  // namespace mla
