// Split combine: merge the fp32 partial outputs of a sequence's pieces by
// their log-sum-exp (the merge of partial outputs, cnblogs FlashMLA notes,
// section 4; num_splits from get_mla_metadata, section 6):
//     L = ln sum_k exp(lse_k),   out = sum_k exp(lse_k - L) * o_k.
// Pieces with lse_k = -inf (no visible key) weigh nothing; if every piece is
// empty the row gets out = 0 and lse = -inf.  Sequences with a single piece
// were written directly by the main kernel and are skipped here.
//
// One wave per query row.  The kernel is latency-bound at small batch, so
// each wave makes two dependent trips to memory: the split range (scalar
// loads), then the piece LSEs (lane k holds piece k) together with the partial
// rows of up to kUnroll pieces (64 lanes x 8 value dims, two 16-byte loads per
// lane and piece); longer splits take further trips of kUnroll pieces.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2c = 0.69314718055994530942f;
constexpr int kCombineRows = 4;  // waves (query rows) per workgroup
constexpr int kUnroll = 16;      // pieces loaded per trip

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__global__ __launch_bounds__(64 * kCombineRows) void combine_kernel(CombineArgs a) {
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int s0 = sload_i32(a.num_splits + b);
  const int nsplit = sload_i32(a.num_splits + b + 1) - s0;
  const int m = blockIdx.x * kCombineRows + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (nsplit <= 1 || m >= a.M) return;

  const long long stride = (long long)a.h_kv * a.M;  // rows between consecutive pieces
  const long long r0 = ((long long)s0 * a.h_kv + g) * a.M + m;
  const float* lse_row = a.lse_part + r0;

  // Issue the first pieces' partial rows with the LSE loads (lane k holds
  // the LSE of piece c + k), then reduce.
  const float* o_row = a.o_part + r0 * kValueDim + lane * 8;
  const int n0 = nsplit < kUnroll ? nsplit : kUnroll;
  float4 x[kUnroll][2];
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    if (j < n0) {
      const float4* src = reinterpret_cast<const float4*>(o_row + j * stride * kValueDim);
      x[j][0] = src[0];
      x[j][1] = src[1];
    }
  }
  auto lse_at = [&](int c) -> float {
    return c + lane < nsplit ? lse_row[(c + lane) * stride] : -INFINITY;
  };
  const float v0 = lse_at(0);
  float mx = v0;
  for (int c = 64; c < nsplit; c += 64) mx = fmaxf(mx, lse_at(c));
  mx = wave_max(mx);
  float L = -INFINITY;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (mx > -INFINITY) {
    float sum = 0.f;
    for (int c = 0; c < nsplit; c += 64) sum += fast_exp2(((c == 0 ? v0 : lse_at(c)) - mx) * kLog2e);
    L = mx + fast_log2(wave_sum(sum)) * kLn2c;
    const float w0 = fast_exp2((v0 - L) * kLog2e);  // weight of piece lane (first 64)
    auto add = [&](const float4* xj, float wk) {
      acc[0] += wk * xj[0].x; acc[1] += wk * xj[0].y; acc[2] += wk * xj[0].z; acc[3] += wk * xj[0].w;
      acc[4] += wk * xj[1].x; acc[5] += wk * xj[1].y; acc[6] += wk * xj[1].z; acc[7] += wk * xj[1].w;
    };
#pragma unroll
    for (int j = 0; j < kUnroll; ++j)
      if (j < n0) add(x[j], __shfl(w0, j, 64));
    // pieces past the first kUnroll, kUnroll per trip
    for (int k0 = kUnroll; k0 < nsplit; k0 += kUnroll) {
      const int c = k0 & ~63;
      const float wl = fast_exp2(((c == 0 ? v0 : lse_at(c)) - L) * kLog2e);  // weight of piece c + lane
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        if (k0 + j < nsplit) {
          const float4* src = reinterpret_cast<const float4*>(o_row + (k0 + j) * stride * kValueDim);
          x[j][0] = src[0];
          x[j][1] = src[1];
        }
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j)
        if (k0 + j < nsplit) add(x[j], __shfl(wl, (k0 + j) & 63, 64));
    }
  }
  const int hpg = a.h_q / a.h_kv;
  const int t = m / hpg;
  const int h = g * hpg + m % hpg;
  const long long out_row = ((long long)b * a.s_q + t) * a.h_q + h;
  uint4 pk;
  pk.x = pack_bf16(acc[0], acc[1]);
  pk.y = pack_bf16(acc[2], acc[3]);
  pk.z = pack_bf16(acc[4], acc[5]);
  pk.w = pack_bf16(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(a.out + out_row * kValueDim + lane * 8) = pk;
  if (lane == 0) a.lse[out_row] = L;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  dim3 grid((a.M + kCombineRows - 1) / kCombineRows, a.h_kv, a.batch);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(64 * kCombineRows), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
