// Split combine: merge the fp32 partial outputs of a sequence's pieces by
// their log-sum-exp (the merge of partial outputs, cnblogs FlashMLA notes,
// section 4; num_splits from get_mla_metadata, section 6):
//     L = ln sum_k exp(lse_k),   out = sum_k exp(lse_k - L) * o_k.
// Pieces with lse_k = -inf (no visible key) weigh nothing; if every piece is
// empty the row gets out = 0 and lse = -inf.  Sequences with a single piece
// were written directly by the main kernel and are skipped here.
//
// One wave per query row: 64 lanes x 8 value dims, 16-byte loads of the
// partials and one 16-byte bf16 store per lane.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2c = 0.69314718055994530942f;

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int s0 = a.num_splits[b];
  const int nsplit = a.num_splits[b + 1] - s0;
  if (nsplit <= 1 || m >= a.M) return;

  const long long stride = (long long)a.h_kv * a.M;  // rows between consecutive pieces
  const long long r0 = ((long long)s0 * a.h_kv + g) * a.M + m;
  float mx = -INFINITY;
  for (int k = 0; k < nsplit; ++k) mx = fmaxf(mx, a.lse_part[r0 + k * stride]);

  const int hpg = a.h_q / a.h_kv;
  const int t = m / hpg;
  const int h = g * hpg + m % hpg;
  const long long out_row = ((long long)b * a.s_q + t) * a.h_q + h;

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = -INFINITY;
  if (mx > -INFINITY) {
    float sum = 0.f;
    for (int k = 0; k < nsplit; ++k) sum += fast_exp2((a.lse_part[r0 + k * stride] - mx) * kLog2e);
    L = mx + fast_log2(sum) * kLn2c;
    for (int k = 0; k < nsplit; ++k) {
      const float wk = fast_exp2((a.lse_part[r0 + k * stride] - L) * kLog2e);
      const float4* src = reinterpret_cast<const float4*>(a.o_part + (r0 + k * stride) * kValueDim) +
                          lane * 2;
      const float4 x0 = src[0], x1 = src[1];
      acc[0] += wk * x0.x; acc[1] += wk * x0.y; acc[2] += wk * x0.z; acc[3] += wk * x0.w;
      acc[4] += wk * x1.x; acc[5] += wk * x1.y; acc[6] += wk * x1.z; acc[7] += wk * x1.w;
    }
  }
  uint4 pk;
  pk.x = pack_bf16(acc[0], acc[1]);
  pk.y = pack_bf16(acc[2], acc[3]);
  pk.z = pack_bf16(acc[4], acc[5]);
  pk.w = pack_bf16(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(a.out + out_row * kValueDim + lane * 8) = pk;
  if (lane == 0) a.lse[out_row] = L;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  dim3 grid((a.M + 3) / 4, a.h_kv, a.batch);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
