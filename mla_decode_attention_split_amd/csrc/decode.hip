// Instances of the decode kernel for tiles of up to 64 query rows, and the
// launch dispatch over all tile shapes (128-row tiles: decode_wide.hip).
#include "decode_kernel.hpp"

namespace mla {

#define MLA_DECODE_PARAMS                                                                   \
  const uint16_t* __restrict__, const uint16_t* __restrict__, const int32_t* __restrict__,  \
      const int32_t* __restrict__, const int32_t* __restrict__, uint16_t* __restrict__,      \
      float* __restrict__, uint16_t* __restrict__, float* __restrict__, DecodeArgs
// The 16-row and 32-row tiles load key stages non-temporally when they are
// the part's only row tile (one m-tile); the 64-row tile (two row groups of
// 32 rows) measured ~0.7 us slower with it on the ragged batch and always
// keeps the default policy.
#define MLA_DECODE_INSTANCES(E)                                                           \
  template __global__ void decode_kernel<16, 1, 4, false, false, E>(MLA_DECODE_PARAMS);  \
  template __global__ void decode_kernel<16, 1, 4, false, true, E>(MLA_DECODE_PARAMS);   \
  template __global__ void decode_kernel<16, 2, 2, false, false, E>(MLA_DECODE_PARAMS);  \
  template __global__ void decode_kernel<16, 2, 2, false, true, E>(MLA_DECODE_PARAMS);   \
  template __global__ void decode_kernel<32, 2, 2, false, false, E>(MLA_DECODE_PARAMS);  \
  template __global__ void decode_kernel<16, 1, 4, true, false, E>(MLA_DECODE_PARAMS);   \
  template __global__ void decode_kernel<16, 1, 4, true, true, E>(MLA_DECODE_PARAMS);    \
  template __global__ void decode_kernel<16, 2, 2, true, false, E>(MLA_DECODE_PARAMS);   \
  template __global__ void decode_kernel<16, 2, 2, true, true, E>(MLA_DECODE_PARAMS);    \
  template __global__ void decode_kernel<32, 2, 2, true, false, E>(MLA_DECODE_PARAMS);
MLA_DECODE_INSTANCES(Bf16)
MLA_DECODE_INSTANCES(F16)

template <int R, int RG, int DG, bool QG, typename E>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const int grid = a.num_parts * a.m_tiles * a.h_kv;
  auto go = [&](auto ntk) {
    hipLaunchKernelGGL((decode_kernel<R, RG, DG, QG, decltype(ntk)::value, E>), dim3(grid), dim3(64 * RG * DG),
                       0, stream, a.q, a.kv, a.block_table, a.seqlens, a.meta, a.out, a.lse, a.o_part,
                       a.lse_part, a);
  };
  if constexpr (R == 32) go(std::false_type{});
  else if (a.m_tiles == 1) go(std::true_type{});
  else go(std::false_type{});
  return hipGetLastError();
}

template <bool QG, typename E>
static hipError_t launch_q(const DecodeArgs& a, int tile_rows, hipStream_t stream) {
  switch (tile_rows) {
    case 16: return launch_t<16, 1, 4, QG, E>(a, stream);
    case 32: return launch_t<16, 2, 2, QG, E>(a, stream);
    case 64: return launch_t<32, 2, 2, QG, E>(a, stream);
    case 128:
      if constexpr (QG) return hipErrorInvalidValue;  // one KV head only
      else return launch_decode_wide(a, stream);
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
