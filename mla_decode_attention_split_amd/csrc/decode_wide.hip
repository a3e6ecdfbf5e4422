// Instances of the decode kernel's WIDE tile (one KV head): 128 query rows
// per workgroup, four waves of 32 rows, each wave holding all 512 value dims of its rows
// (output accumulators in AGPRs) and contracting all 576 dims of its scores.
// Built without the VGPR-form MFMA option the other tiles use, so that the
// output accumulators can live in AGPRs.
#include "decode_kernel.hpp"

namespace mla {

#define MLA_WIDE_PARAMS                                                                     \
  const uint16_t* __restrict__, const uint16_t* __restrict__, const int32_t* __restrict__,  \
      const int32_t* __restrict__, const int32_t* __restrict__, uint16_t* __restrict__,      \
      float* __restrict__, uint16_t* __restrict__, float* __restrict__, DecodeArgs
// Key stages load non-temporally when the tile is the part's only row tile
// (one m-tile); otherwise the other m-tiles of the part read the same pages
// from L2.
template __global__ void decode_kernel<32, 4, 1, false, false, Bf16>(MLA_WIDE_PARAMS);
template __global__ void decode_kernel<32, 4, 1, false, true, Bf16>(MLA_WIDE_PARAMS);
template __global__ void decode_kernel<32, 4, 1, false, false, F16>(MLA_WIDE_PARAMS);
template __global__ void decode_kernel<32, 4, 1, false, true, F16>(MLA_WIDE_PARAMS);

template <typename E>
static hipError_t launch_w(const DecodeArgs& a, hipStream_t stream) {
  const int grid = a.num_parts * a.m_tiles;
  auto go = [&](auto ntk) {
    hipLaunchKernelGGL((decode_kernel<32, 4, 1, false, decltype(ntk)::value, E>), dim3(grid), dim3(256), 0,
                       stream, a.q, a.kv, a.block_table, a.seqlens, a.meta, a.out, a.lse, a.o_part,
                       a.lse_part, a);
  };
  if (a.m_tiles == 1) go(std::true_type{});
  else go(std::false_type{});
  return hipGetLastError();
}

// One KV head (the host picks 64-row tiles for more).
hipError_t launch_decode_wide(const DecodeArgs& a, hipStream_t stream) {
  if (a.h_kv != 1) return hipErrorInvalidValue;
  return a.f16 ? launch_w<F16>(a, stream) : launch_w<Bf16>(a, stream);
}

}  // namespace mla
