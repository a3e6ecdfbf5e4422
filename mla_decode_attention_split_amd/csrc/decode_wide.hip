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
// Key stages always load non-temporally.  Even when two row tiles of a part
// read the same pages (more than 128 rows per KV head), the second reading
// them again from HBM instead of from L2 measured faster (mtp kernel
// 177.2 -> 174.0 us): the tile is bound by its arithmetic, not by HBM.
template __global__ void decode_kernel<32, 4, 1, false, true, Bf16>(MLA_WIDE_PARAMS);
template __global__ void decode_kernel<32, 4, 1, false, true, F16>(MLA_WIDE_PARAMS);

template <typename E>
static hipError_t launch_w(const DecodeArgs& a, hipStream_t stream) {
  const int grid = a.num_parts * a.m_tiles;
  hipLaunchKernelGGL((decode_kernel<32, 4, 1, false, true, E>), dim3(grid), dim3(256), 0, stream, a.q,
                     a.kv, a.block_table, a.seqlens, a.meta, a.out, a.lse, a.o_part, a.lse_part, a);
  return hipGetLastError();
}

// One KV head (the host picks 64-row tiles for more).
hipError_t launch_decode_wide(const DecodeArgs& a, hipStream_t stream) {
  if (a.h_kv != 1) return hipErrorInvalidValue;
  return a.f16 ? launch_w<F16>(a, stream) : launch_w<Bf16>(a, stream);
}

}  // namespace mla
