// Split-KV tile scheduler: one workgroup turns cache_seqlens into the
// partition of every sequence's keys over `num_parts` parts.
//
// Block scheduling (FlashMLA explainer, jsxs2.com, section 3.1) and the
// get_mla_metadata call (cnblogs FlashMLA notes, section 6) are named on the
// pages; the partition rule is this library's, stated in mla_decode.h:
// cost-interval partition at 32-key granularity with a per-sequence fixed
// cost, so that ragged batches spread over the compute units.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

constexpr int kSchedThreads = 1024;

__device__ __forceinline__ long long units_of(int n) { return ((long long)n + kStage - 1) / kStage; }

// Block-wide exclusive scan of one int64 per thread; returns the prefix and
// writes the block total to *total.
__device__ long long block_exclusive_scan(long long v, long long* scratch, long long* total) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  long long x = v;
  for (int off = 1; off < 64; off <<= 1) {
    long long y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  if (wave == 0) {
    long long w = lane < (kSchedThreads / 64) ? scratch[lane] : 0;
    for (int off = 1; off < 16; off <<= 1) {
      long long y = __shfl_up(w, off, 64);
      if (lane >= off) w += y;
    }
    if (lane < (kSchedThreads / 64)) scratch[16 + lane] = w;
  }
  __syncthreads();
  long long wave_prefix = wave > 0 ? scratch[16 + wave - 1] : 0;
  *total = scratch[16 + kSchedThreads / 64 - 1];
  __syncthreads();
  return wave_prefix + x - v;
}

__global__ __launch_bounds__(kSchedThreads) void sched_kernel(const int32_t* __restrict__ seqlens,
                                                              int batch, int num_parts,
                                                              int fixed_cost,
                                                              int32_t* __restrict__ meta,
                                                              int32_t* __restrict__ num_splits) {
  // C[b] = sum of cost over sequences before b; C[batch] = total.
  __shared__ long long C[kMaxBatch + 1];
  __shared__ long long scratch[32];
  const int tid = threadIdx.x;
  const int per = (batch + kSchedThreads - 1) / kSchedThreads;
  const int b0 = tid * per;

  // 1. per-thread run of consecutive sequences: local sums, then block scan.
  long long local = 0;
  for (int i = 0; i < per; ++i) {
    int b = b0 + i;
    if (b < batch) local += units_of(seqlens[b]) + fixed_cost;
  }
  long long total;
  long long base = block_exclusive_scan(local, scratch, &total);
  for (int i = 0; i < per; ++i) {
    int b = b0 + i;
    if (b < batch) {
      C[b] = base;
      base += units_of(seqlens[b]) + fixed_cost;
    }
  }
  if (tid == 0) C[batch] = total;
  __syncthreads();

  long long T = (total + num_parts - 1) / num_parts;
  if (T < 1) T = 1;

  // first / last part holding a piece of sequence b
  auto first_part = [&](int b) -> long long {
    long long u = C[b + 1] - C[b] - fixed_cost;
    return u > 0 ? (C[b] + fixed_cost) / T : (C[b] + fixed_cost - 1) / T;
  };
  auto last_part = [&](int b) -> long long {
    long long u = C[b + 1] - C[b] - fixed_cost;
    return u > 0 ? (C[b] + fixed_cost + u - 1) / T : (C[b] + fixed_cost - 1) / T;
  };

  // 2. num_splits = exclusive prefix of pieces per sequence.
  long long lp = 0;
  for (int i = 0; i < per; ++i) {
    int b = b0 + i;
    if (b < batch) lp += last_part(b) - first_part(b) + 1;
  }
  long long ptotal;
  long long pbase = block_exclusive_scan(lp, scratch, &ptotal);
  for (int i = 0; i < per; ++i) {
    int b = b0 + i;
    if (b < batch) {
      num_splits[b] = (int32_t)pbase;
      pbase += last_part(b) - first_part(b) + 1;
    }
  }
  if (tid == 0) num_splits[batch] = (int32_t)ptotal;

  // 3. per part: first sequence with last_part >= p, last with first_part <= p.
  for (int p = tid; p < num_parts; p += kSchedThreads) {
    int lo = 0, hi = batch;  // first b with last_part(b) >= p
    while (lo < hi) {
      int mid = (lo + hi) >> 1;
      if (last_part(mid) >= p) hi = mid; else lo = mid + 1;
    }
    int bb = lo;
    lo = -1;
    hi = batch - 1;  // last b with first_part(b) <= p
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (first_part(mid) <= p) lo = mid; else hi = mid - 1;
    }
    int be = lo;
    int32_t w[kMetaWords] = {0, 0, -1, 0, 0, 0, 0, 0};
    if (bb < batch && be >= 0 && bb <= be) {
      long long ub = C[bb + 1] - C[bb] - fixed_cost;
      long long ue = C[be + 1] - C[be] - fixed_cost;
      long long u_begin = 0, u_end = 0;
      if (ub > 0) {
        u_begin = (long long)p * T - C[bb] - fixed_cost;
        if (u_begin < 0) u_begin = 0;
      }
      if (ue > 0) {
        u_end = (long long)(p + 1) * T - C[be] - fixed_cost;
        if (u_end > ue) u_end = ue;
      }
      long long tok_end = u_end * kStage;
      if (tok_end > seqlens[be]) tok_end = seqlens[be];
      w[0] = bb;
      w[1] = (int32_t)(u_begin * kStage);
      w[2] = be;
      w[3] = (int32_t)tok_end;
      w[4] = (int32_t)(p - first_part(bb));
    }
    i32x4* dst = reinterpret_cast<i32x4*>(meta + (long long)p * kMetaWords);
    dst[0] = i32x4{w[0], w[1], w[2], w[3]};
    dst[1] = i32x4{w[4], w[5], w[6], w[7]};
  }
}

hipError_t launch_sched(const int32_t* seqlens, int batch, int num_parts, int fixed_cost,
                        int32_t* meta, int32_t* num_splits, hipStream_t stream) {
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kSchedThreads), 0, stream, seqlens, batch,
                     num_parts, fixed_cost, meta, num_splits);
  return hipGetLastError();
}

}  // namespace mla
