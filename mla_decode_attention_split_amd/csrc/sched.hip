// Split-KV tile scheduler: one workgroup turns cache_seqlens into the
// partition of every sequence's keys over `num_parts` parts.
//
// Block scheduling (FlashMLA explainer, jsxs2.com, section 3.1) and the
// get_mla_metadata call (cnblogs FlashMLA notes, section 6) are named on the
// pages; the partition rule is this library's, stated in mla_decode.h:
// cost-interval partition at 32-key granularity on a line counted in half
// units, with a per-sequence fixed cost split over the sequence's two ends
// and every unit placed at its midpoint, so that ragged batches spread over
// the compute units and equal sequences split into equal pieces.
//
// The kernel is latency-bound (a few hundred integers), so it is built to
// touch global memory once per input and once per output: cache_seqlens is
// staged in LDS (up to 4096 sequences), the prefix costs C_b stay in LDS, and each part finds its
// first and last sequence by binary search against the first positions of
// parts p and p + 1 ("part of x <= p" is "x < first position of p + 1").
// Integer divisions (software-emulated on the GPU) are only taken a constant
// number of times per thread.
//
// Positions, for sequence b with U_b units and fixed cost f (half units):
//   C_b = sum over b' < b of (2 U_b' + 2 f)
//   KF_b = C_b + f + 1 (first unit's midpoint), KL_b = C_b + f + 2 U_b - 1
//   (last unit's midpoint); both C_b + f for a sequence with no unit.
//   The parts share the line evenly: position x is in part
//   floor(x num_parts / C_B), so part p holds positions [F_p, F_{p+1}) with
//   F_p = ceil(p C_B / num_parts); when C_B < 2 num_parts every part holds 2
//   positions instead (part floor(x / 2), F_p = 2 p).
//   Units of b before part p: max(0, ceil((F_p - C_b - f - 1) / 2)).
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

// The even share of the cost line among the parts (see the rule above).
struct PartLine {
  long long total, parts;
  __device__ __forceinline__ bool span2() const { return total < 2 * parts; }
  // part of cost position x >= 0
  __device__ __forceinline__ long long part_of(long long x) const {
    return span2() ? x >> 1 : x * parts / total;
  }
  // first position of part p (p <= parts)
  __device__ __forceinline__ long long first_of(long long p) const {
    return span2() ? 2 * p : (p * total + parts - 1) / parts;
  }
};

__device__ __forceinline__ long long units_of(int n) { return ((long long)n + kStage - 1) / kStage; }

// Block-wide exclusive scan of one int64 per thread; *total gets the sum.
template <int NT>
__device__ __forceinline__ long long block_exclusive_scan(long long v, long long* scratch,
                                                          long long* total) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const long long x = wave_inclusive_sum_i64(v);
  if constexpr (NT == 64) {
    *total = readlane_i64(x, 63);
    return x - v;
  } else {
    constexpr int NW = NT / 64;
    if (lane == 63) scratch[wave] = x;
    __syncthreads();
    long long wave_prefix = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const long long s = scratch[i];
      if (i < wave) wave_prefix += s;
      tot += s;
    }
    __syncthreads();  // scratch is reused by the next scan
    *total = tot;
    return wave_prefix + x - v;
  }
}

template <int NT, int MAXB>
__global__ __launch_bounds__(NT) void sched_kernel(const int32_t* __restrict__ seqlens, int batch,
                                                   int num_parts, int fixed_cost,
                                                   int32_t* __restrict__ meta,
                                                   int32_t* __restrict__ num_splits) {
  // cache_seqlens is staged in LDS unless that would not fit beside C.
  constexpr bool kSlInLds = MAXB <= 4096;
  __shared__ long long C[MAXB + 1];  // C[b] = cost of the sequences before b
  __shared__ int SL_lds[kSlInLds ? MAXB : 1];
  __shared__ int NS_lds[kSlInLds ? MAXB + 1 : 1];
  auto SL = [&](int b) -> int { return kSlInLds ? SL_lds[b] : seqlens[b]; };
  // num_splits as written by this kernel (read back only after the barrier)
  auto NS = [&](int b) -> int { return kSlInLds ? NS_lds[b] : num_splits[b]; };
  __shared__ long long scratch[NT / 64];
  const int tid = threadIdx.x;
  const int per = (batch + NT - 1) / NT;
  const int b0 = tid * per;
  const long long fc = fixed_cost;

  // 1. seqlens -> LDS, per-thread cost of a run of consecutive sequences.
  long long local = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < batch) {
      const int n = seqlens[b];
      if constexpr (kSlInLds) SL_lds[b] = n;
      local += 2 * units_of(n) + 2 * fc;
    }
  }
  long long total;
  long long base = block_exclusive_scan<NT>(local, scratch, &total);
  const PartLine line{total, num_parts};

  // 2. prefix costs, and pieces per sequence = last part - first part + 1.
  long long pieces = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < batch) {
      C[b] = base;
      const long long u = units_of(SL(b));
      const long long first = line.part_of(base + fc + (u > 0 ? 1 : 0));
      const long long last = line.part_of(base + fc + (u > 0 ? 2 * u - 1 : 0));
      pieces += last - first + 1;
      base += 2 * u + 2 * fc;
    }
  }
  if (tid == 0) C[batch] = total;
  long long ptotal;
  long long pbase = block_exclusive_scan<NT>(pieces, scratch, &ptotal);
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < batch) {
      num_splits[b] = (int32_t)pbase;
      if constexpr (kSlInLds) NS_lds[b] = (int32_t)pbase;
      const long long cb = C[b];
      const long long u = units_of(SL(b));
      const long long first = line.part_of(cb + fc + (u > 0 ? 1 : 0));
      const long long last = line.part_of(cb + fc + (u > 0 ? 2 * u - 1 : 0));
      pbase += last - first + 1;
    }
  }
  if (tid == 0) {
    num_splits[batch] = (int32_t)ptotal;
    if constexpr (kSlInLds) NS_lds[batch] = (int32_t)ptotal;
  }
  __threadfence_block();
  __syncthreads();  // C and num_splits complete

  // Cost positions that decide a sequence's first and last part:
  //   last part  = part_of(KL_b), first part = part_of(KF_b)
  auto KL = [&](int b) -> long long {
    const long long cb = C[b], u2 = C[b + 1] - cb - 2 * fc;  // 2 U_b
    return cb + fc + (u2 > 0 ? u2 - 1 : 0);
  };
  auto KF = [&](int b) -> long long {
    const long long cb = C[b];
    return cb + fc + (C[b + 1] - cb - 2 * fc > 0 ? 1 : 0);
  };

  // 3. per part: first sequence with last part >= p, last with first part <= p.
  for (int p = tid; p < num_parts; p += NT) {
    const long long lo_key = line.first_of(p);       // last part >= p  <=>  KL >= F_p
    const long long hi_key = line.first_of(p + 1);   // first part <= p <=>  KF < F_{p+1}
    int lo = 0, hi = batch;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (KL(mid) >= lo_key) hi = mid; else lo = mid + 1;
    }
    const int bb = lo;
    lo = -1;
    hi = batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (KF(mid) < hi_key) lo = mid; else hi = mid - 1;
    }
    const int be = lo;
    i32x4 w0 = {0, 0, -1, 0}, w1 = {0, 0, 0, 0};
    if (bb < batch && be >= 0 && bb <= be) {
      const long long ub = (C[bb + 1] - C[bb]) / 2 - fc;
      const long long ue = (C[be + 1] - C[be]) / 2 - fc;
      long long u_begin = 0, u_end = 0;
      if (ub > 0) {  // units of bb whose midpoint lies before this part
        const long long a = lo_key - C[bb] - fc - 1;
        u_begin = a > 0 ? (a + 1) / 2 : 0;
      }
      if (ue > 0) {  // units of be whose midpoint lies before the next part
        const long long a = hi_key - C[be] - fc - 1;
        u_end = a > 0 ? (a + 1) / 2 : 0;
        if (u_end > ue) u_end = ue;
      }
      long long tok_end = u_end * kStage;
      if (tok_end > SL(be)) tok_end = SL(be);
      w0 = i32x4{bb, (int32_t)(u_begin * kStage), be, (int32_t)tok_end};
      // partial slot of bb's piece (num_splits[bb] + its split index), both
      // sequence lengths, and the partial slot of be's piece (split 0)
      w1 = i32x4{NS(bb) + (int32_t)(p - line.part_of(KF(bb))), SL(bb), SL(be), NS(be)};
    }
    i32x4* dst = reinterpret_cast<i32x4*>(meta + (long long)p * kMetaWords);
    dst[0] = w0;
    dst[1] = w1;
  }
}

// Fast variant for up to 1024 sequences and 4096 parts: 256 threads, every
// per-sequence quantity in LDS.  Each part finds its first and last sequence
// by binary search over the sequences' last and first parts (both
// non-decreasing).  Same output as sched_kernel.
constexpr int kSmallThreads = 256;
constexpr int kSmallBatch = 1024;
constexpr int kSmallParts = 4096;

__global__ __launch_bounds__(kSmallThreads) void sched_small_kernel(
    const int32_t* __restrict__ seqlens, int batch, int num_parts, int fixed_cost,
    int32_t* __restrict__ meta, int32_t* __restrict__ num_splits) {
  __shared__ long long C[kSmallBatch + 1];
  __shared__ int SL[kSmallBatch], FP[kSmallBatch], LP[kSmallBatch], NS[kSmallBatch];
  __shared__ long long scratch[kSmallThreads / 64];
  const int tid = threadIdx.x;
  const int per = (batch + kSmallThreads - 1) / kSmallThreads;
  const int b0 = tid * per;
  const long long fc = fixed_cost;

  long long local = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < batch) {
      const int n = seqlens[b];
      SL[b] = n;
      local += 2 * units_of(n) + 2 * fc;
    }
  }
  long long total;
  long long base = block_exclusive_scan<kSmallThreads>(local, scratch, &total);
  const PartLine line{total, num_parts};
  auto part_of = [&](long long x) -> int { return (int)line.part_of(x); };
  long long pieces = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < batch) {
      C[b] = base;
      const long long u = units_of(SL[b]);
      const int first = part_of(base + fc + (u > 0 ? 1 : 0));
      const int last = part_of(base + fc + (u > 0 ? 2 * u - 1 : 0));
      FP[b] = first;
      LP[b] = last;
      pieces += last - first + 1;
      base += 2 * u + 2 * fc;
    }
  }
  if (tid == 0) C[batch] = total;
  long long ptotal;
  long long pbase = block_exclusive_scan<kSmallThreads>(pieces, scratch, &ptotal);
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < batch) {
      num_splits[b] = (int32_t)pbase;
      NS[b] = (int32_t)pbase;
      pbase += LP[b] - FP[b] + 1;
    }
  }
  if (tid == 0) num_splits[batch] = (int32_t)ptotal;
  __syncthreads();  // FP, LP, C, NS complete

  for (int p = tid; p < num_parts; p += kSmallThreads) {
    // Part p's first sequence is the smallest b with LP[b] >= p (batch if
    // none: the part is empty); its last is the largest b with FP[b] <= p
    // (-1 if none).  Both arrays are non-decreasing in b.
    int lo = 0, hi = batch;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (LP[mid] >= p) hi = mid;
      else lo = mid + 1;
    }
    const int bb = lo;
    lo = 0;
    hi = batch;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (FP[mid] > p) hi = mid;
      else lo = mid + 1;
    }
    const int be = lo - 1;
    i32x4 w0 = {0, 0, -1, 0}, w1 = {0, 0, 0, 0};
    if (bb < batch && be >= 0 && bb <= be) {
      const long long lo_key = line.first_of(p), hi_key = line.first_of(p + 1);
      const long long ub = (C[bb + 1] - C[bb]) / 2 - fc;
      const long long ue = (C[be + 1] - C[be]) / 2 - fc;
      long long u_begin = 0, u_end = 0;
      if (ub > 0) {  // units of bb whose midpoint lies before this part
        const long long a = lo_key - C[bb] - fc - 1;
        u_begin = a > 0 ? (a + 1) / 2 : 0;
      }
      if (ue > 0) {  // units of be whose midpoint lies before the next part
        const long long a = hi_key - C[be] - fc - 1;
        u_end = a > 0 ? (a + 1) / 2 : 0;
        if (u_end > ue) u_end = ue;
      }
      long long tok_end = u_end * kStage;
      if (tok_end > SL[be]) tok_end = SL[be];
      w0 = i32x4{bb, (int32_t)(u_begin * kStage), be, (int32_t)tok_end};
      w1 = i32x4{NS[bb] + (p - FP[bb]), SL[bb], SL[be], NS[be]};
    }
    i32x4* dst = reinterpret_cast<i32x4*>(meta + (long long)p * kMetaWords);
    dst[0] = w0;
    dst[1] = w1;
  }
}

hipError_t launch_sched(const int32_t* seqlens, int batch, int num_parts, int fixed_cost,
                        int32_t* meta, int32_t* num_splits, hipStream_t stream) {
  if (batch <= kSmallBatch && num_parts <= kSmallParts)
    hipLaunchKernelGGL(sched_small_kernel, dim3(1), dim3(kSmallThreads), 0, stream, seqlens, batch,
                       num_parts, fixed_cost, meta, num_splits);
  else if (batch <= 1024)
    hipLaunchKernelGGL((sched_kernel<256, 1024>), dim3(1), dim3(256), 0, stream, seqlens, batch,
                       num_parts, fixed_cost, meta, num_splits);
  else
    hipLaunchKernelGGL((sched_kernel<1024, kMaxBatch>), dim3(1), dim3(1024), 0, stream, seqlens,
                       batch, num_parts, fixed_cost, meta, num_splits);
  return hipGetLastError();
}

}  // namespace mla
