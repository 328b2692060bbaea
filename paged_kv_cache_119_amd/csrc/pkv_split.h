// Work-balanced split shared by the decode kernels: the batch's chunks, row
// by row (sequence major), cut into equal slices, one per worker wavefront.
#pragma once

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

// Chunks of a row of L tokens; invalid and empty contexts have none.
template <int TC>
__device__ __forceinline__ int row_chunks(int L, int maxb, int B, int min_len = 1) {
  return (L >= min_len && L > 0 && L <= maxb * B) ? (L + TC - 1) / TC : 0;
}

// floor(x / d) for d >= 1 without the slow 64-bit integer division: a double
// estimate corrected to the exact quotient with 64-bit multiplies.
__device__ __forceinline__ uint64_t udiv64(uint64_t x, uint64_t d) {
  uint64_t q = (uint64_t)((double)x / (double)d);
  while (q > 0 && q * d > x) --q;
  while ((q + 1) * d <= x) ++q;
  return q;
}

__device__ __forceinline__ uint64_t uni64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Workers share the cost space in equal slices: worker w owns positions
// [min(total, w * slice), min(total, (w + 1) * slice)).  At most G workers,
// each slice at least kMinWorkerChunks long.
__device__ __forceinline__ uint64_t slice_of(uint64_t total, int G) {
  const uint64_t want = total / (uint64_t)kMinWorkerChunks;  // constant divisor
  const uint64_t workers = max((uint64_t)1, min((uint64_t)G, want));
  return max((uint64_t)1, udiv64(total + workers - 1, workers));
}

// Prefix of the chunk count over sequences into LDS (cum[0] = 0, cum[S] =
// total; a sequence has `rows` rows of row_chunks chunks each) and a copy of
// the context lengths, computed by one wavefront: each lane sums a contiguous
// run, then a scan.  Contexts shorter than min_len count as invalid.
template <int TC>
__device__ __forceinline__ void build_cost_prefix(const DecodeParams &a, int rows, int64_t *cum, int32_t *lens,
                                                  int lane, int min_len = 1) {
  const int S = a.S;
  const int per = (S + 63) / 64;
  const int s0 = min(S, lane * per);
  const int s1 = min(S, s0 + per);
  int64_t run = 0;
  for (int s = s0; s < s1; ++s) {
    const int L = a.lens[s];
    lens[s] = L;
    run += (int64_t)rows * row_chunks<TC>(L, a.maxb, a.B, min_len);
  }
  int64_t incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  int64_t x = incl - run;  // exclusive prefix of this lane's run
  if (lane == 0) cum[0] = 0;
  for (int s = s0; s < s1; ++s) {
    x += (int64_t)rows * row_chunks<TC>(lens[s], a.maxb, a.B, min_len);
    cum[s + 1] = x;
  }
}

}  // namespace pkv
