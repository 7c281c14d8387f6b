// Packed (varlen) batches: which sequence a workgroup's tile belongs to.
//
// With tiles of R rows, sequence s (tokens cu[s] .. cu[s+1]-1) owns the tile
// slots [ts(s), ts(s) + ceil(len_s / R)) with ts(s) = floor(cu[s] / R) + s.
// Since floor((a + len) / R) - floor(a / R) >= floor(len / R), consecutive
// starts differ by at least ceil(len_s / R) (and by at least one), so the
// slots of different sequences never overlap, ts is strictly increasing, and
// all tiles fit in floor(N / R) + nseq slots (N = cu[nseq]); at most one slot
// per sequence stays empty.  A slot finds its sequence by a search over
// cu_seqlens: O(log nseq) loads (a binary search per lane, or a 64-way search
// per wave), whatever the number or the lengths of the sequences.
#pragma once

#include <hip/hip_runtime.h>

namespace diffattn {

__host__ __device__ __forceinline__ long long slot_start(const int* cu, int s, int R) {
  return (long long)(cu[s] / R) + s;
}

// Largest s in [0, nseq) with slot_start(s) <= t (nseq >= 1; slot_start(0) = 0).
__device__ __forceinline__ int slot_sequence(const int* cu, int nseq, long long t, int R) {
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (slot_start(cu, mid, R) <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// The same, found by a whole wave at once (every lane active, t uniform): the
// 64 lanes test 64 evenly spaced sequences, a ballot narrows the range 64-fold
// per round, so 2048 sequences take two rounds of one load each instead of
// eleven loads one after another.  slot_start is increasing in s, so the lanes
// that pass form a prefix.
__device__ __forceinline__ int slot_sequence_wave(const int* cu, int nseq, long long t, int R) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = nseq - 1;  // the answer lies in [lo, hi]
  while (lo < hi) {
    const int step = (hi - lo + 63) / 64;  // >= 1
    const int probe = min(lo + (lane + 1) * step, hi);
    const bool ok = slot_start(cu, probe, R) <= t;
    const int k = __popcll(__ballot(ok));  // probes lo + step .. lo + k step pass
    const int base = lo + k * step;
    if (base >= hi && k > 0) {
      lo = hi;
    } else {
      hi = min(base + step - 1, hi);
      lo = base;
    }
  }
  return lo;
}

// Slots to launch for nseq sequences of N tokens in all (N < 0: unknown, then
// bounded by nseq * max_len).
__host__ __forceinline__ long long slot_count(long long N, int nseq, long long max_len, int R) {
  const long long n = N >= 0 ? N : (long long)nseq * max_len;
  return n / R + nseq;
}

}  // namespace diffattn
