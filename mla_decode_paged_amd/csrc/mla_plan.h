// Split-KV work plan, computed by one workgroup of T threads (the body of
// mla_get_metadata, and of the plan workgroup of mla_absorb_q_with_plan).
//
// FlashMLA's usage plans the tile schedule and split counts once per decode
// step from the cache lengths and reuses them for every layer (FlashMLA
// release news, usage example); the SC11 note likewise picks how to spread
// one decode over its cores by batch count and sequence length. This plan is
// the library's own: sequences with pages are laid end to end on a cost line,
// F + pages units each (F = split_overhead), and slot s takes the units
// [s q, (s+1) q) with q = ceil(total / num_slots). Every page lands in exactly
// one slot; the pages of one sequence inside one slot form a piece (a split).
//
// Block scans give each sequence's start on the cost line and its split
// prefix, then every slot finds its first and last sequence by binary search.
// All integer; the result is bit-identical to the interval definition above
// for any T.
#pragma once

#include <hip/hip_runtime.h>

#include "mla_device.h"
#include "mla_host.h"

namespace mla {

__device__ __forceinline__ int pages_of(int L) { return L > 0 ? (L + kPage - 1) / kPage : 0; }

// Exclusive prefix sum over the T threads of the workgroup; also returns the
// total. wave_sums holds T / 64 + 1 ints of LDS.
template <int T>
__device__ int block_exclusive_scan(int v, int* wave_sums, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wave_sums[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < T / 64; ++w) {
      const int x = wave_sums[w];
      wave_sums[w] = run;
      run += x;
    }
    wave_sums[T / 64] = run;
  }
  __syncthreads();
  const int excl = incl - v + wave_sums[wave];
  *total = wave_sums[T / 64];
  __syncthreads();  // wave_sums is reused by the next scan
  return excl;
}

// The plan for b sequences over n_slots slots, by the T threads of one
// workgroup. C and NS are LDS arrays of b + 1 ints (cost-line starts with
// C[b] = total, split prefix with NS[b] = all pieces); wave_sums T / 64 + 1.
template <int T>
__device__ void plan_block(const int32_t* seqlens, int b, int n_slots, int F, int32_t* meta, int32_t* ns_out,
                           int* C, int* NS, int* wave_sums) {
  const int tid = threadIdx.x;
  const int per = (b + T - 1) / T;
  const int lo = min(tid * per, b), hi = min(lo + per, b);

  int local = 0;
  for (int i = lo; i < hi; ++i) {
    const int pg = pages_of(seqlens[i]);
    local += pg > 0 ? F + pg : 0;
  }
  int total;
  int run = block_exclusive_scan<T>(local, wave_sums, &total);
  for (int i = lo; i < hi; ++i) {
    C[i] = run;
    const int pg = pages_of(seqlens[i]);
    run += pg > 0 ? F + pg : 0;
  }
  if (tid == 0) C[b] = total;
  const int q = total > 0 ? max(1, (total + n_slots - 1) / n_slots) : 1;

  int nsplit = 0;
  for (int i = lo; i < hi; ++i) {
    const int pg = pages_of(seqlens[i]);
    if (pg > 0) nsplit += (C[i] + F + pg - 1) / q - (C[i] + F) / q + 1;
  }
  int total_splits;
  run = block_exclusive_scan<T>(nsplit, wave_sums, &total_splits);
  for (int i = lo; i < hi; ++i) {
    NS[i] = run;
    const int pg = pages_of(seqlens[i]);
    if (pg > 0) run += (C[i] + F + pg - 1) / q - (C[i] + F) / q + 1;
  }
  if (tid == 0) NS[b] = total_splits;
  __syncthreads();

  for (int i = tid; i <= b; i += T) ns_out[i] = NS[i];

  for (int s = tid; s < n_slots; s += T) {
    int* m = meta + (long long)s * MLA_META_WORDS;
    const long long lo_u = (long long)s * q;
    const long long hi_u = min((long long)(s + 1) * q, (long long)total);
    int bf = 0, bl = -1;
    if (lo_u < total) {
      // first sequence whose cost interval ends past lo_u
      int a = 0, e = b;  // search in [a, e)
      while (a < e) {
        const int mid = (a + e) >> 1;
        if (C[mid + 1] > lo_u) e = mid; else a = mid + 1;
      }
      bf = a;
      if (C[bf] + F < hi_u) {
        // last sequence whose pages start before hi_u
        a = 0;
        e = b;
        while (a < e) {
          const int mid = (a + e) >> 1;
          if (C[mid] + F < hi_u) a = mid + 1; else e = mid;
        }
        bl = a - 1;
      }
    }
    if (bl < bf) {
      m[0] = 0; m[1] = 0; m[2] = -1; m[3] = 0; m[4] = 0;
    } else {
      const long long sb = C[bf] + F, sl = C[bl] + F;
      m[0] = bf;
      m[1] = (int)(max(lo_u, sb) - sb);
      m[2] = bl;
      m[3] = (int)(min(hi_u, (long long)C[bl + 1]) - sl);
      m[4] = NS[bf] + (s - (int)(sb / q));
    }
    m[5] = 0; m[6] = 0; m[7] = 0;
  }
}

// Host-side argument checks of the plan (shared by both entry points).
inline int check_plan_args(const char* fn, const int32_t* cache_seqlens, int b, int num_slots, int split_overhead,
                           const int32_t* tile_meta, const int32_t* num_splits) {
  if (!cache_seqlens || !tile_meta || !num_splits)
    return set_error(MLA_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
  if (b < 1 || b > MLA_MAX_BATCH)
    return set_error(MLA_ERR_INVALID_ARG, "%s: b must be in [1, %d] (got %d)", fn, MLA_MAX_BATCH, b);
  if (num_slots < 1 || num_slots > (1 << 20))
    return set_error(MLA_ERR_INVALID_ARG, "%s: num_slots must be in [1, 2^20] (got %d)", fn, num_slots);
  if (split_overhead < 0) return set_error(MLA_ERR_INVALID_ARG, "%s: split_overhead must be >= 0", fn);
  return MLA_OK;
}

}  // namespace mla
