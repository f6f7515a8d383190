// plan_impl.h -- the two steps of the routing plan as workgroup-level
// device functions: a chunk's histogram (with the counts, offsets and slot
// totals built by the workgroup that finishes last), and a chunk's stable
// positions.  Included by plan.hip (the plan launches), plan_noalloc.hip
// through those launches, and fused.hip (the single-launch path).
//
// "MORI CCO: Next-Generation Collective Communication Object for GPUs",
// section "Zero-copy MoE dispatch -> expert -> combine": dispatch returns a
// receive count per rank and a routing object that combine reuses.
#pragma once

#include "cco_internal.h"

namespace cco {
namespace {

constexpr int kPlanWaves = kPlanThreads / kWave;

// LDS words of each step for E experts.
__host__ __device__ constexpr int plan_count_lds_words(int E) { return E + 4 + kPlanWaves; }
__host__ __device__ constexpr int plan_rank_lds_words(int E) { return (kPlanWaves + 1) * E; }

// Exclusive scan of n (<= 4 * 256) ints in LDS, in place; returns the total.
// 256 threads, each owning 4 consecutive entries.
__device__ __forceinline__ int32_t block_exclusive_scan_1024(int32_t *v, int n,
                                                           int32_t *wave_sums) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  int32_t loc[4];
  int32_t sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = tid * 4 + q;
    loc[q] = (i < n) ? v[i] : 0;
    sum += loc[q];
  }
  // inclusive scan of the per-thread sums across the wavefront
  int32_t incl = sum;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int32_t up = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += up;
  }
  if (lane == kWave - 1) wave_sums[wave] = incl;
  __syncthreads();
  int32_t wave_base = 0, total = 0;
  for (int w = 0; w < kPlanWaves; ++w) {
    if (w < wave) wave_base += wave_sums[w];
    total += wave_sums[w];
  }
  int32_t run = wave_base + incl - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = tid * 4 + q;
    if (i < n) v[i] = run;
    run += loc[q];
  }
  __syncthreads();
  return total;
}

// Histogram of this workgroup's chunk; the workgroup that finishes last
// (every one, with `single`: the batch is one chunk) turns the histograms
// into counts, offsets, totals and the status word.
// `lds` holds at least plan_count_lds_words(E) words; returns true in the
// workgroup that built the counts and offsets.
__device__ __forceinline__ bool plan_count_chunk(const MoeArgs &a, const int32_t *__restrict__ idx,
                                                 int32_t n_pairs, int32_t nblk, int chunk,
                                                 bool single, int32_t *lds) {
  const int E = a.E;
  const int tid = threadIdx.x;
  int32_t *lh = lds;  // [E + 1]; entry E counts ids outside [0, E)
  int32_t *wave_sums = lds + E + 1;        // [kPlanWaves]
  int32_t &is_last = lds[E + 1 + kPlanWaves];
  int32_t &over = lds[E + 2 + kPlanWaves];

  for (int e = tid; e <= E; e += kPlanThreads) lh[e] = 0;
  __syncthreads();

  const int64_t base = (int64_t)chunk * kPlanChunk;
  int bad = 0;
#pragma unroll
  for (int i = 0; i < kPlanPerThread; ++i) {
    const int64_t f = base + i * kPlanThreads + tid;
    if (f < n_pairs) {
      const int e = idx[f];
      if ((unsigned)e < (unsigned)E)
        atomicAdd(&lh[e], 1);
      else
        bad = 1;
    }
  }
  if (bad) atomicAdd(&lh[E], 1);
  __syncthreads();

  int32_t *hb = a.hist + (int64_t)chunk * (E + 1);
  for (int e = tid; e <= E; e += kPlanThreads) hb[e] = lh[e];

  // publish this chunk's histogram, then take a ticket; the workgroup that
  // draws the last ticket sees every histogram
  __threadfence();
  __syncthreads();
  if (tid == 0) is_last = single || (atomicAdd(a.ticket, 1) == nblk - 1);
  __syncthreads();
  if (!is_last) return false;
  __threadfence();

  // per expert: total over chunks, and each chunk's exclusive prefix.  A
  // thread takes two of the E + 1 columns at a time (with 256 experts the
  // thread that owns expert 0 also owns the invalid-id column), and the
  // chunks' counts of both are loaded kBatch at a time, so that the loads
  // of a batch are in flight together rather than one after another
  constexpr int kBatch = 32;
  for (int e0 = tid; e0 <= E; e0 += 2 * kPlanThreads) {
    const int e1 = e0 + kPlanThreads;
    const bool two = e1 <= E;
    int32_t run0 = 0, run1 = 0;
    for (int b0 = 0; b0 < nblk; b0 += kBatch) {
      int32_t v0[kBatch], v1[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int64_t row = (int64_t)(b0 + i) * (E + 1);
        v0[i] = (b0 + i < nblk) ? a.hist[row + e0] : 0;
        v1[i] = (two && b0 + i < nblk) ? a.hist[row + e1] : 0;
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        if (b0 + i < nblk) {
          const int64_t row = (int64_t)(b0 + i) * (E + 1);
          a.hist[row + e0] = run0;
          run0 += v0[i];
          if (two) {
            a.hist[row + e1] = run1;
            run1 += v1[i];
          }
        }
    }
    lh[e0] = run0;
    if (two) lh[e1] = run1;
  }
  __syncthreads();
  const int32_t bad_total = lh[E];
  for (int e = tid; e < E; e += kPlanThreads) a.counts[e] = lh[e];
  __syncthreads();

  // global exclusive prefix over experts; slots are contiguous expert
  // ranges, so slot-local offsets are differences of it
  const int32_t total = block_exclusive_scan_1024(lh, E, wave_sums);
  lh[E] = total;
  __syncthreads();
  const int eps = a.eps;
  for (int e = tid; e < E; e += kPlanThreads) a.expert_off[e] = lh[e] - lh[(e / eps) * eps];
  if (tid == 0) over = 0;
  __syncthreads();
  for (int s = tid; s < a.S; s += kPlanThreads) {
    const int32_t st = lh[(s + 1) * eps] - lh[s * eps];
    a.slot_total[s] = st;
    if ((int64_t)st > a.cap) atomicOr(&over, 1);
  }
  __syncthreads();
  if (tid == 0) {
    a.status[0] = bad_total ? -5 /* CCO_ERR_BAD_EXPERT */ : (over ? -4 /* CCO_ERR_CAPACITY */ : 0);
    *a.ticket = 0;  // ready for the next plan (ordered by the stream)
  }
  return true;
}

// Stable positions of this workgroup's chunk (needs the counts and offsets).
// `lds` holds at least plan_rank_lds_words(E) words.
__device__ __forceinline__ void plan_rank_chunk(const MoeArgs &a, const int32_t *__restrict__ idx,
                                                int32_t n_pairs, int chunk, int32_t *lds) {
  const int E = a.E;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  int32_t *run = lds;          // [E]: next row of each expert for this chunk
  int32_t *wcnt = lds + E;     // [kPlanWaves][E]: pairs per expert in each wave this round

  // this thread's ids of every round (E marks an invalid pair or none),
  // loaded before the offsets so that all of these loads are in flight at
  // once
  const int64_t base = (int64_t)chunk * kPlanChunk;
  int ids[kPlanPerThread];
#pragma unroll
  for (int r = 0; r < kPlanPerThread; ++r) {
    const int64_t f = base + r * kPlanThreads + tid;
    const int v = f < n_pairs ? idx[f] : E;
    ids[r] = (unsigned)v < (unsigned)E ? v : E;
  }
  const int32_t *hb = a.hist + (int64_t)chunk * (E + 1);
  for (int e = tid; e < E; e += kPlanThreads) {
    run[e] = a.expert_off[e] + hb[e];
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) wcnt[w * E + e] = 0;
  }
  __syncthreads();

  // id bits to compare: ids are in [0, E], E itself marking an invalid pair
  const int nbits = 32 - __clz(E);
#pragma unroll
  for (int r = 0; r < kPlanPerThread; ++r) {
    const int64_t f = base + r * kPlanThreads + tid;
    const int e = ids[r];
    // lanes of this wavefront holding the same id
    uint64_t same = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const int bit = (e >> b) & 1;
      const uint64_t ones = __ballot(bit);
      same &= bit ? ones : ~ones;
    }
    const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(same >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)same, 0));
    const int cnt = __popcll(same);
    const bool leader = (rank == 0);
    if (leader && e < E) wcnt[wave * E + e] = cnt;
    __syncthreads();
    if (f < n_pairs) {
      int32_t p = -1;
      if (e < E) {
        p = run[e] + rank;
        for (int w = 0; w < wave; ++w) p += wcnt[w * E + e];
        if ((int64_t)p >= a.cap) p = -1;  // past the slot's capacity: dropped
      }
      a.pos[f] = p;
      a.eid[f] = (e < E) ? e : -1;
    }
    __syncthreads();
    if (leader && e < E) {
      atomicAdd(&run[e], cnt);
      wcnt[wave * E + e] = 0;
    }
  }
}

}  // namespace
}  // namespace cco
