// plan.hip -- routing plan: per-expert histogram, exclusive scan, stable
// positions ordered by the flat pair index t*K + j.
//
// "MORI CCO: Next-Generation Collective Communication Object for GPUs",
// section "Zero-copy MoE dispatch -> expert -> combine": dispatch returns a
// receive count per rank (total_recv) and a routing object that combine
// reuses.  Here the routing object is pos[t][j], the receive row of every
// pair, and the receive counts are slot_total[s].
//
// The plan is one stable counting sort by expert id (a single-digit LSD
// radix pass), split in two launches:
//   plan_count: each workgroup histograms a chunk of 2048 pairs in LDS and
//     publishes it; the last workgroup to finish (ticket counter) turns the
//     per-chunk histograms into per-chunk exclusive prefixes, writes the
//     expert counts, the slot-local expert offsets, the slot totals and the
//     status word, and resets the ticket.
//   plan_rank: each workgroup walks its chunk again in flat order, 256 pairs
//     at a time.  Inside a wavefront, lanes holding the same expert id are
//     found with one ballot per id bit (wave64 has no match instruction);
//     a lane's rank among them is the popcount of the lower lanes of that
//     mask (mbcnt).  Per-wave counts in LDS order the four wavefronts, and a
//     running count per expert orders the 256-pair rounds.  A pair whose row
//     would fall at or past the slot's capacity gets pos -1 (dropped; the
//     status word reports the overflow).
// A batch of one chunk (at most 2048 pairs, e.g. decode) runs both in one
// workgroup of one launch, plan_single_kernel.
#include <algorithm>

#include "plan_impl.h"

namespace cco {
namespace {

__global__ __launch_bounds__(kPlanThreads) void plan_count_kernel(MoeArgs a,
                                                                  const int32_t *__restrict__ idx,
                                                                  int32_t n_pairs, int32_t nblk) {
  extern __shared__ int32_t lds[];
  plan_count_chunk(a, idx, n_pairs, nblk, blockIdx.x, false, lds);
}

__global__ __launch_bounds__(kPlanThreads) void plan_rank_kernel(MoeArgs a,
                                                                 const int32_t *__restrict__ idx,
                                                                 int32_t n_pairs) {
  extern __shared__ int32_t lds[];
  plan_rank_chunk(a, idx, n_pairs, blockIdx.x, lds);
}

// The whole plan of a one-chunk batch in one workgroup: the offsets the
// count part writes are read back by the same workgroup after a barrier.
__global__ __launch_bounds__(kPlanThreads) void plan_single_kernel(MoeArgs a,
                                                                   const int32_t *__restrict__ idx,
                                                                   int32_t n_pairs) {
  extern __shared__ int32_t lds[];
  plan_count_chunk(a, idx, n_pairs, 1, 0, true, lds);
  __threadfence_block();
  __syncthreads();
  plan_rank_chunk(a, idx, n_pairs, 0, lds);
}

}  // namespace

hipError_t launch_plan_count(const MoeArgs &a, const int32_t *idx, int32_t n_pairs,
                             int32_t nblk, hipStream_t st) {
  const size_t lds = (size_t)plan_count_lds_words(a.E) * sizeof(int32_t);
  hipLaunchKernelGGL(plan_count_kernel, dim3(nblk), dim3(kPlanThreads), lds, st, a, idx,
                     n_pairs, nblk);
  return hipGetLastError();
}

hipError_t launch_plan_rank(const MoeArgs &a, const int32_t *idx, int32_t n_pairs,
                            int32_t nblk, hipStream_t st) {
  const size_t lds = (size_t)plan_rank_lds_words(a.E) * sizeof(int32_t);
  hipLaunchKernelGGL(plan_rank_kernel, dim3(nblk), dim3(kPlanThreads), lds, st, a, idx,
                     n_pairs);
  return hipGetLastError();
}

hipError_t launch_plan_single(const MoeArgs &a, const int32_t *idx, int32_t n_pairs,
                              hipStream_t st) {
  const size_t lds =
      (size_t)std::max(plan_count_lds_words(a.E), plan_rank_lds_words(a.E)) * sizeof(int32_t);
  hipLaunchKernelGGL(plan_single_kernel, dim3(1), dim3(kPlanThreads), lds, st, a, idx, n_pairs);
  return hipGetLastError();
}

}  // namespace cco
