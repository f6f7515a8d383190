// fused.hip -- the whole path (plan, dispatch, expert gate/up and down,
// combine) in one persistent launch.
//
// "MORI CCO: Next-Generation Collective Communication Object for GPUs",
// sections "Mega-MoE: mega-kernel co-design with FlyDSL" (dispatch, expert
// GEMM and combine fused into one kernel, with no synchronisation between
// kernels) and "In-kernel compute-communication fusion" (the stages overlap
// at tile granularity inside one launch instead of at kernel boundaries).
// The stages do the same arithmetic as the five-launch path (plan.hip,
// dispatch.hip, expert.hip, combine.hip share their device code with this
// file), so plan, dispatch and combine-of-the-same-rows are bit-identical to
// it; the expert tiles are the same tiles, summed over the whole K range
// (this path never splits a tile into K-ranges).
//
// One workgroup per CU (the GEMM ring takes all of the LDS).  Every
// workgroup walks the phases in order, claiming work items from counters:
//   P1  histogram chunks of 2048 pairs; the workgroup finishing last builds
//       the counts, offsets, slot totals and status word (plan.hip), then
//       the tables this kernel needs (per-expert tile prefixes of both GEMMs
//       and of the 256-row m-tiles) and zeroes the dependency counters;
//   P2  rank chunks (stable positions), after the tables;
//   D   dispatch of 16-token blocks, after every rank chunk; each block then
//       counts the rows it delivered per expert;
//   G   gate/up tiles: per-XCD ranges of the tile list (neighbouring tiles
//       share weight panels in that XCD's L2), then the other XCDs' ranges;
//       a tile starts once every row of its expert has arrived, and counts
//       itself done for its (expert, m-tile);
//   W   down tiles, the same way; a tile starts once every gate/up tile of
//       its (expert, m-tile) is done;
//   C   combine of 16-token blocks; a block starts once the down tiles of
//       every row its tokens read are done.
// A workgroup leaves a phase only when every item of it has been claimed, and
// every wait is for items of an earlier phase, so the waits form no cycle.
// Producers publish with an agent-scope release (each wavefront's stores have
// completed; the XCD's L2 is written back) and consumers acquire at agent
// scope (L1 and non-coherent L2 lines invalidated) before reading: the XCDs'
// L2 caches are not coherent with each other.  Every wait is bounded: one
// that gives up sets the status word to CCO_ERR_TIMEOUT and an abort flag that
// ends every other wait at once, so the kernel always exits.
//
// SWITCHED OFF: the first launch of this kernel on the GPU (the small
// config) ended in a GPU memory fault whose cause is not yet shown; every
// address the kernel computes was checked in bounds on the CPU for that
// routing.  Until the cause is found the kernel is not built (define
// CCO_BUILD_FUSED to build it) and cco_moe_fused returns CCO_ERR_DISABLED.
#include "combine_impl.h"
#include "dispatch_impl.h"
#include "gemm_tile.h"
#include "plan_impl.h"

#ifdef CCO_BUILD_FUSED

namespace cco {
namespace {

constexpr int kFusedThreads = kGemmWaves * kWave;
static_assert(kFusedThreads == kPlanThreads, "the plan steps run on the GEMM's workgroup");
constexpr int kBlockTokens = 16;  // tokens per dispatch / combine item
constexpr int kFusedMaxTopk = 8;  // the general instantiation takes any K up to this
// Polls of a wait before it gives up: each poll sleeps ~256 cycles and reads
// two counters at agent scope (about a microsecond each), so about 2 s.
constexpr int kSpinLimit = 1 << 20;
constexpr int kErrTimeout = -8;  // CCO_ERR_TIMEOUT

// Counter words (FusedArgs::q), zero between launches: the last workgroup
// out clears them.
enum : int {
  Q_P1 = 0, Q_P2, Q_D, Q_C,  // item claims
  Q_EXIT,                    // workgroups done
  Q_SCAN,                    // tables built (0 / 1)
  Q_RANK,                    // rank chunks done
  Q_DISP,                    // dispatch items done
  Q_ABORT,                   // a wait gave up
  Q_G = 16,                  // [kNumXcd] gate/up claims per XCD range
  Q_W = Q_G + kNumXcd,       // [kNumXcd] down claims per XCD range
  Q_WORDS = Q_W + kNumXcd
};

struct FusedArgs {
  const int32_t *idx;    // [T][K] expert ids
  const u32x4 *x;        // [T][H] bf16 tokens
  const float *w;        // [T][K] routing weights
  u32x4 *out;            // [T][H] bf16 output
  int32_t T, n_pairs, nblk, nd, nc;
  GemmDesc gu, dn;       // the two GEMMs (gu.ntiles == 0: identity experts)
  int32_t *q;            // [Q_WORDS] counters
  int32_t *pre_g;        // [E + 1] gate/up tiles before expert e
  int32_t *pre_w;        // [E + 1] down tiles before expert e
  int32_t *pre_mt;       // [E + 1] 256-row m-tiles before expert e
  int32_t *arrived;      // [E] rows of each expert dispatched
  int32_t *gu_done;      // [m-tiles] gate/up tiles done per (expert, m-tile)
  int32_t *dn_done;      // [m-tiles] down tiles done per (expert, m-tile)
};

__device__ __forceinline__ int atomic_load_agent(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread-level bounded wait for *p >= target; false if it gave up (or
// another wait already had).
// (q: the counter words; the abort flag is among them.)
__device__ __forceinline__ bool spin_geq(const int32_t *q, const int32_t *p, int target) {
  if (atomic_load_agent(p) >= target) return true;
  for (int n = 0; n < kSpinLimit; ++n) {
    __builtin_amdgcn_s_sleep(4);
    if (atomic_load_agent(p) >= target) return true;
    if (atomic_load_agent(q + Q_ABORT) != 0) return false;
  }
  return false;
}

__device__ __forceinline__ void give_up(int32_t *q, int32_t *status) {
  __hip_atomic_store(q + Q_ABORT, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(status, kErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup-level: wait until *p >= target, then acquire (every thread may
// read what the producers published).
__device__ __forceinline__ void acquire_geq(int32_t *q, int32_t *status, const int32_t *p,
                                            int target) {
  if (threadIdx.x == 0) {
    if (!spin_geq(q, p, target)) give_up(q, status);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// Workgroup-level: publish this workgroup's stores, then add v to *p.
__device__ __forceinline__ void release_add(int32_t *p, int v) {
  wait_vmcnt<0>();  // this wavefront's stores have reached the L2
  __syncthreads();  // ... and every other wavefront's
  if (threadIdx.x == 0) __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Next item of a phase with one counter: thread 0 claims, every thread gets
// it (uniform).  The LDS word is free again when this returns.
__device__ __forceinline__ int claim(int32_t *ctr, int32_t *bc) {
  if (threadIdx.x == 0) bc[0] = atomicAdd(ctr, 1);
  __syncthreads();
  const int i = __builtin_amdgcn_readfirstlane(bc[0]);
  __syncthreads();
  return i;
}

// Next unit of a GEMM whose `total` units are split into kNumXcd contiguous
// ranges: this XCD's range first, then the others in turn (k, uniform, is
// the range being drained, counted from this XCD).  -1 when all are claimed.
__device__ __forceinline__ int claim_unit(int32_t *ctr, int total, int xcd, int &k,
                                          int32_t *bc) {
  if (threadIdx.x == 0) {
    int L = -1;
    while (k < kNumXcd) {
      const int y = (xcd + k) % kNumXcd;
      const int b = (int)((int64_t)total * y / kNumXcd);
      const int e = (int)((int64_t)total * (y + 1) / kNumXcd);
      if (e > b) {
        const int u = atomicAdd(&ctr[y], 1);
        if (u < e - b) {
          L = b + u;
          break;
        }
      }
      ++k;
    }
    bc[0] = L;
    bc[1] = k;
  }
  __syncthreads();
  const int L = __builtin_amdgcn_readfirstlane(bc[0]);
  k = __builtin_amdgcn_readfirstlane(bc[1]);
  __syncthreads();
  return L;
}

// Expert of list position L: the largest e with pre[e] <= L (pre is a
// non-decreasing prefix, L < pre[E]).
__device__ __forceinline__ int expert_of(const int32_t *pre, int E, int L) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= L)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// The tables of the GEMM phases, built by the workgroup that built the
// counts (it still holds the global exclusive prefix over experts in LDS,
// lh[0..E]).  Tables are [E + 1] prefixes; the dependency counters of this
// launch are zeroed here, before any phase that uses them can start.
__device__ __forceinline__ void build_tables(const MoeArgs &a, const FusedArgs &f, int32_t *lh,
                                             int32_t *scr) {
  const int E = a.E;
  const int tid = threadIdx.x;
  int32_t *tg = scr, *tw = scr + 1056, *tm = scr + 2 * 1056, *ws = scr + 3 * 1056;
  for (int e = tid; e < E; e += kFusedThreads) {
    // rows of e inside its slot (the plan drops rows past the capacity)
    const int s0 = (e / a.eps) * a.eps;
    const int64_t off = lh[e] - lh[s0];
    int64_t n = lh[e + 1] - lh[e];
    if (off + n > a.cap) n = a.cap - off;
    const int rows = n > 0 ? (int)n : 0;
    if (f.gu.ntiles > 0) {
      const ExpertTiles g = expert_tiles(rows, f.gu.ntiles);
      tg[e] = g.units;
      tw[e] = expert_tiles(rows, f.dn.ntiles).units;
      tm[e] = g.q + (g.rem > 0);
    } else {
      tg[e] = tw[e] = tm[e] = 0;
    }
    f.arrived[e] = 0;
  }
  __syncthreads();
  const int32_t ng = block_exclusive_scan_1024(tg, E, ws);
  const int32_t nw = block_exclusive_scan_1024(tw, E, ws);
  const int32_t nm = block_exclusive_scan_1024(tm, E, ws);
  for (int e = tid; e < E; e += kFusedThreads) {
    f.pre_g[e] = tg[e];
    f.pre_w[e] = tw[e];
    f.pre_mt[e] = tm[e];
  }
  if (tid == 0) {
    f.pre_g[E] = ng;
    f.pre_w[E] = nw;
    f.pre_mt[E] = nm;
  }
  for (int i = tid; i < nm; i += kFusedThreads) {
    f.gu_done[i] = 0;
    f.dn_done[i] = 0;
  }
  __syncthreads();
}

// One tile of a GEMM phase: decode list position L, wait for its inputs,
// compute, count it done.
template <bool SWIGLU>
__device__ __forceinline__ void fused_tile(const MoeArgs &a, const FusedArgs &f, char *smem,
                                           int L, int32_t *bc) {
  const GemmDesc &g = SWIGLU ? f.gu : f.dn;
  const int32_t *pre = SWIGLU ? f.pre_g : f.pre_w;
  if (threadIdx.x == 0) {
    const int e = expert_of(pre, a.E, L);
    bc[0] = e;
    bc[1] = L - pre[e];
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(bc[0]);
  const int r = __builtin_amdgcn_readfirstlane(bc[1]);
  __syncthreads();
  const int rows = __builtin_amdgcn_readfirstlane(rows_of(a, e));
  const ExpertTiles et = expert_tiles(rows, g.ntiles);
  const TileRef t = decode_tile(et, r, rows);
  const int mt = __builtin_amdgcn_readfirstlane(f.pre_mt[e]) + t.m_tile;
  if (SWIGLU) {
    acquire_geq(f.q, a.status, f.arrived + e, rows);
  } else {
    const ExpertTiles eg = expert_tiles(rows, f.gu.ntiles);
    acquire_geq(f.q, a.status, f.gu_done + mt, tiles_per_mtile(eg, t.m_tile, f.gu.ntiles));
  }
  const int nk = g.kdim / kBK;
  if (t.kind == 2)
    run_tile<kBM / 2, 2 * kBN, kStagesHalf, SWIGLU>(a, g, smem, e, t.n_tile, t.row0,
                                                    t.rows_valid, 0, nk, nullptr);
  else
    run_tile<kBM, kBN, kStages, SWIGLU>(a, g, smem, e, t.n_tile, t.row0, t.rows_valid, 0, nk,
                                        nullptr);
  release_add((SWIGLU ? f.gu_done : f.dn_done) + mt, 1);
}

// KT, NVL: top-k and row length of the dispatch and combine loops (see
// dispatch_impl.h, combine_impl.h); GV: vectors per lane of each row in
// flight in combine, chosen so that combine fits the registers beside the
// kernel's other state.
template <int KT, int NVL, int GV>
__global__ __launch_bounds__(kFusedThreads) void fused_kernel(MoeArgs a, FusedArgs f) {
  extern __shared__ __align__(1024) char smem[];
  int32_t *sm = (int32_t *)smem;
  // accumulators in AGPRs, as in the grouped GEMM (see expert.hip)
  asm volatile("" ::: "a0");
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int xcd = blockIdx.x % kNumXcd;
  const int K = a.K;
  int32_t *bc = sm + 7 * 1056;  // broadcast words, clear of the plan's and tables' LDS

  // ---- P1: histograms; the last one builds counts, offsets and tables
  for (;;) {
    const int i = claim(f.q + Q_P1, bc);
    if (i >= f.nblk) break;
    if (plan_count_chunk(a, f.idx, f.n_pairs, f.nblk, i, false, sm)) {
      build_tables(a, f, sm, sm + 1056);
      release_add(f.q + Q_SCAN, 1);
    }
  }
  // ---- P2: stable positions
  bool have_scan = false;
  for (;;) {
    const int i = claim(f.q + Q_P2, bc);
    if (i >= f.nblk) break;
    if (!have_scan) {
      acquire_geq(f.q, a.status, f.q + Q_SCAN, 1);
      have_scan = true;
    }
    plan_rank_chunk(a, f.idx, f.n_pairs, i, sm);
    release_add(f.q + Q_RANK, 1);
  }
  // ---- D: dispatch, 16 tokens per item, one wavefront per token
  const int nvec = a.H / 8;
  bool have_rank = false;
  for (;;) {
    const int i = claim(f.q + Q_D, bc);
    if (i >= f.nd) break;
    if (!have_rank) {
      acquire_geq(f.q, a.status, f.q + Q_RANK, f.nblk);
      have_rank = true;
    }
    const int t0 = i * kBlockTokens;
    const int t1 = min(f.T, t0 + kBlockTokens);
    for (int t = t0 + wave; t < t1; t += kGemmWaves)
      dispatch_token<KT, false, NVL>(a, f.x + (int64_t)t * nvec, nvec, nullptr, 0, f.w, f.idx, t,
                                     0, lane, K);
    // publish the rows, then count them per expert
    wait_vmcnt<0>();
    __syncthreads();
    if (tid == 0) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    for (int p = t0 * K + tid; p < t1 * K; p += kFusedThreads) {
      const int e = a.eid[p];
      const int pos = a.pos[p];
      if (e >= 0 && pos >= 0 && (int64_t)pos < a.cap) atomicAdd(f.arrived + e, 1);
    }
    release_add(f.q + Q_DISP, 1);
  }
  if (!have_scan) acquire_geq(f.q, a.status, f.q + Q_SCAN, 1);
  // ---- G and W: the expert GEMMs
  if (f.gu.ntiles > 0) {
    const int ng = __builtin_amdgcn_readfirstlane(f.pre_g[a.E]);
    int k = 0;
    for (;;) {
      const int L = claim_unit(f.q + Q_G, ng, xcd, k, bc);
      if (L < 0) break;
      fused_tile<true>(a, f, smem, L, bc);
    }
    const int nw = __builtin_amdgcn_readfirstlane(f.pre_w[a.E]);
    k = 0;
    for (;;) {
      const int L = claim_unit(f.q + Q_W, nw, xcd, k, bc);
      if (L < 0) break;
      fused_tile<false>(a, f, smem, L, bc);
    }
  }
  // ---- C: combine, 16 tokens per item
  const uint64_t src_win = f.gu.ntiles > 0 ? a.off_out : a.off_disp_x;
  have_rank = false;
  for (;;) {
    const int i = claim(f.q + Q_C, bc);
    if (i >= f.nc) break;
    if (!have_rank) {
      acquire_geq(f.q, a.status, f.q + Q_RANK, f.nblk);
      have_rank = true;
    }
    const int t0 = i * kBlockTokens;
    const int t1 = min(f.T, t0 + kBlockTokens);
    if (f.gu.ntiles > 0) {
      // every row the block reads: its (expert, m-tile) down tiles done
      bool ok = true;
      for (int p = t0 * K + tid; p < t1 * K; p += kFusedThreads) {
        const int e = a.eid[p];
        const int pos = a.pos[p];
        if (e < 0 || pos < 0 || (int64_t)pos >= a.cap) continue;
        const int rows = rows_of(a, e);
        const int m = (pos - a.expert_off[e]) / kBM;
        const ExpertTiles ed = expert_tiles(rows, f.dn.ntiles);
        ok = ok && spin_geq(f.q, f.dn_done + f.pre_mt[e] + m, tiles_per_mtile(ed, m, f.dn.ntiles));
      }
      if (!ok) give_up(f.q, a.status);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __syncthreads();
    } else {
      // identity experts: the rows are the dispatched tokens themselves
      acquire_geq(f.q, a.status, f.q + Q_DISP, f.nd);
    }
    for (int t = t0 + wave; t < t1; t += kGemmWaves)
      combine_token<KT, NVL, GV>(a, src_win, f.w, f.idx, f.out, t, 0, lane);
    __syncthreads();
  }
  // the last workgroup out has seen every counter exhausted: clear them for
  // the next launch (ordered by the stream)
  if (tid == 0 && atomicAdd(f.q + Q_EXIT, 1) == (int)gridDim.x - 1) {
    for (int w = 0; w < Q_WORDS; ++w) f.q[w] = 0;
  }
}

constexpr size_t kFusedLds =
    std::max((size_t)ring_bytes(kBM, kBN, kStages, kBK),
             (size_t)ring_bytes(kBM / 2, 2 * kBN, kStagesHalf, kBK));
static_assert(kFusedLds >= (size_t)(7 * 1056 + 8) * 4, "the plan, the tables and the broadcast words fit");

template <int KT, int NVL, int GV>
hipError_t launch_fused_kt(const MoeArgs &a, const FusedArgs &f, int nwg, hipStream_t st) {
  hipLaunchKernelGGL((fused_kernel<KT, NVL, GV>), dim3(nwg), dim3(kFusedThreads), kFusedLds, st,
                     a, f);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fused(const MoeArgs &a, const FusedBuffers &b, const int32_t *idx,
                        const uint16_t *x, const float *w, const uint16_t *w13,
                        const uint16_t *w2, uint16_t *out, int32_t T, int num_cus,
                        hipStream_t st) {
  FusedArgs f{};
  f.idx = idx;
  f.x = (const u32x4 *)x;
  f.w = w;
  f.out = (u32x4 *)out;
  f.T = T;
  f.n_pairs = T * a.K;
  f.nblk = (f.n_pairs + kPlanChunk - 1) / kPlanChunk;
  f.nd = f.nc = (T + kBlockTokens - 1) / kBlockTokens;
  f.q = b.q;
  f.pre_g = b.pre_g;
  f.pre_w = b.pre_w;
  f.pre_mt = b.pre_mt;
  f.arrived = b.arrived;
  f.gu_done = b.gu_done;
  f.dn_done = b.dn_done;
  f.gu.ntiles = 0;
  f.dn.ntiles = 0;
  if (a.I > 0) {
    f.gu = gemm_desc_gate_up(a, w13);
    f.dn = gemm_desc_down(a, w2);
  }
  const int nwg = gemm_workgroups(num_cus);
  // token rows of one wavefront: fixed-length loops for the common shapes
  const int per_lane = (a.H / 8) % kWave == 0 ? (a.H / 8) / kWave : 0;
  if (a.K == 8 && per_lane == 14) return launch_fused_kt<8, 14, 2>(a, f, nwg, st);
  if (a.K == 2 && per_lane == 8) return launch_fused_kt<2, 8, 4>(a, f, nwg, st);
  return launch_fused_kt<-kFusedMaxTopk, 0, 0>(a, f, nwg, st);
}

}  // namespace cco

#else  // CCO_BUILD_FUSED

namespace cco {

hipError_t launch_fused(const MoeArgs &, const FusedBuffers &, const int32_t *, const uint16_t *,
                        const float *, const uint16_t *, const uint16_t *, uint16_t *, int32_t,
                        int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace cco

#endif  // CCO_BUILD_FUSED
