// expert.hip -- grouped SwiGLU expert GEMMs on gfx950 bf16 MFMA.
//
// "MORI CCO: Next-Generation Collective Communication Object for GPUs",
// section "Zero-copy MoE dispatch -> expert -> combine", step 2: the expert
// GEMM reads its input in place from the receive window and writes its
// output straight into the combine staging window, row i for row i.  The
// expert function itself (SwiGLU) is this library's reading:
//   gate/up:  h = bf16( silu(X Wg^T) * (X Wu^T) )   X = receive rows of e
//   down:     y = bf16( h Wd^T )
// with fp32 accumulation on the matrix cores.
//
// Both are "NT" GEMMs (A and B K-contiguous).  Work is a list of tiles
// built on the device from the plan's counts, so the host never learns the
// row counts: per expert, 256 x 256 tiles, and for a remainder of at most
// 128 rows a 128 x 512 tile.  A persistent grid (one workgroup per CU)
// walks the list: the tiles are split into kNumXcd contiguous ranges, one
// per XCD, so the workgroups sharing an L2 work on neighbouring tiles -- the
// m-tiles of one (expert, n-tile) reuse one weight panel, the n-tiles of one
// expert reuse its receive rows.  Once its own range is done, a workgroup
// takes what is left of the other XCDs' ranges.
//
// Inside a tile, 4 wavefronts (one per SIMD) interleave their MFMAs with
// LDS fragment reads and with direct global -> LDS loads of a later K-step
// into a ring of stages; see run_tile.
//
// Gate/up fusion: the B tile interleaves 32-row blocks of the gate and up
// projections so that each wavefront holds, for the same 32 intermediate
// columns, the gate accumulator in block 2p and the up accumulator in block
// 2p+1 with identical lane layouts; the SwiGLU epilogue is elementwise.
#include "gemm_tile.h"

namespace cco {
namespace {
// Persistent grouped GEMM over every expert's tiles.  List order inside an
// expert: n-tile major, m-tile minor, so the m-tiles of one weight panel run
// side by side; with a half remainder, the pair of column tiles (2j, 2j+1)
// lists the remainder tile j that spans both and then its full m-tiles.
// TAIL = false runs the whole tiles; TAIL = true, launched after it, the
// K-ranges of the split tiles (each instantiation keeps only its own
// epilogue, so the main one's register allocation is not disturbed).
// A8: the A rows are the 8-bit receive rows of an 8-bit dispatch (gate/up
// only), read as bf16(binary32(e4m3 * scale)).
template <bool SWIGLU, bool TAIL, bool A8 = false>
__global__ __launch_bounds__(kGemmWaves * kWave) void grouped_gemm_kernel(MoeArgs a, GemmDesc g) {
  constexpr int NT = kGemmWaves * kWave;
  // The ring of the running tile shape takes all of the LDS.  Between tiles
  // (and before the first) it is idle, and its first words serve as scratch
  // for the tile hand-out.
  extern __shared__ __align__(1024) char smem[];
  int32_t *scratch = (int32_t *)smem;

  // Keep the MFMA accumulators in AGPRs.  With two wavefronts per SIMD the
  // kernel fits in 256 registers, and the compiler then picks the form of
  // v_mfma that reads and writes C/D in ordinary VGPRs; on gfx950 that form
  // draws more power, and the clock drops (a register-only MFMA loop ran 1.83
  // PFLOP/s with AGPR accumulators vs 1.32 with VGPR ones, random bf16
  // operands).  An empty asm statement that clobbers an AGPR marks the
  // kernel as using AGPRs, which selects the AGPR form.
  asm volatile("" ::: "a0");
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int E = a.E;
  const int ntl = g.ntiles;

  // tiles per expert and their exclusive prefix over experts, held in
  // registers: thread t owns experts t * PER .. t * PER + PER - 1
  constexpr int PER = (kMaxExperts + NT - 1) / NT;
  int32_t loc[PER], pre[PER];
  int total;
  {
    int32_t sum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid * PER + q;
      loc[q] = (e < E) ? expert_tiles(rows_of(a, e), ntl).units : 0;
      sum += loc[q];
    }
    int32_t incl = sum;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int32_t up = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += up;
    }
    if (lane == kWave - 1) scratch[wave] = incl;
    __syncthreads();
    int32_t run = incl - sum;
    total = 0;
    for (int w = 0; w < kGemmWaves; ++w) {
      const int32_t wt = scratch[w];
      if (w < wave) run += wt;
      total += wt;
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      pre[q] = run;
      run += loc[q];
    }
    total = uniform(total);
    __syncthreads();
  }

  // tiles are split into kNumXcd contiguous ranges; the workgroups of XCD x
  // (block id % kNumXcd, the hardware's round-robin placement) take the
  // tiles of range x in order from a counter, so the tiles running at once
  // on one XCD are neighbours and share weight panels and receive rows in
  // that XCD's L2.  Ranges split by tile count cost unevenly (remainder
  // tiles run longer), so a workgroup whose range is exhausted takes tiles
  // from the others' counters.
  const int xcd = blockIdx.x % kNumXcd;
  // K-step and ring depths of this instantiation: the 8-bit rows always
  // take K-steps of 64 (whatever the build's K-step for bf16 rows)
  constexpr int BKI = A8 ? 64 : kBK;
  constexpr int SF = A8 ? 5 : kStages, SH = A8 ? 2 : kStagesHalf;
  const int nk = g.kdim / BKI;
  const int W = gridDim.x / kNumXcd;
  // own range first; then, once it is exhausted, the other XCDs' ranges in
  // turn (the tiles still left there at the end): the XCDs finish together
  // whatever their ranges cost.  A unit is the same work on any XCD, so
  // the result does not depend on who takes it.
  //
  // seen[]: the counters of every range, read once this workgroup's own
  // range is done; a range already exhausted then is skipped without an
  // atomic of its own (counters only grow during a launch).
  int32_t seen[kNumXcd];
  int32_t ahead = -1;  // thread 0: a unit of the current range claimed ahead
#pragma unroll
  for (int q = 0; q < kNumXcd; ++q) seen[q] = 0;
  for (int d = 0; d < kNumXcd; ++d) {
  const int rx = (xcd + d) % kNumXcd;  // the range's XCD
  if (d == 1) {
    __syncthreads();  // every thread has read the last unit
    if (tid < kNumXcd)
      scratch[4 + tid] = __hip_atomic_load(&g.queue[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kNumXcd; ++q) seen[q] = uniform(scratch[4 + q]);
  }
  int seen_rx = 0;
#pragma unroll
  for (int q = 0; q < kNumXcd; ++q) seen_rx = q == rx ? seen[q] : seen_rx;
  const int t_begin = (int)((int64_t)total * rx / kNumXcd);
  const int t_end = (int)((int64_t)total * (rx + 1) / kNumXcd);

  // The last round of an XCD's range is short when its U tiles leave a
  // small remainder R over the XCD's W workgroups.  Then the last R tiles
  // are cut into P ranges of K-steps each, which fills that round; every
  // range writes fp32 partial sums, and split_fixup_kernel adds a tile's
  // ranges in order once all of them are done.  The counter hands out
  // units: the U - R whole tiles (main launch), or the R * P ranges, tile
  // by tile (tail launch).
  const int U = t_end - t_begin;
  const int R = U % W;
  int P = (g.allow_split && U < kSplitMaxRounds * W && R > 0 && 2 * R <= W)
              ? min(W / R, nk / kMinSplitSteps)
              : 1;
  if (P < 2) P = 1;
  const int n_whole = P > 1 ? U - R : U;
  const int n_units = TAIL ? (P > 1 ? R * P : 0) : n_whole;
  if (d > 0 && seen_rx >= n_units) continue;

  for (;;) {
    __syncthreads();  // every thread has read the previous unit
    // the unit claimed during the previous tile of this range, if any
    if (tid == 0) scratch[0] = ahead >= 0 ? ahead : atomicAdd(&g.queue[rx], 1);
    ahead = -1;
    __syncthreads();
    // the unit and everything derived from it are wavefront-uniform: keep
    // them in scalar registers, so that per-K-step offsets stay scalar
    const int u = uniform(scratch[0]);
    if (u >= n_units) break;
    const int v = u;                     // tail: the unit is a K-range of a split tile
    const int L = t_begin + (TAIL ? n_whole + v / P : u);
    // the thread owning expert e with L in [pre, pre + loc) posts (e, L - pre)
#pragma unroll
    for (int q = 0; q < PER; ++q)
      if (L >= pre[q] && L < pre[q] + loc[q]) {
        scratch[1] = tid * PER + q;
        scratch[2] = L - pre[q];
      }
    __syncthreads();
    const int e = uniform(scratch[1]);
    const int r = uniform(scratch[2]);
    __syncthreads();  // scratch read everywhere before the ring refills
    const int rows = uniform(rows_of(a, e));
    const ExpertTiles et = expert_tiles(rows, ntl);
    const TileRef tr = decode_tile(et, r, rows);
    const int kind = tr.kind, n_tile = tr.n_tile, m_tile = tr.m_tile, row0 = tr.row0,
              rows_valid = tr.rows_valid;
    // K-range of this unit, and where its partial sums go
    int kb = 0, nkt = nk;
    float *part = nullptr;
    if (TAIL) {
      const int piece = v % P;
      kb = piece * nk / P;
      nkt = (piece + 1) * nk / P - kb;
      part = g.split_ws + (int64_t)(rx * W + v) * kSplitTileFloats;
      if (piece == 0 && tid == 0) {
        int32_t *d = g.split_desc + (rx * (W / 2) + v / P) * kSplitDescInts;
        d[0] = kind;
        d[1] = e;
        d[2] = n_tile;
        d[3] = row0;
        d[4] = rows_valid;
        d[5] = P;
        d[6] = rx * W + v;  // workspace slot of the first range
      }
    }
    // The next unit of this range is claimed once the K loop is done and
    // read after the epilogue, so the atomic's round trip overlaps the
    // epilogue.  Its address offset is an opaque zero: with a visibly
    // uniform address the compiler would derive the lane's result right
    // after the atomic and wait for it there.
    auto claim_ahead = [&]() __attribute__((always_inline)) {
      int z = 0;
      asm volatile("" : "+v"(z));
      if (tid == 0) ahead = atomicAdd(&g.queue[rx] + z, 1);
    };
    if (kind == 2)
      run_tile<kBM / 2, 2 * kBN, SH, SWIGLU, BKI, A8>(
          a, g, smem, e, n_tile, row0, rows_valid, kb, nkt, part, claim_ahead);
    else
      run_tile<kBM, kBN, SF, SWIGLU, BKI, A8>(a, g, smem, e, n_tile, row0, rows_valid, kb,
                                                   nkt, part, claim_ahead);
  }
  }
  // the last workgroup out has seen every counter exhausted: rearm them for
  // the next launch (ordered by the stream)
  if (tid == 0 && atomicAdd(&g.queue[kNumXcd], 1) == (int)gridDim.x - 1) {
#pragma unroll
    for (int q = 0; q <= kNumXcd; ++q) g.queue[q] = 0;
  }
}

// Sums the K-ranges of each split tile in range order (fp32), applies the
// epilogue of the GEMM (SwiGLU for gate/up) and writes the bf16 rows that
// exist.  kFixBands workgroups share a tile, one band of rows each, four
// output columns per thread and 16-byte loads; the last band to finish
// frees the tile's descriptor for the next launch.  Runs on the GEMM's
// stream after it, so every range's partial sums are visible.
constexpr int kFixBands = 16;

template <bool SWIGLU>
__global__ __launch_bounds__(256) void split_fixup_kernel(MoeArgs a, GemmDesc g) {
  int32_t *d = g.split_desc + (blockIdx.x / kFixBands) * kSplitDescInts;
  const int band = blockIdx.x % kFixBands;
  const int kind = uniform(d[0]);
  if (kind == 0) return;
  const int e = uniform(d[1]);
  const int n_tile = uniform(d[2]);
  const int row0 = uniform(d[3]);
  const int rows = uniform(d[4]);
  const int P = uniform(d[5]);
  const int slot0 = uniform(d[6]);
  const int BM = kind == 1 ? kBM : kBM / 2;
  const int BN = kind == 1 ? kBN : 2 * kBN;
  const int TN = BN / (kGemmWaves / (BM / 128));  // accumulator columns per wavefront
  const int out_cols = SWIGLU ? BN / 2 : BN;
  const float *ws = g.split_ws + (int64_t)slot0 * kSplitTileFloats;
  const int64_t grow0 = (int64_t)a.expert_off[e] + row0;
  uint16_t *C = (uint16_t *)slot_addr(a, e / a.eps, g.c_win, (uint64_t)grow0 * g.ldc * 2) +
                (int64_t)n_tile * out_cols;
  // four consecutive accumulator columns, summed over the ranges in order
  auto sum4 = [&](int row, int col) __attribute__((always_inline)) {
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int p = 0; p < P; ++p) {
      const float4 v = *(const float4 *)(ws + (int64_t)p * kSplitTileFloats + row * BN + col);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    return acc;
  };
  const int rpb = BM / kFixBands;
  const int r0 = band * rpb;
  const int nr = min(rows - r0, rpb);
  const int g4 = out_cols / 4;
  for (int idx = threadIdx.x; idx < nr * g4; idx += blockDim.x) {
    const int row = r0 + idx / g4, oc = (idx % g4) * 4;
    float y[4];
    if (SWIGLU) {
      // output column oc of wavefront column wnb: gate in accumulator
      // block 2 (rr / 32), up in the block after it
      const int wnb = oc / (TN / 2), rr = oc % (TN / 2);
      const int cg = wnb * TN + (rr / 32) * 64 + rr % 32;
      const float4 gs = sum4(row, cg), us = sum4(row, cg + 32);
      y[0] = silu(gs.x) * us.x;
      y[1] = silu(gs.y) * us.y;
      y[2] = silu(gs.z) * us.z;
      y[3] = silu(gs.w) * us.w;
    } else {
      const float4 ys = sum4(row, oc);
      y[0] = ys.x;
      y[1] = ys.y;
      y[2] = ys.z;
      y[3] = ys.w;
    }
    uint2 o;
    o.x = (uint32_t)f32_to_bf16_rne(y[0]) | ((uint32_t)f32_to_bf16_rne(y[1]) << 16);
    o.y = (uint32_t)f32_to_bf16_rne(y[2]) | ((uint32_t)f32_to_bf16_rne(y[3]) << 16);
    *(uint2 *)(C + (int64_t)row * g.ldc + oc) = o;
  }
  // every band has read the descriptor before the last one clears it
  __syncthreads();
  if (threadIdx.x == 0 && atomicAdd(&d[7], 1) == kFixBands - 1) {
    d[7] = 0;
    d[0] = 0;
  }
}

constexpr size_t kGemmLds =
    std::max(std::max((size_t)ring_bytes(kBM, kBN, kStages, kBK),
                      (size_t)ring_bytes(kBM / 2, 2 * kBN, kStagesHalf, kBK)),
             std::max((size_t)ring_bytes(kBM, kBN, 5, 64, true),
                      (size_t)ring_bytes(kBM / 2, 2 * kBN, 2, 64, true)));

// The tail and fixup launches follow only when the GEMM may split, that is
// when it can have fewer than kSplitMaxRounds rounds: every expert's rows R
// take at least ntiles * R / kBM tiles, so T * K routed rows take at least
// ntiles * T * K / kBM.
template <bool SWIGLU, bool A8 = false>
hipError_t launch_gemm(const MoeArgs &a, GemmDesc g, int32_t T, int num_cus, hipStream_t st) {
  const int nwg = gemm_workgroups(num_cus);
  const int64_t min_tiles = (int64_t)g.ntiles * T * a.K / kBM;
  // a tile is cut into at least two ranges of kMinSplitSteps K-steps, so a
  // shorter K never splits
  g.allow_split = min_tiles < (int64_t)kSplitMaxRounds * nwg &&
                  g.kdim / (A8 ? 64 : kBK) >= 2 * kMinSplitSteps;
  hipLaunchKernelGGL((grouped_gemm_kernel<SWIGLU, false, A8>), dim3(nwg), dim3(kGemmWaves * kWave),
                     kGemmLds, st, a, g);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !g.allow_split) return err;
  // the split tiles' K-ranges, with counters of their own
  GemmDesc gt = g;
  gt.queue = g.queue + 2 * (kNumXcd + 1);
  hipLaunchKernelGGL((grouped_gemm_kernel<SWIGLU, true, A8>), dim3(nwg), dim3(kGemmWaves * kWave),
                     kGemmLds, st, a, gt);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  // kFixBands workgroups per descriptor (at most half an XCD's workgroups
  // per XCD); those of free descriptors return at once
  hipLaunchKernelGGL(split_fixup_kernel<SWIGLU>, dim3(nwg / 2 * kFixBands), dim3(256), 0, st, a,
                     g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_gate_up(const MoeArgs &a, const uint16_t *w13, int32_t T, int num_cus,
                                 int32_t a8_ns, hipStream_t st) {
  GemmDesc g = gemm_desc_gate_up(a, w13);
  g.queue = a.gemm_queue;
  g.split_ws = a.split_ws;
  g.split_desc = a.split_desc;
  if (a8_ns < 0) return launch_gemm<true>(a, g, T, num_cus, st);
  // 8-bit rows: blocks of H / ns values, 2^kshift K-steps each (checked by
  // the caller: a power of two)
  g.a8_ns = a8_ns;
  g.a8_kshift = 0;
  if (a8_ns > 0)
    while ((64 << g.a8_kshift) < a.H / a8_ns) ++g.a8_kshift;
  return launch_gemm<true, true>(a, g, T, num_cus, st);
}

hipError_t launch_expert_down(const MoeArgs &a, const uint16_t *w2, int32_t T, int num_cus,
                              hipStream_t st) {
  GemmDesc g = gemm_desc_down(a, w2);
  g.queue = a.gemm_queue + kNumXcd + 1;
  g.split_ws = a.split_ws;
  g.split_desc = a.split_desc;
  return launch_gemm<false>(a, g, T, num_cus, st);
}

}  // namespace cco


