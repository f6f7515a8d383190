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
// expert reuse its receive rows.
//
// Inside a tile, 8 wavefronts in two groups alternate between a memory
// phase (LDS fragment reads, then direct global -> LDS loads of a later
// K-step into a ring of stages) and a compute phase (MFMAs only); see
// run_tile.
//
// Gate/up fusion: the B tile interleaves 32-row blocks of the gate and up
// projections so that each wavefront holds, for the same 32 intermediate
// columns, the gate accumulator in block 2p and the up accumulator in block
// 2p+1 with identical lane layouts; the SwiGLU epilogue is elementwise.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "cco_internal.h"

namespace cco {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

struct GemmDesc {
  uint64_t a_win;        // A rows: window of the expert's slot, row stride lda
  int32_t lda;
  const uint16_t *w;     // B: weights of expert 0; expert e at w + e * w_estride
  int64_t w_estride;
  int32_t ldb;
  uint64_t c_win;        // C rows: window of the expert's slot, row stride ldc
  int32_t ldc;
  int32_t kdim;          // reduction length
  int32_t ntiles;        // tiles along N
  int32_t up_off;        // gate/up: first row of the up projection (= I)
  int32_t *queue;        // [kNumXcd] next-tile counters + [1] exit counter
};

// Rows of expert e that fit its slot (a slot overflow is reported by the
// plan; the rows past the capacity were never written).
__device__ __forceinline__ int rows_of(const MoeArgs &a, int e) {
  const int64_t off = a.expert_off[e];
  int64_t n = a.counts[e];
  if (off + n > a.cap) n = a.cap - off;
  return n > 0 ? (int)n : 0;
}

// Wait until at most N vector-memory operations of this wavefront are in
// flight (the direct-to-LDS loads included).
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8), issued through the builtin so that the
// compiler's own wait insertion sees them.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without the memory fence of __syncthreads(): that fence
// waits for every outstanding load, prefetches of later stages included.
// Callers order their own LDS traffic with explicit vmcnt waits.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

// One 16-byte-per-lane direct load from global memory into LDS: lane l's
// 16 bytes land at lds_base + 16 * l (lds_base is wavefront-uniform).
__device__ __forceinline__ void load_lds_16(const void *gptr, char *lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t *)gptr, (lds_void_t *)lds_base, 16, 0, 0);
}

// LDS tile layout: rows of BK bf16 (ROWB bytes), unpadded, 16-byte chunks
// XOR-swizzled per row so that the 16 rows one fragment read touches fall
// on distinct bank groups: physical chunk = logical chunk ^ swz(row).
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  return (row / (16 / CPR)) % CPR;
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time
// indices for register arrays).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;

// Full tile 256 x 256 x 32 with a 4-deep ring; the 128 x 512 remainder tile
// (a 40 KiB stage) keeps the ring within the LDS with 3 stages.
constexpr int kBM = 256, kBN = 256, kBK = 32, kStages = 4, kStagesHalf = 3;

// Tile: BM rows x BN columns of one expert on 8 wavefronts, two per SIMD,
// in a ping-pong schedule.  Wavefront (g, s) -- group g = wave / 4, SIMD
// s = wave % 4 -- owns the 32-row blocks g, g+2, g+4, ... (interleaved, so a
// half-empty tile still splits evenly) and columns [s*BN/4, (s+1)*BN/4), as
// 32x32 blocks of v_mfma_f32_32x32x16_bf16.
//
// Both operands go global -> LDS through a STAGES-deep ring of direct
// 16-byte-per-lane loads (XOR-swizzled rows, free of bank conflicts).  Time
// is cut into phases by workgroup barriers; in every phase one group runs
// only MFMAs on fragments already in registers while the other reads its
// next fragments from LDS and then issues its share of a later stage's loads.
// Group 1 starts one barrier late, so the two wavefronts of a SIMD always
// sit in opposite phases and the matrix core never waits for memory.
//
// n_tile counts BN-wide column tiles (for gate/up: BN/2 intermediate
// columns, gate and up interleaved in 32-row blocks); rows [row0, row0 +
// rows_valid) of expert e are computed.  Every wavefront of the workgroup
// calls this with the same arguments.
template <int BM, int BN, int STAGES, bool SWIGLU>
__device__ __forceinline__ void run_tile(const MoeArgs &a, const GemmDesc &g, char *smem, int e,
                                         int n_tile, int row0, int rows_valid, int lag) {
  constexpr int BK = kBK;
  constexpr int NW = 8;
  constexpr int WM = 2, WN = 4;
  constexpr int TN = BN / WN;           // columns per wavefront
  constexpr int FN = TN / 32;           // 32-column blocks per wavefront
  constexpr int MB = BM / 32;           // 32-row blocks per tile
  constexpr int FM = MB / WM;           // 32-row blocks per wavefront
  constexpr int ROWB = BK * 2;          // bytes per LDS row
  constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;      // rows filled by one 1 KiB wavefront load
  constexpr int A_BYTES = BM * ROWB;
  constexpr int STAGE_BYTES = (BM + BN) * ROWB;
  constexpr int LA = BM / (RPI * NW);   // A loads per wavefront per stage
  constexpr int LB = BN / (RPI * NW);   // B loads per wavefront per stage
  constexpr int LPS = LA + LB;
  constexpr int KSUB = BK / 16;         // MFMA sub-steps per K-step
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "tile / wavefront mismatch");
  static_assert(!SWIGLU || FN % 2 == 0, "gate/up: gate and up blocks come in pairs");
  static_assert(32 % RPI == 0, "a load must not straddle two 32-row blocks");
  static_assert(STAGES >= 3 && (STAGES - 2) * LPS < 64, "stage count / vmcnt range");
  static_assert(FM >= 1 && FN >= 1, "tile too small for 8 wavefronts");

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = wave / WN;   // ping-pong group == row half
  const int wn = wave % WN;    // SIMD == column quarter
  const int slot = e / a.eps;
  const int64_t grow0 = (int64_t)a.expert_off[e] + row0;
  const int nk = g.kdim / BK;

  const char *A = slot_addr(a, slot, g.a_win, (uint64_t)grow0 * g.lda * 2);
  const char *B = (const char *)(g.w + (int64_t)e * g.w_estride);

  // byte offset (at k = 0) of the chunk each lane loads; rows past the
  // expert's last row re-read that row, so the load count never varies
  const int ld_row = lane / CPR;
  const int ld_pchunk = lane % CPR;
  uint32_t oa[LA], ob[LB];
#pragma unroll
  for (int q = 0; q < LA; ++q) {
    const int row = (q * NW + wave) * RPI + ld_row;
    const int rr = row < rows_valid ? row : rows_valid - 1;
    oa[q] = (uint32_t)rr * (uint32_t)g.lda * 2u + (uint32_t)((ld_pchunk ^ swz<CPR>(row)) * 16);
  }
#pragma unroll
  for (int q = 0; q < LB; ++q) {
    const int row = (q * NW + wave) * RPI + ld_row;
    uint32_t grow;
    if (SWIGLU) {
      // wavefront column block jb: pair jb / 2, gate (even) or up (odd)
      const int wnb = row / TN, jb = (row % TN) / 32, sub = row % 32;
      const int i = n_tile * (BN / 2) + wnb * (TN / 2) + (jb / 2) * 32 + sub;
      grow = (jb & 1) ? (uint32_t)(g.up_off + i) : (uint32_t)i;
    } else {
      grow = (uint32_t)(n_tile * BN + row);
    }
    ob[q] = grow * (uint32_t)g.ldb * 2u + (uint32_t)((ld_pchunk ^ swz<CPR>(row)) * 16);
  }
  // this wavefront's share of the loads of K-step kt (the tail re-loads the
  // last one), into its ring stage; K-steps run from lag, wrapping
  auto issue_stage = [&](int kt) __attribute__((always_inline)) {
    int kc = (kt < nk ? kt : nk - 1) + lag;
    if (kc >= nk) kc -= nk;
    char *sbase = smem + (kt % STAGES) * STAGE_BYTES;
    const char *Ak = A + (int64_t)kc * ROWB;
    const char *Bk = B + (int64_t)kc * ROWB;
#pragma unroll
    for (int q = 0; q < LA; ++q) load_lds_16(Ak + oa[q], sbase + (q * NW + wave) * 1024);
#pragma unroll
    for (int q = 0; q < LB; ++q)
      load_lds_16(Bk + ob[q], sbase + A_BYTES + (q * NW + wave) * 1024);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  // this wavefront's blocks (grp + 2 i) holding rows: a prefix i < nact
  const int mblocks = (rows_valid + 31) / 32;
  const int nact = min(FM, max(0, (mblocks - grp + WM - 1) / WM));

  // Ping-pong over K-steps, for a wavefront with NACT active row blocks.
  // Phase 2k:   group 0 reads K-step k (memory), group 1 multiplies k-1.
  // Phase 2k+1: group 0 multiplies k, group 1 reads k.
  // Stage k must be complete everywhere before phase 2k: every wavefront
  // waits for its own share of it before the barrier that ends phase 2k-1
  // (group 0 after multiplying k-1, group 1 after reading k-1).
  auto k_loop = [&](auto nact_c) __attribute__((always_inline)) {
    constexpr int NACT = decltype(nact_c)::value;
    constexpr int NF = NACT > 0 ? NACT : 1;
    bf16x8 fa[KSUB][NF], fb[KSUB][FN];
    // prologue: K-steps 0 .. STAGES-2 in flight, stage 0 complete
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p) issue_stage(p);
    wait_vmcnt<(STAGES - 2) * LPS>();
    stage_barrier();
    if (grp == 1) stage_barrier();  // group 1 runs one phase behind
    for (int kt = 0; kt < nk; ++kt) {
      // memory phase: this K-step's fragments, then a later stage's loads.
      // The fragment reads go first: a wavefront issues in order, and its
      // direct-to-LDS loads can sit in the issue queue until the address
      // unit takes them; the LDS reads must not wait behind them.
      if (NACT > 0) {
        const char *sA = smem + (kt % STAGES) * STAGE_BYTES;
        const char *sB = sA + A_BYTES;
#pragma unroll
        for (int s = 0; s < KSUB; ++s) {
          const int c = s * 2 + (lane >> 5);
#pragma unroll
          for (int i = 0; i < NACT; ++i) {
            const int row = (grp + i * WM) * 32 + (lane & 31);
            fa[s][i] = *(const bf16x8 *)(sA + row * ROWB + ((c ^ swz<CPR>(row)) * 16));
          }
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int row = wn * TN + j * 32 + (lane & 31);
            fb[s][j] = *(const bf16x8 *)(sB + row * ROWB + ((c ^ swz<CPR>(row)) * 16));
          }
        }
      }
      issue_stage(kt + STAGES - 1);
      wait_lgkmcnt0();
      if (grp == 1) wait_vmcnt<(STAGES - 2) * LPS>();  // own share of stage kt+1
      stage_barrier();
      // compute phase
#pragma unroll
      for (int s = 0; s < KSUB; ++s)
#pragma unroll
        for (int i = 0; i < NACT; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
      if (grp == 0) wait_vmcnt<(STAGES - 2) * LPS>();  // own share of stage kt+1
      stage_barrier();
    }
    if (grp == 0) stage_barrier();  // both groups pass the same number of barriers
    wait_vmcnt<0>();  // the tail's re-loads land before the ring is reused
  };
  // one specialisation per active-block count (wavefront-uniform branch)
  static_for<FM + 1>([&](auto c) __attribute__((always_inline)) {
    if (nact == decltype(c)::value) k_loop(c);
  });
  // every wavefront is done with the LDS before the next tile refills it
  __syncthreads();

  // epilogue: lane holds column (lane % 32) of each 32x32 block, rows
  // 8 * (v / 4) + 4 * (lane / 32) + v % 4 for accumulator element v
  uint16_t *C = (uint16_t *)slot_addr(a, slot, g.c_win, (uint64_t)grow0 * g.ldc * 2);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if (i >= nact) continue;
    const int rb = (grp + i * WM) * 32;
    if (SWIGLU) {
#pragma unroll
      for (int p = 0; p < FN / 2; ++p) {
        const int col = n_tile * (BN / 2) + wn * (TN / 2) + p * 32 + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = rb + (v / 4) * 8 + (lane / 32) * 4 + (v % 4);
          if (row < rows_valid) {
            const float h = silu(acc[i][2 * p][v]) * acc[i][2 * p + 1][v];
            C[(int64_t)row * g.ldc + col] = f32_to_bf16_rne(h);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n_tile * BN + wn * TN + j * 32 + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = rb + (v / 4) * 8 + (lane / 32) * 4 + (v % 4);
          if (row < rows_valid) C[(int64_t)row * g.ldc + col] = f32_to_bf16_rne(acc[i][j][v]);
        }
      }
    }
  }
}

// Work list of one expert: its rows R = 256 q + r are covered by q full
// 256-row m-tiles and, for r > 0, a remainder.  A remainder of more than 128
// rows is one more 256-row m-tile; one of at most 128 rows is a 128-row tile
// twice as wide (when the column tiles pair up), so a few leftover rows cost
// half the work of a full tile instead of all of it.
struct ExpertTiles {
  int q;       // full 256-row m-tiles
  int rem;     // rows of the remainder (0: none)
  bool half;   // remainder as 128 x (2 BN) tiles
  int units;   // tiles in the list
};

__device__ __forceinline__ ExpertTiles expert_tiles(int rows, int ntl) {
  ExpertTiles t;
  t.q = rows / kBM;
  t.rem = rows - t.q * kBM;
  t.half = t.rem > 0 && t.rem <= kBM / 2 && ntl % 2 == 0;
  t.units = t.half ? (ntl / 2) * (2 * t.q + 1) : (t.q + (t.rem > 0)) * ntl;
  return t;
}

// Persistent grouped GEMM over every expert's tiles.  List order inside an
// expert: n-tile major, m-tile minor, so the m-tiles of one weight panel run
// side by side; with a half remainder, the pair of column tiles (2j, 2j+1)
// lists its full m-tiles and then the remainder tile j that spans both.
template <bool SWIGLU>
__global__ __launch_bounds__(8 * kWave) void grouped_gemm_kernel(MoeArgs a, GemmDesc g) {
  constexpr int NT = 8 * kWave;
  extern __shared__ __align__(1024) char smem[];  // the ring of the running tile shape
  __shared__ int32_t tile_prefix[kMaxExperts + 1];
  __shared__ int32_t scan_tmp[8];
  __shared__ int32_t next_tile;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int E = a.E;
  const int ntl = g.ntiles;

  // tiles per expert -> exclusive prefix over experts
  {
    constexpr int PER = (kMaxExperts + NT - 1) / NT;
    int32_t loc[PER];
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
    if (lane == kWave - 1) scan_tmp[wave] = incl;
    __syncthreads();
    int32_t run = incl - sum;
    for (int w = 0; w < wave; ++w) run += scan_tmp[w];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid * PER + q;
      if (e <= E) tile_prefix[e] = run;
      run += loc[q];
    }
    if (tid == NT - 1) tile_prefix[E] = run;  // the total (E may equal NT * PER)
    __syncthreads();
  }

  const int total = tile_prefix[E];
  // tiles are split into kNumXcd contiguous ranges; the workgroups of XCD x
  // (block id % kNumXcd, the hardware's round-robin placement) take the
  // tiles of range x in order from a counter, so the tiles running at once
  // on one XCD are neighbours and share weight panels and receive rows in
  // that XCD's L2
  const int xcd = blockIdx.x % kNumXcd;
  const int t_begin = (int)((int64_t)total * xcd / kNumXcd);
  const int t_end = (int)((int64_t)total * (xcd + 1) / kNumXcd);
  const int nk = g.kdim / kBK;

  for (;;) {
    if (tid == 0) next_tile = t_begin + atomicAdd(&g.queue[xcd], 1);
    __syncthreads();
    const int L = next_tile;
    if (L >= t_end) break;

    // expert e owns list entries [prefix[e], prefix[e+1])
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_prefix[mid] <= L) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int rows = rows_of(a, e);
    const ExpertTiles et = expert_tiles(rows, ntl);
    const int r = L - tile_prefix[e];
    // Tiles sharing a weight panel or receive rows run side by side on one
    // XCD; rotating the K order by a small tile-dependent lag keeps them from
    // missing the same L2 lines at the same moment.
    if (et.half) {
      const int per = 2 * et.q + 1;
      const int j = r / per;
      const int rr = r - j * per;
      if (rr < 2 * et.q) {
        const int n_tile = 2 * j + rr / et.q;
        const int m_tile = rr % et.q;
        run_tile<kBM, kBN, kStages, SWIGLU>(a, g, smem, e, n_tile, m_tile * kBM, kBM,
                                            (n_tile % 8 + m_tile % 4) % nk);
      } else {
        run_tile<kBM / 2, 2 * kBN, kStagesHalf, SWIGLU>(a, g, smem, e, j, et.q * kBM, et.rem,
                                                        (j % 8 + et.q % 4) % nk);
      }
    } else {
      const int mt_e = et.q + (et.rem > 0);
      const int n_tile = r / mt_e;
      const int m_tile = r - n_tile * mt_e;
      run_tile<kBM, kBN, kStages, SWIGLU>(a, g, smem, e, n_tile, m_tile * kBM,
                                          min(kBM, rows - m_tile * kBM),
                                          (n_tile % 8 + m_tile % 4) % nk);
    }
  }
  // the last workgroup out has seen every counter exhausted: rearm them for
  // the next launch (ordered by the stream)
  if (tid == 0 && atomicAdd(&g.queue[kNumXcd], 1) == (int)gridDim.x - 1) {
#pragma unroll
    for (int q = 0; q <= kNumXcd; ++q) g.queue[q] = 0;
  }
}

constexpr size_t kGemmLds =
    std::max((size_t)kStages * (kBM + kBN) * kBK * 2,
             (size_t)kStagesHalf * (kBM / 2 + 2 * kBN) * kBK * 2);

template <bool SWIGLU>
hipError_t launch_gemm(const MoeArgs &a, const GemmDesc &g, int num_cus, hipStream_t st) {
  int nwg = ((num_cus + kNumXcd - 1) / kNumXcd) * kNumXcd;  // one workgroup per CU
  auto kern = grouped_gemm_kernel<SWIGLU>;
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(8 * kWave), kGemmLds, st, a, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_gate_up(const MoeArgs &a, const uint16_t *w13, int num_cus,
                                 hipStream_t st) {
  GemmDesc g;
  g.a_win = a.off_disp_x;
  g.lda = a.H;
  g.w = w13;
  g.w_estride = (int64_t)2 * a.I * a.H;
  g.ldb = a.H;
  g.c_win = a.off_hbuf;
  g.ldc = a.I;
  g.kdim = a.H;
  g.ntiles = a.I / (kBN / 2);
  g.up_off = a.I;
  g.queue = a.gemm_queue;
  return launch_gemm<true>(a, g, num_cus, st);
}

hipError_t launch_expert_down(const MoeArgs &a, const uint16_t *w2, int num_cus,
                              hipStream_t st) {
  GemmDesc g;
  g.a_win = a.off_hbuf;
  g.lda = a.I;
  g.w = w2;
  g.w_estride = (int64_t)a.H * a.I;
  g.ldb = a.I;
  g.c_win = a.off_out;
  g.ldc = a.H;
  g.kdim = a.I;
  g.ntiles = a.H / kBN;
  g.up_off = 0;
  g.queue = a.gemm_queue + kNumXcd + 1;
  return launch_gemm<false>(a, g, num_cus, st);
}

}  // namespace cco
