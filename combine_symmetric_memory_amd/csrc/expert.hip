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
// (expert, m-tile, n-tile) built on the device from the plan's counts, so
// the host never learns the row counts.  A persistent grid walks the list:
// the tiles are split into kNumXcd contiguous ranges, one per XCD, so the
// workgroups sharing an L2 work on neighbouring tiles -- the m-tiles of one
// (expert, n-tile) reuse one weight panel, the n-tiles of one expert reuse
// its receive rows.
//
// Tile: BM x BN x BK, WM x WN wavefronts, each owning (BM/WM) x (BN/WN) as
// 32x32 blocks of v_mfma_f32_32x32x16_bf16.  Operands go global -> registers
// -> LDS (double buffered, rows padded by 16 bytes) -> registers; the next
// K-slice is fetched while the current one is multiplied.
//
// Gate/up fusion: the B tile interleaves 32-row blocks of the gate and up
// projections so that each wavefront holds, for the same 32 intermediate
// columns, the gate accumulator in block 2p and the up accumulator in block
// 2p+1 with identical lane layouts; the SwiGLU epilogue is elementwise.
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
};

// Rows of expert e that fit its slot (a slot overflow is reported by the
// plan; the rows past the capacity were never written).
__device__ __forceinline__ int rows_of(const MoeArgs &a, int e) {
  const int64_t off = a.expert_off[e];
  int64_t n = a.counts[e];
  if (off + n > a.cap) n = a.cap - off;
  return n > 0 ? (int)n : 0;
}

template <int BM, int BN, int BK, int WM, int WN, bool SWIGLU>
__global__ __launch_bounds__(WM *WN *kWave) void grouped_gemm_kernel(MoeArgs a, GemmDesc g) {
  constexpr int NT = WM * WN * kWave;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int LDS_STRIDE = BK + 8;  // elements; 16-byte pad per row
  constexpr int A_ELEMS = BM * LDS_STRIDE;
  constexpr int B_ELEMS = BN * LDS_STRIDE;
  constexpr int STAGE = A_ELEMS + B_ELEMS;
  constexpr int CPR = BK / 8;  // 16-byte chunks per tile row
  constexpr int CA = BM * CPR / NT;
  constexpr int CB = BN * CPR / NT;
  static_assert(BM * CPR % NT == 0 && BN * CPR % NT == 0, "tile/threads mismatch");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be 32-aligned");
  static_assert(!SWIGLU || FN % 2 == 0, "gate/up pairs need an even block count");

  extern __shared__ __align__(16) uint16_t smem[];
  __shared__ int32_t tile_prefix[kMaxExperts + 1];
  __shared__ int32_t scan_tmp[NT / kWave];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int E = a.E;

  // m-tiles per expert -> exclusive prefix (serial per wavefront chunk)
  {
    constexpr int PER = (kMaxExperts + NT - 1) / NT;
    int32_t loc[PER];
    int32_t sum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid * PER + q;
      loc[q] = (e < E) ? (rows_of(a, e) + BM - 1) / BM : 0;
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

  const int ntl = g.ntiles;
  const int total = tile_prefix[E] * ntl;
  const int nwg_x = gridDim.x / kNumXcd;
  const int xcd = blockIdx.x % kNumXcd;
  const int li = blockIdx.x / kNumXcd;
  const int t_end = (int)((int64_t)total * (xcd + 1) / kNumXcd);

  for (int L = (int)((int64_t)total * xcd / kNumXcd) + li; L < t_end; L += nwg_x) {
    // decode (expert, n-tile, m-tile): expert e owns [prefix[e], prefix[e+1]) * ntl
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_prefix[mid] * ntl <= L) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int mt_e = tile_prefix[e + 1] - tile_prefix[e];
    const int r = L - tile_prefix[e] * ntl;
    const int n_tile = r / mt_e;
    const int m_tile = r - n_tile * mt_e;
    const int row0 = m_tile * BM;
    const int rows_valid = min(BM, rows_of(a, e) - row0);
    const int slot = e / a.eps;
    const int64_t grow0 = (int64_t)a.expert_off[e] + row0;

    const uint16_t *A = (const uint16_t *)slot_addr(a, slot, g.a_win, (uint64_t)grow0 * g.lda * 2);
    const uint16_t *B = g.w + (int64_t)e * g.w_estride;

    const uint16_t *pa[CA];
    const uint16_t *pb[CB];
    int la[CA], lb[CB];
#pragma unroll
    for (int q = 0; q < CA; ++q) {
      const int c = tid + q * NT;
      const int row = c / CPR, kc = c % CPR;
      const int rr = row < rows_valid ? row : rows_valid - 1;
      pa[q] = A + (int64_t)rr * g.lda + kc * 8;
      la[q] = row * LDS_STRIDE + kc * 8;
    }
#pragma unroll
    for (int q = 0; q < CB; ++q) {
      const int c = tid + q * NT;
      const int row = c / CPR, kc = c % CPR;
      int64_t grow;
      if (SWIGLU) {
        const int wnb = row / TN, jb = (row % TN) / 32, sub = row % 32;
        const int i = n_tile * (BN / 2) + wnb * (TN / 2) + (jb >> 1) * 32 + sub;
        grow = (jb & 1) ? (int64_t)g.up_off + i : (int64_t)i;
      } else {
        grow = (int64_t)n_tile * BN + row;
      }
      pb[q] = B + grow * g.ldb + kc * 8;
      lb[q] = A_ELEMS + row * LDS_STRIDE + kc * 8;
    }

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    u32x4 ra[CA], rb[CB];
#pragma unroll
    for (int q = 0; q < CA; ++q) ra[q] = *(const u32x4 *)pa[q];
#pragma unroll
    for (int q = 0; q < CB; ++q) rb[q] = *(const u32x4 *)pb[q];
#pragma unroll
    for (int q = 0; q < CA; ++q) *(u32x4 *)(smem + la[q]) = ra[q];
#pragma unroll
    for (int q = 0; q < CB; ++q) *(u32x4 *)(smem + lb[q]) = rb[q];
    __syncthreads();

    const int nk = g.kdim / BK;
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      // prefetch the next K-slice; the last step re-reads its own slice so
      // that the loads are unconditional and the registers never leave VGPRs
      const int koff = (kt + 1 < nk ? kt + 1 : kt) * BK;
#pragma unroll
      for (int q = 0; q < CA; ++q) ra[q] = *(const u32x4 *)(pa[q] + koff);
#pragma unroll
      for (int q = 0; q < CB; ++q) rb[q] = *(const u32x4 *)(pb[q] + koff);
      // keep the prefetch at the top of the step, ahead of the MFMAs
      __builtin_amdgcn_sched_barrier(0);
      const uint16_t *sA = smem + cur * STAGE;
      const uint16_t *sB = sA + A_ELEMS;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int kofs = kk * 16 + (lane / 32) * 8;
        bf16x8 fa[FM], fb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          fa[i] = *(const bf16x8 *)(sA + (wm * TM + i * 32 + (lane & 31)) * LDS_STRIDE + kofs);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          fb[j] = *(const bf16x8 *)(sB + (wn * TN + j * 32 + (lane & 31)) * LDS_STRIDE + kofs);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      // the other buffer was last read before the previous barrier
      uint16_t *dst = smem + (cur ^ 1) * STAGE;
#pragma unroll
      for (int q = 0; q < CA; ++q) *(u32x4 *)(dst + la[q]) = ra[q];
#pragma unroll
      for (int q = 0; q < CB; ++q) *(u32x4 *)(dst + lb[q]) = rb[q];
      __syncthreads();
    }

    // epilogue: lane holds column (lane % 32) of each 32x32 block, rows
    // 8 * (v / 4) + 4 * (lane / 32) + v % 4 for accumulator element v
    uint16_t *C = (uint16_t *)slot_addr(a, slot, g.c_win, (uint64_t)grow0 * g.ldc * 2);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (SWIGLU) {
#pragma unroll
        for (int p = 0; p < FN / 2; ++p) {
          const int col = n_tile * (BN / 2) + wn * (TN / 2) + p * 32 + (lane & 31);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = wm * TM + i * 32 + (v / 4) * 8 + (lane / 32) * 4 + (v % 4);
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
            const int row = wm * TM + i * 32 + (v / 4) * 8 + (lane / 32) * 4 + (v % 4);
            if (row < rows_valid) C[(int64_t)row * g.ldc + col] = f32_to_bf16_rne(acc[i][j][v]);
          }
        }
      }
    }
  }
}

constexpr int kBM = 128, kBN = 128, kBK = 64, kWM = 2, kWN = 2;
constexpr int kGemmOccupancy = 2;  // workgroups per CU (LDS: 2 x 72 KiB)

template <bool SWIGLU>
hipError_t launch_gemm(const MoeArgs &a, const GemmDesc &g, int num_cus, hipStream_t st) {
  constexpr size_t lds = 2 * (size_t)(kBM + kBN) * (kBK + 8) * sizeof(uint16_t);
  int nwg = num_cus * kGemmOccupancy;
  nwg = ((nwg + kNumXcd - 1) / kNumXcd) * kNumXcd;
  auto kern = grouped_gemm_kernel<kBM, kBN, kBK, kWM, kWN, SWIGLU>;
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(kWM * kWN * kWave), lds, st, a, g);
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
  return launch_gemm<false>(a, g, num_cus, st);
}

}  // namespace cco
