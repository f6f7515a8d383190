// gemm_tile.h -- one tile of the grouped expert GEMMs on gfx950 bf16 MFMA,
// and the per-expert tile list.  Included by expert.hip (the grouped GEMM
// launches) and fused.hip (the single-launch path); everything here has
// internal linkage.
//
// "MORI CCO: Next-Generation Collective Communication Object for GPUs",
// section "Zero-copy MoE dispatch -> expert -> combine", step 2: the expert
// GEMM reads its rows in place from the receive window and writes its output
// straight into the combine staging window, row i for row i.
#pragma once

#include <algorithm>
#include <type_traits>
#include <utility>

#include "cco_internal.h"

namespace cco {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// fp32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32, which
// the compiler emits for a plain conversion (two values per instruction).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// silu(z) = z / (1 + e^-z); the reciprocal is the hardware's (about 1 ulp of
// fp32), far below the bf16 rounding that follows.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

struct GemmDesc {
  uint64_t a_win;        // A rows: window of the expert's slot, row stride lda
  int32_t lda;
  const uint16_t *w;     // B: weights of expert 0; expert e at w + e * w_estride
  int64_t w_estride;
  int64_t w_bytes;       // bytes of one expert's weight matrix
  int32_t ldb;
  uint64_t c_win;        // C rows: window of the expert's slot, row stride ldc
  int32_t ldc;
  int32_t kdim;          // reduction length
  int32_t ntiles;        // tiles along N
  int32_t up_off;        // gate/up: first row of the up projection (= I)
  int32_t *queue;        // [kNumXcd] next-tile counters + [1] exit counter
  int32_t allow_split;   // nonzero: the tail and fixup launches follow this GEMM
  float *split_ws;       // fp32 partial sums of split tiles: one slot per workgroup
  int32_t *split_desc;   // [workgroups / 2][kSplitDescInts] split tiles, kind 0 = free
  // 8-bit A rows (gate/up after an 8-bit dispatch): each row holds kdim e4m3
  // values and then a8_ns fp32 scales, one per block of kdim / a8_ns values
  // = 2^a8_kshift K-steps of 64; a8_ns == 0: no scales
  int32_t a8_ns;
  int32_t a8_kshift;
};

// Rows of expert e that fit its slot (a slot overflow is reported by the
// plan; the rows past the capacity were never written).
__device__ __forceinline__ int rows_of(const MoeArgs &a, int e) {
  const int64_t off = a.expert_off[e];
  int64_t n = a.counts[e];
  if (off + n > a.cap) n = a.cap - off;
  return n > 0 ? (int)n : 0;
}

// Wait until at most N vector-memory operations (the direct-to-LDS loads
// included) / at most N LDS reads of this wavefront are in flight.  LDS
// reads return in order, so a partial lgkmcnt wait names a prefix of them.
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8), issued through the builtin so that the
// compiler's own wait insertion sees them.  Both are scheduling barriers
// too: no instruction moves across a wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
  __builtin_amdgcn_sched_barrier(0);
}
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier without the memory fence of __syncthreads(): that fence
// waits for every outstanding load, prefetches of later stages included.
// Callers order their own LDS traffic with explicit vmcnt waits.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8_t;

// A wavefront-uniform value the compiler cannot prove uniform (it came from
// memory) moved into scalar registers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const char *uniform(const char *p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const char *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// LDS byte address (as the ds_* instructions see it) of a shared pointer.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const lds_char_t *)p;
}

// Buffer resource of a raw byte range (stride 0, 32-bit dword format word
// of the gfx9 family); loads past num_bytes return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_range_rsrc(const void *base,
                                                                  uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)num_bytes,
                                           0x00020000);
}

// One 16-byte-per-lane direct load into LDS: lane l's 16 bytes, read at
// byte voff (per lane) + soff (wavefront-uniform) of the range, land at
// lds_base + 16 * l (lds_base wavefront-uniform).  Only scalar work besides
// the load itself: the offsets are registers the caller keeps.
__device__ __forceinline__ void buffer_load_lds_16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                   uint32_t soff, char *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds_base, 16, (int)voff, (int)soff,
                                           0, 0);
}
// The same with 4 bytes per lane (lane l's dword lands at lds_base + 4 l).
__device__ __forceinline__ void buffer_load_lds_4(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                  uint32_t soff, char *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds_base, 4, (int)voff, (int)soff,
                                           0, 0);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const u32x2 lds_u32x2_t;
typedef __attribute__((address_space(3))) const float lds_f32_t;

// Eight OCP e4m3 values (bytes in K order) times their fp32 scale, as the
// bf16 A fragment of one MFMA: each value decoded exactly
// (v_cvt_pk_f32_fp8), multiplied by s in binary32 and rounded to bf16
// (v_cvt_pk_bf16_f32), both roundings to nearest even.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(u32x2 q, float s) {
  const f32x2 f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, false);
  const f32x2 f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, true);
  const f32x2 f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, false);
  const f32x2 f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, true);
  bf16x8 r;
  r[0] = (__bf16)(f0.x * s);
  r[1] = (__bf16)(f0.y * s);
  r[2] = (__bf16)(f1.x * s);
  r[3] = (__bf16)(f1.y * s);
  r[4] = (__bf16)(f2.x * s);
  r[5] = (__bf16)(f2.y * s);
  r[6] = (__bf16)(f3.x * s);
  r[7] = (__bf16)(f3.y * s);
  return r;
}

// Values 2Q, 2Q + 1 of the same conversion, into r (a quarter of the
// fragment, so that the work can be spread between MFMAs).
template <int Q>
__device__ __forceinline__ void e4m3x2_to_bf16(bf16x8 &r, u32x2 q, float s) {
  const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)(Q < 2 ? q.x : q.y), (Q & 1) != 0);
  r[2 * Q] = (__bf16)(f.x * s);
  r[2 * Q + 1] = (__bf16)(f.y * s);
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

// K-step of the expert GEMMs' main loop: 64 (rows read 128 bytes at a
// time) by default, or 32 (64 bytes at a time, twice the L1 -> L2 requests
// of the same bytes; about 1% slower on the DeepSeek-V3 shapes).  Both
// divide every K the boundary accepts (H a multiple of 256, I of 128).
#ifndef CCO_GEMM_BK
#define CCO_GEMM_BK 64
#endif
// Full tile 256 x 256 and the 128 x 512 remainder tile.  With K-steps of
// 32: a 5-deep ring of 32 KiB stages, and a 4-deep one of 40 KiB.  With
// K-steps of 64 the full tile keeps its operands in rings of their own, two
// 32 KiB slots of A and three of B (STAGES == 5 names that layout), and the
// remainder tile two stages of 80 KiB.  Every ring fits the 160 KiB of LDS,
// which the kernel keeps for it alone.
constexpr int kBM = 256, kBN = 256, kBK = CCO_GEMM_BK;
static_assert(kBK == 32 || kBK == 64, "K-step of 32 or 64");
constexpr int kStages = 5, kStagesHalf = kBK == 64 ? 2 : 4;
constexpr int kGemmLdsBytes = 160 * 1024;

// LDS bytes of a tile's ring (STAGES == 5 with K-steps of 64: two A slots
// and three B slots)
constexpr int ring_bytes(int bm, int bn, int stages, int bk, bool a8 = false) {
  const int a = a8 ? bm * bk + 1024 : bm * bk * 2;  // A slot: rows (and 8-bit rows' scales)
  const int b = bn * bk * 2;
  return (bk == 64 && stages == 5) ? 2 * a + 3 * b : stages * (a + b);
}

// Wavefronts per workgroup: one per SIMD.
constexpr int kGemmWaves = 4;

// Split of a short last round: a tile cut into K-ranges keeps at least this
// many K-steps per range.  Each range's fp32 partial sums take one
// workspace slot of kSplitTileFloats (either tile shape has that many
// accumulators).
constexpr int kMinSplitSteps = 8;
// Only GEMMs of fewer rounds than this split their last one: with more,
// the short round is a small part of the time, and the dynamic hand-out
// already fills much of it.
constexpr int kSplitMaxRounds = 4;
static_assert(kBM * kBN == kSplitTileFloats && (kBM / 2) * (2 * kBN) == kSplitTileFloats,
              "a workspace slot holds one tile's accumulators");

// Tile: BM rows x BN columns of one expert on 4 wavefronts, one per SIMD,
// each owning a 128 x 128 block of the output as 4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16 with the accumulators in AGPRs.  Wavefront w sits
// at (wm, wn) = (w / WN, w % WN) of a WM x WN grid; its row blocks are
// wm, wm + WM, wm + 2 WM, ... (interleaved, so a partly empty tile still
// splits evenly) and its columns [wn * 128, wn * 128 + 128).
//
// The LDS operand reads set the pace: a SIMD moves about 26 bytes per clock
// from LDS into registers, and a 4 x 4 block tile needs 8 fragment reads per
// 16 MFMAs (1 KiB each) -- half an MFMA's worth of time per read, which the
// MFMAs hide.  (Two wavefronts per SIMD halve the register budget; 4 x 2
// block tiles then need 12 reads per 16 MFMAs, more than the matrix core's
// time covers.)
//
// Both operands go global -> LDS through a STAGES-deep ring of direct
// 16-byte-per-lane buffer loads (XOR-swizzled rows, free of bank conflicts).
// A K-step of 32 is two MFMA sub-steps; while one sub-step's MFMAs run, the
// wavefront reads the next sub-step's fragments and issues its share of a
// later stage's loads between them.  One barrier per K-step, between its
// two sub-steps, makes the next stage visible to every wavefront and frees
// the ring slot of the previous one.
//
// BK = 64 (four sub-steps): one wavefront load covers 128 contiguous bytes
// of 8 rows instead of 64 bytes of 16, so a K-step's bytes take half the
// L1 -> L2 requests.  Two stages (the remainder tile): K-step kt reads stage
// kt % 2.  The one barrier per K-step sits in sub-step 3, after its first
// row of MFMAs: every wavefront has then read its last fragments of stage kt
// and has its share of stage kt+1 in LDS, so stage kt+1 is complete and
// stage kt's slot is free.  Right after it the wavefront reads the fragments
// of (kt+1, 0) and starts the loads of stage kt+2 into the freed slot, which
// go on through sub-steps 0 and 1 of K-step kt+1; they have landed by the
// barrier of K-step kt+1.
//
// Split rings (the full tile): the same sub-steps and barrier, but the
// weights, which come from HBM, are loaded two K-steps ahead of their use
// and the receive rows, mostly L2 hits, one.  One stage of 64 KiB in flight
// per CU leaves the HBM stream short of bytes in flight; a third 64 KiB
// stage does not fit, a third B slot of 32 KiB does.
//
// n_tile counts BN-wide column tiles (for gate/up: BN/2 intermediate
// columns, gate and up interleaved in 32-row blocks); rows [row0, row0 +
// rows_valid) of expert e are computed over the nkt K-steps from kb on.
// With part == nullptr the result goes to the expert's output rows;
// otherwise the fp32 sums of this K-range are written to part, row-major
// [BM][BN] in the accumulators' column order.  Every wavefront of the
// workgroup calls this with the same arguments.  after_kloop() runs once
// the K loop's loads have all landed, before the results are written (the
// caller issues the next tile's hand-out there, so that its round trip
// overlaps the epilogue).
struct NoHook {
  __device__ void operator()() const {}
};
template <int BM, int BN, int STAGES, bool SWIGLU, int BK = kBK, bool A8 = false,
          class Hook = NoHook>
__device__ __forceinline__ void run_tile(const MoeArgs &a, const GemmDesc &g, char *smem, int e,
                                         int n_tile, int row0, int rows_valid, int kb, int nkt,
                                         float *part, Hook after_kloop = Hook{}) {
  constexpr int NW = kGemmWaves;
  constexpr int WM = BM / 128;          // wavefront rows
  constexpr int WN = NW / WM;           // wavefront columns
  constexpr int TN = BN / WN;           // columns per wavefront
  constexpr int FN = TN / 32;           // 32-column blocks per wavefront
  constexpr int MB = BM / 32;           // 32-row blocks per tile
  constexpr int FM = MB / WM;           // 32-row blocks per wavefront
  constexpr int ROWB = BK * 2;          // bytes per LDS row (B, and bf16 A)
  constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;      // rows filled by one 1 KiB wavefront load
  // A8: 8-bit A rows, BK bytes per row, and after them the K-step's row
  // scales (one wavefront load of 64 rows' dwords each, 256 rows' worth)
  constexpr int ROWB_A = A8 ? BK : ROWB;
  constexpr int CPR_A = ROWB_A / 16;
  constexpr int RPI_A = 1024 / ROWB_A;
  constexpr int A_DATA = BM * ROWB_A;
  constexpr int A_BYTES = A_DATA + (A8 ? 1024 : 0);
  constexpr int STAGE_BYTES = A_BYTES + BN * ROWB;
  constexpr int LAD = BM / (RPI_A * NW);     // A row loads per wavefront per stage
  constexpr int LA = LAD + (A8 ? 1 : 0);     // ... and the scale load
  constexpr int LB = BN / (RPI * NW);   // B loads per wavefront per stage
  constexpr int LPS = LA + LB;
  constexpr int KSUB = BK / 16;         // MFMA sub-steps per K-step
  // K-steps of 64 with STAGES == 5: separate rings for the operands, two
  // slots of A and three of B (each slot one K-step of one operand)
  constexpr bool SPLIT = KSUB == 4 && STAGES == 5;
  constexpr int B_BYTES = BN * ROWB;
  constexpr int RING_A = SPLIT ? 2 : STAGES;         // A slots (or whole stages)
  constexpr int B_RING_OFF = SPLIT ? RING_A * A_BYTES : A_BYTES;
  constexpr int RING_BYTES = SPLIT ? 2 * A_BYTES + 3 * B_BYTES : STAGES * STAGE_BYTES;
  static_assert(WM * WN == NW && FM == 4 && FN == 4, "4 x 4 blocks of 32 x 32 per wavefront");
  static_assert((KSUB == 2 && STAGES >= 3 && (STAGES - 2) * LPS < 64) ||
                    (KSUB == 4 && (STAGES == 2 || STAGES == 5) && LPS < 64),
                "K-steps of 32 with 3 or more stages, or of 64 with two stages or split rings");
  static_assert(BM % (RPI_A * NW) == 0 && BN % (RPI * NW) == 0, "tile / wavefront mismatch");
  static_assert(32 % RPI == 0 && 32 % RPI_A == 0, "a load must not straddle two 32-row blocks");
  static_assert(!A8 || (KSUB == 4 && BM <= 256), "8-bit A: K-steps of 64, at most 256 rows");
  static_assert(RING_BYTES <= kGemmLdsBytes, "the ring must fit the LDS");

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / WN;
  const int wn = wave % WN;
  // the tile's parameters are wavefront-uniform; keep them (and the operand
  // descriptors built from them) in scalar registers
  e = uniform(e);
  n_tile = uniform(n_tile);
  row0 = uniform(row0);
  rows_valid = uniform(rows_valid);
  kb = uniform(kb);
  const int slot = e / a.eps;
  const int64_t grow0 = (int64_t)uniform(a.expert_off[e]) + row0;
  const int nk = uniform(nkt);

  const char *A = uniform(slot_addr(a, slot, g.a_win, (uint64_t)grow0 * g.lda * 2));
  const char *B = uniform((const char *)(g.w + (int64_t)e * g.w_estride));
  // operand byte ranges: the tile's receive rows, the expert's weights
  const __amdgpu_buffer_rsrc_t ra =
      byte_range_rsrc(A, (uint32_t)rows_valid * (uint32_t)g.lda * 2u);
  const __amdgpu_buffer_rsrc_t rb = byte_range_rsrc(B, (uint32_t)g.w_bytes);

  // byte offset (at k = 0) of the chunk each lane loads; rows past the
  // expert's last row re-read that row, so the load count never varies
  const int ld_row = lane / CPR;
  const int ld_pchunk = lane % CPR;
  uint32_t oa[LA], ob[LB];
#pragma unroll
  for (int q = 0; q < LAD; ++q) {
    const int row = (q * NW + wave) * RPI_A + lane / CPR_A;
    const int rr = row < rows_valid ? row : rows_valid - 1;
    oa[q] = (uint32_t)rr * (uint32_t)g.lda * 2u +
            (uint32_t)(((lane % CPR_A) ^ swz<CPR_A>(row)) * 16);
    asm volatile("" : "+v"(oa[q]));
  }
  if constexpr (A8) {
    // the scale load: row wave * 64 + lane (rows past the tile's re-read
    // the last row; their scales are never used); scales follow the kdim
    // value bytes of the row
    const int row = wave * kWave + lane;
    const int rr = row < rows_valid ? row : rows_valid - 1;
    oa[LAD] = (uint32_t)rr * (uint32_t)g.lda * 2u + (uint32_t)g.kdim;
    asm volatile("" : "+v"(oa[LAD]));
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
    asm volatile("" : "+v"(ob[q]));
  }
  // LDS fragment addresses, per ring stage and MFMA sub-step.  The rows of
  // one wavefront's blocks differ by multiples of 32, so they share the row
  // swizzle and differ by constant offsets (folded into the instructions).
  // Kept opaque so the compiler does not recompute them inside the loop.
  // With split rings: A slot st for fa_addr, B slot 0 for fb_addr (slot s
  // adds s * B_BYTES).
  constexpr int NSA = RING_A, NSB = SPLIT ? 1 : STAGES;
  uint32_t fa_addr[NSA][KSUB], fb_addr[NSB][KSUB];
  // A8: the address of this lane's row scale (row block wm) in each A slot
  uint32_t fsc_addr[A8 ? NSA : 1];
  {
    const int l = lane & 31;
    const uint32_t base = lds_addr(smem);
    constexpr int SLOT_A = SPLIT ? A_BYTES : STAGE_BYTES;
    if constexpr (A8) {
#pragma unroll
      for (int st = 0; st < NSA; ++st) {
        fsc_addr[st] = base + st * SLOT_A + A_DATA + (wm * 32 + l) * 4;
        asm volatile("" : "+v"(fsc_addr[st]));
      }
    }
#pragma unroll
    for (int sk = 0; sk < KSUB; ++sk) {
      const int c = sk * 2 + (lane >> 5);
      const uint32_t lp = (uint32_t)(l * ROWB + ((c ^ swz<CPR>(l)) * 16));
      // 8-bit A: the sub-step's 16 values of row l are one 16-byte chunk;
      // lanes 32..63 take its second half
      const uint32_t lpa =
          A8 ? (uint32_t)(l * ROWB_A + ((sk ^ swz<CPR_A>(l)) * 16) + (lane >> 5) * 8) : lp;
#pragma unroll
      for (int st = 0; st < NSA; ++st) {
        fa_addr[st][sk] = base + st * SLOT_A + wm * 32 * ROWB_A + lpa;
        asm volatile("" : "+v"(fa_addr[st][sk]));
      }
#pragma unroll
      for (int st = 0; st < NSB; ++st) {
        fb_addr[st][sk] = base + st * STAGE_BYTES + B_RING_OFF + wn * TN * ROWB + lp;
        asm volatile("" : "+v"(fb_addr[st][sk]));
      }
    }
  }

  // the K-step's byte offset into an A row (soff is the B rows' offset, 2
  // bytes per value), and the byte offset of its scale within the row's
  // scales (soff / ROWB is the K-step)
  auto a_koff = [&](uint32_t soff) __attribute__((always_inline)) {
    return A8 ? soff >> 1 : soff;
  };
  auto a_scoff = [&](uint32_t soff) __attribute__((always_inline)) {
    return ((soff / ROWB) >> g.a8_kshift) * 4u;
  };
  // load q (0 .. LPS-1: A loads, then B loads) of this wavefront's share of
  // K-step kt (K-steps kb, kb + 1, ...; past the range the tail re-loads
  // the last one) into ring stage ST.  Scalar offsets only.
  auto issue_load = [&](auto st_c, auto q_c, uint32_t soff) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value, q = decltype(q_c)::value;
    char *sbase = smem + ST * STAGE_BYTES;
    if constexpr (q < LAD)
      buffer_load_lds_16(ra, oa[q], a_koff(soff), sbase + (q * NW + wave) * 1024);
    else if constexpr (q < LA)
      buffer_load_lds_4(ra, oa[q], a_scoff(soff), sbase + A_DATA + wave * 256);
    else
      buffer_load_lds_16(rb, ob[q - LA], soff, sbase + A_BYTES + ((q - LA) * NW + wave) * 1024);
  };
  // split rings: A load q into A slot SL; B load q into B slot bsl
  // (wavefront-uniform)
  auto issue_a = [&](auto sl_c, auto q_c, uint32_t soff) __attribute__((always_inline)) {
    constexpr int SL = decltype(sl_c)::value, q = decltype(q_c)::value;
    if constexpr (q < LAD)
      buffer_load_lds_16(ra, oa[q], a_koff(soff), smem + SL * A_BYTES + (q * NW + wave) * 1024);
    else
      buffer_load_lds_4(ra, oa[q], a_scoff(soff), smem + SL * A_BYTES + A_DATA + wave * 256);
  };
  auto issue_b = [&](int bsl, auto q_c, uint32_t soff) __attribute__((always_inline)) {
    constexpr int q = decltype(q_c)::value;
    buffer_load_lds_16(rb, ob[q], soff, smem + B_RING_OFF + bsl * B_BYTES + (q * NW + wave) * 1024);
  };
  auto k_offset = [&](int kt) __attribute__((always_inline)) {
    return (uint32_t)(kb + (kt < nk ? kt : nk - 1)) * ROWB;
  };

  // this wavefront's blocks (wm + WM i) holding rows: a prefix i < nact
  const int mblocks = (rows_valid + 31) / 32;
  const int nact = min(FM, max(0, (mblocks - wm + WM - 1) / WM));
  uint16_t *C = (uint16_t *)slot_addr(a, slot, g.c_win, (uint64_t)grow0 * g.ldc * 2);

  // The whole tile for a wavefront with NACT active row blocks: the
  // accumulators live only inside one specialisation.
  auto k_loop = [&](auto nact_c) __attribute__((always_inline)) {
    constexpr int NACT = decltype(nact_c)::value;
    constexpr int NF = NACT > 0 ? NACT : 1;
    f32x16 acc[NF][FN];
#pragma unroll
    for (int i = 0; i < NF; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    constexpr int NRD = NACT > 0 ? NACT + FN : 0;  // fragment reads per sub-step
    constexpr int H0 = LPS / 2;                     // loads issued in sub-step 0
    constexpr int H1 = LPS - H0;                    // ... and in sub-step 1
    // fragments of the two sub-steps (double buffer: one is multiplied while
    // the other is read).  Read order: the FN B fragments, then the NACT A
    // fragments, so that row i of MFMAs can start once A fragment i is in.
    // A8: the A fragments are 8 bytes of e4m3 values; sc[s][i] is the scale
    // of row block i in A slot s, read with the first fragments of its
    // K-step (before them, so that waiting for a fragment covers it).
    std::conditional_t<A8, u32x2, bf16x8> fa[2][NF];
    bf16x8 fb[2][FN];
    float sc[2][NF];
    constexpr int NSC = A8 ? NACT : 0;  // scale reads with a K-step's first fragments
    const bool unit_scale = !A8 || g.a8_ns == 0;
    auto read_frag = [&](auto buf_c, auto st_c, auto sk_c, auto r_c) __attribute__((always_inline)) {
      constexpr int BUF = decltype(buf_c)::value, ST = decltype(st_c)::value;
      constexpr int SK = decltype(sk_c)::value, r = decltype(r_c)::value;
      if constexpr (r < FN)
        fb[BUF][r] = *((lds_bf16x8_t *)(uintptr_t)fb_addr[ST][SK] + r * 32 * ROWB / 16);
      else if constexpr (A8)
        fa[BUF][r - FN] =
            *(lds_u32x2_t *)(uintptr_t)(fa_addr[ST][SK] + (r - FN) * WM * 32 * ROWB_A);
      else
        fa[BUF][r - FN] =
            *((lds_bf16x8_t *)(uintptr_t)fa_addr[ST][SK] + (r - FN) * WM * 32 * ROWB / 16);
    };
    auto read_scale = [&](auto st_c, auto i_c) __attribute__((always_inline)) {
      constexpr int ST = decltype(st_c)::value, i = decltype(i_c)::value;
      if constexpr (A8) {
        const float v = *(lds_f32_t *)(uintptr_t)(fsc_addr[ST] + i * WM * 32 * 4);
        sc[ST][i] = unit_scale ? 1.0f : v;
      }
    };
    // The MFMAs of a sub-step (K-steps of 64): NACT rows of FN MFMAs from
    // fragment buffer BUFM (A of slot MST), one item after each MFMA; with
    // SYNC the items start after row 0 and the barrier.  Before row i a
    // progressive lgkmcnt wait lets the row start as soon as its A fragment
    // (and the B fragments read before it) are in.  8-bit A: the fragment of
    // row i + 1 is converted during the MFMAs of row i, a quarter after each
    // (its wait moves up one row), so that only row 0's conversion stands
    // between the LDS reads and the matrix cores.
    auto mfma_rows = [&](auto bufm_c, auto mst_c, auto sync_c, auto nrds_c, auto nit_c,
                         auto &&item, auto &&sync) __attribute__((always_inline)) {
      constexpr int BUFM = decltype(bufm_c)::value, MST = decltype(mst_c)::value;
      constexpr bool SYNC = decltype(sync_c)::value;
      constexpr int NRDS = decltype(nrds_c)::value, NIT = decltype(nit_c)::value;
      [[maybe_unused]] bf16x8 cva[NF];
      static_for<NACT>([&](auto i_c) __attribute__((always_inline)) {
        constexpr int i = decltype(i_c)::value;
        constexpr int BEFORE = SYNC ? (i == 0 ? 0 : (i - 1) * FN) : i * FN;
        constexpr int ISSUED = BEFORE < NRDS ? BEFORE : NRDS;
        constexpr int NEED = (A8 && i + 1 < NACT) ? i + 1 : i;  // last A fragment needed
        wait_lgkmcnt<(NACT - 1 - NEED) + ISSUED>();
        bf16x8 av;
        if constexpr (A8) {
          if constexpr (i == 0) cva[0] = e4m3x8_to_bf16(fa[BUFM][0], sc[MST][0]);
          av = cva[i];
        } else {
          av = fa[BUFM][i];
        }
        static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
          constexpr int j = decltype(j_c)::value;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[BUFM][j], av, acc[i][j], 0, 0, 0);
          if constexpr (!(SYNC && i == 0)) {
            constexpr int m = BEFORE + j;
            if constexpr (m < NIT) item(std::integral_constant<int, m>{});
          }
          if constexpr (A8 && i + 1 < NACT)
            e4m3x2_to_bf16<j>(cva[i + 1], fa[BUFM][i + 1], sc[MST][i + 1]);
        });
        if constexpr (SYNC && i == 0) sync();
      });
      if constexpr (SYNC && NACT == 0) sync();
      // items the MFMAs did not cover (few active rows)
      constexpr int COVERED = NACT == 0 ? 0 : (SYNC ? (NACT - 1) * FN : NACT * FN);
      static_for<(NIT > COVERED) ? NIT - COVERED : 0>([&](auto t_c) __attribute__((always_inline)) {
        item(std::integral_constant<int, COVERED + decltype(t_c)::value>{});
      });
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // prologue: K-steps 0 .. STAGES-2 in flight; stage 0 complete
    // everywhere; the fragments of (K-step 0, sub-step 0) read into buffer 0
    if constexpr (!SPLIT) {
      static_for<STAGES - 1>([&](auto p_c) __attribute__((always_inline)) {
        const uint32_t soff = k_offset(decltype(p_c)::value);
        static_for<LPS>([&](auto q_c) __attribute__((always_inline)) { issue_load(p_c, q_c, soff); });
      });
      wait_vmcnt<(STAGES - 2) * LPS>();
    } else {
      // split rings: A and B of K-step 0, then B of K-step 1 (may stay in
      // flight)
      const uint32_t s0 = k_offset(0), s1 = k_offset(1);
      static_for<LA>([&](auto q_c) __attribute__((always_inline)) { issue_a(I0{}, q_c, s0); });
      static_for<LB>([&](auto q_c) __attribute__((always_inline)) { issue_b(0, q_c, s0); });
      static_for<LB>([&](auto q_c) __attribute__((always_inline)) { issue_b(1, q_c, s1); });
      wait_vmcnt<LB>();
    }
    stage_barrier();
    static_for<NSC>([&](auto i_c) __attribute__((always_inline)) { read_scale(I0{}, i_c); });
    static_for<NRD>([&](auto r_c) __attribute__((always_inline)) { read_frag(I0{}, I0{}, I0{}, r_c); });

    if constexpr (KSUB == 2) {
    // K-step kt, whose stage is ST = kt % STAGES.  Each wavefront issues, in
    // order (one item after each MFMA):
    //  sub-step 0: MFMAs of (kt, 0) from buffer 0; items: the reads of
    //    (kt, 1) into buffer 1, then H0 loads of K-step kt+STAGES-1 (into
    //    the slot K-step kt-1 used, free since the previous barrier);
    //  sub-step 1: MFMAs of (kt, 1) from buffer 1; after the first row:
    //    wait for its own reads of stage kt and its own share of stage kt+1,
    //    barrier (stage kt+1 complete everywhere, stage kt's slot free from
    //    the next K-step on); items: the reads of (kt+1, 0) into buffer 0,
    //    then the other H1 loads.
    // Before MFMA row i, a progressive lgkmcnt wait lets the row start as
    // soon as its A fragment (and the B fragments read before it) are in.
    auto step = [&](auto st_c, int kt) __attribute__((always_inline)) {
      constexpr int ST = decltype(st_c)::value;
      constexpr int NST = (ST + 1) % STAGES;            // stage of K-step kt+1
      constexpr int LST = (ST + STAGES - 1) % STAGES;   // stage of K-step kt+STAGES-1
      const uint32_t soff = k_offset(kt + STAGES - 1);
      // ---- sub-step 0
      static_for<NACT>([&](auto i_c) __attribute__((always_inline)) {
        constexpr int i = decltype(i_c)::value;
        // new reads issued before row i: one per earlier MFMA, at most NRD
        constexpr int ISSUED = (i * FN < NRD) ? i * FN : NRD;
        wait_lgkmcnt<(NACT - 1 - i) + ISSUED>();
        static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
          constexpr int j = decltype(j_c)::value, m = i * FN + j;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[0][j], fa[0][i], acc[i][j], 0, 0, 0);
          if constexpr (m < NRD) read_frag(I1{}, st_c, I1{}, std::integral_constant<int, m>{});
          else if constexpr (m - NRD < H0)
            issue_load(std::integral_constant<int, LST>{}, std::integral_constant<int, m - NRD>{}, soff);
        });
      });
      // items the MFMAs did not cover (few active rows)
      constexpr int NMF = NACT * FN;
      static_for<(NRD + H0 > NMF) ? NRD + H0 - NMF : 0>([&](auto t_c) __attribute__((always_inline)) {
        constexpr int m = NMF + decltype(t_c)::value;
        if constexpr (m < NRD) read_frag(I1{}, st_c, I1{}, std::integral_constant<int, m>{});
        else issue_load(std::integral_constant<int, LST>{}, std::integral_constant<int, m - NRD>{}, soff);
      });
      // ---- sub-step 1
      // The barrier of K-step kt: every wavefront's share of stage kt+1 has
      // landed, and every wavefront's reads of stage kt are complete (the
      // DMA that next refills stage kt's slot is issued after this barrier).
      auto sync = [&]() __attribute__((always_inline)) {
        wait_lgkmcnt<0>();                      // own reads of stage kt done
        wait_vmcnt<(STAGES - 3) * LPS + H0>();  // own share of stage kt+1
        stage_barrier();                        // ... for every wavefront
      };
      if constexpr (NACT == 0) sync();
      static_for<NACT>([&](auto i_c) __attribute__((always_inline)) {
        constexpr int i = decltype(i_c)::value;
        // items start after row 0 (and the barrier)
        constexpr int ISSUED = (i == 0) ? 0 : (((i - 1) * FN < NRD) ? (i - 1) * FN : NRD);
        wait_lgkmcnt<(NACT - 1 - i) + ISSUED>();
        static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
          constexpr int j = decltype(j_c)::value, m = (i - 1) * FN + j;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[1][j], fa[1][i], acc[i][j], 0, 0, 0);
          if constexpr (i >= 1) {
            if constexpr (m < NRD) read_frag(I0{}, std::integral_constant<int, NST>{}, I0{}, std::integral_constant<int, m>{});
            else if constexpr (m - NRD < H1)
              issue_load(std::integral_constant<int, LST>{}, std::integral_constant<int, H0 + m - NRD>{}, soff);
          }
        });
        if constexpr (i == 0) sync();
      });
      constexpr int NMF1 = NACT > 0 ? (NACT - 1) * FN : 0;
      static_for<(NRD + H1 > NMF1) ? NRD + H1 - NMF1 : 0>([&](auto t_c) __attribute__((always_inline)) {
        constexpr int m = NMF1 + decltype(t_c)::value;
        if constexpr (m < NRD) read_frag(I0{}, std::integral_constant<int, NST>{}, I0{}, std::integral_constant<int, m>{});
        else issue_load(std::integral_constant<int, LST>{}, std::integral_constant<int, H0 + m - NRD>{}, soff);
      });
    };
    // K-steps in rounds of STAGES, so that each step's stage is a constant
    int kt = 0;
    for (; kt + STAGES <= nk; kt += STAGES)
      static_for<STAGES>([&](auto p) __attribute__((always_inline)) {
        step(p, kt + decltype(p)::value);
      });
    static_for<STAGES - 1>([&](auto p) __attribute__((always_inline)) {
      if (kt + decltype(p)::value < nk) step(p, kt + decltype(p)::value);
    });
    } else if constexpr (!SPLIT) {
    // K-steps of 64: sub-steps 0..3 of K-step kt multiply fragment buffers
    // 0, 1, 0, 1 and, one item after each MFMA, read the next sub-step's
    // fragments into the other buffer and issue loads: [L3, L3 + L0) of
    // stage kt+1 in sub-step 0, the rest in sub-step 1; in sub-step 3, after
    // its first row and the barrier, the fragments of (kt+1, 0) and loads
    // [0, L3) of stage kt+2 into the slot stage kt used.
    constexpr int L3 = LPS / 4, L0 = LPS / 2, L1 = LPS - L3 - L0;
    auto substep = [&](auto bufm_c, auto rbuf_c, auto rst_c, auto rsk_c, auto lst_c, auto q0_c,
                       auto nq_c, uint32_t soff, auto sync_c, auto mst_c)
                       __attribute__((always_inline)) {
      constexpr int RBUF = decltype(rbuf_c)::value;  // reads: into buffer RBUF,
      constexpr int RST = decltype(rst_c)::value;    //   of stage slot RST,
      constexpr int RSK = decltype(rsk_c)::value;    //   sub-step RSK
      constexpr int LST = decltype(lst_c)::value;    // loads: into slot LST,
      constexpr int Q0 = decltype(q0_c)::value;      //   loads Q0 ..
      constexpr int NQ = decltype(nq_c)::value;      //   .. Q0 + NQ - 1
      constexpr bool SYNC = decltype(sync_c)::value;
      // the sub-step with the barrier reads the next K-step's first
      // fragments, and (A8) before them its scales
      constexpr int NSCS = SYNC ? NSC : 0;
      constexpr int NRDS = NRD + NSCS;
      constexpr int NIT = NRDS + NQ;
      auto item = [&](auto m_c) __attribute__((always_inline)) {
        constexpr int m = decltype(m_c)::value;
        if constexpr (m < NSCS)
          read_scale(std::integral_constant<int, RST>{}, std::integral_constant<int, m>{});
        else if constexpr (m < NRDS)
          read_frag(std::integral_constant<int, RBUF>{}, std::integral_constant<int, RST>{},
                    std::integral_constant<int, RSK>{}, std::integral_constant<int, m - NSCS>{});
        else
          issue_load(std::integral_constant<int, LST>{},
                     std::integral_constant<int, Q0 + m - NRDS>{}, soff);
      };
      // the barrier of the K-step: this wavefront's reads of the current
      // stage and its loads of the next one are done, then every
      // wavefront's
      auto sync = [&]() __attribute__((always_inline)) {
        wait_lgkmcnt<0>();
        wait_vmcnt<0>();
        stage_barrier();
      };
      mfma_rows(bufm_c, mst_c, sync_c, std::integral_constant<int, NRDS>{},
                std::integral_constant<int, NIT>{}, item, sync);
    };
    using IT = std::true_type;
    using IF = std::false_type;
    auto step = [&](auto st_c, int kt) __attribute__((always_inline)) {
      constexpr int ST = decltype(st_c)::value;  // stage of K-step kt
      constexpr int NS = 1 - ST;                 // stage of K-steps kt-1 and kt+1
      using S = std::integral_constant<int, ST>;
      using N = std::integral_constant<int, NS>;
      const uint32_t s1 = k_offset(kt + 1), s2 = k_offset(kt + 2);
      substep(I0{}, I1{}, S{}, I1{}, N{}, std::integral_constant<int, L3>{},
              std::integral_constant<int, L0>{}, s1, IF{}, S{});
      substep(I1{}, I0{}, S{}, std::integral_constant<int, 2>{}, N{},
              std::integral_constant<int, L3 + L0>{}, std::integral_constant<int, L1>{}, s1, IF{},
              S{});
      substep(I0{}, I1{}, S{}, std::integral_constant<int, 3>{}, N{}, I0{}, I0{}, s1, IF{}, S{});
      substep(I1{}, I0{}, N{}, I0{}, S{}, I0{}, std::integral_constant<int, L3>{}, s2, IT{}, S{});
    };
    // the first loads of stage 1 (those sub-step 3 of the step before issues)
    static_for<L3>([&](auto q_c) __attribute__((always_inline)) {
      issue_load(I1{}, q_c, k_offset(1));
    });
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
      step(I0{}, kt);
      step(I1{}, kt + 1);
    }
    if (kt < nk) step(I0{}, kt);
    } else {
    // Split rings (K-steps of 64): K-step kt reads A slot kt % 2 and B slot
    // kt % 3.  After the barrier of K-step j the wavefront issues, in this
    // order, its A loads of K-step j+2 and its B loads of K-step j+3 (the
    // batch of j), spread as in the two-stage schedule: [0, L3) in sub-step 3
    // of j, the rest in sub-steps 0 and 1 of j+1.  So at the barrier of
    // K-step kt the last LB loads issued are the B loads of kt+2: after
    // vmcnt(LB) the A and B loads of kt+1 have landed, and B streams two
    // K-steps ahead of its use, A one.  The barrier frees A slot kt % 2 and B
    // slot kt % 3, the targets of the next batch.
    constexpr int L3 = LPS / 4, L0 = LPS / 2, L1 = LPS - L3 - L0;
    // item q of a batch: A load q into A slot AS at K offset sa, or B load
    // q - LA into B slot bsl at K offset sb
    auto batch_item = [&](auto as_c, auto q_c, int bsl, uint32_t sa, uint32_t sb)
                          __attribute__((always_inline)) {
      constexpr int q = decltype(q_c)::value;
      if constexpr (q < LA)
        issue_a(as_c, q_c, sa);
      else
        issue_b(bsl, std::integral_constant<int, q - LA>{}, sb);
    };
    // fragment read r of a sub-step: B from the given address (the B slot is
    // a runtime value), A from slot AST
    auto read_frag_s = [&](auto buf_c, auto ast_c, auto sk_c, auto r_c, uint32_t fbsk)
                           __attribute__((always_inline)) {
      constexpr int BUF = decltype(buf_c)::value, AST = decltype(ast_c)::value;
      constexpr int SK = decltype(sk_c)::value, r = decltype(r_c)::value;
      if constexpr (r < FN)
        fb[BUF][r] = *((lds_bf16x8_t *)(uintptr_t)fbsk + r * 32 * ROWB / 16);
      else if constexpr (A8)
        fa[BUF][r - FN] =
            *(lds_u32x2_t *)(uintptr_t)(fa_addr[AST][SK] + (r - FN) * WM * 32 * ROWB_A);
      else
        fa[BUF][r - FN] =
            *((lds_bf16x8_t *)(uintptr_t)fa_addr[AST][SK] + (r - FN) * WM * 32 * ROWB / 16);
    };
    auto substep = [&](auto bufm_c, auto rbuf_c, auto rast_c, auto rsk_c, uint32_t rfb,
                       auto las_c, auto q0_c, auto nq_c, int lbs, uint32_t sa, uint32_t sb,
                       auto sync_c, auto mst_c) __attribute__((always_inline)) {
      constexpr int RBUF = decltype(rbuf_c)::value;  // reads: into buffer RBUF,
      constexpr int Q0 = decltype(q0_c)::value;      // batch items Q0 ..
      constexpr int NQ = decltype(nq_c)::value;      //   .. Q0 + NQ - 1
      constexpr bool SYNC = decltype(sync_c)::value;
      // the sub-step with the barrier reads the next K-step's first
      // fragments, and (A8) before them its scales
      constexpr int NSCS = SYNC ? NSC : 0;
      constexpr int NRDS = NRD + NSCS;
      constexpr int NIT = NRDS + NQ;
      auto item = [&](auto m_c) __attribute__((always_inline)) {
        constexpr int m = decltype(m_c)::value;
        if constexpr (m < NSCS)
          read_scale(rast_c, std::integral_constant<int, m>{});
        else if constexpr (m < NRDS)
          read_frag_s(std::integral_constant<int, RBUF>{}, rast_c, rsk_c,
                      std::integral_constant<int, m - NSCS>{}, rfb);
        else
          batch_item(las_c, std::integral_constant<int, Q0 + m - NRDS>{}, lbs, sa, sb);
      };
      // the barrier of the K-step: this wavefront's reads of the current
      // slots are done and its loads up to those of kt+1 have landed, then
      // every wavefront's
      auto sync = [&]() __attribute__((always_inline)) {
        wait_lgkmcnt<0>();
        wait_vmcnt<LB>();
        stage_barrier();
      };
      mfma_rows(bufm_c, mst_c, sync_c, std::integral_constant<int, NRDS>{},
                std::integral_constant<int, NIT>{}, item, sync);
    };
    using IT = std::true_type;
    using IF = std::false_type;
    auto step = [&](auto st_c, int kt, int bs) __attribute__((always_inline)) {
      constexpr int ST = decltype(st_c)::value;  // A slot of K-step kt
      using S = std::integral_constant<int, ST>;
      using N = std::integral_constant<int, 1 - ST>;
      const int bs1 = bs == 2 ? 0 : bs + 1;     // B slot of kt+1
      const int bs2 = bs1 == 2 ? 0 : bs1 + 1;   // B slot of kt+2 (and of kt-1)
      const uint32_t s1 = k_offset(kt + 1), s2 = k_offset(kt + 2), s3 = k_offset(kt + 3);
      const uint32_t bo = (uint32_t)bs * B_BYTES, bo1 = (uint32_t)bs1 * B_BYTES;
      // the batch of kt-1 (A of kt+1, B of kt+2) in sub-steps 0 and 1
      substep(I0{}, I1{}, S{}, I1{}, fb_addr[0][1] + bo, N{}, std::integral_constant<int, L3>{},
              std::integral_constant<int, L0>{}, bs2, s1, s2, IF{}, S{});
      substep(I1{}, I0{}, S{}, std::integral_constant<int, 2>{}, fb_addr[0][2] + bo, N{},
              std::integral_constant<int, L3 + L0>{}, std::integral_constant<int, L1>{}, bs2, s1, s2,
              IF{}, S{});
      substep(I0{}, I1{}, S{}, std::integral_constant<int, 3>{}, fb_addr[0][3] + bo, N{}, I0{},
              I0{}, bs2, s1, s2, IF{}, S{});
      // barrier; fragments of (kt+1, 0); the first of the batch of kt (A of
      // kt+2 into A slot ST, B of kt+3 into B slot bs)
      substep(I1{}, I0{}, N{}, I0{}, fb_addr[0][0] + bo1, S{}, I0{},
              std::integral_constant<int, L3>{}, bs, s2, s3, IT{}, S{});
    };
    // the first items of the batch of K-step -1: A of 1 (slot 1), B of 2
    // (slot 2)
    {
      const uint32_t s1 = k_offset(1), s2 = k_offset(2);
      static_for<L3>([&](auto q_c) __attribute__((always_inline)) {
        batch_item(I1{}, q_c, 2, s1, s2);
      });
    }
    int kt = 0, bs = 0;
    for (; kt + 2 <= nk; kt += 2) {
      step(I0{}, kt, bs);
      bs = bs == 2 ? 0 : bs + 1;
      step(I1{}, kt + 1, bs);
      bs = bs == 2 ? 0 : bs + 1;
    }
    if (kt < nk) step(I0{}, kt, bs);
    }
    wait_lgkmcnt<0>();
    wait_vmcnt<0>();  // the tail's re-loads land before the ring is reused
    // every wavefront is done with the LDS before the next tile refills it
    __syncthreads();
    after_kloop();

    // The MFMAs take the weights as their first operand, so each 32x32
    // block holds the tile transposed: lane holds output row (lane % 32) of
    // the block and, for accumulator element v, output column
    // 8 * (v / 4) + 4 * (lane / 32) + v % 4 -- runs of four consecutive
    // columns of one row.
    if (part != nullptr) {
      // partial sums of a K-range: straight from the accumulators, four
      // consecutive floats of a row per store
      static_for<NACT>([&](auto i_c) __attribute__((always_inline)) {
        constexpr int i = decltype(i_c)::value;
        const int row = (wm + i * WM) * 32 + (lane & 31);
        static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
          constexpr int j = decltype(j_c)::value;
          asm volatile("" : "+a"(acc[i][j]));
          float *prow = part + row * BN + wn * TN + j * 32 + (lane / 32) * 4;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(float4 *)(prow + q * 8) = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                    acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        });
      });
      return;
    }

    // Epilogue, through the (now idle) ring: the wavefronts write the tile,
    // rounded to bf16, row-major into LDS, four columns (8 bytes) per write;
    // then all threads copy the rows that exist to the staging window in
    // 16-byte pieces.  Rows carry 16 bytes of padding (they stay 16-byte
    // aligned for the copy), so the 32 rows one half-wavefront writes fall
    // on at most two rows of banks.  The empty asm
    // statements pin each block's accumulator reads after the previous
    // block's LDS writes, which keeps the compiler from hoisting every
    // accumulator into VGPRs at once.
    constexpr int OUT_COLS = SWIGLU ? BN / 2 : BN;
    constexpr int OROWB = OUT_COLS * 2 + 16;
    static_assert(BM * OROWB <= kGemmLdsBytes, "the output tile must fit the LDS");
    typedef __attribute__((address_space(3))) u32x2 lds_w_u32x2_t;
    typedef __attribute__((address_space(3))) const u32x4 lds_u32x4_t;
    lds_char_t *otile = (lds_char_t *)smem;
    auto pack2 = [](float lo, float hi) __attribute__((always_inline)) {
      return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
    };
    static_for<NACT>([&](auto i_c) __attribute__((always_inline)) {
      constexpr int i = decltype(i_c)::value;
      lds_char_t *orow = otile + ((wm + i * WM) * 32 + (lane & 31)) * OROWB + (lane / 32) * 8;
      if constexpr (SWIGLU) {
        static_for<FN / 2>([&](auto p_c) __attribute__((always_inline)) {
          constexpr int p = decltype(p_c)::value;
          asm volatile("" : "+a"(acc[i][2 * p]), "+a"(acc[i][2 * p + 1]));
          const int col = wn * (TN / 2) + p * 32;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float h[4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
              h[c] = silu(acc[i][2 * p][4 * q + c]) * acc[i][2 * p + 1][4 * q + c];
            u32x2 w2;
            w2.x = pack2(h[0], h[1]);
            w2.y = pack2(h[2], h[3]);
            *(lds_w_u32x2_t *)(orow + (col + q * 8) * 2) = w2;
          }
        });
      } else {
        static_for<FN>([&](auto j_c) __attribute__((always_inline)) {
          constexpr int j = decltype(j_c)::value;
          asm volatile("" : "+a"(acc[i][j]));
          const int col = wn * TN + j * 32;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            u32x2 w2;
            w2.x = pack2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
            w2.y = pack2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            *(lds_w_u32x2_t *)(orow + (col + q * 8) * 2) = w2;
          }
        });
      }
    });
    __syncthreads();
    constexpr int CHUNKS = OUT_COLS * 2 / 16;  // 16-byte pieces per row
    u32x4 *dst = (u32x4 *)(C + (int64_t)n_tile * OUT_COLS);
    const int ldc16 = g.ldc / 8;
    for (int idx = tid; idx < rows_valid * CHUNKS; idx += NW * kWave) {
      const int row = idx / CHUNKS, ch = idx % CHUNKS;
      dst[(int64_t)row * ldc16 + ch] = *((lds_u32x4_t *)(otile + row * OROWB) + ch);
    }
    __syncthreads();  // the ring is read out before the next tile refills it
  };
  // one specialisation per active-block count (wavefront-uniform branch)
  static_for<FM + 1>([&](auto c) __attribute__((always_inline)) {
    if (nact == decltype(c)::value) k_loop(c);
  });
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

// Tile r (0 <= r < units) of an expert with `rows` rows, in list order:
// n-tile major, m-tile minor; with a half remainder, the column-tile pair
// (2j, 2j+1) lists the remainder tile j that spans both (kind 2: 128 rows x
// 2 BN) and then its full m-tiles (kind 1: BM x BN).  The remainder tile
// streams both weight panels with one K-step in flight and is the slowest
// tile of the group: started first, it leads, and the full tiles started
// after it catch up and read its panels from L2 (listed last, it fell
// behind and read them again).
struct TileRef {
  int kind, n_tile, m_tile, row0, rows_valid;
};

__device__ __forceinline__ TileRef decode_tile(const ExpertTiles &et, int r, int rows) {
  TileRef t;
  if (et.half && r % (2 * et.q + 1) == 0) {
    t.kind = 2;
    t.n_tile = r / (2 * et.q + 1);
    t.m_tile = et.q;
    t.row0 = et.q * kBM;
    t.rows_valid = et.rem;
  } else {
    if (et.half) {
      const int per = 2 * et.q + 1;
      const int j = r / per;
      const int rr = r - j * per - 1;
      t.n_tile = 2 * j + rr / et.q;
      t.m_tile = rr % et.q;
    } else {
      const int mt_e = et.q + (et.rem > 0);
      t.n_tile = r / mt_e;
      t.m_tile = r - t.n_tile * mt_e;
    }
    t.kind = 1;
    t.row0 = t.m_tile * kBM;
    t.rows_valid = min(kBM, rows - t.row0);
  }
  return t;
}

// Descriptors of the two expert GEMMs over the windows of `a` (the tile
// queues and the split-tile state are the caller's to set).
inline GemmDesc gemm_desc_gate_up(const MoeArgs &a, const uint16_t *w13) {
  GemmDesc g{};
  g.a_win = a.off_disp_x;
  g.lda = a.H;
  g.w = w13;
  g.w_estride = (int64_t)2 * a.I * a.H;
  g.w_bytes = g.w_estride * 2;
  g.ldb = a.H;
  g.c_win = a.off_hbuf;
  g.ldc = a.I;
  g.kdim = a.H;
  g.ntiles = a.I / (kBN / 2);
  g.up_off = a.I;
  return g;
}

inline GemmDesc gemm_desc_down(const MoeArgs &a, const uint16_t *w2) {
  GemmDesc g{};
  g.a_win = a.off_hbuf;
  g.lda = a.I;
  g.w = w2;
  g.w_estride = (int64_t)a.H * a.I;
  g.w_bytes = g.w_estride * 2;
  g.ldb = a.I;
  g.c_win = a.off_out;
  g.ldc = a.H;
  g.kdim = a.I;
  g.ntiles = a.H / kBN;
  g.up_off = 0;
  return g;
}

// Tiles of one expert's GEMM that cover its m-tile m (rows [256 m, 256 m +
// 256)): every column tile, or every pair of them for a half remainder.
__device__ __forceinline__ int tiles_per_mtile(const ExpertTiles &et, int m, int ntl) {
  return (et.half && m == et.q) ? ntl / 2 : ntl;
}

}  // namespace
}  // namespace cco
