// cco_internal.h -- types shared by the host side and the kernels of the
// cco_moe library.  Not installed; the public interface is include/cco_moe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cco {

// 16-byte vector of 32-bit lanes as a first-class clang vector (arrays of
// these stay in registers; HIP's struct-based uint4 does not reliably).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Wavefront width of CDNA (gfx950).
constexpr int kWave = 64;
// XCDs on one MI355X; workgroups are handed to XCDs round-robin by id, so
// id % kNumXcd names the XCD (and its L2) a workgroup runs on.
constexpr int kNumXcd = 8;
// Limits checked on the host before any launch.
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopk = 32;
// Plan kernels: one workgroup per chunk of flat (token, k) pairs.
constexpr int kPlanThreads = 256;
constexpr int kPlanPerThread = 8;
constexpr int kPlanChunk = kPlanThreads * kPlanPerThread;

// Everything a kernel needs to address the windows of one MoE layer,
// passed by value so it lands in kernel-argument space (the device
// communicator idiom of the MORI CCO Guide, "Concepts").
struct MoeArgs {
  char *base;          // heap base
  uint64_t stride;     // bytes per slot
  uint64_t off_disp_x; // window offsets inside every slot
  uint64_t off_meta;
  uint64_t off_hbuf;
  uint64_t off_out;
  int64_t cap;         // rows per slot
  int32_t K, H, E, S, eps, I;
  int32_t *pos;        // [max_tokens * K]: receive row of each pair (-1: dropped)
  int32_t *eid;        // [max_tokens * K]: expert id of each pair (-1: invalid)
  int32_t *counts;     // [E]
  int32_t *expert_off; // [E]
  int32_t *slot_total; // [S]
  int32_t *status;     // [1]
  int32_t *hist;       // [plan blocks][E + 1] scratch
  int32_t *ticket;     // [1] scratch, zero between plans
  int32_t *gemm_queue; // [4][kNumXcd + 1] tile queues: the two expert GEMMs, then their split-tile tails; zero between launches
  float *split_ws;     // [gemm_workgroups][kSplitTileFloats] partial sums of split GEMM tiles
  int32_t *split_desc; // [gemm_workgroups / 2][kSplitDescInts] split tiles, zero between launches
  uint32_t eps_magic;  // ceil(2^20 / eps): slot_of() without a division
};

// slot(e) = e / eps as (e * ceil(2^20 / eps)) >> 20, exact whenever
// e * eps < 2^20, which e < E <= kMaxExperts = 1024 guarantees.
__host__ __device__ inline int slot_of(const MoeArgs &a, int e) {
  return (int)(((uint32_t)e * a.eps_magic) >> 20);
}
inline uint32_t eps_magic_of(int eps) { return ((1u << 20) + (uint32_t)eps - 1u) / (uint32_t)eps; }

// The expert GEMMs run one workgroup per CU, in whole XCDs.
inline int gemm_workgroups(int num_cus) { return ((num_cus + kNumXcd - 1) / kNumXcd) * kNumXcd; }
// fp32 accumulators of one GEMM tile (256 x 256, or 128 x 512), and the
// words describing one tile whose K-steps were split over workgroups.
constexpr int kSplitTileFloats = 256 * 256;
constexpr int kSplitDescInts = 8;

// Address of byte `off` of window `win_off` in slot `s`:
// base + s * stride + win_off + off.
__host__ __device__ inline char *slot_addr(const MoeArgs &a, int s, uint64_t win_off,
                                          uint64_t off) {
  return a.base + (uint64_t)s * a.stride + win_off + off;
}

// Split of a token row (nvec 16-byte vectors) over `parts` wavefronts of
// nvl vectors per lane, for the row kernels (dispatch, combine).  nvl is one
// of the fixed lengths the kernels are built for (1, 2, 4, 7, 8, 14, 16), or
// 0 for the general loop over the whole row (parts = 1).  Rows go one
// wavefront each while T alone gives kRowWaves wavefronts; smaller batches
// split each row into the fewest parts that reach that many, so that every
// CU takes part.
constexpr int kRowWaves = 4096;
struct RowSplit {
  int nvl, parts;
};
inline RowSplit row_split(int nvec, int64_t T) {
  if (nvec <= 0 || nvec % kWave != 0) return {0, 1};
  const int per_lane = nvec / kWave;
  static const int kLens[] = {16, 14, 8, 7, 4, 2, 1};
  RowSplit best{0, 1};
  for (int nvl : kLens) {
    if (per_lane % nvl != 0) continue;
    best = {nvl, per_lane / nvl};
    if (T * best.parts >= kRowWaves) break;
  }
  return best;
}

// Launchers, one per kernel file.  Each returns the hipError_t of its launch.
hipError_t launch_plan_count(const MoeArgs &a, const int32_t *idx, int32_t n_pairs,
                             int32_t nblk, hipStream_t st);
hipError_t launch_plan_rank(const MoeArgs &a, const int32_t *idx, int32_t n_pairs,
                            int32_t nblk, hipStream_t st);
// Both plan steps in one workgroup, for n_pairs <= kPlanChunk.
hipError_t launch_plan_single(const MoeArgs &a, const int32_t *idx, int32_t n_pairs,
                              hipStream_t st);
hipError_t launch_dispatch(const MoeArgs &a, const uint16_t *x, const float *w,
                           const int32_t *idx, int32_t T, hipStream_t st);
// Tokens of H bytes (8-bit, H % 16 == 0) with ns fp32 scales per token.
hipError_t launch_dispatch_fp8(const MoeArgs &a, const uint8_t *x8, const float *scales,
                               int32_t ns, const float *w, const int32_t *idx, int32_t T,
                               hipStream_t st);
hipError_t launch_combine(const MoeArgs &a, uint64_t src_win, const float *w,
                          const int32_t *idx, uint16_t *out, int32_t T, hipStream_t st);
hipError_t launch_copy_in(const MoeArgs &a, int32_t slot, const uint16_t *src,
                          uint64_t dst_win, hipStream_t st);

// State of the single-launch path (fused.hip), part of the routing state:
// counters (zero between launches) and per-launch tables.
constexpr int kFusedCounterWords = 64;
struct FusedBuffers {
  int32_t *q;        // [kFusedCounterWords]
  int32_t *pre_g;    // [E + 1]
  int32_t *pre_w;    // [E + 1]
  int32_t *pre_mt;   // [E + 1]
  int32_t *arrived;  // [E]
  int32_t *gu_done;  // [fused_mtiles]
  int32_t *dn_done;  // [fused_mtiles]
};
// 256-row m-tiles of all experts together: sum over e of ceil(rows_e / 256)
// <= T * K / 256 + E.
inline int64_t fused_mtiles(int64_t max_tokens, int K, int E) {
  return E + (max_tokens * K + 255) / 256;
}
// The whole path (plan, dispatch, both expert GEMMs, combine) in one
// persistent launch of one workgroup per CU.
hipError_t launch_fused(const MoeArgs &a, const FusedBuffers &b, const int32_t *idx,
                        const uint16_t *x, const float *w, const uint16_t *w13,
                        const uint16_t *w2, uint16_t *out, int32_t T, int num_cus,
                        hipStream_t st);

// Expert GEMMs of the T planned tokens.  `num_cus` sizes the persistent
// grids.  a8_ns < 0: the receive rows are bf16; otherwise they are the
// 8-bit rows of an 8-bit dispatch with a8_ns scales each (H / a8_ns a
// power-of-two multiple of 64 when a8_ns > 0), read as
// bf16(binary32(e4m3 * scale)) by gate/up.
hipError_t launch_expert_gate_up(const MoeArgs &a, const uint16_t *w13, int32_t T, int num_cus,
                                 int32_t a8_ns, hipStream_t st);
hipError_t launch_expert_down(const MoeArgs &a, const uint16_t *w2, int32_t T, int num_cus,
                              hipStream_t st);

}  // namespace cco
