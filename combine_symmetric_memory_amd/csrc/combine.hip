// combine.hip -- gather every token's expert rows back from the slots and
// sum them with the routing weights.
//
// "MORI CCO: Next-Generation Collective Communication Object for GPUs",
// section "Zero-copy MoE dispatch -> expert -> combine", step 3: each rank
// reads its tokens back from the combine staging buffers of the ranks that
// own the experts and applies the weights.  Row j of token t sits at
//   base + slot(idx[t][j]) * stride + src_window + pos[t][j] * (2 * H).
//
//   out[t][h] = bf16( fma(w[t][K-1], y_{K-1}[h], ... fma(w[t][0], y_0[h], 0)) )
// in fp32, in j order, rounded once to nearest even.  One wavefront per
// token (per part of its row when the batch is small, see row_split); each
// lane owns 8 output elements per 16-byte vector and issues the K row loads
// before it accumulates.  Every output element has one owner:
// no atomics, the result does not depend on scheduling.
//
// copy_in_kernel serves the same section's note: an expert output that is
// not the staging view is copied into the view first (its row count read on
// the device, so the host never waits for it).
#include "combine_impl.h"

namespace cco {
namespace {

constexpr int kCombineWaves = 4;

// One wavefront per token part: wavefront g sums part g % parts of token
// g / parts.
template <int KT, int NVL>
__global__ __launch_bounds__(kCombineWaves *kWave) void combine_kernel(
    MoeArgs a, uint64_t src_win, const float *__restrict__ w, const int32_t *__restrict__ idx,
    u32x4 *__restrict__ out, int32_t T, int32_t parts) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int gw = blockIdx.x * kCombineWaves + wave;
  const int t = gw / parts, part = gw - t * parts;
  const int lane = threadIdx.x & (kWave - 1);
  if (t >= T) return;
  combine_token<KT, NVL>(a, src_win, w, idx, out, t, part, lane);
}

template <int KT, int NVL>
hipError_t launch_nvl(const MoeArgs &a, uint64_t src_win, const float *w, const int32_t *idx,
                      uint16_t *out, int32_t T, int32_t parts, hipStream_t st) {
  const int64_t nwaves = (int64_t)T * parts;
  const int nblk = (int)((nwaves + kCombineWaves - 1) / kCombineWaves);
  hipLaunchKernelGGL((combine_kernel<KT, NVL>), dim3(nblk), dim3(kCombineWaves * kWave), 0, st,
                     a, src_win, w, idx, (u32x4 *)out, T, parts);
  return hipGetLastError();
}

// Fixed-length row parts (row_split) for K <= 8; K above 8 keeps the general
// loop.
template <int KT>
hipError_t launch_k(const MoeArgs &a, uint64_t src_win, const float *w, const int32_t *idx,
                    uint16_t *out, int32_t T, hipStream_t st) {
  const RowSplit rs = (KT > 0 && KT <= 8) ? row_split(a.H / 8, T) : RowSplit{0, 1};
  switch (rs.nvl) {
    case 1: return launch_nvl<KT, 1>(a, src_win, w, idx, out, T, rs.parts, st);
    case 2: return launch_nvl<KT, 2>(a, src_win, w, idx, out, T, rs.parts, st);
    case 4: return launch_nvl<KT, 4>(a, src_win, w, idx, out, T, rs.parts, st);
    case 7: return launch_nvl<KT, 7>(a, src_win, w, idx, out, T, rs.parts, st);
    case 8: return launch_nvl<KT, 8>(a, src_win, w, idx, out, T, rs.parts, st);
    case 14: return launch_nvl<KT, 14>(a, src_win, w, idx, out, T, rs.parts, st);
    case 16: return launch_nvl<KT, 16>(a, src_win, w, idx, out, T, rs.parts, st);
    default: return launch_nvl<KT, 0>(a, src_win, w, idx, out, T, 1, st);
  }
}

// Copy slot_total[slot] rows of `src` into window dst_win of `slot`.
__global__ __launch_bounds__(256) void copy_in_kernel(MoeArgs a, int32_t slot,
                                                      const u32x4 *__restrict__ src,
                                                      uint64_t dst_win) {
  int64_t rows = a.slot_total[slot];
  if (rows > a.cap) rows = a.cap;
  const int64_t nvec = rows * (a.H / 8);
  u32x4 *dst = (u32x4 *)slot_addr(a, slot, dst_win, 0);
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * blockDim.x)
    dst[v] = src[v];
}

}  // namespace

hipError_t launch_combine(const MoeArgs &a, uint64_t src_win, const float *w,
                          const int32_t *idx, uint16_t *out, int32_t T, hipStream_t st) {
  if (T == 0) return hipSuccess;
  switch (a.K) {
    case 1: return launch_k<1>(a, src_win, w, idx, out, T, st);
    case 2: return launch_k<2>(a, src_win, w, idx, out, T, st);
    case 4: return launch_k<4>(a, src_win, w, idx, out, T, st);
    case 6: return launch_k<6>(a, src_win, w, idx, out, T, st);
    case 8: return launch_k<8>(a, src_win, w, idx, out, T, st);
    default: return launch_k<0>(a, src_win, w, idx, out, T, st);
  }
}

hipError_t launch_copy_in(const MoeArgs &a, int32_t slot, const uint16_t *src, uint64_t dst_win,
                          hipStream_t st) {
  hipLaunchKernelGGL(copy_in_kernel, dim3(2048), dim3(256), 0, st, a, slot, (const u32x4 *)src,
                     dst_win);
  return hipGetLastError();
}

}  // namespace cco
