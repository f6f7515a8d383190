// dispatch.hip -- scatter token rows into the receive windows of the slots.
//
// "MORI CCO: Next-Generation Collective Communication Object for GPUs",
// section "Zero-copy MoE dispatch -> expert -> combine", step 1: the
// dispatch kernel writes each token straight into the symmetric receive
// buffer of every rank that owns one of its experts, with no staging copy.
// The receive address is slot arithmetic (section "What is MORI CCO?"):
//   base + slot(e) * stride + DISP_X + pos[t][j] * (2 * H).
//
// One wavefront per token (per part of its row when the batch is small, see
// row_split).  The token's K destinations are wave-uniform (scalar loads of
// idx and pos), the row is read once in 16-byte vectors (up to 16 per lane
// in flight) and each vector is stored K times; 64 lanes x 16 B make every
// store instruction one contiguous 1 KiB run.  Lanes 0..K-1 also write the
// per-row metadata {t*K + j, w[t][j], e}.
//
// The same kernel moves tokens the caller has quantized to 8 bits (the
// op's dispatch takes the tokens' scales beside them and hands back the
// received scales, same section, step 1).  A receive row keeps its 2H bytes:
// the token's H bytes go first and its ns fp32 scales right after them, so
// an 8-bit row moves half the bytes of a bf16 one.
#include "dispatch_impl.h"

namespace cco {
namespace {

constexpr int kDispatchWaves = 4;

// x holds T rows of row_bytes (a multiple of 16); scales (SCALED only) T
// rows of ns floats.  Wavefront g moves part g % parts of token g / parts.
template <int KT, bool SCALED, int NVL>
__global__ __launch_bounds__(kDispatchWaves *kWave) void dispatch_kernel(
    MoeArgs a, const u32x4 *__restrict__ x, int32_t row_bytes, const float *__restrict__ scales,
    int32_t ns, const float *__restrict__ w, const int32_t *__restrict__ idx, int32_t T,
    int32_t parts) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int gw = blockIdx.x * kDispatchWaves + wave;
  const int t = gw / parts, part = gw - t * parts;
  const int lane = threadIdx.x & (kWave - 1);
  if (t >= T) return;
  const int nvec = row_bytes / 16;
  const u32x4 *xr = x + (int64_t)t * nvec;
  const float *sc = SCALED ? scales + (int64_t)t * ns : nullptr;
  dispatch_token<KT, SCALED, NVL>(a, xr, nvec, sc, ns, w, idx, t, part, lane, a.K);
}

template <int KT, bool SCALED, int NVL>
hipError_t launch_nvl(const MoeArgs &a, const void *x, int32_t row_bytes, const float *scales,
                      int32_t ns, const float *w, const int32_t *idx, int32_t T, int32_t parts,
                      hipStream_t st) {
  const int64_t nwaves = (int64_t)T * parts;
  const int nblk = (int)((nwaves + kDispatchWaves - 1) / kDispatchWaves);
  hipLaunchKernelGGL((dispatch_kernel<KT, SCALED, NVL>), dim3(nblk),
                     dim3(kDispatchWaves * kWave), 0, st, a, (const u32x4 *)x, row_bytes, scales,
                     ns, w, idx, T, parts);
  return hipGetLastError();
}

template <int KT, bool SCALED>
hipError_t launch_k(const MoeArgs &a, const void *x, int32_t row_bytes, const float *scales,
                    int32_t ns, const float *w, const int32_t *idx, int32_t T, hipStream_t st) {
  const RowSplit rs = row_split(row_bytes / 16, T);
  switch (rs.nvl) {
    case 1: return launch_nvl<KT, SCALED, 1>(a, x, row_bytes, scales, ns, w, idx, T, rs.parts, st);
    case 2: return launch_nvl<KT, SCALED, 2>(a, x, row_bytes, scales, ns, w, idx, T, rs.parts, st);
    case 4: return launch_nvl<KT, SCALED, 4>(a, x, row_bytes, scales, ns, w, idx, T, rs.parts, st);
    case 7: return launch_nvl<KT, SCALED, 7>(a, x, row_bytes, scales, ns, w, idx, T, rs.parts, st);
    case 8: return launch_nvl<KT, SCALED, 8>(a, x, row_bytes, scales, ns, w, idx, T, rs.parts, st);
    case 14: return launch_nvl<KT, SCALED, 14>(a, x, row_bytes, scales, ns, w, idx, T, rs.parts, st);
    case 16: return launch_nvl<KT, SCALED, 16>(a, x, row_bytes, scales, ns, w, idx, T, rs.parts, st);
    default: return launch_nvl<KT, SCALED, 0>(a, x, row_bytes, scales, ns, w, idx, T, 1, st);
  }
}

template <bool SCALED>
hipError_t launch_any_k(const MoeArgs &a, const void *x, int32_t row_bytes, const float *scales,
                        int32_t ns, const float *w, const int32_t *idx, int32_t T,
                        hipStream_t st) {
  if (T == 0) return hipSuccess;
  switch (a.K) {
    case 1: return launch_k<1, SCALED>(a, x, row_bytes, scales, ns, w, idx, T, st);
    case 2: return launch_k<2, SCALED>(a, x, row_bytes, scales, ns, w, idx, T, st);
    case 4: return launch_k<4, SCALED>(a, x, row_bytes, scales, ns, w, idx, T, st);
    case 6: return launch_k<6, SCALED>(a, x, row_bytes, scales, ns, w, idx, T, st);
    case 8: return launch_k<8, SCALED>(a, x, row_bytes, scales, ns, w, idx, T, st);
    default: return launch_k<0, SCALED>(a, x, row_bytes, scales, ns, w, idx, T, st);
  }
}

}  // namespace

hipError_t launch_dispatch(const MoeArgs &a, const uint16_t *x, const float *w,
                           const int32_t *idx, int32_t T, hipStream_t st) {
  return launch_any_k<false>(a, x, a.H * 2, nullptr, 0, w, idx, T, st);
}

hipError_t launch_dispatch_fp8(const MoeArgs &a, const uint8_t *x8, const float *scales,
                               int32_t ns, const float *w, const int32_t *idx, int32_t T,
                               hipStream_t st) {
  if (ns > 0) return launch_any_k<true>(a, x8, a.H, scales, ns, w, idx, T, st);
  return launch_any_k<false>(a, x8, a.H, nullptr, 0, w, idx, T, st);
}

}  // namespace cco
