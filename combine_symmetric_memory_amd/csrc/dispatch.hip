// dispatch.hip -- scatter token rows into the receive windows of the slots.
//
// "MORI CCO: Next-Generation Collective Communication Object for GPUs",
// section "Zero-copy MoE dispatch -> expert -> combine", step 1: the
// dispatch kernel writes each token straight into the symmetric receive
// buffer of every rank that owns one of its experts, with no staging copy.
// The receive address is slot arithmetic (section "What is MORI CCO?"):
//   base + slot(e) * stride + DISP_X + pos[t][j] * (2 * H).
//
// One wavefront per token.  The token's K destinations are wave-uniform
// (scalar loads of idx and pos), the row is read once in 16-byte vectors
// (up to 16 per lane in flight) and each vector is stored K times; 64 lanes
// x 16 B make every store instruction one contiguous 1 KiB run.  Lanes 0..K-1 also write the
// per-row metadata {t*K + j, w[t][j], e}.
#include "cco_internal.h"

namespace cco {
namespace {

constexpr int kDispatchWaves = 4;

struct RowMeta {
  int32_t src;
  float w;
  int32_t e;
};

template <int KT>
__device__ __forceinline__ void dispatch_token(const MoeArgs &a, const u32x4 *__restrict__ xr,
                                               const float *__restrict__ w,
                                               const int32_t *__restrict__ idx, int t, int lane,
                                               int K) {
  constexpr int KM = KT > 0 ? KT : kMaxTopk;
  const int nk = KT > 0 ? KT : K;
  u32x4 *dst[KM];
  const int nvec = a.H / 8;
  const uint64_t rb = (uint64_t)a.H * 2;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    dst[j] = nullptr;
    if (j < nk) {
      const int f = t * nk + j;
      const int e = idx[f];
      const int p = a.pos[f];
      if ((unsigned)e < (unsigned)a.E && p >= 0 && (int64_t)p < a.cap)
        dst[j] = (u32x4 *)slot_addr(a, e / a.eps, a.off_disp_x, (uint64_t)p * rb);
    }
  }
  // the row in chunks of up to kChunk vectors per lane (the whole row for
  // H <= 8192): all of a chunk's loads are in flight before its K stores
  constexpr int kChunk = 16;
  for (int v0 = 0; v0 < nvec; v0 += kChunk * kWave) {
    u32x4 r[kChunk];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int v = v0 + c * kWave + lane;
      if (v < nvec) r[c] = xr[v];
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < nk && dst[j] != nullptr) {
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          const int v = v0 + c * kWave + lane;
          if (v < nvec) dst[j][v] = r[c];
        }
      }
    }
  }
  if (lane < nk) {
    const int f = t * nk + lane;
    const int e = idx[f];
    const int p = a.pos[f];
    if ((unsigned)e < (unsigned)a.E && p >= 0 && (int64_t)p < a.cap) {
      RowMeta *m = (RowMeta *)slot_addr(a, e / a.eps, a.off_meta, (uint64_t)p * sizeof(RowMeta));
      m->src = f;
      m->w = w[f];
      m->e = e;
    }
  }
}

template <int KT>
__global__ __launch_bounds__(kDispatchWaves *kWave) void dispatch_kernel(
    MoeArgs a, const u32x4 *__restrict__ x, const float *__restrict__ w,
    const int32_t *__restrict__ idx, int32_t T) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t = blockIdx.x * kDispatchWaves + wave;
  const int lane = threadIdx.x & (kWave - 1);
  if (t >= T) return;
  const u32x4 *xr = x + (int64_t)t * (a.H / 8);
  dispatch_token<KT>(a, xr, w, idx, t, lane, a.K);
}

template <int KT>
hipError_t launch_k(const MoeArgs &a, const uint16_t *x, const float *w, const int32_t *idx,
                    int32_t T, hipStream_t st) {
  const int nblk = (T + kDispatchWaves - 1) / kDispatchWaves;
  hipLaunchKernelGGL(dispatch_kernel<KT>, dim3(nblk), dim3(kDispatchWaves * kWave), 0, st, a,
                     (const u32x4 *)x, w, idx, T);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const MoeArgs &a, const uint16_t *x, const float *w,
                           const int32_t *idx, int32_t T, hipStream_t st) {
  if (T == 0) return hipSuccess;
  switch (a.K) {
    case 1: return launch_k<1>(a, x, w, idx, T, st);
    case 2: return launch_k<2>(a, x, w, idx, T, st);
    case 4: return launch_k<4>(a, x, w, idx, T, st);
    case 6: return launch_k<6>(a, x, w, idx, T, st);
    case 8: return launch_k<8>(a, x, w, idx, T, st);
    default: return launch_k<0>(a, x, w, idx, T, st);
  }
}

}  // namespace cco
