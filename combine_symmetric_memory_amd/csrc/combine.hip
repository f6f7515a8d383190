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
#include "cco_internal.h"

namespace cco {
namespace {

constexpr int kCombineWaves = 4;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Two fp32 values -> packed bf16 (lo, hi), round to nearest even: gfx950's
// v_cvt_pk_bf16_f32, which the compiler emits for a plain conversion.
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// NVL > 0 (K <= 8 only): wavefront g sums part g % parts of token
// g / parts, NVL vectors per lane (the row is a whole number of such parts),
// in groups of G vectors with fixed address offsets and no bounds tests.
// NVL == 0: one wavefront per token, the general loop over the row.
template <int KT, int NVL>
__global__ __launch_bounds__(kCombineWaves *kWave) void combine_kernel(
    MoeArgs a, uint64_t src_win, const float *__restrict__ w, const int32_t *__restrict__ idx,
    u32x4 *__restrict__ out, int32_t T, int32_t parts) {
  constexpr int KM = KT > 0 ? KT : kMaxTopk;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int gw = blockIdx.x * kCombineWaves + wave;
  const int t = gw / parts, part = gw - t * parts;
  const int lane = threadIdx.x & (kWave - 1);
  if (t >= T) return;
  const int nk = KT > 0 ? KT : a.K;
  const int nvec = a.H / 8;
  const uint64_t rb = (uint64_t)a.H * 2;

  const u32x4 *src[KM];
  float wj[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    src[j] = nullptr;
    wj[j] = 0.0f;
    if (j < nk) {
      const int f = t * nk + j;
      const int e = idx[f];
      const int p = a.pos[f];
      wj[j] = w[f];
      if ((unsigned)e < (unsigned)a.E && p >= 0 && (int64_t)p < a.cap)
        src[j] = (const u32x4 *)slot_addr(a, slot_of(a, e), src_win, (uint64_t)p * rb);
    }
  }
  u32x4 *orow = out + (int64_t)t * nvec;
  // for K <= 8 two vectors per lane are in flight (2K row loads issued
  // before any math); the rows are read once, so the loads stream past the
  // caches
  auto accumulate = [&](const u32x4 (&r)[KM]) __attribute__((always_inline)) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < nk && src[j] != nullptr) {
        const uint32_t c[4] = {r[j].x, r[j].y, r[j].z, r[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = __builtin_fmaf(wj[j], bf16_lo(c[q]), acc[2 * q]);
          acc[2 * q + 1] = __builtin_fmaf(wj[j], bf16_hi(c[q]), acc[2 * q + 1]);
        }
      }
    }
    u32x4 o;
    o.x = pack_bf16_rne(acc[0], acc[1]);
    o.y = pack_bf16_rne(acc[2], acc[3]);
    o.z = pack_bf16_rne(acc[4], acc[5]);
    o.w = pack_bf16_rne(acc[6], acc[7]);
    return o;
  };
  if (NVL > 0 && KM <= 8) {
    // G vectors per lane of each of the K rows in flight (7 x 8 loads for
    // H = 7168, K = 8), then their sums
    constexpr int G = NVL % 7 == 0 ? 7 : (NVL < 4 ? NVL : 4);
    static_assert(NVL <= 0 || NVL % G == 0, "row length must be a whole number of groups");
    const int v0 = part * NVL * kWave;
#pragma unroll
    for (int g = 0; g < (NVL > 0 ? NVL / G : 0); ++g) {
      // issued vector by vector across the K rows, so that the first sums
      // wait only for the first loads
      u32x4 r[G][KM];
#pragma unroll
      for (int c = 0; c < G; ++c)
#pragma unroll
        for (int j = 0; j < KM; ++j)
          if (j < nk && src[j] != nullptr)
            r[c][j] = __builtin_nontemporal_load(src[j] + v0 + (g * G + c) * kWave + lane);
      u32x4 *o = orow + v0 + g * G * kWave + lane;
#pragma unroll
      for (int c = 0; c < G; ++c) o[c * kWave] = accumulate(r[c]);
    }
    return;
  }
  int v = lane;
  if (KM <= 8)
  for (; v + kWave < nvec; v += 2 * kWave) {
    u32x4 r0[KM], r1[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < nk && src[j] != nullptr) {
        r0[j] = __builtin_nontemporal_load(&src[j][v]);
        r1[j] = __builtin_nontemporal_load(&src[j][v + kWave]);
      }
    orow[v] = accumulate(r0);
    orow[v + kWave] = accumulate(r1);
  }
  for (; v < nvec; v += kWave) {
    u32x4 r0[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < nk && src[j] != nullptr) r0[j] = __builtin_nontemporal_load(&src[j][v]);
    orow[v] = accumulate(r0);
  }
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
