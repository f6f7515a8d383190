// combine_impl.h -- one wavefront's share of the combine: a token's output
// row (or a part of it) as the weighted sum of its K expert rows.  Included
// by combine.hip and fused.hip.
//
// "MORI CCO: Next-Generation Collective Communication Object for GPUs",
// section "Zero-copy MoE dispatch -> expert -> combine", step 3: each token
// reads its rows back from the staging buffers of the ranks that own its
// experts and sums them with its routing weights:
//   out[t][h] = bf16( fma(w[t][K-1], y_{K-1}[h], ... fma(w[t][0], y_0[h], 0)) )
// in fp32, in j order, rounded once to nearest even.
#pragma once

#include "cco_internal.h"

namespace cco {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Two fp32 values -> packed bf16 (lo, hi), round to nearest even: gfx950's
// v_cvt_pk_bf16_f32, which the compiler emits for a plain conversion.
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// One wavefront's share (`lane` is its lane): part `part` of token t's output
// row.  KT > 0: K == KT; KT == 0: any K; KT < 0: any K up to -KT.
// NVL > 0 (K <= 8 only): NVL vectors per lane (the row is a whole number of
// such parts), in groups of G vectors with fixed address offsets and no
// bounds tests (GV > 0 sets G; it must divide NVL).  NVL == 0: the whole row
// (part 0), the general loop.
template <int KT, int NVL, int GV = 0>
__device__ __forceinline__ void combine_token(const MoeArgs &a, uint64_t src_win,
                                              const float *__restrict__ w,
                                              const int32_t *__restrict__ idx,
                                              u32x4 *__restrict__ out, int t, int part, int lane) {
  constexpr int KM = KT > 0 ? KT : (KT < 0 ? -KT : kMaxTopk);
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
    constexpr int G = GV > 0 ? GV : (NVL % 7 == 0 ? 7 : (NVL < 4 ? NVL : 4));
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

}  // namespace
}  // namespace cco
