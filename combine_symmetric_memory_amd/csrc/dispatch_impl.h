// dispatch_impl.h -- one wavefront's share of the dispatch: a token row (or
// a part of it) stored into the receive rows of its K pairs, and the per-row
// metadata.  Included by dispatch.hip and fused.hip.
//
// "MORI CCO: Next-Generation Collective Communication Object for GPUs",
// section "Zero-copy MoE dispatch -> expert -> combine", step 1: the token
// goes straight into the receive buffer of every rank that owns one of its
// experts, at a slot address (section "What is MORI CCO?").
#pragma once

#include "cco_internal.h"

namespace cco {
namespace {

struct RowMeta {
  int32_t src;
  float w;
  int32_t e;
};

// Row bytes of the token go to the K receive rows of its pairs; with SCALED
// the ns fp32 scales sc[0..ns) follow the token's nvec * 16 bytes.  NVL > 0:
// this wavefront moves part `part` of the row, NVL vectors per lane (the
// row is a whole number of such parts), with no per-vector bounds test and
// fixed address offsets; part 0 also moves the scales and the metadata.
// NVL == 0: the whole row (part 0).
template <int KT, bool SCALED, int NVL>
__device__ __forceinline__ void dispatch_token(const MoeArgs &a, const u32x4 *__restrict__ xr,
                                               int nvec, const float *__restrict__ sc, int ns,
                                               const float *__restrict__ w,
                                               const int32_t *__restrict__ idx, int t, int part,
                                               int lane, int K) {
  constexpr int KM = KT > 0 ? KT : (KT < 0 ? -KT : kMaxTopk);  // KT < 0: any K up to -KT
  const int nk = KT > 0 ? KT : K;
  u32x4 *dst[KM];
  const uint64_t rb = (uint64_t)a.H * 2;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    dst[j] = nullptr;
    if (j < nk) {
      const int f = t * nk + j;
      const int e = idx[f];
      const int p = a.pos[f];
      if ((unsigned)e < (unsigned)a.E && p >= 0 && (int64_t)p < a.cap)
        dst[j] = (u32x4 *)slot_addr(a, slot_of(a, e), a.off_disp_x, (uint64_t)p * rb);
    }
  }
  // the first 64 scales are loaded with the row, one per lane
  float s0 = 0.0f;
  if (SCALED && part == 0 && lane < ns) s0 = sc[lane];
  if (NVL > 0) {
    // the whole part in flight before its K stores
    const int v0 = part * NVL * kWave;
    u32x4 r[NVL > 0 ? NVL : 1];
#pragma unroll
    for (int c = 0; c < NVL; ++c) r[c] = xr[v0 + c * kWave + lane];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < nk && dst[j] != nullptr) {
        u32x4 *d = dst[j] + v0 + lane;
#pragma unroll
        for (int c = 0; c < NVL; ++c) d[c * kWave] = r[c];
      }
    }
  }
  // otherwise the row in chunks of up to kChunk vectors per lane (the whole
  // row for H <= 8192): all of a chunk's loads are in flight before its K
  // stores
  constexpr int kChunk = 16;
  for (int v0 = 0; NVL == 0 && v0 < nvec; v0 += kChunk * kWave) {
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
  if (SCALED && part == 0) {
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < nk && dst[j] != nullptr && lane < ns) ((float *)(dst[j] + nvec))[lane] = s0;
    for (int i = kWave + lane; i < ns; i += kWave) {
      const float si = sc[i];
#pragma unroll
      for (int j = 0; j < KM; ++j)
        if (j < nk && dst[j] != nullptr) ((float *)(dst[j] + nvec))[i] = si;
    }
  }
  if (part == 0 && lane < nk) {
    const int f = t * nk + lane;
    const int e = idx[f];
    const int p = a.pos[f];
    if ((unsigned)e < (unsigned)a.E && p >= 0 && (int64_t)p < a.cap) {
      RowMeta *m = (RowMeta *)slot_addr(a, slot_of(a, e), a.off_meta, (uint64_t)p * sizeof(RowMeta));
      m->src = f;
      m->w = w[f];
      m->e = e;
    }
  }
}

}  // namespace
}  // namespace cco
