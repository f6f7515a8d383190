// plan_noalloc.hip -- the routing plan for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts
// that forbid allocation): no cco_moe object, caller-owned outputs, and the
// plan kernels' scratch in a file-scope device array of fixed size.
//
// The scratch holds the per-chunk histograms and exclusive prefixes, the
// chunk ticket, and each pair's expert id.  Each GPU the library runs on
// holds one copy of the array until the process ends, at its own address:
// the host looks that address up once per device (hipGetSymbolAddress, with
// the device current) and passes it to the kernels.  The array's name in
// host code is only a host-side stand-in and is never used as an address.
//
// Every call on one GPU shares that GPU's array and leaves its contents
// behind; the ticket, the only word that must start at zero, is cleared by a
// small kernel on the call's stream before the count kernel reads it.  Calls
// that overlap on one GPU (two streams, two host threads) race on the
// array: serialise them.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/cco_moe.h"
#include "cco_internal.h"

namespace {

// Largest batch the fixed scratch serves: 2^19 (token, k) pairs and
// kMaxExperts experts.
constexpr int64_t kNoAllocMaxPairs = int64_t(1) << 19;
constexpr int64_t kNoAllocMaxChunks = kNoAllocMaxPairs / cco::kPlanChunk;
// Layout in int32 words: [eid: max pairs][hist: max chunks x (E + 1)][ticket]
constexpr int64_t kEidWords = kNoAllocMaxPairs;
constexpr int64_t kHistWords = kNoAllocMaxChunks * (cco::kMaxExperts + 1);
constexpr int64_t kScratchWords = kEidWords + kHistWords + 64;
static_assert(kNoAllocMaxPairs % cco::kPlanChunk == 0, "whole chunks");

// About 3 MiB per GPU.
static __device__ __align__(256) int32_t scratch[kScratchWords];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
int32_t *g_scratch[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of this device's scratch array, looked up on the first call
// on the device (with that device current).
int32_t *scratch_of(int dev) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = (int32_t *)p;
  }
  return g_scratch[dev];
}

__global__ void clear_words_kernel(int32_t *p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

}  // namespace

extern "C" int cco_moe_plan_noalloc(const int32_t *topk_idx, int32_t T, int32_t K, int32_t E,
                                    int32_t S, int64_t cap, int32_t *pos, int32_t *counts,
                                    int32_t *expert_off, int32_t *slot_total, int32_t *status,
                                    void *stream) {
  if (T < 0 || K < 1 || K > cco::kMaxTopk || E < 1 || E > cco::kMaxExperts || S < 1 ||
      E % S != 0 || cap < 0 || cap > INT32_MAX)
    return CCO_ERR_INVALID_ARG;
  if ((int64_t)T * K > kNoAllocMaxPairs) return CCO_ERR_TOO_LARGE;
  if (!counts || !expert_off || !slot_total || !status || (T > 0 && (!topk_idx || !pos)))
    return CCO_ERR_INVALID_ARG;
  if (!aligned4(counts) || !aligned4(expert_off) || !aligned4(slot_total) || !aligned4(status) ||
      (T > 0 && (!aligned4(topk_idx) || !aligned4(pos))))
    return CCO_ERR_INVALID_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return CCO_ERR_HIP;
  if (dev >= kMaxDevices) return CCO_ERR_INVALID_ARG;
  int32_t *sp = scratch_of(dev);
  if (!sp) return CCO_ERR_HIP;

  cco::MoeArgs a{};
  a.cap = cap;
  a.K = K;
  a.E = E;
  a.S = S;
  a.eps = E / S;
  a.eps_magic = cco::eps_magic_of(a.eps);
  a.pos = pos;
  a.counts = counts;
  a.expert_off = expert_off;
  a.slot_total = slot_total;
  a.status = status;
  a.eid = sp;
  a.hist = sp + kEidWords;
  a.ticket = sp + kEidWords + kHistWords;

  hipStream_t st = (hipStream_t)stream;
  const int32_t n_pairs = T * K;
  const int32_t nblk = n_pairs > 0 ? (n_pairs + cco::kPlanChunk - 1) / cco::kPlanChunk : 1;
  if (n_pairs > 0 && nblk == 1)
    return cco::launch_plan_single(a, topk_idx, n_pairs, st) == hipSuccess ? CCO_OK
                                                                           : CCO_ERR_HIP;
  hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(64), 0, st, a.ticket, 1);
  if (hipGetLastError() != hipSuccess) return CCO_ERR_HIP;
  if (cco::launch_plan_count(a, topk_idx, n_pairs, nblk, st) != hipSuccess) return CCO_ERR_HIP;
  if (n_pairs > 0 && cco::launch_plan_rank(a, topk_idx, n_pairs, nblk, st) != hipSuccess)
    return CCO_ERR_HIP;
  return CCO_OK;
}
