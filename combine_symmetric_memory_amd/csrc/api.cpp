// api.cpp -- the C ABI of include/cco_moe.h: argument checks, the symmetric
// heap, window layout, routing state, kernel launches, status.
//
// "MORI CCO Guide", sections "Memory and Windows" and "C++ API": symmetric
// memory sits at the same offset in every rank's slot, windows are
// registered over it, and resources are owned by (and freed with) the
// object that made them.  "MORI CCO: Next-Generation Collective
// Communication Object for GPUs", section "Zero-copy MoE dispatch -> expert
// -> combine": the MoE op hands out views of symmetric memory and allocates
// nothing per call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/cco_moe.h"
#include "cco_internal.h"

using cco::MoeArgs;

namespace {

constexpr uint64_t kSlotAlign = 2ull << 20;  // slot stride granularity (2 MiB)
constexpr uint64_t kWinAlign = 4096;         // window start alignment
constexpr uint64_t kGuardBytes = 256;        // guard bytes after every window
constexpr unsigned char kGuardByte = 0xA5;

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// The kernels read and write rows in 16-byte vectors and routing data in
// 4-byte words.
bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) return;
    ok = (prev == dev) || hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

struct TimedPair {
  hipEvent_t start, stop;
};

}  // namespace

struct cco_moe {
  cco_sym_heap *heap = nullptr;
  cco_moe_shape shape{};
  int32_t S = 0, eps = 0;
  int64_t cap = 0;
  cco_moe_layout lay{};  // absolute offsets inside a slot
  void *state = nullptr; // routing state (one device allocation)
  MoeArgs args{};
  int32_t max_plan_blocks = 0;
  int32_t planned_T = -1;  // T of the last plan (host-side order check)
  bool disp_8bit = false;  // the last dispatch moved 8-bit tokens with scales
  int32_t disp_ns = 0;     // ... and that many scales per token
  int num_cus = 0;
  cco::FusedBuffers fused{};
  bool timing = false;
  std::vector<TimedPair> pending[CCO_NUM_KERNEL_KINDS];
  int32_t timed_launches[CCO_NUM_KERNEL_KINDS] = {};
  double timed_ms[CCO_NUM_KERNEL_KINDS] = {};
};

struct cco_sym_heap {
  int device = 0;
  int32_t nslots = 0;
  uint64_t stride = 0;
  uint64_t used = 0;
  char *base = nullptr;
  std::vector<cco_moe *> objs;
};

namespace {

// Shape checks shared by every entry point; no HIP calls.
bool shape_ok(const cco_moe_shape *s, int32_t nslots) {
  if (!s || nslots < 1) return false;
  if (s->max_tokens < 0 || s->hidden <= 0 || s->topk < 1 || s->num_experts < 1) return false;
  if (s->hidden % 8 != 0) return false;
  if (s->topk > cco::kMaxTopk || s->num_experts > cco::kMaxExperts) return false;
  if (s->num_experts % nslots != 0) return false;
  if (s->inter < 0) return false;
  if (s->inter > 0 && (s->inter % 128 != 0 || s->hidden % 256 != 0)) return false;
  // the expert GEMMs address one expert's weights through a 31-bit byte range
  if (s->inter > 0 && (int64_t)4 * s->inter * s->hidden > INT32_MAX) return false;
  // int32 row and pair indices
  const int64_t eps = s->num_experts / nslots;
  const int64_t cap = (int64_t)s->max_tokens * std::min<int64_t>(s->topk, eps);
  if ((int64_t)s->max_tokens * s->topk > INT32_MAX || cap > INT32_MAX) return false;
  return true;
}

bool layout_of(const cco_moe_shape *s, int32_t nslots, cco_moe_layout *L) {
  if (!shape_ok(s, nslots)) return false;
  const int64_t eps = s->num_experts / nslots;
  const int64_t cap = (int64_t)s->max_tokens * std::min<int64_t>(s->topk, eps);
  const uint64_t H = (uint64_t)s->hidden, I = (uint64_t)s->inter;
  std::memset(L, 0, sizeof(*L));
  L->cap = cap;
  uint64_t off = 0;
  auto place = [&](uint64_t bytes, uint64_t *o, uint64_t *b) {
    *o = off;
    *b = bytes;
    off = align_up(off + bytes + kGuardBytes, kWinAlign);
  };
  place((uint64_t)cap * H * 2, &L->disp_x, &L->disp_x_bytes);
  place((uint64_t)cap * 12, &L->disp_meta, &L->disp_meta_bytes);
  if (I > 0) {
    place((uint64_t)cap * I * 2, &L->hbuf, &L->hbuf_bytes);
    place((uint64_t)cap * H * 2, &L->out_tok, &L->out_tok_bytes);
  }
  // total footprint is carried in out_tok + out_tok_bytes's successor: the
  // caller recomputes it through required_bytes()
  return true;
}

uint64_t required_bytes(const cco_moe_layout &L) {
  uint64_t end = 0;
  const uint64_t o[4] = {L.disp_x, L.disp_meta, L.hbuf, L.out_tok};
  const uint64_t b[4] = {L.disp_x_bytes, L.disp_meta_bytes, L.hbuf_bytes, L.out_tok_bytes};
  for (int i = 0; i < 4; ++i)
    if (b[i] > 0) end = std::max(end, align_up(o[i] + b[i] + kGuardBytes, kWinAlign));
  return end;
}

int32_t plan_blocks(int64_t n_pairs) {
  const int64_t nb = (n_pairs + cco::kPlanChunk - 1) / cco::kPlanChunk;
  return (int32_t)std::max<int64_t>(1, nb);
}

// Launch `fn` (returning hipError_t), bracketed by timing events if enabled.
template <class F>
int timed_launch(cco_moe *m, int kind, hipStream_t st, F &&fn) {
  if (!m->timing) return fn() == hipSuccess ? CCO_OK : CCO_ERR_HIP;
  TimedPair tp{nullptr, nullptr};
  auto drop = [&tp] {
    if (tp.start) (void)hipEventDestroy(tp.start);
    if (tp.stop) (void)hipEventDestroy(tp.stop);
  };
  if (hipEventCreate(&tp.start) != hipSuccess || hipEventCreate(&tp.stop) != hipSuccess ||
      hipEventRecord(tp.start, st) != hipSuccess) {
    drop();
    return CCO_ERR_HIP;
  }
  if (fn() != hipSuccess || hipEventRecord(tp.stop, st) != hipSuccess) {
    drop();
    return CCO_ERR_HIP;
  }
  m->pending[kind].push_back(tp);
  return CCO_OK;
}

void free_moe(cco_moe *m) {
  for (auto &v : m->pending)
    for (auto &tp : v) {
      (void)hipEventDestroy(tp.start);
      (void)hipEventDestroy(tp.stop);
    }
  if (m->state) (void)hipFree(m->state);
  delete m;
}

}  // namespace

extern "C" {

const char *cco_status_string(int st) {
  switch (st) {
    case CCO_OK: return "CCO_OK";
    case CCO_INFO_COPIED: return "CCO_INFO_COPIED";
    case CCO_ERR_INVALID_ARG: return "CCO_ERR_INVALID_ARG";
    case CCO_ERR_OUT_OF_MEMORY: return "CCO_ERR_OUT_OF_MEMORY";
    case CCO_ERR_HIP: return "CCO_ERR_HIP";
    case CCO_ERR_CAPACITY: return "CCO_ERR_CAPACITY";
    case CCO_ERR_BAD_EXPERT: return "CCO_ERR_BAD_EXPERT";
    case CCO_ERR_HEAP_FULL: return "CCO_ERR_HEAP_FULL";
    case CCO_ERR_TOO_LARGE: return "CCO_ERR_TOO_LARGE";
    case CCO_ERR_TIMEOUT: return "CCO_ERR_TIMEOUT";
    case CCO_ERR_DISABLED: return "CCO_ERR_DISABLED";
    default: return "unknown cco status";
  }
}

int cco_sym_heap_create(int device, int32_t nslots, uint64_t per_slot_bytes, cco_sym_heap **out) {
  if (!out || nslots < 1 || per_slot_bytes == 0 || device < 0) return CCO_ERR_INVALID_ARG;
  *out = nullptr;
  const uint64_t stride = align_up(per_slot_bytes, kSlotAlign);
  if (stride / kSlotAlign > (UINT64_MAX / kSlotAlign) / (uint64_t)nslots) return CCO_ERR_INVALID_ARG;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) return CCO_ERR_HIP;
  if (device >= ndev) return CCO_ERR_INVALID_ARG;
  DeviceGuard dg(device);
  if (!dg.ok) return CCO_ERR_HIP;
  void *p = nullptr;
  const hipError_t err = hipMalloc(&p, stride * (uint64_t)nslots);
  if (err == hipErrorOutOfMemory) return CCO_ERR_OUT_OF_MEMORY;
  if (err != hipSuccess) return CCO_ERR_HIP;
  auto *h = new (std::nothrow) cco_sym_heap;
  if (!h) {
    (void)hipFree(p);
    return CCO_ERR_OUT_OF_MEMORY;
  }
  h->device = device;
  h->nslots = nslots;
  h->stride = stride;
  h->base = (char *)p;
  *out = h;
  return CCO_OK;
}

int cco_sym_heap_destroy(cco_sym_heap *heap) {
  if (!heap) return CCO_OK;
  int rc = CCO_OK;
  {
    DeviceGuard dg(heap->device);
    if (hipDeviceSynchronize() != hipSuccess) rc = CCO_ERR_HIP;
    for (cco_moe *m : heap->objs) free_moe(m);
    if (heap->base && hipFree(heap->base) != hipSuccess) rc = CCO_ERR_HIP;
  }
  delete heap;
  return rc;
}

void *cco_sym_heap_slot_ptr(const cco_sym_heap *heap, int32_t slot, uint64_t offset) {
  if (!heap || slot < 0 || slot >= heap->nslots || offset >= heap->stride) return nullptr;
  return heap->base + (uint64_t)slot * heap->stride + offset;
}

int cco_sym_heap_info(const cco_sym_heap *heap, void **base, uint64_t *stride, int32_t *nslots,
                      uint64_t *used) {
  if (!heap) return CCO_ERR_INVALID_ARG;
  if (base) *base = heap->base;
  if (stride) *stride = heap->stride;
  if (nslots) *nslots = heap->nslots;
  if (used) *used = heap->used;
  return CCO_OK;
}

uint64_t cco_moe_required_slot_bytes(const cco_moe_shape *shape, int32_t nslots) {
  cco_moe_layout L;
  if (!layout_of(shape, nslots, &L)) return 0;
  return required_bytes(L);
}

int cco_moe_layout_of(const cco_moe_shape *shape, int32_t nslots, cco_moe_layout *out) {
  if (!out || !layout_of(shape, nslots, out)) return CCO_ERR_INVALID_ARG;
  return CCO_OK;
}

int cco_moe_create(cco_sym_heap *heap, const cco_moe_shape *shape, cco_moe **out) {
  if (!heap || !shape || !out) return CCO_ERR_INVALID_ARG;
  *out = nullptr;
  cco_moe_layout L;
  if (!layout_of(shape, heap->nslots, &L)) return CCO_ERR_INVALID_ARG;
  const uint64_t need = required_bytes(L);
  const uint64_t start = align_up(heap->used, kWinAlign);
  if (start + need > heap->stride) return CCO_ERR_HEAP_FULL;

  DeviceGuard dg(heap->device);
  if (!dg.ok) return CCO_ERR_HIP;
  auto *m = new (std::nothrow) cco_moe;
  if (!m) return CCO_ERR_OUT_OF_MEMORY;
  m->heap = heap;
  m->shape = *shape;
  m->S = heap->nslots;
  m->eps = shape->num_experts / heap->nslots;
  m->cap = L.cap;
  m->lay = L;
  m->lay.disp_x += start;
  m->lay.disp_meta += start;
  if (L.hbuf_bytes) m->lay.hbuf += start;
  if (L.out_tok_bytes) m->lay.out_tok += start;

  const int64_t npairs = (int64_t)shape->max_tokens * shape->topk;
  m->max_plan_blocks = plan_blocks(npairs);
  const int E = shape->num_experts;
  if (hipDeviceGetAttribute(&m->num_cus, hipDeviceAttributeMultiprocessorCount, heap->device) !=
          hipSuccess ||
      m->num_cus <= 0) {
    delete m;
    return CCO_ERR_HIP;
  }
  // routing state: pos, eid, counts, expert_off, slot_total, status, ticket,
  // GEMM tile queues, split-tile descriptors, hist, and (with experts) the
  // split tiles' partial sums, 256-byte aligned
  const int nwg = cco::gemm_workgroups(m->num_cus);
  const size_t n_desc = (size_t)(nwg / 2) * cco::kSplitDescInts;
  const size_t n_mt = (size_t)cco::fused_mtiles(shape->max_tokens, shape->topk, E);
  const size_t n_fused = cco::kFusedCounterWords + 3 * (size_t)(E + 1) + E + 2 * n_mt;
  const size_t n_head = (size_t)npairs * 2 + (size_t)E * 2 + (size_t)m->S + 2 +
                        4 * (cco::kNumXcd + 1) + n_desc + (size_t)m->max_plan_blocks * (E + 1) +
                        n_fused;
  const size_t ws_at = (n_head + 63) / 64 * 64;
  const size_t n_ws = shape->inter > 0 ? (size_t)nwg * cco::kSplitTileFloats : 0;
  const size_t n_i32 = ws_at + n_ws;
  void *st = nullptr;
  hipError_t err = hipMalloc(&st, std::max<size_t>(n_i32, 1) * sizeof(int32_t));
  if (err != hipSuccess) {
    delete m;
    return err == hipErrorOutOfMemory ? CCO_ERR_OUT_OF_MEMORY : CCO_ERR_HIP;
  }
  m->state = st;
  if (hipMemset(st, 0, n_i32 * sizeof(int32_t)) != hipSuccess) {
    free_moe(m);
    return CCO_ERR_HIP;
  }
  int32_t *p = (int32_t *)st;
  MoeArgs &a = m->args;
  a.base = heap->base;
  a.stride = heap->stride;
  a.off_disp_x = m->lay.disp_x;
  a.off_meta = m->lay.disp_meta;
  a.off_hbuf = m->lay.hbuf;
  a.off_out = m->lay.out_tok;
  a.cap = m->cap;
  a.K = shape->topk;
  a.H = shape->hidden;
  a.E = E;
  a.S = m->S;
  a.eps = m->eps;
  a.eps_magic = cco::eps_magic_of(m->eps);
  a.I = shape->inter;
  a.pos = p;               p += npairs;
  a.eid = p;               p += npairs;
  a.counts = p;            p += E;
  a.expert_off = p;        p += E;
  a.slot_total = p;        p += m->S;
  a.status = p;            p += 1;
  a.ticket = p;            p += 1;
  a.gemm_queue = p;        p += 4 * (cco::kNumXcd + 1);
  a.split_desc = p;        p += n_desc;
  m->fused.q = p;          p += cco::kFusedCounterWords;
  m->fused.pre_g = p;      p += E + 1;
  m->fused.pre_w = p;      p += E + 1;
  m->fused.pre_mt = p;     p += E + 1;
  m->fused.arrived = p;    p += E;
  m->fused.gu_done = p;    p += n_mt;
  m->fused.dn_done = p;    p += n_mt;
  a.hist = p;
  a.split_ws = n_ws ? (float *)((int32_t *)st + ws_at) : nullptr;

  // guard bytes after every window of every slot
  const uint64_t wo[4] = {m->lay.disp_x, m->lay.disp_meta, m->lay.hbuf, m->lay.out_tok};
  const uint64_t wb[4] = {L.disp_x_bytes, L.disp_meta_bytes, L.hbuf_bytes, L.out_tok_bytes};
  for (int s = 0; s < m->S; ++s)
    for (int i = 0; i < 4; ++i)
      if (wb[i] > 0 &&
          hipMemset(heap->base + (uint64_t)s * heap->stride + wo[i] + wb[i], kGuardByte,
                    kGuardBytes) != hipSuccess) {
        free_moe(m);
        return CCO_ERR_HIP;
      }
  if (hipDeviceSynchronize() != hipSuccess) {
    free_moe(m);
    return CCO_ERR_HIP;
  }
  heap->used = start + need;
  heap->objs.push_back(m);
  *out = m;
  return CCO_OK;
}

int cco_moe_get_layout(const cco_moe *m, cco_moe_layout *out) {
  if (!m || !out) return CCO_ERR_INVALID_ARG;
  *out = m->lay;
  return CCO_OK;
}

int cco_moe_get_routing(const cco_moe *m, cco_moe_routing *out) {
  if (!m || !out) return CCO_ERR_INVALID_ARG;
  out->pos = m->args.pos;
  out->counts = m->args.counts;
  out->expert_off = m->args.expert_off;
  out->slot_total = m->args.slot_total;
  out->status = m->args.status;
  return CCO_OK;
}

int cco_moe_plan(cco_moe *m, const int32_t *topk_idx, int32_t T, void *stream) {
  if (!m || T < 0 || T > m->shape.max_tokens || (T > 0 && (!topk_idx || !aligned(topk_idx, 4))))
    return CCO_ERR_INVALID_ARG;
  DeviceGuard dg(m->heap->device);
  if (!dg.ok) return CCO_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  const int32_t n_pairs = T * m->shape.topk;
  const int32_t nblk = plan_blocks(n_pairs);
  MoeArgs a = m->args;
  if (n_pairs > 0 && nblk == 1) {
    // one chunk: count and rank in one launch
    const int rc = timed_launch(m, 0, st, [&] {
      return cco::launch_plan_single(a, topk_idx, n_pairs, st);
    });
    if (rc != CCO_OK) return rc;
    m->planned_T = T;
    return CCO_OK;
  }
  int rc = timed_launch(m, 0, st, [&] { return cco::launch_plan_count(a, topk_idx, n_pairs, nblk, st); });
  if (rc != CCO_OK) return rc;
  if (n_pairs > 0) {
    // plan_rank also records each pair's expert id in the routing state, so
    // that dispatch and combine need only the routing object
    rc = timed_launch(m, 1, st, [&] {
      return cco::launch_plan_rank(a, topk_idx, n_pairs, nblk, st);
    });
    if (rc != CCO_OK) return rc;
  }
  m->planned_T = T;
  return CCO_OK;
}

int cco_moe_dispatch(cco_moe *m, const uint16_t *x, const float *weights, int32_t T, void *stream) {
  if (!m || T < 0 || T != m->planned_T || (T > 0 && (!x || !weights))) return CCO_ERR_INVALID_ARG;
  if (T > 0 && (!aligned(x, 16) || !aligned(weights, 4))) return CCO_ERR_INVALID_ARG;
  DeviceGuard dg(m->heap->device);
  if (!dg.ok) return CCO_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  m->disp_8bit = false;
  if (T == 0) return CCO_OK;
  MoeArgs a = m->args;
  return timed_launch(m, 2, st, [&] { return cco::launch_dispatch(a, x, weights, a.eid, T, st); });
}

int cco_moe_dispatch_fp8(cco_moe *m, const uint8_t *x8, const float *scales, int32_t ns,
                         const float *weights, int32_t T, void *stream) {
  if (!m || T < 0 || T != m->planned_T) return CCO_ERR_INVALID_ARG;
  const int32_t H = m->shape.hidden;
  if (H % 16 != 0 || ns < 0 || (int64_t)ns * 4 > H) return CCO_ERR_INVALID_ARG;
  if (T > 0 && (!x8 || !weights || (ns > 0 && !scales))) return CCO_ERR_INVALID_ARG;
  if (T > 0 && (!aligned(x8, 16) || !aligned(weights, 4) || (ns > 0 && !aligned(scales, 4))))
    return CCO_ERR_INVALID_ARG;
  DeviceGuard dg(m->heap->device);
  if (!dg.ok) return CCO_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  m->disp_8bit = true;
  m->disp_ns = ns;
  if (T == 0) return CCO_OK;
  MoeArgs a = m->args;
  return timed_launch(m, 7, st, [&] {
    return cco::launch_dispatch_fp8(a, x8, scales, ns, weights, a.eid, T, st);
  });
}

int cco_moe_expert(cco_moe *m, const uint16_t *w13, const uint16_t *w2, void *stream) {
  if (!m || m->planned_T < 0) return CCO_ERR_INVALID_ARG;
  if (m->shape.inter == 0) return CCO_OK;  // identity experts
  if (!w13 || !w2 || !aligned(w13, 16) || !aligned(w2, 16)) return CCO_ERR_INVALID_ARG;
  // 8-bit receive rows: their scale blocks must be whole runs of K-steps
  // of 64 (a power of two of them), or absent
  int32_t a8_ns = -1;
  if (m->disp_8bit) {
    const int32_t ns = m->disp_ns, H = m->shape.hidden;
    if (ns > 0) {
      if (H % ns != 0) return CCO_ERR_INVALID_ARG;
      const int32_t ksteps = (H / ns) / 64;
      if ((H / ns) % 64 != 0 || (ksteps & (ksteps - 1)) != 0) return CCO_ERR_INVALID_ARG;
    }
    a8_ns = ns;
  }
  DeviceGuard dg(m->heap->device);
  if (!dg.ok) return CCO_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  if (m->planned_T == 0) return CCO_OK;
  MoeArgs a = m->args;
  const int32_t T = m->planned_T;
  int rc = timed_launch(m, 3, st,
                        [&] { return cco::launch_expert_gate_up(a, w13, T, m->num_cus, a8_ns, st); });
  if (rc != CCO_OK) return rc;
  return timed_launch(m, 4, st,
                      [&] { return cco::launch_expert_down(a, w2, T, m->num_cus, st); });
}

void *cco_moe_dispatch_view(cco_moe *m, int32_t slot) {
  if (!m || slot < 0 || slot >= m->S) return nullptr;
  return m->heap->base + (uint64_t)slot * m->heap->stride + m->lay.disp_x;
}

void *cco_moe_combine_in_view(cco_moe *m, int32_t slot) {
  if (!m || slot < 0 || slot >= m->S) return nullptr;
  const uint64_t win = m->shape.inter > 0 ? m->lay.out_tok : m->lay.disp_x;
  return m->heap->base + (uint64_t)slot * m->heap->stride + win;
}

int cco_moe_combine(cco_moe *m, const void *const *expert_out, const float *weights, uint16_t *out,
                    int32_t T, void *stream) {
  if (!m || T < 0 || T != m->planned_T || (T > 0 && (!weights || !out))) return CCO_ERR_INVALID_ARG;
  if (T > 0 && (!aligned(out, 16) || !aligned(weights, 4))) return CCO_ERR_INVALID_ARG;
  if (expert_out)
    for (int s = 0; s < m->S; ++s)
      if (expert_out[s] && !aligned(expert_out[s], 16)) return CCO_ERR_INVALID_ARG;
  DeviceGuard dg(m->heap->device);
  if (!dg.ok) return CCO_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  if (T == 0) return CCO_OK;
  const uint64_t win = m->shape.inter > 0 ? m->lay.out_tok : m->lay.disp_x;
  if (m->shape.inter == 0 && m->disp_8bit) {
    // identity experts would hand combine the 8-bit receive rows as bf16
    for (int s = 0; s < m->S; ++s) {
      const void *src = expert_out ? expert_out[s] : nullptr;
      if (!src || src == cco_moe_combine_in_view(m, s)) return CCO_ERR_INVALID_ARG;
    }
  }
  MoeArgs a = m->args;
  bool copied = false;
  if (expert_out) {
    for (int s = 0; s < m->S; ++s) {
      const void *src = expert_out[s];
      if (!src || src == cco_moe_combine_in_view(m, s)) continue;
      const int rc = timed_launch(m, 6, st, [&] {
        return cco::launch_copy_in(a, s, (const uint16_t *)src, win, st);
      });
      if (rc != CCO_OK) return rc;
      copied = true;
    }
  }
  const int rc = timed_launch(m, 5, st, [&] {
    return cco::launch_combine(a, win, weights, a.eid, out, T, st);
  });
  if (rc != CCO_OK) return rc;
  return copied ? CCO_INFO_COPIED : CCO_OK;
}

int cco_moe_fused(cco_moe *m, const int32_t *topk_idx, const uint16_t *x, const float *weights,
                  const uint16_t *w13, const uint16_t *w2, uint16_t *out, int32_t T,
                  void *stream) {
  if (!m || T < 0 || T > m->shape.max_tokens) return CCO_ERR_INVALID_ARG;
  if (m->shape.topk > 8) return CCO_ERR_INVALID_ARG;  // the single launch takes top-k <= 8
  if (T > 0 && (!topk_idx || !x || !weights || !out)) return CCO_ERR_INVALID_ARG;
  if (T > 0 && (!aligned(topk_idx, 4) || !aligned(x, 16) || !aligned(weights, 4) ||
                !aligned(out, 16)))
    return CCO_ERR_INVALID_ARG;
  if (m->shape.inter > 0 && (!w13 || !w2 || !aligned(w13, 16) || !aligned(w2, 16)))
    return CCO_ERR_INVALID_ARG;
  if (T == 0) {
    // nothing to move: the plan of an empty batch (zero counts)
    const int rc = cco_moe_plan(m, topk_idx, 0, stream);
    if (rc == CCO_OK) m->disp_8bit = false;
    return rc;
  }
  DeviceGuard dg(m->heap->device);
  if (!dg.ok) return CCO_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  MoeArgs a = m->args;
  hipError_t err = hipSuccess;
  const int rc = timed_launch(m, 9, st, [&] {
    err = cco::launch_fused(a, m->fused, topk_idx, x, weights, w13, w2, out, T, m->num_cus, st);
    return err;
  });
  if (err == hipErrorNotSupported) return CCO_ERR_DISABLED;  // not built (see fused.hip)
  if (rc != CCO_OK) return rc;
  m->planned_T = T;
  m->disp_8bit = false;
  return CCO_OK;
}

int cco_moe_stage_in_sdma(cco_moe *m, int32_t slot, const void *src, int32_t rows,
                          void *stream) {
  if (!m || slot < 0 || slot >= m->S || rows < 0 || (int64_t)rows > m->cap) return CCO_ERR_INVALID_ARG;
  if (rows == 0) return CCO_OK;
  if (!src || !aligned(src, 16)) return CCO_ERR_INVALID_ARG;
  char *dst = (char *)cco_moe_combine_in_view(m, slot);
  if (src == dst) return CCO_OK;  // already the staging view
  const uint64_t n = (uint64_t)rows * (uint64_t)m->shape.hidden * 2;
  const char *s = (const char *)src;
  if (s < dst + n && dst < s + n) return CCO_ERR_INVALID_ARG;
  DeviceGuard dg(m->heap->device);
  if (!dg.ok) return CCO_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  // hipMemcpyDeviceToDeviceNoCU: a device-to-device copy on the copy
  // engines, with no kernel on the compute units
  return timed_launch(m, 8, st, [&] {
    return hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDeviceNoCU, st);
  });
}

int cco_moe_status(cco_moe *m, void *stream, int32_t *slot_total, int32_t *expert_counts) {
  if (!m) return CCO_ERR_INVALID_ARG;
  DeviceGuard dg(m->heap->device);
  if (!dg.ok) return CCO_ERR_HIP;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return CCO_ERR_HIP;
  if (slot_total && hipMemcpy(slot_total, m->args.slot_total, sizeof(int32_t) * m->S,
                              hipMemcpyDeviceToHost) != hipSuccess)
    return CCO_ERR_HIP;
  if (expert_counts && hipMemcpy(expert_counts, m->args.counts,
                                 sizeof(int32_t) * m->shape.num_experts,
                                 hipMemcpyDeviceToHost) != hipSuccess)
    return CCO_ERR_HIP;
  int32_t word = 0;
  if (hipMemcpy(&word, m->args.status, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return CCO_ERR_HIP;
  return word;
}

int cco_moe_set_timing(cco_moe *m, int enable) {
  if (!m) return CCO_ERR_INVALID_ARG;
  m->timing = enable != 0;
  return CCO_OK;
}

int cco_moe_timing_summary(cco_moe *m, int32_t *launches, double *total_ms) {
  if (!m) return CCO_ERR_INVALID_ARG;
  DeviceGuard dg(m->heap->device);
  int rc = CCO_OK;
  for (int k = 0; k < CCO_NUM_KERNEL_KINDS; ++k) {
    for (auto &tp : m->pending[k]) {
      float ms = 0.0f;
      if (hipEventSynchronize(tp.stop) != hipSuccess ||
          hipEventElapsedTime(&ms, tp.start, tp.stop) != hipSuccess)
        rc = CCO_ERR_HIP;
      m->timed_launches[k] += 1;
      m->timed_ms[k] += ms;
      (void)hipEventDestroy(tp.start);
      (void)hipEventDestroy(tp.stop);
    }
    m->pending[k].clear();
    if (launches) launches[k] = m->timed_launches[k];
    if (total_ms) total_ms[k] = m->timed_ms[k];
    m->timed_launches[k] = 0;
    m->timed_ms[k] = 0.0;
  }
  return rc;
}

}  // extern "C"
