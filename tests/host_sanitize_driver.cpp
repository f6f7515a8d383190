// Calls the host-side logic of the cco_moe library (argument checks, shape
// limits, window layout, status strings, null-handle paths) for a build of
// csrc/api.cpp with AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_host_sanitizers.py).  The kernel launchers are stubs: without
// a device no call reaches them.  Exit status 0 when every result is the
// documented one.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "cco_moe.h"
#include "../combine_symmetric_memory_amd/csrc/cco_internal.h"

namespace cco {
hipError_t launch_plan_count(const MoeArgs &, const int32_t *, int32_t, int32_t, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_plan_rank(const MoeArgs &, const int32_t *, int32_t, int32_t, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_plan_single(const MoeArgs &, const int32_t *, int32_t, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_dispatch(const MoeArgs &, const uint16_t *, const float *, const int32_t *,
                           int32_t, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_dispatch_fp8(const MoeArgs &, const uint8_t *, const float *, int32_t,
                               const float *, const int32_t *, int32_t, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_combine(const MoeArgs &, uint64_t, const float *, const int32_t *, uint16_t *,
                          int32_t, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_copy_in(const MoeArgs &, int32_t, const uint16_t *, uint64_t, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_expert_gate_up(const MoeArgs &, const uint16_t *, int32_t, int, int32_t,
                                 hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_expert_down(const MoeArgs &, const uint16_t *, int32_t, int, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_fused(const MoeArgs &, const FusedBuffers &, const int32_t *, const uint16_t *,
                        const float *, const uint16_t *, const uint16_t *, uint16_t *, int32_t,
                        int, hipStream_t) {
  return hipErrorInvalidValue;
}
}  // namespace cco

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                                         \
    }                                                                   \
  } while (0)

static cco_moe_shape shape(int T, int H, int K, int E, int I) {
  cco_moe_shape s;
  s.max_tokens = T;
  s.hidden = H;
  s.topk = K;
  s.num_experts = E;
  s.inter = I;
  return s;
}

int main() {
  for (int c = -11; c <= 2; ++c) CHECK(cco_status_string(c) != nullptr);

  // valid shapes: the windows are ordered, aligned and sized as declared
  const cco_moe_shape ok[] = {shape(128, 256, 2, 8, 512), shape(8192, 7168, 8, 256, 2048),
                              shape(4096, 4096, 2, 8, 14336), shape(16384, 7168, 8, 256, 0),
                              shape(1, 64, 1, 4, 0), shape(256, 8, 32, 1024, 0)};
  const int slots[] = {4, 8, 8, 8, 2, 8};
  for (int i = 0; i < 6; ++i) {
    const uint64_t need = cco_moe_required_slot_bytes(&ok[i], slots[i]);
    CHECK(need > 0);
    cco_moe_layout L;
    std::memset(&L, 0xCD, sizeof(L));
    CHECK(cco_moe_layout_of(&ok[i], slots[i], &L) == CCO_OK);
    const int64_t eps = ok[i].num_experts / slots[i];
    const int64_t cap = (int64_t)ok[i].max_tokens * (ok[i].topk < eps ? ok[i].topk : eps);
    CHECK(L.cap == cap);
    CHECK(L.disp_x_bytes == (uint64_t)cap * ok[i].hidden * 2);
    CHECK(L.disp_meta >= L.disp_x + L.disp_x_bytes);
    CHECK(L.disp_meta_bytes == (uint64_t)cap * 12);
    if (ok[i].inter > 0) {
      CHECK(L.hbuf >= L.disp_meta + L.disp_meta_bytes && L.out_tok >= L.hbuf + L.hbuf_bytes);
      CHECK(L.out_tok + L.out_tok_bytes <= need);
    } else {
      CHECK(L.hbuf_bytes == 0 && L.out_tok_bytes == 0);
      CHECK(L.disp_meta + L.disp_meta_bytes <= need);
    }
    CHECK(L.disp_x % 256 == 0 && L.disp_meta % 256 == 0);
  }

  // invalid shapes: zero bytes and CCO_ERR_INVALID_ARG, nothing else touched
  const cco_moe_shape bad[] = {
      shape(128, 250, 2, 8, 512),       // H % 8
      shape(128, 256, 0, 8, 512),       // K < 1
      shape(128, 256, 33, 64, 512),     // K > 32
      shape(128, 256, 2, 6, 512),       // E % S (4 slots)
      shape(128, 256, 2, 2048, 512),    // E > 1024
      shape(128, 256, 2, 8, 500),       // I % 128
      shape(128, 200, 2, 8, 512),       // H % 256 with experts
      shape(128, 65536, 2, 8, 16384),   // gate+up weights >= 2 GiB
      shape(-1, 256, 2, 8, 512),        // negative T
      shape(1 << 30, 256, 8, 8, 0),     // T * K past int32
  };
  for (const cco_moe_shape &s : bad) {
    CHECK(cco_moe_required_slot_bytes(&s, 4) == 0);
    cco_moe_layout L;
    CHECK(cco_moe_layout_of(&s, 4, &L) == CCO_ERR_INVALID_ARG);
  }
  CHECK(cco_moe_required_slot_bytes(nullptr, 4) == 0);
  CHECK(cco_moe_required_slot_bytes(&ok[0], 0) == 0);
  CHECK(cco_moe_layout_of(&ok[0], 4, nullptr) == CCO_ERR_INVALID_ARG);

  // heap arguments checked before the runtime
  cco_sym_heap *h = reinterpret_cast<cco_sym_heap *>(0x1);
  CHECK(cco_sym_heap_create(0, 0, 1 << 20, &h) == CCO_ERR_INVALID_ARG);
  CHECK(cco_sym_heap_create(0, 4, 0, &h) == CCO_ERR_INVALID_ARG);
  CHECK(cco_sym_heap_create(-1, 4, 1 << 20, &h) == CCO_ERR_INVALID_ARG);
  CHECK(cco_sym_heap_create(0, 4, 1 << 20, nullptr) == CCO_ERR_INVALID_ARG);
  CHECK(cco_sym_heap_create(0, 1 << 30, UINT64_MAX / 2, &h) == CCO_ERR_INVALID_ARG);
  CHECK(cco_sym_heap_destroy(nullptr) == CCO_OK);
  CHECK(cco_sym_heap_slot_ptr(nullptr, 0, 0) == nullptr);
  CHECK(cco_sym_heap_info(nullptr, nullptr, nullptr, nullptr, nullptr) == CCO_ERR_INVALID_ARG);

  // every entry point refuses a null object
  cco_moe *m = nullptr;
  cco_moe_layout L;
  cco_moe_routing R;
  CHECK(cco_moe_create(nullptr, &ok[0], &m) == CCO_ERR_INVALID_ARG);
  CHECK(cco_moe_get_layout(nullptr, &L) == CCO_ERR_INVALID_ARG);
  CHECK(cco_moe_get_routing(nullptr, &R) == CCO_ERR_INVALID_ARG);
  CHECK(cco_moe_plan(nullptr, nullptr, 0, nullptr) == CCO_ERR_INVALID_ARG);
  CHECK(cco_moe_dispatch(nullptr, nullptr, nullptr, 0, nullptr) == CCO_ERR_INVALID_ARG);
  CHECK(cco_moe_dispatch_fp8(nullptr, nullptr, nullptr, 0, nullptr, 0, nullptr) ==
        CCO_ERR_INVALID_ARG);
  CHECK(cco_moe_expert(nullptr, nullptr, nullptr, nullptr) == CCO_ERR_INVALID_ARG);
  CHECK(cco_moe_combine(nullptr, nullptr, nullptr, nullptr, 0, nullptr) == CCO_ERR_INVALID_ARG);
  CHECK(cco_moe_status(nullptr, nullptr, nullptr, nullptr) == CCO_ERR_INVALID_ARG);
  CHECK(cco_moe_stage_in_sdma(nullptr, 0, nullptr, 0, nullptr) == CCO_ERR_INVALID_ARG);
  CHECK(cco_moe_fused(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) ==
        CCO_ERR_INVALID_ARG);
  CHECK(cco_moe_dispatch_view(nullptr, 0) == nullptr);
  CHECK(cco_moe_combine_in_view(nullptr, 0) == nullptr);
  CHECK(cco_moe_set_timing(nullptr, 1) == CCO_ERR_INVALID_ARG);
  CHECK(cco_moe_timing_summary(nullptr, nullptr, nullptr) == CCO_ERR_INVALID_ARG);
  std::printf("host sanitizer driver ok\n");
  return 0;
}
