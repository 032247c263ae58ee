// Host-only stand-ins for the kernel launchers that api.cpp dispatches to, so
// that the C-ABI layer's validation code can be built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer and driven without a GPU.
// Each launcher records that it was reached and touches no memory; the
// workspace-size queries return fixed non-zero sizes so that every workspace
// check runs.
#include "../../hybrid_linear_memory_amd/csrc/arl2_internal.h"

int g_launches = 0;

namespace {
hipError_t reached() {
  ++g_launches;
  return hipSuccess;
}
size_t sized(const arl2::Dims& d, size_t per_head) { return (size_t)d.B * d.H * per_head; }
}  // namespace

const char* hipGetErrorString(hipError_t) { return "stub"; }

namespace arl2 {

hipError_t generic_feature_map(const Dims&, const void*, const void*, void*, bool, hipStream_t) {
  return reached();
}
hipError_t generic_attention(const Dims&, const void*, const void*, const void*, void*, int64_t,
                             int64_t, hipStream_t) {
  return reached();
}
hipError_t generic_inter_read(const Dims&, const void*, const float*, const void*, void*, void*,
                              hipStream_t) {
  return reached();
}
size_t generic_state_commit_ws_bytes(const Dims& d) { return sized(d, 4096); }
hipError_t generic_state_commit(const Dims&, const void*, const void*, const float*, const float*,
                                const float*, float*, void*, hipStream_t) {
  return reached();
}
hipError_t mfma_feature_maps(const Dims&, const FeatureMapJob*, int, hipStream_t) {
  return reached();
}
hipError_t mfma_feature_map(const Dims&, const void*, const void*, void*, bool, hipStream_t) {
  return reached();
}
hipError_t mfma_attention(const Dims&, const void*, const void*, const void*, void*, int64_t,
                          int64_t, hipStream_t) {
  return reached();
}
hipError_t mfma_attention_lse(const Dims&, const void*, const void*, const void*, void*, float*,
                              hipStream_t) {
  return reached();
}
hipError_t mfma_inter_read(const Dims&, const void*, const float*, const void*, void*, void*,
                           hipStream_t) {
  return reached();
}
size_t mfma_read_ws_bytes(const Dims& d) { return sized(d, 32768); }
hipError_t mfma_read_prepare(const Dims&, const void*, const float*, void*, hipStream_t) {
  return reached();
}
size_t mfma_read_prepared_ws_bytes(const Dims& d) { return sized(d, 8192); }
hipError_t mfma_read_prepared(const Dims&, const void*, const void*, const void*, const void*,
                              void*, void*, void*, void*, size_t, hipStream_t) {
  return reached();
}
hipError_t mfma_clean_pass_prepared(const Dims&, const void*, const void*, const void*,
                                    const void*, const void*, const void*, const void*,
                                    const float*, const float*, const float*, float*, void*, void*,
                                    void*, void*, void*, hipStream_t) {
  return reached();
}
hipError_t generic_read_prepare(const Dims&, const void*, const float*, float*, hipStream_t) {
  return reached();
}
hipError_t mfma_read(const Dims&, const void*, const void*, const void*, const void*,
                     const float*, void*, void*, void*, void*, hipStream_t) {
  return reached();
}
size_t mfma_commit_ws_bytes(const Dims& d) { return sized(d, 65536); }
size_t mfma_clean_commit_ws_bytes(const Dims& d) { return sized(d, 32768); }
hipError_t mfma_commit(const Dims&, const void*, const void*, const void*, const void*,
                       const float*, const float*, const float*, float*, void*, hipStream_t) {
  return reached();
}
size_t mfma_state_commit_ws_bytes(const Dims& d) { return sized(d, 65536); }
hipError_t mfma_state_commit(const Dims&, const void*, const void*, const float*, const float*,
                             const float*, float*, void*, hipStream_t) {
  return reached();
}
size_t token_level_scan_ws_bytes(const Dims& d) { return sized(d, 16384); }
hipError_t token_level_scan(const Dims&, const void*, const void*, const void*, const float*,
                            const float*, const float*, float*, const void*, void*, void*, void*,
                            hipStream_t) {
  return reached();
}
size_t attn_backward_ws_bytes(const Dims& d) { return sized(d, 16384); }
size_t read_backward_ws_bytes(const Dims& d) { return sized(d, 16384); }
size_t commit_backward_ws_bytes(const Dims& d) { return sized(d, 16384); }
hipError_t attn_backward(const Dims&, const void*, const void*, const void*, const void*,
                         const float*, const void*, void*, void*, void*, bool, void*,
                         hipStream_t) {
  return reached();
}
hipError_t read_backward(const Dims&, const void*, const void*, const void*, const void*,
                         const float*, const void*, const float*, const void*, void*, void*,
                         void*, float*, float*, bool, void*, hipStream_t) {
  return reached();
}
hipError_t attn_lse_f32(const Dims&, const void*, const void*, float*, hipStream_t) {
  return reached();
}
hipError_t commit_backward(const Dims&, const void*, const void*, const void*, const void*,
                           const float*, const float*, const float*, const float*, void*, void*,
                           float*, float*, float*, float*, float*, bool, void*, hipStream_t) {
  return reached();
}
hipError_t copy_state(const float*, float*, size_t, hipStream_t) { return reached(); }
size_t noalloc_scratch_bytes() { return (size_t)8 << 20; }
hipError_t noalloc_scratch(void** ptr) {
  static char stand_in[16];
  *ptr = stand_in;                 // never dereferenced by the validation code
  return hipSuccess;
}

}  // namespace arl2
