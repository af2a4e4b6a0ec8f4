// Host-only stand-ins for the library's kernel launchers, so that the host runtime
// (runtime.cpp) links into a CPU test program built with sanitizers. No GPU is present
// in that program: every launcher returns g_stub_launch (hipErrorNotSupported unless
// the program sets it; with the real HIP runtime and no GPU no call gets this far, the
// runtime's first HIP allocation fails first).
#include "../../looped_ngpt_transformer_amd/csrc/kernels.h"

hipError_t g_stub_launch = hipErrorNotSupported;

namespace dory {
int gemm_pick_splits(int, int, int, int) { return 1; }
hipError_t launch_expand_mxfp8(const uint8_t*, const uint8_t*, int64_t, int64_t, void*, hipStream_t) {
  return g_stub_launch;
}
hipError_t launch_gemm(const GemmArgs&, hipStream_t) { return g_stub_launch; }
hipError_t launch_arrange_frag(const void*, int64_t, int64_t, void*, hipStream_t) { return g_stub_launch; }
hipError_t launch_mfma_rate(int, int, long long*, float*, hipStream_t) { return g_stub_launch; }
hipError_t launch_update(const UpdateArgs&, hipStream_t) { return g_stub_launch; }
hipError_t launch_stage_input(const float*, float*, void*, int, int, int, hipStream_t, const int32_t*, void*) {
  return g_stub_launch;
}
hipError_t launch_scatter_rows(const float*, const int32_t*, int, int, float*, hipStream_t) { return g_stub_launch; }
hipError_t launch_resume_state(const float*, const float*, const int32_t*, int, int, float*, float*, void*, int,
                               hipStream_t) {
  return g_stub_launch;
}
hipError_t launch_rope_kv(const RopeArgs&, hipStream_t) { return g_stub_launch; }
hipError_t launch_rope_kv_tiles(const RopeArgs&, hipStream_t) { return g_stub_launch; }
hipError_t launch_rope_table(const int32_t*, int, const double*, int, size_t, float*, hipStream_t) {
  return g_stub_launch;
}
hipError_t launch_attn_rows(const AttnArgs&, int, int*, hipStream_t) { return g_stub_launch; }
hipError_t launch_attn_prefill(const AttnArgs&, hipStream_t) { return g_stub_launch; }
size_t attn_rows_part_floats(int, int, int, int, int) { return 0; }
hipError_t launch_swiglu(const float*, int, int, int, void*, int, hipStream_t) { return g_stub_launch; }
hipError_t launch_apply_deltas(int32_t*, const int32_t*, int, void*, size_t, hipStream_t) { return g_stub_launch; }
hipError_t launch_fill_kv(const KVLayout&, int, int, int, int, const void*, const void*, hipStream_t) {
  return g_stub_launch;
}
hipError_t launch_quantize_mxfp8(const void*, int, int64_t, int64_t, uint8_t*, uint8_t*, hipStream_t) {
  return g_stub_launch;
}
hipError_t launch_embed(const void*, int, int64_t, int, const int32_t*, int, float*, hipStream_t) {
  return g_stub_launch;
}
hipError_t launch_logit_scale(const float*, int, size_t, float*, int64_t, int, int64_t, const float*, hipStream_t) {
  return g_stub_launch;
}
hipError_t noalloc_scratch(void**) { return hipErrorNotSupported; }
hipError_t launch_sample_top_p(const float*, int64_t, int, int64_t, float, float, const float*, int32_t*, hipStream_t) {
  return g_stub_launch;
}
hipError_t launch_spec_accept(int, int, int64_t, const float*, int64_t, const float*, int64_t, const int32_t*, float,
                              float, const float*, const float*, int32_t*, int32_t*, hipStream_t) {
  return g_stub_launch;
}
hipError_t launch_quantize_nvfp4(const void*, int, int64_t, int64_t, uint8_t*, uint8_t*, float*, hipStream_t) {
  return g_stub_launch;
}
hipError_t launch_expand_nvfp4(const uint8_t*, const uint8_t*, const float*, int64_t, int64_t, void*, hipStream_t) {
  return g_stub_launch;
}
}  // namespace dory
