// Stand-ins for the device side of libtv (launchers, launch planning, the
// static scratch), so that the C ABI layer (tv_api.cpp) can be built and
// exercised on the host alone, under AddressSanitizer and
// UndefinedBehaviorSanitizer. Each records that it was reached and what it
// was given; none touches the pointers it receives.
#include "launch_stubs.h"

namespace stub {
Record last;
int calls = 0;
static void hit(const char* name, int B, int n_max, int elem_bytes, size_t ws_bytes, const void* ws) {
  ++calls;
  last = Record{name, B, n_max, elem_bytes, ws_bytes, ws};
}
}  // namespace stub

namespace tv {

hipError_t launch_v_layout(const void*, void*, long n_blocks, int D, int elem_bytes, bool to_rows, hipStream_t) {
  stub::hit(to_rows ? "v_layout_rows" : "v_layout_blocked", static_cast<int>(n_blocks), D, elem_bytes, 0, nullptr);
  return hipSuccess;
}
hipError_t launch_build_tree(const int32_t*, const int32_t*, int B, int n_max, uint64_t*, int32_t*, int32_t*,
                             hipStream_t) {
  stub::hit("build_tree", B, n_max, 0, 0, nullptr);
  return hipSuccess;
}
hipError_t launch_accept(const int32_t*, const int32_t*, const int32_t*, const uint64_t*, const int32_t*,
                         const int32_t*, const int32_t*, int B, int n_max, int32_t*, int32_t*, int32_t*, int32_t*,
                         hipStream_t) {
  stub::hit("accept", B, n_max, 0, 0, nullptr);
  return hipSuccess;
}
hipError_t launch_accept_typical(const int32_t*, const int32_t*, const float*, const float*, float, float,
                                 const int32_t*, const uint64_t*, const int32_t*, const int32_t*, const int32_t*,
                                 int B, int n_max, int32_t*, int32_t*, int32_t*, int32_t*, hipStream_t) {
  stub::hit("accept_typical", B, n_max, 0, 0, nullptr);
  return hipSuccess;
}
hipError_t launch_eagle2_tree(const float*, const int32_t*, const int32_t*, int B, int, int, int, int n_max,
                              int32_t*, int32_t*, float*, int32_t*, hipStream_t) {
  stub::hit("eagle2_tree", B, n_max, 0, 0, nullptr);
  return hipSuccess;
}
hipError_t launch_speculative_sample(const void*, const void*, int elem_bytes, int, const int32_t*, const float*,
                                     const float*, int B, int L, float*, float*, int32_t*, int32_t*, float* stats,
                                     hipStream_t) {
  stub::hit("speculative_sample", B, L, elem_bytes, 0, stats);
  return hipSuccess;
}
hipError_t launch_typical_stats(const void*, int elem_bytes, int, const int32_t*, const int32_t*, const int32_t*,
                                const int32_t*, int B, int n_max, float*, float*, int32_t*, hipStream_t) {
  stub::hit("typical_stats", B, n_max, elem_bytes, 0, nullptr);
  return hipSuccess;
}
hipError_t launch_accept_commit(const int32_t*, const int32_t*, const int32_t*, const uint64_t*, const int32_t*,
                                const int32_t*, const int32_t*, int B, int n_max, int32_t*, int32_t*, int32_t*,
                                int32_t*, void*, void*, int, int, int, int elem_bytes, const int32_t*, int32_t*,
                                const tv_paged_kv* pk, hipStream_t) {
  stub::hit("accept_commit", B, n_max, elem_bytes, 0, nullptr);
  (void)pk;
  return hipSuccess;
}
hipError_t launch_commit(void*, void*, int B, int, int, int, int elem_bytes, const int32_t*, const int32_t*,
                         const int32_t*, int n_max, int32_t*, const tv_paged_kv* pk, hipStream_t) {
  stub::hit(pk ? "commit_paged" : "commit", B, n_max, elem_bytes, 0, nullptr);
  return hipSuccess;
}
// a plan whose workspace grows with the shapes like the real one (two
// splits' 16-bit partials plus their row statistics, past a 16 KiB head)
AttnPlan plan_attention_bf16(const tv_attn_args* a) {
  AttnPlan p{};
  p.waves = 4;
  p.qt = 2;
  const int rows = a->Hq / a->Hkv * a->n_max;
  p.row_blocks = (rows + 255) / 256;
  p.splits = 2;
  p.rows_pad = p.row_blocks * 256;
  p.fused = false;
  p.workspace_bytes = size_t(16384) + size_t(p.splits) * a->B * a->Hkv * p.rows_pad * (size_t(a->D) * 2 + 8);
  return p;
}
hipError_t launch_attention_bf16(const tv_attn_args* a, const AttnPlan&, const tv_paged_kv* pk, const int32_t* parents,
                                 hipStream_t) {
  stub::hit(pk ? (parents ? "attention_bf16_paged_build" : "attention_bf16_paged")
               : parents ? "attention_bf16_build" : "attention_bf16",
            a->B, a->n_max, 2, a->workspace_bytes, a->workspace);
  return hipSuccess;
}
hipError_t launch_attention_f32(const tv_attn_args* a, hipStream_t) {
  stub::hit("attention_f32", a->B, a->n_max, 4, a->workspace_bytes, a->workspace);
  return hipSuccess;
}
static char g_scratch[64];
hipError_t scratch_workspace(void** ptr) {
  *ptr = g_scratch;
  return hipSuccess;
}

}  // namespace tv
