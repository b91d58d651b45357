// The C ABI's host checks, run on the host alone under AddressSanitizer and
// UndefinedBehaviorSanitizer (tv_api.cpp linked with the stand-ins of
// launch_stubs.cpp): every rejection test_abi.py makes through ctypes, plus
// the accepted calls, which must reach the matching launcher with the
// arguments they were given. Prints "ok <checks>" or the failing checks.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>

#include "launch_stubs.h"
#include "tv.h"

namespace {

int checks = 0, failures = 0;

void expect(int line, int got, int want) {
  ++checks;
  if (got != want) {
    ++failures;
    std::printf("FAIL line %d: status %d, expected %d\n", line, got, want);
  }
}
#define EXPECT(call, want) expect(__LINE__, static_cast<int>(call), static_cast<int>(want))

// the call must have reached launcher `name` (and nothing else since `before`)
void reached(int line, int before, const char* name) {
  ++checks;
  if (stub::calls != before + 1 || std::strcmp(stub::last.name, name) != 0) {
    ++failures;
    std::printf("FAIL line %d: expected one call of %s, got %d calls (last %s)\n", line, name,
                stub::calls - before, stub::calls > before ? stub::last.name : "none");
  }
}
#define REACHED(before, name) reached(__LINE__, before, name)

// never dereferenced: the stand-ins do not touch pointers
void* const F = reinterpret_cast<void*>(0x1000);
int32_t* const I = static_cast<int32_t*>(F);
uint64_t* const U = static_cast<uint64_t*>(F);
float* const FL = static_cast<float*>(F);

tv_attn_args attn(int B = 8, int n_max = 60, int Hq = 32, int Hkv = 8, int D = 128, int cap = 4160,
                  int dtype = TV_BF16) {
  tv_attn_args a;
  std::memset(&a, 0, sizeof(a));
  a.q = a.k_new = a.v_new = F;
  a.k_cache = a.v_cache = F;
  a.prefix_len = a.n_nodes = I;
  a.anc = U;
  a.depth = a.err = I;
  a.out = F;
  a.B = B;
  a.n_max = n_max;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.cap = cap;
  a.dtype = dtype;
  a.rope_theta = 10000.0f;
  return a;
}

void build_tree_accept_commit() {
  EXPECT(tv_build_tree(I, I, -1, 5, U, I, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_build_tree(I, I, 1, 0, U, I, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_build_tree(I, I, 1, 65, U, I, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_build_tree(nullptr, I, 1, 5, U, I, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_build_tree(nullptr, nullptr, 0, 5, nullptr, nullptr, nullptr, nullptr), TV_OK);
  int c = stub::calls;
  EXPECT(tv_build_tree(I, I, 3, 64, U, I, I, nullptr), TV_OK);
  REACHED(c, "build_tree");

  EXPECT(tv_accept(I, I, I, U, I, I, nullptr, 1, 70, I, I, I, nullptr, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_accept(I, I, I, U, I, I, nullptr, 1, 5, nullptr, I, I, nullptr, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_accept(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 5, nullptr, nullptr, nullptr,
                   nullptr, nullptr),
         TV_OK);
  c = stub::calls;
  EXPECT(tv_accept(I, I, I, U, I, I, nullptr, 2, 5, I, I, I, nullptr, nullptr), TV_OK);
  REACHED(c, "accept");

  // commit: Hkv, cap (>= n_max, multiple of 64), D, dtype, pointers
  EXPECT(tv_commit(F, F, 1, 0, 10, 128, TV_BF16, I, I, I, 5, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_commit(F, F, 1, 2, 4, 128, TV_BF16, I, I, I, 5, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_commit(F, F, 1, 2, 100, 128, TV_BF16, I, I, I, 5, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_commit(F, F, 1, 2, 64, 96, TV_BF16, I, I, I, 5, I, nullptr), TV_ERR_UNSUPPORTED);
  EXPECT(tv_commit(F, F, 1, 2, 64, 128, 7, I, I, I, 5, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_commit(nullptr, F, 1, 2, 64, 128, TV_BF16, I, I, I, 5, I, nullptr), TV_ERR_INVALID_ARG);
  c = stub::calls;
  EXPECT(tv_commit(F, F, 4, 2, 128, 64, TV_F32, I, I, I, 5, I, nullptr), TV_OK);
  REACHED(c, "commit");
  EXPECT(stub::last.elem_bytes, 4);

  auto ac = [](int B, int n_max, int Hkv, int cap, int D, int dtype, void* k, int32_t* plen_out) {
    return tv_accept_commit(I, I, I, U, I, I, nullptr, B, n_max, I, I, I, nullptr, k, F, Hkv, cap, D, dtype, I,
                            plen_out, nullptr);
  };
  EXPECT(ac(-1, 5, 8, 128, 128, TV_BF16, F, I), TV_ERR_INVALID_ARG);
  EXPECT(ac(1, 0, 8, 128, 128, TV_BF16, F, I), TV_ERR_INVALID_ARG);
  EXPECT(ac(1, 65, 8, 128, 128, TV_BF16, F, I), TV_ERR_INVALID_ARG);
  EXPECT(ac(1, 5, 0, 128, 128, TV_BF16, F, I), TV_ERR_INVALID_ARG);
  EXPECT(ac(1, 5, 8, 100, 128, TV_BF16, F, I), TV_ERR_INVALID_ARG);
  EXPECT(ac(1, 5, 8, 4, 128, TV_BF16, F, I), TV_ERR_INVALID_ARG);
  EXPECT(ac(1, 5, 8, 128, 128, 7, F, I), TV_ERR_INVALID_ARG);
  EXPECT(ac(1, 5, 8, 128, 96, TV_BF16, F, I), TV_ERR_UNSUPPORTED);
  EXPECT(ac(1, 5, 8, 128, 128, TV_BF16, nullptr, I), TV_ERR_INVALID_ARG);
  EXPECT(ac(1, 5, 8, 128, 128, TV_BF16, F, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(ac(0, 5, 8, 128, 128, TV_BF16, nullptr, I), TV_OK);
  c = stub::calls;
  EXPECT(ac(8, 60, 8, 4160, 128, TV_BF16, F, I), TV_OK);
  REACHED(c, "accept_commit");
  EXPECT(stub::last.elem_bytes, 2);
}

void typical() {
  const float nan = std::numeric_limits<float>::quiet_NaN();
  auto typ = [](int B, int n_max, int V, int dtype, float eps, float delta, const void* logits, float* ent) {
    return tv_accept_typical(logits, dtype, V, I, I, U, I, I, nullptr, B, n_max, eps, delta, ent, FL, I, I, I, I,
                             nullptr, nullptr);
  };
  EXPECT(typ(-1, 5, 32000, TV_BF16, 0.09f, 0.3f, F, FL), TV_ERR_INVALID_ARG);
  EXPECT(typ(70000, 5, 32000, TV_BF16, 0.09f, 0.3f, F, FL), TV_ERR_INVALID_ARG);
  EXPECT(typ(1, 0, 32000, TV_BF16, 0.09f, 0.3f, F, FL), TV_ERR_INVALID_ARG);
  EXPECT(typ(1, 65, 32000, TV_BF16, 0.09f, 0.3f, F, FL), TV_ERR_INVALID_ARG);
  EXPECT(typ(1, 5, 0, TV_BF16, 0.09f, 0.3f, F, FL), TV_ERR_INVALID_ARG);
  EXPECT(typ(1, 5, 32000, 3, 0.09f, 0.3f, F, FL), TV_ERR_INVALID_ARG);
  EXPECT(typ(1, 5, 32000, TV_BF16, nan, 0.3f, F, FL), TV_ERR_INVALID_ARG);
  EXPECT(typ(1, 5, 32000, TV_BF16, 0.09f, nan, F, FL), TV_ERR_INVALID_ARG);
  EXPECT(typ(1, 5, 32000, TV_BF16, 0.09f, 0.3f, nullptr, FL), TV_ERR_INVALID_ARG);
  EXPECT(typ(1, 5, 32000, TV_BF16, 0.09f, 0.3f, F, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(typ(0, 5, 32000, TV_BF16, 0.09f, 0.3f, nullptr, nullptr), TV_OK);
  const int c = stub::calls;
  EXPECT(typ(8, 60, 32000, TV_F32, 0.09f, 0.3f, F, FL), TV_OK);
  ++checks;
  if (stub::calls != c + 2 || std::strcmp(stub::last.name, "accept_typical") != 0) {
    ++failures;
    std::printf("FAIL typical: expected the statistics and the scan launchers\n");
  }
}

void attention() {
  EXPECT(tv_tree_attention(nullptr, nullptr), TV_ERR_INVALID_ARG);
  tv_attn_args a = attn(8, 60, 30);
  EXPECT(tv_tree_attention(&a, nullptr), TV_ERR_INVALID_ARG);   // Hq % Hkv
  a = attn(8, 65);
  EXPECT(tv_tree_attention(&a, nullptr), TV_ERR_INVALID_ARG);
  a = attn(8, 60, 32, 8, 128, 10);
  EXPECT(tv_tree_attention(&a, nullptr), TV_ERR_INVALID_ARG);
  a = attn(8, 60, 32, 8, 128, 4156);
  EXPECT(tv_tree_attention(&a, nullptr), TV_ERR_INVALID_ARG);
  a = attn(8, 60, 32, 8, 96);
  EXPECT(tv_tree_attention(&a, nullptr), TV_ERR_UNSUPPORTED);
  a = attn(8, 60, 32, 8, 64);   // bf16 at head dim 64: the vector-ALU kernel, no workspace
  EXPECT(tv_tree_attention_workspace_size(&a), 0);
  {
    const int c0 = stub::calls;
    EXPECT(tv_tree_attention(&a, nullptr), TV_OK);
    REACHED(c0, "attention_f32");
  }
  a = attn(8, 60, 32, 8, 96, 4160, TV_F32);
  EXPECT(tv_tree_attention(&a, nullptr), TV_ERR_UNSUPPORTED);
  a = attn(8, 60, 32, 8, 128, 4160, 9);
  EXPECT(tv_tree_attention(&a, nullptr), TV_ERR_INVALID_ARG);
  a = attn(1, 60, 8192, 1);   // group above the bf16 kernel's bound
  EXPECT(tv_tree_attention(&a, nullptr), TV_ERR_UNSUPPORTED);
  a = attn();
  a.q = nullptr;
  EXPECT(tv_tree_attention(&a, nullptr), TV_ERR_INVALID_ARG);
  a = attn(0);
  EXPECT(tv_tree_attention(&a, nullptr), TV_OK);
  a = attn();
  const size_t need = tv_tree_attention_workspace_size(&a);
  EXPECT(need > 0, 1);
  a.workspace = F;
  a.workspace_bytes = need - 1;
  EXPECT(tv_tree_attention(&a, nullptr), TV_ERR_INVALID_ARG);
  a.workspace_bytes = need;
  int c = stub::calls;
  EXPECT(tv_tree_attention(&a, nullptr), TV_OK);
  REACHED(c, "attention_bf16");
  a = attn(8, 60, 32, 8, 128, 4160, TV_F32);
  EXPECT(tv_tree_attention_workspace_size(&a), 0);
  c = stub::calls;
  EXPECT(tv_tree_attention(&a, nullptr), TV_OK);
  REACHED(c, "attention_f32");
  a = attn(8, 60, 30);
  EXPECT(tv_tree_attention_workspace_size(&a), 0);
  EXPECT(tv_tree_attention_workspace_size(nullptr), 0);

  // the tree built inside the attention: the attention's checks plus the
  // parents and the two tree outputs; fp32 takes the two launches
  EXPECT(tv_tree_attention_from_parents(nullptr, I, U, I, nullptr), TV_ERR_INVALID_ARG);
  a = attn();
  a.workspace = F;
  a.workspace_bytes = need;
  EXPECT(tv_tree_attention_from_parents(&a, nullptr, U, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_tree_attention_from_parents(&a, I, nullptr, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_tree_attention_from_parents(&a, I, U, nullptr, nullptr), TV_ERR_INVALID_ARG);
  a.workspace_bytes = need - 1;
  EXPECT(tv_tree_attention_from_parents(&a, I, U, I, nullptr), TV_ERR_INVALID_ARG);
  a.workspace_bytes = need;
  a.anc = nullptr;   // (not read)
  a.depth = nullptr;
  c = stub::calls;
  EXPECT(tv_tree_attention_from_parents(&a, I, U, I, nullptr), TV_OK);
  REACHED(c, "attention_bf16_build");
  a = attn(8, 60, 32, 8, 128, 4160, TV_F32);
  c = stub::calls;
  EXPECT(tv_tree_attention_from_parents(&a, I, U, I, nullptr), TV_OK);
  ++checks;
  if (stub::calls != c + 2 || std::strcmp(stub::last.name, "attention_f32") != 0) {
    ++failures;
    std::printf("FAIL from_parents fp32: expected build_tree then attention_f32\n");
  }
  a = attn(0);
  EXPECT(tv_tree_attention_from_parents(&a, nullptr, nullptr, nullptr, nullptr), TV_OK);

  // the allocation-free entry point: same checks, its own scratch, a size limit
  EXPECT(tv_tree_attention_noalloc(nullptr, nullptr), TV_ERR_INVALID_ARG);
  a = attn(8, 0);
  EXPECT(tv_tree_attention_noalloc(&a, nullptr), TV_ERR_INVALID_ARG);
  a = attn();
  a.out = nullptr;
  EXPECT(tv_tree_attention_noalloc(&a, nullptr), TV_ERR_INVALID_ARG);
  a = attn(32, 64, 64, 8, 128, 4096);
  EXPECT(tv_tree_attention_workspace_size(&a) > (size_t(48) << 20), 1);
  EXPECT(tv_tree_attention_noalloc(&a, nullptr), TV_ERR_SCRATCH);
  a = attn();
  c = stub::calls;
  EXPECT(tv_tree_attention_noalloc(&a, nullptr), TV_OK);
  REACHED(c, "attention_bf16");
  EXPECT(stub::last.ws != nullptr && stub::last.ws_bytes == (size_t(48) << 20), 1);

  // paged
  auto pk = [](int max_pages, int num_pages, const int32_t* table) {
    tv_paged_kv p;
    p.block_table = table;
    p.max_pages = max_pages;
    p.num_pages = num_pages;
    return p;
  };
  tv_attn_args ok = attn(8, 60, 32, 8, 128, 65 * 64);
  ok.workspace = F;
  ok.workspace_bytes = size_t(1) << 40;
  tv_paged_kv p = pk(65, 100, I);
  EXPECT(tv_tree_attention_paged(&ok, nullptr, nullptr), TV_ERR_INVALID_ARG);
  p = pk(65, 100, nullptr);
  EXPECT(tv_tree_attention_paged(&ok, &p, nullptr), TV_ERR_INVALID_ARG);
  p = pk(0, 100, I);
  EXPECT(tv_tree_attention_paged(&ok, &p, nullptr), TV_ERR_INVALID_ARG);
  p = pk(65, 0, I);
  EXPECT(tv_tree_attention_paged(&ok, &p, nullptr), TV_ERR_INVALID_ARG);
  p = pk(65, 100, I);
  a = attn(8, 60, 32, 8, 128, 64 * 64);
  EXPECT(tv_tree_attention_paged(&a, &p, nullptr), TV_ERR_INVALID_ARG);
  a = attn(8, 60, 32, 8, 128, 300 * 64);
  tv_paged_kv p300 = pk(300, 100, I);
  EXPECT(tv_tree_attention_paged(&a, &p300, nullptr), TV_ERR_UNSUPPORTED);
  a = attn(8, 60, 32, 8, 64, 65 * 64, TV_F32);
  EXPECT(tv_tree_attention_paged(&a, &p, nullptr), TV_ERR_UNSUPPORTED);
  a = attn(0, 60, 32, 8, 128, 65 * 64);
  EXPECT(tv_tree_attention_paged(&a, &p, nullptr), TV_OK);
  c = stub::calls;
  EXPECT(tv_tree_attention_paged(&ok, &p, nullptr), TV_OK);
  REACHED(c, "attention_bf16_paged");
  EXPECT(tv_commit_paged(F, F, nullptr, 1, 2, 128, TV_BF16, I, I, I, 5, I, nullptr), TV_ERR_INVALID_ARG);
  tv_paged_kv pn = pk(65, 100, nullptr);
  EXPECT(tv_commit_paged(F, F, &pn, 1, 2, 128, TV_BF16, I, I, I, 5, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_commit_paged(F, F, &p, 1, 2, 96, TV_BF16, I, I, I, 5, I, nullptr), TV_ERR_UNSUPPORTED);
  EXPECT(tv_commit_paged(nullptr, F, &p, 1, 2, 128, TV_BF16, I, I, I, 5, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_commit_paged(nullptr, nullptr, &p, 0, 2, 128, TV_BF16, nullptr, nullptr, nullptr, 5, nullptr, nullptr),
         TV_OK);
  c = stub::calls;
  EXPECT(tv_commit_paged(F, F, &p, 2, 2, 128, TV_BF16, I, I, I, 5, I, nullptr), TV_OK);
  REACHED(c, "commit_paged");

  // the paged fused calls: the checks of their separate calls
  EXPECT(tv_tree_attention_paged_from_parents(&ok, nullptr, I, U, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_tree_attention_paged_from_parents(&ok, &pn, I, U, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_tree_attention_paged_from_parents(&ok, &p, nullptr, U, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_tree_attention_paged_from_parents(&ok, &p, I, nullptr, I, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(tv_tree_attention_paged_from_parents(&ok, &p, I, U, nullptr, nullptr), TV_ERR_INVALID_ARG);
  a = attn(8, 60, 32, 8, 128, 300 * 64);
  EXPECT(tv_tree_attention_paged_from_parents(&a, &p300, I, U, I, nullptr), TV_ERR_UNSUPPORTED);
  a = attn(8, 60, 32, 8, 64, 65 * 64, TV_F32);
  EXPECT(tv_tree_attention_paged_from_parents(&a, &p, I, U, I, nullptr), TV_ERR_UNSUPPORTED);
  a = attn(0, 60, 32, 8, 128, 65 * 64);
  EXPECT(tv_tree_attention_paged_from_parents(&a, &p, nullptr, nullptr, nullptr, nullptr), TV_OK);
  c = stub::calls;
  EXPECT(tv_tree_attention_paged_from_parents(&ok, &p, I, U, I, nullptr), TV_OK);
  REACHED(c, "attention_bf16_paged_build");
  auto acp = [](const tv_paged_kv* pp, int B, int n_max, int D, int dtype, void* k) {
    return tv_accept_commit_paged(I, I, I, U, I, I, nullptr, B, n_max, I, I, I, nullptr, k, F, pp, 8, D, dtype, I, I,
                                  nullptr);
  };
  EXPECT(acp(nullptr, 1, 5, 128, TV_BF16, F), TV_ERR_INVALID_ARG);
  EXPECT(acp(&pn, 1, 5, 128, TV_BF16, F), TV_ERR_INVALID_ARG);
  EXPECT(acp(&p, 1, 65, 128, TV_BF16, F), TV_ERR_INVALID_ARG);
  EXPECT(acp(&p, 1, 5, 96, TV_BF16, F), TV_ERR_UNSUPPORTED);
  EXPECT(acp(&p300, 1, 5, 128, TV_BF16, F), TV_ERR_UNSUPPORTED);
  EXPECT(acp(&p, 1, 5, 128, 7, F), TV_ERR_INVALID_ARG);
  EXPECT(acp(&p, 1, 5, 128, TV_BF16, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(acp(&p, 0, 5, 128, TV_BF16, nullptr), TV_OK);
  c = stub::calls;
  EXPECT(acp(&p, 8, 60, 128, TV_BF16, F), TV_OK);
  REACHED(c, "accept_commit");
}

void drafting_and_sampling() {
  auto e2 = [](int B, int S, int K, int M, int n, const float* conf) {
    return tv_eagle2_tree(conf, I, I, B, S, K, M, n, I, I, FL, I, nullptr);
  };
  EXPECT(e2(-1, 6, 8, 8, 60, FL), TV_ERR_INVALID_ARG);
  EXPECT(e2(2, 0, 8, 8, 60, FL), TV_ERR_INVALID_ARG);
  EXPECT(e2(2, 6, 0, 8, 60, FL), TV_ERR_INVALID_ARG);
  EXPECT(e2(2, 6, 8, 0, 60, FL), TV_ERR_INVALID_ARG);
  EXPECT(e2(2, 6, 8, 8, 0, FL), TV_ERR_INVALID_ARG);
  EXPECT(e2(2, 6, 8, 8, 65, FL), TV_ERR_INVALID_ARG);
  EXPECT(e2(2, 7, 8, 10, 60, FL), TV_ERR_UNSUPPORTED);   // 560 proposals
  EXPECT(e2(2, 6, 8, 8, 60, nullptr), TV_ERR_INVALID_ARG);
  EXPECT(e2(0, 6, 8, 8, 60, nullptr), TV_OK);
  int c = stub::calls;
  EXPECT(e2(2, 6, 8, 8, 60, FL), TV_OK);
  REACHED(c, "eagle2_tree");

  const size_t ws = tv_speculative_sample_workspace_size(8, 5);
  EXPECT(ws == size_t(8) * 11 * 2 * 4, 1);
  EXPECT(tv_speculative_sample_workspace_size(0, 5), 0);
  EXPECT(tv_speculative_sample_workspace_size(8, 65), 0);
  auto ss = [](int B, int L, int V, int dtype, const void* p, size_t wsb) {
    return tv_speculative_sample(p, F, dtype, V, I, FL, FL, B, L, FL, FL, I, I, F, wsb, nullptr);
  };
  EXPECT(ss(-1, 5, 32000, TV_BF16, F, ws), TV_ERR_INVALID_ARG);
  EXPECT(ss(8, 0, 32000, TV_BF16, F, ws), TV_ERR_INVALID_ARG);
  EXPECT(ss(8, 65, 32000, TV_BF16, F, ws), TV_ERR_INVALID_ARG);
  EXPECT(ss(8, 5, 0, TV_BF16, F, ws), TV_ERR_INVALID_ARG);
  EXPECT(ss(8, 5, 32000, 9, F, ws), TV_ERR_INVALID_ARG);
  EXPECT(ss(8, 5, 32000, TV_BF16, nullptr, ws), TV_ERR_INVALID_ARG);
  EXPECT(ss(8, 5, 32000, TV_BF16, F, ws - 1), TV_ERR_INVALID_ARG);
  EXPECT(ss(0, 5, 32000, TV_BF16, nullptr, ws), TV_OK);
  c = stub::calls;
  EXPECT(ss(8, 5, 32000, TV_BF16, F, ws), TV_OK);
  REACHED(c, "speculative_sample");
}

void layout() {
  // addresses only: the checks are arithmetic on them, the stub touches nothing
  void* a = reinterpret_cast<void*>(uintptr_t{0x10000});
  void* b = reinterpret_cast<void*>(uintptr_t{0x40000000});
  auto lay = [](const void* s, void* d, int64_t n, int cap, int D, int dtype, int to_rows) {
    return tv_v_cache_layout(s, d, n, cap, D, dtype, to_rows, nullptr);
  };
  EXPECT(lay(a, b, -1, 128, 128, TV_BF16, 0), TV_ERR_INVALID_ARG);
  EXPECT(lay(a, b, 16, 0, 128, TV_BF16, 0), TV_ERR_INVALID_ARG);
  EXPECT(lay(a, b, 16, 100, 128, TV_BF16, 0), TV_ERR_INVALID_ARG);
  EXPECT(lay(a, b, 16, 128, 128, TV_BF16, 2), TV_ERR_INVALID_ARG);
  EXPECT(lay(a, b, 16, 128, 128, 7, 0), TV_ERR_INVALID_ARG);
  EXPECT(lay(a, b, 16, 128, 96, TV_BF16, 0), TV_ERR_UNSUPPORTED);
  EXPECT(lay(a, b, int64_t{1} << 31, 64, 128, TV_BF16, 0), TV_ERR_UNSUPPORTED);
  EXPECT(lay(a, b, int64_t{1} << 62, 128, 128, TV_BF16, 0), TV_ERR_UNSUPPORTED);   // n * cap/64 overflows
  EXPECT(lay(nullptr, b, 16, 128, 128, TV_BF16, 0), TV_ERR_INVALID_ARG);
  EXPECT(lay(static_cast<char*>(a) + 8, b, 16, 128, 128, TV_BF16, 0), TV_ERR_INVALID_ARG);
  EXPECT(lay(a, a, 16, 128, 128, TV_BF16, 0), TV_ERR_INVALID_ARG);
  EXPECT(lay(a, static_cast<char*>(a) + 0x7fff0, 16, 128, 128, TV_BF16, 0), TV_ERR_INVALID_ARG);
  EXPECT(lay(nullptr, nullptr, 0, 128, 128, TV_BF16, 0), TV_OK);
  int c = stub::calls;
  EXPECT(lay(a, static_cast<char*>(a) + 0x80000, 16, 128, 128, TV_BF16, 0), TV_OK);   // adjacent, no overlap
  REACHED(c, "v_layout_blocked");
  EXPECT(stub::last.B, 32);
  EXPECT(stub::last.n_max, 128);
  c = stub::calls;
  EXPECT(lay(a, b, 100, 64, 64, TV_F32, 1), TV_OK);
  REACHED(c, "v_layout_rows");
  EXPECT(stub::last.elem_bytes, 4);
}

void strings() {
  for (int s = TV_OK; s <= TV_ERR_SCRATCH; ++s) {
    const char* t = tv_status_string(static_cast<tv_status>(s));
    ++checks;
    if (t == nullptr || std::strlen(t) == 0) {
      ++failures;
      std::printf("FAIL status string %d\n", s);
    }
  }
  ++checks;
  if (std::strncmp(tv_version(), "tv ", 3) != 0) {
    ++failures;
    std::printf("FAIL version\n");
  }
}

}  // namespace

int main() {
  build_tree_accept_commit();
  typical();
  attention();
  drafting_and_sampling();
  layout();
  strings();
  if (failures) {
    std::printf("failures %d of %d checks\n", failures, checks);
    return 1;
  }
  std::printf("ok %d\n", checks);
  return 0;
}
