// Exercises the C ABI's host logic (plan creation, workspace layout, table
// generation, argument validation, aliasing checks) under the sanitizers.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "internal.h"
#include "s4dplr.h"
#include "tables.h"

int stub_launch_count();

#define CHECK(c)                                                       \
  do {                                                                 \
    if (!(c)) {                                                        \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                                        \
    }                                                                  \
  } while (0)

// The per-entry table formulas that the no-allocation path evaluates on the
// device (tables.h) reproduce the plan's host-built tables bit for bit.
static int check_table_formulas(const s4dplr_plan* p, const void* ws) {
  std::vector<unsigned char> store(p->tables_bytes + 256, 0);
  unsigned char* w = reinterpret_cast<unsigned char*>(
      (reinterpret_cast<uintptr_t>(store.data()) + 255) & ~uintptr_t(255));
  const s4::TableSpec a = s4::plan_table_spec(p, w);
  for (long g = 0; g < s4::table_entries(a); ++g) s4::table_entry(a, g);
  CHECK(std::memcmp(w, ws, p->tables_bytes) == 0);
  return 0;
}

int main() {
  const int Ls[] = {2, 4, 32, 1024, 2048, 16384, 32768, 65536};
  for (int L : {2, 16, 512, 4096, 32768, 65536})
    for (unsigned rank : {1u, 2u, 4u}) {
      s4dplr_plan* p = nullptr;
      CHECK(s4dplr_plan_create(&p, 2, 8, L, 1, S4DPLR_RANK(rank)) == S4DPLR_OK && p);
      size_t bytes = 0;
      CHECK(s4dplr_plan_workspace_bytes(p, &bytes) == S4DPLR_OK);
      std::vector<unsigned char> store(bytes + 256);
      void* ws = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(store.data()) + 255) & ~uintptr_t(255));
      CHECK(s4dplr_plan_init(p, ws, nullptr) == S4DPLR_OK);
      CHECK(check_table_formulas(p, ws) == 0);
      s4dplr_plan_destroy(p);
    }
  const int Ns[] = {1, 3, 64, 256};
  for (int L : Ls)
    for (int N : Ns)
      for (unsigned flags : {0u, 1u, 3u, 4u}) {
        s4dplr_plan* p = nullptr;
        CHECK(s4dplr_plan_create(&p, 3, N, L, 2, flags) == S4DPLR_OK && p);
        size_t bytes = 0;
        CHECK(s4dplr_plan_workspace_bytes(p, &bytes) == S4DPLR_OK && bytes % 256 == 0);
        // a real host buffer stands in for the workspace (tables are copied in)
        std::vector<unsigned char> store(bytes + 256);
        void* ws = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(store.data()) + 255) & ~uintptr_t(255));
        CHECK(s4dplr_plan_init(p, ws, nullptr) == S4DPLR_OK);
        CHECK(check_table_formulas(p, ws) == 0);
        CHECK(s4dplr_plan_init(p, static_cast<char*>(ws) + 8, nullptr) == S4DPLR_ERR_WORKSPACE);
        // compute entry points reach their launchers; the stubs never
        // dereference these synthetic, widely spaced device-style addresses
        const uintptr_t base = uintptr_t(1) << 40, gap = uintptr_t(1) << 34;
        const float* f = reinterpret_cast<const float*>(base);
        float* u = reinterpret_cast<float*>(base + gap);
        float* y = reinterpret_cast<float*>(base + 2 * gap);
        float* K = reinterpret_cast<float*>(base + 3 * gap);
        const int before = stub_launch_count();
        CHECK(s4dplr_kernel_gen(p, f, f, nullptr, f, f, f, K, ws, nullptr) == S4DPLR_OK);
        CHECK(s4dplr_forward(p, f, f, nullptr, f, f, f, nullptr, u, nullptr, y, ws, nullptr) == S4DPLR_OK);
        CHECK(s4dplr_conv_apply(p, u, y, ws, nullptr) == S4DPLR_OK);
        CHECK(s4dplr_forward_noalloc(p, f, f, nullptr, f, f, f, nullptr, u, K, y, nullptr) == S4DPLR_OK);
        CHECK(s4dplr_forward_noalloc(p, f, f, nullptr, f, f, f, nullptr, u, K, u, nullptr) == S4DPLR_ERR_ALIAS);
        CHECK(s4dplr_forward_noalloc(p, f, f, nullptr, f, f, f, nullptr, nullptr, K, y, nullptr) == S4DPLR_ERR_NULL);
        {
          float* kh = reinterpret_cast<float*>(base + 8 * gap);
          const s4dplr_status want = (flags & S4DPLR_ZOH) ? S4DPLR_ERR_UNSUPPORTED : S4DPLR_OK;
          CHECK(s4dplr_generating_function(p, f, f, nullptr, f, f, f, kh, ws, nullptr) == want);
          CHECK(s4dplr_generating_function(p, f, f, nullptr, f, f, f, nullptr, ws, nullptr) ==
                S4DPLR_ERR_NULL);
          // khat overlapping the workspace or a parameter
          const s4dplr_status alias = (flags & S4DPLR_ZOH) ? S4DPLR_ERR_UNSUPPORTED : S4DPLR_ERR_ALIAS;
          CHECK(s4dplr_generating_function(p, f, f, nullptr, f, f, f, static_cast<float*>(ws), ws,
                                           nullptr) == alias);
          CHECK(s4dplr_generating_function(p, f, f, nullptr, f, f, f, const_cast<float*>(f), ws,
                                           nullptr) == alias);
        }
        CHECK(s4dplr_recurrent_prepare(p, f, f, nullptr, f, f, f, ws, nullptr) == S4DPLR_OK);
        {
          float* g = reinterpret_cast<float*>(base + 4 * gap);
          float* o = reinterpret_cast<float*>(base + 5 * gap);
          CHECK(s4dplr_conv_bwd(p, u, K, nullptr, g, y, o, nullptr, ws, nullptr) == S4DPLR_OK);
          const s4dplr_status want_kg = S4DPLR_OK;
          float* outs = reinterpret_cast<float*>(base + 6 * gap);
          const size_t cb = 2 * 3 * (size_t)N;   // floats of one [H][N] complex output
          CHECK(s4dplr_kernel_gen_bwd(p, f, f, nullptr, f, f, f, K, outs, outs + cb, nullptr,
                                      outs + 2 * cb, outs + 3 * cb, outs + 4 * cb, ws,
                                      nullptr) == want_kg);
        }
        CHECK(s4dplr_recurrent_scan(p, nullptr, u, 7, K, y, ws, nullptr) == S4DPLR_OK);
        CHECK(s4dplr_recurrent_scan(p, nullptr, u, 7, K, u, ws, nullptr) == S4DPLR_ERR_ALIAS);
        if (flags & S4DPLR_BLOCK) {
          float* xo = reinterpret_cast<float*>(base + 7 * gap);
          CHECK(s4dplr_block_forward(p, xo, f, f, f, f, nullptr, f, f, f, nullptr, f, f, xo, ws,
                                     nullptr) == S4DPLR_OK);
        }
        CHECK(stub_launch_count() > before);
        CHECK(s4dplr_forward(p, f, f, nullptr, f, f, f, nullptr, u, nullptr, u, ws, nullptr) == S4DPLR_ERR_ALIAS);
        CHECK(s4dplr_conv_fwd(p, u, K, nullptr, y, nullptr, nullptr) == S4DPLR_ERR_NULL);
        s4dplr_plan_destroy(p);
      }
  // the recurrent scan's work split covers every pole with at most 32 lanes
  // per sequence and 8 poles per lane
  for (int N = 1; N <= 256; ++N)
    for (long rows : {1L, 7L, 64L, 1000L, 8192L, 16384L, 1L << 20}) {
      int ppl = 0, lg = -1;
      s4::recurrent_shape(N, rows, &ppl, &lg);
      CHECK(ppl == 1 || ppl == 2 || ppl == 4 || ppl == 8);
      CHECK(lg >= 0 && lg <= 5);
      CHECK((ppl << lg) >= N);
    }
  {
    // the no-allocation forward rejects plans whose forward scratch exceeds
    // the static array (H = 64, L = 65536, batch = 4: about 241 MiB)
    s4dplr_plan* big = nullptr;
    CHECK(s4dplr_plan_create(&big, 64, 64, 65536, 4, 0) == S4DPLR_OK);
    const uintptr_t base = uintptr_t(1) << 40, gap = uintptr_t(1) << 34;
    const float* f = reinterpret_cast<const float*>(base);
    float* u = reinterpret_cast<float*>(base + gap);
    float* y = reinterpret_cast<float*>(base + 2 * gap);
    CHECK(s4dplr_forward_noalloc(big, f, f, nullptr, f, f, f, nullptr, u, nullptr, y, nullptr) ==
          S4DPLR_ERR_TOO_LARGE);
    s4dplr_plan_destroy(big);
    CHECK(s4dplr_plan_create(&big, 128, 64, 16384, 8, 0) == S4DPLR_OK);
    CHECK(s4dplr_forward_noalloc(big, f, f, nullptr, f, f, f, nullptr, u, nullptr, y, nullptr) ==
          S4DPLR_OK);
    s4dplr_plan_destroy(big);
  }
  {
    // rank-r plans: the forward-side entry points accept them, the recurrent
    // view and the parameter gradients reject them; invalid rank fields
    const uintptr_t base = uintptr_t(1) << 40, gap = uintptr_t(1) << 34;
    const float* f = reinterpret_cast<const float*>(base);
    float* u = reinterpret_cast<float*>(base + gap);
    float* y = reinterpret_cast<float*>(base + 2 * gap);
    float* K = reinterpret_cast<float*>(base + 3 * gap);
    for (int L : {64, 4096, 65536})
      for (int r : {2, 3, 4}) {
        s4dplr_plan* q = nullptr;
        CHECK(s4dplr_plan_create(&q, 3, 16, L, 2, S4DPLR_RANK(r) | S4DPLR_BLOCK) == S4DPLR_OK);
        size_t bytes = 0;
        CHECK(s4dplr_plan_workspace_bytes(q, &bytes) == S4DPLR_OK);
        std::vector<unsigned char> store(bytes + 256);
        void* ws = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(store.data()) + 255) & ~uintptr_t(255));
        CHECK(s4dplr_plan_init(q, ws, nullptr) == S4DPLR_OK);
        CHECK(s4dplr_kernel_gen(q, f, f, nullptr, f, f, f, K, ws, nullptr) == S4DPLR_OK);
        CHECK(s4dplr_forward(q, f, f, f, f, f, f, nullptr, u, K, y, ws, nullptr) == S4DPLR_OK);
        CHECK(s4dplr_forward_noalloc(q, f, f, nullptr, f, f, f, nullptr, u, K, y, nullptr) ==
              S4DPLR_OK);
        CHECK(s4dplr_generating_function(q, f, f, nullptr, f, f, f, K, ws, nullptr) == S4DPLR_OK);
        CHECK(s4dplr_recurrent_prepare(q, f, f, nullptr, f, f, f, ws, nullptr) ==
              S4DPLR_ERR_UNSUPPORTED);
        float* outs = reinterpret_cast<float*>(base + 6 * gap);
        CHECK(s4dplr_kernel_gen_bwd(q, f, f, nullptr, f, f, f, K, outs, nullptr, nullptr, nullptr,
                                    nullptr, nullptr, ws, nullptr) == S4DPLR_ERR_UNSUPPORTED);
        float* xo = reinterpret_cast<float*>(base + 7 * gap);
        CHECK(s4dplr_block_forward(q, xo, f, f, f, f, nullptr, f, f, f, nullptr, f, f, xo, ws,
                                   nullptr) == S4DPLR_OK);
        s4dplr_plan_destroy(q);
      }
    s4dplr_plan* q = nullptr;
    CHECK(s4dplr_plan_create(&q, 3, 16, 64, 2, S4DPLR_RANK(5)) == S4DPLR_ERR_UNSUPPORTED && !q);
    CHECK(s4dplr_plan_create(&q, 3, 16, 64, 2, S4DPLR_RANK(2) | S4DPLR_DIAGONAL) ==
          S4DPLR_ERR_UNSUPPORTED);
    CHECK(s4dplr_plan_create(&q, 3, 16, 64, 2, S4DPLR_RANK(1)) == S4DPLR_OK);
    s4dplr_plan_destroy(q);
  }
  s4dplr_plan* p = nullptr;
  CHECK(s4dplr_plan_create(&p, 1, 1, 3, 1, 0) == S4DPLR_ERR_SHAPE && !p);
  CHECK(s4dplr_plan_create(&p, 1, 1, 4, 1, 8) == S4DPLR_ERR_UNSUPPORTED);
  CHECK(s4dplr_plan_create(&p, 1, 1, 4, 1, S4DPLR_ZOH) == S4DPLR_ERR_UNSUPPORTED);
  CHECK(s4dplr_plan_create(nullptr, 1, 1, 4, 1, 0) == S4DPLR_ERR_NULL);
  for (int s = -1; s < 9; ++s) CHECK(std::strlen(s4dplr_status_string(static_cast<s4dplr_status>(s))) > 0);
  s4dplr_plan_destroy(nullptr);
  std::puts("host sanitizer driver: ok");
  return 0;
}
