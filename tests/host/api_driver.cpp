// Drives the host side of the C ABI (planner, table check, argument checks)
// over many random descriptions; built with the address and undefined-
// behaviour sanitizers against hip_stubs.cpp, so any out-of-bounds access or
// undefined operation in that code aborts the run.  Prints "ok" at the end.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "mla.h"

extern int g_decode_launches, g_merge_launches, g_combine_launches, g_prepare_launches,
    g_project_launches;
extern std::vector<int64_t> g_expect_local;

#define CHECK(c)                                                    \
  do {                                                              \
    if (!(c)) {                                                     \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                     \
    }                                                               \
  } while (0)

namespace {

// 256-byte aligned host scratch standing in for device buffers (never read
// or written by the stubs).
struct Buf {
  std::vector<unsigned char> raw;
  void* p;
  explicit Buf(size_t n) : raw(n + 512) {
    p = raw.data() + ((256 - (reinterpret_cast<uintptr_t>(raw.data()) & 255)) & 255);
  }
};

int64_t local_len(int64_t L, int W, int r) {
  const int64_t n = (L - r + W - 1) / W;
  return n > 0 ? n : 0;
}

}  // namespace

int main() {
  std::mt19937_64 rng(12345);
  auto uni = [&](int64_t lo, int64_t hi) {
    return std::uniform_int_distribution<int64_t>(lo, hi)(rng);
  };
  const int page_sizes[] = {1, 3, 16, 32, 64, 128};
  const int cu_counts[] = {8, 80, 256, 304};
  Buf dummy(1 << 16);
  int plans = 0;
  for (int it = 0; it < 600; ++it) {
    mla_decode_desc d{};
    d.batch = (int)uni(1, 40);
    d.q_len = (int)uni(1, 8);
    d.num_heads = (int)(it % 3 == 0 ? uni(1, 300) : (it % 3 == 1 ? 96 : 128));
    d.kv_lora_rank = 512;
    d.rope_dim = 64;
    d.page_size = page_sizes[uni(0, 5)];
    d.kv_dtype = (int)uni(0, 3);
    d.dcp_size = it % 4 == 0 ? (int)uni(2, 8) : 1;
    d.dcp_rank = (int)uni(0, d.dcp_size - 1);
    d.num_cus = cu_counts[uni(0, 3)];
    d.force_splits = it % 5 == 0 ? (int)uni(1, 9) : 0;
    std::vector<int32_t> lens(d.batch);
    const int64_t cap = it % 7 == 0 ? 400000 : (it % 2 ? 5000 : 300);
    for (auto& L : lens) L = (int32_t)uni(d.q_len, cap);
    const size_t cap_bytes = mla_plan_max_bytes(&d);
    CHECK(cap_bytes > 0);
    std::vector<unsigned char> plan_raw(cap_bytes + 16);
    void* plan =
        plan_raw.data() + ((16 - (reinterpret_cast<uintptr_t>(plan_raw.data()) & 15)) & 15);
    size_t plan_bytes = 0, ws_bytes = 0;
    // Too small a plan buffer is rejected without writing past it.
    CHECK(mla_decode_plan(&d, lens.data(), plan, cap_bytes / 2, &plan_bytes, &ws_bytes) ==
          MLA_ERR_WORKSPACE_TOO_SMALL || cap_bytes / 2 >= cap_bytes);
    CHECK(mla_decode_plan(&d, lens.data(), plan, cap_bytes, &plan_bytes, &ws_bytes) == MLA_OK);
    CHECK(plan_bytes <= cap_bytes);
    ++plans;
    // A decode call with the host blob as the "device" plan: the stub walks it.
    g_expect_local.assign(d.batch, 0);
    int64_t max_local = 1;
    for (int b = 0; b < d.batch; ++b) {
      g_expect_local[b] = local_len(lens[b], d.dcp_size, d.dcp_rank);
      if (g_expect_local[b] > max_local) max_local = g_expect_local[b];
    }
    Buf ws(ws_bytes + 256);
    const int before = g_decode_launches;
    CHECK(mla_decode(plan, plan, dummy.p, dummy.p, dummy.p,
                     static_cast<const float*>(dummy.p), 1 << 20,
                     static_cast<const int32_t*>(dummy.p), max_local,
                     static_cast<const int32_t*>(dummy.p), 0.07f, ws.p, ws_bytes,
                     static_cast<float*>(dummy.p), static_cast<float*>(dummy.p),
                     nullptr) == MLA_OK);
    CHECK(g_decode_launches == before + 1);
    // Argument errors: nothing is launched.
    if (ws_bytes > 0)
      CHECK(mla_decode(plan, plan, dummy.p, dummy.p, dummy.p, static_cast<const float*>(dummy.p),
                       1 << 20, static_cast<const int32_t*>(dummy.p), max_local,
                       static_cast<const int32_t*>(dummy.p), 0.07f, ws.p, ws_bytes - 1,
                       static_cast<float*>(dummy.p), static_cast<float*>(dummy.p),
                       nullptr) == MLA_ERR_WORKSPACE_TOO_SMALL);
    CHECK(mla_decode(plan, plan, dummy.p, dummy.p, dummy.p, static_cast<const float*>(dummy.p),
                     1 << 20, static_cast<const int32_t*>(dummy.p), max_local - 1 > 0 ?
                     max_local - 1 : 0, static_cast<const int32_t*>(dummy.p), 0.07f, ws.p,
                     ws_bytes, static_cast<float*>(dummy.p), static_cast<float*>(dummy.p),
                     nullptr) == MLA_ERR_INVALID_ARG || max_local <= 1);
    CHECK(mla_decode(plan, plan, static_cast<unsigned char*>(dummy.p) + 4, dummy.p, dummy.p,
                     static_cast<const float*>(dummy.p), 1 << 20,
                     static_cast<const int32_t*>(dummy.p), max_local,
                     static_cast<const int32_t*>(dummy.p), 0.07f, ws.p, ws_bytes,
                     static_cast<float*>(dummy.p), static_cast<float*>(dummy.p),
                     nullptr) == MLA_ERR_INVALID_ARG);
    CHECK(g_decode_launches == before + 1);

    // The table check on a paged table built for these lengths, then broken.
    if (it % 4 == 0 && max_local < 20000) {
      const int ps = d.page_size;
      std::vector<int32_t> table((size_t)d.batch * max_local, -1);
      int64_t next_page = 1;
      for (int b = 0; b < d.batch; ++b)
        for (int64_t j = 0; j < g_expect_local[b]; ++j) {
          if (j % ps == 0) ++next_page;
          table[(size_t)b * max_local + j] = (int32_t)(next_page * ps + j % ps);
        }
      const int64_t slots = (next_page + 1) * ps;
      int64_t bb = 7, bj = 7;
      CHECK(mla_check_table(&d, lens.data(), table.data(), max_local, slots, &bb, &bj) == MLA_OK);
      CHECK(bb == 7 && bj == 7);
      const int b = (int)uni(0, d.batch - 1);
      if (g_expect_local[b] > 1) {
        const int64_t j = uni(1, g_expect_local[b] - 1);
        table[(size_t)b * max_local + j] = (int32_t)slots;  // past the pool
        CHECK(mla_check_table(&d, lens.data(), table.data(), max_local, slots, &bb, &bj) ==
              MLA_ERR_INVALID_ARG);
        CHECK(bb == b && bj == j);
      }
    }
  }
  // Invalid descriptions and null arguments.
  mla_decode_desc bad{};
  bad.batch = 1; bad.q_len = 1; bad.num_heads = 1; bad.kv_lora_rank = 512; bad.rope_dim = 32;
  bad.page_size = 64; bad.dcp_size = 1; bad.num_cus = 8;
  CHECK(mla_plan_max_bytes(&bad) == 0);
  CHECK(mla_plan_max_bytes(nullptr) == 0);
  size_t pb = 0, wb = 0;
  int32_t one = 1;
  CHECK(mla_decode_plan(&bad, &one, dummy.p, 1 << 16, &pb, &wb) == MLA_ERR_UNSUPPORTED);
  CHECK(mla_check_table(nullptr, &one, &one, 1, 1, nullptr, nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_lse_combine(nullptr, nullptr, 2, 10, nullptr, nullptr, nullptr) ==
        MLA_ERR_INVALID_ARG);
  CHECK(mla_lse_combine(static_cast<const float*>(dummy.p), static_cast<const float*>(dummy.p), 0,
                        10, static_cast<float*>(dummy.p), static_cast<float*>(dummy.p),
                        nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_lse_combine(static_cast<const float*>(dummy.p), static_cast<const float*>(dummy.p), 3,
                        10, static_cast<float*>(dummy.p), static_cast<float*>(dummy.p),
                        nullptr) == MLA_OK);
  CHECK(g_combine_launches == 1);
  CHECK(mla_prepare(4, 0, 1, dummy.p, dummy.p, dummy.p, dummy.p, dummy.p,
                    static_cast<const int32_t*>(dummy.p), static_cast<const float*>(dummy.p), 8,
                    static_cast<const int32_t*>(dummy.p), dummy.p,
                    static_cast<unsigned char*>(dummy.p) + 256, dummy.p,
                    static_cast<float*>(dummy.p), 16, nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(mla_lse_combine_project(static_cast<const float*>(dummy.p),
                                static_cast<const float*>(dummy.p), 0, 4, 4, dummy.p, dummy.p,
                                nullptr, nullptr) == MLA_ERR_INVALID_ARG);
  CHECK(std::strcmp(mla_status_string(MLA_ERR_HIP), "HIP runtime error") == 0);
  std::printf("plans %d decode launches %d\nok\n", plans, g_decode_launches);
  return 0;
}
