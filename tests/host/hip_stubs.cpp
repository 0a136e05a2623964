// Host-only stand-ins for the kernel launchers and the two HIP runtime calls
// of mla_api.cpp, so that the planner and the argument checks can be built
// and run under the address and undefined-behaviour sanitizers without a GPU.
//
// The decode launcher receives the plan through DecodeArgs::plan; the driver
// passes the host blob there, so this stub walks it and checks every unit
// against the header: each workgroup's unit range, each unit's request, row
// group, token range and partial slot, and that the units of every
// (request, row group) cover the request's local range exactly once.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kernels.h"
#include "kernels_step.h"
#include "plan_layout.h"

int g_decode_launches = 0, g_merge_launches = 0, g_combine_launches = 0;
int g_prepare_launches = 0, g_project_launches = 0;
// Local length of every request of the decode call being checked (set by the driver).
std::vector<int64_t> g_expect_local;

#define REQUIRE(c)                                                      \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "plan check failed: %s (line %d)\n", #c, __LINE__); \
      std::abort();                                                     \
    }                                                                   \
  } while (0)

namespace mla {

hipError_t launch_decode(int kv, bool paged, int grid, const DecodeArgs& a, hipStream_t) {
  ++g_decode_launches;
  const uint8_t* blob = a.plan;
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(blob);
  REQUIRE(h->magic == kPlanMagic && h->kv_dtype == kv && grid == h->num_wgs);
  REQUIRE(paged == (h->page_size % kTile == 0));
  const int32_t* wgb = reinterpret_cast<const int32_t*>(blob + h->off_wg);
  const Unit* units = reinterpret_cast<const Unit*>(blob + h->off_units);
  const ReqParts* reqs = reinterpret_cast<const ReqParts*>(blob + h->off_reqs);
  REQUIRE(wgb[0] == 0 && wgb[h->num_wgs] == h->num_units);
  for (int x = 0; x < h->num_wgs; ++x) REQUIRE(wgb[x] <= wgb[x + 1]);
  const int B = h->batch, G = h->row_groups;
  std::vector<std::vector<std::pair<int, int>>> cover((size_t)B * G);
  std::vector<int> part_seen(h->num_parts > 0 ? h->num_parts : 1, 0);
  for (int u = 0; u < h->num_units; ++u) {
    const Unit& un = units[u];
    REQUIRE(un.b >= 0 && un.b < B && un.g >= 0 && un.g < G);
    REQUIRE(un.j0 >= 0 && un.j0 <= un.j1 && un.j1 <= h->max_local);
    if (un.part >= 0) {
      REQUIRE(un.part < h->num_parts && reqs[un.b].num_parts > 1);
      REQUIRE(un.part >= reqs[un.b].first_part &&
              un.part < reqs[un.b].first_part + reqs[un.b].num_parts);
      part_seen[un.part]++;
    } else {
      REQUIRE(reqs[un.b].num_parts == 1);
    }
    cover[(size_t)un.b * G + un.g].push_back({un.j0, un.j1});
  }
  for (int p = 0; p < h->num_parts; ++p) REQUIRE(part_seen[p] == G);
  REQUIRE((int)g_expect_local.size() == B);
  for (int b = 0; b < B; ++b) {
    const int64_t n = g_expect_local[b];
    REQUIRE(n <= h->max_local);
    for (int g = 0; g < G; ++g) {
      const auto& v = cover[(size_t)b * G + g];
      REQUIRE(!v.empty());
      std::vector<char> seen((size_t)n + 1, 0);
      int64_t covered = 0;
      for (const auto& r : v) {
        REQUIRE(r.second <= n);
        for (int j = r.first; j < r.second; ++j) {
          REQUIRE(!seen[j]);
          seen[j] = 1;
          ++covered;
        }
      }
      REQUIRE(covered == n);
    }
  }
  return hipSuccess;
}

hipError_t launch_merge_split(const SplitReq* split, int num_split_reqs, int rows, int max_parts,
                              const uint16_t*, const float*, const float*, float*, float*,
                              hipStream_t) {
  ++g_merge_launches;
  REQUIRE(num_split_reqs > 0 && rows > 0 && max_parts > 1);
  // The driver passes the host plan as the device plan, so the records can
  // be read here: every one is split, and max_parts is their largest count.
  int largest = 0;
  for (int i = 0; i < num_split_reqs; ++i) {
    REQUIRE(split[i].b >= 0 && split[i].first_part >= 0 && split[i].pad == 0);
    REQUIRE(split[i].num_parts > 1 && split[i].num_parts <= max_parts);
    largest = split[i].num_parts > largest ? split[i].num_parts : largest;
  }
  REQUIRE(largest == max_parts);
  return hipSuccess;
}

hipError_t launch_lse_combine(const float*, const float*, int nparts, int64_t rows, float*,
                              float*, hipStream_t) {
  ++g_combine_launches;
  REQUIRE(nparts >= 1 && rows > 0);
  return hipSuccess;
}

hipError_t launch_prepare(const PrepareArgs& a, hipStream_t) {
  ++g_prepare_launches;
  REQUIRE(a.T >= 0 && a.H >= 1);
  return hipSuccess;
}

hipError_t launch_combine_project(const float*, const float*, int nparts, int T, int H,
                                  const uint16_t*, uint16_t*, float*, hipStream_t) {
  ++g_project_launches;
  REQUIRE(nparts >= 1 && T >= 0 && H >= 1);
  return hipSuccess;
}

hipError_t noalloc_scratch(void** ptr) {
  // A fake, never dereferenced device address (the stub decode launch only
  // walks the plan).
  *ptr = reinterpret_cast<void*>(uintptr_t(1) << 40);
  return hipSuccess;
}

}  // namespace mla

extern "C" hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}

extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_t* p, int) {
  std::memset(p, 0, sizeof(*p));
  p->multiProcessorCount = 256;
  return hipSuccess;
}
