// Host-side checks of the C ABI, built with the host address and undefined-behaviour
// sanitizers (tests/test_host_sanitize.py compiles api.hip that way and links this
// program against it).  Every call made here is either host-only (describe, workspace
// sizes, status strings) or one that the library must refuse before any launch: the
// pointers are never valid device memory, and the program runs with no GPU visible.
// Exit status 0 when every expectation holds; a sanitizer report aborts the run.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "mbq.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "FAILED line %d: %s\n", line, what);
    ++failures;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// Addresses that are never dereferenced on the host; the library may only test them for
// NULL and alignment.
// A refusal: a negative status other than MBQ_ERR_DEVICE (which only a launch returns).
bool refused(mbq_status st) { return st < 0 && st != MBQ_ERR_DEVICE; }

void* fake(uintptr_t off) { return reinterpret_cast<void*>(uintptr_t(1) << 20 | off); }
float* ffake(uintptr_t off) { return static_cast<float*>(fake(off)); }
int32_t* ifake(uintptr_t off) { return static_cast<int32_t*>(fake(off)); }
uint16_t* hfake(uintptr_t off) { return static_cast<uint16_t*>(fake(off)); }

void describe_grid() {
  const int32_t ns[] = {-1, 0, 1, 15, 16, 17, 18944, 1 << 28, (1 << 28) + 1, INT32_MAX};
  const int32_t ks[] = {-64, 0, 32, 48, 64, 96, 100, 256, 3584, 1 << 28, INT32_MAX};
  const int32_t gs[] = {-32, 0, 16, 32, 64, 96, 128, 256, 512};
  const int32_t ss[] = {-1, 0, 1, 2, 3, 4, 5};
  for (int32_t n : ns)
    for (int32_t k : ks)
      for (int32_t g : gs)
        for (int32_t s : ss) {
          mbq_desc d;
          std::memset(&d, 0xA5, sizeof(d));
          const mbq_status st = mbq_describe(n, k, g, s, &d);
          const bool group_ok = g == 32 || g == 64 || g == 128 || g == 256;
          const bool shape_ok = n >= 1 && n <= (1 << 28) && k >= g && k <= (1 << 28) && g > 0 && k % g == 0;
          if (!group_ok || s < 1 || s > 4) {
            EXPECT(st == MBQ_ERR_UNSUPPORTED);
          } else if (!shape_ok) {
            EXPECT(st == MBQ_ERR_SHAPE);
          } else {
            EXPECT(st == MBQ_OK);
            EXPECT(d.n == n && d.k == k && d.group == g && d.slices == s && d.bits == 2);
            EXPECT(d.row_blocks == (n + 15) / 16 && d.k_tiles == (k + 255) / 256);
            EXPECT(d.groups_padded == d.k_tiles * 256 / g);
            EXPECT(d.params_offset % 256 == 0 && d.slice_stride % 256 == 0);
            EXPECT(d.total_bytes == d.slice_stride * uint64_t(s));
          }
        }
  EXPECT(mbq_describe(16, 256, 64, 1, nullptr) == MBQ_ERR_ARG);
}

void status_strings() {
  for (int s = -10; s <= 2; ++s) EXPECT(mbq_status_str(mbq_status(s)) != nullptr);
  EXPECT(mbq_abi_version() == MBQ_ABI_VERSION);
}

void workspace_queries(const mbq_desc& d) {
  size_t b = 0;
  const int32_t ts[] = {-1, 0, 1, 4, 16, 17, 33, 64, 65, 2048, 1 << 24, (1 << 24) + 1};
  for (int32_t t : ts) {
    for (mbq_dtype x : {MBQ_F32, MBQ_BF16, mbq_dtype(7)}) {
      const mbq_status a = mbq_linear_workspace(&d, t, x, &b);
      EXPECT(a == MBQ_OK || a < 0);
      const mbq_status c = mbq_route_linear_workspace(&d, t, x, &b);
      EXPECT(c == MBQ_OK || c < 0);
      for (int32_t r : {-8, 0, 8, 12, 16, 32, 40}) {
        const mbq_status e = mbq_linear_lowrank_workspace(&d, t, x, r, &b);
        EXPECT(e == MBQ_OK || e < 0);
      }
    }
    const mbq_status p = mbq_route_prepare_workspace(&d, t, &b);
    EXPECT(p == MBQ_OK || p < 0);
    for (int32_t h : {-1, 0, 64, 256, 4096}) {
      const mbq_status m = mbq_route_mlp_workspace(t, d.k, h, &b);
      EXPECT(m == MBQ_OK || m < 0);
    }
  }
  EXPECT(mbq_linear_workspace(&d, 16, MBQ_BF16, nullptr) == MBQ_ERR_ARG);
  EXPECT(mbq_linear_workspace(nullptr, 16, MBQ_BF16, &b) == MBQ_ERR_ARG);
}

void refused_calls(const mbq_desc& d) {
  mbq_desc bad = d;
  bad.total_bytes += 256;
  mbq_desc old = d;
  old.abi = MBQ_ABI_VERSION - 1;
  void* blob = fake(0);
  // packs: missing, misaligned, inconsistent
  EXPECT(mbq_pack(nullptr, fake(0), MBQ_F32, blob, nullptr, nullptr) == MBQ_ERR_ARG);
  EXPECT(mbq_pack(&d, nullptr, MBQ_F32, blob, nullptr, nullptr) == MBQ_ERR_ARG);
  EXPECT(mbq_pack(&d, fake(0), MBQ_F32, fake(16), nullptr, nullptr) == MBQ_ERR_ARG);
  EXPECT(mbq_pack(&d, fake(2), MBQ_F32, blob, nullptr, nullptr) == MBQ_ERR_ARG);
  EXPECT(refused(mbq_pack(&bad, fake(0), MBQ_F32, blob, nullptr, nullptr)));
  EXPECT(mbq_pack(&old, fake(0), MBQ_F32, blob, nullptr, nullptr) == MBQ_ERR_UNSUPPORTED);
  EXPECT(refused(mbq_pack_bitplane(&d, fake(0), mbq_dtype(9), blob, nullptr, nullptr)));
  EXPECT(refused(mbq_pack_rows(&d, -16, 16, fake(0), MBQ_F32, blob, nullptr, nullptr)));
  EXPECT(refused(mbq_pack_rows(&d, 3, 16, fake(0), MBQ_F32, blob, nullptr, nullptr)));
  EXPECT(refused(mbq_pack_rows(&d, 0, d.n + 16, fake(0), MBQ_F32, blob, nullptr, nullptr)));
  // routing: slices, shapes, pointers
  EXPECT(refused(mbq_route(4, d.k, 0, fake(0), MBQ_F32, ffake(0), ffake(0), ifake(0), ifake(0), ifake(0), nullptr)));
  EXPECT(refused(mbq_route(4, d.k, 5, fake(0), MBQ_F32, ffake(0), ffake(0), ifake(0), ifake(0), ifake(0), nullptr)));
  EXPECT(refused(mbq_route(-1, d.k, 3, fake(0), MBQ_F32, ffake(0), ffake(0), ifake(0), ifake(0), ifake(0), nullptr)));
  EXPECT(refused(mbq_route(4, d.k, 3, fake(0), MBQ_F32, nullptr, ffake(0), ifake(0), ifake(0), ifake(0), nullptr)));
  EXPECT(refused(mbq_route(4, d.k, 3, fake(0), MBQ_F32, ffake(0), nullptr, ifake(0), ifake(0), ifake(0), nullptr)));
  EXPECT(refused(mbq_route(4, d.k, 3, fake(0), MBQ_F32, ffake(0), ffake(0), ifake(0), ifake(0), ifake(2), nullptr)));
  EXPECT(refused(mbq_regroup(4, 0, ifake(0), ifake(0), ifake(0), nullptr)));
  EXPECT(refused(mbq_regroup(4, 3, nullptr, ifake(0), ifake(0), nullptr)));
  EXPECT(refused(mbq_route_mlp(4, d.k, 3, 64, fake(0), MBQ_BF16, hfake(0), ffake(0), ffake(0), ffake(0), -0.5,
                       ffake(0), ifake(0), ifake(0), ifake(0), fake(0), 0, nullptr)));
  EXPECT(refused(mbq_route_mlp(4, d.k, 3, 64, fake(0), MBQ_BF16, hfake(0), ffake(0), ffake(0), ffake(0), 0.5,
                       ffake(0), ifake(0), ifake(0), ifake(0), nullptr, 0, nullptr)));
  // linears: every pointer in turn missing or misaligned, bad dtypes, t out of range
  const mbq_opts bad_opts[] = {{7, 0, 0, 0}, {0, 9, 0, 0}, {0, 0, -1, 0}, {0, 0, 0, 3}};
  for (const mbq_opts& o : bad_opts)
    EXPECT(mbq_linear(&d, blob, 4, fake(0), MBQ_BF16, ifake(0), ifake(0), fake(0), MBQ_BF16, nullptr, 0, &o,
                      nullptr) == MBQ_ERR_ARG);
  for (int which = 0; which < 5; ++which)
    for (uintptr_t mis : {uintptr_t(0), uintptr_t(2)}) {
      const void* ptr[5] = {blob, fake(0), ifake(0), ifake(0), fake(0)};
      if (mis) ptr[which] = static_cast<const char*>(ptr[which]) + mis;
      else ptr[which] = nullptr;
      const mbq_status st = mbq_linear(&d, ptr[0], 4, ptr[1], MBQ_BF16, static_cast<const int32_t*>(ptr[2]),
                                       static_cast<const int32_t*>(ptr[3]), const_cast<void*>(ptr[4]), MBQ_BF16,
                                       nullptr, 0, nullptr, nullptr);
      EXPECT(st == MBQ_ERR_ARG);
      const mbq_status ss = mbq_linear_static(&d, ptr[0], 4, ptr[1], MBQ_BF16, static_cast<const int32_t*>(ptr[2]),
                                              static_cast<const int32_t*>(ptr[3]), const_cast<void*>(ptr[4]),
                                              MBQ_BF16, nullptr, nullptr);
      EXPECT(ss == MBQ_ERR_ARG);
    }
  EXPECT(mbq_linear(&d, blob, -1, fake(0), MBQ_BF16, ifake(0), ifake(0), fake(0), MBQ_BF16, nullptr, 0, nullptr,
                    nullptr) == MBQ_ERR_SHAPE);
  EXPECT(mbq_linear(&d, blob, 4, fake(0), mbq_dtype(5), ifake(0), ifake(0), fake(0), MBQ_BF16, nullptr, 0, nullptr,
                    nullptr) == MBQ_ERR_ARG);
  EXPECT(refused(mbq_linear(&bad, blob, 4, fake(0), MBQ_BF16, ifake(0), ifake(0), fake(0), MBQ_BF16, nullptr, 0, nullptr,
                    nullptr)));
  // a workspace too small for a split-K decode
  size_t need = 0;
  if (mbq_linear_workspace(&d, 16, MBQ_BF16, &need) == MBQ_OK && need > 0)
    EXPECT(mbq_linear(&d, blob, 16, fake(0), MBQ_BF16, ifake(0), ifake(0), fake(0), MBQ_BF16, fake(0), need - 1,
                      nullptr, nullptr) == MBQ_ERR_WORKSPACE);
  // the static entry point refuses sizes beyond its buffer
  if (mbq_linear_workspace(&d, 64, MBQ_BF16, &need) == MBQ_OK && need > MBQ_STATIC_SCRATCH_BYTES)
    EXPECT(mbq_linear_static(&d, blob, 64, fake(0), MBQ_BF16, ifake(0), ifake(0), fake(0), MBQ_BF16, nullptr,
                             nullptr) == MBQ_ERR_WORKSPACE);
  // routed step, prepared step, low-rank
  EXPECT(mbq_route_linear(&d, blob, 16, fake(0), MBQ_BF16, nullptr, ffake(0), ifake(0), ifake(0), ifake(0), fake(0),
                          MBQ_BF16, fake(0), 1 << 30, nullptr, nullptr) == MBQ_ERR_ARG);
  EXPECT(mbq_route_linear(&d, blob, 16, fake(0), MBQ_BF16, ffake(2), ffake(0), ifake(0), ifake(0), ifake(0), fake(0),
                          MBQ_BF16, fake(0), 1 << 30, nullptr, nullptr) == MBQ_ERR_ARG);
  EXPECT(refused(mbq_route_prepare(&d, 16, fake(0), ffake(0), fake(0), 0, nullptr)));
  EXPECT(refused(mbq_route_prepare(&d, 65, fake(0), ffake(0), fake(0), 1 << 30, nullptr)));
  EXPECT(refused(mbq_route_linear_prepared(&d, blob, 16, fake(0), 0, ffake(0), ifake(0), ifake(0), ifake(0), fake(0),
                                   MBQ_BF16, nullptr)));
  for (int32_t r : {0, 12, 40})
    EXPECT(refused(mbq_linear_lowrank(&d, blob, 4, fake(0), MBQ_BF16, ifake(0), ifake(0), hfake(0), hfake(0), r, fake(0),
                              MBQ_BF16, fake(0), 1 << 30, nullptr, nullptr)));
  EXPECT(mbq_linear_lowrank(&d, blob, 4, fake(0), MBQ_BF16, ifake(0), ifake(0), nullptr, hfake(0), 16, fake(0),
                            MBQ_BF16, fake(0), 1 << 30, nullptr, nullptr) == MBQ_ERR_ARG);
}

}  // namespace

int main() {
  describe_grid();
  status_strings();
  const int32_t shapes[][4] = {{18944, 3584, 128, 3}, {11008, 4096, 128, 3}, {200, 640, 32, 4},
                               {17, 768, 256, 1}, {5120, 13824, 128, 3}, {64, 64, 64, 2},
                               {32768, 13824, 128, 3}};   // its split-K workspace at 64 tokens exceeds the static buffer
  for (const auto& s : shapes) {
    mbq_desc d;
    if (mbq_describe(s[0], s[1], s[2], s[3], &d) != MBQ_OK) {
      std::fprintf(stderr, "describe failed for %d %d %d %d\n", s[0], s[1], s[2], s[3]);
      return 2;
    }
    workspace_queries(d);
    refused_calls(d);
  }
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("abi host checks passed\n");
  return 0;
}
