// Host-only driver for the HIP-free argument validator, built with g++ and
// address/undefined-behaviour sanitizers by tests/test_validate_host.py.
// Every call below must return the stated status; nothing touches HIP.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "twnorm.h"
#include "twnorm_validate.hpp"

static int failures = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    tw_status got_ = (call);                                                            \
    if (got_ != (want)) {                                                               \
      std::printf("line %d: %s -> %d, want %d (%s)\n", __LINE__, #call, (int)got_,      \
                  (int)(want), twv::last_error());                                      \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

int main() {
  const uintptr_t base = uintptr_t(1) << 40;
  auto P = [&](uintptr_t mb) { return reinterpret_cast<const void*>(base + (mb << 20)); };
  const void* parts[2] = {P(0), P(64)};
  const void* res = P(128);
  const void* w = P(192);
  const void* out = P(256);
  const void* rout = P(320);
  // valid
  EXPECT(twv::check_fused(parts, 2, 4, 64, TW_BF16, res, w, 1e-5f, out, rout, 0), TW_OK);
  EXPECT(twv::check_fused(parts, 2, 4, 64, TW_BF16, res, w, 1e-5f, out, res, 0), TW_OK);
  // invalid arguments
  EXPECT(twv::check_fused(nullptr, 2, 4, 64, TW_BF16, res, w, 1e-5f, out, rout, 0), TW_ERR_INVALID_ARG);
  EXPECT(twv::check_fused(parts, 0, 4, 64, TW_BF16, res, w, 1e-5f, out, rout, 0), TW_ERR_INVALID_ARG);
  EXPECT(twv::check_fused(parts, 2, -1, 64, TW_BF16, res, w, 1e-5f, out, rout, 0), TW_ERR_INVALID_ARG);
  EXPECT(twv::check_fused(parts, 2, 4, 0, TW_BF16, res, w, 1e-5f, out, rout, 0), TW_ERR_INVALID_ARG);
  EXPECT(twv::check_fused(parts, 2, 4, 64, TW_BF16, res, w, std::nanf(""), out, rout, 0), TW_ERR_INVALID_ARG);
  EXPECT(twv::check_fused(parts, 2, 4, 64, TW_BF16, res, w, -1.0f, out, rout, 0), TW_ERR_INVALID_ARG);
  EXPECT(twv::check_fused(parts, 2, 4, 64, (tw_dtype)9, res, w, 1e-5f, out, rout, 0), TW_ERR_INVALID_ARG);
  EXPECT(twv::check_fused(parts, 2, INT64_MAX / 2, 64, TW_BF16, res, w, 1e-5f, out, rout, 0), TW_ERR_INVALID_ARG);
  EXPECT(twv::check_fused(parts, 2, 4, INT64_MAX / 4, TW_BF16, res, w, 1e-5f, out, rout, 0), TW_ERR_INVALID_ARG);
  // unsupported
  EXPECT(twv::check_fused(parts, 2, 4, 12, TW_BF16, res, w, 1e-5f, out, rout, 0), TW_ERR_UNSUPPORTED);
  EXPECT(twv::check_fused(parts, 2, 4, 64, TW_BF16, P(128) /*aligned*/, w, 1e-5f,
                          reinterpret_cast<const char*>(out) + 8, rout, 0), TW_ERR_UNSUPPORTED);
  // aliasing
  EXPECT(twv::check_fused(parts, 2, 4, 64, TW_BF16, res, w, 1e-5f, parts[1], rout, 0), TW_ERR_ALIAS);
  EXPECT(twv::check_fused(parts, 2, 4, 64, TW_BF16, res, w, 1e-5f, out,
                          reinterpret_cast<const char*>(res) + 16, 0), TW_ERR_ALIAS);
  // gather variant
  const void* ag[2] = {P(400), P(464)};
  EXPECT(twv::check_fused_allgather(parts, 2, 4, 64, TW_BF16, res, w, 1e-5f, ag, 2, 4, 8, rout, 0), TW_OK);
  EXPECT(twv::check_fused_allgather(parts, 2, 4, 64, TW_BF16, res, w, 1e-5f, ag, 2, 5, 8, rout, 0), TW_ERR_INVALID_ARG);
  EXPECT(twv::check_fused_allgather(parts, 2, 4, 64, TW_BF16, res, w, 1e-5f, ag, 0, 0, 8, rout, 0), TW_ERR_INVALID_ARG);
  // traffic-pattern measurement aid
  const void* msrc[3] = {P(512), P(576), P(512)};   // sources may coincide
  const void* mdst[2] = {P(640), P(704)};
  EXPECT(twv::check_mix(msrc, 3, mdst, 2, 64 << 20, 0), TW_OK);
  const void* madj[2] = {P(640), P(641)};            // adjacent 1 MiB ranges
  EXPECT(twv::check_mix(msrc, 3, madj, 2, 1 << 20, 0), TW_OK);
  EXPECT(twv::check_mix(msrc, 3, madj, 2, (1 << 20) + 16, 0), TW_ERR_ALIAS);
  const void* mbad[1] = {P(520)};                    // inside srcs[0]'s 64 MiB
  EXPECT(twv::check_mix(msrc, 3, mbad, 1, 64 << 20, 0), TW_ERR_ALIAS);
  EXPECT(twv::check_mix(msrc, 0, mdst, 2, 1024, 0), TW_ERR_INVALID_ARG);
  EXPECT(twv::check_mix(msrc, 18, mdst, 2, 1024, 0), TW_ERR_INVALID_ARG);
  EXPECT(twv::check_mix(msrc, 3, mdst, 17, 1024, 0), TW_ERR_INVALID_ARG);
  EXPECT(twv::check_mix(msrc, 3, mdst, 2, 1000, 0), TW_ERR_UNSUPPORTED);
  EXPECT(twv::check_mix(nullptr, 3, mdst, 2, 1024, 0), TW_ERR_INVALID_ARG);
  // shape choice covers every width it accepts, for every n; a CU-limited
  // call (8 of 256 CUs) uses at most 10 wavefronts and refuses wider rows
  for (int n = 1; n <= 16; ++n)
    for (int64_t h = 8; h <= 65536; h += 8) {
      twv::Shape s{};
      const bool limited = (h & 128) != 0;
      const tw_status st = twv::choose_shape(TW_BF16, h, n, (h & 64) ? 1 : 4096, limited ? 8 : 256, 256, &s);
      if (limited && h > 40960) {
        if (st != TW_ERR_UNSUPPORTED) { ++failures; break; }
        continue;
      }
      if (st != TW_OK) { ++failures; break; }
      const int64_t chunks = h * 2 / 16;
      const int max_waves = limited ? 10 : 16;
      if (s.k == 0 ? (s.team < chunks || s.team > 32) : ((int64_t)s.waves * 64 * s.k < chunks || s.waves > max_waves)) {
        std::printf("bad shape for h=%lld n=%d\n", (long long)h, n);
        ++failures;
        break;
      }
    }
  std::printf("%s (%d failures)\n", failures ? "FAIL" : "OK", failures);
  return failures ? 1 : 0;
}
