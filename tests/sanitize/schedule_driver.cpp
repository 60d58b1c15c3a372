// Host-only driver for a sanitizer build (AddressSanitizer + UndefinedBehavior
// Sanitizer, built with g++) of the schedule generator: builds, validates,
// chooses and simulates every mask / schedule / grid / gang cap / band over a
// range of small shapes, plus the workload shapes on 256 workgroups.  Exits
// non-zero if a combination that must build fails, or a built schedule does
// not validate or deadlocks under jitter; the sanitizers abort on any memory
// or undefined-behaviour error.
#include <cstdio>
#include <string>

#include "../../scheduling_persistent_fa_amd/csrc/schedule.hpp"

using namespace dash;

static int g_fail = 0;

static void check(int mask, int kind, int Nq, int Nk, int g, int groups, int P, bool xcd, int walk, int cap,
                  int bl = -1, int br = -1) {
  Schedule s;
  std::string err = build_schedule(mask, kind, Nq, Nk, g, groups, P, xcd, walk, cap, &s, bl, br);
  if (!err.empty()) return;  // unsupported combinations are allowed to be rejected
  std::string v = validate_schedule(s);
  if (!v.empty()) {
    std::printf("invalid: mask %d kind %d Nq %d Nk %d g %d groups %d P %d cap %d band %d %d: %s\n", mask, kind, Nq, Nk,
                g, groups, P, cap, bl, br, v.c_str());
    ++g_fail;
    return;
  }
  double mk = 0, wt = 0;
  for (uint64_t seed : {0ULL, 7ULL, 0xDEADBEEFULL}) {
    if (!simulate_schedule(s, 1.0, 0.5, seed, &mk, &wt)) {
      std::printf("deadlock: mask %d kind %d Nq %d Nk %d seed %llu\n", mask, kind, Nq, Nk, (unsigned long long)seed);
      ++g_fail;
    }
  }
}

int main() {
  long long n = 0;
  for (int Nq = 1; Nq <= 7; ++Nq)
    for (int Nk = 1; Nk <= 9; ++Nk)
      for (int g = 1; g <= 2; ++g)
        for (int P : {1, 3, 8, 13})
          for (int cap : {0, 1, 2, 3})
            for (int kind = 0; kind <= 4; ++kind) {
              for (int mask = 0; mask <= 1; ++mask) {
                check(mask, kind, Nq, Nk, g, 2, P, true, -1, cap);
                check(mask, kind, Nq, Nk, g, 2, P, false, kind == 4 ? 2 : -1, cap);
                ++n;
              }
              for (int bl = -1; bl <= 3; ++bl)
                for (int br = -1; br <= 2; ++br) {
                  check(kMaskBand, kind, Nq, Nk, g, 2, P, true, -1, cap, bl, br);
                  ++n;
                }
            }
  // the workload shapes on 256 workgroups
  check(kMaskCausal, kSymShift, 16, 16, 1, 64, 256, true, -1, 0);
  check(kMaskFull, kShift, 32, 32, 1, 48, 256, true, -1, 0);
  check(kMaskFull, kShift, 128, 128, 1, 16, 256, true, -1, 0);
  check(kMaskCausal, kSymShift, 128, 128, 1, 16, 256, true, -1, 0);
  check(kMaskCausal, kSymShift, 64, 64, 4, 8, 256, true, -1, 0);
  check(kMaskFull, kShift, 32, 128, 1, 16, 256, true, -1, 32);
  check(kMaskBand, kShift, 128, 128, 1, 16, 256, true, -1, 0, 32, 0);
  // the adaptive rule on many shapes
  for (int N = 1; N <= 300; N += 7)
    for (int mask = 0; mask <= 1; ++mask) {
      int kind = 0, cap = 0;
      if (!choose_schedule(mask, N, N + (mask ? 3 : 0), 128, 1, 256, &kind, &cap).empty()) ++g_fail;
    }
  std::printf("%lld combinations, %d failures\n", n, g_fail);
  return g_fail ? 1 : 0;
}
