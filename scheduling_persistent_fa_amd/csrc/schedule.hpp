// Host-side DASH schedule generator, validator and DAG simulator.
// Plain C++17, no HIP dependency.
//
// A step is one (query head, query tile qi, key/value tile kj) pair.  A chain
// is every step of one key/value tile of one key/value group: its query tiles
// in the schedule's walk, and at each query tile the group's g query heads in
// ascending order.  A chain runs contiguously on one workgroup so dK/dV stay
// in registers ("Resumo Técnico: DASH ...", §2.1, restrictions).  Taking the
// heads inside the walk keeps the lock-step spacing of the walk: two chains
// of one gang reach a dQ tile at least g steps apart.
// Each step carries its ordinal: the position of its contribution in the
// accumulation sequence of its dQ tile, which fixes the summation order.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace dash {

// kMaskBand: key/value tile kj is visible from query tile qi when
// -band_l <= kj - qi - (Nk - Nq) <= band_r (a negative extent is unbounded);
// causal is the band (unbounded, 0).
enum : int { kMaskFull = 0, kMaskCausal = 1, kMaskBand = 2 };
enum : int { kSerial = 0, kDescQ = 1, kShift = 2, kSymShift = 3, kAtomic = 4 };

constexpr int32_t kFirstFlag = 1 << 28;
constexpr int32_t kLastFlag = 1 << 29;
constexpr int32_t kOrdMask = (1 << 28) - 1;

struct StepRec {
  int32_t head;      // b * Hq + hq
  int32_t qi;        // query tile
  int32_t kj;        // key/value tile
  int32_t ordflags;  // ordinal | kFirstFlag | kLastFlag
};

struct Schedule {
  int mask = 0, kind = 0, walk = 0;  // walk: the ordering schedule (== kind unless kind is ATOMIC)
  int Nq = 0, Nk = 0;                // query tiles and key/value tiles per sequence
  int g = 1, groups = 1, P = 1;
  bool xcd_local = true;
  int max_gang = 0;                  // 0: natural gang size (N for shift, N/2 for symmetric shift)
  int band_l = -1, band_r = -1;      // kMaskBand extents in tiles (-1: unbounded)
  std::vector<int32_t> offsets;  // P + 1
  std::vector<StepRec> steps;
};

// Returns an empty string on success, else the reason (unsupported combination).
// Nq query tiles, Nk key/value tiles.  The causal mask is aligned at the
// bottom right: query tile qi sees key/value tiles 0 .. qi + Nk - Nq.
std::string build_schedule(int mask, int kind, int Nq, int Nk, int g, int groups, int P, bool xcd_local,
                           int atomic_walk, int max_gang, Schedule* out, int band_l = -1, int band_r = -1);
// Query tiles [*lo, *hi] that see key/value tile kj, and key/value tiles seen
// by query tile qi (empty when *lo > *hi).
void visible_q(const Schedule& s, int kj, int* lo, int* hi);
void visible_k(const Schedule& s, int qi, int* lo, int* hi);
// Empty string if valid, else the first violation found.
std::string validate_schedule(const Schedule& s);
// The deterministic schedule (and gang cap) chosen for a shape; empty string
// on success.  A band mask (extents band_l, band_r in tiles) takes SHIFT where
// the band shift applies (a sliding band: band_r = 0, and Nk = Nq with an
// even band_l or Nk - Nq >= band_l, band_l < Nq), else DESC_Q.
std::string choose_schedule(int mask, int Nq, int Nk, int D, int g, int P, int* kind, int* max_gang,
                            int band_l = -1, int band_r = -1);
// Whether the band shift covers a band (see build_schedule).
bool band_shift_applies(int Nq, int Nk, int band_l, int band_r);
// Unit-cost DAG simulation; returns false on deadlock.  With jitter_seed != 0
// step i of workgroup w costs c * jitter_factor(jitter_seed, w, i) of compute
// (uniform in [0.5, 1.5)); 0 keeps every step at c.
bool simulate_schedule(const Schedule& s, double c, double r, uint64_t jitter_seed, double* makespan,
                       double* total_wait);
double jitter_factor(uint64_t seed, int w, int i);

}  // namespace dash
