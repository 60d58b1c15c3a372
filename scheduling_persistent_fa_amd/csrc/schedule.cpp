// Host-side DASH schedule generator, validator and DAG simulator.
//
// Schedules ("Resumo Técnico: DASH ...", §2.2; "DASH如何革新LLM确定性训练", §2.3):
//  SERIAL    each chain walks query tiles ascending; a dQ tile accumulates
//            key/value tiles in ascending order (the serialized baseline).
//  DESC_Q    same accumulation order, query tiles walked descending (§2.2.A).
//  SHIFT     full mask: a gang of N workgroups per key/value group; the
//            workgroup keeping key/value tile p visits query tiles
//            p, p+1, ..., N-1, 0, ..., p-1, so the t-th contribution to every
//            dQ tile arrives at step t and no two workgroups meet (§2.2.B).
//            With Nq query and Nk key/value tiles: min(Nq, Nk) members (more
//            would meet on a query tile); the member holding kv tile i visits
//            query tiles (i + t) mod Nq, and with Nk > Nq member p holds kv
//            tiles p, p + Nq, ... in turn.
//  SYM_SHIFT causal mask: a gang of N/2 workgroups; member p keeps tile p
//            through a dense rectangle phase (query tiles N/2..N-1, shifted)
//            and its own triangle part, then tile N-1-p through the folded
//            triangle, N+1 steps per member (§2.2.B, symmetric shift).
//            With Nk > Nq (bottom-right causal) that runs on the square of kv
//            tiles R..Nk-1, R = Nk - Nq; member p then takes the dense kv
//            tiles p, p + N/2, ... < R, each visiting query tiles
//            (tile + t) mod Nq.
// Gang schedules order each dQ tile's contributions by lock-step time (the
// step's position in its workgroup's list for that group), ties by kj.  A
// gang may be capped below its natural size (N, or N/2): its members then
// take their units in rounds, which keeps a gang on one chiplet.
#include "schedule.hpp"

#include <algorithm>
#include <queue>
#include <utility>

namespace dash {

namespace {
// Tile-distance extents of a mask: (dl, dr), -1 unbounded.
void extents(const Schedule& s, int* dl, int* dr) {
  if (s.mask == kMaskCausal) {
    *dl = -1;
    *dr = 0;
  } else if (s.mask == kMaskBand) {
    *dl = s.band_l;
    *dr = s.band_r;
  } else {
    *dl = -1;
    *dr = -1;
  }
}
}  // namespace

void visible_q(const Schedule& s, int kj, int* lo, int* hi) {
  int dl, dr;
  extents(s, &dl, &dr);
  const int off = s.Nk - s.Nq;
  *lo = dr < 0 ? 0 : std::max(0, kj - off - dr);
  *hi = dl < 0 ? s.Nq - 1 : std::min(s.Nq - 1, kj - off + dl);
}

void visible_k(const Schedule& s, int qi, int* lo, int* hi) {
  int dl, dr;
  extents(s, &dl, &dr);
  const int off = s.Nk - s.Nq;
  *lo = dl < 0 ? 0 : std::max(0, qi + off - dl);
  *hi = dr < 0 ? s.Nk - 1 : std::min(s.Nk - 1, qi + off + dr);
}

namespace {

struct Triple {
  int32_t head, qi, kj;
};

// Append one chain with first/last flags.
void push_chain(std::vector<StepRec>& dst, const std::vector<Triple>& chain,
                const std::vector<int32_t>& ords) {
  const size_t n = chain.size();
  for (size_t i = 0; i < n; ++i) {
    int32_t f = ords[i];
    if (i == 0) f |= kFirstFlag;
    if (i + 1 == n) f |= kLastFlag;
    dst.push_back({chain[i].head, chain[i].qi, chain[i].kj, f});
  }
}

std::string build_list_scheduled(const Schedule& s, std::vector<std::vector<StepRec>>& per_wg) {
  // Chains in (group, kj) order go to the workgroup with the least work so
  // far (unit cost per step; ties to the lowest index).
  using Slot = std::pair<long long, int>;
  std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> heap;
  for (int w = 0; w < s.P; ++w) heap.push({0, w});
  std::vector<Triple> chain;
  std::vector<int32_t> ords;
  for (int grp = 0; grp < s.groups; ++grp) {
    for (int kj = 0; kj < s.Nk; ++kj) {
      int lo, hi;  // the query tiles that see kv tile kj
      visible_q(s, kj, &lo, &hi);
      if (lo > hi) continue;  // seen by no query tile: no chain
      chain.clear();
      ords.clear();
      for (int t = 0; t <= hi - lo; ++t) {
        const int qi = (s.walk == kDescQ) ? (hi - t) : (lo + t);
        int klo, khi;
        visible_k(s, qi, &klo, &khi);
        for (int u = 0; u < s.g; ++u) {
          chain.push_back({grp * s.g + u, qi, kj});
          ords.push_back(kj - klo);  // ascending key/value order for every dQ tile
        }
      }
      Slot top = heap.top();
      heap.pop();
      push_chain(per_wg[top.second], chain, ords);
      heap.push({top.first + static_cast<long long>(chain.size()), top.second});
    }
  }
  return {};
}

// Workgroup index of member p of gang gi.  Workgroups are dispatched round
// robin over the 8 chiplets (index w runs on chiplet w % 8).  With xcd_local:
//  * shift gangs, when the grid is a multiple of 8 x 16: runs of 16
//    consecutive members share a chiplet, so the query tile member p reads
//    one step after member p+1 is usually still in that chiplet's L2
//    (measured: ~2 % faster at 16384 x 128 than the mapping below);
//  * otherwise members get indices congruent modulo the gang count.
// Without xcd_local each gang occupies a contiguous index range.
int gang_slot(int gi, int p, int n_gangs, int gang, const Schedule& s) {
  constexpr int kChiplets = 8, kRun = 16;
  if (!s.xcd_local) return gi * gang + p;
  if (s.walk == kShift && s.P % (kChiplets * kRun) == 0) {
    const int m = gi * gang + p;
    const int k = (m / (kChiplets * kRun)) * kRun + m % kRun;
    return (m / kRun) % kChiplets + kChiplets * k;
  }
  return p * n_gangs + gi;
}

std::string build_gang(const Schedule& s, std::vector<std::vector<StepRec>>& per_wg) {
  const int N = s.Nq;
  const int M = N / 2;        // symmetric shift: tile pairs of the square causal part
  const int R = s.Nk - s.Nq;  // symmetric shift: dense kv tiles in front of that square
  // natural gang: one member per key/value tile up to one per query tile
  // (shift), one per tile pair (symmetric shift)
  const int natural = (s.walk == kShift) ? std::min(s.Nk, N) : M;
  const int gang = (s.max_gang > 0 && s.max_gang < natural) ? s.max_gang : natural;
  const int n_gangs = s.P / gang;
  if (n_gangs < 1) return "gang of " + std::to_string(gang) + " workgroups exceeds " + std::to_string(s.P);
  // Per member: its chains as (kj, walk of one head), units taken in rounds:
  // member p keeps units p, p + gang, p + 2*gang, ...
  std::vector<std::vector<std::pair<int, std::vector<int>>>> member(gang);
  auto shifted = [N](int kj) {
    std::vector<int> w(N);
    for (int t = 0; t < N; ++t) w[t] = (kj + t) % N;
    return std::make_pair(kj, std::move(w));
  };
  for (int p = 0; p < gang; ++p) {
    if (s.walk == kShift) {
      for (int i = p; i < s.Nk; i += gang) member[p].push_back(shifted(i));
      continue;
    }
    for (int i = p; i < M; i += gang) {
      std::vector<int> a, b;
      for (int t = 0; t < M; ++t) a.push_back(M + (i + t) % M);   // dense rectangle
      for (int q = i; q < M; ++q) a.push_back(q);                  // own triangle part
      for (int q = N - 1; q >= N - 1 - i; --q) b.push_back(q);     // folded triangle
      member[p].push_back({R + i, std::move(a)});
      member[p].push_back({R + N - 1 - i, std::move(b)});
    }
    for (int d = p; d < R; d += gang) member[p].push_back(shifted(d));
  }
  // Ordinals: rank of (position, kj) among the contributors of each
  // (head-in-group u, qi).  Identical for every group, so computed once.
  std::vector<std::vector<std::pair<int, int>>> bucket(static_cast<size_t>(s.g) * N);
  for (int p = 0; p < gang; ++p) {
    int pos = 0;
    for (auto& ch : member[p])
      for (int qi : ch.second)
        for (int u = 0; u < s.g; ++u) bucket[static_cast<size_t>(u) * N + qi].push_back({pos++, ch.first});
  }
  std::vector<int32_t> rank(static_cast<size_t>(s.g) * N * s.Nk, -1);  // [u][qi][kj]
  for (int u = 0; u < s.g; ++u)
    for (int qi = 0; qi < N; ++qi) {
      auto& v = bucket[static_cast<size_t>(u) * N + qi];
      std::sort(v.begin(), v.end());
      for (size_t r = 0; r < v.size(); ++r)
        rank[(static_cast<size_t>(u) * N + qi) * s.Nk + v[r].second] = static_cast<int32_t>(r);
    }
  std::vector<Triple> chain;
  std::vector<int32_t> ords;
  for (int grp = 0; grp < s.groups; ++grp) {
    const int gi = grp % n_gangs;
    for (int p = 0; p < gang; ++p) {
      const int w = gang_slot(gi, p, n_gangs, gang, s);
      for (auto& ch : member[p]) {
        chain.clear();
        ords.clear();
        for (int qi : ch.second)
          for (int u = 0; u < s.g; ++u) {
            chain.push_back({grp * s.g + u, qi, ch.first});
            ords.push_back(rank[(static_cast<size_t>(u) * N + qi) * s.Nk + ch.first]);
          }
        push_chain(per_wg[w], chain, ords);
      }
    }
  }
  return {};
}

// Shift on a sliding-window band (dl, 0): units of dl + 1 steps per head
// (an unclipped key/value tile; a pair of tiles clipped at the first and the
// last query tile when Nk - Nq >= dl; the symmetric shift of the corner
// triangle when Nk = Nq and dl is even), every chain walked in descending
// query order.  The units of all groups are dealt round-robin over the
// workgroups (unit i: workgroup i mod P, round i / P); a step's lock-step key
// is round * unit length + its position in the unit, and each dQ tile ranks
// its contributors by (key, kj).
std::string build_band_shift(const Schedule& s, std::vector<std::vector<StepRec>>& per_wg) {
  const int N = s.Nq, off = s.Nk - s.Nq, dl = s.band_l;
  if (!band_shift_applies(s.Nq, s.Nk, s.band_l, s.band_r))
    return "band shift needs a sliding band (right = 0, 1 <= left < Nq tiles) on a square grid with an even left "
           "extent, or Nk - Nq >= left";
  using Chain = std::pair<int, std::vector<int>>;
  std::vector<std::vector<Chain>> units;
  for (int kj = off; kj < off + N - dl; ++kj) {
    std::vector<int> w;
    for (int t = 0; t <= dl; ++t) w.push_back(kj - off + dl - t);
    units.push_back({{kj, std::move(w)}});
  }
  if (off >= dl) {
    for (int ell = 1; ell <= dl; ++ell) {
      std::vector<int> wb, wt;
      for (int t = 0; t < ell; ++t) wb.push_back(ell - 1 - t);
      for (int t = 0; t < dl + 1 - ell; ++t) wt.push_back(N - 1 - t);
      units.push_back({{off - dl - 1 + ell, std::move(wb)}, {off + N - dl - 1 + ell, std::move(wt)}});
    }
  } else {  // off == 0, dl even
    const int M = dl / 2, base = N - dl;
    for (int p = 0; p < M; ++p) {
      std::vector<int> a, b;
      for (int t = 0; t < M; ++t) a.push_back(base + M + (p + t) % M);
      for (int q = p; q < M; ++q) a.push_back(base + q);
      for (int q = dl - 1; q >= dl - 1 - p; --q) b.push_back(base + q);
      units.push_back({{base + p, std::move(a)}, {base + dl - 1 - p, std::move(b)}});
    }
  }
  const long long U = static_cast<long long>(units.size());
  const long long L = static_cast<long long>(dl + 1) * s.g;
  // Units are dealt in this order: the units that keep the shift's lock-step
  // slots (unclipped tiles, first/last pairs) of every group, then the
  // corner-triangle units of every group.  A triangle unit dealt into the
  // same round as its group's unclipped units would reach some dQ tiles at
  // the same lock-step position as one of them.  The i-th unit dealt goes to
  // workgroup i mod P in round i / P.
  const long long n_al = U - (off < dl ? dl / 2 : 0);
  auto dealt = [&](long long grp, long long u) {
    return u < n_al ? grp * n_al + u : static_cast<long long>(s.groups) * n_al + grp * (U - n_al) + (u - n_al);
  };
  struct DealtUnit {
    long long i;                  // position in the dealing order
    std::vector<StepRec> steps;   // its chains, flagged and ranked
  };
  std::vector<DealtUnit> dealt_units;
  // Groups are independent (their dQ tiles differ), so ranks are formed one
  // group at a time.
  std::vector<std::vector<std::pair<long long, int>>> bucket(static_cast<size_t>(s.g) * N);  // (u, qi)
  std::vector<int32_t> rank(static_cast<size_t>(s.g) * N * s.Nk, -1);                       // [u][qi][kj]
  std::vector<Triple> chain;
  std::vector<int32_t> ords;
  for (int grp = 0; grp < s.groups; ++grp) {
    for (auto& v : bucket) v.clear();
    for (long long u = 0; u < U; ++u) {
      const long long i = dealt(grp, u);
      long long pos = (i / s.P) * L;
      for (const Chain& ch : units[u])
        for (int qi : ch.second)
          for (int h = 0; h < s.g; ++h) bucket[static_cast<size_t>(h) * N + qi].push_back({pos++, ch.first});
    }
    for (size_t hq = 0; hq < bucket.size(); ++hq) {
      auto& v = bucket[hq];
      std::sort(v.begin(), v.end());
      for (size_t r = 0; r < v.size(); ++r) rank[hq * s.Nk + v[r].second] = static_cast<int32_t>(r);
    }
    for (long long u = 0; u < U; ++u) {
      const long long i = dealt(grp, u);
      DealtUnit du{i, {}};
      for (const Chain& ch : units[u]) {
        chain.clear();
        ords.clear();
        for (int qi : ch.second)
          for (int h = 0; h < s.g; ++h) {
            chain.push_back({grp * s.g + h, qi, ch.first});
            ords.push_back(rank[(static_cast<size_t>(h) * N + qi) * s.Nk + ch.first]);
          }
        push_chain(du.steps, chain, ords);
      }
      dealt_units.push_back(std::move(du));
    }
  }
  // Each workgroup runs its units in the order they were dealt (round by round).
  std::sort(dealt_units.begin(), dealt_units.end(),
            [](const DealtUnit& x, const DealtUnit& y) { return x.i < y.i; });
  for (DealtUnit& du : dealt_units) {
    const int w = gang_slot(0, static_cast<int>(du.i % s.P), 1, s.P, s);
    per_wg[w].insert(per_wg[w].end(), du.steps.begin(), du.steps.end());
  }
  return {};
}

}  // namespace

bool band_shift_applies(int Nq, int Nk, int band_l, int band_r) {
  const int off = Nk - Nq;
  if (band_r != 0 || band_l < 1 || Nq < band_l + 1 || off < 0) return false;
  return off >= band_l || (off == 0 && band_l % 2 == 0);
}

std::string choose_schedule(int mask, int Nq, int Nk, int D, int g, int P, int* kind, int* max_gang, int band_l,
                            int band_r) {
  if (Nq < 1 || Nk < 1 || D < 1 || g < 1 || P < 1) return "sizes must be positive";
  if (mask == kMaskBand) {
    if (Nk < Nq) return "a band mask needs Sk >= Sq";
    // measured on MI355X: the band shift beats the descending walk (sliding window of 4096 over 16384 tokens)
    *kind = band_shift_applies(Nq, Nk, band_l, band_r) ? kShift : kDescQ;
    *max_gang = 0;
    return "";
  }
  if (mask != kMaskFull && mask != kMaskCausal) return "unknown mask";
  if (mask == kMaskCausal && Nk < Nq) return "a causal mask needs Sk >= Sq";
  const int N = Nq;
  // Measured on MI355X: the gang schedules are the fastest deterministic ones
  // for every shape tried, whatever D and g; D and g are kept in the key.
  (void)D;
  (void)g;
  int units = 0;  // natural gang size
  if (mask == kMaskFull) {
    *kind = kShift;
    units = std::min(Nq, Nk);
  } else if (N % 2 == 0) {
    *kind = kSymShift;
    units = N / 2;
  } else {
    *kind = kDescQ;
  }
  *max_gang = (units > P) ? P : 0;
  return "";
}

std::string build_schedule(int mask, int kind, int Nq, int Nk, int g, int groups, int P, bool xcd_local,
                           int atomic_walk, int max_gang, Schedule* out, int band_l, int band_r) {
  if (Nq < 1 || Nk < 1 || g < 1 || groups < 1 || P < 1) return "sizes must be positive";
  if (mask != kMaskFull && mask != kMaskCausal && mask != kMaskBand) return "unknown mask";
  if (mask == kMaskBand && Nk < Nq) return "a band mask needs at least as many key/value tiles as query tiles";
  if (kind < kSerial || kind > kAtomic) return "unknown schedule";
  if (Nq > 32767 || Nk > 32767) return "too many tiles";
  if (mask == kMaskCausal && Nk < Nq) return "a causal mask needs at least as many key/value tiles as query tiles";
  {
    // Step indices are int32 on the device (bound: every tile pair visible).
    if ((long long)Nq * Nk * g * groups > 0x7fffffffLL) return "too many steps for 32-bit step indices";
  }
  int walk = kind;
  if (kind == kAtomic) {
    walk = (atomic_walk < 0) ? (mask == kMaskFull ? kSerial : kDescQ) : atomic_walk;
    if (walk < kSerial || walk > kSymShift) return "unknown atomic walk";
  }
  if (walk == kShift && mask == kMaskCausal) return "shift scheduling needs a full or band mask";
  if (walk == kSymShift && mask != kMaskCausal) return "symmetric shift needs a causal mask";
  if (walk == kSymShift && (Nq % 2)) return "symmetric shift needs an even tile count";
  Schedule s;
  s.mask = mask;
  s.kind = kind;
  s.walk = walk;
  s.Nq = Nq;
  s.Nk = Nk;
  s.g = g;
  s.groups = groups;
  s.P = P;
  s.xcd_local = xcd_local;
  s.max_gang = max_gang > 0 ? max_gang : 0;
  s.band_l = mask == kMaskBand ? (band_l < 0 ? -1 : band_l) : -1;
  s.band_r = mask == kMaskBand ? (band_r < 0 ? -1 : band_r) : -1;
  std::vector<std::vector<StepRec>> per_wg(P);
  std::string err = (walk == kSerial || walk == kDescQ) ? build_list_scheduled(s, per_wg)
                    : (walk == kShift && mask == kMaskBand) ? build_band_shift(s, per_wg)
                                                             : build_gang(s, per_wg);
  if (!err.empty()) return err;
  s.offsets.resize(P + 1);
  size_t total = 0;
  for (int w = 0; w < P; ++w) {
    s.offsets[w] = static_cast<int32_t>(total);
    total += per_wg[w].size();
  }
  s.offsets[P] = static_cast<int32_t>(total);
  s.steps.reserve(total);
  for (auto& v : per_wg) s.steps.insert(s.steps.end(), v.begin(), v.end());
  *out = std::move(s);
  return {};
}

namespace {
// SplitMix64's output function (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014), used as a counter-based
// generator: the draw for (seed, workgroup w, list position i) mixes
// seed ^ (w << 32 | i) advanced by one golden-ratio increment.
uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9e3779b97f4a7c15ULL;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}
}  // namespace

double jitter_factor(uint64_t seed, int w, int i) {
  if (seed == 0) return 1.0;
  const uint64_t x = seed ^ ((static_cast<uint64_t>(static_cast<uint32_t>(w)) << 32) | static_cast<uint32_t>(i));
  return 0.5 + static_cast<double>(splitmix64(x) >> 11) * 0x1.0p-53;
}

bool simulate_schedule(const Schedule& s, double c, double r, uint64_t jitter_seed, double* makespan,
                       double* total_wait) {
  const size_t tiles = static_cast<size_t>(s.g) * s.groups * s.Nq;
  std::vector<int32_t> count(tiles, 0);
  std::vector<double> done_at(tiles, 0.0);
  std::vector<int32_t> idx(s.P, 0);
  std::vector<double> t(s.P, 0.0);
  long long remaining = static_cast<long long>(s.steps.size());
  double wait = 0.0;
  while (remaining > 0) {
    bool progressed = false;
    for (int w = 0; w < s.P; ++w) {
      const int32_t end = s.offsets[w + 1];
      while (s.offsets[w] + idx[w] < end) {
        const StepRec& st = s.steps[s.offsets[w] + idx[w]];
        const size_t key = static_cast<size_t>(st.head) * s.Nq + st.qi;
        const int32_t ord = st.ordflags & kOrdMask;
        if (count[key] != ord) break;
        const double ready = t[w] + c * jitter_factor(jitter_seed, w, idx[w]);
        const double start = std::max(ready, done_at[key]);
        wait += start - ready;
        t[w] = start + r;
        done_at[key] = t[w];
        count[key] = ord + 1;
        ++idx[w];
        --remaining;
        progressed = true;
      }
    }
    if (!progressed) return false;
  }
  double mk = 0.0;
  for (double x : t) mk = std::max(mk, x);
  if (makespan) *makespan = mk;
  if (total_wait) *total_wait = wait;
  return true;
}

std::string validate_schedule(const Schedule& s) {
  const int Nq = s.Nq, Nk = s.Nk;
  const long long heads = static_cast<long long>(s.g) * s.groups;
  if (static_cast<int>(s.offsets.size()) != s.P + 1) return "offset table size";
  if (s.offsets[0] != 0 || s.offsets[s.P] != static_cast<int32_t>(s.steps.size())) return "offset table bounds";
  std::vector<uint8_t> seen(static_cast<size_t>(heads) * Nq * Nk, 0);
  std::vector<int32_t> owner(static_cast<size_t>(s.groups) * Nk, -1);
  long long covered = 0;
  for (int w = 0; w < s.P; ++w) {
    if (s.offsets[w + 1] < s.offsets[w]) return "offsets decrease";
    long long run = -1;  // chain key (group * Nk + kj) of the open chain
    for (int32_t i = s.offsets[w]; i < s.offsets[w + 1]; ++i) {
      const StepRec& st = s.steps[i];
      if (st.head < 0 || st.head >= heads || st.qi < 0 || st.qi >= Nq || st.kj < 0 || st.kj >= Nk)
        return "step index out of range";
      int klo, khi;
      visible_k(s, st.qi, &klo, &khi);
      if (st.kj < klo || st.kj > khi) return "masked tile pair scheduled";
      const size_t pair = (static_cast<size_t>(st.head) * Nq + st.qi) * Nk + st.kj;
      if (seen[pair]) return "tile pair scheduled twice";
      seen[pair] = 1;
      ++covered;
      const long long ck = static_cast<long long>(st.head / s.g) * Nk + st.kj;
      if (st.ordflags & kFirstFlag) {
        if (run >= 0) return "chain not closed before the next starts";
        if (owner[ck] >= 0) return "chain split";
        owner[ck] = w;
        run = ck;
      }
      if (run != ck) return "chain interrupted";
      if (st.ordflags & kLastFlag) run = -1;
    }
    if (run >= 0) return "list ends inside a chain";
  }
  long long expect = 0;
  for (int qi = 0; qi < Nq; ++qi) {
    int klo, khi;
    visible_k(s, qi, &klo, &khi);
    expect += std::max(0, khi - klo + 1);
  }
  if (covered != expect * heads) return "coverage mismatch";
  for (size_t c = 0; c < owner.size(); ++c) {
    int lo, hi;
    visible_q(s, static_cast<int>(c % Nk), &lo, &hi);
    if ((owner[c] >= 0) != (lo <= hi)) return "missing or extra chain";
  }
  // ordinals of each dQ tile: exactly 0..count-1
  std::vector<uint8_t> ordseen(static_cast<size_t>(heads) * Nq * Nk, 0);
  for (const StepRec& st : s.steps) {
    const int32_t ord = st.ordflags & kOrdMask;
    int klo, khi;
    visible_k(s, st.qi, &klo, &khi);
    const int32_t lim = khi - klo + 1;
    if (ord < 0 || ord >= lim) return "ordinal out of range";
    const size_t k = (static_cast<size_t>(st.head) * Nq + st.qi) * Nk + ord;
    if (ordseen[k]) return "ordinal repeated";
    ordseen[k] = 1;
  }
  double mk, wt;
  if (!simulate_schedule(s, 1.0, 1.0, 0, &mk, &wt)) return "deadlock";
  return {};
}

}  // namespace dash
