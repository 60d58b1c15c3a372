// C ABI of libdash_attn.so (declared in include/dash_attn.h).
//
// Everything is validated before anything is enqueued.  The library owns a
// per-device cache of uploaded step lists and, when the caller passes no
// workspace, a grow-only per-device workspace; both live until process exit.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/dash_attn.h"
#include "kernels.hpp"
#include "schedule.hpp"

struct dash_schedule {
  dash::Schedule s;
};

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DASH_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

struct DeviceInfo {
  int num_cu = 0, lds = 0, clock_khz = 0;
};

std::mutex g_mu;
std::map<int, DeviceInfo> g_devinfo;

int device_info(int dev, DeviceInfo* out) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_devinfo.find(dev);
  if (it == g_devinfo.end()) {
    hipDeviceProp_t p;
    hipError_t e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    DeviceInfo d;
    d.num_cu = p.multiProcessorCount;
    d.lds = (int)p.sharedMemPerBlock;
    d.clock_khz = p.clockRate;
    it = g_devinfo.emplace(dev, d).first;
  }
  *out = it->second;
  return DASH_OK;
}

// Uploaded step lists, keyed by everything that shapes them.
struct DevSchedule {
  int32_t* steps = nullptr;
  int32_t* offsets = nullptr;
  long long num_steps = 0;
};
// dev, mask, kind, Nq, Nk, g, groups, P, xcd, walk, cap, band_l, band_r
using SchedKey = std::tuple<int, int, int, int, int, int, int, int, int, int, int, int, int>;
std::map<SchedKey, DevSchedule> g_sched;

struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::map<int, Workspace> g_ws;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// One semaphore word per (64-row dQ block, wave holding dQ tiles of it).
constexpr size_t kSemWordsPerBlock = 8;

struct WsLayout {
  size_t ws_dq, delta, sem, err, dummy, total;
};

// Sq query rows per head; Sw (a multiple of 64) workspace rows per head, the
// query tiles' virtual rows (see TileGrid).
WsLayout ws_layout(int B, int Hq, int Sq, int Sw, int D) {
  WsLayout L;
  const size_t rows = (size_t)B * Hq * Sq;
  const size_t wrows = (size_t)B * Hq * Sw;
  size_t off = 0;
  L.ws_dq = off;
  off = align256(off + wrows * D * sizeof(float));
  L.delta = off;
  off = align256(off + rows * sizeof(float));
  L.sem = off;
  off = align256(off + (size_t)B * Hq * (Sw / 64) * kSemWordsPerBlock * sizeof(int));
  L.err = off;
  off = align256(off + 16);
  L.dummy = off;  // 8 dQ tiles' worth of scratch for writes with no destination
  off = align256(off + 8 * 1024 * sizeof(float));
  L.total = off;
  return L;
}

// Returned by check_sizes when there are no query rows (B = 0 or Sq = 0).
constexpr int kEmpty = 1;

// A mask as a window around the bottom-right diagonal: query row i sees key
// j when -wl <= j - (i + Sk - Sq) <= wr, -1 meaning unbounded.  kind is the
// schedule-level mask: full (both unbounded), causal (wl unbounded, wr = 0)
// or band (anything else).
struct Mask {
  int kind = dash::kMaskFull;
  int wl = -1, wr = -1;
  bool aligned() const { return kind != dash::kMaskFull; }
};

// From the DASH_MASK_* enum; kind = -1 if unknown.
Mask mask_from_enum(int mask) {
  Mask m;
  if (mask == DASH_MASK_FULL) return m;
  if (mask == DASH_MASK_CAUSAL) {
    m.kind = dash::kMaskCausal;
    m.wr = 0;
    return m;
  }
  m.kind = -1;
  return m;
}

// From window extents; a side that reaches past every key is unbounded
// (left >= Sk - 1, right >= Sq - 1), so a window may reduce to the full or
// the causal mask.  kind = -1 if an extent is below -1.
Mask mask_from_window(int wl, int wr, int Sq, int Sk) {
  Mask m;
  if (wl < -1 || wr < -1) {
    m.kind = -1;
    return m;
  }
  m.wl = (wl < 0 || (long long)wl >= (long long)Sk - 1) ? -1 : wl;
  m.wr = (wr < 0 || (long long)wr >= (long long)Sq - 1) ? -1 : wr;
  if (m.wl < 0 && m.wr < 0) m.kind = dash::kMaskFull;
  else if (m.wl < 0 && m.wr == 0) m.kind = dash::kMaskCausal;
  else m.kind = dash::kMaskBand;
  return m;
}

int check_sizes(int B, int Hq, int Hkv, int Sq, int Sk, int D, const Mask& mask) {
  if (B < 0 || Sq < 0 || Sk < 0) return fail(DASH_ERR_INVALID_ARG, "sizes must not be negative");
  if (Hq <= 0 || Hkv <= 0 || D <= 0) return fail(DASH_ERR_INVALID_ARG, "head counts and head dimension must be positive");
  if (Hq % Hkv) return fail(DASH_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
  if (mask.kind < 0) return fail(DASH_ERR_INVALID_ARG, "unknown mask or negative window extent");
  if (mask.aligned() && Sk < Sq)
    return fail(DASH_ERR_INVALID_ARG, "a causal or windowed mask needs Sk >= Sq (it is aligned at the bottom right)");
  if (D != 64 && D != 128) return fail(DASH_ERR_UNSUPPORTED, "head dimension must be 64 or 128");
  if (Sq > (1 << 24) || Sk > (1 << 24)) return fail(DASH_ERR_UNSUPPORTED, "sequence longer than 2^24 rows");
  if ((long long)B * Hq * (std::max(Sq, Sk) + 256LL) * D >= (1LL << 40))
    return fail(DASH_ERR_UNSUPPORTED, "problem too large");
  if (B == 0 || Sq == 0) return kEmpty;
  if (Sk == 0) return fail(DASH_ERR_INVALID_ARG, "no keys: the softmax of an empty row is undefined");
  return DASH_OK;
}

int check_ptrs(const void* const* ptrs, int nptr) {
  for (int i = 0; i < nptr; ++i) {
    if (!ptrs[i]) return fail(DASH_ERR_INVALID_ARG, "null tensor pointer (argument " + std::to_string(i) + ")");
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % 16) return fail(DASH_ERR_INVALID_ARG, "tensor pointer not 16-byte aligned");
  }
  return DASH_OK;
}

// Tile grid of one backward call.  Key/value tiles: Nk = ceil(Sk / T), the
// last one possibly partial.  Query tiles cover virtual rows, virtual row =
// query row + qshift.  Full mask: qshift = 0, Nq = ceil(Sq / T).  Causal and
// banded masks (bottom right, offset Sk - Sq = diag_off * T + qshift): the query tiles
// are aligned with the key/value tiles, so query tile qi meets the diagonal
// in key/value tile qi + diag_off exactly as in the square case, and
// Nq = Nk - diag_off (the first tile starts qshift rows before row 0).
struct TileGrid {
  int T, Nq, Nk, qshift, diag_off, Sw;
};

TileGrid tile_grid(int Sq, int Sk, int T, bool aligned) {
  TileGrid t;
  t.T = T;
  t.Nk = (Sk + T - 1) / T;
  if (aligned) {
    t.diag_off = (Sk - Sq) / T;
    t.qshift = (Sk - Sq) % T;
    t.Nq = t.Nk - t.diag_off;
  } else {
    t.diag_off = 0;
    t.qshift = 0;
    t.Nq = (Sq + T - 1) / T;
  }
  t.Sw = t.Nq * T;
  return t;
}

float default_scale(float s, int D) { return s > 0.f ? s : 1.0f / std::sqrt((float)D); }

}  // namespace

extern "C" {

const char* dash_status_string(int status) {
  switch (status) {
    case DASH_OK: return "ok";
    case DASH_ERR_INVALID_ARG: return "invalid argument";
    case DASH_ERR_UNSUPPORTED: return "unsupported";
    case DASH_ERR_HIP: return "HIP runtime error";
    case DASH_ERR_INVALID_SCHEDULE: return "invalid schedule";
    case DASH_ERR_TIMEOUT: return "semaphore wait timed out";
    case DASH_ERR_WORKSPACE: return "workspace too small or misaligned";
    default: return "unknown status";
  }
}

const char* dash_last_error(void) { return g_last_error.c_str(); }

int dash_device_info(int device, int* num_cu, int* lds_bytes, int* clock_khz) {
  DeviceInfo d;
  int st = device_info(device, &d);
  if (st) return st;
  if (num_cu) *num_cu = d.num_cu;
  if (lds_bytes) *lds_bytes = d.lds;
  if (clock_khz) *clock_khz = d.clock_khz;
  return DASH_OK;
}

int dash_schedule_build(int mask, int schedule, int N, int g, int groups, int P, int xcd_local, int atomic_walk,
                        int max_gang, dash_schedule** out) {
  return dash_schedule_build_qk(mask, schedule, N, N, g, groups, P, xcd_local, atomic_walk, max_gang, out);
}

int dash_schedule_build_qk(int mask, int schedule, int Nq, int Nk, int g, int groups, int P, int xcd_local,
                           int atomic_walk, int max_gang, dash_schedule** out) {
  if (!out) return fail(DASH_ERR_INVALID_ARG, "null output");
  *out = nullptr;
  auto s = std::make_unique<dash_schedule>();
  if (max_gang < 0) return fail(DASH_ERR_INVALID_ARG, "negative gang cap");
  std::string err = dash::build_schedule(mask, schedule, Nq, Nk, g, groups, P, xcd_local != 0, atomic_walk, max_gang, &s->s);
  if (!err.empty()) {
    const bool bad = (Nq < 1 || Nk < 1 || g < 1 || groups < 1 || P < 1 || (mask != 0 && mask != 1) || schedule < 0 ||
                      schedule > 4 || (mask == 1 && Nk < Nq));
    return fail(bad ? DASH_ERR_INVALID_ARG : DASH_ERR_UNSUPPORTED, err);
  }
  *out = s.release();
  return DASH_OK;
}

int dash_schedule_build_band(int schedule, int Nq, int Nk, int band_left, int band_right, int g, int groups, int P,
                             int xcd_local, int atomic_walk, int max_gang, dash_schedule** out) {
  if (!out) return fail(DASH_ERR_INVALID_ARG, "null output");
  *out = nullptr;
  if (max_gang < 0) return fail(DASH_ERR_INVALID_ARG, "negative gang cap");
  if (band_left < -1 || band_right < -1) return fail(DASH_ERR_INVALID_ARG, "band extents must be >= -1");
  auto s = std::make_unique<dash_schedule>();
  std::string err = dash::build_schedule(dash::kMaskBand, schedule, Nq, Nk, g, groups, P, xcd_local != 0, atomic_walk,
                                         max_gang, &s->s, band_left, band_right);
  if (!err.empty()) {
    const bool bad = (Nq < 1 || Nk < Nq || g < 1 || groups < 1 || P < 1 || schedule < 0 || schedule > 4);
    return fail(bad ? DASH_ERR_INVALID_ARG : DASH_ERR_UNSUPPORTED, err);
  }
  *out = s.release();
  return DASH_OK;
}

int dash_schedule_num_workgroups(const dash_schedule* s) { return s ? s->s.P : 0; }
long long dash_schedule_num_steps(const dash_schedule* s) { return s ? (long long)s->s.steps.size() : 0; }

int dash_schedule_export(const dash_schedule* s, int32_t* offsets, int32_t* steps) {
  if (!s || !offsets || !steps) return fail(DASH_ERR_INVALID_ARG, "null argument");
  std::memcpy(offsets, s->s.offsets.data(), s->s.offsets.size() * sizeof(int32_t));
  std::memcpy(steps, s->s.steps.data(), s->s.steps.size() * sizeof(dash::StepRec));
  return DASH_OK;
}

int dash_schedule_validate(const dash_schedule* s) {
  if (!s) return fail(DASH_ERR_INVALID_ARG, "null schedule");
  std::string err = dash::validate_schedule(s->s);
  return err.empty() ? DASH_OK : fail(DASH_ERR_INVALID_SCHEDULE, err);
}

int dash_schedule_simulate(const dash_schedule* s, double c, double r, double* makespan, double* total_wait) {
  if (!s) return fail(DASH_ERR_INVALID_ARG, "null schedule");
  if (!dash::simulate_schedule(s->s, c, r, makespan, total_wait)) return fail(DASH_ERR_INVALID_SCHEDULE, "deadlock");
  return DASH_OK;
}

void dash_schedule_free(dash_schedule* s) { delete s; }

int dash_schedule_choose_qk(int mask, int Nq, int Nk, int D, int g, int P, int* schedule, int* max_gang) {
  if (!schedule || !max_gang) return fail(DASH_ERR_INVALID_ARG, "null output");
  std::string err = dash::choose_schedule(mask, Nq, Nk, D, g, P, schedule, max_gang);
  return err.empty() ? DASH_OK : fail(DASH_ERR_INVALID_ARG, err);
}

int dash_schedule_choose_band(int Nq, int Nk, int band_left, int band_right, int D, int g, int P, int* schedule,
                              int* max_gang) {
  if (!schedule || !max_gang) return fail(DASH_ERR_INVALID_ARG, "null output");
  if (band_left < -1 || band_right < -1) return fail(DASH_ERR_INVALID_ARG, "band extents must be >= -1");
  std::string err = dash::choose_schedule(dash::kMaskBand, Nq, Nk, D, g, P, schedule, max_gang, band_left, band_right);
  return err.empty() ? DASH_OK : fail(DASH_ERR_INVALID_ARG, err);
}

int dash_schedule_choose(int mask, int N, int D, int g, int P, int* schedule, int* max_gang) {
  return dash_schedule_choose_qk(mask, N, N, D, g, P, schedule, max_gang);
}

static int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                    int Sq, int Sk, int D, float softmax_scale, const Mask& mask, void* stream) {
  const void* ptrs[] = {q, k, v, o, lse};
  int st = check_sizes(B, Hq, Hkv, Sq, Sk, D, mask);
  if (st == kEmpty) return DASH_OK;  // no query rows: nothing to write
  if (st) return st;
  st = check_ptrs(ptrs, 5);
  if (st) return st;
  if ((long long)B * Hq > 65535) return fail(DASH_ERR_UNSUPPORTED, "B*Hq exceeds the grid limit");
  hipError_t e = dash::launch_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, default_scale(softmax_scale, D), mask.wl,
                                  mask.wr, (hipStream_t)stream);
  return e == hipSuccess ? DASH_OK : hip_fail(e, "forward launch");
}

int dash_attn_fwd_qk(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int Sq, int Sk, int D, float softmax_scale, int mask, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, softmax_scale, mask_from_enum(mask), stream);
}

int dash_attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                         int Sq, int Sk, int D, float softmax_scale, int window_left, int window_right,
                         void* stream) {
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, softmax_scale,
                  mask_from_window(window_left, window_right, Sq, Sk), stream);
}

int dash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int S,
                  int D, float softmax_scale, int mask, void* stream) {
  return dash_attn_fwd_qk(q, k, v, o, lse, B, Hq, Hkv, S, S, D, softmax_scale, mask, stream);
}

int dash_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D, size_t* bytes) {
  if (!bytes) return fail(DASH_ERR_INVALID_ARG, "null output");
  if (B < 0 || Hq <= 0 || Hkv <= 0 || S < 0 || D <= 0) return fail(DASH_ERR_INVALID_ARG, "sizes must not be negative");
  // Any key length and tile: at most round_up(S, T) + T virtual rows per head.
  *bytes = ws_layout(B, Hq, S, ((S + 127) / 128) * 128 + 128, D).total;
  return DASH_OK;
}

int dash_attn_bwd_delta(const void* o, const void* dO, float* delta, int B, int H, int S, int D, void* stream) {
  const void* ptrs[] = {o, dO, delta};
  int st = check_sizes(B, H, H, S, S, D, Mask());
  if (st == kEmpty) return DASH_OK;
  if (st) return st;
  st = check_ptrs(ptrs, 3);
  if (st) return st;
  hipError_t e = dash::launch_delta(o, dO, delta, (long long)B * H * S, D, nullptr, 0, nullptr, 0, (hipStream_t)stream);
  return e == hipSuccess ? DASH_OK : hip_fail(e, "delta launch");
}

static int zero_bf16(void* p, long long elems, int D, hipStream_t st) {
  // bf16 zero is all-zero bits: clear elems/2 32-bit words (elems is even, D is)
  const hipError_t e = dash::launch_delta(nullptr, nullptr, nullptr, 0, D, (int*)p, elems / 2, nullptr, 0, st);
  return e == hipSuccess ? DASH_OK : hip_fail(e, "zero-fill launch");
}

static int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                    void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int D, float softmax_scale,
                    const Mask& mask, int schedule, const dash_bwd_opts* opts, void* stream) {
  const void* ptrs[] = {q, k, v, o, dO, lse, dq, dk, dv};
  int st = check_sizes(B, Hq, Hkv, Sq, Sk, D, mask);
  if (st != DASH_OK && st != kEmpty) return st;
  if (schedule < DASH_SCHED_SERIAL || schedule > DASH_SCHED_AUTO) return fail(DASH_ERR_INVALID_ARG, "unknown schedule");
  const long long kv_elems = (long long)B * Hkv * Sk * D;
  if (st == kEmpty) {
    // No query rows: dQ is empty and dK = dV = 0 (no key receives any gradient).
    if (kv_elems == 0) return DASH_OK;
    const void* kv_ptrs[] = {dk, dv};
    st = check_ptrs(kv_ptrs, 2);
    if (st) return st;
    st = zero_bf16(dk, kv_elems, D, (hipStream_t)stream);
    return st ? st : zero_bf16(dv, kv_elems, D, (hipStream_t)stream);
  }
  st = check_ptrs(ptrs, 9);
  if (st) return st;
  dash_bwd_opts op;
  std::memset(&op, 0, sizeof(op));
  if (opts) {
    if (opts->struct_size == 0 || opts->struct_size > sizeof(dash_bwd_opts))
      return fail(DASH_ERR_INVALID_ARG, "dash_bwd_opts.struct_size must be sizeof(dash_bwd_opts)");
    std::memcpy(&op, opts, opts->struct_size);
  }
  hipStream_t strm = (hipStream_t)stream;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  DeviceInfo di;
  st = device_info(dev, &di);
  if (st) return st;

  const int T = op.tile ? op.tile : (std::min(Sq, Sk) < 512 ? 64 : 128);
  if (T != 64 && T != 128) return fail(DASH_ERR_UNSUPPORTED, "tile must be 64 or 128");
  const TileGrid tg = tile_grid(Sq, Sk, T, mask.aligned());
  const int Nq = tg.Nq, Nk = tg.Nk;
  // band extents in tiles: a window of w rows reaches ceil(w / T) tiles off the diagonal tile
  const int band_l = mask.kind == dash::kMaskBand && mask.wl >= 0 ? (mask.wl + T - 1) / T : -1;
  const int band_r = mask.kind == dash::kMaskBand && mask.wr >= 0 ? (mask.wr + T - 1) / T : -1;
  const int P = op.num_workgroups > 0 ? op.num_workgroups : di.num_cu;
  if (op.num_workgroups < 0) return fail(DASH_ERR_INVALID_ARG, "negative workgroup count");
  if (op.max_gang < 0) return fail(DASH_ERR_INVALID_ARG, "negative gang cap");
  const int g = Hq / Hkv;
  if (schedule == DASH_SCHED_AUTO) {
    int cap = 0;
    std::string err = dash::choose_schedule(mask.kind, Nq, Nk, D, g, P, &schedule, &cap, band_l, band_r);
    if (!err.empty()) return fail(DASH_ERR_INVALID_ARG, err);
    if (op.max_gang == 0) op.max_gang = cap;
  }
  const int groups = B * Hkv;
  const bool atomic = schedule == DASH_SCHED_ATOMIC;
  const int xcd = op.xcd_local >= 0 ? 1 : 0;
  const int walk = atomic ? op.atomic_walk : -1;
  const float scale = default_scale(softmax_scale, D);

  // Co-residency: the semaphore waits need every workgroup resident at once.
  if (!atomic) {
    bool fits = false;
    e = dash::bwd_kernel_fits(D, T, false, di.num_cu, P, &fits);
    if (e != hipSuccess) return hip_fail(e, "occupancy query");
    if (!fits) return fail(DASH_ERR_UNSUPPORTED, "persistent grid larger than the co-resident capacity");
  }

  // Step lists (validated once, then cached on the device).
  DevSchedule ds;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    SchedKey key{dev, mask.kind, schedule, Nq, Nk, g, groups, P, xcd, atomic ? (walk < 0 ? -1 : walk) : -1, op.max_gang,
                 band_l, band_r};
    auto it = g_sched.find(key);
    if (it == g_sched.end()) {
      dash::Schedule s;
      std::string err = dash::build_schedule(mask.kind, schedule, Nq, Nk, g, groups, P, xcd != 0, walk, op.max_gang, &s,
                                             band_l, band_r);
      if (!err.empty()) return fail(DASH_ERR_UNSUPPORTED, err);
      err = dash::validate_schedule(s);
      if (!err.empty()) return fail(DASH_ERR_INVALID_SCHEDULE, err);
      DevSchedule d;
      d.num_steps = (long long)s.steps.size();
      e = hipMalloc((void**)&d.steps, std::max<size_t>(16, s.steps.size() * sizeof(dash::StepRec)));
      if (e != hipSuccess) return hip_fail(e, "hipMalloc(steps)");
      e = hipMalloc((void**)&d.offsets, s.offsets.size() * sizeof(int32_t));
      if (e != hipSuccess) { (void)hipFree(d.steps); return hip_fail(e, "hipMalloc(offsets)"); }
      e = hipMemcpy(d.steps, s.steps.data(), s.steps.size() * sizeof(dash::StepRec), hipMemcpyHostToDevice);
      if (e == hipSuccess)
        e = hipMemcpy(d.offsets, s.offsets.data(), s.offsets.size() * sizeof(int32_t), hipMemcpyHostToDevice);
      if (e != hipSuccess) { (void)hipFree(d.steps); (void)hipFree(d.offsets); return hip_fail(e, "hipMemcpy(schedule)"); }
      it = g_sched.emplace(key, d).first;
    }
    ds = it->second;
  }

  // Workspace.
  const WsLayout L = ws_layout(B, Hq, Sq, tg.Sw, D);
  char* ws = nullptr;
  if (op.workspace) {
    if (reinterpret_cast<uintptr_t>(op.workspace) % 256) return fail(DASH_ERR_WORKSPACE, "workspace not 256-byte aligned");
    if (op.workspace_bytes < L.total) return fail(DASH_ERR_WORKSPACE, "workspace too small");
    ws = (char*)op.workspace;
  } else {
    std::lock_guard<std::mutex> lk(g_mu);
    Workspace& w = g_ws[dev];
    if (w.bytes < L.total) {
      // The previous buffer may still be in use by queued work on any stream.
      if (w.ptr) {
        e = hipDeviceSynchronize();
        if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
        (void)hipFree(w.ptr);
        w.ptr = nullptr;
        w.bytes = 0;
      }
      e = hipMalloc(&w.ptr, L.total);
      if (e != hipSuccess) return hip_fail(e, "hipMalloc(workspace)");
      w.bytes = L.total;
    }
    ws = (char*)w.ptr;
  }
  float* ws_dq = (float*)(ws + L.ws_dq);
  float* delta = (float*)(ws + L.delta);
  int* sem = (int*)(ws + L.sem);
  int* err = (int*)(ws + L.err);
  const long long rows = (long long)B * Hq * Sq;
  const long long n_sem = (long long)((L.err - L.sem) / 4) + 4;  // semaphores, padding and the error word

  const long long ws_elems = (long long)B * Hq * tg.Sw * D;
  e = dash::launch_delta(o, dO, delta, rows, D, sem, n_sem, atomic ? ws_dq : nullptr, atomic ? ws_elems : 0, strm);
  if (e != hipSuccess) return hip_fail(e, "preprocess launch");

  dash::BwdLaunch bl;
  bl.q = q;
  bl.k = k;
  bl.v = v;
  bl.dO = dO;
  bl.lse = lse;
  bl.delta = delta;
  bl.ws = ws_dq;
  bl.sem = sem;
  bl.err = err;
  bl.dummy = (float*)(ws + L.dummy);
  bl.dk = dk;
  bl.dv = dv;
  bl.steps = ds.steps;
  bl.offsets = ds.offsets;
  bl.stall = op.stall_cycles_out;
  const unsigned long long budget_cycles = op.spin_timeout_cycles ? op.spin_timeout_cycles : (1ULL << 33);
  // wait budget in 100 MHz real-time ticks, from shader cycles at the device clock
  bl.spin_ticks = (long long)((double)budget_cycles * 1e5 / std::max(1, di.clock_khz));
  if (bl.spin_ticks < 1) bl.spin_ticks = 1;
  bl.scale = scale;
  bl.Sq = Sq;
  bl.Sk = Sk;
  bl.D = D;
  bl.T = T;
  bl.g = g;
  bl.wl = mask.wl;
  bl.wr = mask.wr;
  bl.qshift = tg.qshift;
  bl.nblk = tg.Sw / 64;
  bl.diag_off = tg.diag_off;
  bl.P = P;
  bl.atomic = atomic;
  // Key/value tiles that no query tile sees have no chain: their dK/dV are zero.
  if (band_l >= 0 && tg.diag_off > band_l) {
    st = zero_bf16(dk, kv_elems, D, strm);
    if (!st) st = zero_bf16(dv, kv_elems, D, strm);
    if (st) return st;
  }
  if (op.event_start) {
    e = hipEventRecord((hipEvent_t)op.event_start, strm);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(start)");
  }
  e = dash::launch_bwd(bl, strm);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  if (op.event_stop) {
    e = hipEventRecord((hipEvent_t)op.event_stop, strm);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(stop)");
  }
  e = dash::launch_dq_finalize(ws_dq, dq, ws_elems, D, scale, atomic, tg.Sw / 64, tg.qshift, Sq, strm);
  if (e != hipSuccess) return hip_fail(e, "finalize launch");

  if (op.sync_check) {
    e = hipStreamSynchronize(strm);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    int h_err = 0;
    e = hipMemcpy(&h_err, err, sizeof(int), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(error word)");
    if (h_err) return fail(DASH_ERR_TIMEOUT, "a workgroup timed out waiting on a dQ semaphore");
  }
  return DASH_OK;
}

int dash_attn_bwd_qk(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                     void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int D, float softmax_scale,
                     int mask, int schedule, const dash_bwd_opts* opts, void* stream) {
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, Sq, Sk, D, softmax_scale, mask_from_enum(mask), schedule,
                  opts, stream);
}

int dash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                  void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int S, int D, float softmax_scale, int mask,
                  int schedule, const dash_bwd_opts* opts, void* stream) {
  return dash_attn_bwd_qk(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, S, S, D, softmax_scale, mask, schedule, opts,
                          stream);
}

int dash_attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                         void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                         float softmax_scale, int window_left, int window_right, int schedule,
                         const dash_bwd_opts* opts, void* stream) {
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, Sq, Sk, D, softmax_scale,
                  mask_from_window(window_left, window_right, Sq, Sk), schedule, opts, stream);
}

}  // extern "C"
