// C ABI of libdash_attn.so (declared in include/dash_attn.h).
//
// Everything is validated before anything is enqueued.  The library owns a
// bounded per-device cache of uploaded step lists, one grow-only workspace per
// (device, stream) for callers that pass none, and one host-visible word per
// device in which the dQ finalize kernel records a semaphore give-up; all of
// it lives until process exit (evicted step lists are freed earlier).
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
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

// Host phases of each call as roctx ranges (rocprofv3 --marker-trace shows
// them beside the kernels; without a tool attached they cost a branch).
struct Range {
  explicit Range(const char* name) { roctxRangePushA(name); }
  ~Range() { roctxRangePop(); }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

// DASH_LOG=1 in the environment: one line per backward call and per step
// list built, on stderr.
bool log_on() {
  static const bool on = [] {
    const char* v = std::getenv("DASH_LOG");
    return v != nullptr && v[0] != '\0' && v[0] != '0';
  }();
  return on;
}

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DASH_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

struct DeviceInfo {
  int num_cu = 0, num_xcd = 0, lds = 0, clock_khz = 0;
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
    e = hipDeviceGetAttribute(&d.num_xcd, hipDeviceAttributeNumberOfXccs, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(NumberOfXccs)");
    it = g_devinfo.emplace(dev, d).first;
  }
  *out = it->second;
  return DASH_OK;
}

// Uploaded step lists, keyed by everything that shapes them.  The host copy
// stays alive with the entry, so that the asynchronous upload never reads
// freed memory.  At most kSchedCacheEntries entries are kept; the least
// recently used one is evicted (after a device synchronisation, since queued
// kernels may still read it).
struct DevSchedule {
  int32_t* steps = nullptr;
  int32_t* offsets = nullptr;
  long long num_steps = 0;
  std::shared_ptr<dash::Schedule> host;
  unsigned long long last_use = 0;
  // Recorded after the upload on the uploading stream; a call on another
  // stream waits for it until it is seen complete (then it is released).
  hipEvent_t uploaded = nullptr;
  hipStream_t upload_stream = nullptr;
};
// dev, mask, kind, Nq, Nk, g, groups, P, xcd, walk, cap, band_l, band_r
using SchedKey = std::tuple<int, int, int, int, int, int, int, int, int, int, int, int, int>;
std::map<SchedKey, DevSchedule> g_sched;
unsigned long long g_sched_clock = 0;
constexpr size_t kSchedCacheEntries = 64;

// Library-managed workspaces, one per (device, stream): calls on different
// streams never share semaphores or dQ accumulators.  Calls on one stream are
// ordered by the stream, so they can share one.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::map<std::pair<int, void*>, Workspace> g_ws;

// Per device: a host-visible word that the dQ finalize kernel sets when a
// workgroup of the persistent kernel gave up waiting on a semaphore (pinned,
// mapped host memory), and the co-resident workgroup capacity per kernel
// family (occupancy queries are not repeated per call).
struct DeviceState {
  int* sticky_host = nullptr;
  int* sticky_dev = nullptr;
  std::map<std::tuple<int, int, bool>, int> per_cu;  // (D, T, atomic) -> workgroups per CU
};
std::map<int, DeviceState> g_dev;

// Pinned word of `dev`, allocated on first use (nullptr if that fails).
int sticky_word(int dev, int** host, int** devp) {
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceState& d = g_dev[dev];
  if (!d.sticky_host) {
    void* h = nullptr;
    hipError_t e = hipHostMalloc(&h, 64, hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(error word)");
    void* dp = nullptr;
    e = hipHostGetDevicePointer(&dp, h, 0);
    if (e != hipSuccess) { (void)hipHostFree(h); return hip_fail(e, "hipHostGetDevicePointer(error word)"); }
    std::memset(h, 0, 64);
    d.sticky_host = (int*)h;
    d.sticky_dev = (int*)dp;
  }
  *host = d.sticky_host;
  *devp = d.sticky_dev;
  return DASH_OK;
}

// Takes (and clears) a give-up that an earlier call on `dev` recorded.
int take_sticky_error(int dev) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_dev.find(dev);
  if (it == g_dev.end() || !it->second.sticky_host) return DASH_OK;
  volatile int* w = it->second.sticky_host;
  if (*w == 0) return DASH_OK;
  *w = 0;
  return fail(DASH_ERR_TIMEOUT,
              "an earlier backward call on this device gave up waiting on a dQ semaphore; its dQ, dK and dV were "
              "set to NaN");
}

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
  if ((long long)Sq * D * 2 >= (1LL << 31))  // one head's query rows are addressed with 32-bit offsets
    return fail(DASH_ERR_UNSUPPORTED, "one head's query rows exceed 2 GiB");
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

// The allocation-free entry point keeps everything in the per-device static
// scratch array of noalloc.hip: [0, 256) the give-up word, then the
// workspace, then the step lists.  Per device it remembers whose step lists
// the scratch holds, so a repeated shape copies nothing.  Host copies of the
// lists it uploaded stay alive (the copies are asynchronous), at most
// kSchedCacheEntries of them; evicting one synchronises the device first.
constexpr size_t kNoallocStickyBytes = 256;
struct NoallocDevice {
  bool have_key = false;
  SchedKey key;
};
std::map<int, NoallocDevice> g_noalloc;
std::map<SchedKey, std::pair<std::shared_ptr<dash::Schedule>, unsigned long long>> g_noalloc_host;
unsigned long long g_noalloc_clock = 0;

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

int dash_device_info(int device, int* num_cu, int* num_xcd, int* lds_bytes, int* clock_khz) {
  DeviceInfo d;
  int st = device_info(device, &d);
  if (st) return st;
  if (num_cu) *num_cu = d.num_cu;
  if (num_xcd) *num_xcd = d.num_xcd;
  if (lds_bytes) *lds_bytes = d.lds;
  if (clock_khz) *clock_khz = d.clock_khz;
  return DASH_OK;
}

int dash_check_async_error(void* stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  bool noalloc_used = false;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    noalloc_used = g_noalloc.count(dev) != 0;
  }
  if (noalloc_used) {  // the allocation-free entry point's give-up word, in its scratch
    char* base = nullptr;
    e = dash::noalloc_scratch(dev, &base);
    if (e != hipSuccess) return hip_fail(e, "no-alloc scratch");
    int word = 0;
    e = hipMemcpy(&word, base, sizeof(int), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(no-alloc error word)");
    if (word) {
      const int zero = 0;
      e = hipMemcpy(base, &zero, sizeof(int), hipMemcpyHostToDevice);
      if (e != hipSuccess) return hip_fail(e, "hipMemcpy(no-alloc error word)");
      (void)take_sticky_error(dev);
      return fail(DASH_ERR_TIMEOUT,
                  "an earlier backward call on this device gave up waiting on a dQ semaphore; its dQ, dK and dV "
                  "were set to NaN");
    }
  }
  return take_sticky_error(dev);
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

int dash_schedule_simulate(const dash_schedule* s, double c, double r, uint64_t jitter_seed, double* makespan,
                           double* total_wait) {
  if (!s) return fail(DASH_ERR_INVALID_ARG, "null schedule");
  if (!(c >= 0.0) || !(r >= 0.0)) return fail(DASH_ERR_INVALID_ARG, "step costs must be non-negative");
  if (!dash::simulate_schedule(s->s, c, r, jitter_seed, makespan, total_wait))
    return fail(DASH_ERR_INVALID_SCHEDULE, "deadlock");
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
  Range r("dash_attn_fwd");
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

int dash_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D, int mask, int schedule, size_t* bytes) {
  if (!bytes) return fail(DASH_ERR_INVALID_ARG, "null output");
  if (B < 0 || Hq <= 0 || Hkv <= 0 || S < 0 || D <= 0) return fail(DASH_ERR_INVALID_ARG, "sizes must not be negative");
  if (mask != DASH_MASK_FULL && mask != DASH_MASK_CAUSAL) return fail(DASH_ERR_INVALID_ARG, "unknown mask");
  if (schedule < DASH_SCHED_SERIAL || schedule > DASH_SCHED_AUTO) return fail(DASH_ERR_INVALID_ARG, "unknown schedule");
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

// Everything a backward call decides before it touches a buffer: validated
// sizes and options, the tile grid, the schedule, and the workspace layout.
struct BwdPlan {
  dash_bwd_opts op;
  int dev = 0;
  DeviceInfo di;
  TileGrid tg;
  int B = 0, Hq = 0, Hkv = 0, Sq = 0, Sk = 0, D = 0;
  int T = 0, P = 0, g = 1, groups = 1, schedule = 0, xcd = 1, walk = -1, band_l = -1, band_r = -1;
  bool atomic = false, empty = false;
  float scale = 0.f;
  long long kv_elems = 0;
  WsLayout L;
  SchedKey key;
};

// Validates a backward call and fills `pl` (no device work, no allocation).
// pl->empty: no query rows, only dK = dV = 0 to write.
static int bwd_plan(const void* const* ptrs, int B, int Hq, int Hkv, int Sq, int Sk, int D, float softmax_scale,
                    const Mask& mask, int schedule, const dash_bwd_opts* opts, BwdPlan* pl) {
  int st = check_sizes(B, Hq, Hkv, Sq, Sk, D, mask);
  if (st != DASH_OK && st != kEmpty) return st;
  if (schedule < DASH_SCHED_SERIAL || schedule > DASH_SCHED_AUTO) return fail(DASH_ERR_INVALID_ARG, "unknown schedule");
  pl->B = B;
  pl->Hq = Hq;
  pl->Hkv = Hkv;
  pl->Sq = Sq;
  pl->Sk = Sk;
  pl->D = D;
  pl->kv_elems = (long long)B * Hkv * Sk * D;
  if (st == kEmpty) {
    pl->empty = true;
    if (pl->kv_elems == 0) return DASH_OK;
    return check_ptrs(ptrs + 7, 2);  // dk, dv
  }
  st = check_ptrs(ptrs, 9);
  if (st) return st;
  dash_bwd_opts& op = pl->op;
  std::memset(&op, 0, sizeof(op));
  if (opts) {
    if (opts->struct_size == 0 || opts->struct_size > sizeof(dash_bwd_opts))
      return fail(DASH_ERR_INVALID_ARG, "dash_bwd_opts.struct_size must be sizeof(dash_bwd_opts)");
    std::memcpy(&op, opts, opts->struct_size);
  }
  hipError_t e = hipGetDevice(&pl->dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  st = device_info(pl->dev, &pl->di);
  if (st) return st;

  const int T = op.tile ? op.tile : (std::min(Sq, Sk) < 512 ? 64 : 128);
  if (T != 64 && T != 128) return fail(DASH_ERR_UNSUPPORTED, "tile must be 64 or 128");
  pl->T = T;
  pl->tg = tile_grid(Sq, Sk, T, mask.aligned());
  const int Nq = pl->tg.Nq, Nk = pl->tg.Nk;
  // band extents in tiles: a window of w rows reaches ceil(w / T) tiles off the diagonal tile
  pl->band_l = mask.kind == dash::kMaskBand && mask.wl >= 0 ? (mask.wl + T - 1) / T : -1;
  pl->band_r = mask.kind == dash::kMaskBand && mask.wr >= 0 ? (mask.wr + T - 1) / T : -1;
  if (op.num_workgroups < 0) return fail(DASH_ERR_INVALID_ARG, "negative workgroup count");
  if (op.max_gang < 0) return fail(DASH_ERR_INVALID_ARG, "negative gang cap");
  pl->P = op.num_workgroups > 0 ? op.num_workgroups : pl->di.num_cu;
  pl->g = Hq / Hkv;
  if (schedule == DASH_SCHED_AUTO) {
    int cap = 0;
    std::string err = dash::choose_schedule(mask.kind, Nq, Nk, D, pl->g, pl->P, &schedule, &cap, pl->band_l, pl->band_r);
    if (!err.empty()) return fail(DASH_ERR_INVALID_ARG, err);
    if (op.max_gang == 0) op.max_gang = cap;
  }
  pl->schedule = schedule;
  pl->groups = B * Hkv;
  pl->atomic = schedule == DASH_SCHED_ATOMIC;
  if (op.debug_delay_seed && pl->atomic) return fail(DASH_ERR_INVALID_ARG, "delay injection needs a deterministic schedule");
  pl->xcd = op.xcd_local >= 0 ? 1 : 0;
  pl->walk = pl->atomic ? op.atomic_walk : -1;
  pl->scale = default_scale(softmax_scale, D);
  pl->L = ws_layout(B, Hq, Sq, pl->tg.Sw, D);
  pl->key = SchedKey{pl->dev, mask.kind, schedule, Nq, Nk, pl->g, pl->groups, pl->P, pl->xcd,
                     pl->atomic ? (pl->walk < 0 ? -1 : pl->walk) : -1, op.max_gang, pl->band_l, pl->band_r};

  // Co-residency: the semaphore waits need every workgroup resident at once.
  if (!pl->atomic) {
    int per_cu = -1;
    {
      std::lock_guard<std::mutex> lk(g_mu);
      auto& m = g_dev[pl->dev].per_cu;
      auto it = m.find(std::make_tuple(D, T, false));
      if (it != m.end()) per_cu = it->second;
    }
    if (per_cu < 0) {
      e = dash::bwd_kernel_per_cu(D, T, false, &per_cu);
      if (e != hipSuccess) return hip_fail(e, "occupancy query");
      std::lock_guard<std::mutex> lk(g_mu);
      g_dev[pl->dev].per_cu[std::make_tuple(D, T, false)] = per_cu;
    }
    if ((long long)per_cu * pl->di.num_cu < pl->P)
      return fail(DASH_ERR_UNSUPPORTED, "persistent grid larger than the co-resident capacity");
  }
  return DASH_OK;
}

// Builds and validates the step lists of a plan (host memory only).
static int build_host_schedule(const BwdPlan& pl, int mask_kind, std::shared_ptr<dash::Schedule>* out) {
  Range r("dash: build and validate step lists");
  auto s = std::make_shared<dash::Schedule>();
  std::string err = dash::build_schedule(mask_kind, pl.schedule, pl.tg.Nq, pl.tg.Nk, pl.g, pl.groups, pl.P, pl.xcd != 0,
                                         pl.walk, pl.op.max_gang, s.get(), pl.band_l, pl.band_r);
  if (!err.empty()) return fail(DASH_ERR_UNSUPPORTED, err);
  err = dash::validate_schedule(*s);
  if (!err.empty()) return fail(DASH_ERR_INVALID_SCHEDULE, err);
  if (log_on())
    std::fprintf(stderr, "[dash] step lists: schedule %d, %d x %d tiles, g %d, %d groups, %d workgroups, %zu steps\n",
                 pl.schedule, pl.tg.Nq, pl.tg.Nk, pl.g, pl.groups, pl.P, s->steps.size());
  *out = std::move(s);
  return DASH_OK;
}

// The plan's step lists on its device: from the cache, or built, validated
// and uploaded on `strm` (asynchronously; the host copy stays in the cache).
static int device_schedule(const BwdPlan& pl, int mask_kind, hipStream_t strm, DevSchedule* out) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_sched.find(pl.key);
  if (it == g_sched.end()) {
    if (g_sched.size() >= kSchedCacheEntries) {
      auto lru = g_sched.begin();
      for (auto j = g_sched.begin(); j != g_sched.end(); ++j)
        if (j->second.last_use < lru->second.last_use) lru = j;
      hipError_t e = hipDeviceSynchronize();  // queued kernels may still read the evicted lists
      if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
      (void)hipFree(lru->second.steps);
      (void)hipFree(lru->second.offsets);
      if (lru->second.uploaded) (void)hipEventDestroy(lru->second.uploaded);
      g_sched.erase(lru);
    }
    std::shared_ptr<dash::Schedule> s;
    int st = build_host_schedule(pl, mask_kind, &s);
    if (st) return st;
    Range r("dash: upload step lists");
    DevSchedule d;
    d.num_steps = (long long)s->steps.size();
    hipError_t e = hipMalloc((void**)&d.steps, std::max<size_t>(16, s->steps.size() * sizeof(dash::StepRec)));
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(steps)");
    e = hipMalloc((void**)&d.offsets, s->offsets.size() * sizeof(int32_t));
    if (e != hipSuccess) { (void)hipFree(d.steps); return hip_fail(e, "hipMalloc(offsets)"); }
    e = hipMemcpyAsync(d.steps, s->steps.data(), s->steps.size() * sizeof(dash::StepRec), hipMemcpyHostToDevice, strm);
    if (e == hipSuccess)
      e = hipMemcpyAsync(d.offsets, s->offsets.data(), s->offsets.size() * sizeof(int32_t), hipMemcpyHostToDevice, strm);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&d.uploaded, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(d.uploaded, strm);
    if (e != hipSuccess) {
      (void)hipFree(d.steps);
      (void)hipFree(d.offsets);
      if (d.uploaded) (void)hipEventDestroy(d.uploaded);
      return hip_fail(e, "hipMemcpyAsync(schedule)");
    }
    d.upload_stream = strm;
    d.host = std::move(s);
    it = g_sched.emplace(pl.key, std::move(d)).first;
  }
  DevSchedule& d = it->second;
  if (d.uploaded && d.upload_stream != strm) {
    // The lists may still be in flight on the uploading stream.
    hipError_t e = hipEventQuery(d.uploaded);
    if (e == hipSuccess) {
      (void)hipEventDestroy(d.uploaded);
      d.uploaded = nullptr;
    } else if (e == hipErrorNotReady) {
      e = hipStreamWaitEvent(strm, d.uploaded, 0);
      if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(schedule upload)");
    } else {
      return hip_fail(e, "hipEventQuery(schedule upload)");
    }
  }
  d.last_use = ++g_sched_clock;
  *out = d;
  return DASH_OK;
}

// Enqueues the three kernels of a planned call on `strm` with workspace `ws`
// (pl.L.total bytes) and step lists `ds`; `sticky` is the device address of
// the host-visible give-up word (may be null).
static int bwd_enqueue(const BwdPlan& pl, const void* const* ptrs, const Mask& mask, char* ws, const DevSchedule& ds,
                       int* sticky, hipStream_t strm) {
  Range r("dash: enqueue backward kernels");
  if (log_on())
    std::fprintf(stderr,
                 "[dash] bwd B %d Hq %d Hkv %d Sq %d Sk %d D %d mask %d window (%d, %d) schedule %d tile %d "
                 "workgroups %d gang cap %d workspace %zu bytes\n",
                 pl.B, pl.Hq, pl.Hkv, pl.Sq, pl.Sk, pl.D, mask.kind, mask.wl, mask.wr, pl.schedule, pl.T, pl.P,
                 pl.op.max_gang, (size_t)pl.L.total);
  const void *q = ptrs[0], *k = ptrs[1], *v = ptrs[2], *o = ptrs[3], *dO = ptrs[4];
  const float* lse = (const float*)ptrs[5];
  void *dq = const_cast<void*>(ptrs[6]), *dk = const_cast<void*>(ptrs[7]), *dv = const_cast<void*>(ptrs[8]);
  const dash_bwd_opts& op = pl.op;
  const WsLayout& L = pl.L;
  const int D = pl.D;
  float* ws_dq = (float*)(ws + L.ws_dq);
  float* delta = (float*)(ws + L.delta);
  int* sem = (int*)(ws + L.sem);
  int* err = (int*)(ws + L.err);
  const long long rows = (long long)pl.B * pl.Hq * pl.Sq;
  const long long n_sem = (long long)((L.err - L.sem) / 4) + 4;  // semaphores, padding and the error word
  const long long ws_elems = (long long)pl.B * pl.Hq * pl.tg.Sw * D;
  hipError_t e = dash::launch_delta(o, dO, delta, rows, D, sem, n_sem, pl.atomic ? ws_dq : nullptr,
                                    pl.atomic ? ws_elems : 0, strm);
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
  bl.xcc = op.xcc_id_out;
  bl.delay_seed = op.debug_delay_seed;
  const unsigned long long budget_cycles = op.spin_timeout_cycles ? op.spin_timeout_cycles : (1ULL << 33);
  // wait budget in 100 MHz real-time ticks, from shader cycles at the device clock
  bl.spin_ticks = (long long)((double)budget_cycles * 1e5 / std::max(1, pl.di.clock_khz));
  if (bl.spin_ticks < 1) bl.spin_ticks = 1;
  bl.scale = pl.scale;
  bl.Sq = pl.Sq;
  bl.Sk = pl.Sk;
  bl.D = D;
  bl.T = pl.T;
  bl.g = pl.g;
  bl.wl = mask.wl;
  bl.wr = mask.wr;
  bl.qshift = pl.tg.qshift;
  bl.nblk = pl.tg.Sw / 64;
  bl.diag_off = pl.tg.diag_off;
  bl.P = pl.P;
  bl.atomic = pl.atomic;
  // Key/value tiles that no query tile sees have no chain: their dK/dV are zero.
  if (pl.band_l >= 0 && pl.tg.diag_off > pl.band_l) {
    int st = zero_bf16(dk, pl.kv_elems, D, strm);
    if (!st) st = zero_bf16(dv, pl.kv_elems, D, strm);
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
  dash::FinalizeLaunch fl;
  fl.ws = ws_dq;
  fl.dq = dq;
  fl.dk = dk;
  fl.dv = dv;
  fl.err = err;
  fl.sticky = sticky;
  fl.ws_elems = ws_elems;
  fl.kv_elems = pl.kv_elems;
  fl.D = D;
  fl.scale = pl.scale;
  fl.atomic_layout = pl.atomic;
  fl.nblk = pl.tg.Sw / 64;
  fl.qshift = pl.tg.qshift;
  fl.Sq = pl.Sq;
  e = dash::launch_dq_finalize(fl, strm);
  if (e != hipSuccess) return hip_fail(e, "finalize launch");

  if (op.sync_check) {
    e = hipStreamSynchronize(strm);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    int h_err = 0;
    e = hipMemcpy(&h_err, err, sizeof(int), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(error word)");
    if (h_err) {
      (void)take_sticky_error(pl.dev);  // reported here, not again by the next call
      return fail(DASH_ERR_TIMEOUT, "a workgroup timed out waiting on a dQ semaphore; dQ, dK and dV were set to NaN");
    }
  }
  return DASH_OK;
}

static int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                    void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int D, float softmax_scale,
                    const Mask& mask, int schedule, const dash_bwd_opts* opts, void* stream) {
  Range r("dash_attn_bwd");
  const void* ptrs[] = {q, k, v, o, dO, lse, dq, dk, dv};
  BwdPlan pl;
  int st = bwd_plan(ptrs, B, Hq, Hkv, Sq, Sk, D, softmax_scale, mask, schedule, opts, &pl);
  if (st) return st;
  hipStream_t strm = (hipStream_t)stream;
  if (pl.empty) {
    // No query rows: dQ is empty and dK = dV = 0 (no key receives any gradient).
    if (pl.kv_elems == 0) return DASH_OK;
    st = zero_bf16(dk, pl.kv_elems, D, strm);
    return st ? st : zero_bf16(dv, pl.kv_elems, D, strm);
  }
  st = take_sticky_error(pl.dev);
  if (st) return st;
  int *sticky_host = nullptr, *sticky_dev = nullptr;
  st = sticky_word(pl.dev, &sticky_host, &sticky_dev);
  if (st) return st;
  DevSchedule ds;
  st = device_schedule(pl, mask.kind, strm, &ds);
  if (st) return st;

  char* ws = nullptr;
  const dash_bwd_opts& op = pl.op;
  if (op.workspace) {
    if (reinterpret_cast<uintptr_t>(op.workspace) % 256) return fail(DASH_ERR_WORKSPACE, "workspace not 256-byte aligned");
    if (op.workspace_bytes < pl.L.total) return fail(DASH_ERR_WORKSPACE, "workspace too small");
    ws = (char*)op.workspace;
  } else {
    std::lock_guard<std::mutex> lk(g_mu);
    Workspace& w = g_ws[std::make_pair(pl.dev, stream)];
    if (w.bytes < pl.L.total) {
      // The previous buffer may still be in use by work queued on this stream.
      if (w.ptr) {
        hipError_t e = hipStreamSynchronize(strm);
        if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
        (void)hipFree(w.ptr);
        w.ptr = nullptr;
        w.bytes = 0;
      }
      hipError_t e = hipMalloc(&w.ptr, pl.L.total);
      if (e != hipSuccess) return hip_fail(e, "hipMalloc(workspace)");
      w.bytes = pl.L.total;
    }
    ws = (char*)w.ptr;
  }
  return bwd_enqueue(pl, ptrs, mask, ws, ds, sticky_dev, strm);
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

int dash_attn_bwd_qk_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                             const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk,
                             int D, float softmax_scale, int mask, int schedule, const dash_bwd_opts* opts,
                             void* stream) {
  Range r("dash_attn_bwd_qk_noalloc");
  const void* ptrs[] = {q, k, v, o, dO, lse, dq, dk, dv};
  const Mask mk = mask_from_enum(mask);
  BwdPlan pl;
  int st = bwd_plan(ptrs, B, Hq, Hkv, Sq, Sk, D, softmax_scale, mk, schedule, opts, &pl);
  if (st) return st;
  hipStream_t strm = (hipStream_t)stream;
  if (pl.empty) {
    if (pl.kv_elems == 0) return DASH_OK;
    st = zero_bf16(dk, pl.kv_elems, D, strm);
    return st ? st : zero_bf16(dv, pl.kv_elems, D, strm);
  }
  if (pl.op.workspace)
    return fail(DASH_ERR_INVALID_ARG, "the allocation-free entry point uses its own scratch: opts->workspace must be NULL");

  // Step lists on the host (built and validated on a shape's first call).
  std::shared_ptr<dash::Schedule> hs;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_noalloc_host.find(pl.key);
    if (it != g_noalloc_host.end()) {
      it->second.second = ++g_noalloc_clock;
      hs = it->second.first;
    }
  }
  if (!hs) {
    st = build_host_schedule(pl, mk.kind, &hs);
    if (st) return st;
  }
  const size_t steps_bytes = hs->steps.size() * sizeof(dash::StepRec);
  const size_t off_ws = kNoallocStickyBytes;
  const size_t off_steps = align256(off_ws + pl.L.total);
  const size_t off_offsets = align256(off_steps + steps_bytes);
  const size_t need = off_offsets + hs->offsets.size() * sizeof(int32_t);
  if (need > dash::kNoallocScratchBytes)
    return fail(DASH_ERR_WORKSPACE, "problem needs " + std::to_string(need) +
                                        " bytes of scratch; the allocation-free entry point has " +
                                        std::to_string(dash::kNoallocScratchBytes));
  char* base = nullptr;
  hipError_t e = dash::noalloc_scratch(pl.dev, &base);
  if (e != hipSuccess) return hip_fail(e, "no-alloc scratch (hipGetSymbolAddress)");

  {
    std::lock_guard<std::mutex> lk(g_mu);
    NoallocDevice& nd = g_noalloc[pl.dev];
    if (!nd.have_key || !(nd.key == pl.key)) {
      if (!g_noalloc_host.count(pl.key)) {
        if (g_noalloc_host.size() >= kSchedCacheEntries) {
          auto lru = g_noalloc_host.begin();
          for (auto j = g_noalloc_host.begin(); j != g_noalloc_host.end(); ++j)
            if (j->second.second < lru->second.second) lru = j;
          e = hipDeviceSynchronize();  // its copy may still be in flight
          if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
          g_noalloc_host.erase(lru);
        }
        g_noalloc_host.emplace(pl.key, std::make_pair(hs, ++g_noalloc_clock));
      }
      e = hipMemcpyAsync(base + off_steps, hs->steps.data(), steps_bytes, hipMemcpyHostToDevice, strm);
      if (e == hipSuccess)
        e = hipMemcpyAsync(base + off_offsets, hs->offsets.data(), hs->offsets.size() * sizeof(int32_t),
                           hipMemcpyHostToDevice, strm);
      if (e != hipSuccess) {
        nd.have_key = false;
        return hip_fail(e, "hipMemcpyAsync(no-alloc step lists)");
      }
      nd.have_key = true;
      nd.key = pl.key;
    }
  }
  DevSchedule ds;
  ds.steps = (int32_t*)(base + off_steps);
  ds.offsets = (int32_t*)(base + off_offsets);
  ds.num_steps = (long long)hs->steps.size();
  st = bwd_enqueue(pl, ptrs, mk, base + off_ws, ds, (int*)base, strm);
  if (st == DASH_ERR_TIMEOUT) {  // reported by sync_check: clear the give-up word, it is not reported again
    const int zero = 0;
    (void)hipMemcpy(base, &zero, sizeof(int), hipMemcpyHostToDevice);
  }
  return st;
}

}  // extern "C"
