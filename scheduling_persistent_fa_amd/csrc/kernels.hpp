// Host-side launchers of the gfx950 attention kernels (kernels.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace dash {

struct BwdLaunch {
  const void* q;
  const void* k;
  const void* v;
  const void* dO;
  const float* lse;
  const float* delta;
  float* ws;           // fp32 dQ accumulator, fragment order
  int* sem;            // one per (query head, 64-row block)
  int* err;            // error word (non-zero: a wait timed out)
  float* dummy;        // 8 x 1024 floats absorbing writes with no destination
  void* dk;
  void* dv;
  const int32_t* steps;    // 4 ints per step
  const int32_t* offsets;  // P + 1
  unsigned long long* stall;
  int* xcc;                // optional: per workgroup, the chiplet (XCC) it ran on
  uint32_t delay_seed;     // non-zero: seeded sleeps around the dQ waits and releases (testing only)
  long long spin_ticks;    // wait budget in 100 MHz real-time ticks
  float scale;
  int Sq, Sk, D, T, g, P;
  int wl, wr;    // window around the bottom-right diagonal in rows (-1: unbounded); causal = (-1, 0)
  int qshift;    // virtual query row = query row + qshift (aligns query tiles with key/value tiles)
  int nblk;      // 64-row dQ workspace blocks per query head
  int diag_off;  // windowed masks: query tile qi's diagonal runs through key/value tile qi + diag_off
  bool atomic;
};

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                      int Sq, int Sk, int D, float scale, int wl, int wr, hipStream_t st);
hipError_t launch_delta(const void* o, const void* dO, float* delta, long long rows, int D, int* zero_i32,
                        long long n_zero_i32, float* zero_f32, long long n_zero_f32, hipStream_t st);
hipError_t launch_bwd(const BwdLaunch& L, hipStream_t st);
// Co-resident workgroups per compute unit of the persistent kernel family
// (the minimum over its variants).
hipError_t bwd_kernel_per_cu(int D, int T, bool atomic, int* per_cu);

struct FinalizeLaunch {
  const float* ws;     // fp32 dQ accumulator, fragment order
  void* dq;
  void* dk;            // written with NaN (with dv and dq) when *err is set
  void* dv;
  const int* err;      // error word of the persistent kernel
  int* sticky;         // optional host-visible word set to 1 when *err is set
  long long ws_elems;  // workspace floats
  long long kv_elems;  // elements of dk (and of dv)
  int D;
  float scale;
  bool atomic_layout;
  int nblk, qshift, Sq;
};
hipError_t launch_dq_finalize(const FinalizeLaunch& F, hipStream_t st);

// Scratch of the allocation-free entry point (noalloc.hip): a static device
// array of this many bytes per GPU.
constexpr size_t kNoallocScratchBytes = size_t(144) << 20;
// Device address of `dev`'s scratch array; `dev` must be the current device.
// The first call per device resolves it with hipGetSymbolAddress.
hipError_t noalloc_scratch(int dev, char** out);

}  // namespace dash
