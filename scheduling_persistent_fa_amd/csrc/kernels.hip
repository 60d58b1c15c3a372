// HIP kernels for softmax attention forward and the DASH deterministic
// backward pass on gfx950 (MI355X, CDNA4).
//
// Sources (cited by page title and section):
//   [summary] "Resumo Técnico: DASH – Agendamento de Atenção Determinístico
//             para Treinamento de LLM de Alto Rendimento" (gist.science)
//   [news]    "DASH如何革新LLM确定性训练" (pwwt.cn)
//
// Matrix-core conventions (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) .. +7
//   B (16 x 32): lane l holds col l%32, k = 8*(l/32) .. +7
//   C (32 x 32): lane l, register r holds col l%32, row 8*(r/4) + 4*(l/32) + r%4
// Contractions may use any permutation of k as long as A and B agree.  A C
// tile whose rows are the contraction index therefore feeds the next MFMA
// directly: registers 8e..8e+7 form the operand for rows
// 16e + {4h..4h+3, 8+4h..8+4h+3} (h = l/32), and the partner operand is read
// from LDS with the gfx950 transposing read ds_read_b64_tr_b16, which gives
// each lane four consecutive rows of one column of a 4 x 16 row-major block.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "kernels.hpp"

namespace dash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Four bf16 values, one column of a 4 x 16 block, per lane (see header).
__device__ __forceinline__ bf16x4 lds_tr4(const LDS char* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)p);
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 lds_row8(const LDS char* p) { return *(const LDS bf16x8*)p; }

// Operand from two transposing reads: rows row0 + (l%16)/4 and row0 + 8 + (l%16)/4
// (pitch in bytes), columns col0 + 16*((l/16)%2) + 4*(l%4) (bf16 elements).  Lane
// l receives rows row0..row0+3 then row0+8..row0+11 of column col0 + l%32: the
// k-permutation of a C tile reused as an operand.
__device__ __forceinline__ bf16x8 lds_tr8_split(const LDS char* base, int pitch_bytes, int row0, int col0,
                                                int lane) {
  const int r = row0 + ((lane & 15) >> 2);
  const int c = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const LDS char* p = base + r * pitch_bytes + c * 2;
  return cat8(lds_tr4(p), lds_tr4(p + 8 * pitch_bytes));
}

// Operand from two transposing reads with the lane part of the address already
// applied, p = block + ((l%16)/4) * pitch + (16*((l/16)%2) + 4*(l%4)) * 2: lane l
// receives rows 0..3 then 4..7 of column l%32 of the block.
__device__ __forceinline__ bf16x8 lds_tr8_at(const LDS char* p, int pitch_bytes) {
  return cat8(lds_tr4(p), lds_tr4(p + 4 * pitch_bytes));
}

// Device-scope (sc1) 16-byte accesses to one dQ workspace tile of 4 KiB.
// sc1 makes a load or store coherent across the chiplets: it bypasses the
// chiplet-local caches that other chiplets cannot see.
constexpr int kDeviceScope = 16;  // cache-policy operand of the buffer intrinsics: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const float* tile) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(tile), (short)0, 4096, 0x00020000);
}

// A pointer that is the same in every lane, read from the first lane so that
// the compiler keeps it in scalar registers (a descriptor built from it then
// needs no per-lane loop).
template <class X>
__device__ __forceinline__ X* uniform_ptr(X* p) {
  const unsigned long long u = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
  return (X*)(((unsigned long long)hi << 32) | lo);
}

// Keeps a value opaque to the optimiser, so that addresses formed from it
// fold their constant parts into instruction offsets instead of being
// precomputed and held in registers.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Waits until every vector memory access of this wave has completed.  The
// inline-asm wait orders the surrounding memory accesses (memory clobber); the
// builtin repeats it for the compiler's own wait-count tracking, which does not
// read inline asm.  Without it a later use of a load issued before this point
// gets a wait for everything issued since, including a semaphore store.
__device__ __forceinline__ void wait_vmem_all() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt left at their maxima
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int first) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[first + e];
  return r;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------
// Forward: O = softmax(scale Q K^T) V, LSE (natural log).  One workgroup per
// (32*NW query rows, query head); each wave keeps 32 query rows of Q in
// registers and computes S^T = K Q^T so that a lane owns one query row; the
// online softmax ([summary] §2: the backward consumes the forward's LSE) is
// then per lane plus one exchange between the two half-waves.
//
// Masks are windows around the bottom-right diagonal: query row i sees key j
// when -wl <= j - (i + Sk - Sq) <= wr, with kUnbounded for an open side (full
// mask: both open; causal: wr = 0).
// ---------------------------------------------------------------------------
constexpr int kUnbounded = 1 << 29;

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 1) void fwd_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                         const __bf16* __restrict__ v, __bf16* __restrict__ o,
                                                         float* __restrict__ lse, int Hq, int g, int Sq, int Sk,
                                                         float scale_log2, int wl, int wr) {
  constexpr int KVT = 64;               // key/value rows per LDS tile
  constexpr int PITCH = 2 * D + 48;     // bytes per LDS row: 16-byte row reads and transposing reads conflict-free
  constexpr int TILE_BYTES = KVT * PITCH;
  constexpr int DC = D / 16;            // 16-wide d chunks
  constexpr int DB = D / 32;            // 32-wide d blocks
  constexpr int NT = 64 * NW;
  constexpr int CHUNKS = KVT * D / 8;   // 16-byte chunks per K or V tile
  constexpr int CPT = CHUNKS / NT;      // chunks per thread
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE_BYTES];
  LDS char* base = (LDS char*)smem;

  const int lane = lane_id(), w = wave_id(), h2 = lane >> 5, c32 = lane & 31;
  const int head = blockIdx.y;  // b * Hq + hq
  const int kvh = head / g;
  const int q_base = blockIdx.x * 32 * NW;
  const int q_row = q_base + 32 * w + c32;  // this lane's query row (past Sq on a ragged last block)
  const int q_ld = min(q_row, Sq - 1);      // rows past Sq read a valid row and are not stored
  const __bf16* qh = q + (size_t)head * Sq * D;
  const __bf16* kh = k + (size_t)kvh * Sk * D;
  const __bf16* vh = v + (size_t)kvh * Sk * D;
  const int off = Sk - Sq;  // the diagonal key of query row i is i + off

  bf16x8 qb[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) qb[c] = *(const bf16x8*)(qh + (size_t)q_ld * D + 16 * c + 8 * h2);

  // Key/value tiles of 64 rows; the last one may be partial (rows past Sk
  // read row Sk - 1 and are masked out of the softmax).
  const int kv_tiles = (Sk + KVT - 1) / KVT;
  // tiles holding a key some row of this workgroup sees
  const int t_beg = wl >= kUnbounded ? 0 : max(0, (q_base + off - wl) / KVT);
  const int t_end = wr >= kUnbounded ? kv_tiles : min(kv_tiles, (q_base + 32 * NW - 1 + off + wr) / KVT + 1);
  const bool windowed = wl < kUnbounded || wr < kUnbounded;

  bf16x8 pk[CPT], pv[CPT];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = threadIdx.x + i * NT, row = min(t * KVT + ch / (D / 8), Sk - 1), col = (ch % (D / 8)) * 8;
      pk[i] = *(const bf16x8*)(kh + (size_t)row * D + col);
      pv[i] = *(const bf16x8*)(vh + (size_t)row * D + col);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = threadIdx.x + i * NT, row = ch / (D / 8), col = (ch % (D / 8)) * 8;
      *(LDS bf16x8*)(base + (2 * buf) * TILE_BYTES + row * PITCH + col * 2) = pk[i];
      *(LDS bf16x8*)(base + (2 * buf + 1) * TILE_BYTES + row * PITCH + col * 2) = pv[i];
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_part = 0.f;

  load_tile(t_beg);
  store_tile(0);
  __syncthreads();
  for (int t = t_beg; t < t_end; ++t) {
    const int buf = (t - t_beg) & 1;
    const LDS char* sk = base + (2 * buf) * TILE_BYTES;
    const LDS char* sv = base + (2 * buf + 1) * TILE_BYTES;
    if (t + 1 < t_end) load_tile(t + 1);
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < DC; ++c) s[kb] = mfma32(lds_row8(sk + (kb * 32 + c32) * PITCH + (16 * c + 8 * h2) * 2), qb[c], s[kb]);
    }
    float mt = -INFINITY;
    const bool tail = (t + 1) * KVT > Sk;  // the ragged last tile
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[kb][r] * scale_log2;
        if (windowed || tail) {
          const int kv = t * KVT + kb * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
          const int d = kv - (q_row + off);
          if (d > wr || d < -wl || kv >= Sk) x = -INFINITY;
        }
        s[kb][r] = x;
        mt = fmaxf(mt, x);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // A window can hide whole tiles from a row: while the row has seen no key
    // its maximum stays -inf, and 0 stands in for it in the exponents so that
    // no inf - inf occurs (its P and its rescaling factor are then 0).
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[kb][r] - m_use);
        s[kb][r] = p;
        rs += p;
      }
    l_part = l_part * alpha + rs;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    // O^T[d][q] += V^T[d][kv] P^T[kv][q]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bf16x8 bp = pack8(s[kb], 8 * e);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[db] = mfma32(lds_tr8_split(sv, PITCH, kb * 32 + 16 * e + 4 * h2, db * 32, lane), bp, acc[db]);
      }
    if (t + 1 < t_end) {
      __syncthreads();  // everyone done with the other buffer's previous tile
      store_tile(buf ^ 1);
      __syncthreads();
    }
  }
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  const float inv = 1.f / l_tot;
  if (q_row >= Sq) return;
  __bf16* oh = o + (size_t)head * Sq * D + (size_t)q_row * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 out;
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = (__bf16)(acc[db][4 * j + i] * inv);
      *(bf16x4*)(oh + db * 32 + 8 * j + 4 * h2) = out;
    }
  if (h2 == 0) lse[(size_t)head * Sq + q_row] = (m_run + __log2f(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------
// Backward preprocess: Delta_i = sum_d dO_id O_id (fp32), and zeroing of the
// semaphores, the error word and (for the atomic variant) the dQ workspace.
// Cleared with stores from this kernel rather than memset so that the whole
// backward can be captured into a graph.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const __bf16* __restrict__ o, const __bf16* __restrict__ dO,
                                                     float* __restrict__ delta, long long rows,
                                                     int* __restrict__ zero_i32, long long n_zero_i32,
                                                     float* __restrict__ zero_f32, long long n_zero_f32) {
  constexpr int TPR = D / 8;  // threads per row
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gid / TPR;
  float acc = 0.f;
  if (row < rows) {
    const int col = (int)(gid % TPR) * 8;
    const bf16x8 a = *(const bf16x8*)(o + row * D + col);
    const bf16x8 b = *(const bf16x8*)(dO + row * D + col);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < rows && (gid % TPR) == 0) delta[row] = acc;
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = gid; i < n_zero_i32; i += stride) zero_i32[i] = 0;
  for (long long i = gid * 4; i < n_zero_f32; i += stride * 4) *(f32x4*)(zero_f32 + i) = f32x4{};
}

// Q / dO / K rows (2D bytes) are stored in LDS without padding, with 16-byte
// chunk c of row r at chunk c ^ lds_swizzle<D>(r).  Sixteen consecutive rows
// then put one logical chunk into sixteen distinct 16-byte bank groups (the
// 16-byte row reads are conflict-free), and four consecutive rows from a
// multiple of four put one 64-byte block into four distinct bank groups of
// four (the transposing reads take 2 cycles instead of 4).  For D = 128 the
// row's low two bits pick the 64-byte block and the next two the chunk in it;
// for D = 64 (two rows per 256-byte bank line) bit 1 picks the block and bits
// 2-3 the chunk.
template <int D>
__device__ __forceinline__ int lds_swizzle(int r) {
  if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// ---------------------------------------------------------------------------
// LDS row pitches.  gfx950's LDS has 64 four-byte banks.  A 16-byte row read
// serves 16 lanes (16 consecutive rows) per cycle and is conflict-free when
// the pitch in words is 4 x odd modulo 64, as for the 144-byte P^T / dS^T rows
// (64 columns plus padding).  A transposing read serves 32 lanes (4 rows x 64
// bytes) per cycle; at such a pitch two of the four rows share banks, so it
// takes 4 cycles instead of 2 (only pitches of 64 bytes modulo 256 avoid that,
// and those make the row reads conflict), and the 8-byte P^T / dS^T stores
// take 16 cycles instead of 8.  The Q / dO / K rows use the swizzle above
// instead of padding, which makes both kinds of read conflict-free; measured
// against padded rows, that gains about 1%, so the conflicts are not what
// bounds the kernel.
// ---------------------------------------------------------------------------
// Persistent backward.  One workgroup per compute unit walks its step list
// (built on the host); each chain (key/value tile x its query heads) runs
// contiguously with dK/dV in registers ([summary] §2.1).  Per 64-row query
// block the workgroup adds its dQ partial into the fp32 workspace either in
// the order fixed by the step's ordinal -- waiting on a per-block semaphore
// in global memory -- or, for the non-deterministic ceiling, with fp32
// atomic adds.
//
// Work split.  The T key/value rows of a tile are held by T/32 wave pairs
// (two waves per SIMD).  Both waves of pair p keep K and V rows 32p..32p+31
// as MFMA operands; wave h of the pair computes S and dP for query rows
// 32h..32h+31 of the 64-row block, then both write P^T and dS^T (bf16) to
// LDS, and wave h accumulates the d columns [h*D/2, (h+1)*D/2) of dK and dV
// over all 64 query rows.  The 2*D/32 C tiles of the block's dQ partial are
// spread over the waves.
//
// Ragged lengths and windows.  Query tile qi covers the virtual rows
// qi*T .. qi*T+T-1, virtual row = query row + qshift; qshift > 0 only for a
// windowed (causal or banded) mask whose offset Sk - Sq is not a multiple of
// T, and it aligns the query tiles with the key/value tiles so that the
// diagonal crosses tile pair (qi, qi + diag_off) at the same local positions
// as in the square case.  A tile pair is masked element-wise only when some
// of its pairs fall outside the window, or it is the ragged last tile.
// Virtual rows outside 0 .. Sq-1 read a valid row and get LSE = +inf, so
// their P, dS and every contribution they make are exactly zero.  Key/value
// rows past Sk in the last tile read row Sk - 1 and are masked out of P like
// the upper triangle of a diagonal tile; their dK/dV rows go to the dummy
// tiles.
//
// Workspace dQ layout: per (query head, 64-row block of virtual rows) a 64 x D fp32 block
// stored as 32 x 32 MFMA C tiles (tile = qb * D/32 + db).  The deterministic
// schedules keep a tile as [register / 4][lane][register % 4], so one wave
// access is a 16-byte-per-lane, 1 KiB contiguous transfer; the atomic variant
// keeps [register][lane] (256 contiguous bytes per wave access), because
// fp32 atomics are per element.
//
// Ordering protocol of the deterministic schedules.  The workspace and the
// semaphores are only touched with device-scope relaxed atomic loads and
// stores, which bypass the chiplet-local caches that are not coherent across
// the device; no cache write-back or invalidate is issued.  Each wave that
// holds dQ tiles, for the block computed in sub-step s:
//   1. at the end of s, spins until sem == ordinal (usually already seen by
//      an early read), then issues the loads of its tiles of the block (for
//      ordinal 0 through an empty buffer range, so that they return zeros);
//   2. after the S/dP phase of s+1, adds its partial and writes the tiles
//      back;
//   3. after the dK/dV contraction of s+1 -- once the wave has waited for all
//      of its outstanding vector memory operations, so the writes are
//      complete at device scope -- one lane stores sem = ordinal + 1.
// When s+1 begins a new key/value chain, steps 2 and 3 happen at its start,
// around the loads of the new K/V tile, instead.
// Deferring the writes and the release overlaps their latency with compute;
// the release never waits on another workgroup, so no cycle can form.
// ---------------------------------------------------------------------------
struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dO;
  const float* lse;
  const float* delta;
  float* ws;
  int* sem;
  int* err;
  float* dummy;      // 8 tiles of 1024 floats that absorb writes with no destination
  __bf16* dk;
  __bf16* dv;
  const int4* steps;
  const int* offsets;
  unsigned long long* stall;
  int* xcc;          // optional: chiplet id per workgroup
  unsigned delay_seed;
  long long spin_ticks;
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
  int Sq, Sk, g;
  int wl, wr;        // window: query row i sees key j when -wl <= j - (i + Sk - Sq) <= wr (kUnbounded: open)
  int qshift;        // virtual query row = query row + qshift
  int nblk;          // 64-row workspace blocks per query head (virtual rows / 64)
  int diag_off;      // query tile qi's diagonal runs through key/value tile qi + diag_off (windowed masks)
};

// Semaphore words per 64-row dQ block: one per wave that holds dQ tiles.
constexpr int kSemPerBlock = 8;

// Chiplet (XCC) of the executing wave: bits 3:0 of hardware register 20
// (XCC_ID) on gfx950.
__device__ __forceinline__ int xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15; }

// Delay injection (the testing instantiation only): 0..63 sleeps of 64
// clocks, from a hash of (seed, workgroup, step, sub-step, wave, site) --
// MurmurHash3's 32-bit finaliser (Appleby) -- so every run of a seed
// perturbs the timing the same way and different seeds differently.  All
// inputs are wave-uniform, so the loop is a scalar loop.
__device__ __forceinline__ void debug_delay(unsigned seed, int wg, int i, int sub, int w, int site) {
  unsigned h = seed ^ ((unsigned)wg * 0x9E3779B1u) ^ ((unsigned)i * 0x85EBCA77u) ^
               ((unsigned)(sub * 64 + w * 4 + site) * 0xC2B2AE3Du);
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  const int n = (int)__builtin_amdgcn_readfirstlane(h & 63u);
  for (int k = 0; k < n; ++k) __builtin_amdgcn_s_sleep(1);
}

template <int T>
constexpr int bwd_threads() {
  return 64 * 2 * (T / 32);
}

// LEFT: the window has a left edge (a band other than causal / full): each
// element then needs a second comparison, which the other masks skip.
// DELAY: seeded sleeps before each semaphore wait and release (a separate
// instantiation for testing the ordering protocol under perturbed timing).
template <int D, int T, bool ATOMIC, bool LEFT, bool DELAY>
__global__ __launch_bounds__(bwd_threads<T>(), 1) void bwd_kernel(BwdArgs a) {
  constexpr int NP = T / 32;          // wave pairs; pair p owns key/value rows 32p .. 32p+31
  constexpr int NW = 2 * NP;          // waves
  constexpr int NT = 64 * NW;
  constexpr int M = 64;               // query rows per sub-step
  constexpr int SUBS = T / M;
  constexpr int DC = D / 16;
  constexpr int DB = D / 32;
  constexpr int DH = DB / 2;          // 32-wide d blocks of dK / dV per wave
  constexpr int NQT = 2 * DB;         // 32 x 32 dQ tiles per 64-row block
  constexpr int TPW = (NQT + NW - 1) / NW;
  constexpr bool SHARE_K = (NW % DB) == 0;  // a wave's dQ tiles share one d block
  constexpr int KC = T / 16;          // 16-row key/value chunks of the dQ contraction
  constexpr int QC = M / 16;          // 16-row query chunks of the dK / dV contraction
  constexpr int PQ = 2 * D;           // LDS pitch (bytes) of Q / dO / K rows, unpadded (see lds_swizzle)
  constexpr int PS = (M + 8) * 2;     // LDS pitch (bytes) of P^T / dS^T rows
  constexpr int QBUF = M * PQ;
  constexpr int DSBUF = T * PS;
  constexpr int OFF_Q = 0;                       // [2][M][PQ]
  constexpr int OFF_DO = OFF_Q + 2 * QBUF;       // [2][M][PQ]
  constexpr int OFF_K = OFF_DO + 2 * QBUF;       // [T][PQ]
  constexpr int OFF_PT = OFF_K + T * PQ;         // [T][PS]  P^T
  constexpr int OFF_DS = OFF_PT + T * PS;        // [2][T][PS]  dS^T, double-buffered (contracted for dQ one sub-step late)
  constexpr int OFF_STAT = OFF_DS + 2 * DSBUF;   // [2][2][M] f32: LSE (log2 domain), -Delta
  constexpr int OFF_FLAG = OFF_STAT + 4 * M * 4;
  constexpr int SMEM = OFF_FLAG + 16;
  constexpr int QCH = M * D / 8 / NT;            // 16-byte chunks per thread of one Q (or dO) block
  constexpr int KCH = T * D / 8 / NT;            // 16-byte chunks per thread of one K tile
  static_assert(QCH >= 1 && (M * D / 8) % NT == 0 && KCH >= 1 && (T * D / 8) % NT == 0, "tile split");
  static_assert(NT >= 2 * M, "one statistic per thread");
  static_assert(DH >= 1 && SUBS >= 1, "shape");
  static_assert(SMEM <= 160 * 1024, "LDS");
  static_assert(NW <= kSemPerBlock || NQT <= kSemPerBlock, "semaphore words");
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  LDS char* base = (LDS char*)smem;
  volatile LDS int* s_flag = (volatile LDS int*)(base + OFF_FLAG);

  const int lane = lane_id(), w = wave_id(), h2 = lane >> 5, c32 = lane & 31;
  const int hf = w & 1;                 // query half (S, dP) and d half (dK, dV) of this wave
  const int kv0 = 32 * (w >> 1);        // first key/value row of this wave's pair
  const int kv_local = kv0 + c32;
  // Step lists are read-only for the kernel's lifetime: read them through the
  // constant address space so that they become scalar loads.
  const CONST_AS int* steps = (const CONST_AS int*)a.steps;
  const CONST_AS int* offsets = (const CONST_AS int*)a.offsets;
  auto step_at = [&](int i) { return make_int4(steps[4 * i], steps[4 * i + 1], steps[4 * i + 2], steps[4 * i + 3]); };
  const int wg = blockIdx.x;
  const int beg = offsets[wg], end = offsets[wg + 1];
  const int Sq = a.Sq, Sk = a.Sk, g = a.g;
  const int nblk = a.nblk, diag_off = a.diag_off, qshift = a.qshift;
  unsigned long long stall = 0;
  const unsigned long long t_start = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) *s_flag = 0;
  if (a.xcc && threadIdx.x == 0) a.xcc[wg] = xcc_id();

  // Per-lane LDS byte offsets.
  const int tr_row = 8 * h2 + ((lane & 15) >> 2), tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int o_trs = opaque(tr_row * PS + tr_col * 2);                  // transposing reads, pitch PS
  // Byte offset of 16-byte chunk `chunk` of Q / dO / K row `row`.
  auto qk_chunk = [](int row, int chunk) { return row * PQ + 16 * (chunk ^ lds_swizzle<D>(row)); };
  // The swizzled Q / dO / K rows in XOR form: chunk pair c of this lane's Q / dO
  // (K) row read sits at r_q ^ (c << 5) (r_k ^ ...), and 64-byte column block
  // blk of the transposing read of rows 8h + 4e + (l%16)/4 at
  // t_dk[e] ^ ((blk ^ hf*DH) << 6).  The XOR touches only bits 5..7 of a
  // 2D-byte row, and buffer offsets are multiples of 2D bytes, so they add after
  // it.  The XORs are redone per sub-step, so that no per-chunk address stays
  // live across the loop.
  const int swq = lds_swizzle<D>(32 * hf + c32), swk = lds_swizzle<D>(kv0 + c32);
  const int r_q = opaque((32 * hf + c32) * PQ + 16 * (h2 ^ (swq & 1)) + 32 * (swq >> 1));
  const int r_k = opaque((kv0 + c32) * PQ + 16 * (h2 ^ (swk & 1)) + 32 * (swk >> 1));
  int t_dk[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    // the block bits of the swizzle come from tr_a, its chunk bits, (row >> 2) & 3, from h and e
    const int tr_a = (lane & 15) >> 2, tr_q = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int row = 8 * h2 + 4 * e + tr_a, blk_bits = D == 128 ? tr_a : (tr_a >> 1);
    t_dk[e] = opaque((row * PQ + 64 * blk_bits + 16 * (tr_q ^ ((2 * h2 + e) & 3)) + 8 * (lane & 1)) ^ ((hf * DH) << 6));
  }
  const int o_rowt = opaque(kv_local * PS + 16 * h2);                  // P^T / dS^T rows of this lane
  const int o_stt = opaque(kv_local * PS + (32 * hf + 4 * h2) * 2);    // P^T / dS^T stores
  const int o_stat = opaque((32 * hf + 4 * h2) * 4);                   // LSE / Delta of this lane's rows

  // Prefetch registers for the next Q/dO block and one LSE-or-Delta value.
  // LDS holds LSE·log2e (the exponent's offset) and −Delta (the initial value
  // of the dP accumulator, so that the MFMAs produce dP − Delta).
  bf16x8 pq[QCH], pdo[QCH];
  float pstat = 0.f;
  const int st_tid = threadIdx.x < 2 * M ? threadIdx.x : 0;
  const float st_mul = st_tid < M ? kLog2e : -1.f;
  // Q / dO rows through buffer descriptors over the head's rows: a row
  // outside 0 .. Sq-1 lies outside the descriptor's range and reads as zeros
  // (its LSE of +inf below already makes every contribution of it zero).
  auto load_block = [&](int head, int vrow0) {  // vrow0: first virtual row of the block
    const int row0 = vrow0 - qshift;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(uniform_ptr(a.q + (size_t)head * Sq * D)), (short)0, Sq * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rdo = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(uniform_ptr(a.dO + (size_t)head * Sq * D)), (short)0, Sq * D * 2, 0x00020000);
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int ch = threadIdx.x + i * NT;
      const int off = (row0 + ch / (D / 8)) * (2 * D) + (ch % (D / 8)) * 16;  // negative: out of range
      pq[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      pdo[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rdo, off, 0, 0));
    }
    const int srow = row0 + (st_tid & (M - 1));
    const bool valid = srow >= 0 && srow < Sq;
    const float* src = st_tid < M ? a.lse : a.delta;
    const float x = src[(size_t)head * Sq + min(max(srow, 0), Sq - 1)];
    pstat = valid ? x : (st_tid < M ? INFINITY : 0.f);  // LSE = +inf: P = 0 on rows outside the sequence
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int ch = threadIdx.x + i * NT, row = ch / (D / 8), col = (ch % (D / 8)) * 8;
      *(LDS bf16x8*)(base + OFF_Q + buf * QBUF + qk_chunk(row, col / 8)) = pq[i];
      *(LDS bf16x8*)(base + OFF_DO + buf * QBUF + qk_chunk(row, col / 8)) = pdo[i];
    }
    if (threadIdx.x < 2 * M) *(LDS float*)(base + OFF_STAT + (buf * 2 * M + threadIdx.x) * 4) = pstat * st_mul;
  };

  bf16x8 vb[DC];  // V rows of this pair as MFMA operands (K is read from LDS)
  f32x16 dk_acc[DH], dv_acc[DH];
  // Chain epilogue: single writer of dK (scaled) and dV for this wave's rows and d half.
  // Each tensor's 32 x DH*32 block of this wave goes through LDS -- the P^T / dS^T
  // buffers, which nothing else touches between a barrier that follows their last
  // reads and the next sub-step's first barrier -- so that it leaves as 16-byte row
  // chunks instead of one 2-byte store per accumulator element.
  constexpr int EP = DH * 64 + 16;  // staging row pitch (bytes): the rows 4 apart of one write fall in other banks
  constexpr int CPR = DH * 4;       // 16-byte chunks per staged row
  static_assert(NW * 32 * EP <= 3 * T * PS, "epilogue staging fits the P^T / dS^T buffers");
  bool epi_pending = false;
  int epi_kvh = 0, epi_kj = 0;
  auto write_dkdv = [&](int kvh_, int kj_) {
    // Buffer descriptors over the tile's rows inside the sequence: stores to
    // rows past Sk fall outside the range and are dropped.
    const int kv_valid = Sk - kj_ * T;
    const int nbytes = min(kv_valid, T) * D * 2;
    const size_t tile0 = ((size_t)kvh_ * Sk + (size_t)kj_ * T) * D;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(a.dk + tile0), (short)0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(a.dv + tile0), (short)0, nbytes, 0x00020000);
    const int tid_e = opaque((int)threadIdx.x);  // recomputed here, not kept live
    const int l_e = tid_e & 63, w_e = tid_e >> 6;
    LDS char* ep = base + OFF_PT + w_e * 32 * EP;
    // element (row 8(r/4) + 4h + r%4, column 32j + l%32) of the C tiles
    const int o_put = 4 * (l_e >> 5) * EP + 2 * (l_e & 31);
    // first element of the block in the tensor: row 32 * pair, column block DH * half
    const int o_blk = 2 * (32 * (w_e >> 1) * D + (w_e & 1) * DH * 32);
    auto put = [&](const f32x16 (&acc)[DH], float mul, __amdgpu_buffer_rsrc_t rs) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int j = 0; j < DH; ++j)
          *(LDS __bf16*)(ep + o_put + (8 * (r >> 2) + (r & 3)) * EP + 64 * j) = (__bf16)(acc[j][r] * mul);
      }
      // chunk c = l + 64u of the block: row c / CPR, 16 bytes at (c % CPR) * 16
#pragma unroll
      for (int u = 0; u < 32 * CPR / 64; ++u) {
        const int c = l_e + 64 * u, row = c / CPR, col = c % CPR;
        const f32x4 v = *(const LDS f32x4*)(ep + row * EP + 16 * col);
        __builtin_amdgcn_raw_buffer_store_b128(v, rs, o_blk + 2 * row * D + 16 * col, 0, 0);
      }
    };
    put(dk_acc, a.scale, rk);
    put(dv_acc, 1.f, rv);  // the same staging rows: this wave's reads above precede these writes
  };
  int buf = 0;
  // dQ of each 64-row block is contracted one sub-step late: the block of
  // sub-step s (its dS^T kept in one of two LDS buffers) is contracted in the
  // S/dP phase of sub-step s+1, interleaved with that sub-step's softmax, so
  // that each wave keeps the matrix core busy while its exponentials run on
  // the vector ALU.  Deterministic schedules then add the
  // predecessor's partial (read at the end of sub-step s, after the wait on
  // the block's semaphore) and write the sum back; the semaphore is released
  // after the dK/dV contraction of s+1, once the writes are complete.  When
  // s+1 starts a new key/value chain the block is contracted, written and
  // released at the chain start instead, before K is replaced.
  f32x16 pprev[TPW];
  // The vector-memory sequence of a sub-step is the same on every path (a
  // missing prefetch re-reads the current block, a missing write goes to the
  // dummy tiles), so the compiler's wait counts stay exact and no wait drains
  // more than the operation it is for.
  float* p_ws = a.dummy;  // block whose contraction is pending (the dummy tiles if none)
  int* p_sem = nullptr;   // its semaphore, if it is a real block (deterministic)
  int p_val = 0;
  int p_buf = 0;          // LDS buffer holding its dS^T
  bool p_real = false;    // atomic variant: a block is pending
  int* r_sem = nullptr;   // semaphore to release once this wave's writes are complete
  int r_val = 0;
  constexpr bool EVEN = (NQT % NW) == 0;  // every wave holds NQT / NW dQ tiles
  const bool has_tiles = EVEN || w < NQT;
#pragma unroll
  for (int ti = 0; ti < TPW; ++ti) pprev[ti] = f32x16{};

  // dQ partial = dS K over all T key/value rows of the pending block, for
  // this wave's C tiles (chain starts and the drain; the sub-step loop
  // interleaves the same contraction with its softmax).  The K^T and dS^T
  // operands of chunk c+1 are read while chunk c's MFMA runs.
  auto dq_contract = [&](f32x16 (&dq)[TPW]) {
    if (!has_tiles) return;
    const int dbw = w % DB;
    const int ko0 = opaque(t_dk[0] ^ ((hf * DH ^ dbw) << 6)), ko1 = opaque(t_dk[1] ^ ((hf * DH ^ dbw) << 6));
    const LDS char* pds0 = base + OFF_DS + p_buf * DSBUF + o_trs;
    auto ka_at = [&](int c) {
      return cat8(lds_tr4(base + OFF_K + ko0 + 16 * c * PQ), lds_tr4(base + OFF_K + ko1 + 16 * c * PQ));
    };
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
      const int qb = (w + NW * ti) / DB;
      const LDS char* pds = pds0 + qb * 64;
      f32x16 acc = f32x16{};
      bf16x8 ka[2], sa[2];
      ka[0] = ka_at(0);
      sa[0] = lds_tr8_at(pds, PS);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if (c + 1 < KC) {
          ka[(c + 1) & 1] = ka_at(c + 1);
          sa[(c + 1) & 1] = lds_tr8_at(pds + 16 * (c + 1) * PS, PS);
        }
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma32(sa[c & 1], ka[c & 1], acc);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      dq[ti] = acc;
    }
  };
  // Write out the pending block's contracted partial: deterministic
  // schedules add the predecessor's partial (zeros for a first contribution)
  // and store the sum to the block's tiles, to the dummy tiles when nothing is
  // pending, and mark its semaphore for release; the atomic variant adds with
  // fp32 atomics when a block is pending.
  auto dq_store = [&](const f32x16 (&dq)[TPW]) {
    if constexpr (ATOMIC) {
      if (p_real) {
#pragma unroll
        for (int ti = 0; ti < TPW; ++ti) {
          const int t_idx = w + NW * ti;
          if (EVEN || t_idx < NQT) {
            float* p = p_ws + t_idx * 1024 + lane;
#pragma unroll
            for (int r = 0; r < 16; ++r)
              __hip_atomic_fetch_add(p + r * 64, dq[ti][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    } else {
      if (has_tiles) {
#pragma unroll
        for (int ti = 0; ti < TPW; ++ti) {
          const int t_idx = w + NW * ti;
          const __amdgpu_buffer_rsrc_t rs =
              ws_rsrc(uniform_ptr((EVEN || t_idx < NQT) ? p_ws : a.dummy) + t_idx * 1024);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = dq[ti][4 * q4 + e] + pprev[ti][4 * q4 + e];
            __builtin_amdgcn_raw_buffer_store_b128(v4, rs, (q4 * 64 + lane) * 16, 0, kDeviceScope);
          }
        }
      }
      r_sem = p_sem;
      r_val = p_val;
    }
  };
  auto dq_finish = [&]() {
    f32x16 dq[TPW];
    dq_contract(dq);
    dq_store(dq);
  };
  if (beg < end) {
    const int4 r0 = step_at(beg);
    load_block(r0.x, r0.y * T);
    store_block(0);
  }

  // Step records are read one step ahead, so that no sub-step waits for a
  // scalar load of its own record or of the next block's.
  int4 rec_next = beg < end ? step_at(beg) : make_int4(0, 0, 0, 0);
  for (int i = beg; i < end; ++i) {
    const int4 rec = rec_next;
    if (i + 1 < end) rec_next = step_at(i + 1);
    const int head = rec.x, qi = rec.y, kj = rec.z, ordf = rec.w;
    const int ord = ordf & ((1 << 28) - 1);
    const bool first = ordf & (1 << 28), last = ordf & (1 << 29);
    const int kvh = head / g;
    const __bf16* kh = a.k + ((size_t)kvh * Sk + (size_t)kj * T) * D;
    const __bf16* vh = a.v + ((size_t)kvh * Sk + (size_t)kj * T) * D;
    const int kv_valid = Sk - kj * T;  // key/value rows of this tile inside the sequence (>= T but on the last)
    if (first) {
      // New chain.  The new chain's V and K rows are requested first; while
      // they arrive, the previous chain's last block is contracted (its dS^T
      // and K are still in LDS) and written, and it is released as soon as
      // both have completed, rather than a sub-step into the new chain: where
      // members change chains at different rounds (the causal symmetric
      // shift), the block's successor is mid-chain and would otherwise wait
      // for this chain start.  Then the new V rows stay in registers and the
      // K tile goes to LDS; the previous chain's dK/dV are written only after
      // that, so that waiting for these loads never waits for those writes to
      // drain.
      const bool flush = __builtin_amdgcn_readfirstlane((int)(ATOMIC ? p_real : p_sem != nullptr));
      // Buffer descriptors over the tile's rows inside the sequence: rows past
      // Sk read as zeros (they are masked out of P).  Per-lane offsets are
      // recomputed from the lane's index here rather than kept live.
      {
        const int nbytes = min(kv_valid, T) * D * 2;
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(uniform_ptr(vh)), (short)0, nbytes, 0x00020000);
        const int tid = opaque((int)threadIdx.x);
        const int vo = (kv0 + (tid & 31)) * (2 * D) + 16 * ((tid >> 5) & 1);
#pragma unroll
        for (int c = 0; c < DC; ++c)
          vb[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, vo + 32 * c, 0, 0));
      }
      bf16x8 kt[KCH];
      {
        const int nbytes = min(kv_valid, T) * D * 2;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(uniform_ptr(kh)), (short)0, nbytes, 0x00020000);
        // chunk (tid + u * NT) of the row-major tile; the whole offset stays in
        // the range-checked vector offset
        const int ko = opaque((int)threadIdx.x) * 16;
#pragma unroll
        for (int u = 0; u < KCH; ++u)
          kt[u] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, ko + u * NT * 16, 0, 0));
      }
      // the pending block is contracted and written while the new rows arrive
      if (flush) dq_finish();
      if constexpr (!ATOMIC) {
        if (flush) {
          wait_vmem_all();
          if constexpr (DELAY) debug_delay(a.delay_seed, wg, i, 0, w, 0);
          if (r_sem != nullptr && lane == 0) __hip_atomic_store(r_sem, r_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          r_sem = nullptr;
        }
      }
      // Nothing is pending any more: the contraction in the next S/dP phase
      // writes to the dummy tiles.
      p_ws = a.dummy;
      p_sem = nullptr;
      p_real = false;
      __syncthreads();  // every wave is done with the previous chain's K
      const int tid_k = opaque((int)threadIdx.x);  // staging addresses recomputed here, not kept live
#pragma unroll
      for (int u = 0; u < KCH; ++u) {
        const int ch = tid_k + u * NT, row = ch / (D / 8), col = (ch % (D / 8)) * 8;
        *(LDS bf16x8*)(base + OFF_K + qk_chunk(row, col / 8)) = kt[u];
      }
      if (epi_pending) write_dkdv(epi_kvh, epi_kj);
      epi_pending = false;
#pragma unroll
      for (int j = 0; j < DH; ++j) {
        dk_acc[j] = f32x16{};
        dv_acc[j] = f32x16{};
      }
    }
    // Key offset of this tile from the query tile's diagonal tile, in rows.  The
    // tile is partly masked when some pair falls outside the window (in the
    // key-aligned grid of a windowed mask, local key - local row ranges over
    // -(T-1) .. T-1), or when it is the ragged last key/value tile.
    const int dd = (kj - qi - diag_off) * T;
    const bool mask_on = dd > a.wr - (T - 1) || dd < (T - 1) - a.wl || kv_valid < T;

    // Unrolled, so that each sub-step's code is specialised for its place in
    // the tile (which block comes next, which buffers it uses).
#pragma unroll
    for (int sub = 0; sub < SUBS; ++sub) {
      __syncthreads();  // B1: Q/dO/LSE/Delta of this block (and sK) visible; P^T and this dS^T buffer free
      // Prefetch the next block while this one is computed (issued before this
      // sub-step's dQ writes, so staging it never waits for them).
      int nhead = head, nrow = qi * T + sub * M;  // no next block: re-read this one
      if (sub + 1 < SUBS) {
        nrow = qi * T + (sub + 1) * M;
      } else if (i + 1 < end) {
        nhead = rec_next.x;
        nrow = rec_next.y * T;
      }
      const LDS float* slse = (const LDS float*)(base + OFF_STAT + buf * 2 * M * 4);
      const LDS float* sdel = slse + M;

      f32x16 dqp[TPW];
      {
        // S = Q K^T and dP - Delta = dO V^T - Delta for query rows 32*hf .. +31 x this
        // pair's 32 key/value columns: the dP accumulator starts at -Delta of its row
        // (row 8j + 4*h2 + e of the half in element 4j + e).
        f32x16 s = f32x16{}, dp;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 nd = *(const LDS f32x4*)((const LDS char*)sdel + o_stat + 32 * j);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[4 * j + e] = nd[e];
        }
        // One 16-wide d chunk at a time, double-buffered: chunk c+1's Q, dO and
        // K operands are read while chunk c's two MFMAs run.
        bf16x8 aq[3], ado[3], bk[3];
        const int rq = opaque(buf * QBUF + r_q), rk = opaque(r_k);
        auto fetch = [&](int c, int sl) {
          aq[sl] = lds_row8(base + OFF_Q + (rq ^ (c << 5)));
          ado[sl] = lds_row8(base + OFF_DO + (rq ^ (c << 5)));
          bk[sl] = lds_row8(base + OFF_K + (rk ^ (c << 5)));
        };
        fetch(0, 0);
        if (DC > 1) fetch(1, 1);
        // the next block's loads go out after the first operand reads
        load_block(nhead, nrow);
        // Each contraction runs at raised wave priority, so that while one wave
        // of a SIMD issues matrix-core instructions the other wave's vector and
        // LDS work fills the gaps.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          if (c + 2 < DC) fetch(c + 2, (c + 2) % 3);
          s = mfma32(aq[c % 3], bk[c % 3], s);
          dp = mfma32(ado[c % 3], vb[c], dp);
          // chunk c+2's three reads between and after chunk c's two MFMAs
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        // P = exp2(S*scale*log2e - LSE*log2e); dS = P * (dP - Delta), the second
        // accumulator holding dP - Delta already; both to LDS
        // transposed, four rows of this lane at a time.  Interleaved with it, the
        // pending block's dQ partial = dS K (its dS^T in the other buffer): after
        // each group of four rows the wave issues the next dQ MFMAs, which run on
        // the matrix core while the next group's exponentials run on the vector
        // ALU.
        // Element (8j + e) of this lane has key - diagonal key = rel - (8j + e); under
        // mask_on P is zero where that exceeds wr (hi > 8j + e) or falls below -wl
        // (lo < 8j + e), and in every row of a key/value column past Sk.  The bounds are
        // made opaque so that the comparisons are formed here rather than kept live
        // across the loop.
        const int rel = kv_local - (sub * M + 32 * hf + 4 * h2) + dd;
        int hi = kv_local >= kv_valid ? kUnbounded : rel - a.wr;
        int lo = rel + a.wl;
        asm volatile("" : "+v"(hi), "+v"(lo));
        LDS char* ds_out = base + OFF_DS + buf * DSBUF + o_stt;
        constexpr int NDQ = TPW * KC;  // dQ MFMAs of this wave
        static_assert(NDQ % 4 == 0, "dQ chunks per group of rows");
        constexpr int PER_J = NDQ / 4;
        static_assert(SHARE_K, "a wave's dQ tiles share one d block");
        const int dbw = w % DB;
        const int ko0 = opaque(t_dk[0] ^ ((hf * DH ^ dbw) << 6)), ko1 = opaque(t_dk[1] ^ ((hf * DH ^ dbw) << 6));
        const LDS char* pds0 = base + OFF_DS + p_buf * DSBUF + o_trs;
#pragma unroll
        for (int ti = 0; ti < TPW; ++ti) dqp[ti] = f32x16{};
        // Two copies of the loop: tile pairs that need no element mask (every
        // pair of a full mask, all but the diagonal pairs of a causal one) skip
        // the per-element comparisons.
        auto softmax_dq = [&](auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        f32x4 l4[2];
        l4[0] = *(const LDS f32x4*)((const LDS char*)slse + o_stat);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // operands of this group's dQ MFMAs (their latency hides behind the exponentials)
          bf16x8 ka[PER_J], sa[PER_J];
          if (has_tiles) {
#pragma unroll
            for (int u = 0; u < PER_J; ++u) {
              const int uu = j * PER_J + u, ti = uu / KC, c = uu % KC;
              const int qb = (w + NW * ti) / DB;
              ka[u] = cat8(lds_tr4(base + OFF_K + ko0 + 16 * c * PQ), lds_tr4(base + OFF_K + ko1 + 16 * c * PQ));
              sa[u] = lds_tr8_at(pds0 + qb * 64 + 16 * c * PS, PS);
            }
          }
          if (j + 1 < 4) {
            l4[(j + 1) & 1] = *(const LDS f32x4*)((const LDS char*)slse + o_stat + 32 * (j + 1));
          }
          bf16x4 tp, ts;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * j + e;
            float p = __builtin_amdgcn_exp2f(s[r] * a.scale_log2 - l4[j & 1][e]);
            if (MASKED && (hi > 8 * j + e || (LEFT && lo < 8 * j + e))) p = 0.f;
            tp[e] = (__bf16)p;
            ts[e] = (__bf16)(p * dp[r]);
          }
          *(LDS bf16x4*)(base + OFF_PT + o_stt + 16 * j) = tp;
          *(LDS bf16x4*)(ds_out + 16 * j) = ts;
          if (has_tiles) {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int u = 0; u < PER_J; ++u) {
              const int uu = j * PER_J + u, ti = uu / KC;
              dqp[ti] = mfma32(sa[u], ka[u], dqp[ti]);
            }
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        };
        if (mask_on) softmax_dq(std::true_type{});
        else softmax_dq(std::false_type{});
      }
      dq_store(dqp);
      __syncthreads();  // B2: P^T, dS^T complete

      const int blk = qi * SUBS + sub;
      float* wsb = a.ws + ((size_t)head * nblk + blk) * (size_t)(M * D);
      int* semp = a.sem + ((size_t)head * nblk + blk) * kSemPerBlock + w;
      // First look at this block's semaphore now, so that its latency is hidden
      // behind the dK/dV contraction (in the lockstep schedules the predecessor
      // has usually released it by now); the wait below only polls if not.
      int sem_seen = 0;
      if constexpr (!ATOMIC) sem_seen = __hip_atomic_load(semp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // dV += P^T dO, dK += dS^T Q over the block's 64 query rows, d half hf.
      // Lightly software-pipelined: the next chunk's P^T/dS^T rows and each
      // B operand are read one MFMA ahead of their use (scheduling barriers
      // keep that order), which hides part of the LDS latency.
      {
        bf16x8 ap[2], ads[2];
        const LDS char* ds_in = base + OFF_DS + buf * DSBUF + o_rowt;
        const int td[2] = {opaque(buf * QBUF + t_dk[0]), opaque(buf * QBUF + t_dk[1])};
        ap[0] = lds_row8(base + OFF_PT + o_rowt);
        ads[0] = lds_row8(ds_in);
        // d block j of this wave's half of dO (is_do) or Q, query chunk c
        auto tr_dkdv = [&](bool is_do, int c, int j) {
          const LDS char* b_ = base + (is_do ? OFF_DO : OFF_Q) + 16 * c * PQ;
          return cat8(lds_tr4(b_ + (td[0] ^ (j << 6))), lds_tr4(b_ + (td[1] ^ (j << 6))));
        };
        // B operands of query chunk c+1 are read while chunk c's MFMAs run.
        bf16x8 bdo[2][DH], bq[2][DH];
#pragma unroll
        for (int j = 0; j < DH; ++j) {
          bdo[0][j] = tr_dkdv(true, 0, j);
          bq[0][j] = tr_dkdv(false, 0, j);
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int c = 0; c < QC; ++c) {
          const int sl = c & 1;
          if (c + 1 < QC) {
            ap[sl ^ 1] = lds_row8(base + OFF_PT + o_rowt + 32 * (c + 1));
            ads[sl ^ 1] = lds_row8(ds_in + 32 * (c + 1));
#pragma unroll
            for (int j = 0; j < DH; ++j) {
              bdo[sl ^ 1][j] = tr_dkdv(true, c + 1, j);
              bq[sl ^ 1][j] = tr_dkdv(false, c + 1, j);
            }
          }
#pragma unroll
          for (int j = 0; j < DH; ++j) {
            dv_acc[j] = mfma32(ap[sl], bdo[sl][j], dv_acc[j]);
            dk_acc[j] = mfma32(ads[sl], bq[sl][j], dk_acc[j]);
          }
          // chunk c+1's reads spread between chunk c's MFMAs
#pragma unroll
          for (int m = 0; m < 2 * DH; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, (2 + 8 * DH / 2 + 2 * DH - 1) / (2 * DH), 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
      }
      if constexpr (!ATOMIC) {
        // Release the block written in the S/dP phase as soon as its writes
        // have had the dK/dV contraction to complete (successors wait on it).
        wait_vmem_all();
        if constexpr (DELAY) debug_delay(a.delay_seed, wg, i, sub, w, 1);
        if (r_sem != nullptr && lane == 0) __hip_atomic_store(r_sem, r_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        r_sem = nullptr;
      }

      // The other Q/dO buffer is free (read before B1): stage the prefetched block.
      store_block(buf ^ 1);

      // This block is now the pending one.
      p_buf = buf;
      buf ^= 1;
      if constexpr (ATOMIC) {
        p_ws = wsb;
        p_real = true;
      } else {
        // Wait for this block's predecessor, then start reading its partial.  (The
        // early value is consumed on every path, so it is never left pending.)
        if constexpr (DELAY) debug_delay(a.delay_seed, wg, i, sub, w, 2);
        const bool ready = __builtin_amdgcn_readfirstlane(sem_seen) == ord;
        bool give_up = false;
        if (has_tiles && ord > 0 && !ready) {
          const unsigned long long t0 = __builtin_amdgcn_s_memtime();
          const long long deadline = (long long)__builtin_amdgcn_s_memrealtime() + a.spin_ticks;
          while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(semp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != ord) {
            if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0) {
              give_up = true;
              break;
            }
            if ((long long)__builtin_amdgcn_s_memrealtime() > deadline) {
              if (lane == 0) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              give_up = true;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
          stall += __builtin_amdgcn_s_memtime() - t0;
        }
        // The reads are issued on every path of a wave holding tiles (an ordinal
        // of zero or a wave that gave up reads its tiles and ignores them), so that
        // no path merge copies the registers before the loads complete.
        if (has_tiles) {
#pragma unroll
          for (int ti = 0; ti < TPW; ++ti) {
            const int t_idx = w + NW * ti;
            asm volatile("" ::: "memory");  // the reads stay after the wait above
            // A first contribution (ordinal 0) has no predecessor: an empty
            // buffer range makes these loads return zeros without reading
            // memory, so the sum needs no select.
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                wsb + (t_idx < NQT ? t_idx : t_idx % NQT) * 1024, (short)0, ord > 0 ? 4096 : 0, 0x00020000);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const f32x4 v4 = __builtin_amdgcn_raw_buffer_load_b128(rs, (q4 * 64 + lane) * 16, 0, kDeviceScope);
#pragma unroll
              for (int e = 0; e < 4; ++e) pprev[ti][4 * q4 + e] = v4[e];
            }
          }
        }
        const bool real = has_tiles && !give_up;
        p_ws = real ? wsb : a.dummy;
        p_sem = real ? semp : nullptr;
        p_val = ord + 1;
        // After a give-up the error word makes every later wait of the call
        // return at once, so the workgroup runs to the end of its list without
        // waiting (no wave leaves the loop early, so the barriers stay matched).
        if (give_up && lane == 0) *s_flag = 1;
      }
    }

    if (last) {  // written at the next chain's start, or after the loop
      epi_pending = true;
      epi_kvh = kvh;
      epi_kj = kj;
    }
  }
  // Drain: the last block of this wave (K and its dS^T are still in LDS),
  // skipped after a give-up (the call's outputs are then discarded).
  __syncthreads();
  if (!*s_flag) {
    const bool flush = __builtin_amdgcn_readfirstlane((int)(ATOMIC ? p_real : p_sem != nullptr));
    if (flush) {
      dq_finish();
      if constexpr (!ATOMIC) {
        wait_vmem_all();
        if constexpr (DELAY) debug_delay(a.delay_seed, wg, end, 0, w, 3);
        if (r_sem != nullptr && lane == 0) __hip_atomic_store(r_sem, r_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  // The last chain's dK/dV, staged in the P^T / dS^T buffers once every wave is
  // done with the drain's dS^T reads.
  __syncthreads();
  if (epi_pending) write_dkdv(epi_kvh, epi_kj);
  if (a.stall && threadIdx.x == 0) {
    a.stall[2 * wg] = stall;
    a.stall[2 * wg + 1] = __builtin_amdgcn_s_memtime() - t_start;
  }
}

// dQ = bf16(scale * workspace), undoing the fragment order.  One thread per
// (block, tile, register group of four, lane): four rows of one column.
// Deterministic layout (X4): tile as [register / 4][lane][register % 4]; the
// atomic layout: tile as [register][lane].  Workspace blocks hold virtual
// rows (query row + qshift, nblk blocks per head); rows outside 0 .. Sq-1
// are not written.
//
// If the persistent kernel gave up on a semaphore wait (*err != 0), the
// workspace is incomplete: dQ, dK and dV are all written with NaN instead,
// and the host-visible word `sticky` (if any) is set, so that the failure
// shows in the outputs and in the next call's status rather than as
// plausible wrong gradients.
template <int D, bool X4>
__global__ __launch_bounds__(256) void dq_finalize_kernel(const float* __restrict__ ws, __bf16* __restrict__ dq,
                                                          long long n_groups, float scale, int nblk, int qshift,
                                                          int Sq, const int* __restrict__ err, int* sticky,
                                                          __bf16* __restrict__ dk, __bf16* __restrict__ dv,
                                                          long long kv_elems) {
  const long long f = (long long)blockIdx.x * 256 + threadIdx.x;
  const bool failed = *err != 0;
  if (failed) {
    if (f == 0 && sticky) __hip_atomic_store(sticky, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const __bf16 nan = __builtin_bit_cast(__bf16, (unsigned short)0x7FC0);
    const long long stride = (long long)gridDim.x * 256;
    for (long long i = f; i < kv_elems; i += stride) {
      dk[i] = nan;
      dv[i] = nan;
    }
  }
  if (f >= n_groups) return;
  constexpr int GROUPS_PER_BLOCK = 64 * D / 4;
  const long long blk = f / GROUPS_PER_BLOCK;  // (head, 64-row block)
  const long long head = blk / nblk;
  const int rem = (int)(f % GROUPS_PER_BLOCK);
  const int tile = rem / 256, j = (rem % 256) / 64, l = rem % 64;
  const int qb = tile / (D / 32), db = tile % (D / 32);
  const int col = db * 32 + (l & 31);
  const int row0 = (int)(blk % nblk) * 64 + qb * 32 + 8 * j + 4 * (l >> 5) - qshift;
  __bf16* out = dq + (size_t)head * Sq * D;
  f32x4 v;
  if constexpr (X4) {
    v = *(const f32x4*)(ws + (size_t)blk * 64 * D + tile * 1024 + j * 256 + l * 4);
  } else {
    const float* src = ws + (size_t)blk * 64 * D + tile * 1024 + (4 * j) * 64 + l;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = src[e * 64];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (row0 + e >= 0 && row0 + e < Sq)
      out[(size_t)(row0 + e) * D + col] = failed ? __builtin_bit_cast(__bf16, (unsigned short)0x7FC0)
                                                 : (__bf16)(v[e] * scale);
}

}  // namespace

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                      int Sq, int Sk, int D, float scale, int wl, int wr, hipStream_t st) {
  wl = wl < 0 ? kUnbounded : wl;
  wr = wr < 0 ? kUnbounded : wr;
  const int g = Hq / Hkv;
  const float sl2 = scale * kLog2e;
  const bool big = Sq >= 1024;  // 128 query rows per workgroup, else 64
  dim3 grid((Sq + (big ? 127 : 63)) / (big ? 128 : 64), B * Hq);
  auto qp = (const __bf16*)q;
  auto kp = (const __bf16*)k;
  auto vp = (const __bf16*)v;
  auto op = (__bf16*)o;
  if (D == 128) {
    if (big) hipLaunchKernelGGL((fwd_kernel<128, 4>), grid, dim3(256), 0, st, qp, kp, vp, op, lse, Hq, g, Sq, Sk, sl2, wl, wr);
    else hipLaunchKernelGGL((fwd_kernel<128, 2>), grid, dim3(128), 0, st, qp, kp, vp, op, lse, Hq, g, Sq, Sk, sl2, wl, wr);
  } else {
    if (big) hipLaunchKernelGGL((fwd_kernel<64, 4>), grid, dim3(256), 0, st, qp, kp, vp, op, lse, Hq, g, Sq, Sk, sl2, wl, wr);
    else hipLaunchKernelGGL((fwd_kernel<64, 2>), grid, dim3(128), 0, st, qp, kp, vp, op, lse, Hq, g, Sq, Sk, sl2, wl, wr);
  }
  return hipGetLastError();
}

hipError_t launch_delta(const void* o, const void* dO, float* delta, long long rows, int D, int* zero_i32,
                        long long n_zero_i32, float* zero_f32, long long n_zero_f32, hipStream_t st) {
  const long long threads = rows * (D / 8);
  long long blocks = (threads + 255) / 256;
  const long long zb = (std::max(n_zero_i32, n_zero_f32 / 4) + 255) / 256;
  if (blocks < zb) blocks = std::min<long long>(zb, 65536);
  if (blocks < 1) blocks = 1;
  if (D == 128)
    hipLaunchKernelGGL((delta_kernel<128>), dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)o, (const __bf16*)dO,
                       delta, rows, zero_i32, n_zero_i32, zero_f32, n_zero_f32);
  else
    hipLaunchKernelGGL((delta_kernel<64>), dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)o, (const __bf16*)dO,
                       delta, rows, zero_i32, n_zero_i32, zero_f32, n_zero_f32);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdLaunch& L, hipStream_t st) {
  BwdArgs a;
  a.q = (const __bf16*)L.q;
  a.k = (const __bf16*)L.k;
  a.v = (const __bf16*)L.v;
  a.dO = (const __bf16*)L.dO;
  a.lse = L.lse;
  a.delta = L.delta;
  a.ws = L.ws;
  a.sem = L.sem;
  a.err = L.err;
  a.dummy = L.dummy;
  a.dk = (__bf16*)L.dk;
  a.dv = (__bf16*)L.dv;
  a.steps = (const int4*)L.steps;
  a.offsets = L.offsets;
  a.stall = L.stall;
  a.xcc = L.xcc;
  a.delay_seed = L.delay_seed;
  a.spin_ticks = L.spin_ticks;
  a.scale = L.scale;
  a.scale_log2 = L.scale * kLog2e;
  a.Sq = L.Sq;
  a.Sk = L.Sk;
  a.g = L.g;
  a.wl = L.wl < 0 ? kUnbounded : L.wl;
  a.wr = L.wr < 0 ? kUnbounded : L.wr;
  a.qshift = L.qshift;
  a.nblk = L.nblk;
  a.diag_off = L.diag_off;
  dim3 grid(L.P);
  const bool left = a.wl < kUnbounded;
#define DASH_BWD_CASE(D_, T_)                                                                          \
  if (L.D == D_ && L.T == T_) {                                                                        \
    const dim3 block(bwd_threads<T_>());                                                               \
    if (L.atomic) {                                                                                    \
      if (left) hipLaunchKernelGGL((bwd_kernel<D_, T_, true, true, false>), grid, block, 0, st, a);    \
      else hipLaunchKernelGGL((bwd_kernel<D_, T_, true, false, false>), grid, block, 0, st, a);        \
    } else if (L.delay_seed) {                                                                         \
      if (left) hipLaunchKernelGGL((bwd_kernel<D_, T_, false, true, true>), grid, block, 0, st, a);    \
      else hipLaunchKernelGGL((bwd_kernel<D_, T_, false, false, true>), grid, block, 0, st, a);        \
    } else {                                                                                           \
      if (left) hipLaunchKernelGGL((bwd_kernel<D_, T_, false, true, false>), grid, block, 0, st, a);   \
      else hipLaunchKernelGGL((bwd_kernel<D_, T_, false, false, false>), grid, block, 0, st, a);       \
    }                                                                                                  \
    return hipGetLastError();                                                                          \
  }
  DASH_BWD_CASE(128, 128)
  DASH_BWD_CASE(64, 128)
  DASH_BWD_CASE(128, 64)
  DASH_BWD_CASE(64, 64)
#undef DASH_BWD_CASE
  return hipErrorInvalidValue;
}

namespace {
// Workgroups per CU of every variant of one (D, T, atomic) family (all must fit).
template <int D, int T, bool ATOMIC>
hipError_t min_occupancy(int* per_cu) {
  const int nt = bwd_threads<T>();
  int v[4] = {0, 0, 1 << 30, 1 << 30};
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v[0], bwd_kernel<D, T, ATOMIC, false, false>, nt, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v[1], bwd_kernel<D, T, ATOMIC, true, false>, nt, 0);
  if constexpr (!ATOMIC) {
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v[2], bwd_kernel<D, T, false, false, true>, nt, 0);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v[3], bwd_kernel<D, T, false, true, true>, nt, 0);
  }
  *per_cu = std::min(std::min(v[0], v[1]), std::min(v[2], v[3]));
  return e;
}
}  // namespace

hipError_t bwd_kernel_per_cu(int D, int T, bool atomic, int* per_cu) {
  hipError_t e = hipErrorInvalidValue;
#define DASH_OCC_CASE(D_, T_) \
  if (D == D_ && T == T_) e = atomic ? min_occupancy<D_, T_, true>(per_cu) : min_occupancy<D_, T_, false>(per_cu);
  DASH_OCC_CASE(128, 128)
  DASH_OCC_CASE(64, 128)
  DASH_OCC_CASE(128, 64)
  DASH_OCC_CASE(64, 64)
#undef DASH_OCC_CASE
  return e;
}

hipError_t launch_dq_finalize(const FinalizeLaunch& F, hipStream_t st) {
  const long long n_f4 = F.ws_elems / 4;
  const unsigned blocks = (unsigned)std::max<long long>(1, (n_f4 + 255) / 256);
  auto dq = (__bf16*)F.dq;
  auto dk = (__bf16*)F.dk;
  auto dv = (__bf16*)F.dv;
#define DASH_FIN(D_, X4_)                                                                                          \
  hipLaunchKernelGGL((dq_finalize_kernel<D_, X4_>), dim3(blocks), dim3(256), 0, st, F.ws, dq, n_f4, F.scale, F.nblk, \
                     F.qshift, F.Sq, F.err, F.sticky, dk, dv, F.kv_elems)
  if (F.D == 128) {
    if (F.atomic_layout) DASH_FIN(128, false);
    else DASH_FIN(128, true);
  } else {
    if (F.atomic_layout) DASH_FIN(64, false);
    else DASH_FIN(64, true);
  }
#undef DASH_FIN
  return hipGetLastError();
}

}  // namespace dash
