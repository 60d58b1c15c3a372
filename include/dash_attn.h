/*
 * dash_attn.h -- C ABI of the deterministic attention backward library
 * (libdash_attn.so) for AMD Instinct MI355X (gfx950).
 *
 * The library computes softmax attention forward (O, LSE) and backward
 * (dQ, dK, dV) with the tile schedules of DASH, "Deterministic Attention
 * Scheduling for High-Throughput".  Sources, cited by page title and section:
 *   [summary] "Resumo Técnico: DASH – Agendamento de Atenção Determinístico
 *             para Treinamento de LLM de Alto Rendimento" (gist.science)
 *   [news]    "DASH如何革新LLM确定性训练" (pwwt.cn)
 *   [ascend]  the Ascend 910B essay on deterministic FlashAttentionGrad
 *             (ocdem.com); prior art on other hardware, cited only for the
 *             mask and shape scenarios it lists
 *
 * Conventions shared by every entry point:
 *  - Tensors are contiguous row-major BHSD: Q, O, dO, dQ are [B, Hq, Sq, D];
 *    K, V, dK, dV are [B, Hkv, Sk, D] (Sq = Sk = S in the entry points that
 *    take one length); all bfloat16 (2-byte) device buffers.  LSE is
 *    [B, Hq, Sq] float32 (natural logarithm).  Every device pointer must be
 *    16-byte aligned.  The caller owns all buffers.
 *  - Query head hq reads key/value head hq / (Hq / Hkv) (grouped-query
 *    attention with contiguous groups).
 *  - The causal mask is aligned at the bottom right: key j is visible to
 *    query i iff j <= i + Sk - Sq (j <= i when Sq = Sk).
 *  - softmax_scale <= 0 selects 1/sqrt(D).
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *    Device work is enqueued on it and the call returns without waiting;
 *    the caller keeps buffers alive until the stream has passed the work.
 *  - Return value: DASH_OK (0) or a negative status.  Arguments are checked
 *    before anything is enqueued; on error nothing is launched and
 *    dash_last_error() describes the problem.  No exception crosses the ABI.
 *  - Supported: D in {64, 128}; Hq a multiple of Hkv; any sequence lengths
 *    (the last tile may be partial).  Empty problems are valid: with B = 0
 *    or no query rows nothing is launched (pointers may then be NULL),
 *    except that the backward pass writes dK = dV = 0 when Sq = 0 and
 *    Sk > 0.  Query rows with no keys (Sk = 0, Sq > 0) are invalid: their
 *    softmax is undefined.
 */
#ifndef DASH_ATTN_H
#define DASH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum dash_status {
  DASH_OK = 0,
  DASH_ERR_INVALID_ARG = -1,      /* null pointer, negative size, no keys, Hq % Hkv != 0 */
  DASH_ERR_UNSUPPORTED = -2,      /* valid but not implemented: D, tile, mask/schedule pair, gang > workgroups, size */
  DASH_ERR_HIP = -3,              /* a HIP runtime call failed */
  DASH_ERR_INVALID_SCHEDULE = -4, /* a step list failed validation */
  DASH_ERR_TIMEOUT = -5,          /* a workgroup gave up waiting on a dQ semaphore (see dash_check_async_error) */
  DASH_ERR_WORKSPACE = -6         /* caller workspace too small or misaligned */
};

enum dash_mask { DASH_MASK_FULL = 0, DASH_MASK_CAUSAL = 1 };

/*
 * Backward schedules.  The first four are deterministic: each dQ tile
 * accumulates its key/value contributions in an order fixed by the schedule
 * ([summary] §1: a fixed accumulation order for dQ gives bitwise
 * reproducibility), enforced by per-dQ-tile semaphores in global memory.
 *   SERIAL    serialized fixed-order baseline: ascending query walk,
 *             ascending key/value order per dQ tile ([summary] §1, §4).
 *   DESC_Q    descending query-tile walk, same order ([summary] §2.2.A).
 *   SHIFT     full mask only: cyclic shift, the workgroup holding key/value
 *             tile i visits query tiles i, i+1, ..., N-1, 0, ..., i-1
 *             ([summary] §2.2.B; [news] §2.3).  A gang of N workgroups per
 *             key/value group.
 *   SYM_SHIFT causal mask only: tiles i and N-1-i paired on one workgroup,
 *             dense rectangle then folded triangle ([summary] §2.2.B).  N
 *             even; a gang of N/2 workgroups per key/value group.
 *   ATOMIC    non-deterministic ceiling: fp32 atomic adds into dQ in any
 *             order ([summary] §1, the non-deterministic counterpart).
 */
enum dash_schedule_kind {
  DASH_SCHED_SERIAL = 0,
  DASH_SCHED_DESC_Q = 1,
  DASH_SCHED_SHIFT = 2,
  DASH_SCHED_SYM_SHIFT = 3,
  DASH_SCHED_ATOMIC = 4,
  DASH_SCHED_AUTO = 5      /* deterministic; the library picks one with dash_schedule_choose */
};

/* Optional knobs of dash_attn_bwd.  Zero-initialise, then set struct_size. */
typedef struct dash_bwd_opts {
  uint32_t struct_size;      /* sizeof(dash_bwd_opts) */
  int num_workgroups;        /* persistent workgroups; 0 = one per compute unit */
  int tile;                  /* tile edge 64 or 128; 0 = 64 when min(Sq, Sk) < 512 else 128 */
  int atomic_walk;           /* ATOMIC only: walk of SERIAL/DESC_Q/SHIFT/SYM_SHIFT; <0 = SERIAL (full) / DESC_Q (causal) */
  int xcd_local;             /* gang members on one chiplet where possible: 1 (default when 0) / -1 off */
  void* workspace;           /* optional device workspace, 256-byte aligned; NULL = library-managed */
  size_t workspace_bytes;    /* size of `workspace` (>= dash_attn_bwd_workspace_bytes) */
  unsigned long long* stall_cycles_out; /* optional device buffer [num_workgroups][2]: cycles spent waiting
                                           on dQ semaphores, cycles in the persistent kernel (per workgroup) */
  unsigned long long spin_timeout_cycles; /* semaphore wait budget per wait; 0 = 2^33 cycles (~3.6 s) */
  int sync_check;            /* 1: synchronise the stream and report DASH_ERR_TIMEOUT / HIP faults */
  void* event_start;         /* optional hipEvent_t recorded on `stream` just before the persistent kernel */
  void* event_stop;          /* optional hipEvent_t recorded on `stream` just after it */
  int max_gang;              /* SHIFT / SYM_SHIFT (and their ATOMIC walks): cap on the gang size; a capped
                                gang takes its key/value tiles (or tile pairs) in rounds, so more gangs run
                                side by side.  0 = natural size (N, or N/2); negative = DASH_ERR_INVALID_ARG.
                                The band shift of dash_attn_bwd_window deals its units over all workgroups
                                and ignores this cap. */
  uint32_t debug_delay_seed; /* testing: non-zero runs a separate build of the persistent kernel that sleeps
                                a seeded 0..63 x 64 clocks before every dQ semaphore wait and release (a hash
                                of seed, workgroup, step, wave); the result must be bitwise that of seed 0.
                                Deterministic schedules only (ATOMIC: DASH_ERR_INVALID_ARG). */
  int* xcc_id_out;           /* optional device buffer [num_workgroups]: the chiplet (XCC) each workgroup ran
                                on, read from the hardware register */
} dash_bwd_opts;

/*
 * Forward pass: O = softmax(scale * Q K^T [+ causal mask]) V and its
 * log-sum-exp per query row.  O is bfloat16 [B,Hq,S,D], lse float32 [B,Hq,S].
 * The backward pass takes O and lse from here.
 */
int dash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int S, int D, float softmax_scale, int mask,
                  void* stream);

/*
 * Forward pass with Sq query rows and Sk key/value rows: Q, O bfloat16
 * [B,Hq,Sq,D], K, V bfloat16 [B,Hkv,Sk,D], lse float32 [B,Hq,Sq].  The causal
 * mask is aligned at the bottom right (query row i sees keys 0 .. i + Sk - Sq)
 * and needs Sk >= Sq (DASH_ERR_INVALID_ARG otherwise).  dash_attn_fwd is the
 * case Sq = Sk = S.
 */
int dash_attn_fwd_qk(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int D, float softmax_scale, int mask,
                     void* stream);

/*
 * Forward pass with a banded (sliding-window) mask: query row i sees key j
 * when -window_left <= j - (i + Sk - Sq) <= window_right, i.e. up to
 * window_left keys before its diagonal key and window_right after it; -1
 * leaves a side unbounded, so (-1, -1) is the full mask and (-1, 0) the
 * causal one (banded masks are among the scenarios [ascend]'s abstract
 * requires a deterministic backward to serve).  A side at least as wide as the sequence
 * is unbounded.  A bounded side needs Sk >= Sq (DASH_ERR_INVALID_ARG
 * otherwise).  Shapes as in dash_attn_fwd_qk.
 */
int dash_attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int Sq, int Sk, int D, float softmax_scale,
                         int window_left, int window_right, void* stream);

/*
 * Failure reporting of the backward calls.  A persistent workgroup that waits
 * longer than spin_timeout_cycles on a dQ semaphore (which only happens when
 * the grid is not co-resident, e.g. another kernel holds compute units) gives
 * up; every later wait of the call then returns at once, so the kernel ends
 * without further waiting.  The call's dQ, dK and dV are
 * then written with NaN, and a per-device host-visible word records the
 * failure: the next dash_attn_bwd* call on the device returns
 * DASH_ERR_TIMEOUT (and launches nothing), as does dash_check_async_error.
 * With sync_check the call itself synchronises and returns it.
 *
 * Workspace.  With opts->workspace NULL the library keeps one grow-only
 * workspace per (device, stream): calls on one stream share it in stream
 * order; calls on different streams never share one.  (A destroyed stream's
 * workspace is kept until process exit; a new stream with the same handle
 * value reuses it.)  The first call of a shape allocates its step lists and
 * copies them with hipMemcpyAsync on `stream`; later calls of the shape
 * allocate nothing as long as the workspace is large enough.  Up to 64 step
 * lists are cached per process; evicting one synchronises the device.
 *
 * Backward pass: dQ, dK, dV (bfloat16) from Q, K, V, O, dO (bfloat16) and
 * lse (float32).  schedule is a dash_schedule_kind; DASH_SCHED_AUTO runs
 * the one dash_schedule_choose picks (with its gang cap unless opts sets
 * max_gang).  Runs the Delta = rowsum(dO * O) preprocess, the persistent
 * backward kernel (one workgroup per compute unit; each key/value tile's
 * chain stays on one workgroup with dK/dV in registers, [summary] §2.1), and
 * the dQ fp32 -> bf16 finalize.  For the deterministic schedules the result
 * is bitwise identical from run to run.  It is also independent of
 * num_workgroups whenever the accumulation order does not depend on it:
 * always for SERIAL and DESC_Q, and for SHIFT / SYM_SHIFT while the gang is
 * not capped (a gang cap, given or chosen by AUTO, changes the order).  The
 * order of the band shift of dash_attn_bwd_window depends on how its units
 * fall into rounds of num_workgroups.
 * `opts` may be NULL.
 */
int dash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                  const float* lse, void* dq, void* dk, void* dv,
                  int B, int Hq, int Hkv, int S, int D, float softmax_scale, int mask,
                  int schedule, const dash_bwd_opts* opts, void* stream);

/*
 * Backward pass with Sq query rows and Sk key/value rows (shapes and mask as
 * in dash_attn_fwd_qk; dQ like Q, dK/dV like K).  Tile grid: Nk = ceil(Sk/T)
 * key/value tiles; full mask: Nq = ceil(Sq/T) query tiles; causal: the query
 * tiles start (Sk - Sq) mod T rows before the first query row, so that they
 * line up with the key/value tiles, and Nq = Nk - floor((Sk - Sq)/T).
 * Schedules over the Nq x Nk tile grid: SERIAL and DESC_Q walk the
 * query tiles that see each key/value tile; SHIFT (full mask) runs a gang of
 * min(Nq, Nk) workgroups, the member holding key/value tile i visiting query
 * tiles (i + t) mod Nq (with Nk > Nq member p holds tiles p, p + Nq, ... in
 * turn); SYM_SHIFT (causal, Nq even) runs the square schedule on the last Nq
 * key/value tiles and hands the Nk - Nq fully visible ones to the same N/2
 * members in shifted rounds.  dash_attn_bwd_workspace_bytes with S = Sq gives
 * enough workspace.
 */
int dash_attn_bwd_qk(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv,
                     int B, int Hq, int Hkv, int Sq, int Sk, int D, float softmax_scale, int mask,
                     int schedule, const dash_bwd_opts* opts, void* stream);

/*
 * Backward pass with the banded mask of dash_attn_fwd_window.  The tile grid
 * is the causal one of dash_attn_bwd_qk (query tiles aligned with the
 * key/value tiles); a window of w rows reaches ceil(w / T) tiles off the
 * diagonal tile, and only tile pairs inside that band are scheduled.  SERIAL,
 * DESC_Q and ATOMIC (default walk DESC_Q) serve every band; walked
 * descending, the chains of neighbouring key/value tiles reach each dQ tile
 * in ordinal order, one step apart.  SHIFT serves sliding bands (window
 * right edge 0, left edge of 1 .. Nq-1 tiles) when Nk = Nq and the left
 * extent is even, or Nk - Nq >= the left extent: units of left + 1 steps
 * (an unclipped key/value tile; the pair of tiles clipped at the first and
 * the last query tile; the symmetric shift of the corner triangle) are
 * dealt round-robin over the workgroups, and each dQ tile ranks its
 * contributors by lock-step position.  AUTO picks SHIFT where it applies,
 * else DESC_Q (dash_schedule_choose_band).  SYM_SHIFT, and SHIFT elsewhere,
 * are DASH_ERR_UNSUPPORTED unless the window reduces to the full or causal
 * mask.  Keys that no query sees get dK = dV = 0.
 */
int dash_attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dO,
                         const float* lse, void* dq, void* dk, void* dv,
                         int B, int Hq, int Hkv, int Sq, int Sk, int D, float softmax_scale,
                         int window_left, int window_right, int schedule,
                         const dash_bwd_opts* opts, void* stream);

/*
 * Allocation-free backward pass, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, results and bits as dash_attn_bwd_qk,
 * but it calls no hipMalloc, hipFree or other allocating device routine: the
 * workspace (fp32 dQ accumulator, Delta, semaphores, error word) and the
 * step lists live in a static device array of 144 MiB per GPU (allocated
 * when the library's code object holding it is first used in the process,
 * held until the process ends).  Problems whose workspace plus step lists
 * exceed it return DASH_ERR_WORKSPACE before anything is launched (B1 Hq16
 * S16384 D128 needs about 133 MiB).  opts->workspace must be NULL
 * (DASH_ERR_INVALID_ARG).  Step lists are built in host memory on a shape's
 * first call and copied into the array with hipMemcpyAsync on `stream` when
 * the shape differs from the previous call's on the device.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams, or from several threads) race and give wrong
 * results; calls on one stream are ordered.  A semaphore give-up writes NaN
 * to dQ, dK, dV and is reported by dash_check_async_error (or by this call
 * with sync_check), not by the next call.
 */
int dash_attn_bwd_qk_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                             const float* lse, void* dq, void* dk, void* dv,
                             int B, int Hq, int Hkv, int Sq, int Sk, int D, float softmax_scale, int mask,
                             int schedule, const dash_bwd_opts* opts, void* stream);

/* Bytes of device workspace dash_attn_bwd needs for these sizes (fp32 dQ
 * accumulator over the query tiles' rows, Delta, semaphores, error word,
 * scratch tiles); an upper bound valid for any key length and tile when
 * S = Sq.  mask (DASH_MASK_*) and schedule (dash_schedule_kind) are checked
 * but do not change the size: every schedule uses the same layout.  Returns
 * DASH_OK or DASH_ERR_INVALID_ARG. */
int dash_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D, int mask, int schedule, size_t* bytes);

/* Synchronises `stream`, then returns DASH_ERR_TIMEOUT (and clears the
 * record) if a backward call on the current device gave up on a dQ semaphore
 * since the last report, else DASH_OK (DASH_ERR_HIP if synchronising fails). */
int dash_check_async_error(void* stream);

/* Delta[b,h,i] = sum_d dO[b,h,i,d] * O[b,h,i,d] in fp32 ([B*H*S] float32
 * output), the preprocess step of the backward pass, exposed for testing. */
int dash_attn_bwd_delta(const void* o, const void* dO, float* delta, int B, int H, int S, int D,
                        void* stream);

/* ---- host-only schedule interface (no GPU needed) ---------------------- */

/* Opaque per-workgroup step lists for one problem shape. */
typedef struct dash_schedule dash_schedule;

/* Build step lists for `groups` key/value groups of g query heads each,
 * N tiles per sequence and P workgroups.  schedule may be any of the five
 * kinds (ATOMIC builds the walk of `atomic_walk` as in dash_bwd_opts).
 * xcd_local != 0 places the members of a gang on indices congruent modulo
 * the gang count; max_gang caps gang sizes as in dash_bwd_opts.  *out
 * receives a schedule to free with dash_schedule_free. */
int dash_schedule_build(int mask, int schedule, int N, int g, int groups, int P, int xcd_local,
                        int atomic_walk, int max_gang, dash_schedule** out);

/* Same for Nq query tiles and Nk key/value tiles (causal: Nk >= Nq, aligned
 * at the bottom right; gang schedules extended as in dash_attn_bwd_qk). */
int dash_schedule_build_qk(int mask, int schedule, int Nq, int Nk, int g, int groups, int P, int xcd_local,
                           int atomic_walk, int max_gang, dash_schedule** out);

/* Same for a band mask in tile units: key/value tile kj is visible from query
 * tile qi when -band_left <= kj - qi - (Nk - Nq) <= band_right (-1 leaves a
 * side unbounded; Nk >= Nq).  Key/value tiles that no query tile sees get
 * no chain; each dQ tile ranks its visible key/value tiles in ascending
 * order.  SERIAL, DESC_Q and ATOMIC for every band; SHIFT for the sliding
 * bands of dash_attn_bwd_window (DASH_ERR_UNSUPPORTED otherwise). */
int dash_schedule_build_band(int schedule, int Nq, int Nk, int band_left, int band_right, int g, int groups,
                             int P, int xcd_local, int atomic_walk, int max_gang, dash_schedule** out);

int dash_schedule_num_workgroups(const dash_schedule* s);
long long dash_schedule_num_steps(const dash_schedule* s);

/* Copy the lists out: offsets[P+1] (step index where each workgroup's list
 * starts) and steps[4*num_steps] as (head, qi, kj, ord | flags) with
 * flags bit 28 = first step of a chain, bit 29 = last step of a chain. */
int dash_schedule_export(const dash_schedule* s, int32_t* offsets, int32_t* steps);

/* DASH_OK, or DASH_ERR_INVALID_SCHEDULE if any step is out of range or
 * masked, a tile pair is missing or repeated, a chain is split, a dQ tile's
 * ordinals are not 0..count-1, or the lists can deadlock. */
int dash_schedule_validate(const dash_schedule* s);

/* Unit-cost DAG model ([news] §2.2; [summary] §2.1): each step costs c of
 * compute then r of reduction, a reduction waits for its dQ tile's previous
 * ordinal.  jitter_seed != 0 scales the compute cost of step i of workgroup w
 * by a factor in [0.5, 1.5): 0.5 + (splitmix64(seed ^ (w << 32 | i)) >> 11)
 * * 2^-53, with SplitMix64's output function (Steele, Lea and Flood, OOPSLA
 * 2014) applied to its argument plus 0x9e3779b97f4a7c15; 0 = no jitter.
 * Returns makespan and total waiting time; DASH_ERR_INVALID_SCHEDULE if the
 * lists deadlock, DASH_ERR_INVALID_ARG for negative costs. */
int dash_schedule_simulate(const dash_schedule* s, double c, double r, uint64_t jitter_seed,
                           double* makespan, double* total_wait);

void dash_schedule_free(dash_schedule* s);

/* Adaptive choice among the deterministic schedules for one problem shape:
 * N tiles per sequence, head dim D, g query heads per key/value head, P
 * workgroups.  The rule comes from measurements on MI355X, where the gang
 * schedules beat SERIAL and DESC_Q on every measured shape (full and causal,
 * D = 64 and 128, g = 1 and 4); the pages' H800 preference for DESC_Q at
 * D > 64 ([summary] §3, register spilling) does not carry over, because
 * dK/dV never spill in this kernel.  So:
 *   full mask                 -> SHIFT
 *   causal mask, N even       -> SYM_SHIFT
 *   causal mask, N odd        -> DESC_Q
 * and a gang larger than P (N, or N/2, > P) is capped at P (*max_gang = P,
 * the gang takes its tiles in rounds); otherwise *max_gang = 0.  D and g are
 * part of the key but do not change the choice on this hardware.
 * DASH_ERR_INVALID_ARG for non-positive sizes or an unknown mask. */
int dash_schedule_choose(int mask, int N, int D, int g, int P, int* schedule, int* max_gang);

/* Same for Nq query tiles and Nk key/value tiles: full mask -> SHIFT (gang of
 * min(Nq, Nk), capped at P); causal -> SYM_SHIFT when Nq is even, else DESC_Q. */
int dash_schedule_choose_qk(int mask, int Nq, int Nk, int D, int g, int P, int* schedule, int* max_gang);

/* Same for a band mask in tile units (as in dash_schedule_build_band): SHIFT
 * where the band shift applies (measured faster than DESC_Q on MI355X for a
 * 4096-key sliding window over 16384 tokens), else DESC_Q; *max_gang = 0. */
int dash_schedule_choose_band(int Nq, int Nk, int band_left, int band_right, int D, int g, int P, int* schedule,
                              int* max_gang);

/* ---- misc -------------------------------------------------------------- */

const char* dash_status_string(int status);
/* Message of the last error raised on the calling thread ("" if none). */
const char* dash_last_error(void);
/* Compute units, chiplets (XCDs), LDS bytes per workgroup and shader clock
 * (kHz) of a device; any output may be NULL. */
int dash_device_info(int device, int* num_cu, int* num_xcd, int* lds_bytes, int* clock_khz);

#ifdef __cplusplus
}
#endif

#endif /* DASH_ATTN_H */
