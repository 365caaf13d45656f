// Device-side building blocks shared by the pgemm kernels (gfx950 only).
//
//  * vector types for the v_mfma_f32_16x16x32_{f16,bf16} operands;
//  * buffer resources and direct-to-LDS 16-byte loads
//    (buffer_load_dwordx4 ... lds), whose out-of-range lanes read zero;
//  * the LDS ring: S slots, each an A tile [BM][BK] followed by a B tile
//    [BN][BK], stored as 16-byte granules with an XOR swizzle;
//  * the workgroup -> output-tile map (XCD-aware, grouped);
//  * credit counters in LDS (wait / trigger).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pgemm {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWave = 64;

// Buffer resource word 3 for raw (unswizzled, untyped) buffers on gfx9 parts.
constexpr int kRsrcWord3 = 0x00020000;
// Any byte offset at or above the resource's size reads as zero; this one is
// used for lanes whose chunk lies past K.  Resource sizes stay below it.
constexpr uint32_t kOobOffset = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}

// One wave-wide direct-to-LDS load: lane l copies 16 bytes from
// rsrc + voffset(l) + soffset to lds_base + 1024 G + 16 * l.  `lds_base` and
// `soffset` must be wave-uniform.  Out-of-range reads return zero.  Callers
// keep the row part of an offset in voffset and only the K offset in
// soffset, and send a lane whose chunk lies past K to kOobOffset: then a
// lane reads zero exactly when its element is outside the matrix, whether or
// not the hardware adds soffset before the bound check.
//
// The LDS destination is held in M0.  Writing M0 while an earlier
// direct-to-LDS load is still being issued stalls the wave (on gfx950 an
// MFMA stream with one such load every 4 to 8 MFMAs lost 17-26 cycles per
// load when each load set M0, 2-9 when they shared one value), so up to four
// consecutive 1 KiB destinations are reached from one base through the
// instruction offset (G KiB, at most 4095 bytes).  That offset is added to
// the global address too, so voffset is lowered by as much: the 32-bit sum
// wraps (checked on the device), and a lane sent to kOobOffset stays out of
// range.  Loads that pass the same lds_base share M0.
template <int G>
__device__ __forceinline__ void load_lds_x4(__amdgpu_buffer_rsrc_t rsrc, char *lds_base, uint32_t voffset,
                                            uint32_t soffset) {
  static_assert(G >= 0 && G < 4, "the instruction offset holds at most 4095 bytes");
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)lds_base, 16, voffset - 1024u * G, soffset, 1024 * G, 0);
}

// s_waitcnt through the builtin, so that the compiler's own wait insertion
// sees it and does not add a stricter one after it.  gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8; an all-ones field
// means "do not wait on this counter".
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// ----------------------------------------------------------------- ring ---
//
// A ring slot holds the A tile (rows of lhs) and then the B tile (rows of
// rhs), both K-contiguous.  A row of BK halves is CPR = BK/8 granules of 16
// bytes.  Logical chunk c of row r is stored at position c ^ swz(r), where
// swz(r) = (r / 2) mod CPR.  The fragment reads of a 16x16x32 MFMA (lane l
// reads row base + l % 16 at chunk 4 kk + l / 16, base a multiple of 16)
// then run at the LDS read rate of a linear access for both row widths;
// the previous swizzle, (r / (16 / CPR)) mod CPR, which suits lanes reading
// 32 rows at one chunk, ran the 64-byte rows at two thirds of that (measured
// with ds_read_b128 on gfx950).  The direct-to-LDS writes fill 1 KiB
// contiguously per instruction and never conflict.
template <int BK>
struct RingRow {
  static constexpr int CPR = BK / 8;              // granules per row
  static constexpr int ROW_BYTES = BK * 2;
  static_assert(BK == 32 || BK == 64, "BK must be 32 or 64");
  __device__ __forceinline__ static int swz(int r) { return (r >> 1) % CPR; }
};

// Work of a workgroup: output tile (bm, bn) and K piece `split`.
// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2: ids are first regrouped so that every XCD receives a contiguous run.
// The K piece is the slowest-varying part of the id, so the workgroups of
// one XCD share a K piece (and with it the slice of lhs they read); tiles
// are then walked in groups of `group_m` row panels so that concurrently
// resident tiles share A and B panels.
__device__ __forceinline__ void block_work(int64_t bid, int64_t nblocks, int tiles_m, int tiles_n, int group_m,
                                           int *bm, int *bn, int *split) {
  constexpr int kXcds = 8;
  int64_t per = nblocks / kXcds;
  int64_t id = bid;
  if (bid < per * kXcds) id = (bid % kXcds) * per + bid / kXcds;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  *split = (int)(id / tiles);
  id %= tiles;
  int64_t span = (int64_t)group_m * tiles_n;
  int64_t g = id / span;
  int64_t first = g * group_m;
  int64_t gsize = tiles_m - first < group_m ? tiles_m - first : group_m;
  int64_t in = id % span;
  *bm = (int)(first + in % gsize);
  *bn = (int)(in / gsize);
}

// -------------------------------------------------------------- credits ---
//
// Monotonic LDS counters.  trigger adds one; a waiter for round r of a slot
// waits until the counter reaches (r + 1) * (number of triggering waves).
// A wait polls with s_sleep between reads and gives up after `max_polls`
// reads, recording the failure in *err (so a protocol error can never hang
// the device).
//
// The counter read and the increment are issued as inline assembly.  The
// compiler treats every LDS access that follows a direct-to-LDS load as a
// possible alias of it and would put `s_waitcnt vmcnt(0)` in front, i.e.
// wait for every load in flight, which would undo the pipeline.  Ordering is
// explicit instead: a producer waits for its own loads with a counted
// `s_waitcnt vmcnt` before it triggers `full`; a consumer waits for its
// fragment reads (`s_waitcnt lgkmcnt(0)`) before it triggers `empty`; and
// LDS executes one wave's accesses in issue order.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

__device__ __forceinline__ uint32_t credit_peek(const uint32_t *ctr) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(ctr)) : "memory");
  return __builtin_amdgcn_readfirstlane(v);
}

// The counter's value as an ordinary LDS load: the compiler places the wait
// for it before its first use, so it can be issued well ahead of that.  For
// waves that issue no direct-to-LDS loads (those would make the compiler wait
// for them before any LDS read it cannot prove disjoint).
__device__ __forceinline__ uint32_t credit_load(const uint32_t *ctr) {
  return __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void credit_trigger(uint32_t *ctr) {
  if ((threadIdx.x & (kWave - 1)) == 0)
    asm volatile("ds_add_u32 %0, %1" ::"v"(lds_addr(ctr)), "v"(1u) : "memory");
}

// Timing jitter for testing the credit protocol.  A producer/consumer
// launch takes a debug word: bit 0 skips the seeding of `empty` (the
// protocol then cannot start, and the bounded waits give up), and bits 1-31
// hold a jitter seed.  With a non-zero seed, each wave sleeps 0 to 7 times
// 256 clocks before each credit operation.  The count is a hash of the seed,
// the workgroup, the wave, the position in the K sequence and the call site,
// so producers and consumers meet in orders their natural timing does not
// give, while the results must stay the same.  The hash is lowbias32
// (C. Wellons, "Hash function prospector", 2018).  With seed 0 the cost is
// one scalar compare per site.
__device__ __forceinline__ void jitter_sleep(uint32_t seed, int wave, uint32_t pos, uint32_t site) {
  if (seed) {
    uint32_t h = seed ^ (blockIdx.x * 0x9E3779B9u) ^ ((uint32_t)wave << 24) ^ (pos * 4u + site);
    h ^= h >> 16;
    h *= 0x7FEB352Du;
    h ^= h >> 15;
    h *= 0x846CA68Bu;
    h ^= h >> 16;
    for (uint32_t i = 0, n = h & 7u; i < n; ++i) __builtin_amdgcn_s_sleep(4);
  }
}

__device__ __forceinline__ void credit_wait(const uint32_t *ctr, uint32_t target, uint32_t max_polls,
                                            uint32_t *err) {
  uint32_t polls = 0;
  while (credit_peek(ctr) < target) {
    if (++polls > max_polls) {
      if ((threadIdx.x & (kWave - 1)) == 0) atomicOr(err, 1u);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  compiler_fence();
}

}  // namespace pgemm
