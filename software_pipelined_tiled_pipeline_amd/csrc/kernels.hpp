// The pgemm kernels.
//
//  s32_nn_kernel  int32 NN, one output per thread, VALU multiply-add,
//                 prologue / steady / epilogue over a two-slot ring whose
//                 slot roles are swapped after every tile.
//  nt_swap_kernel f16/bf16 NT, one schedule for all waves: every wave runs
//                 MFMA on tile t and, in tile t's last k32 step, refills
//                 tile t's slot with its share of tile t+S (direct-to-LDS
//                 loads); one workgroup barrier per tile (two on the
//                 large tile's two-slot ring, see kSplitSync).
//  nt_ws_kernel   f16/bf16 NT, producer waves and consumer waves coordinated
//                 by per-slot full/empty credit counters in LDS.
//  nt_ws_persistent_kernel
//                 the same roles over a fixed grid that strides through the
//                 output tiles, the ring and its credits running across them.
//
// The f16/bf16 kernels multiply with v_mfma_f32_16x16x32 (wave_mma.hpp).
//
// Pipelining follows Croqtile ch.6 ("Synchronization: pipelines, events and
// double buffering") and the modulo schedule of the TileLang chapter
// "pipeline-sync-multibuffer" (section 2.3: prologue, rolled steady body,
// epilogue; section 2.4: a buffer written in stage 0 and read S-1 stages
// later needs S versions).
#pragma once

#include <type_traits>

#include "wave_mma.hpp"

namespace pgemm {

// ================================================================ int32 NN

// Output tile (px, py) is out[16 px .. 16 px + 15][16 py .. 16 py + 15], and
// thread (qx, qy) of the workgroup owns element (16 px + qx, 16 py + qy);
// tile t of lhs is rows 16 px.., columns 16 t..; tile t of rhs is rows
// 16 t.., columns 16 py...  Elements outside the matrices load as zero.
// The grid is one-dimensional: workgroup b takes tiles b, b + gridDim.x, ...
// (tile id = py * tiles_m + px), so that any shape launches within the
// dispatch limits; a grid with one workgroup per tile takes one tile each.
template <int S>
__global__ void __launch_bounds__(256) s32_nn_kernel(const int32_t *__restrict__ lhs,
                                                     const int32_t *__restrict__ rhs,
                                                     int32_t *__restrict__ out, int M, int N, int K, int tiles_m,
                                                     int64_t tiles) {
  constexpr int T = 16;
  __shared__ int32_t lhs_s[S][T][T];
  __shared__ int32_t rhs_s[S][T][T];
  const int qx = threadIdx.x / T, qy = threadIdx.x % T;
  const int n_k = K / T + (K % T != 0);  // K + T - 1 could overflow

  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int px = (int)(tile % tiles_m), py = (int)(tile / tiles_m);
    const int gm = px * T + qx, gn = py * T + qy;
    int32_t a_reg = 0, b_reg = 0;
    auto fetch = [&](int t) {  // global -> registers
      const int ka = t * T + qy, kb = t * T + qx;
      a_reg = (gm < M && ka < K) ? lhs[(int64_t)gm * K + ka] : 0;
      b_reg = (kb < K && gn < N) ? rhs[(int64_t)kb * N + gn] : 0;
    };
    auto put = [&](int slot) {  // registers -> LDS slot
      lhs_s[slot][qx][qy] = a_reg;
      rhs_s[slot][qx][qy] = b_reg;
    };
    uint32_t acc = 0;  // wraps modulo 2^32
    auto mac = [&](int slot) {
#pragma unroll
      for (int k = 0; k < T; ++k) acc += (uint32_t)lhs_s[slot][qx][k] * (uint32_t)rhs_s[slot][k][qy];
    };

    if constexpr (S == 1) {
      for (int t = 0; t < n_k; ++t) {
        fetch(t);
        put(0);
        __syncthreads();
        mac(0);
        __syncthreads();
      }
    } else {
      if (n_k > 0) {
        int cur = 0, nxt = 1;
        fetch(0);  // prologue: tile 0 into the current slot
        put(cur);
        __syncthreads();
        for (int t = 1; t < n_k; ++t) {  // steady state
          fetch(t);                      // loads of tile t in flight ...
          mac(cur);                      // ... while tile t-1 is consumed
          put(nxt);
          __syncthreads();
          const int tmp = cur;  // swap the slot names, not the bytes
          cur = nxt;
          nxt = tmp;
        }
        mac(cur);  // epilogue: drain the last tile
        // the next output tile's prologue writes slot 0, which every
        // thread may still be reading here
        __syncthreads();
      }
    }
    if (gm < M && gn < N) out[(int64_t)gm * N + gn] = (int32_t)acc;
  }
}

// ============================================================== NT common

// Direct-to-LDS fill of one ring slot.  The slot's INSTR wave-instructions
// (64 granules each: first the A tile rows, then the B tile rows) are split
// over the loading waves; this wave issues instructions first .. first+count-1.
// Granule g of a tile is row g / CPR, position g % CPR, which holds logical
// chunk (g % CPR) ^ swz(row): the global source is chosen to match.  Rows past
// the matrix edge fall outside the buffer resource and read zero; chunks past
// K are sent to an out-of-range offset (K is a multiple of 8, so a chunk is
// either wholly inside or wholly outside).
template <int BM, int BN, int BK>
struct SlotLoader {
  using Row = RingRow<BK>;
  static constexpr bool DIRECT = true;
  static constexpr int CPR = Row::CPR;
  static constexpr int A_INSTR = BM * CPR / kWave;
  static constexpr int INSTR = (BM + BN) * CPR / kWave;
  static constexpr int SLOT_BYTES = (BM + BN) * Row::ROW_BYTES;
  static constexpr int RPI = kWave / CPR;  // rows per instruction
  // Within instruction jj (of the A or the B tile), lane l covers row
  // jj * RPI + l / CPR, whose swizzle ((jj * RPI + l / CPR) / 2) mod CPR
  // depends on jj only through jj mod PAR (RPI / 2 = 32 / CPR is a multiple
  // of CPR / PAR).
  static constexpr int PAR = CPR / 4;
  static_assert((RPI / 2) * PAR % CPR == 0, "swizzle period in instructions");
  static_assert(A_INSTR % PAR == 0, "instruction parity is the same in both tiles");
  static_assert((BM * CPR) % kWave == 0 && (BN * CPR) % kWave == 0, "tiles fill whole instructions");

  __amdgpu_buffer_rsrc_t ra, rb;
  int pitch;  // elements per row of lhs and rhs (the full K)
  int klen;   // K extent this workgroup reads, from column kb on
  int nk;     // K tiles in that extent
  int rot;    // the workgroup's K tiles are visited from tile `rot` on, wrapping
  uint32_t lane_off[PAR];  // (l / CPR) * row bytes + chunk * 16, per parity
  int lane_k[PAR];         // chunk * 8: the lane's first k within the tile

  // Tiles cover rows m0.. of lhs and n0.. of rhs, columns kb .. kb+klen-1.
  // The resources start at column kb and end at the last row's end, so a
  // row past the matrix edge is out of range while every in-matrix element
  // of the K range is inside.
  __device__ __forceinline__ void init(const uint16_t *lhs, const uint16_t *rhs, int M, int N, int K, int kb,
                                       int klen_, int m0, int n0, int rot_ = 0) {
    pitch = K;
    klen = klen_;
    nk = (klen + BK - 1) / BK;
    rot = rot_;
    const int rows_a = M - m0 < BM ? M - m0 : BM;
    const int rows_b = N - n0 < BN ? N - n0 : BN;
    ra = make_rsrc(lhs + (int64_t)m0 * K + kb, ((uint32_t)rows_a * (uint32_t)K - (uint32_t)kb) * 2u);
    rb = make_rsrc(rhs + (int64_t)n0 * K + kb, ((uint32_t)rows_b * (uint32_t)K - (uint32_t)kb) * 2u);
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int p = 0; p < PAR; ++p) {
      const int chunk = (lane % CPR) ^ Row::swz(p * RPI + lane / CPR);
      lane_off[p] = (uint32_t)(lane / CPR) * (uint32_t)K * 2u + (uint32_t)chunk * 16u;
      lane_k[p] = chunk * 8;
    }
  }

  // Instruction j = first + i of the slot for the t-th K tile of the sequence
  // (lane l -> granule 64 j + l); p = j mod PAR, passed as a constant (every
  // caller's first instruction is a multiple of PAR, as is A_INSTR) so that
  // the per-lane arrays stay in registers.  `first` is a multiple of 4 and i
  // a constant after unrolling, so instructions first + 4q .. first + 4q + 3
  // share one LDS base (one M0 value).  The t-th tile is K tile
  // (t + rot) mod nk; t >= nk (issued past the end) stays out of range.
  __device__ __forceinline__ void load_one(char *slot, int t, int first, int i, int p) const {
    const int j = first + i;
    const bool is_a = j < A_INSTR;
    const int jj = is_a ? j : j - A_INSTR;
    int kt = t;
    if (t < nk) {
      kt = t + rot;
      if (kt >= nk) kt -= nk;
    }
    const int k0 = kt * BK;
    uint32_t voff = lane_off[p] + (uint32_t)(jj * RPI) * (uint32_t)pitch * 2u;
    if (lane_k[p] >= klen - k0) voff = kOobOffset;  // chunk past K (every lane, past the last tile)
    char *base = slot + (first + (i & ~3)) * (kWave * 16);
    const __amdgpu_buffer_rsrc_t rs = is_a ? ra : rb;
    switch (i & 3) {
      case 0: load_lds_x4<0>(rs, base, voff, (uint32_t)k0 * 2u); break;
      case 1: load_lds_x4<1>(rs, base, voff, (uint32_t)k0 * 2u); break;
      case 2: load_lds_x4<2>(rs, base, voff, (uint32_t)k0 * 2u); break;
      default: load_lds_x4<3>(rs, base, voff, (uint32_t)k0 * 2u); break;
    }
  }

  // Instructions first .. first+COUNT-1 of the slot for tile t.
  template <int COUNT>
  __device__ __forceinline__ void load(char *slot, int t, int first, int lane) const {
    (void)lane;
#pragma unroll
    for (int i = 0; i < COUNT; ++i) load_one(slot, t, first, i, i % PAR);
  }
};

// Register-staged fill of one ring slot, for the calls the direct path
// cannot take: rows that do not start on 16 bytes (K not a multiple of 8),
// and panels whose byte span passes the 32-bit offsets of a buffer resource
// (long K).  It fills exactly the slot layout of SlotLoader (instruction j,
// lane l -> granule 64 j + l at the same swizzled position), so consumers
// are unchanged.  Each lane builds its 16-byte granule in registers from
// global loads with 64-bit addresses:
//   - K a multiple of 8: one 16-byte load per granule (a granule then lies
//     wholly inside or wholly outside the K range);
//   - otherwise eight 2-byte loads, each guarded by the K bound, so that an
//     element past K is zero and never read (Croqtile ch.5, predicated
//     execution with `if`: partial tiles are protected element by element).
// Rows past the matrix edge are zero.  The choice between the two is made
// once per launch (the same for every wave).  The granule is then written
// with ds_write_b128; a load call returns with its writes issued, so the
// LDS wait that precedes the next barrier or credit trigger covers them.
// Tiles at or past the end of the sequence write nothing (no later read of
// those slots is used).
template <int BM, int BN, int BK>
struct StagedLoader {
  using Row = RingRow<BK>;
  static constexpr bool DIRECT = false;
  static constexpr int CPR = Row::CPR;
  static constexpr int A_INSTR = BM * CPR / kWave;
  static constexpr int INSTR = (BM + BN) * CPR / kWave;
  static constexpr int SLOT_BYTES = (BM + BN) * Row::ROW_BYTES;
  static constexpr int RPI = kWave / CPR;
  static constexpr int PAR = CPR / 4;

  const uint16_t *pa, *pb;  // element (row 0, column kb) of the tile's lhs / rhs rows
  int64_t pitch;            // elements per row (the full K)
  int rows_a, rows_b;       // rows of the tile inside the matrices
  int klen, nk, rot;
  bool vec;                 // K a multiple of 8: 16-byte loads
  int lrow;                 // l / CPR: the lane's row within an instruction
  int lane_k[PAR];          // chunk * 8 per parity, as in SlotLoader

  __device__ __forceinline__ void init(const uint16_t *lhs, const uint16_t *rhs, int M, int N, int K, int kb,
                                       int klen_, int m0, int n0, int rot_ = 0) {
    pitch = K;
    klen = klen_;
    nk = (klen + BK - 1) / BK;
    rot = rot_;
    vec = (K & 7) == 0;
    rows_a = M - m0 < BM ? M - m0 : BM;
    rows_b = N - n0 < BN ? N - n0 : BN;
    pa = lhs + (int64_t)m0 * K + kb;
    pb = rhs + (int64_t)n0 * K + kb;
    const int lane = threadIdx.x & (kWave - 1);
    lrow = lane / CPR;
#pragma unroll
    for (int p = 0; p < PAR; ++p) lane_k[p] = ((lane % CPR) ^ Row::swz(p * RPI + lane / CPR)) * 8;
  }

  // The granule of instruction j for the t-th K tile of the sequence, in
  // registers (zero outside the matrices).
  __device__ __forceinline__ u32x4 fetch(int t, int j, int p) const {
    const bool is_a = j < A_INSTR;
    const int jj = is_a ? j : j - A_INSTR;
    int kt = t + rot;
    if (kt >= nk) kt -= nk;
    const int row = jj * RPI + lrow;
    const int k = kt * BK + lane_k[p];  // relative to the workgroup's first column
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < (is_a ? rows_a : rows_b)) {
      const uint16_t *src = (is_a ? pa : pb) + (int64_t)row * pitch + k;
      if (vec) {
        if (k < klen) v = *reinterpret_cast<const u32x4 *>(src);
      } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = k + e < klen ? (uint32_t)src[e] : 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = h[2 * q] | (h[2 * q + 1] << 16);
      }
    }
    return v;
  }

  __device__ __forceinline__ static void put(char *slot, int j, u32x4 v) {
    const int lane = threadIdx.x & (kWave - 1);
    *reinterpret_cast<u32x4 *>(slot + j * (kWave * 16) + lane * 16) = v;
  }

  __device__ __forceinline__ void load_one(char *slot, int t, int j, int p) const {
    if (t >= nk) return;
    put(slot, j, fetch(t, j, p));
  }

  // The largest batch of at most four instructions that divides `count`
  // and is a whole number of parity periods.
  static constexpr int batch(int count) {
    for (int b = 4; b > 0; --b)
      if (count % b == 0 && b % PAR == 0) return b;
    return 0;
  }

  // Instructions first .. first+COUNT-1 of the slot for tile t, in batches
  // of up to four granules: a batch's global loads, then its LDS writes
  // (four granules in flight bound the staging registers).
  template <int COUNT>
  __device__ __forceinline__ void load(char *slot, int t, int first, int lane) const {
    (void)lane;
    if (t >= nk) return;
    constexpr int B = batch(COUNT);
    static_assert(B > 0, "batches keep the parity pattern");
#pragma unroll
    for (int b = 0; b < COUNT; b += B) {
      u32x4 v[B];
#pragma unroll
      for (int i = 0; i < B; ++i) v[i] = fetch(t, first + b + i, i % PAR);
#pragma unroll
      for (int i = 0; i < B; ++i) put(slot, first + b + i, v[i]);
    }
  }
};

// Load issuers for mixed_step: call i issues instruction first + i of the
// slot for `tile` (first is a multiple of the loader's parity period).
template <class Loader>
struct RefillLoads {
  Loader ld;
  char *slot;
  int tile, first;
  __device__ __forceinline__ void operator()(int i) const { ld.load_one(slot, tile, first, i, i % Loader::PAR); }
};
struct NoLoads {
  __device__ __forceinline__ void operator()(int) const {}
};

// First K tile a workgroup visits.  A K-split product streams its operands
// from HBM, and when all workgroups walk K in step, every one requests the
// same 128-byte column window of rows 32 KiB apart, which crowds a few HBM
// channels (4.1 TB/s for that pattern on its own, 6.3 TB/s with staggered
// starts).  Split plans therefore start each output tile at its own K tile
// and wrap around; the order depends on the tile only, so every variant and
// stage count still gives the same bits for a given plan.  Unsplit plans
// keep increasing k: their concurrently resident tiles share A and B panels
// in L2 only while they walk K in step, and staggered starts measured 2-10 %
// slower at 4096^3 and 8192^3.
template <bool SPLIT>
__device__ __forceinline__ int k_rotation(int bm, int bn, int n_k) {
  if (!SPLIT || n_k <= 1) return 0;
  return (int)(((int64_t)bm * 17 + bn) % n_k);
}

// Workgroup barrier that also orders this wave's LDS accesses before it.
__device__ __forceinline__ void lds_barrier() {
  wait_lgkmcnt0();
  __builtin_amdgcn_s_barrier();
}

template <int BN>
struct Staging {
  static constexpr int PITCH = BN * 2 + 16;  // padding spreads rows over banks
};

// Geometry of one NT kernel instance: output tile BM x BN, K tile BK, S ring
// slots, WGM x WGN math waves (each owning a (BM/WGM) x (BN/WGN) block) and
// P producer waves (0 for the single-schedule kernel).
//
// Every NT kernel computes the K range [kb, kb + klen) of its tile, with
// kb = split * k_chunk.  Without a K split (SPLIT false, one piece) that is
// all of K and the epilogue rounds to T and stores the tile; with one, the
// epilogue stores the fp32 tile into its piece's plane of `partial`
// ([splits][M][ldp]) and reduce_splits adds the planes up afterwards.
template <int BM_, int BN_, int BK_, int S_, int WGM_, int WGN_, int P_, int OCC_ = 1>
struct NtGeom {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_;
  static constexpr int WGM = WGM_, WGN = WGN_, P = P_;
  static constexpr int OCC = OCC_;  // waves per SIMD the register budget allows
  static constexpr int CW = WGM * WGN;  // math waves
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int THREADS = (CW + P) * kWave;
  using Loader = SlotLoader<BM, BN, BK>;
  static constexpr int LOADERS = P > 0 ? P : CW;  // waves that fill the ring
  static constexpr int PER_LOADER = Loader::INSTR / LOADERS;
  static constexpr int RING_BYTES = S * Loader::SLOT_BYTES;
  static constexpr int STAGE_BYTES = BM * Staging<BN>::PITCH;
  static constexpr int CTR_OFFSET = RING_BYTES > STAGE_BYTES ? RING_BYTES : STAGE_BYTES;
  static constexpr int LDS_BYTES = CTR_OFFSET + (P > 0 ? 2 * S * 4 : 0);
  // Registers per wave: a SIMD's 512 are shared evenly by the waves it holds
  // (every wave of a kernel gets the same count, in steps of 8).
  static constexpr int WAVES_PER_SIMD = (CW + P + 3) / 4;
  static constexpr int REGS = (512 / WAVES_PER_SIMD) / 8 * 8;
  // A consumer holds two fragment sets (reads the next k32 step during the
  // current one) when its accumulators, both sets and about 28 registers
  // of addresses and counters fit.
  static constexpr bool TWO_SETS = WM / 16 * (WN / 16) * 4 + 2 * (WM / 16 + WN / 16) * 4 + 28 <= REGS;
  static_assert(Loader::INSTR % LOADERS == 0, "loads split evenly");
  static_assert(PER_LOADER % 4 == 0, "every loader's first instruction starts a group of four (one M0 value)");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave blocks are whole 16x16 MFMA tiles");
  static_assert(S <= 4, "vmcnt wait table covers three tiles in flight");
  static_assert(P > 0 || S * PER_LOADER < 64, "in-flight loads fit the 6-bit vmcnt");
};

// ======================================================= NT, single schedule

// Every wave fills its share of the ring with direct-to-LDS loads and runs
// MFMA on its own block; one workgroup barrier per K tile.  The fragments of
// k32 step kk+1 are read while step kk's MFMAs run (two fragment sets), and
// the barrier sits at the start of a tile's last step rather than at the
// tile boundary, so the stream of MFMAs does not stop at tiles:
//
//   barrier before the last step of tile t:
//     - each wave first waits for its own loads of tile t+1 (RAW: tile t+1
//       is complete once every wave has passed);
//     - every read of tile t has been issued and drained (WAR: tile t's slot
//       is free once every wave has passed);
//   after it: all loads of tile t+S into tile t's slot are issued, spread
//   over that step's MFMAs, while the first fragments of tile t+1 are read
//   and tile t's last MFMAs run.
//
// The loads of a tile are issued S-1 tiles ahead (at the barrier in tile
// t-S, when its slot comes free) and have S-1 tiles minus one step to land.
// A tile of a single k32 step (BK = 32) has its barrier at the start of its
// only step; the fragment sets then alternate per tile, so the loop body
// covers two tiles.  S = 1 has a single slot and runs fill -> barrier ->
// compute -> barrier.  The 256 x 256 tile with two 64-deep slots splits the
// barrier in two (kSplitSync).
// Two barriers per tile for the two-slot ring of 64-deep tiles on the large
// tile (64 MFMAs per wave and k32 step).  With one barrier, the refill of
// tile t's slot can start only at that barrier (the start of tile t's last
// step) and must land by the next one, one tile later; the loads, issued
// over the first of those two steps, then have about one step to land, and
// waves waited for them on most tiles.  Yet the slot is free as soon as
// tile t's last fragments have been read (halfway through its first step),
// and tile t+2 is first read only in the second half of tile t+1's last
// step.  A WAR barrier at the first point and a RAW barrier at the second
// give each refill load between two and three steps to land (between one
// and two with the single barrier).
//
// SplitSyncPlacement<NM> places the work of a tile's two k32 steps among
// their NM MFMAs each (see WaveTile::sched_step).  First step: the reads of
// the second step's fragments, one every REA MFMAs from MFMA RA0 on; the
// WAR barrier before MFMA WAR; NLA refill loads, one every LEA MFMAs from
// LA0 on.  Second step: the other NLB refill loads, one every LEB MFMAs
// from LB0 on; the RAW barrier before MFMA RAW; the reads of the next
// tile's first-step fragments, one every REB MFMAs from RB0 on.
template <int NM>
struct SplitSyncPlacement;
template <>
struct SplitSyncPlacement<64> {  // one wave per SIMD, 128 x 128 blocks
  static constexpr int RA0 = 1, REA = 2, WAR = 40, LA0 = 42, LEA = 4, NLA = 6;
  static constexpr int LB0 = 2, LEB = 4, NLB = 10, RAW = 44, RB0 = 45, REB = 1;
};
template <class G, class Loader, class W>
constexpr bool kSplitSync = G::P == 0 && G::S == 2 && Loader::DIRECT && W::NK == 2 && W::TM * W::TN == 64;

template <typename T, class G, bool SPLIT, bool STAGED>
__global__ void __launch_bounds__(G::THREADS, G::OCC)
    nt_swap_kernel(const uint16_t *__restrict__ lhs, const uint16_t *__restrict__ rhs,
                   uint16_t *__restrict__ out, int M, int N, int K, int tiles_m, int tiles_n, int group_m,
                   int k_chunk, float *__restrict__ partial, int ldp) {
  static_assert(G::P == 0, "single-schedule kernel has no producer waves");
  // Epilogue arguments are read into SGPRs up front: a scalar load still in
  // flight when the main loop starts would turn the loop's first fragment
  // wait into a wait for every outstanding LDS read.
  __asm__ volatile("" ::"s"(out), "s"(partial), "s"(ldp));
  using Loader = std::conditional_t<STAGED, StagedLoader<G::BM, G::BN, G::BK>, typename G::Loader>;
  using Row = RingRow<G::BK>;
  using W = WaveTile<T, G::WM, G::WN, G::BK>;
  constexpr int S = G::S;
  constexpr int NK = W::NK;
  static_assert(NK == 1 || NK % 2 == 0, "fragment sets alternate per step and line up per tile or tile pair");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bm, bn, split;
  block_work(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, &bm, &bn, &split);
  const int m0 = bm * G::BM, n0 = bn * G::BN;
  const int wm = wave / G::WGN, wn = wave % G::WGN;
  const int kb = split * k_chunk;
  const int klen = K - kb < k_chunk ? K - kb : k_chunk;

  const int n_k = klen > 0 ? (klen + G::BK - 1) / G::BK : 0;
  Loader ld;
  ld.init(lhs, rhs, M, N, K, kb, klen, m0, n0, k_rotation<SPLIT>(bm, bn, n_k));
  W w;
  w.zero();
  auto slot_ptr = [&](int s) { return smem + s * Loader::SLOT_BYTES; };
  const int first = wave * G::PER_LOADER;
  const int r = W::lane_row(lane), chunk = W::lane_chunk(lane), sw = Row::swz(r);
  auto lane_a = [&](int s) { return slot_ptr(s) + (wm * G::WM + r) * Row::ROW_BYTES; };
  auto lane_b = [&](int s) { return slot_ptr(s) + (G::BM + wn * G::WN + r) * Row::ROW_BYTES; };

  if constexpr (S == 1) {
    typename W::Frags f;
    for (int t = 0; t < n_k; ++t) {
      ld.template load<G::PER_LOADER>(slot_ptr(0), t, first, lane);
      wait_vmcnt<0>();
      lds_barrier();
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        W::read_frags(f, lane_a(0), lane_b(0), kk, chunk, sw);
        w.mma_step(f);
      }
      lds_barrier();
    }
  } else if constexpr (kSplitSync<G, Loader, W>) {
    // Two slots of 64-deep tiles, two barriers per tile (see kSplitSync):
    //   step 0 of tile t (f[0]): reads of tile t's step 1 into f[1] over the
    //     first half; WAR barrier once they have landed (slot t is free
    //     everywhere); then the first loads of tile t+2 into slot t;
    //   step 1 of tile t (f[1]): the rest of those loads; RAW barrier once
    //     this wave's loads of tile t+1 have landed (tile t+1 is complete);
    //     then the reads of tile t+1's step 0 into f[0].
    // Every tile runs the same two steps, the last ones included (their
    // loads read zeros into slots that are not read again, and the last
    // reads are never used): one code path keeps the accumulators in place.
    constexpr int PER = G::PER_LOADER;
    using Pl = SplitSyncPlacement<W::TM * W::TN>;
    static_assert(PER == Pl::NLA + Pl::NLB, "the placement issues every load of the wave's share");
    typename W::Frags f[2];
    for (int j = 0; j < 2; ++j) ld.template load<PER>(slot_ptr(j), j, first, lane);
    wait_vmcnt<PER>();  // tile 0 landed
    lds_barrier();
    if (n_k > 0) W::read_frags(f[0], lane_a(0), lane_b(0), 0, chunk, sw);
    auto war = []() __attribute__((always_inline)) { lds_barrier(); };
    auto raw = []() __attribute__((always_inline)) {
      wait_vmcnt<PER>();  // still in flight: the PER loads of tile t+2
      __builtin_amdgcn_s_barrier();
    };
    const int p1 = ((4 + chunk) ^ sw) * 16, p0 = (chunk ^ sw) * 16;
    for (int t = 0; t < n_k; ++t) {
      const int s = t & 1, s1 = s ^ 1;
      RefillLoads<Loader> refill{ld, slot_ptr(s), t + 2, first};
      auto refill_rest = [&](int i) __attribute__((always_inline)) { refill(i + Pl::NLA); };
      constexpr int NR = W::TM + W::TN;
      w.template sched_step<Pl::RA0, Pl::REA, NR, Pl::LA0, Pl::LEA, Pl::NLA, Pl::WAR>(
          f[0], typename W::FragReads{f[1], lane_a(s), lane_b(s), p1}, refill, war);
      w.template sched_step<Pl::RB0, Pl::REB, NR, Pl::LB0, Pl::LEB, Pl::NLB, Pl::RAW>(
          f[1], typename W::FragReads{f[0], lane_a(s1), lane_b(s1), p0}, refill_rest, raw);
    }
  } else {
    // The prologue issues tiles 0 .. S-1.  Loads of tiles at or past the
    // end read only out-of-range offsets (zeros into slots no later tile
    // uses); issuing them anyway keeps every vmcnt target static.
    constexpr int PER = G::PER_LOADER;
    typename W::Frags f[2];
    NoLoads no_load;
    for (int j = 0; j < S; ++j) ld.template load<PER>(slot_ptr(j), j, first, lane);
    wait_vmcnt<(S - 1) * PER>();  // tile 0 landed
    lds_barrier();
    if (n_k > 0) W::read_frags(f[0], lane_a(0), lane_b(0), 0, chunk, sw);
    // Barrier of tile t, then its last step on f[C], which reads the first
    // fragments of tile t+1 into f[C ^ 1] and refills tile t's slot with
    // tile t+S.  Still in flight at the wait: tiles t+2 .. t+S-1.
    auto last_step = [&](int t, auto cur) __attribute__((always_inline)) {
      constexpr int C = decltype(cur)::value;
      wait_vmcnt<(S - 2) * PER>();  // tile t+1 landed
      lds_barrier();
      const int s1 = (t + 1) % S;
      if constexpr (Loader::DIRECT) {
        w.template mixed_step<true, PER>(f[C], f[C ^ 1], lane_a(s1), lane_b(s1), 0, chunk, sw,
                                         RefillLoads<Loader>{ld, slot_ptr(t % S), t + S, first});
      } else {
        // staged loads wait for their data before writing it: issued after
        // the step's MFMAs, their latency does not stall the MFMA stream
        w.template mixed_step<true, 0>(f[C], f[C ^ 1], lane_a(s1), lane_b(s1), 0, chunk, sw, no_load);
        ld.template load<PER>(slot_ptr(t % S), t + S, first, lane);
      }
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    if constexpr (NK == 1) {
      // One step per tile, f[t & 1] holding tile t.  The last tile runs the
      // same step as the others: its reads of the tile after it and its
      // refill only touch slots that are not read again (the refill reads
      // zeros), and one code path keeps the accumulators in place.
      for (int t = 0; t < n_k; t += 2) {
        last_step(t, C0{});
        if (t + 1 < n_k) last_step(t + 1, C1{});
      }
    } else {
      // steps 0 .. NK-2 of tile t; the last step then runs on f[1]
      auto head = [&](int t) __attribute__((always_inline)) {
        const int s = t % S;
#pragma unroll
        for (int kk = 0; kk + 1 < NK; ++kk)
          w.template mixed_step<true, 0>(f[kk & 1], f[(kk + 1) & 1], lane_a(s), lane_b(s), kk + 1, chunk, sw,
                                         no_load);
      };
      for (int t = 0; t + 1 < n_k; ++t) {
        head(t);
        last_step(t, C1{});
      }
      if (n_k > 0) {
        head(n_k - 1);
        w.template mixed_step<false, 0>(f[1], f[0], lane_a(0), lane_b(0), 0, chunk, sw, no_load);
      }
    }
  }
  // Loads of tiles past the end are still in flight (they read zeros); none
  // may land after this point, where the ring becomes the staging tile or
  // the workgroup ends.
  wait_vmcnt<0>();
  w.settle();
  if constexpr (SPLIT) {
    w.store_partial(partial + (int64_t)split * M * ldp, ldp, M, N, m0 + wm * G::WM, n0 + wn * G::WN, lane);
  } else {
    __syncthreads();  // ring no longer read: reuse it as the staging tile
    w.stage(smem, Staging<G::BN>::PITCH, wm * G::WM, wn * G::WN, lane);
    __syncthreads();
    store_staged<G::BM, G::BN, G::THREADS>(smem, Staging<G::BN>::PITCH, out, M, N, m0, n0, tid);
  }
}

// ========================================================= NT, WS (credits)

template <typename T, class G, bool SPLIT, bool STAGED>
__global__ void __launch_bounds__(G::THREADS)
    nt_ws_kernel(const uint16_t *__restrict__ lhs, const uint16_t *__restrict__ rhs,
                 uint16_t *__restrict__ out, int M, int N, int K, int tiles_m, int tiles_n, int group_m,
                 int k_chunk, float *__restrict__ partial, int ldp, uint32_t max_polls, uint32_t debug,
                 uint32_t *err) {
  static_assert(G::P > 0, "producer/consumer kernel needs producer waves");
  // Arguments used only inside or after the K loop are read into SGPRs up
  // front: a scalar load still in flight at the loop head (scalar loads
  // return out of order) turns the first fragment wait of every tile into a
  // wait for all outstanding LDS reads.
  __asm__ volatile("" ::"s"(out), "s"(partial), "s"(ldp), "s"(err), "s"(max_polls));
  const bool skip_seed = debug & 1u;  // test hooks (see jitter_sleep)
  const uint32_t jit = debug >> 1;
  using Loader = std::conditional_t<STAGED, StagedLoader<G::BM, G::BN, G::BK>, typename G::Loader>;
  using Row = RingRow<G::BK>;
  constexpr int S = G::S, C = G::CW, P = G::P;
  // Each tile loaded whole by one producer (so one trigger of a slot's
  // `full` per round), or shared by all producers (P triggers): shared when
  // K is split or when a tile takes more loads than vmcnt can count (BK =
  // 64); see the producer below.
  constexpr bool kWholeTiles = !SPLIT && Loader::INSTR < 64;
  constexpr int FP = kWholeTiles ? 1 : P;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  uint32_t *full = reinterpret_cast<uint32_t *>(smem + G::CTR_OFFSET);
  uint32_t *empty = full + S;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bm, bn, split;
  block_work(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, &bm, &bn, &split);
  const int m0 = bm * G::BM, n0 = bn * G::BN;
  const int kb = split * k_chunk;
  const int klen = K - kb < k_chunk ? K - kb : k_chunk;
  const int n_k = klen > 0 ? (klen + G::BK - 1) / G::BK : 0;
  auto slot_ptr = [&](int s) { return smem + s * Loader::SLOT_BYTES; };

  if (tid < 2 * S) full[tid] = 0u;  // full[0..S) and empty[0..S)
  __syncthreads();

  using W = WaveTile<T, G::WM, G::WN, G::BK, false>;
  W w;
  const int wm = wave / G::WGN, wn = wave % G::WGN;
  // Consumers whose block leaves room for two fragment sets within the
  // register budget (the 64 x 64 blocks of the 128 x 128 tile, not the
  // 128 x 64 ones of the large tile) read the next k32 step while the
  // current step's MFMAs run.
  constexpr bool kTwoSets = G::TWO_SETS;
  if (wave < C) {
    // ---------------------------------------------------------- consumer
    if (!skip_seed)
      for (int s = 0; s < S; ++s) credit_trigger(&empty[s]);  // every slot starts free
    w.zero();
    if constexpr (kTwoSets) {
      // The first step of tile t+1 is read during the last step of tile t,
      // so slot t is released as soon as its last reads have landed and
      // `full` of tile t+1 is waited for before that last step (its counter
      // is read at the start of the tile, so that a credit that has already
      // arrived costs no LDS round trip).  The fragment sets alternate per
      // k32 step; with one step per K tile they alternate per tile, and the
      // loop body covers two tiles.  Every tile runs the same code, the last
      // one included (it reads the slot after it: landed or never-written
      // data that is no longer refilled and is never used): with a separate
      // tail the compiler kept the accumulators in other registers there and
      // copied them right before MFMAs, a hazard it cannot see through the
      // inline asm.
      constexpr int NK = W::NK;
      const int r = W::lane_row(lane), chunk = W::lane_chunk(lane), sw = Row::swz(r);
      auto lane_a = [&](int s) { return slot_ptr(s) + (wm * G::WM + r) * Row::ROW_BYTES; };
      auto lane_b = [&](int s) { return slot_ptr(s) + (G::BM + wn * G::WN + r) * Row::ROW_BYTES; };
      typename W::Frags f[2];
      NoLoads no_load;
      if (n_k > 0) {
        jitter_sleep(jit, wave, 0, 1);
        credit_wait(&full[0], (uint32_t)FP, max_polls, err);
        W::read_frags(f[0], lane_a(0), lane_b(0), 0, chunk, sw);
      }
      // tile t, whose first step runs on f[F0]
      auto tile = [&](int t, auto f0) __attribute__((always_inline)) {
        constexpr int F0 = decltype(f0)::value;
        const int s = t % S, s1 = (t + 1) % S;
        const uint32_t next = credit_load(&full[s1]);
#pragma unroll
        for (int kk = 0; kk + 1 < NK; ++kk)
          w.template mixed_step<true, 0>(f[(F0 + kk) & 1], f[(F0 + kk + 1) & 1], lane_a(s), lane_b(s), kk + 1,
                                         chunk, sw, no_load);
        wait_lgkmcnt0();  // the last fragment reads of slot s are done
        jitter_sleep(jit, wave, t, 0);
        credit_trigger(&empty[s]);
        const uint32_t target = (uint32_t)FP * ((uint32_t)((t + 1) / S) + 1u);
        jitter_sleep(jit, wave, t + 1, 1);
        if (t + 1 < n_k && __builtin_amdgcn_readfirstlane(next) < target)
          credit_wait(&full[s1], target, max_polls, err);
        w.template mixed_step<true, 0>(f[(F0 + NK - 1) & 1], f[(F0 + NK) & 1], lane_a(s1), lane_b(s1), 0, chunk,
                                       sw, no_load);
      };
      using C0 = std::integral_constant<int, 0>;
      using C1 = std::integral_constant<int, 1>;
      if constexpr (NK % 2 == 0) {
        for (int t = 0; t < n_k; ++t) tile(t, C0{});
      } else {
        for (int t = 0; t < n_k; t += 2) {
          tile(t, C0{});
          if (t + 1 < n_k) tile(t + 1, C1{});
        }
      }
      w.settle();
    } else {
      // `full` of the next tile's slot is read at the start of each tile and
      // checked after its MFMAs, so a credit that has already arrived costs no
      // LDS round trip; only a short one is waited for.
      uint32_t seen = 0;
      for (int t = 0; t < n_k; ++t) {
        const int s = t % S;
        const uint32_t target = (uint32_t)FP * ((uint32_t)(t / S) + 1u);
        jitter_sleep(jit, wave, t, 1);
        if (seen < target) credit_wait(&full[s], target, max_polls, err);
        compiler_fence();
        const uint32_t next = t + 1 < n_k ? credit_load(&full[(t + 1) % S]) : 0u;
        char *base = slot_ptr(s);
        w.template mma_ktile<2>(base + wm * G::WM * Row::ROW_BYTES, base + (G::BM + wn * G::WN) * Row::ROW_BYTES,
                                lane);
        wait_lgkmcnt0();  // this slot's fragment reads are done (MFMAs read registers)
        jitter_sleep(jit, wave, t, 0);
        credit_trigger(&empty[s]);
        seen = __builtin_amdgcn_readfirstlane(next);
      }
      w.settle();
    }
  } else {
    // ---------------------------------------------------------- producer
    Loader ld;
    ld.init(lhs, rhs, M, N, K, kb, klen, m0, n0, k_rotation<SPLIT>(bm, bn, n_k));
    if constexpr (kWholeTiles) {
      // Producer p loads tiles p, p + P, p + 2P, ... whole, each straight
      // into its slot once the slot's `empty` credit arrives, and adds to
      // `full` as soon as that tile has landed.  The producers take turns
      // rather than all waking on the same credit and issuing their shares
      // at once, and no `full` waits for a later tile's slot to come free.
      for (int t = wave - C; t < n_k; t += P) {
        const int s = t % S;
        jitter_sleep(jit, wave, t, 2);
        credit_wait(&empty[s], (uint32_t)C * ((uint32_t)(t / S) + 1u), max_polls, err);
        ld.template load<Loader::INSTR>(slot_ptr(s), t, 0, lane);
        if constexpr (Loader::DIRECT)
          wait_vmcnt<0>();  // tile t landed
        else
          wait_lgkmcnt0();  // this wave's writes of tile t are done
        jitter_sleep(jit, wave, t, 3);
        credit_trigger(&full[s]);
      }
    } else {
      // K split (skinny products, streamed from HBM) or BK = 64: every
      // producer loads its share of every tile, so that each keeps LAG + 1
      // tiles of loads in flight.  `full` of tile t is triggered after the
      // loads of tile t + LAG are issued, when its own have landed.  LAG =
      // S - 2 keeps the consumers fed: the tile they need next is complete
      // once the producer holds the credit of the slot they just released.
      // Staged loads have written the tile by the time the call returns, so
      // `full` follows at once (LAG = 0), after the LDS writes complete.
      const int first = (wave - C) * G::PER_LOADER;
      constexpr int PER = G::PER_LOADER;
      constexpr int LAG = (Loader::DIRECT && S >= 2) ? S - 2 : 0;
      static_assert((LAG + 1) * PER < 64, "loads in flight fit the 6-bit vmcnt");
      for (int t = 0; t < n_k; ++t) {
        const int s = t % S;
        jitter_sleep(jit, wave, t, 2);
        credit_wait(&empty[s], (uint32_t)C * ((uint32_t)(t / S) + 1u), max_polls, err);
        ld.template load<PER>(slot_ptr(s), t, first, lane);
        if (t >= LAG) {
          if constexpr (Loader::DIRECT)
            wait_vmcnt<LAG * PER>();  // tile t - LAG landed
          else
            wait_lgkmcnt0();  // this wave's writes of tile t are done
          jitter_sleep(jit, wave, t, 3);
          credit_trigger(&full[(t - LAG) % S]);
        }
      }
      if constexpr (LAG >= 2) {
        if (n_k >= 2) {
          wait_vmcnt<PER>();
          jitter_sleep(jit, wave, n_k, 3);
          credit_trigger(&full[(n_k - 2) % S]);
        }
      }
      if constexpr (LAG >= 1) {
        if (n_k >= 1) {
          wait_vmcnt<0>();
          jitter_sleep(jit, wave, n_k + 1, 3);
          credit_trigger(&full[(n_k - 1) % S]);
        }
      }
    }
  }
  if constexpr (SPLIT) {
    if (wave < C)
      w.store_partial(partial + (int64_t)split * M * ldp, ldp, M, N, m0 + wm * G::WM, n0 + wn * G::WN, lane);
  } else {
    __syncthreads();  // all tiles consumed: the ring becomes the staging tile
    if (wave < C) w.stage(smem, Staging<G::BN>::PITCH, wm * G::WM, wn * G::WN, lane);
    __syncthreads();
    store_staged<G::BM, G::BN, G::THREADS>(smem, Staging<G::BN>::PITCH, out, M, N, m0, n0, tid);
  }
}

// ============================================== NT, WS, persistent schedule

// Persistent producer/consumer kernel (Croqtile ch.5, "persistent scheduling
// and the if guard"): a fixed grid of at most one workgroup per CU, each
// striding over output tiles tile_iter # block_id = tile_iter * gridDim.x +
// blockIdx.x while that is below the tile count.  The producers stream one
// continuous sequence of (tile, K tile) pairs through the ring, so the next
// tile's loads overlap the last MMAs and the epilogue of the current one;
// the credit counters keep counting across tiles (round of sequence entry g
// = g / S).  Consumers store each finished tile straight from registers, as
// the ring is already refilling.  Results are bit-identical to nt_ws_kernel
// (same tiles, same k order per element).
template <typename T, class G>
__global__ void __launch_bounds__(G::THREADS)
    nt_ws_persistent_kernel(const uint16_t *__restrict__ lhs, const uint16_t *__restrict__ rhs,
                            uint16_t *__restrict__ out, int M, int N, int K, int tiles_m, int tiles_n, int group_m,
                            uint32_t max_polls, uint32_t debug, uint32_t *err) {
  static_assert(G::P > 0, "producer/consumer kernel needs producer waves");
  __asm__ volatile("" ::"s"(out), "s"(err), "s"(max_polls));  // see nt_ws_kernel
  const bool skip_seed = debug & 1u;
  const uint32_t jit = debug >> 1;
  using Loader = typename G::Loader;
  using Row = RingRow<G::BK>;
  constexpr int S = G::S, C = G::CW, P = G::P;
  // whole entries by one producer, or shared by all of them (BK = 64), as
  // in nt_ws_kernel
  constexpr bool kWholeTiles = Loader::INSTR < 64;
  constexpr int FP = kWholeTiles ? 1 : P;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  uint32_t *full = reinterpret_cast<uint32_t *>(smem + G::CTR_OFFSET);
  uint32_t *empty = full + S;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  const int n_k = K > 0 ? (K + G::BK - 1) / G::BK : 0;
  // tiles tile_iter * gridDim.x + blockIdx.x below `tiles` (gridDim.x <= tiles)
  const int my_tiles = (int)((tiles - 1 - blockIdx.x) / gridDim.x) + 1;
  auto tile_of = [&](int it, int *bm, int *bn) {
    int split;
    block_work((int64_t)it * gridDim.x + blockIdx.x, tiles, tiles_m, tiles_n, group_m, bm, bn, &split);
  };
  auto slot_ptr = [&](int s) { return smem + s * Loader::SLOT_BYTES; };

  if (tid < 2 * S) full[tid] = 0u;  // full[0..S) and empty[0..S)
  __syncthreads();

  if (wave < C) {
    // ---------------------------------------------------------- consumer
    WaveTile<T, G::WM, G::WN, G::BK, false> w;
    const int wm = wave / G::WGN, wn = wave % G::WGN;
    if (!skip_seed)
      for (int s = 0; s < S; ++s) credit_trigger(&empty[s]);  // every slot starts free
    // `full` of the next entry's slot is read at the start of each entry and
    // checked after its MFMAs, as in nt_ws_kernel
    const uint32_t total = (uint32_t)my_tiles * (uint32_t)n_k;
    uint32_t g = 0, seen = 0;  // position in the workgroup's (tile, K tile) sequence
    for (int it = 0; it < my_tiles; ++it) {
      int bm, bn;
      tile_of(it, &bm, &bn);
      w.zero();
      for (int t = 0; t < n_k; ++t, ++g) {
        const int s = (int)(g % S);
        const uint32_t target = (uint32_t)FP * (g / S + 1u);
        jitter_sleep(jit, wave, g, 1);
        if (seen < target) credit_wait(&full[s], target, max_polls, err);
        compiler_fence();
        const uint32_t next = g + 1 < total ? credit_load(&full[(g + 1) % S]) : 0u;
        char *base = slot_ptr(s);
        w.template mma_ktile<(G::WM > 64 ? 2 : 1)>(base + wm * G::WM * Row::ROW_BYTES,
                                                    base + (G::BM + wn * G::WN) * Row::ROW_BYTES, lane);
        wait_lgkmcnt0();  // this slot's fragment reads are done (MFMAs read registers)
        jitter_sleep(jit, wave, g, 0);
        credit_trigger(&empty[s]);
        seen = __builtin_amdgcn_readfirstlane(next);
      }
      w.settle();
      w.store_direct(out, M, N, bm * G::BM + wm * G::WM, bn * G::BN + wn * G::WN, lane);
    }
  } else {
    // ---------------------------------------------------------- producer
    const uint32_t total = (uint32_t)my_tiles * (uint32_t)n_k;
    if constexpr (kWholeTiles) {
      // As in nt_ws_kernel: producer p loads entries p, p + P, ... of the
      // sequence whole, direct to LDS once the slot's `empty` credit
      // arrives, and adds to `full` once the entry has landed, now across
      // tile boundaries.
      Loader ld;
      int cur = -1;
      for (uint32_t g = (uint32_t)(wave - C); g < total; g += P) {
        const int it = (int)(g / (uint32_t)n_k), t = (int)(g - (uint32_t)it * (uint32_t)n_k);
        if (it != cur) {
          int bm, bn;
          tile_of(it, &bm, &bn);
          ld.init(lhs, rhs, M, N, K, 0, K, bm * G::BM, bn * G::BN);
          cur = it;
        }
        const int s = (int)(g % S);
        jitter_sleep(jit, wave, g, 2);
        credit_wait(&empty[s], (uint32_t)C * (g / S + 1u), max_polls, err);
        ld.template load<Loader::INSTR>(slot_ptr(s), t, 0, lane);
        wait_vmcnt<0>();  // entry g landed
        jitter_sleep(jit, wave, g, 3);
        credit_trigger(&full[s]);
      }
    } else {
      // BK = 64: every producer loads its share of each entry, and `full`
      // of entry g is triggered LAG = S - 2 entries later, as nt_ws_kernel
      // does for its shared tiles.
      constexpr int PER = G::PER_LOADER;
      constexpr int LAG = S >= 2 ? S - 2 : 0;
      static_assert((LAG + 1) * PER < 64, "loads in flight fit the 6-bit vmcnt");
      const int first = (wave - C) * PER;
      Loader ld;
      uint32_t g = 0;
      for (int it = 0; it < my_tiles; ++it) {
        int bm, bn;
        tile_of(it, &bm, &bn);
        ld.init(lhs, rhs, M, N, K, 0, K, bm * G::BM, bn * G::BN);
        for (int t = 0; t < n_k; ++t, ++g) {
          const int s = (int)(g % S);
          jitter_sleep(jit, wave, g, 2);
          credit_wait(&empty[s], (uint32_t)C * (g / S + 1u), max_polls, err);
          ld.template load<PER>(slot_ptr(s), t, first, lane);
          if (g >= (uint32_t)LAG) {
            wait_vmcnt<LAG * PER>();  // entry g - LAG landed
            jitter_sleep(jit, wave, g, 3);
            credit_trigger(&full[(g - LAG) % S]);
          }
        }
      }
      if constexpr (LAG >= 2) {
        if (g >= 2) {
          wait_vmcnt<PER>();
          jitter_sleep(jit, wave, g, 3);
          credit_trigger(&full[(g - 2) % S]);
        }
      }
      if constexpr (LAG >= 1) {
        if (g >= 1) {
          wait_vmcnt<0>();
          jitter_sleep(jit, wave, g + 1, 3);
          credit_trigger(&full[(g - 1) % S]);
        }
      }
      (void)total;
    }
  }
}

}  // namespace pgemm
