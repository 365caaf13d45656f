// Consumer-side math and the output epilogue.
//
// A wave owns a WM x WN block of the output, held as (WM/16) x (WN/16) fp32
// accumulators of v_mfma_f32_16x16x32.  Operand roles: src0 is the rhs
// fragment (16 rows n) and src1 the lhs fragment (16 rows m), so each
// accumulator holds a transposed 16x16 output block:
//   lane l, register r of acc[i][j] -> out[m0 + 16 i + l % 16][n0 + 16 j + 4 (l / 16) + r],
// i.e. a lane's four registers are four consecutive columns of one row.
//
// Both fragments are read the same way from a ring slot: lane l reads row
// (base + l % 16) at chunk 4 kk + l / 16 (eight consecutive k), for the k32
// step kk of the tile.  Every output element accumulates the k32 steps in
// increasing k, so any tile shape, stage count or variant gives the same
// bits.
//
// On gfx950 this shape sustains the same MFMA rate per clock as 32x32x16 and
// draws less power per flop (a quarter of the accumulator traffic per
// instruction), which matters on a chip whose clock is set by its power
// limit.  The MFMAs are written as inline asm with the accumulator tied to
// the destination: with the builtin, a loop body that updates each of 64
// small accumulators more than once is register-allocated with copies
// between AGPRs and VGPRs.  The compiler's hazard tracking does not look
// inside asm statements, so the wait states an MFMA result needs before
// other instructions read it are inserted by hand (settle(), zero()).
#pragma once

#include "device_common.hpp"

namespace pgemm {

template <typename T>
struct Mfma;

template <>
struct Mfma<_Float16> {
  // acc += src0 x src1^T over 32 k; ACC_AGPR picks the register file of acc
  template <bool ACC_AGPR>
  __device__ __forceinline__ static void run(u32x4 src0, u32x4 src1, f32x4 &acc) {
    if constexpr (ACC_AGPR)
      asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(src0), "v"(src1));
    else
      asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(src0), "v"(src1));
  }
  // fp32 -> binary16, round to nearest even (v_cvt_f16_f32 in the default mode)
  __device__ __forceinline__ static u32x2 pack4(float a, float b, float c, float d) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    h4 h = {(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
    return __builtin_bit_cast(u32x2, h);
  }
};

template <>
struct Mfma<__bf16> {
  template <bool ACC_AGPR>
  __device__ __forceinline__ static void run(u32x4 src0, u32x4 src1, f32x4 &acc) {
    if constexpr (ACC_AGPR)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(src0), "v"(src1));
    else
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(src0), "v"(src1));
  }
  // fp32 -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32)
  __device__ __forceinline__ static u32x2 pack4(float a, float b, float c, float d) {
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    b4 h = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
    return __builtin_bit_cast(u32x2, h);
  }
};

// ACC_AGPR: accumulators in AGPRs (one wave per SIMD, 256 of them) or in
// VGPRs (kernels with several waves per SIMD and a smaller block).
template <typename T, int WM, int WN, int BK, bool ACC_AGPR = true>
struct WaveTile {
  static constexpr int TM = WM / 16;
  static constexpr int TN = WN / 16;
  static constexpr int NK = BK / 32;  // k32 steps per K tile
  static_assert(WM % 16 == 0 && WN % 16 == 0 && BK % 32 == 0, "whole 16x16x32 MFMA tiles");
  using Row = RingRow<BK>;
  f32x4 acc[TM][TN];

  // lane -> row within a 16-row block / 16-byte chunk within a k32 step
  __device__ __forceinline__ static int lane_row(int lane) { return lane & 15; }
  __device__ __forceinline__ static int lane_chunk(int lane) { return lane >> 4; }

  // Ties every accumulator to its register at this point of the program:
  // accumulator reads and writes cannot move across it or across the
  // volatile asm statements around it.
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (ACC_AGPR)
          asm volatile("" : "+a"(acc[i][j]));
        else
          asm volatile("" : "+v"(acc[i][j]));
      }
  }

  // Zeroes the accumulators, with the wait states a register written by a
  // VALU instruction needs before an MFMA reads it as srcC.
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
    pin();
    asm volatile("s_nop 4");
  }

  // Wait states between the last MFMA and any other instruction that reads
  // or overwrites its accumulator (24; an 8-pass MFMA result needs 11).
  __device__ __forceinline__ void settle() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    pin();
  }

  // Fragments of one k32 step: TN rhs and TM lhs 16-byte pieces per lane.
  struct Frags {
    u32x4 b[TN], a[TM];
  };

  // `lane_a` / `lane_b` point at the lane's row of the wave's first lhs /
  // rhs block in a slot (blocks are 16 rows apart); chunk = lane_chunk(l),
  // s = swz(lane_row(l)), the same for every block since blocks start at
  // multiples of 16 rows.
  __device__ __forceinline__ static void read_frags(Frags &f, const char *lane_a, const char *lane_b, int kk,
                                                    int chunk, int s) {
    const int p = ((4 * kk + chunk) ^ s) * 16;
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = *reinterpret_cast<const u32x4 *>(lane_b + 16 * j * Row::ROW_BYTES + p);
#pragma unroll
    for (int i = 0; i < TM; ++i) f.a[i] = *reinterpret_cast<const u32x4 *>(lane_a + 16 * i * Row::ROW_BYTES + p);
  }

  __device__ __forceinline__ void mma_step(const Frags &f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) Mfma<T>::template run<ACC_AGPR>(f.b[j], f.a[i], acc[i][j]);
  }

  // One K tile from a ring slot with a single fragment set: the rhs pieces
  // of a k32 step first, then the lhs pieces, each AHEAD block rows before
  // the MFMAs that use it (a ring of AHEAD + 1 lhs pieces).  a_rows /
  // b_rows: LDS address of the first of this wave's lhs / rhs rows in the
  // slot.
  template <int AHEAD>
  __device__ __forceinline__ void mma_ktile(const char *a_rows, const char *b_rows, int lane) {
    static_assert(AHEAD >= 0 && AHEAD < TM, "lhs pieces read ahead within the k32 step");
    constexpr int NA = AHEAD + 1;
    const int r = lane_row(lane);
    const int chunk = lane_chunk(lane);
    const int s = Row::swz(r);
    const char *lane_a = a_rows + r * Row::ROW_BYTES;
    const char *lane_b = b_rows + r * Row::ROW_BYTES;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int p = ((4 * kk + chunk) ^ s) * 16;
      u32x4 b[TN], a[NA];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = *reinterpret_cast<const u32x4 *>(lane_b + 16 * j * Row::ROW_BYTES + p);
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) a[i] = *reinterpret_cast<const u32x4 *>(lane_a + 16 * i * Row::ROW_BYTES + p);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (i + AHEAD < TM)
          a[(i + AHEAD) % NA] = *reinterpret_cast<const u32x4 *>(lane_a + 16 * (i + AHEAD) * Row::ROW_BYTES + p);
#pragma unroll
        for (int j = 0; j < TN; ++j) Mfma<T>::template run<ACC_AGPR>(b[j], a[i % NA], acc[i][j]);
      }
    }
  }

  // One k32 step: the TM*TN MFMAs on `cf`, interleaved in a fixed order
  // with (when READS) the TM+TN fragment reads of the next step into `nf`,
  // one every RE MFMAs over the first half of the step, and NLOAD calls
  // ld_fn(0 .. NLOAD-1), one every TM*TN/NLOAD MFMAs.  Reads finish early so
  // that the wait before a barrier or before the next step finds them done;
  // loads are spread over the whole step.  sched_barrier(0) after every
  // MFMA pins the order: global loads spaced out between MFMAs never pile up
  // in the texture-address queue, where a full queue would stall the wave's
  // in-order issue, MFMAs included.
  template <bool READS, int NLOAD, class LoadFn>
  __device__ __forceinline__ void mixed_step(const Frags &cf, Frags &nf, const char *lane_a, const char *lane_b,
                                             int nkk, int chunk, int s, LoadFn &&ld_fn) {
    constexpr int NM = TM * TN;
    constexpr int NR = TM + TN;
    constexpr int RE = NM / NR / 2 > 0 ? NM / NR / 2 : 1;  // MFMAs per read
    static_assert(!READS || NR * RE <= NM, "reads fit in the step");
    static_assert(NLOAD == 0 || NM % NLOAD == 0, "loads spread evenly");
    constexpr int LE = NLOAD > 0 ? NM / (NLOAD > 0 ? NLOAD : 1) : NM + 1;  // MFMAs per load
    const int p = ((4 * nkk + chunk) ^ s) * 16;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int m = i * TN + j;
        Mfma<T>::template run<ACC_AGPR>(cf.b[j], cf.a[i], acc[i][j]);
        if constexpr (READS) {
          if (m % RE == RE - 1 && m / RE < NR) {
            const int r = m / RE;
            if (r < TN)
              nf.b[r] = *reinterpret_cast<const u32x4 *>(lane_b + 16 * r * Row::ROW_BYTES + p);
            else
              nf.a[r - TN] = *reinterpret_cast<const u32x4 *>(lane_a + 16 * (r - TN) * Row::ROW_BYTES + p);
          }
        }
        if constexpr (NLOAD > 0) {
          if (m % LE == LE - 1) ld_fn(m / LE);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  }

  // Fragment reads for sched_step: call r reads piece r of the next step
  // (the TN rhs pieces, then the TM lhs pieces) into `nf`.
  struct FragReads {
    Frags &nf;
    const char *lane_a, *lane_b;
    int p;  // byte offset of the lane's chunk: ((4 kk + chunk) ^ swz) * 16
    __device__ __forceinline__ void operator()(int r) const {
      if (r < TN)
        nf.b[r] = *reinterpret_cast<const u32x4 *>(lane_b + 16 * r * Row::ROW_BYTES + p);
      else
        nf.a[r - TN] = *reinterpret_cast<const u32x4 *>(lane_a + 16 * (r - TN) * Row::ROW_BYTES + p);
    }
  };

  // One k32 step: the TM*TN MFMAs on `cf` in the fixed order, with other
  // work at fixed MFMA indices: NRD calls rd(0 .. NRD-1), one every RE
  // MFMAs from MFMA R0 on; NLD calls ld(0 .. NLD-1), one every LE MFMAs
  // from L0 on; and sync() right before MFMA SYNC (never when SYNC < 0).
  // sched_barrier(0) after every MFMA pins the order.
  template <int R0, int RE, int NRD, int L0, int LE, int NLD, int SYNC, class RdFn, class LdFn, class SyncFn>
  __device__ __forceinline__ void sched_step(const Frags &cf, RdFn &&rd, LdFn &&ld, SyncFn &&sync) {
    constexpr int NM = TM * TN;
    static_assert(NRD == 0 || R0 + (NRD - 1) * RE < NM, "reads fit in the step");
    static_assert(NLD == 0 || L0 + (NLD - 1) * LE < NM, "loads fit in the step");
    static_assert(SYNC < NM, "sync point inside the step");
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int m = i * TN + j;
        if (m == SYNC) sync();
        Mfma<T>::template run<ACC_AGPR>(cf.b[j], cf.a[i], acc[i][j]);
        if constexpr (NRD > 0) {
          if (m >= R0 && (m - R0) % RE == 0 && (m - R0) / RE < NRD) rd((m - R0) / RE);
        }
        if constexpr (NLD > 0) {
          if (m >= L0 && (m - L0) % LE == 0 && (m - L0) / LE < NLD) ld((m - L0) / LE);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  }

  // Writes the fp32 accumulators, unrounded, to a row-major partial-sum
  // matrix (row pitch ldp floats, a multiple of 4) at (row0, col0); rows
  // past M and column groups past N are skipped.  Each lane stores its four
  // consecutive columns as one 16-byte piece.  Call settle() first.
  __device__ __forceinline__ void store_partial(float *base, int ldp, int M, int N, int row0, int col0,
                                                int lane) const {
    const int r = lane_row(lane);
    const int g = lane_chunk(lane);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = row0 + 16 * i + r;
      if (row >= M) continue;
      float *rp = base + (int64_t)row * ldp;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = col0 + 16 * j + 4 * g;
        if (col < N) *reinterpret_cast<f32x4 *>(rp + col) = acc[i][j];
      }
    }
  }

  // Rounds the accumulators to T and stores them straight to out[M][N] at
  // (row0, col0), for kernels whose LDS ring is still in use when a tile
  // ends.  Lanes with chunk g and g^1 hold columns 4g..4g+3 of one row in
  // blocks j and j+1; they trade one quad (one cross-lane exchange) so that
  // each owns eight consecutive columns, of block j for even g and of block
  // j+1 for odd g, and writes them as one 16-byte store.  Rows past M and
  // columns past N are skipped.  Call settle() first.
  __device__ __forceinline__ void store_direct(uint16_t *out, int M, int N, int row0, int col0, int lane) const {
    static_assert(TN % 2 == 0, "column blocks are paired");
    const int r = lane_row(lane);
    const int g = lane_chunk(lane);
    const int odd = g & 1;
    const bool vec_ok = (N & 7) == 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = row0 + 16 * i + r;
#pragma unroll
      for (int j = 0; j < TN; j += 2) {
        const f32x4 &a0 = acc[i][j];
        const f32x4 &a1 = acc[i][j + 1];
        const u32x2 p0 = Mfma<T>::pack4(a0[0], a0[1], a0[2], a0[3]);
        const u32x2 p1 = Mfma<T>::pack4(a1[0], a1[1], a1[2], a1[3]);
        const u32x2 snd = odd ? p0 : p1;
        u32x2 rcv;
        rcv[0] = (uint32_t)__shfl_xor((int)snd[0], 16);
        rcv[1] = (uint32_t)__shfl_xor((int)snd[1], 16);
        const u32x4 v = odd ? u32x4{rcv[0], rcv[1], p1[0], p1[1]} : u32x4{p0[0], p0[1], rcv[0], rcv[1]};
        if (row >= M) continue;
        uint16_t *rp = out + (int64_t)row * N;
        const int col = col0 + 16 * (j + odd) + 8 * (g >> 1);
        if (vec_ok && col + 8 <= N) {
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(rp + col));
        } else {
#pragma unroll
          for (int x = 0; x < 8; ++x)
            if (col + x < N) rp[col + x] = (uint16_t)(v[x / 2] >> (16 * (x % 2)));
        }
      }
    }
  }

  // Rounds the accumulators to T and writes them into an LDS staging tile
  // (row pitch `pitch` bytes) at this wave's (row0, col0), one 8-byte piece
  // per block.  Call settle() first.
  __device__ __forceinline__ void stage(char *st, int pitch, int row0, int col0, int lane) const {
    const int r = lane_row(lane);
    const int g = lane_chunk(lane);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const f32x4 &a = acc[i][j];
        const u32x2 v = Mfma<T>::pack4(a[0], a[1], a[2], a[3]);
        char *dst = st + (row0 + 16 * i + r) * pitch + (col0 + 16 * j + 4 * g) * 2;
        *reinterpret_cast<u32x2 *>(dst) = v;
      }
  }
};

// Copies a staged BM x BN tile (2-byte elements, row pitch `pitch` bytes) to
// out[m0.., n0..] with 16-byte stores where the row piece is in range and
// aligned, element stores at a ragged right edge, nothing past M.
//
// The 16-byte output stores (here and in WaveTile::store_direct) are
// non-temporal: the output is not read again by the kernel, and the tiles
// resident on one XCD at a time write as much output as its L2 holds (32
// tiles of 256 x 256 f16 = 4 MiB), which with ordinary stores can push the
// lhs and rhs panels of the next tiles out of L2.  Measured: f16 8192^3
// single schedule S = 2 +3-6 %, producer/consumer unchanged, 4096^3 up to
// +1 %.  K-split partial sums keep ordinary stores (reduce_splits reads them
// right after).
template <int BM, int BN, int THREADS>
__device__ __forceinline__ void store_staged(const char *st, int pitch, uint16_t *out, int M, int N,
                                             int m0, int n0, int tid) {
  constexpr int CH = BN / 8;  // 16-byte pieces per tile row
  const bool vec_ok = (N % 8) == 0;
  for (int idx = tid; idx < BM * CH; idx += THREADS) {
    const int row = idx / CH;
    const int c = idx % CH;
    const int gm = m0 + row;
    const int gn = n0 + 8 * c;
    if (gm >= M || gn >= N) continue;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(st + row * pitch + c * 16);
    uint16_t *dst = out + (int64_t)gm * N + gn;
    if (vec_ok && gn + 8 <= N) {
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
    } else {
#pragma unroll
      for (int x = 0; x < 8; ++x)
        if (gn + x < N) dst[x] = (uint16_t)(v[x / 2] >> (16 * (x % 2)));
    }
  }
}

// out[m][n] = round_T(sum over s of part[s][m][n]) for the K pieces of a
// split product, summed in increasing s (so the result does not depend on
// the order in which the pieces finished).  part is [splits][M][ldp] fp32.
template <typename T>
__global__ void __launch_bounds__(256) reduce_splits(const float *__restrict__ part, uint16_t *__restrict__ out,
                                                     int M, int N, int ldp, int splits) {
  const int64_t q = ldp / 4;
  const int64_t total = (int64_t)M * q;
  const int64_t plane = (int64_t)M * ldp;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int row = (int)(idx / q);
    const int col = (int)(idx % q) * 4;
    if (col >= N) continue;
    const float *p = part + (int64_t)row * ldp + col;
    f32x4 s = *reinterpret_cast<const f32x4 *>(p);
    for (int k = 1; k < splits; ++k) s = s + *reinterpret_cast<const f32x4 *>(p + k * plane);
    const u32x2 v = Mfma<T>::pack4(s[0], s[1], s[2], s[3]);
    uint16_t *dst = out + (int64_t)row * N + col;
    if ((N & 3) == 0) {
      *reinterpret_cast<u32x2 *>(dst) = v;
    } else {
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if (col + x < N) dst[x] = (uint16_t)(v[x / 2] >> (16 * (x % 2)));
    }
  }
}

}  // namespace pgemm
