// Consumer-side math and the output epilogue.
//
// A wave owns a WM x WN block of the output, held as (WM/32) x (WN/32) fp32
// accumulators of v_mfma_f32_32x32x16.  Operand roles: src0 is the rhs
// fragment (32 rows n) and src1 the lhs fragment (32 rows m), so each
// accumulator holds a transposed 32x32 output block:
//   lane l, register r of acc[i][j] ->
//     out[m0 + 32 i + l % 32][n0 + 32 j + 8 (r / 4) + 4 (l / 32) + r % 4],
// i.e. registers 4q..4q+3 are four consecutive columns of one row, which the
// epilogue writes as one 8-byte piece.
//
// Both fragments are read the same way from a ring slot: lane l reads row
// (base + l % 32) at chunk 2 kk + l / 32 (eight consecutive k), for the k16
// step kk of the tile.  Every output element accumulates the k16 steps in
// increasing k, so any tile shape, stage count or variant gives the same
// bits.
#pragma once

#include "device_common.hpp"

namespace pgemm {

template <typename T>
struct Mfma;

template <>
struct Mfma<_Float16> {
  __device__ __forceinline__ static f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
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
  __device__ __forceinline__ static f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // fp32 -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32)
  __device__ __forceinline__ static u32x2 pack4(float a, float b, float c, float d) {
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    b4 h = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
    return __builtin_bit_cast(u32x2, h);
  }
};

template <typename T, int WM, int WN, int BK>
struct WaveTile {
  static constexpr int TM = WM / 32;
  static constexpr int TN = WN / 32;
  using Row = RingRow<BK>;
  f32x16 acc[TM][TN];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  }

  // Fragments of one k16 step: TN rhs and TM lhs 16-byte pieces per lane.
  struct Frags {
    u32x4 b[TN], a[TM];
  };

  // Lane l reads row (base + l % 32) at chunk 2 kk + l / 32 of the K tile;
  // `lane_a` / `lane_b` already point at that row of the wave's first block.
  // `lane_a` / `lane_b` point at the lane's row of the wave's first lhs /
  // rhs block in a slot; s = swz(l % 32).
  __device__ __forceinline__ static void read_frags(Frags &f, const char *lane_a, const char *lane_b, int kk,
                                                    int hi, int s) {
    const int p = ((2 * kk + hi) ^ s) * 16;
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = *reinterpret_cast<const u32x4 *>(lane_b + 32 * j * Row::ROW_BYTES + p);
#pragma unroll
    for (int i = 0; i < TM; ++i) f.a[i] = *reinterpret_cast<const u32x4 *>(lane_a + 32 * i * Row::ROW_BYTES + p);
  }

  __device__ __forceinline__ void mma_step(const Frags &f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = Mfma<T>::run(f.b[j], f.a[i], acc[i][j]);
  }

  // One K tile from a ring slot.  a_rows / b_rows: LDS address of the first
  // of this wave's lhs / rhs rows in the slot; both are multiples of 32 rows
  // from the tile start, so the swizzle term depends on l % 32 only.  With
  // PREFETCH the fragments of step kk+1 are read while step kk's MFMAs run
  // (two fragment sets live); without it one set is live and latency is left
  // to the other waves of the SIMD.
  template <bool PREFETCH>
  __device__ __forceinline__ void mma_ktile(const char *a_rows, const char *b_rows, int lane) {
    const int r = lane & 31;
    const int hi = lane >> 5;
    const int s = Row::swz(r);
    const char *lane_a = a_rows + r * Row::ROW_BYTES;
    const char *lane_b = b_rows + r * Row::ROW_BYTES;
    constexpr int NK = BK / 16;
    if constexpr (PREFETCH) {
      Frags f[2];
      read_frags(f[0], lane_a, lane_b, 0, hi, s);
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        if (kk + 1 < NK) read_frags(f[(kk + 1) & 1], lane_a, lane_b, kk + 1, hi, s);
        mma_step(f[kk & 1]);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        Frags f;
        read_frags(f, lane_a, lane_b, kk, hi, s);
        mma_step(f);
      }
    }
  }

  // One k16 step: the TM*TN MFMAs on `cf`, with, in a fixed interleave
  // (one read every TM*TN/(TM+TN) MFMAs, one load every TM*TN/NLOAD), the
  // fragment reads of the next step into `nf` when READS and NLOAD calls
  // ld_fn(0 .. NLOAD-1).  sched_barrier(0) after every MFMA pins the order:
  // global loads spaced out between MFMAs never pile up in the
  // texture-address queue, where a full queue would stall the wave's
  // in-order issue, MFMAs included.
  template <bool READS, int NLOAD, class LoadFn>
  __device__ __forceinline__ void mixed_step(const Frags &cf, Frags &nf, const char *lane_a, const char *lane_b,
                                             int nkk, int hi, int s, LoadFn &&ld_fn) {
    constexpr int NM = TM * TN;
    constexpr int NR = TM + TN;
    static_assert(NM % NR == 0 || !READS, "reads spread evenly");
    static_assert(NLOAD == 0 || NM % NLOAD == 0, "loads spread evenly");
    constexpr int RE = NM / NR;                         // MFMAs per read
    constexpr int LE = NLOAD > 0 ? NM / (NLOAD > 0 ? NLOAD : 1) : NM + 1;  // MFMAs per load
    const int p = ((2 * nkk + hi) ^ s) * 16;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int m = i * TN + j;
        acc[i][j] = Mfma<T>::run(cf.b[j], cf.a[i], acc[i][j]);
        if constexpr (READS) {
          if (m % RE == RE - 1) {
            const int r = m / RE;
            if (r < TN)
              nf.b[r] = *reinterpret_cast<const u32x4 *>(lane_b + 32 * r * Row::ROW_BYTES + p);
            else
              nf.a[r - TN] = *reinterpret_cast<const u32x4 *>(lane_a + 32 * (r - TN) * Row::ROW_BYTES + p);
          }
        }
        if constexpr (NLOAD > 0) {
          if (m % LE == LE - 1) ld_fn(m / LE);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  }

  // Writes the fp32 accumulators, unrounded, to a row-major partial-sum
  // matrix (row pitch ldp floats, a multiple of 4) at (row0, col0); rows
  // past M and column groups past N are skipped.  Each lane stores 16 bytes
  // (four consecutive columns) per register quad.
  __device__ __forceinline__ void store_partial(float *base, int ldp, int M, int N, int row0, int col0,
                                                int lane) const {
    const int r = lane & 31;
    const int hi = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = row0 + 32 * i + r;
      if (row >= M) continue;
      float *rp = base + (int64_t)row * ldp;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = col0 + 32 * j + 8 * q + 4 * hi;
          const f32x16 &a = acc[i][j];
          if (col < N) *reinterpret_cast<f32x4 *>(rp + col) = f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
        }
    }
  }

  // Rounds the accumulators to T and stores them straight to out[M][N] at
  // (row0, col0), for kernels whose LDS ring is still in use when a tile
  // ends.  Lane l (row l % 32) holds columns 8q + 4 (l / 32) .. +3 of each
  // 32-column block; lanes l and l + 32 trade two of their four quads (one
  // cross-lane exchange) so that each lane then owns two runs of eight
  // consecutive columns and writes them as 16-byte stores.  Rows past M and
  // columns past N are skipped.
  __device__ __forceinline__ void store_direct(uint16_t *out, int M, int N, int row0, int col0, int lane) const {
    const int r = lane & 31;
    const int hi = lane >> 5;
    const bool vec_ok = (N & 7) == 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = row0 + 32 * i + r;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const f32x16 &a = acc[i][j];
        u32x2 p[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) p[q] = Mfma<T>::pack4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
        // lane hi=0 keeps quads 0, 2 and sends 1, 3; lane hi=1 the reverse
        const u32x2 s0 = hi ? p[0] : p[1], s1 = hi ? p[2] : p[3];
        u32x2 r0, r1;
        r0[0] = (uint32_t)__shfl_xor((int)s0[0], 32);
        r0[1] = (uint32_t)__shfl_xor((int)s0[1], 32);
        r1[0] = (uint32_t)__shfl_xor((int)s1[0], 32);
        r1[1] = (uint32_t)__shfl_xor((int)s1[1], 32);
        // hi=0: columns 0-7 (own quad 0, partner's quad 0) and 16-23;
        // hi=1: columns 8-15 (partner's quad 1, own quad 1) and 24-31
        const u32x4 c0 = hi ? u32x4{r0[0], r0[1], p[1][0], p[1][1]} : u32x4{p[0][0], p[0][1], r0[0], r0[1]};
        const u32x4 c1 = hi ? u32x4{r1[0], r1[1], p[3][0], p[3][1]} : u32x4{p[2][0], p[2][1], r1[0], r1[1]};
        if (row >= M) continue;
        uint16_t *rp = out + (int64_t)row * N;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 v = h ? c1 : c0;
          const int col = col0 + 32 * j + 16 * h + 8 * hi;
          if (vec_ok && col + 8 <= N) {
            *reinterpret_cast<u32x4 *>(rp + col) = v;
          } else {
#pragma unroll
            for (int x = 0; x < 8; ++x)
              if (col + x < N) rp[col + x] = (uint16_t)(v[x / 2] >> (16 * (x % 2)));
          }
        }
      }
    }
  }

  // Rounds the accumulators to T and writes them into an LDS staging tile
  // (row pitch `pitch` bytes) at this wave's (row0, col0).
  __device__ __forceinline__ void stage(char *st, int pitch, int row0, int col0, int lane) const {
    const int r = lane & 31;
    const int hi = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16 &a = acc[i][j];
          u32x2 v = Mfma<T>::pack4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
          char *dst = st + (row0 + 32 * i + r) * pitch + (col0 + 32 * j + 8 * q + 4 * hi) * 2;
          *reinterpret_cast<u32x2 *>(dst) = v;
        }
  }
};

// Copies a staged BM x BN tile (2-byte elements, row pitch `pitch` bytes) to
// out[m0.., n0..] with 16-byte stores where the row piece is in range and
// aligned, element stores at a ragged right edge, nothing past M.
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
      *reinterpret_cast<u32x4 *>(dst) = v;
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
