// Kernel instances the library dispatches to, by variant, tile size and
// stage count.
#pragma once

#include "kernels.hpp"

namespace pgemm {

// Single schedule, large tile: 256 x 256 output tile, four waves (one per
// SIMD, up to 512 registers each) of 128 x 128.  K tile 64 (64 KiB slots)
// for one or two slots, 32 (32 KiB slots) for three or four.
template <int S>
using SwapGeom = NtGeom<256, 256, (S <= 2 ? 64 : 32), S, 2, 2, 0>;

// Producer/consumer, large tile: 256 x 256 output tile, eight consumer waves
// of 128 x 64 (two per SIMD) and two producer waves, so two SIMDs hold three
// waves, every wave is capped at 168 registers and a consumer holds one
// fragment set.  (Four producers, one per SIMD, cap the registers the same
// way and measured 0.2-1.2 % slower at every stage count at 8192^3 and at
// 4096^3: fewer waves compete for the issue slots of the SIMDs.)  K tile 64 (64 KiB slots) for one or two slots, 32 (32 KiB slots) for
// three or four, so that the ring and the output staging tile fit in 160 KiB
// of LDS.  (A 256 x 128 tile with four consumers and four producers, one of
// each per SIMD, gives each wave 256 registers and the consumers two
// fragment sets, but measured 10-20 % slower at 8192^3: a lone consumer per
// SIMD idles it at every credit wait, and the narrower tile reads a third
// more from L2 per flop.)
template <int S>
using WsGeom = NtGeom<256, 256, (S <= 2 ? 64 : 32), S, 2, 4, 2>;

// Small tile, for products with too few 256 x 256 tiles to fill the chip
// (and, with a K split, for skinny ones): 128 x 128 output tile, K tile 64
// (32 KiB slots, so four slots take 128 KiB).  Single schedule: eight waves
// of 64 x 32, two per SIMD, so that one wave's MFMAs run while the other
// waits on its loads or fragment reads (5 % faster on the ragged
// 4095 x 1000 x 1000 product than four waves of 64 x 64).
// Producer/consumer: four consumer waves of 64 x 64 and two producer waves
// (eight consumers of 64 x 32 measured slower; four producers no faster at
// the best stage count of the skinny, ragged or 2048^3 products).
template <int S>
using SwapGeomSmall = NtGeom<128, 128, 64, S, 2, 4, 0, 1>;
template <int S>
using WsGeomSmall = NtGeom<128, 128, 64, S, 2, 2, 2>;

constexpr int kSwapMaxStages = 4;
constexpr int kSwapDefaultStages = 2;
constexpr int kWsMaxStages = 4;
constexpr int kWsDefaultStages = 4;

}  // namespace pgemm
