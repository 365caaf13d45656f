// Kernel instances the library dispatches to, by variant and stage count.
#pragma once

#include "kernels.hpp"

namespace pgemm {

// Single schedule: 256 x 256 output tile, four waves (one per SIMD, up to
// 512 registers each) of 128 x 128.  K tile 64 (64 KiB slots) for one or
// two slots, 32 (32 KiB slots) for three or four.
template <int S>
using SwapGeom = NtGeom<256, 256, (S <= 2 ? 64 : 32), S, 2, 2, 0>;

// Producer/consumer: 256 x 256 output tile, eight consumer waves of
// 128 x 64 (two per SIMD) and four producer waves (one per SIMD), so every
// wave is capped at 168 registers.  K tile 64 (64 KiB slots) for one or two
// slots, 32 (32 KiB slots) for three or four, so that the ring and the
// output staging tile fit in 160 KiB of LDS.
template <int S>
using WsGeom = NtGeom<256, 256, (S <= 2 ? 64 : 32), S, 2, 4, 4>;

constexpr int kSwapMaxStages = 4;
constexpr int kSwapDefaultStages = 2;
constexpr int kWsMaxStages = 4;
constexpr int kWsDefaultStages = 4;

}  // namespace pgemm
