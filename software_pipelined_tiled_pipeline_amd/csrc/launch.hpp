// Host-side launch interface between the C-ABI unit (pgemm_api.hip), which
// validates and plans every call, and the instance units (inst_*.hip), each
// of which compiles the NT kernels of one element type and one loader and
// launches them.  Splitting the instances over several units lets them
// compile in parallel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pgemm.h"

namespace pgemm {

// One planned NT call, resolved on the host.
struct NtLaunch {
  const uint16_t *lhs, *rhs;
  uint16_t *out;
  int M, N, K;
  int tile;          // 256 or 128
  int stages;        // ring slots
  int split;         // K pieces (1: none)
  int k_chunk;       // K elements per piece
  int ldp;           // row pitch of the partial-sum planes, in floats
  bool ws;           // producer/consumer variant
  bool persistent;   // persistent producer/consumer schedule (direct loader only)
  int64_t grid;      // workgroups of a persistent launch
  float *part;       // [split][M][ldp] fp32 partial sums of a split plan
  hipStream_t stream;
  int dev;           // current device (below 64)
  uint32_t polls;    // poll limit of a credit wait
  uint32_t debug;    // test hooks: bit 0, consumers do not seed `empty`;
                     // bits 1-31, a credit-timing jitter seed (0: none)
  uint32_t *err;     // device error word
};

// Output-tile walk order shared by every NT launch: groups of this many row
// panels (see block_work).
constexpr int kGroupM = 4;

// Defined in inst_{f16,bf16}_{direct,staged}.hip.  Each launches the plan's
// GEMM kernel and, for a split plan, the reduction after it.
pgemm_status launch_f16_direct(const NtLaunch &a);
pgemm_status launch_f16_staged(const NtLaunch &a);
pgemm_status launch_bf16_direct(const NtLaunch &a);
pgemm_status launch_bf16_staged(const NtLaunch &a);

}  // namespace pgemm
