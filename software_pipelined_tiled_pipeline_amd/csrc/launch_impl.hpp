// Launch templates of the NT kernels, included by the instance units only.
#pragma once

#include <atomic>

#include "instances.hpp"
#include "launch.hpp"

namespace pgemm {
namespace launch_detail {

inline pgemm_status launched() { return hipGetLastError() == hipSuccess ? PGEMM_OK : PGEMM_ERR_LAUNCH; }

// Raises the dynamic-LDS limit of a kernel instance once per device;
// `done_mask` is that instance's own record of the devices already set.
template <typename Kern>
pgemm_status allow_lds(Kern kern, int bytes, int dev, std::atomic<uint64_t> &done_mask) {
  const uint64_t bit = 1ull << dev;
  if (done_mask.load(std::memory_order_acquire) & bit) return PGEMM_OK;
  if (hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                          bytes) != hipSuccess)
    return PGEMM_ERR_LAUNCH;
  done_mask.fetch_or(bit, std::memory_order_acq_rel);
  return PGEMM_OK;
}

inline int cdiv_i(int a, int b) { return (int)(((int64_t)a + b - 1) / b); }

template <typename T, class G, bool SPLIT, bool WS, bool STAGED>
pgemm_status launch_nt(const NtLaunch &a) {
  static std::atomic<uint64_t> lds_set{0};
  const int tm = cdiv_i(a.M, G::BM), tn = cdiv_i(a.N, G::BN);
  const dim3 grid((unsigned)((int64_t)tm * tn * a.split));
  if constexpr (WS) {
    auto kern = nt_ws_kernel<T, G, SPLIT, STAGED>;
    pgemm_status st = allow_lds(kern, G::LDS_BYTES, a.dev, lds_set);
    if (st != PGEMM_OK) return st;
    hipLaunchKernelGGL(kern, grid, dim3(G::THREADS), G::LDS_BYTES, a.stream, a.lhs, a.rhs, a.out, a.M, a.N, a.K, tm,
                       tn, kGroupM, a.k_chunk, a.part, a.ldp, a.polls, a.debug, a.err);
  } else {
    auto kern = nt_swap_kernel<T, G, SPLIT, STAGED>;
    pgemm_status st = allow_lds(kern, G::LDS_BYTES, a.dev, lds_set);
    if (st != PGEMM_OK) return st;
    hipLaunchKernelGGL(kern, grid, dim3(G::THREADS), G::LDS_BYTES, a.stream, a.lhs, a.rhs, a.out, a.M, a.N, a.K, tm,
                       tn, kGroupM, a.k_chunk, a.part, a.ldp);
  }
  pgemm_status st = launched();
  if (st != PGEMM_OK || !SPLIT) return st;
  int64_t blocks = ((int64_t)a.M * (a.ldp / 4) + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(reduce_splits<T>, dim3((unsigned)blocks), dim3(256), 0, a.stream, a.part, a.out, a.M, a.N, a.ldp,
                     a.split);
  return launched();
}

template <typename T, class G>
pgemm_status launch_ws_persistent(const NtLaunch &a) {
  static std::atomic<uint64_t> lds_set{0};
  auto kern = nt_ws_persistent_kernel<T, G>;
  pgemm_status st = allow_lds(kern, G::LDS_BYTES, a.dev, lds_set);
  if (st != PGEMM_OK) return st;
  const int tm = cdiv_i(a.M, G::BM), tn = cdiv_i(a.N, G::BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)a.grid), dim3(G::THREADS), G::LDS_BYTES, a.stream, a.lhs, a.rhs, a.out, a.M,
                     a.N, a.K, tm, tn, kGroupM, a.polls, a.debug, a.err);
  return launched();
}

template <typename T, template <int> class Geo>
pgemm_status launch_ws_persistent_s(const NtLaunch &a) {
  switch (a.stages) {
    case 1: return launch_ws_persistent<T, Geo<1>>(a);
    case 2: return launch_ws_persistent<T, Geo<2>>(a);
    case 3: return launch_ws_persistent<T, Geo<3>>(a);
    case 4: return launch_ws_persistent<T, Geo<4>>(a);
  }
  return PGEMM_ERR_STAGES;
}

template <typename T, template <int> class Geo, bool SPLIT, bool WS, bool STAGED>
pgemm_status launch_nt_s(const NtLaunch &a) {
  switch (a.stages) {
    case 1: return launch_nt<T, Geo<1>, SPLIT, WS, STAGED>(a);
    case 2: return launch_nt<T, Geo<2>, SPLIT, WS, STAGED>(a);
    case 3: return launch_nt<T, Geo<3>, SPLIT, WS, STAGED>(a);
    case 4: return launch_nt<T, Geo<4>, SPLIT, WS, STAGED>(a);
  }
  return PGEMM_ERR_STAGES;
}

// Every NT plan of one element type and loader: the large tile (never
// split), the small tile unsplit or split, and (direct loader only) the
// persistent producer/consumer schedule.
template <typename T, bool STAGED>
pgemm_status launch_any(const NtLaunch &a) {
  if constexpr (!STAGED) {
    if (a.persistent)
      return a.tile == 256 ? launch_ws_persistent_s<T, WsGeom>(a) : launch_ws_persistent_s<T, WsGeomSmall>(a);
  } else {
    if (a.persistent) return PGEMM_ERR_LAUNCH;  // the planner never asks for it
  }
  if (a.tile == 256)
    return a.ws ? launch_nt_s<T, WsGeom, false, true, STAGED>(a) : launch_nt_s<T, SwapGeom, false, false, STAGED>(a);
  if (a.split == 1)
    return a.ws ? launch_nt_s<T, WsGeomSmall, false, true, STAGED>(a)
                : launch_nt_s<T, SwapGeomSmall, false, false, STAGED>(a);
  return a.ws ? launch_nt_s<T, WsGeomSmall, true, true, STAGED>(a)
              : launch_nt_s<T, SwapGeomSmall, true, false, STAGED>(a);
}

}  // namespace launch_detail
}  // namespace pgemm
