// C-ABI of the pgemm library: argument checks, kernel choice, launch.
//
// Every call validates its arguments before touching HIP, picks one kernel
// instance from (element type, variant, stages), and enqueues it on the
// caller's stream without waiting.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "pgemm.h"
#include "instances.hpp"

// Device-side error word: a credit wait that runs past its poll limit sets
// bit 0.  One copy per device; the host reaches it through its address.
__device__ uint32_t pgemm_error_word;

namespace {

using namespace pgemm;

constexpr int kLdsLimit = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int64_t kMaxDim = (int64_t)1 << 31;
// Buffer offsets inside a 256-row panel must stay below 2^31 bytes.
constexpr int64_t kMaxKNt = (int64_t)1 << 22;
constexpr int kGroupM = 8;
constexpr uint32_t kDefaultPolls = 1u << 24;

std::atomic<uint32_t> g_max_polls{kDefaultPolls};
std::atomic<int> g_skip_seed{0};

// ------------------------------------------------------------- geometry

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <class G>
void fill_nt(pgemm_kernel_info *i, int64_t M, int64_t N, int64_t K) {
  i->block_m = G::BM;
  i->block_n = G::BN;
  i->block_k = G::BK;
  i->stages = G::S;
  i->producer_waves = G::P;
  i->consumer_waves = G::CW;
  i->threads = G::THREADS;
  i->lds_bytes = G::LDS_BYTES;
  i->grid = cdiv(M, G::BM) * cdiv(N, G::BN);
  i->k_tiles = cdiv(K, G::BK);
}

pgemm_status plan(pgemm_op op, int stages, int64_t M, int64_t N, int64_t K, pgemm_kernel_info *info,
                  int *stages_out) {
  if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return PGEMM_ERR_SHAPE;
  std::memset(info, 0, sizeof *info);
  switch (op) {
    case PGEMM_OP_S32_NN: {
      int s = stages == 0 ? 2 : stages;
      if (s != 1 && s != 2) return PGEMM_ERR_STAGES;
      info->block_m = 16;
      info->block_n = 16;
      info->block_k = 16;
      info->stages = s;
      info->consumer_waves = 4;
      info->threads = 256;
      info->lds_bytes = s * 2 * 16 * 16 * 4;
      info->grid = cdiv(M, 16) * cdiv(N, 16);
      info->k_tiles = cdiv(K, 16);
      *stages_out = s;
      return PGEMM_OK;
    }
    case PGEMM_OP_NT_SWAP: {
      if (K >= kMaxKNt) return PGEMM_ERR_SHAPE;
      int s = stages == 0 ? kSwapDefaultStages : stages;
      if (s == 1) fill_nt<SwapGeom<1>>(info, M, N, K);
      else if (s == 2) fill_nt<SwapGeom<2>>(info, M, N, K);
      else if (s == 3) fill_nt<SwapGeom<3>>(info, M, N, K);
      else if (s == 4) fill_nt<SwapGeom<4>>(info, M, N, K);
      else return PGEMM_ERR_STAGES;
      *stages_out = s;
      break;
    }
    case PGEMM_OP_NT_WS: {
      if (K >= kMaxKNt) return PGEMM_ERR_SHAPE;
      int s = stages == 0 ? kWsDefaultStages : stages;
      if (s == 1) fill_nt<WsGeom<1>>(info, M, N, K);
      else if (s == 2) fill_nt<WsGeom<2>>(info, M, N, K);
      else if (s == 3) fill_nt<WsGeom<3>>(info, M, N, K);
      else if (s == 4) fill_nt<WsGeom<4>>(info, M, N, K);
      else return PGEMM_ERR_STAGES;
      *stages_out = s;
      break;
    }
    default:
      return PGEMM_ERR_STAGES;
  }
  if (info->lds_bytes > kLdsLimit) return PGEMM_ERR_LDS;
  return PGEMM_OK;
}

// --------------------------------------------------------------- device

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
uint32_t *g_err_ptr[kMaxDevices];
std::mutex g_dev_mutex;

pgemm_status current_device(int *dev_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PGEMM_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return PGEMM_ERR_DEVICE;
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    st = g_dev_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return PGEMM_ERR_LAUNCH;
      st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
      if (st == 1) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(pgemm_error_word)) != hipSuccess) return PGEMM_ERR_LAUNCH;
        g_err_ptr[dev] = static_cast<uint32_t *>(p);
      }
      g_dev_state[dev].store(st, std::memory_order_release);
    }
  }
  if (st != 1) return PGEMM_ERR_DEVICE;
  *dev_out = dev;
  return PGEMM_OK;
}

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

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Pointer rules: a pointer may be NULL only when the matrix it addresses is
// empty; non-NULL pointers must be 16-byte aligned.
pgemm_status check_ptrs(const void *lhs, const void *rhs, const void *out, int64_t M, int64_t N, int64_t K) {
  if ((M * K > 0 && !lhs) || (N * K > 0 && !rhs) || (M * N > 0 && !out)) return PGEMM_ERR_NULL;
  if ((lhs && misaligned(lhs)) || (rhs && misaligned(rhs)) || (out && misaligned(out))) return PGEMM_ERR_ALIGN;
  return PGEMM_OK;
}

pgemm_status launched() { return hipGetLastError() == hipSuccess ? PGEMM_OK : PGEMM_ERR_LAUNCH; }

template <typename T, class G>
pgemm_status launch_swap(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out, int M, int N, int K,
                         hipStream_t stream, int dev) {
  auto kern = nt_swap_kernel<T, G>;
  static std::atomic<uint64_t> lds_set{0};
  pgemm_status st = allow_lds(kern, G::LDS_BYTES, dev, lds_set);
  if (st != PGEMM_OK) return st;
  const int tm = (int)cdiv(M, G::BM), tn = (int)cdiv(N, G::BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)(tm * (int64_t)tn)), dim3(G::THREADS), G::LDS_BYTES, stream, lhs, rhs,
                     out, M, N, K, tm, tn, kGroupM);
  return launched();
}

template <typename T, class G>
pgemm_status launch_ws(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out, int M, int N, int K,
                       hipStream_t stream, int dev) {
  auto kern = nt_ws_kernel<T, G>;
  static std::atomic<uint64_t> lds_set{0};
  pgemm_status st = allow_lds(kern, G::LDS_BYTES, dev, lds_set);
  if (st != PGEMM_OK) return st;
  const int tm = (int)cdiv(M, G::BM), tn = (int)cdiv(N, G::BN);
  uint32_t polls = g_max_polls.load(std::memory_order_relaxed);
  int skip = g_skip_seed.load(std::memory_order_relaxed);
  hipLaunchKernelGGL(kern, dim3((unsigned)(tm * (int64_t)tn)), dim3(G::THREADS), G::LDS_BYTES, stream, lhs, rhs, out,
                     M, N, K, tm, tn, kGroupM, polls, skip, g_err_ptr[dev]);
  return launched();
}

template <typename T>
pgemm_status nt_entry(pgemm_op op, const uint16_t *lhs, const uint16_t *rhs, uint16_t *out, int64_t M, int64_t N,
                      int64_t K, int stages, void *stream) {
  pgemm_status st = check_ptrs(lhs, rhs, out, M, N, K);
  if (st != PGEMM_OK) return st;
  pgemm_kernel_info info;
  int s = 0;
  st = plan(op, stages, M, N, K, &info, &s);
  if (st != PGEMM_OK) return st;
  if (K % 8 != 0) return PGEMM_ERR_ALIGN;  // rows of lhs/rhs must start on 16 bytes
  if (M == 0 || N == 0) return PGEMM_OK;
  int dev = 0;
  st = current_device(&dev);
  if (st != PGEMM_OK) return st;
  hipStream_t h = static_cast<hipStream_t>(stream);
  const int m = (int)M, n = (int)N, k = (int)K;
  if (op == PGEMM_OP_NT_SWAP) {
    switch (s) {
      case 1: return launch_swap<T, SwapGeom<1>>(lhs, rhs, out, m, n, k, h, dev);
      case 2: return launch_swap<T, SwapGeom<2>>(lhs, rhs, out, m, n, k, h, dev);
      case 3: return launch_swap<T, SwapGeom<3>>(lhs, rhs, out, m, n, k, h, dev);
      case 4: return launch_swap<T, SwapGeom<4>>(lhs, rhs, out, m, n, k, h, dev);
    }
  } else {
    switch (s) {
      case 1: return launch_ws<T, WsGeom<1>>(lhs, rhs, out, m, n, k, h, dev);
      case 2: return launch_ws<T, WsGeom<2>>(lhs, rhs, out, m, n, k, h, dev);
      case 3: return launch_ws<T, WsGeom<3>>(lhs, rhs, out, m, n, k, h, dev);
      case 4: return launch_ws<T, WsGeom<4>>(lhs, rhs, out, m, n, k, h, dev);
    }
  }
  return PGEMM_ERR_STAGES;
}

}  // namespace

extern "C" {

pgemm_status pgemm_s32_nn(const int32_t *lhs, const int32_t *rhs, int32_t *out, int64_t M, int64_t N, int64_t K,
                          int stages, void *stream) {
  pgemm_status st = check_ptrs(lhs, rhs, out, M, N, K);
  if (st != PGEMM_OK) return st;
  pgemm_kernel_info info;
  int s = 0;
  st = plan(PGEMM_OP_S32_NN, stages, M, N, K, &info, &s);
  if (st != PGEMM_OK) return st;
  if (M == 0 || N == 0) return PGEMM_OK;
  int dev = 0;
  st = current_device(&dev);
  if (st != PGEMM_OK) return st;
  const dim3 grid((unsigned)cdiv(M, 16), (unsigned)cdiv(N, 16));
  hipStream_t h = static_cast<hipStream_t>(stream);
  if (s == 1)
    hipLaunchKernelGGL(s32_nn_kernel<1>, grid, dim3(256), 0, h, lhs, rhs, out, (int)M, (int)N, (int)K);
  else
    hipLaunchKernelGGL(s32_nn_kernel<2>, grid, dim3(256), 0, h, lhs, rhs, out, (int)M, (int)N, (int)K);
  return launched();
}

pgemm_status pgemm_f16_nt(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out, int64_t M, int64_t N, int64_t K,
                          int stages, void *stream) {
  return nt_entry<_Float16>(PGEMM_OP_NT_SWAP, lhs, rhs, out, M, N, K, stages, stream);
}

pgemm_status pgemm_f16_nt_ws(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out, int64_t M, int64_t N,
                             int64_t K, int stages, void *stream) {
  return nt_entry<_Float16>(PGEMM_OP_NT_WS, lhs, rhs, out, M, N, K, stages, stream);
}

pgemm_status pgemm_bf16_nt(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out, int64_t M, int64_t N, int64_t K,
                           int stages, void *stream) {
  return nt_entry<__bf16>(PGEMM_OP_NT_SWAP, lhs, rhs, out, M, N, K, stages, stream);
}

pgemm_status pgemm_bf16_nt_ws(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out, int64_t M, int64_t N,
                              int64_t K, int stages, void *stream) {
  return nt_entry<__bf16>(PGEMM_OP_NT_WS, lhs, rhs, out, M, N, K, stages, stream);
}

pgemm_status pgemm_query(pgemm_op op, int stages, int64_t M, int64_t N, int64_t K, pgemm_kernel_info *info) {
  if (!info) return PGEMM_ERR_NULL;
  int s = 0;
  return plan(op, stages, M, N, K, info, &s);
}

pgemm_status pgemm_sync_status(void *stream) {
  int dev = 0;
  pgemm_status st = current_device(&dev);
  if (st != PGEMM_OK) return st;
  hipStream_t h = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(h) != hipSuccess) return PGEMM_ERR_LAUNCH;
  uint32_t word = 0;
  if (hipMemcpy(&word, g_err_ptr[dev], sizeof word, hipMemcpyDeviceToHost) != hipSuccess) return PGEMM_ERR_LAUNCH;
  if (word) {
    const uint32_t zero = 0;
    if (hipMemcpy(g_err_ptr[dev], &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess) return PGEMM_ERR_LAUNCH;
    return PGEMM_ERR_TIMEOUT;
  }
  return PGEMM_OK;
}

void pgemm_set_ws_debug(int64_t max_polls, int skip_seed) {
  uint32_t p = max_polls <= 0 ? kDefaultPolls : (max_polls > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)max_polls);
  g_max_polls.store(p, std::memory_order_relaxed);
  g_skip_seed.store(skip_seed ? 1 : 0, std::memory_order_relaxed);
}

const char *pgemm_strerror(pgemm_status status) {
  switch (status) {
    case PGEMM_OK: return "ok";
    case PGEMM_ERR_NULL: return "a required pointer is NULL";
    case PGEMM_ERR_SHAPE: return "M, N or K out of range";
    case PGEMM_ERR_STAGES: return "unsupported number of stages";
    case PGEMM_ERR_ALIGN: return "pointer not 16-byte aligned, or K not a multiple of 8 for an NT call";
    case PGEMM_ERR_LDS: return "tile ring exceeds the LDS budget";
    case PGEMM_ERR_LAUNCH: return "HIP launch or query failed";
    case PGEMM_ERR_TIMEOUT: return "a credit wait exceeded its poll limit";
    case PGEMM_ERR_DEVICE: return "current device is not gfx950";
  }
  return "unknown status";
}

int pgemm_abi_version(void) { return PGEMM_ABI_VERSION; }

}  // extern "C"
