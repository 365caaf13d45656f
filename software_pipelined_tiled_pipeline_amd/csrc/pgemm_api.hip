// C-ABI of the pgemm library: argument checks, planning, launch.
//
// Every call validates its arguments before touching HIP, plans the launch
// (tile size, ring slots, K split) on the host, and enqueues its kernels on
// the caller's stream without waiting.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "pgemm.h"
#include "instances.hpp"
#include "launch.hpp"
#include "planner.hpp"

// Device-side error word: a credit wait that runs past its poll limit sets
// bit 0.  One copy per device; the host reaches it through its address.
__device__ uint32_t pgemm_error_word;

// Static K-split scratch of pgemm_f16_nt_ws_static: fp32 partial sums for
// callers that cannot allocate.  Every split the planner chooses fits (a
// split has at most 256 small tiles over all its pieces: split x tiles x
// 128 x 128 floats = 16 MiB).  One copy per device, held until the process
// ends.  Host code never uses this name as an address (on the host it is a
// stand-in, not device memory): it uses g_scratch_ptr[dev], taken with
// hipGetSymbolAddress when the library first meets the device.
constexpr int64_t kStaticScratchBytes = PGEMM_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

namespace {

using namespace pgemm;

constexpr int kLdsLimit = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int64_t kMaxDim = (int64_t)1 << 31;
// The direct-to-LDS loads address a tile's panel (its rows over the K range)
// through one buffer resource with 32-bit byte offsets that must stay below
// 2^31: a panel of `tile` rows of K elements qualifies while tile * K < 2^30.
constexpr int64_t kDirectPanelElems = (int64_t)1 << 30;
constexpr uint32_t kDefaultPolls = 1u << 24;

std::atomic<uint32_t> g_max_polls{kDefaultPolls};
std::atomic<int> g_skip_seed{0};
std::atomic<uint32_t> g_jitter{0};

// ------------------------------------------------------------- planning
//
// The plan of an NT call: tile size, ring slots and K split.  Large tiles
// (256 x 256 single schedule, 256 x 128 producer/consumer) when they alone
// nearly fill the chip, small (128 x 128) ones otherwise; a product that even then leaves most CUs idle and has a
// long K is split along K into pieces whose fp32 partial tiles a second
// kernel adds up.  pgemm_set_tiling can force either choice.

constexpr int kLargeTile = 256, kSmallTile = 128;
constexpr int64_t kFillTiles = 192;   // 3/4 of the 256 CUs
constexpr int64_t kSplitBelow = 128;  // small tiles that leave half the CUs idle
constexpr int kMaxSplit = 16;
constexpr int64_t kMinPieceK = 512;   // K elements per piece, at least
constexpr int kPieceAlign = 64;       // the small tile's K tile

std::atomic<int> g_force_tile{0};
std::atomic<int> g_force_split{0};
std::atomic<int> g_persist_mode{0};  // 0 planned, 1 never, 2 always (producer/consumer calls)

// Persistent producer/consumer schedule: a grid of at most kCUs x (workgroups
// that fit a CU's LDS, at most 2) workgroups striding over the tiles.  The
// planner does not choose it: with tiles of equal size it removes neither
// the last wave's quantisation nor more than the per-tile fill and epilogue,
// and it measured no faster than the per-tile kernel at 4096^3 and 8192^3.
// pgemm_set_persistent(2) selects it.
constexpr int64_t kCUs = 256;  // compute units of an MI355X
// A dispatch's size in work-items per dimension is a 32-bit field.  The int32
// kernel walks its tiles from a grid of at most this many workgroups (2^28
// work-items); an NT plan whose grid reaches 2^32 work-items is refused.
constexpr int64_t kS32MaxGrid = (int64_t)1 << 20;
constexpr int64_t kMaxWorkItems = (int64_t)1 << 32;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
  int tile = 0;         // 256 or 128 (NT calls), 16 (int32 call)
  int stages = 0;
  int split = 1;        // K pieces
  bool persistent = false;
  bool staged = false;  // register-staged, element-guarded loads
  int64_t k_chunk = 0;  // K elements per piece (K itself without a split)
  int64_t ldp = 0;      // row pitch of the partial-sum planes, in floats
  pgemm_kernel_info info{};
};

// LDS of an NT instance as the pipeline planner sees it: the K loop is two
// statements, the fill (stage 0, order 0) writing the ring and the MMA
// (stage S-1, order 1) reading it, which gives the ring's version count;
// the ring (live over the loop) and the epilogue staging tile (live after
// it) are packed into one arena; the credit counters of the
// producer/consumer kernel follow the arena.
template <class G>
int64_t planned_lds() {
  using namespace planner;
  const std::vector<int> stage{0, G::S - 1}, order{0, 1};
  const std::vector<Access> acc{{0, 0, true}, {1, 0, false}};
  if (!validate(stage, order, acc)) return -1;
  const int v = versions(0, stage, order, acc);
  const std::vector<Block> blocks{{(int64_t)v * G::Loader::SLOT_BYTES, 16, 0, 1}, {G::STAGE_BYTES, 16, 1, 2}};
  std::vector<int64_t> off;
  return pack(blocks, &off) + (G::P > 0 ? 2 * G::S * 4 : 0);
}

template <class G>
void fill_nt(Plan *p, int64_t M, int64_t N) {
  pgemm_kernel_info *i = &p->info;
  i->block_m = G::BM;
  i->block_n = G::BN;
  i->block_k = G::BK;
  i->stages = G::S;
  i->producer_waves = G::P;
  i->consumer_waves = G::CW;
  i->threads = G::THREADS;
  // the kernel's static layout must be the planned one
  const int64_t lds = planned_lds<G>();
  i->lds_bytes = lds == G::LDS_BYTES ? G::LDS_BYTES : -1;
  i->grid = cdiv(M, G::BM) * cdiv(N, G::BN) * p->split;
  i->k_tiles = cdiv(p->k_chunk, G::BK);
  i->k_split = p->split;
  if (p->persistent) {
    const int64_t per_cu = std::min<int64_t>(2, kLdsLimit / G::LDS_BYTES);
    i->grid = std::min<int64_t>(i->grid, kCUs * per_cu);
    i->persistent = 1;
  }
  i->staged = p->staged ? 1 : 0;
  i->workspace_bytes = p->split > 1 ? p->split * M * p->ldp * (int64_t)sizeof(float) : 0;
}

template <template <int> class Geo>
bool fill_nt_s(Plan *p, int s, int64_t M, int64_t N) {
  switch (s) {
    case 1: fill_nt<Geo<1>>(p, M, N); return true;
    case 2: fill_nt<Geo<2>>(p, M, N); return true;
    case 3: fill_nt<Geo<3>>(p, M, N); return true;
    case 4: fill_nt<Geo<4>>(p, M, N); return true;
  }
  return false;
}

int64_t split_workspace_bytes(int split, int64_t M, int64_t N) {
  return split > 1 ? split * M * (cdiv(N, 4) * 4) * (int64_t)sizeof(float) : 0;
}

// `avail`: bytes of workspace the call can use for a K split's partial sums;
// a split that would need more is not planned.
void choose_tiling(Plan *p, int64_t M, int64_t N, int64_t K, int64_t avail, bool ws) {
  const int force_tile = g_force_tile.load(std::memory_order_relaxed);
  const int force_split = g_force_split.load(std::memory_order_relaxed);
  const int64_t large = cdiv(M, kLargeTile) * cdiv(N, ws ? WsGeom<1>::BN : SwapGeom<1>::BN);
  p->tile = force_tile ? force_tile : (large >= kFillTiles ? kLargeTile : kSmallTile);
  int split = 1;
  if (p->tile == kSmallTile && K > 0) {
    const int64_t small = cdiv(M, kSmallTile) * cdiv(N, kSmallTile);
    if (force_split) {
      split = force_split;
    } else if (small < kSplitBelow && K >= 2 * kMinPieceK) {
      int64_t want = 2 * kSplitBelow / (small > 0 ? small : 1);
      if (want > kMaxSplit) want = kMaxSplit;
      if (want > K / kMinPieceK) want = K / kMinPieceK;
      split = (int)(want < 1 ? 1 : want);
    }
  }
  p->split = 1;
  p->k_chunk = K;
  if (split > 1) {
    p->k_chunk = cdiv(cdiv(K, split), kPieceAlign) * kPieceAlign;
    p->split = (int)cdiv(K, p->k_chunk);  // no empty pieces
    if (p->split <= 1 || split_workspace_bytes(p->split, M, N) > avail) {
      p->split = 1;
      p->k_chunk = K;
    }
  }
  p->ldp = cdiv(N, 4) * 4;
  // rows that do not start on 16 bytes, or a panel past the direct loads'
  // 32-bit offsets, take the register-staged loader
  p->staged = (K % 8) != 0 || (int64_t)p->tile * K >= kDirectPanelElems;
}

pgemm_status plan(pgemm_op op, int stages, int64_t M, int64_t N, int64_t K, int64_t avail, Plan *p) {
  if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return PGEMM_ERR_SHAPE;
  *p = Plan{};
  pgemm_kernel_info *info = &p->info;
  switch (op) {
    case PGEMM_OP_S32_NN: {
      const int s = stages == 0 ? 2 : stages;
      if (s != 1 && s != 2) return PGEMM_ERR_STAGES;
      p->tile = 16;
      p->stages = s;
      p->k_chunk = K;
      info->block_m = 16;
      info->block_n = 16;
      info->block_k = 16;
      info->stages = s;
      info->consumer_waves = 4;
      info->threads = 256;
      info->lds_bytes = s * 2 * 16 * 16 * 4;
      info->grid = std::min<int64_t>(cdiv(M, 16) * cdiv(N, 16), kS32MaxGrid);
      info->k_tiles = cdiv(K, 16);
      info->k_split = 1;
      return PGEMM_OK;
    }
    case PGEMM_OP_NT_SWAP:
    case PGEMM_OP_NT_WS: {
      const bool ws = op == PGEMM_OP_NT_WS;
      const int s = stages == 0 ? (ws ? kWsDefaultStages : kSwapDefaultStages) : stages;
      if (s < 1 || s > (ws ? kWsMaxStages : kSwapMaxStages)) return PGEMM_ERR_STAGES;
      p->stages = s;
      choose_tiling(p, M, N, K, avail, ws);
      // the persistent kernel has the direct loader only
      if (ws && p->split == 1 && !p->staged) p->persistent = g_persist_mode.load(std::memory_order_relaxed) == 2;
      bool ok;
      if (p->tile == kLargeTile)
        ok = ws ? fill_nt_s<WsGeom>(p, s, M, N) : fill_nt_s<SwapGeom>(p, s, M, N);
      else
        ok = ws ? fill_nt_s<WsGeomSmall>(p, s, M, N) : fill_nt_s<SwapGeomSmall>(p, s, M, N);
      if (!ok) return PGEMM_ERR_STAGES;
      break;
    }
    default:
      return PGEMM_ERR_STAGES;
  }
  if (info->lds_bytes < 0 || info->lds_bytes > kLdsLimit) return PGEMM_ERR_LDS;
  if (info->grid * info->threads >= kMaxWorkItems) return PGEMM_ERR_SHAPE;
  return PGEMM_OK;
}

// --------------------------------------------------------------- device

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
uint32_t *g_err_ptr[kMaxDevices];
float *g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device
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
        void *sp = nullptr;
        if (hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch)) != hipSuccess || !sp) return PGEMM_ERR_LAUNCH;
        g_scratch_ptr[dev] = static_cast<float *>(sp);
      }
      g_dev_state[dev].store(st, std::memory_order_release);
    }
  }
  if (st != 1) return PGEMM_ERR_DEVICE;
  *dev_out = dev;
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

// ------------------------------------------------------------ workspace
//
// fp32 partial sums of K-split products live in a buffer the caller owns and
// registers per (device, stream) with pgemm_set_workspace.  A GEMM call
// never allocates, frees or waits: without a registered buffer large enough
// for the split, it runs the same tiling unsplit.  The registry lock is held
// from the lookup until the call's two kernels are enqueued, so that calls
// made on one stream by several host threads cannot interleave their
// kernels on the shared buffer.
struct Workspace {
  int dev;
  void *stream;
  float *ptr;
  int64_t bytes;
};
std::mutex g_work_mutex;
std::vector<Workspace> g_work;

// Caller holds g_work_mutex.
const Workspace *find_workspace(int dev, void *stream) {
  for (const auto &e : g_work)
    if (e.dev == dev && e.stream == stream) return &e;
  return nullptr;
}

// --------------------------------------------------------------- launch

enum class Elem { F16, BF16 };

pgemm_status launch(Elem e, const NtLaunch &a, bool staged) {
  if (e == Elem::F16) return staged ? launch_f16_staged(a) : launch_f16_direct(a);
  return staged ? launch_bf16_staged(a) : launch_bf16_direct(a);
}

// `use_static`: a split plan keeps its partial sums in the device's static
// scratch (PGEMM_ERR_WORKSPACE if they do not fit) instead of the stream's
// registered workspace.
pgemm_status nt_entry(Elem e, pgemm_op op, const uint16_t *lhs, const uint16_t *rhs, uint16_t *out, int64_t M,
                      int64_t N, int64_t K, int stages, void *stream, bool use_static = false) {
  pgemm_status st = check_ptrs(lhs, rhs, out, M, N, K);
  if (st != PGEMM_OK) return st;
  Plan p;
  st = plan(op, stages, M, N, K, INT64_MAX, &p);  // argument checks (the split is settled below)
  if (st != PGEMM_OK) return st;
  if (M == 0 || N == 0) return PGEMM_OK;
  int dev = 0;
  st = current_device(&dev);
  if (st != PGEMM_OK) return st;
  std::unique_lock<std::mutex> lock;
  float *part = nullptr;
  if (p.split > 1 && use_static) {
    if (p.info.workspace_bytes > kStaticScratchBytes) return PGEMM_ERR_WORKSPACE;
    part = g_scratch_ptr[dev];
  } else if (p.split > 1) {
    lock = std::unique_lock<std::mutex>(g_work_mutex);
    const Workspace *w = find_workspace(dev, stream);
    const int64_t avail = w ? w->bytes : 0;
    if (avail < p.info.workspace_bytes) {
      st = plan(op, stages, M, N, K, avail, &p);  // the same tiling, unsplit
      if (st != PGEMM_OK) return st;
      lock.unlock();
    } else {
      part = w->ptr;
    }
  }
  NtLaunch a{};
  a.lhs = lhs;
  a.rhs = rhs;
  a.out = out;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.tile = p.tile;
  a.stages = p.stages;
  a.split = p.split;
  a.k_chunk = (int)p.k_chunk;
  a.ldp = (int)p.ldp;
  a.ws = op == PGEMM_OP_NT_WS;
  a.persistent = p.persistent;
  a.grid = p.info.grid;
  a.part = part;
  a.stream = static_cast<hipStream_t>(stream);
  a.dev = dev;
  a.polls = g_max_polls.load(std::memory_order_relaxed);
  a.debug = (g_skip_seed.load(std::memory_order_relaxed) ? 1u : 0u) |
            (g_jitter.load(std::memory_order_relaxed) << 1);
  a.err = g_err_ptr[dev];
  return launch(e, a, p.staged);
}

}  // namespace

extern "C" {

pgemm_status pgemm_s32_nn(const int32_t *lhs, const int32_t *rhs, int32_t *out, int64_t M, int64_t N, int64_t K,
                          int stages, void *stream) {
  pgemm_status st = check_ptrs(lhs, rhs, out, M, N, K);
  if (st != PGEMM_OK) return st;
  Plan p;
  st = plan(PGEMM_OP_S32_NN, stages, M, N, K, 0, &p);
  if (st != PGEMM_OK) return st;
  if (M == 0 || N == 0) return PGEMM_OK;
  int dev = 0;
  st = current_device(&dev);
  if (st != PGEMM_OK) return st;
  const dim3 grid((unsigned)p.info.grid);
  const int tiles_m = (int)cdiv(M, 16);
  const int64_t tiles = cdiv(M, 16) * cdiv(N, 16);
  hipStream_t h = static_cast<hipStream_t>(stream);
  if (p.stages == 1)
    hipLaunchKernelGGL(s32_nn_kernel<1>, grid, dim3(256), 0, h, lhs, rhs, out, (int)M, (int)N, (int)K, tiles_m,
                       tiles);
  else
    hipLaunchKernelGGL(s32_nn_kernel<2>, grid, dim3(256), 0, h, lhs, rhs, out, (int)M, (int)N, (int)K, tiles_m,
                       tiles);
  return launched();
}

pgemm_status pgemm_f16_nt(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out, int64_t M, int64_t N, int64_t K,
                          int stages, void *stream) {
  return nt_entry(Elem::F16, PGEMM_OP_NT_SWAP, lhs, rhs, out, M, N, K, stages, stream);
}

pgemm_status pgemm_f16_nt_ws(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out, int64_t M, int64_t N,
                             int64_t K, int stages, void *stream) {
  return nt_entry(Elem::F16, PGEMM_OP_NT_WS, lhs, rhs, out, M, N, K, stages, stream);
}

pgemm_status pgemm_f16_nt_ws_static(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out, int64_t M, int64_t N,
                                    int64_t K, int stages, void *stream) {
  return nt_entry(Elem::F16, PGEMM_OP_NT_WS, lhs, rhs, out, M, N, K, stages, stream, true);
}

pgemm_status pgemm_bf16_nt(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out, int64_t M, int64_t N, int64_t K,
                           int stages, void *stream) {
  return nt_entry(Elem::BF16, PGEMM_OP_NT_SWAP, lhs, rhs, out, M, N, K, stages, stream);
}

pgemm_status pgemm_bf16_nt_ws(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out, int64_t M, int64_t N,
                              int64_t K, int stages, void *stream) {
  return nt_entry(Elem::BF16, PGEMM_OP_NT_WS, lhs, rhs, out, M, N, K, stages, stream);
}

pgemm_status pgemm_query(pgemm_op op, int stages, int64_t M, int64_t N, int64_t K, pgemm_kernel_info *info) {
  if (!info) return PGEMM_ERR_NULL;
  Plan p;
  pgemm_status st = plan(op, stages, M, N, K, INT64_MAX, &p);
  if (st == PGEMM_OK) *info = p.info;
  return st;
}

pgemm_status pgemm_set_workspace(void *stream, void *workspace, int64_t bytes) {
  if (bytes < 0) return PGEMM_ERR_SHAPE;
  if (bytes > 0 && !workspace) return PGEMM_ERR_NULL;
  if (workspace && misaligned(workspace)) return PGEMM_ERR_ALIGN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PGEMM_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_work_mutex);
  for (size_t i = 0; i < g_work.size(); ++i)
    if (g_work[i].dev == dev && g_work[i].stream == stream) {
      g_work.erase(g_work.begin() + (std::ptrdiff_t)i);
      break;
    }
  if (workspace && bytes > 0) g_work.push_back(Workspace{dev, stream, static_cast<float *>(workspace), bytes});
  return PGEMM_OK;
}

pgemm_status pgemm_set_tiling(int tile, int k_split) {
  if (tile != 0 && tile != kLargeTile && tile != kSmallTile) return PGEMM_ERR_SHAPE;
  if (k_split < 0 || k_split > kMaxSplit) return PGEMM_ERR_SHAPE;
  if (k_split > 1 && tile != kSmallTile) return PGEMM_ERR_SHAPE;
  g_force_tile.store(tile, std::memory_order_relaxed);
  g_force_split.store(k_split, std::memory_order_relaxed);
  return PGEMM_OK;
}

pgemm_status pgemm_plan_versions(int32_t n_stmts, const int32_t *stage, const int32_t *order, int32_t n_access,
                                 const pgemm_access *access, int32_t n_buffers, int32_t *versions) {
  if (n_stmts < 0 || n_access < 0 || n_buffers < 0) return PGEMM_ERR_SHAPE;
  if ((n_stmts > 0 && (!stage || !order)) || (n_access > 0 && !access) || (n_buffers > 0 && !versions))
    return PGEMM_ERR_NULL;
  std::vector<int> st(stage, stage + n_stmts), ord(order, order + n_stmts);
  std::vector<planner::Access> acc;
  for (int32_t i = 0; i < n_access; ++i) {
    const pgemm_access &a = access[i];
    if (a.stmt < 0 || a.stmt >= n_stmts || a.buffer < 0 || a.buffer >= n_buffers) return PGEMM_ERR_SHAPE;
    acc.push_back(planner::Access{a.stmt, a.buffer, a.write != 0});
  }
  for (int32_t i = 0; i < n_stmts; ++i)
    if (st[(size_t)i] < 0) return PGEMM_ERR_STAGES;
  if (!planner::validate(st, ord, acc)) return PGEMM_ERR_STAGES;
  for (int32_t b = 0; b < n_buffers; ++b) versions[b] = planner::versions(b, st, ord, acc);
  return PGEMM_OK;
}

pgemm_status pgemm_plan_arena(int32_t n, const pgemm_lds_block *blocks, int64_t *offsets, int64_t *arena_bytes,
                              int64_t *no_reuse_bytes) {
  if (n < 0) return PGEMM_ERR_SHAPE;
  if ((n > 0 && (!blocks || !offsets)) || !arena_bytes || !no_reuse_bytes) return PGEMM_ERR_NULL;
  std::vector<planner::Block> bl;
  int64_t sum = 0;
  for (int32_t i = 0; i < n; ++i) {
    const pgemm_lds_block &b = blocks[i];
    if (b.bytes < 0 || b.versions < 1 || b.align < 1 || (b.align & (b.align - 1)) || b.start >= b.end)
      return PGEMM_ERR_SHAPE;
    bl.push_back(planner::Block{b.bytes * b.versions, b.align, b.start, b.end});
    sum += b.bytes * b.versions;
  }
  std::vector<int64_t> off;
  *arena_bytes = planner::pack(bl, &off);
  *no_reuse_bytes = sum;
  for (int32_t i = 0; i < n; ++i) offsets[i] = off[(size_t)i];
  return PGEMM_OK;
}

pgemm_status pgemm_set_persistent(int mode) {
  if (mode < 0 || mode > 2) return PGEMM_ERR_SHAPE;
  g_persist_mode.store(mode, std::memory_order_relaxed);
  return PGEMM_OK;
}

pgemm_status pgemm_debug_status(void *stream) {
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

void pgemm_set_ws_jitter(uint32_t seed) { g_jitter.store(seed & 0x7FFFFFFFu, std::memory_order_relaxed); }

const char *pgemm_strerror(pgemm_status status) {
  switch (status) {
    case PGEMM_OK: return "ok";
    case PGEMM_ERR_NULL: return "a required pointer is NULL";
    case PGEMM_ERR_SHAPE: return "M, N or K out of range, or an unsupported tiling request";
    case PGEMM_ERR_STAGES: return "unsupported number of stages";
    case PGEMM_ERR_ALIGN: return "pointer not 16-byte aligned";
    case PGEMM_ERR_LDS: return "tile ring exceeds the LDS budget";
    case PGEMM_ERR_LAUNCH: return "HIP launch or query failed";
    case PGEMM_ERR_TIMEOUT: return "a credit wait exceeded its poll limit";
    case PGEMM_ERR_DEVICE: return "current device is not gfx950";
    case PGEMM_ERR_WORKSPACE: return "the K-split partial sums exceed the static scratch (PGEMM_STATIC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

int pgemm_abi_version(void) { return PGEMM_ABI_VERSION; }

}  // extern "C"
