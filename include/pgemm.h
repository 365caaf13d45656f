/*
 * pgemm: software-pipelined tiled GEMM for AMD Instinct MI355X (gfx950).
 *
 * Plain C interface: host or device pointers and sizes only, no HIP or torch
 * types.  Every GEMM call enqueues one kernel (two for a K-split product)
 * on the caller's HIP stream and returns without waiting for it.  No GEMM
 * call allocates, frees or synchronises: all device memory (operands,
 * output, the optional K-split workspace) belongs to the caller.
 *
 * Operation (Croqtile tutorial ch.6, "Synchronization: pipelines, events and
 * double buffering": the int32 listing with swap and the f16 1P1C listing
 * with events):
 *     out[m, n] = sum over k of lhs[m, k] * rhs(k, n)
 * starting from zero (the output is not accumulated into).
 *
 * Common rules for every GEMM entry point
 *   - lhs, rhs, out: DEVICE pointers on the current HIP device, row-major and
 *     contiguous (leading dimensions are K, N or K, and N).  They must be
 *     16-byte aligned.  The caller owns all three buffers; the library keeps
 *     no reference after the call returns.  `out` is fully overwritten and
 *     must not overlap lhs or rhs.
 *   - M, N, K >= 0 and each below 2^31.  M == 0 or N == 0: nothing is
 *     launched.  K == 0: out is filled with zeros.
 *   - stages: number of LDS ring slots (buffer versions) the K loop rotates
 *     through; 0 picks the library default for the entry point.
 *   - stream: a hipStream_t passed as void*; NULL is the null stream.
 *   - Errors in the arguments are reported before any HIP call is made, and
 *     nothing is enqueued.  PGEMM_ERR_LAUNCH reports a failed launch.
 *   - Calls may be made concurrently on different streams.  The only shared
 *     state a call touches is the K-split workspace registered for its
 *     (device, stream); calls on one stream from several host threads are
 *     serialised around it by the library.
 */
#ifndef PGEMM_H
#define PGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PGEMM_ABI_VERSION 3

typedef enum {
  PGEMM_OK = 0,
  PGEMM_ERR_NULL = 1,    /* a required pointer is NULL                       */
  PGEMM_ERR_SHAPE = 2,   /* negative or too large M, N, K; bad tiling request;
                            an NT grid of 2^32 or more work-items            */
  PGEMM_ERR_STAGES = 3,  /* stages outside the set the entry point supports  */
  PGEMM_ERR_ALIGN = 4,   /* a pointer is not 16-byte aligned                 */
  PGEMM_ERR_LDS = 5,     /* the tile ring for these stages exceeds LDS       */
  PGEMM_ERR_LAUNCH = 6,  /* the HIP launch (or a HIP query) failed           */
  PGEMM_ERR_TIMEOUT = 7, /* a credit wait exceeded its poll limit            */
  PGEMM_ERR_DEVICE = 8,  /* the current device is not gfx950                 */
  PGEMM_ERR_WORKSPACE = 9 /* pgemm_f16_nt_ws_static: the plan's K-split
                            partial sums exceed the static scratch          */
} pgemm_status;

/* Variant codes used by the query functions. */
typedef enum {
  PGEMM_OP_S32_NN = 0,   /* pgemm_s32_nn                                     */
  PGEMM_OP_NT_SWAP = 1,  /* pgemm_f16_nt / pgemm_bf16_nt                     */
  PGEMM_OP_NT_WS = 2     /* pgemm_f16_nt_ws / pgemm_bf16_nt_ws               */
} pgemm_op;

/*
 * int32 NN GEMM, single-schedule double buffering with swapped buffer
 * handles (Croqtile ch.6, "double buffering with swap": prologue loads tile
 * 0, the steady state loads tile t while computing tile t-1, the epilogue
 * drains the last tile).
 *   lhs: int32 [M, K], rhs: int32 [K, N], out: int32 [M, N].
 *   Sums wrap modulo 2^32 (two's complement).  Results are exact.
 *   Each workgroup is 16 x 16 threads owning a 16 x 16 output tile; K is
 *   cut into tiles of 16.  stages: 1 (one buffer, serial) or 2 (default).
 *   The grid has one workgroup per output tile up to 2^20 workgroups; a
 *   larger output is walked by that many, each taking every 2^20-th tile.
 */
pgemm_status pgemm_s32_nn(const int32_t *lhs, const int32_t *rhs, int32_t *out,
                          int64_t M, int64_t N, int64_t K, int stages, void *stream);

/*
 * f16 NT GEMM, single-schedule variant: every wavefront both fills ring
 * slots and runs MFMA, one workgroup barrier per K tile (Croqtile ch.6,
 * swap double buffering applied to the f16 kernel; with more than two slots
 * the handles rotate instead of swapping).
 *   lhs: IEEE binary16 bits [M, K], rhs: binary16 bits [N, K] (row n of rhs
 *   is column n of the right operand), out: binary16 bits [M, N].
 *   Any K below 2^31.  Rows are copied into the LDS ring with 16-byte
 *   direct-to-LDS loads when K is a multiple of 8 and a tile's rows span
 *   less than 2^31 bytes (tile * K < 2^30); otherwise (Croqtile ch.5,
 *   predicated execution with `if`) with a register-staged loader whose
 *   64-bit addressed loads are guarded element by element (elements past K
 *   or past the matrix edge are zero).  Both fill the same ring layout, so
 *   the two give identical bits.
 *   Products are exact and accumulate in fp32 in increasing k; the output is
 *   rounded to nearest-even.  stages: 1..4 (default 2).
 *
 * Tiling (every NT call): the host plans 256 x 256 output tiles when they
 * alone nearly fill the 256 CUs, else 128 x 128 tiles; a product that then
 * still leaves half the CUs idle and has K >= 1024 is split along K into
 * up to 16 pieces (multiples of 64), each workgroup computing one tile over
 * one piece into an fp32 workspace, and a second kernel adds the pieces in
 * increasing order and rounds.  The split is taken only when the caller has
 * registered a workspace of at least pgemm_query's workspace_bytes for the
 * call's stream (pgemm_set_workspace); otherwise the call runs the same
 * tiling unsplit.  For a given plan the result is deterministic; different
 * plans (tile size, K split) may differ in the last bits.
 */
pgemm_status pgemm_f16_nt(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out,
                          int64_t M, int64_t N, int64_t K, int stages, void *stream);

/*
 * f16 NT GEMM, producer/consumer variant (Croqtile ch.6, "1P1C kernel with
 * events"; ch.5, structured concurrent regions): producer wavefronts fill
 * ring slot t mod stages after waiting for its `empty` credit and then
 * signal `full`; consumer wavefronts seed one `empty` credit per slot before
 * the K loop, wait for `full`, run MFMA and return `empty`.  The credits are
 * monotonic counters in LDS.  Same layouts, rules, tiling and numerics as
 * pgemm_f16_nt; for the same plan both give bit-identical results.
 * stages: 1..4 (default 4).
 */
pgemm_status pgemm_f16_nt_ws(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out,
                             int64_t M, int64_t N, int64_t K, int stages, void *stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, plan, kernels and results as pgemm_f16_nt_ws, except that a
 * K-split plan keeps its fp32 partial sums in a static scratch array that
 * the library holds on each device it runs on (PGEMM_STATIC_SCRATCH_BYTES,
 * until the process ends) instead of the stream's registered workspace; it
 * never allocates, frees or waits.  Every split the planner chooses fits;
 * a forced one (pgemm_set_tiling) needing more returns PGEMM_ERR_WORKSPACE
 * before anything is enqueued.  All calls on one device share that scratch:
 * calls that may run at the same time on one device (other streams, other
 * host threads) race on it and must be serialised by the caller.  Nothing
 * in it needs clearing: each call writes every partial sum it reads.
 */
#define PGEMM_STATIC_SCRATCH_BYTES (16ll << 20)
pgemm_status pgemm_f16_nt_ws_static(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out,
                                    int64_t M, int64_t N, int64_t K, int stages, void *stream);

/* bfloat16 counterparts: bf16 operands, fp32 accumulation, bf16 output
 * rounded to nearest-even.  Same rules as the f16 calls. */
pgemm_status pgemm_bf16_nt(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out,
                           int64_t M, int64_t N, int64_t K, int stages, void *stream);
pgemm_status pgemm_bf16_nt_ws(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out,
                              int64_t M, int64_t N, int64_t K, int stages, void *stream);

/*
 * Launch geometry the library would use for (op, stages, M, N, K), without
 * launching.  Host-only: makes no HIP call.  Returns the same argument
 * status the GEMM call would (PGEMM_ERR_STAGES, PGEMM_ERR_SHAPE,
 * PGEMM_ERR_LDS); on PGEMM_OK fills *info.  A plan with k_split > 1 is the
 * one a call runs when its stream has a registered workspace of at least
 * workspace_bytes; without one the call runs it with k_split 1.
 */
typedef struct {
  int32_t block_m, block_n, block_k; /* output tile and K tile            */
  int32_t stages;                    /* ring slots actually used           */
  int32_t producer_waves;            /* 0 for single-schedule kernels      */
  int32_t consumer_waves;            /* waves running the math             */
  int32_t threads;                   /* threads per workgroup              */
  int32_t lds_bytes;                 /* LDS per workgroup                  */
  int64_t grid;                      /* workgroups launched (all pieces)   */
  int64_t k_tiles;                   /* K tiles per workgroup (per piece)  */
  int32_t k_split;                   /* K pieces; 1 = no split             */
  int32_t persistent;                /* 1: persistent schedule (see below) */
  int64_t workspace_bytes;           /* fp32 workspace of a split, else 0  */
  int32_t staged;                    /* 1: register-staged guarded loads   */
} pgemm_kernel_info;

pgemm_status pgemm_query(pgemm_op op, int stages, int64_t M, int64_t N, int64_t K,
                         pgemm_kernel_info *info);

/*
 * K-split workspace (the caller owns it; Croqtile ch.5, "data-dependent and
 * persistent grids": a launch on `stream s` only enqueues, so nothing the
 * call needs may be allocated or awaited inside it).  Registers `bytes` of
 * device memory at `workspace` (16-byte aligned) for later NT calls on
 * `stream` (a hipStream_t as void*, NULL = the null stream) on the current
 * device, replacing any earlier registration for that pair; workspace NULL
 * with bytes 0 removes it.  The library keeps only the pointer: the caller
 * must not free the buffer, or destroy the stream, while it is registered
 * or while calls that used it may still run, and must not register one
 * buffer for two streams.  Calls whose plan needs more than the registered
 * bytes run unsplit.  PGEMM_ERR_SHAPE for bytes < 0, PGEMM_ERR_NULL for a
 * NULL workspace with bytes > 0, PGEMM_ERR_ALIGN for a misaligned one.
 */
pgemm_status pgemm_set_workspace(void *stream, void *workspace, int64_t bytes);

/*
 * Debug status of the credit protocol.  Waits for `stream`, then reads and
 * clears the device-side error word that the producer/consumer kernels set
 * when a credit wait runs past its poll limit.  Returns PGEMM_ERR_TIMEOUT if
 * any such wait gave up since the last call, else PGEMM_OK (or
 * PGEMM_ERR_LAUNCH if HIP fails).  A kernel that gave up has still exited,
 * but its output is undefined.  Not a GEMM call: it synchronises the host.
 */
pgemm_status pgemm_debug_status(void *stream);

/* Tuning and test hook: forces the tiling of later NT calls in this
 * process.  tile: 0 = planned automatically, 128 or 256 = that output tile;
 * k_split: 0 = planned automatically, 1 = no split, 2..16 = that many K
 * pieces (small tiles only; fewer if K has fewer 64-wide pieces).
 * PGEMM_ERR_SHAPE for any other combination (nothing changes).  Not meant
 * to be changed while other threads launch. */
pgemm_status pgemm_set_tiling(int tile, int k_split);

/* Tuning and test hook: the schedule of later producer/consumer calls
 * without a K split.  mode 0: planned (the per-tile kernel: the persistent
 * one measured no faster on these workloads), 1: never, 2: always.  The persistent kernel
 * launches at most 256 x (workgroups that fit a CU's LDS, at most 2)
 * workgroups; each strides over the output tiles (tile_iter * grid +
 * block, guarded by the tile count; Croqtile ch.5, "persistent scheduling
 * and the if guard"), its producers streaming the next tile's K tiles
 * through the ring while the consumers finish the current one.  The
 * results are bit-identical to the per-tile kernel.  PGEMM_ERR_SHAPE for
 * any other mode.  Not meant to be changed while other threads launch. */
pgemm_status pgemm_set_persistent(int mode);

/* Test hook for the credit protocol.  Sets, for later *_ws launches in this
 * process, the poll limit of every credit wait (0 restores the default) and
 * whether consumers skip seeding the `empty` credits (which the protocol
 * needs: without the seeds the first producer wait can never succeed). */
void pgemm_set_ws_debug(int64_t max_polls, int skip_seed);

/* Test hook for the credit protocol (Croqtile ch.6, "credit flow of a single
 * stage": a consumer may only read a slot its producer has filled, and a
 * producer may only refill a slot its consumers have released, whatever
 * the timing).  A non-zero seed (its low 31 bits) makes every wave of later
 * *_ws launches in this process sleep a pseudo-random 0 to 1792 clocks
 * before each of its credit waits and triggers.  The count depends on the
 * seed, the workgroup, the wave, the K tile and the site, so producers and
 * consumers meet in orders their natural timing does not give.  The
 * results must not change.  0 turns it off (the default), leaving one
 * scalar compare per credit operation. */
void pgemm_set_ws_jitter(uint32_t seed);

/*
 * Pipeline planner (host only, no HIP call), the rules the library applies
 * to size each kernel's LDS ring (TileLang ch.22, "pipeline-sync-
 * multibuffer": §2.2 stage/order validity, §2.4 version count, §3.3 arena
 * packing).
 *
 * pgemm_plan_versions: statements 0 .. n_stmts-1 of a pipelined loop body,
 * annotated with stage[i] >= 0 and order[i] (all orders distinct), and their
 * buffer accesses.  The annotation is valid when every buffer a statement
 * reads that another writes has the writer in an earlier stage, or in the
 * same stage and earlier in order; else PGEMM_ERR_STAGES.  On success
 * versions[b] = use - def + 1 for each buffer b (def: earliest stage that
 * writes it, use: latest stage that reads it), 1 for a buffer the body never
 * writes, and one less whenever the count is at least 2 but no writer
 * precedes a reader both in order and in stage.  PGEMM_ERR_SHAPE for
 * negative counts or indices out of range, PGEMM_ERR_NULL for a missing
 * array.  The caller owns all arrays.
 */
typedef struct {
  int32_t stmt;   /* statement index */
  int32_t buffer; /* buffer index */
  int32_t write;  /* 1: the statement writes the buffer; 0: it reads it */
} pgemm_access;

pgemm_status pgemm_plan_versions(int32_t n_stmts, const int32_t *stage, const int32_t *order,
                                 int32_t n_access, const pgemm_access *access,
                                 int32_t n_buffers, int32_t *versions);

/*
 * pgemm_plan_arena: packs n buffers, each `versions` copies of `bytes` kept
 * as one block and live over program points [start, end), into one LDS
 * arena.  Blocks are placed in order of (start, larger first, index); the
 * blocks whose interval ended by then return to a sorted, coalesced free
 * list; a block takes the hole that wastes least after alignment, else new
 * space at the arena's top (a free hole reaching the top is grown).
 * Writes offsets[i], the arena size and the sum of all blocks (no reuse).
 * PGEMM_ERR_SHAPE for bytes < 0, versions < 1, align not a power of two or
 * start >= end; PGEMM_ERR_NULL for a missing array.
 */
typedef struct {
  int64_t bytes;    /* bytes of one version                     */
  int32_t versions; /* copies kept                              */
  int32_t align;    /* alignment in bytes, a power of two       */
  int32_t start;    /* first program point the buffer is live   */
  int32_t end;      /* first program point it is dead again     */
} pgemm_lds_block;

pgemm_status pgemm_plan_arena(int32_t n, const pgemm_lds_block *blocks, int64_t *offsets,
                              int64_t *arena_bytes, int64_t *no_reuse_bytes);

const char *pgemm_strerror(pgemm_status status);
int pgemm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PGEMM_H */
