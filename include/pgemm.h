/*
 * pgemm: software-pipelined tiled GEMM for AMD Instinct MI355X (gfx950).
 *
 * Plain C interface: host or device pointers and sizes only, no HIP or torch
 * types.  Every GEMM call enqueues one kernel on the caller's HIP stream and
 * returns without waiting for it.
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
 *   - Calls are stateless and may be made concurrently on different streams.
 */
#ifndef PGEMM_H
#define PGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PGEMM_ABI_VERSION 1

typedef enum {
  PGEMM_OK = 0,
  PGEMM_ERR_NULL = 1,    /* a required pointer is NULL                       */
  PGEMM_ERR_SHAPE = 2,   /* negative or too large M, N, K                    */
  PGEMM_ERR_STAGES = 3,  /* stages outside the set the entry point supports  */
  PGEMM_ERR_ALIGN = 4,   /* a pointer is not 16-byte aligned                 */
  PGEMM_ERR_LDS = 5,     /* the tile ring for these stages exceeds LDS       */
  PGEMM_ERR_LAUNCH = 6,  /* the HIP launch (or a HIP query) failed           */
  PGEMM_ERR_TIMEOUT = 7, /* a credit wait exceeded its poll limit            */
  PGEMM_ERR_DEVICE = 8   /* the current device is not gfx950                 */
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
 */
pgemm_status pgemm_s32_nn(const int32_t *lhs, const int32_t *rhs, int32_t *out,
                          int64_t M, int64_t N, int64_t K, int stages, void *stream);

/*
 * f16 NT GEMM, single-schedule variant: every wavefront both fills the next
 * ring slot and runs MFMA on the current one, one workgroup barrier per K
 * tile (Croqtile ch.6, swap double buffering, applied to the f16 kernel).
 *   lhs: IEEE binary16 bits [M, K], rhs: binary16 bits [N, K] (row n of rhs
 *   is column n of the right operand), out: binary16 bits [M, N].
 *   Products are exact and accumulate in fp32 in increasing k; the output is
 *   rounded to nearest-even.  stages: 1 or 2 (default 2).
 */
pgemm_status pgemm_f16_nt(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out,
                          int64_t M, int64_t N, int64_t K, int stages, void *stream);

/*
 * f16 NT GEMM, producer/consumer variant (Croqtile ch.6, "1P1C kernel with
 * events"; ch.5, structured concurrent regions): producer wavefronts fill
 * ring slot t mod stages after waiting for its `empty` credit and then
 * signal `full`; consumer wavefronts seed one `empty` credit per slot before
 * the K loop, wait for `full`, run MFMA and return `empty`.  The credits are
 * monotonic counters in LDS.  Same layouts and numerics as pgemm_f16_nt; for
 * the same shape both give bit-identical results.  stages: 1..4 (default 4).
 */
pgemm_status pgemm_f16_nt_ws(const uint16_t *lhs, const uint16_t *rhs, uint16_t *out,
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
 * PGEMM_ERR_LDS); on PGEMM_OK fills *info.
 */
typedef struct {
  int32_t block_m, block_n, block_k; /* output tile and K tile            */
  int32_t stages;                    /* ring slots actually used           */
  int32_t producer_waves;            /* 0 for single-schedule kernels      */
  int32_t consumer_waves;            /* waves running the math             */
  int32_t threads;                   /* threads per workgroup              */
  int32_t lds_bytes;                 /* LDS per workgroup                  */
  int64_t grid;                      /* workgroups launched                */
  int64_t k_tiles;                   /* cdiv(K, block_k)                   */
} pgemm_kernel_info;

pgemm_status pgemm_query(pgemm_op op, int stages, int64_t M, int64_t N, int64_t K,
                         pgemm_kernel_info *info);

/*
 * Waits for `stream`, then reads and clears the device-side error word that
 * the producer/consumer kernels set when a credit wait runs past its poll
 * limit.  Returns PGEMM_ERR_TIMEOUT if any such wait gave up since the last
 * call, else PGEMM_OK (or PGEMM_ERR_LAUNCH if HIP fails).  A kernel that gave
 * up has still exited, but its output is undefined.
 */
pgemm_status pgemm_sync_status(void *stream);

/* Test hook for the credit protocol.  Sets, for later *_ws launches in this
 * process, the poll limit of every credit wait (0 restores the default) and
 * whether consumers skip seeding the `empty` credits (which the protocol
 * needs: without the seeds the first producer wait can never succeed). */
void pgemm_set_ws_debug(int64_t max_polls, int skip_seed);

const char *pgemm_strerror(pgemm_status status);
int pgemm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PGEMM_H */
