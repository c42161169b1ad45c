/* Split-KV decode attention for GQA (C ABI).
 *
 * Follows the Hy3 Preview inference case study, section "1. Attention
 * dynamic scheduling": every request's attention is cut into tiles of one
 * size, a task map built before the call shares the tiles out over a fixed
 * number of workers by the global tile count (greedy fill), one workgroup
 * per worker computes its tasks' partial results, and a combine step
 * merges the splits.  Shapes are Hy3's attention (CANN deployment article,
 * section 一): query heads in groups of 8 per KV head, head_dim 128.
 *
 * Per request b and query head j (KV head h = j / 8):
 *   o[b][j] = softmax(q[b][j] . K_h^T / sqrt(128)) V_h
 * over the request's cached tokens; a request with no tokens gives zeros.
 *
 * Readings (where the pages leave a step open): tiles of `tile` tokens
 * (256 by default); the plan walks the (request, KV head) rows in order and
 * gives each worker consecutive tiles until it holds ceil(total tiles /
 * workers), so a worker's share of a row is one contiguous split. */
#ifndef HY3ATTN_H
#define HY3ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HY3ATTN_OK 0
#define HY3ATTN_ERR_INVALID (-1)   /* bad argument (null pointer, bad shape)   */
#define HY3ATTN_ERR_SPACE (-2)     /* a caller buffer is too small              */
#define HY3ATTN_ERR_HIP (-3)       /* a HIP launch failed                       */

#define HY3ATTN_HEAD_DIM 128       /* the only head_dim supported               */
#define HY3ATTN_GROUP 8            /* query heads per KV head                    */
#define HY3ATTN_TILE 256           /* the default tile (KV tokens)               */

/* Largest task count a plan for B requests, n_kv_heads KV heads and
 * n_workers workers can produce (each row boundary adds at most one task
 * per worker): n_workers + B * n_kv_heads. */
int64_t hy3attn_max_tasks(int B, int n_kv_heads, int n_workers);

/* Bytes of device workspace hy3attn_decode needs for max_tasks tasks: per
 * task the unnormalised partial output (8 x 128 float) and the running
 * maximum and sum (8 + 8 float), both in log2 units of the scores. */
size_t hy3attn_workspace_bytes(int64_t max_tasks);

/* The task map (host memory; the plan reads kv_len and nothing else).
 *   kv_len[B]                  cached tokens per request (>= 0)
 *   tile, n_workers            >= 1
 *   tasks[max_tasks][4]        out: (request, kv head, first tile, end tile)
 *   worker_begin[n_workers+1]  out: worker w runs tasks worker_begin[w] ..
 *                                   worker_begin[w+1]-1
 *   row_begin[B*n_kv_heads+1]  out: row b*n_kv_heads+h owns tasks
 *                                   row_begin[r] .. row_begin[r+1]-1
 *   n_tasks                    out: tasks written
 * Returns HY3ATTN_OK, HY3ATTN_ERR_INVALID or HY3ATTN_ERR_SPACE (max_tasks
 * smaller than the plan). */
int hy3attn_plan(const int32_t *kv_len, int B, int n_kv_heads, int tile, int n_workers,
                 int32_t *tasks, int64_t max_tasks, int32_t *worker_begin, int32_t *row_begin,
                 int64_t *n_tasks);

/* Decode attention with a plan (all pointers device memory, launched on
 * `stream`, a hipStream_t; asynchronous).
 *   q          bf16 [B][Hq][128]                       Hq = 8 * n_kv_heads
 *   k, v       bf16 [n_kv_heads][total][128]           request b's tokens at
 *                                                       rows kv_start[b] ..
 *   kv_start   int32 [B+1], kv_start[0] = 0, non-decreasing, total = kv_start[B]
 *   tasks, worker_begin, row_begin: the plan, copied to device memory, made
 *              with the same tile and n_workers
 *   n_rows     rows of the plan (its row_begin holds n_rows + 1 entries); must
 *              equal B * n_kv_heads, else HY3ATTN_ERR_INVALID
 *   workspace  hy3attn_workspace_bytes(n_tasks) bytes, 256-byte aligned
 *   out        bf16 [B][Hq][128]
 * q, k and v must be 16-byte aligned and out 8-byte aligned (else
 * HY3ATTN_ERR_INVALID).  A task whose tiles lie past its request's length
 * (a plan made for other lengths) contributes nothing; rows then hold the
 * attention over the tokens their tasks do cover.  The kernels bound every
 * plan entry before using it: task ranges are clamped to [0, n_tasks), and
 * a task whose request or KV head lies outside [0, B) x [0, n_kv_heads), or
 * whose tile range is empty or negative, is an empty split.
 * The scale is 1/sqrt(128).  Two kernels: one workgroup per worker, then
 * one per (request, KV head, query head) for the combine.  Returns HY3ATTN_OK,
 * HY3ATTN_ERR_INVALID or HY3ATTN_ERR_HIP. */
int hy3attn_decode(const void *q, const void *k, const void *v, const int32_t *kv_start, int B,
                   int n_kv_heads, int tile, const int32_t *tasks, int64_t n_tasks,
                   const int32_t *worker_begin, int n_workers, const int32_t *row_begin,
                   int64_t n_rows, void *workspace, size_t ws_bytes, void *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HY3ATTN_H */
