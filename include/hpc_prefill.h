/*
 * hpc_prefill.h — C ABI of causal prefill / extend attention over the paged
 * KV cache on AMD Instinct MI355X (gfx950).
 *
 * "vLLM x HPC-Ops: High-Performance Attention and MoE Backends from Tencent
 * Hunyuan", §Attention Across Prefill, Extend and Decode Shapes measures the
 * same attention backend on prefill ("q512") and extend shapes besides
 * decode; the pages give no formula.  What is computed (the plain reading):
 * sequence b holds L_b = seq_lens[b] tokens in the paged cache (layout and
 * dtypes as in hpc_decode.h), of which the last n_b = q_start[b+1] -
 * q_start[b] are this step's new tokens, already written to the cache.  The
 * new token j of sequence b, at position p = L_b - n_b + j, is query row
 * q_start[b] + j and attends causally to cached tokens t <= p:
 *
 *     out[row, hq] = softmax_{t <= p}(sm_scale <q[row, hq], k_scale K_t>) . (v_scale V_t)
 *     lse[row, hq] = ln sum_{t <= p} exp(sm_scale <q[row, hq], k_scale K_t>)
 *
 * with KV head h = hq / G.  A prompt is n_b = L_b; decode is n_b = 1.
 *
 * Work is cut into units (sequence, block of 16 queries, KV head); the host
 * planner orders them by decreasing cost (KV tiles seen by the block's last
 * query) and the kernel runs one workgroup per unit.
 *
 * Conventions as in hpc_decode.h: status codes, host checks before any HIP
 * call, caller-owned buffers, no allocation, no synchronisation.
 */
#ifndef HPC_PREFILL_H
#define HPC_PREFILL_H

#include <stdint.h>

#include "hpc_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

#define HPC_PREFILL_QUERY_BLOCK 16
#define HPC_PREFILL_UNIT_WORDS  4

/*
 * Number of work units, sum_b ceil(n_b / 16) * num_kv_heads, for host
 * q_start [batch + 1] (q_start[0] = 0, non-decreasing); negative status for
 * NULL, batch < 1, num_kv_heads < 1 or a decreasing / non-zero-based q_start.
 */
int64_t hpc_prefill_units(const int32_t* q_start, int32_t batch, int32_t num_kv_heads);

/*
 * The work list, pure host code: every unit (b, query block j, KV head h)
 * with its cost c = (p_last / 64) + 1, p_last the position of the block's
 * last query, written as 4 int32 words (b, j, h, c) per unit, ordered by
 * decreasing c, ties in increasing (b, j, h).  seq_lens [batch] host.
 * Returns the number of units, or HPC_ERR_NULL / HPC_ERR_INVALID (n_b > L_b,
 * L_b > max_pages_per_seq * 64, negative lengths, bad q_start) /
 * HPC_ERR_TOO_SMALL (capacity in units below hpc_prefill_units).
 */
int64_t hpc_prefill_plan(const int32_t* q_start, const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                         int32_t max_pages_per_seq, int32_t* work, int64_t capacity_units);

/*
 * Causal attention of every new token on `stream`, one workgroup per unit
 * of `work_dev` (the device copy of a list from hpc_prefill_plan, n_units
 * entries).
 *
 * params       heads, page geometry, kv dtype and scales as for decode
 *              (tile_math and fused_merge must be 0; sm_scale * k_scale must
 *              be positive)
 * total_q      rows of q / out / lse (= q_start[batch])
 * q            device bf16 [total_q][Hq][128]
 * q_start      device int32 [batch + 1]; must hold the values the plan was made from
 * k_cache, v_cache, block_table: as for hpc_decode_attn; every page a unit
 *              reads must be in [0, num_pages) (an id outside reads as zeros)
 * seq_lens     device int32 [batch]: L_b, the plan's values
 * out, lse     device bf16 [total_q][Hq][128] / fp32 [total_q][Hq]
 * Errors: NULL pointers, bad shapes or params -> HPC_ERR_NULL /
 * HPC_ERR_INVALID / HPC_ERR_UNSUPPORTED before any HIP call; a failed launch
 * -> HPC_ERR_HIP.
 */
int hpc_prefill_attn(const hpc_decode_params* params, int32_t batch, int32_t total_q, const void* q,
                     const int32_t* q_start, const void* k_cache, const void* v_cache, const int32_t* block_table,
                     const int32_t* seq_lens, const int32_t* work_dev, int32_t n_units, void* out, float* lse,
                     void* stream);

/* The host-side checks of hpc_prefill_attn alone (never calls HIP). */
int hpc_prefill_check(const hpc_decode_params* params, int32_t batch, int32_t total_q, const void* q,
                      const int32_t* q_start, const void* k_cache, const void* v_cache, const int32_t* block_table,
                      const int32_t* seq_lens, const int32_t* work_dev, int32_t n_units, const void* out,
                      const float* lse);

#ifdef __cplusplus
}
#endif

#endif /* HPC_PREFILL_H */
