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
 * Work is cut into units (sequence, block of 16 queries, KV head).  A unit
 * costs the number of 64-token KV tiles its last query sees.  The host
 * planner can also spread the units over a grid the way the decode scheduler
 * of §Attention Backend: Dynamic Load-Balanced Scheduling spreads tiles: no
 * work entry much longer than ceil(T / W) tiles (T = all units' tiles, W =
 * n_workers), a longer unit cut into contiguous shares whose partial results
 * are merged by log-sum-exp.  The pages apply that balancing to decode; using
 * it for extend batches with one long context is the reading used here.
 * Entries run longest first, one workgroup each.
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
#define HPC_PREFILL_ENTRY_WORDS 8   /* (b, query block j, KV head h, tiles, t0, t1, slot, 0)        */
#define HPC_PREFILL_MERGE_WORDS 8   /* (b, query block j, KV head h, shares S, first slot, 0, 0, 0)  */

/*
 * Number of units, sum_b ceil(n_b / 16) * num_kv_heads, for host q_start
 * [batch + 1] (q_start[0] = 0, non-decreasing); negative status for NULL,
 * batch < 1, num_kv_heads < 1 or a decreasing / non-zero-based q_start.
 */
int64_t hpc_prefill_units(const int32_t* q_start, int32_t batch, int32_t num_kv_heads);

/* int32 words enough for hpc_prefill_plan of this batch shape with n_workers
 * (>= 0): 8 (units + n_workers) + 8 units; negative status as above. */
int64_t hpc_prefill_plan_size(const int32_t* q_start, int32_t batch, int32_t num_kv_heads, int32_t n_workers);

/*
 * The work list, pure host code.  Unit (b, j, h) sees tiles [0, n_u),
 * n_u = (p_last / 64) + 1 with p_last the position of the block's last query.
 * With n_workers = W > 0, T = sum n_u and q = max(ceil(T / W),
 * min_share_tiles), a unit with n_u > 2 q is cut into S = ceil(n_u / q)
 * entries, share k covering tiles [k q, min((k + 1) q, n_u)) and writing
 * partial slot base_u + k (bases numbered in unit order); every other unit
 * is one entry with slot -1 (writes out / lse directly).  n_workers = 0 cuts
 * nothing.  A cut costs a partial write and a merge, which pays only where
 * one unit would outlast the rest of the grid: a unit of up to 2 q tiles,
 * started first, ends within a step that the grid's throughput bounds, and
 * min_share_tiles (>= 1) keeps short units of small batches whole.  On
 * MI355X, two workers per compute unit (two workgroups fit a CU) and a
 * 16-tile minimum share measured best.
 * Layout (int32): entries[n_entries][8] = (b, j, h, t1 - t0, t0, t1, slot, 0),
 * longest first, ties by t0 and then in unit order; then merge[n_merge][8] =
 * (b, j, h, S, base_u, 0, 0, 0) for the cut units, in unit order.
 * counts[3] receives n_entries, n_merge, n_partials.  seq_lens [batch] host.
 * Errors: HPC_ERR_NULL; HPC_ERR_INVALID (n_b > L_b, L_b > max_pages_per_seq
 * * 64, negative lengths or n_workers, min_share_tiles < 1, bad q_start);
 * HPC_ERR_TOO_SMALL (capacity below the words needed; hpc_prefill_plan_size
 * is enough).
 */
int hpc_prefill_plan(const int32_t* q_start, const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                     int32_t max_pages_per_seq, int32_t n_workers, int32_t min_share_tiles, int32_t* work,
                     int64_t capacity_words, int32_t* counts);

/* Workspace bytes for n_partials partial slots: fp32 outputs
 * [n_partials][16][G][128], then (256-byte aligned) fp32 lse
 * [n_partials][16][G]; 0 for none; negative status for bad heads. */
int64_t hpc_prefill_workspace_size(int32_t n_partials, int32_t num_q_heads, int32_t num_kv_heads);

/*
 * Causal attention of every new token on `stream`: one workgroup per entry
 * of `work_dev` (the device copy of a list from hpc_prefill_plan), then, when
 * n_merge > 0, the log-sum-exp merge of the cut units.
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
 * work_dev     device int32 words of the plan; n_entries, n_merge, n_partials
 *              its counts
 * workspace    device, >= hpc_prefill_workspace_size(n_partials, ...) bytes
 *              (may be NULL when that is 0)
 * out, lse     device bf16 [total_q][Hq][128] / fp32 [total_q][Hq]
 * Errors: NULL pointers, bad shapes or params -> HPC_ERR_NULL /
 * HPC_ERR_INVALID / HPC_ERR_UNSUPPORTED; counts no plan can have
 * (partials without merge records or the reverse, fewer than two partials
 * per merge record, more partials than entries) -> HPC_ERR_PLAN_MISMATCH; a
 * small workspace -> HPC_ERR_TOO_SMALL; all before any HIP call.  A failed
 * launch -> HPC_ERR_HIP.  The kernels trust the words of work_dev (an
 * entry or record naming a sequence, head or slot outside the plan's ranges
 * is skipped).
 */
int hpc_prefill_attn(const hpc_decode_params* params, int32_t batch, int32_t total_q, const void* q,
                     const int32_t* q_start, const void* k_cache, const void* v_cache, const int32_t* block_table,
                     const int32_t* seq_lens, const int32_t* work_dev, int32_t n_entries, int32_t n_merge,
                     int32_t n_partials, void* workspace, int64_t workspace_bytes, void* out, float* lse,
                     void* stream);

/* The host-side checks of hpc_prefill_attn alone (never calls HIP). */
int hpc_prefill_check(const hpc_decode_params* params, int32_t batch, int32_t total_q, const void* q,
                      const int32_t* q_start, const void* k_cache, const void* v_cache, const int32_t* block_table,
                      const int32_t* seq_lens, const int32_t* work_dev, int32_t n_entries, int32_t n_merge,
                      int32_t n_partials, const void* workspace, int64_t workspace_bytes, const void* out,
                      const float* lse);

#ifdef __cplusplus
}
#endif

#endif /* HPC_PREFILL_H */
