/*
 * hpc_prologue.h — C ABI of the decode step's fused prologue on AMD Instinct
 * MI355X (gfx950): QK-norm, RoPE and the paged KV-cache append of each
 * sequence's new token, with FP8 quantisation of the new K/V for an fp8
 * cache and, optionally, of the query.
 *
 * "vLLM x HPC-Ops: High-Performance Attention and MoE Backends from Tencent
 * Hunyuan", §Attention Backend: Dynamic Load-Balanced Scheduling (the
 * paragraph on the fused attention prologue), combines QK-Norm, RoPE, the
 * KV-cache write and, in FP8, query quantisation in one kernel; "vLLM und
 * Tencent Hunyuan streamen zwei HPC-Backends ...", §Warum ist dynamisches
 * Scheduling entscheidend für Attention?, names the same fusion.  The pages
 * give no formulas; the forms used (the plainest readings):
 *
 *   for sequence b with new-token position p = positions[b] (the number of
 *   tokens cached before this step), each query head and each KV head x:
 *     y   = x / sqrt(mean_d(x_d^2) + eps) * w        (w = q_norm_w or k_norm_w)
 *     a_i = p * theta^(-i/64),  i = 0 .. 63
 *     r_i      = y_i cos a_i - y_{i+64} sin a_i
 *     r_{i+64} = y_{i+64} cos a_i + y_i sin a_i
 *   q_out = bf16(r) for query heads; for KV head h, K <- r and V <- v_in go
 *   to row p % 64 of page block_table[b][p / 64], head h.  A bf16 cache
 *   stores bf16 (nearest-even; V unchanged); an fp8 cache stores
 *   e4m3(x / scale) (nearest-even, saturated to +-448) with k_scale / v_scale.
 *   With q_fp8 given, it receives e4m3(q / q_scale) as well.
 *
 * A sequence whose position is negative (a padding slot), at least
 * max_pages_per_seq * 64, or whose page id lies outside [0, num_pages)
 * writes nothing to the cache, and its q_out (and q_fp8) rows are zeros.
 * After the call the decode step of hpc_decode.h runs with lengths
 * positions[b] + 1.
 *
 * Conventions as in hpc_decode.h: status codes (0 = ok, HPC_ERR_* < 0),
 * every host-checkable condition checked before any HIP call, caller-owned
 * buffers, no allocation, no synchronisation; `stream` is a hipStream_t.
 */
#ifndef HPC_PROLOGUE_H
#define HPC_PROLOGUE_H

#include <stdint.h>

#include "hpc_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct hpc_prologue_params {
    int32_t num_q_heads;        /* Hq, a multiple of num_kv_heads                     */
    int32_t num_kv_heads;       /* H_kv >= 1                                          */
    int32_t head_dim;           /* must be 128                                        */
    int32_t page_size;          /* must be 64                                         */
    int32_t max_pages_per_seq;  /* row stride of block_table                          */
    int32_t num_pages;          /* pages in k_cache / v_cache                         */
    int32_t kv_dtype;           /* HPC_KV_BF16 or HPC_KV_FP8_E4M3                     */
    float   eps;                /* RMS-norm epsilon, >= 0 and finite                  */
    float   rope_theta;         /* RoPE base, > 1 and finite                          */
    float   k_scale;            /* fp8 cache: K code = e4m3(k / k_scale); > 0         */
    float   v_scale;            /* fp8 cache: V code = e4m3(v / v_scale); > 0         */
    float   q_scale;            /* q_fp8 code = e4m3(q / q_scale); > 0 when q_fp8 set */
} hpc_prologue_params;

/*
 * One prologue step on `stream` (one kernel launch, one wave per
 * (sequence, head)).
 *
 * q_in         device bf16 [batch][Hq][128]: the new token's query projection
 * k_in, v_in   device bf16 [batch][H_kv][128]: its key and value projections
 * q_norm_w     device bf16 [128]; k_norm_w device bf16 [128]
 * positions    device int32 [batch]: the new token's position per sequence
 * block_table  device int32 [batch][max_pages_per_seq]
 * k_cache, v_cache  device bf16 or fp8 [num_pages][H_kv][64][128]; one row
 *              per (sequence, KV head) is written, nothing else is touched
 * q_out        device bf16 [batch][Hq][128] (may not alias the inputs)
 * q_fp8        device fp8 e4m3 [batch][Hq][128], or NULL
 * Errors: NULL pointers -> HPC_ERR_NULL; head_dim != 128, page_size != 64,
 * an unknown kv_dtype -> HPC_ERR_UNSUPPORTED; batch < 1, bad head counts,
 * max_pages_per_seq or num_pages < 1, a negative or non-finite eps, theta
 * <= 1, a non-positive scale that is used -> HPC_ERR_INVALID; a failed
 * launch -> HPC_ERR_HIP.  batch * (Hq + H_kv) must stay below 2^31.
 */
int hpc_decode_prologue(const hpc_prologue_params* params, int32_t batch, const void* q_in, const void* k_in,
                        const void* v_in, const void* q_norm_w, const void* k_norm_w, const int32_t* positions,
                        const int32_t* block_table, void* k_cache, void* v_cache, void* q_out, void* q_fp8,
                        void* stream);

/* The host-side checks of hpc_decode_prologue alone (never calls HIP). */
int hpc_decode_prologue_check(const hpc_prologue_params* params, int32_t batch, const void* q_in,
                              const void* k_in, const void* v_in, const void* q_norm_w, const void* k_norm_w,
                              const int32_t* positions, const int32_t* block_table, const void* k_cache,
                              const void* v_cache, const void* q_out, const void* q_fp8);

#ifdef __cplusplus
}
#endif

#endif /* HPC_PROLOGUE_H */
