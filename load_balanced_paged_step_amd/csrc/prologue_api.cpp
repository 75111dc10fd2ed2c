// C ABI of the fused decode prologue (see hpc_prologue.h): host checks, then
// one launch on the caller's stream.  Every check runs before any HIP call.

#include <cmath>
#include <cstdint>

#include "hpc_prologue.h"
#include "internal.h"

extern "C" int hpc_decode_prologue_check(const hpc_prologue_params* p, int32_t batch, const void* q_in,
                                         const void* k_in, const void* v_in, const void* q_norm_w,
                                         const void* k_norm_w, const int32_t* positions,
                                         const int32_t* block_table, const void* k_cache, const void* v_cache,
                                         const void* q_out, const void* q_fp8) {
    if (!p || !q_in || !k_in || !v_in || !q_norm_w || !k_norm_w || !positions || !block_table || !k_cache ||
        !v_cache || !q_out)
        return HPC_ERR_NULL;
    if (p->head_dim != HPC_DECODE_HEAD_DIM || p->page_size != HPC_DECODE_PAGE) return HPC_ERR_UNSUPPORTED;
    if (p->kv_dtype != HPC_KV_BF16 && p->kv_dtype != HPC_KV_FP8_E4M3) return HPC_ERR_UNSUPPORTED;
    if (batch < 1 || p->num_kv_heads < 1 || p->num_q_heads < p->num_kv_heads ||
        p->num_q_heads % p->num_kv_heads != 0)
        return HPC_ERR_INVALID;
    if (p->max_pages_per_seq < 1 || p->num_pages < 1) return HPC_ERR_INVALID;
    if (!std::isfinite(p->eps) || p->eps < 0.0f) return HPC_ERR_INVALID;
    if (!std::isfinite(p->rope_theta) || !(p->rope_theta > 1.0f)) return HPC_ERR_INVALID;
    if (p->kv_dtype == HPC_KV_FP8_E4M3 &&
        (!std::isfinite(p->k_scale) || !(p->k_scale > 0.0f) || !std::isfinite(p->v_scale) || !(p->v_scale > 0.0f)))
        return HPC_ERR_INVALID;
    if (q_fp8 && (!std::isfinite(p->q_scale) || !(p->q_scale > 0.0f))) return HPC_ERR_INVALID;
    if (static_cast<int64_t>(batch) * (p->num_q_heads + p->num_kv_heads) >= INT32_MAX) return HPC_ERR_INVALID;
    if (static_cast<int64_t>(batch) * p->max_pages_per_seq >= INT32_MAX) return HPC_ERR_INVALID;
    return HPC_OK;
}

extern "C" int hpc_decode_prologue(const hpc_prologue_params* p, int32_t batch, const void* q_in, const void* k_in,
                                   const void* v_in, const void* q_norm_w, const void* k_norm_w,
                                   const int32_t* positions, const int32_t* block_table, void* k_cache,
                                   void* v_cache, void* q_out, void* q_fp8, void* stream) {
    const int status = hpc_decode_prologue_check(p, batch, q_in, k_in, v_in, q_norm_w, k_norm_w, positions,
                                                 block_table, k_cache, v_cache, q_out, q_fp8);
    if (status != HPC_OK) return status;
    hpcd::PrologueArgs a{};
    a.q_in = static_cast<const uint16_t*>(q_in);
    a.k_in = static_cast<const uint16_t*>(k_in);
    a.v_in = static_cast<const uint16_t*>(v_in);
    a.q_norm_w = static_cast<const uint16_t*>(q_norm_w);
    a.k_norm_w = static_cast<const uint16_t*>(k_norm_w);
    a.positions = positions;
    a.block_table = block_table;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.q_out = static_cast<uint16_t*>(q_out);
    a.q_fp8 = static_cast<uint8_t*>(q_fp8);
    a.batch = batch;
    a.num_q_heads = p->num_q_heads;
    a.num_kv_heads = p->num_kv_heads;
    a.max_pages_per_seq = p->max_pages_per_seq;
    a.num_pages = p->num_pages;
    a.kv_fp8 = p->kv_dtype == HPC_KV_FP8_E4M3 ? 1 : 0;
    a.eps = p->eps;
    a.k_scale = p->k_scale;
    a.v_scale = p->v_scale;
    a.q_scale = p->q_scale;
    a.log2_theta_over_64 = std::log2(static_cast<double>(p->rope_theta)) / 64.0;
    return hpcd::launch_prologue(a, stream) == 0 ? HPC_OK : HPC_ERR_HIP;
}
