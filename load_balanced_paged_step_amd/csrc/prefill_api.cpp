// C ABI of causal prefill / extend attention (see hpc_prefill.h): the host
// work-list planner, host checks, and the launch on the caller's stream.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "hpc_prefill.h"
#include "internal.h"

namespace {

constexpr int kQB = HPC_PREFILL_QUERY_BLOCK;

bool valid_q_start(const int32_t* q_start, int32_t batch) {
    if (q_start[0] != 0) return false;
    for (int32_t b = 0; b < batch; ++b)
        if (q_start[b + 1] < q_start[b]) return false;
    return true;
}

}  // namespace

extern "C" int64_t hpc_prefill_units(const int32_t* q_start, int32_t batch, int32_t num_kv_heads) {
    if (!q_start) return HPC_ERR_NULL;
    if (batch < 1 || num_kv_heads < 1 || !valid_q_start(q_start, batch)) return HPC_ERR_INVALID;
    int64_t units = 0;
    for (int32_t b = 0; b < batch; ++b) units += (int64_t(q_start[b + 1]) - q_start[b] + kQB - 1) / kQB;
    return units * num_kv_heads;
}

extern "C" int64_t hpc_prefill_plan(const int32_t* q_start, const int32_t* seq_lens, int32_t batch,
                                    int32_t num_kv_heads, int32_t max_pages_per_seq, int32_t* work,
                                    int64_t capacity_units) {
    if (!q_start || !seq_lens || !work) return HPC_ERR_NULL;
    if (max_pages_per_seq < 1) return HPC_ERR_INVALID;
    const int64_t units = hpc_prefill_units(q_start, batch, num_kv_heads);
    if (units < 0) return units;
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t n = int64_t(q_start[b + 1]) - q_start[b];
        if (seq_lens[b] < 0 || n > seq_lens[b] || int64_t(seq_lens[b]) > int64_t(max_pages_per_seq) * HPC_DECODE_PAGE)
            return HPC_ERR_INVALID;
    }
    if (capacity_units < units) return HPC_ERR_TOO_SMALL;
    struct Unit {
        int32_t b, j, h, cost;
    };
    std::vector<Unit> list;
    list.reserve(static_cast<std::size_t>(units));
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t n = q_start[b + 1] - q_start[b];
        const int32_t L = seq_lens[b];
        for (int32_t j = 0; j * kQB < n; ++j) {
            const int32_t last = L - n + std::min(kQB * (j + 1), n) - 1;
            const int32_t cost = last / HPC_DECODE_PAGE + 1;
            for (int32_t h = 0; h < num_kv_heads; ++h) list.push_back({b, j, h, cost});
        }
    }
    std::stable_sort(list.begin(), list.end(), [](const Unit& x, const Unit& y) { return x.cost > y.cost; });
    for (std::size_t i = 0; i < list.size(); ++i) {
        work[4 * i + 0] = list[i].b;
        work[4 * i + 1] = list[i].j;
        work[4 * i + 2] = list[i].h;
        work[4 * i + 3] = list[i].cost;
    }
    return units;
}

extern "C" int hpc_prefill_check(const hpc_decode_params* p, int32_t batch, int32_t total_q, const void* q,
                                 const int32_t* q_start, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens, const int32_t* work_dev,
                                 int32_t n_units, const void* out, const float* lse) {
    if (!p || !q || !q_start || !k_cache || !v_cache || !block_table || !seq_lens || !out || !lse)
        return HPC_ERR_NULL;
    if (n_units > 0 && !work_dev) return HPC_ERR_NULL;
    if (p->head_dim != HPC_DECODE_HEAD_DIM || p->page_size != HPC_DECODE_PAGE) return HPC_ERR_UNSUPPORTED;
    if (p->kv_dtype != HPC_KV_BF16 && p->kv_dtype != HPC_KV_FP8_E4M3) return HPC_ERR_UNSUPPORTED;
    if (p->num_kv_heads < 1 || p->num_q_heads < p->num_kv_heads || p->num_q_heads % p->num_kv_heads != 0)
        return HPC_ERR_INVALID;
    if (p->num_q_heads / p->num_kv_heads > HPC_DECODE_MAX_GROUP) return HPC_ERR_UNSUPPORTED;
    if (p->tile_math != HPC_TILE_MATH_MFMA || p->fused_merge != 0) return HPC_ERR_UNSUPPORTED;
    if (p->max_pages_per_seq < 1 || p->num_pages < 1) return HPC_ERR_INVALID;
    if (!std::isfinite(p->sm_scale) || !std::isfinite(p->k_scale) || !std::isfinite(p->v_scale))
        return HPC_ERR_INVALID;
    // the kernel keeps its running max on raw scores, which needs a positive score scale
    if (!(static_cast<double>(p->sm_scale) * p->k_scale > 0.0)) return HPC_ERR_INVALID;
    if (batch < 1 || total_q < 0 || n_units < 0) return HPC_ERR_INVALID;
    // q row offsets (16 rows of one block, all heads) and tile indices must fit the kernels' int32 math
    if (int64_t(total_q) * p->num_q_heads * HPC_DECODE_HEAD_DIM * 2 >= INT32_MAX * int64_t(64)) return HPC_ERR_INVALID;
    if (int64_t(batch) * p->max_pages_per_seq >= INT32_MAX) return HPC_ERR_INVALID;
    if (int64_t(p->num_q_heads) * HPC_DECODE_HEAD_DIM * 2 * HPC_PREFILL_QUERY_BLOCK >= INT32_MAX) return HPC_ERR_INVALID;
    return HPC_OK;
}

extern "C" int hpc_prefill_attn(const hpc_decode_params* p, int32_t batch, int32_t total_q, const void* q,
                                const int32_t* q_start, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* seq_lens, const int32_t* work_dev,
                                int32_t n_units, void* out, float* lse, void* stream) {
    const int status = hpc_prefill_check(p, batch, total_q, q, q_start, k_cache, v_cache, block_table, seq_lens,
                                         work_dev, n_units, out, lse);
    if (status != HPC_OK) return status;
    hpcd::PrefillArgs a{};
    a.q = q;
    a.q_start = q_start;
    a.k = k_cache;
    a.v = v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.work = work_dev;
    a.out = out;
    a.lse = lse;
    a.batch = batch;
    a.num_q_heads = p->num_q_heads;
    a.num_kv_heads = p->num_kv_heads;
    a.group = p->num_q_heads / p->num_kv_heads;
    a.max_pages_per_seq = p->max_pages_per_seq;
    a.num_pages = p->num_pages;
    a.qk_scale_log2 = static_cast<float>(static_cast<double>(p->sm_scale) * p->k_scale * 1.4426950408889634);
    a.v_scale = p->v_scale;
    return hpcd::launch_prefill(a, n_units, p->kv_dtype == HPC_KV_FP8_E4M3, stream) == 0 ? HPC_OK : HPC_ERR_HIP;
}
