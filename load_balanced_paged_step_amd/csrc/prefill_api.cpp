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

extern "C" int64_t hpc_prefill_plan_size(const int32_t* q_start, int32_t batch, int32_t num_kv_heads,
                                         int32_t n_workers) {
    const int64_t units = hpc_prefill_units(q_start, batch, num_kv_heads);
    if (units < 0) return units;
    if (n_workers < 0) return HPC_ERR_INVALID;
    // entries: every unit once, plus at most one more per worker share
    // (sum ceil(n_u / q) <= sum (n_u / q + 1) <= W + units), then merge records
    return int64_t(HPC_PREFILL_ENTRY_WORDS) * (units + n_workers) + int64_t(HPC_PREFILL_MERGE_WORDS) * units;
}

extern "C" int hpc_prefill_plan(const int32_t* q_start, const int32_t* seq_lens, int32_t batch,
                                int32_t num_kv_heads, int32_t max_pages_per_seq, int32_t n_workers,
                                int32_t min_share_tiles, int32_t* work, int64_t capacity_words, int32_t* counts) {
    if (!q_start || !seq_lens || !work || !counts) return HPC_ERR_NULL;
    if (max_pages_per_seq < 1 || n_workers < 0 || min_share_tiles < 1) return HPC_ERR_INVALID;
    const int64_t units = hpc_prefill_units(q_start, batch, num_kv_heads);
    if (units < 0) return static_cast<int>(units);
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t n = int64_t(q_start[b + 1]) - q_start[b];
        if (seq_lens[b] < 0 || n > seq_lens[b] || int64_t(seq_lens[b]) > int64_t(max_pages_per_seq) * HPC_DECODE_PAGE)
            return HPC_ERR_INVALID;
    }
    struct Unit {
        int32_t b, j, h, tiles;
    };
    std::vector<Unit> list;
    list.reserve(static_cast<std::size_t>(units));
    int64_t T = 0;
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t n = q_start[b + 1] - q_start[b];
        const int32_t L = seq_lens[b];
        for (int32_t j = 0; j * kQB < n; ++j) {
            const int32_t last = L - n + std::min(kQB * (j + 1), n) - 1;   // the block's last query position
            const int32_t tiles = last / HPC_DECODE_PAGE + 1;              // tiles that query sees
            for (int32_t h = 0; h < num_kv_heads; ++h) {
                list.push_back({b, j, h, tiles});
                T += tiles;
            }
        }
    }
    // balanced shares, q = max(ceil(T / W), min_share_tiles): a unit longer
    // than 2 q is cut at multiples of q (so the cut units of one KV head read
    // the same tiles in their k-th shares) and its partials are merged
    // afterwards.  A unit of at most 2 q tiles stays whole: it starts first
    // and ends within the step, whose length the grid's throughput sets
    // (n_workers = 0: no cuts).
    const int64_t q = n_workers > 0
                          ? std::max<int64_t>(std::max<int64_t>(1, (T + n_workers - 1) / n_workers), min_share_tiles)
                          : INT32_MAX;
    struct Entry {
        int32_t b, j, h, t0, t1, slot;
    };
    std::vector<Entry> entries;
    std::vector<int32_t> merge;
    int32_t partials = 0;
    for (const Unit& u : list) {
        const int64_t s = (u.tiles + q - 1) / q;
        if (u.tiles <= 2 * q) {
            entries.push_back({u.b, u.j, u.h, 0, u.tiles, -1});
            continue;
        }
        for (int64_t k = 0; k < s; ++k)
            entries.push_back({u.b, u.j, u.h, static_cast<int32_t>(k * q),
                               static_cast<int32_t>(std::min<int64_t>((k + 1) * q, u.tiles)),
                               partials + static_cast<int32_t>(k)});
        merge.insert(merge.end(), {u.b, u.j, u.h, static_cast<int32_t>(s), partials, 0, 0, 0});
        partials += static_cast<int32_t>(s);
    }
    const int64_t n_merge = static_cast<int64_t>(merge.size()) / HPC_PREFILL_MERGE_WORDS;
    const int64_t words = int64_t(HPC_PREFILL_ENTRY_WORDS) * entries.size() + int64_t(HPC_PREFILL_MERGE_WORDS) * n_merge;
    if (capacity_words < words) return HPC_ERR_TOO_SMALL;
    // longest entries first; ties by first tile, then in unit order, so that
    // equal shares over the same tiles are dispatched together
    std::stable_sort(entries.begin(), entries.end(), [](const Entry& x, const Entry& y) {
        return x.t1 - x.t0 != y.t1 - y.t0 ? x.t1 - x.t0 > y.t1 - y.t0 : x.t0 < y.t0;
    });
    for (std::size_t i = 0; i < entries.size(); ++i) {
        int32_t* e = work + HPC_PREFILL_ENTRY_WORDS * i;
        const Entry& x = entries[i];
        e[0] = x.b;
        e[1] = x.j;
        e[2] = x.h;
        e[3] = x.t1 - x.t0;
        e[4] = x.t0;
        e[5] = x.t1;
        e[6] = x.slot;
        e[7] = 0;
    }
    std::copy(merge.begin(), merge.end(), work + HPC_PREFILL_ENTRY_WORDS * entries.size());
    counts[0] = static_cast<int32_t>(entries.size());
    counts[1] = static_cast<int32_t>(n_merge);
    counts[2] = partials;
    return HPC_OK;
}

extern "C" int64_t hpc_prefill_workspace_size(int32_t n_partials, int32_t num_q_heads, int32_t num_kv_heads) {
    if (n_partials < 0 || num_kv_heads < 1 || num_q_heads < num_kv_heads || num_q_heads % num_kv_heads != 0)
        return HPC_ERR_INVALID;
    const int64_t G = num_q_heads / num_kv_heads;
    const int64_t rows = int64_t(n_partials) * kQB * G;
    const int64_t lse_off = (rows * HPC_DECODE_HEAD_DIM * 4 + 255) / 256 * 256;
    return n_partials == 0 ? 0 : lse_off + rows * 4;
}

extern "C" int hpc_prefill_check(const hpc_decode_params* p, int32_t batch, int32_t total_q, const void* q,
                                 const int32_t* q_start, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens, const int32_t* work_dev,
                                 int32_t n_entries, int32_t n_merge, int32_t n_partials, const void* workspace,
                                 int64_t workspace_bytes, const void* out, const float* lse) {
    if (!p || !q || !q_start || !k_cache || !v_cache || !block_table || !seq_lens || !out || !lse)
        return HPC_ERR_NULL;
    if (n_entries > 0 && !work_dev) return HPC_ERR_NULL;
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
    if (batch < 1 || total_q < 0 || n_entries < 0 || n_merge < 0 || n_partials < 0) return HPC_ERR_INVALID;
    // every cut unit has at least two shares, each an entry of its own
    if ((n_merge > 0) != (n_partials > 0) || 2 * int64_t(n_merge) > n_partials || n_partials > n_entries)
        return HPC_ERR_PLAN_MISMATCH;
    const int64_t need = hpc_prefill_workspace_size(n_partials, p->num_q_heads, p->num_kv_heads);
    if (need > 0 && !workspace) return HPC_ERR_NULL;
    if (workspace_bytes < need) return HPC_ERR_TOO_SMALL;
    // q row offsets (16 rows of one block, all heads) and tile indices must fit the kernels' int32 math
    if (int64_t(total_q) * p->num_q_heads * HPC_DECODE_HEAD_DIM * 2 >= INT32_MAX * int64_t(64)) return HPC_ERR_INVALID;
    if (int64_t(batch) * p->max_pages_per_seq >= INT32_MAX) return HPC_ERR_INVALID;
    if (int64_t(p->num_q_heads) * HPC_DECODE_HEAD_DIM * 2 * HPC_PREFILL_QUERY_BLOCK >= INT32_MAX) return HPC_ERR_INVALID;
    if (int64_t(n_merge) * (p->num_q_heads / p->num_kv_heads) >= INT32_MAX) return HPC_ERR_INVALID;
    return HPC_OK;
}

extern "C" int hpc_prefill_attn(const hpc_decode_params* p, int32_t batch, int32_t total_q, const void* q,
                                const int32_t* q_start, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* seq_lens, const int32_t* work_dev,
                                int32_t n_entries, int32_t n_merge, int32_t n_partials, void* workspace,
                                int64_t workspace_bytes, void* out, float* lse, void* stream) {
    const int status = hpc_prefill_check(p, batch, total_q, q, q_start, k_cache, v_cache, block_table, seq_lens,
                                         work_dev, n_entries, n_merge, n_partials, workspace, workspace_bytes, out,
                                         lse);
    if (status != HPC_OK) return status;
    const int32_t G = p->num_q_heads / p->num_kv_heads;
    const int64_t rows = int64_t(n_partials) * kQB * G;
    const int64_t lse_off = (rows * HPC_DECODE_HEAD_DIM * 4 + 255) / 256 * 256;
    hpcd::PrefillArgs a{};
    a.q = q;
    a.q_start = q_start;
    a.k = k_cache;
    a.v = v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.work = work_dev;
    a.merge = work_dev ? work_dev + int64_t(HPC_PREFILL_ENTRY_WORDS) * n_entries : nullptr;
    a.out = out;
    a.lse = lse;
    a.o_part = n_partials > 0 ? static_cast<float*>(workspace) : nullptr;
    a.lse_part = n_partials > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + lse_off) : nullptr;
    a.n_partials = n_partials;
    a.batch = batch;
    a.num_q_heads = p->num_q_heads;
    a.num_kv_heads = p->num_kv_heads;
    a.group = G;
    a.max_pages_per_seq = p->max_pages_per_seq;
    a.num_pages = p->num_pages;
    a.qk_scale_log2 = static_cast<float>(static_cast<double>(p->sm_scale) * p->k_scale * 1.4426950408889634);
    a.v_scale = p->v_scale;
    return hpcd::launch_prefill(a, n_entries, n_merge, p->kv_dtype == HPC_KV_FP8_E4M3, stream) == 0 ? HPC_OK
                                                                                                   : HPC_ERR_HIP;
}
