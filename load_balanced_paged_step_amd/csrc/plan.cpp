// Per-step tile scheduler and plan bookkeeping (host only, no HIP).
//
// Schedule: "vLLM x HPC-Ops: High-Performance Attention and MoE Backends from
// Tencent Hunyuan", §Attention Backend: Dynamic Load-Balanced Scheduling —
// every KV sequence is cut into uniform 64-token tiles and tiles are given to
// the persistent grid's workers by actual work, recomputed each decode step.
// The partition used is contiguous equal shares floor(w*T/W) of the
// unit-major tile list; the word layout is documented in hpc_decode.h.
//
// Implementation: one forward sweep.  Worker ranges are increasing and
// contiguous, so a single cursor over the units (advanced past units that end
// at or before the range start) finds every (worker, unit) overlap in
// O(W + U) steps.

#include "hpc_decode.h"

#include <cstddef>
#include <cstdint>
#include <vector>

namespace {

constexpr int64_t kPage = HPC_DECODE_PAGE;

struct Entry {
    int32_t unit, t0, t1, slot;
};

}  // namespace

extern "C" int64_t hpc_decode_plan_size(int32_t batch, int32_t num_kv_heads, int32_t n_workers) {
    if (batch < 0 || num_kv_heads < 1 || n_workers < 1) return HPC_ERR_INVALID;
    const int64_t U = static_cast<int64_t>(batch) * num_kv_heads;
    const int64_t W = n_workers;
    return HPC_PLAN_HEADER_WORDS + (W + 1) + 4 * (W + U) + 3 * U;
}

extern "C" int hpc_decode_plan(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                               int32_t n_workers, int32_t* plan, int64_t plan_capacity) {
    if (plan == nullptr || (batch > 0 && seq_lens == nullptr)) return HPC_ERR_NULL;
    if (batch < 0 || num_kv_heads < 1 || n_workers < 1) return HPC_ERR_INVALID;

    const int64_t H = num_kv_heads;
    const int64_t U = static_cast<int64_t>(batch) * H;
    const int64_t W = n_workers;

    // tile offset of every unit: start[u] = sum of n over units before u
    std::vector<int64_t> start(static_cast<std::size_t>(U) + 1);
    start[0] = 0;
    for (int64_t b = 0; b < batch; ++b) {
        const int32_t L = seq_lens[b];
        if (L < 0) return HPC_ERR_INVALID;
        const int64_t tiles = (static_cast<int64_t>(L) + kPage - 1) / kPage;
        for (int64_t h = 0; h < H; ++h) {
            const int64_t u = b * H + h;
            start[u + 1] = start[u] + tiles;
        }
    }
    const int64_t T = start[U];
    if (T > INT32_MAX - 1) return HPC_ERR_INVALID;

    std::vector<Entry> entries;
    entries.reserve(static_cast<std::size_t>(W + U));
    std::vector<int32_t> worker_ptr(static_cast<std::size_t>(W) + 1);
    int64_t cursor = 0;  // first unit that may still own tiles
    for (int64_t w = 0; w < W; ++w) {
        worker_ptr[w] = static_cast<int32_t>(entries.size());
        int64_t lo = (w * T) / W;
        const int64_t hi = ((w + 1) * T) / W;
        while (lo < hi) {
            while (start[cursor + 1] <= lo) ++cursor;
            const int64_t end = hi < start[cursor + 1] ? hi : start[cursor + 1];
            entries.push_back({static_cast<int32_t>(cursor), static_cast<int32_t>(lo - start[cursor]),
                               static_cast<int32_t>(end - start[cursor]), -1});
            lo = end;
        }
    }
    worker_ptr[W] = static_cast<int32_t>(entries.size());

    // entries per unit, then partial slot blocks for units split over >= 2 workers
    std::vector<int32_t> parts(static_cast<std::size_t>(U), 0);
    for (const Entry& e : entries) ++parts[e.unit];
    std::vector<int32_t> first_slot(static_cast<std::size_t>(U), 0);
    int64_t n_partials = 0;
    int64_t n_combine = 0;
    for (int64_t u = 0; u < U; ++u) {
        if (parts[u] >= 2) {
            first_slot[u] = static_cast<int32_t>(n_partials);
            n_partials += parts[u];
        }
        if (parts[u] != 1) ++n_combine;
    }
    std::vector<int32_t> next_slot(first_slot);
    for (Entry& e : entries)
        e.slot = parts[e.unit] >= 2 ? next_slot[e.unit]++ : -1;

    const int64_t E = static_cast<int64_t>(entries.size());
    const int64_t words = HPC_PLAN_HEADER_WORDS + (W + 1) + 4 * E + 3 * n_combine;
    if (plan_capacity < words) return HPC_ERR_TOO_SMALL;

    int32_t* p = plan;
    const int32_t header[HPC_PLAN_HEADER_WORDS] = {
        HPC_PLAN_VERSION, batch, num_kv_heads, n_workers, static_cast<int32_t>(T),
        static_cast<int32_t>(E), static_cast<int32_t>(n_partials), static_cast<int32_t>(n_combine),
        HPC_DECODE_PAGE, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < HPC_PLAN_HEADER_WORDS; ++i) *p++ = header[i];
    for (int64_t w = 0; w <= W; ++w) *p++ = worker_ptr[w];
    for (const Entry& e : entries) {
        *p++ = e.unit;
        *p++ = e.t0;
        *p++ = e.t1;
        *p++ = e.slot;
    }
    for (int64_t u = 0; u < U; ++u) {
        if (parts[u] == 1) continue;
        *p++ = static_cast<int32_t>(u);
        *p++ = parts[u];
        *p++ = parts[u] >= 2 ? first_slot[u] : 0;
    }
    return HPC_OK;
}

// Static split-KV baseline in the same word layout (the schedule the balanced
// scheduler is measured against in §Attention Decode under Mixed-Length
// Batches).  Every unit is cut into `splits` equal shares of its own tiles;
// each non-empty share is one worker with one entry.
extern "C" int64_t hpc_decode_plan_static_size(int32_t batch, int32_t num_kv_heads, int32_t splits) {
    if (batch < 0 || num_kv_heads < 1 || splits < 1) return HPC_ERR_INVALID;
    const int64_t U = static_cast<int64_t>(batch) * num_kv_heads;
    const int64_t W = U * splits > 1 ? U * splits : 1;
    return HPC_PLAN_HEADER_WORDS + (W + 1) + 4 * W + 3 * U;
}

extern "C" int hpc_decode_plan_static(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                                      int32_t splits, int32_t* plan, int64_t plan_capacity) {
    if (plan == nullptr || (batch > 0 && seq_lens == nullptr)) return HPC_ERR_NULL;
    if (batch < 0 || num_kv_heads < 1 || splits < 1) return HPC_ERR_INVALID;
    const int64_t H = num_kv_heads;
    const int64_t U = static_cast<int64_t>(batch) * H;

    std::vector<Entry> entries;
    std::vector<int32_t> parts(static_cast<std::size_t>(U), 0);
    int64_t T = 0;
    for (int64_t b = 0; b < batch; ++b) {
        const int32_t L = seq_lens[b];
        if (L < 0) return HPC_ERR_INVALID;
        const int64_t n = (static_cast<int64_t>(L) + kPage - 1) / kPage;
        T += n * H;
        if (n == 0) continue;
        const int64_t chunk = (n + splits - 1) / splits;
        const int32_t k_count = static_cast<int32_t>((n + chunk - 1) / chunk);
        for (int64_t h = 0; h < H; ++h) {
            const int64_t u = b * H + h;
            parts[u] = k_count;
            for (int64_t t0 = 0; t0 < n; t0 += chunk)
                entries.push_back({static_cast<int32_t>(u), static_cast<int32_t>(t0),
                                   static_cast<int32_t>(t0 + chunk < n ? t0 + chunk : n), -1});
        }
    }
    if (T > INT32_MAX - 1) return HPC_ERR_INVALID;

    const int64_t E = static_cast<int64_t>(entries.size());
    const int64_t W = E > 0 ? E : 1;
    if (W > INT32_MAX - 1) return HPC_ERR_INVALID;
    std::vector<int32_t> first_slot(static_cast<std::size_t>(U), 0);
    int64_t n_partials = 0, n_combine = 0;
    for (int64_t u = 0; u < U; ++u) {
        if (parts[u] >= 2) {
            first_slot[u] = static_cast<int32_t>(n_partials);
            n_partials += parts[u];
        }
        if (parts[u] != 1) ++n_combine;
    }
    std::vector<int32_t> next_slot(first_slot);
    for (Entry& e : entries) e.slot = parts[e.unit] >= 2 ? next_slot[e.unit]++ : -1;

    const int64_t words = HPC_PLAN_HEADER_WORDS + (W + 1) + 4 * E + 3 * n_combine;
    if (plan_capacity < words) return HPC_ERR_TOO_SMALL;
    int32_t* p = plan;
    const int32_t header[HPC_PLAN_HEADER_WORDS] = {
        HPC_PLAN_VERSION, batch, num_kv_heads, static_cast<int32_t>(W), static_cast<int32_t>(T),
        static_cast<int32_t>(E), static_cast<int32_t>(n_partials), static_cast<int32_t>(n_combine),
        HPC_DECODE_PAGE, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < HPC_PLAN_HEADER_WORDS; ++i) *p++ = header[i];
    for (int64_t w = 0; w <= W; ++w) *p++ = static_cast<int32_t>(w < E ? w : E);
    for (const Entry& e : entries) {
        *p++ = e.unit;
        *p++ = e.t0;
        *p++ = e.t1;
        *p++ = e.slot;
    }
    for (int64_t u = 0; u < U; ++u) {
        if (parts[u] == 1) continue;
        *p++ = static_cast<int32_t>(u);
        *p++ = parts[u];
        *p++ = parts[u] >= 2 ? first_slot[u] : 0;
    }
    return HPC_OK;
}

extern "C" int32_t hpc_decode_static_splits(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                                            int32_t n_cus, int32_t max_splits) {
    if (batch > 0 && seq_lens == nullptr) return HPC_ERR_NULL;
    if (batch < 0 || num_kv_heads < 1 || n_cus < 1 || max_splits < 1) return HPC_ERR_INVALID;
    int64_t n_max = 1;
    for (int32_t b = 0; b < batch; ++b) {
        if (seq_lens[b] < 0) return HPC_ERR_INVALID;
        const int64_t n = (static_cast<int64_t>(seq_lens[b]) + kPage - 1) / kPage;
        if (n > n_max) n_max = n;
    }
    const int64_t U = static_cast<int64_t>(batch) * num_kv_heads;
    int64_t S = 1;
    while (U * S < n_cus && 2 * S <= max_splits && 2 * S <= n_max) S *= 2;
    return static_cast<int32_t>(S);
}

namespace {

// [start, end) tile ranges of the units that have tiles, in unit order, and
// the total T; false for a negative length or 2^31 - 1 tiles or more
bool unit_ranges(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads, std::vector<int64_t>& s0,
                 std::vector<int64_t>& s1, int64_t& T) {
    T = 0;
    for (int32_t b = 0; b < batch; ++b) {
        if (seq_lens[b] < 0) return false;
        const int64_t n = (static_cast<int64_t>(seq_lens[b]) + kPage - 1) / kPage;
        for (int32_t h = 0; h < num_kv_heads && n > 0; ++h) {
            s0.push_back(T);
            T += n;
            s1.push_back(T);
        }
    }
    return T <= INT32_MAX - 1;
}

// over the W workers of the balanced partition: the costliest worker (its
// tiles plus entry_cost per unit its range touches) and the entry count
void worker_costs(const std::vector<int64_t>& s0, const std::vector<int64_t>& s1, int64_t T, int64_t W,
                  double entry_cost, double& worst, int64_t& entries_total) {
    worst = 0.0;
    entries_total = 0;
    const std::size_t U = s0.size();
    std::size_t u = 0;
    for (int64_t w = 0; w < W; ++w) {
        const int64_t a = w * T / W, e = (w + 1) * T / W;
        if (a == e) continue;
        while (u < U && s1[u] <= a) ++u;
        int64_t entries = 0;
        for (std::size_t v = u; v < U && s0[v] < e; ++v) ++entries;
        entries_total += entries;
        const double c = static_cast<double>(e - a) + entry_cost * static_cast<double>(entries);
        if (c > worst) worst = c;
    }
}

}  // namespace

extern "C" int32_t hpc_decode_choose_workers(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                                             int32_t min_workers, int32_t max_workers, float entry_cost) {
    if (batch > 0 && seq_lens == nullptr) return HPC_ERR_NULL;
    if (batch < 0 || num_kv_heads < 1 || min_workers < 1 || max_workers < min_workers || !(entry_cost >= 0.f) ||
        !(entry_cost < 1e30f))
        return HPC_ERR_INVALID;
    std::vector<int64_t> s0, s1;
    int64_t T = 0;
    if (!unit_ranges(seq_lens, batch, num_kv_heads, s0, s1, T)) return HPC_ERR_INVALID;
    if (T == 0) return max_workers;
    int32_t best = max_workers;
    double best_cost = 0.0;
    for (int32_t W = max_workers; W >= min_workers; --W) {
        double worst;
        int64_t entries;
        worker_costs(s0, s1, T, W, entry_cost, worst, entries);
        if (W == max_workers || worst < best_cost * (1.0 - HPC_DECODE_MIN_GAIN) - 1e-9) {
            best = W;
            best_cost = worst;
        }
    }
    return best;
}

extern "C" int32_t hpc_decode_pick_workers(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                                           int32_t kv_dtype, int32_t n_cus) {
    if (batch > 0 && seq_lens == nullptr) return HPC_ERR_NULL;
    if (n_cus < 2 || n_cus > (1 << 20)) return HPC_ERR_INVALID;
    if (kv_dtype != HPC_KV_BF16 && kv_dtype != HPC_KV_FP8_E4M3) return HPC_ERR_UNSUPPORTED;
    const int32_t w1 = hpc_decode_choose_workers(seq_lens, batch, num_kv_heads, n_cus / 2, n_cus,
                                                 HPC_DECODE_ENTRY_COST);
    if (w1 < 0 || kv_dtype != HPC_KV_FP8_E4M3) return w1;
    std::vector<int64_t> s0, s1;
    int64_t T = 0;
    unit_ranges(seq_lens, batch, num_kv_heads, s0, s1, T);   // valid: checked above
    if (T == 0) return w1;
    double worst;
    int64_t entries;
    worker_costs(s0, s1, T, w1, HPC_DECODE_ENTRY_COST, worst, entries);
    // dense entries (1.5 or more per worker) on an fp8 cache: two workers
    // per compute unit
    return 2 * entries >= 3 * static_cast<int64_t>(w1) ? 2 * n_cus : w1;
}

extern "C" int64_t hpc_decode_plan_words(const int32_t* plan) {
    if (plan == nullptr) return HPC_ERR_NULL;
    if (plan[0] != HPC_PLAN_VERSION || plan[8] != HPC_DECODE_PAGE) return HPC_ERR_PLAN_MISMATCH;
    const int64_t W = plan[3], E = plan[5], C = plan[7];
    if (W < 1 || E < 0 || C < 0) return HPC_ERR_PLAN_MISMATCH;
    return HPC_PLAN_HEADER_WORDS + (W + 1) + 4 * E + 3 * C;
}

extern "C" int64_t hpc_decode_workspace_size(const int32_t* plan, int32_t num_q_heads,
                                             int32_t num_kv_heads) {
    if (plan == nullptr) return HPC_ERR_NULL;
    if (plan[0] != HPC_PLAN_VERSION) return HPC_ERR_PLAN_MISMATCH;
    if (num_kv_heads < 1 || num_q_heads < num_kv_heads || num_q_heads % num_kv_heads != 0)
        return HPC_ERR_INVALID;
    const int64_t G = num_q_heads / num_kv_heads;
    const int64_t P = plan[6];
    if (P <= 0) return 0;
    const int64_t o_bytes = P * G * HPC_DECODE_HEAD_DIM * 4;
    const int64_t lse_off = (o_bytes + 255) / 256 * 256;
    return lse_off + P * G * 4;
}

extern "C" const char* hpc_status_string(int status) {
    switch (status) {
        case HPC_OK: return "ok";
        case HPC_ERR_NULL: return "null pointer argument";
        case HPC_ERR_INVALID: return "invalid size, count or length";
        case HPC_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case HPC_ERR_PLAN_MISMATCH: return "plan does not match the call";
        case HPC_ERR_TOO_SMALL: return "plan buffer or workspace too small";
        case HPC_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}
