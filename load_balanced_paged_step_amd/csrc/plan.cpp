// Per-step tile scheduler and plan bookkeeping (host only, no HIP).
//
// Schedule: "vLLM x HPC-Ops: High-Performance Attention and MoE Backends from
// Tencent Hunyuan", §Attention Backend: Dynamic Load-Balanced Scheduling —
// every KV sequence is cut into uniform 64-token tiles and tiles are given to
// the persistent grid's workers by actual work, recomputed each decode step.
// The partition used is contiguous equal shares floor(w*T/W) of the
// unit-major tile list; the word layout is documented in hpc_decode.h.  The
// priced partition (this library's extension) evens out cost instead of
// tiles, a unit's first tile costing an entry price more than the others.
//
// Implementation: one forward sweep.  Worker ranges are increasing and
// contiguous, so a single cursor over the units (advanced past units that end
// at or before the range start) finds every (worker, unit) overlap in
// O(W + U) steps.

#include "hpc_decode.h"

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <vector>

namespace {

constexpr int64_t kPage = HPC_DECODE_PAGE;

struct Entry {
    int32_t unit, t0, t1, slot;
};

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
            if (T > INT32_MAX - 1) return false;
        }
    }
    return true;
}

// Worker boundaries s[0..W] of the tile list.  Plain: s_w = floor(w T / W).
// Priced by c quarter tiles: a tile costs 4 and a unit's first tile c more,
// A(j) is the cost of the tiles before j and C = A(T), and s_w is the
// largest j with A(j) <= floor(w C / W).  The price applies only when
// W <= T, C >= (4 + c + 1) W (each worker's share then exceeds the costliest
// tile, so no worker is left without one) and C < 2^31; the return value is
// the price applied (0: plain).
int32_t boundaries(const std::vector<int64_t>& s0, const std::vector<int64_t>& s1, int64_t T, int64_t W,
                   int32_t price, std::vector<int64_t>& s) {
    s.assign(static_cast<std::size_t>(W) + 1, 0);
    const int64_t K = static_cast<int64_t>(s0.size());
    const int64_t c = price;
    const int64_t C = 4 * T + c * K;
    if (c <= 0 || W > T || C < (4 + c + 1) * W || C >= (int64_t(1) << 31)) {
        for (int64_t w = 0; w <= W; ++w) s[w] = w * T / W;
        return 0;
    }
    int64_t k = 0;   // the last unit whose first tile's cost prefix is <= tau
    for (int64_t w = 0; w <= W; ++w) {
        const int64_t tau = w * C / W;
        while (k + 1 < K && 4 * s0[k + 1] + c * (k + 1) <= tau) ++k;
        // A(s0[k] + t) = 4 s0[k] + c k for t = 0, 4 (s0[k] + t) + c (k + 1) after
        const int64_t rem = tau - (4 * s0[k] + c * k) - c;
        const int64_t n = s1[k] - s0[k];
        s[w] = s0[k] + (rem < 4 ? 0 : std::min(n, rem / 4));
    }
    return price;
}

// over the W workers of a partition: the costliest worker (its tiles plus
// entry_cost per unit its range touches) and the entry count
void worker_costs(const std::vector<int64_t>& s0, const std::vector<int64_t>& s1, const std::vector<int64_t>& s,
                  double entry_cost, double& worst, int64_t& entries_total) {
    worst = 0.0;
    entries_total = 0;
    const int64_t W = static_cast<int64_t>(s.size()) - 1;
    const std::size_t U = s0.size();
    std::size_t u = 0;
    for (int64_t w = 0; w < W; ++w) {
        const int64_t a = s[w], e = s[w + 1];
        if (a == e) continue;
        while (u < U && s1[u] <= a) ++u;
        int64_t entries = 0;
        for (std::size_t v = u; v < U && s0[v] < e; ++v) ++entries;
        entries_total += entries;
        const double cost = static_cast<double>(e - a) + entry_cost * static_cast<double>(entries);
        if (cost > worst) worst = cost;
    }
}

}  // namespace

extern "C" int64_t hpc_decode_plan_size(int32_t batch, int32_t num_kv_heads, int32_t n_workers) {
    if (batch < 0 || num_kv_heads < 1 || n_workers < 1) return HPC_ERR_INVALID;
    const int64_t U = static_cast<int64_t>(batch) * num_kv_heads;
    const int64_t W = n_workers;
    return HPC_PLAN_HEADER_WORDS + (W + 1) + 4 * (W + U) + 3 * U;
}

extern "C" int hpc_decode_plan(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                               int32_t n_workers, int32_t* plan, int64_t plan_capacity) {
    return hpc_decode_plan_priced(seq_lens, batch, num_kv_heads, n_workers, 0, plan, plan_capacity);
}

extern "C" int hpc_decode_plan_priced(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                                      int32_t n_workers, int32_t entry_price, int32_t* plan,
                                      int64_t plan_capacity) {
    if (plan == nullptr || (batch > 0 && seq_lens == nullptr)) return HPC_ERR_NULL;
    if (batch < 0 || num_kv_heads < 1 || n_workers < 1 || entry_price < 0 ||
        entry_price > HPC_DECODE_MAX_ENTRY_PRICE)
        return HPC_ERR_INVALID;

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
    std::vector<int64_t> s0, s1, bound;
    int64_t T_ne = 0;
    unit_ranges(seq_lens, batch, num_kv_heads, s0, s1, T_ne);   // valid: checked above
    const int32_t price = boundaries(s0, s1, T, W, entry_price, bound);

    std::vector<Entry> entries;
    entries.reserve(static_cast<std::size_t>(W + U));
    std::vector<int32_t> worker_ptr(static_cast<std::size_t>(W) + 1);
    int64_t cursor = 0;  // first unit that may still own tiles
    for (int64_t w = 0; w < W; ++w) {
        worker_ptr[w] = static_cast<int32_t>(entries.size());
        int64_t lo = bound[w];
        const int64_t hi = bound[w + 1];
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
        HPC_DECODE_PAGE, price, 0, 0, 0, 0, 0, 0};
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
    std::vector<int64_t> bound;
    for (int32_t W = max_workers; W >= min_workers; --W) {
        double worst;
        int64_t entries;
        boundaries(s0, s1, T, W, 0, bound);
        worker_costs(s0, s1, bound, entry_cost, worst, entries);
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
    std::vector<int64_t> bound;
    boundaries(s0, s1, T, w1, 0, bound);
    worker_costs(s0, s1, bound, HPC_DECODE_ENTRY_COST, worst, entries);
    // dense entries (1.5 or more per worker) on an fp8 cache: two workers
    // per compute unit
    return 2 * entries >= 3 * static_cast<int64_t>(w1) ? 2 * n_cus : w1;
}

extern "C" int32_t hpc_decode_pick_entry_price(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                                               int32_t kv_dtype, int32_t n_workers) {
    if (batch > 0 && seq_lens == nullptr) return HPC_ERR_NULL;
    if (batch < 0 || num_kv_heads < 1 || n_workers < 1) return HPC_ERR_INVALID;
    if (kv_dtype != HPC_KV_BF16 && kv_dtype != HPC_KV_FP8_E4M3) return HPC_ERR_UNSUPPORTED;
    std::vector<int64_t> s0, s1;
    int64_t T = 0;
    if (!unit_ranges(seq_lens, batch, num_kv_heads, s0, s1, T)) return HPC_ERR_INVALID;
    if (T == 0) return 0;
    const double entry_cost = kv_dtype == HPC_KV_FP8_E4M3 ? HPC_DECODE_ENTRY_COST_FP8 : HPC_DECODE_ENTRY_COST;
    std::vector<int64_t> bound;
    double best_cost, worst;
    int64_t entries;
    boundaries(s0, s1, T, n_workers, 0, bound);
    worker_costs(s0, s1, bound, entry_cost, best_cost, entries);
    int32_t best = 0;
    for (int32_t price : {2, 4, 8, 16}) {
        if (boundaries(s0, s1, T, n_workers, price, bound) == 0) continue;
        worker_costs(s0, s1, bound, entry_cost, worst, entries);
        if (worst < best_cost * (1.0 - HPC_DECODE_MIN_GAIN) - 1e-9) {
            best = price;
            best_cost = worst;
        }
    }
    return best;
}

extern "C" int32_t hpc_decode_pick_merge(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                                         int32_t n_workers, int32_t entry_price) {
    if (batch > 0 && seq_lens == nullptr) return HPC_ERR_NULL;
    if (batch < 0 || num_kv_heads < 1 || n_workers < 1 || entry_price < 0 ||
        entry_price > HPC_DECODE_MAX_ENTRY_PRICE)
        return HPC_ERR_INVALID;
    std::vector<int64_t> s0, s1;
    int64_t T = 0;
    if (!unit_ranges(seq_lens, batch, num_kv_heads, s0, s1, T)) return HPC_ERR_INVALID;
    if (T == 0) return 1;
    std::vector<int64_t> bound;
    boundaries(s0, s1, T, n_workers, entry_price, bound);
    // workers per unit: each non-empty range [a, e) adds one to every unit it meets
    const std::size_t U = s0.size();
    std::vector<int32_t> shares(U, 0);
    std::size_t u = 0;
    for (int64_t w = 0; w < n_workers; ++w) {
        const int64_t a = bound[w], e = bound[w + 1];
        if (a == e) continue;
        while (u < U && s1[u] <= a) ++u;
        for (std::size_t v = u; v < U && s0[v] < e; ++v) ++shares[v];
    }
    int32_t most = 1;
    for (std::size_t v = 0; v < U; ++v) most = shares[v] > most ? shares[v] : most;
    if (most == 1) return 1;   // nothing to merge: the merge kernel's launch is saved
    return (T <= n_workers && most <= HPC_DECODE_FUSED_MAX_SHARES) ? 1 : 0;
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
