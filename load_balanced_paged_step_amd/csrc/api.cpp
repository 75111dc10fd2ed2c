// C ABI entry point of the decode step: host-side validation, then the
// decode and merge launches on the caller's stream (see hpc_decode.h).
// Every check below runs before the first HIP call.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "hpc_decode.h"
#include "internal.h"

namespace hpcd {

namespace {
// tracing window: the caller's device buffer and its size, read by every
// decode launch (lock-free; set and cleared by the host calls below)
std::atomic<unsigned long long*> g_trace_buf{nullptr};
std::atomic<int64_t> g_trace_bytes{0};
}  // namespace

unsigned long long* trace_buffer(int n_workers) {
    unsigned long long* b = g_trace_buf.load(std::memory_order_acquire);
    if (b == nullptr || g_trace_bytes.load(std::memory_order_acquire) < int64_t(64) * n_workers) return nullptr;
    return b;
}

}  // namespace hpcd

namespace {

struct ProfileWindow {
    std::mutex mu;
    bool active = false;
    int32_t capacity = 0;
    int32_t used = 0;
    std::vector<hipEvent_t> ev;   // 4 per call: decode start / end, merge start / end (kernel timestamps)
    std::vector<uint8_t> launched;  // per call: bit 0 decode kernel, bit 1 merge kernel
};
ProfileWindow g_prof;

// events for one profiled call, or -1 outside a profiling window
int claim_profile_events(hipEvent_t ev[4], bool has_decode, bool has_combine) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (!g_prof.active || g_prof.used >= g_prof.capacity) return -1;
    const int idx = g_prof.used++;
    for (int i = 0; i < 4; ++i) ev[i] = g_prof.ev[4 * static_cast<std::size_t>(idx) + i];
    g_prof.launched[idx] = static_cast<uint8_t>((has_decode ? 1 : 0) | (has_combine ? 2 : 0));
    return idx;
}

void destroy_events() {
    for (hipEvent_t e : g_prof.ev)
        if (e) (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.launched.clear();
}

}  // namespace

extern "C" int hpc_decode_check(const hpc_decode_params* p, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* plan_host,
                                const int32_t* plan_dev, const void* workspace,
                                int64_t workspace_bytes, const void* out, const float* lse) {
    if (!p || !q || !k_cache || !v_cache || !block_table || !seq_lens || !plan_host || !plan_dev ||
        !out || !lse)
        return HPC_ERR_NULL;
    if (p->head_dim != HPC_DECODE_HEAD_DIM || p->page_size != HPC_DECODE_PAGE) return HPC_ERR_UNSUPPORTED;
    if (p->kv_dtype != HPC_KV_BF16 && p->kv_dtype != HPC_KV_FP8_E4M3) return HPC_ERR_UNSUPPORTED;
    if (p->num_kv_heads < 1 || p->num_q_heads < p->num_kv_heads || p->num_q_heads % p->num_kv_heads != 0)
        return HPC_ERR_INVALID;
    const int32_t G = p->num_q_heads / p->num_kv_heads;
    if (G > HPC_DECODE_MAX_GROUP) return HPC_ERR_UNSUPPORTED;
    if (p->tile_math != HPC_TILE_MATH_MFMA && p->tile_math != HPC_TILE_MATH_VALU) return HPC_ERR_INVALID;
    if (p->tile_math == HPC_TILE_MATH_VALU && G > hpcd::kValuMaxGroup) return HPC_ERR_UNSUPPORTED;
    if (p->fused_merge != 0 && p->fused_merge != 1) return HPC_ERR_INVALID;
    if (p->fused_merge) return HPC_ERR_UNSUPPORTED;   // the host-planned step has no in-kernel merge
    if (p->entry_price < 0 || p->entry_price > HPC_DECODE_MAX_ENTRY_PRICE) return HPC_ERR_INVALID;
    if (p->max_pages_per_seq < 1 || p->num_pages < 1) return HPC_ERR_INVALID;
    if (!std::isfinite(p->sm_scale) || !std::isfinite(p->k_scale) || !std::isfinite(p->v_scale))
        return HPC_ERR_INVALID;

    // plan header against the call
    const int32_t* hdr = plan_host;
    if (hdr[0] != HPC_PLAN_VERSION || hdr[8] != HPC_DECODE_PAGE) return HPC_ERR_PLAN_MISMATCH;
    const int32_t B = hdr[1], Hkv = hdr[2], W = hdr[3], E = hdr[5], P = hdr[6], C = hdr[7];
    if (Hkv != p->num_kv_heads || B < 0 || W < 1 || E < 0 || P < 0 || C < 0) return HPC_ERR_PLAN_MISMATCH;
    const int64_t U = static_cast<int64_t>(B) * Hkv;
    const int32_t* worker_ptr = plan_host + HPC_PLAN_HEADER_WORDS;
    const int32_t* entries = worker_ptr + (W + 1);
    const int32_t* combine = entries + 4 * static_cast<int64_t>(E);
    if (worker_ptr[0] != 0 || worker_ptr[W] != E) return HPC_ERR_PLAN_MISMATCH;
    for (int32_t w = 0; w < W; ++w)
        if (worker_ptr[w + 1] < worker_ptr[w]) return HPC_ERR_PLAN_MISMATCH;
    for (int64_t e = 0; e < E; ++e) {
        const int32_t u = entries[4 * e], t0 = entries[4 * e + 1], t1 = entries[4 * e + 2],
                      slot = entries[4 * e + 3];
        if (u < 0 || u >= U || t0 < 0 || t1 <= t0 || slot < -1 || slot >= P) return HPC_ERR_PLAN_MISMATCH;
        if (t1 > p->max_pages_per_seq) return HPC_ERR_INVALID;   // a length beyond the block table
    }
    for (int64_t c = 0; c < C; ++c) {
        const int32_t u = combine[3 * c], S = combine[3 * c + 1], base = combine[3 * c + 2];
        if (u < 0 || u >= U || S < 0 || S == 1 || base < 0 || static_cast<int64_t>(base) + S > P)
            return HPC_ERR_PLAN_MISMATCH;
    }
    const int64_t need = hpc_decode_workspace_size(plan_host, p->num_q_heads, p->num_kv_heads);
    if (need < 0) return static_cast<int>(need);
    if (need > 0 && (workspace == nullptr)) return HPC_ERR_NULL;
    if (workspace_bytes < need) return HPC_ERR_TOO_SMALL;
    return HPC_OK;
}

namespace {

// The launches of a host-planned step, after hpc_decode_check has passed.
int launch_planned(const hpc_decode_params* p, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_table, const int32_t* seq_lens, const int32_t* plan_host,
                   const int32_t* plan_dev, void* workspace, void* out, float* lse, void* stream) {
    const int32_t G = p->num_q_heads / p->num_kv_heads;
    const int32_t Hkv = plan_host[2], W = plan_host[3], E = plan_host[5], P = plan_host[6],
                  C = plan_host[7];

    float* o_part = static_cast<float*>(workspace);
    const int64_t o_bytes = static_cast<int64_t>(P) * G * HPC_DECODE_HEAD_DIM * 4;
    float* lse_part = P > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + (o_bytes + 255) / 256 * 256)
                            : nullptr;

    const int64_t e_off = HPC_PLAN_HEADER_WORDS + (W + 1);
    hpcd::DecodeArgs da{};
    da.q = q;
    da.k = k_cache;
    da.v = v_cache;
    da.block_table = block_table;
    da.seq_lens = seq_lens;
    da.worker_ptr = plan_dev + HPC_PLAN_HEADER_WORDS;
    da.entries = plan_dev + e_off;
    da.out = out;
    da.lse = lse;
    da.o_part = o_part;
    da.lse_part = lse_part;
    da.batch = plan_host[1];
    da.max_partials = P;
    da.num_kv_heads = Hkv;
    da.group = G;
    da.max_pages_per_seq = p->max_pages_per_seq;
    da.num_pages = p->num_pages;
    da.qk_scale_log2 = static_cast<float>(static_cast<double>(p->sm_scale) * p->k_scale * 1.4426950408889634);
    da.v_scale = p->v_scale;

    hpcd::CombineArgs ca{};
    ca.combine = plan_dev + e_off + 4 * static_cast<int64_t>(E);
    ca.o_part = o_part;
    ca.lse_part = lse_part;
    ca.out = out;
    ca.lse = lse;
    ca.num_kv_heads = Hkv;
    ca.group = G;
    ca.max_partials = P;

    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    claim_profile_events(ev, E > 0, C > 0);
    if (E > 0 && hpcd::launch_decode(da, p->kv_dtype, p->tile_math, W, false, stream, ev[0], ev[1]) != 0) return HPC_ERR_HIP;
    if (C > 0 && hpcd::launch_combine(ca, C, false, stream, ev[2], ev[3]) != 0) return HPC_ERR_HIP;
    return HPC_OK;
}

}  // namespace

extern "C" int hpc_decode_attn(const hpc_decode_params* p, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* plan_host,
                               const int32_t* plan_dev, void* workspace, int64_t workspace_bytes,
                               void* out, float* lse, void* stream) {
    const int status = hpc_decode_check(p, q, k_cache, v_cache, block_table, seq_lens, plan_host,
                                        plan_dev, workspace, workspace_bytes, out, lse);
    if (status != HPC_OK) return status;
    return launch_planned(p, q, k_cache, v_cache, block_table, seq_lens, plan_host, plan_dev, workspace, out,
                          lse, stream);
}

extern "C" int64_t hpc_decode_plan_workspace_bound(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                                   int32_t n_workers) {
    if (batch < 0 || n_workers < 1 || num_kv_heads < 1 || num_q_heads < num_kv_heads ||
        num_q_heads % num_kv_heads != 0)
        return HPC_ERR_INVALID;
    // every split entry has a slot, and a plan has at most W + U - 1 entries
    const int64_t partials = static_cast<int64_t>(n_workers) + static_cast<int64_t>(batch) * num_kv_heads;
    const int64_t G = num_q_heads / num_kv_heads;
    const int64_t o_bytes = partials * G * HPC_DECODE_HEAD_DIM * 4;
    return (o_bytes + 255) / 256 * 256 + partials * G * 4;
}

extern "C" int hpc_decode_plan_attn(const hpc_decode_params* p, const int32_t* seq_lens_host, int32_t batch,
                                    int32_t n_workers, int32_t* plan_host, int64_t plan_capacity,
                                    int32_t* plan_dev, const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens, void* workspace,
                                    int64_t workspace_bytes, void* out, float* lse, void* stream) {
    if (!p || !plan_host || !plan_dev) return HPC_ERR_NULL;
    if (p->entry_price < 0 || p->entry_price > HPC_DECODE_MAX_ENTRY_PRICE) return HPC_ERR_INVALID;
    int status = hpc_decode_plan_priced(seq_lens_host, batch, p->num_kv_heads, n_workers, p->entry_price, plan_host,
                                        plan_capacity);
    if (status != HPC_OK) return status;
    status = hpc_decode_check(p, q, k_cache, v_cache, block_table, seq_lens, plan_host, plan_dev, workspace,
                              workspace_bytes, out, lse);
    if (status != HPC_OK) return status;
    const int64_t words = hpc_decode_plan_words(plan_host);
    if (words < 0) return static_cast<int>(words);
    if (static_cast<const void*>(plan_dev) == static_cast<const void*>(plan_host)) {
        // in place: the kernels read the plan from the caller's pinned host
        // buffer, which must be mapped at the same address on the device
        hipPointerAttribute_t attr{};
        if (hipPointerGetAttributes(&attr, plan_host) != hipSuccess || attr.type != hipMemoryTypeHost ||
            attr.devicePointer != static_cast<void*>(plan_host)) {
            (void)hipGetLastError();
            return HPC_ERR_INVALID;
        }
    } else if (hipMemcpyAsync(plan_dev, plan_host, static_cast<size_t>(words) * sizeof(int32_t),
                              hipMemcpyHostToDevice, static_cast<hipStream_t>(stream)) != hipSuccess) {
        return HPC_ERR_HIP;
    }
    return launch_planned(p, q, k_cache, v_cache, block_table, seq_lens, plan_host, plan_dev, workspace, out,
                          lse, stream);
}

// ---------------------------------------------------------------------------
// Device-scheduled step: the kernels derive the schedule from seq_lens.

namespace {

// partial slots of the device-scheduled step: two per worker (its first and
// its last entry are the only ones that can be split)
int64_t step_partials_bound(int32_t /*batch*/, int32_t /*num_kv_heads*/, int32_t n_workers) {
    return 2 * static_cast<int64_t>(n_workers);
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// device-scheduled workspace: partial outputs, partial lse, per-unit merge records
struct StepLayout {
    int64_t o_off, lse_off, rec_off, total;
};

StepLayout step_layout(int64_t partials, int64_t G, int64_t units) {
    StepLayout L{};
    L.o_off = 0;
    L.lse_off = align256(partials * G * HPC_DECODE_HEAD_DIM * 4);
    L.rec_off = align256(L.lse_off + partials * G * 4);
    L.total = L.rec_off + 6 * units * 4;
    return L;
}

}  // namespace

extern "C" int64_t hpc_decode_step_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                                  int32_t n_workers) {
    if (batch < 0 || n_workers < 1 || num_kv_heads < 1 || num_q_heads < num_kv_heads ||
        num_q_heads % num_kv_heads != 0)
        return HPC_ERR_INVALID;
    return step_layout(step_partials_bound(batch, num_kv_heads, n_workers), num_q_heads / num_kv_heads,
                       static_cast<int64_t>(batch) * num_kv_heads)
        .total;
}

extern "C" int hpc_decode_step_check(const hpc_decode_params* p, int32_t batch, int32_t n_workers, const void* q,
                                     const void* k_cache, const void* v_cache, const int32_t* block_table,
                                     const int32_t* seq_lens, const void* workspace, int64_t workspace_bytes,
                                     const void* out, const float* lse) {
    if (!p || !q || !k_cache || !v_cache || !block_table || !seq_lens || !out || !lse) return HPC_ERR_NULL;
    if (p->head_dim != HPC_DECODE_HEAD_DIM || p->page_size != HPC_DECODE_PAGE) return HPC_ERR_UNSUPPORTED;
    if (p->kv_dtype != HPC_KV_BF16 && p->kv_dtype != HPC_KV_FP8_E4M3) return HPC_ERR_UNSUPPORTED;
    if (p->num_kv_heads < 1 || p->num_q_heads < p->num_kv_heads || p->num_q_heads % p->num_kv_heads != 0)
        return HPC_ERR_INVALID;
    if (p->num_q_heads / p->num_kv_heads > HPC_DECODE_MAX_GROUP) return HPC_ERR_UNSUPPORTED;
    if (p->tile_math != HPC_TILE_MATH_MFMA && p->tile_math != HPC_TILE_MATH_VALU) return HPC_ERR_INVALID;
    if (p->tile_math == HPC_TILE_MATH_VALU && p->num_q_heads / p->num_kv_heads > hpcd::kValuMaxGroup)
        return HPC_ERR_UNSUPPORTED;
    if (p->fused_merge != 0 && p->fused_merge != 1) return HPC_ERR_INVALID;
    if (p->entry_price < 0 || p->entry_price > HPC_DECODE_MAX_ENTRY_PRICE) return HPC_ERR_INVALID;
    if (p->max_pages_per_seq < 1 || p->num_pages < 1) return HPC_ERR_INVALID;
    if (!std::isfinite(p->sm_scale) || !std::isfinite(p->k_scale) || !std::isfinite(p->v_scale))
        return HPC_ERR_INVALID;
    if (batch < 1 || n_workers < 1) return HPC_ERR_INVALID;
    if (batch > hpcd::kDeviceSchedMaxBatch || n_workers > hpcd::kDeviceSchedMaxWorkers ||
        static_cast<int64_t>(batch) * p->num_kv_heads > hpcd::kDeviceSchedMaxUnits)
        return HPC_ERR_UNSUPPORTED;
    // every tile index the kernels form must fit in int32
    if (static_cast<int64_t>(batch) * p->max_pages_per_seq * p->num_kv_heads >= INT32_MAX) return HPC_ERR_INVALID;
    const int64_t need = hpc_decode_step_workspace_size(batch, p->num_q_heads, p->num_kv_heads, n_workers);
    if (need < 0) return static_cast<int>(need);
    if (need > 0 && workspace == nullptr) return HPC_ERR_NULL;
    if (workspace_bytes < need) return HPC_ERR_TOO_SMALL;
    return HPC_OK;
}

extern "C" int hpc_decode_step(const hpc_decode_params* p, int32_t batch, int32_t n_workers, const void* q,
                               const void* k_cache, const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, void* workspace, int64_t workspace_bytes, void* out,
                               float* lse, void* stream) {
    const int status = hpc_decode_step_check(p, batch, n_workers, q, k_cache, v_cache, block_table, seq_lens,
                                             workspace, workspace_bytes, out, lse);
    if (status != HPC_OK) return status;
    const int32_t G = p->num_q_heads / p->num_kv_heads;
    const int64_t P = step_partials_bound(batch, p->num_kv_heads, n_workers);
    const StepLayout L = step_layout(P, G, static_cast<int64_t>(batch) * p->num_kv_heads);
    char* ws = static_cast<char*>(workspace);
    float* o_part = reinterpret_cast<float*>(ws + L.o_off);
    float* lse_part = reinterpret_cast<float*>(ws + L.lse_off);
    int32_t* records = reinterpret_cast<int32_t*>(ws + L.rec_off);

    hpcd::DecodeArgs da{};
    da.q = q;
    da.k = k_cache;
    da.v = v_cache;
    da.block_table = block_table;
    da.seq_lens = seq_lens;
    da.out = out;
    da.lse = lse;
    da.o_part = o_part;
    da.lse_part = lse_part;
    da.merge_records = records;
    da.batch = batch;
    da.max_partials = static_cast<int32_t>(P);
    da.num_kv_heads = p->num_kv_heads;
    da.group = G;
    da.max_pages_per_seq = p->max_pages_per_seq;
    da.num_pages = p->num_pages;
    da.qk_scale_log2 = static_cast<float>(static_cast<double>(p->sm_scale) * p->k_scale * 1.4426950408889634);
    da.v_scale = p->v_scale;
    da.fused_merge = p->fused_merge;
    da.entry_price = p->entry_price;

    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    hpcd::CombineArgs ca{};
    ca.combine = records;
    ca.o_part = o_part;
    ca.lse_part = lse_part;
    ca.out = out;
    ca.lse = lse;
    ca.num_kv_heads = p->num_kv_heads;
    ca.group = G;
    ca.max_partials = static_cast<int32_t>(P);

    ca.n_workers = n_workers;
    const int64_t units = static_cast<int64_t>(batch) * p->num_kv_heads;
    const bool any_split = n_workers > 1 && !p->fused_merge;   // fused: the decode kernel merges

    claim_profile_events(ev, true, any_split);
    if (hpcd::launch_decode(da, p->kv_dtype, p->tile_math, n_workers, true, stream, ev[0], ev[1]) != 0) return HPC_ERR_HIP;
    if (any_split && hpcd::launch_combine(ca, static_cast<int>(units), true, stream, ev[2], ev[3]) != 0)
        return HPC_ERR_HIP;
    return HPC_OK;
}

extern "C" int hpc_decode_plan_device(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                                      int32_t n_workers, int32_t entry_price, int32_t max_pages_per_seq,
                                      int32_t* plan, int64_t plan_capacity, void* stream) {
    if (!seq_lens || !plan) return HPC_ERR_NULL;
    if (batch < 1 || num_kv_heads < 1 || n_workers < 1 || max_pages_per_seq < 1 || entry_price < 0 ||
        entry_price > HPC_DECODE_MAX_ENTRY_PRICE)
        return HPC_ERR_INVALID;
    if (batch > hpcd::kPlanDeviceMaxBatch || n_workers > hpcd::kPlanDeviceMaxWorkers ||
        static_cast<int64_t>(batch) * num_kv_heads > hpcd::kPlanDeviceMaxUnits)
        return HPC_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(batch) * max_pages_per_seq * num_kv_heads >= INT32_MAX) return HPC_ERR_INVALID;
    if (plan_capacity < hpc_decode_plan_size(batch, num_kv_heads, n_workers)) return HPC_ERR_TOO_SMALL;
    return hpcd::launch_plan_device(seq_lens, batch, num_kv_heads, n_workers, entry_price, max_pages_per_seq, plan,
                                    stream) == 0
               ? HPC_OK
               : HPC_ERR_HIP;
}

extern "C" int hpc_decode_trace_start(void* device_buffer, int64_t bytes) {
    if (device_buffer == nullptr) return HPC_ERR_NULL;
    if (bytes < 64) return HPC_ERR_INVALID;
    hpcd::g_trace_buf.store(nullptr, std::memory_order_release);
    hpcd::g_trace_bytes.store(bytes, std::memory_order_release);
    hpcd::g_trace_buf.store(static_cast<unsigned long long*>(device_buffer), std::memory_order_release);
    return HPC_OK;
}

extern "C" int64_t hpc_decode_wall_clock_hz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        khz <= 0)
        return HPC_ERR_HIP;
    return int64_t(khz) * 1000;
}

extern "C" int hpc_decode_trace_stop(void) {
    hpcd::g_trace_buf.store(nullptr, std::memory_order_release);
    hpcd::g_trace_bytes.store(0, std::memory_order_release);
    return HPC_OK;
}

extern "C" int hpc_decode_profile_start(int32_t capacity) {
    if (capacity < 1) return HPC_ERR_INVALID;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    destroy_events();
    g_prof.ev.assign(4 * static_cast<std::size_t>(capacity), nullptr);
    g_prof.launched.assign(static_cast<std::size_t>(capacity), 0);
    for (hipEvent_t& e : g_prof.ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            e = nullptr;
            destroy_events();
            g_prof.active = false;
            return HPC_ERR_HIP;
        }
    }
    g_prof.capacity = capacity;
    g_prof.used = 0;
    g_prof.active = true;
    return HPC_OK;
}

extern "C" int hpc_decode_profile_stop(double* decode_ms, double* combine_ms, int32_t* n_calls) {
    if (!decode_ms || !combine_ms || !n_calls) return HPC_ERR_NULL;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    double dsum = 0.0, csum = 0.0;
    int rc = HPC_OK;
    for (int32_t i = 0; i < g_prof.used; ++i) {
        float a = 0.f, b = 0.f;
        if (g_prof.launched[i] & 1) {
            if (hipEventSynchronize(g_prof.ev[4 * i + 1]) != hipSuccess ||
                hipEventElapsedTime(&a, g_prof.ev[4 * i], g_prof.ev[4 * i + 1]) != hipSuccess) {
                rc = HPC_ERR_HIP;
                break;
            }
            dsum += a;
        }
        if (g_prof.launched[i] & 2) {
            if (hipEventSynchronize(g_prof.ev[4 * i + 3]) != hipSuccess ||
                hipEventElapsedTime(&b, g_prof.ev[4 * i + 2], g_prof.ev[4 * i + 3]) != hipSuccess) {
                rc = HPC_ERR_HIP;
                break;
            }
            csum += b;
        }
    }
    *decode_ms = dsum;
    *combine_ms = csum;
    *n_calls = g_prof.used;
    destroy_events();
    g_prof.active = false;
    g_prof.used = 0;
    g_prof.capacity = 0;
    return rc;
}
