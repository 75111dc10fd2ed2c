// Internal interface between the host-side C ABI (api.cpp) and the HIP
// kernels (decode_kernels.hip).  Not installed; no torch or HIP types.
#pragma once

#include <cstdint>

namespace hpcd {

constexpr int kHeadDim = 128;
constexpr int kPage = 64;
constexpr int kWaves = 4;                 // waves per decode workgroup
constexpr int kDecodeThreads = 64 * kWaves;
constexpr int kCombineThreads = 256;
constexpr int kPlanThreads = 1024;
constexpr int kValuMaxGroup = 8;          // query heads per KV head the VALU tile math holds

// Limits of the device-scheduled path: the lengths, their tile prefix and
// the per-unit split tables live in LDS of every workgroup.
constexpr int kDeviceSchedMaxBatch = 2048;
constexpr int kDeviceSchedMaxUnits = 4096;
constexpr int kDeviceSchedMaxWorkers = 65536;   // keeps every schedule quotient below 2^20
// Limits of the plan-materialising kernel (one workgroup, everything in LDS).
constexpr int kPlanDeviceMaxBatch = 2048;
constexpr int kPlanDeviceMaxWorkers = 2048;
constexpr int kPlanDeviceMaxUnits = 4096;

struct DecodeArgs {
    const void* q;               // bf16 [B][Hq][128]
    const void* k;               // bf16|fp8 [num_pages][H_kv][64][128]
    const void* v;
    const int32_t* block_table;  // [B][max_pages_per_seq]
    const int32_t* seq_lens;     // [B]
    const int32_t* worker_ptr;   // host plan words (device copy); unused when scheduled on device
    const int32_t* entries;      // host plan words (device copy), 4 per entry
    void* out;                   // bf16 [B][Hq][128]
    float* lse;                  // [B][Hq]
    float* o_part;               // [n_partials][G][128]
    float* lse_part;             // [n_partials][G]
    int32_t* merge_records;      // device schedule: [units][6] merge records (see decode_kernels.hip)
    int32_t batch;
    int32_t num_kv_heads;
    int32_t group;               // G = Hq / H_kv, 1..16
    int32_t max_pages_per_seq;
    int32_t num_pages;
    int32_t max_partials;        // partial slots in the workspace
    float qk_scale_log2;         // sm_scale * k_scale * log2(e)
    float v_scale;
    int32_t fused_merge;         // device schedule: the decode kernel merges split units itself
    int32_t entry_price;         // device schedule: the partition's price of a unit start, quarter tiles
};

struct CombineArgs {
    const int32_t* combine;      // merge records: host plan list (3 words each) or per-unit device records
    int32_t n_workers;           // W (device records)
    const float* o_part;
    const float* lse_part;
    void* out;
    float* lse;
    int32_t num_kv_heads;
    int32_t group;
    int32_t max_partials;        // partial slots in the workspace
};

struct PrologueArgs {
    const uint16_t* q_in;        // bf16 [B][Hq][128]
    const uint16_t* k_in;        // bf16 [B][H_kv][128]
    const uint16_t* v_in;        // bf16 [B][H_kv][128]
    const uint16_t* q_norm_w;    // bf16 [128]
    const uint16_t* k_norm_w;    // bf16 [128]
    const int32_t* positions;    // [B]
    const int32_t* block_table;  // [B][max_pages_per_seq]
    void* k_cache;               // bf16|fp8 [num_pages][H_kv][64][128]
    void* v_cache;
    uint16_t* q_out;             // bf16 [B][Hq][128]
    uint8_t* q_fp8;              // e4m3 [B][Hq][128] or null
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t max_pages_per_seq;
    int32_t num_pages;
    int32_t kv_fp8;              // 1: fp8 e4m3 cache, 0: bf16
    float eps;
    float k_scale, v_scale, q_scale;
    double log2_theta_over_64;   // log2(theta) / 64: the angle of dimension i is p * 2^(-i * this)
};

struct PrefillArgs {
    const void* q;               // bf16 [total][Hq][128]
    const int32_t* q_start;      // [B + 1]
    const void* k;               // bf16|fp8 [num_pages][H_kv][64][128]
    const void* v;
    const int32_t* block_table;  // [B][max_pages_per_seq]
    const int32_t* seq_lens;     // [B]: cached tokens, the chunk's new tokens included
    const int32_t* work;         // [n_entries][8]: (sequence, query block, KV head, cost, t0, t1, slot, 0)
    const int32_t* merge;        // [n_merge][8]: (sequence, query block, KV head, shares, first slot, 0...)
    void* out;                   // bf16 [total][Hq][128]
    float* lse;                  // [total][Hq]
    float* o_part;               // [n_partials][16][G][128]: partial outputs of split units
    float* lse_part;             // [n_partials][16][G]
    int32_t n_partials;
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t max_pages_per_seq;
    int32_t num_pages;
    float qk_scale_log2;
    float v_scale;
};

// All return the hipError_t of the launch as int (0 = success).
// device_sched: the decode kernel derives the schedule from seq_lens itself
// and writes one merge record per unit for the merge kernel.
// ev_start / ev_stop (hipEvent_t or null): events that the launch itself
// stamps when the kernel starts and ends, i.e. the kernel's own duration.
// tile_math: HPC_TILE_MATH_MFMA or HPC_TILE_MATH_VALU (the latter needs group <= 8).
int launch_decode(const DecodeArgs& a, int kv_dtype, int tile_math, int n_workers, bool device_sched, void* stream,
                  void* ev_start = nullptr, void* ev_stop = nullptr);
int launch_combine(const CombineArgs& a, int n_records, bool device_sched, void* stream,
                   void* ev_start = nullptr, void* ev_stop = nullptr);
int launch_prologue(const PrologueArgs& a, void* stream);
// The tracing window's device buffer when it is on and holds n_workers
// workers' stamps (8 words each), else null (api.cpp).
unsigned long long* trace_buffer(int n_workers);
int launch_prefill(const PrefillArgs& a, int n_entries, int n_merge, bool kv_fp8, void* stream);
int launch_plan_device(const int32_t* seq_lens, int batch, int num_kv_heads, int n_workers, int entry_price,
                       int max_pages_per_seq, int32_t* plan, void* stream);

}  // namespace hpcd
