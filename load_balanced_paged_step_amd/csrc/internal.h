// Internal interface between the host-side C ABI (api.cpp) and the HIP
// kernels (decode_kernels.hip).  Not installed; no torch or HIP types.
#pragma once

#include <cstdint>

namespace hpcd {

constexpr int kHeadDim = 128;
constexpr int kPage = 64;
constexpr int kWaves = 4;                 // waves per decode workgroup
constexpr int kDecodeThreads = 64 * kWaves;
constexpr int kCombineThreads = 1024;

struct DecodeArgs {
    const void* q;               // bf16 [B][Hq][128]
    const void* k;               // bf16|fp8 [num_pages][H_kv][64][128]
    const void* v;
    const int32_t* block_table;  // [B][max_pages_per_seq]
    const int32_t* seq_lens;     // [B]
    const int32_t* worker_ptr;   // plan words (device)
    const int32_t* entries;      // plan words (device), 4 per entry
    void* out;                   // bf16 [B][Hq][128]
    float* lse;                  // [B][Hq]
    float* o_part;               // [n_partials][G][128]
    float* lse_part;             // [n_partials][G]
    int32_t num_kv_heads;
    int32_t group;               // G = Hq / H_kv, 1..16
    int32_t max_pages_per_seq;
    int32_t num_pages;
    float qk_scale_log2;         // sm_scale * k_scale * log2(e)
    float v_scale;
};

struct CombineArgs {
    const int32_t* combine;      // plan words (device), 3 per record
    const float* o_part;
    const float* lse_part;
    void* out;
    float* lse;
    int32_t num_kv_heads;
    int32_t group;
};

// Both return the hipError_t of the launch as int (0 = success).
int launch_decode(const DecodeArgs& a, int kv_dtype, int n_workers, void* stream);
int launch_combine(const CombineArgs& a, int n_combine, void* stream);

}  // namespace hpcd
