// hpc_decode_step_noalloc: the device-scheduled decode step with its scratch
// (fp32 partial outputs and log-sum-exps, per-unit merge records) taken from
// a fixed array in device memory instead of a caller-supplied workspace, for
// callers that cannot allocate device memory.
//
// The array is a file-scope __device__ variable, so every GPU the library
// runs on holds its own copy, at its own address, for as long as the process
// lives.  Its host-side name is not a device address: the device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever handed to kernels.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "hpc_decode.h"

namespace {

constexpr int64_t kScratchBytes = int64_t(16) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};
const char kPresent = 0;   // non-null marker for the host checks, which only test pointers for null

// Device address of `scratch` on the current device, looked up on the first
// call on that device; nullptr (and *status set) when the lookup fails.
void* scratch_on_current_device(int* status) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *status = HPC_ERR_HIP;
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            *status = HPC_ERR_HIP;
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int64_t hpc_decode_step_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int hpc_decode_step_noalloc(const hpc_decode_params* p, int32_t batch, int32_t n_workers,
                                       const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                                       void* stream) {
    if (!p) return HPC_ERR_NULL;
    // the in-kernel merge counts arrivals in the scratch across calls, at
    // offsets that move with the batch shape; only the merge-kernel mode,
    // which rewrites every record it reads, can share one array between calls
    if (p->fused_merge != 0) return p->fused_merge == 1 ? HPC_ERR_UNSUPPORTED : HPC_ERR_INVALID;
    if (batch < 1 || n_workers < 1) return HPC_ERR_INVALID;
    const int64_t need = hpc_decode_step_workspace_size(batch, p->num_q_heads, p->num_kv_heads, n_workers);
    if (need < 0) return static_cast<int>(need);
    if (need > kScratchBytes) return HPC_ERR_TOO_SMALL;
    // every other host check before any HIP call (the checks never dereference the workspace)
    const int check = hpc_decode_step_check(p, batch, n_workers, q, k_cache, v_cache, block_table, seq_lens,
                                            &kPresent, kScratchBytes, out, lse);
    if (check != HPC_OK) return check;
    int status = HPC_OK;
    void* ws = scratch_on_current_device(&status);
    if (!ws) return status;
    return hpc_decode_step(p, batch, n_workers, q, k_cache, v_cache, block_table, seq_lens, ws, kScratchBytes, out,
                           lse, stream);
}
