// The decode step's prologue on gfx950: QK-norm, RoPE and the paged append
// of the new token's K/V (fp8-quantised for an fp8 cache), one fused launch.
//
// "vLLM x HPC-Ops ...", §Attention Backend: Dynamic Load-Balanced Scheduling
// (the paragraph on the fused attention prologue) fuses QK-Norm, RoPE, the
// KV-cache write and, in FP8, query quantisation into one kernel, so the new
// token's q/k/v are read from HBM once and written once.  The pages give no
// formula; the forms used here:
//   * RMS norm of each head's 128 values with a per-dimension weight shared
//     by all heads (one for queries, one for keys), then
//   * RoPE in rotate-half form: dimension i pairs with i + 64, angle
//     p * theta^(-i/64) at the new token's position p;
//   * K and V go to row p % 64 of page block_table[b][p / 64]; an fp8 cache
//     stores e4m3(x / scale), nearest-even, saturated to +-448;
//   * the query is written in bf16 and, if asked for, as e4m3(q / q_scale).
//
// Layout of the work: one wave64 per (sequence, head).  Lane l holds
// dimensions l and l + 64 of its head, which are exactly a RoPE pair, so the
// rotation needs no data exchange; the mean square is one wave reduction.
// Waves of query heads write q_out; a wave of a KV head normalises and
// rotates K and copies (or quantises) V into the cache.  The rotation angle
// is formed and reduced in fp64 (positions reach 2^17 and beyond, where an
// fp32 angle would already be off by ~1e-2 rad); the rest runs in fp32.
// The kernel is latency-bound: a 64q/8kv batch of 32 moves about 1.3 MB.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace hpcd {
namespace {

constexpr int kPrologueWaves = 4;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, nearest with ties to even (the inputs here are finite)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// two fp32 values -> two OCP e4m3 codes (low byte = a), saturated to +-448;
// the conversion rounds to nearest-even
__device__ __forceinline__ uint16_t f32x2_to_e4m3(float a, float b) {
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return static_cast<uint16_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFF);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

__global__ void __launch_bounds__(64 * kPrologueWaves)
prologue_kernel(PrologueArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * kPrologueWaves + (threadIdx.x >> 6));
    const int heads = a.num_q_heads + a.num_kv_heads;
    if (wave >= a.batch * heads) return;
    const int b = wave / heads;
    const int h = wave - b * heads;
    const bool is_q = h < a.num_q_heads;

    // the new token's slot (uniform over the wave)
    const int pos = a.positions[b];
    int page = -1;
    if (pos >= 0 && pos < a.max_pages_per_seq * kPage) {
        page = a.block_table[static_cast<int64_t>(b) * a.max_pages_per_seq + pos / kPage];
        if (page >= a.num_pages) page = -1;
    }
    const bool valid = page >= 0;

    // inputs first, so the loads are in flight while the angle is formed
    const uint16_t* src = is_q ? a.q_in + (static_cast<int64_t>(b) * a.num_q_heads + h) * kHeadDim
                               : a.k_in + (static_cast<int64_t>(b) * a.num_kv_heads + (h - a.num_q_heads)) * kHeadDim;
    const uint16_t* wsrc = is_q ? a.q_norm_w : a.k_norm_w;
    const float x1 = bf16_to_f32(src[lane]);
    const float x2 = bf16_to_f32(src[lane + 64]);
    const float w1 = bf16_to_f32(wsrc[lane]);
    const float w2 = bf16_to_f32(wsrc[lane + 64]);
    uint16_t v1 = 0, v2 = 0;
    const int kvh = h - a.num_q_heads;
    if (!is_q && valid) {
        const uint16_t* vsrc = a.v_in + (static_cast<int64_t>(b) * a.num_kv_heads + kvh) * kHeadDim;
        v1 = vsrc[lane];
        v2 = vsrc[lane + 64];
    }

    // angle p * theta^(-lane/64), in fp64
    float c = 1.0f, s = 0.0f;
    if (valid && pos > 0) {
        const double ang = static_cast<double>(pos) * exp2(-static_cast<double>(lane) * a.log2_theta_over_64);
        double sd, cd;
        sincos(ang, &sd, &cd);
        c = static_cast<float>(cd);
        s = static_cast<float>(sd);
    }

    // RMS norm, then the rotation
    const float ms = wave_sum(x1 * x1 + x2 * x2) * (1.0f / kHeadDim);
    const float inv = 1.0f / __builtin_sqrtf(ms + a.eps);
    const float y1 = x1 * inv * w1;
    const float y2 = x2 * inv * w2;
    const float r1 = y1 * c - y2 * s;
    const float r2 = y2 * c + y1 * s;

    if (is_q) {
        const int64_t o = (static_cast<int64_t>(b) * a.num_q_heads + h) * kHeadDim;
        a.q_out[o + lane] = valid ? f32_to_bf16(r1) : 0;
        a.q_out[o + lane + 64] = valid ? f32_to_bf16(r2) : 0;
        if (a.q_fp8) {
            const uint16_t codes = valid ? f32x2_to_e4m3(__fdiv_rn(r1, a.q_scale), __fdiv_rn(r2, a.q_scale)) : 0;
            a.q_fp8[o + lane] = static_cast<uint8_t>(codes & 0xFF);
            a.q_fp8[o + lane + 64] = static_cast<uint8_t>(codes >> 8);
        }
        return;
    }
    if (!valid) return;
    const int64_t slot = ((static_cast<int64_t>(page) * a.num_kv_heads + kvh) * kPage + pos % kPage) * kHeadDim;
    if (a.kv_fp8) {
        uint8_t* kc = static_cast<uint8_t*>(a.k_cache) + slot;
        uint8_t* vc = static_cast<uint8_t*>(a.v_cache) + slot;
        const uint16_t kcodes = f32x2_to_e4m3(__fdiv_rn(r1, a.k_scale), __fdiv_rn(r2, a.k_scale));
        const uint16_t vcodes = f32x2_to_e4m3(__fdiv_rn(bf16_to_f32(v1), a.v_scale),
                                              __fdiv_rn(bf16_to_f32(v2), a.v_scale));
        kc[lane] = static_cast<uint8_t>(kcodes & 0xFF);
        kc[lane + 64] = static_cast<uint8_t>(kcodes >> 8);
        vc[lane] = static_cast<uint8_t>(vcodes & 0xFF);
        vc[lane + 64] = static_cast<uint8_t>(vcodes >> 8);
    } else {
        uint16_t* kc = static_cast<uint16_t*>(a.k_cache) + slot;
        uint16_t* vc = static_cast<uint16_t*>(a.v_cache) + slot;
        kc[lane] = f32_to_bf16(r1);
        kc[lane + 64] = f32_to_bf16(r2);
        vc[lane] = v1;
        vc[lane + 64] = v2;
    }
}

}  // namespace

int launch_prologue(const PrologueArgs& a, void* stream) {
    const int64_t waves = static_cast<int64_t>(a.batch) * (a.num_q_heads + a.num_kv_heads);
    const int grid = static_cast<int>((waves + kPrologueWaves - 1) / kPrologueWaves);
    if (grid == 0) return 0;
    hipLaunchKernelGGL(prologue_kernel, dim3(grid), dim3(64 * kPrologueWaves), 0,
                       static_cast<hipStream_t>(stream), a);
    return static_cast<int>(hipGetLastError());
}

}  // namespace hpcd
