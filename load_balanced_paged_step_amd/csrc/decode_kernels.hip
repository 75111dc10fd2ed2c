// Persistent paged GQA decode attention and the log-sum-exp merge, for
// CDNA4 (gfx950).
//
// Method: "vLLM x HPC-Ops: High-Performance Attention and MoE Backends from
// Tencent Hunyuan", §Attention Backend: Dynamic Load-Balanced Scheduling —
// 64-token KV tiles spread evenly over a persistent grid; a sequence split
// over several workers is merged afterwards (log-sum-exp, the reading used
// here; the pages do not describe the merge).  Head shape (8 query heads per
// KV head, head dim 128): "vLLM und Tencent Hunyuan streamen zwei
// HPC-Backends ...", §Zwei neue HPC-Backends im vLLM-Ökosystem.  The pages'
// own kernels target Hopper; nothing of their design is assumed here.
//
// Decode kernel (one workgroup = one worker of the plan, 4 waves):
//  * every wave takes a fixed 16-token slice (rows 16*wave .. 16*wave+15) of
//    every 64-token tile of the worker's entries and keeps its own online
//    softmax state; the four states are merged through LDS at the end of
//    each entry, so a workgroup emits one result per entry;
//  * K and V rows are read straight from HBM into VGPRs with buffer loads
//    whose range is the valid part of the page: rows past the sequence end
//    (and tiles past the entry end, used to keep the prefetch ring
//    branch-free) come back as zeros without touching memory;
//  * S = K Q^T on MFMA 16x16x32 bf16 (rows = 16 tokens, columns = the G <= 16
//    query heads of the group, zero-padded); P V on MFMA 16x16x16 bf16 as
//    O^T = V^T P^T, with V^T operands built in registers by byte permutes
//    (each lane holds 4 token rows x 8 dims), so the softmax state and the
//    accumulator share one lane<->head layout and no LDS is needed per tile;
//  * fp8 tiles are widened to bf16 exactly (every E4M3FN value is a bf16
//    value) with the hardware convert; k_scale folds into the score scale,
//    v_scale into the output.
// Lane layout: lane = n + 16 g (n = lane & 15, g = lane >> 4).
//   QK:  A = K rows [token n][dims 32g+8kk .. +8], B = Q^T [head n][same dims],
//        D[token 4g+i][head n] in register i.
//   PV:  A = V^T [dim 8n+nb][tokens 4g .. 4g+3], B = P^T [tokens 4g+i][head n],
//        D[dim 8(4g+i)+nb][head n] in register i of accumulator nb.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hpc_decode.h"
#include "internal.h"

namespace hpcd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw (untyped) buffer, gfx9 family
constexpr uint32_t kSelLo = 0x05040100u;        // v_perm: low halves of (a, b) -> {a.lo, b.lo}
constexpr uint32_t kSelHi = 0x07060302u;        // v_perm: high halves -> {a.hi, b.hi}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                             kRsrcWord3);
}

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& x) {
    static_assert(sizeof(To) == sizeof(From), "size mismatch");
    return __builtin_bit_cast(To, x);
}

// two E4M3FN codes (16-bit half HI of x) -> two bf16, exact
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t x) {
    return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI));
}

__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t lo4, uint32_t hi4) {
    return u32x4{fp8x2_to_bf16x2<false>(lo4), fp8x2_to_bf16x2<true>(lo4),
                 fp8x2_to_bf16x2<false>(hi4), fp8x2_to_bf16x2<true>(hi4)};
}

// Per KV element type: what one wave loads from one tile, and how it becomes
// MFMA operands.  Offsets are relative to the (page, kv head) block.
template <int KV>
struct KvTile;

template <>
struct KvTile<HPC_KV_BF16> {
    static constexpr uint32_t kRow = kHeadDim * 2;   // bytes per token row
    u32x4 k[4];   // K row 16*wave+n, dims 32g .. 32g+31
    u32x4 v[4];   // V rows 16*wave+4g+i, dims 8n .. 8n+7
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                         int wave, int n, int g) {
        const uint32_t ko = (16 * wave + n) * kRow + 64 * g;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) k[kk] = __builtin_amdgcn_raw_buffer_load_b128(rk, ko + 16 * kk, 0, 0);
        const uint32_t vo = (16 * wave + 4 * g) * kRow + 16 * n;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo + i * kRow, 0, 0);
    }
    __device__ __forceinline__ bf16x8 k_op(int kk) const { return bitcast<bf16x8>(k[kk]); }
    __device__ __forceinline__ u32x4 v_row(int i) const { return v[i]; }
};

template <>
struct KvTile<HPC_KV_FP8_E4M3> {
    static constexpr uint32_t kRow = kHeadDim;       // bytes per token row
    u32x4 k[2];   // K row 16*wave+n, dims 32g .. 32g+31 (fp8)
    u32x2 v[4];   // V rows 16*wave+4g+i, dims 8n .. 8n+7 (fp8)
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                         int wave, int n, int g) {
        const uint32_t ko = (16 * wave + n) * kRow + 32 * g;
        k[0] = __builtin_amdgcn_raw_buffer_load_b128(rk, ko, 0, 0);
        k[1] = __builtin_amdgcn_raw_buffer_load_b128(rk, ko + 16, 0, 0);
        const uint32_t vo = (16 * wave + 4 * g) * kRow + 8 * n;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b64(rv, vo + i * kRow, 0, 0);
    }
    __device__ __forceinline__ bf16x8 k_op(int kk) const {
        const u32x4& src = k[kk >> 1];
        const int d = 2 * (kk & 1);
        return bitcast<bf16x8>(fp8x8_to_bf16x8(src[d], src[d + 1]));
    }
    __device__ __forceinline__ u32x4 v_row(int i) const { return fp8x8_to_bf16x8(v[i][0], v[i][1]); }
};

template <int KV>
struct TileSlot {
    KvTile<KV> data;
    int valid;    // valid token rows of the tile (0..64); 0 for a padding slot
};

// Scalars of the decode launch; the pointers are separate __restrict__
// kernel arguments so the plan words, block table and lengths are known not
// to be written by the kernel and load through the scalar unit.
struct DecodeScalars {
    int32_t num_kv_heads, group, max_pages_per_seq, num_pages;
    float qk_scale_log2, v_scale;
};

template <int KV, int PF>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const __bf16* __restrict__ q, const char* __restrict__ kcache, const char* __restrict__ vcache,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ worker_ptr, const int32_t* __restrict__ entries,
    __bf16* __restrict__ out, float* __restrict__ lse, float* __restrict__ o_part,
    float* __restrict__ lse_part, DecodeScalars a) {
    __shared__ float s_acc[kWaves][4][8][64];
    __shared__ float s_m[kWaves][64];
    __shared__ float s_l[kWaves][64];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int G = a.group;
    const int Hkv = a.num_kv_heads;
    const int Hq = G * Hkv;
    constexpr uint32_t kRow = KvTile<KV>::kRow;
    constexpr uint64_t kBlock = static_cast<uint64_t>(kPage) * kRow;   // one (page, head) block

    const int e_begin = worker_ptr[blockIdx.x];
    const int e_end = worker_ptr[blockIdx.x + 1];

    for (int e = e_begin; e < e_end; ++e) {
        const int u = entries[4 * e + 0];
        const int t0 = entries[4 * e + 1];
        const int t1 = entries[4 * e + 2];
        const int slot = entries[4 * e + 3];
        const int b = u / Hkv;
        const int h = u - b * Hkv;
        const int L = seq_lens[b];
        const int32_t* bt = block_table + static_cast<int64_t>(b) * a.max_pages_per_seq;
        const char* kbase = kcache;
        const char* vbase = vcache;

        // Q^T operand: head n, dims 32g + 8kk .. +8 (zero for padding heads)
        bf16x8 qop[4];
        if (n < G) {
            const u32x4* qp = reinterpret_cast<const u32x4*>(
                q + (static_cast<int64_t>(b) * Hq + h * G + n) * kHeadDim + 32 * g);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) qop[kk] = bitcast<bf16x8>(qp[kk]);
        } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) qop[kk] = bitcast<bf16x8>(u32x4{0u, 0u, 0u, 0u});
        }

        auto issue = [&](TileSlot<KV>& s, int t) {
            int valid = 0;
            const char* kp = kbase;
            const char* vp = vbase;
            if (t < t1) {
                const int page = bt[t];
                if (static_cast<unsigned>(page) < static_cast<unsigned>(a.num_pages)) {
                    const int rem = L - t * kPage;
                    valid = rem < 0 ? 0 : (rem > kPage ? kPage : rem);
                    const uint64_t off = (static_cast<uint64_t>(page) * Hkv + h) * kBlock;
                    kp += off;
                    vp += off;
                }
            }
            // the clamp above may be selected as a VALU op; the value is wave-uniform,
            // and the buffer descriptor must live in SGPRs
            valid = __builtin_amdgcn_readfirstlane(valid);
            s.valid = valid;
            s.data.load(make_rsrc(kp, valid * kRow), make_rsrc(vp, valid * kRow), wave, n, g);
        };

        float m = -INFINITY;   // running max (log2 domain), uniform over g
        float l = 0.f;         // this lane's share of the running sum
        f32x4 acc[8];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

        auto consume = [&](const TileSlot<KV>& s) {
            f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s.data.k_op(kk), qop[kk], sc, 0, 0, 0);
            const int r0 = 16 * wave + 4 * g;
            float mt = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc[i] = (r0 + i < s.valid) ? sc[i] * a.qk_scale_log2 : -INFINITY;
                mt = fmaxf(mt, sc[i]);
            }
            mt = fmaxf(mt, __shfl_xor(mt, 16));
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float m_new = fmaxf(m, mt);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m - m_use);
            float p[4];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = __builtin_amdgcn_exp2f(sc[i] - m_use);
                psum += p[i];
            }
            l = l * alpha + psum;
            m = m_new;
            const bf16x4 pop = bf16x4{static_cast<__bf16>(p[0]), static_cast<__bf16>(p[1]),
                                      static_cast<__bf16>(p[2]), static_cast<__bf16>(p[3])};
            u32x4 rows[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) rows[i] = s.data.v_row(i);
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int d = nb >> 1;
                const uint32_t sel = (nb & 1) ? kSelHi : kSelLo;
                const u32x2 vt = u32x2{__builtin_amdgcn_perm(rows[1][d], rows[0][d], sel),
                                       __builtin_amdgcn_perm(rows[3][d], rows[2][d], sel)};
                acc[nb] = acc[nb] * alpha;
                acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bitcast<bf16x4>(vt), pop, acc[nb], 0, 0, 0);
            }
        };

        TileSlot<KV> ring[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) issue(ring[j], t0 + j);
        for (int t = t0; t < t1; t += PF) {
#pragma unroll
            for (int j = 0; j < PF; ++j) {
                if (t + j < t1) {
                    consume(ring[j]);
                    issue(ring[j], t + j + PF);
                }
            }
        }

        // ---- merge the four waves' states for this entry ----
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        s_m[wave][lane] = m;
        s_l[wave][lane] = l;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) s_acc[wave][i][nb][lane] = acc[nb][i];
        __syncthreads();

        float ms[kWaves], wsum = 0.f, M = -INFINITY;
#pragma unroll
        for (int s = 0; s < kWaves; ++s) {
            ms[s] = s_m[s][lane];
            M = fmaxf(M, ms[s]);
        }
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float wt[kWaves];
#pragma unroll
        for (int s = 0; s < kWaves; ++s) {
            wt[s] = __builtin_amdgcn_exp2f(ms[s] - M_use);
            wsum += wt[s] * s_l[s][lane];
        }
        float o[8];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            float x = 0.f;
#pragma unroll
            for (int s = 0; s < kWaves; ++s) x += wt[s] * s_acc[s][wave][nb][lane];
            o[nb] = x;
        }
        if (n < G) {
            const float inv = (wsum > 0.f) ? a.v_scale / wsum : 0.f;
            const float lse_val = (wsum > 0.f) ? (M + __log2f(wsum)) * kLn2 : -INFINITY;
            const int hq = h * G + n;
            const int dim0 = 32 * g + 8 * wave;   // this wave merges register i = wave
            if (slot < 0) {
                bf16x8 ov;
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) ov[nb] = static_cast<__bf16>(o[nb] * inv);
                *reinterpret_cast<bf16x8*>(out +
                                           (static_cast<int64_t>(b) * Hq + hq) * kHeadDim + dim0) = ov;
                if (wave == 0 && g == 0) lse[static_cast<int64_t>(b) * Hq + hq] = lse_val;
            } else {
                float* dst = o_part + (static_cast<int64_t>(slot) * G + n) * kHeadDim + dim0;
                *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
                *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
                if (wave == 0 && g == 0) lse_part[static_cast<int64_t>(slot) * G + n] = lse_val;
            }
        }
        __syncthreads();
    }
}

// Merge of split units: one workgroup per (merge record, query head of the
// group), 1024 threads = 32 partial lanes x 32 dim quads.  Lane pl folds the
// partials i = pl, pl + 32, ... into a running (max, weighted sum, weight)
// triple, issuing up to eight partials' loads before using any of them; the
// 32 triples then meet in LDS and are merged once more by log-sum-exp.
constexpr int kMergeLanes = kCombineThreads / 32;
constexpr int kMergeUnroll = 8;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
    __shared__ f32x4 s_acc[kMergeLanes][32];
    __shared__ float s_m[kMergeLanes];
    __shared__ float s_w[kMergeLanes];

    const int G = a.group;
    const int c = blockIdx.x / G;
    const int n = blockIdx.x - c * G;
    const int u = a.combine[3 * c + 0];
    const int S = a.combine[3 * c + 1];
    const int base = a.combine[3 * c + 2];
    const int Hkv = a.num_kv_heads;
    const int b = u / Hkv;
    const int h = u - b * Hkv;
    const int64_t row = static_cast<int64_t>(b) * (G * Hkv) + h * G + n;
    const int t = threadIdx.x;
    const int dq = t & 31;
    const int pl = t >> 5;
    __bf16* out = static_cast<__bf16*>(a.out) + row * kHeadDim;

    if (S == 0) {   // empty sequence: out = 0, lse = -inf
        if (pl == 0) *reinterpret_cast<u32x2*>(out + 4 * dq) = u32x2{0u, 0u};
        if (t == 0) a.lse[row] = -INFINITY;
        return;
    }

    float m = -INFINITY;          // running max of the folded lse values (log2 units)
    float w = 0.f;                // running sum of 2^(lse - m)
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i0 = pl; i0 < S; i0 += kMergeLanes * kMergeUnroll) {
        float l[kMergeUnroll];
        f32x4 o[kMergeUnroll];
#pragma unroll
        for (int k = 0; k < kMergeUnroll; ++k) {
            const int i = i0 + k * kMergeLanes;
            const int64_t p = static_cast<int64_t>(base + (i < S ? i : 0)) * G + n;
            l[k] = (i < S) ? a.lse_part[p] * kLog2e : -INFINITY;
            o[k] = *reinterpret_cast<const f32x4*>(a.o_part + p * kHeadDim + 4 * dq);
        }
        float mk = m;
#pragma unroll
        for (int k = 0; k < kMergeUnroll; ++k) mk = fmaxf(mk, l[k]);
        const float m_use = (mk == -INFINITY) ? 0.f : mk;
        const float f = __builtin_amdgcn_exp2f(m - m_use);
        acc *= f;
        w *= f;
#pragma unroll
        for (int k = 0; k < kMergeUnroll; ++k) {
            const float e = __builtin_amdgcn_exp2f(l[k] - m_use);
            acc += e * o[k];
            w += e;
        }
        m = mk;
    }
    s_acc[pl][dq] = acc;
    if (dq == 0) {
        s_m[pl] = m;
        s_w[pl] = w;
    }
    __syncthreads();
    if (pl == 0) {
        float M = -INFINITY;
#pragma unroll
        for (int j = 0; j < kMergeLanes; ++j) M = fmaxf(M, s_m[j]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
        float ws = 0.f;
#pragma unroll 8
        for (int j = 0; j < kMergeLanes; ++j) {
            const float e = __builtin_amdgcn_exp2f(s_m[j] - M_use);
            r += e * s_acc[j][dq];
            ws += e * s_w[j];
        }
        const float inv = ws > 0.f ? 1.f / ws : 0.f;
        const bf16x4 ov = bf16x4{static_cast<__bf16>(r[0] * inv), static_cast<__bf16>(r[1] * inv),
                                 static_cast<__bf16>(r[2] * inv), static_cast<__bf16>(r[3] * inv)};
        *reinterpret_cast<bf16x4*>(out + 4 * dq) = ov;
        if (dq == 0) a.lse[row] = ws > 0.f ? (M + __log2f(ws)) * kLn2 : -INFINITY;
    }
}

// tiles in flight per wave (register ring depth)
#ifndef HPC_DECODE_PREFETCH_BF16
#define HPC_DECODE_PREFETCH_BF16 4
#endif
#ifndef HPC_DECODE_PREFETCH_FP8
#define HPC_DECODE_PREFETCH_FP8 4
#endif
constexpr int kPrefetchBf16 = HPC_DECODE_PREFETCH_BF16;
constexpr int kPrefetchFp8 = HPC_DECODE_PREFETCH_FP8;

}  // namespace

int launch_decode(const DecodeArgs& a, int kv_dtype, int n_workers, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const DecodeScalars sc{a.num_kv_heads, a.group, a.max_pages_per_seq, a.num_pages, a.qk_scale_log2, a.v_scale};
    const __bf16* q = static_cast<const __bf16*>(a.q);
    const char* k = static_cast<const char*>(a.k);
    const char* v = static_cast<const char*>(a.v);
    __bf16* out = static_cast<__bf16*>(a.out);
    if (kv_dtype == HPC_KV_BF16)
        hipLaunchKernelGGL((decode_kernel<HPC_KV_BF16, kPrefetchBf16>), dim3(n_workers), dim3(kDecodeThreads), 0, s,
                           q, k, v, a.block_table, a.seq_lens, a.worker_ptr, a.entries, out, a.lse, a.o_part,
                           a.lse_part, sc);
    else
        hipLaunchKernelGGL((decode_kernel<HPC_KV_FP8_E4M3, kPrefetchFp8>), dim3(n_workers), dim3(kDecodeThreads), 0, s,
                           q, k, v, a.block_table, a.seq_lens, a.worker_ptr, a.entries, out, a.lse, a.o_part,
                           a.lse_part, sc);
    return static_cast<int>(hipGetLastError());
}

int launch_combine(const CombineArgs& a, int n_combine, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(combine_kernel, dim3(n_combine * a.group), dim3(kCombineThreads), 0, s, a);
    return static_cast<int>(hipGetLastError());
}

}  // namespace hpcd
