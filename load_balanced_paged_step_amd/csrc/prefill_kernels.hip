// Causal prefill / extend attention over the paged KV cache on gfx950.
//
// "vLLM x HPC-Ops ...", §Attention Across Prefill, Extend and Decode Shapes
// measures the attention backend on prefill ("q512") and extend shapes as
// well as decode; the pages give no kernel design for them.  What is
// computed (the plain reading): sequence b holds L_b cached tokens whose last
// n_b are this step's new tokens; new token j, at position
// p = L_b - n_b + j, is a query over the cached tokens t <= p.
//
// Work: one workgroup (4 waves, or two groups of 4 on small grids) per work
// entry of a host-made list: a unit (sequence b, KV head h, block of 16
// consecutive queries) whole, or a contiguous share of a long unit's KV
// tiles, which writes a normalised fp32 partial and log-sum-exp that
// prefill_merge_kernel folds afterwards.  Entries run longest first (cost =
// the 64-token KV tiles they cover), so short ones fill in behind.
//  * Each wave owns heads w, w + 4, w + 8, w + 12 (< G) of the KV head's
//    query group: per head a 16-query row block, whose Q stays in registers.
//  * Per 64-token tile, K and V (one page of head h) are loaded by all 256
//    threads with buffer loads whose range ends at the sequence's last token
//    (rows past it read as zeros: a poisoned tail cannot reach the sums),
//    written to LDS (fp8 widened to bf16 exactly) and read by all four
//    waves: K row-major with rows padded by 32 bytes, V transposed (each
//    thread transposes a 4-token x 8-dim block on the way in) in the order
//    the P V operand reads it.  The next tile's loads are in flight while
//    the current tile is computed.
//  * S^T = K Q^T on MFMA 16x16x32 bf16 (16 KV tokens x 16 queries), exp2
//    domain online softmax per query, P V on MFMA 16x16x32 bf16 as
//    O^T = V^T P^T with P taken straight from the score registers.
//  * The causal mask is applied on the tiles that reach past the block's
//    first query position; tokens > p score -inf.
// Lane layout (lane = n + 16 g): QK: A = K [token n][dims 32 kk + 8 g ..],
// B = Q^T [query n][same dims], D[token 4 g + i][query n] in register i.
// PV (32-token chunk c): A = V^T [dim 8 n + nb][tokens 4 g .. 4 g + 3 of
// 16-token blocks 2c and 2c + 1], B = P^T, D[dim 8 (4 g + i) + nb][query n]
// in register i of accumulator nb.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdint>
#include <type_traits>

#include "internal.h"

namespace hpcd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQBlock = 16;                       // queries per unit
constexpr int kLdsRow = kHeadDim * 2 + 32;        // bytes per LDS row: 256 + 32 pad (half the bank
                                                  // conflicts of a 16-byte pad, measured)
constexpr uint32_t kRsrcWord3 = 0x00020000u;      // raw (untyped) buffer
constexpr uint32_t kSelLo = 0x05040100u;          // v_perm: {b.lo, a.lo}
constexpr uint32_t kSelHi = 0x07060302u;          // v_perm: {b.hi, a.hi}
constexpr float kLn2 = 0.69314718055994531f;

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& x) {
    static_assert(sizeof(To) == sizeof(From), "size mismatch");
    return __builtin_bit_cast(To, x);
}

// max of x over lanes l and l ^ 16 (l ^ 32): the lane-swap instructions put
// each lane's value and its partner's in the two results, in VALU, where a
// shuffle would take a round trip through the LDS unit
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(bitcast<uint32_t>(x), bitcast<uint32_t>(x), false, false);
    return fmaxf(bitcast<float>(r[0]), bitcast<float>(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(bitcast<uint32_t>(x), bitcast<uint32_t>(x), false, false);
    return fmaxf(bitcast<float>(r[0]), bitcast<float>(r[1]));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

// four E4M3FN codes -> four bf16 (exact: every E4M3FN value is a bf16 value)
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t x) {
    return u32x2{bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false)),
                 bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true))};
}

// two fp32 -> two bf16 (nearest-even) in one word, a in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(a))) |
           (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(b))) << 16);
}

// V^T in LDS: dim d's 64 tokens take 128 bytes, two dims per 256-byte line
// (line d >> 1, half d & 1).  Within each 32-token chunk cc the tokens are
// kept in the order the P V operand takes them: for g = 0..3, tokens
// 4g .. 4g+3 of 16-token block 2cc, then the same of block 2cc + 1, so that
// lane (n, g) reads its operand for dim 8n + nb as one 16-byte run at byte
// 64 cc + 16 g of the dim.  The sixteen 16-byte chunks of a line are XOR-
// swizzled by (line >> 2) & 15: the 16 lanes of one read (n = 0..15, lines
// 4n + (nb >> 1)) then hit 16 distinct chunk positions, i.e. distinct banks.
__device__ __forceinline__ int vt_offset(int d, int byte) {   // byte of the dim's 128, 8-aligned
    const int line = d >> 1;
    const int q = ((d & 1) << 3) | (byte >> 4);
    return line * 256 + ((q ^ ((line >> 2) & 15)) << 4) + (byte & 15);
}

// One 64-token tile of K and V in flight, staged by the 64 NW threads of a
// group.  K: 16-byte chunks of the row-major tile (16 KiB bf16 = 16 per 4
// threads, 8 KiB fp8 = 8).  V: thread (j, m) = (tid >> 4 + 4 NW p, tid & 15)
// holds tokens 4j .. 4j+3, dims 8m .. 8m+7 (16 bytes per token in bf16, 8 in
// fp8), for each of its 4 / NW passes p, which it transposes into V^T on the
// way to LDS.
template <bool FP8, int NW>
struct TileRegs {
    static constexpr int kThr = 64 * NW;
    static constexpr int kRep = 4 / NW;
    static constexpr int kKLoads = (FP8 ? 2 : 4) * kRep;
    typedef typename std::conditional<FP8, u32x2, u32x4>::type VRow;
    u32x4 k[kKLoads];
    VRow v[4 * kRep];

    // rows [0, valid) of page `page`, KV head h; everything else reads as 0
    __device__ __forceinline__ void load(const PrefillArgs& a, int page, int h, int valid, int tid) {
        const int64_t elem = FP8 ? 1 : 2;
        const int64_t head_bytes = int64_t(kPage) * kHeadDim * elem;
        const bool ok = page >= 0 && page < a.num_pages;
        const int64_t off = ok ? (int64_t(page) * a.num_kv_heads + h) * head_bytes : 0;
        const uint32_t bytes = ok ? static_cast<uint32_t>(valid * kHeadDim * elem) : 0u;
        const auto rk = make_rsrc(static_cast<const char*>(a.k) + off, bytes);
        const auto rv = make_rsrc(static_cast<const char*>(a.v) + off, bytes);
#pragma unroll
        for (int i = 0; i < kKLoads; ++i) {
            const int c = tid + kThr * i;              // 16-byte chunk of the tile, row-major
            k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, c * 16, 0, 0);
        }
        const int m = tid & 15;
        constexpr int row = kHeadDim * (FP8 ? 1 : 2);
#pragma unroll
        for (int pp = 0; pp < kRep; ++pp) {
            const int j = (tid >> 4) + (kThr >> 4) * pp;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (FP8)
                    v[4 * pp + i] = __builtin_amdgcn_raw_buffer_load_b64(rv, (4 * j + i) * row + 8 * m, 0, 0);
                else
                    v[4 * pp + i] = __builtin_amdgcn_raw_buffer_load_b128(rv, (4 * j + i) * row + 16 * m, 0, 0);
            }
        }
    }

    __device__ __forceinline__ void store(char* lds_k, char* lds_v, int tid) const {
#pragma unroll
        for (int i = 0; i < kKLoads; ++i) {
            const int c = tid + kThr * i;
            if constexpr (FP8) {
                const int row = c >> 3, col = (c & 7) * 32;      // 16 codes -> 32 bytes of bf16
                char* pk = lds_k + row * kLdsRow + col;
                const u32x2 k0 = fp8x4_to_bf16x4(k[i][0]), k1 = fp8x4_to_bf16x4(k[i][1]);
                const u32x2 k2 = fp8x4_to_bf16x4(k[i][2]), k3 = fp8x4_to_bf16x4(k[i][3]);
                *reinterpret_cast<u32x4*>(pk) = u32x4{k0[0], k0[1], k1[0], k1[1]};
                *reinterpret_cast<u32x4*>(pk + 16) = u32x4{k2[0], k2[1], k3[0], k3[1]};
            } else {
                const int row = c >> 4, col = (c & 15) * 16;
                *reinterpret_cast<u32x4*>(lds_k + row * kLdsRow + col) = k[i];
            }
        }
        // V: token rows of 8 dims (bf16 pairs per word) -> for each dim, its 4 tokens
        const int m = tid & 15;
#pragma unroll
        for (int pp = 0; pp < kRep; ++pp) {
            u32x4 vb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (FP8) {
                    const u32x2 lo = fp8x4_to_bf16x4(v[4 * pp + i][0]), hi = fp8x4_to_bf16x4(v[4 * pp + i][1]);
                    vb[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                } else {
                    vb[i] = v[4 * pp + i];
                }
            }
            const int j = (tid >> 4) + (kThr >> 4) * pp;
            const int tb = (j >> 3) * 64 + (j & 3) * 16 + ((j >> 2) & 1) * 8;   // byte of token 4j in a dim's 128
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const u32x2 lo = u32x2{__builtin_amdgcn_perm(vb[1][p], vb[0][p], kSelLo),
                                       __builtin_amdgcn_perm(vb[3][p], vb[2][p], kSelLo)};
                const u32x2 hi = u32x2{__builtin_amdgcn_perm(vb[1][p], vb[0][p], kSelHi),
                                       __builtin_amdgcn_perm(vb[3][p], vb[2][p], kSelHi)};
                *reinterpret_cast<u32x2*>(lds_v + vt_offset(8 * m + 2 * p, tb)) = lo;
                *reinterpret_cast<u32x2*>(lds_v + vt_offset(8 * m + 2 * p + 1, tb)) = hi;
            }
        }
    }
};

// NG groups of 4 waves share a unit: group gg takes tiles gg, gg + NG, ...
// with its own LDS tile, and at the end the groups' softmax states are
// merged in LDS.  Two waves per SIMD are the point either way (two
// workgroups per CU with NG = 1, two groups with NG = 2), so the register
// budget is held to 2 waves per SIMD where the accumulators allow (HPW <= 2).
template <bool FP8, int HPW, int NG, int NW>
__global__ void __launch_bounds__(64 * NW * NG) __attribute__((amdgpu_waves_per_eu(2, 4)))
prefill_kernel(PrefillArgs a) {
    static_assert(HPW <= 2 && (NW == 2 || NW == 4), "two waves per SIMD: at most two heads per wave");
    constexpr int kThreads = 64 * NW;   // threads of one group
    // per group one tile buffer (K rows, then V^T), or with two groups two
    // buffers used by alternate rounds (measured: one barrier per round pays
    // there; with one group per workgroup, two barriers around a single
    // buffer run 4-7% faster on the extend batches)
    constexpr int kKBytes = kPage * kLdsRow;
    constexpr int kBufBytes = kKBytes + kHeadDim * kPage * 2;
    constexpr int kBufs = NG == 2 ? 2 : 1;
    __shared__ __attribute__((aligned(16))) char lds[NG * kBufs * kBufBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int gg = wave_all / NW;     // group of this wave
    const int wave = wave_all % NW;   // wave within the group: owns heads hbase + wave + NW r
    const int tid_g = tid & (kThreads - 1);
    const int n = lane & 15;          // query column / K row / V dim group
    const int g = lane >> 4;          // lane group
    char* const grp = lds + gg * kBufs * kBufBytes;
    char* lds_k = grp;              // the buffers of the round being computed
    char* lds_v = grp + kKBytes;

    // the entry: tiles [t0, t1) of unit (b, qb, h), written to partial slot `slot` (-1: out / lse)
    const int32_t* w = a.work + 8 * static_cast<int64_t>(blockIdx.x);
    const int b = __builtin_amdgcn_readfirstlane(w[0]);
    const int qb = __builtin_amdgcn_readfirstlane(w[1]);
    const int h = __builtin_amdgcn_readfirstlane(w[2]);
    const int e_t0 = __builtin_amdgcn_readfirstlane(w[4]);
    const int e_t1 = __builtin_amdgcn_readfirstlane(w[5]);
    const int slot = __builtin_amdgcn_readfirstlane(w[6]);
    if (b < 0 || b >= a.batch || h < 0 || h >= a.num_kv_heads || qb < 0) return;
    const int r0 = a.q_start[b];
    const int nq_seq = a.q_start[b + 1] - r0;
    if (qb * kQBlock >= nq_seq) return;
    int L = a.seq_lens[b];
    L = L < 0 ? 0 : (L > a.max_pages_per_seq * kPage ? a.max_pages_per_seq * kPage : L);
    const int q0 = qb * kQBlock;                                  // first query of the block in the chunk
    const int nq = nq_seq - q0 < kQBlock ? nq_seq - q0 : kQBlock;   // queries in the block
    const int pos0 = L - nq_seq + q0;                             // position of the block's first query
    const int last = pos0 + nq - 1;                               // position of its last query
    const int unit_tiles = last < 0 ? 0 : last / kPage + 1;   // tiles the block's last query sees
    const int t_lo = e_t0 < 0 ? 0 : (e_t0 > unit_tiles ? unit_tiles : e_t0);
    const int t_hi = e_t1 < t_lo ? t_lo : (e_t1 > unit_tiles ? unit_tiles : e_t1);
    const int G = a.group;
    if (slot >= a.n_partials) return;       // not a slot of this plan: write nothing

    // this workgroup's heads of the query group: hbase .. hbase + NW HPW - 1
    // (grid y splits a larger group over several workgroups)
    const int hbase = static_cast<int>(blockIdx.y) * (NW * HPW);
    // Q of this wave's heads: row block r holds head hg = hbase + wave + NW r
    bf16x8 qop[HPW][4];
#pragma unroll
    for (int r = 0; r < HPW; ++r) {
        const int hg = hbase + wave + NW * r;
        const int64_t row_stride = int64_t(a.num_q_heads) * kHeadDim * 2;
        const char* base = static_cast<const char*>(a.q) + (int64_t(r0 + q0) * a.num_q_heads + h * G + hg) * kHeadDim * 2;
        const uint32_t bytes = (hg < G && nq > 0) ? static_cast<uint32_t>((nq - 1) * row_stride + kHeadDim * 2) : 0u;
        const auto rq = make_rsrc(base, bytes);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qop[r][kk] = bitcast<bf16x8>(__builtin_amdgcn_raw_buffer_load_b128(
                rq, static_cast<int>(n * row_stride + (32 * kk + 8 * g) * 2), 0, 0));
    }

    f32x4 acc[HPW][8];
    float m[HPW], l[HPW];
#pragma unroll
    for (int r = 0; r < HPW; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[r][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int32_t* bt = a.block_table + int64_t(b) * a.max_pages_per_seq;
    auto rows_in = [&](int t) { const int r = L - t * kPage; return r < kPage ? r : kPage; };

    // one tile, already in LDS: scores, online softmax, P V
    auto compute = [&](int t) {
        // S^T blocks: 4 x 16 KV tokens against each row block's 16 queries
        f32x4 sc[HPW][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int r = 0; r < HPW; ++r) sc[r][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 kop = *reinterpret_cast<const bf16x8*>(lds_k + (16 * kb + n) * kLdsRow + (32 * kk + 8 * g) * 2);
#pragma unroll
                for (int r = 0; r < HPW; ++r)
                    sc[r][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[r][kk], sc[r][kb], 0, 0, 0);
            }
        }

        // online softmax per query column n, exp2 domain.  The running max m
        // is kept on raw scores (c = qk_scale_log2 > 0 keeps their order), and
        // p = 2^(s c - m c) is one FMA per score.  Only tiles that reach past
        // the block's first query carry masked tokens.
        const int tok0 = t * kPage;
        const bool masked_tile = tok0 + kPage - 1 > pos0;
        const int qpos = pos0 + n;
        const float c = a.qk_scale_log2;
        if (masked_tile) {
#pragma unroll
            for (int r = 0; r < HPW; ++r)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (tok0 + 16 * kb + 4 * g + i > qpos) sc[r][kb][i] = -INFINITY;
        }
        // P^T operands of 32-token chunks: lane group g's 8 k-slots are tokens
        // 4g .. 4g+3 of 16-token block 2c and of block 2c + 1
        bf16x8 pop[HPW][2];
#pragma unroll
        for (int r = 0; r < HPW; ++r) {
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sc[r][kb][i]);
            mt = max_xor32(max_xor16(mt));
            const float m_new = fmaxf(m[r], mt);
            const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;   // the new max, scaled
            const float alpha = __builtin_amdgcn_exp2f(m[r] * c - mc);
            m[r] = m_new;
            float p[4][4], ps[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) p[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r][kb][i], c, -mc));
                ps[kb] = (p[kb][0] + p[kb][1]) + (p[kb][2] + p[kb][3]);
            }
            // a pairwise sum: depth 4 where a running sum would chain 16 adds
            const float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
                pop[r][cc] = bf16x8{static_cast<__bf16>(p[2 * cc][0]), static_cast<__bf16>(p[2 * cc][1]),
                                    static_cast<__bf16>(p[2 * cc][2]), static_cast<__bf16>(p[2 * cc][3]),
                                    static_cast<__bf16>(p[2 * cc + 1][0]), static_cast<__bf16>(p[2 * cc + 1][1]),
                                    static_cast<__bf16>(p[2 * cc + 1][2]), static_cast<__bf16>(p[2 * cc + 1][3])};
            l[r] = l[r] * alpha + psum;
            // the accumulators change only where a running max grew; skip the
            // rescale when it grew nowhere in the wave
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) acc[r][nb] = acc[r][nb] * alpha;
            }
        }

        // O^T += V^T P^T on 32-token chunks (MFMA 16x16x32): the V^T operand of
        // lane (n, g) is dim 8n + nb over the same 8 tokens as its P slots,
        // one 16-byte read of the transposed tile
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const u32x4 vt = *reinterpret_cast<const u32x4*>(lds_v + vt_offset(8 * n + nb, 64 * cc + 16 * g));
#pragma unroll
                for (int r = 0; r < HPW; ++r)
                    acc[r][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(vt), pop[r][cc], acc[r][nb],
                                                                         0, 0, 0);
            }
        }
    };

    // tile t goes global -> registers -> LDS; one tile in flight in registers
    // per group while the group computes the one before.  Every wave meets
    // every barrier; a group past the unit's last tile only waits.
    {
        TileRegs<FP8, NW> rg;
        const int rounds = (t_hi - t_lo + NG - 1) / NG;
        if constexpr (kBufs == 1) {
            if (t_lo + gg < t_hi) rg.load(a, bt[t_lo + gg], h, rows_in(t_lo + gg), tid_g);
            for (int i = 0; i < rounds; ++i) {
                const int t = t_lo + NG * i + gg;
                __syncthreads();              // every wave is done with the previous tile
                rg.store(lds_k, lds_v, tid_g);
                __syncthreads();              // the tile is in LDS
                if (t + NG < t_hi) rg.load(a, bt[t + NG], h, rows_in(t + NG), tid_g);
                compute(t);
            }
        } else {
            // round i computes its tile from buffer i & 1, then stores the
            // next tile into the other buffer and loads the one after it:
            // one barrier per round
            if (t_lo + gg < t_hi) {
                rg.load(a, bt[t_lo + gg], h, rows_in(t_lo + gg), tid_g);
                rg.store(grp, grp + kKBytes, tid_g);
            }
            if (t_lo + NG + gg < t_hi) rg.load(a, bt[t_lo + NG + gg], h, rows_in(t_lo + NG + gg), tid_g);
            for (int i = 0; i < rounds; ++i) {
                const int t = t_lo + NG * i + gg;
                // round i's tile is in its buffer, and every wave is done with
                // the other buffer (round i - 1)
                __syncthreads();
                lds_k = grp + (i & 1) * kBufBytes;
                lds_v = lds_k + kKBytes;
                if (t < t_hi) compute(t);
                if (t + NG < t_hi) {
                    char* nxt = grp + ((i + 1) & 1) * kBufBytes;
                    rg.store(nxt, nxt + kKBytes, tid_g);
                    if (t + 2 * NG < t_hi) rg.load(a, bt[t + 2 * NG], h, rows_in(t + 2 * NG), tid_g);
                }
            }
        }
    }
    if constexpr (NG == 2) {
        // group 1 leaves its state in LDS (over the tile buffers, exactly
        // HPW * 34 values per lane), group 0 merges it by log-sum-exp
        float* st = reinterpret_cast<float*>(lds);
        const int sl = wave * 64 + lane;   // this lane's column of the state
        __syncthreads();
        if (gg == 1) {
#pragma unroll
            for (int r = 0; r < HPW; ++r) {
#pragma unroll
                for (int nb = 0; nb < 8; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) st[((r * 8 + nb) * 4 + i) * kThreads + sl] = acc[r][nb][i];
                st[(HPW * 32 + r) * kThreads + sl] = m[r];
                st[(HPW * 33 + r) * kThreads + sl] = l[r];
            }
        }
        __syncthreads();
        if (gg == 1) return;
#pragma unroll
        for (int r = 0; r < HPW; ++r) {
            const float m1 = st[(HPW * 32 + r) * kThreads + sl];
            const float l1 = st[(HPW * 33 + r) * kThreads + sl];
            const float mx = fmaxf(m[r], m1);                       // raw scores, as in the tile loop
            const float mu = (mx == -INFINITY) ? 0.f : mx * a.qk_scale_log2;
            const float f0 = __builtin_amdgcn_exp2f(m[r] * a.qk_scale_log2 - mu);
            const float f1 = __builtin_amdgcn_exp2f(m1 * a.qk_scale_log2 - mu);
            m[r] = mx;
            l[r] = l[r] * f0 + l1 * f1;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[r][nb][i] = acc[r][nb][i] * f0 + st[((r * 8 + nb) * 4 + i) * kThreads + sl] * f1;
        }
    }

    // epilogue: out = acc / l, lse = (m + log2 l) ln 2; a query with no
    // visible token gets 0 and -inf
#pragma unroll
    for (int r = 0; r < HPW; ++r) {
        const int hg = hbase + wave + NW * r;
        if (hg >= G) break;
        float lt = l[r];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        if (n >= nq) continue;
        const float inv = lt > 0.f ? a.v_scale / lt : 0.f;
        const float lse_v = lt > 0.f ? (m[r] * a.qk_scale_log2 + __log2f(lt)) * kLn2 : -INFINITY;
        if (slot >= 0) {
            // a share of a cut unit: its normalised fp32 output and log-sum-exp
            const int64_t prow = (int64_t(slot) * kQBlock + n) * G + hg;
            float* po = a.o_part + prow * kHeadDim;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *reinterpret_cast<f32x4*>(po + 32 * g + 8 * i) =
                    f32x4{acc[r][0][i] * inv, acc[r][1][i] * inv, acc[r][2][i] * inv, acc[r][3][i] * inv};
                *reinterpret_cast<f32x4*>(po + 32 * g + 8 * i + 4) =
                    f32x4{acc[r][4][i] * inv, acc[r][5][i] * inv, acc[r][6][i] * inv, acc[r][7][i] * inv};
            }
            if (g == 0) a.lse_part[prow] = lse_v;
            continue;
        }
        const int64_t row = int64_t(r0 + q0 + n) * a.num_q_heads + h * G + hg;
        char* o = static_cast<char*>(a.out) + row * kHeadDim * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 pk = u32x4{pack_bf16x2(acc[r][0][i] * inv, acc[r][1][i] * inv),
                                   pack_bf16x2(acc[r][2][i] * inv, acc[r][3][i] * inv),
                                   pack_bf16x2(acc[r][4][i] * inv, acc[r][5][i] * inv),
                                   pack_bf16x2(acc[r][6][i] * inv, acc[r][7][i] * inv)};
            *reinterpret_cast<u32x4*>(o + (32 * g + 8 * i) * 2) = pk;
        }
        if (g == 0) a.lse[row] = lse_v;
    }
}

// Compute units of the current device (looked up once per device).
int device_cus() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

// Log-sum-exp merge of the shares of each cut unit: one workgroup per
// (merge record, query head of the group); thread (row, part) folds dims
// 8 part .. +8 of query row `row` over the unit's S partial slots.  Shares
// are read in chunks of kMergeChunk whose loads are all issued before any is
// used (one memory round trip per chunk), and chunks are folded with a
// running max.
constexpr int kMergeChunk = 16;

__global__ void __launch_bounds__(256) prefill_merge_kernel(PrefillArgs a) {
    const int G = a.group;
    const int rec_i = static_cast<int>(blockIdx.x) / G;
    const int hg = static_cast<int>(blockIdx.x) - rec_i * G;
    const int32_t* rec = a.merge + 8 * static_cast<int64_t>(rec_i);
    const int b = rec[0], qb = rec[1], h = rec[2], S = rec[3], base = rec[4];
    if (b < 0 || b >= a.batch || h < 0 || h >= a.num_kv_heads || qb < 0 || S < 1 || base < 0 ||
        base > a.n_partials - S)
        return;
    const int r0 = a.q_start[b];
    const int q0 = qb * kQBlock;
    const int nq_seq = a.q_start[b + 1] - r0;
    const int nq = nq_seq - q0 < kQBlock ? nq_seq - q0 : kQBlock;
    const int row = threadIdx.x >> 4, part = threadIdx.x & 15;
    if (row >= nq) return;
    constexpr float kLog2e = 1.4426950408889634f;
    const int64_t stride = int64_t(kQBlock) * G;                     // one share's rows
    const int64_t prow0 = (int64_t(base) * kQBlock + row) * G + hg;  // this row in the first share
    const float* lp = a.lse_part + prow0;
    const float* op = a.o_part + prow0 * kHeadDim + 8 * part;
    float M = -INFINITY, wsum = 0.f;
    f32x4 o0 = f32x4{0.f, 0.f, 0.f, 0.f}, o1 = o0;
    for (int s0 = 0; s0 < S; s0 += kMergeChunk) {
        float l[kMergeChunk];
        f32x4 p0[kMergeChunk], p1[kMergeChunk];
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i) {
            if (s0 + i < S) {
                const f32x4* po = reinterpret_cast<const f32x4*>(op + (s0 + i) * stride * kHeadDim);
                l[i] = lp[(s0 + i) * stride];
                p0[i] = po[0];
                p1[i] = po[1];
            } else {
                l[i] = -INFINITY;
                p0[i] = p1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        float mc = M;
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i) mc = fmaxf(mc, l[i]);
        if (mc == -INFINITY) continue;                      // no share of this chunk sees a token yet
        const float alpha = __builtin_amdgcn_exp2f((M - mc) * kLog2e);   // 0 while M = -inf
        o0 *= alpha;
        o1 *= alpha;
        wsum *= alpha;
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i) {
            const float wt = __builtin_amdgcn_exp2f((l[i] - mc) * kLog2e);
            o0 += wt * p0[i];
            o1 += wt * p1[i];
            wsum += wt;
        }
        M = mc;
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const int64_t orow = int64_t(r0 + q0 + row) * a.num_q_heads + h * G + hg;
    *reinterpret_cast<u32x4*>(static_cast<char*>(a.out) + (orow * kHeadDim + 8 * part) * 2) =
        u32x4{pack_bf16x2(o0[0] * inv, o0[1] * inv), pack_bf16x2(o0[2] * inv, o0[3] * inv),
              pack_bf16x2(o1[0] * inv, o1[1] * inv), pack_bf16x2(o1[2] * inv, o1[3] * inv)};
    if (part == 0) a.lse[orow] = wsum > 0.f ? M + __logf(wsum) : -INFINITY;
}

// A workgroup takes NW HPW heads of an entry's query group (NW waves of HPW
// heads); a larger group is split over grid y, so every wave keeps at most
// two heads and two waves share a SIMD (measured on extends: 4 heads per wave
// at one wave per SIMD ran at 650 TFLOP/s where two heads per wave ran at
// 930).  Groups of at most 4 heads take 2 waves per workgroup, so no wave
// idles and four workgroups share a CU.  With fewer than two waves per SIMD
// the grid cannot hide one entry's tile chain behind other workgroups, so two
// groups of NW waves split each entry's tiles (NG = 2); otherwise a
// workgroup is one group.
template <bool FP8, int HPW, int NW>
void launch_cfg(const PrefillArgs& a, int n_entries, hipStream_t s) {
    const int ny = (a.group + NW * HPW - 1) / (NW * HPW);
    if (static_cast<int64_t>(n_entries) * ny * NW < 8 * static_cast<int64_t>(device_cus()))
        hipLaunchKernelGGL((prefill_kernel<FP8, HPW, 2, NW>), dim3(n_entries, ny), dim3(2 * 64 * NW), 0, s, a);
    else
        hipLaunchKernelGGL((prefill_kernel<FP8, HPW, 1, NW>), dim3(n_entries, ny), dim3(64 * NW), 0, s, a);
}

template <bool FP8>
int launch_fp8(const PrefillArgs& a, int n_entries, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.group <= 2)
        launch_cfg<FP8, 1, 2>(a, n_entries, s);
    else if (a.group <= 4)
        launch_cfg<FP8, 2, 2>(a, n_entries, s);
    else
        launch_cfg<FP8, 2, 4>(a, n_entries, s);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_prefill(const PrefillArgs& a, int n_entries, int n_merge, bool kv_fp8, void* stream) {
    if (n_entries > 0) {
        const int e = kv_fp8 ? launch_fp8<true>(a, n_entries, stream) : launch_fp8<false>(a, n_entries, stream);
        if (e) return e;
    }
    if (n_merge > 0) {
        hipLaunchKernelGGL(prefill_merge_kernel, dim3(n_merge * a.group), dim3(256), 0,
                           static_cast<hipStream_t>(stream), a);
        return static_cast<int>(hipGetLastError());
    }
    return 0;
}

}  // namespace hpcd
