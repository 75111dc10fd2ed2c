// Persistent paged GQA decode attention, the log-sum-exp merge, and the
// on-device form of the per-step schedule, for CDNA4 (gfx950).
//
// Method: "vLLM x HPC-Ops: High-Performance Attention and MoE Backends from
// Tencent Hunyuan", §Attention Backend: Dynamic Load-Balanced Scheduling —
// 64-token KV tiles spread evenly over a persistent grid, recomputed every
// decode step; a sequence split over several workers is merged afterwards
// (log-sum-exp, the reading used here; the pages do not describe the merge).
// Head shape (8 query heads per KV head, head dim 128): "vLLM und Tencent
// Hunyuan streamen zwei HPC-Backends ...", §Zwei neue HPC-Backends im
// vLLM-Ökosystem.  The pages' kernels target Hopper; none of their design is
// assumed here.
//
// Decode kernel (one workgroup = one worker, 4 waves):
//  * the worker's tiles come either from the host plan's entries or from the
//    schedule derived on the device from the lengths (device_schedule.h);
//    both walk the same tile sequence;
//  * every wave owns a fixed 16-token slice (rows 16*wave .. +15) of every
//    64-token tile and keeps its own online-softmax state; at the end of an
//    entry each wave leaves its state in one of two LDS slots without
//    waiting, and once both slots are taken (or the range ends) the four
//    states of each pending entry meet and one result per entry is written;
//  * a ring of PF = 2 slots is kept in flight across entry boundaries: each
//    slot holds the K/V rows of one tile (bf16) or of two consecutive tiles
//    of one entry (fp8, so a slot holds as many bytes either way), and for
//    an entry's first tile also that entry's Q, so changing sequence never
//    drains the load pipeline; the loop leaves only at the end of a full
//    ring turn, and a slot that ends an entry is refilled before the entry
//    is flushed;
//  * with the device schedule, each unit's merge record is written in the
//    prologue by the worker holding the unit's first tile;
//  * K, V and Q are read with buffer loads whose range is the valid part of
//    the page (rows past a sequence's end, padding heads and ring slots past
//    the worker's last tile read as zeros without touching memory); K/V use
//    the nontemporal cache policy, since every byte is read exactly once;
//  * S = K Q^T on MFMA 16x16x32 bf16 (16 tokens x up to 16 heads, padded);
//    P V on MFMA 16x16x16 bf16 as O^T = V^T P^T, V^T operands built in
//    registers by byte permutes (each lane holds 4 token rows x 8 dims);
//  * fp8 tiles are widened to bf16 exactly (every E4M3FN value is a bf16
//    value); k_scale folds into the score scale, v_scale into the output.
// Merge kernel: SPLIT workgroups per (split unit, query head), SPLIT = 4
// for small grids (a unit shared by many workers is read by several CUs),
// 1 for many units.  On request (device schedule), the decode kernel's
// last-arriving worker of each split unit merges it instead, counted with
// one atomic per unit after an agent-scope release; that is correct for
// any batch but was slower than the merge kernel on every batch measured.
// The VALU tile math (dot2 products instead of MFMA, G <= 8) shares the
// ring, schedule and merges.
// Lane layout: lane = n + 16 g (n = lane & 15, g = lane >> 4).
//   QK:  A = K rows [token n][8 dims per k-step, in the order KvTile loads
//        them], B = Q^T [head n][the same dims], D[token 4g+i][head n] in
//        register i.
//   PV:  A = V^T [dim 8n+nb][tokens 4g .. 4g+3], B = P^T [tokens 4g+i][head n],
//        D[dim 8(4g+i)+nb][head n] in register i of accumulator nb.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdint>

#include "device_schedule.h"
#include "hpc_decode.h"
#include "internal.h"

namespace hpcd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
#ifndef HPC_DECODE_PENDING
#define HPC_DECODE_PENDING 2
#endif
constexpr int kPending = HPC_DECODE_PENDING;   // entry ends merged together
constexpr int kFusedUnroll = 8;                 // partials' loads in flight per lane, in-kernel merge
constexpr float kLn2 = 0.6931471805599453f;
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw (untyped) buffer, gfx9 family
#ifndef HPC_DECODE_KV_POLICY
#define HPC_DECODE_KV_POLICY 2
#endif
constexpr int kPolicyStream = HPC_DECODE_KV_POLICY;   // K/V buffer-load cache policy (2: nontemporal)
constexpr uint32_t kSelLo = 0x05040100u;       // v_perm: low halves of (a, b) -> {a.lo, b.lo}
constexpr uint32_t kSelHi = 0x07060302u;       // v_perm: high halves -> {a.hi, b.hi}
// device-scheduled merge record of a unit: {workers sharing it (0: empty),
// its first worker, that worker's partial slot, first tile P_u, total tiles T, -}
constexpr int kRecordWords = 6;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                             kRsrcWord3);
}

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& x) {
    static_assert(sizeof(To) == sizeof(From), "size mismatch");
    return __builtin_bit_cast(To, x);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// x over lanes l and l ^ 16 (l ^ 32), combined: the lane-swap instructions
// put each lane's value and its partner's in the two results, in VALU,
// where a shuffle would take a round trip through the LDS unit
__device__ __forceinline__ uint2 swap_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(bitcast<uint32_t>(x), bitcast<uint32_t>(x), false, false);
    return uint2{r[0], r[1]};
}
__device__ __forceinline__ uint2 swap_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(bitcast<uint32_t>(x), bitcast<uint32_t>(x), false, false);
    return uint2{r[0], r[1]};
}
__device__ __forceinline__ float max_xor16(float x) {
    const uint2 r = swap_xor16(x);
    return fmaxf(bitcast<float>(r.x), bitcast<float>(r.y));
}
__device__ __forceinline__ float max_xor32(float x) {
    const uint2 r = swap_xor32(x);
    return fmaxf(bitcast<float>(r.x), bitcast<float>(r.y));
}
__device__ __forceinline__ float sum_xor16(float x) {
    const uint2 r = swap_xor16(x);
    return bitcast<float>(r.x) + bitcast<float>(r.y);
}
__device__ __forceinline__ float sum_xor32(float x) {
    const uint2 r = swap_xor32(x);
    return bitcast<float>(r.x) + bitcast<float>(r.y);
}

// buffer cache policy sc1: the access is coherent at agent scope, across
// every XCD's L2 (a store writes through, a load reads the coherent copy)
constexpr int kPolicyAgent = 16;

// one word written / read coherently at agent scope (a relaxed atomic: a
// global store or load with sc1)
template <typename T>
__device__ __forceinline__ void store_agent(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T load_agent(const T* p) {
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// ---- VALU tile math (the alternative to MFMA, selected per launch) ----
// Largest query-head group the VALU tile math holds (its accumulators are
// 8 heads x 8 dims per lane).
constexpr int kValuHeads = kValuMaxGroup;
static_assert(kValuHeads == 8, "the VALU accumulators are laid out for 8 heads");

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two bf16 products summed into an fp32 accumulator (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(a), bitcast<bf16x2>(b), c, false);
}

// a lane of the same 16-lane row, chosen by a DPP control word (every
// control used here names a valid lane for every lane, so the bound control
// bit only lets the move fold into the instruction that uses it)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(x), CTRL, 0xf, 0xf, true));
}
constexpr int kDppSwap1 = 0xB1;    // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppSwap2 = 0x4E;    // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRor4 = 0x124;    // row_ror:4
constexpr int kDppRor8 = 0x128;    // row_ror:8

// max / sum over the 16 lanes of each row, the result in every lane of it
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<kDppSwap1>(x));
    x = fmaxf(x, dpp_f<kDppSwap2>(x));
    x = fmaxf(x, dpp_f<kDppRor4>(x));
    return fmaxf(x, dpp_f<kDppRor8>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<kDppSwap1>(x);
    x += dpp_f<kDppSwap2>(x);
    x += dpp_f<kDppRor4>(x);
    return x + dpp_f<kDppRor8>(x);
}

// Per KV element type: what one wave loads from one tile, and how it becomes
// MFMA operands.  Offsets are relative to the (page, kv head) block.
template <int KV>
struct KvTile;

template <>
struct KvTile<HPC_KV_BF16> {
    static constexpr uint32_t kRow = kHeadDim * 2;   // bytes per token row
    u32x4 k[4];   // K row 16*wave+n, dims 32kk+8g .. +8 (one 64-byte run per row per load)
    u32x4 v[4];   // V rows 16*wave+4g+i, dims 8n .. 8n+7
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                         int wave, int n, int g) {
        const uint32_t ko = (16 * wave + n) * kRow + 16 * g;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            k[kk] = __builtin_amdgcn_raw_buffer_load_b128(rk, ko + 64 * kk, 0, kPolicyStream);
        const uint32_t vo = (16 * wave + 4 * g) * kRow + 16 * n;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo + i * kRow, 0, kPolicyStream);
    }
    __device__ __forceinline__ bf16x8 k_op(int kk) const { return bitcast<bf16x8>(k[kk]); }
    __device__ __forceinline__ u32x4 v_row(int i) const { return v[i]; }
    // byte offset, in a bf16 Q row, of the 8 dims lane group g supplies in QK step kk
    // (dims 32kk + 8g .. +8, the same k order as the K operand)
    static __device__ __forceinline__ uint32_t q_offset(int kk, int g) { return 64 * kk + 16 * g; }
};

template <>
struct KvTile<HPC_KV_FP8_E4M3> {
    static constexpr uint32_t kRow = kHeadDim;       // bytes per token row
    // K row 16*wave+n, bytes 16g .. +16 (k[0]) and 64 + 16g .. +16 (k[1]): each
    // load instruction reads whole 64-byte halves of the rows.  The QK steps
    // take the dims in this order (step kk, group g: dims 64 (kk >> 1) + 16g +
    // 8 (kk & 1) .. +8); the Q operand is loaded in the same order (q_offset).
    u32x4 k[2];
    u32x2 v[4];   // V rows 16*wave+4g+i, dims 8n .. 8n+7 (fp8)
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                         int wave, int n, int g) {
        const uint32_t ko = (16 * wave + n) * kRow + 16 * g;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            k[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, ko + 64 * j, 0, kPolicyStream);
        const uint32_t vo = (16 * wave + 4 * g) * kRow + 8 * n;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = __builtin_amdgcn_raw_buffer_load_b64(rv, vo + i * kRow, 0, kPolicyStream);
    }
    __device__ __forceinline__ bf16x8 k_op(int kk) const {
        const u32x4& x = k[kk >> 1];
        return bitcast<bf16x8>((kk & 1) ? fp8x8_to_bf16x8(x[2], x[3]) : fp8x8_to_bf16x8(x[0], x[1]));
    }
    __device__ __forceinline__ u32x4 v_row(int i) const { return fp8x8_to_bf16x8(v[i][0], v[i][1]); }
    static __device__ __forceinline__ uint32_t q_offset(int kk, int g) {
        return 128 * (kk >> 1) + 32 * g + 16 * (kk & 1);
    }
};

// Where a tile comes from and where its entry's result goes; all wave-uniform
// (scalar registers, packed to keep a deep ring within the SGPR budget).
struct TileInfo {
    int bits;     // valid token rows (0..64) | first << 7 | last << 8 | real << 9 | kv head << 10
    int row;      // b * Hq + h * G: first query head row of the entry
    int part;     // output target of the entry (see TileRef::part)
    int page;     // physical page of the tile (its scalar load may still be in flight)
    int page2;    // tile pairs: page of the entry's next tile, held in the same slot
    int valid2;   // tile pairs: valid rows of that tile (0: the slot holds one tile)
    __device__ __forceinline__ int valid() const { return bits & 127; }
    __device__ __forceinline__ bool first() const { return (bits >> 7) & 1; }
    __device__ __forceinline__ bool last() const { return (bits >> 8) & 1; }
    __device__ __forceinline__ bool real() const { return (bits >> 9) & 1; }
    __device__ __forceinline__ int head() const { return bits >> 10; }
};

// One slot of the prefetch ring: the K/V rows of NT consecutive tiles of one
// entry (NT = 2 for fp8, so a slot holds as many bytes as one bf16 tile), in
// flight or arrived.
template <int KV, int NT>
struct TileSlot {
    KvTile<KV> kv[NT];
    u32x4 q[4];   // Q^T operand of the entry, loaded only for an entry's first tile
    TileInfo info;
};

// Host-planned tile source: walks this worker's entries in the plan words.
// The worker's first 64 entries (and their sequence lengths) are fetched once
// into the lanes of a few vector registers, lane i holding entry i, so moving
// to the next entry is a lane read, not a chain of dependent memory loads;
// entries beyond those are read from memory.
struct HostWalker {
    const int32_t* entries;
    const int32_t* seq_lens;
    int H, e, e0, e_end;
    int b, h, t, tb, L, part;
    bool have, at_entry_start;
    int c_u, c_t0, c_t1, c_part, c_len;   // lane i: entry e0 + i

    __device__ __forceinline__ void load_entry() {
        have = e < e_end;
        if (!have) return;
        const int i = e - e0;
        int u, len;
        if (i < 64) {
            u = __builtin_amdgcn_readlane(c_u, i);
            t = __builtin_amdgcn_readlane(c_t0, i);
            tb = __builtin_amdgcn_readlane(c_t1, i);
            part = __builtin_amdgcn_readlane(c_part, i);
            len = __builtin_amdgcn_readlane(c_len, i);
        } else {
            u = entries[4 * e + 0];
            t = entries[4 * e + 1];
            tb = entries[4 * e + 2];
            part = entries[4 * e + 3];
            // through the constant address space: the kernel never writes the
            // lengths, and such a load always takes the scalar unit (as a
            // vector load, issued behind the ring's loads, waiting for it
            // would wait for all of them)
            len = ((const __attribute__((address_space(4))) int32_t*)(seq_lens))[u / H];
        }
        b = u / H;
        h = u - b * H;
        L = len;
        at_entry_start = true;
        ++e;
    }
    __device__ __forceinline__ void init(const int32_t* worker_ptr, const int32_t* ent, const int32_t* lens,
                                         int num_kv_heads, int w) {
        entries = ent;
        seq_lens = lens;
        H = num_kv_heads;
        e = e0 = worker_ptr[w];
        e_end = worker_ptr[w + 1];
        const int idx = e0 + static_cast<int>(threadIdx.x & 63);
        c_u = c_t0 = c_t1 = c_part = c_len = 0;
        if (idx < e_end) {
            // an entry's four words start at a 4-byte boundary only (the plan's
            // header and worker_ptr come first), so they are copied, not read
            // through an int4 pointer
            int4 ew;
            __builtin_memcpy(&ew, ent + 4 * static_cast<int64_t>(idx), sizeof(ew));
            c_u = ew.x;
            c_t0 = ew.y;
            c_t1 = ew.z;
            c_part = ew.w;
            c_len = lens[ew.x / num_kv_heads];
        }
        load_entry();
    }
    __device__ __forceinline__ bool next(TileRef& r) {
        if (!have) return false;
        r.b = b;
        r.h = h;
        r.t = t;
        r.L = L;
        r.first = at_entry_start;
        r.last = (t == tb - 1);
        r.part = part;
        at_entry_start = false;
        if (++t == tb) load_entry();
        return true;
    }
};

// Scalars of the decode launch; pointers are separate __restrict__ kernel
// arguments so plan words, block table and lengths are known read-only and
// load through the scalar unit.
struct DecodeScalars {
    int32_t batch, num_kv_heads, group, max_pages_per_seq, num_pages;
    int32_t max_partials;   // partial slots the workspace holds
    float qk_scale_log2, v_scale;
    int32_t n_workers;      // the grid size (passed so no hidden argument is read)
    int32_t entry_price;    // device schedule: the partition's price of a unit start (quarter tiles)
};

// Passes kernel arguments through one empty scalar-register asm, so that
// they are fetched together at the first use of any of them instead of one
// dependent fetch each where they are first used.  The asm is not volatile
// and touches no memory, so later loads stay known as unclobbered (and keep
// going through the scalar unit).
template <typename A, typename B, typename C, typename D>
__device__ __forceinline__ void fetch_args(A& a, B& b, C& c, D& d) {
    asm("" : "+s"(a), "+s"(b), "+s"(c), "+s"(d));
}

// FUSED (device schedule only): the in-kernel merge of split units, as its
// own instantiation, so that the default kernels carry none of its code or
// register pressure
template <int KV, int PF, int NT, bool DEV, bool VALU, bool TRACE, bool FUSED>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const __bf16* __restrict__ q, const char* __restrict__ kcache, const char* __restrict__ vcache,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ worker_ptr, const int32_t* __restrict__ entries,
    __bf16* __restrict__ out, float* __restrict__ lse, float* __restrict__ o_part,
    float* __restrict__ lse_part, int32_t* __restrict__ merge_records, unsigned long long* __restrict__ stamps,
    DecodeScalars a) {
    static_assert(DEV || !FUSED, "the in-kernel merge needs the device schedule");
    // entry ends: register i of every wave's eight accumulators, as two
    // 16-byte halves per lane, so each wave stores and loads whole f32x4s
    // entry ends (MFMA tile math): up to kPending entries' states wait in
    // LDS, each wave depositing its own without a barrier, and are merged
    // together when the slots are full or the worker's range ends
    __shared__ f32x4 s_acc[kPending][4][kWaves][2][64];
    __shared__ float s_m[kPending][kWaves][64];
    __shared__ float s_l[kPending][kWaves][64];
    __shared__ int32_t s_pend[kPending][2];   // output row and target of each pending entry
    __shared__ int32_t s_last;                 // in-kernel merge: this worker arrived last at the unit
    extern __shared__ int32_t s_dyn[];   // device schedule: len[B], tile prefix[B + 1] (, NE prefix[B + 1])
    // VALU tile math: each wave's copy of its entry's Q ([head][dim group g]
    // [k-step], in the K operand's dim order), and the entry-end exchange
    // (per wave and dim group: 8 heads x 128 dims of output sums, and the
    // wave's running max and sum per head)
    __shared__ u32x4 s_vq[kWaves][kValuHeads][4][4];
    __shared__ u32x4 s_vq_sink[kWaves][4][4];
    __shared__ f32x4 s_vacc[kPending][kWaves][4][kValuHeads][kHeadDim / 4];
    __shared__ float s_vm[kPending][kWaves][kValuHeads];
    __shared__ float s_vl[kPending][kWaves][kValuHeads];

    // the host-planned walker reads lengths inside the tile loop: it keeps the
    // argument itself, whose read-only, unaliased provenance lets those reads
    // go through the scalar unit (a pointer that came out of the asm below
    // has lost it, and a vector load there would make the loop wait for
    // every load in flight)
    const int32_t* __restrict__ lens_loop = seq_lens;
    fetch_args(seq_lens, a.batch, a.max_pages_per_seq, a.n_workers);
    // tracing window (the TRACE instantiation, launched only while a window
    // is on): wall-clock stamps of this worker's phases, each stored by
    // thread 0 when taken
    int n_consumed = 0, n_ended = 0;
    auto stamp = [&](int i) {
        if (threadIdx.x == 0) stamps[8 * static_cast<int64_t>(blockIdx.x) + i] = wall_clock64();
    };
    if constexpr (TRACE) stamp(0);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int G = a.group;
    const int Hkv = a.num_kv_heads;
    const int Hq = G * Hkv;
    const int w = blockIdx.x;
    constexpr uint32_t kRow = KvTile<KV>::kRow;
    constexpr uint64_t kBlock = static_cast<uint64_t>(kPage) * kRow;   // one (page, head) block

    // ---- this worker's tile source ----
    Sched sched;
    DeviceWalker dwalk;
    HostWalker hwalk;
    int64_t w_begin = 0, w_end = 0;
    int u_first = 0;
    // in-kernel merge: the units of the worker's first and last tiles and
    // the workers sharing each, taken here so that the schedule need not
    // stay live through the tile loop
    int fm_u[2] = {0, 0}, fm_S[2] = {0, 0};
    if constexpr (DEV) {
        int32_t* const s_ne = s_dyn + 2 * a.batch + 1;   // allocated when entry_price > 0
        build_prefix(seq_lens, a.batch, a.max_pages_per_seq, s_dyn, s_dyn + a.batch,
                     a.entry_price > 0 ? s_ne : nullptr);
        sched.len = s_dyn;
        sched.pb = s_dyn + a.batch;
        sched.ne = s_ne;
        sched.B = a.batch;
        sched.H = Hkv;
        sched.W = a.n_workers;
        sched.set_tiles(static_cast<int64_t>(Hkv) * s_dyn[2 * a.batch]);
        sched.set_price(a.entry_price);
        int b0 = 0, h0 = 0, t0 = 0, L0 = -1;
        if (sched.c != 0) {
            sched.priced_range_uniform(w, w_begin, w_end, b0, h0, t0);
        } else {
            w_begin = uniform(static_cast<int>(sched.equal_begin(w)));   // T < 2^31
            w_end = uniform(static_cast<int>(sched.equal_begin(w + 1)));
            if (w_begin < w_end) sched.locate_uniform_len(w_begin, b0, h0, t0, L0);
        }
        if (w_begin < w_end) {
            dwalk.init_at(sched, w, w_begin, w_end, b0, h0, t0, L0);
            u_first = dwalk.b * Hkv + dwalk.h;    // the unit of the worker's first tile
            if constexpr (FUSED) {
                int bB, hB, tB, LB;
                sched.locate_uniform_len(w_end - 1, bB, hB, tB, LB);
                fm_u[0] = u_first;
                fm_u[1] = bB * Hkv + hB;
                fm_S[0] = sched.parts(dwalk.b, dwalk.h);
                fm_S[1] = fm_u[1] == u_first ? 0 : sched.parts(bB, hB);
            }
        } else {
            dwalk.remaining = 0;                   // an empty worker: only bookkeeping below
        }
    } else {
        hwalk.init(worker_ptr, entries, lens_loop, Hkv, w);
        if (!hwalk.have) return;
    }

    // Filling a ring slot: `plan_tile` takes the next tile of the worker and
    // starts the scalar load of its page id; `load_tile` issues the K/V (and,
    // for an entry's first tile, Q) loads.
    auto plan_tile = [&](TileInfo& s) {
        TileRef r;
        bool ok;
        if constexpr (DEV) ok = dwalk.next(r);
        else ok = hwalk.next(r);
        int page = 0, h = 0, row = 0, part = -1, first = 0, last = 0, rem = 0;
        if (ok) {
            const int b = uniform(r.b);
            const int t = uniform(r.t);
            h = uniform(r.h);
            page = block_table[static_cast<int64_t>(b) * a.max_pages_per_seq + t];
            rem = uniform(r.L) - t * kPage;
            row = b * Hq + h * G;
            first = r.first;
            last = r.last;
            part = r.part;
        }
        int page2 = 0, valid2 = 0;
        if constexpr (NT == 2) {
            // the entry's next tile shares the slot (same sequence, head and Q)
            if (ok && !last) {
                TileRef r2;
                if constexpr (DEV) dwalk.next(r2);
                else hwalk.next(r2);
                const int t2 = uniform(r2.t);
                page2 = block_table[static_cast<int64_t>(uniform(r2.b)) * a.max_pages_per_seq + t2];
                const int rem2 = uniform(r2.L) - t2 * kPage;
                valid2 = rem2 < 0 ? 0 : (rem2 > kPage ? kPage : rem2);
                last = r2.last;
            }
        }
        const int valid = rem < 0 ? 0 : (rem > kPage ? kPage : rem);
        s.bits = uniform(valid | (first ? 1 << 7 : 0) | (last ? 1 << 8 : 0) | (ok ? 1 << 9 : 0) | (h << 10));
        s.page = page;
        s.row = uniform(row);
        s.part = uniform(part);
        s.page2 = page2;
        s.valid2 = uniform(valid2);
    };
    auto load_tile = [&](TileSlot<KV, NT>& s, const TileInfo& info) {
        s.info = info;
        int page = uniform(info.page);
        if (static_cast<unsigned>(page) >= static_cast<unsigned>(a.num_pages)) {
            s.info.bits &= ~127;
            page = 0;
        }
        // Q^T operand of a new entry: head n, in the K operand's dim order
        // (KvTile::q_offset); heads >= G read
        // as zero, and so does all of it for a tile that does not start an entry.
        // Issued before the K/V loads, so that it has landed whenever they have.
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(q + static_cast<int64_t>(info.row) * kHeadDim, info.first() ? G * kHeadDim * 2 : 0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            s.q[kk] = __builtin_amdgcn_raw_buffer_load_b128(rq, n * kHeadDim * 2 + KvTile<KV>::q_offset(kk, g), 0, 0);
        const uint64_t off = (static_cast<uint64_t>(page) * Hkv + info.head()) * kBlock;
        const uint32_t kv_bytes = static_cast<uint32_t>(s.info.valid()) * kRow;
        s.kv[0].load(make_rsrc(kcache + off, kv_bytes), make_rsrc(vcache + off, kv_bytes), wave, n, g);
        if constexpr (NT == 2) {
            int page2 = uniform(info.page2);
            int valid2 = info.valid2;
            if (static_cast<unsigned>(page2) >= static_cast<unsigned>(a.num_pages)) {
                s.info.valid2 = 0;
                valid2 = 0;
                page2 = 0;
            }
            const uint64_t off2 = (static_cast<uint64_t>(page2) * Hkv + info.head()) * kBlock;
            const uint32_t kv_bytes2 = static_cast<uint32_t>(valid2) * kRow;
            s.kv[1].load(make_rsrc(kcache + off2, kv_bytes2), make_rsrc(vcache + off2, kv_bytes2), wave, n, g);
        }
    };

    TileSlot<KV, NT> ring[PF];
    TileInfo planned[PF];   // the tile each slot loads next
#pragma unroll
    for (int j = 0; j < PF; ++j) plan_tile(planned[j]);
    // Slots are issued in ring order, each slot's Q before its K/V: the
    // loop's first wait (for slot 0) must leave the later slots in flight on
    // the path that enters the loop too, so the scheduler may not reorder
    // these loads across slots.
#pragma unroll
    for (int j = 0; j < PF; ++j) {
        load_tile(ring[j], planned[j]);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (TRACE) stamp(1);

    // Device schedule, while the first tiles are in flight: empty sequences
    // get out = 0, lse = -inf and a merge record saying so, from worker
    // u mod W; every other unit's record {S_u, first worker, its slot, P_u,
    // T} is written by the worker holding the unit's first tile, here
    // rather than at the entry's end, so no entry end waits for it.  Units
    // are in tile order, so this worker's are the ones from the unit of its
    // first tile on whose first tile lies before its range ends; such a
    // unit is its first entry (slot 2w when split) if it starts the range,
    // else its last (slot 2w + 1 when split).  All records are rewritten
    // every step.
    if constexpr (DEV) {
        const int U = a.batch * Hkv;
        for (int u = w + a.n_workers * static_cast<int>(threadIdx.x); u < U;
             u += a.n_workers * kDecodeThreads) {
            const int b = u / Hkv;
            if (sched.len[b] != 0) continue;
            const int64_t row = static_cast<int64_t>(b) * Hq + (u - b * Hkv) * G;
            for (int i = 0; i < G * 16; ++i)
                *reinterpret_cast<u32x4*>(out + (row + (i >> 4)) * kHeadDim + 8 * (i & 15)) = u32x4{0u, 0u, 0u, 0u};
            for (int i = 0; i < G; ++i) lse[row + i] = -INFINITY;
            if constexpr (FUSED) store_agent(merge_records + kRecordWords * u, 0);
            else merge_records[kRecordWords * u] = 0;
        }
        if (w_begin == w_end) return;
        for (int u = u_first + static_cast<int>(threadIdx.x); u < U; u += kDecodeThreads) {
            const int b = u / Hkv;
            const int h = u - b * Hkv;
            const int64_t pu = sched.unit_start(b, h);
            if (pu >= w_end) break;
            if (pu < w_begin || sched.len[b] == 0) continue;
            const int S = sched.parts(b, h);
            int32_t* rec = merge_records + kRecordWords * u;
            const int32_t words[5] = {S, w, S >= 2 ? 2 * w + (pu == w_begin ? 0 : 1) : -1, static_cast<int32_t>(pu),
                                      static_cast<int32_t>(sched.T)};
            if constexpr (FUSED) {
                // the in-kernel merge reads them from other XCDs within this
                // launch: stored coherently at agent scope
#pragma unroll
                for (int i = 0; i < 5; ++i) store_agent(rec + i, words[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 5; ++i) rec[i] = words[i];
            }
        }
    }

    float m = -INFINITY;   // running max (log2 domain), uniform over g
    float l = 0.f;         // this lane's share of the running sum
    f32x4 acc[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 qop[4];

    // An entry ends: this wave's state goes to pending slot npend (every
    // wave sees the same entries, so npend is the same in all of them), and
    // the wave goes on without waiting for the others.
    int npend = 0;
    auto deposit = [&](const TileInfo& ts) {
        l = sum_xor32(sum_xor16(l));
        const int p = npend;
        s_m[p][wave][lane] = m;
        s_l[p][wave][lane] = l;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s_acc[p][i][wave][0][lane] = f32x4{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
            s_acc[p][i][wave][1][lane] = f32x4{acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
        }
        if (threadIdx.x == 0) {
            s_pend[p][0] = ts.row;
            s_pend[p][1] = ts.part;
        }
        ++npend;
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // The pending entries meet: one (o, lse) per head and entry, bf16 out for
    // a whole unit, an fp32 partial otherwise.  Wave w merges accumulator
    // register w of all four waves (dims 32g + 8w .. +8 of head n).
    auto merge_pending = [&]() {
        __syncthreads();
        for (int p = 0; p < npend; ++p) {
            const int row = s_pend[p][0];
            const int part = s_pend[p][1];
            float ms[kWaves], M = -INFINITY;
#pragma unroll
            for (int s = 0; s < kWaves; ++s) {
                ms[s] = s_m[p][s][lane];
                M = fmaxf(M, ms[s]);
            }
            const float M_use = (M == -INFINITY) ? 0.f : M;
            float wt[kWaves], wsum = 0.f;
#pragma unroll
            for (int s = 0; s < kWaves; ++s) {
                wt[s] = __builtin_amdgcn_exp2f(ms[s] - M_use);
                wsum += wt[s] * s_l[p][s][lane];
            }
            float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < kWaves; ++s) {
                const f32x4 lo = s_acc[p][wave][s][0][lane];
                const f32x4 hi = s_acc[p][wave][s][1][lane];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    o[k] += wt[s] * lo[k];
                    o[4 + k] += wt[s] * hi[k];
                }
            }
            const int slot = part;
            if (n < G) {
                const float inv = (wsum > 0.f) ? a.v_scale / wsum : 0.f;
                const float lse_val = (wsum > 0.f) ? (M + __log2f(wsum)) * kLn2 : -INFINITY;
                const int dim0 = 32 * g + 8 * wave;
                if (slot < 0) {
                    bf16x8 ov;
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb) ov[nb] = static_cast<__bf16>(o[nb] * inv);
                    *reinterpret_cast<bf16x8*>(out + static_cast<int64_t>(row + n) * kHeadDim + dim0) = ov;
                    if (wave == 0 && g == 0) lse[row + n] = lse_val;
                } else if (slot < a.max_partials) {   // a slot is always in range; the test keeps stray writes out
                    const int64_t pidx = static_cast<int64_t>(slot) * G + n;
                    const f32x4 lo4 = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
                    const f32x4 hi4 = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
                    if constexpr (FUSED) {
                        // read by another worker of this launch: written through to agent scope
                        const __amdgpu_buffer_rsrc_t ro = make_rsrc(o_part, 0xFFFFFFFFu);
                        const uint32_t off = static_cast<uint32_t>((pidx * kHeadDim + dim0) * 4);
                        __builtin_amdgcn_raw_buffer_store_b128(bitcast<u32x4>(lo4), ro, off, 0, kPolicyAgent);
                        __builtin_amdgcn_raw_buffer_store_b128(bitcast<u32x4>(hi4), ro, off + 16, 0, kPolicyAgent);
                        if (wave == 0 && g == 0)
                            __builtin_amdgcn_raw_buffer_store_b32(bitcast<uint32_t>(lse_val), make_rsrc(lse_part, 0xFFFFFFFFu),
                                                                  static_cast<uint32_t>(pidx * 4), 0, kPolicyAgent);
                    } else {
                        float* dst = o_part + pidx * kHeadDim + dim0;
                        *reinterpret_cast<f32x4*>(dst) = lo4;
                        *reinterpret_cast<f32x4*>(dst + 4) = hi4;
                        if (wave == 0 && g == 0) lse_part[pidx] = lse_val;
                    }
                }
            }
        }
        __syncthreads();
        npend = 0;
    };

    auto consume = [&](const TileSlot<KV, NT>& s) {
        // the slot's Q registers are read on every tile (a select, not a
        // branch): a load whose result went unread could have its register
        // reused while still in flight, which forces a wait for every load
        const bool fq = s.info.first();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const u32x4 prev = bitcast<u32x4>(qop[kk]);
            qop[kk] = bitcast<bf16x8>(u32x4{fq ? s.q[kk][0] : prev[0], fq ? s.q[kk][1] : prev[1],
                                            fq ? s.q[kk][2] : prev[2], fq ? s.q[kk][3] : prev[3]});
        }
        const int r0 = 16 * wave + 4 * g;
        f32x4 sc[NT];
        float mt = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            sc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                sc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s.kv[tt].k_op(kk), qop[kk], sc[tt], 0, 0, 0);
            const int valid = tt == 0 ? s.info.valid() : s.info.valid2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc[tt][i] = (r0 + i < valid) ? sc[tt][i] * a.qk_scale_log2 : -INFINITY;
                mt = fmaxf(mt, sc[tt][i]);
            }
        }
        mt = max_xor32(max_xor16(mt));
        const float m_new = fmaxf(m, mt);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - m_use);
        float psum = 0.f;
        bf16x4 pop[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = __builtin_amdgcn_exp2f(sc[tt][i] - m_use);
                psum += p[i];
            }
            pop[tt] = bf16x4{static_cast<__bf16>(p[0]), static_cast<__bf16>(p[1]), static_cast<__bf16>(p[2]),
                             static_cast<__bf16>(p[3])};
        }
        l = l * alpha + psum;
        m = m_new;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[nb] = acc[nb] * alpha;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            u32x4 rows[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) rows[i] = s.kv[tt].v_row(i);
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int d = nb >> 1;
                const uint32_t sel = (nb & 1) ? kSelHi : kSelLo;
                const u32x2 vt = u32x2{__builtin_amdgcn_perm(rows[1][d], rows[0][d], sel),
                                       __builtin_amdgcn_perm(rows[3][d], rows[2][d], sel)};
                acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bitcast<bf16x4>(vt), pop[tt], acc[nb], 0, 0, 0);
            }
        }
    };

    // ---- VALU tile math ----
    // K: lane (n, g) holds token row 16 wave + n, dims of group g (the MFMA
    // K operand registers).  Scores: dot2 over the lane's 32 dims against
    // the entry's Q (read from this wave's LDS copy), then summed over the
    // four dim groups by a reduce-scatter of half-wave and row swaps that
    // leaves 4 heads per register, one head per 16-lane row: register R,
    // row r holds head hid[R] of that row (R = head / 4) for token row n.
    // The softmax then runs on 2 registers.  V: lane (n, g) holds rows
    // 16 wave + 4g + i (i < 4), dims 8n .. 8n+7 (the MFMA V registers); P
    // reaches it as bf16 pairs of rows (4g + 2j, 4g + 2j + 1) gathered from
    // the row holding the head, and P V is dot2 over those token pairs into
    // vacc[head][dim 8n + e], a partial sum over the lane's 4 rows.  vm[R]
    // (running max) is the same in the 16 lanes of a row; vl[R] is the
    // lane's token share of the running sum.
    float vm[2], vl[2], vacc[kValuHeads][8];
#pragma unroll
    for (int R = 0; R < 2; ++R) {
        vm[R] = -INFINITY;
        vl[R] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < kValuHeads; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) vacc[h][e] = 0.f;

    // Which head each row of a reduced register holds: the same swaps applied
    // to head numbers (a swap returns, in any one lane, two halves of one
    // source register, so those lanes' sum belongs to that register's head).
    int hid[2];
#pragma unroll
    for (int R = 0; R < 2; ++R) {
        const auto x = __builtin_amdgcn_permlane32_swap(4u * R, 4u * R + 1u, false, false);
        const auto y = __builtin_amdgcn_permlane32_swap(4u * R + 2u, 4u * R + 3u, false, false);
        hid[R] = static_cast<int>(__builtin_amdgcn_permlane16_swap(x[0], y[0], false, false)[0]);
    }
    // and the row of each head (wave-uniform)
    int row_of[kValuHeads];
#pragma unroll
    for (int h = 0; h < kValuHeads; ++h) {
        const int R = h >> 2;
        const int i0 = __builtin_amdgcn_readlane(hid[R], 0), i1 = __builtin_amdgcn_readlane(hid[R], 16),
                  i2 = __builtin_amdgcn_readlane(hid[R], 32);
        row_of[h] = i0 == h ? 0 : (i1 == h ? 1 : (i2 == h ? 2 : 3));
    }

    // sum of four heads' partial dot products over the four dim groups:
    // row r of the result holds the head hid[R] says, for token row n
    auto reduce4 = [](float d0, float d1, float d2, float d3) -> float {
        const auto a = __builtin_amdgcn_permlane32_swap(bitcast<uint32_t>(d0), bitcast<uint32_t>(d1), false, false);
        const auto b = __builtin_amdgcn_permlane32_swap(bitcast<uint32_t>(d2), bitcast<uint32_t>(d3), false, false);
        const float x = bitcast<float>(a[0]) + bitcast<float>(a[1]);
        const float y = bitcast<float>(b[0]) + bitcast<float>(b[1]);
        const auto c = __builtin_amdgcn_permlane16_swap(bitcast<uint32_t>(x), bitcast<uint32_t>(y), false, false);
        return bitcast<float>(c[0]) + bitcast<float>(c[1]);
    };

    auto consume_valu = [&](const TileSlot<KV, NT>& s) {
        // the slot's Q words go to LDS on every tile (so its load registers
        // are read on every path, as in the MFMA body): into this wave's copy
        // for an entry's first tile (lane (n, g) holds head n), else into a
        // sink.  LDS accesses of one wave complete in order, so the reads
        // below see them.
        const bool to_copy = s.info.first() && n < kValuHeads;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u32x4* dst = to_copy ? &s_vq[wave][n & (kValuHeads - 1)][g][kk] : &s_vq_sink[wave][g][kk];
            *dst = s.q[kk];
        }
        // partial dot products: k-step outer, so the 8 heads' Q of one step
        // are read together and the 8 accumulator chains interleave
        float d[NT][kValuHeads];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int h = 0; h < kValuHeads; ++h) d[tt][h] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u32x4 qw[kValuHeads];
#pragma unroll
            for (int h = 0; h < kValuHeads; ++h) qw[h] = s_vq[wave][h][g][kk];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const u32x4 kw = bitcast<u32x4>(s.kv[tt].k_op(kk));
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int h = 0; h < kValuHeads; ++h) d[tt][h] = dot2(kw[j], qw[h][j], d[tt][h]);
            }
        }
        const int kr = 16 * wave + n;   // this lane's K row in the tile
        float sc[NT][2], mt[2] = {-INFINITY, -INFINITY};
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int valid = tt == 0 ? s.info.valid() : s.info.valid2;
#pragma unroll
            for (int R = 0; R < 2; ++R) {
                const float x = reduce4(d[tt][4 * R], d[tt][4 * R + 1], d[tt][4 * R + 2], d[tt][4 * R + 3]);
                sc[tt][R] = (kr < valid) ? x * a.qk_scale_log2 : -INFINITY;
                mt[R] = fmaxf(mt[R], sc[tt][R]);
            }
        }
        float mu[2], alpha[2];
        bool grew = false;
#pragma unroll
        for (int R = 0; R < 2; ++R) {
            const float m_new = fmaxf(vm[R], row16_max(mt[R]));
            mu[R] = (m_new == -INFINITY) ? 0.f : m_new;
            alpha[R] = __builtin_amdgcn_exp2f(vm[R] - mu[R]);
            grew |= m_new > vm[R];
            vm[R] = m_new;
        }
        float p[NT][2];
#pragma unroll
        for (int R = 0; R < 2; ++R) {
            float ps = 0.f;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                p[tt][R] = __builtin_amdgcn_exp2f(sc[tt][R] - mu[R]);
                ps += p[tt][R];
            }
            vl[R] = vl[R] * alpha[R] + ps;
        }
        // rescale the output sums only when some running max grew (alpha is
        // exactly 1 wherever it did not); a head's factor is uniform over its row
        if (__builtin_amdgcn_ballot_w64(grew) != 0) {
#pragma unroll
            for (int h = 0; h < kValuHeads; ++h) {
                const float f = bitcast<float>(
                    __builtin_amdgcn_readlane(bitcast<int>(alpha[h >> 2]), 16 * row_of[h]));
#pragma unroll
                for (int e = 0; e < 8; ++e) vacc[h][e] *= f;
            }
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            // bf16 pairs of P over rows (t, t + 1): a lane of even token row
            // packs (p[t], p[t + 1]); lane (n, g) reads token rows 4g and
            // 4g + 2 from the row holding each head
            uint32_t pk[2];
#pragma unroll
            for (int R = 0; R < 2; ++R) {
                const float pn = dpp_f<kDppSwap1>(p[tt][R]);
                pk[R] = bitcast<uint32_t>(bf16x2{static_cast<__bf16>(p[tt][R]), static_cast<__bf16>(pn)});
            }
            uint32_t pp[kValuHeads][2];
#pragma unroll
            for (int h = 0; h < kValuHeads; ++h)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    pp[h][j] = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(
                        4 * (16 * row_of[h] + 4 * g + 2 * j), static_cast<int>(pk[h >> 2])));
            u32x4 rows[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) rows[i] = s.kv[tt].v_row(i);
            // V pairs over the same rows, one per dim: (v[4g+2j][d], v[4g+2j+1][d])
            uint32_t vp[2][8];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int dd = 0; dd < 4; ++dd) {
                    vp[j][2 * dd] = __builtin_amdgcn_perm(rows[2 * j + 1][dd], rows[2 * j][dd], kSelLo);
                    vp[j][2 * dd + 1] = __builtin_amdgcn_perm(rows[2 * j + 1][dd], rows[2 * j][dd], kSelHi);
                }
#pragma unroll
            for (int h = 0; h < kValuHeads; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) vacc[h][e] = dot2(vp[1][e], pp[h][1], dot2(vp[0][e], pp[h][0], vacc[h][e]));
        }
    };

    // Entry ends of the VALU tile math, as for the MFMA one: each wave
    // deposits its state in pending slot nvpend without waiting (its output
    // sums for its 4 rows, dims 8n ..; each head's running max and sum from
    // the first lane of the head's row), and the pending entries meet when
    // the slots are full or the range ends.
    int nvpend = 0;
    auto deposit_valu = [&](const TileInfo& ts) {
        const int p = nvpend;
#pragma unroll
        for (int h = 0; h < kValuHeads; ++h) {
            s_vacc[p][wave][g][h][2 * n] = f32x4{vacc[h][0], vacc[h][1], vacc[h][2], vacc[h][3]};
            s_vacc[p][wave][g][h][2 * n + 1] = f32x4{vacc[h][4], vacc[h][5], vacc[h][6], vacc[h][7]};
        }
#pragma unroll
        for (int R = 0; R < 2; ++R) {
            const float lw = row16_sum(vl[R]);
            if (n == 0) {
                s_vm[p][wave][hid[R]] = vm[R];
                s_vl[p][wave][hid[R]] = lw;
            }
        }
        if (threadIdx.x == 0) {
            s_pend[p][0] = ts.row;
            s_pend[p][1] = ts.part;
        }
        ++nvpend;
#pragma unroll
        for (int R = 0; R < 2; ++R) {
            vm[R] = -INFINITY;
            vl[R] = 0.f;
        }
#pragma unroll
        for (int h = 0; h < kValuHeads; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) vacc[h][e] = 0.f;
    };
    // thread t: head t / 32, dims 4 (t % 32) .. +4 of each pending entry,
    // over 4 waves x 4 dim groups
    auto merge_pending_valu = [&]() {
        __syncthreads();
        const int hh = static_cast<int>(threadIdx.x) >> 5;
        const int dq = static_cast<int>(threadIdx.x) & 31;
        for (int p = 0; p < nvpend; ++p) {
            const int row = s_pend[p][0];
            const int part = s_pend[p][1];
            float ms[kWaves], M = -INFINITY;
#pragma unroll
            for (int w4 = 0; w4 < kWaves; ++w4) {
                ms[w4] = s_vm[p][w4][hh];
                M = fmaxf(M, ms[w4]);
            }
            const float M_use = (M == -INFINITY) ? 0.f : M;
            float wsum = 0.f;
            f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w4 = 0; w4 < kWaves; ++w4) {
                const float wt = __builtin_amdgcn_exp2f(ms[w4] - M_use);
                wsum += wt * s_vl[p][w4][hh];
                f32x4 sw = s_vacc[p][w4][0][hh][dq];
#pragma unroll
                for (int gg = 1; gg < 4; ++gg) sw += s_vacc[p][w4][gg][hh][dq];
                o += wt * sw;
            }
            if (hh < G) {
                const float inv = (wsum > 0.f) ? a.v_scale / wsum : 0.f;
                const float lse_val = (wsum > 0.f) ? (M + __log2f(wsum)) * kLn2 : -INFINITY;
                const int slot = part;
                if (slot < 0) {
                    const bf16x4 ov = bf16x4{static_cast<__bf16>(o[0] * inv), static_cast<__bf16>(o[1] * inv),
                                             static_cast<__bf16>(o[2] * inv), static_cast<__bf16>(o[3] * inv)};
                    *reinterpret_cast<bf16x4*>(out + static_cast<int64_t>(row + hh) * kHeadDim + 4 * dq) = ov;
                    if (dq == 0) lse[row + hh] = lse_val;
                } else if (slot < a.max_partials) {   // a slot is always in range; the test keeps stray writes out
                    const int64_t pidx = static_cast<int64_t>(slot) * G + hh;
                    if constexpr (FUSED) {
                        // read by another worker of this launch: written through to agent scope
                        __builtin_amdgcn_raw_buffer_store_b128(bitcast<u32x4>(o * inv), make_rsrc(o_part, 0xFFFFFFFFu),
                                                               static_cast<uint32_t>((pidx * kHeadDim + 4 * dq) * 4), 0,
                                                               kPolicyAgent);
                        if (dq == 0)
                            __builtin_amdgcn_raw_buffer_store_b32(bitcast<uint32_t>(lse_val), make_rsrc(lse_part, 0xFFFFFFFFu),
                                                                  static_cast<uint32_t>(pidx * 4), 0, kPolicyAgent);
                    } else {
                        *reinterpret_cast<f32x4*>(o_part + pidx * kHeadDim + 4 * dq) = o * inv;
                        if (dq == 0) lse_part[pidx] = lse_val;
                    }
                }
            }
        }
        __syncthreads();
        nvpend = 0;
    };

    // One exit, at the end of a full ring turn: every path back to the top
    // has re-issued all PF slots, so the compiler's load-counter waits let
    // the other PF - 1 tiles stay in flight.  Slots are filled in tile order,
    // so once slot 0 comes back empty all slots are; a later slot of the last
    // turn may be consumed empty, which changes nothing (its scores are all
    // -inf).  Slot 0 holds a tile on entry (workers without tiles returned
    // above).  A slot that ends an entry is refilled before the entry's
    // state is deposited, so the barriers of a merge, which wait for the
    // slowest wave, run with every slot's loads in flight.
    for (;;) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            if constexpr (VALU) consume_valu(ring[j]);
            else consume(ring[j]);
            if constexpr (TRACE) {
                if (n_consumed++ == 0) stamp(2);
            }
            const TileInfo ended = ring[j].info;
            plan_tile(planned[j]);
            load_tile(ring[j], planned[j]);
            if (ended.last()) {
                if constexpr (TRACE) ++n_ended;
                if constexpr (VALU) {
                    deposit_valu(ended);
                    if (nvpend == kPending) merge_pending_valu();
                } else {
                    deposit(ended);
                    if (npend == kPending) merge_pending();
                }
            }
        }
        if (!ring[0].info.real()) break;
    }
    if constexpr (TRACE) stamp(3);
    if constexpr (VALU) {
        if (nvpend > 0) merge_pending_valu();
    } else {
        if (npend > 0) merge_pending();
    }

    // In-kernel merge (the FUSED instantiation): every partial of this
    // worker is written.  Partials and merge records cross XCDs only through
    // agent-coherent (sc1) stores and loads, so no L2 write-back or
    // invalidate is needed: each wave waits until its stores have completed,
    // and after the barrier one atomic count per split unit the worker holds
    // a share of (its first entry, and its last when that is another unit)
    // goes to the unit's merge record.  The worker that brings the count to
    // S_u merges the unit and sets the count back to zero, so the records
    // are ready for the next step.  No worker waits for another.
    if constexpr (FUSED) {
        {
            // this wave's partial and record stores (agent-coherent) have completed
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
#pragma unroll 1
            for (int k = 0; k < 2; ++k) {
                const int u = fm_u[k];
                const int bu = u / Hkv;
                const int S = fm_S[k];   // 0 for a second unit that is the first
                if (S < 2) continue;
                int32_t* rec = merge_records + kRecordWords * u;
                if (threadIdx.x == 0) {
                    const int before = __hip_atomic_fetch_add(rec + 5, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    const int last = before == S - 1;
                    if (last) store_agent(rec + 5, 0);
                    s_last = last;
                }
                __syncthreads();
                if (s_last) {
                    // the unit's partial slots, from its record (stored by its first
                    // worker, agent-coherently, before that worker's count), and
                    // the partials, read coherently too: no L2 invalidate
                    const int w_first = load_agent(rec + 1), first_slot = load_agent(rec + 2);
                    const int64_t Pu = load_agent(rec + 3), T = load_agent(rec + 4);
                    const __amdgpu_buffer_rsrc_t ro = make_rsrc(o_part, 0xFFFFFFFFu);
                    const __amdgpu_buffer_rsrc_t rl = make_rsrc(lse_part, 0xFFFFFFFFu);
                    auto slot_of = [&](int kk) -> int {
                        if (kk == 0) return first_slot;
                        if (static_cast<int64_t>(a.n_workers) <= T) return 2 * (w_first + kk);
                        return 2 * small_quot((Pu + kk + 1) * a.n_workers - 1, T);
                    };
                    const int64_t row0 = static_cast<int64_t>(bu) * Hq + (u - bu * Hkv) * G;
                    const int dq = static_cast<int>(threadIdx.x) & 31;
                    for (int hh = static_cast<int>(threadIdx.x) >> 5; hh < G; hh += kDecodeThreads / 32) {
                        float mm = -INFINITY, ww = 0.f;
                        f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
                        for (int i0 = 0; i0 < S; i0 += kFusedUnroll) {
                            float lv[kFusedUnroll];
                            f32x4 ov[kFusedUnroll];
#pragma unroll
                            for (int j = 0; j < kFusedUnroll; ++j) {
                                const int i = i0 + j;
                                const int slot = slot_of(i < S ? i : 0);
                                const int64_t pidx = (slot < a.max_partials ? static_cast<int64_t>(slot) : 0) * G + hh;
                                const float lp = bitcast<float>(__builtin_amdgcn_raw_buffer_load_b32(
                                    rl, static_cast<uint32_t>(pidx * 4), 0, kPolicyAgent));
                                lv[j] = (i < S && slot < a.max_partials) ? lp * kLog2e : -INFINITY;
                                ov[j] = bitcast<f32x4>(__builtin_amdgcn_raw_buffer_load_b128(
                                    ro, static_cast<uint32_t>((pidx * kHeadDim + 4 * dq) * 4), 0, kPolicyAgent));
                            }
                            float mk = mm;
#pragma unroll
                            for (int j = 0; j < kFusedUnroll; ++j) mk = fmaxf(mk, lv[j]);
                            const float m_use = (mk == -INFINITY) ? 0.f : mk;
                            const float f = __builtin_amdgcn_exp2f(mm - m_use);
                            o *= f;
                            ww *= f;
#pragma unroll
                            for (int j = 0; j < kFusedUnroll; ++j) {
                                const float e = __builtin_amdgcn_exp2f(lv[j] - m_use);
                                o += e * ov[j];
                                ww += e;
                            }
                            mm = mk;
                        }
                        const float inv = ww > 0.f ? 1.f / ww : 0.f;
                        const bf16x4 res = bf16x4{static_cast<__bf16>(o[0] * inv), static_cast<__bf16>(o[1] * inv),
                                                  static_cast<__bf16>(o[2] * inv), static_cast<__bf16>(o[3] * inv)};
                        *reinterpret_cast<bf16x4*>(out + (row0 + hh) * kHeadDim + 4 * dq) = res;
                        if (dq == 0) lse[row0 + hh] = ww > 0.f ? (mm + __log2f(ww)) * kLn2 : -INFINITY;
                    }
                }
                __syncthreads();   // s_last is rewritten for the next unit
            }
        }
    }
    if constexpr (TRACE) {
        stamp(4);
        if (threadIdx.x == 0) {
            unsigned long long* st = stamps + 8 * static_cast<int64_t>(w);
            st[5] = DEV ? static_cast<unsigned long long>(w_end - w_begin) : 0ull;
            st[6] = static_cast<unsigned long long>(n_ended);
            // where the worker ran: XCC_ID register (high word), HW_ID (low: CU, SH, SE, ...)
            const unsigned hw_id = __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));
            const unsigned xcc_id = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (31 << 11));
            st[7] = (static_cast<unsigned long long>(xcc_id) << 32) | hw_id;
        }
    }
}

// Merge of split units: SPLIT workgroups per (merge record, query head of
// the group), each merging 128 / SPLIT of the dims.  SPLIT = 4 (few records)
// lets a unit shared by many workers be read by several compute units at
// once; SPLIT = 1 (many records) keeps the grid small when most records need
// little or no work.  256 threads = kLanes partial lanes x kQuads dim quads.
// Lane pl folds partials i = pl, pl + kLanes, ... into a running (max,
// weighted sum, weight) triple, issuing up to eight partials' loads before
// using any of them; the triples are then merged by log-sum-exp, within each
// wave with lane shuffles and the 4 wave results in LDS.  The records are the
// host plan's merge list, or, for the device-scheduled step, one record per
// unit written by the decode kernel.
constexpr int kMergeUnroll = 8;
constexpr int kMergeGridBudget = 1024;   // largest grid the 4-way split may take (4 per CU)

template <bool DEV, int SPLIT>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
    constexpr int kMergeSplit = SPLIT;
    constexpr int kMergeQuads = kHeadDim / 4 / kMergeSplit;   // dim quads per workgroup
    constexpr int kMergeLanes = kCombineThreads / kMergeQuads;
    static_assert(kMergeQuads <= 32, "at least two partial lanes per wave");
    __shared__ f32x4 s_acc[kCombineThreads / 64][kMergeQuads];
    __shared__ float s_m[kCombineThreads / 64];
    __shared__ float s_w[kCombineThreads / 64];

    fetch_args(a.combine, a.o_part, a.lse_part, a.group);
    const int G = a.group;
    const int Hkv = a.num_kv_heads;
    const int qd = blockIdx.x % kMergeSplit;
    const int cn = blockIdx.x / kMergeSplit;
    const int c = cn / G;
    const int n = cn - c * G;
    int u, S, base = 0;
    int w_first = 0, first_slot = 0, W = a.n_workers;
    int64_t Pu = 0, T = 1;
    if constexpr (DEV) {
        const int32_t* rec = a.combine + kRecordWords * c;
        u = c;
        S = rec[0];
        if (S <= 1) return;   // empty (written by the decode kernel) or written directly
        w_first = rec[1];
        first_slot = rec[2];
        Pu = rec[3];
        T = rec[4];
    } else {
        const int32_t* rec = a.combine + 3 * c;
        u = rec[0];
        S = rec[1];
        base = rec[2];
    }
    // partial slot of the k-th worker of the unit
    auto slot_of = [&](int k) -> int {
        if constexpr (!DEV) return base + k;
        if (k == 0) return first_slot;
        // later workers start inside the unit, so it is their first entry (slot 2w)
        if (static_cast<int64_t>(W) <= T) return 2 * (w_first + k);
        return 2 * small_quot((Pu + k + 1) * W - 1, T);   // one tile per worker
    };
    const int b = u / Hkv;
    const int h = u - b * Hkv;
    const int64_t row = static_cast<int64_t>(b) * (G * Hkv) + h * G + n;
    const int t = threadIdx.x;
    const int dq = t % kMergeQuads;
    const int pl = t / kMergeQuads;
    const int dim0 = 4 * (kMergeQuads * qd + dq);
    __bf16* out = static_cast<__bf16*>(a.out) + row * kHeadDim;

    if (S == 0) {   // empty sequence: out = 0, lse = -inf
        if (pl == 0) *reinterpret_cast<u32x2*>(out + dim0) = u32x2{0u, 0u};
        if (t == 0 && qd == 0) a.lse[row] = -INFINITY;
        return;
    }
    if (static_cast<int64_t>(slot_of(0)) >= a.max_partials || static_cast<int64_t>(slot_of(S - 1)) >= a.max_partials ||
        (!DEV && static_cast<int64_t>(base) + S > a.max_partials)) {   // never for a consistent schedule: NaN
        if (pl == 0) *reinterpret_cast<u32x2*>(out + dim0) = u32x2{0x7fc07fc0u, 0x7fc07fc0u};
        if (t == 0 && qd == 0) a.lse[row] = __builtin_nanf("");
        return;
    }

    float m = -INFINITY;          // running max of the folded lse values (log2 units)
    float w = 0.f;                // running sum of 2^(lse - m)
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i0 = pl; i0 < S; i0 += kMergeLanes * kMergeUnroll) {
        float lv[kMergeUnroll];
        f32x4 o[kMergeUnroll];
#pragma unroll
        for (int k = 0; k < kMergeUnroll; ++k) {
            const int i = i0 + k * kMergeLanes;
            const int64_t p = static_cast<int64_t>(slot_of(i < S ? i : 0)) * G + n;
            lv[k] = (i < S) ? a.lse_part[p] * kLog2e : -INFINITY;
            o[k] = *reinterpret_cast<const f32x4*>(a.o_part + p * kHeadDim + dim0);
        }
        float mk = m;
#pragma unroll
        for (int k = 0; k < kMergeUnroll; ++k) mk = fmaxf(mk, lv[k]);
        const float m_use = (mk == -INFINITY) ? 0.f : mk;
        const float f = __builtin_amdgcn_exp2f(m - m_use);
        acc *= f;
        w *= f;
#pragma unroll
        for (int k = 0; k < kMergeUnroll; ++k) {
            const float e = __builtin_amdgcn_exp2f(lv[k] - m_use);
            acc += e * o[k];
            w += e;
        }
        m = mk;
    }
    // fold the partial lanes of each wave with shuffles (lanes that differ
    // only in bits at or above log2(kMergeQuads) hold the same dims), then
    // the 4 waves through LDS
#pragma unroll
    for (int off = kMergeQuads; off < 64; off <<= 1) {
        const float m2 = __shfl_xor(m, off);
        const float w2 = __shfl_xor(w, off);
        f32x4 a2;
#pragma unroll
        for (int i = 0; i < 4; ++i) a2[i] = __shfl_xor(acc[i], off);
        const float M = fmaxf(m, m2);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        const float f1 = __builtin_amdgcn_exp2f(m - M_use);
        const float f2 = __builtin_amdgcn_exp2f(m2 - M_use);
        acc = acc * f1 + a2 * f2;
        w = w * f1 + w2 * f2;
        m = M;
    }
    const int wave = t >> 6;
    if ((t & 63) < kMergeQuads) {
        s_acc[wave][dq] = acc;
        if (dq == 0) {
            s_m[wave] = m;
            s_w[wave] = w;
        }
    }
    __syncthreads();
    if (t < kMergeQuads) {
        float M = -INFINITY;
#pragma unroll
        for (int j = 0; j < kCombineThreads / 64; ++j) M = fmaxf(M, s_m[j]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
        float ws = 0.f;
#pragma unroll
        for (int j = 0; j < kCombineThreads / 64; ++j) {
            const float e = __builtin_amdgcn_exp2f(s_m[j] - M_use);
            r += e * s_acc[j][dq];
            ws += e * s_w[j];
        }
        const float inv = ws > 0.f ? 1.f / ws : 0.f;
        const bf16x4 ov = bf16x4{static_cast<__bf16>(r[0] * inv), static_cast<__bf16>(r[1] * inv),
                                 static_cast<__bf16>(r[2] * inv), static_cast<__bf16>(r[3] * inv)};
        *reinterpret_cast<bf16x4*>(out + dim0) = ov;
        if (dq == 0 && qd == 0) a.lse[row] = ws > 0.f ? (M + __log2f(ws)) * kLn2 : -INFINITY;
    }
}

// The device schedule written out in the host plan's word layout, by one
// workgroup, so it can be compared word for word with the host planner.
__global__ __launch_bounds__(kPlanThreads) void plan_device_kernel(const int32_t* __restrict__ seq_lens, int B,
                                                                   int H, int W, int entry_price, int max_pages,
                                                                   int32_t* __restrict__ plan) {
    extern __shared__ int32_t s_dyn[];
    __shared__ int32_t s_tmp[kPlanThreads / 64];
    const int U = B * H;
    int32_t* s_len = s_dyn;               // [B]
    int32_t* s_pb = s_len + B;            // [B + 1]
    int32_t* s_ne = s_pb + B + 1;         // [B + 1] sequences with tiles before b
    int32_t* s_cnt = s_ne + B + 1;        // [W]   entries per worker -> worker_ptr
    int32_t* s_base = s_cnt + W;          // [U]   split slots per unit -> base
    int32_t* s_cidx = s_base + U;         // [U]   merge record flag -> record index
    build_prefix(seq_lens, B, max_pages, s_len, s_pb, s_ne);
    Sched sched;
    sched.len = s_len;
    sched.pb = s_pb;
    sched.ne = s_ne;
    sched.B = B;
    sched.H = H;
    sched.W = W;
    sched.set_tiles(static_cast<int64_t>(H) * s_pb[B]);
    sched.set_price(entry_price);
    const int t = threadIdx.x;

    for (int w = t; w < W; w += kPlanThreads) {
        DeviceWalker dw;
        dw.init(sched, w, sched.range_begin(w), sched.range_begin(w + 1), false);
        TileRef r;
        int cnt = 0;
        while (dw.next(r)) cnt += r.first ? 1 : 0;
        s_cnt[w] = cnt;
    }
    for (int u = t; u < U; u += kPlanThreads) {
        const int b = u / H;
        const int S = sched.parts(b, u - b * H);
        s_base[u] = S >= 2 ? S : 0;
        s_cidx[u] = S != 1 ? 1 : 0;
    }
    __syncthreads();
    const int E = block_scan_inplace<kPlanThreads>(s_cnt, W, s_tmp);
    const int P = block_scan_inplace<kPlanThreads>(s_base, U, s_tmp);
    const int C = block_scan_inplace<kPlanThreads>(s_cidx, U, s_tmp);

    int32_t* wp = plan + HPC_PLAN_HEADER_WORDS;
    int32_t* ent = wp + W + 1;
    int32_t* comb = ent + 4 * E;
    if (t < HPC_PLAN_HEADER_WORDS) {
        const int32_t hdr[10] = {HPC_PLAN_VERSION, B, H, W, static_cast<int32_t>(sched.T), E, P, C, HPC_DECODE_PAGE,
                                 sched.c};
        plan[t] = t < 10 ? hdr[t] : 0;
    }
    if (t == 0) wp[W] = E;
    for (int w = t; w < W; w += kPlanThreads) {
        wp[w] = s_cnt[w];
        const int64_t beg = sched.range_begin(w), end = sched.range_begin(w + 1);
        if (beg == end) continue;
        int b0, h0, t0;
        sched.locate(beg, b0, h0, t0);
        const int k0 = sched.rank_in_unit(w, b0, h0, t0);
        DeviceWalker dw;
        dw.init(sched, w, beg, end, false);
        TileRef r;
        int e = s_cnt[w] - 1;
        int ta = 0;
        while (dw.next(r)) {
            if (r.first) {
                ++e;
                ta = r.t;
            }
            if (r.last) {
                const int u = r.b * H + r.h;
                // the walker numbers split entries by worker (2w first, 2w + 1 last);
                // the plan numbers them by unit: base_u + rank of the worker in the unit
                const int slot = r.part < 0 ? -1 : (r.part == 2 * w ? s_base[u] + k0 : s_base[u]);
                ent[4 * e + 0] = u;
                ent[4 * e + 1] = ta;
                ent[4 * e + 2] = r.t + 1;
                ent[4 * e + 3] = slot;
            }
        }
    }
    for (int u = t; u < U; u += kPlanThreads) {
        const int b = u / H;
        const int S = sched.parts(b, u - b * H);
        if (S == 1) continue;
        const int i = s_cidx[u];
        comb[3 * i + 0] = u;
        comb[3 * i + 1] = S;
        comb[3 * i + 2] = S >= 2 ? s_base[u] : 0;
    }
}

// tiles in flight per wave (register ring depth)
#ifndef HPC_DECODE_PREFETCH_BF16
#define HPC_DECODE_PREFETCH_BF16 2
#endif
#ifndef HPC_DECODE_PREFETCH_FP8
#define HPC_DECODE_PREFETCH_FP8 2
#endif
// fp8: two tiles of an entry per ring slot (a slot then holds as many bytes as a bf16 tile)
#ifndef HPC_DECODE_PAIR_FP8
#define HPC_DECODE_PAIR_FP8 1
#endif
constexpr int kPrefetchBf16 = HPC_DECODE_PREFETCH_BF16;
constexpr int kPrefetchFp8 = HPC_DECODE_PREFETCH_FP8;

template <int KV, int PF, bool DEV, bool VALU, bool FUSED>
void launch_decode_f(const DecodeArgs& a, int n_workers, size_t lds, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const DecodeScalars sc{a.batch,        a.num_kv_heads,  a.group,   a.max_pages_per_seq, a.num_pages,
                           a.max_partials, a.qk_scale_log2, a.v_scale, n_workers, a.entry_price};
    constexpr int kTilesPerSlot = KV == HPC_KV_FP8_E4M3 ? HPC_DECODE_PAIR_FP8 + 1 : 1;
    unsigned long long* const stamps = trace_buffer(n_workers);
    const auto q = static_cast<const __bf16*>(a.q);
    const auto k = static_cast<const char*>(a.k);
    const auto v = static_cast<const char*>(a.v);
    const auto out = static_cast<__bf16*>(a.out);
    if (stamps)
        hipExtLaunchKernelGGL((decode_kernel<KV, PF, kTilesPerSlot, DEV, VALU, true, FUSED>), dim3(n_workers),
                              dim3(kDecodeThreads), static_cast<std::uint32_t>(lds), s, e0, e1, 0u, q, k, v,
                              a.block_table, a.seq_lens, a.worker_ptr, a.entries, out, a.lse, a.o_part, a.lse_part,
                              a.merge_records, stamps, sc);
    else
        hipExtLaunchKernelGGL((decode_kernel<KV, PF, kTilesPerSlot, DEV, VALU, false, FUSED>), dim3(n_workers),
                              dim3(kDecodeThreads), static_cast<std::uint32_t>(lds), s, e0, e1, 0u, q, k, v,
                              a.block_table, a.seq_lens, a.worker_ptr, a.entries, out, a.lse, a.o_part, a.lse_part,
                              a.merge_records, stamps, sc);
}

template <int KV, int PF, bool DEV, bool VALU>
void launch_decode_t(const DecodeArgs& a, int n_workers, size_t lds, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if constexpr (DEV) {
        if (a.fused_merge) {
            launch_decode_f<KV, PF, true, VALU, true>(a, n_workers, lds, s, e0, e1);
            return;
        }
    }
    launch_decode_f<KV, PF, DEV, VALU, false>(a, n_workers, lds, s, e0, e1);
}

}  // namespace

namespace {
template <bool VALU>
void launch_decode_m(const DecodeArgs& a, int kv_dtype, int n_workers, bool device_sched, size_t lds,
                     hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if (kv_dtype == HPC_KV_BF16) {
        if (device_sched) launch_decode_t<HPC_KV_BF16, kPrefetchBf16, true, VALU>(a, n_workers, lds, s, e0, e1);
        else launch_decode_t<HPC_KV_BF16, kPrefetchBf16, false, VALU>(a, n_workers, lds, s, e0, e1);
    } else {
        if (device_sched) launch_decode_t<HPC_KV_FP8_E4M3, kPrefetchFp8, true, VALU>(a, n_workers, lds, s, e0, e1);
        else launch_decode_t<HPC_KV_FP8_E4M3, kPrefetchFp8, false, VALU>(a, n_workers, lds, s, e0, e1);
    }
}
}  // namespace

int launch_decode(const DecodeArgs& a, int kv_dtype, int tile_math, int n_workers, bool device_sched, void* stream,
                  void* ev_start, void* ev_stop) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t e0 = static_cast<hipEvent_t>(ev_start), e1 = static_cast<hipEvent_t>(ev_stop);
    // device schedule: lengths and tile prefix, and the NE prefix when priced
    const size_t lds =
        device_sched ? ((a.entry_price > 0 ? 3 : 2) * static_cast<size_t>(a.batch) + (a.entry_price > 0 ? 2 : 1)) *
                           sizeof(int32_t)
                     : 0;
    if (tile_math == HPC_TILE_MATH_VALU) launch_decode_m<true>(a, kv_dtype, n_workers, device_sched, lds, s, e0, e1);
    else launch_decode_m<false>(a, kv_dtype, n_workers, device_sched, lds, s, e0, e1);
    return static_cast<int>(hipGetLastError());
}

int launch_combine(const CombineArgs& a, int n_records, bool device_sched, void* stream, void* ev_start,
                   void* ev_stop) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t e0 = static_cast<hipEvent_t>(ev_start), e1 = static_cast<hipEvent_t>(ev_stop);
    const bool wide = static_cast<int64_t>(n_records) * a.group * 4 <= kMergeGridBudget;
    const dim3 grid(static_cast<unsigned>(n_records * a.group * (wide ? 4 : 1)));
    if (device_sched) {
        if (wide) hipExtLaunchKernelGGL(combine_kernel<true, 4>, grid, dim3(kCombineThreads), 0u, s, e0, e1, 0u, a);
        else hipExtLaunchKernelGGL(combine_kernel<true, 1>, grid, dim3(kCombineThreads), 0u, s, e0, e1, 0u, a);
    } else {
        if (wide) hipExtLaunchKernelGGL(combine_kernel<false, 4>, grid, dim3(kCombineThreads), 0u, s, e0, e1, 0u, a);
        else hipExtLaunchKernelGGL(combine_kernel<false, 1>, grid, dim3(kCombineThreads), 0u, s, e0, e1, 0u, a);
    }
    return static_cast<int>(hipGetLastError());
}

int launch_plan_device(const int32_t* seq_lens, int batch, int num_kv_heads, int n_workers, int entry_price,
                       int max_pages_per_seq, int32_t* plan, void* stream) {
    const int U = batch * num_kv_heads;
    const size_t lds = (static_cast<size_t>(3 * batch + 2) + n_workers + 2 * static_cast<size_t>(U)) * sizeof(int32_t);
    hipLaunchKernelGGL(plan_device_kernel, dim3(1), dim3(kPlanThreads), lds, static_cast<hipStream_t>(stream),
                       seq_lens, batch, num_kv_heads, n_workers, entry_price, max_pages_per_seq, plan);
    return static_cast<int>(hipGetLastError());
}

}  // namespace hpcd
