// The per-step tile schedule computed on the GPU, shared by the decode
// kernel, the merge kernel and the plan-materialising kernel.
//
// It is the same schedule the host planner writes (plan.cpp): sequences cut
// into 64-token tiles, units u = b * H + h in batch-major order, worker w
// owning global tiles [floor(w T / W), floor((w + 1) T / W)); the split
// partials of a unit take consecutive slots after those of every earlier
// split unit.  Here each workgroup derives what it needs from the device
// copy of the lengths, using closed forms instead of the host's sweep:
//   owner(j)  = floor(((j + 1) W - 1) / T)             worker of tile j (W <= T)
//   S_u       = owner(P_u + n_u - 1) - owner(P_u) + 1   workers sharing unit u
//               (W > T: every non-empty worker holds one tile, so S_u = n_u)
//   base_u    = sum over u' < u with S_u' >= 2 of S_u'
// (§Attention Backend: Dynamic Load-Balanced Scheduling, "vLLM x HPC-Ops:
// High-Performance Attention and MoE Backends from Tencent Hunyuan").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hpcd {

__device__ __forceinline__ int tiles_of(int L) { return (L + 63) >> 6; }

__device__ __forceinline__ int wave_inclusive_sum(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    return x;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
    return x;
}

// Lengths (clamped to [0, max_pages * 64]) into s_len[B] and the exclusive
// prefix of tile counts into s_pb[B + 1].  Every thread of the block calls
// it; s_tmp needs NT / 64 ints.  Ends with a barrier.
template <int NT>
__device__ void build_prefix(const int32_t* __restrict__ seq_lens, int B, int max_pages, int32_t* s_len,
                             int32_t* s_pb, int32_t* s_tmp) {
    const int t = threadIdx.x;
    const int per = (B + NT - 1) / NT;
    const int lo = t * per;
    const int hi = min(B, lo + per);
    const int cap = max_pages * 64;
    int sum = 0;
    for (int b = lo; b < hi; ++b) {
        int L = seq_lens[b];
        L = L < 0 ? 0 : (L > cap ? cap : L);
        s_len[b] = L;
        sum += tiles_of(L);
    }
    const int incl = wave_inclusive_sum(sum);
    if ((t & 63) == 63) s_tmp[t >> 6] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < (t >> 6); ++w) run += s_tmp[w];
    for (int b = lo; b < hi; ++b) {
        s_pb[b] = run;
        run += tiles_of(s_len[b]);
    }
    if (t == NT - 1) s_pb[B] = run;
    __syncthreads();
}

struct Sched {
    const int32_t* len;   // LDS [B]
    const int32_t* pb;    // LDS [B + 1]
    int B, H, W;
    int64_t T;

    __device__ __forceinline__ int tiles(int b) const { return tiles_of(len[b]); }
    __device__ __forceinline__ int64_t unit_start(int b, int h) const {
        return static_cast<int64_t>(H) * pb[b] + static_cast<int64_t>(h) * tiles(b);
    }
    __device__ __forceinline__ int64_t range_begin(int w) const { return (static_cast<int64_t>(w) * T) / W; }
    __device__ __forceinline__ int owner(int64_t j) const {    // valid for W <= T
        return static_cast<int>(((j + 1) * W - 1) / T);
    }
    // number of workers that share unit (b, h)
    __device__ __forceinline__ int parts(int b, int h) const {
        const int n = tiles(b);
        if (n == 0) return 0;
        if (static_cast<int64_t>(W) > T) return n;
        const int64_t a = unit_start(b, h);
        return owner(a + n - 1) - owner(a) + 1;
    }
    // (b, h, t) of global tile j, 0 <= j < T
    __device__ __forceinline__ void locate(int64_t j, int& b, int& h, int& t) const {
        int lo = 0, hi = B;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (static_cast<int64_t>(H) * pb[mid] <= j) lo = mid;
            else hi = mid;
        }
        b = lo;
        const int n = tiles(b);
        const int64_t r = j - static_cast<int64_t>(H) * pb[b];
        h = static_cast<int>(r / n);
        t = static_cast<int>(r - static_cast<int64_t>(h) * n);
    }
    // k such that worker w (whose range starts at tile `t_first` of unit
    // (b, h)) is the k-th worker of that unit
    __device__ __forceinline__ int rank_in_unit(int w, int b, int h, int t_first) const {
        if (static_cast<int64_t>(W) > T) return t_first;
        return w - owner(unit_start(b, h));
    }
};

// base_u of two units at once: sum over u' < u of S_u' for split units.
// Wave-level (every wave computes it for itself; no barrier).
__device__ __forceinline__ void split_bases_wave(const Sched& s, int u1, int u2, int& base1, int& base2) {
    int a1 = 0, a2 = 0;
    const int umax = max(u1, u2);
    for (int u = threadIdx.x & 63; u < umax; u += 64) {
        const int b = u / s.H;
        const int S = s.parts(b, u - b * s.H);
        const int c = S >= 2 ? S : 0;
        if (u < u1) a1 += c;
        if (u < u2) a2 += c;
    }
    base1 = wave_sum(a1);
    base2 = wave_sum(a2);
}

// Block-wide form of the same (NT threads, all must call); s_tmp needs
// 2 * NT / 64 ints.
template <int NT>
__device__ void split_bases(const Sched& s, int u1, int u2, int& base1, int& base2, int32_t* s_tmp) {
    int a1 = 0, a2 = 0;
    const int umax = max(u1, u2);
    for (int u = threadIdx.x; u < umax; u += NT) {
        const int b = u / s.H;
        const int S = s.parts(b, u - b * s.H);
        const int c = S >= 2 ? S : 0;
        if (u < u1) a1 += c;
        if (u < u2) a2 += c;
    }
    a1 = wave_sum(a1);
    a2 = wave_sum(a2);
    __syncthreads();   // s_tmp may still be read by an earlier caller
    if ((threadIdx.x & 63) == 0) {
        s_tmp[2 * (threadIdx.x >> 6)] = a1;
        s_tmp[2 * (threadIdx.x >> 6) + 1] = a2;
    }
    __syncthreads();
    base1 = 0;
    base2 = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        base1 += s_tmp[2 * w];
        base2 += s_tmp[2 * w + 1];
    }
}

// Walks one worker's tiles in order, entry by entry.  Device-scheduled form:
// the entries come from the worker's tile range; a host-planned form with the
// same interface reads them from the plan words (decode_kernels.hip).
struct TileRef {
    int b, h, t;       // sequence, kv head, tile of the unit
    int L;             // sequence length
    bool first, last;  // first / last tile of its entry
    int part;          // -1: direct output; >= 0: partial slot; kPartFirst / kPartLast: resolved later
};

constexpr int kPartFirst = -2;   // the worker's first entry, split
constexpr int kPartLast = -3;    // the worker's last entry, split

struct DeviceWalker {
    const Sched* s;
    int b, h, t, n;          // next tile to hand out
    int64_t remaining;       // tiles of the worker not yet handed out
    bool at_start;           // the next tile is the worker's first
    int cur_part;            // part code of the entry holding the next tile

    __device__ __forceinline__ void init(const Sched& sched, int64_t begin, int64_t end) {
        s = &sched;
        remaining = end - begin;
        at_start = true;
        if (remaining > 0) {
            sched.locate(begin, b, h, t);
            n = sched.tiles(b);
            const bool split = (t > 0) || (static_cast<int64_t>(n - t) > remaining);
            cur_part = split ? kPartFirst : -1;
        } else {
            b = h = t = n = 0;
            cur_part = -1;
        }
    }

    __device__ __forceinline__ bool next(TileRef& r) {
        if (remaining <= 0) return false;
        r.b = b;
        r.h = h;
        r.t = t;
        r.L = s->len[b];
        r.first = (t == 0) || at_start;
        r.last = (t == n - 1) || (remaining == 1);
        r.part = cur_part;
        at_start = false;
        --remaining;
        ++t;
        if (t == n && remaining > 0) {   // on to the next unit that has tiles
            t = 0;
            ++h;
            if (h == s->H) {
                h = 0;
                do { ++b; } while (s->tiles(b) == 0);
            }
            n = s->tiles(b);
            // an entry after the first starts at tile 0; it is split only if
            // the worker's range ends inside it (then it is the last entry)
            cur_part = (static_cast<int64_t>(n) > remaining) ? kPartLast : -1;
        }
        return true;
    }
};

}  // namespace hpcd
