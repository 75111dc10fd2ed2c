// The per-step tile schedule computed on the GPU, shared by the decode
// kernel, the merge kernel and the plan-materialising kernel.
//
// It is the same schedule the host planner writes (plan.cpp): sequences cut
// into 64-token tiles, units u = b * H + h in batch-major order, worker w
// owning global tiles [floor(w T / W), floor((w + 1) T / W)) (or the priced
// partition below); the split
// partials of a unit take consecutive slots after those of every earlier
// split unit.  Here each workgroup derives what it needs from the device
// copy of the lengths, using closed forms instead of the host's sweep:
//   owner(j)  = floor(((j + 1) W - 1) / T)             worker of tile j (W <= T)
//   S_u       = owner(P_u + n_u - 1) - owner(P_u) + 1   workers sharing unit u
//               (W > T: every non-empty worker holds one tile, so S_u = n_u)
//   base_u    = sum over u' < u with S_u' >= 2 of S_u'
// (§Attention Backend: Dynamic Load-Balanced Scheduling, "vLLM x HPC-Ops:
// High-Performance Attention and MoE Backends from Tencent Hunyuan").
//
// Priced partition (this library's extension, hpc_decode_plan_priced): a
// tile costs 4, a unit's first tile c more; with A(j) the cost of tiles
// before j and C = A(T), worker w starts at the largest j with
// A(j) <= floor(w C / W), and the worker of tile j is the one whose cost
// window (floor(w C / W), floor((w + 1) C / W)] holds A(j + 1):
//   owner(j)  = floor((A(j + 1) W - 1) / C)
// With NE_b the sequences with tiles before b, unit (b, h) starts at cost
// H (4 P_b + c NE_b) + h (4 n_b + c), P_b being the tile prefix per head.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

extern "C" __device__ int __ockl_wfred_add_i32(int);
extern "C" __device__ int __ockl_wfscan_add_i32(int, bool);

namespace hpcd {

__device__ __forceinline__ int tiles_of(int L) { return (L + 63) >> 6; }

// floor(x / y) for 0 <= x < 2^62, 1 <= y < 2^31 when the quotient is below
// 2^20: a single-precision estimate (conversions, reciprocal and product
// leave a relative error below 2^-21, so the estimate is off by at most one)
// corrected with exact integer products.  Much shorter than a 64-bit integer
// or double division.
__device__ __forceinline__ int small_quot(int64_t x, int64_t y) {
    int q = static_cast<int>(static_cast<float>(x) * __builtin_amdgcn_rcpf(static_cast<float>(y)));
    if (static_cast<int64_t>(q) * y > x) --q;
    else if (static_cast<int64_t>(q + 1) * y <= x) ++q;
    return q;
}

// floor(x / y) when the quotient is at most qmax < 2^16 and qmax * y < 2^32:
// the single-precision estimate is off by at most one (as above), clamping it
// to qmax keeps the 32-bit products below from wrapping, and one step fixes it.
__device__ __forceinline__ uint32_t quot_u32(uint32_t x, uint32_t y, uint32_t qmax) {
    uint32_t q = static_cast<uint32_t>(static_cast<float>(x) * __builtin_amdgcn_rcpf(static_cast<float>(y)));
    q = min(q, qmax);
    const uint32_t p = q * y;
    if (p > x) --q;
    else if (x - p >= y) ++q;
    return q;
}

__device__ __forceinline__ int wave_inclusive_sum(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    return x;
}

__device__ __forceinline__ int wave_sum(int x) { return __ockl_wfred_add_i32(x); }

// Lengths (clamped to [0, max_pages * 64]) into s_len[B] and the exclusive
// prefix of tile counts into s_pb[B + 1], and, when s_ne is not null, the
// exclusive count of sequences with tiles into s_ne[B + 1]; built by the
// first wave alone (wave-wide scans, 64 sequences at a time).  Every thread
// of the block calls it and it ends with the block's only barrier.
__device__ void build_prefix(const int32_t* __restrict__ seq_lens, int B, int max_pages, int32_t* s_len,
                             int32_t* s_pb, int32_t* s_ne = nullptr) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int cap = max_pages * 64;
        int carry = 0, carry_ne = 0;
        for (int b0 = 0; b0 < B; b0 += 64) {
            const int b = b0 + lane;
            int L = b < B ? seq_lens[b] : 0;
            L = L < 0 ? 0 : (L > cap ? cap : L);
            const int n = tiles_of(L);
            const int incl = __ockl_wfscan_add_i32(n, true);
            if (b < B) {
                s_len[b] = L;
                s_pb[b] = carry + incl - n;
            }
            carry += __shfl(incl, 63);
            if (s_ne != nullptr) {
                const unsigned long long have = __ballot(n > 0);
                if (b < B) s_ne[b] = carry_ne + __popcll(have & ((1ull << lane) - 1ull));
                carry_ne += __popcll(have);
            }
        }
        if (lane == 0) {
            s_pb[B] = carry;
            if (s_ne != nullptr) s_ne[B] = carry_ne;
        }
    }
    __syncthreads();
}

struct Sched {
    const int32_t* len;   // LDS [B]
    const int32_t* pb;    // LDS [B + 1]
    const int32_t* ne;    // LDS [B + 1], sequences with tiles before b (priced partition only)
    int B, H, W;          // W <= 65536
    int64_t T;            // < 2^31
    int64_t qT, rT;       // T = qT W + rT
    int c;                // entry price applied (0: equal tile shares)
    int32_t C, qC, rC;    // priced: total cost C < 2^31, C = qC W + rC

    __device__ __forceinline__ void set_tiles(int64_t tiles) {
        T = tiles;
        const uint32_t t32 = static_cast<uint32_t>(tiles);
        qT = t32 / static_cast<uint32_t>(W);
        rT = tiles - qT * W;
        c = 0;
    }
    // after set_tiles, with ne filled: applies the price where the rule
    // allows it (W <= T, C >= (4 + c + 1) W, C < 2^31), as the host does
    __device__ __forceinline__ void set_price(int price) {
        if (price <= 0 || static_cast<int64_t>(W) > T) return;
        const int64_t cost = 4 * T + static_cast<int64_t>(price) * H * ne[B];
        if (cost < static_cast<int64_t>(4 + price + 1) * W || cost >= (int64_t(1) << 31)) return;
        c = price;
        C = static_cast<int32_t>(cost);
        qC = static_cast<int32_t>(static_cast<uint32_t>(cost) / static_cast<uint32_t>(W));
        rC = C - qC * W;
    }
    // priced: cost of the tiles before sequence b, per kv head (H times it is A(P_b))
    __device__ __forceinline__ int64_t seq_cost(int b) const {
        return 4 * static_cast<int64_t>(pb[b]) + static_cast<int64_t>(c) * ne[b];
    }
    // priced: A at the start of unit (b, h)
    __device__ __forceinline__ int64_t unit_cost_start(int b, int h) const {
        return static_cast<int64_t>(H) * seq_cost(b) + static_cast<int64_t>(h) * (4 * tiles(b) + c);
    }
    // priced: the worker whose cost window holds a = A(j + 1), 1 <= a <= C
    __device__ __forceinline__ int owner_at_cost(int64_t a) const { return small_quot(a * W - 1, C); }

    __device__ __forceinline__ int tiles(int b) const { return tiles_of(len[b]); }
    __device__ __forceinline__ int64_t unit_start(int b, int h) const {
        return static_cast<int64_t>(H) * pb[b] + static_cast<int64_t>(h) * tiles(b);
    }
    // priced: floor(w C / W) = w qC + floor(w rC / W), for w < W (then < C);
    // 32-bit as equal_begin, with C < 2^31 in place of T
    __device__ __forceinline__ int64_t tau(int w) const {
        const uint32_t uw = static_cast<uint32_t>(w);
        const uint32_t uW = static_cast<uint32_t>(W);
        return static_cast<int64_t>(uw * static_cast<uint32_t>(qC) +
                                    quot_u32(uw * static_cast<uint32_t>(rC), uW, uW - 1));
    }
    // priced: the largest j with A(j) <= tau < C, given the last sequence b
    // whose cost prefix is <= tau (a sequence with tiles, as tau < C).  j
    // lies in the unit h of b whose cost span holds tau, at the tiles t of
    // that unit that fit: A(start + t) = start + c + 4 t for t >= 1, and
    // t < n as tau is below the next unit's start.  32-bit: H unit <= C < 2^31
    // and H <= 4096, within quot_u32's bounds.
    __device__ __forceinline__ int64_t cut_in(int b, int64_t tau_w, int& h, int& t) const {
        const int n = tiles(b);
        const int unit = 4 * n + c;
        const int r = static_cast<int>(tau_w - static_cast<int64_t>(H) * seq_cost(b));   // < H * unit < 2^31
        h = static_cast<int>(quot_u32(static_cast<uint32_t>(r), static_cast<uint32_t>(unit),
                                      static_cast<uint32_t>(H - 1)));   // < H
        const int rem = r - h * unit - c;
        t = rem < 4 ? 0 : min(n - 1, rem >> 2);
        return static_cast<int64_t>(H) * pb[b] + static_cast<int64_t>(h) * n + t;
    }
    // equal shares: floor(w T / W) = w qT + floor(w rT / W) for 0 <= w <= W,
    // all in 32 bits: w qT <= T < 2^31, w rT < W^2 <= 2^32, and the quotient
    // is below W <= 2^16 (at most W - 1, with (W - 1) W < 2^32)
    __device__ __forceinline__ int64_t equal_begin(int w) const {
        const uint32_t uw = static_cast<uint32_t>(w);
        const uint32_t uW = static_cast<uint32_t>(W);
        return static_cast<int64_t>(uw * static_cast<uint32_t>(qT) +
                                    quot_u32(uw * static_cast<uint32_t>(rT), uW, uW - 1));
    }
    // floor(w T / W) = w qT + floor(w rT / W), with w rT < W^2; priced: the
    // largest j with A(j) <= floor(w C / W), the last sequence whose cost
    // prefix is at most that found by binary search (per-thread form)
    __device__ __forceinline__ int64_t range_begin(int w) const {
        if (c == 0) return equal_begin(w);
        if (w >= W) return T;
        const int64_t tw = tau(w);
        int lo = 0, hi = B;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (static_cast<int64_t>(H) * seq_cost(mid) <= tw) lo = mid;
            else hi = mid;
        }
        int h, t;
        return cut_in(lo, tw, h, t);
    }
    // priced, wave-uniform w < W, whole wave active: both ends of worker w's
    // range from one pass of the lanes over the sequences (64 at a time,
    // each lane testing one sequence's cost prefix against both bounds),
    // and the sequence, head and tile of its first tile when the range is
    // not empty
    __device__ __forceinline__ void priced_range_uniform(int w, int64_t& begin, int64_t& end, int& b, int& h,
                                                         int& t) const {
        const int64_t t0 = tau(w);
        const bool last = w + 1 >= W;
        const int64_t t1 = last ? t0 : tau(w + 1);
        // every cost prefix H (4 P_b + c NE_b) and bound is at most C < 2^31
        const int u0 = static_cast<int>(t0), u1 = static_cast<int>(t1);
        int n0 = 0, n1 = 0;
        for (int b0 = 0; b0 < B; b0 += 64) {
            const int bb = b0 + (threadIdx.x & 63);
            const int sc = bb < B ? H * (4 * pb[bb] + c * ne[bb]) : INT32_MAX;
            const int k0 = __popcll(__ballot(sc <= u0));
            const int k1 = __popcll(__ballot(sc <= u1));
            n0 += k0;
            n1 += k1;
            if (k1 < 64) break;   // the prefix only grows: no later sequence is within either bound
        }
        b = __builtin_amdgcn_readfirstlane(n0 - 1);
        begin = __builtin_amdgcn_readfirstlane(static_cast<int>(cut_in(b, t0, h, t)));   // < T < 2^31
        h = __builtin_amdgcn_readfirstlane(h);
        t = __builtin_amdgcn_readfirstlane(t);
        if (last) {
            end = T;
        } else {
            int h1, tt1;
            end = __builtin_amdgcn_readfirstlane(
                static_cast<int>(cut_in(__builtin_amdgcn_readfirstlane(n1 - 1), t1, h1, tt1)));
        }
    }
    __device__ __forceinline__ int owner(int64_t j) const {    // valid for W <= T (quotient < W)
        return small_quot((j + 1) * W - 1, T);
    }
    // number of workers that share unit (b, h)
    __device__ __forceinline__ int parts(int b, int h) const {
        const int n = tiles(b);
        if (n == 0) return 0;
        if (static_cast<int64_t>(W) > T) return n;
        if (c != 0) {
            const int64_t a = unit_cost_start(b, h);
            return owner_at_cost(a + 4 * n + c) - owner_at_cost(a + 4 + c) + 1;
        }
        const int64_t a = unit_start(b, h);
        return owner(a + n - 1) - owner(a) + 1;
    }
    // (b, h, t) of global tile j, 0 <= j < T: b is the last sequence whose
    // tiles start at or before j (such a sequence has tiles).
    __device__ __forceinline__ void split_tile(int64_t j, int b_, int& b, int& h, int& t) const {
        b = b_;
        const int n = tiles(b);
        const int r = static_cast<int>(j - static_cast<int64_t>(H) * pb[b]);   // < H * n < 2^31
        h = r / n;
        t = r - h * n;
    }
    // per-thread form: binary search over the non-decreasing prefix
    __device__ __forceinline__ void locate(int64_t j, int& b, int& h, int& t) const {
        int lo = 0, hi = B;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (static_cast<int64_t>(H) * pb[mid] <= j) lo = mid;
            else hi = mid;
        }
        split_tile(j, lo, b, h, t);
    }
    // wave-uniform j, whole wave active: the lanes test 64 sequences at once
    // and count the ones that start at or before j
    __device__ __forceinline__ void locate_uniform(int64_t j, int& b, int& h, int& t) const {
        int count = 0;
        for (int b0 = 0; b0 < B; b0 += 64) {
            const int bb = b0 + (threadIdx.x & 63);
            const bool le = bb < B && static_cast<int64_t>(H) * pb[bb] <= j;
            const int c = __popcll(__ballot(le));
            count += c;
            if (c < 64) break;
        }
        split_tile(j, __builtin_amdgcn_readfirstlane(count - 1), b, h, t);
    }
    // locate_uniform for 0 <= j < T, also giving the sequence's length L; the
    // prefix and length of the sequence found come from the lane that read
    // them, not from a second LDS read, and the arithmetic is 32-bit (H P_b
    // <= T < 2^31; the head index is below H <= 4096, with H n <= T).
    // Prefixes are non-decreasing, so the lanes at or before j are the first
    // `cnt` of each chunk, and a chunk with none ends the search in the
    // previous chunk's last lane.
    __device__ __forceinline__ void locate_uniform_len(int64_t j, int& b, int& h, int& t, int& L) const {
        const int lane = threadIdx.x & 63;
        const uint32_t uj = static_cast<uint32_t>(j);
        int at = 0, p = 0, l = 0;
        for (int b0 = 0; b0 < B; b0 += 64) {
            const int bb = b0 + lane;
            int pc = INT32_MAX, lc = 0;
            if (bb < B) {
                pc = H * pb[bb];
                lc = len[bb];
            }
            const int cnt = __popcll(__ballot(static_cast<uint32_t>(pc) <= uj));
            if (cnt > 0) {
                at = b0 + cnt - 1;
                p = __builtin_amdgcn_readlane(pc, cnt - 1);
                l = __builtin_amdgcn_readlane(lc, cnt - 1);
            }
            if (cnt < 64) break;
        }
        b = at;
        L = l;
        const uint32_t n = static_cast<uint32_t>(tiles_of(l));
        const uint32_t r = uj - static_cast<uint32_t>(p);   // < H n
        const uint32_t hh = __builtin_amdgcn_readfirstlane(quot_u32(r, n, static_cast<uint32_t>(H - 1)));
        h = static_cast<int>(hh);
        t = static_cast<int>(r - hh * n);
    }
    // k such that worker w (whose range starts at tile `t_first` of unit
    // (b, h)) is the k-th worker of that unit
    __device__ __forceinline__ int rank_in_unit(int w, int b, int h, int t_first) const {
        if (static_cast<int64_t>(W) > T) return t_first;
        if (c != 0) return w - owner_at_cost(unit_cost_start(b, h) + 4 + c);
        return w - owner(unit_start(b, h));
    }
};

// Block-wide exclusive scan of arr[0..count) in LDS (NT threads, all must
// call); returns the total.  s_tmp needs NT / 64 ints.
template <int NT>
__device__ int block_scan_inplace(int32_t* arr, int count, int32_t* s_tmp) {
    const int t = threadIdx.x;
    const int per = (count + NT - 1) / NT;
    const int lo = t * per;
    const int hi = min(count, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += arr[i];
    const int incl = __ockl_wfscan_add_i32(sum, true);
    __syncthreads();   // s_tmp may still be read by an earlier call
    if ((t & 63) == 63) s_tmp[t >> 6] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < (t >> 6); ++w) run += s_tmp[w];
    for (int i = lo; i < hi; ++i) {
        const int x = arr[i];
        arr[i] = run;
        run += x;
    }
    int total = 0;
    for (int w = 0; w < NT / 64; ++w) total += s_tmp[w];
    __syncthreads();
    return total;
}

// Walks one worker's tiles in order, entry by entry.  Device-scheduled form:
// the entries come from the worker's tile range; a host-planned form with the
// same interface reads them from the plan words (decode_kernels.hip).
struct TileRef {
    int b, h, t;       // sequence, kv head, tile of the unit
    int L;             // sequence length
    bool first, last;  // first / last tile of its entry
    int part;          // -1: direct output; >= 0: partial slot
};

// Device-scheduled walker.  Partial slots are worker-indexed: a split entry
// is either the worker's first entry (slot 2w) or its last (slot 2w + 1) —
// only those two can extend past the worker's range.
struct DeviceWalker {
    const Sched* s;
    int w;                   // this worker
    int b, h, t, n;          // next tile to hand out; n = tiles of sequence b
    int L;                   // length of sequence b
    int64_t remaining;       // tiles of the worker not yet handed out
    bool at_start;           // the next tile is the worker's first
    int cur_part;            // of the entry holding the next tile

    __device__ __forceinline__ void start_entry(bool worker_first) {
        const bool split = (t > 0) || (static_cast<int64_t>(n - t) > remaining);
        cur_part = split ? 2 * w + (worker_first ? 0 : 1) : -1;
    }

    // wave_uniform: begin is the same in every lane and the whole wave is active
    __device__ __forceinline__ void init(const Sched& sched, int worker, int64_t begin, int64_t end,
                                         bool wave_uniform) {
        int b0 = 0, h0 = 0, t0 = 0;
        if (end > begin) {
            if (wave_uniform) sched.locate_uniform(begin, b0, h0, t0);
            else sched.locate(begin, b0, h0, t0);
        }
        init_at(sched, worker, begin, end, b0, h0, t0);
    }
    // the same, with the first tile's sequence, head and tile already known
    // (L0 >= 0: the length of sequence b0, already read)
    __device__ __forceinline__ void init_at(const Sched& sched, int worker, int64_t begin, int64_t end, int b0,
                                            int h0, int t0, int L0 = -1) {
        s = &sched;
        w = worker;
        remaining = end - begin;
        at_start = true;
        if (remaining > 0) {
            b = b0;
            h = h0;
            t = t0;
            L = L0 >= 0 ? L0 : sched.len[b];
            n = tiles_of(L);
            start_entry(true);
        } else {
            b = h = t = n = L = 0;
            cur_part = -1;
        }
    }

    __device__ __forceinline__ bool next(TileRef& r) {
        if (remaining <= 0) return false;
        r.b = b;
        r.h = h;
        r.t = t;
        r.L = L;
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
                do { ++b; } while (s->len[b] == 0);
                L = s->len[b];
                n = tiles_of(L);
            }
            start_entry(false);
        }
        return true;
    }
};

}  // namespace hpcd
