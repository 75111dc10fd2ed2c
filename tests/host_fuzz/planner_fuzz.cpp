// Host-only fuzz of the library's planners, built with
// AddressSanitizer and UBSan by tests/test_host_sanitizers.py (no GPU, no
// HIP runtime).  Every plan is written into a buffer of exactly the size its
// size query returned, so a write past the bound is caught; coverage
// invariants are checked on every plan.  The kernel launch entry points are
// stubs here.

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "hpc_decode.h"
#include "hpc_prefill.h"
#include "hpc_prologue.h"
#include "../../load_balanced_paged_step_amd/csrc/internal.h"

namespace hpcd {
int launch_prefill(const PrefillArgs&, int, int, bool, void*) { return 0; }
int launch_prologue(const PrologueArgs&, void*) { return 0; }
}  // namespace hpcd

#define CHECK(c)                                                            \
    do {                                                                    \
        if (!(c)) {                                                         \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            std::exit(1);                                                   \
        }                                                                   \
    } while (0)

int main() {
    std::mt19937_64 rng(1234);
    auto uni = [&](int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); };
    int64_t plans = 0;
    for (int it = 0; it < 3000; ++it) {
        const int32_t B = static_cast<int32_t>(uni(0, 40));
        const int32_t H = static_cast<int32_t>(uni(1, 8));
        std::vector<int32_t> lens(static_cast<std::size_t>(B) + 1);
        int64_t T = 0;
        for (int32_t b = 0; b < B; ++b) {
            const int r = static_cast<int>(uni(0, 9));
            lens[b] = r == 0 ? 0 : static_cast<int32_t>(r < 7 ? uni(1, 300) : uni(1, 20000));
            T += (int64_t(lens[b]) + 63) / 64 * H;
        }
        // decode: the balanced planner
        const int32_t W = static_cast<int32_t>(uni(1, 600));
        const int64_t cap = hpc_decode_plan_size(B, H, W);
        CHECK(cap > 0);
        std::vector<int32_t> plan(static_cast<std::size_t>(cap));
        CHECK(hpc_decode_plan(B ? lens.data() : nullptr, B, H, W, plan.data(), cap) == HPC_OK);
        CHECK(hpc_decode_plan_words(plan.data()) <= cap);
        const int32_t E = plan[5];
        int64_t covered = 0;
        for (int32_t e = 0; e < E; ++e) {
            const int32_t* en = plan.data() + HPC_PLAN_HEADER_WORDS + (W + 1) + 4 * e;
            CHECK(en[1] < en[2]);
            covered += en[2] - en[1];
        }
        CHECK(covered == T);
        ++plans;
        // the priced partition: same buffer bound, every tile once, no empty worker when applied
        const int32_t price = static_cast<int32_t>(uni(0, HPC_DECODE_MAX_ENTRY_PRICE));
        std::vector<int32_t> pplan(static_cast<std::size_t>(cap));
        CHECK(hpc_decode_plan_priced(B ? lens.data() : nullptr, B, H, W, price, pplan.data(), cap) == HPC_OK);
        CHECK(hpc_decode_plan_words(pplan.data()) <= cap);
        CHECK(pplan[9] == 0 || pplan[9] == price);
        covered = 0;
        for (int32_t e = 0; e < pplan[5]; ++e) {
            const int32_t* en = pplan.data() + HPC_PLAN_HEADER_WORDS + (W + 1) + 4 * e;
            CHECK(en[1] < en[2]);
            covered += en[2] - en[1];
        }
        CHECK(covered == T);
        if (pplan[9] != 0)
            for (int32_t w = 0; w < W; ++w) CHECK(pplan[HPC_PLAN_HEADER_WORDS + w + 1] > pplan[HPC_PLAN_HEADER_WORDS + w]);
        const int32_t pick = hpc_decode_pick_entry_price(B ? lens.data() : nullptr, B, H,
                                                         uni(0, 1) ? HPC_KV_BF16 : HPC_KV_FP8_E4M3, W);
        CHECK(pick == 0 || pick == 2 || pick == 4 || pick == 8 || pick == 16);
        // the merge mode: in-kernel when nothing is split, or with no more tiles than workers
        // and no merge record counting more than the limit
        int32_t most = 1;
        const int32_t* rec = pplan.data() + HPC_PLAN_HEADER_WORDS + (W + 1) + 4 * pplan[5];
        for (int32_t c = 0; c < pplan[7]; ++c) most = rec[3 * c + 1] > most ? rec[3 * c + 1] : most;
        CHECK(hpc_decode_pick_merge(B ? lens.data() : nullptr, B, H, W, price) ==
              ((most == 1 || (T <= W && most <= HPC_DECODE_FUSED_MAX_SHARES)) ? 1 : 0));
        ++plans;
        // the static split-KV planner
        const int32_t S = static_cast<int32_t>(uni(1, 64));
        const int64_t scap = hpc_decode_plan_static_size(B, H, S);
        CHECK(scap > 0);
        std::vector<int32_t> splan(static_cast<std::size_t>(scap));
        CHECK(hpc_decode_plan_static(B ? lens.data() : nullptr, B, H, S, splan.data(), scap) == HPC_OK);
        CHECK(hpc_decode_plan_words(splan.data()) <= scap);
        ++plans;
        // worker-count rules
        const int32_t lo = static_cast<int32_t>(uni(1, 200)), hi = lo + static_cast<int32_t>(uni(0, 60));
        const int32_t cw = hpc_decode_choose_workers(B ? lens.data() : nullptr, B, H, lo, hi, 0.5f);
        CHECK(cw >= lo && cw <= hi);
        const int32_t pw = hpc_decode_pick_workers(B ? lens.data() : nullptr, B, H,
                                                   uni(0, 1) ? HPC_KV_BF16 : HPC_KV_FP8_E4M3, hi + 1);
        CHECK(pw >= 1);
        // prefill: chunks of new tokens within the lengths
        if (B > 0) {
            std::vector<int32_t> qs(static_cast<std::size_t>(B) + 1, 0);
            for (int32_t b = 0; b < B; ++b) qs[b + 1] = qs[b] + static_cast<int32_t>(uni(0, std::min<int64_t>(lens[b], 70)));
            const int32_t maxp = static_cast<int32_t>(20000 / 64 + 2);
            const int32_t PW = static_cast<int32_t>(uni(0, 700));
            const int32_t ms = static_cast<int32_t>(uni(1, 20));
            const int64_t pcap = hpc_prefill_plan_size(qs.data(), B, H, PW);
            CHECK(pcap > 0);
            std::vector<int32_t> work(static_cast<std::size_t>(pcap));
            int32_t counts[3] = {-1, -1, -1};
            CHECK(hpc_prefill_plan(qs.data(), lens.data(), B, H, maxp, PW, ms, work.data(), pcap, counts) == HPC_OK);
            CHECK(8 * int64_t(counts[0]) + 8 * int64_t(counts[1]) <= pcap);
            int64_t tiles = 0, want = 0;
            for (int32_t e = 0; e < counts[0]; ++e) tiles += work[8 * e + 3];
            for (int32_t b = 0; b < B; ++b) {
                const int32_t n = qs[b + 1] - qs[b];
                for (int32_t j = 0; 16 * j < n; ++j) {
                    const int32_t last = lens[b] - n + std::min(16 * (j + 1), n) - 1;
                    want += int64_t(last / 64 + 1) * H;
                }
            }
            CHECK(tiles == want);
            // one word short is refused, never overrun
            if (counts[0] > 0) {
                std::vector<int32_t> tight(static_cast<std::size_t>(8 * counts[0] + 8 * counts[1] - 1));
                CHECK(hpc_prefill_plan(qs.data(), lens.data(), B, H, maxp, PW, ms, tight.data(),
                                       static_cast<int64_t>(tight.size()), counts) == HPC_ERR_TOO_SMALL);
            }
            ++plans;
        }
    }
    std::printf("fuzzed %lld plans\n", static_cast<long long>(plans));
    return 0;
}
