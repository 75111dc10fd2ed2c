/*
 * hpc_decode.h — C ABI of the load-balanced paged GQA decode-attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  One decode step of attention over a paged KV cache: for
 * every sequence b and query head hq (KV head h = hq / G, G = Hq / H_kv)
 *
 *     out[b, hq] = softmax_t(sm_scale * <q[b, hq], k_scale * K_t>) . (v_scale * V_t)
 *     lse[b, hq] = ln sum_t exp(sm_scale * <q[b, hq], k_scale * K_t>)
 *
 * over the L_b cached tokens t of sequence b, with K_t / V_t read from page
 * block_table[b, t / 64], row t % 64.  An empty sequence gives out = 0 and
 * lse = -inf.  The schedule follows the per-step load-balanced decode
 * scheduler of "vLLM x HPC-Ops: High-Performance Attention and MoE Backends
 * from Tencent Hunyuan", §Attention Backend: Dynamic Load-Balanced
 * Scheduling: every sequence's KV is cut into uniform 64-token tiles, the
 * tiles are spread evenly over a persistent grid, and a sequence split over
 * several workers is merged from its partial (o, lse) results by log-sum-exp
 * (the merge itself is not described on the pages; log-sum-exp is the
 * reading used here).  Head shape: 64 query heads over 8 KV heads, head dim
 * 128 ("vLLM und Tencent Hunyuan streamen zwei HPC-Backends ...",
 * §Zwei neue HPC-Backends im vLLM-Ökosystem); page size 64 and the
 * fp8_e4m3 cache come from §Using HPC-Ops Backends in vLLM.
 *
 * Conventions for every entry point
 *  - Status codes are returned, never thrown; 0 is success, negatives are
 *    the HPC_ERR_* values below.  Every condition checkable on the host is
 *    checked before any HIP call, and nothing is launched on failure.
 *  - Every buffer belongs to the caller.  The library allocates no device
 *    memory, keeps no state between calls (apart from the optional
 *    profiling window below) and never synchronises the stream.
 *  - "device" pointers must be device memory usable on the current HIP
 *    device; "host" pointers are ordinary CPU memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - Calls are thread-safe except the profiling window, which is global.
 */
#ifndef HPC_DECODE_H
#define HPC_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define HPC_OK                 0
#define HPC_ERR_NULL          -1   /* a required pointer is NULL                     */
#define HPC_ERR_INVALID       -2   /* a size / count / length is out of range        */
#define HPC_ERR_UNSUPPORTED   -3   /* head_dim != 128, page != 64, G > 16, dtype ... */
#define HPC_ERR_PLAN_MISMATCH -4   /* plan header disagrees with the call            */
#define HPC_ERR_TOO_SMALL     -5   /* plan buffer or workspace too small             */
#define HPC_ERR_HIP           -6   /* a HIP runtime call or kernel launch failed     */

/* ---- KV-cache element types --------------------------------------------- */
#define HPC_KV_BF16      0   /* bfloat16                                            */
#define HPC_KV_FP8_E4M3  1   /* OCP FP8 E4M3FN (torch.float8_e4m3fn), x = code*scale */

/* ---- Tile arithmetic (how a tile's scores and P V are computed) ---------- */
#define HPC_TILE_MATH_MFMA  0   /* matrix cores: QK^T and P V as 16x16 bf16 MFMA tiles  */
#define HPC_TILE_MATH_VALU  1   /* vector ALU only: bf16 dot2 products; needs G <= 8    */

#define HPC_DECODE_HEAD_DIM   128
#define HPC_DECODE_PAGE       64   /* tokens per page = tokens per scheduling tile */
#define HPC_DECODE_MAX_GROUP  16   /* query heads per KV head supported            */
#define HPC_PLAN_HEADER_WORDS 16
#define HPC_PLAN_VERSION      1

/* Shapes and scales of one decode step. */
typedef struct hpc_decode_params {
    int32_t num_q_heads;        /* Hq; a multiple of num_kv_heads, Hq / H_kv <= 16   */
    int32_t num_kv_heads;       /* H_kv >= 1                                         */
    int32_t head_dim;           /* must be 128                                       */
    int32_t page_size;          /* must be 64                                        */
    int32_t max_pages_per_seq;  /* row stride of block_table, in int32 elements      */
    int32_t num_pages;          /* physical pages in k_cache and v_cache (>= 1)      */
    int32_t kv_dtype;           /* HPC_KV_BF16 or HPC_KV_FP8_E4M3                    */
    float   sm_scale;           /* softmax scale, normally 1/sqrt(head_dim)          */
    float   k_scale;            /* per-tensor dequantisation scale of K (1 for bf16) */
    float   v_scale;            /* per-tensor dequantisation scale of V (1 for bf16) */
    int32_t tile_math;          /* HPC_TILE_MATH_MFMA (0, the default) or          */
                                /* HPC_TILE_MATH_VALU; both compute the same       */
                                /* attention, the kernel being HBM-bound either    */
                                /* way; VALU with G > 8 is HPC_ERR_UNSUPPORTED     */
    int32_t fused_merge;        /* 0 (default): split sequences are merged by a    */
                                /* second kernel.  1: hpc_decode_step only; the    */
                                /* worker that finishes a split unit last merges   */
                                /* it, and no second kernel runs.  Pays off when   */
                                /* few workers share a unit (short sequences);     */
                                /* correct for any batch.  The step's workspace    */
                                /* must be zero-filled before its first use with   */
                                /* this mode, and every step leaves it so.  The    */
                                /* host-planned entry points return                */
                                /* HPC_ERR_UNSUPPORTED for 1; other values are     */
                                /* HPC_ERR_INVALID.                                */
    int32_t entry_price;        /* the partition's price of a unit start, in       */
                                /* quarter tiles, 0 .. HPC_DECODE_MAX_ENTRY_PRICE  */
                                /* (else HPC_ERR_INVALID): 0 (default) gives equal */
                                /* tile shares, > 0 the priced partition of        */
                                /* hpc_decode_plan_priced.  Used where the library */
                                /* partitions: hpc_decode_step (on the device) and */
                                /* hpc_decode_plan_attn; hpc_decode_attn follows   */
                                /* the plan it is given.                           */
} hpc_decode_params;

#define HPC_DECODE_MAX_ENTRY_PRICE 64   /* quarter tiles: 16 tiles per unit start */

/*
 * Upper bound, in int32 words, of the plan for this batch shape:
 * 16 + (W + 1) + 4 (W + U) + 3 U with U = batch * num_kv_heads, W = n_workers
 * (a work list holds at most W + U - 1 entries and at most U merge records).
 * The plan is the work list of the per-step scheduler of "vLLM x HPC-Ops
 * ...", §Attention Backend: Dynamic Load-Balanced Scheduling (tiles spread
 * evenly over a persistent grid); the bound lets a caller size the plan
 * buffer once per batch shape, before the lengths are known.
 * Returns a negative status for batch < 0, num_kv_heads < 1 or n_workers < 1.
 */
int64_t hpc_decode_plan_size(int32_t batch, int32_t num_kv_heads, int32_t n_workers);

/*
 * Per-step scheduler (§Attention Backend: Dynamic Load-Balanced Scheduling;
 * the German page, §Warum ist dynamisches Scheduling entscheidend für
 * Attention?, adds that tiles follow each sequence's length in the current
 * step).  Pure host code; no HIP call.
 *
 * seq_lens   host int32[batch], KV lengths of this step (>= 0).
 * plan       host int32[plan_capacity] output.
 *
 * Units u = b * num_kv_heads + h each hold n_u = ceil(L_b / 64) tiles; with
 * T = sum n_u, worker w (0 <= w < n_workers) owns tiles
 * [floor(w T / W), floor((w + 1) T / W)) of the unit-major tile list, cut
 * at unit boundaries into entries.  Layout (int32 words):
 *   header[16]      {version=1, batch, H_kv, W, T, E, n_partials, n_combine, 64, 0...}
 *   worker_ptr[W+1] worker w's entries are [worker_ptr[w], worker_ptr[w+1])
 *   entries[E][4]   (unit, t0, t1, slot): tiles [t0, t1) of the unit; slot -1
 *                   means this entry is the unit's only one and writes out/lse
 *                   directly, otherwise it writes partial number `slot`
 *   combine[n_combine][3]  (unit, S_u, base_u) for every unit with S_u != 1
 *                   entries: S_u >= 2 partials in slots [base_u, base_u + S_u),
 *                   or S_u = 0 for an empty sequence
 * Errors: NULL pointers, batch < 0, H_kv < 1, W < 1, a negative length, or
 * T >= 2^31 -> HPC_ERR_NULL / HPC_ERR_INVALID; capacity below the words the
 * plan needs -> HPC_ERR_TOO_SMALL.  On error `plan` is left unspecified.
 */
int hpc_decode_plan(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                    int32_t n_workers, int32_t* plan, int64_t plan_capacity);

/*
 * The scheduler above with the partition priced.  It extends the rule of
 * §Attention Backend: Dynamic Load-Balanced Scheduling ("vLLM x HPC-Ops:
 * High-Performance Attention and MoE Backends from Tencent Hunyuan"), which
 * spreads tiles by actual work; the pages price tiles only.  A worker pays for every unit it starts as
 * well as for its tiles: the entry's end, the Q reload and, for a split
 * unit, a partial.  Tile j costs 4 (quarter tiles), plus entry_price when it
 * is the first tile of its unit; with A(j) the cost of tiles 0 .. j-1 and
 * C = A(T), worker w starts at the largest j with A(j) <= floor(w C / W).
 * entry_price = 0 is hpc_decode_plan word for word.  The price applies only
 * when W <= T, C >= (4 + entry_price + 1) W (no worker is left without
 * tiles) and C < 2^31; otherwise the plan is the plain one.  Header word 9
 * holds the price applied (0 when declined).  Errors as hpc_decode_plan,
 * plus HPC_ERR_INVALID for entry_price outside 0 .. HPC_DECODE_MAX_ENTRY_PRICE.
 */
int hpc_decode_plan_priced(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                           int32_t n_workers, int32_t entry_price, int32_t* plan,
                           int64_t plan_capacity);

/*
 * Static split-KV schedule in the same word layout, for comparison with the
 * balanced one (the pages measure their scheduler against a static split-KV
 * schedule, §Attention Decode under Mixed-Length Batches, without defining
 * it; this is the common form).  Pure host code; no HIP call.
 *
 * Every unit with n_u >= 1 tiles is cut into shares of c_u = ceil(n_u /
 * splits) tiles, [k c_u, min((k + 1) c_u, n_u)); every non-empty share is
 * one worker holding one entry, in (unit, share) order, so W = number of
 * shares (at least 1: an all-empty batch keeps one idle worker).  Slots and
 * merge records follow the same rule as hpc_decode_plan.  The plan runs
 * through hpc_decode_attn like any other.
 * hpc_decode_plan_static_size: a word bound for (batch, num_kv_heads,
 * splits), or a negative status for batch < 0, H_kv < 1 or splits < 1.
 * Errors of hpc_decode_plan_static as for hpc_decode_plan (splits < 1 ->
 * HPC_ERR_INVALID).
 */
int64_t hpc_decode_plan_static_size(int32_t batch, int32_t num_kv_heads, int32_t splits);
int hpc_decode_plan_static(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                           int32_t splits, int32_t* plan, int64_t plan_capacity);

/* Worker count for a step, pure host code.  The balanced partition gives
 * every worker floor((w+1)T/W) - floor(wT/W) tiles (§Attention Backend:
 * Dynamic Load-Balanced Scheduling, "vLLM x HPC-Ops: High-Performance
 * Attention and MoE Backends from Tencent Hunyuan": tiles spread by actual
 * work over a grid that keeps every compute unit busy), but a worker also
 * pays for each entry (unit) its range touches: the entry's end and, when
 * the unit is split, its partial.  This returns the W in [min_workers,
 * max_workers] whose costliest worker, priced as its tiles plus entry_cost
 * tiles per entry, is cheapest: scanning down from max_workers, a smaller W
 * replaces the best so far only when it prices at least HPC_DECODE_MIN_GAIN
 * (1%) below it, so near-ties keep the larger W.  With the lengths
 * of a batch whose sequence boundaries fall on worker boundaries at some W
 * just below the compute-unit count, that W wins (one entry per worker).
 * The pages price tiles only; entry_cost is this library's extension
 * (about 0.5 measured on MI355X: ~0.6 us per entry end against ~1.25 us
 * per 32 KiB tile).  Returns W (>= 1), or HPC_ERR_NULL (NULL lengths with
 * batch > 0), HPC_ERR_INVALID (batch < 0, num_kv_heads < 1, min_workers < 1,
 * max_workers < min_workers, entry_cost negative or not finite, a negative
 * length, 2^31 - 1 tiles or more).  An all-empty batch returns max_workers. */
int32_t hpc_decode_choose_workers(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                                  int32_t min_workers, int32_t max_workers, float entry_cost);

/* The entry price of the worker-count rules, in tiles (about 0.6 us per
 * entry end against about 1.25 us per 32 KiB tile, measured on MI355X), and
 * the least relative gain for which the rule leaves more compute units idle
 * (a bf16 64q/8kv batch priced 0.25% cheaper at 255 workers measured 0.5%
 * slower than at 256). */
#define HPC_DECODE_ENTRY_COST 0.5f
#define HPC_DECODE_MIN_GAIN 0.01

/* The entry cost, in tiles, of hpc_decode_pick_entry_price on an fp8 cache:
 * a 16 KiB fp8 tile streams in about half a bf16 tile's time while an entry
 * end costs the same, so an entry weighs four times as many tiles (fitted on
 * MI355X: 32 sequences of 64q/8kv fp8, lengths log-uniform in [128, 65536],
 * fastest at 8 quarter tiles per unit start, at W = 256 and at W = 512). */
#define HPC_DECODE_ENTRY_COST_FP8 2.0f
/* Worker count for a device-scheduled step on a GPU with n_cus compute
 * units (>= 2), pure host code: the size of the persistent grid that keeps
 * every compute unit busy (§Attention Backend: Dynamic Load-Balanced
 * Scheduling, "vLLM x HPC-Ops: High-Performance Attention and MoE Backends
 * from Tencent Hunyuan").  W1 = hpc_decode_choose_workers over
 * [n_cus / 2, n_cus] with HPC_DECODE_ENTRY_COST.  On an fp8 cache whose
 * W1-worker partition has 1.5 entries per worker or more, it returns
 * 2 n_cus instead: two co-resident workgroups per compute unit then hide
 * entry ends and fp8's narrower loads better than one (measured on MI355X:
 * 32 sequences of 64q/8kv fp8, lengths log-uniform in [128, 65536], 154.7 ->
 * 145.5 us; on bf16 caches and on fp8 batches with about one entry per
 * worker, one workgroup per CU was as fast or faster).  The count is a
 * multiple of n_cus in that case: with W between n_cus and 2 n_cus some
 * compute units carry two workers and others one.  Errors as
 * hpc_decode_choose_workers, plus HPC_ERR_INVALID for n_cus < 2 or above
 * 2^20 and HPC_ERR_UNSUPPORTED for an unknown kv_dtype. */
int32_t hpc_decode_pick_workers(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads, int32_t kv_dtype,
                                int32_t n_cus);

/* Entry price for a step of n_workers workers (the params field
 * entry_price), pure host code; the price extends the work-based tile
 * spreading of §Attention Backend: Dynamic Load-Balanced Scheduling ("vLLM
 * x HPC-Ops ...").  Among the prices 0, 2, 4, 8 and 16 quarter
 * tiles, each partition (hpc_decode_plan_priced) is priced by its costliest
 * worker, as its tiles plus an entry cost per unit its range touches
 * (HPC_DECODE_ENTRY_COST on a bf16 cache, HPC_DECODE_ENTRY_COST_FP8 on fp8).
 * Scanning up from 0, a price replaces the best so far only when its
 * partition prices at least HPC_DECODE_MIN_GAIN below it, and a price the
 * partition declines is skipped, so a batch whose plain partition already
 * fits unit boundaries keeps price 0.  Returns the price (>= 0), or
 * HPC_ERR_NULL, HPC_ERR_INVALID (batch < 0, num_kv_heads < 1, n_workers < 1,
 * a negative length, 2^31 - 1 tiles or more) or HPC_ERR_UNSUPPORTED (an
 * unknown kv_dtype). */
int32_t hpc_decode_pick_entry_price(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                                    int32_t kv_dtype, int32_t n_workers);

/* The most workers that may share one sequence-head unit for
 * hpc_decode_pick_merge to keep the merge in the decode kernel. */
#define HPC_DECODE_FUSED_MAX_SHARES 8

/* Merge mode for a device-scheduled step (the params field fused_merge),
 * pure host code.  Split-KV decode merges a sequence split over several
 * workers from their partial results (§Attention Backend: Dynamic
 * Load-Balanced Scheduling, "vLLM x HPC-Ops: High-Performance Attention and
 * MoE Backends from Tencent Hunyuan"; the log-sum-exp merge is the reading
 * used here).  Over the partition the step will use (n_workers workers,
 * entry_price applied as hpc_decode_plan_priced applies it), it counts the
 * workers whose tile range meets each (sequence, KV head) unit.  Returns 1
 * (merge in the decode kernel) when no unit is split, or when the batch has
 * no more tiles than workers (each worker holds at most one) and no unit is
 * shared by more than HPC_DECODE_FUSED_MAX_SHARES workers; else 0 (merge
 * kernel).  Measured on MI355X as whole steps (W = 256 and the worker-count
 * rule's W): batches of 10 to 128 tiles with 2 to 8 workers per unit ran
 * 0.2-0.8 us faster with the in-kernel merge; batches with more tiles than
 * workers ran as fast or up to 0.4 us faster with the merge kernel, and
 * units shared by 16 or more workers up to 14 us faster, since the last
 * worker folds all of a unit's partials alone.
 * For hpc_decode_step; hpc_decode_step_noalloc takes fused_merge = 0 only.
 * Negative status: HPC_ERR_NULL for NULL lengths with batch > 0,
 * HPC_ERR_INVALID for batch < 0, num_kv_heads < 1, n_workers < 1,
 * entry_price outside 0 .. HPC_DECODE_MAX_ENTRY_PRICE, a negative length or
 * 2^31 - 1 tiles or more. */
int32_t hpc_decode_pick_merge(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads, int32_t n_workers,
                              int32_t entry_price);

/* Split count of the static split-KV baseline for a batch: the smallest
 * power of two S with batch * num_kv_heads * S >= n_cus (one share per
 * compute unit at least), capped at max_splits and at the largest unit's
 * tile count (the pages leave the static heuristic open; this is the rule
 * used here).  Negative status for NULL lengths, batch < 0, H_kv < 1,
 * n_cus < 1, max_splits < 1 or a negative length. */
int32_t hpc_decode_static_splits(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads, int32_t n_cus,
                                 int32_t max_splits);

/* Words actually used by a plan written by hpc_decode_plan (the work list
 * of §Attention Backend: Dynamic Load-Balanced Scheduling, "vLLM x HPC-Ops
 * ..."; from its header), or a negative status for a NULL pointer or a
 * malformed header. */
int64_t hpc_decode_plan_words(const int32_t* plan);

/*
 * Device workspace, in bytes, that hpc_decode_attn needs for this plan:
 * n_partials * G * 128 fp32 partial outputs followed (256-byte aligned) by
 * n_partials * G fp32 partial log-sum-exps.  0 when no sequence is split.
 * The partials are those of sequences the scheduler of §Attention Backend:
 * Dynamic Load-Balanced Scheduling ("vLLM x HPC-Ops ...") spreads over
 * several workers; the pages do not describe how they are combined, and the
 * log-sum-exp merge is the reading used here.  plan is host memory (the
 * words of hpc_decode_plan or hpc_decode_plan_static); a negative status is
 * returned for a NULL or malformed plan or heads that do not group.
 */
int64_t hpc_decode_workspace_size(const int32_t* plan, int32_t num_q_heads,
                                  int32_t num_kv_heads);

/*
 * One decode step on `stream`: the persistent decode kernel (grid = the
 * plan's W workgroups, each walking its entries), then, when the plan has
 * merge records, the log-sum-exp merge kernel.  This is the attention of
 * "vLLM x HPC-Ops ...", §Attention Backend: Dynamic Load-Balanced
 * Scheduling, run over a plan made by hpc_decode_plan: each worker streams
 * its 64-token tiles of K and V (one page each) and keeps an online softmax;
 * a sequence held by several workers is merged by log-sum-exp.  The decode
 * shapes measured on the pages (§Attention Decode under Mixed-Length
 * Batches) are 64 x 0.5K and 1 x 128K + 31 x 4K tokens.
 *
 * q            device bf16 [batch][Hq][128], contiguous
 * k_cache      device bf16 or fp8 [num_pages][H_kv][64][128], contiguous
 * v_cache      same layout and type as k_cache
 * block_table  device int32 [batch][max_pages_per_seq]; entries of tiles the
 *              plan covers must lie in [0, num_pages) (others are never read;
 *              an id outside that range is read as a page of zeros)
 * seq_lens     device int32 [batch]; must equal the lengths the plan was made from
 * plan_host    host copy of the plan (sizes the grids without a device sync)
 * plan_dev     device copy of the same words
 * workspace    device, >= hpc_decode_workspace_size bytes (may be NULL if that is 0)
 * out          device bf16 [batch][Hq][128]
 * lse          device fp32 [batch][Hq], natural log
 * The host checks the plan against the call (version, H_kv, entry bounds
 * against max_pages_per_seq) before launching.  All device buffers must
 * stay valid until the stream work completes; plan_host only until return.
 */
int hpc_decode_attn(const hpc_decode_params* params, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                    const int32_t* plan_host, const int32_t* plan_dev, void* workspace,
                    int64_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * The host-side checks of hpc_decode_attn (the decode step of §Attention
 * Backend: Dynamic Load-Balanced Scheduling, "vLLM x HPC-Ops ...") alone,
 * with the same arguments
 * (no stream): returns the status hpc_decode_attn would return before
 * launching anything.  Never calls HIP and never dereferences device pointers.
 */
int hpc_decode_check(const hpc_decode_params* params, const void* q, const void* k_cache,
                     const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                     const int32_t* plan_host, const int32_t* plan_dev, const void* workspace,
                     int64_t workspace_bytes, const void* out, const float* lse);

/*
 * Workspace, in bytes, that is enough for hpc_decode_attn (the split-KV
 * partials of §Attention Decode under Mixed-Length Batches, "vLLM x HPC-Ops
 * ...") under any plan of
 * this batch size and worker count (a plan has at most W + B*H_kv - 1
 * entries, so at most that many partial slots).  Negative status for
 * batch < 0, n_workers < 1 or heads that do not group.
 */
int64_t hpc_decode_plan_workspace_bound(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t n_workers);

/*
 * A host-planned decode step in one call, for callers that hold the step's
 * lengths on the host (the per-step scheduler of §Attention Backend: Dynamic
 * Load-Balanced Scheduling, then the attention): hpc_decode_plan of
 * seq_lens_host into plan_host, the host checks of hpc_decode_attn, an
 * asynchronous copy of the plan's words to plan_dev queued on `stream`, and
 * the kernels of hpc_decode_attn on the same stream.
 *
 * seq_lens_host  host int32 [batch]: the lengths seq_lens (device) holds
 * plan_host      host buffer of plan_capacity >= hpc_decode_plan_size words.
 *                Pinned memory (hipHostMalloc) makes the copy asynchronous;
 *                the caller must not rewrite the buffer until that copy has
 *                executed on the stream (two buffers used in turn, each
 *                guarded by an event recorded after the call, suffice)
 * plan_dev       device buffer of at least as many words, valid until the
 *                stream work completes; or plan_host itself, when plan_host
 *                is pinned memory mapped at the same address on the device
 *                (hipHostMalloc, torch pin_memory): the kernels then read the
 *                plan in place, over the host link, no copy is queued, and
 *                the buffer must stay unchanged until the kernels have run.
 *                Any other host pointer passed as plan_dev is HPC_ERR_INVALID
 * workspace      device, >= hpc_decode_workspace_size of the plan made here
 *                (hpc_decode_plan_workspace_bound is always enough)
 * Other arguments as for hpc_decode_attn.  Every check (planner arguments,
 * plan against params, workspace size, the in-place pointer query) runs
 * before anything is queued; a failed copy or launch returns HPC_ERR_HIP.
 */
int hpc_decode_plan_attn(const hpc_decode_params* params, const int32_t* seq_lens_host, int32_t batch,
                         int32_t n_workers, int32_t* plan_host, int64_t plan_capacity, int32_t* plan_dev,
                         const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                         const int32_t* seq_lens, void* workspace, int64_t workspace_bytes, void* out,
                         float* lse, void* stream);

/*
 * Device-scheduled decode step (no host plan).  The same per-step schedule
 * as hpc_decode_plan (§Attention Backend: Dynamic Load-Balanced Scheduling)
 * is derived inside the decode kernel from the device copy of the lengths:
 * every workgroup scans the tile counts of the batch in LDS and finds its
 * own tile range and entries.  A split entry writes its partial result to a
 * worker-indexed slot; the worker holding a sequence's first tile writes that
 * sequence's merge record (how many workers share it, which is the first),
 * and the merge kernel launched after it combines the partials by
 * log-sum-exp.  Empty sequences are written by the decode kernel.  Every
 * record is rewritten at every call.
 * Nothing crosses from the host per step except the two launches, so the
 * call can be captured in a HIP graph.
 *
 * batch        sequences in q / block_table / seq_lens (1 .. 2048, and
 *              batch * H_kv <= 4096)
 * n_workers    persistent workgroups W (the plan's W), 1 .. 65536
 * seq_lens     device int32 [batch]; lengths are clamped to
 *              [0, max_pages_per_seq * 64] so no read leaves the block table
 * workspace    device, >= hpc_decode_step_workspace_size(batch, Hq, H_kv, W);
 *              calls that may run concurrently (other streams) need
 *              separate workspaces.  With params->fused_merge = 1 the merge
 *              kernel is not launched: the decode kernel's last worker to
 *              finish a split sequence merges it, counting arrivals in the
 *              workspace, which must be zero-filled before its first use in
 *              that mode (every call leaves the counts at zero)
 * Other arguments as for hpc_decode_attn.  Errors as hpc_decode_attn, plus
 * HPC_ERR_UNSUPPORTED beyond those limits and HPC_ERR_INVALID when
 * batch * max_pages_per_seq * H_kv does not fit in int32.
 */
int hpc_decode_step(const hpc_decode_params* params, int32_t batch, int32_t n_workers, const void* q,
                    const void* k_cache, const void* v_cache, const int32_t* block_table,
                    const int32_t* seq_lens, void* workspace, int64_t workspace_bytes, void* out,
                    float* lse, void* stream);

/* The host-side checks of hpc_decode_step (§Attention Backend: Dynamic
 * Load-Balanced Scheduling, "vLLM x HPC-Ops ...") alone (never calls HIP). */
int hpc_decode_step_check(const hpc_decode_params* params, int32_t batch, int32_t n_workers,
                          const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens, const void* workspace,
                          int64_t workspace_bytes, const void* out, const float* lse);

/* Workspace bytes hpc_decode_step needs for any lengths (the partials of
 * sequences split over workers, which the pages' split-KV decode merges:
 * §Attention Decode under Mixed-Length Batches, "vLLM x HPC-Ops ..."): P = 2 W partial
 * slots (a worker's first and last entries are the only ones that can be
 * split, and they use slots 2w and 2w + 1): fp32 outputs [P][G][128], then
 * (256-byte aligned) fp32 lse [P][G], then (aligned) int32 merge records
 * [batch * H_kv][6]. */
int64_t hpc_decode_step_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t n_workers);

/*
 * hpc_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results as hpc_decode_step, with the step's scratch
 * (partial outputs, partial log-sum-exps and merge records, the layout of
 * hpc_decode_step_workspace_size) held in a fixed device array that the
 * library owns instead of a workspace argument.  The call allocates nothing
 * and frees nothing.
 *
 * The array holds hpc_decode_step_noalloc_max_bytes() bytes (16 MiB) on every
 * GPU the library runs on, kept until the process ends.  Shapes whose
 * hpc_decode_step_workspace_size exceeds it return HPC_ERR_TOO_SMALL before
 * any HIP call (for example W = 1024 workers with G = 16 heads per KV head);
 * W = 256 fits up to G = 16, W = 1024 up to G = 8.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls that can overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.  Nothing in the array has
 * to start at zero: every merge record the step reads is written by the same
 * call.  params->fused_merge must be 0 (the in-kernel merge keeps arrival
 * counts between calls; 1 returns HPC_ERR_UNSUPPORTED).  The array's device
 * address is looked up on the first call on each device, with the stream's
 * device current; a failed lookup returns HPC_ERR_HIP.
 * Other arguments, limits and errors as hpc_decode_step.
 */
int hpc_decode_step_noalloc(const hpc_decode_params* params, int32_t batch, int32_t n_workers, const void* q,
                            const void* k_cache, const void* v_cache, const int32_t* block_table,
                            const int32_t* seq_lens, void* out, float* lse, void* stream);

/* Bytes of the fixed scratch array of hpc_decode_step_noalloc (per GPU). */
int64_t hpc_decode_step_noalloc_max_bytes(void);

/*
 * The device-derived schedule (§Attention Backend: Dynamic Load-Balanced
 * Scheduling, "vLLM x HPC-Ops ...") written out on `stream` into device `plan`
 * (int32 words, capacity >= hpc_decode_plan_size) in exactly the layout of
 * hpc_decode_plan_priced with the same entry_price, so the two can be
 * compared word for word.  One
 * workgroup; limits: batch <= 2048, n_workers <= 2048, batch * H_kv <= 4096
 * (else HPC_ERR_UNSUPPORTED).  Lengths are clamped as in hpc_decode_step.
 */
int hpc_decode_plan_device(const int32_t* seq_lens, int32_t batch, int32_t num_kv_heads,
                           int32_t n_workers, int32_t entry_price, int32_t max_pages_per_seq,
                           int32_t* plan, int64_t plan_capacity, void* stream);

/* Human-readable name of a status code (static storage). */
const char* hpc_status_string(int status);

/*
 * Optional profiling window (measurement only; global state guarded by a
 * lock).  Between start and stop every hpc_decode_attn or hpc_decode_step
 * call launches its decode kernel and its merge kernel with a pair of HIP
 * events that the dispatch itself stamps at the kernel's start and end (the
 * kernel's own execution time, not the queue gaps around it; at most
 * `capacity` calls are recorded).  stop synchronises those events and
 * returns the summed kernel durations in ms and the number of calls
 * recorded.  Returns HPC_ERR_HIP on event failures.
 */
int hpc_decode_profile_start(int32_t capacity);
int hpc_decode_profile_stop(double* decode_ms, double* combine_ms, int32_t* n_calls);

/*
 * Tracing window (measurement only).  While it is on, every decode-kernel
 * launch with W workers, W * 64 <= bytes, records for each worker w eight
 * uint64 words at device_buffer + 8 w: stamps of the device's constant
 * wall clock (hipDeviceAttributeWallClockRate, 100 MHz on MI355X) at kernel
 * entry, once the first ring slots' loads are issued, after the first tile
 * is consumed, after the last, and at the end (entry merges and any
 * in-kernel merge done); then the worker's tile count (device schedule; 0
 * with a host plan), its entry count, and where it ran: the XCC_ID hardware
 * register in the high 32 bits, HW_ID (CU, shader array and engine ids) in
 * the low 32.  Workers without tiles leave their words untouched.  Each
 * launch overwrites the buffer (device memory, caller-owned, valid while
 * the window is on); a launch with more workers than it holds records
 * nothing.  Stamps of workers on different XCDs are not comparable (their
 * clocks differ by up to about 2 us); durations within one worker are.
 * Inside the window the launches use a separate instantiation of the decode
 * kernel that takes the stamps; outside it the untraced kernel runs, with
 * no trace code at all.  Errors: HPC_ERR_NULL, HPC_ERR_INVALID (bytes <
 * 64).  No HIP call.
 */
int hpc_decode_trace_start(void* device_buffer, int64_t bytes);
int hpc_decode_trace_stop(void);

/* Rate of the clock the tracing stamps count, in Hz, for the current device
 * (hipDeviceAttributeWallClockRate); HPC_ERR_HIP if HIP cannot report it. */
int64_t hpc_decode_wall_clock_hz(void);

#ifdef __cplusplus
}
#endif

#endif /* HPC_DECODE_H */
