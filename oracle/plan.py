"""The per-step tile schedule, written out plainly (integer algorithm).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The HPC-Ops blog (§Attention Backend: Dynamic Load-Balanced Scheduling)
says the scheduler runs every decode step, cuts every KV sequence into
uniform 64-token tiles, and hands tiles to the persistent grid's workers
according to the actual work; the German retelling (§Warum ist dynamisches
Scheduling entscheidend für Attention?) adds that tiles go to compute units
in proportion to each sequence's actual length in the current generation
step.  The pages fix neither the partition rule nor the work-list format.
The reading used here (and, independently, by the C++ planner):

  1. units u = b * H_kv + h (batch-major); n_u = ceil(L_b / 64) tiles; one
     tile costs one, the last partial tile included;
  2. P = exclusive prefix sum of n_u, T = P[U];
  3. worker w owns global tiles [s_w, s_{w+1}) with s_w = floor(w * T / W);
  4. for w = 0..W-1 and, inside, increasing u, every unit whose tile range
     meets worker w's range gives one entry (u, t0, t1) of unit-local tile
     indices; worker_ptr[w + 1] is the running entry count;
  5. S_u = number of entries of unit u.  S_u = 1: slot -1 (the worker
     writes the final output).  S_u >= 2: the units with S >= 2, in
     increasing u, take consecutive blocks of partial slots; the k-th entry
     of u in entry order gets slot base_u + k.  Units with S_u != 1 are
     listed for the merge as (u, S_u, base_u), base_u = 0 when S_u = 0.

Priced partition (this build's extension; the pages price tiles only).  A
worker also pays for each unit it touches, an entry end and possibly a
partial.  With entry_cost_q = c > 0 (in quarter tiles), step 3 becomes:

  3'. tile j costs 4, plus c when j is the first tile of a unit;
      A(j) = the cost of tiles 0 .. j-1, C = A(T);
      s_w = the largest j in [0, T] with A(j) <= floor(w * C / W).

With c = 0 this is s_w = floor(w T / W) again.  c is applied only when
W <= T and C >= (4 + c + 1) W, so that every worker's share of the cost
exceeds one tile's and no worker is left without tiles, and C < 2^31.
Otherwise the plan is the plain one.

Serialised as int32 words:
  header[16] = {1, B, H_kv, W, T, E, n_partials, n_combine, 64, c applied, 0, ..., 0}
  worker_ptr[W + 1], entries[E][4] = (u, t0, t1, slot), combine[n_combine][3].

Pinned by ``tests/test_oracle_plan.py``: an independent quota-filling
construction, the coverage / balance / contiguity / slot-bijection
invariants, exhaustive small cases, and a hand-worked schedule stored
under ``tests/golden/``.
"""

from __future__ import annotations

import numpy as np

PAGE = 64
HEADER_WORDS = 16
PLAN_VERSION = 1


def plan_size_words(batch: int, num_kv_heads: int, n_workers: int) -> int:
    """Upper bound on the plan's int32 word count (E <= W + U - 1, n_combine <= U)."""
    U = batch * num_kv_heads
    return HEADER_WORDS + (n_workers + 1) + 4 * (n_workers + U) + 3 * U


TILE_COST_Q = 4    # one tile, in quarter tiles


def priced_boundaries(n_tiles_per_unit, n_workers: int, entry_cost_q: int):
    """(worker boundaries s[0..W], the entry cost applied) of the priced
    partition 3' for units of the given tile counts."""
    n, W, c = list(n_tiles_per_unit), int(n_workers), int(entry_cost_q)
    T = sum(n)
    first = set()
    start = 0
    for k in n:
        if k > 0:
            first.add(start)
        start += k
    C = TILE_COST_Q * T + c * len(first)
    if c <= 0 or W > T or C < (TILE_COST_Q + c + 1) * W or C >= 2**31:
        return [(w * T) // W for w in range(W + 1)], 0
    A = [0]                          # A[j] = cost of tiles 0 .. j-1
    for j in range(T):
        A.append(A[-1] + TILE_COST_Q + (c if j in first else 0))
    s = []
    for w in range(W + 1):
        tau = (w * C) // W
        j = T
        while A[j] > tau:            # the largest j with A(j) <= tau
            j -= 1
        s.append(j)
    return s, c


def build_plan(seq_lens, num_kv_heads: int, n_workers: int, entry_cost_q: int = 0) -> np.ndarray:
    lens = [int(x) for x in seq_lens]
    B, H, W = len(lens), int(num_kv_heads), int(n_workers)
    if W < 1 or H < 1 or any(L < 0 for L in lens) or entry_cost_q < 0:
        raise ValueError("invalid plan arguments")
    U = B * H
    n = [(lens[u // H] + PAGE - 1) // PAGE for u in range(U)]
    P = [0]
    for u in range(U):
        P.append(P[-1] + n[u])
    T = P[U]
    s, c_applied = priced_boundaries(n, W, entry_cost_q)

    entries = []          # [u, t0, t1]
    worker_ptr = [0]
    for w in range(W):
        for u in range(U):
            lo = max(s[w], P[u])
            hi = min(s[w + 1], P[u + 1])
            if lo < hi:
                entries.append([u, lo - P[u], hi - P[u]])
        worker_ptr.append(len(entries))

    S = [0] * U
    for e in entries:
        S[e[0]] += 1
    base = [0] * U
    running = 0
    for u in range(U):
        if S[u] >= 2:
            base[u] = running
            running += S[u]
    n_partials = running

    seen = [0] * U
    slots = []
    for e in entries:
        u = e[0]
        if S[u] == 1:
            slots.append(-1)
        else:
            slots.append(base[u] + seen[u])
        seen[u] += 1

    combine = [[u, S[u], base[u]] for u in range(U) if S[u] != 1]

    header = [PLAN_VERSION, B, H, W, T, len(entries), n_partials, len(combine), PAGE, c_applied]
    header += [0] * (HEADER_WORDS - len(header))
    words = list(header) + worker_ptr
    for e, slot in zip(entries, slots):
        words += [e[0], e[1], e[2], slot]
    for c in combine:
        words += c
    return np.asarray(words, dtype=np.int32)


def parse_plan(words) -> dict:
    w = np.asarray(words, dtype=np.int64)
    hdr = w[:HEADER_WORDS]
    W, E, C = int(hdr[3]), int(hdr[5]), int(hdr[7])
    o = HEADER_WORDS
    worker_ptr = w[o:o + W + 1]
    o += W + 1
    entries = w[o:o + 4 * E].reshape(E, 4)
    o += 4 * E
    combine = w[o:o + 3 * C].reshape(C, 3)
    o += 3 * C
    return {
        "version": int(hdr[0]), "batch": int(hdr[1]), "num_kv_heads": int(hdr[2]),
        "n_workers": W, "n_tiles": int(hdr[4]), "n_entries": E, "n_partials": int(hdr[6]),
        "n_combine": C, "tile": int(hdr[8]), "entry_cost_q": int(hdr[9]), "worker_ptr": worker_ptr,
        "entries": entries,
        "combine": combine, "n_words": o,
    }


# ---------------------------------------------------------------------------
# Static split-KV baseline (the schedule the pages compare against).
#
# The HPC-Ops blog (§Attention Backend: Dynamic Load-Balanced Scheduling and
# §Attention Decode under Mixed-Length Batches) measures the balanced
# scheduler against a static split-KV schedule without defining it.  The
# reading used here is the common one: every unit is cut into the same number
# S of splits, each split taking an equal share of that unit's own tiles, and
# every non-empty split is launched as its own worker.  A batch with one long
# sequence therefore gets splits of very different sizes.
#
#   c_u = ceil(n_u / S) tiles per split of unit u (n_u >= 1);
#   split k of u covers tiles [k c_u, min((k + 1) c_u, n_u)), for k with k c_u < n_u;
#   workers are the non-empty splits in (u, k) order, one entry each;
#   slots and the merge list follow the same rule as the balanced plan.
#
# The words use the balanced plan's layout; W (header word 3) is the number of
# non-empty splits, at least 1 (an all-empty batch keeps one idle worker).

def static_split_count(seq_lens, num_kv_heads: int, n_cus: int, max_splits: int = 128) -> int:
    """The split count a static split-KV launch picks here: the smallest power
    of two S with U * S >= n_cus (enough splits to give every compute unit one),
    at most max_splits and at most the largest unit's tile count."""
    lens = [int(x) for x in seq_lens]
    U = len(lens) * int(num_kv_heads)
    n_max = max([(L + PAGE - 1) // PAGE for L in lens] + [1])
    S = 1
    while U * S < n_cus and 2 * S <= max_splits and 2 * S <= n_max:
        S *= 2
    return S


def build_static_plan(seq_lens, num_kv_heads: int, splits: int) -> np.ndarray:
    lens = [int(x) for x in seq_lens]
    B, H, S_req = len(lens), int(num_kv_heads), int(splits)
    if S_req < 1 or H < 1 or any(L < 0 for L in lens):
        raise ValueError("invalid plan arguments")
    U = B * H
    n = [(lens[u // H] + PAGE - 1) // PAGE for u in range(U)]
    T = sum(n)

    entries = []
    for u in range(U):
        if n[u] == 0:
            continue
        c = (n[u] + S_req - 1) // S_req
        k = 0
        while k * c < n[u]:
            entries.append([u, k * c, min((k + 1) * c, n[u])])
            k += 1
    W = max(1, len(entries))
    worker_ptr = list(range(len(entries) + 1)) + [len(entries)] * (W - len(entries))

    S = [0] * U
    for e in entries:
        S[e[0]] += 1
    base = [0] * U
    running = 0
    for u in range(U):
        if S[u] >= 2:
            base[u] = running
            running += S[u]
    seen = [0] * U
    slots = []
    for e in entries:
        u = e[0]
        slots.append(-1 if S[u] == 1 else base[u] + seen[u])
        seen[u] += 1
    combine = [[u, S[u], base[u]] for u in range(U) if S[u] != 1]

    header = [PLAN_VERSION, B, H, W, T, len(entries), running, len(combine), PAGE]
    header += [0] * (HEADER_WORDS - len(header))
    words = list(header) + worker_ptr
    for e, slot in zip(entries, slots):
        words += [e[0], e[1], e[2], slot]
    for c in combine:
        words += c
    return np.asarray(words, dtype=np.int32)
