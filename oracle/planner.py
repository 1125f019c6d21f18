"""Work partitions of split-KV decode attention, as plain integer Python.

TEST INFRASTRUCTURE ONLY (see the package header).

Balanced plan -- xiaodao.ai "HPC-Ops 把 TPOT 降 48.8%，用户未必快一半", section
"为什么 batch 越大，数字越漂亮": each request's live KV is cut into 64-token tiles
and the global tile list is spread as evenly as possible over persistent
workers, so long sequences get more work and short ones only what they have;
bitbyai.com "vLLM × HPC-Ops: …", section "Breaking Down the Kernels": the
schedule is recomputed every decode step from the live lengths.

Readings taken where the pages are silent (all integer, so the GPU planner
must reproduce them bit for bit):

* sequence s = b * Hkv + g (request-major); n_s = ceil(L_b / 64) tiles;
  C = exclusive prefix sum of n_s; N = C[S].
* "as evenly as possible" = contiguous floor partition of the global tile
  list: W' = 0 if N == 0 else min(W, max(1, N // min_tiles)); worker w owns
  global tiles [w*N // W', (w+1)*N // W') (64-bit products).
* a worker's range is cut at sequence boundaries into items (s, t0, t1) in
  sequence order; items are listed worker by worker.
* split(item) = rank of the item among the items of its sequence;
  num_splits[s] = number of such items; sequences with more than one item get
  consecutive partial slots partial_base[s] + split, where partial_base is
  the exclusive prefix sum of (num_splits if num_splits > 1 else 0); items of
  unsplit sequences have slot -1 (they write the output directly).
* merge_list = sequences whose num_splits != 1 (split ones are combined,
  empty ones get a zero output row), in increasing s.

Per-item cost (bitbyai.com "vLLM × HPC-Ops: …", section "Breaking Down the
Kernels": the scheduler weighs work by progress; here, the plainest form of it):
each item a worker starts costs a fixed overhead on top of its tiles, so with
item_cost c > 0 every non-empty sequence is preceded in the global list by c
virtual tiles. Positions: C'[s] = C[s] + c * (non-empty sequences before s),
N' = N + c * (non-empty sequences); W' = 0 if N == 0 else min(W, max(1, N' // min_tiles));
worker w owns positions [w*N' // W', (w+1)*N' // W'); its items are the real
tiles [C'[s] + c, C'[s] + c + n_s) it owns. c = 0 is the plain partition above.
A worker whose range covers only virtual positions of a sequence gets no item
for it, and may get no item at all.

Dynamic tail (bitbyai.com, same section: the scheduler evaluates progress
dynamically). The persistent workers do not all run at the same speed, so the
last part of the work is not given to anyone in advance: with tail_den d > 0,
the last T = N' // d positions are cut into D = min(ceil(T / tail_chunk), 4 W) chunks
(at most four per worker, so the work list has a size bound) that workers claim
at run time, each the moment it has finished what it holds. The
first A = N' - T positions are split evenly over W_s = min(W', A) workers
(W' still from N'; a worker left without a static position goes straight to
the chunks, so every virtual worker owns at least one position). Virtual
worker v < W_s owns [v*A // W_s, (v+1)*A // W_s), virtual worker W_s + c owns
[A + c*T // D, A + (c+1)*T // D); items, split ranks and slots follow the
virtual workers in order, so the result does not depend on which worker claims
which chunk. tail_den 0 is the plan without a tail (then W_s = W').

Item order within a worker (bitbyai.com, same section: the scheduler
prioritizes nearly-finished short requests while spreading longer ones evenly
over the grid). The partition above already spreads long sequences evenly;
what is left to choose is the order in which a worker runs the items it holds.
item_order 0 runs them in list (position) order. item_order 1 runs first the
sequences it holds whole -- the short requests, finished by this worker alone,
which write their output directly -- and then the pieces of sequences shared
with other workers. item_order 2 is the reverse choice: the shared pieces
first, so that the partial results of split sequences are complete sooner.
Both keep list order inside each of the two classes. An item's split rank is
its rank in list order, so the order never changes a split rank, a partial
slot or the combine order: the output is the same bits in every order.

Static split-KV (the comparison the pages describe in the same section):
flavour "splits" fixes the number of splits per sequence,
S_split = clamp(ceil(W / S), 1, max_pages), chunk_s = ceil(n_s / S_split);
flavour "chunk" fixes the split size from the longest request the page table
can hold, chunk = ceil(max_pages / S_split), and reserves S_split slots for
every sequence (short ones carry empty tasks). Partial slot = s * S_split + k
when a sequence has more than one non-empty chunk.

Parity pins (tests/test_oracle_planner.py): a hand-derived plan for the tiny
workload (tests/golden/plan_tiny_w4.json); a brute-force tile-by-tile
construction on random small cases; coverage, balance and slot properties.
"""

PAGE = 64


def tile_counts(seq_lens, hkv):
    return [(int(L) + PAGE - 1) // PAGE for L in seq_lens for _ in range(hkv)]


def active_workers(N, num_workers, min_tiles):
    if N == 0:
        return 0
    return min(num_workers, max(1, N // min_tiles))


def balanced_plan(seq_lens, hkv, num_workers, min_tiles=1, item_cost=0, tail_den=0, tail_chunk=1, item_order=0):
    n = tile_counts(seq_lens, hkv)
    S = len(n)
    C = [0] * (S + 1)
    for s in range(S):
        C[s + 1] = C[s] + n[s]
    N = C[S]
    # global positions: c virtual tiles in front of every non-empty sequence
    start = [0] * (S + 1)                        # first position of sequence s (virtual part)
    for s in range(S):
        start[s + 1] = start[s] + (n[s] + item_cost if n[s] > 0 else 0)
    Np = start[S]
    Wp = 0 if N == 0 else min(num_workers, max(1, Np // min_tiles))
    T = Np // tail_den if (tail_den > 0 and N > 0) else 0     # positions of the dynamic tail
    A = Np - T
    D = min(-(-T // tail_chunk), 4 * num_workers) if T > 0 else 0
    Ws = min(Wp, A)                              # workers with a static range
    bounds = [w * A // Ws for w in range(Ws)] + [A + c * T // D for c in range(D)] + [Np]
    V = Ws + D                                   # virtual workers: W_s static, then D chunks

    items = []                                   # (virtual worker, s, t0, t1)
    worker_off = [0]
    first = 0                                    # first sequence not wholly before the worker
    for w in range(V):
        a = bounds[w]
        e = bounds[w + 1]
        while first < S and start[first + 1] <= a:
            first += 1
        s = first
        while s < S and start[s] < e:            # sequences overlapping positions [a, e)
            if n[s] > 0:
                r0 = start[s] + item_cost        # real tiles of s: positions [r0, r0 + n_s)
                lo, hi = max(a, r0), min(e, r0 + n[s])
                if lo < hi:
                    items.append((w, s, lo - r0, hi - r0))
            s += 1
        worker_off.append(len(items))

    num_splits = [0] * S
    split = []
    for _, s, _, _ in items:
        split.append(num_splits[s])
        num_splits[s] += 1
    partial_base = [0] * S
    acc = 0
    for s in range(S):
        partial_base[s] = acc
        if num_splits[s] > 1:
            acc += num_splits[s]
    slots = [partial_base[s] + k if num_splits[s] > 1 else -1
             for (_, s, _, _), k in zip(items, split)]
    if item_order:
        # within each virtual worker: a stable partition into the items of sequences it
        # holds whole (unsplit) and the pieces of split sequences; order 1 runs the whole
        # ones first, order 2 the pieces first; ranks and slots travel with their items
        order = []
        for w in range(V):
            idx = list(range(worker_off[w], worker_off[w + 1]))
            whole = [i for i in idx if num_splits[items[i][1]] == 1]
            piece = [i for i in idx if num_splits[items[i][1]] != 1]
            order += whole + piece if item_order == 1 else piece + whole
        items = [items[i] for i in order]
        split = [split[i] for i in order]
        slots = [slots[i] for i in order]
    return dict(
        C=C, N=N, Np=Np, S=S, Wp=Wp, Ws=Ws, D=D, V=V, n_items=len(items), worker_off=worker_off,
        item_s=[it[1] for it in items], item_t0=[it[2] for it in items],
        item_t1=[it[3] for it in items], item_split=split, item_slot=slots,
        num_splits=num_splits, partial_base=partial_base, n_partials=acc,
        merge_list=[s for s in range(S) if num_splits[s] != 1],
    )


def static_splits(num_seqs, num_workers, max_pages):
    return max(1, min(-(-num_workers // max(num_seqs, 1)), max_pages))


def static_partition(seq_lens, hkv, num_workers, max_pages, flavour="splits"):
    """Items (s, k, t0, t1, slot) of the static split-KV schedule."""
    n = tile_counts(seq_lens, hkv)
    S = len(n)
    ss = static_splits(S, num_workers, max_pages)
    fixed_chunk = -(-max_pages // ss)
    items = []
    for s in range(S):
        if n[s] == 0:
            continue
        chunk = -(-n[s] // ss) if flavour == "splits" else fixed_chunk
        nchunks = -(-n[s] // chunk)
        for k in range(ss):
            t0, t1 = k * chunk, min((k + 1) * chunk, n[s])
            if t0 < t1:
                items.append((s, k, t0, t1, s * ss + k if nchunks > 1 else -1))
    return dict(S_split=ss, items=items)
