"""Plain CPU oracle of one MoE routing-and-balancing layer step.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the GPU library.

Floating point is fp64 from the exact input values (bf16 bit patterns or fp32);
integer stages use Python integers in explicit loops, with numpy only for
plain counting and sorting.  Each function names the passage it follows:

* Libra README (page "Libra: Effective yet Efficient Load Balancing for
  Large-Scale MoE Inference"), section "Key Ideas": lookahead predictor,
  locality-aware replication planning (Phase 1 / Phase 2), two-stage
  MoE_local / MoE_remote execution.
* FreeBalance ("FreeBalance: Pre-Routing Online MoE Load Balancing via Residual
  Workload Prediction"): section 2.1 (top-k router and weighted MoE output),
  eq. 2-5 (early router on the previous layer's hidden states, predicted
  workload vector), section 4 "Metrics" (top-k hit rate, max/mean load).
* Relief ("A Per-Step Load-Balancing Engine for Expert-Parallel MoE Serving"):
  "The Relief Algorithm" / Algorithm 1 (bidirectional pairwise halving over
  replica edges, edge-coloured rounds), "Effective Utilization Metric"
  (spatial balance), "The Per-Step Optimum Problem" (min-max LP).

Where the pages leave a step open, the reading taken here is stated at the
function.  Parity pins: every function here is pinned by ``-m "not gpu"``
tests (hand-worked examples, closed forms, brute force, invariants); none
is "parity unpinned".
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "widen", "router_logits", "softmax", "topk", "route", "lookahead_hit",
    "histogram", "host_sets", "even_split", "modeled_loads", "plan",
    "signed_move", "split", "split_transfers", "colour_transfers", "permute", "gather_rows",
    "silu", "swiglu", "moe_dense", "moe_via_groups", "combine", "spatial",
    "static_loads",
]


# ---------------------------------------------------------------------------
# input widening


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of an input array: fp32 as is; bf16 bit patterns
    (uint16) by placing them in the high half of an fp32 word."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# (1) gate, softmax, top-k, lookahead  -- FreeBalance sec. 2.1 and eq. 2-4;
#     Libra "Key Ideas", lookahead predictor


def router_logits(h64: np.ndarray, w64: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Linear router g(X) = X W + 1 b^T (FreeBalance eq. 4).  W is stored as
    [E, d] (one row per expert), so this is X W^T + b."""
    return h64 @ w64.T + np.asarray(b, dtype=np.float64)[None, :]


def softmax(z: np.ndarray) -> np.ndarray:
    """Softmax over all E experts of each token's logits.  Reading: the router
    weights are the softmax probabilities of the selected experts, not
    renormalised over the top-k (FreeBalance sec. 2.1 gives only W,I = topk(G(h)))."""
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=1, keepdims=True)


def topk(z: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """The k experts with the largest logits, listed by descending logit; equal
    logits go to the lower expert id.  Also returns gap = z_(k) - z_(k+1), the
    distance between the k-th and (k+1)-th largest logits (+inf when k == E)."""
    T, E = z.shape
    order = np.argsort(-z, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    zs = np.take_along_axis(z, order, axis=1)
    if k < E:
        gap = zs[:, k - 1] - zs[:, k]
    else:
        gap = np.full(T, np.inf)
    return idx, gap


def route(h, w_cur, b_cur, w_next, b_next, k: int, dtype: str):
    """Gate of the current layer plus the lookahead gate (Libra "Key Ideas":
    layer i+1's gate applied to layer i's hidden states; FreeBalance eq. 2).

    Returns idx [T,k], w [T,k] (softmax probability of each selected expert),
    gap [T] (fp64), idx_next [T,k] (or None) and the fp64 logits."""
    h64 = widen(h, dtype)
    z = router_logits(h64, widen(w_cur, dtype), b_cur)
    p = softmax(z)
    idx, gap = topk(z, k)
    w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    idx_next = None
    if w_next is not None:
        zn = router_logits(h64, widen(w_next, dtype), b_next)
        idx_next, _ = topk(zn, k)
    return idx, w, gap, idx_next, z


def lookahead_hit(idx_pred: np.ndarray, idx: np.ndarray) -> float:
    """Top-k hit rate: the fraction of final top-k assignments recovered by the
    early routing pass (FreeBalance sec. 4 "Metrics"), |pred(t) & actual(t)|
    summed over tokens, divided by T*k."""
    T, k = idx.shape
    hits = 0
    for t in range(T):
        hits += len(set(int(v) for v in idx_pred[t]) & set(int(v) for v in idx[t]))
    return hits / float(T * k)


# ---------------------------------------------------------------------------
# (2) histograms -- Libra "Key Ideas" (demand of each GPU's own tokens);
#     FreeBalance eq. 5 (predicted workload vector n_e)


def histogram(idx: np.ndarray, G: int, E: int) -> np.ndarray:
    """counts[s][e] = number of pairs (t, j) with owner(t) = s and idx[t,j] = e,
    where tokens are owned in contiguous blocks of T/G (data-parallel
    attention: rank s owns tokens [s*T/G, (s+1)*T/G)).  Column sums are
    FreeBalance's workload vector n_e (eq. 5).  Ids outside [0, E) are not
    counted."""
    T = idx.shape[0]
    per = T // G
    counts = np.zeros((G, E), dtype=np.int64)
    for s in range(G):
        ids = np.asarray(idx[s * per:(s + 1) * per]).ravel().astype(np.int64)
        ids = ids[(ids >= 0) & (ids < E)]
        counts[s] = np.bincount(ids, minlength=E)
    return counts


# ---------------------------------------------------------------------------
# (3) replication plan -- Libra "Key Ideas", locality-aware expert replication
#     planning, Phase 1 and Phase 2


def host_sets(home: Sequence[int], replica: Optional[np.ndarray], E: int) -> List[set]:
    """H(e): the home rank of e plus every rank whose replica slots list e.
    Slot entries that are -1, out of [0,E), equal to the home, or repeated
    are ignored."""
    hosts = [{int(home[e])} for e in range(E)]
    if replica is not None:
        G, N = replica.shape
        for r in range(G):
            for i in range(N):
                e = int(replica[r][i])
                if 0 <= e < E:
                    hosts[e].add(r)
    return hosts


def even_split(R: int, hosts_sorted: Sequence[int]) -> Dict[int, int]:
    """Whole-token even split of a remote pool of R pairs over m hosts listed by
    ascending rank: each host gets R div m, and the first R mod m hosts one more.
    (Reading: tokens are whole; this is also the split stage's starting point.)"""
    m = len(hosts_sorted)
    q, rem = divmod(int(R), m)
    return {h: q + (1 if i < rem else 0) for i, h in enumerate(hosts_sorted)}


def _remote_pool(c, hosts_e: set, e: int, G: int) -> int:
    return sum(int(c[s][e]) for s in range(G) if s not in hosts_e)


def modeled_loads(c, hosts: List[set], G: int, E: int) -> List[int]:
    """Rank loads the plan balances: a host of e serves its own tokens of e
    (MoE_local) plus its even-split share of e's remote pool (the tokens of e
    owned by non-hosts, MoE_remote)."""
    load = [0] * G
    for e in range(E):
        Hs = sorted(hosts[e])
        share = even_split(_remote_pool(c, hosts[e], e, G), Hs)
        for r in Hs:
            load[r] += int(c[r][e]) + share[r]
    return load


def static_loads(c, home, G: int, E: int) -> List[int]:
    """Loads with no balancing: every pair of e is served by home(e)."""
    load = [0] * G
    for e in range(E):
        load[int(home[e])] += sum(int(c[s][e]) for s in range(G))
    return load


def plan(c, home, G: int, E: int, N: int, L: int, return_loads: bool = False,
         phase2: bool = True):
    """Locality-aware replication plan from a (predicted) count matrix c[G][E].

    Phase 1 (locality): each rank imports the L non-resident experts most
    requested by its own tokens -- candidates are experts with home(e) != r and
    c[r][e] > 0, ordered by c[r][e] descending, then expert id ascending.

    Phase 2 (balance), with the remaining slots (each rank holds at most N
    replicas in total): repeatedly take the most-loaded rank a (ties: lower
    rank) and walk its hosted experts by their load on a (own tokens plus its
    share of the remote pool) descending, ties lower id, skipping experts with
    an empty remote pool.  For each, the candidate is the least-loaded rank b
    (ties: lower rank) that does not host e and has a free slot.  The move is
    taken if it lowers the pair maximum, max(load_a', load_b') < load_a; the
    first expert whose move is taken ends the walk and the loop restarts.  The
    loop stops when no expert of a yields a move or no rank has a free slot.

    Returns replica[G][N] (slot order = import order, Phase 1 first, padded
    with -1), and optionally the final modeled loads.  ``phase2=False`` stops
    after Phase 1.
    """
    hosts = [{int(home[e])} for e in range(E)]
    slots: List[List[int]] = [[] for _ in range(G)]

    # Phase 1
    for r in range(G):
        cand = [e for e in range(E) if int(home[e]) != r and int(c[r][e]) > 0]
        cand.sort(key=lambda e: (-int(c[r][e]), e))
        for e in cand[:min(L, N)]:
            hosts[e].add(r)
            slots[r].append(e)

    # Phase 2
    while phase2 and any(len(slots[r]) < N for r in range(G)):
        load = modeled_loads(c, hosts, G, E)
        a = max(range(G), key=lambda r: (load[r], -r))
        contrib = {}
        for e in range(E):
            if a in hosts[e]:
                share = even_split(_remote_pool(c, hosts[e], e, G), sorted(hosts[e]))
                contrib[e] = int(c[a][e]) + share[a]
        moved = False
        for e in sorted(contrib, key=lambda e: (-contrib[e], e)):
            if _remote_pool(c, hosts[e], e, G) == 0:
                continue
            elig = [b for b in range(G) if b not in hosts[e] and len(slots[b]) < N]
            if not elig:
                continue
            b = min(elig, key=lambda r: (load[r], r))
            trial = [set(s) for s in hosts]
            trial[e].add(b)
            new = modeled_loads(c, trial, G, E)
            if max(new[a], new[b]) < load[a]:
                hosts[e].add(b)
                slots[b].append(e)
                moved = True
                break
        if not moved:
            break

    replica = np.full((G, N), -1, dtype=np.int32)
    for r in range(G):
        for i, e in enumerate(slots[r]):
            replica[r][i] = e
    if return_loads:
        return replica, modeled_loads(c, hosts, G, E)
    return replica


# ---------------------------------------------------------------------------
# (4) split -- Relief "The Relief Algorithm", Algorithm 1 (one pass), run
#     for a fixed number of passes over an edge-coloured round schedule


def split_transfers(home, hosts: List[set], E: int) -> List[Tuple[int, int, int]]:
    """One transfer per replica: (u = home(e), v = replica rank, e), listed by
    expert ascending then v ascending; experts with empty pools included, so
    the schedule depends on the placement only."""
    out = []
    for e in range(E):
        u = int(home[e])
        for v in sorted(hosts[e]):
            if v != u:
                out.append((u, v, e))
    return out


def colour_transfers(transfers) -> List[int]:
    """Greedy edge colouring in list order: each transfer takes the smallest
    colour not yet used at either of its ranks, so a colour class (round) is
    rank-disjoint."""
    used: Dict[int, set] = {}
    colours = []
    for (u, v, _e) in transfers:
        cu, cv = used.setdefault(u, set()), used.setdefault(v, set())
        col = 0
        while col in cu or col in cv:
            col += 1
        cu.add(col)
        cv.add(col)
        colours.append(col)
    return colours


def signed_move(gap: int, shift: int, mass_u: int, mass_v: int) -> int:
    """Tokens one transfer moves from u to v (negative: from v to u), given
    gap = load[u] - load[v]: the gap divided by 2**shift and rounded toward
    zero (shift 1: half the gap, so the pair's larger load can only fall),
    then kept within the mass the giving side holds of the expert's pool,
    i.e. clamped to [-mass_v, mass_u]."""
    f = abs(gap) >> shift
    if gap < 0:
        f = -f
    return max(-mass_v, min(mass_u, f))


def split(c, home, replica, G: int, E: int, passes: int = 12, eps: int = 0,
          trace: Optional[list] = None):
    """All-integer per-step split of every replicated expert's remote pool
    over its hosts.

    * Fixed load: each host of e serves its own tokens of e (MoE_local).  An
      expert with no replica also sends its whole remote pool to its home.
    * Replicated experts start from the even split of the remote pool (hosts by
      ascending rank).  mass x[e][h] = pairs of e's pool currently on host h.
    * For each pass, for each round (colour) in order, for each transfer
      t = (u, v, e) of the round (Relief, "The Relief Algorithm"): one signed
      flow of e's pool between u and v -- half the load difference, rounded
      toward zero and capped by what the giving side holds (``signed_move``)
      -- applied at once if it exceeds eps in magnitude, so the next
      transfer and round read the updated loads (Gauss-Seidel).
      Reading for experts with more than two hosts: the replica edges form a
      star around the home, and the limit is the giving host's own mass.
      Whole tokens instead of Q11.20, since hot experts exceed 2047 pairs.

    Returns host_count[E][G] (remote pairs of e served by rank r; the whole
    pool at home for unreplicated experts) and load[G].  ``trace``, if given,
    receives the max load before the first move and after every move.
    """
    hosts = host_sets(home, replica, E)
    load = [0] * G
    x: Dict[int, Dict[int, int]] = {}
    host_count = np.zeros((E, G), dtype=np.int64)
    for e in range(E):
        R = _remote_pool(c, hosts[e], e, G)
        for s in hosts[e]:
            load[s] += int(c[s][e])
        if len(hosts[e]) == 1:
            h = int(home[e])
            load[h] += R
            host_count[e][h] = R
        else:
            x[e] = even_split(R, sorted(hosts[e]))
            for h, m in x[e].items():
                load[h] += m

    transfers = split_transfers(home, hosts, E)
    colours = colour_transfers(transfers)
    n_rounds = (max(colours) + 1) if colours else 0
    rounds = [[t for t, col in zip(transfers, colours) if col == r] for r in range(n_rounds)]
    if trace is not None:
        trace.append(max(load))
    for _p in range(passes):
        for rnd in rounds:
            for (u, v, e) in rnd:
                f = signed_move(load[u] - load[v], 1, x[e][u], x[e][v])
                if abs(f) > eps:
                    load[u] -= f
                    load[v] += f
                    x[e][u] -= f
                    x[e][v] += f
                    if trace is not None:
                        trace.append(max(load))
    for e, xe in x.items():
        for h, m in xe.items():
            host_count[e][h] = m
    return host_count, np.array(load, dtype=np.int64)


# ---------------------------------------------------------------------------
# (5) permutation -- Libra "Key Ideas", two-stage locality-aware execution
#     (MoE_local segment, then MoE_remote segment)


def permute(idx: np.ndarray, home, replica, host_count, G: int, E: int):
    """Destination and order of every token-expert pair.

    Pair p = t*k + j with expert e = idx[t,j] and owner s = owner(t):
    * local (segment 0) if s hosts e: it stays on s;
    * remote (segment 1) otherwise: with rho = number of remote pairs of e with
      a smaller pair id, it goes to the first host h (ascending rank) with
      rho < sum of host_count[e][h'] over hosts h' <= h; pairs past that sum
      go to the highest-ranked host.
    Group key = (segment*G + dest)*E + e.  perm lists pair ids sorted by
    (key, pair id); pos is its inverse; group_off[2GE+1] is the exclusive
    prefix of group sizes.  Pairs with an expert id outside [0,E) are left out
    (pos = -1) and group_off[-1] counts only the others.
    """
    T, k = idx.shape
    per = T // G
    hosts = host_sets(home, replica, E)
    sorted_hosts = [sorted(h) for h in hosts]
    seen_remote = [0] * E
    keys = []
    for t in range(T):
        s = t // per
        for j in range(k):
            e = int(idx[t][j])
            if not (0 <= e < E):
                continue
            if s in hosts[e]:
                seg, dest = 0, s
            else:
                seg = 1
                rho = seen_remote[e]
                seen_remote[e] += 1
                dest = sorted_hosts[e][-1]
                cum = 0
                for h in sorted_hosts[e]:
                    cum += max(int(host_count[e][h]), 0)
                    if rho < cum:
                        dest = h
                        break
            keys.append(((seg * G + dest) * E + e, t * k + j))
    keys.sort()
    ngroups = 2 * G * E
    sizes = np.zeros(ngroups, dtype=np.int64)
    for key, _p in keys:
        sizes[key] += 1
    group_off = np.zeros(ngroups + 1, dtype=np.int64)
    group_off[1:] = np.cumsum(sizes)
    perm = np.array([p for _key, p in keys], dtype=np.int64)
    pos = np.full(T * k, -1, dtype=np.int64)
    pos[perm] = np.arange(len(perm))
    return group_off, perm, pos


def gather_rows(h: np.ndarray, perm: np.ndarray, k: int) -> np.ndarray:
    """X_perm[q] = h[perm[q] div k] (a copy of the token's row, any dtype)."""
    return np.asarray(h)[np.asarray(perm) // k]


# ---------------------------------------------------------------------------
# (6) experts, weighted combine -- FreeBalance sec. 2.1; SwiGLU experts


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu(x64: np.ndarray, w13_64: np.ndarray, w2_64: np.ndarray) -> np.ndarray:
    """SwiGLU expert: W13 holds the gate rows [0, I) then the up rows [I, 2I);
    y = (SiLU(x W_gate^T) * (x W_up^T)) W2^T, fp64, no intermediate rounding."""
    inter = w13_64.shape[0] // 2
    gu = x64 @ w13_64.T
    return (silu(gu[:, :inter]) * gu[:, inter:]) @ w2_64.T


ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray]]


def moe_dense(h64: np.ndarray, idx: np.ndarray, w: np.ndarray, expert: ExpertFn,
              tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """MoE(h) = sum over the selected experts i of W_i * expert_i(h)
    (FreeBalance sec. 2.1), straight from the routing, with no plan, split or
    permutation.  ``expert(e)`` returns fp64 (W13, W2).  ``tokens`` restricts
    the computation to some rows (returned in that order)."""
    if tokens is None:
        tokens = np.arange(h64.shape[0])
    tokens = np.asarray(tokens)
    out = np.zeros((len(tokens), h64.shape[1]))
    sel = np.asarray(idx)[tokens]
    for e in np.unique(sel):
        if e < 0:
            continue
        rows, cols = np.nonzero(sel == e)
        w13, w2 = expert(int(e))
        y = swiglu(h64[tokens[rows]], w13, w2)
        out[rows] += np.asarray(w)[tokens[rows], cols][:, None] * y
    return out


def moe_via_groups(h64: np.ndarray, idx: np.ndarray, w: np.ndarray, expert: ExpertFn,
                   group_off: np.ndarray, perm: np.ndarray, pos: np.ndarray, E: int):
    """The same layer output computed the way the balanced path does it: each
    group's rows run through their expert (group g's expert is g mod E), then
    out[t] = sum_j w[t,j] * Y[pos[t*k+j]] with j ascending.  Returns (out, Y)."""
    T, k = idx.shape
    Y = np.zeros((len(perm), h64.shape[1]))
    ngroups = len(group_off) - 1
    for e in range(E):
        # every group of expert e (rows are independent, so they run together)
        rows = [np.arange(int(group_off[g]), int(group_off[g + 1])) for g in range(e, ngroups, E)]
        rows = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
        if len(rows) == 0:
            continue
        w13, w2 = expert(e)
        Y[rows] = swiglu(h64[np.asarray(perm)[rows] // k], w13, w2)
    return combine(Y, pos, w, T, k), Y


def combine(Y: np.ndarray, pos: np.ndarray, w: np.ndarray, T: int, k: int,
            shared: Optional[np.ndarray] = None) -> np.ndarray:
    """out[t] = sum_{j ascending} w[t,j] * Y[pos[t*k+j]]  (+ shared[t]);
    pairs with pos < 0 contribute nothing."""
    out = np.zeros((T, Y.shape[1]))
    for t in range(T):
        for j in range(k):
            q = int(pos[t * k + j])
            if q >= 0:
                out[t] += float(w[t][j]) * Y[q]
    if shared is not None:
        out += shared
    return out


# ---------------------------------------------------------------------------
# metrics -- Relief "Effective Utilization Metric"; FreeBalance sec. 4 Metrics


def spatial(load: Sequence[int]) -> float:
    """Spatial balance sum(L_i) / (G * max L_i); its inverse is the max/mean
    imbalance ratio."""
    load = [int(v) for v in load]
    m = max(load)
    return 1.0 if m == 0 else sum(load) / (len(load) * m)
