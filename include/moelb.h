/*
 * moelb -- MoE routing-and-balancing hot path for AMD Instinct MI355X (gfx950).
 *
 * One MoE layer step on one GPU, with the expert-parallel group's G ranks kept
 * as integer bookkeeping:
 *
 *   moelb_gate_topk   router GEMM + softmax + top-k, and the lookahead router
 *   moelb_histogram   per-rank token-expert counts
 *   moelb_plan        locality-aware replication plan (Phase 1, Phase 2)
 *   moelb_split       all-integer pairwise-halving split of remote pools
 *   moelb_permute     local/remote, rank- and expert-sorted pair order (+ rows)
 *   moelb_grouped_ffn masked grouped SwiGLU expert GEMMs
 *   moelb_combine     top-k weighted sum of expert outputs (+ shared expert)
 *
 * and around them: the split's round schedule made once per placement
 * (moelb_split_schedule, moelb_split_scheduled), split variants for
 * comparison (moelb_split_variant), an earlier step's split dealt again
 * (moelb_split_stale), FreeBalance's expert-swap planner (moelb_plan_swaps),
 * the permutation in two phases (moelb_permute_local, moelb_permute_remote),
 * the FFN in stages (moelb_grouped_ffn_stages) and expert weights packed once
 * for the FFN's weight streams (moelb_pack_weights).
 *
 * Conventions for every entry point:
 *  - Plain C ABI.  Every pointer argument is DEVICE memory owned by the caller
 *    (e.g. a PyTorch tensor's data pointer), unless stated otherwise; the
 *    library keeps no pointer after the call returns and allocates nothing.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without waiting; outputs are valid once the stream has
 *    reached that point.
 *  - Arguments are checked on the host before anything is launched.  A bad
 *    argument returns MOELB_EINVAL and launches nothing.  Sizes must be exact
 *    multiples where stated: unsupported shapes are errors, never fallbacks.
 *  - Contents of device buffers cannot be checked on the host; for each entry
 *    point the behaviour on out-of-range device values is stated and is memory
 *    safe.
 *  - bf16 tensors are raw IEEE bfloat16 bit patterns (uint16); fp32 is IEEE
 *    binary32.  Matrices are row-major.
 *  - Thread safety: calls keep no state and may be made from several threads.
 */
#ifndef MOELB_H
#define MOELB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moelb_status {
  MOELB_OK = 0,
  MOELB_EINVAL = 1,     /* bad argument; nothing was launched                  */
  MOELB_ELAUNCH = 2,    /* a kernel launch or runtime call failed              */
  MOELB_EWORKSPACE = 3  /* workspace pointer NULL or smaller than required     */
};

enum moelb_dtype {
  MOELB_F32 = 0,        /* fp32 storage and fp32 arithmetic                    */
  MOELB_BF16 = 1        /* bf16 storage, fp32 accumulation (MFMA)             */
};

/* Limits checked by every entry point. */
#define MOELB_MAX_E 256   /* experts                  */
#define MOELB_MAX_K 16    /* experts per token        */
#define MOELB_MAX_G 64    /* virtual EP ranks         */
#define MOELB_MAX_N 8     /* replica slots per rank   */

int moelb_version(void);                  /* major*10000 + minor*100 + patch */
const char* moelb_status_string(int status);

/*
 * Router of the current layer and lookahead router of the next layer.
 *
 * Computes, per token t (FreeBalance, "FreeBalance: Pre-Routing Online MoE Load
 * Balancing via Residual Workload Prediction", section 2.1 and eq. 2-4; Libra
 * README "Key Ideas", lookahead predictor):
 *   z[t,e]   = h[t,:] . w_cur[e,:] + b_cur[e]           (fp32 accumulation)
 *   idx[t,:] = the k experts with the largest z, by descending z, ties to the
 *              lower expert id
 *   wts[t,j] = softmax over all E of z[t,:], at expert idx[t,j] (no
 *              renormalisation over the top-k)
 *   gap[t]   = z_(k) - z_(k+1), k-th minus (k+1)-th largest (+inf if k == E)
 *   idx_next = the same top-k rule on h[t,:] . w_next[e,:] + b_next[e]
 *
 *  h       [T,d]  dtype          hidden states of the current layer
 *  w_cur   [E,d]  dtype          router weight, one row per expert
 *  b_cur   [E]    fp32           router bias
 *  w_next  [E,d]  dtype or NULL  next layer's router (NULL: no lookahead,
 *  b_next  [E]    fp32 or NULL                        idx_next must be NULL)
 *  idx     [T,k]  int32  out
 *  wts     [T,k]  fp32   out
 *  gap     [T]    fp32   out, may be NULL
 *  idx_next[T,k]  int32  out, NULL iff w_next is NULL
 * Requires 1 <= k <= min(E, 16), E <= 256, d % 8 == 0, T >= 0.
 */
int moelb_gate_topk(const void* h, int T, int d, int E, int k, int dtype,
                    const void* w_cur, const float* b_cur,
                    const void* w_next, const float* b_next,
                    int32_t* idx, float* wts, float* gap, int32_t* idx_next,
                    void* stream);

/*
 * Per-rank histogram (Libra "Key Ideas": demand of each GPU's own tokens;
 * FreeBalance eq. 5: the workload vector n_e is the column sum).
 *   counts[s,e] = #{(t,j) : t div (T/G) == s, idx[t,j] == e}
 *  idx          [T,k] int32
 *  counts       [G,E] int32 out (overwritten)
 *  expert_total [E]   int32 out or NULL: column sums of counts
 * Ids outside [0,E) are not counted.  Requires T % G == 0, G <= 64, E <= 256.
 */
int moelb_histogram(const int32_t* idx, int T, int k, int E, int G,
                    int32_t* counts, int32_t* expert_total, void* stream);

/*
 * Locality-aware replication plan (Libra README "Key Ideas": Phase 1 imports
 * the L = N*alpha non-resident experts most requested by each GPU's own
 * tokens; Phase 2 repeatedly replicates the hottest expert of the most-loaded
 * GPU to the least-loaded eligible GPU).  Exact rules:
 *  Phase 1: per rank r, experts e with home[e] != r and counts[r,e] > 0, by
 *    counts[r,e] descending then e ascending; the first min(L, N) are imported.
 *  Load model: a host of e serves its own tokens of e plus its share of e's
 *    remote pool R(e) (pairs of e owned by non-hosts), split evenly in whole
 *    tokens over the hosts by ascending rank (R div m each, the first R mod m
 *    hosts one more).
 *  Phase 2, while some rank has a free slot: a = most-loaded rank (ties: lower
 *    rank).  Among experts hosted at a with R(e) > 0, walk by a's load of e
 *    descending (ties: lower e); b = least-loaded rank (ties: lower) that does
 *    not host e and has a free slot; take the first move with
 *    max(load_a', load_b') < load_a.  Stop when a has no such move.
 *  counts    [G,E] int32   (predicted counts, e.g. from the lookahead)
 *  home      [E]   int32   resident rank of each expert, in [0,G)
 *  replica   [G,N] int32 out: imports of each rank in import order, -1 padded
 *  plan_load [G]   int32 out or NULL: modeled loads of the final plan
 * Requires 0 <= L <= N <= 8, G <= 64, E <= 256.  home entries outside [0,G)
 * are read as rank 0.  Counts must be >= 0 and their total below 2^31.
 */
int moelb_plan(const int32_t* counts, const int32_t* home, int G, int E, int N, int L,
               int32_t* replica, int32_t* plan_load, void* stream);

/*
 * All-integer per-step split (Relief, "A Per-Step Load-Balancing Engine for
 * Expert-Parallel MoE Serving", "The Relief Algorithm", Algorithm 1).
 *  Hosts H(e) = home[e] plus every rank whose replica row lists e (entries -1,
 *  outside [0,E) or equal to the home are ignored; repeats count once).
 *  Fixed load: each host serves its own tokens of e; an unreplicated expert's
 *  whole remote pool goes to its home.  A replicated expert's pool starts
 *  evenly split (as in moelb_plan).  One transfer (home(e), v, e) per replica
 *  rank v, listed by e then v ascending; greedy edge colouring (smallest
 *  colour free at both ranks) gives rank-disjoint rounds.  `passes` times, for
 *  every round in colour order, every transfer of the round does
 *    gap = load[u]-load[v]; delta = min(|gap| >> 1, mass of the heavier side);
 *    if delta > eps, move delta pairs from the heavier to the lighter rank,
 *  and the next round reads the updated loads.
 *  counts     [G,E] int32   actual counts of this step
 *  home       [E]   int32
 *  replica    [G,N] int32   placement in force for this step
 *  host_count [E,G] int32 out: remote pairs of e served by rank r (0 at
 *                            non-hosts; the whole pool at home if unreplicated)
 *  load       [G]   int32 out: rank loads after the split
 * Requires 0 <= passes <= 1024, eps >= 0, G <= 64, N <= 8, E <= 256.
 */
int moelb_split(const int32_t* counts, const int32_t* home, const int32_t* replica,
                int G, int E, int N, int passes, int eps,
                int32_t* host_count, int32_t* load, void* stream);

/*
 * Budgeted expert-swap planner (FreeBalance section 3.3, eq. 6-8 and
 * Algorithm 1): the alternative to replication -- experts trade places, so
 * every rank keeps its number of experts and no split is needed (run the rest
 * of the path with home_out and no replicas).
 *   n_e = sum_s counts[s,e] (predicted pairs); L_r = sum of n_e over the
 *   experts on r.  While L_a - L_b > tau for a = most-loaded and b =
 *   least-loaded rank (ties: lower rank) and both have budget left: among the
 *   experts on a and on b that have not moved yet, swap the pair with the
 *   largest positive drop of Phi(L) = max_r L_r + gamma * sum_r (L_r -
 *   mean)^2, gamma = gamma_num / gamma_den (ties: lower e_a, then lower e_b);
 *   stop if no pair lowers Phi.  Each swap spends one of both ranks'
 *   max_swaps_per_rank (every swap moves two equal-sized experts, so the
 *   page's per-rank transfer budget is a swap count).
 *  counts   [G,E] int32  predicted counts (the lookahead histogram), >= 0,
 *                        totalling below 2^24 pairs (exact 64-bit scores)
 *  home     [E]   int32  current placement (entries outside [0,G) read as 0)
 *  home_out [E]   int32 out: placement after the swaps (may be `home` itself)
 *  swaps    [E/2][2] int32 out or NULL: (e_a, e_b) in acceptance order
 *  n_swaps  [1]   int32 out or NULL: number of swaps
 *  load     [G]   int32 out: rank loads after the swaps
 * Requires G <= 64, E <= 256, tau >= 0, 0 <= gamma_num <= 2^12,
 * 1 <= gamma_den <= 2^20, max_swaps_per_rank >= 0.
 */
int moelb_plan_swaps(const int32_t* counts, const int32_t* home, int G, int E, int tau,
                     int gamma_num, int gamma_den, int max_swaps_per_rank,
                     int32_t* home_out, int32_t* swaps, int32_t* n_swaps, int32_t* load,
                     void* stream);

/*
 * Split variants on the same transfers (Relief, "Ablation Results (Table
 * III)"; Libra README "Key Ideas", adaptive token sharding), for comparing
 * balance and latency.  moelb_split is variant MOELB_SPLIT_RELIEF; passes = 0
 * of any pairwise variant is the even ("hash") split.
 *  MOELB_SPLIT_NO_REVERSE   Relief's move only when the home is the heavier
 *                           side (mass only flows from home to replica).
 *  MOELB_SPLIT_JACOBI       every transfer of a pass reads the loads of the
 *                           pass start and moves |gap| >> 2 (damped),
 *                           capped by the giver's current mass.
 *  MOELB_SPLIT_LIBRA_GREEDY pools start on their homes; repeatedly the
 *                           most-loaded rank a (ties: lower rank) hands
 *                           min(mass, (load[a]-load[b]) >> 1) tokens of its
 *                           replicated expert with the most mass on a (ties:
 *                           lower id) to that expert's least-loaded other
 *                           host b (ties: lower rank), if load[a]-load[b] >= 2;
 *                           at most passes x (number of replica transfers)
 *                           moves.
 *  MOELB_SPLIT_WATER_FILL   pools start from the even split; each pass every
 *                           replicated expert re-deals its whole pool R from
 *                           one snapshot of the loads, over levels l_h = load
 *                           - own mass on host h: the largest z with sum of
 *                           max(0, z - l_h) <= R is filled, the tokens left go
 *                           one each to hosts with l_h <= z (ascending rank);
 *                           stops after a pass that changes nothing (eps and
 *                           the schedule are not used).
 *  MOELB_SPLIT_PROPORTIONAL as MOELB_SPLIT_WATER_FILL, but each pool is
 *                           re-dealt in proportion to 1 / (l_h + 1), exactly:
 *                           host h gets the floor of its rational share, and
 *                           the tokens left go one each to the hosts with the
 *                           largest remainders (ties: lower rank).  Requires
 *                           G <= 16 (else MOELB_EINVAL).
 * Same arguments, outputs and requirements as moelb_split; counts must be
 * non-negative.  An unknown variant returns MOELB_EINVAL.
 */
/*
 * Round schedule of the split (Relief, "The Relief Algorithm": the edge
 * colouring depends on the placement only and is computed once per placement
 * change, not per step).  moelb_split_schedule writes, for home/replica, the
 * transfer list and its greedy colouring into `schedule` (MOELB_SPLIT_SCHEDULE_INTS
 * int32: n, number of colours, then (u, v, colour) per transfer).
 * moelb_split_scheduled is moelb_split_variant with such a schedule: if it
 * lists exactly this placement's transfers, the split uses its colours (the
 * same ones it would compute); otherwise (or with schedule = NULL) it colours
 * the transfers itself.  Outputs are identical either way.
 */
#define MOELB_SPLIT_SCHEDULE_INTS (2 + 3 * MOELB_MAX_G * MOELB_MAX_N)
int moelb_split_schedule(const int32_t* home, const int32_t* replica, int G, int E, int N,
                         int32_t* schedule, void* stream);
int moelb_split_scheduled(const int32_t* counts, const int32_t* home, const int32_t* replica,
                          const int32_t* schedule, int G, int E, int N, int passes, int eps,
                          int variant, int32_t* host_count, int32_t* load, void* stream);

enum moelb_split_variant {
  MOELB_SPLIT_RELIEF = 0,
  MOELB_SPLIT_NO_REVERSE = 1,
  MOELB_SPLIT_JACOBI = 2,
  MOELB_SPLIT_LIBRA_GREEDY = 3,
  MOELB_SPLIT_WATER_FILL = 4,
  MOELB_SPLIT_PROPORTIONAL = 5
};
int moelb_split_variant(const int32_t* counts, const int32_t* home, const int32_t* replica,
                        int G, int E, int N, int passes, int eps, int variant,
                        int32_t* host_count, int32_t* load, void* stream);

/*
 * Stale split: an earlier step's split dealt again on this step's counts
 * (Relief, "Failure of Existing Approaches": deciding the split less often
 * than every step).  Same placement conventions and outputs as moelb_split.
 * Each replicated expert's remote pool R (its pairs owned by non-hosts) is
 * dealt over its current hosts in the fractions p_h / P, p_h =
 * max(host_count_prev[e,h], 0), P = sum of p_h over those hosts: host h gets
 * floor(R p_h / P), and the R - sum(floors) hosts with the largest remainders
 * (ties: lower rank) one more; if P = 0 the pool is split evenly (R div m
 * each, the lowest R mod m hosts one more).  Unreplicated pools stay at home.
 *  host_count_prev [E,G] int32  shares of the earlier step (moelb_split's
 *                               host_count); must not overlap host_count
 *  counts [G,E] int32 >= 0 (totalling below 2^31), home [E], replica [G,N]
 *  host_count [E,G] int32 out, load [G] int32 out
 * Requires G <= 64, N <= 8, E <= 256; host_count == host_count_prev returns
 * MOELB_EINVAL.
 */
int moelb_split_stale(const int32_t* counts, const int32_t* home, const int32_t* replica,
                      int G, int E, int N, const int32_t* host_count_prev,
                      int32_t* host_count, int32_t* load, void* stream);

/*
 * Local/remote permutation (Libra README "Key Ideas": two-stage locality-aware
 * execution, MoE_local on the token's own GPU, MoE_remote on the others).
 *  Pair p = t*k + j, expert e = idx[t,j], owner s = t div (T/G).  Local
 *  (segment 0, destination s) if s hosts e; otherwise remote (segment 1): with
 *  rho = number of remote pairs of e with a smaller pair id, the destination is
 *  the first host h (ascending rank) with rho < sum_{h' <= h} host_count[e,h']
 *  (negative entries read as 0); pairs past that sum go to the highest host.
 *  Group key (segment*G + destination)*E + e.  perm lists pair ids by (key,
 *  pair id); pos is its inverse; group_off is the exclusive prefix of the
 *  2*G*E group sizes.  Pairs whose id is outside [0,E) are left out: pos = -1,
 *  and group_off[2GE] counts only valid pairs.
 *  h          [T,d]    dtype         rows to gather (may be NULL iff x_perm is NULL)
 *  idx        [T,k]    int32
 *  home       [E], replica [G,N], host_count [E,G]   int32 (from moelb_split)
 *  ws         workspace of moelb_permute_workspace_bytes(T,k,E,G) bytes
 *  group_off  [2*G*E+1] int32 out
 *  perm, pos  [T*k]     int32 out
 *  x_perm     [T*k,d]   dtype out or NULL: x_perm[q] = h[perm[q] div k]
 * Requires T % G == 0, k <= 16, E <= 256, G <= 64, N <= 8, d % 8 == 0.
 * With x_perm NULL, T*k <= 8192 and E*G <= 2048 the call is one launch of one
 * workgroup (the same outputs; the workspace is then not touched), else four.
 */
size_t moelb_permute_workspace_bytes(int T, int k, int E, int G);
int moelb_permute(const void* h, const int32_t* idx, int T, int d, int k, int E, int G, int N,
                  int dtype, const int32_t* home, const int32_t* replica,
                  const int32_t* host_count, void* ws, size_t ws_bytes,
                  int32_t* group_off, int32_t* perm, int32_t* pos, void* x_perm,
                  void* stream);

/*
 * moelb_permute without a workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, serving loops, harnesses that
 * forbid hipMalloc).  The workspace is a fixed array of
 * MOELB_PERMUTE_NOALLOC_WS_BYTES in device memory, one per device the
 * library runs on, held until the process ends; the call allocates and
 * frees nothing.  Same arguments (less ws, ws_bytes), outputs and errors as
 * moelb_permute, plus MOELB_EWORKSPACE (nothing launched) when
 * moelb_permute_workspace_bytes(T, k, E, G) exceeds that size, and
 * MOELB_ELAUNCH if the array's device address cannot be obtained.  Every
 * call on a device shares that device's array: calls that overlap on one
 * device (other streams, other threads) race and must be ordered by the
 * caller.  No initial contents are needed.
 */
#define MOELB_PERMUTE_NOALLOC_WS_BYTES (32u << 20)
int moelb_permute_noalloc(const void* h, const int32_t* idx, int T, int d, int k, int E, int G, int N,
                          int dtype, const int32_t* home, const int32_t* replica,
                          const int32_t* host_count, int32_t* group_off, int32_t* perm, int32_t* pos,
                          void* x_perm, void* stream);

/*
 * The same permutation in two phases (Libra README "Key Ideas": MoE_local
 * starts right after gating; the token sharding of the remote pairs runs
 * beside it).  Calling moelb_permute_local and then moelb_permute_remote with
 * the same arguments and the same workspace (untouched in between) gives
 * exactly moelb_permute's outputs.
 *  moelb_permute_local needs no host_count: it writes group_off[0..G*E]
 *  (the local groups; group_off[G*E] = number of local pairs), the perm
 *  entries below group_off[G*E], pos of every local pair, pos = -1 for remote
 *  pairs, and the local rows of x_perm (if given).  The local groups can be
 *  computed from this point on (moelb_grouped_ffn over the first G*E groups).
 *  moelb_permute_remote takes host_count (from moelb_split) and writes
 *  group_off[G*E+1..2*G*E], the remaining perm entries, pos of the remote
 *  pairs and their x_perm rows.  Its workspace must hold the local phase's
 *  state for the same idx, home and replica.
 * Same requirements and errors as moelb_permute.
 */
int moelb_permute_local(const void* h, const int32_t* idx, int T, int d, int k, int E, int G, int N,
                        int dtype, const int32_t* home, const int32_t* replica, void* ws,
                        size_t ws_bytes, int32_t* group_off, int32_t* perm, int32_t* pos,
                        void* x_perm, void* stream);
int moelb_permute_remote(const void* h, const int32_t* idx, int T, int d, int k, int E, int G, int N,
                         int dtype, const int32_t* home, const int32_t* replica,
                         const int32_t* host_count, void* ws, size_t ws_bytes,
                         int32_t* group_off, int32_t* perm, int32_t* pos, void* x_perm,
                         void* stream);

/*
 * Masked grouped SwiGLU expert FFN (Libra README "Repository Layout": FusedMoE
 * over masked tokens; FreeBalance section 2.1: expert_i(h)).
 *  Group g covers rows [group_off[g], group_off[g+1]) and uses expert g mod E
 *  (replicas alias the expert's weights).  With rank >= 0 only groups whose
 *  rank (g div E) mod G equals `rank` are computed (one virtual rank's share);
 *  rank = -1 computes all groups.  For each computed row q:
 *    a = SiLU(x_q . W13[e, 0:I]^T) * (x_q . W13[e, I:2I]^T)   (rounded to dtype)
 *    y[q] = a . W2[e]^T                                       (rounded to dtype)
 *  with fp32 accumulation.  x_q is x[q], or x[gather[q] div gather_k] when
 *  `gather` is given (the rows are read straight from the unpermuted hidden
 *  states: pass moelb_permute's perm and the top-k).  Rows outside every
 *  computed group are not written.
 *  x          [rows_x,d]  dtype    rows (X_perm, or h when gather is given)
 *  group_off  [num_groups+1] int32 non-decreasing offsets in [0, rows]
 *  gather     [rows] int32 or NULL; gather_k >= 1
 *  w13        [E,2*inter,d] dtype  gate rows then up rows, K-contiguous
 *  w2         [E,d,inter]   dtype  K-contiguous
 *  ws         workspace of moelb_grouped_ffn_workspace_bytes(...) bytes
 *             (schedule tables and the SwiGLU activations; no initial
 *             contents needed)
 *  y          [rows,d]      dtype out
 *  Device offsets are clamped: group g covers [lo, hi) with lo =
 *  clamp(group_off[g], 0, rows), hi = clamp(group_off[g+1], lo, rows).
 *  Computed groups are taken expert by expert (e ascending, then g
 *  ascending) and at most `rows` rows are computed in all; with offsets
 *  that are not non-decreasing, groups can overlap (a row computed by
 *  several groups gets one of their results) and rows past that total are
 *  not computed.  Every row read or written stays inside the buffers either
 *  way.  gather entries outside [0, rows_x*gather_k) read row 0.
 * Requires rows >= 0, rows_x >= 1 when rows > 0, d % 8 == 0, inter % 8 == 0,
 * E <= 256, num_groups % E == 0 when rank >= 0, num_groups <= 32768, and
 * 32-bit byte offsets inside each operand (rows_x*d, rows*inter and
 * 2*inter*d elements below 2^32 bytes).
 */
size_t moelb_grouped_ffn_workspace_bytes(int rows, int num_groups, int E, int d, int inter,
                                         int dtype);
int moelb_grouped_ffn(const void* x, int rows_x, int rows, const int32_t* group_off,
                      int num_groups, int E, int G, int rank,
                      const int32_t* gather, int gather_k,
                      int d, int inter, int dtype, const void* w13, const void* w2,
                      void* ws, size_t ws_bytes, void* y, void* stream);

/*
 * The same FFN in stages, for callers that schedule or time them apart:
 * MOELB_FFN_SCHEDULE (expert-major row order and tile tables, from group_off,
 * rank and gather, into ws), MOELB_FFN_GATE_UP (x -> SwiGLU activations in
 * ws), MOELB_FFN_DOWN (activations -> y).  `stages` is a bitwise OR of them;
 * moelb_grouped_ffn runs MOELB_FFN_ALL.  A stage reads what the earlier
 * stages left in ws, so the calls of one FFN take the same arguments and the
 * same ws, in stage order on one stream.  Same requirements and errors as
 * moelb_grouped_ffn; stages outside [1, MOELB_FFN_ALL] (after removing the
 * MOELB_FFN_PACKED_WEIGHTS option) return MOELB_EINVAL.
 */
enum moelb_ffn_stage {
  MOELB_FFN_SCHEDULE = 1,
  MOELB_FFN_GATE_UP = 2,
  MOELB_FFN_DOWN = 4,
  MOELB_FFN_ALL = 7,
  /* option, ORed with the stages: w13 and w2 are in the packed layout of
   * moelb_pack_weights (w13 packed with rows = 2*inter, K = d; w2 with rows =
   * d, K = inter).  Requires bf16, d % 64 == 0, inter % 64 == 0; outputs are
   * identical to the row-major call's. */
  MOELB_FFN_PACKED_WEIGHTS = 8
};
int moelb_grouped_ffn_stages(int stages, const void* x, int rows_x, int rows,
                             const int32_t* group_off, int num_groups, int E, int G, int rank,
                             const int32_t* gather, int gather_k, int d, int inter, int dtype,
                             const void* w13, const void* w2, void* ws, size_t ws_bytes,
                             void* y, void* stream);

/*
 * Expert weights in the packed layout the grouped FFN reads with
 * MOELB_FFN_PACKED_WEIGHTS (a layout of this library, not of the pages): the
 * 8 rows of a row block and one 64-wide K step are one contiguous KiB, so
 * each 64-lane DMA instruction of the GEMMs reads one KiB of DRAM instead of
 * 128-byte pieces of 8 rows.  For callers that load expert weights once and
 * run many steps (weights streamed by decode batches gain most).
 *  w       [E][rows][K] bf16, row-major
 *  packed  [E][rows/8][K/64][8][64] bf16 out: element (e, r, k) at
 *          ((e*rows/8 + r/8)*(K/64) + k/64)*512 + (r%8)*64 + k%64
 * w and packed are device buffers of E*rows*K elements, 16-byte aligned,
 * not overlapping.  Requires bf16, rows % 8 == 0, K % 64 == 0; otherwise
 * MOELB_EINVAL before any launch.
 */
int moelb_pack_weights(const void* w, int E, int rows, int K, int dtype, void* packed, void* stream);

/*
 * Top-k weighted combine (FreeBalance section 2.1: MoE(h) = sum_i W_i
 * expert_i(h); Libra "Repository Layout": the combine kernel).
 *   out[t] = sum_{j=0..k-1, ascending} wts[t,j] * y[pos[t*k+j]]  (+ shared[t])
 *  accumulated in fp32 and rounded to dtype.  Pairs with pos < 0 or
 *  pos >= rows_y contribute nothing.
 *  y      [rows_y,d] dtype
 *  pos    [T*k] int32, wts [T*k] fp32
 *  shared [T,d] dtype or NULL (added unweighted)
 *  out    [T,d] dtype out
 * Requires d % 8 == 0, 1 <= k <= 16.
 */
int moelb_combine(const void* y, int rows_y, const int32_t* pos, const float* wts, int T, int k,
                  int d, int dtype, const void* shared, void* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOELB_H */
