// Per-rank histograms, the replication plan and the Relief split.
//
// * Histogram -- Libra README "Key Ideas" (each GPU's own token demand) and
//   FreeBalance eq. 5 (the workload vector).  One workgroup per virtual rank,
//   LDS bins; each wave first folds the lanes that share lane 0's expert into
//   one LDS atomic (ballot), which takes the hot expert off the atomic path.
// * Plan -- Libra README "Key Ideas", locality-aware expert replication
//   planning (Phase 1 imports, Phase 2 balancing).  One workgroup; counts,
//   host masks and slots live in LDS.  Phase 1 runs one wave per rank (wave
//   argmax per import).  Phase 2 runs in one wave: lane r holds rank r's load,
//   each lane owns four experts; every step evaluates all candidate moves in
//   parallel and keeps the best accepted one by (load on the most-loaded rank,
//   then lower id) -- the move the sequential walk takes first -- with wave
//   reductions, and only the moved expert's contributions are updated.
// * Split -- Relief ("A Per-Step Load-Balancing Engine for Expert-Parallel MoE
//   Serving"), "The Relief Algorithm" and Algorithm 1: pairwise halving over
//   replica edges in edge-coloured, rank-disjoint rounds, no atomics in the
//   relaxation.  Whole tokens in int32.  Setup is parallel over experts (host
//   masks by atomic OR, transfer offsets by a block scan); the colouring and
//   the rounds run in one wave, whose own in-order LDS accesses order the
//   rounds without barriers.
#include <climits>

#include "common.h"

namespace {

// ---------------------------------------------------------------- histogram

constexpr int HIST_THREADS = 1024;
constexpr int HIST_BATCH = 16;  // ids loaded per thread before their atomics

__global__ __launch_bounds__(HIST_THREADS) void histogram_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                                  int E, int G, int32_t* __restrict__ counts) {
  __shared__ int bins[MOELB_MAX_E];
  const int s = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) bins[e] = 0;
  __syncthreads();
  const size_t per = (size_t)(T / G) * k;
  const int32_t* p = idx + (size_t)s * per;
  // HIST_BATCH coalesced loads in flight per thread before their atomics: the
  // loop would otherwise wait out one load latency per id
  for (size_t base = 0; base < per; base += (size_t)HIST_BATCH * blockDim.x) {
    int ev[HIST_BATCH];
#pragma unroll
    for (int u = 0; u < HIST_BATCH; ++u) {
      const size_t q = base + (size_t)u * blockDim.x + threadIdx.x;
      ev[u] = q < per ? p[q] : -1;
    }
#pragma unroll
    for (int u = 0; u < HIST_BATCH; ++u) {
      const int e = ev[u];
      const bool valid = e >= 0 && e < E;
      // fold the lanes that share lane 0's expert into one atomic
      const int e0 = __shfl(e, 0, MOELB_WAVE);
      const bool same = valid && e == e0;
      const uint64_t m = __ballot(same);
      if (lane_id() == 0 && same) atomicAdd(&bins[e0], __popcll(m));
      if (valid && !same) atomicAdd(&bins[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) counts[(size_t)s * E + e] = bins[e];
}

__global__ void column_sum_kernel(const int32_t* __restrict__ counts, int G, int E, int32_t* __restrict__ total) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int acc = 0;
    for (int s = 0; s < G; ++s) acc += counts[(size_t)s * E + e];
    total[e] = acc;
  }
}

// ---------------------------------------------------------------- shared helpers

// Share of a remote pool R for the host at position pos of m hosts.
__device__ __forceinline__ int even_share(int R, int m, int pos) { return R / m + (pos < R % m ? 1 : 0); }

// Position of rank r among the set bits of mask (ascending).
__device__ __forceinline__ int host_pos(uint64_t mask, int r) {
  return __popcll(mask & ((r == 0) ? 0ull : (~0ull >> (64 - r))));
}

__device__ __forceinline__ int clamp_rank(int h, int G) { return (h >= 0 && h < G) ? h : 0; }

// ---------------------------------------------------------------- plan

constexpr int PLAN_THREADS = 256;  // >= MOELB_MAX_E: one thread per expert

__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(const int32_t* __restrict__ counts,
                                                             const int32_t* __restrict__ home, int G, int E, int N,
                                                             int L, int32_t* __restrict__ replica,
                                                             int32_t* __restrict__ plan_load) {
  extern __shared__ __align__(16) int plan_smem[];
  int* c = plan_smem;                                         // [G][E]
  uint64_t* hostmask = reinterpret_cast<uint64_t*>(c + ((G * E + 1) & ~1));  // [E]
  int* slots = reinterpret_cast<int*>(hostmask + E);          // [G][N]
  int* nslots = slots + G * N;                                // [G]
  int* load = nslots + G;                                     // [G]

  const int tid = threadIdx.x;
  const int e = tid;
  for (int i = tid; i < G * E; i += blockDim.x) c[i] = counts[i];
  for (int i = tid; i < G * N; i += blockDim.x) slots[i] = -1;
  for (int r = tid; r < G; r += blockDim.x) nslots[r] = 0;
  int my_home = 0;
  if (e < E) {
    my_home = clamp_rank(home[e], G);
    hostmask[e] = 1ull << my_home;
  }
  __syncthreads();

  // Phase 1: wave w handles ranks w, w+4, ...: L rounds of a wave argmax over
  // (count desc, id asc) among non-resident experts with positive count.
  {
    const int wave = tid >> 6, lane = tid & 63, nwaves = blockDim.x >> 6;
    for (int r = wave; r < G; r += nwaves) {
      const int take = min(L, N);
      for (int i = 0; i < take; ++i) {
        int bc = 0, be = 0x7fffffff;
        for (int x = lane; x < E; x += 64) {
          const int hx = clamp_rank(home[x], G);
          const int cx = c[r * E + x];
          bool used = false;
          for (int j = 0; j < i; ++j) used |= slots[r * N + j] == x;
          if (hx != r && cx > 0 && !used && (cx > bc || (cx == bc && x < be))) {
            bc = cx;
            be = x;
          }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const int oc = __shfl_xor(bc, o, 64), oe = __shfl_xor(be, o, 64);
          if (oc > bc || (oc == bc && oe < be)) {
            bc = oc;
            be = oe;
          }
        }
        if (bc <= 0) break;  // uniform across the wave
        if (lane == 0) slots[r * N + i] = be;
      }
      if (lane == 0) {
        int n = 0;
        while (n < take && slots[r * N + n] >= 0) ++n;
        nslots[r] = n;
      }
    }
  }
  __syncthreads();
  // host masks from the Phase 1 imports
  if (e < E) {
    uint64_t m = hostmask[e];
    for (int r = 0; r < G; ++r)
      for (int j = 0; j < nslots[r]; ++j)
        if (slots[r * N + j] == e) m |= 1ull << r;
    hostmask[e] = m;
  }
  __syncthreads();

  // Phase 2 starts from the modeled loads of the Phase 1 placement
  for (int r = tid; r < G; r += blockDim.x) load[r] = 0;
  int* Rarr = reinterpret_cast<int*>(hostmask + E) + G * N + 2 * G;  // [E] remote pool per expert
  __syncthreads();
  if (e < E) {
    const uint64_t mask = hostmask[e];
    const int m = __popcll(mask);
    int R = 0;
    for (int s = 0; s < G; ++s)
      if (!((mask >> s) & 1ull)) R += c[s * E + e];
    Rarr[e] = R;
    int pos = 0;
    for (int s = 0; s < G; ++s)
      if ((mask >> s) & 1ull) {
        atomicAdd(&load[s], c[s * E + e] + even_share(R, m, pos));
        ++pos;
      }
  }
  __syncthreads();
  if (tid >= 64) return;

  // Phase 2 runs in one wave, everything in registers or LDS that only this
  // wave touches: lane r holds rank r's load and slot count; lane l owns
  // experts l, l+64, l+128, l+192 (mask and remote pool).  A move changes only
  // the contributions of the replicated expert, so loads update incrementally.
  const int lane = tid;
  int my_load = lane < G ? load[lane] : 0;
  int my_nslots = lane < G ? nslots[lane] : N;
  uint64_t emask[4];
  int eR[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int x = lane + 64 * q;
    emask[q] = x < E ? hostmask[x] : 0ull;
    eR[q] = x < E ? Rarr[x] : 0;
  }
  for (int step = 0; step <= G * N; ++step) {
    // most-loaded rank (ties: lowest) and whether any slot is free
    int a_load = lane < G ? my_load : INT_MIN, a = lane < G ? lane : 0x7fffffff;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const int ol = __shfl_xor(a_load, o, 64), oa = __shfl_xor(a, o, 64);
      if (ol > a_load || (ol == a_load && oa < a)) {
        a_load = ol;
        a = oa;
      }
    }
    if (__ballot(lane < G && my_nslots < N) == 0ull) break;
    // candidate move of each owned expert hosted on a: least-loaded eligible b
    int bb[4] = {-1, -1, -1, -1}, bl[4] = {0, 0, 0, 0};
    for (int r = 0; r < G; ++r) {
      const int lr = __shfl(my_load, r, 64), nr = __shfl(my_nslots, r, 64);
      if (nr >= N) continue;  // uniform
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (!((emask[q] >> r) & 1ull) && (bb[q] < 0 || lr < bl[q])) {
          bb[q] = r;
          bl[q] = lr;
        }
      }
    }
    unsigned long long key = 0ull;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int x = lane + 64 * q;
      const uint64_t mask = emask[q];
      if (x < E && ((mask >> a) & 1ull) && eR[q] > 0 && bb[q] >= 0) {
        const int b = bb[q];
        const int m = __popcll(mask);
        const int share_a = even_share(eR[q], m, host_pos(mask, a));
        const uint64_t mask2 = mask | (1ull << b);
        const int R2 = eR[q] - c[b * E + x];
        const int new_a = a_load - share_a + even_share(R2, m + 1, host_pos(mask2, a));
        const int new_b = bl[q] + c[b * E + x] + even_share(R2, m + 1, host_pos(mask2, b));
        if (max(new_a, new_b) < a_load) {
          const int contrib = c[a * E + x] + share_a;
          const unsigned long long k2 = (static_cast<unsigned long long>(static_cast<unsigned>(contrib)) << 16) |
                                        (static_cast<unsigned long long>(255 - x) << 8) | static_cast<unsigned>(b);
          key = k2 > key ? k2 : key;
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long ok = __shfl_xor(key, o, 64);
      key = ok > key ? ok : key;
    }
    if (key == 0ull) break;
    const int be = 255 - static_cast<int>((key >> 8) & 0xffull);
    const int b = static_cast<int>(key & 0xffull);
    // owner's state of be before the move, broadcast
    const int owner = be & 63, qq = be >> 6;
    uint64_t om = 0ull;
    int oR = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q == qq) {
        om = emask[q];
        oR = eR[q];
      }
    const uint64_t mask_old = __shfl(om, owner, 64);
    const int R_old = __shfl(oR, owner, 64);
    const uint64_t mask_new = mask_old | (1ull << b);
    const int R_new = R_old - c[b * E + be];
    // every rank updates its own load with be's contribution change
    if (lane < G) {
      const int m0 = __popcll(mask_old), m1 = m0 + 1;
      const int cr = c[lane * E + be];
      const int before = ((mask_old >> lane) & 1ull) ? cr + even_share(R_old, m0, host_pos(mask_old, lane)) : 0;
      const int after = ((mask_new >> lane) & 1ull) ? cr + even_share(R_new, m1, host_pos(mask_new, lane)) : 0;
      my_load += after - before;
      if (lane == b) {
        slots[b * N + my_nslots] = be;
        my_nslots += 1;
      }
    }
    if (lane == owner) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q == qq) {
          emask[q] = mask_new;
          eR[q] = R_new;
        }
    }
  }
  // every slot written in Phase 2 was written by this wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  for (int i = lane; i < G * N; i += 64) replica[i] = slots[i];
  if (plan_load && lane < G) plan_load[lane] = my_load;
}

// ---------------------------------------------------------------- swap planner
//
// FreeBalance ("FreeBalance: Pre-Routing Online MoE Load Balancing via
// Residual Workload Prediction"), section 3.3 and Algorithm 1: pairwise
// expert swaps between the most- and the least-loaded rank, each the one
// with the largest drop of Phi(L) = max L + gamma * sum (L - mean)^2 (eq. 8;
// a swap moves d = n_a - n_b pairs from a to b, so the variance term drops
// by 2 d (L_a - L_b - d), eq. 6-7), ties to the lower e_a then e_b; an
// expert moves at most once, each rank takes part in at most `budget` swaps,
// and planning stops when L_a - L_b <= tau or no swap lowers Phi.  Exact
// integer arithmetic: the benefit is kept times gamma's denominator.  One
// workgroup: wave 0 finds the rank pair, every thread scores candidate
// pairs, block reductions pick the swap, thread 0 applies it.

constexpr int SWAP_THREADS = 256;  // >= MOELB_MAX_E

__device__ __forceinline__ long long wave_max_i64(long long v) {
  for (int o = 32; o > 0; o >>= 1) {
    const long long w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ int wave_min_i32(int v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}

__global__ __launch_bounds__(SWAP_THREADS) void swap_plan_kernel(const int32_t* __restrict__ counts,
                                                                  const int32_t* __restrict__ home_in, int G, int E,
                                                                  int tau, int gamma_num, int gamma_den, int budget,
                                                                  int32_t* __restrict__ home_out,
                                                                  int32_t* __restrict__ swaps,
                                                                  int32_t* __restrict__ n_swaps,
                                                                  int32_t* __restrict__ load_out) {
  __shared__ int n[MOELB_MAX_E], where[MOELB_MAX_E], moved[MOELB_MAX_E];
  __shared__ int list_a[MOELB_MAX_E], list_b[MOELB_MAX_E];
  __shared__ int load[MOELB_MAX_G], left[MOELB_MAX_G];
  __shared__ long long red_b[SWAP_THREADS / 64];
  __shared__ int red_t[SWAP_THREADS / 64];
  __shared__ int s_a, s_b, s_other, s_na, s_nb, s_stop, s_nsw;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int r = tid; r < G; r += SWAP_THREADS) {
    load[r] = 0;
    left[r] = budget;
  }
  if (tid == 0) s_nsw = 0;
  __syncthreads();
  if (tid < E) {
    int sum = 0;
    for (int s2 = 0; s2 < G; ++s2) sum += counts[(size_t)s2 * E + tid];
    const int h = home_in[tid];
    n[tid] = sum;
    where[tid] = (h >= 0 && h < G) ? h : 0;
    moved[tid] = 0;
    atomicAdd(&load[where[tid]], sum);
  }
  __syncthreads();
  for (;;) {
    if (wave == 0) {
      // a: most loaded (ties lower rank), b: least loaded (ties lower rank)
      const int l = lane < G ? load[lane] : 0;
      const long long ka = lane < G ? (long long)l * 64 + (63 - lane) : LLONG_MIN;
      const int a = 63 - (int)(wave_max_i64(ka) & 63);
      const long long kb = lane < G ? -(long long)l * 64 + (63 - lane) : LLONG_MIN;
      const int b = 63 - (int)(wave_max_i64(kb) & 63);
      // largest load outside {a, b}
      const long long ko = (lane < G && lane != a && lane != b) ? (long long)l : LLONG_MIN;
      const long long other = wave_max_i64(ko);
      if (lane == 0) {
        s_a = a;
        s_b = b;
        s_other = other == LLONG_MIN ? INT_MIN : (int)other;
        s_stop = (load[a] - load[b] <= tau || left[a] == 0 || left[b] == 0) ? 1 : 0;
        s_na = 0;
        s_nb = 0;
      }
    }
    __syncthreads();
    if (s_stop) break;
    const int a = s_a, b = s_b;
    if (tid < E && !moved[tid]) {
      if (where[tid] == a) list_a[atomicAdd(&s_na, 1)] = tid;
      if (where[tid] == b) list_b[atomicAdd(&s_nb, 1)] = tid;
    }
    __syncthreads();
    const int na = s_na, nb = s_nb;
    const long long la = load[a], lb = load[b], gap = la - lb;
    const long long other = s_other;
    long long best = 0;  // benefit x gamma_den; only positive ones count
    int best_t = INT_MAX;
    for (int i = tid; i < na * nb; i += SWAP_THREADS) {
      const int ea = list_a[i / nb], eb = list_b[i % nb];
      const long long d = (long long)n[ea] - n[eb];
      const long long na2 = la - d, nb2 = lb + d;
      long long m = na2 > nb2 ? na2 : nb2;
      m = other > m ? other : m;
      const long long ben = (long long)gamma_den * (la - m) + (long long)gamma_num * 2 * d * (gap - d);
      const int t = (ea << 8) | eb;
      if (ben > 0 && (ben > best || (ben == best && t < best_t))) {
        best = ben;
        best_t = t;
      }
    }
    // block arg-max of the benefit, then the smallest (e_a, e_b) among its holders
    const long long wb = wave_max_i64(best);
    const int wt = wave_min_i32(best == wb ? best_t : INT_MAX);
    if (lane == 0) {
      red_b[wave] = wb;
      red_t[wave] = wt;
    }
    __syncthreads();
    if (tid == 0) {
      long long bb = 0;
      int bt = INT_MAX;
      for (int w = 0; w < SWAP_THREADS / 64; ++w)
        if (red_b[w] > bb || (red_b[w] == bb && red_t[w] < bt)) {
          bb = red_b[w];
          bt = red_t[w];
        }
      if (bb <= 0) {
        s_stop = 1;
      } else {
        const int ea = bt >> 8, eb = bt & 255;
        const int d = n[ea] - n[eb];
        load[a] -= d;
        load[b] += d;
        where[ea] = b;
        where[eb] = a;
        moved[ea] = moved[eb] = 1;
        --left[a];
        --left[b];
        if (swaps) {
          swaps[2 * s_nsw] = ea;
          swaps[2 * s_nsw + 1] = eb;
        }
        ++s_nsw;
      }
    }
    __syncthreads();
    if (s_stop) break;
  }
  if (tid < E) home_out[tid] = where[tid];
  if (tid < G) load_out[tid] = load[tid];
  if (tid == 0 && n_swaps) *n_swaps = s_nsw;
}

// ---------------------------------------------------------------- split

constexpr int SPLIT_THREADS = 256;                        // >= MOELB_MAX_E: one thread per expert
constexpr int MAX_TRANSFERS = MOELB_MAX_G * MOELB_MAX_N;  // one per replica slot
constexpr int COLOUR_WORDS = 32;                          // up to 1024 colours
constexpr int TR_PER_LANE = MAX_TRANSFERS / 64;

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

// variant: MOELB_SPLIT_* (include/moelb.h).  Relief, and the two ablations
// that change one ingredient of its pairwise move, share the round schedule;
// Libra's greedy sharding starts from the pools on their homes and needs no
// schedule.
__global__ __launch_bounds__(SPLIT_THREADS) void split_kernel(const int32_t* __restrict__ counts,
                                                               const int32_t* __restrict__ home,
                                                               const int32_t* __restrict__ replica, int G, int E,
                                                               int N, int passes, int eps, int variant,
                                                               const int32_t* __restrict__ sched_in,
                                                               int32_t* __restrict__ sched_out,
                                                               int32_t* __restrict__ host_count,
                                                               int32_t* __restrict__ load_out) {
  __shared__ unsigned long long hostmask[MOELB_MAX_E];
  __shared__ int xhome[MOELB_MAX_E];        // pool mass on the home rank (replicated experts)
  __shared__ int toff[MOELB_MAX_E + 1];     // first transfer of each expert
  __shared__ int t_u[MAX_TRANSFERS], t_v[MAX_TRANSFERS], t_x[MAX_TRANSFERS];
  __shared__ int t_e[MAX_TRANSFERS];
  __shared__ unsigned used[MOELB_MAX_G][COLOUR_WORDS];
  __shared__ int load[MOELB_MAX_G];
  __shared__ int snap[MOELB_MAX_G];         // Jacobi: loads at the start of the pass
  __shared__ int wave_sum[SPLIT_THREADS / 64];
  const bool greedy = variant == MOELB_SPLIT_LIBRA_GREEDY;
  const bool no_reverse = variant == MOELB_SPLIT_NO_REVERSE;
  const bool jacobi = variant == MOELB_SPLIT_JACOBI;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int e = tid;
  for (int r = tid; r < G; r += blockDim.x) load[r] = 0;
  for (int i = tid; i < G * COLOUR_WORDS; i += blockDim.x) used[i / COLOUR_WORDS][i % COLOUR_WORDS] = 0u;
  // replica slots (at most 2 per thread) are fetched with the home ranks
  const int rs0 = tid < G * N ? replica[tid] : -1;
  const int rs1 = tid + SPLIT_THREADS < G * N ? replica[tid + SPLIT_THREADS] : -1;
  int my_home = 0;
  if (e < E) {
    my_home = clamp_rank(home[e], G);
    hostmask[e] = 1ull << my_home;
  }
  __syncthreads();
  // replica slots set their host bits
  if (rs0 >= 0 && rs0 < E) atomicOr(&hostmask[rs0], 1ull << (tid / N));
  if (rs1 >= 0 && rs1 < E) atomicOr(&hostmask[rs1], 1ull << ((tid + SPLIT_THREADS) / N));
  __syncthreads();

  // fixed loads, initial even split, unreplicated pools.  Counts are loaded 8
  // ranks at a time (independent loads in flight together).
  uint64_t mask = 0;
  int R = 0, m = 0;
  if (e < E) {
    mask = hostmask[e];
    m = __popcll(mask);
  }
  for (int s0 = 0; s0 < G; s0 += 8) {
    int cs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) cs[i] = (counts && e < E && s0 + i < G) ? counts[(size_t)(s0 + i) * E + e] : 0;
    if (e < E) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (s0 + i >= G) break;
        if ((mask >> (s0 + i)) & 1ull)
          atomicAdd(&load[s0 + i], cs[i]);
        else
          R += cs[i];
      }
    }
  }
  if (e < E && host_count) {
    for (int r = 0; r < G; ++r) host_count[(size_t)e * G + r] = 0;
    if (m == 1) host_count[(size_t)e * G + my_home] = R;  // its load is added with the shares below
  }
  // transfer list: (home(e), v, e) for e ascending, v ascending; offsets by a block scan
  {
    const int cnt = (e < E) ? m - 1 : 0;
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wave_sum[w];
    if (e < E) toff[e] = base + incl - cnt;
    if (tid == SPLIT_THREADS - 1) toff[E] = base + incl;  // E <= SPLIT_THREADS
  }
  __syncthreads();
  {
    // shares of the pools (even split, or for the greedy the whole pool on the
    // home; an unreplicated pool all at its home), summed over the wave per rank
    const bool repl = e < E && m > 1;
    int t = repl ? toff[e] : 0, pos = 0;
    for (int r = 0; r < G; ++r) {
      int share = 0;
      if (repl && ((mask >> r) & 1ull)) {
        share = greedy ? (r == my_home ? R : 0) : even_share(R, m, pos);
        ++pos;
        if (r == my_home) {
          xhome[e] = share;
        } else {
          t_u[t] = my_home;
          t_v[t] = r;
          t_e[t] = e;
          t_x[t] = share;
          ++t;
        }
      } else if (e < E && m == 1 && r == my_home) {
        share = R;
      }
      if (share != 0) atomicAdd(&load[r], share);
    }
  }
  const int n = toff[E];
  __syncthreads();
  if (tid >= 64) return;

  if (greedy) {
    // Libra's sharding, one wave: the most-loaded rank a hands
    // min(mass, gap >> 1) tokens of its replicated expert with the most mass
    // on it (ties: lower id) to that expert's least-loaded other host b
    // (ties: lower rank), if load[a] - load[b] >= 2; lane l owns experts
    // l + 64 q.  At most passes x n moves.
    const int max_moves = passes * max(1, n);
    for (int it = 0; it < max_moves; ++it) {
      unsigned long long key = 0ull;
      if (lane < G) key = ((unsigned long long)((uint32_t)load[lane] ^ 0x80000000u) << 6) | (unsigned)(63 - lane);
      const int a = 63 - (int)(wave_max_u64(key) & 63);
      const int load_a = load[a];
      unsigned long long best = 0ull;
      int best_b = 0, best_d = 0;
      for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        if (e >= E) break;
        const int t0 = toff[e], t1 = toff[e + 1];
        if (t1 == t0) continue;  // unreplicated
        const int hh = t_u[t0];  // the home
        int mass_a = 0, b = -1, lb = 0;
        if (hh == a) {
          mass_a = xhome[e];
        } else {
          b = hh;
          lb = load[hh];
        }
        for (int t = t0; t < t1; ++t) {
          const int v = t_v[t];
          if (v == a) {
            mass_a = t_x[t];
          } else {
            const int l = load[v];
            if (b < 0 || l < lb || (l == lb && v < b)) {
              b = v;
              lb = l;
            }
          }
        }
        if (mass_a > 0 && (long long)load_a - lb >= 2) {
          const unsigned long long k = ((unsigned long long)(uint32_t)mass_a << 8) | (unsigned)(255 - e);
          if (k > best) {
            best = k;
            best_b = b;
            best_d = min(mass_a, (int)(((long long)load_a - lb) >> 1));
          }
        }
      }
      const unsigned long long wbest = wave_max_u64(best);
      if (wbest == 0ull) break;
      const int e = 255 - (int)(wbest & 255);
      if (lane == (e & 63)) {
        const int b = best_b, d = best_d;
        load[a] -= d;
        load[b] += d;
        const int t0 = toff[e], t1 = toff[e + 1];
        if (t_u[t0] == a) xhome[e] -= d;
        if (t_u[t0] == b) xhome[e] += d;
        for (int t = t0; t < t1; ++t) {
          if (t_v[t] == a) t_x[t] -= d;
          if (t_v[t] == b) t_x[t] += d;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
    for (int t = lane; t < n; t += 64) {
      const int x = t_e[t];
      host_count[(size_t)x * G + t_v[t]] = t_x[t];
      if (t == toff[x]) host_count[(size_t)x * G + t_u[t]] = xhome[x];
    }
    for (int r = lane; r < G; r += 64) load_out[r] = load[r];
    return;
  }

  // One wave from here.  The round schedule depends on the placement only: a
  // schedule from moelb_split_schedule for this same transfer list is used as
  // it is (checked transfer by transfer); otherwise greedy edge colouring in
  // list order.  Fast path: lane r holds rank r's used colours below 64 in a
  // register; if some transfer finds none free, the colouring is redone with
  // LDS words (1024 colours).
  int my_col[TR_PER_LANE];
#pragma unroll
  for (int q = 0; q < TR_PER_LANE; ++q) my_col[q] = 0;
  int ncol = 0;
  bool wide = false;
  bool scheduled = false;
  if (sched_in && sched_in[0] == n && sched_in[1] >= 0 && sched_in[1] <= n) {
    bool diff = false;
    for (int t = lane; t < n; t += 64)
      diff |= sched_in[2 + 3 * t] != t_u[t] || sched_in[3 + 3 * t] != t_v[t] || sched_in[4 + 3 * t] < 0 ||
              sched_in[4 + 3 * t] >= sched_in[1];
    scheduled = __ballot(diff) == 0ull;
    if (scheduled) {
      ncol = sched_in[1];
#pragma unroll
      for (int q = 0; q < TR_PER_LANE; ++q)
        if (lane + 64 * q < n) my_col[q] = sched_in[4 + 3 * (lane + 64 * q)];
    }
  }
  if (!scheduled) {
    uint32_t used_lo = 0u, used_hi = 0u;  // rank `lane`'s used colours 0..63
    const int my_u = lane < n ? t_u[lane] : 0, my_v = lane < n ? t_v[lane] : 0;
    for (int t = 0; t < n; ++t) {
      const int src = t & 63;
      int u, v;
      if (t < 64) {  // endpoints from registers, broadcast with readlane
        u = __builtin_amdgcn_readlane(my_u, src);
        v = __builtin_amdgcn_readlane(my_v, src);
      } else {
        u = t_u[t];
        v = t_v[t];
        u = __builtin_amdgcn_readfirstlane(u);
        v = __builtin_amdgcn_readfirstlane(v);
      }
      const uint32_t blo = __builtin_amdgcn_readlane(used_lo, u) | __builtin_amdgcn_readlane(used_lo, v);
      const uint32_t bhi = __builtin_amdgcn_readlane(used_hi, u) | __builtin_amdgcn_readlane(used_hi, v);
      if ((blo & bhi) == ~0u) {
        wide = true;
        break;
      }
      const int col = blo != ~0u ? __builtin_ctz(~blo) : 32 + __builtin_ctz(~bhi);
      if (lane == u || lane == v) {
        if (col < 32)
          used_lo |= 1u << col;
        else
          used_hi |= 1u << (col - 32);
      }
#pragma unroll
      for (int q = 0; q < TR_PER_LANE; ++q)
        if (t == lane + 64 * q) my_col[q] = col;
      ncol = max(ncol, col + 1);
    }
  }
  if (!scheduled && wide) {
    ncol = 0;
    for (int t = 0; t < n; ++t) {
      const int u = t_u[t], v = t_v[t];
      const unsigned fr = lane < COLOUR_WORDS ? ~(used[u][lane] | used[v][lane]) : 0u;
      const uint64_t nz = __ballot(fr != 0u);
      const int w = nz ? __ffsll(static_cast<long long>(nz)) - 1 : 0;
      const int col = w * 32 + __builtin_ctz(__shfl(fr, w, 64) | (nz ? 0u : 1u));
      if (lane == w) {
        used[u][w] |= 1u << (col & 31);
        used[v][w] |= 1u << (col & 31);
      }
#pragma unroll
      for (int q = 0; q < TR_PER_LANE; ++q)
        if (t == lane + 64 * q) my_col[q] = col;
      ncol = max(ncol, col + 1);
    }
  }
  if (sched_out) {
    // schedule only: the transfer list and its colours, nothing else
    if (lane == 0) {
      sched_out[0] = n;
      sched_out[1] = ncol;
    }
#pragma unroll
    for (int q = 0; q < TR_PER_LANE; ++q) {
      const int t = lane + 64 * q;
      if (t < n) {
        sched_out[2 + 3 * t] = t_u[t];
        sched_out[3 + 3 * t] = t_v[t];
        sched_out[4 + 3 * t] = my_col[q];
      }
    }
    return;
  }
  // relaxation: passes x rounds; the transfers of a round touch disjoint
  // ranks (and experts), and one wave applies them in order with its own LDS
  // accesses.  A pass that moves nothing leaves every later pass unchanged,
  // so the loop stops there.
  if (n <= 64) {
    // one transfer per lane, its endpoints and mass in registers (a scalar
    // walk over the transfers in round order, loads and masses in lanes of
    // registers moved by readlane, was exact but twice as slow: 72 against 36
    // us for 12 passes over 30 transfers)
    const bool has = lane < n;
    const int u = has ? t_u[lane] : 0, v = has ? t_v[lane] : 0, x = has ? t_e[lane] : 0;
    const int col = has ? my_col[0] : -1;
    int tx = has ? t_x[lane] : 0;
    for (int p = 0; p < passes; ++p) {
      bool moved = false;
      if (jacobi) {
        for (int r = lane; r < G; r += 64) snap[r] = load[r];
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      }
      for (int rd = 0; rd < ncol; ++rd) {
        if (col == rd) {
          const int lu = load[u], lv = load[v], xh = xhome[x];
          const int gap = jacobi ? snap[u] - snap[v] : lu - lv;
          int delta = (gap < 0 ? -gap : gap) >> (jacobi ? 2 : 1);
          delta = min(delta, gap > 0 ? xh : tx);
          if (no_reverse && gap <= 0) delta = 0;
          if (delta > eps) {
            const int sd = gap > 0 ? delta : -delta;  // mass moved from u to v
            load[u] = lu - sd;
            load[v] = lv + sd;
            xhome[x] = xh - sd;
            tx += sd;
            moved = true;
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      }
      if (__ballot(moved) == 0ull) break;
    }
    if (has) t_x[lane] = tx;
  } else {
    for (int p = 0; p < passes; ++p) {
      bool moved = false;
      if (jacobi) {
        for (int r = lane; r < G; r += 64) snap[r] = load[r];
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      }
      for (int rd = 0; rd < ncol; ++rd) {
#pragma unroll
        for (int q = 0; q < TR_PER_LANE; ++q) {
          const int t = lane + 64 * q;
          if (t < n && my_col[q] == rd) {
            const int u = t_u[t], v = t_v[t], x = t_e[t];
            const int gap = jacobi ? snap[u] - snap[v] : load[u] - load[v];
            int delta = (gap < 0 ? -gap : gap) >> (jacobi ? 2 : 1);
            const int limit = gap > 0 ? xhome[x] : t_x[t];
            delta = min(delta, limit);
            if (no_reverse && gap <= 0) delta = 0;
            if (delta > eps) {
              if (gap > 0) {
                load[u] -= delta;
                load[v] += delta;
                xhome[x] -= delta;
                t_x[t] += delta;
              } else {
                load[v] -= delta;
                load[u] += delta;
                t_x[t] -= delta;
                xhome[x] += delta;
              }
              moved = true;
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      }
      if (__ballot(moved) == 0ull) break;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  for (int t = lane; t < n; t += 64) {
    const int x = t_e[t];
    host_count[(size_t)x * G + t_v[t]] = t_x[t];
    if (t == toff[x]) host_count[(size_t)x * G + t_u[t]] = xhome[x];  // t_u is x's home
  }
  for (int r = lane; r < G; r += 64) load_out[r] = load[r];
}

// ---------------------------------------------------------------- water-filling and proportional splits

// Unsigned integers of PW 32-bit words, least significant first, for the
// proportional rule's exact shares: with at most PROP_MAX_HOSTS hosts, a
// product of the other hosts' (level + 1), each at most 2^31, times a pool
// below 2^31, stays below 2^496.
constexpr int PW = 16;
constexpr int PROP_MAX_HOSTS = 16;

__device__ __forceinline__ void big_set(uint32_t (&a)[PW], uint32_t v) {
#pragma unroll
  for (int i = 0; i < PW; ++i) a[i] = i == 0 ? v : 0u;
}
__device__ __forceinline__ void big_copy(uint32_t (&a)[PW], const uint32_t (&b)[PW]) {
#pragma unroll
  for (int i = 0; i < PW; ++i) a[i] = b[i];
}
__device__ __forceinline__ void big_mul(uint32_t (&a)[PW], uint32_t f) {
  uint64_t c = 0;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const uint64_t t = (uint64_t)a[i] * f + c;
    a[i] = (uint32_t)t;
    c = t >> 32;
  }
}
__device__ __forceinline__ void big_add(uint32_t (&a)[PW], const uint32_t (&b)[PW]) {
  uint64_t c = 0;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const uint64_t t = (uint64_t)a[i] + b[i] + c;
    a[i] = (uint32_t)t;
    c = t >> 32;
  }
}
// a -= b, for a >= b
__device__ __forceinline__ void big_sub(uint32_t (&a)[PW], const uint32_t (&b)[PW]) {
  int64_t br = 0;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int64_t t = (int64_t)a[i] - (int64_t)b[i] - br;
    a[i] = (uint32_t)t;
    br = t < 0 ? 1 : 0;
  }
}
__device__ __forceinline__ int big_cmp(const uint32_t (&a)[PW], const uint32_t (&b)[PW]) {
#pragma unroll
  for (int i = PW - 1; i >= 0; --i)
    if (a[i] != b[i]) return a[i] < b[i] ? -1 : 1;
  return 0;
}
// p = product of f[j] over j < m, j != r (f indexed by constants only, so it
// stays in registers)
__device__ __forceinline__ void big_prod_except(uint32_t (&p)[PW], const uint32_t (&f)[PROP_MAX_HOSTS], int m,
                                                int r) {
  big_set(p, 1u);
#pragma unroll
  for (int j = 0; j < PROP_MAX_HOSTS; ++j)
    if (j < m && j != r) big_mul(p, f[j]);
}

// A remainder estimate in double is within 1e-5 of the exact fractional share
// (R < 2^31, about twenty roundings of 2^-53); estimates further apart than
// this band order the remainders without the exact comparison.
constexpr double PROP_BAND = 1e-4;

// out = R P_r - q S: host r's exact remainder times S, for its floor q
__device__ __forceinline__ void big_rem(uint32_t (&out)[PW], int R, const uint32_t (&f)[PROP_MAX_HOSTS], int m,
                                        const uint32_t (&S)[PW], int r, int q) {
  uint32_t T[PW];
  big_prod_except(out, f, m, r);
  big_mul(out, (uint32_t)R);
  big_copy(T, S);
  big_mul(T, (uint32_t)q);
  big_sub(out, T);
}

// S = sum over r < m of P_r, the product of the f other than f[r]
__device__ __forceinline__ void big_pool_sum(uint32_t (&S)[PW], const uint32_t (&f)[PROP_MAX_HOSTS], int m) {
  uint32_t T[PW];
  big_set(S, 0u);
  for (int r = 0; r < m; ++r) {
    big_prod_except(T, f, m, r);
    big_add(S, T);
  }
}

// Relief's proportional relaxation ("Ablation Results (Table III)"; the rule
// is a reading): R tokens over m hosts in proportion to 1 / (l_j + 1), with
// f[j] = l_j + 1 and hosts in ascending rank.  Host r's exact share is
// R P_r / S, P_r the product of the other hosts' f and S the sum of the P_r;
// each host gets the floor, and the R - sum(floors) hosts with the largest
// remainders R P_r mod S (ties: lower rank) one more.  Each share is first
// estimated in double.  Where the estimate's fractional part lies at least
// PROP_BAND from a whole number, its floor is the exact floor; otherwise the
// floor is settled by exact comparisons.  Remainders are ordered by their
// estimates, and where two estimates fall within PROP_BAND by exact
// remainders, formed again for that pair.  S is formed only when one of
// these exact steps needs it.
__device__ void proportional_shares(int R, int m, const uint32_t (&f)[PROP_MAX_HOSTS],
                                    int (&give)[PROP_MAX_HOSTS]) {
  uint32_t S[PW], RP[PW], T[PW];
  bool have_s = false;
  double tot = 0.0;
  double frac[PROP_MAX_HOSTS];
#pragma unroll
  for (int j = 0; j < PROP_MAX_HOSTS; ++j) {
    if (j < m) tot += 1.0 / (double)f[j];
    give[j] = 0;
    frac[j] = 0.0;
  }
  int sumq = 0;
  for (int r = 0; r < m; ++r) {
    uint32_t fr = 1u;
#pragma unroll
    for (int j = 0; j < PROP_MAX_HOSTS; ++j) fr = j == r ? f[j] : fr;
    const double ex = (double)R / (double)fr / tot;
    int q = min(max((int)floor(ex), 0), R);
    const double part = ex - floor(ex);
    if (part < PROP_BAND || part > 1.0 - PROP_BAND) {
      if (!have_s) {
        big_pool_sum(S, f, m);
        have_s = true;
      }
      big_prod_except(RP, f, m, r);
      big_mul(RP, (uint32_t)R);
      for (;;) {  // q S <= R P_r (q = 0 always holds)
        big_copy(T, S);
        big_mul(T, (uint32_t)q);
        if (q > 0 && big_cmp(T, RP) > 0)
          --q;
        else
          break;
      }
      for (;;) {  // (q + 1) S > R P_r (holds by q = R, as P_r <= S)
        big_copy(T, S);
        big_mul(T, (uint32_t)(q + 1));
        if (big_cmp(T, RP) <= 0)
          ++q;
        else
          break;
      }
    }
#pragma unroll
    for (int j = 0; j < PROP_MAX_HOSTS; ++j)
      if (j == r) {
        give[j] = q;
        frac[j] = ex - (double)q;
      }
    sumq += q;
  }
  const int left = R - sumq;
  if (left == 0) return;
  uint32_t plus = 0;  // hosts that get one more
  for (int r = 0; r < m; ++r) {
    double frac_r = 0.0;  // frac[r] and give[r], read with constant indexes
    int q_r = 0;
#pragma unroll
    for (int j = 0; j < PROP_MAX_HOSTS; ++j) {
      frac_r = j == r ? frac[j] : frac_r;
      q_r = j == r ? give[j] : q_r;
    }
    int above = 0;      // hosts whose remainder ranks before r's
    uint32_t near = 0;  // hosts whose estimate lies within the band of r's
#pragma unroll
    for (int j = 0; j < PROP_MAX_HOSTS; ++j) {
      if (j >= m || j == r) continue;
      const double dlt = frac[j] - frac_r;
      if (dlt > PROP_BAND)
        ++above;
      else if (dlt >= -PROP_BAND)
        near |= 1u << j;
    }
    if (near) {
      if (!have_s) {
        big_pool_sum(S, f, m);
        have_s = true;
      }
      big_rem(RP, R, f, m, S, r, q_r);
      while (near) {
        const int j = __ffs(near) - 1;
        near &= near - 1u;
        int q_j = 0;
#pragma unroll
        for (int i = 0; i < PROP_MAX_HOSTS; ++i) q_j = i == j ? give[i] : q_j;
        big_rem(T, R, f, m, S, j, q_j);
        const int c = big_cmp(T, RP);
        above += (c > 0 || (c == 0 && j < r)) ? 1 : 0;
      }
    }
    if (above < left) plus |= 1u << r;
  }
#pragma unroll
  for (int j = 0; j < PROP_MAX_HOSTS; ++j) give[j] += (int)((plus >> j) & 1u);
}

// One proportional pass of one replicated expert (pool R over the m hosts in
// mask, from the snapshot loads less its own masses x): new masses, their
// change added to the loads; `changed` set if any mass moved.
__device__ __forceinline__ void proportional_pass(int R, int m, uint64_t mask, const int* snap, int32_t* x, int* load,
                                                  int& changed) {
  // hosts in ascending rank: slot j holds the j-th set bit of mask (G <= 16)
  uint32_t f[PROP_MAX_HOSTS];
  int hs[PROP_MAX_HOSTS], give[PROP_MAX_HOSTS];
  uint64_t mm = mask;
#pragma unroll
  for (int j = 0; j < PROP_MAX_HOSTS; ++j) {
    hs[j] = mm ? __ffsll(static_cast<long long>(mm)) - 1 : 0;
    f[j] = mm ? (uint32_t)(snap[hs[j]] - x[hs[j]]) + 1u : 1u;
    mm &= mm - 1ull;
  }
  proportional_shares(R, m, f, give);
#pragma unroll
  for (int j = 0; j < PROP_MAX_HOSTS; ++j) {
    if (j >= m) continue;
    const int h = hs[j];
    if (give[j] != x[h]) {
      changed = 1;
      atomicAdd(&load[h], give[j] - x[h]);
      x[h] = give[j];
    }
  }
}

// Relief's water-filling and proportional ablations ("Ablation Results
// (Table III)"; the rules are readings): replicated pools start from the even
// split; each pass, every replicated expert redistributes its whole pool R
// over its hosts from one snapshot of the loads, less its own mass on each
// host (levels l_h).  Water filling (prop = 0): the largest level z with
// sum_h max(0, z - l_h) <= R is filled, and the tokens left go one each to the
// hosts with l_h <= z in ascending rank.  Proportional (PROP): shares in
// proportion to 1 / (l_h + 1), exactly (proportional_shares; at most
// PROP_MAX_HOSTS hosts, i.e. G <= 16).  Stops after a pass that changes
// nothing.  One thread per expert; host_count holds the masses between passes.
template <bool PROP>
__global__ __launch_bounds__(SPLIT_THREADS) void split_water_fill_kernel(const int32_t* __restrict__ counts,
                                                                          const int32_t* __restrict__ home,
                                                                          const int32_t* __restrict__ replica,
                                                                          int G, int E, int N, int passes,
                                                                          int32_t* __restrict__ host_count,
                                                                          int32_t* __restrict__ load_out) {
  __shared__ unsigned long long hostmask[MOELB_MAX_E];
  __shared__ int load[MOELB_MAX_G];
  __shared__ int snap[MOELB_MAX_G];
  __shared__ int changed;
  const int tid = threadIdx.x;
  const int e = tid;
  for (int r = tid; r < G; r += blockDim.x) load[r] = 0;
  const int rs0 = tid < G * N ? replica[tid] : -1;
  const int rs1 = tid + SPLIT_THREADS < G * N ? replica[tid + SPLIT_THREADS] : -1;
  int my_home = 0;
  if (e < E) {
    my_home = clamp_rank(home[e], G);
    hostmask[e] = 1ull << my_home;
  }
  __syncthreads();
  if (rs0 >= 0 && rs0 < E) atomicOr(&hostmask[rs0], 1ull << (tid / N));
  if (rs1 >= 0 && rs1 < E) atomicOr(&hostmask[rs1], 1ull << ((tid + SPLIT_THREADS) / N));
  __syncthreads();
  uint64_t mask = 0;
  int m = 0, R = 0;
  int32_t* x = host_count + (size_t)(e < E ? e : 0) * G;
  if (e < E) {
    mask = hostmask[e];
    m = __popcll(mask);
    for (int s = 0; s < G; ++s) {
      const int c = counts[(size_t)s * E + e];
      if ((mask >> s) & 1ull)
        atomicAdd(&load[s], c);
      else
        R += c;
    }
    int pos = 0;
    for (int h = 0; h < G; ++h) {
      int share = 0;
      if ((mask >> h) & 1ull) {
        share = m == 1 ? R : even_share(R, m, pos);
        ++pos;
        atomicAdd(&load[h], share);
      }
      x[h] = share;
    }
  }
  const bool repl = e < E && m > 1;
  for (int p = 0; p < passes; ++p) {
    __syncthreads();
    for (int r = tid; r < G; r += blockDim.x) snap[r] = load[r];
    if (tid == 0) changed = 0;
    __syncthreads();
    if constexpr (PROP) {
      if (repl) proportional_pass(R, m, mask, snap, x, load, changed);
    } else if (repl) {
      int lo = INT_MAX;
      for (int h = 0; h < G; ++h)
        if ((mask >> h) & 1ull) lo = min(lo, snap[h] - x[h]);
      int hi = lo + R;
      while (lo < hi) {  // largest affordable level
        const int mid = lo + (hi - lo + 1) / 2;
        long long need = 0;
        for (int h = 0; h < G; ++h)
          if ((mask >> h) & 1ull) need += max(0, mid - (snap[h] - x[h]));
        if (need <= R)
          lo = mid;
        else
          hi = mid - 1;
      }
      int left = R;
      for (int h = 0; h < G; ++h)
        if ((mask >> h) & 1ull) left -= max(0, lo - (snap[h] - x[h]));
      for (int h = 0; h < G; ++h) {
        if (!((mask >> h) & 1ull)) continue;
        const int l = snap[h] - x[h];
        int give = max(0, lo - l);
        if (left > 0 && l <= lo) {
          ++give;
          --left;
        }
        if (give != x[h]) {
          changed = 1;
          atomicAdd(&load[h], give - x[h]);
          x[h] = give;
        }
      }
    }
    __syncthreads();
    if (!changed) break;
  }
  __syncthreads();
  for (int r = tid; r < G; r += blockDim.x) load_out[r] = load[r];
}

// ---------------------------------------------------------------- stale split

// The split of an earlier step reused (Relief, "Failure of Existing
// Approaches": how often the split is decided).  One thread per expert: the
// hosts (home + replica slots) serve their own pairs; a replicated expert's
// remote pool R is dealt in the fractions of host_count_prev over its current
// hosts (negative entries read as 0), floor(R p_h / P) each plus one for the
// R - sum(floors) hosts with the largest remainders (ties: lower rank), or
// evenly if P = 0; an unreplicated pool stays at home.
__global__ __launch_bounds__(SPLIT_THREADS) void split_stale_kernel(const int32_t* __restrict__ counts,
                                                                     const int32_t* __restrict__ home,
                                                                     const int32_t* __restrict__ replica, int G,
                                                                     int E, int N,
                                                                     const int32_t* __restrict__ prev,
                                                                     int32_t* __restrict__ host_count,
                                                                     int32_t* __restrict__ load_out) {
  __shared__ unsigned long long hostmask[MOELB_MAX_E];
  __shared__ int load[MOELB_MAX_G];
  const int tid = threadIdx.x;
  const int e = tid;
  for (int r = tid; r < G; r += blockDim.x) load[r] = 0;
  const int rs0 = tid < G * N ? replica[tid] : -1;
  const int rs1 = tid + SPLIT_THREADS < G * N ? replica[tid + SPLIT_THREADS] : -1;
  int my_home = 0;
  if (e < E) {
    my_home = clamp_rank(home[e], G);
    hostmask[e] = 1ull << my_home;
  }
  __syncthreads();
  if (rs0 >= 0 && rs0 < E) atomicOr(&hostmask[rs0], 1ull << (tid / N));
  if (rs1 >= 0 && rs1 < E) atomicOr(&hostmask[rs1], 1ull << ((tid + SPLIT_THREADS) / N));
  __syncthreads();
  if (e < E) {
    const uint64_t mask = hostmask[e];
    const int m = __popcll(mask);
    int R = 0;
    for (int s = 0; s < G; ++s) {
      const int c = counts[(size_t)s * E + e];
      if ((mask >> s) & 1ull)
        atomicAdd(&load[s], c);
      else
        R += c;
    }
    const int32_t* pe = prev + (size_t)e * G;
    long long P = 0;
    if (m > 1)
      for (int h = 0; h < G; ++h)
        if ((mask >> h) & 1ull) P += max(pe[h], 0);
    long long given = 0;  // sum of the floors
    if (m > 1 && P > 0)
      for (int h = 0; h < G; ++h)
        if ((mask >> h) & 1ull) given += (long long)R * max(pe[h], 0) / P;
    const long long left = R - given;
    int pos = 0;
    for (int h = 0; h < G; ++h) {
      int share = 0;
      if ((mask >> h) & 1ull) {
        if (m == 1) {
          share = R;
        } else if (P == 0) {
          share = even_share(R, m, pos);
        } else {
          const long long q = (long long)R * max(pe[h], 0);
          const long long rem = q % P;
          // place of h among the hosts by (remainder descending, rank ascending)
          int before = 0;
          for (int g = 0; g < G; ++g) {
            if (g == h || !((mask >> g) & 1ull)) continue;
            const long long rg = (long long)R * max(pe[g], 0) % P;
            before += (rg > rem || (rg == rem && g < h)) ? 1 : 0;
          }
          share = (int)(q / P) + (before < left ? 1 : 0);
        }
        ++pos;
        atomicAdd(&load[h], share);
      }
      host_count[(size_t)e * G + h] = share;
    }
  }
  __syncthreads();
  for (int r = tid; r < G; r += blockDim.x) load_out[r] = load[r];
}

}  // namespace

extern "C" int moelb_histogram(const int32_t* idx, int T, int k, int E, int G, int32_t* counts,
                               int32_t* expert_total, void* stream) {
  if (T < 0 || k < 1 || k > MOELB_MAX_K || E < 1 || E > MOELB_MAX_E || G < 1 || G > MOELB_MAX_G) return MOELB_EINVAL;
  if (T % G != 0 || !counts || (T > 0 && !idx)) return MOELB_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(histogram_kernel, dim3(G), dim3(HIST_THREADS), 0, s, idx, T, k, E, G, counts);
  MOELB_CHECK_LAUNCH();
  if (expert_total) {
    hipLaunchKernelGGL(column_sum_kernel, dim3(1), dim3(256), 0, s, counts, G, E, expert_total);
    MOELB_CHECK_LAUNCH();
  }
  return MOELB_OK;
}

extern "C" int moelb_plan(const int32_t* counts, const int32_t* home, int G, int E, int N, int L,
                          int32_t* replica, int32_t* plan_load, void* stream) {
  if (G < 1 || G > MOELB_MAX_G || E < 1 || E > MOELB_MAX_E || N < 0 || N > MOELB_MAX_N || L < 0 || L > N)
    return MOELB_EINVAL;
  if (!counts || !home || (N > 0 && !replica)) return MOELB_EINVAL;
  if (N == 0 && !plan_load) return MOELB_OK;
  const size_t lds =
      (size_t)((G * E + 1) & ~1) * 4 + (size_t)E * 8 + (size_t)G * N * 4 + (size_t)G * 8 + (size_t)E * 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!moelb_allow_lds(plan_kernel, lds)) return MOELB_ELAUNCH;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(PLAN_THREADS), lds, s, counts, home, G, E, N, L, replica,
                     plan_load);
  MOELB_CHECK_LAUNCH();
  return MOELB_OK;
}

extern "C" int moelb_split_scheduled(const int32_t* counts, const int32_t* home, const int32_t* replica,
                                     const int32_t* schedule, int G, int E, int N, int passes, int eps, int variant,
                                     int32_t* host_count, int32_t* load, void* stream) {
  if (G < 1 || G > MOELB_MAX_G || E < 1 || E > MOELB_MAX_E || N < 0 || N > MOELB_MAX_N) return MOELB_EINVAL;
  if (passes < 0 || passes > 1024 || eps < 0) return MOELB_EINVAL;
  if (variant < MOELB_SPLIT_RELIEF || variant > MOELB_SPLIT_PROPORTIONAL) return MOELB_EINVAL;
  // the proportional rule's exact arithmetic holds at most 16 hosts per expert
  if (variant == MOELB_SPLIT_PROPORTIONAL && G > 16) return MOELB_EINVAL;
  if (!counts || !home || (N > 0 && !replica) || !host_count || !load) return MOELB_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (variant == MOELB_SPLIT_WATER_FILL || variant == MOELB_SPLIT_PROPORTIONAL) {
    if (variant == MOELB_SPLIT_PROPORTIONAL)
      hipLaunchKernelGGL(split_water_fill_kernel<true>, dim3(1), dim3(SPLIT_THREADS), 0, s, counts, home,
                         N > 0 ? replica : home, G, E, N, passes, host_count, load);
    else
      hipLaunchKernelGGL(split_water_fill_kernel<false>, dim3(1), dim3(SPLIT_THREADS), 0, s, counts, home,
                         N > 0 ? replica : home, G, E, N, passes, host_count, load);
    MOELB_CHECK_LAUNCH();
    return MOELB_OK;
  }
  hipLaunchKernelGGL(split_kernel, dim3(1), dim3(SPLIT_THREADS), 0, s, counts, home, N > 0 ? replica : home, G, E,
                     N, passes, eps, variant, schedule, nullptr, host_count, load);
  MOELB_CHECK_LAUNCH();
  return MOELB_OK;
}

extern "C" int moelb_split_variant(const int32_t* counts, const int32_t* home, const int32_t* replica, int G,
                                   int E, int N, int passes, int eps, int variant, int32_t* host_count,
                                   int32_t* load, void* stream) {
  return moelb_split_scheduled(counts, home, replica, nullptr, G, E, N, passes, eps, variant, host_count, load,
                               stream);
}

extern "C" int moelb_split_schedule(const int32_t* home, const int32_t* replica, int G, int E, int N,
                                    int32_t* schedule, void* stream) {
  if (G < 1 || G > MOELB_MAX_G || E < 1 || E > MOELB_MAX_E || N < 0 || N > MOELB_MAX_N) return MOELB_EINVAL;
  if (!home || (N > 0 && !replica) || !schedule) return MOELB_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(split_kernel, dim3(1), dim3(SPLIT_THREADS), 0, s, nullptr, home, N > 0 ? replica : home, G, E,
                     N, 0, 0, (int)MOELB_SPLIT_RELIEF, nullptr, schedule, nullptr, nullptr);
  MOELB_CHECK_LAUNCH();
  return MOELB_OK;
}

extern "C" int moelb_split(const int32_t* counts, const int32_t* home, const int32_t* replica, int G, int E,
                           int N, int passes, int eps, int32_t* host_count, int32_t* load, void* stream) {
  return moelb_split_variant(counts, home, replica, G, E, N, passes, eps, MOELB_SPLIT_RELIEF, host_count, load,
                             stream);
}

extern "C" int moelb_plan_swaps(const int32_t* counts, const int32_t* home, int G, int E, int tau, int gamma_num,
                                int gamma_den, int max_swaps_per_rank, int32_t* home_out, int32_t* swaps,
                                int32_t* n_swaps, int32_t* load, void* stream) {
  if (G < 1 || G > MOELB_MAX_G || E < 1 || E > MOELB_MAX_E) return MOELB_EINVAL;
  if (tau < 0 || gamma_num < 0 || gamma_num > (1 << 12) || gamma_den < 1 || gamma_den > (1 << 20) ||
      max_swaps_per_rank < 0)
    return MOELB_EINVAL;
  if (!counts || !home || !home_out || !load) return MOELB_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(swap_plan_kernel, dim3(1), dim3(SWAP_THREADS), 0, s, counts, home, G, E, tau, gamma_num,
                     gamma_den, max_swaps_per_rank, home_out, swaps, n_swaps, load);
  MOELB_CHECK_LAUNCH();
  return MOELB_OK;
}

extern "C" int moelb_split_stale(const int32_t* counts, const int32_t* home, const int32_t* replica, int G, int E,
                                 int N, const int32_t* host_count_prev, int32_t* host_count, int32_t* load,
                                 void* stream) {
  if (G < 1 || G > MOELB_MAX_G || E < 1 || E > MOELB_MAX_E || N < 0 || N > MOELB_MAX_N) return MOELB_EINVAL;
  if (!counts || !home || (N > 0 && !replica) || !host_count_prev || !host_count || !load) return MOELB_EINVAL;
  if (host_count == host_count_prev) return MOELB_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(split_stale_kernel, dim3(1), dim3(SPLIT_THREADS), 0, s, counts, home, N > 0 ? replica : home,
                     G, E, N, host_count_prev, host_count, load);
  MOELB_CHECK_LAUNCH();
  return MOELB_OK;
}
