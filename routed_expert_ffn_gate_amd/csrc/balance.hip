// Per-rank histograms, the replication plan and the Relief split.
//
// * Histogram -- Libra README "Key Ideas" (each GPU's own token demand) and
//   FreeBalance eq. 5 (the workload vector).  One workgroup per virtual rank,
//   LDS bins; each wave first folds the lanes that share lane 0's expert into
//   one LDS atomic (ballot), which takes the hot expert off the atomic path.
// * Plan -- Libra README "Key Ideas", locality-aware expert replication
//   planning (Phase 1 imports, Phase 2 balancing).  One workgroup; counts,
//   host masks, slots and loads live in LDS.  Phase 1 runs one wave per rank
//   (wave argmax per import).  Each Phase 2 step evaluates every expert's
//   candidate move in parallel (one thread per expert) and keeps the best
//   accepted one by (load on the most-loaded rank, then lower id) -- the same
//   move the sequential walk takes first.
// * Split -- Relief ("A Per-Step Load-Balancing Engine for Expert-Parallel MoE
//   Serving"), "The Relief Algorithm" and Algorithm 1: pairwise halving over
//   replica edges in edge-coloured, rank-disjoint rounds, one barrier per
//   round, no atomics in the relaxation.  Whole tokens in int32.
#include "common.h"

namespace {

// ---------------------------------------------------------------- histogram

constexpr int HIST_THREADS = 1024;

__global__ __launch_bounds__(HIST_THREADS) void histogram_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                                  int E, int G, int32_t* __restrict__ counts) {
  __shared__ int bins[MOELB_MAX_E];
  const int s = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) bins[e] = 0;
  __syncthreads();
  const size_t per = (size_t)(T / G) * k;
  const int32_t* p = idx + (size_t)s * per;
  const size_t n_iter = (per + blockDim.x - 1) / blockDim.x;
  for (size_t it = 0; it < n_iter; ++it) {
    const size_t q = it * blockDim.x + threadIdx.x;
    const int e = q < per ? p[q] : -1;
    const bool valid = e >= 0 && e < E;
    // fold the lanes that share lane 0's expert into one atomic
    const int e0 = __shfl(e, 0, MOELB_WAVE);
    const bool same = valid && e == e0;
    const uint64_t m = __ballot(same);
    if (lane_id() == 0 && same) atomicAdd(&bins[e0], __popcll(m));
    if (valid && !same) atomicAdd(&bins[e], 1);
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
  __shared__ int s_a, s_any_free;
  __shared__ unsigned long long s_best;

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

  // Phase 2
  for (int step = 0; step <= G * N; ++step) {
    for (int r = tid; r < G; r += blockDim.x) load[r] = 0;
    if (tid == 0) s_best = 0ull;
    __syncthreads();
    int R = 0, m = 0;
    uint64_t mask = 0;
    if (e < E) {
      mask = hostmask[e];
      m = __popcll(mask);
      for (int s = 0; s < G; ++s)
        if (!((mask >> s) & 1ull)) R += c[s * E + e];
      int pos = 0;
      for (int s = 0; s < G; ++s)
        if ((mask >> s) & 1ull) {
          atomicAdd(&load[s], c[s * E + e] + even_share(R, m, pos));
          ++pos;
        }
    }
    __syncthreads();
    if (tid == 0) {
      int a = 0, any = 0;
      for (int r = 0; r < G; ++r) {
        if (load[r] > load[a]) a = r;
        any |= nslots[r] < N;
      }
      s_a = a;
      s_any_free = any;
    }
    __syncthreads();
    if (!s_any_free) break;
    const int a = s_a;
    int best_b = -1;
    if (e < E && ((mask >> a) & 1ull) && R > 0) {
      int b = -1;
      for (int r = 0; r < G; ++r)
        if (!((mask >> r) & 1ull) && nslots[r] < N && (b < 0 || load[r] < load[b])) b = r;
      if (b >= 0) {
        const int share_a = even_share(R, m, host_pos(mask, a));
        const uint64_t mask2 = mask | (1ull << b);
        const int R2 = R - c[b * E + e];
        const int new_a = load[a] - share_a + even_share(R2, m + 1, host_pos(mask2, a));
        const int new_b = load[b] + c[b * E + e] + even_share(R2, m + 1, host_pos(mask2, b));
        if (max(new_a, new_b) < load[a]) {
          const int contrib = c[a * E + e] + share_a;
          const unsigned long long key =
              (static_cast<unsigned long long>(static_cast<unsigned>(contrib)) << 16) | (0xffffu - e);
          atomicMax(&s_best, key);
          best_b = b;
        }
      }
    }
    __syncthreads();
    const unsigned long long best = s_best;
    if (best == 0ull) break;
    const int be = 0xffff - static_cast<int>(best & 0xffffull);
    if (e == be) {
      hostmask[e] = mask | (1ull << best_b);
      slots[best_b * N + nslots[best_b]] = e;
      nslots[best_b] += 1;
    }
    __syncthreads();
  }

  for (int i = tid; i < G * N; i += blockDim.x) replica[i] = slots[i];
  if (plan_load) {
    // final modeled loads
    for (int r = tid; r < G; r += blockDim.x) load[r] = 0;
    __syncthreads();
    if (e < E) {
      const uint64_t mask = hostmask[e];
      const int m = __popcll(mask);
      int R = 0;
      for (int s = 0; s < G; ++s)
        if (!((mask >> s) & 1ull)) R += c[s * E + e];
      int pos = 0;
      for (int s = 0; s < G; ++s)
        if ((mask >> s) & 1ull) {
          atomicAdd(&load[s], c[s * E + e] + even_share(R, m, pos));
          ++pos;
        }
    }
    __syncthreads();
    for (int r = tid; r < G; r += blockDim.x) plan_load[r] = load[r];
  }
}

// ---------------------------------------------------------------- split

constexpr int SPLIT_THREADS = 256;
constexpr int MAX_TRANSFERS = MOELB_MAX_G * MOELB_MAX_N;  // one per replica slot
constexpr int COLOUR_WORDS = 32;                          // up to 1024 colours

__global__ __launch_bounds__(SPLIT_THREADS) void split_kernel(const int32_t* __restrict__ counts,
                                                               const int32_t* __restrict__ home,
                                                               const int32_t* __restrict__ replica, int G, int E,
                                                               int N, int passes, int eps,
                                                               int32_t* __restrict__ host_count,
                                                               int32_t* __restrict__ load_out) {
  __shared__ uint64_t hostmask[MOELB_MAX_E];
  __shared__ int xhome[MOELB_MAX_E];        // pool mass on the home rank (replicated experts)
  __shared__ int toff[MOELB_MAX_E + 1];     // first transfer of each expert
  __shared__ int t_u[MAX_TRANSFERS], t_v[MAX_TRANSFERS], t_e[MAX_TRANSFERS], t_x[MAX_TRANSFERS];
  __shared__ int t_col[MAX_TRANSFERS];
  __shared__ int order[MAX_TRANSFERS];      // transfers sorted by colour
  __shared__ int round_off[MAX_TRANSFERS + 1];
  __shared__ unsigned used[MOELB_MAX_G][COLOUR_WORDS];
  __shared__ int load[MOELB_MAX_G];
  __shared__ int s_rounds, s_ntr;

  const int tid = threadIdx.x;
  const int e = tid;
  for (int r = tid; r < G; r += blockDim.x) load[r] = 0;
  for (int i = tid; i < G * COLOUR_WORDS; i += blockDim.x) used[i / COLOUR_WORDS][i % COLOUR_WORDS] = 0u;
  int my_home = 0;
  uint64_t mask = 0;
  if (e < E) {
    my_home = clamp_rank(home[e], G);
    mask = 1ull << my_home;
    for (int r = 0; r < G; ++r)
      for (int j = 0; j < N; ++j)
        if (replica[r * N + j] == e) mask |= 1ull << r;
    hostmask[e] = mask;
  }
  __syncthreads();

  // fixed loads, initial even split, unreplicated pools
  int R = 0, m = 0;
  if (e < E) {
    m = __popcll(mask);
    for (int s = 0; s < G; ++s) {
      const int cs = counts[(size_t)s * E + e];
      if ((mask >> s) & 1ull)
        atomicAdd(&load[s], cs);
      else
        R += cs;
    }
    for (int r = 0; r < G; ++r) host_count[(size_t)e * G + r] = 0;
    if (m == 1) {
      atomicAdd(&load[my_home], R);
      host_count[(size_t)e * G + my_home] = R;
    }
  }
  // transfer list: (home(e), v, e) for e ascending, v ascending
  if (tid == 0) {
    int n = 0;
    for (int x = 0; x < E; ++x) {
      toff[x] = n;
      n += __popcll(hostmask[x]) - 1;
    }
    toff[E] = n;
    s_ntr = n;
  }
  __syncthreads();
  if (e < E && m > 1) {
    int t = toff[e], pos = 0;
    for (int r = 0; r < G; ++r) {
      if (!((mask >> r) & 1ull)) continue;
      const int share = even_share(R, m, pos++);
      atomicAdd(&load[r], share);
      if (r == my_home) {
        xhome[e] = share;
      } else {
        t_u[t] = my_home;
        t_v[t] = r;
        t_e[t] = e;
        t_x[t] = share;
        ++t;
      }
    }
  }
  __syncthreads();

  // greedy edge colouring in list order, then transfers grouped by colour
  if (tid == 0) {
    const int n = s_ntr;
    int ncol = 0;
    for (int t = 0; t < n; ++t) {
      const int u = t_u[t], v = t_v[t];
      int col = 0;
      for (int w = 0; w < COLOUR_WORDS; ++w) {
        const unsigned fr = ~(used[u][w] | used[v][w]);
        if (fr) {
          col = w * 32 + __builtin_ctz(fr);
          break;
        }
      }
      used[u][col >> 5] |= 1u << (col & 31);
      used[v][col >> 5] |= 1u << (col & 31);
      t_col[t] = col;
      ncol = max(ncol, col + 1);
    }
    // counting sort by colour
    for (int r = 0; r <= ncol; ++r) round_off[r] = 0;
    for (int t = 0; t < n; ++t) round_off[t_col[t] + 1] += 1;
    for (int r = 0; r < ncol; ++r) round_off[r + 1] += round_off[r];
    for (int r = 0; r < ncol; ++r) {
      int q = round_off[r];
      for (int t = 0; t < n; ++t)
        if (t_col[t] == r) order[q++] = t;
    }
    s_rounds = ncol;
  }
  __syncthreads();

  // relaxation: passes x rounds, transfers of a round in parallel
  const int nrounds = s_rounds;
  for (int p = 0; p < passes; ++p) {
    for (int rd = 0; rd < nrounds; ++rd) {
      const int q = round_off[rd] + tid;
      if (q < round_off[rd + 1]) {
        const int t = order[q];
        const int u = t_u[t], v = t_v[t], x = t_e[t];
        const int gap = load[u] - load[v];
        int delta = (gap < 0 ? -gap : gap) >> 1;
        const int limit = gap > 0 ? xhome[x] : t_x[t];
        delta = min(delta, limit);
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
        }
      }
      __syncthreads();
    }
  }

  if (e < E && m > 1) {
    host_count[(size_t)e * G + my_home] = xhome[e];
    for (int t = toff[e]; t < toff[e + 1]; ++t) host_count[(size_t)e * G + t_v[t]] = t_x[t];
  }
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
  const size_t lds = (size_t)((G * E + 1) & ~1) * 4 + (size_t)E * 8 + (size_t)G * N * 4 + (size_t)G * 8;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!moelb_allow_lds(plan_kernel, lds)) return MOELB_ELAUNCH;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(PLAN_THREADS), lds, s, counts, home, G, E, N, L, replica,
                     plan_load);
  MOELB_CHECK_LAUNCH();
  return MOELB_OK;
}

extern "C" int moelb_split(const int32_t* counts, const int32_t* home, const int32_t* replica, int G, int E,
                           int N, int passes, int eps, int32_t* host_count, int32_t* load, void* stream) {
  if (G < 1 || G > MOELB_MAX_G || E < 1 || E > MOELB_MAX_E || N < 0 || N > MOELB_MAX_N) return MOELB_EINVAL;
  if (passes < 0 || passes > 1024 || eps < 0) return MOELB_EINVAL;
  if (!counts || !home || (N > 0 && !replica) || !host_count || !load) return MOELB_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(split_kernel, dim3(1), dim3(SPLIT_THREADS), 0, s, counts, home, N > 0 ? replica : home, G, E,
                     N, passes, eps, host_count, load);
  MOELB_CHECK_LAUNCH();
  return MOELB_OK;
}
