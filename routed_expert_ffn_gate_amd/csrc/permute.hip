// Local/remote permutation of token-expert pairs, and the optional row gather.
//
// Definition: Libra README "Key Ideas", two-stage locality-aware execution:
// pairs whose expert is hosted (resident or replicated) on the token's own
// rank form the MoE_local segment; the others are dispatched (MoE_remote) to a
// host chosen by the per-step split (Relief, "The Relief Algorithm").
//
// Deterministic stable counting sort in four launches:
//   1. count: one workgroup per chunk of up to MAX_CHUNK tokens (chunk_tokens()
//      shrinks it for small batches so the ranking runs on more workgroups
//      with shorter serial loops; chunks never straddle a
//      rank), LDS histogram of the chunk's experts;
//   2. scan: one workgroup per expert scans its chunk counts in token order,
//      giving each chunk's base rank inside its local group (reset per rank)
//      or inside the expert's remote pool; group sizes follow from the counts
//      and host_count; one more workgroup scans the group sizes into group_off;
//   3. rank + scatter: one workgroup per chunk; wave 0 ranks the chunk's pairs
//      in pair-id order with a ballot match loop over 64-pair steps (ranks of
//      equal experts inside a step from popcount below the lane) and writes
//      pos/perm; then all waves copy each token's row once into its k
//      destinations (read once, written k times).
//
// Batches of at most 8192 pairs with no rows to copy run the same sort in one
// workgroup instead (permute_one_wg_kernel below): at decode sizes the four
// launches cost more than their work.
//
// Two-phase form (the two stages run apart, so MoE_local can start before
// the split exists): the local phase does all of the above except what
// depends on host_count -- it places the local pairs and keeps each remote
// pair's place rho in its expert's remote pool; the remote phase turns
// host_count into host ranges and remote group offsets (after the local
// total) and places the remote pairs.  Both phases together give exactly the
// one-call result.
#include "common.h"

namespace {

constexpr int MAX_CHUNK = 128;

// Tokens per chunk: enough chunks (about 1024) to spread the ranking over the
// GPU, between 16 and MAX_CHUNK tokens.
inline int chunk_tokens(int T, int G) {
  const int per = T / G;
  const int want = (1024 + G - 1) / G;  // chunks per rank
  const int c = (per + want - 1) / want;
  return c < 16 ? 16 : (c > MAX_CHUNK ? MAX_CHUNK : c);
}
constexpr int SCAN_THREADS = 1024;

struct PermuteWs {
  int32_t* chunk_counts;  // [nchunks][E]
  int32_t* chunk_base;    // [nchunks][E]
  int32_t* host_rank;     // [E][G]  hosts of e in ascending rank, -1 padded
  int32_t* host_lo;       // [E][G]  first remote rank (rho) served by that host
  int32_t* host_hi;       // [E][G]  one past the last
  int32_t* gsize;         // [2GE]
  int32_t* remote_total;  // [E]    size of each expert's remote pool
  int32_t* rho;           // [T*k]  two-phase form: remote pair's place in its pool, -1 otherwise
};

inline size_t ws_layout(int T, int k, int E, int G, PermuteWs* w, char* base) {
  const int per = T / G;
  const int chunk = chunk_tokens(T, G);
  const int nchr = (per + chunk - 1) / chunk;
  const size_t nchunks = (size_t)G * (nchr > 0 ? nchr : 1);
  size_t off = 0;
  auto take = [&](int32_t** p, size_t n) {
    if (w) *p = reinterpret_cast<int32_t*>(base + off);
    off += moelb_align256(n * sizeof(int32_t));
  };
  PermuteWs dummy;
  PermuteWs* t = w ? w : &dummy;
  take(&t->chunk_counts, nchunks * E);
  take(&t->chunk_base, nchunks * E);
  take(&t->host_rank, (size_t)E * G);
  take(&t->host_lo, (size_t)E * G);
  take(&t->host_hi, (size_t)E * G);
  take(&t->gsize, (size_t)2 * G * E);
  take(&t->remote_total, (size_t)E);
  take(&t->rho, (size_t)T * k);
  return off;
}

// Host masks of experts [0, E) into LDS, by the whole workgroup: each expert's
// home bit, then one replica entry per thread ORed in (no thread walks the
// replica table).  Entries outside [0, E) are ignored.
__device__ __forceinline__ void block_host_masks(const int32_t* __restrict__ home,
                                                 const int32_t* __restrict__ replica, int G, int N, int E,
                                                 uint64_t* hmask) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int h = home[e];
    h = (h >= 0 && h < G) ? h : 0;
    hmask[e] = 1ull << h;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < G * N; q += blockDim.x) {
    const int e = replica[q];
    if (e >= 0 && e < E) atomicOr(reinterpret_cast<unsigned long long*>(&hmask[e]), 1ull << (q / N));
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ idx, int T, int k, int E, int G,
                                                    int chunk, int nchr, int32_t* __restrict__ chunk_counts) {
  __shared__ int bins[MOELB_MAX_E];
  const int c = blockIdx.x;
  const int s = c / nchr, ci = c % nchr;
  const int per = T / G;
  const int t0 = s * per + ci * chunk;
  const int t1 = min(t0 + chunk, (s + 1) * per);
  for (int e = threadIdx.x; e < E; e += blockDim.x) bins[e] = 0;
  __syncthreads();
  const int np = max(0, t1 - t0) * k;
  for (int q = threadIdx.x; q < np; q += blockDim.x) {
    const int e = idx[(size_t)t0 * k + q];
    if (e >= 0 && e < E) atomicAdd(&bins[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_counts[(size_t)c * E + e] = bins[e];
}

// Expert e's remote pool (R pairs, in pair-id order) over its hosts in
// ascending rank: host i serves places [host_lo, host_hi) -- host_count[e,h]
// pairs each (negative read as 0), the highest host also the rest; the sizes
// of the remote groups follow.  One wave, lane h for rank h (G <= 64): the
// host's place is a wave prefix sum of the hosts' shares, capped at R + 1
// (capped sums of non-negative shares stay associative).
__device__ void remote_ranges_wave(int e, uint64_t mask, int R, const int32_t* __restrict__ host_count, int E,
                                   int G, PermuteWs ws) {
  const int h = threadIdx.x & (MOELB_WAVE - 1);
  const bool host = h < G && ((mask >> h) & 1ull);
  const int hc = host ? max(host_count[(size_t)e * G + h], 0) : 0;
  const long long cap = (long long)R + 1;
  long long incl = min((long long)hc, cap);
#pragma unroll
  for (int o = 1; o < MOELB_WAVE; o <<= 1) {
    const long long v = __shfl_up(incl, o, MOELB_WAVE);
    if (h >= o) incl = min(incl + v, cap);
  }
  const long long up = __shfl_up(incl, 1, MOELB_WAVE);
  const int excl = h == 0 ? 0 : (int)min(up, (long long)R);
  const int m = __popcll(mask);
  const int i = __popcll(mask & lanemask_lt());  // this host's index among e's hosts
  const int hi_all = i == m - 1 ? R : (int)min(incl, (long long)R);  // the highest host takes the rest
  if (host) {
    const int lo = excl;
    const int hi = hi_all;
    ws.host_rank[(size_t)e * G + i] = h;
    ws.host_lo[(size_t)e * G + i] = lo;
    ws.host_hi[(size_t)e * G + i] = hi;
  }
  if (h < G) {
    ws.gsize[(size_t)(1 * G + h) * E + e] = host ? hi_all - excl : 0;
    if (h >= m) ws.host_rank[(size_t)e * G + h] = -1;
  }
}

// One workgroup per expert: a block scan over the chunks (token order) of the
// pair (local count, remote count).  A chunk's local base is its exclusive
// local prefix minus that of its rank's first chunk; its remote base is the
// exclusive remote prefix (rho of its first remote pair).
constexpr int ESCAN_THREADS = 256;

__global__ __launch_bounds__(ESCAN_THREADS) void expert_scan_kernel(const int32_t* __restrict__ home,
                                                                    const int32_t* __restrict__ replica,
                                                                    const int32_t* __restrict__ host_count, int E,
                                                                    int G, int N, int nchr, PermuteWs ws) {
  __shared__ int part_l[ESCAN_THREADS], part_r[ESCAN_THREADS];
  __shared__ int rank_first[MOELB_MAX_G];
  __shared__ uint64_t s_mask;
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid == 0) {
    int h = home[e];
    h = (h >= 0 && h < G) ? h : 0;
    s_mask = 1ull << h;
  }
  __syncthreads();
  for (int q = tid; q < G * N; q += ESCAN_THREADS)
    if (replica[q] == e) atomicOr(reinterpret_cast<unsigned long long*>(&s_mask), 1ull << (q / N));
  __syncthreads();
  const uint64_t mask = s_mask;
  const int nch = G * nchr;
  const int seg = (nch + ESCAN_THREADS - 1) / ESCAN_THREADS;
  const int c0 = min(tid * seg, nch), c1 = min(c0 + seg, nch);
  int sl = 0, sr = 0;
  for (int c = c0; c < c1; ++c) {
    const int cnt = ws.chunk_counts[(size_t)c * E + e];
    if ((mask >> (c / nchr)) & 1ull) sl += cnt; else sr += cnt;
  }
  part_l[tid] = sl;
  part_r[tid] = sr;
  __syncthreads();
  for (int o = 1; o < ESCAN_THREADS; o <<= 1) {
    const int vl = tid >= o ? part_l[tid - o] : 0;
    const int vr = tid >= o ? part_r[tid - o] : 0;
    __syncthreads();
    part_l[tid] += vl;
    part_r[tid] += vr;
    __syncthreads();
  }
  int rl = part_l[tid] - sl, rr = part_r[tid] - sr;  // exclusive prefixes at c0
  for (int c = c0; c < c1; ++c) {
    const int cnt = ws.chunk_counts[(size_t)c * E + e];
    if ((mask >> (c / nchr)) & 1ull) {
      ws.chunk_base[(size_t)c * E + e] = rl;  // rank offset subtracted below
      if (c % nchr == 0) rank_first[c / nchr] = rl;
      rl += cnt;
    } else {
      ws.chunk_base[(size_t)c * E + e] = rr;
      rr += cnt;
    }
  }
  __syncthreads();
  for (int c = tid; c < nch; c += ESCAN_THREADS) {
    const int s = c / nchr;
    if ((mask >> s) & 1ull) ws.chunk_base[(size_t)c * E + e] -= rank_first[s];
  }
  const int total_l = part_l[ESCAN_THREADS - 1];
  const int R = part_r[ESCAN_THREADS - 1];
  if (tid < G) {
    const int s = tid;
    int size = 0;
    if ((mask >> s) & 1ull) {
      // local prefix where the next host rank starts (or the total)
      int nx = total_l;
      for (int s2 = s + 1; s2 < G; ++s2)
        if ((mask >> s2) & 1ull) {
          nx = rank_first[s2];
          break;
        }
      size = nx - rank_first[s];
    }
    ws.gsize[(size_t)(0 * G + s) * E + e] = size;
  }
  if (tid == 0) ws.remote_total[e] = R;
  if (host_count && tid < MOELB_WAVE) remote_ranges_wave(e, mask, R, host_count, E, G, ws);
}

// Remote phase: host ranges of every expert (one wave per expert).
__global__ __launch_bounds__(256) void remote_ranges_kernel(const int32_t* __restrict__ home,
                                                            const int32_t* __restrict__ replica,
                                                            const int32_t* __restrict__ host_count, int E, int G,
                                                            int N, PermuteWs ws) {
  __shared__ uint64_t hmask[MOELB_MAX_E];
  block_host_masks(home, replica, G, N, E, hmask);
  const int e = blockIdx.x * (blockDim.x / MOELB_WAVE) + threadIdx.x / MOELB_WAVE;
  if (e >= E) return;
  remote_ranges_wave(e, hmask[e], ws.remote_total[e], host_count, E, G, ws);
}

// Exclusive scan of the 2GE group sizes into group_off (one workgroup).
// With `base`, offsets start at *base (the remote groups after the local
// total, which is group_off[G*E] itself: every thread reads the same value
// that the first write stores back).
__global__ __launch_bounds__(SCAN_THREADS) void group_scan_kernel(const int32_t* __restrict__ gsize, int ngroups,
                                                                  const int32_t* base, int32_t* group_off) {
  __shared__ int part[SCAN_THREADS];
  const int tid = threadIdx.x;
  const int seg = (ngroups + SCAN_THREADS - 1) / SCAN_THREADS;
  const int b0 = min(tid * seg, ngroups), b1 = min(b0 + seg, ngroups);
  int sum = 0;
  for (int g = b0; g < b1; ++g) sum += gsize[g];
  part[tid] = sum;
  __syncthreads();
  for (int o = 1; o < SCAN_THREADS; o <<= 1) {
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  const int b = base ? *base : 0;
  int run = b + part[tid] - sum;
  for (int g = b0; g < b1; ++g) {
    group_off[g] = run;
    run += gsize[g];
  }
  if (tid == SCAN_THREADS - 1) group_off[ngroups] = b + part[tid];
}

constexpr int RS_STAGE_EG = 4096;  // 48 KiB of LDS host ranges

// LOCAL_ONLY (local phase of the two-phase form): remote pairs get pos -1 and
// their place rho in ws.rho (every other pair -1 there); no perm entry or row
// copy for them yet.
template <typename T, bool LOCAL_ONLY>
__global__ __launch_bounds__(256) void rank_scatter_kernel(const T* __restrict__ h, const int32_t* __restrict__ idx,
                                                           int Ttok, int d, int k, int E, int G, int N, int chunk,
                                                           int nchr,
                                                           const int32_t* __restrict__ home,
                                                           const int32_t* __restrict__ replica, PermuteWs ws,
                                                           const int32_t* __restrict__ group_off,
                                                           int32_t* __restrict__ perm, int32_t* __restrict__ pos,
                                                           T* __restrict__ x_perm) {
  __shared__ int cnt[MOELB_MAX_E];
  __shared__ uint64_t hmask[MOELB_MAX_E];
  __shared__ int qpos[MAX_CHUNK * MOELB_MAX_K];
  // host ranges of every expert in LDS when they fit (E*G <= RS_STAGE_EG):
  // a remote pair's host search then reads LDS, not a chain of global loads
  extern __shared__ int hr_lds[];  // [3][E*G]: host rank, first place, end place
  const bool staged = !LOCAL_ONLY && E * G <= RS_STAGE_EG;
  const int32_t* h_rank = staged ? hr_lds : ws.host_rank;
  const int32_t* h_lo = staged ? hr_lds + E * G : ws.host_lo;
  const int32_t* h_hi = staged ? hr_lds + 2 * E * G : ws.host_hi;
  if (staged)
    for (int i = threadIdx.x; i < E * G; i += blockDim.x) {
      hr_lds[i] = ws.host_rank[i];
      hr_lds[E * G + i] = ws.host_lo[i];
      hr_lds[2 * E * G + i] = ws.host_hi[i];
    }
  const int c = blockIdx.x;
  const int s = c / nchr, ci = c % nchr;
  const int per = Ttok / G;
  const int t0 = s * per + ci * chunk;
  const int t1 = min(t0 + chunk, (s + 1) * per);
  const int ntok = max(0, t1 - t0);
  const int np = ntok * k;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  block_host_masks(home, replica, G, N, E, hmask);
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const uint64_t below = lanemask_lt();
    for (int p0 = 0; p0 < np; p0 += 64) {
      const int pl = p0 + lane;
      const bool inr = pl < np;
      const size_t pid = (size_t)t0 * k + pl;
      const int e = inr ? idx[pid] : -1;
      const bool valid = inr && e >= 0 && e < E;
      int rank = 0;
      uint64_t remaining = __ballot(valid);
      while (remaining) {
        const int leader = __builtin_ctzll(remaining);
        const int el = __builtin_amdgcn_readlane(e, leader);
        const uint64_t m = __ballot(valid && e == el);
        const int base = cnt[el];
        if (valid && e == el) rank = base + __popcll(m & below);
        if (lane == leader) cnt[el] = base + __popcll(m);
        remaining &= ~m;
      }
      int q = -1;
      int rho = -1;
      if (valid) {
        rank += ws.chunk_base[(size_t)c * E + e];
        const uint64_t mask = hmask[e];
        int key = -1;
        if ((mask >> s) & 1ull) {
          key = (0 * G + s) * E + e;
        } else if (LOCAL_ONLY) {
          rho = rank;
        } else {
          // rank is rho, this pair's place in e's remote pool
          int i = 0;
          while (i + 1 < G && h_rank[e * G + i + 1] >= 0 && rank >= h_hi[e * G + i]) ++i;
          const int hst = h_rank[e * G + i];
          rank -= h_lo[e * G + i];
          key = (1 * G + hst) * E + e;
        }
        if (key >= 0) {
          q = group_off[key] + rank;
          perm[q] = static_cast<int32_t>(pid);
        }
      }
      if (inr) {
        pos[pid] = q;
        qpos[pl] = q;
        if (LOCAL_ONLY) ws.rho[pid] = rho;
      }
    }
  }
  __syncthreads();
  if (x_perm == nullptr) return;
  // copy each token's row to its k destinations in 16-byte chunks: each
  // thread loads U chunks before it stores any (U loads in flight), and the
  // stores are non-temporal -- x_perm is written once and not read here, and
  // keeping it out of the caches raised the copy from 4.4 to 4.9 TB/s
  const int nvec = d * (int)sizeof(T) / 16;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  constexpr int U = 8;
  const int items = ntok * nvec;
  for (int i0 = threadIdx.x; i0 < items; i0 += U * 256) {
    u32x4 val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * 256;
      if (i < items) {
        const int tl = i / nvec;
        val[u] = reinterpret_cast<const u32x4*>(h + (size_t)(t0 + tl) * d)[i - tl * nvec];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * 256;
      if (i < items) {
        const int tl = i / nvec, v = i - tl * nvec;
        for (int j = 0; j < k; ++j) {
          const int q = qpos[tl * k + j];
          if (q >= 0) __builtin_nontemporal_store(val[u], reinterpret_cast<u32x4*>(x_perm + (size_t)q * d) + v);
        }
      }
    }
  }
}

// Remote phase: one thread per pair places the remote pairs (rho >= 0) with
// the host ranges; then the workgroup copies their rows (16-byte chunks).
constexpr int RS_THREADS = 256;

template <typename T>
__global__ __launch_bounds__(RS_THREADS) void remote_scatter_kernel(const T* __restrict__ h,
                                                                    const int32_t* __restrict__ idx, int P, int d,
                                                                    int k, int E, int G, PermuteWs ws,
                                                                    const int32_t* __restrict__ group_off,
                                                                    int32_t* __restrict__ perm,
                                                                    int32_t* __restrict__ pos, T* __restrict__ x_perm) {
  __shared__ int qs[RS_THREADS];
  __shared__ int any;
  const int pid = blockIdx.x * RS_THREADS + threadIdx.x;
  if (threadIdx.x == 0) any = 0;
  __syncthreads();
  int q = -1;
  const int rho = pid < P ? ws.rho[pid] : -1;
  if (rho >= 0) {
    const int e = idx[pid];  // valid: the local phase kept rho only for valid pairs
    int i = 0;
    while (i + 1 < G && ws.host_rank[(size_t)e * G + i + 1] >= 0 && rho >= ws.host_hi[(size_t)e * G + i]) ++i;
    const int hst = ws.host_rank[(size_t)e * G + i];
    q = group_off[(1 * G + hst) * E + e] + rho - ws.host_lo[(size_t)e * G + i];
    perm[q] = pid;
    pos[pid] = q;
    any = 1;
  }
  qs[threadIdx.x] = q;
  __syncthreads();
  if (x_perm == nullptr || !any) return;
  const int nvec = d * (int)sizeof(T) / 16;
  for (int i = 0; i < RS_THREADS; ++i) {
    const int qi = qs[i];
    if (qi < 0) continue;
    const int p = blockIdx.x * RS_THREADS + i;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4* src = reinterpret_cast<const u32x4*>(h + (size_t)(p / k) * d);
    u32x4* dst = reinterpret_cast<u32x4*>(x_perm + (size_t)qi * d);
    for (int v = threadIdx.x; v < nvec; v += RS_THREADS) __builtin_nontemporal_store(src[v], dst + v);
  }
}

// ---------------------------------------------------------------- one-workgroup form
//
// Small batches (decode) spend the four-launch sort on launch latency.  Up to
// OW_MAX_PAIRS pairs with E*G <= OW_MAX_EG, and no rows to copy, the same
// result comes from one workgroup, everything but the inputs and outputs in
// LDS:
//   1. each wave takes segments of pairs (a rank's tokens cut into J pieces,
//      so there are at least as many segments as waves) and ranks every pair
//      among the pairs of its expert in its segment: the lanes holding expert
//      e OR their bits into a per-wave LDS word for e, read it back, and take
//      ranks from the popcount below the lane; the lowest such lane adds the
//      count to the segment's counter of e and clears the word;
//   2. one thread per expert walks the segments in token order, turning each
//      segment's count into its base (inside the rank's local group when the
//      rank hosts e, inside e's remote pool otherwise), and deals the remote
//      pool over the hosts (host ranges and remote group sizes);
//   3. a block scan of the 2GE group sizes gives group_off;
//   4. the waves walk their segments again and place every pair.
// Pair ranks are stable (pair-id order), so the result is the four-launch
// form's, bit for bit.
constexpr int OW_THREADS = 1024;
constexpr int OW_WAVES = OW_THREADS / MOELB_WAVE;
constexpr int OW_MAX_PAIRS = 8192;  // ranks inside a segment fit 16 bits
constexpr int OW_MAX_EG = 2048;

// Token pieces per rank: enough segments to give every wave one.
__host__ __device__ inline int ow_pieces(int G) { return G >= OW_WAVES ? 1 : (OW_WAVES + G - 1) / G; }

struct OwLds {
  size_t hmask, wmask, segcnt, lrank, goff, hrank, hlo, hhi, part, total;
};

__host__ __device__ inline OwLds ow_lds(int E, int G, int P) {
  const int nseg = G * ow_pieces(G);
  OwLds L;
  size_t off = 0;
  auto take = [&](size_t* field, size_t bytes) {
    *field = off;
    off += (bytes + 15) & ~static_cast<size_t>(15);
  };
  take(&L.hmask, (size_t)E * 8);
  take(&L.wmask, (size_t)OW_WAVES * E * 8);
  take(&L.segcnt, (size_t)nseg * E * 4);
  take(&L.lrank, (size_t)P * 2);
  take(&L.goff, ((size_t)2 * G * E + 1) * 4);
  take(&L.hrank, (size_t)E * G * 4);
  take(&L.hlo, (size_t)E * G * 4);
  take(&L.hhi, (size_t)E * G * 4);
  take(&L.part, (size_t)(OW_WAVES + 1) * 4);
  L.total = off;
  return L;
}

__global__ __launch_bounds__(OW_THREADS) void permute_one_wg_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int G, int N, const int32_t* __restrict__ home,
    const int32_t* __restrict__ replica, const int32_t* __restrict__ host_count, int32_t* __restrict__ group_off,
    int32_t* __restrict__ perm, int32_t* __restrict__ pos) {
  extern __shared__ __align__(16) char ow_smem[];
  const int per = T / G;
  const int J = ow_pieces(G);
  const int nseg = G * J;
  const OwLds L = ow_lds(E, G, T * k);
  uint64_t* hmask = reinterpret_cast<uint64_t*>(ow_smem + L.hmask);
  int* segcnt = reinterpret_cast<int*>(ow_smem + L.segcnt);
  uint16_t* lrank = reinterpret_cast<uint16_t*>(ow_smem + L.lrank);
  int* goff = reinterpret_cast<int*>(ow_smem + L.goff);
  int* hrank = reinterpret_cast<int*>(ow_smem + L.hrank);
  int* hlo = reinterpret_cast<int*>(ow_smem + L.hlo);
  int* hhi = reinterpret_cast<int*>(ow_smem + L.hhi);
  int* part = reinterpret_cast<int*>(ow_smem + L.part);
  const int tid = threadIdx.x, lane = tid & (MOELB_WAVE - 1), w = tid / MOELB_WAVE;
  uint64_t* wm = reinterpret_cast<uint64_t*>(ow_smem + L.wmask) + (size_t)w * E;
  for (int i = tid; i < nseg * E; i += OW_THREADS) segcnt[i] = 0;
  for (int i = lane; i < E; i += MOELB_WAVE) wm[i] = 0ull;
  block_host_masks(home, replica, G, N, E, hmask);  // its barriers also cover the clearing above

  // 1. ranks inside (segment, expert); one wave's LDS traffic is in order, so
  //    the OR, the reads and the leader's update need no barrier
  const uint64_t below = lanemask_lt();
  for (int seg = w; seg < nseg; seg += OW_WAVES) {
    const int s = seg / J, j = seg % J;
    const int p1 = (s * per + ((j + 1) * per) / J) * k;
    int* cnt = segcnt + (size_t)seg * E;
    for (int pb = (s * per + (j * per) / J) * k; pb < p1; pb += MOELB_WAVE) {
      const int p = pb + lane;
      const int e = p < p1 ? idx[p] : -1;
      const bool valid = e >= 0 && e < E;
      if (valid) atomicOr(reinterpret_cast<unsigned long long*>(&wm[e]), 1ull << lane);
      __builtin_amdgcn_wave_barrier();
      const uint64_t m = valid ? wm[e] : 0ull;
      const int base = valid ? cnt[e] : 0;
      __builtin_amdgcn_wave_barrier();
      if (valid && (m & below) == 0ull) {
        cnt[e] = base + __popcll(m);
        wm[e] = 0ull;
      }
      __builtin_amdgcn_wave_barrier();
      if (valid) lrank[p] = static_cast<uint16_t>(base + __popcll(m & below));
    }
  }
  __syncthreads();

  // 2. segment bases, local group sizes, host ranges and remote group sizes
  if (tid < E) {
    const int e = tid;
    const uint64_t mask = hmask[e];
    int loc = 0, rem = 0;
    for (int seg = 0; seg < nseg; ++seg) {
      const int s = seg / J;
      const int c = segcnt[seg * E + e];
      if ((mask >> s) & 1ull) {
        if (seg % J == 0) loc = 0;
        segcnt[seg * E + e] = loc;
        loc += c;
      } else {
        segcnt[seg * E + e] = rem;
        rem += c;
      }
      if (seg % J == J - 1) goff[s * E + e] = ((mask >> s) & 1ull) ? loc : 0;
    }
    // remote pool [0, rem) over the hosts in ascending rank: host_count[e,h]
    // places each (negative read as 0), capped at the pool, the highest host
    // also the rest
    const int m = __popcll(mask);
    int i = 0, run = 0;
    for (int hst = 0; hst < G; ++hst) {
      int size = 0;
      if ((mask >> hst) & 1ull) {
        const long long hc = max(host_count[(size_t)e * G + hst], 0);
        const int hi = i == m - 1 ? rem : (int)min((long long)run + hc, (long long)rem);
        hrank[e * G + i] = hst;
        hlo[e * G + i] = run;
        hhi[e * G + i] = hi;
        size = hi - run;
        run = hi;
        ++i;
      }
      goff[(G + hst) * E + e] = size;
    }
    for (; i < G; ++i) hrank[e * G + i] = -1;
  }
  __syncthreads();

  // 3. group sizes -> exclusive offsets (each thread a contiguous run)
  const int ng = 2 * G * E;
  const int run_len = (ng + OW_THREADS - 1) / OW_THREADS;
  const int g0 = min(tid * run_len, ng), g1 = min(g0 + run_len, ng);
  int sum = 0;
  for (int g = g0; g < g1; ++g) sum += goff[g];
  int incl = sum;
#pragma unroll
  for (int o = 1; o < MOELB_WAVE; o <<= 1) {
    const int v = __shfl_up(incl, o, MOELB_WAVE);
    if (lane >= o) incl += v;
  }
  if (lane == MOELB_WAVE - 1) part[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int v = lane < OW_WAVES ? part[lane] : 0;
    int wi = v;
#pragma unroll
    for (int o = 1; o < OW_WAVES; o <<= 1) {
      const int u = __shfl_up(wi, o, MOELB_WAVE);
      if (lane >= o) wi += u;
    }
    if (lane < OW_WAVES) part[lane] = wi - v;
    if (lane == OW_WAVES - 1) part[OW_WAVES] = wi;
  }
  __syncthreads();
  int acc = part[w] + incl - sum;
  for (int g = g0; g < g1; ++g) {
    const int size = goff[g];
    goff[g] = acc;
    acc += size;
  }
  if (tid == 0) goff[ng] = part[OW_WAVES];
  __syncthreads();
  for (int g = tid; g <= ng; g += OW_THREADS) group_off[g] = goff[g];

  // 4. place every pair
  for (int seg = w; seg < nseg; seg += OW_WAVES) {
    const int s = seg / J, j = seg % J;
    const int p1 = (s * per + ((j + 1) * per) / J) * k;
    const int* base = segcnt + (size_t)seg * E;
    for (int p = (s * per + (j * per) / J) * k + lane; p < p1; p += MOELB_WAVE) {
      const int e = idx[p];
      int q = -1;
      if (e >= 0 && e < E) {
        const int r = base[e] + lrank[p];
        if ((hmask[e] >> s) & 1ull) {
          q = goff[s * E + e] + r;
        } else {
          // r is rho, the pair's place in e's remote pool
          int i = 0;
          while (i + 1 < G && hrank[e * G + i + 1] >= 0 && r >= hhi[e * G + i]) ++i;
          q = goff[(G + hrank[e * G + i]) * E + e] + r - hlo[e * G + i];
        }
        perm[q] = p;
      }
      pos[p] = q;
    }
  }
}

}  // namespace

extern "C" size_t moelb_permute_workspace_bytes(int T, int k, int E, int G) {
  if (G < 1 || E < 1 || T < 0) return 0;
  return ws_layout(T, k, E, G, nullptr, nullptr);
}

// Arguments other than the workspace.
static int permute_args(const void* h, const int32_t* idx, int T, int d, int k, int E, int G, int N, int dtype,
                        const int32_t* home, const int32_t* replica, const int32_t* group_off, const int32_t* perm,
                        const int32_t* pos, const void* x_perm) {
  if (T < 0 || d <= 0 || d % 8 != 0 || k < 1 || k > MOELB_MAX_K || E < 1 || E > MOELB_MAX_E || G < 1 ||
      G > MOELB_MAX_G || N < 0 || N > MOELB_MAX_N || T % G != 0 || !moelb_dtype_ok(dtype))
    return MOELB_EINVAL;
  if (!home || (N > 0 && !replica) || !group_off || (T > 0 && (!idx || !perm || !pos))) return MOELB_EINVAL;
  if (x_perm && !h) return MOELB_EINVAL;
  if ((reinterpret_cast<uintptr_t>(h) | reinterpret_cast<uintptr_t>(x_perm)) & 15) return MOELB_EINVAL;
  if ((size_t)T * k > 0x7fffffffull) return MOELB_EINVAL;
  return MOELB_OK;
}

static int permute_check(const void* h, const int32_t* idx, int T, int d, int k, int E, int G, int N, int dtype,
                         const int32_t* home, const int32_t* replica, void* ws, size_t ws_bytes,
                         const int32_t* group_off, const int32_t* perm, const int32_t* pos, const void* x_perm) {
  const int st = permute_args(h, idx, T, d, k, E, G, N, dtype, home, replica, group_off, perm, pos, x_perm);
  if (st != MOELB_OK) return st;
  const size_t need = ws_layout(T, k, E, G, nullptr, nullptr);
  if (!ws || ws_bytes < need) return MOELB_EWORKSPACE;
  return MOELB_OK;
}

// count, expert scan, group scan (all groups, or the local ones), rank+scatter
static int permute_launch(bool local_only, const void* h, const int32_t* idx, int T, int d, int k, int E, int G,
                          int N, int dtype, const int32_t* home, const int32_t* replica,
                          const int32_t* host_count, void* ws, int32_t* group_off, int32_t* perm, int32_t* pos,
                          void* x_perm, hipStream_t s) {
  PermuteWs w;
  ws_layout(T, k, E, G, &w, static_cast<char*>(ws));
  const int per = T / G;
  const int chunk = chunk_tokens(T, G);
  const int nchr = per > 0 ? (per + chunk - 1) / chunk : 1;
  const int nchunks = G * nchr;
  const int32_t* rep = N > 0 ? replica : home;
  if (!local_only && !x_perm && (long long)T * k <= OW_MAX_PAIRS && E * G <= OW_MAX_EG) {
    const size_t lds = ow_lds(E, G, T * k).total;
    if (!moelb_allow_lds(permute_one_wg_kernel, lds)) return MOELB_ELAUNCH;
    hipLaunchKernelGGL(permute_one_wg_kernel, dim3(1), dim3(OW_THREADS), lds, s, idx, T, k, E, G, N, home, rep,
                       host_count, group_off, perm, pos);
    MOELB_CHECK_LAUNCH();
    return MOELB_OK;
  }
  hipLaunchKernelGGL(count_kernel, dim3(nchunks), dim3(256), 0, s, idx, T, k, E, G, chunk, nchr, w.chunk_counts);
  MOELB_CHECK_LAUNCH();
  hipLaunchKernelGGL(expert_scan_kernel, dim3(E), dim3(ESCAN_THREADS), 0, s, home, rep,
                     local_only ? nullptr : host_count, E, G, N, nchr, w);
  MOELB_CHECK_LAUNCH();
  hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(SCAN_THREADS), 0, s, w.gsize, (local_only ? 1 : 2) * G * E,
                     nullptr, group_off);
  MOELB_CHECK_LAUNCH();
  const size_t rs_lds = (!local_only && E * G <= RS_STAGE_EG) ? (size_t)3 * E * G * sizeof(int) : 0;
#define PERMUTE_SCATTER(TY, LO)                                                                                  \
  hipLaunchKernelGGL((rank_scatter_kernel<TY, LO>), dim3(nchunks), dim3(256), rs_lds, s, static_cast<const TY*>(h), \
                     idx, T, d, k, E, G, N, chunk, nchr, home, rep, w, group_off, perm, pos, static_cast<TY*>(x_perm))
  if (dtype == MOELB_BF16) {
    if (local_only) PERMUTE_SCATTER(uint16_t, true); else PERMUTE_SCATTER(uint16_t, false);
  } else {
    if (local_only) PERMUTE_SCATTER(float, true); else PERMUTE_SCATTER(float, false);
  }
#undef PERMUTE_SCATTER
  MOELB_CHECK_LAUNCH();
  return MOELB_OK;
}

extern "C" int moelb_permute(const void* h, const int32_t* idx, int T, int d, int k, int E, int G, int N, int dtype,
                             const int32_t* home, const int32_t* replica, const int32_t* host_count, void* ws,
                             size_t ws_bytes, int32_t* group_off, int32_t* perm, int32_t* pos, void* x_perm,
                             void* stream) {
  const int st = permute_check(h, idx, T, d, k, E, G, N, dtype, home, replica, ws, ws_bytes, group_off, perm, pos,
                               x_perm);
  if (st != MOELB_OK) return st;
  if (!host_count) return MOELB_EINVAL;
  return permute_launch(false, h, idx, T, d, k, E, G, N, dtype, home, replica, host_count, ws, group_off, perm, pos,
                        x_perm, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- no-allocation form

// Workspace of moelb_permute_noalloc: a fixed array in device memory (one per
// device the library runs on, held until the process ends).  Its host-side
// name is not a device address: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[MOELB_PERMUTE_NOALLOC_WS_BYTES];

// Device address of `scratch` on the current device, looked up once per device
// (the first call made with that device current) and remembered; NULL if the
// lookup fails.
static void* scratch_address() {
  static std::mutex mu;
  static std::vector<std::pair<int, void*>> known;  // (device, address)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& x : known)
    if (x.first == dev) return x.second;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
  known.emplace_back(dev, p);
  return p;
}

extern "C" int moelb_permute_noalloc(const void* h, const int32_t* idx, int T, int d, int k, int E, int G, int N,
                                     int dtype, const int32_t* home, const int32_t* replica,
                                     const int32_t* host_count, int32_t* group_off, int32_t* perm, int32_t* pos,
                                     void* x_perm, void* stream) {
  // arguments, then the workspace size, both before any device call
  const int st = permute_args(h, idx, T, d, k, E, G, N, dtype, home, replica, group_off, perm, pos, x_perm);
  if (st != MOELB_OK) return st;
  if (!host_count) return MOELB_EINVAL;
  if (ws_layout(T, k, E, G, nullptr, nullptr) > MOELB_PERMUTE_NOALLOC_WS_BYTES) return MOELB_EWORKSPACE;
  void* ws = scratch_address();
  if (!ws) return MOELB_ELAUNCH;
  return permute_launch(false, h, idx, T, d, k, E, G, N, dtype, home, replica, host_count, ws, group_off, perm, pos,
                        x_perm, static_cast<hipStream_t>(stream));
}

extern "C" int moelb_permute_local(const void* h, const int32_t* idx, int T, int d, int k, int E, int G, int N,
                                   int dtype, const int32_t* home, const int32_t* replica, void* ws,
                                   size_t ws_bytes, int32_t* group_off, int32_t* perm, int32_t* pos, void* x_perm,
                                   void* stream) {
  const int st = permute_check(h, idx, T, d, k, E, G, N, dtype, home, replica, ws, ws_bytes, group_off, perm, pos,
                               x_perm);
  if (st != MOELB_OK) return st;
  return permute_launch(true, h, idx, T, d, k, E, G, N, dtype, home, replica, nullptr, ws, group_off, perm, pos,
                        x_perm, static_cast<hipStream_t>(stream));
}

extern "C" int moelb_permute_remote(const void* h, const int32_t* idx, int T, int d, int k, int E, int G, int N,
                                    int dtype, const int32_t* home, const int32_t* replica,
                                    const int32_t* host_count, void* ws, size_t ws_bytes, int32_t* group_off,
                                    int32_t* perm, int32_t* pos, void* x_perm, void* stream) {
  const int st = permute_check(h, idx, T, d, k, E, G, N, dtype, home, replica, ws, ws_bytes, group_off, perm, pos,
                               x_perm);
  if (st != MOELB_OK) return st;
  if (!host_count) return MOELB_EINVAL;
  PermuteWs w;
  ws_layout(T, k, E, G, &w, static_cast<char*>(ws));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t* rep = N > 0 ? replica : home;
  hipLaunchKernelGGL(remote_ranges_kernel, dim3((E + 3) / 4), dim3(256), 0, s, home, rep, host_count, E, G, N, w);
  MOELB_CHECK_LAUNCH();
  hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(SCAN_THREADS), 0, s, w.gsize + (size_t)G * E, G * E,
                     group_off + (size_t)G * E, group_off + (size_t)G * E);
  MOELB_CHECK_LAUNCH();
  const int P = T * k;
  if (P == 0) return MOELB_OK;
  const int nb = (P + RS_THREADS - 1) / RS_THREADS;
  if (dtype == MOELB_BF16)
    hipLaunchKernelGGL(remote_scatter_kernel<uint16_t>, dim3(nb), dim3(RS_THREADS), 0, s,
                       static_cast<const uint16_t*>(h), idx, P, d, k, E, G, w, group_off, perm, pos,
                       static_cast<uint16_t*>(x_perm));
  else
    hipLaunchKernelGGL(remote_scatter_kernel<float>, dim3(nb), dim3(RS_THREADS), 0, s, static_cast<const float*>(h),
                       idx, P, d, k, E, G, w, group_off, perm, pos, static_cast<float*>(x_perm));
  MOELB_CHECK_LAUNCH();
  return MOELB_OK;
}
