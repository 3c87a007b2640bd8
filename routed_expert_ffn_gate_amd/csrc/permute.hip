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

__device__ __forceinline__ uint64_t host_mask(const int32_t* home, const int32_t* replica, int G, int N, int e) {
  int h = home[e];
  h = (h >= 0 && h < G) ? h : 0;
  uint64_t m = 1ull << h;
  for (int r = 0; r < G; ++r)
    for (int j = 0; j < N; ++j)
      if (replica[r * N + j] == e) m |= 1ull << r;
  return m;
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
// of the remote groups follow.
__device__ void remote_ranges(int e, uint64_t mask, int R, const int32_t* __restrict__ host_count, int E, int G,
                              PermuteWs ws) {
  const int m = __popcll(mask);
  int cum = 0, i = 0;
  for (int h = 0; h < G; ++h) {
    int size = 0;
    if ((mask >> h) & 1ull) {
      const int hc = max(host_count[(size_t)e * G + h], 0);
      const int lo = min(cum, R);
      cum = (cum > R - hc) ? R + 1 : cum + hc;  // saturating: stays > R once past it
      int hi = min(cum, R);
      if (i == m - 1) hi = R;                    // the highest host takes the rest
      size = hi - lo;
      ws.host_rank[(size_t)e * G + i] = h;
      ws.host_lo[(size_t)e * G + i] = lo;
      ws.host_hi[(size_t)e * G + i] = hi;
      ++i;
    }
    ws.gsize[(size_t)(1 * G + h) * E + e] = size;
  }
  for (; i < G; ++i) ws.host_rank[(size_t)e * G + i] = -1;
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
  if (tid == 0) s_mask = host_mask(home, replica, G, N, e);
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
  if (tid == 0) {
    ws.remote_total[e] = R;
    if (host_count) remote_ranges(e, mask, R, host_count, E, G, ws);
  }
}

// Remote phase: host ranges of every expert (thread e).
__global__ __launch_bounds__(256) void remote_ranges_kernel(const int32_t* __restrict__ home,
                                                            const int32_t* __restrict__ replica,
                                                            const int32_t* __restrict__ host_count, int E, int G,
                                                            int N, PermuteWs ws) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  remote_ranges(e, host_mask(home, replica, G, N, e), ws.remote_total[e], host_count, E, G, ws);
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
  const int c = blockIdx.x;
  const int s = c / nchr, ci = c % nchr;
  const int per = Ttok / G;
  const int t0 = s * per + ci * chunk;
  const int t1 = min(t0 + chunk, (s + 1) * per);
  const int ntok = max(0, t1 - t0);
  const int np = ntok * k;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    cnt[e] = 0;
    hmask[e] = host_mask(home, replica, G, N, e);
  }
  __syncthreads();
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
          while (i + 1 < G && ws.host_rank[(size_t)e * G + i + 1] >= 0 && rank >= ws.host_hi[(size_t)e * G + i]) ++i;
          const int hst = ws.host_rank[(size_t)e * G + i];
          rank -= ws.host_lo[(size_t)e * G + i];
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
  // copy each token's row to its k destinations: 16-byte chunks
  const int nvec = d * (int)sizeof(T) / 16;
  for (int tl = 0; tl < ntok; ++tl) {
    const uint4* src = reinterpret_cast<const uint4*>(h + (size_t)(t0 + tl) * d);
    for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
      const uint4 val = src[v];
      for (int j = 0; j < k; ++j) {
        const int q = qpos[tl * k + j];
        if (q >= 0) reinterpret_cast<uint4*>(x_perm + (size_t)q * d)[v] = val;
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
    const uint4* src = reinterpret_cast<const uint4*>(h + (size_t)(p / k) * d);
    uint4* dst = reinterpret_cast<uint4*>(x_perm + (size_t)qi * d);
    for (int v = threadIdx.x; v < nvec; v += RS_THREADS) dst[v] = src[v];
  }
}

}  // namespace

extern "C" size_t moelb_permute_workspace_bytes(int T, int k, int E, int G) {
  if (G < 1 || E < 1 || T < 0) return 0;
  return ws_layout(T, k, E, G, nullptr, nullptr);
}

static int permute_check(const void* h, const int32_t* idx, int T, int d, int k, int E, int G, int N, int dtype,
                         const int32_t* home, const int32_t* replica, void* ws, size_t ws_bytes,
                         const int32_t* group_off, const int32_t* perm, const int32_t* pos, const void* x_perm) {
  if (T < 0 || d <= 0 || d % 8 != 0 || k < 1 || k > MOELB_MAX_K || E < 1 || E > MOELB_MAX_E || G < 1 ||
      G > MOELB_MAX_G || N < 0 || N > MOELB_MAX_N || T % G != 0 || !moelb_dtype_ok(dtype))
    return MOELB_EINVAL;
  if (!home || (N > 0 && !replica) || !group_off || (T > 0 && (!idx || !perm || !pos))) return MOELB_EINVAL;
  if (x_perm && !h) return MOELB_EINVAL;
  if ((reinterpret_cast<uintptr_t>(h) | reinterpret_cast<uintptr_t>(x_perm)) & 15) return MOELB_EINVAL;
  if ((size_t)T * k > 0x7fffffffull) return MOELB_EINVAL;
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
  hipLaunchKernelGGL(count_kernel, dim3(nchunks), dim3(256), 0, s, idx, T, k, E, G, chunk, nchr, w.chunk_counts);
  MOELB_CHECK_LAUNCH();
  hipLaunchKernelGGL(expert_scan_kernel, dim3(E), dim3(ESCAN_THREADS), 0, s, home, rep,
                     local_only ? nullptr : host_count, E, G, N, nchr, w);
  MOELB_CHECK_LAUNCH();
  hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(SCAN_THREADS), 0, s, w.gsize, (local_only ? 1 : 2) * G * E,
                     nullptr, group_off);
  MOELB_CHECK_LAUNCH();
#define PERMUTE_SCATTER(TY, LO)                                                                                  \
  hipLaunchKernelGGL((rank_scatter_kernel<TY, LO>), dim3(nchunks), dim3(256), 0, s, static_cast<const TY*>(h), \
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
  hipLaunchKernelGGL(remote_ranges_kernel, dim3((E + 255) / 256), dim3(256), 0, s, home, rep, host_count, E, G, N, w);
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
