// Masked grouped SwiGLU expert FFN.
//
// Definition: FreeBalance ("FreeBalance: Pre-Routing Online MoE Load Balancing
// via Residual Workload Prediction") section 2.1 -- each selected expert runs
// on the token and the outputs are combined with the router weights; Libra
// README "Repository Layout" -- a FusedMoE over masked tokens, with replicas
// aliasing their expert's weights.  SwiGLU: a = SiLU(x W_gate^T) * (x W_up^T),
// y = a W2^T.
//
// Design (gfx950):
//  * Schedule kernel: rows of every selected group are renumbered
//    expert-major ("virtual rows"): all groups of expert e (its local and
//    remote groups on every rank) become one contiguous range, tiled by BM
//    rows.  Replica groups of one expert therefore share M tiles, the weights
//    of an expert stream through each M block once, and tail waste is per
//    expert rather than per group.  Tile tables and the virtual->physical row
//    map live in the caller's workspace; nothing is read back to the host.
//  * Gate/up GEMM: M tile of 256 virtual rows gathered through the row map
//    (optionally straight from h through the permutation, so X_perm need not
//    exist), N tile = 128 gate rows + the matching 128 up rows of W13, so the
//    SwiGLU is fused into the epilogue; writes a[v, :] in bf16, virtual-row
//    order (contiguous for the next GEMM).
//  * Down GEMM: a (contiguous) x W2^T, N tile 256, scatters y rows back to
//    their physical (permuted) rows.
//  * Both GEMMs: 256 threads (4 waves, 2 x 2), wave tile 128 x 128 on bf16
//    MFMA 32x32x16 with fp32 accumulators (256 per lane).  With K a multiple
//    of 64, A and B tiles of 256 x 64 stream global -> LDS by direct-to-LDS
//    loads through a ring of five 32 KiB half-stages (ffn_mfma_dma_kernel; the
//    down GEMM as a persistent kernel when K / 64 >= 3); otherwise they are
//    staged through registers into a double-buffered 144 KiB LDS tile
//    (ffn_mfma_kernel).  Tile ids are remapped so each XCD (workgroups go
//    round-robin over the 8 XCDs) works on a contiguous tile range, keeping A
//    blocks and weight slices in its own L2.
//  * fp32 storage uses a SIMT fp32 GEMM with the same schedule.
#include "common.h"

namespace {

constexpr int MF_BM = 256;  // MFMA path M tile
constexpr int MF_BN = 256;  // B rows per tile
constexpr int MF_BK = 64;
constexpr int MF_THREADS = 256;
constexpr int MF_LDS_STRIDE = MF_BK + 8;  // bf16 elements per LDS row
constexpr size_t MF_LDS_BYTES = 2ull * 2 * MF_BM * MF_LDS_STRIDE * sizeof(uint16_t);

constexpr int SF_BM = 64;  // SIMT fp32 path
constexpr int SF_BN = 64;
constexpr int SF_BK = 16;

constexpr int SCHED_MIN_BM = 64;

struct FfnSched {
  int32_t* eoff;      // [E+1]   virtual row offset of each expert
  int32_t* gvb;       // [num_groups] virtual row base of each group (capped at rows)
  int32_t* mt_e;      // [max_mtiles] expert of each M tile
  int32_t* mt_v0;     // [max_mtiles] first virtual row of each M tile
  int32_t* n_mtiles;  // [1]
  int32_t* rowmap;    // [rows] physical row of each virtual row
  int32_t* asrc;      // [rows] row of x the gate/up GEMM reads for each virtual row
  void* amid;         // [rows][inter] SwiGLU activations, virtual row order
  int wpacked;        // W13 and W2 in the packed layout (moelb_pack_weights)
};

inline size_t max_mtiles(int rows, int E) { return (size_t)(rows + SCHED_MIN_BM - 1) / SCHED_MIN_BM + E; }

inline size_t sched_layout(int rows, int num_groups, int E, int inter, int dtype, FfnSched* s, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += moelb_align256(bytes);
    return p;
  };
  const size_t mt = max_mtiles(rows, E);
  char* p_eoff = take((size_t)(E + 1) * 4);
  char* p_gvb = take((size_t)num_groups * 4);
  char* p_mte = take(mt * 4);
  char* p_mtv = take(mt * 4);
  char* p_n = take(4);
  char* p_rm = take((size_t)rows * 4);
  char* p_as = take((size_t)rows * 4);
  char* p_am = take((size_t)rows * inter * moelb_elem_bytes(dtype));
  if (s) {
    s->eoff = reinterpret_cast<int32_t*>(p_eoff);
    s->gvb = reinterpret_cast<int32_t*>(p_gvb);
    s->mt_e = reinterpret_cast<int32_t*>(p_mte);
    s->mt_v0 = reinterpret_cast<int32_t*>(p_mtv);
    s->n_mtiles = reinterpret_cast<int32_t*>(p_n);
    s->rowmap = reinterpret_cast<int32_t*>(p_rm);
    s->asrc = reinterpret_cast<int32_t*>(p_as);
    s->amid = p_am;
  }
  return off;
}

// ---------------------------------------------------------------- schedule

// Expert-major virtual row order: every selected group of expert e gets a
// contiguous range inside e's range [eoff[e], eoff[e+1]); M tiles of BM rows
// never straddle experts.  One workgroup; the group offsets are staged
// through LDS in chunks (two passes: sizes per expert, then each group's
// start), so no thread waits on a chain of global loads.  Group g covers the
// clamped rows [lo, hi), lo = clamp(group_off[g], 0, rows), hi =
// clamp(group_off[g+1], lo, rows); an unselected group counts as empty.  The
// groups of one expert get consecutive ranges in group order, so gvb over
// g = e, e+E, e+2E, ... is non-decreasing and the next group starts where
// the previous one ends (the row map relies on this).
constexpr int SCHED_CHUNK = 4096;

__global__ __launch_bounds__(256) void sched_kernel(const int32_t* __restrict__ group_off, int num_groups, int E, int G,
                                                    int rank, int rows, int BM, FfnSched s) {
  __shared__ int goff[SCHED_CHUNK + 1];
  __shared__ int eoff[MOELB_MAX_E + 1];
  __shared__ int toff[MOELB_MAX_E + 1];
  const int tid = threadIdx.x;
  const int e = tid;
  // walk the groups of expert e, chunk by chunk: add each selected group's
  // size to run, and (write) record every group's start first, capped at rows
  // (64-bit: offsets that overlap can add up past 2^31)
  auto walk = [&](bool write, long long& run) {
    for (int base = 0; base < num_groups; base += SCHED_CHUNK) {
      const int cnt = min(SCHED_CHUNK, num_groups - base);
      __syncthreads();
      for (int i = tid; i <= cnt; i += blockDim.x) goff[i] = group_off[base + i];
      __syncthreads();
      if (e < E) {
        for (int g = base + (e - base % E + E) % E; g < base + cnt; g += E) {
          const bool sel = rank < 0 || ((g / E) % G) == rank;
          const int lo = min(max(goff[g - base], 0), rows);
          const int hi = min(max(goff[g - base + 1], lo), rows);
          if (write) s.gvb[g] = (int)min(run, (long long)rows);
          if (sel) run += hi - lo;
        }
      }
    }
  };
  long long n = 0;
  walk(false, n);
  // expert offsets (clamped to rows) and M-tile offsets: two block scans
  // (Hillis-Steele over the 256 threads, one per expert)
  auto scan = [&](long long v) {  // inclusive prefix of v over threads
    __shared__ long long part[256];
    part[tid] = v;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const long long add = tid >= o ? part[tid - o] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    return part[tid];
  };
  const long long incl = scan(e < E ? n : 0);
  const int lo_row = (int)min(incl - (e < E ? n : 0), (long long)rows);
  const int hi_row = (int)min(incl, (long long)rows);
  const int ntile = e < E ? (hi_row - lo_row + BM - 1) / BM : 0;
  const long long tincl = scan(ntile);
  if (e < E) {
    eoff[e] = lo_row;
    toff[e] = (int)(tincl - ntile);
  }
  if (e == E - 1) {
    eoff[E] = hi_row;
    toff[E] = (int)tincl;
    *s.n_mtiles = (int)tincl;
  }
  __syncthreads();
  long long start = e < E ? eoff[e] : 0;
  walk(true, start);
  if (e < E) {
    s.eoff[e] = eoff[e];
    for (int i = toff[e]; i < toff[e + 1]; ++i) {
      s.mt_e[i] = e;
      s.mt_v0[i] = eoff[e] + (i - toff[e]) * BM;
    }
  }
  if (e == 0) s.eoff[E] = eoff[E];
}

// Inclusive prefix of v over the 256 threads of a workgroup (4 waves):
// shuffles inside each wave, then the totals of the waves below.  part4 holds
// 4 values; every thread of the workgroup must call it.
__device__ __forceinline__ long long block_incl_scan_256(long long v, long long* part4) {
  const int lane = threadIdx.x & (MOELB_WAVE - 1), w = threadIdx.x / MOELB_WAVE;
#pragma unroll
  for (int o = 1; o < MOELB_WAVE; o <<= 1) {
    const long long y = __shfl_up(v, o, MOELB_WAVE);
    if (lane >= o) v += y;
  }
  if (lane == MOELB_WAVE - 1) part4[w] = v;
  __syncthreads();
  long long add = 0;
  for (int i = 0; i < w; ++i) add += part4[i];
  __syncthreads();  // part4 is reused by the next call
  return v + add;
}

// The schedule and the row map in one launch, for up to SCHED_FUSED_GROUPS
// groups: every workgroup stages group_off in LDS and derives the expert
// offsets and the groups' virtual bases itself (the same walk as
// sched_kernel, from LDS), then maps its 256 virtual rows as rowmap_kernel
// does; workgroup 0 also writes the tables the GEMMs read (expert offsets,
// virtual bases, M tiles, one thread per tile).  The second launch and the
// single workgroup's serial tile writes were most of the schedule's time.
constexpr int SCHED_FUSED_GROUPS = 4096;

__global__ __launch_bounds__(256) void sched_rowmap_kernel(const int32_t* __restrict__ group_off, int num_groups,
                                                           int E, int G, int rank, int rows, int BM,
                                                           const int32_t* __restrict__ gather, int gather_k,
                                                           int rows_x, FfnSched s) {
  __shared__ int goff[SCHED_FUSED_GROUPS + 1];
  __shared__ int gvb[SCHED_FUSED_GROUPS];
  __shared__ int eoff[MOELB_MAX_E + 1];
  __shared__ int toff[MOELB_MAX_E + 1];
  __shared__ long long part4[4];
  const int tid = threadIdx.x;
  const int e = tid;
  for (int i = tid; i <= num_groups; i += blockDim.x) goff[i] = group_off[i];
  __syncthreads();
  // rows of expert e's selected groups (clamped as in sched_kernel)
  long long n = 0;
  if (e < E)
    for (int g = e; g < num_groups; g += E) {
      const bool sel = rank < 0 || ((g / E) % G) == rank;
      const int lo = min(max(goff[g], 0), rows);
      const int hi = min(max(goff[g + 1], lo), rows);
      if (sel) n += hi - lo;
    }
  const long long incl = block_incl_scan_256(e < E ? n : 0, part4);
  const int lo_row = (int)min(incl - (e < E ? n : 0), (long long)rows);
  const int hi_row = (int)min(incl, (long long)rows);
  const int ntile = e < E ? (hi_row - lo_row + BM - 1) / BM : 0;
  const long long tincl = block_incl_scan_256(ntile, part4);
  if (e < E) {
    eoff[e] = lo_row;
    toff[e] = (int)(tincl - ntile);
    // virtual bases of e's groups, in group order from e's first row
    long long run = lo_row;
    for (int g = e; g < num_groups; g += E) {
      const bool sel = rank < 0 || ((g / E) % G) == rank;
      const int lo = min(max(goff[g], 0), rows);
      const int hi = min(max(goff[g + 1], lo), rows);
      gvb[g] = (int)min(run, (long long)rows);
      if (sel) run += hi - lo;
    }
  }
  if (e == E - 1) {
    eoff[E] = hi_row;
    toff[E] = (int)tincl;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int i = tid; i <= E; i += blockDim.x) s.eoff[i] = eoff[i];
    for (int g = tid; g < num_groups; g += blockDim.x) s.gvb[g] = gvb[g];
    if (tid == 0) *s.n_mtiles = toff[E];
    // tile i belongs to the last expert with toff <= i (experts without
    // tiles share their successor's offset and are skipped that way)
    for (int i = tid; i < toff[E]; i += blockDim.x) {
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (toff[mid] <= i) lo = mid; else hi = mid - 1;
      }
      s.mt_e[i] = lo;
      s.mt_v0[i] = eoff[lo] + (i - toff[lo]) * BM;
    }
  }
  const int v = blockIdx.x * blockDim.x + tid;
  if (v >= eoff[E]) return;
  int lo = 0, hi = E - 1;  // eoff[0] = 0 <= v
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (eoff[mid] <= v) lo = mid; else hi = mid - 1;
  }
  const int ev = lo;
  int jl = 0, jh = (num_groups - 1 - ev) / E;  // groups ev, ev+E, ... below num_groups
  while (jl < jh) {
    const int mid = (jl + jh + 1) >> 1;
    if (gvb[ev + mid * E] <= v) jl = mid; else jh = mid - 1;
  }
  const int g = ev + jl * E;
  const long long q64 = (long long)min(max(goff[g], 0), rows) + (v - gvb[g]);
  const int q = (int)min(max(q64, 0ll), (long long)rows - 1);
  s.rowmap[v] = q;
  const int src = gather ? gather[q] / gather_k : q;
  s.asrc[v] = (src >= 0 && src < rows_x) ? src : 0;
}

// Virtual -> physical row map, and the row of x each virtual row reads
// (through the gather, when the rows come straight from the unpermuted hidden
// states).  One thread per virtual row v < eoff[E]: its expert e is the last
// one with eoff[e] <= v (offsets staged in LDS), its group the last group g
// of e with gvb[g] <= v, and its physical row clamp(group_off[g]) + (v -
// gvb[g]).  So every virtual row a GEMM tile can read is written, and with a
// row in [0, rows) (by the schedule's construction, and clamped besides),
// whatever the device offsets hold.
__global__ __launch_bounds__(256) void rowmap_kernel(const int32_t* __restrict__ group_off, int num_groups, int E,
                                                     int rows, const int32_t* __restrict__ gather, int gather_k,
                                                     int rows_x, FfnSched s) {
  __shared__ int eo[MOELB_MAX_E + 1];
  for (int i = threadIdx.x; i <= E; i += blockDim.x) eo[i] = s.eoff[i];
  __syncthreads();
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= eo[E]) return;
  int lo = 0, hi = E - 1;  // eo[0] = 0 <= v
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (eo[mid] <= v) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  int jl = 0, jh = (num_groups - 1 - e) / E;  // groups e, e+E, ... below num_groups
  while (jl < jh) {
    const int mid = (jl + jh + 1) >> 1;
    if (s.gvb[e + mid * E] <= v) jl = mid; else jh = mid - 1;
  }
  const int g = e + jl * E;
  const long long q64 = (long long)min(max(group_off[g], 0), rows) + (v - s.gvb[g]);
  const int q = (int)min(max(q64, 0ll), (long long)rows - 1);
  s.rowmap[v] = q;
  const int src = gather ? gather[q] / gather_k : q;
  s.asrc[v] = (src >= 0 && src < rows_x) ? src : 0;
}

// XCD-aware tile id: workgroups go round-robin over 8 XCDs; give each XCD a
// contiguous range of tiles.  Returns -1 for workgroups with no tile.
__device__ __forceinline__ int xcd_tile(int total) {
  const int per = (total + 7) / 8;
  const int bid = blockIdx.x;
  const int t = (bid & 7) * per + (bid >> 3);
  return ((bid >> 3) < per && t < total) ? t : -1;
}

// Grouped tile order: GROUP_M consecutive M tiles x every N tile, M fastest.
// The ~32 tiles an XCD runs at once then share a few A row blocks and weight
// slices, which its L2 serves, instead of streaming a whole expert's weights
// per M tile.
constexpr int GROUP_M = 8;
__device__ __forceinline__ void grouped_tile(int t, int n_mtiles, int ntn, int& mt, int& nt, int GM = GROUP_M) {
  const int group = t / (GM * ntn);
  const int first = group * GM;
  const int gm = min(GM, n_mtiles - first);
  const int local = t - group * GM * ntn;
  nt = local / gm;
  mt = first + local % gm;
}

// ---------------------------------------------------------------- bf16 MFMA GEMM

// MODE 0: gate/up GEMM with SwiGLU epilogue -> amid (virtual rows, K = d).
// MODE 1: down GEMM amid x W2^T -> y (physical rows, K = inter).
//
// 256 threads = 4 waves in a 2 x 2 grid; wave tile 128 x 128 = 4 x 4 MFMA
// 32x32x16 fragments (256 fp32 accumulators per lane).  Global loads: lane
// (tid & 7) takes one 16-byte chunk of rows (tid >> 3) + 32 i, so 8 lanes read
// a 128-byte row segment.  Rows outside the tile's expert range read a valid
// row (their results are discarded); only the K tail is zero-filled.
template <int MODE>
__global__ __launch_bounds__(MF_THREADS) void ffn_mfma_kernel(const uint16_t* __restrict__ x, int rows_x,
                                                               const int32_t* __restrict__ gather, int gather_k,
                                                               const uint16_t* __restrict__ w, FfnSched s, int d,
                                                               int inter, int ntn, uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) char smem[];
  const int n_mtiles = *s.n_mtiles;
  const int tile = xcd_tile(n_mtiles * ntn);
  if (tile < 0) return;
  int mt, nt;
  grouped_tile(tile, n_mtiles, ntn, mt, nt);
  const int e = s.mt_e[mt];
  const int v0 = s.mt_v0[mt];
  const int vend = s.eoff[e + 1];
  const int K = MODE == 0 ? d : inter;
  const uint16_t* amid = static_cast<const uint16_t*>(s.amid);

  uint16_t* As = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Bs = As + 2 * MF_BM * MF_LDS_STRIDE;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int lc = (tid & 7) * 8;  // element offset of this lane's 16-byte chunk
  const int lr0 = tid >> 3;       // first of its rows (then + 32 i)

  // uniform bases; per-row 32-bit element offsets (the host checks they fit)
  const uint16_t* abase = MODE == 0 ? x : amid;
  const uint16_t* bbase = w + (MODE == 0 ? (size_t)e * 2 * inter * d : (size_t)e * d * inter);
  uint32_t aoff[8], boff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = lr0 + 32 * i;
    int v = v0 + r;
    v = v < vend ? v : v0;  // tiles always start with a valid row
    if (MODE == 0) {
      aoff[i] = (uint32_t)min(max(s.asrc[v], 0), rows_x - 1) * (uint32_t)d;
      int c = nt * 128 + (r & 127);
      c = c < inter ? c : 0;
      boff[i] = (uint32_t)((r < 128) ? c : inter + c) * (uint32_t)d;
    } else {
      aoff[i] = (uint32_t)v * (uint32_t)inter;
      int c = nt * 256 + r;
      c = c < d ? c : 0;
      boff[i] = (uint32_t)c * (uint32_t)inter;
    }
  }

  int nb[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
    nb[ni] = MODE == 0 ? (wn * 64 + (ni & 1) * 32 + (ni >> 1) * 128)  // gate 0, gate 1, up 0, up 1
                       : (wn * 128 + ni * 32);

  f32x16_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  uint4 ra[8], rb[8];
  const int KT = (K + MF_BK - 1) / MF_BK;
  const int fr = lane & 31;        // row (A) / column (B) of this lane in a fragment
  const int fk = (lane >> 5) * 8;  // k offset inside a 16-wide k step

  // full K step: no masks
#define MOELB_FFN_GLOAD(K0)                                                       \
  do {                                                                            \
    const uint32_t kk_ = (uint32_t)((K0) + lc);                                   \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                               \
      ra[i] = *reinterpret_cast<const uint4*>(abase + (aoff[i] + kk_));           \
      rb[i] = *reinterpret_cast<const uint4*>(bbase + (boff[i] + kk_));           \
    }                                                                             \
  } while (0)
  // last, partial K step: every load stays inside its row; lanes past K zero
#define MOELB_FFN_GLOAD_TAIL(K0)                                                  \
  do {                                                                            \
    const int kk_ = (K0) + lc;                                                    \
    const bool ok_ = kk_ < K;                                                     \
    const uint32_t ko_ = ok_ ? (uint32_t)kk_ : 0u;                                \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                               \
      const uint4 ta = *reinterpret_cast<const uint4*>(abase + (aoff[i] + ko_));  \
      const uint4 tb = *reinterpret_cast<const uint4*>(bbase + (boff[i] + ko_));  \
      ra[i].x = ok_ ? ta.x : 0u;                                                  \
      ra[i].y = ok_ ? ta.y : 0u;                                                  \
      ra[i].z = ok_ ? ta.z : 0u;                                                  \
      ra[i].w = ok_ ? ta.w : 0u;                                                  \
      rb[i].x = ok_ ? tb.x : 0u;                                                  \
      rb[i].y = ok_ ? tb.y : 0u;                                                  \
      rb[i].z = ok_ ? tb.z : 0u;                                                  \
      rb[i].w = ok_ ? tb.w : 0u;                                                  \
    }                                                                             \
  } while (0)
  const int KTF = K / MF_BK;  // full K steps

  if (KTF > 0)
    MOELB_FFN_GLOAD(0);
  else
    MOELB_FFN_GLOAD_TAIL(0);
  for (int kt = 0; kt < KT; ++kt) {
    uint16_t* Ab = As + (kt & 1) * MF_BM * MF_LDS_STRIDE;
    uint16_t* Bb = Bs + (kt & 1) * MF_BM * MF_LDS_STRIDE;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<uint4*>(Ab + (lr0 + 32 * i) * MF_LDS_STRIDE + lc) = ra[i];
      *reinterpret_cast<uint4*>(Bb + (lr0 + 32 * i) * MF_LDS_STRIDE + lc) = rb[i];
    }
    if (kt + 1 < KTF)
      MOELB_FFN_GLOAD((kt + 1) * MF_BK);
    else if (kt + 1 < KT)
      MOELB_FFN_GLOAD_TAIL((kt + 1) * MF_BK);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < MF_BK / 16; ++ks) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8_t*>(Ab + (wm * 128 + mi * 32 + fr) * MF_LDS_STRIDE + ks * 16 + fk);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        bfr[ni] = *reinterpret_cast<const bf16x8_t*>(Bb + (nb[ni] + fr) * MF_LDS_STRIDE + ks * 16 + fk);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
  }
#undef MOELB_FFN_GLOAD
#undef MOELB_FFN_GLOAD_TAIL

  // Epilogue: stage the output tile in LDS as bf16, then write 16-byte chunks
  // of whole row segments.  Accumulator layout: lane holds column (lane % 32)
  // of each fragment, rows (r / 4) * 8 + (lane / 32) * 4 + r % 4.
  constexpr int BN_OUT = MODE == 0 ? 128 : 256;
  constexpr int CS = BN_OUT + 8;
  uint16_t* Cs = reinterpret_cast<uint16_t*>(smem);
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 128 + mi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      if (MODE == 0) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const float g = acc[mi][f][r], u = acc[mi][f + 2][r];
          Cs[row * CS + wn * 64 + f * 32 + fr] = f32_to_bf16(silu_f32(g) * u);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) Cs[row * CS + wn * 128 + ni * 32 + fr] = f32_to_bf16(acc[mi][ni][r]);
      }
    }
  }
  __syncthreads();
  constexpr int CPR = BN_OUT / 8;  // 16-byte chunks per row
  const int n0 = nt * BN_OUT;
  const int nout = MODE == 0 ? inter : d;
  for (int c = tid; c < MF_BM * CPR; c += MF_THREADS) {
    const int row = c / CPR, ch = c % CPR;
    const int v = v0 + row;
    const int col = n0 + ch * 8;
    if (v >= vend || col >= nout) continue;
    const uint4 val = *reinterpret_cast<const uint4*>(Cs + row * CS + ch * 8);
    if (MODE == 0) {
      *reinterpret_cast<uint4*>(y + (size_t)v * inter + col) = val;
    } else {
      const int prow = min(max(s.rowmap[v], 0), rows_x - 1);
      *reinterpret_cast<uint4*>(y + (size_t)prow * d + col) = val;
    }
  }
}

// ---------------------------------------------------------------- bf16 MFMA GEMM, direct-to-LDS

// Same tile, waves and epilogue as ffn_mfma_kernel, for K % 64 == 0 (one
// workgroup per tile: used when K / 64 < 3; longer K runs in the persistent
// kernels below, which share this pipeline).
//  * Tiles of A and B stream global -> LDS with global_load_lds_dwordx4 (no
//    staging registers, no ds_write), in 64-wide K steps: each row request is
//    a whole 128-byte line, and each wave-instruction fills 1 KiB of LDS
//    (8 rows x 128 B), swizzled as below.
//  * LDS is a ring of five 32 KiB half-stages (A or B of one K step, 256 rows
//    x 64): A of step t in slot (2t) % 5, B of step t in slot (2t+1) % 5.  While
//    step t computes, steps t+1 and half of t+2 are in flight (160 KiB total).
//  * A wave blocks while the texture unit accepts a burst of loads, so the
//    refills are spread one instruction per four MFMAs over the step: B of
//    step t+2 during the last sub-step of t (after the barrier that frees its
//    slot) and the first of t+1, A of step t+3 during the second and third
//    sub-steps of t+1.
//  * The four 16-wide k sub-steps of a step are software-pipelined over two
//    fragment register sets (sub-step j+1 is read while j's MFMAs run, its
//    B fragments before its A fragments).  One barrier per step, behind the
//    third sub-step: every wave has read step t's stage and has its part of
//    step t+1 landed.  The persistent kernels peel the first and last steps,
//    so the steps between run with literal flags and no branch.
//  * The loads are issued from inline asm, so the compiler neither knows nor
//    waits for them: the vmcnt waits are explicit, and the compiler's own LDS
//    waits stay exact (a known LDS DMA makes it wait for every LDS read).
constexpr int DL_BK = 64;
constexpr int DL_HALF = MF_BM * DL_BK;  // elements of one half-stage
constexpr int DL_SLOTS = 5;
constexpr size_t DL_LDS_MAIN = (size_t)DL_SLOTS * DL_HALF * sizeof(uint16_t);
constexpr size_t DL_LDS_EPI = (size_t)MF_BM * (256 + 8) * sizeof(uint16_t);
constexpr size_t DL_LDS_BYTES = DL_LDS_MAIN > DL_LDS_EPI ? DL_LDS_MAIN : DL_LDS_EPI;

// 16-byte chunk c (0..7) of LDS row r sits in slot c ^ (((r >> 1) ^ (r << 2)) & 7):
// conflict-free fragment reads whether the LDS serves 8 or 16 lanes per pass.
__device__ __forceinline__ int dl_slot(int row, int chunk) { return chunk ^ (((row >> 1) ^ (row << 2)) & 7); }

// Weight addressing.  Byte offset of 16-byte chunk `chunk` (0..7) of the
// first 64-wide K step of an expert's weight row `row` (K elements per row),
// in the row-major layout or the packed one ([row/8][K/64][8][64]: the 8 rows
// of a block and one K step are one contiguous KiB, so a DMA instruction that
// loads 8 rows x 128 bytes reads one KiB of DRAM instead of 8 pieces 4 KiB
// or more apart).  One K step moves every row's data by w_step elements.
__device__ __forceinline__ uint32_t w_off(int row, int K, int chunk, bool packed) {
  return packed ? ((uint32_t)(row >> 3) * (uint32_t)K * 8u + (uint32_t)(row & 7) * 64u + (uint32_t)chunk * 8u) * 2u
                : ((uint32_t)row * (uint32_t)K + (uint32_t)chunk * 8u) * 2u;
}
__device__ __forceinline__ int w_step(bool packed) { return packed ? 512 : DL_BK; }

// 16 bytes per lane, global -> LDS: byte offset voff from the wave-uniform
// base sbase; lane i lands at LDS byte address m0 + 16 i.
// M0 is a reserved register, so the compiler warns that it does not preserve
// it across this asm; the build checks that no compiler code uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dl_copy16(uint32_t voff, const void* sbase, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
// The same copy marked non-temporal: lines read once, which the caches
// should give up first.
__device__ __forceinline__ void dl_copy16_nt(uint32_t voff, const void* sbase, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int MODE>
__global__ __launch_bounds__(MF_THREADS) void ffn_mfma_dma_kernel(const uint16_t* __restrict__ x, int rows_x,
                                                                   const int32_t* __restrict__ gather, int gather_k,
                                                                   const uint16_t* __restrict__ w, FfnSched s,
                                                                   int d, int inter, int ntn,
                                                                   uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) char smem[];
  const int n_mtiles = *s.n_mtiles;
  const int tile = xcd_tile(n_mtiles * ntn);
  if (tile < 0) return;
  int mt, nt;
  grouped_tile(tile, n_mtiles, ntn, mt, nt);
  const int e = s.mt_e[mt];
  const int v0 = s.mt_v0[mt];
  const int vend = s.eoff[e + 1];
  const int K = MODE == 0 ? d : inter;
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);
  const uint32_t lds_u32 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave >> 1, wn = wave & 1;

  // DMA rows of this lane: block (wave*8 + j) of 8 rows, row (lane >> 3) in it,
  // slot (lane & 7) <- global chunk dl_slot(row, slot); byte offsets
  const uint16_t* abase = MODE == 0 ? x : static_cast<const uint16_t*>(s.amid);
  const uint16_t* bbase = w + (MODE == 0 ? (size_t)e * 2 * inter * d : (size_t)e * d * inter);
  const int wstep = w_step(s.wpacked);  // elements one K step moves a weight row
  uint32_t aoff[8], boff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (wave * 8 + j) * 8 + (lane >> 3);
    const int chunk = dl_slot(r, lane & 7);
    int v = v0 + r;
    v = v < vend ? v : v0;
    if (MODE == 0) {
      aoff[j] = ((uint32_t)min(max(s.asrc[v], 0), rows_x - 1) * (uint32_t)d + chunk * 8) * 2u;
      int c = nt * 128 + (r & 127);
      c = c < inter ? c : 0;
      boff[j] = w_off((r < 128) ? c : inter + c, d, chunk, s.wpacked);
    } else {
      aoff[j] = ((uint32_t)v * (uint32_t)inter + chunk * 8) * 2u;
      int c = nt * 256 + r;
      c = c < d ? c : 0;
      boff[j] = w_off(c, inter, chunk, s.wpacked);
    }
  }

  int nb[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
    nb[ni] = MODE == 0 ? (wn * 64 + (ni & 1) * 32 + (ni >> 1) * 128) : (wn * 128 + ni * 32);

  f32x16_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  const int KT = K / DL_BK;
  const int nh = 2 * KT;  // half-stages: 2t = A of step t, 2t+1 = B of step t
#define DL_COPY(J, JJ)                                                                                 \
  {                                                                                                    \
    const int j_ = (J);                                                                                \
    const uint16_t* base_ = ((j_ & 1) ? bbase : abase) + (size_t)(j_ >> 1) * ((j_ & 1) ? wstep : DL_BK); \
    dl_copy16((j_ & 1) ? boff[JJ] : aoff[JJ], base_,                                                   \
              lds_u32 + (uint32_t)(((j_ % DL_SLOTS) * DL_HALF + (wave_s * 8 + (JJ)) * 8 * DL_BK) * 2)); \
  }
  // LDS element offsets (inside a half-stage) of this lane's fragments, per
  // 16-wide k sub-step
  const int fr = lane & 31;
  const int fh = lane >> 5;
  int aro[4][4], bro[4][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * 128 + i * 32 + fr;
      const int rb = nb[i] + fr;
      aro[ks][i] = ra * DL_BK + dl_slot(ra, ks * 2 + fh) * 8;
      bro[ks][i] = rb * DL_BK + dl_slot(rb, ks * 2 + fh) * 8;
    }
  bf16x8_t xa[4], xb[4], ya[4], yb[4];
  // One k sub-step: per 32-row block mi, read the next set's fragments (from
  // sub-step KS of half-stages SA/SB, if RD), run its 4 MFMAs on the current
  // set, then issue DMA instruction J0+mi of half-stage J (if DO).
#define DL_SUB(FA, FB, NA, NB, SA, SB, KS, RD, DO, J, J0)                                              \
  _Pragma("unroll") for (int mi = 0; mi < 4; ++mi) {                                                   \
    if (RD) {                                                                                          \
      /* B fragments first (blocks 0, 1 then 2, 3), then A: every read lands                       \
         at least 12 MFMAs before the next sub-step needs it */                                        \
      if (mi < 2) {                                                                                    \
        NB[2 * mi] = *reinterpret_cast<const bf16x8_t*>((SB) + bro[KS][2 * mi]);                       \
        NB[2 * mi + 1] = *reinterpret_cast<const bf16x8_t*>((SB) + bro[KS][2 * mi + 1]);               \
      } else {                                                                                         \
        NA[2 * mi - 4] = *reinterpret_cast<const bf16x8_t*>((SA) + aro[KS][2 * mi - 4]);               \
        NA[2 * mi - 3] = *reinterpret_cast<const bf16x8_t*>((SA) + aro[KS][2 * mi - 3]);               \
      }                                                                                                \
    }                                                                                                  \
    _Pragma("unroll") for (int ni = 0; ni < 4; ++ni)                                                   \
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FB[ni], FA[mi], acc[mi][ni], 0, 0, 0);     \
    if (DO) DL_COPY(J, (J0) + mi)                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                                 \
  }

  // the output row of this thread's tile row (down GEMM: physical row of the
  // virtual row), fetched now so its latency hides behind the K loop
  int out_row = 0;
  if (MODE == 1) {
    const int v = v0 + tid;
    out_row = v < vend ? min(max(s.rowmap[v], 0), rows_x - 1) : -1;
  }
  // the epilogue's scalar arguments are loaded before the loop: a scalar load
  // still in flight would make every LDS wait in the loop a full drain
  asm volatile("" ::"s"(y), "s"(rows_x));
  for (int j = 0; j < DL_SLOTS && j < nh; ++j)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) DL_COPY(j, jj)
  {
    // 8 instructions per half-stage and wave: wait for A_0 and B_0 only
    const int after = min(DL_SLOTS, nh) - 2;
    if (after >= 3)
      asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else if (after == 2)
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xa[i] = *reinterpret_cast<const bf16x8_t*>(lds + aro[0][i]);
    xb[i] = *reinterpret_cast<const bf16x8_t*>(lds + DL_HALF + bro[0][i]);
  }
  // One K step.  B1: issue the second half of B_kt+1; A2: issue A_kt+2; MORE:
  // a step follows (wait for its stages, barrier, read its first fragments);
  // B2: issue the first half of B_kt+2.  The loop runs the steps whose flags
  // are all true with literal flags, so its body has no branches; the first
  // and the last two steps are peeled.
#define DL_STEP(KT_, B1, A2, MORE, B2)                                                                 \
  {                                                                                                    \
    const int kt_ = (KT_);                                                                             \
    const uint16_t* sa = lds + ((2 * kt_) % DL_SLOTS) * DL_HALF;                                       \
    const uint16_t* sb = lds + ((2 * kt_ + 1) % DL_SLOTS) * DL_HALF;                                   \
    DL_SUB(xa, xb, ya, yb, sa, sb, 1, true, B1, 2 * kt_ + 3, 4)                                        \
    DL_SUB(ya, yb, xa, xb, sa, sb, 2, true, A2, 2 * kt_ + 4, 0)                                        \
    DL_SUB(xa, xb, ya, yb, sa, sb, 3, true, A2, 2 * kt_ + 4, 4)                                        \
    if (MORE) {                                                                                        \
      /* A_kt+2 is the only half-stage issued after B_kt+1; lgkmcnt(0): this                           \
         wave's reads of step kt have landed before any wave refills its slots */                      \
      if (B2)                                                                                          \
        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");                                    \
      else                                                                                             \
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");                                    \
      __builtin_amdgcn_s_barrier();                                                                    \
      asm volatile("" ::: "memory");                                                                   \
    }                                                                                                  \
    /* last sub-step: read step kt+1's first, refill A_kt's slot with the                              \
       first half of B_kt+2 */                                                                         \
    const uint16_t* na = lds + ((2 * kt_ + 2) % DL_SLOTS) * DL_HALF;                                   \
    const uint16_t* nbs = lds + ((2 * kt_ + 3) % DL_SLOTS) * DL_HALF;                                  \
    DL_SUB(ya, yb, xa, xb, na, nbs, 0, MORE, B2, 2 * kt_ + 5, 0)                                       \
  }
  if (KT >= 4) {
    DL_STEP(0, false, false, true, true)
    for (int kt = 1; kt + 2 < KT; ++kt) DL_STEP(kt, true, true, true, true)
    DL_STEP(KT - 2, true, false, true, false)
    DL_STEP(KT - 1, false, false, false, false)
  } else {
    for (int kt = 0; kt < KT; ++kt)
      DL_STEP(kt, kt >= 1 && kt + 1 < KT, kt >= 1 && kt + 2 < KT, kt + 1 < KT, kt + 2 < KT)
  }
#undef DL_STEP
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#undef DL_COPY
#undef DL_SUB

  // acc[mi][ni] holds its 32x32 block transposed (B fragment as the MFMA's
  // first operand): lane -> row (lane % 32) of block mi, element j -> column
  // (j / 4) * 8 + (lane / 32) * 4 + j % 4 of block ni, so a lane owns runs of 4
  // adjacent output columns and stages them with 8-byte LDS writes.
  constexpr int BN_OUT = MODE == 0 ? 128 : 256;
  constexpr int CS = BN_OUT + 8;
  uint16_t* Cs = lds;
  int* orow = reinterpret_cast<int*>(lds + MF_BM * CS);  // down GEMM: output row per tile row
  __syncthreads();
  if (MODE == 1) orow[tid] = out_row;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int row = wm * 128 + mi * 32 + fr;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (MODE == 0) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          float o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = silu_f32(acc[mi][f][q * 4 + i]) * acc[mi][f + 2][q * 4 + i];
          *reinterpret_cast<uint2*>(Cs + row * CS + wn * 64 + f * 32 + q * 8 + fh * 4) =
              make_uint2(bf16x2_pack(o[0], o[1]), bf16x2_pack(o[2], o[3]));
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const f32x16_t& a4 = acc[mi][ni];
          *reinterpret_cast<uint2*>(Cs + row * CS + wn * 128 + ni * 32 + q * 8 + fh * 4) =
              make_uint2(bf16x2_pack(a4[q * 4], a4[q * 4 + 1]), bf16x2_pack(a4[q * 4 + 2], a4[q * 4 + 3]));
        }
      }
    }
  }
  __syncthreads();
  constexpr int CPR = BN_OUT / 8;  // 16-byte chunks per row
  const int n0 = nt * BN_OUT;
  const int nout = MODE == 0 ? inter : d;
#pragma unroll 4
  for (int c = tid; c < MF_BM * CPR; c += MF_THREADS) {
    const int row = c / CPR, ch = c % CPR;
    const int v = v0 + row;
    const int col = n0 + ch * 8;
    if (v >= vend || col >= nout) continue;
    const uint4 val = *reinterpret_cast<const uint4*>(Cs + row * CS + ch * 8);
    if (MODE == 0) {
      *reinterpret_cast<uint4*>(y + (size_t)v * inter + col) = val;
    } else {
      *reinterpret_cast<uint4*>(y + (size_t)orow[row] * d + col) = val;
    }
  }
}

// ---------------------------------------------------------------- persistent GEMMs
//
// With K / 64 >= 3 both GEMMs run as persistent kernels: one workgroup per CU
// walks its tiles, and the K steps of consecutive tiles form one stream
// through the same 5-slot LDS ring, so the next tile's first steps load while
// the current tile finishes and stores.  The DMA offsets switch to the next
// tile two steps before a tile's end (from then on every refill belongs to
// it).  The epilogue stages the output through the ring slot of the tile's
// last B half-stage (free once its last sub-step has read it; the A slot
// beside it already takes the next refill), 32 KiB per round with XOR-swizzled
// 16-byte chunks: the gate/up GEMM's SwiGLU output in two rounds of 128 rows,
// the down GEMM's output in four rounds of 64 rows.

struct DlTile {
  int nt, e, v0, vend;
};

// Tile j of this workgroup: XCD x = blockIdx % 8 owns the contiguous range
// [x*per, (x+1)*per) of the grouped tile order and its workgroups take it in
// turn, so the tiles running at once on an XCD stay neighbours in that order.
__device__ __forceinline__ int dl_tile_id(int j, int total) {
  const int per = (total + 7) / 8;
  const int lo = (blockIdx.x >> 3) + j * (gridDim.x >> 3);
  const int t = (blockIdx.x & 7) * per + lo;
  return (lo < per && t < total) ? t : -1;
}

// Group height of the persistent tile order: the gate/up GEMM groups 8 M
// tiles; the down GEMM about 64 tiles per group (64 / N tiles, 2 .. 8 M tiles).
// Measured against 8 for both: C3's down GEMM 3 % faster with 4 (16 N
// tiles), C5's 3 % slower with 4 (8 N tiles), the gate/up GEMMs 1 % slower.
template <int MODE>
__device__ __forceinline__ int dl_group_m(int ntn) {
  return MODE == 0 ? GROUP_M : min(8, max(2, 64 / ntn));
}

template <int MODE>
__device__ __forceinline__ DlTile dl_tile(int t, int n_mtiles, int ntn, const FfnSched& s) {
  DlTile c;
  int mt, nt;
  grouped_tile(t, n_mtiles, ntn, mt, nt, dl_group_m<MODE>(ntn));
  c.nt = nt;
  c.e = s.mt_e[mt];
  c.v0 = s.mt_v0[mt];
  c.vend = s.eoff[c.e + 1];
  return c;
}

// Output row held by lane l of wave w.  In store round rd, iteration i, lane l
// of wave w stores staging row rl = 2w + (l>>5) + 8i, which is tile row
// (rl>>5)*128 + 32*rd + (rl&31); lane l holds the row of round l>>4, half
// (l>>3)&1, iteration l&7 (rows past the expert's end give row 0, unused).
__device__ __forceinline__ int dl_out_row(const DlTile& c, const FfnSched& s, int rows_y, int wave, int lane) {
  const int rl = 2 * wave + ((lane >> 3) & 1) + 8 * (lane & 7);
  const int row = (rl >> 5) * 128 + 32 * (lane >> 4) + (rl & 31);
  const int v = c.v0 + row;
  return v < c.vend ? min(max(s.rowmap[v], 0), rows_y - 1) : 0;
}

// Gate/up GEMM: the source rows of this lane's 8 DMA rows of tile c (rows
// past the expert's end repeat its first row), kept inside [0, rows_x).
__device__ __forceinline__ void dl_src_rows(const DlTile& c, const FfnSched& s, int rows_x, int wave, int lane,
                                            int (&src)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int v = c.v0 + (wave * 8 + j) * 8 + (lane >> 3);
    v = v < c.vend ? v : c.v0;
    src[j] = min(max(s.asrc[v], 0), rows_x - 1);
  }
}

template <int MODE>
__global__ __launch_bounds__(MF_THREADS) void ffn_persistent_kernel(const uint16_t* __restrict__ x, int rows_x,
                                                                    const uint16_t* __restrict__ w, FfnSched s,
                                                                    int rows_y, int d, int inter, int ntn,
                                                                    uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) char smem[];
  const int n_mtiles = *s.n_mtiles;
  const int total = n_mtiles * ntn;
  int ntiles = 0;
  while (dl_tile_id(ntiles, total) >= 0) ++ntiles;
  if (ntiles == 0) return;
  const int KT = (MODE == 0 ? d : inter) / DL_BK;
  const int nsteps = ntiles * KT;
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);
  const uint32_t lds_u32 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave >> 1, wn = wave & 1;
  const uint16_t* abase = MODE == 0 ? x : static_cast<const uint16_t*>(s.amid);

  // tile being stored (cur), the next one, and the DMA byte offsets of the
  // tile being loaded: block (wave*8 + j) of 8 rows, row (lane >> 3) in it,
  // slot (lane & 7) <- global chunk dl_slot(row, slot).  Gate/up: A rows come
  // through the source-row table (src holds the next tile's), B rows are 128
  // gate rows then the matching 128 up rows.
  DlTile cur = dl_tile<MODE>(dl_tile_id(0, total), n_mtiles, ntn, s);
  DlTile nxt = ntiles > 1 ? dl_tile<MODE>(dl_tile_id(1, total), n_mtiles, ntn, s) : cur;
  int src[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const uint16_t* bbase;
  const int wstep = w_step(s.wpacked);  // elements one K step moves a weight row
  uint32_t aoff[8], boff[8];
#define DL_OFFSETS(C)                                                                                  \
  {                                                                                                    \
    bbase = w + (MODE == 0 ? (size_t)(C).e * 2 * inter * d : (size_t)(C).e * d * inter);               \
    _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                                    \
      const int r = (wave * 8 + j) * 8 + (lane >> 3);                                                  \
      const int chunk = dl_slot(r, lane & 7);                                                          \
      if (MODE == 0) {                                                                                 \
        aoff[j] = ((uint32_t)src[j] * (uint32_t)d + chunk * 8) * 2u;                                   \
        int col = (C).nt * 128 + (r & 127);                                                            \
        col = col < inter ? col : 0;                                                                   \
        boff[j] = w_off((r < 128) ? col : inter + col, d, chunk, s.wpacked);                           \
      } else {                                                                                         \
        int v = (C).v0 + r;                                                                            \
        v = v < (C).vend ? v : (C).v0;                                                                 \
        aoff[j] = ((uint32_t)v * (uint32_t)inter + chunk * 8) * 2u;                                    \
        int col = (C).nt * 256 + r;                                                                    \
        col = col < d ? col : 0;                                                                       \
        boff[j] = w_off(col, inter, chunk, s.wpacked);                                                 \
      }                                                                                                \
    }                                                                                                  \
  }
  if (MODE == 0) dl_src_rows(cur, s, rows_x, wave, lane, src);
  DL_OFFSETS(cur)
  if (MODE == 0 && ntiles > 1) dl_src_rows(nxt, s, rows_x, wave, lane, src);
  int out_row = MODE == 1 ? dl_out_row(cur, s, rows_y, wave, lane) : 0;

  f32x16_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // DMA instruction JJ into ring slot SLOT of the A (ISB false) or B operand
  // of a K step that is KK steps into its tile
#define DL_COPY(SLOT, KK, ISB, JJ)                                                                     \
  {                                                                                                    \
    const uint16_t* base_ = ((ISB) ? bbase : abase) + (size_t)(KK) * ((ISB) ? wstep : DL_BK);          \
    dl_copy16((ISB) ? boff[JJ] : aoff[JJ], base_,                                                      \
              lds_u32 + (uint32_t)(((SLOT) * DL_HALF + (wave_s * 8 + (JJ)) * 8 * DL_BK) * 2));         \
  }
  // LDS element offsets (inside a half-stage) of this lane's fragments: A
  // block i adds i * 32 rows, B block i DL_NBO(i) rows (the swizzle of a row
  // depends on row % 32 only).  Gate/up: B blocks 0, 1 are gate rows, 2, 3 the
  // matching up rows.
  const int fr = lane & 31;
  const int fh = lane >> 5;
  const int fsw = ((fr >> 1) ^ (fr << 2)) & 7;
  int aro[4], bro[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    aro[ks] = (wm * 128 + fr) * DL_BK + (((ks * 2 + fh) ^ fsw) * 8);
    bro[ks] = ((MODE == 0 ? wn * 64 : wn * 128) + fr) * DL_BK + (((ks * 2 + fh) ^ fsw) * 8);
  }
#define DL_NBO(I) (MODE == 0 ? (((I) & 1) * 32 + ((I) >> 1) * 128) : (I) * 32)
  bf16x8_t xa[4], xb[4], ya[4], yb[4];
  // One k sub-step: per 32-row block mi, read the next set's fragments (from
  // sub-step KS of half-stages SA/SB, if RD), run its 4 MFMAs on the current
  // set (B fragment first: the accumulator holds the block transposed), then
  // issue DMA instruction J0+mi of half-stage SLOT (if DO).
#define DL_SUB(FA, FB, NA, NB, SA, SB, KS, RD, DO, SLOT, KK, ISB, J0)                                  \
  _Pragma("unroll") for (int mi = 0; mi < 4; ++mi) {                                                   \
    if (RD) {                                                                                          \
      /* B fragments first (blocks 0, 1 then 2, 3), then A: every read lands                       \
         at least 12 MFMAs before the next sub-step needs it */                                        \
      if (mi < 2) {                                                                                    \
        NB[2 * mi] = *reinterpret_cast<const bf16x8_t*>((SB) + bro[KS] + DL_NBO(2 * mi) * DL_BK);       \
        NB[2 * mi + 1] = *reinterpret_cast<const bf16x8_t*>((SB) + bro[KS] + DL_NBO(2 * mi + 1) * DL_BK); \
      } else {                                                                                         \
        NA[2 * mi - 4] = *reinterpret_cast<const bf16x8_t*>((SA) + aro[KS] + (2 * mi - 4) * 32 * DL_BK); \
        NA[2 * mi - 3] = *reinterpret_cast<const bf16x8_t*>((SA) + aro[KS] + (2 * mi - 3) * 32 * DL_BK); \
      }                                                                                                \
    }                                                                                                  \
    _Pragma("unroll") for (int ni = 0; ni < 4; ++ni)                                                   \
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FB[ni], FA[mi], acc[mi][ni], 0, 0, 0);     \
    if (DO) DL_COPY(SLOT, KK, ISB, (J0) + mi)                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                                 \
  }

  // values loaded by the compiler's own loads are waited for here, before any
  // DMA is in flight; scalar loads still pending would make every LDS wait in
  // the loop a full drain
  asm volatile("" ::"s"(y), "s"(rows_y), "s"(nxt.e), "s"(nxt.v0), "s"(nxt.vend), "s"(nxt.nt), "s"(cur.v0),
               "s"(cur.vend), "s"(cur.nt));
  asm volatile("" ::"v"(src[0]), "v"(src[1]), "v"(src[2]), "v"(src[3]), "v"(src[4]), "v"(src[5]), "v"(src[6]),
               "v"(src[7]), "v"(out_row));
  const int nh = 2 * nsteps;
  for (int j = 0; j < DL_SLOTS && j < nh; ++j)  // steps 0..2 of the first tile (K/64 >= 3)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) DL_COPY(j, j >> 1, j & 1, jj)
  {
    // 8 instructions per half-stage and wave: wait for A_0 and B_0 only
    const int after = min(DL_SLOTS, nh) - 2;
    if (after >= 3)
      asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else if (after == 2)
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xa[i] = *reinterpret_cast<const bf16x8_t*>(lds + aro[0] + i * 32 * DL_BK);
    xb[i] = *reinterpret_cast<const bf16x8_t*>(lds + DL_HALF + bro[0] + DL_NBO(i) * DL_BK);
  }
  // One K step (step kt of the tile, step g of the stream).  B1: issue the
  // second half of B_g+1; SWITCH: then point the refills at the next tile; A2:
  // issue A_g+2; MORE: a step follows (wait for its stages, barrier); B2: issue
  // the first half of B_g+2; RD0: read step g+1's first fragments (not at a
  // tile's end: they are read after the epilogue).  Inside a tile, the steps
  // 1 .. KT-3 have all flags true and run in a loop with literal flags, so its
  // body has no branches; the first and the last two steps are peeled.
#define DL_STEP(B1, SWITCH, A2, MORE, B2, RD0)                                                         \
  {                                                                                                    \
    /* ring slots of half-stages 2g .. 2g+4, places of steps g+1, g+2 in their tiles */                \
    const int s0 = (2 * g) % DL_SLOTS;                                                                 \
    const int s1 = s0 + 1 < DL_SLOTS ? s0 + 1 : s0 + 1 - DL_SLOTS;                                     \
    const int s2 = s1 + 1 < DL_SLOTS ? s1 + 1 : s1 + 1 - DL_SLOTS;                                     \
    const int s3 = s2 + 1 < DL_SLOTS ? s2 + 1 : s2 + 1 - DL_SLOTS;                                     \
    const int s4 = s3 + 1 < DL_SLOTS ? s3 + 1 : s3 + 1 - DL_SLOTS;                                     \
    const int k1 = kt + 1 < KT ? kt + 1 : kt + 1 - KT;                                                 \
    const int k2 = kt + 2 < KT ? kt + 2 : kt + 2 - KT;                                                 \
    /* slot offsets opaque to the compiler: it would otherwise precompute the                          \
       fragment addresses of every slot and hold them all in registers */                              \
    int o0 = s0 * DL_HALF, o1 = s1 * DL_HALF, o2 = s2 * DL_HALF, o3 = s3 * DL_HALF;                    \
    asm volatile("" : "+s"(o0), "+s"(o1), "+s"(o2), "+s"(o3));                                         \
    const uint16_t* sa = lds + o0;                                                                     \
    const uint16_t* sb = lds + o1;                                                                     \
    DL_SUB(xa, xb, ya, yb, sa, sb, 1, true, B1, s3, k1, true, 4)                                       \
    if (SWITCH) {                                                                                      \
      /* the next tile's offsets are computed here, not hoisted: they would                            \
         otherwise be held beside the current ones */                                                  \
      asm volatile("" : "+v"(src[0]), "+v"(src[1]), "+v"(src[2]), "+v"(src[3]), "+v"(src[4]),         \
                   "+v"(src[5]), "+v"(src[6]), "+v"(src[7]));                                          \
      DL_OFFSETS(nxt)                                                                                  \
    }                                                                                                  \
    DL_SUB(ya, yb, xa, xb, sa, sb, 2, true, A2, s4, k2, false, 0)                                      \
    DL_SUB(xa, xb, ya, yb, sa, sb, 3, true, A2, s4, k2, false, 4)                                      \
    if (MORE) {                                                                                        \
      /* A_g+2 is the only half-stage issued after B_g+1; lgkmcnt(0): this                             \
         wave's reads of step g have landed before any wave refills its slots */                       \
      if (B2)                                                                                          \
        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");                                    \
      else                                                                                             \
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");                                    \
      __builtin_amdgcn_s_barrier();                                                                    \
      asm volatile("" ::: "memory");                                                                   \
    }                                                                                                  \
    /* last sub-step: refill A_g's slot s0 with the first half of B_g+2 */                             \
    const uint16_t* na = lds + o2;                                                                     \
    const uint16_t* nbs = lds + o3;                                                                    \
    DL_SUB(ya, yb, xa, xb, na, nbs, 0, RD0, B2, s0, k2, true, 0)                                       \
  }
  int g = 0;  // step of the whole stream; half-stages 2g (A) and 2g+1 (B)
  for (int jcur = 0; jcur < ntiles; ++jcur) {
    // K / 64 >= 3: steps 0 (peeled), 1 .. KT-3 (loop), KT-2 and KT-1 (peeled)
    const bool last = jcur + 1 == ntiles;
    int kt = 0;
    DL_STEP(g >= 1, false, g >= 1, true, true, true)
    for (kt = 1, ++g; kt + 2 < KT; ++kt, ++g) DL_STEP(true, false, true, true, true, true)
    DL_STEP(true, !last, !last, true, !last, true)
    ++kt, ++g;
    DL_STEP(!last, false, !last, !last, !last, false)
    ++g;
    // ---- epilogue of tile jcur, staged through the slot of its last B
    // half-stage (free once its last sub-step has read it; the A slot beside
    // it already takes the next refill), 32 KiB per round
    const int gl = g - 1;
    uint16_t* Cs = lds + ((2 * gl + 1) % DL_SLOTS) * DL_HALF;
    __syncthreads();
    const bool has_nn = jcur + 2 < ntiles;
    const DlTile nn = has_nn ? dl_tile<MODE>(dl_tile_id(jcur + 2, total), n_mtiles, ntn, s) : nxt;
    const int next_out_row = (MODE == 1 && jcur + 1 < ntiles) ? dl_out_row(nxt, s, rows_y, wave, lane) : 0;
    asm volatile("" ::"s"(nn.e), "s"(nn.v0), "s"(nn.vend), "s"(nn.nt));
    if (MODE == 0) {
      // SwiGLU of the tile's 256 x 128 outputs in two rounds; in round rd
      // every wave stages its blocks mi = 2rd, 2rd+1: staging row
      // wm*64 + (mi-2rd)*32 + fr (256 B, chunk c at c ^ (row & 15))
      const int n0 = cur.nt * 128;
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) {
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
          const int mi = 2 * rd + m2;
          const int r = wm * 64 + m2 * 32 + fr;
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int f = 0; f < 2; ++f) {
              float o[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) o[i] = silu_f32(acc[mi][f][q * 4 + i]) * acc[mi][f + 2][q * 4 + i];
              const int chunk = wn * 8 + f * 4 + q;
              *reinterpret_cast<uint2*>(Cs + r * 128 + ((chunk ^ (r & 15)) * 8) + fh * 4) =
                  make_uint2(bf16x2_pack(o[0], o[1]), bf16x2_pack(o[2], o[3]));
            }
          __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = tid + MF_THREADS * i;
          const int rl = c >> 4, ch = c & 15;
          const int v = cur.v0 + (rl >> 6) * 128 + rd * 64 + (rl & 63);
          const int col = n0 + ch * 8;
          const uint4 val = *reinterpret_cast<const uint4*>(Cs + rl * 128 + ((ch ^ (rl & 15)) * 8));
          // non-temporal: the activations (P x I) far exceed the caches and
          // are read once, by the down GEMM
          if (v < cur.vend && col < inter) store_nt16(y + (size_t)v * inter + col, val);
        }
        __syncthreads();
      }
    } else {
      // four rounds; in round rd every wave stages its block mi = rd: staging
      // row wm*32 + fr (512 B, chunk c at c ^ (row & 15))
      const int n0 = cur.nt * 256;
#pragma unroll
      for (int rd = 0; rd < 4; ++rd) {
        const int r = wm * 32 + fr;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) {
            const f32x16_t& a4 = acc[rd][ni];
            const int chunk = wn * 16 + ni * 4 + q;
            *reinterpret_cast<uint2*>(Cs + r * 256 + ((chunk ^ (r & 15)) * 8) + fh * 4) =
                make_uint2(bf16x2_pack(a4[q * 4], a4[q * 4 + 1]), bf16x2_pack(a4[q * 4 + 2], a4[q * 4 + 3]));
          }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = tid + MF_THREADS * i;
          const int rl = c >> 5, ch = c & 31;  // rl = 2*wave + (lane >> 5) + 8*i
          const int v = cur.v0 + (rl >> 5) * 128 + rd * 32 + (rl & 31);
          const int col = n0 + ch * 8;
          const int orow = __shfl(out_row, rd * 16 + (lane >> 5) * 8 + i, 64);
          const uint4 val = *reinterpret_cast<const uint4*>(Cs + rl * 256 + ((ch ^ (rl & 15)) * 8));
          // non-temporal: Y (P x d) is read once, by the combine
          if (v < cur.vend && col < d) store_nt16(y + (size_t)orow * d + col, val);
        }
        __syncthreads();
      }
    }
    // source rows of the tile after next (first used at its offsets switch)
    if (MODE == 0 && has_nn) dl_src_rows(nn, s, rows_x, wave, lane, src);
    cur = nxt;
    nxt = nn;
    out_row = next_out_row;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
    // first fragments of the next tile (its first step landed before the epilogue)
    if (gl + 1 < nsteps) {
      const uint16_t* na = lds + ((2 * gl + 2) % DL_SLOTS) * DL_HALF;
      const uint16_t* nbs = lds + ((2 * gl + 3) % DL_SLOTS) * DL_HALF;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xa[i] = *reinterpret_cast<const bf16x8_t*>(na + aro[0] + i * 32 * DL_BK);
        xb[i] = *reinterpret_cast<const bf16x8_t*>(nbs + bro[0] + DL_NBO(i) * DL_BK);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#undef DL_COPY
#undef DL_SUB
#undef DL_OFFSETS
#undef DL_STEP
#undef DL_NBO
}

// ---------------------------------------------------------------- bf16 MFMA GEMM, 64-row tiles

// For few rows per expert (decode batches: tens of rows per expert), where
// the GEMMs stream expert weights and a 256-row tile would be mostly
// repeated rows: M tiles of 64 rows, the same 256 B rows per tile (gate/up:
// 128 gate rows and the matching 128 up rows; down: 256 output columns).
// One workgroup per tile, 4 waves; wave w takes all 64 A rows and B rows
// [32w, 32w+32) and [128+32w, ...) (gate/up: the gate and up rows of the same
// 32 columns, so the SwiGLU stays in the wave) or [64w, 64w+64) (down), as
// 2 x 2 blocks of v_mfma_f32_32x32x16_bf16.  A (8 KiB) and B (32 KiB) of each
// 64-wide K step stream global -> LDS with global_load_lds_dwordx4 into a
// ring of three stages, two steps ahead of the one computed; one barrier per
// step.  Each lane stores its four adjacent output columns straight from the
// accumulators (8 bytes).  Measured on the decode shape (T = 512, d = 2048,
// E = 128, k = 8, I = 768) and dropped: a persistent form with a four-stage
// ring streaming across tile boundaries (slower); 128-column tiles with a
// five-stage ring, twice the tiles for a smaller last round (gate/up 0.135
// against 0.125 ms); a four-stage ring (the same); a two-stage ring with two
// workgroups per CU (the same).  The depth of the stream is not what bounds
// these GEMMs at about 4.2 TB/s; the weights' row-major read pattern was
// (packed weights: 4.5 TB/s, gate/up 0.125 -> 0.114 ms).  128-column tiles
// with packed weights, for a better-balanced last round: still slower (0.120
// to 0.124 ms).  Weights are read non-temporally where one tile uses them:
// W13 in the gate/up GEMM (the tiles of an expert that share it run at the
// same time) and W2 of experts whose rows fit one tile.  The stream then no
// longer evicts the activations: the down GEMM finds its inputs cached, the
// next step's gate its hidden states and router (decode step 0.280 -> 0.265
// ms).  All of W2 read that way made the down GEMM slower (a hot expert's
// 64-row tiles share its W2 slices).
constexpr int SK_BM = 64;
constexpr int SK_BN = 256;
constexpr int SK_STAGE = (SK_BM + SK_BN) * DL_BK;  // elements per stage
constexpr int SK_STAGES = 3;
constexpr size_t SK_LDS_BYTES = (size_t)SK_STAGES * SK_STAGE * sizeof(uint16_t);
constexpr int SK_VPS = 10;  // DMA instructions per wave and stage: 2 of A, 8 of B

template <int MODE>
__global__ __launch_bounds__(MF_THREADS) void ffn_skinny_kernel(const uint16_t* __restrict__ x, int rows_x,
                                                                const uint16_t* __restrict__ w, FfnSched s,
                                                                int rows_y, int d, int inter, int ntn,
                                                                uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) char smem[];
  const int n_mtiles = *s.n_mtiles;
  const int tile = xcd_tile(n_mtiles * ntn);
  if (tile < 0) return;
  int mt, nt;
  grouped_tile(tile, n_mtiles, ntn, mt, nt);
  const int e = s.mt_e[mt];
  const int v0 = s.mt_v0[mt];
  const int vend = s.eoff[e + 1];
  const int K = MODE == 0 ? d : inter;
  const int KT = K / DL_BK;
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);
  const uint32_t lds_u32 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);

  // DMA rows of this lane: A block (wave*2 + j) of 8 rows, B block (wave*8 + j)
  // of 8 rows; row (lane >> 3) in the block, slot (lane & 7) <- global chunk
  // dl_slot(row, slot); byte offsets from the operand bases
  const uint16_t* abase = MODE == 0 ? x : static_cast<const uint16_t*>(s.amid);
  const uint16_t* bbase = w + (MODE == 0 ? (size_t)e * 2 * inter * d : (size_t)e * d * inter);
  const int wstep = w_step(s.wpacked);  // elements one K step moves a weight row
  uint32_t aoff[2], boff[8];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = (wave * 2 + j) * 8 + (lane >> 3);
    int v = v0 + r;
    v = v < vend ? v : v0;  // rows past the expert's end repeat its first row
    const uint32_t src = MODE == 0 ? (uint32_t)min(max(s.asrc[v], 0), rows_x - 1) : (uint32_t)v;
    aoff[j] = (src * (uint32_t)K + dl_slot(r, lane & 7) * 8) * 2u;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (wave * 8 + j) * 8 + (lane >> 3);
    uint32_t brow;
    if (MODE == 0) {
      int c = nt * 128 + (r & 127);
      c = c < inter ? c : 0;
      brow = (uint32_t)((r < 128) ? c : inter + c);
    } else {
      const int c = nt * 256 + r;
      brow = (uint32_t)(c < d ? c : 0);
    }
    boff[j] = w_off((int)brow, K, dl_slot(r, lane & 7), s.wpacked);
  }
  // the weight rows are read by this tile alone: the gate/up GEMM's W13 (the
  // tiles of one expert that share it run at the same time), or W2 of an
  // expert whose rows fit one tile
  const bool w_once = MODE == 0 || (v0 == s.eoff[e] && vend - v0 <= SK_BM);
  // issue K step KTI into its ring stage (SK_VPS instructions per wave)
  auto issue = [&](int kti) {
    const uint32_t st = lds_u32 + (uint32_t)((kti % SK_STAGES) * SK_STAGE) * 2u;
    const size_t ko = (size_t)kti * DL_BK;
#pragma unroll
    for (int j = 0; j < 2; ++j) dl_copy16(aoff[j], abase + ko, st + (uint32_t)((wave_s * 2 + j) * 8 * DL_BK) * 2u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t dst = st + (uint32_t)((SK_BM + (wave_s * 8 + j) * 8) * DL_BK) * 2u;
      if (w_once)
        dl_copy16_nt(boff[j], bbase + (size_t)kti * wstep, dst);
      else
        dl_copy16(boff[j], bbase + (size_t)kti * wstep, dst);
    }
  };

  // fragment rows: A blocks mi = 0, 1 (rows 32 mi + lane % 32); B blocks ni:
  // gate/up rows 32 wave + ni * 128, down rows 64 wave + 32 ni
  const int fr = lane & 31;
  const int fh = lane >> 5;
  int arow[2], brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    arow[i] = i * 32 + fr;
    brow[i] = SK_BM + (MODE == 0 ? wave * 32 + i * 128 : wave * 64 + i * 32) + fr;
  }
  f32x16_t acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // the epilogue's output rows, fetched now so their latency hides behind the K loop
  int orow[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int v = v0 + mi * 32 + fr;
    orow[mi] = v < vend ? (MODE == 0 ? v : min(max(s.rowmap[v], 0), rows_y - 1)) : -1;
  }
  asm volatile("" ::"v"(orow[0]), "v"(orow[1]), "s"(y));
  issue(0);
  if (KT > 1) issue(1);
  for (int kt = 0; kt < KT; ++kt) {
    // step kt landed (only step kt+1 may still be in flight), and every wave
    // has finished step kt-1, whose stage the refill below takes
    if (kt + 1 < KT)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(SK_VPS) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + 2 < KT) issue(kt + 2);
    const uint16_t* st = lds + (kt % SK_STAGES) * SK_STAGE;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = *reinterpret_cast<const bf16x8_t*>(st + arow[i] * DL_BK + dl_slot(arow[i], ks * 2 + fh) * 8);
        fb[i] = *reinterpret_cast<const bf16x8_t*>(st + brow[i] * DL_BK + dl_slot(brow[i], ks * 2 + fh) * 8);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ni], fa[mi], acc[mi][ni], 0, 0, 0);
    }
  }
  // acc[mi][ni] holds its block transposed: lane -> row (lane % 32) of block
  // mi, element j -> column (j / 4) * 8 + (lane / 32) * 4 + j % 4 of block ni
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    if (orow[mi] < 0) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (MODE == 0) {
        const int col = nt * 128 + wave * 32 + q * 8 + fh * 4;
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = silu_f32(acc[mi][0][q * 4 + i]) * acc[mi][1][q * 4 + i];
        if (col < inter)
          *reinterpret_cast<uint2*>(y + (size_t)orow[mi] * inter + col) =
              make_uint2(bf16x2_pack(o[0], o[1]), bf16x2_pack(o[2], o[3]));
      } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int col = nt * 256 + wave * 64 + ni * 32 + q * 8 + fh * 4;
          const f32x16_t& a4 = acc[mi][ni];
          if (col < d)
            *reinterpret_cast<uint2*>(y + (size_t)orow[mi] * d + col) =
                make_uint2(bf16x2_pack(a4[q * 4], a4[q * 4 + 1]), bf16x2_pack(a4[q * 4 + 2], a4[q * 4 + 3]));
        }
      }
    }
  }
}

// ---------------------------------------------------------------- fp32 SIMT GEMM

template <int MODE>
__global__ __launch_bounds__(256) void ffn_simt_kernel(const float* __restrict__ x, int rows_x,
                                                       const int32_t* __restrict__ gather, int gather_k,
                                                       const float* __restrict__ w, FfnSched s, int d, int inter,
                                                       int ntn, float* __restrict__ y) {
  __shared__ float As[SF_BK][SF_BM + 1];
  __shared__ float Bs[SF_BK][SF_BN + 1];
  __shared__ const float* arow[SF_BM];
  __shared__ const float* brow[SF_BN];
  const int tile = xcd_tile(*s.n_mtiles * ntn);
  if (tile < 0) return;
  const int mt = tile / ntn, nt = tile % ntn;
  const int e = s.mt_e[mt];
  const int v0 = s.mt_v0[mt];
  const int vend = s.eoff[e + 1];
  const int K = MODE == 0 ? d : inter;
  const float* amid = static_cast<const float*>(s.amid);
  const int tid = threadIdx.x;
  if (tid < SF_BM) {
    const int v = v0 + tid;
    const float* p = nullptr;
    if (v < vend) {
      if (MODE == 0) {
        p = x + (size_t)min(max(s.asrc[v], 0), rows_x - 1) * d;
      } else {
        p = amid + (size_t)v * inter;
      }
    }
    arow[tid] = p;
  } else if (tid < SF_BM + SF_BN) {
    const int j = tid - SF_BM;
    const float* p = nullptr;
    if (MODE == 0) {
      const int c = nt * 32 + (j & 31);
      if (c < inter) p = w + ((size_t)e * 2 * inter + (j < 32 ? c : inter + c)) * d;
    } else {
      const int c = nt * 64 + j;
      if (c < d) p = w + ((size_t)e * d + c) * inter;
    }
    brow[j] = p;
  }
  __syncthreads();
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += SF_BK) {
    for (int i = tid; i < SF_BK * SF_BM; i += 256) {
      const int r = i / SF_BK, kk = i % SF_BK;
      const float* pa = arow[r];
      As[kk][r] = (pa && k0 + kk < K) ? pa[k0 + kk] : 0.f;
      const float* pb = brow[r];
      Bs[kk][r] = (pb && k0 + kk < K) ? pb[k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < SF_BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
      b[0] = Bs[kk][tx * 2];
      b[1] = Bs[kk][tx * 2 + 1];
      b[2] = Bs[kk][32 + tx * 2];
      b[3] = Bs[kk][32 + tx * 2 + 1];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = v0 + ty * 4 + i;
    if (v >= vend) continue;
    if (MODE == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = nt * 32 + tx * 2 + j;
        if (c < inter) y[(size_t)v * inter + c] = silu_f32(acc[i][j]) * acc[i][j + 2];
      }
    } else {
      const size_t prow = (size_t)min(max(s.rowmap[v], 0), rows_x - 1) * d;
      const int cols[4] = {tx * 2, tx * 2 + 1, 32 + tx * 2, 32 + tx * 2 + 1};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = nt * 64 + cols[j];
        if (c < d) y[prow + c] = acc[i][j];
      }
    }
  }
}

}  // namespace

// Few rows per expert: the 64-row tile kernels (a host-side rule on the
// shapes, so every stage of one FFN call takes the same tile height).
static bool skinny_rows(int rows, int num_groups, int E) {
  (void)num_groups;
  return (size_t)rows < (size_t)128 * E;
}

// One workgroup per compute unit (a multiple of the 8 XCDs).
static int persistent_grid() {
  const int cus = moelb_compute_units();
  return cus < 8 ? 256 : cus & ~7;
}

extern "C" size_t moelb_grouped_ffn_workspace_bytes(int rows, int num_groups, int E, int d, int inter, int dtype) {
  (void)d;
  if (rows < 0 || num_groups < 1 || E < 1 || inter < 1 || !moelb_dtype_ok(dtype)) return 0;
  return sched_layout(rows, num_groups, E, inter, dtype, nullptr, nullptr);
}

extern "C" int moelb_grouped_ffn_stages(int stages, const void* x, int rows_x, int rows, const int32_t* group_off,
                                        int num_groups, int E, int G, int rank, const int32_t* gather, int gather_k,
                                        int d, int inter, int dtype, const void* w13, const void* w2, void* ws,
                                        size_t ws_bytes, void* y, void* stream) {
  const bool packed = stages & MOELB_FFN_PACKED_WEIGHTS;
  stages &= ~MOELB_FFN_PACKED_WEIGHTS;
  if (stages < 1 || stages > MOELB_FFN_ALL) return MOELB_EINVAL;
  if (rows < 0 || rows_x < 0 || num_groups < 1 || num_groups > 32768 || E < 1 || E > MOELB_MAX_E) return MOELB_EINVAL;
  if (d <= 0 || d % 8 != 0 || inter <= 0 || inter % 8 != 0 || !moelb_dtype_ok(dtype)) return MOELB_EINVAL;
  // packed weights: the bf16 GEMMs that stream whole 64-wide K steps read them
  if (packed && (dtype != MOELB_BF16 || d % 64 != 0 || inter % 64 != 0)) return MOELB_EINVAL;
  if (rank >= 0 && (G < 1 || rank >= G || num_groups % E != 0)) return MOELB_EINVAL;
  if (gather && gather_k < 1) return MOELB_EINVAL;
  if (!group_off || !w13 || !w2 || (rows > 0 && (!x || !y || rows_x < 1))) return MOELB_EINVAL;
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w13) | reinterpret_cast<uintptr_t>(w2) |
       reinterpret_cast<uintptr_t>(y)) & 15)
    return MOELB_EINVAL;
  // 32-bit byte offsets inside the GEMM kernels (per operand, from its base)
  const size_t eb = moelb_elem_bytes(dtype);
  if ((size_t)rows_x * d * eb >= (1ull << 32) || (size_t)rows * inter * eb >= (1ull << 32) ||
      (size_t)2 * inter * d * eb >= (1ull << 32))
    return MOELB_EINVAL;
  const size_t need = sched_layout(rows, num_groups, E, inter, dtype, nullptr, nullptr);
  if (!ws || ws_bytes < need) return MOELB_EWORKSPACE;
  FfnSched sc;
  sched_layout(rows, num_groups, E, inter, dtype, &sc, static_cast<char*>(ws));
  sc.wpacked = packed ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = dtype == MOELB_BF16;
  const bool skinny_tiles = bf && skinny_rows(rows, num_groups, E) && d % DL_BK == 0 && inter % DL_BK == 0;
  const int BM = bf ? (skinny_tiles ? SK_BM : MF_BM) : SF_BM;
  const bool run_up = stages & MOELB_FFN_GATE_UP, run_down = stages & MOELB_FFN_DOWN;
  if (stages & MOELB_FFN_SCHEDULE) {
    if (num_groups <= SCHED_FUSED_GROUPS) {
      hipLaunchKernelGGL(sched_rowmap_kernel, dim3(rows > 0 ? (rows + 255) / 256 : 1), dim3(256), 0, s, group_off,
                         num_groups, E, G < 1 ? 1 : G, rank, rows, BM, gather, gather_k, rows_x, sc);
      MOELB_CHECK_LAUNCH();
    } else {
      hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(256), 0, s, group_off, num_groups, E, G < 1 ? 1 : G, rank,
                         rows, BM, sc);
      MOELB_CHECK_LAUNCH();
      if (rows > 0)
        hipLaunchKernelGGL(rowmap_kernel, dim3((rows + 255) / 256), dim3(256), 0, s, group_off, num_groups, E, rows,
                           gather, gather_k, rows_x, sc);
      MOELB_CHECK_LAUNCH();
    }
  }
  const size_t mtiles = (size_t)(rows + BM - 1) / BM + E;
  if (bf) {
    if (!moelb_allow_lds(ffn_mfma_kernel<0>, MF_LDS_BYTES) || !moelb_allow_lds(ffn_mfma_kernel<1>, MF_LDS_BYTES))
      return MOELB_ELAUNCH;
    const int ntn0 = (inter + 127) / 128;
    const int ntn1 = (d + 255) / 256;
    // direct-to-LDS pipeline when K is a multiple of its 64-wide step
    const bool dma0 = d % DL_BK == 0, dma1 = inter % DL_BK == 0;  // else the register-staged kernel
    const bool pers0 = dma0 && d / DL_BK >= 3;                      // persistent kernels
    const bool pers1 = dma1 && inter / DL_BK >= 3;
    // 64-row tiles where experts average fewer than 128 rows (each 256-row
    // tile would be mostly repeated rows) and both K are whole 64-wide steps
    const bool skinny = skinny_rows(rows, num_groups, E) && dma0 && dma1;
    const size_t mtiles_sk = (size_t)(rows + SK_BM - 1) / SK_BM + E;
    if (skinny && (!moelb_allow_lds(ffn_skinny_kernel<0>, SK_LDS_BYTES) ||
                   !moelb_allow_lds(ffn_skinny_kernel<1>, SK_LDS_BYTES)))
      return MOELB_ELAUNCH;
    if ((dma0 && !moelb_allow_lds(ffn_mfma_dma_kernel<0>, DL_LDS_BYTES)) ||
        (dma1 && !moelb_allow_lds(ffn_mfma_dma_kernel<1>, DL_LDS_BYTES)) ||
        (pers0 && !moelb_allow_lds(ffn_persistent_kernel<0>, DL_LDS_BYTES)) ||
        (pers1 && !moelb_allow_lds(ffn_persistent_kernel<1>, DL_LDS_BYTES)))
      return MOELB_ELAUNCH;
    if (run_up) {
      if (skinny)
        hipLaunchKernelGGL(ffn_skinny_kernel<0>, dim3(mtiles_sk * ntn0 + 8), dim3(MF_THREADS), SK_LDS_BYTES, s,
                           static_cast<const uint16_t*>(x), rows_x, static_cast<const uint16_t*>(w13), sc, rows, d,
                           inter, ntn0, static_cast<uint16_t*>(sc.amid));
      else if (pers0)
        hipLaunchKernelGGL(ffn_persistent_kernel<0>, dim3(persistent_grid()), dim3(MF_THREADS), DL_LDS_BYTES, s,
                           static_cast<const uint16_t*>(x), rows_x, static_cast<const uint16_t*>(w13), sc, rows, d,
                           inter, ntn0, static_cast<uint16_t*>(sc.amid));
      else if (dma0)
        hipLaunchKernelGGL(ffn_mfma_dma_kernel<0>, dim3(mtiles * ntn0 + 8), dim3(MF_THREADS), DL_LDS_BYTES, s,
                           static_cast<const uint16_t*>(x), rows_x, gather, gather_k,
                           static_cast<const uint16_t*>(w13), sc, d, inter, ntn0, static_cast<uint16_t*>(sc.amid));
      else
        hipLaunchKernelGGL(ffn_mfma_kernel<0>, dim3(mtiles * ntn0 + 8), dim3(MF_THREADS), MF_LDS_BYTES, s,
                           static_cast<const uint16_t*>(x), rows_x, gather, gather_k,
                           static_cast<const uint16_t*>(w13), sc, d, inter, ntn0, static_cast<uint16_t*>(sc.amid));
      MOELB_CHECK_LAUNCH();
    }
    if (run_down) {
      if (skinny)
        hipLaunchKernelGGL(ffn_skinny_kernel<1>, dim3(mtiles_sk * ntn1 + 8), dim3(MF_THREADS), SK_LDS_BYTES, s,
                           nullptr, rows, static_cast<const uint16_t*>(w2), sc, rows, d, inter, ntn1,
                           static_cast<uint16_t*>(y));
      else if (pers1)
        hipLaunchKernelGGL(ffn_persistent_kernel<1>, dim3(persistent_grid()), dim3(MF_THREADS), DL_LDS_BYTES, s,
                           nullptr, rows, static_cast<const uint16_t*>(w2), sc, rows, d, inter, ntn1,
                           static_cast<uint16_t*>(y));
      else if (dma1)
        hipLaunchKernelGGL(ffn_mfma_dma_kernel<1>, dim3(mtiles * ntn1 + 8), dim3(MF_THREADS), DL_LDS_BYTES, s,
                           static_cast<const uint16_t*>(sc.amid), rows, nullptr, 1,
                           static_cast<const uint16_t*>(w2), sc, d, inter, ntn1, static_cast<uint16_t*>(y));
      else
        hipLaunchKernelGGL(ffn_mfma_kernel<1>, dim3(mtiles * ntn1 + 8), dim3(MF_THREADS), MF_LDS_BYTES, s,
                           static_cast<const uint16_t*>(sc.amid), rows, nullptr, 1,
                           static_cast<const uint16_t*>(w2), sc, d, inter, ntn1, static_cast<uint16_t*>(y));
      MOELB_CHECK_LAUNCH();
    }
  } else {
    const int ntn0 = (inter + 31) / 32;
    const int ntn1 = (d + 63) / 64;
    if (run_up) {
      hipLaunchKernelGGL(ffn_simt_kernel<0>, dim3(mtiles * ntn0 + 8), dim3(256), 0, s, static_cast<const float*>(x),
                         rows_x, gather, gather_k, static_cast<const float*>(w13), sc, d, inter, ntn0,
                         static_cast<float*>(sc.amid));
      MOELB_CHECK_LAUNCH();
    }
    if (run_down) {
      hipLaunchKernelGGL(ffn_simt_kernel<1>, dim3(mtiles * ntn1 + 8), dim3(256), 0, s,
                         static_cast<const float*>(sc.amid), rows, nullptr, 1, static_cast<const float*>(w2), sc, d,
                         inter, ntn1, static_cast<float*>(y));
      MOELB_CHECK_LAUNCH();
    }
  }
  return MOELB_OK;
}

// ---------------------------------------------------------------- packed weights

// One thread per 16-byte chunk of w ([E][rows][K] bf16, K/8 chunks per row):
// chunk c of row (e, r) goes to chunk ((e*rows/8 + r/8)*(K/64) + c/8)*64 +
// (r%8)*8 + c%8 of the packed array.  Reads are coalesced; each group of 8
// threads writes 128 contiguous bytes.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint4* __restrict__ w, long long nchunks, int rows,
                                                           int K, uint4* __restrict__ packed) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nchunks) return;
  const int cpr = K / 8;
  const long long row_all = i / cpr;
  const int c = (int)(i - row_all * cpr);
  const long long e = row_all / rows;
  const int r = (int)(row_all - e * rows);
  const long long dst = ((e * (rows / 8) + r / 8) * (K / 64) + c / 8) * 64 + (r % 8) * 8 + (c % 8);
  packed[dst] = w[i];
}

extern "C" int moelb_pack_weights(const void* w, int E, int rows, int K, int dtype, void* packed, void* stream) {
  if (E < 1 || rows < 8 || rows % 8 != 0 || K < 64 || K % 64 != 0 || dtype != MOELB_BF16) return MOELB_EINVAL;
  if (!w || !packed) return MOELB_EINVAL;
  if ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(packed)) & 15) return MOELB_EINVAL;
  const unsigned long long bytes = (unsigned long long)E * rows * K * 2ull;
  const uintptr_t a = reinterpret_cast<uintptr_t>(w), b = reinterpret_cast<uintptr_t>(packed);
  if (a < b + bytes && b < a + bytes) return MOELB_EINVAL;  // overlapping
  const long long nchunks = (long long)(bytes / 16);
  const long long blocks = (nchunks + 255) / 256;
  if (blocks > 0x7fffffffll) return MOELB_EINVAL;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(w), nchunks, rows, K, static_cast<uint4*>(packed));
  MOELB_CHECK_LAUNCH();
  return MOELB_OK;
}

extern "C" int moelb_grouped_ffn(const void* x, int rows_x, int rows, const int32_t* group_off, int num_groups, int E,
                                 int G, int rank, const int32_t* gather, int gather_k, int d, int inter, int dtype,
                                 const void* w13, const void* w2, void* ws, size_t ws_bytes, void* y, void* stream) {
  return moelb_grouped_ffn_stages(MOELB_FFN_ALL, x, rows_x, rows, group_off, num_groups, E, G, rank, gather, gather_k,
                                  d, inter, dtype, w13, w2, ws, ws_bytes, y, stream);
}
