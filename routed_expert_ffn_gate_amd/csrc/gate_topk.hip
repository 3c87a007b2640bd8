// Router GEMM of the current layer and the lookahead router of the next layer,
// with softmax, top-k and the k-th/(k+1)-th logit gap fused into the epilogue.
//
// Definition: FreeBalance ("FreeBalance: Pre-Routing Online MoE Load Balancing
// via Residual Workload Prediction"), section 2.1 (W,I = topk(G(h))) and
// eq. 2-4 (the same linear router g(X) = XW + 1b^T applied to the previous
// layer's hidden states); Libra README "Key Ideas" (layer i+1's gate on layer
// i's hidden states).
//
// Design (gfx950): one GEMM with N = 2E columns (current router rows, then the
// lookahead router's rows), so h -- the only large operand -- is read from HBM
// once.  A workgroup owns BM tokens and all N columns, so every logit of a
// token ends up in one workgroup for the epilogue: BM = 128, or 64 where the
// batch has too few 128-token blocks to fill the CUs.  8 waves: 2 (token
// halves) x 4 (column quarters); each wave runs bf16 MFMA 16x16x32 on a
// (BM/2) x (16*NF) tile.  In the register-staged form, h tiles are staged
// through LDS (double buffered, one barrier per K step) and router rows go
// straight from global/L2 into registers, since each wave needs only its own
// columns; the direct-to-LDS form is described above its kernel.  The
// epilogue writes biased fp32 logits to LDS and 2-8 lanes per token and
// direction select the top-(k+2) with a register insertion list (one median
// instruction per entry), merged across those lanes by DPP; the selection is
// exact (see topk_epilogue).
#include "common.h"

namespace {

constexpr int GATE_BM = 128;       // tokens per workgroup (the direct-to-LDS form also takes 64)
constexpr int GATE_BK = 64;        // K per pipeline step
constexpr int GATE_THREADS = 512;  // 8 waves
constexpr int A_STRIDE = GATE_BK + 8;  // bf16 elements per LDS row (16 B pad)

// Selection keys of logit v of expert id: the float's bits mapped to an
// order-preserving unsigned integer, followed by 255 - id, so a larger key is
// a larger logit and equal logits rank the lower id first.  The fast key
// keeps the top 24 bits of the logit (logits within 2^-15 relative of each
// other share a bucket and rank by id); the exact key keeps all 32.
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  const uint32_t b = __float_as_uint(v);
  return b ^ ((b & 0x80000000u) ? 0xffffffffu : 0x80000000u);
}
__device__ __forceinline__ uint32_t topk_key(float v, int id) {
  return (ordered_bits(v) & 0xffffff00u) | (uint32_t)(255 - id);
}
__device__ __forceinline__ uint64_t topk_key_exact(float v, int id) {
  return ((uint64_t)ordered_bits(v) << 8) | (uint64_t)(255 - id);
}

// Sorted (descending) insertion of key x into a register list of KL keys, one
// instruction per entry: the new entry i is the median of x, the old entry i
// and the old entry i-1 (x itself where it belongs, the entry above it
// shifted down below that, the old entry above), so every entry is computed
// from the old list, last entry first, with no chain between them.
__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
template <int KL>
__device__ __forceinline__ void list_insert(uint32_t (&l)[KL], uint32_t x) {
#pragma unroll
  for (int i = KL - 1; i > 0; --i) l[i] = med3_u32(x, l[i], l[i - 1]);
  l[0] = x > l[0] ? x : l[0];
}

// Partner key in the merge round of lane groups of 2M (DPP, no LDS round
// trip): rounds 1 and 2 swap within quads, round 4 mirrors each half-row of 8
// lanes.  Any pairing that joins the two halves of every group of 2M lanes
// merges correctly.
template <int M>
__device__ __forceinline__ uint32_t merge_partner(uint32_t v) {
  static_assert(M == 1 || M == 2 || M == 4, "token groups of 2, 4 or 8 lanes");
  constexpr int ctrl = M == 1 ? 0xB1 : M == 2 ? 0x4E : 0x141;
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, 0xF, 0xF, false);
}

template <int M, int KL>
__device__ __forceinline__ void merge_round(uint32_t (&l)[KL]) {
  uint32_t p[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) p[i] = merge_partner<M>(l[i]);
#pragma unroll
  for (int i = 0; i < KL; ++i) list_insert<KL>(l, p[i]);
}

// The KL largest keys of a token's E logits in `row`: each of the token's lpt
// lanes (sub = 0..lpt-1) scans every lpt-th logit (four loads ahead of their
// inserts), then the partial lists are merged across those lanes, so every
// lane ends with the whole list.  All lanes of the wave take part (inactive
// tokens scan nothing), in uniform control flow.
template <int KL>
__device__ __forceinline__ void select_keys(const float* row, bool active, int E, int sub, int lpt, uint32_t (&l)[KL]) {
#pragma unroll
  for (int i = 0; i < KL; ++i) l[i] = 0;  // below every real key
  if (active) {
    int e = sub;
    for (; e + 3 * lpt < E; e += 4 * lpt) {
      const float v0 = row[e], v1 = row[e + lpt], v2 = row[e + 2 * lpt], v3 = row[e + 3 * lpt];
      list_insert<KL>(l, topk_key(v0, e));
      list_insert<KL>(l, topk_key(v1, e + lpt));
      list_insert<KL>(l, topk_key(v2, e + 2 * lpt));
      list_insert<KL>(l, topk_key(v3, e + 3 * lpt));
    }
    for (; e < E; e += lpt) list_insert<KL>(l, topk_key(row[e], e));
  }
  if (lpt > 1) merge_round<1>(l);
  if (lpt > 2) merge_round<2>(l);
  if (lpt > 4) merge_round<4>(l);
}

// Epilogue over `ntok` tokens whose logits (bias included) sit in LDS rows of
// `stride` floats: columns [0,E) current, [E,2E) lookahead (if has_next).
// The 512 threads split into directions (two if has_next), then tokens of
// `lpt` adjacent lanes (a power of two, 2..8): direction = tid / per_dir,
// token = (tid % per_dir) / lpt, sub = tid % lpt.
//
// Selection is exact: the k+2 largest fast keys are found first.  If entries
// k and k+1 fall in different buckets, no logit outside the first k+1
// entries shares entry k's bucket, so those entries are exactly the k+1
// largest logits, in exact order unless two adjacent ones share a bucket.
// A token where either fails (rare: a few in ten thousand here) is selected
// again by the whole wave, by exact keys: each lane holds a few of the
// token's logits and k+1 wave-wide maxima give the order.  One workgroup per
// CU means the slowest wave sets the kernel's time, so this path is kept
// short rather than merely rare.
template <int KL>
__device__ __forceinline__ void topk_epilogue(const float* z, int stride, int ntok, int lpt, int tok0, int T, int E,
                                              int k, bool has_next, int32_t* __restrict__ idx,
                                              float* __restrict__ wts, float* __restrict__ gap,
                                              int32_t* __restrict__ idx_next) {
  const int tid = threadIdx.x;
  const int per_dir = has_next ? GATE_THREADS / 2 : GATE_THREADS;
  const int dir = tid / per_dir;
  const int tl = (tid % per_dir) / lpt;
  const int sub = tid & (lpt - 1);
  const bool active = tl < ntok;
  const int t = tok0 + tl;
  const float* row = z + tl * stride + dir * E;
  uint32_t l[KL];
  select_keys<KL>(row, active, E, sub, lpt, l);
  int li[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) li[i] = min(255 - (int)(l[i] & 0xffu), E - 1);  // unused entries stay in the row
  // buckets of entries k and k+1, and adjacent equal buckets among 0..k (k is
  // a runtime value: no dynamic register indexing)
  uint32_t bk = 0u, bk1 = 1u;
  bool tie_run = false;
#pragma unroll
  for (int j = 0; j < KL; ++j) {
    if (j == k) bk = l[j] >> 8;
    if (j == k + 1) bk1 = l[j] >> 8;
    if (j + 1 < KL && j + 1 <= k && (l[j] >> 8) == (l[j + 1] >> 8)) tie_run = true;
  }
  const bool redo = active && ((k + 2 <= E && bk == bk1) || tie_run);
  uint64_t todo = __ballot(redo);
  while (todo != 0ull) {
    // one such token per round, all 64 lanes on it (E <= 256: four logits per lane)
    const int src = __ffsll(static_cast<long long>(todo)) - 1;
    const int first = src & ~(lpt - 1);
    todo &= ~(((lpt == 64 ? 0ull : (1ull << lpt)) - 1ull) << first);
    const int off = __shfl(static_cast<int>(row - z), src, MOELB_WAVE);
    const int lane = threadIdx.x & (MOELB_WAVE - 1);
    uint64_t mine[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      mine[q] = e < E ? topk_key_exact(z[off + e], e) : 0ull;
    }
    int ids[KL];
#pragma unroll
    for (int r = 0; r < KL; ++r) {
      uint64_t b = mine[0];
#pragma unroll
      for (int q = 1; q < 4; ++q) b = mine[q] > b ? mine[q] : b;
#pragma unroll
      for (int m = 1; m < MOELB_WAVE; m <<= 1) {
        const uint64_t o = __shfl_xor(b, m, MOELB_WAVE);
        b = o > b ? o : b;
      }
      ids[r] = min(255 - (int)(b & 0xffu), E - 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) mine[q] = mine[q] == b ? 0ull : mine[q];
    }
    if (lane >= first && lane < first + lpt) {
#pragma unroll
      for (int i = 0; i < KL; ++i) li[i] = ids[i];
    }
  }
  if (dir == 0) {
    // softmax denominator over all E logits of this token (no weights wanted:
    // a lookahead-only block of the split launch)
    const float mx = active ? row[li[0]] : 0.f;
    float s = 0.f;
    if (active && wts) {
      // four loads ahead of their terms; the terms are added in scan order
      int e = sub;
      for (; e + 3 * lpt < E; e += 4 * lpt) {
        const float z0 = row[e], z1 = row[e + lpt], z2 = row[e + 2 * lpt], z3 = row[e + 3 * lpt];
        s += __expf(z0 - mx);
        s += __expf(z1 - mx);
        s += __expf(z2 - mx);
        s += __expf(z3 - mx);
      }
      for (; e < E; e += lpt) s += __expf(row[e] - mx);
    }
    for (int m = 1; m < lpt; m <<= 1) s += __shfl_xor(s, m, MOELB_WAVE);
    if (active && sub == 0 && t < T) {
      const float inv = 1.0f / s;
#pragma unroll
      for (int j = 0; j < KL; ++j) {
        if (j < k) {
          idx[(size_t)t * k + j] = li[j];
          if (wts) wts[(size_t)t * k + j] = __expf(row[li[j]] - mx) * inv;
        }
      }
      if (gap) {
        float g = INFINITY;
#pragma unroll
        for (int j = 1; j < KL; ++j)
          if (j == k && k < E) g = row[li[j - 1]] - row[li[j]];
        gap[t] = g;
      }
    }
  } else if (active && sub == 0 && t < T) {
#pragma unroll
    for (int j = 0; j < KL; ++j)
      if (j < k) idx_next[(size_t)t * k + j] = li[j];
  }
}

// ---------------------------------------------------------------- bf16 MFMA kernel

template <int NF, int KL>
__global__ __launch_bounds__(GATE_THREADS) void gate_topk_bf16_kernel(
    const uint16_t* __restrict__ h, int T, int d, int E, int k, const uint16_t* __restrict__ w_cur,
    const float* __restrict__ b_cur, const uint16_t* __restrict__ w_next, const float* __restrict__ b_next,
    int32_t* __restrict__ idx, float* __restrict__ wts, float* __restrict__ gap, int32_t* __restrict__ idx_next,
    int zstride) {
  extern __shared__ __align__(16) char smem[];
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);  // [2][GATE_BM][A_STRIDE]
  float* Z = reinterpret_cast<float*>(smem);          // [64][zstride], after the K loop

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const int tok0 = blockIdx.x * GATE_BM;
  const bool has_next = w_next != nullptr;
  const int N = has_next ? 2 * E : E;

  // A staging: 128 rows x 64 k = 1024 chunks of 16 B, two per thread.
  int a_row[2], a_kc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid * 2 + i;
    a_row[i] = c >> 3;
    a_kc[i] = (c & 7) * 8;
  }
  // B: wave's columns, fragment ni covers columns colbase + ni*16 + (lane % 16).
  const int colbase = wn * NF * 16;
  const uint16_t* brow[NF];
  bool bvalid[NF];
#pragma unroll
  for (int ni = 0; ni < NF; ++ni) {
    const int col = colbase + ni * 16 + (lane & 15);
    bvalid[ni] = col < N;
    const uint16_t* base = col < E ? w_cur + (size_t)col * d : w_next + (size_t)(col - E) * d;
    brow[ni] = bvalid[ni] ? base : w_cur;
  }
  const int bk = (lane >> 4) * 8;  // k offset of this lane inside a 32-wide k step

  f32x4_t acc[4][NF];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < NF; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 areg[2];
  bf16x8_t breg[2][NF];
  const uint4 zero4 = make_uint4(0, 0, 0, 0);

  auto load_a = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = tok0 + a_row[i];
      const int kk = k0 + a_kc[i];
      areg[i] = (t < T && kk < d) ? *reinterpret_cast<const uint4*>(h + (size_t)t * d + kk) : zero4;
    }
  };
  auto load_b = [&](int k0) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int ni = 0; ni < NF; ++ni) {
        const int kk = k0 + ks * 32 + bk;
        const uint4 v = (bvalid[ni] && kk < d) ? *reinterpret_cast<const uint4*>(brow[ni] + kk) : zero4;
        breg[ks][ni] = __builtin_bit_cast(bf16x8_t, v);
      }
  };

  const int KT = (d + GATE_BK - 1) / GATE_BK;
  load_a(0);
  load_b(0);
  for (int kt = 0; kt < KT; ++kt) {
    uint16_t* Ab = As + (kt & 1) * GATE_BM * A_STRIDE;
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(Ab + a_row[i] * A_STRIDE + a_kc[i]) = areg[i];
    bf16x8_t bcur[2][NF];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int ni = 0; ni < NF; ++ni) bcur[ks][ni] = breg[ks][ni];
    if (kt + 1 < KT) {
      load_a((kt + 1) * GATE_BK);
      load_b((kt + 1) * GATE_BK);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int r = wm * 64 + mi * 16 + (lane & 15);
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(Ab + r * A_STRIDE + ks * 32 + bk);
#pragma unroll
        for (int ni = 0; ni < NF; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bcur[ks][ni], acc[mi][ni], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // LDS is reused for the logits

  // Epilogue, one token half (64 rows) at a time.
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int ni = 0; ni < NF; ++ni) {
        const int col = colbase + ni * 16 + (lane & 15);
        if (col < N) {
          const float bias = col < E ? b_cur[col] : b_next[col - E];
#pragma unroll
          for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = mi * 16 + (lane >> 4) * 4 + i;
              Z[r * zstride + col] = acc[mi][ni][i] + bias;
            }
        }
      }
    }
    __syncthreads();
    const int t0 = tok0 + half * 64;
    const int ntok = min(64, T - t0);
    if (ntok > 0) topk_epilogue<KL>(Z, zstride, ntok, has_next ? 4 : 8, t0, T, E, k, has_next, idx, wts, gap, idx_next);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- bf16 MFMA kernel, direct-to-LDS

// The same waves and epilogue as gate_topk_bf16_kernel, for N = 64 * NF
// columns and d % 64 == 0, with BM = 128 or 64 tokens per workgroup.  The h
// tile (BM x 64) and the router rows (N x 64) of each 64-wide K step stream
// global -> LDS with
// global_load_lds_dwordx4 into S swizzled stages (16-byte chunk c of row r in
// slot c ^ (((r >> 1) ^ (r << 2)) & 7): conflict-free 16-row fragment reads).
// A wave is held up while the texture unit accepts a burst of loads, so the
// refill of a stage is spread over the MFMAs of the following sub-steps.
// Fragment reads are software-pipelined against the MFMAs over two register
// sets; one barrier per K step; waits are explicit vmcnt.
__device__ __forceinline__ int gt_slot(int row, int chunk) { return chunk ^ (((row >> 1) ^ (row << 2)) & 7); }

// 16 bytes per lane, global -> LDS: byte offset voff from the wave-uniform base
// sbase, lane i lands at LDS byte address m0 + 16 i.  Issued from inline asm so
// the compiler's LDS wait tracking stays exact; completion is tracked by the
// caller's explicit vmcnt waits.
// M0 is a reserved register, so the compiler warns that it does not preserve
// it across this asm; the build checks that no compiler code uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void gt_copy16(uint32_t voff, const void* sbase, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Split launch (gridDim.y == 2, for few token blocks): the blocks with y = 0
// run the current router alone and the blocks with y = 1 the lookahead router
// alone (its top-k indices only), so twice as many workgroups each read half
// the router rows; N = 64 * NF then covers E columns (padding columns read row
// 0 and are never selected).
template <int NF, int KL, int S, int BM>
__global__ __launch_bounds__(GATE_THREADS) void gate_topk_dma_kernel(
    const uint16_t* __restrict__ h, int T, int d, int E, int k, const uint16_t* __restrict__ w_cur_in,
    const float* __restrict__ b_cur_in, const uint16_t* __restrict__ w_next_in, const float* __restrict__ b_next_in,
    int32_t* __restrict__ idx_in, float* __restrict__ wts_in, float* __restrict__ gap_in,
    int32_t* __restrict__ idx_next_in, int zstride) {
  const bool split = gridDim.y == 2;
  const bool look = split && blockIdx.y == 1;
  const uint16_t* w_cur = look ? w_next_in : w_cur_in;
  const float* b_cur = look ? b_next_in : b_cur_in;
  const uint16_t* w_next = split ? nullptr : w_next_in;
  const float* b_next = split ? nullptr : b_next_in;
  int32_t* idx = look ? idx_next_in : idx_in;
  float* wts = look ? nullptr : wts_in;
  float* gap = look ? nullptr : gap_in;
  int32_t* idx_next = split ? nullptr : idx_next_in;
  constexpr int BK = 64;
  constexpr int N = 64 * NF;
  constexpr int AV = BM / 64;             // h-row DMA instructions per wave and K step
  constexpr int MI = BM / 32;             // 16-row blocks of a wave's BM/2 tokens
  constexpr int STAGE = (BM + N) * BK;    // elements: A rows, then B rows
  constexpr int VPS = AV + NF;            // DMA instructions per wave and K step
  // the logits of all BM tokens fit in the stages' LDS
  constexpr bool ONE_PASS = (size_t)BM * (N + 4) * 4 <= (size_t)S * STAGE * 2;
  extern __shared__ __align__(16) char smem[];
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);
  float* Z = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const int tok0 = blockIdx.x * BM;
  const bool has_next = w_next != nullptr;
  const int KT = d / BK;

  // DMA rows of this lane: 8-row blocks, row (lane >> 3), slot (lane & 7);
  // byte offsets from a wave-uniform base (h, or the router matrix that holds
  // the whole 8-row block: E is a multiple of 32 here)
  uint32_t aoff[AV];
#pragma unroll
  for (int j = 0; j < AV; ++j) {
    const int r = (wave * AV + j) * 8 + (lane >> 3);
    const int t = min(tok0 + r, T - 1);  // rows past T are computed and dropped
    aoff[j] = ((uint32_t)t * (uint32_t)d + gt_slot(r, lane & 7) * 8) * 2u;
  }
  uint32_t boff[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int r = (wave * NF + j) * 8 + (lane >> 3);
    boff[j] = ((uint32_t)(r < E ? r : min(r - E, E - 1)) * (uint32_t)d + gt_slot(r, lane & 7) * 8) * 2u;
  }
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds_u32 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
  // DMA instruction U (0..VPS-1) of K step KTI: U < AV are h rows, the rest router rows
#define GT_COPY(KTI, U)                                                                            \
  {                                                                                                \
    const int kti_ = (KTI);                                                                        \
    const uint32_t st_ = lds_u32 + (uint32_t)((kti_ % S) * STAGE) * 2u;                            \
    if ((U) < AV) {                                                                                \
      const int ja_ = (U) < AV ? (U) : 0;                                                          \
      gt_copy16(aoff[ja_], h + (size_t)kti_ * BK, st_ + (uint32_t)((wave_s * AV + ja_) * 8 * BK) * 2u); \
    } else {                                                                                       \
      const int jb_ = (U) >= AV ? (U) - AV : 0;                                                    \
      const uint16_t* m_ = (w_next == nullptr || (wave_s * NF + jb_) * 8 < E) ? w_cur : w_next;      \
      gt_copy16(boff[jb_], m_ + (size_t)kti_ * BK,                                                 \
                st_ + (uint32_t)((BM + (wave_s * NF + jb_) * 8) * BK) * 2u);                       \
    }                                                                                              \
  }

  // fragment rows are (multiple of 16) + (lane % 16): one lane term per 32-wide k sub-step
  const int fr = lane & 15;
  const int swz = ((fr >> 1) ^ (fr << 2)) & 7;
  int kofs[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) kofs[ks] = fr * BK + (((ks * 4 + (lane >> 4)) ^ swz) * 8);
  const int arow0 = wm * (BM / 2) * BK;
  const int brow0 = (BM + wn * NF * 16) * BK;

  f32x4_t acc[MI][NF];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NF; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bf16x8_t xa[MI], xb[NF], ya[MI], yb[NF];
  // refill of a freed stage: instructions [0, H1) right after the barrier that
  // frees it, [H1, VPS) during the next step's first sub-step (two stages: all
  // at once, it is needed one step later)
  constexpr int H1 = S >= 3 ? (VPS + 1) / 2 : VPS;
  constexpr int BPM = (NF + MI - 1) / MI;  // router fragments read per 16-row block
  // One 32-wide k sub-step: per 16-row block mi, read the next set's fragments
  // (sub-step KS of stage RS, if RD), run the block's NF MFMAs on the current
  // set, and issue a share of DMA instructions [P0, P1) of K step KI (if DO).
#define GT_SUB(FA, FB, NA, NB, RS, KS, RD, DO, KI, P0, P1)                                         \
  _Pragma("unroll") for (int mi = 0; mi < MI; ++mi) {                                              \
    if (RD) {                                                                                      \
      const uint16_t* rs_ = (RS);                                                                  \
      NA[mi] = *reinterpret_cast<const bf16x8_t*>(rs_ + arow0 + mi * 16 * BK + kofs[KS]);          \
      _Pragma("unroll") for (int q = 0; q < BPM; ++q) {                                            \
        const int i_ = mi * BPM + q;                                                               \
        if (i_ < NF) NB[i_] = *reinterpret_cast<const bf16x8_t*>(rs_ + brow0 + i_ * 16 * BK + kofs[KS]); \
      }                                                                                            \
    }                                                                                              \
    _Pragma("unroll") for (int ni = 0; ni < NF; ++ni)                                              \
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(FA[mi], FB[ni], acc[mi][ni], 0, 0, 0); \
    if (DO) {                                                                                      \
      constexpr int per_ = ((P1) - (P0) + MI - 1) / MI;                                            \
      _Pragma("unroll") for (int q = 0; q < per_; ++q) {                                           \
        const int u_ = (P0) + mi * per_ + q;                                                       \
        if (u_ < (P1)) GT_COPY(KI, u_)                                                             \
      }                                                                                            \
    }                                                                                              \
    __builtin_amdgcn_sched_barrier(0);                                                             \
  }

  // this lane's logit biases, fetched now so the latency hides behind the K loop
  float bias[NF];
#pragma unroll
  for (int ni = 0; ni < NF; ++ni) {
    const int col = wn * NF * 16 + ni * 16 + (lane & 15);
    bias[ni] = col < E ? b_cur[col] : (b_next ? b_next[col - E] : 0.f);
  }
  // scalar loads still in flight would turn every LDS wait of the loop into a full drain
  asm volatile("" ::"s"(idx), "s"(wts), "s"(idx_next), "s"(gap));
  for (int t = 0; t < S; ++t)
    if (t < KT) {
#pragma unroll
      for (int u = 0; u < VPS; ++u) GT_COPY(t, u)
    }
  {
    const int after = min(S, KT) - 1;  // steps issued after step 0
    if (after >= 3)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * VPS) : "memory");
    else if (after == 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * VPS) : "memory");
    else if (after == 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VPS) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) xa[i] = *reinterpret_cast<const bf16x8_t*>(lds + arow0 + i * 16 * BK + kofs[0]);
#pragma unroll
  for (int i = 0; i < NF; ++i) xb[i] = *reinterpret_cast<const bf16x8_t*>(lds + brow0 + i * 16 * BK + kofs[0]);
  // One K step.  P2: second part of the refill of the stage freed one step
  // ago (during the first sub-step); MORE: a step follows -- wait until it
  // landed (the AHEAD steps issued after it, all of their instructions issued
  // by now, may still be in flight; lgkmcnt(0): this wave's reads of step kt
  // are done before its stage is refilled), barrier; R2: first part of the
  // refill of step kt's stage with step kt+S (during the second sub-step).
  // The steady steps run with literal flags, so their body has no branch.
#define GT_STEP(P2, MORE, R2, AHEAD)                                                               \
  {                                                                                                \
    GT_SUB(xa, xb, ya, yb, lds + (kt % S) * STAGE, 1, true, (P2), kt - 1 + S, H1, VPS)             \
    if (MORE) {                                                                                    \
      const int ahead_ = (AHEAD);                                                                  \
      if (ahead_ >= 2)                                                                             \
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * VPS) : "memory");                   \
      else if (ahead_ == 1)                                                                        \
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(VPS) : "memory");                       \
      else                                                                                         \
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");                                \
      __builtin_amdgcn_s_barrier();                                                                \
      asm volatile("" ::: "memory");                                                               \
    }                                                                                              \
    GT_SUB(ya, yb, xa, xb, lds + ((kt + 1) % S) * STAGE, 0, (MORE), (R2), kt + S, 0, H1)           \
  }
#define GT_STEP_ANY                                                                                \
  GT_STEP(S >= 3 && kt >= 1 && kt - 1 + S < KT, kt + 1 < KT, kt + 1 < KT && kt + S < KT,          \
          min(S - 2, KT - 2 - kt))
  int kt = 0;
  GT_STEP_ANY
  // steps 1 .. KT-S-1: every refill issued, S-2 steps in flight at the wait
  for (kt = 1; kt + S < KT; ++kt) GT_STEP(S >= 3, true, true, S - 2)
  for (; kt < KT; ++kt) GT_STEP_ANY
#undef GT_STEP_ANY
#undef GT_STEP
#undef GT_COPY
#undef GT_SUB
  __syncthreads();  // LDS is reused for the logits

  const int colbase = wn * NF * 16;
  const int dirs = has_next ? 2 : 1;
  if constexpr (ONE_PASS) {
    // all BM tokens' logits fit in LDS: one selection pass
#pragma unroll
    for (int ni = 0; ni < NF; ++ni) {
      const int col = colbase + ni * 16 + (lane & 15);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = wm * (BM / 2) + mi * 16 + (lane >> 4) * 4 + i;
          Z[r * zstride + col] = acc[mi][ni][i] + bias[ni];
        }
    }
    __syncthreads();
    const int ntok = min(BM, T - tok0);
    topk_epilogue<KL>(Z, zstride, ntok, GATE_THREADS / (BM * dirs), tok0, T, E, k, has_next, idx, wts, gap,
                      idx_next);
  } else {
    for (int half = 0; half < 2; ++half) {
      if (wm == half) {
#pragma unroll
        for (int ni = 0; ni < NF; ++ni) {
          const int col = colbase + ni * 16 + (lane & 15);
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = mi * 16 + (lane >> 4) * 4 + i;
              Z[r * zstride + col] = acc[mi][ni][i] + bias[ni];
            }
        }
      }
      __syncthreads();
      const int t0 = tok0 + half * (BM / 2);
      const int ntok = min(BM / 2, T - t0);
      if (ntok > 0)
        topk_epilogue<KL>(Z, zstride, ntok, GATE_THREADS / ((BM / 2) * dirs), t0, T, E, k, has_next, idx, wts, gap,
                          idx_next);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- fp32 kernel

template <int KL>
__global__ __launch_bounds__(GATE_THREADS) void gate_topk_f32_kernel(
    const float* __restrict__ h, int T, int d, int E, int k, const float* __restrict__ w_cur,
    const float* __restrict__ b_cur, const float* __restrict__ w_next, const float* __restrict__ b_next,
    int32_t* __restrict__ idx, float* __restrict__ wts, float* __restrict__ gap, int32_t* __restrict__ idx_next,
    int zstride) {
  extern __shared__ __align__(16) char smem[];
  float* Z = reinterpret_cast<float*>(smem);  // [64][zstride]
  const int tok0 = blockIdx.x * 64;
  const bool has_next = w_next != nullptr;
  const int N = has_next ? 2 * E : E;
  const int ntok = min(64, T - tok0);
  for (int o = threadIdx.x; o < 64 * N; o += blockDim.x) {
    const int tl = o / N, col = o % N;
    if (tl >= ntok) continue;
    const float* hr = h + (size_t)(tok0 + tl) * d;
    const float* wr = col < E ? w_cur + (size_t)col * d : w_next + (size_t)(col - E) * d;
    float s = 0.f;
    for (int kk = 0; kk < d; kk += 4) {
      const float4 a = *reinterpret_cast<const float4*>(hr + kk);
      const float4 b = *reinterpret_cast<const float4*>(wr + kk);
      s = fmaf(a.x, b.x, s);
      s = fmaf(a.y, b.y, s);
      s = fmaf(a.z, b.z, s);
      s = fmaf(a.w, b.w, s);
    }
    Z[tl * zstride + col] = s + (col < E ? b_cur[col] : b_next[col - E]);
  }
  __syncthreads();
  topk_epilogue<KL>(Z, zstride, ntok, has_next ? 4 : 8, tok0, T, E, k, has_next, idx, wts, gap, idx_next);
}

int zstride_for(int N) { return ((N + 63) / 64) * 64 + 4; }

int compute_units() { return moelb_compute_units(); }

template <int KL>
int launch_bf16(int NF, const void* h, int T, int d, int E, int k, const void* w_cur, const float* b_cur,
                const void* w_next, const float* b_next, int32_t* idx, float* wts, float* gap,
                int32_t* idx_next, hipStream_t s) {
  const int N = w_next ? 2 * E : E;
  const int zs = zstride_for(N);
  const size_t lds_a = 2ull * GATE_BM * A_STRIDE * 2;
  const size_t lds_z = 64ull * zs * 4;
  const size_t lds = lds_a > lds_z ? lds_a : lds_z;
  const dim3 grid((T + GATE_BM - 1) / GATE_BM);
  const auto* hh = static_cast<const uint16_t*>(h);
  const auto* wc = static_cast<const uint16_t*>(w_cur);
  const auto* wx = static_cast<const uint16_t*>(w_next);
#define MOELB_GATE_CASE(nf)                                                                        \
  case nf:                                                                                         \
    if (!moelb_allow_lds(gate_topk_bf16_kernel<nf, KL>, lds)) return MOELB_ELAUNCH;                \
    hipLaunchKernelGGL((gate_topk_bf16_kernel<nf, KL>), grid, dim3(GATE_THREADS), lds, s, hh, T, d, E, k, \
                       wc, b_cur, wx, b_next, idx, wts, gap, idx_next, zs);                        \
    break;
  switch (NF) {
    MOELB_GATE_CASE(1)
    MOELB_GATE_CASE(2)
    MOELB_GATE_CASE(3)
    MOELB_GATE_CASE(4)
    MOELB_GATE_CASE(5)
    MOELB_GATE_CASE(6)
    MOELB_GATE_CASE(7)
    MOELB_GATE_CASE(8)
    default:
      return MOELB_EINVAL;
  }
#undef MOELB_GATE_CASE
  MOELB_CHECK_LAUNCH();
  return MOELB_OK;
}

template <int NF, int KL, int S, int BM>
int launch_dma_nf(const void* h, int T, int d, int E, int k, const void* w_cur, const float* b_cur, const void* w_next,
                  const float* b_next, int32_t* idx, float* wts, float* gap, int32_t* idx_next, bool split,
                  hipStream_t s) {
  const int N = 64 * NF;
  const int zs = zstride_for(N);
  const size_t lds_main = (size_t)S * (BM + N) * 64 * 2;
  const size_t lds_z = 64ull * zs * 4;
  const size_t lds = lds_main > lds_z ? lds_main : lds_z;
  if (!moelb_allow_lds(gate_topk_dma_kernel<NF, KL, S, BM>, lds)) return MOELB_ELAUNCH;
  hipLaunchKernelGGL((gate_topk_dma_kernel<NF, KL, S, BM>), dim3((T + BM - 1) / BM, split ? 2 : 1),
                     dim3(GATE_THREADS), lds, s,
                     static_cast<const uint16_t*>(h), T, d, E, k, static_cast<const uint16_t*>(w_cur), b_cur,
                     static_cast<const uint16_t*>(w_next), b_next, idx, wts, gap, idx_next, zs);
  MOELB_CHECK_LAUNCH();
  return MOELB_OK;
}

// Direct-to-LDS variant: N = 64 * NF columns (NF <= 7), d % 64 == 0; 64-token
// blocks (half64) for NF <= 4 only.
template <int KL>
int launch_dma(int NF, bool half64, const void* h, int T, int d, int E, int k, const void* w_cur, const float* b_cur,
               const void* w_next, const float* b_next, int32_t* idx, float* wts, float* gap, int32_t* idx_next,
               bool split, hipStream_t s) {
#define MOELB_DMA(nf, st, bm) \
  return launch_dma_nf<nf, KL, st, bm>(h, T, d, E, k, w_cur, b_cur, w_next, b_next, idx, wts, gap, idx_next, split, s)
  if (half64) {
    switch (NF) {
      case 1: MOELB_DMA(1, 3, 64);
      case 2: MOELB_DMA(2, 3, 64);
      case 3: MOELB_DMA(3, 3, 64);
      case 4: MOELB_DMA(4, 3, 64);
      default: return MOELB_EINVAL;
    }
  }
  switch (NF) {
    // (a four-stage ring for N <= 192, three steps ahead, measured no faster
    // on the decode, GLM-4.5 and OLMoE shapes; four waves of 64 x N/2 tiles,
    // a quarter fewer fragment reads, slower on every shape: 113-117 against
    // 99-110 us on Qwen3-235B's, 120 against 91 on GLM-4.5's)
    case 1: MOELB_DMA(1, 3, 128);
    case 2: MOELB_DMA(2, 3, 128);
    case 3: MOELB_DMA(3, 3, 128);
    case 4: MOELB_DMA(4, 3, 128);
    case 5: MOELB_DMA(5, 2, 128);
    case 6: MOELB_DMA(6, 2, 128);
    case 7: MOELB_DMA(7, 2, 128);
    default: return MOELB_EINVAL;
  }
#undef MOELB_DMA
}

template <int KL>
int launch_f32(const void* h, int T, int d, int E, int k, const void* w_cur, const float* b_cur,
               const void* w_next, const float* b_next, int32_t* idx, float* wts, float* gap,
               int32_t* idx_next, hipStream_t s) {
  const int N = w_next ? 2 * E : E;
  const int zs = zstride_for(N);
  const size_t lds = 64ull * zs * 4;
  if (!moelb_allow_lds(gate_topk_f32_kernel<KL>, lds)) return MOELB_ELAUNCH;
  hipLaunchKernelGGL((gate_topk_f32_kernel<KL>), dim3((T + 63) / 64), dim3(GATE_THREADS), lds, s,
                     static_cast<const float*>(h), T, d, E, k, static_cast<const float*>(w_cur), b_cur,
                     static_cast<const float*>(w_next), b_next, idx, wts, gap, idx_next, zs);
  MOELB_CHECK_LAUNCH();
  return MOELB_OK;
}

}  // namespace

extern "C" int moelb_gate_topk(const void* h, int T, int d, int E, int k, int dtype, const void* w_cur,
                               const float* b_cur, const void* w_next, const float* b_next, int32_t* idx,
                               float* wts, float* gap, int32_t* idx_next, void* stream) {
  if (T < 0 || d <= 0 || d % 8 != 0 || E < 1 || E > MOELB_MAX_E || k < 1 || k > MOELB_MAX_K || k > E)
    return MOELB_EINVAL;
  if (!moelb_dtype_ok(dtype)) return MOELB_EINVAL;
  if (!w_cur || !b_cur || (w_next == nullptr) != (b_next == nullptr)) return MOELB_EINVAL;
  if (T > 0 && (!h || !idx || !wts || (w_next == nullptr) != (idx_next == nullptr))) return MOELB_EINVAL;
  if ((reinterpret_cast<uintptr_t>(h) | reinterpret_cast<uintptr_t>(w_cur) |
       reinterpret_cast<uintptr_t>(w_next)) & 15)
    return MOELB_EINVAL;
  if (T == 0) return MOELB_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == MOELB_BF16) {
    const int N = w_next ? 2 * E : E;
    const int NF = (N + 63) / 64;
    const int nfmax = k <= 8 ? 7 : 6;
    const bool dma_ok = d % 64 == 0 && (size_t)T * d * 2 < (1ull << 32);
    // few token blocks: one workgroup per router and block (twice the
    // workgroups, each reading half the router rows)
    const int blocks = (T + GATE_BM - 1) / GATE_BM;
    const int NFs = (E + 63) / 64;
    const bool split = w_next && dma_ok && NFs <= nfmax && 2 * blocks <= compute_units();
    const bool fused = dma_ok && N % 64 == 0 && NF <= nfmax;
    if (split || fused) {
      const int nf = split ? NFs : NF;
      // still fewer workgroups than CUs with 64-token blocks: take them (half
      // the h rows and MFMAs per workgroup; the router rows are read as before)
      const bool half64 = nf <= 4 && (split ? 2 : 1) * ((T + 63) / 64) <= compute_units();
      if (k <= 2) return launch_dma<4>(nf, half64, h, T, d, E, k, w_cur, b_cur, w_next, b_next, idx, wts, gap, idx_next, split, s);
      if (k <= 4) return launch_dma<6>(nf, half64, h, T, d, E, k, w_cur, b_cur, w_next, b_next, idx, wts, gap, idx_next, split, s);
      if (k <= 8) return launch_dma<10>(nf, half64, h, T, d, E, k, w_cur, b_cur, w_next, b_next, idx, wts, gap, idx_next, split, s);
      return launch_dma<18>(nf, half64, h, T, d, E, k, w_cur, b_cur, w_next, b_next, idx, wts, gap, idx_next, split, s);
    }
    if (k <= 2) return launch_bf16<4>(NF, h, T, d, E, k, w_cur, b_cur, w_next, b_next, idx, wts, gap, idx_next, s);
    if (k <= 4) return launch_bf16<6>(NF, h, T, d, E, k, w_cur, b_cur, w_next, b_next, idx, wts, gap, idx_next, s);
    if (k <= 8) return launch_bf16<10>(NF, h, T, d, E, k, w_cur, b_cur, w_next, b_next, idx, wts, gap, idx_next, s);
    return launch_bf16<18>(NF, h, T, d, E, k, w_cur, b_cur, w_next, b_next, idx, wts, gap, idx_next, s);
  }
  if (k <= 2) return launch_f32<4>(h, T, d, E, k, w_cur, b_cur, w_next, b_next, idx, wts, gap, idx_next, s);
  if (k <= 4) return launch_f32<6>(h, T, d, E, k, w_cur, b_cur, w_next, b_next, idx, wts, gap, idx_next, s);
  if (k <= 8) return launch_f32<10>(h, T, d, E, k, w_cur, b_cur, w_next, b_next, idx, wts, gap, idx_next, s);
  return launch_f32<18>(h, T, d, E, k, w_cur, b_cur, w_next, b_next, idx, wts, gap, idx_next, s);
}
