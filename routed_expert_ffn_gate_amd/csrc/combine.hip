// Top-k weighted combine of expert outputs (+ an always-on shared expert).
//
// Definition: FreeBalance ("FreeBalance: Pre-Routing Online MoE Load Balancing
// via Residual Workload Prediction") section 2.1: MoE(h) = sum_i W_i
// expert_i(h); Libra README "Repository Layout": the combine kernel.
//
// HBM-bound gather-reduce: one workgroup per token (grid-stride), each thread
// owns 16-byte column chunks of the row; the k expert rows are fetched with
// all loads of a chunk issued before the fp32 accumulation (j ascending, so
// the summation order is fixed), then rounded once to the storage type.
#include "common.h"

namespace {

constexpr int CMB_THREADS = 256;

template <typename T> struct Vec;
template <> struct Vec<uint16_t> {
  static constexpr int n = 8;
  static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    return make_uint4(bf16x2_pack(f[0], f[1]), bf16x2_pack(f[2], f[3]), bf16x2_pack(f[4], f[5]),
                      bf16x2_pack(f[6], f[7]));
  }
};
template <> struct Vec<float> {
  static constexpr int n = 4;
  static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};

template <typename T, int KMAX>
__global__ __launch_bounds__(CMB_THREADS) void combine_kernel(const T* __restrict__ y, int rows_y,
                                                              const int32_t* __restrict__ pos,
                                                              const float* __restrict__ wts, int Ttok, int k, int d,
                                                              const T* __restrict__ shared, T* __restrict__ out) {
  constexpr int VN = Vec<T>::n;
  const int nvec = d / VN;
  for (int t = blockIdx.x; t < Ttok; t += gridDim.x) {
    int q[KMAX];
    float wt[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      q[j] = -1;
      wt[j] = 0.f;
      if (j < k) {
        const int p = pos[(size_t)t * k + j];
        q[j] = (p >= 0 && p < rows_y) ? p : -1;
        wt[j] = wts[(size_t)t * k + j];
      }
    }
    for (int v = threadIdx.x; v < nvec; v += CMB_THREADS) {
      // Y rows are read once (non-temporal: 0.48 -> 0.42 ms at T = 32768,
      // d = 4096, k = 8, with the FFN's Y stores non-temporal too)
      uint4 raw[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        raw[j] = q[j] >= 0 ? load_nt16(reinterpret_cast<const uint4*>(y + (size_t)q[j] * d) + v) : make_uint4(0, 0, 0, 0);
      float acc[VN];
#pragma unroll
      for (int i = 0; i < VN; ++i) acc[i] = 0.f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (q[j] < 0) continue;
        float f[VN];
        Vec<T>::unpack(raw[j], f);
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] = fmaf(wt[j], f[i], acc[i]);
      }
      if (shared) {
        float f[VN];
        Vec<T>::unpack(reinterpret_cast<const uint4*>(shared + (size_t)t * d)[v], f);
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] += f[i];
      }
      reinterpret_cast<uint4*>(out + (size_t)t * d)[v] = Vec<T>::pack(acc);
    }
  }
}

template <typename T>
int launch(const void* y, int rows_y, const int32_t* pos, const float* wts, int Ttok, int k, int d,
           const void* shared, void* out, hipStream_t s) {
  const dim3 grid(Ttok < 65536 ? Ttok : 65536);
  const auto* yy = static_cast<const T*>(y);
  const auto* sh = static_cast<const T*>(shared);
  auto* o = static_cast<T*>(out);
  if (k <= 2)
    hipLaunchKernelGGL((combine_kernel<T, 2>), grid, dim3(CMB_THREADS), 0, s, yy, rows_y, pos, wts, Ttok, k, d, sh, o);
  else if (k <= 4)
    hipLaunchKernelGGL((combine_kernel<T, 4>), grid, dim3(CMB_THREADS), 0, s, yy, rows_y, pos, wts, Ttok, k, d, sh, o);
  else if (k <= 8)
    hipLaunchKernelGGL((combine_kernel<T, 8>), grid, dim3(CMB_THREADS), 0, s, yy, rows_y, pos, wts, Ttok, k, d, sh, o);
  else
    hipLaunchKernelGGL((combine_kernel<T, 16>), grid, dim3(CMB_THREADS), 0, s, yy, rows_y, pos, wts, Ttok, k, d, sh, o);
  MOELB_CHECK_LAUNCH();
  return MOELB_OK;
}

}  // namespace

extern "C" int moelb_combine(const void* y, int rows_y, const int32_t* pos, const float* wts, int T, int k, int d,
                             int dtype, const void* shared, void* out, void* stream) {
  if (T < 0 || rows_y < 0 || k < 1 || k > MOELB_MAX_K || d <= 0 || d % 8 != 0 || !moelb_dtype_ok(dtype))
    return MOELB_EINVAL;
  if (T > 0 && (!pos || !wts || !out)) return MOELB_EINVAL;
  if (rows_y > 0 && !y) return MOELB_EINVAL;
  if ((reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(shared) | reinterpret_cast<uintptr_t>(out)) & 15)
    return MOELB_EINVAL;
  if (T == 0) return MOELB_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == MOELB_BF16) return launch<uint16_t>(y, rows_y, pos, wts, T, k, d, shared, out, s);
  return launch<float>(y, rows_y, pos, wts, T, k, d, shared, out, s);
}

extern "C" int moelb_version(void) { return 100; }  // 0.1.0

extern "C" const char* moelb_status_string(int status) {
  switch (status) {
    case MOELB_OK:
      return "ok";
    case MOELB_EINVAL:
      return "invalid argument";
    case MOELB_ELAUNCH:
      return "kernel launch or runtime call failed";
    case MOELB_EWORKSPACE:
      return "workspace missing or too small";
    default:
      return "unknown status";
  }
}
