// Shared device helpers for the moelb kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <utility>
#include <vector>

#include "moelb.h"

#define MOELB_WAVE 64

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- bf16 <-> fp32

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even.  NaN stays NaN.  Branch-free (one compare
// and a select), so unrolled epilogues stay straight-line code.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x40u;
  return static_cast<uint16_t>(((u & 0x7fffffffu) > 0x7f800000u) ? quiet : rounded);
}

// Two floats to packed bf16 (lo in bits 0..15), rounded to nearest even by the
// hardware conversion (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16x2_pack(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// 16-byte non-temporal store and load: for streams much larger than the
// caches that are written or read exactly once (the hint keeps them from
// evicting reusable lines).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt16(void* p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// SiLU(z) = z / (1 + e^-z) with the hardware exponential and reciprocal (each
// within about one ulp); the IEEE division sequence would cost ten instructions.
__device__ __forceinline__ float silu_f32(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & (MOELB_WAVE - 1); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOELB_WAVE);
  return v;
}

// ---------------------------------------------------------------- host helpers

#define MOELB_CHECK_LAUNCH()                                   \
  do {                                                         \
    if (hipGetLastError() != hipSuccess) return MOELB_ELAUNCH; \
  } while (0)

static inline size_t moelb_align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }
static inline bool moelb_dtype_ok(int dtype) { return dtype == MOELB_F32 || dtype == MOELB_BF16; }
static inline size_t moelb_elem_bytes(int dtype) { return dtype == MOELB_F32 ? 4 : 2; }

// Compute units of the current device, queried once per device (so a launch
// recorded by stream capture makes no device query); 256 if the query fails.
static inline int moelb_compute_units() {
  static std::mutex mu;
  static std::vector<std::pair<int, int>> known;  // (device, compute units)
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& x : known)
    if (x.first == dev) return x.second;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  known.emplace_back(dev, cus);
  return cus;
}

// Kernels that use more than 64 KiB of dynamic LDS must opt in (gfx950 has 160
// KiB per CU).  The attribute is set once per kernel, size and device and
// remembered, so later launches -- including ones recorded by stream capture
// into a graph -- make no attribute call.
template <typename Kern>
static inline bool moelb_allow_lds(Kern kernel, size_t bytes) {
  if (bytes <= 65536) return true;
  struct Done {
    const void* fn;
    size_t bytes;
    int dev;
  };
  static std::mutex mu;
  static std::vector<Done> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const void* fn = reinterpret_cast<const void*>(kernel);
  std::lock_guard<std::mutex> lock(mu);
  for (const Done& x : done)
    if (x.fn == fn && x.dev == dev && x.bytes >= bytes) return true;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes)) != hipSuccess)
    return false;
  done.push_back({fn, bytes, dev});
  return true;
}
