// Shared host/device helpers for libmdmp (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "mdmp.h"

namespace mdmp {

// thread-local error message behind mp_last_error()
void set_error(const std::string& msg);

#define MP_HIP(expr)                                                                 \
  do {                                                                               \
    hipError_t _e = (expr);                                                          \
    if (_e != hipSuccess) {                                                          \
      ::mdmp::set_error(std::string(#expr) + ": " + hipGetErrorString(_e));          \
      return MP_ERR_HIP;                                                             \
    }                                                                                \
  } while (0)

#define MP_TRY(expr)                \
  do {                              \
    int _s = (expr);                \
    if (_s != MP_OK) return _s;     \
  } while (0)

#define MP_CHECK_LAUNCH() MP_HIP(hipGetLastError())

inline int arg_error(const std::string& msg) {
  set_error(msg);
  return MP_ERR_ARG;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// bump allocator over a caller-provided workspace
struct Arena {
  char* base;
  size_t size, off;
  bool dry;  // dry run: only measure
  Arena(void* b, size_t s, bool d = false) : base((char*)b), size(s), off(0), dry(d) {}
  template <class T>
  T* take(int64_t count) {
    size_t bytes = align_up(sizeof(T) * (size_t)(count > 0 ? count : 1));
    T* p = dry ? nullptr : (T*)(base + off);
    off += bytes;
    return p;
  }
  bool ok() const { return dry || off <= size; }
};

// ---------------------------------------------------------------- device helpers
// Work-groups reach the 8 XCDs (each with its own L2) round-robin in launch order.
// xcd_order() maps launch index b of `total` work-groups to a logical index such that
// each XCD walks consecutive chunks of `chunk` logical indices, chunks alternating
// between XCDs; the tail past the last full round keeps its launch order.
__device__ __forceinline__ int64_t xcd_order(int64_t b, int64_t total, int64_t chunk) {
  constexpr int64_t kX = 8;
  const int64_t full = total / (kX * chunk) * (kX * chunk);
  if (b >= full) return b;
  const int64_t x = b % kX, k = b / kX;
  return ((k / chunk) * kX + x) * chunk + k % chunk;
}

// logistic function with the hardware reciprocal (v_rcp_f32, 1 ulp) instead of an
// IEEE division; 1 + exp(-x) = inf gives 0
__device__ __forceinline__ float sigm(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float silu(float x) { return x * sigm(x); }
// d/dx silu = s (1 + x (1 - s)), s = sigmoid(x)
__device__ __forceinline__ float dsilu(float x) {
  float s = sigm(x);
  return s * (1.0f + x * (1.0f - s));
}

// bf16 storage as raw 16-bit, round to nearest even
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
// float -> bf16 bits, round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two floats -> packed bf16 pair (a in the low half), one v_cvt_pk_bf16_f32, same rounding
typedef float f2v_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk2bf(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2v_t{a, b}, bf2v_t));
}

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(uint16_t v) { return bf2f(v); }

template <class T>
struct FeatIO;
template <>
struct FeatIO<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <>
struct FeatIO<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(uint16_t* p, float v) { *p = f2bf(v); }
};

template <int W>
__device__ __forceinline__ float group_sum(float v) {
  // butterfly over aligned groups of W lanes (W a power of two <= 64)
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace mdmp
