// Internal helpers of the HIP library (never included by anything outside
// csrc/). Error state, argument checks and small device utilities.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "nestspec.h"

namespace nest {

// Per-thread message behind nest_last_error().
std::string& last_error();

// Record a formatted message and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clear the message and return NEST_OK.
int ok();

// Check hipGetLastError() after a launch. Returns NEST_OK or NEST_EHIP.
int check_launch(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr int kWave = 64;

}  // namespace nest

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Wave-wide maximum of a float (all 64 lanes end with the result).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Wave-wide sum of a float (butterfly order, all lanes end with the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

namespace nest {
// 16-byte load with the nontemporal hint, for data that one call streams
// through once (weight planes and scales, KV planes): on MI355X a streaming
// read with the hint sustains ~7.0 TB/s against ~6.3 TB/s without it.
typedef unsigned nt_u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldnt16(const void* p) {
  const nt_u4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ldnt_f4(const void* p) {
  const uint4 v = ldnt16(p);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
}  // namespace nest

// Orderable 64-bit argmax key: larger value first, then the lower index.
// -0 is folded to +0 so that equal values tie on the index.
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t idx) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7fffffffu) == 0) b = 0;
  uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<unsigned long long>(ord) << 32) | static_cast<unsigned long long>(0xffffffffu - idx);
}

__device__ __forceinline__ uint32_t argmax_key_index(unsigned long long key) {
  return 0xffffffffu - static_cast<uint32_t>(key & 0xffffffffull);
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int o) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  lo = __shfl_xor(lo, o, 64);
  hi = __shfl_xor(hi, o, 64);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// clamp(rint(x / s), -127, 127) with x / s the IEEE quotient, computed as
// t = x * r with r = 1/s (itself correctly rounded). |x / s| <= 127(1 + 2^-23),
// so |t - x/s| and |fl(x/s) - x/s| are both below 1.6e-5. When t is more
// than 3e-5 away from the nearest half-integer, t, x/s and fl(x/s) lie on
// the same side of it and round alike. Only near a tie is the quotient
// formed exactly. s == 0 gives 0; an r that overflows takes the exact path.
__device__ __forceinline__ int quant_act(float x, float s, float r) {
  if (s == 0.0f) return 0;
  const float t = x * r;
  float q;
  if (fabsf(t - floorf(t) - 0.5f) > 3.0e-5f && r < INFINITY)
    q = rintf(t);
  else
    q = rintf(x / s);
  q = q < -127.0f ? -127.0f : (q > 127.0f ? 127.0f : q);
  return static_cast<int>(q);
}
