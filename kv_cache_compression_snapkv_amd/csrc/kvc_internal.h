// Internal helpers shared by the kvc HIP kernels and the host glue.
// Not part of the public ABI (see include/kvc.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvc.h"

namespace kvc {

constexpr int kGroup = 32;  // default quantization group (tokens for keys, channels for values)

// The cache's group size: 32 (also for 0) or 16.
inline bool group_ok(int g) { return g == 0 || g == 16 || g == 32; }
inline int cache_group(const kvc_cache* c) { return c->group == 0 ? kGroup : c->group; }

// ---------------------------------------------------------------- host side
void set_last_hip_error(hipError_t e);
// Returns KVC_OK or KVC_ERR_HIP after checking hipGetLastError().
kvc_status check_launch();

inline bool dtype_ok(kvc_dtype d) { return d == KVC_F32 || d == KVC_BF16; }
inline bool head_dim_ok(int D) { return D >= 32 && D <= 256 && D % 32 == 0; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// n / d and n % d for 0 <= n < 2^22, d >= 1, from rcp within a few ulps of 1/d:
// the truncated float quotient is off by at most one, which the remainder test
// corrects (cheaper than an integer division by a runtime divisor).
struct QR {
  int q, r;
};
__device__ __forceinline__ QR small_divmod(int n, int d, float rcp) {
  int q = static_cast<int>(static_cast<float>(n) * rcp);
  int r = n - q * d;
  if (r < 0) {
    --q;
    r += d;
  } else if (r >= d) {
    ++q;
    r -= d;
  }
  return QR{q, r};
}

// ---------------------------------------------------------------- number formats
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// float32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = static_cast<_Float16>(x);  // v_cvt_f16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

// Load element i of a model-dtype tensor as float32.
template <typename T> __device__ __forceinline__ float load_f32(const T* p, size_t i);
template <> __device__ __forceinline__ float load_f32<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_f32<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}

// ---------------------------------------------------------------- group quantizer
// One group's parameters: fp16 scale and zero-point, rounded first; codes use the
// stored values and one IEEE reciprocal: code = clamp(rint((x - z) * (1/s)), 0, 2^b-1).
// A zero or non-finite scale gives all-zero codes.
struct GroupQ {
  float z;
  float inv;
  uint32_t meta;  // scale bits | zero bits << 16
  bool ok;
};

__device__ __forceinline__ GroupQ make_group(float lo, float hi, float qmax) {
  GroupQ g;
  const float sf = __fdiv_rn(hi - lo, qmax);
  const uint32_t sb = f32_to_f16_bits(sf);
  const uint32_t zb = f32_to_f16_bits(lo);
  const float s = f16_bits_to_f32(sb);
  g.z = f16_bits_to_f32(zb);
  g.meta = sb | (zb << 16);
  g.ok = (s != 0.0f) && __builtin_isfinite(s);
  g.inv = g.ok ? __fdiv_rn(1.0f, s) : 0.0f;
  return g;
}

__device__ __forceinline__ uint32_t code_of(float x, float z, float inv, bool ok, float qmax) {
  if (!ok) return 0u;
  const float t = __fmul_rn(__fsub_rn(x, z), inv);
  const float r = fminf(fmaxf(__builtin_rintf(t), 0.0f), qmax);
  return static_cast<uint32_t>(r);
}

}  // namespace kvc
