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
// stored values and one float32 reciprocal: code = clamp(rint((x - z) * (1/s)), 0, 2^b-1).
// A zero or non-finite scale gives all-zero codes.
//
// Both quotients are the correctly rounded float32 results, taken without a
// division sequence:
//   (hi - lo) / qmax as q0 = (hi - lo) * c with c = 1/qmax rounded, then one
//   correction with its exact remainder: q0 + fma(-q0, qmax, hi - lo) * c;
//   1/s as the hardware reciprocal estimate r0 corrected by one Newton step,
//   r0 + fma(-s, r0, 1) * r0.
// Checked exhaustively against IEEE division: the first for qmax = 3 and 15 and
// every finite hi - lo >= 0; the second for every positive finite fp16 s with
// r0 anywhere within 2 ulp of 1/s.
struct GroupQ {
  float z;
  float inv;
  uint32_t meta;  // scale bits | zero bits << 16
  bool ok;
};

__device__ __forceinline__ GroupQ make_group(float lo, float hi, float qmax) {
  GroupQ g;
  const float d = __fsub_rn(hi, lo);
  const float c = 1.0f / qmax;  // a constant once qmax is
  const float q0 = __fmul_rn(d, c);
  const float sf = __builtin_isfinite(q0) ? __builtin_fmaf(__builtin_fmaf(-q0, qmax, d), c, q0) : q0;
  const uint32_t sb = f32_to_f16_bits(sf);
  const uint32_t zb = f32_to_f16_bits(lo);
  const float s = f16_bits_to_f32(sb);
  g.z = f16_bits_to_f32(zb);
  g.meta = sb | (zb << 16);
  g.ok = (s != 0.0f) && __builtin_isfinite(s);
  const float r0 = __builtin_amdgcn_rcpf(s);
  g.inv = g.ok ? __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0) : 0.0f;
  // the codes of such a group are (x - z) * 0 = 0; a zero of 0 there keeps an
  // infinite fp16 zero-point from making that product NaN (x is finite)
  if (!g.ok) g.z = 0.0f;
  return g;
}

}  // namespace kvc
