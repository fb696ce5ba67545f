// Single-query decode attention over the compressed cache (MiniKV Eq. 1 and
// Alg. 1 decoding; blog attention hook: one softmax over exact recent tokens
// and dequantized older ones; query head h reads KV head h / G).
//
// Split-K: workgroup (s, j, b) owns a range of packed-history tokens of KV head
// j (or, for the last split, the bf16 residual plus the appended token) and all
// G query heads that read it, so every cache byte is read once.  Each split
// keeps a running max m, sum l and unnormalized output o per head (online
// softmax in log2 units); a second kernel merges the splits:
// M = max m_s, o = sum_s 2^(m_s-M) o_s / sum_s 2^(m_s-M) l_s.
#include <algorithm>

#include "kvc_internal.h"

namespace kvc {

kvc_status launch_flush(const kvc_cache* c, const void* k_new, const void* v_new, kvc_dtype dt,
                        hipStream_t st);
bool cache_ok(const kvc_cache* c);
kvc_status cache_shape_status(const kvc_cache* c);

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;   // tokens per tile
constexpr int kGMax = 16;   // query heads per KV head
constexpr int kMaxD = 256;
constexpr int kTargetBlocks = 2048;

struct AttnArgs {
  const void* q;
  const void* k_new;
  const void* v_new;
  const uint32_t *k_codes, *k_meta, *v_codes, *v_meta;
  uint16_t *k_res, *v_res;
  float* part_o;   // [B][Hkv][ns][G][D]
  float2* part_ml; // [B][Hkv][ns][G]
  int Hq, Hkv, G, D, q_cap, r_cap;
  int q_len;     // packed history tokens
  int r_total;   // residual tokens attended (including the appended one)
  int r_new;     // residual row of the appended token, or -1 if none
  int nsplit;    // history splits; split index nsplit is the residual
  int chunk;     // history tokens per split (multiple of kTile)
  float scale2;  // log2(e)/sqrt(D)
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <typename T, int BITS>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(AttnArgs a) {
  __shared__ float q_s[kGMax * kMaxD];
  __shared__ float2 kmeta_s[2 * kMaxD];
  __shared__ float2 vmeta_s[kTile * (kMaxD / kGroup)];
  __shared__ float p_s[kGMax * kTile];
  __shared__ float alpha_s[kGMax], m_s[kGMax], l_s[kGMax];
  __shared__ float red_s[kThreads * kGMax];

  constexpr int per = 32 / BITS;
  constexpr uint32_t mask = (1u << BITS) - 1u;
  const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int bj = b * a.Hkv + j;
  const int D = a.D, G = a.G, ngv = D / kGroup;
  const int tid = threadIdx.x;
  const bool resid = (s == a.nsplit);

  const T* qp = static_cast<const T*>(a.q) + static_cast<size_t>(b * a.Hq + j * G) * D;
  for (int e = tid; e < G * D; e += kThreads) q_s[e] = load_f32(qp, e);
  if (tid < G) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.0f;
  }
  const T* knp = static_cast<const T*>(a.k_new) + static_cast<size_t>(bj) * D;
  const T* vnp = static_cast<const T*>(a.v_new) + static_cast<size_t>(bj) * D;
  const uint16_t* kres = a.k_res + static_cast<size_t>(bj) * a.r_cap * D;
  const uint16_t* vres = a.v_res + static_cast<size_t>(bj) * a.r_cap * D;
  const size_t qc = a.q_cap;
  const uint32_t* kc = a.k_codes + static_cast<size_t>(bj) * qc * (D * BITS / 32);
  const uint32_t* km = a.k_meta + static_cast<size_t>(bj) * (qc / kGroup) * D;
  const uint32_t* vc = a.v_codes + static_cast<size_t>(bj) * (qc * BITS / 32) * D;
  const uint32_t* vm = a.v_meta + static_cast<size_t>(bj) * qc * ngv;

  int t_begin, t_end;
  if (resid) {
    t_begin = 0;
    t_end = a.r_total;
  } else {
    t_begin = s * a.chunk;
    t_end = min(a.q_len, t_begin + a.chunk);
  }

  const int P = kThreads / D;        // value-phase threads per channel
  const int vc_ch = tid % D, vpart = tid / D;
  float o[kGMax];
#pragma unroll
  for (int h = 0; h < kGMax; ++h) o[h] = 0.0f;
  __syncthreads();

  for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
    const int ntok = min(kTile, t_end - t0);
    if (!resid) {
      for (int e = tid; e < 2 * D; e += kThreads) {
        const int gi = e / D, c = e % D;
        if (gi * kGroup < ntok) {
          const uint32_t m = km[static_cast<size_t>(t0 / kGroup + gi) * D + c];
          kmeta_s[e] = make_float2(f16_bits_to_f32(m & 0xFFFFu), f16_bits_to_f32(m >> 16));
        }
      }
      for (int e = tid; e < kTile * ngv; e += kThreads) {
        const int t = e / ngv;
        if (t < ntok) {
          const uint32_t m = vm[static_cast<size_t>(t0) * ngv + e];
          vmeta_s[e] = make_float2(f16_bits_to_f32(m & 0xFFFFu), f16_bits_to_f32(m >> 16));
        }
      }
    }
    __syncthreads();
    // ---- scores: thread (token t, quarter of the channels)
    {
      const int t = tid >> 2, part = tid & 3;
      const int cpp = D / 4;
      const int c0 = part * cpp;
      float acc[kGMax];
#pragma unroll
      for (int h = 0; h < kGMax; ++h) acc[h] = 0.0f;
      if (t < ntok) {
        if (!resid) {
          const uint32_t* row = kc + static_cast<size_t>(t0 + t) * (D / per);
          const int gl = t / kGroup;
          uint32_t word = 0;
          for (int c = c0; c < c0 + cpp; ++c) {
            if (c == c0 || c % per == 0) word = row[c / per];
            const float code = static_cast<float>((word >> (BITS * (c % per))) & mask);
            const float2 sz = kmeta_s[gl * D + c];
            const float kh = fmaf(code, sz.x, sz.y);
#pragma unroll
            for (int h = 0; h < kGMax; ++h)
              if (h < G) acc[h] = fmaf(q_s[h * D + c], kh, acc[h]);
          }
        } else {
          const int r = t0 + t;
          for (int c = c0; c < c0 + cpp; ++c) {
            const float kh = (r == a.r_new) ? bf16_to_f32(f32_to_bf16(load_f32(knp, c)))
                                            : bf16_to_f32(kres[static_cast<size_t>(r) * D + c]);
#pragma unroll
            for (int h = 0; h < kGMax; ++h)
              if (h < G) acc[h] = fmaf(q_s[h * D + c], kh, acc[h]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < kGMax; ++h) {
        acc[h] += __shfl_xor(acc[h], 1);
        acc[h] += __shfl_xor(acc[h], 2);
      }
      if (part == 0) {
#pragma unroll
        for (int h = 0; h < kGMax; ++h)
          if (h < G) p_s[h * kTile + t] = (t < ntok) ? acc[h] * a.scale2 : -INFINITY;
      }
    }
    __syncthreads();
    // ---- online softmax: wave w owns heads w, w+4, ...
    {
      const int w = tid >> 6, lane = tid & 63;
      for (int h = w; h < G; h += kThreads / 64) {
        const float x = p_s[h * kTile + lane];
        const float mt = wave_max(x);
        const float mold = m_s[h];
        const float mnew = fmaxf(mold, mt);
        const float alpha = (mold == -INFINITY) ? 0.0f : exp2f(mold - mnew);
        const float p = (x == -INFINITY) ? 0.0f : exp2f(x - mnew);
        const float ls = wave_sum(p);
        p_s[h * kTile + lane] = p;
        if (lane == 0) {
          alpha_s[h] = alpha;
          m_s[h] = mnew;
          l_s[h] = l_s[h] * alpha + ls;
        }
      }
    }
    __syncthreads();
    // ---- values: thread (channel, part)
    if (vpart < P) {
#pragma unroll
      for (int h = 0; h < kGMax; ++h)
        if (h < G) o[h] *= alpha_s[h];
      const int c = vc_ch, jg = c / kGroup;
      if (!resid) {
        const int nrow = ntok / per;
        for (int r = vpart; r < nrow; r += P) {
          const uint32_t word = vc[(static_cast<size_t>(t0) / per + r) * D + c];
#pragma unroll
          for (int i = 0; i < per; ++i) {
            const int t = r * per + i;
            const float code = static_cast<float>((word >> (BITS * i)) & mask);
            const float2 sz = vmeta_s[t * ngv + jg];
            const float vh = fmaf(code, sz.x, sz.y);
#pragma unroll
            for (int h = 0; h < kGMax; ++h)
              if (h < G) o[h] = fmaf(p_s[h * kTile + t], vh, o[h]);
          }
        }
      } else {
        for (int t = vpart; t < ntok; t += P) {
          const int r = t0 + t;
          const float vh = (r == a.r_new) ? bf16_to_f32(f32_to_bf16(load_f32(vnp, c)))
                                          : bf16_to_f32(vres[static_cast<size_t>(r) * D + c]);
#pragma unroll
          for (int h = 0; h < kGMax; ++h)
            if (h < G) o[h] = fmaf(p_s[h * kTile + t], vh, o[h]);
        }
      }
    }
    __syncthreads();
  }

  // the residual split stores the appended token (its only writer)
  if (resid && a.r_new >= 0) {
    uint16_t* kw = a.k_res + (static_cast<size_t>(bj) * a.r_cap + a.r_new) * D;
    uint16_t* vw = a.v_res + (static_cast<size_t>(bj) * a.r_cap + a.r_new) * D;
    for (int c = tid; c < D; c += kThreads) {
      kw[c] = f32_to_bf16(load_f32(knp, c));
      vw[c] = f32_to_bf16(load_f32(vnp, c));
    }
  }
  // combine the value-phase parts and write this split's partial state
  if (vpart < P) {
#pragma unroll
    for (int h = 0; h < kGMax; ++h)
      if (h < G) red_s[(h * P + vpart) * D + vc_ch] = o[h];
  }
  __syncthreads();
  const int ns = a.nsplit + 1;
  float* po = a.part_o + (static_cast<size_t>(bj) * ns + s) * G * D;
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, c = e % D;
    float acc = 0.0f;
    for (int p = 0; p < P; ++p) acc += red_s[(h * P + p) * D + c];
    po[e] = acc;
  }
  if (tid < G) a.part_ml[(static_cast<size_t>(bj) * ns + s) * G + tid] = make_float2(m_s[tid], l_s[tid]);
}

__global__ __launch_bounds__(kThreads) void merge_kernel(const float* part_o, const float2* part_ml,
                                                          float* out, int Hq, int Hkv, int G, int D,
                                                          int ns) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int j = h / G, hl = h % G;
  const size_t bj = static_cast<size_t>(b) * Hkv + j;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part_ml[(bj * ns + s) * G + hl].x);
  float L = 0.0f;
  for (int s = 0; s < ns; ++s) {
    const float2 ml = part_ml[(bj * ns + s) * G + hl];
    if (ml.y > 0.0f) L += ml.y * exp2f(ml.x - M);
  }
  const float invL = 1.0f / L;
  for (int c = threadIdx.x; c < D; c += kThreads) {
    float acc = 0.0f;
    for (int s = 0; s < ns; ++s) {
      const float2 ml = part_ml[(bj * ns + s) * G + hl];
      if (ml.y > 0.0f) acc += exp2f(ml.x - M) * part_o[((bj * ns + s) * G + hl) * D + c];
    }
    out[(static_cast<size_t>(b) * Hq + h) * D + c] = acc * invL;
  }
}

void plan_splits(int q_len, int B, int Hkv, int* nsplit, int* chunk) {
  if (q_len <= 0) {
    *nsplit = 0;
    *chunk = kTile;
    return;
  }
  const int target = std::max(1, (kTargetBlocks + B * Hkv - 1) / (B * Hkv));
  const int tiles = (q_len + kTile - 1) / kTile;
  const int per = (tiles + target - 1) / target;
  *chunk = per * kTile;
  *nsplit = (q_len + *chunk - 1) / *chunk;
}

size_t decode_ws_bytes(const kvc_cache* c, int G) {
  int ns, ch;
  plan_splits(c->q_cap, c->batch, c->kv_heads, &ns, &ch);
  const int target = std::max(1, (kTargetBlocks + c->batch * c->kv_heads - 1) / (c->batch * c->kv_heads));
  ns = std::max(ns, target) + 1;
  const size_t units = static_cast<size_t>(c->batch) * c->kv_heads * ns * G;
  return align_up(units * c->head_dim * sizeof(float), 256) + units * sizeof(float2);
}

}  // namespace
}  // namespace kvc

extern "C" kvc_status kvc_decode_attn(kvc_cache* cache, const void* q, const void* k_new,
                                      const void* v_new, kvc_dtype dtype, int32_t Hq, float* out,
                                      void* ws, size_t* ws_bytes, void* stream) {
  using namespace kvc;
  if (!cache_ok(cache) || !ws_bytes) return KVC_ERR_NULL;
  if (!dtype_ok(dtype)) return KVC_ERR_DTYPE;
  kvc_status s = cache_shape_status(cache);
  if (s != KVC_OK) return s;
  const int Hkv = cache->kv_heads;
  if (Hq < 1 || Hq % Hkv != 0 || Hq / Hkv > kGMax) return KVC_ERR_SHAPE;
  const int G = Hq / Hkv;
  const size_t need = decode_ws_bytes(cache, G);
  if (!ws) {
    *ws_bytes = need;
    return KVC_OK;
  }
  if (!q || !k_new || !v_new || !out) return KVC_ERR_NULL;
  if (*ws_bytes < need) return KVC_ERR_WORKSPACE;
  const int R = cache->residual;
  if (cache->r_len + 1 > cache->r_cap) return KVC_ERR_CAPACITY;
  const bool flush = (cache->r_len + 1 == R + kGroup);
  if (flush && cache->q_len + kGroup > cache->q_cap) return KVC_ERR_CAPACITY;
  hipStream_t st = static_cast<hipStream_t>(stream);

  AttnArgs a;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  if (flush) {
    s = launch_flush(cache, k_new, v_new, dtype, st);
    if (s != KVC_OK) return s;
    cache->q_len += kGroup;
    cache->r_len = R;
    a.r_total = R;
    a.r_new = -1;
  } else {
    a.r_new = cache->r_len;
    a.r_total = cache->r_len + 1;
    cache->r_len += 1;
  }
  a.k_codes = cache->k_codes;
  a.k_meta = cache->k_meta;
  a.v_codes = cache->v_codes;
  a.v_meta = cache->v_meta;
  a.k_res = cache->k_res;
  a.v_res = cache->v_res;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.D = cache->head_dim;
  a.q_cap = cache->q_cap;
  a.r_cap = cache->r_cap;
  a.q_len = cache->q_len;
  plan_splits(cache->q_len, cache->batch, Hkv, &a.nsplit, &a.chunk);
  const int ns = a.nsplit + 1;
  const size_t units = static_cast<size_t>(cache->batch) * Hkv * ns * G;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float2*>(static_cast<char*>(ws) + align_up(units * a.D * sizeof(float), 256));
  a.scale2 = 1.4426950408889634f / sqrtf(static_cast<float>(a.D));
  dim3 grid(ns, Hkv, cache->batch);
  if (dtype == KVC_F32) {
    if (cache->bits == 2)
      hipLaunchKernelGGL((attn_split_kernel<float, 2>), grid, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((attn_split_kernel<float, 4>), grid, dim3(kThreads), 0, st, a);
  } else {
    if (cache->bits == 2)
      hipLaunchKernelGGL((attn_split_kernel<uint16_t, 2>), grid, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((attn_split_kernel<uint16_t, 4>), grid, dim3(kThreads), 0, st, a);
  }
  s = check_launch();
  if (s != KVC_OK) return s;
  hipLaunchKernelGGL(merge_kernel, dim3(Hq, cache->batch), dim3(kThreads), 0, st, a.part_o, a.part_ml,
                     out, Hq, Hkv, G, a.D, ns);
  return check_launch();
}
