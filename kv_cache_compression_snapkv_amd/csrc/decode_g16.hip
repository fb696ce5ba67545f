// Single-query decode attention over a cache quantized in groups of 16 (MiniKV
// Sec. 5.1's group size; Alg. 1 decoding: one softmax over the dequantized
// history followed by the bf16 residual, the appended token included).
//
// One workgroup per (query head, batch row, split of the token range; the
// splits' partial softmax states are merged by merge_g16_kernel).  Tokens are scored in chunks of
// kChunk, one token per thread, with the history dequantized in float32 as
// stored (zero + code * scale, each rounded); a running maximum and sum give one
// online softmax over the chunks; the values are accumulated one channel per
// thread.  This path is deliberately plain: with 16-token key groups every MFMA
// column tile of the group-32 kernel would need its own scaled query operand,
// so the group-16 layout gets a direct kernel of its own.
#include <algorithm>

#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kG16 = 16;
constexpr int kChunk = 256;  // threads per workgroup = tokens per chunk; D <= 256 channels

struct G16Args {
  const void* q;
  const void* k_new;
  const void* v_new;
  const uint32_t *k_codes, *k_meta, *v_codes, *v_meta;
  uint16_t *k_res, *v_res;
  float* out;
  float2* part_ml;  // [B][Hq][S] running (max, sum) of each split (S > 1)
  float* part_o;    // [B][Hq][S][D] its unnormalized output
  int Hq, Hkv, G, D, q_len, q_cap, r_total, r_new, r_start, r_cap;
  int span;         // tokens per split, a multiple of kChunk
  float scale;      // 1/sqrt(D)
};

// Block-wide maximum / sum of one value per thread (every thread gets it).
__device__ __forceinline__ float block_reduce(float x, float* sh, bool is_max) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float y = __shfl_xor(x, o);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = x;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < kChunk / 64; ++i) r = is_max ? fmaxf(r, sh[i]) : r + sh[i];
  __syncthreads();  // sh is reused by the next reduction
  return r;
}

// Dequantized value of a code: zero + code * scale, in float32 (two roundings).
__device__ __forceinline__ float dq(uint32_t code, uint32_t meta) {
  return __fadd_rn(f16_bits_to_f32(meta >> 16), __fmul_rn(static_cast<float>(code), f16_bits_to_f32(meta & 0xFFFFu)));
}

template <typename T, int BITS>
__global__ __launch_bounds__(kChunk) void decode_g16_kernel(G16Args a) {
  __shared__ float qs[256];
  __shared__ float ps[kChunk];
  __shared__ float red[kChunk / 64];
  __shared__ uint32_t kms[kChunk / kG16][256];        // key meta of the chunk's 16 groups
  __shared__ uint32_t vcs[kChunk * BITS / 32][256];   // value code word rows of the chunk
  __shared__ uint32_t vms[kChunk][256 / kG16];        // value meta of the chunk's tokens
  constexpr int per = 32 / BITS;  // codes per word
  constexpr uint32_t mask = (1u << BITS) - 1u;
  const int h = blockIdx.x, b = blockIdx.y, sp = blockIdx.z, tid = threadIdx.x;
  const int D = a.D;
  const size_t bj = static_cast<size_t>(b) * a.Hkv + h / a.G;
  const T* qp = static_cast<const T*>(a.q) + (static_cast<size_t>(b) * a.Hq + h) * D;
  const T* knp = static_cast<const T*>(a.k_new) + bj * D;
  const T* vnp = static_cast<const T*>(a.v_new) + bj * D;
  if (tid < D) qs[tid] = load_f32(qp, tid);
  __syncthreads();
  const int nkw = D / per;   // key words per token
  const int ngv = D / kG16;  // value groups per token
  const uint32_t* kc = a.k_codes + bj * a.q_cap * nkw;
  const uint32_t* km = a.k_meta + bj * (a.q_cap / kG16) * D;
  const uint32_t* vc = a.v_codes + bj * (a.q_cap / per) * D;
  const uint32_t* vm = a.v_meta + bj * a.q_cap * ngv;
  const uint16_t* kr = a.k_res + bj * a.r_cap * D;  // [r_cap][D], token-major
  const uint16_t* vr = a.v_res + bj * D * a.r_cap;  // [D][r_cap], channel-major
  auto ring = [&](int t) {
    const int p = a.r_start + t;
    return p >= a.r_cap ? p - a.r_cap : p;
  };
  const int NT = min(a.q_len + a.r_total, (sp + 1) * a.span);  // end of this split's tokens
  // values: tpc threads per channel, each with its own share of the tokens and
  // its own partial output (all scaled alike), summed at the end
  const int tpc = kChunk / D;  // >= 1 (D <= 256)
  const int c = tid % D, part = tid / D;
  float m = -INFINITY, l = 0.0f, o = 0.0f;  // o: this thread's part of channel c
  for (int t0 = sp * a.span; t0 < NT; t0 += kChunk) {
    const int t = t0 + tid;
    // packed tokens of this chunk: [t0, t0 + np), whole groups (t0 and q_len are
    // multiples of 16); their key meta, value code rows and value meta go to LDS
    // with coalesced loads, all issued before the first use
    const int np = max(0, min(kChunk, a.q_len - t0));
    for (int e = tid; e < (np / kG16) * D; e += kChunk) {
      const int gi = e / D, c = e - gi * D;
      kms[gi][c] = km[static_cast<size_t>(t0 / kG16 + gi) * D + c];
    }
    for (int e = tid; e < (np / per) * D; e += kChunk) {
      const int r = e / D, c = e - r * D;
      vcs[r][c] = vc[static_cast<size_t>(t0 / per + r) * D + c];
    }
    for (int e = tid; e < np * ngv; e += kChunk) vms[e / ngv][e % ngv] = vm[static_cast<size_t>(t0) * ngv + e];
    __syncthreads();
    float s = -INFINITY;
    if (t < NT) {
      float acc = 0.0f;
      if (t < a.q_len) {
        const uint32_t* kw = kc + static_cast<size_t>(t) * nkw;
        const uint32_t* mrow = kms[tid / kG16];
        for (int w = 0; w < nkw; ++w) {
          const uint32_t word = kw[w];
#pragma unroll
          for (int i = 0; i < per; ++i) {
            const int c = w * per + i;
            acc = fmaf(qs[c], dq((word >> (BITS * i)) & mask, mrow[c]), acc);
          }
        }
      } else {
        const int tr = t - a.q_len;
        if (tr == a.r_new) {
          for (int c = 0; c < D; ++c) acc = fmaf(qs[c], bf16_to_f32(f32_to_bf16(load_f32(knp, c))), acc);
        } else {
          const uint4* row = reinterpret_cast<const uint4*>(kr + static_cast<size_t>(ring(tr)) * D);
          for (int c8 = 0; c8 < D / 8; ++c8) {
            const uint4 w = row[c8];
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              acc = fmaf(qs[8 * c8 + 2 * i], __uint_as_float(u[i] << 16), acc);
              acc = fmaf(qs[8 * c8 + 2 * i + 1], __uint_as_float(u[i] & 0xFFFF0000u), acc);
            }
          }
        }
      }
      s = acc * a.scale;
    }
    // every chunk holds a token (t0 < NT), so the maximum is finite
    const float mn = fmaxf(m, block_reduce(s, red, true));
    const float alpha = __expf(m - mn);  // 0 for the first chunk
    const float p = t < NT ? __expf(s - mn) : 0.0f;
    ps[tid] = p;
    l = l * alpha + block_reduce(p, red, false);  // its barriers also publish ps
    m = mn;
    if (part < tpc) {
      float acc = o * alpha;
      const int tn = min(kChunk, NT - t0);
      // packed tokens, from the staged rows (words part, part + tpc, ...)
      const int jc = c / kG16;
      for (int i0 = part * per; i0 < np; i0 += tpc * per) {
        const uint32_t word = vcs[i0 / per][c];
#pragma unroll
        for (int u = 0; u < per; ++u)
          acc = fmaf(ps[i0 + u], dq((word >> (BITS * u)) & mask, vms[i0 + u][jc]), acc);
      }
      // residual tokens, 8 at a time: the first is a multiple of 8 from the
      // ring start (q_len and t0 are multiples of 16), and r_start and r_cap are
      // multiples of 8, so the 8 ring rows of a channel are one 16-byte load
      // (rows past the residual are read but not used)
      const float vnew = bf16_to_f32(f32_to_bf16(load_f32(vnp, c)));
      for (int i0 = np + 8 * part; i0 < tn; i0 += 8 * tpc) {
        const int tr0 = t0 + i0 - a.q_len;
        const uint4 w = *reinterpret_cast<const uint4*>(vr + static_cast<size_t>(c) * a.r_cap + ring(tr0));
        const uint32_t u4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float x = (tr0 + u == a.r_new) ? vnew : __uint_as_float(u & 1 ? u4[u >> 1] & 0xFFFF0000u : u4[u >> 1] << 16);
          if (i0 + u < tn) acc = fmaf(ps[i0 + u], x, acc);
        }
      }
      o = acc;
    }
    __syncthreads();  // ps is rewritten by the next chunk
  }
  // sum the parts of each channel (ps is free after the last chunk's barrier)
  if (part < tpc) ps[part * D + c] = o;
  __syncthreads();
  if (tid < D) {
    o = 0.0f;
    for (int p2 = 0; p2 < tpc; ++p2) o += ps[p2 * D + tid];
  }
  const size_t bh = static_cast<size_t>(b) * a.Hq + h;
  if (gridDim.z == 1) {
    if (tid < D) a.out[bh * D + tid] = o / l;
  } else {
    const size_t ps_i = bh * gridDim.z + sp;
    if (tid < D) a.part_o[ps_i * D + tid] = o;
    if (tid == 0) a.part_ml[ps_i] = make_float2(m, l);
  }
  // the appended token joins the ring (written by split 0 of the first query
  // head of its KV head; no workgroup reads that row in this call)
  if (a.r_new >= 0 && h % a.G == 0 && sp == 0 && tid < D) {
    const int p = ring(a.r_new);
    a.k_res[(bj * a.r_cap + p) * D + tid] = f32_to_bf16(load_f32(knp, tid));
    a.v_res[(bj * D + tid) * a.r_cap + p] = f32_to_bf16(load_f32(vnp, tid));
  }
}

// The S splits of (b, h) merged: with M = max_s m_s, out = sum_s e^(m_s - M) o_s
// / sum_s e^(m_s - M) l_s (every split holds at least one token).
__global__ __launch_bounds__(kChunk) void merge_g16_kernel(const float2* part_ml, const float* part_o, float* out,
                                                           int Hq, int D, int S) {
  const size_t bh = static_cast<size_t>(blockIdx.y) * Hq + blockIdx.x;
  const int c = threadIdx.x;
  if (c >= D) return;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part_ml[bh * S + s].x);
  float L = 0.0f, acc = 0.0f;
  for (int s = 0; s < S; ++s) {
    const float2 ml = part_ml[bh * S + s];
    const float w = __expf(ml.x - M);
    L += w * ml.y;
    acc += w * part_o[(bh * S + s) * D + c];
  }
  out[bh * D + c] = acc / L;
}

}  // namespace

// Splits of the token range for a call: enough workgroups to fill the GPU
// (about 2048), at least one chunk each.  Bounded by the capacities so that the
// workspace query and the call agree.
int g16_splits(int B, int Hq, int tokens) {
  const int chunks = std::max(1, (tokens + kChunk - 1) / kChunk);
  return std::max(1, std::min(chunks, (2048 + B * Hq - 1) / (B * Hq)));
}
size_t g16_ws_bytes(const kvc_cache* c, int Hq) {
  const int S = g16_splits(c->batch, Hq, c->q_cap + c->r_cap);
  if (S == 1) return 0;
  const size_t n = static_cast<size_t>(c->batch) * Hq * S;
  return align_up(n * sizeof(float2), 256) + n * c->head_dim * sizeof(float);
}

// Launch for a cache whose group is 16, after the host has appended the new
// token (r_total, r_new as for the group-32 kernel: r_new = -1 after a flush).
kvc_status launch_decode_g16(const kvc_cache* c, const void* q, const void* k_new, const void* v_new, kvc_dtype dt,
                             int Hq, int r_total, int r_new, float* out, void* ws, hipStream_t st) {
  G16Args a;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_codes = c->k_codes;
  a.k_meta = c->k_meta;
  a.v_codes = c->v_codes;
  a.v_meta = c->v_meta;
  a.k_res = c->k_res;
  a.v_res = c->v_res;
  a.out = out;
  a.Hq = Hq;
  a.Hkv = c->kv_heads;
  a.G = Hq / c->kv_heads;
  a.D = c->head_dim;
  a.q_len = c->q_len;
  a.q_cap = c->q_cap;
  a.r_total = r_total;
  a.r_new = r_new;
  a.r_start = c->r_start;
  a.r_cap = c->r_cap;
  a.scale = 1.0f / sqrtf(static_cast<float>(c->head_dim));
  // splits: at most the capacity-bound count (the workspace is sized for it),
  // trimmed so that none is empty
  const int NT = c->q_len + r_total;
  const int smax = g16_splits(c->batch, Hq, c->q_cap + c->r_cap);
  int S = std::min(smax, g16_splits(c->batch, Hq, NT));
  a.span = kChunk * (((NT + S - 1) / S + kChunk - 1) / kChunk);
  S = (NT + a.span - 1) / a.span;
  const size_t n = static_cast<size_t>(c->batch) * Hq * smax;
  a.part_ml = static_cast<float2*>(ws);
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(n * sizeof(float2), 256));
  const dim3 grid(Hq, c->batch, S);
  if (dt == KVC_F32) {
    if (c->bits == 2) hipLaunchKernelGGL((decode_g16_kernel<float, 2>), grid, dim3(kChunk), 0, st, a);
    else hipLaunchKernelGGL((decode_g16_kernel<float, 4>), grid, dim3(kChunk), 0, st, a);
  } else {
    if (c->bits == 2) hipLaunchKernelGGL((decode_g16_kernel<uint16_t, 2>), grid, dim3(kChunk), 0, st, a);
    else hipLaunchKernelGGL((decode_g16_kernel<uint16_t, 4>), grid, dim3(kChunk), 0, st, a);
  }
  kvc_status s = check_launch();
  if (s != KVC_OK || S == 1) return s;
  hipLaunchKernelGGL(merge_g16_kernel, dim3(Hq, c->batch), dim3(kChunk), 0, st, a.part_ml, a.part_o, out, Hq,
                     c->head_dim, S);
  return check_launch();
}

}  // namespace kvc
