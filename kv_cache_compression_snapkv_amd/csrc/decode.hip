// Single-query decode attention over the compressed cache (MiniKV Eq. 1 and
// Alg. 1 decoding; blog attention hook: one softmax over exact recent tokens and
// dequantized older ones; query head h reads KV head h / G).
//
// Work split.  The tokens of one (batch, KV head) are cut into 32-token tiles:
// Q/32 packed-history tiles (one key group each) followed by the bf16 residual
// tiles.  Every wavefront owns a contiguous run of tiles for up to 8 query heads
// of that KV head and keeps its own online-softmax state; the four waves of a
// workgroup merge through LDS, M = max m_w, o = sum_w 2^(m_w-M) o_w,
// l = sum_w 2^(m_w-M) l_w (log2 units), and write the output directly when one
// workgroup covers the whole (batch, KV head), else a partial that a small
// merge kernel combines the same way.  (No cross-workgroup atomics: a
// device-scope release fence costs an L2 write-back per wavefront.)
//
// Contractions on MFMA (v_mfma_f32_16x16x32_bf16).  Rows of the 16-row operand
// are (head, split) pairs: row 2h holds the bf16 truncation of a float32 value
// and row 2h+1 the bf16 truncation of its remainder, so hi+lo carries 16
// significant bits and products accumulate in fp32.
//   keys:   S[t] = sum_c A[c] B[c][t] with B = 1 + code*2^(pos-7), the code OR-ed
//           into the mantissa of bf16 1.0 (one bitwise op per two codes), and
//           A = q*scale*2^(7-pos) per group; the 1.0 offset is removed by the
//           same A against an all-(-1) operand and the zero-point added by
//           split(q*zero) against an all-ones operand.
//   values: o[c] = sum_t A[t] B[t][c] with the same code encoding and
//           A = p*scale*2^(7-pos) per (token, 32-channel group), with the same
//           two corrections (A x -1, split(p*zero) x 1).
//   residual: B = bf16 keys/values as stored, A = q or p split in two.
#include <algorithm>

#include "kvc_internal.h"

namespace kvc {

kvc_status launch_flush(const kvc_cache* c, const void* k_new, const void* v_new, kvc_dtype dt,
                        hipStream_t st);
bool cache_ok(const kvc_cache* c);
kvc_status cache_shape_status(const kvc_cache* c);

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kHB = 8;              // query heads per head block (2 MFMA rows each)
constexpr int kPrefetch = 2;        // history tiles in flight per wave

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kOne2 = 0x3F803F80u;     // two bf16 1.0
constexpr uint32_t kNegOne2 = 0xBF80BF80u;  // two bf16 -1.0

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

// x = hi + lo with hi, lo bf16 (truncations); eff = hi + lo as float.
struct Split {
  uint32_t hi, lo;
  float eff;
};
__device__ __forceinline__ Split split2(float x) {
  Split s;
  const uint32_t hb = __float_as_uint(x) & 0xFFFF0000u;
  const float r = x - __uint_as_float(hb);
  const uint32_t lb = __float_as_uint(r) & 0xFFFF0000u;
  s.hi = hb >> 16;
  s.lo = lb >> 16;
  s.eff = __uint_as_float(hb) + __uint_as_float(lb);
  return s;
}

// bf16 bit position of the code inside register jj of an unpacked word.
// 2-bit: jj 0..2 -> 0,2,4 and jj 3 -> 0 (after a 6-bit shift); 4-bit: 0.
template <int BITS> __device__ __forceinline__ int code_pos(int jj) {
  return BITS == 2 ? (jj < 3 ? 2 * jj : 0) : 0;
}

// Four bf16x2 registers from one packed word: register jj holds codes of the
// pair (p, p + half-word span) as 1 + code*2^(pos-7).
// 2-bit (16 codes, i at bits 2i): `half` picks pairs 0..3 or 4..7, pair p =
//   codes (p, p+8).  4-bit (8 codes, i at bits 4i): pair p = codes (p, p+4).
template <int BITS> __device__ __forceinline__ u32x4 unpack4(uint32_t w, int half) {
  u32x4 r;
  if (BITS == 2) {
    const uint32_t x = w >> (8 * half);
    r.x = (x & 0x00030003u) | kOne2;
    r.y = (x & 0x000C000Cu) | kOne2;
    r.z = (x & 0x00300030u) | kOne2;
    r.w = ((x >> 6) & 0x00030003u) | kOne2;
  } else {
    r.x = (w & 0x000F000Fu) | kOne2;
    r.y = ((w >> 4) & 0x000F000Fu) | kOne2;
    r.z = ((w >> 8) & 0x000F000Fu) | kOne2;
    r.w = ((w >> 12) & 0x000F000Fu) | kOne2;
  }
  return r;
}

// Channel held in k-slot (8*lq + 2*jj + e) of k-step s for a packed history key.
template <int BITS, int KS> __device__ __forceinline__ int key_channel(int s, int lq, int jj, int e) {
  if (BITS == 2) {
    const int hw = lq * KS + s;  // half-word index within the token's codes
    return 16 * (hw >> 1) + 4 * (hw & 1) + jj + 8 * e;
  }
  return 8 * (lq * KS + s) + jj + 4 * e;
}
// Token (within a 32-token tile) held in value k-slot (8*lq + 2*jj + e).
template <int BITS> __device__ __forceinline__ int value_token(int lq, int jj, int e) {
  if (BITS == 2) return 16 * (lq >> 1) + 4 * (lq & 1) + jj + 8 * e;
  return 8 * lq + jj + 4 * e;
}
// Token of column n in key column tile ct: tile 0 holds tokens {0..7,16..23},
// tile 1 holds {8..15,24..31}, so one lane's two tokens are a value slot pair.
__device__ __forceinline__ int col_token(int ct, int n) { return 16 * (n >> 3) + (n & 7) + 8 * ct; }

struct DecArgs {
  const void* q;
  const void* k_new;
  const void* v_new;
  const uint32_t *k_codes, *k_meta, *v_codes, *v_meta;
  uint16_t *k_res, *v_res;  // k_res [bj][r_cap][D], v_res [bj][D][r_cap]
  float* part_o;            // [bjh][nb][8][D] (used when nb > 1)
  float2* part_ml;          // [bjh][nb][8]
  float* out;               // [B][Hq][D]
  int Hq, Hkv, G, HB, q_cap, r_cap;
  int q_len, r_total, r_new;
  int nb, tpw;
  float scale2;  // log2(e)/sqrt(D)
};

// LDS layout (bytes), shared by host sizing and the kernel.
struct Lds {
  int qf, qx, ares, wave0, wave_bytes, total;
  int ak, akz, av, avz, pbuf;  // offsets inside one wave's region
};
__host__ __device__ inline Lds lds_layout(int KS, int Gb) {
  const int D = 32 * KS, R2 = 2 * Gb;
  Lds L;
  L.qf = 0;
  L.qx = Gb * D * 4;
  L.ares = 2 * Gb * D * 4;
  L.wave0 = (L.ares + KS * R2 * 64 + 15) / 16 * 16;
  L.ak = 0;
  L.akz = KS * R2 * 64;
  L.av = 2 * KS * R2 * 64;
  L.avz = 3 * KS * R2 * 64;
  L.pbuf = 4 * KS * R2 * 64;
  L.wave_bytes = (L.pbuf + Gb * 32 * 4 + 15) / 16 * 16;
  L.total = L.wave0 + kWaves * L.wave_bytes;
  return L;
}

template <typename T>
__device__ __forceinline__ uint32_t load_bf16_pair(const T* p, int i) {
  return static_cast<uint32_t>(f32_to_bf16(load_f32(p, i))) |
         (static_cast<uint32_t>(f32_to_bf16(load_f32(p, i + 1))) << 16);
}

// All-reduce over the 16 lanes of a DPP row: swap neighbours, swap pairs,
// mirror within 8, mirror within 16.
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp<0x140>(x));  // row_mirror
  return x;
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T, int BITS, int KS>
__global__ __launch_bounds__(kThreads, (KS == 2 || KS == 4) ? 2 : 1) void decode_kernel(DecArgs a) {
  constexpr int D = 32 * KS;
  constexpr int NGV = KS;  // value channel groups
  constexpr int NW = D * BITS / 32;  // key words per token
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 15, lq = lane >> 4;
  const int b = blockIdx.z, jh = blockIdx.y;
  const int j = jh / a.HB, hb = jh % a.HB;
  const int bj = b * a.Hkv + j;
  const int bjh = bj * a.HB + hb;
  const int h0 = hb * kHB;
  const int Gb = min(kHB, a.G - h0);
  const int R2 = 2 * Gb;
  const Lds L = lds_layout(KS, Gb);
  float* qf = reinterpret_cast<float*>(smem + L.qf);
  float* qx = reinterpret_cast<float*>(smem + L.qx);
  uint16_t* ares = reinterpret_cast<uint16_t*>(smem + L.ares);
  unsigned char* wbase = smem + L.wave0 + wave * L.wave_bytes;
  uint16_t* AK = reinterpret_cast<uint16_t*>(wbase + L.ak);
  uint16_t* AKz = reinterpret_cast<uint16_t*>(wbase + L.akz);
  uint16_t* AV = reinterpret_cast<uint16_t*>(wbase + L.av);
  uint16_t* AVz = reinterpret_cast<uint16_t*>(wbase + L.avz);
  float* pbuf = reinterpret_cast<float*>(wbase + L.pbuf);

  // ---------------------------------------------------------------- setup (block)
  // q (plain and scaled for the key operand) and the residual key operand
  // split(q) in natural channel order, from one load per element
  const T* qp = static_cast<const T*>(a.q) + (static_cast<size_t>(b) * a.Hq + j * a.G + h0) * D;
  for (int e = tid; e < Gb * D; e += kThreads) {
    const float v = load_f32(qp, e);
    const int h = e / D, c = e % D;
    qf[e] = v;
    const int jj = (BITS == 2) ? (c & 3) : 0;  // key register index of channel c
    qx[e] = v * static_cast<float>(1 << (7 - code_pos<BITS>(jj)));
    const Split sp = split2(v);
    ares[((c >> 5) * R2 + 2 * h) * 32 + (c & 31)] = static_cast<uint16_t>(sp.hi);
    ares[((c >> 5) * R2 + 2 * h + 1) * 32 + (c & 31)] = static_cast<uint16_t>(sp.lo);
  }
  const size_t qc = a.q_cap;
  const uint32_t* kc = a.k_codes + static_cast<size_t>(bj) * qc * NW;
  const uint32_t* km = a.k_meta + static_cast<size_t>(bj) * (qc / kGroup) * D;
  const uint32_t* vc = a.v_codes + static_cast<size_t>(bj) * (qc * BITS / 32) * D;
  const uint32_t* vm = a.v_meta + static_cast<size_t>(bj) * qc * NGV;
  const uint16_t* kr = a.k_res + static_cast<size_t>(bj) * a.r_cap * D;
  const uint16_t* vr = a.v_res + static_cast<size_t>(bj) * D * a.r_cap;
  const T* knp = static_cast<const T*>(a.k_new) + static_cast<size_t>(bj) * D;
  const T* vnp = static_cast<const T*>(a.v_new) + static_cast<size_t>(bj) * D;

  const int sp = blockIdx.x * kWaves + wave;
  const int NTh = a.q_len / kGroup;
  const int NT = NTh + (a.r_total + kGroup - 1) / kGroup;
  const int tb = sp * a.tpw, te = min(NT, tb + a.tpw);

  f32x4 oacc[2 * NGV], vcorr[NGV];
#pragma unroll
  for (int i = 0; i < 2 * NGV; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NGV; ++i) vcorr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.f, 0.f};
  const bool row_on = ln < R2;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const u32x4 ones4 = {kOne2, kOne2, kOne2, kOne2};
  const u32x4 neg4 = {kNegOne2, kNegOne2, kNegOne2, kNegOne2};

  // Per tile, D/2 key channel pairs and D/2 value (group, token pair) items;
  // lane l owns positions l + 64u and loops over the heads, so its meta loads do
  // not depend on the head and can be issued a tile ahead.
  constexpr int NP = (D / 2 + 63) / 64;
  constexpr int NKW = (BITS == 2) ? KS / 2 + (KS & 1) : KS;  // key words a lane reads per token
  struct HistRegs {
    uint32_t kw[2][NKW];  // key code words, per column tile
    uint32_t km[NP][2];  // key meta of the lane's channel pairs
    uint32_t vm[NP][2];  // value meta of the lane's token pairs
    u32x2 vw[NGV];       // value code words, per channel group
  };
  auto load_hist = [&](int tile, HistRegs& r) {
    const int t0 = tile * kGroup;
    const int w_first = (BITS == 2) ? ((lq * KS) >> 1) : lq * KS;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const uint32_t* row = kc + (t0 + col_token(ct, ln)) * NW + w_first;
      if constexpr (NKW == 4) {
        const u32x4 w4 = *reinterpret_cast<const u32x4*>(row);
        r.kw[ct][0] = w4.x; r.kw[ct][1] = w4.y; r.kw[ct][2] = w4.z; r.kw[ct][3] = w4.w;
      } else if constexpr (NKW == 2) {
        const u32x2 w2 = *reinterpret_cast<const u32x2*>(row);
        r.kw[ct][0] = w2.x; r.kw[ct][1] = w2.y;
      } else {
#pragma unroll
        for (int i = 0; i < NKW; ++i) r.kw[ct][i] = (w_first + i < NW) ? row[i] : 0u;
      }
    }
    const uint32_t* kmg = km + tile * D;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int pi = lane + 64 * u;
      r.km[u][0] = r.km[u][1] = r.vm[u][0] = r.vm[u][1] = 0u;
      if (pi < D / 2) {
        const int s = pi >> 4, q4 = (pi >> 2) & 3, jj = pi & 3;
        r.km[u][0] = kmg[key_channel<BITS, KS>(s, q4, jj, 0)];
        r.km[u][1] = kmg[key_channel<BITS, KS>(s, q4, jj, 1)];
        const int g = pi >> 4, pr = pi & 15;
        r.vm[u][0] = vm[(t0 + value_token<BITS>(pr >> 2, pr & 3, 0)) * NGV + g];
        r.vm[u][1] = vm[(t0 + value_token<BITS>(pr >> 2, pr & 3, 1)) * NGV + g];
      }
    }
    const int wrow = (BITS == 2) ? (t0 / 16 + (lq >> 1)) : (t0 / 8 + lq);
    const uint32_t* vrow = vc + wrow * D;
#pragma unroll
    for (int g = 0; g < NGV; ++g) r.vw[g] = *reinterpret_cast<const u32x2*>(vrow + 32 * g + 2 * ln);
  };

  // ---- the online softmax update shared by both tile kinds.  x[hh][ct] are
  // log2-scaled scores (-inf when masked); returns p in place and rescales the
  // accumulators when a running max moves (skipped when no lane's moves, which
  // leaves the result bit-identical).
  auto softmax_update = [&](float (&x)[2][2]) {
    float alpha[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float mt = max16(fmaxf(x[hh][0], x[hh][1]));
      const float mnew = fmaxf(m_run[hh], mt);
      if (mnew == -INFINITY) {
        alpha[hh] = 1.0f;
        x[hh][0] = x[hh][1] = 0.0f;
      } else {
        alpha[hh] = exp2f(m_run[hh] - mnew);
        x[hh][0] = exp2f(x[hh][0] - mnew);
        x[hh][1] = exp2f(x[hh][1] - mnew);
      }
      m_run[hh] = mnew;
      l_part[hh] = l_part[hh] * alpha[hh] + x[hh][0] + x[hh][1];
      const int head = 2 * lq + hh;
      if (head < Gb) {
        pbuf[head * 32 + col_token(0, ln)] = x[hh][0];
        pbuf[head * 32 + col_token(1, ln)] = x[hh][1];
      }
    }
    if (__any(alpha[0] != 1.0f || alpha[1] != 1.0f)) {
#pragma unroll
      for (int i = 0; i < 2 * NGV; ++i) {
        oacc[i][0] *= alpha[0];
        oacc[i][1] *= alpha[0];
        oacc[i][2] *= alpha[1];
        oacc[i][3] *= alpha[1];
      }
#pragma unroll
      for (int g = 0; g < NGV; ++g) {
        vcorr[g][0] *= alpha[0];
        vcorr[g][1] *= alpha[0];
        vcorr[g][2] *= alpha[1];
        vcorr[g][3] *= alpha[1];
      }
    }
    wave_sync();
  };

  // ---- one packed-history tile from its prefetched registers
  auto process_hist = [&](const HistRegs& cur, int tile) {
    // key operand A (query x group scale) and split(query x zero-point)
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int pi = lane + 64 * u;
      if (pi < D / 2) {
        const int s = pi >> 4, q4 = (pi >> 2) & 3, jj = pi & 3;
        const int c0 = key_channel<BITS, KS>(s, q4, jj, 0), c1 = key_channel<BITS, KS>(s, q4, jj, 1);
        const float sc0 = f16_bits_to_f32(cur.km[u][0] & 0xFFFFu), sc1 = f16_bits_to_f32(cur.km[u][1] & 0xFFFFu);
        const float zp0 = f16_bits_to_f32(cur.km[u][0] >> 16), zp1 = f16_bits_to_f32(cur.km[u][1] >> 16);
        const int ob = s * R2 * 32 + 8 * q4 + 2 * jj;
#pragma unroll 1
        for (int h = 0; h < Gb; ++h) {
          const Split a0 = split2(qx[h * D + c0] * sc0), a1 = split2(qx[h * D + c1] * sc1);
          const Split z0 = split2(qf[h * D + c0] * zp0), z1 = split2(qf[h * D + c1] * zp1);
          const int o_hi = ob + 64 * h, o_lo = o_hi + 32;
          *reinterpret_cast<uint32_t*>(AK + o_hi) = a0.hi | (a1.hi << 16);
          *reinterpret_cast<uint32_t*>(AK + o_lo) = a0.lo | (a1.lo << 16);
          *reinterpret_cast<uint32_t*>(AKz + o_hi) = z0.hi | (z1.hi << 16);
          *reinterpret_cast<uint32_t*>(AKz + o_lo) = z0.lo | (z1.lo << 16);
        }
      }
    }
    wave_sync();
    // key MFMAs: two 16-token column tiles, then the offset/zero corrections
    f32x4 accS[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 accC = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 af = row_on ? *reinterpret_cast<const u32x4*>(AK + (s * R2 + ln) * 32 + 8 * lq) : zero4;
      const u32x4 az = row_on ? *reinterpret_cast<const u32x4*>(AKz + (s * R2 + ln) * 32 + 8 * lq) : zero4;
      uint32_t kw0, kw1;
      int half = 0;
      if constexpr (BITS == 2) {
        const int hw = (lq * KS) & 1;  // parity of the lane's first half-word
        half = (hw + s) & 1;
        const int i0 = s >> 1, i1 = (s + 1) >> 1;  // word index for hw == 0 / hw == 1
        kw0 = hw ? cur.kw[0][i1] : cur.kw[0][i0];
        kw1 = hw ? cur.kw[1][i1] : cur.kw[1][i0];
      } else {
        kw0 = cur.kw[0][s];
        kw1 = cur.kw[1][s];
      }
      accS[0] = mfma(af, unpack4<BITS>(kw0, half), accS[0]);
      accS[1] = mfma(af, unpack4<BITS>(kw1, half), accS[1]);
      accC = mfma(af, neg4, accC);
      accC = mfma(az, ones4, accC);
    }
    float x[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bool ok = 2 * lq + hh < Gb;
      const float corr = accC[2 * hh] + accC[2 * hh + 1];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        x[hh][ct] = ok ? (accS[ct][2 * hh] + accS[ct][2 * hh + 1] + corr) * a.scale2 : -INFINITY;
    }
    softmax_update(x);
    // value operand A (p x token scale per group) and split(p x zero-point)
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int vi = lane + 64 * u;
      if (vi < D / 2) {
        const int g = vi >> 4, pr = vi & 15, jj = pr & 3;
        const int t_lo = value_token<BITS>(pr >> 2, jj, 0), t_hi = value_token<BITS>(pr >> 2, jj, 1);
        const float f = static_cast<float>(1 << (7 - code_pos<BITS>(jj)));
        const float sc0 = f16_bits_to_f32(cur.vm[u][0] & 0xFFFFu) * f;
        const float sc1 = f16_bits_to_f32(cur.vm[u][1] & 0xFFFFu) * f;
        const float zp0 = f16_bits_to_f32(cur.vm[u][0] >> 16), zp1 = f16_bits_to_f32(cur.vm[u][1] >> 16);
        const int ob = g * R2 * 32 + 2 * pr;
#pragma unroll 1
        for (int h = 0; h < Gb; ++h) {
          const float p0 = pbuf[h * 32 + t_lo], p1 = pbuf[h * 32 + t_hi];
          const Split a0 = split2(p0 * sc0), a1 = split2(p1 * sc1);
          const Split z0 = split2(p0 * zp0), z1 = split2(p1 * zp1);
          const int o_hi = ob + 64 * h, o_lo = o_hi + 32;
          *reinterpret_cast<uint32_t*>(AV + o_hi) = a0.hi | (a1.hi << 16);
          *reinterpret_cast<uint32_t*>(AV + o_lo) = a0.lo | (a1.lo << 16);
          *reinterpret_cast<uint32_t*>(AVz + o_hi) = z0.hi | (z1.hi << 16);
          *reinterpret_cast<uint32_t*>(AVz + o_lo) = z0.lo | (z1.lo << 16);
        }
      }
    }
    wave_sync();
    const int half = (BITS == 2) ? (lq & 1) : 0;
#pragma unroll
    for (int g = 0; g < NGV; ++g) {
      const u32x4 af = row_on ? *reinterpret_cast<const u32x4*>(AV + (g * R2 + ln) * 32 + 8 * lq) : zero4;
      const u32x4 az = row_on ? *reinterpret_cast<const u32x4*>(AVz + (g * R2 + ln) * 32 + 8 * lq) : zero4;
      oacc[2 * g] = mfma(af, unpack4<BITS>(cur.vw[g].x, half), oacc[2 * g]);
      oacc[2 * g + 1] = mfma(af, unpack4<BITS>(cur.vw[g].y, half), oacc[2 * g + 1]);
      vcorr[g] = mfma(af, neg4, vcorr[g]);
      vcorr[g] = mfma(az, ones4, vcorr[g]);
    }
    wave_sync();
  };

  // ---- packed history tiles [tb, th_end) with a kPrefetch-deep register ring:
  // the slot just consumed is refilled with the tile kPrefetch ahead
  const int th_end = min(te, NTh);
  HistRegs ring[kPrefetch];
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u)
    if (tb + u < th_end) load_hist(tb + u, ring[u]);
  __syncthreads();  // the block's q setup is complete
  for (int tile = tb; tile < th_end; tile += kPrefetch) {
#pragma unroll
    for (int u = 0; u < kPrefetch; ++u) {
      const int t = tile + u;
      if (t < th_end) {
        process_hist(ring[u], t);
        if (t + kPrefetch < th_end) load_hist(t + kPrefetch, ring[u]);
      }
    }
  }

  // ---- residual tiles: bf16 keys/values as stored (appended token from the input)
  for (int tile = max(tb, NTh); tile < te; ++tile) {
    const int t0 = (tile - NTh) * kGroup;
    const bool has_new = a.r_new >= t0 && a.r_new < t0 + kGroup;
    f32x4 accS[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int t = t0 + col_token(ct, ln);
      const int tc = min(t, a.r_total - 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        u32x4 bf = *reinterpret_cast<const u32x4*>(kr + static_cast<size_t>(tc) * D + 32 * s + 8 * lq);
        if (t >= a.r_total) bf = zero4;
        if (has_new && t == a.r_new) {
          const int c = 32 * s + 8 * lq;
          bf.x = load_bf16_pair(knp, c);
          bf.y = load_bf16_pair(knp, c + 2);
          bf.z = load_bf16_pair(knp, c + 4);
          bf.w = load_bf16_pair(knp, c + 6);
        }
        const u32x4 af = row_on ? *reinterpret_cast<const u32x4*>(ares + (s * R2 + ln) * 32 + 8 * lq) : zero4;
        accS[ct] = mfma(af, bf, accS[ct]);
      }
    }
    float x[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bool okh = 2 * lq + hh < Gb;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const bool ok = okh && t0 + col_token(ct, ln) < a.r_total;
        x[hh][ct] = ok ? (accS[ct][2 * hh] + accS[ct][2 * hh + 1]) * a.scale2 : -INFINITY;
      }
    }
    softmax_update(x);
    // values: A = p in natural token order, B = values as stored (channel-major)
    for (int i = lane; i < Gb * 16; i += 64) {
      const int h = i % Gb, pr = i / Gb;
      const Split a0 = split2(pbuf[h * 32 + 2 * pr]);
      const Split a1 = split2(pbuf[h * 32 + 2 * pr + 1]);
      const int o_hi = (2 * h) * 32 + 2 * pr, o_lo = o_hi + 32;
      *reinterpret_cast<uint32_t*>(AV + o_hi) = a0.hi | (a1.hi << 16);
      *reinterpret_cast<uint32_t*>(AV + o_lo) = a0.lo | (a1.lo << 16);
    }
    wave_sync();
    const u32x4 af = row_on ? *reinterpret_cast<const u32x4*>(AV + ln * 32 + 8 * lq) : zero4;
    const int tl = t0 + 8 * lq;                     // first token of this lane's 8 slots
    const int tlc = min(tl, (a.r_total - 1) & ~7);  // an in-range chunk for loading
    const bool clean = tl + 8 <= a.r_total && !(a.r_new >= tl && a.r_new < tl + 8);
#pragma unroll
    for (int g = 0; g < NGV; ++g) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = 32 * g + 2 * ln + u;
        u32x4 bf = *reinterpret_cast<const u32x4*>(vr + static_cast<size_t>(c) * a.r_cap + tlc);
        if (!clean) {
          // zero slots past the residual, substitute the appended token
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = tl + e;
            uint32_t hv = (bf[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            if (t == a.r_new) hv = f32_to_bf16(load_f32(vnp, c));
            else if (t >= a.r_total) hv = 0u;
            bf[e >> 1] = (bf[e >> 1] & (0xFFFF0000u >> (16 * (e & 1)))) | (hv << (16 * (e & 1)));
          }
        }
        oacc[2 * g + u] = mfma(af, bf, oacc[2 * g + u]);
      }
    }
    wave_sync();
  }

  // the wave that owns the appended token's tile stores it
  if (a.r_new >= 0 && hb == 0 && te > tb && tb <= NTh + a.r_new / kGroup && NTh + a.r_new / kGroup < te) {
    uint16_t* kw = a.k_res + (static_cast<size_t>(bj) * a.r_cap + a.r_new) * D;
    uint16_t* vw = a.v_res + static_cast<size_t>(bj) * D * a.r_cap + a.r_new;
    for (int c = lane; c < D; c += 64) {
      kw[c] = f32_to_bf16(load_f32(knp, c));
      vw[static_cast<size_t>(c) * a.r_cap] = f32_to_bf16(load_f32(vnp, c));
    }
  }

  // ---------------------------------------------------------------- merge the block's waves
  // Each wave leaves (o[Gb][D], m[Gb], l[Gb]) in its own LDS region (its operand
  // area is no longer needed); after one barrier the block combines the four.
  float* wst = reinterpret_cast<float*>(wbase);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int head = 2 * lq + hh;
    const float l = sum16(l_part[hh]);
    if (head < Gb) {
      if (ln == 0) {
        wst[Gb * D + head] = m_run[hh];
        wst[Gb * D + Gb + head] = l;
      }
#pragma unroll
      for (int g = 0; g < NGV; ++g) {
        const float corr = vcorr[g][2 * hh] + vcorr[g][2 * hh + 1];
        float2 v;
        v.x = oacc[2 * g][2 * hh] + oacc[2 * g][2 * hh + 1] + corr;
        v.y = oacc[2 * g + 1][2 * hh] + oacc[2 * g + 1][2 * hh + 1] + corr;
        *reinterpret_cast<float2*>(wst + head * D + 32 * g + 2 * ln) = v;
      }
    }
  }
  __syncthreads();
  const bool final_out = gridDim.x == 1;
  const size_t pb = (static_cast<size_t>(bjh) * gridDim.x + blockIdx.x) * kHB;
  for (int e = tid; e < Gb * D; e += kThreads) {
    const int h = e / D, c = e % D;
    float mw[kWaves], lw[kWaves], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* ws_w = reinterpret_cast<const float*>(smem + L.wave0 + w * L.wave_bytes);
      mw[w] = ws_w[Gb * D + h];
      lw[w] = ws_w[Gb * D + Gb + h];
      M = fmaxf(M, mw[w]);
    }
    float Lsum = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (lw[w] > 0.0f) {
        const float f = exp2f(mw[w] - M);
        Lsum += lw[w] * f;
        acc += f * reinterpret_cast<const float*>(smem + L.wave0 + w * L.wave_bytes)[h * D + c];
      }
    }
    if (final_out) {
      a.out[(static_cast<size_t>(b) * a.Hq + j * a.G + h0 + h) * D + c] = acc / Lsum;
    } else {
      a.part_o[(pb + h) * D + c] = acc;
      if (c == 0) a.part_ml[pb + h] = make_float2(M, Lsum);
    }
  }
}

// Combine the per-block partials of each (batch, KV head, head block): the
// split weights 2^(m_s - M)/L per head go to LDS first, then every output is an
// independent-load weighted sum over the splits.
constexpr int kMaxNb = 64;
__global__ __launch_bounds__(kThreads) void merge_kernel(const float* part_o, const float2* part_ml, float* out,
                                                         int Hq, int Hkv, int G, int HB, int D, int nb) {
  __shared__ float wgt[kHB][kMaxNb];
  const int jh = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int j = jh / HB, hb = jh % HB, h0 = hb * kHB;
  const int Gb = min(kHB, G - h0);
  const size_t base = ((static_cast<size_t>(b) * Hkv + j) * HB + hb) * nb;
  // one 64-lane wave per head: lane s holds split s
  const int wave = tid >> 6, lane = tid & 63;
  for (int h = wave; h < Gb; h += kThreads / 64) {
    const float2 ml = lane < nb ? part_ml[(base + lane) * kHB + h] : make_float2(-INFINITY, 0.0f);
    float M = ml.x;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float f = ml.y > 0.0f ? exp2f(ml.x - M) : 0.0f;
    float Lsum = f * ml.y;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) Lsum += __shfl_xor(Lsum, o);
    if (lane < nb) wgt[h][lane] = f / Lsum;
  }
  __syncthreads();
  for (int e = tid; e < Gb * D; e += kThreads) {
    const int h = e / D, c = e % D;
    const float* po = part_o + (base * kHB + h) * D + c;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 4 <= nb; s += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] += wgt[h][s + u] * po[static_cast<size_t>(s + u) * kHB * D];
    }
    for (; s < nb; ++s) acc[0] += wgt[h][s] * po[static_cast<size_t>(s) * kHB * D];
    out[(static_cast<size_t>(b) * Hq + j * G + h0 + h) * D + c] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
}

struct Plan {
  int tpw, nb;  // tiles per wave, blocks per (batch, KV head, head block)
};
// One round of resident workgroups: as many blocks per unit as fit the chip at
// once (two workgroups per CU when the kernel fits two waves per SIMD), then
// spread the unit's tiles evenly over their waves.
constexpr int kCUs = 256;
Plan plan(int NT, int units, int KS) {
  const int per_cu = (KS == 2 || KS == 4) ? 2 : 1;
  Plan p;
  int nb = std::max(1, kCUs * per_cu / units);
  nb = std::min(nb, (NT + kWaves - 1) / kWaves);  // no block without a tile
  nb = std::min(nb, kMaxNb);
  p.tpw = (NT + kWaves * nb - 1) / (kWaves * nb);
  p.nb = (NT + kWaves * p.tpw - 1) / (kWaves * p.tpw);
  return p;
}

struct WsLayout {
  size_t part_ml, part_o, total;
  int nb_max;
};
WsLayout ws_layout(const kvc_cache* c, int HB) {
  const int units = c->batch * c->kv_heads * HB;
  const int NTmax = c->q_cap / kGroup + (c->r_cap + kGroup - 1) / kGroup;
  int nmax = 1;
  // nb is not monotone in NT; take the maximum over every possible length
  for (int nt = 1; nt <= NTmax; ++nt) nmax = std::max(nmax, plan(nt, units, c->head_dim / 32).nb);
  WsLayout w;
  w.nb_max = nmax;
  w.part_ml = 0;
  w.part_o = align_up(static_cast<size_t>(units) * nmax * kHB * sizeof(float2), 256);
  w.total = w.part_o + static_cast<size_t>(units) * nmax * kHB * c->head_dim * sizeof(float);
  return w;
}

template <typename T, int BITS>
kvc_status launch_decode(const DecArgs& a, int KS, int B, hipStream_t st) {
  const int Gmax = std::min(kHB, a.G);
  const Lds L = lds_layout(KS, Gmax);
  dim3 grid(a.nb, a.Hkv * a.HB, B);
  switch (KS) {
#define KVC_CASE(k)                                                                                      \
  case k:                                                                                                \
    if (L.total > 65536) {                                                                               \
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<T, BITS, k>),     \
                                         hipFuncAttributeMaxDynamicSharedMemorySize, L.total);           \
      if (e != hipSuccess) {                                                                             \
        set_last_hip_error(e);                                                                           \
        return KVC_ERR_HIP;                                                                              \
      }                                                                                                  \
    }                                                                                                    \
    hipLaunchKernelGGL((decode_kernel<T, BITS, k>), grid, dim3(kThreads), L.total, st, a);              \
    break;
    KVC_CASE(1) KVC_CASE(2) KVC_CASE(3) KVC_CASE(4) KVC_CASE(5) KVC_CASE(6) KVC_CASE(7) KVC_CASE(8)
#undef KVC_CASE
    default: return KVC_ERR_SHAPE;
  }
  kvc_status st2 = check_launch();
  if (st2 != KVC_OK || a.nb == 1) return st2;
  hipLaunchKernelGGL(merge_kernel, dim3(a.Hkv * a.HB, B), dim3(kThreads), 0, st, a.part_o, a.part_ml, a.out,
                     a.Hq, a.Hkv, a.G, a.HB, 32 * KS, a.nb);
  return check_launch();
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
  if (Hq < 1 || Hq % Hkv != 0 || Hq / Hkv > 16) return KVC_ERR_SHAPE;
  const int G = Hq / Hkv;
  const int HB = (G + kHB - 1) / kHB;
  const WsLayout W = ws_layout(cache, HB);
  if (!ws) {
    *ws_bytes = W.total;
    return KVC_OK;
  }
  if (!q || !k_new || !v_new || !out) return KVC_ERR_NULL;
  if (*ws_bytes < W.total) return KVC_ERR_WORKSPACE;
  const int R = cache->residual;
  if (cache->r_len + 1 > cache->r_cap) return KVC_ERR_CAPACITY;
  const bool flush = (cache->r_len + 1 == R + kGroup);
  if (flush && cache->q_len + kGroup > cache->q_cap) return KVC_ERR_CAPACITY;
  hipStream_t st = static_cast<hipStream_t>(stream);

  DecArgs a;
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
  a.HB = HB;
  a.q_cap = cache->q_cap;
  a.r_cap = cache->r_cap;
  a.q_len = cache->q_len;
  const int units = cache->batch * Hkv * HB;
  const int NT = a.q_len / kGroup + (a.r_total + kGroup - 1) / kGroup;
  const Plan p = plan(NT, units, cache->head_dim / 32);
  a.tpw = p.tpw;
  a.nb = p.nb;
  char* w = static_cast<char*>(ws);
  a.part_ml = reinterpret_cast<float2*>(w + W.part_ml);
  a.part_o = reinterpret_cast<float*>(w + W.part_o);
  a.out = out;
  a.scale2 = 1.4426950408889634f / sqrtf(static_cast<float>(cache->head_dim));
  const int KS = cache->head_dim / 32;
  if (dtype == KVC_F32)
    return cache->bits == 2 ? launch_decode<float, 2>(a, KS, cache->batch, st)
                            : launch_decode<float, 4>(a, KS, cache->batch, st);
  return cache->bits == 2 ? launch_decode<uint16_t, 2>(a, KS, cache->batch, st)
                          : launch_decode<uint16_t, 4>(a, KS, cache->batch, st);
}
