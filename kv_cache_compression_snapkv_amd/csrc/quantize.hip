// Group quantization + bit packing of kept tokens (prompt compression) and the
// residual flush of a decode step.
//
// MiniKV Sec. 4.4 (INT2 quantization kernel: codes bit-shifted into INT32,
// keys along channels' token groups, values per token, fp16 scale/zero) and
// Alg. 1 (prefill Quant; decoding flush of the streaming residual); blog
// "Quantization" (KIVI grouping; recent tokens kept exact until a group fills).
//
// One workgroup owns one G-token block of one (batch, KV head), G the group size
// (32, or MiniKV's 16): the block's
// gathered keys and values are staged in LDS (bfloat16 inputs as they are,
// float32 inputs as float32; the layout is sized by a bound DM >= D so that
// small heads take little LDS), the per-channel key
// groups and per-token value groups get their fp16 scale/zero, and the codes
// are packed: keys along channels (a word holds 32/b channels of one token),
// values along tokens (a word holds 32/b tokens of one channel).
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kThreads = 256;

// Staged element as float32 (bf16 -> float32 is exact).
__device__ __forceinline__ float as_f32(float x) { return x; }
__device__ __forceinline__ float as_f32(uint16_t x) { return bf16_to_f32(x); }

// S: staged element type, DM: head-dim bound.  Rows are 16 bytes longer than
// DM elements (16-byte aligned rows; a column walk changes bank every row).
template <typename S, int DM, int G> struct QuantLds {
  static constexpr int LD = DM + 16 / sizeof(S);
  S k[G][LD];
  S v[G][LD];
  float2 kq[DM];        // per key channel: (zero, 1/scale), both 0 for a zero or non-finite scale
  float2 vq[G][DM / G];  // per value token group
};

// The 16 / sizeof(S) elements of a 16-byte LDS piece as float32.
__device__ __forceinline__ void unpack16(const uint4& w, float (&f)[8]) {  // bf16
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void unpack16(const uint4& w, float (&f)[4]) {  // float32
  f[0] = __uint_as_float(w.x);
  f[1] = __uint_as_float(w.y);
  f[2] = __uint_as_float(w.z);
  f[3] = __uint_as_float(w.w);
}
// Elements c, c+1 (c even) of a staged row as float32.
__device__ __forceinline__ float2 pair_f32(const uint16_t* p) {
  const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
  return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xFFFF0000u));
}
__device__ __forceinline__ float2 pair_f32(const float* p) { return *reinterpret_cast<const float2*>(p); }

// Code of x in a group (z, inv), as a float bit pattern: t = (x - z) * inv is
// clamped to [0, qmax] and 1.5 * 2^23 is added.  Floats in [2^23, 2^24) are
// spaced 1 apart, so the sum is that constant plus rint(t), ties to even, and
// the integer sits in the low mantissa bits; rounding commutes with a clamp to
// integer bounds.  A zero or non-finite scale has inv = 0 and z = 0, so t is 0
// for finite x: code 0.
constexpr float kRoundAdd = 12582912.0f;  // 1.5 * 2^23
constexpr uint32_t kRoundBits = 0x4B400000u;
__device__ __forceinline__ uint32_t code_bits(float x, float2 q, float qmax) {
  const float t = __fmul_rn(__fsub_rn(x, q.x), q.y);
  return __float_as_uint(__fadd_rn(fminf(fmaxf(t, 0.0f), qmax), kRoundAdd));
}
// A word is the wrapping sum of code_bits(...) << (BITS * slot) over its 32/BITS
// slots; subtracting the constant's share, code_bias, leaves the packed codes.
// add_code forms acc + (bits << shift) as one v_lshl_add_u32: the empty asm
// keeps the running sum opaque, so the compiler does not regroup the chain into
// separate shifts and three-way adds.
__device__ __forceinline__ uint32_t add_code(uint32_t acc, uint32_t bits, int shift) {
  acc += bits << shift;
  asm("" : "+v"(acc));
  return acc;
}
template <int BITS> constexpr uint32_t code_bias() {
  uint32_t c = 0;
  for (int i = 0; i < 32 / BITS; ++i) c += kRoundBits << (BITS * i);
  return c;
}

// Lane exchange within a quad: dpp_f<0xB1> gives lane l the value of lane
// l ^ 1, dpp_f<0x4E> that of l ^ 2.
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Quantize the G tokens staged in L and write them at token offset q0 of the
// (batch, KV head) slice whose base pointers are given.  Row segments and the
// group parameters are read as 16-byte LDS vectors.
template <int BITS, typename S, int DM, int G>
__device__ __forceinline__ void quantize_block(QuantLds<S, DM, G>& L, int D, int q0, uint32_t* k_codes, uint32_t* k_meta,
                               uint32_t* v_codes, uint32_t* v_meta) {
  constexpr int VEC = 16 / sizeof(S);
  const int tid = threadIdx.x;
  const float qmax = static_cast<float>((1 << BITS) - 1);
  const int ngv = D / G;
  // Extremes are exact in any order, so the groups' walks are split over lanes
  // and combined with quad-lane exchanges.  One pass over 2D items (a multiple
  // of 64, so every wave in it is whole) walks both tensors; item e then makes
  // one group: a key channel when bit 1 of e is clear, a value group when set.
  //   keys: lanes 4p..4p+3 walk channels 2p, 2p+1 over the tokens of one
  //   residue mod 4 each; lane 4p+k (k = 0, 1) makes channel 2p+k.
  //   values: within each run of 2G items, item u walks half h = bit 1 of u of
  //   group jv = e / 2G of token t = 2(u / 4) + (u & 1); lanes u and u ^ 2
  //   combine, and the h = 1 lane makes the group.
  for (int e = tid; e < 2 * D; e += kThreads) {
    const int p = e >> 2, qt = e & 3;
    float2 x = pair_f32(&L.k[qt][2 * p]);
    float lo0 = x.x, hi0 = x.x, lo1 = x.y, hi1 = x.y;
#pragma unroll
    for (int i = 1; i < G / 4; ++i) {
      x = pair_f32(&L.k[qt + 4 * i][2 * p]);
      lo0 = fminf(lo0, x.x);
      hi0 = fmaxf(hi0, x.x);
      lo1 = fminf(lo1, x.y);
      hi1 = fmaxf(hi1, x.y);
    }
    const int u = e & (2 * G - 1), jv = e / (2 * G), h = (u >> 1) & 1;
    const int t = ((u >> 2) << 1) | (u & 1);
    const uint4* seg = reinterpret_cast<const uint4*>(&L.v[t][jv * G + (G / 2) * h]);
    float f[VEC];
    unpack16(seg[0], f);
    float vlo = f[0], vhi = f[0];
#pragma unroll
    for (int q = 0; q < (G / 2) / VEC; ++q) {
      if (q) unpack16(seg[q], f);
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        vlo = fminf(vlo, f[i]);
        vhi = fmaxf(vhi, f[i]);
      }
    }
    lo0 = fminf(lo0, dpp_f<0xB1>(lo0));
    hi0 = fmaxf(hi0, dpp_f<0xB1>(hi0));
    lo1 = fminf(lo1, dpp_f<0xB1>(lo1));
    hi1 = fmaxf(hi1, dpp_f<0xB1>(hi1));
    lo0 = fminf(lo0, dpp_f<0x4E>(lo0));
    hi0 = fmaxf(hi0, dpp_f<0x4E>(hi0));
    lo1 = fminf(lo1, dpp_f<0x4E>(lo1));
    hi1 = fmaxf(hi1, dpp_f<0x4E>(hi1));
    vlo = fminf(vlo, dpp_f<0x4E>(vlo));
    vhi = fmaxf(vhi, dpp_f<0x4E>(vhi));
    const bool is_val = qt >= 2;
    const GroupQ g = make_group(is_val ? vlo : (qt ? lo1 : lo0), is_val ? vhi : (qt ? hi1 : hi0), qmax);
    if (is_val) {
      L.vq[t][jv] = make_float2(g.z, g.inv);
      v_meta[static_cast<size_t>(q0 + t) * ngv + jv] = g.meta;
    } else {
      const int c = 2 * p + qt;
      L.kq[c] = make_float2(g.z, g.inv);
      k_meta[static_cast<size_t>(q0 / G) * D + c] = g.meta;
    }
  }
  __syncthreads();
  constexpr int per = 32 / BITS;
  const int nw = D / per;  // key words per token
  // key words: word w of token t holds channels w*per.. of t; the G lanes of a
  // token block share w (their parameter reads are broadcasts)
  for (int e = tid; e < G * nw; e += kThreads) {
    const int w = e / G, t = e % G;
    const uint4* xs = reinterpret_cast<const uint4*>(&L.k[t][w * per]);
    const uint4* qs = reinterpret_cast<const uint4*>(&L.kq[w * per]);
    uint32_t word = 0;
#pragma unroll
    for (int p = 0; p < per / VEC; ++p) {
      float f[VEC];
      unpack16(xs[p], f);
#pragma unroll
      for (int i = 0; i < VEC; i += 2) {
        const uint4 qq = qs[(p * VEC + i) / 2];  // parameters of channels i, i+1 of this piece
        const int c = p * VEC + i;
        word = add_code(word, code_bits(f[i], make_float2(__uint_as_float(qq.x), __uint_as_float(qq.y)), qmax),
                        BITS * c);
        word = add_code(word, code_bits(f[i + 1], make_float2(__uint_as_float(qq.z), __uint_as_float(qq.w)), qmax),
                        BITS * (c + 1));
      }
    }
    k_codes[static_cast<size_t>(q0 + t) * nw + w] = word - code_bias<BITS>();
  }
  // value words: word row r of channel c holds tokens r*per..; lanes 2i and
  // 2i+1 take the channel pair c, c+1 (same group, same parameters) over the
  // first and the second half of the row's tokens, add their partial sums, and
  // each stores one channel's word
  constexpr int rows = G / per;  // value word rows per block
  constexpr int half = per / 2;
  const float rcp_d = __builtin_amdgcn_rcpf(static_cast<float>(D));
  for (int e = tid; e < rows * D; e += kThreads) {
    const QR rc = D == DM ? QR{static_cast<int>(static_cast<unsigned>(e) / DM), static_cast<int>(static_cast<unsigned>(e) % DM)}
                          : small_divmod(e, D, rcp_d);
    const int r = rc.q, hb = rc.r & 1, c = rc.r & ~1, j = c / G;
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const int t = r * per + hb * half + i;
      const float2 q = L.vq[t][j];
      const float2 x = pair_f32(&L.v[t][c]);
      w0 = add_code(w0, code_bits(x.x, q, qmax), BITS * i);
      w1 = add_code(w1, code_bits(x.y, q, qmax), BITS * i);
    }
    const uint32_t mine = hb ? w1 : w0, other = hb ? w0 : w1;  // this lane's channel, the partner's
    const uint32_t from = static_cast<uint32_t>(
        __builtin_amdgcn_mov_dpp(static_cast<int>(other), 0xB1, 0xF, 0xF, true));  // lane ^ 1's partial of it
    const uint32_t lo_half = hb ? from : mine, hi_half = hb ? mine : from;
    v_codes[(static_cast<size_t>(q0) / per + r) * D + c + hb] =
        lo_half + (hi_half << (BITS * half)) - code_bias<BITS>();
  }
}

struct QuantArgs {
  const void* k;
  const void* v;
  const int32_t* idx;
  int n, D, Hkv, k_sel, W, Q, T, q_cap, r_cap;
  uint32_t *k_codes, *k_meta, *v_codes, *v_meta;
  uint16_t *k_res, *v_res;
};

// Stage `count` kept tokens starting at kept index t_first (rows beyond count
// are zero) as float32 rows of L.k / L.v.  Every 16-byte load of the G rows is
// issued before the first LDS store: one memory round trip for the positions,
// one for the data.
template <typename T, int DM, int G>
__device__ __forceinline__ void stage_rows(QuantLds<T, DM, G>& L, const QuantArgs& a, int D, int bj, int t_first,
                                           int count) {
  constexpr int VEC = 16 / sizeof(T);                      // elements per 16 bytes
  constexpr int MAXV = (G * DM / VEC + kThreads - 1) / kThreads;  // pieces per thread at D = DM
  const int ppr = D / VEC, total = G * ppr;                // pieces per row, per tensor
  const T* k = static_cast<const T*>(a.k) + static_cast<size_t>(bj) * a.n * D;
  const T* v = static_cast<const T*>(a.v) + static_cast<size_t>(bj) * a.n * D;
  const int tid = threadIdx.x;
  const float rcp_ppr = __builtin_amdgcn_rcpf(static_cast<float>(ppr));
  int pos[MAXV], tt[MAXV], cc[MAXV];  // piece e: row tt, element cc
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int e = tid + i * kThreads;
    constexpr unsigned kp = DM / VEC;
    const QR rc = D == DM ? QR{static_cast<int>(static_cast<unsigned>(e) / kp),
                               static_cast<int>(static_cast<unsigned>(e) % kp)}
                          : small_divmod(e, ppr, rcp_ppr);
    tt[i] = rc.q;
    cc[i] = rc.r * VEC;
  }
  // Kept token t is selected position idx[t] for t < k_sel, then the window;
  // positions are clamped into the prompt so that a malformed idx cannot
  // address outside k/v.  Every idx entry a thread needs is requested before
  // any is used (the entry index is clamped into the selection, so each load is
  // in bounds): one round trip.
  int raw[MAXV];
  const bool from_idx = a.idx != nullptr && a.k_sel > 0;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) raw[i] = 0;
  if (from_idx) {
    const int32_t* ib = a.idx + static_cast<size_t>(bj) * a.k_sel;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) raw[i] = ib[min(t_first + tt[i], a.k_sel - 1)];
  }
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int e = tid + i * kThreads, t = t_first + tt[i];
    const int p = a.idx == nullptr ? t : (t < a.k_sel ? raw[i] : a.n - a.W + (t - a.k_sel));
    pos[i] = (e < total && tt[i] < count) ? min(max(p, 0), a.n - 1) : 0;
  }
  uint4 kv[MAXV], vv[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int e = tid + i * kThreads;
    const size_t src = static_cast<size_t>(pos[i]) * D + cc[i];
    kv[i] = vv[i] = make_uint4(0, 0, 0, 0);
    if (e < total && tt[i] < count) {
      kv[i] = *reinterpret_cast<const uint4*>(k + src);
      vv[i] = *reinterpret_cast<const uint4*>(v + src);
    }
  }
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int e = tid + i * kThreads;
    if (e < total) {
      *reinterpret_cast<uint4*>(&L.k[tt[i]][cc[i]]) = kv[i];
      *reinterpret_cast<uint4*>(&L.v[tt[i]][cc[i]]) = vv[i];
    }
  }
}

// One workgroup's block; D is the head dimension (the constant DM when they are
// equal, so that the index arithmetic and loop bounds fold at compile time).
template <typename T, int BITS, int DM, int G>
__device__ __forceinline__ void quantize_body(QuantLds<T, DM, G>& L, const QuantArgs& a, int D) {
  const int blk = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int bj = b * a.Hkv + j;
  const int tid = threadIdx.x;
  const int nqb = a.Q / G;
  if (blk < nqb) {
    const int t0 = blk * G;
    stage_rows<T, DM, G>(L, a, D, bj, t0, G);
    __syncthreads();
    const size_t qc = a.q_cap;
    quantize_block<BITS>(L, D, t0, a.k_codes + static_cast<size_t>(bj) * qc * (D * BITS / 32),
                         a.k_meta + static_cast<size_t>(bj) * (qc / G) * D,
                         a.v_codes + static_cast<size_t>(bj) * (qc * BITS / 32) * D,
                         a.v_meta + static_cast<size_t>(bj) * qc * (D / G));
  } else {
    // residual: kept tokens [Q, T) -> bf16 ring rows 0..T-Q-1
    const int r0 = (blk - nqb) * G;
    const int nr = min(G, a.T - a.Q - r0);
    stage_rows<T, DM, G>(L, a, D, bj, a.Q + r0, nr);
    __syncthreads();
    uint16_t* kr = a.k_res + static_cast<size_t>(bj) * a.r_cap * D;  // [r_cap][D]
    uint16_t* vr = a.v_res + static_cast<size_t>(bj) * D * a.r_cap;  // [D][r_cap]
    // keys token-major, values channel-major; 8 bf16 (16 bytes) per store
    for (int e = tid; e < nr * (D / 8); e += kThreads) {
      const int t = e / (D / 8), c = (e % (D / 8)) * 8;
      uint4 w;
      auto bf = [&](int cc) { return static_cast<uint32_t>(f32_to_bf16(as_f32(L.k[t][cc]))); };
      w.x = bf(c) | (bf(c + 1) << 16);
      w.y = bf(c + 2) | (bf(c + 3) << 16);
      w.z = bf(c + 4) | (bf(c + 5) << 16);
      w.w = bf(c + 6) | (bf(c + 7) << 16);
      *reinterpret_cast<uint4*>(kr + static_cast<size_t>(r0 + t) * D + c) = w;
    }
    const int nc8 = (nr + 7) / 8;  // 8-token chunks (r0 and r_cap are multiples of 8)
    for (int e = tid; e < D * nc8; e += kThreads) {
      const int c = e / nc8, t8 = (e % nc8) * 8;
      uint16_t h[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) h[u] = f32_to_bf16(as_f32(L.v[t8 + u][c]));
      uint16_t* dst = vr + static_cast<size_t>(c) * a.r_cap + r0 + t8;
      if (t8 + 8 <= nr) {
        uint4 w;
        w.x = h[0] | (static_cast<uint32_t>(h[1]) << 16);
        w.y = h[2] | (static_cast<uint32_t>(h[3]) << 16);
        w.z = h[4] | (static_cast<uint32_t>(h[5]) << 16);
        w.w = h[6] | (static_cast<uint32_t>(h[7]) << 16);
        *reinterpret_cast<uint4*>(dst) = w;
      } else {
        for (int u = 0; t8 + u < nr; ++u) dst[u] = h[u];
      }
    }
  }
}

template <typename T, int BITS, int DM, int G>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs a) {
  __shared__ __attribute__((aligned(16))) QuantLds<T, DM, G> L;
  if (a.D == DM) quantize_body<T, BITS>(L, a, DM);
  else quantize_body<T, BITS>(L, a, a.D);
}

struct FlushArgs {
  const void* k_new;
  const void* v_new;
  int D, Hkv, R, r_old, r_start, q_len, q_cap, r_cap;
  int store_new;  // the appended token stays in the ring (it is in no flushed group)
  uint32_t *k_codes, *k_meta, *v_codes, *v_meta;
  uint16_t *k_res, *v_res;
};

// Decode-step flush of gridDim.z groups: the residual ring held r_old tokens
// and the appended token makes it r_old+1.  Group i (blockIdx.z) quantizes ring
// tokens i*G .. i*G+G-1 (the appended token, from the inputs, when it falls in
// that range) and appends them to the packed history at q_len + i*G.  With one
// group (the default policy) the ring held R+G-1 and the appended token takes
// ring row r_start + r_old unless R == 0; with R/G groups (the whole-residual
// policy) the appended token is the last group's last token.  The host then
// advances r_start by G times the group count.  Keys are staged with 16-byte
// row loads, values with 16-byte loads of 8 consecutive ring rows of one channel
// (r_start and r_cap are multiples of 8, so such a chunk never wraps).
template <typename T, int BITS, int DM, int G>
__device__ __forceinline__ void flush_body(QuantLds<uint16_t, DM, G>& L, const FlushArgs& a, int D) {
  const int j = blockIdx.x, b = blockIdx.y, grp = blockIdx.z;
  const int bj = b * a.Hkv + j;
  const int tid = threadIdx.x;
  const int t_first = grp * G;          // first residual token of this group
  const int r_new = a.r_old - t_first;  // the appended token's index inside this group's tokens
  const T* kn = static_cast<const T*>(a.k_new) + static_cast<size_t>(bj) * D;
  const T* vn = static_cast<const T*>(a.v_new) + static_cast<size_t>(bj) * D;
  uint16_t* kr = a.k_res + static_cast<size_t>(bj) * a.r_cap * D;  // [r_cap][D]
  uint16_t* vr = a.v_res + static_cast<size_t>(bj) * D * a.r_cap;  // [D][r_cap]
  auto ring = [&](int t) {  // residual token t (t < r_cap) -> ring row
    const int p = a.r_start + t;
    return p >= a.r_cap ? p - a.r_cap : p;
  };
  const int cpr = D / 8;  // 16-byte chunks per key row
  for (int e = tid; e < G * cpr; e += kThreads) {
    const int t = e / cpr, c8 = (e % cpr) * 8;
    *reinterpret_cast<uint4*>(&L.k[t][c8]) =
        *reinterpret_cast<const uint4*>(kr + static_cast<size_t>(ring(t_first + t)) * D + c8);
  }
  for (int e = tid; e < D * (G / 8); e += kThreads) {
    const int c = e / (G / 8), t8 = (e % (G / 8)) * 8;
    const uint4 w = *reinterpret_cast<const uint4*>(vr + static_cast<size_t>(c) * a.r_cap + ring(t_first + t8));
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      L.v[t8 + 2 * i][c] = static_cast<uint16_t>(ws[i] & 0xFFFFu);
      L.v[t8 + 2 * i + 1][c] = static_cast<uint16_t>(ws[i] >> 16);
    }
  }
  __syncthreads();
  // the appended token: quantized with the group it falls in, or stored in the
  // ring (by the first group only)
  if (r_new < G || (a.store_new && grp == 0)) {
    for (int c = tid; c < D; c += kThreads) {
      const uint16_t kb = f32_to_bf16(load_f32(kn, c)), vb = f32_to_bf16(load_f32(vn, c));
      if (r_new < G) {
        L.k[r_new][c] = kb;
        L.v[r_new][c] = vb;
      } else {
        const int p = ring(a.r_old);
        kr[static_cast<size_t>(p) * D + c] = kb;
        vr[static_cast<size_t>(c) * a.r_cap + p] = vb;
      }
    }
  }
  __syncthreads();
  const size_t qc = a.q_cap;
  quantize_block<BITS>(L, D, a.q_len + t_first, a.k_codes + static_cast<size_t>(bj) * qc * (D * BITS / 32),
                       a.k_meta + static_cast<size_t>(bj) * (qc / G) * D,
                       a.v_codes + static_cast<size_t>(bj) * (qc * BITS / 32) * D,
                       a.v_meta + static_cast<size_t>(bj) * qc * (D / G));
}

template <typename T, int BITS, int DM, int G>
__global__ __launch_bounds__(kThreads) void flush_kernel(FlushArgs a) {
  __shared__ __attribute__((aligned(16))) QuantLds<uint16_t, DM, G> L;  // the ring holds bf16
  if (a.D == DM) flush_body<T, BITS>(L, a, DM);
  else flush_body<T, BITS>(L, a, a.D);
}

// Head-dim bound of the LDS layout.
int dm_for(int D) { return D <= 64 ? 64 : D <= 128 ? 128 : 256; }

template <typename T, int G>
void launch_quantize_g(const QuantArgs& a, int bits, dim3 grid, hipStream_t st) {
  const int dm = dm_for(a.D);
#define KVC_Q(B_, DM_) hipLaunchKernelGGL((quantize_kernel<T, B_, DM_, G>), grid, dim3(kThreads), 0, st, a)
  if (bits == 2) {
    if (dm == 64) KVC_Q(2, 64); else if (dm == 128) KVC_Q(2, 128); else KVC_Q(2, 256);
  } else {
    if (dm == 64) KVC_Q(4, 64); else if (dm == 128) KVC_Q(4, 128); else KVC_Q(4, 256);
  }
#undef KVC_Q
}

template <typename T>
kvc_status launch_quantize(const QuantArgs& a, int bits, int group, int B, hipStream_t st) {
  const int nblk = a.Q / group + (a.T - a.Q + group - 1) / group;
  if (nblk == 0) return KVC_OK;
  dim3 grid(nblk, a.Hkv, B);
  if (group == 16) launch_quantize_g<T, 16>(a, bits, grid, st);
  else launch_quantize_g<T, kGroup>(a, bits, grid, st);
  return check_launch();
}

}  // namespace

// Flush of ngroups groups of the cache's group size (1, or R/g with the
// whole-residual policy) in one launch; c is the state before the decode step.
kvc_status launch_flush(const kvc_cache* c, int ngroups, const void* k_new, const void* v_new, kvc_dtype dt,
                        hipStream_t st) {
  FlushArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.D = c->head_dim;
  a.Hkv = c->kv_heads;
  a.R = c->residual;
  a.r_old = c->r_len;
  a.r_start = c->r_start;
  a.q_len = c->q_len;
  a.q_cap = c->q_cap;
  a.r_cap = c->r_cap;
  a.k_codes = c->k_codes;
  a.k_meta = c->k_meta;
  a.v_codes = c->v_codes;
  a.v_meta = c->v_meta;
  a.k_res = c->k_res;
  a.v_res = c->v_res;
  a.store_new = c->r_len - (ngroups - 1) * cache_group(c) >= cache_group(c);
  dim3 grid(c->kv_heads, c->batch, ngroups);
  const int dm = dm_for(a.D);
  const bool g16 = cache_group(c) == 16;
#define KVC_FG(T_, B_, G_)                                                                                     \
  do {                                                                                                         \
    if (dm == 64) hipLaunchKernelGGL((flush_kernel<T_, B_, 64, G_>), grid, dim3(kThreads), 0, st, a);        \
    else if (dm == 128) hipLaunchKernelGGL((flush_kernel<T_, B_, 128, G_>), grid, dim3(kThreads), 0, st, a); \
    else hipLaunchKernelGGL((flush_kernel<T_, B_, 256, G_>), grid, dim3(kThreads), 0, st, a);                \
  } while (0)
#define KVC_F(T_, B_)                     \
  do {                                    \
    if (g16) KVC_FG(T_, B_, 16);          \
    else KVC_FG(T_, B_, kGroup);          \
  } while (0)
  if (dt == KVC_F32) {
    if (c->bits == 2) KVC_F(float, 2); else KVC_F(float, 4);
  } else {
    if (c->bits == 2) KVC_F(uint16_t, 2); else KVC_F(uint16_t, 4);
  }
#undef KVC_F
#undef KVC_FG
  return check_launch();
}

bool cache_ok(const kvc_cache* c) {
  return c && c->k_codes && c->k_meta && c->v_codes && c->v_meta && c->k_res && c->v_res;
}

kvc_status cache_shape_status(const kvc_cache* c) {
  if ((c->bits != 2 && c->bits != 4) || !group_ok(c->group)) return KVC_ERR_BITS;
  const int g = cache_group(c);
  if (c->batch < 1 || c->kv_heads < 1 || !head_dim_ok(c->head_dim) || c->residual < 0 ||
      c->q_cap < 0 || c->q_cap % kGroup != 0 || c->r_cap < 0 || c->r_cap % 8 != 0 || c->q_len < 0 || c->r_len < 0 ||
      c->q_len % g != 0)
    return KVC_ERR_SHAPE;
  if (c->r_start < 0 || c->r_start % 8 != 0 || (c->r_cap > 0 && c->r_start >= c->r_cap)) return KVC_ERR_SHAPE;
  if (c->flush_all != 0 && (c->flush_all != 1 || c->residual < g || c->residual % g != 0)) return KVC_ERR_SHAPE;
  if (c->q_len > c->q_cap || c->r_len > c->r_cap || c->r_cap < c->residual + g)
    return KVC_ERR_CAPACITY;
  return KVC_OK;
}

}  // namespace kvc

extern "C" kvc_status kvc_quantize(const void* k, const void* v, kvc_dtype dtype, int32_t n,
                                   const int32_t* idx, int32_t k_sel, int32_t W, kvc_cache* cache,
                                   void* stream) {
  using namespace kvc;
  if (!k || !v || !cache_ok(cache)) return KVC_ERR_NULL;
  if (!dtype_ok(dtype)) return KVC_ERR_DTYPE;
  kvc_status s = cache_shape_status(cache);
  if (s != KVC_OK) return s;
  if (n < 1) return KVC_ERR_SHAPE;
  int T;
  if (idx) {
    if (W < 1 || W > n || k_sel < 0 || k_sel > n - W) return KVC_ERR_SHAPE;
    T = k_sel + W;
  } else {
    T = n;
  }
  if (cache->q_len != 0 || cache->r_len != 0) return KVC_ERR_CAPACITY;
  const int R = cache->residual;
  const int g = cache_group(cache);
  const int Q = cache->flush_all ? g * (T / g) : g * (std::max(T - R, 0) / g);
  if (Q > cache->q_cap || T - Q > cache->r_cap) return KVC_ERR_CAPACITY;
  QuantArgs a;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.n = n;
  a.D = cache->head_dim;
  a.Hkv = cache->kv_heads;
  a.k_sel = idx ? k_sel : 0;
  a.W = idx ? W : 0;
  a.Q = Q;
  a.T = T;
  a.q_cap = cache->q_cap;
  a.r_cap = cache->r_cap;
  a.k_codes = cache->k_codes;
  a.k_meta = cache->k_meta;
  a.v_codes = cache->v_codes;
  a.v_meta = cache->v_meta;
  a.k_res = cache->k_res;
  a.v_res = cache->v_res;
  hipStream_t st = static_cast<hipStream_t>(stream);
  s = dtype == KVC_F32 ? launch_quantize<float>(a, cache->bits, g, cache->batch, st)
                       : launch_quantize<uint16_t>(a, cache->bits, g, cache->batch, st);
  if (s != KVC_OK) return s;
  cache->q_len = Q;
  cache->r_len = T - Q;
  cache->r_start = 0;
  return KVC_OK;
}
