// Prefill attention that also returns the attention each key accumulates
// (MiniKV Sec. 4.3 "Selective KV Compatible Attention Kernels", Fig. 9: a
// FlashAttention-style prefill with a second output, the attention summed along
// each key column, at O(l_key) extra memory).  Query head h reads KV head h / G.
//
// The column sums here are of the *normalized* causal probabilities (H2O's
// accumulated attention, the ranking the blog's "Eviction" section and
// PyramidKV's "Baselines" describe).  MiniKV's kernel leaves each row's
// normalization out; normalizing needs only the row's log-sum-exp, n floats per
// head, which the forward pass produces anyway.  So the work is two passes:
//
//   fa_fwd_kernel   FlashAttention forward: O = softmax(Q K^T / sqrt(D)) V row
//                   by row (causal), plus lse_r = m_r + log2(l_r) in log2 units.
//   colsum_kernel   one workgroup per 64-key block of a KV head walks every
//                   later query row of the G heads, recomputes the logits and
//                   adds 2^(x - lse_r) per key: A_cumul in a fixed order (no
//                   atomics, deterministic).
//
// Contractions on MFMA.  Scores are computed transposed, S^T = K Q^T (A = key
// rows, B = query rows; bf16: v_mfma_f32_16x16x32_bf16, fp32: 16x16x4 f32), so
// a lane ends up holding query row ln and keys 4*lq..4*lq+3 of each 16-key
// tile -- exactly the k-slots the product O^T = V^T P^T takes as its B operand
// when the 32 keys of a tile are ordered (4lq..4lq+3, 16+4lq..16+4lq+3) per lane
// quarter; the A operand V^T then comes from a transposed copy of the value
// tile in LDS.  With bf16 inputs P is carried as a bf16 truncation plus a bf16
// remainder (two MFMAs, about 16 significant bits); fp32 inputs use the fp32
// MFMA on P as is.
#include <algorithm>

#include "kvc_internal.h"

namespace kvc {

kvc_status launch_variance(const float* raw, int rows, int N, float* var, hipStream_t st);  // select.hip

namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kKT = 32;       // keys per staged tile (forward pass)
constexpr int kColKeys = 64;  // keys per wave (column-sum pass; kPfWaves blocks per workgroup)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Eight k-slots of one lane for one 32-wide MFMA step (32 dims, or 32 keys).
template <typename T> struct Frag;
template <> struct Frag<uint16_t> {
  u32x4 v;  // slot e in half e%2 of register e/2
  __device__ __forceinline__ void load8(const unsigned char* p) { v = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void load4x2(const unsigned char* p0, const unsigned char* p1) {
    const u32x2 a = *reinterpret_cast<const u32x2*>(p0), b = *reinterpret_cast<const u32x2*>(p1);
    v = u32x4{a.x, a.y, b.x, b.y};
  }
  __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
};
template <> struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void load8(const unsigned char* p) {
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 16);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ void load4x2(const unsigned char* p0, const unsigned char* p1) {
    const float4 a = *reinterpret_cast<const float4*>(p0), b = *reinterpret_cast<const float4*>(p1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
};

// Two transposing 8-byte LDS reads (ds_read_b64_tr_b16: within each quarter of
// the wave, lane i receives element e of the read of lane 4e + i/4, element
// i%4), joined into one 8-slot fragment.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 tr_pair(const unsigned char* p0, const unsigned char* p1) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua.x, ua.y, ub.x, ub.y};
}

// acc[row 4*lq+i][col ln] += sum over the 8 k-slots of every lane quarter.
__device__ __forceinline__ f32x4 mma(const Frag<uint16_t>& a, const Frag<uint16_t>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v), __builtin_bit_cast(bf16x8, b.v),
                                                 c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<float>& a, const Frag<float>& b, f32x4 c) {
#pragma unroll
  for (int u = 0; u < 8; ++u) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[u], b.v[u], c, 0, 0, 0);
  return c;
}

// P operands from the 8 probabilities of a lane (slot e: p[e]).  bf16: hi =
// truncation, lo = truncation of the remainder; fp32: as is (lo unused).
constexpr uint32_t kHi = 0xFFFF0000u;
constexpr uint32_t kHighHalves = 0x07060302u;  // v_perm: high halves of (src1, src0)
__device__ __forceinline__ void p_frags(const float (&p)[8], Frag<uint16_t>& hi, Frag<uint16_t>& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t u0 = __float_as_uint(p[2 * m]), u1 = __float_as_uint(p[2 * m + 1]);
    const float r0 = p[2 * m] - __uint_as_float(u0 & kHi), r1 = p[2 * m + 1] - __uint_as_float(u1 & kHi);
    h[m] = __builtin_amdgcn_perm(u1, u0, kHighHalves);
    l[m] = __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), kHighHalves);
  }
  hi.v = u32x4{h[0], h[1], h[2], h[3]};
  lo.v = u32x4{l[0], l[1], l[2], l[3]};
}
__device__ __forceinline__ void p_frags(const float (&p)[8], Frag<float>& hi, Frag<float>&) {
#pragma unroll
  for (int e = 0; e < 8; ++e) hi.v[e] = p[e];
}

// All-reduce over the 16 lanes of a DPP row.
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}
// Over the four lanes ln, ln+16, ln+32, ln+48 (the lanes that share a query row).
__device__ __forceinline__ float max_q(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float sum_q(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

struct PfArgs {
  const void *q, *k, *v;  // [B][Hq][n][D], [B][Hkv][n][D] x2
  float* out;             // [B][Hq][n][D]
  float* lse;             // [B][Hq][n] m + log2(l), log2 units
  float* lse_out;         // [B][Hq][n] the same in natural-log units, or null
  float* acc;             // [B][Hkv][n]
  int B, Hq, Hkv, G, n, Gc, ngr, nrb, units;
  float scale2;           // log2(e)/sqrt(D)
};

// LDS staging of one key tile: keys row-major (rows padded by 16 bytes, so the
// 16 lanes reading 16-byte pieces of 16 different rows hit distinct banks) and
// values transposed, channel-major (rows padded by 8 or 16 bytes).
template <typename T, int KS> struct PfGeom {
  static constexpr int D = 32 * KS;
  static constexpr int ES = sizeof(T);
  static constexpr int KROW = D * ES + 16;
  // bf16 values are staged row-major like the keys (rows 32 bytes longer: the
  // transposing reads of 4 rows x 32 bytes by 16 lanes then cover all banks);
  // fp32 values transposed, channel-major
  static constexpr bool VTR = ES == 2;
  static constexpr int VROW = VTR ? D * ES + 32 : kKT * ES + 16;
  static constexpr int VOFF = kKT * KROW;
  static constexpr int STAGE = VOFF + (VTR ? kKT : D) * VROW;
  static constexpr int PIECES = D * ES / 16;            // 16-byte pieces per key row
  static constexpr int KLOADS = (kKT * PIECES + kPfThreads - 1) / kPfThreads;
  // (key pair, piece) items, key pair fastest: the transposed stores of one
  // channel by the lanes of a wave then fall in distinct bank pairs (with the
  // piece fastest, lanes 8 channel rows apart shared two bank groups)
  static constexpr int VITEMS = (kKT / 2) * PIECES;
  static constexpr int VLOADS = (VITEMS + kPfThreads - 1) / kPfThreads;
};

// Forward pass.  Workgroup: 4 waves, one KV head; wave w takes query head
// hg*Gc + w%Gc and 32 rows r0 + 32*(w/Gc) .. (Gc = 4, 2 or 1 heads of the group,
// so the 4 waves share every staged key/value tile).  Grid (units, row blocks):
// consecutive workgroups are different units (KV head, head group), so with 8
// units per sequence each accelerator die's L2 serves one KV head; the row
// blocks run last-first (the longest causal ranges start first).
// Three workgroups per CU for 16-bit inputs (168 VGPRs, no spill at D = 128): a
// third wave per SIMD overlaps more of the others' softmax with products.  fp32
// inputs keep two (their D = 128 fragments would spill).
template <typename T, int KS>
__global__ __launch_bounds__(kPfThreads, sizeof(T) == 2 ? 3 : 2) void fa_fwd_kernel(PfArgs a) {
  using Gm = PfGeom<T, KS>;
  constexpr int D = Gm::D, ES = Gm::ES;
  constexpr int NCT = D / 16;  // channel tiles of the output
  constexpr bool SPLIT = ES == 2;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int ln = lane & 15, lq = lane >> 4;
  const int unit = blockIdx.x, rb = a.nrb - 1 - static_cast<int>(blockIdx.y);
  const int bj = unit / a.ngr, hg = unit % a.ngr;  // (b, KV head), head group
  const int b = bj / a.Hkv, j = bj % a.Hkv;
  const int h = j * a.G + hg * a.Gc + wave % a.Gc;
  const int RB = 32 * (kPfWaves / a.Gc);
  const int r0 = rb * RB;
  const int wr0 = r0 + 32 * (wave / a.Gc);
  const int n = a.n;
  const int last_key = min(r0 + RB - 1, n - 1);
  const int nkt = last_key / kKT + 1;
  const bool active = wr0 < n;
  const int wkt_last = min(wr0 + 31, n - 1) / kKT;  // this wave's last key tile (causal)

  const unsigned char* kg = static_cast<const unsigned char*>(a.k) + static_cast<size_t>(bj) * n * D * ES;
  const unsigned char* vg = static_cast<const unsigned char*>(a.v) + static_cast<size_t>(bj) * n * D * ES;
  const size_t qrow0 = (static_cast<size_t>(b) * a.Hq + h) * n;

  // the wave's queries: rows wr0 + 16 rs + ln, dims 32 s + 8 lq ..
  Frag<T> qf[2][KS];
#pragma unroll
  for (int rs = 0; rs < 2; ++rs) {
    const int row = wr0 + 16 * rs + ln;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (row < n)
        qf[rs][s].load8(static_cast<const unsigned char*>(a.q) + ((qrow0 + row) * D + 32 * s + 8 * lq) * ES);
      else
        qf[rs][s].zero();
    }
  }

  // staging of tile t into registers, then into LDS buffer `buf`
  u32x4 kst[Gm::KLOADS], vst[Gm::VTR ? 1 : Gm::VLOADS][2], vrow[Gm::KLOADS];
  auto fetch = [&](int t) {
    const int kb = t * kKT;
#pragma unroll
    for (int u = 0; u < Gm::KLOADS; ++u) {
      const int e = tid + kPfThreads * u;
      const int key = e / Gm::PIECES, pc = e % Gm::PIECES;
      kst[u] = u32x4{0u, 0u, 0u, 0u};
      if (e < kKT * Gm::PIECES && kb + key < n)
        kst[u] = *reinterpret_cast<const u32x4*>(kg + (static_cast<size_t>(kb + key) * D * ES) + 16 * pc);
    }
    if constexpr (Gm::VTR) {
#pragma unroll
      for (int u = 0; u < Gm::KLOADS; ++u) {
        const int e = tid + kPfThreads * u;
        const int key = e / Gm::PIECES, pc = e % Gm::PIECES;
        vrow[u] = u32x4{0u, 0u, 0u, 0u};
        if (e < kKT * Gm::PIECES && kb + key < n)
          vrow[u] = *reinterpret_cast<const u32x4*>(vg + (static_cast<size_t>(kb + key) * D * ES) + 16 * pc);
      }
    } else {
#pragma unroll
      for (int u = 0; u < Gm::VLOADS; ++u) {
        const int e = tid + kPfThreads * u;
        const int kp = e % (kKT / 2), pc = e / (kKT / 2);  // key pair fastest
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          vst[u][w] = u32x4{0u, 0u, 0u, 0u};
          if (e < Gm::VITEMS && kb + 2 * kp + w < n)
            vst[u][w] = *reinterpret_cast<const u32x4*>(vg + (static_cast<size_t>(kb + 2 * kp + w) * D * ES) + 16 * pc);
        }
      }
    }
  };
  auto stash = [&](int buf) {
    unsigned char* Ks = smem + buf * Gm::STAGE;
    unsigned char* Vt = Ks + Gm::VOFF;
#pragma unroll
    for (int u = 0; u < Gm::KLOADS; ++u) {
      const int e = tid + kPfThreads * u;
      if (e < kKT * Gm::PIECES) {
        *reinterpret_cast<u32x4*>(Ks + (e / Gm::PIECES) * Gm::KROW + 16 * (e % Gm::PIECES)) = kst[u];
        if constexpr (Gm::VTR)
          *reinterpret_cast<u32x4*>(Vt + (e / Gm::PIECES) * Gm::VROW + 16 * (e % Gm::PIECES)) = vrow[u];
      }
    }
    if constexpr (!Gm::VTR) {
#pragma unroll
      for (int u = 0; u < Gm::VLOADS; ++u) {
        const int e = tid + kPfThreads * u;
        if (e < Gm::VITEMS) {
          const int kp = e % (kKT / 2), pc = e / (kKT / 2);  // key pair fastest
          // 4 channels of keys 2kp, 2kp+1: two dwords per channel
#pragma unroll
          for (int c = 0; c < 4; ++c)
            *reinterpret_cast<u32x2*>(Vt + (4 * pc + c) * Gm::VROW + 8 * kp) = u32x2{vst[u][0][c], vst[u][1][c]};
        }
      }
    }
  };

  f32x4 oacc[NCT][2];
#pragma unroll
  for (int c = 0; c < NCT; ++c) oacc[c][0] = oacc[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.f, 0.f};

  auto compute = [&](int buf, int t) {
    const unsigned char* Ks = smem + buf * Gm::STAGE;
    const unsigned char* Vt = Ks + Gm::VOFF;
    const int kb = t * kKT;
    f32x4 s[2][2];  // [key subtile][row subtile]
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt][0] = s[kt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sx = 0; sx < KS; ++sx) {
        Frag<T> kf;
        kf.load8(Ks + (16 * kt + ln) * Gm::KROW + (32 * sx + 8 * lq) * ES);
        s[kt][0] = mma(kf, qf[0][sx], s[kt][0]);
        s[kt][1] = mma(kf, qf[1][sx], s[kt][1]);
      }
    }
    // log2-scaled logits; causal and length masks only where a key can pass a
    // row of this wave or the end of the prompt
    const bool need_mask = kb + kKT - 1 > wr0 || kb + kKT > n;
    float p[2][8];  // [row subtile][slot]: slot e < 4 key 4lq+e, e >= 4 key 16+4lq+e-4
    float alpha[2];
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) {
      const int row = wr0 + 16 * rs + ln;
      float mt = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kt = e >> 2, i = e & 3;
        float x = s[kt][rs][i];
        if (need_mask) {
          const int key = kb + 16 * kt + 4 * lq + i;
          if (key > row || key >= n) x = -INFINITY;
        }
        p[rs][e] = x;
        mt = fmaxf(mt, x);
      }
      mt = max_q(mt) * a.scale2;
      const float mnew = fmaxf(m_run[rs], mt);
      const float msafe = mnew == -INFINITY ? 0.0f : mnew;
      alpha[rs] = __builtin_amdgcn_exp2f(m_run[rs] - msafe);
      float ls = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[rs][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(p[rs][e], a.scale2, -msafe));
        ls += p[rs][e];
      }
      l_part[rs] = l_part[rs] * alpha[rs] + ls;
      m_run[rs] = mnew;
    }
    if (__any(alpha[0] != 1.0f || alpha[1] != 1.0f)) {
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) oacc[c][rs] *= alpha[rs];
    }
    Frag<T> ph[2], pl[2];
    p_frags(p[0], ph[0], pl[0]);
    p_frags(p[1], ph[1], pl[1]);
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      Frag<T> vf;
      if constexpr (Gm::VTR) {
        // A = V^T: lane (ln, lq) takes channel 16c + ln of keys 4lq..4lq+3 and
        // 16+4lq..16+4lq+3.  A transposing LDS read gives lane ln of a lane
        // quarter element e of lane 4e + ln/4's 8-byte read, so lane j of the
        // quarter reads channels 16c + 4(j%4) .. +3 of key 4lq + j/4 (+16).
        const unsigned char* va = Vt + (4 * lq + (ln >> 2)) * Gm::VROW + (16 * c + 4 * (ln & 3)) * ES;
        vf.v = tr_pair(va, va + 16 * Gm::VROW);
      } else {
        const unsigned char* vr = Vt + (16 * c + ln) * Gm::VROW;
        vf.load4x2(vr + 4 * lq * ES, vr + (16 + 4 * lq) * ES);
      }
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) {
        oacc[c][rs] = mma(vf, ph[rs], oacc[c][rs]);
        if constexpr (SPLIT) oacc[c][rs] = mma(vf, pl[rs], oacc[c][rs]);
      }
    }
  };

  fetch(0);
  stash(0);
  __syncthreads();
  for (int t = 0; t < nkt; ++t) {
    const bool more = t + 1 < nkt;
    if (more) fetch(t + 1);
    if (active && t <= wkt_last) compute(t & 1, t);
    if (more) stash((t + 1) & 1);
    __syncthreads();
  }
  if (!active) return;

  // O = o / l; lse = m + log2(l); lanes of quarter lq hold channels 16c+4lq..+3
#pragma unroll
  for (int rs = 0; rs < 2; ++rs) {
    const int row = wr0 + 16 * rs + ln;
    const float l = sum_q(l_part[rs]);
    if (row < n) {
      const float inv = 1.0f / l;
      float* o = a.out + (qrow0 + row) * D + 4 * lq;
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const f32x4 v = oacc[c][rs] * inv;
        *reinterpret_cast<float4*>(o + 16 * c) = make_float4(v[0], v[1], v[2], v[3]);
      }
      if (lq == 0) {
        const float lse2 = m_run[rs] + __log2f(l);
        a.lse[qrow0 + row] = lse2;
        if (a.lse_out) a.lse_out[qrow0 + row] = lse2 * 0.6931471805599453f;  // ln 2
      }
    }
  }
}

// Column sums.  Workgroup: kPfWaves x 64 keys of one (b, KV head); wave w holds
// keys key0 + 64w .. +63 as MFMA A operands.  The (16-row tile, head) items with
// rows >= key0 are taken in stages of kPfWaves / WPI items: each wave (or pair
// of waves for fp32) copies one item's query tile and row lse values into LDS,
// double-buffered with one barrier per stage, and all four waves read every
// staged tile, so the query rows are fetched once per 256 keys rather than once
// per 64.  A wave skips the items whose rows all lie above its keys, and only
// items that reach past one of its keys (or past n) take the masked path.  Each
// lane adds 2^(x - lse_row) for its keys over the items in order, then the 16
// lanes of a key are summed in a fixed order: deterministic, no atomics.  Grid
// (B*Hkv, key blocks) as in the forward pass.
template <typename T, int KS>
__global__ __launch_bounds__(kPfThreads, 2) void colsum_kernel(PfArgs a) {
  constexpr int D = 32 * KS, ES = sizeof(T);
  constexpr int WPI = ES == 2 ? 1 : 2;          // waves copying one item
  constexpr int NI = kPfWaves / WPI;            // items per stage
  constexpr int ROW = D * ES + 16;              // padded LDS row pitch, bytes
  constexpr int ITEM = 16 * ROW;
  constexpr int PIECES = D * ES / 16;           // 16-byte pieces per row
  constexpr int LOADS = 16 * PIECES / (64 * WPI);  // = KS copies per lane
  static_assert(LOADS * 64 * WPI == 16 * PIECES, "item copy split");
  __shared__ __attribute__((aligned(16))) unsigned char qs[2][NI * ITEM];
  __shared__ float ls[2][NI * 16];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int ln = lane & 15, lq = lane >> 4;
  const int bj = blockIdx.x;
  const int b = bj / a.Hkv, j = bj % a.Hkv;
  const int n = a.n, G = a.G;
  const int key0 = blockIdx.y * (kColKeys * kPfWaves);
  const int kw0 = key0 + kColKeys * wave;  // this wave's first key
  const unsigned char* kg = static_cast<const unsigned char*>(a.k) + static_cast<size_t>(bj) * n * D * ES;
  Frag<T> kf[4][KS];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int key = kw0 + 16 * kt + ln;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (key < n) kf[kt][s].load8(kg + (static_cast<size_t>(key) * D + 32 * s + 8 * lq) * ES);
      else kf[kt][s].zero();
    }
  }
  float cs[4][4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) cs[kt][i] = 0.0f;
  const int rt0 = key0 / 16, nrt = (n + 15) / 16;
  const int items = G * (nrt - rt0);
  const int nst = (items + NI - 1) / NI;
  const unsigned char* qg = static_cast<const unsigned char*>(a.q);
  const size_t hrow0 = (static_cast<size_t>(b) * a.Hq + static_cast<size_t>(j) * G) * n;  // head j*G, row 0

  // this wave's share of one item's copy: item wave / WPI of the stage,
  // 16-byte pieces (wave % WPI) * 64 * LOADS + lane + 64u of the 16-row tile
  const int my_item = wave / WPI, my_part = wave % WPI;
  u32x4 stg[LOADS];
  float lst = INFINITY;
  auto fetch = [&](int st) {
    const int it = st * NI + my_item;  // wave-uniform
    const int rt = rt0 + it / G, g = it % G;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = my_part * 64 * LOADS + lane + 64 * u;
      const int r = c / PIECES, pc = c % PIECES;
      const int row = rt * 16 + r;
      if (it < items && row < n)
        stg[u] = *reinterpret_cast<const u32x4*>(qg + ((hrow0 + static_cast<size_t>(g) * n + row) * D) * ES + 16 * pc);
      else
        stg[u] = u32x4{0u, 0u, 0u, 0u};
    }
    if (my_part == 0 && lane < 16) {
      const int row = rt * 16 + lane;
      lst = it < items && row < n ? a.lse[hrow0 + static_cast<size_t>(g) * n + row] : INFINITY;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = my_part * 64 * LOADS + lane + 64 * u;
      *reinterpret_cast<u32x4*>(&qs[buf][my_item * ITEM + (c / PIECES) * ROW + 16 * (c % PIECES)]) = stg[u];
    }
    if (my_part == 0 && lane < 16) ls[buf][my_item * 16 + lane] = lst;
  };
  auto item = [&](int buf, int ii, int rt, auto masked) {
    const int row = rt * 16 + ln;
    const unsigned char* qt = &qs[buf][ii * ITEM + ln * ROW];
    Frag<T> qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s].load8(qt + (32 * s + 8 * lq) * ES);
    const float lr = ls[buf][ii * 16 + ln];
    f32x4 s4[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s4[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) s4[kt] = mma(kf[kt][s], qf[s], s4[kt]);
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s4[kt][i], a.scale2, -lr));
        if constexpr (decltype(masked)::value) {
          const int key = kw0 + 16 * kt + 4 * lq + i;
          if (key > row || key >= n) pv = 0.0f;
        }
        cs[kt][i] += pv;
      }
  };

  fetch(0);
  stash(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < nst;
    if (more) fetch(st + 1);
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
      const int it = st * NI + ii;
      const int rt = rt0 + it / G;
      // rows rt*16..rt*16+15 against keys kw0..kw0+63: skip when every key lies
      // past every row; mask when some key does, or when keys reach n
      if (it < items && kw0 < n && rt * 16 + 15 >= kw0) {
        if (kw0 + kColKeys - 1 > rt * 16 || kw0 + kColKeys > n) item(buf, ii, rt, std::true_type{});
        else item(buf, ii, rt, std::false_type{});
      }
    }
    if (more) stash(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float t = sum16(cs[kt][i]);
      const int key = kw0 + 16 * kt + 4 * lq + i;
      if (ln == 0 && key < n) a.acc[static_cast<size_t>(bj) * n + key] = t;
    }
}

template <typename T, int KS>
kvc_status launch_prefill_t(const PfArgs& a, bool colsums, hipStream_t st) {
  using Gm = PfGeom<T, KS>;
  const int bytes = 2 * Gm::STAGE;
  const void* fk = reinterpret_cast<const void*>(&fa_fwd_kernel<T, KS>);
  if (bytes > 65536) {
    const hipError_t e = hipFuncSetAttribute(fk, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) {
      set_last_hip_error(e);
      return KVC_ERR_HIP;
    }
  }
  hipLaunchKernelGGL((fa_fwd_kernel<T, KS>), dim3(a.units, a.nrb), dim3(kPfThreads), bytes, st, a);
  kvc_status s = check_launch();
  if (s != KVC_OK || !colsums) return s;
  const int nkb = (a.n + kColKeys * kPfWaves - 1) / (kColKeys * kPfWaves);
  hipLaunchKernelGGL((colsum_kernel<T, KS>), dim3(a.B * a.Hkv, nkb), dim3(kPfThreads), 0, st, a);
  return check_launch();
}

template <typename T>
kvc_status launch_prefill(const PfArgs& a, int D, bool colsums, hipStream_t st) {
  switch (D) {
    case 32: return launch_prefill_t<T, 1>(a, colsums, st);
    case 64: return launch_prefill_t<T, 2>(a, colsums, st);
    case 128: return launch_prefill_t<T, 4>(a, colsums, st);
    default: return KVC_ERR_SHAPE;
  }
}

bool prefill_dim_ok(int D) { return D == 32 || D == 64 || D == 128; }

}  // namespace
}  // namespace kvc

extern "C" kvc_status kvc_prefill_attn(const void* q, const void* k, const void* v, kvc_dtype dtype, int32_t B,
                                       int32_t Hq, int32_t Hkv, int32_t n, int32_t D, float* out, float* acc,
                                       float* var, float* lse, void* ws, size_t* ws_bytes, void* stream) {
  using namespace kvc;
  if (!ws_bytes) return KVC_ERR_NULL;
  if (!dtype_ok(dtype)) return KVC_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || n < 1 || !prefill_dim_ok(D)) return KVC_ERR_SHAPE;
  const size_t need = align_up(static_cast<size_t>(B) * Hq * n * sizeof(float), 256);
  if (!ws) {
    *ws_bytes = need;
    return KVC_OK;
  }
  if (!q || !k || !v || !out || (var && !acc)) return KVC_ERR_NULL;
  if (*ws_bytes < need) return KVC_ERR_WORKSPACE;
  PfArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = static_cast<float*>(ws);
  a.lse_out = lse;
  a.acc = acc;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.n = n;
  a.Gc = a.G % 4 == 0 ? 4 : a.G % 2 == 0 ? 2 : 1;
  a.ngr = a.G / a.Gc;
  a.units = B * Hkv * a.ngr;
  const int RB = 32 * (kPfWaves / a.Gc);
  a.nrb = (n + RB - 1) / RB;
  a.scale2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  hipStream_t st = static_cast<hipStream_t>(stream);
  kvc_status s = dtype == KVC_F32 ? launch_prefill<float>(a, D, acc != nullptr, st)
                                  : launch_prefill<uint16_t>(a, D, acc != nullptr, st);
  if (s != KVC_OK || !var) return s;
  return launch_variance(acc, B * Hkv, n, var, st);
}
