// SnapKV/PyramidKV observation-window selection (blog "Eviction": SnapKV;
// PyramidKV "KV Cache Selection").
//
// For KV head j the R = G*W window rows (G query heads x W last prompt queries)
// attend causally to the prompt.  The scorer is a dense contraction
// Q_w[R][D] x K[n][D]^T on MFMA (bf16 inputs: v_mfma_f32_16x16x32_bf16; fp32
// inputs: v_mfma_f32_16x16x4_f32), in two passes over K:
//   pass 1: per 128-column chunk, each row's max and sum of 2^(x - max)
//           (x = logit * log2(e)/sqrt(D), causal mask), merged per row by a
//           small kernel into (M_r, 1/L_r);
//   pass 2: column sums of 2^(x - M_r)/L_r over the rows for candidates
//           c < n-W, written in fixed order (deterministic).
// Then the scores are max-pooled and mapped to order-preserving uint32 keys and
// the k'-th largest is found by a radix select (rows up to 32k candidates: one
// workgroup per (b, j), keys in registers, 4x8-bit digits; longer rows: 4096-
// candidate chunks over many workgroups, 8+12+12-bit digits); an index-order
// scan emits every key above the threshold plus the lowest-index ties, so idx
// comes out ascending with ties to the lower index.
#include <algorithm>

#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBlock = 128;  // rows per pass over the staged chunk (8 tiles of 16)
constexpr int kScoreWaves = 4;  // waves per scorer workgroup (two row tiles each; 8 waves x one tile measured slower)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

struct ScoreArgs {
  const void* q_win;  // [B][Hq][W][D]
  const void* k;      // [B][Hkv][n][D]
  float2* stats;      // pass 1: [B][Hkv][nc1][R] (max, sum) in log2 units
  float* rowstat;     // [B][Hkv][R] M + log2(L): 2^(x - it) is x's softmax weight
  float* raw;         // [B][Hkv][N] column sums
  const float* lse;   // or null: window row w of head h at lse[(b*Hq + h)*lse_stride + w], natural log
  int lse_stride;
  int Hq, Hkv, G, n, W, R, N, nc1;
  float scale2;
};

// Fragment of 8 consecutive channels for one lane, and the MFMA that consumes it.
template <typename T> struct Frag;
template <> struct Frag<uint16_t> {
  bf16x8 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const bf16x8*>(p); }
  __device__ __forceinline__ void zero() {
    for (int i = 0; i < 8; ++i) v[i] = static_cast<__bf16>(0.0f);
  }
};
template <> struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void load(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ void zero() {
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
};

// acc[row = 4*(lane/16)+i][col = lane%16] += sum_k A[row][k] B[k][col] over one
// 32-channel step; lane (r, q) supplies channels 32s+8q..+7 of its row/column.
__device__ __forceinline__ f32x4 mma(const Frag<uint16_t>& a, const Frag<uint16_t>& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<float>& a, const Frag<float>& b, f32x4 acc) {
#pragma unroll
  for (int u = 0; u < 8; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[u], b.v[u], acc, 0, 0, 0);
  return acc;
}

template <typename T> struct ChunkCols { static constexpr int value = 128; };
template <> struct ChunkCols<float> { static constexpr int value = 64; };

// 2^x for x <= 0 (or -inf): the hardware exp2 needs no range reduction here.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// All-reduce over the 16 lanes of a DPP row (the lanes that share an MFMA
// output row): swap neighbours, swap pairs, mirror within 8, mirror within 16.
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}
// Sum over the four lanes l, l^16, l^32, l^48 (the lane quarters of one column).
__device__ __forceinline__ float sum_quarters(float x) {
  const int lane = threadIdx.x & 63;
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x += __uint_as_float(lane < 32 ? s32[1] : s32[0]);  // + value of lane ^ 32
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x += __uint_as_float((lane & 16) ? s16[0] : s16[1]);  // + value of lane ^ 16
  return x;
}

// Window rows row0[u]..row0[u]+15 (u < NT) of one wave against the CH = 16*CT
// columns of chunk `chunk` (first column c0): MFMA products with the key
// fragments that kload(ct, s, frag) supplies, then pass 1 writes each row's
// (max, sum) for the chunk and pass 2 adds the rows' softmax weights to the
// lane's column partials (reduced over lanes and waves once, at the end).
// FULL: every column of the chunk is visible to every row (no causal mask).
// st: pass 2's per-row M + log2(L), +inf for rows beyond R (weight 2^-inf = 0).
template <typename T, int KS, int PASS, int NT, bool FULL, int TPW, int CT, typename KLoad>
__device__ __forceinline__ void score_tiles(const ScoreArgs& a, int bj, int chunk, int c0,
                                            const Frag<T> (&qf)[TPW][KS], const int (&row0)[TPW],
                                            const float (&st)[TPW][4], float (&colacc)[CT], KLoad kload) {
  const int lane = threadIdx.x & 63, ln = lane & 15, lq = lane >> 4;
  // pass 1 keeps at most two tiles of products live (registers); pass 2 takes
  // all NT at once, so each key fragment feeds NT products
  constexpr int TG = (PASS == 1 && NT > 2) ? 2 : NT;
  static_assert(NT % TG == 0, "whole tile groups");
#pragma unroll
  for (int gi = 0; gi < NT / TG; ++gi) {
    const int ug = gi * TG;
    f32x4 acc[TG][CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int u = 0; u < TG; ++u) acc[u][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        Frag<T> kf;
        kload(ct, s, kf);
#pragma unroll
        for (int u = 0; u < TG; ++u) acc[u][ct] = mma(qf[ug + u][s], kf, acc[u][ct]);
      }
    }
    if (PASS == 1) {
      // per row: max over the row's 16 lanes x CT columns, then the sum of
      // 2^(x - M) with x = logit * scale2 (scale2 > 0, so max(x) = scale2 * max)
#pragma unroll
      for (int u = 0; u < TG; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = row0[ug + u] + 4 * lq + i;
          float v[CT];
          if (FULL) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) v[ct] = acc[u][ct][i];
          } else {
            const int lim = a.n - a.W + (r % a.W);  // last key this row may see
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              const int c = c0 + ct * 16 + ln;
              v[ct] = (c <= lim && c < a.n) ? acc[u][ct][i] : -INFINITY;
            }
          }
          float mx = v[0];
#pragma unroll
          for (int ct = 1; ct < CT; ++ct) mx = fmaxf(mx, v[ct]);
          const float m = max16(mx) * a.scale2;
          float l = 0.0f;
          if (FULL || m != -INFINITY) {
            l = fast_exp2(__builtin_fmaf(v[0], a.scale2, -m));
#pragma unroll
            for (int ct = 1; ct < CT; ++ct) l += fast_exp2(__builtin_fmaf(v[ct], a.scale2, -m));
          }
          l = sum16(l);
          if (ln == 0 && r < a.R)
            a.stats[(static_cast<size_t>(bj) * a.nc1 + chunk) * a.R + r] = make_float2(m, l);
        }
      }
    } else {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        float v = fast_exp2(__builtin_fmaf(acc[0][ct][0], a.scale2, -st[ug][0]));
#pragma unroll
        for (int u = 0; u < TG; ++u) {
#pragma unroll
          for (int i = (u == 0 ? 1 : 0); i < 4; ++i)
            v += fast_exp2(__builtin_fmaf(acc[u][ct][i], a.scale2, -st[ug + u][i]));
        }
        colacc[ct] += v;
      }
    }
    if (NT / TG > 1) __builtin_amdgcn_sched_barrier(0);  // one tile group's products live at a time
  }
}

// A wave with any window row computes its tiles (rows beyond R have zero
// queries; pass 1 does not store them and pass 2 weights them 0): all TPW of
// them (ALL), or, when its last tile is idle, only the first (the two-tile
// scorer); in pass 1 whether the chunk needs causal masks selects the
// instantiation.
template <bool ALL, typename T, int KS, int PASS, int TPW, int CT, typename KLoad>
__device__ __forceinline__ void score_rows(const ScoreArgs& a, int bj, int chunk, int c0, bool full,
                                           const Frag<T> (&qf)[TPW][KS], const int (&row0)[TPW],
                                           const float (&st)[TPW][4], float (&colacc)[CT], KLoad kload) {
  if (row0[0] >= a.R) return;  // wave-uniform
  constexpr int NT1 = ALL ? TPW : 1;
  const bool all = ALL || row0[TPW - 1] < a.R;
  if (PASS == 2 || full) {
    if (all) score_tiles<T, KS, PASS, TPW, true>(a, bj, chunk, c0, qf, row0, st, colacc, kload);
    else score_tiles<T, KS, PASS, NT1, true>(a, bj, chunk, c0, qf, row0, st, colacc, kload);
  } else {
    if (all) score_tiles<T, KS, PASS, TPW, false>(a, bj, chunk, c0, qf, row0, st, colacc, kload);
    else score_tiles<T, KS, PASS, NT1, false>(a, bj, chunk, c0, qf, row0, st, colacc, kload);
  }
}

// Pass 2's row statistics for the lane's rows: from rowstat_kernel, or (lse
// given) log2(e) times window row r % W of query head r / W of the KV head.
template <int TPW>
__device__ __forceinline__ void load_rowstat(const ScoreArgs& a, int bj, const int (&row0)[TPW], float (&st)[TPW][4]) {
  const int lq = (threadIdx.x & 63) >> 4;
  const int b = bj / a.Hkv, j = bj - b * a.Hkv;
#pragma unroll
  for (int u = 0; u < TPW; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0[u] + 4 * lq + i;
      if (r >= a.R) {
        st[u][i] = INFINITY;
      } else if (a.lse) {
        const int g = r / a.W, w = r - g * a.W;
        st[u][i] = a.lse[(static_cast<size_t>(b) * a.Hq + j * a.G + g) * a.lse_stride + w] * 1.4426950408889634f;
      } else {
        st[u][i] = a.rowstat[static_cast<size_t>(bj) * a.R + r];
      }
    }
}

// NWAVE waves per workgroup (4: two 16-row tiles per wave, 8: one), 128 rows
// per pass over the staged chunk.
template <typename T, int KS, int PASS, int NWAVE>
__global__ __launch_bounds__(64 * NWAVE, (NWAVE == 8 ? 2 : 4)) void score_kernel(ScoreArgs a) {
  constexpr int NTHR = 64 * NWAVE, TPW = 8 / NWAVE;
  constexpr int CH = ChunkCols<T>::value;
  constexpr int D = KS * 32;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int LD = D + PAD;  // padded LDS row (elements)
  constexpr int CT = CH / 16;  // column tiles per chunk
  __shared__ __attribute__((aligned(16))) T ks[CH * LD];
  static_assert(NWAVE * 4 * CH * sizeof(float) <= CH * LD * sizeof(T), "partials fit in the key chunk");

  const int chunk = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int bj = b * a.Hkv + j;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 15, lq = lane >> 4;
  const int c0 = chunk * CH;
  const int ncol_valid = (PASS == 1) ? a.n : a.N;

  // stage the key chunk (zero-filled beyond the valid columns): every 16-byte
  // load is issued before the first LDS store, so the chunk costs one memory
  // round trip rather than one per loop iteration
  const T* kp = static_cast<const T*>(a.k) + static_cast<size_t>(bj) * a.n * D;
  const T* qbase = static_cast<const T*>(a.q_win) + static_cast<size_t>(b * a.Hq + j * a.G) * a.W * D;
  // query fragments of a row block: lane (ln, lq) holds row ln of each of its
  // two tiles, channels 32s+8lq..+7; the first block's are requested together
  // with the key chunk
  Frag<T> qf[TPW][KS];
  int row0[TPW];
  auto load_q = [&](int rb) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      row0[u] = rb + (wave + NWAVE * u) * 16;  // first row of this wave's tile u
      const int r = row0[u] + ln;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (r < a.R) qf[u][s].load(qbase + static_cast<size_t>(r) * D + 32 * s + 8 * lq);
        else qf[u][s].zero();
      }
    }
  };
  load_q(0);
  constexpr int VEC = 16 / sizeof(T);
  constexpr int NV = CH * D / VEC / NTHR;  // 16-byte pieces per thread
  static_assert(CH * D / VEC % NTHR == 0, "chunk must split evenly");
  uint4 kv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = tid + i * NTHR;
    const int c = e / (D / VEC), d = (e % (D / VEC)) * VEC;
    const int cc = min(c0 + c, a.n - 1);  // always in bounds; zeroed below if invalid
    kv[i] = *reinterpret_cast<const uint4*>(kp + static_cast<size_t>(cc) * D + d);
  }
  const bool chunk_valid = c0 + CH <= ncol_valid;  // no zero fill needed
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = tid + i * NTHR;
    const int c = e / (D / VEC), d = (e % (D / VEC)) * VEC;
    *reinterpret_cast<uint4*>(&ks[c * LD + d]) =
        (chunk_valid || c0 + c < ncol_valid) ? kv[i] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  // Chunks clear of the causal window (pass 1) or of the candidate bound (pass
  // 2) need no per-element masks.
  const bool full = c0 + CH <= ((PASS == 1) ? a.n - a.W + 1 : a.N);
  float colacc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) colacc[ct] = 0.0f;

  for (int rb = 0; rb < a.R; rb += kRowBlock) {
    if (rb > 0) load_q(rb);
    float st[TPW][4];
    if (PASS == 2) load_rowstat<TPW>(a, bj, row0, st);
    score_rows<false, T, KS, PASS, TPW>(a, bj, chunk, c0, full, qf, row0, st, colacc, [&](int ct, int s, Frag<T>& kf) {
      kf.load(&ks[(ct * 16 + ln) * LD + 32 * s + 8 * lq]);
    });
  }

  if (PASS == 2) {
    // column partials of every lane quarter of every wave, summed in a fixed order
    __syncthreads();  // the key chunk is dead: its LDS takes the partials
    float* colred = reinterpret_cast<float*>(ks);  // [NWAVE * 4][CH]
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) colred[(wave * 4 + lq) * CH + ct * 16 + ln] = colacc[ct];
    __syncthreads();
    for (int c = tid; c < CH; c += NTHR) {
      float v = colred[c];
#pragma unroll
      for (int w = 1; w < NWAVE * 4; ++w) v += colred[w * CH + c];
      if (c0 + c < a.N) a.raw[static_cast<size_t>(bj) * a.N + c0 + c] = v;
    }
  }
}

// ---------------------------------------------------------------- pipelined scorer
// bf16 keys, D in {32, 64, 128}, R <= 64*TPW (4 waves, TPW row tiles of 16
// each; tile u of wave w holds rows (w + 4u)*16..+15): each workgroup walks chunks
// ch = blockIdx.x, + gridDim.x, ... of its (b, j); while it computes chunk k the
// direct-to-LDS loads of chunk k+1 are in flight (two LDS buffers), so the
// memory latency hides behind the MFMA and softmax work and no VGPRs hold
// staged data.  Staged layout: 16-byte piece p of chunk row r sits in slot
// r*P + (p ^ sw(r)) (P pieces per row).  One 1 KB load covers whole rows (one
// contiguous kilobyte of K), and the 16 rows of an MFMA fragment read 16
// distinct bank groups for any fixed piece.
constexpr int kPipeCH = 128;  // columns per chunk (also the pass-1 statistics granularity)
constexpr int kPipeBuf = 2;   // chunk buffers per workgroup: kPipeBuf - 1 chunks in flight
constexpr int kPipeWaves = 4;
constexpr int kLdsPerCU = 160 * 1024;

template <int KS> struct PipeGeom {
  static constexpr int D = 32 * KS;
  static constexpr int P = D / 8;                 // 16-byte pieces per key row
  static constexpr int CH = kPipeCH;
  static constexpr int BYTES = CH * D * 2;        // one staged chunk
  static constexpr int NI = BYTES / 1024;         // 1 KB direct-to-LDS loads per chunk
  static constexpr int NIW = NI / kPipeWaves;     // per wave
  static constexpr int SWDIV = P >= 16 ? 1 : 16 / P;
  static constexpr int SWMOD = P >= 16 ? 16 : P;
  static constexpr int LDS = kPipeBuf * BYTES + kPipeWaves * CH * 4;
  // resident workgroups per CU: what LDS allows, at most 2 (registers: up to
  // 256 per lane for the four row tiles of R > 128)
  static constexpr int WGS = kLdsPerCU / LDS < 2 ? kLdsPerCU / LDS : 2;
  static_assert(NI % kPipeWaves == 0 && NIW * (kPipeBuf - 1) < 64, "loads split evenly; vmcnt range");
  // depends on r mod 16 only
  __device__ static int sw(int r) { return (r / SWDIV) % SWMOD; }
};

template <int N> __device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `later` chunk fills of NIW loads each (the ones issued
// after the chunk about to be used) are outstanding.
template <int NIW, int L = kPipeBuf - 1>
__device__ __forceinline__ void wait_chunks(int later) {
  if constexpr (L == 0) {
    wait_vmem<0>();
  } else {
    if (later >= L) wait_vmem<L * NIW>();
    else wait_chunks<NIW, L - 1>(later);
  }
}

// One 16-byte direct-to-LDS load per lane: lane l's bytes land at dst + 16*l.
__device__ __forceinline__ void lds_load16(const void* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// The lane's source offsets (elements) within a chunk for this wave's loads:
// load ii fills slot j = (wave*NIW + ii)*64 + lane, i.e. row j/P, piece (j%P)^sw.
// (The row of a load is off / D.)
template <int KS> struct PipeOffsets {
  int off[PipeGeom<KS>::NIW];
  __device__ __forceinline__ PipeOffsets(int wave, int lane) {
    using G = PipeGeom<KS>;
#pragma unroll
    for (int ii = 0; ii < G::NIW; ++ii) {
      const int j = (wave * G::NIW + ii) * 64 + lane;
      const int r = j / G::P;
      off[ii] = r * G::D + ((j % G::P) ^ G::sw(r)) * 8;
    }
  }
};

// This wave's share of the direct-to-LDS loads of the chunk whose first column
// is c0 (in the last chunk, rows past the key count read the last key: they are
// masked or unused).
template <int KS>
__device__ __forceinline__ void pipe_fill(const uint16_t* kp, const PipeOffsets<KS>& po, int c0, int n,
                                          unsigned char* dst, int wave) {
  using G = PipeGeom<KS>;
  const uint16_t* base = kp + static_cast<size_t>(c0) * G::D;
  if (c0 + G::CH <= n) {
#pragma unroll
    for (int ii = 0; ii < G::NIW; ++ii) lds_load16(base + po.off[ii], dst + (wave * G::NIW + ii) * 1024);
  } else {
#pragma unroll
    for (int ii = 0; ii < G::NIW; ++ii) {
      const int excess = max(0, c0 + po.off[ii] / G::D - (n - 1));  // rows to step back
      lds_load16(base + po.off[ii] - excess * G::D, dst + (wave * G::NIW + ii) * 1024);
    }
  }
}

// Workgroup barrier that waits for this wave's LDS operations only: the
// direct-to-LDS loads of later chunks stay in flight across it (a
// __syncthreads() would wait for every outstanding memory operation).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int KS, int PASS, int TPW>
__global__ __launch_bounds__(64 * kPipeWaves, PipeGeom<KS>::WGS) void score_pipe_kernel(ScoreArgs a) {
  using G = PipeGeom<KS>;
  constexpr int NWAVE = kPipeWaves, CH = G::CH, CT = CH / 16, D = G::D, NB = kPipeBuf;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  unsigned char* ring = smem;                                      // [NB][BYTES]
  float* colred = reinterpret_cast<float*>(smem + NB * G::BYTES);  // [NWAVE][CH]
  const int j = blockIdx.y, b = blockIdx.z;
  const int bj = b * a.Hkv + j;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int ln = lane & 15, lq = lane >> 4;
  const int nchunk = ((PASS == 1 ? a.n : a.N) + CH - 1) / CH;
  const int g = gridDim.x;
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + static_cast<size_t>(bj) * a.n * D;
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q_win) + static_cast<size_t>(b * a.Hq + j * a.G) * a.W * D;

  int ch = blockIdx.x;  // < nchunk
  const PipeOffsets<KS> po(wave, lane);
#pragma unroll
  for (int i = 0; i < NB - 1; ++i)
    if (ch + i * g < nchunk) pipe_fill<KS>(kp, po, (ch + i * g) * CH, a.n, ring + i * G::BYTES, wave);
  // the wave's window rows (all R rows fit one block) and, in pass 2, their statistics
  Frag<uint16_t> qf[TPW][KS];
  int row0[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    row0[u] = (wave + NWAVE * u) * 16;
    const int r = row0[u] + ln;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      if (r < a.R) qf[u][s2].load(qbase + static_cast<size_t>(r) * D + 32 * s2 + 8 * lq);
      else qf[u][s2].zero();
    }
  }
  float st[TPW][4];
  if (PASS == 2) load_rowstat<TPW>(a, bj, row0, st);
  // fragment (ct, s) of lane (ln, lq): row ct*16 + ln, piece 4s + lq
  int foff[KS];
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2) foff[s2] = (ln * G::P + ((4 * s2 + lq) ^ G::sw(ln))) * 16;

  for (int k = 0; ch < nchunk; ++k, ch += g) {
    const int ahead = ch + (NB - 1) * g;
    if (ahead < nchunk) pipe_fill<KS>(kp, po, ahead * CH, a.n, ring + ((k + NB - 1) % NB) * G::BYTES, wave);
    wait_chunks<G::NIW>(min(NB - 1, (nchunk - 1 - ch) / g));  // this chunk's loads (and all older accesses) are done
    lds_barrier();  // every wave's share of this chunk has landed
    const unsigned char* cur = ring + (k % NB) * G::BYTES;
    const int c0 = ch * CH;
    const bool full = c0 + CH <= ((PASS == 1) ? a.n - a.W + 1 : a.N);
    float colacc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) colacc[ct] = 0.0f;
    score_rows<true, uint16_t, KS, PASS, TPW>(a, bj, ch, c0, full, qf, row0, st, colacc, [&](int ct, int s2, Frag<uint16_t>& kf) {
      kf.load(reinterpret_cast<const uint16_t*>(cur + ct * 16 * G::P * 16 + foff[s2]));
    });
    if (PASS == 2) {
      if (row0[0] < a.R) {  // wave-uniform; idle waves leave zeros
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const float v = sum_quarters(colacc[ct]);
          if (lq == 0) colred[wave * CH + ct * 16 + ln] = v;
        }
      } else if (lq == 0) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) colred[wave * CH + ct * 16 + ln] = 0.0f;
      }
      lds_barrier();  // also: every wave is done with this buffer before it is refilled
      if (tid < CH) {
        float v = colred[tid];
#pragma unroll
        for (int w = 1; w < NWAVE; ++w) v += colred[w * CH + tid];
        if (c0 + tid < a.N) a.raw[static_cast<size_t>(bj) * a.N + c0 + tid] = v;
      }
    } else {
      lds_barrier();  // every wave is done with this buffer before it is refilled
    }
  }
}

// Per row: M = max over chunks, L = sum l_k 2^(m_k - M); stored as M + log2(L).  One wave
// per row; lane i takes chunks i, i+64, ... (one round of loads for up to 64
// chunks, i.e. rows of 8k keys), then the wave reduces max and sum.
constexpr int kRowsPerBlock = kThreads / 64;
__device__ __forceinline__ float wave_max(float x) {
  x = max16(x);
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum(float x) { return sum_quarters(sum16(x)); }
__global__ __launch_bounds__(kThreads) void rowstat_kernel(ScoreArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int j = blockIdx.y, b = blockIdx.z;
  if (r >= a.R) return;  // wave-uniform
  const size_t bj = static_cast<size_t>(b) * a.Hkv + j;
  const float2* st = a.stats + bj * a.nc1 * a.R + r;
  float m = -INFINITY, l = 0.0f;  // this lane's chunks, merged
  for (int c0 = 0; c0 < a.nc1; c0 += 64) {
    const int c = c0 + lane;
    const float2 ml = c < a.nc1 ? st[static_cast<size_t>(c) * a.R] : make_float2(-INFINITY, 0.0f);
    const float M = fmaxf(m, ml.x);
    if (M != -INFINITY) {
      l = (m == -INFINITY ? 0.0f : l * exp2f(m - M)) + (ml.x == -INFINITY ? 0.0f : ml.y * exp2f(ml.x - M));
      m = M;
    }
  }
  const float M = wave_max(m);
  const float L = wave_sum(m == -INFINITY ? 0.0f : l * exp2f(m - M));
  if (lane == 0) a.rowstat[bj * a.R + r] = M + log2f(L);
}

constexpr int kTopThreads = 1024;

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;  // -0 ranks as +0
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by
// 1, 2, 4, 8 within each row of 16 lanes, then row 0's total into row 1 and row
// 2's into row 3 (row_bcast:15), then rows 0-1's total into rows 2-3
// (row_bcast:31).  Lanes without a source add 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Histogram votes of a thread's consecutive candidates: one LDS atomic per run
// of valid keys with equal bins, adding the run length.  Neighbouring
// candidates mostly share their leading key byte, so one vote per key would put
// nearly every lane of a wave on one address in the first pass (the LDS
// serializes those): measured 4.6 us of a 14 us top-k at the 8B shape.
template <int KPT>
__device__ __forceinline__ void hist_add_runs(int* hist, const bool (&valid)[KPT], const uint32_t (&bin)[KPT]) {
  int run = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    run = valid[i] ? run + 1 : 0;
    const bool cont = i + 1 < KPT && valid[i + 1] && bin[i + 1] == bin[i];
    if (valid[i] && !cont) atomicAdd(&hist[bin[i]], run);
    if (!cont) run = 0;
  }
}

// Digit selection of one radix pass by one wave (after the barrier that ends
// the votes): lane l holds bins 255-4l .. 252-4l (counted from the top), one
// wave scan of their sums, and the lane whose bin first reaches krem writes
// (digit, krem - above).  It clears the 256 bins for the next pass (no one
// reads them before the next barrier).
__device__ __forceinline__ void select_digit_wave(int* hist, int krem, uint32_t* sel) {
  const int lane = threadIdx.x & 63;
  int4* h4 = reinterpret_cast<int4*>(hist) + 63 - lane;  // bins 252-4l .. 255-4l
  const int4 w = *h4;
  *h4 = make_int4(0, 0, 0, 0);
  const int c[4] = {w.w, w.z, w.y, w.x};  // bins 255-4l, 254-4l, ...
  const int tot = c[0] + c[1] + c[2] + c[3];
  int above = wave_incl_scan(tot) - tot;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (above < krem && above + c[i] >= krem) {
      sel[0] = static_cast<uint32_t>(255 - 4 * lane - i);
      sel[1] = static_cast<uint32_t>(krem - above);
    }
    above += c[i];
  }
}

// Block-wide exclusive prefix sum with one barrier; sh (kTopThreads/64 ints)
// must not be written again before a later barrier.
__device__ int block_exclusive_scan1(int x, int* sh) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int inc = wave_incl_scan(x);
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int i = 0; i < kTopThreads / 64; ++i) base += i < w ? sh[i] : 0;
  return base + inc - x;
}

constexpr int kMaxPoolHalf = 4;  // pooling kernels up to 9 use the register window
constexpr int kChunkKpt = 4;                          // candidates per thread in the chunked path
constexpr int kChunk = kTopThreads * kChunkKpt;       // candidates per workgroup in the chunked path
constexpr int kWideBins = 4096;                       // 12-bit digits of radix passes 2 and 3
constexpr int kSelSlots = 8;

// Digit selection over NB >= kTopThreads bins: thread t takes the NB/kTopThreads
// bins below the top's t-th group, a block scan gives the count above its first
// bin, and the thread whose bin first reaches krem writes (digit, krem - above).
template <int NB>
__device__ __forceinline__ void select_digit_wide(const int* cnt, int krem, int* scan_sh, uint32_t* sel) {
  constexpr int BPT = NB / kTopThreads;
  const int t = threadIdx.x;
  int c[BPT], tot = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    c[i] = cnt[NB - 1 - (t * BPT + i)];
    tot += c[i];
  }
  int above = block_exclusive_scan1(tot, scan_sh);
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    if (above < krem && above + c[i] >= krem) {
      sel[0] = static_cast<uint32_t>(NB - 1 - (t * BPT + i));
      sel[1] = static_cast<uint32_t>(krem - above);
    }
    above += c[i];
  }
}

struct TopArgs {
  const float* raw;  // [B][Hkv] rows of N scores, ld apart
  uint32_t* keys;    // [B][Hkv][NP] (chunked path)
  float* scores;     // pooled scores out, or null
  int32_t* idx;      // [B][Hkv][kk]
  int* hist1;        // [B][Hkv][nch][256] per-chunk counts of the top key byte (chunked path)
  int* ghist;        // [B][Hkv][2][kWideBins] counts of the 12-bit digits of passes 2 and 3
  uint32_t* sel;     // [B][Hkv][kSelSlots]: (prefix, remaining k) after passes 1, 2 and 3
  int2* cnt;         // [B][Hkv][nch] (keys above the threshold, keys equal to it) per chunk
  int Hkv, N, kk, pool, NP, nch;
  int ld;  // row stride of raw (>= N)
};

// Long score rows: the candidates are split into chunks of kChunk, one
// workgroup each (thread t owns kChunkKpt consecutive candidates), and the
// radix select runs as a chain of launches over all chunks of all heads:
//   chunk_pool_kernel    pooled keys, per-chunk counts of the top key byte;
//   chunk_hist_kernel    (x2) merge the previous digit's counts, pick the digit,
//                        count the next 12 bits of the keys still in play;
//   chunk_count_kernel   pick the last digit (the threshold key), count each
//                        chunk's keys above and equal to it;
//   chunk_emit_kernel    emit in index order from the chunk counts before it.
// Each launch picks the previous digit redundantly in every workgroup; the
// first chunk's workgroup stores it for the next launch.
__device__ __forceinline__ uint4 load_chunk_keys(const TopArgs& a, size_t bj, int cb) {
  return *reinterpret_cast<const uint4*>(a.keys + bj * a.NP + cb);
}
__device__ __forceinline__ uint32_t key_at(const uint4& k, int i) { return i == 0 ? k.x : i == 1 ? k.y : i == 2 ? k.z : k.w; }

__global__ __launch_bounds__(kTopThreads) void chunk_pool_kernel(TopArgs a) {
  // raw[c0 - kMaxPoolHalf + i], positions outside the row replaced by the
  // nearest end value (the maximum of a window clipped to the row)
  __shared__ __attribute__((aligned(16))) float rs[kChunk + 2 * kMaxPoolHalf];
  __shared__ int hist[256];
  const int ch = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const size_t bj = static_cast<size_t>(b) * a.Hkv + j;
  const int tid = threadIdx.x;
  const int N = a.N, h = a.pool / 2, c0 = ch * kChunk;
  const float* raw = a.raw + bj * a.ld;
  if (tid < 256) hist[tid] = 0;
  if (ch == 0)  // the counts of passes 2 and 3 are accumulated by later launches
    for (int i = tid; i < 2 * kWideBins; i += kTopThreads) a.ghist[bj * 2 * kWideBins + i] = 0;
  for (int i = tid; i < kChunk + 2 * kMaxPoolHalf; i += kTopThreads)
    rs[i] = raw[min(max(c0 - kMaxPoolHalf + i, 0), N - 1)];
  __syncthreads();
  const int cb = c0 + tid * kChunkKpt;
  uint32_t key[kChunkKpt];
  if (h <= kMaxPoolHalf) {
    // window positions cb - 4 .. cb + kChunkKpt + 3 through aligned 16-byte
    // LDS reads (per-float reads of slots 4 floats apart conflict on the banks)
    constexpr int NWIN = kChunkKpt + 2 * kMaxPoolHalf;
    float win[NWIN];
    const float4* w4 = reinterpret_cast<const float4*>(rs + tid * kChunkKpt);
#pragma unroll
    for (int i = 0; i < NWIN / 4; ++i) {
      const float4 x = w4[i];
      win[4 * i] = x.x;
      win[4 * i + 1] = x.y;
      win[4 * i + 2] = x.z;
      win[4 * i + 3] = x.w;
    }
#pragma unroll
    for (int i = 0; i < kChunkKpt; ++i) {
      float m = win[i + kMaxPoolHalf];
#pragma unroll
      for (int d = 1; d <= kMaxPoolHalf; ++d)
        if (d <= h) m = fmaxf(m, fmaxf(win[i + kMaxPoolHalf - d], win[i + kMaxPoolHalf + d]));
      const int c = cb + i;
      key[i] = c < N ? order_key(m) : 0u;
      if (a.scores && c < N) a.scores[bj * N + c] = m;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kChunkKpt; ++i) {
      const int c = cb + i;
      key[i] = 0u;
      if (c < N) {
        float m = raw[c];
        const int lo = max(0, c - h), hi = min(N - 1, c + h);
        for (int d = lo; d <= hi; ++d) m = fmaxf(m, raw[d]);
        key[i] = order_key(m);
        if (a.scores) a.scores[bj * N + c] = m;
      }
    }
  }
  *reinterpret_cast<uint4*>(a.keys + bj * a.NP + cb) = make_uint4(key[0], key[1], key[2], key[3]);
  if (a.kk == 0) return;
  bool valid[kChunkKpt];
  uint32_t bin[kChunkKpt];
#pragma unroll
  for (int i = 0; i < kChunkKpt; ++i) {
    valid[i] = cb + i < N;
    bin[i] = key[i] >> 24;
  }
  hist_add_runs<kChunkKpt>(hist, valid, bin);
  __syncthreads();
  if (tid < 256) a.hist1[(bj * a.nch + ch) * 256 + tid] = hist[tid];
}

// PASS 2: digit 1 from the per-chunk byte counts, then counts of key bits
// 12..23 among keys with that top byte.  PASS 3: digit 2 from pass 2's counts,
// then counts of bits 0..11 among keys with that 20-bit prefix.
template <int PASS>
__global__ __launch_bounds__(kTopThreads) void chunk_hist_kernel(TopArgs a) {
  __shared__ __attribute__((aligned(16))) int hist[kWideBins];
  __shared__ int scan_sh[kTopThreads / 64 + 1];
  __shared__ uint32_t sel_sh[2];
  const int ch = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const size_t bj = static_cast<size_t>(b) * a.Hkv + j;
  const int tid = threadIdx.x;
  uint32_t prefix, pmask;
  int krem;
  if (PASS == 2) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    {
      const int bin = tid & 255;
      int s = 0;
      for (int c = tid >> 8; c < a.nch; c += kTopThreads / 256) s += a.hist1[(bj * a.nch + c) * 256 + bin];
      atomicAdd(&hist[bin], s);
    }
    __syncthreads();
    if (tid < 64) select_digit_wave(hist, a.kk, sel_sh);
    __syncthreads();
    prefix = sel_sh[0] << 24;
    pmask = 0xFF000000u;
  } else {
    for (int i = tid; i < kWideBins; i += kTopThreads) hist[i] = a.ghist[bj * 2 * kWideBins + i];
    __syncthreads();
    select_digit_wide<kWideBins>(hist, static_cast<int>(a.sel[bj * kSelSlots + 1]), scan_sh, sel_sh);
    __syncthreads();
    prefix = a.sel[bj * kSelSlots] | (sel_sh[0] << 12);
    pmask = 0xFFFFF000u;
  }
  krem = static_cast<int>(sel_sh[1]);
  if (ch == 0 && tid == 0) {
    a.sel[bj * kSelSlots + 2 * (PASS - 2)] = prefix;
    a.sel[bj * kSelSlots + 2 * (PASS - 2) + 1] = static_cast<uint32_t>(krem);
  }
  __syncthreads();
  for (int i = tid; i < kWideBins; i += kTopThreads) hist[i] = 0;
  __syncthreads();
  constexpr int shift = PASS == 2 ? 12 : 0;
  const int cb = ch * kChunk + tid * kChunkKpt;
  const uint4 k4 = load_chunk_keys(a, bj, cb);
  bool valid[kChunkKpt];
  uint32_t bin[kChunkKpt];
#pragma unroll
  for (int i = 0; i < kChunkKpt; ++i) {
    const uint32_t key = key_at(k4, i);
    valid[i] = cb + i < a.N && (key & pmask) == prefix;
    bin[i] = (key >> shift) & (kWideBins - 1);
  }
  hist_add_runs<kChunkKpt>(hist, valid, bin);
  __syncthreads();
  int* g = a.ghist + (bj * 2 + (PASS - 2)) * kWideBins;
  for (int i = tid; i < kWideBins; i += kTopThreads)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

__global__ __launch_bounds__(kTopThreads) void chunk_count_kernel(TopArgs a) {
  __shared__ int hist[kWideBins];
  __shared__ int scan_sh[kTopThreads / 64 + 1];
  __shared__ uint32_t sel_sh[2];
  const int ch = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const size_t bj = static_cast<size_t>(b) * a.Hkv + j;
  const int tid = threadIdx.x;
  for (int i = tid; i < kWideBins; i += kTopThreads) hist[i] = a.ghist[(bj * 2 + 1) * kWideBins + i];
  __syncthreads();
  select_digit_wide<kWideBins>(hist, static_cast<int>(a.sel[bj * kSelSlots + 3]), scan_sh, sel_sh);
  __syncthreads();
  const uint32_t tau = a.sel[bj * kSelSlots + 2] | sel_sh[0];
  if (ch == 0 && tid == 0) {
    a.sel[bj * kSelSlots + 4] = tau;
    a.sel[bj * kSelSlots + 5] = sel_sh[1];
  }
  const int cb = ch * kChunk + tid * kChunkKpt;
  const uint4 k4 = load_chunk_keys(a, bj, cb);
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < kChunkKpt; ++i) {
    const uint32_t key = key_at(k4, i);
    const bool ok = cb + i < a.N;
    gt += (ok && key > tau) ? 1 : 0;
    eq += (ok && key == tau) ? 1 : 0;
  }
  // both counts in 16-bit halves (at most kChunk = 4096 each)
  const int inc = wave_incl_scan((gt << 16) | eq);
  if ((tid & 63) == 63) scan_sh[tid >> 6] = inc;
  __syncthreads();
  if (tid == 0) {
    int t = 0;
#pragma unroll
    for (int i = 0; i < kTopThreads / 64; ++i) t += scan_sh[i];
    a.cnt[bj * a.nch + ch] = make_int2(t >> 16, t & 0xFFFF);
  }
}

// Chunk ch's keys above the threshold go after those of chunks 0..ch-1; of the
// keys equal to it the first krem in index order are taken.
__global__ __launch_bounds__(kTopThreads) void chunk_emit_kernel(TopArgs a) {
  __shared__ int scan_sh[kTopThreads / 64 + 1];
  __shared__ int before[2];
  const int ch = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const size_t bj = static_cast<size_t>(b) * a.Hkv + j;
  const int tid = threadIdx.x;
  const uint32_t tau = a.sel[bj * kSelSlots + 4];
  const int krem = static_cast<int>(a.sel[bj * kSelSlots + 5]);
  if (tid < 64) {
    int g = 0, e = 0;
    for (int c = tid; c < ch; c += 64) {
      const int2 v = a.cnt[bj * a.nch + c];
      g += v.x;
      e += v.y;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      g += __shfl_xor(g, o);
      e += __shfl_xor(e, o);
    }
    if (tid == 0) {
      before[0] = g;
      before[1] = e;
    }
  }
  __syncthreads();
  const int g_before = before[0], e_before = before[1];
  const int cb = ch * kChunk + tid * kChunkKpt;
  const uint4 k4 = load_chunk_keys(a, bj, cb);
  // keys taken before this thread's: the larger ones plus min(krem, equal ones)
  // before it, over this chunk and the chunks before it (one scan of both
  // counts in 16-bit halves)
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < kChunkKpt; ++i) {
    const uint32_t key = key_at(k4, i);
    const bool ok = cb + i < a.N;
    n_gt += (ok && key > tau) ? 1 : 0;
    n_eq += (ok && key == tau) ? 1 : 0;
  }
  const int bfr = block_exclusive_scan1((n_gt << 16) | n_eq, scan_sh);
  int eq_rank = (bfr & 0xFFFF) + e_before;
  int pos = g_before + (bfr >> 16) + min(krem, eq_rank);
  int32_t* idx = a.idx + bj * a.kk;
#pragma unroll
  for (int i = 0; i < kChunkKpt; ++i) {
    const uint32_t key = key_at(k4, i);
    const bool ok = cb + i < a.N;
    const bool eq = ok && key == tau;
    const bool take = ok && (key > tau || (eq && eq_rank < krem));
    eq_rank += eq ? 1 : 0;
    if (take && pos < a.kk) idx[pos] = cb + i;
    pos += take ? 1 : 0;
  }
}

// Short score rows (N <= KPT * 1024): the raw scores are staged in LDS once,
// thread t owns the KPT consecutive candidates [t*KPT, t*KPT + KPT) and keeps
// their pooled keys in registers for the four radix passes (two barriers each),
// and the index-order emission needs one block scan.
template <int KPT>
__global__ __launch_bounds__(kTopThreads) void pool_topk_lds_kernel(TopArgs a) {
  // raw scores of positions -kMaxPoolHalf .. KPT*kTopThreads + kMaxPoolHalf - 1:
  // the row, padded on both sides with copies of its end values
  extern __shared__ __attribute__((aligned(16))) float rs_pad[];
  __shared__ __attribute__((aligned(16))) int hist[256];
  __shared__ int scan_sh[kTopThreads / 64 + 1];
  __shared__ uint32_t sel_sh[2];
  const int j = blockIdx.x, b = blockIdx.y;
  const size_t bj = static_cast<size_t>(b) * a.Hkv + j;
  const int tid = threadIdx.x;
  const int N = a.N, h = a.pool / 2;  // N >= 1
  const float* raw = a.raw + bj * a.ld;
  int32_t* idx = a.idx + bj * a.kk;
  float* rs = rs_pad + kMaxPoolHalf;
  {
    float v[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) v[i] = raw[min(tid + i * kTopThreads, N - 1)];
    float e = 0.0f;
    if (tid < 2 * kMaxPoolHalf) e = raw[tid < kMaxPoolHalf ? 0 : N - 1];
#pragma unroll
    for (int i = 0; i < KPT; ++i) rs[tid + i * kTopThreads] = v[i];
    if (tid < kMaxPoolHalf) rs[tid - kMaxPoolHalf] = e;
    else if (tid < 2 * kMaxPoolHalf) rs[KPT * kTopThreads + tid - kMaxPoolHalf] = e;
  }
  if (tid < 256) hist[tid] = 0;
  __syncthreads();
  const int cb = tid * KPT;
  uint32_t key[KPT];
  if (h <= kMaxPoolHalf) {
    // the thread's widest pooling window, positions cb - 4 .. cb + KPT + 3, in
    // registers through aligned 16-byte LDS reads (one float per lane from
    // slots 8 floats apart would conflict on the LDS banks); the padding
    // repeats the end values, which gives the maximum of a window clipped to
    // the row
    constexpr int NWIN = KPT + 2 * kMaxPoolHalf;
    float win[NWIN];
    const float4* w4 = reinterpret_cast<const float4*>(rs + cb - kMaxPoolHalf);
#pragma unroll
    for (int i = 0; i < NWIN / 4; ++i) {
      const float4 x = w4[i];
      win[4 * i] = x.x;
      win[4 * i + 1] = x.y;
      win[4 * i + 2] = x.z;
      win[4 * i + 3] = x.w;
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      // window of candidate cb + i: win[i + 4 - h .. i + 4 + h]
      float m = win[i + kMaxPoolHalf];
#pragma unroll
      for (int d = 1; d <= kMaxPoolHalf; ++d)
        if (d <= h) m = fmaxf(m, fmaxf(win[i + kMaxPoolHalf - d], win[i + kMaxPoolHalf + d]));
      const int c = cb + i;
      key[i] = c < N ? order_key(m) : 0u;
      if (a.scores && c < N) a.scores[bj * N + c] = m;
    }
  } else {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = cb + i;
      key[i] = 0u;
      if (c < N) {
        float m = rs[c];
        const int lo = max(0, c - h), hi = min(N - 1, c + h);
        for (int d = lo; d <= hi; ++d) m = fmaxf(m, rs[d]);
        key[i] = order_key(m);
        if (a.scores) a.scores[bj * N + c] = m;
      }
    }
  }
  if (a.kk == 0) return;
  if (a.kk == N) {
    for (int c = tid; c < N; c += kTopThreads) idx[c] = c;
    return;
  }
  uint32_t prefix = 0, pmask = 0;
  int krem = a.kk;
  // per pass: votes (the histogram was cleared before the previous barrier),
  // a barrier, wave 0's digit selection (which clears the bins again), a
  // barrier; sel_sh is read before wave 0 next writes it, one barrier later
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    bool valid[KPT];
    uint32_t bin[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      valid[i] = cb + i < N && (key[i] & pmask) == prefix;
      bin[i] = (key[i] >> shift) & 255u;
    }
    hist_add_runs<KPT>(hist, valid, bin);
    __syncthreads();
    if (tid < 64) select_digit_wave(hist, krem, sel_sh);
    __syncthreads();
    prefix |= sel_sh[0] << shift;
    pmask |= 255u << shift;
    krem = static_cast<int>(sel_sh[1]);
  }
  // prefix is the k'-th largest key: take every larger key and the krem
  // lowest-index keys equal to it, in index order.  The keys taken before this
  // thread's are the larger ones plus min(krem, equal ones) before it: one scan
  // of both counts, packed in 16-bit halves (N <= 32768).
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool ok = cb + i < N;
    n_gt += (ok && key[i] > prefix) ? 1 : 0;
    n_eq += (ok && key[i] == prefix) ? 1 : 0;
  }
  const int before = block_exclusive_scan1((n_gt << 16) | n_eq, scan_sh);
  int eq_rank = before & 0xFFFF;
  int pos = (before >> 16) + min(eq_rank, krem);
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool ok = cb + i < N;
    const bool eq = ok && key[i] == prefix;
    const bool take = ok && (key[i] > prefix || (eq && eq_rank < krem));
    eq_rank += eq ? 1 : 0;
    if (take && pos < a.kk) idx[pos] = cb + i;
    pos += take ? 1 : 0;
  }
}

template <typename T, int PASS>
kvc_status launch_score(const ScoreArgs& a, int KS, dim3 grid, hipStream_t st) {
  switch (KS) {
#define KVC_CASE(k)                                                                     \
  case k:                                                                               \
    hipLaunchKernelGGL((score_kernel<T, k, PASS, kScoreWaves>), grid, dim3(64 * kScoreWaves), 0, st, a); \
    break;
    KVC_CASE(1) KVC_CASE(2) KVC_CASE(3) KVC_CASE(4) KVC_CASE(5) KVC_CASE(6) KVC_CASE(7) KVC_CASE(8)
#undef KVC_CASE
    default: return KVC_ERR_SHAPE;
  }
  return check_launch();
}

// Rows longer than one workgroup's LDS take the chunked top-k, and so do rows
// whose heads are too few to spread one workgroup per head over the chip.
constexpr int kChunkedMinN = 32 * kTopThreads;
bool chunked_topk(int N) { return N > kChunkedMinN; }

kvc_status run_chunked_topk(const TopArgs& t, int B, hipStream_t st) {
  const dim3 grid(t.nch, t.Hkv, B);
  hipLaunchKernelGGL(chunk_pool_kernel, grid, dim3(kTopThreads), 0, st, t);
  kvc_status s = check_launch();
  if (s != KVC_OK || t.kk == 0) return s;
  hipLaunchKernelGGL(chunk_hist_kernel<2>, grid, dim3(kTopThreads), 0, st, t);
  if ((s = check_launch()) != KVC_OK) return s;
  hipLaunchKernelGGL(chunk_hist_kernel<3>, grid, dim3(kTopThreads), 0, st, t);
  if ((s = check_launch()) != KVC_OK) return s;
  hipLaunchKernelGGL(chunk_count_kernel, grid, dim3(kTopThreads), 0, st, t);
  if ((s = check_launch()) != KVC_OK) return s;
  hipLaunchKernelGGL(chunk_emit_kernel, grid, dim3(kTopThreads), 0, st, t);
  return check_launch();
}

// Pipelined scorer launch: one round of the workgroups the CUs hold at once,
// each walking an equal share of its head's chunks.
template <int KS, int PASS, int TPW>
kvc_status launch_pipe(const ScoreArgs& a, int B, hipStream_t st) {
  const void* k = reinterpret_cast<const void*>(&score_pipe_kernel<KS, PASS, TPW>);
  constexpr int bytes = PipeGeom<KS>::LDS;
  if (bytes > 65536) {  // idempotent; made on every launch (no state kept between calls)
    const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) {
      set_last_hip_error(e);
      return KVC_ERR_HIP;
    }
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  const int nchunk = ((PASS == 1 ? a.n : a.N) + PipeGeom<KS>::CH - 1) / PipeGeom<KS>::CH;
  const int heads = a.Hkv * B;
  const int per_head = std::max(1, std::min(nchunk, (PipeGeom<KS>::WGS * cus + heads - 1) / heads));
  hipLaunchKernelGGL((score_pipe_kernel<KS, PASS, TPW>), dim3(per_head, a.Hkv, B), dim3(64 * kPipeWaves), bytes, st, a);
  return check_launch();
}

template <int PASS>
kvc_status launch_pipe_any(const ScoreArgs& a, int KS, int B, hipStream_t st) {
  const bool t4 = a.R > 128;
#define KVC_PIPE(k) \
  case k: return t4 ? launch_pipe<k, PASS, 4>(a, B, st) : launch_pipe<k, PASS, 2>(a, B, st);
  switch (KS) {
    KVC_PIPE(1) KVC_PIPE(2) KVC_PIPE(4)
    default: return KVC_ERR_SHAPE;
  }
#undef KVC_PIPE
}
bool pipe_ok(int KS, int R) { return (KS == 1 || KS == 2 || KS == 4) && R <= 256; }

// The window scores: pass 1 and rowstat_kernel find each row's normalizer
// (unless a.lse gives them: pass 2 reads those directly), then pass 2.
template <typename T>
kvc_status run_scores(const ScoreArgs& a, int KS, int B, hipStream_t st) {
  constexpr int CH = ChunkCols<T>::value;
  const bool pipe = sizeof(T) == 2 && pipe_ok(KS, a.R);
  if (!a.lse) {
    kvc_status s = pipe ? launch_pipe_any<1>(a, KS, B, st) : launch_score<T, 1>(a, KS, dim3(a.nc1, a.Hkv, B), st);
    if (s != KVC_OK) return s;
    hipLaunchKernelGGL(rowstat_kernel, dim3((a.R + kRowsPerBlock - 1) / kRowsPerBlock, a.Hkv, B), dim3(kThreads), 0,
                       st, a);
    if ((s = check_launch()) != KVC_OK) return s;
  }
  return pipe ? launch_pipe_any<2>(a, KS, B, st) : launch_score<T, 2>(a, KS, dim3((a.N + CH - 1) / CH, a.Hkv, B), st);
}

// Launch of pool_topk_lds_kernel<KPT> with its padded score row in dynamic LDS
// (above the 64 KB default from KPT = 16 on).
template <int KPT> kvc_status launch_topk_lds(const TopArgs& t, int B, hipStream_t st) {
  constexpr size_t lds = static_cast<size_t>(KPT * kTopThreads + 2 * kMaxPoolHalf) * sizeof(float);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&pool_topk_lds_kernel<KPT>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) {
      set_last_hip_error(e);
      return KVC_ERR_HIP;
    }
  }
  hipLaunchKernelGGL(pool_topk_lds_kernel<KPT>, dim3(t.Hkv, B), dim3(kTopThreads), lds, st, t);
  return check_launch();
}

kvc_status run_topk(const TopArgs& t, int B, hipStream_t st) {
  if (chunked_topk(t.N)) return run_chunked_topk(t, B, st);
  // short rows: raw scores in LDS, keys in registers
  const int kpt = (t.N + kTopThreads - 1) / kTopThreads;
  if (kpt <= 8) return launch_topk_lds<8>(t, B, st);
  if (kpt <= 16) return launch_topk_lds<16>(t, B, st);
  return launch_topk_lds<32>(t, B, st);
}

// Position-only selection, the same for every (b, KV head): entry e of a row
// is e for the s leading sinks, else the candidate N - k' + e (the last k' - s
// candidates).  Grid-stride over the rows * k' entries.
constexpr int kRecentThreads = 256;
__global__ __launch_bounds__(kRecentThreads) void recent_kernel(int32_t* idx, size_t total, int kk, int s,
                                                                int base) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * kRecentThreads + threadIdx.x; i < total;
       i += static_cast<size_t>(gridDim.x) * kRecentThreads) {
    const int e = static_cast<int>(i % static_cast<size_t>(kk));
    idx[i] = e < s ? e : base + e;
  }
}

// Population variance over the N scores of each (b, KV head): one pass of
// float64 sums of x and x^2 (var = (sum x^2 - (sum x)^2 / N) / N), reduced in
// a fixed order (deterministic).  One 1024-thread workgroup per (b, j).
constexpr int kVarThreads = 1024;
__global__ __launch_bounds__(kVarThreads) void variance_kernel(const float* raw, int N, float* var) {
  __shared__ double sh[2][kVarThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* s = raw + static_cast<size_t>(blockIdx.x) * N;
  double a = 0.0, q = 0.0;
#pragma unroll 8
  for (int c = tid; c < N; c += kVarThreads) {
    const double x = s[c];
    a += x;
    q += x * x;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o);
    q += __shfl_xor(q, o);
  }
  if (lane == 0) {
    sh[0][w] = a;
    sh[1][w] = q;
  }
  __syncthreads();
  if (tid == 0) {
    double sa = 0.0, sq = 0.0;
    for (int i = 0; i < kVarThreads / 64; ++i) {
      sa += sh[0][i];
      sq += sh[1][i];
    }
    var[blockIdx.x] = static_cast<float>(fmax(sq - sa * sa / N, 0.0) / N);
  }
}

// Workspace of the scorer (per-chunk and per-row statistics) and of the top-k.
struct ScoreWs {
  int nc1;
  size_t stats, row, total;
};
ScoreWs score_ws(kvc_dtype dtype, int B, int Hkv, int G, int n, int D, int W) {
  const bool pipe = dtype != KVC_F32 && pipe_ok(D / 32, G * W);
  const int CH = pipe ? kPipeCH : dtype == KVC_F32 ? ChunkCols<float>::value : ChunkCols<uint16_t>::value;
  const size_t units = static_cast<size_t>(B) * Hkv;
  ScoreWs w;
  w.nc1 = (n + CH - 1) / CH;
  w.stats = align_up(units * w.nc1 * (G * W) * sizeof(float2), 256);
  w.row = align_up(units * (G * W) * sizeof(float2), 256);
  w.total = w.stats + w.row;
  return w;
}
struct TopWs {
  int nch;
  size_t keys, hist1, ghist, sel, cnt, total;
};
TopWs top_ws(int B, int Hkv, int N) {
  const size_t units = static_cast<size_t>(B) * Hkv;
  TopWs w;
  w.nch = (N + kChunk - 1) / kChunk;  // chunked top-k
  w.keys = align_up(units * w.nch * kChunk * sizeof(uint32_t), 256);
  w.hist1 = align_up(units * w.nch * 256 * sizeof(int), 256);
  w.ghist = align_up(units * 2 * kWideBins * sizeof(int), 256);
  w.sel = align_up(units * kSelSlots * sizeof(uint32_t), 256);
  w.cnt = align_up(units * w.nch * sizeof(int2), 256);
  w.total = w.keys + w.hist1 + w.ghist + w.sel + w.cnt;
  return w;
}

ScoreArgs score_args(const void* q_win, const void* k, int Hq, int Hkv, int n, int D, int W, const ScoreWs& sw,
                     char* w, float* raw) {
  ScoreArgs a;
  a.q_win = q_win;
  a.k = k;
  a.stats = reinterpret_cast<float2*>(w);
  a.rowstat = reinterpret_cast<float*>(w + sw.stats);
  a.raw = raw;
  a.lse = nullptr;
  a.lse_stride = 0;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.n = n;
  a.W = W;
  a.R = a.G * W;
  a.N = n - W;
  a.nc1 = sw.nc1;
  a.scale2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  return a;
}
TopArgs top_args(const float* raw, int Hkv, int N, int kk, int pool, const TopWs& tw, char* w, int32_t* idx,
                 float* scores) {
  TopArgs t;
  t.raw = raw;
  t.keys = reinterpret_cast<uint32_t*>(w);
  t.hist1 = reinterpret_cast<int*>(w + tw.keys);
  t.ghist = reinterpret_cast<int*>(w + tw.keys + tw.hist1);
  t.sel = reinterpret_cast<uint32_t*>(w + tw.keys + tw.hist1 + tw.ghist);
  t.cnt = reinterpret_cast<int2*>(w + tw.keys + tw.hist1 + tw.ghist + tw.sel);
  t.scores = scores;
  t.idx = idx;
  t.Hkv = Hkv;
  t.N = N;
  t.kk = kk;
  t.pool = pool;
  t.nch = tw.nch;
  t.NP = tw.nch * kChunk;
  t.ld = N;
  return t;
}
bool score_shape_ok(int B, int Hq, int Hkv, int n, int D, int W) {
  return B >= 1 && Hkv >= 1 && Hq >= 1 && Hq % Hkv == 0 && head_dim_ok(D) && n >= 1 && W >= 1 && W <= n;
}

}  // namespace

// idx rows of kk entries: the first s positions, then base + e (recent_kernel);
// with s = kk every row is 0, 1, ..., kk-1.
kvc_status launch_recent(int32_t* idx, size_t total, int kk, int s, int base, hipStream_t st) {
  const size_t blocks = std::min<size_t>((total + kRecentThreads - 1) / kRecentThreads, 4096);
  hipLaunchKernelGGL(recent_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kRecentThreads), 0, st, idx, total,
                     kk, s, base);
  return check_launch();
}
kvc_status launch_identity(int32_t* idx, size_t total, int kk, hipStream_t st) {
  return launch_recent(idx, total, kk, kk, 0, st);
}

// Population variance of each of `rows` rows of N floats (variance_kernel).
kvc_status launch_variance(const float* raw, int rows, int N, float* var, hipStream_t st) {
  hipLaunchKernelGGL(variance_kernel, dim3(rows), dim3(kVarThreads), 0, st, raw, N, var);
  return check_launch();
}

}  // namespace kvc

namespace kvc {
namespace {
// kvc_select and kvc_select_lse (lse NULL: the normalizers from pass 1).
kvc_status select_impl(const void* q_win, const void* k, const float* lse, int lse_stride, kvc_dtype dtype,
                       int32_t B, int32_t Hq, int32_t Hkv, int32_t n, int32_t D, int32_t W, int32_t pool,
                       int32_t budget, int32_t* idx, float* scores, void* ws, size_t* ws_bytes, void* stream) {
  if (!ws_bytes) return KVC_ERR_NULL;
  if (!dtype_ok(dtype)) return KVC_ERR_DTYPE;
  if (!score_shape_ok(B, Hq, Hkv, n, D, W) || pool < 1 || pool % 2 == 0) return KVC_ERR_SHAPE;
  const int N = n - W;
  const ScoreWs sw = score_ws(dtype, B, Hkv, Hq / Hkv, n, D, W);
  const TopWs tw = top_ws(B, Hkv, N);
  const size_t sz_raw = align_up(static_cast<size_t>(B) * Hkv * N * sizeof(float), 256);
  const size_t need = sw.total + sz_raw + tw.total;
  if (!ws) {
    *ws_bytes = need;
    return KVC_OK;
  }
  const int kk = budget < 0 ? N : std::min(budget, N);
  if (!q_win || !k || (kk > 0 && !idx)) return KVC_ERR_NULL;
  if (*ws_bytes < need) return KVC_ERR_WORKSPACE;
  if (N == 0) return KVC_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (kk == N && !scores) return launch_identity(idx, static_cast<size_t>(B) * Hkv * N, N, st);
  char* w = static_cast<char*>(ws);
  float* raw = reinterpret_cast<float*>(w + sw.total);
  ScoreArgs a = score_args(q_win, k, Hq, Hkv, n, D, W, sw, w, raw);
  a.lse = lse;
  a.lse_stride = lse_stride;
  const TopArgs t = top_args(raw, Hkv, N, kk, pool, tw, w + sw.total + sz_raw, idx, scores);
  kvc_status s = dtype == KVC_F32 ? run_scores<float>(a, D / 32, B, st) : run_scores<uint16_t>(a, D / 32, B, st);
  if (s != KVC_OK) return s;
  return run_topk(t, B, st);
}
}  // namespace
}  // namespace kvc

extern "C" kvc_status kvc_select(const void* q_win, const void* k, kvc_dtype dtype, int32_t B, int32_t Hq,
                                 int32_t Hkv, int32_t n, int32_t D, int32_t W, int32_t pool, int32_t budget,
                                 int32_t* idx, float* scores, void* ws, size_t* ws_bytes, void* stream) {
  return kvc::select_impl(q_win, k, nullptr, 0, dtype, B, Hq, Hkv, n, D, W, pool, budget, idx, scores, ws, ws_bytes,
                          stream);
}

extern "C" kvc_status kvc_select_lse(const void* q_win, const void* k, const float* lse, int32_t lse_stride,
                                     kvc_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t n, int32_t D,
                                     int32_t W, int32_t pool, int32_t budget, int32_t* idx, float* scores, void* ws,
                                     size_t* ws_bytes, void* stream) {
  if (!ws_bytes || (ws && !lse)) return KVC_ERR_NULL;
  if (lse_stride < W) return KVC_ERR_SHAPE;
  return kvc::select_impl(q_win, k, lse, lse_stride, dtype, B, Hq, Hkv, n, D, W, pool, budget, idx, scores, ws,
                          ws_bytes, stream);
}

extern "C" kvc_status kvc_window_scores(const void* q_win, const void* k, kvc_dtype dtype, int32_t B, int32_t Hq,
                                        int32_t Hkv, int32_t n, int32_t D, int32_t W, float* raw, float* var,
                                        void* ws, size_t* ws_bytes, void* stream) {
  using namespace kvc;
  if (!ws_bytes) return KVC_ERR_NULL;
  if (!dtype_ok(dtype)) return KVC_ERR_DTYPE;
  if (!score_shape_ok(B, Hq, Hkv, n, D, W)) return KVC_ERR_SHAPE;
  const int N = n - W;
  const ScoreWs sw = score_ws(dtype, B, Hkv, Hq / Hkv, n, D, W);
  if (!ws) {
    *ws_bytes = sw.total;
    return KVC_OK;
  }
  if (!q_win || !k || (N > 0 && !raw)) return KVC_ERR_NULL;
  if (*ws_bytes < sw.total) return KVC_ERR_WORKSPACE;
  if (N == 0) return KVC_OK;  // no candidates: nothing written (var included)
  hipStream_t st = static_cast<hipStream_t>(stream);
  const ScoreArgs a = score_args(q_win, k, Hq, Hkv, n, D, W, sw, static_cast<char*>(ws), raw);
  kvc_status s = dtype == KVC_F32 ? run_scores<float>(a, D / 32, B, st) : run_scores<uint16_t>(a, D / 32, B, st);
  if (s != KVC_OK || !var) return s;
  return launch_variance(raw, B * Hkv, N, var, st);
}

extern "C" kvc_status kvc_topk(const float* raw, int32_t B, int32_t Hkv, int32_t N, int32_t pool, int32_t budget,
                               int32_t* idx, float* scores, void* ws, size_t* ws_bytes, void* stream) {
  using namespace kvc;
  if (!ws_bytes) return KVC_ERR_NULL;
  if (B < 1 || Hkv < 1 || N < 0 || pool < 1 || pool % 2 == 0) return KVC_ERR_SHAPE;
  const TopWs tw = top_ws(B, Hkv, N);
  if (!ws) {
    *ws_bytes = tw.total;
    return KVC_OK;
  }
  const int kk = budget < 0 ? N : std::min(budget, N);
  if ((N > 0 && !raw) || (kk > 0 && !idx)) return KVC_ERR_NULL;
  if (*ws_bytes < tw.total) return KVC_ERR_WORKSPACE;
  if (N == 0) return KVC_OK;
  const TopArgs t = top_args(raw, Hkv, N, kk, pool, tw, static_cast<char*>(ws), idx, scores);
  return run_topk(t, B, static_cast<hipStream_t>(stream));
}

extern "C" kvc_status kvc_select_recent(int32_t B, int32_t Hkv, int32_t n, int32_t W, int32_t budget, int32_t sinks,
                                        int32_t* idx, void* stream) {
  using namespace kvc;
  if (B < 1 || Hkv < 1 || W < 1 || W > n || sinks < 0) return KVC_ERR_SHAPE;
  const int N = n - W;
  const int kk = budget < 0 ? N : std::min(budget, N);
  if (kk == 0) return KVC_OK;
  if (!idx) return KVC_ERR_NULL;
  return launch_recent(idx, static_cast<size_t>(B) * Hkv * kk, kk, std::min(sinks, kk), N - kk,
                       static_cast<hipStream_t>(stream));
}

extern "C" kvc_status kvc_select_h2o(const float* acc, int32_t B, int32_t Hkv, int32_t n, int32_t W, int32_t budget,
                                     int32_t* idx, void* ws, size_t* ws_bytes, void* stream) {
  using namespace kvc;
  if (!ws_bytes) return KVC_ERR_NULL;
  if (B < 1 || Hkv < 1 || W < 1 || W > n) return KVC_ERR_SHAPE;
  const int N = n - W;
  const TopWs tw = top_ws(B, Hkv, N);
  if (!ws) {
    *ws_bytes = tw.total;
    return KVC_OK;
  }
  const int kk = budget < 0 ? N : std::min(budget, N);
  if ((N > 0 && !acc) || (kk > 0 && !idx)) return KVC_ERR_NULL;
  if (*ws_bytes < tw.total) return KVC_ERR_WORKSPACE;
  if (N == 0) return KVC_OK;
  // the first n - W entries of each accumulated-attention row, no pooling
  TopArgs t = top_args(acc, Hkv, N, kk, 1, tw, static_cast<char*>(ws), idx, nullptr);
  t.ld = n;
  return run_topk(t, B, static_cast<hipStream_t>(stream));
}
