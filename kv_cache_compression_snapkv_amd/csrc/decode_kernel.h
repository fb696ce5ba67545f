// Single-query decode attention over the compressed cache (MiniKV Eq. 1 and
// Alg. 1 decoding; blog attention hook: one softmax over exact recent tokens and
// dequantized older ones; query head h reads KV head h / G).
//
// Work split.  The tokens of one (batch, KV head) are cut into 32-token tiles:
// ceil(Q/32) packed-history tiles (one or two key groups each) followed by the
// bf16 residual tiles.  Every wavefront owns a contiguous run of tiles for up to 4 query heads
// of that KV head and keeps its own online-softmax state; the waves of a
// workgroup merge through LDS, M = max m_w, o = sum_w 2^(m_w-M) o_w,
// l = sum_w 2^(m_w-M) l_w (log2 units), and write the output directly when one
// workgroup covers the whole (batch, KV head) -- short histories, 8 waves --
// else a partial that a small merge kernel combines the same way.  (No
// cross-workgroup atomics: a device-scope release fence costs an L2 write-back
// per wavefront.)  Within a wave the history tiles are software-pipelined: the
// key stage of tile t+1 and the value stage of tile t share each LDS barrier.
//
// Contractions on MFMA (v_mfma_f32_16x16x32_bf16).  A float32 operand value x is
// carried as two bf16 rows, hi = x truncated to bf16 and lo = (x - hi) truncated,
// so hi + lo holds 16 significant bits and products accumulate in fp32.
//   keys:   S[t] = sum_c A[c] B[c][t] with B = 1 + code*2^(pos-7): the code is
//           OR-ed into the mantissa of bf16 1.0 (one v_and_or_b32 per two codes)
//           and A = q*scale*2^(7-pos) per (group, channel) in rows 2h, 2h+1.
//           Rows 8+2h, 9+2h of the same operand hold -split(q*zero); one more
//           MFMA of that operand against all -1 gives, per head, the exact sum
//           of the A pieces (the 1.0 offset to remove) and the zero-point term.
//   values: o[c] = sum_t A[t] B[t][c] with the same code encoding and
//           A = p*scale*2^(7-pos) per (token, value group); each lane adds
//           p*zero - (hi + lo) for the pieces it wrote into a float32 register,
//           and the lanes of a group are summed once at the end of the run.
//   residual: B = bf16 keys/values as stored, A = q or p split in two.
//
// Group size GS (MiniKV Sec. 5.1 quantizes in groups of 16; KIVI in groups of
// 32).  Tiles are 32 tokens either way (an MFMA's k-depth for the values).
// GS = 32: one key group per tile; key column tile ct holds tokens
// {0..7,16..23} + 8ct, and one scaled operand serves both.  GS = 16: key column
// tile ct holds the tokens of key group ct (16ct..16ct+15), each with its own
// scaled operand and offset MFMA; each value MFMA covers 16 consecutive
// channels, one value group, with its own operand (two per 32 channels instead
// of one).  A history of an odd number of 16-token groups ends in a half tile:
// its second column tile is masked, and its value metadata is read from the
// first half (the slots past the history are never written, so their scales
// could be anything; codes and key data there only meet zero weights or masked
// scores).
#pragma once

#include "kvc_internal.h"

namespace kvc {
namespace {


constexpr int kHB = 4;    // query heads per workgroup (MFMA rows 2h, 2h+1)
constexpr int kTile = 32; // tokens per tile
constexpr int kXcds = 8;  // accelerator dies; workgroup i runs on die i % kXcds

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kOne2 = 0x3F803F80u;     // two bf16 1.0
constexpr uint32_t kNegOne2 = 0xBF80BF80u;  // two bf16 -1.0
constexpr uint32_t kHi = 0xFFFF0000u;
constexpr uint32_t kHighHalves = 0x07060302u;  // v_perm: high halves of (src1, src0)

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

// Global load, optionally with the non-temporal hint (streamed data read once:
// measured 12-15% more HBM bandwidth on this access pattern).
template <bool NT, typename V> __device__ __forceinline__ V ldg(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Load at a wave-uniform base plus a per-lane byte offset (the scalar-base
// addressing form: no per-lane 64-bit address arithmetic per tile).
template <bool NT, typename V> __device__ __forceinline__ V ldo(const uint32_t* base, uint32_t byte_off) {
  return ldg<NT>(reinterpret_cast<const V*>(reinterpret_cast<const unsigned char*>(base) + byte_off));
}

// A value the compiler must keep in a VGPR (VOP3 instructions such as
// v_and_or_b32 take no literal operand on this target).
__device__ __forceinline__ uint32_t vreg(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

struct Consts {
  uint32_t one, m0, m1, m2, m4;
};

// bf16 pair {hi(x0), hi(x1)} and {lo(x0), lo(x1)}: truncations of x and of its
// remainder.  eff0/eff1 = hi + lo as float (exact).
struct Pair {
  uint32_t hi, lo;
};
__device__ __forceinline__ Pair split_pair(float x0, float x1) {
  const uint32_t u0 = __float_as_uint(x0), u1 = __float_as_uint(x1);
  const float r0 = x0 - __uint_as_float(u0 & kHi);
  const float r1 = x1 - __uint_as_float(u1 & kHi);
  Pair p;
  p.hi = __builtin_amdgcn_perm(u1, u0, kHighHalves);
  p.lo = __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), kHighHalves);
  return p;
}
__device__ __forceinline__ float piece_sum(float x) {
  const float h = __uint_as_float(__float_as_uint(x) & kHi);
  return h + __uint_as_float(__float_as_uint(x - h) & kHi);
}

// Packed-word layout inside MFMA operands.  An operand is 4 registers, i.e. 8
// bf16 k-slots e = 0..7 (register e/2, half e%2).
//   2-bit word (16 codes, code i at bits 2i), half hf: k-slot e holds code
//     e/2 + 4*hf + 8*(e%2).  Two register forms:
//       wave-uniform hf: registers m = e/2 + 4*hf from w, w>>6, w>>12, the code
//         at bit position 2*(m%3) of each bf16 half (10 instructions per word);
//       per-lane hf: the hf = 0 form applied to w >> 8*hf, position
//         2*((e/2)%3) (6 instructions per half-word).
//   4-bit word (8 codes, code i at bits 4i): register m = e/2 holds codes
//     (m, m+4) at position 0 (from w>>4m).
template <int BITS> __device__ __forceinline__ int slot_code(int e, int hf) {
  return BITS == 2 ? (e >> 1) + 4 * hf + 8 * (e & 1) : (e >> 1) + 4 * (e & 1);
}
template <int BITS> __device__ __forceinline__ int slot_pos(int e, int hf, bool uniform) {
  return BITS == 2 ? 2 * (((e >> 1) + (uniform ? 4 * hf : 0)) % 3) : 0;
}
template <int BITS> __device__ __forceinline__ u32x4 unpack(uint32_t w, int hf, const Consts& k) {
  u32x4 r;
  if (BITS == 2) {
    const uint32_t w6 = w >> 6, w12 = w >> 12;
    if (hf == 0) {
      r.x = (w & k.m0) | k.one;
      r.y = (w & k.m1) | k.one;
      r.z = (w & k.m2) | k.one;
      r.w = (w6 & k.m0) | k.one;
    } else {
      r.x = (w6 & k.m1) | k.one;
      r.y = (w6 & k.m2) | k.one;
      r.z = (w12 & k.m0) | k.one;
      r.w = (w12 & k.m1) | k.one;
    }
  } else {
    r.x = (w & k.m4) | k.one;
    r.y = ((w >> 4) & k.m4) | k.one;
    r.z = ((w >> 8) & k.m4) | k.one;
    r.w = ((w >> 12) & k.m4) | k.one;
  }
  return r;
}
// 2-bit half-word chosen per lane: shift amount sh = 8*hf (a per-lane value).
__device__ __forceinline__ u32x4 unpack_lane(uint32_t w, uint32_t sh, const Consts& k) {
  return unpack<2>(w >> sh, 0, k);
}

// Keys: lane quarter lq, k-step s reads half-word hw = lq*KS + s of the
// token's codes (2-bit) or word lq*KS + s (4-bit).
template <int BITS, int KS> __device__ __forceinline__ int key_channel(int s, int lq, int e) {
  if (BITS == 2) {
    const int hw = lq * KS + s;
    return 16 * (hw >> 1) + slot_code<2>(e, hw & 1);
  }
  return 8 * (lq * KS + s) + slot_code<4>(e, 0);
}
template <int BITS, int KS> __device__ __forceinline__ int key_pos(int s, int lq, int e) {
  // the half is wave-uniform when KS is even
  return BITS == 2 ? slot_pos<2>(e, (lq * KS + s) & 1, (KS & 1) == 0) : 0;
}
// Values: lane quarter lq reads word row lq/2, half lq%2 (2-bit) or row lq (4-bit).
template <int BITS> __device__ __forceinline__ int value_token(int lq, int e) {
  if (BITS == 2) return 16 * (lq >> 1) + slot_code<2>(e, lq & 1);
  return 8 * lq + slot_code<4>(e, 0);
}
template <int BITS> __device__ __forceinline__ int value_pos(int lq, int e) {
  return BITS == 2 ? slot_pos<2>(e, lq & 1, false) : 0;
}
// Token of column n in key column tile ct.
template <int GS> __device__ __forceinline__ int col_token(int ct, int n) {
  return GS == 16 ? 16 * ct + n : 16 * (n >> 3) + (n & 7) + 8 * ct;
}
// Output MFMA i (of 2*KS, 16 channels each): the channel its lane ln's column
// holds, and the value group whose operand it takes.  GS = 32: MFMAs 2g, 2g+1
// take the even and odd channels of 32-channel group g; GS = 16: MFMA i takes
// channels 16i..16i+15, group i.
template <int GS> __device__ __forceinline__ int out_chan(int i, int ln) {
  return GS == 16 ? 16 * i + ln : 32 * (i >> 1) + 2 * ln + (i & 1);
}
template <int GS> __device__ __forceinline__ int out_group(int i) { return GS == 16 ? i : i >> 1; }

struct DecArgs {
  const void* q;
  const void* k_new;
  const void* v_new;
  const uint32_t *k_codes, *k_meta, *v_codes, *v_meta;
  uint16_t *k_res, *v_res;  // k_res [bj][r_cap][D], v_res [bj][D][r_cap]
  float* part_o;            // [bjh][nb][kHB][D] (used when nb > 1)
  float2* part_ml;          // [bjh][nb][kHB]
  float* out;               // [B][Hq][D]
  int B, Hq, Hkv, G, HB, hbs, q_cap, r_cap;  // hbs: query heads per workgroup (<= kHB)
  int q_len, r_total, r_new;
  int r_start;  // ring row of residual token 0 (residual token t is row (r_start + t) % r_cap)
  int nb;
  float scale2;  // log2(e)/sqrt(D)
  // Host-side index arithmetic (no integer division in the kernel's setup):
  float rcp_hkv, rcp_hb, rcp_xhb;      // 1/Hkv, 1/HB, 1/(kXcds*HB) for small_divmod
  int split_nA;                         // history split (see hist_split)
  float split_hA, split_hB;
  int sp_new;                           // wave of the unit holding the appended token's tile, or -1
};


// LDS layout (bytes), shared by host sizing and the kernel.  Operand areas hold
// the MFMA rows of 32 bf16 per k-step (keys) or channel group (values), padded
// so that both the 16-byte fragment reads (8 lanes, rows ln..ln+7) and the
// dword writes (lanes of two blocks) fall in distinct banks: rows are kRowW
// dwords apart and blocks blk_w(HBS) dwords (16 mod 32) apart.
//
// With HBS heads per workgroup only rows 2h, 2h+1, 8+2h, 9+2h (h < HBS) can be
// non-zero; for HBS < kHB those rows are stored compactly followed by one zero
// row that every other row maps to (the fragment reads of those lanes become
// broadcasts of the zero row).
constexpr int kRowW = 20;
__host__ __device__ constexpr int phys_rows(int hbs) { return hbs == kHB ? 16 : 4 * hbs + 1; }
__host__ __device__ constexpr int blk_w(int hbs) { return (phys_rows(hbs) * kRowW + 15) / 32 * 32 + 16; }
template <int HBS> __device__ __forceinline__ int arow(int r) {
  if (HBS == kHB) return r;
  const int h = (r & 7) >> 1;
  return h < HBS ? (r >> 3) * 2 * HBS + (r & 7) : 4 * HBS;
}
struct Lds {
  int wave0, wave_bytes, total;
  int ak, av, pbuf, vcorr, ring;  // offsets inside one wave's region
};
// Key operands per tile (one per key group) and value operands per tile (one
// per value group: D/GS of them).
__host__ __device__ constexpr int key_ops(int gs) { return 32 / gs; }
__host__ __device__ constexpr int val_ops(int KS, int gs) { return 32 * KS / gs; }
// value-correction slots per head (one per value group, at least 8)
__host__ __device__ constexpr int vcs_w(int KS, int gs) { return val_ops(KS, gs) > 8 ? val_ops(KS, gs) : 8; }
__host__ __device__ constexpr Lds lds_layout(int KS, int nwv, int hbs, int ring_bytes, int gs) {
  Lds L{};
  L.wave0 = 0;
  L.ak = 0;
  L.av = key_ops(gs) * KS * blk_w(hbs) * 4;
  L.pbuf = L.av + val_ops(KS, gs) * blk_w(hbs) * 4;
  L.vcorr = L.pbuf + hbs * 32 * 4;
  L.ring = (L.vcorr + hbs * vcs_w(KS, gs) * 4 + 15) / 16 * 16;
  // the final merge reuses the region for (o[hbs][D], m[hbs], l[hbs])
  L.ring = (L.ring > (hbs * 32 * KS + 2 * hbs) * 4) ? L.ring : ((hbs * 32 * KS + 2 * hbs) * 4 + 15) / 16 * 16;
  L.wave_bytes = L.ring + ring_bytes;
  L.total = L.wave0 + nwv * L.wave_bytes;
  return L;
}

// Staging of packed history tiles in LDS.  A tile image holds the tile's key
// codes, key meta, value meta and value codes back to back, copied from memory
// by direct-to-LDS loads of 16 bytes per lane (1 KB per instruction, whatever
// the pattern in which the lanes later read them: narrow or scattered loads
// straight into registers reach measurably less of the memory bandwidth).
// Used where kRingSlots images per wave still let kMinDmaBlocks 4-wave
// workgroups share a CU; elsewhere tiles go through registers.
constexpr int kRingSlots = 2;
constexpr int kMinDmaBlocks = 2;
constexpr int kLdsBytesPerCu = 160 * 1024;
// Image bytes: key codes 4*D*bits, key meta 4*D per key group, value meta
// 4*32 per value group, value codes 4*D*bits.
__host__ __device__ constexpr int img_bytes(int KS, int bits, int gs) {
  return 4 * 32 * KS * 2 * bits + 4 * 32 * KS * key_ops(gs) + 4 * 32 * val_ops(KS, gs);
}
__host__ __device__ constexpr int dma_blocks(int bits, int KS, int nwv, int hbs, int gs) {
  return nwv == 4 && hbs == 1
             ? kLdsBytesPerCu /
                   (4 * (lds_layout(KS, nwv, hbs, 0, gs).wave_bytes + kRingSlots * img_bytes(KS, bits, gs)))
             : 0;
}
__host__ __device__ constexpr bool use_dma(int bits, int KS, int nwv, int hbs, int gs) {
  return dma_blocks(bits, KS, nwv, hbs, gs) >= kMinDmaBlocks;
}
__host__ __device__ constexpr Lds kernel_lds(int bits, int KS, int nwv, int hbs, int gs) {
  return lds_layout(KS, nwv, hbs, use_dma(bits, KS, nwv, hbs, gs) ? kRingSlots * img_bytes(KS, bits, gs) : 0, gs);
}
template <bool B> struct Tag {
  static constexpr bool value = B;
};
// Wait until at most N vector-memory operations of this wave are outstanding
// (the direct-to-LDS loads are not tracked by the compiler's own waits).
template <int N> __device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Elements i, i+1 (i even) and i..i+7 (i % 8 == 0) of an input row as bf16
// pairs (low half = lower index), with one or two vector loads.
__device__ __forceinline__ uint32_t bf16_pair(float x0, float x1) {
  return static_cast<uint32_t>(f32_to_bf16(x0)) | (static_cast<uint32_t>(f32_to_bf16(x1)) << 16);
}
__device__ __forceinline__ float as_f32(float x) { return x; }
__device__ __forceinline__ float as_f32(uint16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ uint32_t load_bf16x2(const uint16_t* p, int i) {
  return *reinterpret_cast<const uint32_t*>(p + i);
}
__device__ __forceinline__ uint32_t load_bf16x2(const float* p, int i) {
  const float2 v = *reinterpret_cast<const float2*>(p + i);
  return bf16_pair(v.x, v.y);
}
__device__ __forceinline__ u32x4 load_bf16x8(const uint16_t* p, int i) {
  return *reinterpret_cast<const u32x4*>(p + i);
}
__device__ __forceinline__ u32x4 load_bf16x8(const float* p, int i) {
  const float4 a = *reinterpret_cast<const float4*>(p + i), b = *reinterpret_cast<const float4*>(p + i + 4);
  return u32x4{bf16_pair(a.x, a.y), bf16_pair(a.z, a.w), bf16_pair(b.x, b.y), bf16_pair(b.z, b.w)};
}

// All-reduce over the 16 lanes of a DPP row: swap neighbours, swap pairs,
// mirror within 8, mirror within 16.
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
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

// First history tile of wave w of a unit (w = NWT gives NTh): the prefix sums of
// a per-wave share that is non-increasing in w, rounded, so the runs partition
// [0, NTh).  Waves w >= NWT - NTr also hold a residual tile and get kResW fewer
// history tiles than the others (none if the even share is below kResW).  The
// shares (nA waves of hA tiles, then waves of hB tiles) come from the host.
constexpr float kResW = 5.0f;
struct SplitParams {
  int nA;
  float hA, hB;
};
inline SplitParams split_params(int NWT, int NTh, int NTr) {
  SplitParams p;
  if (NTr <= 0 || NTr >= NWT) {
    p.nA = NWT;
    p.hA = static_cast<float>(NTh) / static_cast<float>(NWT);
    p.hB = 0.0f;
  } else {
    p.nA = NWT - NTr;
    p.hB = std::max(0.0f, (static_cast<float>(NTh) + kResW * NTr) / NWT - kResW);
    p.hA = (static_cast<float>(NTh) - p.hB * NTr) / p.nA;
  }
  return p;
}
__device__ __forceinline__ int hist_split(int w, int NWT, int NTh, int nA, float hA, float hB) {
  if (w >= NWT) return NTh;
  const float c = static_cast<float>(min(w, nA)) * hA + static_cast<float>(max(w - nA, 0)) * hB;
  return min(NTh, static_cast<int>(c + 0.5f));
}

// Resident workgroups per CU that the register budget allows (the occupancy
// the planner assumes): 4-wave groups at up to 168 VGPRs fit three per CU.
template <int BITS, int KS, int NWV, int HBS, int GS> constexpr int min_blocks() {
  if (use_dma(BITS, KS, NWV, HBS, GS))
    return dma_blocks(BITS, KS, NWV, HBS, GS) < 4 ? dma_blocks(BITS, KS, NWV, HBS, GS) : 4;
  return NWV == 8 ? 1 : (KS <= 4 ? (HBS == 1 ? 4 : 3) : KS <= 6 ? 2 : 1);
}

// HBS: query heads per workgroup, kHB (up to four heads of a KV head) or 1
// (one head: multi-head attention, and the short runs).
// GS: quantization group (16 or 32).
template <typename T, int BITS, int KS, int NWV, int HBS, int GS>
__global__ __launch_bounds__(64 * NWV, (min_blocks<BITS, KS, NWV, HBS, GS>())) void decode_kernel(DecArgs a) {
  static_assert(GS == 16 || GS == 32, "group size");
  constexpr int D = 32 * KS;
  constexpr int NTHR = 64 * NWV;
  constexpr int NGV = D / GS;               // value channel groups (value operands per tile)
  constexpr int NKG = 32 / GS;              // key groups per tile (key operands per tile)
  constexpr int NO = 2 * KS;                // output MFMAs (16 channels each)
  constexpr int NW = D * BITS / 32;         // key words per token
  constexpr int NP = (D / 2 + 63) / 64;     // key operand pairs per lane per tile
  constexpr int NPV = (NGV * 16 + 63) / 64; // value operand pairs per lane per tile
  constexpr int VCS = vcs_w(KS, GS);        // value-correction slots per head
  constexpr int PAIR = BITS == 2 ? 8 : 4;   // code distance of the two halves of a register
  // History tiles in flight per wave, in two register rings: the key part of
  // tile t (codes, meta) is consumed one iteration before its value part, so
  // its slot frees earlier.  A slot is refilled as soon as it frees, so key
  // loads lead their use by NK-1 whole iterations and value loads by NV-1.
  // Each slot is a separate copy of the loop body (slots are compile-time), and
  // a short run executes most of its code once: two slots beat four there
  // (less code to fetch), and one slot exposes the load latency.
  constexpr int NK = 2;
  constexpr int NV = 2;
  constexpr int NPER = NK == NV ? NK : NK * NV;  // loop period (ring slots are compile-time)
  // Long runs stream each packed tile once; short runs share tiles between the
  // head workgroups of a unit through L2, so they keep the default policy.
  constexpr bool NTL = NWV == 4;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  // the wave index is wave-uniform: say so, so that tile indices, loop control
  // and tile base addresses live in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int ln = lane & 15, lq = lane >> 4;
  // Workgroup -> (unit bj, head block hb).  With one workgroup per unit and
  // several head blocks, the head blocks of a unit get linear ids 8 apart:
  // workgroups are dispatched round-robin over the 8 XCDs, so they share one L2
  // and the unit's packed cache is fetched from memory once.
  int bj, hb;
  {
    const int U = a.B * a.Hkv;
    const int L = blockIdx.y + gridDim.y * blockIdx.z;  // gridDim.x == 1 here when HB > 1
    if (gridDim.x == 1 && a.HB > 1) {
      const QR gr = small_divmod(L, kXcds * a.HB, a.rcp_xhb);
      const int ug = min(kXcds, U - gr.q * kXcds);  // units in this group
      if (ug == kXcds) {
        bj = gr.q * kXcds + gr.r % kXcds;
        hb = gr.r / kXcds;
      } else {
        const QR u = small_divmod(gr.r, ug, __builtin_amdgcn_rcpf(static_cast<float>(ug)));
        bj = gr.q * kXcds + u.r;
        hb = u.q;
      }
    } else {
      const QR yb = small_divmod(blockIdx.y, a.HB, a.rcp_hb);
      bj = blockIdx.z * a.Hkv + yb.q;
      hb = yb.r;
    }
  }
  const QR bq = small_divmod(bj, a.Hkv, a.rcp_hkv);
  const int b = bq.q, j = bq.r;
  const int bjh = bj * a.HB + hb;
  const int h0 = hb * a.hbs;
  const int Gb = min(a.hbs, a.G - h0);
  constexpr Lds L = kernel_lds(BITS, KS, NWV, HBS, GS);
  constexpr bool DMA = use_dma(BITS, KS, NWV, HBS, GS);
  constexpr int BLK = blk_w(HBS);
  const int rk = arow<HBS>(ln);  // operand row this lane reads
  unsigned char* wbase = smem + L.wave0 + wave * L.wave_bytes;
  uint16_t* AK = reinterpret_cast<uint16_t*>(wbase + L.ak);
  uint16_t* AV = reinterpret_cast<uint16_t*>(wbase + L.av);
  float* pbuf = reinterpret_cast<float*>(wbase + L.pbuf);
  float* vcs = reinterpret_cast<float*>(wbase + L.vcorr);

  Consts K;
  K.one = vreg(kOne2);
  K.m0 = vreg(0x00030003u);
  K.m1 = vreg(0x000C000Cu);
  K.m2 = vreg(0x00300030u);
  K.m4 = vreg(0x000F000Fu);

  const size_t qc = a.q_cap;
  const uint16_t* kr = a.k_res + static_cast<size_t>(bj) * a.r_cap * D;
  // With no packed history the (never used) prefetches read this unit's residual
  // keys instead: at least 32*D*2 bytes, more than one history tile's 16*D.
  const bool hist = a.q_len > 0;
  const uint32_t* kres32 = reinterpret_cast<const uint32_t*>(kr);
  const uint32_t* kc = hist ? a.k_codes + static_cast<size_t>(bj) * qc * NW : kres32;
  const uint32_t* km = hist ? a.k_meta + static_cast<size_t>(bj) * (qc / GS) * D : kres32;
  const uint32_t* vc = hist ? a.v_codes + static_cast<size_t>(bj) * (qc * BITS / 32) * D : kres32;
  const uint32_t* vm = hist ? a.v_meta + static_cast<size_t>(bj) * qc * NGV : kres32;
  const uint16_t* vr = a.v_res + static_cast<size_t>(bj) * D * a.r_cap;
  const T* knp = static_cast<const T*>(a.k_new) + static_cast<size_t>(bj) * D;
  const T* vnp = static_cast<const T*>(a.v_new) + static_cast<size_t>(bj) * D;
  auto rrow = [&](int t) {  // residual token -> ring row (t < r_cap)
    const int p = a.r_start + t;
    return p >= a.r_cap ? p - a.r_cap : p;
  };

  // Tiles of this wave: every NWT-th residual tile counted from the last wave,
  // and a contiguous run of history tiles.  When there are fewer residual tiles
  // than waves, the last NTr waves hold one each and take correspondingly fewer
  // history tiles (a residual tile costs about kResW history tiles: eight times
  // the bytes, loaded without prefetch), so the waves of a unit finish together.
  const int NWT = gridDim.x * NWV;  // waves of this unit
  const int sp = blockIdx.x * NWV + wave;
  const int NTh = (a.q_len + kTile - 1) / kTile;
  const int NTr = (a.r_total + kTile - 1) / kTile;
  // history tile whose second 16 tokens lie past the history (odd group count), or -1
  const int half_tile = (a.q_len % kTile) != 0 ? NTh - 1 : -1;
  const int tb = hist_split(sp, NWT, NTh, a.split_nA, a.split_hA, a.split_hB);
  const int th_end = hist_split(sp + 1, NWT, NTh, a.split_nA, a.split_hA, a.split_hB);
  const int r_first = NWT - 1 - sp;  // residual tiles r_first, r_first + NWT, ...
  // Every prefetch is issued on every path (clamped to an existing tile) so the
  // number of loads in flight is the same at each wait and the compiler can wait
  // for exactly the tile it needs.
  const int hlast = max(th_end - 1, 0);

  // Per tile, D/2 key operand pairs and D/2 value operand pairs; lane l owns
  // pairs l + 64u for every head, so its meta loads do not depend on the head.
  constexpr int NKW = (BITS == 2) ? KS / 2 + (KS & 1) : KS;  // key words a lane reads per token
  struct KRegs {
    uint32_t kw[2][NKW];     // key code words, per column tile
    uint32_t km[NKG][NP][2]; // key meta of the lane's channel pairs, per key group
  };
  struct VRegs {
    uint32_t vm[NPV][2];  // value meta of the lane's token pairs
    uint32_t vw[NO];      // value code words, per output MFMA
  };
  // Per-lane byte offsets inside a tile (the tile bases are wave-uniform).
  const int w_first = (BITS == 2) ? ((lq * KS) >> 1) : lq * KS;
  constexpr uint32_t kCtRows = GS == 16 ? 16 : 8;  // token offset of column tile 1
  const uint32_t off_k = static_cast<uint32_t>(col_token<GS>(0, ln) * NW + w_first) * 4u;  // + ct * kCtRows rows
  uint32_t off_km[NP], off_vm[NPV], off_vm_h[NPV];  // off_vm_h: the half tile's (second half read from the first)
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int pi = min(lane + 64 * u, D / 2 - 1);
    const int s = pi >> 4, q4 = (pi >> 2) & 3, m = pi & 3;
    off_km[u] = static_cast<uint32_t>(key_channel<BITS, KS>(s, q4, 2 * m)) * 4u;  // + PAIR channels, + D per group
  }
#pragma unroll
  for (int u = 0; u < NPV; ++u) {
    const int pi = min(lane + 64 * u, NGV * 16 - 1);
    const int g = pi >> 4, pr = pi & 15;
    const int tok = value_token<BITS>(pr >> 2, 2 * (pr & 3));  // the pair's first token; + PAIR in the same half
    off_vm[u] = static_cast<uint32_t>(tok * NGV + g) * 4u;
    off_vm_h[u] = static_cast<uint32_t>((tok >= 16 ? tok - 16 : tok) * NGV + g) * 4u;
  }
  // value code words: row lq/2 (2-bit) or lq (4-bit); GS = 32: channels
  // 32g + 2ln, +1 (one 8-byte load per group), GS = 16: channel 16i + ln
  const uint32_t off_vw =
      static_cast<uint32_t>(((BITS == 2) ? (lq >> 1) : lq) * D + (GS == 16 ? ln : 2 * ln)) * 4u;
  // A tile's key part (codes at kt, meta at kmg) and value part (meta at vmt,
  // codes at vct) into registers, from memory or from a staged LDS image.
  auto read_k = [&](const uint32_t* kt, const uint32_t* kmg, KRegs& r, auto tag) {
    constexpr bool nt = decltype(tag)::value;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const uint32_t o = off_k + ct * kCtRows * NW * 4;
      if constexpr (NKW == 4 && (BITS == 4 || (KS & 1) == 0)) {
        const u32x4 w4 = ldo<nt, u32x4>(kt, o);
        r.kw[ct][0] = w4.x; r.kw[ct][1] = w4.y; r.kw[ct][2] = w4.z; r.kw[ct][3] = w4.w;
      } else if constexpr (NKW == 2 && (BITS == 4 || (KS & 1) == 0)) {
        const u32x2 w2 = ldo<nt, u32x2>(kt, o);
        r.kw[ct][0] = w2.x; r.kw[ct][1] = w2.y;
      } else {
#pragma unroll
        for (int i = 0; i < NKW; ++i) r.kw[ct][i] = (w_first + i < NW) ? ldo<nt, uint32_t>(kt, o + 4 * i) : 0u;
      }
    }
#pragma unroll
    for (int g = 0; g < NKG; ++g)
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        r.km[g][u][0] = r.km[g][u][1] = 0u;
        if (lane + 64 * u < D / 2) {
          r.km[g][u][0] = ldo<nt, uint32_t>(kmg, off_km[u] + g * D * 4);
          r.km[g][u][1] = ldo<nt, uint32_t>(kmg, off_km[u] + g * D * 4 + PAIR * 4);
        }
      }
  };
  auto read_v = [&](const uint32_t* vmt, const uint32_t* vct, VRegs& r, auto tag, bool half) {
    constexpr bool nt = decltype(tag)::value;
#pragma unroll
    for (int u = 0; u < NPV; ++u) {
      r.vm[u][0] = r.vm[u][1] = 0u;
      if (lane + 64 * u < NGV * 16) {
        const uint32_t o = half ? off_vm_h[u] : off_vm[u];
        r.vm[u][0] = ldo<nt, uint32_t>(vmt, o);
        r.vm[u][1] = ldo<nt, uint32_t>(vmt, o + PAIR * NGV * 4);
      }
    }
    if constexpr (GS == 32) {
#pragma unroll
      for (int g = 0; g < KS; ++g) {
        const u32x2 w = ldo<nt, u32x2>(vct, off_vw + 128 * g);
        r.vw[2 * g] = w.x;
        r.vw[2 * g + 1] = w.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NO; ++i) r.vw[i] = ldo<nt, uint32_t>(vct, off_vw + 64 * i);
    }
  };
  auto k_tile = [&](int tile) { return kc + static_cast<size_t>(tile) * kTile * NW; };
  auto km_tile = [&](int tile) { return km + static_cast<size_t>(tile) * NKG * D; };
  auto vm_tile = [&](int tile) { return vm + static_cast<size_t>(tile) * kTile * NGV; };
  auto vc_tile = [&](int tile) { return vc + static_cast<size_t>(tile) * (kTile * BITS / 32) * D; };
  auto load_k = [&](int tile, KRegs& r) { read_k(k_tile(tile), km_tile(tile), r, Tag<NTL>{}); };
  auto load_v = [&](int tile, VRegs& r) {
    read_v(vm_tile(tile), vc_tile(tile), r, Tag<NTL>{}, GS == 16 && tile == half_tile);
  };

  // LDS staging (DMA kernels): ring slot i holds the key part of tile ka and the
  // value part of tile vb, i.e. what one pipelined iteration consumes.
  constexpr int IMG = img_bytes(KS, BITS, GS);
  constexpr int IMG_KM = 4 * D * BITS, IMG_VM = IMG_KM + 4 * D * NKG, IMG_VC = IMG_VM + 4 * kTile * NGV;
  constexpr int VM_HALF = 4 * 16 * NGV;  // value meta bytes of 16 tokens
  constexpr int NDMA = (IMG + 1023) / 1024;  // direct-to-LDS loads per slot fill
  unsigned char* ring = wbase + L.ring;
  auto dma_fill = [&](int ka, int vb, int slot) {
    if constexpr (DMA) {
      unsigned char* dst = ring + slot * IMG;
      const unsigned char* kcb = reinterpret_cast<const unsigned char*>(k_tile(ka));
      const unsigned char* kmb = reinterpret_cast<const unsigned char*>(km_tile(ka));
      const unsigned char* vmb = reinterpret_cast<const unsigned char*>(vm_tile(vb));
      const unsigned char* vcb = reinterpret_cast<const unsigned char*>(vc_tile(vb));
      const bool vhalf = GS == 16 && vb == half_tile;
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const uint32_t e = 1024u * i + 16u * static_cast<uint32_t>(lane);  // image byte this lane copies
        if (e < static_cast<uint32_t>(IMG)) {
          uint32_t evm = e - IMG_VM;  // value meta: the half tile's second half from its first
          if (vhalf && evm >= VM_HALF) evm -= VM_HALF;
          const unsigned char* src = e < IMG_KM   ? kcb + e
                                     : e < IMG_VM ? kmb + (e - IMG_KM)
                                     : e < IMG_VC ? vmb + evm
                                                  : vcb + (e - IMG_VC);
          __builtin_amdgcn_global_load_lds(src, dst + 1024 * i, 16, 0, 2 /* non-temporal */);
        }
      }
    }
  };
  auto slot_k = [&](int slot, KRegs& r) {
    const unsigned char* img = ring + slot * IMG;
    read_k(reinterpret_cast<const uint32_t*>(img), reinterpret_cast<const uint32_t*>(img + IMG_KM), r, Tag<false>{});
  };
  auto slot_v = [&](int slot, VRegs& r) {
    const unsigned char* img = ring + slot * IMG;
    read_v(reinterpret_cast<const uint32_t*>(img + IMG_VM), reinterpret_cast<const uint32_t*>(img + IMG_VC), r,
           Tag<false>{}, false);
  };

  // ---------------------------------------------------------------- setup
  // Each wave loads the query values of its lanes' key channel pairs (they never
  // change) and its first history tiles before anything waits; meanwhile its
  // operand rows that no head writes are zeroed.  No workgroup barrier.
  const T* qp = static_cast<const T*>(a.q) + (static_cast<size_t>(b) * a.Hq + j * a.G + h0) * D;
  // loaded as stored and converted after every setup load is issued, so that no
  // load waits for the query's
  T qr0[NP][HBS], qr1[NP][HBS];
  int cpair[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int pi = min(lane + 64 * u, D / 2 - 1);
    const int s = pi >> 4, q4 = (pi >> 2) & 3, m = pi & 3;
    cpair[u] = key_channel<BITS, KS>(s, q4, 2 * m);
#pragma unroll
    for (int h = 0; h < HBS; ++h) {
      const int hc = min(h, Gb - 1);
      qr0[u][h] = qp[hc * D + cpair[u]];
      qr1[u][h] = qp[hc * D + cpair[u] + PAIR];
    }
  }
  // ---- residual tiles are bf16 as stored.  A lane holds, per tile, the 8
  // tokens from 8*lq of its NO value channels (out_chan) and the 8-channel
  // slices of its two key columns; the appended token (not yet in the ring)
  // comes from the inputs: its key channels 32s+8lq.. and value channels
  // out_chan(i, ln) for substitution, and channels lane+64i for storing it into
  // the ring.
  struct ResRegs {
    u32x4 v[NO];
    u32x4 k[2][KS];
  };
  constexpr int NST = (D + 63) / 64;
  struct NewRegs {
    u32x4 kn[KS];
    uint32_t vn[NO];  // bf16 in the low half
    T st_k[NST], st_v[NST];  // as stored in the inputs
  };
  auto res_load = [&](int rt, ResRegs& r) {
    const int t0 = rt * kTile;
    const int tlc = rrow(min(t0 + 8 * lq, (a.r_total - 1) & ~7));  // an in-range 8-token chunk (ring row)
#pragma unroll
    for (int i = 0; i < NO; ++i)
      r.v[i] = *reinterpret_cast<const u32x4*>(vr + static_cast<size_t>(out_chan<GS>(i, ln)) * a.r_cap + tlc);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int tc = rrow(min(t0 + col_token<GS>(ct, ln), a.r_total - 1));
#pragma unroll
      for (int s = 0; s < KS; ++s)
        r.k[ct][s] = *reinterpret_cast<const u32x4*>(kr + static_cast<size_t>(tc) * D + 32 * s + 8 * lq);
    }
  };
  auto res_new = [&](NewRegs& n) {
#pragma unroll
    for (int s = 0; s < KS; ++s) n.kn[s] = load_bf16x8(knp, 32 * s + 8 * lq);
#pragma unroll
    for (int i = 0; i < NO; ++i) n.vn[i] = f32_to_bf16(load_f32(vnp, out_chan<GS>(i, ln)));
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int c = min(lane + 64 * i, D - 1);
      n.st_k[i] = knp[c];
      n.st_v[i] = vnp[c];
    }
  };
  // This wave processes the tile holding the appended token (if any).
  const int r_new_tile = a.r_new >= 0 ? a.r_new / kTile : -1;
  const bool new_here = sp == a.sp_new;  // r_new_tile is r_first + a multiple of NWT
  // Short runs: a wave with no history tiles issues its first residual tile's
  // loads and the appended token's at once, with the query loads (one memory
  // round trip before its first result instead of three).  Elsewhere the tile
  // loads are issued when the tile starts (fewer registers held).
  constexpr bool kEarly = NWV == 8 && KS <= 4;
  const bool early = kEarly && tb >= th_end && r_first < NTr;
  ResRegs rres;
  NewRegs rnew;

  // register rings (no staging) or ring slots: fill f holds the key part of
  // tile tb+f and the value part of tile tb+f-1
  KRegs kring[DMA ? 1 : NK];
  VRegs vring[DMA ? 1 : NV];
  if constexpr (DMA) {
#pragma unroll
    for (int f = 0; f < kRingSlots; ++f) dma_fill(min(tb + f, hlast), min(max(tb + f - 1, 0), hlast), f);
  } else if (early) {
    res_load(r_first, rres);
  } else {
#pragma unroll
    for (int u = 0; u < NK; ++u) load_k(min(tb + u, hlast), kring[u]);
#pragma unroll
    for (int u = 0; u < NV; ++u) load_v(min(tb + u, hlast), vring[u]);
  }
  if (early && new_here) res_new(rnew);
  {
    uint32_t* zero_area = reinterpret_cast<uint32_t*>(wbase);
    for (int e = lane; e < (L.pbuf >> 2); e += 64) zero_area[e] = 0u;  // AK and AV of this wave
  }
  wave_sync();
  // scores come out of the MFMAs already in log2 units: q is scaled once
  float qa0[NP][HBS], qa1[NP][HBS];
#pragma unroll
  for (int u = 0; u < NP; ++u)
#pragma unroll
    for (int h = 0; h < HBS; ++h) {
      qa0[u][h] = as_f32(qr0[u][h]) * a.scale2;
      qa1[u][h] = as_f32(qr1[u][h]) * a.scale2;
    }

  f32x4 oacc[NO];
#pragma unroll
  for (int i = 0; i < NO; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float vcorr[NPV][HBS];
#pragma unroll
  for (int u = 0; u < NPV; ++u)
#pragma unroll
    for (int h = 0; h < HBS; ++h) vcorr[u][h] = 0.0f;
  float m_run[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.f, 0.f};
  const u32x4 neg4 = {vreg(kNegOne2), vreg(kNegOne2), vreg(kNegOne2), vreg(kNegOne2)};
  const uint32_t vsh = 8u * static_cast<uint32_t>(lq & 1);  // value half-word of this lane (2-bit)
  const int nhh = (HBS > 1 && Gb > 1) ? 2 : 1;              // head rows per lane quarter in use

  // ---- the online softmax update shared by both tile kinds.  x[hh][ct] are
  // log2-scaled scores (-inf when masked); writes p to pbuf and rescales the
  // accumulators when a running max moves (skipped when no lane's moves, which
  // leaves the result bit-identical).
  auto softmax_update = [&](float (&x)[2][2]) {
    float alpha[2] = {1.0f, 1.0f};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (hh >= nhh) continue;  // no lane holds a second head
      const float mt = max16(fmaxf(x[hh][0], x[hh][1]));
      const float mnew = fmaxf(m_run[hh], mt);
      if (mnew == -INFINITY) {
        x[hh][0] = x[hh][1] = 0.0f;
      } else {
        // arguments are <= 0 (or -inf): the hardware exp2 is exact enough and
        // needs no range reduction
        alpha[hh] = __builtin_amdgcn_exp2f(m_run[hh] - mnew);
        x[hh][0] = __builtin_amdgcn_exp2f(x[hh][0] - mnew);
        x[hh][1] = __builtin_amdgcn_exp2f(x[hh][1] - mnew);
      }
      m_run[hh] = mnew;
      l_part[hh] = l_part[hh] * alpha[hh] + x[hh][0] + x[hh][1];
      const int head = 2 * lq + hh;
      if (head < Gb) {
        pbuf[head * 32 + col_token<GS>(0, ln)] = x[hh][0];
        pbuf[head * 32 + col_token<GS>(1, ln)] = x[hh][1];
      }
    }
    if (__any(alpha[0] != 1.0f || alpha[1] != 1.0f)) {
#pragma unroll
      for (int i = 0; i < NO; ++i) {
        oacc[i][0] *= alpha[0];
        oacc[i][1] *= alpha[0];
        if constexpr (HBS > 1) {  // rows 2-3 of a lane quarter hold the second head
          oacc[i][2] *= alpha[1];
          oacc[i][3] *= alpha[1];
        }
      }
      // per-head factors for the value corrections (lanes of quarter h/2 hold head h)
#pragma unroll
      for (int h = 0; h < HBS; ++h) {
        const float ah = HBS == 1 ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha[0]), 0))
                                  : __shfl(alpha[h & 1], 16 * (h >> 1));
#pragma unroll
        for (int u = 0; u < NPV; ++u) vcorr[u][h] *= ah;
      }
    }
  };

  // ---- key stage of a history tile: in the operand of each key group,
  // rows 2h, 2h+1 = split(q*scale*2^(7-pos)), rows 8+2h, 9+2h = -split(q*zero)
  auto k_stage = [&](const KRegs& cur) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int pi = lane + 64 * u;
      if (pi < D / 2) {
        const int s = pi >> 4, q4 = (pi >> 2) & 3, m = pi & 3;
        const float f = static_cast<float>(1 << (7 - key_pos<BITS, KS>(s, q4, 2 * m)));
#pragma unroll
        for (int g = 0; g < NKG; ++g) {
          const float sc0 = f16_bits_to_f32(cur.km[g][u][0] & 0xFFFFu) * f;
          const float sc1 = f16_bits_to_f32(cur.km[g][u][1] & 0xFFFFu) * f;
          const float zp0 = f16_bits_to_f32(cur.km[g][u][0] >> 16), zp1 = f16_bits_to_f32(cur.km[g][u][1] >> 16);
          uint32_t* dst = reinterpret_cast<uint32_t*>(AK) + (g * KS + s) * BLK + 4 * q4 + m;
#pragma unroll
          for (int h = 0; h < HBS; ++h) {
            if (h < Gb) {
              const Pair pa = split_pair(qa0[u][h] * sc0, qa1[u][h] * sc1);
              const Pair pz = split_pair(qa0[u][h] * zp0, qa1[u][h] * zp1);
              dst[arow<HBS>(2 * h) * kRowW] = pa.hi;
              dst[arow<HBS>(2 * h + 1) * kRowW] = pa.lo;
              dst[arow<HBS>(8 + 2 * h) * kRowW] = pz.hi ^ 0x80008000u;
              dst[arow<HBS>(9 + 2 * h) * kRowW] = pz.lo ^ 0x80008000u;
            }
          }
        }
      }
    }
  };
  // ---- key MFMAs of a history tile (operand rows visible): log2-scaled
  // scores; column tile ct takes key group ct's operand (GS = 16) or the one
  // operand (GS = 32).  A half tile's second column tile is masked.
  auto k_mma = [&](const KRegs& cur, float (&x)[2][2], bool half) {
    f32x4 accS[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 accC[NKG];
#pragma unroll
    for (int g = 0; g < NKG; ++g) accC[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 af[NKG];
#pragma unroll
      for (int g = 0; g < NKG; ++g)
        af[g] = *reinterpret_cast<const u32x4*>(AK + 2 * ((g * KS + s) * BLK + rk * kRowW + 4 * lq));
      const u32x4& af1 = af[NKG - 1];
      if constexpr (BITS == 2 && (KS & 1) == 0) {
        accS[0] = mfma(af[0], unpack<2>(cur.kw[0][s >> 1], s & 1, K), accS[0]);
        accS[1] = mfma(af1, unpack<2>(cur.kw[1][s >> 1], s & 1, K), accS[1]);
      } else if constexpr (BITS == 2) {
        const int hw0 = (lq * KS) & 1;  // parity of the lane's first half-word
        const uint32_t sh = 8 * ((hw0 + s) & 1);
        const int i0 = s >> 1, i1 = (s + 1) >> 1;  // word index for hw0 == 0 / hw0 == 1
        const uint32_t kw0 = hw0 ? cur.kw[0][i1] : cur.kw[0][i0];
        const uint32_t kw1 = hw0 ? cur.kw[1][i1] : cur.kw[1][i0];
        accS[0] = mfma(af[0], unpack_lane(kw0, sh, K), accS[0]);
        accS[1] = mfma(af1, unpack_lane(kw1, sh, K), accS[1]);
      } else {
        accS[0] = mfma(af[0], unpack<4>(cur.kw[0][s], 0, K), accS[0]);
        accS[1] = mfma(af1, unpack<4>(cur.kw[1][s], 0, K), accS[1]);
      }
#pragma unroll
      for (int g = 0; g < NKG; ++g) accC[g] = mfma(af[g], neg4, accC[g]);
    }
    // lanes of quarters 0-1 hold rows 0-7 (minus the offset of heads 2lq, 2lq+1),
    // quarters 2-3 rows 8-15 (their zero-point terms)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float corr[NKG];
#pragma unroll
      for (int g = 0; g < NKG; ++g) {
        const float own = accC[g][2 * hh] + accC[g][2 * hh + 1];
        // lanes 0-31 take the zero-point sums of lanes 32-63
        corr[g] = own + __uint_as_float(__builtin_amdgcn_permlane32_swap(
                            __float_as_uint(own), __float_as_uint(own), false, false)[1]);
      }
      const bool ok = 2 * lq + hh < Gb;
      x[hh][0] = ok ? accS[0][2 * hh] + accS[0][2 * hh + 1] + corr[0] : -INFINITY;
      x[hh][1] = ok && !half ? accS[1][2 * hh] + accS[1][2 * hh + 1] + corr[NKG - 1] : -INFINITY;
    }
  };
  // ---- value stage of a history tile: in the operand of each value group,
  // rows 2h, 2h+1 = split(p*scale*2^(7-pos)); the lane keeps p*zero - (hi + lo)
  // of its pieces in vcorr
  auto v_stage = [&](const VRegs& cur) {
#pragma unroll
    for (int u = 0; u < NPV; ++u) {
      const int vi = lane + 64 * u;
      if (vi < NGV * 16) {
        const int g = vi >> 4, pr = vi & 15, q4 = pr >> 2, m = pr & 3;
        const int t_lo = value_token<BITS>(q4, 2 * m), t_hi = t_lo + PAIR;
        const float f = static_cast<float>(1 << (7 - value_pos<BITS>(q4, 2 * m)));
        const float sc0 = f16_bits_to_f32(cur.vm[u][0] & 0xFFFFu) * f;
        const float sc1 = f16_bits_to_f32(cur.vm[u][1] & 0xFFFFu) * f;
        const float zp0 = f16_bits_to_f32(cur.vm[u][0] >> 16), zp1 = f16_bits_to_f32(cur.vm[u][1] >> 16);
        uint32_t* dst = reinterpret_cast<uint32_t*>(AV) + g * BLK + pr;
#pragma unroll
        for (int h = 0; h < HBS; ++h) {
          if (h < Gb) {
            const float p0 = pbuf[h * 32 + t_lo], p1 = pbuf[h * 32 + t_hi];
            const float x0 = p0 * sc0, x1 = p1 * sc1;
            const Pair pa = split_pair(x0, x1);
            dst[arow<HBS>(2 * h) * kRowW] = pa.hi;
            dst[arow<HBS>(2 * h + 1) * kRowW] = pa.lo;
            vcorr[u][h] += (__builtin_fmaf(p0, zp0, -piece_sum(x0)) + __builtin_fmaf(p1, zp1, -piece_sum(x1)));
          }
        }
      }
    }
  };
  // ---- value MFMAs of a history tile (output MFMA i takes value group out_group(i))
  auto v_mma = [&](const VRegs& cur) {
    u32x4 af;
#pragma unroll
    for (int i = 0; i < NO; ++i) {
      if (GS == 16 || (i & 1) == 0)
        af = *reinterpret_cast<const u32x4*>(AV + 2 * (out_group<GS>(i) * BLK + rk * kRowW + 4 * lq));
      if constexpr (BITS == 2) oacc[i] = mfma(af, unpack_lane(cur.vw[i], vsh, K), oacc[i]);
      else oacc[i] = mfma(af, unpack<4>(cur.vw[i], 0, K), oacc[i]);
    }
  };

  // ---- packed history tiles [tb, th_end), software-pipelined: the key stage
  // of tile t+1 and the value stage of tile t share each barrier.  Tile tb+i
  // lives in kring[i % NK] and vring[i % NV]; the key slot of tile t+1 is
  // refilled with tile t+1+NK once its key MFMAs are issued, the value slot of
  // tile t with tile t+NV once its value MFMAs are.
  if constexpr (DMA) {
    // Iteration tt consumes fill tt-tb+1 (slot (tt-tb+1) % kRingSlots) and then
    // refills that slot kRingSlots fills ahead; before a slot is read, only the
    // younger fills may still be in flight.
    constexpr int kWait = (kRingSlots - 1) * NDMA;
    wait_vmem<kWait>();
    if (tb < th_end) {
      KRegs k0;
      slot_k(0, k0);
      k_stage(k0);
      wave_sync();
      float x[2][2];
      k_mma(k0, x, GS == 16 && tb == half_tile);
      softmax_update(x);
      wave_sync();
    }
    dma_fill(min(tb + kRingSlots, hlast), min(tb + kRingSlots - 1, hlast), 0);
    for (int t = tb; t < th_end; t += kRingSlots) {
#pragma unroll
      for (int u = 0; u < kRingSlots; ++u) {
        const int tt = t + u;
        const int slot = (u + 1) % kRingSlots;
        if (tt < th_end) {
          const bool nxt = tt + 1 < th_end;
          wait_vmem<kWait>();
          KRegs kn;
          VRegs vcur;
          slot_k(slot, kn);
          slot_v(slot, vcur);
          // unconditional: the last iteration's key part is a clamped copy of
          // an existing tile, and its operand rows are never read
          k_stage(kn);
          v_stage(vcur);
          wave_sync();
          float x[2][2];
          if (nxt) k_mma(kn, x, GS == 16 && tt + 1 == half_tile);
          v_mma(vcur);
          if (nxt) softmax_update(x);
          wave_sync();
        }
        dma_fill(min(tt + 1 + kRingSlots, hlast), min(tt + kRingSlots, hlast), slot);
      }
    }
    wait_vmem<0>();  // no copy may land in this wave's LDS after it moves on
  } else {
  if (tb < th_end) {
    k_stage(kring[0]);
    wave_sync();
    float x[2][2];
    k_mma(kring[0], x, GS == 16 && tb == half_tile);
    softmax_update(x);
    wave_sync();
  }
  load_k(min(tb + NK, hlast), kring[0]);
  for (int t = tb; t < th_end; t += NPER) {
#pragma unroll
    for (int u = 0; u < NPER; ++u) {
      const int tt = t + u;
      KRegs& kn = kring[(u + 1) % NK];
      VRegs& vcur = vring[u % NV];
      if (tt < th_end) {
        const bool nxt = tt + 1 < th_end;
        k_stage(kn);  // unconditional, as above
        v_stage(vcur);
        wave_sync();
        float x[2][2];
        if (nxt) k_mma(kn, x, GS == 16 && tt + 1 == half_tile);
        v_mma(vcur);
        if (nxt) softmax_update(x);
        wave_sync();
      }
      load_k(min(tt + 1 + NK, hlast), kn);
      load_v(min(tt + NV, hlast), vcur);
    }
  }
  }

  // ---- residual tiles: bf16 keys/values as stored (appended token from the
  // input).  Their key operand split(q), in natural channel order, goes to this
  // wave's key area (no longer needed): rows 2h, 2h+1 for h < Gb, zeros elsewhere.
  if (r_first < NTr) {
    uint32_t* ak32 = reinterpret_cast<uint32_t*>(AK);
    for (int e = lane; e < KS * BLK; e += 64) ak32[e] = 0u;
    wave_sync();
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      if (lane + 64 * u < D / 2) {
#pragma unroll
        for (int h = 0; h < HBS; ++h) {
          if (h < Gb) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const int c = cpair[u] + i * PAIR;
              const float v = i ? qa1[u][h] : qa0[u][h];
              const float r = v - __uint_as_float(__float_as_uint(v) & kHi);
              uint16_t* blk = AK + 2 * ((c >> 5) * BLK) + (c & 31);
              blk[2 * arow<HBS>(2 * h) * kRowW] = static_cast<uint16_t>(__float_as_uint(v) >> 16);
              blk[2 * arow<HBS>(2 * h + 1) * kRowW] = static_cast<uint16_t>(__float_as_uint(r) >> 16);
            }
          }
        }
      }
    }
    wave_sync();
  }
  for (int rt = r_first; rt < NTr; rt += NWT) {
    const int t0 = rt * kTile;
    const bool has_new = rt == r_new_tile;
    const bool pre = early && rt == r_first;  // loaded at setup
    const int tl = t0 + 8 * lq;               // first token of this lane's 8 value slots
    // value rows of this lane (8 tokens of NO channels), requested first
    u32x4 vraw[NO];
    if (pre) {
#pragma unroll
      for (int i = 0; i < NO; ++i) vraw[i] = rres.v[i];
    } else {
      const int tlc = rrow(min(tl, (a.r_total - 1) & ~7));  // an in-range chunk for loading (ring row)
#pragma unroll
      for (int i = 0; i < NO; ++i)
        vraw[i] = *reinterpret_cast<const u32x4*>(vr + static_cast<size_t>(out_chan<GS>(i, ln)) * a.r_cap + tlc);
    }
    f32x4 accS[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int t = t0 + col_token<GS>(ct, ln);
      const int tc = rrow(min(t, a.r_total - 1));
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        u32x4 bf = pre ? rres.k[ct][s] : *reinterpret_cast<const u32x4*>(kr + static_cast<size_t>(tc) * D + 32 * s + 8 * lq);
        if (t >= a.r_total) bf = u32x4{0u, 0u, 0u, 0u};
        if (has_new && t == a.r_new) bf = pre ? rnew.kn[s] : load_bf16x8(knp, 32 * s + 8 * lq);
        const u32x4 af = *reinterpret_cast<const u32x4*>(AK + 2 * (s * BLK + rk * kRowW + 4 * lq));
        accS[ct] = mfma(af, bf, accS[ct]);
      }
    }
    float x[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bool okh = 2 * lq + hh < Gb;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const bool ok = okh && t0 + col_token<GS>(ct, ln) < a.r_total;
        x[hh][ct] = ok ? accS[ct][2 * hh] + accS[ct][2 * hh + 1] : -INFINITY;
      }
    }
    softmax_update(x);
    wave_sync();
    // values: A = p in natural token order (rows of group area 0), B = values as
    // stored (channel-major)
    for (int i = lane; i < Gb * 16; i += 64) {
      const int h = i % Gb, pr = i / Gb;
      const Pair pa = split_pair(pbuf[h * 32 + 2 * pr], pbuf[h * 32 + 2 * pr + 1]);
      uint32_t* dst = reinterpret_cast<uint32_t*>(AV) + pr;
      dst[arow<HBS>(2 * h) * kRowW] = pa.hi;
      dst[arow<HBS>(2 * h + 1) * kRowW] = pa.lo;
    }
    wave_sync();
    const u32x4 af = *reinterpret_cast<const u32x4*>(AV + 2 * (rk * kRowW + 4 * lq));
    const bool clean = tl + 8 <= a.r_total && !(a.r_new >= tl && a.r_new < tl + 8);
    // for the lane's 8 value slots (2 per 32-bit word): keep[w] selects the ring
    // values kept, put[w] the appended token's slot; slots past the residual are 0
    uint32_t keep[4], put[4];
    const int enew = (a.r_new >= tl && a.r_new < tl + 8) ? a.r_new - tl : -1;  // slot of the appended token
    {
      const int nvld = min(max(a.r_total - tl, 0), 8);  // slots inside the residual
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        keep[w] = ((2 * w < nvld && 2 * w != enew) ? 0x0000FFFFu : 0u) |
                  ((2 * w + 1 < nvld && 2 * w + 1 != enew) ? 0xFFFF0000u : 0u);
        put[w] = (2 * w == enew ? 0x0000FFFFu : 0u) | (2 * w + 1 == enew ? 0xFFFF0000u : 0u);
      }
    }
#pragma unroll
    for (int i = 0; i < NO; ++i) {
      u32x4 bf = vraw[i];
      if (!clean) {
        uint32_t hv = 0u;  // the appended token's value of channel out_chan(i, ln)
        if (enew >= 0) hv = pre ? rnew.vn[i] : f32_to_bf16(load_f32(vnp, out_chan<GS>(i, ln)));
        const uint32_t h2 = hv | (hv << 16);
#pragma unroll
        for (int w = 0; w < 4; ++w) bf[w] = (bf[w] & keep[w]) | (h2 & put[w]);
      }
      oacc[i] = mfma(af, bf, oacc[i]);
    }
    wave_sync();
  }

  // the wave that owns the appended token's tile stores it (the first head block's)
  if (new_here && hb == 0) {
    uint16_t* kw = a.k_res + (static_cast<size_t>(bj) * a.r_cap + rrow(a.r_new)) * D;
    uint16_t* vw = a.v_res + static_cast<size_t>(bj) * D * a.r_cap + rrow(a.r_new);
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int c = lane + 64 * i;
      if (c < D) {
        kw[c] = f32_to_bf16(early ? as_f32(rnew.st_k[i]) : load_f32(knp, c));
        vw[static_cast<size_t>(c) * a.r_cap] = f32_to_bf16(early ? as_f32(rnew.st_v[i]) : load_f32(vnp, c));
      }
    }
  }

  // ---- value corrections: sum the lanes of each channel group (one DPP row)
#pragma unroll
  for (int u = 0; u < NPV; ++u) {
    const int g = (lane + 64 * u) >> 4;
#pragma unroll
    for (int h = 0; h < HBS; ++h) {
      const float s = sum16(vcorr[u][h]);
      if (ln == 0 && g < NGV) vcs[h * VCS + g] = s;
    }
  }
  wave_sync();

  // ---------------------------------------------------------------- merge the block's waves
  // Each wave leaves (o[Gb][D], m[Gb], l[Gb]) in its own LDS region (its operand
  // area is no longer needed); after one barrier the block combines them.
  float corr_g[2][NGV];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int g = 0; g < NGV; ++g) corr_g[hh][g] = vcs[min(2 * lq + hh, HBS - 1) * VCS + g];
  wave_sync();
  float* wst = reinterpret_cast<float*>(wbase);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int head = 2 * lq + hh;
    const float l = sum16(l_part[hh]);
    if (head < Gb) {
      if (ln == 0) {
        wst[HBS * D + head] = m_run[hh];
        wst[HBS * D + HBS + head] = l;
      }
      if constexpr (GS == 32) {
#pragma unroll
        for (int g = 0; g < KS; ++g) {
          float2 v;
          v.x = oacc[2 * g][2 * hh] + oacc[2 * g][2 * hh + 1] + corr_g[hh][g];
          v.y = oacc[2 * g + 1][2 * hh] + oacc[2 * g + 1][2 * hh + 1] + corr_g[hh][g];
          *reinterpret_cast<float2*>(wst + head * D + 32 * g + 2 * ln) = v;
        }
      } else {
#pragma unroll
        for (int i = 0; i < NO; ++i)
          wst[head * D + out_chan<GS>(i, ln)] = oacc[i][2 * hh] + oacc[i][2 * hh + 1] + corr_g[hh][i];
      }
    }
  }
  __syncthreads();
  const bool final_out = gridDim.x == 1;
  const size_t pb = (static_cast<size_t>(bjh) * gridDim.x + blockIdx.x) * kHB;
  for (int e = tid; e < Gb * D; e += NTHR) {
    const int h = e / D, c = e % D;
    float mw[NWV], lw[NWV], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float* ws_w = reinterpret_cast<const float*>(smem + L.wave0 + w * L.wave_bytes);
      mw[w] = ws_w[HBS * D + h];
      lw[w] = ws_w[HBS * D + HBS + h];
      M = fmaxf(M, mw[w]);
    }
    float Lsum = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      if (lw[w] > 0.0f) {
        const float f = __builtin_amdgcn_exp2f(mw[w] - M);
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

// The kernel instantiations of one group size: 8-wave workgroups (short runs)
// with one head; 4-wave workgroups with one head or kHB heads.
template <typename T, int BITS, int KS, int NWV, int HBS, int GS> const void* kernel_ptr() {
  return reinterpret_cast<const void*>(&decode_kernel<T, BITS, KS, NWV, HBS, GS>);
}
template <int GS> const void* kernel_for_gs(int dt, int bits, int KS, int nwv, int hbs) {
#define KVC_PTRS(k)                                                                                    \
  case k:                                                                                              \
    if (dt == KVC_F32)                                                                                 \
      return bits == 2 ? kernel_ptr<float, 2, k, NWV, HBS, GS>() : kernel_ptr<float, 4, k, NWV, HBS, GS>(); \
    return bits == 2 ? kernel_ptr<uint16_t, 2, k, NWV, HBS, GS>() : kernel_ptr<uint16_t, 4, k, NWV, HBS, GS>();
  if (nwv == 8) {
    if (hbs != 1) return nullptr;
    constexpr int NWV = 8, HBS = 1;
    switch (KS) { KVC_PTRS(1) KVC_PTRS(2) KVC_PTRS(3) KVC_PTRS(4) KVC_PTRS(5) KVC_PTRS(6) default: return nullptr; }
  }
  if (hbs == 1) {
    constexpr int NWV = 4, HBS = 1;
    switch (KS) {
      KVC_PTRS(1) KVC_PTRS(2) KVC_PTRS(3) KVC_PTRS(4) KVC_PTRS(5) KVC_PTRS(6) KVC_PTRS(7) KVC_PTRS(8)
      default: return nullptr;
    }
  }
  constexpr int NWV = 4, HBS = kHB;
  switch (KS) {
    KVC_PTRS(1) KVC_PTRS(2) KVC_PTRS(3) KVC_PTRS(4) KVC_PTRS(5) KVC_PTRS(6) KVC_PTRS(7) KVC_PTRS(8)
    default: return nullptr;
  }
#undef KVC_PTRS
}

}  // namespace
}  // namespace kvc
