// Decode attention over the compressed cache: planning, launches and the C
// entry points (the kernel itself is in decode_kernel.h).
#include <algorithm>
#include <mutex>

#include "decode_kernel.h"

namespace kvc {

kvc_status launch_flush(const kvc_cache* c, int ngroups, const void* k_new, const void* v_new, kvc_dtype dt,
                        hipStream_t st);
bool cache_ok(const kvc_cache* c);
kvc_status cache_shape_status(const kvc_cache* c);
const void* kernel_for_g16(int dt, int bits, int KS, int nwv, int hbs);

namespace {

// Combine the per-block partials of each (batch, KV head, head block).  Every
// output element's thread reads the (m, l) of all splits of its head and its o
// values, all requested before any is used (one memory round trip), and forms
// M = max m_s, out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s in split
// order.  Splits with l = 0 (no tokens) have weight 0.
constexpr int kMaxNb = 64;
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 8;  // splits whose loads are in flight together
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float* part_o, const float2* part_ml, float* out,
                                                              int Hq, int Hkv, int G, int HB, int hbs, int D, int nb) {
  const int jh = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int j = jh / HB, hb = jh % HB, h0 = hb * hbs;
  const int Gb = min(hbs, G - h0);
  const size_t base = ((static_cast<size_t>(b) * Hkv + j) * HB + hb) * nb;
  for (int e = tid; e < Gb * D; e += kMergeThreads) {
    const int h = e / D, c = e % D;
    const float2* ml = part_ml + base * kHB + h;
    const float* po = part_o + (base * kHB + h) * D + c;
    float M = -INFINITY, Lsum = 0.0f, acc = 0.0f;
    for (int s0 = 0; s0 < nb; s0 += kMergeBatch) {
      const int cnt = min(kMergeBatch, nb - s0);
      float2 m[kMergeBatch];
      float o[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        if (u < cnt) {
          m[u] = ml[static_cast<size_t>(s0 + u) * kHB];
          o[u] = po[static_cast<size_t>(s0 + u) * kHB * D];
        }
      }
      float Mb = M;
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u)
        if (u < cnt && m[u].y > 0.0f) Mb = fmaxf(Mb, m[u].x);
      const float r = Mb == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(M - Mb);  // rescale the running sums
      Lsum *= r;
      acc *= r;
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        if (u < cnt && m[u].y > 0.0f) {
          const float f = __builtin_amdgcn_exp2f(m[u].x - Mb);
          Lsum += f * m[u].y;
          acc += f * o[u];
        }
      }
      M = Mb;
    }
    out[(static_cast<size_t>(b) * Hq + j * G + h0 + h) * D + c] = acc / Lsum;
  }
}

// ---------------------------------------------------------------- planning
// Short runs: one workgroup per (batch, KV head, head block) -- eight waves when
// registers allow -- so no merge pass is needed.  Long runs: one round of the
// 4-wave workgroups the chip holds at once (the occupancy query below), spread
// over the units, each unit's tiles evenly over its waves, then merge_kernel.
constexpr int kShortTilesPerWave = 6;
constexpr int kMinTilesPerWave = 3;  // split runs

struct Plan {
  int nb, nwv, hbs;  // workgroups per unit, waves per workgroup, query heads per workgroup
};

// The kernel of a group size (the group-16 instantiations are compiled in their
// own translation unit).
const void* kernel_for(int gs, int dt, int bits, int KS, int nwv, int hbs) {
  return gs == 16 ? kernel_for_g16(dt, bits, KS, nwv, hbs) : kernel_for_gs<32>(dt, bits, KS, nwv, hbs);
}
// Compile-time head count of the kernel that runs hbs heads per workgroup.
int hbs_kernel(int hbs) { return hbs == 1 ? 1 : kHB; }
// Heads per workgroup of a long run: all kHB heads of a group (the packed cache
// is read once per kHB heads), unless that kernel's LDS would not fit a CU (the
// group-16 layout at D = 256: two key and eight more value operands per tile).
int long_hbs(int gs, int bits, int KS, int G) {
  const int h = std::min(kHB, G);
  return h > 1 && kernel_lds(bits, KS, 4, kHB, gs).total > kLdsBytesPerCu ? 1 : h;
}

// Workgroups of the 4-wave long-run kernel resident per CU, and the CU count of
// the current device, queried on every call that plans a long run (no state is
// kept between calls).  Long runs put long_hbs heads in a workgroup.
struct Occupancy {
  int per_cu, cus;
};
// Allows a kernel's dynamic LDS above the 64 KB default (idempotent).
kvc_status allow_lds(const void* k, int bytes) {
  if (!k || bytes <= 65536) return KVC_OK;
  const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) {
    set_last_hip_error(e);
    return KVC_ERR_HIP;
  }
  return KVC_OK;
}
kvc_status occupancy(int gs, int dt, int bits, int KS, int G, Occupancy* oc) {
  int dev = 0, per_cu = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_last_hip_error(e);
    return KVC_ERR_HIP;
  }
  const int hk = hbs_kernel(long_hbs(gs, bits, KS, G));
  const void* k = kernel_for(gs, dt, bits, KS, 4, hk);
  const int bytes = kernel_lds(bits, KS, 4, hk, gs).total;
  const kvc_status s = allow_lds(k, bytes);
  if (s != KVC_OK) return s;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 256, bytes) != hipSuccess || per_cu < 1) per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  oc->per_cu = per_cu;
  oc->cus = cus;
  return KVC_OK;
}

// Heads per workgroup: long runs take long_hbs (lh) heads; short, latency-bound
// runs split the heads so that each wave's per-tile operand work shrinks (the
// extra reads of a short history hit the caches; measured 7% faster per call at
// the 8B shape).
int heads_per_block(int lh, bool short_run) { return short_run ? 1 : lh; }
bool is_short(int NT, int KS) {
  const int nwv_short = KS <= 6 ? 8 : 4;
  return (NT + nwv_short - 1) / nwv_short <= kShortTilesPerWave;
}
// oc is read for long runs only; lh = long_hbs
Plan plan(int NT, int BH, int G, int KS, int lh, const Occupancy& oc) {
  Plan p;
  const bool sh = is_short(NT, KS);
  p.hbs = heads_per_block(lh, sh);
  const int units = BH * ((G + p.hbs - 1) / p.hbs);
  if (sh) {
    p.nwv = KS <= 6 ? 8 : 4;
    p.nb = 1;
    return p;
  }
  p.nwv = 4;
  int nb = std::max(1, oc.cus * oc.per_cu / units);
  // at least kMinTilesPerWave tiles per wave: fewer, fuller splits cost less to
  // merge (measured 5% faster per call at the 128k shape than one tile per wave)
  nb = std::min(nb, (NT + 4 * kMinTilesPerWave - 1) / (4 * kMinTilesPerWave));
  nb = std::min(nb, kMaxNb);
  p.nb = nb;
  return p;
}

// Workspace of the split runs: (m, l) and o[D] for kHB heads per workgroup
// slot.  Sized without the device: the splits of a long run are at most
// min(kMaxNb, ceil(NT / (4 * kMinTilesPerWave))) whatever the occupancy, and that
// bound grows with NT, so the capacity's tile count gives the largest run.
struct WsLayout {
  size_t part_ml, part_o, total;
};
WsLayout ws_layout_for(size_t slots, int D) {
  WsLayout w;
  w.part_ml = 0;
  w.part_o = align_up(slots * kHB * sizeof(float2), 256);
  w.total = w.part_o + slots * kHB * D * sizeof(float);
  return w;
}
size_t max_slots(const kvc_cache* c, int G) {
  const int KS = c->head_dim / 32;
  const int NTmax = c->q_cap / kTile + (c->r_cap + kTile - 1) / kTile;
  if (is_short(NTmax, KS)) return 0;  // every run fits one workgroup per unit
  const int lh = long_hbs(cache_group(c), c->bits, KS, G);
  const size_t units = static_cast<size_t>(c->batch) * c->kv_heads * ((G + lh - 1) / lh);
  const int nb = std::min(kMaxNb, (NTmax + 4 * kMinTilesPerWave - 1) / (4 * kMinTilesPerWave));
  return units * static_cast<size_t>(nb);
}

kvc_status launch_decode(const DecArgs& a, int gs, int dt, int bits, int KS, int nwv, int B, hipStream_t st) {
  const int hk = hbs_kernel(a.hbs);
  const void* k = kernel_for(gs, dt, bits, KS, nwv, hk);
  if (!k) return KVC_ERR_SHAPE;
  const int bytes = kernel_lds(bits, KS, nwv, hk, gs).total;
  kvc_status s = allow_lds(k, bytes);
  if (s != KVC_OK) return s;
  dim3 grid(a.nb, a.Hkv * a.HB, B);
  void* args[] = {const_cast<DecArgs*>(&a)};
  hipError_t e = hipLaunchKernel(k, grid, dim3(64 * nwv), args, bytes, st);
  if (e != hipSuccess) {
    set_last_hip_error(e);
    return KVC_ERR_HIP;
  }
  s = check_launch();
  if (s != KVC_OK || a.nb == 1) return s;
  hipLaunchKernelGGL(merge_kernel, dim3(a.Hkv * a.HB, B), dim3(kMergeThreads), 0, st, a.part_o, a.part_ml, a.out,
                     a.Hq, a.Hkv, a.G, a.HB, a.hbs, 32 * KS, a.nb);
  return check_launch();
}

// Workspace bytes of a decode call on this cache with G query heads per KV
// head (the split partials); never zero, so that a caller's buffer pointer is
// never NULL.
size_t decode_ws_need(const kvc_cache* c, int G) {
  return std::max<size_t>(ws_layout_for(max_slots(c, G), c->head_dim).total, 256);
}

// One decode step, planned before anything is launched: the cache state after
// the step (append, flush), the attention launch shape and the workspace bytes
// this call uses.
struct Step {
  kvc_cache nc;        // state after the step
  bool flush;
  int ngroups;         // flushed groups (1, or R/g for the whole-residual policy)
  int r_total, r_new;  // residual tokens attended; the appended token's index (-1: flushed)
  Plan plan;           // launch shape
  size_t used;         // workspace bytes this call uses
};
kvc_status plan_step(const kvc_cache* cache, int dtype, int Hq, Step* sp) {
  const int R = cache->residual, g = cache_group(cache);
  const int G = Hq / cache->kv_heads, KS = cache->head_dim / 32;
  if (cache->r_len + 1 > cache->r_cap) return KVC_ERR_CAPACITY;
  // tokens a flush moves into the packed history: one group, or with flush_all
  // the whole residual of R tokens (R/g groups, the appended token last)
  const int moved = cache->flush_all ? R : g;
  sp->flush = (cache->r_len + 1 == R + (cache->flush_all ? 0 : g));
  if (sp->flush && cache->q_len + moved > cache->q_cap) return KVC_ERR_CAPACITY;
  sp->nc = *cache;
  sp->ngroups = moved / g;
  if (sp->flush) {
    sp->nc.q_len += moved;
    sp->nc.r_len = cache->r_len + 1 - moved;
    sp->nc.r_start = (cache->r_start + moved) % cache->r_cap;
    sp->r_total = sp->nc.r_len;
    sp->r_new = -1;
  } else {
    sp->r_new = cache->r_len;
    sp->r_total = cache->r_len + 1;
    sp->nc.r_len += 1;
  }
  // tiles: the history's (the last one half full after an odd number of
  // 16-token groups) and the residual's
  const int NT = (sp->nc.q_len + kTile - 1) / kTile + (sp->r_total + kTile - 1) / kTile;
  Occupancy oc{1, 256};
  if (!is_short(NT, KS)) {
    const kvc_status s = occupancy(g, dtype, cache->bits, KS, G, &oc);
    if (s != KVC_OK) return s;
  }
  sp->plan = plan(NT, cache->batch * cache->kv_heads, G, KS, long_hbs(g, cache->bits, KS, G), oc);
  const size_t units = static_cast<size_t>(cache->batch) * cache->kv_heads * ((G + sp->plan.hbs - 1) / sp->plan.hbs);
  sp->used = sp->plan.nb > 1 ? ws_layout_for(units * sp->plan.nb, cache->head_dim).total : 0;
  return KVC_OK;
}

// The attention launch of a planned step (split partials laid out in ws for
// this call's slots).
kvc_status decode_step(const Step& sp, const void* q, const void* k_new, const void* v_new, kvc_dtype dtype, int Hq,
                      float* out, void* ws, hipStream_t st) {
  const kvc_cache& c = sp.nc;
  const Plan& p = sp.plan;
  const int Hkv = c.kv_heads, G = Hq / Hkv, KS = c.head_dim / 32;
  DecArgs a;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.r_total = sp.r_total;
  a.r_new = sp.r_new;
  a.k_codes = c.k_codes;
  a.k_meta = c.k_meta;
  a.v_codes = c.v_codes;
  a.v_meta = c.v_meta;
  a.k_res = c.k_res;
  a.v_res = c.v_res;
  a.B = c.batch;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.q_cap = c.q_cap;
  a.r_cap = c.r_cap;
  a.r_start = c.r_start;
  a.q_len = c.q_len;
  a.hbs = p.hbs;
  a.HB = (G + p.hbs - 1) / p.hbs;
  a.nb = p.nb;
  const size_t slots = static_cast<size_t>(c.batch) * Hkv * a.HB * p.nb;
  const WsLayout W = ws_layout_for(slots, c.head_dim);
  char* w = static_cast<char*>(ws);
  a.part_ml = reinterpret_cast<float2*>(w + W.part_ml);
  a.part_o = reinterpret_cast<float*>(w + W.part_o);
  a.out = out;
  a.scale2 = 1.4426950408889634f / sqrtf(static_cast<float>(c.head_dim));
  a.rcp_hkv = 1.0f / static_cast<float>(Hkv);
  a.rcp_hb = 1.0f / static_cast<float>(a.HB);
  a.rcp_xhb = 1.0f / static_cast<float>(kXcds * a.HB);
  const int NWT = p.nb * p.nwv;
  const SplitParams spl = split_params(NWT, (a.q_len + kTile - 1) / kTile, (a.r_total + kTile - 1) / kTile);
  a.split_nA = spl.nA;
  a.split_hA = spl.hA;
  a.split_hB = spl.hB;
  a.sp_new = a.r_new >= 0 ? NWT - 1 - (a.r_new / kTile) % NWT : -1;
  return launch_decode(a, cache_group(&c), dtype, c.bits, KS, p.nwv, c.batch, st);
}

// Validation shared by both decode entry points (before anything else).
kvc_status decode_args_status(const kvc_cache* cache, kvc_dtype dtype, int Hq) {
  if (!dtype_ok(dtype)) return KVC_ERR_DTYPE;
  const kvc_status s = cache_shape_status(cache);
  if (s != KVC_OK) return s;
  const int Hkv = cache->kv_heads;
  if (Hq < 1 || Hq % Hkv != 0 || Hq / Hkv > 16) return KVC_ERR_SHAPE;
  return KVC_OK;
}

// Enqueue a planned step (flush, then attention) and commit the host state.
// The state goes to *cache only once every launch has been enqueued: the flush
// and the attention kernel write past the current lengths only (codes at
// q_len.., the appended token's ring row), so a failed call leaves the cache as
// it was.
kvc_status run_step(kvc_cache* cache, const Step& sp, const void* q, const void* k_new, const void* v_new,
                    kvc_dtype dtype, int Hq, float* out, void* ws, hipStream_t st) {
  kvc_status s = KVC_OK;
  if (sp.flush) {
    s = launch_flush(cache, sp.ngroups, k_new, v_new, dtype, st);
    if (s != KVC_OK) return s;
  }
  s = decode_step(sp, q, k_new, v_new, dtype, Hq, out, ws, st);
  if (s == KVC_OK) *cache = sp.nc;
  return s;
}

}  // namespace
}  // namespace kvc

extern "C" kvc_status kvc_decode_attn(kvc_cache* cache, const void* q, const void* k_new,
                                      const void* v_new, kvc_dtype dtype, int32_t Hq, float* out,
                                      void* ws, size_t* ws_bytes, void* stream) {
  using namespace kvc;
  if (!cache_ok(cache) || !ws_bytes) return KVC_ERR_NULL;
  kvc_status s = decode_args_status(cache, dtype, Hq);
  if (s != KVC_OK) return s;
  const size_t need = decode_ws_need(cache, Hq / cache->kv_heads);
  if (!ws) {
    *ws_bytes = need;
    return KVC_OK;
  }
  if (!q || !k_new || !v_new || !out) return KVC_ERR_NULL;
  if (*ws_bytes < need) return KVC_ERR_WORKSPACE;
  Step sp;
  s = plan_step(cache, dtype, Hq, &sp);
  if (s != KVC_OK) return s;
  return run_step(cache, sp, q, k_new, v_new, dtype, Hq, out, ws, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- no-allocation variant
// kvc_decode_attn_noalloc takes its scratch (the split partials) from this
// file-scope device array instead of a caller workspace.  Each device holds its
// own copy for the life of the process; host code reaches it only through the
// address hipGetSymbolAddress returns for that device (the symbol's name is a
// host-side stand-in, not a device address).  No kernel needs it cleared: every
// slot a merge reads was written by the same call.  Calls that overlap on one
// device share it and race.
namespace {
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kScratchDevices = 64;
}  // namespace
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
// The device address of `scratch` on the current device, looked up once per
// device (std::call_once) -- the library's only process-wide state besides the
// thread-local error code.
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kScratchDevices];

kvc_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    kvc::set_last_hip_error(e);
    return KVC_ERR_HIP;
  }
  if (dev < 0 || dev >= kScratchDevices) return KVC_ERR_SHAPE;
  ScratchSlot& sl = g_scratch[dev];
  std::call_once(sl.once, [&sl] { sl.err = hipGetSymbolAddress(&sl.ptr, HIP_SYMBOL(scratch)); });
  if (sl.err != hipSuccess || !sl.ptr) {
    kvc::set_last_hip_error(sl.err != hipSuccess ? sl.err : hipErrorInvalidSymbol);
    return KVC_ERR_HIP;
  }
  *out = sl.ptr;
  return KVC_OK;
}
}  // namespace

extern "C" kvc_status kvc_decode_attn_noalloc(kvc_cache* cache, const void* q, const void* k_new,
                                              const void* v_new, kvc_dtype dtype, int32_t Hq, float* out,
                                              void* stream) {
  using namespace kvc;
  if (!cache_ok(cache)) return KVC_ERR_NULL;
  kvc_status s = decode_args_status(cache, dtype, Hq);
  if (s != KVC_OK) return s;
  if (!q || !k_new || !v_new || !out) return KVC_ERR_NULL;
  Step sp;
  s = plan_step(cache, dtype, Hq, &sp);
  if (s != KVC_OK) return s;
  if (sp.used > kScratchBytes) return KVC_ERR_WORKSPACE;
  void* ws = nullptr;
  s = scratch_ptr(&ws);
  if (s != KVC_OK) return s;
  return run_step(cache, sp, q, k_new, v_new, dtype, Hq, out, ws, static_cast<hipStream_t>(stream));
}
