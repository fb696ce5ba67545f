// Host-only parts of the C ABI: per-layer budgets, footprint, cache sizing,
// status strings and the thread-local last-HIP-error code.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "kvc_internal.h"

namespace kvc {
static thread_local int g_last_hip_error = 0;
void set_last_hip_error(hipError_t e) { g_last_hip_error = static_cast<int>(e); }
kvc_status check_launch() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_last_hip_error(e);
    return KVC_ERR_HIP;
  }
  return KVC_OK;
}
}  // namespace kvc

extern "C" int kvc_last_hip_error(void) { return kvc::g_last_hip_error; }

extern "C" const char* kvc_status_string(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_ERR_NULL: return "null pointer";
    case KVC_ERR_SHAPE: return "invalid shape";
    case KVC_ERR_DTYPE: return "invalid dtype";
    case KVC_ERR_BITS: return "invalid bit width";
    case KVC_ERR_CAPACITY: return "cache capacity exceeded or cache not empty";
    case KVC_ERR_WORKSPACE: return "workspace too small";
    case KVC_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

extern "C" kvc_status kvc_cache_sizes(int32_t batch, int32_t kv_heads, int32_t head_dim, int32_t bits,
                                      int32_t group, int32_t q_cap, int32_t r_cap, size_t out[6]) {
  if (!out) return KVC_ERR_NULL;
  if ((bits != 2 && bits != 4) || !kvc::group_ok(group)) return KVC_ERR_BITS;
  const size_t g = group == 0 ? kvc::kGroup : group;
  if (batch < 1 || kv_heads < 1 || !kvc::head_dim_ok(head_dim) || q_cap < 0 || r_cap < 0 ||
      q_cap % kvc::kGroup != 0)
    return KVC_ERR_SHAPE;
  const size_t bh = static_cast<size_t>(batch) * kv_heads;
  const size_t D = head_dim, qc = q_cap, rc = r_cap;
  out[0] = bh * qc * (D * bits / 32) * 4;  // k_codes
  out[1] = bh * (qc / g) * D * 4;          // k_meta
  out[2] = bh * (qc * bits / 32) * D * 4;  // v_codes
  out[3] = bh * qc * (D / g) * 4;          // v_meta
  out[4] = bh * rc * D * 2;                // k_res
  out[5] = bh * rc * D * 2;                // v_res
  return KVC_OK;
}

namespace {

typedef __int128 i128;

// Exact rational value of a binary double >= 1: beta = P / Qd.
void beta_ratio(double beta, i128* P, i128* Qd) {
  int e = 0;
  const double m = frexp(beta, &e);  // beta = m * 2^e, 0.5 <= m < 1
  const int64_t M = static_cast<int64_t>(ldexp(m, 53));
  const int sh = e - 53;
  if (sh >= 0) {
    *P = static_cast<i128>(M) << sh;
    *Qd = 1;
  } else {
    *P = M;
    *Qd = static_cast<i128>(1) << (-sh);
  }
  while (*Qd > 1 && (*P % 2) == 0 && (*Qd % 2) == 0) {
    *P /= 2;
    *Qd /= 2;
  }
}

// Pyramid: x_l = bottom - (bottom - top) * l / (L-1) with top = avg/beta and
// bottom = 2*avg - top, i.e. x_l = [2 avg P (L-1-l) - avg Qd (L-1-2l)] / (P (L-1)).
// Floor, then +1 to the layers with the largest remainders (ties: lower layer).
void pyramid(int L, int64_t avg, double beta, int32_t* out) {
  if (L == 1) {
    out[0] = static_cast<int32_t>(avg);
    return;
  }
  i128 P, Qd;
  beta_ratio(beta, &P, &Qd);
  const i128 den = P * (L - 1);
  std::vector<i128> rem(L);
  int64_t sum = 0;
  for (int l = 0; l < L; ++l) {
    const i128 num = 2 * static_cast<i128>(avg) * P * (L - 1 - l) -
                     static_cast<i128>(avg) * Qd * (L - 1 - 2 * l);
    const i128 fl = num / den;  // num >= 0 for beta >= 1
    rem[l] = num - fl * den;
    out[l] = static_cast<int32_t>(fl);
    sum += static_cast<int64_t>(fl);
  }
  int64_t extra = static_cast<int64_t>(L) * avg - sum;
  std::vector<int> order(L);
  for (int l = 0; l < L; ++l) order[l] = l;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return rem[a] > rem[b]; });
  for (int i = 0; i < extra && i < L; ++i) out[order[i]] += 1;
}


// Weighted: x_l = (L*avg * w_l) / S with S = w_0 + w_1 + ... in order, in IEEE
// double; floor, then +1 to the largest fractional parts (ties: lower layer).
void weighted(int L, int64_t avg, const double* w, int32_t* out) {
  double S = 0.0;
  for (int l = 0; l < L; ++l) S = S + w[l];
  const double tot = static_cast<double>(static_cast<int64_t>(L) * avg);
  std::vector<double> rem(L);
  int64_t sum = 0;
  for (int l = 0; l < L; ++l) {
    const double t = tot * w[l];
    const double x = t / S;
    const double fl = floor(x);
    rem[l] = x - fl;
    out[l] = static_cast<int32_t>(fl);
    sum += static_cast<int64_t>(fl);
  }
  int64_t extra = static_cast<int64_t>(L) * avg - sum;
  extra = std::min<int64_t>(std::max<int64_t>(extra, 0), L);
  std::vector<int> order(L);
  for (int l = 0; l < L; ++l) order[l] = l;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return rem[a] > rem[b]; });
  for (int i = 0; i < extra; ++i) out[order[i]] += 1;
}

kvc_status check_args(const kvc_budget_args* a) {
  const int L = a->layers;
  if (L < 1 || L > 65536 || a->kv_heads < 1 || a->head_dim < 1 || a->prompt_len < 1 ||
      a->window < 0 || a->window > a->prompt_len || a->gen_len < 0 || a->residual < 0)
    return KVC_ERR_SHAPE;
  if (a->bits != 2 && a->bits != 4 && a->bits != 8 && a->bits != 16) return KVC_ERR_BITS;
  if (a->group != 16 && a->group != 32) return KVC_ERR_BITS;
  if (a->meta_bits != 8 && a->meta_bits != 16 && a->meta_bits != 32) return KVC_ERR_BITS;
  return KVC_OK;
}

// Footprint of the applied budgets (see kvc_budget in kvc.h).
void footprint(const kvc_budget_args* a, const int32_t* layer_budget, kvc_footprint* fp) {
  const int L = a->layers;
  const double bpe = a->bits == 16 ? 16.0 : a->bits + 2.0 * a->meta_bits / a->group;
  int64_t kept_sum = 0;
  double total_tokens = 0.0;
  int64_t layout = 0;
  const int64_t D = a->head_dim;
  for (int l = 0; l < L; ++l) {
    const int64_t T = a->avg_budget < 0 ? a->prompt_len : layer_budget[l] + a->window;
    kept_sum += T;
    total_tokens += static_cast<double>(T + a->gen_len);
    if (a->bits == 16) {
      layout += 2 * T * D * 2;
    } else {
      const int64_t g = a->group;
      const int64_t q = g * (std::max<int64_t>(T - a->residual, 0) / g);
      const int64_t pair = 2 * a->meta_bits / 8;
      layout += 2 * q * D * a->bits / 8 + (q / g) * D * pair + q * (D / g) * pair + 2 * (T - q) * D * 2;
    }
  }
  const double frac = static_cast<double>(kept_sum) / (static_cast<double>(L) * a->prompt_len);
  const double per_tok = 2.0 * L * a->kv_heads * a->head_dim * bpe / 8.0;
  fp->bits_per_element = bpe;
  fp->bytes_per_prompt_token = per_tok * frac;
  fp->bytes_total = 2.0 * a->kv_heads * a->head_dim * bpe / 8.0 * total_tokens;
  fp->bytes_layout = static_cast<double>(layout * a->kv_heads);
}

}  // namespace

extern "C" kvc_status kvc_budget(const kvc_budget_args* a, int32_t* layer_budget, kvc_footprint* fp) {
  if (!a || !layer_budget) return KVC_ERR_NULL;
  const kvc_status s = check_args(a);
  if (s != KVC_OK) return s;
  const int L = a->layers;
  if (a->pyramid && a->avg_budget >= 0 && (!(a->beta >= 1.0) || !isfinite(a->beta) || a->beta > 1048576.0))
    return KVC_ERR_SHAPE;
  const int64_t cand = static_cast<int64_t>(a->prompt_len) - a->window;
  if (a->avg_budget < 0) {
    for (int l = 0; l < L; ++l) layer_budget[l] = static_cast<int32_t>(cand);
  } else if (a->pyramid) {
    pyramid(L, a->avg_budget, a->beta, layer_budget);
  } else {
    for (int l = 0; l < L; ++l) layer_budget[l] = a->avg_budget;
  }
  for (int l = 0; l < L; ++l)
    if (layer_budget[l] > cand) layer_budget[l] = static_cast<int32_t>(cand);
  if (fp) footprint(a, layer_budget, fp);
  return KVC_OK;
}

extern "C" kvc_status kvc_budget_weighted(const kvc_budget_args* a, const double* weights, int32_t* layer_budget,
                                          kvc_footprint* fp) {
  if (!a || !weights || !layer_budget) return KVC_ERR_NULL;
  const kvc_status s = check_args(a);
  if (s != KVC_OK) return s;
  const int L = a->layers;
  if (a->avg_budget < 0 || static_cast<int64_t>(L) * a->avg_budget > 2147483647LL) return KVC_ERR_SHAPE;
  double S = 0.0;
  for (int l = 0; l < L; ++l) {
    if (!(weights[l] > 0.0) || !isfinite(weights[l])) return KVC_ERR_SHAPE;
    S = S + weights[l];
  }
  if (!isfinite(S)) return KVC_ERR_SHAPE;
  weighted(L, a->avg_budget, weights, layer_budget);
  const int64_t cand = static_cast<int64_t>(a->prompt_len) - a->window;
  for (int l = 0; l < L; ++l)
    if (layer_budget[l] > cand) layer_budget[l] = static_cast<int32_t>(cand);
  if (fp) footprint(a, layer_budget, fp);
  return KVC_OK;
}
