// C ABI of liblcx (declared in include/lcx.h): argument checks, the fp64
// RoPE scheme arithmetic of step a1, and the launches of steps a2-a10.
// Every check runs before anything is enqueued; nothing here allocates device
// memory or synchronises.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "lcx.h"
#include "lcx_internal.h"

namespace {

thread_local char g_err[512] = "";

lcx_status fail(lcx_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

lcx_status ok() {
  g_err[0] = '\0';
  return LCX_OK;
}

lcx_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(LCX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_scaling(int32_t scheme) {
  return scheme == LCX_ROPE_PI || scheme == LCX_ROPE_NTK || scheme == LCX_ROPE_NTK_PARTS ||
         scheme == LCX_ROPE_YARN || scheme == LCX_ROPE_DYNAMIC_NTK;
}

lcx_status check_cfg(const lcx_rope_cfg* c) {
  if (!c) return fail(LCX_ERR_INVALID_ARG, "rope cfg is NULL");
  if (c->scheme < LCX_ROPE_PLAIN || c->scheme > LCX_ROPE_PAIR_FACTORS)
    return fail(LCX_ERR_INVALID_ARG, "rope scheme %d is not a scheme with frequencies", c->scheme);
  if (c->head_dim < 2 || (c->head_dim & 1))
    return fail(LCX_ERR_INVALID_ARG, "head_dim %d must be even and >= 2", c->head_dim);
  if (!(c->base > 1.0) || !std::isfinite(c->base))
    return fail(LCX_ERR_INVALID_ARG, "base %g must be a finite number > 1", c->base);
  if (is_scaling(c->scheme)) {
    if (c->L_train <= 0) return fail(LCX_ERR_INVALID_ARG, "L_train %lld must be > 0", (long long)c->L_train);
    if (c->L_target < c->L_train)
      return fail(LCX_ERR_INVALID_ARG, "L_target %lld < L_train %lld (s < 1)", (long long)c->L_target,
                  (long long)c->L_train);
  }
  if (c->scheme == LCX_ROPE_DYNAMIC_NTK && c->cur_len < 0)
    return fail(LCX_ERR_INVALID_ARG, "cur_len %lld must be >= 0", (long long)c->cur_len);
  if ((c->scheme == LCX_ROPE_NTK_PARTS || c->scheme == LCX_ROPE_YARN) &&
      !(c->alpha > 0.0 && c->alpha < c->beta && std::isfinite(c->beta)))
    return fail(LCX_ERR_INVALID_ARG, "need 0 < alpha (%g) < beta (%g)", c->alpha, c->beta);
  if (c->scheme == LCX_ROPE_PAIR_FACTORS) {
    if (!c->factors) return fail(LCX_ERR_INVALID_ARG, "PAIR_FACTORS needs factors[d/2]");
    for (int i = 0; i < c->head_dim / 2; ++i)
      if (!(c->factors[i] > 0.0) || !std::isfinite(c->factors[i]))
        return fail(LCX_ERR_INVALID_ARG, "factors[%d] = %g must be finite and > 0", i, c->factors[i]);
  }
  return LCX_OK;
}

// Step a1 (fp64).  The base of the frequency ladder theta_i = base'^(-2i/d)
// ("上下文擴充套件（Context Extension）" 技術原理) is changed by the NTK-aware
// rule base' = base·s^(d/(d-2)) ("上下文窗口扩展技术：从 4K 到 1M" §2.2) or its
// dynamic form with s = l/L_train once l exceeds L_train (§3); NTK-by-parts
// (§2.3) keeps the base and multiplies each pair by a factor chosen from its
// wavelength 2π/theta_i: 1 below L_train/beta, 1/s above L_train/alpha,
// linear in the wavelength in between (continuous at both ends); YaRN (§2.4)
// adds the logit divisor t = 0.1·ln s + 1; PI (§2.1) scales positions by
// L_train/L_target instead of touching the frequencies; per-pair factors
// (LongRoPE, §2.5: one factor per rotation plane, found by a search that is
// not part of this library) divide each pair's frequency by its factor.
void scheme_freqs(const lcx_rope_cfg& c, double* theta, double* pos_factor, double* logit_mult) {
  const int d = c.head_dim;
  const double s = is_scaling(c.scheme) ? (double)c.L_target / (double)c.L_train : 1.0;
  const double ntk_exp = (double)d / (double)(d - 2);
  double base_eff = c.base;
  if (c.scheme == LCX_ROPE_NTK) base_eff = c.base * std::pow(s, ntk_exp);
  if (c.scheme == LCX_ROPE_DYNAMIC_NTK) {
    const int64_t l = c.cur_len > 0 ? c.cur_len : c.L_target;
    if (l > c.L_train) base_eff = c.base * std::pow((double)l / (double)c.L_train, ntk_exp);
  }
  for (int i = 0; i < d / 2; ++i) theta[i] = std::pow(base_eff, -(2.0 * i) / (double)d);
  if (c.scheme == LCX_ROPE_NTK_PARTS || c.scheme == LCX_ROPE_YARN) {
    const double two_pi = 6.283185307179586476925286766559;
    const double wl_short = (double)c.L_train / c.beta;  // below: untouched
    const double wl_long = (double)c.L_train / c.alpha;  // above: fully interpolated
    for (int i = 0; i < d / 2; ++i) {
      const double wl = two_pi / theta[i];
      double f;
      if (wl < wl_short)
        f = 1.0;
      else if (wl > wl_long)
        f = 1.0 / s;
      else
        f = 1.0 - (1.0 - 1.0 / s) * ((wl - wl_short) / (wl_long - wl_short));
      theta[i] *= f;
    }
  }
  if (c.scheme == LCX_ROPE_PAIR_FACTORS)
    for (int i = 0; i < d / 2; ++i) theta[i] /= c.factors[i];
  *pos_factor = c.scheme == LCX_ROPE_PI ? (double)c.L_train / (double)c.L_target : 1.0;
  *logit_mult = c.scheme == LCX_ROPE_YARN ? 1.0 / (0.1 * std::log(s) + 1.0) : 1.0;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

bool strides_ok(const int64_t* st, int64_t mult) {
  return st && st[0] % mult == 0 && st[1] % mult == 0 && st[2] % mult == 0 && st[0] >= 0 &&
         st[1] >= 0 && st[2] >= 0;
}

bool covers(int64_t tab_pos0, int64_t tab_len, int64_t pos0, int64_t n) {
  if (n <= 0) return true;
  return pos0 >= tab_pos0 && pos0 + n <= tab_pos0 + tab_len;
}

lcx_status check_attn(const lcx_attn_args* a, bool chunked) {
  if (!a) return fail(LCX_ERR_INVALID_ARG, "args is NULL");
  if (!a->q || !a->k || !a->v || !a->o || !a->lse)
    return fail(LCX_ERR_INVALID_ARG, "q, k, v, o and lse are required");
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1)
    return fail(LCX_ERR_INVALID_ARG, "B, Hq, Hkv must be >= 1");
  if (a->Hq % a->Hkv) return fail(LCX_ERR_INVALID_ARG, "Hq %d is not a multiple of Hkv %d", a->Hq, a->Hkv);
  if (a->n_q < 0 || a->n_kv < 0) return fail(LCX_ERR_INVALID_ARG, "n_q and n_kv must be >= 0");
  if (a->d != 64 && a->d != 128) return fail(LCX_ERR_UNSUPPORTED, "head dim %d (kernels: 64, 128)", a->d);
  if (a->causal != 1) return fail(LCX_ERR_UNSUPPORTED, "only causal attention is implemented");
  if (a->window < -1) return fail(LCX_ERR_INVALID_ARG, "window %lld < -1", (long long)a->window);
  if (a->n_sink < 0) return fail(LCX_ERR_INVALID_ARG, "n_sink %d < 0", a->n_sink);
  if (a->q_dtype != LCX_BF16 && a->q_dtype != LCX_F16) return fail(LCX_ERR_INVALID_ARG, "q dtype");
  if (a->k_dtype != LCX_BF16 && a->k_dtype != LCX_F16) return fail(LCX_ERR_INVALID_ARG, "k dtype");
  if (a->rope_q && a->q_dtype != LCX_BF16) return fail(LCX_ERR_INVALID_ARG, "rope_q needs bf16 q");
  if (a->rope_k && a->k_dtype != LCX_BF16) return fail(LCX_ERR_INVALID_ARG, "rope_k needs bf16 k");
  if (a->o_dtype != LCX_BF16 && a->o_dtype != LCX_F32) return fail(LCX_ERR_INVALID_ARG, "o dtype");
  if (a->accumulate && (chunked || a->o_dtype != LCX_F32))
    return fail(LCX_ERR_INVALID_ARG, chunked ? "accumulate must be 0 for the chunked driver"
                                             : "accumulate needs an f32 o");
  if (!(a->softmax_scale >= 0.f) || !std::isfinite(a->softmax_scale))
    return fail(LCX_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0 (0: default)");
  if (a->rope_q != 0 && a->rope_q != 1) return fail(LCX_ERR_INVALID_ARG, "rope_q must be 0 or 1");
  if (a->rope_k != 0 && a->rope_k != 1) return fail(LCX_ERR_INVALID_ARG, "rope_k must be 0 or 1");
  if (a->rope) {
    lcx_status st = check_cfg(a->rope);
    if (st != LCX_OK) return st;
    if (a->rope->head_dim != a->d)
      return fail(LCX_ERR_INVALID_ARG, "rope head_dim %d differs from d %d", a->rope->head_dim, a->d);
  }
  if (a->rope_q || a->rope_k) {
    // the tables' configuration also fixes the logit multiplier (YaRN's 1/t):
    // without it the temperature would be dropped silently
    if (!a->rope) return fail(LCX_ERR_INVALID_ARG, "rope_q/rope_k need the rope configuration of the tables");
    if (!a->cos_tab || !a->sin_tab) return fail(LCX_ERR_INVALID_ARG, "RoPE tables missing");
    if (a->rope_q && !covers(a->tab_pos0, a->tab_len, a->q_pos0, a->n_q))
      return fail(LCX_ERR_INVALID_ARG, "table rows do not cover the query positions");
    if (a->rope_k && !covers(a->tab_pos0, a->tab_len, a->k_pos0, a->n_kv))
      return fail(LCX_ERR_INVALID_ARG, "table rows do not cover the key positions");
    if (!aligned16(a->cos_tab) || !aligned16(a->sin_tab))
      return fail(LCX_ERR_UNSUPPORTED, "tables must be 16-byte aligned");
  }
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(LCX_ERR_UNSUPPORTED, "q, k, v, o must be 16-byte aligned");
  if (a->v_tiled != 0 && a->v_tiled != 1) return fail(LCX_ERR_INVALID_ARG, "v_tiled must be 0 or 1");
  if (a->precise_qk != 0 && a->precise_qk != 1) return fail(LCX_ERR_INVALID_ARG, "precise_qk must be 0 or 1");
  // the high/low split is taken from the kernel's own rotation of raw k; a
  // pre-rotated k has already been rounded
  if (a->precise_qk && !a->rope_k)
    return fail(LCX_ERR_UNSUPPORTED, "precise_qk needs raw bf16 k rotated in the kernel (rope_k = 1)");
  if ((reinterpret_cast<uintptr_t>(a->sched) & 7) != 0)
    return fail(LCX_ERR_UNSUPPORTED, "sched must be 8-byte aligned");
  // tile layout: only the batch and head strides are used
  const int64_t v_st[3] = {a->v_strides[0], a->v_strides[1], a->v_tiled ? 8 : a->v_strides[2]};
  if (!strides_ok(a->q_strides, 8) || !strides_ok(a->k_strides, 8) || !strides_ok(v_st, 8))
    return fail(LCX_ERR_UNSUPPORTED, "q/k/v strides must be non-negative multiples of 8 elements");
  if (!strides_ok(a->o_strides, a->o_dtype == LCX_F32 ? 4 : 8))
    return fail(LCX_ERR_UNSUPPORTED, "o strides must keep rows 16-byte aligned");
  if (a->lse_strides[0] < 0 || a->lse_strides[1] < 0)
    return fail(LCX_ERR_INVALID_ARG, "lse strides must be >= 0");
  // the kernel addresses one KV head's keys with 32-bit buffer offsets
  const int64_t lim = (int64_t)1 << 31;
  if (a->n_kv * a->k_strides[2] * 2 >= lim || (!a->v_tiled && a->n_kv * a->v_strides[2] * 2 >= lim) ||
      (a->rope_k && a->n_kv * a->d * 2 >= lim))
    return fail(LCX_ERR_UNSUPPORTED, "one KV head spans 2 GiB or more (split the keys into chunks)");
  if (lcx::sched_grid(lcx::attn_fwd_blocks(a->d, a->B, a->Hkv, a->Hq / a->Hkv, a->n_q),
                      a->sched != nullptr) >= (int64_t)1 << 31)
    return fail(LCX_ERR_UNSUPPORTED, "problem too large for one launch");
  return LCX_OK;
}

lcx::AttnParams make_params(const lcx_attn_args* a) {
  lcx::AttnParams p{};
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint16_t*>(a->k);
  p.v = static_cast<const uint16_t*>(a->v);
  p.o = a->o;
  p.lse = a->lse;
  p.cos_tab = a->cos_tab;
  p.sin_tab = a->sin_tab;
  p.qs_b = a->q_strides[0]; p.qs_h = a->q_strides[1]; p.qs_s = a->q_strides[2];
  p.ks_b = a->k_strides[0]; p.ks_h = a->k_strides[1]; p.ks_s = a->k_strides[2];
  p.vs_b = a->v_strides[0]; p.vs_h = a->v_strides[1]; p.vs_s = a->v_strides[2];
  p.os_b = a->o_strides[0]; p.os_h = a->o_strides[1]; p.os_s = a->o_strides[2];
  p.ls_b = a->lse_strides[0]; p.ls_h = a->lse_strides[1];
  p.n_q = a->n_q; p.n_kv = a->n_kv; p.q_pos0 = a->q_pos0; p.k_pos0 = a->k_pos0;
  p.tab_pos0 = a->tab_pos0;
  p.window = a->window;
  double mult = 1.0;
  if (a->rope) {  // head_dim == d (64 or 128), checked
    double th[lcx::kMaxHalfDim], pf;
    scheme_freqs(*a->rope, th, &pf, &mult);
  }
  const double sigma = a->softmax_scale > 0.f ? (double)a->softmax_scale : mult / std::sqrt((double)a->d);
  p.scale_log2 = (float)(sigma * 1.4426950408889634074);
  p.B = a->B; p.Hq = a->Hq; p.Hkv = a->Hkv; p.G = a->Hq / a->Hkv; p.d = a->d;
  p.n_sink = a->n_sink;
  p.q_mode = a->rope_q ? 2 : (a->q_dtype == LCX_BF16 ? 1 : 0);
  p.k_mode = a->rope_k ? 2 : (a->k_dtype == LCX_BF16 ? 1 : 0);
  p.o_mode = a->o_dtype == LCX_BF16 ? 0 : (a->accumulate ? 2 : 1);
  p.causal = a->causal;
  p.v_tiled = a->v_tiled;
  p.precise_qk = a->precise_qk;
  p.sched = static_cast<unsigned long long*>(a->sched);
  return p;
}

lcx_status check_bwd(const lcx_attn_bwd_args* a) {
  if (!a) return fail(LCX_ERR_INVALID_ARG, "args is NULL");
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1) return fail(LCX_ERR_INVALID_ARG, "B, Hq, Hkv must be >= 1");
  if (a->n_q > 0 && (!a->q || !a->o || !a->lse || !a->d_o || !a->dq || !a->workspace))
    return fail(LCX_ERR_INVALID_ARG, "q, o, lse, d_o, dq and workspace are required when n_q > 0");
  if (a->n_kv > 0 && (!a->k || !a->v || !a->dk || !a->dv))
    return fail(LCX_ERR_INVALID_ARG, "k, v, dk and dv are required when n_kv > 0");
  if (a->Hq % a->Hkv) return fail(LCX_ERR_INVALID_ARG, "Hq %d is not a multiple of Hkv %d", a->Hq, a->Hkv);
  if (a->n_q < 0 || a->n_kv < 0) return fail(LCX_ERR_INVALID_ARG, "n_q and n_kv must be >= 0");
  if (a->d != 64 && a->d != 128) return fail(LCX_ERR_UNSUPPORTED, "head dim %d (kernels: 64, 128)", a->d);
  if (a->causal != 1) return fail(LCX_ERR_UNSUPPORTED, "only causal attention is implemented");
  if (a->window < -1) return fail(LCX_ERR_INVALID_ARG, "window %lld < -1", (long long)a->window);
  if (a->n_sink < 0) return fail(LCX_ERR_INVALID_ARG, "n_sink %d < 0", a->n_sink);
  if (a->o_dtype != LCX_BF16 && a->o_dtype != LCX_F32) return fail(LCX_ERR_INVALID_ARG, "o dtype");
  if (a->grad_dtype != LCX_BF16 && a->grad_dtype != LCX_F32) return fail(LCX_ERR_INVALID_ARG, "grad dtype");
  if (a->unrotate != 0 && a->unrotate != 1) return fail(LCX_ERR_INVALID_ARG, "unrotate must be 0 or 1");
  if (!(a->softmax_scale >= 0.f) || !std::isfinite(a->softmax_scale))
    return fail(LCX_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0 (0: default)");
  if (a->rope) {
    lcx_status st = check_cfg(a->rope);
    if (st != LCX_OK) return st;
    if (a->rope->head_dim != a->d)
      return fail(LCX_ERR_INVALID_ARG, "rope head_dim %d differs from d %d", a->rope->head_dim, a->d);
  }
  if (a->unrotate) {
    if (!a->rope) return fail(LCX_ERR_INVALID_ARG, "unrotate needs the rope configuration of the tables");
    if (!a->cos_tab || !a->sin_tab) return fail(LCX_ERR_INVALID_ARG, "unrotate needs the RoPE tables");
    if (!covers(a->tab_pos0, a->tab_len, a->q_pos0, a->n_q) || !covers(a->tab_pos0, a->tab_len, a->k_pos0, a->n_kv))
      return fail(LCX_ERR_INVALID_ARG, "table rows do not cover the query and key positions");
    if (!aligned16(a->cos_tab) || !aligned16(a->sin_tab))
      return fail(LCX_ERR_UNSUPPORTED, "tables must be 16-byte aligned");
  }
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o) || !aligned16(a->d_o) ||
      !aligned16(a->dq) || !aligned16(a->dk) || !aligned16(a->dv) || !aligned16(a->workspace))
    return fail(LCX_ERR_UNSUPPORTED, "tensors and workspace must be 16-byte aligned");
  if (!strides_ok(a->q_strides, 8) || !strides_ok(a->k_strides, 8) || !strides_ok(a->v_strides, 8) ||
      !strides_ok(a->do_strides, 8))
    return fail(LCX_ERR_UNSUPPORTED, "q/k/v/d_o strides must be non-negative multiples of 8 elements");
  if (!strides_ok(a->o_strides, a->o_dtype == LCX_F32 ? 4 : 8))
    return fail(LCX_ERR_UNSUPPORTED, "o strides must keep rows 16-byte aligned");
  if (!strides_ok(a->dq_strides, 4) || !strides_ok(a->dk_strides, 4) || !strides_ok(a->dv_strides, 4))
    return fail(LCX_ERR_UNSUPPORTED, "gradient strides must be non-negative multiples of 4 elements");
  if (a->lse_strides[0] < 0 || a->lse_strides[1] < 0)
    return fail(LCX_ERR_INVALID_ARG, "lse strides must be >= 0");
  // one 64-row tile is addressed with 32-bit buffer offsets
  const int64_t lim = (int64_t)1 << 24;
  if (a->q_strides[2] >= lim || a->k_strides[2] >= lim || a->v_strides[2] >= lim || a->do_strides[2] >= lim)
    return fail(LCX_ERR_UNSUPPORTED, "row strides must be below 2^24 elements");
  if ((reinterpret_cast<uintptr_t>(a->sched) & 7) != 0)
    return fail(LCX_ERR_UNSUPPORTED, "sched must be 8-byte aligned");
  const int64_t bm = lcx::attn_bwd_rows_per_block(a->d), bk = lcx::attn_bwd_keys_per_block(a->d);
  const bool dyn = a->sched != nullptr;
  // row and key indices of a tile are 32-bit in the kernels
  if (a->n_q > ((int64_t)1 << 31) - 64 || a->n_kv > ((int64_t)1 << 31) - 64)
    return fail(LCX_ERR_UNSUPPORTED, "n_q and n_kv must be below 2^31 - 64");
  if (lcx::sched_grid((int64_t)a->B * a->Hq * ((a->n_q + bm - 1) / bm), dyn) >= (int64_t)1 << 31 ||
      lcx::sched_grid((int64_t)a->B * a->Hkv * ((a->n_kv + bk - 1) / bk), dyn) >= (int64_t)1 << 31 ||
      (a->n_q + 63) / 64 * (a->Hq / a->Hkv) >= (int64_t)1 << 31)
    return fail(LCX_ERR_UNSUPPORTED, "problem too large for one launch");
  return LCX_OK;
}

lcx::BwdParams make_bwd_params(const lcx_attn_bwd_args* a) {
  lcx::BwdParams p{};
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint16_t*>(a->k);
  p.v = static_cast<const uint16_t*>(a->v);
  p.o = a->o;
  p.lse = a->lse;
  p.dout = static_cast<const uint16_t*>(a->d_o);
  p.stats = a->workspace;
  p.sched = static_cast<unsigned long long*>(a->sched);
  p.dq = a->dq; p.dk = a->dk; p.dv = a->dv;
  p.cos_tab = a->cos_tab; p.sin_tab = a->sin_tab;
  p.qs_b = a->q_strides[0]; p.qs_h = a->q_strides[1]; p.qs_s = a->q_strides[2];
  p.ks_b = a->k_strides[0]; p.ks_h = a->k_strides[1]; p.ks_s = a->k_strides[2];
  p.vs_b = a->v_strides[0]; p.vs_h = a->v_strides[1]; p.vs_s = a->v_strides[2];
  p.os_b = a->o_strides[0]; p.os_h = a->o_strides[1]; p.os_s = a->o_strides[2];
  p.dos_b = a->do_strides[0]; p.dos_h = a->do_strides[1]; p.dos_s = a->do_strides[2];
  p.ls_b = a->lse_strides[0]; p.ls_h = a->lse_strides[1];
  p.dqs_b = a->dq_strides[0]; p.dqs_h = a->dq_strides[1]; p.dqs_s = a->dq_strides[2];
  p.dks_b = a->dk_strides[0]; p.dks_h = a->dk_strides[1]; p.dks_s = a->dk_strides[2];
  p.dvs_b = a->dv_strides[0]; p.dvs_h = a->dv_strides[1]; p.dvs_s = a->dv_strides[2];
  p.n_q = a->n_q; p.n_kv = a->n_kv; p.q_pos0 = a->q_pos0; p.k_pos0 = a->k_pos0;
  p.tab_pos0 = a->tab_pos0;
  p.window = a->window;
  double mult = 1.0;
  if (a->rope) {  // head_dim == d (64 or 128), checked
    double th[lcx::kMaxHalfDim], pf;
    scheme_freqs(*a->rope, th, &pf, &mult);
  }
  const double sigma = a->softmax_scale > 0.f ? (double)a->softmax_scale : mult / std::sqrt((double)a->d);
  p.scale = (float)sigma;
  p.scale_log2 = (float)(sigma * 1.4426950408889634074);
  p.B = a->B; p.Hq = a->Hq; p.Hkv = a->Hkv; p.G = a->Hq / a->Hkv; p.d = a->d;
  p.n_sink = a->n_sink;
  p.causal = a->causal;
  p.o_f32 = a->o_dtype == LCX_F32;
  p.grad_f32 = a->grad_dtype == LCX_F32;
  p.unrotate = a->unrotate;
  return p;
}

lcx_status check_decode(const lcx_attn_args* a, int32_t n_splits) {
  lcx_status st = check_attn(a, false);
  if (st != LCX_OK) return st;
  if (a->accumulate) return fail(LCX_ERR_INVALID_ARG, "accumulate must be 0 for decode");
  if (a->n_q > 8) return fail(LCX_ERR_UNSUPPORTED, "decode takes at most 8 new rows (n_q = %lld)", (long long)a->n_q);
  if ((int64_t)(a->Hq / a->Hkv) * a->n_q > 64)
    return fail(LCX_ERR_UNSUPPORTED, "decode needs (Hq/Hkv)·n_q <= 64");
  if (a->rope_k || a->k_dtype != LCX_F16)
    return fail(LCX_ERR_UNSUPPORTED, "decode reads a pre-rotated f16 K cache (rope_k = 0, k_dtype F16)");
  if (a->precise_qk) return fail(LCX_ERR_UNSUPPORTED, "decode has no precise_qk form");
  if (n_splits < 1 || n_splits > 65535) return fail(LCX_ERR_INVALID_ARG, "n_splits %d outside 1..65535", n_splits);
  if (a->B > 65535 || a->Hkv > 65535) return fail(LCX_ERR_UNSUPPORTED, "B and Hkv must be <= 65535");
  return LCX_OK;
}

lcx_status run_decode(const lcx_attn_args* a, int32_t n_splits, float* o_part, float* lse_part,
                      hipStream_t stream) {
  lcx::AttnParams p = make_params(a);
  p.sched = nullptr;  // decode has its own split of the work
  lcx::DecodeParams dp{o_part, lse_part, n_splits};
  hipError_t e = lcx::launch_attn_decode(p, dp, stream);
  if (e != hipSuccess) return hip_status(e, "decode launch");
  return hip_status(lcx::launch_decode_combine(p, dp, stream), "combine launch");
}

// Device scratch of lcx_attn_decode_noalloc (the split partials), a
// file-scope array so that the entry point allocates nothing.  Each device
// the library runs on holds its own copy until the process ends.  In host
// code `scratch` only names the symbol: its device address is looked up once
// per device with that device current and kept in g_scratch_dev, which is
// what kernels receive.
static __device__ __align__(256) char scratch[LCX_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices];

lcx_status decode_scratch(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LCX_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(LCX_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_dev[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_dev[dev];
  return LCX_OK;
}

}  // namespace

extern "C" {

const char* lcx_status_string(lcx_status s) {
  switch (s) {
    case LCX_OK: return "LCX_OK";
    case LCX_ERR_INVALID_ARG: return "LCX_ERR_INVALID_ARG";
    case LCX_ERR_UNSUPPORTED: return "LCX_ERR_UNSUPPORTED";
    case LCX_ERR_HIP: return "LCX_ERR_HIP";
  }
  return "LCX_UNKNOWN_STATUS";
}

const char* lcx_last_error(void) { return g_err; }

lcx_status lcx_rope_freqs(const lcx_rope_cfg* cfg, int64_t pos0, int64_t n_pos, double* inv_freq,
                          double* pos_factor, double* logit_mult, float* cos_tab, float* sin_tab,
                          hipStream_t stream) {
  lcx_status st = check_cfg(cfg);
  if (st != LCX_OK) return st;
  if ((cos_tab == nullptr) != (sin_tab == nullptr))
    return fail(LCX_ERR_INVALID_ARG, "cos_tab and sin_tab must both be given or both be NULL");
  if (n_pos < 0 || pos0 < 0) return fail(LCX_ERR_INVALID_ARG, "pos0 and n_pos must be >= 0");
  const int half = cfg->head_dim / 2;
  if (cos_tab && half > lcx::kMaxHalfDim)
    return fail(LCX_ERR_UNSUPPORTED, "head_dim %d above the table kernel's %d", cfg->head_dim,
                2 * lcx::kMaxHalfDim);
  if (cos_tab && (!aligned16(cos_tab) || !aligned16(sin_tab)))
    return fail(LCX_ERR_UNSUPPORTED, "tables must be 16-byte aligned");
  double th_local[2 * lcx::kMaxHalfDim];
  double* th = th_local;
  double* th_heap = nullptr;
  if (half > 2 * lcx::kMaxHalfDim) th = th_heap = new double[half];
  double pf, lm;
  scheme_freqs(*cfg, th, &pf, &lm);
  if (inv_freq) std::memcpy(inv_freq, th, sizeof(double) * half);
  if (pos_factor) *pos_factor = pf;
  if (logit_mult) *logit_mult = lm;
  lcx_status res = ok();
  if (cos_tab) {
    lcx::RopeTableParams p{};
    p.cos_tab = cos_tab;
    p.sin_tab = sin_tab;
    p.pos0 = pos0;
    p.n_pos = n_pos;
    p.pos_factor = pf;
    p.half = half;
    for (int i = 0; i < half; ++i) p.theta[i] = th[i];
    res = hip_status(lcx::launch_rope_table(p, stream), "rope table launch");
  }
  delete[] th_heap;
  return res;
}

lcx_status lcx_rope_apply_qk(const void* q, void* q_out, const void* k, void* k_out,
                             int32_t out_dtype, int32_t B, int32_t Hq, int32_t Hkv, int64_t n,
                             int32_t d, const int64_t q_strides[3], const int64_t qo_strides[3],
                             const int64_t k_strides[3], const int64_t ko_strides[3], int64_t pos0,
                             const float* cos_tab, const float* sin_tab, int64_t tab_pos0,
                             int64_t tab_len, hipStream_t stream) {
  if ((q == nullptr) != (q_out == nullptr) || (k == nullptr) != (k_out == nullptr))
    return fail(LCX_ERR_INVALID_ARG, "an input needs its output and vice versa");
  if (!q && !k) return fail(LCX_ERR_INVALID_ARG, "nothing to rotate");
  if (out_dtype != LCX_BF16 && out_dtype != LCX_F16) return fail(LCX_ERR_INVALID_ARG, "out dtype");
  if (B < 1 || n < 0 || (q && Hq < 1) || (k && Hkv < 1))
    return fail(LCX_ERR_INVALID_ARG, "bad sizes");
  if (d < 2 || (d & 1)) return fail(LCX_ERR_INVALID_ARG, "d %d must be even", d);
  if (d % 8 || d / 2 > lcx::kMaxHalfDim)
    return fail(LCX_ERR_UNSUPPORTED, "d %d must be a multiple of 8 and <= %d", d, 2 * lcx::kMaxHalfDim);
  if (!cos_tab || !sin_tab) return fail(LCX_ERR_INVALID_ARG, "tables are required");
  if (!covers(tab_pos0, tab_len, pos0, n))
    return fail(LCX_ERR_INVALID_ARG, "table rows do not cover the positions");
  if (!aligned16(cos_tab) || !aligned16(sin_tab)) return fail(LCX_ERR_UNSUPPORTED, "table alignment");
  lcx::RopeApplyParams slots[2];
  int ns = 0;
  const void* ins[2] = {q, k};
  void* outs[2] = {q_out, k_out};
  const int64_t* ist[2] = {q_strides, k_strides};
  const int64_t* ost[2] = {qo_strides, ko_strides};
  const int32_t hs[2] = {Hq, Hkv};
  for (int t = 0; t < 2; ++t) {
    if (!ins[t]) continue;
    if (!ist[t] || !ost[t]) return fail(LCX_ERR_INVALID_ARG, "strides are required");
    if (!strides_ok(ist[t], 8) || !strides_ok(ost[t], 8) || !aligned16(ins[t]) || !aligned16(outs[t]))
      return fail(LCX_ERR_UNSUPPORTED, "rows must be 16-byte aligned");
    if (ins[t] == outs[t]) {
      if (out_dtype != LCX_BF16) return fail(LCX_ERR_INVALID_ARG, "in place needs a bf16 output");
      if (std::memcmp(ist[t], ost[t], 3 * sizeof(int64_t)))
        return fail(LCX_ERR_INVALID_ARG, "in place needs identical strides");
    }
    lcx::RopeApplyParams& p = slots[ns++];
    p.x = static_cast<const uint16_t*>(ins[t]);
    p.y = outs[t];
    p.xs_b = ist[t][0]; p.xs_h = ist[t][1]; p.xs_s = ist[t][2];
    p.ys_b = ost[t][0]; p.ys_h = ost[t][1]; p.ys_s = ost[t][2];
    p.B = B; p.H = hs[t]; p.n = n; p.d = d;
    p.out_f16 = out_dtype == LCX_F16;
    p.pos0 = pos0; p.tab_pos0 = tab_pos0;
    p.cos_tab = cos_tab; p.sin_tab = sin_tab;
  }
  return hip_status(lcx::launch_rope_apply(slots, ns, stream), "rope apply launch");
}

lcx_status lcx_attn_fwd(const lcx_attn_args* a, hipStream_t stream) {
  lcx_status st = check_attn(a, false);
  if (st != LCX_OK) return st;
  if (a->n_q == 0) return ok();
  return hip_status(lcx::launch_attn_fwd(make_params(a), stream), "attention launch");
}

lcx_status lcx_attn_decode(const lcx_attn_args* a, int32_t n_splits, float* o_part, float* lse_part,
                           hipStream_t stream) {
  lcx_status st = check_decode(a, n_splits);
  if (st != LCX_OK) return st;
  if (!o_part || !lse_part) return fail(LCX_ERR_INVALID_ARG, "o_part and lse_part are required");
  if (!aligned16(o_part)) return fail(LCX_ERR_UNSUPPORTED, "o_part must be 16-byte aligned");
  if (a->n_q == 0) return ok();
  return run_decode(a, n_splits, o_part, lse_part, stream);
}

lcx_status lcx_attn_decode_noalloc(const lcx_attn_args* a, int32_t n_splits, hipStream_t stream) {
  lcx_status st = check_decode(a, n_splits);
  if (st != LCX_OK) return st;
  if (a->n_q == 0) return ok();
  // partials: O fp32 [n_splits][B][Hq][n_q][d], then (256-byte aligned) LSE
  // fp32 [n_splits][B][Hq][n_q]; every slot is written by the decode kernel
  // before the combine pass reads it, so nothing needs clearing
  const uint64_t rows = (uint64_t)n_splits * (uint64_t)a->B * (uint64_t)a->Hq * (uint64_t)a->n_q;
  const uint64_t o_bytes = (rows * (uint64_t)a->d * 4u + 255u) & ~(uint64_t)255u;
  const uint64_t need = o_bytes + rows * 4u;
  if (need > LCX_DECODE_SCRATCH_BYTES)
    return fail(LCX_ERR_UNSUPPORTED,
                "decode partials need %llu bytes; the static scratch holds %llu (fewer splits, rows or heads)",
                (unsigned long long)need, (unsigned long long)LCX_DECODE_SCRATCH_BYTES);
  char* base = nullptr;
  st = decode_scratch(&base);
  if (st != LCX_OK) return st;
  return run_decode(a, n_splits, reinterpret_cast<float*>(base),
                    reinterpret_cast<float*>(base + o_bytes), stream);
}

lcx_status lcx_attn_pack_v(const void* v, void* v_tiles, int32_t B, int32_t Hkv, int64_t n,
                           int32_t d, const int64_t v_strides[3], hipStream_t stream) {
  if (!v || !v_tiles || !v_strides) return fail(LCX_ERR_INVALID_ARG, "v, v_tiles and v_strides are required");
  if (B < 1 || Hkv < 1 || n < 1) return fail(LCX_ERR_INVALID_ARG, "B, Hkv and n must be >= 1");
  if (B > 65535 || Hkv > 65535) return fail(LCX_ERR_UNSUPPORTED, "B and Hkv must be <= 65535");
  if (d != 64 && d != 128) return fail(LCX_ERR_UNSUPPORTED, "head dim %d (kernels: 64, 128)", d);
  if (v_strides[0] < 0 || v_strides[1] < 0 || v_strides[2] < 0)
    return fail(LCX_ERR_INVALID_ARG, "strides must be >= 0");
  if (!strides_ok(v_strides, 8) || !aligned16(v) || !aligned16(v_tiles))
    return fail(LCX_ERR_UNSUPPORTED, "rows must be 16-byte aligned");
  lcx::PackVParams p{};
  p.v = static_cast<const uint16_t*>(v);
  p.vt = static_cast<uint16_t*>(v_tiles);
  p.vs_b = v_strides[0]; p.vs_h = v_strides[1]; p.vs_s = v_strides[2];
  p.B = B; p.Hkv = Hkv; p.d = d; p.n = n;
  p.n_tiles = (n + 63) / 64;
  return hip_status(lcx::launch_pack_v(p, stream), "pack launch");
}

lcx_status lcx_attn_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                          int32_t B, int32_t H, int64_t rows, int32_t d,
                          const int64_t acc_strides[3], const int64_t part_strides[3],
                          const int64_t lse_acc_strides[2], const int64_t lse_part_strides[2],
                          void* o_final, int32_t o_final_dtype, const int64_t final_strides[3],
                          hipStream_t stream) {
  if (!o_acc || !lse_acc || !o_part || !lse_part || !acc_strides || !part_strides ||
      !lse_acc_strides || !lse_part_strides)
    return fail(LCX_ERR_INVALID_ARG, "o_acc, lse_acc, o_part, lse_part and strides are required");
  if (B < 1 || H < 1 || rows < 0 || d < 1) return fail(LCX_ERR_INVALID_ARG, "bad sizes");
  if (d % 4 || d > 1024) return fail(LCX_ERR_UNSUPPORTED, "d %d must be a multiple of 4, <= 1024", d);
  if (!strides_ok(acc_strides, 4) || !strides_ok(part_strides, 4) || !aligned16(o_acc) ||
      !aligned16(o_part))
    return fail(LCX_ERR_UNSUPPORTED, "fp32 rows must be 16-byte aligned");
  if (o_final) {
    if (o_final_dtype != LCX_BF16 && o_final_dtype != LCX_F32)
      return fail(LCX_ERR_INVALID_ARG, "o_final dtype");
    if (!final_strides || !strides_ok(final_strides, 4) || !aligned16(o_final))
      return fail(LCX_ERR_UNSUPPORTED, "o_final rows must be aligned");
    if (o_final_dtype == LCX_BF16 && (final_strides[0] % 4 || final_strides[1] % 4 || final_strides[2] % 4))
      return fail(LCX_ERR_UNSUPPORTED, "o_final strides");
  }
  lcx::MergeParams p{};
  p.o_acc = o_acc; p.lse_acc = lse_acc; p.o_part = o_part; p.lse_part = lse_part;
  p.o_final = o_final; p.final_f32 = o_final_dtype == LCX_F32;
  p.as_b = acc_strides[0]; p.as_h = acc_strides[1]; p.as_s = acc_strides[2];
  p.ps_b = part_strides[0]; p.ps_h = part_strides[1]; p.ps_s = part_strides[2];
  if (o_final) { p.fs_b = final_strides[0]; p.fs_h = final_strides[1]; p.fs_s = final_strides[2]; }
  p.la_b = lse_acc_strides[0]; p.la_h = lse_acc_strides[1];
  p.lp_b = lse_part_strides[0]; p.lp_h = lse_part_strides[1];
  p.B = B; p.H = H; p.d = d; p.rows = rows;
  return hip_status(lcx::launch_attn_merge(p, stream), "merge launch");
}

lcx_status lcx_attn_fwd_chunked(const lcx_attn_args* a, int64_t chunk, float* o_acc, float* lse_acc,
                                float* o_part, float* lse_part, hipStream_t stream) {
  lcx_status st = check_attn(a, true);
  if (st != LCX_OK) return st;
  if (chunk <= 0) return fail(LCX_ERR_INVALID_ARG, "chunk %lld must be > 0", (long long)chunk);
  if (a->v_tiled && chunk % 64)
    return fail(LCX_ERR_INVALID_ARG, "chunk %lld must be a multiple of 64 with tiled V", (long long)chunk);
  if (!o_acc || !lse_acc) return fail(LCX_ERR_INVALID_ARG, "o_acc and lse_acc are required");
  if ((o_part == nullptr) != (lse_part == nullptr))
    return fail(LCX_ERR_INVALID_ARG, "o_part and lse_part go together");
  if (!aligned16(o_acc) || (o_part && !aligned16(o_part)))
    return fail(LCX_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  // the final copy is skipped when a->o is the accumulator itself, which
  // holds fp32
  if (a->o == (void*)o_acc && a->o_dtype != LCX_F32)
    return fail(LCX_ERR_INVALID_ARG, "o may alias o_acc only with o_dtype F32");
  if (a->n_q == 0) return ok();
  const int64_t d = a->d, nq = a->n_q;
  const int64_t acc_st[3] = {a->Hq * nq * d, nq * d, d};
  const int64_t lse_st[2] = {a->Hq * nq, nq};
  hipError_t e = lcx::launch_fill_empty(o_acc, lse_acc, a->B, a->Hq, nq, a->d, acc_st[0], acc_st[1],
                                        acc_st[2], lse_st[0], lse_st[1], stream);
  if (e != hipSuccess) return hip_status(e, "fill launch");
  const int64_t n_chunks = (a->n_kv + chunk - 1) / chunk;
  for (int64_t c = 0; c < n_chunks; ++c) {
    const int64_t j0 = c * chunk;
    const int64_t len = (a->n_kv - j0 < chunk) ? a->n_kv - j0 : chunk;
    // causal: rows before the chunk's first key position cannot see it
    int64_t r0 = a->k_pos0 + j0 - a->q_pos0;
    if (r0 < 0) r0 = 0;
    if (r0 >= nq) continue;
    lcx_attn_args s = *a;
    s.q = static_cast<const uint16_t*>(a->q) + r0 * a->q_strides[2];
    s.n_q = nq - r0;
    s.q_pos0 = a->q_pos0 + r0;
    s.k = static_cast<const uint16_t*>(a->k) + j0 * a->k_strides[2];
    s.v = static_cast<const uint16_t*>(a->v) + (a->v_tiled ? (j0 / 64) * 64 * d : j0 * a->v_strides[2]);
    s.n_kv = len;
    s.k_pos0 = a->k_pos0 + j0;
    s.o_dtype = LCX_F32;
    s.lse_strides[0] = lse_st[0];
    s.lse_strides[1] = lse_st[1];
    s.o_strides[0] = acc_st[0]; s.o_strides[1] = acc_st[1]; s.o_strides[2] = acc_st[2];
    if (o_part) {
      s.o = o_part + r0 * d;
      s.lse = lse_part + r0;
      s.accumulate = 0;
    } else {
      s.o = o_acc + r0 * d;
      s.lse = lse_acc + r0;
      s.accumulate = 1;
    }
    lcx::AttnParams p = make_params(&s);
    e = lcx::launch_attn_fwd(p, stream);
    if (e != hipSuccess) return hip_status(e, "attention launch");
    if (o_part) {
      lcx::MergeParams m{};
      m.o_acc = o_acc + r0 * d; m.lse_acc = lse_acc + r0;
      m.o_part = o_part + r0 * d; m.lse_part = lse_part + r0;
      m.as_b = acc_st[0]; m.as_h = acc_st[1]; m.as_s = acc_st[2];
      m.ps_b = acc_st[0]; m.ps_h = acc_st[1]; m.ps_s = acc_st[2];
      m.la_b = lse_st[0]; m.la_h = lse_st[1]; m.lp_b = lse_st[0]; m.lp_h = lse_st[1];
      m.B = a->B; m.H = a->Hq; m.d = a->d; m.rows = nq - r0;
      e = lcx::launch_attn_merge(m, stream);
      if (e != hipSuccess) return hip_status(e, "merge launch");
    }
  }
  // final form: a->o in its dtype, a->lse
  if (a->o != (void*)o_acc || a->lse != lse_acc) {
    e = lcx::launch_finalize(o_acc, lse_acc, a->o, a->o_dtype == LCX_F32 ? 1 : 0, a->lse, a->B, a->Hq, nq,
                             a->d, acc_st, lse_st, a->o_strides, a->lse_strides, stream);
    if (e != hipSuccess) return hip_status(e, "finalize launch");
  }
  return ok();
}

lcx_status lcx_attn_bwd(const lcx_attn_bwd_args* a, hipStream_t stream) {
  lcx_status st = check_bwd(a);
  if (st != LCX_OK) return st;
  return hip_status(lcx::launch_attn_bwd(make_bwd_params(a), stream), "backward launch");
}

}  // extern "C"
