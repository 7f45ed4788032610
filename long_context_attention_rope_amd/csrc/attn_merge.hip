// Merge of partial attention results (step a9) and helpers of the chunked
// driver (step a10).
//
// Two results (O_a, L_a), (O_b, L_b) of the same query row over disjoint key
// sets combine exactly as
//   L = max(L_a, L_b) + log1p(exp(-|L_a - L_b|)),  O = e^(L_a-L) O_a + e^(L_b-L) O_b
// — the running-max rescaling of "上下文擴充套件（Context Extension）",
// FlashAttention 的分塊計算策略, written with log-sum-exp; it is what each ring
// step of "上下文窗口扩展技术：从 4K 到 1M" §5.3 needs (the listing's plain "+="
// of partial outputs would weight the blocks wrongly).  L = -inf is an empty
// partial and acts as the identity.
//
// HBM-bound: one workgroup of up to 256 threads covers whole rows (d/4
// threads per row, 16 bytes each); every thread of a row reads both LSEs
// before the barrier, one thread writes the merged LSE after it.
#include "lcx_device.h"
#include "lcx_internal.h"

namespace lcx {

__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams p, int rows_per_block) {
  const int tpr = p.d >> 2;  // threads per row
  const int lr = threadIdx.x / tpr;
  const int c = threadIdx.x - lr * tpr;
  const int64_t flat = (int64_t)blockIdx.x * rows_per_block + lr;  // over B*H*rows
  const int64_t total = (int64_t)p.B * p.H * p.rows;
  const bool active = lr < rows_per_block && flat < total;
  float la = -INFINITY, lb = -INFINITY;
  int64_t r = 0, bh = 0;
  int b = 0, h = 0;
  if (active) {
    r = flat % p.rows;
    bh = flat / p.rows;
    h = (int)(bh % p.H);
    b = (int)(bh / p.H);
    la = p.lse_acc[b * p.la_b + h * p.la_h + r];
    lb = p.lse_part[b * p.lp_b + h * p.lp_h + r];
  }
  __syncthreads();  // every old LSE is read before any is overwritten
  if (!active) return;
  float wa, wb, L;
  if (lb == -INFINITY) {
    wa = 1.f; wb = 0.f; L = la;
  } else if (la == -INFINITY) {
    wa = 0.f; wb = 1.f; L = lb;
  } else {
    const float mx = fmaxf(la, lb), mn = fminf(la, lb);
    L = mx + log1pf(expf(mn - mx));
    wa = expf(la - L);
    wb = expf(lb - L);
  }
  float* oa = p.o_acc + b * p.as_b + h * p.as_h + r * p.as_s + 4 * c;
  const float* ob = p.o_part + b * p.ps_b + h * p.ps_h + r * p.ps_s + 4 * c;
  const f32x4 va = load_once(reinterpret_cast<const f32x4*>(oa));
  const f32x4 vb = load_once(reinterpret_cast<const f32x4*>(ob));
  f32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = (wa == 0.f ? 0.f : wa * va[e]) + (wb == 0.f ? 0.f : wb * vb[e]);
  *reinterpret_cast<f32x4*>(oa) = o;
  if (p.o_final) {
    if (p.final_f32) {
      float* of = static_cast<float*>(p.o_final) + b * p.fs_b + h * p.fs_h + r * p.fs_s + 4 * c;
      *reinterpret_cast<f32x4*>(of) = o;
    } else {
      uint16_t* of = static_cast<uint16_t*>(p.o_final) + b * p.fs_b + h * p.fs_h + r * p.fs_s + 4 * c;
      u32x2 w = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      *reinterpret_cast<u32x2*>(of) = w;
    }
  }
  if (c == 0) p.lse_acc[b * p.la_b + h * p.la_h + r] = L;
}

hipError_t launch_attn_merge(const MergeParams& p, hipStream_t s) {
  const int tpr = p.d / 4;
  const int rpb = tpr >= 256 ? 1 : 256 / tpr;
  const int64_t total = (int64_t)p.B * p.H * p.rows;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + rpb - 1) / rpb;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)blocks), dim3(rpb * tpr), 0, s, p, rpb);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_empty_kernel(float* o, float* lse, int32_t B, int32_t H,
                                                         int64_t rows, int32_t d, int64_t os_b,
                                                         int64_t os_h, int64_t os_s, int64_t ls_b,
                                                         int64_t ls_h) {
  const int tpr = d >> 2;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t flat = t / tpr;
  const int c = (int)(t - flat * tpr);
  if (flat >= (int64_t)B * H * rows) return;
  const int64_t r = flat % rows;
  const int64_t bh = flat / rows;
  const int h = (int)(bh % H), b = (int)(bh / H);
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  *reinterpret_cast<f32x4*>(o + b * os_b + h * os_h + r * os_s + 4 * c) = z;
  if (c == 0) lse[b * ls_b + h * ls_h + r] = -INFINITY;
}

hipError_t launch_fill_empty(float* o, float* lse, int32_t B, int32_t H, int64_t rows, int32_t d,
                             int64_t os_b, int64_t os_h, int64_t os_s, int64_t ls_b, int64_t ls_h,
                             hipStream_t s) {
  const int64_t total = (int64_t)B * H * rows * (d / 4);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_empty_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, o,
                     lse, B, H, rows, d, os_b, os_h, os_s, ls_b, ls_h);
  return hipGetLastError();
}

struct FinalizeParams {
  const float* o_acc;
  const float* lse_acc;
  void* o;
  float* lse;
  int32_t o_f32, copy_o, copy_lse;
  int32_t B, H, d;
  int64_t rows;
  int64_t as_b, as_h, as_s, la_b, la_h;
  int64_t os_b, os_h, os_s, ls_b, ls_h;
};

__global__ __launch_bounds__(256) void finalize_kernel(FinalizeParams p) {
  const int tpr = p.d >> 2;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t flat = t / tpr;
  const int c = (int)(t - flat * tpr);
  if (flat >= (int64_t)p.B * p.H * p.rows) return;
  const int64_t r = flat % p.rows;
  const int64_t bh = flat / p.rows;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  if (p.copy_o) {
    const f32x4 v = load_once(reinterpret_cast<const f32x4*>(p.o_acc + b * p.as_b + h * p.as_h + r * p.as_s + 4 * c));
    if (p.o_f32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + b * p.os_b + h * p.os_h + r * p.os_s + 4 * c) = v;
    } else {
      u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o) + b * p.os_b + h * p.os_h + r * p.os_s + 4 * c) = w;
    }
  }
  if (p.copy_lse && c == 0) p.lse[b * p.ls_b + h * p.ls_h + r] = p.lse_acc[b * p.la_b + h * p.la_h + r];
}

hipError_t launch_finalize(const float* o_acc, const float* lse_acc, void* o, int32_t o_f32,
                           float* lse, int32_t B, int32_t H, int64_t rows, int32_t d,
                           const int64_t acc_st[3], const int64_t lse_acc_st[2],
                           const int64_t o_st[3], const int64_t lse_st[2], hipStream_t s) {
  FinalizeParams p{};
  p.o_acc = o_acc; p.lse_acc = lse_acc; p.o = o; p.lse = lse;
  p.o_f32 = o_f32;
  p.copy_o = (o != (const void*)o_acc) ? 1 : 0;
  p.copy_lse = (lse != lse_acc) ? 1 : 0;
  p.B = B; p.H = H; p.d = d; p.rows = rows;
  p.as_b = acc_st[0]; p.as_h = acc_st[1]; p.as_s = acc_st[2];
  p.la_b = lse_acc_st[0]; p.la_h = lse_acc_st[1];
  p.os_b = o_st[0]; p.os_h = o_st[1]; p.os_s = o_st[2];
  p.ls_b = lse_st[0]; p.ls_h = lse_st[1];
  const int64_t total = (int64_t)B * H * rows * (d / 4);
  if (total == 0 || (!p.copy_o && !p.copy_lse)) return hipSuccess;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace lcx

// Combine of the split-KV decode partials: for each query row, the n_splits
// (O_s, L_s) pairs (L_s = -inf: a split with no kept key) merge as
// L = log sum_s e^(L_s), O = sum_s e^(L_s - L) O_s, taken about the largest
// L_s.  One workgroup of 256 threads per row: d/4 column groups of 16 bytes
// times 256/(d/4) groups of splits, whose independent loads are in flight
// together; the groups' sums meet in LDS.
namespace lcx {

namespace {

template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const AttnParams p, const DecodeParams dp) {
  constexpr int CG = D / 4;     // column groups of 4 floats
  constexpr int SG = 256 / CG;  // split groups: thread (c, sg) takes splits sg, sg + SG, ...
  __shared__ float wmax[4];
  __shared__ f32x4 part[SG][CG];
  __shared__ float lsum[SG];
  const int64_t row = blockIdx.x;  // (b·Hq + hq)·n_q + r
  const int nq = (int)p.n_q;
  const int r = (int)(row % nq);
  const int64_t bh = row / nq;
  const int hq = (int)(bh % p.Hq);
  const int b = (int)(bh / p.Hq);
  const int64_t rows_all = (int64_t)p.B * p.Hq * nq;
  const int t = threadIdx.x;
  const int c = t % CG, sg = t / CG;
  // The first PRE partials of this thread's splits (sg, sg + SG, ...) are
  // loaded together with the LSEs the row maximum is taken over, so that one
  // memory round trip serves both.  Every split writes its whole partial (an
  // empty one O = 0 and LSE = -inf), so the loads need no condition; empty
  // partials get weight 0.
  constexpr int PRE = 4;
  f32x4 o_pre[PRE];
  float l_pre[PRE];
#pragma unroll
  for (int i = 0; i < PRE; ++i) {
    const int sp = sg + i * SG;
    const bool ok = sp < dp.n_splits;
    const int64_t at = (ok ? sp : 0) * rows_all + row;
    l_pre[i] = ok ? dp.lse_part[at] : -INFINITY;
    o_pre[i] = load_once(reinterpret_cast<const f32x4*>(dp.o_part + at * D + 4 * c));
  }
  // the largest partial LSE of the row (the reference for the weights)
  float m = -INFINITY;
  for (int sp = t; sp < dp.n_splits; sp += 256) m = fmaxf(m, dp.lse_part[sp * rows_all + row]);
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) m = fmaxf(m, __shfl_xor(m, off));
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  const float mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  // weighted sums of this thread's splits: no running rescale
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  auto add = [&](float ls, const f32x4& o) {
    // an empty partial (also every partial when mx is -inf) weighs 0
    const float w = ls == -INFINITY ? 0.f : expf(ls - mx);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += w * o[e];
    l += w;
  };
#pragma unroll
  for (int i = 0; i < PRE; ++i) add(l_pre[i], o_pre[i]);
  for (int sp = sg + PRE * SG; sp < dp.n_splits; sp += SG) {
    const int64_t at = sp * rows_all + row;
    add(dp.lse_part[at], load_once(reinterpret_cast<const f32x4*>(dp.o_part + at * D + 4 * c)));
  }
  part[sg][c] = acc;
  if (c == 0) lsum[sg] = l;
  __syncthreads();
  if (sg != 0) return;
  f32x4 tot = part[0][c];
  float lt = lsum[0];
#pragma unroll
  for (int i = 1; i < SG; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) tot[e] += part[i][c][e];
    lt += lsum[i];
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (p.o_mode == 0) {
    uint16_t* op = static_cast<uint16_t*>(p.o) + b * p.os_b + hq * p.os_h + r * p.os_s + 4 * c;
    u32x2 w = {pack_bf16x2(tot[0] * inv, tot[1] * inv), pack_bf16x2(tot[2] * inv, tot[3] * inv)};
    *reinterpret_cast<u32x2*>(op) = w;
  } else {
    float* op = static_cast<float*>(p.o) + b * p.os_b + hq * p.os_h + r * p.os_s + 4 * c;
    f32x4 w = {tot[0] * inv, tot[1] * inv, tot[2] * inv, tot[3] * inv};
    *reinterpret_cast<f32x4*>(op) = w;
  }
  if (c == 0) p.lse[b * p.ls_b + hq * p.ls_h + r] = lt > 0.f ? mx + logf(lt) : -INFINITY;
}

}  // namespace

hipError_t launch_decode_combine(const AttnParams& p, const DecodeParams& dp, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.Hq * p.n_q;
  if (rows == 0) return hipSuccess;
  if (p.d == 64)
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3((unsigned)rows), dim3(256), 0, s, p, dp);
  else
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3((unsigned)rows), dim3(256), 0, s, p, dp);
  return hipGetLastError();
}

}  // namespace lcx
