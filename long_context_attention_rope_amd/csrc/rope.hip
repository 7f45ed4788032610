// RoPE kernels for gfx950: the cos/sin table (step a2) and the standalone
// Q/K rotation (step a3).
//
// Table: c[r][i] = cos(((pos0 + r)·factor)·theta'_i), s likewise — the angle
// of pair i at a position ("上下文擴充套件（Context Extension）", 技術原理:
// φ_{m,i} = m·θ_i; PI scales m by L_train/L_target, "上下文窗口扩展技术：从 4K 到
// 1M" §2.1).  The angle is formed and evaluated in fp64 and rounded once to
// fp32: at positions near 2^20 an fp32 angle would already be off by ~0.06 rad.
// Within a run of positions the angles advance by the fp64 angle-addition
// recurrence (below).
//
// Rotation: adjacent pairs (x_{2i}, x_{2i+1}) -> (x_{2i}c - x_{2i+1}s,
// x_{2i}s + x_{2i+1}c) (same page, 技術原理: R(m) turns each pair (2i, 2i+1)).
// One thread owns one 16-byte chunk (4 pairs) of one position and walks all
// heads of q and k, so each table entry is read from HBM once.
#include "lcx_device.h"
#include "lcx_internal.h"

namespace lcx {

// Positions are taken in runs of kRun consecutive rows per pair: the first
// angle of a run, ((pos0 + r0)·factor)·theta'_i, is formed and evaluated in
// fp64 (sincos), the following ones by the fp64 angle-addition recurrence
//   cos(a + delta) = cos a·cos delta - sin a·sin delta,
//   sin(a + delta) = sin a·cos delta + cos a·sin delta,
// with delta = factor·theta'_i, also from fp64 sincos.  Each step adds about
// one fp64 rounding (2^-53 relative), so after kRun steps the values differ
// from the directly evaluated ones by ~1e-14, against the 2^-24 of the fp32
// rounding that follows; two sincos per kRun entries instead of one per entry
// leave the kernel bound by its HBM writes.  Lanes take consecutive pairs of
// one run, so each row segment is written by consecutive lanes.
constexpr int kRun = 32;

__global__ __launch_bounds__(256) void rope_table_kernel(RopeTableParams p) {
  const int64_t n_runs = (p.n_pos + kRun - 1) / kRun;
  const int64_t total = n_runs * (int64_t)p.half;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const int64_t run = e / p.half;
    const int i = (int)(e - run * p.half);
    const int64_t r0 = run * kRun;
    const double phi0 = ((double)(p.pos0 + r0) * p.pos_factor) * p.theta[i];
    double s, c, sd, cd;
    sincos(phi0, &s, &c);
    sincos(p.pos_factor * p.theta[i], &sd, &cd);
    const int rows = (int)(p.n_pos - r0 < kRun ? p.n_pos - r0 : kRun);
    float* cp = p.cos_tab + r0 * p.half + i;
    float* sp = p.sin_tab + r0 * p.half + i;
    for (int r = 0; r < rows; ++r) {
      cp[(int64_t)r * p.half] = (float)c;
      sp[(int64_t)r * p.half] = (float)s;
      const double cn = c * cd - s * sd;
      s = s * cd + c * sd;
      c = cn;
    }
  }
}

hipError_t launch_rope_table(const RopeTableParams& p, hipStream_t s) {
  const int64_t total = (p.n_pos + kRun - 1) / kRun * (int64_t)p.half;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

struct RopeApplyLaunch {
  RopeApplyParams slot[2];
  int32_t n_slots;
};

__global__ __launch_bounds__(256) void rope_apply_kernel(RopeApplyLaunch L) {
  const RopeApplyParams& p0 = L.slot[0];
  const int cpr = p0.d >> 3;  // 16-byte chunks per row
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= p0.n * cpr) return;
  const int64_t srow = t / cpr;
  const int c = (int)(t - srow * cpr);
  const int half = p0.d >> 1;
  const int64_t trow = p0.pos0 + srow - p0.tab_pos0;
  const f32x4 cs = load_once(reinterpret_cast<const f32x4*>(p0.cos_tab + trow * half + c * 4));
  const f32x4 sn = load_once(reinterpret_cast<const f32x4*>(p0.sin_tab + trow * half + c * 4));
  for (int sl = 0; sl < L.n_slots; ++sl) {
    const RopeApplyParams& p = L.slot[sl];
    for (int b = 0; b < p.B; ++b) {
      for (int h = 0; h < p.H; ++h) {
        const uint16_t* xp = p.x + b * p.xs_b + h * p.xs_h + srow * p.xs_s + c * 8;
        const u32x4 x = load_once(reinterpret_cast<const u32x4*>(xp));
        const u32x4 y = p.out_f16 ? rotate4_bf16<true>(x, cs, sn) : rotate4_bf16<false>(x, cs, sn);
        uint16_t* yp = static_cast<uint16_t*>(p.y) + b * p.ys_b + h * p.ys_h + srow * p.ys_s + c * 8;
        *reinterpret_cast<u32x4*>(yp) = y;
      }
    }
  }
}

hipError_t launch_rope_apply(const RopeApplyParams* slots, int n_slots, hipStream_t s) {
  if (n_slots <= 0) return hipSuccess;
  RopeApplyLaunch L;
  L.n_slots = n_slots;
  for (int i = 0; i < n_slots; ++i) L.slot[i] = slots[i];
  const int64_t total = slots[0].n * (slots[0].d / 8);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(rope_apply_kernel, dim3((unsigned)blocks), dim3(256), 0, s, L);
  return hipGetLastError();
}

}  // namespace lcx
