// Blockwise causal GQA attention with online softmax for gfx950 (steps a3-a8).
//
// What it computes (per query row i of head h, KV head g = h / (Hq/Hkv)):
//   S_j = sigma·<R(p_i) q_i, R(p_j) k_j> over kept keys j, P = softmax(S),
//   O_i = sum_j P_j v_j, LSE_i = ln sum_j exp(S_j)
// Sources: "AI 大模型窗口上下文进化史" §4 (scaled dot-product attention);
// "上下文擴充套件（Context Extension）" FlashAttention 的分塊計算策略 (Q/K/V split
// into B_r x B_c tiles kept on chip, running max, accumulated output, no n x n
// matrix in HBM) and 第二層 table (GQA); "上下文窗口扩展技术：从 4K 到 1M" §4.1
// (window K_[i-w, i]) and §4.2 (sink tokens 0-3 always kept).
//
// Design (CDNA4, wave64):
//  * Workgroup = 4 waves = 128 query rows of one head; each wave owns 32 rows.
//    KV tiles of 64 keys are staged in LDS (double buffered, next tile's
//    global loads in flight during the current tile's math).
//  * S^T = K·Q^T on v_mfma_f32_32x32x16_f16: the 32x32 accumulator of a wave
//    puts all 32 scores of one query row (for a 32-key block) in lanes l and
//    l^32, so row max / row sum are in-lane plus one permlane32 swap.
//  * The S^T accumulator is, after exp2 and bf16 packing, directly the B
//    operand of O^T += V^T·P^T on v_mfma_f32_32x32x16_bf16; V is transposed
//    while being staged (key order permuted within each 16-key group to match
//    the accumulator's row order), so each MFMA operand is one ds_read_b128.
//  * Q is rotated (RoPE from the fp32 tables) once per workgroup in registers;
//    K is either pre-rotated (f16) or rotated while being staged.
//  * Rotated q/k are rounded once to f16 (8 more bits than bf16 where it
//    matters: it keeps the LSE of short rows within 1e-3), P to bf16.
//  * Online softmax in base 2 with the scale folded into one FMA; the O
//    rescale is skipped while the running max grows by less than 2^8
//    (exact: the final O/l uses the same reference max for both).
//  * Tiles entirely outside the causal / window+sink mask are never visited;
//    only tiles that straddle a mask edge are masked per element.
//  * Block order: longest causal rows first; the G query heads of one KV head
//    are dispatched consecutively to the same XCD so they share K/V in L2.
#include "lcx_device.h"
#include "lcx_internal.h"

namespace lcx {

namespace {

constexpr int NW = 4;          // waves per workgroup
constexpr int BM = kBM;        // 128 query rows per workgroup
constexpr int BN = kBN;        // 64 keys per tile
constexpr float kLazyTau = 8.0f;  // log2 growth allowed before rescaling O

template <int D>
struct Tile {
  static constexpr int KSTR = D + 8;   // f16 elements per K row in LDS (pad: conflict-free reads)
  static constexpr int VSTR = BN + 8;  // bf16 elements per V^T row in LDS
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;  // uint16 elements per buffer
  static constexpr int CPR = D / 8;                // 16-byte chunks per K row
  static constexpr int KCH = BN * CPR / 256;       // K chunks per thread
  static constexpr int KRSTEP = 256 / CPR;         // rows between a thread's chunks
  static constexpr int DPT = D / 16;               // V d-values per thread (4 keys each)
};

// saturate a position difference to +-2^30: every comparison against a key
// offset in [0, BN) keeps its outcome
__device__ __forceinline__ int clamp_i32(int64_t x) {
  return (int)(x > (1 << 30) ? (1 << 30) : (x < -(1 << 30) ? -(1 << 30) : x));
}
__device__ __forceinline__ int clamp_tile(int64_t x) {
  return (int)(x < 0 ? 0 : (x > BN ? BN : x));
}

// Q fragment for the B operand of S^T = K Q^T: lane (n, h2) holds
// q[row n][16c + 8h2 .. +7] for c = 0 .. D/16-1, rotated and in f16.
template <int D>
__device__ __forceinline__ void load_q(const AttnParams& p, const uint16_t* qbase, int64_t qi,
                                       int h2, f16x8 (&qf)[D / 16]) {
  const bool valid = qi < p.n_q;
  const int64_t trow = p.q_pos0 + qi - p.tab_pos0;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const int col = 16 * c + 8 * h2;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (valid) raw = *reinterpret_cast<const u32x4*>(qbase + qi * p.qs_s + col);
    u32x4 w;
    if (p.q_mode == 2) {
      f32x4 cs = {1.f, 1.f, 1.f, 1.f}, sn = {0.f, 0.f, 0.f, 0.f};
      if (valid) {
        cs = *reinterpret_cast<const f32x4*>(p.cos_tab + trow * (D / 2) + col / 2);
        sn = *reinterpret_cast<const f32x4*>(p.sin_tab + trow * (D / 2) + col / 2);
      }
      w = rotate4_bf16<true>(raw, cs, sn);
    } else if (p.q_mode == 1) {
      w = bf16_to_f16_4(raw);
    } else {
      w = raw;
    }
    qf[c] = __builtin_bit_cast(f16x8, w);
  }
}

template <int D, int KMODE>
struct Stager {
  using T = Tile<D>;
  u32x4 kreg[T::KCH];
  f32x4 kcos[KMODE == 2 ? T::KCH : 1];
  f32x4 ksin[KMODE == 2 ? T::KCH : 1];
  uint32_t vreg[4][T::DPT / 2];

  // global -> registers for the tile starting at key j0
  __device__ __forceinline__ void load(const AttnParams& p, const uint16_t* kbase,
                                       const uint16_t* vbase, int64_t j0, int tid) {
    const int kc = tid % T::CPR;
    const int kr0 = tid / T::CPR;
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
      const int64_t j = j0 + kr0 + i * T::KRSTEP;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (j < p.n_kv) z = *reinterpret_cast<const u32x4*>(kbase + j * p.ks_s + kc * 8);
      kreg[i] = z;
      if constexpr (KMODE == 2) {
        f32x4 c1 = {1.f, 1.f, 1.f, 1.f}, s0 = {0.f, 0.f, 0.f, 0.f};
        if (j < p.n_kv) {
          const int64_t trow = p.k_pos0 + j - p.tab_pos0;
          c1 = *reinterpret_cast<const f32x4*>(p.cos_tab + trow * (D / 2) + kc * 4);
          s0 = *reinterpret_cast<const f32x4*>(p.sin_tab + trow * (D / 2) + kc * 4);
        }
        kcos[i] = c1;
        ksin[i] = s0;
      }
    }
    const int vkg = tid & 15;
    const int vdg = tid >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t j = j0 + 4 * vkg + r;
      const uint16_t* src = vbase + j * p.vs_s + vdg * T::DPT;
      if constexpr (T::DPT == 8) {
        u32x4 z = {0u, 0u, 0u, 0u};
        if (j < p.n_kv) z = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int w = 0; w < 4; ++w) vreg[r][w] = z[w];
      } else {
        u32x2 z = {0u, 0u};
        if (j < p.n_kv) z = *reinterpret_cast<const u32x2*>(src);
        vreg[r][0] = z[0];
        vreg[r][1] = z[1];
      }
    }
  }

  // registers -> LDS stage buffer (K row-major f16, V transposed bf16)
  __device__ __forceinline__ void store(uint16_t* stage, int tid) const {
    const int kc = tid % T::CPR;
    const int kr0 = tid / T::CPR;
    uint16_t* ks = stage;
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
      u32x4 w;
      if constexpr (KMODE == 2)
        w = rotate4_bf16<true>(kreg[i], kcos[i], ksin[i]);
      else if constexpr (KMODE == 1)
        w = bf16_to_f16_4(kreg[i]);
      else
        w = kreg[i];
      *reinterpret_cast<u32x4*>(ks + (kr0 + i * T::KRSTEP) * T::KSTR + kc * 8) = w;
    }
    // V^T: key group vkg (keys 4vkg..4vkg+3) goes to slot group perm(vkg % 4)
    // of its 16-key chunk so that the 8 keys an MFMA lane needs are adjacent.
    uint16_t* vt = stage + T::K_ELEMS;
    const int vkg = tid & 15;
    const int vdg = tid >> 4;
    const int g4 = vkg & 3;
    const int slot = 16 * (vkg >> 2) + 4 * ((g4 & 1) * 2 + (g4 >> 1));
#pragma unroll
    for (int e = 0; e < T::DPT; ++e) {
      const int w = e >> 1;
      uint32_t k0, k1, k2, k3;
      if (e & 1) {
        k0 = vreg[0][w] >> 16; k1 = vreg[1][w] >> 16; k2 = vreg[2][w] >> 16; k3 = vreg[3][w] >> 16;
      } else {
        k0 = vreg[0][w] & 0xffffu; k1 = vreg[1][w] & 0xffffu;
        k2 = vreg[2][w] & 0xffffu; k3 = vreg[3][w] & 0xffffu;
      }
      u32x2 pk = {k0 | (k1 << 16), k2 | (k3 << 16)};
      *reinterpret_cast<u32x2*>(vt + (vdg * T::DPT + e) * T::VSTR + slot) = pk;
    }
  }
};

template <int D, int KMODE>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const AttnParams p) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  // ---- block -> (b, q head, q block); longest rows first, KV group per XCD
  const int bid = blockIdx.x;
  int unit, g;
  if (p.xcd_map) {
    const int x = bid & 7;
    const int li = bid >> 3;
    g = li % p.G;
    unit = (li / p.G) * 8 + x;
  } else {
    unit = bid / p.G;
    g = bid % p.G;
  }
  const int hkv = unit % p.Hkv;
  const int t1 = unit / p.Hkv;
  const int b = t1 % p.B;
  const int qrank = t1 / p.B;
  const int qblk = p.n_qblk - 1 - qrank;
  const int hq = hkv * p.G + g;

  const uint16_t* qbase = p.q + b * p.qs_b + hq * p.qs_h;
  const uint16_t* kbase = p.k + b * p.ks_b + hkv * p.ks_h;
  const uint16_t* vbase = p.v + b * p.vs_b + hkv * p.vs_h;

  const int64_t row0 = (int64_t)qblk * BM;
  const int64_t wrow0 = row0 + wave * 32;
  const int64_t qi = wrow0 + l32;  // this lane's query row
  const int64_t qpos = p.q_pos0 + qi;

  // ---- Q fragment (RoPE fused here when q_mode == 2)
  f16x8 qf[D / 16];
  load_q<D>(p, qbase, qi, h2, qf);

  // ---- KV tile range for the whole block
  const int64_t blk_last = (row0 + BM < p.n_q ? row0 + BM : p.n_q) - 1;
  const int64_t qpos_min = p.q_pos0 + row0;
  const int64_t qpos_max = p.q_pos0 + blk_last;
  int64_t j_hi = p.n_kv;
  if (p.causal) {
    const int64_t lim = qpos_max - p.k_pos0 + 1;
    if (lim < j_hi) j_hi = lim;
  }
  int64_t j_lo = 0;
  if (p.window >= 0) {
    const int64_t lo = qpos_min - p.window - p.k_pos0;
    if (lo > j_lo) j_lo = lo;
  }
  int64_t win_t0 = j_lo / BN, win_t1 = j_hi > j_lo ? (j_hi + BN - 1) / BN : win_t0;
  int64_t sink_t1 = 0;
  if (p.window >= 0 && p.n_sink > 0) {
    int64_t se = (int64_t)p.n_sink - p.k_pos0;
    if (se > p.n_kv) se = p.n_kv;
    if (se > j_hi) se = j_hi;
    if (se > 0) sink_t1 = (se + BN - 1) / BN;
    if (sink_t1 > win_t0) sink_t1 = win_t0;
  }
  if (win_t1 < win_t0) win_t1 = win_t0;
  const int64_t n_tiles = sink_t1 + (win_t1 - win_t0);

  // ---- per-lane softmax state (row qi; lanes l and l^32 share the row)
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_run = -INFINITY;  // reference max, log2 units (scaled)
  float l_run = 0.f;        // this lane's partial row sum

  const int64_t wq_last = (wrow0 + 31 < p.n_q ? wrow0 + 31 : p.n_q - 1);
  const int64_t wqpos_min = p.q_pos0 + wrow0;
  const int64_t wqpos_max = p.q_pos0 + (wq_last >= wrow0 ? wq_last : wrow0);

  Stager<D, KMODE> st;
  if (n_tiles > 0) {
    const int64_t j0 = (0 < sink_t1 ? 0 : win_t0) * BN;
    st.load(p, kbase, vbase, j0, tid);
    st.store(smem, tid);
  }
  __syncthreads();

  for (int64_t it = 0; it < n_tiles; ++it) {
    const int64_t tile = it < sink_t1 ? it : win_t0 + (it - sink_t1);
    const int64_t j0 = tile * BN;
    const uint16_t* stage = smem + (it & 1) * T::STAGE;
    const bool has_next = it + 1 < n_tiles;
    if (has_next) {
      const int64_t nt = (it + 1) < sink_t1 ? (it + 1) : win_t0 + (it + 1 - sink_t1);
      st.load(p, kbase, vbase, nt * BN, tid);
    }

    // ---- S^T = K Q^T for two 32-key blocks
    f32x16 sacc[2];
    const uint16_t* ks = stage;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(ks + (kb * 32 + l32) * T::KSTR + 16 * c + 8 * h2);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[c], sacc[kb], 0, 0, 0);
      }
    }

    // ---- mask (only for tiles that straddle a mask edge for this wave)
    const int64_t kpos_min = p.k_pos0 + j0;
    const int64_t kpos_max = p.k_pos0 + (j0 + BN <= p.n_kv ? j0 + BN : p.n_kv) - 1;
    const bool all_kept = (j0 + BN <= p.n_kv) && (!p.causal || kpos_max <= wqpos_min) &&
                          (p.window < 0 || kpos_min >= wqpos_max - p.window ||
                           kpos_max < (int64_t)p.n_sink);
    if (!all_kept) {
      // Branch-free, in 32-bit offsets within the tile: key at offset `off`
      // (position kpos_min + off) is kept iff off < krem (exists),
      // off <= hi (causal), and off >= lo (window) or off < srem (sink).
      const int64_t rel = qpos - kpos_min;
      const int hi = p.causal ? clamp_i32(rel) : (1 << 30);
      const int lo = p.window >= 0 ? clamp_i32(rel - p.window) : -(1 << 30);
      const int srem = clamp_tile((int64_t)p.n_sink - kpos_min);
      const int krem = clamp_tile(p.n_kv - j0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + (r >> 2) * 8 + h2 * 4 + (r & 3);
          const bool ok = (off < krem) & (off <= hi) & ((off >= lo) | (off < srem));
          sacc[kb][r] = ok ? sacc[kb][r] : -INFINITY;
        }
    }

    // ---- online softmax (base 2)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = xor32_max(mx) * p.scale_log2;
    const float m_new = fmaxf(m_run, mx);
    if (__any(m_new > m_run + kLazyTau)) {
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], p.scale_log2, -m_use));
        l_run += pv[r];
      }
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(pv[8 * hlf + 2 * i], pv[8 * hlf + 2 * i + 1]);
        pf[kb * 2 + hlf] = __builtin_bit_cast(bf16x8, w);
      }
    }

    // ---- O^T += V^T P^T
    const uint16_t* vt = stage + T::K_ELEMS;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (db * 32 + l32) * T::VSTR + 16 * kc + 8 * h2);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kc], oacc[db], 0, 0, 0);
      }
    }

    if (has_next) st.store(smem + ((it + 1) & 1) * T::STAGE, tid);
    __syncthreads();
  }

  // ---- epilogue: O = O_acc / l, LSE = ln 2 · (m + log2 l)
  const float l_tot = xor32_sum(l_run);
  if (qi >= p.n_q) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_new = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
  float* lse_ptr = p.lse + b * p.ls_b + hq * p.ls_h + qi;

  if (p.o_mode == 0) {
    uint16_t* op = static_cast<uint16_t*>(p.o) + b * p.os_b + hq * p.os_h + qi * p.os_s;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + r4 * 8 + h2 * 4;
        u32x2 w = {pack_bf16x2(oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv),
                   pack_bf16x2(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d0) = w;
      }
    if (h2 == 0) *lse_ptr = lse_new;
  } else if (p.o_mode == 1) {
    float* op = static_cast<float*>(p.o) + b * p.os_b + hq * p.os_h + qi * p.os_s;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + r4 * 8 + h2 * 4;
        f32x4 w = {oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv, oacc[db][4 * r4 + 2] * inv,
                   oacc[db][4 * r4 + 3] * inv};
        *reinterpret_cast<f32x4*>(op + d0) = w;
      }
    if (h2 == 0) *lse_ptr = lse_new;
  } else {
    // merge into the existing partial: identity when either side is empty
    float* op = static_cast<float*>(p.o) + b * p.os_b + hq * p.os_h + qi * p.os_s;
    const float lse_old = *lse_ptr;
    if (lse_new == -INFINITY) return;
    float wa, wb, lse_m;
    if (lse_old == -INFINITY) {
      wa = 0.f; wb = 1.f; lse_m = lse_new;
    } else {
      const float mxl = fmaxf(lse_old, lse_new);
      const float mnl = fminf(lse_old, lse_new);
      lse_m = mxl + log1pf(expf(mnl - mxl));
      wa = expf(lse_old - lse_m);
      wb = expf(lse_new - lse_m);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + r4 * 8 + h2 * 4;
        f32x4 old = *reinterpret_cast<const f32x4*>(op + d0);
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (lse_old == -INFINITY ? 0.f : wa * old[e]) + wb * (oacc[db][4 * r4 + e] * inv);
        *reinterpret_cast<f32x4*>(op + d0) = w;
      }
    if (h2 == 0) *lse_ptr = lse_m;
  }
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t s, unsigned grid) {
  switch (p.k_mode) {
    case 0: hipLaunchKernelGGL((attn_fwd_kernel<D, 0>), dim3(grid), dim3(256), 0, s, p); break;
    case 1: hipLaunchKernelGGL((attn_fwd_kernel<D, 1>), dim3(grid), dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((attn_fwd_kernel<D, 2>), dim3(grid), dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnParams& p_in, hipStream_t s) {
  AttnParams p = p_in;
  p.n_qblk = (int32_t)((p.n_q + BM - 1) / BM);
  const int64_t units = (int64_t)p.B * p.Hkv * p.n_qblk;
  p.xcd_map = (units % 8 == 0) ? 1 : 0;
  const int64_t grid = units * p.G;
  if (grid == 0) return hipSuccess;
  if (p.d == 64) return launch_d<64>(p, s, (unsigned)grid);
  return launch_d<128>(p, s, (unsigned)grid);
}

}  // namespace lcx
