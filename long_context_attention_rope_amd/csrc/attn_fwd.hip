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
//  * Workgroup = NW waves; each wave owns 32 query rows of one head.  KV tiles
//    of 64 keys are staged in LDS by the whole workgroup.
//  * S^T = K·Q^T on v_mfma_f32_32x32x16_f16: the 32x32 accumulator of a wave
//    puts all 32 scores of one query row (for a 32-key block) in lanes l and
//    l^32, so row max / row sum are in-lane plus one permlane32 swap.
//  * The S^T accumulator is, after exp2 and bf16 packing, directly the B
//    operand of O^T += V^T·P^T on v_mfma_f32_32x32x16_bf16; V is transposed
//    while being staged (key order permuted within each 16-key group to match
//    the accumulator's row order), so each MFMA operand is one ds_read_b128.
//  * Per tile: S(t) = K(t)·Q^T, softmax, O += V(t)·P(t), with tile t+1's
//    buffer loads in flight (their range check zero-fills rows past the last
//    key) and staged into the other LDS buffer at the end; one barrier per
//    tile.  For d = 128 a workgroup is 8 waves (256 rows) and two waves share
//    each SIMD, so one wave's softmax overlaps the other's MFMAs.
//  * Q is rotated (RoPE from the fp32 tables) once per workgroup in registers;
//    K is either pre-rotated (f16) or rotated while being staged.
//  * Rotated q/k are rounded once to f16 (three more mantissa bits than bf16:
//    it keeps the LSE of short rows within 1e-3), P to bf16.
//  * Online softmax in base 2 with the scale folded into one FMA; the O
//    rescale is skipped while the running max grows by less than 2^8
//    (exact: the final O/l uses the same reference max for both).
//  * Tiles entirely outside the causal / window+sink mask are never visited;
//    only tiles that straddle a mask edge are masked per element (branch-free).
//  * Block order: longest causal rows first; the G query heads of one KV head
//    are dispatched consecutively to the same XCD so they share K/V in L2.
#include "lcx_device.h"
#include "lcx_internal.h"

namespace lcx {

namespace {

constexpr int BN = kBN;           // 64 keys per tile
constexpr float kLazyTau = 8.0f;  // log2 growth allowed before rescaling O

template <int D, int NW>
struct Tile {
  static constexpr int NT = 64 * NW;        // threads per workgroup
  static constexpr int BM = 32 * NW;        // query rows per workgroup
  static constexpr int KSTR = D + 8;        // f16 elements per K row in LDS (pad: conflict-free reads)
  static constexpr int VSTR = BN + 8;       // bf16 elements per V^T row in LDS
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int CPR = D / 8;         // 16-byte chunks per K row
  static constexpr int KCH = BN * CPR / NT; // K chunks per thread
  static constexpr int KRSTEP = NT / CPR;   // rows between a thread's chunks
  static constexpr int DPT = D / (4 * NW);  // V d-values per thread (for 4 keys)
  static_assert(KCH >= 1 && DPT >= 2, "tile split");
};

// saturate a position difference to +-2^30: every comparison against a key
// offset in [0, BN) keeps its outcome
__device__ __forceinline__ int clamp_i32(int64_t x) {
  return (int)(x > (1 << 30) ? (1 << 30) : (x < -(1 << 30) ? -(1 << 30) : x));
}
__device__ __forceinline__ int clamp_tile(int64_t x) {
  return (int)(x < 0 ? 0 : (x > BN ? BN : x));
}

// Buffer resource over [base, base + bytes): lane offsets >= bytes read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
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

// K tile staging: global (buffer loads) -> registers -> LDS, row-major f16.
// Per tile the resource starts at the tile's first key and ends at n_kv, so
// rows past the last key read as zero; lane offsets are fixed for the loop.
template <int D, int NW, int KMODE>
struct KStager {
  using T = Tile<D, NW>;
  u32x4 reg[T::KCH];
  f32x4 cs[KMODE == 2 ? T::KCH : 1];
  f32x4 sn[KMODE == 2 ? T::KCH : 1];
  const uint16_t* base;
  const float* cb;
  const float* sb;
  int64_t rs;  // row stride, elements
  int n_kv;
  uint32_t off[T::KCH], toff[KMODE == 2 ? T::KCH : 1];
  int lds_off[T::KCH];

  __device__ __forceinline__ void init(const AttnParams& p, const uint16_t* kbase, int tid) {
    base = kbase;
    rs = p.ks_s;
    n_kv = (int)p.n_kv;
    const int kc = tid % T::CPR;
    const int kr0 = tid / T::CPR;
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
      off[i] = (uint32_t)((kr0 + i * T::KRSTEP) * rs * 2) + (uint32_t)kc * 16u;
      lds_off[i] = (kr0 + i * T::KRSTEP) * T::KSTR + kc * 8;
    }
    if constexpr (KMODE == 2) {
      const int64_t r0 = p.k_pos0 - p.tab_pos0;  // table rows exist for keys 0 .. n_kv-1
      cb = p.cos_tab + r0 * (D / 2);
      sb = p.sin_tab + r0 * (D / 2);
#pragma unroll
      for (int i = 0; i < T::KCH; ++i)
        toff[i] = (uint32_t)(kr0 + i * T::KRSTEP) * (uint32_t)(D * 2) + (uint32_t)kc * 16u;
    }
  }
  __device__ __forceinline__ void load(int j0) {
    const uint32_t rows = n_kv > j0 ? (uint32_t)(n_kv - j0) : 0u;  // tiles past the end: empty range
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + j0 * rs, rows * (uint32_t)(rs * 2));
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) reg[i] = __builtin_amdgcn_raw_buffer_load_b128(r, off[i], 0, 0);
    if constexpr (KMODE == 2) {
      const __amdgpu_buffer_rsrc_t rc = make_rsrc(cb + j0 * (D / 2), rows * (uint32_t)(D * 2));
      const __amdgpu_buffer_rsrc_t rsn = make_rsrc(sb + j0 * (D / 2), rows * (uint32_t)(D * 2));
#pragma unroll
      for (int i = 0; i < T::KCH; ++i) {
        cs[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, toff[i], 0, 0));
        sn[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsn, toff[i], 0, 0));
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* ks) const {
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
      u32x4 w;
      if constexpr (KMODE == 2)
        w = rotate4_bf16<true>(reg[i], cs[i], sn[i]);
      else if constexpr (KMODE == 1)
        w = bf16_to_f16_4(reg[i]);
      else
        w = reg[i];
      *reinterpret_cast<u32x4*>(ks + lds_off[i]) = w;
    }
  }
};

// V tile staging: each thread loads DPT d-values of 4 consecutive keys and
// writes them transposed (V^T[d][key]); key group g of a 16-key chunk goes to
// slot group (g&1)*2 + (g>>1) so that the 8 keys one MFMA lane needs are
// adjacent (the accumulator row order of S^T).
template <int D, int NW>
struct VStager {
  using T = Tile<D, NW>;
  static constexpr int W = T::DPT / 2;  // 32-bit words per key
  uint32_t reg[4][W];
  const uint16_t* base;
  int64_t rs;
  int n_kv;
  uint32_t off;
  int lds_off;

  __device__ __forceinline__ void init(const AttnParams& p, const uint16_t* vbase, int tid) {
    base = vbase;
    rs = p.vs_s;
    n_kv = (int)p.n_kv;
    const int vkg = tid & 15;
    const int vdg = tid >> 4;
    off = (uint32_t)((4 * vkg) * rs * 2) + (uint32_t)(vdg * T::DPT * 2);
    const int g4 = vkg & 3;
    lds_off = (vdg * T::DPT) * T::VSTR + 16 * (vkg >> 2) + 4 * ((g4 & 1) * 2 + (g4 >> 1));
  }
  __device__ __forceinline__ void load(int j0) {
    const uint32_t rows = n_kv > j0 ? (uint32_t)(n_kv - j0) : 0u;  // tiles past the end: empty range
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + j0 * rs, rows * (uint32_t)(rs * 2));
    const uint32_t rb = (uint32_t)(rs * 2);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (W == 4) {
        const u32x4 z = __builtin_amdgcn_raw_buffer_load_b128(r, off + k * rb, 0, 0);
#pragma unroll
        for (int w = 0; w < 4; ++w) reg[k][w] = z[w];
      } else if constexpr (W == 2) {
        const u32x2 z = __builtin_amdgcn_raw_buffer_load_b64(r, off + k * rb, 0, 0);
        reg[k][0] = z[0];
        reg[k][1] = z[1];
      } else {
        reg[k][0] = __builtin_amdgcn_raw_buffer_load_b32(r, off + k * rb, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* vt) const {
#pragma unroll
    for (int e = 0; e < T::DPT; ++e) {
      const int w = e >> 1;
      // bytes {low half of key a, low half of key b} or the high halves
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x2 pk = {__builtin_amdgcn_perm(reg[1][w], reg[0][w], sel),
                  __builtin_amdgcn_perm(reg[3][w], reg[2][w], sel)};
      *reinterpret_cast<u32x2*>(vt + lds_off + e * T::VSTR) = pk;
    }
  }
};

template <int D, int NW>
__device__ __forceinline__ void qk_tile(const uint16_t* ks, const f16x8 (&qf)[D / 16], int l32, int h2,
                                        f32x16 (&s)[2]) {
  using T = Tile<D, NW>;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f16x8 a = *reinterpret_cast<const f16x8*>(ks + (kb * 32 + l32) * T::KSTR + 16 * c + 8 * h2);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[c], s[kb], 0, 0, 0);
    }
  }
}

template <int D, int KMODE, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_fwd_kernel(const AttnParams p) {
  using T = Tile<D, NW>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::K_ELEMS + 2 * T::V_ELEMS];
  auto ks_buf = [&](int i) { return smem + i * T::K_ELEMS; };
  auto vs_buf = [&](int i) { return smem + 2 * T::K_ELEMS + i * T::V_ELEMS; };

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

  const int64_t row0 = (int64_t)qblk * T::BM;
  const int64_t wrow0 = row0 + wave * 32;
  const int64_t qi = wrow0 + l32;  // this lane's query row
  const int64_t qpos = p.q_pos0 + qi;

  // ---- Q fragment (RoPE fused here when q_mode == 2)
  f16x8 qf[D / 16];
  load_q<D>(p, qbase, qi, h2, qf);

  // ---- KV tile range for the whole block: optional sink tiles, then the
  // window / causal range
  const int64_t blk_last = (row0 + T::BM < p.n_q ? row0 + T::BM : p.n_q) - 1;
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
  const int sink_n = (int)sink_t1;
  const int win_0 = (int)win_t0;
  const int ntl = (int)(sink_t1 + (win_t1 - win_t0));
  auto tile_j0 = [&](int t) { return (t < sink_n ? t : win_0 + (t - sink_n)) * BN; };

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

  KStager<D, NW, KMODE> kst;
  VStager<D, NW> vst;
  kst.init(p, kbase, tid);
  vst.init(p, vbase, tid);

  // ---- per-tile pieces of the online softmax
  // mask S(t) (only for tiles that straddle a mask edge for this wave)
  auto mask_tile = [&](f32x16 (&s)[2], const int j0) {
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
          s[kb][r] = ok ? s[kb][r] : -INFINITY;
        }
    }
  };
  // row max of a score tile, in scaled log2 units, shared by lanes l and l^32
  auto tile_max = [&](const f32x16 (&s)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    return xor32_max(mx) * p.scale_log2;
  };
  // move the reference max when the row max grew by more than 2^kLazyTau
  auto rescale = [&](const float mx) {
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
  };
  // P = exp2(S·scale - m) in bf16, row sums, O^T += V^T P^T
  auto exp_pv = [&](const f32x16 (&s)[2], const uint16_t* vt) {
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], p.scale_log2, -m_use));
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
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (db * 32 + l32) * T::VSTR + 16 * kc + 8 * h2);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kc], oacc[db], 0, 0, 0);
      }
    }
  };

  {
    // ---- one tile at a time: S(t), softmax, PV; tile t+1's global loads in
    // flight meanwhile, staged into the other buffer at the end
    if (ntl > 0) {
      kst.load(tile_j0(0));
      vst.load(tile_j0(0));
      kst.store(ks_buf(0));
      vst.store(vs_buf(0));
    }
    __syncthreads();
    for (int t = 0; t < ntl; ++t) {
      if (t + 1 < ntl) {
        kst.load(tile_j0(t + 1));
        vst.load(tile_j0(t + 1));
      }
      f32x16 s_cur[2];
      qk_tile<D, NW>(ks_buf(t & 1), qf, l32, h2, s_cur);
      mask_tile(s_cur, tile_j0(t));
      rescale(tile_max(s_cur));
      exp_pv(s_cur, vs_buf(t & 1));
      if (t + 1 < ntl) {  // the other buffer was last read before the previous barrier
        kst.store(ks_buf((t + 1) & 1));
        vst.store(vs_buf((t + 1) & 1));
      }
      __syncthreads();
    }
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

template <int D, int NW>
hipError_t launch_dn(const AttnParams& p, hipStream_t s, unsigned grid) {
  const dim3 block(64 * NW);
  switch (p.k_mode) {
    case 0: hipLaunchKernelGGL((attn_fwd_kernel<D, 0, NW>), dim3(grid), block, 0, s, p); break;
    case 1: hipLaunchKernelGGL((attn_fwd_kernel<D, 1, NW>), dim3(grid), block, 0, s, p); break;
    default: hipLaunchKernelGGL((attn_fwd_kernel<D, 2, NW>), dim3(grid), block, 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

int attn_rows_per_block(int d) { return 32 * (d == 64 ? kNWd64 : kNWd128); }

hipError_t launch_attn_fwd(const AttnParams& p_in, hipStream_t s) {
  AttnParams p = p_in;
  const int bm = attn_rows_per_block(p.d);
  p.n_qblk = (int32_t)((p.n_q + bm - 1) / bm);
  const int64_t units = (int64_t)p.B * p.Hkv * p.n_qblk;
  p.xcd_map = (units % 8 == 0) ? 1 : 0;
  const int64_t grid = units * p.G;
  if (grid == 0) return hipSuccess;
  if (p.d == 64) return launch_dn<64, kNWd64>(p, s, (unsigned)grid);
  return launch_dn<128, kNWd128>(p, s, (unsigned)grid);
}

}  // namespace lcx
