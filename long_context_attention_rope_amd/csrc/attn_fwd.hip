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
//  * The S^T accumulator is, after exp2 and 16-bit packing, directly the B
//    operand of O^T += V^T·P^T.  From V tiles (lcx_attn_pack_v: f16, keys of
//    each 16-key group in the accumulator's row order) each MFMA operand is
//    one ds_read_b128 and P is packed to f16 (v_mfma_f32_32x32x16_f16); from
//    bf16 V rows the operand takes two transposing reads and P is bf16.
//  * Per tile: S(t) = K(t)·Q^T, softmax, O += V(t)·P(t), with tile t+1's
//    buffer loads in flight (their range check zero-fills rows past the last
//    key) and staged into the other LDS buffer at the end; one barrier per
//    tile.  For d = 128 a workgroup is 8 waves (256 rows) and two waves share
//    each SIMD, so one wave's softmax overlaps the other's MFMAs.
//  * Q is rotated (RoPE from the fp32 tables) once per workgroup in registers;
//    K is either pre-rotated (f16) or rotated while being staged.
//  * Rotated q/k are rounded once to f16 (three more mantissa bits than bf16:
//    it keeps the LSE of short rows within 1e-3); P to f16 against V tiles,
//    to bf16 against V rows.
//  * Online softmax in base 2: Q is scaled by sigma·log2(e) before its f16
//    rounding and the QK^T product starts from -m (the row's reference max)
//    in the accumulator, so the scores come out ready for exp2 with no
//    per-element VALU work.  The reference max moves (and O is rescaled)
//    only when a row's max grows by more than 2^8 (exact: the final O/l uses
//    the same reference max for both).  Row sums add P rounded to f16 (the
//    PV operand itself from tiles), two per v_dot2c into a per-tile partial,
//    then into an fp32 total.
//  * Tiles entirely outside the causal / window+sink mask are never visited;
//    only tiles that straddle a mask edge are masked per element (branch-free).
//  * Block order: longest causal rows first; the G query heads of one KV head
//    are dispatched consecutively to the same XCD so they share K/V in L2.
#include "attn_tile.h"


namespace lcx {

namespace {

constexpr float kLazyTau = 8.0f;  // log2 growth allowed before rescaling O


template <int D, int NW>
struct Tile {
  static constexpr int NT = 64 * NW;          // threads per workgroup
  static constexpr int BM = 32 * NW;          // query rows per workgroup
  static constexpr int CPR = D / 8;           // 16-byte chunks per K / V row
  static constexpr int ELEMS = BN * D;        // 16-bit elements per K or V tile in LDS
  static constexpr int RPL = 1024 / (2 * D);  // rows per wave-wide LDS load (64 lanes x 16 B)
  static constexpr int LPW = BN / RPL / NW;   // such loads per wave per tile
  static constexpr int KCH = BN * CPR / NT;   // K chunks per thread (register staging)
  static constexpr int KRSTEP = NT / CPR;     // rows between a thread's chunks
  static_assert(LPW >= 1 && BN % (RPL * NW) == 0 && KCH >= 1, "tile split");
};

// LDS layout of a K or V tile: row r (key j0 + r) is 2D bytes, unpadded, with
// its 16-byte chunk c stored in slot c ^ swz(r).  The QK^T operand reads take
// one chunk of 16 consecutive rows per 16 lanes; the transposing PV operand
// reads take 4 chunks of 4 consecutive rows per 32 lanes.  Each swizzle puts
// those chunks in distinct 16-byte bank groups of the 256-byte bank line.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  return D == 128 ? ((4 * (r & 3)) ^ (2 * ((r >> 2) & 1)))
                  : ((4 * ((r >> 1) & 1)) ^ (2 * ((r >> 2) & 1)));
}

// The raw words of a lane's Q fragment (q[row][16c + 8h2 .. +7], c = 0 ..
// D/16-1) and, for q_mode 2, their rows of the cos/sin tables.  Every load is
// issued before any result is used, so the fragment costs one memory latency
// rather than one per chunk; a row past the end reads row 0 and is zeroed at
// use.
template <int D>
struct QRaw {
  u32x4 raw[D / 16];
  f32x4 cs[D / 16], sn[D / 16];
  bool valid;
  __device__ __forceinline__ void load(const AttnParams& p, const uint16_t* qbase, int64_t qi, int h2) {
    valid = qi < p.n_q;
    const int64_t r = valid ? qi : 0;
    const uint16_t* q = qbase + r * p.qs_s + 8 * h2;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) raw[c] = *reinterpret_cast<const u32x4*>(q + 16 * c);
    if (p.q_mode == 2) {
      const int64_t t = (p.q_pos0 + r - p.tab_pos0) * (D / 2) + 4 * h2;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        cs[c] = *reinterpret_cast<const f32x4*>(p.cos_tab + t + 8 * c);
        sn[c] = *reinterpret_cast<const f32x4*>(p.sin_tab + t + 8 * c);
      }
    }
  }
  __device__ __forceinline__ u32x4 word(int c) const {
    const u32x4 z = {0u, 0u, 0u, 0u};
    return valid ? raw[c] : z;
  }
};

// Q fragment for the B operand of S^T = K Q^T: lane (n, h2) holds
// q[row n][16c + 8h2 .. +7] for c = 0 .. D/16-1, rotated, scaled by
// sigma·log2(e) and rounded once to f16.
template <int D>
__device__ __forceinline__ void load_q(const AttnParams& p, const uint16_t* qbase, int64_t qi,
                                       int h2, f16x8 (&qf)[D / 16]) {
  QRaw<D> q;
  q.load(p, qbase, qi, h2);
  const float sc = p.scale_log2;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const u32x4 raw = q.word(c);
    u32x4 w;
    if (p.q_mode == 2) {
      w = rotate4_bf16<true>(raw, q.cs[c] * sc, q.sn[c] * sc);
    } else if (p.q_mode == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pack_f16x2(bf16lo(raw[i]) * sc, bf16hi(raw[i]) * sc);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pack_f16x2(f16lo(raw[i]) * sc, f16hi(raw[i]) * sc);
    }
    qf[c] = __builtin_bit_cast(f16x8, w);
  }
}


// f16 high and low parts of a pair of fp32 values: hi = f16(x), lo =
// f16(x - hi) (x - hi is exact in fp32; the f16 MFMA takes lo's subnormal
// values as they are)
struct F16Split {
  uint32_t hi, lo;
};
__device__ __forceinline__ F16Split split_f16x2(float a, float b) {
  const uint32_t hi = pack_f16x2(a, b);
  return {hi, pack_f16x2(a - f16lo(hi), b - f16hi(hi))};
}

// load_q for the precise QK^T form: the rotated, scaled q as f16 high (qh)
// and low (ql) parts
template <int D>
__device__ __forceinline__ void load_q_split(const AttnParams& p, const uint16_t* qbase, int64_t qi,
                                             int h2, f16x8 (&qh)[D / 16], f16x8 (&ql)[D / 16]) {
  QRaw<D> q;
  q.load(p, qbase, qi, h2);
  const float sc = p.scale_log2;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const u32x4 raw = q.word(c);
    float x[8];
    if (p.q_mode == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = bf16lo(raw[i]), x1 = bf16hi(raw[i]);
        x[2 * i] = (x0 * q.cs[c][i] - x1 * q.sn[c][i]) * sc;
        x[2 * i + 1] = (x0 * q.sn[c][i] + x1 * q.cs[c][i]) * sc;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = (p.q_mode == 1 ? bf16lo(raw[i]) : f16lo(raw[i])) * sc;
        x[2 * i + 1] = (p.q_mode == 1 ? bf16hi(raw[i]) : f16hi(raw[i])) * sc;
      }
    }
    u32x4 wh, wl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const F16Split sp = split_f16x2(x[2 * i], x[2 * i + 1]);
      wh[i] = sp.hi;
      wl[i] = sp.lo;
    }
    qh[c] = __builtin_bit_cast(f16x8, wh);
    ql[c] = __builtin_bit_cast(f16x8, wl);
  }
}

// Tile copy global -> LDS with no register round trip: per wave LPW buffer
// loads of 64 lanes x 16 bytes, each filling RPL consecutive LDS rows; lane L
// of load i fills row r = (wave·LPW + i)·RPL + L / CPR, slot L % CPR, with
// the row's chunk (L % CPR) ^ swz(r).  The resource starts at the tile's first
// key and ends at the last key, so rows past the end land as zeros.
template <int D, int NW, bool K_SWZ, bool STREAM = false>
struct LdsCopy {
  using T = Tile<D, NW>;
  const uint16_t* base;
  int64_t rs;  // row stride, elements
  int n_kv;
  int row0;    // first LDS row of this wave (wave-uniform)
  uint32_t off[T::LPW];

  __device__ __forceinline__ void init(const uint16_t* b, int64_t stride, int64_t nkv, int wave,
                                       int lane) {
    base = b;
    rs = stride;
    n_kv = (int)nkv;
    row0 = wave * T::LPW * T::RPL;
#pragma unroll
    for (int i = 0; i < T::LPW; ++i) {
      const int r = row0 + i * T::RPL + lane / T::CPR;
      const int c = (lane % T::CPR) ^ (K_SWZ ? k_swz<D>(r) : v_swz<D>(r));
      off[i] = (uint32_t)(r * rs * 2) + (uint32_t)c * 16u;
    }
  }
  __device__ __forceinline__ void issue(uint16_t* lds, int j0) const {
    const uint32_t rows = n_kv > j0 ? (uint32_t)(n_kv - j0) : 0u;  // tiles past the end: empty range
    const uint32_t rs2 = (uint32_t)(rs * 2);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(reinterpret_cast<const char*>(base) + (uint64_t)(uint32_t)j0 * rs2, rows * rs2);
#pragma unroll
    for (int i = 0; i < T::LPW; ++i) {
      const uint32_t la = (uint32_t)(uintptr_t)(lds_void*)lds + (uint32_t)((row0 + i * T::RPL) * D * 2);
      if constexpr (STREAM)
        lds_copy16_stream(r, off[i], __builtin_amdgcn_readfirstlane(la));
      else
        lds_copy16(r, off[i], __builtin_amdgcn_readfirstlane(la));
    }
  }
};

// Copy of one V tile in the 64-key tile layout (d rows of 64 keys, 128 bytes
// each; contiguous in HBM) into LDS, row r's chunk c in slot c ^ vt_swz(r):
// per wave LPW loads, lane L of load i fills row (wave·LPW + i)·8 + L / 8,
// slot L % 8.  Tiles are whole in HBM (the packer zero-fills past the last
// key), so the resource covers exactly one tile.
__device__ __forceinline__ int vt_swz(int r) { return (r >> 1) & 7; }

template <int D, int NW, bool STREAM = false>
struct LdsCopyVT {
  static constexpr int LPW = D * 128 / 1024 / NW;
  static_assert(LPW >= 1 && D * 128 == LPW * NW * 1024, "V tile split");
  const uint16_t* base;
  int row0;
  uint32_t off[LPW];

  __device__ __forceinline__ void init(const uint16_t* b, int wave, int lane) {
    base = b;
    row0 = wave * LPW * 8;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int r = row0 + i * 8 + lane / 8;
      off[i] = (uint32_t)(r * 128) + (uint32_t)(((lane % 8) ^ vt_swz(r)) * 16);
    }
  }
  __device__ __forceinline__ void issue(uint16_t* lds, int j0) const {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (int64_t)(j0 / BN) * (D * BN), D * BN * 2);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const uint32_t la = (uint32_t)(uintptr_t)(lds_void*)lds + (uint32_t)((row0 + i * 8) * BN * 2);
      if constexpr (STREAM)
        lds_copy16_stream(r, off[i], __builtin_amdgcn_readfirstlane(la));
      else
        lds_copy16(r, off[i], __builtin_amdgcn_readfirstlane(la));
    }
  }
};

// K staging through registers for K that is converted on the way (bf16 -> f16,
// or rotated from the fp32 tables): global (buffer loads) -> registers -> LDS
// in the swizzled layout above.
template <int D, int NW, int KMODE>
struct KRegStage {
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
      const int r = kr0 + i * T::KRSTEP;
      off[i] = (uint32_t)(r * rs * 2) + (uint32_t)kc * 16u;
      lds_off[i] = r * D + 8 * (kc ^ k_swz<D>(r));
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
    const uint32_t rs2 = (uint32_t)(rs * 2);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(reinterpret_cast<const char*>(base) + (uint64_t)(uint32_t)j0 * rs2, rows * rs2);
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
      else
        w = bf16_to_f16_4(reg[i]);
      *reinterpret_cast<u32x4*>(ks + lds_off[i]) = w;
    }
  }
  // precise QK^T form (KMODE 2): the rotated k as f16 high parts into ks and
  // low parts into kls (the same layout)
  __device__ __forceinline__ void store_split(uint16_t* ks, uint16_t* kls) const {
    static_assert(KMODE == 2, "the split is of the kernel's own rotation");
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
      u32x4 wh, wl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = bf16lo(reg[i][j]), x1 = bf16hi(reg[i][j]);
        const F16Split sp = split_f16x2(x0 * cs[i][j] - x1 * sn[i][j], x0 * sn[i][j] + x1 * cs[i][j]);
        wh[j] = sp.hi;
        wl[j] = sp.lo;
      }
      *reinterpret_cast<u32x4*>(ks + lds_off[i]) = wh;
      *reinterpret_cast<u32x4*>(kls + lds_off[i]) = wl;
    }
  }
};

// S^T = K·Q^T - m for NB 32-key blocks of a tile from block kb0 on: lane
// (n, h2) reads chunk 2c + h2 of K row 32(kb0 + kb) + n (koff[c] holds that
// row-in-block and swizzled chunk); the products accumulate onto `init` (-m
// of the lane's row).
template <int D, int NB = 2>
__device__ __forceinline__ void qk_tile(const uint16_t* ks, const int (&koff)[D / 16],
                                        const f16x8 (&qf)[D / 16], const f32x16& init,
                                        f32x16 (&s)[NB], int kb0 = 0) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      const f16x8 a = *reinterpret_cast<const f16x8*>(ks + (kb0 + kb) * 32 * D + koff[c]);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[c], c == 0 ? init : s[kb], 0, 0, 0);
    }
  }
  // keep four operand reads in flight ahead of the products (left to
  // itself the scheduler issues each read one product ahead and waits on it)
  pipeline_reads<(D / 16) * NB, 1, 4, 0>();
}

// qk_tile in the precise form: S^T = Kh·Qh^T + Kh·Ql^T + Kl·Qh^T - m over
// both 32-key blocks (the high and low f16 parts of k in ks and kls, of q in
// qh and ql; the lo·lo term, ~2^-22 relative, is left out)
template <int D>
__device__ __forceinline__ void qk_tile_precise(const uint16_t* ks, const uint16_t* kls, const int (&koff)[D / 16],
                                                const f16x8 (&qh)[D / 16], const f16x8 (&ql)[D / 16],
                                                const f32x16& init, f32x16 (&s)[2]) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f16x8 ah = *reinterpret_cast<const f16x8*>(ks + kb * 32 * D + koff[c]);
      const f16x8 al = *reinterpret_cast<const f16x8*>(kls + kb * 32 * D + koff[c]);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, qh[c], c == 0 ? init : s[kb], 0, 0, 0);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, ql[c], s[kb], 0, 0, 0);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, qh[c], s[kb], 0, 0, 0);
    }
  }
}

// A operand of O^T += V^T·P^T for d-block db and 16-key chunk kc.  Lane l
// (i = l % 16, group G = l / 16, h2 = l / 32) needs V[key][32db + l % 32] for
// the keys 16kc + 4h2 + {0..3} (elements 0-3) and 16kc + 8 + 4h2 + {0..3}
// (4-7): the order of the S^T accumulator rows that form the B operand.
// From the 64-key tile layout (VT) that is one 16-byte read.  From a
// row-major V tile it takes two transposing reads: lane i of a 16-lane group
// fetches 4 d-values (32db + 16(G%2) + 4(i%4) ..) of key (base + i/4) and
// the hardware hands lane i the i-th of them from the four keys; voff[db]
// holds this lane's swizzled address for kc = 0.
template <int D, bool VT>
__device__ __forceinline__ u32x4 pv_operand(const uint16_t* vt, const int (&voff)[4], int db, int kc) {
  if constexpr (VT) {
    // tile layout: row 32db + l32 holds the keys already in accumulator order,
    // so the 8 values are chunk 2kc + h2 of that row; voff[kc] is this lane's
    // swizzled address for db = 0
    return *reinterpret_cast<const u32x4*>(vt + voff[kc] + db * 32 * BN);
  } else {
    const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vt + voff[db] + kc * 16 * D));
    const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vt + voff[db] + (kc * 16 + 8) * D));
    return __builtin_bit_cast(u32x4, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

// O^T += V^T·P^T over NB 32-key blocks of a tile from block kb0 on (pf[i]
// holds 16-key chunk 2kb0 + i): f16 operands from V tiles, bf16 from V rows
template <int D, bool VT, int NB = 2>
__device__ __forceinline__ void pv_tile(const uint16_t* vs, const int (&voff)[4], const u32x4 (&pf)[2 * NB],
                                        f32x16 (&oacc)[D / 32], int kb0 = 0) {
  // key chunk outer: consecutive products go to different accumulators
#pragma unroll
  for (int kc = 0; kc < 2 * NB; ++kc)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const u32x4 a = pv_operand<D, VT>(vs, voff, db, 2 * kb0 + kc);
      if constexpr (VT)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                          __builtin_bit_cast(f16x8, pf[kc]), oacc[db], 0, 0, 0);
      else
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                           __builtin_bit_cast(bf16x8, pf[kc]), oacc[db], 0, 0, 0);
    }
  pipeline_reads<(D / 32) * 2 * NB, 1, 4, 1>();
}

// Online-softmax state and O accumulator of 32 query rows of one head.  Row n
// is held by lanes n and n + 32: they split the scores of each 32-key block
// of the S^T accumulator and the d columns of O^T.
// KEEP_NEG_M holds the QK^T accumulator's start in 16 registers across tiles;
// otherwise it is rebuilt from m_run for each tile (for kernels with no
// registers to spare).
template <int D, bool PF16, bool KEEP_NEG_M>
struct Rows32 {
  f32x16 oacc[D / 32];
  f32x16 neg_m;  // -m_use in every element (KEEP_NEG_M)
  float m_run;  // reference max, log2 units (scaled); -inf before any kept key
  float m_thr;  // a tile max (relative to m_use) above this moves m_run: kLazyTau, or -inf before any kept key
  float l_run;  // this lane's partial row sum
  int64_t qi;   // this lane's row
  int64_t qpos, qpos_min, qpos_max;
  // a tile starting at key j0 is kept whole for every row of the group iff
  // j0 <= kt_hi and (j0 >= kt_lo or j0 < kt_sink): the 64-bit position tests
  // done once, so that each tile decides with 32-bit scalar compares
  int kt_hi, kt_lo, kt_sink;

  __device__ __forceinline__ static int sat_i32(int64_t x) {
    return (int)(x > INT32_MAX ? (int64_t)INT32_MAX : (x < INT32_MIN ? (int64_t)INT32_MIN : x));
  }
  __device__ __forceinline__ void set_kept_tiles(const AttnParams& p) {
    // j0 + BN <= n_kv; causal: k_pos0 + j0 + BN - 1 <= qpos_min
    int64_t hi = p.n_kv - BN;
    if (p.causal) hi = hi < qpos_min - p.k_pos0 - (BN - 1) ? hi : qpos_min - p.k_pos0 - (BN - 1);
    kt_hi = sat_i32(hi);
    // window: k_pos0 + j0 >= qpos_max - window, or every key a sink:
    // k_pos0 + j0 + BN - 1 < n_sink
    kt_lo = p.window >= 0 ? sat_i32(qpos_max - p.window - p.k_pos0) : INT32_MIN;
    kt_sink = sat_i32((int64_t)p.n_sink - p.k_pos0 - (BN - 1));
  }

  __device__ __forceinline__ void init(const AttnParams& p, int64_t row0, int l32) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
    m_run = -INFINITY;
    m_thr = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) neg_m[r] = 0.f;
    qi = row0 + l32;
    qpos = p.q_pos0 + qi;
    const int64_t last = (row0 + 31 < p.n_q ? row0 + 31 : p.n_q - 1);
    qpos_min = p.q_pos0 + row0;
    qpos_max = p.q_pos0 + (last >= row0 ? last : row0);
    set_kept_tiles(p);
  }
  // lane row qi (>= n_q: no row) of a group whose kept positions span
  // [qpos_lo, qpos_hi]
  __device__ __forceinline__ void init_row(const AttnParams& p, int64_t row, int64_t qpos_lo,
                                           int64_t qpos_hi) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
    m_run = -INFINITY;
    m_thr = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) neg_m[r] = 0.f;
    qi = row;
    qpos = p.q_pos0 + row;
    qpos_min = qpos_lo;
    qpos_max = qpos_hi;
    set_kept_tiles(p);
  }
  // mask S(t), blocks kb0 .. kb0 + NB - 1 (only for tiles that straddle a
  // mask edge for these rows)
  template <int NB>
  __device__ __forceinline__ void mask(const AttnParams& p, f32x16 (&s)[NB], int j0, int h2, int kb0 = 0) const {
    if (!(j0 <= kt_hi && (j0 >= kt_lo || j0 < kt_sink))) {
      const int64_t kpos_min = p.k_pos0 + j0;
      // Branch-free, in 32-bit offsets within the tile: key at offset `off`
      // (position kpos_min + off) is kept iff off < krem (exists),
      // off <= hi (causal), and off >= lo (window) or off < srem (sink).
      // off = bias + c with c a constant of the unrolled loop, so every bound
      // is moved by bias once and each element compares against c (an
      // inline constant, no per-element offset registers)
      const int64_t rel = qpos - kpos_min;
      const int hi = p.causal ? clamp_i32(rel) : (1 << 30);
      const int lo = p.window >= 0 ? clamp_i32(rel - p.window) : -(1 << 30);
      const int srem = clamp_tile((int64_t)p.n_sink - kpos_min);
      const int krem = clamp_tile(p.n_kv - j0);
      const int bias = kb0 * 32 + h2 * 4;
      const int a_k = krem - bias, a_hi = hi - bias, a_lo = lo - bias, a_s = srem - bias;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
          const bool ok = (c < a_k) & (c <= a_hi) & ((c >= a_lo) | (c < a_s));
          s[kb][r] = ok ? s[kb][r] : -INFINITY;
        }
    }
  }
  // start of the QK^T accumulator: -m_use, m_use = m_run or 0 before any kept key
  __device__ __forceinline__ f32x16 qk_init() const {
    if constexpr (KEEP_NEG_M) {
      return neg_m;
    } else {
      const float nm = (m_run == -INFINITY) ? 0.f : -m_run;
      f32x16 x;
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = nm;
      return x;
    }
  }
  // max of this lane's half of a row's tile of s = S·scale·log2(e) - m_use
  // (lanes l and l^32 hold the two halves of one row's keys; m_use = m_run,
  // or 0 before any kept key)
  template <int NB>
  __device__ __forceinline__ float tile_max(const f32x16 (&s)[NB]) const {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    return mx;
  }
  // move the reference max when a row max grew by more than 2^kLazyTau, and
  // shift this tile's s to the new reference.  The tile max is relative to
  // m_use, so the test is mx > kLazyTau (mx > -inf before any kept key): one
  // compare against m_thr per tile.  Either half of a row exceeding it sends
  // the wave into the branch, where the two halves' maxima are combined (the
  // two lanes of a row must keep one reference)
  template <int NB>
  __device__ __forceinline__ void rescale(float mx_half, f32x16 (&s)[NB]) {
    if (__any(mx_half > m_thr)) {
      const float mx = xor32_max(mx_half);
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      const float m_new = fmaxf(m_run, m_use + mx);
      const float alpha = (m_run == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      const float m_next = (m_new == -INFINITY) ? 0.f : m_new;
      const float shift = m_next - m_use;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] -= shift;
      m_run = m_new;
      m_thr = (m_new == -INFINITY) ? -INFINITY : kLazyTau;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) neg_m[r] = -m_next;
    }
  }
  // P = exp2(s) packed to f16 (PF16) or bf16: the B operand of PV.  The row
  // sum adds P rounded to f16, two per v_dot2c into a per-tile partial, then
  // into the fp32 total (f16 keeps the sum of a short row within 2^-11).
  template <int NB>
  __device__ __forceinline__ void probs(const f32x16 (&s)[NB], u32x4 (&pf)[2 * NB]) {
    const f16x2 one2 = __builtin_bit_cast(f16x2, 0x3c003c00u);
    float part[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) part[kb] = 0.f;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pv[r] = __builtin_amdgcn_exp2f(s[kb][r]);
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // the dot product takes the packed word itself: read back from w, hipcc
          // (ROCm 7.2) fed element 0 to all four
          const float p0 = pv[8 * hlf + 2 * i], p1 = pv[8 * hlf + 2 * i + 1];
          const uint32_t wh = pack_f16x2(p0, p1);
          part[kb] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, wh), one2, part[kb], false);
          w[i] = PF16 ? wh : pack_bf16x2(p0, p1);
        }
        pf[kb * 2 + hlf] = w;
      }
    }
    if constexpr (NB == 2)
      l_run += part[0] + part[1];
    else
      l_run += part[0];
  }
  // epilogue: O = O_acc / l, LSE = ln 2 · (m + log2 l); o_mode 2 merges into
  // the existing (O, LSE) partial
  __device__ __forceinline__ void store(const AttnParams& p, int b, int hq, int h2) const {
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
        wa = 0.f;
        wb = 1.f;
        lse_m = lse_new;
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
};

// per-lane LDS read offsets of the QK^T (K) and PV (V) operands
template <int D, bool VT>
__device__ __forceinline__ void operand_offsets(int lane, int (&koff)[D / 16], int (&voff)[4]) {
  const int l32 = lane & 31, h2 = lane >> 5;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) koff[c] = l32 * D + 8 * ((2 * c + h2) ^ k_swz<D>(l32));
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = 0;
  if constexpr (VT) {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) voff[kc] = l32 * BN + 8 * ((2 * kc + h2) ^ vt_swz(l32));
  } else {
    const int i = lane & 15, gg = (lane >> 4) & 1;
    const int r = 4 * h2 + (i >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      voff[db] = r * D + 8 * ((4 * db + 2 * gg + ((i & 3) >> 1)) ^ v_swz<D>(r)) + 4 * (i & 1);
  }
}

template <int D, int KMODE, int NW, bool VT, bool PRECISE = false>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_fwd_kernel(const AttnParams p) {
  static_assert(!PRECISE || KMODE == 2, "the precise QK^T form splits the kernel's own rotation of k");
  using T = Tile<D, NW>;
  // Stages of (K, V) tiles in LDS, one array each so that every unrolled step
  // names its stages directly.  Pre-rotated f16 K and V are copied straight
  // to LDS, three stages deep; K converted on the way goes through registers,
  // two stages.
  constexpr int NST = KMODE == 0 ? 3 : 2;
  constexpr int E3 = NST > 2 ? T::ELEMS : 8;
  __shared__ __attribute__((aligned(1024))) uint16_t k_st0[T::ELEMS], k_st1[T::ELEMS], k_st2[E3];
  __shared__ __attribute__((aligned(1024))) uint16_t v_st0[T::ELEMS], v_st1[T::ELEMS], v_st2[E3];
  // low parts of K (precise QK^T form)
  constexpr int EL = PRECISE ? T::ELEMS : 8;
  __shared__ __attribute__((aligned(1024))) uint16_t kl_st0[EL], kl_st1[EL];

  __shared__ int unit_slot;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  const int unit = workgroup_unit(p.sched, &unit_slot);
  if (unit < 0) return;
  // a workgroup holds p.hpb query heads of one KV head, NW / p.hpb waves of
  // 32 rows each per head, so its waves cover the same positions and the
  // tile range they share is the one each of them needs
  const BlockTiles bt = block_tiles(p, unit, T::BM / p.hpb, p.hpb);
  const int wph = NW / p.hpb;
  const int hq = bt.hq + wave / wph;
  const int64_t wrow0 = bt.row0 + 32 * (wave % wph);
  const int ntl = bt.ntl;
  const uint16_t* qbase = p.q + bt.b * p.qs_b + hq * p.qs_h;
  const uint16_t* kbase = p.k + bt.b * p.ks_b + bt.hkv * p.ks_h;
  const uint16_t* vbase = p.v + bt.b * p.vs_b + bt.hkv * p.vs_h;

  // the d = 128 kernels that stage K through registers or read V rows have
  // no 16 registers to spare
  Rows32<D, VT, D == 64 || (KMODE == 0 && VT)> rows;
  rows.init(p, wrow0, l32);
  // Q fragment (RoPE fused into its load when q_mode == 2) and its low part
  // in the precise form; loaded below, once the first tiles are in flight
  f16x8 qf[D / 16], qlo[PRECISE ? D / 16 : 1];

  // ---- staging and per-lane LDS read offsets
  LdsCopy<D, NW, true> kcp;
  LdsCopy<D, NW, false> vcp;
  LdsCopyVT<D, NW> vtcp;
  KRegStage<D, NW, KMODE == 0 ? 1 : KMODE> kreg;
  if constexpr (KMODE == 0)
    kcp.init(kbase, p.ks_s, p.n_kv, wave, lane);
  else
    kreg.init(p, kbase, tid);
  if constexpr (VT)
    vtcp.init(vbase, wave, lane);
  else
    vcp.init(vbase, p.vs_s, p.n_kv, wave, lane);
  int koff[D / 16], voff[4];
  operand_offsets<D, VT>(lane, koff, voff);

  // ---- the tile loop: each step waits for its own copies of tile t + 1,
  // then meets the other waves (after which stage t % NST may be
  // overwritten); unrolled NST times so that every step names its stage
  // arrays directly
  constexpr int kLoadsPerTile = KMODE == 0 ? 2 * T::LPW : T::LPW;  // vector memory ops per wave
  auto issue = [&](uint16_t* ks, uint16_t* vs, int t) {
    const int j0 = bt.j0(t);
    if constexpr (KMODE == 0) kcp.issue(ks, j0);
    if constexpr (VT)
      vtcp.issue(vs, j0);
    else
      vcp.issue(vs, j0);
  };
  // kls, kls_next: the low parts of K (precise form, two stages)
  auto step = [&](const uint16_t* ks, const uint16_t* vs, uint16_t* ks_next, uint16_t* vs_next,
                  const uint16_t* kls, uint16_t* kls_next, int t) {
    const int tn = t + NST - 1;
    const bool pre = tn < ntl;
    if constexpr (KMODE != 0) {
      if (pre) {
        kreg.load(bt.j0(tn));
        issue(ks_next, vs_next, tn);
      }
    }
    f32x16 s_cur[2];
    if constexpr (PRECISE)
      qk_tile_precise<D>(ks, kls, koff, qf, qlo, rows.qk_init(), s_cur);
    else
      qk_tile<D>(ks, koff, qf, rows.qk_init(), s_cur);
    // copies straight to LDS are issued after the QK^T products, so that the
    // first operand reads follow the barrier without the copies' scalar work
    // in front of them
    if constexpr (KMODE == 0) {
      if (pre) issue(ks_next, vs_next, tn);
    }
    rows.mask(p, s_cur, bt.j0(t), h2);
    rows.rescale(rows.tile_max(s_cur), s_cur);
    u32x4 pf[4];
    rows.probs(s_cur, pf);
    pv_tile<D, VT>(vs, voff, pf, rows.oacc);
    if constexpr (PRECISE) {
      if (pre) kreg.store_split(ks_next, kls_next);
    } else if constexpr (KMODE != 0) {
      if (pre) kreg.store(ks_next);
    }
    if (NST > 2 && pre)
      stage_barrier<kLoadsPerTile>();
    else
      stage_barrier<0>();
  };

  if (ntl > 0) {
    if constexpr (KMODE != 0) kreg.load(bt.j0(0));
    issue(k_st0, v_st0, 0);
  }
  if (NST > 2 && ntl > 1) issue(k_st1, v_st1, 1);
  if constexpr (PRECISE)
    load_q_split<D>(p, qbase, rows.qi, h2, qf, qlo);
  else
    load_q<D>(p, qbase, rows.qi, h2, qf);
  if constexpr (KMODE != 0) {
    if (ntl > 0) {
      if constexpr (PRECISE)
        kreg.store_split(k_st0, kl_st0);
      else
        kreg.store(k_st0);
    }
  }
  // draining here costs one memory latency per workgroup and gives the loop
  // a single entry state
  stage_barrier<0>();
  for (int t = 0; t < ntl; t += NST) {
    if constexpr (NST > 2) {
      step(k_st0, v_st0, k_st2, v_st2, kl_st0, kl_st1, t);
      if (t + 1 >= ntl) break;
      step(k_st1, v_st1, k_st0, v_st0, kl_st0, kl_st1, t + 1);
      if (t + 2 >= ntl) break;
      step(k_st2, v_st2, k_st1, v_st1, kl_st0, kl_st1, t + 2);
    } else {
      step(k_st0, v_st0, k_st1, v_st1, kl_st0, kl_st1, t);
      if (t + 1 >= ntl) break;
      step(k_st1, v_st1, k_st0, v_st0, kl_st1, kl_st0, t + 1);
    }
  }

  rows.store(p, bt.b, hq, h2);
}

// Decode: n_q <= 8 new query rows (positions q_pos0 ..) of all G query heads
// of one KV head against a long pre-rotated f16 K cache, the visited KV tiles
// divided among n_splits workgroups per KV head (split-KV).  Waves pair up on
// 32 rows: row rho = 32·(wave / 2) + lane % 32 is head g = rho / n_q,
// position r = rho % n_q, so one K/V tile read from HBM serves every head of
// the group, and the two waves of a pair take the two 32-key halves of each
// tile (half the per-tile latency on the computing waves), each with its own
// running (m, l, O), merged through LDS at the end.  Only the pairs that own
// rows (ceil(G·n_q / 32) <= NW / 2) compute; all NW waves share the copies.
// The step is HBM-bound with little compute per tile, so NST LDS stages keep
// NST - 1 tiles in flight per workgroup (Little's law: the bytes in flight
// must cover the memory latency).  Each workgroup writes an fp32 partial
// (O, LSE) of its tiles; decode_combine_kernel merges them by log-sum-exp.
// [CW §3 (the step's base applies to the new rows), §5.3 merge]
template <int D, int NW, bool VT, int NST>
__global__ __launch_bounds__(64 * NW) void attn_decode_kernel(const AttnParams p, const DecodeParams dp) {
  using T = Tile<D, NW>;
  __shared__ __attribute__((aligned(1024))) uint16_t k_st[NST][T::ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t v_st[NST][T::ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h2 = lane >> 5;
  const int split = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const int nq = (int)p.n_q;
  const int pair = wave >> 1, half = wave & 1;      // wave-uniform
  const bool computes = pair * 32 < p.G * nq;       // wave-uniform

  const int rho = pair * 32 + l32;
  const bool valid = rho < p.G * nq;
  const int g = valid ? rho / nq : 0;
  const int hq = hkv * p.G + g;
  Rows32<D, VT, true> rows;
  rows.init_row(p, valid ? rho - g * nq : nq, p.q_pos0, p.q_pos0 + nq - 1);
  f16x8 qf[D / 16];
  load_q<D>(p, p.q + b * p.qs_b + hq * p.qs_h, rows.qi, h2, qf);

  // this split's share of the tiles the rows visit
  BlockTiles bt;
  tile_range(p, p.q_pos0, p.q_pos0 + nq - 1, bt);
  const int t_begin = (int)((int64_t)split * bt.ntl / dp.n_splits);
  const int ntl = (int)((int64_t)(split + 1) * bt.ntl / dp.n_splits) - t_begin;
  auto j0_of = [&](int t) { return bt.j0(t_begin + t); };

  // the cache is read once per step: streaming copies
  LdsCopy<D, NW, true, true> kcp;
  LdsCopy<D, NW, false, true> vcp;
  LdsCopyVT<D, NW, true> vtcp;
  kcp.init(p.k + b * p.ks_b + hkv * p.ks_h, p.ks_s, p.n_kv, wave, lane);
  if constexpr (VT)
    vtcp.init(p.v + b * p.vs_b + hkv * p.vs_h, wave, lane);
  else
    vcp.init(p.v + b * p.vs_b + hkv * p.vs_h, p.vs_s, p.n_kv, wave, lane);
  int koff[D / 16], voff[4];
  operand_offsets<D, VT>(lane, koff, voff);

  constexpr int kLoads = 2 * T::LPW;  // vector memory ops per wave per tile
  static_assert(kLoads * (NST - 1) <= 63, "outstanding copies must fit vmcnt");
  auto issue = [&](uint16_t* ks, uint16_t* vs, int t) {
    const int j0 = j0_of(t);
    kcp.issue(ks, j0);
    if constexpr (VT)
      vtcp.issue(vs, j0);
    else
      vcp.issue(vs, j0);
  };
#pragma unroll
  for (int i = 0; i < NST - 1; ++i)
    if (i < ntl) issue(k_st[i], v_st[i], i);
  stage_barrier<0>();
  int cur = 0;
  for (int t = 0; t < ntl; ++t) {
    // tile t is in stage t % NST; tile t + NST - 1 goes to the stage tile t - 1 used
    const int nxt = cur == 0 ? NST - 1 : cur - 1;
    const bool pre = t + NST - 1 < ntl;
    if (pre) issue(k_st[nxt], v_st[nxt], t + NST - 1);
    if (computes) {
      const uint16_t* ks = k_st[cur];
      const uint16_t* vs = v_st[cur];
      f32x16 s_cur[1];
      qk_tile<D, 1>(ks, koff, qf, rows.qk_init(), s_cur, half);
      rows.mask(p, s_cur, j0_of(t), h2, half);
      rows.rescale(rows.tile_max(s_cur), s_cur);
      u32x4 pf[2];
      rows.probs(s_cur, pf);
      pv_tile<D, VT, 1>(vs, voff, pf, rows.oacc, half);
    }
    // tile t + 1 landed (the NST - 2 newer tiles may still be in flight)
    if (pre)
      stage_barrier<kLoads * (NST - 2)>();
    else
      stage_barrier<0>();
    cur = cur == NST - 1 ? 0 : cur + 1;
  }

  // The second wave of each pair hands its state to the first through LDS:
  // every copy has landed and every wave has passed the last barrier, so the
  // stages are free.  Per lane: the O slice, m, l (XS floats).
  constexpr int XS = (D / 32) * 16 + 2;
  static_assert(NW / 2 * 64 * XS * 4 <= NST * T::ELEMS * 2, "exchange fits the K stages");
  float* xbuf = reinterpret_cast<float*>(&k_st[0][0]) + (pair * 64 + lane) * XS;
  if (computes && half == 1) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) xbuf[i * 16 + r] = rows.oacc[i][r];
    xbuf[XS - 2] = rows.m_run;
    xbuf[XS - 1] = rows.l_run;
  }
  __syncthreads();
  if (!computes || half == 1) return;
  {
    // merge by the two reference maxima (exact: O and l scale alike)
    const float ma = rows.m_run, mb = xbuf[XS - 2];
    const float m = fmaxf(ma, mb);
    const float fa = (ma == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ma - m);
    const float fb = (mb == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mb - m);
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) rows.oacc[i][r] = rows.oacc[i][r] * fa + xbuf[i * 16 + r] * fb;
    rows.l_run = rows.l_run * fa + xbuf[XS - 1] * fb;
    rows.m_run = m;
  }

  // this split's partial, fp32 [B][Hq][n_q][d] and [B][Hq][n_q]
  AttnParams pp = p;
  const int64_t rows_all = (int64_t)p.B * p.Hq * nq;
  pp.o = dp.o_part + split * rows_all * D;
  pp.lse = dp.lse_part + split * rows_all;
  pp.os_b = (int64_t)p.Hq * nq * D;
  pp.os_h = (int64_t)nq * D;
  pp.os_s = D;
  pp.ls_b = (int64_t)p.Hq * nq;
  pp.ls_h = nq;
  pp.o_mode = 1;
  rows.store(pp, b, hq, h2);
}

// Explicit instantiations: with only the implicit ones from launch_dn, the
// host pass emitted the launch stub of the first k_mode of each head size
// and left the others undefined (the library then fails to load).
#define LCX_ATTN_INST(D, NW)                                                       \
  template __global__ void attn_fwd_kernel<D, 0, NW, false>(const AttnParams);    \
  template __global__ void attn_fwd_kernel<D, 1, NW, false>(const AttnParams);    \
  template __global__ void attn_fwd_kernel<D, 2, NW, false>(const AttnParams);    \
  template __global__ void attn_fwd_kernel<D, 0, NW, true>(const AttnParams);     \
  template __global__ void attn_fwd_kernel<D, 1, NW, true>(const AttnParams);     \
  template __global__ void attn_fwd_kernel<D, 2, NW, true>(const AttnParams);     \
  template __global__ void attn_fwd_kernel<D, 2, NW, false, true>(const AttnParams); \
  template __global__ void attn_fwd_kernel<D, 2, NW, true, true>(const AttnParams);
LCX_ATTN_INST(64, kNWd64)
LCX_ATTN_INST(128, kNWd128)
#undef LCX_ATTN_INST
// decode: 4 waves (the copies' vector memory ops split four ways), NST stages
constexpr int kDecNW = 4;
constexpr int kDecNST128 = 5;  // 5 x 32 KB = all 160 KB of LDS: one workgroup per CU, 4 tiles in flight
constexpr int kDecNST64 = 4;   // 4 x 16 KB: two workgroups per CU
template __global__ void attn_decode_kernel<64, kDecNW, false, kDecNST64>(const AttnParams, const DecodeParams);
template __global__ void attn_decode_kernel<64, kDecNW, true, kDecNST64>(const AttnParams, const DecodeParams);
template __global__ void attn_decode_kernel<128, kDecNW, false, kDecNST128>(const AttnParams, const DecodeParams);
template __global__ void attn_decode_kernel<128, kDecNW, true, kDecNST128>(const AttnParams, const DecodeParams);

template <class K>
hipError_t launch_one(K kernel, const AttnParams& p, hipStream_t s, int64_t units, int block) {
  if (p.sched) launch_sched_init(p.sched, units, s);
  hipLaunchKernelGGL(kernel, dim3((unsigned)sched_grid(units, p.sched != nullptr)), dim3(block), 0, s, p);
  return hipGetLastError();
}

template <int D, int NW, bool VT>
hipError_t launch_dv(const AttnParams& p, hipStream_t s, int64_t units) {
  const int block = 64 * NW;
  switch (p.k_mode) {
    case 0: return launch_one(attn_fwd_kernel<D, 0, NW, VT>, p, s, units, block);
    case 1: return launch_one(attn_fwd_kernel<D, 1, NW, VT>, p, s, units, block);
    default:
      if (p.precise_qk) return launch_one(attn_fwd_kernel<D, 2, NW, VT, true>, p, s, units, block);
      return launch_one(attn_fwd_kernel<D, 2, NW, VT>, p, s, units, block);
  }
}

template <int D, int NW>
hipError_t launch_dn(const AttnParams& p, hipStream_t s, int64_t units) {
  return p.v_tiled ? launch_dv<D, NW, true>(p, s, units) : launch_dv<D, NW, false>(p, s, units);
}

}  // namespace

int attn_heads_per_block(int d, int G) {
  const int nw = d == 64 ? kNWd64 : kNWd128;
  int h = 1;
  while (h < nw && G % (2 * h) == 0) h *= 2;
  return h;
}

int64_t attn_fwd_blocks(int d, int B, int Hkv, int G, int64_t n_q) {
  const int hpb = attn_heads_per_block(d, G);
  const int span = 32 * (d == 64 ? kNWd64 : kNWd128) / hpb;
  return (int64_t)B * Hkv * (G / hpb) * ((n_q + span - 1) / span);
}

int64_t sched_grid(int64_t units, bool dynamic) {
  // with the dynamic order, an eighth more workgroups than units (a multiple
  // of 8, so every XCD gets as many): an XCD can take up to that share of
  // extra units from slower ones, and spare workgroups exit at once
  return dynamic ? units + ((units + 63) / 64) * 8 : units;
}

// the queue words before a launch with a sched buffer: (h, t) = (0, n_x)
__global__ void sched_init_kernel(unsigned long long* q, int64_t n_units) {
  const int x = threadIdx.x;
  if (x < 8) q[x] = (unsigned long long)((n_units - x + 7) / 8) << 32;
}

void launch_sched_init(unsigned long long* sched, int64_t units, hipStream_t s) {
  hipLaunchKernelGGL(sched_init_kernel, dim3(1), dim3(64), 0, s, sched, units);
}

hipError_t launch_attn_decode(const AttnParams& p, const DecodeParams& dp, hipStream_t s) {
  const dim3 grid((unsigned)dp.n_splits, (unsigned)p.Hkv, (unsigned)p.B), block(64 * kDecNW);
  if (p.d == 64) {
    if (p.v_tiled)
      hipLaunchKernelGGL((attn_decode_kernel<64, kDecNW, true, kDecNST64>), grid, block, 0, s, p, dp);
    else
      hipLaunchKernelGGL((attn_decode_kernel<64, kDecNW, false, kDecNST64>), grid, block, 0, s, p, dp);
  } else {
    if (p.v_tiled)
      hipLaunchKernelGGL((attn_decode_kernel<128, kDecNW, true, kDecNST128>), grid, block, 0, s, p, dp);
    else
      hipLaunchKernelGGL((attn_decode_kernel<128, kDecNW, false, kDecNST128>), grid, block, 0, s, p, dp);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const AttnParams& p_in, hipStream_t s) {
  AttnParams p = p_in;
  p.hpb = attn_heads_per_block(p.d, p.G);
  const int span = 32 * (p.d == 64 ? kNWd64 : kNWd128) / p.hpb;
  p.n_qblk = (int32_t)((p.n_q + span - 1) / span);
  const int64_t units = (int64_t)p.B * p.Hkv * p.n_qblk;
  p.xcd_map = (units % 8 == 0) ? 1 : 0;
  const int64_t blocks = units * (p.G / p.hpb);
  if (blocks == 0) return hipSuccess;
  if (p.d == 64) return launch_dn<64, kNWd64>(p, s, blocks);
  return launch_dn<128, kNWd128>(p, s, blocks);
}

}  // namespace lcx
