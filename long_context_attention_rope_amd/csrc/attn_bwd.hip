// Backward pass of the blockwise causal GQA attention for gfx950.
//
// What it computes, for a loss L with dL/dO = dO (the exact gradient of the
// forward definition; the pages use blockwise attention for training but do
// not write its backward pass out):
//   P_ij  = exp(S_ij - LSE_i),  S_ij = sigma·<q~_i, k~_j> over kept keys
//   dV_j  = sum_i P_ij dO_i,    dP_ij = <dO_i, v_j>,   D_i = <dO_i, O_i>
//   dS_ij = P_ij (dP_ij - D_i)
//   dq~_i = sigma sum_j dS_ij k~_j,   dk~_j = sigma sum_i dS_ij q~_i
//   dq_i  = R(p_i)^T dq~_i,  dk_j = R(p_j)^T dk~_j   (optional: raw q, k)
// D_i = sum_j P_ij dP_ij equals <dO_i, O_i> since O_i = sum_j P_ij v_j.
// Sources: "上下文擴充套件（Context Extension）" FlashAttention 的分塊計算策略
// (tiles on chip, no n x n matrix in HBM: P is rebuilt per tile from the
// saved LSE) and 技術原理 (q~ = R(m) q, so the gradient turns back by R^T);
// "AI 大模型窗口上下文进化史" §4 (scaled dot-product attention);
// "上下文窗口扩展技术：从 4K 到 1M" §4.1-§4.2 (window and sink mask).
//
// Design (CDNA4, wave64), three launches:
//  * bwd_stats: per query row (LSE·log2 e, D) into an fp32 workspace.
//  * bwd_dq, query-stationary (the forward's shape): a wave keeps 32 rows'
//    q~ and dO in registers and walks the forward's 64-key tiles.
//    S^T = K·Q^T and dP^T = V·dO^T take row reads of the K and V tiles;
//    P and dS are formed in the accumulator layout, and dQ^T += K^T·dS^T
//    takes transposing reads of the same K tile.
//  * bwd_dkdv, key-stationary: a wave keeps 16 keys' k~ and v in registers
//    and walks the 64-row tiles of q~, dO and the row statistics of every
//    query head of its KV head that keeps those keys.  S = Q·K^T and
//    dP = dO·V^T take row reads; dV^T += dO^T·P and dK^T += Q^T·dS take
//    transposing reads.  The G heads of the group are summed in registers,
//    so every dk, dv row is written once (no atomics).  16 keys per wave on
//    v_mfma_f32_16x16x32_bf16 keep the stationary state at 96 registers, so
//    two waves share each SIMD (with 32 keys on 32x32x16 it took 460
//    registers, one wave per SIMD, and nothing hid its softmax and latency).
//  * The dq products are v_mfma_f32_32x32x16_bf16.  All products take bf16
//    operands with fp32 accumulation: q~ and k~ come in bf16, and P and dS
//    are rounded to bf16 (dS needs bf16's exponent range: its entries shrink
//    with the row length).
//  * Each kernel's tile swizzle serves both its row reads (one 16-byte chunk
//    of each of 16 consecutive rows per 16 lanes) and its transposing reads
//    without LDS bank conflicts.
//  * Tiles are copied global -> LDS with no register round trip, three
//    stages deep, one barrier per step (as in the forward).
#include "attn_tile.h"

namespace lcx {

namespace {

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

constexpr float kLog2e = 1.44269504088896340736f;

// 16-byte chunk c of tile row r sits in slot c ^ b_swz(r).  d = 128 (256-byte
// rows): 16 consecutive rows take 16 distinct slots, and the 4 rows of an
// aligned quad take 4 distinct groups of 4 slots.  d = 64 (two rows per
// 256-byte bank line): the same with the row parity as the line half.
template <int D>
__device__ __forceinline__ int b_swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Copy of the 64-row tile at rows j0 .. j0+63 of a [rows][D] bf16 matrix
// (row stride rs elements) into LDS, row r's chunk c in slot c ^ swz(r):
// per wave LPW loads, lane L of load i fills row (wave·LPW + i)·RPL + L/CPR,
// slot L % CPR.  The resource ends at the last existing row (rows past it
// land as zeros) and spans at most one tile, so any row stride below 2^25
// elements keeps offsets in 32 bits.
// Tiles of the 16-key dK/dV kernel: its transposing reads take 2 chunks of 8
// consecutive rows per 32 lanes (a wave's two halves are served in separate
// passes), so (c ^ s_swz(r)) >> 1 differs over 8 consecutive rows.  For its
// row reads (ds_read_b128, 16 rows x 4 chunks per wave) the bit of row 8
// enters slot bit 2, not bit 0 (D = 128): among the swizzles that keep the
// transposing reads clean, these are the ones the hardware's bank-conflict
// counter reads as zero for both read patterns (the counter gave 4 conflict
// cycles per row read with bit 0, and with the first form for d = 64).
template <int D>
__device__ __forceinline__ int s_swz(int r) {
  return D == 128 ? (((r & 7) << 1) ^ (((r >> 3) & 1) << 2))
                  : ((((r >> 1) & 1) << 2) ^ (((r >> 2) & 1) << 1) ^ (((r >> 3) & 1) << 2));
}

template <int D, bool S16>
__device__ __forceinline__ int tile_swz(int r) {
  return S16 ? s_swz<D>(r) : b_swz<D>(r);
}

template <int D, int NW, bool S16 = false>
struct TileCopy {
  static constexpr int CPR = D / 8;
  static constexpr int RPL = 1024 / (2 * D);
  static constexpr int LPW = BN / RPL / NW;
  static_assert(LPW >= 1 && BN == LPW * RPL * NW, "tile split");
  int64_t rs;
  int64_t n;
  int row0;
  int lane;

  __device__ __forceinline__ void init(int64_t stride, int64_t n_rows, int wave, int lane_) {
    rs = stride;
    n = n_rows;
    row0 = wave * LPW * RPL;
    lane = lane_;
  }
  // the lane offsets are recomputed per copy (a few VALU ops) rather than
  // held in registers across the step
  __device__ __forceinline__ void issue(uint16_t* lds, const uint16_t* base, int64_t j0) const {
    const int64_t left = n - j0;
    const uint32_t rows = left <= 0 ? 0u : (left >= BN ? (uint32_t)BN : (uint32_t)left);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + j0 * rs, rows * (uint32_t)(rs * 2));
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int row = row0 + i * RPL + lane / CPR;
      const uint32_t off = (uint32_t)(row * rs * 2) + (uint32_t)(((lane % CPR) ^ tile_swz<D, S16>(row)) * 16);
      const uint32_t la = (uint32_t)(uintptr_t)(lds_void*)(lds + (row0 + i * RPL) * D);
      lds_copy16(r, off, __builtin_amdgcn_readfirstlane(la));
    }
  }
};

// Row statistics of a 64-row tile copied by one wave: 64 rows x 8 bytes,
// lanes 0-31 in range (lanes past the last row land as zeros); row r at
// float offset 2r.
struct StatsCopy1 {
  static constexpr int FLOATS = 256;  // LDS floats per stage (64 lanes x 16 B)
  __device__ static __forceinline__ void issue(float* lds, const float* rows_base, int64_t n_rows,
                                               int64_t j0, int lane) {
    const int64_t left = n_rows - j0;
    const uint32_t rows = left <= 0 ? 0u : (left >= BN ? (uint32_t)BN : (uint32_t)left);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(rows_base + 2 * j0, rows * 8u);
    const uint32_t la = (uint32_t)(uintptr_t)(lds_void*)lds;
    lds_copy16(r, (uint32_t)lane * 16u, __builtin_amdgcn_readfirstlane(la));
  }
};

// Per-lane LDS offsets (elements) into a swizzled tile.  Row reads (A operand
// of a product over d): lane (m, h) takes chunk 2c + h of row 32rb + m, at
// roff[c] + rb·32·D.  Transposing reads (A operand of a product over the tile
// rows, d-block db, 16-row slice kc): lane (i = l % 16, gg = (l / 16) % 2, h)
// fetches 4 d-values of row 16kc + 4h + i/4 (first read) and of the row 8
// below (second read); the hardware hands lane i element i % 4 of the four
// rows, so the operand holds column 32db + l % 32 of rows 16kc + 4h + {0..3}
// and 16kc + 8 + 4h + {0..3}: the row order of the accumulator that forms the
// B operand.
template <int D>
struct TileOffsets {
  int roff[D / 16];
  int toff[2][D / 32];
  __device__ __forceinline__ void init(int lane) {
    const int m = lane & 31, h = lane >> 5;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) roff[c] = m * D + 8 * ((2 * c + h) ^ b_swz<D>(m));
    const int i = lane & 15, gg = (lane >> 4) & 1;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int r = 4 * h + (i >> 2) + 8 * hf;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        toff[hf][db] = r * D + 8 * ((4 * db + 2 * gg + ((i & 3) >> 1)) ^ b_swz<D>(r)) + 4 * (i & 1);
    }
  }
  __device__ __forceinline__ bf16x8 row_op(const uint16_t* t, int rb, int c) const {
    return *reinterpret_cast<const bf16x8*>(t + rb * 32 * D + roff[c]);
  }
  __device__ __forceinline__ bf16x8 tr_op(const uint16_t* t, int db, int kc) const {
    const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + toff[0][db] + kc * 16 * D));
    const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + toff[1][db] + kc * 16 * D));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// Stationary fragment of 32 rows of a [rows][D] bf16 matrix for the B
// operand of a product over d: lane (n, h) holds row n's elements
// 16c + 8h .. +7 (zeros for a row that does not exist).
template <int D>
__device__ __forceinline__ void load_frag(const uint16_t* base, int64_t row, bool valid, int64_t rs,
                                          int h, bf16x8 (&f)[D / 16]) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (valid) raw = *reinterpret_cast<const u32x4*>(base + row * rs + 16 * c + 8 * h);
    f[c] = __builtin_bit_cast(bf16x8, raw);
  }
}

// bf16 B operands of the two 16-element slices of a 32x32 accumulator
// (slice k = registers 8k .. 8k+7)
__device__ __forceinline__ void pack_half(const f32x16& x, bf16x8 (&f)[2]) {
#pragma unroll
  for (int hlf = 0; hlf < 2; ++hlf) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[8 * hlf + 2 * i], x[8 * hlf + 2 * i + 1]);
    f[hlf] = __builtin_bit_cast(bf16x8, w);
  }
}

// Scale by sigma (dq, dk only), turn back by R(pos)^T when unrotating, and
// store 4 consecutive d-values (two rotation pairs) of one row.
__device__ __forceinline__ void store4(const BwdParams& p, void* dst, int64_t pos, int d0, f32x4 x,
                                       bool rotate) {
  if (rotate) {
    const int64_t trow = pos - p.tab_pos0;
    const f32x2 c = *reinterpret_cast<const f32x2*>(p.cos_tab + trow * (p.d / 2) + d0 / 2);
    const f32x2 s = *reinterpret_cast<const f32x2*>(p.sin_tab + trow * (p.d / 2) + d0 / 2);
    const f32x4 y = {x[0] * c[0] + x[1] * s[0], x[1] * c[0] - x[0] * s[0],
                     x[2] * c[1] + x[3] * s[1], x[3] * c[1] - x[2] * s[1]};
    x = y;
  }
  if (p.grad_f32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + d0) = x;
  } else {
    const u32x2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(dst) + d0) = w;
  }
}

// ---------------------------------------------------------------- row statistics

template <int D>
__global__ __launch_bounds__(256) void bwd_stats_kernel(const BwdParams p) {
  constexpr int LPR = D / 8;       // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;   // rows per workgroup
  const int tid = threadIdx.x;
  const int64_t nrows = (int64_t)p.B * p.Hq * p.n_q;
  const int64_t grow = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int c0 = (tid % LPR) * 8;
  float acc = 0.f, lse = 0.f;
  if (grow < nrows) {
    const int64_t i = grow % p.n_q;
    const int64_t bh = grow / p.n_q;
    const int64_t h = bh % p.Hq, b = bh / p.Hq;
    const u32x4 g = *reinterpret_cast<const u32x4*>(p.dout + b * p.dos_b + h * p.dos_h + i * p.dos_s + c0);
    float gv[8], ov[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gv[2 * e] = bf16lo(g[e]);
      gv[2 * e + 1] = bf16hi(g[e]);
    }
    if (p.o_f32) {
      const float* op = static_cast<const float*>(p.o) + b * p.os_b + h * p.os_h + i * p.os_s + c0;
      const f32x4 a = *reinterpret_cast<const f32x4*>(op);
      const f32x4 c = *reinterpret_cast<const f32x4*>(op + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ov[e] = a[e];
        ov[4 + e] = c[e];
      }
    } else {
      const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.o) + b * p.os_b +
                                                      h * p.os_h + i * p.os_s + c0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ov[2 * e] = bf16lo(w[e]);
        ov[2 * e + 1] = bf16hi(w[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(gv[e], ov[e], acc);
    lse = p.lse[b * p.ls_b + h * p.ls_h + i];
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m);
  if (grow < nrows && tid % LPR == 0) {
    // an empty row (LSE = -inf) gets +inf, so that every P of it is 0
    const f32x2 st = {lse == -INFINITY ? INFINITY : lse * kLog2e, acc};
    *reinterpret_cast<f32x2*>(p.stats + 2 * grow) = st;
  }
}

// ---------------------------------------------------------------- dq

// Tile starts j0 whose 64 keys every row of a wave (positions [qpos_min,
// qpos_max]) keeps: j0 <= hi and (j0 >= lo or j0 < sink).  The 64-bit
// position tests run once per wave, saturated to the int32 range (which keeps
// every outcome for tile starts in [0, 2^31 - 1)), so that each tile decides
// with 32-bit scalar compares.
struct KeptTiles {
  int hi, lo, sink;
  __device__ __forceinline__ static int sat(int64_t x) {
    return (int)(x > INT32_MAX ? (int64_t)INT32_MAX : (x < INT32_MIN ? (int64_t)INT32_MIN : x));
  }
  __device__ __forceinline__ void init(const BwdParams& p, int64_t qpos_min, int64_t qpos_max) {
    // j0 + BN <= n_kv; causal: k_pos0 + j0 + BN - 1 <= qpos_min
    int64_t h = p.n_kv - BN;
    if (p.causal) h = h < qpos_min - p.k_pos0 - (BN - 1) ? h : qpos_min - p.k_pos0 - (BN - 1);
    hi = sat(h);
    // window: k_pos0 + j0 >= qpos_max - window, or every key a sink
    lo = p.window >= 0 ? sat(qpos_max - p.window - p.k_pos0) : INT32_MIN;
    sink = sat((int64_t)p.n_sink - p.k_pos0 - (BN - 1));
  }
  __device__ __forceinline__ bool whole(int j0) const { return j0 <= hi && (j0 >= lo || j0 < sink); }
};

// Key mask of half kb of a 64-key tile for the lane's query row (S^T
// accumulator layout: register r is key kb·32 + (r/4)·8 + 4h + r%4); tiles
// that every row of the wave keeps whole are left alone.  The lane's key
// offset is bias + c with c a constant of the unrolled loop: the bounds are
// shifted by bias once and each element compares against an inline constant.
__device__ __forceinline__ void mask_keys(const BwdParams& p, f32x16& s, int j0, int kb, int64_t qpos,
                                          const KeptTiles& kt, int h) {
  if (kt.whole(j0)) return;
  const int64_t kpos_min = p.k_pos0 + j0;
  const int64_t rel = qpos - kpos_min;
  const int hi = p.causal ? clamp_i32(rel) : (1 << 30);
  const int lo = p.window >= 0 ? clamp_i32(rel - p.window) : -(1 << 30);
  const int srem = clamp_tile((int64_t)p.n_sink - kpos_min);
  const int krem = clamp_tile(p.n_kv - j0);
  const int bias = kb * 32 + h * 4;
  const int a_k = krem - bias, a_hi = hi - bias, a_lo = lo - bias, a_s = srem - bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int c = (r >> 2) * 8 + (r & 3);
    const bool ok = (c < a_k) & (c <= a_hi) & ((c >= a_lo) | (c < a_s));
    s[r] = ok ? s[r] : -INFINITY;
  }
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void bwd_dq_kernel(const BwdParams p) {
  using C = TileCopy<D, NW>;
  constexpr int TE = BN * D;
  __shared__ __attribute__((aligned(1024))) uint16_t k_st[3][TE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_st[3][TE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const BlockTiles bt = block_tiles<32 * NW>(p);
  const int ntl = bt.ntl;
  const int64_t qi = bt.row0 + 32 * wave + l32;
  const bool qvalid = qi < p.n_q;
  const int64_t qpos = p.q_pos0 + qi;
  const int64_t wlast = (bt.row0 + 32 * wave + 31 < p.n_q ? bt.row0 + 32 * wave + 31 : p.n_q - 1);
  const int64_t qpos_min = p.q_pos0 + bt.row0 + 32 * wave;
  const int64_t qpos_max = p.q_pos0 + (wlast >= bt.row0 + 32 * wave ? wlast : bt.row0 + 32 * wave);
  KeptTiles kt;
  kt.init(p, qpos_min, qpos_max);

  bf16x8 qf[D / 16], gf[D / 16];
  load_frag<D>(p.q + bt.b * p.qs_b + bt.hq * p.qs_h, qi, qvalid, p.qs_s, h, qf);
  load_frag<D>(p.dout + bt.b * p.dos_b + bt.hq * p.dos_h, qi, qvalid, p.dos_s, h, gf);
  f32x2 st = {INFINITY, 0.f};  // rows past the end: every P is 0
  if (qvalid) st = *reinterpret_cast<const f32x2*>(p.stats + 2 * (((int64_t)bt.b * p.Hq + bt.hq) * p.n_q + qi));
  const float lse2 = st[0], dsum = st[1];

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[i][r] = 0.f;

  C kcp, vcp;
  const uint16_t* kbase = p.k + bt.b * p.ks_b + bt.hkv * p.ks_h;
  const uint16_t* vbase = p.v + bt.b * p.vs_b + bt.hkv * p.vs_h;
  kcp.init(p.ks_s, p.n_kv, wave, lane);
  vcp.init(p.vs_s, p.n_kv, wave, lane);
  TileOffsets<D> to;
  to.init(lane);

  constexpr int kLoads = 2 * C::LPW;
  auto issue = [&](uint16_t* ks, uint16_t* vs, int t) {
    const int j0 = bt.j0(t);
    kcp.issue(ks, kbase, j0);
    vcp.issue(vs, vbase, j0);
  };
  auto step = [&](const uint16_t* ks, const uint16_t* vs, uint16_t* ks_next, uint16_t* vs_next, int t) {
    const bool pre = t + 2 < ntl;
    if (pre) issue(ks_next, vs_next, t + 2);
    const int j0 = bt.j0(t);
    // two halves of 32 keys: S^T, dP^T, then dQ^T over those keys
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(to.row_op(ks, kb, c), qf[c], sc, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(to.row_op(vs, kb, c), gf[c], dp, 0, 0, 0);
      }
      mask_keys(p, sc, j0, kb, qpos, kt, h);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], p.scale_log2, -lse2));
        sc[r] = pr * (dp[r] - dsum);
      }
      bf16x8 dsf[2];
      pack_half(sc, dsf);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
          dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(to.tr_op(ks, db, 2 * kb + k2), dsf[k2], dqacc[db],
                                                              0, 0, 0);
    }
    if (pre)
      stage_barrier<kLoads>();
    else
      stage_barrier<0>();
  };

  if (ntl > 0) issue(k_st[0], v_st[0], 0);
  if (ntl > 1) issue(k_st[1], v_st[1], 1);
  stage_barrier<0>();
  // tile t is in stage t % 3; tile t + 2 goes to stage (t + 2) % 3
  int cur = 0, nxt = 2;
  for (int t = 0; t < ntl; ++t) {
    step(k_st[cur], v_st[cur], k_st[nxt], v_st[nxt], t);
    cur = cur == 2 ? 0 : cur + 1;
    nxt = nxt == 2 ? 0 : nxt + 1;
  }

  if (!qvalid) return;
  void* dst = p.grad_f32
                  ? (void*)(static_cast<float*>(p.dq) + bt.b * p.dqs_b + bt.hq * p.dqs_h + qi * p.dqs_s)
                  : (void*)(static_cast<uint16_t*>(p.dq) + bt.b * p.dqs_b + bt.hq * p.dqs_h + qi * p.dqs_s);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 x = {dqacc[db][4 * r4] * p.scale, dqacc[db][4 * r4 + 1] * p.scale,
                       dqacc[db][4 * r4 + 2] * p.scale, dqacc[db][4 * r4 + 3] * p.scale};
      store4(p, dst, qpos, db * 32 + r4 * 8 + h * 4, x, p.unrotate != 0);
    }
}

// ---------------------------------------------------------------- dk, dv

// The key block of a workgroup: 32·NW keys of one (batch, KV head), and the
// 64-row tiles [t_lo, t_hi) of query rows that keep any of them.  Blocks run
// from the first keys (the most causal rows) on; with B·Hkv a multiple of 8,
// block id mod 8 (the XCD) fixes the KV head, so the workgroups of one XCD
// stream the same q~ / dO tiles through its L2.
struct KeyBlock {
  int b, hkv;
  int64_t key0;
  int t_lo, t_hi;
};

template <int KB>
__device__ __forceinline__ KeyBlock key_block(const BwdParams& p) {
  KeyBlock kb;
  const int bh = (int)(blockIdx.x % (unsigned)(p.B * p.Hkv));
  const int64_t blk = blockIdx.x / (unsigned)(p.B * p.Hkv);
  kb.hkv = bh % p.Hkv;
  kb.b = bh / p.Hkv;
  kb.key0 = blk * KB;
  const int64_t klast = (kb.key0 + KB < p.n_kv ? kb.key0 + KB : p.n_kv) - 1;
  const int64_t kpos_lo = p.k_pos0 + kb.key0, kpos_hi = p.k_pos0 + klast;
  int64_t r_lo = 0, r_hi = p.n_q;
  if (p.causal && kpos_lo - p.q_pos0 > r_lo) r_lo = kpos_lo - p.q_pos0;
  if (p.window >= 0 && kpos_lo >= (int64_t)p.n_sink) {
    const int64_t lim = kpos_hi + p.window - p.q_pos0 + 1;
    if (lim < r_hi) r_hi = lim;
  }
  if (r_hi <= r_lo) {
    kb.t_lo = kb.t_hi = 0;
  } else {
    kb.t_lo = (int)(r_lo / BN);
    kb.t_hi = (int)((r_hi + BN - 1) / BN);
  }
  return kb;
}

// dK, dV on v_mfma_f32_16x16x32_bf16 with 16 keys per wave: the stationary
// state (k~, v fragments and the dK^T, dV^T accumulators) is 96 registers for
// d = 128, so two waves share each SIMD and hide each other's softmax and LDS
// latency.  Layouts (lane l, i = l % 16, g = l / 16):
//   A operand  lane holds A[i][8g .. 8g+7]
//   B operand  lane holds B[8g .. 8g+7][i]
//   C/D        register r of lane holds C[4g + r][i]
// S = Q·K^T per 16-row block rb: A = q~ rows (row 16rb + i, chunk 4c + g),
// B = k~ of key i; the accumulator gives key i, rows 16rb + 4g + r.  The B
// operand of dV^T += dO^T·P over the 32 rows of half kc is then registers
// 0-3 of blocks 2kc and 2kc+1: rows 32kc + 4g + {0..3} and 32kc + 16 + 4g +
// {0..3}; the A operand dO^T holds the same rows of column 16db + i, two
// transposing reads (lane j of group g reads row 32kc + 4g + j/4, and 16
// below, columns 16db + 4(j % 4) .. +3).
template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dkdv_kernel(const BwdParams p) {
  using C = TileCopy<D, NW, true>;
  constexpr int TE = BN * D;
  constexpr int SE = StatsCopy1::FLOATS;
  __shared__ __attribute__((aligned(1024))) uint16_t q_st[3][TE];
  __shared__ __attribute__((aligned(1024))) uint16_t g_st[3][TE];
  __shared__ __attribute__((aligned(1024))) float s_st[3][SE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15;
  const int g = lane >> 4;

  const KeyBlock kb = key_block<16 * NW>(p);
  const int nrt = kb.t_hi - kb.t_lo;
  const int nsteps = nrt * p.G;
  const int64_t wkey0 = kb.key0 + 16 * wave;
  const int64_t key = wkey0 + i16;
  const bool kvalid = key < p.n_kv;
  const int64_t kpos = p.k_pos0 + key;

  // B operands of S and dP: key i16's elements 32c + 8g .. +7
  bf16x8 kf[D / 32], vf[D / 32];
  {
    const uint16_t* kbase = p.k + kb.b * p.ks_b + kb.hkv * p.ks_h + key * p.ks_s;
    const uint16_t* vbase = p.v + kb.b * p.vs_b + kb.hkv * p.vs_h + key * p.vs_s;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      u32x4 rk = {0u, 0u, 0u, 0u}, rv = {0u, 0u, 0u, 0u};
      if (kvalid) {
        rk = *reinterpret_cast<const u32x4*>(kbase + 32 * c + 8 * g);
        rv = *reinterpret_cast<const u32x4*>(vbase + 32 * c + 8 * g);
      }
      kf[c] = __builtin_bit_cast(bf16x8, rk);
      vf[c] = __builtin_bit_cast(bf16x8, rv);
    }
  }
  f32x4 dkacc[D / 16], dvacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dkacc[db][r] = 0.f;
      dvacc[db][r] = 0.f;
    }

  const bool keys_whole = wkey0 + 16 <= p.n_kv;
  const int64_t wkpos_min = p.k_pos0 + wkey0, wkpos_max = wkpos_min + 15;
  const bool k_sink = kpos < (int64_t)p.n_sink;
  // row tiles (first row at query position q_pos0 + j0) whose 64 rows all
  // keep the wave's 16 keys: rt_lo <= j0 <= rt_hi, with the keys whole; the
  // 64-bit tests once per wave (saturated to int32, which keeps every outcome
  // for j0 in [0, 2^31 - 1)), 32-bit scalar compares per step
  int rt_lo, rt_hi;
  {
    int64_t h = p.n_q - BN;  // j0 + BN <= n_q
    if (p.window >= 0 && !(wkpos_max < (int64_t)p.n_sink)) {
      // q_pos0 + j0 + BN - 1 - window <= wkpos_min
      const int64_t w = wkpos_min + p.window - p.q_pos0 - (BN - 1);
      h = h < w ? h : w;
    }
    rt_hi = KeptTiles::sat(h);
    rt_lo = p.causal ? KeptTiles::sat(wkpos_max - p.q_pos0) : INT32_MIN;  // q_pos0 + j0 >= wkpos_max
  }

  // per-lane LDS offsets: row reads and the first transposing read
  int roff[D / 32], toff[D / 16];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) roff[c] = i16 * D + 8 * ((4 * c + g) ^ s_swz<D>(i16));
  {
    const int r0 = 4 * g + (i16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      toff[db] = r0 * D + 8 * ((2 * db + ((i16 & 3) >> 1)) ^ s_swz<D>(r0)) + 4 * (i16 & 1);
  }

  C qcp, gcp;
  qcp.init(p.qs_s, p.n_q, wave, lane);
  gcp.init(p.dos_s, p.n_q, wave, lane);
  auto step_rows = [&](int s) -> int64_t { return (int64_t)(kb.t_hi - 1 - s / p.G) * BN; };
  auto step_head = [&](int s) -> int { return kb.hkv * p.G + s % p.G; };
  auto issue = [&](uint16_t* qs, uint16_t* gs, float* ss, int s) {
    const int64_t j0 = step_rows(s);
    const int hq = step_head(s);
    qcp.issue(qs, p.q + kb.b * p.qs_b + hq * p.qs_h, j0);
    gcp.issue(gs, p.dout + kb.b * p.dos_b + hq * p.dos_h, j0);
    // the statistics come with wave 0's copies (one 512-byte load instead
    // of one small load per wave)
    if (wave == 0) StatsCopy1::issue(ss, p.stats + 2 * ((int64_t)kb.b * p.Hq + hq) * p.n_q, p.n_q, j0, lane);
  };
  constexpr int kLoads = 2 * C::LPW;  // vector memory ops per step (wave 0: one more)

  auto step = [&](const uint16_t* qs, const uint16_t* gs, const float* ss, uint16_t* qs_n, uint16_t* gs_n,
                  float* ss_n, int s) {
    const bool pre = s + 2 < nsteps;
    if (pre) issue(qs_n, gs_n, ss_n, s + 2);
    const int64_t j0 = step_rows(s);
    const int64_t qpos_t = p.q_pos0 + j0;
    const bool all_kept = keys_whole && (int)j0 >= rt_lo && (int)j0 <= rt_hi;
    const int hi = clamp_i32(qpos_t - kpos);  // causal: row off kept iff hi + off >= 0
    const int lo = p.window >= 0 ? clamp_i32(qpos_t - kpos - p.window) : -(1 << 30);  // lo + off <= 0
    const int rrem = clamp_tile(p.n_q - j0);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      // S, dP for row blocks 2kc, 2kc+1
      f32x4 sc[2], dp[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sc[u][r] = 0.f;
          dp[u][r] = 0.f;
        }
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int rb = 2 * kc + u;
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qs + rb * 16 * D + roff[c]);
          const bf16x8 ag = *reinterpret_cast<const bf16x8*>(gs + rb * 16 * D + roff[c]);
          sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, kf[c], sc[u], 0, 0, 0);
          dp[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, vf[c], dp[u], 0, 0, 0);
        }
      // element (u, r) is row 32kc + 16u + 4g + r of the tile and the lane's key
      if (!all_kept) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int off = 32 * kc + 16 * u + 4 * g + r;
            const bool ok = kvalid & (off < rrem) & (!p.causal | (hi + off >= 0)) & ((lo + off <= 0) | k_sink);
            sc[u][r] = ok ? sc[u][r] : -INFINITY;
          }
      }
      // P = exp2(S·sigma·log2 e - LSE·log2 e), dS = P (dP - D)
      u32x4 wp, wd;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int row = 32 * kc + 16 * u + 4 * g;
        const f32x4 ta = *reinterpret_cast<const f32x4*>(ss + 2 * row);
        const f32x4 tc = *reinterpret_cast<const f32x4*>(ss + 2 * row + 4);
        const float l2[4] = {ta[0], ta[2], tc[0], tc[2]};
        const float dd[4] = {ta[1], ta[3], tc[1], tc[3]};
        float pr[4], ds[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][r], p.scale_log2, -l2[r]));
          ds[r] = pr[r] * (dp[u][r] - dd[r]);
        }
        wp[2 * u] = pack_bf16x2(pr[0], pr[1]);
        wp[2 * u + 1] = pack_bf16x2(pr[2], pr[3]);
        wd[2 * u] = pack_bf16x2(ds[0], ds[1]);
        wd[2 * u + 1] = pack_bf16x2(ds[2], ds[3]);
      }
      const bf16x8 pf = __builtin_bit_cast(bf16x8, wp);
      const bf16x8 dsf = __builtin_bit_cast(bf16x8, wd);
      // dV^T += dO^T·P, dK^T += Q^T·dS over the half's 32 rows
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const int o0 = toff[db] + kc * 32 * D;
        const v4i16 g0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(gs + o0));
        const v4i16 g1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(gs + o0 + 16 * D));
        const v4i16 q0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(qs + o0));
        const v4i16 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(qs + o0 + 16 * D));
        const bf16x8 ga = __builtin_bit_cast(bf16x8, __builtin_shufflevector(g0, g1, 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8 qa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7));
        dvacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga, pf, dvacc[db], 0, 0, 0);
        dkacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, dsf, dkacc[db], 0, 0, 0);
      }
    }
    if (!pre)
      stage_barrier<0>();
    else if (wave == 0)
      stage_barrier<kLoads + 1>();
    else
      stage_barrier<kLoads>();
  };

  if (nsteps > 0) issue(q_st[0], g_st[0], s_st[0], 0);
  if (nsteps > 1) issue(q_st[1], g_st[1], s_st[1], 1);
  stage_barrier<0>();
  int cur = 0, nxt = 2;
  for (int s = 0; s < nsteps; ++s) {
    step(q_st[cur], g_st[cur], s_st[cur], q_st[nxt], g_st[nxt], s_st[nxt], s);
    cur = cur == 2 ? 0 : cur + 1;
    nxt = nxt == 2 ? 0 : nxt + 1;
  }

  if (!kvalid) return;
  void* dkd;
  void* dvd;
  if (p.grad_f32) {
    dkd = static_cast<float*>(p.dk) + kb.b * p.dks_b + kb.hkv * p.dks_h + key * p.dks_s;
    dvd = static_cast<float*>(p.dv) + kb.b * p.dvs_b + kb.hkv * p.dvs_h + key * p.dvs_s;
  } else {
    dkd = static_cast<uint16_t*>(p.dk) + kb.b * p.dks_b + kb.hkv * p.dks_h + key * p.dks_s;
    dvd = static_cast<uint16_t*>(p.dv) + kb.b * p.dvs_b + kb.hkv * p.dvs_h + key * p.dvs_s;
  }
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    const int d0 = db * 16 + g * 4;
    const f32x4 xk = {dkacc[db][0] * p.scale, dkacc[db][1] * p.scale, dkacc[db][2] * p.scale,
                      dkacc[db][3] * p.scale};
    store4(p, dkd, kpos, d0, xk, p.unrotate != 0);
    store4(p, dvd, kpos, d0, dvacc[db], false);
  }
}

constexpr int kBwdNWq128 = 8;  // dq kernel waves (32 rows each)
constexpr int kBwdNWq64 = 4;
constexpr int kBwdNWk = 8;     // dk/dv kernel waves (16 keys each)

template __global__ void bwd_stats_kernel<64>(const BwdParams);
template __global__ void bwd_stats_kernel<128>(const BwdParams);
template __global__ void bwd_dq_kernel<64, kBwdNWq64>(const BwdParams);
template __global__ void bwd_dq_kernel<128, kBwdNWq128>(const BwdParams);
template __global__ void bwd_dkdv_kernel<64, kBwdNWk>(const BwdParams);
template __global__ void bwd_dkdv_kernel<128, kBwdNWk>(const BwdParams);

template <int D, int NWQ>
hipError_t launch_bwd_d(const BwdParams& p_in, hipStream_t s) {
  BwdParams p = p_in;
  // row statistics
  const int64_t nrows = (int64_t)p.B * p.Hq * p.n_q;
  const int64_t rpb = 256 / (D / 8);
  if (nrows > 0) {
    hipLaunchKernelGGL((bwd_stats_kernel<D>), dim3((unsigned)((nrows + rpb - 1) / rpb)), dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // dq (every row; with no keys it writes zeros): the forward's block order
  const int bm = 32 * NWQ;
  p.n_qblk = (int32_t)((p.n_q + bm - 1) / bm);
  const int64_t units = (int64_t)p.B * p.Hkv * p.n_qblk;
  p.xcd_map = (units % 8 == 0) ? 1 : 0;
  if (units > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, NWQ>), dim3((unsigned)(units * p.G)), dim3(64 * NWQ), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // dk, dv (every key; with no rows they are zeros)
  const int64_t kblk = (p.n_kv + 16 * kBwdNWk - 1) / (16 * kBwdNWk);
  if (kblk > 0) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, kBwdNWk>), dim3((unsigned)(kblk * p.B * p.Hkv)),
                       dim3(64 * kBwdNWk), 0, s, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

int attn_bwd_rows_per_block(int d) { return 32 * (d == 64 ? kBwdNWq64 : kBwdNWq128); }
int attn_bwd_keys_per_block(int d) { return 16 * kBwdNWk; }

hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t s) {
  if (p.d == 64) return launch_bwd_d<64, kBwdNWq64>(p, s);
  return launch_bwd_d<128, kBwdNWq128>(p, s);
}

}  // namespace lcx
