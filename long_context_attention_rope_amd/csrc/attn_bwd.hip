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
//  * bwd_stats: per query row -LSE/sigma and -D into two planes of an fp32
//    workspace (plane stride B·Hq·n_q floats): the starts of the S and dP
//    accumulators in the dk/dv kernel.
//  * bwd_dq, query-stationary (the forward's shape): a wave keeps 32 rows'
//    q~ and dO in registers and walks the forward's 64-key tiles.
//    S^T = K·Q^T and dP^T = V·dO^T take row reads of the K and V tiles;
//    P and dS are formed in the accumulator layout, and dQ^T += K^T·dS^T
//    takes transposing reads of the same K tile.
//  * bwd_dkdv, key-stationary: a pair of waves keeps 32 keys' k~ and v in
//    registers and walks the 64-row tiles of q~, dO and the row statistics
//    of every query head of its KV head that keeps those keys.  Each wave
//    of the pair forms S = Q·K^T and dP = dO·V^T for half of the tile's rows
//    (row reads), and after trading one bf16 operand with its partner
//    through LDS one of them accumulates dV^T += dO^T·P, the other dK^T +=
//    Q^T·dS over all 64 rows (transposing reads).  The G heads of the group
//    are summed in registers, so every dk, dv row is written once (no
//    atomics).  Every q~ / dO operand read feeds 32 keys, half the LDS
//    traffic of 16 keys per wave, while each wave holds one 64-register
//    accumulator, so two waves still share each SIMD.
//  * All products are v_mfma_f32_32x32x16_bf16, bf16 operands with fp32
//    accumulation: q~ and k~ come in bf16, and P and dS are rounded to bf16
//    (dS needs bf16's exponent range: its entries shrink with the row
//    length).
//  * The tile swizzle serves both the row reads (one 16-byte chunk of each of
//    16 consecutive rows per 16 lanes) and the transposing reads without LDS
//    bank conflicts.
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
// (row stride rs elements) into LDS, row r's chunk c in slot c ^ b_swz(r):
// per wave LPW loads, lane L of load i fills row (wave·LPW + i)·RPL + L/CPR,
// slot L % CPR.  The resource ends at the last existing row (rows past it
// land as zeros) and spans at most one tile, so any row stride below 2^25
// elements keeps offsets in 32 bits.
template <int D, int NW>
struct TileCopy {
  static constexpr int CPR = D / 8;
  static constexpr int RPL = 1024 / (2 * D);
  static constexpr int LPW = BN / RPL / NW;
  static_assert(LPW >= 1 && BN == LPW * RPL * NW, "tile split");
  uint32_t rs2;  // row stride, bytes
  int row0;
  int lane;

  __device__ __forceinline__ void init(int64_t stride, int wave, int lane_) {
    rs2 = (uint32_t)(stride * 2);
    row0 = wave * LPW * RPL;
    lane = lane_;
  }
  // copy from the tile's first row (rows of them in range, the rest land as
  // zeros) into the stage at LDS byte address lds_addr (wave-uniform); the
  // lane offsets are recomputed per copy (a few VALU ops) rather than held
  // in registers across the step
  __device__ __forceinline__ void issue_rows(uint32_t lds_addr, const uint16_t* tile, uint32_t rows) const {
    // rows is wave-uniform; readfirstlane keeps the resource in SGPRs
    const __amdgpu_buffer_rsrc_t r = make_rsrc(tile, __builtin_amdgcn_readfirstlane(rows * rs2));
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int row = row0 + i * RPL + lane / CPR;
      const uint32_t off = (uint32_t)row * rs2 + (uint32_t)(((lane % CPR) ^ b_swz<D>(row)) * 16);
      lds_copy16(r, off, lds_addr + (uint32_t)((row0 + i * RPL) * D * 2));
    }
  }
};

// Row statistics of a 64-row tile copied by one wave, one copy per plane:
// 64 rows x 4 bytes each, lanes 0-15 in range (lanes past the last row land
// as zeros); plane 0 (-LSE/sigma) of row r at float offset r, plane 1 (-D)
// at PLANE1 + r.
struct StatsCopy1 {
  static constexpr int PLANE1 = 256;       // LDS floats per copy (64 lanes x 16 B)
  static constexpr int FLOATS = 2 * PLANE1;  // LDS floats per stage
  // from the statistics of the tile's first row (rows of them in range);
  // pstride: floats from plane 0 to plane 1
  __device__ static __forceinline__ void issue_rows(uint32_t lds_addr, const float* first, int64_t pstride,
                                                    uint32_t rows, int lane) {
    const uint32_t bytes = __builtin_amdgcn_readfirstlane(rows * 4u);
    lds_copy16(make_rsrc(first, bytes), (uint32_t)lane * 16u, lds_addr);
    lds_copy16(make_rsrc(first + pstride, bytes), (uint32_t)lane * 16u, lds_addr + PLANE1 * 4u);
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
    const u32x4 g = load_once(reinterpret_cast<const u32x4*>(p.dout + b * p.dos_b + h * p.dos_h + i * p.dos_s + c0));
    float gv[8], ov[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gv[2 * e] = bf16lo(g[e]);
      gv[2 * e + 1] = bf16hi(g[e]);
    }
    if (p.o_f32) {
      const float* op = static_cast<const float*>(p.o) + b * p.os_b + h * p.os_h + i * p.os_s + c0;
      const f32x4 a = load_once(reinterpret_cast<const f32x4*>(op));
      const f32x4 c = load_once(reinterpret_cast<const f32x4*>(op + 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ov[e] = a[e];
        ov[4 + e] = c[e];
      }
    } else {
      const u32x4 w = load_once(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.o) + b * p.os_b +
                                                               h * p.os_h + i * p.os_s + c0));
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
    // an empty row (LSE = -inf) gets -inf, so that every P of it is 0
    p.stats[grow] = lse == -INFINITY ? -INFINITY : -lse / p.scale;
    p.stats[nrows + grow] = -acc;
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
  __device__ __forceinline__ bool whole(int j0) const { return (j0 <= hi) & ((j0 >= lo) | (j0 < sink)); }
};

// Key mask of half kb of a 64-key tile for the lane's query row (S^T
// accumulator layout: register r is key kb·32 + (r/4)·8 + 4h + r%4): entries
// outside it become `fill`; the caller skips tiles that every row of the
// wave keeps whole.  The lane's key
// offset is bias + c with c a constant of the unrolled loop: the bounds are
// shifted by bias once and each element compares against an inline constant.
__device__ __forceinline__ void mask_keys(const BwdParams& p, f32x16& s, int j0, int kb, int64_t qpos, int h,
                                          float fill) {
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
    s[r] = ok ? s[r] : fill;
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

  __shared__ int unit_slot;
  const int unit = workgroup_unit(p.sched, &unit_slot);
  if (unit < 0) return;
  const BlockTiles bt = block_tiles(p, unit, 32 * NW, 1);
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
  // LSE·log2 e and D of the lane's row (rows past the end: every P is 0)
  float lse2 = INFINITY, dsum = 0.f;
  if (qvalid) {
    const int64_t row = ((int64_t)bt.b * p.Hq + bt.hq) * p.n_q + qi;
    const float ml = p.stats[row];  // -LSE/sigma, -inf for an empty row
    lse2 = ml == -INFINITY ? INFINITY : -ml * p.scale_log2;
    dsum = -p.stats[(int64_t)p.B * p.Hq * p.n_q + row];
  }

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[i][r] = 0.f;

  C kcp, vcp;
  const uint16_t* kbase = p.k + bt.b * p.ks_b + bt.hkv * p.ks_h;
  const uint16_t* vbase = p.v + bt.b * p.vs_b + bt.hkv * p.vs_h;
  kcp.init(p.ks_s, wave, lane);
  vcp.init(p.vs_s, wave, lane);
  TileOffsets<D> to;
  to.init(lane);

  constexpr int kLoads = 2 * C::LPW;
  const uint32_t lk = (uint32_t)(uintptr_t)(lds_void*)&k_st[0][0];
  const uint32_t lv = (uint32_t)(uintptr_t)(lds_void*)&v_st[0][0];
  auto issue = [&](int st, int t) {
    const int j0 = bt.j0(t);
    const int left = (int)p.n_kv - j0;  // n_kv < 2^31
    const uint32_t rows = left <= 0 ? 0u : (left >= BN ? (uint32_t)BN : (uint32_t)left);
    kcp.issue_rows(lk + (uint32_t)(st * TE * 2), kbase + (int64_t)j0 * p.ks_s, rows);
    vcp.issue_rows(lv + (uint32_t)(st * TE * 2), vbase + (int64_t)j0 * p.vs_s, rows);
  };
  auto step = [&](const uint16_t* ks, const uint16_t* vs, int nxt, int t) {
    const bool pre = t + 2 < ntl;
    const int j0 = bt.j0(t);
    const bool whole = kt.whole(j0);
    // Two halves of 32 keys in four runs of products, the order fixed by
    // scheduling barriers and each operand read issued four products ahead:
    // S^T and dP^T of half 0; those of half 1 with the softmax of half 0
    // between them; the masks (one branch: dS of half 0 -> 0, S^T of half 1
    // -> -inf); dQ^T of half 0 with the softmax of half 1 between its
    // products; dQ^T of half 1.
    f32x16 sc[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[kb][r] = 0.f;
        dp[kb][r] = 0.f;
      }
    // dS = exp2(S·sigma·log2 e - LSE·log2 e) (dP - D) of register r of half kb, in place
    auto soft = [&](int kb, int r) {
      const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], p.scale_log2, -lse2));
      sc[kb][r] = pr * (dp[kb][r] - dsum);
    };
    constexpr int NC = D / 16, NS = 2 * NC, AH = 4;
    {
      // product i of half kb: chunk i / 2, S^T (K rows) or dP^T (V rows)
      auto rd = [&](int i) { return to.row_op((i % NS) & 1 ? vs : ks, i / NS, (i % NS) >> 1); };
      bf16x8 a[2 * NS];
#pragma unroll
      for (int i = 0; i < AH; ++i) a[i] = rd(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2 * NS; ++i) {
        const int kb = i / NS, j = i % NS;
        if (j & 1)
          dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], gf[j >> 1], dp[kb], 0, 0, 0);
        else
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], qf[j >> 1], sc[kb], 0, 0, 0);
        if (i + AH < 2 * NS) a[i + AH] = rd(i + AH);
        if (kb == 1) {
#pragma unroll
          for (int r = j * 16 / NS; r < (j + 1) * 16 / NS; ++r) soft(0, r);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the copy of tile t + 2 after the first product run, so that the first
    // operand reads follow the barrier without its scalar work
    if (pre) issue(nxt, t + 2);
    if (!whole) {
      mask_keys(p, sc[0], j0, 0, qpos, h, 0.f);
      mask_keys(p, sc[1], j0, 1, qpos, h, -INFINITY);
    }
    {
      // product i: 16-key slice 2kb + i / ND of the K tile, d-block i % ND
      constexpr int ND = D / 32, NQ = 2 * ND;
      auto rd = [&](int i) { return to.tr_op(ks, (i % NQ) % ND, 2 * (i / NQ) + (i % NQ) / ND); };
      bf16x8 a[2 * NQ], dsf[2][2];
      pack_half(sc[0], dsf[0]);
#pragma unroll
      for (int i = 0; i < AH; ++i) a[i] = rd(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2 * NQ; ++i) {
        const int kb = i / NQ, j = i % NQ;
        if (i == NQ) pack_half(sc[1], dsf[1]);
        dqacc[j % ND] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], dsf[kb][j / ND], dqacc[j % ND], 0, 0, 0);
        if (i + AH < 2 * NQ) a[i + AH] = rd(i + AH);
        if (kb == 0) {
#pragma unroll
          for (int r = j * 16 / NQ; r < (j + 1) * 16 / NQ; ++r) soft(1, r);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (pre)
      stage_barrier<kLoads>();
    else
      stage_barrier<0>();
  };

  if (ntl > 0) issue(0, 0);
  if (ntl > 1) issue(1, 1);
  stage_barrier<0>();
  // tile t is in stage t % 3; tile t + 2 goes to stage (t + 2) % 3
  int cur = 0, nxt = 2;
  for (int t = 0; t < ntl; ++t) {
    step(k_st[cur], v_st[cur], nxt, t);
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
__device__ __forceinline__ KeyBlock key_block(const BwdParams& p, int unit) {
  KeyBlock kb;
  const int bh = (int)((unsigned)unit % (unsigned)(p.B * p.Hkv));
  const int64_t blk = (unsigned)unit / (unsigned)(p.B * p.Hkv);
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

// dK, dV with pairs of waves on v_mfma_f32_32x32x16_bf16: the two waves of
// pair w/2 hold the same 32 keys (k~ and v as B operands, as in dq) and
// split each 64-row step: role 0 (even wave) forms S and dP of tile rows
// 0-31, role 1 of rows 32-63.  Role 0 accumulates dV^T += dO^T·P over all
// 64 rows and role 1 dK^T += Q^T·dS, so role 0 hands its dS rows and role 1
// its P rows to the partner through LDS (2 KB per wave and step, one buffer
// per step parity).  Every q~ / dO operand read feeds 32 keys, and each
// wave's accumulator is one of dK^T, dV^T (64 registers at d = 128), so two
// waves share each SIMD.
// Layouts (32x32x16; lane l, n = l % 32, h = l / 32): A lane holds
// A[n][8h .. 8h+7], B lane holds B[8h .. 8h+7][n], register r of C holds
// C[8(r/4) + 4h + r%4][n].  S = Q·K^T: A = q~ rows of the role's half
// (TileOffsets row reads), B = k~ of key n; the accumulator gives key n,
// rows 8j + 4h + {0..3}, whose two 16-row slices are the B operands of the
// products over rows (pack_half), matched by the transposing reads of dO^T
// and q~^T (TileOffsets transposing offsets).
// A step: the S products, then the dP products with the exponentials of S
// between them (the row statistics start the accumulators); dS, the
// partner's slices into buffer s % 2, one barrier, the partner's slices read
// back and the 16 products over rows, with the copy of tile s + 2 into the
// stage of tile s - 1 (every wave finished with it before the barrier)
// issued after the last of them.  Buffer s % 2 is written again at step s + 2, after
// the barrier of step s + 1, which the partner passes only after its reads
// of step s.  Each operand read is issued AH products ahead (scheduling
// barriers fix the order).
template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dkdv_kernel(const BwdParams p) {
  using C = TileCopy<D, NW>;
  constexpr int TE = BN * D;
  constexpr int SE = StatsCopy1::FLOATS;
  constexpr int AH = 4;
  // stage st: q~ tile at t_st[st][0], dO tile at t_st[st][1]
  __shared__ __attribute__((aligned(1024))) uint16_t t_st[3][2][TE];
  __shared__ __attribute__((aligned(1024))) float s_st[3][SE];
  __shared__ __attribute__((aligned(1024))) uint16_t x_st[2][NW][2][64 * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave & 1;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  __shared__ int unit_slot;
  const int unit = workgroup_unit(p.sched, &unit_slot);
  if (unit < 0) return;
  const KeyBlock kb = key_block<16 * NW>(p, unit);
  const int nrt = kb.t_hi - kb.t_lo;
  const int nsteps = nrt * p.G;
  const int64_t wkey0 = kb.key0 + 32 * (wave >> 1);
  const int64_t key = wkey0 + l32;
  const bool kvalid = key < p.n_kv;
  const int64_t kpos = p.k_pos0 + key;

  bf16x8 kf[D / 16], vf[D / 16];
  load_frag<D>(p.k + kb.b * p.ks_b + kb.hkv * p.ks_h, key, kvalid, p.ks_s, h, kf);
  load_frag<D>(p.v + kb.b * p.vs_b + kb.hkv * p.vs_h, key, kvalid, p.vs_s, h, vf);
  // role 0: dV^T, role 1: dK^T (register r of block db: d = 32db + 8(r/4) + 4h + r%4, key n)
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  // row tiles (first row at query position q_pos0 + j0) whose rows R0 ..
  // R0 + 31 all keep the pair's 32 keys: rt_lo <= j0 <= rt_hi, with the keys
  // whole; the 64-bit tests once per wave (saturated to int32, which keeps
  // every outcome for j0 in [0, 2^31 - 1)), 32-bit scalar compares per step
  const int R0 = 32 * role;
  const bool keys_whole = wkey0 + 32 <= p.n_kv;
  const int64_t wkpos_min = p.k_pos0 + wkey0, wkpos_max = wkpos_min + 31;
  const bool k_sink = kpos < (int64_t)p.n_sink;
  int rt_lo, rt_hi;
  {
    int64_t hh = p.n_q - R0 - 32;  // j0 + R0 + 32 <= n_q
    if (p.window >= 0 && !(wkpos_max < (int64_t)p.n_sink)) {
      // q_pos0 + j0 + R0 + 31 - window <= wkpos_min
      const int64_t w = wkpos_min + p.window - p.q_pos0 - R0 - 31;
      hh = hh < w ? hh : w;
    }
    rt_hi = KeptTiles::sat(hh);
    rt_lo = p.causal ? KeptTiles::sat(wkpos_max - p.q_pos0 - R0) : INT32_MIN;  // q_pos0 + j0 + R0 >= wkpos_max
  }

  C qcp, gcp;
  qcp.init(p.qs_s, wave, lane);
  gcp.init(p.dos_s, wave, lane);
  // lane offsets into a stage: row reads of the role's 32 rows (q~; dO at
  // + TE), transposing reads of dO (role 0) or q~ (role 1)
  int roff[D / 16], toff[2][D / 32];
  {
    TileOffsets<D> to;
    to.init(lane);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) roff[c] = to.roff[c] + R0 * D;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) toff[hf][db] = to.toff[hf][db] + (role ? 0 : TE);
  }
  // Copy sources of the next step to issue (row tile it, head hkv·G + ig),
  // advanced per issue: steps run over the G heads of a row tile, then the
  // row tile above (no divisions, pointers moved by their strides)
  int it = kb.t_hi - 1, ig = 0;
  const int64_t hq0 = (int64_t)kb.hkv * p.G;
  const uint16_t* iq = p.q + kb.b * p.qs_b + hq0 * p.qs_h + (int64_t)it * BN * p.qs_s;
  const uint16_t* igo = p.dout + kb.b * p.dos_b + hq0 * p.dos_h + (int64_t)it * BN * p.dos_s;
  const float* ist = p.stats + (((int64_t)kb.b * p.Hq + hq0) * p.n_q + (int64_t)it * BN);
  const int64_t pstride = (int64_t)p.B * p.Hq * p.n_q;
  const int64_t q_wrap = (int64_t)(p.G - 1) * p.qs_h + (int64_t)BN * p.qs_s;
  const int64_t g_wrap = (int64_t)(p.G - 1) * p.dos_h + (int64_t)BN * p.dos_s;
  const int64_t s_wrap = (int64_t)(p.G - 1) * p.n_q + BN;
  const uint32_t lt = (uint32_t)(uintptr_t)(lds_void*)&t_st[0][0][0];
  const uint32_t ls = (uint32_t)(uintptr_t)(lds_void*)&s_st[0][0];
  auto issue_next = [&](int st) {
    const int left = (int)p.n_q - it * BN;  // n_q < 2^31
    const uint32_t rows = left <= 0 ? 0u : (left >= BN ? (uint32_t)BN : (uint32_t)left);
    qcp.issue_rows(lt + (uint32_t)(st * 2 * TE * 2), iq, rows);
    gcp.issue_rows(lt + (uint32_t)((st * 2 + 1) * TE * 2), igo, rows);
    // the statistics come with wave 0's copies (one 512-byte load instead
    // of one small load per wave)
    if (wave == 0) StatsCopy1::issue_rows(ls + (uint32_t)(st * SE * 4), ist, pstride, rows, lane);
    if (++ig == p.G) {
      ig = 0;
      --it;
      iq -= q_wrap;
      igo -= g_wrap;
      ist -= s_wrap;
    } else {
      iq += p.qs_h;
      igo += p.dos_h;
      ist += p.n_q;
    }
  };

  // accumulator starts of the step's rows R0 + 8j + 4h + {0..3} (register
  // 4j .. 4j+3): -LSE/sigma for S, -D for dP, 16 bytes of each plane per j
  f32x16 sc0, dp0;
  auto load_stats = [&](int st) {
    const float* sr = s_st[st] + R0 + 4 * h;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 ta = *reinterpret_cast<const f32x4*>(sr + 8 * j);
      const f32x4 tc = *reinterpret_cast<const f32x4*>(sr + StatsCopy1::PLANE1 + 8 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc0[4 * j + e] = ta[e];
        dp0[4 * j + e] = tc[e];
      }
    }
  };

  int ct = kb.t_hi - 1, cg = 0;  // row tile and head of the step
  auto step = [&](int cur, int nxt, int s) {
    const uint16_t* ts = t_st[cur][0];
    const int j0 = ct * BN;
    if (++cg == p.G) {
      cg = 0;
      --ct;
    }
    const bool all_kept = keys_whole && j0 >= rt_lo && j0 <= rt_hi;
    load_stats(cur);
    // products 0 .. D/16-1: S (q~ rows, k~) from -LSE/sigma, so that
    // P = exp2(S'·sigma·log2 e); then dP (dO rows, v) from -D, with the
    // exponentials between them
    constexpr int NC = D / 16, NA = 2 * NC, VP = 16 / NC;
    f32x16 sc = sc0, dp = dp0;
    bf16x8 a[NA];
    auto rd = [&](int i) {
      return *reinterpret_cast<const bf16x8*>(ts + roff[i % NC] + (i < NC ? 0 : TE));
    };
#pragma unroll
    for (int i = 0; i < AH; ++i) a[i] = rd(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if (i < NC) {
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], kf[i], sc, 0, 0, 0);
      } else {
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], vf[i - NC], dp, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < VP; ++v) {
          const int r = (i - NC) * VP + v;
          sc[r] = __builtin_amdgcn_exp2f(sc[r] * p.scale_log2);
        }
      }
      if (i + AH < NA) a[i + AH] = rd(i + AH);
      __builtin_amdgcn_sched_barrier(0);
    }
    // register r: row R0 + 4h + c of the tile with c = 8(r/4) + r%4, key l32;
    // P of a pair outside the mask is 0 (its exponential may have overflowed)
    if (!all_kept) {
      const int64_t qpos_t = p.q_pos0 + j0;
      const int hi = clamp_i32(qpos_t - kpos);  // causal: row off kept iff hi + off >= 0
      const int lo = p.window >= 0 ? clamp_i32(qpos_t - kpos - p.window) : -(1 << 30);  // lo + off <= 0
      const int bias = R0 + 4 * h;
      const int a_r = clamp_tile(p.n_q - (int64_t)j0) - bias, a_hi = hi + bias, a_lo = lo + bias;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = (r >> 2) * 8 + (r & 3);
        const bool ok = kvalid & (c < a_r) & (!p.causal | (a_hi + c >= 0)) & ((a_lo + c <= 0) | k_sink);
        sc[r] = ok ? sc[r] : 0.f;
      }
    }
    // dS = P (dP - D)
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[r] = sc[r] * dp[r];
    bf16x8 pf[2], df[2], own[2];
    pack_half(sc, pf);
    pack_half(dp, df);
    const int buf = s & 1;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      own[k2] = role ? df[k2] : pf[k2];
      *reinterpret_cast<bf16x8*>(&x_st[buf][wave][k2][lane * 8]) = role ? pf[k2] : df[k2];
    }
    stage_barrier<0>();
    // the 16-row slices of tile rows 0-31 (lo) and 32-63 (hi): one pair the
    // wave's own, the other its partner's
    bf16x8 b_lo[2], b_hi[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const bf16x8 part = *reinterpret_cast<const bf16x8*>(&x_st[buf][wave ^ 1][k2][lane * 8]);
      b_lo[k2] = role ? part : own[k2];
      b_hi[k2] = role ? own[k2] : part;
    }
    // role 0: dV^T += dO^T·P, role 1: dK^T += Q^T·dS; product i: 16-row
    // slice i / ND, d-block i % ND
    constexpr int ND = D / 32, NB = 4 * ND;
    bf16x8 t[NB];
    auto rt = [&](int i) {
      const int kc = i / ND, db = i % ND;
      const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(ts + toff[0][db] + kc * 16 * D));
      const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(ts + toff[1][db] + kc * 16 * D));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
#pragma unroll
    for (int i = 0; i < AH; ++i) t[i] = rt(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int kc = i / ND;
      const bf16x8 b = kc < 2 ? b_lo[kc] : b_hi[kc - 2];
      acc[i % ND] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t[i], b, acc[i % ND], 0, 0, 0);
      if (i + AH < NB) t[i + AH] = rt(i + AH);
      __builtin_amdgcn_sched_barrier(0);
      // the copy of tile s + 2 after the last product (not between the
      // barrier and the first operand reads, nor inside the product run); it
      // lands during the next step's S/dP phase
      if (i == NB - 1 && s + 2 < nsteps) issue_next(nxt);
    }
  };

  if (nsteps > 0) issue_next(0);
  if (nsteps > 1) issue_next(1);
  stage_barrier<0>();
  // tile s is in stage s % 3; tile s + 2 goes to stage (s + 2) % 3
  int cur = 0, nxt = 2;
  for (int s = 0; s < nsteps; ++s) {
    step(cur, nxt, s);
    cur = cur == 2 ? 0 : cur + 1;
    nxt = nxt == 2 ? 0 : nxt + 1;
  }

  if (!kvalid) return;
  const bool is_dk = role != 0;
  void* dst;
  if (p.grad_f32)
    dst = is_dk ? (void*)(static_cast<float*>(p.dk) + kb.b * p.dks_b + kb.hkv * p.dks_h + key * p.dks_s)
                : (void*)(static_cast<float*>(p.dv) + kb.b * p.dvs_b + kb.hkv * p.dvs_h + key * p.dvs_s);
  else
    dst = is_dk ? (void*)(static_cast<uint16_t*>(p.dk) + kb.b * p.dks_b + kb.hkv * p.dks_h + key * p.dks_s)
                : (void*)(static_cast<uint16_t*>(p.dv) + kb.b * p.dvs_b + kb.hkv * p.dvs_h + key * p.dvs_s);
  const float f = is_dk ? p.scale : 1.f;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 x = {acc[db][4 * r4] * f, acc[db][4 * r4 + 1] * f, acc[db][4 * r4 + 2] * f,
                       acc[db][4 * r4 + 3] * f};
      store4(p, dst, kpos, db * 32 + r4 * 8 + h * 4, x, is_dk && p.unrotate != 0);
    }
}

constexpr int kBwdNWq128 = 8;  // dq kernel waves (32 rows each)
constexpr int kBwdNWq64 = 4;
constexpr int kBwdNWk = 8;     // dk/dv kernel waves (pairs of waves on 32 keys)

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
  const bool dyn = p.sched != nullptr;
  if (units > 0) {
    if (dyn) launch_sched_init(p.sched, units * p.G, s);
    hipLaunchKernelGGL((bwd_dq_kernel<D, NWQ>), dim3((unsigned)sched_grid(units * p.G, dyn)), dim3(64 * NWQ),
                       0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // dk, dv (every key; with no rows they are zeros)
  const int64_t kblk = (p.n_kv + 16 * kBwdNWk - 1) / (16 * kBwdNWk);
  if (kblk > 0) {
    const int64_t kunits = kblk * p.B * p.Hkv;
    if (dyn) launch_sched_init(p.sched, kunits, s);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, kBwdNWk>), dim3((unsigned)sched_grid(kunits, dyn)),
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
