// Internal interface between the C-ABI layer (lcx_api.hip) and the kernel
// launchers.  Launchers assume validated arguments and only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcx {

constexpr int kMaxHalfDim = 128;  // d/2 limit for the table kernel's argument block

struct RopeTableParams {
  float* cos_tab;
  float* sin_tab;
  int64_t pos0, n_pos;
  double pos_factor;
  int32_t half;  // d/2
  double theta[kMaxHalfDim];
};

struct RopeApplyParams {
  const uint16_t* x;  // one tensor per launch slot (q or k)
  void* y;
  int64_t xs_b, xs_h, xs_s;
  int64_t ys_b, ys_h, ys_s;
  int32_t B, H;
  int64_t n;
  int32_t d;
  int32_t out_f16;
  int64_t pos0, tab_pos0;
  const float* cos_tab;
  const float* sin_tab;
};

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  const float* cos_tab;
  const float* sin_tab;
  int64_t qs_b, qs_h, qs_s;
  int64_t ks_b, ks_h, ks_s;
  int64_t vs_b, vs_h, vs_s;
  int64_t os_b, os_h, os_s;
  int64_t ls_b, ls_h;
  int64_t n_q, n_kv, q_pos0, k_pos0, tab_pos0;
  int64_t window;
  float scale_log2;  // softmax scale times log2(e)
  int32_t B, Hq, Hkv, G, d;
  int32_t n_qblk;
  int32_t n_sink;
  int32_t q_mode;  // 0: f16 pre-rotated, 1: bf16 pre-rotated, 2: bf16 raw + RoPE at load
  int32_t k_mode;  // same codes, selects the kernel instantiation
  int32_t o_mode;  // 0: bf16, 1: f32, 2: f32 merged into the existing (o, lse)
  int32_t xcd_map; // 1: XCD-aware block order
  int32_t hpb;     // query heads per workgroup (forward)
  int32_t causal;
  int32_t v_tiled;  // 1: v in the 64-key tile layout (vs_b, vs_h its strides)
  int32_t precise_qk;  // 1: QK^T from f16 high/low parts of q~ and k~ (k_mode 2 only)
  unsigned long long* sched;  // 8 queue words: dynamic work order (NULL: one unit per block)
};

// backward pass (gradients of the attention rows)
struct BwdParams {
  const uint16_t* q;   // q~ bf16 [B][Hq][n_q][d]
  const uint16_t* k;   // k~ bf16 [B][Hkv][n_kv][d]
  const uint16_t* v;   // bf16 rows
  const void* o;       // forward output, bf16 or f32
  const float* lse;    // forward LSE
  const uint16_t* dout;  // dL/dO bf16
  float* stats;        // workspace fp32 [B][Hq][n_q][2]: (LSE·log2 e, D)
  void* dq;
  void* dk;
  void* dv;
  const float* cos_tab;
  const float* sin_tab;
  int64_t qs_b, qs_h, qs_s;
  int64_t ks_b, ks_h, ks_s;
  int64_t vs_b, vs_h, vs_s;
  int64_t os_b, os_h, os_s;
  int64_t dos_b, dos_h, dos_s;
  int64_t ls_b, ls_h;
  int64_t dqs_b, dqs_h, dqs_s;
  int64_t dks_b, dks_h, dks_s;
  int64_t dvs_b, dvs_h, dvs_s;
  int64_t n_q, n_kv, q_pos0, k_pos0, tab_pos0;
  int64_t window;
  float scale;       // softmax scale sigma
  float scale_log2;  // sigma·log2(e)
  int32_t B, Hq, Hkv, G, d;
  int32_t n_qblk;
  int32_t n_sink;
  int32_t causal;
  int32_t xcd_map;
  int32_t o_f32;     // forward output in fp32 (else bf16)
  int32_t grad_f32;  // dq, dk, dv in fp32 (else bf16)
  int32_t unrotate;  // 1: dq, dk turned back by R(p)^T from the tables
  unsigned long long* sched;  // 8 queue words: dynamic work order (NULL: one unit per block)
};

struct PackVParams {
  const uint16_t* v;
  uint16_t* vt;
  int64_t vs_b, vs_h, vs_s;
  int32_t B, Hkv, d;
  int64_t n, n_tiles;
};

// decode (split-KV): fp32 partials [n_splits][B][Hq][n_q][d] and [n_splits][B][Hq][n_q]
struct DecodeParams {
  float* o_part;
  float* lse_part;
  int32_t n_splits;
};

struct MergeParams {
  float* o_acc;
  float* lse_acc;
  const float* o_part;
  const float* lse_part;
  void* o_final;
  int32_t final_f32;
  int64_t as_b, as_h, as_s;
  int64_t ps_b, ps_h, ps_s;
  int64_t fs_b, fs_h, fs_s;
  int64_t la_b, la_h, lp_b, lp_h;
  int32_t B, H, d;
  int64_t rows;
};

hipError_t launch_rope_table(const RopeTableParams& p, hipStream_t s);
hipError_t launch_rope_apply(const RopeApplyParams* slots, int n_slots, hipStream_t s);
hipError_t launch_attn_fwd(const AttnParams& p, hipStream_t s);
hipError_t launch_attn_decode(const AttnParams& p, const DecodeParams& dp, hipStream_t s);
// merge the decode partials into o (bf16 or f32, strides of p) and lse
hipError_t launch_decode_combine(const AttnParams& p, const DecodeParams& dp, hipStream_t s);
hipError_t launch_attn_merge(const MergeParams& p, hipStream_t s);
hipError_t launch_pack_v(const PackVParams& p, hipStream_t s);
// backward: row statistics, then the dq and the dk/dv kernels
hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t s);
int attn_bwd_rows_per_block(int d);  // dq kernel query rows per workgroup
int attn_bwd_keys_per_block(int d);  // dk/dv kernel keys per workgroup
// fill (o, lse) rows with the empty state (0, -inf); o fp32 contiguous per row
hipError_t launch_fill_empty(float* o, float* lse, int32_t B, int32_t H, int64_t rows, int32_t d,
                             int64_t os_b, int64_t os_h, int64_t os_s, int64_t ls_b, int64_t ls_h,
                             hipStream_t s);

// copy the chunked driver's fp32 accumulators to the caller's O (bf16 or f32)
// and LSE; either copy is skipped when source and destination coincide
hipError_t launch_finalize(const float* o_acc, const float* lse_acc, void* o, int32_t o_f32,
                           float* lse, int32_t B, int32_t H, int64_t rows, int32_t d,
                           const int64_t acc_st[3], const int64_t lse_acc_st[2],
                           const int64_t o_st[3], const int64_t lse_st[2], hipStream_t s);

// attention tiling (shared by the launcher and the host-side validation)
constexpr int kBN = 64;      // keys per KV tile
constexpr int kNWd64 = 4;    // waves (32 query rows each) per workgroup, d = 64
constexpr int kNWd128 = 8;   // d = 128
// query heads per forward workgroup (the largest power of two dividing G and
// the wave count) and the forward grid size
int attn_heads_per_block(int d, int G);
int64_t attn_fwd_blocks(int d, int B, int Hkv, int G, int64_t n_q);
// workgroups of a launch over `units` work units (dynamic: with the queue
// words of a sched buffer), and the kernel that sets those words first
int64_t sched_grid(int64_t units, bool dynamic);
void launch_sched_init(unsigned long long* sched, int64_t units, hipStream_t s);

}  // namespace lcx
