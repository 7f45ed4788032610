/*
 * lcx — long-context scaled-RoPE causal GQA attention on MI355X (gfx950).
 *
 * C ABI of liblcx.so.  Plain pointers and sizes only.  Device pointers are
 * HIP device memory owned by the caller; host pointers are ordinary memory.
 * The library allocates no device memory, never synchronises and never
 * creates streams: all device work is enqueued on the caller's `stream`.  Its
 * only state is the fixed device scratch of lcx_attn_decode_noalloc (one
 * copy per device, held until the process ends) and that array's address per
 * device.  Every argument check happens before anything is
 * enqueued; a non-OK return enqueues nothing (LCX_ERR_HIP: a launch was
 * rejected by the runtime).  Faults inside kernels surface at the caller's
 * next synchronisation.  No C++ exception crosses this boundary.
 * lcx_last_error() gives a per-thread message for the last non-OK return.
 *
 * Sources, by page title and section:
 *   [CE] "上下文擴充套件（Context Extension）" (compassingai.com concept page)
 *   [CW] "上下文窗口扩展技术：从 4K 到 1M" (guijiagi.com)
 *   [JJ] "AI 大模型窗口上下文进化史" (juejin.cn)
 *
 * Layouts.  Q, O: [B][Hq][n][d]; K, V: [B][Hkv][n][d]; each given by element
 * strides {batch, head, seq}; the last dimension is contiguous.  LSE is
 * fp32 [B][Hq][n] with strides {batch, head} and unit row stride.  RoPE
 * tables are fp32 row-major [n_pos][d/2]: row r is position tab_pos0 + r.
 */
#ifndef LCX_H
#define LCX_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LCX_OK = 0,
  LCX_ERR_INVALID_ARG = 1, /* NULL where required, bad sizes, bad scheme parameters */
  LCX_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement (d not 64/128, ...) */
  LCX_ERR_HIP = 3          /* the HIP runtime rejected a launch */
} lcx_status;

/* RoPE schemes.  s = L_target / L_train throughout.
 *   PLAIN        theta_i = base^(-2i/d), pair (2i, 2i+1) of q/k at position m
 *                turned by m·theta_i                        [CE 技術原理 RoPE 定義]
 *   PI           positions scaled: m -> m·L_train/L_target   [CW §2.1; CE 位置插值]
 *   NTK          base -> base·s^(d/(d-2))                     [CW §2.2; CE NTK-aware]
 *   NTK_PARTS    per-pair factor by wavelength: 1 below L_train/beta, 1/s above
 *                L_train/alpha, linear in wavelength between   [CW §2.3]
 *   YARN         NTK_PARTS + logits divided by t = 0.1·ln(s) + 1   [CW §2.4]
 *   DYNAMIC_NTK  base -> base·(l/L_train)^(d/(d-2)) when l > L_train, l = cur_len
 *                                                              [CW §3 动态 NTK]  */
typedef enum {
  LCX_ROPE_NONE = 0,
  LCX_ROPE_PLAIN = 1,
  LCX_ROPE_PI = 2,
  LCX_ROPE_NTK = 3,
  LCX_ROPE_NTK_PARTS = 4,
  LCX_ROPE_YARN = 5,
  LCX_ROPE_DYNAMIC_NTK = 6,
  LCX_ROPE_PAIR_FACTORS = 7 /* theta'_i = theta_i / factors[i]  [CW §2.5 LongRoPE] */
} lcx_rope_scheme;

typedef enum { LCX_BF16 = 0, LCX_F32 = 1, LCX_F16 = 2 } lcx_dtype;

/* The pages' problem statement: scheme, base, head_dim, L_train, L_target and
 * the by-parts ramp parameters ([CW §2.3] signature: head_dim, orig_len,
 * target_len, alpha = 1, beta = 32; [CW §3] base, train_len, head_dim, l). */
typedef struct {
  int32_t scheme;   /* lcx_rope_scheme */
  int32_t head_dim; /* d: even, >= 2 */
  double base;      /* > 1 */
  int64_t L_train;  /* > 0 for every scaling scheme */
  int64_t L_target; /* >= L_train for every scaling scheme */
  int64_t cur_len;  /* DYNAMIC_NTK: current length l; 0 means L_target */
  double alpha;     /* NTK_PARTS / YARN: 0 < alpha < beta (pages: 1) */
  double beta;      /* (pages: 32) */
  const double* factors; /* PAIR_FACTORS: d/2 finite factors > 0, one per rotation plane
                            (host memory, read during the call); ignored otherwise */
} lcx_rope_cfg;

/*
 * Step a1 + a2: scaled frequencies and the cos/sin tables.
 *
 * Host part (always): inv_freq[d/2] = theta'_i (fp64), *pos_factor (1/s for PI,
 * else 1), *logit_mult (1/t for YARN, else 1).  Each output pointer may be NULL.
 * Device part (when cos_tab and sin_tab are non-NULL): fp32 tables
 * [n_pos][d/2], cos/sin(((pos0 + r)·pos_factor)·theta'_i); the angle is formed
 * and evaluated in fp64 and rounded once to fp32.  Both NULL: host-only call
 * (no HIP call is made; stream may be NULL).
 * Errors: INVALID_ARG for cfg NULL, scheme out of range or NONE, d odd or < 2,
 * base <= 1, L_train <= 0 or L_target < L_train (scaling schemes), alpha/beta
 * outside 0 < alpha < beta (NTK_PARTS/YARN), exactly one table pointer NULL,
 * n_pos < 0, pos0 < 0.
 */
lcx_status lcx_rope_freqs(const lcx_rope_cfg* cfg, int64_t pos0, int64_t n_pos, double* inv_freq,
                          double* pos_factor, double* logit_mult, float* cos_tab, float* sin_tab,
                          hipStream_t stream);

/*
 * Step a3, standalone: rotate q [B][Hq][n][d] and/or k [B][Hkv][n][d] (bf16) at
 * positions pos0 .. pos0+n-1 with the tables from lcx_rope_freqs; V is never
 * rotated.  [CE 技術原理: q_m = R(m)·W_q·x_m, k_n = R(n)·W_k·x_n]
 * out_dtype: LCX_BF16 or LCX_F16 (the f16 form keeps 3 more mantissa bits for
 * the QK^T product).  Either (q, q_out) or (k, k_out) may be NULL/NULL.
 * In place (q_out == q) only for LCX_BF16 with identical strides.
 * Errors: INVALID_ARG for bad sizes, a NULL input with a non-NULL output (or
 * the reverse), table range not covering [pos0, pos0+n); UNSUPPORTED for d
 * not a multiple of 8 or misaligned rows (16-byte).
 */
lcx_status lcx_rope_apply_qk(const void* q, void* q_out, const void* k, void* k_out,
                             int32_t out_dtype, int32_t B, int32_t Hq, int32_t Hkv, int64_t n,
                             int32_t d, const int64_t q_strides[3], const int64_t qo_strides[3],
                             const int64_t k_strides[3], const int64_t ko_strides[3], int64_t pos0,
                             const float* cos_tab, const float* sin_tab, int64_t tab_pos0,
                             int64_t tab_len, hipStream_t stream);

/* Arguments of lcx_attn_fwd. */
typedef struct {
  const void* q; /* [B][Hq][n_q][d]; bf16 raw (rope_q = 1) or pre-rotated bf16/f16 */
  const void* k; /* [B][Hkv][n_kv][d]; bf16 raw (rope_k = 1) or pre-rotated bf16/f16 */
  const void* v; /* [B][Hkv][n_kv][d]; bf16, never rotated; or f16 tiles (v_tiled) */
  int32_t q_dtype, k_dtype; /* LCX_BF16 or LCX_F16 (F16 only when pre-rotated) */
  int32_t B, Hq, Hkv, d;    /* Hq % Hkv == 0; d in {64, 128} */
  int64_t n_q, n_kv;
  int64_t q_strides[3], k_strides[3], v_strides[3], o_strides[3]; /* elements */
  int64_t lse_strides[2];                                         /* elements: batch, head */
  int64_t q_pos0, k_pos0; /* absolute position of row 0 / key 0 (chunks, ring share) */
  int32_t rope_q, rope_k; /* 1: rotate while loading the tile, from the tables */
  const float* cos_tab;   /* tables from lcx_rope_freqs; required if rope_q or rope_k */
  const float* sin_tab;
  int64_t tab_pos0, tab_len;
  const lcx_rope_cfg* rope; /* configuration the rotation came from; supplies the YaRN logit
                               multiplier.  Required with rope_q or rope_k; optional for
                               pre-rotated q/k (then pass it, or softmax_scale, whenever the
                               rotation was YaRN's, or its temperature is not applied);
                               head_dim must equal d */
  float softmax_scale;      /* 0: (1/sqrt(d))·logit_mult(rope) */
  int32_t causal;           /* must be 1 */
  int64_t window;           /* -1: none; else key kept iff pos_k >= pos_q - window ... */
  int32_t n_sink;           /* ... or pos_k < n_sink  [CW §4.1, §4.2] */
  void* o;                  /* [B][Hq][n_q][d], o_dtype */
  int32_t o_dtype;          /* LCX_BF16 or LCX_F32 */
  float* lse;               /* fp32 [B][Hq][n_q], natural log; -inf for a row with no key */
  int32_t accumulate;       /* 1: merge into the existing (o f32, lse) in the epilogue */
  int32_t v_tiled;          /* 1: v is in the tile layout of lcx_attn_pack_v; v_strides[0..1]
                               are its batch and head strides (elements), v_strides[2] unused */
  int32_t precise_qk;       /* 1: QK^T from f16 high and low parts of the rotated, scaled q and
                               of the rotated k (three products: hi·hi + hi·lo + lo·hi), which
                               removes their f16 rounding from the logits (relative error
                               ~2^-22 instead of 2^-11) for inputs with large logits.
                               Needs rope_k = 1 (k raw bf16, rotated in the kernel: a
                               pre-rotated k has already been rounded); 2.1-2.2 times the
                               time of the default.  0: one product on operands rounded
                               once to f16. */
  void* sched;              /* optional, LCX_SCHED_BYTES of device memory, 8-byte aligned,
                               caller-owned, overwritten: the queue words of a dynamic work
                               order (lcx_attn_fwd and each chunk of lcx_attn_fwd_chunked;
                               ignored by lcx_attn_decode).  The hardware deals workgroups
                               to the XCDs in turn, so in a static order each XCD does the
                               same share of the work and a slower one keeps the others
                               waiting at the end; with sched, workgroups take their work
                               from per-XCD queues and XCDs that finish early take the last
                               units of the others.  Results are identical either way.
                               Calls that may run at the same time must not share it.
                               NULL: static order. */
} lcx_attn_args;

/* Size of lcx_attn_args.sched. */
#define LCX_SCHED_BYTES 64u

/*
 * Steps a3 (fused) - a8: blockwise causal GQA attention with online softmax.
 *   S = sigma·Q~K~^T over kept keys, P = softmax(S), O = P·V, LSE = ln sum exp S
 * [JJ §4 scaled dot-product attention; CE FlashAttention 的分塊計算策略 (tiles,
 * running max, accumulated output); CE 第二層 (GQA: query head h reads KV head
 * floor(h·Hkv/Hq)); CW §4.1 SWA; CW §4.2 attention sinks].
 * QK^T runs on f16 MFMA (rotated q scaled by sigma·log2 e and k, each
 * rounded once to f16: q·sigma·log2 e and k must lie within the f16 range),
 * PV on f16 MFMA from V tiles (P rounded to f16) or bf16 MFMA from V rows
 * (P rounded to bf16); fp32 accumulation and softmax, row sums of P rounded
 * to f16.
 * Errors: INVALID_ARG for NULL q/k/v/o/lse, sizes <= 0 (n_kv may be 0: all
 * rows empty), Hq % Hkv != 0, window < -1, n_sink < 0, rope_q/rope_k not 0/1,
 * rope_q or rope_k without rope, rope->head_dim != d, tables missing or not
 * covering the rotated positions, accumulate with a bf16 o, f16 with rope on,
 * precise_qk not 0/1; UNSUPPORTED for d not 64/128, causal == 0,
 * non-16-byte-aligned rows, precise_qk without rope_k, sched not 8-byte
 * aligned.
 */
lcx_status lcx_attn_fwd(const lcx_attn_args* a, hipStream_t stream);

/*
 * Decode over a long KV cache (split-KV): n_q <= 8 new query rows at
 * positions q_pos0 .. q_pos0+n_q-1 (usually the last positions) against the
 * cache keys k_pos0 .. k_pos0+n_kv-1, with the same mask rules as
 * lcx_attn_fwd.  The KV tiles the rows visit are divided among n_splits
 * workgroups per KV head; each writes a partial (O, LSE) into the caller's
 * workspace and a combine pass merges them by log-sum-exp into o and lse.
 * [CW §3 动态 NTK: the step's base, from the current length, is applied to
 * the new rows through the tables; the cache keeps the rotation it was
 * written with.  CW §5.3: merge of partial results by LSE.]
 *   a         as for lcx_attn_fwd, with: k pre-rotated f16 (rope_k = 0,
 *             k_dtype = LCX_F16); v rows or tiles (v_tiled); accumulate = 0;
 *             (Hq/Hkv)·n_q <= 64.
 *   n_splits  1 .. 65535 workgroups per KV head (splits with no tile write
 *             an empty partial).
 *   o_part    fp32 [n_splits][B][Hq][n_q][d], lse_part fp32
 *             [n_splits][B][Hq][n_q]: caller-owned workspace, overwritten.
 * Errors: as lcx_attn_fwd, plus INVALID_ARG for n_splits out of range, a NULL
 * workspace or accumulate = 1; UNSUPPORTED for n_q > 8, (Hq/Hkv)·n_q > 64, K
 * not pre-rotated f16, precise_qk = 1, B or Hkv > 65535.
 */
lcx_status lcx_attn_decode(const lcx_attn_args* a, int32_t n_splits, float* o_part, float* lse_part,
                           hipStream_t stream);

/* Size of the static device scratch that lcx_attn_decode_noalloc keeps the
 * split partials in: 16 MiB per device. */
#define LCX_DECODE_SCRATCH_BYTES (16u << 20)

/*
 * lcx_attn_decode without a caller workspace, for callers that cannot
 * allocate device memory (code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid hipMalloc): the split partials live in a
 * file-scope device array of LCX_DECODE_SCRATCH_BYTES per device instead of
 * o_part/lse_part.  Same arguments, kernels and results as lcx_attn_decode
 * with the same n_splits (bit for bit); makes no hipMalloc, hipFree or other
 * allocating call.  The scratch address of the current device is looked up
 * on the first call on that device (hipGetSymbolAddress) and kept.
 *   a, n_splits  as for lcx_attn_decode; the device is the current one, and
 *                `stream` must belong to it.
 * The partials need n_splits·B·Hq·n_q·(d + 1)·4 bytes (the O part rounded up
 * to 256); more than LCX_DECODE_SCRATCH_BYTES is rejected.  The default split
 * count of the Python binding (about 256 workgroups over B·Hkv for d = 128,
 * 512 for d = 64) needs at most 8.5 MiB for any shape decode accepts.
 * Every call on one device shares that device's array and leaves its
 * partials there: calls that may overlap on one device (different streams,
 * different host threads) race and must be ordered by the caller.  Nothing
 * in the array needs clearing (each call writes every partial it reads).
 * Errors: as lcx_attn_decode (without the workspace checks), plus
 * UNSUPPORTED when the partials exceed the scratch; LCX_ERR_HIP when the
 * current device cannot be queried or the scratch address not looked up.
 */
lcx_status lcx_attn_decode_noalloc(const lcx_attn_args* a, int32_t n_splits, hipStream_t stream);

/*
 * Layout step for the PV product (V is not rotated): V converted to f16 and
 * copied into the tile layout that lcx_attn_fwd reads with v_tiled = 1, so
 * that each MFMA operand of O += P·V is one 16-byte LDS read and P can be
 * kept in f16 (the same role as the pre-rotation of K to f16 by
 * lcx_rope_apply_qk).  [上下文擴充套件 FlashAttention 的分塊計算策略]
 * The conversion is exact for magnitudes in [2^-14, 65504]; smaller values
 * keep an absolute precision of 2^-24 and larger ones become infinite.
 *   v        [B][Hkv][n][d] bf16, strides v_strides (elements), rows 16-byte aligned
 *   v_tiles  [B][Hkv][T][d][64] f16, T = ceil(n / 64), contiguous, caller-owned:
 *            tile t, row e holds V[64t + key][e] for the 64 keys of the tile,
 *            the keys of each 16-key group in the order 0-3, 8-11, 4-7, 12-15
 *            (the row order of the QK^T accumulator); keys >= n are zeros.
 * For lcx_attn_args: v = v_tiles, v_tiled = 1, v_strides = {Hkv·T·64·d, T·64·d, 0}.
 * A call over a key range [j0, j0 + n_kv) of the packed buffer passes
 * v = v_tiles + (j0 / 64)·64·d with j0 a multiple of 64 (the chunked driver
 * needs chunk % 64 == 0).
 * Errors: INVALID_ARG for NULL pointers, B/Hkv < 1, n < 1, negative strides;
 * UNSUPPORTED for d not 64 or 128, unaligned pointers or rows.
 */
lcx_status lcx_attn_pack_v(const void* v, void* v_tiles, int32_t B, int32_t Hkv, int64_t n,
                           int32_t d, const int64_t v_strides[3], hipStream_t stream);

/*
 * Step a9: acc <- merge(acc, part) row by row over [B][H][rows]:
 *   L = max(La, Lb) + log1p(exp(-|La - Lb|)),  O = e^(La-L)·Oa + e^(Lb-L)·Ob,
 * a -inf partial being the identity.  [CE FlashAttention running-max merge;
 * CW §5.3 per-step partial attention merged into the output]
 * O tensors fp32 with element strides {batch, head, row}; LSE strides
 * {batch, head}, unit row stride.  o_final (optional, LCX_BF16 or LCX_F32) also
 * receives the merged O.
 * Errors: INVALID_ARG for NULL required pointers or bad sizes; UNSUPPORTED for
 * d not a multiple of 4.
 */
lcx_status lcx_attn_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                          int32_t B, int32_t H, int64_t rows, int32_t d,
                          const int64_t acc_strides[3], const int64_t part_strides[3],
                          const int64_t lse_acc_strides[2], const int64_t lse_part_strides[2],
                          void* o_final, int32_t o_final_dtype, const int64_t final_strides[3],
                          hipStream_t stream);

/*
 * Step a10: the single-GPU share of ring attention.  Keys are taken in chunks
 * of `chunk` (KV block c at key positions k_pos0 + c·chunk ..), each chunk's
 * partial attention is computed for the query rows that can see it and merged
 * into (o_acc, lse_acc) — fp32 [B][Hq][n_q][d] and [B][Hq][n_q], contiguous,
 * caller-owned.  With o_part/lse_part (same shapes) non-NULL each chunk is
 * written there and merged by lcx_attn_merge; with both NULL the merge runs in
 * the attention epilogue.  At the end a->o receives the result in a->o_dtype
 * and a->lse the LSE (a->o may be o_acc itself when o_dtype is F32, likewise
 * a->lse may be lse_acc).  [CW §5.1-5.4 Ring Attention; kwkr.cn news 38338
 * §2.2 ring computation with online aggregation]
 * Errors: as lcx_attn_fwd, plus INVALID_ARG for chunk <= 0, NULL o_acc/lse_acc,
 * exactly one of o_part/lse_part NULL, a->accumulate != 0, a->o == o_acc with
 * o_dtype other than F32.
 */
lcx_status lcx_attn_fwd_chunked(const lcx_attn_args* a, int64_t chunk, float* o_acc, float* lse_acc,
                                float* o_part, float* lse_part, hipStream_t stream);

/* Arguments of lcx_attn_bwd.  The forward quantities must be those of the
 * lcx_attn_fwd call being differentiated (same scale, mask and positions). */
typedef struct {
  const void* q;    /* q~ = R(p) q: rotated queries, bf16 [B][Hq][n_q][d] */
  const void* k;    /* k~ = R(p) k: rotated keys, bf16 [B][Hkv][n_kv][d] */
  const void* v;    /* bf16 [B][Hkv][n_kv][d] rows (not the tile layout) */
  const void* o;    /* forward output [B][Hq][n_q][d], o_dtype */
  const float* lse; /* forward LSE fp32 [B][Hq][n_q] (natural log; -inf: row with no key) */
  const void* d_o;  /* dL/dO, bf16 [B][Hq][n_q][d] */
  int32_t o_dtype;  /* LCX_BF16 or LCX_F32 */
  int32_t B, Hq, Hkv, d; /* Hq % Hkv == 0; d in {64, 128} */
  int64_t n_q, n_kv;
  int64_t q_strides[3], k_strides[3], v_strides[3], o_strides[3], do_strides[3]; /* elements */
  int64_t lse_strides[2];  /* elements: batch, head (unit row stride) */
  int64_t q_pos0, k_pos0;  /* absolute positions of row 0 / key 0 */
  const lcx_rope_cfg* rope; /* as in lcx_attn_args: required with unrotate; head_dim == d */
  float softmax_scale;      /* 0: (1/sqrt(d))·logit_mult(rope), as in the forward */
  int32_t causal;           /* must be 1 */
  int64_t window;           /* -1: none (same mask rules as lcx_attn_fwd) */
  int32_t n_sink;
  int32_t unrotate;         /* 1: dq = R(p)^T dq~ and dk = R(p)^T dk~ (the gradients of the raw
                               q, k) from the tables; 0: the gradients of q~ and k~ */
  const float* cos_tab;     /* tables of lcx_rope_freqs; required with unrotate, covering */
  const float* sin_tab;     /* the query and the key positions */
  int64_t tab_pos0, tab_len;
  void* dq;                 /* [B][Hq][n_q][d], grad_dtype, overwritten */
  void* dk;                 /* [B][Hkv][n_kv][d], grad_dtype, overwritten (summed over the */
  void* dv;                 /* query heads of each KV head) */
  int32_t grad_dtype;       /* LCX_F32 or LCX_BF16 */
  int64_t dq_strides[3], dk_strides[3], dv_strides[3]; /* elements */
  float* workspace;         /* fp32, 2·B·Hq·n_q floats (e.g. [B][Hq][n_q][2]), contiguous,
                               16-byte aligned, caller-owned scratch, overwritten: per-row
                               statistics of the forward's softmax (from lse) and
                               D = <dO, O>, in a layout internal to the library */
  void* sched;              /* optional, LCX_SCHED_BYTES, 8-byte aligned, caller-owned,
                               overwritten: the dynamic work order of the dq and dk/dv
                               kernels, as lcx_attn_args.sched; NULL: static order */
} lcx_attn_bwd_args;

/*
 * Backward pass of lcx_attn_fwd: the gradients dq, dk, dv of a loss with
 * dL/dO = d_o, by the chain rule through the softmax and the rotation:
 *   P = exp(S - LSE) (rebuilt per tile from the saved LSE, S = sigma·q~·k~^T
 *   over kept keys), dV = P^T dO, dP = dO V^T, D = rowsum(dO ∘ O),
 *   dS = P ∘ (dP - D), dq~ = sigma·dS·k~, dk~ = sigma·dS^T·q~, and with
 *   unrotate dq = R(p)^T dq~, dk = R(p)^T dk~.
 * [上下文擴充套件 FlashAttention 的分塊計算策略 (blockwise, no n x n matrix kept);
 * 技術原理 (q~ = R(m)·W_q·x); AI 大模型窗口上下文进化史 §4; 上下文窗口扩展技术 §4.1,
 * §4.2 (mask).  The pages give no backward pass: this is the exact gradient.]
 * Products on bf16 MFMA (P and dS rounded to bf16), fp32 accumulation; the
 * forward's f16 q~/k~ option does not apply (pass bf16 q~, k~).
 * Pointers of the query side (q, o, lse, d_o, dq, workspace) may be NULL when
 * n_q = 0, those of the key side (k, v, dk, dv) when n_kv = 0; with no rows
 * dk = dv = 0, with no keys dq = 0.
 * Errors: INVALID_ARG for NULL pointers, bad sizes, Hq % Hkv != 0, window <
 * -1, n_sink < 0, bad dtypes, unrotate without rope or without tables covering
 * the positions, rope->head_dim != d;
 * UNSUPPORTED for d not 64/128, causal == 0, non-16-byte-aligned rows or
 * pointers, a row stride of 2^24 elements or more, sched not 8-byte aligned,
 * n_q or n_kv above 2^31 - 64, more work units than one launch holds.
 */
lcx_status lcx_attn_bwd(const lcx_attn_bwd_args* a, hipStream_t stream);

/* Name of a status code (static string). */
const char* lcx_status_string(lcx_status s);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* lcx_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LCX_H */
