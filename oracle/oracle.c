/*
 * ORACLE — test infrastructure only.
 *
 * A plain, slow, fp64 CPU implementation of what the scaled-RoPE causal GQA
 * attention path computes, written from the definitions on the source pages.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header, table or constant generator
 * with the GPU library, and it is never a fallback for it.
 *
 * Sources (page title, section):
 *   [CE]  "上下文擴充套件（Context Extension）" (compassingai.com concept page):
 *         §"A. RoPE 系縮放方案" (method table), §"技術原理 — RoPE 位置編碼的數學機制
 *         與擴充套件" (RoPE definition, PI, NTK-aware, YaRN), §"FlashAttention 的分塊
 *         計算策略" (softmax(QK^T)V and the running-max merge), §"第二層：注意力計算
 *         效率" (GQA row of the efficiency table).
 *   [CW]  "上下文窗口扩展技术：从 4K 到 1M" (guijiagi.com): §2.1 PI, §2.2 NTK-aware,
 *         §2.3 NTK-by-parts, §2.4 YaRN, §3 动态 NTK, §4.1 SWA, §4.2 StreamingLLM,
 *         §5.3 Ring Attention (per-block attention + merge).
 *   [JJ]  "AI 大模型窗口上下文进化史" (juejin.cn), §4: scaled dot-product attention.
 *
 * Readings where the pages are silent, garbled or contradict one another are
 * marked READING below; every one of them is listed in the design notes.
 *
 * Parity pins (what each function is checked against, in the CPU tests):
 *   oracle_rope_freqs : s = 1 gives plain RoPE bit for bit for every scheme;
 *                       NTK-aware lowest frequency = plain / s; by-parts ends
 *                       at 1 and 1/s, continuous, monotone; dynamic = base
 *                       for l <= L_train and = NTK-aware(l/L_train) above;
 *                       geometric frequency ladder with ratio base^(-2/d);
 *                       PI 4K->8K position factor 0.5 (golden file);
 *                       per-pair factors: all 1 = plain, all s = PI's
 *                       angles, by-parts ratios = NTK-by-parts.
 *                       The NTK-by-parts ramp interior and the YaRN
 *                       temperature direction have no printed value:
 *                       parity unpinned for those two readings.
 *   oracle_rope_table : position 0 is the identity; angle addition across
 *                       rows; PI row s*k = plain row k; cos^2+sin^2 = 1.
 *   oracle_rope_rotate: norm preservation; q_m.k_n depends on m-n only;
 *                       matches the matrix exponential of the rotation
 *                       generator (brute force).
 *   oracle_attn_rows  : K = 0 gives LSE = ln(count) and O = mean of kept V
 *                       for causal / window / sink masks; probability rows
 *                       sum to 1; two-key rows are a logistic of the score
 *                       gap (YaRN temperature included); GQA equals MHA with
 *                       repeated K/V; full n x n brute force for n <= 64.
 *   oracle_merge      : any chunking of the keys, merged in any order,
 *                       equals the one-shot rows.
 *   oracle_attn_bwd   : every element of dq, dk, dv against Richardson-
 *                       extrapolated central differences of oracle_attn_rows
 *                       on inputs whose perturbations are exact bf16 values
 *                       (RoPE, YaRN temperature, GQA, offsets, window+sinks,
 *                       empty rows); sum_j dv_j = sum of dO over non-empty
 *                       rows; sum_j R(p_j) dk_j = 0; sum <q, dq> = sum <k, dk>;
 *                       V = 0 gives dq = dk = 0; one-key rows; GQA = summed
 *                       MHA with repeated K/V.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Scheme ids used by this oracle's entry points. */
enum {
  OR_NONE = 0,
  OR_PLAIN = 1,
  OR_PI = 2,
  OR_NTK = 3,
  OR_NTK_PARTS = 4,
  OR_YARN = 5,
  OR_DYNAMIC_NTK = 6,
  OR_PAIR_FACTORS = 7
};

static const double OR_PI_CONST = 3.14159265358979323846264338327950288;

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads the later calls use (timing only; the results do not depend on it). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Plain RoPE frequency ladder: theta_i = base^(-2i/d), i = 0 .. d/2-1.
 * [CE] 技術原理 (θ_i = 10000^(-2i/d), each pair (2i, 2i+1) rotated by m·θ_i). */
static void plain_theta(double base, int d, double* theta) {
  for (int i = 0; i < d / 2; ++i) theta[i] = pow(base, -(2.0 * i) / (double)d);
}

/*
 * Step a1: the scaled frequency vector theta'[d/2], the position factor
 * (positions are multiplied by it before the angle is formed) and the logit
 * multiplier applied to q.k on top of 1/sqrt(d).
 *
 *   PLAIN        theta' = theta, factor 1.
 *   PI           factor = L_train / L_target          [CW §2.1: m' = m·L_train/L_target;
 *                                                      CE: angle (m/s)·θ_i]
 *   NTK          base' = base · s^(d/(d-2))            [CW §2.2, CE 技術原理 NTK-aware]
 *   NTK_PARTS    theta'_i = theta_i · r_i, with wavelength lambda_i = 2π/theta_i:
 *                r_i = 1 for lambda_i < L_train/beta (short wavelengths untouched),
 *                r_i = 1/s for lambda_i > L_train/alpha (long wavelengths fully
 *                interpolated), linear in lambda in between.       [CW §2.3]
 *                READING: the page's listing puts the lower threshold at
 *                L_train·beta/(2π) (above the upper one for beta = 32, so the
 *                middle branch could never run) and ramps in the direction
 *                that jumps at both ends, against its own "smooth transition"
 *                text; this reading keeps the thresholds ordered and the ramp
 *                continuous, and takes the base from the configuration.
 *   YARN         NTK_PARTS frequencies, logit multiplier 1/t with
 *                t = 0.1·ln(s) + 1.                                  [CW §2.4]
 *                READING: logits divided by t as CW §2.4 writes it (the
 *                concept page's "multiply by 1/√t" is not used).
 *   DYNAMIC_NTK  l = cur_len (0 means L_target); base' = base when
 *                l <= L_train, else base·(l/L_train)^(d/(d-2)).       [CW §3]
 *   PAIR_FACTORS theta'_i = theta_i / factors[i], factor 1, multiplier 1.
 *                                                                     [CW §2.5]
 *                READING: the page gives LongRoPE one scale factor per 2-D
 *                rotation plane, chosen by a search; the factor divides that
 *                plane's frequency the way PI's s divides all of them (all
 *                factors = s reproduces PI's angles).  The search is not
 *                part of the path: the factors are an input.
 *
 * s = L_target / L_train.  Returns 0, or -1 for arguments outside the
 * definitions (d odd or < 2, base <= 1, L_train <= 0, L_target < L_train
 * for the scaling schemes, alpha >= beta or alpha <= 0 for the ramp).
 */
int oracle_rope_freqs(int scheme, double base, int d, int64_t L_train, int64_t L_target,
                      int64_t cur_len, double alpha, double beta, const double* factors,
                      double* theta, double* pos_factor, double* logit_mult) {
  if (d < 2 || (d & 1) || !(base > 1.0)) return -1;
  int scaled = (scheme == OR_PI || scheme == OR_NTK || scheme == OR_NTK_PARTS ||
                scheme == OR_YARN || scheme == OR_DYNAMIC_NTK);
  if (scheme < OR_PLAIN || scheme > OR_PAIR_FACTORS) return -1;
  if (scheme == OR_PAIR_FACTORS) {
    if (!factors) return -1;
    for (int i = 0; i < d / 2; ++i)
      if (!(factors[i] > 0.0) || !isfinite(factors[i])) return -1;
  }
  if (scaled && (L_train <= 0 || L_target < L_train)) return -1;
  if ((scheme == OR_NTK_PARTS || scheme == OR_YARN) && !(alpha > 0.0 && alpha < beta)) return -1;

  double s = scaled ? (double)L_target / (double)L_train : 1.0;
  double factor = 1.0, mult = 1.0;

  switch (scheme) {
    case OR_PLAIN:
      plain_theta(base, d, theta);
      break;
    case OR_PI:
      plain_theta(base, d, theta);
      factor = (double)L_train / (double)L_target;
      break;
    case OR_NTK: {
      double b2 = base * pow(s, (double)d / (double)(d - 2));
      plain_theta(b2, d, theta);
      break;
    }
    case OR_NTK_PARTS:
    case OR_YARN: {
      plain_theta(base, d, theta);
      double lam_lo = (double)L_train / beta;
      double lam_hi = (double)L_train / alpha;
      for (int i = 0; i < d / 2; ++i) {
        double lam = 2.0 * OR_PI_CONST / theta[i];
        double r;
        if (lam < lam_lo) {
          r = 1.0;
        } else if (lam > lam_hi) {
          r = 1.0 / s;
        } else {
          double u = (lam - lam_lo) / (lam_hi - lam_lo);
          r = 1.0 - (1.0 - 1.0 / s) * u;
        }
        theta[i] = theta[i] * r;
      }
      if (scheme == OR_YARN) {
        double t = 0.1 * log(s) + 1.0;
        mult = 1.0 / t;
      }
      break;
    }
    case OR_DYNAMIC_NTK: {
      int64_t l = cur_len > 0 ? cur_len : L_target;
      double b2 = base;
      if (l > L_train) b2 = base * pow((double)l / (double)L_train, (double)d / (double)(d - 2));
      plain_theta(b2, d, theta);
      break;
    }
    case OR_PAIR_FACTORS:
      plain_theta(base, d, theta);
      for (int i = 0; i < d / 2; ++i) theta[i] = theta[i] / factors[i];
      break;
  }
  if (pos_factor) *pos_factor = factor;
  if (logit_mult) *logit_mult = mult;
  return 0;
}

/* Step a2: c[m][i] = cos(p_m·theta'_i), s[m][i] = sin(p_m·theta'_i) with
 * p_m = (pos0 + m)·factor, all in fp64.  [CE 技術原理: φ_{m,i} = m·θ_i] */
void oracle_rope_table(const double* theta, int d, double pos_factor, int64_t pos0,
                       int64_t n_pos, double* cos_out, double* sin_out) {
  int h = d / 2;
  for (int64_t m = 0; m < n_pos; ++m) {
    double p = (double)(pos0 + m) * pos_factor;
    for (int i = 0; i < h; ++i) {
      double phi = p * theta[i];
      cos_out[m * h + i] = cos(phi);
      sin_out[m * h + i] = sin(phi);
    }
  }
}

/* Rotate one d-vector at absolute position pos: each adjacent pair
 * (x_{2i}, x_{2i+1}) turns by angle pos·factor·theta'_i,
 *   (x_{2i}, x_{2i+1}) -> (x_{2i}c - x_{2i+1}s, x_{2i}s + x_{2i+1}c).
 * [CE 技術原理: R(m) rotates each pair (2i, 2i+1)]
 * READING: adjacent (interleaved) pairs, counter-clockwise rotation. */
static void rotate_vec(const double* x, double* y, int d, int64_t pos, const double* theta,
                       double pos_factor) {
  double p = (double)pos * pos_factor;
  for (int i = 0; i < d / 2; ++i) {
    double phi = p * theta[i];
    double c = cos(phi), s = sin(phi);
    double x0 = x[2 * i], x1 = x[2 * i + 1];
    y[2 * i] = x0 * c - x1 * s;
    y[2 * i + 1] = x0 * s + x1 * c;
  }
}

/* Step a3 on fp64 rows: out[r] = R(pos[r]) x[r]. */
void oracle_rope_rotate(const double* x, int64_t n, int d, const int64_t* pos, const double* theta,
                        double pos_factor, double* out) {
  for (int64_t r = 0; r < n; ++r) rotate_vec(x + r * d, out + r * d, d, pos[r], theta, pos_factor);
}

static inline double bf16_bits_to_f64(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Mask: key position kp is kept for query position qp when kp <= qp (causal,
 * self included) and, with a window w >= 0, when kp >= qp - w or kp < n_sink.
 * [CW §4.1: keys K_[i-w, i]; CW §4.2: tokens 0-3 always kept + the window]
 * READING: the window is inclusive, w+1 keys with self. */
static inline int kept(int64_t qp, int64_t kp, int causal, int64_t window, int n_sink) {
  if (causal && kp > qp) return 0;
  if (window >= 0 && !(kp >= qp - window || kp < (int64_t)n_sink)) return 0;
  return 1;
}

/*
 * Steps a4-a8 for a set of query rows, from their definitions:
 *   q~ = R(q_pos) q,  k~_j = R(k_pos0 + j) k_j           (V is not rotated)
 *   S_j = sm_scale · <q~, k~_j>  over kept keys j         [JJ §4; CE FlashAttention]
 *   M = max S,  Z = sum exp(S_j - M),  P_j = exp(S_j - M)/Z
 *   LSE = M + ln Z,  O = sum_j P_j v_j
 * An empty row gives LSE = -inf and O = 0.
 * The KV head of query head h is floor(h·Hkv/Hq)  [CE 第二層 table: GQA —
 * several query heads share one KV head; READING: contiguous groups].
 *
 * q_rows  : [n_rows][d] bf16 bits, the raw (unrotated) query rows
 * q_pos   : absolute position of each row; q_head, q_batch: its head/batch
 * k, v    : [B][Hkv][n_kv][d] bf16 bits, raw
 * rope    : 0 = no rotation (inputs used as given)
 * p_out   : optional [n_rows][n_kv] probabilities (0 for masked keys)
 * Returns 0, or -1 on bad arguments.
 */
int oracle_attn_rows(const uint16_t* q_rows, const int64_t* q_pos, const int32_t* q_head,
                     const int32_t* q_batch, int64_t n_rows, const uint16_t* k, const uint16_t* v,
                     int32_t B, int32_t Hq, int32_t Hkv, int64_t n_kv, int64_t k_pos0, int32_t d,
                     const double* theta, double pos_factor, int32_t rope, double sm_scale,
                     int32_t causal, int64_t window, int32_t n_sink, double* o_out,
                     double* lse_out, double* p_out) {
  if (d < 2 || (d & 1) || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || B <= 0 || n_kv < 0) return -1;
  for (int64_t r = 0; r < n_rows; ++r)
    if (q_head[r] < 0 || q_head[r] >= Hq || q_batch[r] < 0 || q_batch[r] >= B) return -1;

  /* which (batch, kv head) pairs the rows need */
  int64_t nheads = (int64_t)B * Hkv;
  char* need = (char*)calloc((size_t)nheads, 1);
  for (int64_t r = 0; r < n_rows; ++r) {
    int g = (int)(((int64_t)q_head[r] * Hkv) / Hq);
    need[(int64_t)q_batch[r] * Hkv + g] = 1;
  }
  /* rotated keys per needed head (step 3 of the definition, done once per key) */
  double** krot = (double**)calloc((size_t)nheads, sizeof(double*));
  for (int64_t bh = 0; bh < nheads; ++bh) {
    if (!need[bh]) continue;
    krot[bh] = (double*)malloc((size_t)n_kv * d * sizeof(double));
    const uint16_t* kb = k + bh * n_kv * d;
    double* dst = krot[bh];
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n_kv; ++j) {
      double tmp[1024];
      double* x = (d <= 1024) ? tmp : (double*)malloc(sizeof(double) * d);
      for (int c = 0; c < d; ++c) x[c] = bf16_bits_to_f64(kb[j * d + c]);
      if (rope)
        rotate_vec(x, dst + j * d, d, k_pos0 + j, theta, pos_factor);
      else
        memcpy(dst + j * d, x, sizeof(double) * d);
      if (x != tmp) free(x);
    }
  }

#pragma omp parallel
  {
    double* qv = (double*)malloc(sizeof(double) * d);
    double* qr = (double*)malloc(sizeof(double) * d);
    double* sc = (double*)malloc(sizeof(double) * (n_kv > 0 ? n_kv : 1));
    char* keep = (char*)malloc((size_t)(n_kv > 0 ? n_kv : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
      int64_t b = q_batch[r];
      int g = (int)(((int64_t)q_head[r] * Hkv) / Hq);
      const double* kr = krot[b * Hkv + g];
      const uint16_t* vb = v + (b * Hkv + g) * n_kv * d;
      for (int c = 0; c < d; ++c) qv[c] = bf16_bits_to_f64(q_rows[r * d + c]);
      if (rope)
        rotate_vec(qv, qr, d, q_pos[r], theta, pos_factor);
      else
        memcpy(qr, qv, sizeof(double) * d);

      double mx = -INFINITY;
      for (int64_t j = 0; j < n_kv; ++j) {
        keep[j] = (char)kept(q_pos[r], k_pos0 + j, causal, window, n_sink);
        if (!keep[j]) continue;
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += qr[c] * kr[j * d + c];
        sc[j] = sm_scale * acc;
        if (sc[j] > mx) mx = sc[j];
      }
      double* o = o_out + r * d;
      for (int c = 0; c < d; ++c) o[c] = 0.0;
      if (mx == -INFINITY) { /* no kept key */
        lse_out[r] = -INFINITY;
        if (p_out)
          for (int64_t j = 0; j < n_kv; ++j) p_out[r * n_kv + j] = 0.0;
        continue;
      }
      double z = 0.0;
      for (int64_t j = 0; j < n_kv; ++j)
        if (keep[j]) z += exp(sc[j] - mx);
      lse_out[r] = mx + log(z);
      for (int64_t j = 0; j < n_kv; ++j) {
        double p = keep[j] ? exp(sc[j] - mx) / z : 0.0;
        if (p_out) p_out[r * n_kv + j] = p;
        if (p == 0.0) continue;
        const uint16_t* vj = vb + j * d;
        for (int c = 0; c < d; ++c) o[c] += p * bf16_bits_to_f64(vj[c]);
      }
    }
    free(qv);
    free(qr);
    free(sc);
    free(keep);
  }
  for (int64_t bh = 0; bh < nheads; ++bh) free(krot[bh]);
  free(krot);
  free(need);
  return 0;
}

/* R(m)^T applied to one d-vector: each pair turns back by pos·factor·theta'_i,
 *   (y_{2i}, y_{2i+1}) -> (y_{2i}c + y_{2i+1}s, -y_{2i}s + y_{2i+1}c).
 * The transpose of the rotation above: the chain rule through x~ = R(m) x. */
static void rotate_vec_t(const double* y, double* x, int d, int64_t pos, const double* theta,
                         double pos_factor) {
  double p = (double)pos * pos_factor;
  for (int i = 0; i < d / 2; ++i) {
    double phi = p * theta[i];
    double c = cos(phi), s = sin(phi);
    double y0 = y[2 * i], y1 = y[2 * i + 1];
    x[2 * i] = y0 * c + y1 * s;
    x[2 * i + 1] = -y0 * s + y1 * c;
  }
}

/*
 * Gradient of steps a4-a8 (the backward pass).
 * READING: the pages use blockwise attention for training but never write its
 * backward pass out; this is the exact gradient of the forward definition in
 * oracle_attn_rows for a loss L with dL/dO = dO, by the chain rule:
 *   dV_j    = sum_i P_ij dO_i
 *   dP_ij   = <dO_i, v_j>,   D_i = sum_j P_ij dP_ij
 *   dS_ij   = P_ij (dP_ij - D_i)                 (softmax Jacobian)
 *   dq~_i   = sm_scale sum_j dS_ij k~_j,   dk~_j = sm_scale sum_i dS_ij q~_i
 *   dq_i    = R(p_i)^T dq~_i,  dk_j = R(p_j)^T dk~_j   (rope = 0: dq = dq~, dk = dk~)
 * i runs over the rows of every query head that reads KV head g (GQA), j over
 * the keys kept for row i (same mask as the forward); an empty row adds nothing.
 *
 * q, dout : [B][Hq][n_q][d] bf16 bits (raw q when rope = 1); query row r is at
 *           position q_pos0 + r
 * k, v    : [B][Hkv][n_kv][d] bf16 bits; key j at position k_pos0 + j
 * row_sel : optional [B][Hq][n_q] flags, the rows whose dq is computed
 * key_sel : optional [B][Hkv][n_kv] flags, the keys whose dk, dv are computed
 *           (NULL: all).  A row is visited when its dq is wanted or when it
 *           keeps a selected key; unselected outputs are 0.
 * dq      : optional fp64 [B][Hq][n_q][d]; dk, dv: optional fp64 [B][Hkv][n_kv][d]
 * Returns 0, or -1 on bad arguments.
 */
int oracle_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                    int32_t B, int32_t Hq, int32_t Hkv, int64_t n_q, int64_t n_kv, int32_t d,
                    int64_t q_pos0, int64_t k_pos0, const double* theta, double pos_factor,
                    int32_t rope, double sm_scale, int32_t causal, int64_t window, int32_t n_sink,
                    const uint8_t* row_sel, const uint8_t* key_sel, double* dq, double* dk,
                    double* dv) {
  if (d < 2 || (d & 1) || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || B <= 0 || n_q < 0 || n_kv < 0)
    return -1;
  const int G = Hq / Hkv;
  const int64_t nheads = (int64_t)B * Hkv;
  if (dq) memset(dq, 0, sizeof(double) * (size_t)(B * (int64_t)Hq * n_q * d));
  if (dk) memset(dk, 0, sizeof(double) * (size_t)(nheads * n_kv * d));
  if (dv) memset(dv, 0, sizeof(double) * (size_t)(nheads * n_kv * d));
  const int want_keys = (dk != NULL || dv != NULL);

  /* selected keys: a compact index per (batch, kv head), in key order */
  int64_t* sel_start = (int64_t*)calloc((size_t)nheads + 1, sizeof(int64_t));
  for (int64_t bh = 0; bh < nheads; ++bh) {
    int64_t c = 0;
    if (want_keys)
      for (int64_t j = 0; j < n_kv; ++j) c += key_sel ? (key_sel[bh * n_kv + j] != 0) : 1;
    sel_start[bh + 1] = sel_start[bh] + c;
  }
  const int64_t n_sel = sel_start[nheads];
  int64_t* sel_key = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_sel > 0 ? n_sel : 1));
  for (int64_t bh = 0; bh < nheads && want_keys; ++bh) {
    int64_t c = sel_start[bh];
    for (int64_t j = 0; j < n_kv; ++j)
      if (!key_sel || key_sel[bh * n_kv + j]) sel_key[c++] = j;
  }

  /* which (batch, kv head) pairs are needed, and their rotated keys */
  char* need = (char*)calloc((size_t)nheads, 1);
  for (int64_t bh = 0; bh < nheads; ++bh) {
    if (sel_start[bh + 1] > sel_start[bh]) need[bh] = 1;
    if (dq)
      for (int gq = 0; gq < G && !need[bh]; ++gq)
        for (int64_t r = 0; r < n_q; ++r) {
          int64_t row = ((bh / Hkv) * Hq + (bh % Hkv) * G + gq) * n_q + r;
          if (!row_sel || row_sel[row]) {
            need[bh] = 1;
            break;
          }
        }
  }
  double** krot = (double**)calloc((size_t)nheads, sizeof(double*));
  for (int64_t bh = 0; bh < nheads; ++bh) {
    if (!need[bh]) continue;
    krot[bh] = (double*)malloc((size_t)(n_kv > 0 ? n_kv : 1) * d * sizeof(double));
    const uint16_t* kb = k + bh * n_kv * d;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n_kv; ++j) {
      double* x = (double*)malloc(sizeof(double) * d);
      for (int c = 0; c < d; ++c) x[c] = bf16_bits_to_f64(kb[j * d + c]);
      if (rope)
        rotate_vec(x, krot[bh] + j * d, d, k_pos0 + j, theta, pos_factor);
      else
        memcpy(krot[bh] + j * d, x, sizeof(double) * d);
      free(x);
    }
  }

  /* per-thread accumulators of dk~ and dv for the selected keys */
  int nthr = 1;
#ifdef _OPENMP
  nthr = omp_get_max_threads();
#endif
  double* acc_k = (double*)calloc((size_t)nthr * (size_t)(n_sel > 0 ? n_sel : 1) * d, sizeof(double));
  double* acc_v = (double*)calloc((size_t)nthr * (size_t)(n_sel > 0 ? n_sel : 1) * d, sizeof(double));
  const int64_t n_rows = (int64_t)B * Hq * n_q;

#pragma omp parallel
  {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    double* my_k = acc_k + (size_t)tid * (size_t)(n_sel > 0 ? n_sel : 1) * d;
    double* my_v = acc_v + (size_t)tid * (size_t)(n_sel > 0 ? n_sel : 1) * d;
    double* qv = (double*)malloc(sizeof(double) * d);
    double* qr = (double*)malloc(sizeof(double) * d);
    double* go = (double*)malloc(sizeof(double) * d);
    double* gq = (double*)malloc(sizeof(double) * d);
    double* sc = (double*)malloc(sizeof(double) * (n_kv > 0 ? n_kv : 1));
    double* pr = (double*)malloc(sizeof(double) * (n_kv > 0 ? n_kv : 1));
    double* ds = (double*)malloc(sizeof(double) * (n_kv > 0 ? n_kv : 1));
    char* keep = (char*)malloc((size_t)(n_kv > 0 ? n_kv : 1));
#pragma omp for schedule(dynamic, 4)
    for (int64_t row = 0; row < n_rows; ++row) {
      const int64_t r = row % n_q;
      const int64_t bhq = row / n_q;
      const int h = (int)(bhq % Hq);
      const int64_t b = bhq / Hq;
      const int g = (int)(((int64_t)h * Hkv) / Hq);
      const int64_t bh = b * Hkv + g;
      const int64_t qpos = q_pos0 + r;
      const int want_dq = dq != NULL && (!row_sel || row_sel[row]);
      int sees_sel = 0;
      for (int64_t c = sel_start[bh]; c < sel_start[bh + 1] && !sees_sel; ++c)
        sees_sel = kept(qpos, k_pos0 + sel_key[c], causal, window, n_sink);
      if (!want_dq && !sees_sel) continue;

      const double* kr = krot[bh];
      const uint16_t* vb = v + bh * n_kv * d;
      for (int c = 0; c < d; ++c) {
        qv[c] = bf16_bits_to_f64(q[row * d + c]);
        go[c] = bf16_bits_to_f64(dout[row * d + c]);
      }
      if (rope)
        rotate_vec(qv, qr, d, qpos, theta, pos_factor);
      else
        memcpy(qr, qv, sizeof(double) * d);

      /* forward quantities of this row: scores, max, probabilities */
      double mx = -INFINITY;
      for (int64_t j = 0; j < n_kv; ++j) {
        keep[j] = (char)kept(qpos, k_pos0 + j, causal, window, n_sink);
        if (!keep[j]) continue;
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += qr[c] * kr[j * d + c];
        sc[j] = sm_scale * acc;
        if (sc[j] > mx) mx = sc[j];
      }
      if (mx == -INFINITY) continue; /* empty row: no gradient */
      double z = 0.0;
      for (int64_t j = 0; j < n_kv; ++j)
        if (keep[j]) z += exp(sc[j] - mx);
      /* dP_ij, D_i, dS_ij */
      double dsum = 0.0;
      for (int64_t j = 0; j < n_kv; ++j) {
        pr[j] = keep[j] ? exp(sc[j] - mx) / z : 0.0;
        ds[j] = 0.0;
        if (!keep[j]) continue;
        const uint16_t* vj = vb + j * d;
        double dp = 0.0;
        for (int c = 0; c < d; ++c) dp += go[c] * bf16_bits_to_f64(vj[c]);
        ds[j] = dp; /* dP for now */
        dsum += pr[j] * dp;
      }
      for (int64_t j = 0; j < n_kv; ++j) ds[j] = keep[j] ? pr[j] * (ds[j] - dsum) : 0.0;

      if (want_dq) {
        for (int c = 0; c < d; ++c) gq[c] = 0.0;
        for (int64_t j = 0; j < n_kv; ++j) {
          if (!keep[j]) continue;
          for (int c = 0; c < d; ++c) gq[c] += ds[j] * kr[j * d + c];
        }
        for (int c = 0; c < d; ++c) gq[c] *= sm_scale;
        if (rope)
          rotate_vec_t(gq, dq + row * d, d, qpos, theta, pos_factor);
        else
          memcpy(dq + row * d, gq, sizeof(double) * d);
      }
      for (int64_t c = sel_start[bh]; c < sel_start[bh + 1]; ++c) {
        const int64_t j = sel_key[c];
        if (!keep[j]) continue;
        for (int e = 0; e < d; ++e) {
          my_k[c * d + e] += sm_scale * ds[j] * qr[e];
          my_v[c * d + e] += pr[j] * go[e];
        }
      }
    }
    free(qv);
    free(qr);
    free(go);
    free(gq);
    free(sc);
    free(pr);
    free(ds);
    free(keep);
  }

  /* reduce the per-thread sums, then dk = R(p_j)^T dk~ */
  for (int64_t bh = 0; bh < nheads && want_keys; ++bh) {
    for (int64_t c = sel_start[bh]; c < sel_start[bh + 1]; ++c) {
      const int64_t j = sel_key[c];
      double* tk = (double*)malloc(sizeof(double) * d);
      for (int e = 0; e < d; ++e) {
        double sk = 0.0, sv = 0.0;
        for (int t = 0; t < nthr; ++t) {
          sk += acc_k[((size_t)t * (size_t)(n_sel > 0 ? n_sel : 1) + c) * d + e];
          sv += acc_v[((size_t)t * (size_t)(n_sel > 0 ? n_sel : 1) + c) * d + e];
        }
        tk[e] = sk;
        if (dv) dv[(bh * n_kv + j) * d + e] = sv;
      }
      if (dk) {
        if (rope)
          rotate_vec_t(tk, dk + (bh * n_kv + j) * d, d, k_pos0 + j, theta, pos_factor);
        else
          memcpy(dk + (bh * n_kv + j) * d, tk, sizeof(double) * d);
      }
      free(tk);
    }
  }
  free(acc_k);
  free(acc_v);
  for (int64_t bh = 0; bh < nheads; ++bh) free(krot[bh]);
  free(krot);
  free(need);
  free(sel_key);
  free(sel_start);
  return 0;
}

/*
 * Step a9: combine per-chunk results of the same rows.  For chunks c with
 * (LSE_c, O_c):  LSE = log sum_c exp(LSE_c) (taken about the largest term),
 * O = sum_c exp(LSE_c - LSE)·O_c; an all-empty row stays (-inf, 0).
 * [CE FlashAttention: running max + rescaled accumulation; CW §5.3: each ring
 * step's partial attention is merged into the output]
 * READING: the listing's plain "+=" of partial outputs is replaced by the
 * rescaled merge, so chunked and one-shot results agree.
 *
 * lse_parts: [n_chunks][rows], o_parts: [n_chunks][rows][d].
 */
void oracle_merge(const double* lse_parts, const double* o_parts, int64_t n_chunks, int64_t rows,
                  int d, double* lse_out, double* o_out) {
  for (int64_t r = 0; r < rows; ++r) {
    double mx = -INFINITY;
    for (int64_t c = 0; c < n_chunks; ++c)
      if (lse_parts[c * rows + r] > mx) mx = lse_parts[c * rows + r];
    double* o = o_out + r * d;
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    if (mx == -INFINITY) {
      lse_out[r] = -INFINITY;
      continue;
    }
    double z = 0.0;
    for (int64_t c = 0; c < n_chunks; ++c) z += exp(lse_parts[c * rows + r] - mx);
    double lse = mx + log(z);
    lse_out[r] = lse;
    for (int64_t c = 0; c < n_chunks; ++c) {
      double w = exp(lse_parts[c * rows + r] - lse);
      if (w == 0.0) continue;
      const double* oc = o_parts + (c * rows + r) * d;
      for (int i = 0; i < d; ++i) o[i] += w * oc[i];
    }
  }
}
