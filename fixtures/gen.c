/*
 * Seeded synthetic inputs shared by the GPU path's tests/bench and by the
 * oracle's tests.  This file holds no attention or RoPE arithmetic: it only
 * turns (seed, tensor_id, flat index) into a bf16 sample of N(0,1).
 *
 * Generator (counter based, random access):
 *   key      = mix(seed * G + tensor_id * G2 + 1)
 *   a, b     = mix(key + (2p+1) * G), mix(key + (2p+2) * G)   for pair p
 *   u1       = ((a >> 11) + 0.5) * 2^-53          in (0, 1)
 *   u2       =  (b >> 11)        * 2^-53          in [0, 1)
 *   r        = sqrt(-2 ln u1)
 *   z[2p]    = r cos(2 pi u2),  z[2p+1] = r sin(2 pi u2)   (Box-Muller)
 *   out      = bf16(float(z))   both roundings to nearest even
 * where mix is the SplitMix64 finaliser (Steele, Lea, Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014) and G is its
 * golden-ratio increment.  Element i of a tensor depends only on
 * (seed, tensor_id, i), so any slice can be regenerated on its own.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define FX_GAMMA 0x9E3779B97F4A7C15ULL
#define FX_GAMMA2 0xD1B54A32D192ED03ULL

static inline uint64_t fx_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint16_t fx_f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) { /* inf / nan: keep, quiet nan */
    return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  }
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

static inline void fx_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
  uint64_t a = fx_mix(key + (2 * p + 1) * FX_GAMMA);
  uint64_t b = fx_mix(key + (2 * p + 2) * FX_GAMMA);
  double u1 = ((double)(a >> 11) + 0.5) * (1.0 / 9007199254740992.0);
  double u2 = (double)(b >> 11) * (1.0 / 9007199254740992.0);
  double r = sqrt(-2.0 * log(u1));
  double ang = 6.283185307179586476925286766559 * u2;
  *z0 = r * cos(ang);
  *z1 = r * sin(ang);
}

static inline uint64_t fx_key(uint64_t seed, uint32_t tensor_id) {
  return fx_mix(seed * FX_GAMMA + (uint64_t)tensor_id * FX_GAMMA2 + 1ULL);
}

/* Fill out[0..count) with elements offset..offset+count-1 of tensor
 * (seed, tensor_id), as bf16 bit patterns. */
void fx_fill_bf16(uint64_t seed, uint32_t tensor_id, uint64_t offset, uint64_t count,
                  uint16_t* out) {
  uint64_t key = fx_key(seed, tensor_id);
  int64_t n = (int64_t)count;
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t t = 0; t < n; ++t) {
    uint64_t idx = offset + (uint64_t)t;
    double z0, z1;
    fx_pair(key, idx >> 1, &z0, &z1);
    out[t] = fx_f32_to_bf16_rne((float)((idx & 1) ? z1 : z0));
  }
}

/* Gather: out[r*row_len + c] = element idx[r]*row_len + c, for rows given by
 * flat row indices (used to regenerate sampled rows of a large tensor). */
void fx_fill_rows_bf16(uint64_t seed, uint32_t tensor_id, const int64_t* row_idx, int64_t n_rows,
                       int64_t row_len, uint16_t* out) {
  uint64_t key = fx_key(seed, tensor_id);
#pragma omp parallel for schedule(static) if (n_rows > 64)
  for (int64_t r = 0; r < n_rows; ++r) {
    for (int64_t c = 0; c < row_len; ++c) {
      uint64_t idx = (uint64_t)row_idx[r] * (uint64_t)row_len + (uint64_t)c;
      double z0, z1;
      fx_pair(key, idx >> 1, &z0, &z1);
      out[r * row_len + c] = fx_f32_to_bf16_rne((float)((idx & 1) ? z1 : z0));
    }
  }
}

/* Plain fp64 samples (before rounding), for distribution tests. */
void fx_fill_f64(uint64_t seed, uint32_t tensor_id, uint64_t offset, uint64_t count, double* out) {
  uint64_t key = fx_key(seed, tensor_id);
  for (uint64_t t = 0; t < count; ++t) {
    uint64_t idx = offset + t;
    double z0, z1;
    fx_pair(key, idx >> 1, &z0, &z1);
    out[t] = (idx & 1) ? z1 : z0;
  }
}
