// Layout step for the PV product: V [B][Hkv][n][d] (bf16) converted to f16
// (exact for magnitudes in [2^-14, 65504]) into 64-key tiles [d][64] whose
// keys are in the row order of the QK^T accumulator, so that the attention
// kernel reads each PV operand with one 16-byte LDS load.  Keys past n are
// zeros.
// Source: "上下文擴充套件（Context Extension）" FlashAttention 的分塊計算策略
// (K/V processed in blocks of B_c keys).
#include "lcx_device.h"
#include "lcx_internal.h"

namespace lcx {

namespace {

constexpr int kTileKeys = 64;

// key stored at position p of a tile row: within each 16-key group the keys
// 0-3, 8-11, 4-7, 12-15
__device__ __forceinline__ int tile_key(int p) {
  return (p & ~15) | ((p & 4) << 1) | ((p & 8) >> 1) | (p & 3);
}

// one workgroup per (tile, head, batch): the 64 x d block goes through LDS
template <int D>
__global__ __launch_bounds__(256) void pack_v_kernel(const PackVParams p) {
  constexpr int STR = D + 8;  // padded LDS row (16-bit elements)
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTileKeys * STR];
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const uint16_t* src = p.v + b * p.vs_b + h * p.vs_h;
  const int64_t j0 = (int64_t)t * kTileKeys;
  for (int idx = threadIdx.x; idx < kTileKeys * (D / 8); idx += 256) {
    const int key = idx / (D / 8), ch = idx % (D / 8);
    u32x4 w = {0u, 0u, 0u, 0u};
    if (j0 + key < p.n) w = load_once(reinterpret_cast<const u32x4*>(src + (j0 + key) * p.vs_s + ch * 8));
    *reinterpret_cast<u32x4*>(tile + key * STR + ch * 8) = w;
  }
  __syncthreads();
  uint16_t* dst = p.vt + (((int64_t)b * p.Hkv + h) * p.n_tiles + t) * (D * kTileKeys);
  for (int idx = threadIdx.x; idx < D * (kTileKeys / 8); idx += 256) {
    const int e = idx / (kTileKeys / 8), p0 = (idx % (kTileKeys / 8)) * 8;
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = pack_f16x2(__uint_as_float((uint32_t)tile[tile_key(p0 + 2 * q) * STR + e] << 16),
                        __uint_as_float((uint32_t)tile[tile_key(p0 + 2 * q + 1) * STR + e] << 16));
    *reinterpret_cast<u32x4*>(dst + e * kTileKeys + p0) = w;
  }
}

}  // namespace

hipError_t launch_pack_v(const PackVParams& p, hipStream_t s) {
  if (p.n_tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)p.n_tiles, (unsigned)p.Hkv, (unsigned)p.B);
  if (p.d == 64)
    hipLaunchKernelGGL(pack_v_kernel<64>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(pack_v_kernel<128>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace lcx
