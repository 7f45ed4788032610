// Tile machinery shared by the gfx950 attention kernels (forward, decode and
// backward): LDS copies that bypass registers, the barrier between pipelined
// tile steps, buffer resources with zero-filled tails, and the range of
// 64-key tiles a block of query rows visits under the causal / window+sink
// mask.  Device-only, header-internal (anonymous namespace).
#pragma once

#include "lcx_device.h"
#include "lcx_internal.h"

namespace lcx {

namespace {

constexpr int BN = kBN;  // 64 keys per tile

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// s_waitcnt immediate (gfx9 encoding) that waits for all but n vector memory
// operations and nothing else
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Workgroup barrier between tile steps.  Before it this wave's LDS reads have
// returned (lgkmcnt 0) and all but its newest `n_vm` vector memory ops (the
// copy of a later tile) have landed; the compiler-only fences keep every
// memory access on its side.  __syncthreads() would also drain the copies
// still in flight.
template <int N_VM>
__device__ __forceinline__ void stage_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(N_VM) & ~(15 << 8));
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// saturate a position difference to +-2^30: every comparison against a key
// offset in [0, BN) keeps its outcome
__device__ __forceinline__ int clamp_i32(int64_t x) {
  return (int)(x > (1 << 30) ? (1 << 30) : (x < -(1 << 30) ? -(1 << 30) : x));
}
__device__ __forceinline__ int clamp_tile(int64_t x) {
  return (int)(x < 0 ? 0 : (x > BN ? BN : x));
}

// Scheduling constraint for a run of N MFMAs, each fed by R LDS operand reads
// of the same basic block: the reads of the first AHEAD products, then one
// product and the reads of a later one alternately, then the last AHEAD
// products, so that AHEAD products' reads are in flight while products issue
// (left to itself the scheduler issues each read one product ahead and waits
// on it).  Only the order changes; the waits are still inserted by the
// compiler.
template <int N, int R, int AHEAD, int ID>
__device__ __forceinline__ void pipeline_reads() {
  constexpr int AH = N > AHEAD ? AHEAD : N;
  __builtin_amdgcn_sched_group_barrier(0x100, AH * R, ID);  // LDS reads
#pragma unroll
  for (int i = 0; i < N - AH; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, R, ID);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AH, ID);
}

// Buffer resource over [base, base + bytes): lane offsets >= bytes read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One buffer load of 16 bytes per lane straight into LDS: lane L's bytes land
// at LDS address lds_addr + 16 L (lds_addr wave-uniform, through M0).  Written
// as an asm block rather than the compiler builtin so that the compiler does
// not track it: with the builtin it put waits for the copy just issued in
// front of the reads of an unrelated stage in one of the unrolled steps.  The
// kernels wait for these copies themselves (vmcnt in stage_barrier).  Nothing
// else in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                           uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(lds_addr)
      : "memory", "m0");
}
// The same for data read once (a decode step's pass over the KV cache): the
// non-temporal policy (sc0 nt) streams it without keeping it in the caches,
// which a plain read kernel measured at 7.1 against 6.2 TB/s on this part.
__device__ __forceinline__ void lds_copy16_stream(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                                  uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen sc0 nt lds"
      :
      : "v"(voff), "s"(rsrc), "s"(lds_addr)
      : "memory", "m0");
}
// cache-policy operand of the buffer-load builtins for such once-read data
constexpr int kLoadStream = 3;  // sc0 | nt
#pragma clang diagnostic pop

// Block (or work unit) bid -> (batch, KV head, hpb query heads of it starting
// at hq, a query block of `span` rows) and the KV tiles it visits: optional
// sink tiles, then the window / causal range.  Blocks run longest causal rows
// first (first rows first under a short window); with xcd_map the G / hpb
// blocks of one (KV head, query block) are consecutive on one XCD (block id
// mod 8), sharing its K/V in that L2.
struct BlockTiles {
  int b, hq, hkv;
  int64_t row0;
  int ntl, sink_n, win_0;
  __device__ __forceinline__ int j0(int t) const { return (t < sink_n ? t : win_0 + (t - sink_n)) * BN; }
};

template <class P>
__device__ __forceinline__ void tile_range(const P& p, int64_t qpos_min, int64_t qpos_max,
                                           BlockTiles& bt);

template <class P>
__device__ __forceinline__ BlockTiles block_tiles(const P& p, int bid, int span, int hpb) {
  BlockTiles bt;
  const int gpb = p.G / hpb;  // blocks per (KV head, query block)
  int unit, g;
  if (p.xcd_map) {
    const int x = bid & 7;
    const int li = bid >> 3;
    g = li % gpb;
    unit = (li / gpb) * 8 + x;
  } else {
    unit = bid / gpb;
    g = bid % gpb;
  }
  bt.hkv = unit % p.Hkv;
  const int t1 = unit / p.Hkv;
  bt.b = t1 % p.B;
  const int qrank = t1 / p.B;
  // longest causal rows first; under a window that covers at most a quarter
  // of the rows, where nearly all blocks visit the same number of tiles, the
  // first rows first instead: a block's first tiles (the start of its window)
  // were then read by the blocks before it and hit in L2, where in the other
  // order they are the ones no block has read yet
  const bool first_rows_first = p.window >= 0 && (p.window + BN) * 4 <= p.n_q;
  const int qblk = first_rows_first ? qrank : p.n_qblk - 1 - qrank;
  bt.hq = bt.hkv * p.G + g * hpb;
  bt.row0 = (int64_t)qblk * span;
  const int64_t blk_last = (bt.row0 + span < p.n_q ? bt.row0 + span : p.n_q) - 1;
  tile_range(p, p.q_pos0 + bt.row0, p.q_pos0 + blk_last, bt);
  return bt;
}

// the KV tiles that query positions [qpos_min, qpos_max] visit: optional sink
// tiles, then the window / causal range
template <class P>
__device__ __forceinline__ void tile_range(const P& p, int64_t qpos_min, int64_t qpos_max,
                                           BlockTiles& bt) {
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
  bt.sink_n = (int)sink_t1;
  bt.win_0 = (int)win_t0;
  bt.ntl = (int)(sink_t1 + (win_t1 - win_t0));
}

// Dynamic work order of a launch (forward and backward attention kernels).
// The work units are the block ids of the kernel's static order (longest
// rows first; unit v on XCD v mod 8 next to the units that share its K/V, or
// its q~/dO, in that XCD's L2).  The hardware hands workgroups to the XCDs in
// turn (block id mod 8), so in the static order every XCD gets the same
// share of the work, and an XCD that runs slower than the others (they
// differ by a few per cent under this load) leaves them idle at the end.
// With a sched buffer the launch has more workgroups than units; each takes a
// unit from the queue of its own XCD, front first (longest first), and once
// that queue is empty takes the back (shortest) unit of another queue, or
// exits when all are empty.  Faster XCDs thus take over the last units of
// slower ones.  Queue x holds v = x + 8i for i in [h, t): its 64-bit word
// packs h (low half) and t (high half), set to (0, n_x) before the launch
// (launch_sched_init).  A front take adds 1 to h and owns index h if h < t
// held; a back take lowers t by one with a compare-and-swap only while
// h < t, so a failed take never moves t below h.  Returns the unit, or -1
// when every queue is empty; called by one thread.
__device__ __forceinline__ int take_unit(unsigned long long* q) {
  const int x = blockIdx.x & 7;
  {
    const unsigned long long old = __hip_atomic_fetch_add(q + x, 1ull, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
    const unsigned h = (unsigned)old, t = (unsigned)(old >> 32);
    if (h < t) return x + 8 * (int)h;
  }
  for (int k = 1; k < 8; ++k) {
    unsigned long long* w = q + ((x + k) & 7);
    unsigned long long old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
      const unsigned h = (unsigned)old, t = (unsigned)(old >> 32);
      if (h >= t) break;
      const unsigned long long nw = ((unsigned long long)(t - 1) << 32) | h;
      if (__hip_atomic_compare_exchange_strong(w, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT))
        return ((x + k) & 7) + 8 * (int)(t - 1);
    }
  }
  return -1;
}

// The work unit of this workgroup: its block id, or with `sched` the unit
// thread 0 takes from the queues, handed to every wave through `slot` (LDS);
// -1 when the queues are empty.  Every thread of the workgroup calls it.
__device__ __forceinline__ int workgroup_unit(unsigned long long* sched, int* slot) {
  if (!sched) return (int)blockIdx.x;
  if (threadIdx.x == 0) *slot = take_unit(sched);
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*slot);
}

}  // namespace

}  // namespace lcx
