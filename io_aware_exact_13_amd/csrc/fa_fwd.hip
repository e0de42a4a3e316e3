// Fused exact attention forward for MI355X (gfx950 / CDNA4).
//
// What is computed: O = softmax(scale * Q K^T [lower-triangular]) V and the
// per-row natural-log logsumexp, for bf16 Q, K, V in [B][H][N][d] layout.
// The method is the IO-aware tiled forward described on the pages:
//   * "为什么Flash Attention能将注意力计算提速数倍而不损失精度", 分块计算(Tiling):
//     tiles of Q, K, V held on chip, the N x N matrices never reach HBM;
//     在线Softmax技巧: running max / exp-sum, rescale by exp(m_old - m_new);
//     核函数融合: one kernel reads Q, K, V once and writes O once.
//   * "FlashAttention的Triton实现：IO-aware注意力机制底层原理", Triton实现 and
//     FA1 vs FA2: one workgroup per block of query rows, the K/V blocks in the
//     inner loop; fp32 statistics and accumulator; P rounded to bf16 before
//     the P V product.
//   * FlashAttention-2 (same page 2, section Flash Attention 2): parallel over
//     batch x head x query block; each wave owns whole query rows, so the
//     softmax reductions never cross waves.
//   * "GPU Kernel 入门：Triton / FlashAttention", FlashAttention与在线softmax:
//     the statistics m, l, acc, and the single division acc / l at the end.
//
// gfx950 design (not taken from the pages):
//   * Both products run on v_mfma_f32_32x32x16_bf16.  S^T = K Q^T is formed
//     with K as the A operand (from LDS) and Q^T as the B operand (registers,
//     loaded once), so each lane's accumulator column is one query row:
//     lane l holds query l%32 and 16 keys per 32x32 block.  Row max needs one
//     cross-lane step (lane l <-> l^32); row sums stay per lane until the end.
//   * O^T += V^T P^T takes P straight from the S^T accumulators (no LDS
//     round trip): the keys a lane holds are a fixed permutation of the
//     MFMA's K index, and the V^T operand is gathered with the same
//     permutation by ds_read_b64_tr_b16, which reads V in its natural
//     row-major LDS layout and hands each lane 4 consecutive keys of one
//     column.
//   * K and V tiles go HBM -> LDS with global_load_lds_dwordx4 (no VGPR
//     staging), double buffered: the loads of tile j+1 are in flight while
//     tile j is computed; one workgroup barrier per tile.
//   * LDS rows are XOR-swizzled in 16-byte chunks so that the 32 rows read
//     by one MFMA operand fetch and the 4-row groups of the transposed reads
//     spread over all banks.
//   * The softmax works in base 2 with scale*log2(e) folded into one FMA
//     before v_exp_f32.  The reference maximum is moved only when the row
//     maximum grows by more than kSlack (2^8), so the 64-register
//     accumulator rescale is skipped on most tiles; the result is exact for
//     any reference value (it cancels in acc / l) and P stays <= 2^8.
//   * Workgroup order: heads vary fastest, so with B*H a multiple of 8 every
//     head stays on one XCD (workgroups are dealt round-robin to the 8 XCDs)
//     and its K/V stream is shared in that XCD's L2.  Under the causal mask
//     the longest query blocks launch first.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "fa.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

constexpr int kBC = 64;           // keys per K/V tile
constexpr int kGroupWaves = 4;    // waves per ping-pong group, 32 query rows each
constexpr int kWaves = 2 * kGroupWaves;
constexpr int kThreads = kWaves * 64;
constexpr int kBR = kWaves * 32;  // query rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.0f;    // log2 units the reference max may lag the true max
constexpr unsigned kNoRecord = 0x80000000u;   // buffer offset past any tile: reads return 0

// LDS geometry.  Rows are padded instead of swizzled: K rows by 16 bytes, so
// the 16 consecutive rows of an A-operand fetch start 4 banks apart; V rows
// by 64 bytes, so the 4 rows of a transposed read start 16 banks apart.
// Both layouts measured conflict-free on gfx950, and padding keeps every
// per-step address a per-lane base plus an immediate.
template <int D>
struct Geom {
  static constexpr int kRowBytes = 2 * D;                   // one K or V row in HBM
  static constexpr int kDataChunks = kRowBytes / 16;        // 16-byte chunks with data per row
  static constexpr int kKStride = kRowBytes + 16;
  static constexpr int kVStride = kRowBytes + 64;
  static constexpr int kKTile = kBC * kKStride;
  static constexpr int kVTile = kBC * kVStride;
  static constexpr int kKOff[2] = {0, kKTile};              // LDS byte offset of K buffer s
  static constexpr int kVOff[2] = {2 * kKTile, 2 * kKTile + kVTile};
  static constexpr int kLdsBytes = 2 * kKTile + 2 * kVTile;
  static constexpr int kKSlots = kKTile / 16;               // 16-byte LDS slots per K tile
  static constexpr int kVSlots = kVTile / 16;
  static constexpr int kKLoads = (kKSlots + kThreads - 1) / kThreads;   // copies per thread per tile
  static constexpr int kVLoads = (kVSlots + kThreads - 1) / kThreads;
  // every wave-wide copy lands inside its tile
  static_assert(kKSlots % 64 == 0 && kVSlots % 64 == 0, "tile not a whole number of wave copies");
};

// One thread's share of the HBM -> LDS copy of a tile.  Copy i of wave w fills
// the 1 KiB of LDS at base + (kWaves i + w) KiB, lane t the 16 bytes at + 16 t,
// so each lane fetches the global chunk that belongs in its slot.  Slots in
// the row padding get an offset no buffer reaches (the copy writes zeros).
template <int D, int STRIDE, int NLOADS>
struct TileCopy {
  unsigned voff[NLOADS];

  __device__ __forceinline__ void init(int wave, int lane) {
    constexpr int kSlotsPerRow = STRIDE / 16;
#pragma unroll
    for (int i = 0; i < NLOADS; ++i) {
      const int slot = (i * kWaves + wave) * 64 + lane;
      const int row = slot / kSlotsPerRow, chunk = slot % kSlotsPerRow;
      const bool data = chunk < Geom<D>::kDataChunks && row < kBC;
      voff[i] = data ? (unsigned)(row * Geom<D>::kRowBytes + chunk * 16) : kNoRecord;
    }
  }

  // Copy key rows [key0, key0 + kBC) of one head into the LDS tile at `dst`.
  // The buffer starts at row key0 and ends at row N, so rows past the end of
  // the sequence read as zeros.
  __device__ __forceinline__ void issue(const char* head, int key0, int n, char* dst, int wave) const {
    // Device pass only: with the buffer-resource type in this template body,
    // clang's host pass drops the launch stubs of some kernel instances.
#if defined(__HIP_DEVICE_COMPILE__)
    const char* base = head + (size_t)key0 * Geom<D>::kRowBytes;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)base, 0, (n - key0) * Geom<D>::kRowBytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < NLOADS; ++i) {
      if ((i * kWaves + wave) * 64 < STRIDE / 16 * kBC)     // wave-uniform: skip copies past the tile
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + (i * kWaves + wave) * 1024),
                                                 16, voff[i], 0, 0, 0);
    }
#endif
  }
};

// Running state of one wave: 32 query rows, lane l owns row l % 32.
template <int D>
struct RowState {
  f32x16 acc[D / 32];   // O^T accumulators: lane holds column (r/4)*8 + 4h + r%4 of each 32-col tile
  float m_ref;          // reference max, log2 units of the scaled score
  float l_part;         // this lane's share of the exponential sum
};

// S^T = K Q^T for one tile (fp32, unscaled).  A operand: K row 32 kb + l32,
// columns 16 ks + 8 h .. +7; B operand: Q^T from registers.
template <int D>
__device__ __forceinline__ void scores(const char* Kt, int k_lane, const bf16x8 (&qf)[D / 16],
                                       f32x16 (&s)[kBC / 32]) {
  using G = Geom<D>;
#pragma unroll
  for (int kb = 0; kb < kBC / 32; ++kb) {
    bf16x8 a[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      a[ks] = *reinterpret_cast<const bf16x8*>(Kt + k_lane + kb * 32 * G::kKStride + ks * 32);
    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int ks = 1; ks < D / 16; ++ks)
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], qf[ks], s[kb], 0, 0, 0);
  }
}

// Online-softmax update for one tile: mask, row max, lazy rescale of the
// accumulators, P = exp2(S * c - m) in bf16, row sum in fp32.
template <int D, bool MASKED>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[kBC / 32], int key0, int lim, int h, float c_log2,
                                             RowState<D>& st, bf16x8 (&pf)[kBC / 16]) {
  constexpr int kKb = kBC / 32;
  if (MASKED) {
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + kb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        if (key > lim) s[kb][r] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_tile = mx * c_log2;
  const bool grow = m_tile > st.m_ref + kSlack;
  const float m_new = grow ? m_tile : st.m_ref;
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    const float alpha = __builtin_amdgcn_exp2f(st.m_ref - m_new);   // 0 on the first tile
    st.l_part *= alpha;
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[ct][r] *= alpha;
      asm volatile("" : "+v"(st.acc[ct]));
    }
  }
  st.m_ref = m_new;
  const float neg_m = (m_new == -INFINITY) ? 0.f : -m_new;
  // P is summed in fp32 (the logsumexp needs the unrounded weights) and
  // rounded to bf16 for the MFMA.
  float l_even = 0.f, l_odd = 0.f;
#pragma unroll
  for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c_log2, neg_m));
      if (r & 1) l_odd += p; else l_even += p;
      pf[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
    }
  st.l_part += l_even + l_odd;
  // Materialise P and the statistics here: without these empty asm uses the
  // compiler sinks the exponentials next to the MFMAs that consume them,
  // i.e. into the other slot, which defeats the ping-pong.
#pragma unroll
  for (int t = 0; t < kBC / 16; ++t) asm volatile("" : "+v"(pf[t]));
  asm volatile("" : "+v"(st.l_part), "+v"(st.m_ref));
}

// O^T += V^T P^T.  k-step t covers keys 16t..16t+15 of the tile; lane half h
// supplies keys 16t + 4h + {0..3} (elements 0..3) and 16t + 8 + 4h + {0..3}
// (elements 4..7), matching the S^T layout.  The transposed read gives lane a
// of each 16-lane group column cbase + a of 4 consecutive rows when lane a
// points at row a/4, columns cbase + 4(a%4).
template <int D>
__device__ __forceinline__ void accumulate_pv(const char* Vt, int v_lane, const bf16x8 (&pf)[kBC / 16],
                                              RowState<D>& st) {
  using G = Geom<D>;
#pragma unroll
  for (int t = 0; t < kBC / 16; ++t) {
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct) {
      const char* p = Vt + v_lane + t * 16 * G::kVStride + ct * 64;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 8 * G::kVStride));
      const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      st.acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pf[t],
                                                           st.acc[ct], 0, 0, 0);
    }
  }
}

// Everything the blocks need besides the running state.
template <int D>
struct Ctx {
  const char* Kh;
  const char* Vh;
  char* lds;
  int N, n_tiles, lim, wave, h, k_lane, v_lane;
  float c_log2;
  TileCopy<D, Geom<D>::kKStride, Geom<D>::kKLoads> kcopy;
  TileCopy<D, Geom<D>::kVStride, Geom<D>::kVLoads> vcopy;
};

// Start the copies of K_{j+2} (into K_j's buffer) and V_{j+1} (into
// V_{j-1}'s buffer); every wave issues its share.
template <int D>
__device__ __forceinline__ void issue_copies(const Ctx<D>& c, int j, char* k_fill, char* v_fill) {
  if (j + 2 < c.n_tiles) c.kcopy.issue(c.Kh, (j + 2) * kBC, c.N, k_fill, c.wave);
  if (j + 1 < c.n_tiles) c.vcopy.issue(c.Vh, (j + 1) * kBC, c.N, v_fill, c.wave);
}

// Workgroup barrier between slots.  Not __syncthreads(): its release fence
// would also wait for the asynchronous K/V copies, which are meant to stay in
// flight across one slot boundary (wait_copies() waits for them explicitly).
// Every LDS read of a block is consumed by an MFMA inside that block, so no
// read is outstanding here; the memory clobber keeps the compiler from moving
// LDS accesses across the barrier and the scheduling fences keep each block's
// arithmetic inside its slot.
__device__ __forceinline__ void slot_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// MFMA block of tile j: O += V_j P_j (16 MFMAs at d=128), then
// S_{j+1} = K_{j+1} Q^T (16 MFMAs), as one software-pipelined stream: the LDS
// operands of step i + kAhead are requested before the MFMA of step i, so each
// MFMA finds its operand already in registers.  Only one wave per SIMD is in
// its MFMA block at a time, so the block has to hide its own LDS latency.
// Consecutive MFMAs write different accumulators.  S_{j+1} is computed even
// after the last tile (from whatever the buffer holds; the result is unused)
// to keep the block branch-free.
template <int D>
__device__ __forceinline__ void mfma_block(const Ctx<D>& c, const char* k_read, const char* v_read,
                                           const bf16x8 (&qf)[D / 16], const bf16x8 (&pf)[kBC / 16],
                                           f32x16 (&s)[kBC / 32], RowState<D>& st) {
  using G = Geom<D>;
  constexpr int kCt = D / 32, kKs = kBC / 16, kKb = kBC / 32, kDs = D / 16;
  constexpr int kPV = kKs * kCt;        // P V steps: (t, ct), ct fastest
  constexpr int kS = kDs * kKb;         // S steps: (ks, kb), kb fastest
  constexpr int kSteps = kPV + kS;
  constexpr int kAhead = 8;
  bf16x8 opnd[kSteps];
  auto fetch = [&](int i) {
    if (i < kPV) {
      const int t = i / kCt, ct = i % kCt;
      const char* p = v_read + c.v_lane + t * 16 * G::kVStride + ct * 64;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 8 * G::kVStride));
      opnd[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      const int ks = (i - kPV) / kKb, kb = (i - kPV) % kKb;
      opnd[i] = *reinterpret_cast<const bf16x8*>(k_read + c.k_lane + kb * 32 * G::kKStride + ks * 32);
    }
  };
  auto mfma = [&](int i) {
    if (i < kPV) {
      const int t = i / kCt, ct = i % kCt;
      st.acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[i], pf[t], st.acc[ct], 0, 0, 0);
    } else {
      const int ks = (i - kPV) / kKb, kb = (i - kPV) % kKb;
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[i], qf[ks], ks == 0 ? f32x16{} : s[kb], 0, 0, 0);
    }
  };
  static_assert(kPV >= kAhead && kS >= kAhead, "pipeline deeper than a phase");
  // Scheduling groups (mask 0x100: LDS reads, 0x008: MFMA) pin the order.
#pragma unroll
  for (int i = 0; i < kAhead; ++i) fetch(i);
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);
#pragma unroll
  for (int i = 0; i < kPV - kAhead; ++i) {          // P V steps, prefetching P V operands
    fetch(i + kAhead);
    mfma(i);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
#pragma unroll
  for (int i = kPV - kAhead; i < kSteps - kAhead; ++i) {   // prefetching S operands
    fetch(i + kAhead);
    mfma(i);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
#pragma unroll
  for (int i = kSteps - kAhead; i < kSteps; ++i) {
    mfma(i);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
}

// The two groups' schedules.  Slots are separated by workgroup barriers;
// group 0 runs MFMA blocks in even slots and VALU blocks in odd slots, group 1
// the opposite, so on every SIMD (one wave of each group) the matrix unit
// works on one wave's products while the other wave does its softmax.
//   group 0:  S_0 | V(0) | M(0) | V(1) | M(1) | ... | V(n-1) | M(n-1) | -
//   group 1:   -  | S_0  | V(0) | M(0) | V(1) | ... | M(n-2) | V(n-1) | M(n-1)
// K_j is read in slots 2j, 2j+1 and V_j in 2j+2, 2j+3, so the copies of
// K_{j+2} and V_{j+1} start at slot 2j+2 and are waited for at the end of
// slot 2j+3.  A period's four buffers (K_{j+1}, V_j read; K_j's and V_{j-1}'s
// being refilled) are distinct restrict pointers: that lets the compiler keep
// the copies in flight across the LDS reads; the explicit waits order them.
template <int D, bool MASKED>
__device__ __forceinline__ void period_g0(const Ctx<D>& c, int j, const char* __restrict__ k_read,
                                          const char* __restrict__ v_read, char* __restrict__ k_fill,
                                          char* __restrict__ v_fill, const bf16x8 (&qf)[D / 16],
                                          f32x16 (&s)[kBC / 32], bf16x8 (&pf)[kBC / 16], RowState<D>& st) {
  slot_barrier();                          // slot 2j+1
  softmax_tile<D, MASKED>(s, j * kBC, c.lim, c.h, c.c_log2, st, pf);
  if (j > 0) wait_copies();                // copies started at slot 2j
  slot_barrier();                          // slot 2j+2
  issue_copies<D>(c, j, k_fill, v_fill);
  mfma_block<D>(c, k_read, v_read, qf, pf, s, st);
}

template <int D, bool MASKED>
__device__ __forceinline__ void period_g1(const Ctx<D>& c, int j, const char* __restrict__ k_read,
                                          const char* __restrict__ v_read, char* __restrict__ k_fill,
                                          char* __restrict__ v_fill, const bf16x8 (&qf)[D / 16],
                                          f32x16 (&s)[kBC / 32], bf16x8 (&pf)[kBC / 16], RowState<D>& st) {
  slot_barrier();                          // slot 2j+2
  issue_copies<D>(c, j, k_fill, v_fill);
  softmax_tile<D, MASKED>(s, j * kBC, c.lim, c.h, c.c_log2, st, pf);
  slot_barrier();                          // slot 2j+3
  mfma_block<D>(c, k_read, v_read, qf, pf, s, st);
  wait_copies();
}

// Run period j of group G: buffers by the parity of j.
template <int D, int G, bool MASKED>
__device__ __forceinline__ void period(const Ctx<D>& c, int j, const bf16x8 (&qf)[D / 16],
                                       f32x16 (&s)[kBC / 32], bf16x8 (&pf)[kBC / 16], RowState<D>& st) {
  using Gm = Geom<D>;
  const int par = j & 1;
  char* k_same = c.lds + par * Gm::kKTile;                        // K_j's buffer
  char* k_other = c.lds + (par ^ 1) * Gm::kKTile;                 // K_{j+1}
  char* v_same = c.lds + 2 * Gm::kKTile + par * Gm::kVTile;       // V_j
  char* v_other = c.lds + 2 * Gm::kKTile + (par ^ 1) * Gm::kVTile;  // V_{j-1}, refilled with V_{j+1}
  if (G == 0) period_g0<D, MASKED>(c, j, k_other, v_same, k_same, v_other, qf, s, pf, st);
  else        period_g1<D, MASKED>(c, j, k_other, v_same, k_same, v_other, qf, s, pf, st);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                   const __bf16* __restrict__ V, __bf16* __restrict__ O, float* __restrict__ LSE,
                   int BH, int N, int n_qblocks, float c_log2) {
  using G = Geom<D>;
  constexpr int kDs = D / 16;
  constexpr int kCt = D / 32;

  __shared__ __attribute__((aligned(1024))) char lds[G::kLdsBytes];

  Ctx<D> c;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  c.h = lane >> 5;                  // which half of the 64 lanes
  const int l32 = lane & 31;        // this lane's query row within the wave
  const int group = c.wave / kGroupWaves;

  // ---- workgroup -> (head, query block)
  const int wg = blockIdx.x;
  const int bh = wg % BH;
  const int qb = CAUSAL ? (n_qblocks - 1 - wg / BH) : (wg / BH);
  const int q0 = qb * kBR;
  const int qrow = q0 + c.wave * 32 + l32;   // this lane's query
  c.N = N;
  c.lim = CAUSAL ? min(qrow, N - 1) : N - 1;   // last key this lane may see
  c.c_log2 = c_log2;
  c.lds = lds;

  const size_t head_off = (size_t)bh * (size_t)N * D;
  c.Kh = reinterpret_cast<const char*>(K + head_off);
  c.Vh = reinterpret_cast<const char*>(V + head_off);

  // ---- key tiles: every wave walks the workgroup's n_tiles (under the causal
  // mask, tiles wholly past a wave's rows are masked out by its softmax).
  const int kv_end = CAUSAL ? min(N, q0 + kBR) : N;
  c.n_tiles = (kv_end + kBC - 1) / kBC;
  // tiles from j_mask on hold keys past the end or past some query of the block
  int j_mask = (N - 1) / kBC;                           // the tile holding key N-1
  if (CAUSAL) j_mask = min(j_mask, q0 / kBC);           // first tile with a key > q0
  j_mask = min(j_mask, c.n_tiles);

  // ---- per-lane offsets
  c.k_lane = l32 * G::kKStride + c.h * 16;
  c.v_lane = (4 * c.h + ((lane & 15) >> 2)) * G::kVStride + (((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2;
  c.kcopy.init(c.wave, lane);
  c.vcopy.init(c.wave, lane);

  // ---- prologue: K_0, V_0, K_1 in flight while Q is fetched
  c.kcopy.issue(c.Kh, 0, N, lds + G::kKOff[0], c.wave);
  c.vcopy.issue(c.Vh, 0, N, lds + G::kVOff[0], c.wave);
  if (c.n_tiles > 1) c.kcopy.issue(c.Kh, kBC, N, lds + G::kKOff[1], c.wave);

  // Q^T operand: lane holds Q[qrow][16*ks + 8*h .. +7] for each k-step
  bf16x8 qf[kDs];
  {
    const bool ok = qrow < N;
    const bf16x8* src = reinterpret_cast<const bf16x8*>(Q + head_off + (size_t)(ok ? qrow : 0) * D);
#pragma unroll
    for (int ks = 0; ks < kDs; ++ks) {
      bf16x8 x = src[ks * 2 + c.h];
      if (!ok) x = bf16x8{};
      qf[ks] = x;
    }
  }

  RowState<D> st;
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) st.acc[ct] = f32x16{};
  st.m_ref = -INFINITY;
  st.l_part = 0.f;
  f32x16 s[kBC / 32];
  bf16x8 pf[kBC / 16];

  wait_copies();
  slot_barrier();                                 // slot 0
  if (group == 0) {
    scores<D>(lds + G::kKOff[0], c.k_lane, qf, s);
    int j = 0;
    for (; j < j_mask; ++j) period<D, 0, false>(c, j, qf, s, pf, st);
    for (; j < c.n_tiles; ++j) period<D, 0, true>(c, j, qf, s, pf, st);
    slot_barrier();                               // slot 2n+1: idle
  } else {
    slot_barrier();                               // slot 1
    scores<D>(lds + G::kKOff[0], c.k_lane, qf, s);
    int j = 0;
    for (; j < j_mask; ++j) period<D, 1, false>(c, j, qf, s, pf, st);
    for (; j < c.n_tiles; ++j) period<D, 1, true>(c, j, qf, s, pf, st);
  }

  // ---- epilogue: O = acc / l (bf16), LSE = (m_ref + log2 l) * ln 2
  const float l_tot = st.l_part + __shfl_xor(st.l_part, 32);
  if (qrow < N) {
    const float inv = 1.0f / l_tot;
    __bf16* orow = O + head_off + (size_t)qrow * D;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int c0 = ct * 32 + r4 * 8 + c.h * 4;
        const __bf16 b0 = (__bf16)(st.acc[ct][r4 * 4 + 0] * inv);
        const __bf16 b1 = (__bf16)(st.acc[ct][r4 * 4 + 1] * inv);
        const __bf16 b2 = (__bf16)(st.acc[ct][r4 * 4 + 2] * inv);
        const __bf16 b3 = (__bf16)(st.acc[ct][r4 * 4 + 3] * inv);
        u32x2 w;
        w[0] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        w[1] = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        *reinterpret_cast<u32x2*>(orow + c0) = w;
      }
    if (c.h == 0) LSE[(size_t)bh * N + qrow] = (st.m_ref + log2f(l_tot)) * kLn2;
  }
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

}  // namespace

extern "C" const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer argument";
    case FA_ERR_SHAPE: return "B, H and N must be >= 1 and the grid must fit the launch limits";
    case FA_ERR_HEAD_DIM: return "head dimension d must be 64 or 128";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_FLAG: return "causal must be 0 or 1";
    case FA_ERR_ALIAS: return "output buffers overlap an input or each other";
    default: return "unknown status";
  }
}

static int check_shape(int B, int H, int N, int d, int causal, long long* blocks) {
  if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (causal != 0 && causal != 1) return FA_ERR_FLAG;
  const long long bh = (long long)B * H;
  const long long nqb = ((long long)N + kBR - 1) / kBR;
  const long long g = bh * nqb;
  // grid size in work-items must fit 32 bits; heads must index in int
  if (bh > 0x7fffffffLL || g * kThreads > 0xffffffffLL) return FA_ERR_SHAPE;
  // one head's K or V must stay below 2 GiB (buffer offsets are 32-bit)
  if ((long long)N * d * 2 >= 0x80000000LL) return FA_ERR_SHAPE;
  *blocks = g;
  return FA_OK;
}

extern "C" int fa_fwd_tile(int B, int H, int N, int d, int causal, int* rows_per_block,
                           int* keys_per_tile, int* waves, long long* blocks) {
  long long g = 0;
  const int st = check_shape(B, H, N, d, causal, &g);
  if (st != FA_OK) return st;
  if (rows_per_block) *rows_per_block = kBR;
  if (keys_per_tile) *keys_per_tile = kBC;
  if (waves) *waves = kWaves;
  if (blocks) *blocks = g;
  return FA_OK;
}

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  long long blocks = 0;
  const int st = check_shape(B, H, N, d, causal, &blocks);
  if (st != FA_OK) return st;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                        reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o);
  if ((mis & 15u) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return FA_ERR_ALIGN;
  const size_t elems = (size_t)B * H * (size_t)N * d;
  const size_t tb = elems * 2, lb = (size_t)B * H * (size_t)N * 4;
  if (overlaps(o, tb, q, tb) || overlaps(o, tb, k, tb) || overlaps(o, tb, v, tb) ||
      overlaps(lse, lb, q, tb) || overlaps(lse, lb, k, tb) || overlaps(lse, lb, v, tb) ||
      overlaps(lse, lb, o, tb))
    return FA_ERR_ALIAS;

  const int BH = B * H;
  const int nqb = (N + kBR - 1) / kBR;
  const float c_log2 = scale * kLog2e;
  const __bf16* Q = static_cast<const __bf16*>(q);
  const __bf16* Kp = static_cast<const __bf16*>(k);
  const __bf16* Vp = static_cast<const __bf16*>(v);
  __bf16* Op = static_cast<__bf16*>(o);
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (d == 128) {
    if (causal) hipLaunchKernelGGL((fa_fwd_kernel<128, true>), grid, block, 0, stream, Q, Kp, Vp, Op, lse, BH, N, nqb, c_log2);
    else        hipLaunchKernelGGL((fa_fwd_kernel<128, false>), grid, block, 0, stream, Q, Kp, Vp, Op, lse, BH, N, nqb, c_log2);
  } else {
    if (causal) hipLaunchKernelGGL((fa_fwd_kernel<64, true>), grid, block, 0, stream, Q, Kp, Vp, Op, lse, BH, N, nqb, c_log2);
    else        hipLaunchKernelGGL((fa_fwd_kernel<64, false>), grid, block, 0, stream, Q, Kp, Vp, Op, lse, BH, N, nqb, c_log2);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}
