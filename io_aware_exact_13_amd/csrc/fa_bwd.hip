// Gradients of the fused exact attention forward, for MI355X (gfx950 / CDNA4).
//
// What is computed: for the forward O = softmax(scale Q K^T [lower-triangular])
// V with its per-row natural-log logsumexp LSE, and an upstream gradient dO,
// the gradients dQ, dK, dV (bf16, [B][H][N][d]).  The method is the
// recomputation backward of the pages: the N x N matrices are never stored;
// each kernel rebuilds its tiles of S and P on chip from Q, K and the LSE the
// forward wrote ("为什么Flash Attention能将注意力计算提速数倍而不损失精度",
// 反向传播中的重计算策略; the forward keeps only O and the row statistics,
// 分块计算(Tiling)).  The chain rule through the softmax gives, per row i,
//     P = exp(S - LSE),  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
//     dS = P (dP - D),   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
//
// gfx950 design (not taken from the pages):
//   * Two launches on the caller's stream: dQ by query blocks (K and V
//     tiles stream through LDS), which also forms D = rowsum(dO * O) for its
//     rows and writes it to the caller's fp32 workspace; then dK and dV by
//     key blocks (Q and dO tiles and those rows' LSE and D stream through
//     LDS).  Each output is written by one workgroup: no atomics, and the
//     result is bitwise reproducible.
//   * All products run on v_mfma_f32_32x32x16_bf16 with the operand that a
//     lane owns for the whole loop as the B operand (Q and dO rows in the dQ
//     kernel, K and V rows in the dK/dV kernel), so every accumulator column
//     is one of the lane's own rows.  They sit in registers, except the
//     dK/dV kernel's K rows, which stay in LDS for the whole kernel: with
//     them in registers the kernel needs more than 256 registers per lane
//     and runs one wave per SIMD instead of two.  P and dS go from the
//     accumulators straight into the next MFMA's B operand (bf16), and the
//     matching A operand (K^T, dO^T, Q^T) is read with ds_read_b64_tr_b16
//     from the row-major LDS tile, with the same key/query permutation.
//   * LDS tiles use one 16-byte-chunk XOR swizzle that keeps both the row
//     reads and the transposed reads free of bank conflicts (cdna4.h).
//   * Tiles are copied HBM -> LDS by buffer_load ... lds, double buffered,
//     one workgroup barrier per tile; copies past the last row read zeros.

#include <math.h>

#include <mutex>
#include <type_traits>

#include "cdna4.h"
#include "fa.h"

// Device memory of fa_bwd_noalloc: its D workspace, FA_NOALLOC_ROWS fp32
// values (8 MiB), one copy per GPU, held until the process ends.  Host code
// never passes this name to a kernel (on the host it is only a stand-in): it
// looks up each device's address once and passes that.
static __device__ __align__(256) float scratch[FA_NOALLOC_ROWS];

namespace {

// Waves per SIMD the two gradient kernels are compiled for: 2 at d = 128
// (about 240 registers a lane), 3 at d = 64, whose kernels fit in 168
// registers (5% faster on the 2K d = 64 workload than at 2).
template <int D> constexpr int kWavesPerSimd = D == 64 ? 3 : 2;

using namespace cdna4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXcds = 8;           // accelerator dies; workgroups are dealt to them round-robin
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQBlock = kWaves * 32;   // query rows per dQ workgroup
constexpr int kKTile = 64;             // keys per K/V tile in the dQ kernel
// The dK/dV kernel: FA_BWD_KV_WAVES waves of 32 keys each; 4 (two
// workgroups per CU, 32-row query tiles, one barrier per 32 MFMAs a wave) or
// 8 (one workgroup per CU, 64-row query tiles as two 32-row halves, one
// barrier per 64 MFMAs).  The default is the measured choice; a build may
// override it to measure the other.
#ifndef FA_BWD_KV_WAVES
#define FA_BWD_KV_WAVES 4
#endif
static_assert(FA_BWD_KV_WAVES == 4 || FA_BWD_KV_WAVES == 8, "waves per dK/dV workgroup");
constexpr int kKvWaves = FA_BWD_KV_WAVES;
// Race-check build (FA_BWD_EXTRA_BARRIER=1): after each tile's LDS reads,
// wait for every memory operation and hold a workgroup barrier, so that no
// wave can start the next tile's copy into a buffer another wave may still
// read.  Its gradients must equal the default build's bit for bit.
#ifndef FA_BWD_EXTRA_BARRIER
#define FA_BWD_EXTRA_BARRIER 0
#endif
__device__ __forceinline__ void race_check_barrier() {
  if constexpr (FA_BWD_EXTRA_BARRIER) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
  }
}
constexpr int kKvThreads = kKvWaves * 64;
constexpr int kKBlock = kKvWaves * 32;   // keys per dK/dV workgroup
constexpr int kQTile = kKvWaves == 8 ? 64 : 32;   // query rows per Q/dO tile in the dK/dV kernel
constexpr int kQHalves = kQTile / 32;             // 32-row halves of a tile, one after another

// Workgroup -> (head, block): each XCD walks whole heads one after another,
// so the workgroups running on it share one head's streamed tiles in its L2.
__device__ __forceinline__ void head_and_block(int n_blocks, int BH, int* bh, int* blk) {
  const int wg = blockIdx.x;
  const int n_wg = BH * n_blocks;
  const int logical = (n_wg % kXcds == 0) ? (wg % kXcds) * (n_wg / kXcds) + wg / kXcds : wg;
  *bh = logical / n_blocks;
  *blk = logical % n_blocks;
}

// Store a 32 x 32 fp32 accumulator block C[i = column][j = row] (one row per
// lane) times `mul` as bf16 into row `row` of a [.][D] matrix, columns
// 32 ct + (r / 4) 8 + 4 h + r % 4 (four consecutive columns per 8-byte store).
template <int D>
__device__ __forceinline__ void store_row_block(__bf16* rowp, const f32x16& acc, int ct, int h, float mul) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const int c0 = ct * 32 + r4 * 8 + h * 4;
    u32x2 w;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const __bf16 lo = (__bf16)(acc[r4 * 4 + 2 * half] * mul);
      const __bf16 hi = (__bf16)(acc[r4 * 4 + 2 * half + 1] * mul);
      w[half] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *reinterpret_cast<u32x2*>(rowp + c0) = w;
  }
}

// Lane l's B operand of one row for k-step ks: elements 16 ks + 8 (l / 32) .. +7.
template <int D>
__device__ __forceinline__ void load_row_operands(const __bf16* rowp, bool ok, int h, bf16x8 (&f)[D / 16]) {
  const bf16x8* src = reinterpret_cast<const bf16x8*>(rowp);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    bf16x8 x = ok ? src[ks * 2 + h] : bf16x8{};
    f[ks] = x;
  }
}

// ---------------------------------------------------------------- dQ
// One workgroup per (head, block of 128 query rows); lane l of wave w owns
// query q0 + 32 w + l % 32.  First D = rowsum(dO * O) of the rows (also
// written out for the dK/dV kernel), then per 64-key tile:
//   S^T  = K Q^T,  dP^T = V dO^T          (A: K, V rows from LDS; B: Q, dO in registers)
//   P    = exp2(S^T c - LSE log2 e),  dS = P (dP - D)   (masked keys give 0)
//   dQ^T += K^T dS^T                      (A: K^T by transposed reads; B: dS from registers)
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D>, kWavesPerSimd<D>))) void fa_bwd_dq_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const __bf16* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ Delta, __bf16* __restrict__ dQ, int BH, int N, int n_qblocks, float c_log2, float scale) {
  constexpr int kDs = D / 16, kCt = D / 32, kKb = kKTile / 32;
  constexpr int kTileBytes = kKTile * 2 * D;
  using Copy = TileCopy<D, kKTile, kThreads>;
  __shared__ __attribute__((aligned(1024))) char lds[4 * kTileBytes];   // K 0, K 1, V 0, V 1

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bh, qi;
  head_and_block(n_qblocks, BH, &bh, &qi);
  const int qb = CAUSAL ? (n_qblocks - 1 - qi) : qi;
  const int q0 = qb * kQBlock;
  const int qrow = q0 + wave * 32 + l32;
  const bool qok = qrow < N;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const char* Kh = reinterpret_cast<const char*>(K + head_off);
  const char* Vh = reinterpret_cast<const char*>(V + head_off);

  const int kv_end = CAUSAL ? min(N, q0 + kQBlock) : N;
  const int n_tiles = (kv_end + kKTile - 1) / kKTile;
  const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;      // last key this lane's row sees

  Copy copy;
  copy.init(tid);
#pragma unroll
  for (int i = 0; i < Copy::kIssues; ++i) {
    copy.issue(Kh, 0, kv_end, lds, tid, i);
    copy.issue(Vh, 0, kv_end, lds + 2 * kTileBytes, tid, i);
  }

  bf16x8 qf[kDs], dof[kDs];
  load_row_operands<D>(Q + head_off + (size_t)(qok ? qrow : 0) * D, qok, h, qf);
  load_row_operands<D>(dO + head_off + (size_t)(qok ? qrow : 0) * D, qok, h, dof);
  const float neg_lse2 = qok ? -LSE[(size_t)bh * N + qrow] * kLog2e : 0.f;
  // D = rowsum(dO * O) of this lane's row: the lane holds half of the row's
  // elements (16 ks + 8 h .. +7), the lane 32 apart the other half.  Written
  // to the workspace for the dK/dV kernel, which runs after this one.
  float dlt;
  {
    bf16x8 of[kDs];
    load_row_operands<D>(O + head_off + (size_t)(qok ? qrow : 0) * D, qok, h, of);
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < kDs; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf((float)of[ks][e], (float)dof[ks][e], part);
    const unsigned u = __builtin_bit_cast(unsigned, part);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    dlt = __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
    if (qok && h == 0) Delta[(size_t)bh * N + qrow] = dlt;
  }

  f32x16 acc[kCt];
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) acc[ct] = f32x16{};

  // One key tile.  MASKED: the tile holds a key past N or past some row's
  // diagonal; other tiles skip the visibility test.  `buf` (the tile's
  // double buffer) is a compile-time constant, so the LDS addresses are the
  // lanes' offsets plus immediates.
  auto tile = [&](auto masked, auto buf, int j) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's copies of tile j
    __syncthreads();                                   // everyone's; tile j-1 no longer read
    if (j + 1 < n_tiles) {
#pragma unroll
      for (int i = 0; i < Copy::kIssues; ++i) {
        copy.issue(Kh, (j + 1) * kKTile, kv_end, lds + (buf ^ 1) * kTileBytes, tid, i);
        copy.issue(Vh, (j + 1) * kKTile, kv_end, lds + (2 + (buf ^ 1)) * kTileBytes, tid, i);
      }
    }
    const char* Kt = lds + buf * kTileBytes;
    const char* Vt = lds + (2 + buf) * kTileBytes;

    f32x16 s[kKb], dp[kKb];
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb) { s[kb] = f32x16{}; dp[kb] = f32x16{}; }
#pragma unroll
    for (int ks = 0; ks < kDs; ++ks)
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb) {
        s[kb] = mfma32(row_operand<D>(Kt, 32 * kb, ks, lane), qf[ks], s[kb]);
        dp[kb] = mfma32(row_operand<D>(Vt, 32 * kb, ks, lane), dof[ks], dp[kb]);
      }

    // register r of block kb: key j 64 + 4 h + (32 kb + (r / 4) 8 + r % 4),
    // visible (masked tiles) when that is <= lim
    const int room = lim - j * kKTile - 4 * h;
    bf16x8 dsf[kKTile / 16];
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c_log2, neg_lse2));
        const float p = (!kMasked || room >= kb * 32 + (r >> 2) * 8 + (r & 3)) ? pe : 0.f;
        dsf[kb * 2 + (r >> 3)][r & 7] = (__bf16)(p * (dp[kb][r] - dlt));
      }

#pragma unroll
    for (int t = 0; t < kKTile / 16; ++t)
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct) acc[ct] = mfma32(tr_operand<D>(Kt, 16 * t, ct, lane), dsf[t], acc[ct]);
    race_check_barrier();
  };
  // Tiles [0, j_hi) hold keys visible to every row of the block (at most
  // its first row and below N); they go unmasked in pairs, the first of
  // each in buffer 0, and the rest masked in pairs.
  const int j_hi = min(CAUSAL ? (q0 + 1) / kKTile : N / kKTile, N / kKTile) & ~1;
  int j = 0;
  for (; j < j_hi; j += 2) {
    tile(std::false_type{}, std::integral_constant<int, 0>{}, j);
    tile(std::false_type{}, std::integral_constant<int, 1>{}, j + 1);
  }
  for (; j < n_tiles; j += 2) {
    tile(std::true_type{}, std::integral_constant<int, 0>{}, j);
    if (j + 1 < n_tiles) tile(std::true_type{}, std::integral_constant<int, 1>{}, j + 1);
  }

  if (qok) {
    __bf16* rowp = dQ + head_off + (size_t)qrow * D;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) store_row_block<D>(rowp, acc[ct], ct, h, scale);
  }
}

// ---------------------------------------------------------------- dK, dV
// One workgroup per (head, block of kKBlock keys); lane l of wave w owns key
// k0 + 32 w + l % 32.  Per query tile, for each of its 32-row halves:
//   S  = Q K^T,  dP = dO V^T              (A: Q, dO rows from LDS; B: K rows
//                                          from the resident LDS block, V in registers)
//   P  = exp2(S c - LSE log2 e),  dS = P (dP - D)      (rows past N or above the key give 0)
//   dV^T += dO^T P,  dK^T += Q^T dS       (A: dO^T, Q^T by transposed reads; B: P, dS)
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D>, kWavesPerSimd<D>))) void fa_bwd_dkdv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    __bf16* __restrict__ dK, __bf16* __restrict__ dV, int BH, int N, int n_kblocks, float c_log2,
    float scale) {
  constexpr int kDs = D / 16, kCt = D / 32;
  constexpr int kTileBytes = kQTile * 2 * D;
  constexpr int kStatBytes = 512;                        // 64 LSE then 64 D floats
  static_assert(kQTile <= 64, "one statistics copy covers 64 rows");
  constexpr int kBufBytes = 2 * kTileBytes + kStatBytes;  // Q tile, dO tile, statistics
  constexpr int kKBytes = kKBlock * 2 * D;                // the workgroup's K rows, resident
  using Copy = TileCopy<D, kQTile, kKvThreads>;
  using KCopy = TileCopy<D, kKBlock, kKvThreads>;
  __shared__ __attribute__((aligned(1024))) char lds[kKBytes + 2 * kBufBytes];
  char* const kblk = lds + 2 * kBufBytes;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bh, kbk;
  head_and_block(n_kblocks, BH, &bh, &kbk);
  const int k0 = kbk * kKBlock;
  const int key = k0 + wave * 32 + l32;
  const bool kok = key < N;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const char* Qh = reinterpret_cast<const char*>(Q + head_off);
  const char* dOh = reinterpret_cast<const char*>(dO + head_off);
  const float* Lh = LSE + (size_t)bh * N;
  const float* Dh = Delta + (size_t)bh * N;

  const int t0 = CAUSAL ? k0 / kQTile : 0;                  // first query tile with a row >= k0
  const int n_qt = (N + kQTile - 1) / kQTile;

  Copy copy;
  copy.init(tid);
  auto issue_tile = [&](int i, char* dst) {
#pragma unroll
    for (int c = 0; c < Copy::kIssues; ++c) {
      copy.issue(Qh, i * kQTile, N, dst, tid, c);
      copy.issue(dOh, i * kQTile, N, dst + kTileBytes, tid, c);
    }
    if (wave == 0) {
      copy_row_stats(Lh, i * kQTile, N, dst + 2 * kTileBytes, lane);
      copy_row_stats(Dh, i * kQTile, N, dst + 2 * kTileBytes + 256, lane);
    }
  };
  {
    KCopy kc;
    kc.init(tid);
#pragma unroll
    for (int c = 0; c < KCopy::kIssues; ++c)
      kc.issue(reinterpret_cast<const char*>(K + head_off), k0, N, kblk, tid, c);
  }
  if (t0 < n_qt) issue_tile(t0, lds);

  bf16x8 vf[kDs];
  load_row_operands<D>(V + head_off + (size_t)(kok ? key : 0) * D, kok, h, vf);

  f32x16 acc_dk[kCt], acc_dv[kCt];
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) { acc_dk[ct] = f32x16{}; acc_dv[ct] = f32x16{}; }

  // One query tile.  MASKED: the tile holds a query row past N or a (key,
  // query) pair above the diagonal for some wave of the workgroup; other
  // tiles skip the visibility test.  `buf` is the tile's double buffer, a
  // compile-time constant on the unmasked tiles (their LDS addresses are
  // then the lanes' offsets plus immediates).
  auto tile = [&](auto masked, auto buf, int i) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's copies of tile i
    __syncthreads();                                   // everyone's; tile i-1 no longer read
    if (i + 1 < n_qt) issue_tile(i + 1, lds + (buf ^ 1) * kBufBytes);
    const char* Qt = lds + buf * kBufBytes;
    const char* dOt = Qt + kTileBytes;
    const char* St = Qt + 2 * kTileBytes;

#pragma unroll
    for (int hf = 0; hf < kQHalves; ++hf) {   // the tile's 32-row halves, one after another
      // (kept apart: overlapping the halves would need both halves' S and dP
      // in registers at once)
      if (hf > 0) __builtin_amdgcn_sched_barrier(0);
      const int r0 = 32 * hf;
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < kDs; ++ks) {
        s = mfma32(row_operand<D>(Qt, r0, ks, lane), row_operand<D>(kblk, 32 * wave, ks, lane), s);
        dp = mfma32(row_operand<D>(dOt, r0, ks, lane), vf[ks], dp);
      }

      // register r: query i kQTile + r0 + (r / 4) 8 + 4 h + r % 4; its LSE
      // and D sit four at a time in the statistics tile
      bf16x8 pf[2], dsf[2];
      // masked tiles: register r holds query q = i kQTile + r0 + 4 h + (8 m + e);
      // it is visible when q - key = dq + 8 m + e >= 0 and 8 m + e < N - (q - 8 m - e)
      const int qb = i * kQTile + r0 + 4 * h;
      const int dq = qb - key, rem = N - qb;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 lse4 = *reinterpret_cast<const f32x4*>(St + (r0 + 8 * m + 4 * h) * 4);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(St + 256 + (r0 + 8 * m + 4 * h) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * m + e;
          const float pe = __builtin_amdgcn_exp2f(fmaf(s[r], c_log2, -lse4[e] * kLog2e));
          float p = pe;
          if constexpr (kMasked) p = (8 * m + e < rem && (!CAUSAL || dq >= -(8 * m + e))) ? pe : 0.f;
          pf[r >> 3][r & 7] = (__bf16)p;
          dsf[r >> 3][r & 7] = (__bf16)(p * (dp[r] - d4[e]));
        }
      }

#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) {
          acc_dv[ct] = mfma32(tr_operand<D>(dOt, r0 + 16 * t, ct, lane), pf[t], acc_dv[ct]);
          acc_dk[ct] = mfma32(tr_operand<D>(Qt, r0 + 16 * t, ct, lane), dsf[t], acc_dk[ct]);
        }
    }
    race_check_barrier();
  };
  // Every (key, query) pair of tile i is visible to the whole workgroup
  // when its first query is at or past the block's last key and its last
  // query is below N.  Tiles go in pairs, the first of each in buffer 0:
  // masked pairs up to i_lo, unmasked pairs up to i_hi, masked pairs after.
  const int i_lo = min(n_qt, t0 + ((max(t0, CAUSAL ? (k0 + kKBlock - 1 + kQTile - 1) / kQTile : t0) - t0 + 1) & ~1));
  const int i_hi = i_lo + ((max(i_lo, min(n_qt, N / kQTile)) - i_lo) & ~1);
  auto masked_pairs = [&](int& i, int end) __attribute__((always_inline)) {
    for (; i < end; i += 2) {
      tile(std::true_type{}, std::integral_constant<int, 0>{}, i);
      if (i + 1 < end) tile(std::true_type{}, std::integral_constant<int, 1>{}, i + 1);
    }
  };
  int i = t0;
  masked_pairs(i, i_lo);
  for (; i < i_hi; i += 2) {
    tile(std::false_type{}, std::integral_constant<int, 0>{}, i);
    tile(std::false_type{}, std::integral_constant<int, 1>{}, i + 1);
  }
  masked_pairs(i, n_qt);

  if (kok) {
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
      store_row_block<D>(dK + head_off + (size_t)key * D, acc_dk[ct], ct, h, scale);
      store_row_block<D>(dV + head_off + (size_t)key * D, acc_dv[ct], ct, h, 1.0f);
    }
  }
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

template <int D, bool CAUSAL>
void launch_bwd(const __bf16* q, const __bf16* k, const __bf16* v, const __bf16* o, const float* lse,
                const __bf16* dout, __bf16* dq, __bf16* dk, __bf16* dv, float* delta, int BH, int N,
                float scale, hipStream_t stream) {
  const float c_log2 = scale * kLog2e;
  const int nqb = (N + kQBlock - 1) / kQBlock;
  hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(BH * nqb)), dim3(kThreads), 0, stream,
                     q, k, v, dout, o, lse, delta, dq, BH, N, nqb, c_log2, scale);
  const int nkb = (N + kKBlock - 1) / kKBlock;
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(BH * nkb)), dim3(kKvThreads), 0, stream,
                     q, k, v, dout, lse, delta, dk, dv, BH, N, nkb, c_log2, scale);
}

}  // namespace

// Host checks shared by fa_bwd and fa_bwd_noalloc (delta == nullptr: the
// workspace is the library's own).  Returns FA_OK or an FA_ERR_* code; no
// HIP call.
static int check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, float* delta, bool own_delta, int B, int H,
                     int N, int d, float scale, int causal) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || (!own_delta && !delta)) return FA_ERR_NULL;
  if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (causal != 0 && causal != 1) return FA_ERR_FLAG;
  const long long bh = (long long)B * H;
  const long long blocks = bh * (((long long)N + kQBlock - 1) / kQBlock);
  const long long rows = bh * N;
  if (bh > 0x7fffffffLL || blocks * kThreads > 0xffffffffLL || rows > 0x7fffffffLL * 16LL ||
      (long long)N * d * 2 >= 0x80000000LL)
    return FA_ERR_SHAPE;
  if (own_delta && rows > FA_NOALLOC_ROWS) return FA_ERR_SCRATCH;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                        reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                        reinterpret_cast<uintptr_t>(dout) | reinterpret_cast<uintptr_t>(dq) |
                        reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv);
  if ((mis & 15u) != 0 || ((reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(delta)) & 3u) != 0)
    return FA_ERR_ALIGN;
  const size_t tb = (size_t)rows * d * 2, lb = (size_t)rows * 4;
  const void* ins[6] = {q, k, v, o, lse, dout};
  const size_t in_bytes[6] = {tb, tb, tb, tb, lb, tb};
  void* outs[4] = {dq, dk, dv, delta};
  const size_t out_bytes[4] = {tb, tb, tb, lb};
  const int n_outs = own_delta ? 3 : 4;
  for (int a = 0; a < n_outs; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlaps(outs[a], out_bytes[a], ins[b], in_bytes[b])) return FA_ERR_ALIAS;
    for (int b = a + 1; b < n_outs; ++b)
      if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

static void dispatch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int N,
                         int d, float scale, int causal, hipStream_t stream) {
  const int BHi = B * H;
  const __bf16* Q = static_cast<const __bf16*>(q);
  const __bf16* Kp = static_cast<const __bf16*>(k);
  const __bf16* Vp = static_cast<const __bf16*>(v);
  const __bf16* Op = static_cast<const __bf16*>(o);
  const __bf16* dOp = static_cast<const __bf16*>(dout);
  __bf16* dQp = static_cast<__bf16*>(dq);
  __bf16* dKp = static_cast<__bf16*>(dk);
  __bf16* dVp = static_cast<__bf16*>(dv);
  if (d == 128) {
    if (causal) launch_bwd<128, true>(Q, Kp, Vp, Op, lse, dOp, dQp, dKp, dVp, delta, BHi, N, scale, stream);
    else        launch_bwd<128, false>(Q, Kp, Vp, Op, lse, dOp, dQp, dKp, dVp, delta, BHi, N, scale, stream);
  } else {
    if (causal) launch_bwd<64, true>(Q, Kp, Vp, Op, lse, dOp, dQp, dKp, dVp, delta, BHi, N, scale, stream);
    else        launch_bwd<64, false>(Q, Kp, Vp, Op, lse, dOp, dQp, dKp, dVp, delta, BHi, N, scale, stream);
  }
}

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int N,
                      int d, float scale, int causal, hipStream_t stream) {
  const int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, false, B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  dispatch_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices];     // each device's address of `scratch`, looked up on first use
}  // namespace

// The address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
static int scratch_of_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return FA_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return FA_ERR_DEVICE;
    }
    g_scratch[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch[dev];
  return FA_OK;
}

extern "C" int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                              float scale, int causal, hipStream_t stream) {
  const int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, nullptr, true, B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  float* delta = nullptr;
  const int sd = scratch_of_current_device(&delta);
  if (sd != FA_OK) return sd;
  // D is overwritten by the first kernel before anything reads it: nothing to clear
  dispatch_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}
