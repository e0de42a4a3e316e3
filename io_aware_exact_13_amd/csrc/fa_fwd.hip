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
//   * Workgroup: 8 waves (two per SIMD) of 32 query rows each, 256 rows, at
//     d = 128; at d = 64, where the rings take 64 KiB of LDS, 4 waves and
//     128 rows, two workgroups per CU (their waves drift apart on the shared
//     SIMDs: 4% faster there).  K/V tiles of 64 keys.  K and V go HBM -> LDS with buffer_load ... lds
//     (no VGPR staging; the buffer's record count zero-fills rows past the
//     last key the workgroup can see), each through a ring of four LDS
//     buffers, copied two steps before use.  One workgroup barrier per tile.
//   * Each wave runs a three-stage software pipeline: in step j it issues,
//     as one interleaved instruction stream, the MFMAs of S_{j+1} = K_{j+1}
//     Q^T, those of O += V_{j-1} P_{j-1}, and the softmax of tile j
//     (S_j -> P_j), plus the copies of K_{j+3} and V_{j+1}.  The softmax VALU
//     work then issues under the wave's own MFMAs and the other wave's.
//   * The softmax works in base 2 with scale*log2(e) folded into one FMA
//     before v_exp_f32.  Any reference maximum gives the same acc / l, so
//     the reference lags the true row maximum: for d = 128 it moves only
//     when the tile's row maximum passes it by more than a slack (at most
//     kSlack = 2^8, and less while the new key's weight would exceed kShare
//     of the row's sum so far), so the accumulator rescale is skipped on
//     most tiles.  For d = 64, where the MFMA work per tile halves and the
//     softmax's VALU work does not, the first FA_D64_MAX_TILES tiles take the
//     row maximum and the rest do not form it: P is taken against the
//     current reference, and only if a lane's tile sum of P passes its limit
//     (kPMax = 2^32, or kShare of the lane's sum so far) does the wave redo
//     the tile with the true maximum.
//   * Workgroup order: workgroups are dealt round-robin to the 8 XCDs, each
//     with its own L2.  The block index is remapped so that an XCD walks
//     whole heads one after another: the workgroups running on it at any
//     time stream the same head's K/V through its L2.  Blocks that start
//     after a head's first batch re-read its K/V past the L2, so those reads
//     grow faster than N.  Under the causal mask a head's longest query
//     blocks launch first.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include <algorithm>
#include <functional>
#include <queue>
#include <vector>

#include "fa.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// Tile parameters are compile-time constants.  The defaults are the measured
// choice; a build may override them to measure another candidate (the
// library's own build does not).
#ifndef FA_WAVES_D128
#define FA_WAVES_D128 8
#endif
#ifndef FA_WAVES_D64
#define FA_WAVES_D64 4
#endif
#ifndef FA_OPERAND_AHEAD
#define FA_OPERAND_AHEAD 2
#endif
// VALU instructions of the softmax the scheduler places after each MFMA of a
// step (the rest follow the step's last MFMA).
#ifndef FA_VALU_PER_MFMA
#define FA_VALU_PER_MFMA 3
#endif
// Row groups per wave at d = 128: 1 (32 query rows per wave, 64-key tiles,
// two waves per SIMD), or 2 (64 rows per wave, 32-key tiles, one wave per
// SIMD with up to 512 registers a lane): each K or V operand read from LDS
// then feeds two MFMAs, which halves the LDS operand bytes per FLOP.
#ifndef FA_GROUPS_D128
#define FA_GROUPS_D128 1
#endif
static_assert(FA_GROUPS_D128 == 1 || FA_GROUPS_D128 == 2, "row groups per wave at d = 128");
template <int D> constexpr int kGroupsOf = D == 128 ? FA_GROUPS_D128 : 1;
template <int D> constexpr int kBCOf = kGroupsOf<D> == 2 ? 32 : 64;   // keys per K/V tile
template <int D> constexpr int kKbOf = kBCOf<D> / 32;                 // 32-key blocks per tile
template <int D> constexpr int kWavesPerSimdOf = kGroupsOf<D> == 2 ? 1 : 2;
// Waves per workgroup: 8 at d = 128 (one workgroup per CU, 128 KiB of LDS),
// 4 at d = 64 (64 KiB, two workgroups per CU, whose waves share the SIMDs
// and drift apart); 4 at d = 128 with two row groups per wave.
template <int D> constexpr int kWavesOf = D == 64 ? FA_WAVES_D64 : (FA_GROUPS_D128 == 2 ? 4 : FA_WAVES_D128);
static_assert(FA_WAVES_D128 == 4 || FA_WAVES_D128 == 8, "waves per workgroup at d = 128");
static_assert(FA_WAVES_D64 == 4 || FA_WAVES_D64 == 8, "waves per workgroup at d = 64");
template <int D> constexpr int kThreadsOf = kWavesOf<D> * 64;
template <int D> constexpr int kBROf = kWavesOf<D> * 32 * kGroupsOf<D>;   // query rows per workgroup
__host__ __device__ constexpr int keys_per_tile(int d) { return d == 64 ? kBCOf<64> : kBCOf<128>; }
__host__ __device__ constexpr int rows_per_block(int d) { return d == 64 ? kBROf<64> : kBROf<128>; }
__host__ __device__ constexpr int threads_per_block(int d) { return d == 64 ? kThreadsOf<64> : kThreadsOf<128>; }
constexpr int kXcds = 8;          // accelerator dies; workgroups are dealt to them round-robin
constexpr int kMaxSplits = 64;    // key ranges per query block in the split-KV forward

// Split-KV under the causal mask: query block b (0-based) sees about b + 1
// units of key tiles, and is cut into ceil((b + 1) / r) key ranges, so that
// ranges hold about r units each whatever the block.  causal_units(k, r) is
// the number of ranges of blocks 0 .. k-1: sum over i = 1 .. k of ceil(i / r)
// = r q (q + 1) / 2 + (q + 1)(k - q r) with q = k / r.
__host__ __device__ constexpr long long causal_units(long long k, long long r) {
  return r * (k / r) * (k / r + 1) / 2 + (k / r + 1) * (k % r);
}
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Reference maximum.  By default it lags the running row maximum (see
// softmax_tile and softmax_tile_lagged).  A build with FA_EXACT_MAX=1 keeps
// the reference at the running maximum itself, so the largest weight seen so
// far is exactly 1 (for measuring what the lag costs in accuracy and saves in
// time).
#ifndef FA_EXACT_MAX
#define FA_EXACT_MAX 0
#endif
// A build with FA_EXTRA_BARRIER=1 adds, after every step's LDS reads, a wait
// for all of the wave's memory operations and a workgroup barrier: slower,
// and its results must equal the default build's bit for bit (a race on the
// LDS rings would show as a difference).
#ifndef FA_EXTRA_BARRIER
#define FA_EXTRA_BARRIER 0
#endif
// The lag is bounded two ways.  (a) Size: P stays <= 2^kSlack (d = 128) and
// a lane's tile sum <= kPMax (d = 64).  (b) Share: a key whose weight against
// the lagging reference would exceed kShare of the row's sum so far moves
// the reference to the true maximum (FA_LAG_SHARE = 0 turns this off).  Every
// weight rounded to bf16 is then either <= 1 (at most the reference key's,
// which is exactly 1) or less than kShare of its row's final sum, so the
// rounding of one large weight adds at most 2^-8 kShare max|v| to |O|; with
// the true maximum itself as reference (the online softmax as written) the
// largest weight is 1 and exact.
#ifndef FA_LAG_SHARE
#define FA_LAG_SHARE 0.25f
#endif
constexpr float kPMax = 4294967296.0f;   // 2^32: largest tile sum of P a lane may reach before the reference moves
constexpr float kSlack = FA_EXACT_MAX ? 0.0f : 8.0f;    // log2 units the reference max may lag the true max
constexpr float kShare = FA_LAG_SHARE;   // largest share of the row's sum a lagged weight may take (0: no limit)
// d = 64 forms no row maximum on most tiles (softmax_tile_lagged), but the
// first FA_D64_MAX_TILES tiles of a workgroup's range take the row maximum
// (softmax_tile): there the row's sum is still small, so the share rule would
// make the no-maximum path recompute most tiles.
#ifndef FA_D64_MAX_TILES
#define FA_D64_MAX_TILES 8
#endif
// d = 128 on the same path as d = 64 (no row maximum past the first tiles)
#ifndef FA_NOMAX_D128
#define FA_NOMAX_D128 0
#endif

// LDS geometry: unpadded rows with XOR-swizzled 16-byte chunks, so a tile is
// exactly 16 KiB (d=128) and every wave copies the same number of 1 KiB
// pieces of it.  K: chunk c of row r sits at chunk c ^ fk(r); the 16
// consecutive rows of an A-operand fetch then cover all 64 banks.  V: the
// mask moves whole 64-byte column groups (fv(r) touches only the group bits),
// so the 4 rows of one transposed read land in 4 different bank groups.  Both
// masks depend on the row modulo 16, which a 32-row or 16-row step does not
// change.
template <int D>
struct Geom {
  static constexpr int kRowBytes = 2 * D;                   // one K or V row
  static constexpr int kChunks = kRowBytes / 16;            // 16-byte chunks per row
  static constexpr int kTile = kBCOf<D> * kRowBytes;        // one K or V tile
  static constexpr int kRing = 4;                           // LDS buffers per operand
  static constexpr int kLdsBytes = 2 * kRing * kTile;
  __host__ __device__ static constexpr int k_buf(int b) { return b * kTile; }            // K buffer b
  __host__ __device__ static constexpr int v_buf(int b) { return (kRing + b) * kTile; }  // V buffer b
  // V buffer b relative to the V region, whose start is folded into the
  // lanes' V read offsets so that every LDS read immediate stays below 64 KiB
  __host__ __device__ static constexpr int v_rel(int b) { return b * kTile; }
  static constexpr int kLoads = kTile / (kThreadsOf<D> * 16);    // 1 KiB copies per wave per tile
  static_assert(kLoads * kThreadsOf<D> * 16 == kTile, "tile not a whole number of wave copies");
  __host__ __device__ static constexpr int fk(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __host__ __device__ static constexpr int fv(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }
};

// One thread's share of the HBM -> LDS copy of a tile (buffer_load ... lds).
// Copy i of wave w fills the 1 KiB of LDS at base + (W i + w) KiB (W waves), lane t
// the 16 bytes at + 16 t, so each lane fetches the global chunk that the
// swizzle puts in its slot.  The swizzle of a slot's row does not depend on
// i, so copy i reads at the lane's offset plus i * W KiB.
template <int D, bool IS_V>
struct TileCopy {
  unsigned voff;

  __device__ __forceinline__ void init(int wave, int lane) {
    using G = Geom<D>;
    const int slot = wave * 64 + lane;
    const int row = slot / G::kChunks, pchunk = slot % G::kChunks;
    const int lchunk = pchunk ^ (IS_V ? G::fv(row) : G::fk(row));
    voff = (unsigned)(row * G::kRowBytes + lchunk * 16);
  }

  // Copy key rows [key0, key0 + kBCOf<D>) of one head into the LDS tile at `dst`.
  // The buffer runs from row key0 to row N: rows past the end read as zeros,
  // and a tile wholly past the end copies nothing but zeros (no branch).
  __device__ __forceinline__ void issue(const char* head, int key0, int n, char* dst, int wave, int i) const {
    using G = Geom<D>;
    // Device pass only: with the buffer-resource type in this template body,
    // clang's host pass drops the launch stubs of some kernel instances.
#if defined(__HIP_DEVICE_COMPILE__)
    const int rows = max(n - key0, 0);
    const char* base = head + (size_t)min(key0, n) * G::kRowBytes;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, rows * G::kRowBytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + (i * kWavesOf<D> + wave) * 1024), 16,
                                             voff + i * kWavesOf<D> * 1024, 0, 0, 0);
#endif
  }
};

// Wait until at most N of this wave's vector-memory operations are in
// flight (copies complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else static_assert(N == 2 || N == 4 || N == 8, "copies per step");
}

// Combine a per-lane value with the lane 32 apart using the gfx950
// cross-half swap (a VALU op; a shuffle would go through the LDS crossbar).
// After the swap of x with itself, the two results hold, in every lane, the
// values of lanes l % 32 and l % 32 + 32 -- in either order, which max and sum
// do not care about.
__device__ __forceinline__ float max_halves(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_elementwise_maximum(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Running state of one wave: 32 query rows, lane l owns row l % 32.
template <int D>
struct RowState {
  f32x16 acc[D / 32];   // O^T accumulators: lane holds column (r/4)*8 + 4h + r%4 of each 32-col tile
  float m_ref;          // reference max, log2 units of the scaled score
  float l_part;         // this lane's share of the exponential sum
  float slack;          // how far (log2 units) the tile maximum may pass m_ref before the reference moves
};

// The slack the share rule allows for a row whose exponential sum so far is
// l_row: the new maximum's weight 2^slack must stay <= kShare l_row, and
// <= 2^kSlack.  0 before the first key (l_row = 0: any finite maximum moves
// the reference).
__device__ __forceinline__ float share_slack(float l_row) {
  return fminf(kSlack, fmaxf(0.f, __builtin_amdgcn_logf(l_row) + __builtin_log2f(kShare)));
}

// Register sets of one pipeline stage, per row group g of the wave: the S^T
// accumulators of a tile, P^T as bf16 B operands, and Q^T.
template <int D> using SSet = f32x16[kGroupsOf<D>][kKbOf<D>];
template <int D> using PSet = bf16x8[kGroupsOf<D>][kBCOf<D> / 16];
template <int D> using QSet = bf16x8[kGroupsOf<D>][D / 16];

// S^T = K Q^T for one tile (fp32, unscaled) for each row group, not
// overlapped with anything (used once, for S_0).  A operand: K row
// 32 kb + l32, columns 16 ks + 8 h .. +7; B operand: Q^T from registers.
template <int D>
__device__ __forceinline__ void scores(const char* Kt, const int (&k_off)[D / 16], const QSet<D>& qf, SSet<D>& s) {
  using G = Geom<D>;
#pragma unroll
  for (int kb = 0; kb < kKbOf<D>; ++kb) {
    bf16x8 a[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      a[ks] = *reinterpret_cast<const bf16x8*>(Kt + k_off[ks] + kb * 32 * G::kRowBytes);
#pragma unroll
    for (int g = 0; g < kGroupsOf<D>; ++g) {
      s[g][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], qf[g][0], f32x16{}, 0, 0, 0);
#pragma unroll
      for (int ks = 1; ks < D / 16; ++ks)
        s[g][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], qf[g][ks], s[g][kb], 0, 0, 0);
    }
  }
}

// Transposed read of the V^T operand for P V k-step t, column tile ct: lane
// a of each 16-lane group points at row a/4 of a 4-row group, columns
// cbase + 4(a%4), and receives column cbase + a of the 4 rows; the two
// reads cover keys 16t + 4h + {0..3} and 16t + 8 + 4h + {0..3}, the keys the
// lane's half holds in the S^T accumulator layout.
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const char* Vt, int v_off_ct, int t) {
  using G = Geom<D>;
  const char* p = Vt + v_off_ct + t * 16 * G::kRowBytes;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 8 * G::kRowBytes));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Online-softmax update for one tile: mask, row max, reference-max update,
// P = exp2(S * c - m) in bf16, row sum in fp32.  Returns alpha, the factor
// the accumulators must be multiplied by (1 unless the reference moved), and
// sets *rescale when some lane of the wave needs it.
//
// The slack follows the share rule (kShare): it is set from the row's sum at
// REFRESH steps (the first of every four) and drops to 0 for a row whose
// reference moved, until the next refresh.  The row's sum only grows while
// the reference stays, so a slack taken from an earlier, smaller sum is
// still within the rule.
template <int D, bool MASKED, bool REFRESH>
__device__ __forceinline__ float softmax_tile(f32x16 (&s)[kKbOf<D>], int key0, int lim, int h, float c_log2,
                                              RowState<D>& st, bf16x8 (&pf)[kBCOf<D> / 16], bool* rescale) {
  constexpr int kKb = kKbOf<D>;
  if (MASKED) {
    // register r of block kb holds key key0 + 4 h + (32 kb + 8 (r / 4) + r % 4),
    // visible while that offset is <= room: one compare per score
    const int room = lim - key0 - 4 * h;
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + (r >> 2) * 8 + (r & 3) > room) s[kb][r] = -INFINITY;
  }
  // row max: a three-way tree over this lane's 16 kKb scores (v_max3),
  // then the other half's
  float part[16 * kKb];
#pragma unroll
  for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) part[kb * 16 + r] = s[kb][r];
  int n = 16 * kKb;
#pragma unroll
  for (int round = 0; round < 6; ++round) {
    if (n <= 1) break;
    const int m = (n + 2) / 3;
#pragma unroll
    for (int r = 0; r < m; ++r) {
      const float a = part[3 * r];
      const float b = 3 * r + 1 < n ? part[3 * r + 1] : a;
      const float c = 3 * r + 2 < n ? part[3 * r + 2] : a;
      part[r] = __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
    }
    n = m;
  }
  const float m_tile = max_halves(part[0]) * c_log2;
  // the reference moves when the tile's maximum passes it by more than the
  // slack: kSlack, or (share rule) so much that the new maximum's weight
  // 2^(m_tile - m_ref) would pass kShare of the row's sum
  constexpr bool kRule = kShare > 0.f && !FA_EXACT_MAX;
  if constexpr (kRule && REFRESH) st.slack = share_slack(sum_halves(st.l_part));
  const bool grow = m_tile > st.m_ref + (kRule ? st.slack : kSlack);
  if constexpr (kRule) st.slack = grow ? 0.f : st.slack;
  const float m_new = grow ? m_tile : st.m_ref;
  *rescale = __builtin_amdgcn_ballot_w64(grow) != 0;
  // 0 while the row has seen no key (acc and l are still 0): no exp2 of
  // (-inf) - (-inf) when this tile shows it none either
  const float alpha = (st.m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m_ref - m_new);
  st.m_ref = m_new;
  const float neg_m = (m_new == -INFINITY) ? 0.f : -m_new;
  // P is summed in fp32 (the logsumexp needs the unrounded weights) and
  // rounded to bf16 for the MFMA.
  float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c_log2, neg_m));
      l4[r & 3] += p;
      pf[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
    }
  st.l_part = st.l_part * alpha + ((l4[0] + l4[1]) + (l4[2] + l4[3]));
  // Materialise P and the statistics here: without these empty asm uses the
  // compiler sinks the exponentials into the next step, next to the MFMAs
  // that consume them, where they would no longer overlap this step's MFMAs.
#pragma unroll
  for (int t = 0; t < kBCOf<D> / 16; ++t) asm volatile("" : "+v"(pf[t]));
  asm volatile("" : "+v"(st.l_part), "+v"(st.m_ref));
  return alpha;
}

// P = exp2(S c + neg_m) for one tile, rounded to bf16 for the MFMA; returns
// this lane's share of the tile's row sum, taken over the fp32 P (the
// logsumexp needs the unrounded weights).
template <int D>
__device__ __forceinline__ float exp_tile(const f32x16 (&s)[kKbOf<D>], float c_log2, float neg_m,
                                          bf16x8 (&pf)[kBCOf<D> / 16]) {
  float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < kKbOf<D>; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c_log2, neg_m));
      l4[r & 3] += p;
      pf[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
    }
  return (l4[0] + l4[1]) + (l4[2] + l4[3]);
}

// Online softmax of one tile against the current reference maximum, without
// a row maximum (the d = 64 path): any reference gives the same acc / l, so
// the reference is only moved when keeping it would let P grow past kPMax.  The lane's tile
// sum bounds every P it holds, so one compare per lane detects that (and
// catches the first tile, where the reference is -inf and P is inf or NaN).
// Returns whether some lane of the wave must redo the tile with a new
// reference (softmax_redo); *lt receives this lane's tile sum.
template <int D, bool MASKED>
__device__ __forceinline__ bool softmax_tile_lagged(f32x16 (&s)[kKbOf<D>], int key0, int lim, int h, float c_log2,
                                                    float m_ref, float l_part, bf16x8 (&pf)[kBCOf<D> / 16],
                                                    float* lt) {
  constexpr int kKb = kKbOf<D>;
  if (MASKED) {
    // register r of block kb holds key key0 + 4 h + (32 kb + 8 (r / 4) + r % 4),
    // visible while that offset is <= room: one compare per score
    const int room = lim - key0 - 4 * h;
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + (r >> 2) * 8 + (r & 3) > room) s[kb][r] = -INFINITY;
  }
  float sum = exp_tile<D>(s, c_log2, -m_ref, pf);
  // Materialise P and the sum here: without these empty asm uses the
  // compiler sinks the exponentials into the next step, next to the MFMAs
  // that consume them, where they would no longer overlap this step's MFMAs.
#pragma unroll
  for (int t = 0; t < kBCOf<D> / 16; ++t) asm volatile("" : "+v"(pf[t]));
  asm volatile("" : "+v"(sum));
  *lt = sum;
  // accepted: every P of the lane is <= its tile sum, which is <= 1 (no
  // weight above the reference key's) or <= kShare of the lane's share of
  // the row's sum so far, and <= kPMax
  float limit = kPMax;
  if constexpr (kShare > 0.f) limit = fminf(kPMax, fmaxf(1.f, kShare * l_part));
  return __builtin_amdgcn_ballot_w64(!(sum <= limit)) != 0;
}

// The rare path of softmax_tile: the row maximum of the (masked) tile, the
// reference moved up to it where it is larger, and P recomputed.  Returns
// alpha = exp2(m_old - m_new), the factor for the running sum and the
// accumulators (0 on the first tile, 1 where the reference stays).
template <int D>
__device__ __forceinline__ float softmax_redo(const f32x16 (&s)[kKbOf<D>], float c_log2, RowState<D>& st,
                                              bf16x8 (&pf)[kBCOf<D> / 16], float* lt) {
  constexpr int kKb = kKbOf<D>;
  // row max: a three-way tree over this lane's 16 kKb scores, then the other
  // half's.  The IEEE maximum (NaN-propagating) maps to v_maximum3_f32 and,
  // unlike fmaxf, needs no canonicalising moves of the MFMA results.
  float part[16 * kKb];
#pragma unroll
  for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) part[kb * 16 + r] = s[kb][r];
  int n = 16 * kKb;
#pragma unroll
  for (int round = 0; round < 6; ++round) {
    if (n <= 1) break;
    const int m = (n + 2) / 3;
#pragma unroll
    for (int r = 0; r < m; ++r) {
      const float a = part[3 * r];
      const float b = 3 * r + 1 < n ? part[3 * r + 1] : a;
      const float c = 3 * r + 2 < n ? part[3 * r + 2] : a;
      part[r] = __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
    }
    n = m;
  }
  const float m_tile = max_halves(part[0]) * c_log2;
  const float m_new = fmaxf(st.m_ref, m_tile);
  const float alpha = (m_new == st.m_ref) ? 1.f : __builtin_amdgcn_exp2f(st.m_ref - m_new);
  st.m_ref = m_new;
  *lt = exp_tile<D>(s, c_log2, (m_new == -INFINITY) ? 0.f : -m_new, pf);
  return alpha;
}

// Everything a pipeline step needs besides the running state.
template <int D>
struct Ctx {
  const char* Kh;
  const char* Vh;
  char* lds;
  int N, kv_end, n_tiles, wave, h;
  int lim[kGroupsOf<D>];   // last key each of the lane's rows (one per row group) may see
  float c_log2;
  int k_off[D / 16];    // lane's LDS offset of its K operand for k-step ks (32-row block 0)
  int v_off[D / 32];    // lane's LDS offset of its first transposed V read for column tile ct
  TileCopy<D, false> kcopy;
  TileCopy<D, true> vcopy;
};

// One pipeline step, iteration j.  In flight on entry: S_j (fp32, in s_in)
// and P_{j-1} (bf16, in p_in); K_{j+1} and V_{j-1} have landed in LDS (their
// copies went out two steps earlier).  The step
//   - starts the copies of K_{j+3} (into K_{j-1}'s buffer) and V_{j+1} (into
//     V_{j-3}'s buffer), read two steps later;
//   - runs, as one interleaved instruction stream, the MFMAs of
//     S_{j+1} = K_{j+1} Q^T and of O += V_{j-1} P_{j-1} together with the
//     softmax of tile j (S_j -> P_j): the wave's own VALU work issues in the
//     shadow of its MFMAs;
//   - if the reference maximum moved, multiplies O by alpha_j after the
//     O += V_{j-1} P_{j-1} products (O must not yet hold tile j).
// The LDS buffers read and the ones being filled are distinct restrict
// pointers: the compiler then keeps the copies in flight across the reads
// (the next step's explicit wait orders them).
template <int D, bool MASKED, bool NOMAX, bool REFRESH>
__device__ __forceinline__ void step(const char* __restrict__ k_read, const char* __restrict__ v_read,
                                     char* __restrict__ k_fill, char* __restrict__ v_fill, const Ctx<D>& c,
                                     int j, const QSet<D>& qf, SSet<D>& s_in, SSet<D>& s_out, const PSet<D>& p_in,
                                     PSet<D>& p_out, RowState<D> (&st)[kGroupsOf<D>]) {
  using G = Geom<D>;
  constexpr int kG = kGroupsOf<D>, kBC = kBCOf<D>;
  constexpr int kCt = D / 32, kKs = kBC / 16, kKb = kKbOf<D>, kDs = D / 16;
  constexpr int kPV = kKs * kCt;        // P V operand reads: (t, ct), ct fastest
  constexpr int kS = kDs * kKb;         // S operand reads: (ks, kb), kb fastest
  static_assert(kPV == kS, "P V and S operand reads are interleaved one to one");
  constexpr int kAhead = FA_OPERAND_AHEAD;   // operand pairs requested ahead

  // this wave's copies of K_{j+1}, V_{j-1} (issued two steps ago; the
  // previous step's copies may still be in flight) ...
  wait_vmcnt<2 * G::kLoads>();
  __builtin_amdgcn_s_barrier();                      // ... and everyone's; j-1's reads done
  __builtin_amdgcn_sched_barrier(0);

  // Read i: P V product (t, ct) with t fastest, S product (ks, kb) with ks
  // fastest, so reads 2m and 2m + 1 accumulate into one block each.  Each
  // accumulator still sums its k-steps in ascending order.
  bf16x8 v_op[kPV], k_op[kS];
  auto pv_index = [](int i, int& t, int& ct) { t = i % kKs; ct = i / kKs; };
  auto s_index = [](int i, int& ks, int& kb) { ks = i % kDs; kb = i / kDs; };
  auto fetch = [&](int i) {             // operands of P V read i and S read i
    int t, ct, ks, kb;
    pv_index(i, t, ct);
    v_op[i] = v_operand<D>(v_read, c.v_off[ct], t);
    s_index(i, ks, kb);
    k_op[i] = *reinterpret_cast<const bf16x8*>(k_read + c.k_off[ks] + kb * 32 * G::kRowBytes);
  };
  // each operand feeds one MFMA per row group
  auto mfma_pv = [&](int i) {
    int t, ct;
    pv_index(i, t, ct);
#pragma unroll
    for (int g = 0; g < kG; ++g)
      st[g].acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_op[i], p_in[g][t], st[g].acc[ct], 0, 0, 0);
  };
  auto mfma_s = [&](int i) {
    int ks, kb;
    s_index(i, ks, kb);
#pragma unroll
    for (int g = 0; g < kG; ++g)
      s_out[g][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_op[i], qf[g][ks], ks == 0 ? f32x16{} : s_out[g][kb],
                                                             0, 0, 0);
  };
  static_assert(kKs % 2 == 0 && kDs % 2 == 0, "reads go in pairs that share an accumulator");
  // The copies go out between the MFMAs: a copy instruction holds up its
  // wave for tens of cycles at issue, which the MFMAs already in the pipe
  // cover.
  constexpr int kCopies = 2 * G::kLoads;
  constexpr int kCopyEvery = kPV / kCopies;
  static_assert(kCopyEvery >= 2 && kCopyEvery * kCopies == kPV, "copies spread over the step's MFMA pairs");
  auto copy = [&](int q) {
    if (q < G::kLoads) c.kcopy.issue(c.Kh, (j + 3) * kBC, c.kv_end, k_fill, c.wave, q);
    else c.vcopy.issue(c.Vh, (j + 1) * kBC, c.kv_end, v_fill, c.wave, q - G::kLoads);
  };
  // Issue order per pair of reads: both P V products (back to back on one
  // accumulator), then both S products (likewise).  Against alternating the
  // two kinds read by read, the chip runs this order about 0.7% faster at the
  // same results; the MFMA unit forwards a result to the next instruction
  // that accumulates onto it.
#pragma unroll
  for (int i = 0; i < kAhead; ++i) fetch(i);
#pragma unroll
  for (int i = 0; i < kPV; i += 2) {
    if (i + kAhead < kPV) fetch(i + kAhead);
    if (i + 1 + kAhead < kPV) fetch(i + 1 + kAhead);
    mfma_pv(i);
    mfma_pv(i + 1);
    mfma_s(i);
    mfma_s(i + 1);
    if (i % kCopyEvery == 1 || (i + 1) % kCopyEvery == 1) copy((i + 1) / kCopyEvery);
  }
  // NOMAX (d = 64 past its first tiles): the lagged reference without a row
  // maximum (about 5% faster there; no gain for d = 128, whose MFMA work per
  // tile hides the max tree)
  constexpr bool kNoMax = NOMAX && !FA_EXACT_MAX;
  bool rescale[kG];
  float alpha[kG], lt[kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    rescale[g] = false;
    alpha[g] = 1.f;
    lt[g] = 0.f;
    if constexpr (kNoMax)
      rescale[g] = softmax_tile_lagged<D, MASKED>(s_in[g], j * kBC, c.lim[g], c.h, c.c_log2, st[g].m_ref,
                                                  st[g].l_part, p_out[g], &lt[g]);
    else
      alpha[g] = softmax_tile<D, MASKED, REFRESH>(s_in[g], j * kBC, c.lim[g], c.h, c.c_log2, st[g], p_out[g],
                                                  &rescale[g]);
  }
  // Interleave: each operand pair is 2 kG MFMAs, its operand reads and an
  // equal share of the softmax's VALU work between and after them (mask
  // 0x008 MFMA, 0x100 LDS read, 0x002 VALU, 0x010 VMEM).
  __builtin_amdgcn_sched_group_barrier(0x100, 3 * kAhead, 0);
#pragma unroll
  for (int i = 0; i < kPV; ++i) {
    if (i + kAhead < kPV) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int m = 0; m < 2 * kG; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m == 2 * kG - 1 && i % kCopyEvery == 1) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, FA_VALU_PER_MFMA, 0);
    }
  }
  if constexpr (FA_EXTRA_BARRIER) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    if constexpr (kNoMax) {
      if (rescale[g]) {
        alpha[g] = softmax_redo<D>(s_in[g], c.c_log2, st[g], p_out[g], &lt[g]);
        st[g].l_part *= alpha[g];
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
          for (int r = 0; r < 16; ++r) st[g].acc[ct][r] *= alpha[g];
      }
      st[g].l_part += lt[g];
    } else if (rescale[g]) {
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[g].acc[ct][r] *= alpha[g];
    }
  }
}

// Four steps, one turn of the LDS rings, S/P register sets swapped between
// steps.  Step j reads K_{j+1} from K buffer (j+1)%4 and V_{j-1} from V
// buffer (j-1)%4, and fills K buffer (j+3)%4 and V buffer (j+1)%4.
// The share rule's slack is refreshed at the first step of every four.
template <int D, bool MASKED, int PH, bool NOMAX = false>
__device__ __forceinline__ void step_at(const Ctx<D>& c, int j, const QSet<D>& qf, SSet<D>& sa, SSet<D>& sb,
                                        PSet<D>& pa, PSet<D>& pb, RowState<D> (&st)[kGroupsOf<D>]) {
  using G = Geom<D>;
  constexpr int R = G::kRing;
  if constexpr (PH % 2 == 0)
    step<D, MASKED, NOMAX, PH == 0>(c.lds + G::k_buf((PH + 1) % R), c.lds + G::v_rel((PH + R - 1) % R),
                                    c.lds + G::k_buf((PH + 3) % R), c.lds + G::v_buf((PH + 1) % R), c, j, qf, sa,
                                    sb, pa, pb, st);
  else
    step<D, MASKED, NOMAX, PH == 0>(c.lds + G::k_buf((PH + 1) % R), c.lds + G::v_rel((PH + R - 1) % R),
                                    c.lds + G::k_buf((PH + 3) % R), c.lds + G::v_buf((PH + 1) % R), c, j, qf, sb,
                                    sa, pb, pa, st);
}

template <int D, bool MASKED, bool NOMAX = false>
__device__ __forceinline__ void step_quad(const Ctx<D>& c, int j, const QSet<D>& qf, SSet<D>& sa, SSet<D>& sb,
                                          PSet<D>& pa, PSet<D>& pb, RowState<D> (&st)[kGroupsOf<D>]) {
  step_at<D, MASKED, 0, NOMAX>(c, j, qf, sa, sb, pa, pb, st);
  step_at<D, MASKED, 1, NOMAX>(c, j + 1, qf, sa, sb, pa, pb, st);
  step_at<D, MASKED, 2, NOMAX>(c, j + 2, qf, sa, sb, pa, pb, st);
  step_at<D, MASKED, 3, NOMAX>(c, j + 3, qf, sa, sb, pa, pb, st);
}

// SPLIT: the workgroup covers one contiguous range of its query block's
// visible key tiles and writes an fp32 partial (O_s = acc / l over its keys,
// LSE_s) to Opart / Lpart ([n_splits][B*H][N][d], [n_splits][B*H][N]);
// fa_merge_kernel combines them.  Without the mask every block has n_splits
// ranges; under it, with r_units > 0, block b has ceil((b + 1) / r_units)
// (causal_units), the longest blocks' ranges first.  Otherwise the workgroup
// covers all the tiles and writes O (bf16) and LSE.
template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(kThreadsOf<D>) __attribute__((amdgpu_waves_per_eu(kWavesPerSimdOf<D>, kWavesPerSimdOf<D>)))
void fa_fwd_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                   const __bf16* __restrict__ V, __bf16* __restrict__ O, float* __restrict__ LSE,
                   float* __restrict__ Opart, float* __restrict__ Lpart,
                   int BH, int N, int n_qblocks, int n_splits, int r_units, float c_log2) {
  using G = Geom<D>;
  constexpr int kDs = D / 16;
  constexpr int kCt = D / 32;
  constexpr int kG = kGroupsOf<D>;
  constexpr int kBC = kBCOf<D>;

  __shared__ __attribute__((aligned(1024))) char lds[G::kLdsBytes];

  Ctx<D> c;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  c.h = lane >> 5;                  // which half of the 64 lanes
  const int l32 = lane & 31;        // this lane's query row within each 32-row group

  // ---- workgroup -> (head, query block).  Workgroups are dealt round-robin
  // to the 8 XCDs; the logical index gives each XCD a contiguous run of whole
  // heads, walked head by head, so the XCD's running workgroups share one
  // head's K/V stream in its L2.
  const int wg = blockIdx.x;
  const bool kUnits = SPLIT && CAUSAL && r_units > 0;   // ranges in proportion to the block's length
  const int per_head = kUnits ? (int)causal_units(n_qblocks, r_units) : n_qblocks * (SPLIT ? n_splits : 1);
  const int n_wg = BH * per_head;
  const int logical = (n_wg % kXcds == 0) ? (wg % kXcds) * (n_wg / kXcds) + wg / kXcds : wg;
  const int bh = logical / per_head;
  int qb, split = 0, n_ranges = SPLIT ? n_splits : 1;
  if (kUnits) {
    // the w-th range of the head in block order, counted from the last
    // (longest) block: the largest qb with causal_units(qb) <= w
    const int w = per_head - 1 - logical % per_head;
    int lo = 0, hi = n_qblocks;
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (causal_units(mid, r_units) <= w) lo = mid;
      else hi = mid;
    }
    qb = lo;
    split = w - (int)causal_units(qb, r_units);
    n_ranges = (qb + r_units) / r_units;
  } else {
    const int qi = SPLIT ? (logical % per_head) / n_splits : logical % per_head;
    split = SPLIT ? (logical % per_head) % n_splits : 0;
    qb = CAUSAL ? (n_qblocks - 1 - qi) : qi;
  }
  constexpr int kBR = kBROf<D>;
  const int q0 = qb * kBR;
  // this lane's queries: row l32 of each of the wave's 32-row groups
  int qrow[kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    qrow[g] = q0 + (c.wave * kG + g) * 32 + l32;
    c.lim[g] = CAUSAL ? min(qrow[g], N - 1) : N - 1;   // last key the row may see
  }
  c.N = N;
  c.c_log2 = c_log2;
  c.lds = lds;

  const size_t head_off = (size_t)bh * (size_t)N * D;
  c.Kh = reinterpret_cast<const char*>(K + head_off);
  c.Vh = reinterpret_cast<const char*>(V + head_off);

  // ---- key tiles: every wave walks the workgroup's n_tiles (under the causal
  // mask, tiles wholly past a wave's rows are masked out by its softmax).
  const int kv_end = CAUSAL ? min(N, q0 + kBR) : N;
  const int all_tiles = (kv_end + kBC - 1) / kBC;
  // this workgroup's tiles [j0, n_tiles): all of them, or one split's share
  const int j0 = SPLIT ? (int)((long long)split * all_tiles / n_ranges) : 0;
  c.n_tiles = SPLIT ? (int)((long long)(split + 1) * all_tiles / n_ranges) : all_tiles;
  c.kv_end = min(kv_end, c.n_tiles * kBC);              // copies past it read zeros, no traffic
  // tiles from j_mask on hold keys past the end or past some query of the block
  int j_mask = N / kBC;                                 // the first tile holding a key >= N
  if (CAUSAL) j_mask = min(j_mask, q0 / kBC);           // first tile with a key > q0
  j_mask = min(j_mask, c.n_tiles);
  const size_t prow = ((size_t)split * BH + bh) * (size_t)N;   // partial row base (SPLIT)
  if (SPLIT && j0 == c.n_tiles) {                       // an empty share: O_s = 0, LSE_s = -inf
#pragma unroll
    for (int g = 0; g < kG; ++g)
      if (qrow[g] < N) {
        float* op = Opart + (prow + qrow[g]) * D;
#pragma unroll
        for (int t = 0; t < D / 8; ++t) *reinterpret_cast<f32x4*>(op + 8 * t + 4 * c.h) = f32x4{0.f, 0.f, 0.f, 0.f};
        if (c.h == 0) Lpart[prow + qrow[g]] = -INFINITY;
      }
    return;
  }

  // ---- per-lane offsets
#pragma unroll
  for (int ks = 0; ks < kDs; ++ks)
    c.k_off[ks] = l32 * G::kRowBytes + (((2 * ks + c.h) ^ G::fk(l32)) << 4);
  {
    const int a = lane & 15, cg = (lane >> 4) & 1;
    const int row = 4 * c.h + (a >> 2);
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct)
      c.v_off[ct] = G::v_buf(0) + row * G::kRowBytes + (((4 * ct + 2 * cg + ((a & 3) >> 1)) ^ G::fv(row)) << 4) +
                    8 * (a & 1);
  }
  c.kcopy.init(c.wave, lane);
  c.vcopy.init(c.wave, lane);

  // ---- prologue: K_0 and K_1 in flight while Q is fetched; V buffer 1 (read
  // as "V_{-1}" by step 0, with P_{-1} = 0) is zero-filled.
#pragma unroll
  for (int i = 0; i < G::kLoads; ++i) {
    c.kcopy.issue(c.Kh, j0 * kBC, c.kv_end, lds + G::k_buf(0), c.wave, i);
    c.kcopy.issue(c.Kh, (j0 + 1) * kBC, c.kv_end, lds + G::k_buf(1), c.wave, i);
  }
#pragma unroll
  for (int i = 0; i < G::kLoads; ++i) {   // the copies step j0+1 waits for: K_{j0+2} and V_{j0}
    c.kcopy.issue(c.Kh, (j0 + 2) * kBC, c.kv_end, lds + G::k_buf(2), c.wave, i);
    c.vcopy.issue(c.Vh, j0 * kBC, c.kv_end, lds + G::v_buf(0), c.wave, i);
  }
  for (int i = tid; i < G::kTile / 8; i += kThreadsOf<D>)   // V_{-1} = 0
    reinterpret_cast<u32x2*>(lds + G::v_buf(G::kRing - 1))[i] = u32x2{0u, 0u};

  // Q^T operand: lane holds Q[qrow[g]][16*ks + 8*h .. +7] for each k-step
  QSet<D> qf;
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const bool ok = qrow[g] < N;
    const bf16x8* src = reinterpret_cast<const bf16x8*>(Q + head_off + (size_t)(ok ? qrow[g] : 0) * D);
#pragma unroll
    for (int ks = 0; ks < kDs; ++ks) {
      bf16x8 x = src[ks * 2 + c.h];
      if (!ok) x = bf16x8{};
      qf[g][ks] = x;
    }
  }

  RowState<D> st[kG];
  SSet<D> sa, sb;
  PSet<D> pa, pb;
#pragma unroll
  for (int g = 0; g < kG; ++g) {
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) st[g].acc[ct] = f32x16{};
    st[g].m_ref = -INFINITY;
    st[g].l_part = 0.f;
    st[g].slack = 0.f;
#pragma unroll
    for (int t = 0; t < kBC / 16; ++t) pa[g][t] = bf16x8{};
  }

  wait_vmcnt<2 * G::kLoads>();                          // K_0, K_1
  __syncthreads();
  scores<D>(lds + G::k_buf(0), c.k_off, qf, sa);       // S_{j0}

  // ---- main loop, four steps per trip so the LDS ring positions (tile
  // j - j0 modulo 4) are constants
  int j = j0;
  const int j_fast = max(j0, j_mask);                   // tiles [j0, j_fast) need no mask
  // d = 64: the row maximum on the first FA_D64_MAX_TILES tiles, none after
  constexpr bool kNoMax = D == 64 || FA_NOMAX_D128;
  if constexpr (kNoMax) {
    const int j_max = min(j_fast, j0 + FA_D64_MAX_TILES);
    for (; j + 4 <= j_max; j += 4) step_quad<D, false, false>(c, j, qf, sa, sb, pa, pb, st);
  }
  for (; j + 4 <= j_fast; j += 4) step_quad<D, false, kNoMax>(c, j, qf, sa, sb, pa, pb, st);
  for (; j + 4 <= c.n_tiles; j += 4) step_quad<D, true, kNoMax>(c, j, qf, sa, sb, pa, pb, st);
  if (j < c.n_tiles) step_at<D, true, 0, kNoMax>(c, j++, qf, sa, sb, pa, pb, st);
  if (j < c.n_tiles) step_at<D, true, 1, kNoMax>(c, j++, qf, sa, sb, pa, pb, st);
  if (j < c.n_tiles) step_at<D, true, 2, kNoMax>(c, j++, qf, sa, sb, pa, pb, st);
  // ---- O += V_{n-1} P_{n-1}: V_{n-1} is in ring buffer (n-1-j0) % 4
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  {
    const int last = c.n_tiles - 1 - j0;
    const char* vt = lds + G::v_rel(last % G::kRing);
    const PSet<D>& pl = ((last + 1) & 1) ? pb : pa;
#pragma unroll
    for (int t = 0; t < kBC / 16; ++t)
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct) {
        const bf16x8 vop = v_operand<D>(vt, c.v_off[ct], t);
#pragma unroll
        for (int g = 0; g < kG; ++g)
          st[g].acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pl[g][t], st[g].acc[ct], 0, 0, 0);
      }
  }

  // ---- epilogue: O = acc / l (bf16), LSE = (m_ref + log2 l) * ln 2
  float l_tot[kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) l_tot[g] = sum_halves(st[g].l_part);
  if (SPLIT) {
    // fp32 partial; a row with no visible key in this share has l = 0
#pragma unroll
    for (int g = 0; g < kG; ++g)
      if (qrow[g] < N) {
        const float inv = l_tot[g] > 0.f ? 1.0f / l_tot[g] : 0.f;
        float* op = Opart + (prow + qrow[g]) * D;
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            *reinterpret_cast<f32x4*>(op + ct * 32 + r4 * 8 + c.h * 4) =
                f32x4{st[g].acc[ct][r4 * 4] * inv, st[g].acc[ct][r4 * 4 + 1] * inv,
                      st[g].acc[ct][r4 * 4 + 2] * inv, st[g].acc[ct][r4 * 4 + 3] * inv};
        if (c.h == 0)
          Lpart[prow + qrow[g]] = l_tot[g] > 0.f ? (st[g].m_ref + log2f(l_tot[g])) * kLn2 : -INFINITY;
      }
    return;
  }
  // O = acc / l in bf16, staged group by group through this wave's 32-row
  // slice of the K ring (idle since the barrier above: every K read and copy
  // has finished) so that the stores to HBM are whole rows, 16 bytes a lane:
  // a lane's own accumulators hold 8-byte pieces of one row, which stored
  // directly touch 32 rows per instruction.  Chunk ch of staged row r sits at
  // 16-byte slot ch ^ (r % kChunks) of the row, so the 32 rows written by one
  // instruction spread over the banks.
  {
    constexpr int kChunks = G::kChunks;
    static_assert(kWavesOf<D> * 32 * G::kRowBytes <= G::kRing * G::kTile, "staging fits the K ring");
    char* stage = lds + G::k_buf(0) + c.wave * 32 * G::kRowBytes;
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      // the previous group's read-back has returned before its slots are rewritten
      if (g > 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const float inv = qrow[g] < N ? 1.0f / l_tot[g] : 0.f;
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const __bf16 b0 = (__bf16)(st[g].acc[ct][r4 * 4 + 0] * inv);
          const __bf16 b1 = (__bf16)(st[g].acc[ct][r4 * 4 + 1] * inv);
          const __bf16 b2 = (__bf16)(st[g].acc[ct][r4 * 4 + 2] * inv);
          const __bf16 b3 = (__bf16)(st[g].acc[ct][r4 * 4 + 3] * inv);
          u32x2 w;
          w[0] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
          w[1] = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
          // columns ct*32 + r4*8 + 4h .. +3: chunk 4ct + r4, half h
          const int ch = ct * 4 + r4;
          *reinterpret_cast<u32x2*>(stage + l32 * G::kRowBytes + ((ch ^ (l32 % kChunks)) << 4) + 8 * c.h) = w;
        }
      // the wave reads back what its other lanes wrote: wait for the writes
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int row0 = q0 + (c.wave * kG + g) * 32;
#pragma unroll
      for (int i = 0; i < kChunks / 2; ++i) {
        const int q = i * 64 + lane, r = q / kChunks, ch = q % kChunks;
        const u32x4 val = *reinterpret_cast<const u32x4*>(stage + r * G::kRowBytes + ((ch ^ (r % kChunks)) << 4));
        if (row0 + r < N) *reinterpret_cast<u32x4*>(O + head_off + (size_t)(row0 + r) * D + ch * 8) = val;
      }
    }
  }
#pragma unroll
  for (int g = 0; g < kG; ++g)
    if (qrow[g] < N && c.h == 0) LSE[(size_t)bh * N + qrow[g]] = (st[g].m_ref + log2f(l_tot[g])) * kLn2;
}

// Merge of n_splits partial results of the same rows over disjoint key
// ranges: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.  This
// is the two-block merge of the online softmax ("为什么Flash Attention能将注意力
// 计算提速数倍而不损失精度", 在线Softmax技巧) applied to n blocks at once, with
// the blocks' statistics folded into their logsumexps.  D/8 lanes per row,
// 8 columns each.  With r_units > 0 (under the causal mask) a row of query
// block b has ceil((b + 1) / r_units) partials, else n_splits.
template <int D>
__global__ __launch_bounds__(256) void fa_merge_kernel(const float* __restrict__ Opart,
                                                       const float* __restrict__ Lpart, __bf16* __restrict__ O,
                                                       float* __restrict__ LSE, long long rows, int N,
                                                       int n_splits, int r_units) {
  constexpr int kLanes = D / 8;
  constexpr int kRows = 256 / kLanes;
  const long long row = (long long)blockIdx.x * kRows + threadIdx.x / kLanes;
  const int c0 = (threadIdx.x % kLanes) * 8;
  if (row >= rows) return;
  if (r_units > 0) n_splits = ((int)(row % N) / kBROf<D> + r_units) / r_units;
  float m = -INFINITY;
  for (int sp = 0; sp < n_splits; ++sp) m = fmaxf(m, Lpart[(size_t)sp * rows + row]);
  float z = 0.f;
  f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f}, a1 = a0;
  for (int sp = 0; sp < n_splits; ++sp) {
    const float ls = Lpart[(size_t)sp * rows + row];
    const float w = (ls == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((ls - m) * kLog2e);
    z += w;
    const f32x4* src = reinterpret_cast<const f32x4*>(Opart + ((size_t)sp * rows + row) * D + c0);
    a0 += w * src[0];
    a1 += w * src[1];
  }
  const float inv = 1.0f / z;
  uint32_t packed[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x0 = (e < 2 ? a0[2 * e] : a1[2 * e - 4]) * inv;
    const float x1 = (e < 2 ? a0[2 * e + 1] : a1[2 * e - 3]) * inv;
    packed[e] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1) << 16);
  }
  *reinterpret_cast<u32x4*>(O + row * D + c0) = u32x4{packed[0], packed[1], packed[2], packed[3]};
  if (c0 == 0) LSE[row] = m + log2f(z) * kLn2;
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
    case FA_ERR_SPLITS: return "n_splits must be between 1 and 64";
    case FA_ERR_SCRATCH: return "B*H*N exceeds the library's own workspace (FA_NOALLOC_ROWS rows)";
    case FA_ERR_DEVICE: return "the current device or the address of the library's workspace is unavailable";
    default: return "unknown status";
  }
}

static int check_shape(int B, int H, int N, int d, int causal, long long* blocks) {
  if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (causal != 0 && causal != 1) return FA_ERR_FLAG;
  const long long bh = (long long)B * H;
  const int kBR = rows_per_block(d);
  const long long nqb = ((long long)N + kBR - 1) / kBR;
  const long long g = bh * nqb;
  // grid size in work-items must fit 32 bits; heads must index in int
  if (bh > 0x7fffffffLL || g * threads_per_block(d) > 0xffffffffLL) return FA_ERR_SHAPE;
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
  if (rows_per_block) *rows_per_block = ::rows_per_block(d);
  if (keys_per_tile) *keys_per_tile = ::keys_per_tile(d);
  if (waves) *waves = threads_per_block(d) / 64;
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
  const int nqb = (N + rows_per_block(d) - 1) / rows_per_block(d);
  const float c_log2 = scale * kLog2e;
  const __bf16* Q = static_cast<const __bf16*>(q);
  const __bf16* Kp = static_cast<const __bf16*>(k);
  const __bf16* Vp = static_cast<const __bf16*>(v);
  __bf16* Op = static_cast<__bf16*>(o);
  const dim3 grid((unsigned)blocks), block(threads_per_block(d));
  float* np = nullptr;
  if (d == 128) {
    if (causal) hipLaunchKernelGGL((fa_fwd_kernel<128, true, false>), grid, block, 0, stream, Q, Kp, Vp, Op, lse, np, np, BH, N, nqb, 1, 1, c_log2);
    else        hipLaunchKernelGGL((fa_fwd_kernel<128, false, false>), grid, block, 0, stream, Q, Kp, Vp, Op, lse, np, np, BH, N, nqb, 1, 1, c_log2);
  } else {
    if (causal) hipLaunchKernelGGL((fa_fwd_kernel<64, true, false>), grid, block, 0, stream, Q, Kp, Vp, Op, lse, np, np, BH, N, nqb, 1, 1, c_log2);
    else        hipLaunchKernelGGL((fa_fwd_kernel<64, false, false>), grid, block, 0, stream, Q, Kp, Vp, Op, lse, np, np, BH, N, nqb, 1, 1, c_log2);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// A model of the split-KV forward's time, used to choose its ranges: list
// scheduling of the workgroups, in dispatch order, onto the XCDs' compute
// units (each XCD takes a contiguous run of the grid when the grid is a
// multiple of 8, else every 8th workgroup), each costing its key tiles plus a
// fixed overhead, then the merge's round trip of the fp32 partials.  The
// constants were fitted to side-by-side measurements on one MI355X (causal
// shares of 2 to 8 heads of 8K-16K tokens): per 64-key tile 1.35 us at
// d = 128 and 0.40 us at d = 64 (two workgroups per CU, each at half speed),
// 6 and 4 tiles of overhead per workgroup, and the merge at 8 TB/s plus 20 us.
constexpr int kModelKeys = 64;   // the model's unit of work: a 64-key tile, whatever the kernel's own tile
static double split_model_time(int B, int H, int N, int d, int causal, int n_splits, int r_units) {
  const int br = rows_per_block(d);
  const int nqb = (N + br - 1) / br;
  const long long bh = (long long)B * H;
  const double tile_s = d == 128 ? 1.35e-6 : 0.40e-6, ovh = d == 128 ? 6.0 : 4.0;
  const int per_cu = d == 64 ? 2 : 1;
  std::vector<int> head;   // one head's workgroups, in dispatch order: their key tiles
  for (int qb = nqb - 1; qb >= 0; --qb) {
    const int t = ((causal ? std::min(N, (qb + 1) * br) : N) + kModelKeys - 1) / kModelKeys;
    const int n = r_units > 0 ? (qb + r_units) / r_units : n_splits;
    for (int sp = n - 1; sp >= 0; --sp)
      head.push_back((int)((long long)(sp + 1) * t / n - (long long)sp * t / n));
  }
  const long long total = bh * (long long)head.size();
  double span = 0.0;
  for (int x = 0; x < kXcds; ++x) {
    std::priority_queue<double, std::vector<double>, std::greater<double>> cu;
    for (int i = 0; i < 32 * per_cu; ++i) cu.push(0.0);
    auto place = [&](long long i) {
      const double t0 = cu.top();
      cu.pop();
      cu.push(t0 + (head[(size_t)(i % (long long)head.size())] + ovh) * per_cu);
    };
    if (total % kXcds == 0)
      for (long long i = x * (total / kXcds); i < (x + 1) * (total / kXcds); ++i) place(i);
    else
      for (long long i = x; i < total; i += kXcds) place(i);
    double end = 0.0;
    while (!cu.empty()) {
      end = std::max(end, cu.top());
      cu.pop();
    }
    span = std::max(span, end);
  }
  const double merge = n_splits > 1 ? 2.0 * n_splits * (double)bh * N * d * 4 / 8e12 + 20e-6 : 0.0;
  return span * tile_s + merge;
}

// The range rule fa_fwd_splitkv uses for n_splits: 0 (every query block cut
// into n_splits ranges) or, under the causal mask, r > 0 (block b cut into
// ceil((b + 1) / r) ranges, r = ceil(blocks per head / n_splits)), whichever
// the model above says is faster.
static int split_rule(int B, int H, int N, int d, int causal, int n_splits) {
  if (!causal || n_splits <= 1) return 0;
  const int nqb = (N + rows_per_block(d) - 1) / rows_per_block(d);
  const int r = (nqb + n_splits - 1) / n_splits;
  const double t_uniform = split_model_time(B, H, N, d, causal, n_splits, 0);
  const double t_prop = split_model_time(B, H, N, d, causal, n_splits, r);
  return t_prop < t_uniform ? r : 0;
}

extern "C" int fa_fwd_splitkv_ranges(int B, int H, int N, int d, int causal, int n_splits, int* r_units) {
  long long blocks = 0;
  const int st = check_shape(B, H, N, d, causal, &blocks);
  if (st != FA_OK) return st;
  if (n_splits < 1 || n_splits > kMaxSplits) return FA_ERR_SPLITS;
  if (r_units) *r_units = split_rule(B, H, N, d, causal, n_splits);
  return FA_OK;
}

extern "C" int fa_fwd_splitkv_plan(int B, int H, int N, int d, int causal, int* n_splits,
                                   size_t* o_part_bytes, size_t* lse_part_bytes) {
  long long blocks = 0;
  const int st = check_shape(B, H, N, d, causal, &blocks);
  if (st != FA_OK) return st;
  // enough workgroups for two rounds of the ones the GPU holds at once (256
  // CUs, one workgroup each at d = 128, two at d = 64), at least 8 key tiles
  // per range of the longest query block (shorter ranges do not pay for the
  // merge launch), at most 16.  More splits balance the causal block lengths
  // better but cost the fp32 partials' round trip through HBM
  // (2 n_splits B H N d 4 bytes).
  // the split count (1: fa_fwd alone, no merge) with the smallest modelled
  // time, each count with its own range rule; ranges of at least 8 key tiles
  // on the longest block; at most 16
  const long long tiles = ((long long)N + kModelKeys - 1) / kModelKeys;
  long long n = 1;
  if (blocks < 2LL * 256 * (d == 64 ? 2 : 1)) {       // fa_fwd alone fills fewer than two rounds
    double best = split_model_time(B, H, N, d, causal, 1, 0);
    for (int c = 2; c <= 16 && c <= tiles / 8; ++c) {
      const int rule = split_rule(B, H, N, d, causal, c);
      const double t = split_model_time(B, H, N, d, causal, c, rule);
      if (t < best) {
        best = t;
        n = c;
      }
    }
  }
  if (n_splits) *n_splits = (int)n;
  const size_t rows = (size_t)B * H * (size_t)N;
  if (o_part_bytes) *o_part_bytes = (size_t)n * rows * d * 4;
  if (lse_part_bytes) *lse_part_bytes = (size_t)n * rows * 4;
  return FA_OK;
}

extern "C" int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int N, int d, float scale, int causal, int n_splits,
                              float* o_part, float* lse_part, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !o_part || !lse_part) return FA_ERR_NULL;
  long long blocks = 0;
  const int st = check_shape(B, H, N, d, causal, &blocks);
  if (st != FA_OK) return st;
  if (n_splits < 1 || n_splits > kMaxSplits) return FA_ERR_SPLITS;
  if (blocks * n_splits * threads_per_block(d) > 0xffffffffLL) return FA_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                        reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                        reinterpret_cast<uintptr_t>(o_part);
  if ((mis & 15u) != 0 || ((reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(lse_part)) & 3u) != 0)
    return FA_ERR_ALIGN;
  const size_t rows = (size_t)B * H * (size_t)N;
  const size_t tb = rows * d * 2, lb = rows * 4;
  const size_t ob = (size_t)n_splits * rows * d * 4, pb = (size_t)n_splits * rows * 4;
  const void* ins[3] = {q, k, v};
  const void* outs[4] = {o, lse, o_part, lse_part};
  const size_t out_bytes[4] = {tb, lb, ob, pb};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 3; ++b)
      if (overlaps(outs[a], out_bytes[a], ins[b], tb)) return FA_ERR_ALIAS;
    for (int b = a + 1; b < 4; ++b)
      if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return FA_ERR_ALIAS;
  }

  const int BH = B * H;
  const int nqb = (N + rows_per_block(d) - 1) / rows_per_block(d);
  const float c_log2 = scale * kLog2e;
  const __bf16* Q = static_cast<const __bf16*>(q);
  const __bf16* Kp = static_cast<const __bf16*>(k);
  const __bf16* Vp = static_cast<const __bf16*>(v);
  __bf16* Op = static_cast<__bf16*>(o);
  __bf16* nb = nullptr;
  float* nl = nullptr;
  // the range rule: n_splits per query block, or under the mask (if the
  // model prefers it) ceil((b + 1) / r) for query block b, at most n_splits
  const int r = split_rule(B, H, N, d, causal, n_splits);
  const long long n_wg = r > 0 ? (long long)BH * causal_units(nqb, r) : blocks * n_splits;
  const dim3 grid((unsigned)n_wg), block(threads_per_block(d));
  if (d == 128) {
    if (causal) hipLaunchKernelGGL((fa_fwd_kernel<128, true, true>), grid, block, 0, stream, Q, Kp, Vp, nb, nl, o_part, lse_part, BH, N, nqb, n_splits, r, c_log2);
    else        hipLaunchKernelGGL((fa_fwd_kernel<128, false, true>), grid, block, 0, stream, Q, Kp, Vp, nb, nl, o_part, lse_part, BH, N, nqb, n_splits, 1, c_log2);
    hipLaunchKernelGGL((fa_merge_kernel<128>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream,
                       o_part, lse_part, Op, lse, (long long)rows, N, n_splits, r);
  } else {
    if (causal) hipLaunchKernelGGL((fa_fwd_kernel<64, true, true>), grid, block, 0, stream, Q, Kp, Vp, nb, nl, o_part, lse_part, BH, N, nqb, n_splits, r, c_log2);
    else        hipLaunchKernelGGL((fa_fwd_kernel<64, false, true>), grid, block, 0, stream, Q, Kp, Vp, nb, nl, o_part, lse_part, BH, N, nqb, n_splits, 1, c_log2);
    hipLaunchKernelGGL((fa_merge_kernel<64>), dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, stream,
                       o_part, lse_part, Op, lse, (long long)rows, N, n_splits, r);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}
