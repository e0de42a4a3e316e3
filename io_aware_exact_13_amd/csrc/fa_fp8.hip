// FP8 (OCP E4M3) attention forward for MI355X (gfx950 / CDNA4).
//
// "为什么Flash Attention能将注意力计算提速数倍而不损失精度", section Flash
// Attention 3 (FP8 low-precision support): the forward on the FP8 matrix
// units at twice the bf16 rate, with incoherent processing against the
// quantisation error.  The page gives no scheme; the one implemented here:
//   * E4M3 operands with one dequantisation factor per (batch, head) and
//     tensor, made by fa_quant_fp8 (fa_quant8.hip), Q and K optionally after
//     a shared random-sign Hadamard rotation that leaves Q K^T unchanged;
//   * the online softmax of the bf16 path with P rounded to E4M3 instead of
//     bf16, taken against the running row maximum (P <= 1, the largest
//     weight so far exactly 1); the running sum adds the fp32 P.
//
// gfx950 design:
//   * Both products run on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32
//     accumulation; 64 cycles, twice the bf16 work per cycle).
//     S^T = K Q^T: A is 32 bytes of a K row from LDS, B is 32 bytes of Q
//     from registers (loaded once).  The K rows of each 32-row block are
//     fetched in a permuted order chosen so that accumulator element r of
//     block b of lane half h is key 32h + 16b + r: each lane half owns 32
//     contiguous keys of the 64-key tile.
//   * O^T += V^T P^T: the B operand is the lane's 32 P values packed to
//     E4M3 in key order (no data movement).  The V^T operand is read with
//     ds_read_b64_tr_b8 from V in its natural row-major layout: in each
//     16-lane group, lane a loads 8 bytes of row a/2 and receives column a of
//     the group's 8 rows, i.e. 8 consecutive keys of one head-dim column.
//   * LDS rows are unpadded with XOR-swizzled 16-byte chunks; one mask
//     serves both the K row reads and the transposed V reads without bank
//     conflicts.  K and V tiles (64 keys, 8 KiB at d = 128) move HBM -> LDS
//     by buffer_load ... lds through four-buffer rings, two steps ahead.
//   * Workgroups of 4 waves (128 query rows, 64 KiB of LDS at d = 128), two
//     per CU: each SIMD then runs waves of two independent workgroups, which
//     drift apart, so one's softmax overlaps the other's MFMAs and barrier
//     waits (7% faster than 8-wave workgroups of 256 rows, which hold both
//     waves of a SIMD to the same barrier every tile).
//   * The step structure, XCD-aware workgroup order and epilogue follow the
//     bf16 forward (fa_fwd.hip): per step, S_{j+1}, O += V_{j-1} P_{j-1} and
//     the softmax of tile j interleave in one instruction stream.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "fa.h"

// VALU instructions of the softmax the scheduler places after each MFMA of a
// step (the rest follow the step's last MFMA); a build may override them to
// measure other placements
#ifndef FA8_VALU_PER_MFMA_D128
#define FA8_VALU_PER_MFMA_D128 16
#endif
#ifndef FA8_VALU_PER_MFMA_D64
#define FA8_VALU_PER_MFMA_D64 32
#endif
// Race-check build (FA8_EXTRA_BARRIER=1): after each step's LDS reads, wait
// for every memory operation and hold a workgroup barrier, so no wave can
// refill a ring buffer another wave may still read.  Its results must equal
// the default build's bit for bit.
#ifndef FA8_EXTRA_BARRIER
#define FA8_EXTRA_BARRIER 0
#endif

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;

constexpr int kBC = 64;           // keys per K/V tile
constexpr int kWaves = 4;         // waves per workgroup, 32 query rows each
constexpr int kThreads = kWaves * 64;
constexpr int kBR = kWaves * 32;  // query rows per workgroup
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  // format fields 0, 0: both operands E4M3; zero scale operands select the
  // unscaled instruction
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// LDS geometry of an E4M3 tile: 64 rows of D bytes, 16-byte chunk c of row r
// stored at chunk c ^ f(r).
//  * K row reads (ds_read_b128): the 16 lanes of a read fetch one logical
//    chunk of 16 rows whose bits 0, 1, 2, 5 vary; with D = 128 two rows share
//    a 256-byte bank line (bit 0), and f takes 8 values over bits 1, 2, 5.
//  * V transposed reads (ds_read_b64_tr_b8): 32 lanes fetch chunks 2ct and
//    2ct + 1 of 8 consecutive rows; f moves rows only by even chunk steps
//    over bits 1, 2 (bit 5 is fixed there), so the even and odd chunks stay
//    apart and the 16 pieces land in distinct banks.
//  * f ignores row bits 3 and 4, so the 8-row steps of the V reads and the
//    16-row step between K blocks keep a lane's offsets fixed.
template <int D>
struct Geom8 {
  static constexpr int kRowBytes = D;
  static constexpr int kChunks = D / 16;
  static constexpr int kTile = kBC * kRowBytes;
  static constexpr int kRing = 4;
  static constexpr int kLdsBytes = 2 * kRing * kTile;
  static constexpr int kIssues = kTile / (kWaves * 1024);   // 1 KiB copies per wave per tile
  static_assert(kIssues * kWaves * 1024 == kTile, "tile copy split");
  __host__ __device__ static constexpr int f(int r) {
    return D == 128 ? ((((r >> 1) & 3) << 1) | ((r >> 5) & 1)) : ((((r >> 2) & 1) << 1) | ((r >> 5) & 1));
  }
  __host__ __device__ static constexpr int k_buf(int b) { return b * kTile; }
  __host__ __device__ static constexpr int v_buf(int b) { return (kRing + b) * kTile; }
};

// The K row that lane row i of S block b reads: accumulator element r of
// lane half h then holds key 32h + 16b + r (i = 8(r/4) + 4h + r%4).
__host__ __device__ constexpr int s_key(int b, int i) {
  return 32 * ((i >> 2) & 1) + 16 * b + 8 * (i >> 4) + 4 * ((i >> 3) & 1) + (i & 3);
}

// One wave's share of an HBM -> LDS tile copy, kIssues pieces of 1 KiB; the
// lane fetches the global chunk the swizzle puts in its slot (the swizzle
// depends on row bit 5, so each piece has its own offset).  Rows past `n`
// read as zeros.
template <int D>
struct TileCopy8 {
  unsigned voff[Geom8<D>::kIssues];
  __device__ __forceinline__ void init(int wave, int lane) {
    using G = Geom8<D>;
#pragma unroll
    for (int i = 0; i < G::kIssues; ++i) {
      const int slot = (i * kWaves + wave) * 64 + lane;
      const int row = slot / G::kChunks, pchunk = slot % G::kChunks;
      voff[i] = (unsigned)(row * G::kRowBytes + ((pchunk ^ G::f(row)) << 4));
    }
  }
  __device__ __forceinline__ void issue(const char* head, int key0, int n, char* dst, int wave) const {
    using G = Geom8<D>;
#if defined(__HIP_DEVICE_COMPILE__)
    const int rows = max(n - key0, 0);
    const char* base = head + (size_t)min(key0, n) * G::kRowBytes;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, rows * G::kRowBytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < G::kIssues; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + (i * kWaves + wave) * 1024), 16, voff[i],
                                               0, 0, 0);
#endif
  }
};

__device__ __forceinline__ float max_halves(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_elementwise_maximum(__builtin_bit_cast(float, (unsigned)r[0]),
                                       __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

template <int D>
struct RowState8 {
  f32x16 acc[D / 32];   // O^T accumulators (head-dim rows, this lane's query column)
  float m_ref;          // running row maximum, log2 units of the scaled score
  float l_part;         // this lane's share of the exponential sum
};

template <int D>
struct Ctx8 {
  const char* Kh;
  const char* Vh;
  char* lds;
  int kv_end, n_tiles, lim, wave, h;
  float c_log2;
  int k_off[D / 64][2];   // lane's LDS offsets of its two K chunks for k-step s (block 0)
  int v_off[D / 32];      // lane's LDS offset of its first transposed V read, column tile ct (V region)
  TileCopy8<D> kcopy, vcopy;
};

// A operand of S block b, k-step s: 32 bytes of K row s_key(b, l32).
template <int D>
__device__ __forceinline__ i32x8 k_operand(const char* kt, const Ctx8<D>& c, int s, int b) {
  using G = Geom8<D>;
  const i32x4 lo = *reinterpret_cast<const i32x4*>(kt + c.k_off[s][0] + b * 16 * G::kRowBytes);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(kt + c.k_off[s][1] + b * 16 * G::kRowBytes);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A operand of O += V P, column tile ct: four transposed reads, keys
// 32h + 8t .. +7 of head-dim column 32 ct + l32 for t = 0..3.
template <int D>
__device__ __forceinline__ i32x8 v_operand(const char* vt, int v_off_ct) {
  using G = Geom8<D>;
  i32x2 r[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    r[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(vt + v_off_ct + t * 8 * G::kRowBytes));
  return i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
}

// S^T = K Q^T for one tile, not overlapped (the first tile).
template <int D>
__device__ __forceinline__ void scores(const char* kt, const Ctx8<D>& c, const i32x8 (&qf)[D / 64],
                                       f32x16 (&s)[2]) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    s[b] = mfma8(k_operand<D>(kt, c, 0, b), qf[0], f32x16{});
#pragma unroll
    for (int ks = 1; ks < D / 64; ++ks) s[b] = mfma8(k_operand<D>(kt, c, ks, b), qf[ks], s[b]);
  }
}

// Online-softmax update of one tile against the running maximum: mask, row
// max, alpha = exp2(m_old - m_new), P = exp2(S c - m_new) <= 1 packed to
// E4M3 in key order, row sum of the fp32 P.  Sets *rescale when some lane of
// the wave has a new maximum.
template <int D, bool MASKED>
__device__ __forceinline__ float softmax_tile(f32x16 (&s)[2], int key0, int lim, int h, float c_log2,
                                              RowState8<D>& st, i32x8& pf, bool* rescale) {
  if (MASKED) {
    // register r of block b holds key key0 + 32 h + (16 b + r): one compare per score
    const int room = lim - key0 - 32 * h;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (16 * b + r > room) s[b][r] = -INFINITY;
  }
  float part[32];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) part[b * 16 + r] = s[b][r];
  int n = 32;
#pragma unroll
  for (int round = 0; round < 6; ++round) {
    if (n <= 1) break;
    const int m = (n + 2) / 3;
#pragma unroll
    for (int r = 0; r < m; ++r) {
      const float a = part[3 * r];
      const float b = 3 * r + 1 < n ? part[3 * r + 1] : a;
      const float cc = 3 * r + 2 < n ? part[3 * r + 2] : a;
      part[r] = __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, cc));
    }
    n = m;
  }
  const float m_tile = max_halves(part[0]) * c_log2;
  const bool grow = m_tile > st.m_ref;
  const float m_new = grow ? m_tile : st.m_ref;
  *rescale = __builtin_amdgcn_ballot_w64(grow) != 0;
  // 0 while the row has seen no key (acc and l are still 0): no exp2 of
  // (-inf) - (-inf) when this tile shows it none either
  const float alpha = (st.m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m_ref - m_new);
  st.m_ref = m_new;
  const float neg_m = (m_new == -INFINITY) ? 0.f : -m_new;
  float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int b = w >> 2, r0 = 4 * (w & 3);
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = __builtin_amdgcn_exp2f(fmaf(s[b][r0 + e], c_log2, neg_m));
      l4[e] += p[e];
    }
    // the old bytes 2, 3 kept by this conversion are replaced by the next one
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pf[w], false);
    pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], lo, true);
  }
  st.l_part = st.l_part * alpha + ((l4[0] + l4[1]) + (l4[2] + l4[3]));
  asm volatile("" : "+v"(pf));
  asm volatile("" : "+v"(st.l_part), "+v"(st.m_ref));
  return alpha;
}

// One pipeline step, iteration j (as in the bf16 forward): in flight on
// entry S_j (s_in) and P_{j-1} (p_in); K_{j+1} and V_{j-1} are in LDS.  The
// step copies K_{j+3} and V_{j+1}, and interleaves the MFMAs of S_{j+1} and
// O += V_{j-1} P_{j-1} with the softmax of tile j.
template <int D, bool MASKED>
__device__ __forceinline__ void step(const char* __restrict__ k_read, const char* __restrict__ v_read,
                                     char* __restrict__ k_fill, char* __restrict__ v_fill, const Ctx8<D>& c,
                                     int j, const i32x8 (&qf)[D / 64], f32x16 (&s_in)[2], f32x16 (&s_out)[2],
                                     const i32x8& p_in, i32x8& p_out, RowState8<D>& st) {
  constexpr int kN = D / 32;            // S MFMAs (k-step, block) = P V MFMAs (column tiles)
  if constexpr (Geom8<D>::kIssues == 2) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  i32x8 v_op[kN], k_op[kN];
  auto fetch = [&](int i) {
    v_op[i] = v_operand<D>(v_read, c.v_off[i]);
    k_op[i] = k_operand<D>(k_read, c, i >> 1, i & 1);
  };
  auto mfma = [&](int i) {
    st.acc[i] = mfma8(v_op[i], p_in, st.acc[i]);
    const int ks = i >> 1, b = i & 1;
    s_out[b] = mfma8(k_op[i], qf[ks], ks == 0 ? f32x16{} : s_out[b]);
  };
  fetch(0);
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    if (i + 1 < kN) fetch(i + 1);
    mfma(i);
    if (i == 0) c.kcopy.issue(c.Kh, (j + 3) * kBC, c.kv_end, k_fill, c.wave);
    if (i == 1) c.vcopy.issue(c.Vh, (j + 1) * kBC, c.kv_end, v_fill, c.wave);
  }
  bool rescale = false;
  const float alpha = softmax_tile<D, MASKED>(s_in, j * kBC, c.lim, c.h, c.c_log2, st, p_out, &rescale);
  // each MFMA pair: the next pair's LDS reads (4 transposed + 2 row reads),
  // two MFMAs, and a share of the softmax's VALU work after each (mask 0x008
  // MFMA, 0x100 LDS read, 0x002 VALU)
  constexpr int kValu = D == 128 ? FA8_VALU_PER_MFMA_D128 : FA8_VALU_PER_MFMA_D64;
  __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    if (i + 1 < kN) __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
  }
  if constexpr (FA8_EXTRA_BARRIER) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (rescale) {
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[ct][r] *= alpha;
  }
}

template <int D, bool MASKED, int PH>
__device__ __forceinline__ void step_at(const Ctx8<D>& c, int j, const i32x8 (&qf)[D / 64], f32x16 (&sa)[2],
                                        f32x16 (&sb)[2], i32x8& pa, i32x8& pb, RowState8<D>& st) {
  using G = Geom8<D>;
  constexpr int R = G::kRing;
  const char* kr = c.lds + G::k_buf((PH + 1) % R);
  const char* vr = c.lds + G::k_buf((PH + R - 1) % R);     // V region base is folded into v_off
  char* kf = c.lds + G::k_buf((PH + 3) % R);
  char* vf = c.lds + G::v_buf((PH + 1) % R);
  if constexpr (PH % 2 == 0) step<D, MASKED>(kr, vr, kf, vf, c, j, qf, sa, sb, pa, pb, st);
  else step<D, MASKED>(kr, vr, kf, vf, c, j, qf, sb, sa, pb, pa, st);
}

template <int D, bool MASKED>
__device__ __forceinline__ void step_quad(const Ctx8<D>& c, int j, const i32x8 (&qf)[D / 64], f32x16 (&sa)[2],
                                          f32x16 (&sb)[2], i32x8& pa, i32x8& pb, RowState8<D>& st) {
  step_at<D, MASKED, 0>(c, j, qf, sa, sb, pa, pb, st);
  step_at<D, MASKED, 1>(c, j + 1, qf, sa, sb, pa, pb, st);
  step_at<D, MASKED, 2>(c, j + 2, qf, sa, sb, pa, pb, st);
  step_at<D, MASKED, 3>(c, j + 3, qf, sa, sb, pa, pb, st);
}

template <int D, bool CAUSAL>
// 2 waves per SIMD at d = 128 (230 registers a lane), 3 at d = 64 (158; 4%
// faster on the 2K d = 64 workload, with three workgroups per CU).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, D == 64 ? 3 : 2)))
void fa_fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                       const uint8_t* __restrict__ V, const float* __restrict__ q_descale,
                       const float* __restrict__ k_descale, const float* __restrict__ v_descale,
                       __bf16* __restrict__ O, float* __restrict__ LSE, int BH, int N, int n_qblocks,
                       float scale_log2) {
  using G = Geom8<D>;
  constexpr int kKs = D / 64;
  constexpr int kCt = D / 32;
  __shared__ __attribute__((aligned(1024))) char lds[G::kLdsBytes];

  Ctx8<D> c;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  c.h = lane >> 5;
  const int l32 = lane & 31;

  // workgroup -> (head, query block), XCD-aware as in the bf16 forward
  const int wg = blockIdx.x;
  const int n_wg = BH * n_qblocks;
  const int logical = (n_wg % kXcds == 0) ? (wg % kXcds) * (n_wg / kXcds) + wg / kXcds : wg;
  const int bh = logical / n_qblocks;
  const int qi = logical % n_qblocks;
  const int qb = CAUSAL ? (n_qblocks - 1 - qi) : qi;
  const int q0 = qb * kBR;
  const int qrow = q0 + c.wave * 32 + l32;
  c.lim = CAUSAL ? min(qrow, N - 1) : N - 1;
  c.c_log2 = scale_log2 * q_descale[bh] * k_descale[bh];
  const float dv = v_descale[bh];
  c.lds = lds;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  c.Kh = reinterpret_cast<const char*>(K + head_off);
  c.Vh = reinterpret_cast<const char*>(V + head_off);

  const int kv_end = CAUSAL ? min(N, q0 + kBR) : N;
  c.n_tiles = (kv_end + kBC - 1) / kBC;
  c.kv_end = kv_end;
  int j_mask = N / kBC;                                 // the first tile holding a key >= N
  if (CAUSAL) j_mask = min(j_mask, q0 / kBC);
  j_mask = min(j_mask, c.n_tiles);

  // per-lane LDS offsets
  {
    const int row = s_key(0, l32);
#pragma unroll
    for (int s = 0; s < kKs; ++s)
#pragma unroll
      for (int u = 0; u < 2; ++u) c.k_off[s][u] = row * G::kRowBytes + (((4 * s + 2 * c.h + u) ^ G::f(row)) << 4);
    const int a = lane & 15, g = lane >> 4;
    const int vrow = 32 * (g >> 1) + (a >> 1);
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct)
      c.v_off[ct] = G::v_buf(0) + vrow * G::kRowBytes + (((2 * ct + (g & 1)) ^ G::f(vrow)) << 4) + 8 * (a & 1);
  }
  c.kcopy.init(c.wave, lane);
  c.vcopy.init(c.wave, lane);

  // prologue: K_0, K_1, then K_2 and V_0; V buffer kRing-1 ("V_{-1}") zeroed
  c.kcopy.issue(c.Kh, 0, c.kv_end, lds + G::k_buf(0), c.wave);
  c.kcopy.issue(c.Kh, kBC, c.kv_end, lds + G::k_buf(1), c.wave);
  c.kcopy.issue(c.Kh, 2 * kBC, c.kv_end, lds + G::k_buf(2), c.wave);
  c.vcopy.issue(c.Vh, 0, c.kv_end, lds + G::v_buf(0), c.wave);
  for (int i = tid; i < G::kTile / 8; i += kThreads)
    reinterpret_cast<u32x2*>(lds + G::v_buf(G::kRing - 1))[i] = u32x2{0u, 0u};

  // Q^T operand: lane holds Q8[qrow][64 s + 32 h .. +31]
  i32x8 qf[kKs];
  {
    const bool ok = qrow < N;
    const i32x4* src = reinterpret_cast<const i32x4*>(Q + head_off + (size_t)(ok ? qrow : 0) * D);
#pragma unroll
    for (int s = 0; s < kKs; ++s) {
      i32x4 lo = src[4 * s + 2 * c.h], hi = src[4 * s + 2 * c.h + 1];
      if (!ok) lo = hi = i32x4{0, 0, 0, 0};
      qf[s] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }

  RowState8<D> st;
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) st.acc[ct] = f32x16{};
  st.m_ref = -INFINITY;
  st.l_part = 0.f;
  f32x16 sa[2], sb[2];
  i32x8 pa = i32x8{0, 0, 0, 0, 0, 0, 0, 0}, pb = pa;

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the prologue's copies and Q
  __syncthreads();
  scores<D>(lds + G::k_buf(0), c, qf, sa);

  int j = 0;
  for (; j + 4 <= j_mask; j += 4) step_quad<D, false>(c, j, qf, sa, sb, pa, pb, st);
  for (; j + 4 <= c.n_tiles; j += 4) step_quad<D, true>(c, j, qf, sa, sb, pa, pb, st);
  if (j < c.n_tiles) step_at<D, true, 0>(c, j++, qf, sa, sb, pa, pb, st);
  if (j < c.n_tiles) step_at<D, true, 1>(c, j++, qf, sa, sb, pa, pb, st);
  if (j < c.n_tiles) step_at<D, true, 2>(c, j++, qf, sa, sb, pa, pb, st);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  {
    const int last = c.n_tiles - 1;
    const char* vt = lds + G::k_buf(last % G::kRing);
    const i32x8 pl = ((last + 1) & 1) ? pb : pa;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) st.acc[ct] = mfma8(v_operand<D>(vt, c.v_off[ct]), pl, st.acc[ct]);
  }

  const float l_tot = sum_halves(st.l_part);
  // O = acc * dv / l in bf16, staged through this wave's slice of the K ring
  // (idle since the barrier above) and stored as whole rows, 16 bytes a lane,
  // as in the bf16 forward: chunk ch of staged row r sits at slot
  // ch ^ (r % kOutChunks).  Four waves of 32 rows of 2D bytes fill the ring
  // exactly.
  {
    constexpr int kOutRow = 2 * D;                  // bytes of one bf16 output row
    constexpr int kOutChunks = kOutRow / 16;
    static_assert(kWaves * 32 * kOutRow <= G::kRing * G::kTile, "staging fits the K ring");
    char* stage = lds + G::k_buf(0) + c.wave * 32 * kOutRow;
    const float inv = qrow < N ? dv / l_tot : 0.f;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const __bf16 b0 = (__bf16)(st.acc[ct][r4 * 4 + 0] * inv);
        const __bf16 b1 = (__bf16)(st.acc[ct][r4 * 4 + 1] * inv);
        const __bf16 b2 = (__bf16)(st.acc[ct][r4 * 4 + 2] * inv);
        const __bf16 b3 = (__bf16)(st.acc[ct][r4 * 4 + 3] * inv);
        u32x2 w;
        w[0] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        w[1] = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        // columns ct*32 + r4*8 + 4h .. +3: chunk 4ct + r4, half h
        const int ch = ct * 4 + r4;
        *reinterpret_cast<u32x2*>(stage + l32 * kOutRow + ((ch ^ (l32 % kOutChunks)) << 4) + 8 * c.h) = w;
      }
    // the wave reads back what its other lanes wrote: wait for the writes
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int row0 = q0 + c.wave * 32;
#pragma unroll
    for (int i = 0; i < kOutChunks / 2; ++i) {
      const int q = i * 64 + lane, r = q / kOutChunks, ch = q % kOutChunks;
      const u32x4 val = *reinterpret_cast<const u32x4*>(stage + r * kOutRow + ((ch ^ (r % kOutChunks)) << 4));
      if (row0 + r < N) *reinterpret_cast<u32x4*>(O + head_off + (size_t)(row0 + r) * D + ch * 8) = val;
    }
  }
  if (qrow < N && c.h == 0) LSE[(size_t)bh * N + qrow] = (st.m_ref + log2f(l_tot)) * kLn2;
}
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int check_shape8(int B, int H, int N, int d, long long* bh_out) {
  if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  const long long bh = (long long)B * H;
  if (bh > 0x7fffffffLL) return FA_ERR_SHAPE;
  if ((long long)N * d >= 0x80000000LL) return FA_ERR_SHAPE;    // one head's bytes fit a 32-bit buffer range
  *bh_out = bh;
  return FA_OK;
}

}  // namespace

extern "C" int fa_fwd_fp8_tile(int B, int H, int N, int d, int causal, int* rows_per_block, int* keys_per_tile,
                               int* waves, long long* blocks) {
  long long bh = 0;
  const int st = check_shape8(B, H, N, d, &bh);
  if (st != FA_OK) return st;
  if (causal != 0 && causal != 1) return FA_ERR_FLAG;
  const long long nqb = ((long long)N + kBR - 1) / kBR;
  if (bh * nqb * kThreads > 0xffffffffLL) return FA_ERR_SHAPE;
  if (rows_per_block) *rows_per_block = kBR;
  if (keys_per_tile) *keys_per_tile = kBC;
  if (waves) *waves = kWaves;
  if (blocks) *blocks = bh * nqb;
  return FA_OK;
}

extern "C" int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_descale,
                          const float* k_descale, const float* v_descale, void* o, float* lse, int B, int H, int N,
                          int d, float scale, int causal, hipStream_t stream) {
  if (!q8 || !k8 || !v8 || !q_descale || !k_descale || !v_descale || !o || !lse) return FA_ERR_NULL;
  long long bh = 0;
  int st = check_shape8(B, H, N, d, &bh);
  if (st != FA_OK) return st;
  if (causal != 0 && causal != 1) return FA_ERR_FLAG;
  const long long nqb = ((long long)N + kBR - 1) / kBR;
  if (bh * nqb * kThreads > 0xffffffffLL) return FA_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(q8) | reinterpret_cast<uintptr_t>(k8) |
                        reinterpret_cast<uintptr_t>(v8) | reinterpret_cast<uintptr_t>(o);
  const uintptr_t mis4 = reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(q_descale) |
                         reinterpret_cast<uintptr_t>(k_descale) | reinterpret_cast<uintptr_t>(v_descale);
  if ((mis & 15u) != 0 || (mis4 & 3u) != 0) return FA_ERR_ALIGN;
  const size_t elems = (size_t)bh * N * d;
  const size_t ob = 2 * elems, lb = (size_t)bh * N * 4, db = (size_t)bh * 4;
  const void* ins[6] = {q8, k8, v8, q_descale, k_descale, v_descale};
  const size_t in_bytes[6] = {elems, elems, elems, db, db, db};
  for (int i = 0; i < 6; ++i)
    if (overlaps(o, ob, ins[i], in_bytes[i]) || overlaps(lse, lb, ins[i], in_bytes[i])) return FA_ERR_ALIAS;
  if (overlaps(o, ob, lse, lb)) return FA_ERR_ALIAS;

  const uint8_t* Q = static_cast<const uint8_t*>(q8);
  const uint8_t* Kp = static_cast<const uint8_t*>(k8);
  const uint8_t* Vp = static_cast<const uint8_t*>(v8);
  __bf16* Op = static_cast<__bf16*>(o);
  const float sl = scale * kLog2e;
  const dim3 grid((unsigned)(bh * nqb)), block(kThreads);
  if (d == 128) {
    if (causal) hipLaunchKernelGGL((fa_fwd_fp8_kernel<128, true>), grid, block, 0, stream, Q, Kp, Vp, q_descale, k_descale, v_descale, Op, lse, (int)bh, N, (int)nqb, sl);
    else        hipLaunchKernelGGL((fa_fwd_fp8_kernel<128, false>), grid, block, 0, stream, Q, Kp, Vp, q_descale, k_descale, v_descale, Op, lse, (int)bh, N, (int)nqb, sl);
  } else {
    if (causal) hipLaunchKernelGGL((fa_fwd_fp8_kernel<64, true>), grid, block, 0, stream, Q, Kp, Vp, q_descale, k_descale, v_descale, Op, lse, (int)bh, N, (int)nqb, sl);
    else        hipLaunchKernelGGL((fa_fwd_fp8_kernel<64, false>), grid, block, 0, stream, Q, Kp, Vp, q_descale, k_descale, v_descale, Op, lse, (int)bh, N, (int)nqb, sl);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}
