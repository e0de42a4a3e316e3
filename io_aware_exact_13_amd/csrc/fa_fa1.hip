// The FA1 loop order of the tiled attention forward, kept as an ablation of
// the FA2 order that fa_fwd uses (MI355X, gfx950).
//
// The pages give two loop orders for the same exact result.  The first
// ("为什么Flash Attention能将注意力计算提速数倍而不损失精度", 分块计算(Tiling),
// the two-loop pseudocode; "FlashAttention的Triton实现：IO-aware注意力机制底层原理",
// FA1 vs FA2) walks the K/V blocks in the outer loop and the Q blocks in the
// inner one, so the running O_i, l_i and m_i of every query block are read
// from HBM and written back once per K/V block.  The second (FA2, fa_fwd)
// keeps them on chip.  This file runs the first order to measure what it
// costs: one launch per 64-key block j, each updating every query block's
// (O_i, l_i, m_i) in an fp32 workspace, then one launch that writes O (bf16)
// and LSE.
//
// Per (query block i, key block j), as the pseudocode with its two slips
// read the plain way (the block's weights are taken against the new maximum,
// and the new statistics are written back):
//   m_new = max(m_i, rowmax S_ij),  P = exp(S_ij - m_new),
//   l_new = exp(m_i - m_new) l_i + rowsum P,
//   O_i   = (exp(m_i - m_new) l_i O_i + P V_j) / l_new,   write O_i, l_new, m_new.
// S is scaled and masked as in fa_fwd; m is kept in log2 units of the scaled
// score, and LSE = (m + log2 l) ln 2 at the end.

#include <math.h>

#include "cdna4.h"
#include "fa.h"

namespace {

using namespace cdna4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBR = kWaves * 32;   // query rows per workgroup
constexpr int kBC = 64;            // keys per K/V block

__device__ __forceinline__ float max_halves(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// One K/V block j against query blocks i0 .. n_qblocks-1 of every head.
// Lane l of wave w owns query q0 + 32 w + l % 32; its O_i row lives in the
// fp32 workspace Oacc between launches, its m and l in M and L.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fa1_block_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    float* __restrict__ Oacc, float* __restrict__ M, float* __restrict__ L, int BH, int N, int n_qblocks,
    int i0, int j, float c_log2) {
  constexpr int kDs = D / 16, kCt = D / 32, kKb = kBC / 32;
  constexpr int kTileBytes = kBC * 2 * D;
  using Copy = TileCopy<D, kBC, kThreads>;
  __shared__ __attribute__((aligned(1024))) char lds[2 * kTileBytes];   // K_j, V_j

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per_head = n_qblocks - i0;
  const int bh = blockIdx.x / per_head;
  const int qb = i0 + blockIdx.x % per_head;
  const int qrow = qb * kBR + wave * 32 + l32;
  const bool qok = qrow < N;
  const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;
  const size_t head_off = (size_t)bh * (size_t)N * D;

  Copy copy;
  copy.init(tid);
#pragma unroll
  for (int i = 0; i < Copy::kIssues; ++i) {
    copy.issue(reinterpret_cast<const char*>(K + head_off), j * kBC, N, lds, tid, i);
    copy.issue(reinterpret_cast<const char*>(V + head_off), j * kBC, N, lds + kTileBytes, tid, i);
  }

  bf16x8 qf[kDs];
  {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(Q + head_off + (size_t)(qok ? qrow : 0) * D);
#pragma unroll
    for (int ks = 0; ks < kDs; ++ks) qf[ks] = qok ? src[ks * 2 + h] : bf16x8{};
  }
  // this row's running statistics and output from HBM (the first block starts them)
  const size_t srow = (size_t)bh * N + (qok ? qrow : 0);
  const float m_i = (j == 0 || !qok) ? -INFINITY : M[srow];
  const float l_i = (j == 0 || !qok) ? 0.f : L[srow];
  f32x16 acc[kCt];
  float* orow = Oacc + srow * D;
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j != 0 && qok) x = *reinterpret_cast<const f32x4*>(orow + ct * 32 + r4 * 8 + h * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[ct][r4 * 4 + e] = x[e];
    }

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const char* Kt = lds;
  const char* Vt = lds + kTileBytes;

  // S^T = K_j Q_i^T: register r of block kb holds key j 64 + 32 kb + (r/4) 8 + 4 h + r%4
  f32x16 s[kKb];
#pragma unroll
  for (int kb = 0; kb < kKb; ++kb) s[kb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < kDs; ++ks)
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb) s[kb] = mfma32(row_operand<D>(Kt, 32 * kb, ks, lane), qf[ks], s[kb]);

  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j * kBC + kb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
      s[kb][r] = key <= lim ? s[kb][r] * c_log2 : -INFINITY;
      mx = fmaxf(mx, s[kb][r]);
    }
  const float m_new = fmaxf(m_i, max_halves(mx));
  const float alpha = (m_i == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_i - m_new);
  const float neg_m = (m_new == -INFINITY) ? 0.f : -m_new;
  bf16x8 pf[kBC / 16];
  float lsum = 0.f;
#pragma unroll
  for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(s[kb][r] + neg_m);
      lsum += p;
      pf[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
    }
  const float l_new = alpha * l_i + sum_halves(lsum);
  // O_i l_i alpha + P V_j, then divided by l_new
  const float keep = alpha * l_i;
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[ct][r] *= keep;
#pragma unroll
  for (int t = 0; t < kBC / 16; ++t)
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) acc[ct] = mfma32(tr_operand<D>(Vt, 16 * t, ct, lane), pf[t], acc[ct]);

  if (qok) {
    const float inv = l_new > 0.f ? 1.0f / l_new : 0.f;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<f32x4*>(orow + ct * 32 + r4 * 8 + h * 4) =
            f32x4{acc[ct][r4 * 4] * inv, acc[ct][r4 * 4 + 1] * inv, acc[ct][r4 * 4 + 2] * inv,
                  acc[ct][r4 * 4 + 3] * inv};
    if (h == 0) {
      M[srow] = m_new;
      L[srow] = l_new;
    }
  }
}

// O (bf16) and LSE from the workspace after the last block.
template <int D>
__global__ __launch_bounds__(256) void fa1_finish_kernel(const float* __restrict__ Oacc, const float* __restrict__ M,
                                                         const float* __restrict__ L, __bf16* __restrict__ O,
                                                         float* __restrict__ LSE, long long rows) {
  constexpr int kLanes = D / 8;
  const long long row = (long long)blockIdx.x * (256 / kLanes) + threadIdx.x / kLanes;
  const int c0 = (threadIdx.x % kLanes) * 8;
  if (row >= rows) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(Oacc + row * D + c0);
  const f32x4 a = src[0], b = src[1];
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    w[e] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a[2 * e]) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a[2 * e + 1]) << 16);
    w[2 + e] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b[2 * e]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b[2 * e + 1]) << 16);
  }
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<u32x4*>(O + row * D + c0) = u32x4{w[0], w[1], w[2], w[3]};
  if (c0 == 0) LSE[row] = (M[row] + log2f(L[row])) * kLn2;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

template <int D, bool CAUSAL>
void launch_fa1(const __bf16* q, const __bf16* k, const __bf16* v, __bf16* o, float* lse, float* oacc,
                float* m, float* l, int BH, int N, float c_log2, hipStream_t stream) {
  const int nqb = (N + kBR - 1) / kBR;
  const int n_blocks = (N + kBC - 1) / kBC;
  for (int j = 0; j < n_blocks; ++j) {
    // under the mask, query blocks wholly before key block j see none of it
    const int i0 = CAUSAL ? (j * kBC) / kBR : 0;
    hipLaunchKernelGGL((fa1_block_kernel<D, CAUSAL>), dim3((unsigned)(BH * (nqb - i0))), dim3(kThreads), 0, stream,
                       q, k, v, oacc, m, l, BH, N, nqb, i0, j, c_log2);
  }
  const long long rows = (long long)BH * N;
  hipLaunchKernelGGL((fa1_finish_kernel<D>), dim3((unsigned)((rows + 256 / (D / 8) - 1) / (256 / (D / 8)))),
                     dim3(256), 0, stream, oacc, m, l, o, lse, rows);
}

}  // namespace

extern "C" int fa_fwd_fa1order(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                               int N, int d, float scale, int causal, float* o_acc, float* m, float* l,
                               hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !o_acc || !m || !l) return FA_ERR_NULL;
  if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (causal != 0 && causal != 1) return FA_ERR_FLAG;
  const long long bh = (long long)B * H;
  const long long blocks = bh * (((long long)N + kBR - 1) / kBR);
  if (bh > 0x7fffffffLL || blocks * kThreads > 0xffffffffLL || (long long)N * d * 2 >= 0x80000000LL)
    return FA_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                        reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                        reinterpret_cast<uintptr_t>(o_acc);
  if ((mis & 15u) != 0 ||
      ((reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(l)) & 3u) != 0)
    return FA_ERR_ALIGN;
  const size_t rows = (size_t)bh * N;
  const size_t tb = rows * d * 2, lb = rows * 4, ab = rows * d * 4;
  const void* ins[3] = {q, k, v};
  const void* outs[5] = {o, lse, o_acc, m, l};
  const size_t out_bytes[5] = {tb, lb, ab, lb, lb};
  for (int a = 0; a < 5; ++a) {
    for (int b = 0; b < 3; ++b)
      if (overlaps(outs[a], out_bytes[a], ins[b], tb)) return FA_ERR_ALIAS;
    for (int b = a + 1; b < 5; ++b)
      if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return FA_ERR_ALIAS;
  }
  const float c_log2 = scale * kLog2e;
  const __bf16* Q = static_cast<const __bf16*>(q);
  const __bf16* Kp = static_cast<const __bf16*>(k);
  const __bf16* Vp = static_cast<const __bf16*>(v);
  __bf16* Op = static_cast<__bf16*>(o);
  const int BHi = (int)bh;
  if (d == 128) {
    if (causal) launch_fa1<128, true>(Q, Kp, Vp, Op, lse, o_acc, m, l, BHi, N, c_log2, stream);
    else        launch_fa1<128, false>(Q, Kp, Vp, Op, lse, o_acc, m, l, BHi, N, c_log2, stream);
  } else {
    if (causal) launch_fa1<64, true>(Q, Kp, Vp, Op, lse, o_acc, m, l, BHi, N, c_log2, stream);
    else        launch_fa1<64, false>(Q, Kp, Vp, Op, lse, o_acc, m, l, BHi, N, c_log2, stream);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}
