// E4M3 quantisation of attention operands for MI355X (gfx950): one scale per
// (batch, head), with optional incoherent processing (a random-sign
// Sylvester-Hadamard rotation) for Q and K.
//
// "为什么Flash Attention能将注意力计算提速数倍而不损失精度", section Flash
// Attention 3 (FP8 low-precision support): FP8 operands, and incoherent
// processing against the quantisation error.  The page gives no scheme; the
// one implemented here:
//   * code = RNE_e4m3(y * 448 / amax) with amax the head's largest |y|
//     (raised to 2^-117 if smaller and non-zero, so that 448 / amax stays
//     finite), and descale = amax / 448 (times 1/sqrt(d) after a rotation);
//   * rotation y = (sigma o x) H by the fast Walsh-Hadamard butterfly in
//     fp32: widths 1 .. 16 inside a thread, 32 and 64 across the row's lanes
//     (DPP quad permutes), each pair (a, b) -> (a + b, a - b).
// Two passes over the input: the first finds each workgroup's amax and
// leaves it in the (not yet written) code buffer, a small kernel reduces
// those per head into `descale`, and the second pass writes the codes; a
// last kernel turns amax into the descale factor.  No atomics, so every
// result is bitwise reproducible.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "fa.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;
constexpr float kAmaxMin = 0x1p-117f;   // smallest amax of a non-zero head: 448 / amax stays finite

// The amax a head's scale is taken from: 0 for an all-zero head, else at least 2^-117.
__device__ __forceinline__ float amax_used(float am) { return am > 0.f ? fmaxf(am, kAmaxMin) : 0.f; }

// ------------------------------------------------------------ quantisation
//
// Threads take 32 consecutive elements of a row (64 bytes of bf16), D/32
// threads per row (a quad of lanes at d = 128, a pair at d = 64); a 256-thread
// workgroup covers kQPass rows per pass and kQIter passes, all of one head
// (so each workgroup feeds one amax).

constexpr int kQThreads = 256;
constexpr int kQIter = 2;
constexpr int kQElems = 32;

// Sign words of the lane's 32 columns: bit 31 set where the rotation
// negates the column (bit c of the 128-bit mask).
__device__ __forceinline__ void sign_words(int col0, uint64_t slo, uint64_t shi, unsigned (&sg)[kQElems]) {
#pragma unroll
  for (int e = 0; e < kQElems; ++e) {
    const int bit = col0 + e;
    const uint64_t word = bit < 64 ? slo : shi;
    sg[e] = (unsigned)((word >> (bit & 63)) & 1) << 31;
  }
}

// The row chunk as fp32, with the sign flips and the Walsh-Hadamard
// butterflies applied when ROT: stages of width 1 .. 16 inside the thread,
// 32 and 64 across the row's lanes (lane xor 1, xor 2, by DPP quad
// permutes).  The lower element of a pair becomes a + b, the upper a - b, as
// the oracle's order fixes; across lanes that is fma(+-1, v, other), whose
// product is exact, so the sum is rounded once as a + b or a - b would be.
template <int D, bool ROT>
__device__ __forceinline__ void row_chunk(const __bf16* __restrict__ X, size_t head_off, int row, int N, int c,
                                          const unsigned (&sg)[kQElems], float (&v)[kQElems]) {
  if (row < N) {
    const u32x4* src = reinterpret_cast<const u32x4*>(X + head_off + (size_t)row * D + kQElems * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 raw = src[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * q + 2 * e] = __builtin_bit_cast(float, raw[e] << 16);
        v[8 * q + 2 * e + 1] = __builtin_bit_cast(float, raw[e] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kQElems; ++e) v[e] = 0.f;
  }
  if constexpr (ROT) {
#pragma unroll
    for (int e = 0; e < kQElems; ++e) v[e] = __builtin_bit_cast(float, __builtin_bit_cast(unsigned, v[e]) ^ sg[e]);
#pragma unroll
    for (int w = 1; w < kQElems; w <<= 1)
#pragma unroll
      for (int i = 0; i < kQElems; ++i)
        if ((i & w) == 0) {
          const float a = v[i], b = v[i + w];
          v[i] = a + b;
          v[i + w] = a - b;
        }
#pragma unroll
    for (int m = 1; m < D / kQElems; m <<= 1) {
      const float sgn = (c & m) ? -1.f : 1.f;
#pragma unroll
      for (int e = 0; e < kQElems; ++e) {
        const int bits = __builtin_bit_cast(int, v[e]);
        const int ob = m == 1 ? __builtin_amdgcn_mov_dpp(bits, 0xB1, 0xF, 0xF, true)    // quad_perm [1,0,3,2]
                              : __builtin_amdgcn_mov_dpp(bits, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
        v[e] = fmaf(sgn, v[e], __builtin_bit_cast(float, ob));
      }
    }
  }
}

// Pass 1: the workgroup's largest |y|, stored as float number rb of the
// head's (not yet written) code buffer.
template <int D, bool ROT>
__global__ __launch_bounds__(kQThreads) void fp8_amax_kernel(const __bf16* __restrict__ X, uint8_t* __restrict__ X8,
                                                             int N, int nrb, uint64_t slo, uint64_t shi) {
  constexpr int kPer = D / kQElems, kPass = kQThreads / kPer;
  const int bh = blockIdx.x / nrb, rb = blockIdx.x % nrb;
  const int tid = threadIdx.x, c = tid % kPer;
  const size_t head_off = (size_t)bh * N * D;
  unsigned sg[kQElems];
  sign_words(kQElems * c, slo, shi, sg);
  float m = 0.f;
#pragma unroll
  for (int it = 0; it < kQIter; ++it) {
    float v[kQElems];
    row_chunk<D, ROT>(X, head_off, rb * kPass * kQIter + it * kPass + tid / kPer, N, c, sg, v);
#pragma unroll
    for (int e = 0; e < kQElems; ++e) m = fmaxf(m, fabsf(v[e]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float wm[kQThreads / 64];
  if ((tid & 63) == 0) wm[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kQThreads / 64; ++w) m = fmaxf(m, wm[w]);
    reinterpret_cast<float*>(X8 + head_off)[rb] = m;
  }
}

// The head's amax from the nrb workgroup maxima, into amax[bh].
__global__ __launch_bounds__(256) void fp8_reduce_kernel(const uint8_t* __restrict__ X8, float* __restrict__ amax,
                                                        size_t head_bytes, int nrb) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  const float* part = reinterpret_cast<const float*>(X8 + (size_t)bh * head_bytes);
  float m = 0.f;
  for (int i = tid; i < nrb; i += 256) m = fmaxf(m, part[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float wm[4];
  if ((tid & 63) == 0) wm[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) amax[bh] = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
}

template <int D, bool ROT>
__global__ __launch_bounds__(kQThreads) void fp8_quant_kernel(const __bf16* __restrict__ X, uint8_t* __restrict__ X8,
                                                              const float* __restrict__ amax, int N, int nrb,
                                                              uint64_t slo, uint64_t shi) {
  constexpr int kPer = D / kQElems, kPass = kQThreads / kPer;
  const int bh = blockIdx.x / nrb, rb = blockIdx.x % nrb;
  const int tid = threadIdx.x, c = tid % kPer;
  const size_t head_off = (size_t)bh * N * D;
  const float am = amax_used(amax[bh]);
  const float s = am > 0.f ? kE4M3Max / am : 1.f;
  unsigned sg[kQElems];
  sign_words(kQElems * c, slo, shi, sg);
#pragma unroll
  for (int it = 0; it < kQIter; ++it) {
    const int row = rb * kPass * kQIter + it * kPass + tid / kPer;
    float v[kQElems];
    row_chunk<D, ROT>(X, head_off, row, N, c, sg, v);
    if (row < N) {
      u32x4 w[2];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * q] * s, v[4 * q + 1] * s, 0, false);
        w[q >> 2][q & 3] = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(v[4 * q + 2] * s, v[4 * q + 3] * s, lo, true);
      }
      u32x4* dst = reinterpret_cast<u32x4*>(X8 + head_off + (size_t)row * D + kQElems * c);
      dst[0] = w[0];
      dst[1] = w[1];
    }
  }
}

// amax -> descale in place: amax / 448, times 1/sqrt(d) after a rotation.
__global__ void fp8_descale_kernel(float* __restrict__ p, int n, int rot, float inv_sqrt_d) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    float dsc = amax_used(p[i]) / kE4M3Max;
    if (rot) dsc = dsc * inv_sqrt_d;
    p[i] = dsc;
  }
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

extern "C" int fa_quant_fp8(const void* x, void* x8, float* descale, int B, int H, int N, int d, int rotate,
                            uint64_t sign_lo, uint64_t sign_hi, hipStream_t stream) {
  if (!x || !x8 || !descale) return FA_ERR_NULL;
  long long bh = 0;
  const int st = check_shape8(B, H, N, d, &bh);
  if (st != FA_OK) return st;
  if (rotate != 0 && rotate != 1) return FA_ERR_FLAG;
  if ((reinterpret_cast<uintptr_t>(x) & 15u) || (reinterpret_cast<uintptr_t>(x8) & 15u) ||
      (reinterpret_cast<uintptr_t>(descale) & 3u))
    return FA_ERR_ALIGN;
  const size_t elems = (size_t)bh * N * d;
  if (overlaps(x8, elems, x, 2 * elems) || overlaps(descale, (size_t)bh * 4, x, 2 * elems) ||
      overlaps(descale, (size_t)bh * 4, x8, elems))
    return FA_ERR_ALIAS;
  const int rows_per_wg = (kQThreads * kQElems / d) * kQIter;
  const long long nrb = ((long long)N + rows_per_wg - 1) / rows_per_wg;
  if (nrb * bh > 0x7fffffffLL / kQThreads) return FA_ERR_SHAPE;
  const unsigned grid = (unsigned)(nrb * bh);
  const unsigned small = (unsigned)((bh + 255) / 256);
  const __bf16* X = static_cast<const __bf16*>(x);
  uint8_t* X8 = static_cast<uint8_t*>(x8);
  // the codes' buffer first holds each workgroup's amax (nrb floats per head,
  // at most N d bytes), then descale holds each head's amax, then the codes
  // and the factors are written
  const size_t head_bytes = (size_t)N * d;
  const dim3 g(grid), blk(kQThreads);
  if (d == 128) {
    if (rotate) hipLaunchKernelGGL((fp8_amax_kernel<128, true>), g, blk, 0, stream, X, X8, N, (int)nrb, sign_lo, sign_hi);
    else        hipLaunchKernelGGL((fp8_amax_kernel<128, false>), g, blk, 0, stream, X, X8, N, (int)nrb, sign_lo, sign_hi);
  } else {
    if (rotate) hipLaunchKernelGGL((fp8_amax_kernel<64, true>), g, blk, 0, stream, X, X8, N, (int)nrb, sign_lo, sign_hi);
    else        hipLaunchKernelGGL((fp8_amax_kernel<64, false>), g, blk, 0, stream, X, X8, N, (int)nrb, sign_lo, sign_hi);
  }
  hipLaunchKernelGGL(fp8_reduce_kernel, dim3((unsigned)bh), dim3(256), 0, stream, X8, descale, head_bytes, (int)nrb);
  if (d == 128) {
    if (rotate) hipLaunchKernelGGL((fp8_quant_kernel<128, true>), g, blk, 0, stream, X, X8, descale, N, (int)nrb, sign_lo, sign_hi);
    else        hipLaunchKernelGGL((fp8_quant_kernel<128, false>), g, blk, 0, stream, X, X8, descale, N, (int)nrb, sign_lo, sign_hi);
  } else {
    if (rotate) hipLaunchKernelGGL((fp8_quant_kernel<64, true>), g, blk, 0, stream, X, X8, descale, N, (int)nrb, sign_lo, sign_hi);
    else        hipLaunchKernelGGL((fp8_quant_kernel<64, false>), g, blk, 0, stream, X, X8, descale, N, (int)nrb, sign_lo, sign_hi);
  }
  const float inv_sqrt_d = (float)(1.0 / sqrt((double)d));
  hipLaunchKernelGGL(fp8_descale_kernel, dim3(small), dim3(256), 0, stream, descale, (int)bh, rotate, inv_sqrt_d);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

