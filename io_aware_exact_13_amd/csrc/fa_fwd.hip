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
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

constexpr int kBR = 128;          // query rows per workgroup
constexpr int kBC = 64;           // keys per K/V tile
constexpr int kWaves = 4;         // waves per workgroup, 32 query rows each
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.0f;    // log2 units the reference max may lag the true max

template <int D>
struct Geom {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;           // 16-byte chunks per row
  static constexpr int kTileBytes = kBC * kRowBytes;       // one K or V tile
  static constexpr int kStageBytes = 2 * kTileBytes;       // K then V
  static constexpr int kLdsBytes = 2 * kStageBytes;        // two stages
  static constexpr int kLoadsPerTile = kTileBytes / (kThreads * 16);
  static_assert(kLoadsPerTile * kThreads * 16 == kTileBytes, "tile not a whole number of loads");
};

// Chunk-level XOR swizzle of a tile row.  Rows r and r+k get distinct masks
// for the 16 consecutive rows of an A-operand fetch (D=128; 8 rows for D=64),
// and the masks of 4 aligned rows differ in bits 1..2 so that the two chunks
// each row contributes to a transposed read land in different banks.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 7) << 1) | ((row >> 3) & 1);
  else return ((row & 3) << 1) | ((row >> 2) & 1);
}

// Enqueue the HBM -> LDS copy of one K or V tile (kBC rows starting at key0).
// global_load_lds writes lane t's 16 bytes to LDS base + 16 t, so each lane
// fetches the global chunk that the swizzle places in its slot.  Rows past
// the end of the sequence re-read row N-1: those keys are masked to -inf in S
// (P = 0) and the V values they bring are finite, so they add exactly 0.
template <int D>
__device__ __forceinline__ void load_tile(const char* __restrict__ head, int key0, int n,
                                          char* lds_tile, int wave, int lane) {
  using G = Geom<D>;
#pragma unroll
  for (int i = 0; i < G::kLoadsPerTile; ++i) {
    const int slot = (i * kWaves + wave) * 1024;            // wave-uniform LDS offset
    const int byte = slot + lane * 16;
    const int row = byte / G::kRowBytes;
    const int pchunk = (byte % G::kRowBytes) >> 4;
    const int lchunk = pchunk ^ swz<D>(row);
    const int grow = min(key0 + row, n - 1);
    const char* src = head + (size_t)grow * G::kRowBytes + (lchunk << 4);
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(lds_tile + slot), 16, 0, 0);
  }
}

// Running state of one wave: 32 query rows, lane l owns row l % 32.
template <int D>
struct RowState {
  f32x16 acc[D / 32];   // O^T accumulators: lane holds column (r/4)*8 + 4h + r%4 of each 32-col tile
  float m_ref;          // reference max, log2 units of the scaled score
  float l_part;         // this lane's share of the exponential sum
};

// One K/V tile for one wave: S^T = K Q^T, mask, online softmax, O^T += V^T P^T,
// and the copy of the next tile into the other LDS stage.  The stages are
// passed as separate restrict pointers: nothing read here aliases the stage
// being filled, which lets the compiler keep the asynchronous LDS copy in
// flight across these LDS reads (the loop waits for it explicitly).
template <int D, bool CAUSAL>
__device__ __forceinline__ void tile_step(const char* __restrict__ Kt, const char* __restrict__ Vt,
                                          char* __restrict__ next_stage, bool prefetch,
                                          const char* Kh, const char* Vh, int key0, int N,
                                          int q0, int qrow, int wave, int lane,
                                          const bf16x8 (&qf)[D / 16], float c_log2,
                                          RowState<D>& st) {
  using G = Geom<D>;
  constexpr int kDs = D / 16;   // MFMA k-steps over the head dimension (S product)
  constexpr int kCt = D / 32;   // 32-wide column tiles of O^T
  constexpr int kKb = kBC / 32; // 32-key blocks of S^T per tile
  constexpr int kKs = kBC / 16; // MFMA k-steps over keys (P V product)
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int a16 = lane & 15;
  const int cg = (lane >> 4) & 1;

  if (prefetch) {
    load_tile<D>(Kh, key0 + kBC, N, next_stage, wave, lane);
    load_tile<D>(Vh, key0 + kBC, N, next_stage + G::kTileBytes, wave, lane);
  }

  // A wave whose rows all precede this tile's first key sees none of it.
  if (CAUSAL && key0 > q0 + wave * 32 + 31) return;

  // ---- S^T = K Q^T  (fp32, unscaled).  A operand: K row 32 kb + l32, chunk 2 ks + h.
  const int k_swz = swz<D>(l32);                    // swz depends on row & 15 only
  f32x16 s[kKb];
#pragma unroll
  for (int kb = 0; kb < kKb; ++kb) {
    s[kb] = f32x16{};
    const char* krow = Kt + (kb * 32 + l32) * G::kRowBytes;
#pragma unroll
    for (int ks = 0; ks < kDs; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + (((ks * 2 + h) ^ k_swz) << 4));
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
    }
  }

  // ---- masks: keys past the end, and keys after the query under the causal mask
  const bool tail = key0 + kBC > N;
  const bool diag = CAUSAL && (key0 + kBC - 1 > q0 + wave * 32);
  if (tail || diag) {
    const int lim = CAUSAL ? min(qrow, N - 1) : (N - 1);
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + kb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        if (key > lim) s[kb][r] = -INFINITY;
      }
  }

  // ---- online softmax (base 2)
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
    for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[ct][r] *= alpha;
  }
  st.m_ref = m_new;
  const float neg_m = (m_new == -INFINITY) ? 0.f : -m_new;

  // P is summed in fp32 (the logsumexp needs the unrounded weights) and
  // rounded to bf16 for the MFMA.
  bf16x8 pf[kKs];
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

  // ---- O^T += V^T P^T.  k-step t covers keys 16t..16t+15 of the tile; lane
  // half h supplies keys 16t + 4h + {0..3} (elements 0..3) and
  // 16t + 8 + 4h + {0..3} (elements 4..7), matching the S^T layout.  The
  // transposed read gives lane a of each 16-lane group column cbase + a of
  // 4 consecutive rows when lane a points at row a/4, columns cbase + 4(a%4).
#pragma unroll
  for (int t = 0; t < kKs; ++t) {
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
      const int col = ct * 32 + cg * 16 + 4 * (a16 & 3);
      const int chunk = col >> 3;
      const int sub = (col & 7) * 2;
      const int row_lo = 16 * t + 4 * h + (a16 >> 2);
      const int row_hi = row_lo + 8;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_t*)(Vt + row_lo * G::kRowBytes + ((chunk ^ swz<D>(row_lo)) << 4) + sub));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_t*)(Vt + row_hi * G::kRowBytes + ((chunk ^ swz<D>(row_hi)) << 4) + sub));
      const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      st.acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pf[t],
                                                           st.acc[ct], 0, 0, 0);
    }
  }
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

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;      // which half of the 64 lanes
  const int l32 = lane & 31;    // this lane's query row within the wave

  // ---- workgroup -> (head, query block)
  const int wg = blockIdx.x;
  const int bh = wg % BH;
  const int qb = CAUSAL ? (n_qblocks - 1 - wg / BH) : (wg / BH);
  const int q0 = qb * kBR;
  const int qrow = q0 + wave * 32 + l32;               // this lane's query

  const size_t head_off = (size_t)bh * (size_t)N * D;
  const char* Kh = reinterpret_cast<const char*>(K + head_off);
  const char* Vh = reinterpret_cast<const char*>(V + head_off);

  // ---- key range
  int kv_end = N;
  if (CAUSAL) kv_end = min(N, q0 + kBR);
  const int n_tiles = (kv_end + kBC - 1) / kBC;

  // ---- start the first K/V tile while Q is fetched
  load_tile<D>(Kh, 0, N, lds, wave, lane);
  load_tile<D>(Vh, 0, N, lds + G::kTileBytes, wave, lane);

  // ---- Q^T operand: lane holds Q[qrow][16*ks + 8*h .. +7] for each k-step
  bf16x8 qf[kDs];
  {
    const bool ok = qrow < N;
    const bf16x8* src = reinterpret_cast<const bf16x8*>(Q + head_off + (size_t)(ok ? qrow : 0) * D);
#pragma unroll
    for (int ks = 0; ks < kDs; ++ks) {
      bf16x8 x = src[ks * 2 + h];
      if (!ok) x = bf16x8{};
      qf[ks] = x;
    }
  }

  RowState<D> st;
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) st.acc[ct] = f32x16{};
  st.m_ref = -INFINITY;
  st.l_part = 0.f;

  for (int j = 0; j < n_tiles; ++j) {
    const int stage = j & 1;
    char* cur = lds + stage * G::kStageBytes;
    char* nxt = lds + (stage ^ 1) * G::kStageBytes;
    // Tile j has landed (this thread's copies); after the barrier everyone's
    // copies are visible and everyone has finished tile j-1, whose stage the
    // next copy overwrites.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    tile_step<D, CAUSAL>(cur, cur + G::kTileBytes, nxt, j + 1 < n_tiles, Kh, Vh, j * kBC, N,
                         q0, qrow, wave, lane, qf, c_log2, st);
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
        const int c0 = ct * 32 + r4 * 8 + h * 4;
        const __bf16 b0 = (__bf16)(st.acc[ct][r4 * 4 + 0] * inv);
        const __bf16 b1 = (__bf16)(st.acc[ct][r4 * 4 + 1] * inv);
        const __bf16 b2 = (__bf16)(st.acc[ct][r4 * 4 + 2] * inv);
        const __bf16 b3 = (__bf16)(st.acc[ct][r4 * 4 + 3] * inv);
        u32x2 w;
        w[0] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        w[1] = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        *reinterpret_cast<u32x2*>(orow + c0) = w;
      }
    if (h == 0) LSE[(size_t)bh * N + qrow] = (st.m_ref + log2f(l_tot)) * kLn2;
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
